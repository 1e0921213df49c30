"""Plain float64 CPU oracle of the FlashDecoder per-latent-frame decode step.

TEST INFRASTRUCTURE: used only by the tests, the smoke check and the CPU
baseline of the benchmark.  It shares no code with the HIP path.

Sources (cited by page title and section):
  [FD]  "FlashDecoder: Real-Time Latent-to-Pixel Streaming Decoder with
        Transformers", academ.us/article/2607.14898.
  [PF]  paperfeed.app summary of the same paper (2026-W29), section
        "The mechanism, concretely".

What is computed, per latent frame z_t (shape [C'][H'][W']):
  1. Tokens: z_t flattened into raster-order spatial tokens ([FD] §3.2 "Latent
     Projection", Eq. 1) after a p x p PixelUnshuffle fold of space into
     channels ([FD] §4.3 "Generalization Across Latent Spaces").
  2. H = X W_in^T + b_in  ([FD] Eq. 1).
  3. Per block, pre-norm ([FD] §3.2 "Base Architecture"):
       A = LN1(H);  [Q|K|V] = A W_qkv^T + b_qkv
       append (K, V) of this frame to the block's cache, evicting the oldest
       frame beyond W_frm ([FD] §3.3 "Frame-by-Frame Processing", Eq. 2)
       O = softmax(Q K_c^T / sqrt(hd)) V_c per head, over every cached key,
           with no mask ([FD] §3.3 "Attention Pattern")
       H += O W_o^T + b_o
       H += GELU(LN2(H) W_1^T + b_1) W_2^T + b_2
  4. R = LNf(H) W_out^T + b_out, then each token's R row is shuffled into a
     out_t x P x P x 3 pixel block ([FD] §3.4 "Step 3: Spatial Upsampling":
     linear projection then PixelShuffle).

Readings of points the pages leave open (each listed in the design notes):
  LayerNorm (not RMSNorm) with affine gain/shift, biased variance, eps 1e-5;
  a final LayerNorm before the unpatchify projection; exact erf GELU; plain
  multi-head attention (one KV head per query head); no positional encoding
  and no KV-norm; every Linear has a bias; score scale 1/sqrt(head_dim); the
  window counts the current frame, so frame 0 sees only itself; cached frames
  are concatenated oldest first; patch features ordered (c, dy, dx); pixel
  channels of a token ordered (tau, dy, dx, c) and written to a
  [out_t][H][W][out_c] frame; no clamp on pixels.
The paper's block ([FD] §3.2), when the config asks for it:
  RMSNorm x / sqrt(mean x^2 + eps) g for every pre-sublayer and the final
  norm; grouped-query attention with G KV heads, query head j reading KV
  head floor(j G / heads); KV-norm = the same RMS norm over each K and V head
  vector with gains kn_g, vn_g; 3D rotary positions on Q and K (after
  KV-norm): head dims split (hd - 4 floor(hd/6), 2 floor(hd/6), 2 floor(hd/6))
  between time, height and width, consecutive pairs, base 10000, temporal
  position relative to the current window (oldest cached frame 0).
The temporal-first upsampling tail ([FD] §3.4), when the config has
n_refine > 0 (it then replaces step 4):
  Y = final norm of H; P = Y W_tu^T + b_tu, [N][r_t D] (Eq. 3); column block
  k of P (columns k D .. (k+1) D - 1) becomes sub-frame k, so the r_t N
  sub-frame tokens are ordered (k, n); n_refine blocks of the same kind as the
  backbone's process them with the same streaming mechanism, one step per
  latent frame, the cache holding W latent frames = r_t W sub-frames (every
  token of a step sees all of them, no mask); rotary temporal positions count
  sub-frames (sub-frame k of window frame f at r_t f + k); then a norm and a
  2-layer MLP D -> up_hidden -> r_s^2 C with GELU between, and a PixelShuffle
  per sub-frame token: sub-frame k is pixel frame k of the latent frame.

Precision: float64 for every step.
"""
from __future__ import annotations

import collections
import concurrent.futures
import math
import os
from typing import Dict, List, Optional

import numpy as np
from scipy.special import erf
from threadpoolctl import threadpool_limits


# --------------------------------------------------------------------------
# Primitives
# --------------------------------------------------------------------------
def patchify(z: np.ndarray, p: int) -> np.ndarray:
    """Latent frame [C'][H'][W'] -> tokens [N][C' p^2].

    [FD] §3.2 Eq. 1 flattens a frame into H'W' raster-order tokens; [FD] §4.3
    first folds each p x p block of space into channels (PixelUnshuffle).
    Token n = i (W'/p) + j holds feature f = c p^2 + dy p + dx, equal to
    z[c][i p + dy][j p + dx].
    """
    C, H, W = z.shape
    x = np.asarray(z, dtype=np.float64).reshape(C, H // p, p, W // p, p)
    # axes (c, i, dy, j, dx) -> (i, j, c, dy, dx)
    x = x.transpose(1, 3, 0, 2, 4)
    return np.ascontiguousarray(x.reshape((H // p) * (W // p), C * p * p))


def unpatchify(r: np.ndarray, tok_h: int, tok_w: int, out_t: int, P: int,
               out_c: int) -> np.ndarray:
    """Token outputs [N][out_t P P out_c] -> pixels [out_t][tok_h P][tok_w P][out_c].

    [FD] §3.4 "Step 3": project to C r_s^2 channels, then PixelShuffle.  Token
    n = i tok_w + j, channel ((tau P + dy) P + dx) out_c + c lands at
    pixel[tau][i P + dy][j P + dx][c].
    """
    x = np.asarray(r, dtype=np.float64).reshape(tok_h, tok_w, out_t, P, P, out_c)
    # axes (i, j, tau, dy, dx, c) -> (tau, i, dy, j, dx, c)
    x = x.transpose(2, 0, 3, 1, 4, 5)
    return np.ascontiguousarray(x.reshape(out_t, tok_h * P, tok_w * P, out_c))


def linear(x: np.ndarray, w: np.ndarray, b: np.ndarray) -> np.ndarray:
    """y = x W^T + b, with W stored [out][in] ([FD] Eq. 1, Eq. 3 "Linear")."""
    return x @ w.T + b


def layer_norm(x: np.ndarray, g: np.ndarray, b: np.ndarray,
               eps: float) -> np.ndarray:
    """Per row: (x - mean) / sqrt(biased variance + eps) * g + b.

    [FD] §3.2 places a norm before each sublayer; this build reads it as
    LayerNorm with affine parameters.
    """
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * g + b


def rms_norm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """Per row: x / sqrt(mean(x^2) + eps) * g  (RMSNorm, [FD] §3.2 "Base
    Architecture": RMSNorm before each sublayer)."""
    return x / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps) * g


def pre_norm(cfg, x: np.ndarray, g: np.ndarray, b: np.ndarray) -> np.ndarray:
    """The pre-sublayer norm the config names: LayerNorm or RMSNorm."""
    if cfg.norm == "rms":
        return rms_norm(x, g, cfg.ln_eps)
    return layer_norm(x, g, b, cfg.ln_eps)


def kv_norm(x: np.ndarray, g: np.ndarray, head_dim: int, eps: float) -> np.ndarray:
    """RMS-normalise every head vector of x [N][heads*hd] and scale by g [hd]
    ([FD] §3.2: keys and values are normalised within attention; read as
    RMSNorm over each head's dimensions)."""
    n = x.shape[0]
    h = x.reshape(n, -1, head_dim)
    return rms_norm(h, g, eps).reshape(n, -1)


def rope_split(head_dim: int):
    """Head dimensions given to the (temporal, height, width) rotations:
    hd - 4 floor(hd/6), 2 floor(hd/6), 2 floor(hd/6), in that order."""
    s = 2 * (head_dim // 6)
    return head_dim - 2 * s, s, s


def rope_angles(cfg, t_pos, i_pos, j_pos) -> np.ndarray:
    """Rotation angle of every dimension pair: [n][hd/2].

    [FD] §3.2: 3D rotary embeddings applied separately to the temporal and
    the two spatial axes.  Part a of size d_a rotates its pairs k = 0 ..
    d_a/2-1 by pos_a * theta^(-2k/d_a).  t_pos, i_pos, j_pos: [n] positions.
    """
    parts = []
    for size, pos in zip(rope_split(cfg.head_dim), (t_pos, i_pos, j_pos)):
        k = np.arange(size // 2, dtype=np.float64)
        freq = cfg.rope_theta ** (-2.0 * k / size)
        parts.append(np.asarray(pos, dtype=np.float64)[:, None] * freq[None, :])
    return np.concatenate(parts, axis=1)


def apply_rope(x: np.ndarray, angles: np.ndarray, head_dim: int) -> np.ndarray:
    """Rotate every consecutive pair (2k, 2k+1) of every head vector of
    x [n][heads*hd] by angles [n][hd/2]: (a, b) -> (a cos - b sin, a sin + b cos)."""
    n = x.shape[0]
    h = x.reshape(n, -1, head_dim // 2, 2)
    c = np.cos(angles)[:, None, :]
    s = np.sin(angles)[:, None, :]
    a, b = h[..., 0], h[..., 1]
    out = np.stack([a * c - b * s, a * s + b * c], axis=-1)
    return out.reshape(n, -1)


def token_rope_angles(cfg, frame_pos: float) -> np.ndarray:
    """Angles for the N tokens of one frame at temporal position frame_pos:
    token n = i tok_w + j sits at (frame_pos, i, j)."""
    n = np.arange(cfg.n_tokens)
    return rope_angles(cfg, np.full(cfg.n_tokens, frame_pos, dtype=np.float64),
                       n // cfg.tok_w, n % cfg.tok_w)


def subframe_rope_angles(cfg, frame_pos: float) -> np.ndarray:
    """Angles for the r_t N tokens one latent frame has after temporal
    upsampling, at window position frame_pos: token k N + n sits at temporal
    position r_t frame_pos + k (positions count sub-frames) and at the row and
    column of spatial token n."""
    return np.concatenate([token_rope_angles(cfg, cfg.out_t * frame_pos + k)
                           for k in range(cfg.out_t)], axis=0)


def subframe_tokens(p: np.ndarray, r_t: int) -> np.ndarray:
    """[FD] §3.4 Step 1: the expanded channels of P [N][r_t D] read as r_t new
    temporal positions.  Returns [r_t N][D]; row k N + n is column block k of
    token n (columns k D .. (k+1) D - 1)."""
    n, c = p.shape
    d = c // r_t
    return np.concatenate([p[:, k * d:(k + 1) * d] for k in range(r_t)], axis=0)


def gelu(x: np.ndarray) -> np.ndarray:
    """Exact GELU: x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2))."""
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def host_threads() -> int:
    """Threads for the per-head pool: the host's allotment, i.e.
    OMP_NUM_THREADS when set (the CPU share given to this process), else the
    CPUs this process may run on."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        return int(env)
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:
        return max(1, os.cpu_count() or 1)


def _head_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                    allowed: Optional[np.ndarray], rows: int) -> np.ndarray:
    """One head: softmax(q k^T / sqrt(hd)) v, two-pass softmax per query row.

    Masked scores (allowed == False) take no part in the max or the sum.
    Query rows are processed `rows` at a time only to bound memory; each row
    is computed exactly as if alone.
    """
    hd = q.shape[1]
    scale = 1.0 / math.sqrt(hd)
    out = np.empty((q.shape[0], v.shape[1]), dtype=np.float64)
    for r0 in range(0, q.shape[0], rows):
        r1 = min(q.shape[0], r0 + rows)
        s = (q[r0:r1] @ k.T) * scale
        if allowed is not None:
            s = np.where(allowed[r0:r1], s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)                      # exp(-inf) = 0 for masked keys
        out[r0:r1] = (e @ v) / e.sum(axis=1, keepdims=True)
    return out


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, n_heads: int,
              allowed: Optional[np.ndarray] = None,
              n_kv_heads: Optional[int] = None) -> np.ndarray:
    """Multi-head attention of queries [Nq][n_heads*hd] over keys/values
    [Nk][G*hd], G = n_kv_heads (default n_heads).

    Query head j uses columns j*hd .. (j+1)*hd - 1 of q and KV head
    floor(j G / n_heads) of k and v (grouped-query attention, [FD] §3.2; with
    G = n_heads it is plain multi-head attention); the head outputs are
    concatenated in query-head order.  With `allowed` = None every key is
    visible: the mask-free pattern of [FD] §3.3 "Attention Pattern".  Heads
    are independent and run on a thread pool (numpy releases the GIL), which
    changes wall time only.
    """
    D = q.shape[1]
    hd = D // n_heads
    G = n_kv_heads or n_heads
    rows = max(1, min(q.shape[0], (1 << 24) // max(1, k.shape[0])))
    out = np.empty((q.shape[0], D), dtype=np.float64)

    def one(j):
        c = slice(j * hd, (j + 1) * hd)
        g = j * G // n_heads
        ck = slice(g * hd, (g + 1) * hd)
        out[:, c] = _head_attention(q[:, c], k[:, ck], v[:, ck], allowed, rows)

    with threadpool_limits(limits=1, user_api="blas"):
        with concurrent.futures.ThreadPoolExecutor(min(n_heads, host_threads())) as ex:
            list(ex.map(one, range(n_heads)))
    return out


def as_f64_weights(w: dict) -> dict:
    """Copy a weight dict (float32 arrays) to float64."""
    out = {k: np.asarray(v, dtype=np.float64) for k, v in w.items()
           if k not in ("layers", "refine")}
    for key in ("layers", "refine"):
        if key in w:
            out[key] = [{k: np.asarray(v, dtype=np.float64) for k, v in lw.items()}
                        for lw in w[key]]
    return out


def split_qkv(cfg, qkv: np.ndarray, lw: dict):
    """Columns of the QKV projection -> (Q [N][heads*hd], K, V [N][G*hd]),
    with K and V RMS-normalised per head when the config asks for KV-norm."""
    nq = cfg.n_heads * cfg.head_dim
    nk = cfg.kv_heads * cfg.head_dim
    q, k, v = qkv[:, :nq], qkv[:, nq:nq + nk], qkv[:, nq + nk:]
    if cfg.kv_norm:
        k = kv_norm(k, lw["kn_g"], cfg.head_dim, cfg.ln_eps)
        v = kv_norm(v, lw["vn_g"], cfg.head_dim, cfg.ln_eps)
    return q, k, v


def spatial_upsample(cfg, w: dict, hr: np.ndarray) -> np.ndarray:
    """[FD] §3.4 Step 3 on the r_t N refined tokens of one latent frame:
    norm, 2-layer MLP D -> up_hidden -> r_s^2 C (GELU between), then a
    PixelShuffle of every token; sub-frame k (rows k N .. (k+1) N - 1) becomes
    pixel frame k.  Returns [r_t][H' r_s][W' r_s][C]."""
    a = pre_norm(cfg, hr, w["lnr_g"], w["lnr_b"])
    s = linear(gelu(linear(a, w["w_s1"], w["b_s1"])), w["w_s2"], w["b_s2"])
    n = cfg.n_tokens
    return np.stack([unpatchify(s[k * n:(k + 1) * n], cfg.tok_h, cfg.tok_w, 1,
                                cfg.out_patch, cfg.out_c)[0]
                     for k in range(cfg.out_t)], axis=0)


# --------------------------------------------------------------------------
# Streaming decoder
# --------------------------------------------------------------------------
class StreamingDecoder:
    """Frame-by-frame decode with a rolling per-block KV cache.

    [FD] §3.3 "Frame-by-Frame Processing": at each step the frame is projected
    (Eq. 1), each block appends the frame's keys and values to its cache and
    evicts the oldest frame once the cache holds more than W_frm frames
    (Eq. 2), and the frame's queries attend to the whole cache.  W_frm counts
    the current frame ([FD] §3.3 first paragraph: a frame sees itself and the
    immediately preceding frame when W_frm = 2; [PF]: W_frm - 1 = 1 previous
    frame), so frame 0 attends to itself only.
    """

    def __init__(self, cfg, weights: dict, mlp_operands=None):
        """mlp_operands: optional callable (name, array) -> array applied to
        the four operands of the MLP products before they are multiplied,
        names "fc1_act" (normed input), "fc1_w" (W_1), "fc2_act" (GELU
        output), "fc2_w" (W_2).  It models reduced-precision MLP GEMMs
        ([FD] §4.6 "Inference Optimization" item (4): FP8 MLP layers); None
        (the default) leaves every operand exact."""
        self.cfg = cfg
        self.w = as_f64_weights(weights)
        self.mlp_operands = mlp_operands
        self.reset()

    def reset(self) -> None:
        """Empty every cache; the next frame is frame 0 again.  Caches
        0 .. n_layers-1 belong to the backbone blocks, the rest to the
        refinement blocks of the tail."""
        self.t = 0
        self.cache: List[collections.deque] = [
            collections.deque() for _ in range(self.cfg.n_layers + self.cfg.n_refine)]

    def cached_frames(self, layer: int) -> List[int]:
        """Frame indices held by `layer`'s cache, oldest first."""
        return [f for f, _, _ in self.cache[layer]]

    def cached_kv(self, layer: int, frame: int):
        """(K, V) [n][G*hd] float64 that `layer` cached for `frame` (keys
        before any rotary position); n = N for a backbone block, r_t N for a
        refinement block."""
        for f, k, v in self.cache[layer]:
            if f == frame:
                return k, v
        raise KeyError(frame)

    def _block(self, lw: dict, h: np.ndarray, cache: collections.deque,
               angles) -> np.ndarray:
        """One pre-norm block on this frame's tokens h, with its rolling cache.
        angles(pos): rotary angles of a frame at window position pos."""
        cfg = self.cfg
        a = pre_norm(cfg, h, lw["ln1_g"], lw["ln1_b"])
        q, k, v = split_qkv(cfg, linear(a, lw["w_qkv"], lw["b_qkv"]), lw)
        cache.append((self.t, k, v))
        while len(cache) > cfg.window:
            cache.popleft()
        if cfg.rope:
            q = apply_rope(q, angles(len(cache) - 1), cfg.head_dim)
            kc = np.concatenate([apply_rope(e[1], angles(pos), cfg.head_dim)
                                 for pos, e in enumerate(cache)], axis=0)
        else:
            kc = np.concatenate([e[1] for e in cache], axis=0)
        vc = np.concatenate([e[2] for e in cache], axis=0)
        o = attention(q, kc, vc, cfg.n_heads, n_kv_heads=cfg.kv_heads)
        h = h + linear(o, lw["w_o"], lw["b_o"])
        a = pre_norm(cfg, h, lw["ln2_g"], lw["ln2_b"])
        op = self.mlp_operands or (lambda name, x: x)
        u = gelu(linear(op("fc1_act", a), op("fc1_w", lw["w_1"]), lw["b_1"]))
        return h + linear(op("fc2_act", u), op("fc2_w", lw["w_2"]), lw["b_2"])

    def decode_frame(self, z: np.ndarray) -> np.ndarray:
        """Decode latent z_t [C'][H'][W'] to pixels [out_t][H][W][out_c].

        With rotary positions the cache keeps keys unrotated; at every step
        the cached frames take temporal positions 0 .. n_valid-1 of the
        current window, oldest first (the current frame last), and the keys
        and queries are rotated at those positions ([FD] §3.3 step (2), §4.3
        "Long Video Decoding": positions relative to the current window).
        """
        cfg, w = self.cfg, self.w
        x = patchify(z, cfg.patch)
        h = linear(x, w["w_in"], w["b_in"])
        for l, lw in enumerate(w["layers"]):
            h = self._block(lw, h, self.cache[l], lambda pos: token_rope_angles(cfg, pos))
        y = pre_norm(cfg, h, w["lnf_g"], w["lnf_b"])
        if cfg.n_refine == 0:
            pix = unpatchify(linear(y, w["w_out"], w["b_out"]), cfg.tok_h, cfg.tok_w,
                             cfg.out_t, cfg.out_patch, cfg.out_c)
        else:
            hr = subframe_tokens(linear(y, w["w_tu"], w["b_tu"]), cfg.out_t)
            for r, lw in enumerate(w["refine"]):
                hr = self._block(lw, hr, self.cache[cfg.n_layers + r],
                                 lambda pos: subframe_rope_angles(cfg, pos))
            pix = spatial_upsample(cfg, w, hr)
        self.t += 1
        return pix


# --------------------------------------------------------------------------
# Full-sequence masked formulation (brute force)
# --------------------------------------------------------------------------
def block_causal_window_mask(frames: int, n_tok: int, window: int) -> np.ndarray:
    """[T'N][T'N] boolean: query of frame fq may see key of frame fk iff
    0 <= fq - fk <= window - 1.

    This is the sliding-window pattern of [FD] §3.3 "Attention Pattern"
    (bidirectional inside a frame, the last W_frm frames in time) written as
    the explicit mask a single full-sequence pass needs ([FD] §3.3
    "Training-Inference Consistency"; §4.2 "SW-CA").
    """
    f = np.repeat(np.arange(frames), n_tok)
    d = f[:, None] - f[None, :]
    return (d >= 0) & (d <= window - 1)


def bruteforce_decode(cfg, weights: dict, latents: List[np.ndarray]) -> List[np.ndarray]:
    """All frames in one pass over the whole token sequence, with the mask.

    Same blocks as the streaming decoder, but every block sees all T' N tokens
    at once and the temporal window is imposed by `block_causal_window_mask`
    instead of by the cache.  Returns pixels per frame.
    """
    w = as_f64_weights(weights)
    N, T = cfg.n_tokens, len(latents)
    x = np.concatenate([patchify(z, cfg.patch) for z in latents], axis=0)
    allowed = block_causal_window_mask(T, N, cfg.window)
    ang = None
    if cfg.rope:
        # Absolute frame indices: rotary scores depend on position
        # differences only, so this equals the window-relative positions of
        # the streaming decoder up to rounding.
        ang = np.concatenate([token_rope_angles(cfg, t) for t in range(T)], axis=0)
    h = linear(x, w["w_in"], w["b_in"])
    for lw in w["layers"]:
        h = _masked_block(cfg, lw, h, allowed, ang)
    y = pre_norm(cfg, h, w["lnf_g"], w["lnf_b"])
    if cfg.n_refine == 0:
        r = linear(y, w["w_out"], w["b_out"])
        return [unpatchify(r[t * N:(t + 1) * N], cfg.tok_h, cfg.tok_w, cfg.out_t,
                           cfg.out_patch, cfg.out_c) for t in range(T)]
    # Tail over all T' r_t N sub-frame tokens, ordered (t, k, n); the window
    # is the same W latent frames, now of r_t N tokens each.
    rt, d = cfg.out_t, cfg.d_model
    p = linear(y, w["w_tu"], w["b_tu"])
    hr = np.concatenate([p[t * N:(t + 1) * N, k * d:(k + 1) * d]
                         for t in range(T) for k in range(rt)], axis=0)
    allowed = block_causal_window_mask(T, rt * N, cfg.window)
    if cfg.rope:
        ang = np.concatenate([token_rope_angles(cfg, rt * t + k)
                              for t in range(T) for k in range(rt)], axis=0)
    for lw in w["refine"]:
        hr = _masked_block(cfg, lw, hr, allowed, ang)
    return [spatial_upsample(cfg, w, hr[t * rt * N:(t + 1) * rt * N]) for t in range(T)]


def _masked_block(cfg, lw: dict, h: np.ndarray, allowed: np.ndarray,
                  ang: Optional[np.ndarray]) -> np.ndarray:
    """One pre-norm block over a whole token sequence with an explicit mask;
    ang: absolute rotary angles of every token (None without rotation)."""
    a = pre_norm(cfg, h, lw["ln1_g"], lw["ln1_b"])
    q, k, v = split_qkv(cfg, linear(a, lw["w_qkv"], lw["b_qkv"]), lw)
    if cfg.rope:
        q = apply_rope(q, ang, cfg.head_dim)
        k = apply_rope(k, ang, cfg.head_dim)
    o = attention(q, k, v, cfg.n_heads, allowed, n_kv_heads=cfg.kv_heads)
    h = h + linear(o, lw["w_o"], lw["b_o"])
    a = pre_norm(cfg, h, lw["ln2_g"], lw["ln2_b"])
    return h + linear(gelu(linear(a, lw["w_1"], lw["b_1"])), lw["w_2"], lw["b_2"])
