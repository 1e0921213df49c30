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


def gelu(x: np.ndarray) -> np.ndarray:
    """Exact GELU: x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2))."""
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


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
              allowed: Optional[np.ndarray] = None) -> np.ndarray:
    """Multi-head attention of queries [Nq][D] over keys/values [Nk][D].

    Head j uses columns j*hd .. (j+1)*hd - 1 of q, k and v; the head outputs
    are concatenated in the same column order.  With `allowed` = None every
    key is visible: the mask-free pattern of [FD] §3.3 "Attention Pattern".
    Heads are independent and run on a thread pool (numpy releases the GIL),
    which changes wall time only.
    """
    D = q.shape[1]
    hd = D // n_heads
    rows = max(1, min(q.shape[0], (1 << 24) // max(1, k.shape[0])))
    out = np.empty((q.shape[0], D), dtype=np.float64)

    def one(j):
        c = slice(j * hd, (j + 1) * hd)
        out[:, c] = _head_attention(q[:, c], k[:, c], v[:, c], allowed, rows)

    with threadpool_limits(limits=1, user_api="blas"):
        with concurrent.futures.ThreadPoolExecutor(min(n_heads, _threads())) as ex:
            list(ex.map(one, range(n_heads)))
    return out


def as_f64_weights(w: dict) -> dict:
    """Copy a weight dict (float32 arrays) to float64."""
    out = {k: np.asarray(v, dtype=np.float64) for k, v in w.items()
           if k != "layers"}
    out["layers"] = [{k: np.asarray(v, dtype=np.float64) for k, v in lw.items()}
                     for lw in w["layers"]]
    return out


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

    def __init__(self, cfg, weights: dict):
        self.cfg = cfg
        self.w = as_f64_weights(weights)
        self.reset()

    def reset(self) -> None:
        """Empty every cache; the next frame is frame 0 again."""
        self.t = 0
        self.cache: List[collections.deque] = [
            collections.deque() for _ in range(self.cfg.n_layers)]

    def cached_frames(self, layer: int) -> List[int]:
        """Frame indices held by `layer`'s cache, oldest first."""
        return [f for f, _, _ in self.cache[layer]]

    def cached_kv(self, layer: int, frame: int):
        """(K, V) [N][D] float64 that `layer` cached for `frame`."""
        for f, k, v in self.cache[layer]:
            if f == frame:
                return k, v
        raise KeyError(frame)

    def decode_frame(self, z: np.ndarray) -> np.ndarray:
        """Decode latent z_t [C'][H'][W'] to pixels [out_t][H][W][out_c]."""
        cfg, w = self.cfg, self.w
        D = cfg.d_model
        x = patchify(z, cfg.patch)
        h = linear(x, w["w_in"], w["b_in"])
        for l, lw in enumerate(w["layers"]):
            a = layer_norm(h, lw["ln1_g"], lw["ln1_b"], cfg.ln_eps)
            qkv = linear(a, lw["w_qkv"], lw["b_qkv"])
            q, k, v = qkv[:, :D], qkv[:, D:2 * D], qkv[:, 2 * D:]
            cache = self.cache[l]
            cache.append((self.t, k, v))
            while len(cache) > cfg.window:
                cache.popleft()
            kc = np.concatenate([e[1] for e in cache], axis=0)
            vc = np.concatenate([e[2] for e in cache], axis=0)
            o = attention(q, kc, vc, cfg.n_heads)
            h = h + linear(o, lw["w_o"], lw["b_o"])
            a = layer_norm(h, lw["ln2_g"], lw["ln2_b"], cfg.ln_eps)
            u = gelu(linear(a, lw["w_1"], lw["b_1"]))
            h = h + linear(u, lw["w_2"], lw["b_2"])
        r = linear(layer_norm(h, w["lnf_g"], w["lnf_b"], cfg.ln_eps),
                   w["w_out"], w["b_out"])
        self.t += 1
        return unpatchify(r, cfg.tok_h, cfg.tok_w, cfg.out_t, cfg.out_patch,
                          cfg.out_c)


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
    D, N, T = cfg.d_model, cfg.n_tokens, len(latents)
    x = np.concatenate([patchify(z, cfg.patch) for z in latents], axis=0)
    allowed = block_causal_window_mask(T, N, cfg.window)
    h = linear(x, w["w_in"], w["b_in"])
    for lw in w["layers"]:
        a = layer_norm(h, lw["ln1_g"], lw["ln1_b"], cfg.ln_eps)
        qkv = linear(a, lw["w_qkv"], lw["b_qkv"])
        q, k, v = qkv[:, :D], qkv[:, D:2 * D], qkv[:, 2 * D:]
        o = attention(q, k, v, cfg.n_heads, allowed)
        h = h + linear(o, lw["w_o"], lw["b_o"])
        a = layer_norm(h, lw["ln2_g"], lw["ln2_b"], cfg.ln_eps)
        h = h + linear(gelu(linear(a, lw["w_1"], lw["b_1"])), lw["w_2"], lw["b_2"])
    r = linear(layer_norm(h, w["lnf_g"], w["lnf_b"], cfg.ln_eps),
               w["w_out"], w["b_out"])
    return [unpatchify(r[t * N:(t + 1) * N], cfg.tok_h, cfg.tok_w, cfg.out_t,
                       cfg.out_patch, cfg.out_c) for t in range(T)]
