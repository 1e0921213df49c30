"""Seeded synthetic workloads for the FlashDecoder per-frame decode step.

This module is shared by the CPU oracle, the tests and the benchmark.  It holds
the workload table and the seeded generators only; none of the decoder's
arithmetic lives here.

Sources (web pages on FlashDecoder; cited by title and section):
  [FD]  "FlashDecoder: Real-Time Latent-to-Pixel Streaming Decoder with
        Transformers", academ.us/article/2607.14898.

Workloads.  The pages evaluate on 25-frame UltraVideo clips at 480p/720p/1080p
and on >400-frame 720p videos ([FD] §4.1 "Evaluation Data", §4.3 "Long Video
Decoding").  Neither dataset nor trained weights exist here, so every tensor is
drawn from a seeded generator with the Wan2.1 / Wan2.2 latent shapes the pages
use ([FD] §4 preamble: 4x16x16 latents; §4.3 "Generalization Across Latent
Spaces": 4x8x8 latents folded by a 2x2 PixelUnshuffle).

Random numbers.  A counter-based SplitMix64 (Steele, Lea and Flood, "Fast
splittable pseudorandom number generators", OOPSLA 2014) keyed by
(seed, tensor id, element index) gives 64-bit words; two words give two
uniforms in (0, 1) and one standard normal by the Box-Muller transform (Box and
Muller, 1958): z = sqrt(-2 ln u1) * cos(2 pi u2).
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os
from typing import Dict, List

import numpy as np

WEIGHT_SEED = 1
LATENT_SEED = 2
INIT_STD = 0.02
AR1_RHO = 0.9


@dataclasses.dataclass(frozen=True)
class DecoderConfig:
    """Shape of one decoder and of the latent video it decodes.

    latent_c/h/w: C', H', W' of one latent frame.
    patch:        p, the PixelUnshuffle factor folded into channels (1 or 2).
    d_model, n_heads, head_dim, mlp_dim, n_layers: Transformer sizes.
    window:       W_frm, latent frames held in the rolling KV cache.
    out_t, out_patch, out_c: each token emits out_t x P x P x out_c pixels.
    frames:       T', latent frames in the synthetic video.
    bf16_weights: weights are rounded to bf16 once, for both sides.
    latents:      "iid" (N(0,1) per element) or "ar1" (rho = 0.9 in time).
    """
    name: str
    latent_c: int
    latent_h: int
    latent_w: int
    patch: int
    d_model: int
    n_heads: int
    head_dim: int
    mlp_dim: int
    n_layers: int
    window: int
    out_t: int
    out_patch: int
    out_c: int
    frames: int
    bf16_weights: bool
    latents: str = "iid"
    ln_eps: float = 1e-5
    # The paper's block ([FD] §3.2 "Base Architecture"); the defaults give the
    # simplified block (LayerNorm, one KV head per query head, no KV-norm, no
    # positions).
    n_kv_heads: int = 0          # G KV heads (grouped-query attention); 0 = n_heads
    norm: str = "layer"          # "layer" (LayerNorm) or "rms" (RMSNorm)
    kv_norm: bool = False        # RMS-normalise every K and V head vector
    rope: bool = False           # 3D rotary positions on Q and K
    rope_theta: float = 10000.0
    # The temporal-first upsampling tail ([FD] §3.4).  0 refinement blocks
    # gives the single linear unpatchify.  With n_refine > 0, out_t is the
    # temporal factor r_t and out_patch the spatial factor r_s: a D -> r_t D
    # linear, n_refine blocks over the r_t N sub-frame tokens, then a 2-layer
    # MLP D -> up_hidden -> r_s^2 out_c and a PixelShuffle per sub-frame.
    n_refine: int = 0
    up_hidden: int = 0           # hidden width of the spatial MLP; 0 = d_model
    # Independent video streams the GPU decodes together (stream b takes the
    # latents of seed LATENT_SEED + b); the oracle decodes each on its own.
    batch: int = 1

    # ---- derived sizes -------------------------------------------------
    @property
    def kv_heads(self) -> int:
        return self.n_kv_heads or self.n_heads

    @property
    def qkv_dim(self) -> int:
        """Output columns of the QKV projection: Q, then K, then V heads."""
        return (self.n_heads + 2 * self.kv_heads) * self.head_dim

    @property
    def tok_h(self) -> int:
        return self.latent_h // self.patch

    @property
    def tok_w(self) -> int:
        return self.latent_w // self.patch

    @property
    def n_tokens(self) -> int:
        """L_frm: spatial tokens per latent frame."""
        return self.tok_h * self.tok_w

    @property
    def c_in(self) -> int:
        """Channels per token after the PixelUnshuffle fold."""
        return self.latent_c * self.patch * self.patch

    @property
    def c_out(self) -> int:
        """Pixel values one token emits."""
        return self.out_t * self.out_patch * self.out_patch * self.out_c

    @property
    def up_dim(self) -> int:
        """Hidden width of the tail's spatial MLP."""
        return self.up_hidden or self.d_model

    @property
    def sub_c_out(self) -> int:
        """Pixel values one sub-frame token of the tail emits: r_s^2 out_c."""
        return self.out_patch * self.out_patch * self.out_c

    @property
    def n_sub_tokens(self) -> int:
        """Tokens of one latent frame after temporal upsampling: r_t N."""
        return self.out_t * self.n_tokens

    @property
    def pix_h(self) -> int:
        return self.tok_h * self.out_patch

    @property
    def pix_w(self) -> int:
        return self.tok_w * self.out_patch

    @property
    def latent_shape(self):
        return (self.latent_c, self.latent_h, self.latent_w)

    @property
    def pixel_shape(self):
        return (self.out_t, self.pix_h, self.pix_w, self.out_c)

    def replace(self, **kw) -> "DecoderConfig":
        return dataclasses.replace(self, **kw)


def _big(name, c, h, w, p, layers, frames, latents="iid"):
    return DecoderConfig(name=name, latent_c=c, latent_h=h, latent_w=w, patch=p,
                         d_model=1024, n_heads=16, head_dim=64, mlp_dim=4096,
                         n_layers=layers, window=2, out_t=4, out_patch=16,
                         out_c=3, frames=frames, bf16_weights=True,
                         latents=latents)


CONFIGS: Dict[str, DecoderConfig] = {
    # Tiny fp32 smoke case: 64 tokens of 16 channels, one block.
    "tiny": DecoderConfig(name="tiny", latent_c=16, latent_h=8, latent_w=8,
                          patch=1, d_model=64, n_heads=4, head_dim=16,
                          mlp_dim=256, n_layers=1, window=2, out_t=4,
                          out_patch=8, out_c=3, frames=5, bf16_weights=False),
    # 480p Wan2.1 latent (8x spatial): 60x104x16, 2x2 unshuffle -> 1560 tokens.
    "480p": _big("480p", 16, 60, 104, 2, 16, 21),
    # 720p Wan2.2 latent (16x spatial): 45x80x48 -> 3600 tokens.
    "720p": _big("720p", 48, 45, 80, 1, 24, 21),
    # 1080p Wan2.2 latent: 68x120x48 -> 8160 tokens, 7 latent frames.
    "1080p": _big("1080p", 48, 68, 120, 1, 24, 7),
    # Long stream at 1080p: 241 temporally correlated latent frames.
    "1080p_long": _big("1080p_long", 48, 68, 120, 1, 24, 241, latents="ar1"),
    # The paper's FlashDecoder-XL backbone ([FD] §4.5 "Model Scaling": D = 1536,
    # 20 blocks, 24 heads in 3 KV groups; §3.2 RMSNorm, KV-norm, 3D-RoPE) on
    # the 720p Wan2.2 latent; MLP width 4 D (not given on the pages).  The
    # temporal refinement blocks and upsampler are not part of this path.
    "xl_720p": DecoderConfig(name="xl_720p", latent_c=48, latent_h=45, latent_w=80,
                             patch=1, d_model=1536, n_heads=24, head_dim=64,
                             mlp_dim=6144, n_layers=20, window=2, out_t=4,
                             out_patch=16, out_c=3, frames=21, bf16_weights=True,
                             n_kv_heads=3, norm="rms", kv_norm=True, rope=True),
    # The whole FlashDecoder-XL decoder ([FD] §4.5: 20 backbone blocks and 2
    # temporal refinement blocks) with the temporal-first upsampling tail of
    # [FD] §3.4 (r_t = 4, r_s = 16) on the same 720p latent.  Spatial MLP
    # hidden width D (not given on the pages).
    "xl_720p_tr": DecoderConfig(name="xl_720p_tr", latent_c=48, latent_h=45,
                                latent_w=80, patch=1, d_model=1536, n_heads=24,
                                head_dim=64, mlp_dim=6144, n_layers=20, window=2,
                                out_t=4, out_patch=16, out_c=3, frames=21,
                                bf16_weights=True, n_kv_heads=3, norm="rms",
                                kv_norm=True, rope=True, n_refine=2),
    # Eight independent 480p streams decoded together ([FD] §3.3: the KV
    # cache scales with the batch B; data-parallel decode of B videos).
    "480p_x8": _big("480p_x8", 16, 60, 104, 2, 16, 21).replace(batch=8),
}


# --------------------------------------------------------------------------
# Counter-based SplitMix64 + Box-Muller
# --------------------------------------------------------------------------
_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def _mix64(z: np.ndarray) -> np.ndarray:
    """SplitMix64 output finaliser (Steele et al. 2014), elementwise, mod 2^64."""
    z = (z ^ (z >> np.uint64(30))) * _M1
    z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def _stream_key(seed: int, tensor_id: int) -> np.uint64:
    with np.errstate(over="ignore"):
        k = _mix64(np.array([np.uint64(seed) * _GOLDEN], dtype=np.uint64))
        k = _mix64(k ^ np.array([np.uint64(tensor_id + 1) * _M2], dtype=np.uint64))
    return k[0]


def standard_normal(seed: int, tensor_id: int, count: int,
                    start: int = 0) -> np.ndarray:
    """`count` standard normals (float64) of stream (seed, tensor_id).

    Element i uses the SplitMix64 words at counters 2i+1 and 2i+2 of the stream;
    `start` skips the first elements, so any slice can be drawn on its own.
    """
    key = _stream_key(seed, tensor_id)
    out = np.empty(count, dtype=np.float64)
    chunk = 1 << 22
    scale = 2.0 ** -53
    with np.errstate(over="ignore"):
        for s in range(0, count, chunk):
            e = min(count, s + chunk)
            idx = np.arange(start + s, start + e, dtype=np.uint64)
            c1 = key + (np.uint64(2) * idx + np.uint64(1)) * _GOLDEN
            c2 = key + (np.uint64(2) * idx + np.uint64(2)) * _GOLDEN
            u1 = ((_mix64(c1) >> np.uint64(11)).astype(np.float64) + 0.5) * scale
            u2 = ((_mix64(c2) >> np.uint64(11)).astype(np.float64) + 0.5) * scale
            out[s:e] = np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * math.pi * u2)
    return out


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); float32 out.

    Inputs are finite here (normals of bounded magnitude), so no NaN/Inf case.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    bits = (bits + np.uint64(0x7FFF) + ((bits >> np.uint64(16)) & np.uint64(1)))
    bits = (bits & np.uint64(0xFFFF0000)).astype(np.uint32)
    return bits.view(np.float32)


# --------------------------------------------------------------------------
# Weights
# --------------------------------------------------------------------------
LAYER_TENSORS = ("ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_o", "b_o",
                 "ln2_g", "ln2_b", "w_1", "b_1", "w_2", "b_2", "kn_g", "vn_g")
GLOBAL_TENSORS = ("w_in", "b_in", "lnf_g", "lnf_b", "w_out", "b_out")
# Parameters of the temporal-first upsampling tail (only with n_refine > 0):
# temporal linear D -> r_t D, the norm after the refinement blocks, and the
# spatial MLP D -> up_hidden -> r_s^2 out_c.
TAIL_TENSORS = ("w_tu", "b_tu", "lnr_g", "lnr_b", "w_s1", "b_s1", "w_s2", "b_s2")


def weight_shapes(cfg: DecoderConfig) -> Dict[str, tuple]:
    """Shapes of every parameter; Linear weights are [out][in]."""
    D, F = cfg.d_model, cfg.mlp_dim
    return {
        "w_in": (D, cfg.c_in), "b_in": (D,),
        "ln1_g": (D,), "ln1_b": (D,),
        "w_qkv": (cfg.qkv_dim, D), "b_qkv": (cfg.qkv_dim,),
        "kn_g": (cfg.head_dim,), "vn_g": (cfg.head_dim,),
        "w_o": (D, D), "b_o": (D,),
        "ln2_g": (D,), "ln2_b": (D,),
        "w_1": (F, D), "b_1": (F,),
        "w_2": (D, F), "b_2": (D,),
        "lnf_g": (D,), "lnf_b": (D,),
        "w_out": (cfg.c_out, D), "b_out": (cfg.c_out,),
        "w_tu": (cfg.out_t * D, D), "b_tu": (cfg.out_t * D,),
        "lnr_g": (D,), "lnr_b": (D,),
        "w_s1": (cfg.up_dim, D), "b_s1": (cfg.up_dim,),
        "w_s2": (cfg.sub_c_out, cfg.up_dim), "b_s2": (cfg.sub_c_out,),
    }


# Stream ids: backbone globals 0.., backbone block l at 64 + 16 l, tail
# globals 50000.., refinement block r at 60000 + 16 r (latents use 1e6 + t).
def _tensor_id(name: str, layer: int) -> int:
    if layer < 0:
        if name in TAIL_TENSORS:
            return 50000 + TAIL_TENSORS.index(name)
        return GLOBAL_TENSORS.index(name)
    if layer >= _REFINE_BASE:
        return 60000 + (layer - _REFINE_BASE) * 16 + LAYER_TENSORS.index(name)
    return 64 + layer * 16 + LAYER_TENSORS.index(name)


_REFINE_BASE = 1 << 12     # layer index of refinement block 0 in the draw jobs


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _draw(cfg: DecoderConfig, name: str, layer: int, seed: int) -> np.ndarray:
    shape = weight_shapes(cfg)[name]
    z = standard_normal(seed, _tensor_id(name, layer), int(np.prod(shape)))
    v = INIT_STD * z
    if name.endswith("_g"):          # LayerNorm gain: 1 + N(0, 0.02^2)
        v = 1.0 + v
    v = v.astype(np.float32).reshape(shape)
    if cfg.bf16_weights:
        v = round_to_bf16(v)
    return v


def make_weights(cfg: DecoderConfig, seed: int = WEIGHT_SEED) -> dict:
    """All decoder parameters as float32 numpy arrays.

    Linear weights and biases ~ N(0, 0.02^2); norm gains ~ 1 + N(0, 0.02^2)
    and shifts ~ N(0, 0.02^2) (shifts are unused with RMSNorm).  With KV-norm
    each layer also has gains kn_g, vn_g [head_dim].  For bf16 workloads every
    value is rounded to bf16 once here, so both sides consume identical values.
    Returns {"w_in", "b_in", "lnf_g", "lnf_b", "w_out", "b_out",
             "layers": [ {ln1_g, ..., b_2[, kn_g, vn_g]} per layer ]}, and with
    n_refine > 0 also the tail: "w_tu", "b_tu", "lnr_g", "lnr_b", "w_s1",
    "b_s1", "w_s2", "b_s2" and "refine": [ per refinement block, as layers ].
    Adding the tail leaves every backbone tensor unchanged.
    """
    layer_tensors = [n for n in LAYER_TENSORS if cfg.kv_norm or n not in ("kn_g", "vn_g")]
    jobs = [(n, -1) for n in GLOBAL_TENSORS]
    jobs += [(n, l) for l in range(cfg.n_layers) for n in layer_tensors]
    if cfg.n_refine:
        jobs += [(n, -1) for n in TAIL_TENSORS]
        jobs += [(n, _REFINE_BASE + r) for r in range(cfg.n_refine) for n in layer_tensors]
    # Tensors are independent streams; numpy releases the GIL in the ufuncs,
    # so a thread pool only changes the wall time, never the values.
    with concurrent.futures.ThreadPoolExecutor(_threads()) as pool:
        vals = list(pool.map(lambda j: _draw(cfg, j[0], j[1], seed), jobs))
    got = dict(zip(jobs, vals))
    w = {n: got[(n, -1)] for n in GLOBAL_TENSORS}
    w["layers"] = [{n: got[(n, l)] for n in layer_tensors}
                   for l in range(cfg.n_layers)]
    if cfg.n_refine:
        for n in TAIL_TENSORS:
            w[n] = got[(n, -1)]
        w["refine"] = [{n: got[(n, _REFINE_BASE + r)] for n in layer_tensors}
                       for r in range(cfg.n_refine)]
    return w


# --------------------------------------------------------------------------
# Latents
# --------------------------------------------------------------------------
def _noise_frame(cfg: DecoderConfig, t: int, seed: int) -> np.ndarray:
    n = int(np.prod(cfg.latent_shape))
    return standard_normal(seed, 1_000_000 + t, n).reshape(cfg.latent_shape)


def make_batched_latents(cfg: DecoderConfig, frames: int | None = None) -> List[np.ndarray]:
    """Latent frames of all cfg.batch streams: frame t is [B][C'][H'][W'],
    stream b drawn as make_latents(seed = LATENT_SEED + b)."""
    per = [make_latents(cfg, frames, seed=LATENT_SEED + b) for b in range(cfg.batch)]
    return [np.stack([p[t] for p in per]) for t in range(len(per[0]))]


def make_latents(cfg: DecoderConfig, frames: int | None = None,
                 seed: int = LATENT_SEED) -> List[np.ndarray]:
    """Latent frames z_0..z_{T'-1}, each float32 [C'][H'][W'].

    "iid": z_t ~ N(0, 1) elementwise.
    "ar1": x_0 = e_0, x_t = rho x_{t-1} + sqrt(1 - rho^2) e_t with rho = 0.9,
           which keeps unit variance while correlating consecutive frames.
    """
    frames = cfg.frames if frames is None else frames
    out = []
    prev = None
    for t in range(frames):
        e = _noise_frame(cfg, t, seed)
        if cfg.latents == "ar1" and prev is not None:
            x = AR1_RHO * prev + math.sqrt(1.0 - AR1_RHO * AR1_RHO) * e
        else:
            x = e
        prev = x
        out.append(x.astype(np.float32))
    return out
