"""Pixel error of FP8 (e4m3) MLP GEMMs, computed with the oracle.

[FD] §4.6 "Inference Optimization" item (4) quantizes every MLP layer to FP8
with static calibration on H100.  This script measures what that costs on the
seeded workloads against the decode tolerance (pixels within max abs 3e-2
and relative L2 1e-2 of the exact decode): the float64 oracle decodes the
same frames twice, once exact and once with the operands of the MLP products
rounded to e4m3, and the pixels are compared.

Variants: FC1 only, FC2 only, both; each with
  per-tensor scales  x ~ e4m3(x s) / s, s = 448 / max|x| of the whole operand
                     (the best a single static scale can do), and
  block scales       per 32 consecutive elements along K, the smallest power
                     of two 2^e with max|x_block| / 2^e <= 448 (an E8M0
                     shared scale of the OCP microscaling format, which
                     gfx950's scaled FP8 matrix instructions take per 32
                     elements of K; chosen so that no element is clipped).
e4m3 is the OCP 8-bit float with 4 exponent bits (bias 7) and 3 mantissa
bits, largest finite 448, rounded to nearest even (torch.float8_e4m3fn).

Usage: python tests/fp8_mlp_study.py [--workload 480p] [--frames 2] [--layers N]
Writes one line per variant.  Calls only the oracle and the workload
generators.
"""
from __future__ import annotations

import argparse
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))

import oracle  # noqa: E402
import workloads as W  # noqa: E402

E4M3_MAX = 448.0


def e4m3(x: np.ndarray) -> np.ndarray:
    """Round to the nearest e4m3 value (ties to even); |x| <= 448 expected."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).to(torch.float64).numpy()


def per_tensor(x: np.ndarray) -> np.ndarray:
    amax = float(np.abs(x).max())
    if amax == 0.0:
        return x.copy()
    s = E4M3_MAX / amax
    return e4m3(np.clip(x * s, -E4M3_MAX, E4M3_MAX)) / s


def block32(x: np.ndarray) -> np.ndarray:
    """E8M0 scale per 32 elements of the last axis (K)."""
    k = x.shape[-1]
    assert k % 32 == 0
    b = x.reshape(x.shape[:-1] + (k // 32, 32))
    amax = np.abs(b).max(axis=-1, keepdims=True)
    e = np.ceil(np.log2(np.where(amax > 0, amax, 1.0) / E4M3_MAX))
    scale = np.exp2(e)
    q = e4m3(np.clip(b / scale, -E4M3_MAX, E4M3_MAX)) * scale
    return q.reshape(x.shape)


VARIANTS = {
    "fc1 per-tensor": ({"fc1_act", "fc1_w"}, per_tensor),
    "fc2 per-tensor": ({"fc2_act", "fc2_w"}, per_tensor),
    "fc1+fc2 per-tensor": ({"fc1_act", "fc1_w", "fc2_act", "fc2_w"}, per_tensor),
    "fc1 block32": ({"fc1_act", "fc1_w"}, block32),
    "fc2 block32": ({"fc2_act", "fc2_w"}, block32),
    "fc1+fc2 block32": ({"fc1_act", "fc1_w", "fc2_act", "fc2_w"}, block32),
}


def hook(names, fn):
    return lambda name, x: fn(x) if name in names else x


def study(cfg, frames: int, variants=VARIANTS, log=print):
    """{variant: (max abs, rel L2)} over frames 0..frames-1 of cfg's stream."""
    weights = W.make_weights(cfg)
    zs = W.make_latents(cfg, frames=frames)
    t0 = time.perf_counter()
    ref = oracle.StreamingDecoder(cfg, weights)
    exact = [ref.decode_frame(z) for z in zs]
    log(f"# {cfg.name}, {cfg.n_layers} blocks, frames 0..{frames - 1}: exact decode "
        f"{time.perf_counter() - t0:.1f} s")
    out = {}
    for name, (names, fn) in variants.items():
        dec = oracle.StreamingDecoder(cfg, weights, mlp_operands=hook(names, fn))
        ma = rl = 0.0
        for z, e in zip(zs, exact):
            p = dec.decode_frame(z)
            ma = max(ma, float(np.abs(p - e).max()))
            rl = max(rl, float(np.linalg.norm(p - e) / np.linalg.norm(e)))
        ok = ma <= 3e-2 and rl <= 1e-2
        out[name] = (ma, rl)
        log(f"{name:22s} max_abs {ma:.3e}  rel_l2 {rl:.3e}  {'meets' if ok else 'fails'} "
            f"3e-2 / 1e-2")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="480p")
    ap.add_argument("--frames", type=int, default=2)
    ap.add_argument("--layers", type=int, default=0, help="override the block count")
    a = ap.parse_args()
    cfg = W.CONFIGS[a.workload]
    if a.layers:
        cfg = cfg.replace(n_layers=a.layers)
    study(cfg, a.frames)


if __name__ == "__main__":
    main()
