"""Write sampled full-size expected pixels from the CPU oracle.

Calls only `oracle` and `workloads`: no value here comes from the GPU path.
For each workload, the oracle decodes latent frames 0, 1 and 2 (frame 0 sees
itself only; frame 1 fills the W = 2 window; frame 2 is the first frame that
evicts), and the file keeps, per frame,
  * `idx_t{t}`: flat indices into the [out_t][H][W][out_c] pixel frame: 8192
    seeded random pixels plus every pixel of 4 whole tokens (the first, the
    last, and two seeded random ones),
  * `val_t{t}`: the oracle's pixels there (float64 computed, stored float32),
  * `l2_t{t}`, `mean_t{t}`: norm and mean of the oracle's whole frame.

Usage: python tests/golden/make_golden.py [workload ...]   (default: all
full-size workloads).  Runtime is minutes per 1080p frame on a few cores.

Late frames of a long stream: `--tail WORKLOAD T` writes WORKLOAD_tT.npz with
the same samples of latent frame T (keys `idx_tail`, `val_tail`, `l2_tail`,
`mean_tail`, `tail_frame`).  Each block looks one frame back, so frame T
depends on latents T-L .. T only (L blocks, refinement blocks included): a
fresh oracle stream over those L+1 latents gives frame T exactly, without
decoding frames 0 .. T-L-1.
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads as W  # noqa: E402

FRAMES = 3
N_RANDOM = 8192


def token_pixel_indices(cfg, n: int) -> np.ndarray:
    i, j = divmod(n, cfg.tok_w)
    P = cfg.out_patch
    tau, dy, dx, c = np.meshgrid(np.arange(cfg.out_t), np.arange(P), np.arange(P),
                                 np.arange(cfg.out_c), indexing="ij")
    flat = ((tau * cfg.pix_h + i * P + dy) * cfg.pix_w + j * P + dx) * cfg.out_c + c
    return flat.ravel()


def sample_indices(cfg, t: int) -> np.ndarray:
    rng = np.random.default_rng(1000 + t)
    total = int(np.prod(cfg.pixel_shape))
    toks = [0, cfg.n_tokens - 1] + list(rng.integers(0, cfg.n_tokens, 2))
    idx = [rng.integers(0, total, N_RANDOM)]
    idx += [token_pixel_indices(cfg, int(n)) for n in toks]
    return np.concatenate(idx).astype(np.int64)


def make(name: str) -> str:
    cfg = W.CONFIGS[name]
    t0 = time.time()
    weights = W.make_weights(cfg)
    latents = W.make_latents(cfg, frames=FRAMES)
    dec = oracle.StreamingDecoder(cfg, weights)
    out = {"workload": np.array(name), "frames": np.array(FRAMES)}
    for t in range(FRAMES):
        pix = dec.decode_frame(latents[t]).ravel()
        idx = sample_indices(cfg, t)
        out[f"idx_t{t}"] = idx
        out[f"val_t{t}"] = pix[idx].astype(np.float32)
        out[f"l2_t{t}"] = np.array(np.linalg.norm(pix))
        out[f"mean_t{t}"] = np.array(pix.mean())
        print(f"{name} frame {t} done at {time.time() - t0:.0f}s", flush=True)
    path = os.path.join(HERE, f"{name}.npz")
    np.savez_compressed(path, **out)
    return path


def make_tail(name: str, t_last: int) -> str:
    cfg = W.CONFIGS[name]
    t0 = time.time()
    weights = W.make_weights(cfg)
    latents = W.make_latents(cfg, frames=t_last + 1)
    first = t_last - (cfg.n_layers + cfg.n_refine)
    assert first >= 0
    dec = oracle.StreamingDecoder(cfg, weights)
    for t in range(first, t_last + 1):
        pix = dec.decode_frame(latents[t])
        print(f"{name} tail: latent {t} done at {time.time() - t0:.0f}s", flush=True)
    pix = pix.ravel()
    idx = sample_indices(cfg, t_last)
    out = {"workload": np.array(name), "tail_frame": np.array(t_last),
           "idx_tail": idx, "val_tail": pix[idx].astype(np.float32),
           "l2_tail": np.array(np.linalg.norm(pix)), "mean_tail": np.array(pix.mean())}
    path = os.path.join(HERE, f"{name}_t{t_last}.npz")
    np.savez_compressed(path, **out)
    return path


if __name__ == "__main__":
    if len(sys.argv) == 4 and sys.argv[1] == "--tail":
        print(make_tail(sys.argv[2], int(sys.argv[3])), flush=True)
        sys.exit(0)
    names = sys.argv[1:] or ["480p", "720p", "1080p", "1080p_long"]
    for n in names:
        print(make(n), flush=True)
