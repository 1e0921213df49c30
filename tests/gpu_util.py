"""Helpers shared by the GPU tests (device buffers via torch, decode loops)."""
from __future__ import annotations

import functools
import sys

import numpy as np

import workloads as W

PIX_MAX_ABS = 3e-2      # pixel tolerance of the decode against the oracle
PIX_REL_L2 = 1e-2


def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    return torch


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(x: np.ndarray, dtype=None):
    torch = torch_cuda()
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.to("cuda")


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float -> bf16 bit patterns (uint16), round to nearest even."""
    return (W.round_to_bf16(np.asarray(x, np.float32)).view(np.uint32) >> 16).astype(np.uint16)


def bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def max_abs(a, b) -> float:
    return float(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)).max())


@functools.lru_cache(maxsize=4)
def cached_weights(cfg):
    return W.make_weights(cfg)


class GpuStream:
    """Decode a latent sequence on the GPU; returns host float32 pixels."""

    def __init__(self, cfg, weights):
        import transformer_latent_pixel_amd as fd
        self.torch = torch_cuda()
        self.cfg = cfg
        self.dec = fd.Decoder(cfg, weights)
        shape = cfg.pixel_shape if cfg.batch == 1 else (cfg.batch,) + cfg.pixel_shape
        self.pix = self.torch.empty(shape, dtype=self.torch.float32, device="cuda")

    def frame(self, z: np.ndarray) -> np.ndarray:
        zt = dev(np.asarray(z, np.float32))
        self.dec.decode_frame(zt, self.pix)
        self.torch.cuda.synchronize()
        return self.pix.cpu().numpy()

    def run(self, zs):
        return [self.frame(z) for z in zs]

    def close(self):
        self.dec.close()


def multi_tile_cfg(**kw):
    """bf16 decoder spanning several GEMM / attention tiles with ragged tails:
    15 x 20 latents -> 300 tokens (256-row tiles + 44, 64-key tiles + 44)."""
    base = dict(name="multi", latent_c=48, latent_h=15, latent_w=20, patch=1,
                d_model=256, n_heads=4, head_dim=64, mlp_dim=1024, n_layers=2,
                window=2, out_t=4, out_patch=16, out_c=3, frames=4,
                bf16_weights=True)
    base.update(kw)
    return W.DecoderConfig(**base)
