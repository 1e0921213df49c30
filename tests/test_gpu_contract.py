"""The boundary's error contract and the ring's untouched rows, on the GPU.

Device errors are injected from the host (fd_debug_fail_after): the launch
that would fail is never made, so the GPU only ever runs valid work.
"""
import numpy as np
import pytest

import oracle
import transformer_latent_pixel_amd as fd
import workloads as W
from gpu_util import (PIX_MAX_ABS, PIX_REL_L2, GpuStream, max_abs, multi_tile_cfg, rel_l2,
                      say)

pytestmark = pytest.mark.gpu


def test_device_error_breaks_the_handle_and_only_destroy_remains():
    cfg = multi_tile_cfg()
    weights = W.make_weights(cfg)
    zs = W.make_latents(cfg)
    lib = fd.load_library()
    g = GpuStream(cfg, weights)
    try:
        h = g.dec.handle
        first = g.frame(zs[0])
        # Three launches of the next frame go through, the fourth "fails".
        g.dec.debug_fail_after(3)
        z = fd_dev(zs[1])
        assert lib.fd_decode_frame(h, z.data_ptr(), g.pix.data_ptr()) == fd.FD_ERR_DEVICE
        g.torch.cuda.synchronize()                  # the three real launches ran
        assert lib.fd_decode_frame(h, z.data_ptr(), g.pix.data_ptr()) == fd.FD_ERR_STATE
        assert lib.fd_reset(h) == fd.FD_ERR_STATE
        info = fd.capi._Info()
        assert lib.fd_query(h, info) == fd.FD_ERR_STATE
        buf = np.empty(cfg.kv_heads * cfg.n_tokens * cfg.head_dim, np.uint16)
        assert lib.fd_debug_read_kv(h, 0, 0, 0, buf.ctypes.data, buf.size) == fd.FD_ERR_STATE
        ring = np.empty(cfg.kv_heads * 320 * cfg.head_dim, np.uint16)
        assert lib.fd_debug_read_ring(h, 0, 0, 0, ring.ctypes.data, ring.size) == fd.FD_ERR_STATE
        assert lib.fd_debug_poison_ring(h) == fd.FD_ERR_STATE
        # Argument errors are still reported as such on a broken handle.
        assert lib.fd_decode_frame(h, None, g.pix.data_ptr()) == fd.FD_ERR_INVALID_ARG
    finally:
        g.close()                                   # fd_destroy on a broken handle
    # The device is healthy: a new handle decodes the same frame 0.
    g2 = GpuStream(cfg, weights)
    try:
        assert np.array_equal(g2.frame(zs[0]), first)
    finally:
        g2.close()


def test_injection_disarmed_or_counted_past_a_frame_changes_nothing():
    cfg = multi_tile_cfg(n_layers=1)
    weights = W.make_weights(cfg)
    zs = W.make_latents(cfg, frames=3)
    ref = GpuStream(cfg, weights)
    g = GpuStream(cfg, weights)
    try:
        exp = ref.run(zs)
        g.dec.debug_fail_after(10_000)
        got = [g.frame(zs[0])]
        g.dec.debug_fail_after(-1)
        got += g.run(zs[1:])
        for a, b in zip(got, exp):
            assert np.array_equal(a, b)
    finally:
        g.close()
        ref.close()


def fd_dev(z):
    import torch
    return torch.from_numpy(np.ascontiguousarray(z, np.float32)).cuda()


@pytest.mark.parametrize("kw", [dict(), dict(window=3, frames=5),
                                dict(n_refine=1, n_layers=1, frames=3)])
def test_poisoned_unwritten_slots_are_never_read(kw):
    # Every slot's token rows are NaN before frame 0: frame t may only read
    # slots written at frames max(0, t-W+1) .. t ([FD] §3.3), so the pixels
    # are finite and bit-identical to a decode without the poison.
    cfg = multi_tile_cfg(**kw)
    weights = W.make_weights(cfg)
    zs = W.make_latents(cfg)
    clean = GpuStream(cfg, weights)
    g = GpuStream(cfg, weights)
    try:
        exp = clean.run(zs)
        g.dec.debug_poison_ring()
        for t, z in enumerate(zs):
            got = g.frame(z)
            assert np.isfinite(got).all(), t
            assert np.array_equal(got, exp[t]), t
        # And after a reset (the slots still hold the old frames), again.
        g.dec.reset()
        g.dec.debug_poison_ring()
        for t, z in enumerate(zs[:2]):
            assert np.array_equal(g.frame(z), exp[t]), t
    finally:
        g.close()
        clean.close()


def _vt_perm(t):
    return (t & ~12) | ((t & 4) << 1) | ((t & 8) >> 1)


@pytest.mark.parametrize("kw", [dict(), dict(latent_h=1, latent_w=5, n_layers=1),
                                dict(n_refine=1, n_layers=1, frames=3),
                                dict(n_kv_heads=2, norm="rms", kv_norm=True, rope=True)])
def test_ring_padding_rows_are_never_written(kw):
    # A slot holds N token rows padded to a multiple of 64; the padding is
    # zeroed at create and must still be zero after every frame, in K rows and
    # in the V^T columns of padded tokens.
    cfg = multi_tile_cfg(**kw)
    g = GpuStream(cfg, W.make_weights(cfg))
    ref = oracle.StreamingDecoder(cfg, W.make_weights(cfg))
    try:
        blocks = cfg.n_layers + cfg.n_refine
        for t, z in enumerate(W.make_latents(cfg)):
            got = g.frame(z)
            exp = ref.decode_frame(z)
            assert max_abs(got, exp) <= PIX_MAX_ABS and rel_l2(got, exp) <= PIX_REL_L2
            for layer in range(blocks):
                n = cfg.n_tokens * (cfg.out_t if layer >= cfg.n_layers else 1)
                n_pad = (n + 63) // 64 * 64
                pad_cols = [_vt_perm(c) for c in range(n, n_pad)]
                for slot in range(cfg.window):
                    k = g.dec.debug_read_ring(layer, slot, 0)
                    v = g.dec.debug_read_ring(layer, slot, 1)
                    assert k.shape[1] == n_pad and v.shape[2] == n_pad
                    assert not k[:, n:, :].any(), (t, layer, slot)
                    assert not v[:, :, pad_cols].any(), (t, layer, slot)
                    # the token rows of the slot written at this frame are set
                    if slot == t % cfg.window:
                        assert k[:, :n, :].any() and v[:, :, [_vt_perm(c) for c in range(n)]].any()
                    # and the raw read agrees with the unpadded one
                    kv = g.dec.debug_read_kv(layer, slot, 0)
                    assert np.array_equal(kv, k[:, :n, :])
            say(f"ring padding clean after frame {t}")
    finally:
        g.close()
