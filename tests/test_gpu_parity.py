"""Full decode on the GPU against the CPU oracle, plus ring bookkeeping.

Tolerance on pixels: max abs error <= 3e-2 and relative L2 error <= 1e-2
(bf16 operands, fp32 accumulation).  Ring bookkeeping is compared exactly.
"""
import os

import numpy as np
import pytest

import oracle
import transformer_latent_pixel_amd as fd
import workloads as W
from gpu_util import (PIX_MAX_ABS, PIX_REL_L2, GpuStream, bits_to_f64,
                      cached_weights, max_abs, multi_tile_cfg, rel_l2, say)

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def _compare_stream(cfg, weights=None, frames=None):
    weights = weights if weights is not None else W.make_weights(cfg)
    zs = W.make_latents(cfg, frames=frames)
    ref = oracle.StreamingDecoder(cfg, weights)
    g = GpuStream(cfg, weights)
    try:
        for t, z in enumerate(zs):
            got = g.frame(z)
            exp = ref.decode_frame(z)
            ma, rl = max_abs(got, exp), rel_l2(got, exp)
            say(f"{cfg.name} t={t} max_abs={ma:.3e} rel_l2={rl:.3e}")
            assert ma <= PIX_MAX_ABS and rl <= PIX_REL_L2, (t, ma, rl)
    finally:
        g.close()


def test_tiny_workload_matches_oracle():
    _compare_stream(W.CONFIGS["tiny"])


@pytest.mark.parametrize("kw", [
    dict(),
    dict(window=1),
    dict(window=3, frames=5),
    dict(patch=2, latent_c=16, latent_h=20, latent_w=30),   # 150 tokens, 2x2 fold
    dict(latent_h=16, latent_w=16, n_layers=1),             # 256 tokens, no tail
    dict(latent_h=1, latent_w=5, n_layers=1),               # 5 tokens
])
def test_multi_tile_decoder_matches_oracle(kw):
    _compare_stream(multi_tile_cfg(**kw))


# The paper's block ([FD] §3.2): RMSNorm, grouped-query attention, KV-norm,
# 3D rotary positions (temporal positions advance with every frame).
PAPER = dict(n_kv_heads=2, norm="rms", kv_norm=True, rope=True)


@pytest.mark.parametrize("kw", [
    dict(PAPER, frames=5),
    dict(PAPER, window=3, frames=5),
    dict(PAPER, n_kv_heads=1),
    dict(n_kv_heads=2),                                # GQA only
    dict(norm="rms", kv_norm=True),                    # norms only
    dict(rope=True, frames=5),                         # rotary positions only
    dict(PAPER, latent_h=16, latent_w=16, n_layers=1), # 256 tokens, no tail
])
def test_paper_block_decoder_matches_oracle(kw):
    _compare_stream(multi_tile_cfg(**kw))


def test_paper_block_large_qkv_tiles_match_oracle():
    # 8160 tokens, QKV 2048 columns: the 128x256 QKV tile, two heads per wave.
    cfg = multi_tile_cfg(latent_h=68, latent_w=120, d_model=1024, n_heads=16,
                         n_kv_heads=8, norm="rms", kv_norm=True, rope=True,
                         n_layers=1, frames=3)
    _compare_stream(cfg)


# The temporal-first upsampling tail ([FD] §3.4): a D -> r_t D linear, refinement
# blocks over the r_t N sub-frame tokens (1200 for 300 spatial tokens), and the
# spatial MLP with a PixelShuffle per sub-frame.
@pytest.mark.parametrize("kw", [
    dict(n_refine=2, n_layers=1),
    dict(PAPER, n_refine=2, n_layers=1),
    dict(n_refine=1, n_layers=1, out_t=2, up_hidden=128, window=3, frames=5),
    dict(PAPER, n_refine=1, n_layers=1, out_t=3, up_hidden=384),
])
def test_tail_decoder_matches_oracle(kw):
    _compare_stream(multi_tile_cfg(**kw))


def test_tail_ring_contents_match_oracle():
    # A refinement block caches W latent frames of r_t N sub-frame tokens.
    cfg = multi_tile_cfg(n_refine=1, n_layers=1, frames=3)
    weights = W.make_weights(cfg)
    ref = oracle.StreamingDecoder(cfg, weights)
    g = GpuStream(cfg, weights)
    try:
        n4 = cfg.out_t * cfg.n_tokens
        for t, z in enumerate(W.make_latents(cfg)):
            g.frame(z)
            ref.decode_frame(z)
            for kv in (0, 1):
                got = g.dec.debug_read_kv(cfg.n_layers, t % cfg.window, kv)
                exp = ref.cached_kv(cfg.n_layers, t)[kv]
                exp = exp.reshape(n4, cfg.kv_heads, cfg.head_dim).transpose(1, 0, 2)
                err = np.abs(bits_to_f64(got) - exp).max()
                say(f"tail ring t={t} kv={kv} max_err={err:.3e}")
                assert err < 2e-2 * max(1.0, np.abs(exp).max()), (t, kv, err)
    finally:
        g.close()


# B independent streams decoded together: every GEMM and norm runs over the
# B N stacked rows, attention over B x heads heads, each stream on its own
# ring slots; stream b must match its own oracle stream.
def _compare_batched(cfg, weights=None, zs=None):
    weights = weights if weights is not None else W.make_weights(cfg)
    zs = zs if zs is not None else W.make_batched_latents(cfg)
    refs = [oracle.StreamingDecoder(cfg, weights) for _ in range(cfg.batch)]
    g = GpuStream(cfg, weights)
    outs = []
    try:
        for t, z in enumerate(zs):
            got = g.frame(z)
            outs.append(got)
            for b in range(cfg.batch):
                exp = refs[b].decode_frame(z[b])
                ma, rl = max_abs(got[b], exp), rel_l2(got[b], exp)
                say(f"batched t={t} stream={b} max_abs={ma:.3e} rel_l2={rl:.3e}")
                assert ma <= PIX_MAX_ABS and rl <= PIX_REL_L2, (t, b, ma, rl)
            # ring slot of block 0: stream b's KV heads are b G .. b G + G - 1
            kv = g.dec.debug_read_kv(0, t % cfg.window, 0)
            G = cfg.kv_heads
            for b in range(cfg.batch):
                exp = refs[b].cached_kv(0, t)[0]
                if not cfg.rope:
                    exp = exp.reshape(cfg.n_tokens, G, cfg.head_dim).transpose(1, 0, 2)
                    err = np.abs(bits_to_f64(kv[b * G:(b + 1) * G]) - exp).max()
                    assert err < 2e-2 * max(1.0, np.abs(exp).max()), (t, b, err)
    finally:
        g.close()
    return outs


@pytest.mark.parametrize("kw", [
    dict(batch=3),
    dict(PAPER, batch=2),
    dict(batch=2, n_refine=1, n_layers=1),
    dict(PAPER, batch=2, n_refine=1, n_layers=1),
    dict(batch=4, latent_h=16, latent_w=16, n_layers=1),   # 4 x 256 tokens
])
def test_batched_streams_match_oracle(kw):
    _compare_batched(multi_tile_cfg(**kw))


def test_batched_tiny_workload_matches_oracle():
    # head_dim 16: the one-thread-per-query attention kernel with streams.
    _compare_batched(W.CONFIGS["tiny"].replace(batch=3))


def test_largest_window_matches_oracle():
    # W = FD_MAX_WINDOW: eight cached frames, ring slots reused after frame 8.
    _compare_stream(multi_tile_cfg(window=fd.FD_MAX_WINDOW, frames=11, n_layers=1))


def test_batched_streams_are_independent():
    # Changing one stream's latent leaves every other stream bit-identical.
    cfg = multi_tile_cfg(batch=3, frames=3, n_layers=1)
    w = W.make_weights(cfg)
    zs = W.make_batched_latents(cfg)
    g = GpuStream(cfg, w)
    try:
        a = g.run(zs)
        g.dec.reset()
        zp = [z.copy() for z in zs]
        zp[1][1] += 1.0                      # stream 1, frame 1
        b = g.run(zp)
    finally:
        g.close()
    for t in range(cfg.frames):
        assert np.array_equal(a[t][0], b[t][0]) and np.array_equal(a[t][2], b[t][2])
    assert np.array_equal(a[0][1], b[0][1])
    assert not np.array_equal(a[1][1], b[1][1]) and not np.array_equal(a[2][1], b[2][1])


def test_ring_bookkeeping_and_contents_are_exact():
    cfg = multi_tile_cfg(frames=5)
    weights = W.make_weights(cfg)
    zs = W.make_latents(cfg)
    ref = oracle.StreamingDecoder(cfg, weights)
    g = GpuStream(cfg, weights)
    try:
        info = g.dec.query()
        assert info["frames_decoded"] == 0 and info["n_valid"] == 0
        assert info["slot_frame"] == [-1] * cfg.window
        arena = info["arena_bytes"]
        prev = {}
        for t, z in enumerate(zs):
            g.frame(z)
            ref.decode_frame(z)
            info = g.dec.query()
            assert info["arena_bytes"] == arena
            assert info["frames_decoded"] == t + 1
            assert info["n_valid"] == min(t + 1, cfg.window) == len(ref.cached_frames(0))
            held = sorted(f for f in info["slot_frame"] if f >= 0)
            assert held == ref.cached_frames(0)
            assert info["slot_frame"][t % cfg.window] == t
            for layer in range(cfg.n_layers):
                for kv in (0, 1):
                    slot = t % cfg.window
                    got = g.dec.debug_read_kv(layer, slot, kv)
                    exp = ref.cached_kv(layer, t)[kv]
                    exp = exp.reshape(cfg.n_tokens, cfg.n_heads, cfg.head_dim).transpose(1, 0, 2)
                    err = np.abs(bits_to_f64(got) - exp).max()
                    assert err < 2e-2 * max(1.0, np.abs(exp).max()), (t, layer, kv, err)
                    # The other slots are untouched by this frame.
                    for s in range(cfg.window):
                        if s != slot and (layer, s, kv) in prev:
                            assert np.array_equal(g.dec.debug_read_kv(layer, s, kv),
                                                  prev[(layer, s, kv)])
            prev = {(layer, s, kv): g.dec.debug_read_kv(layer, s, kv)
                    for layer in range(cfg.n_layers) for s in range(cfg.window)
                    for kv in (0, 1)}
    finally:
        g.close()


def test_decode_is_deterministic_and_reset_restarts():
    cfg = multi_tile_cfg()
    weights = W.make_weights(cfg)
    zs = W.make_latents(cfg)
    g = GpuStream(cfg, weights)
    try:
        a = g.run(zs)
        g.dec.reset()
        b = g.run(zs)
    finally:
        g.close()
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_finite_receptive_field_is_bit_exact_on_gpu():
    # Frame t depends on latents t-L .. t only: a fresh stream started at t-L
    # reproduces frame t bit for bit (keys are visited oldest first whatever
    # the slot), one started at t-L+1 does not.
    cfg = multi_tile_cfg(frames=6, n_layers=2)
    weights = W.make_weights(cfg)
    zs = W.make_latents(cfg)
    L = cfg.n_layers
    g = GpuStream(cfg, weights)
    try:
        full = g.run(zs)
        for t in (L, L + 1, cfg.frames - 1):
            g.dec.reset()
            fresh = g.run(zs[t - L:t + 1])
            assert np.array_equal(fresh[-1], full[t]), t
            g.dec.reset()
            short = g.run(zs[t - L + 1:t + 1])
            assert not np.array_equal(short[-1], full[t]), t
    finally:
        g.close()


def test_frame0_attends_only_to_itself_on_gpu():
    cfg = multi_tile_cfg()
    weights = W.make_weights(cfg)
    z0 = W.make_latents(cfg, frames=1)[0]
    g2 = GpuStream(cfg, weights)
    g1 = GpuStream(cfg.replace(window=1), weights)
    try:
        assert np.array_equal(g2.frame(z0), g1.frame(z0))
    finally:
        g2.close()
        g1.close()


def test_profile_filter_selects_launches():
    cfg = multi_tile_cfg(n_layers=3)
    weights = W.make_weights(cfg)
    zs = W.make_latents(cfg, frames=2)
    g = GpuStream(cfg, weights)
    try:
        dec = g.dec
        dec.profile_enable(True)
        g.frame(zs[0])
        every = dec.profile_read()
        L = cfg.n_layers
        assert every["attention"]["launches"] == L
        assert every["layernorm"]["launches"] == 2 * L + 1
        assert every["unpatchify"]["launches"] == 1 and every["state"]["launches"] == 1
        dec.profile_filter(["attention"], 1)
        g.frame(zs[1])
        one = dec.profile_read()
        assert one["attention"]["launches"] == 1 and one["attention"]["ms"] > 0
        assert all(v["launches"] == 0 for k, v in one.items() if k != "attention")
        dec.profile_filter(["qkv", "fc1"], -1)
        dec.reset()
        g.frame(zs[0])
        two = dec.profile_read()
        assert two["qkv"]["launches"] == L and two["fc1"]["launches"] == L
        assert two["attention"]["launches"] == 0 and two["state"]["launches"] == 0
    finally:
        g.close()


def test_invalid_arguments_leave_handle_usable():
    cfg = multi_tile_cfg()
    g = GpuStream(cfg, W.make_weights(cfg))
    try:
        lib = fd.load_library()
        assert lib.fd_decode_frame(g.dec.handle, None, g.pix.data_ptr()) == fd.FD_ERR_INVALID_ARG
        assert lib.fd_decode_frame(g.dec.handle, g.pix.data_ptr() + 2,
                                   g.pix.data_ptr()) == fd.FD_ERR_INVALID_ARG
        assert lib.fd_debug_read_kv(g.dec.handle, 99, 0, 0, None, 0) == fd.FD_ERR_INVALID_ARG
        z = W.make_latents(cfg, frames=1)[0]
        g.frame(z)
        assert g.dec.query()["frames_decoded"] == 1
    finally:
        g.close()


def test_create_reports_oom_for_an_arena_beyond_device_memory():
    # 2^20 tokens, D = 2048, 8 blocks, W = 8: the rings alone need about 550 GB.
    # fd_create sizes the arena and compares it with the free device memory
    # before it allocates or reads any weight.
    cfg = W.DecoderConfig(name="huge", latent_c=16, latent_h=1024, latent_w=1024, patch=1,
                          d_model=2048, n_heads=32, head_dim=64, mlp_dim=8192, n_layers=8,
                          window=8, out_t=4, out_patch=16, out_c=3, frames=1,
                          bf16_weights=True)
    assert fd.config_check(cfg) == fd.FD_OK
    D, F = cfg.d_model, cfg.mlp_dim
    def z(shape):                                  # untouched pages: no host memory used
        return np.zeros(shape, np.float32)
    layer = {"ln1_g": z(D), "ln1_b": z(D), "w_qkv": z((3 * D, D)), "b_qkv": z(3 * D),
             "w_o": z((D, D)), "b_o": z(D), "ln2_g": z(D), "ln2_b": z(D),
             "w_1": z((F, D)), "b_1": z(F), "w_2": z((D, F)), "b_2": z(D)}
    weights = {"w_in": z((D, cfg.c_in)), "b_in": z(D), "lnf_g": z(D), "lnf_b": z(D),
               "w_out": z((cfg.c_out, D)), "b_out": z(cfg.c_out),
               "layers": [layer] * cfg.n_layers}
    with pytest.raises(fd.FdError) as e:
        fd.Decoder(cfg, weights)
    assert e.value.status == fd.FD_ERR_OOM


# ----------------------------------------------------- full-size workloads
def _golden(name):
    path = os.path.join(HERE, "golden", f"{name}.npz")
    if not os.path.exists(path):
        pytest.fail(f"missing {path}: run tests/golden/make_golden.py {name}")
    return np.load(path, allow_pickle=False)


def _check_golden(name, got_frames):
    gold = _golden(name)
    for t, got in enumerate(got_frames[:int(gold["frames"])]):
        flat = got.ravel()
        idx, val = gold[f"idx_t{t}"], gold[f"val_t{t}"]
        ma, rl = max_abs(flat[idx], val), rel_l2(flat[idx], val)
        nrm = float(np.linalg.norm(flat.astype(np.float64)))
        say(f"{name} t={t} sampled max_abs={ma:.3e} rel_l2={rl:.3e} "
            f"frame_l2 gpu={nrm:.6e} oracle={float(gold[f'l2_t{t}']):.6e}")
        assert ma <= PIX_MAX_ABS and rl <= PIX_REL_L2, (t, ma, rl)
        assert abs(nrm / float(gold[f"l2_t{t}"]) - 1.0) < PIX_REL_L2
        assert np.isfinite(flat).all()


def _check_tail_golden(name, t_last, got):
    path = os.path.join(HERE, "golden", f"{name}_t{t_last}.npz")
    if not os.path.exists(path):
        pytest.fail(f"missing {path}: run tests/golden/make_golden.py --tail {name} {t_last}")
    gold = np.load(path, allow_pickle=False)
    assert int(gold["tail_frame"]) == t_last
    flat = got.ravel()
    idx, val = gold["idx_tail"], gold["val_tail"]
    ma, rl = max_abs(flat[idx], val), rel_l2(flat[idx], val)
    nrm = float(np.linalg.norm(flat.astype(np.float64)))
    say(f"{name} t={t_last} sampled max_abs={ma:.3e} rel_l2={rl:.3e} "
        f"frame_l2 gpu={nrm:.6e} oracle={float(gold['l2_tail']):.6e}")
    assert ma <= PIX_MAX_ABS and rl <= PIX_REL_L2, (t_last, ma, rl)
    assert abs(nrm / float(gold["l2_tail"]) - 1.0) < PIX_REL_L2
    assert np.isfinite(flat).all()


def test_batched_480p_stream0_matches_480p_samples():
    # Eight 480p streams decoded together: stream 0 takes the latents of the
    # single-stream 480p workload, so it must match that workload's samples.
    cfg = W.CONFIGS["480p_x8"]
    gold = _golden("480p")
    frames = int(gold["frames"])
    g = GpuStream(cfg, cached_weights(W.CONFIGS["480p"]))
    try:
        got = g.run(W.make_batched_latents(cfg, frames=frames))
    finally:
        g.close()
    _check_golden("480p", [x[0] for x in got])
    for b in range(1, cfg.batch):          # the other streams differ and are sane
        assert not np.array_equal(got[0][b], got[0][0])
        assert np.isfinite(got[-1][b]).all()


def test_batched_xl_decoder_stream0_matches_xl_samples():
    # Two streams through the whole XL decoder (GQA, rotary positions, the
    # upsampling tail): stream 0 takes the single-stream latents.
    cfg = W.CONFIGS["xl_720p_tr"].replace(batch=2)
    gold = _golden("xl_720p_tr")
    g = GpuStream(cfg, cached_weights(W.CONFIGS["xl_720p_tr"]))
    try:
        got = g.run(W.make_batched_latents(cfg, frames=int(gold["frames"])))
    finally:
        g.close()
    _check_golden("xl_720p_tr", [x[0] for x in got])
    assert not np.array_equal(got[0][1], got[0][0]) and np.isfinite(got[-1][1]).all()


@pytest.mark.parametrize("name", ["480p", "720p", "1080p", "xl_720p", "xl_720p_tr"])
def test_full_size_workload_matches_oracle_samples(name):
    cfg = W.CONFIGS[name]
    gold = _golden(name)
    frames = int(gold["frames"])
    g = GpuStream(cfg, cached_weights(cfg))
    try:
        got = g.run(W.make_latents(cfg, frames=frames))
    finally:
        g.close()
    _check_golden(name, got)


def test_long_stream_flat_memory_and_latency():
    import torch
    cfg = W.CONFIGS["1080p_long"]
    weights = cached_weights(W.CONFIGS["1080p"])     # same shapes and seed
    zs = W.make_latents(cfg)
    g = GpuStream(cfg, weights)
    try:
        arena = g.dec.query()["arena_bytes"]
        first = []
        times = []
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for t, z in enumerate(zs):
            zt = torch.from_numpy(z).cuda()
            start.record()
            g.dec.decode_frame(zt, g.pix)
            stop.record()
            stop.synchronize()
            times.append(start.elapsed_time(stop))
            if t < 3:
                first.append(g.pix.cpu().numpy())
            if t == len(zs) - 1:
                last = g.pix.cpu().numpy()
            if t % 60 == 0:
                say(f"long stream t={t} ms={times[-1]:.2f}")
        assert g.dec.query()["arena_bytes"] == arena
        assert g.dec.query()["frames_decoded"] == len(zs)
        free1 = torch.cuda.mem_get_info()[0]
        assert abs(free1 - free0) < 64 << 20
        steady = np.array(times[3:])
        early, late = np.median(steady[:40]), np.median(steady[-40:])
        say(f"long stream p50 early={early:.2f} ms late={late:.2f} ms "
            f"p99={np.percentile(steady, 99):.2f} ms")
        assert late < 1.10 * early
        # Receptive field: a fresh stream over the last L+1 latents gives the
        # last frame bit for bit.
        g.dec.reset()
        L = cfg.n_layers
        fresh = g.run(zs[-(L + 1):])
        assert np.array_equal(fresh[-1], last)
    finally:
        g.close()
    _check_golden("1080p_long", first)
    # The last frame against the oracle (which decodes only the L + 1 latents
    # the frame depends on).
    _check_tail_golden("1080p_long", len(zs) - 1, last)
