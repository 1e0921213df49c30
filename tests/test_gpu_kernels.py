"""Per-step kernels against the oracle's primitives on the same bf16 inputs.

Each test rounds its inputs to bf16 exactly as the device path consumes them
and compares with the oracle's float64 step (oracle.linear / gelu /
layer_norm / attention).
"""
import math

import numpy as np
import pytest

import oracle
import transformer_latent_pixel_amd as fd
import workloads as W
from gpu_util import bf16_bits, bits_to_f64, dev, say, torch_cuda

pytestmark = pytest.mark.gpu


def _rand(seed, tid, shape, scale=1.0):
    return scale * W.standard_normal(seed, tid, int(np.prod(shape))).reshape(shape)


GEMM_SHAPES = [
    (64, 64, 64),         # 64x64 tiles, single tile
    (300, 192, 64),       # ragged M
    (1, 64, 128),         # one row
    (2000, 1024, 512),    # 64x128 tiles, three workgroups per CU
    (2000, 6144, 256),    # 128x256 tiles of 8 waves, ragged last M tile
    (2000, 2048, 320),    # one round of 128x128 tiles (8 waves), 10 K steps of a 4-stage ring
    (2000, 2048, 64),     # 2 K steps: the prologue re-fetches the last one
    (2000, 2048, 2048),   # one round of 128x128 tiles, long K
    (3600, 1536, 512),    # 128x128 tiles of 8 waves over more than one round
    (130, 256, 128),      # 64x128 tiles: the last tile's second wave has no row < m
    (3600, 1024, 4096),   # 128x128 tiles, 8 waves: the 720p FC2 shape (ragged last row band)
    (8160, 1024, 1024),   # one round of 128x256 tiles: 8 waves of 64x64 (1080p out-projection)
]


@pytest.mark.parametrize("m,n,k", GEMM_SHAPES)
@pytest.mark.parametrize("epi", [0, 1, 2])
def test_gemm(m, n, k, epi):
    torch = torch_cuda()
    say(f"gemm epi={epi} m={m} n={n} k={k}")
    rows = (m + 255) // 256 * 256
    a = _rand(11, 1, (rows, k))
    b = _rand(11, 2, (n, k), 0.05)
    bias = _rand(11, 3, (n,), 0.1).astype(np.float32)
    ab, bb = bf16_bits(a), bf16_bits(b)
    ref = oracle.linear(bits_to_f64(ab)[:m], bits_to_f64(bb), bias.astype(np.float64))
    init = _rand(11, 4, (m, n)).astype(np.float32)
    if epi == 2:
        out = torch.zeros((m, n), dtype=torch.int16, device="cuda")
    else:
        out = dev(init if epi == 1 else np.zeros((m, n), np.float32))
    fd.fdk_gemm(epi, dev(ab.view(np.int16)), dev(bb.view(np.int16)), dev(bias), out,
                m, rows, n, k)
    torch.cuda.synchronize()
    if epi == 2:
        got = bits_to_f64(out.cpu().numpy().view(np.uint16))
        ref = oracle.gelu(ref)
        tol = 2.0 ** -8 * np.abs(ref) + 1e-5
    else:
        got = out.cpu().numpy().astype(np.float64)
        if epi == 1:
            ref = ref + init
        tol = 1e-5 * (1.0 + np.abs(ref))
    err = np.abs(got - ref)
    assert (err <= tol).all(), f"max err {err.max()} at {np.unravel_index(err.argmax(), err.shape)}"


@pytest.mark.parametrize("m,d", [(1, 64), (300, 1536), (3600, 1536), (77, 192)])
def test_rmsnorm(m, d):
    torch = torch_cuda()
    say(f"rmsnorm m={m} d={d}")
    x = (_rand(17, 1, (m, d), 2.0) + 0.5).astype(np.float32)
    g = (1.0 + _rand(17, 2, (d,), 0.1)).astype(np.float32)
    out = torch.zeros((m, d), dtype=torch.int16, device="cuda")
    fd.fdk_layernorm(dev(x), m, d, dev(g), None, 1e-5, out, rms=True)
    torch.cuda.synchronize()
    got = bits_to_f64(out.cpu().numpy().view(np.uint16))
    ref = oracle.rms_norm(x.astype(np.float64), g.astype(np.float64), 1e-5)
    err = np.abs(got - ref)
    assert (err <= 2.0 ** -8 * np.abs(ref) + 1e-4).all(), err.max()


@pytest.mark.parametrize("m,d", [(1, 64), (300, 64), (1000, 1024), (8160, 1024), (77, 192)])
def test_layernorm(m, d):
    torch = torch_cuda()
    say(f"layernorm m={m} d={d}")
    x = (_rand(12, 1, (m, d), 2.0) + 0.5).astype(np.float32)
    g = (1.0 + _rand(12, 2, (d,), 0.1)).astype(np.float32)
    b = _rand(12, 3, (d,), 0.1).astype(np.float32)
    out = torch.zeros((m, d), dtype=torch.int16, device="cuda")
    fd.fdk_layernorm(dev(x), m, d, dev(g), dev(b), 1e-5, out)
    torch.cuda.synchronize()
    got = bits_to_f64(out.cpu().numpy().view(np.uint16))
    ref = oracle.layer_norm(x.astype(np.float64), g.astype(np.float64),
                            b.astype(np.float64), 1e-5)
    err = np.abs(got - ref)
    assert (err <= 2.0 ** -8 * np.abs(ref) + 1e-4).all(), err.max()


ATTN_CASES = [
    # heads, n, hd, n_frames, first_slot
    (2, 300, 64, 1, 0),
    (2, 300, 64, 2, 0),
    (2, 300, 64, 2, 1),        # slot order rotated: oldest frame in slot 1
    (2, 300, 64, 3, 2),
    (1, 64, 64, 2, 0),
    (3, 1000, 64, 2, 1),
    (4, 64, 16, 2, 1),          # small head dim (one thread per query)
    (2, 37, 32, 2, 0),
    (3, 130, 32, 3, 2),         # head_dim 32, three frames, rotated slots
    (16, 1560, 64, 2, 1),       # 480p shape: 4 key splits
    (16, 3600, 64, 2, 1),       # 720p shape: 2 key splits, ragged last key tile
    (1, 64, 64, 1, 0),          # one key tile
    # >= 256 workgroups of 512 queries
    (32, 4000, 64, 2, 1),       # ragged last key tile
    (64, 1600, 64, 1, 0),       # one cached frame, whole tiles
    (44, 2600, 64, 3, 2),       # three frames, rotated slots, ragged
    (2, 1, 64, 2, 1),           # one token per frame: 63 of 64 keys padding
    (3, 1, 16, 3, 0),           # one token, head_dim 16
]


def test_gemm_with_no_rows_writes_nothing():
    # m = 0 (an empty token set): the call succeeds and leaves the output alone.
    torch = torch_cuda()
    a = dev(bf16_bits(_rand(11, 1, (256, 64))).view(np.int16))
    b = dev(bf16_bits(_rand(11, 2, (64, 64))).view(np.int16))
    bias = dev(np.zeros(64, np.float32))
    out = dev(np.full((4, 64), 7.0, np.float32))
    for epi in (0, 1):
        fd.fdk_gemm(epi, a, b, bias, out, 0, 256, 64, 64)
    torch.cuda.synchronize()
    assert (out.cpu().numpy() == 7.0).all()


@pytest.mark.parametrize("heads,n,hd,nf,first", ATTN_CASES)
def test_attention(heads, n, hd, nf, first):
    torch = torch_cuda()
    say(f"attention heads={heads} n={n} hd={hd} frames={nf} first_slot={first}")
    fold = math.log2(math.e) / math.sqrt(hd)
    q = _rand(13, 1, (heads, n, hd), 1.5)
    k = _rand(13, 2, (nf, heads, n, hd), 1.5)
    v = _rand(13, 3, (nf, heads, n, hd))
    qb, kb, vb = bf16_bits(q * fold), bf16_bits(k), bf16_bits(v)
    out = torch.zeros((n, heads * hd), dtype=torch.int16, device="cuda")
    fd.fdk_attention(dev(qb.view(np.int16)), dev(kb.view(np.int16)), dev(vb.view(np.int16)),
                     nf, first, heads, n, hd, out)
    got = bits_to_f64(out.cpu().numpy().view(np.uint16))
    # Undo the folding: natural-unit scores are (q*fold).k * ln 2.
    q_nat = bits_to_f64(qb) * math.log(2.0) * math.sqrt(hd)
    qf = q_nat.transpose(1, 0, 2).reshape(n, heads * hd)
    kf = bits_to_f64(kb).transpose(0, 2, 1, 3).reshape(nf * n, heads * hd)
    vf = bits_to_f64(vb).transpose(0, 2, 1, 3).reshape(nf * n, heads * hd)
    ref = oracle.attention(qf, kf, vf, heads)
    err = np.abs(got - ref)
    # Q and K are exact bf16, so the scores are exact to fp32 accumulation.
    # Rounding each weight p_j to bf16 (relative 2^-9, the row sum taken over
    # the same rounded weights) moves O_i by at most 2^-9 max_j |v_j - O_i|;
    # rounding O to bf16 adds 2^-9 |O_i|.
    vmax = np.abs(vf).max(axis=0)
    tol = 2.0 ** -9 * (1.01 * (vmax + np.abs(ref)) + np.abs(ref)) + 1e-4
    assert (err <= tol).all(), f"max err {err.max()}, worst err/tol {(err / tol).max()}"
    assert np.linalg.norm(got - ref) / np.linalg.norm(ref) < 5e-3


@pytest.mark.parametrize("heads,n,nf,splits", [(1, 64, 1, 4), (2, 100, 1, 4), (3, 300, 2, 3)])
def test_attention_forced_key_splits(heads, n, nf, splits):
    # More splits than key tiles leaves some splits empty (frame 0 of a small
    # input); their partials carry zero weight in the merge.
    torch = torch_cuda()
    hd = 64
    say(f"attention forced splits heads={heads} n={n} frames={nf} splits={splits}")
    fold = math.log2(math.e) / math.sqrt(hd)
    q = _rand(19, 1, (heads, n, hd), 1.5)
    k = _rand(19, 2, (nf, heads, n, hd), 1.5)
    v = _rand(19, 3, (nf, heads, n, hd))
    qb, kb, vb = bf16_bits(q * fold), bf16_bits(k), bf16_bits(v)
    out = torch.zeros((n, heads * hd), dtype=torch.int16, device="cuda")
    fd.fdk_attention(dev(qb.view(np.int16)), dev(kb.view(np.int16)), dev(vb.view(np.int16)),
                     nf, 0, heads, n, hd, out, splits=splits)
    got = bits_to_f64(out.cpu().numpy().view(np.uint16))
    q_nat = bits_to_f64(qb) * math.log(2.0) * math.sqrt(hd)
    qf = q_nat.transpose(1, 0, 2).reshape(n, heads * hd)
    kf = bits_to_f64(kb).transpose(0, 2, 1, 3).reshape(nf * n, heads * hd)
    vf = bits_to_f64(vb).transpose(0, 2, 1, 3).reshape(nf * n, heads * hd)
    ref = oracle.attention(qf, kf, vf, heads)
    err = np.abs(got - ref)
    vmax = np.abs(vf).max(axis=0)
    tol = 2.0 ** -9 * (1.01 * (vmax + np.abs(ref)) + np.abs(ref)) + 1e-4
    assert (err <= tol).all(), f"max err {err.max()}, worst err/tol {(err / tol).max()}"


@pytest.mark.parametrize("heads,n,nf,splits", [(4, 300, 2, 3), (16, 3600, 2, 0)])
def test_attention_split_partials_keep_large_values(heads, n, nf, splits):
    # Split partials are stored as fp16, whose range ends at 65504.  V entries
    # around 2^20 (head 0 and every other head) put the normalised partials far
    # past it; the other heads keep V near 1, so both storage paths run in one
    # launch.  splits = 0 is the decoder's own choice (two splits at 3600).
    torch = torch_cuda()
    hd = 64
    say(f"attention large V heads={heads} n={n} frames={nf} splits={splits}")
    fold = math.log2(math.e) / math.sqrt(hd)
    q = _rand(23, 1, (heads, n, hd), 1.5)
    k = _rand(23, 2, (nf, heads, n, hd), 1.5)
    v = _rand(23, 3, (nf, heads, n, hd))
    v[:, 0::2] *= 2.0 ** 20
    qb, kb, vb = bf16_bits(q * fold), bf16_bits(k), bf16_bits(v)
    out = torch.zeros((n, heads * hd), dtype=torch.int16, device="cuda")
    fd.fdk_attention(dev(qb.view(np.int16)), dev(kb.view(np.int16)), dev(vb.view(np.int16)),
                     nf, 1, heads, n, hd, out, splits=splits)
    got = bits_to_f64(out.cpu().numpy().view(np.uint16))
    q_nat = bits_to_f64(qb) * math.log(2.0) * math.sqrt(hd)
    qf = q_nat.transpose(1, 0, 2).reshape(n, heads * hd)
    kf = bits_to_f64(kb).transpose(0, 2, 1, 3).reshape(nf * n, heads * hd)
    vf = bits_to_f64(vb).transpose(0, 2, 1, 3).reshape(nf * n, heads * hd)
    ref = oracle.attention(qf, kf, vf, heads)
    assert np.abs(ref[:, :hd]).max() > 2.0 ** 17        # head 0's partials pass fp16's range
    assert np.isfinite(got).all()
    err = np.abs(got - ref)
    vmax = np.abs(vf).max(axis=0)
    tol = 2.0 ** -9 * (1.01 * (vmax + np.abs(ref)) + np.abs(ref)) + 1e-4
    assert (err <= tol).all(), f"max err {err.max()}, worst err/tol {(err / tol).max()}"


@pytest.mark.parametrize("heads,n", [(2, 1000), (32, 4000)])
def test_attention_rising_scores(heads, n):
    # Key norms grow along the sequence, so later key tiles score far above
    # the earlier ones (about 20 log2 units): the weights of late tiles are
    # large relative to the first tile's, within the range in which the
    # running max stays put.  One split (32 x 4000) and several (2 x 1000).
    torch = torch_cuda()
    hd, nf = 64, 2
    say(f"attention rising scores heads={heads} n={n}")
    fold = math.log2(math.e) / math.sqrt(hd)
    q = _rand(15, 1, (heads, n, hd), 1.0)
    ramp = (0.1 + 6.0 * np.arange(nf * n) / (nf * n)).reshape(nf, 1, n, 1)
    k = _rand(15, 2, (nf, heads, n, hd), 1.0) * ramp
    v = _rand(15, 3, (nf, heads, n, hd))
    qb, kb, vb = bf16_bits(q * fold), bf16_bits(k), bf16_bits(v)
    out = torch.zeros((n, heads * hd), dtype=torch.int16, device="cuda")
    fd.fdk_attention(dev(qb.view(np.int16)), dev(kb.view(np.int16)), dev(vb.view(np.int16)),
                     nf, 1, heads, n, hd, out)
    got = bits_to_f64(out.cpu().numpy().view(np.uint16))
    q_nat = bits_to_f64(qb) * math.log(2.0) * math.sqrt(hd)
    qf = q_nat.transpose(1, 0, 2).reshape(n, heads * hd)
    kf = bits_to_f64(kb).transpose(0, 2, 1, 3).reshape(nf * n, heads * hd)
    vf = bits_to_f64(vb).transpose(0, 2, 1, 3).reshape(nf * n, heads * hd)
    ref = oracle.attention(qf, kf, vf, heads)
    err = np.abs(got - ref)
    vmax = np.abs(vf).max(axis=0)
    tol = 2.0 ** -9 * (1.01 * (vmax + np.abs(ref)) + np.abs(ref)) + 1e-4
    assert (err <= tol).all(), f"max err {err.max()}, worst err/tol {(err / tol).max()}"


@pytest.mark.parametrize("heads,n,mixed", [(2, 1000, False), (32, 4000, False),
                                           (2, 1000, True), (32, 4000, True)])
def test_attention_extreme_scores_move_the_running_max(heads, n, mixed):
    # Queries share one direction u (|u| = 8).  The oldest frame's keys point
    # against it (scores near -80 in log2 units, beyond the range in which
    # the running max may stay at 0), the newest frame's keys along it
    # (scores near +80, weights near 2^160 relative to the first tiles), so
    # the max is set on the first tile and moved up later, with the score
    # offset applied by the extra MFMA chunk: the workgroups of those heads
    # run their tiles a second time with the per-tile check.  mixed: only
    # the even heads have such scores (the odd heads' u has norm 1.5, scores
    # within a few log2 units), so the two kinds of workgroup run side by
    # side.
    torch = torch_cuda()
    hd, nf = 64, 2
    say(f"attention extreme scores heads={heads} n={n} mixed={mixed}")
    fold = math.log2(math.e) / math.sqrt(hd)
    u = _rand(16, 0, (heads, 1, hd))
    norm = np.where(np.arange(heads) % 2 == 1, 1.5, 8.0) if mixed else np.full(heads, 8.0)
    u = norm.reshape(heads, 1, 1) * u / np.linalg.norm(u, axis=-1, keepdims=True)
    q = u + 0.3 * _rand(16, 1, (heads, n, hd))
    sign = np.array([-1.0, 1.0]).reshape(nf, 1, 1, 1)
    k = sign * 7.0 * u[None] + 0.5 * _rand(16, 2, (nf, heads, n, hd))
    v = _rand(16, 3, (nf, heads, n, hd))
    qb, kb, vb = bf16_bits(q * fold), bf16_bits(k), bf16_bits(v)
    out = torch.zeros((n, heads * hd), dtype=torch.int16, device="cuda")
    fd.fdk_attention(dev(qb.view(np.int16)), dev(kb.view(np.int16)), dev(vb.view(np.int16)),
                     nf, 0, heads, n, hd, out)
    got = bits_to_f64(out.cpu().numpy().view(np.uint16))
    q_nat = bits_to_f64(qb) * math.log(2.0) * math.sqrt(hd)
    qf = q_nat.transpose(1, 0, 2).reshape(n, heads * hd)
    kf = bits_to_f64(kb).transpose(0, 2, 1, 3).reshape(nf * n, heads * hd)
    vf = bits_to_f64(vb).transpose(0, 2, 1, 3).reshape(nf * n, heads * hd)
    ref = oracle.attention(qf, kf, vf, heads)
    s0 = (bits_to_f64(qb)[0, :64] @ bits_to_f64(kb)[0, 0, :64].T).max()
    s1 = (bits_to_f64(qb)[0, :64] @ bits_to_f64(kb)[1, 0, :64].T).max()
    assert s0 < -64 and s1 > 64, (s0, s1)        # log2-unit scores of the test's intent
    err = np.abs(got - ref)
    vmax = np.abs(vf).max(axis=0)
    tol = 2.0 ** -9 * (1.01 * (vmax + np.abs(ref)) + np.abs(ref)) + 1e-4
    assert (err <= tol).all(), f"max err {err.max()}, worst err/tol {(err / tol).max()}"


@pytest.mark.parametrize("heads,kv,n,nf,first", [
    (8, 2, 300, 2, 1),          # 4 query heads per KV head, 4 key splits
    (6, 1, 1000, 2, 0),         # one KV head for every query head
    (24, 3, 3600, 2, 1),        # the XL block at 720p: 2 key splits
    (32, 8, 4000, 3, 2),        # one split, three frames
])
def test_attention_grouped_query(heads, kv, n, nf, first):
    # [FD] §3.2: grouped-query attention, KV head floor(j kv / heads).
    torch = torch_cuda()
    hd = 64
    say(f"attention gqa heads={heads} kv={kv} n={n} frames={nf}")
    fold = math.log2(math.e) / math.sqrt(hd)
    q = _rand(18, 1, (heads, n, hd), 1.5)
    k = _rand(18, 2, (nf, kv, n, hd), 1.5)
    v = _rand(18, 3, (nf, kv, n, hd))
    qb, kb, vb = bf16_bits(q * fold), bf16_bits(k), bf16_bits(v)
    out = torch.zeros((n, heads * hd), dtype=torch.int16, device="cuda")
    fd.fdk_attention(dev(qb.view(np.int16)), dev(kb.view(np.int16)), dev(vb.view(np.int16)),
                     nf, first, heads, n, hd, out, kv_heads=kv)
    got = bits_to_f64(out.cpu().numpy().view(np.uint16))
    q_nat = bits_to_f64(qb) * math.log(2.0) * math.sqrt(hd)
    qf = q_nat.transpose(1, 0, 2).reshape(n, heads * hd)
    kf = bits_to_f64(kb).transpose(0, 2, 1, 3).reshape(nf * n, kv * hd)
    vf = bits_to_f64(vb).transpose(0, 2, 1, 3).reshape(nf * n, kv * hd)
    ref = oracle.attention(qf, kf, vf, heads, n_kv_heads=kv)
    err = np.abs(got - ref)
    vmax = np.repeat(np.abs(vf).max(axis=0).reshape(kv, hd), heads // kv, axis=0).ravel()
    tol = 2.0 ** -9 * (1.01 * (vmax + np.abs(ref)) + np.abs(ref)) + 1e-4
    assert (err <= tol).all(), f"max err {err.max()}, worst err/tol {(err / tol).max()}"


def test_attention_uniform_scores_average_every_cached_key():
    # q = 0: every valid key has the same score, so each output row is the
    # mean of V over exactly n_frames * n keys.
    torch = torch_cuda()
    heads, n, hd, nf = 2, 200, 64, 2
    v = _rand(14, 1, (nf, heads, n, hd))
    vb = bf16_bits(v)
    zeros = np.zeros((heads, n, hd), np.uint16)
    kb = bf16_bits(_rand(14, 2, (nf, heads, n, hd)))
    out = torch.zeros((n, heads * hd), dtype=torch.int16, device="cuda")
    fd.fdk_attention(dev(zeros.view(np.int16)), dev(kb.view(np.int16)),
                     dev(vb.view(np.int16)), nf, 1, heads, n, hd, out)
    got = bits_to_f64(out.cpu().numpy().view(np.uint16))
    mean = bits_to_f64(vb).mean(axis=(0, 2))            # [heads][hd]
    ref = np.broadcast_to(mean.reshape(1, heads * hd), got.shape)
    assert np.abs(got - ref).max() < 2.0 ** -8 * np.abs(ref).max() + 1e-3


def test_mfma_probe_runs_and_reads_the_clock():
    # The measurement probe: zero operands sum to exactly zero, random ones
    # to finite values, and every wave's shader clock lies between 0.3 and
    # 3 GHz (the counters are read around its loop).
    torch = torch_cuda()
    wgs = fd.capi.PROBE_WORKGROUPS
    sink = torch.full((wgs * 512,), float("nan"), device="cuda")
    clocks = torch.zeros(wgs * 8 * 2, dtype=torch.int64, device="cuda")
    for zero in (True, False):
        fd.fdk_mfma_probe(zero, 2000, sink, clocks)
        torch.cuda.synchronize()
        s = sink.cpu().numpy()
        assert np.isfinite(s).all()
        if zero:
            assert (s == 0.0).all()
        c = clocks.view(-1, 2).cpu().numpy().astype(np.float64)
        assert (c > 0).all()
        ghz = c[:, 0] / c[:, 1] * 0.1
        say(f"probe zero={zero}: shader clock {ghz.min():.2f}..{ghz.max():.2f} GHz")
        assert ((ghz > 0.3) & (ghz < 3.0)).all()
