"""Pins of the CPU oracle (no GPU).

Sources: [FD] "FlashDecoder: Real-Time Latent-to-Pixel Streaming Decoder with
Transformers" (academ.us/article/2607.14898).  The pages print no worked
numeric example, so the oracle is pinned by library routines, closed forms,
invariants and the brute-force masked formulation.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from oracle_checks import (
    check_attention, check_attention_uniform, check_gelu, check_gqa_attention,
    check_identity_blocks_closed_form, check_kv_norm, check_layer_norm,
    check_linear, check_patchify, check_rms_norm, check_rope_complex,
    check_rope_frequencies, check_rope_relative, check_rope_token_positions,
    check_stream_equals_bruteforce,
    check_uniform_attention_closed_form, check_unpatchify,
    check_unpatchify_bijective, rel_l2, small_cfg, small_paper_cfg, stream,
    check_tail_identity_closed_form, small_tail_cfg)

F64 = 1e-12


# ---------------------------------------------------------------- primitives
@pytest.mark.parametrize("p", [1, 2])
def test_patchify_is_pixel_unshuffle(p):
    # [FD] §4.3: PixelUnshuffle folds p x p space into channels; §3.2 Eq. 1:
    # raster-order tokens.
    assert check_patchify(p) == 0.0


def test_unpatchify_is_pixel_shuffle():
    # [FD] §3.4 Step 3: PixelShuffle after the projection.
    assert check_unpatchify() == 0.0


def test_unpatchify_writes_every_pixel_once():
    assert check_unpatchify_bijective() == 0.0


def test_linear():
    assert check_linear() < F64


def test_layer_norm():
    assert check_layer_norm() < F64


def test_gelu_exact_erf():
    assert check_gelu() < F64


@pytest.mark.parametrize("masked", [False, True])
def test_attention_matches_sdpa(masked):
    assert check_attention(masked) < F64


def test_attention_uniform_scores_give_mean_of_v():
    assert check_attention_uniform() < F64


# -------------------------------------------------------- streaming decoder
STREAM_CASES = [
    dict(),                                         # W = 2, 3 blocks
    dict(window=1),                                 # frames independent
    dict(window=3),
    dict(window=8, frames=6),                       # W >= T': growing cache
    dict(latent_h=1, latent_w=1),                   # N = 1
    dict(latent_h=2, latent_w=2, frames=8),         # N = 4
    dict(latent_h=4, latent_w=4, frames=8, n_layers=2),   # N = 16
    dict(patch=2, latent_h=4, latent_w=8),          # 2x2 unshuffle
    dict(n_heads=1, head_dim=32),
]


@pytest.mark.parametrize("kw", STREAM_CASES)
def test_streaming_equals_bruteforce_masked_pass(kw):
    # [FD] §3.3: frame-by-frame decoding with the rolling cache computes the
    # sliding-window pattern that a full-sequence pass needs a mask for.
    assert check_stream_equals_bruteforce(small_cfg(**kw)) < 1e-12


def test_tiny_workload_streaming_equals_bruteforce():
    assert check_stream_equals_bruteforce(W.CONFIGS["tiny"]) < 1e-12


@pytest.mark.parametrize("window", [1, 2, 3])
def test_causality_future_frames_do_not_matter(window):
    # [FD] §3.3: future frames are never fed, so causality holds by
    # construction; perturbing frames after t leaves frames <= t unchanged.
    cfg = small_cfg(window=window)
    w = W.make_weights(cfg)
    zs = W.make_latents(cfg)
    base = stream(cfg, w, zs)
    bf_base = oracle.bruteforce_decode(cfg, w, zs)
    for t in range(cfg.frames - 1):
        zp = [z.copy() for z in zs]
        for u in range(t + 1, cfg.frames):
            zp[u] = zp[u] + 1.0
        got = stream(cfg, w, zp)
        bf = oracle.bruteforce_decode(cfg, w, zp)
        for u in range(t + 1):
            assert np.array_equal(got[u], base[u])
            assert np.array_equal(bf[u], bf_base[u])
        assert not np.array_equal(got[t + 1], base[t + 1])


@pytest.mark.parametrize("window", [1, 2, 3])
def test_cache_size_is_constant(window):
    # [FD] §3.3 Eq. 2: the cache holds at most W_frm frames.
    cfg = small_cfg(window=window, frames=9)
    dec = oracle.StreamingDecoder(cfg, W.make_weights(cfg))
    shapes = set()
    for t, z in enumerate(W.make_latents(cfg)):
        dec.decode_frame(z)
        n = min(t + 1, window)
        for l in range(cfg.n_layers):
            assert dec.cached_frames(l) == list(range(t + 1 - n, t + 1))
        if t >= window - 1:
            shapes.add(tuple(sum(e[1].size for e in c) for c in dec.cache))
    assert len(shapes) == 1


def test_frame0_attends_only_to_itself():
    # Frame 0 has no predecessor: it equals a W = 1 decode and a one-frame
    # full-sequence pass.
    cfg = small_cfg()
    w = W.make_weights(cfg)
    zs = W.make_latents(cfg)
    a = stream(cfg, w, zs[:1])[0]
    b = stream(cfg.replace(window=1), w, zs[:1])[0]
    c = oracle.bruteforce_decode(cfg, w, zs[:1])[0]
    assert np.array_equal(a, b)
    assert rel_l2(a, c) < 1e-13


def test_reset_restarts_the_stream():
    cfg = small_cfg()
    w = W.make_weights(cfg)
    zs = W.make_latents(cfg)
    dec = oracle.StreamingDecoder(cfg, w)
    first = [dec.decode_frame(z) for z in zs[:3]]
    dec.reset()
    again = [dec.decode_frame(z) for z in zs[:3]]
    for a, b in zip(first, again):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("n_layers", [1, 2, 3])
def test_finite_receptive_field(n_layers):
    # Each block adds one frame of look-back: frame t depends on latents
    # t - L .. t only, so a fresh decoder started at t - L reproduces it
    # exactly, and one started at t - L + 1 does not.
    cfg = small_cfg(n_layers=n_layers, frames=7)
    w = W.make_weights(cfg)
    zs = W.make_latents(cfg)
    full = stream(cfg, w, zs)
    t = cfg.frames - 1
    fresh = stream(cfg, w, zs[t - n_layers:])
    assert np.array_equal(fresh[-1], full[t])
    short = stream(cfg, w, zs[t - n_layers + 1:])
    assert not np.allclose(short[-1], full[t], rtol=0, atol=1e-9)


def test_static_video_gives_identical_frames():
    # Repeated keys leave a softmax unchanged: if z_t = z_0 for every t,
    # every frame decodes like frame 0.
    cfg = small_cfg()
    w = W.make_weights(cfg)
    z0 = W.make_latents(cfg)[0]
    outs = stream(cfg, w, [z0] * cfg.frames)
    for o in outs[1:]:
        assert rel_l2(o, outs[0]) < 1e-13


@pytest.mark.parametrize("kw", [dict(), dict(window=3), dict(n_layers=1)])
def test_uniform_attention_closed_form(kw):
    assert check_uniform_attention_closed_form(small_cfg(**kw)) < 1e-12


@pytest.mark.parametrize("kw", [dict(), dict(patch=2, latent_h=4, latent_w=8)])
def test_identity_blocks_closed_form(kw):
    assert check_identity_blocks_closed_form(small_cfg(**kw)) < 1e-12


def test_permutation_equivariance():
    # No positional encoding: permuting the spatial positions of every frame
    # the same way permutes the output patches the same way (patch = 1).
    cfg = small_cfg()
    w = W.make_weights(cfg)
    zs = W.make_latents(cfg)
    rng = np.random.default_rng(0)
    perm = rng.permutation(cfg.n_tokens)
    zp = [z.reshape(cfg.latent_c, -1)[:, perm].reshape(z.shape) for z in zs]
    a = stream(cfg, w, zs)
    b = stream(cfg, w, zp)
    P = cfg.out_patch
    for x, y in zip(a, b):
        tx = x.reshape(cfg.out_t, cfg.tok_h, P, cfg.tok_w, P, cfg.out_c)
        tx = tx.transpose(1, 3, 0, 2, 4, 5).reshape(cfg.n_tokens, -1)
        ty = y.reshape(cfg.out_t, cfg.tok_h, P, cfg.tok_w, P, cfg.out_c)
        ty = ty.transpose(1, 3, 0, 2, 4, 5).reshape(cfg.n_tokens, -1)
        assert rel_l2(ty, tx[perm]) < 1e-12


# ------------------------------------------------------------- generators
def test_generator_is_standard_normal():
    x = W.standard_normal(3, 5, 200_000)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01
    assert abs((x ** 4).mean() - 3) < 0.05
    assert np.array_equal(W.standard_normal(3, 5, 10, start=7), x[7:17])


def test_bf16_rounding_is_nearest_even():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9,
                     -2.5 - 2 ** -8], dtype=np.float32)
    exp = np.array([1.0, 1.0, 1.0 + 2 ** -6, 1.0, -2.5], dtype=np.float32)
    assert np.array_equal(W.round_to_bf16(vals), exp)


def test_ar1_latents_correlated_unit_variance():
    cfg = W.CONFIGS["1080p_long"].replace(latent_c=4, latent_h=32, latent_w=32)
    zs = W.make_latents(cfg, frames=4)
    for a, b in zip(zs, zs[1:]):
        assert abs(np.corrcoef(a.ravel(), b.ravel())[0, 1] - 0.9) < 0.02
        assert abs(b.std() - 1.0) < 0.03


# ------------------------------------------------------- the paper's block
def test_rms_norm_matches_torch():
    # [FD] §3.2: RMSNorm before each sublayer.
    assert check_rms_norm() < F64


@pytest.mark.parametrize("n_kv", [1, 2, 3, 6])
def test_grouped_query_attention_matches_sdpa(n_kv):
    # [FD] §3.2 / Eq. 2: G KV heads shared by groups of query heads.
    assert check_gqa_attention(n_kv) < F64


def test_kv_norm_closed_form():
    assert check_kv_norm() < F64


def test_rope_is_complex_rotation():
    assert check_rope_complex() < F64


def test_rope_scores_depend_on_position_differences_only():
    # Why window-relative and absolute temporal positions agree ([FD] §4.3).
    assert check_rope_relative() < 1e-9


def test_rope_frequencies_are_the_logspace_of_the_reading():
    # [FD] §3.2 3D-RoPE; head dims (24, 20, 20), theta = 1e4: pair k of a part
    # of d dims turns by pos theta^(-2k/d).
    assert check_rope_frequencies() < F64


def test_rope_token_rows_and_columns():
    # [FD] §3.2 Eq. 1 raster order: token n of a 4 x 6 grid sits at row n // 6,
    # column n % 6; checked against hand-written (n, i, j).
    assert check_rope_token_positions() < F64


def test_rope_split_of_head_dims():
    assert oracle.rope_split(64) == (24, 20, 20)
    assert oracle.rope_split(16) == (8, 4, 4)
    assert oracle.rope_split(12) == (4, 4, 4)


@pytest.mark.parametrize("kw", [dict(), dict(window=1), dict(window=4),
                                dict(n_kv_heads=1), dict(n_kv_heads=4),
                                dict(rope=False), dict(kv_norm=False), dict(norm="layer")])
def test_paper_block_streaming_equals_bruteforce(kw):
    # Streaming rotates cached keys at window-relative positions; the masked
    # full-sequence pass uses absolute frame indices.
    assert check_stream_equals_bruteforce(small_paper_cfg(**kw)) < 1e-12


def test_paper_block_defaults_leave_the_simplified_block_unchanged():
    cfg = small_cfg()
    w = W.make_weights(cfg)
    zs = W.make_latents(cfg, frames=3)
    a = stream(cfg, w, zs)
    b = stream(cfg.replace(n_kv_heads=cfg.n_heads, norm="layer", kv_norm=False,
                           rope=False), w, zs)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


# ------------------------------------------- the temporal-first upsampling tail
def small_paper_tail_cfg(**kw):
    base = dict(n_layers=2, n_refine=2, up_hidden=24)
    base.update(kw)
    return small_paper_cfg(**base)


@pytest.mark.parametrize("kw", [dict(), dict(window=1), dict(window=3), dict(n_refine=1),
                                dict(out_t=3), dict(patch=2, latent_h=4, latent_w=8)])
def test_tail_streaming_equals_bruteforce(kw):
    # [FD] §3.4 Step 2: the refinement blocks use the streaming mechanism of
    # §3.3 with a window of r_t W_frm sub-frames; the masked full-sequence
    # pass over all T' r_t N sub-frame tokens must agree.
    assert check_stream_equals_bruteforce(small_tail_cfg(**kw)) < F64


@pytest.mark.parametrize("kw", [dict(), dict(window=3), dict(n_kv_heads=1), dict(out_t=3)])
def test_paper_tail_streaming_equals_bruteforce(kw):
    # With rotary positions the streaming side rotates at window-relative
    # sub-frame positions r_t f + k; the masked pass at absolute r_t t + k.
    assert check_stream_equals_bruteforce(small_paper_tail_cfg(**kw)) < F64


@pytest.mark.parametrize("kw", [dict(), dict(norm="rms"), dict(out_t=3, out_patch=1)])
def test_tail_identity_blocks_closed_form(kw):
    # Temporal linear, channel-to-time reading, norm, spatial MLP and
    # PixelShuffle against torch and einops (every block adding zero).
    assert check_tail_identity_closed_form(small_tail_cfg(**kw)) < F64


def test_tail_finite_receptive_field():
    # Backbone and refinement blocks each look one latent frame back (W = 2):
    # frame t depends on latents t - (L + R) .. t only.
    cfg = small_tail_cfg(n_layers=2, n_refine=2, frames=7)
    w = W.make_weights(cfg)
    zs = W.make_latents(cfg)
    full = stream(cfg, w, zs)
    t, reach = cfg.frames - 1, cfg.n_layers + cfg.n_refine
    assert np.array_equal(stream(cfg, w, zs[t - reach:])[-1], full[t])
    short = stream(cfg, w, zs[t - reach + 1:])[-1]
    assert not np.allclose(short, full[t], rtol=0, atol=1e-9)


@pytest.mark.parametrize("window", [1, 2, 3])
def test_tail_cache_holds_window_latent_frames_of_subframe_tokens(window):
    # [FD] §3.2 (scaling paragraph): refinement layers cache r_t W_frm L_frm
    # tokens, i.e. W latent frames of r_t N sub-frame tokens.
    cfg = small_tail_cfg(window=window, frames=6)
    dec = oracle.StreamingDecoder(cfg, W.make_weights(cfg))
    for t, z in enumerate(W.make_latents(cfg)):
        dec.decode_frame(z)
        n = min(t + 1, window)
        for l in range(cfg.n_layers + cfg.n_refine):
            assert dec.cached_frames(l) == list(range(t + 1 - n, t + 1))
        for r in range(cfg.n_refine):
            k, v = dec.cached_kv(cfg.n_layers + r, t)
            assert k.shape == v.shape == (cfg.out_t * cfg.n_tokens, cfg.kv_heads * cfg.head_dim)


def test_tail_causality_and_frame0():
    cfg = small_tail_cfg()
    w = W.make_weights(cfg)
    zs = W.make_latents(cfg)
    base = stream(cfg, w, zs)
    zp = [z.copy() for z in zs]
    zp[3] = zp[3] + 1.0
    got = stream(cfg, w, zp)
    assert all(np.array_equal(got[u], base[u]) for u in range(3))
    assert not np.array_equal(got[3], base[3])
    assert np.array_equal(stream(cfg.replace(window=1), w, zs[:1])[0], base[0])
    assert base[0].shape == (cfg.out_t, cfg.pix_h, cfg.pix_w, cfg.out_c)
