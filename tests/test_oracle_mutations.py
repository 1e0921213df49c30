"""Planted mistakes in the oracle must fail at least one pin (CPU only).

Each case patches one oracle function with a plausible slip (dropped term,
wrong sign or index, transposed operand) and runs the pins that guard it.
"""
import math

import numpy as np
import pytest
from scipy.special import erf

import oracle
import oracle.decoder as od
from oracle_checks import (
    check_attention, check_gelu, check_gqa_attention,
    check_identity_blocks_closed_form, check_kv_norm, check_layer_norm,
    check_linear, check_patchify, check_rms_norm, check_rope_complex,
    check_rope_frequencies, check_rope_relative, check_rope_token_positions,
    check_stream_equals_bruteforce,
    check_uniform_attention_closed_form, check_unpatchify, small_cfg,
    small_paper_cfg, check_tail_identity_closed_form, small_tail_cfg)

_orig_attn = od._head_attention


def _ln_unbiased(x, g, b, eps):
    mu = x.mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(x.var(axis=-1, ddof=1, keepdims=True) + eps) * g + b


def _ln_no_shift(x, g, b, eps):
    mu = x.mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(((x - mu) ** 2).mean(-1, keepdims=True) + eps) * g


def _gelu_tanh(x):
    return 0.5 * x * (1 + np.tanh(math.sqrt(2 / math.pi) * (x + 0.044715 * x ** 3)))


def _gelu_sign(x):
    return 0.5 * x * (1.0 - erf(x / math.sqrt(2.0)))


def _linear_no_bias(x, w, b):
    return x @ w.T


def _linear_transposed(x, w, b):
    return x @ (w.T if w.shape[0] != w.shape[1] else w) + b


def _attn_wrong_axis(q, k, v, allowed, rows):
    # softmax normalised over the wrong axis
    s = (q @ k.T) / math.sqrt(q.shape[1])
    if allowed is not None:
        s = np.where(allowed, s, -np.inf)
    with np.errstate(invalid="ignore"):
        e = np.exp(s - s.max(axis=0, keepdims=True))
    e = np.where(np.isfinite(e), e, 0.0)
    return (e @ v) / np.maximum(e.sum(axis=1, keepdims=True), 1e-300)


def _patchify_wrong_order(z, p):
    C, H, Wd = z.shape
    x = np.asarray(z, dtype=np.float64).reshape(C, H // p, p, Wd // p, p)
    x = x.transpose(1, 3, 2, 4, 0)            # (dy, dx, c) feature order
    return np.ascontiguousarray(x.reshape((H // p) * (Wd // p), C * p * p))


def _unpatchify_swapped(r, th, tw, T, P, C):
    x = np.asarray(r, dtype=np.float64).reshape(th, tw, T, P, P, C)
    x = x.transpose(2, 0, 4, 1, 3, 5)          # dy and dx swapped
    return np.ascontiguousarray(x.reshape(T, th * P, tw * P, C))


def _mask_off_by_one(frames, n_tok, window):
    f = np.repeat(np.arange(frames), n_tok)
    d = f[:, None] - f[None, :]
    return (d >= 0) & (d <= window)


def _rope_sign(x, angles, head_dim):
    # rotation by -phi instead of +phi
    return _orig_rope(x, -angles, head_dim)


def _rope_half_split(x, angles, head_dim):
    # pairs (k, k + hd/2) instead of consecutive pairs (2k, 2k+1)
    n = x.shape[0]
    h = x.reshape(n, -1, 2, head_dim // 2)
    c, s_ = np.cos(angles)[:, None, :], np.sin(angles)[:, None, :]
    a, b = h[:, :, 0], h[:, :, 1]
    return np.stack([a * c - b * s_, a * s_ + b * c], axis=2).reshape(n, -1)


def _rms_centered(x, g, eps):
    mu = x.mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(((x - mu) ** 2).mean(-1, keepdims=True) + eps) * g


def _kv_norm_across_heads(x, g, head_dim, eps):
    n = x.shape[0]
    h = x.reshape(n, -1, head_dim)
    return (h / np.sqrt((h * h).mean(axis=(1, 2), keepdims=True) + eps) * g).reshape(n, -1)


def _attention_gqa_modulo(q, k, v, n_heads, allowed=None, n_kv_heads=None):
    # query head j reads KV head j mod G instead of floor(j G / heads)
    D = q.shape[1]
    hd = D // n_heads
    G = n_kv_heads or n_heads
    out = np.empty((q.shape[0], D))
    for j in range(n_heads):
        c, g = slice(j * hd, (j + 1) * hd), j % G
        ck = slice(g * hd, (g + 1) * hd)
        out[:, c] = _orig_attn(q[:, c], k[:, ck], v[:, ck], allowed, q.shape[0])
    return out


_orig_rope = od.apply_rope
_orig_tok_angles = od.token_rope_angles


def _subframes_interleaved(p, r_t):
    # channels read as (d, r) instead of (r, d): column c = d r_t + k
    n, c = p.shape
    return p.reshape(n, c // r_t, r_t).transpose(2, 0, 1).reshape(r_t * n, c // r_t)


def _subframe_angles_latent_units(cfg, frame_pos):
    # temporal positions in latent frames (f + k) instead of sub-frames (r_t f + k)
    return np.concatenate([_orig_tok_angles(cfg, frame_pos + k) for k in range(cfg.out_t)])


def _spatial_tokens_minor(cfg, w, hr):
    # sub-frame k read from rows n r_t + k instead of k N + n
    n = cfg.n_tokens
    hr = hr.reshape(cfg.out_t, n, -1).transpose(1, 0, 2).reshape(cfg.out_t * n, -1)
    return _orig_spatial(cfg, w, hr)


_orig_spatial = od.spatial_upsample


def _token_angles_rows_by_height(cfg, frame_pos):
    # row and column of token n taken as n // tok_h, n % tok_h (the grid's
    # height where its width belongs)
    n = np.arange(cfg.n_tokens)
    return od.rope_angles(cfg, np.full(cfg.n_tokens, frame_pos, dtype=np.float64),
                          n // cfg.tok_h, n % cfg.tok_h)


def _token_angles_axes_swapped(cfg, frame_pos):
    # the row index fed to the column rotation and vice versa
    n = np.arange(cfg.n_tokens)
    return od.rope_angles(cfg, np.full(cfg.n_tokens, frame_pos, dtype=np.float64),
                          n % cfg.tok_w, n // cfg.tok_w)


def _rope_angles_half_exponent(cfg, t_pos, i_pos, j_pos):
    # frequency theta^(-k/d) instead of theta^(-2k/d)
    parts = []
    for size, pos in zip(od.rope_split(cfg.head_dim), (t_pos, i_pos, j_pos)):
        k = np.arange(size // 2, dtype=np.float64)
        parts.append(np.asarray(pos, np.float64)[:, None] * (cfg.rope_theta ** (-k / size))[None])
    return np.concatenate(parts, axis=1)


def _rope_angles_parts_reordered(cfg, t_pos, i_pos, j_pos):
    # (row, column, time) order of the head-dim parts instead of (time, row, column)
    return np.concatenate([_orig_rope_angles(cfg, i_pos, j_pos, t_pos)], axis=1)


_orig_rope_angles = od.rope_angles


def _whole_decoder_pins():
    cfg = small_cfg()
    return max(check_stream_equals_bruteforce(cfg) / 1e-12,
               check_uniform_attention_closed_form(cfg) / 1e-12,
               check_identity_blocks_closed_form(cfg) / 1e-12,
               check_stream_equals_bruteforce(small_paper_cfg()) / 1e-12,
               check_stream_equals_bruteforce(small_paper_cfg(n_layers=2, n_refine=2,
                                                              up_hidden=24)) / 1e-12,
               check_tail_identity_closed_form(small_tail_cfg()) / 1e-12)


def _prim_pins():
    return max(check_layer_norm() / 1e-12, check_gelu() / 1e-12,
               check_linear() / 1e-12, check_attention(False) / 1e-12,
               check_attention(True) / 1e-12,
               check_patchify(2) / 1e-12,
               check_unpatchify() / 1e-12,
               check_rms_norm() / 1e-12, check_gqa_attention(2) / 1e-12,
               check_kv_norm() / 1e-12, check_rope_complex() / 1e-12,
               check_rope_relative() / 1e-9,
               check_rope_frequencies() / 1e-12,
               check_rope_token_positions() / 1e-12)


MUTATIONS = [
    ("layer_norm", _ln_unbiased),
    ("layer_norm", _ln_no_shift),
    ("gelu", _gelu_tanh),
    ("gelu", _gelu_sign),
    ("linear", _linear_no_bias),
    ("linear", _linear_transposed),
    ("_head_attention", _attn_wrong_axis),
    ("patchify", _patchify_wrong_order),
    ("unpatchify", _unpatchify_swapped),
    ("block_causal_window_mask", _mask_off_by_one),
    ("apply_rope", _rope_sign),
    ("apply_rope", _rope_half_split),
    ("rms_norm", _rms_centered),
    ("kv_norm", _kv_norm_across_heads),
    ("attention", _attention_gqa_modulo),
    ("subframe_tokens", _subframes_interleaved),
    ("subframe_rope_angles", _subframe_angles_latent_units),
    ("spatial_upsample", _spatial_tokens_minor),
    ("token_rope_angles", _token_angles_rows_by_height),
    ("token_rope_angles", _token_angles_axes_swapped),
    ("rope_angles", _rope_angles_half_exponent),
    ("rope_angles", _rope_angles_parts_reordered),
]


@pytest.mark.parametrize("name,fn", MUTATIONS, ids=[f"{n}:{f.__name__}" for n, f in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, name, fn):
    monkeypatch.setattr(od, name, fn)
    if hasattr(oracle, name):
        monkeypatch.setattr(oracle, name, fn)
    try:
        worst = max(_prim_pins(), _whole_decoder_pins())
    except Exception:
        worst = float("inf")            # a crash is caught too
    assert worst > 1.0, f"mutation {name}:{fn.__name__} passed every pin"


def test_planted_wrong_scale_is_caught(monkeypatch):
    def bad(q, k, v, allowed, rows):       # scores scaled by 1/hd, not 1/sqrt(hd)
        return _orig_attn(q / math.sqrt(q.shape[1]), k, v, allowed, rows)
    monkeypatch.setattr(od, "_head_attention", bad)
    assert check_attention(False) > 1e-6


def test_unmutated_oracle_passes_every_pin():
    assert max(_prim_pins(), _whole_decoder_pins()) <= 1.0
