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
    check_attention, check_gelu, check_identity_blocks_closed_form,
    check_layer_norm, check_linear, check_patchify,
    check_stream_equals_bruteforce, check_uniform_attention_closed_form,
    check_unpatchify, small_cfg)

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


def _whole_decoder_pins():
    cfg = small_cfg()
    return max(check_stream_equals_bruteforce(cfg) / 1e-12,
               check_uniform_attention_closed_form(cfg) / 1e-12,
               check_identity_blocks_closed_form(cfg) / 1e-12)


def _prim_pins():
    return max(check_layer_norm() / 1e-12, check_gelu() / 1e-12,
               check_linear() / 1e-12, check_attention(False) / 1e-12,
               check_attention(True) / 1e-12,
               check_patchify(2) / 1e-12,
               check_unpatchify() / 1e-12)


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
