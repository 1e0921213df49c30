"""Pins of the CPU oracle against things other than itself.

Each check returns a float error (0 = exact agreement) so that the pin tests
and the planted-mistake tests can share them.  The independent side of every
check is one of: a PyTorch library routine computed in float64 on the CPU
(pixel_unshuffle, pixel_shuffle, layer_norm, gelu, scaled_dot_product_attention,
linear), a closed form, an invariant, or the brute-force masked formulation.
"""
from __future__ import annotations

import math

import numpy as np
import torch
import torch.nn.functional as F
from einops import rearrange

import oracle
import workloads as W


def rel_l2(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def small_cfg(**kw) -> W.DecoderConfig:
    base = dict(name="small", latent_c=6, latent_h=4, latent_w=6, patch=1,
                d_model=32, n_heads=4, head_dim=8, mlp_dim=64, n_layers=3,
                window=2, out_t=2, out_patch=2, out_c=3, frames=6,
                bf16_weights=False)
    base.update(kw)
    return W.DecoderConfig(**base)


def _t(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float64))


# ---------------------------------------------------------------- primitives
def check_patchify(p: int = 2) -> float:
    z = W.standard_normal(7, 1, 5 * 6 * 10).reshape(5, 6, 10)
    x = oracle.patchify(z, p)
    ref = F.pixel_unshuffle(_t(z)[None], p)[0]           # [C p^2][H/p][W/p]
    ref = ref.reshape(ref.shape[0], -1).T                 # raster tokens
    return float(np.abs(x - ref.numpy()).max())


def check_unpatchify() -> float:
    th, tw, T, P, C = 3, 5, 2, 4, 3
    r = W.standard_normal(7, 2, th * tw * T * P * P * C).reshape(th * tw, -1)
    pix = oracle.unpatchify(r, th, tw, T, P, C)
    # Library route: per time step, relabel a token's (dy, dx, c) channels as
    # PixelShuffle's (c, dy, dx) order, shuffle, then move channels last.
    x = _t(r).reshape(th, tw, T, P, P, C).permute(2, 5, 3, 4, 0, 1)
    x = x.reshape(T, C * P * P, th, tw)
    ref = F.pixel_shuffle(x, P).permute(0, 2, 3, 1)        # [T][H][W][C]
    return float(np.abs(pix - ref.numpy()).max())


def check_unpatchify_bijective() -> float:
    th, tw, T, P, C = 3, 4, 2, 2, 3
    n = th * tw * T * P * P * C
    pix = oracle.unpatchify(np.arange(n, dtype=np.float64).reshape(th * tw, -1),
                            th, tw, T, P, C)
    return float(np.abs(np.sort(pix.ravel()) - np.arange(n)).max())


def check_linear() -> float:
    x = W.standard_normal(7, 3, 9 * 5).reshape(9, 5)
    w = W.standard_normal(7, 4, 7 * 5).reshape(7, 5)
    b = W.standard_normal(7, 5, 7)
    return float(np.abs(oracle.linear(x, w, b) - F.linear(_t(x), _t(w), _t(b)).numpy()).max())


def check_layer_norm() -> float:
    x = 3.0 + 2.0 * W.standard_normal(7, 6, 11 * 33).reshape(11, 33)
    g = 1.0 + 0.1 * W.standard_normal(7, 7, 33)
    b = 0.1 * W.standard_normal(7, 8, 33)
    ref = F.layer_norm(_t(x), (33,), _t(g), _t(b), eps=1e-5).numpy()
    return float(np.abs(oracle.layer_norm(x, g, b, 1e-5) - ref).max())


def check_gelu() -> float:
    x = 4.0 * W.standard_normal(7, 9, 1000)
    ref = F.gelu(_t(x), approximate="none").numpy()
    err = np.abs(oracle.gelu(x) - ref).max()
    # GELU(x) - GELU(-x) = x, GELU(0) = 0.
    err = max(err, np.abs(oracle.gelu(x) - oracle.gelu(-x) - x).max())
    err = max(err, abs(float(oracle.gelu(np.array([0.0]))[0])))
    return float(err)


def check_attention(masked: bool) -> float:
    nh, hd, nq, nk = 3, 8, 12, 20
    q = W.standard_normal(7, 10, nq * nh * hd).reshape(nq, nh * hd)
    k = W.standard_normal(7, 11, nk * nh * hd).reshape(nk, nh * hd)
    v = W.standard_normal(7, 12, nk * nh * hd).reshape(nk, nh * hd)
    allowed = None
    if masked:
        allowed = oracle.decoder.block_causal_window_mask(4, 5, 2)[:nq]
    out = oracle.attention(q, k, v, nh, allowed)
    th = lambda a, n: _t(a).reshape(n, nh, hd).transpose(0, 1)   # [h][n][hd]
    ref = F.scaled_dot_product_attention(
        th(q, nq), th(k, nk), th(v, nk),
        attn_mask=None if allowed is None else torch.from_numpy(allowed))
    ref = ref.transpose(0, 1).reshape(nq, nh * hd).numpy()
    return float(np.abs(out - ref).max())


def check_attention_uniform() -> float:
    """q = 0 makes every score equal: the output is the mean of V."""
    nh, hd, nq, nk = 2, 4, 5, 9
    q = np.zeros((nq, nh * hd))
    k = W.standard_normal(7, 13, nk * nh * hd).reshape(nk, nh * hd)
    v = W.standard_normal(7, 14, nk * nh * hd).reshape(nk, nh * hd)
    out = oracle.attention(q, k, v, nh)
    return float(np.abs(out - v.mean(axis=0, keepdims=True)).max())


# ------------------------------------------------------------ whole decoder
def stream(cfg, w, zs):
    dec = oracle.StreamingDecoder(cfg, w)
    return [dec.decode_frame(z) for z in zs]


def check_stream_equals_bruteforce(cfg) -> float:
    w = W.make_weights(cfg)
    zs = W.make_latents(cfg)
    a = stream(cfg, w, zs)
    b = oracle.bruteforce_decode(cfg, w, zs)
    return max(rel_l2(x, y) for x, y in zip(a, b))


def _torch_ln(x, g, b, eps):
    return F.layer_norm(x, (x.shape[-1],), g, b, eps=eps)


def closed_form_uniform_attention(cfg, w, zs):
    """Decoder with W_q = b_q = 0 in every block, written with torch routines.

    All scores are equal, so attention returns the mean of V over exactly the
    valid cached keys: N keys at frame 0 and min(t+1, W) N keys later.  The
    mean is the same row for every query.
    """
    D, N = cfg.d_model, cfg.n_tokens
    tw = {k: _t(v) for k, v in w.items() if k != "layers"}
    lws = [{k: _t(v) for k, v in lw.items()} for lw in w["layers"]]
    vhist = [[] for _ in lws]
    outs = []
    for t, z in enumerate(zs):
        x = F.pixel_unshuffle(_t(z)[None], cfg.patch)[0].reshape(cfg.c_in, N).T
        h = F.linear(x, tw["w_in"], tw["b_in"])
        for l, lw in enumerate(lws):
            a = _torch_ln(h, lw["ln1_g"], lw["ln1_b"], cfg.ln_eps)
            v = F.linear(a, lw["w_qkv"][2 * D:], lw["b_qkv"][2 * D:])
            vhist[l].append(v)
            valid = vhist[l][max(0, t + 1 - cfg.window):t + 1]
            o = torch.cat(valid, 0).mean(0, keepdim=True).expand(N, D)
            h = h + F.linear(o, lw["w_o"], lw["b_o"])
            a = _torch_ln(h, lw["ln2_g"], lw["ln2_b"], cfg.ln_eps)
            h = h + F.linear(F.gelu(F.linear(a, lw["w_1"], lw["b_1"])),
                             lw["w_2"], lw["b_2"])
        r = F.linear(_torch_ln(h, tw["lnf_g"], tw["lnf_b"], cfg.ln_eps),
                     tw["w_out"], tw["b_out"])
        outs.append(_torch_unpatchify(r, cfg))
    return outs


def _torch_unpatchify(r, cfg):
    P, C, T = cfg.out_patch, cfg.out_c, cfg.out_t
    x = r.reshape(cfg.tok_h, cfg.tok_w, T, P, P, C).permute(2, 5, 3, 4, 0, 1)
    x = x.reshape(T, C * P * P, cfg.tok_h, cfg.tok_w)
    return F.pixel_shuffle(x, P).permute(0, 2, 3, 1).numpy()


def zero_query_weights(cfg, w):
    D = cfg.d_model
    for lw in w["layers"]:
        lw["w_qkv"] = lw["w_qkv"].copy()
        lw["b_qkv"] = lw["b_qkv"].copy()
        lw["w_qkv"][:D] = 0.0
        lw["b_qkv"][:D] = 0.0
    return w


def check_uniform_attention_closed_form(cfg) -> float:
    w = zero_query_weights(cfg, W.make_weights(cfg))
    zs = W.make_latents(cfg)
    a = stream(cfg, w, zs)
    b = closed_form_uniform_attention(cfg, w, zs)
    return max(rel_l2(x, y) for x, y in zip(a, b))


def check_identity_blocks_closed_form(cfg) -> float:
    """W_o = b_o = W_2 = b_2 = 0: every block adds zero, so pixels are
    unpatchify(LNf(patchify(z) W_in^T + b_in) W_out^T + b_out)."""
    w = W.make_weights(cfg)
    for lw in w["layers"]:
        for n in ("w_o", "b_o", "w_2", "b_2"):
            lw[n] = np.zeros_like(lw[n])
    zs = W.make_latents(cfg)
    a = stream(cfg, w, zs)
    err = 0.0
    for z, got in zip(zs, a):
        x = F.pixel_unshuffle(_t(z)[None], cfg.patch)[0].reshape(cfg.c_in, -1).T
        h = F.linear(x, _t(w["w_in"]), _t(w["b_in"]))
        r = F.linear(_torch_ln(h, _t(w["lnf_g"]), _t(w["lnf_b"]), cfg.ln_eps),
                     _t(w["w_out"]), _t(w["b_out"]))
        err = max(err, rel_l2(got, _torch_unpatchify(r, cfg)))
    return err


# ------------------------------------------------------- the paper's block
def small_paper_cfg(**kw) -> W.DecoderConfig:
    """small_cfg with the paper's block: RMSNorm, 4 query heads over 2 KV
    heads, KV-norm and 3D rotary positions (head_dim 12: 4 dims per axis)."""
    base = dict(d_model=48, n_heads=4, head_dim=12, n_kv_heads=2, norm="rms",
                kv_norm=True, rope=True)
    base.update(kw)
    return small_cfg(**base)


def check_rms_norm() -> float:
    x = W.standard_normal(8, 1, 6 * 40).reshape(6, 40) * 3.0 + 0.5
    g = 1.0 + 0.1 * W.standard_normal(8, 2, 40)
    ref = F.rms_norm(_t(x), (40,), _t(g), eps=1e-5).numpy()
    return float(np.abs(oracle.rms_norm(x, g, 1e-5) - ref).max())


def check_gqa_attention(n_kv: int) -> float:
    """Grouped-query attention against torch's SDPA with enable_gqa."""
    nh, hd, nq, nk = 6, 8, 10, 14
    q = W.standard_normal(9, 10, nq * nh * hd).reshape(nq, nh * hd)
    k = W.standard_normal(9, 11, nk * n_kv * hd).reshape(nk, n_kv * hd)
    v = W.standard_normal(9, 12, nk * n_kv * hd).reshape(nk, n_kv * hd)
    out = oracle.attention(q, k, v, nh, None, n_kv_heads=n_kv)
    th = lambda a, n, h: _t(a).reshape(n, h, hd).transpose(0, 1)
    ref = F.scaled_dot_product_attention(th(q, nq, nh), th(k, nk, n_kv), th(v, nk, n_kv),
                                         enable_gqa=True)
    ref = ref.transpose(0, 1).reshape(nq, nh * hd).numpy()
    return float(np.abs(out - ref).max())


def check_kv_norm() -> float:
    """Each head vector comes out as x / sqrt(ms + eps) * g: divided by g it has
    mean square ms / (ms + eps) and the direction of x."""
    hd, heads, n, eps = 8, 3, 5, 1e-5
    x = W.standard_normal(10, 1, n * heads * hd).reshape(n, heads * hd) * 2.0
    g = 1.0 + 0.1 * W.standard_normal(10, 2, hd)
    y = oracle.kv_norm(x, g, hd, eps).reshape(n, heads, hd) / g
    xh = x.reshape(n, heads, hd)
    ms = (xh * xh).mean(axis=-1)
    err = np.abs((y * y).mean(axis=-1) - ms / (ms + eps)).max()
    cos = (y * xh).sum(-1) / np.linalg.norm(y, axis=-1) / np.linalg.norm(xh, axis=-1)
    return float(max(err, np.abs(cos - 1.0).max()))


def check_rope_complex() -> float:
    """Rotation of consecutive pairs equals multiplying (a + i b) by e^(i phi),
    with phi_k = pos theta^(-2k/d) per axis part."""
    cfg = small_paper_cfg()
    hd, heads, n = cfg.head_dim, 3, 7
    x = W.standard_normal(11, 1, n * heads * hd).reshape(n, heads * hd)
    t, i, j = np.arange(n) * 1.0, np.arange(n) % 3 * 1.0, np.arange(n) // 2 * 1.0
    out = oracle.apply_rope(x, oracle.rope_angles(cfg, t, i, j), hd)
    z = x.reshape(n, heads, hd // 2, 2)
    z = z[..., 0] + 1j * z[..., 1]
    d_t, d_h, d_w = oracle.rope_split(hd)
    phi = []
    for size, pos in ((d_t, t), (d_h, i), (d_w, j)):
        for kk in range(size // 2):
            phi.append(pos * cfg.rope_theta ** (-2.0 * kk / size))
    phi = np.stack(phi, axis=1)                                  # [n][hd/2]
    r = z * np.exp(1j * phi)[:, None, :]
    ref = np.stack([r.real, r.imag], axis=-1).reshape(n, heads * hd)
    return float(np.abs(out - ref).max())


def check_rope_relative() -> float:
    """Rotated scores depend only on position differences: shifting both
    positions along every axis leaves q_rot . k_rot unchanged."""
    cfg = small_paper_cfg()
    hd = cfg.head_dim
    q = W.standard_normal(12, 1, hd).reshape(1, hd)
    k = W.standard_normal(12, 2, hd).reshape(1, hd)
    worst = 0.0
    for (p, r) in (((2, 1, 3), (0, 4, 1)), ((5, 0, 0), (4, 2, 7))):
        base = None
        for shift in (0.0, 7.0, 123.0):
            a = oracle.apply_rope(q, oracle.rope_angles(cfg, *[np.array([c + shift]) for c in p]), hd)
            b = oracle.apply_rope(k, oracle.rope_angles(cfg, *[np.array([c + shift]) for c in r]), hd)
            s = float((a * b).sum())
            base = s if base is None else base
            worst = max(worst, abs(s - base))
    zero = oracle.apply_rope(q, oracle.rope_angles(cfg, *[np.zeros(1)] * 3), hd)
    return max(worst, float(np.abs(zero - q).max()))


def rope64_cfg(**kw) -> W.DecoderConfig:
    """small_paper_cfg at head_dim 64 (the (24, 20, 20) split of the XL model)
    on a 4 x 6 token grid: tok_h != tok_w, so rows and columns cannot be
    confused."""
    base = dict(d_model=128, n_heads=2, head_dim=64, n_kv_heads=1)
    base.update(kw)
    return small_paper_cfg(**base)


def check_rope_frequencies() -> float:
    """Angles at position 1 on every axis are the per-pair frequencies.  For
    head_dim 64 and theta = 1e4 the reading gives theta^(-2k/24) = 10^(-k/3)
    for the 12 temporal pairs and theta^(-2k/20) = 10^(-2k/5) for the 10 row
    and the 10 column pairs: log-spaced from 1 down to 10^(-11/3) and
    10^(-18/5), written here with numpy's logspace, not the oracle's formula."""
    cfg = rope64_cfg()
    assert cfg.rope_theta == 10000.0
    got = oracle.rope_angles(cfg, np.ones(1), np.ones(1), np.ones(1))[0]
    ref = np.concatenate([np.logspace(0.0, -11.0 / 3.0, 12),
                          np.logspace(0.0, -18.0 / 5.0, 10),
                          np.logspace(0.0, -18.0 / 5.0, 10)])
    return float(np.abs(got - ref).max())


# Tokens of the 4 x 6 grid of rope64_cfg and their (row, column), written out
# by hand: raster order, token n = 6 i + j ([FD] §3.2 Eq. 1).
ROPE_TOKEN_RC = ((0, 0, 0), (5, 0, 5), (6, 1, 0), (7, 1, 1), (16, 2, 4), (23, 3, 5))


def check_rope_token_positions() -> float:
    """token_rope_angles puts token n at (frame_pos, row i, column j) of the
    token grid: against the hand-written (n, i, j) of ROPE_TOKEN_RC, with the
    angles built from the logspace frequencies of check_rope_frequencies."""
    cfg = rope64_cfg()
    assert (cfg.tok_h, cfg.tok_w) == (4, 6)
    ft = np.logspace(0.0, -11.0 / 3.0, 12)
    fs = np.logspace(0.0, -18.0 / 5.0, 10)
    worst = 0.0
    for pos in (0.0, 1.0, 3.0):
        got = oracle.token_rope_angles(cfg, pos)
        assert got.shape == (cfg.n_tokens, 32)
        for n, i, j in ROPE_TOKEN_RC:
            ref = np.concatenate([pos * ft, i * fs, j * fs])
            worst = max(worst, float(np.abs(got[n] - ref).max()))
    return worst


# ------------------------------------------- the temporal-first upsampling tail
def small_tail_cfg(**kw) -> W.DecoderConfig:
    """small_cfg with the tail of [FD] §3.4: r_t = 2 sub-frames, r_s = 2, two
    refinement blocks, spatial MLP hidden width 24 (not d_model, so the two
    MLP widths cannot be confused)."""
    base = dict(n_layers=2, n_refine=2, up_hidden=24)
    base.update(kw)
    return small_cfg(**base)


def check_tail_identity_closed_form(cfg) -> float:
    """Every block, backbone and refinement, made to add zero (W_o = b_o =
    W_2 = b_2 = 0).  The decoder is then the tail's plumbing alone, written
    here with torch and einops: tokens = PixelUnshuffle(z) W_in^T + b_in;
    Y = norm_f; P = Y W_tu^T + b_tu; the expanded channels read as r_t new
    time steps ('n (r d) -> (r n) d'); norm_r; MLP with GELU; a PixelShuffle
    of every sub-frame token ('(r h w) (dy dx c) -> r (h dy) (w dx) c')."""
    w = W.make_weights(cfg)
    for key in ("layers", "refine"):
        for lw in w[key]:
            for n in ("w_o", "b_o", "w_2", "b_2"):
                lw[n] = np.zeros_like(lw[n])
    zs = W.make_latents(cfg)
    got = stream(cfg, w, zs)

    def norm(x, g, b):
        if cfg.norm == "rms":
            return F.rms_norm(x, (x.shape[-1],), g, eps=cfg.ln_eps)
        return F.layer_norm(x, (x.shape[-1],), g, b, eps=cfg.ln_eps)

    err = 0.0
    for z, g in zip(zs, got):
        x = F.pixel_unshuffle(_t(z)[None], cfg.patch)[0].reshape(cfg.c_in, -1).T
        h = F.linear(x, _t(w["w_in"]), _t(w["b_in"]))
        p = F.linear(norm(h, _t(w["lnf_g"]), _t(w["lnf_b"])), _t(w["w_tu"]), _t(w["b_tu"]))
        tok = rearrange(p, "n (r d) -> (r n) d", r=cfg.out_t)
        a = norm(tok, _t(w["lnr_g"]), _t(w["lnr_b"]))
        sv = F.linear(F.gelu(F.linear(a, _t(w["w_s1"]), _t(w["b_s1"]))),
                      _t(w["w_s2"]), _t(w["b_s2"]))
        ref = rearrange(sv, "(r h w) (dy dx c) -> r (h dy) (w dx) c", r=cfg.out_t,
                        h=cfg.tok_h, w=cfg.tok_w, dy=cfg.out_patch, dx=cfg.out_patch,
                        c=cfg.out_c).numpy()
        err = max(err, rel_l2(g, ref))
    return err
