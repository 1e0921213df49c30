"""The C-ABI library loads and exports every declared entry point (no GPU).

Only host-side calls are made here: status strings, config validation, and
argument checks that return before any device work.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import transformer_latent_pixel_amd as fd
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for hdr in ("flashdec.h", "flashdec_kernels.h"):
        text = open(os.path.join(ROOT, "include", hdr)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?\w+\s*\**\s*(\w+)\s*\(", text, re.M):
            names.add(m.group(1))
    return names


def test_library_exists_and_loads():
    assert os.path.exists(fd.lib_path()), "build the library first"
    fd.load_library()


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(fd.lib_path())
    names = declared_functions()
    assert {"fd_create", "fd_decode_frame", "fd_reset", "fd_destroy"} <= names
    for n in names:
        assert hasattr(lib, n), n
    assert names == set(fd.exported_symbols())


def test_status_strings():
    assert fd.status_string(fd.FD_OK) == "ok"
    for s in (fd.FD_ERR_INVALID_ARG, fd.FD_ERR_UNSUPPORTED, fd.FD_ERR_OOM,
              fd.FD_ERR_DEVICE, fd.FD_ERR_STATE):
        assert fd.status_string(s) not in ("ok", "unknown status")
    assert fd.status_string(42) == "unknown status"


@pytest.mark.parametrize("name", list(W.CONFIGS))
def test_workloads_are_supported(name):
    assert fd.config_check(W.CONFIGS[name]) == fd.FD_OK


@pytest.mark.parametrize("change,expect", [
    (dict(window=0), fd.FD_ERR_INVALID_ARG),
    (dict(window=9), fd.FD_ERR_INVALID_ARG),
    (dict(n_heads=15), fd.FD_ERR_INVALID_ARG),        # D != heads * head_dim
    (dict(latent_h=61), fd.FD_ERR_INVALID_ARG),       # not divisible by patch
    (dict(d_model=0), fd.FD_ERR_INVALID_ARG),
    (dict(ln_eps=0.0), fd.FD_ERR_INVALID_ARG),
    (dict(head_dim=128, n_heads=8), fd.FD_ERR_UNSUPPORTED),
    (dict(patch=4, latent_h=60, latent_w=104), fd.FD_ERR_UNSUPPORTED),
    (dict(mlp_dim=4000), fd.FD_ERR_UNSUPPORTED),
    (dict(n_kv_heads=5), fd.FD_ERR_INVALID_ARG),      # does not divide 16 heads
    (dict(n_kv_heads=-1), fd.FD_ERR_INVALID_ARG),
    (dict(norm="other"), fd.FD_ERR_INVALID_ARG),
    (dict(rope=True, rope_theta=0.5), fd.FD_ERR_INVALID_ARG),
    (dict(rope=True, head_dim=32, n_heads=32), fd.FD_ERR_UNSUPPORTED),   # head_dim 64 only
    (dict(kv_norm=True, n_heads=3, d_model=192), fd.FD_ERR_UNSUPPORTED),   # 3 + 2*3 heads: odd
    (dict(n_refine=-1), fd.FD_ERR_INVALID_ARG),
    (dict(up_hidden=-64), fd.FD_ERR_INVALID_ARG),
    (dict(n_refine=2, out_t=9), fd.FD_ERR_INVALID_ARG),   # r_t above FD_MAX_SUBFRAMES
    (dict(n_refine=2, out_patch=4, out_c=3), fd.FD_ERR_UNSUPPORTED),   # 48 channels
    (dict(n_refine=2, up_hidden=1000), fd.FD_ERR_UNSUPPORTED),
])
def test_config_check_rejects(change, expect):
    cfg = W.CONFIGS["480p"].replace(**change)
    assert fd.config_check(cfg) == expect


def test_null_arguments_are_rejected_before_device_work():
    lib = fd.load_library()
    assert lib.fd_create(None, None, None, None) == fd.FD_ERR_INVALID_ARG
    assert lib.fd_decode_frame(None, None, None) == fd.FD_ERR_INVALID_ARG
    assert lib.fd_reset(None) == fd.FD_ERR_INVALID_ARG
    assert lib.fd_graph_enable(None, 1) == fd.FD_ERR_INVALID_ARG
    assert lib.fd_query(None, None) == fd.FD_ERR_INVALID_ARG
    assert lib.fd_debug_read_kv(None, 0, 0, 0, None, 0) == fd.FD_ERR_INVALID_ARG
    assert lib.fd_debug_read_ring(None, 0, 0, 0, None, 0) == fd.FD_ERR_INVALID_ARG
    assert lib.fd_debug_poison_ring(None) == fd.FD_ERR_INVALID_ARG
    assert lib.fd_debug_fail_after(None, 1) == fd.FD_ERR_INVALID_ARG
    assert lib.fd_profile_enable(None, 1) == fd.FD_ERR_INVALID_ARG
    assert lib.fd_profile_filter(None, 0xFFFFFFFF, -1) == fd.FD_ERR_INVALID_ARG
    lib.fd_destroy(None)          # ignored
    assert lib.fdk_gemm(0, None, None, None, None, 1, 64, 64, 64, None) == fd.FD_ERR_INVALID_ARG
    assert lib.fdk_layernorm(None, 1, 64, None, None, 1e-5, 0, None, None) == fd.FD_ERR_INVALID_ARG
    assert lib.fdk_attention(None, None, None, 1, 0, 1, 1, 1, 64, 0, None, None) == fd.FD_ERR_INVALID_ARG
    assert lib.fdk_mfma_probe(0, 1, None, None, None) == fd.FD_ERR_INVALID_ARG


def test_product_path_has_no_fallback(monkeypatch, tmp_path):
    # With the library missing, the binding raises instead of computing.
    import transformer_latent_pixel_amd.capi as capi
    monkeypatch.setattr(capi, "_lib", None)
    monkeypatch.setenv("FLASHDEC_LIB", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        capi.load_library()


def test_qkv_width_must_fill_64_column_tiles():
    # head_dim 16 with one KV head: (4 + 2) 16 = 96 QKV columns, not a
    # multiple of the GEMM's 64-column tile; refused at validation instead of
    # failing at the first decode.
    cfg = W.CONFIGS["tiny"].replace(n_kv_heads=1)
    assert fd.config_check(cfg) == fd.FD_ERR_UNSUPPORTED
    assert fd.config_check(W.CONFIGS["tiny"].replace(n_kv_heads=2)) == fd.FD_OK  # 128


class _NoCalls:
    def __getattr__(self, name):
        raise AssertionError(f"library function {name} called")


def _decoder_without_handle(cfg):
    # A Decoder whose library must not be reached: argument checks in the
    # binding have to refuse the call first.
    import ctypes as ct
    d = fd.Decoder.__new__(fd.Decoder)
    d.cfg = cfg
    d._lib = _NoCalls()
    d._h = ct.c_void_p(0)
    return d


@pytest.mark.parametrize("which", ["latent", "pixels"])
@pytest.mark.parametrize("bad", ["host", "float16", "short", "strided", "list"])
def test_binding_refuses_bad_buffers_before_any_device_work(which, bad):
    import torch
    cfg = W.CONFIGS["tiny"]
    n = {"latent": int(np.prod(cfg.latent_shape)), "pixels": int(np.prod(cfg.pixel_shape))}

    class FakeDev:
        # quacks like a contiguous float32 device tensor of n elements
        def __init__(self, numel, dtype=torch.float32, contig=True, cuda=True):
            self.is_cuda, self.dtype, self._n, self._c = cuda, dtype, numel, contig

        def numel(self):
            return self._n

        def is_contiguous(self):
            return self._c

        def data_ptr(self):
            return 1 << 20

    good = {k: FakeDev(v) for k, v in n.items()}
    arg = {"host": torch.zeros(n[which]),
           "float16": FakeDev(n[which], dtype=torch.float16),
           "short": FakeDev(n[which] - 1),
           "strided": FakeDev(n[which], contig=False),
           "list": [0.0] * 4}[bad]
    args = dict(good)
    args[which] = arg
    d = _decoder_without_handle(cfg)
    with pytest.raises(fd.FdError) as e:
        d.decode_frame(args["latent"], args["pixels"])
    assert e.value.status == fd.FD_ERR_INVALID_ARG
