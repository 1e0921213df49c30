"""ctypes binding of libflashdec.so: same names as the C ABI, marshalling only."""
from __future__ import annotations

import ctypes
import os
from typing import Any, Dict, Optional, Sequence

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))

FD_OK = 0
FD_ERR_INVALID_ARG = -1
FD_ERR_UNSUPPORTED = -2
FD_ERR_OOM = -3
FD_ERR_DEVICE = -4
FD_ERR_STATE = -5
FD_MAX_WINDOW = 8

KERNEL_KINDS = ("state", "patchify", "inproj", "layernorm", "qkv", "attention",
                "oproj", "fc1", "fc2", "unpatchify", "temporal", "spatial")


class FdError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} ({status})")
        self.status = status


FD_NORM_LAYER, FD_NORM_RMS = 0, 1


class _Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "latent_c", "latent_h", "latent_w", "patch", "d_model", "n_heads",
        "head_dim", "mlp_dim", "n_layers", "window", "out_t", "out_patch",
        "out_c")] + [("ln_eps", ctypes.c_float)] + [
        (n, ctypes.c_int32) for n in ("n_kv_heads", "norm", "kv_norm", "rope")] + [
        ("rope_theta", ctypes.c_float)] + [
        (n, ctypes.c_int32) for n in ("n_refine", "up_hidden", "batch")]


_FP = ctypes.POINTER(ctypes.c_float)
_LAYER_FIELDS = ("ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_o", "b_o",
                 "ln2_g", "ln2_b", "w_1", "b_1", "w_2", "b_2", "kn_g", "vn_g")


class _LayerWeights(ctypes.Structure):
    _fields_ = [(n, _FP) for n in _LAYER_FIELDS]


_TAIL_FIELDS = ("w_tu", "b_tu", "lnr_g", "lnr_b", "w_s1", "b_s1", "w_s2", "b_s2")


class _Weights(ctypes.Structure):
    _fields_ = [("w_in", _FP), ("b_in", _FP), ("layers", ctypes.POINTER(_LayerWeights)),
                ("lnf_g", _FP), ("lnf_b", _FP), ("w_out", _FP), ("b_out", _FP),
                ("refine", ctypes.POINTER(_LayerWeights))] + [(n, _FP) for n in _TAIL_FIELDS]


class _Info(ctypes.Structure):
    _fields_ = [("frames_decoded", ctypes.c_int64), ("n_valid", ctypes.c_int32),
                ("window", ctypes.c_int32),
                ("slot_frame", ctypes.c_int32 * FD_MAX_WINDOW),
                ("n_tokens", ctypes.c_int32), ("n_tokens_pad", ctypes.c_int32),
                ("arena_bytes", ctypes.c_uint64), ("weight_bytes", ctypes.c_uint64),
                ("ring_bytes", ctypes.c_uint64), ("workspace_bytes", ctypes.c_uint64)]


_lib = None


def lib_path() -> str:
    return os.environ.get("FLASHDEC_LIB", os.path.join(_PKG, "libflashdec.so"))


def load_library():
    """Load libflashdec.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise ImportError(
            f"{path} not found: build it with `python -m transformer_latent_pixel_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    sig = {
        "fd_status_string": (ctypes.c_char_p, [i32]),
        "fd_config_check": (i32, [ctypes.POINTER(_Config)]),
        "fd_create": (i32, [ctypes.POINTER(_Config), ctypes.POINTER(_Weights), vp,
                            ctypes.POINTER(vp)]),
        "fd_decode_frame": (i32, [vp, vp, vp]),
        "fd_reset": (i32, [vp]),
        "fd_graph_enable": (i32, [vp, i32]),
        "fd_destroy": (None, [vp]),
        "fd_query": (i32, [vp, ctypes.POINTER(_Info)]),
        "fd_debug_read_kv": (i32, [vp, i32, i32, i32, vp, ctypes.c_size_t]),
        "fd_debug_read_ring": (i32, [vp, i32, i32, i32, vp, ctypes.c_size_t]),
        "fd_debug_poison_ring": (i32, [vp]),
        "fd_debug_fail_after": (i32, [vp, i64]),
        "fd_profile_enable": (i32, [vp, i32]),
        "fd_profile_filter": (i32, [vp, ctypes.c_uint32, i32]),
        "fd_profile_read": (i32, [vp, ctypes.POINTER(ctypes.c_double),
                                  ctypes.POINTER(i64), i32]),
        "fdk_gemm": (i32, [i32, vp, vp, vp, vp, i32, i32, i32, i32, vp]),
        "fdk_layernorm": (i32, [vp, i32, i32, vp, vp, ctypes.c_float, i32, vp, vp]),
        "fdk_attention": (i32, [vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp, vp]),
        "fdk_attention_noalloc": (i32, [vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, vp,
                                        vp]),
        "fdk_mfma_probe": (i32, [i32, i32, vp, vp, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def exported_symbols() -> Sequence[str]:
    """Names of the C functions this binding wraps (all must be exported)."""
    return ("fd_status_string", "fd_config_check", "fd_create", "fd_decode_frame",
            "fd_reset", "fd_graph_enable", "fd_destroy", "fd_query", "fd_debug_read_kv",
            "fd_debug_read_ring", "fd_debug_poison_ring", "fd_debug_fail_after",
            "fd_profile_enable", "fd_profile_filter", "fd_profile_read", "fdk_gemm", "fdk_layernorm",
            "fdk_attention", "fdk_attention_noalloc", "fdk_mfma_probe")


def status_string(status: int) -> str:
    return load_library().fd_status_string(status).decode()


def _check(status: int, what: str) -> None:
    if status != FD_OK:
        raise FdError(status, what)


def _ptr(x: Any) -> Optional[int]:
    """Device address of x: None, an int, or an object with data_ptr()."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _dev_f32(x: Any, numel: int, what: str) -> Optional[int]:
    """Device address of a float32 buffer the library reads or writes
    `numel` elements of.  A torch tensor must be a contiguous float32 tensor
    on the GPU holding at least numel elements; anything else is refused here,
    before the call, with FD_ERR_INVALID_ARG (the kernels would otherwise
    access memory out of bounds).  A plain int is taken as a raw device
    address whose size the caller vouches for."""
    if x is None or isinstance(x, int):
        return x
    if hasattr(x, "is_cuda"):
        import torch
        if not x.is_cuda:
            raise FdError(FD_ERR_INVALID_ARG, f"{what}: tensor is not in device memory")
        if x.dtype != torch.float32:
            raise FdError(FD_ERR_INVALID_ARG, f"{what}: dtype {x.dtype}, float32 required")
        if not x.is_contiguous():
            raise FdError(FD_ERR_INVALID_ARG, f"{what}: tensor is not contiguous")
        if x.numel() < numel:
            raise FdError(FD_ERR_INVALID_ARG,
                          f"{what}: {x.numel()} elements, at least {numel} required")
        return int(x.data_ptr())
    raise FdError(FD_ERR_INVALID_ARG, f"{what}: expected a device tensor or an address")


def _stream(stream: Any) -> Optional[int]:
    if stream is None:
        return None
    if isinstance(stream, int):
        return stream
    return int(getattr(stream, "cuda_stream", getattr(stream, "hip_stream", 0))) or None


# Fields of the paper's block and their values when a config omits them.
_BLOCK_DEFAULTS = {"n_kv_heads": 0, "norm": "layer", "kv_norm": 0, "rope": 0,
                   "rope_theta": 10000.0, "n_refine": 0, "up_hidden": 0, "batch": 0}


def _cfg_struct(cfg: Any) -> _Config:
    get = (lambda k: cfg[k]) if isinstance(cfg, dict) else (lambda k: getattr(cfg, k))
    c = _Config()
    for name, _ in _Config._fields_:
        val = get(name) if _has(cfg, name) else _BLOCK_DEFAULTS.get(name, 1e-5)
        if name == "norm":
            c.norm = {"layer": FD_NORM_LAYER, "rms": FD_NORM_RMS}.get(val, -1)
        elif name in ("ln_eps", "rope_theta"):
            setattr(c, name, float(val))
        else:
            setattr(c, name, int(val))
    return c


def _has(cfg, k):
    return (k in cfg) if isinstance(cfg, dict) else hasattr(cfg, k)


def config_check(cfg: Any) -> int:
    """fd_config_check: host-only validation, returns the status code."""
    c = _cfg_struct(cfg)
    return load_library().fd_config_check(ctypes.byref(c))


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


def _fp(a: np.ndarray):
    return a.ctypes.data_as(_FP)


class Decoder:
    """One fd_handle: fd_create / fd_decode_frame / fd_reset / fd_destroy.

    weights: dict with "w_in", "b_in", "lnf_g", "lnf_b", "w_out", "b_out" and
    "layers" (list of dicts with ln1_g .. b_2, plus kn_g and vn_g with
    KV-norm), float32 host arrays, Linear weights [out][in]; with the
    upsampling tail (n_refine > 0) also "refine" (blocks like "layers") and
    "w_tu", "b_tu", "lnr_g", "lnr_b", "w_s1", "b_s1", "w_s2", "b_s2".  They
    are copied into the library's arena at create.
    """

    def __init__(self, cfg: Any, weights: Dict[str, Any], stream: Any = None):
        lib = load_library()
        self._lib = lib
        self.cfg = cfg
        c = _cfg_struct(cfg)
        keep = []

        def blocks(lst):
            arr = (_LayerWeights * max(1, len(lst)))()
            for i, lw in enumerate(lst):
                for n in _LAYER_FIELDS:
                    if lw.get(n) is None:       # KV-norm gains of the simplified block
                        continue
                    a = _f32(lw[n])
                    keep.append(a)
                    setattr(arr[i], n, _fp(a))
            return arr

        w = _Weights()
        names = ("w_in", "b_in", "lnf_g", "lnf_b", "w_out", "b_out")
        if c.n_refine > 0:
            names += _TAIL_FIELDS
            w.refine = blocks(weights["refine"])
        for n in names:
            if weights.get(n) is None:
                continue
            a = _f32(weights[n])
            keep.append(a)
            setattr(w, n, _fp(a))
        w.layers = blocks(weights["layers"])
        h = ctypes.c_void_p()
        _check(lib.fd_create(ctypes.byref(c), ctypes.byref(w), _stream(stream),
                             ctypes.byref(h)), "fd_create")
        self._h = h
        del keep

    @property
    def handle(self) -> int:
        return self._h.value

    def _sizes(self):
        """(latent, pixel) float32 element counts of one call, all streams."""
        c = _cfg_struct(self.cfg)
        b = c.batch or 1
        ph = (c.latent_h // c.patch) * c.out_patch
        pw = (c.latent_w // c.patch) * c.out_patch
        return (b * c.latent_c * c.latent_h * c.latent_w,
                b * c.out_t * ph * pw * c.out_c)

    def decode_frame(self, latent_dev: Any, pixels_dev: Any) -> None:
        """Enqueue one frame: latent fp32 [B][C'][H'][W'] -> pixels fp32
        [B][T][H][W][C] (B = batch streams, no leading axis when B = 1).
        Torch tensors are checked (device, float32, contiguous, size) before
        the call."""
        n_lat, n_pix = self._sizes()
        lat = _dev_f32(latent_dev, n_lat, "fd_decode_frame latent")
        pix = _dev_f32(pixels_dev, n_pix, "fd_decode_frame pixels")
        _check(self._lib.fd_decode_frame(self._h, lat, pix), "fd_decode_frame")

    def reset(self) -> None:
        _check(self._lib.fd_reset(self._h), "fd_reset")

    def graph_enable(self, enable: bool = True) -> None:
        """fd_graph_enable: replay one recorded graph per frame (the handle
        must have been created on a stream other than the default one)."""
        _check(self._lib.fd_graph_enable(self._h, int(bool(enable))), "fd_graph_enable")

    def query(self) -> Dict[str, Any]:
        info = _Info()
        _check(self._lib.fd_query(self._h, ctypes.byref(info)), "fd_query")
        return {"frames_decoded": info.frames_decoded, "n_valid": info.n_valid,
                "window": info.window,
                "slot_frame": list(info.slot_frame)[:info.window],
                "n_tokens": info.n_tokens, "n_tokens_pad": info.n_tokens_pad,
                "arena_bytes": info.arena_bytes, "weight_bytes": info.weight_bytes,
                "ring_bytes": info.ring_bytes,
                "workspace_bytes": info.workspace_bytes}

    def debug_read_kv(self, layer: int, slot: int, kv: int) -> np.ndarray:
        """bf16 bits of one ring slot as uint16 [B G][n][head_dim] (B streams,
        G KV heads; n = N, or out_t N for a refinement block, layer >=
        n_layers)."""
        c = _cfg_struct(self.cfg)
        n_tok = (c.latent_h // c.patch) * (c.latent_w // c.patch)
        if layer >= c.n_layers:
            n_tok *= c.out_t
        heads = (c.batch or 1) * (c.n_kv_heads or c.n_heads)
        out = np.empty((heads, n_tok, c.head_dim), dtype=np.uint16)
        _check(self._lib.fd_debug_read_kv(self._h, layer, slot, kv,
                                           out.ctypes.data, out.size),
               "fd_debug_read_kv")
        return out

    def debug_read_ring(self, layer: int, slot: int, kv: int) -> np.ndarray:
        """One ring slot as stored, padding rows included: keys uint16
        [B G][n_pad][hd], values uint16 [B G][hd][n_pad] (token columns with
        bits 2 and 3 swapped)."""
        c = _cfg_struct(self.cfg)
        n_tok = (c.latent_h // c.patch) * (c.latent_w // c.patch)
        if layer >= c.n_layers:
            n_tok *= c.out_t
        n_pad = (n_tok + 63) // 64 * 64
        heads = (c.batch or 1) * (c.n_kv_heads or c.n_heads)
        shape = (heads, n_pad, c.head_dim) if kv == 0 else (heads, c.head_dim, n_pad)
        out = np.empty(shape, dtype=np.uint16)
        _check(self._lib.fd_debug_read_ring(self._h, layer, slot, kv, out.ctypes.data,
                                             out.size), "fd_debug_read_ring")
        return out

    def debug_poison_ring(self) -> None:
        _check(self._lib.fd_debug_poison_ring(self._h), "fd_debug_poison_ring")

    def debug_fail_after(self, launches: int) -> None:
        _check(self._lib.fd_debug_fail_after(self._h, int(launches)), "fd_debug_fail_after")

    def profile_enable(self, enable: bool = True) -> None:
        _check(self._lib.fd_profile_enable(self._h, int(enable)), "fd_profile_enable")

    def profile_filter(self, kinds=None, layer: int = -1) -> None:
        """Time only the given kernel classes (names of KERNEL_KINDS; None =
        all) and, for layer >= 0, only that block's launches."""
        mask = 0xFFFFFFFF if kinds is None else sum(1 << KERNEL_KINDS.index(k) for k in kinds)
        _check(self._lib.fd_profile_filter(self._h, mask, int(layer)), "fd_profile_filter")

    def profile_read(self) -> Dict[str, Dict[str, float]]:
        n = len(KERNEL_KINDS)
        ms = (ctypes.c_double * n)()
        cnt = (ctypes.c_int64 * n)()
        _check(self._lib.fd_profile_read(self._h, ms, cnt, n), "fd_profile_read")
        return {k: {"ms": ms[i], "launches": cnt[i]} for i, k in enumerate(KERNEL_KINDS)}

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            self._lib.fd_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ------------------------------------------------------ per-step entry points
def fdk_gemm(epi: int, a, b, bias, out, m: int, m_rows_alloc: int, n: int, k: int,
             stream: Any = None) -> None:
    _check(load_library().fdk_gemm(epi, _ptr(a), _ptr(b), _ptr(bias), _ptr(out), m,
                                   m_rows_alloc, n, k, _stream(stream)), "fdk_gemm")


def fdk_layernorm(x, m: int, d: int, g, b, eps: float, out, stream: Any = None,
                  rms: bool = False) -> None:
    _check(load_library().fdk_layernorm(_ptr(x), m, d, _ptr(g), _ptr(b), eps, int(rms),
                                        _ptr(out), _stream(stream)), "fdk_layernorm")


def fdk_attention(q, k, v, n_frames: int, first_slot: int, heads: int, n: int, hd: int,
                  out, stream: Any = None, kv_heads: Optional[int] = None,
                  splits: int = 0) -> None:
    _check(load_library().fdk_attention(_ptr(q), _ptr(k), _ptr(v), n_frames, first_slot,
                                        heads, kv_heads or heads, n, hd, splits, _ptr(out),
                                        _stream(stream)),
           "fdk_attention")


def fdk_attention_noalloc(q, k, v, n_frames: int, first_slot: int, heads: int, n: int,
                          hd: int, out, stream: Any = None, kv_heads: Optional[int] = None,
                          splits: int = 0) -> None:
    """fdk_attention with the library's per-GPU scratch instead of
    allocations; asynchronous on `stream`."""
    _check(load_library().fdk_attention_noalloc(_ptr(q), _ptr(k), _ptr(v), n_frames,
                                                first_slot, heads, kv_heads or heads, n, hd,
                                                splits, _ptr(out), _stream(stream)),
           "fdk_attention_noalloc")


PROBE_WORKGROUPS = 256


def fdk_mfma_probe(zero_operands: bool, iters: int, sink, clocks, stream: Any = None) -> None:
    """Launch the matrix-core rate probe: sink fp32 [256 * 512], clocks
    uint64 (int64 tensors do) [256 * 8][2]; asynchronous on `stream`."""
    _check(load_library().fdk_mfma_probe(int(bool(zero_operands)), int(iters), _ptr(sink),
                                         _ptr(clocks), _stream(stream)), "fdk_mfma_probe")
