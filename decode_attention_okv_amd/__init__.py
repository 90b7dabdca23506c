"""Python binding of libokv (Hadamard-rotated 3-bit KV cache for MI355X).

Argument marshalling only: every step of the write and read paths runs in the
HIP kernels of ``libokv.so``.  PyTorch provides device memory and streams.

The module-level functions carry the names of the C entry points
(``okv_create``, ``okv_write``, ``okv_decode_attn``, ``okv_destroy`` and the
auxiliary calls); :class:`OkvCache` owns the four cache tensors and a handle.

Importing this package fails loudly when ``libokv.so`` has not been built
(``python -m decode_attention_okv_amd.build``).
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "OKV_OK", "OKV_E_INVALID", "OKV_E_ALIGN", "OKV_E_CAPACITY", "OKV_E_UNSUPPORTED", "OKV_E_HIP",
    "OkvError", "OkvConfig", "OkvLayout", "lib", "LIB_PATH", "EXPORTS",
    "okv_create", "okv_write", "okv_decode_attn", "okv_destroy", "okv_strerror", "okv_layout",
    "okv_get_len", "okv_set_len", "okv_set_splits", "okv_get_splits", "okv_max_splits",
    "okv_timing_enable", "okv_timing_read", "okv_set_decode_kernel", "okv_get_decode_kernel",
    "okv_prefill_attn", "okv_read_probe", "read_probe", "okv_decode_attn_noalloc",
    "DECODE_KERNEL", "make_config", "OkvCache",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libokv.so")

OKV_ABI_VERSION = 2
OKV_OK, OKV_E_INVALID, OKV_E_ALIGN, OKV_E_CAPACITY, OKV_E_UNSUPPORTED, OKV_E_HIP = range(6)
QUANT = {"sym": 0, "asym": 1}
DTYPE = {"f32": 0, "f16": 1, "bf16": 2, "e4m3": 3}
ROTATION = {"sign": 0, "so4": 1, "none": 2}
DECODE_KERNEL = {"auto": 0, "per_head": 1, "grouped": 2}

EXPORTS = ("okv_create", "okv_write", "okv_decode_attn", "okv_destroy", "okv_strerror",
           "okv_layout", "okv_get_len", "okv_set_len", "okv_set_splits", "okv_max_splits",
           "okv_get_splits", "okv_timing_enable", "okv_timing_read", "okv_set_decode_kernel",
           "okv_get_decode_kernel", "okv_last_hip_error", "okv_prefill_attn", "okv_so4_calibrate",
           "okv_so4_eval", "okv_read_probe", "okv_decode_attn_noalloc")


class OkvConfig(ctypes.Structure):
    _fields_ = [
        ("abi_version", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("max_tokens", ctypes.c_int32),
        ("block", ctypes.c_int32),
        ("quant", ctypes.c_int32),
        ("scale_dtype", ctypes.c_int32),
        ("in_dtype", ctypes.c_int32),
        ("rotation", ctypes.c_int32),
        ("bits", ctypes.c_int32),
        ("eps", ctypes.c_float),
        ("rot_params", ctypes.POINTER(ctypes.c_float)),
        ("k_codes", ctypes.c_void_p),
        ("v_codes", ctypes.c_void_p),
        ("k_meta", ctypes.c_void_p),
        ("v_meta", ctypes.c_void_p),
    ]


class OkvLayout(ctypes.Structure):
    _fields_ = [("k_codes_bytes", ctypes.c_uint64), ("v_codes_bytes", ctypes.c_uint64),
                ("k_meta_bytes", ctypes.c_uint64), ("v_meta_bytes", ctypes.c_uint64)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m decode_attention_okv_amd.build`")
    # One HIP runtime per process: PyTorch-ROCm ships its own libamdhip64.so.7.  With
    # torch loaded first, the dynamic linker resolves libokv's libamdhip64.so.7 to that
    # same runtime, so tensors and handles share one device context.  Loaded the other
    # way round, the process would hold two HIP runtimes, and the second one to start
    # can fail to find the device.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    so = ctypes.CDLL(LIB_PATH)
    vp, i32, P = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER
    sig = {
        "okv_create": (i32, [P(OkvConfig), P(vp)]),
        "okv_write": (i32, [vp, vp, vp, i32, vp]),
        "okv_decode_attn": (i32, [vp, vp, vp, vp]),
        "okv_decode_attn_noalloc": (i32, [vp, vp, vp, vp]),
        "okv_prefill_attn": (i32, [vp, vp, i32, vp, vp]),
        "okv_destroy": (i32, [vp]),
        "okv_strerror": (ctypes.c_char_p, [ctypes.c_int]),
        "okv_last_hip_error": (ctypes.c_char_p, []),
        "okv_layout": (i32, [P(OkvConfig), P(OkvLayout)]),
        "okv_get_len": (i32, [vp, P(i32)]),
        "okv_set_len": (i32, [vp, i32]),
        "okv_set_splits": (i32, [vp, i32]),
        "okv_max_splits": (i32, [vp, P(i32)]),
        "okv_get_splits": (i32, [vp, P(i32)]),
        "okv_timing_enable": (i32, [vp, i32]),
        "okv_timing_read": (i32, [vp, P(i32), P(ctypes.c_double), P(ctypes.c_double)]),
        "okv_set_decode_kernel": (i32, [vp, i32]),
        "okv_get_decode_kernel": (i32, [vp, P(i32)]),
        "okv_so4_calibrate": (i32, [vp, i32, i32, i32, i32, ctypes.c_float, vp, vp, i32, i32, vp, vp]),
        "okv_so4_eval": (i32, [vp, i32, i32, i32, i32, ctypes.c_float, vp, vp, i32, i32, vp, vp]),
        "okv_read_probe": (i32, [vp, ctypes.c_uint64, vp, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(so, name)
        fn.restype = res
        fn.argtypes = args
    return so


lib = _load()


class OkvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = f"{where}: {lib.okv_strerror(status).decode()} (status {status})"
        if status == OKV_E_HIP:
            msg += f": {lib.okv_last_hip_error().decode()}"
        super().__init__(msg)


def _check(status: int, where: str) -> None:
    if status != OKV_OK:
        raise OkvError(status, where)


def _stream_ptr(stream, device=None):
    """HIP stream handle for a call: `stream` (a torch stream or a raw handle), or by
    default torch's current stream of `device` (a torch.device or index; the current
    device when None).  torch's raw-handle query costs a fraction of a microsecond, where
    building a Stream object costs about three, a noticeable part of a small call."""
    if stream is None:
        import torch
        idx = torch.cuda.current_device() if device is None else (
            device.index if isinstance(device, torch.device) else int(device))
        raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        if raw is not None:
            return ctypes.c_void_p(raw(idx))
        stream = torch.cuda.current_stream(idx)
    if isinstance(stream, ctypes.c_void_p):
        return stream
    return ctypes.c_void_p(getattr(stream, "cuda_stream", stream))


# ---- C entry points with the C names (status codes are returned, not raised) ----

def okv_strerror(status: int) -> str:
    return lib.okv_strerror(status).decode()


def okv_layout(cfg: OkvConfig):
    info = OkvLayout()
    st = lib.okv_layout(ctypes.byref(cfg), ctypes.byref(info))
    return st, info


def okv_create(cfg: OkvConfig):
    h = ctypes.c_void_p()
    st = lib.okv_create(ctypes.byref(cfg), ctypes.byref(h))
    return st, h


def okv_write(h, k_ptr: int, v_ptr: int, n_new: int, stream=None) -> int:
    return lib.okv_write(h, ctypes.c_void_p(k_ptr), ctypes.c_void_p(v_ptr), n_new, _stream_ptr(stream))


def okv_decode_attn(h, q_ptr: int, out_ptr: int, stream=None) -> int:
    return lib.okv_decode_attn(h, ctypes.c_void_p(q_ptr), ctypes.c_void_p(out_ptr), _stream_ptr(stream))


def okv_decode_attn_noalloc(h, q_ptr: int, out_ptr: int, stream=None) -> int:
    return lib.okv_decode_attn_noalloc(h, ctypes.c_void_p(q_ptr), ctypes.c_void_p(out_ptr), _stream_ptr(stream))


def okv_prefill_attn(h, q_ptr: int, n_q: int, out_ptr: int, stream=None) -> int:
    return lib.okv_prefill_attn(h, ctypes.c_void_p(q_ptr), n_q, ctypes.c_void_p(out_ptr), _stream_ptr(stream))


def okv_so4_calibrate(x_ptr: int, n: int, d: int, block: int, bits: int, eps: float, rot_ptr: int,
                      cand_ptr: int, sweeps: int, n_cand: int, trace_ptr: int, stream=None) -> int:
    return lib.okv_so4_calibrate(ctypes.c_void_p(x_ptr), n, d, block, bits, eps, ctypes.c_void_p(rot_ptr),
                                 ctypes.c_void_p(cand_ptr), sweeps, n_cand, ctypes.c_void_p(trace_ptr),
                                 _stream_ptr(stream))


def okv_so4_eval(x_ptr: int, n: int, d: int, block: int, bits: int, eps: float, rot_ptr: int, cand_ptr: int,
                 n_cand: int, group: int, err_ptr: int, stream=None) -> int:
    return lib.okv_so4_eval(ctypes.c_void_p(x_ptr), n, d, block, bits, eps, ctypes.c_void_p(rot_ptr),
                            ctypes.c_void_p(cand_ptr), n_cand, group, ctypes.c_void_p(err_ptr),
                            _stream_ptr(stream))


def _so4_args(x, rot, block, bits):
    import numpy as np
    import torch
    if x.dtype != torch.float32 or x.dim() != 2 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x: contiguous float32 [n][head_dim] on the GPU")
    n, d = x.shape
    r = np.ascontiguousarray(np.asarray(rot, dtype=np.float32).reshape(d // 4, 4, 4))
    return n, d, r


def so4_calibrate(x, rot, cand, block=32, bits=3, eps=1e-6, stream=None):
    """Calibrate the SO(4) blocks of U = B H on the calibration vectors x (device
    float32 [n][d]).  rot: start rotations (d/4, 4, 4); cand: candidate perturbations
    (sweeps, d/4, n_cand, 4, 4) with the identity first.  Returns (rot, trace) as
    NumPy arrays: the calibrated rotations and the total error before and after each
    sweep.  All the work runs in libokv's kernels and its native search loop."""
    import numpy as np
    n, d, r = _so4_args(x, rot, block, bits)
    c = np.ascontiguousarray(np.asarray(cand, dtype=np.float32))
    sweeps, n_cand = c.shape[0], c.shape[2]
    if c.shape != (sweeps, d // 4, n_cand, 4, 4):
        raise ValueError(f"cand: expected (sweeps, {d // 4}, n_cand, 4, 4), got {c.shape}")
    trace = np.zeros(sweeps + 1, dtype=np.float64)
    _check(okv_so4_calibrate(x.data_ptr(), n, d, block, bits, eps, r.ctypes.data, c.ctypes.data, sweeps,
                             n_cand, trace.ctypes.data, stream), "okv_so4_calibrate")
    return r, trace


def so4_eval(x, rot, cand, group, block=32, bits=3, eps=1e-6, stream=None):
    """Errors of the quantisation block holding `group` for each candidate
    (n_cand, 4, 4) applied to R_group (one step of the search)."""
    import numpy as np
    n, d, r = _so4_args(x, rot, block, bits)
    c = np.ascontiguousarray(np.asarray(cand, dtype=np.float32).reshape(-1, 4, 4))
    err = np.zeros(c.shape[0], dtype=np.float64)
    _check(okv_so4_eval(x.data_ptr(), n, d, block, bits, eps, r.ctypes.data, c.ctypes.data, c.shape[0], group,
                        err.ctypes.data, stream), "okv_so4_eval")
    return err


def okv_read_probe(buf_ptr: int, nbytes: int, sink_ptr: int, stream=None) -> int:
    return lib.okv_read_probe(ctypes.c_void_p(buf_ptr), nbytes, ctypes.c_void_p(sink_ptr), _stream_ptr(stream))


def read_probe(buf, sink, stream=None):
    """One streaming-read pass over the device tensor buf (okv_read_probe)."""
    _check(okv_read_probe(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(), stream),
           "okv_read_probe")


def okv_destroy(h) -> int:
    return lib.okv_destroy(h)


def okv_get_len(h):
    n = ctypes.c_int32()
    return lib.okv_get_len(h, ctypes.byref(n)), n.value


def okv_set_len(h, n: int) -> int:
    return lib.okv_set_len(h, n)


def okv_set_splits(h, n: int) -> int:
    return lib.okv_set_splits(h, n)


def okv_get_splits(h):
    n = ctypes.c_int32()
    return lib.okv_get_splits(h, ctypes.byref(n)), n.value


def okv_max_splits(h):
    n = ctypes.c_int32()
    return lib.okv_max_splits(h, ctypes.byref(n)), n.value


def okv_timing_enable(h, on: bool) -> int:
    return lib.okv_timing_enable(h, 1 if on else 0)


def okv_timing_read(h):
    n, a, r = ctypes.c_int32(), ctypes.c_double(), ctypes.c_double()
    st = lib.okv_timing_read(h, ctypes.byref(n), ctypes.byref(a), ctypes.byref(r))
    return st, n.value, a.value, r.value


def okv_set_decode_kernel(h, kind: int) -> int:
    return lib.okv_set_decode_kernel(h, kind)


def okv_get_decode_kernel(h):
    n = ctypes.c_int32()
    return lib.okv_get_decode_kernel(h, ctypes.byref(n)), n.value


def make_config(*, batch, num_q_heads, num_kv_heads, head_dim, max_tokens, block=32,
                quant="sym", scale_dtype="f16", in_dtype="bf16", rotation="sign", eps=1e-6,
                rot_params=None, k_codes=0, v_codes=0, k_meta=0, v_meta=0, bits=3):
    """Fill an OkvConfig; ``rot_params`` is a float32 sequence (kept alive on the
    returned object until okv_create copies it)."""
    import array
    cfg = OkvConfig()
    cfg.abi_version = OKV_ABI_VERSION
    cfg.batch, cfg.num_q_heads, cfg.num_kv_heads = batch, num_q_heads, num_kv_heads
    cfg.head_dim, cfg.max_tokens, cfg.block = head_dim, max_tokens, block
    cfg.quant = QUANT[quant] if isinstance(quant, str) else quant
    cfg.scale_dtype = DTYPE[scale_dtype] if isinstance(scale_dtype, str) else scale_dtype
    cfg.in_dtype = DTYPE[in_dtype] if isinstance(in_dtype, str) else in_dtype
    cfg.rotation = ROTATION[rotation] if isinstance(rotation, str) else rotation
    cfg.eps = eps
    cfg.bits = bits
    if rot_params is not None:
        buf = array.array("f", [float(x) for x in rot_params])
        cfg._rot_buf = buf  # keep alive
        addr, _ = buf.buffer_info()
        cfg.rot_params = ctypes.cast(ctypes.c_void_p(addr), ctypes.POINTER(ctypes.c_float))
    cfg.k_codes, cfg.v_codes, cfg.k_meta, cfg.v_meta = k_codes, v_codes, k_meta, v_meta
    return cfg


class OkvCache:
    """A rotated b-bit KV cache (b = 2, 3 or 4; 3 by default) on one GPU: four
    caller-side tensors plus a handle.

    Shapes follow include/okv.h.  ``rot_params`` is the float32 sign vector (d) or
    the (d/4, 4, 4) SO(4) matrices.
    """

    def __init__(self, *, batch, num_q_heads, num_kv_heads, head_dim, max_tokens, block=32,
                 quant="sym", scale_dtype="f16", in_dtype="bf16", rotation="sign", eps=1e-6,
                 rot_params=None, device="cuda", bits=3):
        import numpy as np
        import torch
        self.batch, self.hq, self.hkv, self.d = batch, num_q_heads, num_kv_heads, head_dim
        self.max_tokens, self.block, self.quant, self.scale_dtype = max_tokens, block, quant, scale_dtype
        self.in_dtype = in_dtype
        self.bits = bits
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        rp = np.asarray(rot_params, dtype=np.float32).ravel()
        cfg = make_config(batch=batch, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                          head_dim=head_dim, max_tokens=max_tokens, block=block, quant=quant,
                          scale_dtype=scale_dtype, in_dtype=in_dtype, rotation=rotation, eps=eps,
                          rot_params=rp, bits=bits)
        st, lay = okv_layout(cfg)
        _check(st, "okv_layout")
        nb = head_dim // block
        shp = (batch, num_kv_heads, max_tokens)
        self.k_codes = torch.empty(shp + (bits * head_dim // 8,), dtype=torch.uint8, device=self.device)
        self.v_codes = torch.empty((batch, num_kv_heads, max_tokens // 32, head_dim, 4 * bits),
                                   dtype=torch.uint8, device=self.device)
        if quant == "asym":
            meta_shape, meta_dtype = shp + (nb, 2), torch.uint8
        else:
            meta_shape, meta_dtype = shp + (nb,), (torch.float32 if scale_dtype == "f32" else torch.float16)
        self.k_meta = torch.empty(meta_shape, dtype=meta_dtype, device=self.device)
        self.v_meta = torch.empty(meta_shape, dtype=meta_dtype, device=self.device)
        for t, n in ((self.k_codes, lay.k_codes_bytes), (self.v_codes, lay.v_codes_bytes),
                     (self.k_meta, lay.k_meta_bytes), (self.v_meta, lay.v_meta_bytes)):
            assert t.numel() * t.element_size() == n
        cfg.k_codes, cfg.v_codes = self.k_codes.data_ptr(), self.v_codes.data_ptr()
        cfg.k_meta, cfg.v_meta = self.k_meta.data_ptr(), self.v_meta.data_ptr()
        with torch.cuda.device(self.device):
            st, self.handle = okv_create(cfg)
        _check(st, "okv_create")

    def _in_check(self, t, shape):
        import torch
        want = torch.float32 if self.in_dtype == "f32" else torch.bfloat16
        if t.dtype != want or tuple(t.shape) != tuple(shape) or not t.is_contiguous() or t.device != self.device:
            raise ValueError(f"expected contiguous {want} {tuple(shape)} on {self.device}, "
                             f"got {t.dtype} {tuple(t.shape)} on {t.device}")

    def _stream(self, stream):
        # the current stream of the cache's own device unless one is given
        return _stream_ptr(stream, self.device) if stream is None else stream

    def write(self, k, v, stream=None):
        n_new = k.shape[1]
        shape = (self.batch, n_new, self.hkv, self.d)
        self._in_check(k, shape)
        self._in_check(v, shape)
        _check(okv_write(self.handle, k.data_ptr(), v.data_ptr(), n_new, self._stream(stream)), "okv_write")

    def decode_attn(self, q, out=None, stream=None):
        import torch
        self._in_check(q, (self.batch, self.hq, self.d))
        if out is None:
            out = torch.empty((self.batch, self.hq, self.d), dtype=torch.float32, device=self.device)
        _check(okv_decode_attn(self.handle, q.data_ptr(), out.data_ptr(), self._stream(stream)), "okv_decode_attn")
        return out

    def prefill_attn(self, q, out=None, stream=None):
        """Causal attention of the last q.shape[1] cached positions (q: [batch, n, hq, d])."""
        import torch
        n = q.shape[1]
        self._in_check(q, (self.batch, n, self.hq, self.d))
        if out is None:
            out = torch.empty((self.batch, n, self.hq, self.d), dtype=torch.float32, device=self.device)
        _check(okv_prefill_attn(self.handle, q.data_ptr(), n, out.data_ptr(), self._stream(stream)), "okv_prefill_attn")
        return out

    @property
    def length(self) -> int:
        st, n = okv_get_len(self.handle)
        _check(st, "okv_get_len")
        return n

    def set_length(self, n: int) -> None:
        _check(okv_set_len(self.handle, n), "okv_set_len")

    def set_splits(self, n: int) -> None:
        _check(okv_set_splits(self.handle, n), "okv_set_splits")

    def splits(self) -> int:
        st, n = okv_get_splits(self.handle)
        _check(st, "okv_get_splits")
        return n

    def set_decode_kernel(self, kind: str) -> None:
        """"auto", "per_head" or "grouped" (see okv_set_decode_kernel)."""
        _check(okv_set_decode_kernel(self.handle, DECODE_KERNEL[kind]), "okv_set_decode_kernel")

    def decode_kernel(self) -> str:
        st, n = okv_get_decode_kernel(self.handle)
        _check(st, "okv_get_decode_kernel")
        return {v: k for k, v in DECODE_KERNEL.items()}[n]

    def timing(self, on: bool) -> None:
        _check(okv_timing_enable(self.handle, on), "okv_timing_enable")

    def timing_read(self):
        st, n, a, r = okv_timing_read(self.handle)
        _check(st, "okv_timing_read")
        return n, a, r

    def close(self) -> None:
        if getattr(self, "handle", None):
            okv_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
