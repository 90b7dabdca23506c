"""The C-ABI library loads, exports what include/okv.h declares and rejects bad
arguments on the host (CPU only: no call here reaches the GPU)."""
import ctypes
import os
import re

import pytest

import decode_attention_okv_amd as okv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "okv.h")).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(okv_\w+)\s*\(", text, re.M)))


def test_every_declared_symbol_is_exported():
    names = header_functions()
    assert {"okv_create", "okv_write", "okv_decode_attn", "okv_destroy"} <= set(names)
    for n in names:
        assert hasattr(okv.lib, n), n
    assert set(names) == set(okv.EXPORTS)


def base(**kw):
    args = dict(batch=2, num_q_heads=8, num_kv_heads=2, head_dim=128, max_tokens=1024, block=32,
                quant="sym", scale_dtype="f16", in_dtype="bf16", rotation="sign",
                rot_params=[1.0] * 128, k_codes=4096, v_codes=8192, k_meta=16384, v_meta=32768)
    args.update(kw)
    return okv.make_config(**args)


def test_largest_slice_is_accepted_4bit():
    st, lay = okv.okv_layout(base(max_tokens=67108704, bits=4))   # (67108704 + 128) x 64 < 2^32
    assert st == okv.OKV_OK and lay.k_codes_bytes == 2 * 2 * 67108704 * 64


def test_largest_slice_is_accepted():
    st, lay = okv.okv_layout(base(max_tokens=89478336))   # (89478336 + 128) x 48 < 2^32
    assert st == okv.OKV_OK and lay.k_codes_bytes == 2 * 2 * 89478336 * 48   # batch 2 x 2 KV heads


def test_layout_sizes():
    st, lay = okv.okv_layout(base())
    assert st == okv.OKV_OK
    rows = 2 * 2 * 1024
    assert lay.k_codes_bytes == rows * 48 and lay.v_codes_bytes == rows * 48
    assert lay.k_meta_bytes == rows * 4 * 2
    st, lay = okv.okv_layout(base(quant="asym", scale_dtype="e4m3", block=64))
    assert st == okv.OKV_OK and lay.k_meta_bytes == rows * 2 * 2
    st, lay = okv.okv_layout(base(scale_dtype="f32", head_dim=256, rot_params=[1.0] * 256))
    assert st == okv.OKV_OK and lay.k_codes_bytes == rows * 96 and lay.k_meta_bytes == rows * 8 * 4
    # code widths 2 and 4: b d / 8 bytes per row, 4 b bytes per value group
    for bits in (2, 4):
        st, lay = okv.okv_layout(base(bits=bits))
        assert st == okv.OKV_OK
        assert lay.k_codes_bytes == rows * bits * 16 and lay.v_codes_bytes == rows * bits * 16
        assert lay.k_meta_bytes == rows * 4 * 2


@pytest.mark.parametrize("kw,status", [
    (dict(abi_version=99), okv.OKV_E_INVALID),
    (dict(batch=0), okv.OKV_E_INVALID),
    (dict(num_q_heads=7), okv.OKV_E_INVALID),            # Hq mod Hkv != 0
    (dict(head_dim=96), okv.OKV_E_INVALID),              # not a power of two
    (dict(block=24), okv.OKV_E_INVALID),                 # does not divide d
    (dict(block=12), okv.OKV_E_INVALID),                 # 8 does not divide m
    (dict(max_tokens=1000), okv.OKV_E_INVALID),          # not a multiple of 32
    (dict(quant=5), okv.OKV_E_INVALID),
    (dict(in_dtype="f16"), okv.OKV_E_INVALID),
    (dict(rotation=3), okv.OKV_E_INVALID),
    (dict(bits=1), okv.OKV_E_INVALID),
    (dict(bits=5), okv.OKV_E_INVALID),
    (dict(bits=8), okv.OKV_E_INVALID),
    (dict(eps=-1.0), okv.OKV_E_INVALID),
    (dict(eps=float("nan")), okv.OKV_E_INVALID),
    (dict(scale_dtype="bf16"), okv.OKV_E_INVALID),
    (dict(scale_dtype="e4m3"), okv.OKV_E_UNSUPPORTED),   # symmetric with FP8 scales: not built
    (dict(quant="asym", scale_dtype="f16"), okv.OKV_E_UNSUPPORTED),
    (dict(head_dim=64, rot_params=[1.0] * 64), okv.OKV_E_UNSUPPORTED),
    (dict(block=16), okv.OKV_E_UNSUPPORTED),
    # one (sequence, KV head) slice of packed codes must stay below 4 GiB
    (dict(max_tokens=89478368), okv.OKV_E_UNSUPPORTED),   # 48 B rows: (89478368 + 128) x 48 > 2^32
    (dict(max_tokens=44739264, head_dim=256, rot_params=[1.0] * 256), okv.OKV_E_UNSUPPORTED),
    (dict(max_tokens=67108736, bits=4), okv.OKV_E_UNSUPPORTED),   # 64 B rows: (67108736 + 128) x 64 >= 2^32
    (dict(batch=65536), okv.OKV_E_UNSUPPORTED),                    # launch grid dimensions
    (dict(num_q_heads=65536, num_kv_heads=2), okv.OKV_E_UNSUPPORTED),
])
def test_rejections(kw, status):
    cfg = base(**{k: v for k, v in kw.items() if k != "abi_version"})
    if "abi_version" in kw:
        cfg.abi_version = kw["abi_version"]
    assert okv.okv_layout(cfg)[0] == status
    st, h = okv.okv_create(cfg)
    assert st == status and not h.value


def test_rotation_none_layout():
    # U = I: no rotation parameters needed; layout as for any rotation
    cfg = base(rotation="none", block=128)
    cfg.rot_params = None
    st, lay = okv.okv_layout(cfg)
    assert st == okv.OKV_OK and lay.k_meta_bytes == 2 * 2 * 1024 * 1 * 2


def test_create_rejects_bad_pointers_and_params_before_gpu():
    st, h = okv.okv_create(base(k_codes=0))
    assert st == okv.OKV_E_INVALID
    st, h = okv.okv_create(base(v_meta=32768 + 4))
    assert st == okv.OKV_E_ALIGN
    st, h = okv.okv_create(base(rot_params=[1.0] * 127 + [0.5]))
    assert st == okv.OKV_E_INVALID                       # a sign that is not +-1
    cfg = base()
    cfg.rot_params = None
    assert okv.okv_create(cfg)[0] == okv.OKV_E_INVALID
    import numpy as np
    bad = np.tile(np.eye(4, dtype=np.float32) * 2, (32, 1, 1)).ravel()
    assert okv.okv_create(base(rotation="so4", rot_params=bad))[0] == okv.OKV_E_INVALID
    assert okv.lib.okv_create(ctypes.byref(base()), None) == okv.OKV_E_INVALID


def test_null_handle_calls():
    null = ctypes.c_void_p()
    assert okv.okv_destroy(null) == okv.OKV_OK
    assert okv.okv_write(null, 16, 16, 1, 0) == okv.OKV_E_INVALID
    assert okv.okv_decode_attn(null, 16, 16, 0) == okv.OKV_E_INVALID
    assert okv.okv_get_len(null)[0] == okv.OKV_E_INVALID
    assert okv.okv_set_splits(null, 4) == okv.OKV_E_INVALID
    assert okv.okv_timing_read(null)[0] == okv.OKV_E_INVALID
    assert okv.okv_set_decode_kernel(null, 0) == okv.OKV_E_INVALID
    assert okv.okv_get_decode_kernel(null)[0] == okv.OKV_E_INVALID
    assert okv.okv_prefill_attn(null, 16, 1, 16, 0) == okv.OKV_E_INVALID
    assert okv.okv_strerror(okv.OKV_E_CAPACITY) == "cache capacity exceeded"


@pytest.mark.parametrize("kw,status", [
    (dict(x=0), okv.OKV_E_INVALID),
    (dict(n=0), okv.OKV_E_INVALID),
    (dict(x=20), okv.OKV_E_ALIGN),
    (dict(bits=5), okv.OKV_E_INVALID),
    (dict(eps=-1.0), okv.OKV_E_INVALID),
    (dict(block=48), okv.OKV_E_INVALID),          # does not divide 128
    (dict(d=96, block=32), okv.OKV_E_UNSUPPORTED),
    (dict(n_cand=0), okv.OKV_E_INVALID),
    (dict(n_cand=2000), okv.OKV_E_INVALID),
    (dict(n=1 << 24), okv.OKV_E_UNSUPPORTED),     # n * d >= 2^31
])
def test_so4_calibration_rejects_before_gpu(kw, status):
    import numpy as np
    a = dict(x=256, n=64, d=128, block=32, bits=3, eps=1e-6, n_cand=4)
    a.update(kw)
    rot = np.tile(np.eye(4, dtype=np.float32), (32, 1, 1))
    cand = np.tile(np.eye(4, dtype=np.float32), (32 * a["n_cand"] if a["n_cand"] > 0 else 1, 1, 1))
    trace = np.zeros(2)
    assert okv.okv_so4_calibrate(a["x"], a["n"], a["d"], a["block"], a["bits"], a["eps"], rot.ctypes.data,
                                 cand.ctypes.data, 1, a["n_cand"], trace.ctypes.data, 0) == status
    err = np.zeros(max(a["n_cand"], 1))
    assert okv.okv_so4_eval(a["x"], a["n"], a["d"], a["block"], a["bits"], a["eps"], rot.ctypes.data,
                            cand.ctypes.data, a["n_cand"], 0, err.ctypes.data, 0) == status
