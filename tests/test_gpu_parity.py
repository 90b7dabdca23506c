"""GPU parity of libokv against the CPU oracle at sizes the oracle finishes quickly.

Codes, scales and zero-points: byte-exact.  Decode output: max |y - y_ref| <=
2e-3 * RMS(y_ref) over each decode call.  Every call goes through the C ABI.
"""
import ctypes

import numpy as np
import pytest
import torch

import okv_synth
from okv_parity import (compare_unit, decode_ref_unit, exact_ties, free_gpu, make_cache, out_error,
                        params_of, round_up, say, unit_inputs)

pytestmark = pytest.mark.gpu

TOL = 2e-3

REDUCED = {
    # name: (overrides, token count, write chunks)
    "tiny_d128_t256": (dict(), 256, [100, 1, 155]),
    "gqa_h32kv8_t32k": (dict(), 1000, [1000]),
    "mha_b4h32_t128k": (dict(batch=2, hq=8, hkv=8), 777, [500, 277]),
    "gqa_b16h64kv8_t128k_asym": (dict(batch=2), 1500, [1500]),
    "so4_d256_b32_t8k": (dict(batch=2), 600, [64, 536]),
}


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def expected_kernel(wl, kernel):
    if kernel != "auto":
        return kernel
    grouped = wl.d in (128, 256) and wl.group in (2, 4, 8) and wl.block in (32, 64, 128)
    return "grouped" if grouped else "per_head"


def run_case(wl, t, chunks, splits=0, steps=0, kernel="auto"):
    """Write t tokens in `chunks`, decode, then `steps` x (append 1, decode).
    Checks every unit's bytes and every decode output against the oracle."""
    _need_gpu()
    p32, u = params_of(wl)
    cache = make_cache(wl, round_up(t + steps + 1, 32), p32)
    if splits:
        cache.set_splits(splits)
    cache.set_decode_kernel(kernel)
    assert cache.decode_kernel() == expected_kernel(wl, kernel)
    k, v = okv_synth.kv_tokens(wl, 0, t, device="cuda")
    pos = 0
    for n in chunks:
        say(wl.name, "okv_write", pos, n)
        cache.write(k[:, pos:pos + n].contiguous(), v[:, pos:pos + n].contiguous())
        pos += n
    assert pos == t and cache.length == t
    errs = []
    k_all, v_all = k, v
    for step in range(steps + 1):
        if step:
            kn, vn = okv_synth.kv_tokens(wl, t + step - 1, 1, device="cuda", step=step)
            say(wl.name, "okv_write append", t + step - 1)
            cache.write(kn, vn)
            k_all = torch.cat([k_all, kn], 1)
            v_all = torch.cat([v_all, vn], 1)
        tt = t + step
        q = okv_synth.queries(wl, step, device="cuda")
        say(wl.name, "okv_decode_attn", cache.decode_kernel(), "T", tt, "splits", cache.splits())
        out = cache.decode_attn(q)
        torch.cuda.synchronize()
        out_h = out.cpu().numpy()
        q_h = okv_synth.host_f32(q)
        y_ref = np.zeros_like(out_h, dtype=np.float64)
        ties = 0
        for b in range(wl.batch):
            for h in range(wl.hkv):
                kh, vh = unit_inputs(k_all, v_all, b, h)
                import oracle
                ref = oracle.write_unit(kh, vh, wl, p32)
                if step == 0 or step == steps:
                    mism = compare_unit(cache, wl, b, h, tt, ref)
                    assert all(x == 0 for x in mism.values()), (b, h, mism)
                    ties += exact_ties(ref, wl)
                y_ref[b, h * wl.group:(h + 1) * wl.group] = decode_ref_unit(wl, q_h, b, h, ref, tt, u)
        err, worst = out_error(out_h, y_ref)
        say(wl.name, f"T={tt} max_err/rms={err:.3e} worst_head={worst:.3e} exact_ties={ties}")
        errs.append(err)
        assert err <= TOL, (tt, err)
    cache.close()
    free_gpu()
    return errs


# every workload with the automatic kernel choice; the grouped workloads also
# with the per-head kernel forced
REDUCED_CASES = [(n, "auto") for n in REDUCED] + [
    (n, "per_head") for n in ("gqa_h32kv8_t32k", "gqa_b16h64kv8_t128k_asym", "so4_d256_b32_t8k")]


@pytest.mark.parametrize("name,kernel", REDUCED_CASES)
def test_write_decode_reduced(name, kernel):
    over, t, chunks = REDUCED[name]
    wl = okv_synth.workload(name).with_(**over)
    run_case(wl, t, chunks, steps=2 if name == "gqa_h32kv8_t32k" else 0, kernel=kernel)


# code widths 2 and 4 (b = 3 above): every format, both decode kernels
WIDTH_CASES = [(n, b, k) for b in (2, 4) for n, k in (
    ("tiny_d128_t256", "auto"), ("mha_b4h32_t128k", "auto"), ("gqa_h32kv8_t32k", "auto"),
    ("gqa_h32kv8_t32k", "per_head"), ("gqa_b16h64kv8_t128k_asym", "auto"),
    ("gqa_b16h64kv8_t128k_asym", "per_head"), ("so4_d256_b32_t8k", "auto"))]


@pytest.mark.parametrize("name,bits,kernel", WIDTH_CASES)
def test_code_widths(name, bits, kernel):
    over, t, chunks = REDUCED[name]
    wl = okv_synth.workload(name).with_(bits=bits, **over)
    run_case(wl, t, chunks, steps=1 if name == "gqa_h32kv8_t32k" else 0, kernel=kernel)


@pytest.mark.parametrize("bits,d,block,quant", [(2, 128, 128, "sym"), (4, 256, 128, "asym"),
                                                (4, 128, 64, "sym"), (2, 256, 256, "asym")])
def test_code_width_block_sizes(bits, d, block, quant):
    meta = "e4m3" if quant == "asym" else "f32"
    rot = "so4" if d == 256 else "sign"
    wl = okv_synth.workload("so4_d256_b32_t8k").with_(
        batch=1, hq=2, hkv=2, d=d, block=block, quant=quant, scale_dtype=meta, rotation=rot, bits=bits)
    run_case(wl, 161, [100, 61], kernel="per_head")


# the unrotated baseline (U = I): per-token blocks (m = d) and blocks of 32/64, both
# decode kernels
@pytest.mark.parametrize("name,over,kernel", [
    ("mha_b4h32_t128k", dict(rotation="none", block=128), "per_head"),
    ("mha_b4h32_t128k", dict(rotation="none"), "per_head"),
    ("gqa_h32kv8_t32k", dict(rotation="none"), "auto"),
    ("gqa_b16h64kv8_t128k_asym", dict(rotation="none"), "auto"),
    ("so4_d256_b32_t8k", dict(rotation="none", block=256), "per_head"),
    ("tiny_d128_t256", dict(rotation="none", bits=4), "auto"),
])
def test_rotation_none(name, over, kernel):
    base, t, chunks = REDUCED[name]
    wl = okv_synth.workload(name).with_(**base).with_(**over)
    run_case(wl, t, chunks, kernel=kernel)


# split counts that reach every load-batch size of the merge (2, 4, 8, 16 and 32 splits
# per thread; 70 and 40 take two batches), at d = 128 (two threads per output) and 256
@pytest.mark.parametrize("t,splits", [(1111, 1), (1111, 3), (1111, 6), (1111, 16), (1111, 32), (4500, 70)])
def test_split_count_invariance(t, splits):
    wl = okv_synth.workload("mha_b4h32_t128k").with_(batch=1, hq=4, hkv=4)
    run_case(wl, t, [t], splits=splits)
    wl = okv_synth.workload("gqa_h32kv8_t32k").with_(batch=1, hq=8, hkv=2)
    run_case(wl, t, [t], splits=splits, kernel="grouped")


@pytest.mark.parametrize("splits", [5, 40])
def test_split_count_invariance_d256(splits):
    wl = okv_synth.workload("so4_d256_b32_t8k").with_(batch=1)
    run_case(wl, 2700, [2700], splits=splits, kernel="grouped")


@pytest.mark.parametrize("d,block,quant", [
    (128, 64, "sym"), (128, 128, "sym"), (128, 32, "asym"), (128, 128, "asym"),
    (256, 64, "sym"), (256, 128, "asym"), (256, 256, "sym"), (256, 256, "asym"),
])
def test_block_sizes(d, block, quant):
    # every quantisation block the library builds, per-head kernel (G = 1) and
    # query groups of 2 (per-head kernel, each KV head read twice)
    meta = "e4m3" if quant == "asym" else "f16"
    rot = "so4" if d == 256 else "sign"
    for hq in (2, 4):
        wl = okv_synth.workload("so4_d256_b32_t8k").with_(
            batch=1, hq=hq, hkv=2, d=d, block=block, quant=quant, scale_dtype=meta, rotation=rot)
        run_case(wl, 300, [200, 100], kernel="per_head")


@pytest.mark.parametrize("t,chunks", [(1, [1]), (32, [32]), (33, [1, 31, 1]), (64, [20, 20, 24]),
                                      (97, [97])])
def test_small_lengths(t, chunks):
    wl = okv_synth.workload("gqa_b16h64kv8_t128k_asym").with_(batch=1, hq=16, hkv=2)
    run_case(wl, t, chunks, kernel="grouped")
    run_case(wl, t, chunks, kernel="per_head")
    wl = okv_synth.workload("so4_d256_b32_t8k").with_(batch=1, hq=4, hkv=1)
    run_case(wl, t, chunks, kernel="grouped")
    wl = okv_synth.workload("tiny_d128_t256")
    run_case(wl, t, chunks)


@pytest.mark.parametrize("kernel", ["grouped", "per_head"])
def test_degenerate_inputs(kernel):
    # all-zero keys: every logit is equal, the output is the mean of the values;
    # constant values: H_d of a constant vector is one spike per vector
    _need_gpu()
    import oracle
    wl = okv_synth.workload("gqa_h32kv8_t32k").with_(batch=1, hq=4, hkv=1)
    p32, u = params_of(wl)
    t = 70
    cache = make_cache(wl, 96, p32)
    cache.set_decode_kernel(kernel)
    k = torch.zeros((1, t, 1, wl.d), dtype=torch.bfloat16, device="cuda")
    v = torch.full((1, t, 1, wl.d), 0.5, dtype=torch.bfloat16, device="cuda")
    v[0, ::3] = -2.0
    say("degenerate okv_write", kernel)
    cache.write(k, v)
    q = okv_synth.queries(wl, 0, device="cuda")
    out = cache.decode_attn(q).cpu().numpy()
    kh, vh = unit_inputs(k, v, 0, 0)
    ref = oracle.write_unit(kh, vh, wl, p32)
    assert all(x == 0 for x in compare_unit(cache, wl, 0, 0, t, ref).values())
    y_ref = decode_ref_unit(wl, okv_synth.host_f32(q), 0, 0, ref, t, u)
    err, _ = out_error(out[0], y_ref)
    assert err <= TOL
    cache.close()


@pytest.mark.parametrize("d,block,quant,hq,kernel,bits", [
    (128, 128, "sym", 1, "per_head", 3), (256, 256, "sym", 2, "per_head", 3),
    (128, 64, "asym", 8, "grouped", 3), (128, 64, "asym", 1, "per_head", 3),
    (128, 128, "sym", 1, "per_head", 4), (128, 64, "asym", 8, "grouped", 4),
    (128, 64, "asym", 1, "per_head", 4), (128, 32, "sym", 4, "grouped", 4),
])
def test_fixed_point_headroom_aligned(d, block, quant, hq, kernel, bits):
    # worst case of the int32 sums of q times codes: the rotated query is constant
    # (every fixed-point element at its limit) and each rotated key block sits at its
    # top code (symmetric: all +-a; asymmetric: 63 of 64 at +a, one at -a), half of
    # the tokens flipped so that the two halves have very different logits
    _need_gpu()
    import oracle
    meta = "e4m3" if quant == "asym" else "f16"
    wl = okv_synth.workload("gqa_h32kv8_t32k").with_(
        batch=1, hq=hq, hkv=1, d=d, block=block, quant=quant, scale_dtype=meta, rotation="sign",
        in_dtype="f32", bits=bits)
    p32, u = params_of(wl)
    t = 96
    yk = np.ones((t, d))
    if quant == "asym":
        yk[:, block - 1::block] = -1.0
    yk[1::2] *= -1.0
    yk *= (0.5 + np.arange(t) / t)[:, None]
    rng = np.random.default_rng(5)
    kx = (yk @ u).astype(np.float32)                       # x = U^T y, as rows
    vx = rng.standard_normal((t, d)).astype(np.float32)
    qx = (np.full((hq, d), 0.05) @ u).astype(np.float32)
    cache = make_cache(wl, 128, p32)
    cache.set_decode_kernel(kernel)
    assert cache.decode_kernel() == kernel
    k = torch.from_numpy(kx).reshape(1, t, 1, d).cuda()
    v = torch.from_numpy(vx).reshape(1, t, 1, d).cuda()
    q = torch.from_numpy(qx).reshape(1, hq, d).cuda()
    say("headroom okv_write/okv_decode_attn", d, block, quant, kernel, "bits", bits)
    cache.write(k, v)
    out = cache.decode_attn(q).cpu().numpy()
    ref = oracle.write_unit(kx, vx, wl, p32)
    assert all(x == 0 for x in compare_unit(cache, wl, 0, 0, t, ref).values())
    y_ref = decode_ref_unit(wl, qx[None], 0, 0, ref, t, u)
    err, _ = out_error(out[0], y_ref)
    say(f"headroom max_err/rms={err:.3e}")
    assert err <= TOL
    cache.close()


@pytest.mark.parametrize("scale_dtype,eps,block,in_dtype", [
    ("f16", 1e-6, 32, "f32"), ("f16", 0.0, 32, "bf16"), ("f16", 0.0, 128, "f32"),
    ("f32", 0.0, 32, "f32"), ("f32", 0.0, 64, "bf16"),
])
def test_tiny_magnitudes_write(scale_dtype, eps, block, in_dtype):
    # vectors from 1e-40 to 1e3 in size (one all-zero token): symmetric scales that are
    # zero or subnormal in their storage type lose relative precision, so |y / s| may
    # pass 3 and the codes must be clipped; scales near the float16 range's top
    # overflow.  Codes and scales byte-exact against the oracle.
    _need_gpu()
    import oracle
    wl = okv_synth.workload("tiny_d128_t256").with_(
        batch=1, hq=2, hkv=1, block=block, quant="sym", scale_dtype=scale_dtype, eps=eps,
        rotation="sign", in_dtype=in_dtype)
    p32, _ = params_of(wl)
    t = 96
    rng = np.random.default_rng(11)
    mag = np.logspace(-40, 3, t)
    kx = (rng.standard_normal((t, wl.d)) * mag[:, None]).astype(np.float32)
    vx = (rng.standard_normal((t, wl.d)) * mag[::-1, None]).astype(np.float32)
    kx[7] = 0.0
    # one outlier element per vector: the other elements of its block sit far below it
    kx[::5, 3] *= 1e4
    k = torch.from_numpy(kx).reshape(1, t, 1, wl.d).to(wl.torch_dtype).cuda()
    v = torch.from_numpy(vx).reshape(1, t, 1, wl.d).to(wl.torch_dtype).cuda()
    cache = make_cache(wl, 128, p32)
    say("tiny magnitudes okv_write", scale_dtype, eps, block, in_dtype)
    cache.write(k, v)
    kh, vh = unit_inputs(k, v, 0, 0)
    ref = oracle.write_unit(kh, vh, wl, p32)
    mism = compare_unit(cache, wl, 0, 0, t, ref)
    assert all(x == 0 for x in mism.values()), mism
    cache.close()


@pytest.mark.parametrize("rotation", ["none", "sign"])
def test_asym_off_centre_blocks_write(rotation):
    # asymmetric blocks whose values sit far from zero relative to their spread (the
    # fast quotient's error bound fails there and the exact rounding takes over), mixed
    # with centred ones; U = I keeps the offsets in every block, the sign flip keeps
    # them only in tokens that are constant plus small noise; byte-exact
    _need_gpu()
    import oracle
    wl = okv_synth.workload("gqa_b16h64kv8_t128k_asym").with_(
        batch=1, hq=8, hkv=1, rotation=rotation, in_dtype="f32")
    p32, _ = params_of(wl)
    t = 96
    rng = np.random.default_rng(23)
    off = rng.uniform(-60.0, 60.0, size=(t, 1))
    spread = np.where(np.arange(t)[:, None] % 3 == 0, 1.0, 0.01)
    kx = (off + spread * rng.standard_normal((t, wl.d))).astype(np.float32)
    vx = (off[::-1] + spread * rng.standard_normal((t, wl.d))).astype(np.float32)
    k = torch.from_numpy(kx).reshape(1, t, 1, wl.d).cuda()
    v = torch.from_numpy(vx).reshape(1, t, 1, wl.d).cuda()
    cache = make_cache(wl, 128, p32)
    say("asym off-centre okv_write", rotation)
    cache.write(k, v)
    ref = oracle.write_unit(kx, vx, wl, p32)
    mism = compare_unit(cache, wl, 0, 0, t, ref)
    assert all(x == 0 for x in mism.values()), mism
    cache.close()


def test_error_paths():
    _need_gpu()
    import decode_attention_okv_amd as okv
    wl = okv_synth.workload("tiny_d128_t256")
    p32, _ = params_of(wl)
    cache = make_cache(wl, 64, p32)
    q = okv_synth.queries(wl, 0, device="cuda")
    out = torch.empty((1, 1, 128), dtype=torch.float32, device="cuda")
    say("error paths")
    assert okv.okv_set_decode_kernel(cache.handle, okv.DECODE_KERNEL["grouped"]) == okv.OKV_E_UNSUPPORTED
    assert okv.okv_set_decode_kernel(cache.handle, 7) == okv.OKV_E_INVALID
    assert cache.decode_kernel() == "per_head"
    assert okv.okv_decode_attn(cache.handle, q.data_ptr(), out.data_ptr()) == okv.OKV_E_INVALID
    k, v = okv_synth.kv_tokens(wl, 0, 65, device="cuda")
    assert okv.okv_write(cache.handle, k.data_ptr(), v.data_ptr(), 65) == okv.OKV_E_CAPACITY
    assert okv.okv_write(cache.handle, k.data_ptr() + 4, v.data_ptr(), 1) == okv.OKV_E_ALIGN
    assert okv.okv_write(cache.handle, k.data_ptr(), v.data_ptr(), 0) == okv.OKV_E_INVALID
    assert cache.length == 0
    cache.write(k[:, :64].contiguous(), v[:, :64].contiguous())
    assert okv.okv_write(cache.handle, k.data_ptr(), v.data_ptr(), 1) == okv.OKV_E_CAPACITY
    assert okv.okv_decode_attn(cache.handle, q.data_ptr() + 4, out.data_ptr()) == okv.OKV_E_ALIGN
    assert okv.okv_decode_attn(cache.handle, q.data_ptr(), out.data_ptr()) == okv.OKV_OK
    torch.cuda.synchronize()
    assert np.isfinite(out.cpu().numpy()).all()
    cache.close()
    assert okv.okv_destroy(ctypes.c_void_p()) == okv.OKV_OK


@pytest.mark.parametrize("nbytes", [16, 4096 * 16 + 48, (1 << 24) + 16 * 77])
def test_read_probe(nbytes):
    # the streaming-read probe reads floor(nbytes / 16) 16-byte elements and writes its
    # sink only when a lane's checksum (xor of element sums) equals 0x9E3779B9: on a zero
    # buffer it stays silent, and planting that value in the first or the last element
    # (the ragged tail) makes exactly one lane write it; argument checks fail before any
    # launch
    _need_gpu()
    import decode_attention_okv_amd as okv
    magic = 0x9E3779B9 - (1 << 32)           # as int32
    n = nbytes // 16
    for planted in (None, 0, n - 1):
        say("okv_read_probe", nbytes, "planted element", planted)
        buf = torch.zeros(4 * n + 4, dtype=torch.int32, device="cuda")
        if planted is not None:
            buf[4 * planted] = magic
        sink = torch.zeros(4, dtype=torch.int32, device="cuda")
        assert okv.okv_read_probe(buf.data_ptr(), nbytes, sink.data_ptr()) == okv.OKV_OK
        torch.cuda.synchronize()
        assert sink.cpu().tolist() == ([0, 0, 0, 0] if planted is None else [magic, 0, 0, 0]), planted
    assert okv.okv_read_probe(buf.data_ptr() + 4, nbytes, sink.data_ptr()) == okv.OKV_E_ALIGN
    assert okv.okv_read_probe(buf.data_ptr(), 15, sink.data_ptr()) == okv.OKV_E_INVALID
    assert okv.okv_read_probe(0, nbytes, sink.data_ptr()) == okv.OKV_E_INVALID


def test_append_overlaps_previous_decode():
    """One-token appends on a second stream, running concurrently with the previous
    decode, give the same outputs bit for bit as the same steps on one stream: an
    append writes position len only and rewrites the earlier codes of the current
    value tile unchanged, and a decode reads positions below len.  Writes stay ordered
    after writes (the side stream waits for the prefill, and its appends follow each
    other on that one stream), as okv_write requires.  The steps cross a 32-token tile
    boundary."""
    _need_gpu()
    for name, over in (("mha_b4h32_t128k", dict(batch=2, hq=4, hkv=4)),
                       ("gqa_b16h64kv8_t128k_asym", dict(batch=2, hq=16, hkv=2))):
        wl = okv_synth.workload(name).with_(**over)
        p32, _ = params_of(wl)
        t0, steps = 1000, 40
        k, v = okv_synth.kv_tokens(wl, 0, t0, device="cuda")
        news = [okv_synth.kv_tokens(wl, t0 + i, 1, device="cuda", step=i + 1) for i in range(steps)]
        qs = [okv_synth.queries(wl, i + 1, device="cuda") for i in range(steps)]
        results = []
        for two_streams in (False, True):
            cache = make_cache(wl, round_up(t0 + steps + 1, 32), p32)
            cache.write(k, v)
            main, side = torch.cuda.current_stream(), torch.cuda.Stream()
            side.wait_stream(main)          # write after write: appends follow the prefill
            say(name, "appends on", "two streams" if two_streams else "one stream")
            outs = []
            for i in range(steps):
                if two_streams:
                    done = torch.cuda.Event()
                    with torch.cuda.stream(side):
                        cache.write(*news[i])
                        done.record(side)
                    main.wait_event(done)
                else:
                    cache.write(*news[i])
                outs.append(cache.decode_attn(qs[i]))
            torch.cuda.synchronize()
            results.append(torch.stack(outs).cpu())
            cache.close()
            free_gpu()
        assert torch.equal(results[0], results[1]), name


def test_asym_zero_point_block_by_hand():
    """The hand-worked asymmetric block of the CPU pins (minimum -1.03125 stored as the
    E4M3 zero-point -1.0, an E4M3 scale tie, exact code ties, a difference y - z that
    float32 rounds onto a tie, and a constant block with scale 0) through okv_write
    with U = I: the stored key row, value codes and metadata equal the hand-typed
    values."""
    _need_gpu()
    import oracle
    from test_oracle_quant import asym_pin_block
    y, codes, meta = asym_pin_block()
    wl = okv_synth.workload("gqa_b16h64kv8_t128k_asym").with_(
        batch=1, hq=1, hkv=1, rotation="none", in_dtype="f32")
    p32, _ = params_of(wl)
    cache = make_cache(wl, 32, p32)
    x = torch.from_numpy(y).reshape(1, 1, 1, 128).cuda()
    say("asym hand-worked block okv_write")
    cache.write(x, (-x).contiguous())
    torch.cuda.synchronize()
    k_u = oracle.unpack_rows(cache.k_codes[0, 0, :1].cpu().numpy(), 128)[0]
    assert k_u.tolist() == codes
    assert cache.k_meta[0, 0, 0].cpu().numpy().view(np.uint8).reshape(2, 2).tolist() == meta
    # the values are -y: a different block, checked against the oracle's quantiser
    v_u = oracle.unpack_vtiles(cache.v_codes[0, 0, :1].cpu().numpy(), 1)[0]
    want_u, want_meta = oracle.quantize_f32(-y[None], wl)
    assert v_u.tolist() == want_u[0].tolist()
    assert cache.v_meta[0, 0, 0].cpu().numpy().view(np.uint8).reshape(2, 2).tolist() == want_meta[0].tolist()
    cache.close()


# grouped decode over every query group it is built for (2, 4, 8) and blocks of 32, 64
# and 128 dims: (head, block) rows in one or two 16-row sets, P.V rows of four heads
@pytest.mark.parametrize("d,block,quant,group,meta", [
    (128, 32, "sym", 8, "f16"), (128, 32, "asym", 8, "e4m3"), (128, 32, "sym", 2, "f32"),
    (128, 64, "sym", 2, "f16"), (128, 64, "asym", 4, "e4m3"), (128, 128, "sym", 8, "f16"),
    (128, 128, "asym", 2, "e4m3"), (256, 32, "sym", 8, "f16"), (256, 64, "asym", 2, "e4m3"),
    (256, 128, "sym", 4, "f32"),
])
def test_grouped_shapes(d, block, quant, group, meta):
    rot = "so4" if d == 256 else "sign"
    wl = okv_synth.workload("gqa_h32kv8_t32k").with_(
        batch=2, hq=2 * group, hkv=2, d=d, block=block, quant=quant, scale_dtype=meta, rotation=rot)
    run_case(wl, 700, [300, 400], steps=1, kernel="grouped")
    run_case(wl, 97, [97], splits=3, kernel="grouped")
