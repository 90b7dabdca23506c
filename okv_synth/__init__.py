"""Seeded synthetic workloads for the rotated 3-bit KV cache.

This module only draws random numbers and describes workload shapes.  It holds
none of the method's arithmetic (no rotation, no quantisation, no attention), so
it may serve both the CPU oracle and the HIP library's tests and benchmark.

Value model (from "Orthogonal Invariance in Activation Space", Section 2.1,
"Empirical Analysis of KV Outliers"): a few percent of the channels of a key or
value head carry extreme magnitudes (Pattern 1), key magnitudes decay along the
sequence (Pattern 2) and middle layers have a denser outlier set (Pattern 3,
8.3 % of the dimensions).  Concretely, per (tensor, KV head):

* every channel c gets a scale sigma_c ~ lognormal(mean 0, sigma 0.5);
* round(frac * d) channels, drawn without replacement, are multiplied by 20 and
  stay outliers for every token;
* the values are N(0, 1) * sigma_c;
* with ``key_decay`` the keys at position p are further scaled by
  (1 + p / 4096) ** -0.3;
* the result is rounded (RNE) to the input dtype.

Queries are N(0, 1) in the input dtype.  Rotation parameters are random signs
(D = diag(+-1)) or, for the SO(4) variant, 4x4 rotations built from pairs of
unit quaternions (x -> qL * x * conj(qR)), as "Orthogonally mixed 3-bit KV
cache", Implementation notes, suggests.

Small per-head arrays (channel scales, outlier sets, rotation parameters) come
from NumPy ``SeedSequence([workload_id, stream, ...])`` so they are identical on
every host.  The bulk normal draws come from a seeded ``torch.Generator`` on the
device the tensor is made on; tests that compare two implementations always
hand both the same tensor (or a host copy of it).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "workload", "channel_model", "rotation_params",
           "kv_tokens", "queries", "query_rows", "so4_candidates"]

# stream ids of the SeedSequence
_S_ROT, _S_KCH, _S_VCH, _S_K, _S_V, _S_Q, _S_STEP, _S_QROWS, _S_CAL = range(9)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    wid: int              # numeric id used in seeds
    batch: int
    hq: int               # query heads
    hkv: int              # key/value heads
    d: int                # head dimension
    tokens: int           # context length written before decoding
    in_dtype: str         # 'f32' | 'bf16'  (k, v and q)
    quant: str            # 'sym' | 'asym'
    block: int            # quantisation block m
    scale_dtype: str      # 'f32' | 'f16' | 'e4m3'
    rotation: str         # 'sign' (U = H_d D) | 'so4' (U = B H_d) | 'none' (U = I)
    outlier_frac: float
    key_decay: bool
    decode_steps: int     # append-one-then-decode steps after the prefill
    eps: float = 1e-6
    bits: int = 3         # code width b (2, 3 or 4)

    @property
    def group(self) -> int:
        return self.hq // self.hkv

    @property
    def torch_dtype(self):
        return torch.float32 if self.in_dtype == "f32" else torch.bfloat16

    def meta_bytes_per_row(self) -> int:
        nblk = self.d // self.block
        return nblk * {"f32": 4, "f16": 2, "e4m3": 2}[self.scale_dtype]

    def row_bytes(self) -> int:
        """Bytes one (token, KV head, tensor) record occupies: codes + metadata."""
        return self.bits * self.d // 8 + self.meta_bytes_per_row()

    def cache_bytes(self, tokens: int | None = None) -> int:
        t = self.tokens if tokens is None else tokens
        return 2 * self.batch * self.hkv * t * self.row_bytes()

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    w.name: w
    for w in [
        # one head, d=128, 256 tokens, fp32 inputs and scales
        Workload("tiny_d128_t256", 1, 1, 1, 1, 128, 256, "f32", "sym", 32, "f32", "sign",
                 0.03, False, 1),
        # Llama-3-8B-shaped GQA: 32 query / 8 KV heads, 32K context, decaying keys
        Workload("gqa_h32kv8_t32k", 2, 1, 32, 8, 128, 32768, "bf16", "sym", 32, "f16", "sign",
                 0.03, True, 256),
        # 7B MHA shape at 128K: batch 4, 32 heads, middle-layer outlier density
        Workload("mha_b4h32_t128k", 3, 4, 32, 32, 128, 131072, "bf16", "sym", 32, "f16", "sign",
                 0.083, False, 20),
        # 70B-shaped per-GPU layer share at 128K: batch 16, 64 q / 8 KV heads, asymmetric fp8 meta
        Workload("gqa_b16h64kv8_t128k_asym", 4, 16, 64, 8, 128, 131072, "bf16", "asym", 64, "e4m3",
                 "sign", 0.03, False, 20),
        # SO(4)-mixed d=256: batch 32, 32 q / 8 KV heads, 8K context
        Workload("so4_d256_b32_t8k", 5, 32, 32, 8, 256, 8192, "bf16", "sym", 32, "f16", "so4",
                 0.03, False, 20),
    ]
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def _rng(wl: Workload, *key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([wl.wid, *key]))


def _quat_left(a):
    a0, a1, a2, a3 = a
    return np.array([[a0, -a1, -a2, -a3], [a1, a0, -a3, a2], [a2, a3, a0, -a1], [a3, -a2, a1, a0]])


def _quat_right(b):
    b0, b1, b2, b3 = b
    return np.array([[b0, -b1, -b2, -b3], [b1, b0, b3, -b2], [b2, -b3, b0, b1], [b3, b2, -b1, b0]])


def rotation_params(wl: Workload, seed: int = 0, dtype=np.float64) -> np.ndarray:
    """Fixed random rotation parameters, drawn once per handle.

    'sign': d values in {+1, -1}.  'so4': (d/4, 4, 4) rotation matrices, row-major,
    R = L(qL) R(conj(qR)) with qL, qR unit quaternions (normalised N(0, I_4); x0 is
    the real part), so R x is the quaternion product qL * x * conj(qR).
    """
    if wl.rotation == "none":              # U = I: no parameters (d ones, unused)
        return np.ones(wl.d, dtype=dtype)
    rng = _rng(wl, _S_ROT, seed)
    if wl.rotation == "sign":
        return np.where(rng.random(wl.d) < 0.5, -1.0, 1.0).astype(dtype)
    mats = []
    for _ in range(wl.d // 4):
        ql = rng.standard_normal(4)
        qr = rng.standard_normal(4)
        ql /= np.linalg.norm(ql)
        qr /= np.linalg.norm(qr)
        qr_conj = qr * np.array([1.0, -1.0, -1.0, -1.0])
        mats.append(_quat_left(ql) @ _quat_right(qr_conj))
    return np.stack(mats).astype(dtype)


def so4_candidates(d: int, sweeps: int, n_cand: int, sigma: float = 0.15, seed: int = 0) -> np.ndarray:
    """Candidate perturbations for the SO(4) calibration search, drawn once:
    (sweeps, d/4, n_cand, 4, 4) float64 rotations; candidate 0 is the identity, the
    others are L(a) R(conj(b)) for unit quaternions a, b near 1 (real part 1, imaginary
    parts sigma * N(0, 1), normalised)."""
    rng = np.random.default_rng(np.random.SeedSequence([_S_CAL, d, sweeps, n_cand, seed]))
    out = np.zeros((sweeps, d // 4, n_cand, 4, 4))
    for s in range(sweeps):
        for g in range(d // 4):
            out[s, g, 0] = np.eye(4)
            for c in range(1, n_cand):
                a = np.concatenate([[1.0], sigma * rng.standard_normal(3)])
                b = np.concatenate([[1.0], sigma * rng.standard_normal(3)])
                a /= np.linalg.norm(a)
                b /= np.linalg.norm(b)
                out[s, g, c] = _quat_left(a) @ _quat_right(b * np.array([1.0, -1.0, -1.0, -1.0]))
    return out


def channel_model(wl: Workload, tensor: str, head: int):
    """Per-channel scale vector (float64, length d) of one (tensor, KV head)."""
    stream = _S_KCH if tensor == "k" else _S_VCH
    rng = _rng(wl, stream, head)
    sigma = rng.lognormal(mean=0.0, sigma=0.5, size=wl.d)
    n_out = int(round(wl.outlier_frac * wl.d))
    if n_out:
        idx = rng.choice(wl.d, size=n_out, replace=False)
        sigma[idx] *= 20.0
    return sigma


def _gen(device, *key: int) -> torch.Generator:
    ss = np.random.SeedSequence(list(key))
    g = torch.Generator(device=device)
    g.manual_seed(int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1)))
    return g


def kv_tokens(wl: Workload, pos0: int, n: int, device="cpu", step: int = -1):
    """K and V for positions [pos0, pos0 + n) of every sequence: [B][n][Hkv][d].

    ``step`` selects an independent draw for decode-time appends (-1: prefill).
    """
    out = []
    for tensor, stream in (("k", _S_K), ("v", _S_V)):
        g = _gen(device, wl.wid, stream, step + 1, pos0)
        x = torch.randn((wl.batch, n, wl.hkv, wl.d), generator=g, device=device,
                        dtype=torch.float32)
        sig = torch.tensor(np.stack([channel_model(wl, tensor, h) for h in range(wl.hkv)]),
                           dtype=torch.float32, device=device)
        x.mul_(sig.view(1, 1, wl.hkv, wl.d))
        if tensor == "k" and wl.key_decay:
            pos = torch.arange(pos0, pos0 + n, device=device, dtype=torch.float64)
            decay = torch.pow(1.0 + pos / 4096.0, -0.3).to(torch.float32)
            x.mul_(decay.view(1, n, 1, 1))
        out.append(x.to(wl.torch_dtype))
    return out[0], out[1]


def queries(wl: Workload, step: int = 0, device="cpu"):
    """One query token per (sequence, query head): [B][Hq][d] in the input dtype."""
    g = _gen(device, wl.wid, _S_Q, step)
    q = torch.randn((wl.batch, wl.hq, wl.d), generator=g, device=device, dtype=torch.float32)
    return q.to(wl.torch_dtype)


def query_rows(wl: Workload, pos0: int, n: int, device="cpu"):
    """Query rows of the new positions [pos0, pos0 + n) of every sequence (prefill):
    [B][n][Hq][d] in the input dtype, N(0,1)."""
    g = _gen(device, wl.wid, _S_QROWS, pos0, n)
    q = torch.randn((wl.batch, n, wl.hq, wl.d), generator=g, device=device, dtype=torch.float32)
    return q.to(wl.torch_dtype)


def host_f32(x: torch.Tensor) -> np.ndarray:
    """Exact float32 host copy of an input tensor (bf16 widens exactly)."""
    return x.detach().to("cpu").to(torch.float32).numpy()


def _check():
    for w in WORKLOADS.values():
        assert w.hq % w.hkv == 0 and w.d % w.block == 0
        assert math.log2(w.d).is_integer()


_check()
