"""Seeded synthetic inputs shared by the GPU path's tests/benchmark and the
CPU oracle. This module draws random numbers and casts them; it holds none of
the attention arithmetic.

Recipe (the same for every caller): one CPU ``torch.Generator`` seeded with
``seed``; draw Q, K, V (then dO, if the case has a backward) as fp32
``randn`` of shape (batch, seqlen, nheads, headdim), each scaled by ``std``
(a power of two, so the scaling is exact); then, if the case has key padding,
the per-sequence key lengths L_b = randint(lo, hi + 1); then, if the case is
sampled, the query rows; finally cast Q, K, V, dO to the working dtype with
round-to-nearest-even (``Tensor.to``). dO is drawn with std 1 in every case.

fp8 cases draw Q, K, V the same way, then store each as e4m3 bytes of
x / descale (``Tensor.to(torch.float8_e4m3fn)``, round to nearest even)
with descale = std / 32, a power of two: values up to ~14 std stay inside
e4m3's range (448), and the dequantised value is e4m3(byte) * descale.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import torch

# Named workloads. Shapes follow the pages' examples: B2 H8 N4096 D128 is the
# shape the from-scratch article times and counts IO for; the GPT-2-small
# (H12 D64, seq 1K) and BERT-large (H16 D64, seq 512) shapes stand in for the
# training runs the pages quote; N = 65536 stands in for the 64K-long task.
# No dataset item is used anywhere: all values are random.


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str            # "f32", "bf16", "f16" or "fp8" (e4m3 bytes + a factor per tensor)
    batch: int
    heads: int
    seqlen: int
    headdim: int
    causal: bool = False
    window: tuple = (-1, -1)
    std: float = 1.0
    backward: bool = False
    pad_range: tuple | None = None      # (lo, hi) inclusive for L_b, or None
    sample_rows: int = 0                # >0: the oracle checks this many rows per head
    extra_rows: tuple = field(default=())

    @property
    def softmax_scale(self) -> float:
        return 1.0 / (self.headdim ** 0.5)


WORKLOADS = {
    "fwd_f32_b1h1n256d64": Workload(
        "fwd_f32_b1h1n256d64", "f32", 1, 1, 256, 64),
    "fwd_bf16_b2h8n4096d128": Workload(
        "fwd_bf16_b2h8n4096d128", "bf16", 2, 8, 4096, 128),
    "fwdbwd_bf16_b8h12n1024d64_causal": Workload(
        "fwdbwd_bf16_b8h12n1024d64_causal", "bf16", 8, 12, 1024, 64,
        causal=True, backward=True),
    "fwdbwd_bf16_b32h16n512d64_keypad": Workload(
        "fwdbwd_bf16_b32h16n512d64_keypad", "bf16", 32, 16, 512, 64,
        std=0.5, backward=True, pad_range=(256, 512)),
    "fwd_bf16_b1h16n65536d128_causal": Workload(
        "fwd_bf16_b1h16n65536d128_causal", "bf16", 1, 16, 65536, 128,
        causal=True, sample_rows=256, extra_rows=(0, 1, 4095, 4096, 4097, 65535)),
    "fwd_bf16_b1h16n65536d128_window4096": Workload(
        "fwd_bf16_b1h16n65536d128_window4096", "bf16", 1, 16, 65536, 128,
        causal=True, window=(4096, 0), sample_rows=256,
        extra_rows=(0, 1, 4095, 4096, 4097, 65535)),
    "fwd_fp8_b2h8n4096d128": Workload(
        "fwd_fp8_b2h8n4096d128", "fp8", 2, 8, 4096, 128, sample_rows=256,
        extra_rows=(0, 1, 4095)),
    "fwd_fp8_b1h16n65536d128_causal": Workload(
        "fwd_fp8_b1h16n65536d128_causal", "fp8", 1, 16, 65536, 128,
        causal=True, sample_rows=256, extra_rows=(0, 1, 4095, 4096, 4097, 65535)),
}

METRIC_WORKLOAD = "fwd_bf16_b2h8n4096d128"

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def make_inputs(w: Workload, seed: int = 0):
    """Draw the inputs of workload ``w`` on the CPU.

    Returns a dict with q, k, v (working dtype, CPU), dout (if w.backward),
    seqlens_k (int32 [B] or None) and rows (int64 [H, R] or None).
    """
    g = torch.Generator(device="cpu").manual_seed(int(seed))
    shape = (w.batch, w.seqlen, w.heads, w.headdim)
    fp8 = w.dtype == "fp8"
    dt = None if fp8 else TORCH_DTYPE[w.dtype]
    out = {}
    if fp8:
        out["descale"] = {}
    for name in ("q", "k", "v"):
        x = torch.randn(shape, generator=g, dtype=torch.float32)
        if w.std != 1.0:
            x.mul_(w.std)
        if fp8:
            descale = w.std / 32.0
            out[name] = x.div_(descale).to(torch.float8_e4m3fn).view(torch.uint8)
            out["descale"][name] = descale
        else:
            out[name] = x.to(dt)
        del x
    out["dout"] = None
    if w.backward:
        out["dout"] = torch.randn(shape, generator=g, dtype=torch.float32).to(dt)
    out["seqlens_k"] = None
    if w.pad_range is not None:
        lo, hi = w.pad_range
        out["seqlens_k"] = torch.randint(lo, hi + 1, (w.batch,), generator=g,
                                         dtype=torch.int64).to(torch.int32)
    out["rows"] = None
    if w.sample_rows:
        rows = []
        for _ in range(w.heads):
            r = torch.randperm(w.seqlen, generator=g)[: w.sample_rows]
            extra = torch.tensor([e for e in w.extra_rows if e < w.seqlen],
                                 dtype=torch.int64)
            rows.append(torch.cat([r, extra]))
        out["rows"] = torch.stack(rows)
    return out


def make_case(batch, seqlen, heads, headdim, dtype="bf16", std=1.0, seed=0,
              backward=False, pad_range=None, seqlens_k=None):
    """Inputs of an ad-hoc shape by the same recipe (tests use it for ragged
    and edge shapes). ``seqlens_k`` given explicitly overrides ``pad_range``."""
    w = Workload("case", dtype, batch, heads, seqlen, headdim, std=std,
                 backward=backward, pad_range=pad_range)
    d = make_inputs(w, seed)
    if seqlens_k is not None:
        d["seqlens_k"] = torch.as_tensor(seqlens_k, dtype=torch.int32)
    return d


# Hashed inputs for sizes too large to draw on the host. Element (i, h, d) of
# tensor `kind` is (table index - 128) / 64 with the index
# (a_kind(i) + b_kind(h, d)) mod 256, a and b integer hashes. Every value is a
# multiple of 1/64 in [-2, 2), exact in bf16, and any subset of rows can be
# rebuilt on the CPU without the rest.
_HASH_MUL = {"q": 2654435761, "k": 2246822519, "v": 3266489917, "dout": 668265263}


def hashed_rows(kind, rows, heads, headdim, device="cpu"):
    """bf16 [len(rows), heads, headdim] of hashed tensor `kind` at sequence
    positions `rows` (an int64 tensor)."""
    mul = _HASH_MUL[kind]
    rows = torch.as_tensor(rows, dtype=torch.int64, device=device)
    a = ((rows * mul) >> 11) & 255                                  # [R]
    hd = torch.arange(heads * headdim, dtype=torch.int64, device=device)
    b = ((hd * (mul | 1) + 12345) >> 7) & 255                       # [H*D]
    idx = (a[:, None] + b[None, :]) & 255
    val = ((idx - 128).to(torch.float32) / 64.0).to(torch.bfloat16)
    return val.view(len(rows), heads, headdim)


def hashed_tensor(kind, batch, seqlen, heads, headdim, device, chunk=1 << 20):
    """The whole [batch, seqlen, heads, headdim] hashed tensor (all batch
    entries alike), built on `device` in chunks of rows."""
    out = torch.empty((batch, seqlen, heads, headdim), dtype=torch.bfloat16, device=device)
    for r0 in range(0, seqlen, chunk):
        r1 = min(seqlen, r0 + chunk)
        out[:, r0:r1] = hashed_rows(kind, torch.arange(r0, r1), heads, headdim, device)
    return out


def hashed_fp8_rows(kind, rows, heads, headdim, device="cpu"):
    """e4m3 bytes (torch.uint8) [len(rows), heads, headdim] of hashed tensor
    `kind`: sign, exponent field 5..8 and mantissa taken from the hash, so
    every byte is a finite value of magnitude 0.25 .. 3.75 (no NaN code)."""
    mul = _HASH_MUL[kind]
    rows = torch.as_tensor(rows, dtype=torch.int64, device=device)
    a = ((rows * mul) >> 11) & 255
    hd = torch.arange(heads * headdim, dtype=torch.int64, device=device)
    b = ((hd * (mul | 1) + 12345) >> 7) & 255
    idx = (a[:, None] + b[None, :]) & 255
    code = ((idx >> 7) << 7) | ((5 + ((idx >> 3) & 3)) << 3) | (idx & 7)
    return code.to(torch.uint8).view(len(rows), heads, headdim)


def hashed_fp8_tensor(kind, batch, seqlen, heads, headdim, device, chunk=1 << 20):
    """The whole [batch, seqlen, heads, headdim] hashed e4m3 tensor on `device`."""
    out = torch.empty((batch, seqlen, heads, headdim), dtype=torch.uint8, device=device)
    for r0 in range(0, seqlen, chunk):
        r1 = min(seqlen, r0 + chunk)
        out[:, r0:r1] = hashed_fp8_rows(kind, torch.arange(r0, r1), heads, headdim, device)
    return out
