"""Seeded synthetic inputs for exact tiled attention.

This module is shared by the HIP path's tests and benchmark and by the CPU
oracle's tests.  It draws random numbers and rounds them to the storage dtype;
it contains none of the attention arithmetic.

Recipe (the same for every workload):

* ``rng = numpy.random.default_rng(seed)``; every tensor is drawn with
  ``rng.standard_normal(shape, dtype=float32)`` in the order the workload
  lists them (prefill: q, k, v, and for the backward pass the output
  gradient dout after them; decode: seqlens first, then q, k-cache,
  v-cache).
* An optional query multiplier (3.0 for the Qwen3-0.6B-shaped workload, 100
  for the stability case) is applied in fp32 *before* rounding.
* bf16 storage rounds each fp32 value once, round-to-nearest-even, done with
  integer bit arithmetic so the result does not depend on any library's
  conversion routine.  The rounded bit patterns are what both the GPU and the
  oracle consume.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


# --------------------------------------------------------------------------
# fp32 <-> bf16 storage conversion (bit arithmetic, round-to-nearest-even)
# --------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (RNE) and return the 16-bit patterns (uint16)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    r = ((u + bias) >> 16).astype(np.uint16)
    if nan.any():
        r = np.where(nan, ((u >> 16) | 0x0040).astype(np.uint16), r)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to the fp32 values they encode (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


BF16_NAN = np.uint16(0x7FC0)


# --------------------------------------------------------------------------
# Workloads
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Prefill:
    """A forward (prefill) workload; q:[B,Hq,Tq,d], k,v:[B,Hkv,Tk,d]."""
    name: str
    B: int
    Hq: int
    Hkv: int
    Tq: int
    Tk: int
    d: int
    causal: bool
    dtype: str = "bf16"          # "bf16", "f32", or "fp8" (E4M3 with block scales)
    q_mult: float = 1.0
    seed: int = 0
    align: str = "top_left"      # causal diagonal: "top_left" or "bottom_right"

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    @property
    def causal_mode(self) -> int:
        """The C ABI's causal argument: 0 none, 1 top-left, 2 bottom-right."""
        if not self.causal:
            return 0
        return 2 if self.align == "bottom_right" else 1

    @property
    def flops(self) -> float:
        """Attention FLOPs, 4*B*Hq*Tq*Tk*d, halved for causal.  For a
        bottom-right chunk (Tq < Tk) the Tk - Tq cached keys are seen by every
        row and the square part is halved: 4*B*Hq*d*Tq*(Tk - Tq + Tq/2)."""
        f = 4.0 * self.B * self.Hq * self.Tq * self.Tk * self.d
        if not self.causal:
            return f
        if self.align == "bottom_right" and self.Tk > self.Tq:
            return 4.0 * self.B * self.Hq * self.d * self.Tq * (self.Tk - self.Tq + self.Tq / 2)
        return f / 2

    @property
    def bwd_flops(self) -> float:
        """Backward FLOPs: the five products S = QK^T (recomputed), dP = dO V^T,
        dV = P^T dO, dQ = dS K, dK = dS^T Q, i.e. 10*B*Hq*Tq*Tk*d, halved
        for causal (2.5 times the forward's)."""
        return 2.5 * self.flops

    @property
    def min_bytes(self) -> int:
        """Bytes that must cross HBM once: q, k, v read; o, lse written (8-bit
        inputs: the codes and their scales read, o written in bf16)."""
        rows = self.B * self.Hq * self.Tq
        if self.dtype == "fp8":
            q = rows * (self.d + 4)
            kv = 2 * self.B * self.Hkv * (self.Tk * self.d + 4)
            return q + kv + rows * self.d * 2 + rows * 4
        es = 2 if self.dtype == "bf16" else 4
        q = rows * self.d * es
        kv = 2 * self.B * self.Hkv * self.Tk * self.d * es
        return 2 * q + kv + rows * 4


@dataclasses.dataclass(frozen=True)
class Decode:
    """A single-query decode workload over a KV cache.

    q:[B,Hq,d]; kcache,vcache:[B,Hkv,Tk_max,d]; seqlens:[B] int32 drawn
    uniformly from [seq_lo, seq_hi] inclusive.
    """
    name: str
    B: int
    Hq: int
    Hkv: int
    Tk_max: int
    d: int
    seq_lo: int
    seq_hi: int
    seed: int = 0
    kv_dtype: str = "bf16"       # "bf16"; "fp8" (E4M3) or "int8" codes with one fp32 scale per row

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d))


# The five workloads the pages' hot path is measured on, and a chunked-prefill
# workload for the bottom-right causal alignment.
SINGLE_HEAD_F32 = Prefill("single-head fp32 attention, T=256, d=64, non-causal",
                          B=1, Hq=1, Hkv=1, Tq=256, Tk=256, d=64, causal=False,
                          dtype="f32")
GPT2_SMALL_MHA = Prefill("GPT-2-small MHA causal prefill, B=8, H=12, T=4096, d=64",
                         B=8, Hq=12, Hkv=12, Tq=4096, Tk=4096, d=64, causal=True)
QWEN3_0P6B_GQA = Prefill("Qwen3-0.6B GQA causal prefill, Hq=16, Hkv=8, T=4096, d=128, Qx3",
                         B=1, Hq=16, Hkv=8, Tq=4096, Tk=4096, d=128, causal=True,
                         q_mult=3.0)
LLAMA3_8B_LONG = Prefill("Llama-3-8B GQA causal prefill, Hq=32, Hkv=8, T=32768, d=128",
                         B=1, Hq=32, Hkv=8, Tq=32768, Tk=32768, d=128, causal=True)
LLAMA3_8B_CHUNK = Prefill("Llama-3-8B GQA chunked prefill, last 4096 of 32768 positions "
                          "(bottom-right causal), Hq=32, Hkv=8, d=128",
                          B=1, Hq=32, Hkv=8, Tq=4096, Tk=32768, d=128, causal=True,
                          align="bottom_right")
GPT2_SMALL_MHA_FP8 = Prefill("GPT-2-small MHA causal prefill in 8 bits (E4M3 q per-row, k/v "
                             "per-head scales), B=8, H=12, T=4096, d=64",
                             B=8, Hq=12, Hkv=12, Tq=4096, Tk=4096, d=64, causal=True, dtype="fp8")
QWEN3_0P6B_GQA_FP8 = Prefill("Qwen3-0.6B GQA causal prefill in 8 bits, Hq=16, Hkv=8, T=4096, "
                             "d=128, Qx3", B=1, Hq=16, Hkv=8, Tq=4096, Tk=4096, d=128, causal=True,
                             q_mult=3.0, dtype="fp8")
LLAMA3_8B_LONG_FP8 = Prefill("Llama-3-8B GQA causal prefill in 8 bits, Hq=32, Hkv=8, T=32768, "
                             "d=128", B=1, Hq=32, Hkv=8, Tq=32768, Tk=32768, d=128, causal=True,
                             dtype="fp8")
FLASH_DECODE = Decode("split-KV decode, B=16, Hq=32, Hkv=8, d=128, seqlen U[1024,32768]",
                      B=16, Hq=32, Hkv=8, Tk_max=32768, d=128, seq_lo=1024, seq_hi=32768)

FLASH_DECODE_FP8 = Decode("split-KV decode over an fp8 (E4M3, per-row scale) cache, B=16, Hq=32, "
                          "Hkv=8, d=128, seqlen U[1024,32768]",
                          B=16, Hq=32, Hkv=8, Tk_max=32768, d=128, seq_lo=1024, seq_hi=32768,
                          kv_dtype="fp8")
FLASH_DECODE_INT8 = Decode("split-KV decode over an int8 (per-row scale) cache, B=16, Hq=32, "
                           "Hkv=8, d=128, seqlen U[1024,32768]",
                           B=16, Hq=32, Hkv=8, Tk_max=32768, d=128, seq_lo=1024, seq_hi=32768,
                           kv_dtype="int8")

WORKLOADS = {
    "single_head_f32": SINGLE_HEAD_F32,
    "gpt2_small_mha": GPT2_SMALL_MHA,
    "qwen3_0p6b_gqa": QWEN3_0P6B_GQA,
    "llama3_8b_long": LLAMA3_8B_LONG,
    "llama3_8b_chunk": LLAMA3_8B_CHUNK,
    "gpt2_small_mha_fp8": GPT2_SMALL_MHA_FP8,
    "qwen3_0p6b_gqa_fp8": QWEN3_0P6B_GQA_FP8,
    "llama3_8b_long_fp8": LLAMA3_8B_LONG_FP8,
    "flash_decode": FLASH_DECODE,
    "flash_decode_fp8": FLASH_DECODE_FP8,
    "flash_decode_int8": FLASH_DECODE_INT8,
}


def _draw(rng: np.random.Generator, shape, dtype: str, mult: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if mult != 1.0:
        x *= np.float32(mult)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f32":
        return x
    raise ValueError(f"unknown dtype {dtype!r}")


def prefill_inputs(w: Prefill, *, seed: Optional[int] = None):
    """Return (q, k, v) as uint16 bf16 patterns or float32 arrays, row-major."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    q = _draw(rng, (w.B, w.Hq, w.Tq, w.d), w.dtype, w.q_mult)
    k = _draw(rng, (w.B, w.Hkv, w.Tk, w.d), w.dtype)
    v = _draw(rng, (w.B, w.Hkv, w.Tk, w.d), w.dtype)
    return q, k, v


def prefill_inputs_with_grad(w: Prefill, *, seed: Optional[int] = None):
    """(q, k, v, dout): q, k, v exactly as prefill_inputs draws them, then the
    output gradient dout [B,Hq,Tq,d] drawn next from the same generator."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    q = _draw(rng, (w.B, w.Hq, w.Tq, w.d), w.dtype, w.q_mult)
    k = _draw(rng, (w.B, w.Hkv, w.Tk, w.d), w.dtype)
    v = _draw(rng, (w.B, w.Hkv, w.Tk, w.d), w.dtype)
    do = _draw(rng, (w.B, w.Hq, w.Tq, w.d), w.dtype)
    return q, k, v, do


def decode_seqlens(w: Decode, *, seed: Optional[int] = None) -> np.ndarray:
    rng = np.random.default_rng(w.seed if seed is None else seed)
    return rng.integers(w.seq_lo, w.seq_hi, w.B, endpoint=True).astype(np.int32)


def decode_inputs(w: Decode, *, seed: Optional[int] = None, poison_tail: bool = False):
    """Return (q, kcache, vcache, seqlens); q/caches as uint16 bf16 patterns.

    With ``poison_tail`` every cache slot at or beyond seqlens[b] holds a bf16
    NaN, so any read past the valid prefix shows up in the output.
    """
    rng = np.random.default_rng(w.seed if seed is None else seed)
    seqlens = rng.integers(w.seq_lo, w.seq_hi, w.B, endpoint=True).astype(np.int32)
    q = _draw(rng, (w.B, w.Hq, w.d), "bf16")
    kc = _draw(rng, (w.B, w.Hkv, w.Tk_max, w.d), "bf16")
    vc = _draw(rng, (w.B, w.Hkv, w.Tk_max, w.d), "bf16")
    if poison_tail:
        for b, n in enumerate(seqlens):
            kc[b, :, n:, :] = BF16_NAN
            vc[b, :, n:, :] = BF16_NAN
    return q, kc, vc, seqlens


E4M3_MAX = 448.0   # largest finite E4M3 value


def quantize_rows_e4m3(x: np.ndarray):
    """Per-row block scaling of fp32 rows (last axis) to 8-bit E4M3 codes, as a
    cache writer would store them: scale = max|row| / 448 (1 for an all-zero
    row), codes = round-to-nearest-even of row / scale, done by torch's
    float8_e4m3fn conversion.  Returns (codes uint8, scales float32)."""
    import torch
    x = np.ascontiguousarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    y = (x / scale[..., None]).astype(np.float32)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


def decode_inputs_fp8(w: Decode, *, seed: Optional[int] = None, poison_tail: bool = False):
    """Return (q, kcodes, vcodes, kscale, vscale, seqlens) for an fp8-cache decode.

    seqlens, q, k and v are drawn exactly as ``decode_inputs`` draws them
    (q rounded to bf16); the fp32 k and v rows are then stored as E4M3 codes
    with one fp32 scale per (sequence, kv head, position).  With
    ``poison_tail`` every slot at or beyond seqlens[b] holds the NaN code 0x7F.
    """
    rng = np.random.default_rng(w.seed if seed is None else seed)
    seqlens = rng.integers(w.seq_lo, w.seq_hi, w.B, endpoint=True).astype(np.int32)
    q = _draw(rng, (w.B, w.Hq, w.d), "bf16")
    k = _draw(rng, (w.B, w.Hkv, w.Tk_max, w.d), "f32")
    v = _draw(rng, (w.B, w.Hkv, w.Tk_max, w.d), "f32")
    kc, ks = quantize_rows_e4m3(k)
    del k
    vc, vs = quantize_rows_e4m3(v)
    del v
    if poison_tail:
        for b, n in enumerate(seqlens):
            kc[b, :, n:, :] = 0x7F
            vc[b, :, n:, :] = 0x7F
    return q, kc, vc, ks, vs, seqlens


INT8_MAX = 127   # largest code magnitude the int8 quantiser writes


def quantize_rows_int8(x: np.ndarray):
    """Per-row symmetric scaling of fp32 rows (last axis) to int8 codes, as a
    cache writer would store them: scale = max|row| / 127 (1 for an all-zero
    row), codes = round-half-to-even of row / scale, in [-127, 127], stored as
    their two's-complement bytes.  Returns (codes uint8, scales float32)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    scale = np.where(amax > 0, amax / np.float32(INT8_MAX), np.float32(1.0)).astype(np.float32)
    y = np.rint(x / scale[..., None])
    codes = np.clip(y, -INT8_MAX, INT8_MAX).astype(np.int8)
    return codes.view(np.uint8), scale


def decode_inputs_int8(w: Decode, *, seed: Optional[int] = None, poison_tail: bool = False):
    """Return (q, kcodes, vcodes, kscale, vscale, seqlens) for an int8-cache
    decode, drawn exactly as ``decode_inputs_fp8`` draws them and stored with
    ``quantize_rows_int8``.  With ``poison_tail`` every slot at or beyond
    seqlens[b] holds the code -128 (which the quantiser never writes)."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    seqlens = rng.integers(w.seq_lo, w.seq_hi, w.B, endpoint=True).astype(np.int32)
    q = _draw(rng, (w.B, w.Hq, w.d), "bf16")
    k = _draw(rng, (w.B, w.Hkv, w.Tk_max, w.d), "f32")
    v = _draw(rng, (w.B, w.Hkv, w.Tk_max, w.d), "f32")
    kc, ks = quantize_rows_int8(k)
    del k
    vc, vs = quantize_rows_int8(v)
    del v
    if poison_tail:
        for b, n in enumerate(seqlens):
            kc[b, :, n:, :] = 0x80
            vc[b, :, n:, :] = 0x80
    return q, kc, vc, ks, vs, seqlens


def quantize_blocks_e4m3(x: np.ndarray, nblock_axes: int):
    """Block scaling over the last `nblock_axes` axes: one scale per block,
    scale = max|block| / 448 (1 for an all-zero block), codes = RNE of
    x / scale (torch's float8_e4m3fn conversion).  Returns (codes uint8,
    scales float32 with the leading axes)."""
    import torch
    x = np.ascontiguousarray(x, dtype=np.float32)
    axes = tuple(range(x.ndim - nblock_axes, x.ndim))
    amax = np.max(np.abs(x), axis=axes)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    y = (x / scale.reshape(scale.shape + (1,) * nblock_axes)).astype(np.float32)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


def prefill_inputs_fp8(w: Prefill, *, seed: Optional[int] = None):
    """Return (q8, k8, v8, qscale, kscale, vscale) for the 8-bit forward.

    q, k and v are drawn in fp32 exactly as ``prefill_inputs`` draws them
    before rounding (q times its multiplier); q is stored with one scale per
    row, k and v with one scale per (batch, kv head)."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    q = _draw(rng, (w.B, w.Hq, w.Tq, w.d), "f32", w.q_mult)
    k = _draw(rng, (w.B, w.Hkv, w.Tk, w.d), "f32")
    v = _draw(rng, (w.B, w.Hkv, w.Tk, w.d), "f32")
    q8, qs = quantize_blocks_e4m3(q, 1)
    k8, ks = quantize_blocks_e4m3(k, 2)
    v8, vs = quantize_blocks_e4m3(v, 2)
    return q8, k8, v8, qs, ks, vs
