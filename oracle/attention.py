"""Plain fp64 CPU reference of exact attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this module (see the package docstring for the page tags cited
below).  It shares no code with the HIP library.

What is computed.  The tiled method reaches exactly this result; it differs
only in the order of floating-point additions ([FUSED07] section
"FlashAttention-наив на numpy", opening paragraph; [LESSON] section "Почему
ответ точный"):

    s_ij  = scale * <q_i, k_j>          over the keys j visible to row i
    O_i   = sum_j softmax_j(s_ij) * v_j
    lse_i = log sum_j exp(s_ij)         ([LESSON] section "Обратный проход":
                                         L_i = m_i + log l_i)

Visibility of key j to query row i:

    non-causal   every j < Tk
    causal       j <= i -- top-left alignment, i.e. the strict upper triangle
                 of the n x m score matrix is masked ([FUSED07],
                 "FlashAttention-наив на numpy", reference attention)
    causal, bottom-right alignment
                 j <= i + (Tk - Tq): query row i sits at absolute position
                 Tk - Tq + i of a sequence whose first Tk - Tq positions
                 are already in the key/value cache (chunked prefill; with
                 Tq = 1 this is the decode rule, where the new token sees
                 every cached key -- [NOTE] section "Prefill i dekodowanie
                 to różne problemy").  With Tq > Tk the first Tq - Tk rows
                 see no key.
    decode       j < seqlens[b]; one query row; scale = 1/sqrt(d)

Grouped-query attention: query head hq reads kv head hq // g, g = Hq / Hkv
([NOTE] section "Prefill i dekodowanie to różne problemy": g query heads share
one KV head).  This is the same as repeating every kv head g times.

A row with no visible key (Tk == 0, seqlen == 0, or the first Tq - Tk rows
under bottom-right alignment) is defined as O = 0, lse = -inf.

Arithmetic is IEEE fp64 throughout; inputs arrive as the exact bf16 bit
patterns (uint16) or fp32 values that the GPU receives and are widened
exactly.
"""
from __future__ import annotations

import math
from typing import Iterable, Sequence, Tuple

import numpy as np

_NEG_INF = -np.inf


# --------------------------------------------------------------------------
# Input widening
# --------------------------------------------------------------------------

def as_f64(x: np.ndarray) -> np.ndarray:
    """Widen stored inputs to fp64 exactly.

    uint16 arrays are bf16 bit patterns: the value is the fp32 whose upper 16
    bits are the pattern and whose lower 16 bits are zero.
    """
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if x.dtype in (np.float32, np.float64):
        return x.astype(np.float64)
    raise TypeError(f"unsupported input dtype {x.dtype}")


_ALIGNS = ("top_left", "bottom_right")


def causal_offset(Tq: int, Tk: int, align: str) -> int:
    """Key j is visible to query row i under the causal mask iff
    j <= i + causal_offset(Tq, Tk, align)."""
    if align not in _ALIGNS:
        raise ValueError(f"unknown causal alignment {align!r}")
    return Tk - Tq if align == "bottom_right" else 0


# --------------------------------------------------------------------------
# Three-pass softmax attention (the definition, written out)
# --------------------------------------------------------------------------

def _rows_three_pass(Qr: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                     visible: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """softmax(scale * Qr K^T) V for a few rows, with a boolean visibility mask.

    Pass 1 takes the row maximum of the visible scores, pass 2 sums
    exp(s - m), pass 3 forms the exp-weighted sum of value rows and divides
    once by that sum ([LESSON] section "Online softmax: нормировка за один
    проход" describes this three-pass stable softmax that the online form
    replaces).
    """
    n = Qr.shape[0]
    dv = V.shape[1]
    O = np.zeros((n, dv))
    lse = np.full(n, _NEG_INF)
    if K.shape[0] == 0:
        return O, lse
    S = (Qr @ K.T) * scale
    S = np.where(visible, S, _NEG_INF)
    m = S.max(axis=1)                                   # pass 1
    has = np.isfinite(m)
    if not has.any():
        return O, lse
    with np.errstate(invalid="ignore"):
        E = np.exp(S[has] - m[has, None])              # pass 2
    l = E.sum(axis=1)
    O[has] = (E @ V) / l[:, None]                       # pass 3
    lse[has] = m[has] + np.log(l)
    return O, lse


def softmax_attention(q, k, v, *, causal: bool, scale: float, row_chunk: int = 256,
                      align: str = "top_left") -> Tuple[np.ndarray, np.ndarray]:
    """Exact attention for q:[B,Hq,Tq,d], k,v:[B,Hkv,Tk,d] -> (O, lse) in fp64.

    Rows are independent, so they are evaluated in chunks of ``row_chunk`` to
    bound memory; under the causal mask a chunk ending at row r only needs
    keys j <= r + off (off from ``causal_offset``), so the keys beyond are
    left out (every one of them would be masked to -inf and contribute
    exp(-inf) = 0).
    """
    q = as_f64(q)
    k = as_f64(k)
    v = as_f64(v)
    B, Hq, Tq, d = q.shape
    Bk, Hkv, Tk, dk = k.shape
    if (Bk, dk) != (B, d) or v.shape[:3] != k.shape[:3] or Hq % max(Hkv, 1):
        raise ValueError("shape mismatch")
    g = Hq // Hkv
    off = causal_offset(Tq, Tk, align)
    O = np.zeros((B, Hq, Tq, v.shape[3]))
    L = np.full((B, Hq, Tq), _NEG_INF)
    for b in range(B):
        for h in range(Hq):
            kh = h // g
            for r0 in range(0, Tq, row_chunk):
                r1 = min(Tq, r0 + row_chunk)
                kend = max(0, min(Tk, r1 + off)) if causal else Tk
                rows = np.arange(r0, r1)[:, None]
                cols = np.arange(kend)[None, :]
                vis = (cols <= rows + off) if causal else np.ones((r1 - r0, kend), bool)
                O[b, h, r0:r1], L[b, h, r0:r1] = _rows_three_pass(
                    q[b, h, r0:r1], k[b, kh, :kend], v[b, kh, :kend], scale, vis)
    return O, L


def softmax_attention_rows(q, k, v, *, causal: bool, scale: float, b: int, h: int,
                           rows: Sequence[int], align: str = "top_left"
                           ) -> Tuple[np.ndarray, np.ndarray]:
    """The same definition evaluated for selected query rows of one (b, h).

    Used where the full output is too large to check against one by one.
    """
    rows = np.asarray(rows, dtype=np.int64)
    Hq = q.shape[1]
    Hkv = k.shape[1]
    kh = h // (Hq // Hkv)
    Qr = as_f64(q[b, h, rows])
    K = as_f64(k[b, kh])
    V = as_f64(v[b, kh])
    off = causal_offset(q.shape[2], K.shape[0], align)
    cols = np.arange(K.shape[0])[None, :]
    vis = (cols <= rows[:, None] + off) if causal else np.ones((len(rows), K.shape[0]), bool)
    return _rows_three_pass(Qr, K, V, scale, vis)


# --------------------------------------------------------------------------
# Backward pass: gradients of O with respect to q, k, v
# --------------------------------------------------------------------------

def attention_backward(q, k, v, do, *, causal: bool, scale: float, align: str = "top_left"):
    """Gradients of the exact attention above, contracted with dO, in fp64.

    The plain chain rule through O = P V, P = softmax(S), S = scale * Q K^T
    (masked entries have P = 0), as restated in [LESSON] section "Обратный
    проход: пересчитать дешевле, чем хранить":

        dV = P^T dO          dP = dO V^T
        dS = P * (dP - rowsum(P * dP))
        dQ = scale * dS K    dK = scale * dS^T Q

    with the row term taken from its definition, rowsum(P * dP), not from
    the identity dO . O that a fast kernel uses.  Under GQA the gradients of
    a kv head add up over its g query heads.  Returns (dq, dk, dv) shaped
    like q, k, v.
    """
    q = as_f64(q)
    k = as_f64(k)
    v = as_f64(v)
    do = as_f64(do)
    B, Hq, Tq, d = q.shape
    _, Hkv, Tk, _ = k.shape
    g = Hq // Hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    rows = np.arange(Tq)[:, None]
    cols = np.arange(Tk)[None, :]
    off = causal_offset(Tq, Tk, align)
    vis = (cols <= rows + off) if causal else np.ones((Tq, Tk), bool)
    for b in range(B):
        for h in range(Hq):
            kh = h // g
            S = scale * (q[b, h] @ k[b, kh].T)
            S = np.where(vis, S, _NEG_INF)
            m = S.max(axis=1, keepdims=True)
            m = np.where(np.isfinite(m), m, 0.0)
            E = np.where(vis, np.exp(S - m), 0.0)
            l = E.sum(axis=1, keepdims=True)
            P = np.divide(E, l, out=np.zeros_like(E), where=l > 0)
            dP = do[b, h] @ v[b, kh].T
            dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
            dv[b, kh] += P.T @ do[b, h]
            dq[b, h] = scale * (dS @ k[b, kh])
            dk[b, kh] += scale * (dS.T @ q[b, h])
    return dq, dk, dv


# --------------------------------------------------------------------------
# The online (tiled) fold -- a second, independent route to the same result
# --------------------------------------------------------------------------

class _RowState:
    """Running statistics of a set of query rows while key blocks are folded
    in one at a time: the largest score seen so far (mx), the sum of
    exp(score - mx) over the keys seen (den) and the exp-weighted sum of
    their value rows (num), all relative to the same mx.

    Absorbing a block is the rescale rule of [FUSED07] section "Online
    softmax: вывод" applied to a block instead of a single score (the
    element form is ``online_weighted_sum``): the new maximum is taken over
    the old one and the block's scores, the old sums are brought to it by
    the factor exp(old - new) and the block's own terms are added.
    """

    def __init__(self, rows: int, width: int):
        self.mx = np.full(rows, _NEG_INF)
        self.den = np.zeros(rows)
        self.num = np.zeros((rows, width))

    def absorb(self, scores: np.ndarray, values: np.ndarray) -> None:
        """Fold one key block in: scores [rows, keys] (hidden keys at -inf),
        values [keys, width]."""
        grown = np.fmax(self.mx, scores.max(axis=1, initial=_NEG_INF))
        # Rows that still have no visible key keep every sum at zero; any
        # finite anchor works for them, 0 avoids (-inf) - (-inf).
        anchor = np.where(np.isinf(grown), 0.0, grown)
        keep = np.exp(self.mx - anchor)            # exp(old max - new max)
        w = np.exp(scores - anchor[:, None])       # exp(score - new max)
        self.den = keep * self.den + w.sum(axis=1)
        self.num = keep[:, None] * self.num + w @ values
        self.mx = grown

    def result(self) -> Tuple[np.ndarray, np.ndarray]:
        """(num / den, mx + log den); rows that saw no key give (0, -inf)."""
        seen = self.den > 0
        out = np.zeros_like(self.num)
        lse = np.full(self.mx.shape, _NEG_INF)
        out[seen] = self.num[seen] / self.den[seen, None]
        lse[seen] = self.mx[seen] + np.log(self.den[seen])
        return out, lse


def _key_blocks_needed(first_row: int, last_row: int, Tk: int, Bc: int, causal: bool,
                       off: int) -> int:
    """Key blocks of width Bc a query block must visit: all of them, or under
    the causal mask only those that begin at or before the last row's
    furthest visible key ([FUSED07] section "FlashAttention-2", change 3:
    later blocks lie wholly above the diagonal)."""
    reach = Tk if not causal else max(0, min(Tk, last_row + off + 1))
    return -(-reach // Bc)


def online_fold_attention(q, k, v, *, causal: bool, scale: float, Br: int = 64,
                          Bc: int = 64, count: bool = False, align: str = "top_left"):
    """Exact attention reached the tiled way, in fp64 (a second route to the
    definition that ``softmax_attention`` writes out).

    The query rows of every (batch, head) are cut into blocks of Br; each
    block keeps a ``_RowState`` and folds the key/value sequence into it in
    blocks of Bc, in order, with the block's masked scores at -inf before
    any maximum is taken.  One division per row at the end gives O and
    lse = max + log(sum) ([LESSON] sections "Прямой проход FlashAttention"
    and "Обратный проход": L = m + log l).  Key blocks that lie wholly
    above the causal diagonal are never visited.  Returns (O, lse) or,
    with ``count``, (O, lse, number of (query block, key block) pairs
    visited).
    """
    qs, ks, vs = as_f64(q), as_f64(k), as_f64(v)
    B, Hq, Tq, _ = qs.shape
    Hkv, Tk, width = ks.shape[1], ks.shape[2], vs.shape[3]
    group = Hq // Hkv
    off = causal_offset(Tq, Tk, align)
    out = np.zeros((B, Hq, Tq, width))
    lse = np.full((B, Hq, Tq), _NEG_INF)
    visited = 0
    key_pos = np.arange(Tk)
    for b, h in ((b, h) for b in range(B) for h in range(Hq)):
        keys, vals = ks[b, h // group], vs[b, h // group]
        for r0 in range(0, Tq, Br):
            r1 = min(Tq, r0 + Br)
            row_pos = np.arange(r0, r1)
            state = _RowState(r1 - r0, width)
            nkb = _key_blocks_needed(r0, r1 - 1, Tk, Bc, causal, off)
            for kb in range(nkb):
                cols = key_pos[kb * Bc:(kb + 1) * Bc]
                sc = scale * (qs[b, h, r0:r1] @ keys[cols].T)
                if causal:
                    hidden = cols[None, :] - row_pos[:, None] > off
                    sc[hidden] = _NEG_INF
                state.absorb(sc, vals[cols])
            visited += nkb
            out[b, h, r0:r1], lse[b, h, r0:r1] = state.result()
    if count:
        return out, lse, visited
    return out, lse


def causal_block_pairs(Tq: int, Tk: int, Br: int, Bc: int, causal: bool) -> int:
    """Number of (query block, key block) pairs the tiled loop visits.

    All ceil(Tq/Br) * ceil(Tk/Bc) pairs without a mask; with the causal mask
    only the pairs whose key block starts at or before the query block's last
    row ([LESSON] practice template, ``count_blocks`` docstring).
    """
    n = 0
    for i0 in range(0, Tq, Br):
        i_last = min(Tq, i0 + Br) - 1
        for j0 in range(0, Tk, Bc):
            if causal and j0 > i_last:
                break
            n += 1
    return n


# --------------------------------------------------------------------------
# Decode: one query per sequence over a KV cache
# --------------------------------------------------------------------------

def decode_attention(q, kcache, vcache, seqlens) -> Tuple[np.ndarray, np.ndarray]:
    """Single-query attention over each sequence's valid cache prefix.

    q:[B,Hq,d]; kcache,vcache:[B,Hkv,Tk_max,d]; seqlens:[B].  Key j of
    sequence b is visible iff j < seqlens[b]; scale = 1/sqrt(d); no other mask.
    Cache slots at or beyond seqlens[b] are never read.  Returns (O[B,Hq,d],
    lse[B,Hq]) in fp64.
    """
    B, Hq, d = q.shape
    Hkv = kcache.shape[1]
    g = Hq // Hkv
    scale = 1.0 / math.sqrt(d)
    O = np.zeros((B, Hq, vcache.shape[3]))
    L = np.full((B, Hq), _NEG_INF)
    for b in range(B):
        n = int(seqlens[b])
        for h in range(Hq):
            K = as_f64(kcache[b, h // g, :n])
            V = as_f64(vcache[b, h // g, :n])
            Qr = as_f64(q[b, h])[None, :]
            o, lse = _rows_three_pass(Qr, K, V, scale, np.ones((1, n), bool))
            O[b, h], L[b, h] = o[0], lse[0]
    return O, L


def e4m3_to_f64(codes) -> np.ndarray:
    """Values of 8-bit floating-point codes in the E4M3 format with no
    infinities (1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
    exponent field 0 encodes subnormals m/8 * 2^-6; the all-ones exponent and
    mantissa, 0x7F and 0xFF, is NaN; largest finite value 448)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    out = sign * mag
    return np.where((e == 15) & (m == 7), np.nan, out)


def fp8_attention_inputs(q8, k8, v8, qscale, kscale, vscale):
    """Dequantise block-scaled E4M3 attention inputs to fp64.

    q8:[B,Hq,Tq,d] with one scale per query row qscale:[B,Hq,Tq];
    k8, v8:[B,Hkv,Tk,d] with one scale per (batch, kv head) kscale,
    vscale:[B,Hkv] -- the FP8 forward path with block scaling ([LESSON]
    section "FlashAttention-2, -3 и дальше"; a row's scale is fixed by the
    whole row, [BOOK5] section 5.4.3, Example 5-7).  Returns (q, k, v) in
    fp64; the attention of the 8-bit inputs is exactly the attention of
    these.
    """
    q = e4m3_to_f64(q8) * np.asarray(qscale, np.float64)[..., None]
    k = e4m3_to_f64(k8) * np.asarray(kscale, np.float64)[..., None, None]
    v = e4m3_to_f64(v8) * np.asarray(vscale, np.float64)[..., None, None]
    return q, k, v


def decode_attention_fp8(q, kcodes, vcodes, kscale, vscale, seqlens) -> Tuple[np.ndarray, np.ndarray]:
    """Decode over an 8-bit cache: dequantize, then the decode definition.

    The cache holds E4M3 codes kcodes, vcodes:[B,Hkv,Tk_max,d] and one fp32
    scale per cached row kscale, vscale:[B,Hkv,Tk_max]; row j of kv head h
    stands for K[b,h,j,:] = kscale[b,h,j] * e4m3(kcodes[b,h,j,:]) (and V
    alike) -- a per-row block scale, the plain form of a block-scaled low-bit
    cache ([NOTE] section on fused dequantisation: the cache is stored
    compressed and expanded inside the attention kernel's tile load).  The
    attention over the expanded rows is exactly ``decode_attention``; rows at
    or past seqlens[b] are never read.
    """
    B, Hq, d = q.shape
    Hkv = kcodes.shape[1]
    g = Hq // Hkv
    scale = 1.0 / math.sqrt(d)
    O = np.zeros((B, Hq, vcodes.shape[3]))
    L = np.full((B, Hq), _NEG_INF)
    for b in range(B):
        n = int(seqlens[b])
        for kh in range(Hkv):
            K = e4m3_to_f64(kcodes[b, kh, :n]) * np.asarray(kscale[b, kh, :n], np.float64)[:, None]
            V = e4m3_to_f64(vcodes[b, kh, :n]) * np.asarray(vscale[b, kh, :n], np.float64)[:, None]
            for h in range(kh * g, (kh + 1) * g):
                Qr = as_f64(q[b, h])[None, :]
                o, lse = _rows_three_pass(Qr, K, V, scale, np.ones((1, n), bool))
                O[b, h], L[b, h] = o[0], lse[0]
    return O, L


def int8_to_f64(codes) -> np.ndarray:
    """Values of 8-bit two's-complement integer codes: code c stands for c
    when its top bit is clear and for c - 256 when it is set (-128 .. 127)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    return np.where(c >= 128, c - 256, c).astype(np.float64)


def decode_attention_int8(q, kcodes, vcodes, kscale, vscale, seqlens) -> Tuple[np.ndarray, np.ndarray]:
    """Decode over an int8 cache: dequantize, then the decode definition.

    Same layout and meaning as ``decode_attention_fp8`` with two's-complement
    integer codes: K[b,h,j,:] = kscale[b,h,j] * int8(kcodes[b,h,j,:]) (V
    alike), the other common low-bit cache format with a per-row block scale
    ([NOTE] section on fused dequantisation).  Rows at or past seqlens[b] are
    never read.
    """
    B, Hq, d = q.shape
    Hkv = kcodes.shape[1]
    g = Hq // Hkv
    scale = 1.0 / math.sqrt(d)
    O = np.zeros((B, Hq, vcodes.shape[3]))
    L = np.full((B, Hq), _NEG_INF)
    for b in range(B):
        n = int(seqlens[b])
        for kh in range(Hkv):
            K = int8_to_f64(kcodes[b, kh, :n]) * np.asarray(kscale[b, kh, :n], np.float64)[:, None]
            V = int8_to_f64(vcodes[b, kh, :n]) * np.asarray(vscale[b, kh, :n], np.float64)[:, None]
            for h in range(kh * g, (kh + 1) * g):
                Qr = as_f64(q[b, h])[None, :]
                o, lse = _rows_three_pass(Qr, K, V, scale, np.ones((1, n), bool))
                O[b, h], L[b, h] = o[0], lse[0]
    return O, L


def decode_split_merge(q, kcache, vcache, seqlens, num_splits: int,
                       tile: int = 64) -> Tuple[np.ndarray, np.ndarray]:
    """Flash-decoding in fp64: split each sequence's keys, merge the partials.

    [NOTE] section "Prefill i dekodowanie to różne problemy" (Flash-decoding):
    with one query there are no rows to spread over blocks, so the key
    sequence is cut into pieces; each piece yields a partial (m, l, o) and a
    last step merges them with the same rescaling rule.  Sequence b is cut
    into chunks of c = tile * ceil(ceil(seqlens[b] / num_splits) / tile) keys;
    chunks that start at or past seqlens[b] are empty (m = -inf, l = 0).

    Merge ([BOOK5] section 5.3.3, Example 5-6 and the update equations after
    it): M = max_s m_s, l = sum_s exp(m_s - M) l_s,
    o = sum_s exp(m_s - M) o_s, O = o / l; empty pieces drop out because
    their weight is exp(-inf) = 0 and their sums are 0.
    """
    B, Hq, d = q.shape
    Hkv = kcache.shape[1]
    g = Hq // Hkv
    scale = 1.0 / math.sqrt(d)
    O = np.zeros((B, Hq, vcache.shape[3]))
    L = np.full((B, Hq), _NEG_INF)
    for b in range(B):
        n = int(seqlens[b])
        per = -(-n // num_splits)
        c = tile * (-(-per // tile)) if n > 0 else tile
        for h in range(Hq):
            Qv = as_f64(q[b, h])
            parts = []
            for s in range(num_splits):
                lo, hi = s * c, min(n, (s + 1) * c)
                if lo >= hi:
                    parts.append((_NEG_INF, 0.0, np.zeros(vcache.shape[3])))
                    continue
                K = as_f64(kcache[b, h // g, lo:hi])
                V = as_f64(vcache[b, h // g, lo:hi])
                sc = (K @ Qv) * scale
                m_s = sc.max()
                e = np.exp(sc - m_s)
                parts.append((m_s, e.sum(), e @ V))
            ms = np.array([p[0] for p in parts])
            if not np.isfinite(ms).any():
                continue
            M = ms.max()
            w = np.exp(ms - M)
            l = sum(w[s] * parts[s][1] for s in range(num_splits))
            o = sum(w[s] * parts[s][2] for s in range(num_splits))
            O[b, h] = o / l
            L[b, h] = M + math.log(l)
    return O, L


# --------------------------------------------------------------------------
# Scalar online normaliser (element by element)
# --------------------------------------------------------------------------

def online_normalizer(xs: Iterable[float]) -> Tuple[float, float]:
    """One pass over xs giving m = max x and l = sum exp(x - m).

    [LESSON] section "Online softmax: нормировка за один проход":
    m' = max(m, x), l' = l * exp(m - m') + exp(x - m'), from m = -inf, l = 0.
    """
    m, l = -math.inf, 0.0
    for x in xs:
        m_new = max(m, x)
        l = l * math.exp(m - m_new) + math.exp(x - m_new)
        m = m_new
    return m, l


def online_weighted_sum(xs: Sequence[float], vs: Sequence) -> Tuple[float, float, np.ndarray, np.ndarray]:
    """One pass giving (m, l, a, o) with a = sum exp(x - m) v and o = a / l.

    Same section as ``online_normaliser``: a' = a * exp(m - m') + exp(x - m') v,
    divided by l once at the end.
    """
    m, l = -math.inf, 0.0
    a = np.zeros_like(np.asarray(vs[0], dtype=np.float64))
    for x, v in zip(xs, vs):
        m_new = max(m, x)
        r = math.exp(m - m_new)
        p = math.exp(x - m_new)
        l = l * r + p
        a = a * r + p * np.asarray(v, dtype=np.float64)
        m = m_new
    return m, l, a, a / l
