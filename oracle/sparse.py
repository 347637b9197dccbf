"""Float64 reference for block-sparse decode over a low-bit key summary
(test infrastructure only; "parity" for the selection step is pinned by
invariants and brute force, not by values the pages print).

The "Faster Than Flash" page (abstract) describes decoding that first scans
a low-bit quantized copy of the keys to estimate which blocks of the history
matter, keeps the blocks a "top-delta" rule admits (without global
synchronization), and computes exact attention over the kept blocks only.
The page defines neither the quantizer nor the rule; the readings taken here
(each implemented independently in the library) are:

* key summary: the history is cut into 16-token blocks (one page of a paged
  cache). For each block and kv head, amax = the largest |k| over the
  block's attended rows and all dims (exact in float32: the keys are bf16);
  inv = float32(7 / amax) and scale = float32(amax / 7) (both rounded once to
  float32; amax = 0 gives inv = scale = 0); every attended element gets the
  4-bit code rint(float32(k * inv)) (round half to even), which lies in
  [-7, 7]. Rows past the length get code 0.
* query for the scan: per (sequence, query head), amax_q = max |q| (float32),
  inv_q = float32(127 / amax_q), s_q = float32(amax_q / 127), and the 8-bit
  query q8 = rint(float32(q * inv_q)) in [-127, 127] (amax_q = 0: all 0).
* estimate: dot[i, h] = sum_d q8[h, d] * code[i, d], an exact integer; for
  block j, dmax = the largest dot over the block's attended tokens, and, in
  float32 with the multiplications in this order,
  est[j, h] = ((float(dmax) * s_q) * scale_j) * scale_log2, with
  scale_log2 = float32(scale * log2 e) -- the block's largest logit, in
  base-2 units, as the summary sees it.
* splits: contiguous ranges of P = ceil(ceil(L / S) / g) * g tokens,
  g = max(16, page size) -- the dense path's boundaries;
* top-delta, per split (no cross-split synchronization): with M[h] the
  largest est over the split's blocks and delta2 = float32(delta * log2 e),
  block j is kept when est[j, h] >= float32(M[h] - delta2) for at least one
  query head h of its kv head (float32 comparison, so both implementations
  take every decision identically).
* result: exact softmax attention (as ``decode_attention``) over the tokens
  of every kept block; delta = +inf keeps every block and gives the dense
  result.
* an 8-bit cache -- E4M3 codes with one float32 scale per kv head for K
  and one for V, or int8 codes with one float32 scale per (position, kv
  head) for each -- : the summary quantizes the keys as
  float32(decode(code) * k_scale) -- the exact product rounded once to
  float32, the precision in which both implementations take every
  decision -- and the rest is unchanged; the exact attention runs over the
  dequantized cache, decode(code) times its scale in float64 (as
  ``decode_attention``).
"""

from __future__ import annotations

import math
from typing import Optional, Tuple

import numpy as np

from .attention import decode_values, history_rows, scale_rows, \
    softmax_attention, split_length

BLOCK = 16


def quantize_block(rows_bf16_bits) -> Tuple[np.ndarray, np.float32]:
    """One block's attended key rows (bf16 bit patterns, [n, D]) ->
    (int codes [n, D], float32 scale), per the reading above."""
    return quantize_block_values(
        decode_values(rows_bf16_bits, "bf16").astype(np.float32))


def summary_keys(rows, kv_dtype: str = "bf16", k_scale=None) -> np.ndarray:
    """Key rows as the summary sees them, float32: bf16 exactly; an 8-bit
    cache as float32(decode(code) * scale) (one rounding of the exact
    product). k_scale: the kv head's scale (E4M3) or a column of the rows'
    scales [n, 1] (int8)."""
    if kv_dtype == "bf16":
        return decode_values(rows, "bf16").astype(np.float32)
    if kv_dtype in ("fp8_e4m3", "int8"):
        x = decode_values(rows, kv_dtype).astype(np.float32)
        return (x * np.asarray(k_scale, dtype=np.float32)).astype(np.float32)
    raise ValueError(f"no key summary for {kv_dtype!r} caches")


def quantize_block_values(x) -> Tuple[np.ndarray, np.float32]:
    """One block's attended key rows as float32 values [n, D] -> (int
    codes [n, D], float32 scale), per the reading above."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.abs(x).max()) if x.size else np.float32(0)
    if amax == 0:
        return np.zeros(x.shape, dtype=np.int64), np.float32(0)
    inv = np.float32(np.float32(7) / amax)
    scale = np.float32(amax / np.float32(7))
    codes = np.rint((x * inv).astype(np.float32)).astype(np.int64)
    return codes, scale


def quantize_query(q_bf16_bits) -> Tuple[np.ndarray, np.float32]:
    """One query head's bf16 bits [D] -> (int8-range codes [D], float32
    scale), per the reading above."""
    x = decode_values(q_bf16_bits, "bf16").astype(np.float32)
    amax = np.float32(np.abs(x).max()) if x.size else np.float32(0)
    if amax == 0:
        return np.zeros(x.shape, dtype=np.int64), np.float32(0)
    inv = np.float32(np.float32(127) / amax)
    s = np.float32(amax / np.float32(127))
    return np.rint((x * inv).astype(np.float32)).astype(np.int64), s


def log2_units(x: float) -> np.float32:
    """float32(x * log2 e) with the product taken in double precision (how
    the library converts the logit scale and delta)."""
    return np.float32(float(np.float32(x)) * 1.4426950408889634)


def key_summary(k, seq_lens, block_table=None, block_size: int = 0,
                kv_dtype: str = "bf16", k_scale=None):
    """Codes (int, same layout as k) and scales for every attended block.

    Contiguous k [B, Hkv, L, D]: scales [B, Hkv, ceil(L/16)].
    Paged pool [NB, Hkv, bs, D]: scales [NB, Hkv, bs/16] (sub-block s of a
    page covers its slots 16s..16s+15). Unattended rows/blocks stay 0.
    k holds bf16 bit patterns, E4M3 codes (kv_dtype "fp8_e4m3") with
    k_scale [Hkv], or int8 codes (kv_dtype "int8") with per-position
    k_scale laid out as ``scale_rows`` reads it.
    """
    paged = block_table is not None and block_size
    codes = np.zeros(k.shape, dtype=np.int64)
    if paged:
        scales = np.zeros((k.shape[0], k.shape[1], block_size // BLOCK),
                          dtype=np.float32)
    else:
        scales = np.zeros((k.shape[0], k.shape[1], -(-k.shape[2] // BLOCK)),
                          dtype=np.float32)
    B = len(seq_lens)
    for b in range(B):
        n = int(seq_lens[b])
        for kvh in range(k.shape[1]):
            for j in range(-(-n // BLOCK)):
                lo, hi = j * BLOCK, min((j + 1) * BLOCK, n)
                rows = history_rows(k, b, kvh, lo, hi, block_table,
                                    block_size)
                if k_scale is None:
                    ks = None
                elif np.ndim(k_scale) == 1:
                    ks = np.asarray(k_scale)[kvh]
                else:
                    ks = scale_rows(k_scale, b, kvh, lo, hi, block_table,
                                    block_size)
                c, s = quantize_block_values(summary_keys(rows, kv_dtype, ks))
                if paged:
                    pos = np.arange(lo, hi)
                    blk = np.asarray(block_table)[b, pos // block_size]
                    codes[blk, kvh, pos % block_size] = c
                    scales[blk[0], kvh, (lo % block_size) // BLOCK] = s
                else:
                    codes[b, kvh, lo:hi] = c
                    scales[b, kvh, j] = s
    return codes, scales


def pack_int4(codes) -> np.ndarray:
    """Int codes in [-8, 7], last axis D -> uint8 [..., D/2]: dim 2m in the
    low nibble of byte m, dim 2m+1 in the high nibble (two's complement)."""
    c = np.asarray(codes, dtype=np.int64) & 0xF
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def records_to_rows(records, head_dim: int) -> np.ndarray:
    """Summary records (uint8 [..., 8 * D]) -> packed rows [..., 16, D / 2]:
    row n's piece p (D / 8 bytes) is stored at byte D / 8 * (n + 16 p)."""
    r = np.asarray(records, dtype=np.uint8)
    cb = head_dim // 8
    x = r.reshape(r.shape[:-1] + (4, 16, cb))          # [.., piece, row, byte]
    return np.swapaxes(x, -3, -2).reshape(r.shape[:-1] + (16, 4 * cb))


def unpack_int4(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.int64)
    lo, hi = p & 0xF, (p >> 4) & 0xF
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.int64)
    out[..., 0::2], out[..., 1::2] = lo, hi
    return np.where(out >= 8, out - 16, out)


def block_scale(scales, b, kvh, j, block_table=None, block_size: int = 0):
    if block_table is None or not block_size:
        return float(scales[b, kvh, j])
    pos = j * BLOCK
    blk = int(np.asarray(block_table)[b, pos // block_size])
    return float(scales[blk, kvh, (pos % block_size) // BLOCK])


def sparse_decode_attention(q, k, v, seq_lens, codes, scales, *, delta: float,
                            num_splits: int, max_seq_len: int,
                            scale: Optional[float] = None, block_table=None,
                            block_size: int = 0, kv_dtype: str = "bf16",
                            k_scale=None, v_scale=None):
    """Block-sparse decode (readings in the module docstring).

    q [B, Hq, D] bf16 bits; k, v bf16 bits, E4M3 codes (kv_dtype
    "fp8_e4m3", with k_scale / v_scale [Hkv]) or int8 codes (kv_dtype
    "int8", per-position scales), contiguous or paged; codes int (layout of
    k), scales as ``key_summary`` returns.
    Returns out [B, Hq, D], lse [B, Hq], est [B, Hq, nblk] (float32 values
    in base-2 units; NaN where no block), kept [B, Hkv, nblk] (bool), with
    nblk = ceil(L / 16).
    """
    qf = decode_values(q, "bf16")
    B, Hq, D = qf.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    sc = scale if scale else 1.0 / math.sqrt(D)
    sl2 = log2_units(sc)
    d2 = log2_units(delta) if math.isfinite(delta) else np.float32(np.inf)
    # Split boundaries as for the dense path: whole pages of max(16, bs).
    P = split_length(max_seq_len, num_splits, max(16, block_size or 0))
    nblk = -(-max(max_seq_len, 1) // BLOCK)
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), -np.inf)
    est = np.full((B, Hq, nblk), np.nan)
    kept = np.zeros((B, Hkv, nblk), dtype=bool)
    for b in range(B):
        n = int(seq_lens[b])
        for kvh in range(Hkv):
            heads = slice(kvh * G, (kvh + 1) * G)
            # 1. estimates from the summary
            qq = [quantize_query(q[b, h]) for h in range(kvh * G, (kvh + 1) * G)]
            q8 = np.stack([x[0] for x in qq])              # [G, D] ints
            sq = [x[1] for x in qq]
            for j in range(-(-n // BLOCK)):
                lo, hi = j * BLOCK, min((j + 1) * BLOCK, n)
                c = history_rows(codes, b, kvh, lo, hi, block_table,
                                 block_size).astype(np.int64)
                s = np.float32(block_scale(scales, b, kvh, j, block_table,
                                           block_size))
                dmax = (q8 @ c.T).max(axis=1)              # exact integers
                for g in range(G):
                    e = np.float32(np.float32(dmax[g]) * sq[g])
                    e = np.float32(e * s)
                    est[b, kvh * G + g, j] = np.float32(e * sl2)
            # 2./3. top-delta inside each split
            for s_ in range(num_splits):
                j0, j1 = s_ * P // BLOCK, min((s_ + 1) * P, n)
                j1 = -(-j1 // BLOCK)
                if j1 <= j0:
                    continue
                e = est[b, heads, j0:j1].astype(np.float32)
                M = e.max(axis=1, keepdims=True)
                thr = (M - d2).astype(np.float32)
                kept[b, kvh, j0:j1] = (e >= thr).any(axis=0)
            # 4. exact attention over the kept tokens
            toks = [t for t in range(n) if kept[b, kvh, t // BLOCK]]
            if not toks:
                continue
            kr = np.concatenate([decode_values(history_rows(
                k, b, kvh, t, t + 1, block_table, block_size), kv_dtype)
                for t in toks])
            vr = np.concatenate([decode_values(history_rows(
                v, b, kvh, t, t + 1, block_table, block_size), kv_dtype)
                for t in toks])
            if k_scale is not None:
                kr = kr * np.concatenate([scale_rows(
                    k_scale, b, kvh, t, t + 1, block_table, block_size)
                    for t in toks])
            if v_scale is not None:
                vr = vr * np.concatenate([scale_rows(
                    v_scale, b, kvh, t, t + 1, block_table, block_size)
                    for t in toks])
            o, l = softmax_attention(sc * (qf[b, heads] @ kr.T), vr)
            out[b, heads] = o
            lse[b, heads] = l
    return out, lse, est, kept
