"""Float64 reference for decode attention (test infrastructure only).

Readings taken where the pages are silent (each is also what the library
implements, written independently there):

* scores are ``scale * <q_h, k_i>`` with ``scale = 1/sqrt(D)`` unless given;
* query head ``h`` reads kv head ``h // (Hq // Hkv)`` (contiguous groups);
* positions ``0 .. seq_lens[b]-1`` are all attended, no mask inside them;
* a history of length 0 gives output 0 and log-sum-exp -inf;
* exposed log-sum-exp values are natural logarithms;
* splits are contiguous token ranges of ``split_length(L, S)`` tokens;
* a quantized (8-bit float E4M3) cache is read as its decoded codes times a
  per-kv-head scale, and attention runs over those dequantized values;
* an 8-bit integer cache is read as its two's-complement codes times one
  scale per (position, kv head), stored in the cache's own row layout
  without the head dimension, and attention again runs over the
  dequantized values.
"""

from __future__ import annotations

import math
from typing import Optional, Tuple

import numpy as np


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns -> float64, exactly.

    A bfloat16 value is the top half of the float32 with the same sign,
    exponent and leading mantissa bits, so shifting the 16 bits into the high
    half of a 32-bit word reproduces that float32 exactly (NaN and inf
    included); widening float32 to float64 is exact.
    """
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):   # NaN payloads widen to NaN
        return u.view(np.float32).astype(np.float64)


def fp8_e4m3_to_f64(codes) -> np.ndarray:
    """8-bit E4M3 floating-point codes (OCP 8-bit float format) -> float64.

    Bit 7 is the sign, bits 6..3 the exponent field e (bias 7), bits 2..0
    the mantissa field m. e = 0: subnormal, (m / 8) * 2^-6. e in 1..15:
    (1 + m / 8) * 2^(e - 7), except e = 15 with m = 7, which is NaN (the
    format has no infinities; its largest finite magnitude is 448).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6,
                   (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))
    mag = np.where((e == 15) & (c & 0x7 == 7), np.nan, mag)
    return sign * mag


def int8_to_f64(codes) -> np.ndarray:
    """8-bit two's-complement codes -> float64: a byte b >= 128 stands for
    b - 256 (so 0x80 is -128 and 0xFF is -1); others for themselves."""
    c = np.asarray(codes)
    if c.dtype == np.int8:
        c = c.view(np.uint8)
    c = c.astype(np.uint8).astype(np.int64)
    return np.where(c >= 128, c - 256, c).astype(np.float64)


def decode_values(arr, dtype: str) -> np.ndarray:
    """Raw input array -> float64 ('bf16': uint16 bit patterns; 'f32';
    'fp8_e4m3': uint8 codes; 'int8': int8 or uint8 bytes)."""
    if dtype == "bf16":
        return bf16_bits_to_f64(arr)
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if dtype == "fp8_e4m3":
        return fp8_e4m3_to_f64(arr)
    if dtype == "int8":
        return int8_to_f64(arr)
    raise ValueError(f"unknown dtype {dtype!r}")


def scale_rows(scale, b: int, kvh: int, lo: int, hi: int, block_table=None,
               block_size: int = 0) -> np.ndarray:
    """Per-position scales for positions lo..hi-1 of sequence b, kv head
    kvh, as a column [n, 1].

    A scale array of one value per kv head ([Hkv]) applies to every
    position. One value per (position, kv head) is laid out like the cache
    without its last axis: [B, Hkv, L'] (any row length L' >= L; entries
    past L are never read), or [NB, Hkv, bs] for a paged pool, where
    position i sits in block block_table[b, i // bs] at slot i % bs.
    """
    sc = np.asarray(scale, dtype=np.float64)
    if sc.ndim == 1:
        return np.full((max(hi - lo, 0), 1), sc[kvh])
    return history_rows(sc[..., None], b, kvh, lo, hi, block_table,
                        block_size)


def history_rows(cache, b: int, kvh: int, lo: int, hi: int,
                 block_table=None, block_size: int = 0) -> np.ndarray:
    """Cache rows for positions lo..hi-1 of sequence b, kv head kvh.

    Contiguous cache: [B, Hkv, L, D], row i is cache[b, kvh, i].
    Paged cache: pool [NB, Hkv, bs, D]; position i lives in block
    block_table[b, i // bs] at slot i % bs (PagedAttention's block table,
    cited by title on the "Faster Than Flash" page's source list).
    """
    if hi <= lo:
        return cache[:0, 0, 0, :]
    if block_table is None or block_size == 0:
        return cache[b, kvh, lo:hi, :]
    pos = np.arange(lo, hi)
    blocks = np.asarray(block_table)[b, pos // block_size]
    return cache[blocks, kvh, pos % block_size, :]


def softmax_attention(scores: np.ndarray, values: np.ndarray
                      ) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention from precomputed scores.

    scores [H, n] (float64), values [n, D] -> (out [H, D], lse [H]).
    out = sum_i e^{s_i} v_i / sum_i e^{s_i}; lse = ln sum_i e^{s_i}, computed
    with the row maximum subtracted before exponentiating. n == 0 gives
    out = 0 and lse = -inf.
    """
    scores = np.asarray(scores, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    H = scores.shape[0]
    D = values.shape[1]
    if scores.shape[1] == 0:
        return np.zeros((H, D)), np.full(H, -np.inf)
    m = scores.max(axis=1, keepdims=True)
    w = np.exp(scores - m)
    z = w.sum(axis=1)
    out = (w @ values) / z[:, None]
    lse = m[:, 0] + np.log(z)
    return out, lse


def decode_attention(q, k, v, seq_lens, *, dtype: str,
                     scale: Optional[float] = None, block_table=None,
                     block_size: int = 0, token_range=None,
                     kv_dtype: Optional[str] = None, k_scale=None,
                     v_scale=None) -> Tuple[np.ndarray, np.ndarray]:
    """Decode attention of one query per (sequence, head) over its history.

    q [B, Hq, D]; k, v contiguous [B, Hkv, L, D] or paged pools
    [NB, Hkv, bs, D] with block_table [B, max_blocks]; seq_lens [B].
    Raw inputs (bf16 as uint16 bits, or float32) are decoded to float64.
    token_range=(lo, hi) restricts every sequence to positions
    lo .. min(hi, seq_lens[b]) - 1 (used for split partials).
    Quantized caches: kv_dtype names the cache's encoding (default: dtype),
    and k_scale / v_scale multiply every decoded key / value: one value per
    kv head ([Hkv]) or one per (position, kv head) (see scale_rows), so
    attention runs over the dequantized cache (the cache precision the
    "What is Flash-Decoding" page asks comparisons to hold fixed, in the
    low-bit form the "Faster Than Flash" abstract scans).
    Returns out [B, Hq, D] and lse [B, Hq] (natural log), float64.
    """
    kvd = kv_dtype or dtype
    qf = decode_values(q, dtype)
    B, Hq, D = qf.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    G = Hq // Hkv
    sc = scale if scale else 1.0 / math.sqrt(D)
    out = np.zeros((B, Hq, D))
    lse = np.full((B, Hq), -np.inf)
    for b in range(B):
        n = int(seq_lens[b])
        lo, hi = (0, n) if token_range is None else (
            token_range[0], min(token_range[1], n))
        if hi <= lo:
            continue
        for kvh in range(Hkv):
            kr = decode_values(history_rows(k, b, kvh, lo, hi, block_table,
                                            block_size), kvd)
            vr = decode_values(history_rows(v, b, kvh, lo, hi, block_table,
                                            block_size), kvd)
            if k_scale is not None:
                kr = kr * scale_rows(k_scale, b, kvh, lo, hi, block_table,
                                     block_size)
            if v_scale is not None:
                vr = vr * scale_rows(v_scale, b, kvh, lo, hi, block_table,
                                     block_size)
            heads = slice(kvh * G, (kvh + 1) * G)
            scores = sc * (qf[b, heads] @ kr.T)
            o, l = softmax_attention(scores, vr)
            out[b, heads] = o
            lse[b, heads] = l
    return out, lse


def split_length(max_seq_len: int, num_splits: int, granule: int = 16) -> int:
    """Tokens per split: ceil(L / S) rounded up to a whole page of
    ``granule`` tokens (16, or the page size of a paged cache when larger).

    The pages say only that the history is cut into parts processed by
    separate blocks; contiguous, equal-length ranges aligned to the page size
    are the plainest reading.
    """
    if num_splits < 1:
        raise ValueError("num_splits must be >= 1")
    per = -(-max(max_seq_len, 1) // num_splits)
    return -(-per // granule) * granule


def split_partials(q, k, v, seq_lens, num_splits: int, *, dtype: str,
                   max_seq_len: int, scale: Optional[float] = None,
                   block_table=None, block_size: int = 0,
                   granule: Optional[int] = None,
                   kv_dtype: Optional[str] = None, k_scale=None,
                   v_scale=None):
    """Per-split partial outputs and log-sum-exps (the method's first step).

    Split s covers positions [s*P, (s+1)*P) clipped to the history, with
    P = split_length(L, S, g), g = max(16, block_size) unless given. Each
    partial is attention over that range alone:
    o_s normalised by its own softmax sum, lse_s = ln of that sum. An empty
    range gives o_s = 0, lse_s = -inf.
    Returns o_part [B, Hq, S, D], lse_part [B, Hq, S].
    """
    P = split_length(max_seq_len, num_splits,
                     granule or max(16, block_size or 0))
    qf = decode_values(q, dtype)
    B, Hq, D = qf.shape
    o_part = np.zeros((B, Hq, num_splits, D))
    lse_part = np.full((B, Hq, num_splits), -np.inf)
    for s in range(num_splits):
        o, l = decode_attention(q, k, v, seq_lens, dtype=dtype, scale=scale,
                                block_table=block_table,
                                block_size=block_size,
                                token_range=(s * P, (s + 1) * P),
                                kv_dtype=kv_dtype, k_scale=k_scale,
                                v_scale=v_scale)
        o_part[:, :, s] = o
        lse_part[:, :, s] = l
    return o_part, lse_part


def combine_partials(o_part, lse_part) -> Tuple[np.ndarray, np.ndarray]:
    """Reduce split partials into the full-history result (second step).

    Each partial o_s is a softmax-weighted mean over its range with total
    weight e^{lse_s}; the full-history mean is therefore the e^{lse_s}-weighted
    mean of the o_s. With M = max_s lse_s for stability:
    out = sum_s e^{lse_s - M} o_s / sum_s e^{lse_s - M},
    lse = M + ln sum_s e^{lse_s - M}. If every lse_s is -inf: out 0, lse -inf.
    o_part [..., S, D], lse_part [..., S].
    """
    o_part = np.asarray(o_part, dtype=np.float64)
    lse_part = np.asarray(lse_part, dtype=np.float64)
    M = lse_part.max(axis=-1, keepdims=True)
    empty = ~np.isfinite(M)
    Msafe = np.where(empty, 0.0, M)
    w = np.where(np.isneginf(lse_part), 0.0, np.exp(lse_part - Msafe))
    z = w.sum(axis=-1)
    zsafe = np.where(z > 0, z, 1.0)
    out = (w[..., None] * o_part).sum(axis=-2) / zsafe[..., None]
    lse = np.where(empty[..., 0], -np.inf, Msafe[..., 0] + np.log(zsafe))
    out = np.where(empty, 0.0, out)
    return out, lse
