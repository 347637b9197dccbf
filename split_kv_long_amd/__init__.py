"""Split-KV (Flash-Decoding) decode attention for MI355X (gfx950).

The compute lives in ``lib/libfd_decode.so`` (hand-written HIP kernels behind
the C ABI in ``include/fd_decode.h``); ``binding`` exposes the same calls to
Python, and ``decode_attention`` below is a convenience wrapper that checks
the tensors, sizes and allocates the outputs with torch before calling
``fd_decode_attn``; ``build_key_summary`` and ``sparse_decode_attention``
do the same for the block-sparse calls.
"""

from __future__ import annotations

from typing import Optional

__all__ = ["decode_attention", "shape_for", "validate_inputs",
           "build_key_summary", "sparse_decode_attention", "sparse_splits"]


def shape_for(q, k_cache, seq_lens, block_table=None, max_seq_len=None,
              scale=None):
    """fd_shape for torch tensors laid out as the C ABI describes.

    For a contiguous cache [B, Hkv, L, D] the length dimension L is also the
    row stride the kernels use, so ``max_seq_len`` may only repeat it; for a
    paged pool it bounds the lengths (default: every block-table entry)."""
    import torch
    from . import binding
    B, Hq, D = q.shape
    if block_table is None:
        _, Hkv, L, _ = k_cache.shape
        if max_seq_len is not None and int(max_seq_len) != L:
            raise ValueError(
                f"max_seq_len={max_seq_len} for a contiguous cache of length "
                f"{L}: the cache's length dimension is its row stride, so "
                "the bound must equal it (slice the cache instead)")
        bs = maxb = nb = 0
    else:
        nb, Hkv, bs, _ = k_cache.shape
        maxb = block_table.shape[1]
        L = int(max_seq_len) if max_seq_len is not None else maxb * bs
    if k_cache.dtype in (torch.float8_e4m3fn, torch.int8):
        if q.dtype != torch.bfloat16:
            raise ValueError("an 8-bit cache takes a bf16 query")
        dt = "fp8_e4m3" if k_cache.dtype == torch.float8_e4m3fn else "int8"
    else:
        if k_cache.dtype != q.dtype or q.dtype not in (torch.bfloat16,
                                                       torch.float32):
            raise ValueError("q and the cache must both be bf16 or fp32 "
                             f"(got {q.dtype} and {k_cache.dtype})")
        dt = {torch.bfloat16: "bf16", torch.float32: "f32"}[q.dtype]
    return binding.make_shape(B, Hq, Hkv, D, L, dt, bs, maxb, nb, scale or 0.0)


def validate_inputs(q, k_cache, v_cache, seq_lens, block_table=None,
                    k_scale=None, v_scale=None, max_seq_len=None,
                    device=None):
    """Raise ValueError unless the tensors have the dtypes, shapes, layout
    and device the C ABI reads them with (the library trusts its pointers:
    a wrong dtype or stride would give wrong results, not an error)."""
    import torch
    dev = q.device if device is None else torch.device(device)

    def need(cond, msg):
        if not cond:
            raise ValueError(msg)

    def on_dev(name, t):
        need(t.device == dev,
             f"{name} is on device {t.device}, expected {dev}")
        need(t.is_contiguous(), f"{name} must be contiguous")

    need(q.dim() == 3, "q must be [batch, num_q_heads, head_dim]")
    need(k_cache.dim() == 4 and v_cache.shape == k_cache.shape
         and v_cache.dtype == k_cache.dtype,
         "k_cache and v_cache must match in dtype and 4-D shape")
    B, Hq, D = q.shape
    need(k_cache.shape[-1] == D, "the caches' head_dim differs from q's")
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache),
                    ("seq_lens", seq_lens)):
        on_dev(name, t)
    need(seq_lens.dtype == torch.int32 and tuple(seq_lens.shape) == (B,),
         f"seq_lens must be int32 [{B}] (got {seq_lens.dtype} "
         f"{tuple(seq_lens.shape)})")
    if block_table is not None:
        on_dev("block_table", block_table)
        need(block_table.dtype == torch.int32 and block_table.dim() == 2
             and block_table.shape[0] == B,
             f"block_table must be int32 [{B}, max_blocks_per_seq]")
    shape = shape_for(q, k_cache, seq_lens, block_table, max_seq_len)
    Hkv = shape.num_kv_heads
    if k_cache.dtype == torch.float8_e4m3fn:
        want = (Hkv,)
    elif k_cache.dtype == torch.int8:
        if block_table is None:
            want = (B, Hkv, -(-shape.max_seq_len // 16) * 16)
        else:
            want = (shape.num_blocks, Hkv, shape.block_size)
    else:
        need(k_scale is None and v_scale is None,
             "scales are only taken with an 8-bit cache")
        return shape
    for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
        need(t is not None, f"an 8-bit cache needs {name}")
        on_dev(name, t)
        need(t.dtype == torch.float32 and tuple(t.shape) == want,
             f"{name} must be fp32 {want} (got {t.dtype} {tuple(t.shape)})")
    return shape


def decode_attention(q, k_cache, v_cache, seq_lens, block_table=None,
                     num_splits: Optional[int] = None, scale=None,
                     max_seq_len=None, return_lse: bool = False,
                     k_scale=None, v_scale=None):
    """out[b, h] = softmax attention of q[b, h] over the first seq_lens[b]
    cached positions (fp32). Tensors must be contiguous on the current GPU;
    seq_lens and block_table are int32. An E4M3 cache
    (torch.float8_e4m3fn) needs k_scale / v_scale fp32 [Hkv]; an int8
    cache needs them per (position, kv head): contiguous [B, Hkv, Lp] with
    Lp = ceil(L / 16) * 16 (rows padded to whole 16-position groups), paged
    [num_blocks, Hkv, block_size]."""
    import torch
    from . import binding
    shape = validate_inputs(q, k_cache, v_cache, seq_lens, block_table,
                            k_scale, v_scale, max_seq_len)
    if scale:
        shape.scale = float(scale)
    if num_splits is None:
        cus = torch.cuda.get_device_properties(q.device).multi_processor_count
        num_splits = binding.fd_plan_splits(shape, cus, -1)
    out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    nbytes = binding.fd_workspace_size(shape, num_splits)
    ws = (torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
          if nbytes else None)
    if k_cache.dtype in (torch.float8_e4m3fn, torch.int8):
        call = (binding.fd_decode_attn_fp8
                if k_cache.dtype == torch.float8_e4m3fn
                else binding.fd_decode_attn_int8)
        call(shape, q, k_cache, v_cache, k_scale, v_scale, block_table,
             seq_lens, num_splits, ws, out, lse)
    else:
        binding.fd_decode_attn(shape, q, k_cache, v_cache, block_table,
                               seq_lens, num_splits, ws, out, lse)
    return (out, lse) if return_lse else out


# Block-sparse calls: tokens per split at most 8192, and tokens per split x
# max(16, query heads per kv head) at most 131072 (the block estimates of a
# split live in on-chip memory).
_SPARSE_MAX_SPLIT = 8192
_SPARSE_MAX_EST = 8192 * 16


def sparse_splits(shape, num_splits: int) -> int:
    """The smallest split count >= num_splits whose splits the block-sparse
    calls accept (doubling; at most 65535)."""
    g = max(16, shape.block_size)
    G = shape.num_q_heads // shape.num_kv_heads
    cap = min(_SPARSE_MAX_SPLIT, _SPARSE_MAX_EST // max(16, G))
    L = max(int(shape.max_seq_len), 1)
    S = max(1, int(num_splits))
    while True:
        P = -(-(-(-L // S)) // g) * g
        if P <= cap or S >= 65535:
            return S
        S = min(65535, 2 * S)


def _sparse_call(name, k_cache):
    import torch
    from . import binding
    suffix = {torch.bfloat16: "", torch.float8_e4m3fn: "_fp8",
              torch.int8: "_int8"}.get(k_cache.dtype)
    if suffix is None:
        raise ValueError("the block-sparse path takes bf16, E4M3 or int8 "
                         f"caches (got {k_cache.dtype})")
    return getattr(binding, name + suffix), bool(suffix)


def _summary_records(shape):
    """Leading dims of the summary (one record per 16-token block)."""
    if shape.block_size == 0:
        return (shape.batch, shape.num_kv_heads, -(-shape.max_seq_len // 16))
    return (shape.num_blocks, shape.num_kv_heads, shape.block_size // 16)


def build_key_summary(q, k_cache, seq_lens, block_table=None, k_scale=None,
                      max_seq_len=None):
    """The 4-bit key summary the block-sparse call scans: (codes, scales)
    tensors on the cache's device, laid out as the C ABI describes
    (contiguous [B, Hkv, ceil(L/16), 8 * D] / [B, Hkv, ceil(L/16)], paged
    [NB, Hkv, bs/16, ...]). q only fixes the head layout of the shape."""
    import torch
    call, scaled = _sparse_call("fd_build_key_summary", k_cache)
    shape = validate_inputs(q, k_cache, k_cache, seq_lens, block_table,
                            k_scale, k_scale, max_seq_len)
    nrec = _summary_records(shape)
    D = shape.head_dim
    dev = k_cache.device
    codes = torch.zeros(nrec + (8 * D,), dtype=torch.uint8, device=dev)
    scales = torch.zeros(nrec, dtype=torch.float32, device=dev)
    if scaled:
        call(shape, k_cache, k_scale, block_table, seq_lens, codes, scales)
    else:
        call(shape, k_cache, block_table, seq_lens, codes, scales)
    return codes, scales


def sparse_decode_attention(q, k_cache, v_cache, seq_lens, summary,
                            delta: float, block_table=None,
                            num_splits: Optional[int] = None, scale=None,
                            max_seq_len=None, k_scale=None, v_scale=None,
                            return_lse: bool = False,
                            return_kept: bool = False):
    """Block-sparse decode: the blocks whose estimated best logit (from the
    summary ``build_key_summary`` returned) comes within ``delta`` (natural
    log units, >= 0; inf keeps everything) of the split's best, for some
    query head of the kv head, then exact attention over them. Tensors as
    for ``decode_attention``; the split count defaults to the planner's,
    raised until the splits fit the sparse path's limits."""
    import torch
    from . import binding
    call, scaled = _sparse_call("fd_decode_attn_sparse", k_cache)
    shape = validate_inputs(q, k_cache, v_cache, seq_lens, block_table,
                            k_scale, v_scale, max_seq_len)
    if scale:
        shape.scale = float(scale)
    if num_splits is None:
        cus = torch.cuda.get_device_properties(q.device).multi_processor_count
        num_splits = sparse_splits(shape, binding.fd_plan_splits(shape, cus,
                                                                 -1))
    codes, scales = summary
    nrec = _summary_records(shape)
    want = {"codes": (codes, torch.uint8, nrec + (8 * shape.head_dim,)),
            "scales": (scales, torch.float32, nrec)}
    for name, (t, dt, shp) in want.items():
        if (not isinstance(t, torch.Tensor) or t.dtype != dt
                or tuple(t.shape) != shp or not t.is_contiguous()
                or t.device != q.device):
            raise ValueError(f"summary {name} must be a contiguous {dt} "
                             f"{shp} tensor on {q.device} (as "
                             "build_key_summary returns)")
    out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    kept = None
    if return_kept:
        kept = torch.zeros(shape.batch, shape.num_kv_heads,
                           -(-shape.max_seq_len // 16), dtype=torch.uint8,
                           device=q.device)
    nbytes = binding.fd_workspace_size(shape, num_splits)
    ws = (torch.empty(nbytes, dtype=torch.uint8, device=q.device)
          if nbytes else None)
    if scaled:
        call(shape, q, k_cache, v_cache, k_scale, v_scale, codes, scales,
             block_table, seq_lens, delta, num_splits, ws, out, lse, kept)
    else:
        call(shape, q, k_cache, v_cache, codes, scales, block_table, seq_lens,
             delta, num_splits, ws, out, lse, kept)
    res = (out,)
    if return_lse:
        res += (lse,)
    if return_kept:
        res += (kept,)
    return res[0] if len(res) == 1 else res
