"""Split-KV (Flash-Decoding) decode attention for MI355X (gfx950).

The compute lives in ``lib/libfd_decode.so`` (hand-written HIP kernels behind
the C ABI in ``include/fd_decode.h``); ``binding`` exposes the same calls to
Python, and ``decode_attention`` below is a convenience wrapper that sizes
and allocates the outputs with torch before calling ``fd_decode_attn``.
"""

from __future__ import annotations

from typing import Optional

__all__ = ["decode_attention", "shape_for"]


def shape_for(q, k_cache, seq_lens, block_table=None, max_seq_len=None,
              scale=None):
    """fd_shape for torch tensors laid out as the C ABI describes."""
    import torch
    from . import binding
    B, Hq, D = q.shape
    if block_table is None:
        _, Hkv, L, _ = k_cache.shape
        bs = maxb = nb = 0
    else:
        nb, Hkv, bs, _ = k_cache.shape
        maxb = block_table.shape[1]
        L = max_seq_len if max_seq_len is not None else maxb * bs
    if max_seq_len is not None:
        L = max_seq_len
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


def decode_attention(q, k_cache, v_cache, seq_lens, block_table=None,
                     num_splits: Optional[int] = None, scale=None,
                     max_seq_len=None, return_lse: bool = False,
                     k_scale=None, v_scale=None):
    """out[b, h] = softmax attention of q[b, h] over the first seq_lens[b]
    cached positions (fp32). Tensors must be on the current GPU. An E4M3
    cache (torch.float8_e4m3fn) needs k_scale / v_scale (fp32 [Hkv]); an
    int8 cache needs them per (position, kv head), laid out like the cache
    without head_dim."""
    import torch
    from . import binding
    if v_cache.dtype != k_cache.dtype or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must match in dtype and shape")
    shape = shape_for(q, k_cache, seq_lens, block_table, max_seq_len, scale)
    if num_splits is None:
        cus = torch.cuda.get_device_properties(q.device).multi_processor_count
        num_splits = binding.fd_plan_splits(shape, cus, -1)
    out = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    nbytes = binding.fd_workspace_size(shape, num_splits)
    ws = (torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
          if nbytes else None)
    if k_cache.dtype in (torch.float8_e4m3fn, torch.int8):
        if k_scale is None or v_scale is None:
            raise ValueError("an 8-bit cache needs k_scale and v_scale")
        call = (binding.fd_decode_attn_fp8
                if k_cache.dtype == torch.float8_e4m3fn
                else binding.fd_decode_attn_int8)
        call(shape, q, k_cache, v_cache, k_scale, v_scale, block_table,
             seq_lens, num_splits, ws, out, lse)
    else:
        binding.fd_decode_attn(shape, q, k_cache, v_cache, block_table,
                               seq_lens, num_splits, ws, out, lse)
    return (out, lse) if return_lse else out
