"""ctypes binding of libfd_decode.so, with the C ABI's names.

Argument marshalling only: torch tensors are turned into device pointers and
the current HIP stream; every step of decode attention runs in the library's
kernels. Loading fails loudly if the library has not been built.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "lib", "libfd_decode.so")

FD_OK = 0
FD_ERR_INVALID_ARG = -1
FD_ERR_UNSUPPORTED = -2
FD_ERR_WORKSPACE = -3
FD_ERR_HIP = -4

FD_DTYPE_F32 = 0
FD_DTYPE_BF16 = 1
FD_DTYPE_FP8_E4M3 = 2
FD_DTYPE_INT8 = 3
_DTYPES = {"f32": FD_DTYPE_F32, "bf16": FD_DTYPE_BF16,
           "fp8_e4m3": FD_DTYPE_FP8_E4M3, "int8": FD_DTYPE_INT8}

SYMBOLS = ["fd_plan_splits", "fd_workspace_size", "fd_decode_attn",
           "fd_decode_partials", "fd_decode_attn_fp8",
           "fd_decode_partials_fp8", "fd_decode_attn_int8",
           "fd_decode_partials_int8", "fd_build_key_summary",
           "fd_decode_attn_sparse", "fd_combine_partials", "fd_status_str",
           "fd_version", "fd_read_probe", "fd_decode_attn_noalloc",
           "fd_build_key_summary_fp8", "fd_decode_attn_sparse_fp8",
           "fd_build_key_summary_int8", "fd_decode_attn_sparse_int8"]


class FdShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32),
                ("max_seq_len", ctypes.c_int32),
                ("block_size", ctypes.c_int32),
                ("max_blocks_per_seq", ctypes.c_int32),
                ("num_blocks", ctypes.c_int32),
                ("dtype", ctypes.c_int32),
                ("scale", ctypes.c_float)]


class FdError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {fd_status_str(status)} ({status})")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    """Load the built library (once). Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m split_kv_long_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, I64, SZ = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                     ctypes.c_size_t)
    SH = ctypes.POINTER(FdShape)
    lib.fd_plan_splits.argtypes = [SH, I, I64, ctypes.POINTER(I)]
    lib.fd_workspace_size.argtypes = [SH, I, ctypes.POINTER(SZ)]
    lib.fd_decode_attn.argtypes = [SH, P, P, P, P, P, I, P, SZ, P, P, P]
    lib.fd_decode_partials.argtypes = [SH, P, P, P, P, P, I, P, P, P]
    lib.fd_decode_attn_fp8.argtypes = [SH, P, P, P, P, P, P, P, I, P, SZ, P,
                                       P, P]
    lib.fd_decode_partials_fp8.argtypes = [SH, P, P, P, P, P, P, P, I, P, P,
                                           P]
    lib.fd_decode_attn_int8.argtypes = [SH, P, P, P, P, P, P, P, I, P, SZ, P,
                                        P, P]
    lib.fd_decode_partials_int8.argtypes = [SH, P, P, P, P, P, P, P, I, P, P,
                                            P]
    lib.fd_build_key_summary.argtypes = [SH, P, P, P, P, P, P]
    lib.fd_decode_attn_sparse.argtypes = [SH, P, P, P, P, P, P, P,
                                          ctypes.c_float, I, P, SZ, P, P, P,
                                          P]
    for nm in ("fd_build_key_summary_fp8", "fd_build_key_summary_int8"):
        getattr(lib, nm).argtypes = [SH, P, P, P, P, P, P, P]
    for nm in ("fd_decode_attn_sparse_fp8", "fd_decode_attn_sparse_int8"):
        getattr(lib, nm).argtypes = [SH, P, P, P, P, P, P, P, P, P,
                                     ctypes.c_float, I, P, SZ, P, P, P, P]
    lib.fd_combine_partials.argtypes = [I, I, I, I, P, P, P, P, P]
    lib.fd_status_str.argtypes = [I]
    lib.fd_status_str.restype = ctypes.c_char_p
    lib.fd_version.argtypes = []
    lib.fd_read_probe.argtypes = [P, SZ, I, I, I, P, P]
    lib.fd_decode_attn_noalloc.argtypes = [SH, P, P, P, P, P, I, P, P, P]
    for name in SYMBOLS:
        if name != "fd_status_str":
            getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def make_shape(batch, num_q_heads, num_kv_heads, head_dim, max_seq_len,
               dtype="bf16", block_size=0, max_blocks_per_seq=0, num_blocks=0,
               scale=0.0) -> FdShape:
    dt = _DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    return FdShape(batch, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                   block_size, max_blocks_per_seq, num_blocks, dt,
                   float(scale or 0.0))


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream or None
    return stream if isinstance(stream, int) else stream.cuda_stream


def _check(fn: str, st: int) -> None:
    if st != FD_OK:
        raise FdError(fn, st)


def fd_status_str(status: int) -> str:
    return load().fd_status_str(int(status)).decode()


def fd_version() -> int:
    return load().fd_version()


def fd_plan_splits(shape: FdShape, num_cus: int, sum_seq_len: int = -1) -> int:
    out = ctypes.c_int(0)
    _check("fd_plan_splits", load().fd_plan_splits(
        ctypes.byref(shape), int(num_cus), int(sum_seq_len), ctypes.byref(out)))
    return out.value


def fd_workspace_size(shape: FdShape, num_splits: int) -> int:
    out = ctypes.c_size_t(0)
    _check("fd_workspace_size", load().fd_workspace_size(
        ctypes.byref(shape), int(num_splits), ctypes.byref(out)))
    return out.value


def fd_decode_attn(shape: FdShape, q, k_cache, v_cache, block_table, seq_lens,
                   num_splits: int, workspace, out, lse_out=None,
                   stream=None, workspace_bytes: Optional[int] = None) -> None:
    """Enqueue decode attention; tensors must be on the current device."""
    ws_bytes = (workspace_bytes if workspace_bytes is not None else
                (0 if workspace is None or isinstance(workspace, int)
                 else workspace.numel() * workspace.element_size()))
    _check("fd_decode_attn", load().fd_decode_attn(
        ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache),
        _ptr(block_table), _ptr(seq_lens), int(num_splits), _ptr(workspace),
        ws_bytes, _ptr(out), _ptr(lse_out), _stream(stream)))


def fd_decode_attn_noalloc(shape: FdShape, q, k_cache, v_cache,
                           block_table, seq_lens, num_splits: int, out,
                           lse_out=None, stream=None) -> None:
    """fd_decode_attn with the library's per-device scratch (no workspace)."""
    _check("fd_decode_attn_noalloc", load().fd_decode_attn_noalloc(
        ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache),
        _ptr(block_table), _ptr(seq_lens), int(num_splits), _ptr(out),
        _ptr(lse_out), _stream(stream)))


def fd_decode_partials(shape: FdShape, q, k_cache, v_cache, block_table,
                       seq_lens, num_splits: int, o_part, lse_part,
                       stream=None) -> None:
    _check("fd_decode_partials", load().fd_decode_partials(
        ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache),
        _ptr(block_table), _ptr(seq_lens), int(num_splits), _ptr(o_part),
        _ptr(lse_part), _stream(stream)))


def fd_decode_attn_fp8(shape: FdShape, q, k_cache, v_cache, k_scale, v_scale,
                       block_table, seq_lens, num_splits: int, workspace,
                       out, lse_out=None, stream=None,
                       workspace_bytes: Optional[int] = None) -> None:
    """Enqueue decode attention over an 8-bit E4M3 cache with per-kv-head
    fp32 scales (shape dtype "fp8_e4m3", q bf16)."""
    ws_bytes = (workspace_bytes if workspace_bytes is not None else
                (0 if workspace is None or isinstance(workspace, int)
                 else workspace.numel() * workspace.element_size()))
    _check("fd_decode_attn_fp8", load().fd_decode_attn_fp8(
        ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache),
        _ptr(k_scale), _ptr(v_scale), _ptr(block_table), _ptr(seq_lens),
        int(num_splits), _ptr(workspace), ws_bytes, _ptr(out), _ptr(lse_out),
        _stream(stream)))


def fd_decode_partials_fp8(shape: FdShape, q, k_cache, v_cache, k_scale,
                           v_scale, block_table, seq_lens, num_splits: int,
                           o_part, lse_part, stream=None) -> None:
    _check("fd_decode_partials_fp8", load().fd_decode_partials_fp8(
        ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache),
        _ptr(k_scale), _ptr(v_scale), _ptr(block_table), _ptr(seq_lens),
        int(num_splits), _ptr(o_part), _ptr(lse_part), _stream(stream)))


def fd_decode_attn_int8(shape: FdShape, q, k_cache, v_cache, k_scale,
                        v_scale, block_table, seq_lens, num_splits: int,
                        workspace, out, lse_out=None, stream=None,
                        workspace_bytes: Optional[int] = None) -> None:
    """Enqueue decode attention over an int8 cache with one fp32 scale per
    (position, kv head) (shape dtype "int8", q bf16; scales laid out like
    the cache without head_dim)."""
    ws_bytes = (workspace_bytes if workspace_bytes is not None else
                (0 if workspace is None or isinstance(workspace, int)
                 else workspace.numel() * workspace.element_size()))
    _check("fd_decode_attn_int8", load().fd_decode_attn_int8(
        ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache),
        _ptr(k_scale), _ptr(v_scale), _ptr(block_table), _ptr(seq_lens),
        int(num_splits), _ptr(workspace), ws_bytes, _ptr(out), _ptr(lse_out),
        _stream(stream)))


def fd_decode_partials_int8(shape: FdShape, q, k_cache, v_cache, k_scale,
                            v_scale, block_table, seq_lens, num_splits: int,
                            o_part, lse_part, stream=None) -> None:
    _check("fd_decode_partials_int8", load().fd_decode_partials_int8(
        ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache),
        _ptr(k_scale), _ptr(v_scale), _ptr(block_table), _ptr(seq_lens),
        int(num_splits), _ptr(o_part), _ptr(lse_part), _stream(stream)))


def fd_build_key_summary(shape: FdShape, k_cache, block_table, seq_lens,
                         codes, scales, stream=None) -> None:
    """4-bit key summary (codes + per-16-token-block scales) of bf16 keys."""
    _check("fd_build_key_summary", load().fd_build_key_summary(
        ctypes.byref(shape), _ptr(k_cache), _ptr(block_table),
        _ptr(seq_lens), _ptr(codes), _ptr(scales), _stream(stream)))


def fd_decode_attn_sparse(shape: FdShape, q, k_cache, v_cache, codes, scales,
                          block_table, seq_lens, delta: float,
                          num_splits: int, workspace, out, lse_out=None,
                          kept_out=None, stream=None,
                          workspace_bytes: Optional[int] = None) -> None:
    """Block-sparse decode: top-delta over the key summary, exact attention
    over the kept 16-token blocks."""
    ws_bytes = (workspace_bytes if workspace_bytes is not None else
                (0 if workspace is None or isinstance(workspace, int)
                 else workspace.numel() * workspace.element_size()))
    _check("fd_decode_attn_sparse", load().fd_decode_attn_sparse(
        ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache),
        _ptr(codes), _ptr(scales), _ptr(block_table), _ptr(seq_lens),
        float(delta), int(num_splits), _ptr(workspace), ws_bytes, _ptr(out),
        _ptr(lse_out), _ptr(kept_out), _stream(stream)))


def _summary8(name, shape, k_cache, k_scale, block_table, seq_lens, codes,
              scales, stream):
    _check(name, getattr(load(), name)(
        ctypes.byref(shape), _ptr(k_cache), _ptr(k_scale), _ptr(block_table),
        _ptr(seq_lens), _ptr(codes), _ptr(scales), _stream(stream)))


def _sparse8(name, shape, q, k_cache, v_cache, k_scale, v_scale, codes,
             scales, block_table, seq_lens, delta, num_splits, workspace, out,
             lse_out, kept_out, stream, workspace_bytes):
    ws_bytes = (workspace_bytes if workspace_bytes is not None else
                (0 if workspace is None or isinstance(workspace, int)
                 else workspace.numel() * workspace.element_size()))
    _check(name, getattr(load(), name)(
        ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache),
        _ptr(k_scale), _ptr(v_scale), _ptr(codes), _ptr(scales),
        _ptr(block_table), _ptr(seq_lens), float(delta), int(num_splits),
        _ptr(workspace), ws_bytes, _ptr(out), _ptr(lse_out), _ptr(kept_out),
        _stream(stream)))


def fd_build_key_summary_fp8(shape: FdShape, k_cache, k_scale, block_table,
                             seq_lens, codes, scales, stream=None) -> None:
    """4-bit key summary of an E4M3 key cache (keys = code x k_scale)."""
    _summary8("fd_build_key_summary_fp8", shape, k_cache, k_scale,
              block_table, seq_lens, codes, scales, stream)


def fd_build_key_summary_int8(shape: FdShape, k_cache, k_scale, block_table,
                              seq_lens, codes, scales, stream=None) -> None:
    """4-bit key summary of an int8 key cache with per-position scales."""
    _summary8("fd_build_key_summary_int8", shape, k_cache, k_scale,
              block_table, seq_lens, codes, scales, stream)


def fd_decode_attn_sparse_fp8(shape: FdShape, q, k_cache, v_cache, k_scale,
                              v_scale, codes, scales, block_table, seq_lens,
                              delta: float, num_splits: int, workspace, out,
                              lse_out=None, kept_out=None, stream=None,
                              workspace_bytes: Optional[int] = None) -> None:
    """Block-sparse decode over an E4M3 cache with per-kv-head scales."""
    _sparse8("fd_decode_attn_sparse_fp8", shape, q, k_cache, v_cache,
             k_scale, v_scale, codes, scales, block_table, seq_lens, delta,
             num_splits, workspace, out, lse_out, kept_out, stream,
             workspace_bytes)


def fd_decode_attn_sparse_int8(shape: FdShape, q, k_cache, v_cache, k_scale,
                               v_scale, codes, scales, block_table, seq_lens,
                               delta: float, num_splits: int, workspace, out,
                               lse_out=None, kept_out=None, stream=None,
                               workspace_bytes: Optional[int] = None) -> None:
    """Block-sparse decode over an int8 cache with per-position scales."""
    _sparse8("fd_decode_attn_sparse_int8", shape, q, k_cache, v_cache,
             k_scale, v_scale, codes, scales, block_table, seq_lens, delta,
             num_splits, workspace, out, lse_out, kept_out, stream,
             workspace_bytes)


def fd_combine_partials(batch: int, num_q_heads: int, head_dim: int,
                        num_splits: int, o_part, lse_part, out, lse_out=None,
                        stream=None) -> None:
    _check("fd_combine_partials", load().fd_combine_partials(
        int(batch), int(num_q_heads), int(head_dim), int(num_splits),
        _ptr(o_part), _ptr(lse_part), _ptr(out), _ptr(lse_out),
        _stream(stream)))


def fd_read_probe(buf, workgroups: int, waves: int, loads_per_lane: int,
                  sink, stream=None, nbytes: Optional[int] = None) -> None:
    """Enqueue the HBM read probe (fd_probe.h) over a device tensor."""
    n = nbytes if nbytes is not None else buf.numel() * buf.element_size()
    _check("fd_read_probe", load().fd_read_probe(
        _ptr(buf), int(n), int(workgroups), int(waves), int(loads_per_lane),
        _ptr(sink), _stream(stream)))
