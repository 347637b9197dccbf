// Host side of the C ABI: argument checks, split planning, workspace sizing
// and the entry points that hand validated calls to the HIP launchers.
//
// Nothing here touches the device; every check runs before anything is
// enqueued, so a rejected call has no effect.

#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "fd_internal.h"

namespace fd {

static bool aligned16(const void* p) {
  return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

static size_t round_up(size_t x, size_t m) { return (x + m - 1) / m * m; }

int check_shape(const fd_shape* s, Shape* out) {
  if (!s) return FD_ERR_INVALID_ARG;
  if (s->batch < 1 || s->num_q_heads < 1 || s->num_kv_heads < 1)
    return FD_ERR_INVALID_ARG;
  if (s->num_q_heads % s->num_kv_heads != 0) return FD_ERR_INVALID_ARG;
  if (s->max_seq_len < 0) return FD_ERR_INVALID_ARG;
  if (s->head_dim <= 0 || (s->head_dim % 16) != 0) return FD_ERR_INVALID_ARG;
  if (s->head_dim != 64 && s->head_dim != 128) return FD_ERR_UNSUPPORTED;
  if (s->dtype != FD_DTYPE_F32 && s->dtype != FD_DTYPE_BF16 &&
      s->dtype != FD_DTYPE_FP8_E4M3 && s->dtype != FD_DTYPE_INT8)
    return FD_ERR_UNSUPPORTED;
  if (!isfinite(s->scale)) return FD_ERR_INVALID_ARG;
  if (s->batch > 65535) return FD_ERR_UNSUPPORTED;       // grid y
  if (s->block_size != 0) {
    if (s->block_size < 0 || s->block_size % 16 != 0 ||
        s->block_size > kMaxBlockSize)
      return FD_ERR_INVALID_ARG;
    int64_t need = ((int64_t)s->max_seq_len + s->block_size - 1) / s->block_size;
    if (s->max_blocks_per_seq < need || s->max_blocks_per_seq < 1)
      return FD_ERR_INVALID_ARG;
    if (s->num_blocks < 1) return FD_ERR_INVALID_ARG;
  }
  Shape r;
  r.B = s->batch;
  r.Hq = s->num_q_heads;
  r.Hkv = s->num_kv_heads;
  r.G = s->num_q_heads / s->num_kv_heads;
  r.D = s->head_dim;
  r.L = s->max_seq_len;
  r.bs = s->block_size;
  r.max_blocks = s->block_size ? s->max_blocks_per_seq : 0;
  r.num_blocks = s->block_size ? s->num_blocks : 0;
  r.dtype = s->dtype;
  r.scale = s->scale > 0.f ? s->scale : (float)(1.0 / sqrt((double)s->head_dim));
  if ((int64_t)r.Hkv * head_groups(r) > INT32_MAX) return FD_ERR_UNSUPPORTED;  // grid x
  // (sequence, kv head) row indices are formed in 32-bit arithmetic
  if ((int64_t)r.B * r.Hkv > INT32_MAX || (int64_t)r.B * r.Hq > INT32_MAX)
    return FD_ERR_UNSUPPORTED;
  if (out) *out = r;
  return FD_OK;
}

int head_groups(const Shape& s) {
  return (s.G + kHeadsPerGroup - 1) / kHeadsPerGroup;
}

static int64_t tokens_per_split64(const Shape& s, int num_splits) {
  const int64_t g = s.bs > 16 ? s.bs : 16;
  const int64_t L = s.L > 0 ? s.L : 1;
  const int64_t per = (L + num_splits - 1) / num_splits;
  return (per + g - 1) / g * g;
}

int tokens_per_split(const Shape& s, int num_splits) {
  return (int)tokens_per_split64(s, num_splits);   // checked by check_splits
}

size_t partial_o_bytes(const Shape& s, int num_splits) {
  return round_up((size_t)s.B * s.Hq * num_splits * s.D * sizeof(float), 256);
}

size_t workspace_bytes(const Shape& s, int num_splits) {
  if (num_splits <= 1) return 0;
  return partial_o_bytes(s, num_splits) +
         round_up((size_t)s.B * s.Hq * num_splits * sizeof(float), 256);
}

static int check_splits(const Shape& s, int num_splits) {
  if (num_splits < 1 || num_splits > kMaxSplits) return FD_ERR_INVALID_ARG;
  // B*Hq*S*D must stay addressable with 64-bit offsets and 32-bit rows.
  if ((int64_t)s.B * s.Hq * num_splits > INT32_MAX) return FD_ERR_UNSUPPORTED;
  if ((int64_t)s.B * s.Hq * 16 > INT32_MAX) return FD_ERR_UNSUPPORTED;   // combine grid
  // split starts s * P stay 32-bit
  if ((int64_t)num_splits * tokens_per_split64(s, num_splits) > INT32_MAX)
    return FD_ERR_UNSUPPORTED;
  return FD_OK;
}

static int check_inputs(const Shape& s, const void* q, const void* k,
                        const void* v, const int32_t* block_table,
                        const int32_t* seq_lens) {
  if (!q || !k || !v || !seq_lens) return FD_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v)) return FD_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(seq_lens) & 3u) != 0) return FD_ERR_INVALID_ARG;
  if (s.bs > 0) {
    if (!block_table) return FD_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(block_table) & 3u) != 0)
      return FD_ERR_INVALID_ARG;
  } else if (block_table) {
    return FD_ERR_INVALID_ARG;
  }
  return FD_OK;
}

// Quantized caches come with their scales and only through their own
// calls: `scaled` is the dtype the entry point takes (FD_DTYPE_FP8_E4M3 or
// FD_DTYPE_INT8), or -1 for the unscaled calls.
static int check_scales(const Shape& s, const float* ks, const float* vs,
                        int scaled) {
  const bool quant =
      s.dtype == FD_DTYPE_FP8_E4M3 || s.dtype == FD_DTYPE_INT8;
  if (scaled < 0) return quant ? FD_ERR_INVALID_ARG : FD_OK;
  if (s.dtype != scaled) return FD_ERR_INVALID_ARG;
  if (!ks || !vs) return FD_ERR_INVALID_ARG;
  // Per-position scales are read 4 at a time.
  const uintptr_t align = s.dtype == FD_DTYPE_INT8 ? 15u : 3u;
  if ((reinterpret_cast<uintptr_t>(ks) & align) != 0 ||
      (reinterpret_cast<uintptr_t>(vs) & align) != 0)
    return FD_ERR_INVALID_ARG;
  return FD_OK;
}

// Compute units of the current device (0 if the query fails: the uniform
// split layout is used then).
static int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
      hipSuccess)
    return 0;
  return cus;
}

static SplitArgs make_split_args(const Shape& s, const void* q, const void* k,
                                 const void* v, const int32_t* bt,
                                 const int32_t* seq_lens, int S) {
  SplitArgs a;
  memset(&a, 0, sizeof(a));
  a.q = q;
  a.k = k;
  a.v = v;
  a.block_table = bt;
  a.seq_lens = seq_lens;
  a.B = s.B;
  a.Hq = s.Hq;
  a.Hkv = s.Hkv;
  a.G = s.G;
  a.L = s.L;
  a.bs = s.bs;
  a.max_blocks = s.max_blocks;
  a.num_blocks = s.num_blocks;
  a.S = S;
  a.P = tokens_per_split(s, S);
  a.nhg = head_groups(s);
  a.scale_log2 = (float)((double)s.scale * 1.4426950408889634);
  return a;
}

}  // namespace fd

using namespace fd;

extern "C" {

int fd_version(void) { return 10100; }   // 1.1.0: int8 cache calls

const char* fd_status_str(int status) {
  switch (status) {
    case FD_OK: return "ok";
    case FD_ERR_INVALID_ARG: return "invalid argument";
    case FD_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case FD_ERR_WORKSPACE: return "workspace missing or too small";
    case FD_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int fd_plan_splits(const fd_shape* shape, int num_cus, int64_t sum_seq_len,
                   int* num_splits) {
  Shape s;
  int st = check_shape(shape, &s);
  if (st != FD_OK) return st;
  if (!num_splits || num_cus < 1) return FD_ERR_INVALID_ARG;
  if (sum_seq_len < -1 || sum_seq_len > (int64_t)s.B * s.L)
    return FD_ERR_INVALID_ARG;
  const int64_t units = (int64_t)s.B * s.Hkv * head_groups(s);
  const int64_t cmin =
      s.dtype == FD_DTYPE_F32 ? kMinSplitTokensF32 : kMinSplitTokens;
  // No split when the sequences alone fill the CUs, when the history is
  // shorter than two minimum splits, or when they fill half the CUs (an
  // 8-bit cache: a few units) and the history is short (the combine then
  // costs more than it saves).
  const bool q8 = s.dtype == FD_DTYPE_FP8_E4M3 || s.dtype == FD_DTYPE_INT8;
  const bool short_batch =
      2 * units >= num_cus || (q8 && units >= kShortHistoryUnits8);
  if (units >= num_cus || s.L < 2 * cmin ||
      (short_batch && s.L < kShortHistoryTokens)) {
    *num_splits = 1;
    return FD_OK;
  }
  const int64_t tokens = (sum_seq_len >= 0 ? sum_seq_len : (int64_t)s.B * s.L);
  const int64_t work = tokens * s.Hkv * head_groups(s);
  const int64_t target = (int64_t)kOccupancy * num_cus;
  int64_t per = (work + target - 1) / target;
  // A ragged batch (a known total below batch x bound): long splits are
  // halved, so the length-aware pieces can even out about two workgroups
  // per CU. Uniform histories keep one workgroup per CU.
  const bool ragged = sum_seq_len >= 0 && sum_seq_len < (int64_t)s.B * s.L;
  // int8 batches of 2..64 run 4-wave pieces, about two per CU: halved at
  // any length.
  const bool i8_pieces = s.dtype == FD_DTYPE_INT8 && s.B > 1 && s.B <= 64;
  if ((ragged && per > kLongSplitTokens) || i8_pieces) per = (per + 1) / 2;
  if (per < cmin) per = cmin;
  const int64_t g = s.bs > 16 ? s.bs : 16;
  per = (per + g - 1) / g * g;
  int64_t S = (s.L + per - 1) / per;
  if (S < 1) S = 1;
  if (S > kMaxSplits) S = kMaxSplits;
  *num_splits = (int)S;
  return FD_OK;
}

int fd_workspace_size(const fd_shape* shape, int num_splits, size_t* bytes) {
  Shape s;
  int st = check_shape(shape, &s);
  if (st != FD_OK) return st;
  if (!bytes) return FD_ERR_INVALID_ARG;
  st = check_splits(s, num_splits);
  if (st != FD_OK) return st;
  *bytes = workspace_bytes(s, num_splits);
  return FD_OK;
}

}  // extern "C"

namespace fd {

static int decode_attn(const fd_shape* shape, const void* q,
                       const void* k_cache, const void* v_cache,
                       const float* k_scale, const float* v_scale,
                       int scaled, const int32_t* block_table,
                       const int32_t* seq_lens, int num_splits,
                       void* workspace, size_t ws_bytes, float* out,
                       float* lse_out, void* stream) {
  Shape s;
  int st = check_shape(shape, &s);
  if (st != FD_OK) return st;
  st = check_splits(s, num_splits);
  if (st != FD_OK) return st;
  st = check_inputs(s, q, k_cache, v_cache, block_table, seq_lens);
  if (st != FD_OK) return st;
  st = check_scales(s, k_scale, v_scale, scaled);
  if (st != FD_OK) return st;
  if (!out || !aligned16(out)) return FD_ERR_INVALID_ARG;
  if (lse_out && (reinterpret_cast<uintptr_t>(lse_out) & 3u) != 0)
    return FD_ERR_INVALID_ARG;
  if (num_splits > 1) {
    if (!workspace || ws_bytes < workspace_bytes(s, num_splits))
      return FD_ERR_WORKSPACE;
    if (!aligned16(workspace)) return FD_ERR_INVALID_ARG;
  }
  SplitArgs a = make_split_args(s, q, k_cache, v_cache, block_table, seq_lens,
                                num_splits);
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  // Batched calls cut each sequence into pieces by its length (the partial
  // slots stay internal to this call, so their layout may differ from
  // fd_decode_partials' uniform splits).
  if (s.B > 1 && num_splits > 1) a.balance_cus = device_cus();
  if (num_splits == 1) {
    a.o_dst = out;
    a.lse_dst = lse_out;
    a.final_out = 1;
    return launch_split(s, a, stream) == 0 ? FD_OK : FD_ERR_HIP;
  }
  float* o_part = static_cast<float*>(workspace);
  float* lse_part = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                             partial_o_bytes(s, num_splits));
  a.o_dst = o_part;
  a.lse_dst = lse_part;
  a.final_out = 0;
  if (launch_split(s, a, stream) != 0) return FD_ERR_HIP;
  CombineArgs c;
  c.o_part = o_part;
  c.lse_part = lse_part;
  c.out = out;
  c.lse_out = lse_out;
  c.B = s.B;
  c.Hq = s.Hq;
  c.S = num_splits;
  return launch_combine(s.D, c, stream) == 0 ? FD_OK : FD_ERR_HIP;
}

static int decode_partials(const fd_shape* shape, const void* q,
                           const void* k_cache, const void* v_cache,
                           const float* k_scale, const float* v_scale,
                           int scaled, const int32_t* block_table,
                           const int32_t* seq_lens, int num_splits,
                           float* o_part, float* lse_part, void* stream) {
  Shape s;
  int st = check_shape(shape, &s);
  if (st != FD_OK) return st;
  st = check_splits(s, num_splits);
  if (st != FD_OK) return st;
  st = check_inputs(s, q, k_cache, v_cache, block_table, seq_lens);
  if (st != FD_OK) return st;
  st = check_scales(s, k_scale, v_scale, scaled);
  if (st != FD_OK) return st;
  if (!o_part || !lse_part || !aligned16(o_part) ||
      (reinterpret_cast<uintptr_t>(lse_part) & 3u) != 0)
    return FD_ERR_INVALID_ARG;
  SplitArgs a = make_split_args(s, q, k_cache, v_cache, block_table, seq_lens,
                                num_splits);
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.o_dst = o_part;
  a.lse_dst = lse_part;
  a.final_out = 0;
  return launch_split(s, a, stream) == 0 ? FD_OK : FD_ERR_HIP;
}

}  // namespace fd

extern "C" {

int fd_decode_attn(const fd_shape* shape, const void* q, const void* k_cache,
                   const void* v_cache, const int32_t* block_table,
                   const int32_t* seq_lens, int num_splits, void* workspace,
                   size_t ws_bytes, float* out, float* lse_out, void* stream) {
  return decode_attn(shape, q, k_cache, v_cache, nullptr, nullptr, -1,
                     block_table, seq_lens, num_splits, workspace, ws_bytes,
                     out, lse_out, stream);
}

int fd_decode_attn_noalloc(const fd_shape* shape, const void* q,
                           const void* k_cache, const void* v_cache,
                           const int32_t* block_table,
                           const int32_t* seq_lens, int num_splits,
                           float* out, float* lse_out, void* stream) {
  Shape s;
  int st = check_shape(shape, &s);
  if (st != FD_OK) return st;
  st = check_splits(s, num_splits);
  if (st != FD_OK) return st;
  const size_t need = workspace_bytes(s, num_splits);
  if (need > kScratchBytes) return FD_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0 && scratch_address(&ws) != 0) return FD_ERR_HIP;
  return decode_attn(shape, q, k_cache, v_cache, nullptr, nullptr, -1,
                     block_table, seq_lens, num_splits, ws, need, out,
                     lse_out, stream);
}

int fd_decode_attn_fp8(const fd_shape* shape, const void* q,
                       const void* k_cache, const void* v_cache,
                       const float* k_scale, const float* v_scale,
                       const int32_t* block_table, const int32_t* seq_lens,
                       int num_splits, void* workspace, size_t ws_bytes,
                       float* out, float* lse_out, void* stream) {
  return decode_attn(shape, q, k_cache, v_cache, k_scale, v_scale,
                     FD_DTYPE_FP8_E4M3,
                     block_table, seq_lens, num_splits, workspace, ws_bytes,
                     out, lse_out, stream);
}

int fd_decode_partials(const fd_shape* shape, const void* q,
                       const void* k_cache, const void* v_cache,
                       const int32_t* block_table, const int32_t* seq_lens,
                       int num_splits, float* o_part, float* lse_part,
                       void* stream) {
  return decode_partials(shape, q, k_cache, v_cache, nullptr, nullptr, -1,
                         block_table, seq_lens, num_splits, o_part, lse_part,
                         stream);
}

int fd_decode_partials_fp8(const fd_shape* shape, const void* q,
                           const void* k_cache, const void* v_cache,
                           const float* k_scale, const float* v_scale,
                           const int32_t* block_table,
                           const int32_t* seq_lens, int num_splits,
                           float* o_part, float* lse_part, void* stream) {
  return decode_partials(shape, q, k_cache, v_cache, k_scale, v_scale,
                         FD_DTYPE_FP8_E4M3,
                         block_table, seq_lens, num_splits, o_part, lse_part,
                         stream);
}

int fd_decode_attn_int8(const fd_shape* shape, const void* q,
                        const void* k_cache, const void* v_cache,
                        const float* k_scale, const float* v_scale,
                        const int32_t* block_table, const int32_t* seq_lens,
                        int num_splits, void* workspace, size_t ws_bytes,
                        float* out, float* lse_out, void* stream) {
  return decode_attn(shape, q, k_cache, v_cache, k_scale, v_scale,
                     FD_DTYPE_INT8, block_table, seq_lens, num_splits,
                     workspace, ws_bytes, out, lse_out, stream);
}

int fd_decode_partials_int8(const fd_shape* shape, const void* q,
                            const void* k_cache, const void* v_cache,
                            const float* k_scale, const float* v_scale,
                            const int32_t* block_table,
                            const int32_t* seq_lens, int num_splits,
                            float* o_part, float* lse_part, void* stream) {
  return decode_partials(shape, q, k_cache, v_cache, k_scale, v_scale,
                         FD_DTYPE_INT8, block_table, seq_lens, num_splits,
                         o_part, lse_part, stream);
}

// The sparse calls take bf16 caches (scaled = -1), E4M3 caches with their
// per-kv-head scales (scaled = FD_DTYPE_FP8_E4M3) or int8 caches with their
// per-position scales (FD_DTYPE_INT8), each through its own entry points.
static int check_sparse_dtype(const Shape& s, int scaled) {
  if (scaled < 0) return s.dtype == FD_DTYPE_BF16 ? FD_OK : FD_ERR_UNSUPPORTED;
  return s.dtype == scaled ? FD_OK : FD_ERR_INVALID_ARG;
}

static int build_key_summary(const fd_shape* shape, const void* k_cache,
                             const float* k_scale, int scaled,
                             const int32_t* block_table,
                             const int32_t* seq_lens, void* codes,
                             float* scales, void* stream) {
  Shape s;
  int st = check_shape(shape, &s);
  if (st != FD_OK) return st;
  st = check_sparse_dtype(s, scaled);
  if (st != FD_OK) return st;
  st = check_inputs(s, k_cache, k_cache, k_cache, block_table, seq_lens);
  if (st != FD_OK) return st;
  if (scaled >= 0 &&
      (!k_scale || (reinterpret_cast<uintptr_t>(k_scale) & 3u) != 0))
    return FD_ERR_INVALID_ARG;
  if (!codes || !scales || !aligned16(codes) ||
      (reinterpret_cast<uintptr_t>(scales) & 3u) != 0)
    return FD_ERR_INVALID_ARG;
  SummaryArgs a;
  memset(&a, 0, sizeof(a));
  a.k = k_cache;
  a.k_scale = scaled >= 0 ? k_scale : nullptr;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.codes = static_cast<uint8_t*>(codes);
  a.scales = scales;
  a.Hkv = s.Hkv;
  a.L = s.L;
  a.bs = s.bs;
  a.max_blocks = s.max_blocks;
  a.num_blocks = s.num_blocks;
  a.nblk_row = (int)(((int64_t)s.L + 15) / 16);   // L may be INT32_MAX
  return launch_summary(s, a, stream) == 0 ? FD_OK : FD_ERR_HIP;
}

int fd_build_key_summary(const fd_shape* shape, const void* k_cache,
                         const int32_t* block_table, const int32_t* seq_lens,
                         void* codes, float* scales, void* stream) {
  return build_key_summary(shape, k_cache, nullptr, -1, block_table, seq_lens,
                           codes, scales, stream);
}

int fd_build_key_summary_fp8(const fd_shape* shape, const void* k_cache,
                             const float* k_scale, const int32_t* block_table,
                             const int32_t* seq_lens, void* codes,
                             float* scales, void* stream) {
  return build_key_summary(shape, k_cache, k_scale, FD_DTYPE_FP8_E4M3,
                           block_table, seq_lens, codes, scales, stream);
}

int fd_build_key_summary_int8(const fd_shape* shape, const void* k_cache,
                              const float* k_scale,
                              const int32_t* block_table,
                              const int32_t* seq_lens, void* codes,
                              float* scales, void* stream) {
  return build_key_summary(shape, k_cache, k_scale, FD_DTYPE_INT8,
                           block_table, seq_lens, codes, scales, stream);
}

static int decode_attn_sparse(const fd_shape* shape, const void* q,
                              const void* k_cache, const void* v_cache,
                              const float* k_scale, const float* v_scale,
                              int scaled, const void* codes,
                              const float* scales, const int32_t* block_table,
                              const int32_t* seq_lens, float delta,
                              int num_splits, void* workspace,
                              size_t ws_bytes, float* out, float* lse_out,
                              uint8_t* kept_out, void* stream) {
  Shape s;
  int st = check_shape(shape, &s);
  if (st != FD_OK) return st;
  st = check_sparse_dtype(s, scaled);
  if (st != FD_OK) return st;
  if (s.G > kMaxSparseG) return FD_ERR_UNSUPPORTED;
  st = check_splits(s, num_splits);
  if (st != FD_OK) return st;
  const int64_t P = tokens_per_split(s, num_splits);
  if (P > kMaxSparseSplit ||
      P * (s.G > kHeadsPerGroup ? s.G : kHeadsPerGroup) > kMaxSparseEst)
    return FD_ERR_UNSUPPORTED;
  st = check_inputs(s, q, k_cache, v_cache, block_table, seq_lens);
  if (st != FD_OK) return st;
  st = check_scales(s, k_scale, v_scale, scaled);
  if (st != FD_OK) return st;
  if (!codes || !scales || !aligned16(codes) ||
      (reinterpret_cast<uintptr_t>(scales) & 3u) != 0)
    return FD_ERR_INVALID_ARG;
  if (isnan(delta) || delta < 0.f) return FD_ERR_INVALID_ARG;
  if (!out || !aligned16(out)) return FD_ERR_INVALID_ARG;
  if (lse_out && (reinterpret_cast<uintptr_t>(lse_out) & 3u) != 0)
    return FD_ERR_INVALID_ARG;
  if (num_splits > 1) {
    if (!workspace || ws_bytes < workspace_bytes(s, num_splits))
      return FD_ERR_WORKSPACE;
    if (!aligned16(workspace)) return FD_ERR_INVALID_ARG;
  }
  SplitArgs a = make_split_args(s, q, k_cache, v_cache, block_table, seq_lens,
                                num_splits);
  a.k_scale = scaled >= 0 ? k_scale : nullptr;
  a.v_scale = scaled >= 0 ? v_scale : nullptr;
  SparseArgs sp;
  sp.codes = static_cast<const uint8_t*>(codes);
  sp.scales = scales;
  sp.kept_out = kept_out;
  sp.delta_log2 = (float)((double)delta * 1.4426950408889634);
  sp.nblk_row = (int)(((int64_t)s.L + 15) / 16);
  float* o_part = static_cast<float*>(workspace);
  float* lse_part = nullptr;
  if (num_splits == 1) {
    a.o_dst = out;
    a.lse_dst = lse_out;
    a.final_out = 1;
    return launch_sparse(s, a, sp, stream) == 0 ? FD_OK : FD_ERR_HIP;
  }
  lse_part = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                      partial_o_bytes(s, num_splits));
  a.o_dst = o_part;
  a.lse_dst = lse_part;
  a.final_out = 0;
  if (launch_sparse(s, a, sp, stream) != 0) return FD_ERR_HIP;
  CombineArgs c;
  c.o_part = o_part;
  c.lse_part = lse_part;
  c.out = out;
  c.lse_out = lse_out;
  c.B = s.B;
  c.Hq = s.Hq;
  c.S = num_splits;
  return launch_combine(s.D, c, stream) == 0 ? FD_OK : FD_ERR_HIP;
}

int fd_decode_attn_sparse(const fd_shape* shape, const void* q,
                          const void* k_cache, const void* v_cache,
                          const void* codes, const float* scales,
                          const int32_t* block_table,
                          const int32_t* seq_lens, float delta,
                          int num_splits, void* workspace, size_t ws_bytes,
                          float* out, float* lse_out, uint8_t* kept_out,
                          void* stream) {
  return decode_attn_sparse(shape, q, k_cache, v_cache, nullptr, nullptr, -1,
                            codes, scales, block_table, seq_lens, delta,
                            num_splits, workspace, ws_bytes, out, lse_out,
                            kept_out, stream);
}

int fd_decode_attn_sparse_fp8(const fd_shape* shape, const void* q,
                              const void* k_cache, const void* v_cache,
                              const float* k_scale, const float* v_scale,
                              const void* codes, const float* scales,
                              const int32_t* block_table,
                              const int32_t* seq_lens, float delta,
                              int num_splits, void* workspace,
                              size_t ws_bytes, float* out, float* lse_out,
                              uint8_t* kept_out, void* stream) {
  return decode_attn_sparse(shape, q, k_cache, v_cache, k_scale, v_scale,
                            FD_DTYPE_FP8_E4M3, codes, scales, block_table,
                            seq_lens, delta, num_splits, workspace, ws_bytes,
                            out, lse_out, kept_out, stream);
}

int fd_decode_attn_sparse_int8(const fd_shape* shape, const void* q,
                               const void* k_cache, const void* v_cache,
                               const float* k_scale, const float* v_scale,
                               const void* codes, const float* scales,
                               const int32_t* block_table,
                               const int32_t* seq_lens, float delta,
                               int num_splits, void* workspace,
                               size_t ws_bytes, float* out, float* lse_out,
                               uint8_t* kept_out, void* stream) {
  return decode_attn_sparse(shape, q, k_cache, v_cache, k_scale, v_scale,
                            FD_DTYPE_INT8, codes, scales, block_table,
                            seq_lens, delta, num_splits, workspace, ws_bytes,
                            out, lse_out, kept_out, stream);
}

int fd_combine_partials(int batch, int num_q_heads, int head_dim,
                        int num_splits, const float* o_part,
                        const float* lse_part, float* out, float* lse_out,
                        void* stream) {
  if (batch < 1 || num_q_heads < 1 || num_splits < 1 ||
      num_splits > kMaxSplits)
    return FD_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return FD_ERR_UNSUPPORTED;
  if ((int64_t)batch * num_q_heads * 16 > INT32_MAX) return FD_ERR_UNSUPPORTED;
  if (!o_part || !lse_part || !out) return FD_ERR_INVALID_ARG;
  if (!aligned16(o_part) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(lse_part) & 3u) != 0 ||
      (lse_out && (reinterpret_cast<uintptr_t>(lse_out) & 3u) != 0))
    return FD_ERR_INVALID_ARG;
  CombineArgs c;
  c.o_part = o_part;
  c.lse_part = lse_part;
  c.out = out;
  c.lse_out = lse_out;
  c.B = batch;
  c.Hq = num_q_heads;
  c.S = num_splits;
  return launch_combine(head_dim, c, stream) == 0 ? FD_OK : FD_ERR_HIP;
}

}  // extern "C"
