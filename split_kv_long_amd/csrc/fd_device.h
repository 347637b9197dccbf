// Device-side helpers shared by the HIP kernels (vector types, base-2
// exp/log, cross-lane reductions, output addressing, the bf16 MFMA operand
// layout and cache loads). Included by the kernel sources only.
#ifndef FD_DEVICE_H
#define FD_DEVICE_H

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fd_internal.h"

namespace fd {

// Cache encodings of the MFMA kernels (dense and block-sparse).
enum : int { kCacheBf16 = 0, kCacheE4M3 = 1, kCacheI8 = 2 };

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.69314718055994531f;
constexpr float kLog2e = 1.44269504088896341f;

__device__ __forceinline__ float fexp2(float x) {
  return __builtin_amdgcn_exp2f(x);   // v_exp_f32; exp2(-inf) = 0
}
__device__ __forceinline__ float flog2(float x) {
  return __builtin_amdgcn_logf(x);    // v_log_f32
}

// Butterfly exchanges across lanes l ^ 16 and l ^ 32 with gfx950's
// v_permlane16_swap / v_permlane32_swap (plain VALU, no LDS round trip):
// with both operands equal to x, the two results hold x from each half, so
// combining them gives every lane the pair's reduction.
__device__ __forceinline__ float max_x16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x),
                                                  __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_x32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                                  __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_x16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x),
                                                  __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_x32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                                  __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Whole-wave max / sum on the VALU: DPP inside each 16-lane row (swap
// neighbours, swap pairs, rotate by 4, rotate by 8), then the row exchanges.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL,
                                                    0xF, 0xF, false));
}
__device__ __forceinline__ float wave_max_f(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x124>(v));
  v = fmaxf(v, dpp_f<0x128>(v));
  return max_x32(max_x16(v));
}
__device__ __forceinline__ float wave_sum_f(float v) {
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x124>(v);
  v += dpp_f<0x128>(v);
  return sum_x32(sum_x16(v));
}

__device__ __forceinline__ int clamp_len(const SplitArgs& a, int b) {
  int n = a.seq_lens[b];
  n = n < 0 ? 0 : n;
  return n > a.L ? a.L : n;
}

// Where head h's result for split s goes.
template <int D>
__device__ __forceinline__ float* o_dst(const SplitArgs& a, int b, int h, int s) {
  return a.final_out ? a.o_dst + ((size_t)b * a.Hq + h) * D
                     : a.o_dst + (((size_t)b * a.Hq + h) * a.S + s) * D;
}
__device__ __forceinline__ float* lse_dst(const SplitArgs& a, int b, int h, int s) {
  if (a.final_out)
    return a.lse_dst ? a.lse_dst + (size_t)b * a.Hq + h : nullptr;
  return a.lse_dst + ((size_t)b * a.Hq + h) * a.S + s;
}

// An empty split (or an empty history when final_out): o = 0, lse = -inf.
// Kept out of line so the hot path's code stays contiguous.
static __device__ __attribute__((noinline)) void write_empty_rows(
    float* o, size_t o_stride, float* lse, size_t lse_stride, int nh, int D) {
  for (int i = threadIdx.x; i < nh * D; i += blockDim.x) {
    const int g = i / D;
    o[g * o_stride + (i - g * D)] = 0.f;
  }
  if (lse)
    for (int g = threadIdx.x; g < nh; g += blockDim.x) lse[g * lse_stride] = -INFINITY;
}

template <int D>
__device__ __forceinline__ void write_empty(const SplitArgs& a, int b, int h0,
                                            int nh, int s) {
  write_empty_rows(o_dst<D>(a, b, h0, s), a.final_out ? D : (size_t)a.S * D,
                   lse_dst(a, b, h0, s), a.final_out ? 1 : (size_t)a.S, nh, D);
}

// Element offset of cache row t (t < the sequence's length) of (b, kvh).
template <int D>
__device__ __forceinline__ size_t row_offset(const SplitArgs& a, int b, int kvh,
                                             int t) {
  if (a.bs == 0) return ((size_t)(b * a.Hkv + kvh) * a.L + t) * D;
  const int page = t / a.bs;
  int blk = a.block_table[(size_t)b * a.max_blocks + page];
  blk = blk < 0 ? 0 : (blk >= a.num_blocks ? a.num_blocks - 1 : blk);
  return (((size_t)blk * a.Hkv + kvh) * a.bs + (t - page * a.bs)) * D;
}

template <int D>
struct MfmaCfg {
  static constexpr int KC = D / 32;   // QK calls per 16-token tile
  static constexpr int NV = D / 16;   // PV calls per subtile
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) {
  return __builtin_bit_cast(bf16x8, x);
}

template <int D>
__device__ __forceinline__ bf16x8 v_kvec(const u32x4 (&vr)[8], int cc, int n) {
  // k-vector for PV call cc: element e = element `idx` of vr[e].
  //   D = 128: lane's row n <-> dim 8n + cc, element cc of its 8-dim chunk.
  //   D = 64 : row n <-> dim 8(n&7) + 4(n>>3) + cc, element cc + 4(n>>3).
  const unsigned sel = (cc & 1) ? 0x07060302u : 0x05040100u;
  u32x4 r;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    unsigned lo, hi;
    if (D == 128) {
      lo = vr[2 * k][cc >> 1];
      hi = vr[2 * k + 1][cc >> 1];
    } else {
      const bool up = n >= 8;
      lo = up ? vr[2 * k][2 + (cc >> 1)] : vr[2 * k][cc >> 1];
      hi = up ? vr[2 * k + 1][2 + (cc >> 1)] : vr[2 * k + 1][cc >> 1];
    }
    r[k] = __builtin_amdgcn_perm(hi, lo, sel);
  }
  return as_bf16x8(r);
}

// Output dim of accumulator element (cc, i) in lane group j.
template <int D>
__device__ __forceinline__ int out_dim(int cc, int i, int j) {
  const int m = 4 * j + i;
  return D == 128 ? 8 * m + cc : 8 * (m & 7) + 4 * (m >> 3) + cc;
}

// 16- and 8-byte cache loads; NT marks them non-temporal (streamed once).
template <bool NT, typename T>
__device__ __forceinline__ u32x4 ld16(const T* p) {
  if (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return *reinterpret_cast<const u32x4*>(p);
}
template <bool NT, typename T>
__device__ __forceinline__ u32x2 ld8(const T* p) {
  if (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return *reinterpret_cast<const u32x2*>(p);
}

// Four 8-bit E4M3 codes (one dword, lowest byte first) -> four bf16, exact
// (every E4M3 value is a bf16 value), with gfx950's packed conversion.
__device__ __forceinline__ uint2 e4m3x4_to_bf16x4(unsigned w) {
  const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  return uint2{__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
}

// Four 8-bit two's-complement integers (one dword, lowest byte first) ->
// four bf16, exact: each byte converts to fp32 with sign extension (one
// instruction per byte), and an integer of magnitude <= 128 has at most 8
// significant bits, so the fp32's low 16 bits are zero and its high half is
// the bf16 value; a byte permute gathers the two high halves.
__device__ __forceinline__ uint2 s8x4_to_bf16x4(unsigned w) {
  const float f0 = (float)(int8_t)w, f1 = (float)(int8_t)(w >> 8);
  const float f2 = (float)(int8_t)(w >> 16), f3 = (float)(int8_t)(w >> 24);
  return uint2{__builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0),
                                     0x07060302u),
               __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2),
                                     0x07060302u)};
}

}  // namespace fd

#endif  // FD_DEVICE_H
