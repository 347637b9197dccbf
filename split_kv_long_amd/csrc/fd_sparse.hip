// Block-sparse decode over a 4-bit key summary, for gfx950.
//
// After the abstract of "Faster Than Flash: Exploiting Attention Sparsity
// for Efficient Long-Context Decoding": a low-bit quantized copy of the keys
// is scanned to estimate which blocks of the history matter, a top-delta rule
// keeps the blocks whose estimated best logit comes within delta of the
// best one (decided inside each split, so no workgroup waits on another),
// and exact attention runs over the kept blocks only. The partials then go
// through the ordinary log-sum-exp combine.
//
// Kernels:
//   summary_kernel<D, QM>
//                       bf16 keys (or 8-bit codes times their scale -- per
//                       kv head for E4M3, per position for int8 -- rounded
//                       once to fp32)
//                       -> 4-bit codes (two per byte, even dim in
//                       the low nibble) + one fp32 scale per 16-token block
//                       and kv head: scale = amax / 7, code =
//                       rint(k * (7 / amax)). A block's codes form one
//                       16 * D/2-byte record, stored in the order the scan's
//                       MFMA operands need: bytes D/8 * (n + 16 p) ..
//                       + D/8 - 1 hold piece p (dims D/4 * p ..) of row n, so
//                       every lane's request is contiguous with its
//                       neighbours'.
//   split_sparse<D, NW, GM, PAGED, CHUNK, MULTI, QM>
//                       one workgroup per (split, kv head, sequence):
//                       phase 1 scans the split's summary blocks (8-bit
//                       query x 4-bit codes, exact, on the int8 matrix
//                       cores), phase 2 keeps blocks per top-delta, phase 3
//                       runs exact attention over the kept blocks (bf16
//                       products; an 8-bit cache's codes are converted to
//                       bf16 in registers, exactly, and its scales applied
//                       as in the dense kernel).
//                       A kv head with more than GM query heads is served
//                       GM heads at a time in phases 1 and 3 (the keep
//                       decision in phase 2 needs every head's estimates).

#include <hip/hip_runtime.h>
#include <math.h>
#include <limits.h>
#include <stdint.h>

#include <type_traits>

#include "fd_device.h"
#include "fd_internal.h"

namespace fd {
namespace {

constexpr int kSumBlock = 16;   // tokens per summary block

// ----------------------------------------------------------------------------
// Key summary.

// One wave per (16-token block, kv head, sequence). Lane l takes row l / 4
// of the block and the quarter l % 4 of its dims. Blocks with no attended
// token are skipped; rows past the length (all 16 rows of a record exist)
// get code 0.
template <int D, int QM>
__global__ __launch_bounds__(64) void summary_kernel(SummaryArgs a) {
  constexpr int QD = D / 4;                  // dims per lane
  const int lane = threadIdx.x;
  const int blk = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  int len = a.seq_lens[b];
  len = len < 0 ? 0 : (len > a.L ? a.L : len);
  const int t0 = blk * kSumBlock;
  if (t0 >= len) return;
  const int r = lane >> 2, part = lane & 3;
  const int t = t0 + r;
  const bool valid = t < len;
  // Block index: the record and scale slot of this (block, kv head).
  size_t bi;
  int page = 0, pb = 0;
  if (a.bs == 0) {
    bi = (size_t)(b * a.Hkv + kvh) * a.nblk_row + blk;
  } else {
    page = t0 / a.bs;
    pb = a.block_table[(size_t)b * a.max_blocks + page];
    pb = pb < 0 ? 0 : (pb >= a.num_blocks ? a.num_blocks - 1 : pb);
    bi = ((size_t)pb * a.Hkv + kvh) * (a.bs / kSumBlock) +
         (t0 - page * a.bs) / kSumBlock;
  }
  size_t row = 0;                            // element offset of row t in K
  if (valid) {
    row = a.bs == 0 ? ((size_t)(b * a.Hkv + kvh) * a.L + t)
                    : ((size_t)pb * a.Hkv + kvh) * a.bs + (t - page * a.bs);
  }
  float x[QD];
  float amax = 0.f;
  if (valid && QM != kCacheBf16) {
    // 8-bit codes -> bf16 (exact) -> fp32, times the scale (one fp32
    // rounding): the kv head's for E4M3, the row's for int8 (rows of a
    // contiguous cache's scales are padded to whole 16-position groups; a
    // paged pool's scales are indexed like its rows).
    const uint8_t* kp = static_cast<const uint8_t*>(a.k) + row * D + part * QD;
    const size_t Lp = ((size_t)a.L + 15) & ~(size_t)15;
    const float ks =
        QM == kCacheE4M3 ? a.k_scale[kvh]
                         : a.k_scale[a.bs == 0 ? (size_t)(b * a.Hkv + kvh) * Lp + t
                                               : row];
#pragma unroll
    for (int c = 0; c < QD / 16; ++c) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(kp + 16 * c);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint2 p = QM == kCacheI8 ? s8x4_to_bf16x4(w[e])
                                       : e4m3x4_to_bf16x4(w[e]);
        x[16 * c + 4 * e] = __uint_as_float(p.x << 16) * ks;
        x[16 * c + 4 * e + 1] = __uint_as_float(p.x & 0xffff0000u) * ks;
        x[16 * c + 4 * e + 2] = __uint_as_float(p.y << 16) * ks;
        x[16 * c + 4 * e + 3] = __uint_as_float(p.y & 0xffff0000u) * ks;
      }
    }
#pragma unroll
    for (int i = 0; i < QD; ++i) amax = fmaxf(amax, fabsf(x[i]));
  } else if (valid) {
    const uint16_t* kp = static_cast<const uint16_t*>(a.k) + row * D + part * QD;
#pragma unroll
    for (int c = 0; c < QD / 8; ++c) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(kp + 8 * c);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[8 * c + 2 * e] = __uint_as_float(w[e] << 16);
        x[8 * c + 2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
      }
    }
#pragma unroll
    for (int i = 0; i < QD; ++i) amax = fmaxf(amax, fabsf(x[i]));
  } else {
#pragma unroll
    for (int i = 0; i < QD; ++i) x[i] = 0.f;
  }
  amax = wave_max_f(amax);                   // DPP and lane swaps, no LDS
  // Correctly rounded fp32 quotients (HIP's default division).
  const float inv = amax > 0.f ? 7.0f / amax : 0.f;
  const float scale = amax > 0.f ? amax / 7.0f : 0.f;
  {
    unsigned packed[QD / 8];
#pragma unroll
    for (int wd = 0; wd < QD / 8; ++wd) {
      unsigned v = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = (int)__builtin_rintf(x[8 * wd + e] * inv);
        v |= ((unsigned)c & 0xFu) << (4 * e);
      }
      packed[wd] = v;
    }
    uint8_t* cp = a.codes + bi * (kSumBlock * D / 2) + (QD / 2) * (r + 16 * part);
    if (QD == 32)
      *reinterpret_cast<u32x4*>(cp) = u32x4{packed[0], packed[1], packed[2], packed[3]};
    else
      *reinterpret_cast<u32x2*>(cp) = u32x2{packed[0], packed[1]};
  }
  if (lane == 0) a.scales[bi] = scale;
}

// ----------------------------------------------------------------------------
// Sparse split kernel.

constexpr int kMaxSparseBlocks = kMaxSparseSplit / kSumBlock;
// Estimates held in LDS: blocks per split x query heads per kv head (the
// host bounds tokens per split x heads per kv head accordingly).
constexpr int kMaxSparseEstimates = kMaxSparseEst / kSumBlock;

// Lane layout as in the dense MFMA kernel (lane l: n = l % 16, j = l / 16;
// S^T = K * Q^T so a lane holds one head n and tokens 4j..4j+3 of a 16-token
// tile). Scan: lane group j covers the code dims [32j, 32j + 32) at
// D = 128 ([16j, 16j + 16) at D = 64), 64 dims per int8 MFMA call; the
// query bytes of each lane follow the order its code bytes arrive in, and
// since every (lane group, byte) pair names one k-slot of the product for
// both operands alike, the sum runs over every dim exactly once.
template <int D, int NW, int GM, bool PAGED, int CHUNK, bool MULTI, int QM>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
void split_sparse(SplitArgs a, SparseArgs sp) {
  constexpr bool F8 = QM != kCacheBf16;        // one byte per element
  constexpr bool I8 = QM == kCacheI8;
  constexpr int KC = D / 32;
  constexpr int NV = D / 16;
  constexpr int DP = D + 4;
  constexpr int CB = D / 8;                    // code bytes per lane per row
  constexpr int HMAX = MULTI ? kMaxSparseG : GM;   // heads per kv head
  __shared__ float est_s[MULTI ? kMaxSparseEstimates
                               : kMaxSparseBlocks * GM];  // [block][head]
  __shared__ float wmax_s[NW][HMAX];
  __shared__ float thr_s[HMAX];                // per-head keep threshold
  __shared__ int cnt_s[NW];                    // kept blocks per wave slice
  __shared__ int16_t list_s[kMaxSparseBlocks]; // kept blocks, ascending
  static_assert(NW * 64 >= kMaxSparseBlocks, "one block per thread");
  __shared__ float mo[NW][GM][DP];
  __shared__ float mm[NW][GM], ml[NW][GM];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, j = lane >> 4;
  const int s = blockIdx.z, b = blockIdx.y;
  const int kvh = blockIdx.x;                  // one head group per kv head
  const int G = a.G, Hkv = a.Hkv, L = a.L, bs = a.bs;
  const int h0 = kvh * G;
  const int nh = G;
  const int nhg = MULTI ? (G + GM - 1) / GM : 1;   // passes of GM heads
  const int lo = s * a.P;
  int len = a.seq_lens[b];
  len = len < 0 ? 0 : (len > L ? L : len);
  const int hi = min(lo + a.P, len);
  if (lo >= hi) {
    write_empty<D>(a, b, h0, nh, s);
    return;
  }
  const int nb = (hi - lo + kSumBlock - 1) / kSumBlock;   // blocks here
  const int jg0 = lo / kSumBlock;
  using KT = typename std::conditional<F8, uint8_t, uint16_t>::type;
  const KT* K = static_cast<const KT*>(a.k);
  const KT* V = static_cast<const KT*>(a.v);
  const uint16_t* Q = static_cast<const uint16_t*>(a.q);

  // Row index (not yet times D) of token t of (b, kvh).
  auto row_of = [&](int t) -> size_t {
    if (!PAGED) return (size_t)(b * Hkv + kvh) * L + t;
    const int page = t / bs;
    int pb = __builtin_amdgcn_readfirstlane(
        a.block_table[(size_t)b * a.max_blocks + page]);
    pb = pb < 0 ? 0 : (pb >= a.num_blocks ? a.num_blocks - 1 : pb);
    return ((size_t)pb * Hkv + kvh) * bs + (t - page * bs);
  };
  auto scale_index = [&](int t) -> size_t {   // t = a block's first token
    if (!PAGED) return (size_t)(b * Hkv + kvh) * sp.nblk_row + t / kSumBlock;
    const int page = t / bs;
    int pb = __builtin_amdgcn_readfirstlane(
        a.block_table[(size_t)b * a.max_blocks + page]);
    pb = pb < 0 ? 0 : (pb >= a.num_blocks ? a.num_blocks - 1 : pb);
    return ((size_t)pb * Hkv + kvh) * (bs / kSumBlock) +
           (t - page * bs) / kSumBlock;
  };

  // Query row of lane column n in the pass over heads hb .. hb + GM - 1;
  // padded columns reuse the pass's first head.
  auto q_row = [&](int hb, int ng) -> const uint16_t* {
    const int qh = h0 + hb + (n < ng ? n : 0);
    return Q + ((size_t)b * a.Hq + qh) * D;
  };

  // ---- phase 1: scan the summary -----------------------------------------
  // The query is rounded to 8 bits per head (q8 = rint(q * 127 / amax_q));
  // the int8 matrix cores then give every token's sum_d q8 * code exactly,
  // and the block estimate is ((float(max dot) * s_q) * scale_blk) *
  // scale_log2, the same float32 operations in the same order as the
  // reference, so every keep decision is reproduced exactly.
  for (int hg = 0; hg < nhg; ++hg) {
    const int hb = hg * GM, ng = min(GM, G - hb);
    const uint16_t* qrow = q_row(hb, ng);
    constexpr int SD = D / 4;                  // scan dims per lane group
    constexpr int NG = SD / 8;                 // 8-dim groups per lane
    constexpr int KM = D / 64;                 // int8 MFMA calls per tile
    // Lane (n, j): head n's dims [SD j, SD j + SD). Codes arrive as nibbles
    // (dim 8m + e in nibble e of dword m); after unpacking, a dword's 8
    // values sit as dims (0, 2, 4, 6) then (1, 3, 5, 7), and the query
    // bytes are laid out in that same order.
    float qv[SD];
#pragma unroll
    for (int c = 0; c < SD / 8; ++c) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(qrow + SD * j + 8 * c);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qv[8 * c + 2 * e] = __uint_as_float(v[e] << 16);
        qv[8 * c + 2 * e + 1] = __uint_as_float(v[e] & 0xffff0000u);
      }
    }
    float qmax = 0.f;
#pragma unroll
    for (int i = 0; i < SD; ++i) qmax = fmaxf(qmax, fabsf(qv[i]));
    qmax = max_x32(max_x16(qmax));             // head n's max |q|
    // Correctly rounded fp32 quotients (HIP's default division).
    const float inv_q = qmax > 0.f ? 127.0f / qmax : 0.f;
    const float s_q = qmax > 0.f ? qmax / 127.0f : 0.f;
    unsigned q8w[2 * NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      int qi[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        qi[e] = (int)__builtin_rintf(qv[8 * g + e] * inv_q);
      }
      q8w[2 * g] = (qi[0] & 0xFF) | ((qi[2] & 0xFF) << 8) |
                   ((qi[4] & 0xFF) << 16) | ((unsigned)(qi[6] & 0xFF) << 24);
      q8w[2 * g + 1] = (qi[1] & 0xFF) | ((qi[3] & 0xFF) << 8) |
                       ((qi[5] & 0xFF) << 16) | ((unsigned)(qi[7] & 0xFF) << 24);
    }
    i32x4 qb[KM];
#pragma unroll
    for (int c = 0; c < KM; ++c)
      qb[c] = i32x4{(int)q8w[4 * c], (int)q8w[4 * c + 1], (int)q8w[4 * c + 2],
                    (int)q8w[4 * c + 3]};
    float wmax = -INFINITY;
    // A wave's blocks go CHUNK at a time: every code and scale request of a
    // chunk is issued before the first product, and the next chunk is
    // requested as soon as the current one is in registers (two register
    // sets, used in turn; the empty asm statements make the compiler wait
    // for exactly those loads there).
    using CT = typename std::conditional<D == 128, u32x4, u32x2>::type;
    auto load_chunk = [&](int jl0, CT (&cw)[CHUNK], float (&bscale)[CHUNK],
                          int (&lastr)[CHUNK]) {
#pragma unroll
      for (int u = 0; u < CHUNK; ++u) {
        const int jl = min(jl0 + NW * u, nb - 1);   // clamped: inside the split
        const int t0 = lo + jl * kSumBlock;
        lastr[u] = min(kSumBlock, hi - t0) - 1;
        const size_t bi = scale_index(t0);    // record = scale slot
        bscale[u] = sp.scales[bi];
        // Streamed once per call, like K and V: non-temporal.
        cw[u] = __builtin_nontemporal_load(reinterpret_cast<const CT*>(
            sp.codes + bi * (kSumBlock * D / 2) + CB * lane));
      }
    };
    auto scan_chunk = [&](int jl0, const CT (&cw)[CHUNK],
                          const float (&bscale)[CHUNK],
                          const int (&lastr)[CHUNK]) {
#pragma unroll
      for (int u = 0; u < CHUNK; ++u) {
        const int jl = jl0 + NW * u;
        if (jl >= nb) break;
        // A 4-bit two's complement code moved into the high nibble of a
        // byte (low nibble zero) is the signed byte 16 * code, so the
        // products are 16 * sum_d q8 * code with no offset to remove:
        // even dims from the low nibbles shifted up, odd dims masked.
        i32x4 acc = i32x4{0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < KM; ++c) {
          const unsigned x0 = cw[u][2 * c], x1 = cw[u][2 * c + 1];
          const i32x4 ca = i32x4{(int)((x0 << 4) & 0xF0F0F0F0u),
                                 (int)(x0 & 0xF0F0F0F0u),
                                 (int)((x1 << 4) & 0xF0F0F0F0u),
                                 (int)(x1 & 0xF0F0F0F0u)};
          acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(ca, qb[c], acc, 0, 0, 0);
        }
        int dm;
        if (lastr[u] == kSumBlock - 1) {      // full block (wave-uniform)
          dm = max(max(acc[0], acc[1]), max(acc[2], acc[3]));
        } else {
          dm = INT_MIN;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (4 * j + i <= lastr[u]) dm = max(dm, acc[i]);
        }
        {
          const auto r16 = __builtin_amdgcn_permlane16_swap(
              (unsigned)dm, (unsigned)dm, false, false);
          dm = max((int)r16[0], (int)r16[1]);
          const auto r32 = __builtin_amdgcn_permlane32_swap(
              (unsigned)dm, (unsigned)dm, false, false);
          dm = max((int)r32[0], (int)r32[1]);
        }
        float e = (float)(dm >> 4) * s_q;      // block max, reference order
        e = e * bscale[u];
        e = e * a.scale_log2;                  // base-2 logit units
        if (j == 0 && n < ng) est_s[jl * G + hb + n] = e;
        wmax = fmaxf(wmax, e);
      }
    };
    CT cwA[CHUNK], cwB[CHUNK];
    float bsA[CHUNK], bsB[CHUNK];
    int lrA[CHUNK], lrB[CHUNK];
    int jl0 = w;
    if (jl0 < nb) load_chunk(jl0, cwA, bsA, lrA);
    while (jl0 < nb) {
#pragma unroll
      for (int u = 0; u < CHUNK; ++u) asm volatile("" ::"v"(cwA[u]));
      __builtin_amdgcn_sched_barrier(0);
      int jn = jl0 + NW * CHUNK;
      if (jn < nb) load_chunk(jn, cwB, bsB, lrB);
      __builtin_amdgcn_sched_barrier(0);
      scan_chunk(jl0, cwA, bsA, lrA);
      jl0 = jn;
      if (jl0 >= nb) break;
#pragma unroll
      for (int u = 0; u < CHUNK; ++u) asm volatile("" ::"v"(cwB[u]));
      __builtin_amdgcn_sched_barrier(0);
      jn = jl0 + NW * CHUNK;
      if (jn < nb) load_chunk(jn, cwA, bsA, lrA);
      __builtin_amdgcn_sched_barrier(0);
      scan_chunk(jl0, cwB, bsB, lrB);
      jl0 = jn;
    }
    if (j == 0 && n < ng) wmax_s[w][hb + n] = wmax;
  }
  __syncthreads();

  // ---- phase 2: top-delta inside the split --------------------------------
  // Thread t decides block t (a split has at most NW * 64 blocks) and the
  // kept blocks are compacted, in ascending order, into list_s.
  if ((int)threadIdx.x < G) {
    const int h = threadIdx.x;
    float M = wmax_s[0][h];
#pragma unroll
    for (int ww = 1; ww < NW; ++ww) M = fmaxf(M, wmax_s[ww][h]);
    thr_s[h] = M - sp.delta_log2;
  }
  __syncthreads();
  int nkept;
  {
    const int jl = threadIdx.x;
    bool keep = false;
    if (jl < nb) {
      for (int h = 0; h < nh; ++h) keep |= est_s[jl * G + h] >= thr_s[h];
      if (sp.kept_out)
        sp.kept_out[(size_t)(b * Hkv + kvh) * sp.nblk_row + jg0 + jl] =
            keep ? 1 : 0;
    }
    const uint64_t mask = __builtin_amdgcn_ballot_w64(keep);
    if (lane == 0) cnt_s[w] = __builtin_popcountll(mask);
    __syncthreads();
    int base = 0;
    nkept = 0;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const int c = cnt_s[ww];
      base += ww < w ? c : 0;
      nkept += c;
    }
    if (keep) {
      const uint64_t below = mask & ((1ull << lane) - 1ull);
      list_s[base + __builtin_popcountll(below)] = (int16_t)jl;
    }
    nkept = __builtin_amdgcn_readfirstlane(nkept);
  }
  __syncthreads();

  // ---- phase 3: exact attention over the kept blocks ----------------------
  // bf16: lane (n, j) requests 16 bytes of key row n at dims 32c + 8j. E4M3
  // (as in the dense kernel): 16 codes at dims 64c' + 16j, which feed two
  // products (dims 64c' + 16j and + 8), and 8 value codes per row; the
  // query fragments follow the same dim order. An E4M3 key scale joins the
  // logit scale and its value scale the final normalisation; int8 scales
  // are per position: a lane requests the key and value scales of its rows
  // 4j..4j+3 of each block (one 16-byte request each), the key scale
  // multiplies the score and the value scale the probability entering the
  // PV product (the softmax sum takes the unscaled one), and masked rows
  // get a zero value scale, so a NaN scale of an unattended slot stays out.
  constexpr int KL = F8 ? D / 64 : KC;         // 16-byte key requests per row
  const float sl2 =
      QM == kCacheE4M3 ? a.scale_log2 * a.k_scale[kvh] : a.scale_log2;
  const float vsc = QM == kCacheE4M3 ? a.v_scale[kvh] : 1.f;
  const size_t Lp = ((size_t)L + 15) & ~(size_t)15;   // L may be INT32_MAX
  auto cvt4 = [](unsigned x) -> uint2 {
    if constexpr (I8) return s8x4_to_bf16x4(x);
    else return e4m3x4_to_bf16x4(x);
  };
  for (int hg = 0; hg < nhg; ++hg) {
    const int hb = hg * GM, ng = min(GM, G - hb);
    const uint16_t* qrow = q_row(hb, ng);
    bf16x8 qf[KC];
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const int d0 = F8 ? 16 * j + 64 * (c >> 1) + 8 * (c & 1) : 8 * j + 32 * c;
      qf[c] = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow + d0));
    }
    f32x4 o[NV];
#pragma unroll
    for (int cc = 0; cc < NV; ++cc) o[cc] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    // Wave w takes kept blocks 2w, 2w + 1, then 2(w + NW), ... in pairs.
    for (int k = 2 * w; k < nkept; k += 2 * NW) {
      const int ja = __builtin_amdgcn_readfirstlane((int)list_s[k]);
      const int jb = k + 1 < nkept                // -1: second half masked
                         ? __builtin_amdgcn_readfirstlane((int)list_s[k + 1])
                         : -1;
      const int ta = lo + ja * kSumBlock;
      const int tb = jb >= 0 ? lo + jb * kSumBlock : ta;
      const int lasta = min(kSumBlock, hi - ta) - 1;
      const int lastb = jb >= 0 ? min(kSumBlock, hi - tb) - 1 : lasta;
      const size_t ra = row_of(ta), rb = row_of(tb);
      // Rows of a page block are consecutive (16 | page size).
      const KT* K0 = K + ra * D;
      const KT* K1 = K + rb * D;
      const KT* V0 = V + ra * D;
      const KT* V1 = V + rb * D;
      using VT = typename std::conditional<F8, u32x2, u32x4>::type;
      u32x4 kr[2][KL];
      VT vraw[8];
      constexpr int KJ = F8 ? 16 : 8, KS = F8 ? 64 : 32;
      const unsigned r0 = (unsigned)(min(n, lasta) * D + KJ * j);
      const unsigned r1 = (unsigned)(min(n, lastb) * D + KJ * j);
#pragma unroll
      for (int c = 0; c < KL; ++c) {
        kr[0][c] = ld16<true>(K0 + r0 + KS * c);
        kr[1][c] = ld16<true>(K1 + r1 + KS * c);
      }
      f32x4 k_sc[2], v_sc[2];
      if constexpr (I8) {
        const size_t sa = (PAGED ? ra : (size_t)(b * Hkv + kvh) * Lp + ta) + 4 * j;
        const size_t sb = (PAGED ? rb : (size_t)(b * Hkv + kvh) * Lp + tb) + 4 * j;
        k_sc[0] = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4*>(a.k_scale + sa));
        k_sc[1] = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4*>(a.k_scale + sb));
        v_sc[0] = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4*>(a.v_scale + sa));
        v_sc[1] = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4*>(a.v_scale + sb));
      }
      const int vcol = D == 128 ? 8 * n : 8 * (n & 7);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const unsigned va = (unsigned)(min(4 * j + e, lasta) * D + vcol);
        const unsigned vb = (unsigned)(min(4 * j + e, lastb) * D + vcol);
        if constexpr (F8) {
          vraw[e] = ld8<true>(V0 + va);
          vraw[4 + e] = ld8<true>(V1 + vb);
        } else {
          vraw[e] = ld16<true>(V0 + va);
          vraw[4 + e] = ld16<true>(V1 + vb);
        }
      }
      f32x4 sacc[2];
#pragma unroll
      for (int tg = 0; tg < 2; ++tg) {
        sacc[tg] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          bf16x8 kop;
          if constexpr (F8) {
            const u32x4 x = kr[tg][c >> 1];
            const uint2 p = cvt4(x[2 * (c & 1)]);
            const uint2 q = cvt4(x[2 * (c & 1) + 1]);
            kop = as_bf16x8(u32x4{p.x, p.y, q.x, q.y});
          } else {
            kop = as_bf16x8(kr[tg][c]);
          }
          sacc[tg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qf[c],
                                                             sacc[tg], 0, 0, 0);
        }
      }
      float sv[8];
      float mx = -INFINITY;
#pragma unroll
      for (int tg = 0; tg < 2; ++tg)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * j + i;
          const bool ok = tg == 0 ? r <= lasta : (jb >= 0 && r <= lastb);
          const float ls = I8 ? sl2 * k_sc[tg][i] : sl2;
          const float x = ok ? sacc[tg][i] * ls : -INFINITY;
          sv[4 * tg + i] = x;
          mx = fmaxf(mx, x);
          if constexpr (I8) v_sc[tg][i] = ok ? v_sc[tg][i] : 0.f;
        }
      mx = max_x32(max_x16(mx));
      const float mn = fmaxf(m_run, mx);
      const float alpha = fexp2(m_run - mn);     // m_run = -inf: 0
      m_run = mn;
      bf16x8 ph, pl;
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = fexp2(sv[e] - mn);
        psum += p;
        const float pw = I8 ? p * v_sc[e >> 2][e & 3] : p;   // value row e
        const __bf16 hb = (__bf16)pw;
        ph[e] = hb;
        pl[e] = (__bf16)(pw - (float)hb);
      }
      l_run = l_run * alpha + psum;
      u32x4 vr[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if constexpr (F8) {
          const uint2 p = cvt4(vraw[e][0]);
          const uint2 q = cvt4(vraw[e][1]);
          vr[e] = u32x4{p.x, p.y, q.x, q.y};
        } else {
          vr[e] = vraw[e];
        }
      }
#pragma unroll
      for (int cc = 0; cc < NV; ++cc) {
        o[cc] *= alpha;
        const bf16x8 vk = v_kvec<D>(vr, cc, n);
        o[cc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vk, ph, o[cc], 0, 0, 0);
        o[cc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vk, pl, o[cc], 0, 0, 0);
      }
    }

    // ---- merge the waves (as in the dense kernel) ---------------------------
    l_run = sum_x32(sum_x16(l_run));
    if (n < ng) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float* rowp = &mo[w][n][out_dim<D>(0, i, j)];
        *reinterpret_cast<f32x4*>(rowp) = f32x4{o[0][i], o[1][i], o[2][i], o[3][i]};
        if (D == 128)
          *reinterpret_cast<f32x4*>(rowp + 4) = f32x4{o[4][i], o[5][i], o[6][i], o[7][i]};
      }
      if (j == 0) {
        mm[w][n] = m_run;
        ml[w][n] = l_run;
      }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < ng * (D / 4); idx += NW * 64) {
      const int g = idx / (D / 4);
      const int d = 4 * (idx - g * (D / 4));
      // As in the dense kernel: every LDS read at once, hardware reciprocal.
      float mw[NW], lw[NW];
      f32x4 ow[NW];
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        mw[ww] = mm[ww][g];
        lw[ww] = ml[ww][g];
        ow[ww] = *reinterpret_cast<const f32x4*>(&mo[ww][g][d]);
      }
      float Mx = mw[0];
#pragma unroll
      for (int ww = 1; ww < NW; ++ww) Mx = fmaxf(Mx, mw[ww]);
      const float Ms = Mx == -INFINITY ? 0.f : Mx;
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      float lsum = 0.f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) {
        const float wt = fexp2(mw[ww] - Ms);
        acc += wt * ow[ww];
        lsum += wt * lw[ww];
      }
      const bool none = Mx == -INFINITY;
      const f32x4 res = acc * (vsc * __builtin_amdgcn_rcpf(lsum));
      *reinterpret_cast<f32x4*>(o_dst<D>(a, b, h0 + hb + g, s) + d) =
          none ? f32x4{0.f, 0.f, 0.f, 0.f} : res;
      if (d == 0) {
        float* l = lse_dst(a, b, h0 + hb + g, s);
        if (l) *l = none ? -INFINITY : (Mx + flog2(lsum)) * kLn2;
      }
    }
    if (hg + 1 < nhg) __syncthreads();       // mo is reused by the next pass
  }
}

// Blocks a wave requests per scan round: 8 for splits of 2048 tokens or
// more (256K, cold summary: 35.3 -> 33.2 us), else 4 (a 512-token split
// gives each wave only 4 blocks; 8 measured 3 % slower at 64K).
// MULTI: more than GM query heads per kv head (served GM at a time).
template <int D, int GM, bool PAGED, bool MULTI, int QM>
void launch_sparse_gm(const Shape& s, const SplitArgs& a, const SparseArgs& sp,
                      hipStream_t st) {
  const dim3 grid((unsigned)s.Hkv, (unsigned)s.B, (unsigned)a.S);
  if (a.P >= 2048)
    hipLaunchKernelGGL((split_sparse<D, 8, GM, PAGED, 8, MULTI, QM>), grid,
                       dim3(8 * 64), 0, st, a, sp);
  else
    hipLaunchKernelGGL((split_sparse<D, 8, GM, PAGED, 4, MULTI, QM>), grid,
                       dim3(8 * 64), 0, st, a, sp);
}

template <int D, bool PAGED, int QM>
void launch_sparse_d(const Shape& s, const SplitArgs& a, const SparseArgs& sp,
                     hipStream_t st) {
  if (s.G <= 8)
    launch_sparse_gm<D, 8, PAGED, false, QM>(s, a, sp, st);
  else if (s.G <= 16)
    launch_sparse_gm<D, 16, PAGED, false, QM>(s, a, sp, st);
  else
    launch_sparse_gm<D, 16, PAGED, true, QM>(s, a, sp, st);
}

template <int QM>
void launch_sparse_dtype(const Shape& s, const SplitArgs& a,
                         const SparseArgs& sp, hipStream_t st) {
  const bool paged = s.bs > 0;
  if (s.D == 128) {
    if (paged) launch_sparse_d<128, true, QM>(s, a, sp, st);
    else launch_sparse_d<128, false, QM>(s, a, sp, st);
  } else {
    if (paged) launch_sparse_d<64, true, QM>(s, a, sp, st);
    else launch_sparse_d<64, false, QM>(s, a, sp, st);
  }
}

}  // namespace

int launch_summary(const Shape& s, const SummaryArgs& a, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  // a.nblk_row = ceil(L / 16), formed in 64 bits by the host (L may be
  // INT32_MAX)
  const dim3 grid((unsigned)a.nblk_row, (unsigned)s.Hkv, (unsigned)s.B);
  if (grid.x == 0) return 0;
  const dim3 blk(64);
  if (s.D == 128) {
    if (s.dtype == FD_DTYPE_FP8_E4M3)
      hipLaunchKernelGGL((summary_kernel<128, kCacheE4M3>), grid, blk, 0, st, a);
    else if (s.dtype == FD_DTYPE_INT8)
      hipLaunchKernelGGL((summary_kernel<128, kCacheI8>), grid, blk, 0, st, a);
    else
      hipLaunchKernelGGL((summary_kernel<128, kCacheBf16>), grid, blk, 0, st, a);
  } else {
    if (s.dtype == FD_DTYPE_FP8_E4M3)
      hipLaunchKernelGGL((summary_kernel<64, kCacheE4M3>), grid, blk, 0, st, a);
    else if (s.dtype == FD_DTYPE_INT8)
      hipLaunchKernelGGL((summary_kernel<64, kCacheI8>), grid, blk, 0, st, a);
    else
      hipLaunchKernelGGL((summary_kernel<64, kCacheBf16>), grid, blk, 0, st, a);
  }
  return (int)hipGetLastError();
}

int launch_sparse(const Shape& s, const SplitArgs& a, const SparseArgs& sp,
                  void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (s.dtype == FD_DTYPE_FP8_E4M3)
    launch_sparse_dtype<kCacheE4M3>(s, a, sp, st);
  else if (s.dtype == FD_DTYPE_INT8)
    launch_sparse_dtype<kCacheI8>(s, a, sp, st);
  else
    launch_sparse_dtype<kCacheBf16>(s, a, sp, st);
  return (int)hipGetLastError();
}

}  // namespace fd
