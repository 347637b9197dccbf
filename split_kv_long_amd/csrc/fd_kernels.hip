// Split-KV decode attention kernels for gfx950 (CDNA4, wave64).
//
// The method (slavadubrov.com, "What is Flash-Decoding", section "Why decode
// needs a different schedule"): the cached history of each sequence is cut
// into splits, separate workgroups process the splits in parallel, each
// emits a partial output with its log-sum-exp, and a reduction combines the
// partials into exact softmax attention over the whole history. Inside a
// split the scores are streamed with a running maximum and normaliser (the
// online softmax named in the last abstract of the INT-FlashAttention related
// list), so one pass over K and V suffices.
//
// Kernels:
//   split_mfma<D, NW, GM, PAGED, SPEC, QM, BAL, PIPE>
//                        bf16, 8-bit E4M3 or int8 K/V (QM), head_dim
//                        64/128. One
//                        workgroup per (split, kv head x group of <= GM
//                        query heads, sequence); NW waves share the split,
//                        each streaming 32-token subtiles one at a time
//                        straight from HBM into registers, and the GQA
//                        group's QK^T and PV tile products run on the
//                        16x16x32 bf16 matrix cores. SPEC: batch one, first
//                        requests before the length is known. BAL: batched
//                        calls, length-aware pieces instead of uniform
//                        splits. PIPE: the reissue-on-arrival schedule
//                        (always for bf16; for E4M3 on long splits of one
//                        sequence).
//   split_f32<D>         fp32 caches: LDS-tiled, plain fp32 FMA, exact fp32
//                        products.
//   combine_kernel<D>    log-sum-exp reduction of the split partials.
// The block-sparse kernels live in fd_sparse.hip.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "fd_device.h"
#include "fd_internal.h"

namespace fd {
namespace {

// ----------------------------------------------------------------------------
// fp32 split kernel (LDS-tiled, plain fp32 FMA).

constexpr int kGenThreads = 256;

// One workgroup per (split, kv head, group of <= 16 query heads, sequence).
// A tile is 16 KB of K and 16 KB of V (64 tokens at D = 64, 32 at D = 128):
// each thread requests its four 16-byte pieces of each at once, the next
// tile's requests go out while the current one is computed, and rows past
// the split's end hold zeros in LDS. Scores are fp32 dot products, four
// lanes per (head, token); the online-softmax update is wave-parallel (one
// wave per head, lanes = tokens); the PV update takes sixteen lanes per
// (head, 4 dims), each over a sixteenth of the tile, summed with DPP.
template <int D>
__global__ __launch_bounds__(kGenThreads) void split_f32(SplitArgs a) {
  constexpr int GH = kHeadsPerGroup;
  constexpr int TILE = 4096 / D;
  constexpr int DP = D + 4;                       // padded K row (b128 reads)
  constexpr int C4 = D / 4;                       // 16-byte pieces per row
  constexpr int NL = TILE * C4 / kGenThreads;     // pieces per thread: 4
  static_assert(NL * kGenThreads == TILE * C4, "tile split");
  __shared__ __align__(16) float q_s[GH][D];
  __shared__ __align__(16) float acc_s[GH][D];
  __shared__ __align__(16) float k_s[TILE][DP];
  __shared__ __align__(16) float v_s[TILE][D];
  __shared__ float p_s[GH][TILE + 1];
  __shared__ float m_s[GH], l_s[GH], al_s[GH];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int s = blockIdx.z, b = blockIdx.y;
  const int kvh = blockIdx.x / a.nhg;
  const int hg = blockIdx.x - kvh * a.nhg;
  const int h0 = kvh * a.G + hg * GH;
  const int nh = min(GH, a.G - hg * GH);
  const int len = clamp_len(a, b);
  const int lo = s * a.P;
  const int hi = min(lo + a.P, len);
  if (lo >= hi) {
    write_empty<D>(a, b, h0, nh, s);
    return;
  }
  const float* K = static_cast<const float*>(a.k);
  const float* V = static_cast<const float*>(a.v);
  const float* Q = static_cast<const float*>(a.q) + ((size_t)b * a.Hq + h0) * D;

  // Rows past the tile's end re-read its last row (attended, so always
  // readable) and are zeroed when stored to LDS: the loads stay
  // unconditional and the pieces stay in registers.
  f32x4 kr[NL], vr[NL];
  auto load_tile = [&](int t0, int nt) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int idx = tid + i * kGenThreads;
      const int r = idx / C4, c = idx - r * C4;
      const size_t off =
          row_offset<D>(a, b, kvh, t0 + (r < nt ? r : nt - 1)) + 4 * c;
      kr[i] = *reinterpret_cast<const f32x4*>(K + off);
      vr[i] = *reinterpret_cast<const f32x4*>(V + off);
    }
  };
  int t0 = lo;
  int nt = min(TILE, hi - t0);
  load_tile(t0, nt);

  for (int i = tid; i < nh * C4; i += kGenThreads) {
    const int g = i / C4, c = i - g * C4;
    *reinterpret_cast<f32x4*>(&q_s[g][4 * c]) =
        *reinterpret_cast<const f32x4*>(Q + (size_t)g * D + 4 * c);
  }
  for (int i = tid; i < nh * D; i += kGenThreads) acc_s[i / D][i % D] = 0.f;
  if (tid < GH) {
    m_s[tid] = -INFINITY;
    l_s[tid] = 0.f;
  }

  for (;;) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int idx = tid + i * kGenThreads;
      const int r = idx / C4, c = idx - r * C4;
      const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
      *reinterpret_cast<f32x4*>(&k_s[r][4 * c]) = r < nt ? kr[i] : z;
      *reinterpret_cast<f32x4*>(&v_s[r][4 * c]) = r < nt ? vr[i] : z;
    }
    __syncthreads();
    const int t1 = t0 + TILE;
    if (t1 < hi) load_tile(t1, min(TILE, hi - t1));   // prefetch

    // Scores: four lanes per (head, token), a quarter of the dims each,
    // summed across the quad.
    for (int i = tid; i < nh * TILE * 4; i += kGenThreads) {
      const int qq = i & 3, gt = i >> 2;
      const int g = gt / TILE, jj = gt - g * TILE;
      float acc = 0.f;
#pragma unroll
      for (int c0 = 0; c0 < C4 / 4; ++c0) {
        const int c = qq * (C4 / 4) + c0;
        const f32x4 qv = *reinterpret_cast<const f32x4*>(&q_s[g][4 * c]);
        const f32x4 kv = *reinterpret_cast<const f32x4*>(&k_s[jj][4 * c]);
        acc = fmaf(qv[0], kv[0], acc);
        acc = fmaf(qv[1], kv[1], acc);
        acc = fmaf(qv[2], kv[2], acc);
        acc = fmaf(qv[3], kv[3], acc);
      }
      acc += dpp_f<0xB1>(acc);
      acc += dpp_f<0x4E>(acc);
      if (qq == 0) p_s[g][jj] = jj < nt ? acc * a.scale_log2 : -INFINITY;
    }
    __syncthreads();
    for (int g = wave; g < nh; g += kGenThreads / 64) {
      const float x = lane < nt ? p_s[g][lane] : -INFINITY;
      const float mx = wave_max_f(x);
      const float mn = fmaxf(m_s[g], mx);
      const float e = lane < nt ? fexp2(x - mn) : 0.f;
      if (lane < TILE) p_s[g][lane] = e;
      const float sum = wave_sum_f(e);
      if (lane == 0) {
        const float al = fexp2(m_s[g] - mn);
        l_s[g] = l_s[g] * al + sum;
        m_s[g] = mn;
        al_s[g] = al;
      }
    }
    __syncthreads();
    // PV: sixteen lanes (one DPP row) per (head, 4 dims), each over a
    // sixteenth of the tile's tokens, summed across the row. Rows past nt
    // hold zeros in v_s and p_s, so every lane runs the same trip count.
    for (int i = tid; i < nh * C4 * 16; i += kGenThreads) {
      const int t = i & 15, gc = i >> 4;
      const int g = gc / C4, c = gc - g * C4;
      f32x4 part = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < TILE / 16; ++u) {
        const int jj = t * (TILE / 16) + u;
        const float pj = p_s[g][jj];
        const f32x4 vv = *reinterpret_cast<const f32x4*>(&v_s[jj][4 * c]);
        part[0] = fmaf(pj, vv[0], part[0]);
        part[1] = fmaf(pj, vv[1], part[1]);
        part[2] = fmaf(pj, vv[2], part[2]);
        part[3] = fmaf(pj, vv[3], part[3]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x = part[e];
        x += dpp_f<0xB1>(x);
        x += dpp_f<0x4E>(x);
        x += dpp_f<0x124>(x);
        x += dpp_f<0x128>(x);
        part[e] = x;
      }
      if (t == 0) {
        const float al = al_s[g];
        f32x4 acc = *reinterpret_cast<const f32x4*>(&acc_s[g][4 * c]);
        acc[0] = fmaf(acc[0], al, part[0]);
        acc[1] = fmaf(acc[1], al, part[1]);
        acc[2] = fmaf(acc[2], al, part[2]);
        acc[3] = fmaf(acc[3], al, part[3]);
        *reinterpret_cast<f32x4*>(&acc_s[g][4 * c]) = acc;
      }
    }
    __syncthreads();
    if (t1 >= hi) break;
    t0 = t1;
    nt = min(TILE, hi - t0);
  }

  for (int i = tid; i < nh * D; i += kGenThreads) {
    const int g = i / D, d = i - g * D;
    o_dst<D>(a, b, h0 + g, s)[d] = acc_s[g][d] / l_s[g];
  }
  if (tid < nh) {
    float* l = lse_dst(a, b, h0 + tid, s);
    if (l) *l = (m_s[tid] + flog2(l_s[tid])) * kLn2;
  }
}

// ----------------------------------------------------------------------------
// MFMA split kernel (bf16).
//
// Lane layout of v_mfma_f32_16x16x32_bf16 used throughout (lane l, n = l%16,
// j = l/16): the A operand's row and the B operand's column are n, and the
// lane holds 8 consecutive k-slots 8j..8j+7 of it; the 16x16 fp32 result has
// column n and rows 4j..4j+3 in the lane.
//
// Scores are computed transposed, S^T = K * Q^T, so that a lane ends up with
// ONE query head (column n) and 8 tokens; that is exactly the lane's share
// of P^T as the B operand of O^T = V^T * P^T, and the O^T result again has
// head n in column n. Every per-head quantity (running max, alpha, sum)
// therefore lives in the lane that needs it; only the max needs a 4-lane
// exchange per subtile.
//
// A wave consumes a 32-token subtile: tokens 16*tg + 4j + i (tg = 0,1,
// i = 0..3) are the rows of the two S^T tiles in lane group j, and the same
// 8 tokens, T_j = {4j..4j+3, 16+4j..16+4j+3}, are lane group j's k-slots in
// the PV product, so P never leaves its lane.
//
// K rows (A operand of QK): lane (n, j) loads 16 bytes of token 16*tg + n at
// dims 32c + 8j (c = 0..D/32-1); Q^T (B operand) uses the same dims.
// V rows (A operand of PV): lane (n, j) loads 16 bytes (8 dims starting at
// 8n for D = 128) of each token in T_j -- every load instruction reads four
// whole 256-byte rows -- and an 8x8 transpose in registers (v_perm_b32)
// turns the 8 tokens x 8 dims block into 8 k-vectors, one per PV call.
//
// P is rounded to bf16 for the matrix cores as a hi/lo pair (p_hi = bf16(p),
// p_lo = bf16(p - p_hi)); both products accumulate in fp32, so the weights
// carry ~16 mantissa bits instead of 8.

// K and V are read with non-temporal loads: every byte is used once, and
// keeping it out of the caches' retained set measured 10-12 % faster on
// long histories.
//
// One workgroup = NW waves on one split of one (sequence, kv head, group of
// at most GM query heads). Wave w owns the 32-token subtiles w, w+NW, ... of
// the split, one in flight at a time (bf16: the next one is requested as the
// current one lands); the other resident waves cover the latency. With SPEC
// (batch 1) a wave's first subtile is requested before the sequence length
// is known: its rows are clamped to the split's range for a full-length
// history, which is always inside the cache, and V rows past the true length
// are zeroed once the length arrives (they may hold anything, NaN included,
// and are multiplied by p = 0). Without SPEC the length comes first and
// nothing past it is read. At the end every wave parks its (O, m, l) in LDS
// and the whole workgroup merges them in one pass.
constexpr int kMaxPages = 1024;   // page ids a workgroup stages in LDS
constexpr float kRefSlack = 8.f;  // exponent-reference slack, base 2

// ----------------------------------------------------------------------------
// Length-aware split pieces for batched calls.
//
// With one split length P for the whole batch, a ragged batch leaves short
// last splits, and the number of busy workgroups rarely fits the CUs: some
// CUs get one more split than others and set the kernel's time. Batched
// fd_decode_attn calls (at most 64 sequences) therefore cut sequence b into
// n_b = ceil(len_b / T) pieces of equal length (rounded to 16), with T >= P
// the smallest multiple of 16 for which sum_b n_b <= target (about two
// workgroups per CU over all kv head units); n_b <= S holds because T >= P.
// Piece p of b goes to split slot p. Workgroups take pieces in dispatch
// order (kv head unit fastest), so the busy ones are the first dispatched
// and spread evenly over the CUs; the B * S - sum n_b idle ones each write
// one unused slot (p >= n_b) as empty, so the combine still reads S valid
// slots per (sequence, head). Every wave computes the same plan from the
// lengths (lane = sequence) with wave-wide reductions and scans: no LDS, no
// barrier, one length load.
struct Piece { int b, slot, lo, hi, unit; };

// Wave-wide integer sum on the VALU: DPP within each 16-lane row (swap
// neighbours, swap pairs, rotate by 4 and by 8), then the row exchanges.
__device__ __forceinline__ int wave_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x124, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false);
  const auto r16 = __builtin_amdgcn_permlane16_swap((unsigned)v, (unsigned)v,
                                                    false, false);
  v = (int)(r16[0] + r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap((unsigned)v, (unsigned)v,
                                                    false, false);
  return (int)(r32[0] + r32[1]);
}
// Inclusive prefix sum over the wave without LDS: shifts by 1, 2, 4 and 8
// inside each 16-lane row (DPP; lanes shifted in from outside the row read
// 0), then each row adds the totals of the rows below it (read from lanes
// 15, 31 and 47 into scalars).
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);   // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(v, 15);
  const int r1 = __builtin_amdgcn_readlane(v, 31);
  const int r2 = __builtin_amdgcn_readlane(v, 47);
  return v + (lane >= 16 ? r0 : 0) + (lane >= 32 ? r1 : 0) +
         (lane >= 48 ? r2 : 0);
}

__device__ Piece balanced_piece(const SplitArgs& a, const int32_t* lens,
                                int L, int P, int units) {
  const int lane = threadIdx.x & 63;
  const int B = a.B, S = a.S;
  int len = 0;
  if (lane < B) {
    len = lens[lane];
    len = len < 0 ? 0 : (len > L ? L : len);
  }
  // Smallest T (multiple of 16, >= P) with sum ceil(len / T) <= target.
  // sum ceil(len / T) lies in [W / T, W / T + B'] (W tokens, B' non-empty
  // sequences), which brackets T; beyond L every sequence is one piece.
  // 64-bit token total (two 16-bit halves keep each wave sum in range);
  // it only brackets the search, which checks every candidate exactly.
  const long long W = ((long long)wave_sum(len >> 16) << 16) +
                      wave_sum(len & 0xFFFF);
  const int Bn = wave_sum(len > 0 ? 1 : 0);
  const int tgt = a.bal_target;
  const long long lmax = max((long long)P, ((long long)L + 15) & ~15LL);
  auto round16 = [&](long long x) {
    return min(lmax, (x + 15) & ~15LL);
  };
  long long tlo = max((long long)P, round16((W + tgt - 1) / tgt));
  long long thi = tgt > Bn ? round16((W + (tgt - Bn) - 1) / (tgt - Bn)) : lmax;
  thi = max(thi, tlo);
  auto pieces = [&](long long T) {          // ceil(len / T), no overflow
    return len > 0 ? (int)(((long long)len + T - 1) / T) : 0;
  };
  while (tlo < thi) {
    const long long T = max(tlo, ((tlo + thi) >> 1) & ~15LL);
    const int cnt = wave_sum(pieces(T));
    if (cnt <= a.bal_target) thi = T;
    else tlo = T + 16;
  }
  const long long T = tlo;
  const int nb = pieces(T);
  const int unused = lane < B ? S - nb : 0;
  const int incl = wave_incl_scan(nb);
  const int eincl = wave_incl_scan(unused);
  const int total = __builtin_amdgcn_readlane(incl, 63);
  // Dispatch-order index: kv head unit fastest, then piece.
  const unsigned gid = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  Piece pc;
  pc.unit = (int)(gid % (unsigned)units);
  const int i = (int)(gid / (unsigned)units);
  if (i < total) {
    const unsigned long long m = __builtin_amdgcn_ballot_w64(
        lane < B && i >= incl - nb && i < incl);
    // bb is wave-uniform (from a ballot): read its values as scalars.
    const int bb = __builtin_amdgcn_readfirstlane(__builtin_ctzll(m));
    pc.b = bb;
    const int lb = __builtin_amdgcn_readlane(len, bb);
    const int npc = __builtin_amdgcn_readlane(nb, bb);
    const int p = i - (__builtin_amdgcn_readlane(incl, bb) - npc);
    const long long len_p =                     // equal pieces
        (((long long)lb + npc - 1) / npc + 15) & ~15LL;
    pc.slot = p;
    pc.lo = (int)min((long long)lb, p * len_p);
    pc.hi = (int)min((long long)lb, p * len_p + len_p);
  } else {
    const int k = i - total;
    const unsigned long long m = __builtin_amdgcn_ballot_w64(
        lane < B && k >= eincl - unused && k < eincl);
    const int bb = __builtin_amdgcn_readfirstlane(__builtin_ctzll(m));
    pc.b = bb;
    pc.slot = __builtin_amdgcn_readlane(nb, bb) +
              (k - (__builtin_amdgcn_readlane(eincl, bb) -
                    __builtin_amdgcn_readlane(unused, bb)));
    pc.lo = pc.hi = 0;
  }
  return pc;
}


// Waves per SIMD the register allocation targets: two wherever a wave
// holds two subtiles of registers (the reissue schedule below: bf16, and
// the 8-bit caches on a single sequence's long splits, whose 8-wave
// workgroups fill a CU at two waves per SIMD anyway), three for the 8-bit
// caches' plain loop.
constexpr int split_waves_per_simd(bool two_sets) { return two_sets ? 2 : 3; }

// 8-bit caches (QM != kCacheBf16). A lane reads 16 bytes = 16 dims of a key
// row per request (dims 16(j + 4c)..+15) and 8 bytes = 8 dims of a value
// row, converts them to bf16 in registers (exact for both encodings) and
// runs the same bf16 products. The QK contraction order is free, so Q's
// fragments simply follow the same dim order.
//   kCacheE4M3: E4M3 codes, one scale per kv head for K and one for V; the
//     key scale is folded into the logit scale and the value scale into the
//     final normalisation.
//   kCacheI8: int8 codes with one fp32 scale per (position, kv head) for K
//     and for V, in rows of whole 16-position groups. A lane loads the
//     scales of the 8 positions whose scores it holds (rows 4j..4j+3 of
//     each 16-row group: one 16-byte request per group, never past the
//     group) without clamping; the key scale multiplies each score, and the
//     value scale multiplies each probability on its way into the PV
//     product, while the softmax sum takes the unscaled probability.
//     Positions at or past the length are masked, whatever their scales.
template <int D, int NW, int GM, bool PAGED, bool SPEC, int QM,
          bool BAL = false, bool PIPE = QM == kCacheBf16>
__global__ __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(split_waves_per_simd(PIPE))))
void split_mfma(
    const void* __restrict__ Kp, const void* __restrict__ Vp,
    const uint16_t* __restrict__ Q, int L, int P, int Hkv, int nhg, int G,
    const int32_t* __restrict__ bt_or_lens, int bs, SplitArgs a) {
  constexpr bool F8 = QM != kCacheBf16;     // one byte per element
  constexpr bool I8 = QM == kCacheI8;
  using KT = typename std::conditional<F8, uint8_t, uint16_t>::type;
  using VT = typename std::conditional<F8, u32x2, u32x4>::type;
  const KT* __restrict__ K = static_cast<const KT*>(Kp);
  const KT* __restrict__ V = static_cast<const KT*>(Vp);
  constexpr int KC = MfmaCfg<D>::KC;
  constexpr int NV = MfmaCfg<D>::NV;
  constexpr int KL = F8 ? D / 64 : D / 32;   // 16-byte K requests per row
  constexpr int DP = D + 4;                 // padded LDS row
  __shared__ float mo[NW][GM][DP];
  __shared__ int pg_s[PAGED ? kMaxPages : 1];
  __shared__ float mm[NW][GM], ml[NW][GM];

  // A contiguous cache has no block table: its preloaded slot carries the
  // lengths, so the length load waits on no kernel-argument read (those go
  // to memory and would delay the wave's first compute).
  const int32_t* __restrict__ bt = PAGED ? bt_or_lens : nullptr;
  const int32_t* __restrict__ lens = PAGED ? a.seq_lens : bt_or_lens;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, j = lane >> 4;
  int unit = blockIdx.x;                    // kv head x head group
  int s = blockIdx.z, b = blockIdx.y;       // output slot, sequence
  int lo = s * P;
  int hi_max = min(lo + P, L);              // split end for a full history
  if constexpr (BAL) {
    // Length-aware pieces (batched calls): every wave derives the same plan
    // from the lengths; the workgroup takes the piece of its dispatch rank.
    const Piece pc = balanced_piece(a, lens, L, P, Hkv * nhg);
    unit = pc.unit;
    b = pc.b;
    s = pc.slot;
    lo = pc.lo;
    hi_max = pc.hi;
  }
  const int kvh = unit / nhg;
  const int hg = unit - kvh * nhg;
  const int h0 = kvh * G + hg * GM;
  const int nh = min(GM, G - hg * GM);
  if (__builtin_expect(lo >= hi_max, 0)) {  // no sequence reaches this split
    write_empty<D>(a, b, h0, nh, s);
    return;
  }

  // Element offset of the row of token t (t a multiple of 16 below the
  // clamp bound; wave-uniform).
  // Paged cache: the block ids of the pages this split can reach are staged
  // in LDS once (one round trip), so no cache request waits on a table read.
  // A split spanning more than kMaxPages pages reads the table directly.
  const int max_blocks = a.max_blocks, num_blocks = a.num_blocks;
  const int pg0 = PAGED ? lo / bs : 0;
  const int npg = PAGED ? (hi_max - 1) / bs - pg0 + 1 : 0;
  const bool staged = PAGED && npg <= kMaxPages;
  if (PAGED && staged) {
    const int32_t* row = bt + (size_t)b * max_blocks + pg0;
    for (int i = threadIdx.x; i < npg; i += NW * 64) {
      const int blk = row[i];
      pg_s[i] = blk < 0 ? 0 : (blk >= num_blocks ? num_blocks - 1 : blk);
    }
    __syncthreads();
  }

  auto group_base = [&](int t) -> size_t {
    if (!PAGED) return ((size_t)(b * Hkv + kvh) * L + t) * D;
    const int page = t / bs;
    int blk;
    if (staged) {
      blk = __builtin_amdgcn_readfirstlane(pg_s[page - pg0]);
    } else {
      blk = __builtin_amdgcn_readfirstlane(bt[(size_t)b * max_blocks + page]);
      blk = blk < 0 ? 0 : (blk >= num_blocks ? num_blocks - 1 : blk);
    }
    return (((size_t)blk * Hkv + kvh) * bs + (t - page * bs)) * D;
  };

  // int8 cache: the per-position scales of the subtile in flight (the
  // lane's rows 4j + e of each 16-row group). Contiguous scale rows are
  // padded to whole groups; a paged pool's pages are whole groups.
  struct Sc { f32x4 k[2], v[2]; };       // key and value scales
  Sc scp;                                 // (part of a subtile's registers)
  const float* __restrict__ k_scales = I8 ? a.k_scale : nullptr;
  const float* __restrict__ v_scales = I8 ? a.v_scale : nullptr;
  const size_t Lp = ((size_t)L + 15) & ~(size_t)15;    // L may be INT32_MAX
  auto scale_row = [&](size_t g, int t) -> size_t {   // g = group_base(t)
    if (PAGED) return g / D;
    return (size_t)(b * Hkv + kvh) * Lp + t;
  };

  // Requests the subtile starting at t0 with every row clamped below `end`.
  // `part` selects the key requests (1), the value requests (2) or both.
  auto load_subtile = [&](int t0, int end, u32x4 (&kr)[2][KL],
                          VT (&vr)[8], int part, Sc& sc) {
    const int last0 = min(15, end - 1 - t0);
    const int last1 = end - 1 - (t0 + 16);
    const size_t g0 = group_base(t0);
    const KT* K0 = K + g0;
    const KT* V0 = V + g0;
    const KT* K1;
    const KT* V1;
    size_t g1;
    int cap1;
    if (last1 >= 0) {
      g1 = group_base(t0 + 16);
      K1 = K + g1;
      V1 = V + g1;
      cap1 = min(15, last1);
    } else {
      g1 = g0 + (size_t)last0 * D;
      K1 = K0 + (size_t)last0 * D;
      V1 = V0 + (size_t)last0 * D;
      cap1 = 0;
    }
    if constexpr (I8) {
      // A group wholly past `end` re-reads the first group's scales.
      const size_t s0 = scale_row(g0, t0) + 4 * j;
      const size_t s1 = last1 >= 0 ? scale_row(g1, t0 + 16) + 4 * j : s0;
      if (part & 1) {
        sc.k[0] = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4*>(k_scales + s0));
        sc.k[1] = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4*>(k_scales + s1));
      }
      if (part & 2) {
        sc.v[0] = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4*>(v_scales + s0));
        sc.v[1] = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4*>(v_scales + s1));
      }
    }
    // Element offsets (16-byte requests): bf16 K dims 8j + 32c, 8-bit K
    // dims 16j + 64c.
    constexpr int KJ = F8 ? 16 : 8, KS = F8 ? 64 : 32;
    const unsigned r0 = (unsigned)(min(n, last0) * D + KJ * j);
    const unsigned r1 = (unsigned)(min(n, cap1) * D + KJ * j);
    if (part & 1) {
#pragma unroll
      for (int c = 0; c < KL; ++c) {
        kr[0][c] = ld16<true>(K0 + r0 + KS * c);
        kr[1][c] = ld16<true>(K1 + r1 + KS * c);
      }
    }
    const int vcol = D == 128 ? 8 * n : 8 * (n & 7);
    if (part & 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const unsigned v0 = (unsigned)(min(4 * j + e, last0) * D + vcol);
        const unsigned v1 = (unsigned)(min(4 * j + e, cap1) * D + vcol);
        if constexpr (F8) {
          vr[e] = ld8<true>(V0 + v0);
          vr[4 + e] = ld8<true>(V1 + v1);
        } else {
          vr[e] = ld16<true>(V0 + v0);
          vr[4 + e] = ld16<true>(V1 + v1);
        }
      }
    }
  };

  // With SPEC the wave's first subtile goes out before anything else,
  // clamped to the split's full-history end; without it (batches whose
  // lengths vary, where many splits are empty or short) the length comes
  // first and nothing past it is read.
  int hi = hi_max;
  if (!SPEC && !BAL) {
    int len = lens[b];
    len = len < 0 ? 0 : (len > L ? L : len);
    hi = min(lo + P, len);
    if (__builtin_expect(lo >= hi, 0)) {
      write_empty<D>(a, b, h0, nh, s);
      return;
    }
  }
  // Q^T fragments. Padded columns (n >= nh) load head h0's row: their
  // scores are computed and never used. Loads return in order, so a wait
  // for Q also waits for every request issued before it: a batch's waves
  // (their length already known) request Q ahead of the first subtile,
  // while a single sequence's waves send the first subtile out first (Q
  // first measured 0.4 us slower at 64K) and so do int8 batches (0.7 %
  // slower with Q first).
  bf16x8 qf[KC];
  auto load_q = [&] {
    const uint16_t* qp =
        Q + ((size_t)b * G * Hkv + h0 + (n < nh ? n : 0)) * D;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const int d0 = F8 ? 16 * j + 64 * (c >> 1) + 8 * (c & 1) : 8 * j + 32 * c;
      qf[c] = as_bf16x8(*reinterpret_cast<const u32x4*>(qp + d0));
    }
  };
  const int t_first = lo + 32 * w;
  constexpr bool kQFirst = !SPEC && !I8;
  if (kQFirst) load_q();
  u32x4 kp[2][KL];
  VT vp[8];
  load_subtile(min(t_first, (hi - 1) & ~15), hi, kp, vp, 3, scp);
  if (!kQFirst) load_q();

  // With SPEC nothing branches on the length before the compute: a split
  // past the end of its sequence computes nothing and is written as empty
  // at the merge.
  if (SPEC) {
    int len = lens[b];
    len = len < 0 ? 0 : (len > L ? L : len);
    hi = min(lo + P, len);
  }
  // Logit scale (base 2), with an E4M3 cache's key scale folded in.
  const float sl2 =
      QM == kCacheE4M3 ? a.scale_log2 * a.k_scale[kvh] : a.scale_log2;

  f32x4 o[NV];
#pragma unroll
  for (int cc = 0; cc < NV; ++cc) o[cc] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  // A wave has one subtile in flight, so the compute tail is on the
  // critical path: it branches (uniformly) around the masking of full
  // subtiles and around unneeded rescales.
  //
  // Reissue on arrival (PIPE): the next subtile's keys are requested once
  // the current keys are in registers, its values once the current values
  // are, each before the current data is used, so a wave's compute never
  // delays its next request (two subtiles of registers). bf16 always runs
  // it (two waves per SIMD); issuing the next subtile earlier, before the
  // current one lands, measured slower. 8-bit subtiles (half the bytes per
  // request, plus the conversions) keep the plain loop where a wave streams
  // few subtiles (E4M3 6-12 %, int8 ~25 % slower at 64K with the schedule)
  // or where int8 pieces want two workgroups per CU (its registers leave
  // room for one); a single sequence's 8-bit splits of 8 or more subtiles
  // per wave run it (E4M3 2-6 %, int8 0.6 % faster at 256K; an int8
  // register set includes the subtile's scales), and so do E4M3 pieces on
  // 4 waves.
  constexpr bool kPipe = PIPE;

  // Four 8-bit codes -> four bf16 (exact).
  auto cvt4 = [](unsigned w) -> uint2 {
    if constexpr (I8) return s8x4_to_bf16x4(w);
    else return e4m3x4_to_bf16x4(w);
  };

  // The k-vector of QK call c for token group tg (bf16 operands).
  auto k_operand = [&](const u32x4 (&kr)[2][KL], int tg, int c) -> bf16x8 {
    if constexpr (F8) {
      const u32x4 x = kr[tg][c >> 1];
      const uint2 p = cvt4(x[2 * (c & 1)]);
      const uint2 q = cvt4(x[2 * (c & 1) + 1]);
      return as_bf16x8(u32x4{p.x, p.y, q.x, q.y});
    } else {
      return as_bf16x8(kr[tg][c]);
    }
  };

  // `after_scores` runs between the softmax step and the PV products.
  auto compute_subtile = [&](int t0, const u32x4 (&kr)[2][KL],
                             const VT (&vraw)[8], Sc& sc,
                             auto&& after_scores) {
    f32x4 sacc[2];
#pragma unroll
    for (int tg = 0; tg < 2; ++tg) {
      sacc[tg] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < KC; ++c)
        sacc[tg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            k_operand(kr, tg, c), qf[c], sacc[tg], 0, 0, 0);
    }
    float sv[8];
    float mx = -INFINITY;
    // Per-score logit scale (an int8 cache's key scale of that position).
    auto lscale = [&](int e) -> float {
      return I8 ? sl2 * sc.k[e >> 2][e & 3] : sl2;
    };
    if (t0 + 32 <= hi) {                    // every token valid (uniform)
#pragma unroll
      for (int tg = 0; tg < 2; ++tg)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x = sacc[tg][i] * lscale(4 * tg + i);
          sv[4 * tg + i] = x;
          mx = fmaxf(mx, x);
        }
    } else {
#pragma unroll
      for (int tg = 0; tg < 2; ++tg)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = t0 + 16 * tg + 4 * j + i;
          const float x =
              tok < hi ? sacc[tg][i] * lscale(4 * tg + i) : -INFINITY;
          sv[4 * tg + i] = x;
          mx = fmaxf(mx, x);
          // A masked position's value scale may be anything (even NaN):
          // its probability is 0 and must stay 0.
          if constexpr (I8) sc.v[tg][i] = tok < hi ? sc.v[tg][i] : 0.f;
        }
    }
    mx = max_x32(max_x16(mx));
    // The exponent reference m_run moves only when the max grows by more
    // than kRefSlack (base 2): p = 2^(s - m_run) then stays below
    // 2^kRefSlack, exact in fp32 and as a bf16 hi/lo pair, and O and l are
    // rescaled only when some lane's reference moves (wave-uniform skip).
    // Before any valid token m_run = -inf; the first valid subtile moves it
    // (alpha = 0 on the still-zero O and l).
    const float mcand = fmaxf(m_run, mx);
    const bool upd = mcand > m_run + kRefSlack;
    float alpha = 1.f;
    if (__builtin_amdgcn_ballot_w64(upd) != 0) {
      alpha = upd ? fexp2(m_run - mcand) : 1.f;
      m_run = upd ? mcand : m_run;
    }
    const float mref = m_run == -INFINITY ? 0.f : m_run;
    bf16x8 ph, pl;
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = fexp2(sv[e] - mref);
      psum += p;
      const float pw = I8 ? p * sc.v[e >> 2][e & 3] : p;   // value row e
      const __bf16 hb = (__bf16)pw;
      ph[e] = hb;
      pl[e] = (__bf16)(pw - (float)hb);
    }
    l_run = l_run * alpha + psum;
    if constexpr (kPipe) {
      // Pin the exponentials here, ahead of the value wait: left alone the
      // compiler sinks them next to their only use, the PV products, which
      // puts them behind the arrival of the wave's last subtile.
      asm volatile("" ::"v"(__builtin_bit_cast(u32x4, ph)),
                   "v"(__builtin_bit_cast(u32x4, pl)));
    }
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
      for (int cc = 0; cc < NV; ++cc) o[cc] *= alpha;
    }
    after_scores();
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
      const bf16x8 vk = v_kvec<D>(vr, cc, n);
      o[cc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vk, ph, o[cc], 0, 0, 0);
      o[cc] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vk, pl, o[cc], 0, 0, 0);
    }
  };

  // The first subtile is consumed without a branch on the length (a branch
  // would let the compiler sink its loads behind the length load). A
  // subtile past hi is fully masked and changes nothing.
  if (SPEC && t_first + 32 > hi) {
    // Rows at or past hi were read speculatively: zero their V.
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int t = t_first + (e < 4 ? 4 * j + e : 12 + 4 * j + e);
      if (t >= hi) vp[e] = VT{};
    }
  }
  if constexpr (kPipe) {
    // Two register sets, used in turn. An empty asm statement that takes a
    // subtile's registers as inputs makes the compiler wait for exactly
    // those loads there; the scheduling barriers keep the next requests
    // between that wait and the first use of the current data.
    u32x4 kq[2][KL];
    VT vq[8];
    Sc scq;
    auto step = [&](int tc, const u32x4 (&kc)[2][KL], const VT (&vc)[8],
                    Sc& scc, u32x4 (&kn)[2][KL], VT (&vn)[8], Sc& scn,
                    auto more_c) {
      constexpr bool more = decltype(more_c)::value;
      const int tn = tc + 32 * NW;
#pragma unroll
      for (int tg = 0; tg < 2; ++tg)
#pragma unroll
        for (int c = 0; c < KL; ++c) asm volatile("" ::"v"(kc[tg][c]));
      __builtin_amdgcn_sched_barrier(0);
      if (more) load_subtile(tn, hi, kn, vn, 1, scn);
      __builtin_amdgcn_sched_barrier(0);
      compute_subtile(tc, kc, vc, scc, [&] {
#pragma unroll
        for (int e = 0; e < 8; ++e) asm volatile("" ::"v"(vc[e]));
        __builtin_amdgcn_sched_barrier(0);
        if (more) load_subtile(tn, hi, kn, vn, 2, scn);
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    // Whether a step requests the next subtile is fixed when the code is
    // generated: with a run-time condition the compiler's wait counts are
    // those of the path that requested nothing, so every step would also
    // wait for the next subtile's keys before using its own values (64K
    // batch-one split kernel 12.4 -> 12.15 us without that wait).
    const int nsub = t_first < hi ? (hi - t_first - 1) / (32 * NW) + 1 : 1;
    int t0 = t_first, rem = nsub;
    for (; rem > 2; rem -= 2, t0 += 64 * NW) {
      step(t0, kp, vp, scp, kq, vq, scq, std::true_type{});
      step(t0 + 32 * NW, kq, vq, scq, kp, vp, scp, std::true_type{});
    }
    if (rem == 2) {
      step(t0, kp, vp, scp, kq, vq, scq, std::true_type{});
      step(t0 + 32 * NW, kq, vq, scq, kp, vp, scp, std::false_type{});
    } else {
      step(t0, kp, vp, scp, kq, vq, scq, std::false_type{});
    }
  } else {
    compute_subtile(t_first, kp, vp, scp, [] {});
    for (int t0 = t_first + 32 * NW; t0 < hi; t0 += 32 * NW) {
      load_subtile(t0, hi, kp, vp, 3, scp);
      // All of the subtile's requests go out before its first use.
      __builtin_amdgcn_sched_barrier(0);
      compute_subtile(t0, kp, vp, scp, [] {});
    }
  }

  // Per-head sum over the 4 lane groups; then park (O, m, l) in LDS.
  l_run = sum_x32(sum_x16(l_run));
  if (n < nh) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float* row = &mo[w][n][out_dim<D>(0, i, j)];
      *reinterpret_cast<f32x4*>(row) = f32x4{o[0][i], o[1][i], o[2][i], o[3][i]};
      if (D == 128)
        *reinterpret_cast<f32x4*>(row + 4) = f32x4{o[4][i], o[5][i], o[6][i], o[7][i]};
    }
    if (j == 0) {
      mm[w][n] = m_run;
      ml[w][n] = l_run;
    }
  }
  __syncthreads();

  // Merge: thread -> (head g, 4 dims); waves that saw no token carry m = -inf.
  // An E4M3 cache's value scale multiplies the normalised output.
  const float vsc = QM == kCacheE4M3 ? a.v_scale[kvh] : 1.f;
  for (int idx = threadIdx.x; idx < nh * (D / 4); idx += NW * 64) {
    const int g = idx / (D / 4);
    const int d = 4 * (idx - g * (D / 4));
    // Every LDS read goes out at once (one round trip), and the
    // normalisation uses the hardware reciprocal (1 ulp).
    float mw[NW], lw[NW];
    f32x4 ow[NW];
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      mw[ww] = mm[ww][g];
      lw[ww] = ml[ww][g];
      ow[ww] = *reinterpret_cast<const f32x4*>(&mo[ww][g][d]);
    }
    float M = mw[0];
#pragma unroll
    for (int ww = 1; ww < NW; ++ww) M = fmaxf(M, mw[ww]);
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    float lsum = 0.f;
    const float Ms = M == -INFINITY ? 0.f : M;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const float wt = fexp2(mw[ww] - Ms);
      acc += wt * ow[ww];
      lsum += wt * lw[ww];
    }
    const bool none = M == -INFINITY;       // no token in this split
    const f32x4 res = acc * (vsc * __builtin_amdgcn_rcpf(lsum));
    *reinterpret_cast<f32x4*>(o_dst<D>(a, b, h0 + g, s) + d) =
        none ? f32x4{0.f, 0.f, 0.f, 0.f} : res;
    if (d == 0) {
      float* l = lse_dst(a, b, h0 + g, s);
      if (l) *l = none ? -INFINITY : (M + flog2(lsum)) * kLn2;
    }
  }
}

// ----------------------------------------------------------------------------
// Log-sum-exp combine of split partials.

// One wave per (sequence, head, 16-dim slice of the output). Lane l takes
// split group g = l/4 and dims 4*(l%4) of the slice; group g reads splits
// g, g+16, g+32, ... . A chunk's loads (8 splits per lane) are all issued
// before any is used, so a chunk costs one memory round trip; chunks merge
// online, and the 16 groups are reduced with cross-lane exchanges. Every
// split slot holds a valid partial (empty splits are o = 0, lse = -inf and
// get weight 0), so no length is needed, and the arguments are scalars the
// hardware preloads: the kernel waits on nothing before its data loads.
template <int D>
__global__ __launch_bounds__(64) void combine_kernel(
    const float* __restrict__ o_part, const float* __restrict__ lse_part,
    float* __restrict__ out_base, float* __restrict__ lse_out, int S) {
  constexpr int SL = D / 16;                // slices per head
  constexpr int CH = 8;                     // splits per lane per chunk
  const int lane = threadIdx.x;
  const int bh = blockIdx.x / SL;
  const int sl = blockIdx.x - bh * SL;
  const int g = lane >> 2, qd = lane & 3;
  const float* lse = lse_part + (size_t)bh * S;
  const float* op = o_part + (size_t)bh * S * D + 16 * sl + 4 * qd;

  float M = -INFINITY, z = 0.f;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int base = 0; base < S; base += 16 * CH) {
    float lv[CH];
    f32x4 ov[CH];
    // Splits past S re-read the last one (every load unconditional, no
    // branch) and are masked once they have arrived.
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const int sp = min(base + g + 16 * k, S - 1);
      lv[k] = lse[sp];
      ov[k] = *reinterpret_cast<const f32x4*>(op + (size_t)sp * D);
    }
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const bool ok = base + g + 16 * k < S;
      lv[k] = ok ? lv[k] : -INFINITY;
      ov[k] = ok ? ov[k] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float mx = lv[0];
#pragma unroll
    for (int k = 1; k < CH; ++k) mx = fmaxf(mx, lv[k]);
    // The 4 lanes of a 16-lane row with the same dims (lane % 4) hold
    // split groups g, g + 1, ...: rotations by 4 and 8 inside the row (DPP,
    // no LDS round trip), then the row exchanges.
    mx = fmaxf(mx, dpp_f<0x124>(mx));
    mx = fmaxf(mx, dpp_f<0x128>(mx));
    mx = max_x32(max_x16(mx));
    const float Mn = fmaxf(M, mx);           // wave-uniform
    if (Mn == -INFINITY) continue;
    const float f = fexp2((M - Mn) * kLog2e);
    acc *= f;
    z *= f;
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      const float wt = fexp2((lv[k] - Mn) * kLog2e);
      acc += wt * ov[k];
      z += wt;
    }
    M = Mn;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float x = acc[i];
    x += dpp_f<0x124>(x);
    x += dpp_f<0x128>(x);
    acc[i] = sum_x32(sum_x16(x));
  }
  z += dpp_f<0x124>(z);
  z += dpp_f<0x128>(z);
  z = sum_x32(sum_x16(z));
  float* out = out_base + (size_t)bh * D + 16 * sl + 4 * qd;
  const f32x4 res = acc * __builtin_amdgcn_rcpf(z);   // 1 ulp
  if (g == 0)
    *reinterpret_cast<f32x4*>(out) =
        M == -INFINITY ? f32x4{0.f, 0.f, 0.f, 0.f} : res;
  if (lane == 0 && sl == 0 && lse_out)
    lse_out[bh] = M == -INFINITY ? -INFINITY : M + flog2(z) * kLn2;
}

// Grid of the split kernels: x = kv head (x head group), y = sequence,
// z = split. Workgroups are dispatched x-fastest and dealt round-robin to the
// 8 XCDs, so this order puts every split index on every XCD (with the split
// index fastest, XCD i would get only splits s = i mod 8: in a batch of
// unequal lengths the low splits, which every sequence fills, would all land
// on the same XCDs) and dispatches the always-full low splits first.
dim3 split_grid(int units, int B, int S) {
  return dim3((unsigned)units, (unsigned)B, (unsigned)S);
}

// Waves per workgroup of the MFMA kernel for a split of P tokens. Measured
// on MI355X: bf16 runs best with 4 waves and the reissue schedule at every
// split length (64K, 256K, the ragged batch and the batch of 64 short
// histories; 8 waves, or 4 waves with two subtiles requested at once, were
// 1-4 % slower). The 8-bit caches (E4M3 and int8; 64K and 256K,
// S = 64..256) run 8 waves from 9 subtiles per split (16 waves were no
// better at 64K, and 0-5 % slower on 8192-token splits), on the plain loop
// except a single sequence's long E4M3 splits (see launch_mfma).
int split_waves(int P, bool f8) {
  const int64_t nsub = ((int64_t)P + 31) / 32;   // P may be near INT32_MAX
  return f8 && nsub > 8 ? 8 : 4;
}

// The leading scalar arguments are what a wave needs before its first K/V
// request; they fit the 14 kernel-argument dwords gfx950 preloads into SGPRs
// at dispatch, so no wave waits on an argument load before its first
// request (such loads queue behind other waves' K/V traffic).
template <int D, int NW, int GM, bool PAGED, bool SPEC, int QM,
          bool BAL = false, bool PIPE = QM == kCacheBf16>
void launch_one(dim3 grid, const SplitArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((split_mfma<D, NW, GM, PAGED, SPEC, QM, BAL, PIPE>), grid,
                     dim3(NW * 64), 0, st, a.k, a.v,
                     static_cast<const uint16_t*>(a.q), a.L, a.P, a.Hkv,
                     a.nhg, a.G, PAGED ? a.block_table : a.seq_lens, a.bs, a);
}

template <int D, bool PAGED, int GM, bool SPEC, int QM, bool BAL = false>
void launch_mfma_spec(dim3 grid, int nw, bool pipe8, const SplitArgs& a,
                      hipStream_t st) {
  constexpr bool F8 = QM != kCacheBf16;
  if constexpr (QM != kCacheBf16 && SPEC) {
    if (pipe8 && nw == 8) {
      launch_one<D, 8, GM, PAGED, SPEC, QM, BAL, true>(grid, a, st);
      return;
    }
  }
  // E4M3 length-aware pieces: 4 waves on the reissue schedule (ragged paged
  // batch of 16 91.0 -> 88.9 us, 8 x 32K 27.6 -> 25.8 us, 16 x 2K even;
  // int8 pieces measured 1 % slower with it and keep their plain loop).
  if constexpr (QM == kCacheE4M3 && BAL) {
    launch_one<D, 4, GM, PAGED, SPEC, QM, BAL, true>(grid, a, st);
    return;
  }
  if (F8 && nw == 8)
    launch_one<D, F8 ? 8 : 4, GM, PAGED, SPEC, QM, BAL>(grid, a, st);
  else
    launch_one<D, 4, GM, PAGED, SPEC, QM, BAL>(grid, a, st);
}

// Speculative first loads pay off for a single sequence (its splits are all
// full when the caller's bound is its length); for a batch, whose lengths
// may differ, they could read splits that turn out empty.
template <int D, bool PAGED, int GM, int QM>
void launch_mfma_gm(dim3 grid, int nw, bool pipe8, const SplitArgs& a,
                    hipStream_t st) {
  if (a.B == 1)
    launch_mfma_spec<D, PAGED, GM, true, QM>(grid, nw, pipe8, a, st);
  else if (a.bal_target > 0 && a.B <= 64)       // lane = sequence
    launch_mfma_spec<D, PAGED, GM, false, QM, true>(grid, nw, false, a, st);
  else
    launch_mfma_spec<D, PAGED, GM, false, QM>(grid, nw, false, a, st);
}

template <int D, bool PAGED, int QM>
void launch_mfma(const Shape& s, SplitArgs a, hipStream_t st) {
  const int gm = s.G <= 8 ? 8 : 16;
  a.nhg = (s.G + gm - 1) / gm;
  // About two workgroups per CU in total, spread over the kv head units.
  a.bal_target = a.balance_cus > 0 && a.S > 1
                     ? max(1, 2 * a.balance_cus / (s.Hkv * a.nhg)) : 0;
  const dim3 grid = split_grid(s.Hkv * a.nhg, s.B, a.S);
  // int8 length-aware pieces (batches of 2..64) run 4 waves: 5-6 % faster
  // than 8 on the ragged batch of 16 when the kernel held ~148 VGPRs (one
  // 8-wave workgroup per CU), and still 1.5-4 % faster at its present
  // 118-126, where two would fit.
  const bool pieces = a.B > 1 && a.B <= 64 && a.bal_target > 0;
  const int nw = QM == kCacheI8 && pieces
                     ? 4 : split_waves(a.P, QM != kCacheBf16);
  // 8-bit caches, one sequence: the reissue schedule from 8 subtiles per
  // wave (E4M3 measured 2-6 % faster at 8 and 32 per wave, even at 4, and
  // at 64K, 2 per wave, 5-8 % slower; int8 0.6 % faster at 32 per wave).
  const bool pipe8 = QM != kCacheBf16 && a.B == 1 &&
                     ((int64_t)a.P + 31) / 32 >= 8 * nw;
  if (gm == 8)
    launch_mfma_gm<D, PAGED, 8, QM>(grid, nw, pipe8, a, st);
  else
    launch_mfma_gm<D, PAGED, 16, QM>(grid, nw, pipe8, a, st);
}

template <int QM>
void launch_mfma_dtype(const Shape& s, const SplitArgs& a, hipStream_t st) {
  const bool paged = s.bs > 0;
  if (s.D == 128) {
    if (paged) launch_mfma<128, true, QM>(s, a, st);
    else launch_mfma<128, false, QM>(s, a, st);
  } else {
    if (paged) launch_mfma<64, true, QM>(s, a, st);
    else launch_mfma<64, false, QM>(s, a, st);
  }
}

}  // namespace

int launch_split(const Shape& s, const SplitArgs& a, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (s.dtype == FD_DTYPE_BF16) {
    launch_mfma_dtype<kCacheBf16>(s, a, st);
  } else if (s.dtype == FD_DTYPE_FP8_E4M3) {
    launch_mfma_dtype<kCacheE4M3>(s, a, st);
  } else if (s.dtype == FD_DTYPE_INT8) {
    launch_mfma_dtype<kCacheI8>(s, a, st);
  } else {
    const dim3 grid = split_grid(s.Hkv * a.nhg, s.B, a.S);
    const dim3 block(kGenThreads);
    if (s.D == 128)
      hipLaunchKernelGGL((split_f32<128>), grid, block, 0, st, a);
    else
      hipLaunchKernelGGL((split_f32<64>), grid, block, 0, st, a);
  }
  return (int)hipGetLastError();
}

// ----------------------------------------------------------------------------
// Scratch for fd_decode_attn_noalloc: the partials of one call live in this
// array instead of a caller's workspace. Each device holds its own copy
// (until the process ends); host code never uses the array's name as an
// address, only the pointer hipGetSymbolAddress returns for the current
// device, looked up once per device.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

int scratch_address(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return (int)hipErrorInvalidDevice;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return 0;
}

int launch_combine(int D, const CombineArgs& a, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (D == 128)
    hipLaunchKernelGGL((combine_kernel<128>), dim3((unsigned)(a.B * a.Hq * 8)),
                       dim3(64), 0, st, a.o_part, a.lse_part, a.out,
                       a.lse_out, a.S);
  else
    hipLaunchKernelGGL((combine_kernel<64>), dim3((unsigned)(a.B * a.Hq * 4)),
                       dim3(64), 0, st, a.o_part, a.lse_part, a.out,
                       a.lse_out, a.S);
  return (int)hipGetLastError();
}

}  // namespace fd
