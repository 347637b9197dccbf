// Internal declarations shared by the host checks and the HIP launchers.
#ifndef FD_INTERNAL_H
#define FD_INTERNAL_H

#include <stddef.h>
#include <stdint.h>

#include "fd_decode.h"

namespace fd {

// Planner constants. A split is never shorter than kMinSplitTokens
// (kMinSplitTokensF32 for fp32 caches); the attended tokens are spread over
// about kOccupancy * num_cus workgroups, twice that for a ragged batch whose
// splits would exceed kLongSplitTokens; a batch that fills half the CUs is
// not split below kShortHistoryTokens. Set from a sweep of batch {1..256} x
// history {512..256K} x splits {1..256} (16 query / 2 kv heads, d 128,
// bf16) and the ragged 16-sequence batch on MI355X: with these values the
// planned split count is within a few percent of the best measured one.
// The same sweep over 8-bit caches added two rules: below
// kShortHistoryTokens, kShortHistoryUnits8 units already run unsplit (half
// the bytes per position make the split pay later), and int8 batches of
// 2..64 sequences halve their splits at any length (their 4-wave pieces
// need about two workgroups per CU).
constexpr int kMinSplitTokens = 128;
constexpr int kMinSplitTokensF32 = 64;   // fp32 path: latency-bound, split finer
constexpr int kOccupancy = 1;
constexpr int kLongSplitTokens = 1024;
constexpr int kShortHistoryTokens = 1024;
constexpr int kShortHistoryUnits8 = 8;   // 8-bit caches: unsplit short
                                         // histories from this many units
constexpr int kMaxSplits = 65535;
constexpr int kMaxBlockSize = 4096;
constexpr int kHeadsPerGroup = 16;   // query heads one workgroup serves
constexpr int kMaxSparseSplit = 8192;   // sparse path: tokens per split
constexpr int kMaxSparseG = 128;        // sparse path: query heads per kv head
// Sparse path: tokens per split x max(16, query heads per kv head), the
// block estimates one workgroup keeps in LDS.
constexpr int kMaxSparseEst = kMaxSparseSplit * kHeadsPerGroup;
// Device-resident scratch of fd_decode_attn_noalloc (one array per device):
// the largest workspace it serves.
constexpr size_t kScratchBytes = (size_t)4 << 20;

// A validated, resolved call shape.
struct Shape {
  int B, Hq, Hkv, G, D, L;
  int bs, max_blocks, num_blocks;
  int dtype;
  float scale;        // resolved (> 0)
};

int check_shape(const fd_shape* s, Shape* out);
int tokens_per_split(const Shape& s, int num_splits);   // P
int head_groups(const Shape& s);                        // ceil(G / 16)
size_t partial_o_bytes(const Shape& s, int num_splits);
size_t workspace_bytes(const Shape& s, int num_splits);

// Kernel arguments (passed by value).
struct SplitArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const float* k_scale;   // E4M3: per-kv-head scales; int8: per-position
  const float* v_scale;   // scales in whole 16-position rows; else null
  float* o_dst;       // out [B,Hq,D] (final) or o_part [B,Hq,S,D]
  float* lse_dst;     // lse_out [B,Hq] (final, may be null) or lse_part
  int B, Hq, Hkv, G, L;
  int bs, max_blocks, num_blocks;
  int S, P, nhg;      // splits, tokens per split, head groups per kv head
  int final_out;      // 1: write normalised output + lse to out/lse_out
  int balance_cus;    // > 0 (CU count): length-aware pieces for batches
  int bal_target;     // set by the launcher: pieces per kv head unit
  float scale_log2;   // scale * log2(e)
};

struct CombineArgs {
  const float* o_part;
  const float* lse_part;
  float* out;
  float* lse_out;     // may be null
  int B, Hq, S;
};

// Key summary builder (4-bit codes + per-16-token-block scales).
struct SummaryArgs {
  const void* k;                // bf16 keys or E4M3 codes, contiguous or paged
  const float* k_scale;         // E4M3: one scale per kv head; else null
  const int32_t* block_table;
  const int32_t* seq_lens;
  uint8_t* codes;               // one 8*D-byte record per 16-token block
  float* scales;                // [B,Hkv,nblk_row] or [NB,Hkv,bs/16]
  int Hkv, L, bs, max_blocks, num_blocks, nblk_row;
};

// Extra arguments of the sparse split kernel.
struct SparseArgs {
  const uint8_t* codes;
  const float* scales;
  uint8_t* kept_out;            // [B,Hkv,nblk_row] or null
  float delta_log2;             // top-delta in base-2 logit units (>= 0)
  int nblk_row;                 // ceil(L / 16)
};

// Launchers (fd_kernels.hip, fd_sparse.hip). Return hipError_t as int.
int launch_split(const Shape& s, const SplitArgs& a, void* stream);
int launch_combine(int D, const CombineArgs& a, void* stream);
int launch_summary(const Shape& s, const SummaryArgs& a, void* stream);
// Device address of the current device's scratch array (looked up once per
// device); returns a hipError_t as int.
int scratch_address(void** ptr);
int launch_sparse(const Shape& s, const SplitArgs& a, const SparseArgs& sp,
                  void* stream);

}  // namespace fd

#endif  // FD_INTERNAL_H
