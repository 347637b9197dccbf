// Host-side driver for the library's argument checks and kernel-argument
// marshalling. It is compiled together with fd_host.cpp under
// AddressSanitizer and UndefinedBehaviorSanitizer, against stub launchers
// and stub device queries (no GPU, no HIP runtime). Every call uses fake,
// suitably aligned device addresses, which the host code never
// dereferences. The stubs check the invariants a kernel relies on:
//   - splits cover the history;
//   - the workspace holds the partials it is handed;
//   - scale pointers exist exactly for the quantized dtypes.
// Prints "ok <calls> launches" and exits 0 when every check holds.
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "fd_internal.h"

// The two device queries the host code makes: device 0, 256 CUs.
hipError_t hipGetDevice(int* device) {
  *device = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t, int) {
  *value = 256;
  return hipSuccess;
}

static int g_fail = 0;
static long g_launches = 0;
static uintptr_t g_ws = 0;        // workspace handed to the current call
static size_t g_ws_bytes = 0;

#define EXPECT(c)                                                          \
  do {                                                                     \
    if (!(c)) {                                                            \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);      \
      ++g_fail;                                                            \
    }                                                                      \
  } while (0)

namespace fd {

static void check_split_args(const Shape& s, const SplitArgs& a) {
  EXPECT(a.S >= 1 && a.S <= kMaxSplits);
  EXPECT(a.P >= 16 && a.P % 16 == 0);
  if (s.bs > 0) EXPECT(a.P % s.bs == 0);
  EXPECT((int64_t)a.S * a.P >= s.L);
  EXPECT(a.B == s.B && a.Hq == s.Hq && a.Hkv == s.Hkv && a.G == s.G);
  EXPECT(a.L == s.L && a.bs == s.bs);
  EXPECT(a.nhg == (s.G + kHeadsPerGroup - 1) / kHeadsPerGroup);
  EXPECT(isfinite(a.scale_log2) && a.scale_log2 > 0.f);
  EXPECT(a.q && a.k && a.v && a.seq_lens && a.o_dst);
  EXPECT((a.block_table != nullptr) == (s.bs > 0));
  const bool quant = s.dtype == FD_DTYPE_FP8_E4M3 || s.dtype == FD_DTYPE_INT8;
  EXPECT((a.k_scale != nullptr) == quant && (a.v_scale != nullptr) == quant);
  if (s.dtype == FD_DTYPE_INT8)
    EXPECT(((uintptr_t)a.k_scale & 15) == 0 && ((uintptr_t)a.v_scale & 15) == 0);
  if (a.final_out) {
    EXPECT(a.S == 1);
  } else if (g_ws) {                // partials inside the workspace
    const uintptr_t o = (uintptr_t)a.o_dst, l = (uintptr_t)a.lse_dst;
    const size_t no = (size_t)a.B * a.Hq * a.S * s.D * 4;
    const size_t nl = (size_t)a.B * a.Hq * a.S * 4;
    EXPECT(o == g_ws && (o & 15) == 0);
    EXPECT(l >= o + no && l + nl <= g_ws + g_ws_bytes);
  }
  EXPECT(a.balance_cus == 0 || a.balance_cus == 256);
  if (a.balance_cus) EXPECT(a.B > 1 && a.S > 1);
}

int launch_split(const Shape& s, const SplitArgs& a, void*) {
  ++g_launches;
  check_split_args(s, a);
  return 0;
}

// The allocation-free entry point's scratch: a fake device address.
static const uintptr_t kScratchAddr = 0x7e0000000000ull;
int scratch_address(void** ptr) {
  *ptr = (void*)kScratchAddr;
  return 0;
}

int launch_combine(int D, const CombineArgs& c, void*) {
  ++g_launches;
  EXPECT(D == 64 || D == 128);
  EXPECT(c.B >= 1 && c.Hq >= 1 && c.S >= 1);
  EXPECT(c.o_part && c.lse_part && c.out);
  if (g_ws) {
    EXPECT((uintptr_t)c.o_part == g_ws);
    EXPECT((uintptr_t)c.lse_part + (size_t)c.B * c.Hq * c.S * 4 <=
           g_ws + g_ws_bytes);
  }
  return 0;
}

int launch_summary(const Shape& s, const SummaryArgs& a, void*) {
  ++g_launches;
  EXPECT(s.dtype == FD_DTYPE_BF16 || s.dtype == FD_DTYPE_FP8_E4M3 ||
         s.dtype == FD_DTYPE_INT8);
  EXPECT((a.k_scale != nullptr) == (s.dtype != FD_DTYPE_BF16));
  EXPECT(a.k && a.seq_lens && a.codes && a.scales);
  EXPECT(a.nblk_row == ((int64_t)s.L + 15) / 16);
  EXPECT((a.block_table != nullptr) == (s.bs > 0));
  return 0;
}

int launch_sparse(const Shape& s, const SplitArgs& a, const SparseArgs& sp,
                  void*) {
  ++g_launches;
  check_split_args(s, a);
  EXPECT(a.P <= kMaxSparseSplit);
  EXPECT(s.G <= kMaxSparseG);
  EXPECT((int64_t)a.P * (s.G > kHeadsPerGroup ? s.G : kHeadsPerGroup) <=
         kMaxSparseEst);
  EXPECT(sp.codes && sp.scales && sp.delta_log2 >= 0.f);
  EXPECT(sp.nblk_row == ((int64_t)s.L + 15) / 16);
  return 0;
}

}  // namespace fd

// Deterministic generator (64-bit LCG, high bits).
static uint64_t g_rng = 0x9E3779B97F4A7C15ull;
static uint32_t rnd() {
  g_rng = g_rng * 6364136223846793005ull + 1442695040888963407ull;
  return (uint32_t)(g_rng >> 33);
}
static int pick(const int* v, int n) { return v[rnd() % (uint32_t)n]; }

int main() {
  const uintptr_t base = 0x7f0000000000ull;   // fake, 256-byte aligned
  void* q = (void*)(base + 0x100);
  void* k = (void*)(base + 0x200);
  void* v = (void*)(base + 0x300);
  int32_t* bt = (int32_t*)(base + 0x400);
  int32_t* lens = (int32_t*)(base + 0x500);
  float* ks = (float*)(base + 0x600);
  float* vs = (float*)(base + 0x700);
  float* out = (float*)(base + 0x800);
  float* lse = (float*)(base + 0x900);
  void* codes = (void*)(base + 0xa00);
  float* cscales = (float*)(base + 0xb00);
  const uintptr_t ws = base + 0x100000;

  const int batches[] = {1, 2, 3, 16, 64, 65, 4096, 65535, 65536, 0, -1};
  const int heads[] = {1, 2, 3, 8, 16, 24, 64, 128, 0};
  const int kvheads[] = {1, 2, 3, 8, 16, 0};
  const int dims[] = {64, 128, 96, 0, 256};
  const int lengths[] = {0, 1, 15, 16, 17, 255, 1000, 65536, 262144,
                         1 << 20, 1 << 24, 2147483647, -1};
  const int pages[] = {0, 0, 16, 32, 48, 256, 4096, 15, 8192, -16};
  const int dtypes[] = {FD_DTYPE_F32, FD_DTYPE_BF16, FD_DTYPE_FP8_E4M3,
                        FD_DTYPE_INT8, 7};
  long oks = 0;
  for (int it = 0; it < 20000; ++it) {
    fd_shape s;
    memset(&s, 0, sizeof s);
    // Mostly values a caller may pass, sometimes anything in the lists.
    const bool any = rnd() % 4 == 0;
    s.batch = pick(batches, any ? 11 : 7);
    s.num_q_heads = pick(heads, any ? 9 : 8);
    s.num_kv_heads = pick(kvheads, any ? 6 : 5);
    s.head_dim = pick(dims, any ? 5 : 2);
    s.max_seq_len = pick(lengths, any ? 13 : 10);
    s.block_size = pick(pages, any ? 10 : 7);
    s.dtype = pick(dtypes, any ? 5 : 4);
    s.scale = (rnd() % 4 == 0) ? -1.f : 0.125f;
    if (s.block_size > 0) {
      const int64_t need =
          ((int64_t)(s.max_seq_len > 0 ? s.max_seq_len : 0) + s.block_size -
           1) / s.block_size;
      s.max_blocks_per_seq = (int32_t)(need > 0x7fffffff ? 0x7fffffff
                                                         : need + (int)(rnd() % 2));
      s.num_blocks = (int32_t)(1 + rnd() % 100000);
    }
    int S = 0;
    const int64_t sum = (rnd() % 2) ? -1 : (int64_t)(rnd() % 1000000);
    const int pst = fd_plan_splits(&s, 256, sum, &S);
    EXPECT(pst <= 0);
    if (pst == FD_OK) EXPECT(S >= 1 && S <= fd::kMaxSplits);
    if (pst != FD_OK || rnd() % 3 == 0) S = (int)(rnd() % 70000) - 2;
    size_t bytes = 0;
    const int wst = fd_workspace_size(&s, S, &bytes);
    EXPECT(wst <= 0);
    g_ws = ws;
    g_ws_bytes = (wst == FD_OK) ? bytes : 0;
    const bool paged = s.block_size > 0;
    const int32_t* tbl = paged ? bt : nullptr;
    const long before = g_launches;
    const int which = (int)(rnd() % 12);
    if (which == 1 || which == 6) g_ws = 0;   // caller's own partials
    int st;
    switch (which) {
      case 0:
        st = fd_decode_attn(&s, q, k, v, tbl, lens, S, (void*)ws, g_ws_bytes,
                            out, lse, nullptr);
        break;
      case 1:
        st = fd_decode_partials(&s, q, k, v, tbl, lens, S, (float*)ws,
                                (float*)(ws + 0x80000000ull), nullptr);
        break;
      case 2:
        st = fd_decode_attn_fp8(&s, q, k, v, ks, vs, tbl, lens, S, (void*)ws,
                                g_ws_bytes, out, lse, nullptr);
        break;
      case 3:
        st = fd_decode_attn_int8(&s, q, k, v, ks, vs, tbl, lens, S,
                                 (void*)ws, g_ws_bytes, out, lse, nullptr);
        break;
      case 4:
        st = fd_build_key_summary(&s, k, tbl, lens, codes, cscales, nullptr);
        break;
      case 5:
        st = fd_decode_attn_sparse(&s, q, k, v, codes, cscales, tbl, lens,
                                   (rnd() % 2) ? 3.f : INFINITY, S, (void*)ws,
                                   g_ws_bytes, out, lse, nullptr, nullptr);
        break;
      case 8:
        st = fd_build_key_summary_fp8(&s, k, ks, tbl, lens, codes, cscales,
                                      nullptr);
        break;
      case 9:
        st = fd_decode_attn_sparse_fp8(&s, q, k, v, ks, vs, codes, cscales,
                                       tbl, lens, (rnd() % 2) ? 3.f : INFINITY,
                                       S, (void*)ws, g_ws_bytes, out, lse,
                                       nullptr, nullptr);
        break;
      case 10:
        st = fd_build_key_summary_int8(&s, k, ks, tbl, lens, codes, cscales,
                                       nullptr);
        break;
      case 11:
        st = fd_decode_attn_sparse_int8(&s, q, k, v, ks, vs, codes, cscales,
                                        tbl, lens, (rnd() % 2) ? 3.f : INFINITY,
                                        S, (void*)ws, g_ws_bytes, out, lse,
                                        nullptr, nullptr);
        break;
      case 7:                                   // partials in the scratch
        g_ws = fd::kScratchAddr;
        g_ws_bytes = fd::kScratchBytes;
        st = fd_decode_attn_noalloc(&s, q, k, v, tbl, lens, S, out, lse,
                                    nullptr);
        if (wst == FD_OK && bytes > fd::kScratchBytes)
          EXPECT(st == FD_ERR_WORKSPACE);
        break;
      default:
        st = fd_combine_partials(s.batch, s.num_q_heads, s.head_dim, S,
                                 (const float*)ws,
                                 (const float*)(ws + 0x80000000ull), out,
                                 nullptr, nullptr);
        break;
    }
    EXPECT(st == FD_OK || st == FD_ERR_INVALID_ARG ||
           st == FD_ERR_UNSUPPORTED || st == FD_ERR_WORKSPACE);
    if (st == FD_OK) {
      ++oks;
      EXPECT(g_launches > before);
    } else {
      EXPECT(g_launches == before);   // a refused call launches nothing
    }
    const char* msg = fd_status_str(st);
    EXPECT(msg && strlen(msg) > 0);
  }
  if (g_fail) {
    fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  printf("ok %ld launches, %ld accepted calls\n", g_launches, oks);
  return 0;
}
