// HBM read probe: a kernel that only streams bytes from device memory, the
// achievable-bandwidth reference for the split kernel (fd_probe.h).

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "fd_decode.h"
#include "fd_probe.h"

namespace fd {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Workgroup w reads elements [w * per, (w + 1) * per) of 16 bytes in steps
// of NW * 64 * U elements: lane l of wave v takes elements
// step + v * 64 + l + u * NW * 64 (u < U), so each load instruction covers
// 1 KB of consecutive bytes. Two register sets: the next step's loads go out
// as soon as the current step's data is in registers, before it is used.
template <int NW, int U>
__global__ __launch_bounds__(NW * 64) void read_probe(
    const u32x4* __restrict__ buf, unsigned per, uint32_t* __restrict__ sink) {
  constexpr unsigned STEP = NW * 64 * U;
  const u32x4* p = buf + (size_t)blockIdx.x * per + threadIdx.x;
  unsigned acc = 0;
  u32x4 a[U], b[U];
#pragma unroll
  for (int u = 0; u < U; ++u) a[u] = __builtin_nontemporal_load(p + u * NW * 64);
  for (unsigned i = 0;;) {
#pragma unroll
    for (int u = 0; u < U; ++u) asm volatile("" ::"v"(a[u]));
    bool more = i + STEP < per;
    if (more) {
#pragma unroll
      for (int u = 0; u < U; ++u)
        b[u] = __builtin_nontemporal_load(p + i + STEP + u * NW * 64);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= a[u][0] ^ a[u][1] ^ a[u][2] ^ a[u][3];
    if (!more) break;
    i += STEP;
#pragma unroll
    for (int u = 0; u < U; ++u) asm volatile("" ::"v"(b[u]));
    more = i + STEP < per;
    if (more) {
#pragma unroll
      for (int u = 0; u < U; ++u)
        a[u] = __builtin_nontemporal_load(p + i + STEP + u * NW * 64);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= b[u][0] ^ b[u][1] ^ b[u][2] ^ b[u][3];
    if (!more) break;
    i += STEP;
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;
}

template <int NW>
int launch_probe(const u32x4* buf, unsigned per, int wg, int u, uint32_t* sink,
                 hipStream_t st) {
  if (u == 2)
    hipLaunchKernelGGL((read_probe<NW, 2>), dim3(wg), dim3(NW * 64), 0, st,
                       buf, per, sink);
  else if (u == 4)
    hipLaunchKernelGGL((read_probe<NW, 4>), dim3(wg), dim3(NW * 64), 0, st,
                       buf, per, sink);
  else if (u == 8)
    hipLaunchKernelGGL((read_probe<NW, 8>), dim3(wg), dim3(NW * 64), 0, st,
                       buf, per, sink);
  else if constexpr (NW <= 8)   // 16 loads per lane: two sets fill 128 VGPRs
    hipLaunchKernelGGL((read_probe<NW, 16>), dim3(wg), dim3(NW * 64), 0, st,
                       buf, per, sink);
  return (int)hipGetLastError();
}

}  // namespace
}  // namespace fd

extern "C" int fd_read_probe(const void* buf, size_t bytes, int workgroups,
                             int waves, int loads_per_lane, uint32_t* sink,
                             void* stream) {
  using namespace fd;
  if (!buf || !sink || (reinterpret_cast<uintptr_t>(buf) & 15u) != 0)
    return FD_ERR_INVALID_ARG;
  if (workgroups < 1 || workgroups > 65535) return FD_ERR_INVALID_ARG;
  if (waves != 4 && waves != 8 && waves != 16) return FD_ERR_INVALID_ARG;
  if (loads_per_lane != 2 && loads_per_lane != 4 && loads_per_lane != 8 &&
      !(loads_per_lane == 16 && waves <= 8))
    return FD_ERR_INVALID_ARG;
  const size_t step = (size_t)waves * 64 * 16 * loads_per_lane;
  if (bytes == 0 || bytes % ((size_t)workgroups * step) != 0)
    return FD_ERR_INVALID_ARG;
  const size_t per = bytes / 16 / (size_t)workgroups;   // elements per WG
  if (per > 0x7FFFFFFFu) return FD_ERR_INVALID_ARG;
  const u32x4* p = static_cast<const u32x4*>(buf);
  hipStream_t st = static_cast<hipStream_t>(stream);
  int err;
  if (waves == 4) err = launch_probe<4>(p, (unsigned)per, workgroups, loads_per_lane, sink, st);
  else if (waves == 8) err = launch_probe<8>(p, (unsigned)per, workgroups, loads_per_lane, sink, st);
  else err = launch_probe<16>(p, (unsigned)per, workgroups, loads_per_lane, sink, st);
  return err == 0 ? FD_OK : FD_ERR_HIP;
}
