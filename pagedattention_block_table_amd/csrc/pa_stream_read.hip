// Plain streaming read of a device buffer: the HBM read ceiling that the decode kernels'
// K/V streams are measured against. Decode moves its bytes with the same 16-byte vector
// loads, one 1 KiB contiguous run per wave instruction, plain or non-temporal; this kernel
// does only that (no table lookups, no arithmetic beyond folding the loaded words
// together), so its rate is what a read-only kernel of that load shape reaches.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pa.h"

namespace pa {
namespace {

constexpr int kReadThreads = 256;

// Each workgroup reads U consecutive 4 KiB runs (one per 256-thread row of 16-byte loads)
// per iteration, all U loads issued before any is used; iterations stride over the grid.
// The loaded words are folded into one value per thread, written only if it equals a
// fixed pattern (so the loads are not dropped and almost nothing is written).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

template <int U, bool NT>
__global__ void __launch_bounds__(kReadThreads) stream_read_kernel(const uint4* __restrict__ p, int64_t n16,
                                                                   uint32_t* sink) {
  const int64_t step = (int64_t)gridDim.x * U * kReadThreads;
  uint32_t acc = 0;
  for (int64_t base = (int64_t)blockIdx.x * U * kReadThreads; base < n16; base += step) {
    uint4 r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint4* q = p + base + u * kReadThreads + threadIdx.x;
      if constexpr (NT) {
        const u32x4_t w = __builtin_nontemporal_load((const u32x4_t*)q);
        r[u] = make_uint4(w.x, w.y, w.z, w.w);
      } else {
        r[u] = *q;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= r[u].x ^ r[u].y ^ r[u].z ^ r[u].w;
  }
  if (acc == 0x9E3779B9u) sink[threadIdx.x] = acc;
}

template <int U>
int launch_read(const void* buf, int64_t n16, int grid, bool nt, uint32_t* sink, hipStream_t st) {
  if (nt)
    hipLaunchKernelGGL((stream_read_kernel<U, true>), dim3(grid), dim3(kReadThreads), 0, st, (const uint4*)buf,
                       n16, sink);
  else
    hipLaunchKernelGGL((stream_read_kernel<U, false>), dim3(grid), dim3(kReadThreads), 0, st, (const uint4*)buf,
                       n16, sink);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // namespace
}  // namespace pa

extern "C" int pa_debug_stream_read(const void* buf, size_t bytes, int unroll, int num_workgroups,
                                    int nontemporal, uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes == 0 || num_workgroups < 0) return PA_ERR_INVALID;
  if (nontemporal != 0 && nontemporal != 1) return PA_ERR_INVALID;
  if (((uintptr_t)buf & 15u) != 0) return PA_ERR_INVALID;
  if (unroll != 4 && unroll != 8 && unroll != 16) return PA_ERR_INVALID;
  const size_t run = (size_t)16 * unroll * pa::kReadThreads;  // bytes per workgroup iteration
  if (bytes % run != 0) return PA_ERR_INVALID;
  const int64_t iters = (int64_t)(bytes / run);
  int64_t grid = num_workgroups == 0 ? iters : num_workgroups;
  if (grid > iters) grid = iters;
  if (grid > 0x7fffffff) return PA_ERR_INVALID;
  const int64_t n16 = (int64_t)(bytes / 16);
  hipStream_t st = (hipStream_t)stream;
  switch (unroll) {
    case 4: return pa::launch_read<4>(buf, n16, (int)grid, nontemporal != 0, sink, st);
    case 8: return pa::launch_read<8>(buf, n16, (int)grid, nontemporal != 0, sink, st);
    default: return pa::launch_read<16>(buf, n16, (int)grid, nontemporal != 0, sink, st);
  }
}
