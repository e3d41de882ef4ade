// KV commit: append a completed block's K/V rows to the cache (Fast-dVLA
// notes, key design 1; Fast-dDrive method summary sec. 3.1).  A plain
// bit-exact copy of [Hkv][n_rows][D] into rows [start, start + n_rows) of one
// sequence, 16 bytes per lane.

#include "bc_internal.h"

namespace bc {
namespace {

__global__ __launch_bounds__(256) void commit_kernel(uint4* __restrict__ cache, const uint4* __restrict__ blk,
                                                     int units_per_row, int n_rows, int Hkv,
                                                     long long head_stride_u, int start, long long total) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int u = (int)(i % units_per_row);
  const long long rh = i / units_per_row;
  const int r = (int)(rh % n_rows);
  const int h = (int)(rh / n_rows);
  cache[h * head_stride_u + (long long)(start + r) * units_per_row + u] = blk[i];
}

}  // namespace

hipError_t launch_commit(void* cache, const void* blk, int dtype, int Hkv, int D,
                         long long seq_stride, long long head_stride, int start, int n_rows,
                         hipStream_t stream) {
  (void)seq_stride;
  const int elem = dtype == BC_BF16 ? 2 : 4;
  const int units_per_row = D * elem / 16;
  const long long head_stride_u = head_stride * elem / 16;
  const long long total = (long long)Hkv * n_rows * units_per_row;
  const int grid = (int)((total + 255) / 256);
  hipLaunchKernelGGL(commit_kernel, dim3(grid), dim3(256), 0, stream, static_cast<uint4*>(cache),
                     static_cast<const uint4*>(blk), units_per_row, n_rows, Hkv, head_stride_u, start,
                     total);
  return hipGetLastError();
}

}  // namespace bc
