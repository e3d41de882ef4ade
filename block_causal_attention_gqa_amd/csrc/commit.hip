// KV commit: append a completed block's K/V rows to the cache (Fast-dVLA
// notes, key design 1; Fast-dDrive method summary sec. 3.1).  A plain
// bit-exact copy of [Hkv][n_rows][D] into rows [start, start + n_rows) of one
// sequence, K and V in one launch, 16 bytes per lane.

#include "bc_internal.h"

namespace bc {
namespace {

__global__ __launch_bounds__(256) void commit_kernel(uint4* __restrict__ kc, uint4* __restrict__ vc,
                                                     const uint4* __restrict__ bk, const uint4* __restrict__ bv,
                                                     int units_per_row, int n_rows, long long head_stride_u,
                                                     int start, long long total) {
  long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= 2 * total) return;
  const bool is_v = i >= total;
  if (is_v) i -= total;
  const int u = (int)(i % units_per_row);
  const long long rh = i / units_per_row;
  const int r = (int)(rh % n_rows);
  const long long h = rh / n_rows;
  const long long dst = h * head_stride_u + (long long)(start + r) * units_per_row + u;
  if (is_v) vc[dst] = bv[i];
  else kc[dst] = bk[i];
}

}  // namespace

hipError_t launch_commit(void* k_cache, void* v_cache, const void* blk_k, const void* blk_v, int dtype,
                         int Hkv, int D, long long head_stride, int start, int n_rows, hipStream_t stream) {
  const int elem = dtype == BC_BF16 ? 2 : 4;
  const int units_per_row = D * elem / 16;
  const long long head_stride_u = head_stride * elem / 16;
  const long long total = (long long)Hkv * n_rows * units_per_row;
  const int grid = (int)((2 * total + 255) / 256);
  hipLaunchKernelGGL(commit_kernel, dim3(grid), dim3(256), 0, stream, static_cast<uint4*>(k_cache),
                     static_cast<uint4*>(v_cache), static_cast<const uint4*>(blk_k),
                     static_cast<const uint4*>(blk_v), units_per_row, n_rows, head_stride_u, start, total);
  return hipGetLastError();
}

}  // namespace bc
