// Stochastic-length training batches: the gather of every user's temporal suffix into one
// padding-free buffer ("Make It Long, Keep It Fast", notes page: element selection and the
// sequence-compression step of batch-level load balancing).
#include "device_common.hpp"
#include "internal.hpp"

namespace stca {

// One thread per 16-byte chunk of a packed row.  The row's user is the last u with
// hist_off[u] <= row (binary search; every thread of a row takes the same path, so the loads
// are broadcasts).  Rows are contiguous per user, so consecutive threads copy consecutive bytes.
__global__ __launch_bounds__(256) void sl_pack_kernel(int n_users, const int64_t *__restrict__ full_off,
                                                      const int64_t *__restrict__ hist_off, int64_t total,
                                                      int row16, const u32x4 *__restrict__ X,
                                                      u32x4 *__restrict__ out) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = gid / row16;
  const int c = (int)(gid % row16);
  if (row >= total) return;
  int lo = 0, hi = n_users;  // hist_off[lo] <= row < hist_off[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (hist_off[mid] <= row)
      lo = mid;
    else
      hi = mid;
  }
  const int64_t src = full_off[lo + 1] - (hist_off[lo + 1] - row);
  out[row * row16 + c] = X[src * row16 + c];
}

hipError_t sl_pack(hipStream_t s, int n_users, const int64_t *full_off, const int64_t *hist_off, int64_t total,
                   int row16, const void *X_full, void *X_packed) {
  if (total <= 0) return hipSuccess;
  const int64_t threads = total * row16;
  hipLaunchKernelGGL(sl_pack_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, n_users, full_off,
                     hist_off, total, row16, (const u32x4 *)X_full, (u32x4 *)X_packed);
  return hipGetLastError();
}

}  // namespace stca
