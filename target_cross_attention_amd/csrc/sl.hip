// Stochastic-length training batches: the gather of every user's temporal suffix into one
// padding-free buffer ("Make It Long, Keep It Fast", notes page: element selection and the
// sequence-compression step of batch-level load balancing).
#include "device_common.hpp"
#include "internal.hpp"

namespace stca {

// Block (x, u) copies packed rows [kRows x, kRows (x + 1)) of user u: the destination segment
// starts at hist_off[u], the source at full_off[u+1] - len (the user's last len rows).  Both
// offsets are uniform per block; consecutive threads copy consecutive 16-byte chunks.
constexpr int kRows = 64;

// A user whose offsets break the contract (packed segment longer than its history, or past
// `total`) is skipped rather than read or written out of bounds.
__global__ __launch_bounds__(256) void sl_pack_kernel(const int64_t *__restrict__ full_off,
                                                      const int64_t *__restrict__ hist_off, int64_t total,
                                                      int row16, const u32x4 *__restrict__ X,
                                                      u32x4 *__restrict__ out) {
  const int u = blockIdx.y;
  const int64_t dst0 = hist_off[u], len = hist_off[u + 1] - dst0;
  const int64_t r0 = (int64_t)blockIdx.x * kRows;
  if (r0 >= len) return;
  const int64_t src0 = full_off[u + 1] - len;
  if (src0 < full_off[u] || dst0 < 0 || dst0 + len > total) return;
  const int64_t rows = len - r0 < kRows ? len - r0 : kRows;
  const int64_t n = rows * row16;
  const u32x4 *src = X + (src0 + r0) * row16;
  u32x4 *dst = out + (dst0 + r0) * row16;
  for (int64_t i = threadIdx.x; i < n; i += 256) dst[i] = src[i];
}

hipError_t sl_pack(hipStream_t s, int n_users, const int64_t *full_off, const int64_t *hist_off, int64_t total,
                   int64_t max_len, int row16, const void *X_full, void *X_packed) {
  if (n_users <= 0 || max_len <= 0) return hipSuccess;
  const dim3 grid((unsigned)((max_len + kRows - 1) / kRows), (unsigned)n_users);
  hipLaunchKernelGGL(sl_pack_kernel, grid, dim3(256), 0, s, full_off, hist_off, total, row16,
                     (const u32x4 *)X_full, (u32x4 *)X_packed);
  return hipGetLastError();
}

}  // namespace stca
