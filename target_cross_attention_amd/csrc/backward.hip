// Elementwise and reduction kernels of the backward pass (gradients of eqs. (2)-(8) for an
// upstream dZ).  The contractions run on the generic fp32-accumulating GEMM; these kernels are
// the pieces between them: the SwiGLU and LayerNorm derivatives, the softmax of the attention
// and its derivative, and deterministic (fixed-order) reductions.  All arithmetic is fp32.
#include <math.h>

#include "device_common.hpp"
#include "internal.hpp"

namespace stca {

static unsigned grid_for(int64_t n, int per_block = 256) {
  int64_t b = (n + per_block - 1) / per_block;
  return (unsigned)(b > 65536 ? 65536 : (b < 1 ? 1 : b));
}

__device__ __forceinline__ float sigmoidf_(float g) { return 1.0f / (1.0f + expf(-g)); }

// ---- fills and sums ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void fill_kernel(int64_t n, float *__restrict__ y, float v) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) y[i] = v;
}

hipError_t fill_f32(hipStream_t s, int64_t n, float *y, float v) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_kernel, dim3(grid_for(n)), dim3(256), 0, s, n, y, v);
  return hipGetLastError();
}

// out[r ldo + c] (+)= sum_k parts[k rows cols + r cols + c], k = 0 .. nparts-1 in order.
__global__ __launch_bounds__(256) void sum_parts_kernel(int64_t rows, int cols, int nparts,
                                                        const float *__restrict__ parts, float *__restrict__ out,
                                                        int64_t ldo, bool accumulate) {
  const int64_t n = rows * cols;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    float *o = out + (i / cols) * ldo + (i % cols);
    float acc = accumulate ? *o : 0.f;
#pragma unroll 8
    for (int k = 0; k < nparts; ++k) acc += parts[(int64_t)k * n + i];
    *o = acc;
  }
}

hipError_t sum_parts2d(hipStream_t s, int64_t rows, int cols, int nparts, const float *parts, float *out,
                       int64_t ldo, bool accumulate) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  hipLaunchKernelGGL(sum_parts_kernel, dim3(grid_for(rows * cols)), dim3(256), 0, s, rows, cols, nparts, parts, out,
                     ldo, accumulate);
  return hipGetLastError();
}

hipError_t sum_parts(hipStream_t s, int64_t n, int nparts, const float *parts, float *out, bool accumulate) {
  return sum_parts2d(s, 1, (int)n, nparts, parts, out, n, accumulate);
}

// ---- SwiGLU: H = A * G * sigmoid(G) and its derivative ----------------------------------------
__global__ __launch_bounds__(256) void swiglu_fwd_kernel(int64_t n, const float *__restrict__ A,
                                                         const float *__restrict__ G, float *__restrict__ H) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const float g = G[i];
    H[i] = A[i] * g * sigmoidf_(g);
  }
}

hipError_t swiglu_fwd(hipStream_t s, int64_t n, const float *A, const float *G, float *H) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(swiglu_fwd_kernel, dim3(grid_for(n)), dim3(256), 0, s, n, A, G, H);
  return hipGetLastError();
}

// dA = dH g s, dG = dH a s (1 + g (1 - s)), s = sigmoid(g).  Each element is read before it is
// written, so dA may alias dH and dG may alias A or G.
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(int64_t n, const float *dH, const float *A, const float *G,
                                                         float *dA, float *dG) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const float dh = dH[i], a = A[i], g = G[i], sg = sigmoidf_(g);
    dG[i] = dh * a * sg * (1.0f + g * (1.0f - sg));
    dA[i] = dh * g * sg;
  }
}

hipError_t swiglu_bwd(hipStream_t s, int64_t n, const float *dH, const float *A, const float *G, float *dA,
                      float *dG) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(swiglu_bwd_kernel, dim3(grid_for(n)), dim3(256), 0, s, n, dH, A, G, dA, dG);
  return hipGetLastError();
}

// ---- LayerNorm derivative (d <= 512) ------------------------------------------------------------
// From the pre-LN rows Y: xh = (y - mean) rstd; dxh = dout gamma;
// dY = rstd (dxh - mean(dxh) - xh mean(dxh xh)).  A workgroup takes `per` consecutive rows (its four
// waves one row at a time) and also sums, per column, dout xh and dout over its rows: those partial
// sums of dgamma and dbeta go to parts[blk][c] and parts[nblk + blk][c], added later in block order.
__global__ __launch_bounds__(256) void ln_bwd_kernel(int64_t rows, int d, int64_t per, const float *__restrict__ dout,
                                                     int64_t ldd, const float *__restrict__ Y, int64_t ldy,
                                                     const float *__restrict__ gamma, float eps,
                                                     float *__restrict__ dY, float *__restrict__ parts) {
  __shared__ float red[4][2][512];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t r0 = (int64_t)blockIdx.x * per, r1 = r0 + per < rows ? r0 + per : rows;
  float pg[8], pb[8], gm[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int c = lane + 64 * e;
    pg[e] = pb[e] = 0.f;
    gm[e] = c < d ? gamma[c] : 0.f;
  }
  // Rows one ahead: the next row's Y and dout are loaded while this row is reduced.
  float ny[8], ngo[8];
  auto load_row = [&](int64_t row) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = lane + 64 * e;
      const bool ok = row < r1 && c < d;
      ny[e] = ok ? Y[row * ldy + c] : 0.f;
      ngo[e] = ok ? dout[row * ldd + c] : 0.f;
    }
  };
  load_row(r0 + wave);
  for (int64_t row = r0 + wave; row < r1; row += 4) {
    float y[8], go_[8], g[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      y[e] = ny[e];
      go_[e] = ngo[e];
    }
    load_row(row + 4);
    float sum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) sum += y[e];
    const float mean = wave_sum(sum) / (float)d;
    float q = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = lane + 64 * e;
      const float t = c < d ? y[e] - mean : 0.f;
      q += t * t;
    }
    const float rstd = 1.0f / sqrtf(wave_sum(q) / (float)d + eps);
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = lane + 64 * e;
      if (c < d) {
        const float xh = (y[e] - mean) * rstd, go = go_[e];
        g[e] = go * gm[e];
        s1 += g[e];
        s2 += g[e] * xh;
        pg[e] = fmaf(go, xh, pg[e]);
        pb[e] += go;
        y[e] = xh;
      } else {
        g[e] = 0.f;
      }
    }
    const float m1 = wave_sum(s1) / (float)d, m2 = wave_sum(s2) / (float)d;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = lane + 64 * e;
      if (c < d) dY[row * d + c] = rstd * (g[e] - m1 - y[e] * m2);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    red[wave][0][lane + 64 * e] = pg[e];
    red[wave][1][lane + 64 * e] = pb[e];
  }
  __syncthreads();
  for (int c = threadIdx.x; c < d; c += 256) {
    parts[(int64_t)blockIdx.x * d + c] = red[0][0][c] + red[1][0][c] + red[2][0][c] + red[3][0][c];
    parts[(int64_t)(gridDim.x + blockIdx.x) * d + c] = red[0][1][c] + red[1][1][c] + red[2][1][c] + red[3][1][c];
  }
}

hipError_t ln_bwd(hipStream_t s, int64_t rows, int d, const float *dout, int64_t ldd, const float *Y, int64_t ldy,
                  const float *gamma, float eps, float *dY, float *dgamma, float *dbeta, float *parts,
                  int max_blocks) {
  if (rows <= 0) return hipSuccess;
  int64_t per = (rows + max_blocks - 1) / max_blocks;
  per = per < 16 ? 16 : per;
  const int nblk = (int)((rows + per - 1) / per);
  hipLaunchKernelGGL(ln_bwd_kernel, dim3((unsigned)nblk), dim3(256), 0, s, rows, d, per, dout, ldd, Y, ldy, gamma, eps,
                     dY, parts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = sum_parts(s, d, nblk, parts, dgamma, true)) != hipSuccess) return e;
  return sum_parts(s, d, nblk, parts + (int64_t)nblk * d, dbeta, true);
}

// out[r] = sum_c A[r][c] B[r][c] (one wave per row).
__global__ __launch_bounds__(256) void rowdot_kernel(int64_t rows, int d, const float *__restrict__ A,
                                                     const float *__restrict__ B, float *__restrict__ out) {
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= rows) return;
  float acc = 0.f;
  for (int c = lane; c < d; c += 64) acc += A[r * d + c] * B[r * d + c];
  acc = wave_sum(acc);
  if (lane == 0) out[r] = acc;
}

hipError_t rowdot(hipStream_t s, int64_t rows, int d, const float *A, const float *B, float *out) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(rowdot_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, rows, d, A, B, out);
  return hipGetLastError();
}

// y[i] = x[i] (fp32 copy of a strided block: rows x d from ldx into ldy).
__global__ __launch_bounds__(256) void copy_rows_kernel(int64_t rows, int d, const float *__restrict__ x, int64_t ldx,
                                                        float *__restrict__ y, int64_t ldy) {
  const int64_t n = rows * d;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / d;
    const int c = (int)(i % d);
    y[r * ldy + c] = x[r * ldx + c];
  }
}

hipError_t copy_rows(hipStream_t s, int64_t rows, int d, const float *x, int64_t ldx, float *y, int64_t ldy) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(copy_rows_kernel, dim3(grid_for(rows * d)), dim3(256), 0, s, rows, d, x, ldx, y, ldy);
  return hipGetLastError();
}

// ---- attention over a user's history as ragged products (eq. (13) and its derivative) --------
// Query rows r = t h + j (target t, head j), u_r = U[r] unscaled (scores are scale * u_r . X~_k with
// scale = 1/sqrt(d_h)).  User u owns R_u = m_u h query rows and L_u history rows; its score matrix
// S_u (R_u x Lp_u, Lp_u = L_u rounded up to 4, padding columns kept at zero) sits at element sbase_u
// of a buffer holding all users' matrices back to back.  Three descriptor shapes per user:
//   0: S-shape  (R x L, k = d):   S = U X~^T, dA = dabar X~^T          (B transposed)
//   1: row-shape (R x d, k = L):  abar = alpha X~, du = dS X~
//   2: key-shape (L x d, k = R):  dX~ = alpha^T dabar + dS^T U          (A transposed)

// Largest u in [0, n) with off[u] <= x (off nondecreasing, off[0] = 0 <= x < off[n]).
__device__ __forceinline__ int segment_of(const int64_t *__restrict__ off, int n, int64_t x) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// One workgroup: users in blocks of 1024 with a block-wide prefix sum of R_u Lp_u.  The offsets are
// checked against the batch's totals and bounds first (as the forward's work list does); if they
// break them, or the score matrices would not fit the max_scores elements of the workspace, every
// descriptor is written empty (no product or row pass then touches memory through it) and the
// results of the call are meaningless: stca_validate_batch reports such batches.
__global__ __launch_bounds__(1024) void ragged_plan_kernel(int n_users, const int64_t *__restrict__ hoff,
                                                           const int64_t *__restrict__ toff, int h, int d,
                                                           int64_t total_L, int64_t total_T, int64_t max_L,
                                                           int64_t max_T, int64_t max_scores,
                                                           RaggedDesc *__restrict__ descs) {
  __shared__ int64_t sc[1024];
  __shared__ int bad_all;
  const int tid = threadIdx.x;
  if (tid == 0) bad_all = 0;
  __syncthreads();
  {
    int bad = 0;
    for (int u = tid; u < n_users; u += 1024)
      bad |= offsets_violation(u, n_users, hoff, toff, total_L, total_T, max_L, max_T) & ~kBatchEmptyHistory;
    if (bad) atomicOr(&bad_all, bad);
  }
  __syncthreads();
  for (int pass = 0; pass < 2; ++pass) {
    const bool write = pass == 1;
    int64_t carry = 0;
    for (int base = 0; base < n_users; base += 1024) {
      const int u = base + tid;
      int64_t R = 0, L = 0, Lp = 0, L0 = 0, T0 = 0;
      if (u < n_users && bad_all == 0) {
        L0 = hoff[u];
        T0 = toff[u];
        L = hoff[u + 1] - L0;
        R = (toff[u + 1] - T0) * h;
        Lp = (L + 3) & ~(int64_t)3;
      }
      const int64_t cnt = R * Lp;
      sc[tid] = cnt;
      __syncthreads();
      for (int off = 1; off < 1024; off <<= 1) {
        const int64_t a = tid >= off ? sc[tid - off] : 0;
        __syncthreads();
        sc[tid] += a;
        __syncthreads();
      }
      if (write && u < n_users) {
        if (bad_all == 0) {
          const int64_t sbase = carry + sc[tid] - cnt, qrow = T0 * h * d, hrow = L0 * d;
          descs[u] = RaggedDesc{(int32_t)R, (int32_t)L, d, 0, qrow, d, hrow, d, sbase, Lp};
          descs[n_users + u] = RaggedDesc{(int32_t)R, d, (int32_t)L, 0, sbase, Lp, hrow, d, qrow, d};
          descs[2 * n_users + u] = RaggedDesc{(int32_t)L, d, (int32_t)R, 0, sbase, Lp, qrow, d, hrow, d};
        } else {
          const RaggedDesc empty{0, 0, 0, 0, 0, 0, 0, 0, 0, 0};  // zero sizes and strides
          descs[u] = descs[n_users + u] = descs[2 * n_users + u] = empty;
        }
      }
      carry += sc[1023];
      __syncthreads();
    }
    if (!write) {
      if (tid == 0 && carry > max_scores) bad_all |= kBatchOverflow;
      __syncthreads();
    }
  }
}

hipError_t ragged_plan(hipStream_t s, int n_users, const int64_t *hist_off, const int64_t *tgt_off, int h, int d,
                       int64_t total_L, int64_t total_T, int64_t max_L, int64_t max_T, int64_t max_scores,
                       RaggedDesc *descs) {
  if (n_users <= 0) return hipSuccess;
  hipLaunchKernelGGL(ragged_plan_kernel, dim3(1), dim3(1024), 0, s, n_users, hist_off, tgt_off, h, d, total_L, total_T,
                     max_L, max_T, max_scores, descs);
  return hipGetLastError();
}

// Per query row (one wave): MODE 0 computes lse_r = log sum_k e^{scale S_rk} and replaces S_r by
// alpha_r = exp(scale S_r - lse_r); MODE 1 does the replacement with the given lse_r; MODE 2 turns
// dA_r (in S2) into dS_r = alpha_r (dA_r - D_r).  Padding columns become zero.
template <int MODE>
__global__ __launch_bounds__(256) void ragged_rows_kernel(int64_t rows, int h, int n_users,
                                                          const int64_t *__restrict__ tgt_off,
                                                          const RaggedDesc *__restrict__ sdesc, float *__restrict__ S,
                                                          float *__restrict__ S2, float scale, float *__restrict__ lse,
                                                          const float *__restrict__ D) {
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= rows) return;
  const int u = segment_of(tgt_off, n_users, r / h);
  const RaggedDesc dsc = sdesc[u];
  const int64_t L = dsc.N, Lp = dsc.ldc;
  const int64_t off = dsc.c_off + (r - tgt_off[u] * h) * Lp;
  float *row = S + off;
  if (MODE == 2) {
    float *drow = S2 + off;
    const float Dr = D[r];
    for (int64_t k = lane; k < Lp; k += 64) drow[k] = k < L ? row[k] * (drow[k] - Dr) : 0.f;
    return;
  }
  float l;
  if (MODE == 0) {
    float mx = -INFINITY;
    for (int64_t k = lane; k < L; k += 64) mx = fmaxf(mx, scale * row[k]);
    mx = wave_max(mx);
    float sum = 0.f;
    for (int64_t k = lane; k < L; k += 64) sum += expf(scale * row[k] - mx);
    l = mx + logf(wave_sum(sum));
    if (lane == 0) lse[r] = l;
  } else {
    l = lse[r];
  }
  for (int64_t k = lane; k < Lp; k += 64) row[k] = k < L ? expf(scale * row[k] - l) : 0.f;
}

hipError_t ragged_rows(hipStream_t s, int mode, int64_t rows, int h, int n_users, const int64_t *tgt_off,
                       const RaggedDesc *sdesc, float *S, float *S2, float scale, float *lse, const float *D) {
  if (rows <= 0) return hipSuccess;
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (mode == 0)
    hipLaunchKernelGGL(ragged_rows_kernel<0>, grid, dim3(256), 0, s, rows, h, n_users, tgt_off, sdesc, S, S2, scale,
                       lse, D);
  else if (mode == 1)
    hipLaunchKernelGGL(ragged_rows_kernel<1>, grid, dim3(256), 0, s, rows, h, n_users, tgt_off, sdesc, S, S2, scale,
                       lse, D);
  else
    hipLaunchKernelGGL(ragged_rows_kernel<2>, grid, dim3(256), 0, s, rows, h, n_users, tgt_off, sdesc, S, S2, scale,
                       lse, D);
  return hipGetLastError();
}

}  // namespace stca
