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

// Column sums in two fixed-order stages: parts[b][c] = sum of rows b*rows_per .. of column c.
__global__ __launch_bounds__(256) void colsum_parts_kernel(int64_t rows, int cols, const float *__restrict__ A,
                                                           int64_t lda, int64_t rows_per, float *__restrict__ parts) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= cols) return;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per;
  const int64_t r1 = r0 + rows_per < rows ? r0 + rows_per : rows;
  float acc = 0.f;
  for (int64_t r = r0; r < r1; ++r) acc += A[r * lda + c];
  parts[(int64_t)blockIdx.y * cols + c] = acc;
}

hipError_t colsum(hipStream_t s, int64_t rows, int cols, const float *A, int64_t lda, float *parts, int max_parts,
                  float *out) {
  if (rows <= 0) return hipSuccess;
  int nparts = (int)((rows + 255) / 256);
  if (nparts > max_parts) nparts = max_parts;
  const int64_t per = (rows + nparts - 1) / nparts;
  nparts = (int)((rows + per - 1) / per);
  hipLaunchKernelGGL(colsum_parts_kernel, dim3((unsigned)((cols + 255) / 256), (unsigned)nparts), dim3(256), 0, s,
                     rows, cols, A, lda, per, parts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return sum_parts(s, cols, nparts, parts, out, true);
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

// ---- LayerNorm derivative: one wave per row (d <= 512) -----------------------------------------
// From the pre-LN rows Y: xh = (y - mean) rstd; dxh = dout gamma;
// dY = rstd (dxh - mean(dxh) - xh mean(dxh xh)); Pg = dout xh (rows summed later into dgamma).
__global__ __launch_bounds__(256) void ln_bwd_kernel(int64_t rows, int d, const float *__restrict__ dout,
                                                     int64_t ldd, const float *__restrict__ Y, int64_t ldy,
                                                     const float *__restrict__ gamma, float eps,
                                                     float *__restrict__ dY, float *__restrict__ Pg) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  float y[8], g[8];
  float sum = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int c = lane + 64 * e;
    y[e] = c < d ? Y[row * ldy + c] : 0.f;
    sum += y[e];
  }
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
      const float xh = (y[e] - mean) * rstd, go = dout[row * ldd + c];
      g[e] = go * gamma[c];
      s1 += g[e];
      s2 += g[e] * xh;
      Pg[row * d + c] = go * xh;
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

hipError_t ln_bwd(hipStream_t s, int64_t rows, int d, const float *dout, int64_t ldd, const float *Y, int64_t ldy,
                  const float *gamma, float eps, float *dY, float *Pg) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(ln_bwd_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, rows, d, dout, ldd, Y, ldy,
                     gamma, eps, dY, Pg);
  return hipGetLastError();
}

// ---- attention softmax and its derivative (rows of S are one query row each) -------------------
// Per row r (one wave): with s = scale * S[r][:], lse = max + log(sum exp(s - max)); S[r][:] is
// replaced by alpha = exp(s - lse).
__global__ __launch_bounds__(256) void softmax_rows_kernel(int R, int L, float *__restrict__ S, int64_t lds,
                                                           float scale, float *__restrict__ lse) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= R) return;
  float *row = S + (int64_t)r * lds;
  float mx = -INFINITY;
  for (int k = lane; k < L; k += 64) mx = fmaxf(mx, scale * row[k]);
  mx = wave_max(mx);
  float sum = 0.f;
  for (int k = lane; k < L; k += 64) sum += expf(scale * row[k] - mx);
  const float l = mx + logf(wave_sum(sum));
  for (int k = lane; k < L; k += 64) row[k] = expf(scale * row[k] - l);
  if (lane == 0) lse[r] = l;
}

hipError_t softmax_rows(hipStream_t s, int R, int L, float *S, int64_t lds, float scale, float *lse) {
  if (R <= 0 || L <= 0) return hipSuccess;
  hipLaunchKernelGGL(softmax_rows_kernel, dim3((unsigned)((R + 3) / 4)), dim3(256), 0, s, R, L, S, lds, scale, lse);
  return hipGetLastError();
}

// S[r][k] <- exp(scale * S[r][k] - lse[r]) (the saved softmax).
__global__ __launch_bounds__(256) void softmax_apply_kernel(int R, int L, float *__restrict__ S, int64_t lds,
                                                            float scale, const float *__restrict__ lse) {
  const int64_t n = (int64_t)R * L;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int r = (int)(i / L), k = (int)(i % L);
    S[(int64_t)r * lds + k] = expf(scale * S[(int64_t)r * lds + k] - lse[r]);
  }
}

hipError_t softmax_apply(hipStream_t s, int R, int L, float *S, int64_t lds, float scale, const float *lse) {
  if (R <= 0 || L <= 0) return hipSuccess;
  hipLaunchKernelGGL(softmax_apply_kernel, dim3(grid_for((int64_t)R * L)), dim3(256), 0, s, R, L, S, lds, scale, lse);
  return hipGetLastError();
}

// dS[r][k] = alpha[r][k] (dA[r][k] - D[r]), in place over dA.
__global__ __launch_bounds__(256) void softmax_bwd_kernel(int R, int L, const float *__restrict__ alpha,
                                                          float *__restrict__ dA, int64_t ld,
                                                          const float *__restrict__ D) {
  const int64_t n = (int64_t)R * L;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int r = (int)(i / L), k = (int)(i % L);
    const int64_t o = (int64_t)r * ld + k;
    dA[o] = alpha[o] * (dA[o] - D[r]);
  }
}

hipError_t softmax_bwd(hipStream_t s, int R, int L, const float *alpha, float *dA, int64_t ld, const float *D) {
  if (R <= 0 || L <= 0) return hipSuccess;
  hipLaunchKernelGGL(softmax_bwd_kernel, dim3(grid_for((int64_t)R * L)), dim3(256), 0, s, R, L, alpha, dA, ld, D);
  return hipGetLastError();
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

// ---- attention over a user's history, fp32 (eq. (13) and its derivative) ---------------------
// Query rows r = t h + j (target t, head j) with u_r = U[r] (unscaled: the score of history row k
// is scale * u_r . X~_k, scale = 1/sqrt(d_h)); history rows of target t's user are hist_off[u] ..
// hist_off[u+1]-1.  Each wave takes up to RW heads of one target (so all its rows share a user);
// lane l holds features l + 64 e, e < DPL = d / 64.

// Largest u in [0, n) with off[u] <= x (off nondecreasing, off[0] = 0 <= x < off[n]).
__device__ __forceinline__ int segment_of(const int64_t *__restrict__ off, int n, int64_t x) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <int DPL>
__device__ __forceinline__ void load_row(float (&v)[DPL], const float *__restrict__ p, int lane) {
#pragma unroll
  for (int e = 0; e < DPL; ++e) v[e] = p[lane + 64 * e];
}

template <int DPL>
__device__ __forceinline__ float dot_row(const float (&a)[DPL], const float (&b)[DPL]) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < DPL; ++e) s = fmaf(a[e], b[e], s);
  return s;
}

// Softmax statistics and weighted history: abar_r = sum_k alpha_rk X~_k, lse_r = log sum_k e^{s_rk}.
template <int DPL, int RW>
__global__ __launch_bounds__(256) void attn_fwd_rows_kernel(int64_t T, int h, int n_users,
                                                            const int64_t *__restrict__ hist_off,
                                                            const int64_t *__restrict__ tgt_off,
                                                            const float *__restrict__ Xt, const float *__restrict__ U,
                                                            float scale, float *__restrict__ abar,
                                                            float *__restrict__ lse) {
  constexpr int d = 64 * DPL;
  const int lane = threadIdx.x & 63;
  const int groups = (h + RW - 1) / RW;
  const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t t = gw / groups;
  if (t >= T) return;
  const int j0 = (int)(gw % groups) * RW;
  const int u = segment_of(tgt_off, n_users, t);
  const int64_t k0 = hist_off[u], k1 = hist_off[u + 1];
  float q[RW][DPL], acc[RW][DPL], m[RW], l[RW];
#pragma unroll
  for (int rr = 0; rr < RW; ++rr) {
    const int j = j0 + rr < h ? j0 + rr : h - 1;
    load_row<DPL>(q[rr], U + (t * h + j) * d, lane);
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[rr][e] = 0.f;
    m[rr] = -INFINITY;
    l[rr] = 0.f;
  }
  for (int64_t k = k0; k < k1; ++k) {
    float x[DPL];
    load_row<DPL>(x, Xt + k * d, lane);
#pragma unroll
    for (int rr = 0; rr < RW; ++rr) {
      const float s = scale * wave_sum(dot_row<DPL>(q[rr], x));
      const float mn = fmaxf(m[rr], s);
      const float c = expf(m[rr] - mn), p = expf(s - mn);
      l[rr] = l[rr] * c + p;
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[rr][e] = fmaf(acc[rr][e], c, p * x[e]);
      m[rr] = mn;
    }
  }
#pragma unroll
  for (int rr = 0; rr < RW; ++rr) {
    if (j0 + rr >= h) continue;
    const int64_t r = t * h + j0 + rr;
    const float inv = 1.0f / l[rr];
#pragma unroll
    for (int e = 0; e < DPL; ++e) abar[r * d + lane + 64 * e] = acc[rr][e] * inv;
    if (lane == 0) lse[r] = m[rr] + logf(l[rr]);
  }
}

// du_r = scale sum_k dS_rk X~_k with alpha_rk = exp(scale u_r . X~_k - lse_r),
// dS_rk = alpha_rk (dabar_r . X~_k - D_r), D_r = dabar_r . abar_r.
template <int DPL, int RW>
__global__ __launch_bounds__(256) void attn_bwd_query_kernel(int64_t T, int h, int n_users,
                                                             const int64_t *__restrict__ hist_off,
                                                             const int64_t *__restrict__ tgt_off,
                                                             const float *__restrict__ Xt, const float *__restrict__ U,
                                                             const float *__restrict__ dabar,
                                                             const float *__restrict__ lse,
                                                             const float *__restrict__ D, float scale,
                                                             float *__restrict__ du) {
  constexpr int d = 64 * DPL;
  const int lane = threadIdx.x & 63;
  const int groups = (h + RW - 1) / RW;
  const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t t = gw / groups;
  if (t >= T) return;
  const int j0 = (int)(gw % groups) * RW;
  const int u = segment_of(tgt_off, n_users, t);
  const int64_t k0 = hist_off[u], k1 = hist_off[u + 1];
  float q[RW][DPL], g[RW][DPL], acc[RW][DPL], ls[RW], Dr[RW];
#pragma unroll
  for (int rr = 0; rr < RW; ++rr) {
    const int j = j0 + rr < h ? j0 + rr : h - 1;
    const int64_t r = t * h + j;
    load_row<DPL>(q[rr], U + r * d, lane);
    load_row<DPL>(g[rr], dabar + r * d, lane);
    ls[rr] = lse[r];
    Dr[rr] = D[r];
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[rr][e] = 0.f;
  }
  for (int64_t k = k0; k < k1; ++k) {
    float x[DPL];
    load_row<DPL>(x, Xt + k * d, lane);
#pragma unroll
    for (int rr = 0; rr < RW; ++rr) {
      const float a = wave_sum(dot_row<DPL>(q[rr], x)), b = wave_sum(dot_row<DPL>(g[rr], x));
      const float ds = expf(scale * a - ls[rr]) * (b - Dr[rr]);
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[rr][e] = fmaf(ds, x[e], acc[rr][e]);
    }
  }
#pragma unroll
  for (int rr = 0; rr < RW; ++rr) {
    if (j0 + rr >= h) continue;
    const int64_t r = t * h + j0 + rr;
#pragma unroll
    for (int e = 0; e < DPL; ++e) du[r * d + lane + 64 * e] = scale * acc[rr][e];
  }
}

// dX~_k = sum over the (t, j) rows of k's user of alpha_rk dabar_r + scale dS_rk u_r.
// A wave takes RK consecutive history rows (which may belong to up to RK users).
template <int DPL, int RK>
__global__ __launch_bounds__(256) void attn_bwd_keys_kernel(int64_t L, int h, int n_users,
                                                            const int64_t *__restrict__ hist_off,
                                                            const int64_t *__restrict__ tgt_off,
                                                            const float *__restrict__ Xt, const float *__restrict__ U,
                                                            const float *__restrict__ dabar,
                                                            const float *__restrict__ lse,
                                                            const float *__restrict__ D, float scale,
                                                            float *__restrict__ dXt) {
  constexpr int d = 64 * DPL;
  const int lane = threadIdx.x & 63;
  const int64_t k0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * RK;
  if (k0 >= L) return;
  float x[RK][DPL], acc[RK][DPL];
  int usr[RK];
#pragma unroll
  for (int kk = 0; kk < RK; ++kk) {
    const int64_t k = k0 + kk < L ? k0 + kk : L - 1;
    load_row<DPL>(x[kk], Xt + k * d, lane);
    usr[kk] = k0 + kk < L ? segment_of(hist_off, n_users, k) : -1;
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[kk][e] = 0.f;
  }
  for (int first = 0; first < RK;) {  // the rows of one user at a time (users grow with k)
    const int u = usr[first];
    if (u < 0) break;
    int last = first;
    while (last + 1 < RK && usr[last + 1] == u) ++last;
    const int64_t r0 = tgt_off[u] * h, r1 = tgt_off[u + 1] * h;
    for (int64_t r = r0; r < r1; ++r) {
      float q[DPL], g[DPL];
      load_row<DPL>(q, U + r * d, lane);
      load_row<DPL>(g, dabar + r * d, lane);
      const float ls = lse[r], Dr = D[r];
#pragma unroll
      for (int kk = 0; kk < RK; ++kk) {
        if (kk < first || kk > last) continue;
        const float a = wave_sum(dot_row<DPL>(q, x[kk])), b = wave_sum(dot_row<DPL>(g, x[kk]));
        const float al = expf(scale * a - ls), ds = scale * al * (b - Dr);
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[kk][e] = fmaf(al, g[e], fmaf(ds, q[e], acc[kk][e]));
      }
    }
    first = last + 1;
  }
#pragma unroll
  for (int kk = 0; kk < RK; ++kk) {
    if (k0 + kk >= L) continue;
#pragma unroll
    for (int e = 0; e < DPL; ++e) dXt[(k0 + kk) * d + lane + 64 * e] = acc[kk][e];
  }
}

template <int DPL>
static hipError_t attn_bwd_launch(hipStream_t s, int which, int64_t T, int64_t L, int h, int n_users,
                                  const int64_t *hist_off, const int64_t *tgt_off, const float *Xt, const float *U,
                                  const float *dabar, float *abar, float *lse, const float *D, float scale,
                                  float *out) {
  constexpr int RW = DPL >= 8 ? 2 : 4, RK = 4;
  if (which == 2) {
    const int64_t waves = (L + RK - 1) / RK;
    if (waves == 0) return hipSuccess;
    hipLaunchKernelGGL((attn_bwd_keys_kernel<DPL, RK>), dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, L, h,
                       n_users, hist_off, tgt_off, Xt, U, dabar, lse, D, scale, out);
    return hipGetLastError();
  }
  const int64_t waves = T * ((h + RW - 1) / RW);
  if (waves == 0) return hipSuccess;
  const dim3 grid((unsigned)((waves + 3) / 4));
  if (which == 0)
    hipLaunchKernelGGL((attn_fwd_rows_kernel<DPL, RW>), grid, dim3(256), 0, s, T, h, n_users, hist_off, tgt_off, Xt,
                       U, scale, abar, lse);
  else
    hipLaunchKernelGGL((attn_bwd_query_kernel<DPL, RW>), grid, dim3(256), 0, s, T, h, n_users, hist_off, tgt_off, Xt,
                       U, dabar, lse, D, scale, out);
  return hipGetLastError();
}

static hipError_t attn_bwd_dispatch(hipStream_t s, int which, int d, int64_t T, int64_t L, int h, int n_users,
                                    const int64_t *hist_off, const int64_t *tgt_off, const float *Xt, const float *U,
                                    const float *dabar, float *abar, float *lse, const float *D, float scale,
                                    float *out) {
  switch (d) {
    case 64: return attn_bwd_launch<1>(s, which, T, L, h, n_users, hist_off, tgt_off, Xt, U, dabar, abar, lse, D, scale, out);
    case 128: return attn_bwd_launch<2>(s, which, T, L, h, n_users, hist_off, tgt_off, Xt, U, dabar, abar, lse, D, scale, out);
    case 256: return attn_bwd_launch<4>(s, which, T, L, h, n_users, hist_off, tgt_off, Xt, U, dabar, abar, lse, D, scale, out);
    case 512: return attn_bwd_launch<8>(s, which, T, L, h, n_users, hist_off, tgt_off, Xt, U, dabar, abar, lse, D, scale, out);
    default: return hipErrorInvalidValue;
  }
}

hipError_t attn_rows_fwd(hipStream_t s, int d, int h, int n_users, const int64_t *hist_off, const int64_t *tgt_off,
                         int64_t T, const float *Xt, const float *U, float scale, float *abar, float *lse) {
  return attn_bwd_dispatch(s, 0, d, T, 0, h, n_users, hist_off, tgt_off, Xt, U, nullptr, abar, lse, nullptr, scale,
                           nullptr);
}

hipError_t attn_rows_bwd_query(hipStream_t s, int d, int h, int n_users, const int64_t *hist_off,
                               const int64_t *tgt_off, int64_t T, const float *Xt, const float *U,
                               const float *dabar, const float *lse, const float *D, float scale, float *du) {
  return attn_bwd_dispatch(s, 1, d, T, 0, h, n_users, hist_off, tgt_off, Xt, U, dabar, nullptr, (float *)lse, D,
                           scale, du);
}

hipError_t attn_rows_bwd_keys(hipStream_t s, int d, int h, int n_users, const int64_t *hist_off,
                              const int64_t *tgt_off, int64_t L, const float *Xt, const float *U,
                              const float *dabar, const float *lse, const float *D, float scale, float *dXt) {
  return attn_bwd_dispatch(s, 2, d, 0, L, h, n_users, hist_off, tgt_off, Xt, U, dabar, nullptr, (float *)lse, D,
                           scale, dXt);
}

}  // namespace stca
