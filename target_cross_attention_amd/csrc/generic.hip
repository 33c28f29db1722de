// Plain fp32-accumulating kernels: a tiled GEMM, the SwiGLU gate, row LayerNorm.
// They carry the fp32 debug path and the small per-target projections of the bf16 path
// (eqs. (3), (6), (7) and the u-projection of eq. (13)), whose work is a few d x d
// products per target, negligible next to the per-history-token work.
#include "device_common.hpp"
#include "internal.hpp"

namespace stca {

// ------------------------------------------------------------------------------------------
// C = alpha * A B + beta * C, batched over blockIdx.z.  A: M x K (lda) or, with TRANS_A,
// A[m][k] = At[k * lda + m]; B: K x N (ldb) or, with TRANS_B, B[k][n] = Bt[n * ldb + k].  fp32
// accumulation; beta == 0 never reads C.
// ------------------------------------------------------------------------------------------
constexpr int GT = 64, GK = 16;

template <typename TA, typename TB, typename TC, bool TRANS_B, bool TRANS_A>
__global__ __launch_bounds__(256) void gemm_kernel(int M, int N, int K, const TA *__restrict__ A,
                                                   int64_t lda, int64_t sA, const TB *__restrict__ B,
                                                   int64_t ldb, int64_t sB, TC *__restrict__ C,
                                                   int64_t ldc, int64_t sC, float alpha, float beta) {
  __shared__ float As[GK][GT + 4];
  __shared__ float Bs[GK][GT + 4];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.y * GT, n0 = blockIdx.x * GT;
  A += (int64_t)blockIdx.z * sA;
  B += (int64_t)blockIdx.z * sB;
  C += (int64_t)blockIdx.z * sC;

  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

  for (int k0 = 0; k0 < K; k0 += GK) {
    // A tile: 64 rows x 16 k; thread loads 4 elements (row = tid / 4 ... spread).
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = tid + e * 256;  // 0..1023
      const int r = TRANS_A ? (idx & 63) : (idx >> 4), k = TRANS_A ? (idx >> 6) : (idx & 15);
      const int gm = m0 + r, gk = k0 + k;
      As[k][r] = (gm < M && gk < K) ? ld(TRANS_A ? A + (int64_t)gk * lda + gm : A + (int64_t)gm * lda + gk) : 0.f;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = tid + e * 256;
      int k, c;
      if (TRANS_B) {
        c = idx >> 4;
        k = idx & 15;
      } else {
        k = idx >> 6;
        c = idx & 63;
      }
      const int gk = k0 + k, gn = n0 + c;
      float v = 0.f;
      if (gk < K && gn < N) v = TRANS_B ? ld(B + (int64_t)gn * ldb + gk) : ld(B + (int64_t)gk * ldb + gn);
      Bs[k][c] = v;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < GK; ++k) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[k][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[k][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int gm = m0 + ty * 4 + i;
    if (gm >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gn = n0 + tx * 4 + j;
      if (gn >= N) continue;
      TC *p = C + (int64_t)gm * ldc + gn;
      float v = alpha * acc[i][j];
      if (beta != 0.f) v += beta * ld(p);
      st(p, v);
    }
  }
}

template <typename TA, typename TB, typename TC, bool TB_T, bool TA_T = false>
static hipError_t gemm_t(hipStream_t s, const GemmArgs &g) {
  dim3 grid((g.N + GT - 1) / GT, (g.M + GT - 1) / GT, g.batch);
  hipLaunchKernelGGL((gemm_kernel<TA, TB, TC, TB_T, TA_T>), grid, dim3(256), 0, s, g.M, g.N, g.K,
                     (const TA *)g.A, g.lda, g.sA, (const TB *)g.B, g.ldb, g.sB, (TC *)g.C, g.ldc, g.sC,
                     g.alpha, g.beta);
  return hipGetLastError();
}

hipError_t gemm(hipStream_t s, const GemmArgs &g) {
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0) return hipSuccess;
  // Dispatch on (A type, B type, C type, transB); transposed A only for fp32 outputs.
  if (g.trans_a) {
    if (g.tc_bf16 || g.tb_bf16 || g.trans_b) return hipErrorInvalidValue;
    return g.ta_bf16 ? gemm_t<bf16, float, float, false, true>(s, g) : gemm_t<float, float, float, false, true>(s, g);
  }
#define STCA_GEMM_CASE(ta, tb, tc, TA_, TB_, TC_)                                             \
  if (g.ta_bf16 == ta && g.tb_bf16 == tb && g.tc_bf16 == tc)                                   \
    return g.trans_b ? gemm_t<TA_, TB_, TC_, true>(s, g) : gemm_t<TA_, TB_, TC_, false>(s, g);
  STCA_GEMM_CASE(0, 0, 0, float, float, float)
  STCA_GEMM_CASE(0, 1, 0, float, bf16, float)
  STCA_GEMM_CASE(1, 1, 0, bf16, bf16, float)
  STCA_GEMM_CASE(0, 0, 1, float, float, bf16)
  STCA_GEMM_CASE(0, 1, 1, float, bf16, bf16)
  STCA_GEMM_CASE(1, 1, 1, bf16, bf16, bf16)
  STCA_GEMM_CASE(1, 0, 0, bf16, float, float)
#undef STCA_GEMM_CASE
  return hipErrorInvalidValue;
}

// ------------------------------------------------------------------------------------------
// SwiGLU gate in place: A[i] <- A[i] * SiLU(G[i])   (eq. (1))
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gate_kernel(int64_t n, float *__restrict__ A,
                                                   const float *__restrict__ G) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    A[i] = swiglu_gate(A[i], G[i]);
}

hipError_t swiglu_gate_inplace(hipStream_t s, int64_t n, float *A, const float *G) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(gate_kernel, dim3((unsigned)blocks), dim3(256), 0, s, n, A, G);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Row LayerNorm (biased variance, affine): one wave per row, d <= 512.
// ------------------------------------------------------------------------------------------
template <typename TO>
__global__ __launch_bounds__(256) void layernorm_kernel(int64_t rows, int d, const float *__restrict__ Y,
                                                        int64_t ldy, TO *__restrict__ out, int64_t ldo,
                                                        const float *__restrict__ gamma,
                                                        const float *__restrict__ beta, float eps) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const float *y = Y + row * ldy;
  float v[8];
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int c = lane + 64 * e;
    v[e] = (c < d) ? y[c] : 0.f;
    s += v[e];
  }
  const float mean = wave_sum(s) / (float)d;
  float q = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int c = lane + 64 * e;
    const float t = (c < d) ? v[e] - mean : 0.f;
    q += t * t;
  }
  const float inv = 1.0f / sqrtf(wave_sum(q) / (float)d + eps);
  TO *o = out + row * ldo;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int c = lane + 64 * e;
    if (c < d) st(o + c, (v[e] - mean) * inv * gamma[c] + beta[c]);
  }
}

hipError_t layernorm_rows(hipStream_t s, int64_t rows, int d, const float *Y, int64_t ldy, void *out,
                          int64_t ldo, bool out_bf16, const float *gamma, const float *beta, float eps) {
  if (rows <= 0) return hipSuccess;
  dim3 grid((unsigned)((rows + 3) / 4));
  if (out_bf16)
    hipLaunchKernelGGL(layernorm_kernel<bf16>, grid, dim3(256), 0, s, rows, d, Y, ldy, (bf16 *)out, ldo,
                       gamma, beta, eps);
  else
    hipLaunchKernelGGL(layernorm_kernel<float>, grid, dim3(256), 0, s, rows, d, Y, ldy, (float *)out, ldo,
                       gamma, beta, eps);
  return hipGetLastError();
}

// dst[i] = bf16(src[i]) (round to nearest even), four elements per thread.
__global__ __launch_bounds__(256) void to_bf16_kernel(int64_t n4, const f32x4 *__restrict__ src,
                                                      bf16x4 *__restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n4) return;
  const f32x4 v = src[i];
  dst[i] = bf16x4{f32_to_bf16(v[0]), f32_to_bf16(v[1]), f32_to_bf16(v[2]), f32_to_bf16(v[3])};
}

hipError_t to_bf16(hipStream_t s, int64_t n, const float *src, void *dst) {
  if (n <= 0) return hipSuccess;
  if (n % 4) return hipErrorInvalidValue;
  const int64_t n4 = n / 4;
  hipLaunchKernelGGL(to_bf16_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, n4, (const f32x4 *)src,
                     (bf16x4 *)dst);
  return hipGetLastError();
}

}  // namespace stca
