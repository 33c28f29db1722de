// fp32-accumulating kernels: a tiled GEMM in two forms (vector ALU; fp32 matrix cores, also for
// ragged per-user batches), the SwiGLU gate, row LayerNorm, bf16 conversion.  They carry the fp32
// debug path, the small per-target projections of the bf16 path (eqs. (3), (6), (7) and the
// u-projection of eq. (13), a few d x d products per target, negligible next to the
// per-history-token work) and every product of the backward pass.
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

// ------------------------------------------------------------------------------------------
// The same product on fp32 matrix cores (v_mfma_f32_32x32x2_f32: exact fp32 products, fp32
// accumulation), for fp32 outputs.  128 x 128 output tile per workgroup, four waves of 64 x 64
// (2 x 2 MFMA blocks of 32 x 32), k in steps of 16 through double-buffered LDS tiles stored
// k-contiguous ([row][k], rows padded to 20 floats so the 16-byte fragment reads of 8 lanes fall in
// distinct banks).  Within a step, lane group g = lane / 32 of MFMA j covers k = 8 g + j, so a
// lane's 8 operands of a step are two 16-byte LDS reads.  Operands are read from global memory
// 4 consecutive elements at a time along their contiguous dimension (rows of A, or of At with
// TRANS_A; of Bt with TRANS_B, or of B): that dimension's length and leading dimension must be
// multiples of 4 and the base 16-byte (fp32) or 8-byte (bf16) aligned (see mfma_ok).
// ------------------------------------------------------------------------------------------
constexpr int MT = 128, MK = 16, MKP = 20;

template <typename T> struct vec4_of;
template <> struct vec4_of<float> {
  __device__ __forceinline__ static f32x4 load(const float *p) { return *(const f32x4 *)p; }
};
template <> struct vec4_of<bf16> {
  __device__ __forceinline__ static f32x4 load(const bf16 *p) {
    const u32x2 w = *(const u32x2 *)p;
    return f32x4{__builtin_bit_cast(float, w[0] << 16), __builtin_bit_cast(float, w[0] & 0xffff0000u),
                 __builtin_bit_cast(float, w[1] << 16), __builtin_bit_cast(float, w[1] & 0xffff0000u)};
  }
};

// One operand tile (TT rows x 16 k, TT = 128 or 64) of a K-step, in registers between its global
// load and its LDS store.  KCONT: the operand's k index is contiguous in memory (element (row, k) at
// P[row * ld + k]); otherwise rows are (element (row, k) at P[k * ld + row]).
template <typename T, bool KCONT, int TT = MT> struct TileLoader {
  f32x4 v[2];
  __device__ __forceinline__ void load(const T *__restrict__ P, int64_t ld, int rows, int K, int r0, int k0,
                                       int tid) {
    if constexpr (KCONT) {
#pragma unroll
      for (int e = 0; e < TT / 64; ++e) {
        const int r = (tid >> 2) + 64 * e, k = k0 + (tid & 3) * 4;
        v[e] = (r0 + r < rows && k < K) ? vec4_of<T>::load(P + (int64_t)(r0 + r) * ld + k) : f32x4{0, 0, 0, 0};
      }
    } else if constexpr (TT == 128) {  // a 2 (k) x 4 (rows) block per thread: k = 2 (tid >> 5) + e, rows 4 (tid & 31) ..
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int k = k0 + 2 * (tid >> 5) + e, r = r0 + (tid & 31) * 4;
        v[e] = (k < K && r < rows) ? vec4_of<T>::load(P + (int64_t)k * ld + r) : f32x4{0, 0, 0, 0};
      }
    } else {  // 64 rows: one k, rows 4 (tid & 15) .. per thread
      const int k = k0 + (tid >> 4), r = r0 + (tid & 15) * 4;
      v[0] = (k < K && r < rows) ? vec4_of<T>::load(P + (int64_t)k * ld + r) : f32x4{0, 0, 0, 0};
    }
  }
  __device__ __forceinline__ void store(float (*S)[MKP], int tid) const {
    if constexpr (KCONT) {
#pragma unroll
      for (int e = 0; e < TT / 64; ++e) *(f32x4 *)&S[(tid >> 2) + 64 * e][(tid & 3) * 4] = v[e];
    } else if constexpr (TT == 128) {  // transposed in registers: row r + i gets (k, k + 1) as one 8-byte store
      const int k = 2 * (tid >> 5), r = (tid & 31) * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
        *(f32x2 *)&S[r + i][k] = f32x2{v[0][i], v[1][i]};
      }
    } else {
      const int k = tid >> 4, r = (tid & 15) * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) S[r + i][k] = v[0][i];
    }
  }
};

// RAGGED: blockIdx.z picks a descriptor (one per user of a ragged batch) that gives the product's
// sizes, element offsets and leading dimensions; blocks outside that user's tiles return at once.
// TT: output tile TT x TT (128, or 64 for products with too few 128 x 128 tiles to fill the chip);
// each of the four waves holds (TT/2) x (TT/2), TT/64 x TT/64 MFMA blocks.
template <typename TA, typename TB, bool TRANS_B, bool TRANS_A, bool RAGGED, int TT = MT>
__global__ __launch_bounds__(256) void gemm_mfma_kernel(int M, int N, int K, const TA *__restrict__ A, int64_t lda,
                                                        int64_t sA, const TB *__restrict__ B, int64_t ldb,
                                                        int64_t sB, float *__restrict__ C, int64_t ldc, int64_t sC,
                                                        float alpha, float beta,
                                                        const RaggedDesc *__restrict__ descs) {
  constexpr int BW = TT / 64;  // MFMA blocks per wave along each dimension
  __shared__ __attribute__((aligned(16))) float As[2][TT][MKP];
  __shared__ __attribute__((aligned(16))) float Bs[2][TT][MKP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m0 = blockIdx.y * TT, n0 = blockIdx.x * TT;
  if constexpr (RAGGED) {
    const RaggedDesc dsc = descs[blockIdx.z];
    M = dsc.M;
    N = dsc.N;
    K = dsc.K;
    if (m0 >= M || n0 >= N) return;
    A += dsc.a_off;
    lda = dsc.lda;
    B += dsc.b_off;
    ldb = dsc.ldb;
    C += dsc.c_off;
    ldc = dsc.ldc;
  } else {
    A += (int64_t)blockIdx.z * sA;
    B += (int64_t)blockIdx.z * sB;
    C += (int64_t)blockIdx.z * sC;
  }
  TileLoader<TA, !TRANS_A, TT> la;  // A (row m, k): k-contiguous unless transposed
  TileLoader<TB, TRANS_B, TT> lb;   // B as (row n, k): k-contiguous only when transposed
  f32x16 acc[BW][BW];
#pragma unroll
  for (int i = 0; i < BW; ++i)
#pragma unroll
    for (int j = 0; j < BW; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int wm = (wave >> 1) * (TT / 2), wn = (wave & 1) * (TT / 2), g8 = (lane >> 5) * 8, lr = lane & 31;
  la.load(A, lda, M, K, m0, 0, tid);
  lb.load(B, ldb, N, K, n0, 0, tid);
  la.store(As[0], tid);
  lb.store(Bs[0], tid);
  __syncthreads();
  const int steps = (K + MK - 1) / MK;
  for (int st = 0; st < steps; ++st) {
    const int cur = st & 1;
    const bool more = st + 1 < steps;
    if (more) {
      la.load(A, lda, M, K, m0, (st + 1) * MK, tid);
      lb.load(B, ldb, N, K, n0, (st + 1) * MK, tid);
    }
    f32x4 a[BW][2], b[BW][2];
#pragma unroll
    for (int i = 0; i < BW; ++i) {
      a[i][0] = *(const f32x4 *)&As[cur][wm + 32 * i + lr][g8];
      a[i][1] = *(const f32x4 *)&As[cur][wm + 32 * i + lr][g8 + 4];
      b[i][0] = *(const f32x4 *)&Bs[cur][wn + 32 * i + lr][g8];
      b[i][1] = *(const f32x4 *)&Bs[cur][wn + 32 * i + lr][g8 + 4];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int bi = 0; bi < BW; ++bi)
#pragma unroll
        for (int bj = 0; bj < BW; ++bj)
          acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[bi][j >> 2][j & 3], b[bj][j >> 2][j & 3],
                                                             acc[bi][bj], 0, 0, 0);
    if (more) {
      la.store(As[cur ^ 1], tid);
      lb.store(Bs[cur ^ 1], tid);
    }
    __syncthreads();
  }
  // D layout: lane holds column lr; register e holds row 8 (e >> 2) + 4 (lane >> 5) + (e & 3).
#pragma unroll
  for (int bi = 0; bi < BW; ++bi)
#pragma unroll
    for (int bj = 0; bj < BW; ++bj) {
      const int col = n0 + wn + 32 * bj + lr;
      if (col >= N) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm + 32 * bi + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        if (row >= M) continue;
        float *p = C + (int64_t)row * ldc + col;
        float v = alpha * acc[bi][bj][e];
        if (beta != 0.f) v += beta * *p;
        *p = v;
      }
    }
}

// 128 x 128 tiles, or 64 x 64 where 128 x 128 tiles would give the chip's 256 compute units fewer
// than four workgroups each.
template <typename TA, typename TB, bool TB_T, bool TA_T>
static hipError_t gemm_mfma_t(hipStream_t s, const GemmArgs &g) {
  const int64_t tiles = (int64_t)((g.N + MT - 1) / MT) * ((g.M + MT - 1) / MT) * g.batch;
  if (tiles < 1024) {
    dim3 grid((g.N + 63) / 64, (g.M + 63) / 64, g.batch);
    hipLaunchKernelGGL((gemm_mfma_kernel<TA, TB, TB_T, TA_T, false, 64>), grid, dim3(256), 0, s, g.M, g.N, g.K,
                       (const TA *)g.A, g.lda, g.sA, (const TB *)g.B, g.ldb, g.sB, (float *)g.C, g.ldc, g.sC, g.alpha,
                       g.beta, nullptr);
  } else {
    dim3 grid((g.N + MT - 1) / MT, (g.M + MT - 1) / MT, g.batch);
    hipLaunchKernelGGL((gemm_mfma_kernel<TA, TB, TB_T, TA_T, false>), grid, dim3(256), 0, s, g.M, g.N, g.K,
                       (const TA *)g.A, g.lda, g.sA, (const TB *)g.B, g.ldb, g.sB, (float *)g.C, g.ldc, g.sC, g.alpha,
                       g.beta, nullptr);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// The ragged products of the mixed-precision backward on bf16 matrix cores: fp32 operands are rounded
// to bf16 as they are staged into LDS (v_mfma_f32_32x32x16_bf16, fp32 accumulation and output).
// 128 x 128 output tile per workgroup, four waves of 64 x 64, k in steps of 32 through
// double-buffered LDS tiles [row][k] of 32 bf16 padded to 40 (80-byte rows: the 16-byte fragment
// reads of 16 consecutive rows fall in 64 distinct banks).  Lane group g of a 16-deep k-substep
// holds k = 8 g .. 8 g + 7 of its row, as in the bf16 GEMMs above.
// ------------------------------------------------------------------------------------------
constexpr int XK = 32, XKP = 40;

// 128 rows x 32 k of an fp32 operand between its global load and its LDS store.  KCONT: element
// (row, k) at P[row * ld + k]; otherwise at P[k * ld + row].  K and ld multiples of 4.
template <bool KCONT> struct MixedTile {
  f32x4 v[4];
  // Unconditional loads, so that the compiler can count them: a row chunk past `rows` or a k past K
  // reads the last chunk that the bounds allow (the same addresses the bounded form reads), and the
  // values at k >= K are zeroed in store().  Rows past `rows` feed outputs that are never written.
  __device__ __forceinline__ void load(const float *__restrict__ P, int64_t ld, int rows, int K, int r0, int k0,
                                       int tid) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (KCONT) {
        const int r = min(r0 + (tid >> 3) + 32 * e, rows - 1), k = min(k0 + (tid & 7) * 4, (K - 1) & ~3);
        v[e] = *(const f32x4 *)(P + (int64_t)r * ld + k);
      } else {
        const int k = min(k0 + (tid >> 5) + 8 * e, K - 1), r = min(r0 + (tid & 31) * 4, (rows - 1) & ~3);
        v[e] = *(const f32x4 *)(P + (int64_t)k * ld + r);
      }
    }
  }
  // The bounded form: lanes whose chunk lies past `rows` or K skip the load and hold zeros.
  __device__ __forceinline__ void load_bounded(const float *__restrict__ P, int64_t ld, int rows, int K, int r0,
                                               int k0, int tid) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (KCONT) {
        const int r = (tid >> 3) + 32 * e, k = k0 + (tid & 7) * 4;
        v[e] = (r0 + r < rows && k < K) ? *(const f32x4 *)(P + (int64_t)(r0 + r) * ld + k) : f32x4{0, 0, 0, 0};
      } else {
        const int k = k0 + (tid >> 5) + 8 * e, r = r0 + (tid & 31) * 4;
        v[e] = (k < K && r < rows) ? *(const f32x4 *)(P + (int64_t)k * ld + r) : f32x4{0, 0, 0, 0};
      }
    }
  }
  __device__ __forceinline__ void store(uint16_t (*S)[XKP], int tid, int K, int k0) {
    if (k0 + XK > K) {  // the last slab: zero every value at k >= K
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (KCONT) {
          const int k = k0 + (tid & 7) * 4;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (k + i >= K) v[e][i] = 0.f;
        } else if (k0 + (tid >> 5) + 8 * e >= K) {
          v[e] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (KCONT) {
        const int r = (tid >> 3) + 32 * e, k = (tid & 7) * 4;
        const uint32_t lo = (uint32_t)f32_to_bf16_bits(v[e][0]) | ((uint32_t)f32_to_bf16_bits(v[e][1]) << 16);
        const uint32_t hi = (uint32_t)f32_to_bf16_bits(v[e][2]) | ((uint32_t)f32_to_bf16_bits(v[e][3]) << 16);
        *(uint2 *)&S[r][k] = make_uint2(lo, hi);
      } else {
        const int k = (tid >> 5) + 8 * e, r = (tid & 31) * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) S[r + i][k] = f32_to_bf16_bits(v[e][i]);
      }
    }
  }
};

// PIPE: two register sets per operand: the slab of step s + 2 is loaded during step s and stored at
// the end of step s + 1.  The main loop runs steps in pairs while both of its loads are in range, with
// no conditional load, store or exit inside, so the compiler waits only for the set it stores; the
// last one to three steps follow with plain conditions.  Otherwise one set, loaded one step ahead with
// bounded loads: fewer registers and more workgroups per compute unit, which serves products whose k
// range is a few steps (the history-side products, k = a user's query rows).
template <bool TRANS_B, bool TRANS_A, bool PIPE>
__global__ __launch_bounds__(256) void gemm_mixed_ragged_kernel(const float *__restrict__ A, const float *__restrict__ B,
                                                                float *__restrict__ C, float alpha, float beta,
                                                                const RaggedDesc *__restrict__ descs) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][MT][XKP];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][MT][XKP];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m0 = blockIdx.y * MT, n0 = blockIdx.x * MT;
  const RaggedDesc dsc = descs[blockIdx.z];
  const int M = dsc.M, N = dsc.N, K = dsc.K;
  if (m0 >= M || n0 >= N) return;
  A += dsc.a_off;
  B += dsc.b_off;
  C += dsc.c_off;
  MixedTile<!TRANS_A> la0, la1;  // A (row m, k): k-contiguous unless transposed
  MixedTile<TRANS_B> lb0, lb1;   // B as (row n, k): k-contiguous only when transposed
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64, g8 = (lane >> 5) * 8, lr = lane & 31;
  auto compute = [&](int cur) {
#pragma unroll
    for (int kk = 0; kk < XK / 16; ++kk) {
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        a[i] = *(const bf16x8 *)&As[cur][wm + 32 * i + lr][16 * kk + g8];
        b[i] = *(const bf16x8 *)&Bs[cur][wn + 32 * i + lr][16 * kk + g8];
      }
#pragma unroll
      for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj) acc[bi][bj] = mfma32x32x16(a[bi], b[bj], acc[bi][bj]);
    }
  };
  const int steps = (K + XK - 1) / XK;
  if (!PIPE) {
    la0.load_bounded(A, dsc.lda, M, K, m0, 0, tid);
    lb0.load_bounded(B, dsc.ldb, N, K, n0, 0, tid);
    la0.store(As[0], tid, K, 0);
    lb0.store(Bs[0], tid, K, 0);
    __syncthreads();
    for (int st = 0; st < steps; ++st) {
      const int cur = st & 1;
      const bool more = st + 1 < steps;
      if (more) {
        la0.load_bounded(A, dsc.lda, M, K, m0, (st + 1) * XK, tid);
        lb0.load_bounded(B, dsc.ldb, N, K, n0, (st + 1) * XK, tid);
      }
      compute(cur);
      if (more) {
        la0.store(As[cur ^ 1], tid, K, (st + 1) * XK);
        lb0.store(Bs[cur ^ 1], tid, K, (st + 1) * XK);
      }
      __syncthreads();
    }
  } else if (steps > 0) {
    la0.load(A, dsc.lda, M, K, m0, 0, tid);
    lb0.load(B, dsc.ldb, N, K, n0, 0, tid);
    la0.store(As[0], tid, K, 0);
    lb0.store(Bs[0], tid, K, 0);
    if (steps > 1) {
      la1.load(A, dsc.lda, M, K, m0, XK, tid);
      lb1.load(B, dsc.ldb, N, K, n0, XK, tid);
    }
    __syncthreads();
    int st = 0;
    for (; st + 3 < steps; st += 2) {
      la0.load(A, dsc.lda, M, K, m0, (st + 2) * XK, tid);
      lb0.load(B, dsc.ldb, N, K, n0, (st + 2) * XK, tid);
      compute(0);
      la1.store(As[1], tid, K, (st + 1) * XK);
      lb1.store(Bs[1], tid, K, (st + 1) * XK);
      __syncthreads();
      la1.load(A, dsc.lda, M, K, m0, (st + 3) * XK, tid);
      lb1.load(B, dsc.ldb, N, K, n0, (st + 3) * XK, tid);
      compute(1);
      la0.store(As[0], tid, K, (st + 2) * XK);
      lb0.store(Bs[0], tid, K, (st + 2) * XK);
      __syncthreads();
    }
    // slab st in LDS half 0, slab st + 1 (if any) in register set 1
    const int left = steps - st;
    if (left > 2) {
      la0.load(A, dsc.lda, M, K, m0, (st + 2) * XK, tid);
      lb0.load(B, dsc.ldb, N, K, n0, (st + 2) * XK, tid);
    }
    compute(0);
    if (left > 1) {
      la1.store(As[1], tid, K, (st + 1) * XK);
      lb1.store(Bs[1], tid, K, (st + 1) * XK);
      __syncthreads();
      compute(1);
      if (left > 2) {
        la0.store(As[0], tid, K, (st + 2) * XK);
        lb0.store(Bs[0], tid, K, (st + 2) * XK);
        __syncthreads();
        compute(0);
      }
    }
  }
#pragma unroll
  for (int bi = 0; bi < 2; ++bi)
#pragma unroll
    for (int bj = 0; bj < 2; ++bj) {
      const int col = n0 + wn + 32 * bj + lr;
      if (col >= N) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm + 32 * bi + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        if (row >= M) continue;
        float *p = C + (int64_t)row * dsc.ldc + col;
        float v = alpha * acc[bi][bj][e];
        if (beta != 0.f) v += beta * *p;
        *p = v;
      }
    }
}

// Ragged fp32 products: g gives the operand types, transposes, base pointers, alpha and beta; the
// sizes, offsets and leading dimensions of product z come from descs[z] (z < n), every one at most
// max_m x max_n.  Operands are fp32; every leading dimension and offset a multiple of 4 elements and
// the bases 16-byte aligned, as the vector loads need.
hipError_t gemm_ragged(hipStream_t s, const GemmArgs &g, const RaggedDesc *descs, int n, int64_t max_m,
                       int64_t max_n, bool bf16_mm) {
  if (n <= 0 || max_m <= 0 || max_n <= 0) return hipSuccess;
  if (g.ta_bf16 || g.tb_bf16 || g.tc_bf16 || (g.trans_a && g.trans_b)) return hipErrorInvalidValue;
  if (((uintptr_t)g.A | (uintptr_t)g.B | (uintptr_t)g.C) & 15) return hipErrorInvalidValue;
  const int64_t gx = (max_n + MT - 1) / MT, gy = (max_m + MT - 1) / MT;
  if (gx > INT32_MAX || gy > 65535) return hipErrorInvalidValue;
  for (int z0 = 0; z0 < n; z0 += 65535) {  // grid z holds at most 65535 products
    dim3 grid((unsigned)gx, (unsigned)gy, (unsigned)(n - z0 < 65535 ? n - z0 : 65535));
    auto go = [&](auto kern) {
      hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, 0, 0, 0, (const float *)g.A, (int64_t)0, (int64_t)0,
                         (const float *)g.B, (int64_t)0, (int64_t)0, (float *)g.C, (int64_t)0, (int64_t)0, g.alpha,
                         g.beta, descs + z0);
    };
    auto go_mixed = [&](auto kern) {
      hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, (const float *)g.A, (const float *)g.B, (float *)g.C, g.alpha,
                         g.beta, descs + z0);
    };
    if (bf16_mm) {
      if (g.trans_a)
        go_mixed(gemm_mixed_ragged_kernel<false, true, false>);
      else if (g.trans_b)
        go_mixed(gemm_mixed_ragged_kernel<true, false, true>);
      else
        go_mixed(gemm_mixed_ragged_kernel<false, false, true>);
    } else if (g.trans_a) {
      go(gemm_mfma_kernel<float, float, false, true, true>);
    } else if (g.trans_b) {
      go(gemm_mfma_kernel<float, float, true, false, true>);
    } else {
      go(gemm_mfma_kernel<float, float, false, false, true>);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Whether the matrix-core form applies: fp32 output, enough 64 x 64 tiles to fill the chip (or
// mfma_small), and vector-aligned operands along their contiguous dimension.
static bool mfma_ok(const GemmArgs &g) {
  if (g.tc_bf16) return false;
  const int64_t tiles64 = (int64_t)((g.N + 63) / 64) * ((g.M + 63) / 64) * g.batch;
  if ((tiles64 < 128 && !g.mfma_small) || g.K < 64) return false;
  auto fits = [](const void *p, bool is_bf16, int64_t ld, int64_t stride, int64_t contiguous_len) {
    const uintptr_t align = is_bf16 ? 8 : 16;
    return ((uintptr_t)p % align) == 0 && ld % 4 == 0 && stride % 4 == 0 && contiguous_len % 4 == 0;
  };
  const int64_t a_len = g.trans_a ? g.M : g.K, b_len = g.trans_b ? g.K : g.N;
  return fits(g.A, g.ta_bf16, g.lda, g.sA, a_len) && fits(g.B, g.tb_bf16, g.ldb, g.sB, b_len);
}

static hipError_t gemm_mfma(hipStream_t s, const GemmArgs &g) {
#define STCA_MFMA_CASE(TA_, TB_)                                                                       \
  if (g.trans_a) return g.trans_b ? gemm_mfma_t<TA_, TB_, true, true>(s, g) : gemm_mfma_t<TA_, TB_, false, true>(s, g); \
  return g.trans_b ? gemm_mfma_t<TA_, TB_, true, false>(s, g) : gemm_mfma_t<TA_, TB_, false, false>(s, g);
  if (g.ta_bf16 && g.tb_bf16) { STCA_MFMA_CASE(bf16, bf16) }
  if (g.ta_bf16) { STCA_MFMA_CASE(bf16, float) }
  if (g.tb_bf16) { STCA_MFMA_CASE(float, bf16) }
  STCA_MFMA_CASE(float, float)
#undef STCA_MFMA_CASE
}

hipError_t gemm(hipStream_t s, const GemmArgs &g) {
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0) return hipSuccess;
  if (mfma_ok(g)) return gemm_mfma(s, g);
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
