// bf16 matrix-core GEMM for the mixed-precision backward: C[M x N] = A[M x K] Bt[N x K]^T with A and
// Bt bf16, k-contiguous, fp32 accumulation on v_mfma_f32_32x32x16_bf16, and epilogues that fuse the
// SwiGLU of eq. (1) and its derivative into the product that feeds them.
//
// Tiles: TM x 128 per workgroup of four waves (2 x 2), each wave (TM/2) x 64, i.e. TM/64 x 2 MFMA
// blocks of 32 x 32.  k advances 64 at a time: every thread loads its 16-byte chunks of the next
// k-slab into registers while the current slab's MFMAs run, then writes them to the other half of a
// double-buffered LDS tile.  An LDS row holds 64 bf16 (eight 16-byte chunks); chunk c of row r sits
// in slot c ^ ((r >> 1) & 7), so that the 16 lanes of a fragment read (rows r .. r+15, one chunk)
// and of a tile write (two rows, all chunks) touch 64 distinct banks.
//
// Epilogues (lane l of a wave holds column 32 j + (l & 31) of block j and, in register e of block i,
// row 32 i + 8 (e >> 2) + 4 (l >> 5) + (e & 3): four consecutive rows per register group, which is
// what makes the transposed (row-contiguous) outputs 8-byte stores):
//   kEpiStore / kEpiAcc : C (fp32) = / += the product; batch z at C + z sC.
//   kEpiSwigluFwd       : the columns are up/gate pairs in blocks of 64 (32 up columns of hidden
//                         features 32 q .. 32 q + 31, then the 32 gate columns of the same features),
//                         so a wave holds u and g of the same (row, feature) in one lane: writes
//                         H = u SiLU(g) rounded to bf16 (row-major and transposed) and u, g as bf16
//                         (transposed), the inputs of the derivative.
//   kEpiSwigluBwd       : the product is dH (columns = hidden features); reads u, g (transposed bf16)
//                         and writes dU = dH SiLU(g), dG = dH u SiLU'(g) as bf16, row-major [dU | dG]
//                         and transposed.
#include <algorithm>

#include "device_common.hpp"
#include "internal.hpp"

namespace stca {

STCA_DEBUG_WORD

namespace {

constexpr int kTN = 128, kBK = 64;
// Epilogue staging (the epilogue kernels use 128-row tiles).  Transposed tiles get rows of 128 + 8
// elements (272 bytes), so that the 8-byte writes of 32 lanes into 32 different rows spread over the
// banks and every row stays 16-byte aligned.
constexpr int kTP = 136;
constexpr int kFwdStage = 128 * 64 * 2 + 3 * 64 * kTP * 2;        // H [128][64], H^T, u^T, g^T [64][136]
constexpr int kBwdStage = 128 * 128 * 2 + 128 * kTP * 2;           // dU or dG: [128][128] and [128][136]

__device__ __forceinline__ int nt_slot(int r, int c) { return c ^ ((r >> 1) & 7); }

__device__ __forceinline__ float sigmoid_fast(float g) { return fast_rcp(1.0f + fast_exp2(-g * kLog2e)); }

__device__ __forceinline__ uint16_t bf16_bits(float v) { return f32_to_bf16_bits(v); }
__device__ __forceinline__ float bf16_round(float v) { return bf16_bits_to_f32(f32_to_bf16_bits(v)); }

unsigned grid_for(int64_t n) {
  const int64_t b = (n + 255) / 256;
  return (unsigned)(b < 1 ? 1 : b > 65536 ? 65536 : b);
}

// Four bf16 values as one 8-byte store / load.
__device__ __forceinline__ void store4(uint16_t *p, float a, float b, float c, float d) {
  const uint32_t lo = (uint32_t)bf16_bits(a) | ((uint32_t)bf16_bits(b) << 16);
  const uint32_t hi = (uint32_t)bf16_bits(c) | ((uint32_t)bf16_bits(d) << 16);
  *reinterpret_cast<uint2 *>(p) = make_uint2(lo, hi);
}
__device__ __forceinline__ void load4(const uint16_t *p, float (&v)[4]) {
  const uint2 w = *reinterpret_cast<const uint2 *>(p);
  v[0] = __uint_as_float(w.x << 16);
  v[1] = __uint_as_float(w.x & 0xFFFF0000u);
  v[2] = __uint_as_float(w.y << 16);
  v[3] = __uint_as_float(w.y & 0xFFFF0000u);
}

template <int TM, int EPI>
__global__ __launch_bounds__(256, TM == 128 ? 2 : 1) void gemm_nt_kernel(int M, int N, int K, int ksplit, const bf16 *__restrict__ A,
                                                         int64_t lda, int64_t sA, const bf16 *__restrict__ Bt,
                                                         int64_t ldb, int64_t sB, const NtEpilogue ep) {
  constexpr int MI = TM / 64;         // 32-row blocks per wave
  constexpr int LA = TM * 8 / 256;    // 16-byte chunks of the A slab per thread
  constexpr int LB = kTN * 8 / 256;   // ... of the B slab
  // One LDS block: the double-buffered A and B tiles of the main loop, then the epilogue's staging.
  constexpr int kMainBytes = 2 * (TM + kTN) * 8 * 16;
  constexpr int kEpiBytes = EPI == kEpiSwigluFwd ? kFwdStage : EPI == kEpiSwigluBwd ? kBwdStage : 0;
  __shared__ __attribute__((aligned(16))) char smem[kMainBytes > kEpiBytes ? kMainBytes : kEpiBytes];
  bf16x8(*As)[TM * 8] = reinterpret_cast<bf16x8(*)[TM * 8]>(smem);
  bf16x8(*Bs)[kTN * 8] = reinterpret_cast<bf16x8(*)[kTN * 8]>(smem + 2 * TM * 8 * 16);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, g = lane >> 5;
  const int z = blockIdx.z;
  const int64_t m0 = (int64_t)blockIdx.y * TM;
  const int n0 = blockIdx.x * kTN;
  const int wm = (wave >> 1) * (TM / 2), wn = (wave & 1) * 64;
  // k range: split-K blocks share A and Bt; batches step through them.
  int kb = 0, ke = K;
  if (ksplit > 0) {
    kb = z * ksplit;
    ke = min(K, kb + ksplit);
  } else {
    A += z * sA;
    Bt += z * sB;
  }

  // Two register sets: the slab of step s + 2 is loaded during step s and written to LDS at the end of
  // step s + 1, so every load has two steps of MFMA work to land.
  bf16x8 ra0[LA], rb0[LB], ra1[LA], rb1[LB];
  auto load = [&](int k0, bf16x8(&ra)[LA], bf16x8(&rb)[LB]) {
#pragma unroll
    for (int j = 0; j < LA; ++j) {
      const int q = tid + 256 * j, r = q >> 3, k = k0 + 8 * (q & 7);
      bf16x8 v{};
      if (m0 + r < M && k < ke) {
        v = *reinterpret_cast<const bf16x8 *>(A + (m0 + r) * lda + k);
        if (k + 8 > ke)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (k + e >= ke) v[e] = bf16{};
      }
      ra[j] = v;
    }
#pragma unroll
    for (int j = 0; j < LB; ++j) {
      const int q = tid + 256 * j, r = q >> 3, k = k0 + 8 * (q & 7);
      bf16x8 v{};
      if (n0 + r < N && k < ke) {
        v = *reinterpret_cast<const bf16x8 *>(Bt + (int64_t)(n0 + r) * ldb + k);
        if (k + 8 > ke)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (k + e >= ke) v[e] = bf16{};
      }
      rb[j] = v;
    }
  };
  auto store = [&](int buf, const bf16x8(&ra)[LA], const bf16x8(&rb)[LB]) {
#pragma unroll
    for (int j = 0; j < LA; ++j) {
      const int q = tid + 256 * j, r = q >> 3;
      As[buf][r * 8 + nt_slot(r, q & 7)] = ra[j];
    }
#pragma unroll
    for (int j = 0; j < LB; ++j) {
      const int q = tid + 256 * j, r = q >> 3;
      Bs[buf][r * 8 + nt_slot(r, q & 7)] = rb[j];
    }
  };

  f32x16 acc[MI][2];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int steps = ke > kb ? (ke - kb + kBK - 1) / kBK : 0;
  auto compute = [&](int cur) {
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const int c = 2 * kk + g;
      bf16x8 a[MI], b[2];
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int r = wm + 32 * i + lr;
        a[i] = As[cur][r * 8 + nt_slot(r, c)];
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = wn + 32 * j + lr;
        b[j] = Bs[cur][r * 8 + nt_slot(r, c)];
      }
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(a[i], b[j], acc[i][j]);
    }
  };
  // Step s computes from LDS half s & 1, loads the slab of s + 2 into one register set and writes the
  // other (the slab of s + 1, loaded during step s - 1) into LDS half (s + 1) & 1, which step s - 1
  // finished reading before the barrier that ended it.
  if (steps > 0) {
    load(kb, ra0, rb0);
    store(0, ra0, rb0);
  }
  if (steps > 1) load(kb + kBK, ra1, rb1);
  __syncthreads();
  for (int st = 0; st < steps; st += 2) {
    if (st + 2 < steps) load(kb + (st + 2) * kBK, ra0, rb0);
    compute(0);
    if (st + 1 < steps) store(1, ra1, rb1);
    __syncthreads();
    if (st + 1 >= steps) break;
    if (st + 3 < steps) load(kb + (st + 3) * kBK, ra1, rb1);
    compute(1);
    if (st + 2 < steps) store(0, ra0, rb0);
    __syncthreads();
  }

  // ---- epilogues ----------------------------------------------------------------------------
  auto row_of = [&](int i, int q) -> int64_t { return m0 + wm + 32 * i + 8 * q + 4 * g; };  // + (e & 3)
  if constexpr (EPI == kEpiStore || EPI == kEpiAcc) {
    float *C = ep.C + z * ep.sC;
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = n0 + wn + 32 * j + lr;
        if (col >= N) continue;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int64_t row = row_of(i, e >> 2) + (e & 3);
          if (row < M) {
            float *p = C + row * ep.ldc + col;
            *p = EPI == kEpiAcc ? *p + acc[i][j][e] : acc[i][j][e];
          }
        }
      }
  } else if constexpr (EPI == kEpiSwigluFwd) {
    static_assert(TM == 128, "staging layout");
    // The tile is 128 rows x 64 hidden features (the wave pair wn = 0 / 64 holds features 0-31 /
    // 32-63 of the tile).  Stage H [row][feature] and H^T, u^T, g^T [feature][row] in LDS, then store
    // whole 16-byte row chunks.
    uint16_t *sH = reinterpret_cast<uint16_t *>(smem);
    uint16_t *sHt = sH + 128 * 64, *sUt = sHt + 64 * kTP, *sGt = sUt + 64 * kTP;
    const int fl = (wn >> 1) + lr;          // feature within the tile
    const int f0 = (n0 >> 1);               // first hidden feature of the tile
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int t0 = wm + 32 * i + 8 * q + 4 * g;
        float u[4], gg[4], h[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          u[t] = acc[i][0][4 * q + t];
          gg[t] = acc[i][1][4 * q + t];
          h[t] = u[t] * gg[t] * sigmoid_fast(gg[t]);
          sH[(t0 + t) * 64 + fl] = bf16_bits(h[t]);
        }
        store4(sHt + fl * kTP + t0, h[0], h[1], h[2], h[3]);
        store4(sUt + fl * kTP + t0, u[0], u[1], u[2], u[3]);
        store4(sGt + fl * kTP + t0, gg[0], gg[1], gg[2], gg[3]);
      }
    __syncthreads();
    uint16_t *H = reinterpret_cast<uint16_t *>(ep.H);
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // H: 128 rows x 8 chunks
      const int qd = tid + 256 * j, t = qd >> 3, c = qd & 7;
      if (m0 + t < M)
        *reinterpret_cast<u32x4 *>(H + (m0 + t) * ep.ldh + f0 + 8 * c) =
            *reinterpret_cast<const u32x4 *>(sH + t * 64 + 8 * c);
    }
    uint16_t *dst[3] = {reinterpret_cast<uint16_t *>(ep.Ht), reinterpret_cast<uint16_t *>(ep.Ut),
                        reinterpret_cast<uint16_t *>(ep.Gt)};
    const uint16_t *src[3] = {sHt, sUt, sGt};
#pragma unroll
    for (int a = 0; a < 3; ++a)
#pragma unroll
      for (int j = 0; j < 4; ++j) {  // 64 feature rows x 16 chunks of 8 rows
        const int qd = tid + 256 * j, f = qd >> 4, c = qd & 15;
        if (m0 + 8 * c < M) {  // a partial chunk fills padding columns (< ldt) that no reader uses
          STCA_CHECK(m0 + 8 * c + 8 <= ep.ldt, kDbgGemmPad);
          *reinterpret_cast<u32x4 *>(dst[a] + (int64_t)(f0 + f) * ep.ldt + m0 + 8 * c) =
              *reinterpret_cast<const u32x4 *>(src[a] + f * kTP + 8 * c);
        }
      }
  } else if constexpr (EPI == kEpiSwigluBwd) {
    static_assert(TM == 128, "staging layout");
    // The tile is 128 rows x 128 hidden features.  Each lane reads its u and g (four consecutive rows
    // of one feature: 8 bytes of u^T, g^T) and forms dU, then dG; each goes out through LDS, staged
    // as [row][feature] and [feature][row], in whole 16-byte row chunks.
    const uint16_t *Ut = reinterpret_cast<const uint16_t *>(ep.Ut), *Gt = reinterpret_cast<const uint16_t *>(ep.Gt);
    const int rd = ep.rd;
    uint16_t *dUG = reinterpret_cast<uint16_t *>(ep.dUG), *dUGt = reinterpret_cast<uint16_t *>(ep.dUGt);
    uint16_t *sR = reinterpret_cast<uint16_t *>(smem), *sT = sR + 128 * 128;  // [row][feature], [feature][row]
#pragma unroll
    for (int part = 0; part < 2; ++part) {     // dU, then dG
      if (part) __syncthreads();               // the staging area is free again
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
          const int fl = wn + 32 * jb + lr;
          const int64_t f = n0 + fl;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int t0 = wm + 32 * i + 8 * q + 4 * g;
            float u[4] = {0.f, 0.f, 0.f, 0.f}, gg[4] = {0.f, 0.f, 0.f, 0.f}, v[4];
            if (f < N && m0 + t0 < M) {  // rows up to round_up(M, 4) - 1 < ldt
              STCA_CHECK(m0 + t0 + 4 <= ep.ldt, kDbgGemmPad);
              load4(Ut + f * ep.ldt + m0 + t0, u);
              load4(Gt + f * ep.ldt + m0 + t0, gg);
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const float dh = acc[i][jb][4 * q + t], sg = sigmoid_fast(gg[t]);
              v[t] = part == 0 ? dh * gg[t] * sg : dh * u[t] * sg * (1.0f + gg[t] * (1.0f - sg));
              sR[(t0 + t) * 128 + fl] = bf16_bits(v[t]);
            }
            store4(sT + fl * kTP + t0, v[0], v[1], v[2], v[3]);
          }
        }
      __syncthreads();
      const int64_t col0 = (int64_t)part * rd + n0;  // column of [dU | dG], row of its transpose
#pragma unroll
      for (int j = 0; j < 8; ++j) {  // [row][feature]: 128 rows x 16 chunks
        const int qd = tid + 256 * j, t = qd >> 4, c = qd & 15;
        if (m0 + t < M && n0 + 8 * c < N)
          *reinterpret_cast<u32x4 *>(dUG + (m0 + t) * ep.lddug + col0 + 8 * c) =
              *reinterpret_cast<const u32x4 *>(sR + t * 128 + 8 * c);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {  // [feature][row]: 128 feature rows x 16 chunks
        const int qd = tid + 256 * j, fr = qd >> 4, c = qd & 15;
        if (n0 + fr < N && m0 + 8 * c < M) {
          STCA_CHECK(m0 + 8 * c + 8 <= ep.ldt, kDbgGemmPad);
          *reinterpret_cast<u32x4 *>(dUGt + (col0 + fr) * ep.ldt + m0 + 8 * c) =
              *reinterpret_cast<const u32x4 *>(sT + fr * kTP + 8 * c);
        }
      }
    }
  }
}

template <int TM, int EPI>
hipError_t launch_nt(hipStream_t s, int M, int N, int K, int ksplit, int batch, const void *A, int64_t lda, int64_t sA,
                     const void *Bt, int64_t ldb, int64_t sB, const NtEpilogue &ep) {
  const int64_t gy = ((int64_t)M + TM - 1) / TM;
  if (gy > 65535 || batch > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_nt_kernel<TM, EPI>), dim3((unsigned)((N + kTN - 1) / kTN), (unsigned)gy, (unsigned)batch),
                     dim3(256), 0, s, M, N, K, ksplit, (const bf16 *)A, lda, sA, (const bf16 *)Bt, ldb, sB, ep);
  return hipGetLastError();
}

}  // namespace

hipError_t gemm_nt(hipStream_t s, int epi, int M, int N, int K, int ksplit, int batch, const void *A, int64_t lda,
                   int64_t sA, const void *Bt, int64_t ldb, int64_t sB, const NtEpilogue &ep) {
  if (M <= 0 || N <= 0 || batch <= 0) return hipSuccess;
  if (lda % 8 || ldb % 8 || (((uintptr_t)A | (uintptr_t)Bt) & 15) || (sA | sB) % 8 || ksplit % 8)
    return hipErrorInvalidValue;
  if ((epi == kEpiSwigluFwd || epi == kEpiSwigluBwd) && (ep.ldt % 4 || batch != 1 || ksplit)) return hipErrorInvalidValue;
  if (epi == kEpiSwigluFwd && N % 128) return hipErrorInvalidValue;
  if (epi == kEpiSwigluBwd && N % 8) return hipErrorInvalidValue;
  // 128-row tiles: two workgroups per compute unit (one overlaps the other's loads).
  const bool tall = false;
  switch (epi) {
    case kEpiStore:
      return tall ? launch_nt<256, kEpiStore>(s, M, N, K, ksplit, batch, A, lda, sA, Bt, ldb, sB, ep)
                  : launch_nt<128, kEpiStore>(s, M, N, K, ksplit, batch, A, lda, sA, Bt, ldb, sB, ep);
    case kEpiAcc:
      return tall ? launch_nt<256, kEpiAcc>(s, M, N, K, ksplit, batch, A, lda, sA, Bt, ldb, sB, ep)
                  : launch_nt<128, kEpiAcc>(s, M, N, K, ksplit, batch, A, lda, sA, Bt, ldb, sB, ep);
    case kEpiSwigluFwd:
      return launch_nt<128, kEpiSwigluFwd>(s, M, N, K, 0, 1, A, lda, 0, Bt, ldb, 0, ep);
    case kEpiSwigluBwd:
      return launch_nt<128, kEpiSwigluBwd>(s, M, N, K, 0, 1, A, lda, 0, Bt, ldb, 0, ep);
    default:
      return hipErrorInvalidValue;
  }
}

// ---- small re-layouts for the mixed-precision backward ---------------------------------------
// out[c][r] = in[r][c] (bf16, rows x cols, row strides ldi / ldo), through 64 x 64 LDS tiles so that
// both the reads and the writes are row-contiguous.
__global__ __launch_bounds__(256) void transpose_tiled_kernel(int64_t rows, int cols, const uint16_t *__restrict__ in,
                                                              int64_t ldi, uint16_t *__restrict__ out, int64_t ldo) {
  __shared__ uint16_t t[64][66];
  const int64_t r0 = (int64_t)blockIdx.y * 64;
  const int c0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int k = ty; k < 64; k += 4) {
    const int64_t r = r0 + k;
    const int c = c0 + tx;
    t[k][tx] = (r < rows && c < cols) ? in[r * ldi + c] : 0;
  }
  __syncthreads();
  for (int k = ty; k < 64; k += 4) {
    const int c = c0 + k;
    const int64_t r = r0 + tx;
    if (c < cols && r < rows) out[(int64_t)c * ldo + r] = t[tx][k];
  }
}

hipError_t transpose_tiled_bf16(hipStream_t s, int64_t rows, int cols, const void *in, int64_t ldi, void *out,
                                int64_t ldo) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  const int64_t gy = (rows + 63) / 64;
  if (gy > 65535) {  // in row slabs of 65535 tiles
    for (int64_t r = 0; r < rows; r += 65535 * 64) {
      const int64_t n = std::min<int64_t>(65535 * 64, rows - r);
      hipError_t e = transpose_tiled_bf16(s, n, cols, (const uint16_t *)in + r * ldi, ldi, (uint16_t *)out + r, ldo);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  hipLaunchKernelGGL(transpose_tiled_kernel, dim3((unsigned)((cols + 63) / 64), (unsigned)gy), dim3(256), 0, s, rows,
                     cols, (const uint16_t *)in, ldi, (uint16_t *)out, ldo);
  return hipGetLastError();
}

// Weight layouts for the mixed backward of one history FFN (Wu, Wv: d x rd; Wo: rd x d; bf16):
//   uvt [2rd x d]: row 64 q + t = column 32 q + t of Wu, row 64 q + 32 + t = the same column of Wv
//                  (the up/gate pairs of the kSwigluFwd epilogue), t < 32;
//   uvc [d x 2rd]: row j = [Wu row j | Wv row j] (the B operand of dX = [dU | dG] [Wu | Wv]^T);
//   ot  [d x rd] : Wo^T.
__global__ __launch_bounds__(256) void bwd_weights_kernel(int d, int rd, const uint16_t *__restrict__ Wu,
                                                          const uint16_t *__restrict__ Wv,
                                                          const uint16_t *__restrict__ Wo, uint16_t *__restrict__ uvt,
                                                          uint16_t *__restrict__ uvc, uint16_t *__restrict__ ot) {
  const int64_t n = (int64_t)d * rd;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int j = (int)(i / rd), k = (int)(i % rd);  // Wu[j][k], Wv[j][k]
    const uint16_t u = Wu[i], v = Wv[i];
    const int q = k >> 5, t = k & 31;
    uvt[(int64_t)(64 * q + t) * d + j] = u;
    uvt[(int64_t)(64 * q + 32 + t) * d + j] = v;
    uvc[(int64_t)j * 2 * rd + k] = u;
    uvc[(int64_t)j * 2 * rd + rd + k] = v;
    // Wo is rd x d: element (k', j') with k' * d + j' = i
    const int64_t ko = i / d, jo = i % d;
    ot[jo * rd + ko] = Wo[i];
  }
}

hipError_t bwd_weights(hipStream_t s, int d, int r, const void *Wu, const void *Wv, const void *Wo, void *uvt,
                       void *uvc, void *ot) {
  const int rd = r * d;
  const int64_t n = (int64_t)d * rd;
  hipLaunchKernelGGL(bwd_weights_kernel, dim3(grid_for(n)), dim3(256), 0, s, d, rd, (const uint16_t *)Wu,
                     (const uint16_t *)Wv, (const uint16_t *)Wo, (uint16_t *)uvt, (uint16_t *)uvc, (uint16_t *)ot);
  return hipGetLastError();
}

// LayerNorm derivative of the mixed path (the same arithmetic as ln_bwd, fp32): workgroups walk
// 64-row tiles (tile = blockIdx.x + k gridDim.x), each wave 16 rows of a tile one at a time; dY goes
// out as bf16, row-major (rows x D) and transposed (D x ldt), both staged in LDS so that every global
// store is a whole row chunk.  A workgroup's column sums of dgamma and dbeta over its tiles go to
// parts[blk][c] and parts[gridDim.x + blk][c].
template <int D>
__global__ __launch_bounds__(256) void ln_bwd_bf16_kernel(int64_t rows, const float *__restrict__ dout,
                                                          const float *__restrict__ Y,
                                                          const float *__restrict__ gamma, float eps,
                                                          uint16_t *__restrict__ dY, uint16_t *__restrict__ dYt,
                                                          int64_t ldt, float *__restrict__ parts) {
  constexpr int E = D / 64, TS = 68;  // transposed rows of 64 tokens + 4 (8-byte aligned, 2-way banks)
  __shared__ __attribute__((aligned(16))) uint16_t sR[64 * D];
  __shared__ __attribute__((aligned(16))) uint16_t sT[D * TS];
  __shared__ float red[4][2][D];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float pg[E], pb[E], gm[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    pg[e] = pb[e] = 0.f;
    gm[e] = gamma[lane + 64 * e];
  }
  const int64_t ntiles = (rows + 63) / 64;
  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
  const int64_t r0 = tile * 64;
  __syncthreads();  // the previous tile's stores have read the staging area
  for (int k = 0; k < 16; ++k) {
    const int t = wave * 16 + k;
    const int64_t row = r0 + t;
    float y[E], go[E], dy[E];
    const bool ok = row < rows;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      y[e] = ok ? Y[row * D + lane + 64 * e] : 0.f;
      go[e] = ok ? dout[row * D + lane + 64 * e] : 0.f;
    }
    float sum = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) sum += y[e];
    const float mean = wave_sum(sum) / (float)D;
    float q = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) q += (y[e] - mean) * (y[e] - mean);
    const float rstd = 1.0f / sqrtf(wave_sum(q) / (float)D + eps);
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float xh = (y[e] - mean) * rstd, g = go[e] * gm[e];
      s1 += g;
      s2 += g * xh;
      pg[e] = fmaf(go[e], xh, pg[e]);
      pb[e] += go[e];
      y[e] = xh;
      dy[e] = g;
    }
    const float m1 = wave_sum(s1) / (float)D, m2 = wave_sum(s2) / (float)D;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const uint16_t b = ok ? bf16_bits(rstd * (dy[e] - m1 - y[e] * m2)) : 0;
      sR[t * D + lane + 64 * e] = b;
      sT[(lane + 64 * e) * TS + t] = b;
    }
  }
  __syncthreads();
  // row-major: 64 rows x D/8 chunks of 16 bytes
  for (int qd = threadIdx.x; qd < 64 * (D / 8); qd += 256) {
    const int t = qd / (D / 8), c = qd % (D / 8);
    if (r0 + t < rows)
      *reinterpret_cast<u32x4 *>(dY + (r0 + t) * D + 8 * c) = *reinterpret_cast<const u32x4 *>(sR + t * D + 8 * c);
  }
  // transposed: D rows x 16 chunks of 4 tokens (8 bytes); rows past the end carry zeros
  for (int qd = threadIdx.x; qd < D * 16; qd += 256) {
    const int f = qd >> 4, c = qd & 15;
    if (r0 + 4 * c < rows) {
      STCA_CHECK(r0 + 4 * c + 4 <= ldt, kDbgGemmPad);
      *reinterpret_cast<uint2 *>(dYt + (int64_t)f * ldt + r0 + 4 * c) = *reinterpret_cast<const uint2 *>(sT + f * TS + 4 * c);
    }
  }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    red[wave][0][lane + 64 * e] = pg[e];
    red[wave][1][lane + 64 * e] = pb[e];
  }
  __syncthreads();
  for (int c = threadIdx.x; c < D; c += 256) {
    parts[(int64_t)blockIdx.x * D + c] = red[0][0][c] + red[1][0][c] + red[2][0][c] + red[3][0][c];
    parts[(int64_t)(gridDim.x + blockIdx.x) * D + c] = red[0][1][c] + red[1][1][c] + red[2][1][c] + red[3][1][c];
  }
}

hipError_t ln_bwd_bf16(hipStream_t s, int64_t rows, int d, const float *dout, const float *Y, const float *gamma,
                       float eps, void *dY, void *dYt, int64_t ldt, float *dgamma, float *dbeta, float *parts) {
  if (rows <= 0) return hipSuccess;
  const int64_t nblk = std::min<int64_t>((rows + 63) / 64, 256);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(256), 0, s, rows, dout, Y, gamma, eps, (uint16_t *)dY,
                       (uint16_t *)dYt, ldt, parts);
  };
  switch (d) {
    case 64: go(ln_bwd_bf16_kernel<64>); break;
    case 128: go(ln_bwd_bf16_kernel<128>); break;
    case 256: go(ln_bwd_bf16_kernel<256>); break;
    case 512: go(ln_bwd_bf16_kernel<512>); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if ((e = sum_parts_strided(s, 1, d, (int)nblk, parts, d, d, dgamma, d, true)) != hipSuccess) return e;
  return sum_parts_strided(s, 1, d, (int)nblk, parts + nblk * d, d, d, dbeta, d, true);
}

// out (+)= sum over k of the parts' [rows x cols] blocks (part k at parts + k pstride, row stride ldp),
// in k order.
__global__ __launch_bounds__(256) void sum_parts_strided_kernel(int rows, int cols, int nparts,
                                                                const float *__restrict__ parts, int64_t ldp,
                                                                int64_t pstride, float *__restrict__ out, int64_t ldo,
                                                                bool accumulate) {
  const int64_t n = (int64_t)rows * cols;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / cols, c = i % cols;
    float *o = out + r * ldo + c;
    float a = accumulate ? *o : 0.f;
#pragma unroll 8
    for (int k = 0; k < nparts; ++k) a += parts[k * pstride + r * ldp + c];
    *o = a;
  }
}

hipError_t sum_parts_strided(hipStream_t s, int rows, int cols, int nparts, const float *parts, int64_t ldp,
                             int64_t pstride, float *out, int64_t ldo, bool accumulate) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  hipLaunchKernelGGL(sum_parts_strided_kernel, dim3(grid_for((int64_t)rows * cols)), dim3(256), 0, s, rows, cols,
                     nparts, parts, ldp, pstride, out, ldo, accumulate);
  return hipGetLastError();
}

hipError_t debug_flags_gemm(uint32_t *flags, bool clear) {
  *flags = 0;
#ifdef STCA_DEBUG_BOUNDS
  hipError_t e = hipMemcpyFromSymbol(flags, HIP_SYMBOL(stca_dbg_word), sizeof(uint32_t));
  if (e != hipSuccess || !clear) return e;
  const uint32_t zero = 0;
  return hipMemcpyToSymbol(HIP_SYMBOL(stca_dbg_word), &zero, sizeof(uint32_t));
#else
  (void)clear;
  return hipSuccess;
#endif
}

}  // namespace stca
