// bf16 matrix-core GEMMs for the mixed-precision backward, fp32 accumulation on
// v_mfma_f32_32x32x16_bf16, with epilogues that fuse the SwiGLU of eq. (1) and its derivative into the
// product that feeds them.  Two operand layouts:
//   NT: C[M x N] = A[M x K] Bt[N x K]^T, both k-contiguous (the activation and weight products);
//   TN: C[M x N] = A[K x M]^T B[K x N], both m / n-contiguous (the weight gradients, whose k runs over
//       the rows of row-major activations, so no transposed copy of them is ever written).
//
// Tiles: TM x 128 (TM = 128) per workgroup of four waves (2 x 2), each wave (TM/2) x 64, i.e. TM/64 x 2
// MFMA blocks of 32 x 32; two workgroups per compute unit.  k advances 64 at a time: every thread
// loads its 16-byte chunks of the next k-slab into registers while the current slab's MFMAs run,
// then writes them to the other half of a double-buffered LDS tile.
//   NT slabs are [row][k]: an LDS row holds 64 bf16 (eight 16-byte chunks); chunk c of row r sits in
//   slot c ^ ((r >> 1) & 7), so that the 16 lanes of a fragment read (rows r .. r+15, one chunk) and
//   of a tile write (two rows, all chunks) touch 64 distinct banks.
//   TN slabs are [k][row]: an LDS row holds the 128 m (n) values of one k (sixteen chunks), chunk c
//   of k-row r in slot c ^ 4 (r & 3).  Fragments come from the transposing 64-bit LDS read
//   (ds_read_b64_tr_b16: within each 16-lane group, lane i receives element i % 4 of the 8-byte
//   chunks addressed by lanes 4 j + i / 4, j = 0..3): lane 4 j + q of a group addresses k-row
//   k0 + j and the four rows m0 + 4 q .. m0 + 4 q + 3, so lane i gets rows m0 + i at k0 .. k0 + 3; two
//   such reads give the 8 k of the MFMA operand.  Half a wave reads 4 k-rows x 4 chunks, which the
//   swizzle spreads over all 16 slots: 64 distinct banks.
//
// Epilogues (lane l of a wave holds column 32 j + (l & 31) of block j and, in register e of block i,
// row 32 i + 8 (e >> 2) + 4 (l >> 5) + (e & 3)):
//   kEpiStore / kEpiAcc : C (fp32) = / += the product; batch z at C + z sC.
//   kEpiSwigluFwd       : the columns are up/gate pairs in blocks of 64 (32 up columns of hidden
//                         features 32 q .. 32 q + 31, then the 32 gate columns of the same features),
//                         so a wave holds u and g of the same (row, feature) in one lane: writes
//                         H = u SiLU(g), u and g, rounded to bf16, row-major.
//   kEpiSwigluBwd       : the product is dH (columns = hidden features); reads u, g (row-major bf16)
//                         and writes dU = dH SiLU(g), dG = dH u SiLU'(g) as bf16, row-major [dU | dG].
#include <algorithm>

#include "device_common.hpp"
#include "internal.hpp"

namespace stca {

STCA_DEBUG_WORD

namespace {

constexpr int kTN = 128, kBK = 64;
constexpr int kXcds = 8;  // XCDs of the chip, each with its own L2
// Epilogue staging (128-row tiles): H, u, g [128][64] (forward); u, g [128][128], then dU, dG
// (derivative).
constexpr int kFwdStage = 3 * 128 * 64 * 2;
constexpr int kBwdStage = 2 * 128 * 128 * 2;

__device__ __forceinline__ int nt_slot(int r, int c) { return c ^ ((r >> 1) & 7); }
// Slot of 16-byte chunk c in LDS row r of a 256-byte-row tile read with the transposing LDS read.
__device__ __forceinline__ int tr_slot(int r, int c) { return c ^ ((r & 3) << 2); }
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
// Byte offset, within a 256-byte-row tile laid out by tr_slot, of this lane's address for the
// transposing read that gives lane i of its 16-lane group column col0 + i (col0: the group's first
// column, a multiple of 16) at rows row0 .. row0 + 3 (row0 a multiple of 4).
__device__ __forceinline__ uint32_t tr_lane_offset(int row0, int col0, int lane) {
  const int jj = (lane & 15) >> 2, col = col0 + 4 * (lane & 3), row = row0 + jj;
  return (uint32_t)(row * 256 + (tr_slot(row, col >> 3) << 4) + (col & 7) * 2);
}
__device__ __forceinline__ s16x4 tr_read(const STCA_LDS char *base, uint32_t off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((STCA_LDS s16x4 *)(base + off));
}

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

template <int TM, int EPI, bool TN>
__global__ __launch_bounds__(256, 2) void gemm_nt_kernel(int M, int N, int K, int ksplit, const bf16 *__restrict__ A,
                                                         int64_t lda, int64_t sA, const bf16 *__restrict__ Bt,
                                                         int64_t ldb, int64_t sB, const NtEpilogue ep) {
  constexpr int MI = TM / 64;         // 32-row blocks per wave
  constexpr int LA = TM * 8 / 256;    // 16-byte chunks of the A slab (TM x 64 values) per thread
  constexpr int LB = kTN * 8 / 256;   // ... of the B slab
  static_assert(!TN || TM == 128, "TN slabs are 64 k-rows of 128 values");
  // One LDS block: the double-buffered A and B tiles of the main loop, then the epilogue's staging.
  constexpr int kMainBytes = 2 * (TM + kTN) * 8 * 16;
  constexpr int kEpiBytes = EPI == kEpiSwigluFwd ? kFwdStage : EPI == kEpiSwigluBwd ? kBwdStage : 0;
  __shared__ __attribute__((aligned(16))) char smem[kMainBytes > kEpiBytes ? kMainBytes : kEpiBytes];
  bf16x8(*As)[TM * 8] = reinterpret_cast<bf16x8(*)[TM * 8]>(smem);
  bf16x8(*Bs)[kTN * 8] = reinterpret_cast<bf16x8(*)[kTN * 8]>(smem + 2 * TM * 8 * 16);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 31, g = lane >> 5;
  // Tile of this workgroup: virtual index v runs over column tiles fastest, then row tiles, then
  // batches.  Workgroups are dealt to the 8 XCDs round-robin by launch index b and each XCD has its own
  // L2.  The plain products map b to v so that XCD x = b mod 8 takes the x-th contiguous range of v:
  // the column tiles that share an A row tile, and the tiles of one split-K block, then run on one XCD
  // at about the same time and share its L2.  The SwiGLU epilogues keep v = b, so each XCD works on
  // few column tiles (measured faster for them: 208 against 218 us and 286 against 319 us per
  // 65536-row chunk at d = 256, r = 4).
  int tx, ty, z;
  {
    const int gx = (N + kTN - 1) / kTN, gy = (M + TM - 1) / TM, nb = (int)gridDim.x, b = (int)blockIdx.x;
    const int xcd = b % kXcds, q = nb / kXcds, rem = nb % kXcds;
    const int v = (EPI == kEpiStore || EPI == kEpiAcc) ? xcd * q + (xcd < rem ? xcd : rem) + b / kXcds : b;
    tx = v % gx;
    ty = (v / gx) % gy;
    z = v / (gx * gy);
  }
  const int64_t m0 = (int64_t)ty * TM;
  const int n0 = tx * kTN;
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
  // step s + 1, so every load has two steps of MFMA work to land.  The loads are unconditional, so the
  // compiler can count them and wait only for the set it stores: rows past M (N) read row M - 1
  // (N - 1) and their products land in outputs that are never stored; k beyond the range reads at kb.
  // NT: every chunk read lies inside its row's first lda (ldb) elements, since chunks start at
  // multiples of 8 below ke <= K <= lda and lda is a multiple of 8; the elements at or past ke are
  // zeroed when the last slab is written to LDS, by which time its loads have landed anyway.
  // TN: a chunk is 8 consecutive m (n) of one k-row (M, N multiples of 8); k-rows at or past ke are
  // zeroed in the same way.
  bf16x8 ra0[LA], rb0[LB], ra1[LA], rb1[LB];
  auto load = [&](int k0, bf16x8(&ra)[LA], bf16x8(&rb)[LB]) {
    if constexpr (!TN) {
#pragma unroll
      for (int j = 0; j < LA; ++j) {
        const int q = tid + 256 * j, r = q >> 3, k = k0 + 8 * (q & 7);
        const int64_t row = min(m0 + r, (int64_t)M - 1);
        ra[j] = *reinterpret_cast<const bf16x8 *>(A + row * lda + (k < ke ? k : kb));
      }
#pragma unroll
      for (int j = 0; j < LB; ++j) {
        const int q = tid + 256 * j, r = q >> 3, k = k0 + 8 * (q & 7);
        const int64_t row = min(n0 + r, N - 1);
        rb[j] = *reinterpret_cast<const bf16x8 *>(Bt + row * ldb + (k < ke ? k : kb));
      }
    } else {
#pragma unroll
      for (int j = 0; j < LA; ++j) {
        const int q = tid + 256 * j, kr = k0 + (q >> 4);
        const int col = min((int)m0 + 8 * (q & 15), M - 8);
        ra[j] = *reinterpret_cast<const bf16x8 *>(A + (int64_t)(kr < ke ? kr : kb) * lda + col);
      }
#pragma unroll
      for (int j = 0; j < LB; ++j) {
        const int q = tid + 256 * j, kr = k0 + (q >> 4);
        const int col = min(n0 + 8 * (q & 15), N - 8);
        rb[j] = *reinterpret_cast<const bf16x8 *>(Bt + (int64_t)(kr < ke ? kr : kb) * ldb + col);
      }
    }
  };
  auto store = [&](int buf, int k0, bf16x8(&ra)[LA], bf16x8(&rb)[LB]) {
    if (k0 + kBK > ke) {  // the last slab of the k range
      if constexpr (!TN) {
#pragma unroll
        for (int j = 0; j < LA; ++j) {
          const int k = k0 + 8 * ((tid + 256 * j) & 7);
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (k + e >= ke) ra[j][e] = bf16{};
        }
#pragma unroll
        for (int j = 0; j < LB; ++j) {
          const int k = k0 + 8 * ((tid + 256 * j) & 7);
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (k + e >= ke) rb[j][e] = bf16{};
        }
      } else {
#pragma unroll
        for (int j = 0; j < LA; ++j)
          if (k0 + ((tid + 256 * j) >> 4) >= ke) ra[j] = bf16x8{};
#pragma unroll
        for (int j = 0; j < LB; ++j)
          if (k0 + ((tid + 256 * j) >> 4) >= ke) rb[j] = bf16x8{};
      }
    }
#pragma unroll
    for (int j = 0; j < LA; ++j) {
      const int q = tid + 256 * j;
      if constexpr (!TN)
        As[buf][(q >> 3) * 8 + nt_slot(q >> 3, q & 7)] = ra[j];
      else
        As[buf][(q >> 4) * 16 + tr_slot(q >> 4, q & 15)] = ra[j];
    }
#pragma unroll
    for (int j = 0; j < LB; ++j) {
      const int q = tid + 256 * j;
      if constexpr (!TN)
        Bs[buf][(q >> 3) * 8 + nt_slot(q >> 3, q & 7)] = rb[j];
      else
        Bs[buf][(q >> 4) * 16 + tr_slot(q >> 4, q & 15)] = rb[j];
    }
  };

  f32x16 acc[MI][2];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  // TN fragment addresses: lane group (lane >> 4) covers columns 16 ((lane >> 4) & 1) .. + 15 of its
  // 32-wide block and k 8 g .. 8 g + 7 of each 16-deep substep (two reads of four k-rows).
  uint32_t aoff[MI], boff[2];
  if constexpr (TN) {
#pragma unroll
    for (int i = 0; i < MI; ++i) aoff[i] = tr_lane_offset(8 * g, wm + 32 * i + 16 * ((lane >> 4) & 1), lane);
#pragma unroll
    for (int j = 0; j < 2; ++j) boff[j] = tr_lane_offset(8 * g, wn + 32 * j + 16 * ((lane >> 4) & 1), lane);
  }
  const int steps = ke > kb ? (ke - kb + kBK - 1) / kBK : 0;
  auto compute = [&](int cur) {
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      bf16x8 a[MI], b[2];
      if constexpr (!TN) {
        const int c = 2 * kk + g;
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
      } else {
        const STCA_LDS char *la = (const STCA_LDS char *)&As[cur][0];
        const STCA_LDS char *lb = (const STCA_LDS char *)&Bs[cur][0];
        const uint32_t ko = (uint32_t)kk * 16 * 256;
#pragma unroll
        for (int i = 0; i < MI; ++i)
          a[i] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(tr_read(la, aoff[i] + ko),
                                                                    tr_read(la, aoff[i] + ko + 4 * 256), 0, 1, 2,
                                                                    3, 4, 5, 6, 7));
#pragma unroll
        for (int j = 0; j < 2; ++j)
          b[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(tr_read(lb, boff[j] + ko),
                                                                    tr_read(lb, boff[j] + ko + 4 * 256), 0, 1, 2,
                                                                    3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32x32x16(a[i], b[j], acc[i][j]);
    }
  };
  // Step s computes from LDS half s & 1, loads the slab of s + 2 into one register set and writes the
  // other (the slab of s + 1, loaded during step s - 1) into LDS half (s + 1) & 1, which step s - 1
  // finished reading before the barrier that ended it.  The main loop runs steps in pairs while both
  // of its loads are in range, with no conditional load, store or exit inside, so the compiler keeps
  // one register set per slab and waits only for the slab it stores; the last one to three steps
  // follow with plain conditions.
  if (steps > 0) {  // (an empty k range reads nothing: kb may then lie past the rows)
    load(kb, ra0, rb0);
    store(0, kb, ra0, rb0);
    if (steps > 1) load(kb + kBK, ra1, rb1);
    __syncthreads();
    int st = 0;
    for (; st + 3 < steps; st += 2) {
      load(kb + (st + 2) * kBK, ra0, rb0);
      compute(0);
      store(1, kb + (st + 1) * kBK, ra1, rb1);
      __syncthreads();
      load(kb + (st + 3) * kBK, ra1, rb1);
      compute(1);
      store(0, kb + (st + 2) * kBK, ra0, rb0);
      __syncthreads();
    }
    // slab st in LDS half 0, slab st + 1 (if any) in register set 1
    const int left = steps - st;
    if (left > 2) load(kb + (st + 2) * kBK, ra0, rb0);
    compute(0);
    if (left > 1) {
      store(1, kb + (st + 1) * kBK, ra1, rb1);
      __syncthreads();
      compute(1);
      if (left > 2) {
        store(0, kb + (st + 2) * kBK, ra0, rb0);
        __syncthreads();
        compute(0);
      }
    }
    __syncthreads();  // the epilogues reuse the LDS block
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
    // 32-63 of the tile).  Stage H, u and g [row][feature] in LDS, then store whole 16-byte row
    // chunks.
    uint16_t *sH = reinterpret_cast<uint16_t *>(smem), *sU = sH + 128 * 64, *sG = sU + 128 * 64;
    const int fl = (wn >> 1) + lr;          // feature within the tile
    const int f0 = (n0 >> 1);               // first hidden feature of the tile
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int t0 = wm + 32 * i + 8 * q + 4 * g;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float u = acc[i][0][4 * q + t], gg = acc[i][1][4 * q + t];
          const int o = (t0 + t) * 64 + fl;
          sH[o] = bf16_bits(u * gg * sigmoid_fast(gg));
          sU[o] = bf16_bits(u);
          sG[o] = bf16_bits(gg);
        }
      }
    __syncthreads();
    uint16_t *dst[3] = {reinterpret_cast<uint16_t *>(ep.H), reinterpret_cast<uint16_t *>(ep.U),
                        reinterpret_cast<uint16_t *>(ep.G)};
    const uint16_t *src[3] = {sH, sU, sG};
#pragma unroll
    for (int a = 0; a < 3; ++a)
#pragma unroll
      for (int j = 0; j < 4; ++j) {  // 128 rows x 8 chunks
        const int qd = tid + 256 * j, t = qd >> 3, c = qd & 7;
        if (m0 + t < M)
          *reinterpret_cast<u32x4 *>(dst[a] + (m0 + t) * ep.ldh + f0 + 8 * c) =
              *reinterpret_cast<const u32x4 *>(src[a] + t * 64 + 8 * c);
      }
  } else if constexpr (EPI == kEpiSwigluBwd) {
    static_assert(TM == 128, "staging layout");
    // The tile is 128 rows x 128 hidden features.  The tile's u and g come from their row-major
    // arrays into LDS ([row][feature], 256-byte rows laid out by tr_slot); the transposing read then
    // gives each lane the four consecutive rows of its feature that its accumulator registers hold.
    // dU and dG go out through the same LDS area, [row][feature], in whole 16-byte row chunks.
    const uint16_t *U = reinterpret_cast<const uint16_t *>(ep.U), *G = reinterpret_cast<const uint16_t *>(ep.G);
    uint16_t *dUG = reinterpret_cast<uint16_t *>(ep.dUG);
    uint16_t *sU = reinterpret_cast<uint16_t *>(smem), *sG = sU + 128 * 128;
    {
      u32x4 vu[8], vg[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {  // 128 rows x 16 chunks each
        const int qd = tid + 256 * j, t = qd >> 4;
        const int64_t row = min(m0 + t, (int64_t)M - 1);
        const int col = min(n0 + 8 * (qd & 15), N - 8);
        STCA_CHECK(col + 8 <= ep.ldh, kDbgGemmPad);
        vu[j] = *reinterpret_cast<const u32x4 *>(U + row * ep.ldh + col);
        vg[j] = *reinterpret_cast<const u32x4 *>(G + row * ep.ldh + col);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int qd = tid + 256 * j, t = qd >> 4, o = (t * 16 + tr_slot(t, qd & 15)) * 8;
        *reinterpret_cast<u32x4 *>(sU + o) = vu[j];
        *reinterpret_cast<u32x4 *>(sG + o) = vg[j];
      }
    }
    __syncthreads();
    const STCA_LDS char *lu = (const STCA_LDS char *)sU, *lg = (const STCA_LDS char *)sG;
    uint32_t pu[MI][2][4][2], pg[MI][2][4][2];  // dU, dG of (block i, jb, row group q) as bf16 pairs
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t off = tr_lane_offset(wm + 32 * i + 8 * q + 4 * g, wn + 32 * jb + 16 * ((lane >> 4) & 1), lane);
          const s16x4 u4 = tr_read(lu, off), g4 = tr_read(lg, off);
          float du[4], dg[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float u = __uint_as_float((uint32_t)(uint16_t)u4[t] << 16);
            const float gg = __uint_as_float((uint32_t)(uint16_t)g4[t] << 16);
            const float dh = acc[i][jb][4 * q + t], sg = sigmoid_fast(gg);
            du[t] = dh * gg * sg;
            dg[t] = dh * u * sg * (1.0f + gg * (1.0f - sg));
          }
          pu[i][jb][q][0] = (uint32_t)bf16_bits(du[0]) | ((uint32_t)bf16_bits(du[1]) << 16);
          pu[i][jb][q][1] = (uint32_t)bf16_bits(du[2]) | ((uint32_t)bf16_bits(du[3]) << 16);
          pg[i][jb][q][0] = (uint32_t)bf16_bits(dg[0]) | ((uint32_t)bf16_bits(dg[1]) << 16);
          pg[i][jb][q][1] = (uint32_t)bf16_bits(dg[2]) | ((uint32_t)bf16_bits(dg[3]) << 16);
        }
    __syncthreads();  // every lane has read its u and g: the area takes dU and dG
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int t0 = wm + 32 * i + 8 * q + 4 * g, fl = wn + 32 * jb + lr;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int sh = 16 * (t & 1);
            sU[(t0 + t) * 128 + fl] = (uint16_t)(pu[i][jb][q][t >> 1] >> sh);
            sG[(t0 + t) * 128 + fl] = (uint16_t)(pg[i][jb][q][t >> 1] >> sh);
          }
        }
    __syncthreads();
#pragma unroll
    for (int part = 0; part < 2; ++part) {  // dU into columns n0 .., dG into rd + n0 ..
      const uint16_t *src = part ? sG : sU;
      const int64_t col0 = (int64_t)part * ep.rd + n0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {  // 128 rows x 16 chunks
        const int qd = tid + 256 * j, t = qd >> 4, c = qd & 15;
        if (m0 + t < M && n0 + 8 * c < N)
          *reinterpret_cast<u32x4 *>(dUG + (m0 + t) * ep.lddug + col0 + 8 * c) =
              *reinterpret_cast<const u32x4 *>(src + t * 128 + 8 * c);
      }
    }
  }
}

template <int TM, int EPI, bool TN>
hipError_t launch_nt(hipStream_t s, int M, int N, int K, int ksplit, int batch, const void *A, int64_t lda, int64_t sA,
                     const void *Bt, int64_t ldb, int64_t sB, const NtEpilogue &ep) {
  const int64_t blocks = ((int64_t)M + TM - 1) / TM * ((N + kTN - 1) / kTN) * batch;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_nt_kernel<TM, EPI, TN>), dim3((unsigned)blocks), dim3(256), 0, s, M, N, K, ksplit,
                     (const bf16 *)A, lda, sA, (const bf16 *)Bt, ldb, sB, ep);
  return hipGetLastError();
}

}  // namespace

hipError_t gemm_nt(hipStream_t s, int epi, int M, int N, int K, int ksplit, int batch, const void *A, int64_t lda,
                   int64_t sA, const void *Bt, int64_t ldb, int64_t sB, const NtEpilogue &ep) {
  if (M <= 0 || N <= 0 || batch <= 0) return hipSuccess;
  if (lda % 8 || ldb % 8 || (((uintptr_t)A | (uintptr_t)Bt) & 15) || (sA | sB) % 8 || ksplit % 8)
    return hipErrorInvalidValue;
  if ((epi == kEpiSwigluFwd || epi == kEpiSwigluBwd) && (ep.ldh % 8 || batch != 1 || ksplit)) return hipErrorInvalidValue;
  if (epi == kEpiSwigluFwd && N % 128) return hipErrorInvalidValue;
  if (epi == kEpiSwigluBwd && (N % 8 || ep.lddug % 8)) return hipErrorInvalidValue;
  // 128-row tiles, two workgroups per compute unit (256-row tiles with one measured slower).
  switch (epi) {
    case kEpiStore:
      return launch_nt<128, kEpiStore, false>(s, M, N, K, ksplit, batch, A, lda, sA, Bt, ldb, sB, ep);
    case kEpiAcc:
      return launch_nt<128, kEpiAcc, false>(s, M, N, K, ksplit, batch, A, lda, sA, Bt, ldb, sB, ep);
    case kEpiSwigluFwd:
      return launch_nt<128, kEpiSwigluFwd, false>(s, M, N, K, 0, 1, A, lda, 0, Bt, ldb, 0, ep);
    case kEpiSwigluBwd:
      return launch_nt<128, kEpiSwigluBwd, false>(s, M, N, K, 0, 1, A, lda, 0, Bt, ldb, 0, ep);
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t gemm_tn(hipStream_t s, int epi, int M, int N, int K, int ksplit, int batch, const void *A, int64_t lda,
                   int64_t sA, const void *B, int64_t ldb, int64_t sB, const NtEpilogue &ep) {
  if (M <= 0 || N <= 0 || batch <= 0) return hipSuccess;
  if (M % 8 || N % 8 || lda % 8 || ldb % 8 || lda < M || ldb < N || (((uintptr_t)A | (uintptr_t)B) & 15) ||
      (sA | sB) % 8 || ksplit < 0)
    return hipErrorInvalidValue;
  switch (epi) {
    case kEpiStore:
      return launch_nt<128, kEpiStore, true>(s, M, N, K, ksplit, batch, A, lda, sA, B, ldb, sB, ep);
    case kEpiAcc:
      return launch_nt<128, kEpiAcc, true>(s, M, N, K, ksplit, batch, A, lda, sA, B, ldb, sB, ep);
    default:
      return hipErrorInvalidValue;
  }
}

// ---- weight re-layouts and the LayerNorm derivative of the mixed-precision backward -----------
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
// out as bf16, row-major (rows x D), staged in LDS so that every global store is a whole row chunk.  A workgroup's column sums of dgamma and dbeta over its tiles go to
// parts[blk][c] and parts[gridDim.x + blk][c].
template <int D>
__global__ __launch_bounds__(256) void ln_bwd_bf16_kernel(int64_t rows, const float *__restrict__ dout,
                                                          const float *__restrict__ Y,
                                                          const float *__restrict__ gamma, float eps,
                                                          uint16_t *__restrict__ dY, float *__restrict__ parts) {
  constexpr int E = D / 64;
  __shared__ __attribute__((aligned(16))) uint16_t sR[64 * D];
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
  // Four rows at a time, so that their loads are in flight together and their reductions interleave.
  for (int k = 0; k < 16; k += 4) {
    float y[4][E], go[4][E], dy[4][E];
    bool ok[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int64_t row = r0 + wave * 16 + k + w;
      ok[w] = row < rows;
      const int64_t rr = ok[w] ? row : rows - 1;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        y[w][e] = Y[rr * D + lane + 64 * e];
        go[w][e] = dout[rr * D + lane + 64 * e];
      }
    }
    float sum[4], q[4], s1[4], s2[4], mean[4], rstd[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      sum[w] = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) sum[w] += y[w][e];
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) mean[w] = wave_sum(sum[w]) / (float)D;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      q[w] = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) q[w] += (y[w][e] - mean[w]) * (y[w][e] - mean[w]);
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) rstd[w] = 1.0f / sqrtf(wave_sum(q[w]) / (float)D + eps);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      s1[w] = s2[w] = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float xh = (y[w][e] - mean[w]) * rstd[w], gg = go[w][e] * gm[e];
        s1[w] += gg;
        s2[w] += gg * xh;
        if (ok[w]) {
          pg[e] = fmaf(go[w][e], xh, pg[e]);
          pb[e] += go[w][e];
        }
        y[w][e] = xh;
        dy[w][e] = gg;
      }
    }
    float m1[4], m2[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      m1[w] = wave_sum(s1[w]) / (float)D;
      m2[w] = wave_sum(s2[w]) / (float)D;
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int t = wave * 16 + k + w;
#pragma unroll
      for (int e = 0; e < E; ++e)
        sR[t * D + lane + 64 * e] = ok[w] ? bf16_bits(rstd[w] * (dy[w][e] - m1[w] - y[w][e] * m2[w])) : 0;
    }
  }
  __syncthreads();
  // row-major: 64 rows x D/8 chunks of 16 bytes
  for (int qd = threadIdx.x; qd < 64 * (D / 8); qd += 256) {
    const int t = qd / (D / 8), c = qd % (D / 8);
    if (r0 + t < rows)
      *reinterpret_cast<u32x4 *>(dY + (r0 + t) * D + 8 * c) = *reinterpret_cast<const u32x4 *>(sR + t * D + 8 * c);
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
                       float eps, void *dY, float *dgamma, float *dbeta, float *parts) {
  if (rows <= 0) return hipSuccess;
  const int64_t nblk = std::min<int64_t>((rows + 63) / 64, 256);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(256), 0, s, rows, dout, Y, gamma, eps, (uint16_t *)dY, parts);
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
