// Ragged split-L single-query cross attention in the reordered form of eq. (13)
// ("Make It Long, Keep It Fast", section 2.1: u = (q W_Q) W_K^T, alpha = softmax(u X~^T / sqrt(d_h)),
// then alpha X~; the W_V / W_O projections run afterwards on the per-target results).
//
// Every (target, head) pair of a user is one query row u (d wide).  All m_u * h rows of a user
// attend to that user's encoded history only (ragged target attention over segment offsets,
// section 2.2 of the same notes), so one pass over the user's history serves all of its rows:
// the request-level-batching reuse.
//
// Work item = (user, chunk of the history, group of up to 128 query rows).  A workgroup streams
// its chunk through LDS in 32-token tiles (fetched into registers three tiles ahead, written into a
// 3-slot LDS ring); each of its 4 waves owns 32 query rows and keeps, per row, a running max, a
// running sum and the fp32 accumulator of alpha X~ (online softmax).  A user with one chunk is finalised in place;
// otherwise the partial (max, sum, accumulator) triples are merged by attend_combine.
#include <math.h>

#include <type_traits>

#include "device_common.hpp"
#include "internal.hpp"

namespace stca {

STCA_DEBUG_WORD

__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// One workgroup: the OR of every user's violations into *result.
__global__ __launch_bounds__(1024) void validate_kernel(int n_users, const int64_t *__restrict__ hoff,
                                                        const int64_t *__restrict__ toff, int64_t total_L,
                                                        int64_t total_T, int64_t max_L, int64_t max_T,
                                                        int32_t *__restrict__ result) {
  __shared__ int acc;
  if (threadIdx.x == 0) acc = 0;
  __syncthreads();
  int bad = 0;
  for (int u = threadIdx.x; u < n_users; u += 1024)
    bad |= offsets_violation(u, n_users, hoff, toff, total_L, total_T, max_L, max_T);
  if (bad) atomicOr(&acc, bad);
  __syncthreads();
  if (threadIdx.x == 0) *result = acc;
}

hipError_t validate_batch(hipStream_t s, int n_users, const int64_t *hist_off, const int64_t *tgt_off, int64_t total_L,
                          int64_t total_T, int64_t max_L, int64_t max_T, int32_t *result) {
  hipLaunchKernelGGL(validate_kernel, dim3(1), dim3(1024), 0, s, n_users, hist_off, tgt_off, total_L, total_T, max_L,
                     max_T, result);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// Work list: the segment index tensor turned into (user, chunk, row group) items.
// One workgroup; users in blocks of 1024 with a block-wide prefix sum.  The offsets are checked
// first (an empty history is allowed: its targets get NaN); if they break the batch's stated
// totals or bounds, or the items or partial rows would exceed what the workspace holds, nothing
// is listed, n_items[1] records the violation and the combine writes NaN to every output row, so
// no kernel writes outside its buffers.
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void worklist_kernel(int n_users, const int64_t *__restrict__ hoff,
                                                        const int64_t *__restrict__ toff, int h, int chunk, int rpg,
                                                        int64_t total_L, int64_t total_T, int64_t max_L,
                                                        int64_t max_T, int64_t max_items, int64_t max_part_rows,
                                                        WorkItem *__restrict__ items, int32_t *__restrict__ n_items,
                                                        int32_t *__restrict__ user_nchunks,
                                                        int64_t *__restrict__ part_base,
                                                        int32_t *__restrict__ tgt_user) {
  __shared__ int64_t sc_i[1024];
  __shared__ int64_t sc_p[1024];
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
  // Item and partial-row totals against the workspace bounds (implied by the checks above; kept so
  // that a wrong bound derivation can never turn into an out-of-bounds write).
  int64_t carry_i = 0, carry_p = 0;
  for (int base = 0; base < n_users && bad_all == 0; base += 1024) {
    const int u = base + tid;
    int64_t ni = 0, np = 0;
    if (u < n_users) {
      const int64_t L = hoff[u + 1] - hoff[u];
      const int64_t R = (toff[u + 1] - toff[u]) * h;
      const int64_t nc = L > 0 ? (L + chunk - 1) / chunk : 0;
      ni = R > 0 ? nc * ((R + rpg - 1) / rpg) : 0;
      np = nc > 1 ? nc * R : 0;
    }
    sc_i[tid] = ni;
    sc_p[tid] = np;
    __syncthreads();
    for (int off = 512; off > 0; off >>= 1) {
      if (tid < off) {
        sc_i[tid] += sc_i[tid + off];
        sc_p[tid] += sc_p[tid + off];
      }
      __syncthreads();
    }
    carry_i += sc_i[0];
    carry_p += sc_p[0];
    __syncthreads();
  }
  if (tid == 0 && bad_all == 0 && (carry_i > max_items || carry_p > max_part_rows)) bad_all = kBatchOverflow;
  __syncthreads();
  if (bad_all != 0) {
    if (tid == 0) {
      n_items[0] = 0;
      n_items[1] = bad_all;
    }
    return;
  }

  carry_i = 0;
  carry_p = 0;
  for (int base = 0; base < n_users; base += 1024) {
    const int u = base + tid;
    int64_t ni = 0, np = 0;
    int nc = 0, ng = 0;
    if (u < n_users) {
      const int64_t L = hoff[u + 1] - hoff[u];
      const int64_t R = (toff[u + 1] - toff[u]) * h;
      nc = L > 0 ? (int)((L + chunk - 1) / chunk) : 0;
      ng = (int)((R + rpg - 1) / rpg);
      ni = R > 0 ? (int64_t)nc * ng : 0;
      np = nc > 1 ? (int64_t)nc * R : 0;
      user_nchunks[u] = nc;
      for (int64_t t = toff[u]; t < toff[u + 1]; ++t) tgt_user[t] = u;
    }
    sc_i[tid] = ni;
    sc_p[tid] = np;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int64_t a = tid >= off ? sc_i[tid - off] : 0;
      const int64_t b = tid >= off ? sc_p[tid - off] : 0;
      __syncthreads();
      sc_i[tid] += a;
      sc_p[tid] += b;
      __syncthreads();
    }
    if (u < n_users) {
      part_base[u] = carry_p + sc_p[tid] - np;
      int64_t k = carry_i + sc_i[tid] - ni;
      if (ni > 0)
        for (int c = 0; c < nc; ++c)
          for (int g = 0; g < ng; ++g, ++k) {
            STCA_CHECK(k < max_items, kDbgWorklist);
            items[k] = WorkItem{u, c, g, nc};
          }
    }
    carry_i += sc_i[1023];
    carry_p += sc_p[1023];
    __syncthreads();
  }
  if (tid == 0) {
    n_items[0] = (int32_t)carry_i;
    n_items[1] = 0;
  }
}

hipError_t build_worklist(hipStream_t s, const AttnPlan &p, const int64_t *hist_off, const int64_t *tgt_off,
                          const AttnBuffers &b) {
  hipLaunchKernelGGL(worklist_kernel, dim3(1), dim3(1024), 0, s, p.n_users, hist_off, tgt_off, p.h, p.chunk,
                     attn_rows_per_group(p.d), p.total_L, p.total_T, p.max_L, p.max_T, p.max_items, p.max_part_rows,
                     b.items, b.n_items, b.user_nchunks, b.part_base, b.tgt_user);
  return hipGetLastError();
}

// Work item of this workgroup.  Workgroups are dealt to the chip's 8 XCDs round-robin by index, and
// each XCD has its own L2; item ranges are therefore handed out per XCD (XCD x = blockIdx mod 8 takes
// the x-th eighth of the list, in order), so the row groups of one user, which stream the same
// history chunk, run on one XCD and share its L2.  Returns false for workgroups with no item.
constexpr int kXcds = 8;
__device__ __forceinline__ bool my_item(const WorkItem *__restrict__ items, const int32_t *__restrict__ n_items,
                                        WorkItem &it) {
  const int n = *n_items, b = (int)blockIdx.x;
  const int x = b % kXcds, j = b / kXcds, q = n / kXcds, rem = n % kXcds;
  const int cnt = q + (x < rem ? 1 : 0), base = x * q + (x < rem ? x : rem);
  if (j >= cnt) return false;
  it = items[base + j];
  return true;
}

// ------------------------------------------------------------------------------------------
// bf16 MFMA kernel with 32 query rows per wave (v_mfma_f32_32x32x16_bf16 for both contractions).
// attend_split runs it at d = 64 and 128; d = 256 and 512 run attend16_kernel below, which measured
// faster there.  The kernel stays written for every width (at d = 512 with its two-wave score split),
// which is where the 16-row kernel's pairs come from.
//   scores  S^T[tok x row] = X~_tile[tok x d] U^T[d x row]      (A from LDS, B = U in registers)
//   update  O^T[d x row]  += X~_tile^T[d x tok] P^T[tok x row]  (A from LDS, B = P in registers)
// The accumulator layout of S^T is, per lane, one query row and 16 tokens; taking the
// probabilities of registers 8 kk .. 8 kk + 7 as the B operand of k-step kk pairs them with the
// tokens phi(kk, g, e) = 16 kk + 8 (e>>2) + 4 g + (e&3), which the A operand reads from LDS with
// the transposing 64-bit LDS read (ds_read_b64_tr_b16: within each 16-lane group, lane i gets
// element i%4 of the 8-byte chunks addressed by lanes 4j + i/4, j = 0..3), two per fragment.
// LDS tile layout: 32 rows x d/8 16-byte chunks, chunk c of row t stored at position
// c ^ sigma(t) so both the row-wise and the column-wise reads spread over the banks.
// History tiles stream from HBM through registers into a 3-slot LDS ring.
// ------------------------------------------------------------------------------------------
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;

// Swizzle of the history tile: 16-byte chunk c of row t is stored at chunk position c ^ sigma(t).
// For d >= 128, sigma swaps the two low 2-bit fields of t (bit 4 passes through at d >= 256): a
// bijection on the row index, so the 16 rows of a row-wise read quarter still hit 16 different
// chunk positions, while the 8 rows x 4 chunks touched by a transposed read half-wave land on
// 32 different 8-byte bank pairs.  d = 64 (8 chunks per row) keeps sigma(t) = t & 7.
template <int D> __device__ __forceinline__ int tile_sigma(int t) {
  if constexpr (D >= 256) return ((t & 3) << 2) | ((t >> 2) & 3) | (t & 16);
  else if constexpr (D == 128) return ((t & 3) << 2) | ((t >> 2) & 3);
  else return t & 7;
}

// Softmax running-max slack (log2 units): rescale the accumulators only when a row's maximum
// grows by more than this.  Exact (the same reference maximum normalises numerator and
// denominator); probabilities stay <= 2^kLazy.
constexpr float kLazy = 8.0f;

template <int D>
__global__ __launch_bounds__(256, (D <= 128 ? 2 : 1)) void attend_mfma_kernel(
    const WorkItem *__restrict__ items, const int32_t *__restrict__ n_items, const int64_t *__restrict__ hoff,
    const int64_t *__restrict__ toff, int h, int chunk, const bf16 *__restrict__ Xt,
    const bf16 *__restrict__ U, float *__restrict__ abar, float *__restrict__ part_A,
    float *__restrict__ part_ms, const int64_t *__restrict__ part_base, const AttnBounds bnd) {
  constexpr int CPR = D / 8;                      // 16-byte chunks per history row
  constexpr int SWZ = (CPR < 32 ? CPR : 32) - 1;  // swizzle mask
  constexpr int NKS = D / 16, NOB = D / 32;
  constexpr int INSTR = 32 * D * 2 / 1024;        // 1 KiB wave loads per 32-token tile
  constexpr int LPW = INSTR / 4;                  // per wave
  // Tiles pass through registers into a 3-slot LDS ring: tile k+2 is written while tile k+1's
  // scores and tile k's PV product read the other two slots, and tile k+2+NB is fetched from HBM
  // into the registers it leaves.  NB register sets keep NB tiles in flight per wave: with one,
  // the loads have a single iteration to arrive and the loaded HBM latency sets the pace.  (No
  // direct-to-LDS loads: with one in flight the compiler makes every transposed LDS read wait
  // for all outstanding loads, serialising the pipeline.)
  constexpr int NSL = 3;
  // At d = 512 a wave keeps half of the output features: two waves (wave, wave ^ 1) share a
  // 32-row block, each computes the scores over its half of d, and the pair adds the two partial
  // score tiles through LDS; U and the accumulators then fit in one wave's registers.
  constexpr int FH = attn_feature_halves(D);
  constexpr int NOBW = NOB / FH;                  // output blocks per wave
  constexpr int NKW = NKS / FH;                   // score k-steps per wave
  constexpr int NB = D <= 256 ? 2 : 1;          // register sets (d = 512 has no registers to spare)
  constexpr int NCH = FH > 1 ? 2 : 1;           // score accumulation chains
  static_assert(INSTR % 4 == 0, "tile loads split evenly over 4 waves");
  __shared__ bf16x8 tiles[NSL][32 * CPR];
  // Partial score tiles of the pairs (FH = 2): [tile parity][wave][register quad][lane].
  __shared__ f32x4 exch[FH > 1 ? 2 : 1][FH > 1 ? 4 : 1][4][64];

  WorkItem it;
  if (!my_item(items, n_items, it)) return;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31, gl = lane >> 5;
  const int64_t L0 = hoff[it.user], L1 = hoff[it.user + 1];
  const int64_t t0 = L0 + (int64_t)it.chunk * chunk;
  const int64_t t1 = (t0 + chunk < L1) ? t0 + chunk : L1;
  const int64_t T0 = toff[it.user];
  const int R = (int)((toff[it.user + 1] - T0) * h);
  const int64_t rowbase = T0 * h;
  // The wave index is uniform (readfirstlane), so control flow on it stays scalar; fh is taken
  // from threadIdx.x instead, because with a scalar fh the compiler spills at d = 512.
  const int fh = (int)(threadIdx.x >> 6) % FH;
  const int r0 = it.group * attn_rows_per_group(D) + (wave / FH) * 32;
  const bool wave_active = r0 < R;
  const int myrow = r0 + col;
  const bool row_ok = myrow < R;
  const int ntiles = (int)((t1 - t0 + 31) / 32);
  STCA_CHECK(L0 >= 0 && L0 <= L1 && L1 <= bnd.total_L && t0 < t1, kDbgAttendRange);

  // U rows as B operands (loaded first so that the tile loads below are the youngest in flight):
  // this wave's k-steps fh NKW .. fh NKW + NKW - 1 of the score reduction.
  bf16x8 ub[NKW];
  {
    const bf16 *urow = U + (rowbase + (row_ok ? myrow : 0)) * D + 8 * gl + 16 * NKW * fh;
#pragma unroll
    for (int ks = 0; ks < NKW; ++ks) {
      if (row_ok)
        ub[ks] = *reinterpret_cast<const bf16x8 *>(urow + 16 * ks);
      else
        ub[ks] = bf16x8{};
    }
  }

  // Tile k: wave piece j = wave + 4 jj (1 KiB) holds, at byte 16 i, the 16-byte chunk
  // (i mod CPR) ^ sigma(row) of history row 32 k + row, row = (64 j + i) / CPR (rows past the
  // chunk's end repeat its last row; their scores are masked).
  // Per-lane (row, element offset within the tile) of each piece, fixed for the whole item.
  int frow[LPW];
  uint32_t foff[LPW];
#pragma unroll
  for (int jj = 0; jj < LPW; ++jj) {
    const int slot = (wave + 4 * jj) * 64 + lane;
    const int row = slot / CPR, cs = slot % CPR;
    frow[jj] = row;
    foff[jj] = (uint32_t)(row * D + (cs ^ tile_sigma<D>(row)) * 8);
  }
  const int64_t len = t1 - t0;
  auto fetch = [&](int k, u32x4 (&rg)[LPW]) {
    const bf16 *tile = Xt + (t0 + 32 * (int64_t)k) * D;
    if (32 * (int64_t)(k + 1) <= len) {
#pragma unroll
      for (int jj = 0; jj < LPW; ++jj) {
        STCA_CHECK(32 * (int64_t)k + frow[jj] < len, kDbgAttendFetch);
        rg[jj] = *reinterpret_cast<const u32x4 *>(tile + foff[jj]);
      }
    } else {  // partial last tile: rows past the end repeat the last row
      const int rem = (int)(len - 32 * (int64_t)k);
#pragma unroll
      for (int jj = 0; jj < LPW; ++jj) {
        const int back = frow[jj] < rem ? 0 : (frow[jj] - rem + 1) * D;
        STCA_CHECK(rem > 0 && 32 * (int64_t)k + frow[jj] - back / D < len, kDbgAttendFetch);
        rg[jj] = *reinterpret_cast<const u32x4 *>(tile + (foff[jj] - back));
      }
    }
  };
  auto put = [&](int b, const u32x4 (&rg)[LPW]) {
#pragma unroll
    for (int jj = 0; jj < LPW; ++jj) {
      const int j = wave + 4 * jj;
      tiles[b][j * 64 + lane] = __builtin_bit_cast(bf16x8, rg[jj]);
    }
  };
  // LDS writes of this wave complete, then the workgroup meets; loads in flight stay in flight.
  auto sync = [&]() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // Tile j >= 2 waits in register set (j - 2) mod NB between its fetch and its put.  With two
  // sets every iteration fetches, also past the last tile (it re-reads the last one, from
  // cache): loads issued on some paths only would make the compiler's count of loads in flight
  // conservative at the join, and each put would then wait for every outstanding load.  With
  // one set the put waits for the newest loads anyway, and the fetches stop at the last tile.
  // The re-reads past the end are never consumed; the wave's end waits for them (s_endpgm
  // waits for all outstanding memory operations), so no register is written after it.
  u32x4 rgb[NB][LPW];
  fetch(0, rgb[0]);
  put(0, rgb[0]);
  if (1 < ntiles) {
    fetch(1, rgb[0]);
    put(1, rgb[0]);
  }
  if constexpr (NB > 1) {
#pragma unroll
    for (int b = 0; b < NB; ++b) fetch(min(2 + b, ntiles - 1), rgb[b]);
  } else if (2 < ntiles) {
    fetch(2, rgb[0]);
  }

  f32x16 oacc[NOBW];
#pragma unroll
  for (int ob = 0; ob < NOBW; ++ob) oacc[ob] = f32x16{};
  float m_run = -INFINITY, s_run = 0.f;

  // Per-lane LDS byte offsets.  Row-wise reads (scores): chunk (2 ks + gl) of row col sits at
  // (2 ks) ^ rx with rx = gl ^ sigma(col).  Column-wise transposed reads (PV): lane
  // l = 16 g + 4 j + q points at features 32 ob + 16 (g&1) + 4 q .. +3 of token
  // tau = 16 kk + 8 s + 4 (g>>1) + j; each address is a per-lane base (one of NTB) plus a
  // compile-time offset, see tr_offset().
  const uint32_t row_off = (uint32_t)(col * CPR * 16);
  const uint32_t rx16 = (uint32_t)((gl ^ tile_sigma<D>(col)) * 16);
  constexpr int NTB = D >= 128 ? 8 : 2;
  uint32_t tbase[NTB];
  {
    const int g = lane >> 4, j = (lane >> 2) & 3, q = lane & 3;
    const int g2 = g >> 1, g1 = g & 1, q1 = q >> 1, q0 = q & 1;
    if constexpr (D >= 128) {
      // chunk (4 ob + 2 g1 + q1) ^ sigma(tau), sigma(tau) = 4 j + 2 s + g2 (+ 16 kk at d >= 256):
      // low bits (2 g1 + q1) ^ g2 ^ 2 s, high bits ob ^ (4 kk) ^ j.  Base index = 2 (P'&3) + s.
      const int v1 = (2 * g1 + q1) ^ g2;
#pragma unroll
      for (int pk = 0; pk < 4; ++pk)
#pragma unroll
        for (int sh = 0; sh < 2; ++sh)
          tbase[2 * pk + sh] =
              (uint32_t)((4 * g2 + j) * CPR * 16 + 64 * (pk ^ j) + 16 * (v1 ^ (2 * sh)) + 8 * q0);
    } else {
      const int lo = (2 * g1 + q1) ^ j;
      const int common = (4 * g2 + j) * CPR * 16 + 16 * lo + 8 * q0;
      tbase[0] = (uint32_t)(common + 64 * g2);
      tbase[1] = (uint32_t)(common - 64 * g2);
    }
  }
  // (base index, compile-time byte offset) of the transposed read for (ob, kk, s).
  auto tr_offset = [](int ob, int kk, int sh, int &bi) -> uint32_t {
    if constexpr (D >= 128) {
      const int Pp = ob ^ (D >= 256 ? 4 * kk : 0);
      bi = 2 * (Pp & 3) + sh;
      return (uint32_t)((16 * kk + 8 * sh) * CPR * 16 + 64 * (Pp & ~3));
    } else {
      const int P = ob ^ ((4 * kk + 2 * sh) & (SWZ >> 2));
      bi = P & 1;
      return (uint32_t)((16 * kk + 8 * sh) * CPR * 16 + 64 * P);
    }
  };

  // All tile reads go through this LDS-typed base and 32-bit byte offsets (so they stay
  // ds_read instructions, counted by lgkmcnt only, independent of the tile loads in flight).
  const STCA_LDS char *lds = (const STCA_LDS char *)&tiles[0][0];
  constexpr uint32_t kTileBytes = 32 * CPR * 16;
  // Scores of one tile into NCH accumulation chains.  One chain (d <= 256) saves the per-step sum
  // of two accumulators and its copies; at d = 512 the k-steps alternate between two chains,
  // whose sum lands in fresh registers, leaving both free for the next tile.
  // This wave's k-steps start 32 NKW fh bytes into a row.  The swizzle acts on the chunk index
  // (bits 4.. of the byte offset), which that start may share, so it stays inside the XOR.
  const uint32_t kofs = (uint32_t)(32 * NKW * fh);
  auto scores = [&](uint32_t toff, f32x16 &s0, f32x16 &s1) {
    uint32_t rx = rx16, rb = toff + row_off;
    asm volatile("" : "+v"(rx), "+v"(rb));
#pragma unroll
    for (int ks = 0; ks < NKW; ++ks) {
      const uint32_t off = rb + (((uint32_t)(32 * ks) + kofs) ^ rx);
      const bf16x8 a = *(const STCA_LDS bf16x8 *)(lds + off);
      if (NCH > 1 && (ks & 1))
        s1 = mfma32x32x16(a, ub[ks], ks == 1 ? f32x16{} : s1);
      else
        s0 = mfma32x32x16(a, ub[ks], ks == 0 ? f32x16{} : s0);
    }
  };
  // Raw scores of a tile with `rem` valid tokens -> masked scores and the maximum over this
  // lane's 16 tokens (the other 16 tokens of the row are in lane l ^ 32; see half_max).
  auto row_max = [&](f32x16 &sc, int rem) {
    if (rem < 32) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int tau = 8 * (i >> 2) + 4 * gl + (i & 3);
        if (tau >= rem) sc[i] = -INFINITY;
      }
    }
    float mx = sc[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sc[i]);
    return mx;
  };
  // bf16 probabilities 2^(s - m_run) (B operands of the PV product); their sum goes into s_run.
  auto probs = [&](const f32x16 &sc, bf16x8 (&pb)[2]) {
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = fast_exp2(sc[i] - m_run);
      pb[i >> 3][i & 7] = f32_to_bf16(p);
      psum += p;
    }
    s_run += psum;
  };
  // PV product of one tile.
  auto pv = [&](uint32_t toff, const bf16x8 (&pb)[2], auto FHc) {
    constexpr int OB0 = decltype(FHc)::value * NOBW;  // first output block of this wave
    uint32_t bb[NTB];
#pragma unroll
    for (int i = 0; i < NTB; ++i) {
      bb[i] = tbase[i] + toff;
      asm volatile("" : "+v"(bb[i]));
    }
#pragma unroll
    for (int obw = 0; obw < NOBW; ++obw) {
      const int ob = OB0 + obw;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        s16x4 half[2];
#pragma unroll
        for (int sh = 0; sh < 2; ++sh) {
          int bi = 0;
          const uint32_t C = tr_offset(ob, kk, sh, bi);
          half[sh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((STCA_LDS s16x4 *)(lds + bb[bi] + C));
        }
        const bf16x8 xa = __builtin_bit_cast(bf16x8, __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
        oacc[obw] = mfma32x32x16(xa, pb[kk], oacc[obw]);
      }
    }
  };
  // The same product with its operands read ahead (one wave per row block, d >= 128): the reads
  // for the first PVA output blocks are issued when the step starts, so they land during the
  // score phase, and each later block's reads go out PVA blocks before its MFMAs.
  constexpr bool PVPRE = FH == 1 && D >= 128;
  constexpr int PVA = 2;
  uint32_t pvb[NTB];
  bf16x8 xr[PVA + 1][2];
  auto xt_frag = [&](int ob, int kk) {
    s16x4 half[2];
#pragma unroll
    for (int sh = 0; sh < 2; ++sh) {
      int bi = 0;
      const uint32_t C = tr_offset(ob, kk, sh, bi);
      half[sh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((STCA_LDS s16x4 *)(lds + pvb[bi] + C));
    }
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto pv_start = [&](uint32_t toff) {
#pragma unroll
    for (int i = 0; i < NTB; ++i) {
      pvb[i] = tbase[i] + toff;
      asm volatile("" : "+v"(pvb[i]));
    }
#pragma unroll
    for (int ob = 0; ob < PVA; ++ob)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) xr[ob][kk] = xt_frag(ob, kk);
  };
  auto pv_finish = [&](const bf16x8 (&pb)[2]) {
#pragma unroll
    for (int ob = 0; ob < NOBW; ++ob) {
      if (ob + PVA < NOBW)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) xr[(ob + PVA) % (PVA + 1)][kk] = xt_frag(ob + PVA, kk);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) oacc[ob] = mfma32x32x16(xr[ob % (PVA + 1)][kk], pb[kk], oacc[ob]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using H0 = std::integral_constant<int, 0>;
  using H1 = std::integral_constant<int, (FH > 1 ? 1 : 0)>;
  auto tile_rem = [&](int k) {
    const int64_t r = t1 - (t0 + 32 * (int64_t)k);
    return (int)(r < 32 ? r : 32);
  };
  auto tile_off = [&](int k) { return (uint32_t)((k % NSL) * kTileBytes); };

  // Pipeline: iteration k computes the scores of tile k+1 (matrix cores) while the vector ALU
  // turns the scores of tile k into probabilities, then the PV product of tile k.  Tiles k and
  // k+1 are in LDS; tile k+2 is written from registers into the slot of tile k-1, and tile
  // k+2+NB is fetched into the registers it leaves.  The loop is unrolled NB times so that each
  // step names its register set statically.  The accumulators are touched only by MFMAs inside
  // the loop: when a row maximum outgrows the slack the loop is left, the rescale runs and the
  // tile is finished.  Every path back into the loop arrives after a step on the last register
  // set, so the compiler sees the same loads in flight, in the same order, on each of them.
  // The running maximum starts at the first tile's.
  sync();
  // Pairs (FH = 2): publish this wave's partial score tile of tile k; after the next workgroup
  // barrier the partner adds it (both waves then hold bit-identical scores: a + b = b + a).
  auto publish = [&](int k, const f32x16 &part) {
    if constexpr (FH > 1) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        exch[k & 1][wave][q][lane] = f32x4{part[4 * q], part[4 * q + 1], part[4 * q + 2], part[4 * q + 3]};
    }
  };
  auto with_partner = [&](int k, f32x16 own) {
    if constexpr (FH > 1) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 o = exch[k & 1][wave ^ 1][q][lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) own[4 * q + e] += o[e];
      }
    }
    return own;
  };
  f32x16 sa = f32x16{}, sb = f32x16{};
  auto score_tile = [&]() {
    if constexpr (NCH > 1) return sa + sb;
    else return sa;
  };
  if constexpr (FH == 1) {
    if (wave_active) {
      scores(tile_off(0), sa, sb);
      f32x16 s0 = score_tile();
      m_run = half_max(row_max(s0, tile_rem(0)));
    }
  } else {
    if (wave_active) {
      scores(tile_off(0), sa, sb);
      publish(0, score_tile());
    }
    sync();
    if (wave_active) {
      f32x16 s0 = with_partner(0, score_tile());
      m_run = half_max(row_max(s0, tile_rem(0)));
    }
  }
  auto tail = [&](int k, const f32x16 &sc) {
    bf16x8 pb[2];
    probs(sc, pb);
    if constexpr (FH == 1) {
      pv(tile_off(k), pb, H0{});
    } else {
      if (fh == 0)
        pv(tile_off(k), pb, H0{});
      else
        pv(tile_off(k), pb, H1{});
    }
  };
  // One step on tile k, with register set BI.  Returns true when a row maximum outgrew the
  // slack: the caller then rescales and finishes tile k.  The score MFMAs of tile k+1 go one per
  // group, and each group also turns one score of tile k into its probability (exp2, bf16,
  // running sum) and folds it into the tile's maximum, so that this vector work runs in the
  // matrix cores' shadow (the order is pinned: left alone, the compiler issues all MFMAs
  // first).  The probabilities are computed against the running maximum before the tile's own
  // maximum is known; when that maximum outgrew the slack they are discarded and the caller
  // recomputes them after the rescale.  The PV product of tile k follows.
  constexpr int kRingA = 4, kAheadA = 3;
  constexpr int NGA = NKW > 16 ? NKW : 16;
  auto step = [&](int k, auto BI, f32x16 &sc, float &mx) -> bool {
    constexpr int b = decltype(BI)::value;
    sync();  // tile k+1 is in LDS; tile k-1's slot is free
    if constexpr (NB > 1) {
      if (k + 2 < ntiles) put((k + 2) % NSL, rgb[b]);
      fetch(min(k + 2 + NB, ntiles - 1), rgb[b]);
    } else if (k + 2 < ntiles) {  // one set: its put waits for the newest loads in any case
      put((k + 2) % NSL, rgb[b]);
      if (k + 3 < ntiles) fetch(k + 3, rgb[b]);
    }
    if (!wave_active) return false;
    const bool has_next = k + 1 < ntiles;
    sc = with_partner(k, score_tile());
    const int rem = tile_rem(k);
    if (rem < 32) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int tau = 8 * (i >> 2) + 4 * gl + (i & 3);
        if (tau >= rem) sc[i] = -INFINITY;
      }
    }
    bf16x8 pb[2];
    float psum = 0.f;
    mx = -INFINITY;
    auto element = [&](int i) {
      const float p = fast_exp2(sc[i] - m_run);
      pb[i >> 3][i & 7] = f32_to_bf16(p);
      psum += p;
      mx = fmaxf(mx, sc[i]);
    };
    if (has_next) {
      uint32_t rx = rx16, rb = tile_off(k + 1) + row_off;
      asm volatile("" : "+v"(rx), "+v"(rb));
      auto frag = [&](int ks) { return *(const STCA_LDS bf16x8 *)(lds + rb + (((uint32_t)(32 * ks) + kofs) ^ rx)); };
      bf16x8 fr[kRingA];
#pragma unroll
      for (int q = 0; q < kAheadA; ++q) fr[q] = frag(q);
      if constexpr (PVPRE) pv_start(tile_off(k));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int g = 0; g < NGA; ++g) {
        if (g < NKW) {
          if (g + kAheadA < NKW) fr[(g + kAheadA) % kRingA] = frag(g + kAheadA);
          if (NCH > 1 && (g & 1))
            sb = mfma32x32x16(fr[g % kRingA], ub[g], g == 1 ? f32x16{} : sb);
          else
            sa = mfma32x32x16(fr[g % kRingA], ub[g], g == 0 ? f32x16{} : sa);
        }
        if (g < 16) element(g);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      if constexpr (PVPRE) pv_start(tile_off(k));
#pragma unroll
      for (int i = 0; i < 16; ++i) element(i);
    }
    if (wave_any(mx > m_run + kLazy)) return true;
    s_run += psum;
    if constexpr (PVPRE) {
      pv_finish(pb);
    } else if constexpr (FH == 1) {
      pv(tile_off(k), pb, H0{});
    } else {
      if (fh == 0)
        pv(tile_off(k), pb, H0{});
      else
        pv(tile_off(k), pb, H1{});
      if (has_next) publish(k + 1, score_tile());
    }
    return false;
  };
  // Rescale (rare), then finish tile k.  Both halves of a row take the same new maximum.
  auto rescale_finish = [&](int k, const f32x16 &sc, float mx) {
    const float m_new = fmaxf(m_run, half_max(mx));
    const float sf = fast_exp2(m_run - m_new);
#pragma unroll
    for (int ob = 0; ob < NOBW; ++ob)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[ob][i] *= sf;
    s_run *= sf;
    m_run = m_new;
    tail(k, sc);
    if (k + 1 < ntiles) publish(k + 1, score_tile());  // the step returned before publishing
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, (NB > 1 ? 1 : 0)>;
  int k = 0;
  if constexpr (NB > 1) {
    while (k < ntiles) {  // k is even here, and register set 1 holds the newest loads
      f32x16 sc;
      float mx = 0.f;
      int hk = -1;
      for (;;) {  // the back edge follows a step on set 1 only
        if (step(k, B0{}, sc, mx)) {
          hk = k;
          break;
        }
        if (k + 1 >= ntiles) break;
        if (step(k + 1, B1{}, sc, mx)) {
          hk = k + 1;
          break;
        }
        k += 2;
        if (k >= ntiles) break;
      }
      if (hk < 0) break;
      rescale_finish(hk, sc, mx);
      if (hk == k) {  // stopped on set 0: tile k+1 runs on set 1 before the loop is re-entered
        if (k + 1 >= ntiles) break;
        if (step(k + 1, B1{}, sc, mx)) rescale_finish(k + 1, sc, mx);
      }
      k += 2;
    }
  } else {
    while (true) {
      f32x16 sc;
      float mx = 0.f;
      for (; k < ntiles; ++k)
        if (step(k, B0{}, sc, mx)) break;
      if (k >= ntiles) break;
      rescale_finish(k, sc, mx);
      ++k;
    }
  }

  if (!wave_active) return;
  const float s_tot = half_sum(s_run);
  if (!row_ok) return;
  if (it.n_chunks == 1) {
    const float inv = 1.0f / s_tot;
    STCA_CHECK(rowbase + myrow < bnd.rows, kDbgAttendOut);
    float *dst = abar + (rowbase + myrow) * D + fh * (D / FH);
#pragma unroll
    for (int ob = 0; ob < NOBW; ++ob)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int f0 = 32 * ob + 8 * q + 4 * gl;
        *reinterpret_cast<f32x4 *>(dst + f0) = f32x4{oacc[ob][4 * q] * inv, oacc[ob][4 * q + 1] * inv,
                                                     oacc[ob][4 * q + 2] * inv, oacc[ob][4 * q + 3] * inv};
      }
  } else {
    const int64_t p = part_base[it.user] + (int64_t)it.chunk * R + myrow;
    STCA_CHECK(p >= 0 && p < bnd.part_rows, kDbgAttendPart);
    float *dst = part_A + p * D + fh * (D / FH);
#pragma unroll
    for (int ob = 0; ob < NOBW; ++ob)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int f0 = 32 * ob + 8 * q + 4 * gl;
        *reinterpret_cast<f32x4 *>(dst + f0) =
            f32x4{oacc[ob][4 * q], oacc[ob][4 * q + 1], oacc[ob][4 * q + 2], oacc[ob][4 * q + 3]};
      }
    if (gl == 0 && fh == 0) {
      part_ms[2 * p] = m_run;
      part_ms[2 * p + 1] = s_tot;
    }
  }
}

// ------------------------------------------------------------------------------------------
// bf16 MFMA kernel with 16 query rows per wave (v_mfma_f32_16x16x32_bf16) and eight waves per
// workgroup, two per SIMD, so that one wave's score -> softmax -> PV chain runs while the other's
// waits (a wave then needs ~220 registers at d = 256 instead of ~470; at d = 512 two waves share 16
// rows, each with half of d, as in the 32-row kernel's pairs).
//   scores  S^T[16 tok x 16 row] = X~[16 tok x 32 k] U^T[32 k x 16 row], two token blocks per tile
//   update  O^T[16 f x 16 row]  += X~^T[16 f x 32 tok] P^T[32 tok x 16 row], d/16 feature blocks
// Lane l holds query row l & 15; its score registers hold tokens 4 g + i (block 0) and 16 + 4 g + i
// (block 1), g = l >> 4.  Those eight probabilities are directly its PV B operand if k-slot
// (g, j) stands for token 4 g + j (j < 4) or 16 + 4 g + j - 4 (j >= 4); the A operand then takes,
// per lane group g, rows 4 g .. 4 g + 3 and 16 + 4 g .. 16 + 4 g + 3 of the tile at 16 consecutive
// features, two transposing LDS reads.  The row maximum and sum run over the four lanes of a row.
// LDS tile layout: chunk c of token row t at position c ^ sigma16(t), the linear map of t's low four
// bits that sends bits 0, 1, 2, 3 to 2, 4, 8, 9.  Rows are 512 bytes, so a chunk's banks are set by
// its position mod 16.  The bank-conflict counters of layout variants on gfx950 fit a 16-byte read
// served in four passes of 16 lanes, lanes l and l' sharing a pass when they share bit 5 and the
// parity of bits 2..4, and an 8-byte transposing read in two passes of 32 lanes (the two halves of
// the wave); this map gives every pass of both reads 64 distinct banks (a map that only keeps the
// 16 rows of a row-wise read apart conflicts 2-way).
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ int tile_sigma16(int t) { return ((t & 7) << 1) ^ (((t >> 3) & 1) * 9); }
__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// Reductions over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lanes of a query row) with the lane-swap
// instructions, which stay on the vector ALU.
__device__ __forceinline__ float quad_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float quad_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Tuning constants of the 16-row kernel: staged tile sets per wave at d = 256 (even), score and PV
// operand reads in flight ahead of their MFMAs.
#ifndef STCA_ATT16_NB256
#define STCA_ATT16_NB256 4
#endif
#ifndef STCA_ATT16_SA
#define STCA_ATT16_SA 3
#endif
#ifndef STCA_ATT16_PA
#define STCA_ATT16_PA 3
#endif

template <int D>
__global__ __launch_bounds__(512, 1) void attend16_kernel(
    const WorkItem *__restrict__ items, const int32_t *__restrict__ n_items, const int64_t *__restrict__ hoff,
    const int64_t *__restrict__ toff, int h, int chunk, const bf16 *__restrict__ Xt,
    const bf16 *__restrict__ U, float *__restrict__ abar, float *__restrict__ part_A,
    float *__restrict__ part_ms, const int64_t *__restrict__ part_base, const AttnBounds bnd) {
  static_assert(D == 256 || D == 512, "16-row variant laid out for d = 256 and 512");
  constexpr int CPR = D / 8;                      // 16-byte chunks per history row
  // At d = 512 the two waves w, w ^ 1 share 16 rows: each scores over its half of d and keeps half
  // of the output features, and the pair adds the partial score tiles through LDS.
  constexpr int FH = attn_feature_halves(D);
  constexpr int NKW = D / 32 / FH, NFBW = D / 16 / FH;  // score k-steps, output blocks per wave
  constexpr int INSTR = 32 * D * 2 / 1024;        // 1 KiB wave loads per 32-token tile
  constexpr int LPW = INSTR / 8;                  // per wave
  // Register sets of staged tiles: NB tiles in flight from HBM per wave (four at d = 256, where the
  // staging takes 8 registers a set; two at d = 512, where the kernel is at 256 registers).  Even, so
  // that step k's score buffers sc2[k & 1] follow from its set index.
  constexpr int NSL = 3, NB = D > 256 ? 2 : STCA_ATT16_NB256;
  static_assert(NB % 2 == 0, "score buffers alternate with the register sets");
  static_assert(NB == 2 || NB == 4, "the step loop below is unrolled for two or four register sets");
  constexpr uint32_t kRowBytes = CPR * 16, kTileBytes = 32 * kRowBytes;
  static_assert(INSTR % 8 == 0, "tile loads split evenly over 8 waves");
  __shared__ bf16x8 tiles[NSL][32 * CPR];
  // Partial score tiles of the pairs (FH = 2): [tile parity][wave][token block][lane].
  __shared__ f32x4 exch[FH > 1 ? 2 : 1][FH > 1 ? 8 : 1][2][64];

  WorkItem it;
  if (!my_item(items, n_items, it)) return;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lc = lane & 15, g = lane >> 4;
  const int64_t L0 = hoff[it.user], L1 = hoff[it.user + 1];
  const int64_t t0 = L0 + (int64_t)it.chunk * chunk;
  const int64_t t1 = (t0 + chunk < L1) ? t0 + chunk : L1;
  const int64_t T0 = toff[it.user];
  const int R = (int)((toff[it.user + 1] - T0) * h);
  const int64_t rowbase = T0 * h;
  const int fh = wave % FH;
  const int r0 = it.group * attn_rows_per_group(D) + (wave / FH) * 16;
  const bool wave_active = r0 < R;
  const int myrow = r0 + lc;
  const bool row_ok = myrow < R;
  const int ntiles = (int)((t1 - t0 + 31) / 32);
  STCA_CHECK(L0 >= 0 && L0 <= L1 && L1 <= bnd.total_L && t0 < t1, kDbgAttendRange);

  // U row of this lane as B operands: k = (D / FH) fh + 32 ks + 8 g .. + 7.
  bf16x8 ub[NKW];
  {
    const bf16 *urow = U + (rowbase + (row_ok ? myrow : 0)) * D + (D / FH) * fh + 8 * g;
#pragma unroll
    for (int ks = 0; ks < NKW; ++ks) ub[ks] = row_ok ? *reinterpret_cast<const bf16x8 *>(urow + 32 * ks) : bf16x8{};
  }

  // Tile staging: wave piece j = wave + 8 jj (1 KiB) holds, at byte 16 i, chunk (i mod CPR) ^
  // sigma16(row) of history row 32 k + row, row = (64 j + i) / CPR (rows past the chunk's end repeat
  // its last row; their scores are masked).
  int frow[LPW];
  uint32_t foff[LPW];
#pragma unroll
  for (int jj = 0; jj < LPW; ++jj) {
    const int slot = (wave + 8 * jj) * 64 + lane;
    const int row = slot / CPR, cs = slot % CPR;
    frow[jj] = row;
    foff[jj] = (uint32_t)(row * D + (cs ^ tile_sigma16(row)) * 8);
  }
  // The chunk length (at most the chunk size, an int) is uniform; read it into a scalar register so
  // that the tile tests below are scalar branches on 32-bit values.
  const int len = __builtin_amdgcn_readfirstlane((int)(t1 - t0));
  auto fetch = [&](int k, u32x4 (&rg)[LPW]) {
    const bf16 *tile = Xt + (t0 + 32 * (int64_t)k) * D;
    if (32 * (k + 1) <= len) {
#pragma unroll
      for (int jj = 0; jj < LPW; ++jj) {
        STCA_CHECK(32 * k + frow[jj] < len, kDbgAttendFetch);
        rg[jj] = *reinterpret_cast<const u32x4 *>(tile + foff[jj]);
      }
    } else {  // partial last tile: rows past the end repeat the last row
      const int rem = len - 32 * k;
#pragma unroll
      for (int jj = 0; jj < LPW; ++jj) {
        const int back = frow[jj] < rem ? 0 : (frow[jj] - rem + 1) * D;
        STCA_CHECK(rem > 0 && 32 * k + frow[jj] - back / D < len, kDbgAttendFetch);
        rg[jj] = *reinterpret_cast<const u32x4 *>(tile + (foff[jj] - back));
      }
    }
  };
  auto put = [&](int b, const u32x4 (&rg)[LPW]) {
#pragma unroll
    for (int jj = 0; jj < LPW; ++jj) tiles[b][(wave + 8 * jj) * 64 + lane] = __builtin_bit_cast(bf16x8, rg[jj]);
  };
  auto sync = [&]() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // Register set b holds tile j >= 2 with (j - 2) mod NB = b between its fetch and its put.  Every
  // step fetches (past the last tile it re-reads the last one, which is never consumed), so the
  // compiler sees the same loads in flight on every path and each put waits for the older set only.
  u32x4 rgb[NB][LPW];
  fetch(0, rgb[0]);
  put(0, rgb[0]);
  if (1 < ntiles) {
    fetch(1, rgb[0]);
    put(1, rgb[0]);
  }
#pragma unroll
  for (int b = 0; b < NB; ++b) fetch(min(2 + b, ntiles - 1), rgb[b]);

  // LDS byte offsets.  Scores: token row 16 tb + lc, chunk 4 ks + g at position
  // (4 ks + g) ^ sigma = 4 ks ^ (g ^ sigma): offset row + ((64 ks) ^ (16 x)).  PV: lane 4 j + q of
  // group g reads token 16 h + 4 g + j (sigma = 2 (4 (g & 1) + j) + (g >> 1), the same for both h),
  // features 16 fb + 4 q .. + 3: chunk 2 fb + (q >> 1) at position 2 fb ^ y, y = (q >> 1) ^ sigma,
  // i.e. 2 ((fb & 8) | ((fb & 7) ^ (y >> 1))) + (y & 1); one base per fb & 7.
  const STCA_LDS char *lds = (const STCA_LDS char *)&tiles[0][0];
  uint32_t srow[2], sx[2];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const int t = 16 * tb + lc;
    srow[tb] = (uint32_t)t * kRowBytes;
    sx[tb] = (uint32_t)(16 * (g ^ tile_sigma16(t)));
  }
  uint32_t pvb[8];
  {
    const int j = lc >> 2, q = lc & 3;
    const int sig = tile_sigma16(4 * g + j);
    const int y = (q >> 1) ^ sig;
#pragma unroll
    for (int m = 0; m < 8; ++m)
      pvb[m] = (uint32_t)((4 * g + j) * kRowBytes + 32 * (m ^ (y >> 1)) + 16 * (y & 1) + 8 * (q & 1));
  }

  f32x4 oacc[NFBW];
#pragma unroll
  for (int fb = 0; fb < NFBW; ++fb) oacc[fb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, s_run = 0.f;

  // Rescale (a row maximum outgrew the slack; the first tile always does), then the probabilities of
  // tile k against the new maximum.
  auto rescale_probs = [&](const f32x4 (&sc)[2], float mx, bf16x8 &pb, float &psum) {
    const float m_new = fmaxf(m_run, mx);
    const float sf = fast_exp2(m_run - m_new);
#pragma unroll
    for (int fb = 0; fb < NFBW; ++fb) oacc[fb] *= sf;
    s_run *= sf;
    m_run = m_new;
    psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = fast_exp2(sc[e >> 2][e & 3] - m_run);
      pb[e] = f32_to_bf16(p);
      psum += p;
    }
  };
  auto mask = [&](int k, f32x4 (&sc)[2]) {
    const int remk = len - 32 * k;
    if (remk < 32) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (16 * tb + 4 * g + i >= remk) sc[tb][i] = -INFINITY;
    }
  };
  // Score operand i = 2 ks + tb of tile k: this wave's half of d starts (D / FH) fh features into a
  // row, a multiple of 16 chunks, which the swizzle (low four bits of the chunk index) leaves alone.
  constexpr int SA = STCA_ATT16_SA;
  const uint32_t hofs = (uint32_t)(fh * (D / FH) * 2);
  // The feature half enters the PV bases once here: added per read, next to the slot offset, the
  // compiler recomputed every transposed read's address (three vector instructions each).
#pragma unroll
  for (int m = 0; m < 8; ++m) pvb[m] += hofs;
  auto frag_at = [&](int k, int i) {
    const uint32_t toff = (uint32_t)((k % NSL) * kTileBytes);
    const int ks = i >> 1, tb = i & 1;
    return *(const STCA_LDS bf16x8 *)(lds + toff + srow[tb] + hofs + (((uint32_t)(64 * ks)) ^ sx[tb]));
  };
  // Pairs: publish this wave's partial score tile of tile k; after the next workgroup barrier the
  // partner adds it (both then hold bit-identical scores, a + b = b + a, and take the same decisions).
  auto publish = [&](int k, const f32x4 (&part)[2]) {
    if constexpr (FH > 1) {
      exch[k & 1][wave][0][lane] = part[0];
      exch[k & 1][wave][1][lane] = part[1];
    }
  };
  auto add_partner = [&](int k, f32x4 (&sc)[2]) {
    if constexpr (FH > 1) {
      sc[0] += exch[k & 1][wave ^ 1][0][lane];
      sc[1] += exch[k & 1][wave ^ 1][1][lane];
    }
  };
  // PV product of tile k: the transposed operands of feature block fb + PA are read while block fb
  // multiplies.
  constexpr int PA = STCA_ATT16_PA;
  auto pv = [&](int k, const bf16x8 &pb) {
    const uint32_t toff = (uint32_t)((k % NSL) * kTileBytes);
    // The eight lane bases of this tile's slot.  At d = 512 they are formed once per step (left to
    // itself the compiler re-derived an address per read there); the feature-block offsets then fit
    // the reads' immediates.  At d = 256 the compiler's own choice is as good and needs fewer registers.
    uint32_t bs[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      bs[m] = pvb[m] + toff;
      if constexpr (FH > 1) asm volatile("" : "+v"(bs[m]));
    }
    auto xfrag = [&](int fb) {  // this wave's feature block fb: global block (NFBW fh + fb)
      const uint32_t o = bs[fb & 7] + 256 * (fb >> 3);
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((STCA_LDS s16x4 *)(lds + o));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((STCA_LDS s16x4 *)(lds + o + 16 * kRowBytes));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    bf16x8 xr[PA + 1];
#pragma unroll
    for (int fb = 0; fb < PA; ++fb) xr[fb] = xfrag(fb);
#pragma unroll
    for (int fb = 0; fb < NFBW; ++fb) {
      if (fb + PA < NFBW) xr[(fb + PA) % (PA + 1)] = xfrag(fb + PA);
      oacc[fb] = mfma16x16x32(xr[fb % (PA + 1)], pb, oacc[fb]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Step k: the scores of tile k + 1 on the matrix cores while the vector ALU turns tile k's scores
  // (from step k - 1) into probabilities, one MFMA and one probability per group in an order pinned
  // with sched_barrier; then the PV product of tile k.  The probabilities are taken against the
  // running maximum before the tile's own maximum is known; if that maximum outgrew the slack they
  // are recomputed after the rescale (exact either way).  Score operand reads run SA fragments
  // ahead.  Register set BI holds the staged tile and names the score buffers (tile k's in
  // sc2[BI], tile k + 1's into sc2[BI ^ 1]).
  f32x4 sc2[2][2];
  auto step = [&](int k, auto BI) {
    constexpr int b = decltype(BI)::value;
    sync();  // tile k+1 is in LDS; tile k-1's slot is free
    // Unconditional, like the fetch: past the last tile this writes a tile no step reads into the
    // free slot, and the compiler's count of loads in flight stays the same on every path.
    put((k + 2) % NSL, rgb[b]);
    fetch(min(k + 2 + NB, ntiles - 1), rgb[b]);
    if (!wave_active) return;
    f32x4(&cur)[2] = sc2[b & 1];
    f32x4(&nxt)[2] = sc2[(b & 1) ^ 1];
    add_partner(k, cur);
    mask(k, cur);
    bf16x8 pb;
    float psum = 0.f, mx = -INFINITY;
    auto element = [&](int e) {
      const float v = cur[e >> 2][e & 3];
      const float p = fast_exp2(v - m_run);
      pb[e] = f32_to_bf16(p);
      psum += p;
      mx = fmaxf(mx, v);
    };
    if (k + 1 < ntiles) {
      bf16x8 fr[SA + 1];
#pragma unroll
      for (int i = 0; i < SA; ++i) fr[i] = frag_at(k + 1, i);
      nxt[0] = nxt[1] = f32x4{0.f, 0.f, 0.f, 0.f};
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 2 * NKW; ++i) {
        if (i + SA < 2 * NKW) fr[(i + SA) % (SA + 1)] = frag_at(k + 1, i + SA);
        nxt[i & 1] = mfma16x16x32(fr[i % (SA + 1)], ub[i >> 1], nxt[i & 1]);
        if (i < 8) element(i);
        __builtin_amdgcn_sched_barrier(0);
      }
      publish(k + 1, nxt);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) element(e);
    }
    mx = quad_max(mx);
    if (wave_any(mx > m_run + kLazy)) rescale_probs(cur, mx, pb, psum);
    s_run += psum;
    pv(k, pb);
  };
  sync();
  if (wave_active) {  // scores of the first tile (step 0 adds the partner's half after its barrier)
    sc2[0][0] = sc2[0][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 2 * NKW; ++i) sc2[0][i & 1] = mfma16x16x32(frag_at(0, i), ub[i >> 1], sc2[0][i & 1]);
    publish(0, sc2[0]);
  }
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  using B2 = std::integral_constant<int, (NB > 2 ? 2 : 0)>;
  using B3 = std::integral_constant<int, (NB > 3 ? 3 : 0)>;
  int k = 0;
  for (; k + NB - 1 < ntiles; k += NB) {  // the back edge follows a step on the last register set only
    step(k, B0{});
    step(k + 1, B1{});
    if constexpr (NB > 2) step(k + 2, B2{});
    if constexpr (NB > 3) step(k + 3, B3{});
  }
  if (k < ntiles) step(k, B0{});
  if (k + 1 < ntiles) step(k + 1, B1{});
  if constexpr (NB > 2)
    if (k + 2 < ntiles) step(k + 2, B2{});

  if (!wave_active) return;
  const float s_tot = quad_sum(s_run);
  if (!row_ok) return;
  if (it.n_chunks == 1) {
    const float inv = 1.0f / s_tot;
    STCA_CHECK(rowbase + myrow < bnd.rows, kDbgAttendOut);
    float *dst = abar + (rowbase + myrow) * D + (D / FH) * fh + 4 * g;
#pragma unroll
    for (int fb = 0; fb < NFBW; ++fb) *reinterpret_cast<f32x4 *>(dst + 16 * fb) = oacc[fb] * inv;
  } else {
    const int64_t p = part_base[it.user] + (int64_t)it.chunk * R + myrow;
    STCA_CHECK(p >= 0 && p < bnd.part_rows, kDbgAttendPart);
    float *dst = part_A + p * D + (D / FH) * fh + 4 * g;
#pragma unroll
    for (int fb = 0; fb < NFBW; ++fb) *reinterpret_cast<f32x4 *>(dst + 16 * fb) = oacc[fb];
    if (g == 0 && fh == 0) {
      part_ms[2 * p] = m_run;
      part_ms[2 * p + 1] = s_tot;
    }
  }
}

// ------------------------------------------------------------------------------------------
// fp32 kernel (vector ALU): 16 waves per work item, one wave per query row, the history taken 64 tokens
// at a time.
//   * scores: one token per lane, the lane's dot product of its token row with u (u staged in LDS and
//     read as a broadcast), so a block's maximum costs one wave reduction instead of one per token;
//   * weighted sum: one output feature per lane (E = D / 64 of them), each token's probability read
//     from the lane that scored it; token rows past the chunk are clamped to its last row and carry
//     probability 0.
// ------------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(1024) void attend_f32_kernel(
    const WorkItem *__restrict__ items, const int32_t *__restrict__ n_items, const int64_t *__restrict__ hoff,
    const int64_t *__restrict__ toff, int h, int chunk, const float *__restrict__ Xt,
    const float *__restrict__ U, float *__restrict__ abar, float *__restrict__ part_A,
    float *__restrict__ part_ms, const int64_t *__restrict__ part_base, const AttnBounds bnd) {
  constexpr int E = D / 64;
  constexpr int UJ = E >= 4 ? 8 : 16;  // tokens whose rows are in flight at once in the weighted sum
  constexpr int W = 16;
  __shared__ f32x4 us[W][D / 4];
  WorkItem it;
  if (!my_item(items, n_items, it)) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t L0 = hoff[it.user], L1 = hoff[it.user + 1];
  const int64_t t0 = L0 + (int64_t)it.chunk * chunk;
  const int64_t t1 = (t0 + chunk < L1) ? t0 + chunk : L1;
  const int64_t T0 = toff[it.user];
  const int R = (int)((toff[it.user + 1] - T0) * h);
  const int64_t rowbase = T0 * h;
  const int RG = attn_rows_per_group(D);
  const int rend = (it.group + 1) * RG < R ? (it.group + 1) * RG : R;
  STCA_CHECK(L0 >= 0 && L0 <= L1 && L1 <= bnd.total_L && t0 < t1, kDbgAttendRange);
  float *ul = reinterpret_cast<float *>(us[wave]);

  for (int r = it.group * RG + wave; r < rend; r += W) {
    // The wave's LDS accesses complete in issue order, so the staged row is seen by every lane's reads,
    // and the previous row's reads are done before it is overwritten.
#pragma unroll
    for (int e = 0; e < E; ++e) ul[lane + 64 * e] = U[(rowbase + r) * D + lane + 64 * e];
    float a[E];
#pragma unroll
    for (int e = 0; e < E; ++e) a[e] = 0.f;
    float m = -INFINITY, sl = 0.f;
    for (int64_t p = t0; p < t1; p += 64) {
      const int64_t key = p + lane;
      const int64_t kr = key < t1 ? key : t1 - 1;
      const f32x4 *xr = reinterpret_cast<const f32x4 *>(Xt + kr * D);
      float d0 = 0.f, d1 = 0.f, d2 = 0.f, d3 = 0.f;
#pragma unroll 16
      for (int f = 0; f < D / 4; ++f) {
        const f32x4 x = xr[f], u = us[wave][f];
        d0 = fmaf(x[0], u[0], d0);
        d1 = fmaf(x[1], u[1], d1);
        d2 = fmaf(x[2], u[2], d2);
        d3 = fmaf(x[3], u[3], d3);
      }
      const float sc = key < t1 ? (d0 + d1) + (d2 + d3) : -INFINITY;
      const float m_new = fmaxf(m, wave_max(sc));
      const float sf = exp2f(m - m_new);
      const float pj = exp2f(sc - m_new);
      sl = fmaf(sl, sf, pj);
#pragma unroll
      for (int e = 0; e < E; ++e) a[e] *= sf;
      m = m_new;
      const int nk = (int)(t1 - p < 64 ? t1 - p : 64);
      for (int jb = 0; jb < nk; jb += UJ) {
        float x[UJ][E], w[UJ];
#pragma unroll
        for (int jj = 0; jj < UJ; ++jj) {
          const int64_t row = (p + jb + jj < t1) ? p + jb + jj : t1 - 1;
          w[jj] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pj), jb + jj));
#pragma unroll
          for (int e = 0; e < E; ++e) x[jj][e] = Xt[row * D + lane + 64 * e];
        }
#pragma unroll
        for (int jj = 0; jj < UJ; ++jj)
#pragma unroll
          for (int e = 0; e < E; ++e) a[e] = fmaf(w[jj], x[jj][e], a[e]);
      }
    }
    const float s = wave_sum(sl);
    if (it.n_chunks == 1) {
      const float inv = 1.0f / s;
      STCA_CHECK(rowbase + r < bnd.rows, kDbgAttendOut);
#pragma unroll
      for (int e = 0; e < E; ++e) abar[(rowbase + r) * D + lane + 64 * e] = a[e] * inv;
    } else {
      const int64_t pidx = part_base[it.user] + (int64_t)it.chunk * R + r;
      STCA_CHECK(pidx >= 0 && pidx < bnd.part_rows, kDbgAttendPart);
#pragma unroll
      for (int e = 0; e < E; ++e) part_A[pidx * D + lane + 64 * e] = a[e];
      if (lane == 0) {
        part_ms[2 * pidx] = m;
        part_ms[2 * pidx + 1] = s;
      }
    }
  }
}

// The 16-row kernel serves d = 256 and 512 (measured against the 32-row kernel in same-process A/Bs of
// whole forwards: stress20k 209.8 against 214.5 ms, dense10k 51.14 against 51.33 ms, ragged attention
// 0.172 against 0.200 ms per launch); d = 64 and 128 keep the 32-row kernel.

template <int D>
static hipError_t attend_split_d(hipStream_t s, const AttnPlan &p, bool bf16_path, const int64_t *hoff,
                                 const int64_t *toff, const void *Xt, const void *U, float *abar,
                                 const AttnBuffers &b) {
  const dim3 grid((unsigned)p.max_items), block(256);
  const AttnBounds bnd{p.total_L, p.total_T * p.h, p.max_part_rows};
  if (bf16_path) {
    if constexpr (D >= 256)
      hipLaunchKernelGGL((attend16_kernel<D>), grid, dim3(512), 0, s, b.items, b.n_items, hoff, toff, p.h, p.chunk,
                         (const bf16 *)Xt, (const bf16 *)U, abar, b.part_A, b.part_ms, b.part_base, bnd);
    else
      hipLaunchKernelGGL((attend_mfma_kernel<D>), grid, block, 0, s, b.items, b.n_items, hoff, toff, p.h, p.chunk,
                         (const bf16 *)Xt, (const bf16 *)U, abar, b.part_A, b.part_ms, b.part_base, bnd);
  }
  else
    hipLaunchKernelGGL((attend_f32_kernel<D>), grid, dim3(1024), 0, s, b.items, b.n_items, hoff, toff, p.h, p.chunk,
                       (const float *)Xt, (const float *)U, abar, b.part_A, b.part_ms, b.part_base, bnd);
  return hipGetLastError();
}

hipError_t attend_split(hipStream_t s, const AttnPlan &p, bool bf16_path, const int64_t *hist_off,
                        const int64_t *tgt_off, const void *Xt, const void *U, float *abar,
                        const AttnBuffers &b) {
  if (p.max_items <= 0) return hipSuccess;
  switch (p.d) {
    case 64: return attend_split_d<64>(s, p, bf16_path, hist_off, tgt_off, Xt, U, abar, b);
    case 128: return attend_split_d<128>(s, p, bf16_path, hist_off, tgt_off, Xt, U, abar, b);
    case 256: return attend_split_d<256>(s, p, bf16_path, hist_off, tgt_off, Xt, U, abar, b);
    case 512: return attend_split_d<512>(s, p, bf16_path, hist_off, tgt_off, Xt, U, abar, b);
    default: return hipErrorInvalidValue;
  }
}

// ------------------------------------------------------------------------------------------
// Merge of split-L partial softmax states (exact: rescale each chunk's sum and accumulator by
// 2^(m_c - max_c m_c), then divide).  Fixed chunk order, so the result is deterministic.  Users
// with one chunk were finalised by the attention kernel; users with an empty history get NaN.
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void combine_kernel(int64_t n_rows, int h, int D,
                                                      const int32_t *__restrict__ status,
                                                      const int32_t *__restrict__ tgt_user,
                                                      const int32_t *__restrict__ user_nchunks,
                                                      const int64_t *__restrict__ toff,
                                                      const int64_t *__restrict__ part_base,
                                                      const float *__restrict__ part_A,
                                                      const float *__restrict__ part_ms, float *__restrict__ abar,
                                                      int64_t part_rows) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= n_rows) return;
  float *dst = abar + row * D;
  if (status[1] != 0) {  // the work list found inconsistent offsets: no row was computed
    for (int f = lane; f < D; f += 64) dst[f] = NAN;
    return;
  }
  const int u = tgt_user[row / h];
  const int nc = user_nchunks[u];
  if (nc == 1) return;
  if (nc == 0) {
    for (int f = lane; f < D; f += 64) dst[f] = NAN;
    return;
  }
  const int64_t R = (toff[u + 1] - toff[u]) * h;
  const int64_t r = row - toff[u] * h;
  const int64_t p0 = part_base[u] + r;
  STCA_CHECK(p0 >= 0 && p0 + (int64_t)(nc - 1) * R < part_rows, kDbgCombinePart);
  (void)part_rows;
  float mstar = -INFINITY;
  for (int c = 0; c < nc; ++c) mstar = fmaxf(mstar, part_ms[2 * (p0 + c * R)]);
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float s = 0.f;
  for (int c = 0; c < nc; ++c) {
    const int64_t p = p0 + c * R;
    const float w = exp2f(part_ms[2 * p] - mstar);
    s += part_ms[2 * p + 1] * w;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int f = lane + 64 * e;
      if (f < D) acc[e] += part_A[p * D + f] * w;
    }
  }
  const float inv = 1.0f / s;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int f = lane + 64 * e;
    if (f < D) dst[f] = acc[e] * inv;
  }
}

hipError_t attend_combine(hipStream_t s, const AttnPlan &p, const int64_t *tgt_off, float *abar,
                          const AttnBuffers &b) {
  const int64_t rows = p.total_T * p.h;
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, rows, p.h, p.d,
                     b.n_items, b.tgt_user, b.user_nchunks, tgt_off, b.part_base, b.part_A, b.part_ms, abar,
                     p.max_part_rows);
  return hipGetLastError();
}

// Debug build: the file's check word, read (and cleared) through its symbol.
#ifdef STCA_DEBUG_BOUNDS
__global__ void debug_selftest_kernel() { STCA_CHECK(threadIdx.x != 0, kDbgSelfTest); }
#endif

hipError_t debug_flags_attend(uint32_t *flags, bool clear) {
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

hipError_t debug_selftest(hipStream_t s) {
#ifdef STCA_DEBUG_BOUNDS
  hipLaunchKernelGGL(debug_selftest_kernel, dim3(1), dim3(64), 0, s);
  return hipGetLastError();
#else
  (void)s;
  return hipSuccess;
#endif
}

}  // namespace stca
