// Fused history encode on bf16 MFMA: X~ = LN(((X W_u) * SiLU(X W_v)) W_o), for one layer or for
// all layers of the stack in one launch (each tile of X read once).
//
// Equations: SwiGLU FFN of eq. (1) with the three-matrix shapes of the STCA review page
// (section 2.2), followed by the LayerNorm of eq. (2) ("Make It Long, Keep It Fast", section 2.1).
//
// Work decomposition (gfx950, 64-wide waves, v_mfma_f32_32x32x16_bf16):
//   * waves work in pairs; a pair owns 32 TB history tokens for the whole FFN and each wave keeps
//     all of them in registers as MFMA B operands (TB = 32-token blocks per wave);
//   * rd is walked in steps of 32 hidden features.  In each step wave `role` of a pair computes,
//     for its 16 hidden features and the pair's tokens, the transposed up and gate products in
//     ONE accumulator per 32 tokens: the A operand stacks the 16 W_u columns (rows 0-15) on the 16
//     W_v columns (rows 16-31), so accumulator registers i and i+8 of a lane hold the up and gate
//     value of the same feature and token, and the SwiGLU gate is lane-local;
//   * the gated values of a lane form exactly one B operand (16 hidden features x 32 tokens) of
//     the down product; the pair swaps these through LDS (1 KiB per wave, block and step), and
//     each wave accumulates half of the d outputs, Y^T[d/2 x tokens] += W_o^T[d/2 x 32] H^T;
//   * weights are pre-packed in fragment order (1 KiB = one wave operand), bit for bit as given
//     (the gate applies its exp2 scaling in fp32, so no weight is rounded twice); fragments are
//     staged step by step into LDS with direct global->LDS loads and shared by all waves of the
//     workgroup, or read by each wave from L2 straight into registers (down fragments at d >= 256);
//   * LayerNorm statistics of a token combine the two waves of its pair through LDS;
//   * workgroups are persistent and walk 128-token tiles (64 at d = 512), every layer of a tile
//     before the next tile; the next item's rows and first weight steps are loaded while the
//     current one finishes.  Between the layers of a tile the rows stay on chip (d <= 256: the
//     pair's B operands are written back to the LDS row buffer; d = 512: re-read, from L2).
// d <= 256: a workgroup is 8 waves (TB = 1, two per SIMD; d < 256) or 4 (TB = 2, one per SIMD;
// d = 256) over 128 tokens, whose rows are staged in LDS with coalesced loads and read out in the
// B-operand layout; the up/gate fragments are staged two steps ahead in a 3-slot ring.  d = 512: a
// step of weights is 96 KiB, so only the up/gate part is staged (two slots, one step ahead), the
// rows are loaded straight into registers, and each wave loads its down fragments from L2; 4 waves
// over 64 tokens.
#include <algorithm>
#include <type_traits>

#include "device_common.hpp"
#include "internal.hpp"


namespace stca {

size_t encode_packed_bytes(int d, int r) { return (size_t)(r * d / 32) * (size_t)(3 * d / 16) * 1024; }
size_t encode_layer_stride(int d, int r) { return (encode_packed_bytes(d, r) + 8 * (size_t)d + 255) / 256 * 256; }

// ------------------------------------------------------------------------------------------
// Fragment re-layout.  Step s (hidden features 32s .. 32s+31) holds 3d/16 fragments of 64 lanes x
// 8 bf16, in order:
//   up/gate part, 2 d/16 fragments: fragment role * d/16 + ks: lane l, slot e, row = l & 31:
//       W_u[16 ks + 8 (l>>5) + e][32 s + 16 role + row]        for row < 16,
//       W_v[16 ks + 8 (l>>5) + e][32 s + 16 role + row - 16]   for row >= 16;
//   down part, 2 d/32 fragments for (32-wide output block ob, 16-feature block kk):
//       lane l, slot e = W_o[32 s + phi(kk, l>>5, e)][32 ob + (l&31)],
//     phi(kk, g, e) = 16 kk + 8 (e>>2) + 4 g + (e&3): the hidden feature whose gated value sits in
//     slot e of the lane-group-g B operand built from 16-feature block kk.
//     fragment d/8 + (d/32) (kk ^ owner) + ob, owner = ob / (d/64) the role of the wave that
//     accumulates block ob, so a wave finds its own-feature blocks and its partner-feature blocks
//     as two runs at power-of-two offsets.
// ------------------------------------------------------------------------------------------
// With gamma and beta given, the layer's LayerNorm parameters follow the fragments (gamma, then
// beta, d floats each), so that a multi-layer encode finds every layer's data at one stride.
__global__ __launch_bounds__(256) void encode_pack_kernel(int d, int rd, const uint16_t *__restrict__ Wu,
                                                          const uint16_t *__restrict__ Wv,
                                                          const uint16_t *__restrict__ Wo,
                                                          uint16_t *__restrict__ out,
                                                          const float *__restrict__ gamma,
                                                          const float *__restrict__ beta) {
  const int NKS = d / 16, NOB = d / 32, FPS = 2 * NKS + 2 * NOB;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)(rd / 32) * FPS * 64;
  if (gid >= total) {
    const int64_t i = gid - total;
    if (gamma && i < 2 * d) {
      float *ln = reinterpret_cast<float *>(out + total * 8);
      ln[i] = i < d ? gamma[i] : beta[i - d];
    }
    return;
  }
  const int lane = (int)(gid & 63);
  const int64_t fr = gid >> 6;
  const int s = (int)(fr / FPS), f = (int)(fr % FPS);
  const int col = lane & 31, g = lane >> 5;
  uint16_t v[8];
  if (f < 2 * NKS) {
    const int role = f / NKS, ks = f % NKS;
    const uint16_t *W = col < 16 ? Wu : Wv;
    const int fc = 32 * s + 16 * role + (col & 15);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = W[(int64_t)(16 * ks + 8 * g + e) * rd + fc];
  } else {
    const int idx = f - 2 * NKS;
    const int ob = idx % NOB, kk = (idx / NOB) ^ (ob / (NOB / 2));
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int phi = 16 * kk + 8 * (e >> 2) + 4 * g + (e & 3);
      v[e] = Wo[(int64_t)(32 * s + phi) * d + 32 * ob + col];
    }
  }
  uint16_t *o = out + (fr * 64 + lane) * 8;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = v[e];
}

hipError_t encode_pack(hipStream_t s, int d, int r, const void *Wu, const void *Wv, const void *Wo,
                       void *packed, const float *gamma, const float *beta) {
  const int rd = r * d;
  const int64_t total = (int64_t)(rd / 32) * (3 * d / 16) * 64 + (gamma ? 2 * d : 0);
  hipLaunchKernelGGL(encode_pack_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, d, rd,
                     (const uint16_t *)Wu, (const uint16_t *)Wv, (const uint16_t *)Wo, (uint16_t *)packed,
                     gamma, beta);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------------
// The fused kernel, d <= 256: wave pairs.
// ------------------------------------------------------------------------------------------
template <int D> struct PairShape {
  static constexpr int NKS = D / 16;         // 16-deep k-steps over d (up/gate products)
  static constexpr int NOB = D / 32;         // 32-wide output blocks (down product)
  static constexpr int NOBW = NOB / 2;       // output blocks per wave of a pair
  static constexpr int FUP = 2 * NKS;        // up/gate fragments per step (NKS per role)
  static constexpr int FDN = 2 * NOB;        // down fragments per step, (ob, kk)
  static constexpr int FPS = FUP + FDN;      // fragments per step (3d/16)
  static constexpr int NG = NKS + 2 * NOBW;  // fragment groups per wave and step, 2 MFMAs each
  static constexpr int FD = 2 * NOBW;        // down groups per wave and step
  static_assert(NOBW >= 1, "shape");
};

// Group g of a step's MFMA stream: every third group (while they last) is a down group.
__host__ __device__ constexpr bool pair_is_down(int g, int fd) { return (g % 3) == 2 && (g / 3) < fd; }
__host__ __device__ constexpr int pair_up_idx(int g, int fd) { return g - (g / 3 < fd ? (g + 1) / 3 : fd); }

// LDS fragment ring of the steady steps (reads run STCA_ENC_RING - 1 groups ahead of their MFMAs):
// at TB = 2 a fragment feeds two MFMAs and one group ahead covers the LDS latency; TB = 1 keeps four.
#ifndef STCA_ENC_RING
#define STCA_ENC_RING 2
#endif
#ifndef STCA_ENC_RING_SMALL
#define STCA_ENC_RING_SMALL 4
#endif
// 32-token blocks per wave at d = 256 and at smaller d.
#ifndef STCA_ENC_TB
#define STCA_ENC_TB 2
#endif
#ifndef STCA_ENC_TB_SMALL
#define STCA_ENC_TB_SMALL 1
#endif
#ifndef STCA_ENC_GO
#define STCA_ENC_GO 1
#endif
#ifndef STCA_ENC_STAGGER
#define STCA_ENC_STAGGER 24
#endif
// Up/gate fragment reads in flight ahead of their MFMAs outside the steady loop (every step at
// d = 512, the first and last steps of an item at d = 256).
#ifndef STCA_ENC_UA_WIDE
#define STCA_ENC_UA_WIDE 6
#endif
#ifndef STCA_ENC_UA
#define STCA_ENC_UA 3
#endif
// Steady steps at d = 256: a gate element goes with every MFMA k with k % 3 == STCA_ENC_GATE_PH, a
// staging load with every k with k % 6 == STCA_ENC_STAGE_PH.
#ifndef STCA_ENC_GATE_PH
#define STCA_ENC_GATE_PH 0
#endif
#ifndef STCA_ENC_STAGE_PH
#define STCA_ENC_STAGE_PH 3
#endif

// TB = 32-token blocks per wave: TB = 2 gives 4 waves of up to 512 registers (one per SIMD), TB = 1
// gives 8 waves of up to 256 registers (two per SIMD); either way a workgroup covers 128 tokens.
// At d = 256 TB = 2 reads half as many fragment bytes per MFMA, which saves power: the kernel runs
// at the chip's power limit, and with the step schedule below TB = 2 measures 8-9% faster than
// TB = 1 there (whole forwards); at d = 128 TB = 1 was the faster one when last compared.
// At d = 512 (wide) a step of weights is 96 KiB: only the up/gate part goes through LDS (two
// slots), each wave reads its W_o fragments from L2 into registers one step ahead of their use,
// and the workgroup is 4 waves of one 32-token block (64 tokens), one wave per SIMD.
template <int D, int TB> struct PairLaunch {
  static constexpr bool kWide = D > 256;
  static constexpr int NW = kWide ? 4 : 8 / TB;            // waves per workgroup
  static constexpr int kTokens = (NW / 2) * 32 * TB;       // tokens per workgroup
  // d = 256: the down (W_o) fragments bypass LDS too, streamed from L2 into a register ring half
  // a step ahead of their use; LDS then carries only the up/gate fragments.
  static constexpr bool kGO = STCA_ENC_GO && D == 256;
};

template <int D, int TB, bool LN, typename TO>
__global__ __launch_bounds__((64 * PairLaunch<D, TB>::NW), 1) void encode_pair_kernel(int64_t n_rows, int n_steps,
                                                             const bf16 *__restrict__ X, int64_t ldx,
                                                             const EncodeLayers lay, int64_t ldo, float eps,
                                                             int stagger) {
  using S = PairShape<D>;
  constexpr bool kWide = PairLaunch<D, TB>::kWide;
  constexpr int NW = PairLaunch<D, TB>::NW;
  constexpr int kTokens = PairLaunch<D, TB>::kTokens;
  constexpr bool kGO = PairLaunch<D, TB>::kGO;
  constexpr bool kNoO = kWide || kGO;  // no down fragments in LDS
  // Direct-to-LDS loads per wave and step: fragments go round-robin over the waves; the barrier
  // wait uses the smallest per-wave count, which waits for at least all loads of older steps.
  constexpr int LUV = (S::FUP + NW - 1) / NW, LO = (S::FDN + NW - 1) / NW;
  constexpr int kStepLoads = kGO ? S::FD / 2 : S::FUP / NW + S::FDN / NW;
  constexpr int kRing = TB == 2 ? STCA_ENC_RING : STCA_ENC_RING_SMALL, kAhead = kRing - 1;  // groups in flight
  constexpr uint32_t SLOT = S::FPS * 1024u;                          // bytes of one ring slot
  // Weight ring: slot b holds the up/gate fragments of one step (uvN) and the down fragments of
  // another (oN), see the step schedule below.  Every part is an array of its own so that the
  // compiler sees reads of one slot as independent of the loads landing in another and does not
  // wait for those loads.
  __shared__ bf16x8 uv0[S::FUP][64], uv1[S::FUP][64], uv2[kWide ? 1 : S::FUP][64];
  __shared__ bf16x8 o0[kNoO ? 1 : S::FDN][64], o1[kNoO ? 1 : S::FDN][64], o2[kNoO ? 1 : S::FDN][64];
  auto uv_slot = [&](int b) -> const STCA_LDS char * {
    return (const STCA_LDS char *)(b == 0 ? &uv0[0][0] : b == 1 ? &uv1[0][0] : &uv2[0][0]);
  };
  auto o_slot = [&](int b) -> const STCA_LDS char * {
    return (const STCA_LDS char *)(b == 0 ? &o0[0][0] : b == 1 ? &o1[0][0] : &o2[0][0]);
  };
  // Gated activations swapped within a pair: [step parity][wave][32-token block][lane].
  __shared__ bf16x8 hx[2][NW][TB][64];
  // d <= 256: a tile's rows are staged in LDS, rows 0-63 in ring slot 2 (its up/gate part is
  // loaded only once the rows have been read) and rows 64-127 in xs.
  __shared__ bf16x8 xs[kWide ? 1 : S::FUP][64];

  // The wave index is uniform: keeping it in a scalar register makes the LDS destinations of the
  // staging loads (M0) scalar arithmetic.
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int role = wave & 1, partner = wave ^ 1;
  const int col = lane & 31, grp = lane >> 5;
  const int S_ = n_steps;

  // LayerNorm scale and shift, staged once into LDS (visible after the first barrier) so that the
  // epilogue does not wait on global loads.
  // With several layers, the next item's parameters are written into the other half of a double
  // buffer while an item runs: gb[parity][gamma / beta][feature].
  const int NL = lay.n;
  __shared__ __attribute__((aligned(16))) float gb[LN ? 2 : 1][2][LN ? D : 4];
  if constexpr (LN) {
    for (int i = threadIdx.x; i < D; i += 64 * NW) {
      gb[0][0][i] = lay.gamma[i];
      gb[0][1][i] = lay.beta[i];
    }
  }
  // The layer in flight: its packed weights (and a buffer resource over them for the staging loads).
  const bf16x8 *packed = (const bf16x8 *)lay.packed;
  __amdgpu_buffer_rsrc_t wrs = make_rsrc(packed, (uint32_t)n_steps * SLOT);
  auto use_layer = [&](int l) {
    packed = (const bf16x8 *)((const char *)lay.packed + (int64_t)l * lay.packed_stride);
    wrs = make_rsrc(packed, (uint32_t)n_steps * SLOT);
  };
  auto stage_uv = [&](int t, int b) {
#pragma unroll
    for (int j = 0; j < LUV; ++j) {
      const int f = wave + NW * j;
      if (S::FUP % NW != 0 && f >= S::FUP) break;
      load_lds16(wrs, (STCA_LDS void *)(uv_slot(b) + f * 1024), (uint32_t)(f * 64 + lane) * 16u,
                 (uint32_t)t * SLOT);
    }
  };
  auto stage_o = [&](int t, int b) {
#pragma unroll
    for (int j = 0; j < LO; ++j) {
      const int f = wave + NW * j;
      if (S::FDN % NW != 0 && f >= S::FDN) break;
      load_lds16(wrs, (STCA_LDS void *)(o_slot(b) + f * 1024), (uint32_t)((S::FUP + f) * 64 + lane) * 16u,
                 (uint32_t)t * SLOT);
    }
  };
  // The up/gate fragments of the first steps of a tile; at d <= 256 the third goes into slot 2
  // only after the tile's rows have been read out of it.
  auto stage_first = [&]() {
    stage_uv(0, 0);
    if (S_ > 1) stage_uv(1, 1);
  };

  // d <= 256: tile rows into LDS with coalesced direct-to-LDS loads.  Row r (2d bytes, d/8
  // chunks of 16 bytes) occupies positions r d/8 .. r d/8 + d/8 - 1, chunk c at position
  // r d/8 + (c ^ (r & 7)): eight consecutive rows then put a given chunk in eight different
  // 128-byte bank windows, so the transposing reads below are free of bank conflicts.  Each load
  // fills 64 consecutive positions (1 KiB) from whole rows.  Rows past n_rows read as zeros (or
  // keep stale data): their tokens are independent MFMA columns and are never stored.
  constexpr int CPR = D / 8;                       // 16-byte chunks per row
  constexpr int kXLoads = (kTokens * CPR) / 64;    // 1-KiB loads per tile
  static_assert(kWide || kXLoads == 2 * S::FUP, "a tile's rows fill ring slot 2 and xs exactly");
  auto stage_x = [&](int64_t tl) {
    if constexpr (!kWide) {
      const int64_t r0 = tl * kTokens;
      const int64_t rows = n_rows - r0 < kTokens ? n_rows - r0 : kTokens;
      const __amdgpu_buffer_rsrc_t xr = make_rsrc(X + r0 * ldx, (uint32_t)((rows - 1) * ldx * 2 + 2 * D));
#pragma unroll
      for (int j = 0; j < kXLoads / NW; ++j) {
        const int q = j * NW + wave;
        const int pos = q * 64 + lane, r = pos / CPR, c = (pos % CPR) ^ (r & 7);
        STCA_LDS void *dst = q < S::FUP ? (STCA_LDS void *)&uv2[q][0] : (STCA_LDS void *)&xs[q - S::FUP][0];
        load_lds16(xr, dst, (uint32_t)(r * ldx * 2 + c * 16), 0);
      }
    }
  };

  // The pair's 32 TB tokens of a tile as B operands: lane l holds token tok0 + 32 tb, features
  // 16 ks + 8 (l>>5) + 0..7.
  bf16x8 xb[TB][S::NKS];
  auto load_x = [&](int64_t tl) {
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const int64_t tok = tl * kTokens + (wave >> 1) * 32 * TB + 32 * tb + col;
      const bool valid = tok < n_rows;
      const bf16 *xrow = X + (valid ? tok : 0) * ldx + 8 * grp;
#pragma unroll
      for (int ks = 0; ks < S::NKS; ++ks) {
        if (valid)
          xb[tb][ks] = *reinterpret_cast<const bf16x8 *>(xrow + 16 * ks);
        else
          xb[tb][ks] = bf16x8{};
      }
    }
  };

  // d <= 256: the pair's 32 tokens from the staged rows into the B-operand registers.
  auto read_x = [&]() {
    if constexpr (!kWide) {
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        const int row = (wave >> 1) * 32 * TB + 32 * tb;  // first row of the block (uniform)
        const int r = (row & 63) + col;                    // row within its 64-row half
        const STCA_LDS char *half =
            row < 64 ? (const STCA_LDS char *)&uv2[0][0] : (const STCA_LDS char *)&xs[0][0];
#pragma unroll
        for (int ks = 0; ks < S::NKS; ++ks) {
          const int c = 2 * ks + grp;
          xb[tb][ks] = *(const STCA_LDS bf16x8 *)(half + (r * CPR + (c ^ (r & 7))) * 16);
        }
      }
    }
  };

  // d <= 256, between two layers of a tile: the pair's rows back into the row buffer (the inverse of
  // read_x; both waves of a pair hold the same rows, the first writes them).  The buffer is free:
  // the last step's barrier has passed every read of ring slot 2, and nothing is staged into it
  // before the next layer has read its rows.
  auto write_x = [&]() {
    if constexpr (!kWide) {
      if (role == 0) {
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
          const int row = (wave >> 1) * 32 * TB + 32 * tb;
          const int r = (row & 63) + col;
          STCA_LDS char *half = row < 64 ? (STCA_LDS char *)&uv2[0][0] : (STCA_LDS char *)&xs[0][0];
#pragma unroll
          for (int ks = 0; ks < S::NKS; ++ks) {
            const int c = 2 * ks + grp;
            *(STCA_LDS bf16x8 *)(half + (r * CPR + (c ^ (r & 7))) * 16) = xb[tb][ks];
          }
        }
      }
    }
  };

  // Persistent workgroups walk the token tiles tile = blockIdx.x + k gridDim.x.  A tile's rows and
  // first weight steps are loaded while the previous tile finishes (its last down product,
  // LayerNorm and stores), so only the first tile waits for them.  Every workgroup does the same
  // work per tile, so workgroups that start together would stay in lockstep and load and store
  // in bursts; the first tile therefore starts after a delay that grows with blockIdx.x
  // (stagger sleep units of 64 cycles for the last workgroup).
  if (stagger > 0) {
    const int n = (int)(((int64_t)blockIdx.x * stagger) / (int64_t)gridDim.x);
    for (int i = 0; i < n; ++i) __builtin_amdgcn_s_sleep(1);
  }
  const int64_t n_tiles = (n_rows + kTokens - 1) / kTokens;
  if ((int64_t)blockIdx.x < n_tiles) {
    if constexpr (kWide)
      load_x(blockIdx.x);
    else
      stage_x(blockIdx.x);
    stage_first();
    barrier_vm<0>();
  }
  // Work items are (tile, layer) pairs, a tile's layers one after another.
  int item = 0;
  for (int64_t tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
  for (int layer = 0; layer < NL; ++layer, ++item) {
  const int64_t tok0 = tile * kTokens + (wave >> 1) * 32 * TB + col;  // block tb: + 32 tb
  TO *__restrict__ out = (TO *)lay.out + (int64_t)layer * lay.out_stride;
  const int par = NL > 1 ? (item & 1) : 0;  // LayerNorm parameter buffer of this item
  // Issued after the last loads this item waits for: vector-memory loads complete in order.  The
  // next item is the tile's next layer (its first weight steps; at d = 512 the tile's rows again)
  // or the next tile's first layer (its rows and first weight steps).
  auto prefetch_next = [&]() {
    if (layer + 1 < NL) {
      use_layer(layer + 1);
      if constexpr (kWide) load_x(tile);
      stage_first();
      return;
    }
    const int64_t nt = tile + gridDim.x;
    if (NL > 1) use_layer(0);
    if (nt < n_tiles) {
      if constexpr (kWide)
        load_x(nt);
      else
        stage_x(nt);
      stage_first();
    }
  };
  // LayerNorm parameters of the next item, loaded at the start of this one and written to the other
  // half of gb after the first step's barrier (that half was last read by the previous item).
  constexpr int kGB = (D + 64 * NW - 1) / (64 * NW);
  float gnext[kGB], bnext[kGB];
  auto load_next_gb = [&]() {
    if constexpr (LN) {
      if (NL > 1) {
        const int64_t o = (int64_t)(layer + 1 < NL ? layer + 1 : 0) * lay.ln_stride;
#pragma unroll
        for (int j = 0; j < kGB; ++j) {
          const int i = threadIdx.x + 64 * NW * j;
          gnext[j] = i < D ? lay.gamma[o + i] : 0.f;
          bnext[j] = i < D ? lay.beta[o + i] : 0.f;
        }
      }
    }
  };
  auto store_next_gb = [&]() {
    if constexpr (LN) {
      if (NL > 1) {
#pragma unroll
        for (int j = 0; j < kGB; ++j) {
          const int i = threadIdx.x + 64 * NW * j;
          if (i < D) {
            gb[par ^ 1][0][i] = gnext[j];
            gb[par ^ 1][1][i] = bnext[j];
          }
        }
      }
    }
  };

  f32x16 yacc[S::NOBW][TB];
#pragma unroll
  for (int ob = 0; ob < S::NOBW; ++ob)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) yacc[ob][tb] = f32x16{};
  f32x16 acc[TB];        // up (registers 0-7) and gate (8-15) values of the step in flight
  bf16x8 hb_prev[TB];    // this wave's gated block of the previous step (B operands)
  bf16x8 hp[TB];         // the partner's gated block of the previous step

  // Byte offsets into the ring of this lane's fragments: up/gate of this role, down blocks of
  // this wave's outputs built from its own (kk = role) and the partner's (kk = 1 - role) features.
  const uint32_t lo = (uint32_t)lane * 16u;
  const uint32_t uv_off = (uint32_t)(role * S::NKS) * 1024u + lo;
  const uint32_t own_off = (uint32_t)(S::NOBW * role) * 1024u + lo;
  const uint32_t par_off = own_off + (uint32_t)S::NOB * 1024u;
  auto frag_at = [&](const STCA_LDS char *base, uint32_t off) -> bf16x8 {
    return *(const STCA_LDS bf16x8 *)(base + off);
  };

  auto swap_out = [&](int t, const bf16x8 (&h)[TB]) {
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) hx[t & 1][wave][tb][lane] = h[tb];
  };
  auto swap_in = [&](int t) {
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) hp[tb] = hx[t & 1][partner][tb][lane];
  };
  auto gate_all = [&](const float (&ga)[TB][16], bf16x8 (&h)[TB]) {
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int j = 0; j < 8; ++j) h[tb][j] = f32_to_bf16(swiglu_gate(ga[tb][j], ga[tb][j + 8]));
  };
  auto copy_acc = [&](float (&ga)[TB][16]) {
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int e = 0; e < 16; ++e) ga[tb][e] = acc[tb][e];
  };
  // Up/gate products of one step outside the steady loop (every step at d = 512).  The fragment
  // reads run UA ahead of their MFMAs in a pinned order, so LDS latency hides behind the MFMAs:
  // left to itself the compiler reused one register for every fragment and waited for each read
  // before its MFMA.
  auto up_all = [&](int b) {
    constexpr int UA = kWide ? STCA_ENC_UA_WIDE : STCA_ENC_UA;  // d = 512: a fragment feeds one MFMA, d = 256 two
    bf16x8 fr[UA + 1];
#pragma unroll
    for (int p = 0; p < UA && p < S::NKS; ++p) fr[p] = frag_at(uv_slot(b), uv_off + p * 1024u);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < S::NKS; ++ks) {
      if (ks + UA < S::NKS) fr[(ks + UA) % (UA + 1)] = frag_at(uv_slot(b), uv_off + (ks + UA) * 1024u);
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
        acc[tb] = mfma32x32x16(fr[ks % (UA + 1)], xb[tb][ks], ks == 0 ? f32x16{} : acc[tb]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto down_all = [&](int b) {
#pragma unroll
    for (int ob = 0; ob < S::NOBW; ++ob) {
      const bf16x8 a = frag_at(o_slot(b), own_off + ob * 1024u);
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) yacc[ob][tb] = mfma32x32x16(a, hb_prev[tb], yacc[ob][tb]);
    }
#pragma unroll
    for (int ob = 0; ob < S::NOBW; ++ob) {
      const bf16x8 a = frag_at(o_slot(b), par_off + ob * 1024u);
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) yacc[ob][tb] = mfma32x32x16(a, hp[tb], yacc[ob][tb]);
    }
  };

  if constexpr (kWide) {
    // Step t: up/gate of step t+1 from LDS slot (t+1) % 2, down of step t-1 with W_o fragments
    // loaded from L2 at the start of the step, gate of step t; up/gate of t+2 is staged into
    // the slot step t-1 finished reading and must land by the end of step t.
    auto down_regs = [&](const bf16x8 (&wo)[2][S::NOBW]) {
#pragma unroll
      for (int ob = 0; ob < S::NOBW; ++ob)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) yacc[ob][tb] = mfma32x32x16(wo[0][ob], hb_prev[tb], yacc[ob][tb]);
#pragma unroll
      for (int ob = 0; ob < S::NOBW; ++ob)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) yacc[ob][tb] = mfma32x32x16(wo[1][ob], hp[tb], yacc[ob][tb]);
    };
    auto load_wo = [&](int t, bf16x8 (&wo)[2][S::NOBW]) {
      const bf16x8 *base = packed + ((int64_t)t * S::FPS + S::FUP + S::NOBW * role) * 64 + lane;
#pragma unroll
      for (int ob = 0; ob < S::NOBW; ++ob) {
        wo[0][ob] = base[ob * 64];
        wo[1][ob] = base[(S::NOB + ob) * 64];
      }
    };
    // Step t's W_o fragments (for the down product of its gated block, run in step t + 1) are
    // loaded right after step t's own down product and stay in flight across the step's barrier,
    // so they have the next step's up/gate product to land: issued at the start of the step that
    // uses them, their L2 latency (about 1900 cycles, half of a step, in timestamp probes) was
    // exposed every step.  The first and the last two steps are peeled off the loop, so that the
    // loop body has no conditional loads: with them the compiler's count of loads in flight
    // differed between paths and it waited for the W_o loads at the swap-buffer read.
    // (S_ = r d / 32 >= 16 at d = 512.)
    // The loads are spread over the MFMAs: one wave's 16 staging loads and 16 W_o loads of a step
    // move 32 KiB through the CU's vector-memory path, and issued in bursts they stalled the wave
    // (one per SIMD) with the matrix cores idle.  The staging loads of step t + 2 go out one after
    // every second up/gate MFMA, each W_o pair right after the two down MFMAs that last read it.
    constexpr int kWoLoads = 2 * S::NOBW;  // W_o loads per wave and step
    static_assert(S::FUP % NW == 0 && 2 * LUV <= S::NKS, "one staging load per two up/gate MFMAs");
    bf16x8 wo[2][S::NOBW];
    auto up_stage = [&](int b, int t2, int sb) {
      constexpr int UA = STCA_ENC_UA_WIDE;
      bf16x8 fr[UA + 1];
#pragma unroll
      for (int p = 0; p < UA; ++p) fr[p] = frag_at(uv_slot(b), uv_off + p * 1024u);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < S::NKS; ++ks) {
        if (ks + UA < S::NKS) fr[(ks + UA) % (UA + 1)] = frag_at(uv_slot(b), uv_off + (ks + UA) * 1024u);
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
          acc[tb] = mfma32x32x16(fr[ks % (UA + 1)], xb[tb][ks], ks == 0 ? f32x16{} : acc[tb]);
        if (ks % 2 == 1 && ks / 2 < LUV) {
          const int f = wave + NW * (ks / 2);
          load_lds16(wrs, (STCA_LDS void *)(uv_slot(sb) + f * 1024), (uint32_t)(f * 64 + lane) * 16u,
                     (uint32_t)t2 * SLOT);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    auto down_load = [&](int tn) {  // the down product, each fragment pair then reloaded for step tn
      const bf16x8 *base = packed + ((int64_t)tn * S::FPS + S::FUP + S::NOBW * role) * 64 + lane;
#pragma unroll
      for (int ob = 0; ob < S::NOBW; ++ob) {
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) yacc[ob][tb] = mfma32x32x16(wo[0][ob], hb_prev[tb], yacc[ob][tb]);
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) yacc[ob][tb] = mfma32x32x16(wo[1][ob], hp[tb], yacc[ob][tb]);
        wo[0][ob] = base[ob * 64];
        wo[1][ob] = base[(S::NOB + ob) * 64];
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    auto wide_step = [&](int t, auto DOWN, auto UP, auto STAGE) {
      if constexpr (decltype(DOWN)::value) swap_in(t - 1);
      float ga[TB][16];
      copy_acc(ga);
      if constexpr (decltype(UP)::value) {
        if constexpr (decltype(STAGE)::value)
          up_stage((t + 1) % 2, t + 2, t % 2);
        else
          up_all((t + 1) % 2);
      }
      if constexpr (decltype(DOWN)::value)
        down_load(t);
      else
        load_wo(t, wo);
      bf16x8 h[TB];
      gate_all(ga, h);
      swap_out(t, h);
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) hb_prev[tb] = h[tb];
      barrier_vm<kWoLoads>();  // the W_o loads just issued may stay in flight
    };
    using Yes = std::true_type;
    using No = std::false_type;
    // The item's rows and first fragments landed before the barrier that ended the previous item.
    load_next_gb();
    up_all(0);
    barrier_vm<0>();  // slot 0 is restaged in step 0
    store_next_gb();
    wide_step(0, No{}, Yes{}, Yes{});
    for (int t = 1; t + 2 < S_; ++t) wide_step(t, Yes{}, Yes{}, Yes{});
    wide_step(S_ - 2, Yes{}, Yes{}, No{});
    wide_step(S_ - 1, Yes{}, No{}, No{});
    swap_in(S_ - 1);
    prefetch_next();
    down_regs(wo);
  } else {
    // Step t: the matrix cores run the up/gate products of step t+1 and the down product of step
    // t-1 (own block from registers, partner's block from LDS); the vector ALU gates step t.  The
    // up/gate fragments of step t live in ring slot t % 3, the down fragments of step t in slot
    // t % 3 as well; step t stages up/gate of t+3 (into the slot step t-1 finished reading) and
    // down of t+1, so every load has a full step to land before the barrier that precedes its use.
    // With kGO the down fragments come from L2 instead: fragment di of step t (di < NOBW: the
    // wave's own output blocks built from its own features; otherwise from the partner's) is
    // loaded into a register ring of FD/2 slots, FD/2 down products ahead of its use.
    constexpr int WR = S::FD / 2;
    auto wo_frag = [&](int t, int di) -> bf16x8 {
      const int f = S::FUP + (di < S::NOBW ? 0 : S::NOB) + S::NOBW * role + di % S::NOBW;
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(wrs, (int)lo, (int)((uint32_t)(t * S::FPS + f) * 1024u), 0);
      return __builtin_bit_cast(bf16x8, v);
    };
    bf16x8 wring[WR];
    // Outside the steady steps the ring holds the first WR down fragments of the previous step (the
    // step before refilled it); the other FD - WR are loaded at the start of the step, ahead of its
    // up/gate product, and the last step loads all fragments of the final down product (ring and
    // wfin) before its barrier.  Loaded right before their MFMAs, as before, their L2 latency was
    // exposed twice per item (some 2k cycles of an 89k-cycle item in timestamp probes).
    bf16x8 wfin[S::FD - WR];
    auto down_ring = [&](const bf16x8 (&rest)[S::FD - WR]) {
#pragma unroll
      for (int di = 0; di < S::FD; ++di)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
          yacc[di % S::NOBW][tb] = mfma32x32x16(di < WR ? wring[di] : rest[di - WR],
                                                di < S::NOBW ? hb_prev[tb] : hp[tb], yacc[di % S::NOBW][tb]);
    };

    // The item's rows and first fragments landed before the barrier that ended the previous item.
    read_x();
    load_next_gb();
    barrier_lds();  // every wave has read its rows out of slot 2
    if (S_ > 2) stage_uv(2, 2);
    if constexpr (!kGO) stage_o(0, 0);
    up_all(0);
    barrier_vm<0>();  // slot 0's up/gate part is restaged in step 0

    // Any step, plain order (first and last steps).
    auto general = [&](int t) {
      const bool has_up = t + 1 < S_, has_down = t >= 1, last = t + 1 == S_;
      if (t + 3 < S_) stage_uv(t + 3, t % 3);
      if constexpr (!kGO)
        if (t + 1 < S_) stage_o(t + 1, (t + 1) % 3);
      bf16x8 rest[S::FD - WR];
      if constexpr (kGO)
        if (has_down)
  #pragma unroll
          for (int j = 0; j < S::FD - WR; ++j) rest[j] = wo_frag(t - 1, WR + j);
      if (has_down) swap_in(t - 1);
      float ga[TB][16];
      copy_acc(ga);
      if (has_up) up_all((t + 1) % 3);
      if (has_down) {
        if constexpr (kGO)
          down_ring(rest);
        else
          down_all((t + 2) % 3);
      }
      if constexpr (kGO)
        if (last) {
  #pragma unroll
          for (int j = 0; j < WR; ++j) wring[j] = wo_frag(t, j);
  #pragma unroll
          for (int j = 0; j < S::FD - WR; ++j) wfin[j] = wo_frag(t, WR + j);
        }
      bf16x8 h[TB];
      gate_all(ga, h);
      swap_out(t, h);
  #pragma unroll
      for (int tb = 0; tb < TB; ++tb) hb_prev[tb] = h[tb];
      if (kGO && last)
        barrier_vm<S::FD>();  // the final down product's fragments may stay in flight
      else
        barrier_vm<0>();
      // The next step, if steady, finds its first WR down fragments in the ring.
      if constexpr (kGO)
        if (t + 1 < S_)
  #pragma unroll
          for (int j = 0; j < WR; ++j) wring[j] = wo_frag(t, j);
    };

    // Steady-state step (1 <= t, t + 1 < n_steps) with t % 3 == T3 known at compile time.  The
    // instruction order is pinned (sched_barrier): fragment reads run kAhead groups ahead through a
    // register ring, and one gate element is computed every third MFMA.
    auto steady = [&](int t, auto T3c) {
      constexpr int T3 = decltype(T3c)::value;
      constexpr int BU = (T3 + 1) % 3, BD = (T3 + 2) % 3;
      const bool stage = t + 3 < S_;  // the last steps have nothing left to stage
      // With kGO the up/gate staging loads are spread over the step's MFMAs (one per kSp MFMAs)
      // rather than issued in a burst at its start; they only have to land before step t + 2.
      // They are issued in every steady step: a step with nothing left to stage (t + 3 >= S_)
      // copies the last step's fragments into its free slot (t % 3, not read again in this item;
      // the next item's staging comes after the final step's full drain), so the compiler sees
      // the same loads on every path and its waits for the W_o ring do not cover them.
      constexpr int kMM = TB * S::NG, kSp = kMM / LUV;
      constexpr int kGP = TB == 2 ? STCA_ENC_GATE_PH : 0, kSP = TB == 2 ? STCA_ENC_STAGE_PH : kSp / 2;
      static_assert(kGP >= 0 && kGP < 3 && kSP >= 0 && kSP < kSp, "gate and staging phases within their periods");
      constexpr int kGates = (kMM - kGP + 2) / 3 < 8 * TB ? (kMM - kGP + 2) / 3 : 8 * TB;  // in the MFMA loop
      if constexpr (!kGO)
        if (stage) stage_uv(t + 3, T3);
      if constexpr (!kGO) stage_o(t + 1, BU);
      swap_in(t - 1);
      auto frag = [&](int g) -> bf16x8 {
        if (pair_is_down(g, S::FD)) {
          if constexpr (kGO) return bf16x8{};  // not used: down fragments come from wring
          const int di = g / 3;
          return frag_at(o_slot(BD), (di < S::NOBW ? own_off : par_off) + (di % S::NOBW) * 1024u);
        }
        return frag_at(uv_slot(BU), uv_off + pair_up_idx(g, S::FD) * 1024u);
      };
      float ga[TB][16];
      copy_acc(ga);
      bf16x8 ring[kRing];
  #pragma unroll
      for (int p = 0; p < kAhead; ++p)
        if (!(kGO && pair_is_down(p, S::FD))) ring[p] = frag(p);
      float hv[8 * TB];
      __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
      for (int k = 0; k < kMM; ++k) {
        if constexpr (kGO)
          if (k % kSp == kSP && k / kSp < LUV) {
            const int f = wave + NW * (k / kSp);
            if (S::FUP % NW == 0 || f < S::FUP)
              load_lds16(wrs, (STCA_LDS void *)(uv_slot(T3) + f * 1024), (uint32_t)(f * 64 + lane) * 16u,
                         (uint32_t)(stage ? t + 3 : S_ - 1) * SLOT);
          }
        const int g = k / TB, tb = k % TB;
        if (tb == 0 && g + kAhead < S::NG && !(kGO && pair_is_down(g + kAhead, S::FD)))
          ring[(g + kAhead) % kRing] = frag(g + kAhead);
        if (pair_is_down(g, S::FD)) {
          const int di = g / 3, ob = di % S::NOBW;
          if constexpr (kGO) {
            yacc[ob][tb] = mfma32x32x16(wring[di % WR], di < S::NOBW ? hb_prev[tb] : hp[tb], yacc[ob][tb]);
            // Refill the slot: the second half of this step's fragments, then the first half of
            // the next step's.
            if (tb == TB - 1) wring[di % WR] = di < WR ? wo_frag(t - 1, di + WR) : wo_frag(t, di - WR);
          } else {
            yacc[ob][tb] = mfma32x32x16(ring[g % kRing], di < S::NOBW ? hb_prev[tb] : hp[tb], yacc[ob][tb]);
          }
        } else {
          const int ui = pair_up_idx(g, S::FD);
          acc[tb] = mfma32x32x16(ring[g % kRing], xb[tb][ui], ui == 0 ? f32x16{} : acc[tb]);
        }
        if (k % 3 == kGP && k / 3 < 8 * TB) {
          const int e = k / 3;
          hv[e] = swiglu_gate(ga[e >> 3][e & 7], ga[e >> 3][(e & 7) + 8]);
          asm volatile("" : "+v"(hv[e]));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
  #pragma unroll
      for (int e = kGates; e < 8 * TB; ++e) hv[e] = swiglu_gate(ga[e >> 3][e & 7], ga[e >> 3][(e & 7) + 8]);
      bf16x8 h[TB];
  #pragma unroll
      for (int e = 0; e < 8 * TB; ++e) h[e >> 3][e & 7] = f32_to_bf16(hv[e]);
      swap_out(t, h);
  #pragma unroll
      for (int tb = 0; tb < TB; ++tb) hb_prev[tb] = h[tb];
      // Data read in step t+1 (up/gate of t+2, down of t) was staged in step t-1 or before; this
      // step's loads may stay in flight.  With kGO the loads still in flight are the four down
      // fragments of the next step, issued after everything else; otherwise a step that staged
      // nothing drains all loads.
      if (kGO || stage)
        barrier_vm<kStepLoads>();
      else
        barrier_vm<0>();
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    general(0);
    store_next_gb();
    int t = 1;
    for (; t + 3 < S_; t += 3) {
      steady(t, I1{});
      steady(t + 1, I2{});
      steady(t + 2, I0{});
    }
    for (; t < S_; ++t) general(t);
    if (layer + 1 < NL) write_x();
    // The down product of the last step remains.
    swap_in(S_ - 1);
    if constexpr (kGO) {
      prefetch_next();
      down_ring(wfin);
    } else {
      prefetch_next();
      down_all((S_ - 1) % 3);
    }
  }

  // Epilogue.  Lane l holds tokens tok0 + 32 tb; register i of block ob is output feature
  // 32 (NOBW role + ob) + 8 (i>>2) + 4 (l>>5) + (i&3).  A token's d outputs are spread over
  // lanes l, l^32 of both waves of the pair.
  float mean[TB], inv[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) mean[tb] = 0.f, inv[tb] = 1.f;
  if constexpr (LN) {
    // Swap buffer parity S_ & 1 was last read in step S_ - 1: it carries the per-wave partial
    // sums.  The ring is being restaged for the next tile, and the prefetch loads may stay in
    // flight across these barriers.
    STCA_LDS float *red = (STCA_LDS float *)&hx[S_ & 1][0][0][0];  // [stat][wave][tb][col]
    constexpr int kStat = NW * TB * 32;
    // Each wave holds half of a token's d outputs.  It computes the mean and the sum of squared
    // deviations of its half (two passes over registers), the pair exchanges them once, and the
    // halves combine exactly: mean = (m_a + m_b) / 2, M2 = M2_a + M2_b + (m_a - m_b)^2 d / 4.  Both
    // waves evaluate the same symmetric expressions, so they agree bit for bit.
    float lm[TB], lq[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      float sum = 0.f;
#pragma unroll
      for (int ob = 0; ob < S::NOBW; ++ob)
#pragma unroll
        for (int i = 0; i < 16; ++i) sum += yacc[ob][tb][i];
      lm[tb] = half_sum(sum) * (2.0f / D);
      float sq = 0.f;
#pragma unroll
      for (int ob = 0; ob < S::NOBW; ++ob)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float dv = yacc[ob][tb][i] - lm[tb];
          sq += dv * dv;
        }
      lq[tb] = half_sum(sq);
      if (grp == 0) {
        red[(wave * TB + tb) * 32 + col] = lm[tb];
        red[kStat + (wave * TB + tb) * 32 + col] = lq[tb];
      }
    }
    barrier_lds();
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const float pm = red[(partner * TB + tb) * 32 + col];
      const float pq = red[kStat + (partner * TB + tb) * 32 + col];
      mean[tb] = (lm[tb] + pm) * 0.5f;
      const float dm = lm[tb] - pm;
      const float var = (lq[tb] + pq + dm * dm * (0.25f * D)) * (1.0f / D);
      inv[tb] = 1.0f / sqrtf(var + eps);
    }
  }
  // Output: lane l holds features 32 blk + 8 q + 4 (l>>5) + 0..3 of its token (blk = NOBW role + ob).
  auto normalised = [&](int ob, int tb, int q, float (&v)[4]) {
    const int f0 = 32 * (S::NOBW * role + ob) + 8 * q + 4 * grp;
    if constexpr (LN) {
      const f32x4 gm = *reinterpret_cast<const f32x4 *>(&gb[par][0][f0]);
      const f32x4 bt = *reinterpret_cast<const f32x4 *>(&gb[par][1][f0]);
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = (yacc[ob][tb][4 * q + j] - mean[tb]) * inv[tb] * gm[j] + bt[j];
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = yacc[ob][tb][4 * q + j];
    }
  };
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    const int64_t tok = tok0 + 32 * tb;
    const bool valid = tok < n_rows;
    TO *orow = out + (valid ? tok : 0) * ldo;
#pragma unroll
    for (int ob = 0; ob < S::NOBW; ++ob) {
      if constexpr (sizeof(TO) == 2) {
        // Lanes l and l + 32 hold the same token: one lane swap per dword gives lane l features
        // 16 qp + 0..7 and lane l + 32 features 16 qp + 8..15, so each store writes 32 contiguous
        // bytes per row (16 per lane) instead of 16.
#pragma unroll
        for (int qp = 0; qp < 2; ++qp) {
          uint32_t w[2][2];
#pragma unroll
          for (int qq = 0; qq < 2; ++qq) {
            float v[4];
            normalised(ob, tb, 2 * qp + qq, v);
            w[qq][0] = __builtin_bit_cast(uint32_t, bf16x2_of(v[0], v[1]));
            w[qq][1] = __builtin_bit_cast(uint32_t, bf16x2_of(v[2], v[3]));
          }
#pragma unroll
          for (int dw = 0; dw < 2; ++dw) {
            const auto sw = __builtin_amdgcn_permlane32_swap(w[0][dw], w[1][dw], false, false);
            w[0][dw] = sw[0];
            w[1][dw] = sw[1];
          }
          const int f = 32 * (S::NOBW * role + ob) + 16 * qp + 8 * grp;
          if (valid) *reinterpret_cast<u32x4 *>(orow + f) = u32x4{w[0][0], w[0][1], w[1][0], w[1][1]};
        }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float v[4];
          normalised(ob, tb, q, v);
          const int f0 = 32 * (S::NOBW * role + ob) + 8 * q + 4 * grp;
          if (valid) *reinterpret_cast<f32x4 *>(orow + f0) = f32x4{v[0], v[1], v[2], v[3]};
        }
      }
    }
  }
  barrier_vm<0>();  // the next item restages the ring and reuses the swap and statistics buffers
  }
  }
}

template <int D, bool LN, typename TO>
static hipError_t launch_encode(hipStream_t s, int r, int64_t n_rows, const void *X, int64_t ldx,
                                const EncodeLayers &lay, int64_t ldo, float eps) {
  constexpr int TB = D > 256 ? 1 : D == 256 ? STCA_ENC_TB : STCA_ENC_TB_SMALL;
  using PL = PairLaunch<D, TB>;
  auto kern = encode_pair_kernel<D, TB, LN, TO>;
  // Persistent grid: as many workgroups as fit on the device at once, each walking tiles.  The
  // count is queried on every call (host-only, no device work), so no state is kept between calls.
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 64 * PL::NW, 0);
  if (e != hipSuccess) return e;
  const int64_t resident = std::max(1, cus * per_cu);
  const int64_t tiles = (n_rows + PL::kTokens - 1) / PL::kTokens;
  const int64_t blocks = std::min<int64_t>(tiles, resident);
  // Stagger the first tiles over about half a tile's time only when every workgroup has many
  // items to do, so that the start-up delay is amortised.
  const int stagger = tiles * lay.n >= 8 * blocks ? STCA_ENC_STAGGER * (r * D / 32) : 0;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(64 * PL::NW), 0, s, n_rows, r * D / 32, (const bf16 *)X, ldx,
                     lay, ldo, eps, stagger);
  return hipGetLastError();
}

template <int D>
static hipError_t encode_d(hipStream_t s, int r, int64_t n_rows, const void *X, int64_t ldx,
                           const EncodeLayers &lay, int64_t ldo, bool out_bf16, bool apply_ln, float eps) {
  if (apply_ln)
    return out_bf16 ? launch_encode<D, true, bf16>(s, r, n_rows, X, ldx, lay, ldo, eps)
                    : launch_encode<D, true, float>(s, r, n_rows, X, ldx, lay, ldo, eps);
  return out_bf16 ? launch_encode<D, false, bf16>(s, r, n_rows, X, ldx, lay, ldo, eps)
                  : launch_encode<D, false, float>(s, r, n_rows, X, ldx, lay, ldo, eps);
}

hipError_t encode_mfma_layers(hipStream_t s, int d, int r, int64_t n_rows, const void *X, int64_t ldx,
                              const EncodeLayers &lay, int64_t ldo, bool out_bf16, bool apply_ln, float eps) {
  if (n_rows <= 0) return hipSuccess;
  if (lay.n < 1 || lay.n > STCA_MAX_M) return hipErrorInvalidValue;
  switch (d) {
    case 64: return encode_d<64>(s, r, n_rows, X, ldx, lay, ldo, out_bf16, apply_ln, eps);
    case 128: return encode_d<128>(s, r, n_rows, X, ldx, lay, ldo, out_bf16, apply_ln, eps);
    case 256: return encode_d<256>(s, r, n_rows, X, ldx, lay, ldo, out_bf16, apply_ln, eps);
    case 512: return encode_d<512>(s, r, n_rows, X, ldx, lay, ldo, out_bf16, apply_ln, eps);
    default: return hipErrorInvalidValue;
  }
}

hipError_t encode_mfma(hipStream_t s, int d, int r, int64_t n_rows, const void *X, int64_t ldx,
                       const void *packed, void *out, int64_t ldo, bool out_bf16, bool apply_ln,
                       const float *gamma, const float *beta, float eps) {
  const EncodeLayers lay{packed, 0, out, 0, gamma, beta, 0, 1};
  return encode_mfma_layers(s, d, r, n_rows, X, ldx, lay, ldo, out_bf16, apply_ln, eps);
}

}  // namespace stca
