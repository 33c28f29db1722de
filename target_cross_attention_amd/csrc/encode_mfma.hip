// Fused history encode on bf16 MFMA: X~ = LN(((X W_u) * SiLU(X W_v)) W_o), one launch per layer.
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
//   * weights are pre-packed in fragment order (1 KiB = one wave operand), staged step by step
//     into LDS with direct global->LDS loads and shared by all waves of the workgroup;
//   * LayerNorm statistics of a token combine the two waves of its pair through LDS.
// d <= 256: a workgroup is 8 waves (TB = 1, two per SIMD) or 4 (TB = 2) over 128 tokens, and the
// whole step (up/gate and down fragments) is staged two steps ahead in a 3-slot ring.  d = 512: a
// step of weights is 96 KiB, so only the up/gate part is staged (two slots, one step ahead) and
// each wave loads its down fragments from L2 into registers; 4 waves over 64 tokens.
#include <type_traits>

#include "device_common.hpp"
#include "internal.hpp"

namespace stca {

size_t encode_packed_bytes(int d, int r) { return (size_t)(r * d / 32) * (size_t)(3 * d / 16) * 1024; }

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
__global__ __launch_bounds__(256) void encode_pack_kernel(int d, int rd, const uint16_t *__restrict__ Wu,
                                                          const uint16_t *__restrict__ Wv,
                                                          const uint16_t *__restrict__ Wo,
                                                          uint16_t *__restrict__ out) {
  const int NKS = d / 16, NOB = d / 32, FPS = 2 * NKS + 2 * NOB;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)(rd / 32) * FPS * 64;
  if (gid >= total) return;
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
                       void *packed) {
  const int rd = r * d;
  const int64_t total = (int64_t)(rd / 32) * (3 * d / 16) * 64;
  hipLaunchKernelGGL(encode_pack_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, d, rd,
                     (const uint16_t *)Wu, (const uint16_t *)Wv, (const uint16_t *)Wo, (uint16_t *)packed);
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

#ifndef STCA_ENC_RING
#define STCA_ENC_RING 4
#endif
#ifndef STCA_ENC_TB
#define STCA_ENC_TB 1
#endif

// TB = 32-token blocks per wave: TB = 2 gives 4 waves of up to 512 registers (one per SIMD), TB = 1
// gives 8 waves of up to 256 registers (two per SIMD); either way a workgroup covers 128 tokens.
// At d = 512 (wide) a step of weights is 96 KiB: only the up/gate part goes through LDS (two
// slots), each wave reads its W_o fragments from L2 into registers at the start of the step, and
// the workgroup is 4 waves of one 32-token block (64 tokens), one wave per SIMD.
template <int D, int TB> struct PairLaunch {
  static constexpr bool kWide = D > 256;
  static constexpr int NW = kWide ? 4 : 8 / TB;            // waves per workgroup
  static constexpr int kTokens = (NW / 2) * 32 * TB;       // tokens per workgroup
};

template <int D, int TB, bool LN, typename TO>
__global__ __launch_bounds__((64 * PairLaunch<D, TB>::NW), 1) void encode_pair_kernel(int64_t n_rows, int n_steps,
                                                             const bf16 *__restrict__ X, int64_t ldx,
                                                             const bf16x8 *__restrict__ packed,
                                                             TO *__restrict__ out, int64_t ldo,
                                                             const float *__restrict__ gamma,
                                                             const float *__restrict__ beta, float eps) {
  using S = PairShape<D>;
  constexpr bool kWide = PairLaunch<D, TB>::kWide;
  constexpr int NW = PairLaunch<D, TB>::NW;
  constexpr int kTokens = PairLaunch<D, TB>::kTokens;
  // Direct-to-LDS loads per wave and step: fragments go round-robin over the waves; the barrier
  // wait uses the smallest per-wave count, which waits for at least all loads of older steps.
  constexpr int LUV = (S::FUP + NW - 1) / NW, LO = (S::FDN + NW - 1) / NW;
  constexpr int kStepLoads = S::FUP / NW + S::FDN / NW;
  constexpr int kRing = STCA_ENC_RING, kAhead = STCA_ENC_RING - 1;  // fragment groups in flight
  constexpr uint32_t SLOT = S::FPS * 1024u;                          // bytes of one ring slot
  // Weight ring: slot b holds the up/gate fragments of one step (uvN) and the down fragments of
  // another (oN), see the step schedule below.  Every part is an array of its own so that the
  // compiler sees reads of one slot as independent of the loads landing in another and does not
  // wait for those loads.
  __shared__ bf16x8 uv0[S::FUP][64], uv1[S::FUP][64], uv2[kWide ? 1 : S::FUP][64];
  __shared__ bf16x8 o0[kWide ? 1 : S::FDN][64], o1[kWide ? 1 : S::FDN][64], o2[kWide ? 1 : S::FDN][64];
  auto uv_slot = [&](int b) -> const STCA_LDS char * {
    return (const STCA_LDS char *)(b == 0 ? &uv0[0][0] : b == 1 ? &uv1[0][0] : &uv2[0][0]);
  };
  auto o_slot = [&](int b) -> const STCA_LDS char * {
    return (const STCA_LDS char *)(b == 0 ? &o0[0][0] : b == 1 ? &o1[0][0] : &o2[0][0]);
  };
  // Gated activations swapped within a pair: [step parity][wave][32-token block][lane].
  __shared__ bf16x8 hx[2][NW][TB][64];

  // The wave index is uniform: keeping it in a scalar register makes the LDS destinations of the
  // staging loads (M0) scalar arithmetic.
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int role = wave & 1, partner = wave ^ 1;
  const int col = lane & 31, grp = lane >> 5;
  const int64_t tok0 = (int64_t)blockIdx.x * kTokens + (wave >> 1) * 32 * TB + col;  // block tb: + 32 tb
  const int S_ = n_steps;

  const __amdgpu_buffer_rsrc_t wrs = make_rsrc(packed, (uint32_t)n_steps * SLOT);
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

  // The pair's 32 TB tokens as B operands: lane l holds token tok0 + 32 tb, features
  // 16 ks + 8 (l>>5) + 0..7.
  bf16x8 xb[TB][S::NKS];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    const int64_t tok = tok0 + 32 * tb;
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
  auto up_all = [&](int b) {
#pragma unroll
    for (int ks = 0; ks < S::NKS; ++ks) {
      const bf16x8 a = frag_at(uv_slot(b), uv_off + ks * 1024u);
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) acc[tb] = mfma32x32x16(a, xb[tb][ks], ks == 0 ? f32x16{} : acc[tb]);
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
    stage_uv(0, 0);
    if (S_ > 1) stage_uv(1, 1);
    barrier_vm<0>();
    up_all(0);
    barrier_vm<0>();  // slot 0 is restaged in step 0
    for (int t = 0; t < S_; ++t) {
      const bool has_up = t + 1 < S_, has_down = t >= 1;
      bf16x8 wo[2][S::NOBW];
      if (has_down) load_wo(t - 1, wo);
      if (t + 2 < S_) stage_uv(t + 2, t % 2);
      if (has_down) swap_in(t - 1);
      float ga[TB][16];
      copy_acc(ga);
      if (has_up) up_all((t + 1) % 2);
      if (has_down) down_regs(wo);
      bf16x8 h[TB];
      gate_all(ga, h);
      swap_out(t, h);
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) hb_prev[tb] = h[tb];
      barrier_vm<0>();
    }
    swap_in(S_ - 1);
    bf16x8 wo[2][S::NOBW];
    load_wo(S_ - 1, wo);
    down_regs(wo);
  } else {
    // Step t: the matrix cores run the up/gate products of step t+1 and the down product of step
    // t-1 (own block from registers, partner's block from LDS); the vector ALU gates step t.  The
    // up/gate fragments of step t live in ring slot t % 3, the down fragments of step t in slot
    // t % 3 as well; step t stages up/gate of t+3 (into the slot step t-1 finished reading) and
    // down of t+1, so every load has a full step to land before the barrier that precedes its use.
    stage_uv(0, 0);
    if (S_ > 1) stage_uv(1, 1);
    if (S_ > 2) stage_uv(2, 2);
    stage_o(0, 0);
    barrier_vm<0>();
    up_all(0);
    barrier_vm<0>();  // slot 0's up/gate part is restaged in step 0

    // Any step, plain order (first and last steps).
    auto general = [&](int t) {
      const bool has_up = t + 1 < S_, has_down = t >= 1;
      if (t + 3 < S_) stage_uv(t + 3, t % 3);
      if (t + 1 < S_) stage_o(t + 1, (t + 1) % 3);
      if (has_down) swap_in(t - 1);
      float ga[TB][16];
      copy_acc(ga);
      if (has_up) up_all((t + 1) % 3);
      if (has_down) down_all((t + 2) % 3);
      bf16x8 h[TB];
      gate_all(ga, h);
      swap_out(t, h);
  #pragma unroll
      for (int tb = 0; tb < TB; ++tb) hb_prev[tb] = h[tb];
      barrier_vm<0>();
    };

    // Steady-state step (1 <= t, t + 3 < n_steps) with t % 3 == T3 known at compile time.  The
    // instruction order is pinned (sched_barrier): fragment reads run kAhead groups ahead through a
    // register ring, and one gate element is computed every third MFMA.
    auto steady = [&](int t, auto T3c) {
      constexpr int T3 = decltype(T3c)::value;
      constexpr int BU = (T3 + 1) % 3, BD = (T3 + 2) % 3;
      stage_uv(t + 3, T3);
      stage_o(t + 1, BU);
      swap_in(t - 1);
      auto frag = [&](int g) -> bf16x8 {
        if (pair_is_down(g, S::FD)) {
          const int di = g / 3;
          return frag_at(o_slot(BD), (di < S::NOBW ? own_off : par_off) + (di % S::NOBW) * 1024u);
        }
        return frag_at(uv_slot(BU), uv_off + pair_up_idx(g, S::FD) * 1024u);
      };
      float ga[TB][16];
      copy_acc(ga);
      bf16x8 ring[kRing];
  #pragma unroll
      for (int p = 0; p < kAhead; ++p) ring[p] = frag(p);
      float hv[8 * TB];
      __builtin_amdgcn_sched_barrier(0);
      constexpr int kMM = TB * S::NG;
  #pragma unroll
      for (int k = 0; k < kMM; ++k) {
        const int g = k / TB, tb = k % TB;
        if (tb == 0 && g + kAhead < S::NG) ring[(g + kAhead) % kRing] = frag(g + kAhead);
        if (pair_is_down(g, S::FD)) {
          const int di = g / 3, ob = di % S::NOBW;
          yacc[ob][tb] = mfma32x32x16(ring[g % kRing], di < S::NOBW ? hb_prev[tb] : hp[tb], yacc[ob][tb]);
        } else {
          const int ui = pair_up_idx(g, S::FD);
          acc[tb] = mfma32x32x16(ring[g % kRing], xb[tb][ui], ui == 0 ? f32x16{} : acc[tb]);
        }
        if (k % 3 == 0 && k / 3 < 8 * TB) {
          const int e = k / 3;
          hv[e] = swiglu_gate(ga[e >> 3][e & 7], ga[e >> 3][(e & 7) + 8]);
          asm volatile("" : "+v"(hv[e]));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
  #pragma unroll
      for (int e = (kMM + 2) / 3; e < 8 * TB; ++e) hv[e] = swiglu_gate(ga[e >> 3][e & 7], ga[e >> 3][(e & 7) + 8]);
      bf16x8 h[TB];
  #pragma unroll
      for (int e = 0; e < 8 * TB; ++e) h[e >> 3][e & 7] = f32_to_bf16(hv[e]);
      swap_out(t, h);
  #pragma unroll
      for (int tb = 0; tb < TB; ++tb) hb_prev[tb] = h[tb];
      // Data read in step t+1 (up/gate of t+2, down of t) was staged in step t-1 or before; this
      // step's loads may stay in flight.
      barrier_vm<kStepLoads>();
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    general(0);
    int t = 1;
    for (; t + 5 < S_; t += 3) {
      steady(t, I1{});
      steady(t + 1, I2{});
      steady(t + 2, I0{});
    }
    for (; t < S_; ++t) general(t);
    // The down product of the last step remains.
    swap_in(S_ - 1);
    down_all((S_ - 1) % 3);
  }

  // Epilogue.  Lane l holds tokens tok0 + 32 tb; register i of block ob is output feature
  // 32 (NOBW role + ob) + 8 (i>>2) + 4 (l>>5) + (i&3).  A token's d outputs are spread over
  // lanes l, l^32 of both waves of the pair.
  float mean[TB], inv[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) mean[tb] = 0.f, inv[tb] = 1.f;
  if constexpr (LN) {
    // Ring slot S_ % 3 is no longer read: it carries the per-wave partial sums.
    STCA_LDS float *red = (STCA_LDS float *)uv_slot(kWide ? 0 : S_ % 3);  // [stat][wave][tb][col]
    constexpr int kStat = NW * TB * 32;
    float part[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      float sum = 0.f;
#pragma unroll
      for (int ob = 0; ob < S::NOBW; ++ob)
#pragma unroll
        for (int i = 0; i < 16; ++i) sum += yacc[ob][tb][i];
      part[tb] = half_sum(sum);
      if (grp == 0) red[(wave * TB + tb) * 32 + col] = part[tb];
    }
    barrier_vm<0>();
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      mean[tb] = (part[tb] + red[(partner * TB + tb) * 32 + col]) * (1.0f / D);
      float sq = 0.f;
#pragma unroll
      for (int ob = 0; ob < S::NOBW; ++ob)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float dv = yacc[ob][tb][i] - mean[tb];
          sq += dv * dv;
        }
      part[tb] = half_sum(sq);
      if (grp == 0) red[kStat + (wave * TB + tb) * 32 + col] = part[tb];
    }
    barrier_vm<0>();
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const float var = (part[tb] + red[kStat + (partner * TB + tb) * 32 + col]) * (1.0f / D);
      inv[tb] = 1.0f / sqrtf(var + eps);
    }
  }
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    const int64_t tok = tok0 + 32 * tb;
    if (tok >= n_rows) continue;
    TO *orow = out + tok * ldo;
#pragma unroll
    for (int ob = 0; ob < S::NOBW; ++ob) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int f0 = 32 * (S::NOBW * role + ob) + 8 * q + 4 * grp;
        float v[4];
        if constexpr (LN) {
          const f32x4 gm = *reinterpret_cast<const f32x4 *>(gamma + f0);
          const f32x4 bt = *reinterpret_cast<const f32x4 *>(beta + f0);
#pragma unroll
          for (int j = 0; j < 4; ++j) v[j] = (yacc[ob][tb][4 * q + j] - mean[tb]) * inv[tb] * gm[j] + bt[j];
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) v[j] = yacc[ob][tb][4 * q + j];
        }
        if constexpr (sizeof(TO) == 2) {
          bf16x4 pk;
#pragma unroll
          for (int j = 0; j < 4; ++j) pk[j] = f32_to_bf16(v[j]);
          *reinterpret_cast<bf16x4 *>(orow + f0) = pk;
        } else {
          *reinterpret_cast<f32x4 *>(orow + f0) = f32x4{v[0], v[1], v[2], v[3]};
        }
      }
    }
  }
}

template <int D, bool LN, typename TO>
static hipError_t launch_encode(hipStream_t s, int r, int64_t n_rows, const void *X, int64_t ldx,
                                const void *packed, void *out, int64_t ldo, const float *gamma,
                                const float *beta, float eps) {
  constexpr int TB = D > 256 ? 1 : STCA_ENC_TB;
  using PL = PairLaunch<D, TB>;
  const int64_t blocks = (n_rows + PL::kTokens - 1) / PL::kTokens;
  hipLaunchKernelGGL((encode_pair_kernel<D, TB, LN, TO>), dim3((unsigned)blocks), dim3(64 * PL::NW), 0, s,
                     n_rows, r * D / 32, (const bf16 *)X, ldx, (const bf16x8 *)packed, (TO *)out, ldo, gamma,
                     beta, eps);
  return hipGetLastError();
}

template <int D>
static hipError_t encode_d(hipStream_t s, int r, int64_t n_rows, const void *X, int64_t ldx,
                           const void *packed, void *out, int64_t ldo, bool out_bf16, bool apply_ln,
                           const float *gamma, const float *beta, float eps) {
  if (apply_ln) {
    return out_bf16 ? launch_encode<D, true, bf16>(s, r, n_rows, X, ldx, packed, out, ldo, gamma, beta, eps)
                    : launch_encode<D, true, float>(s, r, n_rows, X, ldx, packed, out, ldo, gamma, beta, eps);
  }
  return out_bf16 ? launch_encode<D, false, bf16>(s, r, n_rows, X, ldx, packed, out, ldo, gamma, beta, eps)
                  : launch_encode<D, false, float>(s, r, n_rows, X, ldx, packed, out, ldo, gamma, beta, eps);
}

hipError_t encode_mfma(hipStream_t s, int d, int r, int64_t n_rows, const void *X, int64_t ldx,
                       const void *packed, void *out, int64_t ldo, bool out_bf16, bool apply_ln,
                       const float *gamma, const float *beta, float eps) {
  if (n_rows <= 0) return hipSuccess;
  switch (d) {
    case 64: return encode_d<64>(s, r, n_rows, X, ldx, packed, out, ldo, out_bf16, apply_ln, gamma, beta, eps);
    case 128: return encode_d<128>(s, r, n_rows, X, ldx, packed, out, ldo, out_bf16, apply_ln, gamma, beta, eps);
    case 256: return encode_d<256>(s, r, n_rows, X, ldx, packed, out, ldo, out_bf16, apply_ln, gamma, beta, eps);
    case 512: return encode_d<512>(s, r, n_rows, X, ldx, packed, out, ldo, out_bf16, apply_ln, gamma, beta, eps);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace stca
