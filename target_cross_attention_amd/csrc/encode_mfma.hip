// Fused history encode on bf16 MFMA: X~ = LN(((X W_u) * SiLU(X W_v)) W_o), one launch per layer.
//
// Equations: SwiGLU FFN of eq. (1) with the three-matrix shapes of the STCA review page
// (section 2.2), followed by the LayerNorm of eq. (2) ("Make It Long, Keep It Fast", section 2.1).
//
// Work decomposition (gfx950, 64-wide waves, v_mfma_f32_32x32x16_bf16):
//   * a workgroup is 4 waves; each wave owns 32 history tokens for the whole FFN;
//   * the wave's 32 input rows stay in registers as MFMA B operands for the whole kernel;
//   * rd is walked in slices of 32 hidden features.  Per slice the wave computes the transposed
//     products A^T = W_u^T X^T and G^T = W_v^T X^T (32 hidden x 32 tokens), applies the gate in
//     registers, and feeds the gated block straight back as the B operand of the down product
//     Y^T += W_o^T H^T.  The accumulator layout of the first product is the operand layout of
//     the second once W_o's rows are pre-permuted (see encode_pack), so the rd-wide hidden
//     activation never leaves the registers: no LDS round trip, no HBM traffic;
//   * weights are pre-packed in fragment order (1 KiB = one wave operand), staged slice by slice
//     into LDS with direct global->LDS loads, double-buffered, and shared by the 4 waves;
//   * the full d-wide output row of each token ends up in two lanes (l, l^32), so the LayerNorm
//     epilogue is an in-register reduction plus one cross-half exchange.
#include <type_traits>

#include "device_common.hpp"
#include "internal.hpp"

namespace stca {

template <int D> struct EncShape {
  static constexpr int NKS = D / 16;             // 16-deep k-steps over d (up/gate products)
  static constexpr int NOB = D / 32;             // 32-wide output blocks (down product)
  static constexpr int FPS = 2 * NKS + 2 * NOB;  // fragments per 32-feature slice of rd
  // At d = 512 a whole slice (96 KiB) cannot be double-buffered in 160 KiB of LDS; the W_o part
  // is then read by each wave from global memory (L2-resident) instead.
  static constexpr bool WO_GLOBAL = (D > 256);
  static constexpr int FPS_LDS = WO_GLOBAL ? 2 * NKS : FPS;
  // Three slice buffers fit in LDS up to d = 256 (3 x 48 KiB).
  static constexpr bool PIPELINED = 3 * FPS_LDS * 1024 <= 160 * 1024;
};

size_t encode_packed_bytes(int d, int r) { return (size_t)(r * d / 32) * (size_t)(3 * d / 16) * 1024; }

// ------------------------------------------------------------------------------------------
// Fragment re-layout.  Slice s (hidden features 32s .. 32s+31) holds, in order:
//   NKS fragments of W_u, NKS of W_v: lane l, slot e = W[16 ks + 8 (l>>5) + e][32 s + (l&31)];
//   2 NOB fragments of W_o, (ob, kk):  lane l, slot e = W_o[32 s + phi(kk, l>>5, e)][32 ob + (l&31)]
//   with phi(kk, g, e) = 16 kk + 8 (e>>2) + 4 g + (e&3), the hidden feature that the up/gate
//   accumulator register 8 kk + e of lane group g holds.
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
    const uint16_t *W = (f < NKS) ? Wu : Wv;
    const int ks = (f < NKS) ? f : f - NKS;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = W[(int64_t)(16 * ks + 8 * g + e) * rd + 32 * s + col];
  } else {
    const int idx = f - 2 * NKS;
    const int ob = idx >> 1, kk = idx & 1;
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
// The fused kernel.
// ------------------------------------------------------------------------------------------
// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedVALU = 0x002, kSchedMFMA = 0x008, kSchedVMEMRead = 0x020, kSchedDSRead = 0x100;

template <int D, bool LN, typename TO>
__global__ __launch_bounds__(256, 1) void encode_mfma_kernel(int64_t n_rows, int n_slices,
                                                             const bf16 *__restrict__ X, int64_t ldx,
                                                             const bf16x8 *__restrict__ packed,
                                                             TO *__restrict__ out, int64_t ldo,
                                                             const float *__restrict__ gamma,
                                                             const float *__restrict__ beta, float eps) {
  using S = EncShape<D>;
  // Three slice buffers when they fit: slices s and s+1 are read while s+2 streams in.
  constexpr int NBUF = S::PIPELINED ? 3 : 2;
  __shared__ bf16x8 wbuf[NBUF][S::FPS_LDS][64];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, grp = lane >> 5;
  const int64_t tok = (int64_t)blockIdx.x * 128 + wave * 32 + col;
  const bool valid = tok < n_rows;

  // Stage slice `s` of the packed weights into LDS buffer `b`: fragment f goes to wbuf[b][f];
  // waves take fragments round-robin.  Each lane moves 16 bytes; the destination of lane i is
  // the fragment base + 16 i.
  auto stage = [&](int s, int b) {
    static_assert(S::FPS_LDS % 4 == 0, "fragments split evenly over 4 waves");
    const bf16x8 *src = packed + (int64_t)s * S::FPS * 64 + lane;
#pragma unroll
    for (int j = 0; j < S::FPS_LDS / 4; ++j) {
      const int f = wave + 4 * j;
      __builtin_amdgcn_global_load_lds(src + f * 64, (STCA_LDS void *)&wbuf[b][f][0], 16, 0, 0);
    }
  };

  stage(0, 0);
  if constexpr (S::PIPELINED) stage(n_slices > 1 ? 1 : 0, 1);

  // The wave's 32 tokens as B operands: lane l holds token (l&31), features 16 ks + 8 (l>>5) + 0..7.
  bf16x8 xb[S::NKS];
  {
    const bf16 *xrow = X + (valid ? tok : 0) * ldx + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < S::NKS; ++ks) {
      if (valid)
        xb[ks] = *reinterpret_cast<const bf16x8 *>(xrow + 16 * ks);
      else
        xb[ks] = bf16x8{};
    }
  }

  f32x16 yacc[S::NOB];
#pragma unroll
  for (int ob = 0; ob < S::NOB; ++ob) yacc[ob] = f32x16{};

  // Up and gate products of one slice (transposed: rows = hidden features, columns = tokens).
  auto up_gate = [&](int b, f32x16 &accA, f32x16 &accG) {
    accA = f32x16{};
    accG = f32x16{};
#pragma unroll
    for (int ks = 0; ks < S::NKS; ++ks) {
      accA = mfma32x32x16(wbuf[b][ks][lane], xb[ks], accA);
      accG = mfma32x32x16(wbuf[b][S::NKS + ks][lane], xb[ks], accG);
    }
  };
  // SwiGLU gate in registers -> bf16 B operands of the down product.
  auto gate = [&](const f32x16 &accA, const f32x16 &accG, bf16x8 (&hb)[2]) {
#pragma unroll
    for (int i = 0; i < 16; ++i) hb[i >> 3][i & 7] = f32_to_bf16(swiglu_gate(accA[i], accG[i]));
  };
  // Down product: Y^T[out x tok] += W_o^T[out x 32] H^T[32 x tok].
  auto down = [&](int s, int b, const bf16x8 (&hb)[2]) {
#pragma unroll
    for (int ob = 0; ob < S::NOB; ++ob) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8 wo;
        if constexpr (S::WO_GLOBAL)
          wo = packed[((int64_t)s * S::FPS + 2 * S::NKS + 2 * ob + kk) * 64 + lane];
        else
          wo = wbuf[b][2 * S::NKS + 2 * ob + kk][lane];
        yacc[ob] = mfma32x32x16(wo, hb[kk], yacc[ob]);
      }
    }
  };

  if constexpr (S::PIPELINED) {
    // Software pipeline over slices with no dependency inside a step.  Step t runs, on the matrix
    // cores, the up/gate products of slice t+1 and the down product of slice t-1 (whose gate was
    // computed in step t-1), and on the vector ALU the gate of slice t.  W_u/W_v and W_o slices
    // live in separate 3-deep LDS rings; a slice is staged two steps before it is read, so each
    // step waits only for loads issued one step earlier.  The instruction order is pinned
    // (sched_barrier): fragment reads run kAhead MFMAs ahead through a register ring.
    constexpr int FUP = 2 * S::NKS, FDN = 2 * S::NOB;
#ifndef STCA_ENC_RING
#define STCA_ENC_RING 8
#endif
    constexpr int kRing = STCA_ENC_RING, kAhead = STCA_ENC_RING - 2;
    constexpr int kLoadsUV = FUP / 4, kLoadsO = FDN / 4;  // direct-to-LDS loads per wave
    static_assert(FUP % 4 == 0 && FDN % 4 == 0, "fragments split evenly over 4 waves");
    bf16x8 (*wuv)[S::FPS_LDS][64] = wbuf;  // wbuf[b][0 .. FUP)       : W_u/W_v ring (3 slots)
    // W_o ring lives in wbuf[b][FUP .. FUP + FDN) of the same three slots.
    auto stage_uv = [&](int t, int b) {
      const bf16x8 *src = packed + (int64_t)t * S::FPS * 64 + lane;
#pragma unroll
      for (int j = 0; j < kLoadsUV; ++j) {
        const int f = wave + 4 * j;
        __builtin_amdgcn_global_load_lds(src + f * 64, (STCA_LDS void *)&wuv[b][f][0], 16, 0, 0);
      }
    };
    auto stage_o = [&](int t, int b) {
      const bf16x8 *src = packed + ((int64_t)t * S::FPS + FUP) * 64 + lane;
#pragma unroll
      for (int j = 0; j < kLoadsO; ++j) {
        const int f = wave + 4 * j;
        __builtin_amdgcn_global_load_lds(src + f * 64, (STCA_LDS void *)&wuv[b][FUP + f][0], 16, 0, 0);
      }
    };
    // MFMA k of a full step: every third one is a down product (16 of 48 at d = 256).
    // Fragment source of MFMA k: up k-th (u/v alternating per k-step) or down (ob, kk) ordered
    // so that MFMAs into the same output block are NOB apart.
    constexpr int kMM = FUP + FDN;
    auto is_down = [](int k) { return (k % 3) == 2 && (k / 3) < FDN; };
    auto up_idx = [](int k) { return k - (k / 3 < FDN ? (k + 1) / 3 : FDN); };
    auto dn_idx = [](int k) { return k / 3; };

    f32x16 accA, accG;   // up/gate accumulators of the slice in flight
    bf16x8 hb_prev[2];   // gated slice t-1: B operands of the down product in step t
    const int S_ = n_slices;

    stage_uv(0, 0);
    if (S_ > 1) stage_uv(1, 1);
    if (S_ > 2) stage_uv(2, 2);
    stage_o(0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    up_gate(0, accA, accG);
    __syncthreads();  // slot 0 of the W_u/W_v ring is restaged in step 0

    // Steady-state step (1 <= t, t + 3 < n_slices) with t % 3 == T3 known at compile time, so
    // every LDS fragment address is a constant offset from one per-lane base.
    auto steady = [&](int t, auto T3c) {
      constexpr int T3 = decltype(T3c)::value;
      constexpr int BU = (T3 + 1) % 3, BD = (T3 + 2) % 3;
      stage_uv(t + 3, T3);
      stage_o(t + 1, (T3 + 1) % 3);
      auto frag = [&](int k) -> bf16x8 {
        if (is_down(k)) {
          const int j = dn_idx(k);
          return wuv[BD][FUP + 2 * (j % S::NOB) + (j / S::NOB)][lane];
        }
        const int i = up_idx(k);
        return wuv[BU][(i & 1) ? S::NKS + (i >> 1) : (i >> 1)][lane];
      };
      float ga[16], gg[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        ga[e] = accA[e];
        gg[e] = accG[e];
      }
      bf16x8 ring[kRing];
#pragma unroll
      for (int p = 0; p < kAhead; ++p) ring[p] = frag(p);
      float hv[16];
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < kMM; ++k) {
        if (k + kAhead < kMM) ring[(k + kAhead) % kRing] = frag(k + kAhead);
        if (is_down(k)) {
          const int j = dn_idx(k);
          yacc[j % S::NOB] = mfma32x32x16(ring[k % kRing], hb_prev[j / S::NOB], yacc[j % S::NOB]);
        } else {
          const int i = up_idx(k);
          if (i & 1)
            accG = mfma32x32x16(ring[k % kRing], xb[i >> 1], i == 1 ? f32x16{} : accG);
          else
            accA = mfma32x32x16(ring[k % kRing], xb[i >> 1], i == 0 ? f32x16{} : accA);
        }
        // gate element e at MFMA 3e (16 elements over the first 48 MFMAs); the empty asm keeps
        // the optimiser from sinking the arithmetic to its use after the MFMA stream.
        if (k % 3 == 0 && k / 3 < 16) {
          hv[k / 3] = swiglu_gate(ga[k / 3], gg[k / 3]);
          asm volatile("" : "+v"(hv[k / 3]));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int e = kMM / 3; e < 16; ++e) hv[e] = swiglu_gate(ga[e], gg[e]);
#pragma unroll
      for (int e = 0; e < 16; ++e) hb_prev[e >> 3][e & 7] = f32_to_bf16(hv[e]);
      // Data read in step t+1 (W_u/W_v slice t+2, W_o slice t) was staged in step t-1 or before;
      // this step's loads may stay in flight.
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kLoadsUV + kLoadsO) : "memory");
      __syncthreads();
    };
    // Any step, plain order (first and last steps).
    auto general = [&](int t) {
      const bool has_up = t + 1 < S_, has_down = t >= 1;
      const bf16x8 *ub = &wuv[(t + 1) % 3][0][lane];
      const bf16x8 *db = &wuv[(t + 2) % 3][FUP][lane];  // slot of slice t-1
      if (t + 3 < S_) stage_uv(t + 3, t % 3);
      if (t + 1 < S_) stage_o(t + 1, (t + 1) % 3);
      float ga[16], gg[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        ga[e] = accA[e];
        gg[e] = accG[e];
      }
      if (has_up) {
#pragma unroll
        for (int ks = 0; ks < S::NKS; ++ks) {
          accA = mfma32x32x16(ub[ks * 64], xb[ks], ks == 0 ? f32x16{} : accA);
          accG = mfma32x32x16(ub[(S::NKS + ks) * 64], xb[ks], ks == 0 ? f32x16{} : accG);
        }
      }
      if (has_down) {
#pragma unroll
        for (int j = 0; j < FDN; ++j)
          yacc[j % S::NOB] = mfma32x32x16(db[(2 * (j % S::NOB) + (j / S::NOB)) * 64], hb_prev[j / S::NOB],
                                          yacc[j % S::NOB]);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) hb_prev[e >> 3][e & 7] = f32_to_bf16(swiglu_gate(ga[e], gg[e]));
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    general(0);
    int t = 1;
    // steady steps t = 1 .. S-4, three at a time starting at t % 3 == 1
    for (; t + 5 < S_; t += 3) {
      steady(t, I1{});
      steady(t + 1, I2{});
      steady(t + 2, I0{});
    }
    for (; t < S_; ++t) general(t);
    // The down product of the last slice remains.
    {
      const bf16x8 *db = &wuv[(S_ - 1) % 3][FUP][lane];
#pragma unroll
      for (int j = 0; j < FDN; ++j)
        yacc[j % S::NOB] = mfma32x32x16(db[(2 * (j % S::NOB) + (j / S::NOB)) * 64], hb_prev[j / S::NOB],
                                        yacc[j % S::NOB]);
    }
  } else {
    for (int s = 0; s < n_slices; ++s) {
      const int b = s & 1;
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();  // slice s is in LDS for every wave; buffer b^1 is no longer read
      if (s + 1 < n_slices) stage(s + 1, b ^ 1);
      f32x16 accA, accG;
      up_gate(b, accA, accG);
      bf16x8 hb[2];
      gate(accA, accG, hb);
      down(s, b, hb);
    }
  }

  // Epilogue.  Lane l holds token (l&31); register i of block ob is output feature
  // 32 ob + 8 (i>>2) + 4 (l>>5) + (i&3); lane l^32 holds the other half of the row.
  float mean = 0.f, inv = 1.f;
  if constexpr (LN) {
    float sum = 0.f;
#pragma unroll
    for (int ob = 0; ob < S::NOB; ++ob)
#pragma unroll
      for (int i = 0; i < 16; ++i) sum += yacc[ob][i];
    sum = half_sum(sum);
    mean = sum * (1.0f / D);
    float sq = 0.f;
#pragma unroll
    for (int ob = 0; ob < S::NOB; ++ob)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float t = yacc[ob][i] - mean;
        sq += t * t;
      }
    sq = half_sum(sq);
    inv = 1.0f / sqrtf(sq * (1.0f / D) + eps);
  }
  if (!valid) return;
  TO *orow = out + tok * ldo;
#pragma unroll
  for (int ob = 0; ob < S::NOB; ++ob) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int f0 = 32 * ob + 8 * q + 4 * grp;
      float v[4];
      if constexpr (LN) {
        const f32x4 gm = *reinterpret_cast<const f32x4 *>(gamma + f0);
        const f32x4 bt = *reinterpret_cast<const f32x4 *>(beta + f0);
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = (yacc[ob][4 * q + j] - mean) * inv * gm[j] + bt[j];
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = yacc[ob][4 * q + j];
      }
      if constexpr (sizeof(TO) == 2) {
        bf16x4 p;
#pragma unroll
        for (int j = 0; j < 4; ++j) p[j] = f32_to_bf16(v[j]);
        *reinterpret_cast<bf16x4 *>(orow + f0) = p;
      } else {
        *reinterpret_cast<f32x4 *>(orow + f0) = f32x4{v[0], v[1], v[2], v[3]};
      }
    }
  }
}

template <int D, bool LN, typename TO>
static hipError_t launch_encode(hipStream_t s, int r, int64_t n_rows, const void *X, int64_t ldx,
                                const void *packed, void *out, int64_t ldo, const float *gamma,
                                const float *beta, float eps) {
  const int64_t blocks = (n_rows + 127) / 128;
  hipLaunchKernelGGL((encode_mfma_kernel<D, LN, TO>), dim3((unsigned)blocks), dim3(256), 0, s, n_rows,
                     r * D / 32, (const bf16 *)X, ldx, (const bf16x8 *)packed, (TO *)out, ldo, gamma, beta,
                     eps);
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
