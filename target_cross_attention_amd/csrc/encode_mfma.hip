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
template <int D, bool LN, typename TO>
__global__ __launch_bounds__(256, 1) void encode_mfma_kernel(int64_t n_rows, int n_slices,
                                                             const bf16 *__restrict__ X, int64_t ldx,
                                                             const bf16x8 *__restrict__ packed,
                                                             TO *__restrict__ out, int64_t ldo,
                                                             const float *__restrict__ gamma,
                                                             const float *__restrict__ beta, float eps) {
  using S = EncShape<D>;
  __shared__ bf16x8 wbuf[2][S::FPS_LDS][64];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, grp = lane >> 5;
  const int64_t tok = (int64_t)blockIdx.x * 128 + wave * 32 + col;
  const bool valid = tok < n_rows;

  // Stage slice `s` of the packed weights into LDS buffer `b`: fragment f goes to wbuf[b][f];
  // waves take fragments round-robin.  Each lane moves 16 bytes; the destination of lane i is
  // the fragment base + 16 i.
  auto stage = [&](int s, int b) {
    const bf16x8 *src = packed + (int64_t)s * S::FPS * 64 + lane;
#pragma unroll
    for (int f = wave; f < S::FPS_LDS; f += 4)
      __builtin_amdgcn_global_load_lds(src + f * 64, (STCA_LDS void *)&wbuf[b][f][0], 16, 0, 0);
  };

  stage(0, 0);

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

  for (int s = 0; s < n_slices; ++s) {
    const int b = s & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // slice s is in LDS for every wave; buffer b^1 is no longer read
    if (s + 1 < n_slices) stage(s + 1, b ^ 1);

    // Up and gate products for hidden features 32 s .. 32 s + 31 (transposed: rows = features).
    f32x16 accA = f32x16{}, accG = f32x16{};
#pragma unroll
    for (int ks = 0; ks < S::NKS; ++ks) {
      const bf16x8 wu = wbuf[b][ks][lane];
      const bf16x8 wv = wbuf[b][S::NKS + ks][lane];
      accA = mfma32x32x16(wu, xb[ks], accA);
      accG = mfma32x32x16(wv, xb[ks], accG);
    }
    // SwiGLU gate in registers -> bf16 B operands of the down product.
    bf16x8 hb[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) hb[i >> 3][i & 7] = f32_to_bf16(swiglu_gate(accA[i], accG[i]));
    // Down product: Y^T[out x tok] += W_o^T[out x 32] H^T[32 x tok].
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
    sum += swap_halves(sum);
    mean = sum * (1.0f / D);
    float sq = 0.f;
#pragma unroll
    for (int ob = 0; ob < S::NOB; ++ob)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float t = yacc[ob][i] - mean;
        sq += t * t;
      }
    sq += swap_halves(sq);
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
