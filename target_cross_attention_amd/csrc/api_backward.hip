// libstca C ABI, backward pass (gradients of eqs. (2)-(8), stca_backward): workspace layout and
// launch sequence.  See include/stca.h.
#include <math.h>

#include <algorithm>

#include "abi_common.hpp"

using namespace stca;

namespace stca_abi {
namespace {

// ---- backward (gradients of eqs. (2)-(8)) ------------------------------------------------------
constexpr int kWgradParts = 32;    // split-K blocks of one weight gradient
constexpr int kLnBlocks = 256;     // row blocks of the LayerNorm derivative (partial column sums)
constexpr int64_t kMixedRows = 65536;  // row chunk of the mixed-precision encode backward

struct BackwardWs {
  float *Xt = nullptr;      // M x total_L x d: encoded history of every layer (fp32)
  float *dXt = nullptr;     // total_L x d
  float *Z = nullptr;       // T x M x d: recomputed forward output
  float *dO = nullptr;      // T x M x d: gradient of every o(i)
  float *qin[STCA_MAX_M] = {}, *qA[STCA_MAX_M] = {}, *qG[STCA_MAX_M] = {}, *qY[STCA_MAX_M] = {};
  float *q[STCA_MAX_M] = {}, *P[STCA_MAX_M] = {}, *U[STCA_MAX_M] = {}, *lse[STCA_MAX_M] = {};
  float *abar[STCA_MAX_M] = {}, *heads[STCA_MAX_M] = {};
  float *dq = nullptr, *qH = nullptr, *qdA = nullptr, *qdG = nullptr, *qdY = nullptr, *dc = nullptr;
  float *dheads = nullptr, *dabar = nullptr, *Dv = nullptr, *du = nullptr, *dP = nullptr;
  float *eA = nullptr, *eG = nullptr, *eH = nullptr, *eY = nullptr, *edY = nullptr;
  float *parts = nullptr;
  int64_t parts_cap = 0;  // floats in parts
  float *S = nullptr, *S2 = nullptr;  // every user's score matrix (R_u x Lp_u), twice
  RaggedDesc *desc = nullptr;         // 3 n_users product descriptors
  int64_t rows = 0;         // history rows per encode-backward chunk
  // fp32 path, with a workspace of the "keep" size: A = X W_u, G = X W_v (M x total_L x rd) and the
  // pre-LN rows Y (M x total_L x d) of every layer, kept from the forward recompute.
  float *kA = nullptr, *kG = nullptr, *kY = nullptr;
  // Mixed-precision path (bf16 storage): bf16 operands for the matrix cores, per row chunk, all
  // row-major: H, u, g (rows x rd), dY (rows x d), [dU | dG] (rows x 2rd); per layer the re-laid-out
  // weights (see bwd_weights) and the forward encode's packed weights.
  void *mH = nullptr, *mU = nullptr, *mG = nullptr, *mdY = nullptr, *mdUG = nullptr;
  void *uvt[STCA_MAX_M] = {}, *uvc[STCA_MAX_M] = {}, *ot[STCA_MAX_M] = {}, *packed[STCA_MAX_M] = {};
};

// Upper bound on sum_u R_u Lp_u (R_u = m_u h query rows, Lp_u = L_u rounded up to 4):
// sum_u m_u L_u <= min(max_T total_L, max_L total_T), plus 3 per target for the rounding.
int64_t score_elems(const stca_dims *dm, const stca_batch *b) {
  const int64_t ml = std::min(b->max_T * b->total_L, b->max_L * b->total_T);
  return (int64_t)dm->h * (ml + 3 * b->total_T);
}

size_t carve_backward(void *base, const stca_dims *dm, const stca_batch *b, BackwardWs &w, bool keep) {
  Carver c(base);
  const bool mixed = dm->dtype == STCA_BF16;
  if (mixed) keep = false;  // the mixed path recomputes the encode per chunk on the bf16 matrix cores
  const int64_t L = b->total_L, T = b->total_T, d = dm->d, h = dm->h, rd = (int64_t)dm->r * dm->d, M = dm->M;
  w.Xt = c.take<float>((size_t)(M * L * d));
  w.dXt = c.take<float>((size_t)(L * d));
  w.Z = c.take<float>((size_t)(T * M * d));
  w.dO = c.take<float>((size_t)(T * M * d));
  for (int i = 0; i < M; ++i) {
    w.qin[i] = i > 0 ? c.take<float>((size_t)(T * d)) : nullptr;
    w.qA[i] = c.take<float>((size_t)(T * rd));
    w.qG[i] = c.take<float>((size_t)(T * rd));
    w.qY[i] = c.take<float>((size_t)(T * d));
    w.q[i] = c.take<float>((size_t)(T * d));
    w.P[i] = c.take<float>((size_t)(T * d));
    w.U[i] = c.take<float>((size_t)(T * h * d));
    w.lse[i] = c.take<float>((size_t)(T * h));
    w.abar[i] = c.take<float>((size_t)(T * h * d));
    w.heads[i] = c.take<float>((size_t)(T * d));
  }
  w.dq = c.take<float>((size_t)(T * d));
  w.qH = c.take<float>((size_t)(T * rd));
  w.qdA = c.take<float>((size_t)(T * rd));
  w.qdG = c.take<float>((size_t)(T * rd));
  w.qdY = c.take<float>((size_t)(T * d));
  w.dc = c.take<float>((size_t)(T * d));
  w.dheads = c.take<float>((size_t)(T * d));
  w.dabar = c.take<float>((size_t)(T * h * d));
  w.Dv = c.take<float>((size_t)(T * h));
  w.du = c.take<float>((size_t)(T * h * d));
  w.dP = c.take<float>((size_t)(T * d));
  w.rows = std::min<int64_t>(std::max<int64_t>(L, 1), mixed ? kMixedRows : kFfnRows);
  if (!mixed) {
    w.eA = c.take<float>((size_t)(w.rows * rd));
    w.eG = c.take<float>((size_t)(w.rows * rd));
    w.eH = c.take<float>((size_t)(w.rows * rd));
  }
  w.eY = c.take<float>((size_t)(w.rows * d));
  if (!mixed) w.edY = c.take<float>((size_t)(w.rows * d));
  w.parts_cap = (int64_t)kWgradParts * std::max<int64_t>(d * rd, M * d * d);
  w.parts = c.take<float>((size_t)w.parts_cap);
  w.S = c.take<float>((size_t)score_elems(dm, b));
  w.S2 = c.take<float>((size_t)score_elems(dm, b));
  w.desc = c.take<RaggedDesc>((size_t)std::max(3 * b->n_users, 1));
  if (mixed) {
    w.mH = c.take<char>((size_t)(w.rows * rd) * 2);
    w.mU = c.take<char>((size_t)(w.rows * rd) * 2);
    w.mG = c.take<char>((size_t)(w.rows * rd) * 2);
    w.mdY = c.take<char>((size_t)(w.rows * d) * 2);
    w.mdUG = c.take<char>((size_t)(w.rows * 2 * rd) * 2);
    for (int i = 0; i < M; ++i) {
      w.uvt[i] = c.take<char>((size_t)(2 * rd * d) * 2);
      w.uvc[i] = c.take<char>((size_t)(2 * rd * d) * 2);
      w.ot[i] = c.take<char>((size_t)(rd * d) * 2);
      w.packed[i] = c.take<char>(encode_packed_bytes(dm->d, dm->r));
    }
  }
  if (keep) {
    w.kA = c.take<float>((size_t)(M * L * rd));
    w.kG = c.take<float>((size_t)(M * L * rd));
    w.kY = c.take<float>((size_t)(M * L * d));
  }
  return round_up(c.off, 256);
}

// C[Mr x Nc] (row stride ldc) += A^T B over K rows: A is K x Mr (row stride lda, bf16 or fp32),
// B is K x Nc fp32 (row stride ldb).  The rows are split into up to kWgradParts blocks whose
// products land in `parts` and are then added in block order.
int wgrad(hipStream_t s, int Mr, int Nc, int64_t K, const void *A, int64_t lda, bool a_bf16, const float *B,
          int64_t ldb, float *C, int64_t ldc, float *parts) {
  if (K <= 0) return STCA_OK;
  int nsplit = (int)std::min<int64_t>(kWgradParts, (K + 255) / 256);
  const int64_t per = (K + nsplit - 1) / nsplit;
  nsplit = (int)((K + per - 1) / per);
  const int64_t full = K / per;
  const size_t aes = a_bf16 ? 2 : 4;
  GemmArgs g;
  g.M = Mr;
  g.N = Nc;
  g.K = (int)per;
  g.batch = (int)full;
  g.A = A;
  g.lda = lda;
  g.sA = per * lda;
  g.ta_bf16 = a_bf16;
  g.trans_a = true;
  g.B = B;
  g.ldb = ldb;
  g.sB = per * ldb;
  g.C = parts;
  g.ldc = Nc;
  g.sC = (int64_t)Mr * Nc;
  g.mfma_small = true;
  if (full > 0) HIP_TRY(gemm(s, g));
  if (full < nsplit) {
    g.K = (int)(K - full * per);
    g.batch = 1;
    g.A = (const char *)A + (size_t)(full * per * lda) * aes;
    g.B = B + full * per * ldb;
    g.C = parts + full * (int64_t)Mr * Nc;
    HIP_TRY(gemm(s, g));
  }
  HIP_TRY(sum_parts2d(s, Mr, Nc, nsplit, parts, C, ldc, true));
  return STCA_OK;
}

// Per-head weight gradients of eq. (13)'s projections: for every head j, columns j dh .. (j+1) dh of
// C (d x d, row stride ldc) += A_j^T B_j over K rows, where A_j is the j-th d-wide column block of A
// (K x h d, row stride h d) and B_j columns j dh .. (j+1) dh of B (K x d, row stride ldb).  One
// product P = A^T B (h d x d: every head's rows against every head's columns) runs on the matrix
// cores, split over row blocks into `parts`; head j's gradient is P's diagonal block (rows j d ..,
// columns j dh ..), whose part sums are added in block order.  The off-diagonal blocks multiply h - 1
// times the needed work, which costs less than h products of dh columns each.  Falls back to one
// wgrad per head when the parts buffer (parts_cap floats) cannot hold one block of P.
int head_wgrad(hipStream_t s, int d, int h, int64_t K, const float *A, const float *B, int64_t ldb, float *C,
               int64_t ldc, float *parts, int64_t parts_cap) {
  if (K <= 0) return STCA_OK;
  const int dh = d / h;
  const int64_t pblock = (int64_t)h * d * d;
  if (pblock > parts_cap) {
    for (int j = 0; j < h; ++j) {
      const int st = wgrad(s, d, dh, K, A + (size_t)j * d, (int64_t)h * d, false, B + j * dh, ldb, C + j * dh, ldc,
                           parts);
      if (st != STCA_OK) return st;
    }
    return STCA_OK;
  }
  int nsplit = (int)std::min<int64_t>({(int64_t)kWgradParts, parts_cap / pblock, (K + 255) / 256});
  const int64_t per = (K + nsplit - 1) / nsplit;
  nsplit = (int)((K + per - 1) / per);
  const int64_t full = K / per;
  GemmArgs g;
  g.M = h * d;
  g.N = d;
  g.K = (int)per;
  g.batch = (int)full;
  g.A = A;
  g.lda = (int64_t)h * d;
  g.sA = per * g.lda;
  g.trans_a = true;
  g.B = B;
  g.ldb = ldb;
  g.sB = per * ldb;
  g.C = parts;
  g.ldc = d;
  g.sC = pblock;
  g.mfma_small = true;
  if (full > 0) HIP_TRY(gemm(s, g));
  if (full < nsplit) {
    g.K = (int)(K - full * per);
    g.batch = 1;
    g.A = A + full * per * g.lda;
    g.B = B + full * per * ldb;
    g.C = parts + full * pblock;
    HIP_TRY(gemm(s, g));
  }
  for (int j = 0; j < h; ++j)
    HIP_TRY(sum_parts_strided(s, d, dh, nsplit, parts + (int64_t)j * d * d + j * dh, d, pblock, C + j * dh, ldc,
                              true));
  return STCA_OK;
}

// C[m x n] = A B (or A B^T with trans_b) + beta C through the generic GEMM (a helper for the products below).
hipError_t mm(hipStream_t s, int m, int n, int k, const void *A, int64_t lda, bool a_bf16, const void *B,
              int64_t ldb, bool b_bf16, bool trans_b, float *C, int64_t ldc, float beta) {
  GemmArgs g;
  g.M = m;
  g.N = n;
  g.K = k;
  g.A = A;
  g.lda = lda;
  g.ta_bf16 = a_bf16;
  g.B = B;
  g.ldb = ldb;
  g.tb_bf16 = b_bf16;
  g.trans_b = trans_b;
  g.C = C;
  g.ldc = ldc;
  g.beta = beta;
  g.mfma_small = true;  // the per-target products have few tiles; the matrix cores still win
  return gemm(s, g);
}

// eq. (1) on n rows with its intermediates kept: A = x W_u, G = x W_v, H = A * SiLU(G), Y = H W_o.
int ffn_saved(hipStream_t s, const stca_dims *dm, const stca_ffn *f, int64_t n, const void *x, bool x_bf16,
              float *A, float *G, float *H, float *Y) {
  const int d = dm->d, rd = dm->r * dm->d;
  const bool wb = dm->dtype == STCA_BF16;
  HIP_TRY(mm(s, (int)n, rd, d, x, d, x_bf16, f->Wu, rd, wb, false, A, rd, 0.f));
  HIP_TRY(mm(s, (int)n, rd, d, x, d, x_bf16, f->Wv, rd, wb, false, G, rd, 0.f));
  HIP_TRY(swiglu_fwd(s, n * rd, A, G, H));
  HIP_TRY(mm(s, (int)n, d, rd, H, rd, false, f->Wo, d, wb, false, Y, d, 0.f));
  return STCA_OK;
}

// Backward of [LN](SwiGLUFFN(x)) for n rows given dout (n x d): weight gradients added into g,
// dx (n x d) written (or added, when accumulate) through the products dA W_u^T + dG W_v^T.
int ffn_backward(hipStream_t s, const stca_dims *dm, const stca_ffn *f, const stca_ffn_grad &g, bool with_ln,
                 int64_t n, const void *x, bool x_bf16, const float *A, const float *G, float *H, const float *Y,
                 const float *dout, float *dY, float *dx, bool accumulate, float *parts) {
  const int d = dm->d, rd = dm->r * dm->d;
  const bool wb = dm->dtype == STCA_BF16;
  int st;
  const float *dy = dout;
  if (with_ln) {
    HIP_TRY(ln_bwd(s, n, d, dout, d, Y, d, f->gamma, dm->ln_eps, dY, g.dgamma, g.dbeta, parts, kLnBlocks));
    dy = dY;
  }
  if ((st = wgrad(s, rd, d, n, H, rd, false, dy, d, g.dWo, d, parts)) != STCA_OK) return st;
  float *dA = H;  // H is spent: dH, then dA, take its place
  HIP_TRY(mm(s, (int)n, rd, d, dy, d, false, f->Wo, d, wb, true, dA, rd, 0.f));
  float *dG = const_cast<float *>(G);
  HIP_TRY(swiglu_bwd(s, n * rd, dA, A, G, dA, dG));
  if ((st = wgrad(s, d, rd, n, x, d, x_bf16, dA, rd, g.dWu, rd, parts)) != STCA_OK) return st;
  if ((st = wgrad(s, d, rd, n, x, d, x_bf16, dG, rd, g.dWv, rd, parts)) != STCA_OK) return st;
  if (dx) {
    HIP_TRY(mm(s, (int)n, d, rd, dA, rd, false, f->Wu, rd, wb, true, dx, d, accumulate ? 1.f : 0.f));
    HIP_TRY(mm(s, (int)n, d, rd, dG, rd, false, f->Wv, rd, wb, true, dx, d, 1.f));
  }
  return STCA_OK;
}

// Mixed-precision backward of eq. (2) for layer i over all history rows, in row chunks: every product
// on the bf16 matrix cores with fp32 accumulation (gemm_nt), the SwiGLU and its derivative fused into
// the products that produce their inputs, the LayerNorm derivative and the weight-gradient sums in
// fp32.  Per chunk of n rows (x = X rows, dXt = dL/dX~ rows):
//   [u | g] = x [W_u | W_v]   -> H = u SiLU(g), u, g (bf16)                             (kEpiSwigluFwd)
//   Y = H W_o                 -> fp32, then the LayerNorm derivative: dY (bf16), dgamma, dbeta
//   dW_o += H^T dY            (TN product over the rows, split; partial sums added in order)
//   dH = dY W_o^T             -> dU = dH SiLU(g), dG = dH u SiLU'(g) (bf16)                (kEpiSwigluBwd)
//   [dW_u | dW_v] += x^T [dU | dG]   (TN, split as dW_o)
//   dX += [dU | dG] [W_u | W_v]^T
// Every intermediate is row-major: the weight gradients read the rows through the TN layout.
int encode_backward_mixed(hipStream_t s, const stca_dims *dm, const stca_ffn &f, const stca_ffn_grad &g, int i,
                          const BackwardWs &bw, int64_t L, const void *X, const float *dXt, float *dX) {
  const int d = dm->d, rd = dm->r * dm->d;
  for (int64_t r0 = 0; r0 < L; r0 += bw.rows) {
    const int n = (int)std::min<int64_t>(bw.rows, L - r0);
    const void *x = (const char *)X + (size_t)r0 * d * 2;
    NtEpilogue e1;
    e1.H = bw.mH;
    e1.U = bw.mU;
    e1.G = bw.mG;
    e1.ldh = rd;
    HIP_TRY(gemm_nt(s, kEpiSwigluFwd, n, 2 * rd, d, 0, 1, x, d, 0, bw.uvt[i], d, 0, e1));
    NtEpilogue e2;
    e2.C = bw.eY;
    e2.ldc = d;
    HIP_TRY(gemm_nt(s, kEpiStore, n, d, rd, 0, 1, bw.mH, rd, 0, bw.ot[i], rd, 0, e2));
    HIP_TRY(ln_bwd_bf16(s, n, d, dXt + (size_t)r0 * d, bw.eY, f.gamma, dm->ln_eps, bw.mdY, g.dgamma, g.dbeta,
                        bw.parts));
    // dW_o (rd x d) over the chunk's rows, split into blocks of ks rows
    {
      const int64_t ks = round_up((n + kWgradParts - 1) / kWgradParts, 64), parts = (n + ks - 1) / ks;
      NtEpilogue e3;
      e3.C = bw.parts;
      e3.ldc = d;
      e3.sC = (int64_t)rd * d;
      HIP_TRY(gemm_tn(s, kEpiStore, rd, d, n, (int)ks, (int)parts, bw.mH, rd, 0, bw.mdY, d, 0, e3));
      HIP_TRY(sum_parts_strided(s, rd, d, (int)parts, bw.parts, d, (int64_t)rd * d, g.dWo, d, true));
    }
    NtEpilogue e4;
    e4.U = bw.mU;
    e4.G = bw.mG;
    e4.ldh = rd;
    e4.dUG = bw.mdUG;
    e4.lddug = 2 * rd;
    e4.rd = rd;
    HIP_TRY(gemm_nt(s, kEpiSwigluBwd, n, rd, d, 0, 1, bw.mdY, d, 0, f.Wo, d, 0, e4));
    // [dW_u | dW_v] (d x 2rd) over the chunk's rows
    {
      const int max_parts = kWgradParts / 2;  // the parts buffer holds 16 blocks of d x 2rd
      const int64_t ks = round_up((n + max_parts - 1) / max_parts, 64), parts = (n + ks - 1) / ks;
      NtEpilogue e5;
      e5.C = bw.parts;
      e5.ldc = 2 * rd;
      e5.sC = (int64_t)d * 2 * rd;
      HIP_TRY(gemm_tn(s, kEpiStore, d, 2 * rd, n, (int)ks, (int)parts, x, d, 0, bw.mdUG, 2 * rd, 0, e5));
      HIP_TRY(sum_parts_strided(s, d, rd, (int)parts, bw.parts, 2 * rd, (int64_t)d * 2 * rd, g.dWu, rd, true));
      HIP_TRY(sum_parts_strided(s, d, rd, (int)parts, bw.parts + rd, 2 * rd, (int64_t)d * 2 * rd, g.dWv, rd, true));
    }
    if (dX) {
      NtEpilogue e6;
      e6.C = dX + (size_t)r0 * d;
      e6.ldc = d;
      HIP_TRY(gemm_nt(s, kEpiAcc, n, d, 2 * rd, 0, 1, bw.mdUG, 2 * rd, 0, bw.uvc[i], 2 * rd, 0, e6));
    }
  }
  return STCA_OK;
}

int check_grads(const stca_dims *dm, const stca_grads *g) {
  if (!g) return fail(STCA_E_ARG, "grads is NULL");
  auto al = [](const void *p) { return aligned16(p); };
  if (!al(g->dX) || !al(g->dxt)) return fail(STCA_E_ALIGN, "dX/dxt not 16-byte aligned");
  for (int i = 0; i < dm->M; ++i) {
    const stca_ffn_grad *fs[2] = {&g->hist[i], &g->query[i]};
    for (int k = 0; k < 2; ++k) {
      const stca_ffn_grad &f = *fs[k];
      const bool need_ln = k == 0 || i == 0 || dm->query_ln;
      if (!f.dWu || !f.dWv || !f.dWo || (need_ln && (!f.dgamma || !f.dbeta)))
        return fail(STCA_E_ARG, "layer %d: %s FFN gradient pointer NULL", i, k ? "query" : "hist");
      if (!al(f.dWu) || !al(f.dWv) || !al(f.dWo) || !al(f.dgamma) || !al(f.dbeta))
        return fail(STCA_E_ALIGN, "layer %d: FFN gradients not 16-byte aligned", i);
    }
    if (!g->dWQ[i] || !g->dWK[i] || !g->dWV[i] || !g->dWO[i] || (i >= 1 && !g->dWC[i]))
      return fail(STCA_E_ARG, "layer %d: attention gradient pointer NULL", i);
    if (!al(g->dWQ[i]) || !al(g->dWK[i]) || !al(g->dWV[i]) || !al(g->dWO[i]) || (i >= 1 && !al(g->dWC[i])))
      return fail(STCA_E_ALIGN, "layer %d: attention gradients not 16-byte aligned", i);
  }
  return STCA_OK;
}

int backward_impl(const stca_dims *dm, const stca_weights *w, const stca_batch *b, const void *X, const void *xt,
                  const float *dZ, const stca_grads *g, void *ws, size_t ws_bytes, hipStream_t s,
                  stca_profiler *prof) {
  int st;
  if ((st = check_dims(dm)) != STCA_OK) return st;
  if ((st = check_batch(b)) != STCA_OK) return st;
  if ((st = check_weights(dm, w)) != STCA_OK) return st;
  if ((st = check_grads(dm, g)) != STCA_OK) return st;
  if (b->total_L > 0 && !X) return fail(STCA_E_ARG, "X is NULL");
  if (b->total_T > 0 && (!xt || !dZ)) return fail(STCA_E_ARG, "xt or dZ is NULL");
  if (!aligned16(X) || !aligned16(xt) || !aligned16(dZ)) return fail(STCA_E_ALIGN, "X/xt/dZ not 16-byte aligned");
  if (b->total_T > (int64_t)1 << 22) return fail(STCA_E_ARG, "total_T %lld exceeds 2^22", (long long)b->total_T);
  BackwardWs bw;
  const size_t need = carve_backward(nullptr, dm, b, bw, false);
  if (!ws || ws_bytes < need)
    return fail(STCA_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes, need);
  if (!aligned16(ws)) return fail(STCA_E_ALIGN, "workspace not 16-byte aligned");
  const bool keep = ws_bytes >= carve_backward(nullptr, dm, b, bw, true);
  carve_backward(ws, dm, b, bw, keep);

  const int d = dm->d, h = dm->h, dh = d / h, M = dm->M, rd = dm->r * dm->d;
  const int64_t L = b->total_L, T = b->total_T;
  const bool bf = dm->dtype == STCA_BF16;
  const float sc = 1.0f / sqrtf((float)dh);

  // Every output starts at zero; the steps below add into them.
  if (g->dX) HIP_TRY(fill_f32(s, L * d, g->dX, 0.f));
  if (g->dxt) HIP_TRY(fill_f32(s, T * d, g->dxt, 0.f));
  for (int i = 0; i < M; ++i) {
    const stca_ffn_grad *fs[2] = {&g->hist[i], &g->query[i]};
    for (const stca_ffn_grad *f : fs) {
      HIP_TRY(fill_f32(s, (int64_t)d * rd, f->dWu, 0.f));
      HIP_TRY(fill_f32(s, (int64_t)d * rd, f->dWv, 0.f));
      HIP_TRY(fill_f32(s, (int64_t)d * rd, f->dWo, 0.f));
      if (f->dgamma) HIP_TRY(fill_f32(s, d, f->dgamma, 0.f));
      if (f->dbeta) HIP_TRY(fill_f32(s, d, f->dbeta, 0.f));
    }
    for (float *p : {g->dWQ[i], g->dWK[i], g->dWV[i], g->dWO[i]}) HIP_TRY(fill_f32(s, (int64_t)d * d, p, 0.f));
    if (i >= 1) HIP_TRY(fill_f32(s, (int64_t)(i + 1) * d * d, g->dWC[i], 0.f));
  }
  if (T == 0) return STCA_OK;  // no target, no gradient
  HIP_TRY(ragged_plan(s, b->n_users, b->hist_off, b->tgt_off, h, d, b->total_L, b->total_T, b->max_L, b->max_T,
                      score_elems(dm, b), bw.desc));
  if (bf) {  // mixed path: weight layouts of every history FFN and the forward encode's packed weights
    for (int i = 0; i < M; ++i) {
      const stca_ffn &f = w->hist[i];
      HIP_TRY(bwd_weights(s, d, dm->r, f.Wu, f.Wv, f.Wo, bw.uvt[i], bw.uvc[i], bw.ot[i]));
      HIP_TRY(encode_pack(s, d, dm->r, f.Wu, f.Wv, f.Wo, bw.packed[i]));
    }
  }
  const int64_t T_rows = b->max_T * h, max_L = b->max_L;  // bounds of the ragged products' sizes
  auto rg = [](const float *A, const float *B, float *C, float alpha, float beta, bool ta, bool tb) {
    GemmArgs g;
    g.A = A;
    g.B = B;
    g.C = C;
    g.alpha = alpha;
    g.beta = beta;
    g.trans_a = ta;
    g.trans_b = tb;
    return g;
  };

  // ---- forward, keeping what the backward needs ----------------------------------------------
  // Per-target steps are timed as STCA_PHASE_BWD_TARGET, the per-history-row ones by their phases.
  auto qffn_in = [&](int i) -> const void * { return i == 0 ? xt : (const void *)bw.qin[i]; };
  auto q_forward = [&](int i) -> int {  // eq. (3) (i = 0) or eq. (7): q(i) from its FFN input
    const stca_ffn &f = w->query[i];
    int st2;
    if ((st2 = ffn_saved(s, dm, &f, T, qffn_in(i), i == 0 && bf, bw.qA[i], bw.qG[i], bw.qH, bw.qY[i])) != STCA_OK)
      return st2;
    if (i == 0 || dm->query_ln)
      HIP_TRY(layernorm_rows(s, T, d, bw.qY[i], d, bw.q[i], d, false, f.gamma, f.beta, dm->ln_eps));
    else
      HIP_TRY(copy_rows(s, T, d, bw.qY[i], d, bw.q[i], d));
    return STCA_OK;
  };
  {
    Phase ph(prof, s, STCA_PHASE_BWD_TARGET);
    if ((st = q_forward(0)) != STCA_OK) return st;
    HIP_TRY(ph.end());
  }
  for (int i = 0; i < M; ++i) {
    float *Xt = bw.Xt + (size_t)i * L * d;
    {
      Phase ph(prof, s, STCA_PHASE_BWD_RECOMPUTE);
      // eq. (2): the mixed path runs the forward's fused encode with an fp32 output; the fp32 path in row
      // chunks, keeping A, G and the pre-LN rows with the keep workspace
      if (bf)
        HIP_TRY(encode_mfma(s, d, dm->r, L, X, d, bw.packed[i], Xt, d, false, true, w->hist[i].gamma,
                            w->hist[i].beta, dm->ln_eps));
      for (int64_t r0 = 0; r0 < (bf ? 0 : L); r0 += bw.rows) {
        const int64_t n = std::min<int64_t>(bw.rows, L - r0);
        float *A = bw.eA, *G = bw.eG, *Y = bw.eY;
        if (keep) {
          A = bw.kA + ((size_t)i * L + r0) * rd;
          G = bw.kG + ((size_t)i * L + r0) * rd;
          Y = bw.kY + ((size_t)i * L + r0) * d;
        }
        if ((st = ffn_saved(s, dm, &w->hist[i], n, (const char *)X + (size_t)r0 * d * esize(dm), bf, A, G, bw.eH,
                            Y)) != STCA_OK)
          return st;
        HIP_TRY(layernorm_rows(s, n, d, Y, d, Xt + (size_t)r0 * d, d, false, w->hist[i].gamma, w->hist[i].beta,
                               dm->ln_eps));
      }
      HIP_TRY(ph.end());
    }
    Phase pt(prof, s, STCA_PHASE_BWD_TARGET);
    HIP_TRY(mm(s, (int)T, d, d, bw.q[i], d, false, w->WQ[i], d, bf, false, bw.P[i], d, 0.f));  // P = q W_Q
    GemmArgs u;  // u_j = P_j W_K,j^T (eq. (13)), unscaled
    u.M = (int)T;
    u.N = d;
    u.K = dh;
    u.batch = h;
    u.A = bw.P[i];
    u.lda = d;
    u.sA = dh;
    u.B = w->WK[i];
    u.ldb = d;
    u.sB = dh;
    u.tb_bf16 = bf;
    u.trans_b = true;
    u.C = bw.U[i];
    u.ldc = (int64_t)h * d;
    u.sC = d;
    HIP_TRY(gemm(s, u));
    HIP_TRY(pt.end());
    {
      Phase ph(prof, s, STCA_PHASE_BWD_ATTEND);
      HIP_TRY(gemm_ragged(s, rg(bw.U[i], Xt, bw.S, 1.f, 0.f, false, true), bw.desc, b->n_users, T_rows, max_L, bf));
      HIP_TRY(ragged_rows(s, 0, T * h, h, b->n_users, b->tgt_off, bw.desc, bw.S, nullptr, sc, bw.lse[i], nullptr));
      HIP_TRY(gemm_ragged(s, rg(bw.S, Xt, bw.abar[i], 1.f, 0.f, false, false), bw.desc + b->n_users, b->n_users,
                          T_rows, d, bf));
      HIP_TRY(ph.end());
    }
    Phase pt2(prof, s, STCA_PHASE_BWD_TARGET);
    GemmArgs v;  // heads_j = abar_j W_V,j
    v.M = (int)T;
    v.N = dh;
    v.K = d;
    v.batch = h;
    v.A = bw.abar[i];
    v.lda = (int64_t)h * d;
    v.sA = d;
    v.B = w->WV[i];
    v.ldb = d;
    v.sB = dh;
    v.tb_bf16 = bf;
    v.C = bw.heads[i];
    v.ldc = d;
    v.sC = dh;
    HIP_TRY(gemm(s, v));
    HIP_TRY(mm(s, (int)T, d, d, bw.heads[i], d, false, w->WO[i], d, bf, false, bw.Z + (size_t)i * d, (int64_t)M * d,
               0.f));  // eq. (6)
    if (i + 1 < M) {  // eq. (7)
      HIP_TRY(concat_project(s, dm, T, bw.Z, (int64_t)M * d, i + 1, xt, w->WC[i + 1], bw.qin[i + 1]));
      if ((st = q_forward(i + 1)) != STCA_OK) return st;
    }
    HIP_TRY(pt2.end());
  }

  // ---- backward, last layer first -------------------------------------------------------------
  HIP_TRY(copy_rows(s, T, M * d, dZ, (int64_t)M * d, bw.dO, (int64_t)M * d));  // eq. (8)
  auto q_backward = [&](int i) -> int {  // consumes bw.dq = dL/dq(i)
    const stca_ffn &f = w->query[i];
    const bool with_ln = i == 0 || dm->query_ln;
    int st2;
    HIP_TRY(swiglu_fwd(s, T * rd, bw.qA[i], bw.qG[i], bw.qH));
    float *dx = i == 0 ? g->dxt : bw.dc;
    if ((st2 = ffn_backward(s, dm, &f, g->query[i], with_ln, T, qffn_in(i), i == 0 && bf, bw.qA[i], bw.qG[i], bw.qH,
                            bw.qY[i], bw.dq, bw.qdY, dx, i == 0, bw.parts)) != STCA_OK)
      return st2;
    if (i == 0) return STCA_OK;
    // c = [o(1) .. o(i) || x_t] W_C(i): gradients of W_C, of every earlier o and of x_t.
    if ((st2 = wgrad(s, i * d, d, T, bw.Z, (int64_t)M * d, false, bw.dc, d, g->dWC[i], d, bw.parts)) != STCA_OK)
      return st2;
    if ((st2 = wgrad(s, d, d, T, xt, d, bf, bw.dc, d, g->dWC[i] + (size_t)i * d * d, d, bw.parts)) != STCA_OK)
      return st2;
    HIP_TRY(mm(s, (int)T, i * d, d, bw.dc, d, false, w->WC[i], d, bf, true, bw.dO, (int64_t)M * d, 1.f));
    if (g->dxt)
      HIP_TRY(mm(s, (int)T, d, d, bw.dc, d, false, (const char *)w->WC[i] + (size_t)i * d * d * esize(dm), d, bf, true,
                 g->dxt, d, 1.f));
    return STCA_OK;
  };
  for (int i = M - 1; i >= 0; --i) {
    Phase pt(prof, s, STCA_PHASE_BWD_TARGET);
    if (i + 1 < M && (st = q_backward(i + 1)) != STCA_OK) return st;
    const float *Xt = bw.Xt + (size_t)i * L * d;
    const float *dO = bw.dO + (size_t)i * d;
    const int64_t ldo = (int64_t)M * d;
    // eq. (6)
    if ((st = wgrad(s, d, d, T, bw.heads[i], d, false, dO, ldo, g->dWO[i], d, bw.parts)) != STCA_OK) return st;
    HIP_TRY(mm(s, (int)T, d, d, dO, ldo, false, w->WO[i], d, bf, true, bw.dheads, d, 0.f));
    // eq. (13), per head: W_V, then the softmax and the two projections in front of it
    if ((st = head_wgrad(s, d, h, T, bw.abar[i], bw.dheads, d, g->dWV[i], d, bw.parts, bw.parts_cap)) != STCA_OK)
      return st;
    GemmArgs da;  // dabar_j = dheads_j W_V,j^T
    da.M = (int)T;
    da.N = d;
    da.K = dh;
    da.batch = h;
    da.A = bw.dheads;
    da.lda = d;
    da.sA = dh;
    da.B = w->WV[i];
    da.ldb = d;
    da.sB = dh;
    da.tb_bf16 = bf;
    da.trans_b = true;
    da.C = bw.dabar;
    da.ldc = (int64_t)h * d;
    da.sC = d;
    HIP_TRY(gemm(s, da));
    HIP_TRY(rowdot(s, T * h, d, bw.dabar, bw.abar[i], bw.Dv));
    HIP_TRY(pt.end());
    {  // alpha again (saved lse), dA = dabar X~^T, dS, then du and dX~ (eq. (13))
      Phase ph(prof, s, STCA_PHASE_BWD_ATTEND);
      const RaggedDesc *d_s = bw.desc, *d_row = bw.desc + b->n_users, *d_key = bw.desc + 2 * b->n_users;
      HIP_TRY(gemm_ragged(s, rg(bw.U[i], Xt, bw.S, 1.f, 0.f, false, true), d_s, b->n_users, T_rows, max_L, bf));
      HIP_TRY(ragged_rows(s, 1, T * h, h, b->n_users, b->tgt_off, d_s, bw.S, nullptr, sc, bw.lse[i], nullptr));
      HIP_TRY(gemm_ragged(s, rg(bw.dabar, Xt, bw.S2, 1.f, 0.f, false, true), d_s, b->n_users, T_rows, max_L, bf));
      HIP_TRY(ragged_rows(s, 2, T * h, h, b->n_users, b->tgt_off, d_s, bw.S, bw.S2, sc, nullptr, bw.Dv));
      HIP_TRY(gemm_ragged(s, rg(bw.S2, Xt, bw.du, sc, 0.f, false, false), d_row, b->n_users, T_rows, d, bf));
      HIP_TRY(gemm_ragged(s, rg(bw.S, bw.dabar, bw.dXt, 1.f, 0.f, true, false), d_key, b->n_users, max_L, d, bf));
      HIP_TRY(gemm_ragged(s, rg(bw.S2, bw.U[i], bw.dXt, sc, 1.f, true, false), d_key, b->n_users, max_L, d, bf));
      HIP_TRY(ph.end());
    }
    Phase pt2(prof, s, STCA_PHASE_BWD_TARGET);
    GemmArgs dp;  // dP_j = du_j W_K,j
    dp.M = (int)T;
    dp.N = dh;
    dp.K = d;
    dp.batch = h;
    dp.A = bw.du;
    dp.lda = (int64_t)h * d;
    dp.sA = d;
    dp.B = w->WK[i];
    dp.ldb = d;
    dp.sB = dh;
    dp.tb_bf16 = bf;
    dp.C = bw.dP;
    dp.ldc = d;
    dp.sC = dh;
    HIP_TRY(gemm(s, dp));
    if ((st = head_wgrad(s, d, h, T, bw.du, bw.P[i], d, g->dWK[i], d, bw.parts, bw.parts_cap)) != STCA_OK) return st;
    if ((st = wgrad(s, d, d, T, bw.q[i], d, false, bw.dP, d, g->dWQ[i], d, bw.parts)) != STCA_OK) return st;
    HIP_TRY(mm(s, (int)T, d, d, bw.dP, d, false, w->WQ[i], d, bf, true, bw.dq, d, 0.f));
    HIP_TRY(pt2.end());
    // eq. (2): LayerNorm and SwiGLU FFN of every history row, in row chunks
    Phase pe(prof, s, STCA_PHASE_BWD_ENCODE);
    if (bf && (st = encode_backward_mixed(s, dm, w->hist[i], g->hist[i], i, bw, L, X, bw.dXt, g->dX)) != STCA_OK)
      return st;
    const size_t xes = esize(dm);
    for (int64_t r0 = 0; r0 < (bf ? 0 : L); r0 += bw.rows) {
      const int64_t n = std::min<int64_t>(bw.rows, L - r0);
      const void *Xc = (const char *)X + (size_t)r0 * d * xes;
      float *A = bw.eA, *G = bw.eG, *Y = bw.eY;
      if (keep) {  // kept from the recompute: only H = A * SiLU(G) is formed again (G is consumed below)
        A = bw.kA + ((size_t)i * L + r0) * rd;
        G = bw.kG + ((size_t)i * L + r0) * rd;
        Y = bw.kY + ((size_t)i * L + r0) * d;
        HIP_TRY(swiglu_fwd(s, n * rd, A, G, bw.eH));
      } else if ((st = ffn_saved(s, dm, &w->hist[i], n, Xc, bf, A, G, bw.eH, Y)) != STCA_OK) {
        return st;
      }
      if ((st = ffn_backward(s, dm, &w->hist[i], g->hist[i], true, n, Xc, bf, A, G, bw.eH, Y,
                             bw.dXt + (size_t)r0 * d, bw.edY, g->dX ? g->dX + (size_t)r0 * d : nullptr, true,
                             bw.parts)) != STCA_OK)
        return st;
    }
    HIP_TRY(pe.end());
  }
  Phase pt(prof, s, STCA_PHASE_BWD_TARGET);
  if ((st = q_backward(0)) != STCA_OK) return st;
  HIP_TRY(pt.end());
  return STCA_OK;
}

}  // namespace
}  // namespace stca_abi

using namespace stca_abi;

extern "C" {

int stca_backward_workspace_size(const stca_dims *dims, const stca_batch *batch, size_t *bytes) {
  int st;
  if ((st = check_dims(dims)) != STCA_OK) return st;
  if ((st = check_batch(batch)) != STCA_OK) return st;
  if (!bytes) return fail(STCA_E_ARG, "bytes is NULL");
  BackwardWs bw;
  *bytes = carve_backward(nullptr, dims, batch, bw, false);
  return STCA_OK;
}

int stca_backward_workspace_size_keep(const stca_dims *dims, const stca_batch *batch, size_t *bytes) {
  int st;
  if ((st = check_dims(dims)) != STCA_OK) return st;
  if ((st = check_batch(batch)) != STCA_OK) return st;
  if (!bytes) return fail(STCA_E_ARG, "bytes is NULL");
  BackwardWs bw;
  *bytes = carve_backward(nullptr, dims, batch, bw, true);
  return STCA_OK;
}

int stca_backward(const stca_dims *dims, const stca_weights *w, const stca_batch *batch, const void *X,
                  const void *xt, const float *dZ, const stca_grads *grads, void *workspace, size_t workspace_bytes,
                  void *stream) {
  return backward_impl(dims, w, batch, X, xt, dZ, grads, workspace, workspace_bytes, (hipStream_t)stream, nullptr);
}

int stca_backward_profiled(const stca_dims *dims, const stca_weights *w, const stca_batch *batch, const void *X,
                           const void *xt, const float *dZ, const stca_grads *grads, void *workspace,
                           size_t workspace_bytes, void *stream, stca_profiler *prof) {
  return backward_impl(dims, w, batch, X, xt, dZ, grads, workspace, workspace_bytes, (hipStream_t)stream, prof);
}

}  // extern "C"
