// libstca C ABI: argument checks, workspace layout, launch sequence of the forward and the other
// calls of include/stca.h (the backward pass is in api_backward.hip).
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "abi_common.hpp"

using namespace stca;

namespace stca_abi {

thread_local std::string g_last_error;

int fail(int status, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int check_dims(const stca_dims *dm) {
  if (!dm) return fail(STCA_E_ARG, "dims is NULL");
  const int d = dm->d, h = dm->h;
  if (!(d == 64 || d == 128 || d == 256 || d == 512)) return fail(STCA_E_DIMS, "d=%d not in {64,128,256,512}", d);
  if (h <= 0 || d % h != 0) return fail(STCA_E_DIMS, "h=%d must be positive and divide d=%d", h, d);
  if (dm->r < 1 || dm->r > 8) return fail(STCA_E_DIMS, "r=%d not in [1,8]", dm->r);
  if (dm->M < 1 || dm->M > STCA_MAX_M) return fail(STCA_E_DIMS, "M=%d not in [1,%d]", dm->M, STCA_MAX_M);
  if (dm->dtype != STCA_F32 && dm->dtype != STCA_BF16) return fail(STCA_E_DIMS, "dtype=%d unknown", dm->dtype);
  if (!(dm->ln_eps > 0.f)) return fail(STCA_E_DIMS, "ln_eps must be > 0");
  if (dm->attn_chunk < 0 || dm->attn_chunk % 32 != 0)
    return fail(STCA_E_DIMS, "attn_chunk=%d must be 0 or a positive multiple of 32", dm->attn_chunk);
  if (dm->encode_layers < 0 || dm->encode_layers > 2)
    return fail(STCA_E_DIMS, "encode_layers=%d must be 0, 1 or 2", dm->encode_layers);
  return STCA_OK;
}

int check_batch(const stca_batch *b) {
  if (!b) return fail(STCA_E_ARG, "batch is NULL");
  if (b->n_users < 0) return fail(STCA_E_ARG, "n_users < 0");
  if (b->total_L < 0 || b->total_T < 0 || b->max_L < 0 || b->max_T < 0)
    return fail(STCA_E_ARG, "negative batch size");
  if (b->total_L > 0 && b->n_users == 0) return fail(STCA_E_ARG, "total_L > 0 with no users");
  if (b->total_T > 0 && b->n_users == 0) return fail(STCA_E_ARG, "total_T > 0 with no users");
  if (b->n_users > 0 && (!b->hist_off || !b->tgt_off)) return fail(STCA_E_ARG, "offsets are NULL");
  if (b->max_L > b->total_L || b->max_T > b->total_T) return fail(STCA_E_ARG, "max_L/max_T exceed totals");
  if (b->n_users > 0 && b->total_L > 0 && b->max_L * (int64_t)b->n_users < b->total_L)
    return fail(STCA_E_ARG, "max_L * n_users < total_L: max_L is not an upper bound");
  if (b->n_users > 0 && b->total_T > 0 && b->max_T * (int64_t)b->n_users < b->total_T)
    return fail(STCA_E_ARG, "max_T * n_users < total_T: max_T is not an upper bound");
  if (!aligned16(b->hist_off) || !aligned16(b->tgt_off)) return fail(STCA_E_ALIGN, "offsets not 16-byte aligned");
  return STCA_OK;
}

int check_ffn(const stca_ffn *f, bool need_ln, const char *what) {
  if (!f) return fail(STCA_E_ARG, "%s: ffn is NULL", what);
  if (!f->Wu || !f->Wv || !f->Wo) return fail(STCA_E_ARG, "%s: W_u/W_v/W_o NULL", what);
  if (need_ln && (!f->gamma || !f->beta)) return fail(STCA_E_ARG, "%s: LayerNorm gamma/beta NULL", what);
  if (!aligned16(f->Wu) || !aligned16(f->Wv) || !aligned16(f->Wo) || (f->gamma && !aligned16(f->gamma)) ||
      (f->beta && !aligned16(f->beta)))
    return fail(STCA_E_ALIGN, "%s: weights not 16-byte aligned", what);
  return STCA_OK;
}

int check_layer_weights(const stca_dims *dm, const stca_weights *w, int i) {
  if (!w->WQ[i] || !w->WK[i] || !w->WV[i] || !w->WO[i]) return fail(STCA_E_ARG, "layer %d: W_Q/W_K/W_V/W_O NULL", i);
  if (!aligned16(w->WQ[i]) || !aligned16(w->WK[i]) || !aligned16(w->WV[i]) || !aligned16(w->WO[i]))
    return fail(STCA_E_ALIGN, "layer %d: attention weights not 16-byte aligned", i);
  (void)dm;
  return STCA_OK;
}

int check_weights(const stca_dims *dm, const stca_weights *w) {
  if (!w) return fail(STCA_E_ARG, "weights are NULL");
  for (int i = 0; i < dm->M; ++i) {
    int st;
    if ((st = check_ffn(&w->hist[i], true, "hist")) != STCA_OK) return st;
    const bool q_ln = (i == 0) || dm->query_ln;
    if ((st = check_ffn(&w->query[i], q_ln, "query")) != STCA_OK) return st;
    if ((st = check_layer_weights(dm, w, i)) != STCA_OK) return st;
    if (i >= 1) {
      if (!w->WC[i]) return fail(STCA_E_ARG, "layer %d: W_C NULL", i);
      if (!aligned16(w->WC[i])) return fail(STCA_E_ALIGN, "layer %d: W_C not aligned", i);
    }
  }
  return STCA_OK;
}

// ---- attention plan -------------------------------------------------------------------------
int auto_chunk(const stca_dims *dm, const stca_batch *b) {
  if (dm->attn_chunk > 0) return dm->attn_chunk;
  // Aim for about four work items per compute unit (one resident workgroup each at d >= 256),
  // enough to balance ragged lengths, while keeping chunks long: every extra chunk of a user
  // writes and re-reads a partial state (max, sum, m h x d accumulator) through HBM.
  const int rpg = attn_rows_per_group(dm->d);
  const int64_t groups = std::max<int64_t>(1, (b->max_T * dm->h + rpg - 1) / rpg);
  const int64_t target_items = 1024;
  int64_t c = (b->total_L * groups + target_items - 1) / target_items;
  c = std::max<int64_t>(c, 512);
  c = std::min<int64_t>(c, std::max<int64_t>(b->max_L, 32));
  c = (c + 31) / 32 * 32;
  return (int)std::min<int64_t>(c, 1 << 30);
}

AttnPlan make_plan(const stca_dims *dm, const stca_batch *b) {
  AttnPlan p;
  p.n_users = b->n_users;
  p.h = dm->h;
  p.d = dm->d;
  p.chunk = auto_chunk(dm, b);
  p.total_L = b->total_L;
  p.total_T = b->total_T;
  p.max_L = b->max_L;
  p.max_T = b->max_T;
  const int rpg = attn_rows_per_group(dm->d);
  const int64_t groups = (b->max_T * dm->h + rpg - 1) / rpg;
  const int64_t chunks_ceil = (b->total_L + p.chunk - 1) / p.chunk;
  // sum_u ceil(L_u / c) ceil(m_u h / 128) <= (total_L / c + n_users) * ceil(max_T h / 128)
  p.max_items = b->total_T > 0 ? (chunks_ceil + b->n_users) * groups : 0;
  // Partial-state rows of users with >= 2 chunks: sum_u ceil(L_u / c) m_u h
  //   <= h (max_T total_L / c + total_T).
  p.max_part_rows = b->max_L > p.chunk ? (int64_t)dm->h * (b->max_T * chunks_ceil + b->total_T) : 0;
  return p;
}

// ---- workspace layout -------------------------------------------------------------------------
struct AttendWs {
  AttnBuffers ab;
  void *U = nullptr;       // T*h x d (dtype)
  float *abar = nullptr;   // T*h x d
  float *obar = nullptr;   // T x d
};

void carve_attend(Carver &c, const stca_dims *dm, const stca_batch *b, const AttnPlan &p, AttendWs &w) {
  const int64_t T = b->total_T, d = dm->d, h = dm->h;
  w.U = c.take<char>((size_t)(T * h * d) * esize(dm));
  w.abar = c.take<float>((size_t)(T * h * d));
  w.obar = c.take<float>((size_t)(T * d));
  w.ab.items = c.take<WorkItem>((size_t)std::max<int64_t>(p.max_items, 1));
  w.ab.n_items = c.take<int32_t>(4);
  w.ab.user_nchunks = c.take<int32_t>((size_t)std::max(b->n_users, 1));
  w.ab.part_base = c.take<int64_t>((size_t)std::max(b->n_users, 1));
  w.ab.tgt_user = c.take<int32_t>((size_t)std::max<int64_t>(T, 1));
  w.ab.part_A = c.take<float>((size_t)(p.max_part_rows * d));
  w.ab.part_ms = c.take<float>((size_t)(p.max_part_rows * 2));
}

void carve_ffn(Carver &c, const stca_dims *dm, int64_t rows, FfnWs &w) {
  const int64_t rc = std::min<int64_t>(std::max<int64_t>(rows, 1), kFfnRows);
  w.A = c.take<float>((size_t)(rc * dm->r * dm->d));
  w.G = c.take<float>((size_t)(rc * dm->r * dm->d));
}


// ---- building blocks --------------------------------------------------------------------------
// out[rows x d] = [LN](SwiGLUFFN(x)) with fp32 accumulation through the generic kernels.
int ffn_generic(hipStream_t s, const stca_dims *dm, const stca_ffn *f, int64_t rows, const void *x, int64_t ldx,
                bool x_bf16, void *out, int64_t ldo, bool out_bf16, bool apply_ln, const FfnWs &w) {
  const int d = dm->d, rd = dm->r * dm->d;
  const bool wb = dm->dtype == STCA_BF16;
  const size_t xes = x_bf16 ? 2 : 4, oes = out_bf16 ? 2 : 4;
  for (int64_t r0 = 0; r0 < rows; r0 += kFfnRows) {
    const int n = (int)std::min<int64_t>(kFfnRows, rows - r0);
    const char *xp = (const char *)x + (size_t)r0 * ldx * xes;
    GemmArgs g;
    g.M = n;
    g.N = rd;
    g.K = d;
    g.A = xp;
    g.lda = ldx;
    g.ta_bf16 = x_bf16;
    g.B = f->Wu;
    g.ldb = rd;
    g.tb_bf16 = wb;
    g.C = w.A;
    g.ldc = rd;
    HIP_TRY(gemm(s, g));
    g.B = f->Wv;
    g.C = w.G;
    HIP_TRY(gemm(s, g));
    HIP_TRY(swiglu_gate_inplace(s, (int64_t)n * rd, w.A, w.G));
    GemmArgs g2;
    g2.M = n;
    g2.N = d;
    g2.K = rd;
    g2.A = w.A;
    g2.lda = rd;
    g2.B = f->Wo;
    g2.ldb = d;
    g2.tb_bf16 = wb;
    if (apply_ln) {
      g2.C = w.G;  // fp32 staging, then LayerNorm into out
      g2.ldc = d;
      HIP_TRY(gemm(s, g2));
      HIP_TRY(layernorm_rows(s, n, d, w.G, d, (char *)out + (size_t)r0 * ldo * oes, ldo, out_bf16, f->gamma, f->beta,
                             dm->ln_eps));
    } else {
      g2.C = (char *)out + (size_t)r0 * ldo * oes;
      g2.ldc = ldo;
      g2.tc_bf16 = out_bf16;
      HIP_TRY(gemm(s, g2));
    }
  }
  return STCA_OK;
}

// c[T x d] = [Zb(1) || ... || Zb(nblk) || x_t] W: the first nblk d-wide blocks of each row of Z
// (row stride ldz, fp32) and x_t (dtype) against the row blocks of W ((nblk+1)d x d, dtype),
// as two GEMMs so the concatenation is never materialised (eqs. (7) and (9)).
hipError_t concat_project(hipStream_t s, const stca_dims *dm, int64_t T, const float *Z, int64_t ldz, int nblk,
                          const void *xt, const void *W, float *c) {
  const int d = dm->d;
  const bool bf = dm->dtype == STCA_BF16;
  GemmArgs g;
  g.M = (int)T;
  g.N = d;
  g.K = nblk * d;
  g.A = Z;
  g.lda = ldz;
  g.B = W;
  g.ldb = d;
  g.tb_bf16 = bf;
  g.C = c;
  g.ldc = d;
  hipError_t e = gemm(s, g);
  if (e != hipSuccess) return e;
  GemmArgs gx = g;
  gx.K = d;
  gx.A = xt;
  gx.lda = d;
  gx.ta_bf16 = bf;
  gx.B = (const char *)W + (size_t)nblk * d * d * esize(dm);
  gx.beta = 1.f;
  return gemm(s, gx);
}

// eq. (2) for all history rows.
int encode_rows(hipStream_t s, const stca_dims *dm, const stca_ffn *f, int64_t rows, const void *X, void *Xt,
                const void *packed, const FfnWs &w) {
  if (dm->dtype == STCA_BF16) {
    HIP_TRY(encode_mfma(s, dm->d, dm->r, rows, X, dm->d, packed, Xt, dm->d, true, true, f->gamma, f->beta,
                        dm->ln_eps));
    return STCA_OK;
  }
  return ffn_generic(s, dm, f, rows, X, dm->d, false, Xt, dm->d, false, true, w);
}

// eqs. (13), (6) for one layer: o[T x d] (row stride ldo) from the encoded history and q.
int attend_layer(hipStream_t s, const stca_dims *dm, const stca_weights *w, int i, const stca_batch *b,
                 const AttnPlan &p, const void *Xt, const float *q, float *o, int64_t ldo, const AttendWs &aw,
                 stca_profiler *prof) {
  const int64_t T = b->total_T;
  if (T == 0) return STCA_OK;
  const int d = dm->d, h = dm->h, dh = d / h;
  const bool bf = dm->dtype == STCA_BF16;
  {
    Phase ph(prof, s, STCA_PHASE_UPROJ);
    // P = q W_Q  (T x d, into obar as scratch)
    GemmArgs g;
    g.M = (int)T;
    g.N = d;
    g.K = d;
    g.A = q;
    g.lda = d;
    g.B = w->WQ[i];
    g.ldb = d;
    g.tb_bf16 = bf;
    g.C = aw.obar;
    g.ldc = d;
    HIP_TRY(gemm(s, g));
    // U[:, j, :] = P[:, head j] W_K[:, head j]^T * log2(e) / sqrt(d_h)
    GemmArgs u;
    u.M = (int)T;
    u.N = d;
    u.K = dh;
    u.batch = h;
    u.A = aw.obar;
    u.lda = d;
    u.sA = dh;
    u.B = w->WK[i];
    u.ldb = d;
    u.sB = dh;
    u.tb_bf16 = bf;
    u.trans_b = true;
    u.C = aw.U;
    u.ldc = (int64_t)h * d;
    u.sC = d;
    u.tc_bf16 = bf;
    u.alpha = 1.4426950408889634f / sqrtf((float)dh);
    HIP_TRY(gemm(s, u));
    HIP_TRY(ph.end());
  }
  {
    Phase ph(prof, s, STCA_PHASE_ATTEND);
    HIP_TRY(attend_split(s, p, bf, b->hist_off, b->tgt_off, Xt, aw.U, aw.abar, aw.ab));
    HIP_TRY(ph.end());
  }
  if (p.max_part_rows > 0 || b->n_users > 0) {
    Phase ph(prof, s, STCA_PHASE_COMBINE);
    HIP_TRY(attend_combine(s, p, b->tgt_off, aw.abar, aw.ab));
    HIP_TRY(ph.end());
  }
  {
    Phase ph(prof, s, STCA_PHASE_PROJECT);
    // obar[:, head j] = abar[:, j, :] W_V[:, head j]
    GemmArgs v;
    v.M = (int)T;
    v.N = dh;
    v.K = d;
    v.batch = h;
    v.A = aw.abar;
    v.lda = (int64_t)h * d;
    v.sA = d;
    v.B = w->WV[i];
    v.ldb = d;
    v.sB = dh;
    v.tb_bf16 = bf;
    v.C = aw.obar;
    v.ldc = d;
    v.sC = dh;
    HIP_TRY(gemm(s, v));
    // o = obar W_O
    GemmArgs g;
    g.M = (int)T;
    g.N = d;
    g.K = d;
    g.A = aw.obar;
    g.lda = d;
    g.B = w->WO[i];
    g.ldb = d;
    g.tb_bf16 = bf;
    g.C = o;
    g.ldc = ldo;
    HIP_TRY(gemm(s, g));
    HIP_TRY(ph.end());
  }
  return STCA_OK;
}

struct ForwardWs {
  void *packed_hist[STCA_MAX_M] = {};
  void *packed_query[STCA_MAX_M] = {};
  void *Xt = nullptr;
  float *q = nullptr;
  float *c = nullptr;
  void *cb = nullptr;  // eq. (7) projection in bf16: the MFMA query FFN's input
  FfnWs ffn;
  AttendWs aw;
};

bool same_ffn(const stca_ffn &a, const stca_ffn &b) { return a.Wu == b.Wu && a.Wv == b.Wv && a.Wo == b.Wo; }

// All M history encodes in one launch (X read once, M encoded buffers) or one launch per layer,
// each followed by that layer's attention (one buffer).  Per layer, the attention then reads an X~
// the encode has just written, which a batch of moderate size finds in the 256 MB last-level cache;
// automatically, the single launch is used where one layer's X~ is far larger than that cache (and
// at d <= 256, where the kernel keeps a tile's rows on chip between layers); stca_dims can force
// either way.
bool fused_encode(const stca_dims *dm, const stca_batch *b) {
  if (dm->dtype != STCA_BF16 || dm->encode_layers == 1) return false;
  if (dm->encode_layers == 2) return true;
  return dm->M > 1 && dm->d <= 256 && b->total_L * dm->d * 2 > ((int64_t)1 << 30);
}

size_t carve_forward(void *base, const stca_dims *dm, const stca_batch *b, const AttnPlan &p, ForwardWs &w,
                     const stca_weights *wt) {
  Carver c(base);
  if (dm->dtype == STCA_BF16) {
    // History FFNs: every layer's fragments and LayerNorm parameters at one stride, for the
    // single multi-layer encode launch.
    const size_t ls = encode_layer_stride(dm->d, dm->r);
    char *hist = c.take<char>(ls * dm->M);
    for (int i = 0; i < dm->M; ++i) w.packed_hist[i] = hist ? hist + ls * i : nullptr;
    const size_t pb = encode_packed_bytes(dm->d, dm->r);
    for (int i = 0; i < dm->M; ++i) w.packed_query[i] = c.take<char>(pb);
    (void)wt;
  }
  const int n_xt = fused_encode(dm, b) ? dm->M : 1;
  w.Xt = c.take<char>((size_t)(b->total_L * dm->d) * esize(dm) * n_xt);
  w.q = c.take<float>((size_t)(b->total_T * dm->d));
  w.c = c.take<float>((size_t)(b->total_T * dm->d));
  if (dm->dtype == STCA_BF16) w.cb = c.take<char>((size_t)(b->total_T * dm->d) * 2);
  if (dm->dtype != STCA_BF16) carve_ffn(c, dm, std::max(b->total_T, b->total_L), w.ffn);
  carve_attend(c, dm, b, p, w.aw);
  return round_up(c.off, 256);
}

int forward_impl(const stca_dims *dm, const stca_weights *w, const stca_batch *b, const void *X, const void *xt,
                 float *Z, void *ws, size_t ws_bytes, void *stream, stca_profiler *prof) {
  int st;
  if ((st = check_dims(dm)) != STCA_OK) return st;
  if ((st = check_batch(b)) != STCA_OK) return st;
  if ((st = check_weights(dm, w)) != STCA_OK) return st;
  if (b->total_L > 0 && !X) return fail(STCA_E_ARG, "X is NULL");
  if (b->total_T > 0 && (!xt || !Z)) return fail(STCA_E_ARG, "xt or Z is NULL");
  if (!aligned16(X) || !aligned16(xt) || !aligned16(Z)) return fail(STCA_E_ALIGN, "X/xt/Z not 16-byte aligned");
  const AttnPlan p = make_plan(dm, b);
  ForwardWs fw;
  const size_t need = carve_forward(nullptr, dm, b, p, fw, w);
  if (!ws || ws_bytes < need)
    return fail(STCA_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes, need);
  if (!aligned16(ws)) return fail(STCA_E_ALIGN, "workspace not 16-byte aligned");
  carve_forward(ws, dm, b, p, fw, w);
  if (b->total_T == 0) return STCA_OK;  // nothing to produce

  hipStream_t s = (hipStream_t)stream;
  const int d = dm->d, M = dm->M;
  const bool bf = dm->dtype == STCA_BF16;

  if (bf) {
    Phase ph(prof, s, STCA_PHASE_PACK);
    for (int i = 0; i < M; ++i)
      HIP_TRY(encode_pack(s, d, dm->r, w->hist[i].Wu, w->hist[i].Wv, w->hist[i].Wo, fw.packed_hist[i],
                          w->hist[i].gamma, w->hist[i].beta));
    // Query FFNs (eqs. (3), (7)) run on the same MFMA kernel; they usually share the history
    // FFN's weights (reused), otherwise they are packed here.
    for (int i = 0; i < M; ++i) {
      void *found = nullptr;
      for (int j = 0; j < M && !found; ++j)
        if (same_ffn(w->hist[j], w->query[i])) found = fw.packed_hist[j];
      for (int j = 0; j < i && !found; ++j)
        if (same_ffn(w->query[j], w->query[i])) found = fw.packed_query[j];
      if (found) {
        fw.packed_query[i] = found;
        continue;
      }
      HIP_TRY(encode_pack(s, d, dm->r, w->query[i].Wu, w->query[i].Wv, w->query[i].Wo, fw.packed_query[i]));
    }
    HIP_TRY(ph.end());
  }
  HIP_TRY(build_worklist(s, p, b->hist_off, b->tgt_off, fw.aw.ab));

  {  // eq. (3): q(1) = LN(SwiGLUFFN(1)(x_t))
    Phase ph(prof, s, STCA_PHASE_QUERY);
    if (bf) {
      const stca_ffn &f = w->query[0];
      HIP_TRY(encode_mfma(s, d, dm->r, b->total_T, xt, d, fw.packed_query[0], fw.q, d, false, true, f.gamma, f.beta,
                          dm->ln_eps));
    } else if ((st = ffn_generic(s, dm, &w->query[0], b->total_T, xt, d, bf, fw.q, d, false, true, fw.ffn)) !=
               STCA_OK) {
      return st;
    }
    HIP_TRY(ph.end());
  }
  // eq. (2) for every layer: in one launch before the loop, or layer by layer inside it.
  const bool fused = fused_encode(dm, b);
  const size_t xt_layer = (size_t)(b->total_L * d) * esize(dm);
  if (fused) {
    Phase ph(prof, s, STCA_PHASE_ENCODE);
    const size_t ls = encode_layer_stride(d, dm->r), pb = encode_packed_bytes(d, dm->r);
    const float *ln0 = reinterpret_cast<const float *>((const char *)fw.packed_hist[0] + pb);
    const EncodeLayers lay{fw.packed_hist[0], (int64_t)ls, fw.Xt, b->total_L * d, ln0, ln0 + d,
                           (int64_t)(ls / sizeof(float)), M};
    HIP_TRY(encode_mfma_layers(s, d, dm->r, b->total_L, X, d, lay, d, true, true, dm->ln_eps));
    HIP_TRY(ph.end());
  }
  for (int i = 0; i < M; ++i) {
    const char *Xt_i = (const char *)fw.Xt + (fused ? xt_layer * i : 0);
    if (!fused) {
      Phase ph(prof, s, STCA_PHASE_ENCODE);
      if ((st = encode_rows(s, dm, &w->hist[i], b->total_L, X, fw.Xt, fw.packed_hist[i], fw.ffn)) != STCA_OK)
        return st;
      HIP_TRY(ph.end());
    }
    if ((st = attend_layer(s, dm, w, i, b, p, Xt_i, fw.q, Z + (size_t)i * d, (int64_t)M * d, fw.aw, prof)) !=
        STCA_OK)
      return st;
    if (i + 1 < M) {  // eq. (7): q(i+1) = SwiGLUFFN([o(1..i) || x_t] W_C) (+LN)
      Phase ph(prof, s, STCA_PHASE_QUERY);
      HIP_TRY(concat_project(s, dm, b->total_T, Z, (int64_t)M * d, i + 1, xt, w->WC[i + 1], fw.c));
      if (bf) {  // bf16 input of the MFMA FFN, fp32 output q
        const stca_ffn &f = w->query[i + 1];
        HIP_TRY(to_bf16(s, b->total_T * d, fw.c, fw.cb));
        HIP_TRY(encode_mfma(s, d, dm->r, b->total_T, fw.cb, d, fw.packed_query[i + 1], fw.q, d, false,
                            dm->query_ln != 0, f.gamma, f.beta, dm->ln_eps));
      } else if ((st = ffn_generic(s, dm, &w->query[i + 1], b->total_T, fw.c, d, false, fw.q, d, false,
                                   dm->query_ln != 0, fw.ffn)) != STCA_OK) {
        return st;
      }
      HIP_TRY(ph.end());
    }
  }
  return STCA_OK;
}

// ---- scratch of the allocation-free attention call (stca_attend_noalloc) -----------------------
// One fixed array per GPU, part of the library's code object: the runtime places it in each
// device's memory when it loads the library there, and it stays until the process ends.  In host
// code `scratch` names a host-side stand-in, not device memory: the device address is taken once
// per device with hipGetSymbolAddress, with that device current, and only that address is used.
constexpr size_t kNoallocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address (its first call on a device looks it up).
int noalloc_scratch(void **out) {
  int dev = 0;
  HIP_TRY(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(STCA_E_HIP, "device %d beyond the %d the library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    HIP_TRY(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)));
    if (!ptr) return fail(STCA_E_HIP, "hipGetSymbolAddress gave no address for the scratch array");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return STCA_OK;
}

}  // namespace stca_abi

// A recorded forward (stca_forward_graph_create): the HIP graph and its executable instance.
struct stca_graph {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
};

using namespace stca_abi;

// =============================================================================================
extern "C" {

int stca_encode_workspace_size(const stca_dims *dims, int64_t n_rows, size_t *bytes) {
  int st;
  if ((st = check_dims(dims)) != STCA_OK) return st;
  if (!bytes) return fail(STCA_E_ARG, "bytes is NULL");
  if (n_rows < 0) return fail(STCA_E_ARG, "n_rows < 0");
  Carver c(nullptr);
  if (dims->dtype == STCA_BF16) {
    c.take<char>(encode_packed_bytes(dims->d, dims->r));
  } else {
    FfnWs f;
    carve_ffn(c, dims, n_rows, f);
  }
  *bytes = round_up(c.off, 256);
  return STCA_OK;
}

int stca_attend_workspace_size(const stca_dims *dims, const stca_batch *batch, size_t *bytes) {
  int st;
  if ((st = check_dims(dims)) != STCA_OK) return st;
  if ((st = check_batch(batch)) != STCA_OK) return st;
  if (!bytes) return fail(STCA_E_ARG, "bytes is NULL");
  const AttnPlan p = make_plan(dims, batch);
  Carver c(nullptr);
  AttendWs aw;
  carve_attend(c, dims, batch, p, aw);
  *bytes = round_up(c.off, 256);
  return STCA_OK;
}

int stca_forward_workspace_size(const stca_dims *dims, const stca_batch *batch, size_t *bytes) {
  int st;
  if ((st = check_dims(dims)) != STCA_OK) return st;
  if ((st = check_batch(batch)) != STCA_OK) return st;
  if (!bytes) return fail(STCA_E_ARG, "bytes is NULL");
  const AttnPlan p = make_plan(dims, batch);
  ForwardWs fw;
  *bytes = carve_forward(nullptr, dims, batch, p, fw, nullptr);
  return STCA_OK;
}

int stca_encode(const stca_dims *dims, const stca_ffn *ffn, int64_t n_rows, const void *X, void *Xt,
                void *workspace, size_t workspace_bytes, void *stream) {
  int st;
  if ((st = check_dims(dims)) != STCA_OK) return st;
  if ((st = check_ffn(ffn, true, "encode")) != STCA_OK) return st;
  if (n_rows < 0) return fail(STCA_E_ARG, "n_rows < 0");
  if (n_rows > 0 && (!X || !Xt)) return fail(STCA_E_ARG, "X or Xt is NULL");
  if (!aligned16(X) || !aligned16(Xt)) return fail(STCA_E_ALIGN, "X/Xt not 16-byte aligned");
  size_t need = 0;
  stca_encode_workspace_size(dims, n_rows, &need);
  if (!workspace || workspace_bytes < need)
    return fail(STCA_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes, need);
  if (!aligned16(workspace)) return fail(STCA_E_ALIGN, "workspace not 16-byte aligned");
  if (n_rows == 0) return STCA_OK;
  hipStream_t s = (hipStream_t)stream;
  Carver c(workspace);
  if (dims->dtype == STCA_BF16) {
    void *packed = c.take<char>(encode_packed_bytes(dims->d, dims->r));
    HIP_TRY(encode_pack(s, dims->d, dims->r, ffn->Wu, ffn->Wv, ffn->Wo, packed));
    return encode_rows(s, dims, ffn, n_rows, X, Xt, packed, FfnWs{});
  }
  FfnWs f;
  carve_ffn(c, dims, n_rows, f);
  return encode_rows(s, dims, ffn, n_rows, X, Xt, nullptr, f);
}

int stca_attend(const stca_dims *dims, const stca_weights *w, int32_t layer, const stca_batch *batch,
                const void *Xt, const float *q, float *o, void *workspace, size_t workspace_bytes, void *stream) {
  int st;
  if ((st = check_dims(dims)) != STCA_OK) return st;
  if ((st = check_batch(batch)) != STCA_OK) return st;
  if (!w) return fail(STCA_E_ARG, "weights are NULL");
  if (layer < 0 || layer >= dims->M) return fail(STCA_E_ARG, "layer %d not in [0, M)", layer);
  if ((st = check_layer_weights(dims, w, layer)) != STCA_OK) return st;
  if (batch->total_L > 0 && !Xt) return fail(STCA_E_ARG, "Xt is NULL");
  if (batch->total_T > 0 && (!q || !o)) return fail(STCA_E_ARG, "q or o is NULL");
  if (!aligned16(Xt) || !aligned16(q) || !aligned16(o)) return fail(STCA_E_ALIGN, "Xt/q/o not 16-byte aligned");
  const AttnPlan p = make_plan(dims, batch);
  Carver c0(nullptr);
  AttendWs aw;
  carve_attend(c0, dims, batch, p, aw);
  const size_t need = round_up(c0.off, 256);
  if (!workspace || workspace_bytes < need)
    return fail(STCA_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes, need);
  if (!aligned16(workspace)) return fail(STCA_E_ALIGN, "workspace not 16-byte aligned");
  if (batch->total_T == 0) return STCA_OK;
  Carver c(workspace);
  carve_attend(c, dims, batch, p, aw);
  hipStream_t s = (hipStream_t)stream;
  HIP_TRY(build_worklist(s, p, batch->hist_off, batch->tgt_off, aw.ab));
  return attend_layer(s, dims, w, layer, batch, p, Xt, q, o, dims->d, aw, nullptr);
}

int stca_attend_noalloc(const stca_dims *dims, const stca_weights *w, int32_t layer, const stca_batch *batch,
                        const void *Xt, const float *q, float *o, void *stream) {
  size_t need = 0;
  int st = stca_attend_workspace_size(dims, batch, &need);
  if (st != STCA_OK) return st;
  if (need > kNoallocScratchBytes)
    return fail(STCA_E_WORKSPACE,
                "batch needs %zu bytes of scratch, more than the %zu of the allocation-free call; use stca_attend "
                "with a workspace",
                need, kNoallocScratchBytes);
  void *ptr = nullptr;
  if ((st = noalloc_scratch(&ptr)) != STCA_OK) return st;
  return stca_attend(dims, w, layer, batch, Xt, q, o, ptr, kNoallocScratchBytes, stream);
}

int stca_forward(const stca_dims *dims, const stca_weights *w, const stca_batch *batch, const void *X,
                 const void *xt, float *Z, void *workspace, size_t workspace_bytes, void *stream) {
  return forward_impl(dims, w, batch, X, xt, Z, workspace, workspace_bytes, stream, nullptr);
}

int stca_forward_profiled(const stca_dims *dims, const stca_weights *w, const stca_batch *batch, const void *X,
                          const void *xt, float *Z, void *workspace, size_t workspace_bytes, void *stream,
                          stca_profiler *prof) {
  return forward_impl(dims, w, batch, X, xt, Z, workspace, workspace_bytes, stream, prof);
}

int stca_predict_workspace_size(const stca_dims *dims, int64_t n_targets, size_t *bytes) {
  int st;
  if ((st = check_dims(dims)) != STCA_OK) return st;
  if (!bytes) return fail(STCA_E_ARG, "bytes is NULL");
  if (n_targets < 0) return fail(STCA_E_ARG, "n_targets < 0");
  Carver c(nullptr);
  c.take<float>((size_t)std::max<int64_t>(n_targets, 1) * dims->d);
  FfnWs f;
  carve_ffn(c, dims, n_targets, f);
  *bytes = round_up(c.off, 256);
  return STCA_OK;
}

int stca_predict(const stca_dims *dims, const void *WZ, const stca_ffn *ffn, int64_t n_targets, const float *Z,
                 const void *xt, float *z, void *workspace, size_t workspace_bytes, void *stream) {
  int st;
  if ((st = check_dims(dims)) != STCA_OK) return st;
  if ((st = check_ffn(ffn, false, "predict")) != STCA_OK) return st;
  if (!WZ) return fail(STCA_E_ARG, "W_Z is NULL");
  if (n_targets < 0) return fail(STCA_E_ARG, "n_targets < 0");
  if (n_targets > INT32_MAX) return fail(STCA_E_ARG, "n_targets = %lld exceeds 2^31 - 1", (long long)n_targets);
  if (n_targets > 0 && (!Z || !xt || !z)) return fail(STCA_E_ARG, "Z, xt or z is NULL");
  if (!aligned16(WZ) || !aligned16(Z) || !aligned16(xt) || !aligned16(z))
    return fail(STCA_E_ALIGN, "W_Z/Z/xt/z not 16-byte aligned");
  size_t need = 0;
  stca_predict_workspace_size(dims, n_targets, &need);
  if (!workspace || workspace_bytes < need)
    return fail(STCA_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes, need);
  if (!aligned16(workspace)) return fail(STCA_E_ALIGN, "workspace not 16-byte aligned");
  if (n_targets == 0) return STCA_OK;
  hipStream_t s = (hipStream_t)stream;
  Carver c(workspace);
  float *cbuf = c.take<float>((size_t)n_targets * dims->d);
  FfnWs f;
  carve_ffn(c, dims, n_targets, f);
  const int d = dims->d, M = dims->M;
  HIP_TRY(concat_project(s, dims, n_targets, Z, (int64_t)M * d, M, xt, WZ, cbuf));
  return ffn_generic(s, dims, ffn, n_targets, cbuf, d, false, z, d, false, false, f);
}

int stca_sl_beta(const stca_sl_params *p, double alpha, double *beta) {
  if (!p || !beta) return fail(STCA_E_ARG, "params or beta is NULL");
  if (!(p->L_min >= 1 && p->L_min < p->L_avg && p->L_avg < p->L_max))
    return fail(STCA_E_ARG, "need 1 <= L_min < L_avg < L_max (got %d, %d, %d)", p->L_min, p->L_avg, p->L_max);
  if (!(alpha > 0)) return fail(STCA_E_ARG, "alpha must be > 0");
  *beta = alpha * (double)(p->L_max - p->L_avg) / (double)(p->L_avg - p->L_min);
  return STCA_OK;
}

int stca_sl_plan(const stca_sl_params *p, int32_t n_users, const int64_t *full_len, const double *s,
                 const int32_t *order, int64_t *len, int64_t *hist_off) {
  double beta;
  int st;
  if ((st = stca_sl_beta(p, 1.0, &beta)) != STCA_OK) return st;
  if (p->L_infer < 1) return fail(STCA_E_ARG, "L_infer must be >= 1");
  if (n_users < 0) return fail(STCA_E_ARG, "n_users < 0");
  if (!hist_off) return fail(STCA_E_ARG, "hist_off is NULL");
  hist_off[0] = 0;
  if (n_users == 0) return STCA_OK;
  if (!full_len || !s || !order || !len) return fail(STCA_E_ARG, "full_len, s, order or len is NULL");
  std::vector<char> seen(n_users, 0);
  for (int32_t i = 0; i < n_users; ++i) {
    if (order[i] < 0 || order[i] >= n_users || seen[order[i]]) return fail(STCA_E_ARG, "order is not a permutation");
    seen[order[i]] = 1;
    if (!(s[i] >= 0.0 && s[i] <= 1.0)) return fail(STCA_E_ARG, "s[%d] = %g outside [0, 1]", i, s[i]);
    if (full_len[i] < 0) return fail(STCA_E_ARG, "full_len[%d] < 0", i);
  }
  // eq. (16), aligned to 8 (nearest, halves up) and clamped; capped by the available history.
  const int64_t lo = 8 * ((p->L_min + 7) / 8), hi = 8 * (p->L_max / 8);
  int64_t total = 0;
  for (int32_t u = 0; u < n_users; ++u) {
    const double raw = (double)p->L_min + s[u] * (double)(p->L_max - p->L_min);
    int64_t L = 8 * (int64_t)floor(raw / 8.0 + 0.5);
    L = std::min(std::max(L, lo), hi);
    L = std::min<int64_t>(L, std::min<int64_t>(full_len[u], p->L_infer));
    len[u] = L;
    total += L;
  }
  // Global length allocation: truncate in the given order until the budget is met exactly.
  int64_t excess = total - (int64_t)n_users * p->L_avg;
  for (int32_t i = 0; i < n_users && excess > 0; ++i) {
    const int32_t u = order[i];
    const int64_t cut = std::min<int64_t>(excess, std::max<int64_t>(len[u] - lo, 0));
    len[u] -= cut;
    excess -= cut;
  }
  for (int32_t u = 0; u < n_users; ++u) hist_off[u + 1] = hist_off[u] + len[u];
  return STCA_OK;
}

int stca_sl_pack(const stca_dims *dims, int32_t n_users, const int64_t *full_off, const int64_t *hist_off,
                 int64_t total, int64_t max_len, const void *X_full, void *X_packed, void *stream) {
  if (!dims) return fail(STCA_E_ARG, "dims is NULL");
  if (dims->dtype != STCA_F32 && dims->dtype != STCA_BF16) return fail(STCA_E_DIMS, "unknown dtype %d", dims->dtype);
  const int64_t row_bytes = (int64_t)dims->d * (dims->dtype == STCA_BF16 ? 2 : 4);
  if (dims->d < 1 || row_bytes % 16 != 0) return fail(STCA_E_DIMS, "d=%d: rows must be a multiple of 16 bytes", dims->d);
  if (n_users < 0 || total < 0 || max_len < 0) return fail(STCA_E_ARG, "n_users, total or max_len < 0");
  if (total > 0 && (n_users == 0 || max_len == 0)) return fail(STCA_E_ARG, "total > 0 with no users or max_len 0");
  if (max_len > total) return fail(STCA_E_ARG, "max_len %lld > total %lld", (long long)max_len, (long long)total);
  if ((int64_t)n_users > 65535) return fail(STCA_E_ARG, "n_users %d > 65535", n_users);
  if (total == 0) return STCA_OK;
  if (!full_off || !hist_off || !X_full || !X_packed) return fail(STCA_E_ARG, "NULL pointer");
  if (!aligned16(X_full) || !aligned16(X_packed) || ((uintptr_t)full_off % 8) || ((uintptr_t)hist_off % 8))
    return fail(STCA_E_ALIGN, "X buffers need 16-byte, offsets 8-byte alignment");
  HIP_TRY(sl_pack((hipStream_t)stream, n_users, full_off, hist_off, total, max_len, (int)(row_bytes / 16), X_full,
                  X_packed));
  return STCA_OK;
}

int stca_litm_plan(int32_t n_users, const int64_t *hist_off, const int64_t *item_id, int32_t T, int64_t *merged_off,
                   int64_t *group_off, int64_t *members, int64_t *n_groups) {
  if (n_users < 0) return fail(STCA_E_ARG, "n_users < 0");
  if (T < 0) return fail(STCA_E_ARG, "T < 0");
  if (!hist_off || !merged_off || !n_groups) return fail(STCA_E_ARG, "hist_off, merged_off or n_groups is NULL");
  if (hist_off[0] != 0) return fail(STCA_E_ARG, "hist_off[0] != 0");
  for (int32_t u = 0; u < n_users; ++u)
    if (hist_off[u + 1] < hist_off[u]) return fail(STCA_E_ARG, "hist_off decreases at user %d", u);
  const int64_t total = hist_off[n_users];
  merged_off[0] = 0;
  *n_groups = 0;
  if (total == 0) {
    for (int32_t u = 0; u < n_users; ++u) merged_off[u + 1] = 0;
    if (group_off) group_off[0] = 0;
    return STCA_OK;
  }
  if (!item_id || !group_off || !members) return fail(STCA_E_ARG, "item_id, group_off or members is NULL");
  // Scan in position order: token p joins the group of the latest earlier token of its user with
  // the same ID if that token is at most T positions back, else it opens a group (groups are
  // numbered in order of their first token).
  std::vector<int64_t> gid(total);
  std::unordered_map<int64_t, int64_t> last;
  int64_t ng = 0;
  for (int32_t u = 0; u < n_users; ++u) {
    last.clear();
    for (int64_t p = hist_off[u]; p < hist_off[u + 1]; ++p) {
      auto it = last.find(item_id[p]);
      if (it != last.end() && p - it->second <= T) {
        gid[p] = gid[it->second];
        it->second = p;
      } else {
        gid[p] = ng++;
        last[item_id[p]] = p;
      }
    }
    merged_off[u + 1] = ng;
  }
  // Members grouped by group, in position order within a group (counting sort).
  std::vector<int64_t> fill(ng + 1, 0);
  for (int64_t p = 0; p < total; ++p) ++fill[gid[p] + 1];
  for (int64_t g = 0; g < ng; ++g) fill[g + 1] += fill[g];
  for (int64_t g = 0; g <= ng; ++g) group_off[g] = fill[g];
  for (int64_t p = 0; p < total; ++p) members[fill[gid[p]]++] = p;
  *n_groups = ng;
  return STCA_OK;
}

int stca_litm_merge(const stca_dims *dims, int64_t n_rows, int64_t n_groups, const int64_t *group_off,
                    const int64_t *members, const void *X, void *X_merged, void *stream) {
  if (!dims) return fail(STCA_E_ARG, "dims is NULL");
  if (dims->dtype != STCA_F32 && dims->dtype != STCA_BF16) return fail(STCA_E_DIMS, "unknown dtype %d", dims->dtype);
  if (dims->d != 64 && dims->d != 128 && dims->d != 256 && dims->d != 512)
    return fail(STCA_E_DIMS, "d=%d not in {64, 128, 256, 512}", dims->d);
  if (n_rows < 0 || n_groups < 0 || n_groups > n_rows) return fail(STCA_E_ARG, "need 0 <= n_groups <= n_rows");
  if (n_groups > ((int64_t)1 << 33)) return fail(STCA_E_ARG, "n_groups too large for one launch");
  if (n_groups == 0) return STCA_OK;
  if (!group_off || !members || !X || !X_merged) return fail(STCA_E_ARG, "NULL pointer");
  if (!aligned16(X) || !aligned16(X_merged) || ((uintptr_t)group_off % 8) || ((uintptr_t)members % 8))
    return fail(STCA_E_ALIGN, "X buffers need 16-byte, index arrays 8-byte alignment");
  HIP_TRY(litm_merge((hipStream_t)stream, dims->dtype == STCA_BF16, dims->d, n_rows, n_groups, group_off, members, X,
                     X_merged));
  return STCA_OK;
}

int stca_forward_graph_create(const stca_dims *dims, const stca_weights *w, const stca_batch *batch, const void *X,
                              const void *xt, float *Z, void *workspace, size_t workspace_bytes, stca_graph **out) {
  if (!out) return fail(STCA_E_ARG, "out is NULL");
  *out = nullptr;
  int st;
  // Argument checks first, on a dry run that records nothing.
  if ((st = check_dims(dims)) != STCA_OK) return st;
  if ((st = check_batch(batch)) != STCA_OK) return st;
  if ((st = check_weights(dims, w)) != STCA_OK) return st;
  size_t need = 0;
  if ((st = stca_forward_workspace_size(dims, batch, &need)) != STCA_OK) return st;
  if (!workspace || workspace_bytes < need)
    return fail(STCA_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", workspace_bytes, need);
  if (batch->total_L > 0 && !X) return fail(STCA_E_ARG, "X is NULL");
  if (batch->total_T > 0 && (!xt || !Z)) return fail(STCA_E_ARG, "xt or Z is NULL");
  if (!aligned16(X) || !aligned16(xt) || !aligned16(Z) || !aligned16(workspace))
    return fail(STCA_E_ALIGN, "X/xt/Z/workspace not 16-byte aligned");
  // Capture on a stream of our own (default priority), then instantiate.
  hipStream_t cs = nullptr;
  HIP_TRY(hipStreamCreateWithFlags(&cs, hipStreamNonBlocking));
  hipGraph_t graph = nullptr;
  hipError_t e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
  if (e == hipSuccess) {
    st = forward_impl(dims, w, batch, X, xt, Z, workspace, workspace_bytes, cs, nullptr);
    const hipError_t e2 = hipStreamEndCapture(cs, &graph);
    if (st == STCA_OK && e2 != hipSuccess) e = e2;
  }
  hipStreamDestroy(cs);
  if (e != hipSuccess) {
    if (graph) hipGraphDestroy(graph);
    return fail(STCA_E_HIP, "graph capture failed: %s", hipGetErrorString(e));
  }
  if (st != STCA_OK) {
    if (graph) hipGraphDestroy(graph);
    return st;
  }
  hipGraphExec_t exec = nullptr;
  e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    hipGraphDestroy(graph);
    return fail(STCA_E_HIP, "hipGraphInstantiate failed: %s", hipGetErrorString(e));
  }
  *out = new stca_graph{graph, exec};
  return STCA_OK;
}

int stca_graph_launch(stca_graph *g, void *stream) {
  if (!g) return fail(STCA_E_ARG, "graph is NULL");
  HIP_TRY(hipGraphLaunch(g->exec, (hipStream_t)stream));
  return STCA_OK;
}

int stca_graph_destroy(stca_graph *g) {
  if (!g) return STCA_OK;
  if (g->exec) hipGraphExecDestroy(g->exec);
  if (g->graph) hipGraphDestroy(g->graph);
  delete g;
  return STCA_OK;
}

int stca_profiler_create(stca_profiler **out) {
  if (!out) return fail(STCA_E_ARG, "out is NULL");
  *out = new stca_profiler();
  return STCA_OK;
}

int stca_profiler_destroy(stca_profiler *p) {
  if (!p) return STCA_OK;
  for (hipEvent_t e : p->pool) hipEventDestroy(e);
  delete p;
  return STCA_OK;
}

int stca_profiler_reset(stca_profiler *p) {
  if (!p) return fail(STCA_E_ARG, "profiler is NULL");
  p->marks.clear();
  p->used = 0;
  return STCA_OK;
}

int stca_profiler_read(stca_profiler *p, stca_profile_report *out) {
  if (!p || !out) return fail(STCA_E_ARG, "profiler or report is NULL");
  memset(out, 0, sizeof *out);
  if (!p->marks.empty()) HIP_TRY(hipEventSynchronize(p->marks.back().b));
  for (const auto &m : p->marks) {
    float ms = 0.f;
    HIP_TRY(hipEventSynchronize(m.b));
    HIP_TRY(hipEventElapsedTime(&ms, m.a, m.b));
    out->ms[m.phase] += ms;
    out->launches[m.phase] += 1;
  }
  return STCA_OK;
}

int stca_validate_batch(const stca_batch *batch, int32_t *result, void *stream) {
  int st;
  if ((st = check_batch(batch)) != STCA_OK) return st;
  if (!result) return fail(STCA_E_ARG, "result is NULL");
  if (((uintptr_t)result & 3u) != 0) return fail(STCA_E_ALIGN, "result not 4-byte aligned");
  HIP_TRY(validate_batch((hipStream_t)stream, batch->n_users, batch->hist_off, batch->tgt_off, batch->total_L,
                         batch->total_T, batch->max_L, batch->max_T, result));
  return STCA_OK;
}

static_assert(kDbgAttendRange == STCA_DBG_ATTEND_RANGE && kDbgAttendFetch == STCA_DBG_ATTEND_FETCH &&
                  kDbgAttendOut == STCA_DBG_ATTEND_OUT && kDbgAttendPart == STCA_DBG_ATTEND_PART &&
                  kDbgCombinePart == STCA_DBG_COMBINE_PART && kDbgWorklist == STCA_DBG_WORKLIST &&
                  kDbgGemmPad == STCA_DBG_GEMM_PAD && kDbgSelfTest == (uint32_t)STCA_DBG_SELFTEST,
              "debug check bits match the header");

int stca_debug_flags(uint32_t *flags, int32_t *checks_enabled, int32_t clear) {
  if (!flags) return fail(STCA_E_ARG, "flags is NULL");
#ifdef STCA_DEBUG_BOUNDS
  if (checks_enabled) *checks_enabled = 1;
  HIP_TRY(hipDeviceSynchronize());
  uint32_t a = 0, g = 0;
  HIP_TRY(debug_flags_attend(&a, clear != 0));
  HIP_TRY(debug_flags_gemm(&g, clear != 0));
  *flags = a | g;
#else
  (void)clear;
  if (checks_enabled) *checks_enabled = 0;
  *flags = 0;
#endif
  return STCA_OK;
}

int stca_debug_selftest(void *stream) {
  HIP_TRY(debug_selftest((hipStream_t)stream));
  return STCA_OK;
}

const char *stca_status_string(int status) {
  switch (status) {
    case STCA_OK: return "ok";
    case STCA_E_ARG: return "invalid argument";
    case STCA_E_DIMS: return "unsupported dimensions";
    case STCA_E_WORKSPACE: return "workspace too small";
    case STCA_E_ALIGN: return "pointer not 16-byte aligned";
    case STCA_E_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char *stca_last_error(void) { return g_last_error.c_str(); }

const char *stca_version(void) { return "libstca 0.1 (gfx950)"; }

}  // extern "C"
