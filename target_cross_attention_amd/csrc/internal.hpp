// Internal (non-exported) interfaces between the C ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace stca {

// ---- generic fp32-accumulating kernels (generic.hip) ----------------------------------------
struct GemmArgs {
  int M = 0, N = 0, K = 0, batch = 1;
  const void *A = nullptr;
  int64_t lda = 0, sA = 0;
  bool ta_bf16 = false;
  const void *B = nullptr;
  int64_t ldb = 0, sB = 0;
  bool tb_bf16 = false, trans_b = false, trans_a = false;
  void *C = nullptr;
  int64_t ldc = 0, sC = 0;
  bool tc_bf16 = false;
  float alpha = 1.f, beta = 0.f;
};
hipError_t gemm(hipStream_t s, const GemmArgs &g);
// One product of a ragged batch: sizes, element offsets from the base pointers, leading dimensions.
struct RaggedDesc {
  int32_t M, N, K, pad;
  int64_t a_off, lda, b_off, ldb, c_off, ldc;
};
hipError_t gemm_ragged(hipStream_t s, const GemmArgs &g, const RaggedDesc *descs, int n, int64_t max_m,
                       int64_t max_n);
hipError_t swiglu_gate_inplace(hipStream_t s, int64_t n, float *A, const float *G);
// C[M x N] (fp32) = A[M x K] Bt[N x K]^T, A and Bt bf16 (exact products, fp32 accumulation) on bf16
// matrix cores; K, lda, ldb multiples of 8, bases 16-byte aligned.
hipError_t gemm_bf16_nt(hipStream_t s, int M, int N, int K, const void *A, int64_t lda, const void *Bt, int64_t ldb,
                        float *C, int64_t ldc);
// out (cols x rows) = in (rows x cols)^T, bf16.
hipError_t transpose_bf16(hipStream_t s, int rows, int cols, const void *in, void *out);
hipError_t layernorm_rows(hipStream_t s, int64_t rows, int d, const float *Y, int64_t ldy, void *out,
                          int64_t ldo, bool out_bf16, const float *gamma, const float *beta, float eps);
// dst[n] (bf16) = src[n] (fp32) rounded to nearest even; n a multiple of 4.
hipError_t to_bf16(hipStream_t s, int64_t n, const float *src, void *dst);

// ---- fused bf16 MFMA encode (encode_mfma.hip) -----------------------------------------------
// Re-layout of one FFN's W_u, W_v (d x rd) and W_o (rd x d) into MFMA fragment order.
size_t encode_packed_bytes(int d, int r);
hipError_t encode_pack(hipStream_t s, int d, int r, const void *Wu, const void *Wv, const void *Wo,
                       void *packed);
// out[n x d] = LN(SwiGLUFFN(X)) (apply_ln) or SwiGLUFFN(X); X bf16 (row stride ldx);
// out bf16 or fp32 (row stride ldo).
hipError_t encode_mfma(hipStream_t s, int d, int r, int64_t n_rows, const void *X, int64_t ldx,
                       const void *packed, void *out, int64_t ldo, bool out_bf16, bool apply_ln,
                       const float *gamma, const float *beta, float eps);

// ---- ragged split-L attention (attend.hip) --------------------------------------------------
// Query rows one attention work item covers: 4 waves x 32 rows, or at d = 512 (where two waves
// split the output features of a 32-row block) 2 x 32 rows.
constexpr int attn_feature_halves(int d) { return d > 256 ? 2 : 1; }
constexpr int attn_rows_per_group(int d) { return 4 * 32 / attn_feature_halves(d); }

struct WorkItem {
  int32_t user, chunk, group, n_chunks;
};

struct AttnPlan {
  int n_users = 0, h = 0, d = 0, chunk = 0;
  int64_t total_L = 0, total_T = 0;
  int64_t max_items = 0;      // grid bound
  int64_t max_part_rows = 0;  // partial-state rows bound
};

struct AttnBuffers {
  WorkItem *items = nullptr;
  int32_t *n_items = nullptr;
  int32_t *user_nchunks = nullptr;
  int64_t *part_base = nullptr;
  int32_t *tgt_user = nullptr;
  float *part_A = nullptr;   // max_part_rows x d
  float *part_ms = nullptr;  // max_part_rows x 2  (running max, sum)
};

hipError_t build_worklist(hipStream_t s, const AttnPlan &p, const int64_t *hist_off, const int64_t *tgt_off,
                          const AttnBuffers &b);
// abar[T*h x d] (fp32): attention-weighted history per (target, head), eq. (13); U (T*h x d) holds
// u pre-scaled by log2(e)/sqrt(d_h).  Xt and U are bf16 (MFMA path) or fp32 (debug path).
hipError_t attend_split(hipStream_t s, const AttnPlan &p, bool bf16_path, const int64_t *hist_off,
                        const int64_t *tgt_off, const void *Xt, const void *U, float *abar,
                        const AttnBuffers &b);
hipError_t attend_combine(hipStream_t s, const AttnPlan &p, const int64_t *tgt_off, float *abar,
                          const AttnBuffers &b);

// ---- stochastic-length batches (sl.hip) -------------------------------------------------------
// X_packed (rows of row16 16-byte chunks) <- the temporal suffix rows of every user of X_full;
// max_len bounds every user's packed length.
// Local same-ID token merging: merged row g = sum of rows members[group_off[g] .. group_off[g+1]).
hipError_t litm_merge(hipStream_t s, bool bf16_rows, int d, int64_t n_rows, int64_t n_groups,
                      const int64_t *group_off, const int64_t *members, const void *X, void *out);
hipError_t sl_pack(hipStream_t s, int n_users, const int64_t *full_off, const int64_t *hist_off, int64_t total,
                   int64_t max_len, int row16, const void *X_full, void *X_packed);

// ---- backward pieces (backward.hip); all fp32 ------------------------------------------------
hipError_t fill_f32(hipStream_t s, int64_t n, float *y, float v);
// out[i] (+)= sum over k of parts[k n + i], in k order (deterministic split-K reduction).
hipError_t sum_parts(hipStream_t s, int64_t n, int nparts, const float *parts, float *out, bool accumulate);
// The same over a rows x cols block: parts are contiguous blocks, out has row stride ldo.
hipError_t sum_parts2d(hipStream_t s, int64_t rows, int cols, int nparts, const float *parts, float *out,
                       int64_t ldo, bool accumulate);
hipError_t swiglu_fwd(hipStream_t s, int64_t n, const float *A, const float *G, float *H);
hipError_t swiglu_bwd(hipStream_t s, int64_t n, const float *dH, const float *A, const float *G, float *dA,
                      float *dG);
// LayerNorm derivative from the pre-LN rows Y (d <= 512): dY (rows x d) written; dgamma and dbeta
// (d each) accumulated through per-block partial sums in parts (2 max_blocks x d floats), added in
// block order.
hipError_t ln_bwd(hipStream_t s, int64_t rows, int d, const float *dout, int64_t ldd, const float *Y, int64_t ldy,
                  const float *gamma, float eps, float *dY, float *dgamma, float *dbeta, float *parts,
                  int max_blocks);
hipError_t rowdot(hipStream_t s, int64_t rows, int d, const float *A, const float *B, float *out);
hipError_t copy_rows(hipStream_t s, int64_t rows, int d, const float *x, int64_t ldx, float *y, int64_t ldy);
// Attention over each user's history as ragged products (see backward.hip): descriptors of the three
// product shapes (3 n_users entries), and the row passes over the users' score matrices
// (mode 0: softmax with lse out, 1: softmax with lse in, 2: dS = alpha (dA - D) into S2).
hipError_t ragged_plan(hipStream_t s, int n_users, const int64_t *hist_off, const int64_t *tgt_off, int h, int d,
                       RaggedDesc *descs);
hipError_t ragged_rows(hipStream_t s, int mode, int64_t rows, int h, int n_users, const int64_t *tgt_off,
                       const RaggedDesc *sdesc, float *S, float *S2, float scale, float *lse, const float *D);

}  // namespace stca
