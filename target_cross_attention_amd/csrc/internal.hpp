// Internal (non-exported) interfaces between the C ABI layer and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include "stca.h"

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
  // true: fp32-output products take the matrix cores whenever their operands allow it, also with too
  // few tiles to fill the chip (split-K remainders, where the vector kernel's few tiles are slower)
  bool mfma_small = false;
};
hipError_t gemm(hipStream_t s, const GemmArgs &g);
// One product of a ragged batch: sizes, element offsets from the base pointers, leading dimensions.
struct RaggedDesc {
  int32_t M, N, K, pad;
  int64_t a_off, lda, b_off, ldb, c_off, ldc;
};
// bf16_mm: the fp32 operands are rounded to bf16 for the bf16 matrix cores (fp32 accumulation), the
// mixed-precision backward's form; otherwise fp32 matrix cores.
hipError_t gemm_ragged(hipStream_t s, const GemmArgs &g, const RaggedDesc *descs, int n, int64_t max_m,
                       int64_t max_n, bool bf16_mm = false);
hipError_t swiglu_gate_inplace(hipStream_t s, int64_t n, float *A, const float *G);
hipError_t layernorm_rows(hipStream_t s, int64_t rows, int d, const float *Y, int64_t ldy, void *out,
                          int64_t ldo, bool out_bf16, const float *gamma, const float *beta, float eps);
// dst[n] (bf16) = src[n] (fp32) rounded to nearest even; n a multiple of 4.
hipError_t to_bf16(hipStream_t s, int64_t n, const float *src, void *dst);

// ---- debug build (-DSTCA_DEBUG_BOUNDS): index-check words of the kernel files ------------------
enum : uint32_t {
  kDbgAttendRange = 1u << 0,     // a work item's history range outside [0, total_L]
  kDbgAttendFetch = 1u << 1,     // a history tile row outside the item's chunk
  kDbgAttendOut = 1u << 2,       // an output row past total_T h
  kDbgAttendPart = 1u << 3,      // a partial-state row past the workspace's partial rows
  kDbgCombinePart = 1u << 4,     // the combine reading partial rows past the workspace's
  kDbgWorklist = 1u << 5,        // a work item written past the list's capacity
  kDbgGemmPad = 1u << 6,         // a transposed operand's row chunk past its row stride
  kDbgSelfTest = 1u << 31,       // set on purpose by stca_debug_selftest
};
// Bits recorded by the kernels of one file since the last clear (0 in the ordinary build, where
// no device memory is touched).
hipError_t debug_flags_attend(uint32_t *flags, bool clear);
hipError_t debug_flags_gemm(uint32_t *flags, bool clear);
// Debug build: one kernel records kDbgSelfTest, to show the mechanism reports what it records.
hipError_t debug_selftest(hipStream_t s);

// ---- fused bf16 MFMA encode (encode_mfma.hip) -----------------------------------------------
// Re-layout of one FFN's W_u, W_v (d x rd) and W_o (rd x d) into MFMA fragment order.
size_t encode_packed_bytes(int d, int r);
hipError_t encode_pack(hipStream_t s, int d, int r, const void *Wu, const void *Wv, const void *Wo,
                       void *packed, const float *gamma = nullptr, const float *beta = nullptr);
// out[n x d] = LN(SwiGLUFFN(X)) (apply_ln) or SwiGLUFFN(X); X bf16 (row stride ldx);
// out bf16 or fp32 (row stride ldo).
hipError_t encode_mfma(hipStream_t s, int d, int r, int64_t n_rows, const void *X, int64_t ldx,
                       const void *packed, void *out, int64_t ldo, bool out_bf16, bool apply_ln,
                       const float *gamma, const float *beta, float eps);
// Several FFNs of the same shape over the same rows in one launch (the history encodes of all
// layers, eq. (2)): out_l = LN_l(SwiGLUFFN_l(X)) for l < n, each tile of X read from memory once.
// Layer l's packed weights, output and LayerNorm parameters sit at fixed strides from layer 0's.
struct EncodeLayers {
  const void *packed;
  int64_t packed_stride;  // bytes
  void *out;
  int64_t out_stride;     // elements
  const float *gamma, *beta;
  int64_t ln_stride;      // floats
  int n;
};
hipError_t encode_mfma_layers(hipStream_t s, int d, int r, int64_t n_rows, const void *X, int64_t ldx,
                              const EncodeLayers &layers, int64_t ldo, bool out_bf16, bool apply_ln, float eps);
// Bytes between consecutive layers' packed weights when each is followed by its LayerNorm
// parameters (gamma then beta, d floats each), as encode_pack writes them when given.
size_t encode_layer_stride(int d, int r);

// ---- ragged split-L attention (attend.hip) --------------------------------------------------
// Query rows one attention work item covers: 4 waves x 32 rows, or at d = 512 (where two waves
// split the output features of a 32-row block) 2 x 32 rows.
constexpr int attn_feature_halves(int d) { return d > 256 ? 2 : 1; }
constexpr int attn_rows_per_group(int d) { return 4 * 32 / attn_feature_halves(d); }

// Sizes the attention kernels check their indices against in the debug build.
struct AttnBounds {
  int64_t total_L, rows, part_rows;
};

struct WorkItem {
  int32_t user, chunk, group, n_chunks;
};

struct AttnPlan {
  int n_users = 0, h = 0, d = 0, chunk = 0;
  int64_t total_L = 0, total_T = 0;
  int64_t max_L = 0, max_T = 0;   // the batch's stated per-user bounds
  int64_t max_items = 0;      // grid bound
  int64_t max_part_rows = 0;  // partial-state rows bound
};

// Violations of the batch contract, as found on the device (the bits of stca_validate_batch; the
// work list adds kBatchOverflow when its own totals exceed the workspace bounds).
constexpr int kBatchBadStart = 1, kBatchBadEnd = 2, kBatchDecreasing = 4, kBatchOverMaxL = 8, kBatchOverMaxT = 16,
              kBatchEmptyHistory = 32, kBatchOverflow = 64;

// Offset checks.  The ragged kernels size their grids, work list and partial-state buffers from the
// host-side totals and bounds of the batch; offsets that disagree with them would make those
// kernels write out of bounds.  offsets_violation() gives the broken conditions of user u as a
// STCA_BATCH_* bit mask (0 = consistent).
__device__ __forceinline__ int offsets_violation(int u, int n_users, const int64_t *__restrict__ hoff,
                                                 const int64_t *__restrict__ toff, int64_t total_L, int64_t total_T,
                                                 int64_t max_L, int64_t max_T) {
  const int64_t h0 = hoff[u], h1 = hoff[u + 1], t0 = toff[u], t1 = toff[u + 1];
  int bad = 0;
  if (u == 0 && (h0 != 0 || t0 != 0)) bad |= kBatchBadStart;
  if (u == n_users - 1 && (h1 != total_L || t1 != total_T)) bad |= kBatchBadEnd;
  if (h1 < h0 || t1 < t0) bad |= kBatchDecreasing;
  if (h1 - h0 > max_L) bad |= kBatchOverMaxL;
  if (t1 - t0 > max_T) bad |= kBatchOverMaxT;
  if (h1 == h0 && t1 > t0) bad |= kBatchEmptyHistory;
  return bad;
}

struct AttnBuffers {
  WorkItem *items = nullptr;
  int32_t *n_items = nullptr;  // [0] items listed, [1] violation bits (0: the batch is consistent)
  int32_t *user_nchunks = nullptr;
  int64_t *part_base = nullptr;
  int32_t *tgt_user = nullptr;
  float *part_A = nullptr;   // max_part_rows x d
  float *part_ms = nullptr;  // max_part_rows x 2  (running max, sum)
};

hipError_t build_worklist(hipStream_t s, const AttnPlan &p, const int64_t *hist_off, const int64_t *tgt_off,
                          const AttnBuffers &b);
// *result = OR over users of the violated conditions (kBatch* bits), 0 for a consistent batch.
hipError_t validate_batch(hipStream_t s, int n_users, const int64_t *hist_off, const int64_t *tgt_off, int64_t total_L,
                          int64_t total_T, int64_t max_L, int64_t max_T, int32_t *result);
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

// ---- bf16 matrix-core GEMM with fused epilogues (gemm_bf16.hip), mixed-precision backward ------
enum { kEpiStore = 0, kEpiAcc = 1, kEpiSwigluFwd = 2, kEpiSwigluBwd = 3 };
struct NtEpilogue {
  float *C = nullptr;            // kEpiStore / kEpiAcc: fp32 output (row stride ldc, batch stride sC)
  int64_t ldc = 0, sC = 0;
  void *H = nullptr;             // kEpiSwigluFwd: H written (bf16, rows x rd, row stride ldh)
  void *U = nullptr, *G = nullptr;  // kEpiSwigluFwd: u, g written; kEpiSwigluBwd: read (same layout)
  int64_t ldh = 0;
  void *dUG = nullptr;           // kEpiSwigluBwd: [dU | dG] (bf16, rows x 2rd, row stride lddug)
  int64_t lddug = 0;
  int rd = 0;
};
// C = A[M x K] Bt[N x K]^T (bf16 operands, k-contiguous rows, lda/ldb multiples of 8, bases 16-byte
// aligned) through epilogue `epi`.  ksplit > 0: blockIdx.z = z takes k in [z ksplit, (z+1) ksplit)
// and writes C + z sC; otherwise batch z reads A + z sA, Bt + z sB and writes C + z sC.
hipError_t gemm_nt(hipStream_t s, int epi, int M, int N, int K, int ksplit, int batch, const void *A, int64_t lda,
                   int64_t sA, const void *Bt, int64_t ldb, int64_t sB, const NtEpilogue &ep);
// C = A[K x M]^T B[K x N] (bf16, row-major with m / n contiguous: M, N, lda, ldb multiples of 8,
// bases 16-byte aligned) through kEpiStore or kEpiAcc; ksplit and batches as for gemm_nt.
hipError_t gemm_tn(hipStream_t s, int epi, int M, int N, int K, int ksplit, int batch, const void *A, int64_t lda,
                   int64_t sA, const void *B, int64_t ldb, int64_t sB, const NtEpilogue &ep);
hipError_t bwd_weights(hipStream_t s, int d, int r, const void *Wu, const void *Wv, const void *Wo, void *uvt,
                       void *uvc, void *ot);
hipError_t sum_parts_strided(hipStream_t s, int rows, int cols, int nparts, const float *parts, int64_t ldp,
                             int64_t pstride, float *out, int64_t ldo, bool accumulate);
// LayerNorm derivative (mixed path) from the pre-LN rows Y (rows x d, fp32) and dout (rows x d): dY
// as bf16 row-major (rows x d), dgamma and dbeta accumulated through per-block partial sums
// (2 min(ceil(rows / 64), 256) d floats of parts).
hipError_t ln_bwd_bf16(hipStream_t s, int64_t rows, int d, const float *dout, const float *Y, const float *gamma,
                       float eps, void *dY, float *dgamma, float *dbeta, float *parts);

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
                       int64_t total_L, int64_t total_T, int64_t max_L, int64_t max_T, int64_t max_scores,
                       RaggedDesc *descs);
hipError_t ragged_rows(hipStream_t s, int mode, int64_t rows, int h, int n_users, const int64_t *tgt_off,
                       const RaggedDesc *sdesc, float *S, float *S2, float scale, float *lse, const float *D);

}  // namespace stca
