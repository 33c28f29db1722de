// Local same-ID token merging (LITM, "TM20K：老师读全文，学生读缩写", notes page, section 4.2.1):
// the device half.  The grouping is integer work done on the host (stca_litm_plan, as the page
// places it before the embedding lookup); this kernel forms each merged token as the sum of its
// members' rows.
#include "device_common.hpp"
#include "internal.hpp"

namespace stca {

// A wave merges G consecutive groups.  Rows move in 16-byte chunks: a row of ROW16 chunks is
// spread over LR = min(ROW16, 64) lanes (CPL = ROW16 / LR chunks each), so one load instruction
// covers RW = 64 / LR whole rows with consecutive lanes on consecutive bytes.  The groups'
// offsets and (when there are at most 64 of them) their member indices are fetched with one
// lane-parallel load each, and the first member row of every group is loaded before any is
// used, so all G row loads are in flight together; further members (repeats) follow.  Sums run
// in fp32 in member order and are rounded once to the storage type.  Indices outside the arrays
// are skipped (caller contract), never dereferenced.
constexpr int kMergeGroups = 16;

template <typename T, int ROW16>
__global__ __launch_bounds__(256) void litm_merge_kernel(int64_t n_rows, int64_t n_groups,
                                                         const int64_t *__restrict__ group_off,
                                                         const int64_t *__restrict__ members,
                                                         const u32x4 *__restrict__ X, u32x4 *__restrict__ out) {
  constexpr int G = kMergeGroups;
  constexpr int LR = ROW16 >= 64 ? 64 : ROW16, RW = 64 / LR, CPL = ROW16 / LR, EC = 16 / sizeof(T);
  constexpr int NP = G / RW;                         // load rounds per wave
  static_assert(G % RW == 0, "groups split evenly over the rows of a load");
  const int lane = threadIdx.x & 63, r = lane / LR, c = lane % LR;
  const int64_t g0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * G;
  if (g0 >= n_groups) return;
  const int ng = n_groups - g0 < G ? (int)(n_groups - g0) : G;
  auto clampj = [&](int64_t j) { return j < 0 ? (int64_t)0 : (j > n_rows ? n_rows : j); };
  const int64_t myoff = lane <= ng ? clampj(group_off[g0 + lane]) : 0;
  const int64_t J0 = __shfl(myoff, 0, 64), J1 = __shfl(myoff, ng, 64);
  const bool fast = J1 - J0 <= 64;
  const int64_t mym = (fast && J0 + lane < J1) ? members[J0 + lane] : -1;
  typedef u32x4 Chunks[CPL];
  auto load_row = [&](int64_t m, Chunks &x) {
#pragma unroll
    for (int q = 0; q < CPL; ++q) x[q] = (m >= 0 && m < n_rows) ? X[m * ROW16 + c + LR * q] : u32x4{};
  };
  Chunks first[NP];
  int64_t jb0[NP], jb1[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int k = p * RW + r;
    jb0[p] = __shfl(myoff, k < ng ? k : ng, 64);
    jb1[p] = __shfl(myoff, k + 1 < ng ? k + 1 : ng, 64);
    const int64_t rel = jb0[p] - J0;
    const int64_t m_fast = __shfl(mym, (int)(rel >= 0 && rel < 64 ? rel : 0), 64);
    const int64_t m = jb0[p] < jb1[p] ? (fast ? m_fast : members[jb0[p]]) : -1;
    load_row(k < ng ? m : -1, first[p]);
  }
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int k = p * RW + r;
    if (k >= ng) continue;
    float acc[CPL][EC];
#pragma unroll
    for (int q = 0; q < CPL; ++q) {
      const T *v = reinterpret_cast<const T *>(&first[p][q]);
#pragma unroll
      for (int e = 0; e < EC; ++e) acc[q][e] = elem<T>::load(v + e);
    }
    for (int64_t j = jb0[p] + 1; j < jb1[p]; ++j) {  // repeats: rare, read their index directly
      Chunks x;
      load_row(members[j], x);
#pragma unroll
      for (int q = 0; q < CPL; ++q) {
        const T *v = reinterpret_cast<const T *>(&x[q]);
#pragma unroll
        for (int e = 0; e < EC; ++e) acc[q][e] += elem<T>::load(v + e);
      }
    }
#pragma unroll
    for (int q = 0; q < CPL; ++q) {
      u32x4 y;
      T *w = reinterpret_cast<T *>(&y);
#pragma unroll
      for (int e = 0; e < EC; ++e) elem<T>::store(w + e, acc[q][e]);
      out[(g0 + k) * ROW16 + c + LR * q] = y;
    }
  }
}

template <typename T>
static hipError_t litm_merge_t(hipStream_t s, int d, int64_t n_rows, int64_t n_groups, const int64_t *group_off,
                               const int64_t *members, const void *X, void *out) {
  const dim3 grid((unsigned)((n_groups + 4 * kMergeGroups - 1) / (4 * kMergeGroups))), block(256);
  const u32x4 *x = (const u32x4 *)X;
  u32x4 *o = (u32x4 *)out;
  switch (d * (int)sizeof(T) / 16) {
    case 8: hipLaunchKernelGGL((litm_merge_kernel<T, 8>), grid, block, 0, s, n_rows, n_groups, group_off, members, x, o); break;
    case 16: hipLaunchKernelGGL((litm_merge_kernel<T, 16>), grid, block, 0, s, n_rows, n_groups, group_off, members, x, o); break;
    case 32: hipLaunchKernelGGL((litm_merge_kernel<T, 32>), grid, block, 0, s, n_rows, n_groups, group_off, members, x, o); break;
    case 64: hipLaunchKernelGGL((litm_merge_kernel<T, 64>), grid, block, 0, s, n_rows, n_groups, group_off, members, x, o); break;
    case 128: hipLaunchKernelGGL((litm_merge_kernel<T, 128>), grid, block, 0, s, n_rows, n_groups, group_off, members, x, o); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t litm_merge(hipStream_t s, bool bf16_rows, int d, int64_t n_rows, int64_t n_groups,
                      const int64_t *group_off, const int64_t *members, const void *X, void *out) {
  if (n_groups <= 0) return hipSuccess;
  return bf16_rows ? litm_merge_t<bf16>(s, d, n_rows, n_groups, group_off, members, X, out)
                   : litm_merge_t<float>(s, d, n_rows, n_groups, group_off, members, X, out);
}

}  // namespace stca
