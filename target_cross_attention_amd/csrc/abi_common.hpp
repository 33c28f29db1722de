// Host-side helpers shared by the files of the C ABI layer (api.hip, api_backward.hip): error
// reporting, argument checks, workspace carving and per-phase event timing.
#pragma once

#include <stdarg.h>
#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/stca.h"
#include "internal.hpp"

// Event pairs recorded around the phases of profiled calls (opaque to callers).
struct stca_profiler {
  std::vector<hipEvent_t> pool;
  size_t used = 0;
  struct Mark {
    int phase;
    hipEvent_t a, b;
  };
  std::vector<Mark> marks;
};

namespace stca_abi {

using namespace stca;

// Detail of this thread's last failure (stca_last_error); fail() records it and returns `status`.
extern thread_local std::string g_last_error;
int fail(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

#define HIP_TRY(expr)                                                                         \
  do {                                                                                        \
    hipError_t e_ = (expr);                                                                   \
    if (e_ != hipSuccess) return fail(STCA_E_HIP, "%s failed: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int check_dims(const stca_dims *dm);
int check_batch(const stca_batch *b);
int check_ffn(const stca_ffn *f, bool need_ln, const char *what);
int check_layer_weights(const stca_dims *dm, const stca_weights *w, int i);
int check_weights(const stca_dims *dm, const stca_weights *w);

struct Carver {
  char *base;
  size_t off = 0;
  explicit Carver(void *b) : base((char *)b) {}
  template <typename T> T *take(size_t count) {
    off = round_up(off, 256);
    T *p = base ? (T *)(base + off) : nullptr;
    off += count * sizeof(T);
    return p;
  }
};

inline size_t esize(const stca_dims *dm) { return dm->dtype == STCA_BF16 ? 2 : 4; }
constexpr int64_t kFfnRows = 32768;  // row chunk of the generic (fp32) FFN path

struct FfnWs {
  float *A = nullptr, *G = nullptr;  // kFfnRows x rd each (generic path)
};

// One event pair around a phase of a profiled call (no-op without a profiler).
struct Phase {
  stca_profiler *p;
  hipStream_t s;
  int phase;
  hipEvent_t b = nullptr;
  hipError_t err = hipSuccess;
  Phase(stca_profiler *p_, hipStream_t s_, int ph) : p(p_), s(s_), phase(ph) {
    if (!p) return;
    hipEvent_t a = take(), e = take();
    if (!a || !e) {
      p = nullptr;
      return;
    }
    p->marks.push_back({phase, a, e});
    b = e;
    err = hipEventRecord(a, s);
  }
  hipEvent_t take() {
    if (p->used == p->pool.size()) {
      if (p->pool.size() >= 65536) return nullptr;
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) return nullptr;
      p->pool.push_back(e);
    }
    return p->pool[p->used++];
  }
  hipError_t end() {
    if (p && b) return hipEventRecord(b, s);
    return err;
  }
};

// c[T x d] = [Z blocks 1..nblk || x_t] W (eqs. (7), (9)), as two GEMMs over Z in place (api.hip).
hipError_t concat_project(hipStream_t s, const stca_dims *dm, int64_t T, const float *Z, int64_t ldz, int nblk,
                          const void *xt, const void *W, float *c);

}  // namespace stca_abi
