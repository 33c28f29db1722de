// Device-side helpers shared by the libstca HIP kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace stca {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

#define STCA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;

// ---- scalar conversions ------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}
// Round-to-nearest-even fp32 -> bf16 (the hardware conversion on gfx950).
__device__ __forceinline__ bf16 f32_to_bf16(float f) { return (bf16)f; }
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (bf16)f);
}

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
__device__ __forceinline__ bf16x2 bf16x2_of(float a, float b) { return bf16x2{(bf16)a, (bf16)b}; }

template <typename T> struct elem;
template <> struct elem<float> {
  __device__ __forceinline__ static float load(const float *p) { return *p; }
  __device__ __forceinline__ static void store(float *p, float v) { *p = v; }
};
template <> struct elem<bf16> {
  __device__ __forceinline__ static float load(const bf16 *p) {
    return bf16_bits_to_f32(*reinterpret_cast<const uint16_t *>(p));
  }
  __device__ __forceinline__ static void store(bf16 *p, float v) { *p = f32_to_bf16(v); }
};

template <typename T> __device__ __forceinline__ float ld(const T *p) { return elem<T>::load(p); }
template <typename T> __device__ __forceinline__ void st(T *p, float v) { elem<T>::store(p, v); }

// ---- math --------------------------------------------------------------------------------
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// a * SiLU(g) = a * g / (1 + e^-g), with e^-g = 2^(-g log2 e).  exp2 of a large positive
// argument gives +inf and rcp(+inf) = 0, so very negative g yields -0 / 0 as it should.
__device__ __forceinline__ float swiglu_gate(float a, float g) {
  return a * g * fast_rcp(1.0f + fast_exp2(-g * kLog2e));
}

// ---- index checks of the debug build (-DSTCA_DEBUG_BOUNDS) -------------------------------------
// A failed check sets bit `code` of a per-file device word with a vector atomic instead of faulting,
// so a kernel always runs to its normal end; the library's stca_debug_flags reads and clears the
// words.  In the ordinary build the checks compile to nothing.
#ifdef STCA_DEBUG_BOUNDS
#define STCA_DEBUG_WORD static __device__ unsigned int stca_dbg_word;
#define STCA_CHECK(cond, code)                                           \
  do {                                                                   \
    if (!(cond)) atomicOr(&stca_dbg_word, (unsigned int)(code));         \
  } while (0)
#else
#define STCA_DEBUG_WORD
#define STCA_CHECK(cond, code) \
  do {                         \
  } while (0)
#endif

// ---- wave (64-lane) reductions -------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// Reductions across the two 32-lane halves of a wave (lane l with lane l ^ 32).
__device__ __forceinline__ float half_sum(float v) { return v + __shfl_xor(v, 32, 64); }
__device__ __forceinline__ float half_max(float v) { return fmaxf(v, __shfl_xor(v, 32, 64)); }

// ---- MFMA ----------------------------------------------------------------------------------
// v_mfma_f32_32x32x16_bf16: D[32x32] += A[32x16] B[16x32].
//   A: lane l holds row (l & 31), 8 k-slots of group (l >> 5).
//   B: lane l holds column (l & 31), 8 k-slots of group (l >> 5).
//   D: lane l holds column (l & 31); register i holds row 8*(i>>2) + 4*(l>>5) + (i&3).
// The k index behind a (group, slot) pair is the same for A and B, so any assignment of
// logical k to (group, slot) gives the right product as long as A and B use the same one.
__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// ---- global -> LDS staging and workgroup barriers -------------------------------------------
// Raw buffer resource over [base, base + bytes): loads at offsets >= bytes return zeros.  Word 3
// is the raw (untyped) buffer format of gfx9-family parts.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}
// 16 bytes per lane from the buffer (byte offset voff + soff) straight into LDS: lane i's bytes
// land at lds + 16 i, lds being wave-uniform.  The MUBUF form is used rather than the FLAT
// global form: the compiler treats a pending FLAT access as possibly either kind of memory and
// then drains every LDS read to zero outstanding, which defeats fragment prefetching.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, STCA_LDS void *lds, uint32_t voff,
                                           uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, voff, soff, 0, 0);
}
// Workgroup barrier after waiting for all but VM of this wave's vector-memory loads and for all
// of its LDS operations.  Unlike __syncthreads() it carries no release fence, which would wait
// for every outstanding LDS-bound load, including those meant to stay in flight across it.
template <int VM> __device__ __forceinline__ void barrier_vm() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(VM) : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Workgroup barrier that waits only for this wave's LDS operations: vector-memory loads (for
// instance direct-to-LDS staging meant for a later phase) may stay in flight across it.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace stca
