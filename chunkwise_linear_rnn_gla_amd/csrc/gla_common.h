// gla_common.h -- device helpers shared by the GLA kernels (gfx950 only).
//
// MFMA conventions used everywhere (16x16 output tiles, wave64):
//   A (16 x K)  : lane l supplies A[l % 16][(l / 16) * KPL + e], e < KPL
//   B (K x 16)  : lane l supplies B[(l / 16) * KPL + e][l % 16]
//   D (16 x 16) : lane l holds    D[(l / 16) * 4 + r][l % 16],  r < 4
// bf16 operands use v_mfma_f32_16x16x32_bf16 (K = 32, KPL = 8); fp32 operands
// use v_mfma_f32_16x16x4_f32 (K = 4, KPL = 1).  Accumulation is always fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gla {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int kWave = 64;
constexpr int kThreads = 256;  // every kernel here runs 4 waves per workgroup

template <typename T> struct Mma;

template <> struct Mma<bf16> {
  static constexpr int K = 32;
  static constexpr int KPL = 8;
  typedef bf16x8 frag;
  __device__ static inline floatx4 run(frag a, frag b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mma<float> {
  static constexpr int K = 4;
  static constexpr int KPL = 1;
  typedef float frag;
  __device__ static inline floatx4 run(frag a, frag b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

__device__ inline float to_f32(float x) { return x; }
__device__ inline float to_f32(bf16 x) { return static_cast<float>(x); }

template <typename T> __device__ inline T from_f32(float x);
template <> __device__ inline float from_f32<float>(float x) { return x; }
template <> __device__ inline bf16 from_f32<bf16>(float x) { return static_cast<bf16>(x); }

// Load a fragment of KPL contiguous elements (16-byte aligned for bf16).
template <typename T>
__device__ inline typename Mma<T>::frag load_frag(const T* p);
template <> __device__ inline bf16x8 load_frag<bf16>(const bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
template <> __device__ inline float load_frag<float>(const float* p) { return *p; }

// Fragment of KPL contiguous elements computed as x[e] * scale[e] in fp32 and
// rounded once to T.  x is T, scale is fp32 (both contiguous).
template <typename T>
__device__ inline typename Mma<T>::frag scaled_frag(const T* x, const float* s);
template <> __device__ inline bf16x8 scaled_frag<bf16>(const bf16* x, const float* s) {
  bf16x8 xv = *reinterpret_cast<const bf16x8*>(x);
  f32x4 s0 = *reinterpret_cast<const f32x4*>(s);
  f32x4 s1 = *reinterpret_cast<const f32x4*>(s + 4);
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = static_cast<bf16>(static_cast<float>(xv[e]) * s0[e]);
    r[e + 4] = static_cast<bf16>(static_cast<float>(xv[e + 4]) * s1[e]);
  }
  return r;
}
template <> __device__ inline float scaled_frag<float>(const float* x, const float* s) {
  return x[0] * s[0];
}
// The same for bf16 operands from fp32 values x (rounded once after scaling).
__device__ inline bf16x8 scaled_frag_from_f32(const float* x, const float* s) {
  const f32x4 x0 = *reinterpret_cast<const f32x4*>(x);
  const f32x4 x1 = *reinterpret_cast<const f32x4*>(x + 4);
  const f32x4 s0 = *reinterpret_cast<const f32x4*>(s);
  const f32x4 s1 = *reinterpret_cast<const f32x4*>(s + 4);
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = static_cast<bf16>(x0[e] * s0[e]);
    r[e + 4] = static_cast<bf16>(x1[e] * s1[e]);
  }
  return r;
}

__device__ inline floatx4 zero4() {
  floatx4 z = {0.f, 0.f, 0.f, 0.f};
  return z;
}

__device__ inline float fast_exp(float x) { return __expf(x); }

// exp for factors of a given I/O type: the fp32 path keeps full accuracy
// (expf); the bf16 path uses the hardware exp2 based __expf, whose relative
// error is far below bf16 rounding for the arguments that occur.
template <typename T> __device__ inline float gexp(float x);
template <> __device__ inline float gexp<float>(float x) { return expf(x); }
template <> __device__ inline float gexp<bf16>(float x) { return __expf(x); }

// Workgroup barrier for LDS hand-offs: waits for this wave's LDS (and scalar
// memory) operations, then for every wave.  Unlike __syncthreads(), whose
// release fence also waits for the wave's outstanding global stores, it does
// not make global stores visible; use it only where the data handed over
// lives in LDS (or was waited for explicitly, as LDS-DMA copies are).
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ds_read_b64_tr_b16: within each 16-lane group, lane 4 a + b receives
// element b of the 8-byte chunks addressed by lanes a, a + 4, a + 8, a + 12.
typedef short v4s16 __attribute__((ext_vector_type(4)));
__device__ inline bf16x4 ds_read_tr(const bf16* p) {
  const v4s16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s16*)(const_cast<bf16*>(p)));
  bf16x4 o;
  __builtin_memcpy(&o, &r, 8);
  return o;
}
__device__ inline bf16x8 join8(bf16x4 a, bf16x4 b) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) { r[e] = a[e]; r[e + 4] = b[e]; }
  return r;
}
// The 16x16x32 bf16 MFMA operand of lane (g, n) over K: rows k0 + 8 g .. + 7
// of column c0 + n of a row-major LDS array (leading dimension ld elements,
// rows 8-byte aligned), with two transposed reads.
__device__ inline bf16x8 col_frag_tr(const bf16* x, int ld, int k0, int c0, int l) {
  const int n = l & 15, g = l >> 4;
  const bf16* p = x + (k0 + 8 * g + (n >> 2)) * ld + c0 + 4 * (n & 3);
  return join8(ds_read_tr(p), ds_read_tr(p + 4 * ld));
}

__device__ inline int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ inline int wave_id() { return threadIdx.x / kWave; }

}  // namespace gla
