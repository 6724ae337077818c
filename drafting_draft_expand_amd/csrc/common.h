// Device-side helpers shared by the gfx950 kernels of the parallel-draft step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "internal.h"

namespace pe {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// f(std::integral_constant<int, i>) for i = 0 .. N-1, unrolled: register
// arrays indexed by i stay in registers.
template <typename F, size_t... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::index_sequence<I...>) {
  (f(std::integral_constant<int, static_cast<int>(I)>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_index_sequence<N>{});
}

// bfloat16 is carried as raw uint16 bit patterns.
typedef uint16_t bf16_t;

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bfloat16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>(0x7fc0);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

// op(v[l], v[l ^ 16]) and op(v[l], v[l ^ 32]) across a wave with the gfx950
// lane-swap instructions (register-only, no LDS round trip): swapping a copy
// of v with itself leaves one result holding rows 0,0,2,2 (halves 0,0) and the
// other rows 1,1,3,3 (halves 1,1) of 16 (32) lanes.
__device__ __forceinline__ float xor16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Two floats -> two bfloat16 packed in one word (lo in bits 0..15), round to
// nearest even, with the gfx950 packed conversion instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Element traits: float (fp32 models) or bf16_t (bf16 models).
template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kVec = 4;  // elements per 16-byte vector
  __device__ static __forceinline__ float load(const float* p) { return *p; }
  __device__ static __forceinline__ float to_f32(float v) { return v; }
  __device__ static __forceinline__ float from_f32(float v) { return v; }
};
template <> struct Elem<bf16_t> {
  static constexpr int kVec = 8;
  __device__ static __forceinline__ float load(const bf16_t* p) { return bf16_to_f32(*p); }
  __device__ static __forceinline__ float to_f32(bf16_t v) { return bf16_to_f32(v); }
  __device__ static __forceinline__ bf16_t from_f32(float v) { return f32_to_bf16(v); }
};

// Dot product of two 16-byte vectors accumulated into fp32.
template <typename T> __device__ __forceinline__ float dot16(u32x4 a, u32x4 b, float acc);
template <> __device__ __forceinline__ float dot16<float>(u32x4 a, u32x4 b, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) acc = fmaf(__uint_as_float(a[i]), __uint_as_float(b[i]), acc);
  return acc;
}
// Note: each vector element is copied to a scalar before the bit cast; a bit
// cast applied directly to an ext_vector element expression was observed to
// read element 0 for every index.
template <> __device__ __forceinline__ float dot16<bf16_t>(u32x4 a, u32x4 b, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t ai = a[i], bi = b[i];
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, ai), __builtin_bit_cast(bf16x2, bi), acc,
                                          false);
  }
  return acc;
}

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
// Raw buffer resources (gfx9 family): word 3 of the descriptor for untyped
// dword access; loads at offsets >= num_records return zeros without a memory
// access.  Cache policy 2 marks a load non-temporal (streamed once).
constexpr int kBufferDword3 = 0x00020000;
constexpr int kCachePolicyStream = 2;

__device__ __forceinline__ u32x4 load16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void store16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// 16 bytes per lane from global memory straight into LDS: lane l of the wave
// writes lds + 16 l (lds wave-uniform).  Issued from inline assembly so that
// the compiler's own wait-count bookkeeping, which cannot tell ring stages
// apart and would wait for every copy before the next LDS read, leaves these
// copies alone: the kernel waits for them itself.  M0 holds the LDS address
// and needs one wait state before the copy reads it.  STREAM marks the read
// non-temporal (data read once, e.g. the KV cache), so it does not displace
// data that is reused from the caches.
template <bool STREAM = false>
__device__ __forceinline__ void dma16(const void* g, void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  const unsigned m = __builtin_amdgcn_readfirstlane(
      static_cast<unsigned>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)lds)));
  if constexpr (STREAM)
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" : : "v"(g), "s"(m) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(g), "s"(m) : "memory", "m0");
#endif
}

// s_waitcnt immediate (gfx9 family): at most n vector-memory operations and no
// LDS / scalar-memory operations outstanding (export count left at its maximum)
constexpr int waitcnt_vm_lgkm0(int n) { return (n & 15) | (((n >> 4) & 3) << 14) | (7 << 4); }


__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// Reduce-scatter of NV per-lane partial sums across the 64 lanes of a wave.
// Afterwards v[0] of lane l holds the full sum of index (l >> (6 - log2(NV)));
// lanes that share an index hold the same value.  NV must be a power of two <= 64.
template <int HALF, int OFF, int NV>
__device__ __forceinline__ void reduce_scatter_step(float (&v)[NV], int lane) {
  if constexpr (HALF >= 1) {
    const bool up = (lane & OFF) != 0;
#pragma unroll
    for (int i = 0; i < HALF; ++i) {
      const float send = up ? v[i] : v[i + HALF];
      const float keep = up ? v[i + HALF] : v[i];
      v[i] = keep + __shfl_xor(send, OFF, 64);
    }
    reduce_scatter_step<HALF / 2, OFF / 2, NV>(v, lane);
  } else if constexpr (OFF >= 1) {
    v[0] += __shfl_xor(v[0], OFF, 64);
    reduce_scatter_step<0, OFF / 2, NV>(v, lane);
  }
}
template <int NV>
__device__ __forceinline__ float wave_reduce_scatter(float (&v)[NV], int lane) {
  static_assert(NV >= 1 && NV <= 64 && (NV & (NV - 1)) == 0, "NV must be a power of two <= 64");
  reduce_scatter_step<NV / 2, 32, NV>(v, lane);
  return v[0];
}
template <int NV> struct Log2 { static constexpr int value = 1 + Log2<NV / 2>::value; };
template <> struct Log2<1> { static constexpr int value = 0; };

// cos/sin of the rotary angle p * inv_freq: the product and its reduction to
// [-pi, pi] are done in double precision, the final sincos in fp32, so the
// angle error stays ~1e-7 rad even at positions of tens of thousands.
__device__ __forceinline__ void rope_cos_sin(int pos, double inv_freq, float& c, float& s) {
  const double ang = static_cast<double>(pos) * inv_freq;
  const double two_pi = 6.283185307179586476925286766559;
  const double r = ang - two_pi * rint(ang * (1.0 / two_pi));
  sincosf(static_cast<float>(r), &s, &c);
}

// Best and runner-up logit of a set of vocabulary rows (ties -> lowest id).
// (both sides evaluated: a short-circuit here becomes a branch per compare)
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return (va > vb) | ((va == vb) & (ia < ib));
}
__device__ __forceinline__ void top2_push(Top2& t, float v, int i) {
  const bool b = better(v, i, t.v1, t.i1);
  t.v2 = b ? t.v1 : (v > t.v2 ? v : t.v2);
  t.v1 = b ? v : t.v1;
  t.i1 = b ? i : t.i1;
}
// (selects rather than a swap, so that no lane takes a branch)
__device__ __forceinline__ Top2 top2_merge(Top2 a, Top2 b) {
  const bool s = better(b.v1, b.i1, a.v1, a.i1);
  Top2 r;
  r.v1 = s ? b.v1 : a.v1;
  r.i1 = s ? b.i1 : a.i1;
  r.v2 = fmaxf(s ? b.v2 : a.v2, s ? a.v1 : b.v1);
  r.pad = s ? b.pad : a.pad;
  return r;
}
__device__ __forceinline__ Top2 top2_empty() {
  Top2 t;
  t.v1 = -INFINITY;
  t.i1 = 0x7fffffff;
  t.v2 = -INFINITY;
  t.pad = 0;
  return t;
}

}  // namespace pe
