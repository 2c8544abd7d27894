// Device primitives for the gfx950 decode-layer kernel: number formats, MFMA
// wrappers, wave reductions and the grid barrier of the persistent launch.
//
// Formats follow the OCP 8-bit float (E4M3FN) and Microscaling (MX v1.0)
// definitions used by "Mono decode layer for DeepSeek-V4.1-Flash on MI355X"
// (vLLM PR 60397), Layout and Design: e4m3 weights/activations/KV codes, E8M0
// block exponents, e2m1 routed-expert weights, bf16 activations.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsl {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ------------------------------------------------------------------ scalar formats

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// float32 -> bf16, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// e4m3fn code -> float: exponent field 1..15 is 2^(e-7)(1+m/8), 0 is m/8 * 2^-6
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t em = c & 0x7Fu;
  float v = em >= 8u ? __uint_as_float((em + 960u) << 20) : (float)em * 0.001953125f;
  return __uint_as_float(__float_as_uint(v) | ((c & 0x80u) << 24));
}

// float -> e4m3fn code, round to nearest even, saturating at +-448
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  uint32_t s = (__float_as_uint(x) >> 24) & 0x80u;
  float a = fabsf(x);
  if (!(a < 448.0f)) return s | 0x7Eu;
  if (a < 0.015625f) return s | (uint32_t)__builtin_rintf(a * 512.0f);  // subnormal steps 2^-9
  uint32_t b = __float_as_uint(a);
  b += 0x7FFFFu + ((b >> 20) & 1u);  // keep 3 mantissa bits, ties to even
  uint32_t code = (((b >> 23) - 120u) << 3) | ((b >> 20) & 7u);
  return s | (code > 0x7Eu ? 0x7Eu : code);
}

// MX shared exponent of a block with maximum magnitude amax (e4m3 elements):
// floor(log2 amax) from the float32 exponent field, less e4m3's emax (8), biased by
// 127, clamped to [0, 254].  An all-zero block gets 0.
__device__ __forceinline__ uint32_t mx_e4m3_exponent(float amax) {
  int e = (int)((__float_as_uint(amax) >> 23) & 0xFFu) - 8;
  return (uint32_t)(e < 0 ? 0 : (e > 254 ? 254 : e));
}
// 2^(127 - X), the factor that brings a block onto the e4m3 grid (X <= 246 here)
__device__ __forceinline__ float mx_inv_scale(uint32_t X) { return __uint_as_float((254u - X) << 23); }
// E8M0 byte as a float (2^(X-127)); X = 0 is the subnormal 2^-127
__device__ __forceinline__ float e8m0_to_f32(uint32_t X) {
  return X ? __uint_as_float(X << 23) : __uint_as_float(0x00400000u);
}

// ------------------------------------------------------------------ MFMA

// C += A . B over K = 32 bf16: lane (i, g) holds row i, K elements [8g, 8g+8).
__device__ __forceinline__ v4f mfma_bf16(v4u a, v4u b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c,
                                                 0, 0, 0);
}

// Two e2m1 values (one byte of w, selected by SEL) times scale -> two bf16 (low = even k)
template <int SEL>
__device__ __forceinline__ uint32_t cvt_fp4x2_bf16(uint32_t w, float scale) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, SEL));
}
// Two e4m3 values (16-bit word HI of w) times scale -> two bf16 (exact for a
// power-of-two scale)
template <bool HI>
__device__ __forceinline__ uint32_t cvt_fp8x2_bf16s(uint32_t w, float scale) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, scale, HI));
}
// Two e4m3 values (word HI of w) -> two floats, exact
template <bool HI>
__device__ __forceinline__ v2f cvt_fp8x2_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
}

// ------------------------------------------------------------------ wave reductions

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
// max over aligned groups of G lanes (G a power of two <= 64)
template <int G>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// ------------------------------------------------------------------ loads / stores

// Every buffer the kernel touches is device (global) memory.  Pointers reach the
// kernel through structs, so the compiler cannot infer that and would emit FLAT
// accesses, whose completion counts against the LDS/scalar counter too (every LDS
// wait would then drain all outstanding loads).  These helpers address the global
// segment explicitly.
template <class T>
__device__ __forceinline__ const __attribute__((address_space(1))) T *gptr(const T *p) {
  return (const __attribute__((address_space(1))) T *)p;
}
template <class T>
__device__ __forceinline__ __attribute__((address_space(1))) T *gptr(T *p) {
  return (__attribute__((address_space(1))) T *)p;
}
template <class T>
__device__ __forceinline__ T ldg(const T *p) { return *gptr(p); }
// Stores are write-through at device scope (relaxed agent-scope atomic stores, which
// gfx950 issues with the sc1 policy): a line another XCD reads later never sits dirty
// in the writer's L2.  Loads are plain.  Together with the rule that every buffer the
// launch produces is written at most once per launch and read only after the grid
// barrier that follows the write, no cache can hold a stale copy of produced data, so
// the grid barrier needs no L2 write-back or invalidate.
template <class U>
__device__ __forceinline__ void st_wt(U *p, U v) {
  __hip_atomic_store(gptr(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class T>
__device__ __forceinline__ void stg(T *p, T v) {
  static_assert(sizeof(T) == 1 || sizeof(T) == 2 || sizeof(T) == 4 || sizeof(T) == 8 || sizeof(T) == 16,
                "store size");
  if constexpr (sizeof(T) == 16) {
    uint64_t w[2];
    __builtin_memcpy(w, &v, 16);
    uint64_t *q = reinterpret_cast<uint64_t *>(p);
    st_wt(q, w[0]);
    st_wt(q + 1, w[1]);
  } else if constexpr (sizeof(T) == 8) {
    uint64_t w;
    __builtin_memcpy(&w, &v, 8);
    st_wt(reinterpret_cast<uint64_t *>(p), w);
  } else if constexpr (sizeof(T) == 4) {
    uint32_t w;
    __builtin_memcpy(&w, &v, 4);
    st_wt(reinterpret_cast<uint32_t *>(p), w);
  } else if constexpr (sizeof(T) == 2) {
    uint16_t w;
    __builtin_memcpy(&w, &v, 2);
    st_wt(reinterpret_cast<uint16_t *>(p), w);
  } else {
    uint8_t w;
    __builtin_memcpy(&w, &v, 1);
    st_wt(reinterpret_cast<uint8_t *>(p), w);
  }
}
__device__ __forceinline__ v4u ld16(const void *p) { return ldg(reinterpret_cast<const v4u *>(p)); }
__device__ __forceinline__ void st16(void *p, v4u v) { stg(reinterpret_cast<v4u *>(p), v); }
__device__ __forceinline__ float4 ld_f4(const float *p) {
  const v4f t = ldg(reinterpret_cast<const v4f *>(p));
  return make_float4(t[0], t[1], t[2], t[3]);
}
__device__ __forceinline__ void st_f4(float *p, float4 v) { stg(reinterpret_cast<v4f *>(p), v4f{v.x, v.y, v.z, v.w}); }
__device__ __forceinline__ float2 ld_f2(const float *p) {
  const v2f t = ldg(reinterpret_cast<const v2f *>(p));
  return make_float2(t[0], t[1]);
}
__device__ __forceinline__ void st_f2(float *p, float2 v) { stg(reinterpret_cast<v2f *>(p), v2f{v.x, v.y}); }

// ------------------------------------------------------------------ grid barrier

// Sync words of a handle (each counter on a 256-byte line of its own).
struct SyncWords {
  unsigned group[8][64];  // arrivals per group of blocks (block index mod 8)
  unsigned top[64];       // groups fully arrived
  unsigned generation;    // completed barriers (monotonic; the barrier's epoch tag)
  unsigned pad1[63];
  unsigned health;        // 0, or a DSL device fault code
  unsigned pad2[63];
  unsigned tasks[64];     // task-queue counters (zeroed at each launch before use)
};

enum : unsigned { kFaultBarrier = 1u, kFaultSlot = 2u };

// All blocks of the launch meet here.  Each wave first waits for its own memory
// operations (its write-through stores are then at the device's coherence point), the
// block meets, and thread 0 arrives with relaxed atomics.  Arrivals are counted in two
// levels (8 group counters, then one top counter) so no single address takes more than
// nblocks/8 atomics; the last arrival bumps the generation word the others poll.  No
// cache maintenance: see stg.  The spin is bounded: a barrier that does not complete
// records kFaultBarrier in the health word and lets the block go on, so the launch
// always drains.
__device__ __forceinline__ void grid_barrier(SyncWords *sw, unsigned nblocks) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned grp = blockIdx.x & 7u;
    const unsigned ngroups = nblocks < 8u ? nblocks : 8u;
    const unsigned per = (nblocks - grp + 7u) / 8u;  // blocks in this group
    const unsigned gen = __hip_atomic_load(gptr(&sw->generation), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);
    const unsigned a = __hip_atomic_fetch_add(gptr(&sw->group[grp][0]), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bool released = false;
    if (a == per - 1u) {
      __hip_atomic_store(gptr(&sw->group[grp][0]), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const unsigned b = __hip_atomic_fetch_add(gptr(&sw->top[0]), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (b == ngroups - 1u) {
        __hip_atomic_store(gptr(&sw->top[0]), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(0);
        __hip_atomic_fetch_add(gptr(&sw->generation), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        released = true;
      }
    }
    if (!released) {
      unsigned spins = 0;
      while (__hip_atomic_load(gptr(&sw->generation), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gen) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins > (1u << 24)) {
          __hip_atomic_fetch_or(gptr(&sw->health), (unsigned)kFaultBarrier, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
      }
    }
  }
  __syncthreads();
}

}  // namespace dsl
