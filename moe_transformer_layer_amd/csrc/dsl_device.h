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
typedef int v4i __attribute__((ext_vector_type(4)));
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

__device__ __forceinline__ int lane_id() { return (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// The value of lane (this lane XOR O), O a power of two below 64: the quad steps and the
// 8-lane step by DPP (quad_perm, and row_ror:8, which within a row of 16 is the XOR), the
// 4-lane step by a bit-masked swizzle, the 16- and 32-lane steps by the permlane swaps.
// None of them forms an LDS address, unlike a general shuffle.
template <int O>
__device__ __forceinline__ float lane_xor(float v) {
  const int u = __float_as_int(v);
  if constexpr (O == 1) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, u, 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
  } else if constexpr (O == 2) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, u, 0x4E, 0xF, 0xF, false));  // quad_perm 2,3,0,1
  } else if constexpr (O == 4) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(u, 0x101F));  // and 0x1F, or 0, xor 4
  } else if constexpr (O == 8) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, u, 0x128, 0xF, 0xF, false));  // row_ror 8
  } else if constexpr (O == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap((uint32_t)u, (uint32_t)u, false, false);
    return __uint_as_float((lane_id() & 16) ? r[0] : r[1]);
  } else {
    static_assert(O == 32, "lane_xor: O is a power of two below 64");
    const auto r = __builtin_amdgcn_permlane32_swap((uint32_t)u, (uint32_t)u, false, false);
    return __uint_as_float((lane_id() & 32) ? r[0] : r[1]);
  }
}
// The same for a step known only after unrolling
__device__ __forceinline__ float lane_xor_n(float v, int o) {
  switch (o) {
    case 1: return lane_xor<1>(v);
    case 2: return lane_xor<2>(v);
    case 4: return lane_xor<4>(v);
    case 8: return lane_xor<8>(v);
    case 16: return lane_xor<16>(v);
    default: return lane_xor<32>(v);
  }
}
// v + (the value of lane XOR O): for the 16- and 32-lane steps the permlane swap's two
// results are that pair in every lane (addition commutes, so the sum is the same bits)
template <int O>
__device__ __forceinline__ float sum_xor(float v) {
  if constexpr (O == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else if constexpr (O == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else {
    return v + lane_xor<O>(v);
  }
}

// max(v, the value of lane XOR O), the same way
template <int O>
__device__ __forceinline__ float max_xor(float v) {
  if constexpr (O == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  } else if constexpr (O == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  } else {
    return fmaxf(v, lane_xor<O>(v));
  }
}

// Sum over the wave, the same in every lane: the XOR butterfly, 32 lanes apart first
__device__ __forceinline__ float wave_sum(float v) {
  v = sum_xor<32>(v);
  v = sum_xor<16>(v);
  v = sum_xor<8>(v);
  v = sum_xor<4>(v);
  v = sum_xor<2>(v);
  return sum_xor<1>(v);
}
// max over aligned groups of G lanes (G a power of two <= 64)
template <int G>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (G >= 64) v = max_xor<32>(v);
  if constexpr (G >= 32) v = max_xor<16>(v);
  if constexpr (G >= 16) v = max_xor<8>(v);
  if constexpr (G >= 8) v = max_xor<4>(v);
  if constexpr (G >= 4) v = max_xor<2>(v);
  if constexpr (G >= 2) v = max_xor<1>(v);
  return v;
}
__device__ __forceinline__ float wave_max(float v) { return group_max<64>(v); }

// Sum over the wave of V per-lane values, transposed: returns, in lane L, the total of
// value L >> (6 - log2 V).  Lane bit 5 is resolved by a permlane32 swap, bit 4 by a
// permlane16 swap (for a pair (A, B) both halves then hold A and B summed over the
// bit), the lower bits by shuffles.
template <int V>
__device__ __forceinline__ float wave_transpose_sum(float (&v)[V], int lane) {
  static_assert(V >= 1 && V <= 64 && (V & (V - 1)) == 0, "V is a power of two");
  float c[V];
#pragma unroll
  for (int i = 0; i < V; i++) c[i] = v[i];
  int n = V;
#pragma unroll
  for (int i = 0; i < V / 2; i++) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(c[i]), __float_as_uint(c[i + V / 2]), false, false);
    c[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  if (V >= 2) n = V / 2;
  if (V >= 4) {
#pragma unroll
    for (int i = 0; i < V / 4; i++) {
      const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(c[i]), __float_as_uint(c[i + V / 4]), false, false);
      c[i] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    n = V / 4;
  }
#pragma unroll
  for (int bit = 3; bit >= 0; bit--) {
    if (n >= 2) {
      const bool hi = (lane >> bit) & 1;
#pragma unroll
      for (int i = 0; i < n / 2; i++) {
        const float send = hi ? c[i] : c[i + n / 2];
        const float keep = hi ? c[i + n / 2] : c[i];
        c[i] = keep + lane_xor_n(send, 1 << bit);
      }
      n /= 2;
    } else {
      c[0] += lane_xor_n(c[0], 1 << bit);
    }
  }
  if (V == 1) {
    // bits 5 and 4 were not reduced above
    const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(c[0]), __float_as_uint(c[0]), false, false);
    c[0] = __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
    const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(c[0]), __float_as_uint(c[0]), false, false);
    c[0] = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
  }
  return c[0];
}

// Arg-max keys: an unsigned 64-bit key whose order is (float value, then lower index):
// high word = the float's bits made order-preserving as an unsigned integer, low word
// = 127 - index.  Exact for every non-NaN value.
__device__ __forceinline__ uint64_t amax_key(float v, int i) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)o << 32) | (uint32_t)(127 - i);
}
__device__ __forceinline__ float amax_key_value(uint64_t k) {
  const uint32_t o = (uint32_t)(k >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
__device__ __forceinline__ int amax_key_index(uint64_t k) { return 127 - (int)(uint32_t)k; }

template <int CTRL>
__device__ __forceinline__ uint64_t amax_dpp(uint64_t k) {
  const uint32_t lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)k, CTRL, 0xF, 0xF, false);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)(k >> 32), CTRL, 0xF, 0xF, false);
  const uint64_t o = ((uint64_t)hi << 32) | lo;
  return o > k ? o : k;
}
// The key of the lane 16 (or 32) positions away across the half boundary
__device__ __forceinline__ uint64_t amax_half(uint64_t k, bool lower, bool is32) {
  const uint32_t lo = (uint32_t)k, hi = (uint32_t)(k >> 32);
  const auto rl = is32 ? __builtin_amdgcn_permlane32_swap(lo, lo, false, false)
                       : __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
  const auto rh = is32 ? __builtin_amdgcn_permlane32_swap(hi, hi, false, false)
                       : __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
  const uint64_t o = ((uint64_t)(lower ? rh[1] : rh[0]) << 32) | (lower ? rl[1] : rl[0]);
  return o > k ? o : k;
}
// Wave-wide maximum key, in every lane: quad and row steps by DPP, the 16- and 32-lane
// halves by the permlane swaps.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t k, int lane) {
  k = amax_dpp<0xB1>(k);   // quad_perm 1,0,3,2
  k = amax_dpp<0x4E>(k);   // quad_perm 2,3,0,1
  k = amax_dpp<0x124>(k);  // row_ror 4
  k = amax_dpp<0x128>(k);  // row_ror 8
  k = amax_half(k, (lane & 16) == 0, false);
  return amax_half(k, lane < 32, true);
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
// 16 bytes of weights, which a launch reads once: a nontemporal (streaming) load, so the
// weight stream does not displace cached activations and scratch, and streams faster
// than cached loads.
__device__ __forceinline__ v4u ldw16(const void *p) {
  return __builtin_nontemporal_load(gptr(reinterpret_cast<const v4u *>(p)));
}
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

// Sync words of a handle (each counter on a 256-byte line of its own).  The counters
// only grow: after R completed barriers group[g] = (blocks in group g) * R, top =
// groups * R and every release[g] = R (mod 2^32), so no barrier resets a word.
struct SyncWords {
  unsigned group[8][64];    // arrivals per group of blocks (block index mod 8)
  unsigned top[64];         // groups fully arrived
  unsigned release[8][64];  // completed barriers: one copy per group, polled by that group
  unsigned tq[64][16];      // wo_a tasks finished per 32-column group of t; only grow
  unsigned cb[128][16];     // down-stage waves finished per 32-column group of the MoE output; only grow
  unsigned ho[152][64];     // producer hand-off counters (kHo* below); only grow
  unsigned health;          // 0, or a DSL device fault code
  unsigned pad2[63];
};

enum : unsigned { kFaultBarrier = 1u, kFaultSlot = 2u };

// Hand-off counters: finished producers of one consumer set, counted after each producer's
// stores have drained.  A row counter has 8 copies that every row increments (its pollers
// spread over 8 lines); a task counter has 8 copies of which task t increments copy t mod 8
// (its increments spread over 8 lines) and its pollers sum them.
//   kHoQ: q rows (qkv_post); kHoKv: kv records and key-offset rows (one counter);
//   kHoQb + h: wq_b tasks of head h; kHoAtt + h: attention items of head h;
//   kHoWq / kHoWkv: wqkv tasks of the q / kv latent columns (task counters);
//   kHoTb + c: quantized t groups of wo_b's K chunk c; kHoWb: wo_b tasks (task counter);
//   kHoU: MoE input rows; kHoRt / kHoSh: router and shared gate/up tasks (task counters);
//   kHoX: the attention input's normalized rows (row counter); kHoO: the layer output's
//   32-column groups (task counter), for the next chained layer; kHoTk: rows whose experts
//   the grid top-k has stored (steps wider than a block's waves).
enum : int {
  kHoQ = 0, kHoKv = 8, kHoQb = 9, kHoAtt = 41, kHoWq = 73, kHoWkv = 81, kHoTb = 89, kHoWb = 97, kHoU = 105,
  kHoRt = 113, kHoSh = 121, kHoX = 129, kHoO = 137, kHoTk = 145, kHoSlots = 146, kHoHeads = 32, kHoTbChunks = 8
};

// Waits until counter id reaches target (modular, like the barrier's release word): lane 0
// polls, the wave follows.  Bounded like the barrier's spin: a count that never arrives
// records kFaultBarrier and lets the wave go on, so the launch always drains.
__device__ __forceinline__ void ho_wait(SyncWords *sw, int id, unsigned target, int lane) {
  if (lane == 0) {
    unsigned spins = 0;
    while ((int)(__hip_atomic_load(gptr(&sw->ho[id][0]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) - target) < 0) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins > (1u << 24)) {
        __hip_atomic_fetch_or(gptr(&sw->health), (unsigned)kFaultBarrier, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  asm volatile("" ::: "memory");  // the consumer's loads stay after the wait
}

// The same for a task counter: waits until its 8 copies sum to target
__device__ __forceinline__ void ho_wait_sum8(SyncWords *sw, int id, unsigned target, int lane) {
  if (lane == 0) {
    unsigned spins = 0;
    for (;;) {
      unsigned sum = 0;
#pragma unroll
      for (int c = 0; c < 8; c++)
        sum += __hip_atomic_load(gptr(&sw->ho[id + c][0]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if ((int)(sum - target) >= 0) break;
      __builtin_amdgcn_s_sleep(1);
      if (++spins > (1u << 24)) {
        __hip_atomic_fetch_or(gptr(&sw->health), (unsigned)kFaultBarrier, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  asm volatile("" ::: "memory");
}

// Counts one finished producer on counter id: the wave's stores are drained first, so the
// counted data are at the coherence point before any consumer can see the count.
__device__ __forceinline__ void ho_count(SyncWords *sw, int id, int lane, unsigned n = 1) {
  __builtin_amdgcn_s_waitcnt(0);
  if (lane == 0) __hip_atomic_fetch_add(gptr(&sw->ho[id][0]), n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Barriers completed on this sync state before the launch.  Every block reads it before
// its first arrival, and no barrier of the launch completes before all blocks have
// arrived, so every block reads the same value.
__device__ __forceinline__ unsigned barrier_base(SyncWords *sw) {
  return __hip_atomic_load(gptr(&sw->release[blockIdx.x & 7u][0]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// All blocks of the launch meet here, in two parts.  barrier_drain: each wave waits for
// its own memory operations (its write-through stores are then at the device's
// coherence point).  A wave may then issue loads that do not depend on the stage before
// (the next stage's weights) and keep them in flight across the meeting.
// grid_barrier_meet: the block meets (no wait on vector memory), and one thread, `bt`,
// arrives with relaxed atomics; it must belong to a wave with no loads in flight, since
// the atomics' results are waited for in issue order.  Arrivals are counted in two
// levels (8 group counters, then one top counter) so no single address takes more than
// nblocks/8 atomics; the last arrival writes the barrier's number into one release word
// per group, and each group polls its own word, so the polls do not queue behind the
// counters' atomics.  *next (thread bt's, in LDS) is the number this barrier completes.
// No cache maintenance: see stg.  The spin is bounded: a barrier that does not complete
// records kFaultBarrier in the health word and lets the block go on, so the launch
// always drains.
__device__ __forceinline__ void barrier_drain() { __builtin_amdgcn_s_waitcnt(0); }

__device__ __forceinline__ void grid_barrier_meet(SyncWords *sw, unsigned nblocks, unsigned *next, unsigned bt) {
  __syncthreads();
  if (threadIdx.x == bt) {
    const unsigned grp = blockIdx.x & 7u;
    const unsigned ngroups = nblocks < 8u ? nblocks : 8u;
    const unsigned per = (nblocks - grp + 7u) / 8u;  // blocks in this group
    const unsigned r = *next;
    const unsigned a = __hip_atomic_fetch_add(gptr(&sw->group[grp][0]), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bool released = false;
    if (a == per * r - 1u) {
      const unsigned b = __hip_atomic_fetch_add(gptr(&sw->top[0]), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (b == ngroups * r - 1u) {
        for (unsigned g = 0; g < ngroups; g++)
          __hip_atomic_store(gptr(&sw->release[g][0]), r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        released = true;
      }
    }
    if (!released) {
      unsigned spins = 0;
      while ((int)(__hip_atomic_load(gptr(&sw->release[grp][0]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) - r) < 0) {
        __builtin_amdgcn_s_sleep(1);
        if (++spins > (1u << 24)) {
          __hip_atomic_fetch_or(gptr(&sw->health), (unsigned)kFaultBarrier, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
      }
    }
    *next = r + 1u;
  }
  __syncthreads();
}

// The arrival half of a grid barrier (thread bt, after a __syncthreads that follows what
// the arrival stands for): the block counts itself for barrier *next and goes on; the
// barrier completes, as grid_barrier_meet's, when every block has arrived.  *fence takes
// the barrier's number for grid_fence_wait.
__device__ __forceinline__ void grid_barrier_arrive(SyncWords *sw, unsigned nblocks, unsigned *next, unsigned *fence) {
  const unsigned grp = blockIdx.x & 7u;
  const unsigned ngroups = nblocks < 8u ? nblocks : 8u;
  const unsigned per = (nblocks - grp + 7u) / 8u;
  const unsigned r = *next;
  const unsigned a = __hip_atomic_fetch_add(gptr(&sw->group[grp][0]), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (a == per * r - 1u) {
    const unsigned b = __hip_atomic_fetch_add(gptr(&sw->top[0]), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (b == ngroups * r - 1u)
      for (unsigned g = 0; g < ngroups; g++)
        __hip_atomic_store(gptr(&sw->release[g][0]), r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  *fence = r;
  *next = r + 1u;
}

// Waits (lane 0; the wave follows) until barrier r has completed, i.e. every block has
// arrived at it; bounded like the barrier's own spin.
__device__ __forceinline__ void grid_fence_wait(SyncWords *sw, unsigned r, int lane) {
  if (lane == 0) {
    unsigned spins = 0;
    while ((int)(__hip_atomic_load(gptr(&sw->release[blockIdx.x & 7u][0]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) -
                 r) < 0) {
      __builtin_amdgcn_s_sleep(1);
      if (++spins > (1u << 24)) {
        __hip_atomic_fetch_or(gptr(&sw->health), (unsigned)kFaultBarrier, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  asm volatile("" ::: "memory");
}

}  // namespace dsl
