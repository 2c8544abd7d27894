// The decode layer as one persistent launch (one block per compute unit) on gfx950,
// and the host runtime behind the C ABI of include/dsl.h.
//
// One launch runs, per layer, the stages of "Mono decode layer for
// DeepSeek-V4.1-Flash on MI355X" (vLLM PR 60397), Purpose, launch table (K1 and
// K2 without the tensor-parallel all-reduces), with a grid barrier between
// dependent stages.  Three draft layers chain inside the same launch ("Mono
// decode for the DSpark draft layers", vLLM PR 62131, Details).  Every stage's
// tasks are split statically over the grid's waves in wave-major order (task t to
// wave t mod waves, consecutive tasks on different compute units); the routed
// experts' tasks follow the routing table every block builds from the top-k.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "dsl_stages.h"

namespace dsl {

// ============================================================== attention front

// Row stages run one row per block: every thread holds E contiguous values, issues
// all of its loads at once, and block reductions combine the rows' sums.

__device__ __forceinline__ int64_t slot_of(const Params &p, const dsl_kv &kv, int req, int t);
__device__ __forceinline__ int64_t record_off(const Params &p, const dsl_kv &kv, int64_t slot);

// The cache byte offset of every key of row m (-1 past the row's keys or for a pad
// row): the causal window [max(0, p - W + 1), p] through the block table, or the row of
// the caller's slot table.  Written for the attention stage, so that it reaches a record
// in one load.
__device__ __forceinline__ void key_offsets_row(const Params &p, const dsl_kv &kv, int m) {
  const int keys = p.swa > 0 ? p.swa : p.W;
  const int pos = ldg(p.pos + m);
  const int req = ldg(kv.row_req + m);
  const int lo = pos - p.W + 1 < 0 ? 0 : pos - p.W + 1;
  for (int j = tid(); j < keys; j += kThreads) {
    int64_t off = -1;
    if (pos >= 0) {
      if (p.swa > 0) {
        const int64_t slot = ldg(kv.key_table + (size_t)m * p.swa + j);
        if (slot >= 0) off = record_off(p, kv, slot);
      } else if (lo + j <= pos) {
        off = record_off(p, kv, slot_of(p, kv, req, lo + j));
      }
    }
    stg(p.s.keyoff + (size_t)m * keys + j, off);
  }
}

// RMSNorm of the layer input, then MXFP8 quantization (kept as exact bf16 values).
// With `fence` (hand-offs in place of the grid barrier after this stage) each row is
// counted on the eight copies of kHoX once its stores have drained and every block has
// arrived at barrier `fence` (so every block has read the counters' starting values).
template <int E>
__device__ __forceinline__ void st_attn_norm_e(const Params &p, const dsl_weights &w, const dsl_kv &kv,
                                               const uint16_t *xin, float *red, bool count = false,
                                               unsigned fence = 0u, unsigned wait_out = 0u, const unsigned *hb = nullptr) {
  const int n = p.h, k = tid() * E;
  const bool act = k < n;
  // a chained layer's input comes from the layer before by hand-off (wait_out: the count
  // of its output's column groups to wait for), not across a grid barrier
  if (wait_out && bid() < p.M) {
    unsigned base = 0;
#pragma unroll
    for (int c = 0; c < 8; c++) base += hb[kHoO + c];
    if (tid() < kWave) ho_wait_sum8(p.sync, kHoO, base + wait_out, tid());
    __syncthreads();
  }
  // with fewer than 3 M blocks the key records of row m are resolved here, by block M + m
  // (or by block m itself with fewer than 2 M blocks); else by the qkv_post stage
  const bool late = (int)gridDim.x >= 3 * p.M, split = (int)gridDim.x >= 2 * p.M;
  if (!late && split && bid() >= p.M && bid() < 2 * p.M) key_offsets_row(p, kv, bid() - p.M);
  for (int m = bid(); m < p.M; m += gridDim.x) {
    if (!split) key_offsets_row(p, kv, m);
    float v[E], gm[E];
    if (act)
      load_bf16<E>(xin + (size_t)m * n + k, v);
    else
#pragma unroll
      for (int e = 0; e < E; e++) v[e] = 0.f;
    load_f32<E>(w.attn_norm + k, act, gm);  // with the row, not after the reduction's barrier
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < E; e++) ss += v[e] * v[e];
    ss = block_sum(ss, red);
    const float r = 1.0f / sqrtf(ss / (float)n + p.eps);
#pragma unroll
    for (int e = 0; e < E; e++) v[e] = act ? v[e] * r * gm[e] : 0.f;
    mx_quant_dequant<E>(v);
    if (act) store_bf16<E>(p.s.xb + (size_t)m * n + k, v);
    if (count) {
      barrier_drain();
      __syncthreads();
      if (tid() < kWave) {
        grid_fence_wait(p.sync, fence, tid());
        if (tid() < 8)
          __hip_atomic_fetch_add(gptr(&p.sync->ho[kHoX + tid()][0]), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

// Byte offset of a slot's record in the cache, or -1 (with a recorded fault) if the slot
// is outside the cache view.
__device__ __forceinline__ int64_t record_off(const Params &p, const dsl_kv &kv, int64_t slot) {
  const int64_t blk = slot / p.B;
  if (slot < 0 || blk >= kv.n_blocks) {
    __hip_atomic_fetch_or(gptr(&p.sync->health), (unsigned)kFaultSlot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return -1;
  }
  return blk * kv.block_stride + (slot - blk * p.B) * (int64_t)(p.D + 16);
}

// Slot of token position t of request req through the block table, or -1.
__device__ __forceinline__ int64_t slot_of(const Params &p, const dsl_kv &kv, int req, int t) {
  const int lb = t / p.B;
  if (req < 0 || req >= kv.n_req || t < 0 || lb >= kv.max_blocks) return -1;
  const int blk = ldg(kv.block_table + (size_t)req * kv.max_blocks + lb);
  return blk < 0 ? -1 : (int64_t)blk * p.B + (t - lb * p.B);
}

// Hand-off targets of layer l: each counter grows by a fixed number per layer, read relative
// to its value at the start of the launch (hb, in LDS)
__device__ __forceinline__ unsigned ho_per_qb(const Params &p) { return (unsigned)((p.D >> 4) * (p.qr / p.pl.kc_qb)); }
__device__ __forceinline__ unsigned hb_sum8(const unsigned *hb, int id) {
  unsigned s = 0;
#pragma unroll
  for (int c = 0; c < 8; c++) s += hb[id + c];
  return s;
}
// tasks per layer of the task counters
__device__ __forceinline__ int ho_t_wq(const Params &p) { return (p.qr >> 4) * (p.h / p.pl.kc_qkv); }
__device__ __forceinline__ int ho_t_wkv(const Params &p) { return (p.D >> 4) * (p.h / p.pl.kc_qkv); }
__device__ __forceinline__ int ho_t_wb(const Params &p) { return (p.h >> 4) * (p.orr / p.pl.kc_ob); }
__device__ __forceinline__ int ho_t_rt(const Params &p) { return p.E * (p.h / p.pl.kc_router); }
__device__ __forceinline__ int ho_t_sh(const Params &p) { return ((2 * p.Is) >> 4) * (p.h / p.pl.kc_sh13); }

// q latent: sum the split-K partials, RMSNorm, MXFP8.  wait(): the caller's wait for the
// partials, made once the norm's weights are on their way.
template <int E, class Wait>
__device__ __forceinline__ void qpost_row(const Params &p, const dsl_weights &w, int m, float *red, Wait wait) {
  const int N = p.qr + p.D, nks = p.h / p.pl.kc_qkv, n = p.qr, k = tid() * E;
  const bool act = k < n;
  float v[E], gm[E];
  load_f32<E>(w.q_norm + k, act, gm);
  wait();
  if (act)
    load_sum_f32<E>(p.s.p_qkv + (size_t)m * N + k, (size_t)p.M * N, nks, v);
  else
#pragma unroll
    for (int e = 0; e < E; e++) v[e] = 0.f;
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < E; e++) ss += v[e] * v[e];
  ss = block_sum(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)n + p.eps);
#pragma unroll
  for (int e = 0; e < E; e++) v[e] = act ? v[e] * r * gm[e] : 0.f;
  mx_quant_dequant<E>(v);
  if (act) store_bf16<E>(p.s.qb + (size_t)m * n + k, v);
}

// kv latent: RMSNorm, then the fp8 record (codes e4m3(v / s), s = amax / 448, then 12
// zero bytes) at the row's slot.  wait(): the caller's wait for the partials, made once
// the norm's weights and the record's place (position, request, block table) are on
// their way.
template <int E, class Wait>
__device__ __forceinline__ void kvpost_row(const Params &p, const dsl_weights &w, const dsl_kv &kv, int m, float *red,
                                           uint8_t *tmp, Wait wait) {
  const int N = p.qr + p.D, nks = p.h / p.pl.kc_qkv, n = p.D, k = tid() * E;
  const bool act = k < n;
  float v[E], gm[E];
  load_f32<E>(w.kv_norm + k, act, gm);
  const int pos = ldg(p.pos + m);
  const int64_t slot = pos >= 0 ? slot_of(p, kv, ldg(kv.row_req + m), pos) : (int64_t)-1;
  wait();
  if (act)
    load_sum_f32<E>(p.s.p_qkv + (size_t)m * N + p.qr + k, (size_t)p.M * N, nks, v);
  else
#pragma unroll
    for (int e = 0; e < E; e++) v[e] = 0.f;
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < E; e++) ss += v[e] * v[e];
  ss = block_sum(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)n + p.eps);
  float am = 0.f;
#pragma unroll
  for (int e = 0; e < E; e++) {
    v[e] = act ? v[e] * r * gm[e] : 0.f;
    am = fmaxf(am, fabsf(v[e]));
  }
  am = block_max(am, red);
  if (pos < 0) return;  // pad row: no KV write
  const float sc = am / 448.0f;
  const int64_t blk = slot / p.B;
  if (slot < 0 || blk >= kv.n_blocks) {  // outside the cache view: recorded, no write
    if (tid() == 0)
      __hip_atomic_fetch_or(gptr(&p.sync->health), (unsigned)kFaultSlot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  uint8_t *rec = kv.base + blk * kv.block_stride + (slot - blk * p.B) * (int64_t)(p.D + 16);
  // codes gathered in LDS, then written as 16-byte stores
  if (act) {
#pragma unroll
    for (int e = 0; e < E; e++) tmp[k + e] = sc > 0.f ? (uint8_t)f32_to_e4m3(v[e] / sc) : (uint8_t)0;
  }
  __syncthreads();
  const int t = tid();
  if (t < n / 16) st16(rec + 16 * t, *reinterpret_cast<const v4u *>(tmp + 16 * t));
  if (t == n / 16) st16(rec + p.D, v4u{__float_as_uint(sc), 0u, 0u, 0u});
}

// tmp: LDS of at least head_dim bytes for the record's codes
// NARROW: the narrow-step kernel (q rank 1024, head dim 512: 2 and 1 elements per thread)
template <bool NARROW>
__device__ __forceinline__ void st_qkv_post(const Params &p, const dsl_weights &w, const dsl_kv &kv, float *red,
                                            uint8_t *tmp, const unsigned *hb, int l, bool fenced, unsigned fence) {
  const int eq = NARROW ? 2 : row_elems(p.qr), ekv = NARROW ? 1 : row_elems(p.D);
  // q of row m on block m, kv of row m on block M + m, row m's key offsets on block 2 M + m
  // (with fewer than 3 M blocks the key offsets come from the norm stage, with fewer than
  // 2 M all of a row's work is block m's)
  if ((int)gridDim.x >= 2 * p.M) {
    const int b = bid();
    // hand-off: every wqkv task of the row's part (q latent, or kv latent) has stored its partials
    auto wait = [&] {
      if (p.ho >= 2) {
        if (tid() == 0) {
          if (b < p.M)
            ho_wait_sum8(p.sync, kHoWq, hb_sum8(hb, kHoWq) + (unsigned)(l + 1) * (unsigned)ho_t_wq(p), 0);
          else
            ho_wait_sum8(p.sync, kHoWkv, hb_sum8(hb, kHoWkv) + (unsigned)(l + 1) * (unsigned)ho_t_wkv(p), 0);
        }
        __syncthreads();
      }
    };
    if (b >= 2 * p.M && b < 3 * p.M) key_offsets_row(p, kv, b - 2 * p.M);
    if (b < p.M) {
      switch (eq) {
        case 2: qpost_row<2>(p, w, b, red, wait); break;
        default:
          if constexpr (!NARROW) {
            if (eq == 1) qpost_row<1>(p, w, b, red, wait);
            else if (eq == 4) qpost_row<4>(p, w, b, red, wait);
            else if (eq == 8) qpost_row<8>(p, w, b, red, wait);
            else qpost_row<16>(p, w, b, red, wait);
          }
          break;
      }
    } else if (b < 2 * p.M) {
      switch (ekv) {
        case 1: kvpost_row<1>(p, w, kv, b - p.M, red, tmp, wait); break;
        default:
          if constexpr (!NARROW) kvpost_row<2>(p, w, kv, b - p.M, red, tmp, wait);
          break;
      }
    }
    if (p.ho && b < 3 * p.M) {
      // hand-off: the row's stores drained in every wave, then one count (a q row on all
      // eight copies of its counter; a kv record or a key-offset row on kHoKv).  A key-offset
      // row waits on nothing else, so with `fence` it first waits for every block's arrival
      // (the counters' starting values read everywhere).
      barrier_drain();
      __syncthreads();
      if (fenced && b >= 2 * p.M && tid() < kWave) grid_fence_wait(p.sync, fence, tid());
      if (tid() < (b < p.M ? 8 : 1))
        __hip_atomic_fetch_add(gptr(&p.sync->ho[b < p.M ? kHoQ + tid() : kHoKv][0]), 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }
  for (int m = bid(); m < p.M; m += gridDim.x) {
    switch (eq) {
      case 2: qpost_row<2>(p, w, m, red, [] {}); break;
      default:
        if constexpr (!NARROW) {
          if (eq == 1) qpost_row<1>(p, w, m, red, [] {});
          else if (eq == 4) qpost_row<4>(p, w, m, red, [] {});
          else if (eq == 8) qpost_row<8>(p, w, m, red, [] {});
          else qpost_row<16>(p, w, m, red, [] {});
        }
        break;
    }
    switch (ekv) {
      case 1: kvpost_row<1>(p, w, kv, m, red, tmp, [] {}); break;
      default:
        if constexpr (!NARROW) kvpost_row<2>(p, w, kv, m, red, tmp, [] {});
        break;
    }
  }
}

// ============================================================== attention

template <int V>
__device__ __forceinline__ void decode_codes(uint64_t c, float out[V]) {
  if constexpr (V == 8) {
    const v2f a = cvt_fp8x2_f32<false>((uint32_t)c), b = cvt_fp8x2_f32<true>((uint32_t)c);
    const v2f d = cvt_fp8x2_f32<false>((uint32_t)(c >> 32)), e = cvt_fp8x2_f32<true>((uint32_t)(c >> 32));
    out[0] = a[0]; out[1] = a[1]; out[2] = b[0]; out[3] = b[1];
    out[4] = d[0]; out[5] = d[1]; out[6] = e[0]; out[7] = e[1];
  } else if constexpr (V == 4) {
    const v2f a = cvt_fp8x2_f32<false>((uint32_t)c), b = cvt_fp8x2_f32<true>((uint32_t)c);
    out[0] = a[0]; out[1] = a[1]; out[2] = b[0]; out[3] = b[1];
  } else if constexpr (V == 2) {
    const v2f a = cvt_fp8x2_f32<false>((uint32_t)c);
    out[0] = a[0]; out[1] = a[1];
  } else {
    out[0] = e4m3_to_f32((uint32_t)c & 0xFFu);
  }
}

template <int V>
__device__ __forceinline__ uint64_t load_codes(const uint8_t *p) {
  if constexpr (V == 8) return ldg(reinterpret_cast<const uint64_t *>(p));
  else if constexpr (V == 4) return ldg(reinterpret_cast<const uint32_t *>(p));
  else if constexpr (V == 2) return ldg(reinterpret_cast<const uint16_t *>(p));
  else return ldg(p);
}

// One (row, head, split): scores q . k / sqrt(D) over up to KS keys (16 or 32) of the
// row's key set, with k = v = scale * e4m3(codes) of the record; returns the partial max,
// the sum of exponentials and (lane l: dims [V l, V l + V)) the exponential-weighted sum
// of values.  Lane j < KS reads key j's record offset and scale; each key's offset
// reaches the wave as a scalar (readlane), every lane loads its V dims of all KS keys in
// one batch and keeps them in registers for the value pass, and the dot products are
// summed across the wave by the transposing butterfly, 16 keys at a time.  The records
// need only the step's own records and key offsets (the caller's wait before the call);
// q, which comes later in the stage chain, is waited for (wait_q) after the record loads
// are issued, so they are in flight during that wait (EARLY; else the caller has waited
// for q as well, and q is loaded with the first records: the general kernel's choice,
// measured faster at 48 rows).
template <int V, int KS, bool EARLY, class WaitQ>
__device__ __forceinline__ void attn_item(const Params &p, const dsl_kv &kv, int m, int hh, int sp, int lane,
                                          float &mx_out, float &l_out, float (&o)[V], WaitQ wait_q) {
  static_assert(KS == 16 || KS == 32, "16 or 32 keys per split");
  const int D = p.D, H = p.H;
  const int keys = p.swa > 0 ? p.swa : p.W;
  const int j0 = sp * KS;
  const int nks = p.qr / p.pl.kc_qb;
  const size_t qstride = (size_t)p.M * H * D;
  const float *qp = p.s.p_q + (size_t)m * H * D + (size_t)hh * D + lane * V;
  float q[V];
  int64_t myoff = -1;
  if (lane < KS && j0 + lane < keys) myoff = ldg(p.s.keyoff + (size_t)m * keys + j0 + lane);
  const float mysc = myoff >= 0 ? ldg(reinterpret_cast<const float *>(kv.base + myoff + D)) : 0.f;
  if constexpr (!EARLY) {
    wait_q();
    load_sum_f32<V>(qp, qstride, nks, q);
  }
  const uint32_t olo = (uint32_t)(uint64_t)myoff, ohi = (uint32_t)((uint64_t)myoff >> 32);
  // key j's record offset, as a scalar
  auto key_off = [&](int j) -> int64_t {
    return (int64_t)(((uint64_t)__builtin_amdgcn_readlane(ohi, j) << 32) | __builtin_amdgcn_readlane(olo, j));
  };
  // every lane's V dims of the KS keys, loaded in one batch and kept for the value pass
  uint64_t codes[KS];
#pragma unroll
  for (int j = 0; j < KS; j++) {
    const int64_t off = key_off(j);
    codes[j] = off >= 0 ? load_codes<V>(kv.base + off + lane * V) : 0ull;
  }
  if constexpr (EARLY) {
    wait_q();
    load_sum_f32<V>(qp, qstride, nks, q);
  }
  float sc[KS / 16];
#pragma unroll
  for (int hf = 0; hf < KS / 16; hf++) {
    float d[16];
#pragma unroll
    for (int j = 0; j < 16; j++) {
      float c[V];
      decode_codes<V>(codes[16 * hf + j], c);
      float a = 0.f;
#pragma unroll
      for (int v = 0; v < V; v++) a += q[v] * c[v];
      d[j] = a;
    }
    sc[hf] = wave_transpose_sum<16>(d, lane);  // lane L: key 16 hf + (L >> 2)
  }
  // lane j < KS: the score of key j
  float sj = __shfl(sc[0], 4 * (lane & 15), kWave);
  if constexpr (KS == 32) {
    const float s1 = __shfl(sc[1], 4 * (lane & 15), kWave);
    sj = lane < 16 ? sj : s1;
  }
  const float my = myoff >= 0 ? sj * mysc * p.attn_scale : -INFINITY;
  const float mx = wave_max(my);
  const float pj = my == -INFINITY ? 0.f : expf(my - mx);
  const float l = wave_sum(pj);
  const float f = pj * mysc;
  // values: the same codes, weighted by exp(score - max) * scale (the empty asm makes
  // the compiler decode them again here instead of keeping all decoded values live)
#pragma unroll
  for (int j = 0; j < KS; j++) asm volatile("" : "+v"(codes[j]));
#pragma unroll
  for (int v = 0; v < V; v++) o[v] = 0.f;
#pragma unroll
  for (int j = 0; j < KS; j++) {
    const float fj = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(f), j));
    float c[V];
    decode_codes<V>(codes[j], c);
#pragma unroll
    for (int v = 0; v < V; v++) o[v] += fj * c[v];
  }
  mx_out = mx;
  l_out = l;
}

// The log-sum-exp combine of S split partials (max, sum, output) of one head dim d, in
// split order: o = sum_s e_s o_s / sum_s e_s l_s with e_s = exp(max_s - max) (the same
// operations, in the same order, as the one-wave combine of st_attention_v).
__device__ __forceinline__ float attn_combine_dim(const float *lo_, const float *lml, int S, int D, int d) {
  float mx = -INFINITY;
  for (int s = 0; s < S; s++) mx = fmaxf(mx, lml[2 * s]);
  float L = 0.f, o = 0.f;
  for (int s = 0; s < S; s++) {
    const float ls = lml[2 * s + 1];
    if (!(ls > 0.f)) continue;
    const float e = expf(lml[2 * s] - mx);
    L += ls * e;
    o += lo_[s * D + d] * e;
  }
  return L > 0.f ? o / L : o;
}

// Attention and the log-sum-exp combine in one stage: a block takes P (row, head) items
// at a time (one if the grid has a block per item, else 8 / S), one wave per split; the
// splits' partials meet in LDS (lds: 8 D + 16 floats), where one wave per item combines
// them, quantizes the output to MXFP8 (a 32-block spans 32 / V lanes) and stores it.
// Pad rows give zeros.
template <int V, bool EARLY = false>
__device__ __forceinline__ void st_attention_v(const Params &p, const Ctx &cx, const dsl_kv &kv, float *lds,
                                               const unsigned *hb, int l) {
  const int S = p.S, D = p.D;
  const int T = p.M * p.H;
  // items per block: one when the grid has a block per item (the item's split waves then
  // have a SIMD each), else as many as the block's waves hold
  const int P = T <= (int)gridDim.x ? 1 : kWavesPerBlock / S;
  const int w = cx.wave, lane = cx.lane, i = w / S, sp = w - i * S;
  float *lo_ = lds, *lml = lds + kWavesPerBlock * D;
  for (int t0 = bid() * P; t0 < T; t0 += gridDim.x * P) {
    const int t = t0 + i;
    if (i < P && t < T) {
      const int m = t / p.H, hh = t - m * p.H;
      float mx = -INFINITY, l_ = 0.f, o[V];
#pragma unroll
      for (int v = 0; v < V; v++) o[v] = 0.f;
      // the head's q (every wq_b task of its columns) and the step's records and key
      // offsets; with EARLY the q wait comes once the record loads are issued
      auto wait_q = [&] {
        if (p.ho) ho_wait(p.sync, kHoQb + hh, hb[kHoQb + hh] + (unsigned)(l + 1) * ho_per_qb(p), lane);
      };
      if constexpr (!EARLY) wait_q();
      if (p.ho) ho_wait(p.sync, kHoKv, hb[kHoKv] + (unsigned)(l + 1) * (unsigned)(2 * p.M), lane);
      // a pad row's key offsets are all -1, so its item gives zeros
      if constexpr (EARLY)
        attn_item<V, kSplitKeys, true>(p, kv, m, hh, sp, lane, mx, l_, o, wait_q);
      else
        attn_item<V, kSplitKeys, false>(p, kv, m, hh, sp, lane, mx, l_, o, [] {});
#pragma unroll
      for (int v = 0; v < V; v++) lo_[w * D + lane * V + v] = o[v];
      if (lane == 0) {
        lml[2 * w] = mx;
        lml[2 * w + 1] = l_;
      }
    }
    __syncthreads();
    if (w < P && t0 + w < T) {
      const int tt = t0 + w, m = tt / p.H, hh = tt - m * p.H;
      float o[V];
#pragma unroll
      for (int v = 0; v < V; v++) o[v] = 0.f;
      float mx = -INFINITY;
      for (int s = 0; s < S; s++) mx = fmaxf(mx, lml[2 * (w * S + s)]);
      float L = 0.f;
      for (int s = 0; s < S; s++) {
        const float ls = lml[2 * (w * S + s) + 1];
        if (!(ls > 0.f)) continue;
        const float e = expf(lml[2 * (w * S + s)] - mx);
        L += ls * e;
#pragma unroll
        for (int v = 0; v < V; v++) o[v] += lo_[(w * S + s) * D + lane * V + v] * e;
      }
      if (L > 0.f) {
#pragma unroll
        for (int v = 0; v < V; v++) o[v] = o[v] / L;
      }
      mx_quant_dequant<V>(o);
      store_bf16<V>(p.s.ob + (size_t)m * p.H * D + (size_t)hh * D + lane * V, o);
      if (p.ho) ho_count(p.sync, kHoAtt + hh, lane);
    }
    __syncthreads();
  }
}

// The narrow kernel's attention (at most 8 rows, head dim 512: the grid has a block per
// item): a block's (row, head) item, one wave per split of KS keys (16 when the row's
// keys fit 8 such splits, else 32), the record loads issued before the wait on q; then
// every wave combines 64 of the head's 512 dims (one per lane) and stores them, and once
// all eight have drained their stores, one counts the item for its head.  Each wave's
// serial work (the item's dot products and value sums, the combine) is what sets this
// stage's time, so the keys and the combine are spread over all eight waves.
template <int KS>
__device__ __forceinline__ void st_attention_narrow_ks(const Params &p, const Ctx &cx, const dsl_kv &kv, float *lds,
                                                       const unsigned *hb, int l, int S) {
  constexpr int V = 8, D = 512;
  const int T = p.M * p.H;
  const int w = cx.wave, lane = cx.lane;
  float *lo_ = lds, *lml = lds + kWavesPerBlock * D;
  for (int t = bid(); t < T; t += gridDim.x) {
    const int m = t / p.H, hh = t - m * p.H;
    if (w < S) {
      float mx = -INFINITY, l_ = 0.f, o[V];
#pragma unroll
      for (int v = 0; v < V; v++) o[v] = 0.f;
      if (p.ho) ho_wait(p.sync, kHoKv, hb[kHoKv] + (unsigned)(l + 1) * (unsigned)(2 * p.M), lane);
      // a pad row's key offsets are all -1, so its item gives zeros
      attn_item<V, KS, true>(p, kv, m, hh, w, lane, mx, l_, o, [&] {
        if (p.ho) ho_wait(p.sync, kHoQb + hh, hb[kHoQb + hh] + (unsigned)(l + 1) * ho_per_qb(p), lane);
      });
#pragma unroll
      for (int v = 0; v < V; v++) lo_[w * D + lane * V + v] = o[v];
      if (lane == 0) {
        lml[2 * w] = mx;
        lml[2 * w + 1] = l_;
      }
    }
    __syncthreads();
    float o[1] = {attn_combine_dim(lo_, lml, S, D, 64 * w + lane)};
    mx_quant_dequant<1>(o);
    store_bf16<1>(p.s.ob + (size_t)m * p.H * D + (size_t)hh * D + 64 * w + lane, o);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's part of the output is at the coherence point
    __syncthreads();
    if (p.ho && w == 0) ho_count(p.sync, kHoAtt + hh, lane);
  }
}

__device__ __forceinline__ void st_attention_narrow(const Params &p, const Ctx &cx, const dsl_kv &kv, float *lds,
                                                    const unsigned *hb, int l) {
  const int keys = p.swa > 0 ? p.swa : p.W;
  if (keys <= 8 * 16)
    st_attention_narrow_ks<16>(p, cx, kv, lds, hb, l, (keys + 15) / 16);
  else
    st_attention_narrow_ks<32>(p, cx, kv, lds, hb, l, p.S);
}

// wo_a output: sum the split-K partials, then MXFP8
template <int E>
__device__ __forceinline__ void st_t_quant_e(const Params &p) {
  const int N = p.orr, nks = (p.H * p.D) / p.pl.kc_oa, k = tid() * E;
  const bool act = k < N;
  for (int m = bid(); m < p.M; m += gridDim.x) {
    float v[E];
    if (act)
      load_sum_f32<E>(p.s.p_t + (size_t)m * N + k, (size_t)p.M * N, nks, v);
    else
#pragma unroll
      for (int e = 0; e < E; e++) v[e] = 0.f;
    mx_quant_dequant<E>(v);
    if (act) store_bf16<E>(p.s.tb + (size_t)m * N + k, v);
  }
}

// t_quant folded into wo_a.  The wo_a tasks of one 32-column group of t (one MX block
// wide: 2 column tiles x the K chunks) count their finished tasks on a counter that only
// grows; the task that finishes a group last sums the group's split-K partials and
// quantizes them, as st_t_quant_e does (same helpers, same order), so no grid barrier and
// row stage are needed between wo_a and wo_b.  Each task's partial stores are drained
// before its count, so they are at the coherence point when the last task reads them
// (the grid barrier's rule, with the counter in place of the barrier).  Used while every
// wave has at most one wo_a task and M <= 16 (two passes of 8 rows for the last task);
// `base` is the group's counter before the layer, read at the start of the launch.
constexpr int kTqGroups = 64;

__device__ __forceinline__ bool tq_fold(const Params &p) {
  const int T = (p.orr >> 4) * ((p.H * p.D) / p.pl.kc_oa);
  return p.M <= 16 && T <= (int)gridDim.x * kWavesPerBlock && p.orr / 32 <= kTqGroups;
}

// The group of this wave's wo_a task, or -1
__device__ __forceinline__ int tq_group(const Params &p, const Ctx &cx) {
  const int ntile = p.orr >> 4, T = ntile * ((p.H * p.D) / p.pl.kc_oa);
  return cx.gw < T ? (cx.gw % ntile) >> 1 : -1;
}

// The last task of group j: t[m][32 j .. 32 j + 32) for every row m.  Lane l takes row
// m0 + l / 8 and columns 32 j + 4 (l % 8) .. + 4; the 8 lanes of a row hold its block.
__device__ __forceinline__ void tq_group_quant(const Params &p, int j, int lane) {
  const int N = p.orr, nks = (p.H * p.D) / p.pl.kc_oa, k = 32 * j + 4 * (lane & 7);
  for (int m0 = 0; m0 < p.M; m0 += 8) {
    const int m = m0 + (lane >> 3);
    float v[4];
    if (m < p.M)
      load_sum_f32<4, 16>(p.s.p_t + (size_t)m * N + k, (size_t)p.M * N, nks, v);  // one batch for 16 heads
    else
#pragma unroll
      for (int e = 0; e < 4; e++) v[e] = 0.f;
    mx_quant_dequant<4>(v);
    if (m < p.M) store_bf16<4>(p.s.tb + (size_t)m * N + k, v);
  }
}

// Hand-off: wo_a's K chunk ks holds heads [ks kc / D, (ks + 1) kc / D) of the attention output;
// wait until every row's item of each has been stored
__device__ __forceinline__ void ho_wait_heads(const Params &p, int ks, int lane, const unsigned *hb, int l) {
  const int nh = p.pl.kc_oa / p.D, h0 = ks * nh;
  for (int h = h0; h < h0 + nh; h++) ho_wait(p.sync, kHoAtt + h, hb[kHoAtt + h] + (unsigned)(l + 1) * (unsigned)p.M, lane);
}

// wo_a without the fold (more than 16 rows), with the hand-off waits
template <int MAXG>
__device__ __forceinline__ void st_wo_a_ho(const Params &p, const Ctx &cx, const dsl_weights &w, const PreA &pf,
                                           const unsigned *hb, int l) {
  const int N = p.orr, K = p.H * p.D, kc = p.pl.kc_oa, ntile = N >> 4, T = ntile * (K / kc);
  int t = cx.gw;
  if (t >= T) return;
  ho_wait_heads(p, t / ntile, cx.lane, hb, l);
  linear_task<kW8T32, MAXG>(t, cx.lane, w.wo_a, w.wo_a_s, nullptr, N, K, kc, p.s.ob, p.M, p.s.p_t, &pf, pf.on);
  for (t += cx.nw; t < T; t += cx.nw) {
    ho_wait_heads(p, t / ntile, cx.lane, hb, l);
    linear_task<kW8T32, MAXG>(t, cx.lane, w.wo_a, w.wo_a_s, nullptr, N, K, kc, p.s.ob, p.M, p.s.p_t);
  }
}

// wq_b with the hand-offs: wait for every q row, then count each finished task for its head
template <int MAXG, bool ONE>
__device__ __forceinline__ void st_wq_b_ho(const Params &p, const Ctx &cx, const dsl_weights &w, const PreA &pf,
                                           const unsigned *hb, int l) {
  const int N = p.H * p.D, K = p.qr, kc = p.pl.kc_qb, ntile = N >> 4, T = ntile * (K / kc);
  int t = cx.gw;
  if (t >= T) return;
  const int c = bid() & 7;
  ho_wait(p.sync, kHoQ + c, hb[kHoQ + c] + (unsigned)(l + 1) * (unsigned)p.M, cx.lane);
  linear_task<kW8T32, MAXG>(t, cx.lane, w.wq_b, w.wq_b_s, nullptr, N, K, kc, p.s.qb, p.M, p.s.p_q, &pf, pf.on);
  ho_count(p.sync, kHoQb + ((t % ntile) << 4) / p.D, cx.lane);
  if constexpr (ONE) return;
  for (t += cx.nw; t < T; t += cx.nw) {
    linear_task<kW8T32, MAXG>(t, cx.lane, w.wq_b, w.wq_b_s, nullptr, N, K, kc, p.s.qb, p.M, p.s.p_q);
    ho_count(p.sync, kHoQb + ((t % ntile) << 4) / p.D, cx.lane);
  }
}

__device__ __forceinline__ void st_wo_a_fold(const Params &p, const Ctx &cx, const dsl_weights &w, const PreA &pf,
                                             unsigned base, const unsigned *hb, int l) {
  const int N = p.orr, K = p.H * p.D, kc = p.pl.kc_oa, nks = K / kc, T = (N >> 4) * nks;
  const int t = cx.gw;
  if (t >= T) return;
  if (p.ho) ho_wait_heads(p, t / (N >> 4), cx.lane, hb, l);
  linear_task<kW8T32, 1>(t, cx.lane, w.wo_a, w.wo_a_s, nullptr, N, K, kc, p.s.ob, p.M, p.s.p_t, &pf, pf.on);
  const int j = tq_group(p, cx);
  __builtin_amdgcn_s_waitcnt(0);  // this task's partials are at the coherence point
  unsigned old = 0;
  if (cx.lane == 0)
    old = __hip_atomic_fetch_add(gptr(&p.sync->tq[j][0]), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  old = (unsigned)__builtin_amdgcn_readfirstlane(old);
  if (old - base != 2u * (unsigned)nks - 1u) return;
  asm volatile("" ::: "memory");  // the partial loads stay after the count
  tq_group_quant(p, j, cx.lane);
  if (p.ho >= 2) ho_count(p.sync, kHoTb + (32 * j) / p.pl.kc_ob, cx.lane);
}

// wqkv with the hand-offs: count each finished task for its part (q or kv latent columns)
// (wait_x: the rows come by hand-off, kHoX, instead of a grid barrier)
template <int MAXG, bool ONE>
__device__ __forceinline__ void st_wqkv_ho(const Params &p, const Ctx &cx, const dsl_weights &w, const PreA &pf,
                                           bool wait_x, const unsigned *hb, int l) {
  const int N = p.qr + p.D, K = p.h, kc = p.pl.kc_qkv, ntile = N >> 4, T = ntile * (K / kc);
  int t = cx.gw;
  if (t >= T) return;
  if (wait_x) {
    const int c = bid() & 7;
    ho_wait(p.sync, kHoX + c, hb[kHoX + c] + (unsigned)(l + 1) * (unsigned)p.M, cx.lane);
  }
  linear_task<kW8T32, MAXG>(t, cx.lane, w.wqkv, w.wqkv_s, nullptr, N, K, kc, p.s.xb, p.M, p.s.p_qkv, &pf, pf.on);
  ho_count(p.sync, (((t % ntile) << 4) < p.qr ? kHoWq : kHoWkv) + (t & 7), cx.lane);
  if constexpr (ONE) return;
  for (t += cx.nw; t < T; t += cx.nw) {
    linear_task<kW8T32, MAXG>(t, cx.lane, w.wqkv, w.wqkv_s, nullptr, N, K, kc, p.s.xb, p.M, p.s.p_qkv);
    ho_count(p.sync, (((t % ntile) << 4) < p.qr ? kHoWq : kHoWkv) + (t & 7), cx.lane);
  }
}

// wo_b with the hand-offs: each task waits for its K chunk's t groups (when wo_a's output
// quantization is folded in) and is counted when done
template <int MAXG, bool ONE>
__device__ __forceinline__ void st_wo_b_ho(const Params &p, const Ctx &cx, const dsl_weights &w, const PreA &pf,
                                           const unsigned *hb, int l, bool wait_tb) {
  const int N = p.h, K = p.orr, kc = p.pl.kc_ob, ntile = N >> 4, T = ntile * (K / kc);
  const unsigned groups = (unsigned)(kc >> 5);
  int t = cx.gw;
  if (t >= T) return;
  if (wait_tb) ho_wait(p.sync, kHoTb + t / ntile, hb[kHoTb + t / ntile] + (unsigned)(l + 1) * groups, cx.lane);
  linear_task<kW8T32, MAXG>(t, cx.lane, w.wo_b, w.wo_b_s, nullptr, N, K, kc, p.s.tb, p.M, p.s.p_a, &pf, pf.on);
  ho_count(p.sync, kHoWb + (t & 7), cx.lane);
  if constexpr (ONE) return;
  for (t += cx.nw; t < T; t += cx.nw) {
    if (wait_tb) ho_wait(p.sync, kHoTb + t / ntile, hb[kHoTb + t / ntile] + (unsigned)(l + 1) * groups, cx.lane);
    linear_task<kW8T32, MAXG>(t, cx.lane, w.wo_b, w.wo_b_s, nullptr, N, K, kc, p.s.tb, p.M, p.s.p_a);
    ho_count(p.sync, kHoWb + (t & 7), cx.lane);
  }
}

// wo_b output a (sum of partials).  Attention-only steps write bf16(a).  Full steps:
// hres = bf16(x + a), u = bf16(RMSNorm_ffn(hres)).  Pad rows give zeros.
template <int E>
__device__ __forceinline__ void st_ffn_norm_e(const Params &p, const dsl_weights &w, const uint16_t *xin, bool last, float *red,
                                              const unsigned *hb, int l) {
  const int h = p.h, nks = p.orr / p.pl.kc_ob, k = tid() * E;
  const bool act = k < h;
  for (int m = bid(); m < p.M; m += gridDim.x) {
    // what does not depend on wo_b first (the row's position, its residual input, the
    // norm's weights), so that those loads are in flight during the wait
    const bool live = ldg(p.pos + m) >= 0;
    float a[E], hr[E], gm[E];
    if (act)
      load_bf16<E>(xin + (size_t)m * h + k, hr);
    else
#pragma unroll
      for (int e = 0; e < E; e++) hr[e] = 0.f;
    load_f32<E>(w.ffn_norm + k, act && p.mode != kModeAttn, gm);
    if (p.ho >= 2) {
      // hand-off: every wo_b task of the layer has stored its partials
      if (tid() == 0) ho_wait_sum8(p.sync, kHoWb, hb_sum8(hb, kHoWb) + (unsigned)(l + 1) * (unsigned)ho_t_wb(p), 0);
      __syncthreads();
    }
    if (act)
      load_sum_f32<E>(p.s.p_a + (size_t)m * h + k, (size_t)p.M * h, nks, a);
    else
#pragma unroll
      for (int e = 0; e < E; e++) a[e] = 0.f;
#pragma unroll
    for (int e = 0; e < E; e++) {
      a[e] = live ? a[e] : 0.f;
      hr[e] = live ? bf16_to_f32(f32_to_bf16(hr[e] + a[e])) : 0.f;
    }
    const size_t off = (size_t)m * h + k;
    if (p.mode == kModeAttn) {
      if (act) store_bf16<E>(p.out + off, a);
      continue;  // (block-uniform)
    }
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < E; e++) ss += hr[e] * hr[e];
    ss = block_sum(ss, red);
    const float r = 1.0f / sqrtf(ss / (float)h + p.eps);
    if (act) {
      store_bf16<E>(p.s.hres + off, hr);
      if (last && p.taps.hres) store_bf16<E>((uint16_t *)p.taps.hres + off, hr);
      if (last && p.taps.attn_out) store_bf16<E>((uint16_t *)p.taps.attn_out + off, a);
      float uu[E];
#pragma unroll
      for (int e = 0; e < E; e++) uu[e] = live ? hr[e] * r * gm[e] : 0.f;
      store_bf16<E>(p.s.u + off, uu);
      if (last && p.taps.moe_in) store_bf16<E>((uint16_t *)p.taps.moe_in + off, uu);
    }
    if (p.ho >= 2) {
      // hand-off: the row's u is out; one count on each copy of the row counter
      barrier_drain();
      __syncthreads();
      if (tid() < 8)
        __hip_atomic_fetch_add(gptr(&p.sync->ho[kHoU + tid()][0]), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ============================================================== MoE

// MXFP8 of 32-element blocks of bf16 rows: block b of n blocks (row b / per, 32 columns from
// 32 (b % per)) from src, one thread per block, as exact bf16 values into dst (the VALU
// experts' operand, and the matrix-core experts' with expert_a8 = 1) and, with code set
// (expert_a8 = 2), also as e4m3 codes and the block's E8M0 exponent into code / ex (the
// scaled matrix instruction's operand; the same quantization, so the two agree exactly).
// The A8W4 variant's expert inputs: "Mono decode layer for DeepSeek-V4.1-Flash on MI355X"
// (vLLM PR 60397), Test Plan (the a8w4 MoE), with the OCP MX block rule of the layer's other
// MXFP8 activations.
__device__ __forceinline__ void mx_block_a8(const uint16_t *src, uint16_t *dst, uint8_t *code, uint8_t *ex, int b,
                                            int per, int ld) {
  const size_t off = (size_t)(b / per) * ld + 32 * (b % per);
  float v[32];
  load_bf16<32>(src + off, v);
  float am = 0.f;
#pragma unroll
  for (int e = 0; e < 32; e++) am = fmaxf(am, fabsf(v[e]));
  const uint32_t X = mx_e4m3_exponent(am);
  const float inv = mx_inv_scale(X), sc = e8m0_to_f32(X);
  v4u cw[2] = {v4u{0, 0, 0, 0}, v4u{0, 0, 0, 0}};
#pragma unroll
  for (int e = 0; e < 32; e++) {
    const uint32_t c = f32_to_e4m3(v[e] * inv);
    v[e] = e4m3_to_f32(c) * sc;
    cw[e >> 4][(e >> 2) & 3] |= c << (8 * (e & 3));
  }
  store_bf16<32>(dst + off, v);
  if (code) {
    st16(code + off, cw[0]);
    st16(code + off + 16, cw[1]);
    stg(ex + off / 32, (uint8_t)X);
  }
}

// A8W4: MXFP8 of the MoE input u [M][h] into uq, by the grid's threads in reverse order (the
// last waves, which have no router or shared gate/up task, take the blocks first).
__device__ __forceinline__ void st_u_quant(const Params &p, const Ctx &cx, const uint16_t *u) {
  const int per = p.h >> 5, n = p.M * per, nt = cx.nw * kWave;
  for (int b = nt - 1 - (cx.gw * kWave + cx.lane); b < n; b += nt) mx_block_a8(u, p.s.uq, p.a8 == 2 ? p.s.uq8 : nullptr, p.s.uqe, b, per, p.h);
}

// A8W4: MXFP8 of the routed SwiGLU outputs z [pairs][I] into zq (one thread per block).
__device__ __forceinline__ void st_z_quant(const Params &p, const Routing &R) {
  const int per = p.I >> 5, n = R.np * per;
  for (int b = bid() * kThreads + tid(); b < n; b += gridDim.x * kThreads) mx_block_a8(p.s.zr, p.s.zq, p.a8 == 2 ? p.s.zq8 : nullptr, p.s.zqe, b, per, p.I);
}

// Router partial logits of one (expert e, K chunk c) task for all rows: lane l takes
// elements c kc + 512 j + 8 l .. + 8 (j < kc / 512, lanes past the chunk idle), the
// lane partials of 8 rows at a time are summed across the wave by the transposing
// butterfly (lane L then holds row L >> 3), written to logits[c][m][e].  Each batch of
// loads is issued before any arithmetic uses it.
template <int J, class Wait>
__device__ __forceinline__ void router_task_j(const Params &p, const float *__restrict__ Wr, const uint16_t *u, int e,
                                              int c, int lane, Wait wait) {
  const int h = p.h, kc = p.pl.kc_router;
  float4 wv[J][2];
  bool on[J];
#pragma unroll
  for (int j = 0; j < J; j++) {
    const int k = c * kc + 512 * j + 8 * lane;
    on[j] = 512 * j + 8 * lane < kc;
    const float *wp = Wr + (size_t)e * h + (on[j] ? k : c * kc);
    const v4u w0 = ldw16(wp), w1 = ldw16(wp + 4);
    wv[j][0] = make_float4(__uint_as_float(w0[0]), __uint_as_float(w0[1]), __uint_as_float(w0[2]), __uint_as_float(w0[3]));
    wv[j][1] = make_float4(__uint_as_float(w1[0]), __uint_as_float(w1[1]), __uint_as_float(w1[2]), __uint_as_float(w1[3]));
  }
  // the weights do not depend on the step: they are on their way before the wait for u
  wait();
  for (int m0 = 0; m0 < p.M; m0 += 8) {
    v4u uv[8][J];
#pragma unroll
    for (int r = 0; r < 8; r++) {
      const int m = m0 + r < p.M ? m0 + r : p.M - 1;
#pragma unroll
      for (int j = 0; j < J; j++)
        uv[r][j] = ld16(u + (size_t)m * h + (on[j] ? c * kc + 512 * j + 8 * lane : c * kc));
    }
    __builtin_amdgcn_sched_barrier(0);
    float acc[8];
#pragma unroll
    for (int r = 0; r < 8; r++) {
      float a = 0.f;
#pragma unroll
      for (int j = 0; j < J; j++) {
        if (!on[j]) continue;
        const float wf[8] = {wv[j][0].x, wv[j][0].y, wv[j][0].z, wv[j][0].w,
                             wv[j][1].x, wv[j][1].y, wv[j][1].z, wv[j][1].w};
#pragma unroll
        for (int q = 0; q < 4; q++) {
          a = fmaf(wf[2 * q], bf16_to_f32(uv[r][j][q] & 0xFFFFu), a);
          a = fmaf(wf[2 * q + 1], bf16_to_f32(uv[r][j][q] >> 16), a);
        }
      }
      acc[r] = a;
    }
    const float tot = wave_transpose_sum<8>(acc, lane);
    const int m = m0 + (lane >> 3);
    if ((lane & 7) == 0 && m < p.M) stg(p.s.logits + ((size_t)c * p.M + m) * p.E + e, tot);
  }
}

// Router partial logits ((expert, K chunk) tasks) and the shared expert's gate/up
// partials, together: both read only the MoE input.
template <bool NARROW>
__device__ __forceinline__ void st_router_shared(const Params &p, const Ctx &cx, const dsl_weights &w, const uint16_t *u,
                                                 const unsigned *hb, int l) {
  const int TR = p.E * (p.h / p.pl.kc_router);
  const int Nsh = 2 * p.Is;
  const int TS = (Nsh >> 4) * (p.h / p.pl.kc_sh13);
  const int J = (p.pl.kc_router + 511) >> 9;
  // hand-off: every row's u is out (a router task waits once its weights are on their way)
  bool waited = p.ho < 2;
  auto wait_u = [&] {
    if (!waited) {
      const int c = bid() & 7;
      ho_wait(p.sync, kHoU + c, hb[kHoU + c] + (unsigned)(l + 1) * (unsigned)p.M, cx.lane);
      waited = true;
    }
  };
  // narrow: a shared gate/up task's first weights are on their way before the wait too
  // (its wave then takes a row's top-k sooner)
  PreA pf = pre_none();
  if constexpr (NARROW) {
    if (cx.gw >= TR && cx.gw < TR + TS) {
      Ctx cs = cx;
      cs.gw = cx.gw - TR;
      linear_prefetch<kW8B128>(linear_prefetch_addr<kW8B128>(cs, w.sh_w13, nullptr, w.sh_w13_s, Nsh, p.h, p.pl.kc_sh13),
                               pf);
    }
  }
  // (narrow: at most one task per wave, which the host checks)
  for (int t = cx.gw; t < TR + TS; t += NARROW ? 1 << 30 : cx.nw) {
    if (t < TR) {
      const int e = t % p.E, c = t / p.E;
      if (J == 1)
        router_task_j<1>(p, w.w_router, u, e, c, cx.lane, wait_u);
      else
        router_task_j<2>(p, w.w_router, u, e, c, cx.lane, wait_u);
      if (p.ho >= 2) ho_count(p.sync, kHoRt + (t & 7), cx.lane);
    } else {
      wait_u();
      linear_task<kW8B128, NARROW ? 1 : 3>(t - TR, cx.lane, w.sh_w13, nullptr, w.sh_w13_s, Nsh, p.h, p.pl.kc_sh13, u,
                                           p.M, p.s.p_sh, &pf, NARROW && pf.on);
      if (p.ho >= 2) ho_count(p.sync, kHoSh + ((t - TR) & 7), cx.lane);
    }
  }
  wait_u();
  if (p.a8) st_u_quant(p, cx, u);
}

// Top-k of one row's router logits (one wave; two experts per lane, v0 for expert lane
// and v1 for expert lane + 64): k rounds of a branch-free wave arg-max on (logit, lower
// id first) keys, so ties go to the lower id and the selections come out in descending
// logit order; the weights are a softmax over the selected k.  Lane j < k returns the
// j-th selection (id -1 and weight 0 for a pad row).
struct TopkLane {
  int id;
  float w;
};

__device__ __forceinline__ TopkLane topk_select(const Params &p, int lane, float v0, float v1, bool live) {
  const int k = p.k, E = p.E;
  if (lane >= E) v0 = -INFINITY;
  if (lane + 64 >= E) v1 = -INFINITY;
  uint64_t k0 = amax_key(v0, lane), k1 = amax_key(v1, lane + 64);
  int myid = -1;
  float myval = -INFINITY;
  for (int j = 0; j < k; j++) {
    const uint64_t best = wave_max_key(k0 > k1 ? k0 : k1, lane);
    if (lane == j) {
      myid = amax_key_index(best);
      myval = amax_key_value(best);
    }
    k0 = k0 == best ? 0ull : k0;
    k1 = k1 == best ? 0ull : k1;
  }
  const float top = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(myval), 0));
  const float ev = lane < k ? expf(myval - top) : 0.f;
  float sum = ev;
  sum += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(sum), 0xB1, 0xF, 0xF, false));   // quad xor 1
  sum += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(sum), 0x4E, 0xF, 0xF, false));   // quad xor 2
  sum += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(sum), 0x141, 0xF, 0xF, false));  // half-row mirror
  return TopkLane{live ? myid : -1, live ? ev / sum : 0.f};
}

// The logits of row m (the router's split-K partials summed in chunk order) for experts
// lane and lane + 64; the logits tap, when given, receives them.
__device__ __forceinline__ void row_logits(const Params &p, int m, int lane, float &v0, float &v1, float *logits_tap) {
  const int E = p.E, nc = p.h / p.pl.kc_router;
  const size_t cs = (size_t)p.M * E;
  const float *lg = p.s.logits + (size_t)m * E;
  v0 = sum_strided(lg + (lane < E ? lane : 0), cs, nc);
  v1 = sum_strided(lg + (lane + 64 < E ? lane + 64 : 0), cs, nc);
  if (logits_tap) {
    if (lane < E) stg(logits_tap + (size_t)m * E + lane, v0);
    if (lane + 64 < E) stg(logits_tap + (size_t)m * E + lane + 64, v1);
  }
}

// Steps of at most one row per wave of a block select in every block: wave m takes row
// m (the same arithmetic in every block, so the same ids everywhere), into R.ids / R.w
// ([M][k]).  No grid barrier is then needed between the router and the experts.
constexpr int kTopkInBlockRows = kWavesPerBlock;

__device__ __forceinline__ void topk_in_block(const Params &p, const Ctx &cx, Routing &R, bool all_live,
                                              float *logits_tap) {
  const int m = cx.wave;
  if (m >= p.M) return;
  float v0, v1;
  row_logits(p, m, cx.lane, v0, v1, logits_tap);
  const TopkLane t = topk_select(p, cx.lane, v0, v1, all_live || ldg(p.pos + m) >= 0);
  if (cx.lane < p.k) {
    R.ids[m * p.k + cx.lane] = t.id;
    R.w[m * p.k + cx.lane] = t.w;
  }
}

// Wider steps: one wave per row over the grid, into the scratch ids / weights; every
// block copies them into its R after the next grid barrier.
__device__ __forceinline__ void topk_in_grid(const Params &p, const Ctx &cx, bool all_live, float *logits_tap) {
  const int m = cx.gw;
  if (m >= p.M) return;
  float v0, v1;
  row_logits(p, m, cx.lane, v0, v1, logits_tap);
  const TopkLane t = topk_select(p, cx.lane, v0, v1, all_live || ldg(p.pos + m) >= 0);
  if (cx.lane < p.k) {
    stg(p.s.tk_ids + (size_t)m * p.k + cx.lane, (int32_t)t.id);
    stg(p.s.tk_w + (size_t)m * p.k + cx.lane, t.w);
  }
}

__device__ __forceinline__ void topk_from_grid(const Params &p, Routing &R) {
  for (int t = tid(); t < p.M * p.k; t += kThreads) {
    R.ids[t] = ldg(p.s.tk_ids + t);
    R.w[t] = ldg(p.s.tk_w + t);
  }
}

// Routing of the current layer in every block's LDS, from the selected ids and weights
// (R.ids / R.w):
// per expert the set of rows that chose it, the distinct-expert list and
// the (row, slot) -> pair map ordered by expert, then by row.
__device__ __forceinline__ void build_routing(const Params &p, const Ctx &cx, Routing &R) {
  const int k = p.k, M = p.M, t0 = tid();
  for (int e = t0; e < 128; e += kThreads) R.rows[e] = 0ull;
  __syncthreads();  // also publishes R.ids / R.w
  for (int t = t0; t < M * k; t += kThreads) {
    const int id = R.ids[t];
    if (id >= 0) atomicOr(&R.rows[id], 1ull << (t / k));
  }
  __syncthreads();
  // counts, starts (exclusive scan in expert order) and the distinct-expert list:
  // wave 0, experts lane and lane + 64
  if (cx.wave == 0) {
    const int lane = cx.lane;
    const int c0 = __popcll(R.rows[lane]), c1 = __popcll(R.rows[lane + 64]);
    R.cnt[lane] = c0;
    R.cnt[lane + 64] = c1;
    // exclusive prefix sums of the counts in expert order, by bit planes (a count is at
    // most M): per plane one ballot, and the bits below the lane counted
    const unsigned long long below = (1ull << lane) - 1ull;
    int s0 = 0, s1 = 0, tot0 = 0, tot1 = 0;
    for (int b = 0; (1 << b) <= M; b++) {
      const unsigned long long m0 = __ballot((c0 >> b) & 1), m1 = __ballot((c1 >> b) & 1);
      s0 += __popcll(m0 & below) << b;
      s1 += __popcll(m1 & below) << b;
      tot0 += __popcll(m0) << b;
      tot1 += __popcll(m1) << b;
    }
    R.start[lane] = s0;
    R.start[lane + 64] = tot0 + s1;
    if (lane == 0) R.np = tot0 + tot1;
    // the distinct experts: in id order for a step of at most 8 rows; wider steps take
    // the experts with more rows first (then by id), so that the round-robin task order
    // gives every wave an even share of the matrix-core experts
    const int cmax = (int)wave_max((float)(c0 > c1 ? c0 : c1));
    if (lane == 0) R.cmax = cmax;
    int at = 0;
    for (int c = M > 8 ? cmax : 0; c >= 0; c--) {
      // c = 0 takes every expert with rows (all of them in id order when M <= 8)
      const bool in0 = c > 0 ? c0 == c : (M <= 8 && c0 > 0), in1 = c > 0 ? c1 == c : (M <= 8 && c1 > 0);
      const unsigned long long b0 = __ballot(in0), b1 = __ballot(in1);
      const int n0 = __popcll(b0);
      if (in0) R.list[at + __popcll(b0 & below)] = lane;
      if (in1) R.list[at + n0 + __popcll(b1 & below)] = lane + 64;
      at += n0 + __popcll(b1);
    }
    if (lane == 0) R.nd = at;
  }
  __syncthreads();
  // pair of (row m, slot): the expert's start plus the rows before m that chose it
  for (int t = t0; t < M * k; t += kThreads) {
    const int id = R.ids[t];
    if (id < 0) continue;
    const int m = t / k;
    const int slot = R.start[id] + __popcll(R.rows[id] & ((1ull << m) - 1ull));
    R.pair[t] = slot;
    R.pair_row[slot] = m;
  }
  __syncthreads();
}

// Shared SwiGLU over all (row, column): z = bf16(swiglu_clamp(gate, up))
__device__ __forceinline__ void st_shared_swiglu(const Params &p, bool all_live, bool wait, const unsigned *hb, int l) {
  const int Is = p.Is, nks = p.h / p.pl.kc_sh13;
  const size_t pstride = (size_t)p.M * 2 * Is;
  const int total = p.M * Is;
  if (wait && bid() * kThreads + (tid() & ~63) < total)
    ho_wait_sum8(p.sync, kHoSh, hb_sum8(hb, kHoSh) + (unsigned)(l + 1) * (unsigned)ho_t_sh(p), tid() & 63);
  for (int idx = bid() * kThreads + tid(); idx < total; idx += gridDim.x * kThreads) {
    const int m = idx / Is, n = idx - m * Is;
    float z = 0.f;
    if (all_live || ldg(p.pos + m) >= 0) {
      const float *b = p.s.p_sh + (size_t)m * 2 * Is;
      const float g = sum_strided(b + n, pstride, nks), u = sum_strided(b + Is + n, pstride, nks);
      z = swiglu_clamp(g, u, p.lim);
    }
    stg(p.s.zsh + idx, (uint16_t)f32_to_bf16(z));
  }
}

template <int NCG>
__device__ __forceinline__ void routed_gate_up_task(const Params &p, const dsl_weights &w, const Routing &R, const uint16_t *u,
                                    int e, int p0, int ce, int tile, int lane) {
  const int i = lane & 15, g = lane >> 4, I = p.I, h = p.h;
  const uint8_t *W = w.ex_w13 + (size_t)e * (2 * I) * (h >> 1);
  const uint8_t *S8 = w.ex_w13_s + (size_t)e * (2 * I) * (h >> 5);
  const uint16_t *xrow[NCG];
  bool xok[NCG];
  v4f acc[2][NCG];
#pragma unroll
  for (int c = 0; c < NCG; c++) {
    const int j = 16 * c + i;
    xok[c] = j < ce;
    xrow[c] = u + (size_t)(xok[c] ? R.pair_row[p0 + j] : 0) * h;
    acc[0][c] = acc[1][c] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  const WStream ws[2] = {wstream<kW4>(W, S8, nullptr, h, tile * 16 + i, 0, g),
                         wstream<kW4>(W, S8, nullptr, h, I + tile * 16 + i, 0, g)};
  if (p.a8 == 2) {
    // A8W4 on the scaled matrix instruction: the same rows' MXFP8 codes and exponents
    const uint8_t *xr8[NCG], *xe[NCG];
#pragma unroll
    for (int c = 0; c < NCG; c++) {
      const size_t r = xok[c] ? (size_t)R.pair_row[p0 + 16 * c + i] : 0;
      xr8[c] = p.s.uq8 + r * h;
      xe[c] = p.s.uqe + r * (h >> 5);
    }
    tiles_a8<2, NCG>(ws, h >> 7, xr8, xe, xok, g, acc);
  } else {
    tiles<kW4, 2, NCG>(ws, h >> 7, xrow, xok, 32 * g, g, acc);
  }
#pragma unroll
  for (int c = 0; c < NCG; c++) {
    const int j = 16 * c + i;
    if (j < ce) {
      uint16_t *z = p.s.zr + (size_t)(p0 + j) * I + tile * 16 + 4 * g;
      const v2u pk = {f32_to_bf16(swiglu_clamp(acc[0][c][0], acc[1][c][0], p.lim)) |
                          (f32_to_bf16(swiglu_clamp(acc[0][c][1], acc[1][c][1], p.lim)) << 16),
                      f32_to_bf16(swiglu_clamp(acc[0][c][2], acc[1][c][2], p.lim)) |
                          (f32_to_bf16(swiglu_clamp(acc[0][c][3], acc[1][c][3], p.lim)) << 16)};
      stg(reinterpret_cast<v2u *>(z), pk);
    }
  }
}

// Down projection of one expert on the matrix unit over NT 16-row tiles of output rows
// (tiles NT tile .. NT tile + NT - 1), for the expert's ce <= 16 NCG pairs.
template <int NCG, int NT>
__device__ __forceinline__ void routed_down_task(const Params &p, const dsl_weights &w, int e, int p0, int ce, int tile, int lane) {
  const int i = lane & 15, g = lane >> 4, I = p.I, h = p.h;
  const uint8_t *W = w.ex_wd + (size_t)e * h * (I >> 1);
  const uint8_t *S8 = w.ex_wd_s + (size_t)e * h * (I >> 5);
  const uint16_t *zin = p.a8 ? p.s.zq : p.s.zr;
  const uint16_t *xrow[NCG];
  bool xok[NCG];
  v4f acc[NT][NCG];
#pragma unroll
  for (int c = 0; c < NCG; c++) {
    const int j = 16 * c + i;
    xok[c] = j < ce;
    xrow[c] = zin + (size_t)(p0 + (xok[c] ? j : 0)) * I;
#pragma unroll
    for (int tt = 0; tt < NT; tt++) acc[tt][c] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  WStream ws[NT];
#pragma unroll
  for (int tt = 0; tt < NT; tt++) ws[tt] = wstream<kW4>(W, S8, nullptr, I, (tile * NT + tt) * 16 + i, 0, g);
  if (p.a8 == 2) {
    // A8W4 on the scaled matrix instruction: the pairs' MXFP8 codes and exponents
    const uint8_t *xr8[NCG], *xe[NCG];
#pragma unroll
    for (int c = 0; c < NCG; c++) {
      const size_t r = (size_t)(p0 + (xok[c] ? 16 * c + i : 0));
      xr8[c] = p.s.zq8 + r * I;
      xe[c] = p.s.zqe + r * (I >> 5);
    }
    tiles_a8<NT, NCG>(ws, I >> 7, xr8, xe, xok, g, acc);
  } else {
    tiles<kW4, NT, NCG>(ws, I >> 7, xrow, xok, 32 * g, g, acc);
  }
#pragma unroll
  for (int tt = 0; tt < NT; tt++)
#pragma unroll
    for (int c = 0; c < NCG; c++) {
      const int j = 16 * c + i;
      if (j < ce) stg(reinterpret_cast<v4f *>(p.s.y + (size_t)(p0 + j) * h + (tile * NT + tt) * 16 + 4 * g), acc[tt][c]);
    }
}

// ------------------------------------------------------------ routed experts on the VALU
//
// An expert that few rows selected is a weight-streaming GEMV: the MXFP4 rows are read
// once and the handful of activation rows are held in registers for the whole task.
// Lane l takes 32-element block l + 64 q of every weight row (q < Q, K = 2048 Q), so
// each load instruction of the wave reads 1 KB of one row contiguously.  A 16-byte
// load holds 32 e2m1 codes; each byte is decoded with its block's E8M0 scale into two
// exact bf16 and multiplied into f32 with a bf16 dot product.  Lane partials of 16
// (row, activation row) outputs are then summed across the wave by a transposing
// butterfly, after which lane L holds the total of output L >> 2.

// acc[v] += dot(weights of one 16-byte load, activations) for one weight row
template <int CE, int Q>
__device__ __forceinline__ void valu_row(const v4u &wv, float scale, const uint32_t (&xq)[CE][16], float *acc) {
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const uint32_t wp0 = cvt_fp4x2_bf16<0>(wv[i], scale), wp1 = cvt_fp4x2_bf16<1>(wv[i], scale);
    const uint32_t wp2 = cvt_fp4x2_bf16<2>(wv[i], scale), wp3 = cvt_fp4x2_bf16<3>(wv[i], scale);
#pragma unroll
    for (int m = 0; m < CE; m++) {
      float a = acc[m];
      a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, wp0), __builtin_bit_cast(v2bf, xq[m][4 * i + 0]), a, false);
      a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, wp1), __builtin_bit_cast(v2bf, xq[m][4 * i + 1]), a, false);
      a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, wp2), __builtin_bit_cast(v2bf, xq[m][4 * i + 2]), a, false);
      a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf, wp3), __builtin_bit_cast(v2bf, xq[m][4 * i + 3]), a, false);
      acc[m] = a;
    }
  }
}

// The lane's activation words of CE rows (blocks lane + 64 q, q < Q): 16 words per block
template <int CE, int Q>
__device__ __forceinline__ void valu_load_x(const uint16_t *const (&rows)[CE], int lane, uint32_t (&xv)[Q][CE][16]) {
#pragma unroll
  for (int q = 0; q < Q; q++)
#pragma unroll
    for (int m = 0; m < CE; m++)
#pragma unroll
      for (int c = 0; c < 4; c++) {
        const v4u t = ld16(rows[m] + 32 * (lane + 64 * q) + 8 * c);
        xv[q][m][4 * c + 0] = t[0]; xv[q][m][4 * c + 1] = t[1];
        xv[q][m][4 * c + 2] = t[2]; xv[q][m][4 * c + 3] = t[3];
      }
}

// E8M0 scales of 16 consecutive weight rows (16 x 64 Q bytes): loaded into registers
// first, written to this wave's LDS once the task's weight loads are in flight (the
// write waits for the scale loads only, which were issued before the weights).
template <int Q>
__device__ __forceinline__ void valu_load_scales(const uint8_t *src, int lane, v4u (&t)[Q]) {
#pragma unroll
  for (int c = 0; c < Q; c++) t[c] = ld16(src + 16 * (lane + 64 * c));
}
template <int Q>
__device__ __forceinline__ void valu_store_scales(uint8_t *dst, int lane, const v4u (&t)[Q]) {
#pragma unroll
  for (int c = 0; c < Q; c++) *reinterpret_cast<v4u *>(dst + 16 * (lane + 64 * c)) = t[c];
}

constexpr int kValuDepth = 16;  // weight rows in flight per wave

// Gate/up of one expert for its CE <= 2 rows over a tile of NR / 2 gate and NR / 2 up
// rows (NR = 32, or 16 for tiles of 8 columns), SwiGLU in the epilogue.  Rows are taken
// in groups of G = 16 / CE (half gate, half up) so one butterfly sums a group's 16
// outputs; gate totals land in lanes 0-31, the matching up totals 32 lanes higher.
template <int CE, int Q, int NR = 32>
__device__ __forceinline__ void routed_gate_up_valu(const Params &p, const dsl_weights &w, const Routing &R,
                                                    const uint16_t *u, int e, int p0, int ce, int tile, int lane,
                                                    uint8_t *sl) {
  constexpr int NB = 64 * Q;   // 32-blocks per weight row
  constexpr int G = 16 / CE;   // rows per group
  constexpr int H = G / 2;     // gate (and up) rows per group
  constexpr int TW = NR / 2;   // gate (and up) rows per task: the tile's columns
  constexpr int SC = NR * Q / 32;  // 1 KB scale chunks per half (TW rows of NB bytes)
  static_assert(NR % G == 0 && SC >= 1, "tile shape");
  constexpr int DEPTH = kValuDepth / Q;
  const int h = p.h, I = p.I;
  const size_t row_bytes = (size_t)h >> 1;
  const uint8_t *W = w.ex_w13 + (size_t)e * (2 * I) * row_bytes;
  const uint8_t *S = w.ex_w13_s + (size_t)e * (2 * I) * NB;
  const uint16_t *rows[CE];
#pragma unroll
  for (int m = 0; m < CE; m++) rows[m] = u + (size_t)R.pair_row[p0 + (m < ce ? m : 0)] * h;
  uint32_t xv[Q][CE][16];
  valu_load_x<CE, Q>(rows, lane, xv);
  v4u scg[SC], scu[SC];
  valu_load_scales<SC>(S + (size_t)(tile * TW) * NB, lane, scg);
  valu_load_scales<SC>(S + (size_t)(I + tile * TW) * NB, lane, scu);
  // weight row r of the task in processing order: group r / G, gate rows then up rows
  auto row_of = [&](int r) -> int {
    const int gi = r / G, rr = r % G;
    return (rr >= H ? I : 0) + tile * TW + gi * H + rr % H;
  };
  v4u ring[DEPTH][Q];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int r = 0; r < DEPTH; r++)
#pragma unroll
    for (int q = 0; q < Q; q++) ring[r][q] = ldw16(W + (size_t)row_of(r) * row_bytes + 16 * (lane + 64 * q));
  __builtin_amdgcn_sched_barrier(0);
  valu_store_scales<SC>(sl, lane, scg);
  valu_store_scales<SC>(sl + TW * NB, lane, scu);
  // row r's scale bytes in LDS, read a row ahead of their use: read where they are used,
  // each LDS round trip stood between two rows' arithmetic
  auto sidx = [&](int r, int q) { return (r % G >= H ? TW * NB : 0) + ((r / G) * H + r % H) * NB + lane + 64 * q; };
  uint32_t sb[Q];
#pragma unroll
  for (int q = 0; q < Q; q++) sb[q] = sl[sidx(0, q)];
  float acc[16];
#pragma unroll
  for (int r = 0; r < NR; r++) {
    const int gi = r / G, rr = r % G, half = rr >= H ? 1 : 0;
    uint32_t sbn[Q];
#pragma unroll
    for (int q = 0; q < Q; q++) sbn[q] = r + 1 < NR ? (uint32_t)sl[sidx(r + 1, q)] : 0u;
    if (rr == 0) {
#pragma unroll
      for (int v = 0; v < 16; v++) acc[v] = 0.f;
    }
    v4u cur[Q];
#pragma unroll
    for (int q = 0; q < Q; q++) cur[q] = ring[r % DEPTH][q];
    if (r + DEPTH < NR) {
#pragma unroll
      for (int q = 0; q < Q; q++)
        ring[r % DEPTH][q] = ldw16(W + (size_t)row_of(r + DEPTH) * row_bytes + 16 * (lane + 64 * q));
    }
#pragma unroll
    for (int q = 0; q < Q; q++) valu_row<CE, Q>(cur[q], e8m0_to_f32(sb[q]), xv[q], acc + (half * H + rr % H) * CE);
    if (rr == G - 1) {
      const float tot = wave_transpose_sum<16>(acc, lane);
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tot), __float_as_uint(tot), false, false);
      const float upv = __uint_as_float(sw[1]);
      const int j = lane >> 2;  // value (half, row, activation row) = (j >> 3, (j & 7) / CE, (j & 7) % CE)
      const int rl = (j & 7) / CE, m = (j & 7) % CE;
      if (lane < 32 && (lane & 3) == 0 && m < ce) {
        stg(p.s.zr + (size_t)(p0 + m) * I + tile * TW + gi * H + rl, (uint16_t)f32_to_bf16(swiglu_clamp(tot, upv, p.lim)));
      }
    }
#pragma unroll
    for (int q = 0; q < Q; q++) sb[q] = sbn[q];
  }
}

// Down projection of one expert for its CE pairs over a tile of NR output rows
template <int CE, int Q, int NR>
__device__ __forceinline__ void routed_down_valu(const Params &p, const dsl_weights &w, int e, int p0, int ce, int tile,
                                                 int lane, uint8_t *sl) {
  constexpr int NB = 64 * Q;
  constexpr int G = 16 / CE;
  static_assert(NR % 16 == 0 && NR * NB <= 4096, "tile rows and their staged scales");
  const int h = p.h, I = p.I;
  const size_t row_bytes = (size_t)I >> 1;
  const uint8_t *W = w.ex_wd + (size_t)e * h * row_bytes;
  const uint8_t *S = w.ex_wd_s + (size_t)e * h * NB;
  const uint16_t *zin = p.a8 ? p.s.zq : p.s.zr;
  const uint16_t *rows[CE];
#pragma unroll
  for (int m = 0; m < CE; m++) rows[m] = zin + (size_t)(p0 + (m < ce ? m : 0)) * I;
  uint32_t xv[Q][CE][16];
  valu_load_x<CE, Q>(rows, lane, xv);
  v4u sc[NR / 16][Q];
#pragma unroll
  for (int b = 0; b < NR / 16; b++) valu_load_scales<Q>(S + (size_t)(tile * NR + 16 * b) * NB, lane, sc[b]);
  constexpr int DEPTH = kValuDepth / Q;
  v4u ring[DEPTH][Q];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int r = 0; r < DEPTH; r++)
#pragma unroll
    for (int q = 0; q < Q; q++) ring[r][q] = ldw16(W + (size_t)(tile * NR + r) * row_bytes + 16 * (lane + 64 * q));
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int b = 0; b < NR / 16; b++) valu_store_scales<Q>(sl + 16 * NB * b, lane, sc[b]);
  // (scale bytes read a row ahead of their use, as in the gate/up tasks)
  uint32_t sb[Q];
#pragma unroll
  for (int q = 0; q < Q; q++) sb[q] = sl[lane + 64 * q];
  float acc[16];
#pragma unroll
  for (int r = 0; r < NR; r++) {
    const int gi = r / G, rr = r % G;
    uint32_t sbn[Q];
#pragma unroll
    for (int q = 0; q < Q; q++) sbn[q] = r + 1 < NR ? (uint32_t)sl[(r + 1) * NB + lane + 64 * q] : 0u;
    if (rr == 0) {
#pragma unroll
      for (int v = 0; v < 16; v++) acc[v] = 0.f;
    }
    v4u cur[Q];
#pragma unroll
    for (int q = 0; q < Q; q++) cur[q] = ring[r % DEPTH][q];
    if (r + DEPTH < NR) {
#pragma unroll
      for (int q = 0; q < Q; q++)
        ring[r % DEPTH][q] = ldw16(W + (size_t)(tile * NR + r + DEPTH) * row_bytes + 16 * (lane + 64 * q));
    }
#pragma unroll
    for (int q = 0; q < Q; q++) valu_row<CE, Q>(cur[q], e8m0_to_f32(sb[q]), xv[q], acc + rr * CE);
    if (rr == G - 1) {
      const float tot = wave_transpose_sum<16>(acc, lane);
      const int j = lane >> 2;  // value (row, pair) = (j / CE, j % CE)
      if ((lane & 3) == 0 && j % CE < ce) stg(p.s.y + (size_t)(p0 + j % CE) * h + tile * NR + gi * G + j / CE, tot);
    }
#pragma unroll
    for (int q = 0; q < Q; q++) sb[q] = sbn[q];
  }
}

// Routed gate/up tasks (selected expert, tile of 16 or 8 rows of gate and of up): task t
// to wave t mod waves.
// NARROW: hidden 4096 and at most 8 rows (one 16-row group).
template <bool NARROW>
__device__ __forceinline__ void st_routed_gate_up(const Params &p, const Ctx &cx, const dsl_weights &w, const Routing &R,
                                  const uint16_t *u, uint8_t *sl) {
  const int qv = NARROW ? 2 : p.h == 2048 ? 1 : p.h == 4096 ? 2 : 0;  // VALU path: K = 2048 q
  // every expert on the VALU path at K = 4096: tiles of 8 columns (32 KB tasks, twice as
  // many).  A last round of tasks that only some waves get then ends twice as soon, and
  // the finer tasks measured faster than splitting only that round.
  const bool halves = qv == 2 && R.cmax <= 2;
  const int tiles_n = p.I >> (halves ? 3 : 4);
  const int T = R.nd * tiles_n;
  for (int t = cx.gw; t < T; t += cx.nw) {
    // wave-uniform: keep them (and the addresses built on them) in scalar registers
    const int tu = __builtin_amdgcn_readfirstlane(t);
    const int q = tu / tiles_n, tile = tu - q * tiles_n;
    const int e = __builtin_amdgcn_readfirstlane(R.list[q]);
    const int ce = __builtin_amdgcn_readfirstlane(R.cnt[e]), p0 = __builtin_amdgcn_readfirstlane(R.start[e]);
    const int ncg = NARROW ? 1 : (ce + 15) >> 4;
    if (qv && ce <= 2) {
      if (!NARROW && qv == 1) {
        if (ce == 1) routed_gate_up_valu<1, 1>(p, w, R, u, e, p0, ce, tile, cx.lane, sl);
        else routed_gate_up_valu<2, 1>(p, w, R, u, e, p0, ce, tile, cx.lane, sl);
      } else if (halves) {
        if (ce == 1) routed_gate_up_valu<1, 2, 16>(p, w, R, u, e, p0, ce, tile, cx.lane, sl);
        else routed_gate_up_valu<2, 2, 16>(p, w, R, u, e, p0, ce, tile, cx.lane, sl);
      } else {
        if (ce == 1) routed_gate_up_valu<1, 2>(p, w, R, u, e, p0, ce, tile, cx.lane, sl);
        else routed_gate_up_valu<2, 2>(p, w, R, u, e, p0, ce, tile, cx.lane, sl);
      }
    } else if (ncg == 1)
      routed_gate_up_task<1>(p, w, R, u, e, p0, ce, tile, cx.lane);
    else if (ncg == 2)
      routed_gate_up_task<2>(p, w, R, u, e, p0, ce, tile, cx.lane);
    else
      routed_gate_up_task<3>(p, w, R, u, e, p0, ce, tile, cx.lane);
  }
}

// Routed down tasks (expert, tile of TR output rows), task t to wave t mod waves
// NARROW: expert inter other than 4096 and at most 8 rows.
template <int TR, bool NARROW>
__device__ __forceinline__ void st_routed_down(const Params &p, const Ctx &cx, const dsl_weights &w, const Routing &R,
                                               uint8_t *sl) {
  const int tiles_n = p.h / TR;
  const int T = R.nd * tiles_n;
  const int qv = p.I == 2048 ? 1 : !NARROW && p.I == 4096 ? 2 : 0;  // VALU path: K = 2048 q
  for (int t = cx.gw; t < T; t += cx.nw) {
    const int q = t / tiles_n, tile = t - q * tiles_n;
    // wave-uniform: keep them (and the addresses built on them) in scalar registers
    const int e = __builtin_amdgcn_readfirstlane(R.list[q]);
    const int ce = __builtin_amdgcn_readfirstlane(R.cnt[e]), p0 = __builtin_amdgcn_readfirstlane(R.start[e]);
    const int ncg = NARROW ? 1 : (ce + 15) >> 4;
    if (qv == 1 && ce <= 4) {
      if (ce == 1) routed_down_valu<1, 1, TR>(p, w, e, p0, ce, tile, cx.lane, sl);
      else if (ce == 2) routed_down_valu<2, 1, TR>(p, w, e, p0, ce, tile, cx.lane, sl);
      else routed_down_valu<4, 1, TR>(p, w, e, p0, ce, tile, cx.lane, sl);
    } else if (qv == 2 && ce <= 2) {
      if (ce == 1) routed_down_valu<1, 2, TR>(p, w, e, p0, ce, tile, cx.lane, sl);
      else routed_down_valu<2, 2, TR>(p, w, e, p0, ce, tile, cx.lane, sl);
    } else if (ncg == 1) {
      routed_down_task<1, TR / 16>(p, w, e, p0, ce, tile, cx.lane);
    } else if (ncg == 2) {
      routed_down_task<2, TR / 16>(p, w, e, p0, ce, tile, cx.lane);
    } else {
      routed_down_task<3, TR / 16>(p, w, e, p0, ce, tile, cx.lane);
    }
  }
}

// Shared down partials, then the routed down tasks: tiles of 16 output rows for a few
// rows (more tasks to spread over the waves), 32 when the step is wide (each task's
// activation rows are then read once per 32 weight rows).
template <bool NARROW>
__device__ __forceinline__ void st_down(const Params &p, const Ctx &cx, const dsl_weights &w, const Routing &R,
                                        uint8_t *sl) {
  const int TS = (p.h >> 4) * (p.Is / p.pl.kc_shd);
  for (int t = cx.gw; t < TS; t += NARROW ? 1 << 30 : cx.nw)  // (narrow: at most one task per wave)
    linear_task<kW8B128, NARROW ? 1 : 3>(t, cx.lane, w.sh_wd, nullptr, w.sh_wd_s, p.h, p.Is, p.pl.kc_shd, p.s.zsh, p.M,
                                         p.s.p_shd);
  if (!NARROW && p.M > 8)
    st_routed_down<32, NARROW>(p, cx, w, R, sl);
  else
    st_routed_down<16, NARROW>(p, cx, w, R, sl);
}

// m = shared + sum_j w_j y_j in float32 (shared first, slots in emission order);
// MoE steps write bf16(m), full steps bf16(hres + m).
__device__ __forceinline__ void st_combine_out(const Params &p, const Routing &R, bool moe_mode, bool last, uint16_t *dst) {
  const int h = p.h, k = p.k, nks = p.Is / p.pl.kc_shd;
  const size_t pstride = (size_t)p.M * h;
  const int total = p.M * h;
  for (int idx = bid() * kThreads + tid(); idx < total; idx += gridDim.x * kThreads) {
    const int m = idx / h, n = idx - m * h;
    const bool live = moe_mode || ldg(p.pos + m) >= 0;
    float mo = 0.f;
    if (live) {
      float yv[8];
#pragma unroll
      for (int j = 0; j < 8; j++) yv[j] = j < k ? ldg(p.s.y + (size_t)R.pair[m * k + j] * h + n) : 0.f;
      mo = sum_strided(p.s.p_shd + idx, pstride, nks);
#pragma unroll
      for (int j = 0; j < 8; j++)
        if (j < k) mo = fmaf(R.w[m * k + j], yv[j], mo);
    }
    if (moe_mode) {
      stg(dst + idx, live ? (uint16_t)f32_to_bf16(mo) : (uint16_t)0);
    } else {
      stg(dst + idx, live ? (uint16_t)f32_to_bf16(bf16_to_f32(ldg(p.s.hres + idx)) + mo) : (uint16_t)0);
      if (last && p.taps.moe_out) stg((uint16_t *)p.taps.moe_out + idx, live ? (uint16_t)f32_to_bf16(mo) : (uint16_t)0);
    }
  }
}

// The combine folded into the down stage (M <= 8).  Both loops of st_down hand task t to
// wave t mod waves, and a task's 16 output columns are tile t mod (h / 16), so when the
// tile count divides the wave count every task of a wave lies in the tile gw mod (h / 16).
// Each wave drains its stores and counts once on the counter of its 32-column group (two
// tiles: one 128-byte line of every partial row, so no line is read before its last
// write); the wave that counts last combines the group's columns for every row, with
// st_combine_out's arithmetic in its order, and no grid barrier and row stage are needed
// between down and combine.  Every wave counts, with tasks or not, so a group takes
// 2 * waves / (h / 16) counts per layer; `cb_base` holds each wave's group counter before
// the layer, read at the start of the launch like the t_quant fold's.
constexpr int kCbGroups = 128;

__device__ __forceinline__ bool cb_fold(const Params &p) {
  const int ntile = p.h >> 4, nw = (int)gridDim.x * kWavesPerBlock;
  // (the last wave stores two bf16 columns at a time)
  const bool al = ((uintptr_t)p.out & 3u) == 0 && ((uintptr_t)p.taps.moe_out & 3u) == 0;
  return p.M <= 8 && (p.h & 31) == 0 && ntile > 0 && nw % ntile == 0 && (p.h >> 5) <= kCbGroups && al;
}

__device__ __forceinline__ int cb_group(const Params &p, const Ctx &cx) { return (cx.gw % (p.h >> 4)) >> 1; }

// The last wave of group g: columns 32 g .. 32 g + 32 of every row.  Lane l takes columns
// 32 g + 2 (l % 16) and + 1 of rows l / 16 and l / 16 + 4; live[i] is row l / 16 + 4 i's.
__device__ __forceinline__ void cb_group_combine(const Params &p, const Routing &R, bool moe_mode, bool last,
                                                 uint16_t *dst, int g, int lane, const bool live[2]) {
  const int h = p.h, k = p.k, nks = p.Is / p.pl.kc_shd;
  const size_t pstride = (size_t)p.M * h;
  const int n = 32 * g + 2 * (lane & 15);
#pragma unroll
  for (int i = 0; i < 2; i++) {
    const int m = (lane >> 4) + 4 * i;
    if (m >= p.M) continue;
    const size_t idx = (size_t)m * h + n;
    float mo[2] = {0.f, 0.f};
    uint32_t hr = 0;
    if (live[i]) {
      float2 yv[8];
#pragma unroll
      for (int j = 0; j < 8; j++) yv[j] = j < k ? ld_f2(p.s.y + (size_t)R.pair[m * k + j] * h + n) : make_float2(0.f, 0.f);
      if (!moe_mode) hr = ldg(reinterpret_cast<const uint32_t *>(p.s.hres + idx));
      load_sum_f32<2>(p.s.p_shd + idx, pstride, nks, mo);
#pragma unroll
      for (int j = 0; j < 8; j++)
        if (j < k) {
          const float wj = R.w[m * k + j];
          mo[0] = fmaf(wj, yv[j].x, mo[0]);
          mo[1] = fmaf(wj, yv[j].y, mo[1]);
        }
    }
    const uint32_t mob = live[i] ? f32_to_bf16(mo[0]) | (f32_to_bf16(mo[1]) << 16) : 0u;
    if (moe_mode) {
      stg(reinterpret_cast<uint32_t *>(dst + idx), mob);
    } else {
      const uint32_t ob = live[i] ? f32_to_bf16(bf16_to_f32(hr & 0xFFFFu) + mo[0]) |
                                        (f32_to_bf16(bf16_to_f32(hr >> 16) + mo[1]) << 16)
                                  : 0u;
      stg(reinterpret_cast<uint32_t *>(dst + idx), ob);
      if (last && p.taps.moe_out) stg(reinterpret_cast<uint32_t *>((uint16_t *)p.taps.moe_out + idx), mob);
    }
  }
}

// After this wave's st_down tasks
__device__ __forceinline__ void cb_count_combine(const Params &p, const Ctx &cx, const Routing &R, bool moe_mode,
                                                 bool last, uint16_t *dst, unsigned *cb_base) {
  const int g = cb_group(p, cx);
  const unsigned per = 2u * (unsigned)(cx.nw / (p.h >> 4));
  const unsigned base = cb_base[cx.wave];
  __builtin_amdgcn_s_waitcnt(0);  // this wave's y and partial stores are at the coherence point
  unsigned old = 0;
  if (cx.lane == 0)
    old = __hip_atomic_fetch_add(gptr(&p.sync->cb[g][0]), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  old = (unsigned)__builtin_amdgcn_readfirstlane(old);
  if (cx.lane == 0) cb_base[cx.wave] = base + per;  // (this wave's own slot)
  if (old - base != per - 1u) return;
  asm volatile("" ::: "memory");  // the group's loads stay after the count
  bool live[2];
#pragma unroll
  for (int i = 0; i < 2; i++) {
    const int m = (cx.lane >> 4) + 4 * i;
    live[i] = moe_mode || (m < p.M && ldg(p.pos + m) >= 0);
  }
  cb_group_combine(p, R, moe_mode, last, dst, g, cx.lane, live);
  // the group's output columns are out: count them for the next chained layer's input norm
  if (p.ho >= 2 && !last) ho_count(p.sync, kHoO + (g & 7), cx.lane);
}

// Each wave's combine group counter, read before its block's first arrival (no down wave
// of the launch can count before every block has arrived at the first barrier)
__device__ __forceinline__ unsigned cb_read_base(const Params &p, const Ctx &cx) {
  return cb_fold(p) ? __hip_atomic_load(gptr(&p.sync->cb[cb_group(p, cx)][0]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                    : 0u;
}

// ============================================================== the persistent launch

// Launch parameters are read per stage through the constant address space: the empty
// asm makes each stage's pointer opaque, so its scalar loads are not merged with (and
// kept live from) another stage's, and nothing uniform stays in registers across the
// launch.  The descriptors (the kernel argument, the weight table) are read-only for
// the whole launch.
typedef const Params __attribute__((address_space(4))) KParams;
typedef const dsl_weights __attribute__((address_space(4))) KWeights;

__device__ __forceinline__ KParams *kparams() {
  KParams *kp = (KParams *)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(kp));
  return kp;
}

// a descriptor copied in 64-bit words by scalar loads
template <typename T>
__device__ __forceinline__ T kload(const __attribute__((address_space(4))) T *src) {
  static_assert(sizeof(T) % 8 == 0, "descriptor size");
  T v;
  const __attribute__((address_space(4))) uint64_t *s = (const __attribute__((address_space(4))) uint64_t *)src;
  uint64_t *d = reinterpret_cast<uint64_t *>(&v);
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 8); i++) d[i] = s[i];
  return v;
}

// Every member of Scratch is a pointer into one allocation
__device__ __forceinline__ Scratch shift_scratch(Scratch s, long long off) {
  static_assert(sizeof(Scratch) % 8 == 0, "scratch descriptor");
  uint64_t *w = reinterpret_cast<uint64_t *>(&s);
#pragma unroll
  for (int i = 0; i < (int)(sizeof(Scratch) / 8); i++) w[i] += (uint64_t)off;
  return s;
}

// Layer l's view: its weights, its cache, its own scratch (each layer writes its
// scratch once per launch), its input (x, or the previous layer's output in this
// layer's scratch) and where its output goes (out, or the next layer's scratch).
struct StageArgs {
  Params p;
  dsl_weights w;
  dsl_kv kv;
  const uint16_t *xin;
  uint16_t *xout;
};

__device__ __forceinline__ StageArgs stage_args(int l) {
  KParams *kp = kparams();
  StageArgs a;
  a.p = kload(kp);
  a.w = kload((KWeights *)kp->w + l);
  a.kv = kload(&kp->kv[l]);
  const Scratch s0 = a.p.s;
  a.p.s = shift_scratch(s0, l * a.p.s_stride);
  a.xin = l == 0 ? a.p.x : a.p.s.xin;
  a.xout = l == a.p.n_layers - 1 ? a.p.out : shift_scratch(s0, (l + 1) * a.p.s_stride).xin;
  return a;
}

// With tracing on, every block stamps the device wall clock at the start of the
// launch, on arriving at and on leaving every grid barrier, at a few points inside the
// MoE and at the end: buf[mark][block].
constexpr int kTraceMarks = 256;  // stamps per block the trace buffer holds

struct Tracer {
  unsigned long long *buf = nullptr;
  int n = 0;
  __device__ __forceinline__ void mark() {
    if (buf && tid() == 0 && n < kTraceMarks) stg(buf + (size_t)n * gridDim.x + bid(), (unsigned long long)wall_clock64());
    n++;
  }
};

// The grid barrier's thread is the first of the last wave: linear_prefetch leaves that
// wave without loads in flight.  SYNC_PF issues the next stage's weight loads (ISSUE)
// between the drain and the meeting.
constexpr unsigned kBarrierThread = kThreads - kWave;

#define SYNC_PF(ISSUE)        \
  do {                        \
    __syncthreads();          \
    tr.mark();                \
    barrier_drain();          \
    ISSUE;                    \
    grid_barrier_meet(sw, nb, &bar_next, kBarrierThread); \
    tr.mark();                \
  } while (0)
#define SYNC() SYNC_PF((void)0)
// A grid barrier, or (where hand-offs replace it) the trace's two stamps only, so that the
// stamps keep their numbering either way
#define SYNC_IF(C)      \
  do {                  \
    if (C) {            \
      SYNC();           \
    } else {            \
      tr.mark();        \
      tr.mark();        \
    }                   \
  } while (0)

#define STAGE(l) const StageArgs A_ = stage_args(l); const Params &p = A_.p; const dsl_weights &w = A_.w; \
  const dsl_kv &kv = A_.kv; const Ctx cx = make_ctx(); (void)p; (void)w; (void)kv; (void)cx

// Two instantiations: the general one, and NARROW for steps of at most 8 rows at the
// full-size dimensions (hidden 4096, q and o rank 1024, head dim 512, expert inter other
// than 4096), which compiles in only the variants those use and, since the t_quant and
// combine folds always apply there, neither of the stages they replace (narrow_ok checks
// all of it on the host).  The narrow kernel is under a third of the general one's code
// with under half the spills, and takes about 6 us less per launch at 6 rows.
template <bool NARROW>
__global__ void __launch_bounds__(kThreads, 1) dsl_layer_kernel(Params p_arg) {
  (void)p_arg;
  __shared__ Routing R;
  __shared__ float red[16];
  __shared__ __attribute__((aligned(16))) uint8_t wave_lds[kWavesPerBlock][4096];  // per-wave scale staging
  __shared__ unsigned bar_next;  // number of the next grid barrier (the barrier thread's)
  __shared__ unsigned tq_base[kWavesPerBlock];  // each wave's wo_a group counter before this layer
  __shared__ unsigned cb_base[kWavesPerBlock];  // each wave's combine group counter before this layer
  const unsigned nb = gridDim.x;
  __shared__ unsigned ho_base[kHoSlots];         // hand-off counters before this launch
  __shared__ unsigned rt_flag;                   // layer + 1 once this block has seen every router task
  __shared__ unsigned bar_fence;                 // the barrier every block arrives at once it has read the bases
  int mode, n_layers, a8, ho, Mrows;
  SyncWords *sw;
  Tracer tr;
  {
    KParams *kp = kparams();
    mode = kp->mode;
    n_layers = kp->n_layers;
    a8 = kp->a8;
    ho = kp->ho;
    Mrows = kp->M;
    sw = kp->sync;
    tr.buf = kp->trace;
  }
  // the barrier's thread reads the barrier base (the last wave has no work on the first
  // stage's critical path)
  if (tid() == kBarrierThread) bar_next = barrier_base(sw) + 1u;
  // the hand-off counters' values before this launch, read before the block's first arrival:
  // no producer of the launch counts before every block has arrived at the first barrier
  if (ho && tid() < kHoSlots)
    ho_base[tid()] = __hip_atomic_load(gptr(&sw->ho[tid()][0]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (tid() == 0) rt_flag = 0u;
  const bool moe_mode = mode == kModeMoe;
  // full hand-offs (ho >= 2) also replace the barriers after wqkv, wo_b, the FFN norm and
  // (steps whose top-k runs in every block, bf16 expert inputs) the router
  const bool ho2 = ho >= 2, ho_router = ho2 && Mrows <= kTopkInBlockRows && !a8;
  // no grid barrier after the router either when the top-k runs over the grid: its row
  // waves wait for the router tasks' counts and count their rows, for which every block
  // then waits
  const bool ho_topk = ho2 && !a8;
  // the grid barrier after the attention-input norm is replaced by a row hand-off too
  // (with a block for every q, kv and key-offset row): its other role, that no block reads
  // a counter's starting value after a producer has counted on it, passes to an early
  // arrival of every block at a barrier that the first producers (the norm rows and the
  // key-offset rows, which wait on nothing else) wait for before counting
  const bool fenced = ho2 && (int)nb >= 3 * Mrows;
  // chained layers hand the layer output to the next layer's input norm when the combine
  // is folded (its last waves count the output's column groups)
  bool out_ho = false;
  tr.mark();
  for (int l = 0; l < n_layers; l++) {
    const bool last = l == n_layers - 1;
    if (!moe_mode) {
      // The first weights of wqkv, wq_b, wo_a and wo_b are loaded between the drain and
      // the grid barrier before them (SYNC_PF), at addresses taken at the start of the
      // stage before, when its launch parameters are at hand.
      PreA pf_wqkv = pre_none();
      PreAddr pa;
      {
        STAGE(l);
        pa = linear_prefetch_addr<kW8T32>(cx, w.wqkv, w.wqkv_s, nullptr, p.qr + p.D, p.h, p.pl.kc_qkv);
        if (l == 0 && cx.lane == 0) {
          // before this block's first arrival, like the barrier base: no wo_a task of the
          // launch can count before every block has arrived at the first barrier
          const int j = tq_group(p, cx);
          tq_base[cx.wave] = j >= 0 && j < kTqGroups
                                 ? __hip_atomic_load(gptr(&p.sync->tq[j][0]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                 : 0u;
          cb_base[cx.wave] = cb_read_base(p, cx);
        }
        if (fenced && l == 0) {
          __syncthreads();  // this block's starting values are all read (ho_base, tq_base, cb_base)
          if (tid() == kBarrierThread) grid_barrier_arrive(sw, nb, &bar_next, &bar_fence);
          __syncthreads();
        }
        const unsigned fence = bar_fence;
        const uint16_t *xin = A_.xin;
        // (layers after the first, when the one before handed its output off: its 32-column
        // groups, counted per layer)
        const unsigned wait_out = l > 0 && out_ho ? (unsigned)l * (unsigned)(p.h >> 5) : 0u;
        if constexpr (NARROW) {
          st_attn_norm_e<8>(p, w, kv, xin, red, fenced, fence, wait_out, ho_base);
        } else {
          switch (row_elems(p.h)) {
            case 1: st_attn_norm_e<1>(p, w, kv, xin, red, fenced, fence, wait_out, ho_base); break;
            case 2: st_attn_norm_e<2>(p, w, kv, xin, red, fenced, fence, wait_out, ho_base); break;
            case 4: st_attn_norm_e<4>(p, w, kv, xin, red, fenced, fence, wait_out, ho_base); break;
            case 8: st_attn_norm_e<8>(p, w, kv, xin, red, fenced, fence, wait_out, ho_base); break;
            default: st_attn_norm_e<16>(p, w, kv, xin, red, fenced, fence, wait_out, ho_base); break;
          }
        }
      }
      if (fenced) {
        linear_prefetch<kW8T32>(pa, pf_wqkv);
        tr.mark();
        tr.mark();
      } else {
        SYNC_PF(linear_prefetch<kW8T32>(pa, pf_wqkv));
      }
      {
        STAGE(l);
        if (ho2)
          st_wqkv_ho<NARROW ? 1 : 3, NARROW>(p, cx, w, pf_wqkv, fenced, ho_base, l);
        else
          linear_all_pre<kW8T32, NARROW ? 1 : 3, NARROW>(cx, w.wqkv, w.wqkv_s, nullptr, p.qr + p.D, p.h, p.pl.kc_qkv, p.s.xb,
                                                 p.M, p.s.p_qkv, pf_wqkv);
      }
      SYNC_IF(!ho2);
      PreA pf_wq_b = pre_none();
      {
        STAGE(l);
        pa = linear_prefetch_addr<kW8T32>(cx, w.wq_b, w.wq_b_s, nullptr, p.H * p.D, p.qr, p.pl.kc_qb);
        st_qkv_post<NARROW>(p, w, kv, red, &wave_lds[0][0], ho_base, l, fenced, bar_fence);
      }
      // With hand-offs ("Mono decode layer for DeepSeek-V4.1-Flash on MI355X", Design: the
      // stages pass data between CTAs through tagged flags) no grid barrier separates
      // qkv_post, wq_b, the attention and wo_a: each consumer waits on the counters of its
      // own producers (every q row; its head's wq_b tasks and the step's records; its K
      // chunk's heads), and the next weights are loaded as soon as a wave is free.
      if (ho) {
        linear_prefetch<kW8T32>(pa, pf_wq_b);
        tr.mark();
        tr.mark();
      } else {
        SYNC_PF(linear_prefetch<kW8T32>(pa, pf_wq_b));
      }
      {
        STAGE(l);
        if (ho)
          st_wq_b_ho<NARROW ? 1 : 3, NARROW>(p, cx, w, pf_wq_b, ho_base, l);
        else
          linear_all_pre<kW8T32, NARROW ? 1 : 3, NARROW>(cx, w.wq_b, w.wq_b_s, nullptr, p.H * p.D, p.qr, p.pl.kc_qb, p.s.qb,
                                                 p.M, p.s.p_q, pf_wq_b);
      }
      SYNC_IF(!ho);
      PreA pf_wo_a = pre_none();
      {
        STAGE(l);
        pa = linear_prefetch_addr<kW8T32>(cx, w.wo_a, w.wo_a_s, nullptr, p.orr, p.H * p.D, p.pl.kc_oa);
        float *lds = reinterpret_cast<float *>(&wave_lds[0][0]);
        if constexpr (NARROW) {
          st_attention_narrow(p, cx, kv, lds, ho_base, l);
        } else {
          switch (p.D) {
            case 64: st_attention_v<1>(p, cx, kv, lds, ho_base, l); break;
            case 128: st_attention_v<2>(p, cx, kv, lds, ho_base, l); break;
            case 256: st_attention_v<4>(p, cx, kv, lds, ho_base, l); break;
            default: st_attention_v<8>(p, cx, kv, lds, ho_base, l); break;
          }
        }
      }
      if (ho) {
        linear_prefetch<kW8T32>(pa, pf_wo_a);
        tr.mark();
        tr.mark();
      } else {
        SYNC_PF(linear_prefetch<kW8T32>(pa, pf_wo_a));
      }
      PreA pf_wo_b = pre_none();
      bool fold;
      {
        STAGE(l);
        fold = NARROW || tq_fold(p);  // (the host picks the narrow kernel only where it holds)
        if (fold) {
          pa = linear_prefetch_addr<kW8T32>(cx, w.wo_b, w.wo_b_s, nullptr, p.h, p.orr, p.pl.kc_ob);
          st_wo_a_fold(p, cx, w, pf_wo_a, tq_base[cx.wave], ho_base, l);
        } else if (ho) {
          st_wo_a_ho<NARROW ? 1 : 3>(p, cx, w, pf_wo_a, ho_base, l);
        } else {
          linear_all_pre<kW8T32, NARROW ? 1 : 3, NARROW>(cx, w.wo_a, w.wo_a_s, nullptr, p.orr, p.H * p.D, p.pl.kc_oa, p.s.ob, p.M,
                                                 p.s.p_t, pf_wo_a);
        }
      }
      if (!fold) {
        SYNC();
        {
          STAGE(l);
          pa = linear_prefetch_addr<kW8T32>(cx, w.wo_b, w.wo_b_s, nullptr, p.h, p.orr, p.pl.kc_ob);
          if constexpr (NARROW) {
            st_t_quant_e<2>(p);
          } else {
            switch (row_elems(p.orr)) {
              case 1: st_t_quant_e<1>(p); break;
              case 2: st_t_quant_e<2>(p); break;
              case 4: st_t_quant_e<4>(p); break;
              case 8: st_t_quant_e<8>(p); break;
              default: st_t_quant_e<16>(p); break;
            }
          }
        }
      }
      if (ho2 && fold) {
        linear_prefetch<kW8T32>(pa, pf_wo_b);
        tr.mark();
        tr.mark();
      } else {
        SYNC_PF(linear_prefetch<kW8T32>(pa, pf_wo_b));
      }
      {
        STAGE(l);
        // (this wave's own slot, read in wo_a)
        if (fold && cx.lane == 0) tq_base[cx.wave] += 2u * (unsigned)((p.H * p.D) / p.pl.kc_oa);
        if (ho2)
          st_wo_b_ho<NARROW ? 1 : 3, NARROW>(p, cx, w, pf_wo_b, ho_base, l, fold);
        else
          linear_all_pre<kW8T32, NARROW ? 1 : 3, NARROW>(cx, w.wo_b, w.wo_b_s, nullptr, p.h, p.orr, p.pl.kc_ob, p.s.tb, p.M,
                                                 p.s.p_a, pf_wo_b);
      }
      SYNC_IF(!ho2);
      {
        STAGE(l);
        const uint16_t *xin = A_.xin;
        if constexpr (NARROW) {
          st_ffn_norm_e<8>(p, w, xin, last, red, ho_base, l);
        } else {
          switch (row_elems(p.h)) {
            case 1: st_ffn_norm_e<1>(p, w, xin, last, red, ho_base, l); break;
            case 2: st_ffn_norm_e<2>(p, w, xin, last, red, ho_base, l); break;
            case 4: st_ffn_norm_e<4>(p, w, xin, last, red, ho_base, l); break;
            case 8: st_ffn_norm_e<8>(p, w, xin, last, red, ho_base, l); break;
            default: st_ffn_norm_e<16>(p, w, xin, last, red, ho_base, l); break;
          }
        }
      }
      if (mode == kModeAttn) {
        tr.mark();
        return;
      }
      SYNC_IF(!ho2);
    }
    {
      STAGE(l);
      // (a MoE step's first stage: before this block's first arrival)
      if (moe_mode && l == 0 && cx.lane == 0) cb_base[cx.wave] = cb_read_base(p, cx);
      st_router_shared<NARROW>(p, cx, w, moe_mode ? p.x : p.s.u, ho_base, l);
    }
    SYNC_IF(!ho_topk);
    {
      STAGE(l);
      if (NARROW || p.M <= kTopkInBlockRows) {
        // no grid barrier between the router and the experts: every block selects the
        // experts of every row itself (with hand-offs, once every router task has stored
        // its partial logits)
        // The router counters are polled by one wave per block, which then raises the
        // block's flag in LDS for its row waves: with every row wave of every block polling
        // them (M x 256 pollers), the polls delayed the counters' own increments by several
        // microseconds.
        if (ho_router && cx.wave < p.M) {
          if (cx.wave == 0) {
            ho_wait_sum8(p.sync, kHoRt, hb_sum8(ho_base, kHoRt) + (unsigned)(l + 1) * (unsigned)ho_t_rt(p), cx.lane);
            if (cx.lane == 0) __hip_atomic_store(&rt_flag, (unsigned)(l + 1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          } else if (cx.lane == 0) {
            // wave 0 of the block always gets here (every step has a row 0), so this ends
            while (__hip_atomic_load(&rt_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != (unsigned)(l + 1))
              __builtin_amdgcn_s_sleep(1);
          }
          asm volatile("" ::: "memory");  // the logit loads stay after the wait
        }
        topk_in_block(p, cx, R, moe_mode, last && bid() == 0 ? p.taps.logits : nullptr);
        tr.mark();
        tr.mark();
      } else {
        if (ho_topk && cx.gw < p.M) {
          ho_wait_sum8(p.sync, kHoRt, hb_sum8(ho_base, kHoRt) + (unsigned)(l + 1) * (unsigned)ho_t_rt(p), cx.lane);
          asm volatile("" ::: "memory");  // the logit loads stay after the wait
        }
        topk_in_grid(p, cx, moe_mode, last ? p.taps.logits : nullptr);
        if (ho_topk) {
          if (cx.gw < p.M) ho_count(p.sync, kHoTk, cx.lane);
          if (cx.wave == 0) ho_wait(p.sync, kHoTk, ho_base[kHoTk] + (unsigned)(l + 1) * (unsigned)p.M, cx.lane);
          __syncthreads();
          tr.mark();
          tr.mark();
        } else {
          SYNC();
        }
        topk_from_grid(p, R);
      }
      build_routing(p, cx, R);
      if (bid() == 0 && p.taps.layer_ids)
        for (int t = tid(); t < p.M * p.k; t += kThreads)
          stg(p.taps.layer_ids + (size_t)l * p.M * p.k + t, R.ids[t]);
      if (bid() == 0 && last) {
        for (int t = tid(); t < p.M * p.k; t += kThreads) {
          if (p.taps.topk_ids) stg(p.taps.topk_ids + t, R.ids[t]);
          if (p.taps.topk_w) stg(p.taps.topk_w + t, R.w[t]);
        }
      }
    }
    tr.mark();
    {
      STAGE(l);
      st_routed_gate_up<NARROW>(p, cx, w, R, p.a8 ? p.s.uq : moe_mode ? p.x : p.s.u, wave_lds[cx.wave]);
      // the shared SwiGLU, off the critical path: its reader, the shared down projection,
      // comes after the next grid barrier
      st_shared_swiglu(p, moe_mode, ho_topk, ho_base, l);
    }
    SYNC();
    if (a8) {
      {
        STAGE(l);
        st_z_quant(p, R);
      }
      SYNC();
    }
    bool cfold;
    {
      STAGE(l);
      cfold = NARROW || cb_fold(p);  // (likewise)
      out_ho = fenced && cfold && !moe_mode;
      st_down<NARROW>(p, cx, w, R, wave_lds[cx.wave]);
      if (cfold) cb_count_combine(p, cx, R, moe_mode, last, A_.xout, cb_base);
    }
    if (!cfold) {
      SYNC();
      {
        STAGE(l);
        st_combine_out(p, R, moe_mode, last, A_.xout);
      }
    }
    if (!last) {
      if (out_ho) {
        // the next layer's input comes by hand-off (kHoO); the block's own waves still
        // finish this layer before any starts the next (the LDS tables and areas are reused)
        __syncthreads();
        tr.mark();
        tr.mark();
      } else {
        SYNC();
      }
    }
    tr.mark();
  }
}

#undef STAGE
#undef SYNC
#undef SYNC_IF

}  // namespace dsl

// ============================================================== host runtime

using namespace dsl;

struct WidthScratch {
  void *buf = nullptr;
  size_t bytes = 0;
  long long stride = 0;  // bytes between layers' scratch
  Scratch s{};
};

struct dsl_layer {
  dsl_dims d{};
  int dev = 0, cus = 0, grid = 0, bpc = 0, S = 1;
  int last_kernel = -1;  // instantiation of the most recent launch: 1 narrow, 0 general
  int handoff = 2;       // producer hand-offs where the launch allows them: 2 all, 1 around the
                         // attention only, 0 none (grid barriers); DSL_HANDOFF overrides
  Plan plan{};
  dsl_weights *dw = nullptr;  // device copy of the weight descriptors
  SyncWords *sync = nullptr;
  unsigned long long *trace = nullptr;  // device buffer of kTraceLen stamps when tracing
  WidthScratch wid[DSL_MAX_ROWS + 1];
};

static constexpr int kTraceLen = kTraceMarks;

static thread_local std::string g_err;

static int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

// The same for the library's other sources (dsl_linear.hip)
int dsl::set_error(int code, const char *msg) {
  g_err = msg;
  return code;
}

#define HIPCHK(call)                                                                          \
  do {                                                                                        \
    hipError_t e_ = (call);                                                                   \
    if (e_ != hipSuccess) return fail(DSL_EHIP, "%s failed: %s", #call, hipGetErrorString(e_)); \
  } while (0)

static bool mult(int v, int m) { return v > 0 && v % m == 0; }

// Elements per thread of a row of n over the block (the device's row_elems)
static int row_elems_host(int n) {
  int e = 1;
  while (e * kThreads < n) e <<= 1;
  return e;
}

// The dimensions and widths the narrow kernel instantiation covers: at most 8 rows (the
// in-block top-k, 16-column down tiles, one 16-row group of every linear), 8 elements per
// thread of a hidden row, 2 of a q-rank and of an o-rank row, head dim 512, hidden 4096
// (the VALU gate/up path for K = 4096) and expert inter other than 4096.
static bool narrow_dims(const dsl_dims &d, int M) {
  return M <= 8 && d.hidden == 4096 && row_elems_host(d.q_rank) == 2 && row_elems_host(d.o_rank) == 2 &&
         d.head_dim == 512 && d.inter != 4096;
}

// The narrow kernel also assumes that both folds apply (it has no t_quant or combine
// stage): the conditions of tq_fold and cb_fold for this launch's grid and buffers.
static bool narrow_ok(const dsl_layer *L, const Params &p) {
  if (!narrow_dims(L->d, p.M)) return false;
  const int nw = L->grid * kWavesPerBlock;
  // at most one task per wave in the dense linears, the router and shared gate/up stage and
  // the shared down (the narrow kernel compiles in only a wave's first task of each)
  const int T[] = {((p.qr + p.D) >> 4) * (p.h / p.pl.kc_qkv), ((p.H * p.D) >> 4) * (p.qr / p.pl.kc_qb),
                   (p.orr >> 4) * ((p.H * p.D) / p.pl.kc_oa), (p.h >> 4) * (p.orr / p.pl.kc_ob),
                   p.E * (p.h / p.pl.kc_router) + ((2 * p.Is) >> 4) * (p.h / p.pl.kc_sh13),
                   (p.h >> 4) * (p.Is / p.pl.kc_shd)};
  for (int t : T)
    if (t > nw) return false;
  const int T_oa = (p.orr >> 4) * ((p.H * p.D) / p.pl.kc_oa);
  const bool tq = p.M <= 16 && T_oa <= nw && p.orr / 32 <= kTqGroups;
  const int ntile = p.h >> 4;
  const bool al = ((uintptr_t)p.out & 3u) == 0 && ((uintptr_t)p.taps.moe_out & 3u) == 0;
  const bool cb = p.M <= 8 && (p.h & 31) == 0 && ntile > 0 && nw % ntile == 0 && (p.h >> 5) <= kCbGroups && al;
  return tq && cb;
}

static int validate_dims(const dsl_dims *d) {
  if (d->max_rows < 1 || d->max_rows > DSL_MAX_ROWS)
    return fail(DSL_EUNSUPPORTED, "max_rows %d outside 1..%d", d->max_rows, DSL_MAX_ROWS);
  if (d->n_layers < 1 || d->n_layers > DSL_MAX_LAYERS)
    return fail(DSL_EUNSUPPORTED, "n_layers %d outside 1..%d", d->n_layers, DSL_MAX_LAYERS);
  if (!mult(d->hidden, 128)) return fail(DSL_EUNSUPPORTED, "hidden %d is not a positive multiple of 128", d->hidden);
  if (!mult(d->q_rank, 128)) return fail(DSL_EUNSUPPORTED, "q_rank %d is not a positive multiple of 128", d->q_rank);
  if (!mult(d->o_rank, 128)) return fail(DSL_EUNSUPPORTED, "o_rank %d is not a positive multiple of 128", d->o_rank);
  if (d->head_dim != 64 && d->head_dim != 128 && d->head_dim != 256 && d->head_dim != 512)
    return fail(DSL_EUNSUPPORTED, "head_dim %d not in {64, 128, 256, 512}", d->head_dim);
  if (d->n_heads < 1 || !mult(d->n_heads * d->head_dim, 128))
    return fail(DSL_EUNSUPPORTED, "n_heads*head_dim %d is not a positive multiple of 128", d->n_heads * d->head_dim);
  if (!mult(d->inter, 128)) return fail(DSL_EUNSUPPORTED, "inter %d is not a positive multiple of 128", d->inter);
  if (!mult(d->shared_inter, 128))
    return fail(DSL_EUNSUPPORTED, "shared_inter %d is not a positive multiple of 128", d->shared_inter);
  if (d->n_experts < 1 || d->n_experts > 128)
    return fail(DSL_EUNSUPPORTED, "n_experts %d outside 1..128", d->n_experts);
  if (d->top_k < 1 || d->top_k > 8 || d->top_k > d->n_experts)
    return fail(DSL_EUNSUPPORTED, "top_k %d outside 1..min(8, n_experts)", d->top_k);
  if (d->window < 1) return fail(DSL_EINVAL, "window %d < 1", d->window);
  if (d->swa_width < 0) return fail(DSL_EINVAL, "swa_width %d < 0", d->swa_width);
  if (d->window > 8 * kSplitKeys || d->swa_width > 8 * kSplitKeys)
    return fail(DSL_EUNSUPPORTED, "window %d / swa_width %d: at most %d keys per row (8 splits of %d)", d->window,
                d->swa_width, 8 * kSplitKeys, kSplitKeys);
  if (d->kv_block < 1) return fail(DSL_EINVAL, "kv_block %d < 1", d->kv_block);
  if (d->expert_a8 < 0 || d->expert_a8 > 2) return fail(DSL_EINVAL, "expert_a8 %d is not 0, 1 or 2", d->expert_a8);
  if (!(d->norm_eps >= 0.f) || !(d->swiglu_limit > 0.f))
    return fail(DSL_EINVAL, "norm_eps must be >= 0 and swiglu_limit > 0");
  return 0;
}

static int pick_kc(int K, int target) {
  int kc = K < target ? K : target;
  kc -= kc % 128;
  while (kc > 128 && K % kc) kc -= 128;
  return kc;
}

static size_t layout(const dsl_layer *L, int M, Scratch *s, char *base) {
  const dsl_dims &d = L->d;
  const Plan &pl = L->plan;
  size_t off = 0;
  auto take = [&](size_t bytes) -> char * {
    off = (off + 255) & ~(size_t)255;
    char *p = base ? base + off : nullptr;
    off += bytes;
    return p;
  };
  const size_t h = d.hidden, qr = d.q_rank, D = d.head_dim, HD = (size_t)d.n_heads * d.head_dim, orr = d.o_rank;
  const size_t E = d.n_experts, k = d.top_k, I = d.inter, Is = d.shared_inter, S = L->S, m = M;
  s->xb = (uint16_t *)take(m * h * 2);
  s->p_qkv = (float *)take((h / pl.kc_qkv) * m * (qr + D) * 4);
  s->qb = (uint16_t *)take(m * qr * 2);
  s->p_q = (float *)take((qr / pl.kc_qb) * m * HD * 4);
  s->keyoff = (int64_t *)take(m * (size_t)(d.swa_width > 0 ? d.swa_width : d.window) * 8);
  (void)S;
  s->ob = (uint16_t *)take(m * HD * 2);
  s->p_t = (float *)take((HD / pl.kc_oa) * m * orr * 4);
  s->tb = (uint16_t *)take(m * orr * 2);
  s->p_a = (float *)take((orr / pl.kc_ob) * m * h * 4);
  s->xin = (uint16_t *)take(m * h * 2);
  s->hres = (uint16_t *)take(m * h * 2);
  s->u = (uint16_t *)take(m * h * 2);
  s->logits = (float *)take((h / pl.kc_router) * m * E * 4);
  s->tk_ids = (int32_t *)take(m * k * 4);
  s->tk_w = (float *)take(m * k * 4);
  s->p_sh = (float *)take((h / pl.kc_sh13) * m * 2 * Is * 4);
  s->zsh = (uint16_t *)take(m * Is * 2);
  s->zr = (uint16_t *)take(m * k * I * 2);
  s->y = (float *)take(m * k * h * 4);
  s->p_shd = (float *)take((Is / pl.kc_shd) * m * h * 4);
  s->uq = d.expert_a8 ? (uint16_t *)take(m * h * 2) : nullptr;
  s->zq = d.expert_a8 ? (uint16_t *)take(m * k * I * 2) : nullptr;
  s->uq8 = d.expert_a8 == 2 ? (uint8_t *)take(m * h) : nullptr;
  s->uqe = d.expert_a8 == 2 ? (uint8_t *)take(m * h / 32) : nullptr;
  s->zq8 = d.expert_a8 == 2 ? (uint8_t *)take(m * k * I) : nullptr;
  s->zqe = d.expert_a8 == 2 ? (uint8_t *)take(m * k * I / 32) : nullptr;
  return (off + 255) & ~(size_t)255;
}

static int get_width(dsl_layer *L, int M, Scratch *out, long long *stride) {
  WidthScratch &w = L->wid[M];
  if (!w.buf) {
    Scratch tmp;
    const size_t per_layer = layout(L, M, &tmp, nullptr);
    const size_t bytes = per_layer * L->d.n_layers;
    HIPCHK(hipSetDevice(L->dev));
    if (hipMalloc(&w.buf, bytes) != hipSuccess) {
      w.buf = nullptr;
      return fail(DSL_ENOMEM, "scratch of width %d (%zu bytes) could not be allocated", M, bytes);
    }
    HIPCHK(hipMemset(w.buf, 0, bytes));
    w.bytes = bytes;
    w.stride = (long long)per_layer;
    layout(L, M, &w.s, (char *)w.buf);
  }
  *out = w.s;
  *stride = w.stride;
  return 0;
}

// The scratch of dsl_decode_step_noalloc: one array per device, which the device holds for
// as long as the library is loaded.  Host code never passes `scratch` itself to a kernel
// (on the host that name is a stand-in, not a device address): dsl_layer_build looks up
// the array's device address on each device once, with that device current, and every
// launch takes that address.  No word of a step's scratch is read before the step's own
// launch writes it, so nothing is cleared between calls.
static constexpr size_t kStaticScratchBytes = (size_t)32 << 20;
static constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
static void *g_static_scratch[kMaxDevices];
static std::mutex g_static_mu;

static int static_scratch_init(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return fail(DSL_EUNSUPPORTED, "device %d beyond the %d the library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_static_mu);
  if (g_static_scratch[dev]) return 0;
  void *ptr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !ptr)
    return fail(DSL_EHIP, "hipGetSymbolAddress of the static scratch on device %d failed: %s", dev, hipGetErrorString(e));
  g_static_scratch[dev] = ptr;
  return 0;
}

static int check_ptr16(const void *p, const char *what) {
  if (!p) return fail(DSL_EINVAL, "%s is NULL", what);
  if ((uintptr_t)p & 15) return fail(DSL_EINVAL, "%s is not 16-byte aligned", what);
  return 0;
}

extern "C" {

const char *dsl_last_error(void) { return g_err.c_str(); }

int dsl_layer_build(const dsl_dims *dims, const dsl_weights *weights, dsl_layer **out) {
  if (!dims || !weights || !out) return fail(DSL_EINVAL, "dims, weights and out must be non-NULL");
  *out = nullptr;
  int rc = validate_dims(dims);
  if (rc) return rc;
  for (int l = 0; l < dims->n_layers; l++) {
    const dsl_weights &w = weights[l];
    const void *ptrs[] = {w.attn_norm, w.q_norm, w.kv_norm, w.ffn_norm, w.wqkv, w.wqkv_s, w.wq_b, w.wq_b_s,
                          w.wo_a, w.wo_a_s, w.wo_b, w.wo_b_s, w.w_router, w.sh_w13, w.sh_w13_s, w.sh_wd,
                          w.sh_wd_s, w.ex_w13, w.ex_w13_s, w.ex_wd, w.ex_wd_s};
    for (size_t i = 0; i < sizeof ptrs / sizeof ptrs[0]; i++)
      if ((rc = check_ptr16(ptrs[i], "a weight pointer"))) return fail(rc, "layer %d weight %zu: %s", l, i, g_err.c_str());
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(DSL_EHIP, "no HIP device");
  hipDeviceProp_t prop;
  HIPCHK(hipGetDeviceProperties(&prop, dev));
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(DSL_EUNSUPPORTED, "device %d is %s, the kernels are built for gfx950", dev, prop.gcnArchName);
  if ((rc = static_scratch_init(dev))) return rc;
  int bpc = 0, bpc_narrow = 0;
  HIPCHK(hipOccupancyMaxActiveBlocksPerMultiprocessor(&bpc, (const void *)dsl_layer_kernel<false>, kThreads, 0));
  HIPCHK(hipOccupancyMaxActiveBlocksPerMultiprocessor(&bpc_narrow, (const void *)dsl_layer_kernel<true>, kThreads, 0));
  if (bpc_narrow < bpc) bpc = bpc_narrow;  // one grid for both kernels
  if (bpc < 1) return fail(DSL_EUNSUPPORTED, "the layer kernel cannot be resident on a compute unit");
  if (bpc > 1) bpc = 1;
  dsl_layer *L = new dsl_layer();
  L->d = *dims;
  L->dev = dev;
  L->cus = prop.multiProcessorCount;
  L->bpc = bpc;
  L->grid = L->cus * bpc;
  const int keys = dims->swa_width > 0 ? dims->swa_width : dims->window;
  L->S = (keys + kSplitKeys - 1) / kSplitKeys;
  L->plan.kc_qkv = pick_kc(dims->hidden, 512);
  L->plan.kc_qb = pick_kc(dims->q_rank, 512);
  L->plan.kc_oa = pick_kc(dims->n_heads * dims->head_dim, 512);
  L->plan.kc_ob = pick_kc(dims->o_rank, 512);
  L->plan.kc_sh13 = pick_kc(dims->hidden, 1024);
  L->plan.kc_shd = pick_kc(dims->shared_inter, 512);
  L->plan.kc_router = pick_kc(dims->hidden, 1024);
  {
    const char *e = getenv("DSL_HANDOFF");
    if (e && e[0] >= '0' && e[0] <= '2') L->handoff = e[0] - '0';
  }
  if (hipMalloc((void **)&L->sync, sizeof(SyncWords)) != hipSuccess ||
      hipMalloc((void **)&L->dw, sizeof(dsl_weights) * dims->n_layers) != hipSuccess) {
    dsl_layer_destroy(L);
    return fail(DSL_ENOMEM, "sync buffer allocation failed");
  }
  if (hipMemset(L->sync, 0, sizeof(SyncWords)) != hipSuccess ||
      hipMemcpy(L->dw, weights, sizeof(dsl_weights) * dims->n_layers, hipMemcpyHostToDevice) != hipSuccess) {
    dsl_layer_destroy(L);
    return fail(DSL_EHIP, "initializing the sync buffer failed");
  }
  *out = L;
  return 0;
}

int dsl_layer_reserve(dsl_layer *L, int32_t M) {
  if (!L) return fail(DSL_EINVAL, "layer is NULL");
  if (M < 1 || M > L->d.max_rows) return fail(DSL_EUNSUPPORTED, "width %d outside 1..%d", M, L->d.max_rows);
  Scratch s;
  long long stride;
  return get_width(L, M, &s, &stride);
}

static int check_kv(const dsl_layer *L, const dsl_kv *kv, int n) {
  const dsl_dims &d = L->d;
  const int64_t record = d.head_dim + 16;
  for (int l = 0; l < n; l++) {
    const dsl_kv &c = kv[l];
    if (!c.base || !c.block_table || !c.row_req) return fail(DSL_EINVAL, "kv[%d]: base, block_table and row_req must be set", l);
    if ((uintptr_t)c.base & 15) return fail(DSL_EINVAL, "kv[%d]: base is not 16-byte aligned", l);
    if (c.block_stride < (int64_t)d.kv_block * record)
      return fail(DSL_EINVAL, "kv[%d]: block stride %lld is below block * RECORD = %lld", l, (long long)c.block_stride,
                  (long long)(d.kv_block * record));
    if (c.block_stride % 16) return fail(DSL_EINVAL, "kv[%d]: block stride %lld is not a multiple of 16", l, (long long)c.block_stride);
    if (c.n_blocks < 1 || c.max_blocks < 1 || c.n_req < 1)
      return fail(DSL_EINVAL, "kv[%d]: n_blocks, max_blocks and n_req must be positive", l);
    if (d.swa_width > 0 && !c.key_table) return fail(DSL_EINVAL, "kv[%d]: index-table mode needs key_table", l);
  }
  // a launch writes each record once and reads it only after the barrier that follows:
  // two layers sharing cache memory would break that
  for (int a = 0; a < n; a++)
    for (int b = a + 1; b < n; b++) {
      const uintptr_t a0 = (uintptr_t)kv[a].base, a1 = a0 + (uintptr_t)(kv[a].n_blocks * kv[a].block_stride);
      const uintptr_t b0 = (uintptr_t)kv[b].base, b1 = b0 + (uintptr_t)(kv[b].n_blocks * kv[b].block_stride);
      if (a0 < b1 && b0 < a1) return fail(DSL_EINVAL, "kv[%d] and kv[%d] overlap: every layer needs a cache of its own", a, b);
    }
  return 0;
}

static int launch(dsl_layer *L, int mode, const void *x, int M, const dsl_kv *kv, const int32_t *pos, void *out,
                  const dsl_taps *taps, void *stream, bool noalloc = false) {
  if (!L) return fail(DSL_EINVAL, "layer is NULL");
  int rc;
  if ((rc = check_ptr16(x, "input"))) return rc;
  if ((rc = check_ptr16(out, "output"))) return rc;
  if (M < 1 || M > L->d.max_rows) return fail(DSL_EUNSUPPORTED, "width %d outside 1..%d", M, L->d.max_rows);
  const int nl = mode == kModeDecode ? L->d.n_layers : 1;
  if (mode != kModeMoe) {
    if (!kv || !pos) return fail(DSL_EINVAL, "kv and positions must be set");
    if ((rc = check_kv(L, kv, nl))) return rc;
  }
  Params p{};
  if (noalloc) {
    // the device's static scratch in place of the width's own: no allocation
    Scratch tmp;
    const size_t per_layer = layout(L, M, &tmp, nullptr), bytes = per_layer * (size_t)nl;
    if (bytes > kStaticScratchBytes)
      return fail(DSL_EUNSUPPORTED, "width %d over %d layer(s) needs %zu bytes of scratch; the no-allocation entry point "
                  "holds %zu", M, nl, bytes, kStaticScratchBytes);
    void *base = (L->dev >= 0 && L->dev < kMaxDevices) ? g_static_scratch[L->dev] : nullptr;
    if (!base) return fail(DSL_EHIP, "the static scratch of device %d was not looked up", L->dev);
    layout(L, M, &p.s, (char *)base);
    p.s_stride = (long long)per_layer;
  } else if ((rc = get_width(L, M, &p.s, &p.s_stride))) {
    return rc;
  }
  const dsl_dims &d = L->d;
  p.h = d.hidden; p.H = d.n_heads; p.D = d.head_dim; p.qr = d.q_rank; p.orr = d.o_rank;
  p.W = d.window; p.swa = d.swa_width; p.E = d.n_experts; p.k = d.top_k; p.I = d.inter;
  p.Is = d.shared_inter; p.B = d.kv_block; p.n_layers = nl; p.a8 = d.expert_a8;
  p.eps = d.norm_eps; p.lim = d.swiglu_limit;
  p.attn_scale = 1.0f / sqrtf((float)d.head_dim);
  p.M = M; p.mode = mode; p.S = L->S; p.pl = L->plan;
  // producer hand-offs around the attention: every row's post-processing on a block of its
  // own (3 M blocks), heads within the counters, wo_a K chunks of whole heads
  // (level 2 also needs wo_b's K chunks within the counters)
  p.ho = mode != kModeMoe && L->grid >= 3 * M && d.n_heads <= kHoHeads && p.pl.kc_oa % d.head_dim == 0
             ? (L->handoff >= 2 && d.o_rank / p.pl.kc_ob <= kHoTbChunks ? 2 : L->handoff)
             : 0;
  p.w = L->dw;
  if (kv)
    for (int l = 0; l < nl; l++) p.kv[l] = kv[l];
  p.pos = pos;
  p.x = (const uint16_t *)x;
  p.out = (uint16_t *)out;
  if (taps) p.taps = *taps;
  p.sync = L->sync;
  p.trace = L->trace;
  void *args[] = {&p};
  HIPCHK(hipSetDevice(L->dev));
  // A plain launch: one block per compute unit is all that fits (the occupancy check at
  // build), so on a device this launch has to itself every block is resident at once.
  // The cooperative launch path costs ~18 us more per launch on this device.
  const bool narrow = narrow_ok(L, p);
  const void *kern = narrow ? (const void *)dsl_layer_kernel<true> : (const void *)dsl_layer_kernel<false>;
  HIPCHK(hipLaunchKernel(kern, dim3(L->grid), dim3(kThreads), args, 0, (hipStream_t)stream));
  L->last_kernel = narrow ? 1 : 0;
  return 0;
}

int dsl_decode_step(dsl_layer *L, const void *x, int32_t M, const dsl_kv *kv, const int32_t *pos, void *out,
                    const dsl_taps *taps, void *stream) {
  return launch(L, kModeDecode, x, M, kv, pos, out, taps, stream);
}

int dsl_decode_step_noalloc(dsl_layer *L, const void *x, int32_t M, const dsl_kv *kv, const int32_t *pos, void *out,
                            const dsl_taps *taps, void *stream) {
  return launch(L, kModeDecode, x, M, kv, pos, out, taps, stream, true);
}

int dsl_attn_step(dsl_layer *L, const void *x, int32_t M, const dsl_kv *kv, const int32_t *pos, void *out,
                  void *stream) {
  return launch(L, kModeAttn, x, M, kv, pos, out, nullptr, stream);
}

int dsl_moe_step(dsl_layer *L, const void *u, int32_t M, void *out, int32_t *ids, float *w, void *stream) {
  dsl_taps t{};
  t.topk_ids = ids;
  t.topk_w = w;
  return launch(L, kModeMoe, u, M, nullptr, nullptr, out, &t, stream);
}

int dsl_layer_health(dsl_layer *L) {
  if (!L) return fail(DSL_EINVAL, "layer is NULL");
  unsigned hw = 0;
  HIPCHK(hipSetDevice(L->dev));
  HIPCHK(hipMemcpy(&hw, &L->sync->health, sizeof hw, hipMemcpyDeviceToHost));
  if (hw) {
    HIPCHK(hipMemset(L->sync, 0, sizeof(SyncWords)));
    return fail(DSL_EDEVICE, "device fault word 0x%x (%s%s)", hw, hw & kFaultBarrier ? "grid barrier timeout " : "",
                hw & kFaultSlot ? "KV slot outside the cache" : "");
  }
  return 0;
}

int dsl_layer_set_trace(dsl_layer *L, int32_t on) {
  if (!L) return fail(DSL_EINVAL, "layer is NULL");
  HIPCHK(hipSetDevice(L->dev));
  if (on && !L->trace) {
    const size_t bytes = (size_t)kTraceLen * L->grid * sizeof(unsigned long long);
    if (hipMalloc((void **)&L->trace, bytes) != hipSuccess) {
      L->trace = nullptr;
      return fail(DSL_ENOMEM, "trace buffer allocation failed");
    }
    HIPCHK(hipMemset(L->trace, 0, bytes));
  } else if (!on && L->trace) {
    HIPCHK(hipFree(L->trace));
    L->trace = nullptr;
  }
  return 0;
}

int dsl_layer_read_trace(dsl_layer *L, double *ns, int32_t n_marks) {
  if (!L || !ns || n_marks < 0) return fail(DSL_EINVAL, "layer and ns must be set");
  if (!L->trace) return fail(DSL_EINVAL, "tracing is off");
  const int G = L->grid;
  std::vector<unsigned long long> buf((size_t)kTraceLen * G);
  HIPCHK(hipSetDevice(L->dev));
  HIPCHK(hipMemcpy(buf.data(), L->trace, buf.size() * sizeof(unsigned long long), hipMemcpyDeviceToHost));
  int khz = 0;
  HIPCHK(hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, L->dev));
  if (khz <= 0) return fail(DSL_EHIP, "device wall clock rate unknown");
  int cnt = 0;
  while (cnt < kTraceLen && buf[(size_t)cnt * G]) cnt++;
  const unsigned long long t0 = buf[0];
  for (int i = 0; i < cnt && i < n_marks; i++)
    for (int b = 0; b < G; b++) {
      const unsigned long long v = buf[(size_t)i * G + b];
      ns[(size_t)i * G + b] = v ? ((double)v - (double)t0) * 1e6 / khz : -1.0;
    }
  return cnt < n_marks ? cnt : n_marks;
}

int dsl_layer_last_kernel(const dsl_layer *L) {
  if (!L) return fail(DSL_EINVAL, "layer is NULL");
  return L->last_kernel;
}

int dsl_layer_grid(const dsl_layer *L, int32_t *blocks, int32_t *threads) {
  if (!L) return fail(DSL_EINVAL, "layer is NULL");
  if (blocks) *blocks = L->grid;
  if (threads) *threads = kThreads;
  return 0;
}

void dsl_layer_destroy(dsl_layer *L) {
  if (!L) return;
  for (auto &w : L->wid)
    if (w.buf) (void)hipFree(w.buf);
  if (L->sync) (void)hipFree(L->sync);
  if (L->trace) (void)hipFree(L->trace);
  if (L->dw) (void)hipFree(L->dw);
  delete L;
}

}  // extern "C"
