// Building blocks of the decode-layer stages: launch parameters and scratch, the
// weight-streaming linears on the bf16 matrix unit, and row helpers (reductions, MX
// quantization, bf16 loads and stores).
//
// Stage list: "Mono decode layer for DeepSeek-V4.1-Flash on MI355X" (vLLM PR
// 60397), Purpose, launch table (K1: seam, wqkv, q/kv norms, KV insert, wq_b;
// K2: split attention, combine, wo_a, wo_b, MoE router, top-k, shared expert,
// MXFP4 experts).  Every stage is called by all blocks of the persistent launch
// and splits its work statically over waves; grid barriers separate the stages.
//
// Linears.  Every weight format the layer stores decodes exactly into bf16 once
// its power-of-two block scale is folded in (e4m3 has 4 significant bits, e2m1
// 2), and every activation the linears read is exactly a bf16 value (MXFP8
// activations are kept as their dequantized values).  So each linear runs as
// bf16 x bf16 products with float32 accumulation on the matrix unit, the weights
// decoded in registers as they stream from HBM.  Only the shared expert's
// float32 128x128 scales are applied to the float32 partial sums, once per
// 128-wide K step.
#pragma once
#include <type_traits>

#include "dsl_device.h"
#include "dsl.h"

namespace dsl {

// Records the message dsl_last_error() returns and gives back code (host side).
int set_error(int code, const char *msg);

constexpr int kThreads = 512;
constexpr int kWavesPerBlock = kThreads / kWave;
constexpr int kSplitKeys = 32;  // keys per attention split

enum Mode : int { kModeDecode = 0, kModeAttn = 1, kModeMoe = 2 };

// Split-K chunk (elements of K per task) of each linear; K / chunk partial sums.
struct Plan {
  int kc_qkv, kc_qb, kc_oa, kc_ob, kc_sh13, kc_shd;
  int kc_router;  // K chunk of a router task (a multiple of 128 dividing hidden)
};

// Per-width scratch (device pointers into one allocation).
struct Scratch {
  uint16_t *xb;            // MXFP8(RMSNorm(x)) as exact bf16 values [M][h]
  float *p_qkv;            // [nks][M][qr + D]
  uint16_t *qb;            // MXFP8(RMSNorm(q latent)) as bf16 [M][qr]
  float *p_q;              // [nks][M][H*D]
  int64_t *keyoff;         // byte offset in the cache of every key record of each row [M][keys], -1 none
  uint16_t *ob;            // MXFP8(attention output) as bf16 [M][H*D]
  float *p_t;              // [nks][M][or]
  uint16_t *tb;            // MXFP8(wo_a output) as bf16 [M][or]
  float *p_a;              // [nks][M][h]
  uint16_t *xin;           // bf16 input of layers after the first [M][h]
  uint16_t *hres;          // bf16 residual after attention [M][h]
  uint16_t *u;             // bf16 MoE input [M][h]
  float *logits;           // router partial logits [hidden / kc_router][M][E]
  int32_t *tk_ids;         // selected experts of steps wider than a block's waves [M][k]
  float *tk_w;             // their weights [M][k]
  float *p_sh;             // [nks][M][2*Is]
  uint16_t *zsh;           // bf16 shared SwiGLU output [M][Is]
  uint16_t *zr;            // bf16 routed SwiGLU output per (row, slot) pair [M*k][I]
  float *y;                // routed expert outputs per pair [M*k][h]
  float *p_shd;            // [nks][M][h]
  uint16_t *uq;            // A8W4: MXFP8(u) as exact bf16 values [M][h], the routed gate/up input
  uint16_t *zq;            // A8W4: MXFP8(z) as exact bf16 values [M*k][I], the routed down input
  uint8_t *uq8;            // A8W4: the same MXFP8(u) as e4m3 codes [M][h] ...
  uint8_t *uqe;            // ... and E8M0 block exponents [M][h / 32] (the matrix-core experts' operand)
  uint8_t *zq8;            // A8W4: MXFP8(z) as e4m3 codes [M*k][I] ...
  uint8_t *zqe;            // ... and E8M0 block exponents [M*k][I / 32]
};

struct Params {
  int h, H, D, qr, orr, W, swa, E, k, I, Is, B, n_layers;
  int a8;  // the routed experts take MXFP8 activations (A8W4): 1 as exact bf16 values, 2 as
           // codes on the scaled matrix instruction
  float eps, lim, attn_scale;
  int M, mode, S;
  int ho;  // the attention's producers hand off through counters instead of grid barriers
  Plan pl;
  const dsl_weights *w;  // device array [n_layers]
  dsl_kv kv[DSL_MAX_LAYERS];
  const int32_t *pos;
  const uint16_t *x;
  uint16_t *out;
  dsl_taps taps;
  Scratch s;             // layer 0's scratch; layer l's is s shifted by l * s_stride bytes
  long long s_stride;
  SyncWords *sync;
  unsigned long long *trace;  // per-stage timestamps of block 0, or null
};

// Routing of the current layer, rebuilt in LDS by every block after the router.
struct Routing {
  int ids[DSL_MAX_ROWS * 8];
  float w[DSL_MAX_ROWS * 8];
  int pair[DSL_MAX_ROWS * 8];      // (row, slot) -> pair index, ordered by expert then row
  int pair_row[DSL_MAX_ROWS * 8];  // pair -> row
  unsigned long long rows[128];    // rows that selected each expert (bit m)
  int cnt[128], start[128], list[128];
  int nd;
  int np;    // (row, slot) pairs routed (live rows times k)
  int cmax;  // the most rows any expert has
};

struct Ctx {
  int lane, wave, gw, nw;  // lane, wave in block, global wave id, waves in grid
};

// The thread index through an empty asm: values derived from it are then recomputed in
// each stage instead of being hoisted out of the layer loop and kept live (spilled)
// across the whole launch.
__device__ __forceinline__ int tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

__device__ __forceinline__ int bid() {
  int b = blockIdx.x;
  asm volatile("" : "+s"(b));
  return b;
}

__device__ __forceinline__ Ctx make_ctx() {
  Ctx c;
  const int t = tid();
  c.lane = t & 63;
  c.wave = t >> 6;
  // wave-major: consecutive task indices go to different blocks (compute units, and
  // round-robin XCDs), so a stage with fewer tasks than waves still spreads its
  // memory traffic over the whole chip
  c.gw = c.wave * (int)gridDim.x + bid();
  c.nw = gridDim.x * kWavesPerBlock;
  return c;
}

// ============================================================== linears on the bf16 matrix unit

// Weight formats of the linears
enum WFmt : int {
  kW8T32 = 0,   // e4m3 [N][K] + one E8M0 per 32x32 tile [N/32][K/32]   (attention linears)
  kW8B128 = 1,  // e4m3 [N][K] + one f32 per 128x128 block [N/128][K/128] (shared expert)
  kW4 = 2,      // e2m1 nibbles [N][K/2] + one E8M0 per 32 along K [N][K/32] (routed experts)
};

// One lane's raw weight bytes for one 128-wide K step: lane (i, g) covers weight row
// n0 + i, K [32g, 32g+32) of the step (16 bytes of e2m1 or 32 of e4m3).
struct RawA {
  v4u a0, a1;
};

// Per-lane stream of one weight tile: row pointer at this lane's first K byte and the
// row's scales at the tile's first K block.
struct WStream {
  const uint8_t *w;
  const uint8_t *s8;   // E8M0 of this lane's row (kW4) or tile row (kW8T32), first block of k0
  const float *s32;    // f32 block scales of the tile (kW8B128), first 128-block of k0
};

template <int FMT>
__device__ __forceinline__ WStream wstream(const uint8_t *W, const uint8_t *S8, const float *S32, int K, int n,
                                           int k0, int g) {
  WStream st;
  if constexpr (FMT == kW4) {
    st.w = W + (size_t)n * (K >> 1) + ((k0 + 32 * g) >> 1);
    st.s8 = S8 + (size_t)n * (K >> 5) + (k0 >> 5);
    st.s32 = nullptr;
  } else if constexpr (FMT == kW8T32) {
    st.w = W + (size_t)n * K + k0 + 32 * g;
    st.s8 = S8 + (size_t)(n >> 5) * (K >> 5) + (k0 >> 5);
    st.s32 = nullptr;
  } else {
    st.w = W + (size_t)n * K + k0 + 32 * g;
    st.s8 = nullptr;
    st.s32 = S32 + (size_t)(n >> 7) * (K >> 7) + (k0 >> 7);
  }
  return st;
}

template <int FMT>
__device__ __forceinline__ void load_a(RawA &r, const WStream &ws, int step) {
  if constexpr (FMT == kW4) {
    // a lane's 16 bytes are half of a 128-byte line whose other half the next step
    // reads: a cached load, so the line is fetched once
    r.a0 = ld16(ws.w + 64 * step);
  } else {
    r.a0 = ldw16(ws.w + 128 * step);
    r.a1 = ldw16(ws.w + 128 * step + 16);
  }
}

// Scales of 4 consecutive steps starting at `step` (a multiple of 4): for E8M0 formats
// the 16 bytes of K blocks [4*step, 4*step + 16) of the lane's scale row (step s, group
// g is byte 4s + g); for f32 block scales the 4 steps' floats.  Requires 16-byte
// aligned scale rows (checked by the caller).
template <int FMT>
__device__ __forceinline__ v4u load_scales4(const WStream &ws, int step) {
  if constexpr (FMT == kW8B128)
    return ld16(ws.s32 + step);
  else
    return ld16(ws.s8 + 4 * step);
}
// Scale of one step: byte g of word j of a 4-step group, or one step's own byte
template <int FMT>
__device__ __forceinline__ float scale_of4(v4u sc4, int j, int g) {
  if constexpr (FMT == kW8B128)
    return __uint_as_float(sc4[j]);
  else
    return e8m0_to_f32((sc4[j] >> (8 * g)) & 0xFFu);
}
template <int FMT>
__device__ __forceinline__ float scale_of1(const WStream &ws, int step, int g) {
  if constexpr (FMT == kW8B128)
    return ldg(ws.s32 + step);
  else
    return e8m0_to_f32(ldg(ws.s8 + 4 * step + g));
}

// Decode one step's raw bytes into 4 x 8 bf16 A fragments (MFMA t takes elements
// 8t..8t+7).  Power-of-two scales are folded in exactly; the f32 block scale of the
// shared expert (sc) is applied to the partial sums instead.
template <int FMT>
__device__ __forceinline__ void decode_a(const RawA &r, float sc, v4u af[4]) {
  if constexpr (FMT == kW4) {
#pragma unroll
    for (int q = 0; q < 4; q++)
      af[q] = v4u{cvt_fp4x2_bf16<0>(r.a0[q], sc), cvt_fp4x2_bf16<1>(r.a0[q], sc), cvt_fp4x2_bf16<2>(r.a0[q], sc),
                  cvt_fp4x2_bf16<3>(r.a0[q], sc)};
  } else {
    const float s8 = FMT == kW8T32 ? sc : 1.0f;
    af[0] = v4u{cvt_fp8x2_bf16s<false>(r.a0[0], s8), cvt_fp8x2_bf16s<true>(r.a0[0], s8),
                cvt_fp8x2_bf16s<false>(r.a0[1], s8), cvt_fp8x2_bf16s<true>(r.a0[1], s8)};
    af[1] = v4u{cvt_fp8x2_bf16s<false>(r.a0[2], s8), cvt_fp8x2_bf16s<true>(r.a0[2], s8),
                cvt_fp8x2_bf16s<false>(r.a0[3], s8), cvt_fp8x2_bf16s<true>(r.a0[3], s8)};
    af[2] = v4u{cvt_fp8x2_bf16s<false>(r.a1[0], s8), cvt_fp8x2_bf16s<true>(r.a1[0], s8),
                cvt_fp8x2_bf16s<false>(r.a1[1], s8), cvt_fp8x2_bf16s<true>(r.a1[1], s8)};
    af[3] = v4u{cvt_fp8x2_bf16s<false>(r.a1[2], s8), cvt_fp8x2_bf16s<true>(r.a1[2], s8),
                cvt_fp8x2_bf16s<false>(r.a1[3], s8), cvt_fp8x2_bf16s<true>(r.a1[3], s8)};
  }
}

// B fragments of one step for one group of 16 activation rows: lane (j, g) holds row
// j's 32 bf16 at K [32g, 32g+32) of the step (rows past the group's end are zero).
__device__ __forceinline__ void load_b(v4u b[4], const uint16_t *row, bool ok, int k) {
#pragma unroll
  for (int t = 0; t < 4; t++) b[t] = ok ? ld16(row + k + 8 * t) : v4u{0, 0, 0, 0};
}

template <int FMT, int NT, int NCG>
__device__ __forceinline__ void step_mfma(const v4u af[NT][4], const float bsc[NT], const v4u b[NCG][4],
                                          v4f acc[NT][NCG]) {
#pragma unroll
  for (int c = 0; c < NCG; c++) {
#pragma unroll
    for (int tt = 0; tt < NT; tt++) {
      if constexpr (FMT == kW8B128) {
        v4f t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < 4; q++) t = mfma_bf16(af[tt][q], b[c][q], t);
        acc[tt][c] += bsc[tt] * t;
      } else {
#pragma unroll
        for (int q = 0; q < 4; q++) acc[tt][c] = mfma_bf16(af[tt][q], b[c][q], acc[tt][c]);
      }
    }
  }
}

// The weight bytes of the first 4 K steps of a wave's first task of a dense linear,
// loaded ahead of the stage: after the previous stage's stores have drained and before
// the grid barrier, so their HBM latency overlaps the barrier.  (The scales are loaded
// with the activations after the barrier.)  on: the wave has such a task and it takes
// the pipelined path (wave-uniform).
struct PreA {
  RawA ra[4];
  bool on;
};

// NT weight tiles of 16 rows times NCG groups of 16 bf16 activation rows over `nsteps`
// 128-wide K steps, software-pipelined in groups of 4 steps: ring buffers hold the raw
// weight bytes and the activation fragments of the next 4 steps and the scales of the
// next group, so every load is issued a group ahead of its use (the last group loads
// nothing; the conditions are uniform over the wave).  Requires nsteps % 4 == 0
// and 16-byte aligned scale rows.  kb = this lane's first activation K index.
// acc[tt][c] lane l ends holding C[4*(l/16) + r][l%16]: weight row n0[tt] + 4*(l/16) + r,
// activation row 16c + l%16.
// With `use` (one tile only) the first group's weight bytes come from *pf.
template <int FMT, int NT, int NCG>
__device__ __forceinline__ void tiles_pipe4(const WStream ws[NT], int nsteps, const uint16_t *const xrow[NCG],
                                            const bool xok[NCG], int kb, int g, v4f acc[NT][NCG],
                                            const PreA *pf = nullptr, bool use = false) {
  constexpr int P = 4;
  constexpr int PB = NCG == 1 ? 4 : (NCG == 2 ? 2 : 1);  // activation ring depth (16 registers per step and group)
  RawA ra[P][NT];
  v4u rb[PB][NCG][4];
  v4u scg[NT], scn[NT];
#pragma unroll
  for (int tt = 0; tt < NT; tt++) {
    scg[tt] = load_scales4<FMT>(ws[tt], 0);
    if (nsteps > P) scn[tt] = load_scales4<FMT>(ws[tt], P);
  }
  if (NT == 1 && use) {
#pragma unroll
    for (int j = 0; j < P; j++) ra[j][0] = pf->ra[j];
  } else {
#pragma unroll
    for (int j = 0; j < P; j++) {
#pragma unroll
      for (int tt = 0; tt < NT; tt++) load_a<FMT>(ra[j][tt], ws[tt], j);
    }
  }
#pragma unroll
  for (int j = 0; j < PB; j++) {
#pragma unroll
    for (int c = 0; c < NCG; c++) load_b(rb[j][c], xrow[c], xok[c], kb + 128 * j);
  }
  for (int s = 0; s < nsteps; s += P) {
    // the last group issues no loads: a prefetch of a step past the end would only be a
    // second round trip that the stage waits for
    const bool more = s + P < nsteps;
#pragma unroll
    for (int j = 0; j < P; j++) {
      const int st = s + j;
      v4u af[NT][4];
      float bsc[NT];
#pragma unroll
      for (int tt = 0; tt < NT; tt++) {
        bsc[tt] = scale_of4<FMT>(scg[tt], j, g);
        decode_a<FMT>(ra[j][tt], bsc[tt], af[tt]);
        if (more) load_a<FMT>(ra[j][tt], ws[tt], st + P);
      }
      step_mfma<FMT, NT, NCG>(af, bsc, rb[j % PB], acc);
      if (st + PB < nsteps) {
#pragma unroll
        for (int c = 0; c < NCG; c++) load_b(rb[j % PB][c], xrow[c], xok[c], kb + 128 * (st + PB));
      }
    }
    if (more) {
      const int gn = s + 2 * P < nsteps ? s + 2 * P : nsteps - P;
#pragma unroll
      for (int tt = 0; tt < NT; tt++) {
        scg[tt] = scn[tt];
        scn[tt] = load_scales4<FMT>(ws[tt], gn);
      }
    }
  }
}

// Any nsteps and alignment: one step at a time, activations one step ahead.
template <int FMT, int NT, int NCG>
__device__ __forceinline__ void tiles_pipe1(const WStream ws[NT], int nsteps, const uint16_t *const xrow[NCG],
                                            const bool xok[NCG], int kb, int g, v4f acc[NT][NCG]) {
  for (int st = 0; st < nsteps; st++) {
    RawA ra[NT];
    v4u af[NT][4];
    float bsc[NT];
    v4u b[NCG][4];
#pragma unroll
    for (int tt = 0; tt < NT; tt++) load_a<FMT>(ra[tt], ws[tt], st);
#pragma unroll
    for (int c = 0; c < NCG; c++) load_b(b[c], xrow[c], xok[c], kb + 128 * st);
#pragma unroll
    for (int tt = 0; tt < NT; tt++) {
      bsc[tt] = scale_of1<FMT>(ws[tt], st, g);
      decode_a<FMT>(ra[tt], bsc[tt], af[tt]);
    }
    step_mfma<FMT, NT, NCG>(af, bsc, b, acc);
  }
}

template <int FMT>
__device__ __forceinline__ bool scales_aligned(const WStream &ws) {
  return FMT == kW8B128 ? ((uintptr_t)ws.s32 & 15) == 0 : ((uintptr_t)ws.s8 & 15) == 0;
}

// ------------------------------------------------------------ A8W4 on the scaled matrix instruction
//
// With MXFP8 activations the routed experts' matrix-core tiles multiply raw codes:
// v_mfma_scale_f32_16x16x128_f8f6f4 takes the MXFP4 weights (A, e2m1) and the MXFP8
// activations (B, e4m3) as they are stored, with one E8M0 exponent per 32-element block of
// each, and sums the 128 exactly scaled products of a K step in f32.  No decode, and one
// instruction per step and tile pair instead of four, so the same registers hold a ring
// twice as deep as the bf16 tiles' (8 steps of weights).
// Operand layouts (read off the instruction on gfx950): A lane (i, g) holds weight row i,
// K [32 g, 32 g + 32) of the step, 16 bytes in K order; B lane (j, g) holds activation row
// j, K [16 g, 16 g + 16) in its first 16 bytes and K [64 + 16 g, 64 + 16 g + 16) in the
// next 16; each lane gives the exponent of block g (K [32 g, 32 g + 32)) of its row; the
// result is laid out as the bf16 instruction's (lane l: weight rows 4 (l / 16) + r,
// activation row l % 16).

// One step's B fragment of one group of 16 activation rows (codes), zero past the group's
// end: the register pair is cleared, then only the group's lanes load into it (no select
// after the loads, which would wait for them)
union B8 {
  v8i v;
  v4u h[2];
};
__device__ __forceinline__ void load_b8(B8 &b, const uint8_t *row, bool ok, int k) {
  b.v = v8i{0, 0, 0, 0, 0, 0, 0, 0};
  if (ok) {
    b.h[0] = ld16(row + k);
    b.h[1] = ld16(row + k + 64);
  }
}

__device__ __forceinline__ v4f mfma_a8w4(const v4u &a, const B8 &bb, v4f c, uint32_t sa, uint32_t sb) {
  const v8i b = bb.v;
  const v4i a4 = __builtin_bit_cast(v4i, a);
  const v8i av = __builtin_shufflevector(a4, v4i{0, 0, 0, 0}, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, b, c, 4, 0, 0, (int)sa, 0, (int)sb);
}

// NT MXFP4 weight tiles times NCG groups of 16 MXFP8 activation rows (codes xrow, block
// exponents xex; xok: the lane's row exists) over nsteps 128-wide K steps, nsteps % P == 0:
// the weights (and each lane's exponent byte of them) P steps ahead and the activations
// (and theirs) PB steps ahead in register rings, each step's weight loads issued before its
// activation loads (loads complete in issue order, so a wait for an activation then
// waits for no weight issued after it).  The result as tiles_pipe4's.
template <int NT, int NCG, int P>
__device__ __forceinline__ void tiles_a8w4(const WStream ws[NT], int nsteps, const uint8_t *const xrow[NCG],
                                           const uint8_t *const xex[NCG], const bool xok[NCG], int g, v4f acc[NT][NCG]) {
  constexpr int PB = NCG == 1 ? P : (NCG == 2 ? P / 2 : (P >= 4 ? P / 4 : 1));
  v4u ra[P][NT];
  uint32_t sa[P][NT];  // the step's four exponent bytes of the lane's weight row; byte g is the lane's
  B8 rb[PB][NCG];
  uint32_t sb[PB][NCG];  // likewise for the lane's activation row
#pragma unroll
  for (int j = 0; j < P; j++)
#pragma unroll
    for (int tt = 0; tt < NT; tt++) {
      ra[j][tt] = ld16(ws[tt].w + 64 * j);
      sa[j][tt] = ldg(reinterpret_cast<const uint32_t *>(ws[tt].s8 + 4 * j));
    }
#pragma unroll
  for (int j = 0; j < PB; j++)
#pragma unroll
    for (int c = 0; c < NCG; c++) {
      load_b8(rb[j][c], xrow[c], xok[c], 128 * j + 16 * g);
      sb[j][c] = ldg(reinterpret_cast<const uint32_t *>(xex[c] + 4 * j));
    }
  for (int s = 0; s < nsteps; s += P) {
    const bool more = s + P < nsteps;
#pragma unroll
    for (int j = 0; j < P; j++) {
      const int st = s + j;
#pragma unroll
      for (int c = 0; c < NCG; c++)
#pragma unroll
        for (int tt = 0; tt < NT; tt++)
          acc[tt][c] = mfma_a8w4(ra[j][tt], rb[j % PB][c], acc[tt][c], (sa[j][tt] >> (8 * g)) & 0xFFu,
                                 (sb[j % PB][c] >> (8 * g)) & 0xFFu);
      if (more) {
#pragma unroll
        for (int tt = 0; tt < NT; tt++) {
          ra[j][tt] = ld16(ws[tt].w + 64 * (st + P));
          sa[j][tt] = ldg(reinterpret_cast<const uint32_t *>(ws[tt].s8 + 4 * (st + P)));
        }
      }
      if (st + PB < nsteps) {
#pragma unroll
        for (int c = 0; c < NCG; c++) {
          load_b8(rb[j % PB][c], xrow[c], xok[c], 128 * (st + PB) + 16 * g);
          sb[j % PB][c] = ldg(reinterpret_cast<const uint32_t *>(xex[c] + 4 * (st + PB)));
        }
      }
    }
  }
}

// Any step count: one step at a time (the small shapes)
template <int NT, int NCG>
__device__ __forceinline__ void tiles_a8w4_1(const WStream ws[NT], int nsteps, const uint8_t *const xrow[NCG],
                                             const uint8_t *const xex[NCG], const bool xok[NCG], int g, v4f acc[NT][NCG]) {
  for (int st = 0; st < nsteps; st++) {
    v4u ra[NT];
    B8 rb[NCG];
    uint32_t sa[NT], sb[NCG];
#pragma unroll
    for (int tt = 0; tt < NT; tt++) {
      ra[tt] = ld16(ws[tt].w + 64 * st);
      sa[tt] = ldg(ws[tt].s8 + 4 * st + g);
    }
#pragma unroll
    for (int c = 0; c < NCG; c++) {
      load_b8(rb[c], xrow[c], xok[c], 128 * st + 16 * g);
      sb[c] = ldg(xex[c] + 4 * st + g);
    }
#pragma unroll
    for (int c = 0; c < NCG; c++)
#pragma unroll
      for (int tt = 0; tt < NT; tt++) acc[tt][c] = mfma_a8w4(ra[tt], rb[c], acc[tt][c], sa[tt], sb[c]);
  }
}

template <int NT, int NCG>
__device__ __forceinline__ void tiles_a8(const WStream ws[NT], int nsteps, const uint8_t *const xrow[NCG],
                                         const uint8_t *const xex[NCG], const bool xok[NCG], int g, v4f acc[NT][NCG]) {
  if (nsteps % 8 == 0)
    tiles_a8w4<NT, NCG, 4>(ws, nsteps, xrow, xex, xok, g, acc);
  else
    tiles_a8w4_1<NT, NCG>(ws, nsteps, xrow, xex, xok, g, acc);
}

// Pipelined path when the step count and scale alignment allow it (always so when the
// first group was loaded ahead, `use`), else the simple one.
template <int FMT, int NT, int NCG>
__device__ __forceinline__ void tiles(const WStream ws[NT], int nsteps, const uint16_t *const xrow[NCG],
                                      const bool xok[NCG], int kb, int g, v4f acc[NT][NCG],
                                      const PreA *pf = nullptr, bool use = false) {
  bool fast = nsteps % 4 == 0;
#pragma unroll
  for (int tt = 0; tt < NT; tt++) fast = fast && scales_aligned<FMT>(ws[tt]);
  if (fast)
    tiles_pipe4<FMT, NT, NCG>(ws, nsteps, xrow, xok, kb, g, acc, pf, use);
  else
    tiles_pipe1<FMT, NT, NCG>(ws, nsteps, xrow, xok, kb, g, acc);
}

// One task (16-row tile, K chunk) of a dense linear y = x . W^T with bf16 rows x [M][K]:
// writes the chunk's partial sums to part[ks][M][N].  One function per row-group count,
// so each gets its own register allocation.
template <int FMT, int NCG>
__device__ __forceinline__ void linear_task_n(int t, int lane, const uint8_t *W, const uint8_t *S8, const float *S32,
                                           int N, int K, int kc, const uint16_t *x, int M, float *part,
                                           const PreA *pf, bool use) {
  const int ntile = N >> 4;
  const int ks = t / ntile, nt = t - ks * ntile;
  const int i = lane & 15, g = lane >> 4;
  float *out = part + (size_t)ks * M * N;
  const int k0 = ks * kc;
  const WStream ws[1] = {wstream<FMT>(W, S8, S32, K, nt * 16 + i, k0, g)};
  const uint16_t *xrow[NCG];
  bool xok[NCG];
  v4f acc[1][NCG];
#pragma unroll
  for (int c = 0; c < NCG; c++) {
    const int m = 16 * c + i;
    xok[c] = m < M;
    xrow[c] = x + (size_t)(xok[c] ? m : 0) * K;
    acc[0][c] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  tiles<FMT, 1, NCG>(ws, kc >> 7, xrow, xok, k0 + 32 * g, g, acc, pf, use);
#pragma unroll
  for (int c = 0; c < NCG; c++) {
    const int m = 16 * c + i;
    if (m < M) stg(reinterpret_cast<v4f *>(out + (size_t)m * N + nt * 16 + 4 * g), acc[0][c]);
  }
}

// MAXG: the most 16-row groups of x the caller can pass (1: M <= 16, and only that
// instantiation is compiled in)
template <int FMT, int MAXG = 3>
__device__ __forceinline__ void linear_task(int t, int lane, const uint8_t *W, const uint8_t *S8, const float *S32,
                                            int N, int K, int kc, const uint16_t *x, int M, float *part,
                                            const PreA *pf = nullptr, bool use = false) {
  const int ncg = (M + 15) >> 4;
  if (MAXG == 1 || ncg == 1)
    linear_task_n<FMT, 1>(t, lane, W, S8, S32, N, K, kc, x, M, part, pf, use);
  else if (ncg == 2)
    linear_task_n<FMT, 2>(t, lane, W, S8, S32, N, K, kc, x, M, part, pf, use);
  else
    linear_task_n<FMT, 3>(t, lane, W, S8, S32, N, K, kc, x, M, part, pf, use);
}

// Task t of a dense linear to global wave t mod waves.
template <int FMT, int MAXG = 3>
__device__ __forceinline__ void linear_all(const Ctx &cx, const uint8_t *W, const uint8_t *S8, const float *S32, int N, int K, int kc,
                           const uint16_t *x, int M, float *part) {
  const int T = (N >> 4) * (K / kc);
  for (int t = cx.gw; t < T; t += cx.nw) linear_task<FMT, MAXG>(t, cx.lane, W, S8, S32, N, K, kc, x, M, part);
}

// The same, the wave's first task starting from the weights linear_prefetch loaded.
// ONE: the caller knows there are no more tasks than waves (only the first task is compiled).
template <int FMT, int MAXG = 3, bool ONE = false>
__device__ __forceinline__ void linear_all_pre(const Ctx &cx, const uint8_t *W, const uint8_t *S8, const float *S32, int N,
                                               int K, int kc, const uint16_t *x, int M, float *part, const PreA &pf) {
  const int T = (N >> 4) * (K / kc);
  int t = cx.gw;
  if (t < T) linear_task<FMT, MAXG>(t, cx.lane, W, S8, S32, N, K, kc, x, M, part, &pf, pf.on);
  if constexpr (ONE) return;
  // (the first task peeled: pf is dead after it)
  for (t += cx.nw; t < T; t += cx.nw) linear_task<FMT, MAXG>(t, cx.lane, W, S8, S32, N, K, kc, x, M, part);
}

// Where this wave's first task of linear_all_pre (same arguments) starts, when it has
// one, takes the pipelined path and is not in the last wave (which holds the grid
// barrier's thread and so must have no loads in flight).  Computed before the drain, so
// that only the loads themselves come between the drain and the barrier.
struct PreAddr {
  WStream ws;
  bool on;
};

template <int FMT>
__device__ __forceinline__ PreAddr linear_prefetch_addr(const Ctx &cx, const uint8_t *W, const uint8_t *S8,
                                                        const float *S32, int N, int K, int kc) {
  const int ntile = N >> 4, T = ntile * (K / kc), t = cx.gw, nsteps = kc >> 7;
  PreAddr a;
  const int tc = t < T ? t : 0;
  const int ks = tc / ntile, nt = tc - ks * ntile, i = cx.lane & 15, g = cx.lane >> 4;
  a.ws = wstream<FMT>(W, S8, S32, K, nt * 16 + i, ks * kc, g);
  a.on = t < T && cx.wave != kWavesPerBlock - 1 && nsteps % 4 == 0 && scales_aligned<FMT>(a.ws);
  return a;
}

// No prefetched weights.  Every field is set, so no earlier value stays live across the
// layer loop; the register fields take arbitrary values (no instructions, and no join
// that would have to wait for a load).
__device__ __forceinline__ PreA pre_none() {
  PreA pf;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    pf.ra[j].a0 = __builtin_nondeterministic_value(pf.ra[j].a0);
    pf.ra[j].a1 = __builtin_nondeterministic_value(pf.ra[j].a1);
  }
  pf.on = false;
  return pf;
}

// Loads the weight bytes of the first group of the task at a into pf.
template <int FMT>
__device__ __forceinline__ void linear_prefetch(const PreAddr &a, PreA &pf) {
  if (!a.on) return;
  pf.on = true;
#pragma unroll
  for (int j = 0; j < 4; j++) load_a<FMT>(pf.ra[j], a.ws, j);
}

// ============================================================== block-level helpers

// Sum / max over the block's threads (fixed order: wave results in wave order).
__device__ __forceinline__ float block_sum(float v, float *red) {
  v = wave_sum(v);
  __syncthreads();
  if ((tid() & 63) == 0) red[tid() >> 6] = v;
  __syncthreads();
  return ((red[0] + red[1]) + (red[2] + red[3])) + ((red[4] + red[5]) + (red[6] + red[7]));
}
__device__ __forceinline__ float block_max(float v, float *red) {
  v = wave_max(v);
  __syncthreads();
  if ((tid() & 63) == 0) red[tid() >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3])), fmaxf(fmaxf(red[4], red[5]), fmaxf(red[6], red[7])));
}

// v[e] = sum over ks < nks (in ks order) of p[ks * stride + e]: the loads of up to B
// partials (BMAX, else 32 registers' worth) are issued together, then added in order, so a
// stage does not wait a round trip per partial.
template <int E, int BMAX = 0>
__device__ __forceinline__ void load_sum_f32(const float *p, size_t stride, int nks, float v[E]) {
  constexpr int B = BMAX > 0 ? BMAX : (E >= 32 ? 1 : (E >= 4 ? 32 / E : 8));
#pragma unroll
  for (int e = 0; e < E; e++) v[e] = 0.f;
  for (int k0 = 0; k0 < nks; k0 += B) {
    float t[B][E];
#pragma unroll
    for (int b = 0; b < B; b++) {
      if (k0 + b < nks) {
        const float *q = p + (size_t)(k0 + b) * stride;
        if constexpr (E >= 4) {
#pragma unroll
          for (int e = 0; e < E; e += 4) {
            const float4 a = ld_f4(q + e);
            t[b][e] = a.x; t[b][e + 1] = a.y; t[b][e + 2] = a.z; t[b][e + 3] = a.w;
          }
        } else {
#pragma unroll
          for (int e = 0; e < E; e++) t[b][e] = ldg(q + e);
        }
      } else {
#pragma unroll
        for (int e = 0; e < E; e++) t[b][e] = 0.f;
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the batch's loads ahead of its adds
#pragma unroll
    for (int b = 0; b < B; b++)
      if (k0 + b < nks) {
#pragma unroll
        for (int e = 0; e < E; e++) v[e] = k0 + b == 0 ? t[b][e] : v[e] + t[b][e];
      }
  }
}

// sum over ks < n (in ks order) of p[ks * stride], up to 8 loads in flight
__device__ __forceinline__ float sum_strided(const float *p, size_t stride, int n) {
  float v;
  load_sum_f32<1>(p, stride, n, &v);
  return v;
}

template <int E>
__device__ __forceinline__ void load_bf16(const uint16_t *p, float v[E]) {
  if constexpr (E >= 8) {
#pragma unroll
    for (int e = 0; e < E; e += 8) {
      const v4u a = ld16(p + e);
#pragma unroll
      for (int q = 0; q < 4; q++) {
        v[e + 2 * q] = bf16_to_f32(a[q] & 0xFFFFu);
        v[e + 2 * q + 1] = bf16_to_f32(a[q] >> 16);
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < E; e++) v[e] = bf16_to_f32(ldg(p + e));
  }
}

// E consecutive floats (16-byte loads when E >= 4; p then 16-byte aligned), or zeros
template <int E>
__device__ __forceinline__ void load_f32(const float *p, bool on, float v[E]) {
  if constexpr (E >= 4) {
#pragma unroll
    for (int e = 0; e < E; e += 4) {
      const v4u a = on ? ld16(p + e) : v4u{0u, 0u, 0u, 0u};
#pragma unroll
      for (int q = 0; q < 4; q++) v[e + q] = __uint_as_float(a[q]);
    }
  } else {
#pragma unroll
    for (int e = 0; e < E; e++) v[e] = on ? ldg(p + e) : 0.f;
  }
}

template <int E>
__device__ __forceinline__ void store_bf16(uint16_t *p, const float v[E]) {
  if constexpr (E >= 8) {
#pragma unroll
    for (int e = 0; e < E; e += 8) {
      v4u a;
#pragma unroll
      for (int q = 0; q < 4; q++) a[q] = f32_to_bf16(v[e + 2 * q]) | (f32_to_bf16(v[e + 2 * q + 1]) << 16);
      st16(p + e, a);
    }
  } else {
#pragma unroll
    for (int e = 0; e < E; e++) stg(p + e, (uint16_t)f32_to_bf16(v[e]));
  }
}

// MX-quantize E contiguous values per thread (32-blocks span 32/E threads) and keep the
// dequantized values: v <- e4m3(v / 2^(X-127)) * 2^(X-127).  Inactive threads hold zeros.
template <int E>
__device__ __forceinline__ void mx_quant_dequant(float v[E]) {
  float am = 0.f;
#pragma unroll
  for (int e = 0; e < E; e++) am = fmaxf(am, fabsf(v[e]));
  if constexpr (E < 32) am = group_max<32 / E>(am);
  const uint32_t X = mx_e4m3_exponent(am);
  const float sc = e8m0_to_f32(X);
  if (X == 0u) {
    // (a block of zeros or of values below 2^-118: its scale 2^-127 is subnormal, so the
    // software rounding)
    const float inv = mx_inv_scale(X);
#pragma unroll
    for (int e = 0; e < E; e++) v[e] = e4m3_to_f32(f32_to_e4m3(v[e] * inv)) * sc;
  } else {
    // gfx950's scaled conversions: v / 2^(X-127) to e4m3 with ties to even, and the codes
    // back times 2^(X-127); the input is clamped to the block's e4m3 range first (past it
    // the conversion gives the NaN code where the software rounding saturates).  Checked
    // bit for bit against the software rounding on 4 M values with a pair probe, ties,
    // subnormal steps, signed zeros and the saturation edge included.
    const float lim = 448.0f * sc;
#pragma unroll
    for (int e = 0; e < E; e += 2) {
      typedef short v2s __attribute__((ext_vector_type(2)));
      const float a = fminf(fmaxf(v[e], -lim), lim), b = E > 1 ? fminf(fmaxf(v[e + 1 < E ? e + 1 : e], -lim), lim) : 0.f;
      const v2s c = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v2s{0, 0}, a, b, sc, false);
      const auto d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((unsigned)(unsigned short)c[0], sc, false);
      v[e] = d[0];
      if (E > 1) v[e + 1 < E ? e + 1 : e] = d[1];
    }
  }
}

// Elements per thread for a row of n values spread over the block (a power of two).
__device__ __forceinline__ int row_elems(int n) {
  int e = 1;
  while (e * kThreads < n) e <<= 1;
  return e;
}

__device__ __forceinline__ float swiglu_clamp(float g, float u, float lim) {
  g = fminf(g, lim);
  u = fminf(fmaxf(u, -lim), lim);
  return g / (1.0f + expf(-g)) * u;
}

}  // namespace dsl
