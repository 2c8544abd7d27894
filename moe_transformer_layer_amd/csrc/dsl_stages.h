// Building blocks of the decode-layer stages: row normalization / MX quantization,
// weight-streaming linears on the bf16 matrix unit, and the device task queue.
//
// Stage list: "Mono decode layer for DeepSeek-V4.1-Flash on MI355X" (vLLM PR
// 60397), Purpose, launch table (K1: seam, wqkv, q/kv norms, KV insert, wq_b;
// K2: split attention, combine, wo_a, wo_b, MoE router, top-k, shared expert,
// MXFP4 experts).  Every stage is called by all blocks of the persistent launch
// and splits its work over waves; grid barriers separate stages.
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

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;
constexpr int kSplitKeys = 32;  // keys per attention split

enum Mode : int { kModeDecode = 0, kModeAttn = 1, kModeMoe = 2 };

// Split-K chunk (elements of K per task) of each linear; K / chunk partial sums.
struct Plan {
  int kc_qkv, kc_qb, kc_oa, kc_ob, kc_sh13, kc_shd;
};

// Per-width scratch (device pointers into one allocation).
struct Scratch {
  uint16_t *xb;            // MXFP8(RMSNorm(x)) as exact bf16 values [M][h]
  float *p_qkv;            // [nks][M][qr + D]
  uint16_t *qb;            // MXFP8(RMSNorm(q latent)) as bf16 [M][qr]
  float *p_q;              // [nks][M][H*D]
  float *att_o, *att_ml;   // split partials [M][H][S][D], [M][H][S][2]
  uint16_t *ob;            // MXFP8(attention output) as bf16 [M][H*D]
  float *p_t;              // [nks][M][or]
  uint16_t *tb;            // MXFP8(wo_a output) as bf16 [M][or]
  float *p_a;              // [nks][M][h]
  uint16_t *xin;           // bf16 input of layers after the first [M][h]
  uint16_t *hres;          // bf16 residual after attention [M][h]
  uint16_t *u;             // bf16 MoE input [M][h]
  float *logits;           // [M][E]
  float *p_sh;             // [nks][M][2*Is]
  uint16_t *zsh;           // bf16 shared SwiGLU output [M][Is]
  uint16_t *zr;            // bf16 routed SwiGLU output per (row, slot) pair [M*k][I]
  float *y;                // routed expert outputs per pair [M*k][h]
  float *p_shd;            // [nks][M][h]
};

struct Params {
  int h, H, D, qr, orr, W, swa, E, k, I, Is, B, n_layers;
  float eps, lim, attn_scale;
  int M, mode, S;
  Plan pl;
  const dsl_weights *w;  // device array [n_layers]
  dsl_kv kv[DSL_MAX_LAYERS];
  const int32_t *pos;
  const uint16_t *x;
  uint16_t *out;
  dsl_taps taps;
  Scratch s;
  SyncWords *sync;
};

// Routing of the current layer, rebuilt in LDS by every block after the router.
struct Routing {
  int ids[DSL_MAX_ROWS * 8];
  float w[DSL_MAX_ROWS * 8];
  int pair[DSL_MAX_ROWS * 8];      // (row, slot) -> pair index, ordered by expert then row
  int pair_row[DSL_MAX_ROWS * 8];  // pair -> row
  int cnt[128], start[128], list[128];
  int nd;
};

struct Ctx {
  int lane, wave, gw, nw;  // lane, wave in block, global wave id, waves in grid
};

__device__ __forceinline__ Ctx make_ctx() {
  Ctx c;
  c.lane = threadIdx.x & 63;
  c.wave = threadIdx.x >> 6;
  c.gw = blockIdx.x * kWavesPerBlock + c.wave;
  c.nw = gridDim.x * kWavesPerBlock;
  return c;
}

// ============================================================== row helpers (one wave per row)

// MX-quantize one row of n values (n a multiple of 32) to e4m3 with one E8M0 per 32,
// optionally after RMSNorm with gamma (r = 1/sqrt(mean(v^2) + eps)), and store the
// dequantized values (exact in bf16).  load4(k) returns values k..k+3.  Lanes work in
// groups of 8 per 32-block.
template <class L4>
__device__ void wave_row_mxq(L4 load4, int n, const float *gamma, float eps, uint16_t *dst, int lane) {
  float r = 1.0f;
  if (gamma) {
    float ss = 0.f;
    for (int k = lane * 4; k < n; k += 4 * kWave) {
      float4 v = load4(k);
      ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
    ss = wave_sum(ss);
    r = 1.0f / sqrtf(ss / (float)n + eps);
  }
  const int nb = n >> 5;
  for (int b0 = 0; b0 < nb; b0 += 8) {
    const int blk = b0 + (lane >> 3);
    const bool act = blk < nb;
    const int k = blk * 32 + (lane & 7) * 4;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (act) {
      float4 t = load4(k);
      v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
      if (gamma) {
#pragma unroll
        for (int e = 0; e < 4; e++) v[e] = v[e] * r * gamma[k + e];
      }
    }
    float am = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
    am = group_max<8>(am);
    const uint32_t X = mx_e4m3_exponent(am);
    const float inv = mx_inv_scale(X), sc = e8m0_to_f32(X);
    uint32_t b[4];
#pragma unroll
    for (int e = 0; e < 4; e++) b[e] = f32_to_bf16(e4m3_to_f32(f32_to_e4m3(v[e] * inv)) * sc);
    if (act) *reinterpret_cast<v2u *>(dst + k) = v2u{b[0] | (b[1] << 16), b[2] | (b[3] << 16)};
  }
}

// ============================================================== linears on the bf16 matrix unit

// Weight formats of the linears
enum WFmt : int {
  kW8T32 = 0,   // e4m3 [N][K] + one E8M0 per 32x32 tile [N/32][K/32]   (attention linears)
  kW8B128 = 1,  // e4m3 [N][K] + one f32 per 128x128 block [N/128][K/128] (shared expert)
  kW4 = 2,      // e2m1 nibbles [N][K/2] + one E8M0 per 32 along K [N][K/32] (routed experts)
};

// A fragments of one 128-wide K step for weight row n = n0 + (lane % 16): lane group
// g = lane / 16 decodes K [32g, 32g+32) of the step into 4 x 8 bf16 (MFMA t takes
// elements 8t..8t+7).  `kk` is the step's first K index.
template <int FMT>
__device__ __forceinline__ void decode_a(const uint8_t *__restrict__ W, const uint8_t *__restrict__ S8, int K, int n,
                                         int kk, int g, v4u af[4]) {
  if constexpr (FMT == kW4) {
    const v4u a = ld16(W + (size_t)n * (K >> 1) + ((kk + 32 * g) >> 1));
    const float sc = e8m0_to_f32(S8[(size_t)n * (K >> 5) + (kk >> 5) + g]);
#pragma unroll
    for (int q = 0; q < 4; q++)
      af[q] = v4u{cvt_fp4x2_bf16<0>(a[q], sc), cvt_fp4x2_bf16<1>(a[q], sc), cvt_fp4x2_bf16<2>(a[q], sc),
                  cvt_fp4x2_bf16<3>(a[q], sc)};
  } else {
    const uint8_t *p = W + (size_t)n * K + kk + 32 * g;
    const v4u a0 = ld16(p), a1 = ld16(p + 16);
    float sc = 1.0f;
    if constexpr (FMT == kW8T32) sc = e8m0_to_f32(S8[(size_t)(n >> 5) * (K >> 5) + (kk >> 5) + g]);
    af[0] = v4u{cvt_fp8x2_bf16s<false>(a0[0], sc), cvt_fp8x2_bf16s<true>(a0[0], sc), cvt_fp8x2_bf16s<false>(a0[1], sc),
                cvt_fp8x2_bf16s<true>(a0[1], sc)};
    af[1] = v4u{cvt_fp8x2_bf16s<false>(a0[2], sc), cvt_fp8x2_bf16s<true>(a0[2], sc), cvt_fp8x2_bf16s<false>(a0[3], sc),
                cvt_fp8x2_bf16s<true>(a0[3], sc)};
    af[2] = v4u{cvt_fp8x2_bf16s<false>(a1[0], sc), cvt_fp8x2_bf16s<true>(a1[0], sc), cvt_fp8x2_bf16s<false>(a1[1], sc),
                cvt_fp8x2_bf16s<true>(a1[1], sc)};
    af[3] = v4u{cvt_fp8x2_bf16s<false>(a1[2], sc), cvt_fp8x2_bf16s<true>(a1[2], sc), cvt_fp8x2_bf16s<false>(a1[3], sc),
                cvt_fp8x2_bf16s<true>(a1[3], sc)};
  }
}

// NT weight tiles of 16 rows (rows n0[tt] + lane%16) times NCG groups of 16 bf16 activation
// rows (xrow[c], valid when xok[c]) over K [k0, k0 + kc).  acc[tt][c] lane l holds
// C[4*(l/16) + r][l%16]: weight row n0[tt] + 4*(l/16) + r, activation row 16c + l%16.
template <int FMT, int NT, int NCG>
__device__ void bf16_tiles(const uint8_t *__restrict__ W, const uint8_t *__restrict__ S8,
                           const float *__restrict__ S32, int K, const int n0[NT], int k0, int kc,
                           const uint16_t *const xrow[NCG], const bool xok[NCG], v4f acc[NT][NCG], int lane) {
  const int i = lane & 15, g = lane >> 4;
  const int steps = kc >> 7;
  for (int s = 0; s < steps; s++) {
    const int kk = k0 + 128 * s;
    v4u af[NT][4];
#pragma unroll
    for (int tt = 0; tt < NT; tt++) decode_a<FMT>(W, S8, K, n0[tt] + i, kk, g, af[tt]);
#pragma unroll
    for (int c = 0; c < NCG; c++) {
      v4u b[4];
#pragma unroll
      for (int t = 0; t < 4; t++) b[t] = xok[c] ? ld16(xrow[c] + kk + 32 * g + 8 * t) : v4u{0, 0, 0, 0};
#pragma unroll
      for (int tt = 0; tt < NT; tt++) {
        if constexpr (FMT == kW8B128) {
          v4f t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int q = 0; q < 4; q++) t = mfma_bf16(af[tt][q], b[q], t);
          acc[tt][c] += S32[(size_t)(n0[tt] >> 7) * (K >> 7) + (kk >> 7)] * t;
        } else {
#pragma unroll
          for (int q = 0; q < 4; q++) acc[tt][c] = mfma_bf16(af[tt][q], b[q], acc[tt][c]);
        }
      }
    }
  }
}

// One task (16-row tile, K chunk) of a dense linear y = x . W^T with bf16 rows x [M][K]:
// writes the chunk's partial sums to part[ks][M][N].
template <int FMT>
__device__ void linear_task(int t, int lane, const uint8_t *W, const uint8_t *S8, const float *S32, int N, int K,
                            int kc, const uint16_t *x, int M, float *part) {
  const int ntile = N >> 4;
  const int ks = t / ntile, nt = t - ks * ntile;
  const int i = lane & 15, g = lane >> 4;
  float *out = part + (size_t)ks * M * N;
  auto run = [&](auto ncg_c) {
    constexpr int NCG = decltype(ncg_c)::value;
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
    const int n0[1] = {nt * 16};
    bf16_tiles<FMT, 1, NCG>(W, S8, S32, K, n0, ks * kc, kc, xrow, xok, acc, lane);
#pragma unroll
    for (int c = 0; c < NCG; c++) {
      const int m = 16 * c + i;
      if (m < M) {
#pragma unroll
        for (int r = 0; r < 4; r++) out[(size_t)m * N + nt * 16 + 4 * g + r] = acc[0][c][r];
      }
    }
  };
  const int ncg = (M + 15) >> 4;
  if (ncg == 1)
    run(std::integral_constant<int, 1>{});
  else if (ncg == 2)
    run(std::integral_constant<int, 2>{});
  else
    run(std::integral_constant<int, 3>{});
}

template <int FMT>
__device__ void linear_all(const Ctx &cx, const uint8_t *W, const uint8_t *S8, const float *S32, int N, int K, int kc,
                           const uint16_t *x, int M, float *part) {
  const int T = (N >> 4) * (K / kc);
  for (int t = cx.gw; t < T; t += cx.nw) linear_task<FMT>(t, cx.lane, W, S8, S32, N, K, kc, x, M, part);
}

__device__ __forceinline__ float swiglu_clamp(float g, float u, float lim) {
  g = fminf(g, lim);
  u = fminf(fmaxf(u, -lim), lim);
  return g / (1.0f + expf(-g)) * u;
}

// Claim the next task of a device queue (one atomic per wave); returns the task id.
__device__ __forceinline__ int claim_task(unsigned *ctr, int lane) {
  unsigned t = 0;
  if (lane == 0) t = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return __shfl((int)t, 0, kWave);
}

}  // namespace dsl
