// A skinny MXFP8 linear, y = MXq(x) . W^T for a few bf16 rows x [M][K] (M <= 48) and a
// row-major e4m3 weight [N][K] with one E8M0 per 32x32 tile, on the same weight-streaming
// matrix-core tiles as the decode layer's attention linears.  Its use: the draft step's head
// GEMMs, which the draft-layer page names as the step's largest remaining cost ("Mono decode
// for the DSpark draft layers", vLLM PR 62131, Details); the page gives their number and time,
// not their shapes or formats, and the readings taken here are the MXFP8 format and numerics
// of the pages' other dense linears ("Mono decode layer for DeepSeek-V4.1-Flash on MI355X",
// vLLM PR 60397, Design: MXFP8 activations quantized per 1x32 block, 32x32 E8M0 weight
// tiles) with a float32 output.
//
// Three launches on the caller's stream: the activations' MXFP8 quantization (kept as exact
// bf16 values) into the workspace; the tiles (task = 16 weight rows times a K chunk; the K
// chunk is all of K when the output tiles alone fill the grid, else split so that tasks do,
// with float32 partials in the workspace); the partials summed in chunk order.
#include <hip/hip_runtime.h>

#include <cstdio>

#include "dsl_stages.h"

namespace dsl {

constexpr int kLinWaves = 1024;  // split K only while the output tiles fill fewer waves (half of the 2048)

// MXFP8 of each 32-block of the rows, one thread per block
__global__ void __launch_bounds__(256) lin_mxq_kernel(const uint16_t *x, uint16_t *xq, int M, int K) {
  const int per = K >> 5, b = blockIdx.x * 256 + threadIdx.x;
  if (b >= M * per) return;
  const size_t off = (size_t)(b / per) * K + 32 * (b % per);
  float v[32];
  load_bf16<32>(x + off, v);
  mx_quant_dequant<32>(v);
  store_bf16<32>(xq + off, v);
}

// Task t = (K chunk t / ntile, 16-row tile t % ntile) to wave t of the grid (one task per
// wave: the host sizes the grid); partials of chunk ks to part[ks][M][N]
template <int NCG>
__global__ void __launch_bounds__(kThreads, 1) lin_tiles_kernel(const uint16_t *xq, int M, int K, const uint8_t *W,
                                                              const uint8_t *S, int N, int kc, float *part) {
  const int t = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6), T = (N >> 4) * (K / kc);
  if (t >= T) return;
  linear_task_n<kW8T32, NCG>(t, threadIdx.x & 63, W, S, nullptr, N, K, kc, xq, M, part, nullptr, false);
}

// y[m][n] = sum over ks (in order) of part[ks][m][n]
__global__ void __launch_bounds__(256) lin_sum_kernel(const float *part, int nks, int MN, float *y) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= MN) return;
  float v = part[i];
  for (int ks = 1; ks < nks; ks++) v += part[(size_t)ks * MN + i];
  y[i] = v;
}

// K chunk: all of K while the output tiles fill the waves, else halved (staying a multiple
// of 128 that divides K) until the tasks do
static int lin_kc(int N, int K) {
  int kc = K;
  while ((N >> 4) * (K / kc) < kLinWaves && kc % 256 == 0 && K % (kc / 2) == 0) kc /= 2;
  return kc;
}

static size_t lin_xq_bytes(int M, int K) { return ((size_t)M * K * 2 + 255) & ~(size_t)255; }

}  // namespace dsl

using namespace dsl;

static int lin_check(int32_t M, int32_t N, int32_t K) {
  char buf[256];
  if (M < 1 || M > DSL_MAX_ROWS) {
    snprintf(buf, sizeof buf, "rows %d outside 1..%d", M, DSL_MAX_ROWS);
    return set_error(DSL_EUNSUPPORTED, buf);
  }
  if (K < 128 || K % 128) {
    snprintf(buf, sizeof buf, "K %d is not a positive multiple of 128", K);
    return set_error(DSL_EUNSUPPORTED, buf);
  }
  if (N < 32 || N % 32) {
    snprintf(buf, sizeof buf, "N %d is not a positive multiple of 32", N);
    return set_error(DSL_EUNSUPPORTED, buf);
  }
  return 0;
}

extern "C" {

int64_t dsl_linear_workspace_bytes(int32_t M, int32_t N, int32_t K) {
  if (lin_check(M, N, K)) return -1;
  const int kc = lin_kc(N, K), nks = K / kc;
  return (int64_t)(lin_xq_bytes(M, K) + (nks > 1 ? (size_t)nks * M * N * 4 : 0));
}

int dsl_linear_mxfp8(const void *x, int32_t M, int32_t K, const uint8_t *w, const uint8_t *w_s, int32_t N, float *y,
                     void *workspace, void *stream) {
  int rc = lin_check(M, N, K);
  if (rc) return rc;
  if (!x || !w || !w_s || !y || !workspace) return set_error(DSL_EINVAL, "x, w, w_s, y and workspace must be set");
  if (((uintptr_t)x | (uintptr_t)w | (uintptr_t)y) & 15) return set_error(DSL_EINVAL, "x, w and y must be 16-byte aligned");
  if ((uintptr_t)workspace & 255) return set_error(DSL_EINVAL, "workspace must be 256-byte aligned");
  const int kc = lin_kc(N, K), nks = K / kc, T = (N >> 4) * nks;
  uint16_t *xq = (uint16_t *)workspace;
  float *part = nks > 1 ? (float *)((char *)workspace + lin_xq_bytes(M, K)) : y;
  hipStream_t st = (hipStream_t)stream;
  char buf[256];
  hipLaunchKernelGGL(lin_mxq_kernel, dim3((M * (K >> 5) + 255) / 256), dim3(256), 0, st, (const uint16_t *)x, xq, M, K);
  const dim3 grid((T + kWavesPerBlock - 1) / kWavesPerBlock), block(kThreads);
  const int ncg = (M + 15) >> 4;
  if (ncg == 1)
    hipLaunchKernelGGL(lin_tiles_kernel<1>, grid, block, 0, st, xq, M, K, w, w_s, N, kc, part);
  else if (ncg == 2)
    hipLaunchKernelGGL(lin_tiles_kernel<2>, grid, block, 0, st, xq, M, K, w, w_s, N, kc, part);
  else
    hipLaunchKernelGGL(lin_tiles_kernel<3>, grid, block, 0, st, xq, M, K, w, w_s, N, kc, part);
  if (nks > 1) hipLaunchKernelGGL(lin_sum_kernel, dim3((M * N + 255) / 256), dim3(256), 0, st, part, nks, M * N, y);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    snprintf(buf, sizeof buf, "launch failed: %s", hipGetErrorString(e));
    return set_error(DSL_EHIP, buf);
  }
  return 0;
}

}  // extern "C"
