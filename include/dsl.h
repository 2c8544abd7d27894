/*
 * dsl.h -- one DeepSeek-V4.1-style decode layer (M <= 48 rows) as one persistent
 * HIP launch on MI355X (gfx950).  C ABI: plain pointers and sizes only.
 *
 * What a step computes ("Mono decode layer for DeepSeek-V4.1-Flash on MI355X",
 * vLLM PR 60397, Purpose, launch table rows K1 and K2):
 *   attention front  RMSNorm(x) -> MXFP8 quantize -> wqkv -> q/kv RMSNorm ->
 *                    fp8 KV-record insert -> MXFP8 quantize -> wq_b
 *   attention back   sliding-window split attention -> log-sum-exp combine ->
 *                    wo_a -> wo_b (each MXFP8, 32x32 E8M0 weight tiles)
 *   MoE              f32 router logits -> top-k (softmax over the selected k) ->
 *                    FP8 shared expert + MXFP4 routed experts, clamped SwiGLU ->
 *                    fixed-order f32 combine
 * with a pre-norm residual: hres = bf16(x + attn), out = bf16(hres + MoE(RMSNorm(hres))).
 * The tensor-parallel all-reduces of the pages are not part of this library.
 *
 * Conventions
 *   - Every call returns 0 or a negative DSL_E* code; dsl_last_error() gives the
 *     message (thread-local).  All argument checks run on the host before any
 *     launch, so every refusal is testable without a GPU.
 *   - Step calls are asynchronous on the given stream (NULL = the null stream).
 *     A device-side failure (a grid barrier that never completed, a slot outside
 *     the cache) is reported by dsl_layer_health().
 *   - The caller owns x, out, the weights, the KV caches and the tables; the
 *     handle owns its sync buffer and one scratch buffer per step width.  The
 *     kernels stream the caller's weight buffers directly and keep no copy of
 *     them (PR 60397, Design).  A handle is not thread-safe, and two steps of
 *     one handle must not run concurrently on different streams.
 *   - Step widths M are 1..dims.max_rows (max_rows <= 48: "Scope", decode only,
 *     at most 48 rows).  Each width gets its own scratch at its first step
 *     ("Design": a scratch per step width); dsl_layer_reserve() allocates it
 *     ahead of time (call it before capturing a step into a HIP graph).
 *   - A step is one plain launch of one block per compute unit (all a unit holds of
 *     this kernel), and its stages meet at grid barriers, so it needs every block
 *     resident at once: give it the device.  A concurrent kernel that holds compute
 *     units only delays it; one that holds them past the barrier's bounded wait
 *     (2^24 polls of the release word, each a device-memory round trip) makes the
 *     step report DSL_EDEVICE instead of hanging.
 *   - positions[r] = -1 marks a pad row: no KV write, ids -1, weights 0 and zero
 *     rows in every output (PR 60397, Test Plan: padded steps mark their unused
 *     rows with slot -1 and the kernels leave them out).  Rows of one request must
 *     have distinct positions.
 */
#ifndef DSL_H
#define DSL_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSL_OK 0
#define DSL_EINVAL (-1)       /* a null pointer, a bad stride, a size out of range  */
#define DSL_EUNSUPPORTED (-2) /* dims or widths the kernels do not cover; not gfx950;
                                 the kernel's block does not fit a compute unit  */
#define DSL_ENOMEM (-3)       /* device allocation failed                            */
#define DSL_EHIP (-4)         /* a HIP runtime call failed (message has the code)    */
#define DSL_EDEVICE (-5)      /* dsl_layer_health: a device-side fault was recorded  */

#define DSL_MAX_ROWS 48
#define DSL_MAX_LAYERS 4

/* Layer dimensions.  All sizes in elements.  Constraints checked by
 * dsl_layer_build: hidden, q_rank, o_rank, inter, shared_inter and
 * n_heads*head_dim positive multiples of 128 (the kernels stream K in steps of
 * 128; the shared expert has 128x128 scale blocks); head_dim in {64, 128, 256,
 * 512}; 1 <= n_experts <= 128; 1 <= top_k <= min(8, n_experts);
 * 1 <= max_rows <= 48; 1 <= n_layers <= DSL_MAX_LAYERS; 1 <= window <= 256;
 * expert_a8 in {0, 1, 2};
 * 0 <= swa_width <= 256 (a row's keys are split over at most 8 waves of 32 keys);
 * kv_block >= 1.  Other values: DSL_EUNSUPPORTED or DSL_EINVAL. */
typedef struct {
  int32_t hidden, n_heads, head_dim, q_rank, o_rank;
  int32_t window;      /* causal sliding window W; a row at position p sees
                          positions [max(0, p-W+1), p] of its request          */
  int32_t swa_width;   /* 0 = causal window mode; > 0 = index-table mode: each
                          row attends to the slots of its key_table row (the draft
                          layers' non-causal rows, 192 wide for window 128 and 5
                          drafts: "Mono decode for the DSpark draft layers",
                          vLLM PR 62131, Details)                               */
  int32_t n_experts, top_k, inter, shared_inter;
  int32_t kv_block;    /* B, tokens per cache block                             */
  int32_t max_rows;    /* largest step width                                    */
  int32_t n_layers;    /* chained layers per step (3 for the draft model)       */
  int32_t expert_a8;   /* 0: the routed experts take the bf16 MoE input (W4A16);
                          1: they take MXFP8 activations (A8W4, the pages' "a8w4
                          MoE": PR 60397, Test Plan): gate/up reads MXq(u) and down
                          reads MXq(z), each per 1x32 block of the bf16 value.  The
                          router and the shared expert keep the bf16 u.
                          2: the same A8W4 layer, with the experts on the matrix
                          cores taking the raw e2m1 and e4m3 codes and their E8M0
                          block exponents on the gfx950 scaled MX instruction
                          (v_mfma_scale_f32_16x16x128_f8f6f4) instead of their
                          exact bf16 values; same products, f32 sums in another
                          order.                                                    */
  float norm_eps;      /* RMSNorm epsilon (1e-6)                                */
  float swiglu_limit;  /* SwiGLU clamp (7.0)                                    */
} dsl_dims;

/* Device pointers to one layer's weights, caller-owned, read in place; they must
 * stay valid until dsl_layer_destroy.  Formats ("Design" and "Layout"):
 *   norms          f32 gammas: attn_norm, ffn_norm [hidden]; q_norm [q_rank];
 *                  kv_norm [head_dim]
 *   MXFP8 linears  e4m3 row-major [N][K] plus one E8M0 byte per 32x32 tile,
 *                  row-major [N/32][K/32]:
 *                  wqkv [q_rank+head_dim][hidden] (q latent rows first),
 *                  wq_b [n_heads*head_dim][q_rank], wo_a [o_rank][n_heads*head_dim],
 *                  wo_b [hidden][o_rank]
 *   router         f32 [n_experts][hidden]
 *   shared expert  e4m3 row-major, f32 scale per 128x128 block:
 *                  sh_w13 [2*shared_inter][hidden] (gate rows, then up rows),
 *                  sh_w13_s [2*shared_inter/128][hidden/128];
 *                  sh_wd [hidden][shared_inter], sh_wd_s [hidden/128][shared_inter/128]
 *   routed experts e2m1 nibbles, low nibble = even k, one E8M0 per 32 along k:
 *                  ex_w13 [n_experts][2*inter][hidden/2], ex_w13_s [n_experts][2*inter][hidden/32]
 *                  ex_wd  [n_experts][hidden][inter/2],   ex_wd_s  [n_experts][hidden][inter/32]
 * All pointers 16-byte aligned. */
typedef struct {
  const float *attn_norm, *q_norm, *kv_norm, *ffn_norm;
  const uint8_t *wqkv, *wqkv_s, *wq_b, *wq_b_s, *wo_a, *wo_a_s, *wo_b, *wo_b_s;
  const float *w_router;
  const uint8_t *sh_w13;
  const float *sh_w13_s;
  const uint8_t *sh_wd;
  const float *sh_wd_s;
  const uint8_t *ex_w13, *ex_w13_s, *ex_wd, *ex_wd_s;
} dsl_weights;

/* One layer's block-paged fp8 KV cache, written in place at each live row's slot.
 * Record (RECORD = head_dim + 16 bytes): head_dim e4m3 codes, then the f32 scale
 * s = amax/448, then 12 zero bytes.  The cache is a [blocks][B][RECORD] view whose
 * block stride must be at least B*RECORD ("[SpecializedDecode] review thread",
 * vLLM PR 61311: the stride check) and a multiple of 16.  The slot of position p
 * of request q is block_table[q][p / B] * B + p % B.  All pointers are device
 * pointers. */
typedef struct {
  uint8_t *base;
  int64_t block_stride;       /* bytes                                           */
  int64_t n_blocks;           /* physical blocks in the view (slot bound)        */
  const int32_t *block_table; /* [n_req][max_blocks] physical block ids          */
  int32_t max_blocks;
  int32_t n_req;              /* rows of block_table (request index bound)       */
  const int32_t *row_req;     /* [M] request index of each row                   */
  const int32_t *key_table;   /* [M][swa_width] physical slots or -1 (index-table
                                 mode only; NULL otherwise)                       */
} dsl_kv;

/* Optional intermediate outputs of the last layer of a step (NULL = not written). */
typedef struct {
  void *attn_out;     /* bf16 [M][hidden]: attention branch output bf16(a)       */
  void *hres;         /* bf16 [M][hidden]: residual after attention             */
  void *moe_in;       /* bf16 [M][hidden]: RMSNorm_ffn(hres), the MoE input      */
  void *moe_out;      /* bf16 [M][hidden]: MoE branch output                     */
  int32_t *topk_ids;  /* [M][top_k], emitted in descending logit order           */
  float *topk_w;      /* [M][top_k]                                              */
  float *logits;      /* [M][n_experts] f32 router logits                        */
  int32_t *layer_ids; /* [n_layers][M][top_k]: the expert ids of every layer     */
} dsl_taps;

typedef struct dsl_layer dsl_layer;

/* Validate dims, query the current device (must be gfx950, and one block of the
 * layer kernel must fit on a compute unit), copy the n_layers weight descriptors (not the weights) and
 * allocate the sync buffer.  weights points to dims->n_layers descriptors.
 * On success *out receives the handle.  Errors: DSL_EINVAL, DSL_EUNSUPPORTED,
 * DSL_ENOMEM, DSL_EHIP. */
int dsl_layer_build(const dsl_dims *dims, const dsl_weights *weights, dsl_layer **out);

/* Allocate the scratch of width M now (otherwise the first step of that width does). */
int dsl_layer_reserve(dsl_layer *layer, int32_t M);

/* One decode step over n_layers chained layers: x bf16 [M][hidden] in, out bf16
 * [M][hidden].  kv points to n_layers cache descriptors (their tables may be
 * shared); positions [M] int32 device array.  taps may be NULL. */
int dsl_decode_step(dsl_layer *layer, const void *x_bf16, int32_t M, const dsl_kv *kv,
                    const int32_t *positions, void *out_bf16, const dsl_taps *taps,
                    void *hip_stream);

/* dsl_decode_step without any allocation, for callers that cannot allocate device
 * memory at step time: code under HIP graph capture (a width's first dsl_decode_step
 * allocates its scratch), tight serving loops, harnesses that forbid allocation.  Same
 * arguments, kernels and results as dsl_decode_step; the step's scratch is a static
 * device array of 32 MiB per GPU (held until the process ends) instead of the width's
 * own, and the call makes no hipMalloc, hipFree or other allocating call.  Limit: the
 * scratch of M rows over dims.n_layers layers must fit 32 MiB (every width up to 48 rows
 * of one layer at hidden 4096 / 128 experts / inter 2048, or three such layers up to 16
 * rows); beyond it the call returns DSL_EUNSUPPORTED and launches nothing.  Every handle
 * on a GPU shares that GPU's array, so two such calls that can overlap on one GPU (two
 * streams, two threads) race: order them on one stream.  No word of the array is read
 * before the step writes it, so it needs no clearing between calls. */
int dsl_decode_step_noalloc(dsl_layer *layer, const void *x_bf16, int32_t M, const dsl_kv *kv,
                            const int32_t *positions, void *out_bf16, const dsl_taps *taps,
                            void *hip_stream);

/* The attention half of layer 0 only: attn_out = bf16(a), no residual add.  Writes
 * the KV records like a full step. */
int dsl_attn_step(dsl_layer *layer, const void *x_bf16, int32_t M, const dsl_kv *kv,
                  const int32_t *positions, void *attn_out_bf16, void *hip_stream);

/* The MoE of layer 0 only, on an already normalized input u bf16 [M][hidden]:
 * moe_out = bf16(shared + sum_j w_j expert_j).  topk_ids [M][top_k] and topk_w
 * [M][top_k] may be NULL. */
int dsl_moe_step(dsl_layer *layer, const void *u_bf16, int32_t M, void *moe_out_bf16,
                 int32_t *topk_ids, float *topk_w, void *hip_stream);

/* A skinny MXFP8 linear, y = MXq(x) . W^T, with float32 accumulation and output: the draft
 * step's head GEMMs ("Mono decode for the DSpark draft layers", vLLM PR 62131, Details, where
 * they are the step's largest cost after its layers), read here in the format and numerics of
 * the layer's other dense linears (PR 60397, Design).  No handle: the call is stateless.
 *   x    bf16 [M][K] device rows, 16-byte aligned; 1 <= M <= 48, K a multiple of 128.
 *        Each 1x32 block along K is MXFP8-quantized (OCP MX: block exponent from the
 *        float32 amax, e4m3 elements rounded to nearest even and saturated) before the
 *        product, as for the layer's attention linears.
 *   w    e4m3 row-major [N][K], 16-byte aligned; w_s one E8M0 per 32x32 tile [N/32][K/32];
 *        N a multiple of 32.  Read in place.
 *   y    float32 [M][N], 16-byte aligned, written whole.
 *   workspace  device memory of dsl_linear_workspace_bytes(M, N, K) bytes, 256-byte
 *        aligned, owned by the caller; overwritten (the quantized rows, and float32 split-K
 *        partials when N / 16 output tiles alone would not fill the grid).
 * Asynchronous on hip_stream (three launches).  Errors: DSL_EUNSUPPORTED for sizes outside
 * the above, DSL_EINVAL for NULL or misaligned pointers, DSL_EHIP for a failed launch. */
int dsl_linear_mxfp8(const void *x_bf16, int32_t M, int32_t K, const uint8_t *w, const uint8_t *w_s, int32_t N,
                     float *y, void *workspace, void *hip_stream);

/* Bytes of workspace dsl_linear_mxfp8 needs for these sizes, or -1 (with dsl_last_error) for
 * sizes it does not take. */
int64_t dsl_linear_workspace_bytes(int32_t M, int32_t N, int32_t K);

/* Synchronizes nothing; reads the device health word after the caller has
 * synchronized.  0 = healthy; DSL_EDEVICE after a recorded device fault (the word
 * is then cleared and the handle's sync state reset). */
int dsl_layer_health(dsl_layer *layer);

/* Tracing for profiling: with on != 0, thread 0 of every block of every later
 * launch stamps the device wall clock at the launch's start, on arriving at and on
 * leaving each grid barrier, at a few points inside the MoE stage and at the end.
 * dsl_layer_read_trace copies the stamps of the most recent traced launch (call
 * after synchronizing) into ns[mark * grid_blocks + block] as nanoseconds since
 * block 0's first stamp (-1 where a block wrote none), for up to n_marks marks
 * (ns holds n_marks * grid_blocks doubles, see dsl_layer_grid), and returns the
 * number of marks written. */
int dsl_layer_set_trace(dsl_layer *layer, int32_t on);
int dsl_layer_read_trace(dsl_layer *layer, double *ns, int32_t n_marks);

/* Which instantiation of the layer kernel the handle's most recent step launched: 1 =
 * the narrow one (steps of at most 8 rows at hidden 4096, q/o rank 1024, head dim 512),
 * 0 = the general one, -1 = no step yet (DSL_EINVAL for a NULL handle).  For tests and
 * reports: the results do not depend on it. */
int dsl_layer_last_kernel(const dsl_layer *layer);

/* Grid the persistent launch uses (blocks, threads per block); for reports. */
int dsl_layer_grid(const dsl_layer *layer, int32_t *blocks, int32_t *threads);

void dsl_layer_destroy(dsl_layer *layer);

const char *dsl_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* DSL_H */
