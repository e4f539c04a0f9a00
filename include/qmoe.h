/*
 * qmoe.h - C ABI of the routed-expert MoE FFN library for AMD MI355X (gfx950).
 *
 * The library computes one routed mixture-of-experts FFN layer of a top-k MoE decoder
 * whose experts are stored as block-quantized low-bit weights:
 *
 *   moe_route              router top-k over expert logits, routing weights over the k
 *                          selected experts, and the token-expert pairs grouped by
 *                          expert. (Strata engine explainer, m.lqnn.cn/news/264700,
 *                          sections "Architecture overview" - the router picks the 10
 *                          active experts of 512 per token - and "Doorbell handshake" -
 *                          expert ids travel together with routing weights; grouping
 *                          by expert as in section "Expert cache", where cached experts
 *                          run in a grouped kernel over the verify window.)
 *   moe_expert_ffn_decode  the expert FFN for a small verify window (T <= 5 tokens per
 *                          sequence, "Speculative decoding" section: 3 drafted tokens,
 *                          up to 5 copied by prompt lookup): int8 block quantization of
 *                          the activations, dequantized low-bit gate/up weights through
 *                          exact per-block int8 dot products ("CPU expert pool" section:
 *                          int8 dot products, activation quantized once and reused over
 *                          many weight rows), SwiGLU, int8 quantization of the hidden
 *                          vector, the down projection, and the routing-weighted combine
 *                          written into the residual ("Doorbell handshake": combine,
 *                          then residual write-back).
 *   moe_expert_ffn_prefill the same layer for a prefill chunk of up to 8192 tokens
 *                          ("Architecture overview": prompts are cut into chunks of at
 *                          most 8192 tokens) with bf16 dequantized weights, bf16
 *                          activations and fp32 accumulation on the matrix cores.
 *
 * Conventions for every entry point:
 *   * Pointers named device are GPU memory of the current HIP device; the caller owns
 *     all memory, including the workspace. The library allocates nothing.
 *   * `stream` is a hipStream_t (NULL = the null stream). Work is enqueued on it and the
 *     call returns without waiting. Calls on one stream are ordered; calls that share
 *     output or workspace buffers must not run concurrently on different streams.
 *   * Arguments are validated before anything is enqueued; on any error nothing is
 *     enqueued. MOE_ERR_HIP means a launch failed; faults during execution surface at
 *     the caller's next synchronization with the stream.
 *   * n_tokens == 0 is valid: the FFN entry points then enqueue nothing, and moe_route
 *     only writes expert_offsets (all zero; the other routing pointers may be NULL).
 *
 * Packed weight layout (one moe_qmatrix holds all E experts of one projection):
 *   codes      uint32 [E][cols/32][rows][bits]   32 unsigned codes of `bits` bits per
 *              block of 32 consecutive columns; code i (0..31) of a block sits in word
 *              i/(32/bits) at bit offset bits*(i % (32/bits)).
 *   scale_min  uint16 [E][cols/32][rows][2]      fp16 scale and fp16 min per block.
 *   weight     w[e][r][c] = scale * code + min    (block b = c/32)
 *   The block axis is the reduction axis (cols); blocks are stored block-column-major
 *   so that one block column of consecutive rows is contiguous (16 B per row at 4-bit,
 *   8 B at 2-bit). codes must be 16-byte aligned, scale_min 4-byte aligned.
 * Projections: gate and up are [rows = d_ff][cols = d_model], down is
 *   [rows = d_model][cols = d_ff]; bits is 4 or 2, the same for all three.
 */
#ifndef QMOE_H
#define QMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1,
  MOE_ERR_UNSUPPORTED = 2,
  MOE_ERR_WORKSPACE_TOO_SMALL = 3,
  MOE_ERR_HIP = 4
} moe_status;

/* Limits checked by every entry point. */
#define MOE_MAX_EXPERTS 1024       /* n_experts                                  */
#define MOE_MAX_TOP_K 64           /* top_k                                      */
#define MOE_MAX_DECODE_TOKENS 512  /* n_tokens of moe_expert_ffn_decode          */
#define MOE_MAX_PREFILL_TOKENS 8192 /* n_tokens of moe_expert_ffn_prefill         */
#define MOE_MAX_ROUTE_TOKENS 65536 /* n_tokens of moe_route                      */

typedef struct {
  const uint32_t* codes;     /* device, [E][cols/32][rows][bits]                    */
  const uint16_t* scale_min; /* device, [E][cols/32][rows][2] fp16 (scale, min)      */
  int32_t rows, cols, bits;
} moe_qmatrix;

typedef struct {
  int32_t d_model;   /* d: multiple of 32, at most 8192                            */
  int32_t d_ff;      /* f: multiple of 32, at most 8192                            */
  int32_t n_experts; /* E: 1..MOE_MAX_EXPERTS                                      */
  int32_t top_k;     /* k: 1..min(E, MOE_MAX_TOP_K)                                */
  moe_qmatrix gate, up, down;
  /* Optional shared expert: one always-active expert in the routed experts' shape and
   * format (rows, cols and bits as gate, up and down; one expert each), run for every
   * token and added to the residual with weight 1 after the routed slots (the model
   * table of the Strata pages counts "10+1" active experts per token, and the engine
   * explainer's memory table keeps a shared expert on the GPU; the pages give it no
   * gate). shared_gate.codes == NULL: none (the other two are then ignored). Supported by
   * the decode entry points for windows of n <= 8 tokens with n*k <= 64 pairs, k + 1 <=
   * 16, d_ff <= 1024, ceil((k+1)/2) * ceil(d_ff/256) <= 18 (k <= 10 at d_ff = 768) and
   * the down and combine stages issued together; otherwise, and by the prefill entry
   * points, MOE_ERR_UNSUPPORTED. */
  moe_qmatrix shared_gate, shared_up, shared_down;
  /* Optional router weights, for moe_layer_decode called without logits: bf16 bit
   * patterns, [E][d] row-major (row e holds expert e's weights), 16-byte aligned.
   * logits[t][e] = sum_c x[t][c] * router_w[e][c], each product exact and the sum in
   * binary64, rounded once to fp32 (the engine explainer's memory table keeps the router
   * on the GPU; the pages give no precision for its weights). NULL: none. */
  const uint16_t* router_w;
} moe_layer;

/* Routing record of n tokens (all device memory), written by moe_route and read by the
 * FFN entry points:
 *   topk_ids        int32 [n][k]  expert of slot j of token t; slot 0 has the largest
 *                                 logit; equal logits (-0 equals +0) order by lower id
 *   topk_w          fp32  [n][k]  w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0) over the
 *                                 k selected (= softmax, then renormalised over the k)
 *   expert_offsets  int32 [E+1]   pairs of expert e are pair_index[off[e] .. off[e+1])
 *   pair_index      int32 [n*k]   pair ids p = t*k + j, grouped by expert, ascending p
 *                                 within an expert (stable counting sort) */
typedef struct {
  int32_t* topk_ids;
  float* topk_w;
  int32_t* expert_offsets;
  int32_t* pair_index;
} moe_routing;

/* Optional intermediate outputs of moe_expert_ffn_decode, for checking (each may be
 * NULL; passing a non-NULL moe_debug selects a slower instance of the same kernels).
 * p = t*k + j is the pair id; with a shared expert, token t's shared pair is p = n*k + t
 * and the [n*k] extents below become [n*k + n]. Layouts:
 *   xq int8 [n][d], xs fp32 [n][d/32]            activation codes and block scales
 *   gate_dots, up_dots int32 [n*k][f][d/32]       exact per-block integer dots
 *   g, u fp32 [n*k][f]                            gate/up projections (rounded to fp32)
 *   h fp32 [n*k][f]                               SwiGLU output, the value quantized
 *   hq int8 [n*k][f], hs fp32 [n*k][f/32]         hidden codes and block scales
 *   down_dots int32 [n*k][d][f/32]                exact per-block integer dots
 *   y fp32 [n*k][d]                               expert output of each pair
 *   logits fp32 [n][E]                            router logits (moe_layer_decode
 *                                                 projecting with router_w only) */
typedef struct {
  int8_t* xq;
  float* xs;
  int32_t* gate_dots;
  int32_t* up_dots;
  float* g;
  float* u;
  float* h;
  int8_t* hq;
  float* hs;
  int32_t* down_dots;
  float* y;
  float* logits;
} moe_debug;

/* Human-readable name of a status code (static storage). */
const char* moe_status_string(moe_status s);

/* Bytes of device workspace moe_route needs for these sizes: 0 up to 64 tokens or 4096
 * token-expert pairs; above that, per-chunk expert histograms of a grouping spread over
 * many workgroups (4 bytes per expert per 2048 pairs). Returns 0 for sizes out of range. */
size_t moe_route_workspace_bytes(int n_tokens, int n_experts, int top_k);

/* Router top-k, routing weights and grouping (see moe_routing for the outputs).
 * logits: device fp32 [n_tokens][n_experts], finite values (NaN/Inf are a caller
 * error with unspecified selection). ws: device workspace of at least
 * moe_route_workspace_bytes(n, E, k) bytes, 256-byte aligned, no initialisation needed
 * (may be NULL when that is 0). Errors: MOE_ERR_INVALID_ARGUMENT for sizes out of range,
 * NULL outputs or a misaligned workspace; MOE_ERR_WORKSPACE_TOO_SMALL. */
moe_status moe_route(const float* logits, int n_tokens, int n_experts, int top_k,
                     const moe_routing* out, void* ws, size_t ws_bytes, void* stream);

/* Bytes of device workspace the FFN entry points need (prefill != 0 for
 * moe_expert_ffn_prefill). Returns 0 if the layer description is invalid. */
size_t moe_ffn_workspace_bytes(const moe_layer* L, int n_tokens, int prefill);

/* Decode-window expert FFN. x: device fp32 [n][d], the layer's MoE input; residual:
 * device fp32 [n][d], updated in place: residual[t] += sum_j w[t][j] * y[t*k+j] (slot
 * order; then the shared expert's output with weight 1, when the layer has one). x may
 * be the residual buffer itself (all of x is read before residual is
 * written); any other overlap is rejected. r: routing from moe_route for the same n,
 * E and k. ws: device workspace of at least moe_ffn_workspace_bytes(L, n, 0) bytes,
 * 256-byte aligned; its contents need no initialisation. dbg: NULL, or debug outputs.
 * Limits: n <= MOE_MAX_DECODE_TOKENS. */
moe_status moe_expert_ffn_decode(const moe_layer* L, const float* x, int n_tokens,
                                 const moe_routing* r, float* residual, void* ws,
                                 size_t ws_bytes, const moe_debug* dbg, void* stream);

/* Stages of moe_expert_ffn_decode, as bits of `stages` below. */
#define MOE_DECODE_PREP 1u     /* int8 quantization of x and the per-expert work list     */
#define MOE_DECODE_GATE_UP 2u  /* gate/up projections, SwiGLU (and for large windows the
                                  int8 quantization of h)                                 */
#define MOE_DECODE_DOWN 4u     /* (for small windows the int8 quantization of h) down
                                  projection of every token-expert pair                   */
#define MOE_DECODE_COMBINE 8u  /* routing-weighted combine into the residual              */
#define MOE_DECODE_ALL 15u

/* moe_expert_ffn_decode split into its stages, for callers that interleave other work
 * (or timing events) between them. The selected stages are enqueued in the order above;
 * a stage reads what the earlier stages wrote into `ws`, so every stage of one layer
 * call must be issued, in order, with the same arguments and workspace. Arguments and
 * errors as moe_expert_ffn_decode; stages == MOE_DECODE_ALL is moe_expert_ffn_decode.
 * MOE_ERR_INVALID_ARGUMENT if stages is 0 or has bits outside MOE_DECODE_ALL. */
moe_status moe_expert_ffn_decode_stages(const moe_layer* L, const float* x, int n_tokens,
                                        const moe_routing* r, float* residual, void* ws,
                                        size_t ws_bytes, const moe_debug* dbg, unsigned stages,
                                        void* stream);

/* The whole routed-expert layer for a decode window: moe_route followed by
 * moe_expert_ffn_decode on the same arguments. Windows of up to 16 tokens are routed inside
 * the first kernel of the layer, larger ones by the routing kernels of moe_route launched
 * first. The router hands expert ids and weights to the expert pass
 * (Strata engine explainer, m.lqnn.cn/news/264700, "Doorbell handshake": routing ends
 * the first half of a layer, combine and residual write-back end the second). logits:
 * device fp32 [n][E], or NULL when the layer has router weights (L->router_w): the
 * layer then projects x onto the router rows first (one more launch in the PREP stage;
 * the logits go to the workspace, and to dbg->logits when given). r receives the
 * routing exactly as moe_route writes it for those logits; all other arguments, limits
 * and errors as moe_expert_ffn_decode, plus MOE_ERR_INVALID_ARGUMENT for NULL logits
 * without router weights when n > 0. n == 0 only writes zero expert offsets. */
moe_status moe_layer_decode(const moe_layer* L, const float* logits, const float* x,
                            int n_tokens, const moe_routing* r, float* residual, void* ws,
                            size_t ws_bytes, const moe_debug* dbg, void* stream);

/* moe_layer_decode split into stages like moe_expert_ffn_decode_stages; here
 * MOE_DECODE_PREP also performs the routing. For windows of n <= 16 tokens with n*k <= 64
 * pairs the expert pass takes its chunks straight from the expert ids: PREP then writes
 * r's topk_ids and topk_w, and MOE_DECODE_GATE_UP writes r's expert_offsets and
 * pair_index; r is complete once both stages have run (always, after the whole call).
 * Larger windows write all of r in PREP. */
moe_status moe_layer_decode_stages(const moe_layer* L, const float* logits, const float* x,
                                   int n_tokens, const moe_routing* r, float* residual, void* ws,
                                   size_t ws_bytes, const moe_debug* dbg, unsigned stages,
                                   void* stream);

/* Bytes of the library's own decode workspace, used by moe_layer_decode_noalloc: one
 * array of this size per GPU the library runs on, held until the process ends. */
#define MOE_NOALLOC_SCRATCH_BYTES (16u << 20)

/* moe_layer_decode without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation). The workspace is the library's static per-GPU array of
 * MOE_NOALLOC_SCRATCH_BYTES bytes (enough for windows of 128 tokens at d_model = 2048,
 * d_ff = 768, top-10 with router weights, and for every window a shared expert allows);
 * nothing is allocated or freed by the call. Arguments, results and errors as moe_layer_decode (dbg = NULL),
 * plus MOE_ERR_WORKSPACE_TOO_SMALL when the sizes need more workspace than the array
 * holds (nothing is enqueued), and MOE_ERR_HIP if the array's device address cannot be
 * resolved. Every call on one GPU uses that GPU's one array, which keeps the last call's
 * contents (the decode path needs no initialised workspace): calls that overlap on one
 * GPU (on different streams, or from different host threads without ordering) race;
 * calls on one stream are ordered and safe. */
moe_status moe_layer_decode_noalloc(const moe_layer* L, const float* logits, const float* x,
                                    int n_tokens, const moe_routing* r, float* residual,
                                    void* stream);

/* Prefill-chunk expert FFN with bf16 arithmetic on the matrix cores: weights are
 * dequantized to bf16 (bf16 of fp32 scale*q + min), x_bf16: device bf16 bits [n][d];
 * gate/up accumulate in fp32; h = bf16(silu(g) * u); down accumulates in fp32;
 * residual (fp32 [n][d]) += routing-weighted sum of the pair outputs (binary64 sum in
 * slot order, rounded once). 4-bit and 2-bit weights. x_bf16 and residual must be
 * 16-byte aligned and must not overlap. r: routing from moe_route for the same n, E and k. ws: at
 * least moe_ffn_workspace_bytes(L, n, 1) bytes, 256-byte aligned, no initialisation
 * needed; it holds h (bf16 [n*k][f]) and the pair outputs (fp32 [n*k][d]).
 * Limits: n <= MOE_MAX_PREFILL_TOKENS; n == 0 enqueues nothing. */
moe_status moe_expert_ffn_prefill(const moe_layer* L, const uint16_t* x_bf16, int n_tokens,
                                  const moe_routing* r, float* residual, void* ws,
                                  size_t ws_bytes, void* stream);

/* Stages of moe_expert_ffn_prefill, as bits of `stages` below. */
#define MOE_PREFILL_PREP 1u     /* M-tile work list and token / grouped-position maps     */
#define MOE_PREFILL_GATE_UP 2u  /* gate/up grouped GEMM with SwiGLU, h in bf16            */
#define MOE_PREFILL_DOWN 4u     /* down grouped GEMM, fp32 pair outputs                   */
#define MOE_PREFILL_COMBINE 8u  /* routing-weighted combine into the residual            */
#define MOE_PREFILL_ALL 15u

/* moe_expert_ffn_prefill split into its stages, with the same contract as
 * moe_expert_ffn_decode_stages: the selected stages are enqueued in the order above and
 * every stage of one layer call must be issued, in order, with the same arguments and
 * workspace. stages == MOE_PREFILL_ALL is moe_expert_ffn_prefill.
 * MOE_ERR_INVALID_ARGUMENT if stages is 0 or has bits outside MOE_PREFILL_ALL. */
moe_status moe_expert_ffn_prefill_stages(const moe_layer* L, const uint16_t* x_bf16,
                                         int n_tokens, const moe_routing* r, float* residual,
                                         void* ws, size_t ws_bytes, unsigned stages,
                                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QMOE_H */
