/*
 * moe.h -- C ABI of the fused Mixture-of-Experts expert layer for AMD MI355X
 * (gfx950). Library: grouped_gemm_softmax_amd/libmoe.so.
 *
 * The layer, per token t of x[T,H]:
 *   1. route    : the k experts with the largest router logits (equal logits
 *                 taken in ascending expert order) and routing weights
 *                 w[t,j] = softmax over those k logits;
 *   2. permute  : the T*k (token, slot) assignments sorted stably by expert
 *                 into per-expert contiguous row blocks of x_perm;
 *   3. gate/up  : per expert e, h = silu(x_perm_e W_gate[e]) * (x_perm_e W_up[e]),
 *                 one grouped GEMM with the SwiGLU in its epilogue, so the gate
 *                 and up products never reach memory;
 *   4. down     : y_perm_e = h_e W_down[e], a second grouped GEMM;
 *   5. combine  : out[t] = sum_j w[t,j] * y_perm[row of (t,j)]
 *                 (+ s_t * shared_expert(x[t]) when a shared expert is given).
 * Sources: the dispatch-kernel post "Triton-MoE-Dispatch-Kernel erreicht
 * 131 % von Megablocks" (lumeric.app), summary paragraph (fused gate+up with
 * SwiGLU, 5 launches per layer); "Triton MoE 核心擊敗 Megablocks" (setupai.cc),
 * key points (block-scheduled grouped GEMM over variable expert batch sizes)
 * and technical deep-dive (top-k routing inside the kernel); the DeepGEMM
 * article (itsolotime.com), section 1.1 (dispatch -> linear1 -> SwiGLU ->
 * linear2 -> combine) and section 3.1 (per-expert contiguous activations);
 * the HPC-Ops article (ntfzh.com), FusedMoE paragraph (re-arrangement, grouped
 * GEMM, weighted reduce).
 *
 * Conventions for every call:
 *   - Tensors are row-major and contiguous. bf16 values are passed as their
 *     16-bit patterns (moe_bf16). Weights: W_gate, W_up [E,H,F]; W_down [E,F,H].
 *   - Every pointer argument is a DEVICE pointer unless stated otherwise. The
 *     caller owns all memory; the library allocates no device memory.
 *   - `stream` is a hipStream_t (NULL = the default stream). Every call only
 *     enqueues work on it and returns without synchronising. Per-expert
 *     counts never travel to the host.
 *   - Arguments are validated on the host before anything is enqueued: on a
 *     validation error (every negative moe_status except MOE_ERR_HIP) nothing
 *     is enqueued and no output is touched. MOE_ERR_HIP reports a HIP runtime
 *     failure at a kernel launch; a call that makes several launches may then
 *     have enqueued the ones before it, so its outputs and workspace are
 *     unspecified.
 *   - Size limits: 0 <= T; 1 <= k <= min(E, 16); 1 <= E <= 1024;
 *     H, F (and Fs) multiples of 8; T*k*max(H, F, Fs) < 2^31. T = 0 is a
 *     successful no-op (then pointers are not inspected).
 *   - Alignment: bf16 tensors and workspaces 16 bytes; fp32 and int32
 *     arrays 4 bytes (MOE_ERR_MISALIGNED otherwise).
 *   - Calls are re-entrant; the only cached state is per-device properties
 *     (and the process-wide settings of moe_set_diagnostics and of the
 *     testing hook moe_set_dispatch_override).
 *   - Diagnostics (read from the environment at the library's first use,
 *     or set with moe_set_diagnostics): MOE_TRACE=1 writes one line per
 *     kernel launch to stderr (kernel, grid, block, LDS, tile shape and
 *     schedule of the grouped GEMMs); MOE_DEBUG=1 makes every call that
 *     takes expert ids from the caller (moe_permute, moe_forward_routed,
 *     moe_backward, moe_route_backward) check them on the GPU first and
 *     return MOE_ERR_BAD_IDS if one lies outside [0, E). The check waits for
 *     its result (the call synchronises its stream, so it cannot be captured
 *     into a graph); with MOE_DEBUG off, ids outside [0, E) are undefined
 *     behaviour.
 *   - Results are deterministic: the same inputs give bit-identical outputs.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t moe_bf16; /* bf16 bit pattern (torch.bfloat16 storage) */

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,         /* null pointer, negative or zero size */
  MOE_ERR_UNSUPPORTED_SHAPE = -2,   /* outside the size limits above */
  MOE_ERR_MISALIGNED = -3,          /* a pointer below its required alignment */
  MOE_ERR_WORKSPACE_TOO_SMALL = -4, /* ws_bytes below the required size */
  MOE_ERR_HIP = -5,                 /* a HIP runtime call or launch failed */
  MOE_ERR_BAD_IDS = -6              /* an expert id outside [0, E) (debug check):
                                       only the check itself was enqueued */
} moe_status;

/* Optional always-on shared expert, added to every token's output. The
 * struct itself is a HOST object; its pointers are device pointers.
 * w_gate, w_up [H,Fs]; w_down [Fs,H]; gate_logits [T] fp32 or NULL.
 * The shared term is s_t * y_sh[t] with s_t = 1 when gate_logits is NULL,
 * else the logistic sigmoid 1/(1+exp(-gate_logits[t])). */
typedef struct {
  const moe_bf16* w_gate;
  const moe_bf16* w_up;
  const moe_bf16* w_down;
  int32_t Fs;
  const float* gate_logits;
} moe_shared_expert;

/* Text for a status code (a static host string; never NULL). */
const char* moe_status_string(int status);

/* Step 1, route. logits fp32 [T,E] (finite values) -> topk_ids int32 [T,k]
 * (expert ids, largest logit first, equal logits in ascending expert order;
 * -0.0 and +0.0 are equal) and topk_w fp32 [T,k] (softmax over the k chosen
 * logits, fp32 arithmetic, max subtracted; sums to 1 up to rounding).
 * Routing inside the kernel, with no host synchronisation, follows the
 * Triton MoE page (setupai.cc), technical deep-dive. */
int moe_route(const float* logits, int T, int E, int k, int32_t* topk_ids,
              float* topk_w, void* stream);

/* Workspace needed by moe_router_route (device bytes) on the current device;
 * 0 when the call needs none or the sizes are invalid. */
size_t moe_router_workspace_bytes(int T, int H, int E, int k);

/* Step 1 with the router projection in front of it. x bf16 [T,H] and
 * w_router bf16 [E,H] (row e is expert e's router vector; both K-contiguous,
 * H % 8 == 0) give the logits
 *   logits[t,e] = sum_h x[t,h] * w_router[e,h]
 * (bf16 products, exact in fp32, accumulated in fp32 in an unspecified
 * order), and topk_ids / topk_w are exactly what moe_route returns on those
 * fp32 logits. logits_out fp32 [T,E] receives the logits when it is not
 * NULL (the routing does not need them in HBM). The routing inside the
 * kernel follows the Triton MoE page (setupai.cc), technical deep-dive; the
 * router projection is the step the pages' routing starts from (gating
 * scores per token and expert) and is not itself given on them.
 * ws: at least moe_router_workspace_bytes(T, H, E, k) device bytes, 16-byte
 * aligned (may be NULL when that is 0). Errors as moe_route, plus
 * MOE_ERR_WORKSPACE_TOO_SMALL. */
int moe_router_route(const moe_bf16* x, const moe_bf16* w_router, int T, int H, int E,
                     int k, float* logits_out, int32_t* topk_ids, float* topk_w,
                     void* ws, size_t ws_bytes, void* stream);

/* Workspace needed by moe_permute (device bytes); 0 for invalid sizes. */
size_t moe_permute_workspace_bytes(int T, int E, int k);

/* Step 2, permute. topk_ids int32 [T,k] (each in [0,E), e.g. from moe_route)
 * and x bf16 [T,H] ->
 *   expert_offsets int32 [E+1]: offsets[e] = first row of expert e,
 *                  offsets[E] = T*k (exclusive prefix of per-expert counts);
 *   row_token int32 [T*k]: row p of x_perm holds token row_token[p];
 *   row_dest  int32 [T*k]: (t,j) went to row row_dest[t*k+j];
 *   x_perm    bf16 [T*k,H]: x_perm[p] = x[row_token[p]] (a bit copy).
 * Within an expert's block rows are in ascending token order (a stable sort
 * of the assignments in t-major, j-minor order); the layout is unpadded.
 * ws: at least moe_permute_workspace_bytes(T,E,k) device bytes of scratch.
 * Ids outside [0,E) are not checked on the device; they give unspecified
 * (but in-bounds) results. Per-expert contiguous activations as in the
 * DeepGEMM article (itsolotime.com), section 3.1; re-arrangement before the
 * grouped GEMM as in the HPC-Ops article (ntfzh.com), FusedMoE paragraph. */
int moe_permute(const moe_bf16* x, const int32_t* topk_ids, int T, int H,
                int E, int k, int32_t* expert_offsets, int32_t* row_token,
                int32_t* row_dest, moe_bf16* x_perm, void* ws,
                size_t ws_bytes, void* stream);

/* Step 3, grouped gate/up GEMM with SwiGLU epilogue. For every expert e and
 * row p in [offsets[e], offsets[e+1]):
 *   h[p,f] = bf16( silu(G) * U ),  G = sum_c x_perm[p,c] W_gate[e,c,f],
 *   U = sum_c x_perm[p,c] W_up[e,c,f], fp32 accumulation,
 *   silu(z) = z/(1+exp(-z)) in fp32, rounded to bf16 to nearest-even.
 * x_perm bf16 [M,H]; expert_offsets int32 [E+1] on the device, non-decreasing
 * from 0 to M (rows outside [0,M) are never read or written whatever the
 * offsets hold); h bf16 [M,F] (caller-owned). G and U stay in registers.
 * Fused gate+up so the SwiGLU input never reaches global memory: the
 * dispatch-kernel post (lumeric.app), summary paragraph. */
int moe_gateup_swiglu(const moe_bf16* x_perm, const int32_t* expert_offsets,
                      int M, int H, int F, int E, const moe_bf16* w_gate,
                      const moe_bf16* w_up, moe_bf16* h, void* stream);

/* Step 4, grouped down GEMM. y_perm[p,c] = bf16( sum_f h[p,f] W_down[e,f,c] )
 * for rows p of expert e; fp32 accumulation. h bf16 [M,F], y_perm bf16 [M,H],
 * expert_offsets as in moe_gateup_swiglu. The down projection (linear2) is
 * its own grouped GEMM as in the DeepGEMM article (itsolotime.com),
 * section 1.1. */
int moe_down(const moe_bf16* h, const int32_t* expert_offsets, int M, int F,
             int H, int E, const moe_bf16* w_down, moe_bf16* y_perm,
             void* stream);

/* Workspace needed by moe_grouped_ffn (device bytes): h bf16 [M,F] rounded
 * up to 256 bytes; 0 for invalid sizes. */
size_t moe_grouped_ffn_workspace_bytes(int M, int F);

/* Steps 3+4: the gate/up+SwiGLU grouped GEMM (as moe_gateup_swiglu) into h,
 * then the down grouped GEMM (as moe_down) into y_perm [M,H]. h lives in the
 * workspace: ws (at least moe_grouped_ffn_workspace_bytes(M,F) device bytes,
 * 16-byte aligned) holds h bf16 [M,F] at its start when the call's work is
 * done. Block-scheduled grouped GEMM over variable expert batch sizes: the
 * Triton MoE page (setupai.cc), key points. */
int moe_grouped_ffn(const moe_bf16* x_perm, const int32_t* expert_offsets,
                    int M, int H, int F, int E, const moe_bf16* w_gate,
                    const moe_bf16* w_up, const moe_bf16* w_down, moe_bf16* y_perm,
                    void* ws, size_t ws_bytes, void* stream);

/* Step 5, combine. out[t,c] = bf16( sum_{j<k} topk_w[t,j] * y_perm[row_dest[t,j], c] ),
 * fp32 accumulation in ascending j. y_perm bf16 [T*k,H]; row_dest int32 [T,k]
 * with values in [0,T*k) (as from moe_permute); topk_w fp32 [T,k];
 * out bf16 [T,H]. The weighted reduce after the grouped GEMM: the HPC-Ops
 * article (ntfzh.com), FusedMoE paragraph. */
int moe_combine(const moe_bf16* y_perm, const int32_t* row_dest,
                const float* topk_w, int T, int H, int k, moe_bf16* out,
                void* stream);

/* Workspace needed by moe_forward (device bytes); Fs = 0 without a shared
 * expert; 0 for invalid sizes. moe_workspace_bytes is the same function. */
size_t moe_forward_workspace_bytes(int T, int H, int F, int E, int k, int Fs);
size_t moe_workspace_bytes(int T, int H, int F, int E, int k, int Fs);

/* The whole layer, steps 1-5, as five kernel launches on `stream` (the
 * launch count of the dispatch-kernel post (lumeric.app), summary paragraph):
 * route (+ per-chunk expert histogram), permute (scan + stable rank + row
 * gather), grouped gate/up+SwiGLU, grouped down, combine. The shared expert,
 * when given, is one more group of the two grouped GEMMs over all T tokens,
 * and its gated output is added in the combine after the routed sum.
 *   x bf16 [T,H]; logits fp32 [T,E]; out bf16 [T,H];
 *   shared: HOST pointer to a moe_shared_expert, or NULL;
 *   topk_ids_out int32 [T,k], topk_w_out fp32 [T,k]: optional device copies
 *   of the routing result (NULL: kept in the workspace);
 *   ws: at least moe_forward_workspace_bytes(...) device bytes of scratch.
 * Results match route -> permute -> grouped_ffn -> combine through the split
 * calls, plus the shared term, except that the down projection's output
 * reaches the combine in fp32 here (the split calls round y_perm to bf16). */
int moe_forward(const moe_bf16* x, const float* logits, int T, int H, int F,
                int E, int k, const moe_bf16* w_gate, const moe_bf16* w_up,
                const moe_bf16* w_down, const moe_shared_expert* shared,
                moe_bf16* out, int32_t* topk_ids_out, float* topk_w_out,
                void* ws, size_t ws_bytes, void* stream);

/* The layer from a routing the caller already has (steps 2-5): topk_ids
 * int32 [T,k] (ids in [0,E); ids outside are not checked on the device and
 * give unspecified but in-bounds results) and topk_w fp32 [T,k], e.g. from
 * moe_router_route, which computes them from x and the router weights with
 * no [T,E] logits in HBM. The routing and its weights as an input of the
 * expert layer follow the DeepGEMM article (itsolotime.com), section 1.3
 * (the Mega MoE buffer layout's input region holds the top-k ids and
 * weights next to x). weights_packed:
 * 0 = row-major weights as in moe_forward, 1 = packed as in
 * moe_forward_packed. Same workspace (moe_forward_workspace_bytes) and
 * output as moe_forward; given the same ids and weights, out equals
 * moe_forward's bit for bit. Four or five launches: expert histogram,
 * permute, gate/up, down, combine. */
int moe_forward_routed(const moe_bf16* x, const int32_t* topk_ids, const float* topk_w, int T,
                       int H, int F, int E, int k, const moe_bf16* w_gate, const moe_bf16* w_up,
                       const moe_bf16* w_down, const moe_shared_expert* shared,
                       int weights_packed, moe_bf16* out, void* ws, size_t ws_bytes,
                       void* stream);

/* ---- Packed weights ----
 * Expert weights do not change between calls, so they can be re-laid out
 * once, when they are loaded, into the order in which the grouped GEMM
 * streams them. With the row-major layout a decode-size tile reads every
 * K-step as 64 rows of 128 bytes spaced 2*N bytes apart; with the packed
 * layout it reads one contiguous run, which HBM delivers faster (the layer
 * at small batch is bound by streaming the weights). Results are identical
 * to the row-major calls (the same products are summed in the same order).
 * This re-layout is not on the pages; it is this library's addition.
 *
 * The packed form of W [G,K,N] (row-major; G groups: E experts, or 1 for a
 * shared expert) occupies moe_pack_weights_bytes(G,K,N) =
 * G * ceil(N/64) * ceil(K/64) * 8192 bytes: blocks of 64 K-rows by 64
 * columns, block (g, nb, kb) at byte ((g*ceil(N/64) + nb)*ceil(K/64) + kb)*8192,
 * each block two 32-row halves of 64 column rows of 64 bytes, a column row
 * holding that column's 32 K-values as four 8-value chunks in a swizzled
 * order, zero past K and past N (a lane's MFMA fragment, 8 K-consecutive
 * values of one column, is one 16-byte read). The order is private to this
 * library: produce packed tensors with moe_pack_weights. */

/* Packed size in bytes of a [G,K,N] weight tensor; 0 for invalid sizes
 * (G < 1, K or N not a positive multiple of 8). */
size_t moe_pack_weights_bytes(int G, int K, int N);

/* w bf16 [G,K,N] (row-major) -> packed (device, at least
 * moe_pack_weights_bytes(G,K,N) bytes, 16-byte aligned, not overlapping w).
 * One kernel on `stream`; w is only read. */
int moe_pack_weights(const moe_bf16* w, int G, int K, int N, moe_bf16* packed,
                     size_t packed_bytes, void* stream);

/* moe_gateup_swiglu with w_gate, w_up packed from [E,H,F]. */
int moe_gateup_swiglu_packed(const moe_bf16* x_perm,
                             const int32_t* expert_offsets, int M, int H,
                             int F, int E, const moe_bf16* w_gate_packed,
                             const moe_bf16* w_up_packed, moe_bf16* h,
                             void* stream);

/* moe_down with w_down packed from [E,F,H]. */
int moe_down_packed(const moe_bf16* h, const int32_t* expert_offsets, int M,
                    int F, int H, int E, const moe_bf16* w_down_packed,
                    moe_bf16* y_perm, void* stream);

/* moe_forward with packed weights: w_gate, w_up packed from [E,H,F],
 * w_down from [E,F,H]; when a shared expert is given, its w_gate and w_up
 * are packed from [1,H,Fs] and its w_down from [1,Fs,H]. Same workspace
 * (moe_forward_workspace_bytes) and outputs as moe_forward. */
int moe_forward_packed(const moe_bf16* x, const float* logits, int T, int H,
                       int F, int E, int k, const moe_bf16* w_gate_packed,
                       const moe_bf16* w_up_packed,
                       const moe_bf16* w_down_packed,
                       const moe_shared_expert* shared_packed, moe_bf16* out,
                       int32_t* topk_ids_out, float* topk_w_out, void* ws,
                       size_t ws_bytes, void* stream);

/* moe_forward_packed without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the call allocates nothing and uses a
 * fixed 128 MiB device array of the library as its workspace, which each GPU
 * holds from the library's load until the process ends. Limit: the layer's
 * workspace, moe_forward_workspace_bytes(T, H, F, E, k, Fs), must be at most
 * 128 MiB (134217728 bytes; e.g. the Mixtral-8x7B-shaped layer up to a few
 * hundred tokens), else the call returns MOE_ERR_WORKSPACE_TOO_SMALL with
 * nothing enqueued. All calls on one GPU share that GPU's array and leave
 * their intermediates in it: calls whose work may overlap on one GPU (on
 * different streams, or from several threads without ordering) race and
 * give unspecified results. Arguments, outputs and errors otherwise as
 * moe_forward_packed; given the same inputs the outputs are bit-identical. */
int moe_forward_packed_noalloc(const moe_bf16* x, const float* logits, int T, int H, int F,
                               int E, int k, const moe_bf16* w_gate_packed,
                               const moe_bf16* w_up_packed, const moe_bf16* w_down_packed,
                               const moe_shared_expert* shared_packed, moe_bf16* out,
                               int32_t* topk_ids_out, float* topk_w_out, void* stream);

/* ---- FP8 weights ----
 * The DeepGEMM article (itsolotime.com), sections 1.1 and 5.3, runs the
 * expert GEMMs on 8-bit (and 4-bit) floating-point operands. Here the
 * weights are 8-bit: each matrix W [G,K,N] is stored as OCP E4M3 codes
 * (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, subnormals, no
 * infinities, largest value 448) with one fp32 scale per (g, n), the
 * smallest power of two s with max_k |W[g,k,n]| <= 448 * s; a weight is
 * code_value * s. The activations stay bf16: every dequantized weight is a
 * bf16 value, so a layer on fp8 weights is exactly the bf16 layer on the
 * dequantized weights (same accumulation in fp32), at half the weight
 * bytes. Codes are rounded to nearest, ties to even. Supported scales are
 * normal fp32 values (columns whose largest |W| is at least 2^-117).
 *
 * Layout of the codes: G x ceil(N/64) x ceil(K/64) blocks of 4096 bytes,
 * block (g, nb, kb) at byte ((g*NB + nb)*KB + kb)*4096; within a block,
 * byte h*2048 + c*32 + p*8 + j holds the code of W[g, kb*64 + h*32 +
 * 8*(p ^ ((c >> 2) & 3)) + j, nb*64 + c] (zero past K or N). Scales:
 * fp32 [G,N]. Both 16-byte aligned; the shared expert's matrices are
 * quantized as G = 1. */

/* Bytes of the codes of a [G,K,N] weight tensor; 0 for invalid sizes. */
size_t moe_fp8_weights_bytes(int G, int K, int N);

/* Quantize bf16 W [G,K,N] (K, N multiples of 8) into codes (at least
 * moe_fp8_weights_bytes bytes) and scales fp32 [G,N]. Once, at load time. */
int moe_quantize_fp8(const moe_bf16* w, int G, int K, int N, uint8_t* codes,
                     size_t codes_bytes, float* scales, void* stream);

/* moe_gateup_swiglu / moe_down on fp8 weights: equal, bit for bit, to the
 * bf16 calls on the dequantized weights. */
int moe_gateup_swiglu_fp8(const moe_bf16* x_perm, const int32_t* expert_offsets, int M, int H,
                          int F, int E, const uint8_t* w_gate, const float* s_gate,
                          const uint8_t* w_up, const float* s_up, moe_bf16* h, void* stream);
int moe_down_fp8(const moe_bf16* h, const int32_t* expert_offsets, int M, int F, int H, int E,
                 const uint8_t* w_down, const float* s_down, moe_bf16* y_perm, void* stream);

/* Shared expert with fp8 weights (HOST struct, device pointers): w_gate,
 * w_up quantized from [1,H,Fs], w_down from [1,Fs,H], with their scales. */
typedef struct {
  const uint8_t* w_gate;
  const float* s_gate;
  const uint8_t* w_up;
  const float* s_up;
  const uint8_t* w_down;
  const float* s_down;
  int32_t Fs;
  const float* gate_logits;
} moe_shared_expert_fp8;

/* moe_forward on fp8 weights (same workspace and outputs). */
int moe_forward_fp8(const moe_bf16* x, const float* logits, int T, int H, int F, int E, int k,
                    const uint8_t* w_gate, const float* s_gate, const uint8_t* w_up,
                    const float* s_up, const uint8_t* w_down, const float* s_down,
                    const moe_shared_expert_fp8* shared, moe_bf16* out, int32_t* topk_ids_out,
                    float* topk_w_out, void* ws, size_t ws_bytes, void* stream);

/* ---- MXFP4 weights ----
 * The 4-bit weights of the same sections of the DeepGEMM article, read as
 * the OCP Microscaling format MXFP4: each matrix W [G,K,N] is stored as E2M1
 * codes (1 sign, 2 exponent bits with bias 1, 1 mantissa bit: magnitudes 0,
 * 0.5, 1, 1.5, 2, 3, 4, 6) and one E8M0 scale byte per 32 K-values of a
 * column, the scale 2^X with X = floor(log2(max |W| of the 32)) - 2 (raised
 * to -125, so dequantized weights stay normal bf16 values; 0 for an all-zero
 * block). A weight is code_value * 2^X, codes rounded to nearest with ties
 * to even and saturating at 6. The activations stay bf16: every dequantized
 * weight is a bf16 value, so a layer on mxfp4 weights is exactly the bf16
 * layer on the dequantized weights, at 4.25 bits per weight.
 *
 * Layout of the codes: G x ceil(N/64) x ceil(K/64) blocks of 2048 bytes,
 * block (g, nb, kb) at byte ((g*NB + nb)*KB + kb)*2048; within a block, byte
 * h*1024 + c*16 + q*4 + i/2 holds, in its low nibble for even i and its high
 * nibble for odd i, the code of W[g, kb*64 + h*32 + 8q + i, nb*64 + c] (zero
 * past K or N). Scale bytes: [G][ceil(N/64)][4*ceil(K/128)][64], byte
 * ((g*NB + nb)*SKB + b)*64 + c for column nb*64 + c and K-values 32b ..
 * 32b+31 (127 past K or N). Both 16-byte aligned; the shared expert's
 * matrices are quantized as G = 1. */

/* Bytes of the codes and of the scale bytes of a [G,K,N] weight tensor; 0
 * for invalid sizes. */
size_t moe_mxfp4_weights_bytes(int G, int K, int N);
size_t moe_mxfp4_scales_bytes(int G, int K, int N);

/* Quantize bf16 W [G,K,N] (K, N multiples of 8) into codes and scale bytes.
 * Once, at load time. Errors as moe_quantize_fp8. */
int moe_quantize_mxfp4(const moe_bf16* w, int G, int K, int N, uint8_t* codes,
                       size_t codes_bytes, uint8_t* scales, size_t scales_bytes, void* stream);

/* moe_gateup_swiglu / moe_down on mxfp4 weights: equal, bit for bit, to the
 * bf16 calls on the dequantized weights. */
int moe_gateup_swiglu_mxfp4(const moe_bf16* x_perm, const int32_t* expert_offsets, int M, int H,
                            int F, int E, const uint8_t* w_gate, const uint8_t* s_gate,
                            const uint8_t* w_up, const uint8_t* s_up, moe_bf16* h,
                            void* stream);
int moe_down_mxfp4(const moe_bf16* h, const int32_t* expert_offsets, int M, int F, int H, int E,
                   const uint8_t* w_down, const uint8_t* s_down, moe_bf16* y_perm, void* stream);

/* Shared expert with mxfp4 weights (HOST struct, device pointers). */
typedef struct {
  const uint8_t* w_gate;
  const uint8_t* s_gate;
  const uint8_t* w_up;
  const uint8_t* s_up;
  const uint8_t* w_down;
  const uint8_t* s_down;
  int32_t Fs;
  const float* gate_logits;
} moe_shared_expert_mxfp4;

/* moe_forward on mxfp4 weights (same workspace and outputs). */
int moe_forward_mxfp4(const moe_bf16* x, const float* logits, int T, int H, int F, int E, int k,
                      const uint8_t* w_gate, const uint8_t* s_gate, const uint8_t* w_up,
                      const uint8_t* s_up, const uint8_t* w_down, const uint8_t* s_down,
                      const moe_shared_expert_mxfp4* shared, moe_bf16* out,
                      int32_t* topk_ids_out, float* topk_w_out, void* ws, size_t ws_bytes,
                      void* stream);

/* ---- MXFP8 weights ----
 * The FP8 expert GEMMs of the same sections of the DeepGEMM article with
 * block scales, read as the OCP Microscaling format MXFP8 with E4M3
 * elements, for the weights only: each matrix W [G,K,N] is stored as E4M3
 * codes (as for moe_quantize_fp8) and one E8M0 scale byte per 32 K-values
 * of a column, the scale 2^X with X = floor(log2(max |W| of the 32)) - 8
 * (the OCP rule: the largest magnitude lands in [256, 512); raised to -117,
 * so dequantized weights stay normal bf16 values; 0 for an all-zero block).
 * A weight is code_value * 2^X, codes rounded to nearest with ties to even
 * and saturating at 448. The activations stay bf16: every dequantized weight
 * is a bf16 value, so a layer on mxfp8 weights is exactly the bf16 layer on
 * the dequantized weights, at 8.25 bits per weight.
 *
 * Layout of the codes: the fp8 block layout above (G x ceil(N/64) x
 * ceil(K/64) blocks of 4096 bytes). Scale bytes: the mxfp4 layout above
 * ([G][ceil(N/64)][4*ceil(K/128)][64], 127 past K or N). Both 16-byte
 * aligned; the shared expert's matrices are quantized as G = 1. */

/* Bytes of the codes and of the scale bytes of a [G,K,N] weight tensor; 0
 * for invalid sizes. */
size_t moe_mxfp8_weights_bytes(int G, int K, int N);
size_t moe_mxfp8_scales_bytes(int G, int K, int N);

/* Quantize bf16 W [G,K,N] (K, N multiples of 8) into codes and scale bytes.
 * Once, at load time. Errors as moe_quantize_fp8. */
int moe_quantize_mxfp8(const moe_bf16* w, int G, int K, int N, uint8_t* codes,
                       size_t codes_bytes, uint8_t* scales, size_t scales_bytes, void* stream);

/* moe_gateup_swiglu / moe_down on mxfp8 weights: equal, bit for bit, to the
 * bf16 calls on the dequantized weights. */
int moe_gateup_swiglu_mxfp8(const moe_bf16* x_perm, const int32_t* expert_offsets, int M, int H,
                            int F, int E, const uint8_t* w_gate, const uint8_t* s_gate,
                            const uint8_t* w_up, const uint8_t* s_up, moe_bf16* h,
                            void* stream);
int moe_down_mxfp8(const moe_bf16* h, const int32_t* expert_offsets, int M, int F, int H, int E,
                   const uint8_t* w_down, const uint8_t* s_down, moe_bf16* y_perm, void* stream);

/* Shared expert with mxfp8 weights (HOST struct, device pointers). */
typedef struct {
  const uint8_t* w_gate;
  const uint8_t* s_gate;
  const uint8_t* w_up;
  const uint8_t* s_up;
  const uint8_t* w_down;
  const uint8_t* s_down;
  int32_t Fs;
  const float* gate_logits;
} moe_shared_expert_mxfp8;

/* moe_forward on mxfp8 weights (same workspace and outputs). */
int moe_forward_mxfp8(const moe_bf16* x, const float* logits, int T, int H, int F, int E, int k,
                      const uint8_t* w_gate, const uint8_t* s_gate, const uint8_t* w_up,
                      const uint8_t* s_up, const uint8_t* w_down, const uint8_t* s_down,
                      const moe_shared_expert_mxfp8* shared, moe_bf16* out,
                      int32_t* topk_ids_out, float* topk_w_out, void* ws, size_t ws_bytes,
                      void* stream);

/* ---- Training backward ----
 * The news page "Triton-Optimierter BF16 Grouped GEMM Kernel beschleunigt
 * MoE-Modelle" (meineki.news), introduction, presents its grouped GEMM for
 * training as well as inference; no page gives the backward, so these calls
 * are the chain rule through steps 2-5 and through the softmax of step 1.
 * With G = x_perm W_gate, U = x_perm W_up, h = silu(G) U, y = h W_down per
 * expert row, w the row's routing weight and the gradient dout of the
 * layer's output out:
 *   g        = dout[token] W_down^T             (fp32, from the bf16 dout)
 *   dh       = w * g                            (fp32)
 *   d_topk_w = <dout[t], y[row of (t,j)]> = <h, g>   (fp32)
 *   dG       = dh * U * silu'(G),  dU = dh * silu(G),
 *              silu'(z) = s(z) (1 + z (1 - s(z))), s the logistic function
 *   dx[t]    = sum_j (dG W_gate^T + dU W_up^T)[row of (t,j)]
 *   dW_gate[e] = x_perm_e^T dG_e, dW_up[e] = x_perm_e^T dU_e,
 *   dW_down[e] = h_e^T dy_e,  dy = bf16(w * dout[token]) per row
 *                             (sums over the expert's rows; 0 for an expert
 *                              with no rows).
 * The gate/up half of the forward is recomputed inside (nothing is kept
 * from moe_forward); the product with W_down^T is taken on the unweighted
 * dout, so d_topk_w = <h, g> needs no recomputed y and no rounding of dy
 * reaches dh. h, G, U, dy (for dW_down only), dG and dU are rounded to bf16
 * between the steps; every product accumulates in fp32. moe_backward
 * covers the routed experts; moe_backward_shared adds the shared expert
 * (below). Weights in the row-major layout of moe_forward. */

/* Bytes of the workspace moe_backward needs (0 for invalid sizes):
 * about T*k*(14 H + 10.25 F) bytes. */
size_t moe_backward_workspace_bytes(int T, int H, int F, int E, int k);

/* Gradients of the routed layer for a given routing (topk_ids, topk_w
 * [T,k], as moe_forward returns them: ids in [0,E), distinct within a
 * token) and output gradient dout [T,H] bf16.
 * Outputs: dx [T,H] bf16; d_topk_w [T,k] fp32; dw_gate, dw_up [E,H,F] and
 * dw_down [E,F,H] fp32 (every element written; all zero when T = 0, which
 * is then the only work and needs only the three weight-gradient pointers).
 * Extra limit: H*F < 2^31. Deterministic. */
int moe_backward(const moe_bf16* x, const int32_t* topk_ids, const float* topk_w, int T, int H,
                 int F, int E, int k, const moe_bf16* w_gate, const moe_bf16* w_up,
                 const moe_bf16* w_down, const moe_bf16* dout, moe_bf16* dx, float* d_topk_w,
                 float* dw_gate, float* dw_up, float* dw_down, void* ws, size_t ws_bytes,
                 void* stream);

/* Gradient of the router logits through the softmax over each token's k
 * selected logits (step 1): d_logits [T,E] fp32, with
 * d_logits[t, id_j] = w_j (d_w_j - sum_i w_i d_w_i) and 0 for the experts
 * not selected (the selection itself has no gradient). */
int moe_route_backward(const int32_t* topk_ids, const float* topk_w, const float* d_topk_w,
                       int T, int E, int k, float* d_logits, void* stream);

/* The shared expert's gradients (a HOST struct of DEVICE pointers): dw_gate,
 * dw_up [H,Fs] and dw_down [Fs,H] fp32 (every element written; zero when
 * T = 0), and d_gate_logits [T] fp32, the gradient of the gate logits
 * (written only when the expert has gate logits; may be NULL otherwise). */
typedef struct {
  float* dw_gate;
  float* dw_up;
  float* dw_down;
  float* d_gate_logits;
} moe_shared_expert_grads;

/* Bytes of the workspace moe_backward_shared needs (0 for invalid sizes):
 * moe_backward's plus about T*(10 H + 10.25 Fs) bytes for the shared
 * expert. Fs = 0 gives moe_backward's. */
size_t moe_backward_shared_workspace_bytes(int T, int H, int F, int E, int k, int Fs);

/* moe_backward with the shared expert of moe_forward (its term
 * s_t * y_sh[t] of the output, s_t = 1 without gate logits, else the
 * logistic sigmoid of the token's gate logit). Not on the pages (the
 * DeepSeek-V3 and Qwen2-MoE layer shapes of the workload definitions carry
 * the shared expert); the chain rule through that term, as the routed
 * rows': the shared expert is one more group over all T tokens with s_t for
 * its routing weight, so
 *   dx[t]        += dG_sh W_sg^T + dU_sh W_su^T   (dx is the layer's whole
 *                                                 input gradient)
 *   d_gate_logits[t] = <dout[t], y_sh[t]> s_t (1 - s_t)
 *   dW_sg = x^T dG_sh, dW_su = x^T dU_sh, dW_sd = h_sh^T bf16(s dout)
 * with the same roundings as the routed rows. shared == NULL: exactly
 * moe_backward (shared_grads is not read). Otherwise shared_grads is
 * required and its pointers are validated like the routed gradients'.
 * Deterministic. */
int moe_backward_shared(const moe_bf16* x, const int32_t* topk_ids, const float* topk_w, int T,
                        int H, int F, int E, int k, const moe_bf16* w_gate, const moe_bf16* w_up,
                        const moe_bf16* w_down, const moe_shared_expert* shared,
                        const moe_bf16* dout, moe_bf16* dx, float* d_topk_w, float* dw_gate,
                        float* dw_up, float* dw_down, moe_shared_expert_grads* shared_grads,
                        void* ws, size_t ws_bytes, void* stream);

/* ---- Diagnostics ----
 * Not part of the layer's arithmetic; for debugging and tuning: a launch log
 * and an id check on demand.
 *
 * moe_set_diagnostics: trace = 1 logs every later kernel launch to stderr
 * (MOE_TRACE), check_ids = 1 turns on the id check of the calls that take
 * caller ids (MOE_DEBUG); 0 turns either off and -1 restores the
 * environment's setting. Process-wide. MOE_OK, or MOE_ERR_INVALID_ARG for
 * values outside -1..1. */
int moe_set_diagnostics(int trace, int check_ids);

/* Counts the entries of topk_ids [T,k] (device, int32) outside [0, E) on
 * `stream`, waits for the count (synchronising the stream) and returns
 * MOE_OK when there are none, MOE_ERR_BAD_IDS otherwise. Needs no
 * workspace (a device integer of the library holds the count). Size
 * limits as for moe_permute; T = 0 is MOE_OK. The check MOE_DEBUG runs. */
int moe_check_topk_ids(const int32_t* topk_ids, int T, int k, int E, void* stream);

/* ---- Testing hook ----
 * Not part of the layer's contract: for tests and benchmarks that compare
 * the library's own kernel variants. Forces, for every later call in this
 * process, the gate/up path of decode-size groups (decode_path: 0 the
 * LDS-ring tile, 1 the register-streaming kernel where it applies) and the
 * grouped GEMMs' tile class (tile_class: 0 small, 1 mid, 2 128-row, 3
 * 256-row); -1 restores the automatic choice. Process-wide and not
 * synchronised with calls in other threads. Returns MOE_OK, or
 * MOE_ERR_INVALID_ARG for values outside those ranges. */
int moe_set_dispatch_override(int decode_path, int tile_class);

/* Testing hook, like moe_set_dispatch_override: where the fused layer
 * combines. mode 1: in the down projection's epilogue whenever its tiles are
 * the decode-size ones (the scatter-add half of gather/scatter fusion: each
 * workgroup counts its rows into per-(token, column tile) integer counters
 * after storing its partial sums at device scope, and the one that completes
 * a tile adds the token's rows in the combine's order, so the result is
 * deterministic and bit-identical to the separate combine); 0 or -1
 * (automatic): in a combine launch of its own after the down projection,
 * which measured as fast or faster on MI355X. Returns MOE_OK, or
 * MOE_ERR_INVALID_ARG outside -1..1. */
int moe_set_combine_override(int mode);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
