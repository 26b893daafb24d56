// Internal launch interface of the MoE kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;

constexpr int kMaxExperts = 1024;     // E limit of the ABI
constexpr int kMaxTopK = 16;          // k limit of the ABI
constexpr int kMaxChunkAssign = 256;  // assignments per routing/permute chunk
constexpr int kPermuteSliceCols = 256;   // x columns copied per permute block
constexpr int kPermChunks = 8;           // routing chunks per permute block
constexpr int kMaxKSplit = 8;         // K-slices of a split down projection

// --- diagnostics (diagnostics.hip) ---
// Launch trace (MOE_TRACE) and the debug check of caller-given ids
// (MOE_DEBUG); both read from the environment at first use, or set by
// moe_set_diagnostics (-1: back to the environment's setting).
bool trace_enabled();
bool check_ids_enabled();
void set_diagnostics(int trace, int check_ids);
void trace_launch(const char* kernel, dim3 grid, dim3 block, size_t lds, const char* fmt, ...)
    __attribute__((format(printf, 5, 6)));
// Counts the ids of ids[0, n) outside [0, E) on `stream` and waits for the
// count (so never inside a captured graph).
hipError_t count_bad_ids(const int32_t* ids, int64_t n, int E, hipStream_t stream, int* bad);
#define MOE_TRACE_LAUNCH(...)                                    \
  do {                                                           \
    if (::moe::trace_enabled()) ::moe::trace_launch(__VA_ARGS__); \
  } while (0)

// --- routing and permutation (route_permute.hip) ---
int route_chunk_tokens(int T, int k);
int route_num_chunks(int T, int k);
hipError_t launch_route(const float* logits, int T, int E, int k,
                        int32_t* topk_ids, float* topk_w,
                        int32_t* hist /* nullable */, hipStream_t stream);
hipError_t launch_hist(const int32_t* topk_ids, int T, int E, int k,
                       int32_t* hist, hipStream_t stream);
// Route + permute (with the row copy) in one launch, for T*k <= 128 and
// E <= 256 (where it is faster than route + permute).
bool route_permute_fits_one_launch(int T, int E, int k);
// Both permutation launches also zero clear[0, nclear) (the arrival counters
// of a down projection that combines in its epilogue; nullptr: nothing).
hipError_t launch_route_permute_small(const float* logits, const bf16_t* x, int T, int H,
                                      int E, int k, int32_t* topk_ids, float* topk_w,
                                      int32_t* expert_offsets, int32_t* row_token,
                                      int32_t* row_dest, bf16_t* x_perm, hipStream_t stream,
                                      int32_t* clear = nullptr, int64_t nclear = 0);
// x_perm == nullptr: row maps and offsets only (no row copy).
hipError_t launch_permute(const bf16_t* x, const int32_t* topk_ids, int T,
                          int H, int E, int k, const int32_t* hist,
                          int32_t* expert_offsets, int32_t* row_token,
                          int32_t* row_dest, bf16_t* x_perm,
                          hipStream_t stream, int32_t* clear = nullptr, int64_t nclear = 0);

// --- grouped GEMM (grouped_gemm.hip) ---
// A segment is a list of groups that share K, N and the weight layout.
// Group g owns activation rows [offsets[g], offsets[g+1]) of `act`
// (offsets == nullptr: one group, rows [0, rows)); its weights are
// w0 + g*w_stride ([K][N], N contiguous, or the packed block layout of
// pack_weights), and w1 likewise when gated.
struct GemmSegment {
  const bf16_t* act;       // [rows, K]
  const int32_t* offsets;  // device [ngroups+1] or nullptr
  const bf16_t* w0;
  const bf16_t* w1;        // gated only
  void* out;               // [rows, N], bf16 or fp32 (GemmProblem::out_f32)
  int64_t w_stride;        // elements between consecutive groups' weights
  int64_t slice_stride;    // elements between K-slice outputs (ksplit > 1)
  int rows;
  int ngroups;
  int K;
  int N;
  int packed = 0;          // weight layout: 0 [K][N] bf16, 1 packed bf16, 2 packed fp8,
                           // 3 packed mxfp4, 5 packed mxfp8
  // fp8 (packed == 2): E4M3 codes in 4 KB blocks (fp8_weight_bytes), each
  // group's output columns scaled by scale0/scale1 + g*N (fp32 powers of two).
  // mxfp4 (packed == 3): E2M1 codes in 2 KB blocks (mxfp4_weight_bytes) and
  // E8M0 scale bytes per 32 K-values of a column (mxfp4_scale_bytes).
  // mxfp8 (packed == 5): E4M3 codes in the fp8 4 KB blocks and the mxfp4
  // scale-byte layout.
  const void* scale0 = nullptr;
  const void* scale1 = nullptr;
  // Optional row map: activation row of row p is gather[p] (`act` is then
  // the un-permuted [gather_rows, K] tensor; map entries are clamped to its
  // rows, so a corrupted map cannot make a load leave it). Only for the tile
  // classes without item chaining (see grouped_gemm_gathers).
  const int32_t* gather = nullptr;
  int gather_rows = 0;
  int ksplit = 1;          // K-slices (> 1 needs fp32 output; the consumer sums them)
  // Epilogues of the training backward (GemmProblem::epi): kStoreGUH also
  // writes G to out2 and U to out3. kSwigluBwd takes the product as
  // g = dout W_down^T (unweighted), reads G, U, h from aux0..aux2 ([rows, N]
  // bf16, like out) and each row's routing weight from wrow, writes
  // dG = w g U silu'(G) to out and dU = w g silu(G) to out2, and for each
  // 16-column fragment the partial sum of h g to part [rows][ceil(N/16)].
  void* out2 = nullptr;
  void* out3 = nullptr;
  const bf16_t* aux0 = nullptr;
  const bf16_t* aux1 = nullptr;
  const bf16_t* aux2 = nullptr;
  const float* wrow = nullptr;
  float* part = nullptr;
};

// Weight layout 4 (GemmSegment::packed): row-major [N][K] per group (K
// contiguous), i.e. the transpose of a [K][N] weight as it is stored; plain
// (not gated) bf16 problems only.
constexpr int kWeightsTransposed = 4;
enum GemmEpilogue { kEpiDefault = 0, kStoreGUH = 1, kSwigluBwd = 2 };

// The combine folded into a decode-size down projection of the fused layer
// (GemmProblem::scat, on when cnt != nullptr; see grouped_gemm_scatters).
// The routed segment's rows are the permuted assignments, the shared
// segment's (if any) the tokens. After storing its fp32 partial sums, a
// workgroup publishes them at device scope and counts each of its rows into
// cnt[token * ceil(N / BF) + column tile] (one vector-memory integer atomic
// per row); the workgroup whose count completes the token's column tile
// (target = k * routed K-slices + shared K-slices) reads every partial sum
// of it and writes out[token] over the tile's columns, with the combine's
// arithmetic in the combine's order: for j < k the slices of row
// row_dest[t*k + j] added in slice order, times topk_w[t*k + j] (1 when
// null), accumulated in ascending j; then the shared rows' slices times the
// sigmoid of gate_logits[t] (1 when null). Nothing waits on another
// workgroup, and the result does not depend on which one completes a tile.
struct ScatterArgs {
  int32_t* cnt = nullptr;  // [T * ceil(N / 64)], zero before the launch
  int target = 0;
  int T = 0, k = 0;
  const int32_t* row_token = nullptr;
  const int32_t* row_dest = nullptr;
  const float* topk_w = nullptr;
  const float* y = nullptr;       // the routed segment's output (slice 0)
  int64_t y_slice_stride = 0;
  int y_slices = 1;
  const float* y_sh = nullptr;    // the shared segment's output, or null
  int64_t ysh_slice_stride = 0;
  int ysh_slices = 1;
  const float* gate_logits = nullptr;
  bf16_t* out = nullptr;          // [T, N]
};

struct GemmProblem {
  GemmSegment seg[2];
  int nseg;
  bool gated;      // out = silu(act w0) * (act w1), else act w0
  bool out_f32;    // store fp32 instead of bf16 (down projection only)
  int rows_hint;   // typical rows per group, picks the tile shape
  int epi = kEpiDefault;  // GemmEpilogue (kStoreGUH: gated; kSwigluBwd: plain, bf16 out)
  ScatterArgs scat;
};

hipError_t launch_grouped_gemm(const GemmProblem& prob, hipStream_t stream);
// Whether the gated problem's tiles can read activations through a row map
// (GemmSegment::gather): true for the large-batch tile classes, whose items
// restart their pipeline anyway (the map is read at each item's start).
bool grouped_gemm_gathers(const GemmProblem& prob);
// Whether the plain fp32-output problem combines in its epilogue
// (GemmProblem::scat): only the decode-size class can, and only when the
// testing hook asks for it (set_scatter_override(1); the reason is at the
// definition).
bool grouped_gemm_scatters(const GemmProblem& prob);

// Sets each segment's K-slices (seg[s].ksplit) for an fp32-output problem on
// a device with `cus` compute units; gated or bf16 problems keep 1.
void grouped_gemm_plan_ksplit(GemmProblem& prob, int cus);
int grouped_gemm_device_cus();
// Testing hook: force the decode-size gate/up path (0 LDS-ring tile, 1
// register-streaming kernel) and the tile class (0 small, 1 mid, 2 large128,
// 3 large) of later launches; -1 restores the automatic choice.
void set_dispatch_override(int decode_path, int tile_class);
// Testing hook: 1 combines in the down projection's epilogue where its
// tiles can; 0 or -1 (automatic) never (a combine launch of its own).
void set_scatter_override(int mode);

// Packed weights: W [G][K][N] as G x ceil(N/64) x ceil(K/64) blocks of
// 64 x 64 (block (g, nb, kb) at element ((g*NB + nb)*KB + kb)*4096), each
// in the GEMM's LDS order (128-byte rows, swizzled 16-byte chunks), zero
// past K and N. A K-step of a decode-size tile is then one contiguous read.
int64_t packed_weight_elems(int G, int K, int N);

// FP8 weights: W [G][K][N] as E4M3 codes with one power-of-two scale per
// (g, n) (the smallest with max_k |W| <= 448 * scale), codes in
// G x ceil(N/64) x ceil(K/64) blocks of 4 KB: [32-row half][64 columns][32
// bytes], the 8-byte chunk of rows 8q..8q+7 of column c at chunk position
// q ^ ((c >> 2) & 3); zero past K and N.
int64_t fp8_weight_bytes(int G, int K, int N);
hipError_t launch_quantize_fp8(const bf16_t* w, int G, int K, int N, uint8_t* codes,
                               float* scales, hipStream_t stream);

// MXFP4 weights (OCP microscaling): W [G][K][N] as E2M1 codes in
// G x ceil(N/64) x ceil(K/64) blocks of 2 KB: [32-row half][64 columns][16
// bytes], byte h*1024 + c*16 + q*4 + i/2 holding rows kb*64 + h*32 + 8q + i
// of column nb*64 + c (low nibble: even i), zero past K and N; and one E8M0
// scale byte per 32 K-values of a column, [G][ceil(N/64)][4*ceil(K/128)][64]
// (127 = 1.0 past K and N).
int64_t mxfp4_weight_bytes(int G, int K, int N);
int64_t mxfp4_scale_bytes(int G, int K, int N);
hipError_t launch_quantize_mxfp4(const bf16_t* w, int G, int K, int N, uint8_t* codes,
                                 uint8_t* scales, hipStream_t stream);

// MXFP8 weights (OCP microscaling, E4M3 elements): W [G][K][N] as E4M3 codes
// in the fp8 block layout (fp8_weight_bytes) and one E8M0 scale byte per 32
// K-values of a column in the mxfp4 scale layout (mxfp4_scale_bytes): scale
// 2^X with X = floor(log2 max|w| of the 32) - 8, at least -117 (0 for an
// all-zero block); codes round to nearest, ties to even, saturating at 448.
hipError_t launch_quantize_mxfp8(const bf16_t* w, int G, int K, int N, uint8_t* codes,
                                 uint8_t* scales, hipStream_t stream);
hipError_t launch_pack_weights(const bf16_t* w, int G, int K, int N, bf16_t* packed,
                               hipStream_t stream);

// --- router GEMM + routing (router.hip) ---
// logits[t,e] = sum_h x[t,h] * w[e,h] (x [T,H], w [E,H], bf16, H % 8 == 0)
// and the top-k routing on them. A plan fixes the block tile (16*nt tokens x
// 16*nb experts) and the K-slices; a fused plan ranks inside the GEMM kernel
// (one launch, no workspace), otherwise the fp32 slice tiles go to `part`
// (router_part_elems floats) and a second launch adds and ranks them.
// logits_out may be null.
struct RouterPlan {
  int nb, nt;        // 16-wide expert and token tiles per block
  int kslice;        // K values per slice (a multiple of 64)
  int nslices;
  bool fused;
};
RouterPlan router_plan(int T, int H, int E, int cus);
size_t router_part_elems(const RouterPlan& p, int T, int E);
hipError_t launch_router(const RouterPlan& p, const bf16_t* x, const bf16_t* w, int T, int H,
                         int E, int k, float* logits_out, float* part, int32_t* topk_ids,
                         float* topk_w, hipStream_t stream);

// --- training backward (backward.hip) ---
// Per assignment row p = row_dest[t,j]: dy[p] = bf16(topk_w[t,j] * dout[t]),
// dout_perm[p] = dout[t], wrow[p] = topk_w[t,j].
hipError_t launch_backward_prep(const bf16_t* dout, const int32_t* row_dest,
                                const float* topk_w, int T, int H, int k, bf16_t* dy,
                                bf16_t* dout_perm, float* wrow, hipStream_t stream);
// d_topk_w[t,j] = sum over q of part[p][q], p = row_dest[t,j], in a fixed order
// (part [A][nq]: the fragments' partial sums of h g).
// The shared expert's term s_t y_sh[t] (s_t = 1, or the sigmoid of the
// gate logit): wrow[t] = s_t, dy[t] = bf16(s_t dout[t]) (for its W_down
// gradient) and offsets = {0, T} (its single group).
hipError_t launch_shared_prep(const bf16_t* dout, const float* gate_logits, int T, int H,
                              bf16_t* dy, float* wrow, int32_t* offsets, hipStream_t stream);
// d_gate[t] = (sum of part[t][0..nq) in order) s_t (1 - s_t): the
// gate-logit gradient from the shared dh product's per-fragment <h, g> sums.
hipError_t launch_shared_gate_grad(const float* part, int nq, const float* gate_logits, int T,
                                   float* d_gate, hipStream_t stream);
hipError_t launch_topk_w_grad(const float* part, int nq, const int32_t* row_dest, int T, int k,
                              float* d_topk_w, hipStream_t stream);
// d_logits [T,E] of the softmax over the k selected logits.
hipError_t launch_route_backward(const int32_t* topk_ids, const float* topk_w,
                                 const float* d_topk_w, int T, int E, int k, float* d_logits,
                                 hipStream_t stream);
// out[e] = sum over rows p in [offsets[e], offsets[e+1]) of a[p]^T b[p]:
// a [rows, M], b [rows, N] bf16, out fp32 [E][M][N] (zero for empty groups;
// offsets == nullptr: every group is empty).
hipError_t launch_kgrouped_gemm(const bf16_t* a, const bf16_t* b, const int32_t* offsets,
                                int E, int M, int N, float* out, hipStream_t stream);

// --- combine (combine.hip) ---
// y_perm/y_shared hold bf16 values (y_f32 == false) or fp32 values; with
// nslices > 1 (fp32 only) they are K-slice partial sums, slice s at
// y + s*stride, added in slice order (nslices_sh likewise for y_shared).
// topk_w == nullptr: every weight is 1.
hipError_t launch_combine(const void* y_perm, bool y_f32, int nslices,
                          int64_t y_slice_stride, const int32_t* row_dest,
                          const float* topk_w, int T, int H, int k,
                          const void* y_shared /* [T,H] or null */, int nslices_sh,
                          int64_t ysh_slice_stride,
                          const float* shared_gate /* [T] or null */,
                          bf16_t* out, hipStream_t stream);

}  // namespace moe
