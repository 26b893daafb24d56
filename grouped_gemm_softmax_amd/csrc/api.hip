// C ABI of the MoE expert layer: argument validation, workspace carving and
// kernel launches. Every argument is checked on the host before anything is
// enqueued; on an error nothing is launched and no output is touched.
#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "../../include/moe.h"
#include "kernels.h"

namespace {

using moe::bf16_t;

constexpr int64_t kIndexLimit = int64_t(1) << 31;

bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int check_dims(int T, int E, int k) {
  if (T < 0 || E < 1 || k < 1) return MOE_ERR_INVALID_ARG;
  if (E > moe::kMaxExperts || k > moe::kMaxTopK || k > E) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (static_cast<int64_t>(T) * k >= kIndexLimit) return MOE_ERR_UNSUPPORTED_SHAPE;
  return MOE_OK;
}

int check_width(int n) {
  if (n < 1) return MOE_ERR_INVALID_ARG;
  if (n % 8 != 0) return MOE_ERR_UNSUPPORTED_SHAPE;
  return MOE_OK;
}

int check_elems(int64_t rows, int64_t cols) {
  return rows * cols >= kIndexLimit ? MOE_ERR_UNSUPPORTED_SHAPE : MOE_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// The debug check of caller-given expert ids (on with MOE_DEBUG=1 or
// moe_set_diagnostics): counts the ids outside [0, E) and waits for the
// count. Off, it costs nothing and enqueues nothing.
int debug_check_ids(const int32_t* ids, int64_t n, int E, void* stream) {
  if (!moe::check_ids_enabled()) return MOE_OK;
  int bad = 0;
  if (moe::count_bad_ids(ids, n, E, static_cast<hipStream_t>(stream), &bad) != hipSuccess)
    return MOE_ERR_HIP;
  return bad ? MOE_ERR_BAD_IDS : MOE_OK;
}

#define MOE_TRY(expr)            \
  do {                           \
    const int rc_ = (expr);      \
    if (rc_ != MOE_OK) return rc_; \
  } while (0)

// bf16 tensors are read and written in 16-byte vectors; fp32/int32 arrays
// element-wise.
int need_bf16(const void* p) {
  if (!p) return MOE_ERR_INVALID_ARG;
  return aligned(p, 16) ? MOE_OK : MOE_ERR_MISALIGNED;
}
int need_word(const void* p) {
  if (!p) return MOE_ERR_INVALID_ARG;
  return aligned(p, 4) ? MOE_OK : MOE_ERR_MISALIGNED;
}

size_t permute_ws_bytes(int T, int E, int k) {
  return align_up(static_cast<size_t>(moe::route_num_chunks(T, k)) * E * sizeof(int32_t), 256);
}

// Workspace layout of moe_forward (each piece 256-byte aligned from ws):
// [hist | topk_ids | topk_w | offsets | row_token | row_dest | x_perm | h |
//  h_shared | y_perm | y_shared]. y_perm and y_shared are fp32 here: the down
// projection's output goes to the combine without a bf16 rounding, whose
// error (half an ulp of |y|, up to ~0.03 at |y| ~ 10) would otherwise reach
// outputs where the k expert terms cancel.
struct ForwardLayout {
  size_t hist, ids, w, offsets, row_token, row_dest, x_perm, h, h_sh, y, y_sh, cnt, total;
  int ksplit;     // K-slices of the routed down projection (y holds that many)
  int ksplit_sh;  // K-slices of the shared expert's (y_shared holds that many)
};

moe::GemmProblem down_problem(const bf16_t* h, const int32_t* offsets, int M, int F,
                              int H, int E, const bf16_t* wd, void* y, int layout,
                              const void* sd = nullptr);

// The fused layer's down projection (routed + optional shared segment) with
// fp32 output; pointers may be null when only the shape matters.
moe::GemmProblem forward_down_problem(int T, int H, int F, int E, int k, int Fs) {
  moe::GemmProblem g2 = down_problem(nullptr, nullptr, T * k, F, H, E, nullptr, nullptr, 0);
  g2.out_f32 = true;
  if (Fs > 0) {
    g2.seg[1] = moe::GemmSegment{nullptr, nullptr, nullptr, nullptr, nullptr, 0, 0, T, 1, Fs, H};
    g2.nseg = 2;
  }
  return g2;
}

ForwardLayout forward_layout(int T, int H, int F, int E, int k, int Fs, int cus) {
  ForwardLayout L;
  moe::GemmProblem g2 = forward_down_problem(T, H, F, E, k, Fs);
  moe::grouped_gemm_plan_ksplit(g2, cus);
  L.ksplit = g2.seg[0].ksplit;
  L.ksplit_sh = g2.nseg > 1 ? g2.seg[1].ksplit : 1;
  const size_t A = static_cast<size_t>(T) * k;
  const size_t S = static_cast<size_t>(L.ksplit);
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align_up(o + bytes, 256); return at; };
  L.hist = take(static_cast<size_t>(moe::route_num_chunks(T, k)) * E * 4);
  L.ids = take(A * 4);
  L.w = take(A * 4);
  L.offsets = take((static_cast<size_t>(E) + 1) * 4);
  L.row_token = take(A * 4);
  L.row_dest = take(A * 4);
  L.x_perm = take(A * H * 2);
  L.h = take(A * F * 2);
  L.h_sh = take(static_cast<size_t>(T) * (Fs > 0 ? Fs : 0) * 2);
  L.y = take(S * A * H * 4);                                       // fp32
  L.y_sh = take(static_cast<size_t>(L.ksplit_sh) * T * (Fs > 0 ? H : 0) * 4);  // fp32
  // arrival counters of a down projection that combines in its epilogue:
  // one per token and 64-column tile of the output
  L.cnt = take(static_cast<size_t>(T) * ((H + 63) / 64) * 4);
  L.total = o;
  return L;
}

// Weight layouts: 0 [K][N] bf16, 1 packed bf16 blocks, 2 packed fp8 codes
// (+ per-column scales), 3 packed mxfp4 codes (+ scale bytes), 5 packed
// mxfp8 codes (the fp8 blocks, + mxfp4-layout scale bytes).
constexpr int kRowMajor = 0, kPackedBf16 = 1, kFp8 = 2, kMxfp4 = 3, kMxfp8 = 5;

// layouts whose codes come with scales (a second pointer per matrix)
bool has_scales(int layout) { return layout == kFp8 || layout == kMxfp4 || layout == kMxfp8; }

// Elements (bf16-sized) between consecutive experts' weight matrices.
int64_t weight_stride(int K, int N, int layout) {
  return layout == kFp8 || layout == kMxfp8 ? moe::fp8_weight_bytes(1, K, N) / 2
         : layout == kMxfp4      ? moe::mxfp4_weight_bytes(1, K, N) / 2
         : layout == kPackedBf16 ? moe::packed_weight_elems(1, K, N)
                                 : static_cast<int64_t>(K) * N;
}

moe::GemmSegment segment(const bf16_t* act, const int32_t* offsets, const bf16_t* w0,
                         const bf16_t* w1, void* out, int rows, int ngroups, int K, int N,
                         int layout, const void* s0, const void* s1) {
  moe::GemmSegment g{act, offsets, w0, w1, out, weight_stride(K, N, layout), 0, rows, ngroups,
                     K, N, layout};
  g.scale0 = s0;
  g.scale1 = s1;
  return g;
}

moe::GemmProblem gateup_problem(const bf16_t* x_perm, const int32_t* offsets, int M,
                                int H, int F, int E, const bf16_t* wg,
                                const bf16_t* wu, bf16_t* h, int layout,
                                const void* sg = nullptr, const void* su = nullptr) {
  moe::GemmProblem p{};
  p.seg[0] = segment(x_perm, offsets, wg, wu, h, M, E, H, F, layout, sg, su);
  p.nseg = 1;
  p.gated = true;
  p.rows_hint = M / E;
  return p;
}

moe::GemmProblem down_problem(const bf16_t* h, const int32_t* offsets, int M, int F,
                              int H, int E, const bf16_t* wd, void* y, int layout,
                              const void* sd) {
  moe::GemmProblem p{};
  p.seg[0] = segment(h, offsets, wd, nullptr, y, M, E, F, H, layout, sd, nullptr);
  p.nseg = 1;
  p.gated = false;
  p.rows_hint = M / E;
  return p;
}

int check_ffn_args(const void* act, const int32_t* offsets, int M, int K, int N, int E,
                   const void* w0, const void* w1, bool need_w1, const void* out) {
  if (M < 0 || E < 1) return MOE_ERR_INVALID_ARG;
  if (E > moe::kMaxExperts) return MOE_ERR_UNSUPPORTED_SHAPE;
  MOE_TRY(check_width(K));
  MOE_TRY(check_width(N));
  MOE_TRY(check_elems(M, K > N ? K : N));
  if (M == 0) return MOE_OK;
  MOE_TRY(need_bf16(act));
  MOE_TRY(need_word(offsets));
  MOE_TRY(need_bf16(w0));
  if (need_w1) MOE_TRY(need_bf16(w1));
  MOE_TRY(need_bf16(out));
  return MOE_OK;
}

}  // namespace

// ---- the forward without allocation ---------------------------------------
// A fixed device array serves as moe_forward_packed's workspace, for callers
// that cannot allocate (graph capture, tight serving loops). Each GPU holds
// its own copy from the library's load until the process ends. In host code
// the array's name only stands for the symbol: its device address is taken
// once per device with hipGetSymbolAddress, and only that address is passed
// to kernels.
constexpr size_t kStaticWorkspaceBytes = size_t(128) << 20;  // 128 MiB
static __device__ __align__(256) char scratch[kStaticWorkspaceBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch` (looked up on the first call on
// that device, with the device current).
int scratch_address(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED_SHAPE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MOE_OK;
}
}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: null pointer or non-positive size";
    case MOE_ERR_UNSUPPORTED_SHAPE: return "MOE_ERR_UNSUPPORTED_SHAPE: size outside the supported limits";
    case MOE_ERR_MISALIGNED: return "MOE_ERR_MISALIGNED: pointer not aligned (bf16 tensors need 16 bytes)";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL: workspace below the required size";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: a HIP runtime call or kernel launch failed";
    case MOE_ERR_BAD_IDS: return "MOE_ERR_BAD_IDS: an expert id outside [0, E) (debug check)";
    default: return "unknown moe status";
  }
}

int moe_route(const float* logits, int T, int E, int k, int32_t* topk_ids,
              float* topk_w, void* stream) {
  MOE_TRY(check_dims(T, E, k));
  MOE_TRY(check_elems(T, E));
  if (T == 0) return MOE_OK;
  MOE_TRY(need_word(logits));
  MOE_TRY(need_word(topk_ids));
  MOE_TRY(need_word(topk_w));
  return hip_status(moe::launch_route(logits, T, E, k, topk_ids, topk_w, nullptr,
                                      static_cast<hipStream_t>(stream)));
}

size_t moe_router_workspace_bytes(int T, int H, int E, int k) {
  if (check_dims(T, E, k) != MOE_OK || check_width(H) != MOE_OK || T == 0) return 0;
  const moe::RouterPlan p = moe::router_plan(T, H, E, moe::grouped_gemm_device_cus());
  return align_up(moe::router_part_elems(p, T, E) * sizeof(float), 256);
}

int moe_router_route(const moe_bf16* x, const moe_bf16* w_router, int T, int H, int E,
                     int k, float* logits_out, int32_t* topk_ids, float* topk_w,
                     void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_dims(T, E, k));
  MOE_TRY(check_width(H));
  MOE_TRY(check_elems(T, H));
  MOE_TRY(check_elems(E, H));
  MOE_TRY(check_elems(T, E));
  if (T == 0) return MOE_OK;
  MOE_TRY(need_bf16(x));
  MOE_TRY(need_bf16(w_router));
  if (logits_out) MOE_TRY(need_word(logits_out));
  MOE_TRY(need_word(topk_ids));
  MOE_TRY(need_word(topk_w));
  const moe::RouterPlan p = moe::router_plan(T, H, E, moe::grouped_gemm_device_cus());
  const size_t need = align_up(moe::router_part_elems(p, T, E) * sizeof(float), 256);
  if (ws_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (need > 0) MOE_TRY(need_bf16(ws));
  return hip_status(moe::launch_router(p, x, w_router, T, H, E, k, logits_out,
                                       static_cast<float*>(ws), topk_ids, topk_w,
                                       static_cast<hipStream_t>(stream)));
}

size_t moe_permute_workspace_bytes(int T, int E, int k) {
  if (check_dims(T, E, k) != MOE_OK) return 0;
  return permute_ws_bytes(T, E, k);
}

int moe_permute(const moe_bf16* x, const int32_t* topk_ids, int T, int H, int E,
                int k, int32_t* expert_offsets, int32_t* row_token,
                int32_t* row_dest, moe_bf16* x_perm, void* ws, size_t ws_bytes,
                void* stream) {
  MOE_TRY(check_dims(T, E, k));
  MOE_TRY(check_width(H));
  MOE_TRY(check_elems(static_cast<int64_t>(T) * k, H));
  if (T == 0) return MOE_OK;
  MOE_TRY(need_bf16(x));
  MOE_TRY(need_word(topk_ids));
  MOE_TRY(need_word(expert_offsets));
  MOE_TRY(need_word(row_token));
  MOE_TRY(need_word(row_dest));
  MOE_TRY(need_bf16(x_perm));
  MOE_TRY(need_bf16(ws));
  if (ws_bytes < permute_ws_bytes(T, E, k)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  MOE_TRY(debug_check_ids(topk_ids, static_cast<int64_t>(T) * k, E, stream));
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t* hist = static_cast<int32_t*>(ws);
  MOE_TRY(hip_status(moe::launch_hist(topk_ids, T, E, k, hist, s)));
  return hip_status(moe::launch_permute(x, topk_ids, T, H, E, k, hist, expert_offsets,
                                        row_token, row_dest, x_perm, s));
}

static int gateup_impl(const moe_bf16* x_perm, const int32_t* expert_offsets, int M, int H,
                       int F, int E, const moe_bf16* w_gate, const moe_bf16* w_up, moe_bf16* h,
                       void* stream, int layout, const void* sg = nullptr,
                       const void* su = nullptr) {
  MOE_TRY(check_ffn_args(x_perm, expert_offsets, M, H, F, E, w_gate, w_up, true, h));
  if (M == 0) return MOE_OK;
  if (has_scales(layout)) {
    MOE_TRY(need_bf16(sg));
    MOE_TRY(need_bf16(su));
  }
  return hip_status(moe::launch_grouped_gemm(
      gateup_problem(x_perm, expert_offsets, M, H, F, E, w_gate, w_up, h, layout, sg, su),
      static_cast<hipStream_t>(stream)));
}

static int down_impl(const moe_bf16* h, const int32_t* expert_offsets, int M, int F, int H,
                     int E, const moe_bf16* w_down, moe_bf16* y_perm, void* stream,
                     int layout, const void* sd = nullptr) {
  MOE_TRY(check_ffn_args(h, expert_offsets, M, F, H, E, w_down, nullptr, false, y_perm));
  if (M == 0) return MOE_OK;
  if (has_scales(layout)) MOE_TRY(need_bf16(sd));
  return hip_status(moe::launch_grouped_gemm(
      down_problem(h, expert_offsets, M, F, H, E, w_down, y_perm, layout, sd),
      static_cast<hipStream_t>(stream)));
}

int moe_gateup_swiglu(const moe_bf16* x_perm, const int32_t* expert_offsets, int M,
                      int H, int F, int E, const moe_bf16* w_gate,
                      const moe_bf16* w_up, moe_bf16* h, void* stream) {
  return gateup_impl(x_perm, expert_offsets, M, H, F, E, w_gate, w_up, h, stream, kRowMajor);
}

int moe_gateup_swiglu_packed(const moe_bf16* x_perm, const int32_t* expert_offsets, int M,
                             int H, int F, int E, const moe_bf16* w_gate_packed,
                             const moe_bf16* w_up_packed, moe_bf16* h, void* stream) {
  return gateup_impl(x_perm, expert_offsets, M, H, F, E, w_gate_packed, w_up_packed, h,
                     stream, kPackedBf16);
}

int moe_down(const moe_bf16* h, const int32_t* expert_offsets, int M, int F, int H,
             int E, const moe_bf16* w_down, moe_bf16* y_perm, void* stream) {
  return down_impl(h, expert_offsets, M, F, H, E, w_down, y_perm, stream, kRowMajor);
}

int moe_down_packed(const moe_bf16* h, const int32_t* expert_offsets, int M, int F, int H,
                    int E, const moe_bf16* w_down_packed, moe_bf16* y_perm, void* stream) {
  return down_impl(h, expert_offsets, M, F, H, E, w_down_packed, y_perm, stream, kPackedBf16);
}

size_t moe_fp8_weights_bytes(int G, int K, int N) {
  if (G < 1 || check_width(K) != MOE_OK || check_width(N) != MOE_OK) return 0;
  return static_cast<size_t>(moe::fp8_weight_bytes(G, K, N));
}

int moe_quantize_fp8(const moe_bf16* w, int G, int K, int N, uint8_t* codes,
                     size_t codes_bytes, float* scales, void* stream) {
  if (G < 1) return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_width(K));
  MOE_TRY(check_width(N));
  MOE_TRY(need_bf16(w));
  MOE_TRY(need_bf16(codes));
  MOE_TRY(need_bf16(scales));
  if (codes_bytes < moe_fp8_weights_bytes(G, K, N)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return hip_status(moe::launch_quantize_fp8(w, G, K, N, codes, scales,
                                             static_cast<hipStream_t>(stream)));
}

int moe_gateup_swiglu_fp8(const moe_bf16* x_perm, const int32_t* expert_offsets, int M, int H,
                          int F, int E, const uint8_t* w_gate, const float* s_gate,
                          const uint8_t* w_up, const float* s_up, moe_bf16* h, void* stream) {
  return gateup_impl(x_perm, expert_offsets, M, H, F, E, reinterpret_cast<const bf16_t*>(w_gate),
                     reinterpret_cast<const bf16_t*>(w_up), h, stream, kFp8, s_gate, s_up);
}

int moe_down_fp8(const moe_bf16* h, const int32_t* expert_offsets, int M, int F, int H, int E,
                 const uint8_t* w_down, const float* s_down, moe_bf16* y_perm, void* stream) {
  return down_impl(h, expert_offsets, M, F, H, E, reinterpret_cast<const bf16_t*>(w_down),
                   y_perm, stream, kFp8, s_down);
}

size_t moe_mxfp4_weights_bytes(int G, int K, int N) {
  if (G < 1 || check_width(K) != MOE_OK || check_width(N) != MOE_OK) return 0;
  return static_cast<size_t>(moe::mxfp4_weight_bytes(G, K, N));
}

size_t moe_mxfp4_scales_bytes(int G, int K, int N) {
  if (G < 1 || check_width(K) != MOE_OK || check_width(N) != MOE_OK) return 0;
  return static_cast<size_t>(moe::mxfp4_scale_bytes(G, K, N));
}

int moe_quantize_mxfp4(const moe_bf16* w, int G, int K, int N, uint8_t* codes,
                       size_t codes_bytes, uint8_t* scales, size_t scales_bytes, void* stream) {
  if (G < 1) return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_width(K));
  MOE_TRY(check_width(N));
  MOE_TRY(need_bf16(w));
  MOE_TRY(need_bf16(codes));
  MOE_TRY(need_bf16(scales));
  if (codes_bytes < moe_mxfp4_weights_bytes(G, K, N) ||
      scales_bytes < moe_mxfp4_scales_bytes(G, K, N))
    return MOE_ERR_WORKSPACE_TOO_SMALL;
  return hip_status(moe::launch_quantize_mxfp4(w, G, K, N, codes, scales,
                                               static_cast<hipStream_t>(stream)));
}

int moe_gateup_swiglu_mxfp4(const moe_bf16* x_perm, const int32_t* expert_offsets, int M, int H,
                            int F, int E, const uint8_t* w_gate, const uint8_t* s_gate,
                            const uint8_t* w_up, const uint8_t* s_up, moe_bf16* h,
                            void* stream) {
  return gateup_impl(x_perm, expert_offsets, M, H, F, E, reinterpret_cast<const bf16_t*>(w_gate),
                     reinterpret_cast<const bf16_t*>(w_up), h, stream, kMxfp4, s_gate, s_up);
}

int moe_down_mxfp4(const moe_bf16* h, const int32_t* expert_offsets, int M, int F, int H, int E,
                   const uint8_t* w_down, const uint8_t* s_down, moe_bf16* y_perm, void* stream) {
  return down_impl(h, expert_offsets, M, F, H, E, reinterpret_cast<const bf16_t*>(w_down),
                   y_perm, stream, kMxfp4, s_down);
}

size_t moe_mxfp8_weights_bytes(int G, int K, int N) {
  if (G < 1 || check_width(K) != MOE_OK || check_width(N) != MOE_OK) return 0;
  return static_cast<size_t>(moe::fp8_weight_bytes(G, K, N));
}

size_t moe_mxfp8_scales_bytes(int G, int K, int N) {
  if (G < 1 || check_width(K) != MOE_OK || check_width(N) != MOE_OK) return 0;
  return static_cast<size_t>(moe::mxfp4_scale_bytes(G, K, N));
}

int moe_quantize_mxfp8(const moe_bf16* w, int G, int K, int N, uint8_t* codes,
                       size_t codes_bytes, uint8_t* scales, size_t scales_bytes, void* stream) {
  if (G < 1) return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_width(K));
  MOE_TRY(check_width(N));
  MOE_TRY(need_bf16(w));
  MOE_TRY(need_bf16(codes));
  MOE_TRY(need_bf16(scales));
  if (codes_bytes < moe_mxfp8_weights_bytes(G, K, N) ||
      scales_bytes < moe_mxfp8_scales_bytes(G, K, N))
    return MOE_ERR_WORKSPACE_TOO_SMALL;
  return hip_status(moe::launch_quantize_mxfp8(w, G, K, N, codes, scales,
                                               static_cast<hipStream_t>(stream)));
}

int moe_gateup_swiglu_mxfp8(const moe_bf16* x_perm, const int32_t* expert_offsets, int M, int H,
                            int F, int E, const uint8_t* w_gate, const uint8_t* s_gate,
                            const uint8_t* w_up, const uint8_t* s_up, moe_bf16* h,
                            void* stream) {
  return gateup_impl(x_perm, expert_offsets, M, H, F, E, reinterpret_cast<const bf16_t*>(w_gate),
                     reinterpret_cast<const bf16_t*>(w_up), h, stream, kMxfp8, s_gate, s_up);
}

int moe_down_mxfp8(const moe_bf16* h, const int32_t* expert_offsets, int M, int F, int H, int E,
                   const uint8_t* w_down, const uint8_t* s_down, moe_bf16* y_perm, void* stream) {
  return down_impl(h, expert_offsets, M, F, H, E, reinterpret_cast<const bf16_t*>(w_down),
                   y_perm, stream, kMxfp8, s_down);
}

size_t moe_pack_weights_bytes(int G, int K, int N) {
  if (G < 1 || check_width(K) != MOE_OK || check_width(N) != MOE_OK) return 0;
  return static_cast<size_t>(moe::packed_weight_elems(G, K, N)) * sizeof(bf16_t);
}

int moe_pack_weights(const moe_bf16* w, int G, int K, int N, moe_bf16* packed,
                     size_t packed_bytes, void* stream) {
  if (G < 1) return MOE_ERR_INVALID_ARG;
  MOE_TRY(check_width(K));
  MOE_TRY(check_width(N));
  MOE_TRY(need_bf16(w));
  MOE_TRY(need_bf16(packed));
  if (packed_bytes < moe_pack_weights_bytes(G, K, N)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return hip_status(moe::launch_pack_weights(w, G, K, N, packed,
                                             static_cast<hipStream_t>(stream)));
}

size_t moe_grouped_ffn_workspace_bytes(int M, int F) {
  if (M < 0 || check_width(F) != MOE_OK || check_elems(M, F) != MOE_OK) return 0;
  return align_up(static_cast<size_t>(M) * F * sizeof(bf16_t), 256);
}

int moe_grouped_ffn(const moe_bf16* x_perm, const int32_t* expert_offsets, int M,
                    int H, int F, int E, const moe_bf16* w_gate,
                    const moe_bf16* w_up, const moe_bf16* w_down, moe_bf16* y_perm,
                    void* ws, size_t ws_bytes, void* stream) {
  // h lives at the start of the workspace
  moe_bf16* h = static_cast<moe_bf16*>(ws);
  MOE_TRY(check_ffn_args(x_perm, expert_offsets, M, H, F, E, w_gate, w_up, true,
                         M == 0 ? nullptr : h));
  MOE_TRY(check_ffn_args(x_perm, expert_offsets, M, F, H, E, w_down, nullptr, false, y_perm));
  if (M == 0) return MOE_OK;
  if (ws_bytes < moe_grouped_ffn_workspace_bytes(M, F)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  MOE_TRY(hip_status(moe::launch_grouped_gemm(
      gateup_problem(x_perm, expert_offsets, M, H, F, E, w_gate, w_up, h, kRowMajor), s)));
  return hip_status(moe::launch_grouped_gemm(
      down_problem(h, expert_offsets, M, F, H, E, w_down, y_perm, kRowMajor), s));
}

int moe_combine(const moe_bf16* y_perm, const int32_t* row_dest, const float* topk_w,
                int T, int H, int k, moe_bf16* out, void* stream) {
  if (T < 0 || k < 1) return MOE_ERR_INVALID_ARG;
  if (k > moe::kMaxTopK) return MOE_ERR_UNSUPPORTED_SHAPE;
  MOE_TRY(check_width(H));
  MOE_TRY(check_elems(static_cast<int64_t>(T) * k, H));
  if (T == 0) return MOE_OK;
  MOE_TRY(need_bf16(y_perm));
  MOE_TRY(need_word(row_dest));
  MOE_TRY(need_word(topk_w));
  MOE_TRY(need_bf16(out));
  return hip_status(moe::launch_combine(y_perm, false, 1, 0, row_dest, topk_w, T, H, k,
                                        nullptr, 1, 0, nullptr, out,
                                        static_cast<hipStream_t>(stream)));
}

size_t moe_forward_workspace_bytes(int T, int H, int F, int E, int k, int Fs) {
  if (check_dims(T, E, k) != MOE_OK || check_width(H) != MOE_OK ||
      check_width(F) != MOE_OK || Fs < 0 || (Fs > 0 && check_width(Fs) != MOE_OK))
    return 0;
  return forward_layout(T, H, F, E, k, Fs, moe::grouped_gemm_device_cus()).total;
}

size_t moe_workspace_bytes(int T, int H, int F, int E, int k, int Fs) {
  return moe_forward_workspace_bytes(T, H, F, E, k, Fs);
}

int moe_set_diagnostics(int trace, int check_ids) {
  if (trace < -1 || trace > 1 || check_ids < -1 || check_ids > 1) return MOE_ERR_INVALID_ARG;
  moe::set_diagnostics(trace, check_ids);
  return MOE_OK;
}

int moe_check_topk_ids(const int32_t* topk_ids, int T, int k, int E, void* stream) {
  MOE_TRY(check_dims(T, E, k));
  if (T == 0) return MOE_OK;
  MOE_TRY(need_word(topk_ids));
  int bad = 0;
  if (moe::count_bad_ids(topk_ids, static_cast<int64_t>(T) * k, E,
                         static_cast<hipStream_t>(stream), &bad) != hipSuccess)
    return MOE_ERR_HIP;
  return bad ? MOE_ERR_BAD_IDS : MOE_OK;
}

int moe_set_dispatch_override(int decode_path, int tile_class) {
  if (decode_path < -1 || decode_path > 1 || tile_class < -1 || tile_class > 3)
    return MOE_ERR_INVALID_ARG;
  moe::set_dispatch_override(decode_path, tile_class);
  return MOE_OK;
}

int moe_set_combine_override(int mode) {
  if (mode < -1 || mode > 1) return MOE_ERR_INVALID_ARG;
  moe::set_scatter_override(mode);
  return MOE_OK;
}

// The layer's weights in one layout (the shared expert's too, when Fs > 0).
struct LayerWeights {
  int layout;
  const bf16_t *wg, *wu, *wd;   // fp8, mxfp4: the codes
  const void *sg, *su, *sd;     // fp8: column scales; mxfp4: scale bytes
  bool shared;
  int Fs;
  const bf16_t *swg, *swu, *swd;
  const void *ssg, *ssu, *ssd;
  const float* gate_logits;
};

LayerWeights bf16_weights(const moe_bf16* wg, const moe_bf16* wu, const moe_bf16* wd,
                          const moe_shared_expert* sh, int layout) {
  LayerWeights W{};
  W.layout = layout;
  W.wg = wg, W.wu = wu, W.wd = wd;
  W.shared = sh != nullptr;
  if (sh) {
    W.Fs = sh->Fs;
    W.swg = sh->w_gate, W.swu = sh->w_up, W.swd = sh->w_down;
    W.gate_logits = sh->gate_logits;
  }
  return W;
}

// The layer from router logits (logits != null: steps 1-5) or from a routing
// the caller made (ids_in / w_in: steps 2-5).
static int forward_impl(const moe_bf16* x, const float* logits, const int32_t* ids_in,
                        const float* w_in, int T, int H, int F, int E, int k,
                        const LayerWeights& W, moe_bf16* out, int32_t* topk_ids_out,
                        float* topk_w_out, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_dims(T, E, k));
  MOE_TRY(check_width(H));
  MOE_TRY(check_width(F));
  const bool shared = W.shared;
  const int Fs = shared ? W.Fs : 0;
  if (shared) MOE_TRY(check_width(Fs));
  const bool fp8 = has_scales(W.layout);  // codes + scales
  const int64_t A = static_cast<int64_t>(T) * k;
  const int64_t widest = (H > F ? H : F) > Fs ? (H > F ? H : F) : Fs;
  MOE_TRY(check_elems(A, widest));
  MOE_TRY(check_elems(T, E));
  if (T == 0) return MOE_OK;
  MOE_TRY(need_bf16(x));
  if (logits) {
    MOE_TRY(need_word(logits));
  } else {
    MOE_TRY(need_word(ids_in));
    MOE_TRY(need_word(w_in));
  }
  MOE_TRY(need_bf16(W.wg));
  MOE_TRY(need_bf16(W.wu));
  MOE_TRY(need_bf16(W.wd));
  if (fp8) {
    MOE_TRY(need_bf16(W.sg));
    MOE_TRY(need_bf16(W.su));
    MOE_TRY(need_bf16(W.sd));
  }
  MOE_TRY(need_bf16(out));
  if (topk_ids_out) MOE_TRY(need_word(topk_ids_out));
  if (topk_w_out) MOE_TRY(need_word(topk_w_out));
  if (shared) {
    MOE_TRY(need_bf16(W.swg));
    MOE_TRY(need_bf16(W.swu));
    MOE_TRY(need_bf16(W.swd));
    if (fp8) {
      MOE_TRY(need_bf16(W.ssg));
      MOE_TRY(need_bf16(W.ssu));
      MOE_TRY(need_bf16(W.ssd));
    }
    if (W.gate_logits) MOE_TRY(need_word(W.gate_logits));
  }
  MOE_TRY(need_bf16(ws));
  const ForwardLayout L = forward_layout(T, H, F, E, k, Fs, moe::grouped_gemm_device_cus());
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (!logits) MOE_TRY(debug_check_ids(ids_in, A, E, stream));

  char* base = static_cast<char*>(ws);
  int32_t* hist = reinterpret_cast<int32_t*>(base + L.hist);
  int32_t* ids = topk_ids_out ? topk_ids_out : reinterpret_cast<int32_t*>(base + L.ids);
  float* w = topk_w_out ? topk_w_out : reinterpret_cast<float*>(base + L.w);
  const int32_t* ids_c = logits ? ids : ids_in;
  const float* w_c = logits ? w : w_in;
  int32_t* offsets = reinterpret_cast<int32_t*>(base + L.offsets);
  int32_t* row_token = reinterpret_cast<int32_t*>(base + L.row_token);
  int32_t* row_dest = reinterpret_cast<int32_t*>(base + L.row_dest);
  bf16_t* x_perm = reinterpret_cast<bf16_t*>(base + L.x_perm);
  bf16_t* h = reinterpret_cast<bf16_t*>(base + L.h);
  bf16_t* h_sh = reinterpret_cast<bf16_t*>(base + L.h_sh);
  float* y = reinterpret_cast<float*>(base + L.y);
  float* y_sh = reinterpret_cast<float*>(base + L.y_sh);
  int32_t* cnt = reinterpret_cast<int32_t*>(base + L.cnt);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int M = static_cast<int>(A);

  // 4's problem (grouped down, shared expert likewise) before any launch:
  // when its tiles also combine (at decode sizes, through the testing hook),
  // the permutation clears their arrival counters. The K-split plan is the
  // same for every weight layout (the workspace size does not depend on it).
  moe::GemmProblem g2 = down_problem(h, offsets, M, F, H, E, W.wd, y, W.layout, W.sd);
  g2.out_f32 = true;
  g2.seg[0].ksplit = L.ksplit;
  g2.seg[0].slice_stride = static_cast<int64_t>(M) * H;
  if (shared) {
    g2.seg[1] = segment(h_sh, nullptr, W.swd, nullptr, y_sh, T, 1, Fs, H, W.layout, W.ssd,
                        nullptr);
    g2.seg[1].slice_stride = static_cast<int64_t>(T) * H;
    g2.seg[1].ksplit = L.ksplit_sh;
    g2.nseg = 2;
  }
  const bool scatter = moe::grouped_gemm_scatters(g2);
  const int64_t ncnt = scatter ? static_cast<int64_t>(T) * ((H + 63) / 64) : 0;
  if (scatter) {
    moe::ScatterArgs& sa = g2.scat;
    sa.cnt = cnt;
    sa.target = k * L.ksplit + (shared ? L.ksplit_sh : 0);
    sa.T = T;
    sa.k = k;
    sa.row_token = row_token;
    sa.row_dest = row_dest;
    sa.topk_w = w_c;
    sa.y = y;
    sa.y_slice_stride = static_cast<int64_t>(M) * H;
    sa.y_slices = L.ksplit;
    sa.y_sh = shared ? y_sh : nullptr;
    sa.ysh_slice_stride = static_cast<int64_t>(T) * H;
    sa.ysh_slices = L.ksplit_sh;
    sa.gate_logits = shared ? W.gate_logits : nullptr;
    sa.out = out;
  }

  // 3's problem first: the large-batch tiles read the rows of x through
  // row_token themselves, and then the permutation copies no rows
  moe::GemmProblem g1 =
      gateup_problem(x_perm, offsets, M, H, F, E, W.wg, W.wu, h, W.layout, W.sg, W.su);
  const bool gather = moe::grouped_gemm_gathers(g1);
  if (gather) {
    g1.seg[0].act = x;
    g1.seg[0].gather = row_token;
    g1.seg[0].gather_rows = T;
  }
  if (logits && !gather && moe::route_permute_fits_one_launch(T, E, k)) {
    // 1+2. small batch: routing and the permutation in one launch
    MOE_TRY(hip_status(moe::launch_route_permute_small(logits, x, T, H, E, k, ids, w, offsets,
                                                       row_token, row_dest, x_perm, s,
                                                       scatter ? cnt : nullptr, ncnt)));
  } else {
    // 1. route + per-chunk histogram, or the histogram of the given routing
    if (logits)
      MOE_TRY(hip_status(moe::launch_route(logits, T, E, k, ids, w, hist, s)));
    else
      MOE_TRY(hip_status(moe::launch_hist(ids_in, T, E, k, hist, s)));
    // 2. permute: scan, stable rank, row maps (+ x_perm rows unless gathered)
    MOE_TRY(hip_status(moe::launch_permute(x, ids_c, T, H, E, k, hist, offsets, row_token,
                                           row_dest, gather ? nullptr : x_perm, s,
                                           scatter ? cnt : nullptr, ncnt)));
  }
  // 3. grouped gate/up + SwiGLU (shared expert as one more group over x)
  if (shared) {
    g1.seg[1] = segment(x, nullptr, W.swg, W.swu, h_sh, T, 1, H, Fs, W.layout, W.ssg, W.ssu);
    g1.nseg = 2;
  }
  MOE_TRY(hip_status(moe::launch_grouped_gemm(g1, s)));
  // 4. grouped down (+ 5. when its tiles combine)
  MOE_TRY(hip_status(moe::launch_grouped_gemm(g2, s)));
  if (scatter) return MOE_OK;
  // 5. combine (+ gated shared term)
  return hip_status(moe::launch_combine(y, true, L.ksplit, static_cast<int64_t>(M) * H,
                                        row_dest, w_c, T, H, k, shared ? y_sh : nullptr,
                                        L.ksplit_sh, static_cast<int64_t>(T) * H,
                                        shared ? W.gate_logits : nullptr, out, s));
}

int moe_forward(const moe_bf16* x, const float* logits, int T, int H, int F, int E,
                int k, const moe_bf16* w_gate, const moe_bf16* w_up,
                const moe_bf16* w_down, const moe_shared_expert* shared,
                moe_bf16* out, int32_t* topk_ids_out, float* topk_w_out, void* ws,
                size_t ws_bytes, void* stream) {
  return forward_impl(x, logits, nullptr, nullptr, T, H, F, E, k,
                      bf16_weights(w_gate, w_up, w_down, shared, kRowMajor), out, topk_ids_out,
                      topk_w_out, ws, ws_bytes, stream);
}

int moe_forward_packed(const moe_bf16* x, const float* logits, int T, int H, int F, int E,
                       int k, const moe_bf16* w_gate_packed, const moe_bf16* w_up_packed,
                       const moe_bf16* w_down_packed, const moe_shared_expert* shared_packed,
                       moe_bf16* out, int32_t* topk_ids_out, float* topk_w_out, void* ws,
                       size_t ws_bytes, void* stream) {
  return forward_impl(x, logits, nullptr, nullptr, T, H, F, E, k,
                      bf16_weights(w_gate_packed, w_up_packed, w_down_packed, shared_packed,
                                   kPackedBf16),
                      out, topk_ids_out, topk_w_out, ws, ws_bytes, stream);
}

int moe_forward_fp8(const moe_bf16* x, const float* logits, int T, int H, int F, int E, int k,
                    const uint8_t* w_gate, const float* s_gate, const uint8_t* w_up,
                    const float* s_up, const uint8_t* w_down, const float* s_down,
                    const moe_shared_expert_fp8* shared, moe_bf16* out, int32_t* topk_ids_out,
                    float* topk_w_out, void* ws, size_t ws_bytes, void* stream) {
  LayerWeights W{};
  W.layout = kFp8;
  W.wg = reinterpret_cast<const bf16_t*>(w_gate);
  W.wu = reinterpret_cast<const bf16_t*>(w_up);
  W.wd = reinterpret_cast<const bf16_t*>(w_down);
  W.sg = s_gate, W.su = s_up, W.sd = s_down;
  W.shared = shared != nullptr;
  if (shared) {
    W.Fs = shared->Fs;
    W.swg = reinterpret_cast<const bf16_t*>(shared->w_gate);
    W.swu = reinterpret_cast<const bf16_t*>(shared->w_up);
    W.swd = reinterpret_cast<const bf16_t*>(shared->w_down);
    W.ssg = shared->s_gate, W.ssu = shared->s_up, W.ssd = shared->s_down;
    W.gate_logits = shared->gate_logits;
  }
  return forward_impl(x, logits, nullptr, nullptr, T, H, F, E, k, W, out, topk_ids_out,
                      topk_w_out, ws, ws_bytes, stream);
}

int moe_forward_mxfp4(const moe_bf16* x, const float* logits, int T, int H, int F, int E, int k,
                      const uint8_t* w_gate, const uint8_t* s_gate, const uint8_t* w_up,
                      const uint8_t* s_up, const uint8_t* w_down, const uint8_t* s_down,
                      const moe_shared_expert_mxfp4* shared, moe_bf16* out,
                      int32_t* topk_ids_out, float* topk_w_out, void* ws, size_t ws_bytes,
                      void* stream) {
  LayerWeights W{};
  W.layout = kMxfp4;
  W.wg = reinterpret_cast<const bf16_t*>(w_gate);
  W.wu = reinterpret_cast<const bf16_t*>(w_up);
  W.wd = reinterpret_cast<const bf16_t*>(w_down);
  W.sg = s_gate, W.su = s_up, W.sd = s_down;
  W.shared = shared != nullptr;
  if (shared) {
    W.Fs = shared->Fs;
    W.swg = reinterpret_cast<const bf16_t*>(shared->w_gate);
    W.swu = reinterpret_cast<const bf16_t*>(shared->w_up);
    W.swd = reinterpret_cast<const bf16_t*>(shared->w_down);
    W.ssg = shared->s_gate, W.ssu = shared->s_up, W.ssd = shared->s_down;
    W.gate_logits = shared->gate_logits;
  }
  return forward_impl(x, logits, nullptr, nullptr, T, H, F, E, k, W, out, topk_ids_out,
                      topk_w_out, ws, ws_bytes, stream);
}

int moe_forward_packed_noalloc(const moe_bf16* x, const float* logits, int T, int H, int F,
                               int E, int k, const moe_bf16* w_gate_packed,
                               const moe_bf16* w_up_packed, const moe_bf16* w_down_packed,
                               const moe_shared_expert* shared_packed, moe_bf16* out,
                               int32_t* topk_ids_out, float* topk_w_out, void* stream) {
  void* ws = nullptr;
  MOE_TRY(scratch_address(&ws));
  // forward_impl checks the arguments first, then that the layer's
  // workspace fits the array (MOE_ERR_WORKSPACE_TOO_SMALL otherwise)
  return forward_impl(x, logits, nullptr, nullptr, T, H, F, E, k,
                      bf16_weights(w_gate_packed, w_up_packed, w_down_packed, shared_packed,
                                   kPackedBf16),
                      out, topk_ids_out, topk_w_out, ws, kStaticWorkspaceBytes, stream);
}

int moe_forward_mxfp8(const moe_bf16* x, const float* logits, int T, int H, int F, int E, int k,
                      const uint8_t* w_gate, const uint8_t* s_gate, const uint8_t* w_up,
                      const uint8_t* s_up, const uint8_t* w_down, const uint8_t* s_down,
                      const moe_shared_expert_mxfp8* shared, moe_bf16* out,
                      int32_t* topk_ids_out, float* topk_w_out, void* ws, size_t ws_bytes,
                      void* stream) {
  LayerWeights W{};
  W.layout = kMxfp8;
  W.wg = reinterpret_cast<const bf16_t*>(w_gate);
  W.wu = reinterpret_cast<const bf16_t*>(w_up);
  W.wd = reinterpret_cast<const bf16_t*>(w_down);
  W.sg = s_gate, W.su = s_up, W.sd = s_down;
  W.shared = shared != nullptr;
  if (shared) {
    W.Fs = shared->Fs;
    W.swg = reinterpret_cast<const bf16_t*>(shared->w_gate);
    W.swu = reinterpret_cast<const bf16_t*>(shared->w_up);
    W.swd = reinterpret_cast<const bf16_t*>(shared->w_down);
    W.ssg = shared->s_gate, W.ssu = shared->s_up, W.ssd = shared->s_down;
    W.gate_logits = shared->gate_logits;
  }
  return forward_impl(x, logits, nullptr, nullptr, T, H, F, E, k, W, out, topk_ids_out,
                      topk_w_out, ws, ws_bytes, stream);
}

int moe_forward_routed(const moe_bf16* x, const int32_t* topk_ids, const float* topk_w, int T,
                       int H, int F, int E, int k, const moe_bf16* w_gate, const moe_bf16* w_up,
                       const moe_bf16* w_down, const moe_shared_expert* shared,
                       int weights_packed, moe_bf16* out, void* ws, size_t ws_bytes,
                       void* stream) {
  if (weights_packed != 0 && weights_packed != 1) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!topk_ids || !topk_w)) return MOE_ERR_INVALID_ARG;
  return forward_impl(x, nullptr, topk_ids, topk_w, T, H, F, E, k,
                      bf16_weights(w_gate, w_up, w_down, shared,
                                   weights_packed == 1 ? kPackedBf16 : kRowMajor),
                      out, nullptr, nullptr, ws, ws_bytes, stream);
}


// ---- training backward ------------------------------------------------------
// Workspace of moe_backward (each piece 256-byte aligned from ws):
// [hist | offsets | row_token | row_dest | x_perm | h | G | U | dy |
//  dout_perm | dG | dU | wrow (fp32) | part (fp32 [A][ceil(F/16)]) |
//  dx parts (fp32, 2 slices)], and for the shared expert (Fs > 0) its own
// [h | G | U | dy | dG | dU (T rows) | wrow | part | dx parts | offsets].
struct BackwardLayout {
  size_t hist, offsets, row_token, row_dest, x_perm, h, g, u, dy, dop, dg, du, wrow, part, dxp;
  size_t hsh, gsh, ush, dysh, dgsh, dush, wsh, psh, dxsh, offsh;
  size_t total;
};

static BackwardLayout backward_layout(int T, int H, int F, int E, int k, int Fs) {
  BackwardLayout L;
  const size_t A = static_cast<size_t>(T) * k;
  const size_t Ts = Fs > 0 ? static_cast<size_t>(T) : 0;  // rows of the shared expert
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align_up(o + bytes, 256); return at; };
  L.hist = take(static_cast<size_t>(moe::route_num_chunks(T, k)) * E * 4);
  L.offsets = take((static_cast<size_t>(E) + 1) * 4);
  L.row_token = take(A * 4);
  L.row_dest = take(A * 4);
  L.x_perm = take(A * H * 2);
  L.h = take(A * F * 2);
  L.g = take(A * F * 2);
  L.u = take(A * F * 2);
  L.dy = take(A * H * 2);
  L.dop = take(A * H * 2);
  L.dg = take(A * F * 2);
  L.du = take(A * F * 2);
  L.wrow = take(A * 4);
  L.part = take(A * ((static_cast<size_t>(F) + 15) / 16) * 4);
  L.dxp = take(2 * A * H * 4);
  L.hsh = take(Ts * Fs * 2);
  L.gsh = take(Ts * Fs * 2);
  L.ush = take(Ts * Fs * 2);
  L.dysh = take(Ts * H * 2);
  L.dgsh = take(Ts * Fs * 2);
  L.dush = take(Ts * Fs * 2);
  L.wsh = take(Ts * 4);
  L.psh = take(Ts * ((static_cast<size_t>(Fs > 0 ? Fs : 0) + 15) / 16) * 4);
  L.dxsh = take(2 * Ts * H * 4);
  L.offsh = take(Fs > 0 ? 2 * 4 : 0);
  L.total = o;
  return L;
}

size_t moe_backward_workspace_bytes(int T, int H, int F, int E, int k) {
  if (check_dims(T, E, k) != MOE_OK || check_width(H) != MOE_OK || check_width(F) != MOE_OK)
    return 0;
  return backward_layout(T, H, F, E, k, 0).total;
}

size_t moe_backward_shared_workspace_bytes(int T, int H, int F, int E, int k, int Fs) {
  if (check_dims(T, E, k) != MOE_OK || check_width(H) != MOE_OK || check_width(F) != MOE_OK ||
      Fs < 0 || (Fs > 0 && check_width(Fs) != MOE_OK))
    return 0;
  return backward_layout(T, H, F, E, k, Fs).total;
}

// The routed layer's backward, and the shared expert's when `sh` is given.
static int backward_impl(const moe_bf16* x, const int32_t* topk_ids, const float* topk_w, int T,
                         int H, int F, int E, int k, const moe_bf16* w_gate,
                         const moe_bf16* w_up, const moe_bf16* w_down,
                         const moe_shared_expert* sh, moe_shared_expert_grads* sg,
                         const moe_bf16* dout, moe_bf16* dx, float* d_topk_w, float* dw_gate,
                         float* dw_up, float* dw_down, void* ws, size_t ws_bytes,
                         void* stream) {
  MOE_TRY(check_dims(T, E, k));
  MOE_TRY(check_width(H));
  MOE_TRY(check_width(F));
  const int64_t A = static_cast<int64_t>(T) * k;
  MOE_TRY(check_elems(A, H > F ? H : F));
  if (static_cast<int64_t>(H) * F >= kIndexLimit) return MOE_ERR_UNSUPPORTED_SHAPE;
  const int Fs = sh ? sh->Fs : 0;
  const float* gate = sh ? sh->gate_logits : nullptr;
  if (sh) {
    MOE_TRY(check_width(Fs));
    MOE_TRY(check_elems(T, H > Fs ? H : Fs));
    if (static_cast<int64_t>(H) * Fs >= kIndexLimit) return MOE_ERR_UNSUPPORTED_SHAPE;
    if (!sg) return MOE_ERR_INVALID_ARG;
    MOE_TRY(need_word(sg->dw_gate));
    MOE_TRY(need_word(sg->dw_up));
    MOE_TRY(need_word(sg->dw_down));
  }
  MOE_TRY(need_word(dw_gate));
  MOE_TRY(need_word(dw_up));
  MOE_TRY(need_word(dw_down));
  if (T > 0) {
    MOE_TRY(need_bf16(x));
    MOE_TRY(need_word(topk_ids));
    MOE_TRY(need_word(topk_w));
    MOE_TRY(need_bf16(w_gate));
    MOE_TRY(need_bf16(w_up));
    MOE_TRY(need_bf16(w_down));
    MOE_TRY(need_bf16(dout));
    MOE_TRY(need_bf16(dx));
    MOE_TRY(need_word(d_topk_w));
    if (sh) {
      MOE_TRY(need_bf16(sh->w_gate));
      MOE_TRY(need_bf16(sh->w_up));
      MOE_TRY(need_bf16(sh->w_down));
      if (gate) {
        MOE_TRY(need_word(gate));
        MOE_TRY(need_word(sg->d_gate_logits));
      }
    }
    MOE_TRY(need_bf16(ws));
  }
  const BackwardLayout L = backward_layout(T, H, F, E, k, Fs);
  if (T > 0 && ws_bytes < L.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (T > 0) MOE_TRY(debug_check_ids(topk_ids, A, E, stream));
  hipStream_t s = static_cast<hipStream_t>(stream);
  using moe::launch_kgrouped_gemm;
  if (T == 0) {
    // no tokens: every weight gradient is zero
    MOE_TRY(hip_status(launch_kgrouped_gemm(nullptr, nullptr, nullptr, E, H, F, dw_gate, s)));
    MOE_TRY(hip_status(launch_kgrouped_gemm(nullptr, nullptr, nullptr, E, H, F, dw_up, s)));
    MOE_TRY(hip_status(launch_kgrouped_gemm(nullptr, nullptr, nullptr, E, F, H, dw_down, s)));
    if (sh) {
      MOE_TRY(hip_status(launch_kgrouped_gemm(nullptr, nullptr, nullptr, 1, H, Fs, sg->dw_gate, s)));
      MOE_TRY(hip_status(launch_kgrouped_gemm(nullptr, nullptr, nullptr, 1, H, Fs, sg->dw_up, s)));
      MOE_TRY(hip_status(launch_kgrouped_gemm(nullptr, nullptr, nullptr, 1, Fs, H, sg->dw_down, s)));
    }
    return MOE_OK;
  }
  char* base = static_cast<char*>(ws);
  auto bf = [&](size_t off) { return reinterpret_cast<bf16_t*>(base + off); };
  auto fp = [&](size_t off) { return reinterpret_cast<float*>(base + off); };
  int32_t* hist = reinterpret_cast<int32_t*>(base + L.hist);
  int32_t* offsets = reinterpret_cast<int32_t*>(base + L.offsets);
  int32_t* row_token = reinterpret_cast<int32_t*>(base + L.row_token);
  int32_t* row_dest = reinterpret_cast<int32_t*>(base + L.row_dest);
  bf16_t *x_perm = bf(L.x_perm), *h = bf(L.h), *g = bf(L.g), *u = bf(L.u), *dy = bf(L.dy);
  bf16_t *dop = bf(L.dop), *dg = bf(L.dg), *du = bf(L.du);
  float *wrow = fp(L.wrow), *part = fp(L.part), *dxp = fp(L.dxp);
  bf16_t *hsh = bf(L.hsh), *gsh = bf(L.gsh), *ush = bf(L.ush), *dysh = bf(L.dysh);
  bf16_t *dgsh = bf(L.dgsh), *dush = bf(L.dush);
  float *wsh = fp(L.wsh), *psh = fp(L.psh), *dxsh = fp(L.dxsh);
  int32_t* offsh = reinterpret_cast<int32_t*>(base + L.offsh);
  const int M = static_cast<int>(A);

  // recompute: permutation (x_perm is kept for the weight
  // gradients) and gate/up storing G and U beside h (the down projection is
  // not needed: the routing-weight gradient comes from dh's epilogue); the
  // shared expert is a second segment over x
  MOE_TRY(hip_status(moe::launch_hist(topk_ids, T, E, k, hist, s)));
  MOE_TRY(hip_status(moe::launch_permute(x, topk_ids, T, H, E, k, hist, offsets, row_token,
                                         row_dest, x_perm, s)));
  moe::GemmProblem g1 =
      gateup_problem(x_perm, offsets, M, H, F, E, w_gate, w_up, h, kRowMajor);
  g1.epi = moe::kStoreGUH;
  g1.seg[0].out2 = g;
  g1.seg[0].out3 = u;
  if (sh) {
    g1.seg[1] = segment(x, nullptr, sh->w_gate, sh->w_up, hsh, T, 1, H, Fs, kRowMajor, nullptr,
                        nullptr);
    g1.seg[1].out2 = gsh;
    g1.seg[1].out3 = ush;
    g1.nseg = 2;
  }
  MOE_TRY(hip_status(moe::launch_grouped_gemm(g1, s)));
  // per row: dy = w dout (for dW_down), dout itself and w; the shared
  // expert's rows are the tokens, with s_t for w
  MOE_TRY(hip_status(
      moe::launch_backward_prep(dout, row_dest, topk_w, T, H, k, dy, dop, wrow, s)));
  if (sh) MOE_TRY(hip_status(moe::launch_shared_prep(dout, gate, T, H, dysh, wsh, offsh, s)));
  // g = dout W_down^T per row (W_down [F][H] is the [N][K] operand), with
  // the SwiGLU backward in the epilogue: dG, dU from dh = w g, and the
  // partial sums of <h, g> for the routing-weight gradient
  auto dh_problem = [&](const bf16_t* act, const int32_t* offs, const bf16_t* wd, bf16_t* dG,
                        int rows, int groups, int n, const bf16_t* G_, const bf16_t* U_,
                        const bf16_t* h_, const float* wr, float* pt, bf16_t* dU) {
    moe::GemmProblem q{};
    q.seg[0] = segment(act, offs, wd, nullptr, dG, rows, groups, H, n, moe::kWeightsTransposed,
                       nullptr, nullptr);
    q.seg[0].aux0 = G_;
    q.seg[0].aux1 = U_;
    q.seg[0].aux2 = h_;
    q.seg[0].wrow = wr;
    q.seg[0].part = pt;
    q.seg[0].out2 = dU;
    q.nseg = 1;
    q.gated = false;
    q.rows_hint = rows / groups;
    q.epi = moe::kSwigluBwd;
    return q;
  };
  MOE_TRY(hip_status(moe::launch_grouped_gemm(
      dh_problem(dop, offsets, w_down, dg, M, E, F, g, u, h, wrow, part, du), s)));
  MOE_TRY(hip_status(moe::launch_topk_w_grad(part, (F + 15) / 16, row_dest, T, k, d_topk_w, s)));
  if (sh) {
    MOE_TRY(hip_status(moe::launch_grouped_gemm(
        dh_problem(dout, nullptr, sh->w_down, dgsh, T, 1, Fs, gsh, ush, hsh, wsh, psh, dush), s)));
    if (gate)
      MOE_TRY(hip_status(
          moe::launch_shared_gate_grad(psh, (Fs + 15) / 16, gate, T, sg->d_gate_logits, s)));
  }
  // dx: dG W_gate^T and dU W_up^T per row (fp32 slices), summed over the
  // token's k rows and the two slices by the combine with unit weights
  // (plus the shared expert's two slices per token). Both products run as
  // the two segments of one launch (twice the items of either alone, which
  // at a few row tiles per expert left half of the CUs idle), while their
  // groups fit the item table.
  auto dx_segment = [&](int slice) {
    return segment(slice ? du : dg, offsets, slice ? w_up : w_gate, nullptr,
                   dxp + static_cast<int64_t>(slice) * M * H, M, E, F, H,
                   moe::kWeightsTransposed, nullptr, nullptr);
  };
  auto dx_shared_segment = [&](int slice) {
    return segment(slice ? dush : dgsh, nullptr, slice ? sh->w_up : sh->w_gate, nullptr,
                   dxsh + static_cast<int64_t>(slice) * T * H, T, 1, Fs, H,
                   moe::kWeightsTransposed, nullptr, nullptr);
  };
  auto plain_f32 = [](int rows_hint) {
    moe::GemmProblem q{};
    q.nseg = 1;
    q.gated = false;
    q.out_f32 = true;
    q.rows_hint = rows_hint;
    return q;
  };
  if (2 * E <= moe::kMaxExperts + 1) {
    moe::GemmProblem g4 = plain_f32(M / E);
    g4.seg[0] = dx_segment(0);
    g4.seg[1] = dx_segment(1);
    g4.nseg = 2;
    MOE_TRY(hip_status(moe::launch_grouped_gemm(g4, s)));
  } else {
    for (int slice = 0; slice < 2; ++slice) {
      moe::GemmProblem g4 = plain_f32(M / E);
      g4.seg[0] = dx_segment(slice);
      MOE_TRY(hip_status(moe::launch_grouped_gemm(g4, s)));
    }
  }
  if (sh) {
    moe::GemmProblem g5 = plain_f32(T);
    g5.seg[0] = dx_shared_segment(0);
    g5.seg[1] = dx_shared_segment(1);
    g5.nseg = 2;
    MOE_TRY(hip_status(moe::launch_grouped_gemm(g5, s)));
  }
  MOE_TRY(hip_status(moe::launch_combine(dxp, true, 2, static_cast<int64_t>(M) * H, row_dest,
                                         nullptr, T, H, k, sh ? dxsh : nullptr, 2,
                                         static_cast<int64_t>(T) * H, nullptr, dx, s)));
  // weight gradients over each expert's rows (the shared expert's: all tokens)
  MOE_TRY(hip_status(launch_kgrouped_gemm(x_perm, dg, offsets, E, H, F, dw_gate, s)));
  MOE_TRY(hip_status(launch_kgrouped_gemm(x_perm, du, offsets, E, H, F, dw_up, s)));
  MOE_TRY(hip_status(launch_kgrouped_gemm(h, dy, offsets, E, F, H, dw_down, s)));
  if (sh) {
    MOE_TRY(hip_status(launch_kgrouped_gemm(x, dgsh, offsh, 1, H, Fs, sg->dw_gate, s)));
    MOE_TRY(hip_status(launch_kgrouped_gemm(x, dush, offsh, 1, H, Fs, sg->dw_up, s)));
    MOE_TRY(hip_status(launch_kgrouped_gemm(hsh, dysh, offsh, 1, Fs, H, sg->dw_down, s)));
  }
  return MOE_OK;
}

int moe_backward(const moe_bf16* x, const int32_t* topk_ids, const float* topk_w, int T, int H,
                 int F, int E, int k, const moe_bf16* w_gate, const moe_bf16* w_up,
                 const moe_bf16* w_down, const moe_bf16* dout, moe_bf16* dx, float* d_topk_w,
                 float* dw_gate, float* dw_up, float* dw_down, void* ws, size_t ws_bytes,
                 void* stream) {
  return backward_impl(x, topk_ids, topk_w, T, H, F, E, k, w_gate, w_up, w_down, nullptr,
                       nullptr, dout, dx, d_topk_w, dw_gate, dw_up, dw_down, ws, ws_bytes,
                       stream);
}

int moe_backward_shared(const moe_bf16* x, const int32_t* topk_ids, const float* topk_w, int T,
                        int H, int F, int E, int k, const moe_bf16* w_gate, const moe_bf16* w_up,
                        const moe_bf16* w_down, const moe_shared_expert* shared,
                        const moe_bf16* dout, moe_bf16* dx, float* d_topk_w, float* dw_gate,
                        float* dw_up, float* dw_down, moe_shared_expert_grads* shared_grads,
                        void* ws, size_t ws_bytes, void* stream) {
  return backward_impl(x, topk_ids, topk_w, T, H, F, E, k, w_gate, w_up, w_down, shared,
                       shared_grads, dout, dx, d_topk_w, dw_gate, dw_up, dw_down, ws, ws_bytes,
                       stream);
}

int moe_route_backward(const int32_t* topk_ids, const float* topk_w, const float* d_topk_w,
                       int T, int E, int k, float* d_logits, void* stream) {
  MOE_TRY(check_dims(T, E, k));
  MOE_TRY(check_elems(T, E));
  if (T == 0) return MOE_OK;
  MOE_TRY(need_word(topk_ids));
  MOE_TRY(need_word(topk_w));
  MOE_TRY(need_word(d_topk_w));
  MOE_TRY(need_word(d_logits));
  MOE_TRY(debug_check_ids(topk_ids, static_cast<int64_t>(T) * k, E, stream));
  return hip_status(moe::launch_route_backward(topk_ids, topk_w, d_topk_w, T, E, k, d_logits,
                                               static_cast<hipStream_t>(stream)));
}

}  // extern "C"
