// Persistent, block-scheduled grouped GEMM for the MoE expert layer (gfx950):
// the choice of tile class and K-split, the dispatch to the tile families,
// and the weight re-layouts (packing, fp8 and mxfp4 quantization). The
// kernels themselves are in grouped_gemm_kernel.h.
#include <atomic>

#include "grouped_gemm_kernel.h"

namespace moe {

// Tile class by typical rows per group: < 16 small, < 64 mid (gate/up only;
// the down projection keeps the small tile; bf16 weights take large128 from
// 24 rows on), < 192 large128, else large. A down projection from 96 rows
// per group on takes large128 only when its expected items (one partial row
// tile per touched group plus the full ones, times the column tiles) fill
// the two workgroups per CU that tile runs with; with few groups (e.g. 8
// experts of 128 rows and a long K) it keeps one 256-row tile per CU.
// set_dispatch_override (the library's testing hook) can force a class.
namespace {
// Dispatch overrides (-1: automatic), set only through the testing hook.
std::atomic<int> g_forced_tile{-1};
std::atomic<int> g_forced_rs{-1};
std::atomic<int> g_forced_scatter{-1};
}  // namespace

void set_dispatch_override(int decode_path, int tile_class) {
  g_forced_rs.store(decode_path, std::memory_order_relaxed);
  g_forced_tile.store(tile_class, std::memory_order_relaxed);
}

void set_scatter_override(int mode) { g_forced_scatter.store(mode, std::memory_order_relaxed); }

int tile_class(const GemmProblem& p) {
  const int forced = g_forced_tile.load(std::memory_order_relaxed);
  if (forced >= 0) return forced;
  const bool bf16 = p.seg[0].packed == 0 || p.seg[0].packed == 1;
  if (p.rows_hint < 16) return kSmall;
  // bf16 weights: from 24 rows per group on, the 128-row tiles stream the
  // weights faster than the mid tile (gate/up) and the small tile (down),
  // padding notwithstanding (the MFMAs are not the bound there): layer
  // 583 -> 531 us at the Mixtral-shaped T = 128, 4950 -> 4355 us at the
  // DeepSeek-V3-shaped T = 1024, 364 -> 310 us at the Qwen2-shaped T = 512;
  // at 16-17 rows the mid and small tiles were ahead (Mixtral-shaped T = 64:
  // 494 against 524 us)
  if (p.rows_hint < 64) return bf16 && p.rows_hint >= 24 ? kLarge128 : kMid;
  if (p.rows_hint >= 192) return kLarge;
  if (p.gated) return kLarge128;
  // bf16 down projections below 96 rows per group: the 256-row tile would
  // be three-quarters padding (Mixtral-shaped T = 256: layer 580 -> 544 us).
  // From 96 rows on, the 256-row tiles stay ahead inside the layer (fp32
  // K-slices): 128-row tiles there took the Mixtral-shaped layer at T = 512
  // (115-140 rows per expert) from 0.67 to 0.72 ms and the DeepSeek-V3-shaped
  // one at T = 4096 from 6.19 to 6.31 ms, although a lone bf16 down
  // projection without K-slices ran faster on them (318 -> 264 us at T = 512)
  if (bf16 && p.rows_hint < 96) return kLarge128;
  int64_t items = 0;
  for (int s = 0; s < p.nseg; ++s) {
    const GemmSegment& S = p.seg[s];
    const int64_t touched = S.ngroups > 1 ? (S.rows < S.ngroups ? S.rows : S.ngroups) : 1;
    items += (touched + S.rows / DownLarge128::BT) * ((S.N + DownLarge128::BF - 1) / DownLarge128::BF);
  }
  return items >= 2 * static_cast<int64_t>(device_cu_count()) ? kLarge128 : kLarge;
}

bool grouped_gemm_gathers(const GemmProblem& p) {
  const int tc = tile_class(p);
  return p.gated && (tc == kLarge || tc == kLarge128);
}

// The decode-size tiles of a plain fp32-output problem on the forward's
// weight layouts (their 16- or 32-row tiles carry the hand-over epilogue),
// when the testing hook asks for it. By default the layer combines in a
// launch of its own: against it, the hand-over measured equal at the
// Mixtral-shaped T = 1 (0.143 ms) and slower wherever a workgroup runs
// several items (Qwen2-shaped T = 16 0.166 -> 0.177 ms, DeepSeek-V3-shaped
// T = 128 2.64 -> 2.80 ms): each item waits for its device-scope stores, its
// counter atomics and its device-scope loads in turn, a few microseconds,
// about the whole combine launch it replaces. Ordinary stores with
// agent-scope fences instead (an L2 write-back and invalidation per item)
// made those layers 1.7-4x slower.
bool grouped_gemm_scatters(const GemmProblem& p) {
  if (g_forced_scatter.load(std::memory_order_relaxed) != 1) return false;
  if (p.gated || !p.out_f32 || p.seg[0].packed == kWeightsTransposed) return false;
  return tile_class(p) == kSmall;
}

void grouped_gemm_plan_ksplit(GemmProblem& p, int cus) {
  // Split K only where the unsplit item count cannot fill the chip: down
  // projections (fp32 partial outputs) with few touched experts or few
  // row tiles. A second segment (the shared expert) whose K is longer is
  // split further while its items are few, so that its items cost about as
  // many K-steps as the routed ones: the schedule gives every workgroup the
  // same number of items, so one long item would set the kernel's time.
  for (int s = 0; s < p.nseg; ++s) p.seg[s].ksplit = 1;
  if (p.gated || !p.out_f32) return;
  const int tc = tile_class(p);
  const int BT = tc == kLarge ? DownLarge::BT : tc == kLarge128 ? DownLarge128::BT : DownSmall::BT;
  const int BF = tc == kLarge ? DownLarge::BF : tc == kLarge128 ? DownLarge128::BF : DownSmall::BF;
  const int BK = tc == kLarge ? DownLarge::BK : tc == kLarge128 ? DownLarge128::BK : DownSmall::BK;
  int64_t items = 0;
  int min_k = 1 << 30;
  for (int s = 0; s < p.nseg; ++s) {
    const GemmSegment& S = p.seg[s];
    // expected row tiles: one partial tile per touched group plus full ones
    const int64_t touched = S.ngroups > 1 ? (S.rows < S.ngroups ? S.rows : S.ngroups) : 1;
    const int64_t mt = touched + S.rows / BT;
    items += mt * ((S.N + BF - 1) / BF);
    min_k = S.K < min_k ? S.K : min_k;
  }
  const int64_t want = 2 * static_cast<int64_t>(cus);
  int split = 1;
  while (split < kMaxKSplit && items * split * 2 <= want && min_k / (split * 2) >= 256 &&
         min_k / (split * 2) >= 4 * BK)
    split *= 2;
  for (int s = 0; s < p.nseg; ++s) p.seg[s].ksplit = split;
  if (p.nseg > 1) {
    const GemmSegment& S1 = p.seg[1];
    const int steps0 = ((p.seg[0].K + BK - 1) / BK + split - 1) / split;  // per routed item
    const int nk1 = (S1.K + BK - 1) / BK;
    const int64_t items1 = static_cast<int64_t>((S1.rows + BT - 1) / BT) * ((S1.N + BF - 1) / BF);
    int ks1 = (nk1 + steps0 / 2) / steps0;
    ks1 = ks1 < 1 ? 1 : (ks1 > kMaxKSplit ? kMaxKSplit : ks1);
    if (ks1 > split && items1 < want && nk1 / ks1 >= 4) p.seg[1].ksplit = ks1;
  }
}

int grouped_gemm_device_cus() { return device_cu_count(); }

namespace {

// Packed weights: one thread per 16-byte chunk of the packed tensor, in
// order (block, 32-row half, column, physical chunk p); the chunk holds the
// column's 8 K-consecutive values 8q..8q+7 of the half, q = p ^ ((c >> 1) & 3)
// (the GEMM's LDS swizzle), or zeros past K or N.
__global__ __launch_bounds__(256) void pack_weights_kernel(
    const bf16_t* __restrict__ w, int K, int N, int nblk, int kblk, int64_t chunks,
    bf16_t* __restrict__ out) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= chunks) return;
  const int pc = static_cast<int>(idx & 3);
  const int c = static_cast<int>((idx >> 2) & 63);
  const int h = static_cast<int>((idx >> 8) & 1);
  int64_t blk = idx >> 9;
  const int kb = static_cast<int>(blk % kblk);
  blk /= kblk;
  const int nb = static_cast<int>(blk % nblk);
  const int64_t g = blk / nblk;
  const int k0 = kb * 64 + h * 32 + (pc ^ ((c >> 1) & 3)) * 8;
  const int n = nb * 64 + c;
  uint32_t v[4] = {0u, 0u, 0u, 0u};
  if (k0 < K && n < N) {  // K is a multiple of 8: all 8 rows are inside K
    const bf16_t* src = w + (g * K + k0) * N + n;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      v[e] = static_cast<uint32_t>(src[(2 * e) * static_cast<int64_t>(N)]) |
             (static_cast<uint32_t>(src[(2 * e + 1) * static_cast<int64_t>(N)]) << 16);
  }
  reinterpret_cast<uint4*>(out)[idx] = uint4{v[0], v[1], v[2], v[3]};
}

// FP8 quantization, step 1: per (g, n) the column's largest |w| over K and
// its scale 2^e, e the smallest integer with that max <= 448 * 2^e (1 for a
// zero column). With max = f * 2^E (frexp, f in [0.5, 1)) and 448 =
// 0.875 * 2^9: e = E - 9 when f <= 0.875, else E - 8 (exact; bf16
// magnitudes order like their bit patterns).
__global__ __launch_bounds__(256) void fp8_scales_kernel(const bf16_t* __restrict__ w, int G,
                                                         int K, int N,
                                                         float* __restrict__ scales) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= static_cast<int64_t>(G) * N) return;
  const int64_t g = idx / N;
  const int n = static_cast<int>(idx % N);
  const bf16_t* p = w + g * K * N + n;
  uint32_t amax = 0;
  for (int k = 0; k < K; ++k) {
    const uint32_t m = p[static_cast<int64_t>(k) * N] & 0x7fffu;
    amax = m > amax ? m : amax;
  }
  float sc = 1.f;
  if (amax != 0) {
    int E;
    const float f = frexpf(__uint_as_float(amax << 16), &E);
    sc = ldexpf(1.f, f <= 0.875f ? E - 9 : E - 8);
  }
  scales[idx] = sc;
}

// E4M3 code of v (|v| <= 448): round to nearest, ties to even, on the code
// grid. Below 2^-6 the grid is m * 2^-9 (m = 8 is the least normal code);
// above, 8 mantissa steps per power of two (a rounding up to the next power
// carries into the exponent field). The sign is v's (also for zeros).
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fminf(fabsf(v), 448.0f);  // saturate (only MXFP8 blocks reach past 448)
  uint32_t code;
  if (a < 0.015625f) {
    code = static_cast<uint32_t>(rintf(a * 512.0f));
  } else {
    const int E = static_cast<int>((__float_as_uint(a) >> 23) & 0xffu) - 127;
    code = static_cast<uint32_t>((E + 7) << 3) +
           static_cast<uint32_t>(rintf((ldexpf(a, -E) - 1.0f) * 8.0f));
  }
  return sign | code;
}

// FP8 quantization, step 2: one thread per 8-byte chunk of the block layout
// (physical chunk p of column c in half h of block (g, nb, kb)); the chunk
// holds rows 8q..8q+7, q = p ^ ((c >> 2) & 3), of that column, each weight
// divided by its column's scale (exact: a power of two) and encoded.
__global__ __launch_bounds__(256) void fp8_encode_kernel(
    const bf16_t* __restrict__ w, int K, int N, int nblk, int kblk, int64_t chunks,
    const float* __restrict__ scales, uint8_t* __restrict__ out) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= chunks) return;
  const int p = static_cast<int>(idx & 3);
  const int c = static_cast<int>((idx >> 2) & 63);
  const int h = static_cast<int>((idx >> 8) & 1);
  int64_t blk = idx >> 9;
  const int kb = static_cast<int>(blk % kblk);
  blk /= kblk;
  const int nb = static_cast<int>(blk % nblk);
  const int64_t g = blk / nblk;
  const int q = p ^ ((c >> 2) & 3);
  const int n = nb * 64 + c;
  const int k0 = kb * 64 + h * 32 + q * 8;
  uint32_t lo = 0, hi = 0;
  if (n < N) {
    int e;
    frexpf(scales[g * N + n], &e);  // scale = 2^(e-1)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k = k0 + j;
      uint32_t code = 0;
      if (k < K) {
        const float x = __uint_as_float(static_cast<uint32_t>(w[(g * K + k) * N + n]) << 16);
        code = e4m3_encode(ldexpf(x, 1 - e));
      }
      if (j < 4) lo |= code << (8 * j);
      else hi |= code << (8 * (j - 4));
    }
  }
  reinterpret_cast<uint2*>(out)[idx] = uint2{lo, hi};
}

// MXFP4 quantization, step 1: one thread per scale byte of the padded
// layout [G][nblk][skb][64]: for column n and K-block b (K-values 32b ..
// 32b+31 inside K) the largest |w| (bf16 magnitudes order like their bit
// patterns); X = floor(log2 amax) - 2 = exponent field - 129 for a normal
// amax, raised to -125 (also for a subnormal amax), 0 for an all-zero block
// and past K or N; the byte is X + 127.
__global__ __launch_bounds__(256) void mxfp4_scales_kernel(const bf16_t* __restrict__ w, int K,
                                                           int N, int nblk, int skb,
                                                           int64_t total,
                                                           uint8_t* __restrict__ out) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= total) return;
  const int c = static_cast<int>(idx & 63);
  int64_t rest = idx >> 6;
  const int b = static_cast<int>(rest % skb);
  rest /= skb;
  const int nb = static_cast<int>(rest % nblk);
  const int64_t g = rest / nblk;
  const int n = nb * 64 + c;
  int X = 0;
  if (n < N && 32 * b < K) {
    const bf16_t* p = w + (g * K + 32 * b) * N + n;
    const int rows = min(32, K - 32 * b);
    uint32_t amax = 0;
    for (int k = 0; k < rows; ++k) {
      const uint32_t m = p[static_cast<int64_t>(k) * N] & 0x7fffu;
      amax = m > amax ? m : amax;
    }
    if (amax != 0) {
      const int e = static_cast<int>(amax >> 7);
      X = e == 0 ? -125 : max(e - 129, -125);
    }
  }
  out[idx] = static_cast<uint8_t>(X + 127);
}

// E2M1 code of v (v = w / 2^X, |v| < 8): round to nearest on the grid 0,
// 0.5, 1, 1.5, 2, 3, 4, 6, a tie going to the code with mantissa bit 0,
// magnitudes above 6 saturating to 6; the sign is v's (also for zeros).
__device__ __forceinline__ uint32_t e2m1_encode(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 28) & 8u;
  const float a = fabsf(v);
  const uint32_t m = a <= 0.25f ? 0u : a < 0.75f ? 1u : a <= 1.25f ? 2u : a < 1.75f ? 3u
                     : a <= 2.5f ? 4u : a < 3.5f ? 5u : a <= 5.0f ? 6u : 7u;
  return sign | m;
}

// MXFP4 quantization, step 2: one thread per dword of the code blocks
// (dword q of column c in half h of block (g, nb, kb)): the codes of rows
// kb*64 + h*32 + 8q + i, i = 0..7, nibble i (low nibble first), each weight
// divided by its K-block's scale (exact: a power of two) and encoded.
__global__ __launch_bounds__(256) void mxfp4_encode_kernel(
    const bf16_t* __restrict__ w, int K, int N, int nblk, int kblk, int skb, int64_t words,
    const uint8_t* __restrict__ scales, uint32_t* __restrict__ out) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= words) return;
  const int q = static_cast<int>(idx & 3);
  const int c = static_cast<int>((idx >> 2) & 63);
  const int h = static_cast<int>((idx >> 8) & 1);
  int64_t blk = idx >> 9;
  const int kb = static_cast<int>(blk % kblk);
  blk /= kblk;
  const int nb = static_cast<int>(blk % nblk);
  const int64_t g = blk / nblk;
  const int n = nb * 64 + c;
  const int k0 = kb * 64 + h * 32 + q * 8;
  uint32_t word = 0;
  if (n < N && k0 < K) {  // K is a multiple of 8: all 8 rows are inside K
    const int X = static_cast<int>(scales[((g * nblk + nb) * skb + k0 / 32) * 64 + c]) - 127;
    const bf16_t* p = w + (g * K + k0) * N + n;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float x = __uint_as_float(static_cast<uint32_t>(p[static_cast<int64_t>(i) * N]) << 16);
      word |= e2m1_encode(ldexpf(x, -X)) << (4 * i);
    }
  }
  out[idx] = word;
}

// MXFP8 quantization, step 1: one thread per scale byte of the padded layout
// [G][nblk][skb][64]: for column n and K-block b the largest |w| (bf16
// magnitudes order like their bit patterns); X = floor(log2 amax) - 8 =
// exponent field - 135 for a normal amax, raised to -117 (also for a
// subnormal amax), 0 for an all-zero block and past K or N; the byte is
// X + 127.
__global__ __launch_bounds__(256) void mxfp8_scales_kernel(const bf16_t* __restrict__ w, int K,
                                                           int N, int nblk, int skb,
                                                           int64_t total,
                                                           uint8_t* __restrict__ out) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= total) return;
  const int c = static_cast<int>(idx & 63);
  int64_t rest = idx >> 6;
  const int b = static_cast<int>(rest % skb);
  rest /= skb;
  const int nb = static_cast<int>(rest % nblk);
  const int64_t g = rest / nblk;
  const int n = nb * 64 + c;
  int X = 0;
  if (n < N && 32 * b < K) {
    const bf16_t* p = w + (g * K + 32 * b) * N + n;
    const int rows = min(32, K - 32 * b);
    uint32_t amax = 0;
    for (int k = 0; k < rows; ++k) {
      const uint32_t m = p[static_cast<int64_t>(k) * N] & 0x7fffu;
      amax = m > amax ? m : amax;
    }
    if (amax != 0) {
      const int e = static_cast<int>(amax >> 7);
      X = e == 0 ? -117 : max(e - 135, -117);
    }
  }
  out[idx] = static_cast<uint8_t>(X + 127);
}

// MXFP8 quantization, step 2: one thread per 8-byte chunk of the fp8 block
// layout (physical chunk p of column c in half h of block (g, nb, kb), rows
// 8q..8q+7, q = p ^ ((c >> 2) & 3)), each weight divided by its K-block's
// scale (exact: a power of two) and encoded, saturating at 448, with the
// weight's own sign.
__global__ __launch_bounds__(256) void mxfp8_encode_kernel(
    const bf16_t* __restrict__ w, int K, int N, int nblk, int kblk, int skb, int64_t chunks,
    const uint8_t* __restrict__ scales, uint8_t* __restrict__ out) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= chunks) return;
  const int p = static_cast<int>(idx & 3);
  const int c = static_cast<int>((idx >> 2) & 63);
  const int h = static_cast<int>((idx >> 8) & 1);
  int64_t blk = idx >> 9;
  const int kb = static_cast<int>(blk % kblk);
  blk /= kblk;
  const int nb = static_cast<int>(blk % nblk);
  const int64_t g = blk / nblk;
  const int q = p ^ ((c >> 2) & 3);
  const int n = nb * 64 + c;
  const int k0 = kb * 64 + h * 32 + q * 8;
  uint32_t lo = 0, hi = 0;
  if (n < N && k0 < K) {  // K is a multiple of 8: all 8 rows are inside K
    const int X = static_cast<int>(scales[((g * nblk + nb) * skb + k0 / 32) * 64 + c]) - 127;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t bits = static_cast<uint32_t>(w[(g * K + k0 + j) * N + n]);
      const float x = __uint_as_float(bits << 16);
      const uint32_t code = (e4m3_encode(ldexpf(fabsf(x), -X)) & 0x7fu) | ((bits >> 8) & 0x80u);
      if (j < 4) lo |= code << (8 * j);
      else hi |= code << (8 * (j - 4));
    }
  }
  reinterpret_cast<uint2*>(out)[idx] = uint2{lo, hi};
}

}  // namespace

hipError_t launch_quantize_mxfp8(const bf16_t* w, int G, int K, int N, uint8_t* codes,
                                 uint8_t* scales, hipStream_t stream) {
  const int nblk = (N + 63) / 64, kblk = (K + 63) / 64, skb = mx_scale_kblocks(K);
  const int64_t total = mxfp4_scale_bytes(G, K, N);
  if (total == 0) return hipSuccess;
  MOE_TRACE_LAUNCH("mxfp8_scales_kernel",
                   dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0,
                   "G=%d K=%d N=%d", G, K, N);
  hipLaunchKernelGGL(mxfp8_scales_kernel, dim3(static_cast<unsigned>((total + 255) / 256)),
                     dim3(256), 0, stream, w, K, N, nblk, skb, total, scales);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t chunks = fp8_weight_bytes(G, K, N) / 8;
  MOE_TRACE_LAUNCH("mxfp8_encode_kernel",
                   dim3(static_cast<unsigned>((chunks + 255) / 256)), dim3(256), 0,
                   "G=%d K=%d N=%d", G, K, N);
  hipLaunchKernelGGL(mxfp8_encode_kernel, dim3(static_cast<unsigned>((chunks + 255) / 256)),
                     dim3(256), 0, stream, w, K, N, nblk, kblk, skb, chunks, scales, codes);
  return hipGetLastError();
}

int64_t mxfp4_weight_bytes(int G, int K, int N) {
  return static_cast<int64_t>(G) * ((N + 63) / 64) * ((K + 63) / 64) * 2048;
}

int64_t mxfp4_scale_bytes(int G, int K, int N) {
  return static_cast<int64_t>(G) * ((N + 63) / 64) * mx_scale_kblocks(K) * 64;
}

hipError_t launch_quantize_mxfp4(const bf16_t* w, int G, int K, int N, uint8_t* codes,
                                 uint8_t* scales, hipStream_t stream) {
  const int nblk = (N + 63) / 64, kblk = (K + 63) / 64, skb = mx_scale_kblocks(K);
  const int64_t total = mxfp4_scale_bytes(G, K, N);
  if (total == 0) return hipSuccess;
  MOE_TRACE_LAUNCH("mxfp4_scales_kernel",
                   dim3(static_cast<unsigned>((total + 255) / 256)), dim3(256), 0,
                   "G=%d K=%d N=%d", G, K, N);
  hipLaunchKernelGGL(mxfp4_scales_kernel, dim3(static_cast<unsigned>((total + 255) / 256)),
                     dim3(256), 0, stream, w, K, N, nblk, skb, total, scales);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t words = mxfp4_weight_bytes(G, K, N) / 4;
  MOE_TRACE_LAUNCH("mxfp4_encode_kernel",
                   dim3(static_cast<unsigned>((words + 255) / 256)), dim3(256), 0,
                   "G=%d K=%d N=%d", G, K, N);
  hipLaunchKernelGGL(mxfp4_encode_kernel, dim3(static_cast<unsigned>((words + 255) / 256)),
                     dim3(256), 0, stream, w, K, N, nblk, kblk, skb, words, scales,
                     reinterpret_cast<uint32_t*>(codes));
  return hipGetLastError();
}

int64_t fp8_weight_bytes(int G, int K, int N) {
  return static_cast<int64_t>(G) * ((N + 63) / 64) * ((K + 63) / 64) * 4096;
}

hipError_t launch_quantize_fp8(const bf16_t* w, int G, int K, int N, uint8_t* codes,
                               float* scales, hipStream_t stream) {
  const int64_t cols = static_cast<int64_t>(G) * N;
  if (cols == 0) return hipSuccess;
  MOE_TRACE_LAUNCH("fp8_scales_kernel",
                   dim3(static_cast<unsigned>((cols + 255) / 256)), dim3(256), 0,
                   "G=%d K=%d N=%d", G, K, N);
  hipLaunchKernelGGL(fp8_scales_kernel, dim3(static_cast<unsigned>((cols + 255) / 256)),
                     dim3(256), 0, stream, w, G, K, N, scales);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t chunks = fp8_weight_bytes(G, K, N) / 8;
  MOE_TRACE_LAUNCH("fp8_encode_kernel",
                   dim3(static_cast<unsigned>((chunks + 255) / 256)), dim3(256), 0,
                   "G=%d K=%d N=%d", G, K, N);
  hipLaunchKernelGGL(fp8_encode_kernel, dim3(static_cast<unsigned>((chunks + 255) / 256)),
                     dim3(256), 0, stream, w, K, N, (N + 63) / 64, (K + 63) / 64, chunks, scales,
                     codes);
  return hipGetLastError();
}

int64_t packed_weight_elems(int G, int K, int N) {
  return static_cast<int64_t>(G) * ((N + 63) / 64) * ((K + 63) / 64) * 4096;
}

hipError_t launch_pack_weights(const bf16_t* w, int G, int K, int N, bf16_t* packed,
                               hipStream_t stream) {
  const int64_t chunks = packed_weight_elems(G, K, N) / 8;
  if (chunks == 0) return hipSuccess;
  MOE_TRACE_LAUNCH("pack_weights_kernel",
                   dim3(static_cast<unsigned>((chunks + 255) / 256)), dim3(256), 0,
                   "G=%d K=%d N=%d", G, K, N);
  hipLaunchKernelGGL(pack_weights_kernel, dim3(static_cast<unsigned>((chunks + 255) / 256)),
                     dim3(256), 0, stream, w, K, N, (N + 63) / 64, (K + 63) / 64, chunks,
                     packed);
  return hipGetLastError();
}

// The register-streaming gate/up serves packed bf16 or fp8 weights of
// small groups when both segments share K, nothing but h is written, and
// the expected items (one partial row tile per touched group plus the full
// ones, times the column tiles) are at most 16 (bf16) or 8 (fp8) per CU.
// Measured against the LDS-ring tiles: bf16 7-8 % faster at 1 and 2 items
// per workgroup slot (Mixtral-shaped T = 1, Qwen2-shaped T = 16), 2-4 % at
// 4 (Mixtral-shaped T = 32), 3-7 % slower at 11 (DeepSeek-V3-shaped
// T = 128), where the ring's shared activation tile and longer streams
// win; fp8 22 % faster at T = 1 and 19 % at Qwen2-shaped T = 16, but 13 %
// slower at Mixtral-shaped T = 32. On mxfp4 codes (one scale byte per 32
// K-values of a column to load beside them) it was slower everywhere.
// The testing hook's decode_path 0 / 1 forces it off / on (for comparisons).
bool use_rs_gateup(const GemmProblem& p) {
  const int forced = g_forced_rs.load(std::memory_order_relaxed);
  if (forced == 0) return false;
  if (p.epi != kEpiDefault) return false;
  int64_t items = 0;
  for (int s = 0; s < p.nseg; ++s) {
    const GemmSegment& S = p.seg[s];
    if (S.packed < 1 || S.packed > 2 || S.packed != p.seg[0].packed || S.gather ||
        S.ksplit != 1 || S.K != p.seg[0].K || S.K < 8)
      return false;
    if (S.packed == 2 && S.N < 16) return false;   // a wave reads 16 columns' scales
    const int64_t touched = S.ngroups > 1 ? (S.rows < S.ngroups ? S.rows : S.ngroups) : 1;
    items += (touched + S.rows / kRsBT) * ((S.N + kRsBF - 1) / kRsBF);
  }
  // fp8 codes: the column scales make each item's epilogue wait for the
  // weight stream in flight, so the bound is tighter
  const int per_cu = p.seg[0].packed == 2 ? 8 : 16;
  return forced == 1 || items <= per_cu * static_cast<int64_t>(device_cu_count());
}

hipError_t launch_grouped_gemm(const GemmProblem& p, hipStream_t stream) {
  for (int s = 0; s < p.nseg; ++s)  // a row map needs the rows it may name
    if (p.seg[s].gather && p.seg[s].gather_rows < 1) return hipErrorInvalidValue;
  // the backward epilogue exists in the transposed-weight bf16 kernels only
  if (p.epi == kSwigluBwd &&
      (p.gated || p.out_f32 || p.seg[0].packed != kWeightsTransposed || p.nseg != 1))
    return hipErrorInvalidValue;
  // the hand-over epilogue exists in the decode-size fp32 tiles only
  if (p.scat.cnt && (!grouped_gemm_scatters(p) || p.scat.T < 1 || p.scat.k < 1 ||
                     p.scat.target < 1 || !p.scat.out || !p.scat.y || !p.scat.row_token ||
                     !p.scat.row_dest || p.scat.y_slices < 1 || p.scat.ysh_slices < 1 ||
                     (p.nseg > 1 && p.seg[1].N != p.seg[0].N)))
    return hipErrorInvalidValue;
  const int tc = tile_class(p);
  if (p.gated && tc == kSmall && use_rs_gateup(p)) return launch_rs(p, stream);
  if (p.seg[0].packed == 3) return launch_mxfp4(p, tc, stream);
  if (p.seg[0].packed == 5) return launch_mxfp8(p, tc, stream);
  if (p.seg[0].packed == 2) return launch_fp8(p, tc, stream);
  if (p.gated) return launch_bf16_gated(p, tc, stream);
  if (p.out_f32) return launch_bf16_plain_f32(p, tc, stream);
  return launch_bf16_plain_bf16(p, tc, stream);
}

}  // namespace moe
