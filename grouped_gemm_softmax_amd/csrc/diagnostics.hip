// Diagnostics of the library: a launch trace and the debug check of
// caller-given expert ids.
//
// Trace: with MOE_TRACE=1 in the environment when the library is first used
// (or after moe_set_diagnostics(1, ...)), every kernel launch writes one line
// to stderr: the kernel, its grid, block and dynamic LDS, and the launch's
// own parameters (for the grouped GEMMs the tile shape, ring depth and
// schedule, the groups and the item bound).
//
// Id check: with MOE_DEBUG=1 (or moe_set_diagnostics(..., 1)) the calls that
// take expert ids from the caller (moe_permute, moe_forward_routed,
// moe_backward, moe_route_backward) first count the ids outside [0, E) on
// the GPU, wait for the count and return MOE_ERR_BAD_IDS, with nothing more
// enqueued, if it is not zero. The count lives in a device integer of the
// library (one per GPU), so the check allocates nothing.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include <atomic>
#include <mutex>

#include "kernels.h"

// Per-GPU counter of the id check (its device address is looked up once per
// device with hipGetSymbolAddress; host code never uses the name itself as
// an address).
static __device__ __align__(256) int id_check_count;

namespace moe {
namespace {

// -1: not yet read from the environment
std::atomic<int> g_trace{-1};
std::atomic<int> g_check{-1};

int from_env(const char* name) {
  const char* v = getenv(name);
  return (v && v[0] && !(v[0] == '0' && v[1] == 0)) ? 1 : 0;
}

int setting(std::atomic<int>& s, const char* env) {
  int v = s.load(std::memory_order_relaxed);
  if (v < 0) {
    v = from_env(env);
    int expected = -1;
    if (!s.compare_exchange_strong(expected, v)) v = expected;
  }
  return v;
}

constexpr int kMaxDevices = 64;
std::mutex g_count_mu;
int* g_count_ptr[kMaxDevices] = {};

hipError_t count_address(int** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_count_mu);
  if (!g_count_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(id_check_count));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_count_ptr[dev] = static_cast<int*>(p);
  }
  *ptr = g_count_ptr[dev];
  return hipSuccess;
}

constexpr int kCheckThreads = 256;

// Counts the ids outside [0, E): a grid-stride pass, one wave-wide sum per
// wave and one (vector-memory) atomic add per wave that found any.
__global__ __launch_bounds__(kCheckThreads) void check_ids_kernel(const int32_t* ids, int64_t n,
                                                                 int E, int* count) {
  int bad = 0;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kCheckThreads + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * kCheckThreads) {
    const int32_t id = ids[i];
    bad += (id < 0 || id >= E) ? 1 : 0;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) bad += __shfl_xor(bad, m, 64);
  if ((threadIdx.x & 63) == 0 && bad > 0) atomicAdd(count, bad);
}

}  // namespace

bool trace_enabled() { return setting(g_trace, "MOE_TRACE") != 0; }
bool check_ids_enabled() { return setting(g_check, "MOE_DEBUG") != 0; }

void set_diagnostics(int trace, int check_ids) {
  g_trace.store(trace < 0 ? from_env("MOE_TRACE") : trace);
  g_check.store(check_ids < 0 ? from_env("MOE_DEBUG") : check_ids);
}

void trace_launch(const char* kernel, dim3 grid, dim3 block, size_t lds, const char* fmt, ...) {
  char extra[256];
  extra[0] = 0;
  if (fmt) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(extra, sizeof(extra), fmt, ap);
    va_end(ap);
  }
  fprintf(stderr, "moe: launch %s grid=%ux%u block=%u lds=%zu%s%s\n", kernel, grid.x, grid.y,
          block.x, lds, extra[0] ? " " : "", extra);
}

hipError_t count_bad_ids(const int32_t* ids, int64_t n, int E, hipStream_t stream, int* bad) {
  *bad = 0;
  if (n <= 0) return hipSuccess;
  int* count = nullptr;
  hipError_t e = count_address(&count);
  if (e != hipSuccess) return e;
  // this path synchronises the stream, so it is never part of a captured
  // graph: a plain memset may clear the counter
  e = hipMemsetAsync(count, 0, sizeof(int), stream);
  if (e != hipSuccess) return e;
  const int64_t blocks64 = (n + kCheckThreads - 1) / kCheckThreads;
  const unsigned blocks = static_cast<unsigned>(blocks64 < 1024 ? blocks64 : 1024);
  MOE_TRACE_LAUNCH("check_ids_kernel", dim3(blocks), dim3(kCheckThreads), 0, "n=%lld E=%d",
                   static_cast<long long>(n), E);
  hipLaunchKernelGGL(check_ids_kernel, dim3(blocks), dim3(kCheckThreads), 0, stream, ids, n, E,
                     count);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  int h = 0;
  e = hipMemcpyAsync(&h, count, sizeof(int), hipMemcpyDeviceToHost, stream);
  if (e != hipSuccess) return e;
  e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return e;
  *bad = h;
  return hipSuccess;
}

}  // namespace moe
