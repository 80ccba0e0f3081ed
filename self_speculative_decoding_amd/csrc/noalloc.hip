// Allocation-free accept: the greedy accept kernel run on host drafts and
// predictions with no context, for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).  Its staging (the block and the predictions), the counters the
// kernel advances and its outputs live in one static device array per GPU.
#include <hip/hip_runtime.h>

#include <mutex>

#include "host.h"
#include "kernels.h"

using namespace ssd;

namespace {

// Ints of the scratch array: block [t_last, d_1..d_k], predictions p_0..p_k,
// result [a, a + 1, emitted a + 1 tokens], then the two counters the kernel
// advances (committed length, emitted count; read back with the result), then
// the emitted-token log.
constexpr int kOffBlock = 0, kOffPost = 32, kOffResult = 64, kOffState = 112, kOffLog = 128;
constexpr int kScratchInts = SSD_NOALLOC_SCRATCH_BYTES / 4;
static_assert(kOffLog + SSD_MAX_BLOCK <= kScratchInts, "scratch layout");
static_assert(kOffResult + 2 + SSD_MAX_BLOCK <= kOffState, "scratch layout");

// Each GPU the library runs on holds its own copy until the process ends.  In
// host code this name is not a device address: the address comes from
// hipGetSymbolAddress (scratch_ptr below).
static __device__ __align__(256) int scratch[kScratchInts];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
int* g_ptr[kMaxDevices] = {};

// This device's address of `scratch`, looked up once per device with that
// device current (the caller's current device).
ssd_status scratch_ptr(int** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SSD_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(SSD_E_UNSUPPORTED, "device %d beyond the %d supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return fail(SSD_E_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_ptr[dev] = (int*)p;
  }
  *out = g_ptr[dev];
  return SSD_OK;
}

// The inputs travel in the kernel arguments, so staging needs no copy.
struct AcceptStage {
  int d[SSD_MAX_BLOCK];   // d_1..d_k at [0, k)
  int p[SSD_MAX_BLOCK];   // p_0..p_k at [0, k]
  int k;
};

// Writes the block (t_last slot -1), the predictions and zero counters.  The
// array keeps the previous call's contents, so every entry the accept kernel
// reads is written here.
__global__ __launch_bounds__(64) void stage_accept_kernel(AcceptStage in, int* s) {
  const int t = threadIdx.x;
  if (t < SSD_MAX_BLOCK) {
    s[kOffBlock + t] = t == 0 ? -1 : (t - 1 < in.k ? in.d[t - 1] : 0);
    s[kOffPost + t] = t <= in.k ? in.p[t] : 0;
  }
  if (t < 16) s[kOffState + t] = 0;
}

}  // namespace

extern "C" ssd_status ssd_test_accept_noalloc(const int32_t* d, const int32_t* p, int32_t k, void* hip_stream,
                                              int32_t* a) {
  clear_error();
  if (!p || !a || (k > 0 && !d)) return fail(SSD_E_ARG, "NULL argument");
  if (k < 0 || k + 1 > SSD_MAX_BLOCK) return fail(SSD_E_ARG, "k=%d outside [0, %d]", k, SSD_MAX_BLOCK - 1);
  int* s = nullptr;
  ssd_status st = scratch_ptr(&s);
  if (st != SSD_OK) return st;
  hipStream_t stream = (hipStream_t)hip_stream;
  AcceptStage in{};
  for (int i = 0; i < k; ++i) in.d[i] = d[i];
  for (int i = 0; i <= k; ++i) in.p[i] = p[i];
  in.k = k;
  stage_accept_kernel<<<1, 64, 0, stream>>>(in, s);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = launch_accept(s + kOffBlock, s + kOffPost, k, s + kOffState, s + kOffLog, s + kOffResult, stream);
  // result [a, a + 1, tokens] and the two counters, in one copy
  int h[kOffState + 2 - kOffResult];
  if (e == hipSuccess) e = hipMemcpyAsync(h, s + kOffResult, sizeof h, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(SSD_E_HIP, "accept (no-alloc): %s", hipGetErrorString(e));
  const int na = h[0], ne = h[1], s0 = h[kOffState - kOffResult], s1 = h[kOffState + 1 - kOffResult];
  if (na < 0 || na > k || ne != na + 1 || s0 != ne || s1 != ne)
    return fail(SSD_E_HIP, "accept kernel produced inconsistent counters");
  *a = na;
  return SSD_OK;
}
