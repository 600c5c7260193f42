// Library-owned scratch for tsv_decode_step_noalloc: one file-scope device
// array per GPU, so that callers which cannot allocate (graph capture, tight
// serving loops) need not pass a workspace.  In host code the array's name is
// only a stand-in for the symbol, never a device address: the address is
// looked up once per device with hipGetSymbolAddress and kept, and only that
// pointer is handed to kernels.
#include <mutex>

#include "tsv_launch.h"

namespace tsv {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

// Clears n 32-bit words (the split-row counters and key slots at the start of
// the workspace layout).
__global__ void k_clear_words(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_ptr[kMaxDevices];      // device address of `scratch` on each device
bool g_cleared[kMaxDevices];   // split-row prefix cleared on that device

}  // namespace

hipError_t noalloc_scratch(hipStream_t s, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  if (!g_cleared[dev]) {
    // the split-row prefix must start at zero; every step leaves it zero.  A
    // kernel rather than a memset, so that a first call under graph capture
    // records a node that replays correctly.
    const int words = (int)(kZeroBytes / sizeof(uint32_t));
    (void)hipGetLastError();  // the check below sees this launch only
    hipLaunchKernelGGL(k_clear_words, dim3((words + 255) / 256), dim3(256), 0, s,
                       static_cast<uint32_t*>(g_ptr[dev]), words);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    g_cleared[dev] = true;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace tsv
