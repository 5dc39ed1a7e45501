// Scratch memory of the allocation-free decode entry point
// (pa_decode_noalloc): one file-scope device array, which every GPU the
// library runs on holds at its own address until the process ends.  Host
// code never uses the array's name as an address (on the host it is only a
// stand-in for the symbol): the first call on a device looks the address up
// with hipGetSymbolAddress, with that device current, and keeps it per
// device.
#include <atomic>

#include "pa_internal.h"

static __device__ __align__(256) unsigned char scratch[pa::kScratchBytes];

namespace pa {

namespace {

constexpr int kScratchDevs = 64;
std::atomic<void*> g_scratch[kScratchDevs];

__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

}  // namespace

void* scratch_address(hipStream_t stream) {
  const int dev = stream_device(stream);
  if (dev < 0 || dev >= kScratchDevs) return nullptr;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return nullptr;
  if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
  void* q = nullptr;
  const hipError_t e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
  if (cur != dev && hipSetDevice(cur) != hipSuccess) return nullptr;
  if (e != hipSuccess || q == nullptr) return nullptr;
  // concurrent first calls on one device store the same address
  g_scratch[dev].store(q, std::memory_order_release);
  return q;
}

hipError_t launch_zero_words(void* p, int64_t words, hipStream_t stream) {
  if (words <= 0) return hipSuccess;
  const int64_t blocks = (words + 255) / 256;
  hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)(blocks < 1024 ? blocks : 1024)),
                     dim3(256), 0, stream, static_cast<uint32_t*>(p), words);
  return hipGetLastError();
}

}  // namespace pa
