// static_scratch.hip -- the library's own device scratch, for callers that
// cannot allocate device memory (code under HIP graph capture, serving loops
// that forbid allocation): ld_decode_step_noalloc runs the decode step with its
// per-pass scratch (activations, attention and split-K partials, tickets,
// arg-max partials, token staging) in this file-scope array instead of the
// caller's arena.
//
// Each GPU the library runs on holds its own copy of `scratch` for the life of
// the process, at its own device address.  In host code the array's name only
// stands for the symbol: the address kernels may use is resolved per device with
// hipGetSymbolAddress (static_scratch_setup) and kept in g_ptr.  Every caller on
// a GPU shares that GPU's copy: calls that overlap on one GPU (two streams, two
// threads) race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "ld_internal.hpp"

namespace ld {

namespace {

static __device__ __align__(256) char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
char* g_ptr[kMaxDevices] = {};

__global__ void k_zero_words(int* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

}  // namespace

hipError_t static_scratch_setup(int device, hipStream_t s) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[device] != nullptr) return hipSuccess;
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  if (cur != device) return hipErrorInvalidDevice;
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (p == nullptr) return hipErrorInvalidSymbol;
  // the tickets at the front start at zero; the kernels re-arm them after every use
  constexpr int n = kScratchTicketBytes / 4;
  hipLaunchKernelGGL(k_zero_words, dim3((n + 255) / 256), dim3(256), 0, s, static_cast<int*>(p), n);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return e;
  g_ptr[device] = static_cast<char*>(p);
  return hipSuccess;
}

char* static_scratch(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  return g_ptr[device];
}

}  // namespace ld
