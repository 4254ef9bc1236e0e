// ekv_decode_step without a caller workspace: the step's scratch (arrival
// counters, per-head page bounds, z_max lower bounds, the decode's candidate
// lists) lives in a fixed-size device array of this library, for callers that
// cannot allocate device memory (code under stream capture, serving loops
// that forbid allocation, harnesses that own all memory).
//
// Each GPU the library runs on holds its own copy of `scratch` until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in symbol): the first call on a device looks up
// that device's address with hipGetSymbolAddress, with the device current,
// and every later call on it uses that address.  The arrival counters at the
// start of the array must be zero before a step; device globals start
// zero-filled, the first call on a device clears them once more with a fill
// kernel on the caller's stream, and every completed step leaves them zero.
// All calls on one GPU share its array: calls that overlap in time on one GPU
// (different streams, or host threads without ordering) race on it.
#include <mutex>

#include "entmaxkv.h"
#include "kernels.h"

namespace {

// the array: arrival counters in a region of their own (one int per (row,
// KV head) pair, never used for anything else, so they stay zero between
// calls whatever shapes the calls use), then the rest of the step's scratch
constexpr size_t kScratchBytes = 64ull << 20;
constexpr size_t kCounterRegion = 64ull << 10;  // 16384 pairs
constexpr int kMaxDevices = 64;
static_assert(kScratchBytes == EKV_NOALLOC_SCRATCH_BYTES, "header and library agree");
static_assert(kCounterRegion == EKV_NOALLOC_COUNTER_BYTES, "header and library agree");

__device__ __align__(256) unsigned char scratch[kScratchBytes];

struct DeviceScratch {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
  bool cleared = false;
};

DeviceScratch g_dev[kMaxDevices];
std::mutex g_clear_mutex;

__global__ void zero_words(unsigned int* p, unsigned int n) {
  const unsigned int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// This device's address of `scratch` (looked up once per device, with the
// device current), or NULL with the HIP error in *err.
void* scratch_ptr(int dev, hipError_t* err) {
  DeviceScratch& d = g_dev[dev];
  std::call_once(d.once, [&d] {
    void* p = nullptr;
    d.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (d.err == hipSuccess && p == nullptr) d.err = hipErrorInvalidSymbol;
    if (d.err == hipSuccess) d.ptr = p;
  });
  *err = d.err;
  return d.ptr;
}

}  // namespace

extern "C" {

ekv_status ekv_decode_step_noalloc(const ekv_cache_desc* desc, const float* q, float scale,
                                   float alpha, const void* K, const void* V,
                                   const int32_t* block_table, const int32_t* seq_lens,
                                   int32_t refresh_last_page, int32_t top_k, void* kmin,
                                   void* kmax, float* ubg, int32_t* sel, int32_t* n_sel,
                                   float* out, float* tau_out, int32_t* n_support,
                                   hipStream_t stream) {
  // every argument is validated, and the scratch sized, before any device call
  const ekv_status st = ekv::validate_step(desc, q, scale, alpha, K, V, block_table, seq_lens,
                                           top_k, kmin, kmax, ubg, sel, n_sel, out, tau_out,
                                           n_support);
  if (st != EKV_OK) return st;
  size_t cbytes = 0;
  const size_t rest = ekv::step_scratch_bytes(desc, top_k, &cbytes);
  if (rest == 0) return EKV_ERR_UNSUPPORTED;
  if (cbytes > kCounterRegion || rest > kScratchBytes - kCounterRegion) return EKV_ERR_WORKSPACE;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return EKV_ERR_HIP;
  hipError_t e = hipSuccess;
  unsigned char* base = (unsigned char*)scratch_ptr(dev, &e);
  if (base == nullptr) return EKV_ERR_HIP;
  {
    // clear the counter region once per device, ahead of this call's work
    std::lock_guard<std::mutex> lock(g_clear_mutex);
    if (!g_dev[dev].cleared) {
      const unsigned int words = (unsigned int)(kCounterRegion / sizeof(unsigned int));
      hipLaunchKernelGGL(zero_words, dim3((words + 255) / 256), dim3(256), 0, stream,
                         (unsigned int*)base, words);
      if (hipGetLastError() != hipSuccess) return EKV_ERR_HIP;
      g_dev[dev].cleared = true;
    }
  }
  return ekv::decode_step_parts(desc, q, scale, alpha, K, V, block_table, seq_lens,
                                refresh_last_page, top_k, kmin, kmax, ubg, sel, n_sel, out,
                                tau_out, n_support, base, kCounterRegion, base + kCounterRegion,
                                kScratchBytes - kCounterRegion, stream);
}

}  // extern "C"
