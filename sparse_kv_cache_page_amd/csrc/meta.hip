// Page metadata builder (EntmaxKV summary page, §2.A: per-page bounding box
// k_min/k_max and per-page key mean/variance).
//
// One wave64 per (physical page, KV head) tile.  The P x d tile is contiguous,
// so lanes read 16-byte chunks of consecutive rows: lane = (row group, chunk),
// kLpr lanes cover one row, 64/kLpr rows are read per wave instruction.
// Min/max are exact; the mean and the population variance use two passes with
// fp64 sums (the second pass re-reads the tile, which is still in L1/L2), and
// are rounded to fp32 once at the end.
#include "blocks.h"
#include "kernels.h"

namespace ekv {
namespace {

template <typename T, int D>
__global__ __launch_bounds__(256) void build_meta_kernel(
    const T* __restrict__ K, const int32_t* __restrict__ bt, const int32_t* __restrict__ lens,
    const int32_t* __restrict__ first_page, int span, int B, int Hkv, int P, int maxP,
    T* __restrict__ kmin, T* __restrict__ kmax, float* __restrict__ mean,
    float* __restrict__ var) {
  const int wave = threadIdx.x / kWave;
  const long long tile = (long long)blockIdx.x * 4 + wave;
  const int g = (int)(tile % Hkv);
  const long long t2 = tile / Hkv;
  const int pr = (int)(t2 % span);
  const int b = (int)(t2 / span);
  if (b >= B) return;
  const int L = lens[b];
  const int np = (L + P - 1) / P;
  const int p = (first_page ? first_page[b] : 0) + pr;
  if (p < 0 || p >= np) return;
  meta_tile<T, D>(K, Hkv, P, bt[(size_t)b * maxP + p], g, page_valid(L, p, P), kmin, kmax, mean, var);
}

template <typename T, int D>
hipError_t launch_meta_t(const Shape& s, const void* K, const int32_t* bt, const int32_t* lens,
                         const int32_t* first_page, int span, void* kmin, void* kmax,
                         float* mean, float* var, hipStream_t stream) {
  const long long tiles = (long long)s.B * span * s.Hkv;
  const long long blocks = (tiles + 3) / 4;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((build_meta_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const T*)K, bt, lens, first_page, span, s.B, s.Hkv, s.P, s.maxP, (T*)kmin,
                     (T*)kmax, mean, var);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_build_meta(const Shape& s, const void* K, const int32_t* bt,
                             const int32_t* lens, const int32_t* first_page, int span,
                             void* kmin, void* kmax, float* mean, float* var,
                             hipStream_t stream) {
  if (s.bf16) {
    if (s.D == 128)
      return launch_meta_t<bf16_t, 128>(s, K, bt, lens, first_page, span, kmin, kmax, mean, var, stream);
    return launch_meta_t<bf16_t, 64>(s, K, bt, lens, first_page, span, kmin, kmax, mean, var, stream);
  }
  if (s.D == 128)
    return launch_meta_t<float, 128>(s, K, bt, lens, first_page, span, kmin, kmax, mean, var, stream);
  return launch_meta_t<float, 64>(s, K, bt, lens, first_page, span, kmin, kmax, mean, var, stream);
}

}  // namespace ekv
