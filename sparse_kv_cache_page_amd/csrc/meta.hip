// Page metadata builder and decode-time append (EntmaxKV summary page, §2.A:
// per-page bounding box k_min/k_max and per-page key mean/variance, stored per
// page, so a new token changes only its own page's record).
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

template <typename T, int D, typename M>
__global__ __launch_bounds__(256) void build_meta_kernel(
    const T* __restrict__ K, const int32_t* __restrict__ bt, const int32_t* __restrict__ lens,
    const int32_t* __restrict__ first_page, int span, int B, int Hkv, int P, int maxP,
    T* __restrict__ kmin, T* __restrict__ kmax, M* __restrict__ mean, M* __restrict__ var) {
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
  meta_tile<T, D, M>(K, Hkv, P, bt[(size_t)b * maxP + p], g, page_valid(L, p, P), kmin, kmax,
                     mean, var);
}

template <typename T, int D, typename M>
hipError_t launch_meta_t(const Shape& s, const void* K, const int32_t* bt, const int32_t* lens,
                         const int32_t* first_page, int span, void* kmin, void* kmax,
                         void* mean, void* var, hipStream_t stream) {
  const long long tiles = (long long)s.B * span * s.Hkv;
  const long long blocks = (tiles + 3) / 4;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL((build_meta_kernel<T, D, M>), dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const T*)K, bt, lens, first_page, span, s.B, s.Hkv, s.P, s.maxP, (T*)kmin,
                     (T*)kmax, (M*)mean, (M*)var);
  return hipGetLastError();
}

// Decode-time append: one wave per (row b, KV head g).  The token at position
// t = lens[b] - 1 goes to slot t % P of page t / P; lanes of the first row
// group write its K and V rows.  Without moments the page's box is updated in
// place: min/max over the page's tokens taken in another order is the same
// exact value, so it equals a rebuild (the first token of a page starts a new
// box).  With moments the page is rebuilt by meta_tile over its valid tokens,
// as ekv_build_page_meta does; a workgroup-scope release/acquire pair makes
// the new row, stored by this wave's lanes, visible to the lanes that read it
// back (all lanes of a workgroup share one CU's vector L1).
template <typename T, int D, typename M>
__global__ __launch_bounds__(256) void append_kernel(
    const T* __restrict__ k_new, const T* __restrict__ v_new, const int32_t* __restrict__ bt,
    const int32_t* __restrict__ lens, int B, int Hkv, int P, int maxP, T* __restrict__ K,
    T* __restrict__ V, T* __restrict__ kmin, T* __restrict__ kmax, M* __restrict__ mean,
    M* __restrict__ var) {
  constexpr int kVec = Elem<T>::kVec;
  constexpr int kLpr = D / kVec;
  const int lane = threadIdx.x % kWave;
  const long long unit = (long long)blockIdx.x * 4 + threadIdx.x / kWave;
  if (unit >= (long long)B * Hkv) return;  // uniform over the wave
  const int b = (int)(unit / Hkv);
  const int g = (int)(unit % Hkv);
  const int L = lens[b];
  if (L < 1) return;
  const int t = L - 1;
  const int p = t / P;
  const int slot = t - p * P;
  const int pi = bt[(size_t)b * maxP + p];
  if (lane < kLpr) {
    const int c = lane;
    const size_t src = ((size_t)b * Hkv + g) * D + c * kVec;
    const size_t dst = (((size_t)pi * Hkv + g) * P + slot) * D + c * kVec;
    const uint4 kw = load16(k_new + src);
    const uint4 vw = load16(v_new + src);
    *reinterpret_cast<uint4*>(K + dst) = kw;
    *reinterpret_cast<uint4*>(V + dst) = vw;
    if (mean == nullptr) {
      const size_t m_off = ((size_t)pi * Hkv + g) * D + c * kVec;
      float x[kVec], mn[kVec], mx[kVec];
      Elem<T>::unpack(kw, x);
      if (slot == 0) {
#pragma unroll
        for (int v = 0; v < kVec; ++v) mn[v] = mx[v] = x[v];
      } else {
        Elem<T>::unpack(load16(kmin + m_off), mn);
        Elem<T>::unpack(load16(kmax + m_off), mx);
#pragma unroll
        for (int v = 0; v < kVec; ++v) {
          mn[v] = fminf(mn[v], x[v]);
          mx[v] = fmaxf(mx[v], x[v]);
        }
      }
      if constexpr (sizeof(T) == 2) {
        uint32_t wn[4], wx[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          wn[i] = (__float_as_uint(mn[2 * i]) >> 16) | (__float_as_uint(mn[2 * i + 1]) & 0xffff0000u);
          wx[i] = (__float_as_uint(mx[2 * i]) >> 16) | (__float_as_uint(mx[2 * i + 1]) & 0xffff0000u);
        }
        *reinterpret_cast<uint4*>(kmin + m_off) = make_uint4(wn[0], wn[1], wn[2], wn[3]);
        *reinterpret_cast<uint4*>(kmax + m_off) = make_uint4(wx[0], wx[1], wx[2], wx[3]);
      } else {
        *reinterpret_cast<float4*>(kmin + m_off) = make_float4(mn[0], mn[1], mn[2], mn[3]);
        *reinterpret_cast<float4*>(kmax + m_off) = make_float4(mx[0], mx[1], mx[2], mx[3]);
      }
    }
  }
  if (mean != nullptr) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    meta_tile<T, D, M>(K, Hkv, P, pi, g, slot + 1, kmin, kmax, mean, var);
  }
}

template <typename T, int D, typename M>
hipError_t launch_append_t(const Shape& s, const void* k_new, const void* v_new,
                           const int32_t* bt, const int32_t* lens, void* K, void* V, void* kmin,
                           void* kmax, void* mean, void* var, hipStream_t stream) {
  const long long units = (long long)s.B * s.Hkv;
  const long long blocks = (units + 3) / 4;
  hipLaunchKernelGGL((append_kernel<T, D, M>), dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const T*)k_new, (const T*)v_new, bt, lens, s.B, s.Hkv, s.P, s.maxP, (T*)K,
                     (T*)V, (T*)kmin, (T*)kmax, (M*)mean, (M*)var);
  return hipGetLastError();
}

// Device-side check of the cache description: one thread per (row, page
// slot); counts rows whose length is outside [0, maxP * P] (bad[0]) and
// block-table entries of a row's valid pages outside [0, Np) (bad[1]).
__global__ __launch_bounds__(256) void validate_kernel(const int32_t* __restrict__ bt,
                                                       const int32_t* __restrict__ lens, int B,
                                                       int P, int maxP, int Np,
                                                       int32_t* __restrict__ bad) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)B * maxP) return;
  const int b = (int)(i / maxP);
  const int p = (int)(i % maxP);
  const int L = lens[b];
  const bool len_ok = L >= 0 && (long long)L <= (long long)maxP * P;
  if (p == 0 && !len_ok) atomicAdd(&bad[0], 1);
  if (!len_ok) return;  // the row's page count is not defined
  if (p < (L + P - 1) / P) {
    const int pi = bt[i];
    if (pi < 0 || pi >= Np) atomicAdd(&bad[1], 1);
  }
}

__global__ void clear2_kernel(int32_t* bad) {
  if (threadIdx.x < 2) bad[threadIdx.x] = 0;
}

// K dtype x head dim x moment dtype
template <template <typename, int, typename> class F, typename... A>
hipError_t dispatch_meta(const Shape& s, A... args) {
  if (s.bf16) {
    if (s.D == 128)
      return s.mom16 ? F<bf16_t, 128, bf16_t>::run(s, args...) : F<bf16_t, 128, float>::run(s, args...);
    return s.mom16 ? F<bf16_t, 64, bf16_t>::run(s, args...) : F<bf16_t, 64, float>::run(s, args...);
  }
  if (s.D == 128)
    return s.mom16 ? F<float, 128, bf16_t>::run(s, args...) : F<float, 128, float>::run(s, args...);
  return s.mom16 ? F<float, 64, bf16_t>::run(s, args...) : F<float, 64, float>::run(s, args...);
}

template <typename T, int D, typename M>
struct AppendOp {
  template <typename... A>
  static hipError_t run(const Shape& s, A... args) { return launch_append_t<T, D, M>(s, args...); }
};
template <typename T, int D, typename M>
struct MetaOp {
  template <typename... A>
  static hipError_t run(const Shape& s, A... args) { return launch_meta_t<T, D, M>(s, args...); }
};

}  // namespace

hipError_t launch_validate(const Shape& s, const int32_t* bt, const int32_t* lens, int32_t* bad,
                           hipStream_t stream) {
  // the counters are cleared by a one-block kernel (no memset node in a
  // captured graph)
  hipLaunchKernelGGL(clear2_kernel, dim3(1), dim3(64), 0, stream, bad);
  const long long n = (long long)s.B * s.maxP;
  const long long blocks = (n + 255) / 256;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(validate_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, bt, lens, s.B,
                     s.P, s.maxP, s.Np, bad);
  return hipGetLastError();
}

hipError_t launch_append(const Shape& s, const void* k_new, const void* v_new,
                         const int32_t* bt, const int32_t* lens, void* K, void* V, void* kmin,
                         void* kmax, void* mean, void* var, hipStream_t stream) {
  return dispatch_meta<AppendOp>(s, k_new, v_new, bt, lens, K, V, kmin, kmax, mean, var, stream);
}

hipError_t launch_build_meta(const Shape& s, const void* K, const int32_t* bt,
                             const int32_t* lens, const int32_t* first_page, int span,
                             void* kmin, void* kmax, void* mean, void* var,
                             hipStream_t stream) {
  return dispatch_meta<MetaOp>(s, K, bt, lens, first_page, span, kmin, kmax, mean, var, stream);
}

}  // namespace ekv
