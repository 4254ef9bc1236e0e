// Page metadata builder (EntmaxKV summary page, §2.A: per-page bounding box
// k_min/k_max and per-page key mean/variance).
//
// One wave64 per (physical page, KV head) tile.  The P x d tile is contiguous,
// so lanes read 16-byte chunks of consecutive rows: lane = (row group, chunk),
// kLpr lanes cover one row, 64/kLpr rows are read per wave instruction.
// Min/max are exact; the mean and the population variance use two passes with
// fp64 sums (the second pass re-reads the tile, which is still in L1/L2), and
// are rounded to fp32 once at the end.
#include "common.h"
#include "kernels.h"

namespace ekv {
namespace {

template <typename T, int D>
__global__ __launch_bounds__(256) void build_meta_kernel(
    const T* __restrict__ K, const int32_t* __restrict__ bt, const int32_t* __restrict__ lens,
    const int32_t* __restrict__ first_page, int span, int B, int Hkv, int P, int maxP,
    T* __restrict__ kmin, T* __restrict__ kmax, float* __restrict__ mean,
    float* __restrict__ var) {
  constexpr int kVec = Elem<T>::kVec;
  constexpr int kLpr = D / kVec;      // lanes per key row
  constexpr int kRows = kWave / kLpr; // rows per wave instruction
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
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
  const int nv = page_valid(L, p, P);
  const int pi = bt[(size_t)b * maxP + p];
  const size_t tile_off = ((size_t)pi * Hkv + g) * (size_t)P * D;
  const T* src = K + tile_off;
  const int c = lane % kLpr;
  const int r0 = lane / kLpr;

  float mn[kVec], mx[kVec];
  double sm[kVec];
#pragma unroll
  for (int v = 0; v < kVec; ++v) {
    mn[v] = __builtin_huge_valf();
    mx[v] = -__builtin_huge_valf();
    sm[v] = 0.0;
  }
  for (int t = r0; t < nv; t += kRows) {
    float x[kVec];
    Elem<T>::unpack(load16(src + (size_t)t * D + c * kVec), x);
#pragma unroll
    for (int v = 0; v < kVec; ++v) {
      mn[v] = fminf(mn[v], x[v]);
      mx[v] = fmaxf(mx[v], x[v]);
      sm[v] += (double)x[v];
    }
  }
#pragma unroll
  for (int o = kLpr; o < kWave; o <<= 1) {
#pragma unroll
    for (int v = 0; v < kVec; ++v) {
      mn[v] = fminf(mn[v], __shfl_xor(mn[v], o, kWave));
      mx[v] = fmaxf(mx[v], __shfl_xor(mx[v], o, kWave));
      sm[v] += __shfl_xor(sm[v], o, kWave);
    }
  }
  double mu[kVec], sq[kVec];
#pragma unroll
  for (int v = 0; v < kVec; ++v) {
    mu[v] = sm[v] / (double)nv;
    sq[v] = 0.0;
  }
  for (int t = r0; t < nv; t += kRows) {
    float x[kVec];
    Elem<T>::unpack(load16(src + (size_t)t * D + c * kVec), x);
#pragma unroll
    for (int v = 0; v < kVec; ++v) {
      const double dlt = (double)x[v] - mu[v];
      sq[v] = fma(dlt, dlt, sq[v]);
    }
  }
#pragma unroll
  for (int o = kLpr; o < kWave; o <<= 1) {
#pragma unroll
    for (int v = 0; v < kVec; ++v) sq[v] += __shfl_xor(sq[v], o, kWave);
  }
  if (r0 != 0) return;

  const size_t m_off = ((size_t)pi * Hkv + g) * D + c * kVec;
  if constexpr (sizeof(T) == 2) {
    // min/max of bf16 values are bf16 values: repack the top halves
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
  if (mean != nullptr) {
#pragma unroll
    for (int v = 0; v < kVec; v += 4) {
      *reinterpret_cast<float4*>(mean + m_off + v) =
          make_float4((float)mu[v], (float)mu[v + 1], (float)mu[v + 2], (float)mu[v + 3]);
      *reinterpret_cast<float4*>(var + m_off + v) = make_float4(
          (float)(sq[v] / nv), (float)(sq[v + 1] / nv), (float)(sq[v + 2] / nv),
          (float)(sq[v + 3] / nv));
    }
  }
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
