// Query-aware page scorer (EntmaxKV summary page, §2.A: a deterministic upper
// bound on the largest score of any token of a page from its bounding box, and
// the Gaussian moments of the page's scores from its key mean/variance).
//
// For one query head and one page, with q+ = max(q, 0) and q- = min(q, 0),
//     sum_j max(q_j kmin_j, q_j kmax_j) = sum_j q+_j kmax_j + q-_j kmin_j
// because the larger end point is kmax when q_j >= 0 and kmin otherwise.  Both
// products are exact in fp64 (fp32 x bf16 or fp32 x fp32 significands fit in
// 53 bits) and one of them is an exact zero, so the fp64 FMA chain only rounds
// in its additions; the bound is then scaled and rounded once to fp32.
//
// Mapping: one (row, KV head) pair per blockIdx.y; kLpr lanes cover one page's
// d coordinates with kVec coordinates each (16- or 8-byte loads of kmin and
// kmax), so a wave scores 64/kLpr pages per step for all G query heads of the
// group; per-head partial sums are reduced over the kLpr lanes with DPP.
// q+ and q- stay in registers as fp64 for the whole launch.
#include "common.h"
#include "kernels.h"

namespace ekv {
namespace {

template <typename T, int N> struct VecLoad;
template <> struct VecLoad<bf16_t, 8> {
  __device__ static void load(const bf16_t* p, float* x) { Elem<bf16_t>::unpack(load16_stream(p), x); }
};
template <> struct VecLoad<bf16_t, 4> {
  __device__ static void load(const bf16_t* p, float* x) {
    const uint2 w = load8_stream(p);
    x[0] = __uint_as_float(w.x << 16);
    x[1] = __uint_as_float(w.x & 0xffff0000u);
    x[2] = __uint_as_float(w.y << 16);
    x[3] = __uint_as_float(w.y & 0xffff0000u);
  }
};
template <> struct VecLoad<float, 4> {
  __device__ static void load(const float* p, float* x) { Elem<float>::unpack(load16_stream(p), x); }
};
template <> struct VecLoad<float, 2> {
  __device__ static void load(const float* p, float* x) {
    const uint2 w = load8_stream(p);
    x[0] = __uint_as_float(w.x);
    x[1] = __uint_as_float(w.y);
  }
};

constexpr int kScoreBlock = 256;

template <typename T, int D, int G, int kVec, bool kGauss>
__global__ __launch_bounds__(kScoreBlock) void score_kernel(
    const float* __restrict__ q, float scale, const T* __restrict__ kmin,
    const T* __restrict__ kmax, const float* __restrict__ mean, const float* __restrict__ var,
    const int32_t* __restrict__ bt, const int32_t* __restrict__ lens, int Hkv, int P, int maxP,
    int pages_per_block, float* __restrict__ ub, float* __restrict__ ubg,
    double* __restrict__ gm, double* __restrict__ gv) {
  constexpr int kLpr = D / kVec;
  constexpr int kPagesPerWave = kWave / kLpr;
  constexpr int kPagesPerStep = kPagesPerWave * (kScoreBlock / kWave);
  static_assert(G <= kLpr, "one lane per head writes the result");

  const int pair = blockIdx.y;
  const int b = pair / Hkv;
  const int g = pair % Hkv;
  const int Hq = Hkv * G;
  const int L = lens[b];
  const int np = (L + P - 1) / P;
  const int p_begin = blockIdx.x * pages_per_block;
  if (p_begin >= np) return;
  const int p_end = min(np, p_begin + pages_per_block);

  const int lane = threadIdx.x % kWave;
  const int c = lane % kLpr;
  const int slot = threadIdx.x / kLpr;  // page slot inside a step

  double qp[G][kVec], qn[G][kVec];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float* qh = q + ((size_t)b * Hq + g * G + h) * D + c * kVec;
#pragma unroll
    for (int v = 0; v < kVec; ++v) {
      const float x = qh[v];
      qp[h][v] = x > 0.0f ? (double)x : 0.0;
      qn[h][v] = x < 0.0f ? (double)x : 0.0;
    }
  }
  const double dscale = (double)scale;

  for (int p = p_begin + slot; p - slot < p_end; p += kPagesPerStep) {
    const bool live = p < p_end;
    const int pp = live ? p : p_begin;
    const int pi = bt[(size_t)b * maxP + pp];
    const size_t off = ((size_t)pi * Hkv + g) * D + c * kVec;
    float lo[kVec], hi[kVec];
    VecLoad<T, kVec>::load(kmin + off, lo);
    VecLoad<T, kVec>::load(kmax + off, hi);
    double acc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      double a = 0.0;
#pragma unroll
      for (int v = 0; v < kVec; ++v) {
        a = fma(qp[h][v], (double)hi[v], a);
        a = fma(qn[h][v], (double)lo[v], a);
      }
      acc[h] = group_sum_f64<kLpr>(a);
    }
    double mg[G], vg[G];
    if constexpr (kGauss) {
      float mu[kVec], s2[kVec];
      if constexpr (kVec >= 4) {
#pragma unroll
        for (int v = 0; v < kVec; v += 4) {
          VecLoad<float, 4>::load(mean + off + v, mu + v);
          VecLoad<float, 4>::load(var + off + v, s2 + v);
        }
      } else {
        VecLoad<float, 2>::load(mean + off, mu);
        VecLoad<float, 2>::load(var + off, s2);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        double am = 0.0, av = 0.0;
#pragma unroll
        for (int v = 0; v < kVec; ++v) {
          const double qd = qp[h][v] + qn[h][v];
          am = fma(qd, (double)mu[v], am);
          av = fma(qd * qd, (double)s2[v], av);
        }
        mg[h] = group_sum_f64<kLpr>(am);
        vg[h] = group_sum_f64<kLpr>(av);
      }
    }
    if (!live) continue;
    float best = -__builtin_huge_valf();
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float u = (float)(dscale * acc[h]);
      best = fmaxf(best, u);
      if (c == h) {
        const size_t o = ((size_t)b * Hq + g * G + h) * maxP + p;
        if (ub != nullptr) ub[o] = u;
        if constexpr (kGauss) {
          gm[o] = dscale * mg[h];
          gv[o] = dscale * dscale * vg[h];
        }
      }
    }
    if (c == 0) ubg[(size_t)pair * maxP + p] = best;
  }
}

template <typename T, int D, int G, int kVec>
hipError_t launch_score_t(const Shape& s, const float* q, float scale, const void* kmin,
                          const void* kmax, const float* mean, const float* var,
                          const int32_t* bt, const int32_t* lens, float* ub, float* ubg,
                          double* gm, double* gv, hipStream_t stream) {
  constexpr int kLpr = D / kVec;
  constexpr int kPagesPerStep = (kWave / kLpr) * (kScoreBlock / kWave);
  // several steps per block keep q's register preload amortised; enough blocks
  // per pair to spread a long row over the chip
  const int steps = s.maxP >= 64 * kPagesPerStep ? 8 : (s.maxP >= 8 * kPagesPerStep ? 4 : 1);
  const int ppb = kPagesPerStep * steps;
  dim3 grid((s.maxP + ppb - 1) / ppb, s.B * s.Hkv);
  if (gm != nullptr) {
    hipLaunchKernelGGL((score_kernel<T, D, G, kVec, true>), grid, dim3(kScoreBlock), 0, stream, q,
                       scale, (const T*)kmin, (const T*)kmax, mean, var, bt, lens, s.Hkv, s.P,
                       s.maxP, ppb, ub, ubg, gm, gv);
  } else {
    hipLaunchKernelGGL((score_kernel<T, D, G, kVec, false>), grid, dim3(kScoreBlock), 0, stream,
                       q, scale, (const T*)kmin, (const T*)kmax, mean, var, bt, lens, s.Hkv,
                       s.P, s.maxP, ppb, ub, ubg, gm, gv);
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_score_d(const Shape& s, const float* q, float scale, const void* kmin,
                          const void* kmax, const float* mean, const float* var,
                          const int32_t* bt, const int32_t* lens, float* ub, float* ubg,
                          double* gm, double* gv, hipStream_t stream) {
  // 16-byte loads while q+/q- fit comfortably in registers, 8-byte loads for
  // the 8-head group (halves the per-lane coordinates, hence the registers)
  constexpr int kV16 = 16 / sizeof(T);
  constexpr int kV8 = 8 / sizeof(T);
  switch (s.G) {
    case 1: return launch_score_t<T, D, 1, kV16>(s, q, scale, kmin, kmax, mean, var, bt, lens, ub, ubg, gm, gv, stream);
    case 2: return launch_score_t<T, D, 2, kV16>(s, q, scale, kmin, kmax, mean, var, bt, lens, ub, ubg, gm, gv, stream);
    case 4: return launch_score_t<T, D, 4, kV16>(s, q, scale, kmin, kmax, mean, var, bt, lens, ub, ubg, gm, gv, stream);
    case 8: return launch_score_t<T, D, 8, kV8>(s, q, scale, kmin, kmax, mean, var, bt, lens, ub, ubg, gm, gv, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_score(const Shape& s, const float* q, float scale, const void* kmin,
                        const void* kmax, const float* mean, const float* var,
                        const int32_t* bt, const int32_t* lens, float* ub, float* ubg,
                        double* gm, double* gv, hipStream_t stream) {
  if (s.bf16) {
    if (s.D == 128) return launch_score_d<bf16_t, 128>(s, q, scale, kmin, kmax, mean, var, bt, lens, ub, ubg, gm, gv, stream);
    return launch_score_d<bf16_t, 64>(s, q, scale, kmin, kmax, mean, var, bt, lens, ub, ubg, gm, gv, stream);
  }
  if (s.D == 128) return launch_score_d<float, 128>(s, q, scale, kmin, kmax, mean, var, bt, lens, ub, ubg, gm, gv, stream);
  return launch_score_d<float, 64>(s, q, scale, kmin, kmax, mean, var, bt, lens, ub, ubg, gm, gv, stream);
}

}  // namespace ekv
