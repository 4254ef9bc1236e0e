// Candidate page selection (EntmaxKV summary page, §2.B).
//
// Top-k: per (row, KV head) one 256-thread workgroup selects the k largest
// bounds with a radix select on the order-preserving uint32 image of the fp32
// bounds.  Each pass splits the keys' current range [lo, hi] into at most 2048
// bins (LDS histogram), a block scan finds the bin holding the k-th largest
// key, and the range narrows to that bin.  The search stops early when every
// key in the chosen bin belongs to the answer; otherwise it ends with the exact
// k-th largest key T and the number r of pages equal to T that still fit.  A block prefix sum over page order then writes, in
// ascending order, every page with key > T and the r lowest-index pages with
// key == T (ties go to the lower page index).
//
// Gaussian-aware: per query head, tau-hat solves
//     F(tau) = sum_p n_p E[(X_p - tau)_+^gamma] = 1,  X_p ~ N(mu_p, s_p^2),
// with E[(X - c)_+^g] = s^g I_g((mu - c)/s) and I_0 = Phi, I_1 = h Phi + phi,
// I_g = h I_{g-1} + (g-1) I_{g-2}.  F is convex and decreasing (gamma >= 1),
// F >= 1 at max_p mu_p - 1, and F' = -gamma sum_p n_p s^(g-1) I_{g-1}, so
// Newton's method started there climbs monotonically to the root.  A second
// kernel keeps page p when (alpha-1) est_{h,p} >= tau-hat_h - delta for some
// head of the group and compacts the kept pages in ascending order.  The
// page's estimated maximum score est is its box bound u (box-bound reading), or
// m + e_n sqrt(v), the expected maximum of its n valid token scores drawn from
// N(m, v) (expected-maximum reading), with e_n = E[max of n iid N(0,1)]
// tabulated once on the host.
#include "blocks.h"
#include "kernels.h"

namespace ekv {
namespace {

constexpr int kSelBlock = 256;
constexpr int kGaussLdsPages = 4096;  // 144 KiB of LDS (mu, sigma, 1/sigma in fp64 and fp32) per head
constexpr int kTauBlock = 1024;
constexpr int kTauWaves = kTauBlock / kWave;
constexpr int kMarkBlock = 1024;
constexpr int kMarkWaves = kMarkBlock / kWave;
constexpr int kMarkChunk = 4096;  // pages whose keep flags are staged in LDS at once

template <bool kLds>
__global__ __launch_bounds__(kSelBlock) void topk_kernel(
    const float* __restrict__ ubg, const int32_t* __restrict__ lens, int P, int maxP, int Hkv,
    int top_k, int32_t* __restrict__ sel, int32_t* __restrict__ n_sel) {
  __shared__ TopkLds<kLds ? kTopkLdsKeys : 1> sm;
  __shared__ TopkRegLds smr;
  const int pair = blockIdx.x;
  const int b = pair / Hkv;
  const int n = (lens[b] + P - 1) / P;
  const int k = min(top_k, n);
  int32_t* out = sel + (size_t)pair * maxP;
  if (k >= n) {
    for (int p = threadIdx.x; p < n; p += kSelBlock) out[p] = p;
  } else if (n <= kBlk * 8) {
    topk_block_reg<8, false>(ubg + (size_t)pair * maxP, n, k, out, smr);
  } else if (n <= kBlk * 16) {
    topk_block_reg<16, false>(ubg + (size_t)pair * maxP, n, k, out, smr);
  } else {
    topk_block<kLds, false>(ubg + (size_t)pair * maxP, n, k, out, sm);
  }
  if (threadIdx.x == 0) n_sel[pair] = k;
}

// --------------------------------------------------------------------------
// Gaussian-aware selection
// --------------------------------------------------------------------------
// I_g(h), I_{g-1}(h) and J(h) for Z ~ N(0,1), in the precision of T, where
// dI_g/dh = g I_{g-1} and J = d^2 I_g / dh^2 = g (g-1) I_{g-2} (phi for g = 1)
template <int kG, typename T>
__device__ inline void partial_moments(T h, T& ig, T& igm1, T& jdd) {
  T Phi, phi;
  if constexpr (sizeof(T) == 8) {
    Phi = 0.5 * erfc(-h * 0.70710678118654752440);
    phi = exp(-0.5 * h * h) * 0.39894228040143267794;
  } else {
    Phi = 0.5f * erfcf(-h * 0.70710678f);
    phi = expf(-0.5f * h * h) * 0.39894228f;
  }
  T i_pp = phi;               // I_{-1} in the recurrence's sense
  T i_prev = Phi;             // I_0
  T i_cur = fma(h, Phi, phi); // I_1
#pragma unroll
  for (int k = 2; k <= kG; ++k) {
    const T nxt = fma(h, i_cur, (T)(k - 1) * i_prev);
    i_pp = i_prev;
    i_prev = i_cur;
    i_cur = nxt;
  }
  ig = i_cur;
  igm1 = i_prev;
  jdd = kG >= 2 ? (T)(kG * (kG - 1)) * i_pp : phi;
}

template <int kG, typename T>
__device__ inline T ipow(T x) {
  T r = 1;
#pragma unroll
  for (int i = 0; i < kG; ++i) r *= x;
  return r;
}

// One page's contribution to F(tau), -F'(tau) and (kCurv) F''(tau), counted
// cnt times; rs = 1 / sd.
template <int kG, bool kCurv, typename T>
__device__ inline void gauss_term(T mz, T sd, T rs, T tau, T cnt, T& f, T& fd, T& fdd) {
  if (sd > 0) {
    const T h = (mz - tau) * rs;
    T ig, igm1, jdd;
    partial_moments<kG>(h, ig, igm1, jdd);
    const T sg1 = ipow<kG - 1>(sd);
    f = fma(cnt, sg1 * sd * ig, f);
    fd = fma(cnt, (T)kG * sg1 * igm1, fd);
    if constexpr (kCurv) fdd = fma(cnt, sg1 * rs * jdd, fdd);
  } else {
    const T x = mz - tau;
    if (x > 0) {
      const T xg1 = ipow<kG - 1>(x);
      f = fma(cnt, xg1 * x, f);
      fd = fma(cnt, (T)kG * xg1, fd);
      if constexpr (kCurv && kG >= 2) fdd = fma(cnt, (T)(kG * (kG - 1)) * ipow<kG - 2>(x), fdd);
    }
  }
}

// Block-wide sums of (a, b, c), returned to every thread: each wave sums its
// lanes with DPP, lane 0 stores the wave's three partials, and after one
// barrier every wave re-reduces them at once, quantity k on lanes 16k..16k+15
// with a 16-lane DPP butterfly (the same order in every wave, so every thread
// gets the same values).  sh holds 2 x 3 x kTauWaves values; successive calls
// alternate halves by `par`, so one barrier per call suffices.
static_assert(kTauWaves == 16, "one 16-lane row per summed quantity");

__device__ inline float wave_sum_t(float x) { return wave_sum_f32(x); }
__device__ inline double wave_sum_t(double x) { return wave_sum_f64(x); }
__device__ inline float row16_sum_t(float x) { return group_sum_f32<16>(x); }
__device__ inline double row16_sum_t(double x) { return group_sum_f64<16>(x); }
__device__ inline float readlane_t(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
__device__ inline double readlane_t(double x, int l) { return readlane_f64(x, l); }

template <typename T>
__device__ inline void block_sum3(T& a, T& b, T& c, T* sh, int par) {
  a = wave_sum_t(a);
  b = wave_sum_t(b);
  c = wave_sum_t(c);
  T* buf = sh + par * 3 * kTauWaves;
  const int w = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (lane == 0) {
    buf[w] = a;
    buf[kTauWaves + w] = b;
    buf[2 * kTauWaves + w] = c;
  }
  __syncthreads();
  T x = lane < 3 * kTauWaves ? buf[lane] : (T)0;
  x = row16_sum_t(x);
  a = readlane_t(x, 0);
  b = readlane_t(x, kTauWaves);
  c = readlane_t(x, 2 * kTauWaves);
}

// tau-hat for one (row, query head).  A coarse fp32 run approaches the root;
// the fp64 run then starts a small margin below it when F >= 1 holds there in
// fp64 (any such point keeps Newton monotone), else at the proven start
// max mu - 1, and stops when F - 1 or the step stops being positive, so its
// result is the monotone Newton limit either way.
template <int kG, bool kLds>
__global__ __launch_bounds__(kTauBlock) void gauss_tau_kernel(
    const double* __restrict__ gm, const double* __restrict__ gv, const int32_t* __restrict__ lens,
    int P, int maxP, int Hq, double a1, double* __restrict__ tau_hat) {
  __shared__ double s_mu[kLds ? kGaussLdsPages : 1];
  __shared__ double s_sd[kLds ? kGaussLdsPages : 1];
  __shared__ float s_mu32[kLds ? kGaussLdsPages : 1];
  __shared__ float s_sd32[kLds ? kGaussLdsPages : 1];
  __shared__ double s_rs[kLds ? kGaussLdsPages : 1];
  __shared__ float s_rs32[kLds ? kGaussLdsPages : 1];
  __shared__ double red[6 * kTauWaves];
  __shared__ float redf[6 * kTauWaves];
  const int bh = blockIdx.x;
  const int b = bh / Hq;
  const int L = lens[b];
  const int n = (L + P - 1) / P;
  if (n == 0) {  // empty row: no pages, no threshold
    if (threadIdx.x == 0) tau_hat[bh] = __builtin_nan("");
    return;
  }
  const double* M = gm + (size_t)bh * maxP;
  const double* V = gv + (size_t)bh * maxP;

  auto mu_of = [&](int p) -> double {
    if constexpr (kLds) return s_mu[p];
    else return a1 * M[p];
  };
  auto sd_of = [&](int p) -> double {
    if constexpr (kLds) return s_sd[p];
    else return a1 * sqrt(V[p]);
  };
  auto mu32_of = [&](int p) -> float {
    if constexpr (kLds) return s_mu32[p];
    else return (float)(a1 * M[p]);
  };
  auto sd32_of = [&](int p) -> float {
    if constexpr (kLds) return s_sd32[p];
    else return (float)(a1 * sqrt(V[p]));
  };
  auto inv = [](auto x) -> decltype(x) { return x > 0 ? (decltype(x))1 / x : (decltype(x))0; };
  auto rs_of = [&](int p) -> double {
    if constexpr (kLds) return s_rs[p];
    else return inv(a1 * sqrt(V[p]));
  };
  auto rs32_of = [&](int p) -> float {
    if constexpr (kLds) return s_rs32[p];
    else return inv((float)(a1 * sqrt(V[p])));
  };
  double zmax = -__builtin_huge_val();
  for (int p = threadIdx.x; p < n; p += kTauBlock) {
    const double mz = a1 * M[p];
    if constexpr (kLds) {
      const double sd = a1 * sqrt(V[p]);
      s_mu[p] = mz;
      s_sd[p] = sd;
      s_mu32[p] = (float)mz;
      s_sd32[p] = (float)sd;
      s_rs[p] = inv(sd);
      s_rs32[p] = inv((float)sd);
    }
    zmax = fmax(zmax, mz);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) zmax = fmax(zmax, __shfl_xor(zmax, o, kWave));
  if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = zmax;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kTauWaves; ++i) zmax = fmax(zmax, red[i]);
  const double safe = zmax - 1.0;  // F(safe) >= 1
  int par = 1;                     // red[0 .. kTauWaves) is still being read

  // Coarse fp32 run: Newton on g = log F, which is nearly linear where a few
  // Gaussian tails dominate (about half the steps of Newton on F), kept inside
  // the bracket (lo, hi) of points seen with F >= 1 and F < 1; a step leaving
  // it falls back to bisection, or, before any point with F < 1 is seen, to a
  // Newton step on F itself (which stays left of the root).
  const double huge = __builtin_huge_val();
  double lo = safe, hi = huge, t = safe;
  for (int it = 0; it < 48 && n > 0; ++it) {
    float f = 0.0f, fd = 0.0f, fdd = 0.0f;  // fdd unused here
    const float tf = (float)t;
    for (int p = threadIdx.x; p < n; p += kTauBlock)
      gauss_term<kG, false, float>(mu32_of(p), sd32_of(p), rs32_of(p), tf,
                                   (float)page_valid(L, p, P), f, fd, fdd);
    block_sum3(f, fd, fdd, redf, par);
    par ^= 1;
    const double fs = f, fds = fd;
    if (fs >= 1.0) lo = fmax(lo, t);
    else hi = fmin(hi, t);
    const bool ok = fs > 0.0 && fds > 0.0;
    double nxt = ok ? t + (double)(logf(f) * f / fd) : t;
    if (ok && fabs(nxt - t) < 1e-6 * (1.0 + fabs(nxt))) {  // converged as far as fp32 goes
      t = nxt;
      break;
    }
    if (!(nxt > lo && nxt < hi)) {
      if (hi < huge) nxt = 0.5 * (lo + hi);
      else if (fds > 0.0) nxt = t + (fs - 1.0) / fds;
      else break;
    }
    t = nxt;
  }

  // fp64 run: monotone Newton on F from a start just below the coarse root
  // (checked: F(start) >= 1 in fp64, else the proven start max mu - 1).  A step
  // ends it without another evaluation when the step itself is below
  // 1e-15 |tau|, or when Newton's error bound after it on the convex F,
  // F'' / (2 |F'|) step^2 (with a factor 4 to spare), is below 1e-16 |tau|.
  const double start = fmax(safe, t - 4e-6 * (1.0 + fabs(t)));
  double tau = start;
  for (int it = 0; it < 200; ++it) {
    double f = 0.0, fd = 0.0, fdd = 0.0;
    for (int p = threadIdx.x; p < n; p += kTauBlock)
      gauss_term<kG, true, double>(mu_of(p), sd_of(p), rs_of(p), tau, (double)page_valid(L, p, P),
                                   f, fd, fdd);
    block_sum3(f, fd, fdd, red, par);
    par ^= 1;
    f -= 1.0;
    if (it == 0 && f < 0.0 && tau > safe) {  // F(start) < 1: start over at the proven point
      tau = safe;
      continue;
    }
    if (!(f > 0.0) || !(fd > 0.0)) break;
    const double step = f / fd;
    const double nxt = tau + step;
    if (!(nxt > tau)) break;
    tau = nxt;
    if (step <= 1e-15 * fabs(tau) || 2.0 * fdd / fd * step * step <= 1e-16 * fabs(tau)) break;
  }
  if (threadIdx.x == 0) tau_hat[bh] = tau;
}

// e_n for n = 0 .. kMaxPageSize (entry 0 unused)
struct ExpMaxTable {
  double e[kMaxPageSize + 1];
};

// Ascending compaction of flag(p) for p < n into out[]; returns the count.
// Per chunk of kMarkChunk pages the flags are evaluated with consecutive
// threads on consecutive pages (coalesced reads) and staged in LDS; each
// thread then writes the kept pages of a contiguous run of them at its
// offset from a block scan.
template <typename Flag>
__device__ int compact_ascending(int n, Flag flag, int32_t* out, uint8_t* s_flag, int* sh) {
  int total = 0;
  for (int c0 = 0; c0 < n; c0 += kMarkChunk) {
    const int m = min(kMarkChunk, n - c0);
#pragma unroll 4
    for (int i = threadIdx.x; i < m; i += kMarkBlock) s_flag[i] = flag(c0 + i) ? 1 : 0;
    __syncthreads();
    const int per = (m + kMarkBlock - 1) / kMarkBlock;
    const int p0 = min(m, (int)threadIdx.x * per);
    const int p1 = min(m, p0 + per);
    int cnt = 0;
    for (int i = p0; i < p1; ++i) cnt += s_flag[i];
    const int incl = block_incl_scan(cnt, sh);
    int pos = total + incl - cnt;
    for (int i = p0; i < p1; ++i)
      if (s_flag[i]) out[pos++] = c0 + i;
    if (threadIdx.x == kMarkBlock - 1) sh[kMarkWaves] = incl;
    __syncthreads();
    total += sh[kMarkWaves];
    __syncthreads();  // s_flag and sh are rewritten by the next chunk
  }
  return total;
}

// Which estimate a Gaussian rule compares: the box bound, the expected
// maximum of the page's tokens, or the page's expected entmax mass.
enum MarkRule { kRuleBound = 0, kRuleEstMax = 1, kRuleMass = 2 };

template <int kRule, int G, int kG>
__global__ __launch_bounds__(kMarkBlock) void gauss_mark_kernel(
    const float* __restrict__ ub, const float* __restrict__ ubg, const double* __restrict__ gm,
    const double* __restrict__ gv, const double* __restrict__ tau_hat,
    const int32_t* __restrict__ lens, int P, int maxP, int Hkv, double a1, double delta,
    ExpMaxTable et, int32_t* __restrict__ sel, int32_t* __restrict__ n_sel) {
  __shared__ uint8_t s_flag[kMarkChunk];
  __shared__ int scan_sh[kMarkWaves + 1];
  __shared__ float s_best[kMarkWaves];
  __shared__ int s_bestp[kMarkWaves];
  const int pair = blockIdx.x;
  const int b = pair / Hkv;
  const int g = pair % Hkv;
  const int Hq = Hkv * G;
  const int L = lens[b];
  const int n = (L + P - 1) / P;
  if (n == 0) {  // empty row: nothing to select (the guard needs a page)
    if (threadIdx.x == 0) n_sel[pair] = 0;
    return;
  }
  const size_t head0 = ((size_t)b * Hq + g * G) * maxP;
  const double* th = tau_hat + (size_t)b * Hq + g * G;
  int32_t* out = sel + (size_t)pair * maxP;
  // every page but the last holds P tokens
  const int n_last = page_valid(L, n - 1, P);
  const double e_full = et.e[P];
  const double e_last = et.e[n_last];
  auto keep = [&](int p) -> bool {
    bool any = false;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const size_t i = head0 + (size_t)h * maxP + p;
      if constexpr (kRule == kRuleMass) {
        // n_p E[(X - tau_hat)_+^gamma], X ~ N((alpha-1) m, (alpha-1)^2 v):
        // the expected entmax mass of the page's tokens, against delta
        const double mz = a1 * gm[i];
        const double sd = a1 * sqrt(gv[i]);
        const double cnt = p == n - 1 ? (double)n_last : (double)P;
        double mass;
        if (sd > 0.0) {
          double ig, igm1, jdd;
          partial_moments<kG>((mz - th[h]) / sd, ig, igm1, jdd);
          mass = cnt * (ipow<kG>(sd) * ig);
        } else {
          const double x = mz - th[h];
          mass = x > 0.0 ? cnt * ipow<kG>(x) : 0.0;
        }
        any |= mass >= delta;
        continue;
      }
      double est;
      if constexpr (kRule == kRuleEstMax) {
        // m + e_n sqrt(v), each operation rounded on its own (no contraction)
        const double e = p == n - 1 ? e_last : e_full;
        est = __dadd_rn(gm[i], __dmul_rn(e, sqrt(gv[i])));
      } else {
        est = (double)ub[((size_t)pair * maxP + p) * G + h];
      }
      any |= __dmul_rn(a1, est) >= th[h] - delta;
    }
    return any;
  };
  const int got = compact_ascending(n, keep, out, s_flag, scan_sh);
  if (got > 0) {
    if (threadIdx.x == 0) n_sel[pair] = got;
    return;
  }
  // nothing cleared the bar: keep the page with the largest group bound
  const float* U = ubg + (size_t)pair * maxP;
  float best = -__builtin_huge_valf();
  int bestp = 0x7fffffff;
  for (int p = threadIdx.x; p < n; p += kMarkBlock) {
    const float u = U[p];
    if (u > best || (u == best && p < bestp)) {
      best = u;
      bestp = p;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ob = __shfl_xor(best, o, kWave);
    const int op = __shfl_xor(bestp, o, kWave);
    if (ob > best || (ob == best && op < bestp)) {
      best = ob;
      bestp = op;
    }
  }
  if (threadIdx.x % kWave == 0) {
    s_best[threadIdx.x / kWave] = best;
    s_bestp[threadIdx.x / kWave] = bestp;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kMarkWaves; ++w)
      if (s_best[w] > best || (s_best[w] == best && s_bestp[w] < bestp)) {
        best = s_best[w];
        bestp = s_bestp[w];
      }
    out[0] = bestp;
    n_sel[pair] = 1;
  }
}

template <int kG>
hipError_t launch_gauss_tau(const Shape& s, const int32_t* lens, double a1, const double* gm,
                            const double* gv, double* tau_hat, hipStream_t stream) {
  if (s.maxP <= kGaussLdsPages)
    hipLaunchKernelGGL((gauss_tau_kernel<kG, true>), dim3(s.B * s.Hq), dim3(kTauBlock), 0, stream,
                       gm, gv, lens, s.P, s.maxP, s.Hq, a1, tau_hat);
  else
    hipLaunchKernelGGL((gauss_tau_kernel<kG, false>), dim3(s.B * s.Hq), dim3(kTauBlock), 0,
                       stream, gm, gv, lens, s.P, s.maxP, s.Hq, a1, tau_hat);
  return hipGetLastError();
}

// e_n = integral of x n phi(x) Phi(x)^(n-1) dx by the trapezoidal rule on
// [-16, 16] with step 1/128: the integrand is analytic and decays like phi, so
// the rule converges geometrically and the truncated tails are below 1e-50.
// The nodes are summed with Neumaier's compensated summation.
const ExpMaxTable& exp_max_table() {
  static const ExpMaxTable table = [] {
    ExpMaxTable t{};
    double comp[kMaxPageSize + 1] = {};
    constexpr int kSteps = 4096;
    constexpr double kHalfWidth = 16.0;
    constexpr double h = 2.0 * kHalfWidth / kSteps;
    const double inv_sqrt_2pi = 0.39894228040143267794;
    for (int i = 0; i <= kSteps; ++i) {
      const double x = -kHalfWidth + i * h;
      const double w = (i == 0 || i == kSteps) ? 0.5 * h : h;
      const double phi = exp(-0.5 * x * x) * inv_sqrt_2pi;
      const double Phi = 0.5 * erfc(-x * 0.70710678118654752440);
      double pw = 1.0;  // Phi^(n-1)
      for (int n = 1; n <= kMaxPageSize; ++n) {
        const double term = w * x * n * phi * pw;
        const double sum = t.e[n] + term;
        comp[n] += fabs(t.e[n]) >= fabs(term) ? (t.e[n] - sum) + term : (term - sum) + t.e[n];
        t.e[n] = sum;
        pw *= Phi;
      }
    }
    for (int n = 1; n <= kMaxPageSize; ++n) t.e[n] += comp[n];
    t.e[0] = 0.0;
    t.e[1] = 0.0;  // symmetric integrand: exactly zero
    return t;
  }();
  return table;
}

template <int kRule, int G, int kG>
void launch_mark_t(const Shape& s, const float* ub, const float* ubg, const double* gm,
                   const double* gv, const double* tau_hat, const int32_t* lens, double a1,
                   double delta, const ExpMaxTable& et, int32_t* sel, int32_t* n_sel,
                   hipStream_t stream) {
  hipLaunchKernelGGL((gauss_mark_kernel<kRule, G, kG>), dim3(s.B * s.Hkv), dim3(kMarkBlock), 0,
                     stream, ub, ubg, gm, gv, tau_hat, lens, s.P, s.maxP, s.Hkv, a1, delta, et,
                     sel, n_sel);
}

template <int G>
hipError_t launch_mark(const Shape& s, int rule, int gamma, const float* ub, const float* ubg,
                       const double* gm, const double* gv, const double* tau_hat,
                       const int32_t* lens, double a1, double delta, const ExpMaxTable& et,
                       int32_t* sel, int32_t* n_sel, hipStream_t stream) {
#define EKV_MARK(R, KG) \
  launch_mark_t<R, G, KG>(s, ub, ubg, gm, gv, tau_hat, lens, a1, delta, et, sel, n_sel, stream)
  if (rule == kRuleBound) {
    EKV_MARK(kRuleBound, 1);
  } else if (rule == kRuleEstMax) {
    EKV_MARK(kRuleEstMax, 1);
  } else {
    switch (gamma) {
      case 1: EKV_MARK(kRuleMass, 1); break;
      case 2: EKV_MARK(kRuleMass, 2); break;
      case 3: EKV_MARK(kRuleMass, 3); break;
      case 4: EKV_MARK(kRuleMass, 4); break;
      default: return hipErrorInvalidValue;
    }
  }
#undef EKV_MARK
  return hipSuccess;
}

}  // namespace

double expected_max_std_normal(int n) {
  if (n < 1 || n > kMaxPageSize) return __builtin_nan("");
  return exp_max_table().e[n];
}

hipError_t launch_topk(const Shape& s, const int32_t* lens, int top_k, const float* ubg,
                       int32_t* sel, int32_t* n_sel, hipStream_t stream) {
  if (s.maxP <= kTopkLdsKeys)
    hipLaunchKernelGGL((topk_kernel<true>), dim3(s.B * s.Hkv), dim3(kSelBlock), 0, stream, ubg,
                       lens, s.P, s.maxP, s.Hkv, top_k, sel, n_sel);
  else
    hipLaunchKernelGGL((topk_kernel<false>), dim3(s.B * s.Hkv), dim3(kSelBlock), 0, stream, ubg,
                       lens, s.P, s.maxP, s.Hkv, top_k, sel, n_sel);
  return hipGetLastError();
}

hipError_t launch_gauss(const Shape& s, const int32_t* lens, float alpha, int gamma, float delta,
                        int rule, const float* ub, const float* ubg, const double* gm,
                        const double* gv, int32_t* sel, int32_t* n_sel, double* tau_hat,
                        hipStream_t stream) {
  const double a1 = (double)alpha - 1.0;
  hipError_t e = hipErrorInvalidValue;
  switch (gamma) {
    case 1: e = launch_gauss_tau<1>(s, lens, a1, gm, gv, tau_hat, stream); break;
    case 2: e = launch_gauss_tau<2>(s, lens, a1, gm, gv, tau_hat, stream); break;
    case 3: e = launch_gauss_tau<3>(s, lens, a1, gm, gv, tau_hat, stream); break;
    case 4: e = launch_gauss_tau<4>(s, lens, a1, gm, gv, tau_hat, stream); break;
  }
  if (e != hipSuccess) return e;
  const ExpMaxTable& et = exp_max_table();
  switch (s.G) {
    case 1: e = launch_mark<1>(s, rule, gamma, ub, ubg, gm, gv, tau_hat, lens, a1, delta, et, sel, n_sel, stream); break;
    case 2: e = launch_mark<2>(s, rule, gamma, ub, ubg, gm, gv, tau_hat, lens, a1, delta, et, sel, n_sel, stream); break;
    case 4: e = launch_mark<4>(s, rule, gamma, ub, ubg, gm, gv, tau_hat, lens, a1, delta, et, sel, n_sel, stream); break;
    case 8: e = launch_mark<8>(s, rule, gamma, ub, ubg, gm, gv, tau_hat, lens, a1, delta, et, sel, n_sel, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace ekv
