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
#include <type_traits>

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

// Top-k of long rows (4096 < n <= 65536 pages): one 1024-thread workgroup per
// (row, KV head) with kPer consecutive keys per thread in registers (no key
// re-reads from memory): range-adaptive 11-bit radix passes over a
// double-buffered LDS histogram, thread t owning digits 2047-2t and 2046-2t
// of the scan, then the same ordered placement as the 256-thread selection
// (every key above the threshold, and the lowest pages among those equal to
// it).  Past 32 keys per thread the rest sit in LDS ([key][thread], 128 KiB
// at 64 keys per thread), where registers would spill.
constexpr int kLongBlock = 1024;
constexpr int kLongWaves = kLongBlock / kWave;
constexpr int kLongRegKeys = 32;

template <int kLdsKeys>
struct TopkLongLds {
  uint32_t lk[kLdsKeys > 0 ? kLdsKeys * kLongBlock : 1];
  int hist[2][2048];
  int wsum[kLongWaves];
  int wsum2[kLongWaves];
  uint32_t mn[kLongWaves], mx[kLongWaves];
  int s_digit, s_above, s_cnt;
};

template <int kPer>
__global__ __launch_bounds__(kLongBlock) void topk_long_kernel(
    const float* __restrict__ ubg, const int32_t* __restrict__ lens, int P, int maxP, int Hkv,
    int top_k, int32_t* __restrict__ sel, int32_t* __restrict__ n_sel) {
  constexpr int kReg = kPer < kLongRegKeys ? kPer : kLongRegKeys;
  __shared__ TopkLongLds<kPer - kReg> sm;
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int pair = blockIdx.x;
  const int b = pair / Hkv;
  const int n = (lens[b] + P - 1) / P;
  const int k = min(top_k, n);
  int32_t* out = sel + (size_t)pair * maxP;
  if (tid == 0) n_sel[pair] = k;
  if (k >= n) {
    for (int p = tid; p < n; p += kLongBlock) out[p] = p;
    return;
  }
  const float* U = ubg + (size_t)pair * maxP;
  const int p0 = tid * kPer;
  const int nv = max(0, min(kPer, n - p0));
  // (16-byte loads of each thread's run where the row is aligned: lanes kPer
  // entries apart touch a cache line each per load instruction)
  uint32_t key[kReg];
  {
    float u[kReg];
    load_run<kReg>(U, p0, p0 + nv, u);
#pragma unroll
    for (int i = 0; i < kReg; ++i) key[i] = order_key(u[i]);
  }
  if constexpr (kPer > kReg) {
    float u[kPer - kReg];
    load_run<kPer - kReg>(U, p0 + kReg, p0 + nv, u);
#pragma unroll
    for (int i = 0; i < kPer - kReg; ++i) sm.lk[i * kLongBlock + tid] = order_key(u[i]);
  }
  // key i of this thread (registers, or LDS past kReg; i is a constant in
  // every unrolled use)
  auto key_at = [&](int i) -> uint32_t {
    return i < kReg ? key[i < kReg ? i : 0] : sm.lk[(i - kReg) * kLongBlock + tid];
  };
  for (int i = tid; i < 2 * 2048; i += kLongBlock) (&sm.hist[0][0])[i] = 0;
  uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    if (i < nv) {
      kmn = min(kmn, key_at(i));
      kmx = max(kmx, key_at(i));
    }
  kmn = wave_min_u32(kmn);
  kmx = wave_max_u32(kmx);
  if (lane == 0) {
    sm.mn[wave] = kmn;
    sm.mx[wave] = kmx;
  }
  __syncthreads();
  uint32_t lo = sm.mn[0], hi = sm.mx[0];
#pragma unroll
  for (int w = 1; w < kLongWaves; ++w) {
    lo = min(lo, sm.mn[w]);
    hi = max(hi, sm.mx[w]);
  }
  int remaining = k;
  bool cut = false;
  for (int pass = 0; pass < 4; ++pass) {
    int* hist = sm.hist[pass & 1];
    int* next = sm.hist[(pass + 1) & 1];
    const uint32_t span = hi - lo;
    const int width = span == 0u ? 0 : 32 - __clz((int)span);
    const int shift = width > 11 ? width - 11 : 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const uint32_t kk = key_at(i);
      if (i < nv && kk >= lo && kk <= hi) atomicAdd(&hist[(kk - lo) >> shift], 1);
    }
    __syncthreads();  // histogram complete
    const int2 h2 = *reinterpret_cast<const int2*>(hist + 2046 - 2 * tid);  // .y higher digit
    *reinterpret_cast<int2*>(next + 2046 - 2 * tid) = make_int2(0, 0);
    const int local = h2.x + h2.y;
    int incl = wave_incl_scan_i32(local);
    if (lane == kWave - 1) sm.wsum[wave] = incl;
    __syncthreads();  // wave totals
    for (int w = 0; w < wave; ++w) incl += sm.wsum[w];
    const int excl = incl - local;
    if (excl < remaining && remaining <= incl) {
      if (excl + h2.y >= remaining) {
        sm.s_digit = 2047 - 2 * tid;
        sm.s_above = excl;
        sm.s_cnt = h2.y;
      } else {
        sm.s_digit = 2046 - 2 * tid;
        sm.s_above = excl + h2.y;
        sm.s_cnt = h2.x;
      }
    }
    __syncthreads();  // chosen bin
    const int digit = sm.s_digit, above = sm.s_above, cnt = sm.s_cnt;
    const uint32_t nlo = lo + ((uint32_t)digit << shift);
    const uint32_t top = shift == 0 ? nlo : nlo + ((1u << shift) - 1u);
    hi = top < hi ? top : hi;
    lo = nlo;
    remaining -= above;
    cut = (cnt == remaining);
    if (cut || shift == 0) break;
  }
  // ordered placement: every key > T (>= T when the bin was cut whole), and
  // the first `remaining` keys equal to T in page order
  const uint32_t T = lo;
  int cg = 0, ce = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const bool v = i < nv;
    const uint32_t kk = key_at(i);
    cg += (v && (cut ? kk >= T : kk > T)) ? 1 : 0;
    ce += (v && !cut && kk == T) ? 1 : 0;
  }
  int gi = wave_incl_scan_i32(cg);
  int ei = wave_incl_scan_i32(ce);
  __syncthreads();  // every thread has read the last pass's wave totals
  if (lane == kWave - 1) {
    sm.wsum[wave] = gi;
    sm.wsum2[wave] = ei;
  }
  __syncthreads();
  for (int w = 0; w < wave; ++w) {
    gi += sm.wsum[w];
    ei += sm.wsum2[w];
  }
  int eq_seen = ei - ce;
  int pos = (gi - cg) + min(eq_seen, remaining);
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const bool v = i < nv;
    const uint32_t kk = key_at(i);
    const bool gt = v && (cut ? kk >= T : kk > T);
    const bool eq = v && !cut && kk == T;
    const bool take = gt || (eq && eq_seen < remaining);
    if (take) out[pos] = p0 + i;
    pos += take ? 1 : 0;
    eq_seen += eq ? 1 : 0;
  }
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

// --------------------------------------------------------------------------
// Non-integer gamma (1 < alpha < 2, alpha not 1 + 1/n): I_g for g = n + f,
// n = floor(g) >= 1, f in (0, 1), from the pair (I_f, I_{f+1}) by the
// recurrence above.  Per launch the pair is tabulated over h as Chebyshev
// series on short pieces, the values at the Chebyshev points coming from a
// quadrature of the defining integrals I_nu(h) = int_0^inf x^nu phi(x - h) dx.
// --------------------------------------------------------------------------
constexpr int kFracGj = 16;          // Gauss-Jacobi nodes on [0, 1], weight x^f
constexpr int kFracGl = 12;          // Gauss-Legendre nodes per panel beyond x = 1
constexpr double kFracPanel = 1.5;   // panel width beyond x = 1
constexpr double kFracHmin = -9.0;   // I_nu(h) < 1e-19 below: taken as 0
constexpr double kFracHmax = 8.5;    // asymptotic series from here on
constexpr double kFracPiece = 0.5;   // Chebyshev piece width in h
constexpr int kFracPieces = 35;      // (kFracHmax - kFracHmin) / kFracPiece
constexpr int kFracN = 17;           // Chebyshev points (degree 16) per piece

// Quadrature rules and exponents of one launch (built on the host).
struct FracRule {
  double gamma, f;  // gamma = n + f
  int n;
  double gj_x[kFracGj], gj_w[kFracGj];  // int_0^1 x^f g(x) dx ~ sum_i w_i g(x_i)
  double gl_x[kFracGl], gl_w[kFracGl];  // int_0^1 g(x) dx ~ sum_i w_i g(x_i)
};

// c[0]: I_f, c[1]: I_{f+1}; piece k covers h in kFracHmin + [k, k+1) kFracPiece
struct FracTable {
  double c[2][kFracPieces][kFracN];
};

// I_f(h) and I_{f+1}(h) by quadrature: [0, 1] by Gauss-Jacobi with the weight
// x^f (the factor that is not smooth at 0), then Gauss-Legendre panels of
// width 1.5 over [max(1, h - 10), max(h, 0) + 10]; the integrand is below
// phi(10) < 1e-22 of its peak outside.  About 4e-15 relative for h in
// [-9, 8.5] (checked against the oracle's adaptive quadrature).
__device__ inline void frac_quad(const FracRule& r, double h, double& i0, double& i1) {
  double a0 = 0.0, a1 = 0.0;
  for (int i = 0; i < kFracGj; ++i) {
    const double x = r.gj_x[i];
    const double ph = r.gj_w[i] * exp(-0.5 * (x - h) * (x - h));
    a0 += ph;
    a1 = fma(ph, x, a1);
  }
  const double lo = fmax(1.0, h - 10.0);
  const double hi = fmax(h, 0.0) + 10.0;
  for (int k = 0; lo + k * kFracPanel < hi; ++k) {
    const double c = lo + k * kFracPanel;
    const double w = fmin(kFracPanel, hi - c);
    for (int i = 0; i < kFracGl; ++i) {
      const double x = fma(w, r.gl_x[i], c);
      const double t = w * r.gl_w[i] * exp(fma(r.f, log(x), -0.5 * (x - h) * (x - h)));
      a0 += t;
      a1 = fma(t, x, a1);
    }
  }
  i0 = a0 * 0.39894228040143267794;
  i1 = a1 * 0.39894228040143267794;
}

// I_nu(h) for h >= 8.5 as E[(h + Z)^nu] (Z below -h weighs less than 1e-17):
// h^nu sum_j C(nu, 2j) (2j - 1)!! h^(-2j), an asymptotic series whose terms
// shrink while 2j < h^2; summed until a term is below 1e-17 of the sum.
__device__ inline double frac_asym(double nu, double h) {
  const double r = 1.0 / (h * h);
  double s = 1.0, t = 1.0;
  for (int j = 1; j < 40; ++j) {
    t *= (nu - 2 * j + 2) * (nu - 2 * j + 1) * (0.5 / j) * r;
    s += t;
    if (fabs(t) < 1e-17 * fabs(s)) break;
  }
  return exp(nu * log(h)) * s;
}

// The table of (I_f, I_{f+1}): values at the Chebyshev points of every piece
// (frac_quad, one point per thread), then their cosine transforms.  Called by
// all nthreads threads of the block; ends with a barrier.  val: LDS scratch.
__device__ inline void build_frac_table(const FracRule& r, FracTable& t, FracTable& val,
                                        int nthreads) {
  for (int i = threadIdx.x; i < kFracPieces * kFracN; i += nthreads) {
    const int k = i / kFracN, j = i % kFracN;
    const double h = kFracHmin + (k + 0.5) * kFracPiece +
                     0.5 * kFracPiece * cospi((j + 0.5) / kFracN);
    frac_quad(r, h, val.c[0][k][j], val.c[1][k][j]);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 2 * kFracPieces * kFracN; i += nthreads) {
    const int q = i / (kFracPieces * kFracN);
    const int k = (i / kFracN) % kFracPieces;
    const int m = i % kFracN;
    double a = 0.0;
    for (int j = 0; j < kFracN; ++j) a = fma(val.c[q][k][j], cospi(m * (j + 0.5) / kFracN), a);
    t.c[q][k][m] = (m == 0 ? 1.0 : 2.0) / kFracN * a;
  }
  __syncthreads();
}

// (I_f(h), I_{f+1}(h)) from the table (Clenshaw), the asymptotic series, or 0.
__device__ inline void frac_pair(const FracRule& r, const FracTable& t, double h, double& i0,
                                 double& i1) {
  if (h >= kFracHmax) {
    i0 = frac_asym(r.f, h);
    i1 = frac_asym(r.f + 1.0, h);
    return;
  }
  if (!(h >= kFracHmin)) {
    i0 = 0.0;
    i1 = 0.0;
    return;
  }
  const int k = min((int)((h - kFracHmin) * (1.0 / kFracPiece)), kFracPieces - 1);
  const double x = (h - (kFracHmin + (k + 0.5) * kFracPiece)) * (2.0 / kFracPiece);
  double b1 = 0.0, b2 = 0.0, d1 = 0.0, d2 = 0.0;
  for (int m = kFracN - 1; m >= 1; --m) {
    const double nb = fma(2.0 * x, b1, t.c[0][k][m] - b2);
    const double nd = fma(2.0 * x, d1, t.c[1][k][m] - d2);
    b2 = b1;
    b1 = nb;
    d2 = d1;
    d1 = nd;
  }
  i0 = fma(x, b1, t.c[0][k][0] - b2);
  i1 = fma(x, d1, t.c[1][k][0] - d2);
}

// I_g(h), I_{g-1}(h) and J = g (g-1) I_{g-2}(h) for g = n + f: the base pair
// (I_f, I_{f+1}) from the table, or (Phi, h Phi + phi) when f = 0 (an integer
// g above the unrolled ones), then upwards I_{nu+1} = h I_nu + nu I_{nu-1};
// I_{f-1} = (I_{f+1} - h I_f) / f is the same relation solved downwards.
__device__ inline void partial_moments_rt(const FracRule& r, const FracTable& t, double h,
                                          double& ig, double& igm1, double& jdd) {
  double b0, b1, bm1;
  if (r.f == 0.0) {
    b0 = 0.5 * erfc(-h * 0.70710678118654752440);
    bm1 = exp(-0.5 * h * h) * 0.39894228040143267794;
    b1 = fma(h, b0, bm1);
  } else {
    frac_pair(r, t, h, b0, b1);
    bm1 = (b1 - h * b0) / r.f;
  }
  double i_pp = bm1, i_prev = b0, i_cur = b1;
  for (int k = 2; k <= r.n; ++k) {
    const double nxt = fma(h, i_cur, (r.f + (double)(k - 1)) * i_prev);
    i_pp = i_prev;
    i_prev = i_cur;
    i_cur = nxt;
  }
  ig = i_cur;
  igm1 = i_prev;
  jdd = r.gamma * (r.gamma - 1.0) * i_pp;
}

// gauss_term for a runtime gamma (fp64).
__device__ inline void gauss_term_rt(const FracRule& r, const FracTable& t, double mz, double sd,
                                     double rs, double tau, double cnt, double& f, double& fd,
                                     double& fdd) {
  if (sd > 0.0) {
    const double h = (mz - tau) * rs;
    if (!(h >= kFracHmin) && r.f != 0.0) return;  // below fp64 resolution of F
    double ig, igm1, jdd;
    partial_moments_rt(r, t, h, ig, igm1, jdd);
    const double sg1 = exp((r.gamma - 1.0) * log(sd));
    f = fma(cnt, sg1 * sd * ig, f);
    fd = fma(cnt, r.gamma * sg1 * igm1, fd);
    fdd = fma(cnt, sg1 * rs * jdd, fdd);
  } else {
    const double x = mz - tau;
    if (x > 0.0) {
      const double xg2 = exp((r.gamma - 2.0) * log(x));
      f = fma(cnt, xg2 * x * x, f);
      fd = fma(cnt, r.gamma * xg2 * x, fd);
      fdd = fma(cnt, r.gamma * (r.gamma - 1.0) * xg2, fdd);
    }
  }
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
// kG = 0: a runtime gamma (fr), whose coarse run is in fp64 as well (the
// fp32 copies of the page statistics are then not kept).
template <int kG, bool kLds>
__global__ __launch_bounds__(kTauBlock) void gauss_tau_kernel(
    const double* __restrict__ gm, const double* __restrict__ gv, const int32_t* __restrict__ lens,
    int P, int maxP, int Hq, double a1, double* __restrict__ tau_hat, FracRule fr) {
  constexpr bool kLds32 = kLds && kG != 0;
  __shared__ double s_mu[kLds ? kGaussLdsPages : 1];
  __shared__ double s_sd[kLds ? kGaussLdsPages : 1];
  __shared__ float s_mu32[kLds32 ? kGaussLdsPages : 1];
  __shared__ float s_sd32[kLds32 ? kGaussLdsPages : 1];
  __shared__ double s_rs[kLds ? kGaussLdsPages : 1];
  __shared__ float s_rs32[kLds32 ? kGaussLdsPages : 1];
  __shared__ double red[6 * kTauWaves];
  __shared__ float redf[6 * kTauWaves];
  struct NoTable {};
  __shared__ std::conditional_t<kG == 0, FracTable, NoTable> s_ft, s_fv;
  const int bh = blockIdx.x;
  const int b = bh / Hq;
  const int L = lens[b];
  const int n = (L + P - 1) / P;
  if (n == 0) {  // empty row: no pages, no threshold
    if (threadIdx.x == 0) tau_hat[bh] = __builtin_nan("");
    return;
  }
  if constexpr (kG == 0) build_frac_table(fr, s_ft, s_fv, kTauBlock);
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
    if constexpr (kLds32) return s_mu32[p];
    else return (float)(a1 * M[p]);
  };
  auto sd32_of = [&](int p) -> float {
    if constexpr (kLds32) return s_sd32[p];
    else return (float)(a1 * sqrt(V[p]));
  };
  auto inv = [](auto x) -> decltype(x) { return x > 0 ? (decltype(x))1 / x : (decltype(x))0; };
  auto rs_of = [&](int p) -> double {
    if constexpr (kLds) return s_rs[p];
    else return inv(a1 * sqrt(V[p]));
  };
  auto rs32_of = [&](int p) -> float {
    if constexpr (kLds32) return s_rs32[p];
    else return inv((float)(a1 * sqrt(V[p])));
  };
  double zmax = -__builtin_huge_val();
  for (int p = threadIdx.x; p < n; p += kTauBlock) {
    const double mz = a1 * M[p];
    if constexpr (kLds) {
      const double sd = a1 * sqrt(V[p]);
      s_mu[p] = mz;
      s_sd[p] = sd;
      s_rs[p] = inv(sd);
      if constexpr (kLds32) {
        s_mu32[p] = (float)mz;
        s_sd32[p] = (float)sd;
        s_rs32[p] = inv((float)sd);
      }
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
    double fs, fds, nxt;
    if constexpr (kG != 0) {
      float f = 0.0f, fd = 0.0f, fdd = 0.0f;  // fdd unused here
      const float tf = (float)t;
      for (int p = threadIdx.x; p < n; p += kTauBlock)
        gauss_term<kG, false, float>(mu32_of(p), sd32_of(p), rs32_of(p), tf,
                                     (float)page_valid(L, p, P), f, fd, fdd);
      block_sum3(f, fd, fdd, redf, par);
      fs = f;
      fds = fd;
      nxt = fs > 0.0 && fds > 0.0 ? t + (double)(logf(f) * f / fd) : t;
    } else {
      double f = 0.0, fd = 0.0, fdd = 0.0;
      for (int p = threadIdx.x; p < n; p += kTauBlock)
        gauss_term_rt(fr, s_ft, mu_of(p), sd_of(p), rs_of(p), t, (double)page_valid(L, p, P), f,
                      fd, fdd);
      block_sum3(f, fd, fdd, red, par);
      fs = f;
      fds = fd;
      nxt = fs > 0.0 && fds > 0.0 ? t + log(f) * f / fd : t;
    }
    par ^= 1;
    if (fs >= 1.0) lo = fmax(lo, t);
    else hi = fmin(hi, t);
    const bool ok = fs > 0.0 && fds > 0.0;
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
    for (int p = threadIdx.x; p < n; p += kTauBlock) {
      if constexpr (kG != 0)
        gauss_term<kG, true, double>(mu_of(p), sd_of(p), rs_of(p), tau,
                                     (double)page_valid(L, p, P), f, fd, fdd);
      else
        gauss_term_rt(fr, s_ft, mu_of(p), sd_of(p), rs_of(p), tau, (double)page_valid(L, p, P),
                      f, fd, fdd);
    }
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
    ExpMaxTable et, int32_t* __restrict__ sel, int32_t* __restrict__ n_sel, FracRule fr) {
  constexpr bool kTable = kRule == kRuleMass && kG == 0;  // runtime gamma
  struct NoTable {};
  __shared__ std::conditional_t<kTable, FracTable, NoTable> s_ft, s_fv;
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
  if constexpr (kTable) build_frac_table(fr, s_ft, s_fv, kMarkBlock);
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
        if constexpr (kTable) {
          double ig = 0.0, igm1, jdd;
          if (sd > 0.0) {
            const double hh = (mz - th[h]) / sd;
            if (hh >= kFracHmin || fr.f == 0.0) partial_moments_rt(fr, s_ft, hh, ig, igm1, jdd);
            mass = cnt * (exp(fr.gamma * log(sd)) * ig);
          } else {
            const double x = mz - th[h];
            mass = x > 0.0 ? cnt * exp(fr.gamma * log(x)) : 0.0;
          }
        } else if (sd > 0.0) {
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
                            const double* gv, double* tau_hat, const FracRule& fr,
                            hipStream_t stream) {
  if (s.maxP <= kGaussLdsPages)
    hipLaunchKernelGGL((gauss_tau_kernel<kG, true>), dim3(s.B * s.Hq), dim3(kTauBlock), 0, stream,
                       gm, gv, lens, s.P, s.maxP, s.Hq, a1, tau_hat, fr);
  else
    hipLaunchKernelGGL((gauss_tau_kernel<kG, false>), dim3(s.B * s.Hq), dim3(kTauBlock), 0,
                       stream, gm, gv, lens, s.P, s.maxP, s.Hq, a1, tau_hat, fr);
  return hipGetLastError();
}

// Nodes and weights of the n-point Gauss-Jacobi rule for the weight
// (1 - y)^a (1 + y)^b on [-1, 1], by the Golub-Welsch method: the nodes are
// the eigenvalues of the symmetric tridiagonal Jacobi matrix of the
// orthonormal Jacobi polynomials, the weights mu0 times the squared first
// components of its unit eigenvectors.  The eigenproblem is solved by the
// implicit-shift QL iteration, carrying only the first row of the
// eigenvector matrix.  Returns false if it does not converge.
bool gauss_jacobi(int n, double a, double b, double* x, double* w) {
  double d[32], e[32], z[32];
  if (n < 1 || n > 32) return false;
  for (int i = 0; i < n; ++i) {
    const double s = 2.0 * i + a + b;
    d[i] = (s == 0.0) ? (b - a) / (a + b + 2.0) : (b * b - a * a) / (s * (s + 2.0));
    if (i + 1 < n) {
      const double k = i + 1.0;
      const double t = 2.0 * k + a + b;
      e[i] = sqrt(4.0 * k * (k + a) * (k + b) * (k + a + b) / (t * t * (t + 1.0) * (t - 1.0)));
    } else {
      e[i] = 0.0;
    }
    z[i] = i == 0 ? 1.0 : 0.0;
  }
  for (int l = 0; l < n; ++l) {
    int iter = 0;
    int m;
    do {
      for (m = l; m < n - 1; ++m) {
        const double dd = fabs(d[m]) + fabs(d[m + 1]);
        if (fabs(e[m]) <= 1e-17 * dd) break;
      }
      if (m != l) {
        if (++iter > 60) return false;
        double g = (d[l + 1] - d[l]) / (2.0 * e[l]);
        double r = hypot(g, 1.0);
        g = d[m] - d[l] + e[l] / (g + (g >= 0.0 ? r : -r));
        double s = 1.0, c = 1.0, p = 0.0;
        int i;
        for (i = m - 1; i >= l; --i) {
          double f = s * e[i];
          const double bb = c * e[i];
          r = hypot(f, g);
          e[i + 1] = r;
          if (r == 0.0) {
            d[i + 1] -= p;
            e[m] = 0.0;
            break;
          }
          s = f / r;
          c = g / r;
          g = d[i + 1] - p;
          r = (d[i] - g) * s + 2.0 * c * bb;
          p = s * r;
          d[i + 1] = g + p;
          g = c * r - bb;
          // the first component of eigenvectors i and i + 1
          f = z[i + 1];
          z[i + 1] = s * z[i] + c * f;
          z[i] = c * z[i] - s * f;
        }
        if (r == 0.0 && i >= l) continue;
        d[l] -= p;
        e[l] = g;
        e[m] = 0.0;
      }
    } while (m != l);
  }
  const double mu0 = exp((a + b + 1.0) * log(2.0) + lgamma(a + 1.0) + lgamma(b + 1.0) -
                         lgamma(a + b + 2.0));
  // ascending nodes
  int idx[32];
  for (int i = 0; i < n; ++i) idx[i] = i;
  for (int i = 1; i < n; ++i)
    for (int j = i; j > 0 && d[idx[j]] < d[idx[j - 1]]; --j) {
      const int t = idx[j];
      idx[j] = idx[j - 1];
      idx[j - 1] = t;
    }
  double sw = 0.0;
  for (int i = 0; i < n; ++i) {
    x[i] = d[idx[i]];
    w[i] = mu0 * z[idx[i]] * z[idx[i]];
    sw += w[i];
  }
  return fabs(sw - mu0) <= 1e-12 * mu0;
}

// The quadrature rules of a runtime gamma, mapped to [0, 1]:
// int_0^1 x^f g dx = 2^(-f-1) int_{-1}^1 (1 + y)^f g((1 + y) / 2) dy.
bool make_frac_rule(double gamma, FracRule& r) {
  r.gamma = gamma;
  r.n = (int)floor(gamma);
  r.f = gamma - r.n;
  double y[32], w[32];
  if (r.f > 0.0) {
    if (!gauss_jacobi(kFracGj, 0.0, r.f, y, w)) return false;
    const double sc = exp(-(r.f + 1.0) * log(2.0));
    for (int i = 0; i < kFracGj; ++i) {
      r.gj_x[i] = 0.5 * (1.0 + y[i]);
      r.gj_w[i] = sc * w[i];
    }
  } else {
    for (int i = 0; i < kFracGj; ++i) r.gj_x[i] = r.gj_w[i] = 0.0;
  }
  if (!gauss_jacobi(kFracGl, 0.0, 0.0, y, w)) return false;
  for (int i = 0; i < kFracGl; ++i) {
    r.gl_x[i] = 0.5 * (1.0 + y[i]);
    r.gl_w[i] = 0.5 * w[i];
  }
  return true;
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
                   const FracRule& fr, hipStream_t stream) {
  hipLaunchKernelGGL((gauss_mark_kernel<kRule, G, kG>), dim3(s.B * s.Hkv), dim3(kMarkBlock), 0,
                     stream, ub, ubg, gm, gv, tau_hat, lens, s.P, s.maxP, s.Hkv, a1, delta, et,
                     sel, n_sel, fr);
}

// gamma: 1 .. 4, or 0 for a runtime gamma (fr)
template <int G>
hipError_t launch_mark(const Shape& s, int rule, int gamma, const float* ub, const float* ubg,
                       const double* gm, const double* gv, const double* tau_hat,
                       const int32_t* lens, double a1, double delta, const ExpMaxTable& et,
                       int32_t* sel, int32_t* n_sel, const FracRule& fr, hipStream_t stream) {
#define EKV_MARK(R, KG) \
  launch_mark_t<R, G, KG>(s, ub, ubg, gm, gv, tau_hat, lens, a1, delta, et, sel, n_sel, fr, stream)
  if (rule == kRuleBound) {
    EKV_MARK(kRuleBound, 1);
  } else if (rule == kRuleEstMax) {
    EKV_MARK(kRuleEstMax, 1);
  } else {
    switch (gamma) {
      case 0: EKV_MARK(kRuleMass, 0); break;
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
  const dim3 g((unsigned)(s.B * s.Hkv));
  if (s.maxP > kBlk * 16 && s.maxP <= kLongBlock * 64) {
    if (s.maxP <= kLongBlock * 16)
      hipLaunchKernelGGL((topk_long_kernel<16>), g, dim3(kLongBlock), 0, stream, ubg, lens, s.P,
                         s.maxP, s.Hkv, top_k, sel, n_sel);
    else if (s.maxP <= kLongBlock * 32)
      hipLaunchKernelGGL((topk_long_kernel<32>), g, dim3(kLongBlock), 0, stream, ubg, lens, s.P,
                         s.maxP, s.Hkv, top_k, sel, n_sel);
    else
      hipLaunchKernelGGL((topk_long_kernel<64>), g, dim3(kLongBlock), 0, stream, ubg, lens, s.P,
                         s.maxP, s.Hkv, top_k, sel, n_sel);
    return hipGetLastError();
  }
  if (s.maxP <= kTopkLdsKeys)
    hipLaunchKernelGGL((topk_kernel<true>), dim3(s.B * s.Hkv), dim3(kSelBlock), 0, stream, ubg,
                       lens, s.P, s.maxP, s.Hkv, top_k, sel, n_sel);
  else
    hipLaunchKernelGGL((topk_kernel<false>), dim3(s.B * s.Hkv), dim3(kSelBlock), 0, stream, ubg,
                       lens, s.P, s.maxP, s.Hkv, top_k, sel, n_sel);
  return hipGetLastError();
}

hipError_t launch_gauss(const Shape& s, const int32_t* lens, float alpha, double gamma,
                        float delta, int rule, const float* ub, const float* ubg,
                        const double* gm, const double* gv, int32_t* sel, int32_t* n_sel,
                        double* tau_hat, hipStream_t stream) {
  const double a1 = (double)alpha - 1.0;
  // gamma 1 .. 4: the unrolled recurrences; any other gamma >= 1 at run time
  const int gi = (gamma == 1.0 || gamma == 2.0 || gamma == 3.0 || gamma == 4.0) ? (int)gamma : 0;
  FracRule fr{};
  if (gi == 0) {
    if (!(gamma >= 1.0) || !make_frac_rule(gamma, fr)) return hipErrorInvalidValue;
  }
  hipError_t e = hipErrorInvalidValue;
  switch (gi) {
    case 0: e = launch_gauss_tau<0>(s, lens, a1, gm, gv, tau_hat, fr, stream); break;
    case 1: e = launch_gauss_tau<1>(s, lens, a1, gm, gv, tau_hat, fr, stream); break;
    case 2: e = launch_gauss_tau<2>(s, lens, a1, gm, gv, tau_hat, fr, stream); break;
    case 3: e = launch_gauss_tau<3>(s, lens, a1, gm, gv, tau_hat, fr, stream); break;
    case 4: e = launch_gauss_tau<4>(s, lens, a1, gm, gv, tau_hat, fr, stream); break;
  }
  if (e != hipSuccess) return e;
  const ExpMaxTable& et = exp_max_table();
  switch (s.G) {
    case 1: e = launch_mark<1>(s, rule, gi, ub, ubg, gm, gv, tau_hat, lens, a1, delta, et, sel, n_sel, fr, stream); break;
    case 2: e = launch_mark<2>(s, rule, gi, ub, ubg, gm, gv, tau_hat, lens, a1, delta, et, sel, n_sel, fr, stream); break;
    case 4: e = launch_mark<4>(s, rule, gi, ub, ubg, gm, gv, tau_hat, lens, a1, delta, et, sel, n_sel, fr, stream); break;
    case 8: e = launch_mark<8>(s, rule, gi, ub, ubg, gm, gv, tau_hat, lens, a1, delta, et, sel, n_sel, fr, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace ekv
