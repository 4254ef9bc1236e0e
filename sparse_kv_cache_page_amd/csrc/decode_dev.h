// Device code of the sparse alpha-entmax decode (EntmaxKV summary page, §2.C),
// shared by the decode kernels and the persistent decode-step kernel: the qk
// work item, the tau / PV head and their helpers.
#pragma once

#include <type_traits>

#include "blocks.h"

namespace ekv {
namespace {


constexpr int kBlock = 256;
constexpr int kRowsPerThread = 16;  // K rows each thread has in flight per item
constexpr int kCandCap = 2048;      // LDS candidates per head; more falls back to global
constexpr int kMaxSplits = 2048;    // splits per head whose offsets fit in LDS at once
constexpr int kMaxSplitsTotal = 65536;  // splits per head (16M token slots at 256 a split)

template <typename T, int D>
struct Geo {
  static constexpr int kVec = Elem<T>::kVec;
  static constexpr int kLpr = D / kVec;                 // lanes per K row
  static constexpr int kRowsPerPass = kBlock / kLpr;    // rows per block-wide load
  static constexpr int kR = kRowsPerPass * kRowsPerThread;  // token slots per item
};

__device__ inline int bits_of(float x) { return __float_as_int(x); }

constexpr int kTailCap = 512;  // LDS candidates per head in the fused tail

// Everything the fused tau / PV tail needs beyond the qk arguments.
template <typename T>
struct TailArgs {
  const T* V;
  int* counters;      // [B*Hkv] arrival counters, zero between launches
  double alpha, gamma;
  int gamma_int;
  float* out;
  float* tau_out;
  int32_t* n_support;
};

struct TailLds {
  float cz[kBlock / kWave][kTailCap];
  int ct[kBlock / kWave][kTailCap];
  int offs[kBlock / kWave][kWave + 1];
  float sp[kBlock / kWave][kWave];
  int st[kBlock / kWave][kWave];
};

__device__ inline uint64_t pack_cand(float z, int ptok) {
  return ((uint64_t)(uint32_t)ptok << 32) | (uint64_t)__float_as_uint(z);
}

// fp64 power for the non-integer exponents; out of line, so that its code and
// constants do not occupy registers in the kernels' hot paths.
__device__ __attribute__((noinline)) double pow_ool(double x, double y) { return pow(x, y); }

__device__ inline double pos_pow(double x, double gamma, int gi) {
  // x > 0
  if (gi > 0) {
    double r = x;
    for (int i = 1; i < gi; ++i) r *= x;
    return r;
  }
  return pow_ool(x, gamma);
}

__device__ inline int wave_incl_scan_i(int x) { return wave_incl_scan_i32(x); }

// Bracketed Newton for f(tau) = sum [z - tau]_+^gamma - 1 = 0 on
// [zmax - 1, zmax - n^(1-alpha)]; eval(tau, f, fd) returns the (uniform)
// sums f = sum [z - tau]_+^gamma and fd = gamma sum [z - tau]_+^(gamma-1).
template <typename Eval>
__device__ inline double newton_tau(double zmax, double nvalid, double alpha, Eval&& eval) {
  double lo = zmax - 1.0;
  double hi = zmax - pow_ool(nvalid, 1.0 - alpha);
  if (hi < lo) hi = lo;
  double tau = lo;
  for (int it = 0; it < 200; ++it) {
    double f, fd;
    eval(tau, f, fd);
    f -= 1.0;
    if (f == 0.0) break;
    if (f > 0.0) lo = tau;
    else hi = tau;
    double nt = fd > 0.0 ? tau + f / fd : 0.5 * (lo + hi);
    // a Newton step below fp64 resolution means converged (checked before the
    // bracket test, which would otherwise turn it into a bisection jump)
    if (fd > 0.0 && fabs(nt - tau) <= 4e-16 * fmax(1.0, fabs(tau))) {
      tau = nt > lo && nt < hi ? nt : tau;
      break;
    }
    if (!(nt > lo && nt < hi)) {
      nt = 0.5 * (lo + hi);
      if (!(nt > lo && nt < hi)) break;
    }
    tau = nt;
  }
  return tau;
}

__device__ inline void tau_term(double z, double tau, double gamma, int gamma_int, double& f,
                                double& fd) {
  const double x = z - tau;
  if (x > 0.0) {
    const double xg1 = gamma_int == 1 ? 1.0 : pos_pow(x, gamma - 1.0, gamma_int - 1);
    f += xg1 * x;
    fd += gamma * xg1;
  }
}

// x^gamma for x >= 0, with gamma a compile-time positive integer kGi, or any
// gamma > 0 when kGi == 0.
template <int kGi>
__device__ inline double powg(double x, double gamma) {
  if constexpr (kGi == 0) {
    return x > 0.0 ? pow_ool(x, gamma) : 0.0;
  } else {
    double r = x;
#pragma unroll
    for (int i = 1; i < kGi; ++i) r *= x;
    return r;
  }
}

// tau of at most 64 candidates, one per lane of the calling wave (z = -inf
// in lanes >= count; thr = z_max - 1).  With F(t) = sum_j [z_j - t]_+^gamma,
// which decreases and equals 1 at tau, candidate i is in the support exactly
// when F(z_i) < 1, so every lane evaluates F at its own candidate.  On the
// support S, F is the smooth sum_S (z - t)^gamma: solved in closed form for
// gamma = 1 (mean) and gamma = 2 (mean and variance), otherwise by Newton
// from the largest score below the support, where the convex, decreasing F
// makes the iterates rise monotonically to the root.  Returns false when the
// tau found disagrees with S (a score within rounding of tau) or gamma < 1;
// the caller then uses the bracketed solver.
template <int kGi>
__device__ inline bool tau_small_t(float zf, int count, double thr, double gamma,
                                   double& tau_out) {
  const int lane = threadIdx.x % kWave;
  const double z = (double)zf;
  double F0 = 0.0, F1 = 0.0;
  int j = 0;
  for (; j + 1 < count; j += 2) {
    const double x0 = (double)__int_as_float(__builtin_amdgcn_readlane(__float_as_int(zf), j)) - z;
    const double x1 = (double)__int_as_float(__builtin_amdgcn_readlane(__float_as_int(zf), j + 1)) - z;
    F0 += powg<kGi>(fmax(x0, 0.0), gamma);
    F1 += powg<kGi>(fmax(x1, 0.0), gamma);
  }
  if (j < count) {
    const double x0 = (double)__int_as_float(__builtin_amdgcn_readlane(__float_as_int(zf), j)) - z;
    F0 += powg<kGi>(fmax(x0, 0.0), gamma);
  }
  const double F = F0 + F1;
  const bool live = lane < count;
  const bool in = live && F < 1.0;
  const int k = __popcll(__ballot(in));
  if (k == 0) return false;
  double tau;
  if constexpr (kGi == 1) {
    tau = (wave_sum_f64(in ? z : 0.0) - 1.0) / k;
  } else if constexpr (kGi == 2) {
    const double m = wave_sum_f64(in ? z : 0.0) / k;
    const double v = wave_sum_f64(in ? (z - m) * (z - m) : 0.0);
    tau = m - sqrt(fmax(0.0, (1.0 - v) / k));
  } else {
    if (!(gamma >= 1.0)) return false;  // F is convex only for gamma >= 1
    const double below = (double)wave_max_f32(live && !in ? zf : -__builtin_huge_valf());
    tau = fmax(thr, below);
    for (int it = 0; it < 64; ++it) {
      const double x = in ? fmax(z - tau, 0.0) : 0.0;
      const double xg1 = kGi > 0 ? powg<(kGi > 1 ? kGi - 1 : 1)>(x, gamma - 1.0)
                                 : (x > 0.0 ? pow_ool(x, gamma - 1.0) : 0.0);
      const double f = wave_sum_f64(xg1 * x) - 1.0;
      const double fd = gamma * wave_sum_f64(xg1);
      if (!(fd > 0.0)) break;
      const double step = f / fd;
      tau += step;
      if (fabs(step) <= 4e-16 * fmax(1.0, fabs(tau))) break;
    }
  }
  const bool bad = live && (in ? !(z > tau) : (z > tau));
  if (__ballot(bad) != 0ull || !(tau >= thr)) return false;
  tau_out = tau;
  return true;
}

__device__ inline bool tau_small(float zf, int count, double thr, double gamma, int gi,
                                 double& tau_out) {
  switch (gi) {
    case 1: return tau_small_t<1>(zf, count, thr, gamma, tau_out);
    case 2: return tau_small_t<2>(zf, count, thr, gamma, tau_out);
    case 3: return tau_small_t<3>(zf, count, thr, gamma, tau_out);
    case 4: return tau_small_t<4>(zf, count, thr, gamma, tau_out);
    default: return tau_small_t<0>(zf, count, thr, gamma, tau_out);
  }
}

// The tau / PV tail of one (row b, KV head g), run by the last workgroup to
// finish that pair's qk items; wave w handles query heads w, w+4, ...  All
// cross-workgroup data is read with device-coherent loads.
template <typename T, int D, int G>
__device__ __forceinline__ void pair_tail(const float2* __restrict__ cand,
                                          const int* __restrict__ cnt,
                                          const float* __restrict__ smax, int splits,
                                          const TailArgs<T>& ta, int b, int g, int Hkv, int P,
                                          int log2P, int L, int nsel, int nsel_raw, int max_sel,
                                          bool has_sel, TailLds& tl) {
  using GE = Geo<T, D>;
  constexpr int kVec = GE::kVec, kLpr = GE::kLpr, kR = GE::kR;
  constexpr int kRowsW = kWave / kLpr;  // value rows per wave pass
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int Hq = Hkv * G;
  const size_t tile_stride = (size_t)P * D;
  const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (kWave - lane));
  float* cz = tl.cz[wave];
  int* ct = tl.ct[wave];
  int* offs = tl.offs[wave];
  for (int h = wave; h < G; h += kBlock / kWave) {
    const size_t bh = (size_t)b * Hq + g * G + h;
    if (nsel_raw > max_sel || nsel_raw < 1) {
      for (int t = lane; t < D; t += kWave) ta.out[bh * D + t] = __builtin_nanf("");
      if (lane == 0) {
        if (ta.tau_out) ta.tau_out[bh] = __builtin_nanf("");
        if (ta.n_support) ta.n_support[bh] = -1;
      }
      continue;
    }
    const int nsplit = ((nsel << log2P) + kR - 1) / kR;
    const float* smax_bh = smax + bh * splits;
    const int* cnt_bh = cnt + bh * splits;
    const uint64_t* cand_bh = reinterpret_cast<const uint64_t*>(cand) + bh * splits * kR;
    float zm = -__builtin_huge_valf();
    for (int s = lane; s < nsplit; s += kWave)
      zm = fmaxf(zm, __hip_atomic_load(smax_bh + s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    zm = wave_max_f32(zm);
    const double zmax = (double)zm;
    const double thr = zmax - 1.0;

    // walk every split's candidates in split order, 64 at a time; fn(z, ptok,
    // keep) is called by the whole wave, keep = the candidate clears zmax - 1
    auto walk = [&](auto&& fn) {
      for (int s0 = 0; s0 < nsplit; s0 += kWave) {
        const int s = s0 + lane;
        const int c = s < nsplit ? __hip_atomic_load(cnt_bh + s, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT) : 0;
        const int incl = wave_incl_scan_i(c);
        const int tot = __shfl(incl, kWave - 1, kWave);
        offs[lane] = incl - c;
        if (lane == kWave - 1) offs[kWave] = incl;
        __builtin_amdgcn_wave_barrier();
        for (int k0 = 0; k0 < tot; k0 += kWave) {
          const int k = k0 + lane;
          float z = -__builtin_huge_valf();
          int ptok = 0;
          if (k < tot) {
            int lo = 0, hi = kWave;  // offs[lo] <= k < offs[hi]
            while (hi - lo > 1) {
              const int mid = (lo + hi) >> 1;
              if (offs[mid] <= k) lo = mid;
              else hi = mid;
            }
            const uint64_t e = __hip_atomic_load(cand_bh + (size_t)(s0 + lo) * kR + (k - offs[lo]),
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            z = __uint_as_float((uint32_t)e);
            ptok = (int)(e >> 32);
          }
          fn(z, ptok, (double)z > thr);
        }
        __builtin_amdgcn_wave_barrier();
      }
    };
    int count = 0;
    walk([&](float z, int ptok, bool keep) {
      const uint64_t mask = __ballot(keep);
      const int pos = count + __popcll(mask & lt);
      if (keep && pos < kTailCap) {
        cz[pos] = z;
        ct[pos] = ptok;
      }
      count += __popcll(mask);
    });
    __builtin_amdgcn_wave_barrier();
    const bool overflow = count > kTailCap;
    const double nvalid = has_sel ? (double)nsel * P : (double)L;
    double tau;
    if (!(count <= kWave &&
          tau_small(lane < count ? cz[lane] : -__builtin_huge_valf(), count, thr, ta.gamma,
                    ta.gamma_int, tau)))
    tau = newton_tau(zmax, nvalid, ta.alpha, [&](double tt, double& f, double& fd) {
      f = 0.0;
      fd = 0.0;
      if (!overflow) {
        for (int c = lane; c < count; c += kWave) tau_term((double)cz[c], tt, ta.gamma, ta.gamma_int, f, fd);
      } else {
        walk([&](float z, int, bool keep) {
          if (keep) tau_term((double)z, tt, ta.gamma, ta.gamma_int, f, fd);
        });
      }
      f = wave_sum_f64(f);
      fd = wave_sum_f64(fd);
    });

    // weights and the value rows of the support, 64 candidates at a time
    float acc[kVec];
#pragma unroll
    for (int v = 0; v < kVec; ++v) acc[v] = 0.0f;
    double psum = 0.0;
    int nsupp = 0;
    const int c_in = lane % kLpr;
    const int rsub = lane / kLpr;
    float* sp = tl.sp[wave];
    int* st = tl.st[wave];
    auto pv_group = [&](float z, int ptok, bool keep) {
      const double x = (double)z - tau;
      const bool flag = keep && x > 0.0;
      const uint64_t mask = __ballot(flag);
      const int m = __popcll(mask);
      if (flag) {
        const float p = (float)pos_pow(x, ta.gamma, ta.gamma_int);
        sp[__popcll(mask & lt)] = p;
        st[__popcll(mask & lt)] = ptok;
        psum += (double)p;
      }
      nsupp += m;
      __builtin_amdgcn_wave_barrier();
      for (int r0 = 0; r0 < m; r0 += kRowsW) {
        const int r = r0 + rsub;
        if (r < m) {
          const int pt = st[r];
          const float p = sp[r];
          const T* row = ta.V + (size_t)(pt >> log2P) * Hkv * tile_stride + g * tile_stride +
                         (size_t)(pt & (P - 1)) * D + c_in * kVec;
          float xv[kVec];
          Elem<T>::unpack(load16(row), xv);
#pragma unroll
          for (int v = 0; v < kVec; ++v) acc[v] = fmaf(p, xv[v], acc[v]);
        }
      }
      __builtin_amdgcn_wave_barrier();
    };
    if (!overflow) {
      for (int k0 = 0; k0 < count; k0 += kWave) {
        const int k = k0 + lane;
        pv_group(k < count ? cz[k] : -__builtin_huge_valf(), k < count ? ct[k] : 0, k < count);
      }
    } else {
      walk(pv_group);
    }
#pragma unroll
    for (int o = kLpr; o < kWave; o <<= 1) {
#pragma unroll
      for (int v = 0; v < kVec; ++v) acc[v] += __shfl_xor(acc[v], o, kWave);
    }
    const double ps = wave_sum_f64(psum);
    const float inv = (float)(1.0 / ps);
    if (lane < kLpr) {
      float* o = ta.out + bh * D + c_in * kVec;
#pragma unroll
      for (int v = 0; v < kVec; v += 4)
        *reinterpret_cast<float4*>(o + v) =
            make_float4(acc[v] * inv, acc[v + 1] * inv, acc[v + 2] * inv, acc[v + 3] * inv);
    }
    if (lane == 0) {
      if (ta.tau_out) ta.tau_out[bh] = (float)tau;
      if (ta.n_support) ta.n_support[bh] = nsupp;
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// Sum two doubles over the block (fixed order, so results are reproducible).
__device__ inline void block_sum2(double& a, double& b, double* sh) {
  a = wave_sum_f64(a);
  b = wave_sum_f64(b);
  const int w = threadIdx.x / kWave;
  if (threadIdx.x % kWave == 0) {
    sh[2 * w] = a;
    sh[2 * w + 1] = b;
  }
  __syncthreads();
  a = (sh[0] + sh[2]) + (sh[4] + sh[6]);
  b = (sh[1] + sh[3]) + (sh[5] + sh[7]);
  __syncthreads();
}

// Ballot compaction of one 256-wide chunk: returns this thread's slot (or -1)
// and the chunk total through `total`.
__device__ inline int chunk_slot(bool flag, int* sh4, int& total) {
  const uint64_t m = __ballot(flag);
  const int lane = threadIdx.x % kWave;
  const int w = threadIdx.x / kWave;
  const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (kWave - lane));
  const int before = __popcll(m & lt);
  if (lane == 0) sh4[w] = __popcll(m);
  __syncthreads();
  int off = 0;
  for (int i = 0; i < w; ++i) off += sh4[i];
  total = (sh4[0] + sh4[1]) + (sh4[2] + sh4[3]);
  __syncthreads();
  return flag ? off + before : -1;
}

// Candidate k of a head, in split order: split by binary search over the
// exclusive offsets s_off[0..nsplit] held in LDS.
__device__ inline float2 cand_at(const float2* __restrict__ cand_bh, const int* s_off, int nsplit,
                                 int kR, int k) {
  int lo = 0, hi = nsplit;  // s_off[lo] <= k < s_off[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_off[mid] <= k) lo = mid;
    else hi = mid;
  }
  return cand_bh[(size_t)lo * kR + (k - s_off[lo])];
}

// Arguments of the qk stage (one (row, KV head, split) work item each).
template <typename T>
struct QkArgs {
  const float* q;
  float zscale;
  const T* K;
  const int32_t* bt;
  const int32_t* lens;
  const int32_t* sel;
  const int32_t* n_sel;
  int max_sel, Hkv, P, log2P, maxP, splits;
  float2* cand;
  int* cnt;
  float* smax;
  // page pruning (both set, or both NULL): per-head page bounds and per-head
  // lower bounds of z_max over the selected tokens
  const float* ub;
  const float* zlb;
  float a1;  // alpha - 1
  int npairs;  // B * Hkv
};

// A selected page whose tokens cannot reach z_max - 1 for any head of the
// group carries no weight (tau >= z_max - 1): its keys need not be read.  The
// test uses z <= (alpha-1) u (the page's box bound) and z_max >= zlb, with
// slack for the fp32 rounding of u and of the key scores (s1) and of zlb
// against the scores the qk stage computes (s2), so a pruned token would have
// been below every head's z_max - 1 in the unpruned computation too.
// The test is split in its two sides: support_bar(zlb) = zlb - 1 - s2 depends
// on the head only, so a page tested against several heads compares its one
// left side with the smallest bar (a NaN bar keeps every page, as a NaN
// comparison does in the per-head form).
__device__ inline float support_bar(float zlb) {
  const float s2 = 1e-4f * (1.0f + fabsf(zlb));
  return zlb - 1.0f - s2;
}
__device__ inline bool page_below_bar(float a1u, float bar) {
  const float s1 = 1e-3f * (1.0f + fabsf(a1u));
  return a1u + s1 < bar;
}
__device__ inline bool page_below_support(float a1u, float zlb) {
  return page_below_bar(a1u, support_bar(zlb));
}

template <typename T, int D, int G, bool kMfma = std::is_same<T, bf16_t>::value>
struct QkLds {
  static constexpr int kR = Geo<T, D>::kR;
  float zl[G][kR];
  int pg_phys[kR + 1];
  int pg_valid[kR + 1];
  __attribute__((aligned(16))) uint16_t qparts[kMfma ? G : 1][3][kMfma ? D : 8];
};

// Scores of the token slots [r_begin, r_end) of an item for the G heads of a
// group into sm.zl[h][r - r_begin]: slot r is token r & (P-1) of page-map
// entry (r >> log2P) - j_begin (physical page sm.pg_phys, valid tokens
// sm.pg_valid; a token at or past the valid count gets -inf and is not read).
// qg: the group's queries [G][D]; qv: for the matrix-core path, this thread's
// elements idx = threadIdx.x + u * kBlock of qg, loaded by the caller (so the
// load can share an earlier round trip).  Called by all threads; ends with a
// barrier (zl complete).
template <typename T, int D, int G, bool kMfma>
__device__ __forceinline__ void qk_score_slots(const float* __restrict__ qg,
                                               const float (&qv)[kMfma ? (G * D + kBlock - 1) / kBlock : 1],
                                               float zscale, const T* __restrict__ K, int Hkv,
                                               int g, int P, int log2P, int r_begin, int r_end,
                                               int j_begin, QkLds<T, D, G, kMfma>& sm) {
  using GE = Geo<T, D>;
  constexpr int kVec = GE::kVec, kLpr = GE::kLpr, kRowsPerPass = GE::kRowsPerPass, kR = GE::kR;
  constexpr int kQPer = (G * D + kBlock - 1) / kBlock;
  auto& zl = sm.zl;
  auto& pg_phys = sm.pg_phys;
  auto& pg_valid = sm.pg_valid;
  auto& qparts = sm.qparts;
  const int c = threadIdx.x % kLpr;
  const int rg = threadIdx.x / kLpr;
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const size_t tile_stride = (size_t)P * D;
  (void)kQPer;
  (void)qparts;
  (void)lane;
  if constexpr (kMfma) {
    // ---- matrix cores: [16 tokens x d] . [d x (G heads x 3 bf16 parts)] ----
    // A rows m = 4*head + part hold q split exactly into three bf16 parts
    // (hi, mid, lo; part 3 is zero), B = K^T of 16 tokens.  Lane l ends with
    // the partial scores of head l/16 (+4 for the second A block) for token
    // l%16 in its 4 accumulators; their sum is the fp32 score.
    constexpr int kKK = D / 32;                            // k steps of 32 dims
    constexpr int kBlocksA = G > 4 ? 2 : 1;
    constexpr int kGroups = kR / 16;                       // 16-token groups per item
    constexpr int kGPW = kGroups / (kBlock / kWave);       // groups per wave
    const int mrow = lane % 16;
    const int kq = lane / 16;
    // split q once per workgroup: qparts[h][part][dim] (bf16 bits)
#pragma unroll
    for (int u = 0; u < kQPer; ++u) {
      const int idx = threadIdx.x + u * kBlock;
      if (idx >= G * D) break;
      const int h = idx / D, dd = idx % D;
      const float x = qv[u];
      const float hi = bf16_round(x);
      const float mid = bf16_round(x - hi);
      const float lo = bf16_round(x - hi - mid);
      qparts[h][0][dd] = (uint16_t)(__float_as_uint(hi) >> 16);
      qparts[h][1][dd] = (uint16_t)(__float_as_uint(mid) >> 16);
      qparts[h][2][dd] = (uint16_t)(__float_as_uint(lo) >> 16);
    }
    __syncthreads();
    bf16x8_t qa[kBlocksA][kKK];
#pragma unroll
    for (int ab = 0; ab < kBlocksA; ++ab) {
      const int h = ab * 4 + mrow / 4;
      const int part = mrow % 4;
#pragma unroll
      for (int kk = 0; kk < kKK; ++kk) {
        uint4 w = make_uint4(0u, 0u, 0u, 0u);
        if (h < G && part < 3) w = *reinterpret_cast<const uint4*>(&qparts[h][part][kk * 32 + kq * 8]);
        qa[ab][kk] = as_bf16x8(w);
      }
    }

    uint4 kb[kGPW][kKK];
    bool valid[kGPW];
#pragma unroll
    for (int u = 0; u < kGPW; ++u) {
      const int grp = wave * kGPW + u;
      const int r = r_begin + grp * 16 + mrow;
      valid[u] = false;
#pragma unroll
      for (int kk = 0; kk < kKK; ++kk) kb[u][kk] = make_uint4(0u, 0u, 0u, 0u);
      if (r < r_end) {
        const int jl = (r >> log2P) - j_begin;
        const int t = r & (P - 1);
        if (t < pg_valid[jl]) {
          valid[u] = true;
          const T* row = K + (size_t)pg_phys[jl] * Hkv * tile_stride + g * tile_stride +
                         (size_t)t * D + kq * 8;
#pragma unroll
          for (int kk = 0; kk < kKK; ++kk) kb[u][kk] = load16_stream(row + kk * 32);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kGPW; ++u) {
      const int rl = (wave * kGPW + u) * 16 + mrow;  // slot inside the item
#pragma unroll
      for (int ab = 0; ab < kBlocksA; ++ab) {
        f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < kKK; ++kk)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ab][kk], as_bf16x8(kb[u][kk]), acc,
                                                        0, 0, 0);
        const int h = ab * 4 + kq;
        if (h < G)
          zl[h][rl] = valid[u] ? ((acc[0] + acc[1]) + acc[2]) * zscale : -__builtin_huge_valf();
      }
    }
    __syncthreads();
  } else {
  float qf[G][kVec];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float4* qh = reinterpret_cast<const float4*>(qg + (size_t)h * D + c * kVec);
#pragma unroll
    for (int v4 = 0; v4 < kVec / 4; ++v4) {
      const float4 x = qh[v4];
      qf[h][4 * v4] = x.x;
      qf[h][4 * v4 + 1] = x.y;
      qf[h][4 * v4 + 2] = x.z;
      qf[h][4 * v4 + 3] = x.w;
    }
  }
  __syncthreads();

  uint4 raw[kRowsPerThread];
  bool valid[kRowsPerThread];
#pragma unroll
  for (int u = 0; u < kRowsPerThread; ++u) {
    const int r = r_begin + rg + u * kRowsPerPass;
    raw[u] = make_uint4(0u, 0u, 0u, 0u);
    valid[u] = false;
    if (r < r_end) {
      const int jl = (r >> log2P) - j_begin;
      const int t = r & (P - 1);
      if (t < pg_valid[jl]) {
        valid[u] = true;
        const T* row = K + (size_t)pg_phys[jl] * Hkv * tile_stride + g * tile_stride +
                       (size_t)t * D + c * kVec;
        raw[u] = load16_stream(row);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kRowsPerThread; ++u) {
    const int rl = rg + u * kRowsPerPass;  // slot inside the item
    float x[kVec];
    Elem<T>::unpack(raw[u], x);
    float zsel = 0.0f;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float a = 0.0f;
#pragma unroll
      for (int v = 0; v < kVec; ++v) a = fmaf(qf[h][v], x[v], a);
      a = group_sum_f32<kLpr>(a);
      if (c == h) zsel = valid[u] ? a * zscale : -__builtin_huge_valf();
    }
    if (c < G) zl[c][rl] = zsel;
  }
  __syncthreads();

  }
}

// One wave per head: the item's maximum over its nrows scores in sm.zl, then
// the candidates z > max - 1 as (z, physical token) pairs in slot order, their
// count and the maximum, at split s of head bh0 + h.  kOutCoherent: another
// workgroup of the same launch reads them (device-coherent stores).
template <typename T, int D, int G, bool kOutCoherent, bool kMfma>
__device__ __forceinline__ void qk_emit(QkLds<T, D, G, kMfma>& sm, int nrows, int r_begin,
                                        int j_begin, int P, int log2P, float2* __restrict__ cand,
                                        int* __restrict__ cnt, float* __restrict__ smax,
                                        size_t bh0, int splits, int s) {
  constexpr int kR = Geo<T, D>::kR;
  auto& zl = sm.zl;
  auto& pg_phys = sm.pg_phys;
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  // one wave per head: split maximum, then the candidates z > max - 1
  for (int h = wave; h < G; h += kBlock / kWave) {
    float m = -__builtin_huge_valf();
    for (int r = lane; r < nrows; r += kWave) m = fmaxf(m, zl[h][r]);
    m = wave_max_f32(m);
    const double thr = (double)m - 1.0;
    const size_t bh = bh0 + h;
    float2* out = cand + (bh * splits + s) * kR;
    int total = 0;
    for (int r0 = 0; r0 < nrows; r0 += kWave) {
      const int r = r0 + lane;
      const float z = r < nrows ? zl[h][r] : -__builtin_huge_valf();
      const bool flag = (double)z > thr;
      const uint64_t mask = __ballot(flag);
      const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (kWave - lane));
      if (flag) {
        const int rr = r_begin + r;
        const int jl = (rr >> log2P) - j_begin;
        const int ptok = pg_phys[jl] * P + (rr & (P - 1));
        if constexpr (kOutCoherent)
          __hip_atomic_store(reinterpret_cast<uint64_t*>(out) + total + __popcll(mask & lt),
                             pack_cand(z, ptok), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
          out[total + __popcll(mask & lt)] = make_float2(z, __int_as_float(ptok));
      }
      total += __popcll(mask);
    }
    if (lane == 0) {
      if constexpr (kOutCoherent) {
        __hip_atomic_store(cnt + bh * splits + s, total, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(smax + bh * splits + s, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        cnt[bh * splits + s] = total;
        smax[bh * splits + s] = m;
      }
    }
  }
}

// What a qk item was about (for the callers' arrival protocols).
struct QkItemInfo {
  bool ran;
  int pair, b, g, L, np, nsel;
};

// One qk work item: scores of one split of a (row, KV head)'s selected token
// slots for the G heads of the group, then per head the split maximum and the
// candidates z > split_max - 1.  kOutCoherent: the candidates, counts and
// maxima are read by another workgroup of the same launch (device-coherent
// stores).  Called by all threads of the workgroup; ends with the LDS of `sm`
// still in use (callers barrier before reuse).
template <typename T, int D, int G, bool kOutCoherent, bool kMfma = std::is_same<T, bf16_t>::value>
__device__ __forceinline__ QkItemInfo qk_item(const QkArgs<T>& a, long long item,
                                              QkLds<T, D, G, kMfma>& sm) {
  using GE = Geo<T, D>;
  constexpr int kLpr = GE::kLpr, kR = GE::kR;
  static_assert(G <= kLpr, "lane c < G stores head c");
  const float* __restrict__ q = a.q;
  const float zscale = a.zscale;
  const T* __restrict__ K = a.K;
  const int32_t* __restrict__ bt = a.bt;
  const int32_t* __restrict__ lens = a.lens;
  const int32_t* sel = a.sel;
  const int32_t* n_sel = a.n_sel;
  const int max_sel = a.max_sel, Hkv = a.Hkv, P = a.P, log2P = a.log2P, maxP = a.maxP;
  const int splits = a.splits;
  float2* __restrict__ cand = a.cand;
  int* __restrict__ cnt = a.cnt;
  float* __restrict__ smax = a.smax;
  auto& pg_phys = sm.pg_phys;
  auto& pg_valid = sm.pg_valid;
  const int Hq = Hkv * G;
  QkItemInfo info{false, 0, 0, 0, 0, 0, 0};
  // split-major numbering: consecutive items are the same split of
  // consecutive pairs, so a workgroup striding over the items visits many
  // splits, and the low splits that short selections use spread over all
  // workgroups (pair-major numbering gave workgroup i only split i % splits)
  const int pair = (int)(item % a.npairs);
  const int s = (int)(item / a.npairs);
  const int b = pair / Hkv;
  const int g = pair % Hkv;
  const int r_begin = s * kR;
  const int j_begin = r_begin >> log2P;
  // the selected page indices this split can cover, loaded before the row
  // length and the selection count are known (same round trip); entries past
  // the count are in bounds but never used
  constexpr int kSpec = (kR + kBlock - 1) / kBlock;
  int spec[kSpec];
#pragma unroll
  for (int u = 0; u < kSpec; ++u) {
    const int i = threadIdx.x + u * kBlock;
    spec[u] = 0;
    if (sel && i < kR && j_begin + i < maxP) spec[u] = sel[(size_t)pair * maxP + j_begin + i];
  }
  // the group's queries (matrix-core path), also requested in that round trip
  constexpr int kQPer = (G * D + kBlock - 1) / kBlock;
  float qv[kMfma ? kQPer : 1];
  if constexpr (kMfma) {
#pragma unroll
    for (int u = 0; u < kQPer; ++u) {
      const int idx = threadIdx.x + u * kBlock;
      qv[u] = idx < G * D ? q[((size_t)b * Hq + g * G) * D + idx] : 0.0f;
    }
  }
  const int L = lens[b];
  const int np = (L + P - 1) / P;
  const int nsel = min(sel ? n_sel[pair] : np, max_sel);
  const int r_end = min(nsel << log2P, r_begin + kR);
  if (r_begin >= r_end) return info;  // uniform over the block
  const int n_pg = ((r_end - 1) >> log2P) - j_begin + 1;  // <= kR

  // page map of this split: physical page and valid tokens per selected page
  // (0 for a page below every head's support, which is then not read, and for
  // a caller's entry outside [0, np): such an entry reads nothing)
  float zlb_h[G];
  if (a.ub) {
#pragma unroll
    for (int h = 0; h < G; ++h) zlb_h[h] = a.zlb[(size_t)b * Hq + g * G + h];
  }
#pragma unroll
  for (int u = 0; u < kSpec; ++u) {
    const int i = threadIdx.x + u * kBlock;
    if (i < n_pg) {
      const int page_raw = sel ? spec[u] : j_begin + i;
      const bool in_row = (unsigned)page_raw < (unsigned)np;
      const int page = in_row ? page_raw : 0;
      pg_phys[i] = bt[(size_t)b * maxP + page];
      bool needed = in_row;
      if (a.ub && in_row) {
        needed = false;
#pragma unroll
        for (int h = 0; h < G; ++h)
          needed |= !page_below_support(a.a1 * a.ub[((size_t)pair * maxP + page) * G + h],
                                        zlb_h[h]);
      }
      pg_valid[i] = needed ? page_valid(L, page, P) : 0;
    }
  }
  qk_score_slots<T, D, G, kMfma>(q + ((size_t)b * Hq + g * G) * D, qv, zscale, K, Hkv, g, P,
                                 log2P, r_begin, r_end, j_begin, sm);
  qk_emit<T, D, G, kOutCoherent, kMfma>(sm, r_end - r_begin, r_begin, j_begin, P, log2P, cand, cnt,
                                        smax, (size_t)b * Hq + g * G, splits, s);
  info = QkItemInfo{true, pair, b, g, L, np, nsel};
  return info;
}

// Arguments of the page-pruning probe (one (row, query head) each).
template <typename T>
struct ZlbArgs {
  const float* q;
  float zscale;
  const T* K;
  const int32_t* bt;
  const int32_t* lens;
  const int32_t* sel;
  const int32_t* n_sel;
  int max_sel, Hq, Hkv, P, maxP;
  const float* ub;
  float* zlb;
};

// Lower bound of z_max over a (row, query head)'s selected tokens: the largest
// score among the valid tokens of the selected page with the largest bound
// for that head (lowest page on ties), in fp32 with kLpr lanes per key row.
// -inf when nothing is selected.
template <typename T, int D>
__device__ __forceinline__ void zlb_head(const ZlbArgs<T>& a, int bh) {
  constexpr int kVec = Elem<T>::kVec;
  constexpr int kLpr = D / kVec;
  constexpr int kRowsPerPass = kBlock / kLpr;
  constexpr int kWaves = kBlock / kWave;
  __shared__ float s_best[kWaves];
  __shared__ int s_bestp[kWaves];
  __shared__ int s_bestphys[kWaves];
  __shared__ float s_z[kWaves];
  const int G = a.Hq / a.Hkv;
  const int b = bh / a.Hq;
  const int g = (bh % a.Hq) / G;
  const int pair = b * a.Hkv + g;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int c = threadIdx.x % kLpr;
  float qv[kVec];
#pragma unroll
  for (int v = 0; v < kVec; ++v) qv[v] = a.q[(size_t)bh * D + c * kVec + v];
  // the selection's slots in rounds of kBatch per thread: a round's page
  // indices, then all their bounds and block-table entries (two dependent
  // loads per round); the first round's indices are requested in the same
  // round trip as the row length and the selection size (slots past n_sel
  // are in bounds, below max_sel, and masked), so up to kBatch * kBlock
  // selected pages cost two round trips before the reduction
  constexpr int kBatch = 32;
  const float* U = a.ub + (size_t)pair * a.maxP * G + (bh % a.Hq) % G;  // stride G per page
  int L = 0, np = 0, nsel = 0;
  float best = -__builtin_huge_valf();
  int bestp = 0x7fffffff, bestphys = 0;
  for (int j0 = 0;; j0 += kBatch * kBlock) {
    int pg[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int j = j0 + threadIdx.x + u * kBlock;
      pg[u] = -1;
      if (j < a.max_sel) pg[u] = a.sel ? a.sel[(size_t)pair * a.maxP + j] : j;
    }
    if (j0 == 0) {
      L = a.lens[b];
      np = (L + a.P - 1) / a.P;
      nsel = min(a.sel ? a.n_sel[pair] : np, a.max_sel);
    }
    float uu[kBatch];
    int ph[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      // a slot past n_sel, or a caller's entry outside the row, is skipped
      const bool ok = j0 + (int)threadIdx.x + u * kBlock < nsel && (unsigned)pg[u] < (unsigned)np;
      if (!ok) pg[u] = -1;
      uu[u] = ok ? U[(size_t)pg[u] * G] : -__builtin_huge_valf();
      ph[u] = ok ? a.bt[(size_t)b * a.maxP + pg[u]] : 0;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (pg[u] >= 0 && (uu[u] > best || (uu[u] == best && pg[u] < bestp))) {
        best = uu[u];
        bestp = pg[u];
        bestphys = ph[u];
      }
    }
    if (j0 + kBatch * kBlock >= nsel) break;  // uniform
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float ob = __shfl_xor(best, o, kWave);
    const int op = __shfl_xor(bestp, o, kWave);
    const int oph = __shfl_xor(bestphys, o, kWave);
    if (ob > best || (ob == best && op < bestp)) {
      best = ob;
      bestp = op;
      bestphys = oph;
    }
  }
  if (lane == 0) {
    s_best[wave] = best;
    s_bestp[wave] = bestp;
    s_bestphys[wave] = bestphys;
  }
  __syncthreads();
  best = s_best[0];
  bestp = s_bestp[0];
  bestphys = s_bestphys[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w)
    if (s_best[w] > best || (s_best[w] == best && s_bestp[w] < bestp)) {
      best = s_best[w];
      bestp = s_bestp[w];
      bestphys = s_bestphys[w];
    }
  if (bestp == 0x7fffffff) {  // uniform: no selected page
    if (threadIdx.x == 0) a.zlb[bh] = -__builtin_huge_valf();
    return;
  }
  const int nv = page_valid(L, bestp, a.P);
  const size_t tile = ((size_t)bestphys * a.Hkv + g) * (size_t)a.P * D;
  float zmax = -__builtin_huge_valf();
  // every lane of a kLpr-lane row group has the same t, so the group sum
  // only combines active lanes
  for (int t = threadIdx.x / kLpr; t < nv; t += kRowsPerPass) {
    float x[kVec];
    Elem<T>::unpack(load16_stream(a.K + tile + (size_t)t * D + c * kVec), x);
    float acc = 0.0f;
#pragma unroll
    for (int v = 0; v < kVec; ++v) acc = fmaf(qv[v], x[v], acc);
    acc = group_sum_f32<kLpr>(acc);
    zmax = fmaxf(zmax, acc * a.zscale);
  }
  zmax = wave_max_f32(zmax);
  if (lane == 0) s_z[wave] = zmax;
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = s_z[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) m = fmaxf(m, s_z[w]);
    a.zlb[bh] = m;
  }
}

// Outputs of one query head of an empty row (no token to attend to): a zero
// output, tau NaN, support 0.  Called by all threads of a workgroup.
__device__ inline void empty_row_head(float* __restrict__ out, float* __restrict__ tau_out,
                                      int32_t* __restrict__ n_support, int bh, int D) {
  for (int t = threadIdx.x; t < D; t += kBlock) out[(size_t)bh * D + t] = 0.0f;
  if (tau_out && threadIdx.x == 0) tau_out[bh] = __builtin_nanf("");
  if (n_support && threadIdx.x == 0) n_support[bh] = 0;
}

// Arguments of the tau / PV stage (one (row, query head) each).
template <typename T>
struct TauArgs {
  const float2* cand;
  const int* cnt;
  const float* smax;
  int splits;
  const T* V;
  const int32_t* lens;
  const int32_t* n_sel;
  bool has_sel;
  int max_sel, Hq, Hkv, P, log2P;
  double alpha, gamma;
  int gamma_int;
  float* out;
  float* tau_out;
  int32_t* n_support;
};

template <typename T, int D>
struct TauLds {
  static constexpr int kRowsPerPass = Geo<T, D>::kRowsPerPass;
  // the value rows' partial sums are written only after the last read of the
  // candidate lists and split offsets, so they share that storage (26 KiB in
  // all instead of 34: six workgroups per compute unit instead of four)
  union {
    struct {
      float c_z[kCandCap];
      int c_t[kCandCap];
      int s_off[kMaxSplits + 1];
    } w;
    float acc_sh[kRowsPerPass][D + 1];
  } u;
  float st_p[kBlock];
  int st_t[kBlock];
  int sh4[4];
  double shd[8];
  double s_tau;
};

// tau and the output of one (row, query head) bh.  Called by all threads of
// the workgroup; the LDS of `sm` is free again when it returns.
template <typename T, int D>
__device__ __forceinline__ void tau_head(const TauArgs<T>& a, int bh, TauLds<T, D>& sm) {
  const float2* __restrict__ cand = a.cand;
  const int* __restrict__ cnt = a.cnt;
  const float* __restrict__ smax = a.smax;
  const int splits = a.splits;
  const T* __restrict__ V = a.V;
  const int32_t* __restrict__ lens = a.lens;
  const int32_t* n_sel = a.n_sel;
  const bool has_sel = a.has_sel;
  const int max_sel = a.max_sel, Hq = a.Hq, Hkv = a.Hkv, P = a.P, log2P = a.log2P;
  const double alpha = a.alpha, gamma = a.gamma;
  const int gamma_int = a.gamma_int;
  float* __restrict__ out = a.out;
  float* __restrict__ tau_out = a.tau_out;
  int32_t* __restrict__ n_support = a.n_support;
  using GE = Geo<T, D>;
  constexpr int kVec = GE::kVec, kLpr = GE::kLpr, kRowsPerPass = GE::kRowsPerPass, kR = GE::kR;
  auto& c_z = sm.u.w.c_z;
  auto& c_t = sm.u.w.c_t;
  auto& s_off = sm.u.w.s_off;
  auto& st_p = sm.st_p;
  auto& st_t = sm.st_t;
  auto& acc_sh = sm.u.acc_sh;
  auto& sh4 = sm.sh4;
  auto& shd = sm.shd;
  auto& s_tau = sm.s_tau;
  const int b = bh / Hq;
  const int h = bh % Hq;
  const int G = Hq / Hkv;
  const int g = h / G;
  const int pair = b * Hkv + g;
  const int L = lens[b];
  const int np = (L + P - 1) / P;
  const int nsel = has_sel ? n_sel[pair] : np;
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  if (np == 0) {
    // empty row: no token to attend to
    empty_row_head(out, tau_out, n_support, bh, D);
    return;
  }
  if (nsel > max_sel || nsel < 1) {
    // outside the launch's bound: flag the row instead of reading past the workspace
    for (int t = threadIdx.x; t < D; t += kBlock) out[(size_t)bh * D + t] = __builtin_nanf("");
    if (tau_out && threadIdx.x == 0) tau_out[bh] = __builtin_nanf("");
    if (n_support && threadIdx.x == 0) n_support[bh] = -1;
    return;
  }
  const int nsplit = ((nsel << log2P) + kR - 1) / kR;
  const float2* cand_bh = cand + (size_t)bh * splits * kR;
  const int* cnt_bh = cnt + (size_t)bh * splits;
  const float* smax_bh = smax + (size_t)bh * splits;

  float zm = -__builtin_huge_valf();
  double zmax = 0.0, thr = 0.0;
  int total_c = 0, count = 0;
  // First try: each split's count, maximum and first kSpec candidate slots
  // in one round of independent loads (slots past the count are ignored).
  constexpr int kSpec = 16;
  bool spec = nsplit * kSpec <= kBlock;
  if (spec) {
    const int s = threadIdx.x / kSpec;
    const int j = threadIdx.x % kSpec;
    int cs = 0;
    float2 e = make_float2(-__builtin_huge_valf(), 0.0f);
    if (s < nsplit) {
      cs = cnt_bh[s];
      zm = smax_bh[s];
      e = cand_bh[(size_t)s * kR + j];
    }
    spec = !__syncthreads_or(cs > kSpec);
    if (spec) {
      zm = wave_max_f32(zm);
      if (lane == 0) st_p[wave] = zm;
      __syncthreads();
      zm = fmaxf(fmaxf(st_p[0], st_p[1]), fmaxf(st_p[2], st_p[3]));
      zmax = (double)zm;
      thr = zmax - 1.0;
      // (s, j) runs in split order, so the compacted list is in split order
      const bool flag = j < cs && (double)e.x > thr;
      int tot;
      const int slot = chunk_slot(flag, sh4, tot);
      if (slot >= 0) {
        c_z[slot] = e.x;
        c_t[slot] = bits_of(e.y);
      }
      count = tot;  // <= kBlock: never an overflow, so total_c is not needed
      __syncthreads();
    }
  }
  // Every candidate in split order, kBlock at a time: fn(k, e, valid) is
  // called by all threads of the block the same number of times (it may hold
  // block barriers), k the candidate's index, valid = k < total_c.  Up to
  // kMaxSplits splits the exclusive offsets of the per-split lists sit in
  // s_off once (filled below); beyond, they are rebuilt for each run of
  // kMaxSplits splits as the walk reaches it.
  auto walk_cands = [&](auto&& fn) {
    if (nsplit <= kMaxSplits) {
      for (int k0 = 0; k0 < total_c; k0 += kBlock) {
        const int k = k0 + threadIdx.x;
        float2 e = make_float2(-__builtin_huge_valf(), 0.0f);
        if (k < total_c) e = cand_at(cand_bh, s_off, nsplit, kR, k);
        fn(k, e, k < total_c);
      }
      return;
    }
    int base = 0;
    for (int c0 = 0; c0 < nsplit; c0 += kMaxSplits) {
      const int c1 = min(nsplit, c0 + kMaxSplits);
      int run = 0;
      for (int s0 = c0; s0 < c1; s0 += kBlock) {
        const int s = s0 + threadIdx.x;
        const int v = s < c1 ? cnt_bh[s] : 0;
        const int incl = block_incl_scan(v, sh4);
        if (s < c1) s_off[s - c0] = run + incl - v;
        if (threadIdx.x == kBlock - 1) sh4[0] = incl;
        __syncthreads();
        run += sh4[0];
        __syncthreads();
      }
      if (threadIdx.x == 0) s_off[c1 - c0] = run;
      __syncthreads();
      for (int k0 = 0; k0 < run; k0 += kBlock) {
        const int k = k0 + threadIdx.x;
        float2 e = make_float2(-__builtin_huge_valf(), 0.0f);
        if (k < run) e = cand_at(cand_bh + (size_t)c0 * kR, s_off, c1 - c0, kR, k);
        fn(base + k, e, k < run);
      }
      base += run;
      __syncthreads();  // s_off is rebuilt for the next run of splits
    }
  };
  if (!spec) {
    // global max, the candidate total and (up to kMaxSplits splits) the
    // exclusive offsets of the per-split candidate lists
    zm = -__builtin_huge_valf();
    int running = 0;
    for (int s0 = 0; s0 < nsplit; s0 += kBlock) {
      const int s = s0 + threadIdx.x;
      int v = 0;
      if (s < nsplit) {
        zm = fmaxf(zm, smax_bh[s]);
        v = cnt_bh[s];
      }
      const int incl = block_incl_scan(v, sh4);
      if (s < nsplit && nsplit <= kMaxSplits) s_off[s] = running + incl - v;
      if (threadIdx.x == kBlock - 1) sh4[0] = incl;  // chunk total (read after the barrier)
      __syncthreads();
      running += sh4[0];
      __syncthreads();
    }
    if (threadIdx.x == 0 && nsplit <= kMaxSplits) s_off[nsplit] = running;
    zm = wave_max_f32(zm);
    if (lane == 0) st_p[wave] = zm;
    __syncthreads();
    zm = fmaxf(fmaxf(st_p[0], st_p[1]), fmaxf(st_p[2], st_p[3]));
    zmax = (double)zm;
    thr = zmax - 1.0;
    total_c = running;

    // candidates that clear the global bar, in split order
    walk_cands([&](int, float2 e, bool) {
      const bool flag = (double)e.x > thr;
      int tot;
      const int slot = chunk_slot(flag, sh4, tot);
      if (slot >= 0 && count + slot < kCandCap) {
        c_z[count + slot] = e.x;
        c_t[count + slot] = bits_of(e.y);
      }
      count += tot;
    });
    __syncthreads();
  }
  const bool overflow = count > kCandCap;
  // number of tokens (an upper bound is enough for the upper end of the bracket)
  const double nvalid = has_sel ? (double)nsel * P : (double)L;

  // value rows of every candidate requested before tau is known (few
  // candidates): their latency overlaps the solve
  constexpr int kPre = 4;
  const int c = threadIdx.x % kLpr;
  const int rg = threadIdx.x / kLpr;
  const size_t tile_stride = (size_t)P * D;
  const bool prefetch = !overflow && count <= kPre * kRowsPerPass;
  uint4 vraw[kPre];
  if (prefetch) {
#pragma unroll
    for (int i = 0; i < kPre; ++i) {
      const int r = rg + i * kRowsPerPass;
      if (r < count) {
        const int pt = c_t[r];
        vraw[i] = load16(V + (size_t)(pt >> log2P) * Hkv * tile_stride + g * tile_stride +
                         (size_t)(pt & (P - 1)) * D + c * kVec);
      }
    }
  }

  // bracketed Newton for  f(tau) = sum [z - tau]_+^gamma - 1 = 0  on
  // [zmax - 1, zmax - n^(1-alpha)];  f' = -gamma sum [z - tau]_+^(gamma-1)
  auto term = [&](double z, double tau, double& f, double& fd) {
    const double x = z - tau;
    if (x > 0.0) {
      const double xg1 = gamma_int == 1 ? 1.0 : pos_pow(x, gamma - 1.0, gamma_int - 1);
      f += xg1 * x;
      fd += gamma * xg1;
    }
  };
  auto newton = [&](auto&& eval) -> double {
    double lo = thr;
    double hi = zmax - pow_ool(nvalid, 1.0 - alpha);
    if (hi < lo) hi = lo;
    double tau = lo;
    for (int it = 0; it < 200; ++it) {
      double f, fd;
      eval(tau, f, fd);
      f -= 1.0;
      if (f == 0.0) break;
      if (f > 0.0) lo = tau;
      else hi = tau;
      double nt = fd > 0.0 ? tau + f / fd : 0.5 * (lo + hi);
      // a Newton step below fp64 resolution means converged (checked before
      // the bracket test, which would otherwise turn it into a bisection jump)
      if (fd > 0.0 && fabs(nt - tau) <= 4e-16 * fmax(1.0, fabs(tau))) {
        tau = nt > lo && nt < hi ? nt : tau;
        break;
      }
      if (!(nt > lo && nt < hi)) {
        nt = 0.5 * (lo + hi);
        if (!(nt > lo && nt < hi)) break;
      }
      tau = nt;
    }
    return tau;
  };

  double tau;
  if (!overflow && count <= kWave) {
    // one wave, no barriers inside the solve
    if (wave == 0) {
      const float zf = lane < count ? c_z[lane] : -__builtin_huge_valf();
      double t;
      if (!tau_small(zf, count, thr, gamma, gamma_int, t)) {
        const double zc = (double)zf;
        t = newton([&](double tt, double& f, double& fd) {
          f = 0.0;
          fd = 0.0;
          term(zc, tt, f, fd);
          f = wave_sum_f64(f);
          fd = wave_sum_f64(fd);
        });
      }
      if (lane == 0) s_tau = t;
    }
    lds_barrier();  // the value-row loads stay in flight
    tau = s_tau;
  } else {
    tau = newton([&](double tt, double& f, double& fd) {
      f = 0.0;
      fd = 0.0;
      if (!overflow) {
        for (int k = threadIdx.x; k < count; k += kBlock) term((double)c_z[k], tt, f, fd);
      } else {
        walk_cands([&](int, float2 e, bool valid) {
          if (valid) term((double)e.x, tt, f, fd);
        });
      }
      block_sum2(f, fd, shd);
    });
  }

  // weights and the value rows of the support
  float acc[kVec];
#pragma unroll
  for (int v = 0; v < kVec; ++v) acc[v] = 0.0f;
  double psum = 0.0;
  int nsupp = 0;
  if (prefetch) {
#pragma unroll
    for (int i = 0; i < kPre; ++i) {
      const int r = rg + i * kRowsPerPass;
      if (r < count) {
        const double x = (double)c_z[r] - tau;
        if (x > 0.0) {
          const float p = (float)pos_pow(x, gamma, gamma_int);
          float xv[kVec];
          Elem<T>::unpack(vraw[i], xv);
#pragma unroll
          for (int v = 0; v < kVec; ++v) acc[v] = fmaf(p, xv[v], acc[v]);
        }
      }
    }
    if (threadIdx.x < count) {
      const double x = (double)c_z[threadIdx.x] - tau;
      if (x > 0.0) {
        psum = (double)(float)pos_pow(x, gamma, gamma_int);
        nsupp = 1;
      }
    }
  } else {
    // one block of candidates: the support's weights and value rows
    auto pv_block = [&](float z, int ptok) {
      const double x = (double)z - tau;
      const bool flag = x > 0.0;
      int m;
      const int slot = chunk_slot(flag, sh4, m);
      nsupp += m;
      if (slot >= 0) {
        const float p = (float)pos_pow(x, gamma, gamma_int);
        st_p[slot] = p;
        st_t[slot] = ptok;
        psum += (double)p;
      }
      __syncthreads();
      for (int r = rg; r < m; r += kRowsPerPass) {
        const int pt = st_t[r];
        const float p = st_p[r];
        const int pi = pt >> log2P;
        const int t = pt & (P - 1);
        const T* row = V + (size_t)pi * Hkv * tile_stride + g * tile_stride + (size_t)t * D + c * kVec;
        float xv[kVec];
        Elem<T>::unpack(load16(row), xv);
#pragma unroll
        for (int v = 0; v < kVec; ++v) acc[v] = fmaf(p, xv[v], acc[v]);
      }
      __syncthreads();
    };
    if (overflow) {
      walk_cands([&](int, float2 e, bool) { pv_block(e.x, bits_of(e.y)); });
    } else {
      for (int base = 0; base < count; base += kBlock) {
        const int k = base + threadIdx.x;
        pv_block(k < count ? c_z[k] : -__builtin_huge_valf(), k < count ? c_t[k] : 0);
      }
    }
    if (threadIdx.x != 0) nsupp = 0;  // the chunk totals are block-wide
  }
  __syncthreads();  // acc_sh overlays the candidate lists: every read of them is done
#pragma unroll
  for (int v = 0; v < kVec; ++v) acc_sh[rg][c * kVec + v] = acc[v];
  double ps = psum, ns = (double)nsupp;
  block_sum2(ps, ns, shd);  // includes the barrier that publishes acc_sh
  const float inv = (float)(1.0 / ps);
  for (int t = threadIdx.x; t < D; t += kBlock) {
    float o = 0.0f;
    for (int r = 0; r < kRowsPerPass; ++r) o += acc_sh[r][t];
    out[(size_t)bh * D + t] = o * inv;
  }
  if (tau_out && threadIdx.x == 0) tau_out[bh] = (float)tau;
  if (n_support && threadIdx.x == 0) n_support[bh] = (int)ns;
}

}  // namespace
}  // namespace ekv
