// Sparse alpha-entmax attention over the selected pages (EntmaxKV summary
// page, §2.C: load only the selected pages' keys and values and compute the
// entmax weights over that reduced set).
//
// Entmax has no online merge rule: tau depends on every score of the head.
// The decode therefore runs in two launches:
//
//  1. qk_kernel -- grid (splits, B*Hkv).  Each workgroup walks a contiguous
//     range of the pair's selected pages, reads each K row once (16-byte lanes,
//     kLpr lanes per row, rows of a page tile are contiguous) and forms the
//     scores of all G query heads of the group from that one read:
//         z = (alpha-1) * scale * <q_h, k>     (fp32 FMA, DPP row reduction).
//     z goes to the workspace (one slot per selected token, -inf for the
//     invalid tail of a row's last page) and each split's max per head to a
//     small side array.
//
//  2. tau_pv_kernel -- grid (B*Hq).  The threshold satisfies
//     tau >= z_max - 1 (the largest weight is at most 1), so only tokens with
//     z > z_max - 1 can carry weight.  The workgroup compacts those candidates
//     into LDS (deterministic ballot order), solves
//         sum_i [z_i - tau]_+^gamma = 1
//     in fp64 with a bracketed Newton iteration (the left end of the bracket
//     has f >= 0, f is convex and decreasing for gamma >= 1), and then reads
//     only the value rows with z_i > tau -- the weights off the support are
//     exact zeros, so no other value row is needed:
//         out = sum_i p_i v_i / sum_i p_i,   p_i = (z_i - tau)^gamma.
#include "common.h"
#include "kernels.h"

namespace ekv {
namespace {

constexpr int kBlock = 256;
constexpr int kQkUnroll = 4;
constexpr int kCandCap = 8192;  // LDS candidates per head; more falls back to global z

template <typename T, int D, int G>
__global__ __launch_bounds__(kBlock) void qk_kernel(
    const float* __restrict__ q, float zscale, const T* __restrict__ K,
    const int32_t* __restrict__ bt, const int32_t* __restrict__ lens,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ n_sel, int max_sel, int pps,
    int Hkv, int P, int log2P, int maxP, long long tmax, int splits, float* __restrict__ zws,
    float* __restrict__ smax) {
  constexpr int kVec = Elem<T>::kVec;
  constexpr int kLpr = D / kVec;
  constexpr int kRowsPerPass = kBlock / kLpr;
  static_assert(G <= kLpr, "lane c < G stores head c");
  __shared__ float red[kBlock / kWave][G];

  const int pair = blockIdx.y;
  const int b = pair / Hkv;
  const int g = pair % Hkv;
  const int Hq = Hkv * G;
  const int L = lens[b];
  const int np = (L + P - 1) / P;
  int nsel = sel ? n_sel[pair] : np;
  nsel = min(nsel, max_sel);
  const int j0 = blockIdx.x * pps;
  if (j0 >= nsel) return;
  const int j1 = min(nsel, j0 + pps);
  const int r_begin = j0 << log2P;
  const int r_end = j1 << log2P;

  const int c = threadIdx.x % kLpr;
  const int rg = threadIdx.x / kLpr;
  const int32_t* selrow = sel ? sel + (size_t)pair * maxP : nullptr;
  const int32_t* btrow = bt + (size_t)b * maxP;
  const size_t tile_stride = (size_t)P * D;

  float qf[G][kVec];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float* qh = q + ((size_t)b * Hq + g * G + h) * D + c * kVec;
#pragma unroll
    for (int v = 0; v < kVec; ++v) qf[h][v] = qh[v];
  }
  float zmx[G];
#pragma unroll
  for (int h = 0; h < G; ++h) zmx[h] = -__builtin_huge_valf();

  float* zbase = zws + ((size_t)b * Hq + g * G) * tmax;

  for (int base = r_begin; base < r_end; base += kRowsPerPass * kQkUnroll) {
    uint4 raw[kQkUnroll];
    bool valid[kQkUnroll];
#pragma unroll
    for (int u = 0; u < kQkUnroll; ++u) {
      const int r = base + rg + u * kRowsPerPass;
      raw[u] = make_uint4(0u, 0u, 0u, 0u);
      valid[u] = false;
      if (r < r_end) {
        const int j = r >> log2P;
        const int t = r & (P - 1);
        const int page = selrow ? selrow[j] : j;
        if (t < page_valid(L, page, P)) {
          valid[u] = true;
          const int pi = btrow[page];
          const T* row = K + ((size_t)pi * Hkv + g) * tile_stride + (size_t)t * D + c * kVec;
          raw[u] = load16_stream(row);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kQkUnroll; ++u) {
      const int r = base + rg + u * kRowsPerPass;
      float x[kVec];
      Elem<T>::unpack(raw[u], x);
      float zsel = 0.0f;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float a = 0.0f;
#pragma unroll
        for (int v = 0; v < kVec; ++v) a = fmaf(qf[h][v], x[v], a);
        a = group_sum_f32<kLpr>(a);
        const float z = valid[u] ? a * zscale : -__builtin_huge_valf();
        zmx[h] = fmaxf(zmx[h], z);
        if (c == h) zsel = z;
      }
      if (c < G && r < r_end) zbase[(size_t)c * tmax + r] = zsel;
    }
  }
  // split max per head: identical in the kLpr lanes of a row, reduce row groups
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int o = kLpr; o < kWave; o <<= 1) zmx[h] = fmaxf(zmx[h], __shfl_xor(zmx[h], o, kWave));
  }
  const int w = threadIdx.x / kWave;
  if (threadIdx.x % kWave == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) red[w][h] = zmx[h];
  }
  __syncthreads();
  if (threadIdx.x < G) {
    float m = red[0][threadIdx.x];
#pragma unroll
    for (int i = 1; i < kBlock / kWave; ++i) m = fmaxf(m, red[i][threadIdx.x]);
    smax[((size_t)b * Hq + g * G + threadIdx.x) * splits + blockIdx.x] = m;
  }
}

__device__ inline double pos_pow(double x, double gamma, int gi) {
  // x > 0
  if (gi > 0) {
    double r = x;
    for (int i = 1; i < gi; ++i) r *= x;
    return r;
  }
  return pow(x, gamma);
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

template <typename T, int D>
__global__ __launch_bounds__(kBlock) void tau_pv_kernel(
    const float* __restrict__ zws, const float* __restrict__ smax, long long tmax, int splits,
    int pps, const T* __restrict__ V, const int32_t* __restrict__ bt,
    const int32_t* __restrict__ lens, const int32_t* __restrict__ sel,
    const int32_t* __restrict__ n_sel, int max_sel, int Hq, int Hkv, int P, int log2P, int maxP,
    double alpha, double gamma, int gamma_int, float* __restrict__ out,
    float* __restrict__ tau_out, int32_t* __restrict__ n_support) {
  constexpr int kVec = Elem<T>::kVec;
  constexpr int kLpr = D / kVec;
  constexpr int kRowsPerPass = kBlock / kLpr;
  __shared__ float c_z[kCandCap];
  __shared__ int c_i[kCandCap];
  __shared__ float st_p[kBlock];
  __shared__ int st_i[kBlock];
  __shared__ float acc_sh[kRowsPerPass][D + 1];
  __shared__ int sh4[4];
  __shared__ double shd[8];

  const int bh = blockIdx.x;
  const int b = bh / Hq;
  const int h = bh % Hq;
  const int G = Hq / Hkv;
  const int g = h / G;
  const int pair = b * Hkv + g;
  const int L = lens[b];
  const int np = (L + P - 1) / P;
  const int nsel = sel ? n_sel[pair] : np;
  if (nsel > max_sel || nsel < 1) {
    // outside the launch's bound: flag the row instead of reading past the workspace
    for (int t = threadIdx.x; t < D; t += kBlock) out[(size_t)bh * D + t] = __builtin_nanf("");
    if (tau_out && threadIdx.x == 0) tau_out[bh] = __builtin_nanf("");
    if (n_support && threadIdx.x == 0) n_support[bh] = -1;
    return;
  }
  const int ntok = nsel << log2P;
  const float* zrow = zws + (size_t)bh * tmax;
  const int nsplit = (nsel + pps - 1) / pps;

  // global max from the split maxima
  float zm = -__builtin_huge_valf();
  for (int s = threadIdx.x; s < nsplit; s += kBlock) zm = fmaxf(zm, smax[(size_t)bh * splits + s]);
  zm = wave_max_f32(zm);
  if (threadIdx.x % kWave == 0) st_p[threadIdx.x / kWave] = zm;
  __syncthreads();
  zm = fmaxf(fmaxf(st_p[0], st_p[1]), fmaxf(st_p[2], st_p[3]));
  __syncthreads();
  const double zmax = (double)zm;
  const double thr = zmax - 1.0;

  // candidates z > zmax - 1, in slot order
  int count = 0;
  int nvalid_local = 0;
  for (int base = 0; base < ntok; base += kBlock) {
    const int i = base + threadIdx.x;
    const float z = i < ntok ? zrow[i] : -__builtin_huge_valf();
    nvalid_local += (z > -__builtin_huge_valf()) ? 1 : 0;
    const bool flag = (double)z > thr;
    int total;
    const int slot = chunk_slot(flag, sh4, total);
    if (slot >= 0 && count + slot < kCandCap) {
      c_z[count + slot] = z;
      c_i[count + slot] = i;
    }
    count += total;
  }
  __syncthreads();
  const bool overflow = count > kCandCap;
  double nv_d = (double)nvalid_local, dummy = 0.0;
  block_sum2(nv_d, dummy, shd);
  const double nvalid = nv_d;

  auto eval = [&](double tau, double& f, double& fd) {
    f = 0.0;
    fd = 0.0;
    const int lim = overflow ? ntok : count;
    for (int k = threadIdx.x; k < lim; k += kBlock) {
      const double z = overflow ? (double)zrow[k] : (double)c_z[k];
      const double x = z - tau;
      if (x > 0.0) {
        const double xg1 = gamma_int == 1 ? 1.0 : pos_pow(x, gamma - 1.0, gamma_int - 1);
        f += xg1 * x;
        fd += gamma * xg1;
      }
    }
    block_sum2(f, fd, shd);
  };

  // bracketed Newton for sum [z - tau]_+^gamma = 1 on [zmax - 1, zmax - n^(1-alpha)]
  double lo = thr;
  double hi = zmax - pow(nvalid, 1.0 - alpha);
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
    if (!(nt > lo && nt < hi)) {
      nt = 0.5 * (lo + hi);
      if (!(nt > lo && nt < hi)) break;
    }
    if (fabs(nt - tau) <= 4e-16 * fmax(1.0, fabs(tau))) {
      tau = nt;
      break;
    }
    tau = nt;
  }

  // weights and the value rows of the support
  const int c = threadIdx.x % kLpr;
  const int rg = threadIdx.x / kLpr;
  const int32_t* selrow = sel ? sel + (size_t)pair * maxP : nullptr;
  const int32_t* btrow = bt + (size_t)b * maxP;
  const size_t tile_stride = (size_t)P * D;
  float acc[kVec];
#pragma unroll
  for (int v = 0; v < kVec; ++v) acc[v] = 0.0f;
  double psum = 0.0;
  int nsupp = 0;
  const int lim = overflow ? ntok : count;
  for (int base = 0; base < lim; base += kBlock) {
    const int k = base + threadIdx.x;
    float z = -__builtin_huge_valf();
    int idx = 0;
    if (k < lim) {
      z = overflow ? zrow[k] : c_z[k];
      idx = overflow ? k : c_i[k];
    }
    const double x = (double)z - tau;
    const bool flag = x > 0.0;
    int m;
    const int slot = chunk_slot(flag, sh4, m);
    nsupp += m;
    if (slot >= 0) {
      const float p = (float)pos_pow(x, gamma, gamma_int);
      st_p[slot] = p;
      st_i[slot] = idx;
      psum += (double)p;
    }
    __syncthreads();
    for (int r = rg; r < m; r += kRowsPerPass) {
      const int i = st_i[r];
      const float p = st_p[r];
      const int j = i >> log2P;
      const int t = i & (P - 1);
      const int page = selrow ? selrow[j] : j;
      const int pi = btrow[page];
      const T* row = V + ((size_t)pi * Hkv + g) * tile_stride + (size_t)t * D + c * kVec;
      float x8[kVec];
      Elem<T>::unpack(load16(row), x8);
#pragma unroll
      for (int v = 0; v < kVec; ++v) acc[v] = fmaf(p, x8[v], acc[v]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int v = 0; v < kVec; ++v) acc_sh[rg][c * kVec + v] = acc[v];
  double ps = psum;
  block_sum2(ps, dummy, shd);  // includes the __syncthreads that publishes acc_sh
  const float inv = (float)(1.0 / ps);
  for (int t = threadIdx.x; t < D; t += kBlock) {
    float o = 0.0f;
    for (int r = 0; r < kRowsPerPass; ++r) o += acc_sh[r][t];
    out[(size_t)bh * D + t] = o * inv;
  }
  if (tau_out && threadIdx.x == 0) tau_out[bh] = (float)tau;
  if (n_support && threadIdx.x == 0) n_support[bh] = nsupp;
}

template <typename T, int D, int G>
hipError_t launch_qk_t(const Shape& s, const DecodePlan& pl, const float* q, float zscale,
                       const void* K, const int32_t* bt, const int32_t* lens, const int32_t* sel,
                       const int32_t* n_sel, float* zws, float* smax, hipStream_t stream) {
  dim3 grid(pl.splits, s.B * s.Hkv);
  hipLaunchKernelGGL((qk_kernel<T, D, G>), grid, dim3(kBlock), 0, stream, q, zscale,
                     (const T*)K, bt, lens, sel, n_sel, pl.max_sel, pl.pages_per_split, s.Hkv,
                     s.P, s.log2P, s.maxP, pl.tmax, pl.splits, zws, smax);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_decode_t(const Shape& s, const DecodePlan& pl, const float* q, float scale,
                           float alpha, const void* K, const void* V, const int32_t* bt,
                           const int32_t* lens, const int32_t* sel, const int32_t* n_sel,
                           float* out, float* tau_out, int32_t* n_support, void* ws,
                           hipStream_t stream) {
  float* zws = (float*)((char*)ws + pl.z_off);
  float* smax = (float*)((char*)ws + pl.smax_off);
  const double a1 = (double)alpha - 1.0;
  const float zscale = (float)(a1 * (double)scale);
  hipError_t e = hipErrorInvalidValue;
  switch (s.G) {
    case 1: e = launch_qk_t<T, D, 1>(s, pl, q, zscale, K, bt, lens, sel, n_sel, zws, smax, stream); break;
    case 2: e = launch_qk_t<T, D, 2>(s, pl, q, zscale, K, bt, lens, sel, n_sel, zws, smax, stream); break;
    case 4: e = launch_qk_t<T, D, 4>(s, pl, q, zscale, K, bt, lens, sel, n_sel, zws, smax, stream); break;
    case 8: e = launch_qk_t<T, D, 8>(s, pl, q, zscale, K, bt, lens, sel, n_sel, zws, smax, stream); break;
  }
  if (e != hipSuccess) return e;
  const double gamma = 1.0 / a1;
  const double gr = rint(gamma);
  const int gamma_int = (gr >= 1.0 && gr <= 64.0 && fabs(gamma - gr) <= 1e-12 * gr) ? (int)gr : 0;
  hipLaunchKernelGGL((tau_pv_kernel<T, D>), dim3(s.B * s.Hq), dim3(kBlock), 0, stream, zws, smax,
                     pl.tmax, pl.splits, pl.pages_per_split, (const T*)V, bt, lens, sel, n_sel,
                     pl.max_sel, s.Hq, s.Hkv, s.P, s.log2P, s.maxP, (double)alpha,
                     gamma_int ? gr : gamma, gamma_int, out, tau_out, n_support);
  return hipGetLastError();
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

DecodePlan make_decode_plan(const Shape& s, int max_sel) {
  DecodePlan pl{};
  pl.max_sel = max_sel;
  const long long pairs = (long long)s.B * s.Hkv;
  // aim for >= 2048 workgroups, 64..256 rows each
  const int min_pps = s.P >= 64 ? 1 : 64 / s.P;
  const int max_pps = s.P >= 256 ? 1 : 256 / s.P;
  long long want = (max_sel * pairs + 2047) / 2048;
  int pps = (int)(want < min_pps ? min_pps : (want > max_pps ? max_pps : want));
  if (pps < 1) pps = 1;
  pl.pages_per_split = pps;
  pl.splits = (max_sel + pps - 1) / pps;
  pl.tmax = (long long)max_sel * s.P;
  pl.z_off = 0;
  pl.z_bytes = align256((size_t)s.B * s.Hq * (size_t)pl.tmax * sizeof(float));
  pl.smax_off = pl.z_off + pl.z_bytes;
  pl.smax_bytes = align256((size_t)s.B * s.Hq * (size_t)pl.splits * sizeof(float));
  pl.total = pl.smax_off + pl.smax_bytes;
  return pl;
}

hipError_t launch_decode(const Shape& s, const DecodePlan& plan, const float* q, float scale,
                         float alpha, const void* K, const void* V, const int32_t* bt,
                         const int32_t* lens, const int32_t* sel, const int32_t* n_sel,
                         float* out, float* tau_out, int32_t* n_support, void* ws,
                         hipStream_t stream) {
  if (s.bf16) {
    if (s.D == 128)
      return launch_decode_t<bf16_t, 128>(s, plan, q, scale, alpha, K, V, bt, lens, sel, n_sel, out, tau_out, n_support, ws, stream);
    return launch_decode_t<bf16_t, 64>(s, plan, q, scale, alpha, K, V, bt, lens, sel, n_sel, out, tau_out, n_support, ws, stream);
  }
  if (s.D == 128)
    return launch_decode_t<float, 128>(s, plan, q, scale, alpha, K, V, bt, lens, sel, n_sel, out, tau_out, n_support, ws, stream);
  return launch_decode_t<float, 64>(s, plan, q, scale, alpha, K, V, bt, lens, sel, n_sel, out, tau_out, n_support, ws, stream);
}

}  // namespace ekv
