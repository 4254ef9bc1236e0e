// Softmax decode over the selected pages, or over the whole cache: the
// comparison side of the EntmaxKV summary page (§3: under softmax every
// dropped token drops mass; §4: its speed comparison is against a full-cache
// softmax decode of the FlashDecoding kind).
//
// Softmax, unlike entmax, has an exact online merge rule: partial results
// (m, l, o) over disjoint token sets, with m the largest score, l the sum of
// exp(s - m) and o the sum of exp(s - m) v, combine by rescaling each to the
// common maximum.  So the decode is a split-page pass and a merge:
//
//  1. softmax_split_kernel -- work items (row, KV head, split of `slots` token
//     slots of the selected pages), split-major so consecutive items fall on
//     different pairs (and XCDs).  The workgroup first resolves the split's
//     pages (selection list, then block table) into an LDS page map, so that
//     no key or value load waits on another global load.  Each lane owns one 16-byte chunk of a key
//     row and of the matching value row; a wave covers kRows token rows per
//     load and keeps kU loads in flight.  The scores of all G query heads of
//     the group come from that one key read (fp32 FMA, DPP row reduction), in
//     base-2 units (q pre-multiplied by scale * log2 e).  Per batch of kU*kRows
//     tokens each wave takes the batch maximum per head, rescales its running
//     sums once, and adds exp2(s - m) v.  Every valid token's value row is
//     read: softmax weights are never exactly zero.  The four waves' partials
//     are merged in LDS and written as the split's (m, l, o).
//  2. softmax_merge_kernel -- one wave per (row, query head): rescales the
//     splits' partials to the common maximum and writes
//         out = o / l,   lse = ln 2 * (m + log2 l)   (natural log).
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace ekv {
namespace {

constexpr int kSmBlock = 256;
constexpr int kSmMaxPages = 1024;  // pages per split (the page map staged in LDS)
constexpr int kSmWaves = kSmBlock / kWave;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T>
struct SmArgs {
  const float* q;
  float qscale;  // scale * log2(e)
  const T* K;
  const T* V;
  const int32_t* bt;
  const int32_t* lens;
  const int32_t* sel;    // NULL: every page of the row
  const int32_t* n_sel;
  int max_sel, npairs, splits, slots, Hq, Hkv, P, log2P, maxP;
  float2* part_ml;  // [B*Hq][splits] (m, l), base-2 units
  float* part_o;    // [B*Hq][splits][D]
};

// Selected pages of a pair (the row's pages when sel is NULL), or -1 when the
// pair's n_sel exceeds the launch bound.
template <typename T>
__device__ inline int pair_pages(const SmArgs<T>& a, int pair, int L) {
  if (a.sel == nullptr) return (L + a.P - 1) >> a.log2P;
  const int n = L > 0 ? a.n_sel[pair] : 0;
  return n > a.max_sel ? -1 : n;
}

template <typename T, int D, int G, int kU>
__global__ __launch_bounds__(kSmBlock) void softmax_split_kernel(SmArgs<T> a) {
  constexpr int kVec = Elem<T>::kVec;
  constexpr int kC = D / kVec;         // lanes per token row
  constexpr int kRows = kWave / kC;    // token rows per wave load
  __shared__ float sm_o[kSmWaves][G][D];
  __shared__ float sm_m[kSmWaves][G];
  __shared__ float sm_l[kSmWaves][G];
  __shared__ int2 sm_page[kSmMaxPages];  // (physical page, valid tokens) of the split

  const int item = blockIdx.x;
  const int pair = item % a.npairs;
  const int split = item / a.npairs;
  const int b = pair / a.Hkv, g = pair % a.Hkv;
  const int L = a.lens[b];
  const int npg = pair_pages(a, pair, L);
  const int n_slots = npg > 0 ? npg << a.log2P : 0;
  const int s0 = split * a.slots;
  if (s0 >= n_slots) return;  // workgroup-uniform: nothing of this pair here
  const int s1 = min(n_slots, s0 + a.slots);

  // the split's page map, resolved once (sel -> block table) so the K/V
  // loads below depend on no other global load
  const int p0 = s0 >> a.log2P;
  const int np = ((s1 - 1) >> a.log2P) - p0 + 1;
  {
    const int32_t* selp = a.sel ? a.sel + (size_t)pair * a.maxP : nullptr;
    const int32_t* btp = a.bt + (size_t)b * a.maxP;
    for (int k = threadIdx.x; k < np; k += kSmBlock) {
      const int lp = selp ? selp[p0 + k] : p0 + k;
      // a caller's entry outside [0, n_b) is a page with no valid token
      const bool in_row = (unsigned)lp < (unsigned)((L + a.P - 1) / a.P);
      sm_page[k] = make_int2(btp[in_row ? lp : 0], in_row ? page_valid(L, lp, a.P) : 0);
    }
  }
  __syncthreads();

  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int c = lane % kC, r = lane / kC;

  // this lane's chunk of the G query rows, in base-2 score units
  float qv[G][kVec];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float* qh = a.q + ((size_t)b * a.Hq + g * G + h) * D + c * kVec;
#pragma unroll
    for (int e = 0; e < kVec; ++e) qv[h][e] = qh[e] * a.qscale;
  }
  float m[G], l[G], acc[G][kVec];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < kVec; ++e) acc[h][e] = 0.f;
  }
  for (int base = s0 + wave * kRows * kU; base < s1; base += kSmWaves * kRows * kU) {
    uint4 kk[kU], vv[kU];
    bool valid[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int j = base + u * kRows + r;
      valid[u] = false;
      kk[u] = make_uint4(0, 0, 0, 0);
      vv[u] = make_uint4(0, 0, 0, 0);
      if (j < s1) {
        const int t = j & (a.P - 1);
        const int2 pg = sm_page[(j >> a.log2P) - p0];
        if (t < pg.y) {
          valid[u] = true;
          const size_t off =
              ((((size_t)pg.x * a.Hkv + g) << a.log2P) + t) * D + (size_t)c * kVec;
          kk[u] = load16_stream(a.K + off);
          vv[u] = load16_stream(a.V + off);
        }
      }
    }
    float sc[kU][G];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      float kf[kVec];
      Elem<T>::unpack(kk[u], kf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float d0 = 0.f;
#pragma unroll
        for (int e = 0; e < kVec; ++e) d0 = fmaf(qv[h][e], kf[e], d0);
        d0 = group_sum_f32<kC>(d0);
        sc[u][h] = valid[u] ? d0 : -INFINITY;
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float bm = sc[0][h];
#pragma unroll
      for (int u = 1; u < kU; ++u) bm = fmaxf(bm, sc[u][h]);
      bm = wave_max_f32(bm);
      const float mn = fmaxf(m[h], bm);
      if (mn > m[h]) {  // wave-uniform
        const float f = exp2f(m[h] - mn);  // 0 when m was -inf
        l[h] *= f;
#pragma unroll
        for (int e = 0; e < kVec; ++e) acc[h][e] *= f;
        m[h] = mn;
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      float vf[kVec];
      Elem<T>::unpack(vv[u], vf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float w = valid[u] ? exp2f(sc[u][h] - m[h]) : 0.f;
        l[h] += w;
#pragma unroll
        for (int e = 0; e < kVec; ++e) acc[h][e] = fmaf(w, vf[e], acc[h][e]);
      }
    }
  }

  // sum over the wave's token rows (lanes with the same chunk)
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int off = kC; off < kWave; off <<= 1) {
      l[h] += __shfl_xor(l[h], off, kWave);
#pragma unroll
      for (int e = 0; e < kVec; ++e) acc[h][e] += __shfl_xor(acc[h][e], off, kWave);
    }
  }
  if (r == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < kVec; ++e) sm_o[wave][h][c * kVec + e] = acc[h][e];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      sm_m[wave][h] = m[h];
      sm_l[wave][h] = l[h];
    }
  }
  __syncthreads();
  const size_t bh0 = (size_t)b * a.Hq + (size_t)g * G;
  for (int i = threadIdx.x; i < G * D; i += kSmBlock) {
    const int h = i / D, d = i % D;
    float mx = sm_m[0][h];
#pragma unroll
    for (int w = 1; w < kSmWaves; ++w) mx = fmaxf(mx, sm_m[w][h]);
    float o = 0.f, lt = 0.f;
#pragma unroll
    for (int w = 0; w < kSmWaves; ++w) {
      const float f = sm_m[w][h] == -INFINITY ? 0.f : exp2f(sm_m[w][h] - mx);
      o = fmaf(f, sm_o[w][h][d], o);
      lt = fmaf(f, sm_l[w][h], lt);
    }
    const size_t ps = (bh0 + h) * a.splits + split;
    a.part_o[ps * D + d] = o;
    if (d == 0) a.part_ml[ps] = make_float2(mx, lt);
  }
}

template <typename T, int D>
__global__ __launch_bounds__(kWave) void softmax_merge_kernel(SmArgs<T> a, float* __restrict__ out,
                                                              float* __restrict__ lse) {
  constexpr int kE = D / kWave;  // output elements per lane
  const int bh = blockIdx.x;
  const int b = bh / a.Hq, h = bh % a.Hq;
  const int pair = b * a.Hkv + h / (a.Hq / a.Hkv);
  const int lane = threadIdx.x;
  const int L = a.lens[b];
  const int npg = pair_pages(a, pair, L);
  float* o = out + (size_t)bh * D;
  if (npg <= 0) {
    // no tokens: zero output and lse = -inf; a row over the launch bound: NaN
    const float fill = npg < 0 ? NAN : 0.f;
#pragma unroll
    for (int e = 0; e < kE; ++e) o[lane + e * kWave] = fill;
    if (lse != nullptr && lane == 0) lse[bh] = npg < 0 ? NAN : -INFINITY;
    return;
  }
  const int used = ((npg << a.log2P) + a.slots - 1) / a.slots;
  const float2* ml = a.part_ml + (size_t)bh * a.splits;
  const float* po = a.part_o + (size_t)bh * a.splits * D;
  float mx = -INFINITY;
  for (int s = lane; s < used; s += kWave) mx = fmaxf(mx, ml[s].x);
  mx = wave_max_f32(mx);
  float lt = 0.f;
  float acc[kE];
#pragma unroll
  for (int e = 0; e < kE; ++e) acc[e] = 0.f;
  // kB splits per round: all their loads are issued before any is used
  constexpr int kB = 8;
  for (int s0 = 0; s0 < used; s0 += kB) {
    float2 v[kB];
    float x[kB][kE];
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      const int s = s0 + j < used ? s0 + j : used - 1;
      v[j] = ml[s];
#pragma unroll
      for (int e = 0; e < kE; ++e) x[j][e] = po[(size_t)s * D + lane + e * kWave];
    }
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      const float f = (s0 + j >= used || v[j].x == -INFINITY) ? 0.f : exp2f(v[j].x - mx);
      lt = fmaf(f, v[j].y, lt);
#pragma unroll
      for (int e = 0; e < kE; ++e) acc[e] = fmaf(f, x[j][e], acc[e]);
    }
  }
  const float inv = 1.f / lt;
#pragma unroll
  for (int e = 0; e < kE; ++e) o[lane + e * kWave] = acc[e] * inv;
  if (lse != nullptr && lane == 0) lse[bh] = kLn2 * (mx + log2f(lt));
}

template <typename T, int D, int G>
hipError_t launch_softmax_tg(const Shape& s, const SoftmaxPlan& pl, const SmArgs<T>& a,
                             float* out, float* lse, hipStream_t stream) {
  constexpr int kU = 4;
  hipLaunchKernelGGL((softmax_split_kernel<T, D, G, kU>), dim3(a.npairs * pl.splits),
                     dim3(kSmBlock), 0, stream, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((softmax_merge_kernel<T, D>), dim3(s.B * s.Hq), dim3(kWave), 0, stream, a,
                     out, lse);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_softmax_t(const Shape& s, const SoftmaxPlan& pl, const float* q, float scale,
                            const void* K, const void* V, const int32_t* bt,
                            const int32_t* lens, const int32_t* sel, const int32_t* n_sel,
                            float* out, float* lse, void* ws, hipStream_t stream) {
  SmArgs<T> a{q,      scale * kLog2e, (const T*)K, (const T*)V, bt,      lens,
              sel,    n_sel,          pl.max_sel,  s.B * s.Hkv, pl.splits, pl.slots,
              s.Hq,   s.Hkv,          s.P,         s.log2P,     s.maxP,
              (float2*)((char*)ws + pl.ml_off), (float*)((char*)ws + pl.o_off)};
  switch (s.G) {
    case 1: return launch_softmax_tg<T, D, 1>(s, pl, a, out, lse, stream);
    case 2: return launch_softmax_tg<T, D, 2>(s, pl, a, out, lse, stream);
    case 4: return launch_softmax_tg<T, D, 4>(s, pl, a, out, lse, stream);
    case 8: return launch_softmax_tg<T, D, 8>(s, pl, a, out, lse, stream);
  }
  return hipErrorInvalidValue;
}

size_t align256_sm(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

SoftmaxPlan make_softmax_plan(const Shape& s, int max_sel) {
  SoftmaxPlan pl{};
  pl.max_sel = max_sel;
  const long long slots = (long long)max_sel * s.P;
  const long long pairs = (long long)s.B * s.Hkv;
  // the largest split (a multiple of the page size) that still gives about
  // 2048 work items, between 256 and 4096 token slots and at most
  // kSmMaxPages pages
  int sps = s.P * kSmMaxPages < 4096 ? s.P * kSmMaxPages : 4096;
  while (sps > 256 && pairs * ((slots + sps - 1) / sps) < 2048) sps >>= 1;
  if (sps < s.P) sps = s.P;
  pl.slots = sps;
  pl.splits = (int)((slots + sps - 1) / sps);
  const size_t heads = (size_t)s.B * s.Hq;
  pl.ml_off = 0;
  pl.o_off = align256_sm(heads * pl.splits * sizeof(float) * 2);
  pl.total = pl.o_off + align256_sm(heads * pl.splits * (size_t)s.D * sizeof(float));
  return pl;
}

hipError_t launch_softmax(const Shape& s, const SoftmaxPlan& plan, const float* q, float scale,
                          const void* K, const void* V, const int32_t* bt, const int32_t* lens,
                          const int32_t* sel, const int32_t* n_sel, float* out, float* lse,
                          void* ws, hipStream_t stream) {
  if (s.bf16) {
    if (s.D == 128)
      return launch_softmax_t<bf16_t, 128>(s, plan, q, scale, K, V, bt, lens, sel, n_sel, out, lse, ws, stream);
    return launch_softmax_t<bf16_t, 64>(s, plan, q, scale, K, V, bt, lens, sel, n_sel, out, lse, ws, stream);
  }
  if (s.D == 128)
    return launch_softmax_t<float, 128>(s, plan, q, scale, K, V, bt, lens, sel, n_sel, out, lse, ws, stream);
  return launch_softmax_t<float, 64>(s, plan, q, scale, K, V, bt, lens, sel, n_sel, out, lse, ws, stream);
}

}  // namespace ekv
