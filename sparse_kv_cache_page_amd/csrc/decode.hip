// Sparse alpha-entmax attention over the selected pages (EntmaxKV summary
// page, §2.C: load only the selected pages' keys and values and compute the
// entmax weights over that reduced set).
//
// Entmax has no online merge rule: tau depends on every score of the head.
// The threshold does satisfy tau >= z_max - 1 (the largest weight is at most
// 1), so only tokens with z > z_max - 1 can carry weight, and since a split's
// own maximum is at most z_max, z > split_max - 1 keeps every such token.
// The decode runs in two launches:
//
//  1. qk_kernel -- work items (row, KV head, split of kR token slots).  The
//     workgroup stages the split's page map in LDS, issues all of its K-row
//     loads at once (16-byte lanes, kLpr lanes per row; rows of a page tile are
//     contiguous), and forms the scores of all G query heads of the group from
//     that one read:  z = (alpha-1) * scale * <q_h, k>  (fp32 FMA, DPP row
//     reduction).  Each wave then owns one head: it takes the split maximum and
//     writes only the candidates z > split_max - 1, as (z, physical token)
//     pairs, plus the split's count and maximum.
//
//  2. tau_pv_kernel -- one workgroup per (row, query head).  It gathers the
//     candidates of every split that clear z_max - 1 into LDS (in split order,
//     so results are reproducible; for up to 16 splits the counts, maxima and
//     first candidate slots are read in one round of loads), solves
//     sum_i [z_i - tau]_+^gamma = 1  in fp64 -- with at most 64 candidates by
//     one wave that finds the support first (tau_small), otherwise by a
//     bracketed Newton iteration -- and reads only the value rows with
//     z_i > tau (for few candidates, all their rows are requested before the
//     solve); the weights off the support are exact zeros:
//         out = sum_i p_i v_i / sum_i p_i,   p_i = (z_i - tau)^gamma.
#include <type_traits>

#include "decode_dev.h"
#include "kernels.h"

namespace ekv {
namespace {

template <typename T, int D, int G, bool kFused>
__global__ __launch_bounds__(kBlock) void qk_kernel(QkArgs<T> a, long long n_items,
                                                    TailArgs<T> ta) {
  using GE = Geo<T, D>;
  constexpr int kR = GE::kR;
  __shared__ QkLds<T, D, G> sm;
  struct NoTail {};
  __shared__ std::conditional_t<kFused, TailLds, NoTail> tl;
  __shared__ int s_last;
  __shared__ int s_wmax[kBlock / kWave];
  // the largest selection any pair uses, requested with the first item's loads
  // and reduced before the second item: items past its split count
  // (split-major numbering) are empty for every pair, so the loop stops there
  // instead of paying a round trip per empty item when selections are far
  // below max_sel
  int mx = 0;
  for (int p = threadIdx.x; p < a.npairs; p += kBlock) {
    const int np = (a.lens[p / a.Hkv] + a.P - 1) / a.P;
    mx = max(mx, min(a.sel ? a.n_sel[p] : np, a.max_sel));
  }
  long long n_used = n_items;
  bool bounded = false;
  for (long long item = blockIdx.x; item < n_used; item += gridDim.x) {
    if (!bounded && item != (long long)blockIdx.x) {  // uniform over the block
      bounded = true;
      const int wm = (int)wave_max_u32((uint32_t)mx);  // mx >= 0
      if (threadIdx.x % kWave == 0) s_wmax[threadIdx.x / kWave] = wm;
      __syncthreads();
      int m = s_wmax[0];
#pragma unroll
      for (int w = 1; w < kBlock / kWave; ++w) m = max(m, s_wmax[w]);
      // split 0 of every pair is always visited: the fused variant writes
      // the outputs of empty rows there
      const long long used = max(1LL, (((long long)m << a.log2P) + kR - 1) / kR);
      n_used = min(n_items, used * a.npairs);
      if (item >= n_used) break;
    }
    const QkItemInfo it = qk_item<T, D, G, kFused>(a, item, sm);
    if (!it.ran) {  // uniform over the block
      if constexpr (kFused) {
        // an empty row has no item to arrive: its first split writes the
        // outputs of the group's heads
        const int pair = (int)(item % a.npairs);
        if (item / a.npairs == 0 && a.lens[pair / a.Hkv] < 1) {
#pragma unroll
          for (int h = 0; h < G; ++h)
            empty_row_head(ta.out, ta.tau_out, ta.n_support, pair * G + h, D);
        }
      }
      continue;
    }
    if constexpr (kFused) {
      // arrival: this item's device-coherent stores drain, the block counts
      // itself once, and the last item of the pair runs the tau / PV tail.
      // Relaxed atomics are enough on gfx950 for the reason given at the
      // scorer's arrival (score_select_kernel): the candidate stores and the
      // tail's loads are agent-scope atomics, and s_waitcnt(0) waits for the
      // stores' acknowledgement before the increment is issued.
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (threadIdx.x == 0) {
        const int nsplit = ((it.nsel << a.log2P) + kR - 1) / kR;
        s_last = __hip_atomic_fetch_add(ta.counters + it.pair, 1, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT) == nsplit - 1;
      }
      __syncthreads();
      if (s_last) {
        const int nsel_raw = a.sel ? a.n_sel[it.pair] : it.np;
        pair_tail<T, D, G>(a.cand, a.cnt, a.smax, a.splits, ta, it.b, it.g, a.Hkv, a.P, a.log2P,
                           it.L, it.nsel, nsel_raw, a.max_sel, a.sel != nullptr, tl);
        if (threadIdx.x == 0)
          __hip_atomic_store(ta.counters + it.pair, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();  // zl and the page map are reused by the next item
  }
}

// Workgroup i probes query head i / pairs of (row, KV head) pair i % pairs:
// consecutive workgroups go to the 8 XCDs in turn, so (for a pair count that
// is a multiple of 8) the G heads of a pair run on one XCD and share its L2
// lines of the pair's page-major bounds.
template <typename T, int D>
__global__ __launch_bounds__(kBlock) void zlb_kernel(ZlbArgs<T> a) {
  const int G = a.Hq / a.Hkv;
  const int npairs = (int)(gridDim.x / (unsigned)G);  // B * Hkv
  const int pair = (int)(blockIdx.x % (unsigned)npairs);
  const int i = (int)(blockIdx.x / (unsigned)npairs);
  zlb_head<T, D>(a, (pair / a.Hkv) * a.Hq + (pair % a.Hkv) * G + i);
}

template <typename T, int D>
__global__ __launch_bounds__(kBlock) void tau_pv_kernel(TauArgs<T> a) {
  __shared__ TauLds<T, D> sm;
  tau_head<T, D>(a, blockIdx.x, sm);
}

template <typename T, int D, int G, bool kFused>
hipError_t launch_qk_t(const Shape& s, const DecodePlan& pl, const float* q, float zscale,
                       float a1, const void* K, const int32_t* bt, const int32_t* lens,
                       const int32_t* sel, const int32_t* n_sel, const float* ub,
                       const float* zlb, float2* cand, int* cnt, float* smax,
                       const TailArgs<T>& ta, hipStream_t stream) {
  const long long items = (long long)s.B * s.Hkv * pl.splits;
  // the fused variant keeps its tail's registers: 2 resident blocks per CU,
  // so one round of persistent blocks; the plain variant fits 4 per CU
  const long long cap = kFused ? 256LL * 2 : pl.qk_grid_cap;
  const long long grid = items < cap ? items : cap;
  const QkArgs<T> a{q,      zscale,  (const T*)K, bt,       lens,      sel,  n_sel,
                    pl.max_sel, s.Hkv, s.P,    s.log2P,  s.maxP,    pl.splits,
                    cand,   cnt,     smax,        ub,       zlb,       a1,
                    (int)(s.B * s.Hkv)};
  hipLaunchKernelGGL((qk_kernel<T, D, G, kFused>), dim3((unsigned)grid), dim3(kBlock), 0, stream,
                     a, items, ta);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_decode_t(const Shape& s, const DecodePlan& pl, const float* q, float scale,
                           float alpha, const void* K, const void* V, const int32_t* bt,
                           const int32_t* lens, const int32_t* sel, const int32_t* n_sel,
                           const float* ub, float* zlb, float* out, float* tau_out,
                           int32_t* n_support, void* ws, bool fused, hipStream_t stream) {
  float2* cand = (float2*)((char*)ws + pl.cand_off);
  int* cnt = (int*)((char*)ws + pl.cnt_off);
  float* smax = (float*)((char*)ws + pl.smax_off);
  const double a1 = (double)alpha - 1.0;
  const float zscale = (float)(a1 * (double)scale);
  const double gamma = 1.0 / a1;
  const double gr = rint(gamma);
  const int gamma_int = (gr >= 1.0 && gr <= 64.0 && fabs(gamma - gr) <= 1e-12 * gr) ? (int)gr : 0;
  TailArgs<T> ta{(const T*)V, fused ? (int*)((char*)ws + pl.counter_off) : nullptr, (double)alpha,
                 gamma_int ? gr : gamma, gamma_int, out, tau_out, n_support};
  if (ub != nullptr) {
    // page pruning: per-head lower bounds of z_max, read by the qk stage
    const ZlbArgs<T> za{q, zscale, (const T*)K, bt, lens, sel, n_sel, pl.max_sel, s.Hq, s.Hkv,
                        s.P, s.maxP, ub, zlb};
    hipLaunchKernelGGL((zlb_kernel<T, D>), dim3(s.B * s.Hq), dim3(kBlock), 0, stream, za);
    const hipError_t pe = hipGetLastError();
    if (pe != hipSuccess) return pe;
  }
  hipError_t e = hipErrorInvalidValue;
  if (fused) {
    switch (s.G) {
      case 1: e = launch_qk_t<T, D, 1, true>(s, pl, q, zscale, (float)a1, K, bt, lens, sel, n_sel, ub, zlb, cand, cnt, smax, ta, stream); break;
      case 2: e = launch_qk_t<T, D, 2, true>(s, pl, q, zscale, (float)a1, K, bt, lens, sel, n_sel, ub, zlb, cand, cnt, smax, ta, stream); break;
      case 4: e = launch_qk_t<T, D, 4, true>(s, pl, q, zscale, (float)a1, K, bt, lens, sel, n_sel, ub, zlb, cand, cnt, smax, ta, stream); break;
      case 8: e = launch_qk_t<T, D, 8, true>(s, pl, q, zscale, (float)a1, K, bt, lens, sel, n_sel, ub, zlb, cand, cnt, smax, ta, stream); break;
    }
    return e;
  }
  switch (s.G) {
    case 1: e = launch_qk_t<T, D, 1, false>(s, pl, q, zscale, (float)a1, K, bt, lens, sel, n_sel, ub, zlb, cand, cnt, smax, ta, stream); break;
    case 2: e = launch_qk_t<T, D, 2, false>(s, pl, q, zscale, (float)a1, K, bt, lens, sel, n_sel, ub, zlb, cand, cnt, smax, ta, stream); break;
    case 4: e = launch_qk_t<T, D, 4, false>(s, pl, q, zscale, (float)a1, K, bt, lens, sel, n_sel, ub, zlb, cand, cnt, smax, ta, stream); break;
    case 8: e = launch_qk_t<T, D, 8, false>(s, pl, q, zscale, (float)a1, K, bt, lens, sel, n_sel, ub, zlb, cand, cnt, smax, ta, stream); break;
  }
  if (e != hipSuccess) return e;
  const TauArgs<T> ta2{cand, cnt, smax, pl.splits, (const T*)V, lens, n_sel, sel != nullptr,
                       pl.max_sel, s.Hq, s.Hkv, s.P, s.log2P, (double)alpha,
                       gamma_int ? gr : gamma, gamma_int, out, tau_out, n_support};
  hipLaunchKernelGGL((tau_pv_kernel<T, D>), dim3(s.B * s.Hq), dim3(kBlock), 0, stream, ta2);
  return hipGetLastError();
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int slots_per_item(const Shape& s) {
  if (s.bf16) return s.D == 128 ? Geo<bf16_t, 128>::kR : Geo<bf16_t, 64>::kR;
  return s.D == 128 ? Geo<float, 128>::kR : Geo<float, 64>::kR;
}

}  // namespace

bool decode_shape_supported(const Shape& s, int max_sel) {
  const long long slots = (long long)max_sel * s.P;
  const long long splits = (slots + slots_per_item(s) - 1) / slots_per_item(s);
  return splits <= kMaxSplitsTotal && (long long)s.Np * s.P < (1LL << 31);
}

DecodePlan make_decode_plan(const Shape& s, int max_sel, bool fused) {
  DecodePlan pl{};
  pl.max_sel = max_sel;
  pl.slots_per_item = slots_per_item(s);
  const long long slots = (long long)max_sel * s.P;
  pl.splits = (int)((slots + pl.slots_per_item - 1) / pl.slots_per_item);
  pl.qk_grid_cap = 256LL * 16;  // CUs x resident workgroups; items beyond loop
  const size_t heads = (size_t)s.B * s.Hq;
  pl.counter_off = 0;
  pl.counter_bytes = fused ? align256((size_t)s.B * s.Hkv * sizeof(int)) : 0;
  pl.cand_off = pl.counter_off + pl.counter_bytes;
  pl.cand_bytes = align256(heads * pl.splits * (size_t)pl.slots_per_item * sizeof(float) * 2);
  pl.cnt_off = pl.cand_off + pl.cand_bytes;
  pl.cnt_bytes = align256(heads * pl.splits * sizeof(int));
  pl.smax_off = pl.cnt_off + pl.cnt_bytes;
  pl.smax_bytes = align256(heads * pl.splits * sizeof(float));
  pl.total = pl.smax_off + pl.smax_bytes;
  return pl;
}

hipError_t launch_decode(const Shape& s, const DecodePlan& plan, const float* q, float scale,
                         float alpha, const void* K, const void* V, const int32_t* bt,
                         const int32_t* lens, const int32_t* sel, const int32_t* n_sel,
                         const float* ub, float* zlb, float* out, float* tau_out,
                         int32_t* n_support, void* ws, bool fused, hipStream_t stream) {
  if (s.bf16) {
    if (s.D == 128)
      return launch_decode_t<bf16_t, 128>(s, plan, q, scale, alpha, K, V, bt, lens, sel, n_sel, ub, zlb, out, tau_out, n_support, ws, fused, stream);
    return launch_decode_t<bf16_t, 64>(s, plan, q, scale, alpha, K, V, bt, lens, sel, n_sel, ub, zlb, out, tau_out, n_support, ws, fused, stream);
  }
  if (s.D == 128)
    return launch_decode_t<float, 128>(s, plan, q, scale, alpha, K, V, bt, lens, sel, n_sel, ub, zlb, out, tau_out, n_support, ws, fused, stream);
  return launch_decode_t<float, 64>(s, plan, q, scale, alpha, K, V, bt, lens, sel, n_sel, ub, zlb, out, tau_out, n_support, ws, fused, stream);
}

}  // namespace ekv
