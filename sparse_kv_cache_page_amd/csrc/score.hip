// Query-aware page scorer (EntmaxKV summary page, §2.A: a deterministic upper
// bound on the largest score of any token of a page from its bounding box, and
// the Gaussian moments of the page's scores from its key mean/variance).
//
// For one query head and one page,
//     sum_j max(q_j kmin_j, q_j kmax_j)
//       = 1/2 sum_j q_j (kmax_j + kmin_j) + |q_j| (kmax_j - kmin_j)
// because the larger end point is kmax when q_j >= 0 and kmin otherwise.  The
// sum, the difference and the two products are formed in fp64 (exact unless
// kmin_j and kmax_j differ by more than 2^45 in magnitude for bf16, 2^29 for
// fp32; otherwise rounded to 53 bits), the terms are added by an fp64 FMA
// chain, and the bound is then halved, scaled and rounded once to fp32: it is
// within an fp32 rounding of the exact value.  This form keeps one fp64 copy
// of q in registers instead of the two halves q+ and q-.
//
// Mapping: workgroup i scores page slice i / pairs of (row, KV head) pair
// i % pairs.  Consecutive workgroups go to the 8 XCDs in turn, so with the
// pair varying fastest every XCD gets the same share of every slice index
// (with 8 KV heads, XCD g holds KV head g of every row): rows of different
// lengths, whose late slices exist only for long rows, cannot pile work onto
// a few XCDs while the others idle.  kLpr lanes cover one page's d
// coordinates with kVec coordinates each (16- or 8-byte loads of kmin and
// kmax), so a wave scores 64/kLpr pages per step for all G query heads of the
// group; the per-head partial sums are finished through LDS.  q stays in
// registers as fp64 for the whole launch.
#include "blocks.h"
#include "kernels.h"

namespace ekv {
namespace {

// Raw storage of one lane's slice of a metadata row (kVec elements of T).
template <int kBytes> struct RawT;
template <> struct RawT<16> {
  using type = uint4;
  __device__ static type load(const void* p) { return load16_stream(p); }
};
template <> struct RawT<8> {
  using type = uint2;
  __device__ static type load(const void* p) { return load8_stream(p); }
};

template <typename T, int N> struct Unpack;
template <> struct Unpack<bf16_t, 8> {
  __device__ static void run(const uint4& w, float* x) { Elem<bf16_t>::unpack(w, x); }
};
template <> struct Unpack<bf16_t, 4> {
  __device__ static void run(const uint2& w, float* x) {
    x[0] = __uint_as_float(w.x << 16);
    x[1] = __uint_as_float(w.x & 0xffff0000u);
    x[2] = __uint_as_float(w.y << 16);
    x[3] = __uint_as_float(w.y & 0xffff0000u);
  }
};
template <> struct Unpack<float, 4> {
  __device__ static void run(const uint4& w, float* x) { Elem<float>::unpack(w, x); }
};
template <> struct Unpack<float, 2> {
  __device__ static void run(const uint2& w, float* x) {
    x[0] = __uint_as_float(w.x);
    x[1] = __uint_as_float(w.y);
  }
};

#ifndef EKV_SCORE_G4_BYTES
#define EKV_SCORE_G4_BYTES 16
#endif
#ifndef EKV_SCORE_DEPTH
#define EKV_SCORE_DEPTH 2
#endif
#ifndef EKV_SCORE_RESIDENT
#define EKV_SCORE_RESIDENT 512
#endif
constexpr int kScoreDepth = EKV_SCORE_DEPTH;  // metadata batches per lane in flight
#ifndef EKV_SCORE_MAX_U
#define EKV_SCORE_MAX_U 4
#endif
constexpr int kScoreMaxU = EKV_SCORE_MAX_U;  // pages per lane per batch, at most
constexpr int kScoreBlock = 256;
constexpr int kScoreWaves = kScoreBlock / kWave;
constexpr int kMaxPagesPerBlock = 512;  // block-table slice staged in LDS
constexpr int kStepTopkKeys = 4096;
// workgroups resident at once (256 CUs x 2 at this kernel's register use):
// one round of blocks avoids a second ramp-up
constexpr int kScoreResidentBlocks = EKV_SCORE_RESIDENT;

// Work split of score_range.  kLpr lanes share one page (kVec coordinates
// each); a lane scores kU pages per batch and keeps kKinds partial sums per
// (page, head): the bound, plus the Gaussian mean and variance.  The kM
// partial sums of a lane are finished through LDS: rows of kPitch doubles
// (odd, so that both the row-wise writes and the column-wise reads of a
// half-wave touch distinct banks).
template <int D, int G, int kVec, bool kGauss>
struct ScoreGeo {
  static constexpr int kLpr = D / kVec;
  static constexpr int kKinds = kGauss ? 3 : 1;
  static constexpr int kLanesUsed = kLpr < 16 ? kLpr : 16;
  static constexpr int kUfit = kLanesUsed / (G * kKinds);
  static constexpr int kU = kUfit < 1 ? 1 : (kUfit > kScoreMaxU ? kScoreMaxU : kUfit);
  static constexpr int kM = kU * kKinds * G;
  static constexpr int kPitch = kM + 1;
};

template <int kPitch>
struct ScoreRedLds {
  double v[kScoreWaves][kWave][kPitch];
};

// Orders the LDS accesses of one wave around an exchange between its lanes
// (a wave's LDS instructions execute in program order).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// This lane's query coordinates for score_range, as fp64: heads of the
// group, coordinates c * kVec .. of its page slot (loaded by the caller, so
// that they share the round trip of the block-table slice).
template <int D, int G, int kVec>
__device__ __forceinline__ void load_q_lane(const float* __restrict__ q, int b, int g, int Hkv,
                                            double (&qd)[G][kVec]) {
  const int c = (threadIdx.x % kWave) % (D / kVec);
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float* qh = q + ((size_t)b * Hkv * G + g * G + h) * D + c * kVec;
#pragma unroll
    for (int v = 0; v < kVec; ++v) qd[h][v] = (double)qh[v];
  }
}

// Scores of pages [p_begin, p_end) of one (row b, KV head g) for the G query
// heads of the group (qd: this lane's coordinates of the group's queries,
// from load_q_lane); s_pi holds the block-table slice block_table[b][p_begin..),
// red is this wave's reduction scratch (kWave rows of kPitch doubles).
//
// Each lane forms, for each of its kU pages and each head, the fp64 partial
// sum over its kVec coordinates and stores it in its LDS row; then lane
// (slot, c) adds column c of the kLpr rows of its page slot in a fixed order,
// so every (page, head) total is finished by one lane, and the group maximum
// is taken over the G lanes that hold one page's heads.
//
// lbest / lbestp: this lane's largest bound and its page so far (the lane
// finishes the bounds of head lane % G only, in increasing page order).
template <typename T, int D, int G, int kVec, bool kGauss, bool kCoherentU = false,
          typename M = float>
__device__ __forceinline__ void score_range(
    const double (&qd)[G][kVec], float scale, const T* __restrict__ kmin,
    const T* __restrict__ kmax, const M* __restrict__ mean, const M* __restrict__ var,
    const int* s_pi, int b, int g, int pair, int Hkv, int maxP, int p_begin, int p_end,
    float* __restrict__ ub, float* __restrict__ ubg, double* __restrict__ gm,
    double* __restrict__ gv, double (*red)[ScoreGeo<D, G, kVec, kGauss>::kPitch],
    float& lbest, int& lbestp) {
  using Geo = ScoreGeo<D, G, kVec, kGauss>;
  constexpr int kLpr = Geo::kLpr;
  constexpr int kPagesPerWave = kWave / kLpr;
  constexpr int kPagesPerStep = kPagesPerWave * kScoreWaves;
  constexpr int kU = Geo::kU;
  constexpr int kKinds = Geo::kKinds;
  constexpr int kM = Geo::kM;
  constexpr int kRawBytes = kVec * (int)sizeof(T);
  constexpr int kMomRaw = kVec * (int)sizeof(M);   // bytes of mean (or var) per lane
  using Raw = RawT<kRawBytes>;
  static_assert(kLpr % G == 0, "a page's heads sit in aligned lane groups");
  const int Hq = Hkv * G;
  const int lane = threadIdx.x % kWave;
  const int c = lane % kLpr;
  const int slot = threadIdx.x / kLpr;  // page slot inside a step
  const int r0 = lane - c;              // first LDS row of this lane's slot

  const double dscale = (double)scale;

  // one batch = kU pages per lane; the next batch's loads are issued before
  // the current batch is reduced, so a wave always has loads in flight
  struct Batch {
    typename Raw::type lo[kU], hi[kU];
    float mu[kGauss ? kU : 1][kVec], s2[kGauss ? kU : 1][kVec];
  };
  auto issue = [&](int base, Batch& bt_) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int p = base + slot + u * kPagesPerStep;
      const int pl = (p < p_end ? p : p_begin) - p_begin;
      const size_t off = ((size_t)s_pi[pl] * Hkv + g) * D + c * kVec;
      bt_.lo[u] = Raw::load(kmin + off);
      bt_.hi[u] = Raw::load(kmax + off);
      if constexpr (kGauss && sizeof(M) == 2) {
        // compact (bf16) moments: kVec values in 2 kVec bytes
        if constexpr (kMomRaw == 16) {
          Elem<bf16_t>::unpack(load16_stream(mean + off), bt_.mu[u]);
          Elem<bf16_t>::unpack(load16_stream(var + off), bt_.s2[u]);
        } else if constexpr (kMomRaw == 8) {
          Unpack<bf16_t, 4>::run(load8_stream(mean + off), bt_.mu[u]);
          Unpack<bf16_t, 4>::run(load8_stream(var + off), bt_.s2[u]);
        } else {
          const uint32_t wm = *reinterpret_cast<const uint32_t*>(mean + off);
          const uint32_t wv = *reinterpret_cast<const uint32_t*>(var + off);
          bt_.mu[u][0] = __uint_as_float(wm << 16);
          bt_.mu[u][1] = __uint_as_float(wm & 0xffff0000u);
          bt_.s2[u][0] = __uint_as_float(wv << 16);
          bt_.s2[u][1] = __uint_as_float(wv & 0xffff0000u);
        }
      } else if constexpr (kGauss) {
        if constexpr (kMomRaw == 32) {
          Elem<float>::unpack(load16_stream(mean + off), bt_.mu[u]);
          Elem<float>::unpack(load16_stream(mean + off + 4), bt_.mu[u] + 4);
          Elem<float>::unpack(load16_stream(var + off), bt_.s2[u]);
          Elem<float>::unpack(load16_stream(var + off + 4), bt_.s2[u] + 4);
        } else if constexpr (kMomRaw == 16) {
          Elem<float>::unpack(load16_stream(mean + off), bt_.mu[u]);
          Elem<float>::unpack(load16_stream(var + off), bt_.s2[u]);
        } else {
          Unpack<float, 2>::run(load8_stream(mean + off), bt_.mu[u]);
          Unpack<float, 2>::run(load8_stream(var + off), bt_.s2[u]);
        }
      }
    }
  };
  auto consume = [&](int base, const Batch& bt_) {
    double* row = red[lane];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      float lo[kVec], hi[kVec];
      Unpack<T, kVec>::run(bt_.lo[u], lo);
      Unpack<T, kVec>::run(bt_.hi[u], hi);
      // max(x kmin, x kmax) = (x (kmax + kmin) + |x| (kmax - kmin)) / 2, the
      // halving applied to the finished sum (exact)
      double sm2[kVec], df2[kVec];
#pragma unroll
      for (int v = 0; v < kVec; ++v) {
        sm2[v] = (double)hi[v] + (double)lo[v];
        df2[v] = (double)hi[v] - (double)lo[v];
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        double a = 0.0;
#pragma unroll
        for (int v = 0; v < kVec; ++v) {
          a = fma(qd[h][v], sm2[v], a);
          a = fma(fabs(qd[h][v]), df2[v], a);
        }
        row[u * kKinds * G + h] = a;
      }
      if constexpr (kGauss) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          double am = 0.0, av = 0.0;
#pragma unroll
          for (int v = 0; v < kVec; ++v) {
            am = fma(qd[h][v], (double)bt_.mu[u][v], am);
            av = fma(qd[h][v] * qd[h][v], (double)bt_.s2[u][v], av);
          }
          row[(u * kKinds + 1) * G + h] = am;
          row[(u * kKinds + 2) * G + h] = av;
        }
      }
    }
    wave_lds_sync();
#pragma unroll
    for (int it = 0; it < (kM + kLpr - 1) / kLpr; ++it) {
      const int m = it * kLpr + c;
      const bool have = m < kM;
      const int u = m / (kKinds * G);
      const int kind = (m / G) % kKinds;
      const int h = m % G;
      const int p = base + slot + u * kPagesPerStep;
      // pairwise sum of the slot's kLpr partials of combination m
      double part[kLpr];
#pragma unroll
      for (int i = 0; i < kLpr; ++i) part[i] = have ? red[r0 + i][m] : 0.0;
#pragma unroll
      for (int w = kLpr / 2; w >= 1; w /= 2) {
#pragma unroll
        for (int i = 0; i < w; ++i) part[i] += part[i + w];
      }
      const double t = part[0];
      const bool live = have && p < p_end;
      const size_t o = ((size_t)b * Hq + g * G + h) * maxP + p;
      const float uh = (float)(dscale * (kind == 0 ? 0.5 * t : t));
      // per-head bounds page-major ([pair][page][G]): the G heads of a page sit
      // in adjacent lanes and adjacent words, so the stores coalesce and a
      // reader of one page gets all its heads from one 4G-byte chunk
      if (kind == 0 && live && ub != nullptr) ub[((size_t)pair * maxP + p) * G + h] = uh;
      if (kind == 0 && live && uh > lbest) {  // pages increase: ties keep the lower
        lbest = uh;
        lbestp = p;
      }
      if constexpr (kGauss) {
        if (kind == 1 && live) gm[o] = dscale * t;
        if (kind == 2 && live) gv[o] = dscale * dscale * t;
      }
      const float best = group_max_f32<G>(have && kind == 0 ? uh : -__builtin_huge_valf());
      if (kind == 0 && h == 0 && live) {
        // the fused select reads these bounds from another workgroup (maybe
        // on another XCD): device-coherent stores there, plain ones otherwise
        if constexpr (kCoherentU)
          __hip_atomic_store(ubg + (size_t)pair * maxP + p, best, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        else
          ubg[(size_t)pair * maxP + p] = best;
      }
    }
    wave_lds_sync();
  };
  // kDepth batches in a ring: while one is reduced, the next kDepth - 1 are
  // in flight; a reduced batch's registers take the batch kDepth steps on
  constexpr int kStride = kPagesPerStep * kU;
  constexpr int kDepth = kScoreDepth;
  Batch ring[kDepth];
#pragma unroll
  for (int d = 0; d < kDepth; ++d)
    if (p_begin + d * kStride < p_end) issue(p_begin + d * kStride, ring[d]);
  bool done = false;
  for (int base = p_begin; !done; base += kDepth * kStride) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      const int cur = base + d * kStride;
      if (!done && cur >= p_end) done = true;
      if (!done) {
        consume(cur, ring[d]);
        if (cur + kDepth * kStride < p_end) issue(cur + kDepth * kStride, ring[d]);
      }
    }
  }
}

// The slice's best page for each head of the group (largest bound, lowest
// page on ties) from the lanes' running bests: lane l follows head l % G.
// Written as {bound bits, page, physical page, 0} to
// hint[(pair * nslices + slice) * G + h]; a slice without a finite bound
// gets page -1.  Called by all threads after the scoring loop.
template <int G>
__device__ __forceinline__ void write_slice_best(float lbest, int lbestp, const int* s_pi,
                                                 int p_begin, int4* __restrict__ hint,
                                                 float (*sb)[G], int (*sp)[G]) {
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const bool mine = lane % G == h;
    const float wb = wave_max_f32(mine ? lbest : -__builtin_huge_valf());
    const uint32_t wp =
        wave_min_u32(mine && lbest == wb ? (uint32_t)lbestp : 0xFFFFFFFFu);
    if (lane == 0) {
      sb[wave][h] = wb;
      sp[wave][h] = (int)wp;
    }
  }
  __syncthreads();
  if (threadIdx.x < G) {
    const int h = threadIdx.x;
    float bv = sb[0][h];
    int bp = sp[0][h];
#pragma unroll
    for (int w = 1; w < kScoreWaves; ++w)
      if (sb[w][h] > bv || (sb[w][h] == bv && (uint32_t)sp[w][h] < (uint32_t)bp)) {
        bv = sb[w][h];
        bp = sp[w][h];
      }
    const bool ok = bv > -__builtin_huge_valf() && bp >= p_begin;
    hint[h] = make_int4(__float_as_int(bv), ok ? bp : -1, ok ? s_pi[bp - p_begin] : 0, 0);
  }
}

// Pages per workgroup: whole batches of per_iter pages, enough workgroups to
// fill the chip once (kScoreResidentBlocks) for short batches, and at most
// kSlicePages, so long rows are cut into many slices that later workgroups
// pick up as earlier ones finish (ragged rows then finish together).
constexpr int kSlicePages = kMaxPagesPerBlock;

int slice_pages(const Shape& s, int per_iter) {
  const long long pairs = (long long)s.B * s.Hkv;
  const long long want_blocks_per_pair = (kScoreResidentBlocks + pairs - 1) / pairs;
  int iters = (int)((s.maxP + per_iter * want_blocks_per_pair - 1) / (per_iter * want_blocks_per_pair));
  const int max_iters = kSlicePages > per_iter ? kSlicePages / per_iter : 1;
  if (iters > max_iters) iters = max_iters;
  if (iters < 1) iters = 1;
  return per_iter * iters;
}

// refresh (box-only metadata): the workgroup holding a row's last page first
// rebuilds that page's bounding box from the K rows (the page a decode step
// has just appended to); only this workgroup reads it, so the barrier below,
// which waits for the stores, publishes it.
template <typename T, int D, int G, int kVec, bool kGauss, typename M = float>
__global__ __launch_bounds__(kScoreBlock) void score_kernel(
    const float* __restrict__ q, float scale, T* __restrict__ kmin,
    T* __restrict__ kmax, const M* __restrict__ mean, const M* __restrict__ var,
    const int32_t* __restrict__ bt, const int32_t* __restrict__ lens, int Hkv, int P, int maxP,
    int pages_per_block, int npairs, float* __restrict__ ub, float* __restrict__ ubg,
    double* __restrict__ gm, double* __restrict__ gv, const T* __restrict__ K, int refresh,
    int4* __restrict__ hint, int nslices) {
  using Geo = ScoreGeo<D, G, kVec, kGauss>;
  __shared__ int s_pi[kMaxPagesPerBlock];
  __shared__ ScoreRedLds<Geo::kPitch> red;
  __shared__ float s_hb[kScoreWaves][G];
  __shared__ int s_hp[kScoreWaves][G];
  const int pair = (int)(blockIdx.x % (unsigned)npairs);
  const int b = pair / Hkv;
  const int g = pair % Hkv;
  const int p_begin = (int)(blockIdx.x / (unsigned)npairs) * pages_per_block;
  // the block-table slice is read in the same round trip as the row length
  // (entries past the row's pages are in bounds and never used)
  for (int i = threadIdx.x; i < pages_per_block && p_begin + i < maxP; i += kScoreBlock)
    s_pi[i] = bt[(size_t)b * maxP + p_begin + i];
  double qd[G][kVec];
  load_q_lane<D, G, kVec>(q, b, g, Hkv, qd);
  const int L = lens[b];
  const int np = (L + P - 1) / P;
  if (p_begin >= np) return;
  const int p_end = min(np, p_begin + pages_per_block);
  if constexpr (!kGauss) {
    if (refresh && p_end == np && threadIdx.x < kWave)
      meta_tile<T, D, float>(K, Hkv, P, bt[(size_t)b * maxP + np - 1], g,
                             page_valid(L, np - 1, P), kmin, kmax, nullptr, nullptr);
  }
  __syncthreads();
  float lbest = -__builtin_huge_valf();
  int lbestp = 0x7fffffff;
  score_range<T, D, G, kVec, kGauss, false, M>(qd, scale, kmin, kmax, mean, var, s_pi, b, g, pair,
                                               Hkv, maxP, p_begin, p_end, ub, ubg, gm, gv,
                                               red.v[threadIdx.x / kWave], lbest, lbestp);
  if (hint != nullptr)
    write_slice_best<G>(lbest, lbestp, s_pi, p_begin,
                        hint + ((size_t)pair * nslices + p_begin / pages_per_block) * G, s_hb,
                        s_hp);
}

// Fused first half of a decode step (top-k policy): optionally rebuild the
// metadata of each row's last page (the page the new token went to), score
// the pages, and let the last workgroup to finish a (row, KV head) run the
// top-k selection over that pair's bounds.  Arrivals are counted in
// `counters` [B*Hkv], which start at zero and are reset by the last arrival.
template <typename T, int D, int G, int kVec, bool kKeysLds>
__global__ __launch_bounds__(kScoreBlock) void score_select_kernel(
    const float* __restrict__ q, float scale, const T* __restrict__ K, T* __restrict__ kmin,
    T* __restrict__ kmax, const int32_t* __restrict__ bt, const int32_t* __restrict__ lens,
    int refresh, int Hkv, int P, int maxP, int pages_per_block, int npairs,
    float* __restrict__ ub, float* __restrict__ ubg,
    int top_k, int32_t* __restrict__ sel, int32_t* __restrict__ n_sel,
    int* __restrict__ counters) {
  using Geo = ScoreGeo<D, G, kVec, false>;
  // the scoring reduction and the selection never use LDS at the same time
  union Lds {
    ScoreRedLds<Geo::kPitch> red;
    TopkRegLds tkr;
    TopkLds<1> tk;
  };
  __shared__ int s_pi[kMaxPagesPerBlock];
  __shared__ Lds sm;
  __shared__ int s_last;
  const int pair = (int)(blockIdx.x % (unsigned)npairs);
  const int b = pair / Hkv;
  const int g = pair % Hkv;
  const int p_begin = (int)(blockIdx.x / (unsigned)npairs) * pages_per_block;
  // the block-table slice is read in the same round trip as the row length
  // (entries past the row's pages are in bounds and never used)
  for (int i = threadIdx.x; i < pages_per_block && p_begin + i < maxP; i += kScoreBlock)
    s_pi[i] = bt[(size_t)b * maxP + p_begin + i];
  double qd[G][kVec];
  load_q_lane<D, G, kVec>(q, b, g, Hkv, qd);
  const int L = lens[b];
  const int np = (L + P - 1) / P;
  if (p_begin >= np) {
    // an empty row has no slice to count: its first workgroup records the
    // empty selection
    if (np == 0 && p_begin == 0 && threadIdx.x == 0) n_sel[pair] = 0;
    return;
  }
  const int p_end = min(np, p_begin + pages_per_block);
  if (refresh && p_end == np && threadIdx.x < kWave) {
    // only this workgroup reads the refreshed page's box: the barrier below
    // (which waits for the stores) is enough to publish it
    meta_tile<T, D, float>(K, Hkv, P, bt[(size_t)b * maxP + np - 1], g,
                           page_valid(L, np - 1, P), kmin, kmax, nullptr, nullptr);
  }
  __syncthreads();
  float lbest = -__builtin_huge_valf();
  int lbestp = 0x7fffffff;
  score_range<T, D, G, kVec, false, true, float>(qd, scale, kmin, kmax, nullptr, nullptr, s_pi, b,
                                                 g, pair, Hkv, maxP, p_begin, p_end, ub, ubg,
                                                 nullptr, nullptr, sm.red.v[threadIdx.x / kWave],
                                                 lbest, lbestp);
  // arrival: every wave waits until its device-coherent bound stores have
  // completed, the barrier gathers the waves, then one relaxed device-scope
  // increment counts the block; the last block of the pair reads every bound
  // back with device-coherent loads.  No cache-wide write-back or
  // invalidation is needed.  Why relaxed atomics suffice here (the HIP
  // memory model alone would want a release on the increment and an acquire
  // in the last block): the bound stores and the loads that read them back
  // bypass the non-coherent caches (agent-scope atomic stores and loads), and
  // s_waitcnt(0) returns only after each store has been acknowledged by the
  // device-coherent level, before the increment is issued; a block that sees
  // the final count therefore finds every other block's stores there.  This
  // rests on how gfx950 executes these instructions, not on the language
  // model; the fused decode's arrival relies on the same argument.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const int nblk = (np + pages_per_block - 1) / pages_per_block;
    s_last = __hip_atomic_fetch_add(&counters[pair], 1, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT) == nblk - 1;
  }
  __syncthreads();
  if (!s_last) return;
  const int k = min(top_k, np);
  int32_t* out = sel + (size_t)pair * maxP;
  if (k >= np) {
    for (int p = threadIdx.x; p < np; p += kScoreBlock) out[p] = p;
  } else if (np <= kBlk * 8) {
    topk_block_reg<8, true>(ubg + (size_t)pair * maxP, np, k, out, sm.tkr);
  } else if (np <= kBlk * 16) {
    topk_block_reg<16, true>(ubg + (size_t)pair * maxP, np, k, out, sm.tkr);
  } else {
    topk_block<false, true>(ubg + (size_t)pair * maxP, np, k, out, sm.tk);
  }
  if (threadIdx.x == 0) {
    n_sel[pair] = k;
    __hip_atomic_store(&counters[pair], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace
ScoreSlices score_box_slices(const Shape& s);
namespace {

template <typename T, int D, int G, int kVec>
hipError_t launch_score_t(const Shape& s, const float* q, float scale, const void* kmin,
                          const void* kmax, const void* mean, const void* var,
                          const int32_t* bt, const int32_t* lens, float* ub, float* ubg,
                          double* gm, double* gv, const void* K, int refresh, int4* hint,
                          hipStream_t stream) {
  constexpr int kLpr = D / kVec;
  constexpr int kPagesPerStep = (kWave / kLpr) * kScoreWaves;
  const bool gauss = gm != nullptr;
  const int per_iter = kPagesPerStep * (gauss ? ScoreGeo<D, G, kVec, true>::kU
                                              : ScoreGeo<D, G, kVec, false>::kU);
  // enough blocks to spread the pairs over the chip (~4 per CU), each block
  // a whole number of iterations (for the box bounds alone, the slices that
  // score_box_slices reports, which size the best-page hints)
  const long long pairs = (long long)s.B * s.Hkv;
  const int ppb = gauss ? slice_pages(s, per_iter) : score_box_slices(s).pages;
  if (!gauss && ppb != slice_pages(s, per_iter)) return hipErrorInvalidValue;
  const long long nblocks = (long long)((s.maxP + ppb - 1) / ppb) * pairs;
  if (nblocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)nblocks);
  const int npairs = (int)pairs;
  if (gauss && s.mom16) {
    hipLaunchKernelGGL((score_kernel<T, D, G, kVec, true, bf16_t>), grid, dim3(kScoreBlock), 0,
                       stream, q, scale, (T*)kmin, (T*)kmax, (const bf16_t*)mean,
                       (const bf16_t*)var, bt, lens, s.Hkv, s.P, s.maxP, ppb, npairs, ub, ubg, gm,
                       gv, (const T*)K, 0, nullptr, 0);
  } else if (gauss) {
    hipLaunchKernelGGL((score_kernel<T, D, G, kVec, true>), grid, dim3(kScoreBlock), 0, stream, q,
                       scale, (T*)kmin, (T*)kmax, (const float*)mean,
                       (const float*)var, bt, lens, s.Hkv, s.P, s.maxP, ppb, npairs, ub, ubg, gm,
                       gv, (const T*)K, 0, nullptr, 0);
  } else {
    hipLaunchKernelGGL((score_kernel<T, D, G, kVec, false>), grid, dim3(kScoreBlock), 0, stream,
                       q, scale, (T*)kmin, (T*)kmax, (const float*)nullptr,
                       (const float*)nullptr, bt, lens, s.Hkv, s.P, s.maxP, ppb, npairs, ub, ubg,
                       gm, gv, (const T*)K, refresh, hint, (s.maxP + ppb - 1) / ppb);
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_score_d(const Shape& s, const float* q, float scale, const void* kmin,
                          const void* kmax, const void* mean, const void* var,
                          const int32_t* bt, const int32_t* lens, float* ub, float* ubg,
                          double* gm, double* gv, const void* K, int refresh, int4* hint,
                          hipStream_t stream) {
  // 16-byte loads while q+/q- fit comfortably in registers, 8-byte loads for
  // the 8-head group (halves the per-lane coordinates, hence the registers),
  // and for the 4-head group when the Gaussian moments are summed too: with
  // 16-byte loads that kernel needed 256 VGPRs + 104 AGPRs (one wave per
  // SIMD); with 8-byte loads 234 VGPRs (two)
  constexpr int kV16 = 16 / sizeof(T);
  constexpr int kV8 = 8 / sizeof(T);
  constexpr int kScoreV4 = EKV_SCORE_G4_BYTES / sizeof(T);
  switch (s.G) {
    case 1: return launch_score_t<T, D, 1, kV16>(s, q, scale, kmin, kmax, mean, var, bt, lens, ub, ubg, gm, gv, K, refresh, hint, stream);
    case 2: return launch_score_t<T, D, 2, kV16>(s, q, scale, kmin, kmax, mean, var, bt, lens, ub, ubg, gm, gv, K, refresh, hint, stream);
    case 4:
      if (gm != nullptr)
        return launch_score_t<T, D, 4, kV8>(s, q, scale, kmin, kmax, mean, var, bt, lens, ub, ubg, gm, gv, K, refresh, hint, stream);
      return launch_score_t<T, D, 4, kScoreV4>(s, q, scale, kmin, kmax, mean, var, bt, lens, ub, ubg, gm, gv, K, refresh, hint, stream);
    case 8: return launch_score_t<T, D, 8, kV8>(s, q, scale, kmin, kmax, mean, var, bt, lens, ub, ubg, gm, gv, K, refresh, hint, stream);
  }
  return hipErrorInvalidValue;
}

template <typename T, int D, int G, int kVec>
hipError_t launch_score_select_t(const Shape& s, const float* q, float scale, const void* K,
                                 void* kmin, void* kmax, const int32_t* bt, const int32_t* lens,
                                 int refresh, float* ub, float* ubg, int top_k, int32_t* sel,
                                 int32_t* n_sel, int* counters, hipStream_t stream) {
  constexpr int kLpr = D / kVec;
  constexpr int kPagesPerStep = (kWave / kLpr) * kScoreWaves;
  const int per_iter = kPagesPerStep * ScoreGeo<D, G, kVec, false>::kU;
  const long long pairs = (long long)s.B * s.Hkv;
  const int ppb = slice_pages(s, per_iter);
  const long long nblocks = (long long)((s.maxP + ppb - 1) / ppb) * pairs;
  if (nblocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)nblocks);
  const int npairs = (int)pairs;
  if (s.maxP <= kStepTopkKeys)
    hipLaunchKernelGGL((score_select_kernel<T, D, G, kVec, true>), grid, dim3(kScoreBlock), 0,
                       stream, q, scale, (const T*)K, (T*)kmin, (T*)kmax, bt, lens, refresh, s.Hkv,
                       s.P, s.maxP, ppb, npairs, ub, ubg, top_k, sel, n_sel, counters);
  else
    hipLaunchKernelGGL((score_select_kernel<T, D, G, kVec, false>), grid, dim3(kScoreBlock), 0,
                       stream, q, scale, (const T*)K, (T*)kmin, (T*)kmax, bt, lens, refresh, s.Hkv,
                       s.P, s.maxP, ppb, npairs, ub, ubg, top_k, sel, n_sel, counters);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_score_select_d(const Shape& s, const float* q, float scale, const void* K,
                                 void* kmin, void* kmax, const int32_t* bt, const int32_t* lens,
                                 int refresh, float* ub, float* ubg, int top_k, int32_t* sel,
                                 int32_t* n_sel, int* counters, hipStream_t stream) {
  constexpr int kV16 = 16 / sizeof(T);
  constexpr int kV8 = 8 / sizeof(T);
  switch (s.G) {
    case 1: return launch_score_select_t<T, D, 1, kV16>(s, q, scale, K, kmin, kmax, bt, lens, refresh, ub, ubg, top_k, sel, n_sel, counters, stream);
    case 2: return launch_score_select_t<T, D, 2, kV16>(s, q, scale, K, kmin, kmax, bt, lens, refresh, ub, ubg, top_k, sel, n_sel, counters, stream);
    case 4: return launch_score_select_t<T, D, 4, kV16>(s, q, scale, K, kmin, kmax, bt, lens, refresh, ub, ubg, top_k, sel, n_sel, counters, stream);
    case 8: return launch_score_select_t<T, D, 8, kV8>(s, q, scale, K, kmin, kmax, bt, lens, refresh, ub, ubg, top_k, sel, n_sel, counters, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_score(const Shape& s, const float* q, float scale, const void* kmin,
                        const void* kmax, const void* mean, const void* var,
                        const int32_t* bt, const int32_t* lens, float* ub, float* ubg,
                        double* gm, double* gv, hipStream_t stream) {
  if (s.bf16) {
    if (s.D == 128) return launch_score_d<bf16_t, 128>(s, q, scale, kmin, kmax, mean, var, bt, lens, ub, ubg, gm, gv, nullptr, 0, nullptr, stream);
    return launch_score_d<bf16_t, 64>(s, q, scale, kmin, kmax, mean, var, bt, lens, ub, ubg, gm, gv, nullptr, 0, nullptr, stream);
  }
  if (s.D == 128) return launch_score_d<float, 128>(s, q, scale, kmin, kmax, mean, var, bt, lens, ub, ubg, gm, gv, nullptr, 0, nullptr, stream);
  return launch_score_d<float, 64>(s, q, scale, kmin, kmax, mean, var, bt, lens, ub, ubg, gm, gv, nullptr, 0, nullptr, stream);
}

ScoreSlices score_box_slices(const Shape& s) {
  // the geometry launch_score_t uses for the box-only kernel
  const int eb = s.bf16 ? 2 : 4;
  const int kv = (s.G == 8 ? 8 : (s.G == 4 ? EKV_SCORE_G4_BYTES : 16)) / eb;
  const int lpr = s.D / kv;
  const int per_step = (kWave / lpr) * kScoreWaves;
  const int kinds_lanes = lpr < 16 ? lpr : 16;
  int ku = kinds_lanes / s.G;
  ku = ku < 1 ? 1 : (ku > kScoreMaxU ? kScoreMaxU : ku);
  ScoreSlices r;
  r.pages = slice_pages(s, per_step * ku);
  r.count = (s.maxP + r.pages - 1) / r.pages;
  return r;
}

hipError_t launch_score_box(const Shape& s, const float* q, float scale, const void* K,
                            void* kmin, void* kmax, const int32_t* bt, const int32_t* lens,
                            int refresh, float* ub, float* ubg, int4* hint, hipStream_t stream) {
  if (s.bf16) {
    if (s.D == 128) return launch_score_d<bf16_t, 128>(s, q, scale, kmin, kmax, nullptr, nullptr, bt, lens, ub, ubg, nullptr, nullptr, K, refresh, hint, stream);
    return launch_score_d<bf16_t, 64>(s, q, scale, kmin, kmax, nullptr, nullptr, bt, lens, ub, ubg, nullptr, nullptr, K, refresh, hint, stream);
  }
  if (s.D == 128) return launch_score_d<float, 128>(s, q, scale, kmin, kmax, nullptr, nullptr, bt, lens, ub, ubg, nullptr, nullptr, K, refresh, hint, stream);
  return launch_score_d<float, 64>(s, q, scale, kmin, kmax, nullptr, nullptr, bt, lens, ub, ubg, nullptr, nullptr, K, refresh, hint, stream);
}

hipError_t launch_score_select(const Shape& s, const float* q, float scale, const void* K,
                               void* kmin, void* kmax, const int32_t* bt, const int32_t* lens,
                               int refresh, float* ub, float* ubg, int top_k, int32_t* sel,
                               int32_t* n_sel, int* counters, hipStream_t stream) {
  if (s.bf16) {
    if (s.D == 128) return launch_score_select_d<bf16_t, 128>(s, q, scale, K, kmin, kmax, bt, lens, refresh, ub, ubg, top_k, sel, n_sel, counters, stream);
    return launch_score_select_d<bf16_t, 64>(s, q, scale, K, kmin, kmax, bt, lens, refresh, ub, ubg, top_k, sel, n_sel, counters, stream);
  }
  if (s.D == 128) return launch_score_select_d<float, 128>(s, q, scale, K, kmin, kmax, bt, lens, refresh, ub, ubg, top_k, sel, n_sel, counters, stream);
  return launch_score_select_d<float, 64>(s, q, scale, K, kmin, kmax, bt, lens, refresh, ub, ubg, top_k, sel, n_sel, counters, stream);
}

}  // namespace ekv
