// Top-k selection fused into the sparse alpha-entmax decode (EntmaxKV summary
// page: §2.B(1) keep the k pages with the largest bounds; §2.C load only the
// selected pages' keys and values; §3 only the support decides the output).
//
// One launch does what ekv_select_pages(TOPK) and the first stage of
// ekv_entmax_decode do, without a round trip through a selection list in
// memory and without a serial per-pair tail.  Per (row, KV head) pair it
// holds a few key items, each owning a run of consecutive splits (the launch
// aims at about 256 key items, one per compute unit), and one selection item
// that writes the top-k list out as sel / n_sel.
//
// With the scorer's hints (the step's path) a key item reads the pair's group
// bounds U and takes each query head's best page over the row as its probe;
// the probe counts if the page is selected, i.e. fewer than k pages rank
// ahead of it (a count, no selection needed), and then zlb, the largest z of
// its tokens, bounds that head's z_max from below.  A page is read only if U
// clears some head's zlb - 1 (tau >= z_max - 1; U >= every head's bound).
// That test is monotone in U, so when at most k pages clear it they are all
// selected and the top-k itself is skipped; otherwise every key item runs it
// (range-adaptive radix select on keys in registers).  Without hints the key
// item runs the top-k first and probes each head's best selected page.  The
// pages to read are shared out over the pair's key items in ascending order
// (every item computes the same list); each item scores its pages for the G
// heads from one read (matrix cores for bf16), in chunks of one split's token
// slots, and writes each chunk's candidates z > chunk_max - 1 as one split.
//
// The tau / PV stage then runs as in ekv_entmax_decode.  Because the final
// candidate set of a head is {z > z_max - 1} over the tokens read, in
// ascending slot order, results are bit-identical to ekv_select_pages followed
// by the pruned ekv_entmax_decode.
#include "decode_dev.h"
#include "kernels.h"

namespace ekv {
namespace {

constexpr int kSelCap = 1024;                 // selected pages per pair held in LDS
constexpr int kSelPer = kSelCap / kBlock;     // of them per thread
constexpr int kProbeBatch = 4;                // probe key rows per thread in flight
#ifndef EKV_STEP_ITEMS
#define EKV_STEP_ITEMS 256
#endif
constexpr long long kStepItems = EKV_STEP_ITEMS;  // workgroups to aim for per launch
#ifndef EKV_STEP_MAX_SPI
#define EKV_STEP_MAX_SPI 1024
#endif
#ifndef EKV_TOPK_FAST
#define EKV_TOPK_FAST 1
#endif

template <typename T>
struct SelQkArgs {
  const float* q;
  float zscale;     // (alpha - 1) * scale
  float a1;         // alpha - 1
  const T* K;
  const int32_t* bt;
  const int32_t* lens;
  const float* ub;   // [pairs][maxP][G] per-head page bounds, or NULL (no pruning)
  const float* ubg;  // [pairs][maxP] group bounds
  int32_t* sel;      // [pairs][maxP] written by split 0
  int32_t* n_sel;    // [pairs] written by split 0
  int top_k, Hkv, P, log2P, maxP, splits, npairs;
  int spi;           // splits per key item
  int nit;           // key items per pair; item nit of a pair writes sel / n_sel
  float2* cand;
  int* cnt;
  float* smax;
  // the scorer's best page per (pair, page slice, head), or NULL:
  // {bound bits, page, physical page, 0} [pairs][nslices][G], slices of
  // slice_pages pages
  const int4* hint;
  int slice_pages, nslices;
};

template <typename T, int D, int G, int kStage = 1>
struct SelQkLds {
  union {
    TopkRegLds tk;
    QkLds<T, D, G> qk;
    uint4 stage[kStage];  // coalesced first-round loads on their way to the owning threads
  } u;
  int s_sel[kSelCap];    // selected pages, ascending
  int s_phys[kSelCap];   // their physical pages
  int s_surv[kSelCap];   // pages read (indices into s_sel), ascending
  unsigned char s_flag[kSelCap];
  float rowz[G * kMaxPageSize];
  float s_best[kBlock / kWave][G];
  int s_bestj[kBlock / kWave][G];   // the page
  int s_bestph[kBlock / kWave][G];  // its physical page
  float zlb[G];
  int probe_phys[G];
  int probe_nv[G];
  int probe_page[G];
  int probe_sel[G];
  uint32_t probe_key[G];
  int rank_part[kBlock / kWave][G];
  int sh4[4];
  int s_m;
  float qraw[G * D];  // the group's queries (the probe of the hinted kernel)
};

// The keys of an item's share of the m pages to read (ascending), then its
// candidates: the item holds splits [s0, s1) of the pair's nsplit, and split
// s owns pages [s * m / nsplit, (s + 1) * m / nsplit) of the list, at most
// kR / P of them since m <= nsplit * kR / P; the union of the item's shares
// is scored in chunks of kR token slots, chunk c written out as split s0 + c,
// and the splits left over as empty (no candidate, maximum -inf).  Every head
// then sees its candidates z > split_max - 1 over all the pages read, in
// ascending slot order, whatever the item boundaries.  page_at(i) gives
// {physical page, page} of list entry i.
template <typename T, int D, int G, bool kMfma, typename PageAt>
__device__ __forceinline__ void read_share(const SelQkArgs<T>& a, QkLds<T, D, G>& qk,
                                           const float* qg,
                                           const float (&qv)[kMfma ? (G * D + kBlock - 1) / kBlock : 1],
                                           int g, int L, size_t bh0, int s0, int s1, int nsplit,
                                           int m, PageAt page_at) {
  constexpr int kR = Geo<T, D>::kR;
  const int P = a.P, log2P = a.log2P;
  const int lo = (int)(((long long)s0 * m) / nsplit);
  const int hi = (int)(((long long)s1 * m) / nsplit);
  const int per = kR >> log2P;  // pages per chunk
  int s = s0;
  for (int base = lo; base < hi; base += per, ++s) {
    if (base > lo) __syncthreads();  // the previous chunk's emit has read the page map
    const int n_pg = min(per, hi - base);
    for (int i = threadIdx.x; i < n_pg; i += kBlock) {
      const int2 pp = page_at(base + i);
      qk.pg_phys[i] = pp.x;
      qk.pg_valid[i] = page_valid(L, pp.y, P);
    }
    // (qk_score_slots barriers before it reads the page map)
    qk_score_slots<T, D, G, kMfma>(qg, qv, a.zscale, a.K, a.Hkv, g, P, log2P, 0, n_pg << log2P,
                                   0, qk);
    qk_emit<T, D, G, false, kMfma>(qk, n_pg << log2P, 0, 0, P, log2P, a.cand, a.cnt, a.smax,
                                   bh0, a.splits, s);
  }
  for (; s < s1; ++s)
    qk_emit<T, D, G, false, kMfma>(qk, 0, 0, 0, P, log2P, a.cand, a.cnt, a.smax, bh0, a.splits,
                                   s);
}

// read_share for bf16 keys with the chunks software-pipelined: the K rows of
// chunk c + 1 are requested as soon as chunk c's scores are formed on the
// matrix cores (one chunk of registers), so an item that reads many chunks
// (pairs whose pages do not prune) has them in flight while chunk c's
// candidates are emitted.  Rows, chunks, scores and candidates are those of read_share
// (the page map is looked up in the caller's list instead of being staged),
// so the results are bit-identical.
template <typename T, int D, int G, typename PageAt>
__device__ __forceinline__ void read_share_mfma(const SelQkArgs<T>& a, QkLds<T, D, G>& qk,
                                                const float (&qv)[(G * D + kBlock - 1) / kBlock],
                                                int g, int L, size_t bh0, int s0, int s1,
                                                int nsplit, int m, PageAt page_at) {
  constexpr int kR = Geo<T, D>::kR;
  constexpr int kQPer = (G * D + kBlock - 1) / kBlock;
  constexpr int kKK = D / 32;                       // k steps of 32 dims
  constexpr int kBlocksA = G > 4 ? 2 : 1;
  constexpr int kGPW = kR / 16 / (kBlock / kWave);  // 16-token groups per wave
  const int P = a.P, log2P = a.log2P;
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int mrow = lane % 16;
  const int kq = lane / 16;
  const size_t tile_stride = (size_t)P * D;
  const int lo = (int)(((long long)s0 * m) / nsplit);
  const int hi = (int)(((long long)s1 * m) / nsplit);
  const int per = kR >> log2P;
  const int nch = (hi - lo + per - 1) / per;  // <= s1 - s0
  auto& zl = qk.zl;
  // q split into three bf16 parts once (as in qk_score_slots)
#pragma unroll
  for (int u = 0; u < kQPer; ++u) {
    const int idx = threadIdx.x + u * kBlock;
    if (idx >= G * D) break;
    const int h = idx / D, dd = idx % D;
    const float x = qv[u];
    const float q_hi = bf16_round(x);
    const float q_mid = bf16_round(x - q_hi);
    const float q_lo = bf16_round(x - q_hi - q_mid);
    qk.qparts[h][0][dd] = (uint16_t)(__float_as_uint(q_hi) >> 16);
    qk.qparts[h][1][dd] = (uint16_t)(__float_as_uint(q_mid) >> 16);
    qk.qparts[h][2][dd] = (uint16_t)(__float_as_uint(q_lo) >> 16);
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
      if (h < G && part < 3) w = *reinterpret_cast<const uint4*>(&qk.qparts[h][part][kk * 32 + kq * 8]);
      qa[ab][kk] = as_bf16x8(w);
    }
  }
  struct Chunk {
    uint4 kb[kGPW][kKK];
    bool valid[kGPW];
  };
  // the K rows of chunk c: row r of the chunk is token r & (P-1) of list
  // entry base + (r >> log2P).  Every lane issues all its loads: a row past
  // the chunk or past its page's valid tokens reads the chunk's first row
  // instead (in bounds, a cache hit) and is masked by `valid`, so the load
  // count is fixed and the next chunk's loads stay in flight while this one
  // is scored
  auto issue = [&](int c, Chunk& ch) {
    const int base = lo + c * per;
    const int n_pg = min(per, hi - base);
    const int r_end = n_pg << log2P;
    const T* safe = a.K + ((size_t)page_at(base).x * a.Hkv + g) * tile_stride + kq * 8;
#pragma unroll
    for (int u = 0; u < kGPW; ++u) {
      const int r = (wave * kGPW + u) * 16 + mrow;
      const int2 pp = page_at(base + min(r >> log2P, n_pg - 1));
      const int t = r & (P - 1);
      ch.valid[u] = r < r_end && t < page_valid(L, pp.y, P);
      const T* row = ch.valid[u] ? a.K + ((size_t)pp.x * a.Hkv + g) * tile_stride +
                                       (size_t)t * D + kq * 8
                                 : safe;
#pragma unroll
      for (int kk = 0; kk < kKK; ++kk) ch.kb[u][kk] = load16_stream(row + kk * 32);
    }
  };
  // scores of chunk c into zl
  auto score = [&](const Chunk& ch) {
#pragma unroll
    for (int u = 0; u < kGPW; ++u) {
      const int rl = (wave * kGPW + u) * 16 + mrow;
#pragma unroll
      for (int ab = 0; ab < kBlocksA; ++ab) {
        f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < kKK; ++kk)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ab][kk], as_bf16x8(ch.kb[u][kk]), acc,
                                                        0, 0, 0);
        const int h = ab * 4 + kq;
        if (h < G)
          zl[h][rl] = ch.valid[u] ? ((acc[0] + acc[1]) + acc[2]) * a.zscale
                                  : -__builtin_huge_valf();
      }
    }
  };
  // per head (one wave each) the chunk maximum and its candidates
  // z > max - 1, as split s0 + c
  auto emit = [&](int c) {
    const int base = lo + c * per;
    const int nrows = min(per, hi - base) << log2P;
    const int s = s0 + c;
    for (int h = wave; h < G; h += kBlock / kWave) {
      float mz = -__builtin_huge_valf();
      for (int r = lane; r < nrows; r += kWave) mz = fmaxf(mz, zl[h][r]);
      mz = wave_max_f32(mz);
      const double thr = (double)mz - 1.0;
      const size_t bh = bh0 + h;
      float2* out = a.cand + (bh * a.splits + s) * kR;
      int total = 0;
      for (int r0 = 0; r0 < nrows; r0 += kWave) {
        const int r = r0 + lane;
        const float z = r < nrows ? zl[h][r] : -__builtin_huge_valf();
        const bool flag = (double)z > thr;
        const uint64_t mask = __ballot(flag);
        const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (kWave - lane));
        if (flag) {
          const int ptok = page_at(base + (r >> log2P)).x * P + (r & (P - 1));
          out[total + __popcll(mask & lt)] = make_float2(z, __int_as_float(ptok));
        }
        total += __popcll(mask);
      }
      if (lane == 0) {
        a.cnt[bh * a.splits + s] = total;
        a.smax[bh * a.splits + s] = mz;
      }
    }
    __syncthreads();  // zl is rewritten by the next chunk
  };
  // the next chunk's rows are requested as soon as this chunk's scores are
  // formed (its registers are free again), and arrive during the emit
  Chunk ch;
  if (nch > 0) issue(0, ch);
  for (int c = 0; c < nch; ++c) {
    score(ch);
    if (c + 1 < nch) issue(c + 1, ch);
    __syncthreads();  // zl complete
    emit(c);
  }
  // the item's splits past its last chunk: empty
  for (int s = s0 + nch; s < s1; ++s)
    for (int h = wave; h < G; h += kBlock / kWave)
      if (lane == 0) {
        a.cnt[(bh0 + h) * a.splits + s] = 0;
        a.smax[(bh0 + h) * a.splits + s] = -__builtin_huge_valf();
      }
}

// The selection item of a pair (the last item index of the launch): the
// top-k pages of the row, ascending, into sel / n_sel (the key items do not
// need the list written out).
template <typename T, int kPer>
__device__ __forceinline__ void selection_item(const SelQkArgs<T>& a, int pair, TopkRegLds& tk) {
  const int b = pair / a.Hkv;
  const int np = (a.lens[b] + a.P - 1) >> a.log2P;
  const int k = min(a.top_k, np);
  int32_t* out = a.sel + (size_t)pair * a.maxP;
  if (threadIdx.x == 0) a.n_sel[pair] = k;
  if (k >= np) {
    for (int p = threadIdx.x; p < np; p += kBlock) out[p] = p;
    return;
  }
  topk_block_reg<kPer, false>(a.ubg + (size_t)pair * a.maxP, np, k, out, tk);
}

// One work item per workgroup: item = it * pairs + pair, item it of a pair
// holding its splits [it * spi, (it + 1) * spi) (item-major: with a multiple
// of 8 pairs, all items of a pair run on one XCD and share its L2 lines of
// the pair's bounds and probe rows).
template <typename T, int D, int G, int kPer>
__global__ __launch_bounds__(kBlock) void sel_qk_kernel(SelQkArgs<T> a) {
  using GE = Geo<T, D>;
  constexpr int kVec = GE::kVec, kLpr = GE::kLpr, kR = GE::kR;
  constexpr int kRowsPerPass = kBlock / kLpr;
  constexpr int kQPer = (G * D + kBlock - 1) / kBlock;
  constexpr bool kMfma = std::is_same<T, bf16_t>::value;
  __shared__ SelQkLds<T, D, G> sm;
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int pair = (int)(blockIdx.x % (unsigned)a.npairs);
  const int it = (int)(blockIdx.x / (unsigned)a.npairs);
  if (it == a.nit) {  // uniform: the pair's selection list
    selection_item<T, kPer>(a, pair, sm.u.tk);
    return;
  }
  const int b = pair / a.Hkv;
  const int g = pair % a.Hkv;
  const int Hq = a.Hkv * G;
  const int P = a.P, log2P = a.log2P, maxP = a.maxP;
  const size_t bh0 = (size_t)b * Hq + (size_t)g * G;
  const float* qg = a.q + bh0 * D;
  const bool prune = a.ub != nullptr;

  // ---- round trip 1: the row length, the pair's group bounds (kPer
  // consecutive pages per thread; entries past the row's pages are in bounds
  // and masked below) and the group's queries
  const int p0 = tid * kPer;
  const float* Ug = a.ubg + (size_t)pair * maxP;
  float uv[kPer];
  load_run<kPer>(Ug, p0, maxP, uv);
  float qv[kMfma ? kQPer : 1];
  if constexpr (kMfma) {
#pragma unroll
    for (int u = 0; u < kQPer; ++u) {
      const int idx = tid + u * kBlock;
      qv[u] = idx < G * D ? qg[idx] : 0.0f;
    }
  }
  const int L = a.lens[b];
  const int np = (L + P - 1) >> log2P;
  const int nsel = min(a.top_k, np);
  const int nsplit = ((nsel << log2P) + kR - 1) / kR;
  const int s0 = it * a.spi;
  const int s1 = min(s0 + a.spi, nsplit);
  if (s0 >= nsplit) return;  // uniform: nothing to read for this item

  // ---- top-k: the nsel largest U, lowest page on ties, placed ascending
  // (thread t's pages precede thread t+1's, so one block scan orders them)
  {
    const int nv = max(0, min(kPer, np - p0));
    uint32_t key[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) key[i] = order_key(uv[i]);
    TopkThr th{0u, 0, true};  // nsel >= np: every page
    if (nsel < np) th = topk_threshold<kPer>(key, nv, nsel, sm.u.tk);
    bool take[kPer], eq[kPer];
    int cg = 0, ce = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const bool v = i < nv;
      take[i] = v && (th.cut ? key[i] >= th.T : key[i] > th.T);
      eq[i] = v && !th.cut && key[i] == th.T;
      cg += take[i] ? 1 : 0;
      ce += eq[i] ? 1 : 0;
    }
    // counts below 2^16 each: one scan of both
    const int both = cg | (ce << 16);
    const int excl = block_incl_scan(both, sm.sh4) - both;
    int eq_seen = excl >> 16;
    int pos = (excl & 0xFFFF) + min(eq_seen, th.rem);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const bool tk = take[i] || (eq[i] && eq_seen < th.rem);
      eq_seen += eq[i] ? 1 : 0;
      if (tk) sm.s_sel[pos] = p0 + i;
      pos += tk ? 1 : 0;
    }
  }
  __syncthreads();

  // ---- the pages to read: all selected pages, or those that can hold a
  // support token of some head of the group
  int m = nsel;
  if (prune) {
    // round trip 2: the selected pages' bounds and physical pages (slots
    // tid + i * kBlock); per head the selected page with the largest bound,
    // lowest page on ties
    float ubs[kSelPer][G];
    float best[G];
    int bestp[G], bestph[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      best[h] = -__builtin_huge_valf();
      bestp[h] = 0x7fffffff;
      bestph[h] = 0;
    }
#pragma unroll
    for (int i = 0; i < kSelPer; ++i) {
      const int j = tid + i * kBlock;
#pragma unroll
      for (int h = 0; h < G; ++h) ubs[i][h] = -__builtin_huge_valf();
      if (j < nsel) {
        const int page = sm.s_sel[j];
        const float* up = a.ub + ((size_t)pair * maxP + page) * G;
        if constexpr (G % 4 == 0) {
#pragma unroll
          for (int h4 = 0; h4 < G; h4 += 4) {
            const float4 v = *reinterpret_cast<const float4*>(up + h4);
            ubs[i][h4] = v.x;
            ubs[i][h4 + 1] = v.y;
            ubs[i][h4 + 2] = v.z;
            ubs[i][h4 + 3] = v.w;
          }
        } else {
#pragma unroll
          for (int h = 0; h < G; ++h) ubs[i][h] = up[h];
        }
        const int phys = a.bt[(size_t)b * maxP + page];
        sm.s_phys[j] = phys;
#pragma unroll
        for (int h = 0; h < G; ++h)
          if (ubs[i][h] > best[h]) {  // slots ascending in i: ties keep the lower page
            best[h] = ubs[i][h];
            bestp[h] = page;
            bestph[h] = phys;
          }
      }
    }
    // per wave: the largest bound (DPP), then the lowest page among the lanes
    // that hold it (DPP), then that lane's physical page (readlane)
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float wb = wave_max_f32(best[h]);
      const uint32_t wp = wave_min_u32(best[h] == wb ? (uint32_t)bestp[h] : 0xFFFFFFFFu);
      const uint64_t at = __ballot(best[h] == wb && (uint32_t)bestp[h] == wp);
      const int src = at ? __ffsll((long long)at) - 1 : 0;
      const int wph = __builtin_amdgcn_readlane(bestph[h], src);
      if (lane == 0) {
        sm.s_best[wave][h] = wb;
        sm.s_bestj[wave][h] = (int)wp;
        sm.s_bestph[wave][h] = wph;
      }
    }
    __syncthreads();
    if (tid < G) {
      const int h = tid;
      float bv = sm.s_best[0][h];
      int bp = sm.s_bestj[0][h], bph = sm.s_bestph[0][h];
#pragma unroll
      for (int w = 1; w < kBlock / kWave; ++w)
        if (sm.s_best[w][h] > bv || (sm.s_best[w][h] == bv && sm.s_bestj[w][h] < bp)) {
          bv = sm.s_best[w][h];
          bp = sm.s_bestj[w][h];
          bph = sm.s_bestph[w][h];
        }
      // bounds are finite unless the inputs are not: fall back to the first
      // selected page
      if (bp < 0 || bp >= np) {
        bp = sm.s_sel[0];
        bph = sm.s_phys[0];
      }
      sm.probe_phys[h] = bph;
      sm.probe_nv[h] = page_valid(L, bp, P);
    }
    __syncthreads();

    // round trip 3: the probe rows; zlb[h] = the largest fp32 z of head h's
    // best page's valid tokens (kLpr lanes per key row)
    {
      const int c = tid % kLpr;
      const int rg = tid / kLpr;
      const int nrows = G * P;
      for (int r0 = 0; r0 < nrows; r0 += kRowsPerPass * kProbeBatch) {
        uint4 w[kProbeBatch];
        float qx[kProbeBatch][kVec];
        bool ok[kProbeBatch];
#pragma unroll
        for (int u = 0; u < kProbeBatch; ++u) {
          const int r = r0 + rg + u * kRowsPerPass;
          const int h = r >> log2P;
          const int t = r & (P - 1);
          ok[u] = r < nrows && t < sm.probe_nv[h < G ? h : 0];
          w[u] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
          for (int v = 0; v < kVec; ++v) qx[u][v] = 0.0f;
          if (ok[u]) {
            w[u] = load16_stream(a.K + ((size_t)sm.probe_phys[h] * a.Hkv + g) * (size_t)P * D +
                                 (size_t)t * D + c * kVec);
            const float4* qh = reinterpret_cast<const float4*>(qg + (size_t)h * D + c * kVec);
#pragma unroll
            for (int v4 = 0; v4 < kVec / 4; ++v4) {
              const float4 x = qh[v4];
              qx[u][4 * v4] = x.x;
              qx[u][4 * v4 + 1] = x.y;
              qx[u][4 * v4 + 2] = x.z;
              qx[u][4 * v4 + 3] = x.w;
            }
          }
        }
#pragma unroll
        for (int u = 0; u < kProbeBatch; ++u) {
          const int r = r0 + rg + u * kRowsPerPass;
          float x[kVec];
          Elem<T>::unpack(w[u], x);
          float acc = 0.0f;
#pragma unroll
          for (int v = 0; v < kVec; ++v) acc = fmaf(qx[u][v], x[v], acc);
          acc = group_sum_f32<kLpr>(acc);  // all lanes of a row group agree on ok[u]
          if (c == 0 && r < nrows) sm.rowz[r] = ok[u] ? acc * a.zscale : -__builtin_huge_valf();
        }
      }
    }
    __syncthreads();
    if (tid < G) {
      float zm = -__builtin_huge_valf();
      for (int t = 0; t < P; ++t) zm = fmaxf(zm, sm.rowz[tid * P + t]);
      sm.zlb[tid] = zm;
    }
    __syncthreads();
    float zl_h[G];
#pragma unroll
    for (int h = 0; h < G; ++h) zl_h[h] = sm.zlb[h];
    // keep flags of the strided slots through LDS, then contiguous chunks of
    // slots per thread, compacted by a block scan into the ascending list of
    // selected slots to read
#pragma unroll
    for (int i = 0; i < kSelPer; ++i) {
      const int j = tid + i * kBlock;
      bool nd = false;
#pragma unroll
      for (int h = 0; h < G; ++h) nd |= !page_below_support(a.a1 * ubs[i][h], zl_h[h]);
      if (j < nsel) sm.s_flag[j] = nd ? 1 : 0;
    }
    __syncthreads();
    int cntf = 0;
#pragma unroll
    for (int i = 0; i < kSelPer; ++i) {
      const int j = tid * kSelPer + i;
      cntf += (j < nsel && sm.s_flag[j]) ? 1 : 0;
    }
    const int incl = block_incl_scan(cntf, sm.sh4);
    int pos = incl - cntf;
#pragma unroll
    for (int i = 0; i < kSelPer; ++i) {
      const int j = tid * kSelPer + i;
      if (j < nsel && sm.s_flag[j]) sm.s_surv[pos++] = j;
    }
    if (tid == kBlock - 1) sm.s_m = incl;
    __syncthreads();
    m = sm.s_m;
  }

  // ---- this item's share of the pages to read (ascending)
  if (!prune) {  // uniform: the selected pages' physical pages into LDS too
    for (int j = tid; j < nsel; j += kBlock) sm.s_phys[j] = a.bt[(size_t)b * maxP + sm.s_sel[j]];
    __syncthreads();
  }
  // (LDS only, so no key load waits behind a block-table load)
  auto page_at = [&](int idx) {
    const int j = prune ? sm.s_surv[idx] : idx;
    return make_int2(sm.s_phys[j], sm.s_sel[j]);
  };
  if constexpr (kMfma)
    read_share_mfma<T, D, G>(a, sm.u.qk, qv, g, L, bh0, s0, s1, nsplit, m, page_at);
  else
    read_share<T, D, G, kMfma>(a, sm.u.qk, qg, qv, g, L, bh0, s0, s1, nsplit, m, page_at);
}

// The same key item with the scorer's hints (the step's path): each head's
// probe page is the best page of its whole row (the best of the slice bests,
// lowest page on ties), known after the first round trip, so the probe rows
// are requested right away.  The probe counts only if that page is selected
// (fewer than nsel pages rank ahead of it; else the head has no bound and
// nothing is skipped), and the pages left to read are those whose group
// bound U clears some head's zlb - 1: U >= every head's bound, so this skips
// a subset of what the per-head test would and every skipped page is still
// below every head's support.  The top-k runs only when more than nsel pages
// clear.  The probe rows of a group must fit one batch
// (G * P <= kProbeBatch * kBlock / kLpr).
template <typename T, int D, int G, int kPer>
__global__ __launch_bounds__(kBlock) void sel_qk_hint_kernel(SelQkArgs<T> a) {
  using GE = Geo<T, D>;
  constexpr int kVec = GE::kVec, kLpr = GE::kLpr, kR = GE::kR;
  constexpr int kRowsPerPass = kBlock / kLpr;
  constexpr int kQPer = (G * D + kBlock - 1) / kBlock;
  constexpr bool kMfma = std::is_same<T, bf16_t>::value;
  constexpr int kHintPer = 4;  // hint entries per lane of wave 0 (<= 256 in all)
  __shared__ SelQkLds<T, D, G, kPer * kBlock / 4 * 9 / 8 + 1> sm;
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int pair = (int)(blockIdx.x % (unsigned)a.npairs);
  const int it = (int)(blockIdx.x / (unsigned)a.npairs);
  if (it == a.nit) {  // uniform: the pair's selection list
    selection_item<T, kPer>(a, pair, sm.u.tk);
    return;
  }
  const int b = pair / a.Hkv;
  const int g = pair % a.Hkv;
  const int Hq = a.Hkv * G;
  const int P = a.P, log2P = a.log2P, maxP = a.maxP;
  const size_t bh0 = (size_t)b * Hq + (size_t)g * G;
  const float* qg = a.q + bh0 * D;

  // ---- round trip 1: group bounds and block-table entries of this thread's
  // kPer pages, the group's queries, the slice hints (wave 0), the row length
  const int p0 = tid * kPer;
  const float* Ug = a.ubg + (size_t)pair * maxP;
  const int32_t* btrow = a.bt + (size_t)b * maxP;
  float uv[kPer];
  int btr[kPer];
  // Thread t owns pages p0 .. p0 + kPer (the ordered compaction below needs
  // each thread's pages consecutive).  When the rows are 16-byte aligned they
  // are read coalesced instead (lane l of a wave takes 16-byte chunk l of a
  // 1 KiB span: 8 cache lines per load instead of 64) and handed to the
  // owning threads through LDS after this round trip.
  constexpr int kC = kPer / 4;  // 16-byte chunks per thread
  // (at 8 pages per thread the four extra barriers cost more than the loads
  // save: gqa decode 19.0 -> 19.9 us; at 32, 25.2 -> 23.7 us on one 131072-token row)
  const bool coal = kPer >= 16 && (maxP & 3) == 0 && ((uintptr_t)Ug & 15) == 0 &&
                    ((uintptr_t)btrow & 15) == 0;
  uint4 cu[kC], cb[kC];
  if (coal) {
#pragma unroll
    for (int j = 0; j < kC; ++j) {
      const int c = tid + j * kBlock;
      cu[j] = make_uint4(0u, 0u, 0u, 0u);
      cb[j] = make_uint4(0u, 0u, 0u, 0u);
      if (4 * c < maxP) {  // maxP % 4 == 0: the whole chunk is in the row
        cu[j] = *reinterpret_cast<const uint4*>(Ug + 4 * c);
        cb[j] = *reinterpret_cast<const uint4*>(btrow + 4 * c);
      }
    }
  } else {
    load_run<kPer>(Ug, p0, maxP, uv);
    load_run<kPer>(btrow, p0, maxP, btr);
  }
  float qv[kQPer];
#pragma unroll
  for (int u = 0; u < kQPer; ++u) {
    const int idx = tid + u * kBlock;
    qv[u] = idx < G * D ? qg[idx] : 0.0f;
  }
  int4 hv[kHintPer];
  const int nhint = a.nslices * G;
#pragma unroll
  for (int u = 0; u < kHintPer; ++u) {
    const int e = lane + u * kWave;
    hv[u] = make_int4(0, -1, 0, 0);
    if (wave == 0 && e < nhint) hv[u] = a.hint[(size_t)pair * nhint + e];
  }
  const int L = a.lens[b];
  const int np = (L + P - 1) >> log2P;
  const int nsel = min(a.top_k, np);
  const int nsplit = ((nsel << log2P) + kR - 1) / kR;
  const int s0 = it * a.spi;
  const int s1 = min(s0 + a.spi, nsplit);
  if (s0 >= nsplit) return;  // uniform: nothing to read for this item
#pragma unroll
  for (int u = 0; u < kQPer; ++u) {
    const int idx = tid + u * kBlock;
    if (idx < G * D) sm.qraw[idx] = qv[u];
  }
  // each head's best page over the row's slices (lane l follows head l % G)
  if (wave == 0) {
    const int nsl = (np + a.slice_pages - 1) / a.slice_pages;
    float lb = -__builtin_huge_valf();
    int lp = 0x7fffffff;
#pragma unroll
    for (int u = 0; u < kHintPer; ++u) {
      const int e = lane + u * kWave;
      const float hu = __int_as_float(hv[u].x);
      const int hp = hv[u].y;
      // slices in order, each with its lowest page among equals: keep the first
      if (e < nsl * G && hp >= 0 && hp < np && hu > lb) {
        lb = hu;
        lp = hp;
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const bool mine = lane % G == h;
      const float wb = wave_max_f32(mine ? lb : -__builtin_huge_valf());
      const uint32_t wp = wave_min_u32(mine && lb == wb ? (uint32_t)lp : 0xFFFFFFFFu);
      if (lane == 0) {
        const bool ok = wp < (uint32_t)np;
        sm.probe_page[h] = ok ? (int)wp : -1;
        sm.probe_nv[h] = ok ? page_valid(L, (int)wp, P) : 0;
        sm.probe_sel[h] = 0;
      }
    }
  }
  lds_barrier();
  if (coal) {
    // chunk i sits at slot i + i / 8, so the owners' reads (kC consecutive
    // chunks per thread) spread over the banks
    uint4* st = sm.u.stage;
#pragma unroll
    for (int j = 0; j < kC; ++j) st[(tid + j * kBlock) * 9 / 8] = cu[j];
    lds_barrier();
#pragma unroll
    for (int j = 0; j < kC; ++j) {
      const uint4 w = st[(tid * kC + j) * 9 / 8];
      uv[4 * j] = __uint_as_float(w.x);
      uv[4 * j + 1] = __uint_as_float(w.y);
      uv[4 * j + 2] = __uint_as_float(w.z);
      uv[4 * j + 3] = __uint_as_float(w.w);
    }
    lds_barrier();
#pragma unroll
    for (int j = 0; j < kC; ++j) st[(tid + j * kBlock) * 9 / 8] = cb[j];
    lds_barrier();
#pragma unroll
    for (int j = 0; j < kC; ++j) {
      const uint4 w = st[(tid * kC + j) * 9 / 8];
      btr[4 * j] = (int)w.x;
      btr[4 * j + 1] = (int)w.y;
      btr[4 * j + 2] = (int)w.z;
      btr[4 * j + 3] = (int)w.w;
    }
    lds_barrier();  // the staging area is reused below
  }
  // the probe pages' physical pages and bounds from their owners' entries
  uint32_t key[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) key[i] = order_key(uv[i]);
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const int pg = sm.probe_page[h];
    if (pg >= p0 && pg < p0 + kPer) {
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        if (p0 + i == pg) {
          sm.probe_phys[h] = btr[i];
          sm.probe_key[h] = key[i];
        }
    }
  }
  lds_barrier();
  // ---- round trip 2, in flight during the selection: the probe rows
  const int c = tid % kLpr;
  const int rg = tid / kLpr;
  uint4 w[kProbeBatch];
  bool okr[kProbeBatch];
#pragma unroll
  for (int u = 0; u < kProbeBatch; ++u) {
    const int r = rg + u * kRowsPerPass;
    const int h = r >> log2P;
    const int t = r & (P - 1);
    okr[u] = r < G * P && t < sm.probe_nv[h < G ? h : 0];
    w[u] = make_uint4(0u, 0u, 0u, 0u);
    if (okr[u])
      w[u] = load16_stream(a.K + ((size_t)sm.probe_phys[h] * a.Hkv + g) * (size_t)P * D +
                           (size_t)t * D + c * kVec);
  }

  // ---- whether each head's probe page is selected: fewer than nsel pages
  // rank ahead of it (larger U, or equal U and a lower page).  The probe that
  // ranks last (smallest U, then highest page) is counted first: if it is
  // selected, so are the others, which is the usual case; otherwise each
  // head's probe is counted.
  const int nv = max(0, min(kPer, np - p0));
  {
    int wh = -1, wp = 0;
    uint32_t wk = 0u;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const int pg = sm.probe_page[h];
      const uint32_t pk = sm.probe_key[h];
      if (pg >= 0 && (wh < 0 || pk < wk || (pk == wk && pg > wp))) {
        wh = h;
        wk = pk;
        wp = pg;
      }
    }
    int c_ = 0;
    if (wh >= 0) {
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        c_ += (i < nv && (key[i] > wk || (key[i] == wk && p0 + i < wp))) ? 1 : 0;
    }
    c_ = wave_sum_i32(c_);
    if (lane == 0) sm.rank_part[wave][0] = c_;
    lds_barrier();
    int rw = 0;
#pragma unroll
    for (int w_ = 0; w_ < kBlock / kWave; ++w_) rw += sm.rank_part[w_][0];
    if (nsel >= np || rw < nsel) {  // uniform
      if (tid < G) sm.probe_sel[tid] = sm.probe_page[tid] >= 0;
    } else {
      int ahead[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const int pg = sm.probe_page[h];
        const uint32_t pk = sm.probe_key[h];
        int cc = 0;
#pragma unroll
        for (int i = 0; i < kPer; ++i)
          cc += (i < nv && (key[i] > pk || (key[i] == pk && p0 + i < pg))) ? 1 : 0;
        ahead[h] = wave_sum_i32(cc);
      }
      lds_barrier();  // every thread has read rank_part[.][0]
      if (lane == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) sm.rank_part[wave][h] = ahead[h];
      }
      lds_barrier();
      if (tid < G) {
        int r = 0;
#pragma unroll
        for (int w_ = 0; w_ < kBlock / kWave; ++w_) r += sm.rank_part[w_][tid];
        sm.probe_sel[tid] = sm.probe_page[tid] >= 0 && r < nsel;
      }
    }
  }
  // (the barrier below, after the probe rows are reduced, publishes probe_sel)

  // ---- zlb[h]: the largest fp32 z of the probe page's valid tokens (kLpr
  // lanes per key row), if that page is selected
#pragma unroll
  for (int u = 0; u < kProbeBatch; ++u) {
    const int r = rg + u * kRowsPerPass;
    const int h = r >> log2P;
    float x[kVec];
    Elem<T>::unpack(w[u], x);
    float acc = 0.0f;
    if (okr[u]) {
#pragma unroll
      for (int v = 0; v < kVec; ++v) acc = fmaf(sm.qraw[h * D + c * kVec + v], x[v], acc);
    }
    acc = group_sum_f32<kLpr>(acc);  // all lanes of a row group agree on okr[u]
    if (c == 0 && r < G * P) sm.rowz[r] = okr[u] ? acc * a.zscale : -__builtin_huge_valf();
  }
  lds_barrier();
  if (tid < G) {
    float zm = -__builtin_huge_valf();
    if (sm.probe_sel[tid])
      for (int t = 0; t < P; ++t) zm = fmaxf(zm, sm.rowz[tid * P + t]);
    sm.zlb[tid] = zm;
  }
  lds_barrier();
  float zl_h[G];
#pragma unroll
  for (int h = 0; h < G; ++h) zl_h[h] = sm.zlb[h];

  // ---- the pages to read, ascending: selected, and U clears some head's
  // zlb - 1 (with the rounding slacks of page_below_support).  The test is
  // monotone in U, so every page that ranks ahead of a clearing page clears
  // too: when at most nsel pages clear, all of them are selected and the
  // top-k itself is not needed; otherwise it decides.
  float bar = __builtin_huge_valf();
  bool bar_nan = false;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float bh = support_bar(zl_h[h]);
    bar_nan |= bh != bh;
    bar = fminf(bar, bh);
  }
  int cntf = 0;
  bool need[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    need[i] = i < nv && (bar_nan || !page_below_bar(a.a1 * uv[i], bar));
    cntf += need[i] ? 1 : 0;
  }
  int incl = block_incl_scan_lds(cntf, sm.sh4);
  if (tid == kBlock - 1) sm.s_m = incl;
  lds_barrier();
  if (sm.s_m > nsel) {  // uniform: the top-k decides which clearing pages are read
    TopkThr th = topk_threshold<kPer>(key, nv, nsel, sm.u.tk);
    bool eq[kPer], take[kPer];
    int cg = 0, ce = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const bool v = i < nv;
      take[i] = v && (th.cut ? key[i] >= th.T : key[i] > th.T);
      eq[i] = v && !th.cut && key[i] == th.T;
      cg += take[i] ? 1 : 0;
      ce += eq[i] ? 1 : 0;
    }
    const int both = cg | (ce << 16);
    int eq_seen = (block_incl_scan_lds(both, sm.sh4) - both) >> 16;
    cntf = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const bool tk = take[i] || (eq[i] && eq_seen < th.rem);
      eq_seen += eq[i] ? 1 : 0;
      need[i] = need[i] && tk;
      cntf += need[i] ? 1 : 0;
    }
    incl = block_incl_scan_lds(cntf, sm.sh4);
  }
  int pos = incl - cntf;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if (need[i]) {
      sm.s_surv[pos] = p0 + i;
      sm.s_phys[pos] = btr[i];
    }
    pos += need[i] ? 1 : 0;
  }
  if (tid == kBlock - 1) sm.s_m = incl;
  lds_barrier();
  const int m = sm.s_m;

  // ---- this item's share of them
  float qmv[kMfma ? kQPer : 1];
#pragma unroll
  for (int u = 0; u < (kMfma ? kQPer : 1); ++u) qmv[u] = qv[u < kQPer ? u : 0];
  auto page_at = [&](int idx) { return make_int2(sm.s_phys[idx], sm.s_surv[idx]); };
  if constexpr (kMfma)
    read_share_mfma<T, D, G>(a, sm.u.qk, qv, g, L, bh0, s0, s1, nsplit, m, page_at);
  else
    read_share<T, D, G, kMfma>(a, sm.u.qk, qg, qmv, g, L, bh0, s0, s1, nsplit, m, page_at);
}

template <typename T, int D>
__global__ __launch_bounds__(kBlock) void tau_pv_step_kernel(TauArgs<T> a) {
  __shared__ TauLds<T, D> sm;
  tau_head<T, D>(a, blockIdx.x, sm);
}

// Whether the hinted kernel takes this shape: at most 4 hints per lane of one
// wave, and the probe rows of a group in one batch.
template <typename T, int D, int G>
bool hint_fits(const Shape& s, const TopkHint& h) {
  constexpr int kLpr = Geo<T, D>::kLpr;
  return h.hint != nullptr && h.nslices * G <= 4 * kWave &&
         G * s.P <= kProbeBatch * (kBlock / kLpr);
}

template <typename T, int D, int G, int kPer>
hipError_t launch_t(const Shape& s, const DecodePlan& pl, const float* q, float zscale, float a1,
                    const void* K, const int32_t* bt, const int32_t* lens, int top_k,
                    const float* ub, const float* ubg, int32_t* sel, int32_t* n_sel,
                    float2* cand, int* cnt, float* smax, const TopkHint& hint,
                    hipStream_t stream) {
  const long long npairs = (long long)s.B * s.Hkv;
  // items per pair: enough for about kStepItems workgroups in all (every item
  // repeats the pair's selection, so no more than that), each holding spi
  // consecutive splits
  long long nit = (kStepItems + npairs - 1) / npairs;
  // without hints every item runs the pair's top-k and probe before its keys;
  // a pair with many splits still gets two items, so two runs of key chunks
  // are in flight per pair (64/8 heads, batch 32, context 131072, page 32:
  // 349 -> 326 us; the hinted kernel measured slower with more items on every
  // workload)
  const bool hinted = ub != nullptr && hint_fits<T, D, G>(s, hint);
  if (!hinted && nit < 2 && pl.splits >= 32) nit = 2;
  nit = nit < 1 ? 1 : (nit > pl.splits ? pl.splits : nit);
  int spi = (int)((pl.splits + nit - 1) / nit);
  spi = spi > EKV_STEP_MAX_SPI ? EKV_STEP_MAX_SPI : spi;
  nit = (pl.splits + spi - 1) / spi;
  // key items, then one selection item per pair
  const long long items = npairs * (nit + 1);
  if (items > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const SelQkArgs<T> a{q,      zscale,    a1,          (const T*)K, bt,      lens,
                       ub,     ubg,       sel,         n_sel,       top_k,   s.Hkv,
                       s.P,    s.log2P,   s.maxP,      pl.splits,   (int)npairs, spi,
                       (int)nit, cand,    cnt,         smax,        hint.hint,
                       hint.slice_pages, hint.nslices};
  if (hinted)
    hipLaunchKernelGGL((sel_qk_hint_kernel<T, D, G, kPer>), dim3((unsigned)items), dim3(kBlock),
                       0, stream, a);
  else
    hipLaunchKernelGGL((sel_qk_kernel<T, D, G, kPer>), dim3((unsigned)items), dim3(kBlock), 0,
                       stream, a);
  return hipGetLastError();
}

template <typename T, int D, int G>
hipError_t launch_g(const Shape& s, const DecodePlan& pl, const float* q, float zscale, float a1,
                    const void* K, const int32_t* bt, const int32_t* lens, int top_k,
                    const float* ub, const float* ubg, int32_t* sel, int32_t* n_sel,
                    float2* cand, int* cnt, float* smax, const TopkHint& hint,
                    hipStream_t stream) {
  if (s.maxP <= kBlock * 8)
    return launch_t<T, D, G, 8>(s, pl, q, zscale, a1, K, bt, lens, top_k, ub, ubg, sel, n_sel, cand, cnt, smax, hint, stream);
  if (s.maxP <= kBlock * 16)
    return launch_t<T, D, G, 16>(s, pl, q, zscale, a1, K, bt, lens, top_k, ub, ubg, sel, n_sel, cand, cnt, smax, hint, stream);
  return launch_t<T, D, G, 32>(s, pl, q, zscale, a1, K, bt, lens, top_k, ub, ubg, sel, n_sel, cand, cnt, smax, hint, stream);
}

template <typename T, int D>
hipError_t launch_d(const Shape& s, const DecodePlan& pl, const float* q, float scale,
                    float alpha, const void* K, const void* V, const int32_t* bt,
                    const int32_t* lens, int top_k, const float* ub, const float* ubg,
                    int32_t* sel, int32_t* n_sel, float* out, float* tau_out, int32_t* n_support,
                    void* ws, const TopkHint& hint, hipStream_t stream) {
  float2* cand = (float2*)((char*)ws + pl.cand_off);
  int* cnt = (int*)((char*)ws + pl.cnt_off);
  float* smax = (float*)((char*)ws + pl.smax_off);
  const double a1 = (double)alpha - 1.0;
  const float zscale = (float)(a1 * (double)scale);
  hipError_t e = hipErrorInvalidValue;
  switch (s.G) {
    case 1: e = launch_g<T, D, 1>(s, pl, q, zscale, (float)a1, K, bt, lens, top_k, ub, ubg, sel, n_sel, cand, cnt, smax, hint, stream); break;
    case 2: e = launch_g<T, D, 2>(s, pl, q, zscale, (float)a1, K, bt, lens, top_k, ub, ubg, sel, n_sel, cand, cnt, smax, hint, stream); break;
    case 4: e = launch_g<T, D, 4>(s, pl, q, zscale, (float)a1, K, bt, lens, top_k, ub, ubg, sel, n_sel, cand, cnt, smax, hint, stream); break;
    case 8: e = launch_g<T, D, 8>(s, pl, q, zscale, (float)a1, K, bt, lens, top_k, ub, ubg, sel, n_sel, cand, cnt, smax, hint, stream); break;
  }
  if (e != hipSuccess) return e;
  const double gamma = 1.0 / a1;
  const double gr = rint(gamma);
  const int gamma_int = (gr >= 1.0 && gr <= 64.0 && fabs(gamma - gr) <= 1e-12 * gr) ? (int)gr : 0;
  const TauArgs<T> ta{cand,   cnt,  smax,  pl.splits, (const T*)V, lens,    n_sel,
                      true,   pl.max_sel, s.Hq, s.Hkv, s.P,       s.log2P, (double)alpha,
                      gamma_int ? gr : gamma, gamma_int, out, tau_out, n_support};
  hipLaunchKernelGGL((tau_pv_step_kernel<T, D>), dim3(s.B * s.Hq), dim3(kBlock), 0, stream, ta);
  return hipGetLastError();
}

}  // namespace

bool topk_decode_fast(const Shape& s, int max_sel) {
  return EKV_TOPK_FAST && max_sel <= kSelCap && s.maxP <= kBlock * 32 &&
         decode_shape_supported(s, max_sel);
}

hipError_t launch_topk_decode(const Shape& s, const DecodePlan& plan, const float* q, float scale,
                              float alpha, const void* K, const void* V, const int32_t* bt,
                              const int32_t* lens, int top_k, const float* ub, const float* ubg,
                              int32_t* sel, int32_t* n_sel, float* out, float* tau_out,
                              int32_t* n_support, void* ws, const TopkHint& hint,
                              hipStream_t stream) {
  if (s.bf16) {
    if (s.D == 128)
      return launch_d<bf16_t, 128>(s, plan, q, scale, alpha, K, V, bt, lens, top_k, ub, ubg, sel, n_sel, out, tau_out, n_support, ws, hint, stream);
    return launch_d<bf16_t, 64>(s, plan, q, scale, alpha, K, V, bt, lens, top_k, ub, ubg, sel, n_sel, out, tau_out, n_support, ws, hint, stream);
  }
  if (s.D == 128)
    return launch_d<float, 128>(s, plan, q, scale, alpha, K, V, bt, lens, top_k, ub, ubg, sel, n_sel, out, tau_out, n_support, ws, hint, stream);
  return launch_d<float, 64>(s, plan, q, scale, alpha, K, V, bt, lens, top_k, ub, ubg, sel, n_sel, out, tau_out, n_support, ws, hint, stream);
}

}  // namespace ekv
