// Host-side launchers of the gfx950 kernels (internal; the public surface is
// include/entmaxkv.h).  Every launcher assumes its arguments were validated by
// the C ABI layer and only enqueues work on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "entmaxkv.h"

namespace ekv {

constexpr int kMaxPageSize = 64;  // largest supported tokens per page

struct Shape {
  int B, Hq, Hkv, G, D, P, log2P, maxP, Np;
  bool bf16;   // K, V, kmin, kmax in bf16 (else fp32)
  bool mom16;  // page mean/var in bf16 (else fp32)
};

// Decode-time append of the token at position lens[b] - 1 of every row: K/V
// rows written, the page's box updated (and its moments rebuilt when mean/var
// are given).
hipError_t launch_append(const Shape& s, const void* k_new, const void* v_new,
                         const int32_t* bt, const int32_t* lens, void* K, void* V, void* kmin,
                         void* kmax, void* mean, void* var, hipStream_t stream);

// Counts of invalid row lengths and block-table entries into bad[0], bad[1].
hipError_t launch_validate(const Shape& s, const int32_t* bt, const int32_t* lens, int32_t* bad,
                           hipStream_t stream);

hipError_t launch_build_meta(const Shape& s, const void* K, const int32_t* bt,
                             const int32_t* lens, const int32_t* first_page, int span,
                             void* kmin, void* kmax, void* mean, void* var,
                             hipStream_t stream);

hipError_t launch_score(const Shape& s, const float* q, float scale, const void* kmin,
                        const void* kmax, const void* mean, const void* var,
                        const int32_t* bt, const int32_t* lens, float* ub, float* ubg,
                        double* gm, double* gv, hipStream_t stream);

// Fused: last-page metadata refresh (optional) + scores + top-k by the last
// workgroup of each (row, KV head); `counters` [B*Hkv] start at zero and are
// left at zero.
hipError_t launch_score_select(const Shape& s, const float* q, float scale, const void* K,
                               void* kmin, void* kmax, const int32_t* bt, const int32_t* lens,
                               int refresh, float* ub, float* ubg, int top_k, int32_t* sel,
                               int32_t* n_sel, int* counters, hipStream_t stream);

// Box-bound scores only (top-k policy metadata), with an optional rebuild of
// each row's last page's box first (refresh).  hint (or NULL): per (pair,
// page slice, head) the slice's best page, {bound bits, page, physical page,
// 0} as int4 [pairs][score_box_slices(s).count][G].
struct ScoreSlices {
  int pages;  // pages per slice (one workgroup each)
  int count;  // slices per pair at max_pages_per_seq
};
ScoreSlices score_box_slices(const Shape& s);
hipError_t launch_score_box(const Shape& s, const float* q, float scale, const void* K,
                            void* kmin, void* kmax, const int32_t* bt, const int32_t* lens,
                            int refresh, float* ub, float* ubg, int4* hint, hipStream_t stream);

hipError_t launch_topk(const Shape& s, const int32_t* lens, int top_k, const float* ubg,
                       int32_t* sel, int32_t* n_sel, hipStream_t stream);

// e_n = E[max of n iid N(0,1)] as tabulated for the expected-maximum policy
// (NaN outside 1 <= n <= kMaxPageSize).
double expected_max_std_normal(int n);

// Gaussian-aware selection; `rule` 0 compares the box bound ub, 1 the
// expected maximum m + e_n sqrt(v) of the page's scores, 2 the page's
// expected entmax mass (against delta).  gamma = 1 / (alpha - 1) >= 1 (an
// integer one exactly when the caller rounded it).
hipError_t launch_gauss(const Shape& s, const int32_t* lens, float alpha, double gamma,
                        float delta, int rule, const float* ub, const float* ubg,
                        const double* gm, const double* gv, int32_t* sel, int32_t* n_sel,
                        double* tau_hat, hipStream_t stream);

// Decode plan: the selected token slots of a (row, KV head) pair are cut into
// splits of `slots_per_item` slots (one qk work item each); the scratch arrays
// sit at fixed offsets inside the caller's workspace.
struct DecodePlan {
  int max_sel;          // upper bound on selected pages per pair
  int slots_per_item;   // token slots per qk work item
  int splits;           // ceil(max_sel * P / slots_per_item)
  long long qk_grid_cap;
  size_t counter_off, counter_bytes;  // fused tail only: int [B*Hkv], zero between launches
  size_t cand_off, cand_bytes;  // (z, physical token) [B*Hq][splits][slots_per_item]
  size_t cnt_off, cnt_bytes;    // int   [B*Hq][splits]
  size_t smax_off, smax_bytes;  // fp32  [B*Hq][splits]
  size_t total;
};

bool decode_shape_supported(const Shape& s, int max_sel);
DecodePlan make_decode_plan(const Shape& s, int max_sel, bool fused);

// ub / zlb (both set or both NULL): per-head page bounds [B][Hq][maxP] in, and
// per-head lower bounds of z_max [B][Hq] out; with them the selected pages
// that cannot hold any head's support are not read.
hipError_t launch_decode(const Shape& s, const DecodePlan& plan, const float* q, float scale,
                         float alpha, const void* K, const void* V, const int32_t* bt,
                         const int32_t* lens, const int32_t* sel, const int32_t* n_sel,
                         const float* ub, float* zlb, float* out, float* tau_out,
                         int32_t* n_support, void* ws, bool fused, hipStream_t stream);

// Top-k selection fused into the decode's key stage (one launch: every work
// item selects, probes its pair's heads with ub (NULL: no pruning) and scores
// an even share of the pages read), then the tau / PV stage.  Only for shapes
// with topk_decode_fast(s, plan.max_sel).
// hint: the box scorer's best page per (pair, page slice, head) for this
// query (NULL: none); with it each head's probe page is known before the
// selection runs.
struct TopkHint {
  const int4* hint;
  int slice_pages, nslices;
};
bool topk_decode_fast(const Shape& s, int max_sel);
hipError_t launch_topk_decode(const Shape& s, const DecodePlan& plan, const float* q, float scale,
                              float alpha, const void* K, const void* V, const int32_t* bt,
                              const int32_t* lens, int top_k, const float* ub, const float* ubg,
                              int32_t* sel, int32_t* n_sel, float* out, float* tau_out,
                              int32_t* n_support, void* ws, const TopkHint& hint,
                              hipStream_t stream);

// Softmax decode (the comparison path): split-page partials (m, l, o) of
// `slots` token slots each, merged per query head.
struct SoftmaxPlan {
  int max_sel;   // upper bound on selected pages per pair
  int slots;     // token slots per split (a multiple of the page size)
  int splits;    // ceil(max_sel * P / slots)
  size_t ml_off;  // float2 [B*Hq][splits]
  size_t o_off;   // float  [B*Hq][splits][D]
  size_t total;
};

SoftmaxPlan make_softmax_plan(const Shape& s, int max_sel);

hipError_t launch_softmax(const Shape& s, const SoftmaxPlan& plan, const float* q, float scale,
                          const void* K, const void* V, const int32_t* bt, const int32_t* lens,
                          const int32_t* sel, const int32_t* n_sel, float* out, float* lse,
                          void* ws, hipStream_t stream);

// The decode step (ekv_decode_step) with its arrival counters and the rest of
// its scratch in separate buffers; validates like the public entry point.
ekv_status decode_step_parts(const ekv_cache_desc* desc, const float* q, float scale,
                             float alpha, const void* K, const void* V,
                             const int32_t* block_table, const int32_t* seq_lens,
                             int32_t refresh_last_page, int32_t top_k, void* kmin, void* kmax,
                             float* ubg, int32_t* sel, int32_t* n_sel, float* out,
                             float* tau_out, int32_t* n_support, void* counters,
                             size_t counter_bytes, void* rest, size_t rest_bytes,
                             hipStream_t stream);

// Host-side validation of the decode step's arguments (everything but its
// scratch), as ekv_decode_step reports it.
ekv_status validate_step(const ekv_cache_desc* desc, const float* q, float scale, float alpha,
                         const void* K, const void* V, const int32_t* block_table,
                         const int32_t* seq_lens, int32_t top_k, const void* kmin,
                         const void* kmax, const float* ubg, const int32_t* sel,
                         const int32_t* n_sel, const float* out, const float* tau_out,
                         const int32_t* n_support);

// Scratch of the decode step besides its counters (0 if the shape, top_k or
// the decode plan is invalid); the counters' bytes go to *counter_bytes.
size_t step_scratch_bytes(const ekv_cache_desc* desc, int32_t top_k, size_t* counter_bytes);

}  // namespace ekv
