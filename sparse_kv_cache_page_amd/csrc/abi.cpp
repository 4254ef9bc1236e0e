// C ABI of the paged entmax decode library: host-side validation, launch
// planning and dispatch to the gfx950 kernels.  Nothing here allocates,
// frees or synchronises; every error is reported before any launch.
#include <math.h>
#include <stdint.h>

#include "entmaxkv.h"
#include "kernels.h"

namespace {

using ekv::Shape;

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int log2_exact(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return (1 << l) == x ? l : -1;
}

ekv_status make_shape(const ekv_cache_desc* d, Shape* s) {
  if (d == nullptr) return EKV_ERR_INVALID_ARG;
  if (d->batch < 1 || d->num_q_heads < 1 || d->num_kv_heads < 1 || d->head_dim < 1 ||
      d->page_size < 1 || d->max_pages_per_seq < 1 || d->num_phys_pages < 1)
    return EKV_ERR_INVALID_ARG;
  if (d->num_q_heads % d->num_kv_heads != 0) return EKV_ERR_INVALID_ARG;
  if (d->kv_dtype != EKV_BF16 && d->kv_dtype != EKV_F32) return EKV_ERR_INVALID_ARG;
  if (d->compact_moments != 0 && d->compact_moments != 1) return EKV_ERR_INVALID_ARG;
  const int G = d->num_q_heads / d->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return EKV_ERR_UNSUPPORTED;
  if (d->head_dim != 64 && d->head_dim != 128) return EKV_ERR_UNSUPPORTED;
  const int l2 = log2_exact(d->page_size);
  if (l2 < 0 || d->page_size > ekv::kMaxPageSize) return EKV_ERR_UNSUPPORTED;
  // token slots of one row and page counts must stay inside int32 indexing
  if ((long long)d->max_pages_per_seq * d->page_size > (1LL << 30)) return EKV_ERR_UNSUPPORTED;
  s->B = d->batch;
  s->Hq = d->num_q_heads;
  s->Hkv = d->num_kv_heads;
  s->G = G;
  s->D = d->head_dim;
  s->P = d->page_size;
  s->log2P = l2;
  s->maxP = d->max_pages_per_seq;
  s->Np = d->num_phys_pages;
  s->bf16 = d->kv_dtype == EKV_BF16;
  s->mom16 = d->compact_moments == 1;
  return EKV_OK;
}

bool ok_vec(const void* p) { return p != nullptr && aligned(p, 16); }
bool ok_i32(const void* p) { return p != nullptr && aligned(p, 4); }
bool ok_f64(const void* p) { return p != nullptr && aligned(p, 8); }

ekv_status from_hip(hipError_t e) { return e == hipSuccess ? EKV_OK : EKV_ERR_HIP; }

}  // namespace

extern "C" {

const char* ekv_status_string(ekv_status status) {
  switch (status) {
    case EKV_OK: return "ok";
    case EKV_ERR_INVALID_ARG: return "invalid argument";
    case EKV_ERR_UNSUPPORTED: return "unsupported shape or parameter";
    case EKV_ERR_WORKSPACE: return "workspace missing or too small";
    case EKV_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

double ekv_gauss_expected_max(int32_t n) { return ekv::expected_max_std_normal(n); }

ekv_status ekv_build_page_meta(const ekv_cache_desc* desc, const void* K,
                               const int32_t* block_table, const int32_t* seq_lens,
                               const int32_t* first_page, int32_t span, void* kmin, void* kmax,
                               void* mean, void* var, hipStream_t stream) {
  Shape s;
  ekv_status st = make_shape(desc, &s);
  if (st != EKV_OK) return st;
  if (!ok_vec(K) || !ok_i32(block_table) || !ok_i32(seq_lens) || !ok_vec(kmin) || !ok_vec(kmax))
    return EKV_ERR_INVALID_ARG;
  if (first_page != nullptr && !aligned(first_page, 4)) return EKV_ERR_INVALID_ARG;
  if ((mean == nullptr) != (var == nullptr)) return EKV_ERR_INVALID_ARG;
  if (mean != nullptr && (!ok_vec(mean) || !ok_vec(var))) return EKV_ERR_INVALID_ARG;
  if (span <= 0 || span > s.maxP) span = s.maxP;
  return from_hip(ekv::launch_build_meta(s, K, block_table, seq_lens, first_page, span, kmin,
                                         kmax, mean, var, stream));
}

ekv_status ekv_validate_cache(const ekv_cache_desc* desc, const int32_t* block_table,
                              const int32_t* seq_lens, int32_t* bad, hipStream_t stream) {
  Shape s;
  ekv_status st = make_shape(desc, &s);
  if (st != EKV_OK) return st;
  if (!ok_i32(block_table) || !ok_i32(seq_lens) || !ok_i32(bad)) return EKV_ERR_INVALID_ARG;
  return from_hip(ekv::launch_validate(s, block_table, seq_lens, bad, stream));
}

ekv_status ekv_append_token(const ekv_cache_desc* desc, const void* k_new, const void* v_new,
                            const int32_t* block_table, const int32_t* seq_lens, void* K,
                            void* V, void* kmin, void* kmax, void* mean, void* var,
                            hipStream_t stream) {
  Shape s;
  ekv_status st = make_shape(desc, &s);
  if (st != EKV_OK) return st;
  if (!ok_vec(k_new) || !ok_vec(v_new) || !ok_i32(block_table) || !ok_i32(seq_lens) ||
      !ok_vec(K) || !ok_vec(V) || !ok_vec(kmin) || !ok_vec(kmax))
    return EKV_ERR_INVALID_ARG;
  if ((mean == nullptr) != (var == nullptr)) return EKV_ERR_INVALID_ARG;
  if (mean != nullptr && (!ok_vec(mean) || !ok_vec(var))) return EKV_ERR_INVALID_ARG;
  return from_hip(ekv::launch_append(s, k_new, v_new, block_table, seq_lens, K, V, kmin, kmax,
                                     mean, var, stream));
}

ekv_status ekv_score_pages(const ekv_cache_desc* desc, const float* q, float scale,
                           const void* kmin, const void* kmax, const void* mean,
                           const void* var, const int32_t* block_table,
                           const int32_t* seq_lens, float* ub, float* ubg, double* gm,
                           double* gv, hipStream_t stream) {
  Shape s;
  ekv_status st = make_shape(desc, &s);
  if (st != EKV_OK) return st;
  if (!ok_vec(q) || !ok_vec(kmin) || !ok_vec(kmax) || !ok_i32(block_table) ||
      !ok_i32(seq_lens) || !ok_i32(ubg))
    return EKV_ERR_INVALID_ARG;
  if (ub != nullptr && !aligned(ub, 4)) return EKV_ERR_INVALID_ARG;
  if (!(scale > 0.0f) || !isfinite(scale)) return EKV_ERR_INVALID_ARG;
  if ((gm == nullptr) != (gv == nullptr)) return EKV_ERR_INVALID_ARG;
  if (gm != nullptr) {
    if (!ok_f64(gm) || !ok_f64(gv) || !ok_vec(mean) || !ok_vec(var)) return EKV_ERR_INVALID_ARG;
  }
  return from_hip(ekv::launch_score(s, q, scale, kmin, kmax, mean, var, block_table, seq_lens,
                                    ub, ubg, gm, gv, stream));
}

ekv_status ekv_select_pages(const ekv_cache_desc* desc, const int32_t* seq_lens, int32_t policy,
                            int32_t top_k, float alpha, float delta, const float* ub,
                            const float* ubg, const double* gm, const double* gv,
                            int32_t* sel, int32_t* n_sel, double* tau_hat,
                            hipStream_t stream) {
  Shape s;
  ekv_status st = make_shape(desc, &s);
  if (st != EKV_OK) return st;
  if (!ok_i32(seq_lens) || !ok_i32(ubg) || !ok_i32(sel) || !ok_i32(n_sel))
    return EKV_ERR_INVALID_ARG;
  if (policy == EKV_SELECT_TOPK) {
    if (top_k < 1) return EKV_ERR_INVALID_ARG;
    return from_hip(ekv::launch_topk(s, seq_lens, top_k, ubg, sel, n_sel, stream));
  }
  if (policy != EKV_SELECT_GAUSS && policy != EKV_SELECT_GAUSS_EST &&
      policy != EKV_SELECT_GAUSS_MASS)
    return EKV_ERR_INVALID_ARG;
  const int rule = policy == EKV_SELECT_GAUSS ? 0 : (policy == EKV_SELECT_GAUSS_EST ? 1 : 2);
  if ((rule == 0 && !ok_i32(ub)) || !ok_f64(gm) || !ok_f64(gv) || !ok_f64(tau_hat))
    return EKV_ERR_INVALID_ARG;
  if (!(alpha > 1.0f) || !isfinite(alpha)) return EKV_ERR_INVALID_ARG;
  if (!(delta >= 0.0f) || !isfinite(delta)) return EKV_ERR_INVALID_ARG;
  // gamma = 1 / (alpha - 1) >= 1 (alpha <= 2), at most 64; within 1e-6 of an
  // integer it is taken as that integer
  if (!((double)alpha <= 2.0)) return EKV_ERR_UNSUPPORTED;
  double gamma = 1.0 / ((double)alpha - 1.0);
  const double gr = rint(gamma);
  if (fabs(gamma - gr) <= 1e-6 * gr) gamma = gr;
  if (gamma > 64.0) return EKV_ERR_UNSUPPORTED;
  return from_hip(ekv::launch_gauss(s, seq_lens, alpha, gamma, delta, rule, ub, ubg, gm, gv, sel,
                                    n_sel, tau_hat, stream));
}

size_t ekv_decode_workspace_bytes(const ekv_cache_desc* desc, int32_t max_sel) {
  Shape s;
  if (make_shape(desc, &s) != EKV_OK) return 0;
  if (max_sel <= 0 || max_sel > s.maxP) max_sel = s.maxP;
  if (!ekv::decode_shape_supported(s, max_sel)) return 0;
  return ekv::make_decode_plan(s, max_sel, false).total;
}

size_t ekv_decode_fused_workspace_bytes(const ekv_cache_desc* desc, int32_t max_sel) {
  Shape s;
  if (make_shape(desc, &s) != EKV_OK) return 0;
  if (max_sel <= 0 || max_sel > s.maxP) max_sel = s.maxP;
  if (!ekv::decode_shape_supported(s, max_sel)) return 0;
  return ekv::make_decode_plan(s, max_sel, true).total;
}

}  // extern "C"

static ekv_status decode_common(const ekv_cache_desc* desc, const float* q, float scale,
                                float alpha, const void* K, const void* V,
                                const int32_t* block_table, const int32_t* seq_lens,
                                const int32_t* sel, const int32_t* n_sel, int32_t max_sel,
                                const float* ub, float* zlb, float* out, float* tau_out,
                                int32_t* n_support, void* ws, size_t ws_bytes, bool fused,
                                hipStream_t stream) {
  Shape s;
  ekv_status st = make_shape(desc, &s);
  if (st != EKV_OK) return st;
  if ((ub == nullptr) != (zlb == nullptr)) return EKV_ERR_INVALID_ARG;
  if (ub != nullptr && (!aligned(ub, 4) || !aligned(zlb, 4))) return EKV_ERR_INVALID_ARG;
  if (!ok_vec(q) || !ok_vec(K) || !ok_vec(V) || !ok_i32(block_table) || !ok_i32(seq_lens) ||
      !ok_vec(out))
    return EKV_ERR_INVALID_ARG;
  if ((sel == nullptr) != (n_sel == nullptr)) return EKV_ERR_INVALID_ARG;
  if (sel != nullptr && (!aligned(sel, 4) || !aligned(n_sel, 4))) return EKV_ERR_INVALID_ARG;
  if (tau_out != nullptr && !aligned(tau_out, 4)) return EKV_ERR_INVALID_ARG;
  if (n_support != nullptr && !aligned(n_support, 4)) return EKV_ERR_INVALID_ARG;
  if (!(alpha > 1.0f) || !isfinite(alpha)) return EKV_ERR_INVALID_ARG;
  if (!(scale > 0.0f) || !isfinite(scale)) return EKV_ERR_INVALID_ARG;
  if (max_sel <= 0 || max_sel > s.maxP) max_sel = s.maxP;
  if (!ekv::decode_shape_supported(s, max_sel)) return EKV_ERR_UNSUPPORTED;
  const ekv::DecodePlan plan = ekv::make_decode_plan(s, max_sel, fused);
  if (ws == nullptr || !aligned(ws, 256) || ws_bytes < plan.total) return EKV_ERR_WORKSPACE;
  return from_hip(ekv::launch_decode(s, plan, q, scale, alpha, K, V, block_table, seq_lens, sel,
                                     n_sel, ub, zlb, out, tau_out, n_support, ws, fused, stream));
}

extern "C" {

ekv_status ekv_entmax_decode(const ekv_cache_desc* desc, const float* q, float scale,
                             float alpha, const void* K, const void* V,
                             const int32_t* block_table, const int32_t* seq_lens,
                             const int32_t* sel, const int32_t* n_sel, int32_t max_sel,
                             const float* ub, float* zlb, float* out, float* tau_out,
                             int32_t* n_support, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
  return decode_common(desc, q, scale, alpha, K, V, block_table, seq_lens, sel, n_sel, max_sel,
                       ub, zlb, out, tau_out, n_support, ws, ws_bytes, false, stream);
}

ekv_status ekv_entmax_decode_fused(const ekv_cache_desc* desc, const float* q, float scale,
                                   float alpha, const void* K, const void* V,
                                   const int32_t* block_table, const int32_t* seq_lens,
                                   const int32_t* sel, const int32_t* n_sel, int32_t max_sel,
                                   const float* ub, float* zlb, float* out, float* tau_out,
                                   int32_t* n_support, void* ws, size_t ws_bytes,
                                   hipStream_t stream) {
  return decode_common(desc, q, scale, alpha, K, V, block_table, seq_lens, sel, n_sel, max_sel,
                       ub, zlb, out, tau_out, n_support, ws, ws_bytes, true, stream);
}

// Arrival counters of the fused score + select launch: B*Hkv ints, zero
// between calls.
static size_t step_counter_bytes(const Shape& s) {
  return (((size_t)s.B * s.Hkv * sizeof(int)) + 255) & ~(size_t)255;
}

size_t ekv_score_select_workspace_bytes(const ekv_cache_desc* desc) {
  Shape s;
  if (make_shape(desc, &s) != EKV_OK) return 0;
  return step_counter_bytes(s);
}

ekv_status ekv_score_select_pages(const ekv_cache_desc* desc, const float* q, float scale,
                                  const void* K, const int32_t* block_table,
                                  const int32_t* seq_lens, int32_t refresh_last_page,
                                  int32_t top_k, void* kmin, void* kmax, float* ub,
                                  float* ubg, int32_t* sel, int32_t* n_sel, void* ws,
                                  size_t ws_bytes, hipStream_t stream) {
  Shape s;
  ekv_status st = make_shape(desc, &s);
  if (st != EKV_OK) return st;
  if (!ok_vec(q) || !ok_vec(K) || !ok_i32(block_table) || !ok_i32(seq_lens) || !ok_vec(kmin) ||
      !ok_vec(kmax) || !ok_i32(ubg) || !ok_i32(sel) || !ok_i32(n_sel))
    return EKV_ERR_INVALID_ARG;
  if (ub != nullptr && !aligned(ub, 4)) return EKV_ERR_INVALID_ARG;
  if (!(scale > 0.0f) || !isfinite(scale)) return EKV_ERR_INVALID_ARG;
  if (top_k < 1) return EKV_ERR_INVALID_ARG;
  if (ws == nullptr || !aligned(ws, 256) || ws_bytes < step_counter_bytes(s))
    return EKV_ERR_WORKSPACE;
  return from_hip(ekv::launch_score_select(s, q, scale, K, kmin, kmax, block_table, seq_lens,
                                           refresh_last_page ? 1 : 0, ub, ubg, top_k, sel,
                                           n_sel, (int*)ws, stream));
}

// Per-head page bounds [B][Hq][maxP] and z_max lower bounds [B][Hq] (fp32) of
// the decode step's page pruning, after its arrival counters.
static size_t step_bound_bytes(const Shape& s) {
  return (((size_t)s.B * s.Hq * s.maxP * sizeof(float)) + 255) & ~(size_t)255;
}
static size_t step_zlb_bytes(const Shape& s) {
  return (((size_t)s.B * s.Hq * sizeof(float)) + 255) & ~(size_t)255;
}

// The box scorer's best-page hints of the decode step: int4 [pairs][slices][G].
static size_t step_hint_bytes(const Shape& s) {
  const ekv::ScoreSlices sl = ekv::score_box_slices(s);
  return (((size_t)s.B * s.Hkv * sl.count * s.G * 16) + 255) & ~(size_t)255;
}

// Workspace of the top-k decode: the decode plan's candidate lists, then the
// z_max lower bounds that the general path (shapes outside the fused
// selection's limits) keeps between its launches.
static size_t topk_decode_bytes(const Shape& s, int max_sel) {
  return ekv::make_decode_plan(s, max_sel, false).total + step_zlb_bytes(s);
}

// Top-k selection and the pruned (ub != NULL) sparse entmax decode: fused
// selection where the shape allows, else ekv_select_pages(TOPK) followed by
// ekv_entmax_decode; the same results either way.  Arguments validated.
static ekv_status topk_decode_launch(const Shape& s, const float* q, float scale, float alpha,
                                     const void* K, const void* V, const int32_t* block_table,
                                     const int32_t* seq_lens, int top_k, const float* ub,
                                     const float* ubg, int32_t* sel, int32_t* n_sel, float* out,
                                     float* tau_out, int32_t* n_support, void* ws,
                                     const ekv::TopkHint& hint, hipStream_t stream) {
  const int max_sel = top_k < s.maxP ? top_k : s.maxP;
  const ekv::DecodePlan plan = ekv::make_decode_plan(s, max_sel, false);
  if (ekv::topk_decode_fast(s, max_sel))
    return from_hip(ekv::launch_topk_decode(s, plan, q, scale, alpha, K, V, block_table, seq_lens,
                                            top_k, ub, ubg, sel, n_sel, out, tau_out, n_support,
                                            ws, hint, stream));
  const hipError_t e = ekv::launch_topk(s, seq_lens, top_k, ubg, sel, n_sel, stream);
  if (e != hipSuccess) return EKV_ERR_HIP;
  float* zlb = ub != nullptr ? (float*)((char*)ws + plan.total) : nullptr;
  return from_hip(ekv::launch_decode(s, plan, q, scale, alpha, K, V, block_table, seq_lens, sel,
                                     n_sel, ub, zlb, out, tau_out, n_support, ws, false, stream));
}

size_t ekv_topk_decode_workspace_bytes(const ekv_cache_desc* desc, int32_t top_k) {
  Shape s;
  if (make_shape(desc, &s) != EKV_OK || top_k < 1) return 0;
  const int max_sel = top_k < s.maxP ? top_k : s.maxP;
  if (!ekv::decode_shape_supported(s, max_sel)) return 0;
  return topk_decode_bytes(s, max_sel);
}

ekv_status ekv_topk_decode(const ekv_cache_desc* desc, const float* q, float scale, float alpha,
                           const void* K, const void* V, const int32_t* block_table,
                           const int32_t* seq_lens, int32_t top_k, const float* ub,
                           const float* ubg, const void* hint, int32_t* sel, int32_t* n_sel,
                           float* out, float* tau_out, int32_t* n_support, void* ws,
                           size_t ws_bytes, hipStream_t stream) {
  Shape s;
  ekv_status st = make_shape(desc, &s);
  if (st != EKV_OK) return st;
  if (!ok_vec(q) || !ok_vec(K) || !ok_vec(V) || !ok_i32(block_table) || !ok_i32(seq_lens) ||
      !ok_i32(ubg) || !ok_i32(sel) || !ok_i32(n_sel) || !ok_vec(out))
    return EKV_ERR_INVALID_ARG;
  if (ub != nullptr && !aligned(ub, 16)) return EKV_ERR_INVALID_ARG;
  if (tau_out != nullptr && !aligned(tau_out, 4)) return EKV_ERR_INVALID_ARG;
  if (n_support != nullptr && !aligned(n_support, 4)) return EKV_ERR_INVALID_ARG;
  if (!(alpha > 1.0f) || !isfinite(alpha)) return EKV_ERR_INVALID_ARG;
  if (!(scale > 0.0f) || !isfinite(scale)) return EKV_ERR_INVALID_ARG;
  if (top_k < 1) return EKV_ERR_INVALID_ARG;
  const int max_sel = top_k < s.maxP ? top_k : s.maxP;
  if (!ekv::decode_shape_supported(s, max_sel)) return EKV_ERR_UNSUPPORTED;
  if (hint != nullptr && !aligned(hint, 16)) return EKV_ERR_INVALID_ARG;
  if (ws == nullptr || !aligned(ws, 256) || ws_bytes < topk_decode_bytes(s, max_sel))
    return EKV_ERR_WORKSPACE;
  const ekv::ScoreSlices sl = ekv::score_box_slices(s);
  return topk_decode_launch(s, q, scale, alpha, K, V, block_table, seq_lens, top_k, ub, ubg, sel,
                            n_sel, out, tau_out, n_support, ws,
                            ekv::TopkHint{(const int4*)hint, sl.pages, sl.count}, stream);
}

size_t ekv_score_hint_bytes(const ekv_cache_desc* desc) {
  Shape s;
  if (make_shape(desc, &s) != EKV_OK) return 0;
  return step_hint_bytes(s);
}

ekv_status ekv_score_box_pages(const ekv_cache_desc* desc, const float* q, float scale,
                               const void* K, const int32_t* block_table,
                               const int32_t* seq_lens, int32_t refresh_last_page, void* kmin,
                               void* kmax, float* ub, float* ubg, void* hint,
                               hipStream_t stream) {
  Shape s;
  ekv_status st = make_shape(desc, &s);
  if (st != EKV_OK) return st;
  if (!ok_vec(q) || !ok_i32(block_table) || !ok_i32(seq_lens) || !ok_vec(kmin) ||
      !ok_vec(kmax) || !ok_i32(ubg))
    return EKV_ERR_INVALID_ARG;
  if (refresh_last_page && !ok_vec(K)) return EKV_ERR_INVALID_ARG;
  if (ub != nullptr && !aligned(ub, 16)) return EKV_ERR_INVALID_ARG;
  if (hint != nullptr && !aligned(hint, 16)) return EKV_ERR_INVALID_ARG;
  if (!(scale > 0.0f) || !isfinite(scale)) return EKV_ERR_INVALID_ARG;
  return from_hip(ekv::launch_score_box(s, q, scale, K, kmin, kmax, block_table, seq_lens,
                                        refresh_last_page ? 1 : 0, ub, ubg, (int4*)hint, stream));
}

size_t ekv_step_workspace_bytes(const ekv_cache_desc* desc, int32_t top_k) {
  Shape s;
  if (make_shape(desc, &s) != EKV_OK || top_k < 1) return 0;
  const int max_sel = top_k < s.maxP ? top_k : s.maxP;
  if (!ekv::decode_shape_supported(s, max_sel)) return 0;
  return step_counter_bytes(s) + step_bound_bytes(s) + step_hint_bytes(s) +
         topk_decode_bytes(s, max_sel);
}

ekv_status ekv_decode_step(const ekv_cache_desc* desc, const float* q, float scale, float alpha,
                           const void* K, const void* V, const int32_t* block_table,
                           const int32_t* seq_lens, int32_t refresh_last_page, int32_t top_k,
                           void* kmin, void* kmax, float* ubg, int32_t* sel, int32_t* n_sel,
                           float* out, float* tau_out, int32_t* n_support, void* ws,
                           size_t ws_bytes, hipStream_t stream) {
  Shape s;
  ekv_status st = make_shape(desc, &s);
  if (st != EKV_OK) return st;
  // counters first, then the rest (an unusable workspace is reported after
  // the other arguments have been validated)
  const size_t cbytes = step_counter_bytes(s);
  const bool fits = ws != nullptr && ws_bytes >= cbytes;
  return ekv::decode_step_parts(desc, q, scale, alpha, K, V, block_table, seq_lens,
                                refresh_last_page, top_k, kmin, kmax, ubg, sel, n_sel, out,
                                tau_out, n_support, fits ? ws : nullptr, fits ? cbytes : 0,
                                fits ? (char*)ws + cbytes : nullptr, fits ? ws_bytes - cbytes : 0,
                                stream);
}

}  // extern "C"

// The decode step with its arrival counters and the rest of its scratch in
// two separate buffers (ekv_decode_step cuts one workspace in two;
// ekv_decode_step_noalloc keeps the counters in a region of their own).
ekv_status ekv::decode_step_parts(const ekv_cache_desc* desc, const float* q, float scale,
                                  float alpha, const void* K, const void* V,
                                  const int32_t* block_table, const int32_t* seq_lens,
                                  int32_t refresh_last_page, int32_t top_k, void* kmin,
                                  void* kmax, float* ubg, int32_t* sel, int32_t* n_sel,
                                  float* out, float* tau_out, int32_t* n_support,
                                  void* counters, size_t counter_bytes, void* rest,
                                  size_t rest_bytes, hipStream_t stream) {
  ekv_status st = ekv::validate_step(desc, q, scale, alpha, K, V, block_table, seq_lens, top_k,
                                     kmin, kmax, ubg, sel, n_sel, out, tau_out, n_support);
  if (st != EKV_OK) return st;
  Shape s;
  make_shape(desc, &s);
  const int max_sel = top_k < s.maxP ? top_k : s.maxP;
  const size_t ubytes = step_bound_bytes(s);
  const size_t hbytes = step_hint_bytes(s);
  const size_t tbytes = topk_decode_bytes(s, max_sel);
  if (counters == nullptr || !aligned(counters, 256) || counter_bytes < step_counter_bytes(s))
    return EKV_ERR_WORKSPACE;
  if (rest == nullptr || !aligned(rest, 256) || rest_bytes < ubytes + hbytes + tbytes)
    return EKV_ERR_WORKSPACE;
  float* ub = (float*)rest;
  int4* hint = (int4*)((char*)rest + ubytes);
  const ekv::ScoreSlices sl = ekv::score_box_slices(s);
  const hipError_t e = ekv::launch_score_box(s, q, scale, K, kmin, kmax, block_table, seq_lens,
                                             refresh_last_page ? 1 : 0, ub, ubg, hint, stream);
  if (e != hipSuccess) return EKV_ERR_HIP;
  return topk_decode_launch(s, q, scale, alpha, K, V, block_table, seq_lens, top_k, ub, ubg, sel,
                            n_sel, out, tau_out, n_support, (char*)rest + ubytes + hbytes,
                            ekv::TopkHint{hint, sl.pages, sl.count}, stream);
}

ekv_status ekv::validate_step(const ekv_cache_desc* desc, const float* q, float scale,
                              float alpha, const void* K, const void* V,
                              const int32_t* block_table, const int32_t* seq_lens,
                              int32_t top_k, const void* kmin, const void* kmax,
                              const float* ubg, const int32_t* sel, const int32_t* n_sel,
                              const float* out, const float* tau_out,
                              const int32_t* n_support) {
  Shape s;
  ekv_status st = make_shape(desc, &s);
  if (st != EKV_OK) return st;
  if (!ok_vec(q) || !ok_vec(K) || !ok_vec(V) || !ok_i32(block_table) || !ok_i32(seq_lens) ||
      !ok_vec(kmin) || !ok_vec(kmax) || !ok_i32(ubg) || !ok_i32(sel) || !ok_i32(n_sel) ||
      !ok_vec(out))
    return EKV_ERR_INVALID_ARG;
  if (tau_out != nullptr && !aligned(tau_out, 4)) return EKV_ERR_INVALID_ARG;
  if (n_support != nullptr && !aligned(n_support, 4)) return EKV_ERR_INVALID_ARG;
  if (!(alpha > 1.0f) || !isfinite(alpha)) return EKV_ERR_INVALID_ARG;
  if (!(scale > 0.0f) || !isfinite(scale)) return EKV_ERR_INVALID_ARG;
  if (top_k < 1) return EKV_ERR_INVALID_ARG;
  const int max_sel = top_k < s.maxP ? top_k : s.maxP;
  if (!ekv::decode_shape_supported(s, max_sel)) return EKV_ERR_UNSUPPORTED;
  return EKV_OK;
}

size_t ekv::step_scratch_bytes(const ekv_cache_desc* desc, int32_t top_k, size_t* counter_bytes) {
  Shape s;
  if (make_shape(desc, &s) != EKV_OK || top_k < 1) return 0;
  const int max_sel = top_k < s.maxP ? top_k : s.maxP;
  if (!ekv::decode_shape_supported(s, max_sel)) return 0;
  *counter_bytes = step_counter_bytes(s);
  return step_bound_bytes(s) + step_hint_bytes(s) + topk_decode_bytes(s, max_sel);
}

extern "C" {

size_t ekv_softmax_workspace_bytes(const ekv_cache_desc* desc, int32_t max_sel) {
  Shape s;
  if (make_shape(desc, &s) != EKV_OK) return 0;
  if (max_sel <= 0 || max_sel > s.maxP) max_sel = s.maxP;
  return ekv::make_softmax_plan(s, max_sel).total;
}

ekv_status ekv_softmax_decode(const ekv_cache_desc* desc, const float* q, float scale,
                              const void* K, const void* V, const int32_t* block_table,
                              const int32_t* seq_lens, const int32_t* sel,
                              const int32_t* n_sel, int32_t max_sel, float* out, float* lse,
                              void* ws, size_t ws_bytes, hipStream_t stream) {
  Shape s;
  ekv_status st = make_shape(desc, &s);
  if (st != EKV_OK) return st;
  if (!ok_vec(q) || !ok_vec(K) || !ok_vec(V) || !ok_i32(block_table) || !ok_i32(seq_lens) ||
      !ok_vec(out))
    return EKV_ERR_INVALID_ARG;
  if ((sel == nullptr) != (n_sel == nullptr)) return EKV_ERR_INVALID_ARG;
  if (sel != nullptr && (!aligned(sel, 4) || !aligned(n_sel, 4))) return EKV_ERR_INVALID_ARG;
  if (lse != nullptr && !aligned(lse, 4)) return EKV_ERR_INVALID_ARG;
  if (!(scale > 0.0f) || !isfinite(scale)) return EKV_ERR_INVALID_ARG;
  if (sel == nullptr || max_sel <= 0 || max_sel > s.maxP) max_sel = s.maxP;
  const ekv::SoftmaxPlan plan = ekv::make_softmax_plan(s, max_sel);
  if (ws == nullptr || !aligned(ws, 256) || ws_bytes < plan.total) return EKV_ERR_WORKSPACE;
  return from_hip(ekv::launch_softmax(s, plan, q, scale, K, V, block_table, seq_lens, sel,
                                      n_sel, out, lse, ws, stream));
}

}  // extern "C"
