// Host-side launchers of the gfx950 kernels (internal; the public surface is
// include/entmaxkv.h).  Every launcher assumes its arguments were validated by
// the C ABI layer and only enqueues work on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ekv {

struct Shape {
  int B, Hq, Hkv, G, D, P, log2P, maxP, Np;
  bool bf16;
};

hipError_t launch_build_meta(const Shape& s, const void* K, const int32_t* bt,
                             const int32_t* lens, const int32_t* first_page, int span,
                             void* kmin, void* kmax, float* mean, float* var,
                             hipStream_t stream);

hipError_t launch_score(const Shape& s, const float* q, float scale, const void* kmin,
                        const void* kmax, const float* mean, const float* var,
                        const int32_t* bt, const int32_t* lens, float* ub, float* ubg,
                        double* gm, double* gv, hipStream_t stream);

hipError_t launch_topk(const Shape& s, const int32_t* lens, int top_k, const float* ubg,
                       int32_t* sel, int32_t* n_sel, hipStream_t stream);

hipError_t launch_gauss(const Shape& s, const int32_t* lens, float alpha, int gamma,
                        float delta, const float* ub, const float* ubg, const double* gm,
                        const double* gv, int32_t* sel, int32_t* n_sel, double* tau_hat,
                        hipStream_t stream);

// Decode plan: how the selected pages of a (row, KV head) pair are split over
// workgroups, and where the scratch arrays sit inside the caller's workspace.
struct DecodePlan {
  int max_sel;       // upper bound on selected pages per pair
  int pages_per_split;
  int splits;        // ceil(max_sel / pages_per_split)
  long long tmax;    // token slots per query head = max_sel * P
  size_t z_off, z_bytes;        // fp32 [B*Hq][tmax]
  size_t smax_off, smax_bytes;  // fp32 [B*Hq][splits]
  size_t total;
};

DecodePlan make_decode_plan(const Shape& s, int max_sel);

hipError_t launch_decode(const Shape& s, const DecodePlan& plan, const float* q, float scale,
                         float alpha, const void* K, const void* V, const int32_t* bt,
                         const int32_t* lens, const int32_t* sel, const int32_t* n_sel,
                         float* out, float* tau_out, int32_t* n_support, void* ws,
                         hipStream_t stream);

}  // namespace ekv
