// Internal helpers shared by the gfx950 kernels of the paged entmax decode
// library: element types, 16-byte vector loads, and wave64 cross-lane
// reductions built on DPP row operations.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "entmaxkv.h"

namespace ekv {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Element types.  Keys/values are bf16 (stored as raw 16-bit patterns) or fp32.
// A lane always moves 16 bytes at a time: 8 bf16 or 4 fp32 elements.
// ---------------------------------------------------------------------------
struct bf16_t {
  uint16_t bits;
};

template <typename T> struct Elem;

template <> struct Elem<bf16_t> {
  static constexpr int kVec = 8;  // elements per 16-byte chunk
  // Widening a bf16 pattern to fp32 is exact: the pattern is the top half of
  // the fp32 word.
  __device__ static inline void unpack(const uint4& w, float* out) {
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(u[i] << 16);
      out[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
  }
};

template <> struct Elem<float> {
  static constexpr int kVec = 4;
  __device__ static inline void unpack(const uint4& w, float* out) {
    out[0] = __uint_as_float(w.x);
    out[1] = __uint_as_float(w.y);
    out[2] = __uint_as_float(w.z);
    out[3] = __uint_as_float(w.w);
  }
};

__device__ inline uint4 load16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Reinterpret 16 bytes as the 8-element bf16 vector of an MFMA operand.
__device__ inline bf16x8_t as_bf16x8(const uint4& w) {
  const u32x4_t v = {w.x, w.y, w.z, w.w};
  return __builtin_bit_cast(bf16x8_t, v);
}

// Round-to-nearest-even of a finite fp32 value to the nearest bf16 value
// (returned as fp32).
__device__ inline float bf16_round(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u;
  return __uint_as_float(r);
}
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Streaming loads for data touched once per step (K/V tiles, page metadata).
__device__ inline uint4 load16_stream(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ inline uint2 load8_stream(const void* p) {
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(v.x, v.y);
}

// Workgroup barrier that orders LDS accesses only: global loads in flight
// stay in flight (a full __syncthreads() also waits for them).
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------------------------
// DPP helpers (gfx9 encodings).  Within a row of 16 lanes, the butterfly
//   quad_perm[1,0,3,2], quad_perm[2,3,0,1], row_half_mirror, row_mirror
// leaves the full 16-lane sum in every lane of the row.
// ---------------------------------------------------------------------------
enum : int {
  kDppQuadSwap1 = 0xB1,      // quad_perm [1,0,3,2]
  kDppQuadSwap2 = 0x4E,      // quad_perm [2,3,0,1]
  kDppRowHalfMirror = 0x141,
  kDppRowMirror = 0x140,
};

// The patterns above read a lane of the same row for every lane, so all rows
// and banks are written and bound_ctrl can be set: the previous contents of
// the destination are then dead and need no initialisation.
template <int kCtrl>
__device__ inline float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xF, 0xF, true));
}

template <int kCtrl>
__device__ inline double dpp_f64(double x) {
  const int2 v = *reinterpret_cast<int2*>(&x);
  int2 r;
  r.x = __builtin_amdgcn_update_dpp(0, v.x, kCtrl, 0xF, 0xF, true);
  r.y = __builtin_amdgcn_update_dpp(0, v.y, kCtrl, 0xF, 0xF, true);
  return *reinterpret_cast<double*>(&r);
}

// Sum over groups of `kLanes` consecutive lanes (kLanes in {1,2,4,8,16,32,64});
// every lane of a group receives the group's total.
template <int kLanes>
__device__ inline float group_sum_f32(float x) {
  if constexpr (kLanes >= 2) x += dpp_f32<kDppQuadSwap1>(x);
  if constexpr (kLanes >= 4) x += dpp_f32<kDppQuadSwap2>(x);
  if constexpr (kLanes >= 8) x += dpp_f32<kDppRowHalfMirror>(x);
  if constexpr (kLanes >= 16) x += dpp_f32<kDppRowMirror>(x);
  if constexpr (kLanes >= 32) x += __shfl_xor(x, 16, kWave);
  if constexpr (kLanes >= 64) x += __shfl_xor(x, 32, kWave);
  return x;
}

// Maximum over groups of `kLanes` consecutive lanes (kLanes in {1,2,4,8,16}),
// returned to every lane of the group.
template <int kLanes>
__device__ inline float group_max_f32(float x) {
  if constexpr (kLanes >= 2) x = fmaxf(x, dpp_f32<kDppQuadSwap1>(x));
  if constexpr (kLanes >= 4) x = fmaxf(x, dpp_f32<kDppQuadSwap2>(x));
  if constexpr (kLanes >= 8) x = fmaxf(x, dpp_f32<kDppRowHalfMirror>(x));
  if constexpr (kLanes >= 16) x = fmaxf(x, dpp_f32<kDppRowMirror>(x));
  static_assert(kLanes <= 16, "groups within one DPP row");
  return x;
}

template <int kLanes>
__device__ inline double group_sum_f64(double x) {
  if constexpr (kLanes >= 2) x += dpp_f64<kDppQuadSwap1>(x);
  if constexpr (kLanes >= 4) x += dpp_f64<kDppQuadSwap2>(x);
  if constexpr (kLanes >= 8) x += dpp_f64<kDppRowHalfMirror>(x);
  if constexpr (kLanes >= 16) x += dpp_f64<kDppRowMirror>(x);
  if constexpr (kLanes >= 32) x += __shfl_xor(x, 16, kWave);
  if constexpr (kLanes >= 64) x += __shfl_xor(x, 32, kWave);
  return x;
}

// Wave-wide reductions of 32-bit values, returned to every lane: the DPP row
// butterfly leaves each row's result in all its lanes, row_bcast15 /
// row_bcast31 carry rows 0-2 into row 3, and lane 63 is read back.  Rows that
// a broadcast does not write keep their own value (old = x).
template <typename Op>
__device__ inline int wave_reduce_b32(int x, Op op) {
  x = op(x, __builtin_amdgcn_update_dpp(0, x, kDppQuadSwap1, 0xF, 0xF, true));
  x = op(x, __builtin_amdgcn_update_dpp(0, x, kDppQuadSwap2, 0xF, 0xF, true));
  x = op(x, __builtin_amdgcn_update_dpp(0, x, kDppRowHalfMirror, 0xF, 0xF, true));
  x = op(x, __builtin_amdgcn_update_dpp(0, x, kDppRowMirror, 0xF, 0xF, true));
  x = op(x, __builtin_amdgcn_update_dpp(x, x, 0x142, 0xA, 0xF, false));  // row_bcast:15
  x = op(x, __builtin_amdgcn_update_dpp(x, x, 0x143, 0xC, 0xF, false));  // row_bcast:31
  return __builtin_amdgcn_readlane(x, 63);
}

__device__ inline float wave_max_f32(float x) {
  return __int_as_float(wave_reduce_b32(__float_as_int(x), [](int a, int b) {
    return __float_as_int(fmaxf(__int_as_float(a), __int_as_float(b)));
  }));
}

__device__ inline uint32_t wave_min_u32(uint32_t x) {
  return (uint32_t)wave_reduce_b32((int)x, [](int a, int b) { return (int)min((uint32_t)a, (uint32_t)b); });
}

__device__ inline uint32_t wave_max_u32(uint32_t x) {
  return (uint32_t)wave_reduce_b32((int)x, [](int a, int b) { return (int)max((uint32_t)a, (uint32_t)b); });
}

// Inclusive prefix sum over the 64 lanes: Hillis-Steele row shifts (lanes
// shifted in from outside the row read 0), then the row broadcasts add the
// totals of the rows below.
__device__ inline int wave_incl_scan_i32(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}

// Sum over the 64 lanes, returned to every lane (wave-uniform): DPP row
// butterfly, then row_bcast15 / row_bcast31 carry the row sums into the last
// row, and lane 63 is read back into a scalar register.  No LDS traffic.
__device__ inline float wave_sum_f32(float x) {
  x = group_sum_f32<16>(x);
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x142, 0xA, 0xF, false));  // row_bcast:15
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x143, 0xC, 0xF, false));  // row_bcast:31
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

// Lane `l`'s value of a double, in a scalar register.
__device__ inline double readlane_f64(double x, int l) {
  const int2 v = *reinterpret_cast<int2*>(&x);
  int2 r;
  r.x = __builtin_amdgcn_readlane(v.x, l);
  r.y = __builtin_amdgcn_readlane(v.y, l);
  return *reinterpret_cast<double*>(&r);
}

__device__ inline double wave_sum_f64(double x) {
  x = group_sum_f64<16>(x);
  const int2 v = *reinterpret_cast<int2*>(&x);
  int2 t;
  t.x = __builtin_amdgcn_update_dpp(0, v.x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  t.y = __builtin_amdgcn_update_dpp(0, v.y, 0x142, 0xA, 0xF, false);
  x += *reinterpret_cast<double*>(&t);
  const int2 v2 = *reinterpret_cast<int2*>(&x);
  t.x = __builtin_amdgcn_update_dpp(0, v2.x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  t.y = __builtin_amdgcn_update_dpp(0, v2.y, 0x143, 0xC, 0xF, false);
  x += *reinterpret_cast<double*>(&t);
  const int2 v3 = *reinterpret_cast<int2*>(&x);
  int2 r;
  r.x = __builtin_amdgcn_readlane(v3.x, 63);
  r.y = __builtin_amdgcn_readlane(v3.y, 63);
  return *reinterpret_cast<double*>(&r);
}

__device__ inline int wave_sum_i32(int x) {
  return wave_reduce_b32(x, [](int a, int b) { return a + b; });
}

// The bf16 value nearest to an fp64 value (ties to an even last bit), as its
// 16-bit pattern, rounded once: the value is first truncated to fp32 with
// the last bit set when anything was dropped (round to odd), which keeps 16
// more bits than bf16 and marks inexact values, so the round to nearest even
// that follows sees the true position of x and cannot land on a false tie.
// For finite x within the fp32 range.
__device__ inline uint32_t bf16_bits_rn(double x) {
  const float f = __double2float_rz(x);
  uint32_t u = __float_as_uint(f);
  u |= (double)f != x ? 1u : 0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Number of valid tokens of logical page p in a row of length L.
__device__ inline int page_valid(int L, int p, int P) {
  const int r = L - p * P;
  return r < P ? r : P;
}

}  // namespace ekv
