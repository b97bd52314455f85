// Device-side pieces shared by the decode kernels (decode_kernels.hip: bf16
// attention and the merge; decode_f32_kernels.hip: fp32 attention): vector
// types, tile constants, softmax helpers, plan records and how a wavefront
// reads a job record.
#pragma once

#include <hip/hip_runtime.h>

#include <math.h>

#include "launch.h"

namespace pagedkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

constexpr int kNW = 4;          // wavefronts per workgroup = KV heads per job
constexpr int kDepth = 2;       // bf16 kernel: K/V tiles in flight per wavefront
constexpr int kWavesPerSimd = 2;  // bf16 kernel: occupancy it is compiled for
constexpr int kTile = 16;       // tokens per tile (MFMA rows)
constexpr int kHeadDim = 128;   // head_dim of the bf16 path
constexpr int kMaxTiles = 64;   // tiles per job: one table entry per lane
constexpr int kMaxMergeThreads = 16 * 128 / 2;  // merge block: G * head_dim / 2 threads
constexpr int kKtRow = 272;     // bf16 kernel: bytes per K row in the LDS transposition area (256 + 16)
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 1 / sum for a softmax denominator: 0 for an empty context (sum 0), NaN
// for a poisoned one (NaN sum), 1 / sum otherwise.
__device__ __forceinline__ float recip_sum(float l) { return l > 0.f ? 1.0f / l : l == 0.f ? 0.f : l; }

__device__ __forceinline__ uint32_t bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two floats as packed bfloat16, rounded to nearest even by the hardware
// conversion (v_cvt_pk_bf16_f32); lo in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2_t{lo, hi}, bf16x2_t));
}

// Max / sum over lanes i, i ^ 16, i ^ 32, i ^ 48 (one column of a 16x16
// MFMA result: rows 4*lq + r live in lanes li + 16*lq).  Each gfx950 lane
// swap (lanes i and i ^ 32, then i and i ^ 16) hands every lane its own value
// and its partner's, without the LDS round trip of a bpermute.
__device__ __forceinline__ float col_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float col_sum(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

__device__ __forceinline__ int32_t clamp_block(int32_t b, int32_t nb) { return min(max(b, 0), nb - 1); }

// The plan, the context lengths and the merge list are never written while
// a decode kernel runs.  Reading them through the constant address space lets
// the compiler use scalar loads, which are tracked apart from the vector
// memory queue: waiting for a job record then never waits for K/V loads or
// output stores in flight.
template <typename T>
__device__ __forceinline__ const __attribute__((address_space(4))) T* as_const(const T* p) {
  return (const __attribute__((address_space(4))) T*)(uintptr_t)p;
}

typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));

// Job record i of the plan, by scalar loads.
__device__ __forceinline__ pa_decode_job load_job(const pa_decode_job* jobs, int64_t i) {
  const auto* q = as_const(reinterpret_cast<const i32x4_t*>(jobs)) + 2 * i;
  const i32x4_t x = q[0], y = q[1];
  return pa_decode_job{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
}

// Four consecutive output values at element index idx (a multiple of 4).
__device__ __forceinline__ void store4(const DecodeArgs& a, int64_t idx, float x0, float x1, float x2, float x3) {
  if (a.out_bf16) {
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(a.out) + idx) =
        make_uint2(bf16_rne(x0) | (bf16_rne(x1) << 16), bf16_rne(x2) | (bf16_rne(x3) << 16));
  } else {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + idx) = make_float4(x0, x1, x2, x3);
  }
}

__device__ __forceinline__ void store1(const DecodeArgs& a, int64_t idx, float x) {
  if (a.out_bf16)
    reinterpret_cast<uint16_t*>(a.out)[idx] = (uint16_t)bf16_rne(x);
  else
    reinterpret_cast<float*>(a.out)[idx] = x;
}

// Job fields as seen by one wavefront (all wave-uniform).
struct JobView {
  int32_t seq, g, t0, cnt, L, rec;
  int32_t L_dev; // the sequence's device length (load_ref requests it with the job's table entries)
  int32_t w;     // wavefront's KV head within the head block
  int32_t grp;   // shared job: its group descriptor
  int32_t part;  // shared job: piece of the shared prefix
  int32_t ncol;  // query columns computed: G, or members x G for a shared job
  int32_t T;     // tiles of the job (cnt counts positions: T for a job, ceil(T / 4) for a wide one)
  bool idle;     // the wavefront's KV head is past the last one: read nothing, write nothing
                 // (in a wide job: the wavefront has no group of the set; it still loads its tiles)
  bool shared;   // the job reads a prefix shared by the members of a group
  bool wide;     // PA_JOB_WIDE: the workgroup's wavefronts share one KV head and exchange tiles
};

// The fields of job record jd for wavefront w (the context length comes
// with the record).  Any record (an empty slot included) gives in-range
// addresses; a wavefront whose KV head is past the last one is idle.
// Kernels built without kWide never receive wide jobs (the launch picks the
// kWide kernel for plans that hold them).
template <bool kWide = false>
__device__ __forceinline__ void view_job(const DecodeArgs& a, const pa_decode_job& jd, int w, int B, JobView& v) {
  v.shared = (jd.head_block & PA_JOB_SHARED) != 0;
  v.wide = kWide && v.shared && (jd.head_block & PA_JOB_WIDE) != 0;
  const int32_t g = v.wide ? (jd.head_block & 0xffff) : (jd.head_block & 0xffff) * kNW + w;
  // A wide job's set: jd.num_parts packs (groups, members per group, members of the last group).
  const int32_t ngr = jd.num_parts & 0xff;
  const int32_t members =
      v.wide ? (w < ngr - 1 ? (jd.num_parts >> 8) & 0xff : (jd.num_parts >> 16) & 0xff) : jd.num_parts;
  v.w = v.wide ? (g & 3) : w;
  v.idle = g < 0 || g >= a.num_kv_heads || (v.shared && a.num_groups <= 0) || (v.wide && w >= ngr);
  const int32_t grp = jd.record_base + (v.wide ? w * ((a.num_kv_heads + 3) / 4) : 0);
  v.grp = v.shared ? min(max(grp, 0), max(a.num_groups - 1, 0)) : 0;
  v.part = max(jd.part, 0);
  v.ncol = v.shared ? min(max(members, 1), 4) * a.group : a.group;
  v.g = min(max(g, 0), a.num_kv_heads - 1);
  v.T = min(max(jd.tile_count, 0), kMaxTiles);
  v.cnt = v.wide ? (v.T + 3) / 4 : v.T;
  v.seq = min(max(jd.seq, 0), a.num_seqs - 1);
  v.t0 = max(jd.tile_begin, 0);
  v.L = min(max(jd.context_len, 0), a.max_blocks * B);
  v.rec = -1;
  if (!v.shared && jd.num_parts > 1) {
    const int64_t r = (int64_t)jd.record_base + (int64_t)w * jd.num_parts + jd.part;
    v.rec = (jd.record_base >= 0 && jd.part >= 0 && jd.part < jd.num_parts && r < a.num_records) ? (int32_t)r : -2;
  }
  if (v.idle) v.rec = -2;
}

}  // namespace
}  // namespace pagedkv
