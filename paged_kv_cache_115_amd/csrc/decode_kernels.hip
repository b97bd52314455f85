// Paged decode attention kernels for gfx950 (CDNA4).
//
// Computed (llminference.xinbetween.com S06 "PagedAttention", the
// paged_attention excerpt under "Implementation"; aicassindra.com
// "tm_paged_attention_deep", "The block table: logical to physical mapping"):
//   out[s][h] = sum_t softmax_t(scale * q[s][h] . K_t[g]) V_t[g],  g = h / G,
// where token t's row is read at physical block table[s][t / B], offset t % B,
// directly inside the kernel: no gathered copy is materialised (S06 "Why this
// needed a custom CUDA kernel").
//
// Work decomposition.  One workgroup of kNW wavefronts per (work item, KV
// head); a work item is one partition of one sequence, built on the host by
// pa_decode_plan, largest first.  A partition's tokens are cut into 16-token
// tiles handed round-robin to the wavefronts.  Each wavefront keeps an
// online-softmax state (running max m, running sum l, unnormalised
// accumulator o) for the G query heads of its KV head; the kNW states are
// merged in LDS in wavefront order.  A sequence held in one partition writes
// its output directly; a split sequence writes (m, l, o) of each partition to
// the workspace and a second, small kernel merges the partitions in partition
// order.  Every floating-point reduction order depends only on logical token
// positions: results are bitwise reproducible and do not depend on physical
// block ids.  Softmax runs in base 2 on scores pre-multiplied by log2(e).
//
// bf16 path (head_dim 128, G <= 16): both contractions run on MFMA.
//   S^T[token][head] = K_tile[16 x 128] . Q^T[128 x 16]  with
//     v_mfma_f32_16x16x32_bf16; K is the A operand, loaded straight from the
//     pool (lane = token row, 16 bytes = 8 dims); Q^T is the B operand, kept in
//     registers (query heads beyond G are zero).
//   O^T[dim][head] += V^T[dims x 16 tokens] . P^T[16 tokens x 16 heads] with
//     v_mfma_f32_16x16x16_bf16.  The S^T result layout (lane holds tokens
//     4q..4q+3 of head lane%16) is exactly the B-operand layout P^T needs, so
//     probabilities never leave registers.  V is read in whole 256-byte rows:
//     the 16 lanes of group q read token 4q + r, lane i taking dims
//     8i .. 8i + 7.  Instance c of the PV product maps its row i to dim
//     8i + c, so its A operand is assembled from the loaded registers by
//     16-bit lane-local shuffles (no LDS round trip, no cross-lane transpose).
//   Probabilities are rounded to bf16 for the PV product and the running sum
//   adds the same rounded values, so numerator and denominator agree.
//   Each wavefront holds the block-table entries of its tiles in one vector
//   register (lane j: its j-th tile) and reads them with readlane; the K/V
//   loads of the next tile are issued before the current tile is computed.
// f32 path (head_dim 64 or 128, any G <= 16): vector ALU; each lane owns
//   head_dim/64 dims, a query-key dot product is a wavefront butterfly sum.
#include <hip/hip_runtime.h>

#include <math.h>

#include "launch.h"

namespace pagedkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kNW = 4;                   // wavefronts per workgroup
constexpr int kMaxGroup = 16;            // query heads per KV head
constexpr int kTile = 16;                // tokens per tile (MFMA rows)
constexpr int kChunk = kTile * kNW * 64; // tokens whose table entries fit one register per wave
constexpr int kTblChunk = 256;           // f32 path: table entries staged in LDS at a time

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

__device__ __forceinline__ int32_t clamp_block(int32_t b, int32_t nb) { return min(max(b, 0), nb - 1); }

// LDS layout shared by the attention kernels (dynamic shared memory, floats):
//   [0, kTblChunk)                         int32 staged table entries (f32 path)
//   m[kNW][kMaxGroup], l[kNW][kMaxGroup]   per-wavefront softmax state
//   o[kNW][G][D + 4]                       per-wavefront accumulators
struct Smem {
  int32_t* tbl;
  float* m;
  float* l;
  float* o;
  int pitch;
};

__device__ __forceinline__ Smem carve(float* base, int G, int D) {
  Smem s;
  s.tbl = reinterpret_cast<int32_t*>(base);
  s.m = base + kTblChunk;
  s.l = s.m + kNW * kMaxGroup;
  s.o = s.l + kNW * kMaxGroup;
  s.pitch = D + 4;
  return s;
}

size_t smem_bytes(int G, int D) {
  return sizeof(float) * (kTblChunk + 2 * kNW * kMaxGroup + (size_t)kNW * G * (D + 4));
}

__device__ __forceinline__ void store_out(const DecodeArgs& a, int64_t idx, float v) {
  if (a.out_bf16)
    reinterpret_cast<uint16_t*>(a.out)[idx] = (uint16_t)bf16_rne(v);
  else
    reinterpret_cast<float*>(a.out)[idx] = v;
}

// A work item whose indices would reach outside the workspace is dropped
// (its plan did not come from pa_decode_plan with these sizes).
__device__ __forceinline__ bool item_ok(const DecodeArgs& a, const pa_work_item& it) {
  if (it.part < 0 || it.part >= it.num_parts) return false;
  if (it.num_parts == 1) return true;
  return it.partial_base >= 0 && (int64_t)it.partial_base + it.num_parts <= a.num_partials;
}

// Token range [start, end) of a work item, with L clamped to the table.
struct Range {
  int32_t s, g, start, end;
};

template <int B>
__device__ __forceinline__ Range item_range(const DecodeArgs& a, const pa_work_item& it) {
  Range r;
  r.g = (int32_t)(blockIdx.x % (uint32_t)a.num_kv_heads);
  r.s = min(max(it.seq, 0), a.num_seqs - 1);
  const int32_t L = min(max(a.lens[r.s], 0), a.max_blocks * B);
  const int32_t P = a.partition > 0 ? a.partition : L;
  r.start = min(it.part * P, L);
  r.end = min(L, r.start + P);
  return r;
}

// Merge the wavefront states held in LDS.  One partition: the output.  Split
// sequence: this partition's record (max, sum, unnormalised o) in the
// workspace, merged later by merge_partials_kernel.
template <int D>
__device__ void finish(const DecodeArgs& a, const pa_work_item& it, int32_t s, int32_t g,
                       const Smem& sm) {
  const int G = a.group;
  const bool split = it.num_parts > 1;
  const int64_t out_base = ((int64_t)s * a.num_q_heads + (int64_t)g * G) * D;
  for (int idx = threadIdx.x; idx < G * D; idx += kNW * 64) {
    const int h = idx / D;
    const int d = idx - h * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kNW; ++w) M = fmaxf(M, sm.m[w * kMaxGroup + h]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < kNW; ++w) {
      const float f = M == -INFINITY ? 0.f : fast_exp2(sm.m[w * kMaxGroup + h] - M);
      den += f * sm.l[w * kMaxGroup + h];
      num += f * sm.o[(w * G + h) * sm.pitch + d];
    }
    if (!split) {
      store_out(a, out_base + idx, den > 0.f ? num / den : 0.f);
    } else {
      const int64_t rec = (int64_t)(it.partial_base + it.part) * a.num_q_heads + (int64_t)g * G + h;
      a.partial_o[rec * D + d] = num;
      if (d == 0) {
        a.partial_ml[2 * rec] = M;
        a.partial_ml[2 * rec + 1] = den;
      }
    }
  }
}

// --------------------------------------------------------------------------
// bf16, head_dim 128: MFMA for QK^T and PV.
// --------------------------------------------------------------------------
template <int B>
__global__ __launch_bounds__(kNW * 64, 2) void decode_bf16_kernel(DecodeArgs a) {
  constexpr int D = 128;
  static_assert(B == 8 || B == 16 || B == 32, "block size");
  extern __shared__ float smem_raw[];
  const int G = a.group;
  const Smem sm = carve(smem_raw, G, D);
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int li = lane & 15;  // MFMA row / column within a 16-lane group
  const int lq = lane >> 4;  // which 16-lane group
  const pa_work_item it = a.items[blockIdx.x / a.num_kv_heads];
  if (!item_ok(a, it)) return;
  const Range rg = item_range<B>(a, it);

  // Q^T fragments: lane holds Q[head li][32*ks + 8*lq .. +8] for ks = 0..3.
  bf16x8_t qf[4];
  {
    const uint4* qrow = reinterpret_cast<const uint4*>(
        reinterpret_cast<const uint16_t*>(a.q) +
        ((int64_t)rg.s * a.num_q_heads + (int64_t)rg.g * G + li) * D);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint4 v = li < G ? qrow[4 * ks + lq] : make_uint4(0, 0, 0, 0);
      qf[ks] = __builtin_bit_cast(bf16x8_t, v);
    }
  }

  float m_run = -INFINITY;
  float l_run = 0.f;
  float4_t o[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) o[c] = float4_t{0.f, 0.f, 0.f, 0.f};

  // Byte addressing: slot row r of KV head g starts at base + r * row_bytes.
  const int64_t row_bytes = (int64_t)a.num_kv_heads * D * 2;
  const char* kbase = reinterpret_cast<const char*>(a.k) + (int64_t)rg.g * D * 2;
  const char* vbase = reinterpret_cast<const char*>(a.v) + (int64_t)rg.g * D * 2;
  const int32_t* trow = a.tables + (int64_t)rg.s * a.max_blocks;
  constexpr int kTilesPerBlock = B >= kTile ? B / kTile : 1;

  for (int32_t c0 = rg.start; c0 < rg.end; c0 += kChunk) {
    const int32_t c1 = min(rg.end, c0 + kChunk);
    const int32_t ntile = (c1 - c0 + kTile - 1) / kTile;
    const int32_t mine = ntile > w ? (ntile - w + kNW - 1) / kNW : 0;
    const int32_t blk0 = c0 / B;
    // Table entries of this wave's tiles: lane j <-> tile w + kNW * j.  Lanes
    // past the last tile read an in-row entry that is never used.
    int32_t tb0, tb1 = 0;
    {
      const int32_t k = w + kNW * lane;
      int32_t e0 = B == 8 ? blk0 + 2 * k : blk0 + k / kTilesPerBlock;
      e0 = min(e0, a.max_blocks - 1);
      tb0 = clamp_block(trow[e0], a.num_blocks);
      if (B == 8) tb1 = clamp_block(trow[min(e0 + 1, a.max_blocks - 1)], a.num_blocks);
    }

    auto load_tile = [&](int i, uint4 (&kf)[4], uint4 (&vf)[4]) {
      const int32_t k = w + kNW * i;
      const int32_t p0 = __builtin_amdgcn_readlane(tb0, i);
      int64_t krow, vrow[4];
      if (B == 8) {
        const int32_t p1 = __builtin_amdgcn_readlane(tb1, i);
        krow = (int64_t)(li < 8 ? p0 : p1) * B + (li & 7);
#pragma unroll
        for (int r = 0; r < 4; ++r) vrow[r] = (int64_t)(lq < 2 ? p0 : p1) * B + ((4 * lq + r) & 7);
      } else {
        const int32_t half = (k % kTilesPerBlock) * kTile;
        krow = (int64_t)p0 * B + half + li;
#pragma unroll
        for (int r = 0; r < 4; ++r) vrow[r] = (int64_t)p0 * B + half + 4 * lq + r;
      }
      const uint4* kr = reinterpret_cast<const uint4*>(kbase + krow * row_bytes);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kf[ks] = kr[4 * ks + lq];
#pragma unroll
      for (int r = 0; r < 4; ++r) vf[r] = reinterpret_cast<const uint4*>(vbase + vrow[r] * row_bytes)[li];
    };

    auto compute_tile = [&](int i, const uint4 (&kf)[4], uint4 (&vf)[4]) {
      const int32_t t0 = c0 + kTile * (w + kNW * i);
      const bool tail = t0 + kTile > c1;  // wave-uniform: only the last tile of a chunk
      if (tail) {
        // Slots past the end hold arbitrary bits; V must be exactly zero there
        // because 0 * NaN would poison the PV product.
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (t0 + 4 * lq + r >= c1) vf[r] = make_uint4(0, 0, 0, 0);
      }
      float4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kf[ks]), qf[ks],
                                                       sacc, 0, 0, 0);
      float x[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        x[r] = sacc[r] * a.scale_log2e;
        if (tail && t0 + 4 * lq + r >= c1) x[r] = -INFINITY;
      }
      float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - m_new);
      uint32_t pb[4];
      float psum = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pb[r] = bf16_rne(fast_exp2(x[r] - m_new));
        psum += __uint_as_float(pb[r] << 16);
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
      const short4_t pfrag = __builtin_bit_cast(
          short4_t, make_uint2(pb[0] | (pb[1] << 16), pb[2] | (pb[3] << 16)));
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int wd = c >> 1;
        uint32_t lo, hi;
        if (c & 1) {
          lo = (word(vf[0], wd) >> 16) | (word(vf[1], wd) & 0xffff0000u);
          hi = (word(vf[2], wd) >> 16) | (word(vf[3], wd) & 0xffff0000u);
        } else {
          lo = (word(vf[0], wd) & 0xffffu) | (word(vf[1], wd) << 16);
          hi = (word(vf[2], wd) & 0xffffu) | (word(vf[3], wd) << 16);
        }
        o[c] *= alpha;
        o[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
            __builtin_bit_cast(short4_t, make_uint2(lo, hi)), pfrag, o[c], 0, 0, 0);
      }
    };

    // Two register sets: the loads of tile i + 1 are in flight while tile i
    // is computed.
    uint4 kA[4], vA[4], kB[4], vB[4];
    if (mine > 0) load_tile(0, kA, vA);
    for (int i = 0; i < mine; i += 2) {
      if (i + 1 < mine) load_tile(i + 1, kB, vB);
      compute_tile(i, kA, vA);
      if (i + 1 >= mine) break;
      if (i + 2 < mine) load_tile(i + 2, kA, vA);
      compute_tile(i + 1, kB, vB);
    }
  }

  // Wavefront state -> LDS.  Lane (li, lq) holds, for head li, the
  // accumulator rows 4*lq + r of instance c: dims 32*lq + 8*r + c.
  float lt = l_run + __shfl_xor(l_run, 16);
  lt = lt + __shfl_xor(lt, 32);
  if (li < G) {
    if (lq == 0) {
      sm.m[w * kMaxGroup + li] = m_run;
      sm.l[w * kMaxGroup + li] = lt;
    }
    float* orow = sm.o + (w * G + li) * sm.pitch + 32 * lq;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      *reinterpret_cast<float4*>(orow + 8 * r) = make_float4(o[0][r], o[1][r], o[2][r], o[3][r]);
      *reinterpret_cast<float4*>(orow + 8 * r + 4) = make_float4(o[4][r], o[5][r], o[6][r], o[7][r]);
    }
  }
  __syncthreads();
  finish<D>(a, it, rg.s, rg.g, sm);
}

// --------------------------------------------------------------------------
// f32: vector ALU.  Lane owns dims lane + 64*j.  Table entries staged in LDS.
// --------------------------------------------------------------------------
template <int B, int D>
__global__ __launch_bounds__(kNW * 64, 2) void decode_f32_kernel(DecodeArgs a) {
  constexpr int DPL = D / 64;
  extern __shared__ float smem_raw[];
  const int G = a.group;
  const Smem sm = carve(smem_raw, G, D);
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const pa_work_item it = a.items[blockIdx.x / a.num_kv_heads];
  if (!item_ok(a, it)) return;
  const Range rg = item_range<B>(a, it);

  float qv[kMaxGroup][DPL];
  float m_run[kMaxGroup], l_run[kMaxGroup], o[kMaxGroup][DPL];
  const float* qrow = reinterpret_cast<const float*>(a.q) +
                      ((int64_t)rg.s * a.num_q_heads + (int64_t)rg.g * G) * D;
#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.f;
#pragma unroll
    for (int j = 0; j < DPL; ++j) {
      qv[h][j] = h < G ? qrow[h * D + lane + 64 * j] : 0.f;
      o[h][j] = 0.f;
    }
  }

  const int64_t row_stride = (int64_t)a.num_kv_heads * D;
  const float* kbase = reinterpret_cast<const float*>(a.k) + (int64_t)rg.g * D;
  const float* vbase = reinterpret_cast<const float*>(a.v) + (int64_t)rg.g * D;
  const int32_t* trow = a.tables + (int64_t)rg.s * a.max_blocks;

  for (int32_t c0 = rg.start; c0 < rg.end; c0 += kTblChunk * B) {
    const int32_t c1 = min(rg.end, c0 + kTblChunk * B);
    const int32_t blk0 = c0 / B;
    const int32_t nblk = (c1 - c0 + B - 1) / B;
    __syncthreads();
    for (int i = threadIdx.x; i < nblk; i += kNW * 64) sm.tbl[i] = clamp_block(trow[blk0 + i], a.num_blocks);
    __syncthreads();
    const int32_t ntile = (c1 - c0 + kTile - 1) / kTile;
    for (int32_t tile = w; tile < ntile; tile += kNW) {
      const int32_t t0 = c0 + tile * kTile;
      const int32_t n = min(kTile, c1 - t0);
      for (int32_t i = 0; i < n; ++i) {
        const int32_t t = t0 + i;
        const int32_t p = sm.tbl[t / B - blk0];
        const int64_t row = ((int64_t)p * B + t % B) * row_stride;
        float kv[DPL], vv[DPL];
#pragma unroll
        for (int j = 0; j < DPL; ++j) {
          kv[j] = kbase[row + lane + 64 * j];
          vv[j] = vbase[row + lane + 64 * j];
        }
#pragma unroll
        for (int h = 0; h < kMaxGroup; ++h) {
          if (h >= G) break;
          float dot = 0.f;
#pragma unroll
          for (int j = 0; j < DPL; ++j) dot += qv[h][j] * kv[j];
#pragma unroll
          for (int off = 32; off >= 1; off >>= 1) dot += __shfl_xor(dot, off);
          const float x = dot * a.scale_log2e;
          const float m_new = fmaxf(m_run[h], x);
          const float alpha = fast_exp2(m_run[h] - m_new);
          const float pr = fast_exp2(x - m_new);
          l_run[h] = l_run[h] * alpha + pr;
#pragma unroll
          for (int j = 0; j < DPL; ++j) o[h][j] = o[h][j] * alpha + pr * vv[j];
          m_run[h] = m_new;
        }
      }
    }
  }

#pragma unroll
  for (int h = 0; h < kMaxGroup; ++h) {
    if (h >= G) break;
    if (lane == 0) {
      sm.m[w * kMaxGroup + h] = m_run[h];
      sm.l[w * kMaxGroup + h] = l_run[h];
    }
#pragma unroll
    for (int j = 0; j < DPL; ++j) sm.o[(w * G + h) * sm.pitch + lane + 64 * j] = o[h][j];
  }
  __syncthreads();
  finish<D>(a, it, rg.s, rg.g, sm);
}

// --------------------------------------------------------------------------
// Split-K merge: for every split sequence and KV head, combine the partition
// records in partition order:
//   M = max_p m_p,  out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p.
// --------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void merge_partials_kernel(DecodeArgs a) {
  const pa_work_item it = a.items[a.num_items + blockIdx.x / a.num_kv_heads];
  const int32_t g = (int32_t)(blockIdx.x % (uint32_t)a.num_kv_heads);
  if (it.num_parts < 2 || it.partial_base < 0 ||
      (int64_t)it.partial_base + it.num_parts > a.num_partials || it.seq < 0 || it.seq >= a.num_seqs)
    return;
  const int G = a.group;
  const int64_t out_base = ((int64_t)it.seq * a.num_q_heads + (int64_t)g * G) * D;
  for (int idx = threadIdx.x; idx < G * D; idx += 256) {
    const int h = idx / D;
    const int d = idx - h * D;
    const int64_t rec0 = (int64_t)it.partial_base * a.num_q_heads + (int64_t)g * G + h;
    float M = -INFINITY;
    for (int p = 0; p < it.num_parts; ++p)
      M = fmaxf(M, a.partial_ml[2 * (rec0 + (int64_t)p * a.num_q_heads)]);
    float num = 0.f, den = 0.f;
    for (int p = 0; p < it.num_parts; ++p) {
      const int64_t rec = rec0 + (int64_t)p * a.num_q_heads;
      const float f = M == -INFINITY ? 0.f : fast_exp2(a.partial_ml[2 * rec] - M);
      den += f * a.partial_ml[2 * rec + 1];
      num += f * a.partial_o[rec * D + d];
    }
    store_out(a, out_base + idx, den > 0.f ? num / den : 0.f);
  }
}

hipError_t launch_merge(const DecodeArgs& a, int32_t num_merges, hipStream_t stream) {
  if (num_merges == 0) return hipSuccess;
  const dim3 grid((unsigned)num_merges * (unsigned)a.num_kv_heads);
  if (a.head_dim == 128)
    hipLaunchKernelGGL(merge_partials_kernel<128>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(merge_partials_kernel<64>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, int32_t num_merges, hipStream_t stream) {
  if (a.num_items == 0) return hipSuccess;
  const dim3 grid((unsigned)a.num_items * (unsigned)a.num_kv_heads);
  const size_t smem = smem_bytes(a.group, 128);
  switch (a.block_size) {
    case 8: hipLaunchKernelGGL(decode_bf16_kernel<8>, grid, dim3(kNW * 64), smem, stream, a); break;
    case 16: hipLaunchKernelGGL(decode_bf16_kernel<16>, grid, dim3(kNW * 64), smem, stream, a); break;
    case 32: hipLaunchKernelGGL(decode_bf16_kernel<32>, grid, dim3(kNW * 64), smem, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_merge(a, num_merges, stream);
}

hipError_t launch_decode_f32(const DecodeArgs& a, int32_t num_merges, hipStream_t stream) {
  if (a.num_items == 0) return hipSuccess;
  const dim3 grid((unsigned)a.num_items * (unsigned)a.num_kv_heads);
  const size_t smem = smem_bytes(a.group, a.head_dim);
  bool launched = false;
#define PA_F32_CASE(BS, DD)                                                                       \
  if (!launched && a.block_size == BS && a.head_dim == DD) {                                      \
    hipLaunchKernelGGL((decode_f32_kernel<BS, DD>), grid, dim3(kNW * 64), smem, stream, a);       \
    launched = true;                                                                              \
  }
  PA_F32_CASE(8, 64)
  PA_F32_CASE(16, 64)
  PA_F32_CASE(32, 64)
  PA_F32_CASE(8, 128)
  PA_F32_CASE(16, 128)
  PA_F32_CASE(32, 128)
#undef PA_F32_CASE
  if (!launched) return hipErrorInvalidValue;
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_merge(a, num_merges, stream);
}

}  // namespace pagedkv
