// Paged decode attention over an fp32 KV pool (head_dim 64 or 128, up to 16
// query heads per KV head, any supported block size).
//
// Computed (llminference.xinbetween.com S06 "PagedAttention", the
// paged_attention excerpt under "Implementation"; aicassindra.com
// "tm_paged_attention_deep", "The block table: logical to physical mapping"):
//   out[s][h] = sum_t softmax_t(scale * q[s][h] . K_t[g]) V_t[g],  g = h / G,
// token t's row read at physical block table[s][t / B], offset t % B.
//
// Same plan, jobs and records as the bf16 kernel (a job is a run of one
// sequence's 16-token tiles for the four KV heads of a head block; wavefront
// w takes KV head 4 * head_block + w; a piece of a cut sequence writes an
// (m, l, o) record that the merge launch combines).  Both contractions run on
// v_mfma_f32_16x16x4_f32, in fp32 throughout:
//   S^T[token][col] = sum_d K[token][d] Q[col][d]: K is the A operand (lane
//     (i, kq) holds row i, dims 16m + 4kq + c over the steps (m, c)), Q the B
//     operand in the same dim order; the dot product's order of dims does not
//     matter, so both are read as 16-byte chunks.
//   O^T[dim][col] += sum_token V[token][dim] P[token][col]: the S^T result
//     holds tokens 4q + r of column i in lane (i, q), which is the B-operand
//     layout of P^T at k-step r when token 4k + r is k-step r's row k.  Instance
//     (b, c) maps its row i to dim 64b + 4i + c, so lane (i, k) supplies its A
//     operand from the 16-byte load of V[token 4k + r][64b + 4i ..]: no
//     transposition, no LDS.
// A job's block-table entries are loaded once, lane i holding entries
// e0 + i and e0 + 64 + i of the job's first entry e0 (jobs span at most 128
// entries: pa_decode caps jobs at 8 * B tiles below 8 slots per block), and
// every row takes its entry from those registers by a cross-lane permute, so
// any block size takes the same path.  Rows past the context read a fixed
// finite row (the new row with the append fused, else the query row) and
// carry probability 0.  With this step's append fused the row of token L - 1
// comes from new_key/new_value.  The next tile's rows are in flight while a
// tile is computed.
#include "decode_common.h"

namespace pagedkv {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Table entry `e` of a job's window (lane i of tb0: entry i, of tb1: entry
// 64 + i); e is per lane, in [0, 128).
__device__ __forceinline__ int32_t window_entry(int32_t tb0, int32_t tb1, int32_t e) {
  const int32_t lo = __shfl(tb0, e & 63), hi = __shfl(tb1, e & 63);
  return e < 64 ? lo : hi;
}

template <int D>
struct F32Tile {
  f32x4_t k[D / 16];     // K row li, dims 16m + 4lq .. + 4
  f32x4_t v[4][D / 64];  // V rows 4lq + r, dims 64b + 4li .. + 4
};

template <int B, int D>
struct F32Rows {
  const DecodeArgs& a;
  const JobView& v;
  int32_t tb0, tb1, e0;
  const float* kbase;
  const float* vbase;
  const float* fill_k;  // finite row for tokens past the context (and the appended token's K)
  const float* fill_v;
  bool fused;
  int li, lq;

  // Row pointer (pool slot, the new row, or the fill row) of token `tok`.
  __device__ __forceinline__ const float* row(const float* base, const float* fill, int32_t tok, int32_t entry) const {
    if (tok >= v.L || (fused && tok == v.L - 1)) return fill;
    const int32_t p = clamp_block(entry, a.num_blocks);
    const int64_t slot = (int64_t)p * B + tok % B;
    return base + slot * ((int64_t)a.num_kv_heads * D);
  }

  // Rows of tile t of the job; t < 0 (a filler past the job's last tile)
  // reads only the fill rows, which stay in the caches.
  __device__ __forceinline__ void load(int32_t t, F32Tile<D>& T) const {
    const int32_t tok0 = t < 0 ? v.L : kTile * (v.t0 + t);
    const int32_t first = (kTile * v.t0) / B;
    // K: row li.
    {
      const int32_t tok = tok0 + li;
      const int32_t e = min(max(tok / B - first, 0), 127);
      const float* r = row(kbase, fill_k, tok, window_entry(tb0, tb1, e));
#pragma unroll
      for (int m = 0; m < D / 16; ++m)
        T.k[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(r + 16 * m + 4 * lq));
    }
    // V: rows 4lq + r (one block for all four when B >= 4).
    int32_t entry = 0;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int32_t tok = tok0 + 4 * lq + rr;
      if (rr == 0 || B < 4) entry = window_entry(tb0, tb1, min(max(tok / B - first, 0), 127));
      const float* r = row(vbase, fill_v, tok, entry);
#pragma unroll
      for (int b = 0; b < D / 64; ++b)
        T.v[rr][b] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(r + 64 * b + 4 * li));
    }
  }
};

template <int D>
struct F32State {
  f32x4_t o[4 * (D / 64)];  // instance (b, c) at 4b + c: rows 4lq + r = dims 64b + 4(4lq + r) + c
  float m, l;
};

template <int D>
__device__ __forceinline__ void compute_f32_tile(const DecodeArgs& a, const JobView& v, int32_t t, int li, int lq,
                                                 const f32x4_t (&qf)[D / 16], const F32Tile<D>& T, F32State<D>& st) {
  const int32_t tok0 = kTile * (v.t0 + t);
  f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < D / 16; ++m)
#pragma unroll
    for (int c = 0; c < 4; ++c) s = __builtin_amdgcn_mfma_f32_16x16x4f32(T.k[m][c], qf[m][c], s, 0, 0, 0);
  float x[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) x[r] = tok0 + 4 * lq + r < v.L ? s[r] * a.scale_log2e : -INFINITY;
  const float mx = col_max(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
  if (__builtin_amdgcn_ballot_w64(mx > st.m) != 0) {
    const float m_new = fmaxf(st.m, mx);
    const float alpha = fast_exp2(st.m - m_new);
    st.l *= alpha;
#pragma unroll
    for (int i = 0; i < 4 * (D / 64); ++i) st.o[i] *= alpha;
    st.m = m_new;
  }
  float p[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) p[r] = fast_exp2(x[r] - st.m);
  st.l += (p[0] + p[1]) + (p[2] + p[3]);
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int b = 0; b < D / 64; ++b)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        st.o[4 * b + c] = __builtin_amdgcn_mfma_f32_16x16x4f32(T.v[r][b][c], p[r], st.o[4 * b + c], 0, 0, 0);
}

template <int B, int D>
__global__ __launch_bounds__(kNW * 64, 2) void decode_f32_kernel(DecodeArgs a) {
  static_assert(D == 64 || D == 128, "head_dim");
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: keeps job fields in SGPRs
  const int li = lane & 15, lq = lane >> 4;
  const int G = a.group;
  for (int32_t k = 0; k < a.jobs_per_workgroup; ++k) {
    const pa_decode_job jd = load_job(a.jobs, (int64_t)k * a.num_workgroups + blockIdx.x);
    if (jd.tile_count <= 0) break;
    JobView v;
    view_job(a, jd, w, B, v);
    if (v.idle || v.rec == -2 || v.L <= 0) continue;
    const int32_t len_dev = as_const(a.lens)[v.seq];
    // Query, B operand: column li is head min(li, G - 1) of the KV head
    // (columns past G repeat the last one and are not written).
    const float* qrow =
        reinterpret_cast<const float*>(a.q) + ((int64_t)v.seq * a.num_q_heads + (int64_t)v.g * G + min(li, G - 1)) * D;
    f32x4_t qf[D / 16];
#pragma unroll
    for (int m = 0; m < D / 16; ++m) qf[m] = *reinterpret_cast<const f32x4_t*>(qrow + 16 * m + 4 * lq);
    // Table window: entries of the job's tokens; those past the context's
    // last entry are replaced by it (never past ceil(L / B)).
    const int32_t* trow = a.tables + (int64_t)v.seq * a.max_blocks;
    const int32_t last_e = (v.L - 1) / B;
    const int32_t e0 = (kTile * v.t0) / B;
    F32Rows<B, D> rows{a, v, trow[min(e0 + lane, last_e)], trow[min(e0 + 64 + lane, last_e)], e0,
                       reinterpret_cast<const float*>(a.k) + (int64_t)v.g * D,
                       reinterpret_cast<const float*>(a.v) + (int64_t)v.g * D, qrow, qrow, a.new_k != nullptr, li, lq};
    if (a.new_k != nullptr) {
      const int64_t nrow = ((int64_t)v.seq * a.num_kv_heads + v.g) * D;
      rows.fill_k = reinterpret_cast<const float*>(a.new_k) + nrow;
      rows.fill_v = reinterpret_cast<const float*>(a.new_v) + nrow;
    }
    F32State<D> st;
    st.m = -INFINITY;
    st.l = 0.f;
#pragma unroll
    for (int i = 0; i < 4 * (D / 64); ++i) st.o[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // Two register slots, the loop unrolled over them so that a fresh load
    // never has to be moved between registers.  The load past the job's last
    // tile is a filler that reads the fill rows only.
    F32Tile<D> ta, tb;
    const int32_t cnt = v.cnt;
    rows.load(0, ta);
    for (int32_t t = 0; t < cnt; t += 2) {
      rows.load(t + 1 < cnt ? t + 1 : -1, tb);
      compute_f32_tile<D>(a, v, t, li, lq, qf, ta, st);
      if (t + 1 >= cnt) break;
      rows.load(t + 2 < cnt ? t + 2 : -1, ta);
      compute_f32_tile<D>(a, v, t + 1, li, lq, qf, tb, st);
    }
    float lt = col_sum(st.l);
    if (len_dev != v.L) lt = NAN;  // planned for another length: never plausible numbers
    if (li >= G) continue;
    if (v.rec < 0) {
      const float inv = recip_sum(lt);
      const int64_t base = ((int64_t)v.seq * a.num_q_heads + (int64_t)v.g * G + li) * D;
#pragma unroll
      for (int b = 0; b < D / 64; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          store4(a, base + 64 * b + 16 * lq + 4 * r, st.o[4 * b + 0][r] * inv, st.o[4 * b + 1][r] * inv,
                 st.o[4 * b + 2][r] * inv, st.o[4 * b + 3][r] * inv);
    } else {
      const int64_t rec = (int64_t)v.rec * G + li;
      float* po = a.partial_o + rec * D;
#pragma unroll
      for (int b = 0; b < D / 64; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          *reinterpret_cast<float4*>(po + 64 * b + 16 * lq + 4 * r) =
              make_float4(st.o[4 * b + 0][r], st.o[4 * b + 1][r], st.o[4 * b + 2][r], st.o[4 * b + 3][r]);
      if (lq == 0) *reinterpret_cast<float2*>(a.partial_ml + 2 * rec) = make_float2(st.m, lt);
    }
  }
}

}  // namespace

hipError_t launch_decode_attention_f32(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)a.num_workgroups), block(kNW * 64);
#define PA_F32_CASE(BS, DD)                                                         \
  if (a.block_size == BS && a.head_dim == DD) {                                     \
    hipLaunchKernelGGL((decode_f32_kernel<BS, DD>), grid, block, 0, stream, a);     \
    return hipGetLastError();                                                       \
  }
  PA_F32_CASE(1, 64)
  PA_F32_CASE(2, 64)
  PA_F32_CASE(4, 64)
  PA_F32_CASE(8, 64)
  PA_F32_CASE(16, 64)
  PA_F32_CASE(32, 64)
  PA_F32_CASE(1, 128)
  PA_F32_CASE(2, 128)
  PA_F32_CASE(4, 128)
  PA_F32_CASE(8, 128)
  PA_F32_CASE(16, 128)
  PA_F32_CASE(32, 128)
#undef PA_F32_CASE
  return hipErrorInvalidValue;
}

}  // namespace pagedkv
