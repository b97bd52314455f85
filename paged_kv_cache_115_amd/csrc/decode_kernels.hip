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
// Schedule.  The grid is a fixed set of persistent workgroups of four
// wavefronts.  The host plan gives every workgroup a list of jobs (a piece of
// one sequence's 16-token tiles, for a block of four KV heads) so that all
// workgroups carry about the same number of tiles; wavefront w of the
// workgroup handles KV head 4 * head_block + w of every job, so the four
// head slices of each slot row are read at about the same time.  A
// wavefront streams through its jobs back to back: the next job's query,
// table entries and first tile are fetched while the current job finishes,
// and within a job the next tile's K/V are in flight while the current one is
// computed.  Each wavefront keeps one online-softmax state (running max m,
// running sum l, unnormalised accumulator o) for the G query heads of its KV
// head.  A job that covers a whole sequence writes the output; a piece of a
// longer sequence writes a (m, l, o) record and merge_partials_kernel, a
// second launch, combines the records of each (sequence, KV head) in piece
// order.  Every floating-point reduction order depends only on logical token
// positions and on the plan: results are bitwise reproducible and do not
// depend on physical block ids.  Softmax runs in base 2 on scores
// pre-multiplied by log2(e).
//
// bf16 path (head_dim 128, G <= 16): both contractions run on MFMA.
//   S^T[token][head] = K_tile[16 x 128] . Q^T[128 x 16]  with
//     v_mfma_f32_16x16x32_bf16; K is the A operand (lane = token row, 16 bytes
//     = 8 dims).  K is read like V below, in whole 256-byte rows, and put into
//     that layout through the wavefront's own LDS area; Q^T is the B operand,
//     kept in registers (query heads beyond G are zero).
//   O^T[dim][head] += V^T[dims x 16 tokens] . P^T[16 tokens x 16 heads] with
//     v_mfma_f32_16x16x16_bf16.  The S^T result layout (lane holds tokens
//     4q..4q+3 of head lane%16) is exactly the B-operand layout P^T needs, so
//     probabilities never leave registers.  V is read in whole 256-byte rows:
//     the 16 lanes of group q read token 4q + r, lane i taking dims
//     8i .. 8i + 7.  Instance c of the PV product maps its row i to dim
//     8i + c, so its A operand is assembled from the loaded registers by
//     16-bit lane-local shuffles (no LDS round trip, no cross-lane transpose).
//   With this step's append fused (new_key/new_value), the tile holding
//   token L - 1 takes that row from the new arrays; the merge launch stores
//   it into its slot afterwards.
//   Probabilities are rounded to bf16 for the PV product and the running sum
//   adds the same rounded values, so numerator and denominator agree.
//   A job's block-table entries sit in one vector register (lane i: tile i)
//   and are read with readlane.
// The fp32 path is in decode_f32_kernels.hip.
#include "decode_common.h"

namespace pagedkv {
namespace {

// --------------------------------------------------------------------------
// bf16, head_dim 128: MFMA for QK^T and PV.
// --------------------------------------------------------------------------
// Addressing state of one job for one wavefront: the job fields and the
// job's block-table entries, one per lane (lane i: tile i).
template <int B>
struct JobRef {
  JobView v;
  int32_t tb0, tb1;
};

// The context length, the table entries and (load_q) the query of one job
// depend only on its record, so they are fetched together.
template <int B, bool kWide>
__device__ __forceinline__ void load_ref(const DecodeArgs& a, const pa_decode_job& jd, int w, int lane, JobRef<B>& J) {
  constexpr int kTilesPerBlock = B >= kTile ? B / kTile : 1;
  view_job<kWide>(a, jd, w, B, J.v);
  // The device length, compared with the planned one when the job is
  // written: requested here, two job boundaries before the job starts, so
  // writing a finished job waits for no load.
  J.v.L_dev = as_const(a.lens)[J.v.seq];
  // Lanes past the job's last tile read an in-row entry that is never used.
  const int32_t* trow = a.tables + (int64_t)J.v.seq * a.max_blocks;
  if (B < 8) {
    // Blocks of fewer than 8 slots: a tile spans kTile / B entries.  Lane i
    // holds entries e + i and e + 64 + i of the job's first entry e, a window
    // of 128 entries = 8 * B tiles; plans for such pools keep every job
    // within it (pa_decode checks).  Entries past the context are loaded
    // with the window but never used.
    const int32_t e = J.v.t0 * (kTile / B) + lane;
    J.tb0 = trow[min(max(e, 0), a.max_blocks - 1)];
    J.tb1 = trow[min(max(e + 64, 0), a.max_blocks - 1)];
  } else {
    const int32_t t = J.v.t0 + lane;
    int32_t e0 = B == 8 ? 2 * t : t / kTilesPerBlock;
    e0 = min(max(e0, 0), a.max_blocks - 1);
    // Raw entries: they are range-checked when used (after readlane), so
    // nothing waits for this load before the job's first tile is issued.
    J.tb0 = trow[e0];
    J.tb1 = B == 8 ? trow[min(e0 + 1, a.max_blocks - 1)] : 0;
  }
}


// Q^T fragments: lane holds Q[column li][32*ks + 8*lq .. +8].  Column li is
// query head li of the job's KV head (li < G), or, for a shared job, head
// li % G of member li / G.  Columns past the last live one repeat it: every
// column's softmax and accumulator are independent and only live columns
// are written, so the repeats cost nothing and the loaded values are not
// touched before the job's first tile.
__device__ __forceinline__ void load_q(const DecodeArgs& a, const JobView& v, int li, int lq, bf16x8_t (&qf)[4]) {
  constexpr int D = 128;
  const int G = a.group;
  const int col = min(li, v.ncol - 1);
  int32_t seq = v.seq;
  if (v.shared && !v.idle) {
    const auto* gd = as_const(reinterpret_cast<const i32x4_t*>(a.groups + v.grp));
    const i32x4_t members = gd[0 + 0];  // num_members, head_block, seq[0], seq[1]
    const i32x4_t more = gd[1];         // seq[2], seq[3], record_base[0], record_base[1]
    const int m = col / G;
    const int32_t s0 = members[2], s1 = members[3], s2 = more[0], s3 = more[1];
    seq = min(max(m == 0 ? s0 : m == 1 ? s1 : m == 2 ? s2 : s3, 0), a.num_seqs - 1);
  }
  const uint4* qrow = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.q) +
                                                     ((int64_t)seq * a.num_q_heads + (int64_t)v.g * G + col % G) * D);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const uint4 x = qrow[4 * ks + lq];
    qf[ks] = __builtin_bit_cast(bf16x8_t, x);
  }
}

// Buffer resource for `bytes` bytes at `base` (raw buffer, gfx9 dword3).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const char* base, int32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, bytes, 0x00020000);
}

// Cache policy of K/V tile loads.  When no block is shared, every byte of
// the pool is read once per call: the loads are marked non-temporal (nt) and
// skip the wavefront's L1 (sc0), which measured +7..11% read bandwidth on
// MI355X.  When sequences share blocks (forked prefixes), the same block is
// read by several wavefronts and default caching keeps it for the others.
template <bool kStream>
__device__ __forceinline__ uint4 load_b128(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  constexpr int kPolicy = kStream ? (1 /* sc0 */ | 2 /* nt */) : 0;
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, kPolicy));
}

template <bool kStream>
__device__ __forceinline__ uint4 load_global(const char* p) {
  if (kStream) return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
  return *reinterpret_cast<const uint4*>(p);
}

// K and V of tile t (of the job starting at tile t0) for KV head g, whose
// raw table entries are e0 (and e1, the second block of an 8-slot-block
// tile; range-checked here): lane (li, lq) gets, of K and of V alike, rows
// 4*lq + r, dims 8*li .. 8*li + 8 (r = 0..3).  One load instruction thus
// covers four whole 256-byte rows (whole cache lines); the layout the QK^T
// product needs, K row li in lane li, is made in LDS (compute_bf16_tile).
// Loads of 16 rows x 64 bytes, that layout directly, read the same bytes at
// 0.67 of peak against 0.82 (measured on tiles of this shape).  For B >= 16 only the first
// `rows` rows are read: the tile's buffer resource covers exactly those rows,
// and a buffer load past the resource returns zeros without touching memory.
// `rows` is 0 for the unconditional filler loads past the end of the stream,
// and below 16 in the last tile of a row, so neither fetches bytes outside
// the context.  The range check covers the vector offset and the
// instruction's immediate, not the scalar offset, so every per-row offset is
// in the vector offset.
template <int B, bool kStream, int kFused>
__device__ __forceinline__ void load_bf16_tile(const DecodeArgs& a, int32_t g, int32_t t0, int32_t e0, int32_t e1,
                                               int32_t t, int32_t rows, int32_t r_new, const char* nk,
                                               const char* nv, int li, int lq, uint4 (&kf)[4], uint4 (&vf)[4]) {
  constexpr int D = 128;
  constexpr int kTilesPerBlock = B >= kTile ? B / kTile : 1;
  const uint32_t row_bytes = (uint32_t)a.num_kv_heads * D * 2;
  const int64_t blk_bytes = (int64_t)row_bytes * B;
  const char* kb = reinterpret_cast<const char*>(a.k) + (int64_t)g * D * 2;
  const char* vb = reinterpret_cast<const char*>(a.v) + (int64_t)g * D * 2;
  if (B < 8) {
    // Blocks of fewer than 8 slots: the tile's rows lie in kTile / B blocks.
    // e0 / e1 are the job's two window registers (lane i: entries i and
    // 64 + i of the job); row 4 * lq + r takes its entry from the lane that
    // holds it (one cross-lane permute per distinct block of the lane's four
    // rows: 1 at B = 4, 2 at B = 2, 4 at B = 1) and is loaded through a
    // per-lane address.  Rows past the context, and filler loads, read a
    // fixed in-bounds row instead (the new row with the append fused, else
    // the first row of q): they are masked in compute.  With the append
    // fused, rows at and after the appended one read the new row.
    constexpr int kE = kTile / B;
    const int32_t jb = t * kE;  // the tile's first entry within the job's window (wave-uniform, < 128)
    const int32_t win = jb < 64 ? e0 : e1;
    const int32_t valid = min(rows, kTile);
    const int32_t first_new = kFused != 0 ? (r_new >= 0 ? r_new : rows <= 0 ? 0 : kTile) : kTile;
    const char* fk = kFused != 0 ? nk : reinterpret_cast<const char*>(a.q);
    const char* fv = kFused != 0 ? nv : reinterpret_cast<const char*>(a.q);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * lq + r;
      const int32_t p = clamp_block(__shfl(win, (jb + row / B) & 63), a.num_blocks);
      const int64_t off = (int64_t)p * blk_bytes + (int64_t)(row % B) * row_bytes + 16 * li;
      const bool pool_row = row < valid && row < first_new;
      kf[r] = load_global<kStream>(pool_row ? kb + off : fk + 16 * li);
      vf[r] = load_global<kStream>(pool_row ? vb + off : fv + 16 * li);
    }
    return;
  }
  const int32_t p0 = clamp_block(e0, a.num_blocks);
  // With the append fused (kFused 1, 2 or 4), row r_new of the tile holding
  // the appended token and the rows after it (past the context; masked in
  // compute) come from the new key/value row, the rows before it from the
  // pool, through per-lane addresses.  kFused 1 loads only that tile so, on a
  // path of its own; kFused 2 loads every tile so (a filler load, rows 0,
  // reads the new row, which stays in L2): one load path, and no wait for
  // the loads in flight where two paths would join, at the price of the
  // buffer loads' cache policy.  kFused 4 is kFused 2 with buffer loads: the
  // host found a 4 GiB window holding both the pool and the new rows, so
  // every lane's row is a 32-bit offset in one buffer resource per pool.
  const int32_t p1f = B == 8 && rows > 8 ? clamp_block(e1, a.num_blocks) : p0;
  auto row_addr = [&](const char* base, int32_t row) {
    if (B == 8) return base + (int64_t)(row < 8 ? p0 : p1f) * blk_bytes + (row & 7) * row_bytes;
    return base + (int64_t)p0 * blk_bytes + ((int64_t)((t0 + t) % kTilesPerBlock) * kTile + row) * row_bytes;
  };
  if (kFused == 4 && B >= kTile) {
    // Per-lane offsets into one buffer window per pool, which also holds the
    // new rows: buffer loads with the streaming cache policy, and 32-bit
    // lane arithmetic.  Rows before the appended one (or before `rows`) come
    // from the pool, the appended row from the new rows, and rows past the
    // context take an offset past every window: such a load returns zeros
    // and reads nothing, as in the tile resource of the unfused path.
    constexpr uint32_t kPastWindow = 0xffff0000u;  // windows are shorter (checked on the host)
    const int32_t lim = r_new >= 0 ? r_new : min(max(rows, 0), kTile);
    const uint32_t tile_rel = (uint32_t)((int64_t)g * D * 2 + (int64_t)p0 * blk_bytes +
                                         (int64_t)((t0 + t) % kTilesPerBlock) * kTile * row_bytes);
    const uint32_t new_rel = (uint32_t)(nk - reinterpret_cast<const char*>(a.new_k)) + 16 * li;
    const uint32_t lane_rel = 4 * lq * row_bytes + 16 * li;
    const __amdgpu_buffer_rsrc_t kr = tile_rsrc(reinterpret_cast<const char*>(a.k_win), (int32_t)a.k_win_bytes);
    const __amdgpu_buffer_rsrc_t vr = tile_rsrc(reinterpret_cast<const char*>(a.v_win), (int32_t)a.v_win_bytes);
    const uint32_t kt_off = a.k_off + tile_rel, vt_off = a.v_off + tile_rel;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * lq + r;
      kf[r] = load_b128<kStream>(
          kr, row < lim ? kt_off + lane_rel + r * row_bytes : row == r_new ? a.nk_off + new_rel : kPastWindow, 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * lq + r;
      vf[r] = load_b128<kStream>(
          vr, row < lim ? vt_off + lane_rel + r * row_bytes : row == r_new ? a.nv_off + new_rel : kPastWindow, 0);
    }
  } else if (kFused == 2 || (kFused == 1 && r_new >= 0)) {
    const int32_t first_new = r_new >= 0 ? r_new : rows <= 0 ? 0 : kTile;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      kf[r] = load_global<kStream>(4 * lq + r >= first_new ? nk + 16 * li : row_addr(kb, 4 * lq + r) + 16 * li);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      vf[r] = load_global<kStream>(4 * lq + r >= first_new ? nv + 16 * li : row_addr(vb, 4 * lq + r) + 16 * li);
  } else if (B == 8) {
    // Rows 0..7 of the tile live in block p0, rows 8..15 in block p1.  A
    // last tile of at most 8 rows has no second block (its table entry lies
    // past the context and is not read): those rows reload block p0 and are
    // masked in compute.
    const int32_t p1 = rows > 8 ? clamp_block(e1, a.num_blocks) : p0;
    const int64_t vblk = (int64_t)(lq < 2 ? p0 : p1) * blk_bytes;
#pragma unroll
    for (int r = 0; r < 4; ++r) kf[r] = load_global<kStream>(kb + vblk + ((4 * lq + r) & 7) * row_bytes + 16 * li);
#pragma unroll
    for (int r = 0; r < 4; ++r) vf[r] = load_global<kStream>(vb + vblk + ((4 * lq + r) & 7) * row_bytes + 16 * li);
  } else {
    // One tile = 16 consecutive slot rows of one block: a buffer resource on
    // the tile's first `rows` rows (scalar registers) plus lane offsets that
    // never change.
    // Every operand is wave-uniform by construction; readfirstlane says so to
    // the compiler, which otherwise wraps each load in a waterfall loop.
    const int64_t tile_off = (int64_t)g * D * 2 + (int64_t)p0 * blk_bytes +
                             (int64_t)((t0 + t) % kTilesPerBlock) * kTile * row_bytes;
    const uint32_t off_lo = __builtin_amdgcn_readfirstlane((uint32_t)tile_off);
    const uint32_t off_hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)tile_off >> 32));
    const int64_t uoff = (int64_t)(((uint64_t)off_hi << 32) | off_lo);
    const int32_t tile_bytes = __builtin_amdgcn_readfirstlane(min(max(rows, 0), kTile) * (int32_t)row_bytes);
    const __amdgpu_buffer_rsrc_t kr = tile_rsrc(reinterpret_cast<const char*>(a.k) + uoff, tile_bytes);
    const __amdgpu_buffer_rsrc_t vr = tile_rsrc(reinterpret_cast<const char*>(a.v) + uoff, tile_bytes);
    const uint32_t voff = 4 * lq * row_bytes + 16 * li;
#pragma unroll
    for (int r = 0; r < 4; ++r) kf[r] = load_b128<kStream>(kr, voff + r * row_bytes, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) vf[r] = load_b128<kStream>(vr, voff + r * row_bytes, 0);
  }
}

struct SoftmaxState {
  float m, l;
  float4_t o[8];
  __device__ __forceinline__ void reset() {
    m = -INFINITY;
    l = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) o[c] = float4_t{0.f, 0.f, 0.f, 0.f};
  }
};

// A plan made for other lengths than the device's context_lens (a plan kept
// from an earlier step, say) must not yield plausible numbers.  When a
// finished job is written (from the stage after the wavefront's last job, or
// directly), its planned length is compared with the sequence's device
// length; on a mismatch the job's softmax sum is written as NaN, and every
// normalisation (recip_sum) passes NaN on, so every output element of the
// sequence is NaN, whether written directly or through the merge of its
// records.  The comparison sits outside the tile loop's hot path: code in
// the loop costs registers there.
__device__ __forceinline__ float sum_or_nan(const JobView& v, float l) { return v.L_dev == v.L ? l : NAN; }

// Scores, online-softmax update and PV accumulation of the 16-token tile
// whose first token is tok0: kf holds the K operand (K row li in lane li,
// after the transposition), vf the V rows as loaded.
__device__ __forceinline__ void tile_math(const DecodeArgs& a, const JobView& v, const bf16x8_t (&qf)[4],
                                          int32_t tok0, int li, int lq, const uint4 (&kf)[4], uint4 (&vf)[4],
                                          SoftmaxState& st) {
  const bool tail = tok0 + kTile > v.L;
  if (tail) {
    // Slots past the end hold arbitrary bits; V must be exactly zero there
    // because 0 * NaN would poison the PV product.
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (tok0 + 4 * lq + r >= v.L) vf[r] = make_uint4(0, 0, 0, 0);
  }
  float4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kf[ks]), qf[ks], sacc, 0, 0, 0);
  float x[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    x[r] = sacc[r] * a.scale_log2e;
    if (tail && tok0 + 4 * lq + r >= v.L) x[r] = -INFINITY;
  }
  const float mx = col_max(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
  // The accumulators and the sum are rescaled only when some column's max
  // grows (a wave-uniform branch): past the first tiles of a long context the
  // max rarely moves.  The first tile of a job always rescales (from a max of
  // -inf, by 0).
  if (__builtin_amdgcn_ballot_w64(mx > st.m) != 0) {
    const float m_new = fmaxf(st.m, mx);
    const float alpha = fast_exp2(st.m - m_new);
    st.l *= alpha;
#pragma unroll
    for (int c = 0; c < 8; ++c) st.o[c] *= alpha;
    st.m = m_new;
  }
  const uint32_t p01 = pack_bf16x2(fast_exp2(x[0] - st.m), fast_exp2(x[1] - st.m));
  const uint32_t p23 = pack_bf16x2(fast_exp2(x[2] - st.m), fast_exp2(x[3] - st.m));
  // The sum takes the rounded probabilities, the ones the PV product uses.
  st.l += ((__uint_as_float(p01 << 16) + __uint_as_float(p01 & 0xffff0000u)) + __uint_as_float(p23 << 16)) +
          __uint_as_float(p23 & 0xffff0000u);
  const short4_t pfrag = __builtin_bit_cast(short4_t, make_uint2(p01, p23));
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    // Lane (li, lq) holds dims 8*li .. 8*li + 8 of rows 4*lq + r in vf[r];
    // instance c takes dim 8*li + c of the four rows: 16-bit halves of word
    // c / 2, gathered by byte permutes.
    const int wd = c >> 1;
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
    const uint32_t lo = __builtin_amdgcn_perm(word(vf[1], wd), word(vf[0], wd), sel);
    const uint32_t hi = __builtin_amdgcn_perm(word(vf[3], wd), word(vf[2], wd), sel);
    st.o[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(short4_t, make_uint2(lo, hi)), pfrag,
                                                        st.o[c], 0, 0, 0);
  }
}

// One 16-token tile (tile t of job v): scores, online-softmax update, PV
// accumulation.
__device__ __forceinline__ void compute_bf16_tile(const DecodeArgs& a, const JobView& v, const bf16x8_t (&qf)[4],
                                                  int32_t t, int li, int lq, uint4 (&kf)[4], uint4 (&vf)[4],
                                                  lds_char* kt, SoftmaxState& st) {
  const int32_t tok0 = kTile * (v.t0 + t);
  if (tok0 >= v.L) return;  // beyond the context (only if the plan and lengths disagree)
  // K row li into lane li, in place (the slot's registers): through the
  // wavefront's LDS area, rows padded to kKtRow bytes so that the 16 rows one
  // read pass touches fall in distinct banks.  LDS operations of a wavefront
  // complete in order, so the reads see the writes, and the next tile's
  // writes follow these reads.
#pragma unroll
  for (int r = 0; r < 4; ++r)
    *reinterpret_cast<lds_u32x4*>(kt + (4 * lq + r) * kKtRow + 16 * li) = __builtin_bit_cast(u32x4_t, kf[r]);
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    kf[ks] = __builtin_bit_cast(uint4, *reinterpret_cast<const lds_u32x4*>(kt + li * kKtRow + 16 * (4 * ks + lq)));
  tile_math(a, v, qf, tok0, li, lq, kf, vf, st);
}

// LDS stores of this wavefront complete, then the workgroup meets.  No wait
// for vector memory: the tile loads in flight stay in flight.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// The kernel for plans with wide jobs computes every position here.  A
// plain position is one tile, as in compute_bf16_tile.  A wide job's
// position covers tiles 4p .. 4p + 3 of the job, of which wavefront w loaded
// tile 4p + w (of the set's KV head, whole rows as for any tile).  Each
// wavefront stores its tile in LDS (K rows in its transposition area, V rows
// in its V area); after a barrier every wavefront scores all four tiles,
// read back in the operand layouts, against its own group of the set.  A
// second barrier keeps the next position's stores behind every wavefront's
// reads.  All four wavefronts take both barriers at every position of every
// wide job (they walk the same job list), idle ones included: those load
// and store their tiles and skip the scoring.  One loop serves both kinds of
// position (with two code paths the registers spill).
__device__ __forceinline__ void compute_position(const DecodeArgs& a, const JobView& v, const bf16x8_t (&qf)[4],
                                                 int32_t p, int w, int li, int lq, const uint4 (&kf)[4],
                                                 uint4 (&vf)[4], lds_char* kt_all, lds_char* vt_all,
                                                 SoftmaxState& st) {
  const bool wide = v.wide;
  lds_char* ktw = kt_all + w * (kTile * kKtRow);
  lds_char* vtw = vt_all + w * (kTile * kHeadDim * 2);
#pragma unroll
  for (int r = 0; r < 4; ++r)
    *reinterpret_cast<lds_u32x4*>(ktw + (4 * lq + r) * kKtRow + 16 * li) = __builtin_bit_cast(u32x4_t, kf[r]);
  if (wide) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      *reinterpret_cast<lds_u32x4*>(vtw + (4 * lq + r) * (kHeadDim * 2) + 16 * li) =
          __builtin_bit_cast(u32x4_t, vf[r]);
    lds_barrier();
  }
  const int n = wide ? kNW : 1;
#pragma unroll 1
  for (int i = 0; i < n; ++i) {
    const int j = wide ? i : w;  // whose LDS area holds the tile
    const int32_t tile = wide ? 4 * p + i : p;
    const int32_t tok0 = kTile * (v.t0 + tile);
    // Past the context only if the plan and lengths disagree.
    if ((!wide || (!v.idle && tile < v.T)) && tok0 < v.L) {
      const lds_char* ktj = kt_all + j * (kTile * kKtRow);
      const lds_char* vtj = vt_all + j * (kTile * kHeadDim * 2);
      uint4 kk[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        kk[ks] =
            __builtin_bit_cast(uint4, *reinterpret_cast<const lds_u32x4*>(ktj + li * kKtRow + 16 * (4 * ks + lq)));
      if (wide) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          vf[r] = __builtin_bit_cast(
              uint4, *reinterpret_cast<const lds_u32x4*>(vtj + (4 * lq + r) * (kHeadDim * 2) + 16 * li));
      }
      tile_math(a, v, qf, tok0, li, lq, kk, vf, st);
    }
  }
  if (wide) lds_barrier();
}

// Finished jobs are staged in LDS and written to memory after the
// wavefront's last job (once the staging area is full, later jobs are
// written directly, and the last job itself is).  On gfx9 the
// vector memory counter retires loads and stores in issue order, so a store
// issued between tile loads makes every later tile wait for the store's
// acknowledgement; staging keeps the tile stream free of stores.
//
// Per wavefront: kStageFloats floats of accumulators (an entry holds, for the
// G live columns, the 32 values of each lane (li, lq): entry float index
// ((k * 4 + lq) * G + li) * 4 + c for k = 0..7, c = 0..3, i.e. o[4 * (k & 1) + c][k >> 1]),
// then (m, l) per (entry, column), then (seq, g, record, lengths agree) per entry.
constexpr int kStageMax = 7;                      // entries per wavefront
constexpr int kStageFloats = kStageMax * 4 * 128; // accumulator floats per wavefront (G = 4 fills 7 entries)
// The kernel for plans with wide jobs also holds the V areas of a position
// (4 x 4 KB) and stages 5 entries, so that two workgroups still fit a
// compute unit's 160 KB of LDS.
constexpr int kStageMaxWide = 5;
constexpr int stage_wave_floats(int n) { return n * 4 * 128 + n * 16 * 2 + n * 4; }

struct Stage {
  float* o;      // accumulator entries
  float* ml;     // [entry][16][2]
  int32_t* meta; // [entry][4]
  int n, cap;    // staged entries, capacity for this G
};

// Write staged entries to out / the workspace records, then empty the stage.
__device__ __forceinline__ void flush_stage(const DecodeArgs& a, Stage& sg, int li, int lq) {
  constexpr int D = 128;
  const int G = a.group;
  for (int e = 0; e < sg.n; ++e) {
    const int32_t seq = __builtin_amdgcn_readfirstlane(sg.meta[4 * e + 0]);
    const int32_t g = __builtin_amdgcn_readfirstlane(sg.meta[4 * e + 1]);
    const int32_t rec = __builtin_amdgcn_readfirstlane(sg.meta[4 * e + 2]);
    const int32_t len_ok = __builtin_amdgcn_readfirstlane(sg.meta[4 * e + 3]);
    if (li >= G || rec < -1) continue;  // -2: a shared job's member without a valid record
    const float* eo = sg.o + e * 128 * G;
    float4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = *reinterpret_cast<const float4*>(eo + ((k * 4 + lq) * G + li) * 4);
    const float m = sg.ml[(e * 16 + li) * 2];
    const float lt = len_ok ? sg.ml[(e * 16 + li) * 2 + 1] : NAN;
    if (rec < 0) {
      const float inv = recip_sum(lt);
      const int64_t base = ((int64_t)seq * a.num_q_heads + (int64_t)g * G + li) * D + 32 * lq;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        store4(a, base + 8 * r, v[2 * r].x * inv, v[2 * r].y * inv, v[2 * r].z * inv, v[2 * r].w * inv);
        store4(a, base + 8 * r + 4, v[2 * r + 1].x * inv, v[2 * r + 1].y * inv, v[2 * r + 1].z * inv,
               v[2 * r + 1].w * inv);
      }
    } else {
      const int64_t rr = (int64_t)rec * G + li;
      float* po = a.partial_o + rr * D + 32 * lq;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        *reinterpret_cast<float4*>(po + 8 * r) = v[2 * r];
        *reinterpret_cast<float4*>(po + 8 * r + 4) = v[2 * r + 1];
      }
      if (lq == 0) *reinterpret_cast<float2*>(a.partial_ml + 2 * rr) = make_float2(m, lt);
    }
  }
  sg.n = 0;
}

// End of a job: stage the output (whole sequence) or the piece's record.
// Lane (li, lq) holds, for head li, accumulator rows 4*lq + r of instance c:
// dims 32*lq + 8*r + c.  With the stage full, or for the wavefront's last job
// (`direct`: no tile load follows its stores), the job is written directly;
// staging the last job and writing it from LDS afterwards cost its wavefront
// about a microsecond at the end of the launch (batch 256, 8 KV heads:
// 38.8 -> 38.4 us).
__device__ __forceinline__ void finish_bf16_job(const DecodeArgs& a, const JobView& v, int li, int lq,
                                                const SoftmaxState& st, Stage& sg, bool direct) {
  constexpr int D = 128;
  const int G = a.group;
  float lt = col_sum(st.l);
  if (v.shared) {
    // Shared prefix piece: column li is head li % G of member li / G.  Each
    // member's record for this piece is staged as an entry of its own (the
    // member's G columns as the first G of the entry), or, with the stage
    // full, written directly.
    if (v.idle) return;
    const auto* gd = as_const(reinterpret_cast<const i32x4_t*>(a.groups + v.grp));
    const i32x4_t x1 = gd[1], x2 = gd[2], x3 = gd[3];  // seq[2..3] rb[0..1] | rb[2..3] np[0..1] | np[2..3] -
    const int members = v.ncol / G;
    const int m = min(li / G, members - 1);
    const int32_t rb = m == 0 ? x1[2] : m == 1 ? x1[3] : m == 2 ? x2[0] : x2[1];
    const int32_t np = m == 0 ? x2[2] : m == 1 ? x2[3] : m == 2 ? x3[0] : x3[1];
    const int64_t rec = (int64_t)rb + (int64_t)v.w * np + v.part;
    const bool valid = rb >= 0 && v.part < np && rec < a.num_records;
    if (!direct && sg.n + members <= sg.cap) {
      const int e = sg.n + m, lg = li % G;
      if (li < v.ncol) {
        float* eo = sg.o + e * 128 * G;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          *reinterpret_cast<float4*>(eo + (((2 * r) * 4 + lq) * G + lg) * 4) =
              make_float4(st.o[0][r], st.o[1][r], st.o[2][r], st.o[3][r]);
          *reinterpret_cast<float4*>(eo + (((2 * r + 1) * 4 + lq) * G + lg) * 4) =
              make_float4(st.o[4][r], st.o[5][r], st.o[6][r], st.o[7][r]);
        }
        if (lq == 0) *reinterpret_cast<float2*>(sg.ml + (e * 16 + lg) * 2) = make_float2(st.m, lt);
        if (lg == 0 && lq == 0) {
          sg.meta[4 * e + 0] = v.seq;
          sg.meta[4 * e + 1] = v.g;
          sg.meta[4 * e + 2] = valid ? (int32_t)rec : -2;
          sg.meta[4 * e + 3] = v.L_dev == v.L;
        }
      }
      sg.n += members;
      return;
    }
    if (li >= v.ncol || !valid) return;
    lt = sum_or_nan(v, lt);
    const int64_t rr = rec * G + li % G;
    float* po = a.partial_o + rr * D + 32 * lq;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      *reinterpret_cast<float4*>(po + 8 * r) = make_float4(st.o[0][r], st.o[1][r], st.o[2][r], st.o[3][r]);
      *reinterpret_cast<float4*>(po + 8 * r + 4) = make_float4(st.o[4][r], st.o[5][r], st.o[6][r], st.o[7][r]);
    }
    if (lq == 0) *reinterpret_cast<float2*>(a.partial_ml + 2 * rr) = make_float2(st.m, lt);
    return;
  }
  if (v.rec == -2) return;
  if (direct || sg.n == sg.cap) {
    if (li >= G) return;
    lt = sum_or_nan(v, lt);
    if (v.rec < 0) {
      const float inv = recip_sum(lt);
      const int64_t base = ((int64_t)v.seq * a.num_q_heads + (int64_t)v.g * G + li) * D + 32 * lq;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        store4(a, base + 8 * r, st.o[0][r] * inv, st.o[1][r] * inv, st.o[2][r] * inv, st.o[3][r] * inv);
        store4(a, base + 8 * r + 4, st.o[4][r] * inv, st.o[5][r] * inv, st.o[6][r] * inv, st.o[7][r] * inv);
      }
    } else {
      const int64_t rec = (int64_t)v.rec * G + li;
      float* po = a.partial_o + rec * D + 32 * lq;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        *reinterpret_cast<float4*>(po + 8 * r) = make_float4(st.o[0][r], st.o[1][r], st.o[2][r], st.o[3][r]);
        *reinterpret_cast<float4*>(po + 8 * r + 4) = make_float4(st.o[4][r], st.o[5][r], st.o[6][r], st.o[7][r]);
      }
      if (lq == 0) *reinterpret_cast<float2*>(a.partial_ml + 2 * rec) = make_float2(st.m, lt);
    }
    return;
  }
  const int e = sg.n;
  if (li < G) {
    float* eo = sg.o + e * 128 * G;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      *reinterpret_cast<float4*>(eo + (((2 * r) * 4 + lq) * G + li) * 4) =
          make_float4(st.o[0][r], st.o[1][r], st.o[2][r], st.o[3][r]);
      *reinterpret_cast<float4*>(eo + (((2 * r + 1) * 4 + lq) * G + li) * 4) =
          make_float4(st.o[4][r], st.o[5][r], st.o[6][r], st.o[7][r]);
    }
    if (lq == 0) *reinterpret_cast<float2*>(sg.ml + (e * 16 + li) * 2) = make_float2(st.m, lt);
  }
  if ((li | lq) == 0) {
    sg.meta[4 * e + 0] = v.seq;
    sg.meta[4 * e + 1] = v.g;
    sg.meta[4 * e + 2] = v.rec;
    sg.meta[4 * e + 3] = v.L_dev == v.L;
  }
  sg.n = e + 1;
}

template <int B, bool kStream, int kFused, bool kWide>
__global__ __launch_bounds__(kNW * 64, kWavesPerSimd) void decode_bf16_kernel(DecodeArgs a) {
  static_assert(B == 1 || B == 2 || B == 4 || B == 8 || B == 16 || B == 32, "block size");
  static_assert(kFused != 4 || B >= 16, "window loads read whole tiles of one block");
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: keeps job fields in SGPRs
  const int li = lane & 15;  // MFMA row / column within a 16-lane group
  const int lq = lane >> 4;  // which 16-lane group
  constexpr int kSM = kWide ? kStageMaxWide : kStageMax;
  constexpr int kSWF = stage_wave_floats(kSM);
  __shared__ float stage_lds[kNW * kSWF];
  __shared__ __attribute__((aligned(16))) char kt_lds[kNW * kTile * kKtRow];
  // V areas of a wide job's position (one byte when the kernel has no wide jobs).
  __shared__ __attribute__((aligned(16))) char vt_lds[kWide ? kNW * kTile * kHeadDim * 2 : 1];
  lds_char* kt = (lds_char*)(kt_lds + w * kTile * kKtRow);
  Stage sg;
  sg.o = stage_lds + w * kSWF;
  sg.ml = sg.o + kSM * 4 * 128;
  sg.meta = reinterpret_cast<int32_t*>(sg.ml + kSM * 16 * 2);
  sg.n = 0;
  sg.cap = min(kSM, kSM * 4 * 128 / (128 * a.group));
  // The workgroup's jobs are the slots k = 0, 1, ... of its column of the
  // job table (entry k * num_workgroups + blockIdx.x); an empty slot
  // (tile_count 0) ends the column.
  // Start-up is a chain of round trips: kernel arguments, job records (and
  // first-tile entries), then the first tile loads.  Each link is one batch:
  // the argument lines holding what the start-up needs (the job table and
  // its shape, the first-tile entries, tables, lengths, q and the pools; see
  // DecodeArgs) are requested together here, and every record the prologue
  // needs is requested before the first of them is waited for.
  // Without the pins the compiler requests argument fields and records one
  // at a time as they are used, each behind a wait for all scalar loads.
  {
    const uint64_t line0 = reinterpret_cast<uint64_t>(a.jobs);
    const uint64_t line0b = reinterpret_cast<uint64_t>(a.k);
    const int32_t line1 = a.num_workgroups, line1b = a.jobs_per_workgroup;
    asm volatile("" ::"s"(line0), "s"(line0b), "s"(line1), "s"(line1b));
  }
  const int32_t jend = a.jobs_per_workgroup;
  if (jend <= 0) return;
  auto record = [&](int32_t k) { return load_job(a.jobs, (int64_t)min(k, jend - 1) * a.num_workgroups + blockIdx.x); };
  // Job lookahead.  cur, nxt and nx2 hold job fields, table entries and
  // lengths; r3 is the raw record of slot s3, the one after nx2, requested a
  // whole job before its fields are needed.  No decision waits on a load
  // issued at the same job boundary: at a boundary the wavefront only
  // consumes r3 (which has long arrived) and requests the next record.
  // The first four records are requested together.
  const pa_decode_job r0 = record(0), r1 = record(1), r2 = record(2);
  pa_decode_job r3 = record(3);
  // First-tile table entries of the first two jobs (when the plan has them;
  // otherwise the same slots of the job table are read and unused): the
  // kDepth = 2 positions issued before the stream starts are tiles 0 and 1
  // of the first job, or tile 0 of each of the first two.
  const auto* fb = as_const(reinterpret_cast<const i32x4_t*>(
      a.first_blocks != nullptr ? a.first_blocks : reinterpret_cast<const int32_t*>(a.jobs)));
  auto first_ids = [&](int32_t k) { return fb[(int64_t)min(k, jend - 1) * a.num_workgroups + blockIdx.x]; };
  static_assert(kDepth == 2, "the first-tile entries cover two positions");
  const i32x4_t f0 = first_ids(0), f1 = first_ids(1);
  asm volatile("" ::"s"(r0.tile_count), "s"(r1.tile_count), "s"(r2.tile_count), "s"(r3.tile_count), "s"(f0),
               "s"(f1));
  int32_t s3 = 3;
  if (r0.tile_count <= 0) return;
  bool hn = jend > 1 && r1.tile_count > 0;
  bool hn2 = hn && jend > 2 && r2.tile_count > 0;

  // The wavefront's tiles form one stream.  Position x is tile x - x0 of the
  // current job (x0 = its first position); the positions past it belong to
  // the next job and the one after.  kDepth + 1 register slots hold
  // positions x .. x + kDepth: while tile x is computed the loads of the next
  // kDepth are in flight.  Every load is issued unconditionally (a position
  // past the end of the stream, or past the jobs known so far, reloads the
  // current job's last tile without fetching anything), so the waits the
  // compiler inserts count exactly the loads in flight.
  JobRef<B> cur, nxt, nx2;
  load_ref<B, kWide>(a, r0, w, lane, cur);
  view_job<kWide>(a, r1, w, B, nxt.v);
  nxt.tb0 = nxt.tb1 = 0;
  // The third job's table entries and the second job's query, and with the
  // plan's first-tile entries the second job's table entries too, are
  // requested after the first two positions (below): the vector memory
  // counter retires loads in issue order, so the first tile's wait would
  // otherwise also wait for them.  The first two positions never reach the
  // third job, and with first-tile entries they read no table.
  view_job<kWide>(a, r2, w, B, nx2.v);
  nx2.tb0 = nx2.tb1 = 0;
  bf16x8_t qc[4], qn[4];
  load_q(a, cur.v, li, lq, qc);
  SoftmaxState st;
  st.reset();
  int32_t x = 0, x0 = 0;
  constexpr int kSlots = kDepth + 1;
  uint4 kf[kSlots][4], vf[kSlots][4];

  // Issue the loads of stream position pos into (ks, vs).  Table entries come
  // from the jobs' table registers, or, with `first` (the positions issued
  // before the stream starts), from the plan's first-tile entries f0, f1 of
  // cur and nxt: scalar values that arrive with the job records, so the
  // first tiles do not wait for the table loads.
  auto issue_at = [&](int32_t pos, uint4 (&ks)[4], uint4 (&vs)[4], bool first, const i32x4_t& f0,
                      const i32x4_t& f1) {
    const int32_t r = pos - x0;
    const int32_t rn = r - cur.v.cnt;
    const int32_t rn2 = rn - nxt.v.cnt;
    const bool in_c = r < cur.v.cnt;
    const bool in_n = !in_c && hn && rn < nxt.v.cnt;
    const bool in_n2 = !in_c && !in_n && hn && hn2 && rn2 < nx2.v.cnt;
    const int32_t tp = in_c ? r : in_n ? rn : in_n2 ? rn2 : cur.v.cnt - 1;
    // A wide job's position covers four tiles; this wavefront loads tile 4 * tp + w.
    const bool wide = kWide && (in_n ? nxt.v.wide : in_n2 ? nx2.v.wide : cur.v.wide);
    const int32_t t = wide ? 4 * tp + w : tp;
    const int32_t g = in_n ? nxt.v.g : in_n2 ? nx2.v.g : cur.v.g;
    const int32_t t0 = in_n ? nxt.v.t0 : in_n2 ? nx2.v.t0 : cur.v.t0;
    int32_t e0, e1;
    if (B < 8) {
      // The job's whole window registers (per lane); see load_bf16_tile.
      e0 = in_n ? nxt.tb0 : in_n2 ? nx2.tb0 : cur.tb0;
      e1 = in_n ? nxt.tb1 : in_n2 ? nx2.tb1 : cur.tb1;
    } else if (first) {
      const i32x4_t f = in_n ? f1 : f0;
      e0 = t <= 0 ? f[0] : f[1];
      e1 = t <= 0 ? f[2] : f[3];
    } else {
      const int32_t tb0 = in_n ? nxt.tb0 : in_n2 ? nx2.tb0 : cur.tb0;
      const int32_t tb1 = in_n ? nxt.tb1 : in_n2 ? nx2.tb1 : cur.tb1;
      e0 = __builtin_amdgcn_readlane(tb0, t);
      e1 = B == 8 ? __builtin_amdgcn_readlane(tb1, t) : 0;
    }
    const int32_t L = in_n ? nxt.v.L : in_n2 ? nx2.v.L : cur.v.L;
    const bool idle = in_n ? nxt.v.idle : in_n2 ? nx2.v.idle : cur.v.idle;
    // Wide jobs: every wavefront loads its tile (the others score it), and
    // the tiles of the last position past the job read nothing.
    const int32_t T = in_n ? nxt.v.T : in_n2 ? nx2.v.T : cur.v.T;
    const bool live = (in_c || in_n || in_n2) && (wide ? t < T : !idle);
    const int32_t rows = live ? L - kTile * (t0 + t) : 0;
    // Row of this step's appended token in the tile, when the append is fused
    // into this launch and the tile holds it.
    const int32_t r_new = (kFused != 0 && live && rows >= 1 && rows <= kTile) ? rows - 1 : -1;
    const int32_t seq = in_n ? nxt.v.seq : in_n2 ? nx2.v.seq : cur.v.seq;
    const int64_t new_row = ((int64_t)seq * a.num_kv_heads + g) * kHeadDim * 2;
    const char* nk = reinterpret_cast<const char*>(a.new_k) + new_row;
    const char* nv = reinterpret_cast<const char*>(a.new_v) + new_row;
    load_bf16_tile<B, kStream, kFused>(a, g, t0, e0, e1, t, rows, r_new, nk, nv, li, lq, ks, vs);
  };
  const i32x4_t none = {0, 0, 0, 0};
  auto issue = [&](int32_t pos, uint4 (&ks)[4], uint4 (&vs)[4]) { issue_at(pos, ks, vs, false, none, none); };
  // Compute position x from slot (ks, vs) after issuing position x + kDepth
  // into slot (kp, vp); false when the stream is done.
  auto step = [&](uint4 (&ks)[4], uint4 (&vs)[4], uint4 (&kp)[4], uint4 (&vp)[4]) {
    issue(x + kDepth, kp, vp);
    if (kWide)
      compute_position(a, cur.v, qc, x - x0, w, li, lq, ks, vs, (lds_char*)kt_lds, (lds_char*)vt_lds, st);
    else
      compute_bf16_tile(a, cur.v, qc, x - x0, li, lq, ks, vs, kt, st);
    ++x;
    if (x - x0 < cur.v.cnt) return true;
    finish_bf16_job(a, cur.v, li, lq, st, sg, !hn);
    if (!hn) return false;
    x0 += cur.v.cnt;
    cur = nxt;
    nxt = nx2;
    // The shifted registers are real copies (an asm move is never folded into
    // renaming), so the fresh loads below write the loop-carried registers
    // themselves.  With plain assignments the shifted values kept their
    // registers under new names, the fresh loads landed in temporaries and
    // the moves into the loop-carried registers waited for every load in
    // flight (measured without the append fused: long contexts, batch 16,
    // 275 -> 264 us; forked prefixes, 32 prompts x 4 samples, 73.5 -> 70.5 us).
    asm volatile("v_mov_b32 %0, %1" : "=v"(cur.tb0) : "v"(cur.tb0));
    asm volatile("v_mov_b32 %0, %1" : "=v"(nxt.tb0) : "v"(nxt.tb0));
    if (B <= 8) {
      asm volatile("v_mov_b32 %0, %1" : "=v"(cur.tb1) : "v"(cur.tb1));
      asm volatile("v_mov_b32 %0, %1" : "=v"(nxt.tb1) : "v"(nxt.tb1));
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      u32x4_t q = __builtin_bit_cast(u32x4_t, qn[k]);
#pragma unroll
      for (int i = 0; i < 4; ++i) asm volatile("v_mov_b32 %0, %1" : "=v"(q[i]) : "v"(q[i]));
      qc[k] = __builtin_bit_cast(bf16x8_t, q);
    }
    hn = hn2;
    // nx2 becomes the job of record r3 (requested one job ago); then the
    // record after it is requested.  Past the column (or at an empty slot)
    // the fields are in-range copies that are never used.
    hn2 = hn && s3 < jend && r3.tile_count > 0;
    load_ref<B, kWide>(a, r3, w, lane, nx2);
    ++s3;
    // The query of the next job first: a shared job reads its group
    // descriptor with a scalar load, and the wait for it would otherwise also
    // wait for the record requested below.
    load_q(a, nxt.v, li, lq, qn);
    r3 = record(s3);
    st.reset();
    return true;
  };
  // The first-tile entries name tiles 0 and 1 of a job; a wide job's first
  // positions need tiles w and 4 + w, so the kernel for wide plans reads the
  // table entries.
  if (B >= 8 && !kWide && a.first_blocks != nullptr) {
#pragma unroll
    for (int u = 0; u < kDepth; ++u) issue_at(u, kf[u], vf[u], true, f0, f1);
    load_ref<B, kWide>(a, r1, w, lane, nxt);
  } else {
    load_ref<B, kWide>(a, r1, w, lane, nxt);
#pragma unroll
    for (int u = 0; u < kDepth; ++u) issue(u, kf[u], vf[u]);
  }
  load_ref<B, kWide>(a, r2, w, lane, nx2);
  load_q(a, nxt.v, li, lq, qn);
  // The slot ring, unrolled so that every slot index is a constant and the
  // slots stay in registers.
  while (true) {
#pragma unroll
    for (int u = 0; u < kSlots; ++u)
      if (!step(kf[u], vf[u], kf[(u + kDepth) % kSlots], vf[(u + kDepth) % kSlots])) goto done;
  }
done:
  flush_stage(a, sg, li, lq);
}

// --------------------------------------------------------------------------
// Merge: for every (sequence, KV head) cut into pieces, combine the piece
// records in piece order,
//   M = max_p m_p,  out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p.
// One workgroup per row with G * D / 2 threads: thread t owns the two
// adjacent outputs 2t, 2t + 1 (head 2t / D).  Pieces are taken in batches,
// all loads of a batch issued together, and the running numerator and
// denominator are rescaled when a later group raises the maximum.  An empty
// sequence (num_parts == 0) gets zeros.
// --------------------------------------------------------------------------
__device__ __forceinline__ void store2(const DecodeArgs& a, int64_t idx, float x0, float x1) {
  if (a.out_bf16)
    *reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(a.out) + idx) = bf16_rne(x0) | (bf16_rne(x1) << 16);
  else
    *reinterpret_cast<float2*>(reinterpret_cast<float*>(a.out) + idx) = make_float2(x0, x1);
}

// The appended rows of a launch with a fused append: the attention launch
// took token L - 1 of every sequence from new_key/new_value; workgroup
// num_merges + s of the merge launch writes sequence s's row (all KV heads,
// K and V) into the slot of position L - 1 of its table.  After the
// attention launch, so no tile load of the same step can see the store.
__device__ __forceinline__ void append_rows(const DecodeArgs& a, int32_t s) {
  if (s >= a.num_seqs) return;
  const int32_t L = a.lens[s];
  if (L <= 0 || L > a.max_blocks * a.block_size) return;
  const int32_t t = L - 1;
  const int32_t p = clamp_block(a.tables[(int64_t)s * a.max_blocks + t / a.block_size], a.num_blocks);
  const int32_t row_vec = a.num_kv_heads * a.head_dim * (a.bf16 ? 2 : 4) / 16;
  const int64_t slot = (int64_t)p * a.block_size + t % a.block_size;
  const uint4* nk = reinterpret_cast<const uint4*>(a.new_k) + (int64_t)s * row_vec;
  const uint4* nv = reinterpret_cast<const uint4*>(a.new_v) + (int64_t)s * row_vec;
  uint4* kd = reinterpret_cast<uint4*>(const_cast<void*>(a.k)) + slot * row_vec;
  uint4* vd = reinterpret_cast<uint4*>(const_cast<void*>(a.v)) + slot * row_vec;
  for (int32_t c = threadIdx.x; c < 2 * row_vec; c += blockDim.x) {
    if (c < row_vec)
      kd[c] = nk[c];
    else
      vd[c - row_vec] = nv[c - row_vec];
  }
}

// Outputs e, e + 1 of head h (dims d, d + 1) of one cut row: its np records
// from record_base, kBatch per round trip (one round trip when np <= kBatch).
// head_dim 64 (fp32 pools).
template <int D, int kBatch>
__device__ __forceinline__ float2 merge_pair(const DecodeArgs& a, int32_t record_base, int np, int h, int d) {
  const int G = a.group;
  const float2* ml_all = reinterpret_cast<const float2*>(a.partial_ml);
  float M = -INFINITY, n0 = 0.f, n1 = 0.f, den = 0.f;
  for (int p0 = 0; p0 < np; p0 += kBatch) {
    float2 ml[kBatch], ov[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      // Past the last piece, reload the last one (same cache line) so every
      // load is issued unconditionally; the values are not used.
      const int64_t rec = (int64_t)(record_base + min(p0 + i, np - 1)) * G + h;
      ml[i] = ml_all[rec];
      ov[i] = *reinterpret_cast<const float2*>(a.partial_o + rec * D + d);
    }
    float mc = M;
#pragma unroll
    for (int i = 0; i < kBatch; ++i)
      if (p0 + i < np) mc = fmaxf(mc, ml[i].x);
    if (mc == -INFINITY) continue;
    const float r = fast_exp2(M - mc);  // 0 while M is still -inf
    n0 *= r;
    n1 *= r;
    den *= r;
    M = mc;
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (p0 + i < np) {
        const float f = fast_exp2(ml[i].x - M);
        den += f * ml[i].y;
        n0 += f * ov[i].x;
        n1 += f * ov[i].y;
      }
    }
  }
  const float inv = recip_sum(den);
  return make_float2(n0 * inv, n1 * inv);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// The same for head_dim 128, where a wavefront's 64 threads cover one head:
// lane i holds the (max, sum) of piece p0 + i, so a batch costs every lane one
// (max, sum) load and kBatch accumulator loads; the batch maximum and the
// denominator are wavefront reductions and piece i's weight is read from
// lane i.
template <int kBatch>
__device__ __forceinline__ float2 merge_pair_wave(const DecodeArgs& a, int32_t record_base, int np, int h, int d,
                                                  int lane) {
  constexpr int D = 128;
  static_assert(kBatch <= 64, "one piece per lane");
  const int G = a.group;
  h = __builtin_amdgcn_readfirstlane(h);
  const float2* ml_all = reinterpret_cast<const float2*>(a.partial_ml);
  float M = -INFINITY, n0 = 0.f, n1 = 0.f, den = 0.f;
  for (int p0 = 0; p0 < np; p0 += kBatch) {
    const int pl = min(p0 + min(lane, kBatch - 1), np - 1);
    const float2 ml = ml_all[(int64_t)(record_base + pl) * G + h];
    float2 ov[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int64_t rec = (int64_t)(record_base + min(p0 + i, np - 1)) * G + h;
      ov[i] = *reinterpret_cast<const float2*>(a.partial_o + rec * D + d);
    }
    const bool live = lane < kBatch && p0 + lane < np;
    const float mc = fmaxf(M, wave_max(live ? ml.x : -INFINITY));
    if (mc == -INFINITY) continue;
    const float r = fast_exp2(M - mc);  // 0 while M is still -inf
    n0 *= r;
    n1 *= r;
    den *= r;
    M = mc;
    const float f = live ? fast_exp2(ml.x - M) : 0.f;
    den += wave_sum(f * ml.y);
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (p0 + i < np) {
        const float fi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), i));
        n0 += fi * ov[i].x;
        n1 += fi * ov[i].y;
      }
    }
  }
  const float inv = recip_sum(den);
  return make_float2(n0 * inv, n1 * inv);
}

// The batch follows the row: 4 pieces for short rows (most of them), 16 or
// kMaxBatch for longer ones, so that a row of up to kMaxBatch pieces takes one
// round trip without every thread of a short row issuing kMaxBatch loads.
template <int D, int kMaxBatch>
__global__ __launch_bounds__(kMaxMergeThreads) void merge_partials_kernel(DecodeArgs a) {
  if ((int32_t)blockIdx.x >= a.num_merges) {
    append_rows(a, (int32_t)blockIdx.x - a.num_merges);
    return;
  }
  const i32x4_t mv = as_const(reinterpret_cast<const i32x4_t*>(a.merges))[blockIdx.x];
  const pa_decode_merge mg{mv[0], mv[1], mv[2], mv[3]};
  if (mg.seq < 0 || mg.seq >= a.num_seqs || mg.kv_head < 0 || mg.kv_head >= a.num_kv_heads) return;
  const int G = a.group;
  const int e = 2 * (int)threadIdx.x;
  if (e >= G * D) return;
  const int h = e / D;
  const int d = e - h * D;
  const int64_t out_idx = ((int64_t)mg.seq * a.num_q_heads + (int64_t)mg.kv_head * G) * D + e;
  const int np = mg.num_parts;
  if (np <= 0) {
    // Planned as empty: zeros, or NaN when the device length says otherwise.
    const float z = a.lens[mg.seq] == 0 ? 0.f : NAN;
    store2(a, out_idx, z, z);
    return;
  }
  if (mg.record_base < 0 || (int64_t)mg.record_base + np > a.num_records) return;
  float2 r;
  if (D == 128) {
    const int lane = threadIdx.x & 63;
    if (np <= 4)
      r = merge_pair_wave<4>(a, mg.record_base, np, h, d, lane);
    else if (np <= 16)
      r = merge_pair_wave<16>(a, mg.record_base, np, h, d, lane);
    else
      r = merge_pair_wave<kMaxBatch>(a, mg.record_base, np, h, d, lane);
  } else {
    if (np <= 4)
      r = merge_pair<D, 4>(a, mg.record_base, np, h, d);
    else
      r = merge_pair<D, kMaxBatch>(a, mg.record_base, np, h, d);
  }
  store2(a, out_idx, r.x, r.y);
}

}  // namespace

hipError_t launch_decode_attention(const DecodeArgs& a, hipStream_t stream) {
  if (a.num_workgroups <= 0 || a.num_jobs <= 0) return hipSuccess;
  const dim3 grid((unsigned)a.num_workgroups);
  bool launched = false;
  if (a.bf16) {
#define PA_BF16_LAUNCH(BS, STREAM, WIDE)                                                                \
  if (a.new_k == nullptr)                                                                               \
    hipLaunchKernelGGL((decode_bf16_kernel<BS, STREAM, 0, WIDE>), grid, dim3(kNW * 64), 0, stream, a);  \
  else if (a.fused_loads == 2)                                                                          \
    hipLaunchKernelGGL((decode_bf16_kernel<BS, STREAM, 2, WIDE>), grid, dim3(kNW * 64), 0, stream, a);  \
  else if (a.fused_loads == 4 && BS >= 16)                                                              \
    hipLaunchKernelGGL((decode_bf16_kernel<(BS >= 16 ? BS : 16), STREAM, 4, WIDE>), grid, dim3(kNW * 64), 0, \
                       stream, a);                                                                      \
  else                                                                                                  \
    hipLaunchKernelGGL((decode_bf16_kernel<BS, STREAM, 1, WIDE>), grid, dim3(kNW * 64), 0, stream, a);
  // Plans with wide jobs (which read prefixes shared by several groups, so
  // their blocks are read more than once) take the kernel that reads them,
  // with caching loads.
#define PA_BF16_CASE(BS)                                                                                \
  case BS:                                                                                              \
    if (a.wide_jobs > 0) {                                                                              \
      PA_BF16_LAUNCH(BS, false, true)                                                                   \
    } else if (a.shared_kv) {                                                                           \
      PA_BF16_LAUNCH(BS, false, false)                                                                  \
    } else {                                                                                            \
      PA_BF16_LAUNCH(BS, true, false)                                                                   \
    }                                                                                                   \
    launched = true;                                                                                    \
    break;
    switch (a.block_size) {
      PA_BF16_CASE(1)
      PA_BF16_CASE(2)
      PA_BF16_CASE(4)
      PA_BF16_CASE(8)
      PA_BF16_CASE(16)
      PA_BF16_CASE(32)
      default: break;
    }
#undef PA_BF16_CASE
#undef PA_BF16_LAUNCH
  } else {
    return launch_decode_attention_f32(a, stream);
  }
  if (!launched) return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_decode_merge(const DecodeArgs& a, hipStream_t stream) {
  const int64_t blocks = (int64_t)a.num_merges + (a.new_k != nullptr ? a.num_seqs : 0);
  if (blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)blocks), block((unsigned)(a.group * a.head_dim / 2));
  if (a.head_dim == 128)
    hipLaunchKernelGGL((merge_partials_kernel<128, 32>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((merge_partials_kernel<64, 8>), grid, block, 0, stream, a);
  return hipGetLastError();
}

hipError_t decode_resident_workgroups_per_cu(int* n) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(n, decode_bf16_kernel<16, true, 0, false>, kNW * 64, 0);
}

}  // namespace pagedkv
