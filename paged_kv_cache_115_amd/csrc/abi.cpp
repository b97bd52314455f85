// C-ABI front of libpagedkv: argument validation, the host-side decode plan,
// workspace sizing and dispatch to the HIP kernels.  Nothing here touches
// device memory contents; launches go on the caller's stream and the library
// never synchronizes.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <limits>
#include <vector>

#include "internal.h"
#include "launch.h"

namespace pagedkv {

namespace {
thread_local char g_error[512] = "";
}

pa_status fail(pa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_error, sizeof(g_error), fmt, ap);
  va_end(ap);
  return st;
}

namespace {

bool aligned(const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

bool supported_block_size(int32_t b) { return b == 1 || b == 2 || b == 4 || b == 8 || b == 16 || b == 32; }

pa_status check_pool(const pa_kv_pool* pool, const char* who) {
  if (!pool) return fail(PA_ERR_INVALID, "%s: pool is NULL", who);
  if (!pool->k || !pool->v) return fail(PA_ERR_INVALID, "%s: pool k/v pointer is NULL", who);
  if (pool->dtype != PA_F32 && pool->dtype != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "%s: dtype %d (supported: 0=f32, 1=bf16)", who, pool->dtype);
  if (pool->num_blocks <= 0 || pool->num_kv_heads <= 0)
    return fail(PA_ERR_INVALID, "%s: num_blocks=%d num_kv_heads=%d must be positive", who,
                pool->num_blocks, pool->num_kv_heads);
  if (!supported_block_size(pool->block_size))
    return fail(PA_ERR_UNSUPPORTED, "%s: block_size %d (supported: 1, 2, 4, 8, 16, 32)", who, pool->block_size);
  const bool d_ok = pool->dtype == PA_F32 ? (pool->head_dim == 64 || pool->head_dim == 128)
                                          : pool->head_dim == 128;
  if (!d_ok)
    return fail(PA_ERR_UNSUPPORTED, "%s: head_dim %d with dtype %d (f32: 64 or 128; bf16: 128)", who,
                pool->head_dim, pool->dtype);
  if (!aligned(pool->k, 16) || !aligned(pool->v, 16))
    return fail(PA_ERR_INVALID, "%s: pool pointers must be 16-byte aligned", who);
  if ((int64_t)pool->num_blocks * pool->block_size > INT32_MAX * (int64_t)64)
    return fail(PA_ERR_INVALID, "%s: pool too large", who);
  return PA_OK;
}

pa_status hip_status(hipError_t e, const char* who) {
  if (e == hipSuccess) return PA_OK;
  return fail(PA_ERR_HIP, "%s: %s", who, hipGetErrorString(e));
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace carve for `heads` (record, query head) pairs: (max, sum) pairs,
// then unnormalised accumulators.
struct WorkspaceLayout {
  size_t ml, o, total;
};

WorkspaceLayout layout(int64_t heads, int64_t d) {
  WorkspaceLayout w;
  w.ml = 0;
  w.o = round_up(sizeof(float) * 2 * heads, 256);
  w.total = w.o + round_up(sizeof(float) * heads * d, 256);
  return w;
}

}  // namespace
}  // namespace pagedkv

using pagedkv::fail;

namespace pagedkv {

int64_t pool_block_bytes(const pa_kv_pool& pool) {
  return (int64_t)pool.block_size * pool.num_kv_heads * pool.head_dim * (pool.dtype == PA_F32 ? 4 : 2);
}

pa_status noalloc_check(const pa_kv_pool* pool, const pa_decode_plan_info* info, int32_t num_q_heads,
                        const char* who) {
  if (!pool || !info) return fail(PA_ERR_INVALID, "%s: pool or info is NULL", who);
  const size_t need = pa_decode_workspace_bytes(info, num_q_heads, pool->head_dim);
  if (need > (size_t)PA_NOALLOC_SCRATCH_BYTES)
    return fail(PA_ERR_INVALID, "%s: the plan needs %zu bytes of workspace, the built-in scratch holds %zu", who,
                need, (size_t)PA_NOALLOC_SCRATCH_BYTES);
  return PA_OK;
}

}  // namespace pagedkv

extern "C" const char* pa_last_error(void) { return pagedkv::g_error; }

extern "C" pa_status pa_reshape_and_cache(const pa_kv_pool* pool, const void* key, const void* value,
                                          const int64_t* slot_mapping, int32_t num_tokens, void* stream) {
  if (pa_status st = pagedkv::check_pool(pool, "pa_reshape_and_cache")) return st;
  if (num_tokens < 0) return fail(PA_ERR_INVALID, "pa_reshape_and_cache: num_tokens %d < 0", num_tokens);
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !slot_mapping)
    return fail(PA_ERR_INVALID, "pa_reshape_and_cache: NULL key/value/slot_mapping");
  if (!pagedkv::aligned(key, 16) || !pagedkv::aligned(value, 16) || !pagedkv::aligned(slot_mapping, 8))
    return fail(PA_ERR_INVALID, "pa_reshape_and_cache: key/value must be 16-byte aligned");
  return pagedkv::hip_status(pagedkv::launch_reshape_and_cache(*pool, key, value, slot_mapping, num_tokens,
                                                               (hipStream_t)stream),
                             "pa_reshape_and_cache");
}

extern "C" pa_status pa_copy_blocks(const pa_kv_pool* pool, const int32_t* pairs, int32_t num_pairs,
                                    void* stream) {
  if (pa_status st = pagedkv::check_pool(pool, "pa_copy_blocks")) return st;
  if (num_pairs < 0) return fail(PA_ERR_INVALID, "pa_copy_blocks: num_pairs %d < 0", num_pairs);
  if (num_pairs == 0) return PA_OK;
  if (!pairs) return fail(PA_ERR_INVALID, "pa_copy_blocks: pairs is NULL");
  if (num_pairs > 65535 * 1024) return fail(PA_ERR_INVALID, "pa_copy_blocks: too many pairs");
  return pagedkv::hip_status(pagedkv::launch_copy_blocks(*pool, pairs, num_pairs, (hipStream_t)stream),
                             "pa_copy_blocks");
}

namespace pagedkv {
namespace {

// The device address of [p, p + bytes) when that whole range is pinned host
// memory mapped into the device's address space; fails otherwise.  A failed
// query leaves an error in the runtime's last-error slot: it is cleared here so
// that the next launch check does not report it.
pa_status mapped_host_range(void* p, int64_t bytes, void** dev, const char* who, const char* name) {
  char* last = static_cast<char*>(p) + bytes - 1;
  hipPointerAttribute_t a0{}, a1{};
  void* d0 = nullptr;
  void* d1 = nullptr;
  const bool ok = hipPointerGetAttributes(&a0, p) == hipSuccess && a0.type == hipMemoryTypeHost &&
                  hipPointerGetAttributes(&a1, last) == hipSuccess && a1.type == hipMemoryTypeHost &&
                  hipHostGetDevicePointer(&d0, p, 0) == hipSuccess &&
                  hipHostGetDevicePointer(&d1, last, 0) == hipSuccess && d0 &&
                  static_cast<char*>(d1) - static_cast<char*>(d0) == bytes - 1;
  if (!ok) {
    (void)hipGetLastError();
    return fail(PA_ERR_INVALID,
                "%s: host_pool %s is not pinned, device-mapped host memory over all %lld bytes "
                "(allocate it with hipHostMalloc or pin_memory=True)",
                who, name, (long long)bytes);
  }
  *dev = d0;
  return PA_OK;
}

pa_status device_memory(const void* p, const char* who, const char* name) {
  hipPointerAttribute_t a{};
  if (hipPointerGetAttributes(&a, p) != hipSuccess || a.type != hipMemoryTypeDevice) {
    (void)hipGetLastError();
    return fail(PA_ERR_INVALID, "%s: device_pool %s is not device memory", who, name);
  }
  return PA_OK;
}

}  // namespace
}  // namespace pagedkv

extern "C" pa_status pa_swap_blocks(const pa_kv_pool* device_pool, const pa_kv_pool* host_pool,
                                    const int32_t* pairs, int32_t num_pairs, int32_t direction,
                                    int32_t engine, void* stream) {
  using namespace pagedkv;
  const char* who = "pa_swap_blocks";
  if (pa_status st = check_pool(device_pool, who)) return st;
  if (!host_pool || !host_pool->k || !host_pool->v) return fail(PA_ERR_INVALID, "%s: host_pool or its k/v is NULL", who);
  if (host_pool->num_blocks <= 0 || host_pool->block_size != device_pool->block_size ||
      host_pool->num_kv_heads != device_pool->num_kv_heads || host_pool->head_dim != device_pool->head_dim ||
      host_pool->dtype != device_pool->dtype)
    return fail(PA_ERR_INVALID, "%s: host_pool must have num_blocks > 0 and the device pool's block shape and dtype",
                who);
  if (!aligned(host_pool->k, 16) || !aligned(host_pool->v, 16))
    return fail(PA_ERR_INVALID, "%s: host_pool pointers must be 16-byte aligned", who);
  if (direction != PA_SWAP_OUT && direction != PA_SWAP_IN)
    return fail(PA_ERR_INVALID, "%s: direction %d (PA_SWAP_OUT=0, PA_SWAP_IN=1)", who, direction);
  if (engine != PA_SWAP_ENGINE_KERNEL && engine != PA_SWAP_ENGINE_MEMCPY)
    return fail(PA_ERR_INVALID, "%s: engine %d (PA_SWAP_ENGINE_KERNEL=0, PA_SWAP_ENGINE_MEMCPY=1)", who, engine);
  if (num_pairs < 0) return fail(PA_ERR_INVALID, "%s: num_pairs %d < 0", who, num_pairs);
  if (num_pairs == 0) return PA_OK;
  if (!pairs) return fail(PA_ERR_INVALID, "%s: pairs is NULL", who);

  const bool out = direction == PA_SWAP_OUT;
  const int32_t n_src = out ? device_pool->num_blocks : host_pool->num_blocks;
  const int32_t n_dst = out ? host_pool->num_blocks : device_pool->num_blocks;
  std::vector<char> seen(n_dst, 0);
  for (int32_t i = 0; i < num_pairs; ++i) {
    const int32_t s = pairs[2 * i], d = pairs[2 * i + 1];
    if (s < 0 || s >= n_src || d < 0 || d >= n_dst)
      return fail(PA_ERR_INVALID, "%s: pair %d = (%d, %d) outside the pools (%d source, %d destination blocks)", who,
                  i, s, d, n_src, n_dst);
    if (seen[d]) return fail(PA_ERR_INVALID, "%s: destination block %d appears twice", who, d);
    seen[d] = 1;
  }

  const int64_t block_bytes = pool_block_bytes(*device_pool);
  const int64_t host_bytes = block_bytes * host_pool->num_blocks;
  void *hk = nullptr, *hv = nullptr;
  if (pa_status st = mapped_host_range(host_pool->k, host_bytes, &hk, who, "k")) return st;
  if (pa_status st = mapped_host_range(host_pool->v, host_bytes, &hv, who, "v")) return st;
  if (pa_status st = device_memory(device_pool->k, who, "k")) return st;
  if (pa_status st = device_memory(device_pool->v, who, "v")) return st;

  const hipStream_t hs = (hipStream_t)stream;
  if (engine == PA_SWAP_ENGINE_KERNEL) {
    const void* sk = out ? device_pool->k : hk;
    const void* sv = out ? device_pool->v : hv;
    void* dk = out ? hk : device_pool->k;
    void* dv = out ? hv : device_pool->v;
    SwapBatch batch;
    for (int32_t i0 = 0; i0 < num_pairs; i0 += kSwapPairsPerLaunch) {
      const int32_t n = std::min(kSwapPairsPerLaunch, num_pairs - i0);
      for (int32_t i = 0; i < n; ++i) {
        batch.src[i] = pairs[2 * (i0 + i)];
        batch.dst[i] = pairs[2 * (i0 + i) + 1];
      }
      if (pa_status st = hip_status(launch_swap_blocks(sk, sv, dk, dv, block_bytes, batch, n, out, hs), who))
        return st;
    }
    return PA_OK;
  }
  // Runtime copies: one hipMemcpyAsync per pool for every run of pairs that continue each
  // other on both sides (src + 1, dst + 1).
  char* src_k = static_cast<char*>(out ? device_pool->k : host_pool->k);
  char* src_v = static_cast<char*>(out ? device_pool->v : host_pool->v);
  char* dst_k = static_cast<char*>(out ? host_pool->k : device_pool->k);
  char* dst_v = static_cast<char*>(out ? host_pool->v : device_pool->v);
  const hipMemcpyKind kind = out ? hipMemcpyDeviceToHost : hipMemcpyHostToDevice;
  for (int32_t i = 0; i < num_pairs;) {
    int32_t j = i + 1;
    while (j < num_pairs && pairs[2 * j] == pairs[2 * (j - 1)] + 1 && pairs[2 * j + 1] == pairs[2 * (j - 1) + 1] + 1)
      ++j;
    const int64_t so = pairs[2 * i] * block_bytes, dof = pairs[2 * i + 1] * block_bytes;
    const size_t bytes = (size_t)((j - i) * block_bytes);
    if (pa_status st = hip_status(hipMemcpyAsync(dst_k + dof, src_k + so, bytes, kind, hs), who)) return st;
    if (pa_status st = hip_status(hipMemcpyAsync(dst_v + dof, src_v + so, bytes, kind, hs), who)) return st;
    i = j;
  }
  return PA_OK;
}

extern "C" int32_t pa_decode_default_workgroups(void) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
    fail(PA_ERR_HIP, "pa_decode_default_workgroups: no device to query");
    return 0;
  }
  if (pagedkv::decode_resident_workgroups_per_cu(&per_cu) != hipSuccess || per_cu <= 0) {
    fail(PA_ERR_HIP, "pa_decode_default_workgroups: occupancy query failed");
    return 0;
  }
  return cus * per_cu;
}

namespace pagedkv {
namespace {

// One candidate schedule: jobs with their workgroup, merge rows, record count.
// A workgroup runs its jobs by rank, then in schedule order.
struct Piece {
  int32_t wg;
  pa_decode_job job;
  int32_t rank = 1;
};
struct Schedule {
  std::vector<Piece> pieces;
  std::vector<pa_decode_merge> merges;
  std::vector<pa_decode_group> groups;
  int64_t records = 0;
  int64_t nwg = 1;
  int32_t group_size = 0;
  bool reread = false;  // some block is read by more than one job (prefix plans)
  bool ranked = false;  // some piece has a rank other than 1
};

constexpr int64_t kStreamCharge = 4;   // cost units (tokens) charged per stream start by the chunk walk
// Cost of one job, in tokens, when the two schedules are compared.  A job
// boundary stalls a wavefront for about one tile, and workgroups holding
// many jobs finish last; 56 is calibrated on MI355X so that the comparison
// picks the faster schedule for the batch shapes measured (largest pieces
// for many short contexts and for lengths near a workgroup's share, chunks
// for long contexts and shared prefixes).
constexpr int64_t kJobCharge = 56;

int64_t tile_rows(int32_t L, int64_t t) { return std::min<int64_t>(16, L - 16 * t); }
// Tokens in tiles [t_begin, t_end) of a context of L tokens (every tile but
// the context's last is full).
int64_t rows_between(int32_t L, int64_t t_begin, int64_t t_end) {
  return std::min<int64_t>(L, 16 * t_end) - 16 * t_begin;
}

// A run of tiles to schedule: tiles [t_begin, t_end) of sequence `seq` for
// KV heads 4*hb .. 4*hb + 3.  A shared stream reads the prefix blocks of a
// prefix group once for all its members (`group` names its descriptor).
// The streams of one item (the head blocks of one sequence's run) are
// consecutive in the stream list and stay together in the layout.
struct Stream {
  int32_t seq, hb, t_begin, t_end, L, group, item;
};

// Equal-work chunks: the items, in alternating length order (longest,
// shortest, second longest, ...), their streams in list order, are laid end
// to end and cut into nwg
// consecutive chunks of equal cost (tokens of each tile, plus kStreamCharge at
// a stream's first tile) at tile boundaries; a tile goes to the workgroup whose
// share holds the tile's midpoint.  Consecutive tiles of one stream on one
// workgroup form jobs of at most `cap` tiles.  Returns, per stream, its
// pieces in order (indices into out.pieces) through `first`/`count`, and the
// order in which the streams were laid out.  With `base` (cost already placed
// on each of the nwg_req workgroups), the shares are not equal but fill every
// workgroup up to one common level: workgroup b's share is max(0, level -
// base[b]), with the level at which the shares add up to the streams' cost.
void chunk_streams(std::vector<Stream>& streams, int64_t nwg_req, int64_t cap, Schedule& out,
                   std::vector<int32_t>& first, std::vector<int32_t>& count, std::vector<int32_t>& order,
                   const std::vector<int64_t>* base = nullptr) {
  // Items: runs of consecutive streams with the same item id.
  std::vector<int32_t> item_first;
  for (size_t i = 0; i < streams.size(); ++i)
    if (i == 0 || streams[i].item != streams[i - 1].item) item_first.push_back((int32_t)i);
  item_first.push_back((int32_t)streams.size());
  const size_t items = item_first.size() - 1;
  auto item_len = [&](size_t it) {  // tokens of the item's first stream
    const Stream& st = streams[item_first[it]];
    return std::min(st.L, 16 * st.t_end) - 16 * st.t_begin;
  };
  std::vector<int32_t> by_len(items);
  for (size_t i = 0; i < items; ++i) by_len[i] = (int32_t)i;
  std::stable_sort(by_len.begin(), by_len.end(), [&](int32_t x, int32_t y) { return item_len(x) > item_len(y); });
  order.clear();
  order.reserve(streams.size());
  auto put = [&](int32_t it) {
    for (int32_t k = item_first[it]; k < item_first[it + 1]; ++k) order.push_back(k);
  };
  for (size_t i = 0, j = items; i < j;) {
    put(by_len[i++]);
    if (i < j) put(by_len[--j]);
  }
  int64_t total = 0, total_tiles = 0;
  for (const Stream& st : streams) {
    total += rows_between(st.L, st.t_begin, st.t_end) + kStreamCharge;
    total_tiles += st.t_end - st.t_begin;
  }
  const int64_t nwg = base ? nwg_req : std::max<int64_t>(1, std::min<int64_t>(nwg_req, total_tiles));
  out.nwg = nwg;
  first.assign(streams.size(), 0);
  count.assign(streams.size(), 0);
  out.pieces.reserve(out.pieces.size() + streams.size() + nwg);
  // Share boundaries with base loads: starts[k] = 2 * (shares of workgroups
  // below k), from the water level over the sorted loads.
  std::vector<int64_t> starts;
  if (base) {
    std::vector<int64_t> sorted(base->begin(), base->end());
    std::sort(sorted.begin(), sorted.end());
    double below = 0, level = (double)sorted[0] + (double)total;
    for (int64_t k = 0; k < nwg; ++k) {  // the level with the k + 1 lightest workgroups under it
      below += (double)sorted[k];
      const double l = ((double)total + below) / (double)(k + 1);
      if (k + 1 == nwg || l <= (double)sorted[k + 1]) {
        level = l;
        break;
      }
    }
    starts.assign(nwg + 1, 0);
    double acc = 0;
    for (int64_t b = 0; b < nwg; ++b) {
      starts[b] = (int64_t)std::ceil(2 * acc);
      acc += std::max(0.0, level - (double)(*base)[b]);
    }
    starts[nwg] = INT64_MAX;
  }
  // The tile whose midpoint m / 2 (m = 2 * cum + c) lies in share w has
  // w = floor(m * nwg / (2 * total)).  m grows from tile to tile, so w only
  // advances: it is tracked against the first m of the next share instead of
  // dividing per tile.
  int64_t cum = 0, w = 0;
  auto share_start = [&](int64_t k) {  // least m with w >= k
    return base ? starts[k] : (k * 2 * total + nwg - 1) / nwg;
  };
  int64_t next = share_start(1);
  for (int32_t si : order) {
    const Stream& st = streams[si];
    first[si] = (int32_t)out.pieces.size();
    const int64_t full_end = std::min<int64_t>(st.t_end, st.L / 16);  // tiles below this are full
    int64_t last_wg = -1;
    for (int64_t t = st.t_begin; t < st.t_end;) {
      const int64_t c = tile_rows(st.L, t) + (t == st.t_begin ? kStreamCharge : 0);
      const int64_t m = 2 * cum + c;
      while (w < nwg - 1 && m >= next) next = share_start(++w + 1);
      if (w != last_wg || out.pieces.back().job.tile_count >= cap) {
        out.pieces.push_back(Piece{(int32_t)w, pa_decode_job{st.seq, (int32_t)t, 0, st.hb, 0, 1, -1, st.L}});
        last_wg = w;
      }
      pa_decode_job& j = out.pieces.back().job;
      // A full tile past the stream's first, and the full tiles after it whose
      // midpoints stay in share w (each one's m is 32 above the previous),
      // join the job together while it has room.
      int64_t k = 1;
      if (t != st.t_begin && t < full_end) {
        k = std::min<int64_t>(full_end - t, cap - j.tile_count);
        if (w < nwg - 1) k = std::min<int64_t>(k, (next - m + 31) / 32);
      }
      j.tile_count += (int32_t)k;
      cum += c + 16 * (k - 1);
      t += k;
    }
    count[si] = (int32_t)out.pieces.size() - first[si];
  }
}

// Chunk schedule of plain (unshared) streams, one per (sequence, head
// block), in two steps: the walk places the pieces (all the cost comparison
// needs), the finish numbers the records and writes the merge rows.  Records
// are per stream: KV head 4*hb + w, piece p at record_base + w * parts + p.
struct ChunkWalk {
  std::vector<Stream> streams;
  std::vector<int32_t> first, count, order;
};
void walk_chunks(const int32_t* lens, int32_t num_seqs, int32_t num_kv_heads, int64_t nwg_req, int64_t cap,
                 Schedule& out, ChunkWalk& cw) {
  const int32_t head_blocks = (num_kv_heads + 3) / 4;
  cw.streams.reserve((size_t)num_seqs * head_blocks);
  for (int32_t s = 0; s < num_seqs; ++s)
    if (lens[s] > 0)
      for (int32_t hb = 0; hb < head_blocks; ++hb)
        cw.streams.push_back(Stream{s, hb, 0, (lens[s] + 15) / 16, lens[s], -1, s});
  chunk_streams(cw.streams, nwg_req, cap, out, cw.first, cw.count, cw.order);
}
pa_status finish_chunks(const int32_t* lens, int32_t num_seqs, int32_t num_kv_heads, const ChunkWalk& cw,
                        Schedule& out) {
  const int32_t head_blocks = (num_kv_heads + 3) / 4;
  const std::vector<Stream>& streams = cw.streams;
  const std::vector<int32_t>& first = cw.first;
  const std::vector<int32_t>& count = cw.count;
  out.merges.reserve((size_t)num_seqs * num_kv_heads);
  std::vector<int32_t> stream_of_seq(num_seqs, -1);
  for (size_t i = 0; i < streams.size(); ++i)
    if (streams[i].hb == 0) stream_of_seq[streams[i].seq] = (int32_t)i;
  for (int32_t i : cw.order) {  // records in layout order
    const int32_t parts = count[i];
    if (parts <= 1) continue;
    const int64_t heads = std::min<int64_t>(4, num_kv_heads - 4 * streams[i].hb);
    for (int32_t p = 0; p < parts; ++p) {
      pa_decode_job& j = out.pieces[first[i] + p].job;
      j.part = p;
      j.num_parts = parts;
      j.record_base = (int32_t)out.records;
    }
    out.records += (int64_t)parts * heads;
    if (out.records > INT32_MAX / 1024) return fail(PA_ERR_INVALID, "pa_decode_plan: plan too large");
  }
  // Merge rows, sequence by sequence: every KV head of an empty sequence
  // (zeros) and of every cut stream.
  for (int32_t s = 0; s < num_seqs; ++s) {
    if (lens[s] == 0) {
      for (int32_t g = 0; g < num_kv_heads; ++g) out.merges.push_back(pa_decode_merge{s, g, 0, -1});
      continue;
    }
    for (int32_t hb = 0; hb < head_blocks; ++hb) {
      const int32_t i = stream_of_seq[s] + hb;
      const pa_decode_job& j = out.pieces[first[i]].job;
      if (count[i] <= 1) continue;
      for (int32_t g = 4 * hb; g < std::min<int32_t>(num_kv_heads, 4 * hb + 4); ++g)
        out.merges.push_back(pa_decode_merge{s, g, j.num_parts, j.record_base + (g - 4 * hb) * j.num_parts});
    }
  }
  return PA_OK;
}

// Compute dies of the device: the dispatcher hands workgroup b to die
// b mod kDies, and the dies do not share their L2 caches (MI355X: 8 XCDs of
// 32 compute units, 4 MB of L2 each).
constexpr int64_t kDies = 8;
// Groups per set (one per wavefront of a workgroup; see schedule_prefix).
constexpr int32_t kSetGroups = 4;
// Cost, in tokens, of a 16-token tile of a prefix that several planned
// groups share and that is placed as below: after the first reader on a die
// the tile comes from that die's L2, not from HBM (measured on MI355X: about
// 1.0 us per tile and wavefront against 1.3 us for a tile from HBM; 12
// balanced best among 4, 8, 12 and 16 on 256 requests over four 2,000-token
// prompts, G = 4).
constexpr int64_t kWideTileCost = 12;
// The same for a set's tile of one KV head (PA_JOB_WIDE), which its four
// wavefronts score against four groups after one read: 8 balanced the same
// batch best among 3, 5, 7, 8, 9, 10 and 12 (attention launch 67.5 us at 8,
// 75.8 us at 12).
constexpr int64_t kSetTileCost = 8;

// Placement of the shared streams of wide prefixes (a key group cut into
// several planned groups, each reading the same prefix blocks) so that the
// reads of one prefix meet in one die's L2.  The streams, ordered by (key
// group, head block), are dealt to the dies at stream granularity in equal
// shares of tiles.  On a die holding m streams and n workgroups, m <= n,
// every stream is cut into the same R = floor(n / m) tile ranges (fewer if
// ranges would be shorter than 8 tiles on average), and the
// pieces, laid out set by set and range by range (range 0 of every stream
// of the set, then range 1, ...), go one per workgroup: the workgroups that
// read range r of one prefix hold it at the same time, all on one die.  (A
// die with more streams than workgroups cuts them, laid end to end, into
// equal consecutive chunks.)  The first half of a die's workgroups run their
// shared piece before their other jobs, the second half after them:
// workgroups b and b + nwg/2 share a compute unit, which then streams from
// HBM with one while it reads from L2 with the other.  Adds each workgroup's
// cost to `base`, `unit` per tile.
void place_wide(const std::vector<Stream>& streams, const std::vector<int32_t>& wide,
                const std::vector<int32_t>& set_of, int64_t nwg, int64_t cap, int64_t unit, Schedule& out,
                std::vector<int32_t>& first, std::vector<int32_t>& count, std::vector<int64_t>& base) {
  const int64_t per_die = nwg / kDies;
  int64_t total = 0;
  for (int32_t i : wide) total += streams[i].t_end - streams[i].t_begin;
  std::vector<std::vector<Piece>> own(streams.size());
  // Tiles [t0, t1) of a stream on slot c (of n) of a die.
  auto put = [&](int64_t die, int32_t si, int32_t t0, int32_t t1, int64_t c, int64_t n) {
    const Stream& st = streams[si];
    const int32_t wg = (int32_t)(die + kDies * (c * per_die / n));
    const int32_t rank = 2 * c >= n ? 2 : 0;
    std::vector<Piece>& v = own[si];
    for (int32_t t = t0; t < t1;) {
      if (v.empty() || v.back().wg != wg || v.back().job.tile_begin + v.back().job.tile_count != t ||
          v.back().job.tile_count >= cap)
        v.push_back(Piece{wg, pa_decode_job{st.seq, t, 0, st.hb, 0, 1, -1, st.L}, rank});
      const int32_t k = std::min<int32_t>(t1 - t, (int32_t)cap - v.back().job.tile_count);
      v.back().job.tile_count += k;
      base[wg] += unit * k;
      t += k;
    }
  };
  int64_t cum = 0;
  size_t k = 0;
  for (int64_t die = 0; die < kDies && k < wide.size(); ++die) {
    // This die's streams: those whose midpoint falls in its share.
    std::vector<int32_t> mine;
    int64_t tiles = 0;
    for (; k < wide.size(); ++k) {
      const int64_t t = streams[wide[k]].t_end - streams[wide[k]].t_begin;
      if (die < kDies - 1 && (2 * cum + t) * kDies >= 2 * total * (die + 1)) break;
      mine.push_back(wide[k]);
      tiles += t;
      cum += t;
    }
    const int64_t m = (int64_t)mine.size();
    if (m == 0) continue;
    if (m <= per_die) {
      // Ranges of at least 8 tiles (each piece is a job and a record per member).
      const int64_t R = std::max<int64_t>(1, std::min<int64_t>(per_die / m, tiles / m / 8)), n = m * R;
      int64_t c = 0;
      for (int64_t a = 0; a < m;) {
        int64_t e = a;
        while (e < m && set_of[mine[e]] == set_of[mine[a]]) ++e;
        for (int64_t r = 0; r < R; ++r)
          for (int64_t j = a; j < e; ++j, ++c) {
            const Stream& st = streams[mine[j]];
            const int64_t T = st.t_end - st.t_begin;
            put(die, mine[j], st.t_begin + (int32_t)(T * r / R), st.t_begin + (int32_t)(T * (r + 1) / R), c, n);
          }
        a = e;
      }
    } else {
      // Tile u of the streams laid end to end goes to chunk floor((2u + 1) n / (2 tiles)).
      int64_t u = 0;
      for (int32_t si : mine)
        for (int32_t t = streams[si].t_begin; t < streams[si].t_end; ++t, ++u)
          put(die, si, t, t + 1, (2 * u + 1) * per_die / (2 * tiles), per_die);
    }
  }
  for (int32_t i : wide) {
    first[i] = (int32_t)out.pieces.size();
    count[i] = (int32_t)own[i].size();
    out.pieces.insert(out.pieces.end(), own[i].begin(), own[i].end());
  }
  out.ranked = true;
}

// Chunk schedule with prefix groups.  A group of n members sharing T tiles
// gives one item of shared streams (tiles [0, T) of the first member, per
// head block) and, per member, an item of its own streams (tiles [T, end)).
// Member records are per (member, head block): the shared pieces first, then
// its own pieces.  Ungrouped sequences are planned as by the plain chunk
// schedule.
pa_status schedule_prefix(const int32_t* lens, int32_t num_seqs, int32_t num_kv_heads, int32_t group_cap,
                          const int32_t* prefix_group, const int32_t* prefix_tokens, int64_t nwg_req, int64_t cap,
                          bool use_sets, Schedule& out) {
  const int32_t head_blocks = (num_kv_heads + 3) / 4;
  // Groups: members in sequence order, cut into groups of at most group_cap.
  std::vector<int32_t> by_key;
  for (int32_t s = 0; s < num_seqs; ++s)
    if (prefix_group[s] >= 0 && lens[s] > 0) by_key.push_back(s);
  std::stable_sort(by_key.begin(), by_key.end(), [&](int32_t x, int32_t y) { return prefix_group[x] < prefix_group[y]; });
  std::vector<std::vector<int32_t>> groups;
  std::vector<int32_t> shared_tiles;
  for (size_t i = 0; i < by_key.size();) {
    size_t j = i;
    while (j < by_key.size() && prefix_group[by_key[j]] == prefix_group[by_key[i]]) ++j;
    // A key group that does not become exactly one planned group (more
    // members than fit, or no whole shared tile) has its prefix blocks read
    // by several jobs.
    if (j - i >= 2 && j - i > (size_t)group_cap) out.reread = true;
    for (size_t k = i; k < j; k += (size_t)group_cap) {
      std::vector<int32_t> g(by_key.begin() + k, by_key.begin() + std::min(j, k + (size_t)group_cap));
      int64_t tok = INT64_MAX;
      for (int32_t m : g) tok = std::min<int64_t>(tok, std::min<int64_t>(prefix_tokens[m], lens[m] - 1));
      const int32_t t = tok > 0 ? (int32_t)(tok / 16) : 0;
      if (g.size() >= 2 && t >= 1) {
        groups.push_back(g);
        shared_tiles.push_back(t);
      } else if (j - i >= 2) {
        out.reread = true;
      }
    }
    i = j;
  }
  std::vector<int32_t> group_of(num_seqs, -1);
  for (size_t gi = 0; gi < groups.size(); ++gi)
    for (int32_t m : groups[gi]) group_of[m] = (int32_t)gi;
  const bool die_aware = nwg_req % kDies == 0 && nwg_req >= 8 * kDies;
  // Wide key groups (cut into several planned groups) are read in sets: up to
  // kSetGroups consecutive groups of one key group with the same shared tiles.  A
  // set's shared tiles are read once per KV head by one workgroup, whose
  // wavefront w scores group w of the set (PA_JOB_WIDE); a wavefront holding
  // one group of at most 16 query columns keeps its registers as for any job.
  std::vector<int32_t> set_first, set_n, set_of_group(groups.size(), -1);
  if (die_aware && use_sets) {
    for (size_t gi = 0; gi < groups.size();) {
      const int32_t key = prefix_group[groups[gi][0]];
      size_t gj = gi;
      while (gj < groups.size() && prefix_group[groups[gj][0]] == key) ++gj;
      if (gj - gi >= 2) {
        for (size_t k = gi; k < gj;) {
          size_t e = k + 1;
          while (e < gj && e - k < (size_t)kSetGroups && shared_tiles[e] == shared_tiles[k]) ++e;
          for (size_t x = k; x < e; ++x) set_of_group[x] = (int32_t)set_first.size();
          set_first.push_back((int32_t)k);
          set_n.push_back((int32_t)(e - k));
          k = e;
        }
      }
      gi = gj;
    }
  }
  // Streams: shared items first in the list, then every sequence's own item.
  std::vector<Stream> streams;
  std::vector<int32_t> shared_of(groups.size() * head_blocks, -1), head_of;
  int32_t item = 0;
  for (size_t gi = 0; gi < groups.size(); ++gi) {
    const int32_t lead = groups[gi][0];
    const int32_t si = set_of_group[gi];
    if (si < 0) {
      for (int32_t hb = 0; hb < head_blocks; ++hb) {
        shared_of[gi * head_blocks + hb] = (int32_t)streams.size();
        head_of.push_back(-1);
        streams.push_back(Stream{lead, hb, 0, shared_tiles[gi], lens[lead], (int32_t)(gi * head_blocks + hb), item});
      }
      ++item;
      continue;
    }
    const int32_t f = set_first[si];
    if ((int32_t)gi == f) {
      for (int32_t hb = 0; hb < head_blocks; ++hb)
        for (int32_t g = 4 * hb; g < std::min<int32_t>(num_kv_heads, 4 * hb + 4); ++g) {
          if (g == 4 * hb) shared_of[gi * head_blocks + hb] = (int32_t)streams.size();
          head_of.push_back(g);
          streams.push_back(Stream{lead, hb, 0, shared_tiles[gi], lens[lead], (int32_t)(gi * head_blocks + hb), item});
        }
      ++item;
    } else {
      for (int32_t hb = 0; hb < head_blocks; ++hb) shared_of[gi * head_blocks + hb] = shared_of[f * head_blocks + hb];
    }
  }
  std::vector<int32_t> own_stream(num_seqs, -1);
  for (int32_t s = 0; s < num_seqs; ++s, ++item) {
    if (lens[s] == 0) continue;
    const int32_t t0 = group_of[s] >= 0 ? shared_tiles[group_of[s]] : 0;
    own_stream[s] = (int32_t)streams.size();
    for (int32_t hb = 0; hb < head_blocks; ++hb) streams.push_back(Stream{s, hb, t0, (lens[s] + 15) / 16, lens[s], -1, item});
  }
  head_of.resize(streams.size(), -1);  // own streams: no KV head of their own
  std::vector<int32_t> first, count, order;
  // Shared streams of wide prefixes (several planned groups of one key group)
  // get a placement of their own when the grid covers every die evenly.
  std::vector<int32_t> wide, rest, set_of(streams.size(), -1);
  if (die_aware) {
    // Groups of one key group are consecutive; a set is one (key group, head
    // block) of a key group planned as several groups.
    int32_t run = -1;
    for (size_t gi = 0; gi < groups.size(); ++gi) {
      const int32_t key = prefix_group[groups[gi][0]];
      if (gi == 0 || prefix_group[groups[gi - 1][0]] != key) ++run;
      if (set_of_group[gi] < 0 || set_first[set_of_group[gi]] != (int32_t)gi) continue;
      for (size_t i = 0; i < streams.size(); ++i)
        if (streams[i].group >= 0 && streams[i].group / head_blocks == (int32_t)gi)
          set_of[i] = run * head_blocks + streams[i].hb;
    }
    // By set, then group.
    std::vector<int32_t> ws;
    for (size_t i = 0; i < streams.size(); ++i) (set_of[i] >= 0 ? ws : rest).push_back((int32_t)i);
    std::stable_sort(ws.begin(), ws.end(), [&](int32_t x, int32_t y) { return set_of[x] < set_of[y]; });
    wide = ws;
  }
  if (wide.empty()) {
    chunk_streams(streams, nwg_req, cap, out, first, count, order);
  } else {
    first.assign(streams.size(), 0);
    count.assign(streams.size(), 0);
    std::vector<int64_t> base(nwg_req, 0);
    place_wide(streams, wide, set_of, nwg_req, cap, set_first.empty() ? kWideTileCost : kSetTileCost, out, first,
               count, base);
    std::vector<Stream> rs;
    rs.reserve(rest.size());
    for (int32_t i : rest) rs.push_back(streams[i]);
    std::vector<int32_t> rf, rc, ro;
    chunk_streams(rs, nwg_req, cap, out, rf, rc, ro, &base);
    for (size_t k = 0; k < rest.size(); ++k) {
      first[rest[k]] = rf[k];
      count[rest[k]] = rc[k];
    }
    for (int32_t k : ro) order.push_back(rest[k]);
  }
  // A member's records are laid out per head block (KV head 4*hb + w, piece
  // p at record_base + w * parts + p), so the head streams of a set within a
  // head block must be cut into equally many pieces.  The die placement cuts
  // them alike unless a die holds more streams than workgroups; the caller
  // then plans without sets.
  for (size_t i = 0; i < streams.size(); ++i)
    if (head_of[i] >= 0 && count[i] != count[shared_of[(size_t)streams[i].group]]) return PA_REPLAN;
  // Records, in layout order of the own streams: a grouped member always has
  // records (its shared pieces and its own); others only when cut.
  std::vector<int32_t> rb((size_t)num_seqs * head_blocks, -1), parts((size_t)num_seqs * head_blocks, 0);
  for (int32_t i : order) {
    const Stream& st = streams[i];
    if (st.group >= 0) continue;
    const int32_t s = st.seq, hb = st.hb;
    const int32_t gi = group_of[s];
    const int32_t ks = gi >= 0 ? count[shared_of[gi * head_blocks + hb]] : 0;
    const int32_t np = ks + count[i];
    if (np <= 1) continue;
    const int64_t heads = std::min<int64_t>(4, num_kv_heads - 4 * hb);
    rb[(size_t)s * head_blocks + hb] = (int32_t)out.records;
    parts[(size_t)s * head_blocks + hb] = np;
    for (int32_t p = 0; p < count[i]; ++p) {
      pa_decode_job& j = out.pieces[first[i] + p].job;
      j.part = ks + p;
      j.num_parts = np;
      j.record_base = (int32_t)out.records;
    }
    out.records += (int64_t)np * heads;
    if (out.records > INT32_MAX / 1024) return fail(PA_ERR_INVALID, "pa_decode_plan: plan too large");
  }
  // Group descriptors (one per group and head block) and shared jobs.
  for (size_t gi = 0; gi < groups.size(); ++gi) {
    for (int32_t hb = 0; hb < head_blocks; ++hb) {
      pa_decode_group d{};
      d.num_members = (int32_t)groups[gi].size();
      d.head_block = hb;
      for (int32_t m = 0; m < 4; ++m) {
        const int32_t s = groups[gi][std::min<size_t>(m, groups[gi].size() - 1)];
        d.seq[m] = s;
        d.record_base[m] = rb[(size_t)s * head_blocks + hb];
        d.num_parts[m] = parts[(size_t)s * head_blocks + hb];
      }
      const int32_t di = (int32_t)out.groups.size();
      out.groups.push_back(d);
      const int32_t si = set_of_group[gi];
      if (si >= 0) {
        if (set_first[si] != (int32_t)gi) continue;
        const int32_t n = set_n[si];
        const int32_t enc = n | ((int32_t)groups[gi].size() << 8) | ((int32_t)groups[gi + n - 1].size() << 16);
        for (size_t i = 0; i < streams.size(); ++i) {
          if (head_of[i] < 0 || streams[i].group != (int32_t)(gi * head_blocks + hb)) continue;
          for (int32_t p = 0; p < count[i]; ++p) {
            pa_decode_job& j = out.pieces[first[i] + p].job;
            j.head_block = head_of[i] | PA_JOB_SHARED | PA_JOB_WIDE;
            j.part = p;
            j.num_parts = enc;
            j.record_base = di;
          }
        }
        continue;
      }
      const int32_t i = shared_of[gi * head_blocks + hb];
      for (int32_t p = 0; p < count[i]; ++p) {
        pa_decode_job& j = out.pieces[first[i] + p].job;
        j.head_block = hb | PA_JOB_SHARED;
        j.part = p;
        j.num_parts = d.num_members;
        j.record_base = di;
      }
    }
    out.group_size = std::max<int32_t>(out.group_size, (int32_t)groups[gi].size());
  }
  // Merge rows, sequence by sequence.
  for (int32_t s = 0; s < num_seqs; ++s) {
    if (lens[s] == 0) {
      for (int32_t g = 0; g < num_kv_heads; ++g) out.merges.push_back(pa_decode_merge{s, g, 0, -1});
      continue;
    }
    for (int32_t hb = 0; hb < head_blocks; ++hb) {
      const int32_t np = parts[(size_t)s * head_blocks + hb];
      if (np <= 1) continue;
      const int32_t b = rb[(size_t)s * head_blocks + hb];
      for (int32_t g = 4 * hb; g < std::min<int32_t>(num_kv_heads, 4 * hb + 4); ++g)
        out.merges.push_back(pa_decode_merge{s, g, np, b + (g - 4 * hb) * np});
    }
  }
  return PA_OK;
}

// Largest pieces first: each sequence's tiles are cut into near-equal pieces
// of at most `cap` tiles (cap = 0: twice the average tiles per workgroup,
// clamped to [4, 64]); one job per (piece, head block).  Fewer, larger jobs than the
// chunks when most sequences fit in one workgroup's share.  Records are per
// sequence: KV head g, piece p at base + g * parts + p.
//
// Placement balances compute units, not workgroups.  With two resident
// workgroups per CU (the default grid), the dispatcher places workgroup b and
// b + nwg/2 on the same CU, and each SIMD of that CU runs one wavefront of
// each: a CU's time follows the tiles of both.  So, for an even grid, jobs
// (largest first) go to the least-loaded pair {b, b + nwg/2} (by tiles; ties
// to the pair that reached that load first, initially by index), and each
// pair's jobs, in that order, go to the lighter of its two workgroups (ties
// to b).  An odd grid places jobs on the least-loaded workgroup directly.
// Each workgroup then runs its jobs smallest first.
// The two workgroups of a compute unit do not share it equally.  Workgroup b
// is dispatched just before b + nwg / 2, on the same compute unit, and its
// wavefronts win the issue arbitration of the SIMDs the two share.  Measured
// on MI355X (batch 256, 8 KV heads, lognormal lengths around 200 tokens)
// with per-wavefront timestamps: while both run, the older
// workgroup streams about 0.51 tiles/us and the younger 0.32; a workgroup
// left alone streams 0.75.  Split evenly by tiles, the older finished about
// 8 us first and the compute unit spent its last quarter at one workgroup.
// pair_end_us models a compute unit's end time from the tiles and jobs of its
// two workgroups (each job also costs kSplitJobUs); schedule_lpt splits each
// pair's jobs to minimise it.
constexpr double kRateOlder = 0.51, kRateYounger = 0.32, kRateAlone = 0.75, kSplitJobUs = 0.5;
constexpr double kPerTileOlder = 1.0 / kRateOlder, kPerTileYounger = 1.0 / kRateYounger,
                 kPerTileAlone = 1.0 / kRateAlone;
constexpr int kSplitMaxJobs = 8;  // pairs with more jobs keep the greedy split

double pair_end_us(double older_tiles, int older_jobs, double younger_tiles, int younger_jobs) {
  const double t_older = older_tiles * kPerTileOlder + kSplitJobUs * older_jobs;
  const double t_younger = younger_tiles * kPerTileYounger + kSplitJobUs * younger_jobs;
  // Both cases computed and one selected: the comparison is unpredictable
  // over the subsets a plan tries, and a branch on it costs more than the
  // arithmetic.
  const double younger_done = kRateYounger * std::max(0.0, t_older - kSplitJobUs * younger_jobs);
  const double older_first = t_older + std::max(0.0, younger_tiles - younger_done) * kPerTileAlone;
  const double older_done = kRateOlder * std::max(0.0, t_younger - kSplitJobUs * older_jobs);
  const double younger_first = t_younger + std::max(0.0, older_tiles - older_done) * kPerTileAlone;
  return t_older <= t_younger ? older_first : younger_first;
}

pa_status schedule_lpt(const int32_t* lens, int32_t num_seqs, int32_t num_kv_heads, int64_t nwg_req,
                       int64_t cap_req, Schedule& out) {
  const int64_t head_blocks = (num_kv_heads + 3) / 4;
  int64_t total = 0;
  for (int32_t s = 0; s < num_seqs; ++s) total += ((int64_t)lens[s] + 15) / 16 * head_blocks;
  // Default piece: twice the average tiles per workgroup.  The pair split
  // balances a compute unit's two workgroups, so pieces coarser than one
  // workgroup's share still balance, with fewer jobs and merge records.
  const int64_t cap = cap_req > 0 ? cap_req : std::min<int64_t>(64, std::max<int64_t>(4, (2 * total + nwg_req - 1) / nwg_req));
  std::vector<pa_decode_job> jobs;
  {
    int64_t n = 0;
    for (int32_t s = 0; s < num_seqs; ++s) n += (((int64_t)lens[s] + 15) / 16 + cap - 1) / cap;
    jobs.reserve((size_t)(n * head_blocks));
    out.merges.reserve((size_t)num_seqs * num_kv_heads);
  }
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t tiles = ((int64_t)lens[s] + 15) / 16;
    if (tiles == 0) {
      for (int32_t g = 0; g < num_kv_heads; ++g) out.merges.push_back(pa_decode_merge{s, g, 0, -1});
      continue;
    }
    const int64_t parts = (tiles + cap - 1) / cap;
    const int64_t base = parts > 1 ? out.records : -1;
    if (parts > 1) {
      for (int32_t g = 0; g < num_kv_heads; ++g)
        out.merges.push_back(pa_decode_merge{s, g, (int32_t)parts, (int32_t)(out.records + g * parts)});
      out.records += parts * num_kv_heads;
      if (out.records > INT32_MAX / 1024) return fail(PA_ERR_INVALID, "pa_decode_plan: plan too large");
    }
    int64_t t0 = 0;
    for (int64_t p = 0; p < parts; ++p) {
      const int64_t cnt = tiles / parts + (p < tiles % parts ? 1 : 0);
      for (int64_t hb = 0; hb < head_blocks; ++hb)
        jobs.push_back(pa_decode_job{s, (int32_t)t0, (int32_t)cnt, (int32_t)hb, (int32_t)p, (int32_t)parts,
                                     (int32_t)(base >= 0 ? base + 4 * hb * parts : -1), lens[s]});
      t0 += cnt;
    }
  }
  const int64_t nwg = std::max<int64_t>(1, std::min<int64_t>(nwg_req, (int64_t)jobs.size()));
  out.nwg = nwg;
  // Jobs by tile count, largest first, ties in generation order (a counting
  // sort: counts are 1..cap).
  std::vector<int32_t> order(jobs.size());
  {
    std::vector<int32_t> start(cap + 2, 0);
    for (const pa_decode_job& j : jobs) start[cap - j.tile_count + 1] += 1;
    for (int64_t c = 1; c <= cap + 1; ++c) start[c] += start[c - 1];
    for (size_t i = 0; i < jobs.size(); ++i) order[start[cap - jobs[i].tile_count]++] = (int32_t)i;
  }
  std::vector<int32_t> placed_wg(jobs.size());
  {
    const bool paired = nwg % 2 == 0;
    const int64_t bins = paired ? nwg / 2 : nwg;
    // Min-heap of bins keyed by (load, arrival): the least-loaded bin first,
    // then the one that reached its load first.  Keys are distinct, so the
    // bin picked at each step does not depend on the heap's shape.  Loads
    // and arrivals stay below 2^31 (tiles and jobs are bounded by the plan
    // size check), so a key packs into one 64-bit word.
    struct Entry {
      uint64_t key;
      int32_t bin;
    };
    std::vector<Entry> heap((size_t)bins);
    for (int64_t b = 0; b < bins; ++b) heap[b] = Entry{(uint64_t)b, (int32_t)b};  // already a heap
    uint64_t arrival = (uint64_t)bins;
    std::vector<int64_t> wg_load(nwg, 0);
    const size_t n = heap.size();
    for (int32_t j : order) {
      const int32_t b = heap[0].bin;
      int32_t w = b;
      if (paired && wg_load[b + bins] < wg_load[b]) w = (int32_t)(b + bins);
      placed_wg[j] = w;
      wg_load[w] += jobs[j].tile_count;
      // The top's load grows: replace it and sift down.
      const Entry e{(((heap[0].key >> 32) + (uint64_t)jobs[j].tile_count) << 32) | arrival++, b};
      size_t i = 0;
      for (;;) {
        size_t c = 2 * i + 1;
        if (c >= n) break;
        if (c + 1 < n && heap[c + 1].key < heap[c].key) ++c;
        if (heap[c].key >= e.key) break;
        heap[i] = heap[c];
        i = c;
      }
      heap[i] = e;
    }
    if (paired) {
      // Each pair's jobs are split between its two workgroups by the
      // modelled end time (pair_end_us), over every subset of the pair's jobs
      // (subset sums built incrementally).  Measured on the batch of 256
      // (8 KV heads): attention launch 39.65 -> 39.1 us.
      std::vector<int32_t> first((size_t)bins + 1, 0), list(jobs.size());
      for (size_t j = 0; j < jobs.size(); ++j) first[placed_wg[j] % bins + 1] += 1;
      for (int64_t b = 0; b < bins; ++b) first[b + 1] += first[b];
      {
        std::vector<int32_t> at(first.begin(), first.end() - 1);
        for (size_t j = 0; j < jobs.size(); ++j) list[at[placed_wg[j] % bins]++] = (int32_t)j;
      }
      double sum[1 << kSplitMaxJobs];
      for (int64_t b = 0; b < bins; ++b) {
        const int32_t* pj = list.data() + first[b];
        const int np = first[b + 1] - first[b];
        if (np < 2 || np > kSplitMaxJobs) continue;
        const uint32_t full = (1u << np) - 1;
        sum[0] = 0;
        for (uint32_t m = 1; m <= full; ++m) sum[m] = sum[m & (m - 1)] + jobs[pj[__builtin_ctz(m)]].tile_count;
        double best = std::numeric_limits<double>::infinity();
        uint32_t best_mask = 0;
        for (uint32_t m = 0; m <= full; ++m) {
          const int older_jobs = __builtin_popcount(m);
          const double e = pair_end_us(sum[m], older_jobs, sum[full] - sum[m], np - older_jobs);
          const bool better = e < best;
          best = better ? e : best;
          best_mask = better ? m : best_mask;
        }
        for (int i = 0; i < np; ++i) placed_wg[pj[i]] = (int32_t)(((best_mask >> i) & 1) ? b : b + bins);
      }
    }
  }
  // Each workgroup runs its jobs smallest first (ties in generation order):
  // job boundaries then fall in the start-up, where every tile waits in the
  // memory queue anyway, and the workgroup ends on its longest, unbroken
  // stream.  Measured on the batch of 256 (8 KV heads): 39.8 against 40.1
  // us in generation order and 40.4 us largest first.
  out.pieces.clear();
  out.pieces.reserve(jobs.size());
  {
    // A counting sort by size, ascending, stable.
    std::vector<int32_t> start(cap + 2, 0);
    for (const pa_decode_job& j : jobs) start[j.tile_count + 1] += 1;
    for (int64_t c = 1; c <= cap + 1; ++c) start[c] += start[c - 1];
    std::vector<int32_t> asc(jobs.size());
    for (size_t i = 0; i < jobs.size(); ++i) asc[start[jobs[i].tile_count]++] = (int32_t)i;
    for (int32_t j : asc) out.pieces.push_back(Piece{placed_wg[j], jobs[j]});
  }
  return PA_OK;
}

// Largest compute-unit cost: tokens of its tiles plus kJobCharge per job,
// summed over the workgroup pair {b, b + nwg/2} that shares a compute unit
// (an odd grid: the largest workgroup cost).  A pair is the unit because the
// two workgroups' shares of the compute unit are uneven (pair_end_us): an
// uneven split within a pair costs little.
int64_t schedule_cost(const Schedule& sc, const int32_t* lens) {
  std::vector<int64_t> cost(sc.nwg, 0);
  for (const Piece& pc : sc.pieces)
    cost[pc.wg] += kJobCharge + rows_between(lens[pc.job.seq], pc.job.tile_begin, pc.job.tile_begin + pc.job.tile_count);
  int64_t m = 0;
  if (sc.nwg % 2 == 0) {
    const int64_t half = sc.nwg / 2;
    for (int64_t b = 0; b < half; ++b) m = std::max(m, cost[b] + cost[b + half]);
  } else {
    for (int64_t c : cost) m = std::max(m, c);
  }
  return m;
}

}  // namespace
}  // namespace pagedkv

namespace pagedkv {
namespace {

// Serialise a schedule: the column-major job table, the merge rows, the
// group descriptors.  The info also records what the plan was made for: the
// batch size, the longest context and a digest of the lengths.
pa_status emit_plan(const Schedule& sc, int32_t schedule_id, int32_t num_kv_heads, const int32_t* lens,
                    int32_t num_seqs, void* plan, size_t capacity, pa_decode_plan_info* info) {
  const std::vector<Piece>& jobs = sc.pieces;
  const std::vector<pa_decode_merge>& merges = sc.merges;
  const int64_t nwg = sc.nwg;
  if (jobs.size() > (size_t)INT32_MAX / 64 || merges.size() > (size_t)INT32_MAX / 64 ||
      sc.groups.size() > (size_t)INT32_MAX / 64)
    return fail(PA_ERR_INVALID, "pa_decode_plan: plan too large");
  // Per-workgroup lists, column-major: slot k of workgroup b is entry
  // k * nwg + b, so a workgroup reads its first jobs without an index load.
  // Slots past a workgroup's last job are empty (tile_count 0).  A
  // workgroup's jobs keep schedule order.
  std::vector<int32_t> count(nwg, 0);
  for (const Piece& pc : jobs) count[pc.wg] += 1;
  int64_t per = 0;
  for (int32_t c : count) per = std::max<int64_t>(per, c);
  if (per * nwg > (int64_t)INT32_MAX / 64) return fail(PA_ERR_INVALID, "pa_decode_plan: plan too large");
  const size_t slots = (size_t)(per * nwg);

  pa_decode_plan_info in{};
  in.num_workgroups = jobs.empty() ? 0 : (int32_t)nwg;
  in.num_jobs = (int32_t)jobs.size();
  in.num_merges = (int32_t)merges.size();
  in.num_records = (int32_t)sc.records;
  in.num_kv_heads = num_kv_heads;
  in.jobs_per_workgroup = jobs.empty() ? 0 : (int32_t)per;
  in.jobs_at = 0;
  in.merges_at = (int32_t)(sizeof(pa_decode_job) * slots);
  in.schedule = schedule_id;
  in.num_groups = (int32_t)sc.groups.size();
  in.groups_at = (int32_t)round_up((size_t)in.merges_at + sizeof(pa_decode_merge) * merges.size(), 64);
  in.group_size = sc.group_size;
  // First-tile table entries: 4 int32 per job slot, written by
  // pa_decode_plan_first_blocks when the caller has the tables on the host.
  in.first_at = (int32_t)round_up((size_t)in.groups_at + sizeof(pa_decode_group) * sc.groups.size(), 64);
  in.first_block_size = 0;
  int64_t tiles = 0;
  in.max_job_tiles = 0;
  for (const Piece& pc : jobs) {
    tiles += pc.job.tile_count;
    in.max_job_tiles = std::max(in.max_job_tiles, pc.job.tile_count);
  }
  in.num_tiles = (int32_t)tiles;
  in.wide_jobs = 0;
  for (const Piece& pc : jobs) in.wide_jobs += (pc.job.head_block & PA_JOB_WIDE) != 0;
  in.num_seqs = num_seqs;
  in.max_context_len = 0;
  for (int32_t i = 0; i < num_seqs; ++i) in.max_context_len = std::max(in.max_context_len, lens[i]);
  in.lens_digest = lens_digest(lens, num_seqs);
  const size_t bytes = (size_t)in.first_at + 16 * slots;
  if (bytes > (size_t)INT32_MAX) return fail(PA_ERR_INVALID, "pa_decode_plan: plan too large");
  in.bytes = (int32_t)bytes;
  *info = in;
  if (bytes > capacity)
    return fail(PA_ERR_INVALID, "pa_decode_plan: capacity %zu < %zu bytes", capacity, bytes);
  // Every byte up to `bytes` is written once: the job slots (jobs, then
  // empty slots), the merge rows, the groups, zeros in the alignment gaps
  // and in the first-tile region.
  if (bytes == 0) return PA_OK;
  char* out = static_cast<char*>(plan);
  char* table = out + in.jobs_at;
  std::vector<int32_t> fill(nwg, 0);
  auto put = [&](const Piece& pc) {
    std::memcpy(table + sizeof(pa_decode_job) * ((size_t)fill[pc.wg]++ * nwg + pc.wg), &pc.job, sizeof(pa_decode_job));
  };
  if (sc.ranked) {
    std::vector<int32_t> by_rank(jobs.size());
    for (size_t i = 0; i < jobs.size(); ++i) by_rank[i] = (int32_t)i;
    std::stable_sort(by_rank.begin(), by_rank.end(), [&](int32_t x, int32_t y) { return jobs[x].rank < jobs[y].rank; });
    for (int32_t i : by_rank) put(jobs[i]);
  } else {
    for (const Piece& pc : jobs) put(pc);
  }
  const pa_decode_job empty{0, 0, 0, 0, 0, 0, -1, 0};
  for (int64_t b = 0; b < nwg; ++b)
    for (int64_t k = fill[b]; k < per; ++k)
      std::memcpy(table + sizeof(pa_decode_job) * (size_t)(k * nwg + b), &empty, sizeof(pa_decode_job));
  const size_t merges_end = (size_t)in.merges_at + sizeof(pa_decode_merge) * merges.size();
  const size_t groups_end = (size_t)in.groups_at + sizeof(pa_decode_group) * sc.groups.size();
  if (!merges.empty()) std::memcpy(out + in.merges_at, merges.data(), sizeof(pa_decode_merge) * merges.size());
  std::memset(out + merges_end, 0, (size_t)in.groups_at - merges_end);
  if (!sc.groups.empty()) std::memcpy(out + in.groups_at, sc.groups.data(), sizeof(pa_decode_group) * sc.groups.size());
  std::memset(out + groups_end, 0, bytes - groups_end);
  return PA_OK;
}

}  // namespace
}  // namespace pagedkv

extern "C" pa_status pa_decode_plan_prefix(const int32_t* context_lens, int32_t num_seqs, int32_t num_kv_heads,
                                           int32_t num_q_heads, int32_t num_workgroups, int32_t max_piece_tiles,
                                           const int32_t* prefix_group, const int32_t* prefix_tokens, void* plan,
                                           size_t capacity, pa_decode_plan_info* info) {
  if (!info || num_seqs < 0 || num_kv_heads <= 0 || num_workgroups <= 0 ||
      (num_seqs > 0 && (!context_lens || !prefix_group || !prefix_tokens)))
    return fail(PA_ERR_INVALID, "pa_decode_plan_prefix: bad arguments");
  if (num_q_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return fail(PA_ERR_INVALID, "pa_decode_plan_prefix: num_q_heads %d not a multiple of num_kv_heads %d",
                num_q_heads, num_kv_heads);
  if (max_piece_tiles < 0 || max_piece_tiles > 64)
    return fail(PA_ERR_INVALID, "pa_decode_plan_prefix: max_piece_tiles %d outside [0, 64]", max_piece_tiles);
  if (capacity > 0 && (!plan || !pagedkv::aligned(plan, 8)))
    return fail(PA_ERR_INVALID, "pa_decode_plan_prefix: plan buffer NULL or not 8-byte aligned");
  int64_t total_tiles = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    if (context_lens[s] < 0) return fail(PA_ERR_INVALID, "pa_decode_plan_prefix: context_lens[%d] < 0", s);
    total_tiles += ((int64_t)context_lens[s] + 15) / 16 * ((num_kv_heads + 3) / 4);
  }
  if (total_tiles > (int64_t)INT32_MAX / 64) return fail(PA_ERR_INVALID, "pa_decode_plan_prefix: plan too large");
  const int32_t group = num_q_heads / num_kv_heads;
  const int32_t group_cap = std::min(4, std::max(1, 16 / group));
  const int64_t cap = max_piece_tiles > 0 ? max_piece_tiles : 64;
  pagedkv::Schedule sc;
  pa_status ps = pagedkv::schedule_prefix(context_lens, num_seqs, num_kv_heads, group_cap, prefix_group, prefix_tokens,
                                          num_workgroups, cap, true, sc);
  if (ps == PA_REPLAN) {  // the sets could not be cut alike: every group reads on its own
    sc = pagedkv::Schedule{};
    ps = pagedkv::schedule_prefix(context_lens, num_seqs, num_kv_heads, group_cap, prefix_group, prefix_tokens,
                                  num_workgroups, cap, false, sc);
  }
  if (ps != PA_OK) return ps;
  const pa_status st =
      pagedkv::emit_plan(sc, PA_SCHEDULE_CHUNKS, num_kv_heads, context_lens, num_seqs, plan, capacity, info);
  // Loads keep blocks in the caches only when some block is read by more
  // than one job; with every shared prefix read once by its group they
  // stream past the caches like unshared blocks.
  if (st == PA_OK) info->flags = sc.reread ? PA_DECODE_SHARED_KV : 0;
  return st;
}

extern "C" pa_status pa_decode_plan(const int32_t* context_lens, int32_t num_seqs, int32_t num_kv_heads,
                                    int32_t num_workgroups, int32_t max_piece_tiles, void* plan,
                                    size_t capacity, pa_decode_plan_info* info) {
  return pa_decode_plan_schedule(context_lens, num_seqs, num_kv_heads, num_workgroups, max_piece_tiles,
                                 PA_SCHEDULE_AUTO, plan, capacity, info);
}

extern "C" pa_status pa_decode_plan_schedule(const int32_t* context_lens, int32_t num_seqs, int32_t num_kv_heads,
                                             int32_t num_workgroups, int32_t max_piece_tiles, int32_t schedule,
                                             void* plan, size_t capacity, pa_decode_plan_info* info) {
  using pagedkv::Piece;
  using pagedkv::Schedule;
  if (!info || num_seqs < 0 || num_kv_heads <= 0 || num_workgroups <= 0 || (num_seqs > 0 && !context_lens))
    return fail(PA_ERR_INVALID, "pa_decode_plan: bad arguments");
  if (max_piece_tiles < 0 || max_piece_tiles > 64)
    return fail(PA_ERR_INVALID, "pa_decode_plan: max_piece_tiles %d outside [0, 64]", max_piece_tiles);
  if (schedule != PA_SCHEDULE_AUTO && schedule != PA_SCHEDULE_CHUNKS && schedule != PA_SCHEDULE_LPT)
    return fail(PA_ERR_INVALID, "pa_decode_plan: unknown schedule %d", schedule);
  if (capacity > 0 && (!plan || !pagedkv::aligned(plan, 8)))
    return fail(PA_ERR_INVALID, "pa_decode_plan: plan buffer NULL or not 8-byte aligned");
  int64_t total_tiles = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    if (context_lens[s] < 0) return fail(PA_ERR_INVALID, "pa_decode_plan: context_lens[%d] < 0", s);
    total_tiles += ((int64_t)context_lens[s] + 15) / 16 * ((num_kv_heads + 3) / 4);
  }
  if (total_tiles > (int64_t)INT32_MAX / 64) return fail(PA_ERR_INVALID, "pa_decode_plan: plan too large");

  // Automatic choice: both schedules are built and the one whose busiest
  // compute unit costs less (tokens plus a charge per job) is kept, the
  // chunks on a tie.
  Schedule chunks, lpt;
  pagedkv::ChunkWalk walk;
  if (schedule != PA_SCHEDULE_LPT)
    pagedkv::walk_chunks(context_lens, num_seqs, num_kv_heads, num_workgroups,
                         max_piece_tiles > 0 ? max_piece_tiles : 64, chunks, walk);
  if (schedule != PA_SCHEDULE_CHUNKS) {
    if (pa_status st = pagedkv::schedule_lpt(context_lens, num_seqs, num_kv_heads, num_workgroups, max_piece_tiles, lpt))
      return st;
  }
  const bool use_lpt = schedule == PA_SCHEDULE_LPT ||
                       (schedule == PA_SCHEDULE_AUTO && !lpt.pieces.empty() &&
                        pagedkv::schedule_cost(lpt, context_lens) < pagedkv::schedule_cost(chunks, context_lens));
  if (!use_lpt) {
    if (pa_status st = pagedkv::finish_chunks(context_lens, num_seqs, num_kv_heads, walk, chunks)) return st;
  }
  return pagedkv::emit_plan(use_lpt ? lpt : chunks, use_lpt ? PA_SCHEDULE_LPT : PA_SCHEDULE_CHUNKS, num_kv_heads,
                            context_lens, num_seqs, plan, capacity, info);
}

extern "C" pa_status pa_decode_plan_first_blocks(void* plan, pa_decode_plan_info* info, const int32_t* tables,
                                                int32_t max_blocks, int32_t num_seqs, int32_t block_size) {
  const char* who = "pa_decode_plan_first_blocks";
  if (!plan || !info) return fail(PA_ERR_INVALID, "%s: plan or info is NULL", who);
  if (!pagedkv::supported_block_size(block_size))
    return fail(PA_ERR_UNSUPPORTED, "%s: block_size %d (supported: 1, 2, 4, 8, 16, 32)", who, block_size);
  // Below 8 slots a tile spans more blocks than the four entries per job
  // slot hold: nothing is written and the flag stays clear.
  if (block_size < 8) return PA_OK;
  const int64_t slots = (int64_t)info->jobs_per_workgroup * info->num_workgroups;
  if (info->jobs_at != 0 || info->first_at % 64 != 0 || slots < 0 ||
      (int64_t)info->first_at < 32 * slots || (int64_t)info->bytes < (int64_t)info->first_at + 16 * slots)
    return fail(PA_ERR_INVALID, "%s: inconsistent plan info", who);
  if (slots > 0 && (!tables || max_blocks <= 0 || num_seqs <= 0))
    return fail(PA_ERR_INVALID, "%s: tables, max_blocks and num_seqs are needed", who);
  const pa_decode_job* jobs = reinterpret_cast<const pa_decode_job*>(static_cast<const char*>(plan) + info->jobs_at);
  int32_t* first = reinterpret_cast<int32_t*>(static_cast<char*>(plan) + info->first_at);
  const int64_t tiles_per_block = block_size >= 16 ? block_size / 16 : 1;
  for (int64_t i = 0; i < slots; ++i) {
    const pa_decode_job& j = jobs[i];
    int32_t* f = first + 4 * i;
    f[0] = f[1] = f[2] = f[3] = 0;
    if (j.tile_count <= 0) continue;
    if (j.seq < 0 || j.seq >= num_seqs)
      return fail(PA_ERR_INVALID, "%s: job slot %lld names sequence %d of %d", who, (long long)i, j.seq, num_seqs);
    const int32_t* row = tables + (int64_t)j.seq * max_blocks;
    // The entries of tiles 0 and 1 of the job: entry t / (B / 16) of tile t,
    // entries 2t and 2t + 1 at B = 8.  Only the sequence's first
    // ceil(L / B) entries are read; a position past them (the second tile of
    // a one-tile job, the second half of a last tile at B = 8) gets 0, which
    // the kernel never loads from.
    const int64_t used = std::min<int64_t>(((int64_t)std::max(j.context_len, 0) + block_size - 1) / block_size,
                                           max_blocks);
    auto entry = [&](int64_t e) { return e >= 0 && e < used ? row[e] : 0; };
    for (int64_t k = 0; k < 2; ++k) {
      const int64_t t = (int64_t)std::max(j.tile_begin, 0) + k;
      const int64_t e0 = block_size == 8 ? 2 * t : t / tiles_per_block;
      f[k] = entry(e0);
      f[2 + k] = block_size == 8 ? entry(e0 + 1) : 0;
    }
  }
  info->first_block_size = block_size;
  info->flags |= PA_DECODE_FIRST_BLOCKS;
  return PA_OK;
}

extern "C" pa_status pa_decode_plan_check_lens(const pa_decode_plan_info* info, const int32_t* context_lens,
                                              int32_t num_seqs) {
  const char* who = "pa_decode_plan_check_lens";
  if (!info || num_seqs < 0 || (num_seqs > 0 && !context_lens)) return fail(PA_ERR_INVALID, "%s: bad arguments", who);
  if (num_seqs != info->num_seqs)
    return fail(PA_ERR_INVALID, "%s: plan made for %d sequences, %d given", who, info->num_seqs, num_seqs);
  if (pagedkv::lens_digest(context_lens, num_seqs) != info->lens_digest)
    return fail(PA_ERR_INVALID, "%s: plan made for other context lengths (a plan from another step?)", who);
  return PA_OK;
}

extern "C" pa_status pa_decode_plan_advance(void* plan, pa_decode_plan_info* info, const int32_t* context_lens,
                                            int32_t num_seqs, int32_t max_job_tiles) {
  const char* who = "pa_decode_plan_advance";
  if (!plan || !info || num_seqs < 0 || (num_seqs > 0 && !context_lens) || max_job_tiles < 0)
    return fail(PA_ERR_INVALID, "%s: bad arguments", who);
  if (num_seqs != info->num_seqs)
    return fail(PA_ERR_INVALID, "%s: the plan is for %d sequences, not %d", who, info->num_seqs, num_seqs);
  if (info->num_groups != 0) return PA_REPLAN;
  const int32_t cap = max_job_tiles > 0 ? std::min(max_job_tiles, 64) : 64;
  const int64_t slots = (int64_t)info->jobs_per_workgroup * info->num_workgroups;
  if (slots < 0 || info->jobs_at < 0 || (int64_t)info->jobs_at + slots * (int64_t)sizeof(pa_decode_job) > info->bytes)
    return fail(PA_ERR_INVALID, "%s: inconsistent plan info", who);
  pa_decode_job* jobs = reinterpret_cast<pa_decode_job*>(static_cast<char*>(plan) + info->jobs_at);
  // Tiles each sequence's jobs cover now (the end of its last piece).
  std::vector<int32_t> end(num_seqs, 0);
  for (int64_t i = 0; i < slots; ++i) {
    const pa_decode_job& j = jobs[i];
    if (j.tile_count <= 0) continue;
    if (j.seq < 0 || j.seq >= num_seqs || j.tile_begin < 0)
      return fail(PA_ERR_INVALID, "%s: job slot %lld names sequence %d", who, (long long)i, j.seq);
    end[j.seq] = std::max(end[j.seq], j.tile_begin + j.tile_count);
  }
  int32_t max_len = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t L = context_lens[s];
    if (L < 0) return fail(PA_ERR_INVALID, "%s: context_lens[%d] < 0", who, s);
    const int32_t tiles = (L + 15) / 16;
    if (tiles != end[s] && (tiles != end[s] + 1 || end[s] == 0)) return PA_REPLAN;
    max_len = std::max(max_len, L);
  }
  for (int64_t i = 0; i < slots; ++i) {
    const pa_decode_job& j = jobs[i];
    if (j.tile_count > 0 && (context_lens[j.seq] + 15) / 16 > end[j.seq] && j.tile_begin + j.tile_count == end[j.seq] &&
        j.tile_count + 1 > cap)
      return PA_REPLAN;
  }
  // Apply: new lengths, the last pieces of grown sequences one tile longer.
  int64_t tiles = 0;
  int32_t longest = 0;
  for (int64_t i = 0; i < slots; ++i) {
    pa_decode_job& j = jobs[i];
    if (j.tile_count <= 0) continue;
    const int32_t L = context_lens[j.seq];
    if ((L + 15) / 16 > end[j.seq] && j.tile_begin + j.tile_count == end[j.seq]) j.tile_count += 1;
    j.context_len = L;
    tiles += j.tile_count;
    longest = std::max(longest, j.tile_count);
  }
  info->num_tiles = (int32_t)tiles;
  info->max_job_tiles = longest;
  info->max_context_len = max_len;
  info->lens_digest = pagedkv::lens_digest(context_lens, num_seqs);
  info->flags &= ~PA_DECODE_FIRST_BLOCKS;
  info->first_block_size = 0;
  return PA_OK;
}

extern "C" size_t pa_decode_workspace_bytes(const pa_decode_plan_info* info, int32_t num_q_heads,
                                            int32_t head_dim) {
  if (!info || info->num_records <= 0 || num_q_heads <= 0 || head_dim <= 0 || info->num_kv_heads <= 0) return 0;
  const int64_t group = num_q_heads / info->num_kv_heads;
  return pagedkv::layout((int64_t)info->num_records * group, head_dim).total;
}

namespace pagedkv {

// Shared front of pa_decode, its two stages and pa_decode_noalloc:
// validation, then the launches the stage mask selects.  `who` names the
// entry point in errors.
// How the attention launch loads tiles with the append fused (0 without
// it); with `a`, also the windows mode 4 reads through.
//
// The tile holding a sequence's appended token mixes pool rows and the new
// row.  Loading it on a path of its own (1) costs a wait for every load in
// flight where the paths join, once per job that ends a sequence; loading
// every tile through per-lane addresses (2) avoids that but loses the
// streaming cache policy of buffer loads on every tile.  Measured on
// MI355X: per-lane addresses everywhere are faster where sequences are short
// (a job end every few tiles: batch 256, mean 200 tokens) and for one query
// head per KV head (batch 64 of up to 2048 tokens, 3%); the separate path
// is faster for long contexts with 4 or 8 query heads per KV head (16 x
// 16-32k tokens, 3%; 2000-token shared prefixes, 2%).  Where per-lane
// addresses win and each pool and its new rows lie within one 4 GiB window
// (4), every tile is read by buffer loads at 32-bit lane offsets in that
// window: the streaming cache policy is kept, with less lane arithmetic than
// 64-bit addresses (batch of 256, 8 KV heads: 39.65 against 39.85 us).
int32_t fused_mode(const pa_kv_pool* pool, const void* new_key, const void* new_value, int32_t num_seqs,
                   int32_t group, const pa_decode_plan_info* info, DecodeArgs* a) {
  if (new_key == nullptr) return 0;
  constexpr int64_t kShortSequenceTiles = 24;
  const int32_t hkv = pool->num_kv_heads;
  const int64_t seq_streams = (int64_t)num_seqs * ((hkv + 3) / 4);
  const bool short_seqs = (int64_t)info->num_tiles < kShortSequenceTiles * seq_streams;
  // Mode 4 (window loads) whenever the tiles are whole blocks and both
  // windows fit: measured at least as fast as 1 and 2 on every batch shape
  // tried (MHA batch 64; GQA batch 256; long contexts, batch 16; forked
  // prefixes; shared system prompts).  Otherwise the separate path for long contexts
  // with 4 or more query heads per KV head, per-lane addresses for the rest.
  const int32_t fallback = !(short_seqs || group < 4 || pool->block_size < 8) ? 1 : 2;
  if (pool->block_size < 16) return fallback;
  const uint64_t pool_bytes = (uint64_t)pool->num_blocks * (uint64_t)pool_block_bytes(*pool);
  const uint64_t new_bytes = (uint64_t)num_seqs * hkv * pool->head_dim * 2;
  DecodeArgs scratch{};
  DecodeArgs& w = a ? *a : scratch;
  auto window = [&](const void* p, const void* n, const void** base, uint32_t* bytes, uint32_t* off,
                    uint32_t* noff) {
    const uint64_t a0 = (uint64_t)(uintptr_t)p, b0 = (uint64_t)(uintptr_t)n;
    const uint64_t lo = std::min(a0, b0), hi = std::max(a0 + pool_bytes, b0 + new_bytes);
    if (hi - lo >= 0xffff0000ull) return false;
    *base = reinterpret_cast<const void*>((uintptr_t)lo);
    *bytes = (uint32_t)(hi - lo);
    *off = (uint32_t)(a0 - lo);
    *noff = (uint32_t)(b0 - lo);
    return true;
  };
  const bool windows = window(pool->k, new_key, &w.k_win, &w.k_win_bytes, &w.k_off, &w.nk_off) &&
                       window(pool->v, new_value, &w.v_win, &w.v_win_bytes, &w.v_off, &w.nv_off);
  return windows ? 4 : fallback;
}

pa_status decode_stages(int stages, const char* who, const pa_kv_pool* pool, const void* q, void* out,
                        int32_t out_dtype, const int32_t* block_tables, int32_t max_blocks_per_seq,
                        const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads, float scale,
                        const void* new_key, const void* new_value, const void* plan,
                        const pa_decode_plan_info* info, void* workspace, size_t workspace_bytes, void* stream) {
  if (pa_status st = pagedkv::check_pool(pool, who)) return st;
  if (!info) return fail(PA_ERR_INVALID, "%s: info is NULL", who);
  if (num_seqs < 0 || max_blocks_per_seq < 0 || info->num_workgroups < 0 || info->num_jobs < 0 ||
      info->jobs_per_workgroup < 0 ||
      info->num_merges < 0 || info->num_records < 0)
    return fail(PA_ERR_INVALID, "%s: negative size", who);
  if (info->num_jobs == 0 && info->num_merges == 0) return PA_OK;
  if (num_seqs == 0) return fail(PA_ERR_INVALID, "%s: a plan with work but num_seqs == 0", who);
  if (num_seqs != info->num_seqs)
    return fail(PA_ERR_INVALID, "%s: plan made for %d sequences, num_seqs is %d", who, info->num_seqs, num_seqs);
  if (!q || !out || !block_tables || !context_lens || !plan)
    return fail(PA_ERR_INVALID, "%s: NULL q/out/block_tables/context_lens/plan", who);
  if (max_blocks_per_seq == 0) return fail(PA_ERR_INVALID, "%s: max_blocks_per_seq == 0", who);
  if ((int64_t)info->max_context_len > (int64_t)max_blocks_per_seq * pool->block_size)
    return fail(PA_ERR_INVALID, "%s: the plan's longest context (%d tokens) needs more than %d table entries of %d slots",
                who, info->max_context_len, max_blocks_per_seq, pool->block_size);
  const int32_t hkv = pool->num_kv_heads;
  if (info->num_kv_heads != hkv)
    return fail(PA_ERR_INVALID, "%s: plan made for %d KV heads, pool has %d", who, info->num_kv_heads, hkv);
  if (num_q_heads <= 0 || num_q_heads % hkv != 0)
    return fail(PA_ERR_INVALID, "%s: num_q_heads %d is not a multiple of num_kv_heads %d", who,
                num_q_heads, hkv);
  const int32_t group = num_q_heads / hkv;
  if (group > 16) return fail(PA_ERR_UNSUPPORTED, "%s: %d query heads per KV head (max 16)", who, group);
  if (out_dtype != PA_F32 && out_dtype != pool->dtype)
    return fail(PA_ERR_UNSUPPORTED, "%s: out_dtype %d must be f32 or the pool dtype", who, out_dtype);
  if (!pagedkv::aligned(q, 16) || !pagedkv::aligned(out, 16) || !pagedkv::aligned(plan, 32))
    return fail(PA_ERR_INVALID, "%s: q/out must be 16-byte and plan 32-byte aligned", who);
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID, "%s: scale is not finite", who);
  if ((new_key == nullptr) != (new_value == nullptr))
    return fail(PA_ERR_INVALID, "%s: new_key and new_value must both be given or both be NULL", who);
  if (new_key && (!pagedkv::aligned(new_key, 16) || !pagedkv::aligned(new_value, 16)))
    return fail(PA_ERR_INVALID, "%s: new_key/new_value must be 16-byte aligned", who);
  if (info->flags & ~(PA_DECODE_SHARED_KV | PA_DECODE_FIRST_BLOCKS))
    return fail(PA_ERR_INVALID, "%s: unknown plan flags 0x%x", who, info->flags);
  const bool first_blocks = (info->flags & PA_DECODE_FIRST_BLOCKS) != 0;
  if (first_blocks && (info->first_block_size != pool->block_size || info->first_at % 64 != 0 ||
                       (int64_t)info->first_at < (int64_t)info->groups_at + 64 * (int64_t)info->num_groups ||
                       (int64_t)info->first_at < (int64_t)info->merges_at + 16 * (int64_t)info->num_merges ||
                       (int64_t)info->bytes < (int64_t)info->first_at +
                                                  16 * (int64_t)info->jobs_per_workgroup * info->num_workgroups))
    return fail(PA_ERR_INVALID,
                "%s: first-tile entries were written for block size %d (pool: %d) or lie outside the plan", who,
                info->first_block_size, pool->block_size);
  if (info->jobs_at != 0 || info->merges_at % 16 != 0 ||
      (info->num_jobs > 0 && (info->num_workgroups == 0 || info->jobs_per_workgroup == 0)) ||
      (int64_t)info->jobs_per_workgroup * info->num_workgroups < (int64_t)info->num_jobs ||
      (int64_t)info->merges_at < 32 * (int64_t)info->jobs_per_workgroup * info->num_workgroups ||
      (int64_t)info->bytes < (int64_t)info->merges_at + 16 * (int64_t)info->num_merges ||
      info->num_groups < 0 || info->wide_jobs < 0 || info->wide_jobs > info->num_jobs ||
      (info->wide_jobs > 0 && info->num_groups == 0) ||
      (info->num_groups > 0 && (info->groups_at % 64 != 0 ||
                                (int64_t)info->groups_at < (int64_t)info->merges_at + 16 * (int64_t)info->num_merges ||
                                (int64_t)info->bytes < (int64_t)info->groups_at + 64 * (int64_t)info->num_groups)))
    return fail(PA_ERR_INVALID, "%s: inconsistent plan info", who);
  if (info->num_groups > 0 && pool->dtype != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "%s: shared-prefix plans need a bf16 pool", who);
  // Below 8 slots per block the kernels hold a window of 128 table entries
  // per job, i.e. 8 * B tiles.
  if (pool->block_size < 8 && info->max_job_tiles > 8 * pool->block_size)
    return fail(PA_ERR_INVALID,
                "%s: at block size %d jobs may cover at most %d tiles (plan with max_piece_tiles <= %d); "
                "the plan's longest covers %d",
                who, pool->block_size, 8 * pool->block_size, 8 * pool->block_size, info->max_job_tiles);
  const auto lay = pagedkv::layout((int64_t)info->num_records * group, pool->head_dim);
  if (info->num_records > 0) {
    if (!workspace) return fail(PA_ERR_INVALID, "%s: workspace is NULL but the plan has records", who);
    if (!pagedkv::aligned(workspace, 256)) return fail(PA_ERR_INVALID, "%s: workspace not 256-byte aligned", who);
    if (workspace_bytes < lay.total)
      return fail(PA_ERR_INVALID, "%s: workspace %zu bytes < %zu needed", who, workspace_bytes, lay.total);
  }
  pagedkv::DecodeArgs a{};
  a.k = pool->k;
  a.v = pool->v;
  a.q = q;
  a.new_k = new_key;
  a.new_v = new_value;
  a.out = out;
  a.tables = block_tables;
  a.lens = context_lens;
  const char* pb = static_cast<const char*>(plan);
  a.jobs = reinterpret_cast<const pa_decode_job*>(pb + info->jobs_at);
  a.merges = reinterpret_cast<const pa_decode_merge*>(pb + info->merges_at);
  a.groups = info->num_groups > 0 ? reinterpret_cast<const pa_decode_group*>(pb + info->groups_at) : nullptr;
  a.first_blocks = first_blocks && pool->dtype == PA_BF16 && pool->block_size >= 8
                       ? reinterpret_cast<const int32_t*>(pb + info->first_at)
                       : nullptr;
  a.num_groups = info->num_groups;
  a.wide_jobs = info->wide_jobs;
  char* ws = static_cast<char*>(workspace);
  a.partial_ml = info->num_records > 0 ? reinterpret_cast<float*>(ws + lay.ml) : nullptr;
  a.partial_o = info->num_records > 0 ? reinterpret_cast<float*>(ws + lay.o) : nullptr;
  a.num_blocks = pool->num_blocks;
  a.block_size = pool->block_size;
  a.num_kv_heads = hkv;
  a.num_q_heads = num_q_heads;
  a.group = group;
  a.head_dim = pool->head_dim;
  a.max_blocks = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.num_workgroups = info->num_workgroups;
  a.jobs_per_workgroup = info->jobs_per_workgroup;
  a.num_jobs = info->num_jobs;
  a.num_merges = info->num_merges;
  a.num_records = info->num_records;
  a.out_bf16 = out_dtype == PA_BF16;
  a.scale_log2e = scale * 1.4426950408889634f;
  a.bf16 = pool->dtype == PA_BF16;
  a.shared_kv = (info->flags & PA_DECODE_SHARED_KV) != 0;
  a.fused_loads = fused_mode(pool, new_key, new_value, num_seqs, group, info, &a);
  if (stages & kStageAttention) {
    if (pa_status st = pagedkv::hip_status(pagedkv::launch_decode_attention(a, (hipStream_t)stream), who)) return st;
  }
  if (stages & kStageMerge) return pagedkv::hip_status(pagedkv::launch_decode_merge(a, (hipStream_t)stream), who);
  return PA_OK;
}

}  // namespace pagedkv

using pagedkv::decode_stages;
using pagedkv::kStageAttention;
using pagedkv::kStageMerge;

#define PA_DECODE_ARGS                                                                                   \
  const pa_kv_pool *pool, const void *q, void *out, int32_t out_dtype, const int32_t *block_tables,      \
      int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t num_seqs, int32_t num_q_heads,    \
      float scale, const void *new_key, const void *new_value, const void *plan,                         \
      const pa_decode_plan_info *info, void *workspace, size_t workspace_bytes, void *stream
#define PA_DECODE_PASS                                                                                   \
  pool, q, out, out_dtype, block_tables, max_blocks_per_seq, context_lens, num_seqs, num_q_heads, scale, \
      new_key, new_value, plan, info, workspace, workspace_bytes, stream

extern "C" int32_t pa_decode_fused_loads(const pa_kv_pool* pool, const void* new_key, const void* new_value,
                                         int32_t num_seqs, int32_t num_q_heads, const pa_decode_plan_info* info) {
  if (!pool || !info || num_seqs < 0 || pool->num_kv_heads <= 0 || num_q_heads <= 0 ||
      num_q_heads % pool->num_kv_heads != 0 || (new_key == nullptr) != (new_value == nullptr)) {
    fail(PA_ERR_INVALID, "pa_decode_fused_loads: bad arguments");
    return -1;
  }
  return pagedkv::fused_mode(pool, new_key, new_value, num_seqs, num_q_heads / pool->num_kv_heads, info, nullptr);
}

extern "C" pa_status pa_decode(PA_DECODE_ARGS) {
  return decode_stages(kStageAttention | kStageMerge, "pa_decode", PA_DECODE_PASS);
}

extern "C" pa_status pa_decode_attention(PA_DECODE_ARGS) {
  return decode_stages(kStageAttention, "pa_decode_attention", PA_DECODE_PASS);
}

extern "C" pa_status pa_decode_merge_pieces(PA_DECODE_ARGS) {
  return decode_stages(kStageMerge, "pa_decode_merge_pieces", PA_DECODE_PASS);
}
