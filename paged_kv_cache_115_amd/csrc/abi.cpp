// C-ABI front of libpagedkv: argument validation, the host-side decode plan,
// workspace sizing and dispatch to the HIP kernels.  Nothing here touches
// device memory contents; launches go on the caller's stream and the library
// never synchronizes.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
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

int32_t elem_bytes(int32_t dtype) { return dtype == PA_F32 ? 4 : 2; }

pa_status check_pool(const pa_kv_pool* pool, const char* who) {
  if (!pool) return fail(PA_ERR_INVALID, "%s: pool is NULL", who);
  if (!pool->k || !pool->v) return fail(PA_ERR_INVALID, "%s: pool k/v pointer is NULL", who);
  if (pool->dtype != PA_F32 && pool->dtype != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "%s: dtype %d (supported: 0=f32, 1=bf16)", who, pool->dtype);
  if (pool->num_blocks <= 0 || pool->num_kv_heads <= 0)
    return fail(PA_ERR_INVALID, "%s: num_blocks=%d num_kv_heads=%d must be positive", who,
                pool->num_blocks, pool->num_kv_heads);
  if (pool->block_size != 8 && pool->block_size != 16 && pool->block_size != 32)
    return fail(PA_ERR_UNSUPPORTED, "%s: block_size %d (supported: 8, 16, 32)", who, pool->block_size);
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

// Workspace carve: (max, sum) pairs | unnormalised accumulators.
struct WorkspaceLayout {
  size_t ml, o, total;
};

WorkspaceLayout layout(int64_t num_partials, int64_t hq, int64_t d) {
  WorkspaceLayout w;
  w.ml = 0;
  w.o = round_up(sizeof(float) * 2 * num_partials * hq, 256);
  w.total = w.o + round_up(sizeof(float) * num_partials * hq * d, 256);
  return w;
}

}  // namespace
}  // namespace pagedkv

using pagedkv::fail;

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

extern "C" pa_status pa_decode_plan(const int32_t* context_lens, int32_t num_seqs, int32_t partition_size,
                                    pa_work_item* items, int32_t capacity, int32_t* num_items,
                                    int32_t* num_merges, int32_t* num_partials) {
  if (!num_items || !num_merges || !num_partials || num_seqs < 0 || capacity < 0 ||
      (num_seqs > 0 && !context_lens))
    return fail(PA_ERR_INVALID, "pa_decode_plan: bad arguments");
  if (partition_size < 0 || (partition_size > 0 && partition_size % 16 != 0))
    return fail(PA_ERR_INVALID, "pa_decode_plan: partition_size %d must be 0 or a positive multiple of 16",
                partition_size);
  struct Entry {
    pa_work_item it;
    int32_t tokens;
  };
  std::vector<Entry> work;
  std::vector<pa_work_item> merges;
  work.reserve(num_seqs);
  int64_t partials = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t L = context_lens[s];
    if (L < 0) return fail(PA_ERR_INVALID, "pa_decode_plan: context_lens[%d] = %d < 0", s, L);
    const int32_t parts = (partition_size > 0 && L > 0) ? (L + partition_size - 1) / partition_size : 1;
    const int32_t base = parts > 1 ? (int32_t)partials : -1;
    if (parts > 1) {
      partials += parts;
      merges.push_back(pa_work_item{s, -1, parts, base});
    }
    for (int32_t p = 0; p < parts; ++p) {
      const int32_t tokens = parts > 1 ? std::min(L - p * partition_size, partition_size) : L;
      work.push_back(Entry{pa_work_item{s, p, parts, base}, tokens});
    }
  }
  const int64_t total = (int64_t)work.size() + (int64_t)merges.size();
  if (partials > INT32_MAX / 64 || total > INT32_MAX / 64)
    return fail(PA_ERR_INVALID, "pa_decode_plan: plan too large");
  // Largest first; ties in (sequence, partition) order so the plan is unique.
  std::stable_sort(work.begin(), work.end(), [](const Entry& x, const Entry& y) { return x.tokens > y.tokens; });
  *num_items = (int32_t)work.size();
  *num_merges = (int32_t)merges.size();
  *num_partials = (int32_t)partials;
  if (total > capacity)
    return fail(PA_ERR_INVALID, "pa_decode_plan: capacity %d < %lld entries", capacity, (long long)total);
  for (size_t i = 0; i < work.size(); ++i) items[i] = work[i].it;
  for (size_t i = 0; i < merges.size(); ++i) items[work.size() + i] = merges[i];
  return PA_OK;
}

extern "C" size_t pa_decode_workspace_bytes(int32_t num_partials, int32_t num_q_heads, int32_t head_dim) {
  if (num_partials <= 0 || num_q_heads <= 0 || head_dim <= 0) return 0;
  return pagedkv::layout(num_partials, num_q_heads, head_dim).total;
}

extern "C" pa_status pa_decode(const pa_kv_pool* pool, const void* q, void* out, int32_t out_dtype,
                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                               float scale, const pa_work_item* items, int32_t num_items,
                               int32_t num_merges, int32_t num_partials, int32_t partition_size,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (pa_status st = pagedkv::check_pool(pool, "pa_decode")) return st;
  if (num_seqs < 0 || num_items < 0 || num_merges < 0 || num_partials < 0 || max_blocks_per_seq < 0)
    return fail(PA_ERR_INVALID, "pa_decode: negative size");
  if ((num_merges > 0) != (num_partials > 0))
    return fail(PA_ERR_INVALID, "pa_decode: num_merges %d and num_partials %d disagree", num_merges, num_partials);
  if (num_items == 0) return PA_OK;
  if (num_seqs == 0) return fail(PA_ERR_INVALID, "pa_decode: work items but num_seqs == 0");
  if (!q || !out || !block_tables || !context_lens || !items)
    return fail(PA_ERR_INVALID, "pa_decode: NULL q/out/block_tables/context_lens/items");
  if (max_blocks_per_seq == 0) return fail(PA_ERR_INVALID, "pa_decode: max_blocks_per_seq == 0");
  const int32_t hkv = pool->num_kv_heads;
  if (num_q_heads <= 0 || num_q_heads % hkv != 0)
    return fail(PA_ERR_INVALID, "pa_decode: num_q_heads %d is not a multiple of num_kv_heads %d",
                num_q_heads, hkv);
  const int32_t group = num_q_heads / hkv;
  if (group > 16) return fail(PA_ERR_UNSUPPORTED, "pa_decode: %d query heads per KV head (max 16)", group);
  if (out_dtype != PA_F32 && out_dtype != pool->dtype)
    return fail(PA_ERR_UNSUPPORTED, "pa_decode: out_dtype %d must be f32 or the pool dtype", out_dtype);
  if (partition_size < 0 || (partition_size > 0 && (partition_size % 16 || partition_size % pool->block_size)))
    return fail(PA_ERR_INVALID, "pa_decode: partition_size %d must be 0 or a multiple of 16 and of B=%d",
                partition_size, pool->block_size);
  if (!pagedkv::aligned(q, 16) || !pagedkv::aligned(out, 16) || !pagedkv::aligned(items, 16))
    return fail(PA_ERR_INVALID, "pa_decode: q/out/items must be 16-byte aligned");
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID, "pa_decode: scale is not finite");
  if (((int64_t)num_items + num_merges) * hkv > INT32_MAX)
    return fail(PA_ERR_INVALID, "pa_decode: num_items * num_kv_heads overflows the grid");
  const auto lay = pagedkv::layout(num_partials, num_q_heads, pool->head_dim);
  if (num_partials > 0) {
    if (!workspace) return fail(PA_ERR_INVALID, "pa_decode: workspace is NULL but num_partials > 0");
    if (!pagedkv::aligned(workspace, 256)) return fail(PA_ERR_INVALID, "pa_decode: workspace not 256-byte aligned");
    if (workspace_bytes < lay.total)
      return fail(PA_ERR_INVALID, "pa_decode: workspace %zu bytes < %zu needed", workspace_bytes, lay.total);
  }
  pagedkv::DecodeArgs a{};
  a.k = pool->k;
  a.v = pool->v;
  a.q = q;
  a.out = out;
  a.tables = block_tables;
  a.lens = context_lens;
  a.items = items;
  char* ws = static_cast<char*>(workspace);
  a.partial_ml = num_partials > 0 ? reinterpret_cast<float*>(ws + lay.ml) : nullptr;
  a.partial_o = num_partials > 0 ? reinterpret_cast<float*>(ws + lay.o) : nullptr;
  a.num_blocks = pool->num_blocks;
  a.block_size = pool->block_size;
  a.num_kv_heads = hkv;
  a.num_q_heads = num_q_heads;
  a.group = group;
  a.head_dim = pool->head_dim;
  a.max_blocks = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.partition = partition_size;
  a.num_partials = num_partials;
  a.num_items = num_items;
  a.out_bf16 = out_dtype == PA_BF16;
  a.scale_log2e = scale * 1.4426950408889634f;
  const hipError_t e = pool->dtype == PA_BF16 ? pagedkv::launch_decode_bf16(a, num_merges, (hipStream_t)stream)
                                              : pagedkv::launch_decode_f32(a, num_merges, (hipStream_t)stream);
  return pagedkv::hip_status(e, "pa_decode");
}
