// Host half of one decode step for a serving loop: the block manager's
// append, the table rows and lengths the kernels read, and the decode plan for
// the new lengths, all written into one caller buffer (pinned host memory) so
// that a step needs one upload.  The block manager appends one token to every
// sequence of the batch (mercemay.com "Paged KV Cache Allocation and the Block
// Table", "Blocks, tables, and the indirection": a block is taken when the
// length reaches a multiple of B; "Sharing blocks between sequences": the
// first write into a shared block copies it); the plan schedules the
// attention over the lengths after that append.
#include <algorithm>
#include <cstring>
#include <vector>

#include "internal.h"

using pagedkv::fail;

namespace {

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace

extern "C" pa_status pa_bm_prepare_decode_step(pa_bm* bm, const int64_t* seqs, int32_t num, int32_t max_blocks,
                                               int32_t num_kv_heads, int32_t num_workgroups, int32_t schedule,
                                               int32_t first_blocks, void* buffer, size_t capacity,
                                               pa_decode_step_layout* layout) {
  const char* who = "pa_bm_prepare_decode_step";
  if (!bm || !layout || num < 0 || max_blocks <= 0 || (num > 0 && !seqs) || (capacity > 0 && !buffer) ||
      reinterpret_cast<uintptr_t>(buffer) % 256 != 0)
    return fail(PA_ERR_INVALID, "%s: bad arguments (the buffer must be 256-byte aligned)", who);
  pa_decode_step_layout lay{};
  lay.num_seqs = num;
  lay.max_blocks = max_blocks;
  lay.slots_at = 0;
  lay.cows_at = (int32_t)align_up(sizeof(int64_t) * num, 256);
  lay.lens_at = (int32_t)align_up((size_t)lay.cows_at + 2 * sizeof(int32_t) * num, 256);
  lay.tables_at = (int32_t)align_up((size_t)lay.lens_at + sizeof(int32_t) * num, 256);
  const size_t tables_end = (size_t)lay.tables_at + sizeof(int32_t) * (size_t)num * (size_t)max_blocks;
  lay.plan_at = (int32_t)align_up(tables_end, 256);
  if ((size_t)lay.plan_at > capacity) {
    lay.bytes = lay.plan_at;
    *layout = lay;
    return fail(PA_ERR_INVALID, "%s: the buffer holds %zu bytes, the step needs more than %d", who, capacity,
                lay.plan_at);
  }
  char* buf = static_cast<char*>(buffer);
  int32_t* lens = reinterpret_cast<int32_t*>(buf + lay.lens_at);
  // Lengths after this step's append; the plan is built for them first, so
  // that a buffer too small for it leaves the block manager unchanged.
  if (pa_status st = pagedkv::bm_step_resolve(bm, seqs, num, lens, who)) return st;
  for (int32_t i = 0; i < num; ++i) lens[i] += 1;
  const int32_t B = pa_bm_block_size(bm);
  for (int32_t i = 0; i < num; ++i)
    if ((int64_t)lens[i] > (int64_t)max_blocks * B)
      return fail(PA_ERR_INVALID, "%s: sequence %lld grows to %d tokens, past max_blocks %d of %d slots", who,
                  (long long)seqs[i], lens[i], max_blocks, B);
  pa_decode_plan_info info{};
  // Below 8 slots per block the kernels' jobs cover at most 8 * B tiles.
  const int32_t max_piece_tiles = B < 8 ? 8 * B : 0;
  // With plan reuse (pa_bm_set_plan_reuse), the last step's plan advances to
  // these lengths when it can; otherwise a new one is built (and kept).
  pagedkv::StepPlanCache& pc = pagedkv::step_plan_cache(bm);
  const size_t plan_room = capacity - (size_t)lay.plan_at;
  bool reused = false;
  if (pc.max_advances > 0 && pc.valid && pc.advances < pc.max_advances && pc.num_kv_heads == num_kv_heads &&
      pc.num_workgroups == num_workgroups && pc.schedule == schedule && pc.max_piece == max_piece_tiles &&
      pc.seqs.size() == (size_t)num && std::equal(pc.seqs.begin(), pc.seqs.end(), seqs)) {
    const pa_status as = pa_decode_plan_advance(pc.plan.data(), &pc.info, lens, num, max_piece_tiles);
    if (as == PA_OK && (size_t)pc.info.bytes <= plan_room) {
      std::memcpy(buf + lay.plan_at, pc.plan.data(), (size_t)pc.info.bytes);
      info = pc.info;
      pc.advances += 1;
      reused = true;
    } else if (as != PA_OK && as != PA_REPLAN) {
      pc.valid = false;
      return as;
    }
  }
  if (!reused) {
    pc.valid = false;
    const pa_status ps = pa_decode_plan_schedule(lens, num, num_kv_heads, num_workgroups, max_piece_tiles, schedule,
                                                 buf + lay.plan_at, plan_room, &info);
    if (ps != PA_OK) {
      lay.bytes = lay.plan_at + info.bytes;
      *layout = lay;
      return ps;  // message left by the planner
    }
    if (pc.max_advances > 0) {
      pc.plan.assign(buf + lay.plan_at, buf + lay.plan_at + info.bytes);
      pc.info = info;
      pc.seqs.assign(seqs, seqs + num);
      pc.num_kv_heads = num_kv_heads;
      pc.num_workgroups = num_workgroups;
      pc.schedule = schedule;
      pc.max_piece = max_piece_tiles;
      pc.advances = 0;
      pc.valid = true;
    }
  }
  // The append (all or nothing).
  int64_t* slots = reinterpret_cast<int64_t*>(buf + lay.slots_at);
  int32_t* cows = reinterpret_cast<int32_t*>(buf + lay.cows_at);
  int32_t n_cows = 0;
  if (pa_status st = pagedkv::bm_step_append(bm, seqs, num, slots, cows, &n_cows, who)) {
    pc.valid = false;
    return st;
  }
  // Table rows: only the first ceil(L / B) entries, the ones the kernels
  // read; the rest of each row keeps whatever the buffer held.
  int32_t* tables = reinterpret_cast<int32_t*>(buf + lay.tables_at);
  if (pa_status st = pagedkv::bm_step_tables(bm, num, tables, max_blocks, who)) return st;
  if (first_blocks && info.num_jobs > 0) {
    if (pa_status st = pa_decode_plan_first_blocks(buf + lay.plan_at, &info, tables, max_blocks, num, B)) return st;
  }
  lay.n_cows = n_cows;
  lay.plan = info;
  lay.bytes = lay.plan_at + info.bytes;
  *layout = lay;
  return PA_OK;
}
