/*
 * pagedkv.h - C ABI of libpagedkv: decode attention over a paged KV cache on
 * AMD Instinct MI355X (gfx950), plus the host-side block manager that hands
 * out the cache's blocks.
 *
 * The method (PagedAttention's memory layout):
 *   - the KV cache is one preallocated pool of fixed-size blocks of B token
 *     slots, keys and values in separate pools of identical shape
 *     [num_blocks][B][num_kv_heads][head_dim]
 *     (aicassindra.com "tm_paged_attention_deep", "Anatomy of a KV block";
 *      llminference.xinbetween.com S06 "PagedAttention", "Implementation");
 *   - each sequence owns a block table mapping logical block t / B to a
 *     physical block; token t lives at flat slot table[t / B] * B + t % B
 *     (synapticradio.com "The KV Cache Is an Allocator Problem", equation in
 *      "What the trace shows");
 *   - blocks come from a free list on demand, carry reference counts so that
 *     sequences can share a prefix, and are copied on the first write into a
 *     shared block (mercemay.com "Paged KV Cache Allocation and the Block
 *     Table", "Blocks, tables, and the indirection" and "Sharing blocks
 *     between sequences");
 *   - the attention kernel walks the table itself instead of gathering blocks
 *     into a contiguous copy first (S06 "Why this needed a custom CUDA kernel";
 *     mercemay.com "What the design costs").
 *
 * Conventions for every GPU entry point:
 *   - all array arguments are DEVICE pointers owned by the caller; the
 *     library never allocates device memory and never synchronizes;
 *   - work is enqueued on `stream` (a hipStream_t; NULL = the null stream)
 *     and calls on one stream run in call order;
 *   - arguments the host can check (null pointers, sizes, dtypes, alignment)
 *     are checked before anything is enqueued; on failure nothing is launched
 *     and a message is left for pa_last_error();
 *   - contents of device arrays (slot values, table entries, lengths) are
 *     preconditions, stated per call; the kernels never read outside the
 *     arrays when the preconditions hold;
 *   - launch failures return PA_ERR_HIP.
 * Supported shapes: dtype F32 or BF16; head_dim 64 or 128 for F32, 128 for
 * BF16; block_size 1, 2, 4, 8, 16 or 32 (below 8, a plan's jobs cover
 * at most 8 * B tiles); num_q_heads a multiple of num_kv_heads with a group
 * of at most 16 query heads per KV head.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID = -1,     /* bad argument (null, size, alignment, precondition seen on host) */
  PA_ERR_UNSUPPORTED = -2, /* valid but not implemented (dtype, head_dim, block size, group) */
  PA_ERR_OOM = -3,         /* block manager: not enough free blocks; state unchanged */
  PA_ERR_NOT_FOUND = -4,   /* block manager: unknown sequence */
  PA_ERR_HIP = -5,         /* a HIP runtime call failed */
  PA_REPLAN = 1            /* pa_decode_plan_advance: the plan cannot follow the new lengths; build a new one */
} pa_status;

typedef enum { PA_F32 = 0, PA_BF16 = 1 } pa_dtype;

/* One layer's KV pool.  k and v each hold num_blocks * block_size *
 * num_kv_heads * head_dim elements of `dtype`, contiguous, in the order
 * [block][slot][kv_head][dim], 16-byte aligned.  Owned by the caller. */
typedef struct pa_kv_pool {
  void* k;
  void* v;
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t dtype; /* pa_dtype */
} pa_kv_pool;

/* Message describing the last non-OK status returned on this thread. */
const char* pa_last_error(void);

/* ---------------------------------------------------------------------------
 * pa_reshape_and_cache - write new tokens' keys and values into their slots.
 *
 * The device half of the append step: pool slot slot_mapping[i] receives
 * key[i] and value[i] (mercemay.com "Blocks, tables, and the indirection",
 * the append listing's cache write at physical * block_size + slot).
 *   key, value   : device, [num_tokens][num_kv_heads][head_dim] of pool dtype,
 *                  contiguous, 16-byte aligned.
 *   slot_mapping : device int64 [num_tokens]; flat slot = block * B + offset.
 *                  A negative slot skips that token (padding).
 * Preconditions: every non-negative slot < num_blocks * block_size; no slot
 * repeats within one call.  The copy is bit-exact.  num_tokens == 0 is a
 * no-op.
 * ------------------------------------------------------------------------- */
pa_status pa_reshape_and_cache(const pa_kv_pool* pool, const void* key, const void* value,
                               const int64_t* slot_mapping, int32_t num_tokens, void* stream);

/* ---------------------------------------------------------------------------
 * pa_copy_blocks - copy-on-write duplication of whole blocks.
 *
 * For every pair p: block pairs[2p+1] of both pools becomes a bit-exact copy
 * of block pairs[2p] (aicassindra.com "Copy-on-write for shared prefixes":
 * the one block at the point of divergence is copied for the writer).
 *   pairs : device int32 [num_pairs][2] = (src, dst).
 * Preconditions: ids in [0, num_blocks); destinations distinct and never a
 * source in the same call.  num_pairs == 0 is a no-op.
 * ------------------------------------------------------------------------- */
pa_status pa_copy_blocks(const pa_kv_pool* pool, const int32_t* pairs, int32_t num_pairs,
                         void* stream);

/* ---------------------------------------------------------------------------
 * pa_swap_blocks - copy whole blocks between the device pool and a pool in
 * pinned host memory: the swap half of preemption.
 *
 * When blocks run out, the scheduler can stop admitting, copy a sequence's
 * cache out to host memory and back later, or discard and recompute it
 * (mercemay.com "Paged KV Cache Allocation and the Block Table", "Three ways
 * contiguous reservation loses memory" and the end of "Blocks, tables, and
 * the indirection"; llminference.xinbetween.com S06, third exercise).  This
 * call is the copy; pa_bm_swap_out / pa_bm_swap_in produce its pairs.
 *   device_pool : the layer's pool, device memory, as for every other call.
 *   host_pool   : caller-owned pool of the same block_size, num_kv_heads,
 *                 head_dim and dtype whose k and v are PINNED host memory
 *                 (hipHostMalloc, or a tensor made with pin_memory=True),
 *                 host_pool->num_blocks blocks each, 16-byte aligned.
 *   pairs       : HOST int32 [num_pairs][2] = (src, dst), read during the
 *                 call only.  PA_SWAP_OUT: src a device block, dst a host
 *                 block; PA_SWAP_IN: src a host block, dst a device block.
 *   engine      : PA_SWAP_ENGINE_KERNEL - kernels move the blocks through
 *                 the host memory's device mapping, up to 240 pairs per
 *                 launch (the fast path: PCIe-bound whatever the layout);
 *                 PA_SWAP_ENGINE_MEMCPY - one hipMemcpyAsync per pool for
 *                 every run of pairs that continue each other on both sides
 *                 (src + 1, dst + 1); per-call cost dominates unless the
 *                 runs are long.
 * Checked on the host before anything is enqueued (PA_ERR_INVALID): ids
 * inside their pools, destinations distinct, both host arrays pinned and
 * device-mapped over their whole extent, both device arrays device memory.
 * The copy is bit-exact.  It is ordered on `stream` like every other call:
 * the host pool holds the swapped-out bytes only once the stream has been
 * synchronized, and host blocks a swap-in reads must not be rewritten by the
 * host before that.  num_pairs == 0 is a no-op.
 * ------------------------------------------------------------------------- */
#define PA_SWAP_OUT 0
#define PA_SWAP_IN 1
#define PA_SWAP_ENGINE_KERNEL 0
#define PA_SWAP_ENGINE_MEMCPY 1
pa_status pa_swap_blocks(const pa_kv_pool* device_pool, const pa_kv_pool* host_pool, const int32_t* pairs,
                         int32_t num_pairs, int32_t direction, int32_t engine, void* stream);

/* ---------------------------------------------------------------------------
 * Decode attention.
 *
 * For each sequence s with L = context_lens[s] tokens and each query head h,
 * with KV head g = h / (num_q_heads / num_kv_heads):
 *   out[s][h] = sum_t softmax_t(scale * <q[s][h], K_t[g]>) * V_t[g],
 * where token t's K/V row is read through the block table
 * (S06 "Implementation", the paged_attention excerpt; aicassindra.com
 *  "The block table: logical to physical mapping").  L counts the token
 * written this step; L == 0 yields zeros.
 *
 * Scheduling.  A sequence's context is cut into 16-token tiles; a job is a
 * piece of consecutive tiles of one (sequence, block of four KV heads)
 * stream, and each persistent workgroup runs a list of jobs.  The host plan
 * (pa_decode_plan, which knows the lengths) builds two schedules and keeps
 * the one whose busiest compute unit costs less: equal-work chunks of the
 * streams laid end to end, cut at tile boundaries (PA_SCHEDULE_CHUNKS), or
 * pieces of at most two workgroups' shares placed largest first on the least
 * loaded compute unit, i.e. pair of workgroups {b, b + nwg/2}, each
 * workgroup then running its pieces smallest first (PA_SCHEDULE_LPT).  The
 * four waves of a workgroup take the four KV heads
 * of each job, so the head slices of a slot row are read together.  A stream
 * cut into several pieces leaves one (max, sum, accumulator) record per
 * piece and KV head in the workspace; a second launch on the same stream
 * merges the records by log-sum-exp in piece order.  The plan is one byte
 * buffer that the caller copies to the device with the other step inputs.
 * ------------------------------------------------------------------------- */
typedef struct pa_decode_job {
  int32_t seq;         /* sequence index */
  int32_t tile_begin;  /* first 16-token tile of the piece */
  int32_t tile_count;  /* tiles in the piece, 1..64; 0 marks an empty slot of the job table */
  int32_t head_block;  /* KV heads 4*head_block .. 4*head_block + 3 */
  int32_t part;        /* piece index within the (sequence, head block) stream */
  int32_t num_parts;   /* pieces of the stream (1: the job writes the output) */
  int32_t record_base; /* workspace record of KV head 4*head_block + w, piece p: record_base + w * num_parts + p */
  int32_t context_len; /* context_lens[seq] as planned: the kernels take the length from here */
} pa_decode_job;

typedef struct pa_decode_merge {
  int32_t seq;
  int32_t kv_head;
  int32_t num_parts;   /* 0: the sequence is empty and its output is zero */
  int32_t record_base; /* first record of this (sequence, KV head), pieces consecutive */
} pa_decode_merge;

typedef struct pa_decode_plan_info {
  int32_t num_workgroups; /* grid of the attention launch */
  int32_t num_jobs;
  int32_t num_merges;     /* grid of the merge launch (0: no merge launch) */
  int32_t num_records;    /* workspace records, one per (sequence, KV head, piece) of cut streams */
  int32_t num_kv_heads;   /* KV heads the plan was made for */
  int32_t jobs_per_workgroup; /* rows of the job table */
  int32_t jobs_at;        /* byte offset (0) of the job table, pa_decode_job [jobs_per_workgroup][num_workgroups]:
                             slot k of workgroup b at k * num_workgroups + b; a workgroup's jobs fill slots
                             0, 1, ... in order, the rest are empty (tile_count 0) */
  int32_t merges_at;      /* byte offset of pa_decode_merge [num_merges] */
  int32_t bytes;          /* total plan bytes */
  int32_t flags;          /* PA_DECODE_* bits; pa_decode_plan sets 0, the caller may set them */
  int32_t schedule;       /* PA_SCHEDULE_* the plan was built with (informational) */
  int32_t num_groups;     /* prefix-group descriptors (pa_decode_plan_prefix; 0 otherwise) */
  int32_t groups_at;      /* byte offset of pa_decode_group [num_groups] */
  int32_t group_size;     /* largest prefix group planned (members sharing one read of the prefix) */
  int32_t first_at;       /* byte offset of int32 [jobs_per_workgroup * num_workgroups][4]: per job slot, the
                             table entries of the job's first two tiles (pa_decode_plan_first_blocks) */
  int32_t first_block_size; /* block size those entries were written for (0: not written) */
  int32_t num_tiles;      /* 16-token tiles the jobs read, summed over jobs (with the append fused,
                             pa_decode picks how tiles are loaded from the tiles per sequence and the
                             query heads per KV head) */
  int32_t num_seqs;       /* sequences the plan was made for: pa_decode refuses another num_seqs */
  int32_t max_context_len; /* longest context planned: pa_decode refuses tables too short for it */
  int32_t wide_jobs;      /* jobs with PA_JOB_WIDE (pa_decode_plan_prefix; 0 otherwise) */
  uint64_t lens_digest;   /* digest of the planned context lengths (pa_decode_plan_check_lens) */
  int32_t max_job_tiles;  /* tiles of the longest job (block sizes below 8 allow at most 8 * B) */
  int32_t reserved2;
} pa_decode_plan_info;

/* A job whose head_block field has this bit reads a prefix shared by the
 * members of a prefix group once for all of them: seq is the group's first
 * member (whose table is read), record_base indexes the pa_decode_group,
 * part is the piece of the shared prefix. */
#define PA_JOB_SHARED (1 << 16)

/* With PA_JOB_SHARED: the job reads the shared prefix for a set of up to four
 * prefix groups of one key group, on one KV head (the low 16 bits of
 * head_block are the KV head g, not a head block).  The workgroup's four
 * wavefronts read the job's tiles four at a time, one tile each, exchange
 * them through LDS, and wavefront w scores all four against group w of the
 * set: every prefix tile of the head is read once for the whole set.
 * record_base indexes the descriptor of the set's first group for head
 * block g / 4; group k of the set has descriptor record_base + k *
 * ceil(num_kv_heads / 4).  num_parts packs the set's shape: bits 0-7 the
 * groups in the set, 8-15 the members of each group but the last, 16-23 the
 * members of the last.  part is the piece of the shared prefix, the same for
 * every member of the set (S06 "What's next": one read of a prefix however
 * many requests share it). */
#define PA_JOB_WIDE (1 << 17)

/* One prefix group for one head block: up to four sequences whose first
 * blocks are the same physical blocks.  Member i's record for KV head
 * 4*head_block + w and piece p is record_base[i] + w * num_parts[i] + p;
 * the shared prefix pieces are its parts 0, 1, ..., its own tiles follow. */
typedef struct pa_decode_group {
  int32_t num_members;
  int32_t head_block;
  int32_t seq[4];
  int32_t record_base[4];
  int32_t num_parts[4];
  int32_t reserved[2];
} pa_decode_group;

/* Schedules pa_decode_plan builds and chooses between. */
#define PA_SCHEDULE_AUTO (-1) /* build both, keep the cheaper (pa_decode_plan) */
#define PA_SCHEDULE_CHUNKS 0  /* equal-work chunks of the concatenated tile streams */
#define PA_SCHEDULE_LPT 1     /* pieces of at most a workgroup's share, largest first onto the least loaded */

/* flags bit: some physical blocks are named by more than one sequence of the
 * batch (forked, shared prefixes; pa_bm_get_stats().shared_blocks > 0).  K/V
 * loads then keep blocks in the caches for the other readers.  Without it
 * every K/V byte is read once and the loads stream past the caches, which is
 * faster when nothing is shared.  Either setting gives identical results. */
#define PA_DECODE_SHARED_KV 1

/* flags bit, set by pa_decode_plan_first_blocks: the plan holds the table
 * entries of every job's first two tiles, so the attention launch issues its
 * first tile loads from the job records without waiting for a table load.
 * The entries must be those of the tables passed to pa_decode (bf16 pools;
 * fp32 ignores them). */
#define PA_DECODE_FIRST_BLOCKS 2

/* Write the first-tile table entries into a plan from the HOST copy of the
 * block tables pa_decode will read (tables: int32 [num_seqs][max_blocks], the
 * same rows), for pools of block_size; sets PA_DECODE_FIRST_BLOCKS and
 * info->first_block_size.  Serving loops export the tables on the host
 * anyway (pa_bm_export); the entries are only valid for those tables.  Block
 * sizes below 8 (a tile spans more blocks than a job slot's four entries)
 * write nothing and leave the flag clear.
 * PA_ERR_INVALID for an inconsistent info or a job naming a sequence past
 * num_seqs. */
pa_status pa_decode_plan_first_blocks(void* plan, pa_decode_plan_info* info, const int32_t* tables,
                                      int32_t max_blocks, int32_t num_seqs, int32_t block_size);

/* Persistent workgroups that fit the current device at full occupancy (all
 * resident at once): compute units times resident decode workgroups per unit.
 * Returns 0 and sets pa_last_error when no device can be queried. */
int32_t pa_decode_default_workgroups(void);

/* pa_decode_plan - build the schedule on the host.
 *   context_lens    : HOST int32 [num_seqs], each >= 0.
 *   num_kv_heads    : KV heads of the pool.
 *   num_workgroups  : persistent workgroups (pa_decode_default_workgroups()).
 *   max_piece_tiles : longest job in tiles, 1..64; 0: the schedule's default
 *                     (see pa_decode_plan_schedule).
 *   plan            : HOST output buffer of `capacity` bytes (8-byte aligned).
 *   info            : filled on success, and with info->bytes set when the
 *                     capacity is too small (PA_ERR_INVALID) so the caller can
 *                     size a second call.
 * Deterministic: the same inputs give the same bytes. */
pa_status pa_decode_plan(const int32_t* context_lens, int32_t num_seqs, int32_t num_kv_heads,
                         int32_t num_workgroups, int32_t max_piece_tiles, void* plan,
                         size_t capacity, pa_decode_plan_info* info);

/* pa_decode_plan with the schedule named: PA_SCHEDULE_AUTO (what
 * pa_decode_plan does), PA_SCHEDULE_CHUNKS or PA_SCHEDULE_LPT.
 *
 * PA_SCHEDULE_CHUNKS: the (sequence, head block) tile streams, in alternating
 *   length order (longest, shortest, second longest, ...), are laid end to
 *   end and cut into one chunk of equal cost per workgroup (cost = tokens, plus
 *   4 per stream start), at tile boundaries: a tile goes to the workgroup
 *   whose share holds its midpoint.  A stream's records are per stream.
 * PA_SCHEDULE_LPT: each sequence is cut into near-equal pieces of at most
 *   max_piece_tiles tiles (0: twice the average tiles per workgroup,
 *   clamped to [4, 64]); one job per (piece, head block); jobs, largest
 *   first, go to the least-loaded compute unit (pair of workgroups b and
 *   b + num_workgroups/2), each pair's jobs are split between its two
 *   workgroups by a model of their uneven shares of the compute unit, and
 *   each workgroup runs its jobs smallest first.  Fewer jobs, coarser balance.
 * Automatic choice: the schedule whose busiest compute unit (the two
 * workgroups of a pair together; the busiest workgroup for an odd grid)
 * costs less, with a job charged as 56 tokens (calibrated on MI355X), the
 * chunks on a tie. */
pa_status pa_decode_plan_schedule(const int32_t* context_lens, int32_t num_seqs, int32_t num_kv_heads,
                                  int32_t num_workgroups, int32_t max_piece_tiles, int32_t schedule, void* plan,
                                  size_t capacity, pa_decode_plan_info* info);

/* pa_decode_plan_prefix - chunk schedule with shared prefixes read once.
 *
 * Cascade decode for forked sequences (S06 "Copy-on-write, for free": n
 * samples of one prompt hold the same prefix blocks): the tiles of a prefix
 * that several sequences of the batch share are read once per head block
 * and scored against the queries of all members together (up to
 * min(4, 16 / G) members per group, G = num_q_heads / num_kv_heads, so that
 * members x G query columns fill one 16-wide MFMA), and every member's own
 * tiles are scheduled as usual; the merge launch combines the shared and the
 * own pieces by log-sum-exp.
 *   prefix_group  : HOST int32 [num_seqs]: sequences with the same value
 *                   >= 0 share their first prefix_tokens tokens (the same
 *                   physical blocks); -1: no sharing.  Larger groups are cut
 *                   into groups of the largest allowed size, in sequence order.
 *   prefix_tokens : HOST int32 [num_seqs]: tokens shared by the sequence's
 *                   group.  A group shares the smallest value of its members,
 *                   rounded down to a multiple of 16 and kept below every
 *                   member's context length (so the token written this step is
 *                   never in the shared part).
 * Other arguments as pa_decode_plan.  Groups of one member, or a shared part
 * of less than one tile, are planned as unshared sequences.  The plan sets
 * PA_DECODE_SHARED_KV in info->flags only when some shared block is still
 * read by more than one job (a group larger than the largest allowed size,
 * or one without a whole shared tile); otherwise every block is read once
 * and the loads stream past the caches.
 * Precondition (not checked): the members' block tables hold the same block
 * ids for the shared tokens; the shared blocks are read through the first
 * member's table. */
pa_status pa_decode_plan_prefix(const int32_t* context_lens, int32_t num_seqs, int32_t num_kv_heads,
                                int32_t num_q_heads, int32_t num_workgroups, int32_t max_piece_tiles,
                                const int32_t* prefix_group, const int32_t* prefix_tokens, void* plan,
                                size_t capacity, pa_decode_plan_info* info);

/* PA_OK when the plan was made for exactly these context lengths (HOST int32
 * [num_seqs]), PA_ERR_INVALID with the first differing sequence otherwise.
 * Plans are made per step, and lengths grow by one every step: a plan kept
 * from an earlier step describes other lengths. */
pa_status pa_decode_plan_check_lens(const pa_decode_plan_info* info, const int32_t* context_lens, int32_t num_seqs);

/* pa_decode_plan_advance - carry a plan to the next step's lengths.
 * Between decode steps every sequence grows by one token (S06
 * "Implementation": the length passed per call; mercemay.com "Blocks,
 * tables, and the indirection": a new block only every B tokens), so most
 * sequences keep their tiles and the rest gain one.  This updates, in place,
 * a plan made by pa_decode_plan / pa_decode_plan_schedule (HOST plan bytes
 * and info) for context_lens (HOST int32 [num_seqs]):
 *   - every job record takes its sequence's new length;
 *   - a sequence whose tile count grew by one extends, in every head block,
 *     the job holding its last tile (its records and merge rows are kept);
 *   - the info's tile count, longest job, longest context and length digest
 *     follow; PA_DECODE_FIRST_BLOCKS is cleared (call
 *     pa_decode_plan_first_blocks again for the new tables).
 * The work stays where it was placed, so the balance drifts with the steps:
 * callers rebuild every few steps.  PA_REPLAN, with the plan unchanged, when
 * the plan cannot follow: a prefix plan (num_groups > 0), a sequence that
 * lost tiles, gained more than one, or went from empty to non-empty, or an
 * extended job longer than max_job_tiles (0: 64; block sizes below 8 need
 * 8 * B).  PA_ERR_INVALID for another num_seqs, a negative length or an
 * inconsistent plan.  O(jobs + num_seqs). */
pa_status pa_decode_plan_advance(void* plan, pa_decode_plan_info* info, const int32_t* context_lens,
                                 int32_t num_seqs, int32_t max_job_tiles);

/* How pa_decode, with these arguments, loads the tiles of its attention
 * launch, for diagnostics and benchmark reports: 0 without new rows; with
 * them (the append fused) 4 = every tile by buffer loads at 32-bit offsets
 * in a 4 GiB window holding the pool and the new rows (block sizes 16 and 32,
 * when both pools' windows fit: place the step's new rows within 4 GiB of the
 * pools for it); otherwise 1 = the tile holding a sequence's new token on a
 * path of its own (long contexts), 2 = every tile through per-lane 64-bit
 * addresses.
 * Depends on the plan's tiles per sequence, the query heads per KV head, the
 * block size and the addresses; reads no memory.  -1 (pa_last_error) for bad
 * arguments. */
int32_t pa_decode_fused_loads(const pa_kv_pool* pool, const void* new_key, const void* new_value, int32_t num_seqs,
                              int32_t num_q_heads, const pa_decode_plan_info* info);

/* Bytes of device workspace pa_decode needs for a plan (0 when no sequence is
 * cut).  The workspace needs no initialisation; it carries records from the
 * attention launch to the merge launch of one call, so calls that may overlap
 * in time (different streams) must not share one. */
size_t pa_decode_workspace_bytes(const pa_decode_plan_info* info, int32_t num_q_heads,
                                 int32_t head_dim);

/* pa_decode - paged decode attention for one batch.
 *   q            : device [num_seqs][num_q_heads][head_dim], pool dtype.
 *   out          : device [num_seqs][num_q_heads][head_dim], out_dtype
 *                  (PA_F32, or the pool dtype: rounded to nearest even).
 *   block_tables : device int32 [num_seqs][max_blocks_per_seq]; the values
 *                  of entries past ceil(L / B) are never used (they may be
 *                  loaded with the row, and need not be valid block ids).
 *   context_lens : device int32 [num_seqs].
 *   scale        : multiplies q.k before the softmax (1/sqrt(head_dim) for
 *                  standard attention; S06 "Implementation").
 *   new_key, new_value : device [num_seqs][num_kv_heads][head_dim], pool
 *                  dtype, 16-byte aligned, or both NULL.  When given, the
 *                  step's append is fused into the call: for every sequence
 *                  with L > 0 the attention launch takes the token at
 *                  logical position L - 1 from these arrays, and the merge
 *                  launch stores it into its slot, table[(L-1)/B] * B +
 *                  (L-1) % B, which is what pa_reshape_and_cache would have
 *                  written there with the slots the block manager hands out.
 *                  Its block must not be shared (the host's copy-on-write has
 *                  run; pa_copy_blocks precedes this call on the stream).
 *   plan, info   : device copy of the bytes pa_decode_plan wrote for the same
 *                  context lengths and num_kv_heads, and its host-side info.
 *   workspace    : device, >= pa_decode_workspace_bytes(info, ...), 256-byte
 *                  aligned; may be NULL when info->num_records == 0.
 * Checked on the host: num_seqs equals the plan's num_seqs and
 * max_blocks_per_seq * B covers the plan's longest context (PA_ERR_INVALID).
 * Preconditions: context_lens equal those given to pa_decode_plan; the first
 * ceil(L / B) table entries of each sequence are in [0, num_blocks).  The
 * lengths are checked on the device as well: every job compares its
 * sequence's context_lens entry with the length it was planned for, and a
 * sequence whose entry differs gets NaN in every output element (never
 * plausible numbers computed over other lengths).  pa_validate_decode checks
 * every precondition on host copies.  Results are deterministic: the order of
 * every floating-point reduction depends only on logical token positions and
 * on the plan, never on physical block ids or on timing. */
pa_status pa_decode(const pa_kv_pool* pool, const void* q, void* out, int32_t out_dtype,
                    const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                    float scale, const void* new_key, const void* new_value, const void* plan,
                    const pa_decode_plan_info* info, void* workspace, size_t workspace_bytes,
                    void* stream);

/* The two launches of pa_decode as separate calls, with the same arguments
 * and checks: pa_decode_attention writes the output of every sequence that
 * is not cut and the records of cut ones; pa_decode_merge_pieces then writes the
 * output of cut and empty sequences and, with new_key/new_value, the appended
 * rows into the pool.  Issued in that order on one stream
 * they equal pa_decode; between them the caller may record events (to time
 * the attention launch alone) or enqueue other work that touches neither the
 * output, the workspace nor the appended rows' slots.  Either returns PA_OK
 * without launching when it has nothing to do. */
pa_status pa_decode_attention(const pa_kv_pool* pool, const void* q, void* out, int32_t out_dtype,
                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                              float scale, const void* new_key, const void* new_value, const void* plan,
                              const pa_decode_plan_info* info, void* workspace, size_t workspace_bytes,
                              void* stream);
pa_status pa_decode_merge_pieces(const pa_kv_pool* pool, const void* q, void* out, int32_t out_dtype,
                                 const int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                                 float scale, const void* new_key, const void* new_value, const void* plan,
                                 const pa_decode_plan_info* info, void* workspace, size_t workspace_bytes,
                                 void* stream);

/* pa_decode_noalloc - pa_decode for callers that cannot allocate device
 * memory: code under stream capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments and checks as pa_decode without the
 * workspace: the records of cut sequences go to a device array inside the
 * library of PA_NOALLOC_SCRATCH_BYTES (32 MiB), one per device, held from the
 * device's first call until the process ends.  The call allocates nothing.
 * A plan whose workspace (pa_decode_workspace_bytes) exceeds the array is
 * refused with PA_ERR_INVALID before anything touches the device.  The array
 * needs no initialisation (each call writes every record it reads) and keeps
 * the last call's contents; all calls on one device share it, so calls that
 * may overlap in time on one device (different streams) race: order them on
 * one stream. */
#define PA_NOALLOC_SCRATCH_BYTES (32u << 20)
pa_status pa_decode_noalloc(const pa_kv_pool* pool, const void* q, void* out, int32_t out_dtype,
                            const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                            int32_t num_seqs, int32_t num_q_heads, float scale, const void* new_key,
                            const void* new_value, const void* plan, const pa_decode_plan_info* info, void* stream);

/* ---------------------------------------------------------------------------
 * Measurement aid (not on the decode path).
 *
 * pa_probe_read - read `bytes` of device memory at `src` once, as a plain
 * stream: num_workgroups workgroups of 256 threads, each reading one
 * contiguous share with 16-byte non-temporal loads, the decode tiles' load
 * width and cache policy.  Its rate is the achievable read bandwidth the
 * decode launch is compared with, beside the published HBM peak.
 *   src  : device, 16-byte aligned; bytes a multiple of 16.
 *   sink : device uint32 [num_workgroups * 256]; written only for a value
 *          the probe's inputs never produce (it keeps the loads alive).
 * PA_ERR_INVALID for NULL pointers, misalignment or num_workgroups <= 0.
 * ------------------------------------------------------------------------- */
pa_status pa_probe_read(const void* src, size_t bytes, int32_t num_workgroups, void* sink, void* stream);

/* ---------------------------------------------------------------------------
 * Validation of device-resident preconditions on HOST copies (a debug aid).
 *
 * The GPU calls check what the host can see (sizes, pointers, alignment) but
 * take the contents of device arrays on trust: a table entry past the pool is
 * clamped into it, and a wrong block or count then shows up as wrong
 * attention scores rather than a crash (mercemay.com "Sharing blocks between
 * sequences"; S06 "Reference counts must be exact").  These calls check those
 * contents on host copies the caller holds anyway (the block manager exports
 * the tables and lengths it uploads) and return PA_ERR_INVALID with the first
 * violation in pa_last_error.  They read nothing on the device and cost time
 * linear in their inputs, so a serving loop runs them only when debugging.
 * ------------------------------------------------------------------------- */

/* Slots of one pa_reshape_and_cache call (HOST int64 [num_tokens]): every
 * non-negative slot below num_blocks * block_size, none repeated. */
pa_status pa_validate_slots(const int64_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                            int32_t block_size);

/* Pairs of one pa_copy_blocks call (HOST int32 [num_pairs][2] = (src, dst)):
 * ids in [0, num_blocks), destinations distinct and never a source. */
pa_status pa_validate_copy_pairs(const int32_t* pairs, int32_t num_pairs, int32_t num_blocks);

/* The inputs of one pa_decode call, from HOST copies: tables int32
 * [num_seqs][max_blocks_per_seq], context_lens int32 [num_seqs], and the
 * plan's bytes as built on the host (plan, info).  Checks that the plan was
 * made for these lengths (its digest and every job's recorded length), that
 * every L fits its table row, that the first ceil(L / B) entries of every row
 * are in [0, num_blocks), and, with fused_append != 0, that no other sequence
 * of the batch names the block that receives a sequence's appended token
 * (the block manager's copy-on-write must have given the writer its own). */
pa_status pa_validate_decode(const pa_kv_pool* pool, const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* context_lens, int32_t num_seqs, const void* plan,
                             const pa_decode_plan_info* info, int32_t fused_append);

/* ---------------------------------------------------------------------------
 * Host block manager (plain C++ on the CPU; not thread-safe: one scheduler
 * thread owns an instance).  Tracks per-sequence block tables and lengths,
 * per-block reference counts and one free list
 * (S06 "The solution", the BlockManager listing; mercemay.com "Sharing
 *  blocks between sequences").
 *
 * Free list: blocks leave in `initial_order` (initial_order[0] first; NULL =
 * ascending ids, as the S06 simulator's tables show); a retired block goes
 * back on top and is the next one handed out.
 * ------------------------------------------------------------------------- */
typedef struct pa_bm pa_bm;

typedef struct pa_bm_stats {
  int32_t num_blocks;
  int32_t free_blocks;
  int32_t used_blocks;
  int32_t num_seqs;
  int64_t logical_tokens; /* sum of sequence lengths (shared tokens count per sharer) */
  int32_t shared_blocks;  /* blocks named by more than one table */
  int32_t pad_;
  int64_t alloc_failures; /* appends refused for lack of blocks */
  int64_t cow_copies;     /* copy-on-write pairs issued */
  int32_t host_blocks;    /* size of the host swap pool */
  int32_t free_host_blocks;
  int32_t swapped_seqs;   /* sequences whose blocks are on the host (counted in num_seqs too) */
  int32_t pad2_;
  int64_t swap_out_blocks; /* device -> host pairs issued */
  int64_t swap_in_blocks;  /* host -> device pairs issued */
  int32_t cached_blocks;    /* prefix cache: full blocks indexed by content */
  int32_t evictable_blocks; /* cached blocks no table names (reusable, not in free_blocks) */
  int64_t prefix_query_tokens; /* prompt tokens looked up */
  int64_t prefix_hit_tokens;   /* of those, found in the cache */
} pa_bm_stats;

/* Returns NULL on bad sizes or if initial_order is not a permutation of
 * [0, num_blocks) (message in pa_last_error). */
pa_bm* pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* initial_order);
void pa_bm_destroy(pa_bm* bm);

/* Append n_new tokens to `seq` (created on first use, S06 listing's
 * setdefault).  A block is taken whenever the length is a multiple of B
 * before a write (mercemay.com append listing).  If the first write lands in
 * a partly filled block that another table also names, that block is first
 * copied to a fresh block: the pair (src, dst) is reported, the table points
 * at dst and src's count drops by one (copy-on-write).  The caller must run
 * pa_copy_blocks on reported pairs before writing the new tokens.
 *   slots_out     : HOST int64 [n_new], flat slot of each new token.
 *   cow_pairs_out : HOST int32 [2] (at most one pair per call), may be NULL
 *                   only if the caller knows no copy can occur.
 *   *n_cow_out    : pairs written (0 or 1).
 * All or nothing: PA_ERR_OOM leaves every table, count and list unchanged. */
pa_status pa_bm_append(pa_bm* bm, int64_t seq, int32_t n_new, int64_t* slots_out,
                       int32_t* cow_pairs_out, int32_t* n_cow_out);

/* One token for each of `num` distinct sequences, in the given order - a
 * decode step.  slots_out: HOST int64 [num]; cow_pairs_out: HOST int32
 * [2*num]; *n_cow_out pairs written.  All or nothing across the whole step. */
pa_status pa_bm_append_step(pa_bm* bm, const int64_t* seqs, int32_t num, int64_t* slots_out,
                            int32_t* cow_pairs_out, int32_t* n_cow_out);

/* child gets a copy of parent's table and length; each named block's count
 * rises by one (prefix sharing).  PA_ERR_NOT_FOUND if parent is unknown,
 * PA_ERR_INVALID if child exists. */
pa_status pa_bm_fork(pa_bm* bm, int64_t parent, int64_t child);

/* Retire `seq`: every block in its table loses one count; those reaching zero
 * return to the free list in table order (mercemay.com: the free list never
 * receives a block another table still names).  Unknown seq: PA_OK, no-op. */
pa_status pa_bm_free(pa_bm* bm, int64_t seq);

/* Table length ceil(L / B) of `seq` (-1 if unknown); copies min(that, cap)
 * entries to HOST `out` (may be NULL when cap == 0).  For a swapped sequence
 * the entries are host-pool blocks. */
int32_t pa_bm_table(const pa_bm* bm, int64_t seq, int32_t* out, int32_t cap);

/* Dense upload arrays for a batch: tables_out HOST int32 [num][max_blocks]
 * (unused entries 0), lens_out HOST int32 [num].  PA_ERR_NOT_FOUND for an
 * unknown sequence, PA_ERR_INVALID if a table exceeds max_blocks. */
pa_status pa_bm_export(const pa_bm* bm, const int64_t* seqs, int32_t num, int32_t max_blocks,
                       int32_t* tables_out, int32_t* lens_out);

/* Prefix groups of a batch, the input of pa_decode_plan_prefix: sequences
 * whose tables start with the same physical block form a group (group_out =
 * batch position of its first member; -1 for a sequence alone with its first
 * block or an empty one); prefix_tokens_out = the group's longest common run
 * of leading blocks, in tokens, capped by its shortest member's length
 * (S06 "Copy-on-write, for free": forked samples keep naming the prompt's
 * blocks).  HOST arrays of num entries.  PA_ERR_NOT_FOUND for an unknown
 * sequence. */
pa_status pa_bm_prefix_groups(const pa_bm* bm, const int64_t* seqs, int32_t num, int32_t* group_out,
                              int32_t* prefix_tokens_out);

/* Swapping (preemption by copying out; mercemay.com "Three ways contiguous
 * reservation loses memory", S06 third exercise).  The host swap pool is a
 * second pool of blocks with its own free list and counts, under the device
 * list's discipline (ascending ids first, last retired reused first).
 *
 * pa_bm_set_host_blocks sizes it (0 at creation); PA_ERR_INVALID while any
 * sequence is swapped out.
 *
 * pa_bm_swap_out moves `num` distinct resident sequences to host blocks:
 * every distinct device block of their tables gets one host block, in batch
 * and table order, so sequences that shared a block share its host copy;
 * then each table is retired as pa_bm_free retires it (a block that a
 * resident sequence still names stays on the device and is copied as well).
 * pairs_out (HOST int32 [cap_pairs][2]) receives the (device, host) copies
 * for pa_swap_blocks(PA_SWAP_OUT), which must run before the freed device
 * blocks are written again; *n_pairs_out the count.  A swapped sequence keeps
 * its length; pa_bm_table returns its host table; append, fork, export and
 * prefix grouping refuse it (PA_ERR_INVALID); pa_bm_free releases its host
 * blocks.  pa_bm_swap_in is the mirror image: (host, device) pairs for
 * pa_swap_blocks(PA_SWAP_IN), which must run before the sequences are read.
 * Both are all or nothing: PA_ERR_OOM when the destination pool is short,
 * PA_ERR_INVALID when cap_pairs is too small or a sequence repeats or is in
 * the wrong state, PA_ERR_NOT_FOUND for an unknown one. */
pa_status pa_bm_set_host_blocks(pa_bm* bm, int32_t num_host_blocks);
pa_status pa_bm_swap_out(pa_bm* bm, const int64_t* seqs, int32_t num, int32_t* pairs_out, int32_t cap_pairs,
                         int32_t* n_pairs_out);
pa_status pa_bm_swap_in(pa_bm* bm, const int64_t* seqs, int32_t num, int32_t* pairs_out, int32_t cap_pairs,
                        int32_t* n_pairs_out);
int32_t pa_bm_swapped(const pa_bm* bm, int64_t seq);            /* 1 swapped, 0 resident, -1 unknown */
int32_t pa_bm_host_refcount(const pa_bm* bm, int32_t host_block); /* -1 if out of range */

/* Prefix caching across requests (S06 "What's next": block contents are
 * hashed so that any two requests with a common prefix share the same
 * physical blocks; the same page's production notes on a radix tree of
 * prefixes).  Off at creation; pa_bm_enable_prefix_cache turns it on while no
 * sequence exists (PA_ERR_INVALID otherwise).
 *
 * pa_bm_append_prompt admits a NEW sequence with its prompt token ids
 * (tokens: HOST int32 [n]).  Its leading full blocks are looked up by content
 * - the block's B token ids after the same cached parent block, found by a
 * 64-bit hash and then compared exactly, so the match is the whole token
 * prefix - from the first block to the first miss, reusing at most
 * (n - 1) / B blocks so that the last token is always computed.  A hit
 * shares the cached block (count + 1); the rest of the prompt takes new
 * blocks.  slots_out (HOST int64 [n]) gets -1 for every reused token, whose
 * keys and values are already in the pool (pa_reshape_and_cache skips
 * negative slots), and the flat slot otherwise; *n_cached_out = reused
 * tokens (a multiple of B).  The prompt's new full blocks become cached when
 * the call returns: write their rows on the stream that later reads them.
 * Cached blocks whose count drops to zero stay cached ("evictable", counted
 * apart from free_blocks); every allocation takes the free list first and
 * then the least recently retired evictable block (a retiring table's blocks
 * are ranked deepest first), dropping the cache entries below it.  All or
 * nothing: PA_ERR_OOM changes nothing; PA_ERR_INVALID if the sequence exists
 * or the cache is off. */
pa_status pa_bm_enable_prefix_cache(pa_bm* bm);
pa_status pa_bm_append_prompt(pa_bm* bm, int64_t seq, const int32_t* tokens, int32_t n, int64_t* slots_out,
                              int32_t* n_cached_out);
int32_t pa_bm_cached(const pa_bm* bm, int32_t block); /* 1 cached, 0 not, -1 out of range */

int32_t pa_bm_len(const pa_bm* bm, int64_t seq);         /* -1 if unknown */
int32_t pa_bm_block_size(const pa_bm* bm);               /* B of the manager, -1 for NULL */
int32_t pa_bm_refcount(const pa_bm* bm, int32_t block);  /* -1 if out of range */
void pa_bm_get_stats(const pa_bm* bm, pa_bm_stats* out);

/* One decode step's host work for a serving loop, in one call and one
 * buffer.  The block manager appends one token to each of the `num` distinct
 * sequences (as pa_bm_append_step, all or nothing), and the buffer receives
 * what the step's GPU calls read, at the offsets the layout reports:
 *   slots  int64 [num]        the new tokens' slots (pa_reshape_and_cache);
 *   cows   int32 [n_cows][2]  copy-on-write pairs (pa_copy_blocks, first);
 *   lens   int32 [num]        context lengths after the append;
 *   tables int32 [num][max_blocks]: of each row only the first ceil(L / B)
 *          entries are written (the only ones the kernels read); the rest
 *          keeps whatever the buffer held;
 *   plan   the decode plan for those lengths (pa_decode_plan_schedule with
 *          `schedule`, default piece length), with the jobs' first-tile
 *          entries when first_blocks != 0; layout->plan is its info.
 * The caller uploads the first layout->bytes bytes in one copy and passes
 * device addresses at the same offsets to pa_copy_blocks and pa_decode (with
 * new_key/new_value the append is fused; see pa_decode).  buffer: HOST,
 * 256-byte aligned, `capacity` bytes (pinned memory lets the upload run
 * asynchronously).  The plan is built before the append, so PA_ERR_INVALID
 * for a buffer too small (layout->bytes then gives the size needed), like
 * every other refusal, leaves the block manager unchanged. */
typedef struct pa_decode_step_layout {
  int32_t bytes;      /* bytes to upload, from offset 0 */
  int32_t num_seqs;
  int32_t max_blocks;
  int32_t n_cows;
  int32_t slots_at;   /* byte offsets in the buffer */
  int32_t cows_at;
  int32_t lens_at;
  int32_t tables_at;
  int32_t plan_at;
  int32_t reserved;
  pa_decode_plan_info plan;
} pa_decode_step_layout;
pa_status pa_bm_prepare_decode_step(pa_bm* bm, const int64_t* seqs, int32_t num, int32_t max_blocks,
                                    int32_t num_kv_heads, int32_t num_workgroups, int32_t schedule,
                                    int32_t first_blocks, void* buffer, size_t capacity,
                                    pa_decode_step_layout* layout);

/* Plan reuse for pa_bm_prepare_decode_step, for serving loops whose batch
 * stays the same from step to step: with max_advances > 0 the manager keeps
 * the plan it built last, and the next calls for the same batch (same
 * sequences in the same order, heads, grid and schedule) advance it to the
 * new lengths (pa_decode_plan_advance) instead of building one, at most
 * max_advances times in a row; then, or when the plan cannot follow, a new
 * one is built.  A plan covers exactly its lengths either way; an advanced
 * one keeps the last build's placement, so its balance drifts a tile or so
 * per 16 steps.  0 (the default) builds every step.  PA_ERR_INVALID for a
 * negative count. */
pa_status pa_bm_set_plan_reuse(pa_bm* bm, int32_t max_advances);

/* Verify that each block's count equals the number of tables naming it, that
 * no named block is on the free list, that no block is lost, and that every
 * table holds ceil(L / B) entries (S06 "Reference counts must be exact"); the
 * same for host blocks and the tables of swapped sequences; and the prefix
 * cache's own consistency (every entry found by its key, parents cached,
 * evictable exactly when cached with count zero).
 * PA_OK or PA_ERR_INVALID with the first violation in pa_last_error. */
pa_status pa_bm_check(const pa_bm* bm);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
