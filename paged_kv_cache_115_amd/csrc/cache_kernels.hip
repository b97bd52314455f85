// Cache-writing kernels: the slot scatter of newly appended tokens, the
// whole-block copy used for copy-on-write, and the block copy between the
// device pool and a pinned host pool used to swap preempted sequences.  All
// are pure byte moves in 16-byte vector loads/stores; rows of one token
// (num_kv_heads * head_dim elements) are contiguous in the pool, so each
// token is one coalesced run and each block one contiguous extent.
#include <hip/hip_runtime.h>

#include "launch.h"

namespace pagedkv {
namespace {

constexpr int kThreads = 256;

// Token i's key row and value row go to flat slot slots[i]
// (mercemay.com "Paged KV Cache Allocation and the Block Table", the cache
// write of the append listing).  One workgroup per token; threads [0, n)
// move the key row, [n, 2n) the value row, n = row bytes / 16.
__global__ __launch_bounds__(kThreads) void reshape_and_cache_kernel(
    uint4* __restrict__ kpool, uint4* __restrict__ vpool, const uint4* __restrict__ key,
    const uint4* __restrict__ value, const int64_t* __restrict__ slots, int64_t num_slots,
    int32_t row_vec) {
  const int64_t tok = blockIdx.x;
  const int64_t slot = slots[tok];
  if (slot < 0 || slot >= num_slots) return;  // padding, or out of the pool
  for (int32_t c = threadIdx.x; c < 2 * row_vec; c += kThreads) {
    const bool is_v = c >= row_vec;
    const int32_t cc = is_v ? c - row_vec : c;
    const uint4* src = is_v ? value : key;
    uint4* dst = is_v ? vpool : kpool;
    dst[slot * row_vec + cc] = src[tok * row_vec + cc];
  }
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Streaming 16-byte moves: every byte is read once and written once, so both
// sides are marked non-temporal.
__device__ __forceinline__ u32x4_t load_stream(const uint4* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}
__device__ __forceinline__ void store_stream(uint4* p, u32x4_t v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
}

constexpr int kCopyUnroll = 4;  // 16-byte vectors in flight per thread

// Block pairs[2p+1] of both pools becomes a copy of block pairs[2p]
// (aicassindra.com "tm_paged_attention_deep", "Copy-on-write for shared
// prefixes").  grid = (pairs, 2 pools, chunks of kThreads * kCopyUnroll
// vectors); each thread loads its kCopyUnroll vectors before storing them.
__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(
    uint4* __restrict__ kpool, uint4* __restrict__ vpool, const int32_t* __restrict__ pairs,
    int32_t num_blocks, int32_t block_vec) {
  const int32_t src = pairs[2 * blockIdx.x];
  const int32_t dst = pairs[2 * blockIdx.x + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  uint4* pool = blockIdx.y ? vpool : kpool;
  const uint4* s0 = pool + (int64_t)src * block_vec;
  uint4* d0 = pool + (int64_t)dst * block_vec;
  constexpr int32_t kChunk = kThreads * kCopyUnroll;
  for (int32_t c0 = blockIdx.z * kChunk + threadIdx.x; c0 < block_vec; c0 += gridDim.z * kChunk) {
    u32x4_t v[kCopyUnroll];
#pragma unroll
    for (int i = 0; i < kCopyUnroll; ++i)
      if (c0 + i * kThreads < block_vec) v[i] = load_stream(s0 + c0 + i * kThreads);
#pragma unroll
    for (int i = 0; i < kCopyUnroll; ++i)
      if (c0 + i * kThreads < block_vec) store_stream(d0 + c0 + i * kThreads, v[i]);
  }
}

// Block dst[i] of the destination pools becomes a copy of block src[i] of the
// source pools, for the pairs of one launch (mercemay.com "Paged KV Cache
// Allocation and the Block Table": preemption copies the cache out to host
// memory and back).  One side is pinned host memory mapped into the device's
// address space, so every load or store on that side is a PCIe transaction;
// the other side is HBM.  kOut: device -> host (HBM loads stream through,
// host stores are plain); otherwise host -> device.  grid = (pairs, 2 pools,
// chunks of kThreads * kCopyUnroll vectors), exactly as copy_blocks_kernel;
// the pair lists travel in the kernel arguments, checked on the host.
template <bool kOut>
__global__ __launch_bounds__(kThreads) void swap_blocks_kernel(
    const uint4* __restrict__ src_k, const uint4* __restrict__ src_v, uint4* __restrict__ dst_k,
    uint4* __restrict__ dst_v, SwapBatch batch, int32_t block_vec) {
  const int32_t src = batch.src[blockIdx.x];
  const int32_t dst = batch.dst[blockIdx.x];
  const uint4* s0 = (blockIdx.y ? src_v : src_k) + (int64_t)src * block_vec;
  uint4* d0 = (blockIdx.y ? dst_v : dst_k) + (int64_t)dst * block_vec;
  constexpr int32_t kChunk = kThreads * kCopyUnroll;
  for (int32_t c0 = blockIdx.z * kChunk + threadIdx.x; c0 < block_vec; c0 += gridDim.z * kChunk) {
    u32x4_t v[kCopyUnroll];
#pragma unroll
    for (int i = 0; i < kCopyUnroll; ++i) {
      if (c0 + i * kThreads >= block_vec) continue;
      const uint4* p = s0 + c0 + i * kThreads;
      v[i] = kOut ? load_stream(p) : *reinterpret_cast<const u32x4_t*>(p);
    }
#pragma unroll
    for (int i = 0; i < kCopyUnroll; ++i) {
      if (c0 + i * kThreads >= block_vec) continue;
      uint4* p = d0 + c0 + i * kThreads;
      if (kOut)
        *reinterpret_cast<u32x4_t*>(p) = v[i];
      else
        store_stream(p, v[i]);
    }
  }
}

int32_t elem_bytes(int32_t dtype) { return dtype == PA_F32 ? 4 : 2; }

}  // namespace

hipError_t launch_reshape_and_cache(const pa_kv_pool& pool, const void* key, const void* value,
                                    const int64_t* slots, int32_t num_tokens, hipStream_t stream) {
  const int32_t row_bytes = pool.num_kv_heads * pool.head_dim * elem_bytes(pool.dtype);
  const int64_t num_slots = (int64_t)pool.num_blocks * pool.block_size;
  hipLaunchKernelGGL(reshape_and_cache_kernel, dim3(num_tokens), dim3(kThreads), 0, stream,
                     (uint4*)pool.k, (uint4*)pool.v, (const uint4*)key, (const uint4*)value, slots,
                     num_slots, row_bytes / 16);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(const pa_kv_pool& pool, const int32_t* pairs, int32_t num_pairs,
                              hipStream_t stream) {
  const int32_t block_vec = (int32_t)(pool_block_bytes(pool) / 16);
  const int32_t chunks = (block_vec + kThreads * kCopyUnroll - 1) / (kThreads * kCopyUnroll);
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(num_pairs, 2, chunks), dim3(kThreads), 0, stream,
                     (uint4*)pool.k, (uint4*)pool.v, pairs, pool.num_blocks, block_vec);
  return hipGetLastError();
}

hipError_t launch_swap_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                              int64_t block_bytes, const SwapBatch& batch, int32_t num_pairs, bool out,
                              hipStream_t stream) {
  const int32_t block_vec = (int32_t)(block_bytes / 16);
  const int32_t chunks = (block_vec + kThreads * kCopyUnroll - 1) / (kThreads * kCopyUnroll);
  const dim3 grid(num_pairs, 2, chunks);
  if (out)
    hipLaunchKernelGGL(swap_blocks_kernel<true>, grid, dim3(kThreads), 0, stream, (const uint4*)src_k,
                       (const uint4*)src_v, (uint4*)dst_k, (uint4*)dst_v, batch, block_vec);
  else
    hipLaunchKernelGGL(swap_blocks_kernel<false>, grid, dim3(kThreads), 0, stream, (const uint4*)src_k,
                       (const uint4*)src_v, (uint4*)dst_k, (uint4*)dst_v, batch, block_vec);
  return hipGetLastError();
}

}  // namespace pagedkv
