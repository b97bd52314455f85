// Measurement aid: a plain streaming read of device memory, the reference
// for what a read-only HBM stream achieves on this GPU with the decode
// kernel's load width and cache policy (16-byte loads marked non-temporal,
// whole rows, contiguous per workgroup).  The decode launch is measured
// against the published HBM peak; this probe says how much of that peak a
// kernel doing nothing but reading reaches, and what fixed cost a launch of
// the same grid pays.  Not on the decode path.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace pagedkv {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;  // 16-byte loads in flight per thread

// Workgroup b reads 16-byte words [b * per, min((b + 1) * per, n16)) of src,
// kProbeUnroll loads in flight per thread; the xor of the words is stored
// only if it equals a value it never takes for the probe's inputs, which
// keeps the loads alive without write traffic.
__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const u32x4_t* src, int64_t n16, int64_t per,
                                                                   uint32_t* sink) {
  const int64_t b = (int64_t)blockIdx.x * per;
  const int64_t e = min(b + per, n16);
  uint32_t acc = 0;
  for (int64_t i = b + threadIdx.x; i < e; i += (int64_t)kProbeUnroll * kProbeThreads) {
    u32x4_t v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) {
      const int64_t j = i + (int64_t)u * kProbeThreads;
      v[u] = j < e ? __builtin_nontemporal_load(src + j) : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  if (acc == 0x7fc0ffeeu) sink[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = acc;
}

}  // namespace
}  // namespace pagedkv

extern "C" pa_status pa_probe_read(const void* src, size_t bytes, int32_t num_workgroups, void* sink, void* stream) {
  const char* who = "pa_probe_read";
  if (!src || !sink || num_workgroups <= 0 || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(src) % 16 != 0)
    return pagedkv::fail(PA_ERR_INVALID, "%s: src/sink NULL, num_workgroups <= 0, or src/bytes not 16-byte aligned",
                         who);
  if (bytes == 0) return PA_OK;
  const int64_t n16 = (int64_t)(bytes / 16);
  const int64_t per = (n16 + num_workgroups - 1) / num_workgroups;
  hipLaunchKernelGGL(pagedkv::probe_read_kernel, dim3((unsigned)num_workgroups), dim3(pagedkv::kProbeThreads), 0,
                     (hipStream_t)stream, reinterpret_cast<const pagedkv::u32x4_t*>(src), n16, per,
                     static_cast<uint32_t*>(sink));
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pagedkv::fail(PA_ERR_HIP, "%s: %s", who, hipGetErrorString(e));
  return PA_OK;
}
