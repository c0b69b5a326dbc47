// Staging copy: device-to-device move of one key/value block into the free
// receive buffer, standing in for the receive from the previous rank ("Ring
// Attention Paper Breakdown: Blockwise Distributed Transformers for
// Near-Infinite Context", section 2: receive into buffer B, then swap).
//
// The copy runs beside a step kernel, which it should disturb as little as
// possible: the loads and stores carry the non-temporal hint (the block is not
// reused from cache by this copy), and the grid is small (kMaxBlocks
// workgroups of four wavefronts: one on half of the CUs), so the step kernel's
// workgroups, which need most of a CU each, still find room on every CU.  The copy then takes a few tens of microseconds for a 32 MiB block,
// well inside one step.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ra_kernels.h"

namespace ra {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;
constexpr int64_t kMaxBlocks = 128;

template <bool kNonTemporal>
__global__ void __launch_bounds__(kThreads) stage_copy_kernel(u32x4 *__restrict__ dst,
                                                              const u32x4 *__restrict__ src,
                                                              int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      v[u] = kNonTemporal ? __builtin_nontemporal_load(src + i + u * stride) : src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (kNonTemporal) __builtin_nontemporal_store(v[u], dst + i + u * stride);
      else dst[i + u * stride] = v[u];
    }
  }
  for (; i < n16; i += stride) {
    const u32x4 v = kNonTemporal ? __builtin_nontemporal_load(src + i) : src[i];
    if (kNonTemporal) __builtin_nontemporal_store(v, dst + i);
    else dst[i] = v;
  }
}

}  // namespace

hipError_t launch_stage_copy(void *dst, const void *src, size_t bytes, hipStream_t s) {
  const int64_t n16 = (int64_t)(bytes / 16);
  int64_t blocks = (n16 + (int64_t)kThreads * kUnroll - 1) / ((int64_t)kThreads * kUnroll);
  if (blocks > kMaxBlocks) blocks = kMaxBlocks;
  if (blocks < 1) blocks = 1;
  stage_copy_kernel<true><<<dim3((unsigned)blocks), dim3(kThreads), 0, s>>>(
      static_cast<u32x4 *>(dst), static_cast<const u32x4 *>(src), n16);
  return hipGetLastError();
}

}  // namespace ra
