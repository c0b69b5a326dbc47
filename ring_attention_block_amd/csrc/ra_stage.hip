// Staging copy: device-to-device move of one key/value block into the free
// receive buffer, standing in for the receive from the previous rank ("Ring
// Attention Paper Breakdown: Blockwise Distributed Transformers for
// Near-Infinite Context", section 2: receive into buffer B, then swap).
//
// The copy runs beside a step kernel, which it should disturb as little as
// possible:
//   * a small grid (kMaxBlocks workgroups of four wavefronts, each copying one
//     contiguous chunk), so the step kernel keeps the compute units;
//   * few registers: buffer loads and stores address the chunk through a
//     32-bit lane offset plus a scalar offset per unrolled access, so a
//     wavefront holds kUnroll 16-byte values and one offset (15 VGPRs, 16
//     allocated).  Two wavefronts of the forward step kernel's full-block
//     (8-wavefront) or diagonal variant at head_dim 128 leave at least 16 of
//     the 512 registers per lane of a SIMD free, so a copy wavefront fits
//     beside them instead of taking the place of a step workgroup;
//   * non-temporal loads and stores (the block is not reused from cache by
//     this copy).
// A 32 MiB block then takes a few tens of microseconds, well inside one step.
// A copy with no step beside it (the step it overlaps is a skipped causal
// block) takes a full-chip grid instead: 8 workgroups per compute unit.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ra_kernels.h"

namespace ra {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 3;
constexpr int64_t kMaxBlocks = 128;
constexpr int64_t kMaxBlocksAlone = 2048;
constexpr int64_t kMaxChunk = (int64_t)1 << 30;   // buffer offsets are 32-bit
constexpr int kNonTemporal = 2;                    // buffer access cache policy: nt
constexpr int kRawBuffer = 0x00020000;             // buffer resource: raw (untyped) 32-bit words

// Workgroup b copies bytes [b * chunk, min((b + 1) * chunk, bytes)) of src to
// dst; chunk and bytes are multiples of 16.  The buffer range check keeps
// every access inside the chunk.
__global__ void __launch_bounds__(kThreads) stage_copy_kernel(char *__restrict__ dst,
                                                              const char *__restrict__ src,
                                                              int64_t bytes, int64_t chunk) {
  const int64_t c0 = (int64_t)blockIdx.x * chunk;
  if (c0 >= bytes) return;
  const uint32_t len = (uint32_t)(bytes - c0 < chunk ? bytes - c0 : chunk);
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(src) + c0, 0, len, kRawBuffer);
  const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(dst + c0, 0, len, kRawBuffer);
  constexpr uint32_t kStep = kThreads * 16;
  uint32_t off = threadIdx.x * 16;
  for (; off + (kUnroll - 1) * kStep < len; off += kUnroll * kStep) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, u * kStep, kNonTemporal);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      __builtin_amdgcn_raw_buffer_store_b128(v[u], rd, off, u * kStep, kNonTemporal);
  }
  for (; off < len; off += kStep) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kNonTemporal);
    __builtin_amdgcn_raw_buffer_store_b128(v, rd, off, 0, kNonTemporal);
  }
}

}  // namespace

hipError_t launch_stage_copy(void *dst, const void *src, size_t bytes, bool alone, hipStream_t s) {
  const int64_t n = (int64_t)bytes;
  constexpr int64_t kPerRound = (int64_t)kThreads * 16 * kUnroll;
  int64_t blocks = (n + kPerRound - 1) / kPerRound;
  const int64_t max_blocks = alone ? kMaxBlocksAlone : kMaxBlocks;
  if (blocks > max_blocks) blocks = max_blocks;
  const int64_t min_blocks = (n + kMaxChunk - 1) / kMaxChunk;
  if (blocks < min_blocks) blocks = min_blocks;
  if (blocks < 1) blocks = 1;
  const int64_t chunk = ((n + blocks - 1) / blocks + 15) & ~(int64_t)15;
  stage_copy_kernel<<<dim3((unsigned)blocks), dim3(kThreads), 0, s>>>(
      static_cast<char *>(dst), static_cast<const char *>(src), n, chunk);
  return hipGetLastError();
}

}  // namespace ra
