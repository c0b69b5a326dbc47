// fp32 ring-step kernel: fold one fp32 key/value block into the state.
//
// Plain fp32 arithmetic (no matrix cores) for small fp32 workloads where the
// tolerance is 1e-5.  A workgroup owns 64 query rows of one (batch, head);
// four lanes share a row and each holds a quarter of the row's q and O.  Key
// and value tiles of 64 rows are staged through LDS.  The state is kept in the
// canonical form after every tile (m is the running maximum).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "ra_kernels.h"

namespace ra {
namespace {

constexpr int kRows = 64;     // query rows per workgroup
constexpr int kKeys = 64;     // keys per LDS tile
constexpr int kThreads = 256; // 4 lanes per query row
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963407f;

template <int D, bool kDiag>
__global__ void __launch_bounds__(kThreads) step_f32_kernel(StepArgs a) {
  constexpr int kPart = D / 4;  // columns per lane
  __shared__ float ks[kKeys][D];
  __shared__ float vs[kKeys][D];

  const int rows = a.rows;         // query rows
  const int kv_rows = a.kv_rows;   // key/value rows (equal to rows on the diagonal)
  const int n_qt = (rows + kRows - 1) / kRows;
  const int bh = blockIdx.x / n_qt;
  const int qt = blockIdx.x % n_qt;
  const int tid = threadIdx.x;
  const int r = tid >> 2, part = tid & 3;
  const int row = qt * kRows + r;
  const bool row_ok = row < rows;
  const size_t base = (size_t)bh * a.row_stride * D;
  const size_t kv_base = (size_t)bh * a.kv_stride * D;
  const int q_bh = bh < a.q_bh ? bh : bh % a.q_bh;   // a query block shared along the batch
  const float *__restrict__ Q = static_cast<const float *>(a.q) + (size_t)q_bh * a.row_stride * D;
  const float *__restrict__ K = static_cast<const float *>(a.k) + kv_base;
  const float *__restrict__ V = static_cast<const float *>(a.v) + kv_base;
  float *__restrict__ O = a.o + base;
  const size_t srow = (size_t)bh * a.row_stride + row;

  const bool read_state = row_ok && !(a.flags & kStepFresh);
  float qv[kPart], ov[kPart];
#pragma unroll
  for (int x = 0; x < kPart; ++x) {
    qv[x] = row_ok ? Q[(size_t)row * D + part * kPart + x] : 0.f;
    ov[x] = read_state ? O[(size_t)row * D + part * kPart + x] : 0.f;
  }
  float m2 = read_state ? a.m[srow] * kLog2e : -INFINITY;  // base-2 running max
  float l = read_state ? a.l[srow] : 0.f;

  const int kv_end = kDiag ? min(kv_rows, (qt + 1) * kRows) : kv_rows;
  for (int k0 = 0; k0 < kv_end; k0 += kKeys) {
    __syncthreads();
    for (int e = tid; e < kKeys * D; e += kThreads) {
      const int kr = e / D, kc = e % D;
      const bool ok = k0 + kr < kv_rows;
      ks[kr][kc] = ok ? K[(size_t)(k0 + kr) * D + kc] : 0.f;
      vs[kr][kc] = ok ? V[(size_t)(k0 + kr) * D + kc] : 0.f;
    }
    __syncthreads();

    float s[kKeys];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int x = 0; x < kPart; ++x) acc = fmaf(qv[x], ks[j][part * kPart + x], acc);
      acc += __shfl_xor(acc, 1);
      acc += __shfl_xor(acc, 2);
      const int key = k0 + j;
      const bool ok = key < kv_rows && (!kDiag || key <= row);
      s[j] = ok ? acc : -INFINITY;
      mx = fmaxf(mx, s[j]);
    }
    const float mt = mx * a.scale_log2;
    const float mn = fmaxf(m2, mt);
    if (mn == -INFINITY) continue;  // nothing visible yet: state unchanged
    const float alpha = (m2 == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m2 - mn);
    l *= alpha;
#pragma unroll
    for (int x = 0; x < kPart; ++x) ov[x] *= alpha;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      const float p = __builtin_amdgcn_exp2f(fmaf(s[j], a.scale_log2, -mn));
      l += p;
#pragma unroll
      for (int x = 0; x < kPart; ++x) ov[x] = fmaf(p, vs[j][part * kPart + x], ov[x]);
    }
    m2 = mn;
  }

  if (row_ok && !(a.flags & kStepFinalize)) {
#pragma unroll
    for (int x = 0; x < kPart; ++x) O[(size_t)row * D + part * kPart + x] = ov[x];
    if (part == 0) {
      a.m[srow] = m2 * kLn2;
      a.l[srow] = l;
    }
  } else if (row_ok) {
    // Finalize in place of the store (as the finalize kernel would).
    const size_t oe = base + (size_t)row * D + part * kPart;
    if (a.o_out) {
#pragma unroll
      for (int x = 0; x < kPart; ++x) {
        const float y = l > 0.f ? ov[x] / l : 0.f;
        if (a.out_bf16) {
          const __bf16 hb = (__bf16)y;
          static_cast<uint16_t *>(a.o_out)[oe + x] = __builtin_bit_cast(uint16_t, hb);
        } else {
          static_cast<float *>(a.o_out)[oe + x] = y;
        }
      }
    }
    if (part == 0 && a.lse_out) {
      // m is rounded to fp32 before the add, as the stored state is.
#pragma clang fp contract(off)
      const float m_nat = m2 * kLn2;
      a.lse_out[srow] = l > 0.f ? m_nat + logf(l) : -INFINITY;
    }
  }
}

}  // namespace

hipError_t launch_step_f32(const StepArgs &a, int d, StepCase c, hipStream_t s,
                           const LaunchTiming &t) {
  const int n_qt = (a.rows + kRows - 1) / kRows;
  const dim3 grid((unsigned)((int64_t)a.bh * n_qt)), block(kThreads);
  const bool diag = c == StepCase::Diag;
  void (*kernel)(StepArgs) = d == 128 ? (diag ? step_f32_kernel<128, true> : step_f32_kernel<128, false>)
                                      : (diag ? step_f32_kernel<64, true> : step_f32_kernel<64, false>);
  return launch_one(kernel, grid, block, s, t.start, t.stop, a);
}

}  // namespace ra
