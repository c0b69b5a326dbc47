// Backward of one ring step ("Ring Attention：把超长序列沿设备环流动", section
// "Backward 需要让梯度也沿环传播"): every (query block i, key/value block j)
// interaction adds to the gradients; the query owner accumulates dQ_i, and the
// dK_j, dV_j of the visiting block accumulate while it travels the ring.  As in
// the FlashAttention backward the pages point to, the probabilities are
// recomputed from the per-row log-sum-exp the forward saved:
//     P  = exp(scale q.k - LSE)        (0 where the causal mask hides the key)
//     dP = dO . v,   dS = P (dP - D),  D = rowsum(dO * O)
//     dQ += scale dS K,   dK += scale dS^T Q,   dV += P^T dO
//
// This file holds the per-row term D and the general step kernel: fp32
// arithmetic on fp32 or bf16 inputs, any supported head_dim.  A workgroup owns
// 64 query rows of one (batch, head) with four lanes per row (as the fp32
// forward kernel); key/value tiles of 32 rows go through LDS.  dQ stays in
// registers; the tile's dS and P go through LDS to form this workgroup's part
// of dK and dV for the tile, which is added to the global accumulators with
// fp32 atomics (several query tiles add to the same keys).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "ra_kernels.h"

namespace ra {
namespace {

constexpr float kLog2e = 1.442695040888963407f;

__device__ __forceinline__ float load_elem(const float *p, size_t i) { return p[i]; }
__device__ __forceinline__ float load_elem(const uint16_t *p, size_t i) {
  return __uint_as_float((uint32_t)p[i] << 16);
}

// D[row] = sum_x dO[row][x] * O[row][x].  Sixteen lanes per row: in step i
// lane l reads column 16i + l, so each step reads a contiguous run of the row;
// the partial sums are combined across the 16 lanes.
template <int D, typename OT, typename DT>
__global__ void __launch_bounds__(256) bwd_prepare_kernel(const OT *__restrict__ o,
                                                          const DT *__restrict__ dout,
                                                          float *__restrict__ delta,
                                                          float *__restrict__ dq,
                                                          int64_t n_rows) {
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int l = threadIdx.x & 15;
  float acc = 0.f;
  if (row < n_rows) {
#pragma unroll
    for (int i = 0; i < D / 16; ++i)
      acc = fmaf(load_elem(dout, (size_t)row * D + 16 * i + l), load_elem(o, (size_t)row * D + 16 * i + l), acc);
  }
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 4);
  acc += __shfl_xor(acc, 8);
  if (row < n_rows && l == 0) delta[row] = acc;
  if (dq && row < n_rows) {     // the rank's dQ accumulator starts at zero
#pragma unroll
    for (int i = 0; i < D / 16; ++i) dq[(size_t)row * D + 16 * i + l] = 0.f;
  }
}

constexpr int kRows = 64;     // query rows per workgroup
constexpr int kKeys = 32;     // keys per tile (LDS: K, V, P, dS, Q, dO tiles fit 160 KiB at d = 128)
constexpr int kThreads = 256; // 4 lanes per row

template <int D, bool kDiag, typename T>
__global__ void __launch_bounds__(kThreads) bwd_step_simple_kernel(BwdArgs a) {
  constexpr int kPart = D / 4;
  __shared__ float ks[kKeys][D + 1];
  __shared__ float vs[kKeys][D + 1];
  __shared__ float ps[kRows][kKeys + 1];
  __shared__ float dss[kRows][kKeys + 1];
  __shared__ float qs[kRows][D + 1];
  __shared__ float dos[kRows][D + 1];

  const int rows = a.rows;
  const int n_qt = (rows + kRows - 1) / kRows;
  const int bh = blockIdx.x / n_qt;
  const int qt = blockIdx.x % n_qt;
  const int tid = threadIdx.x;
  const int r = tid >> 2, part = tid & 3;
  const int row = qt * kRows + r;
  const bool row_ok = row < rows;
  const size_t base = (size_t)bh * rows * D;
  const T *__restrict__ Q = static_cast<const T *>(a.q) + base;
  const T *__restrict__ dO = static_cast<const T *>(a.dout) + base;
  const T *__restrict__ K = static_cast<const T *>(a.k) + base;
  const T *__restrict__ V = static_cast<const T *>(a.v) + base;
  float *__restrict__ dQ = a.dq + base;
  float *__restrict__ dK = a.dk + base;
  float *__restrict__ dV = a.dv + base;
  const size_t srow = (size_t)bh * rows + row;
  const float lse2 = row_ok ? a.lse[srow] * kLog2e : -INFINITY;
  const float dval = row_ok ? a.delta[srow] : 0.f;

  float qv[kPart], dov[kPart], dqv[kPart];
#pragma unroll
  for (int x = 0; x < kPart; ++x) {
    const int col = part * kPart + x;
    qv[x] = row_ok ? load_elem(Q, (size_t)row * D + col) : 0.f;
    dov[x] = row_ok ? load_elem(dO, (size_t)row * D + col) : 0.f;
    dqv[x] = 0.f;
    qs[r][col] = qv[x];
    dos[r][col] = dov[x];
  }

  const int kv_end = kDiag ? min(rows, (qt + 1) * kRows) : rows;
  for (int k0 = 0; k0 < kv_end; k0 += kKeys) {
    __syncthreads();
    for (int e = tid; e < kKeys * D; e += kThreads) {
      const int kr = e / D, kc = e % D;
      const bool ok = k0 + kr < rows;
      ks[kr][kc] = ok ? load_elem(K, (size_t)(k0 + kr) * D + kc) : 0.f;
      vs[kr][kc] = ok ? load_elem(V, (size_t)(k0 + kr) * D + kc) : 0.f;
    }
    __syncthreads();
    // Scores, probabilities and dS of this row against the tile's keys.
    for (int j = 0; j < kKeys; ++j) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int x = 0; x < kPart; ++x) {
        s = fmaf(qv[x], ks[j][part * kPart + x], s);
        dp = fmaf(dov[x], vs[j][part * kPart + x], dp);
      }
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      dp += __shfl_xor(dp, 1);
      dp += __shfl_xor(dp, 2);
      const int key = k0 + j;
      const bool ok = row_ok && key < rows && (!kDiag || key <= row) && lse2 != -INFINITY;
      const float p = ok ? __builtin_amdgcn_exp2f(fmaf(s, a.scale_log2, -lse2)) : 0.f;
      const float ds = p * (dp - dval);
#pragma unroll
      for (int x = 0; x < kPart; ++x) dqv[x] = fmaf(ds, ks[j][part * kPart + x], dqv[x]);
      if (part == 0) {
        ps[r][j] = p;
        dss[r][j] = ds;
      }
    }
    __syncthreads();
    // This workgroup's part of dK and dV for the tile: thread (key j, column
    // group) sums over the 64 rows.
    for (int e = tid; e < kKeys * D; e += kThreads) {
      const int j = e / D, col = e % D;
      const int key = k0 + j;
      if (key >= rows) continue;
      float gk = 0.f, gv = 0.f;
      for (int rr = 0; rr < kRows; ++rr) {
        gk = fmaf(dss[rr][j], qs[rr][col], gk);
        gv = fmaf(ps[rr][j], dos[rr][col], gv);
      }
      if (gk != 0.f) atomicAdd(&dK[(size_t)key * D + col], gk * a.scale);
      if (gv != 0.f) atomicAdd(&dV[(size_t)key * D + col], gv);
    }
  }
  if (row_ok) {
#pragma unroll
    for (int x = 0; x < kPart; ++x) dQ[(size_t)row * D + part * kPart + x] += dqv[x] * a.scale;
  }
}

template <int D, typename T>
hipError_t launch_simple_d(const BwdArgs &a, bool diag, hipStream_t s, const LaunchTiming &t) {
  const int n_qt = (a.rows + kRows - 1) / kRows;
  const dim3 grid((unsigned)((int64_t)a.bh * n_qt)), block(kThreads);
  return launch_one(diag ? bwd_step_simple_kernel<D, true, T> : bwd_step_simple_kernel<D, false, T>,
                    grid, block, s, t.start, t.stop, a);
}

template <int D>
hipError_t launch_prepare_d(const void *o, bool o_bf16, const void *dout, bool do_bf16,
                            float *delta, float *dq, int64_t n_rows, hipStream_t s) {
  const dim3 grid((unsigned)((n_rows + 15) / 16)), block(256);
  const float *of = static_cast<const float *>(o);
  const uint16_t *ob = static_cast<const uint16_t *>(o);
  const float *df = static_cast<const float *>(dout);
  const uint16_t *db = static_cast<const uint16_t *>(dout);
  if (o_bf16 && do_bf16) bwd_prepare_kernel<D><<<grid, block, 0, s>>>(ob, db, delta, dq, n_rows);
  else if (o_bf16) bwd_prepare_kernel<D><<<grid, block, 0, s>>>(ob, df, delta, dq, n_rows);
  else if (do_bf16) bwd_prepare_kernel<D><<<grid, block, 0, s>>>(of, db, delta, dq, n_rows);
  else bwd_prepare_kernel<D><<<grid, block, 0, s>>>(of, df, delta, dq, n_rows);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_prepare(const void *o, bool o_bf16, const void *dout, bool do_bf16,
                              float *delta, float *dq, int64_t n_rows, int d, hipStream_t s) {
  if (d == 128) return launch_prepare_d<128>(o, o_bf16, dout, do_bf16, delta, dq, n_rows, s);
  return launch_prepare_d<64>(o, o_bf16, dout, do_bf16, delta, dq, n_rows, s);
}

hipError_t launch_bwd_step_simple(const BwdArgs &a, int d, bool bf16, StepCase c, hipStream_t s,
                                  const LaunchTiming &t) {
  const bool diag = c == StepCase::Diag;
  if (d == 128)
    return bf16 ? launch_simple_d<128, uint16_t>(a, diag, s, t)
                : launch_simple_d<128, float>(a, diag, s, t);
  return bf16 ? launch_simple_d<64, uint16_t>(a, diag, s, t) : launch_simple_d<64, float>(a, diag, s, t);
}

}  // namespace ra
