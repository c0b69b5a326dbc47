// Elementwise kernels on the running softmax state: init, merge, finalize.
// All three are bound by HBM bandwidth; each thread moves one float4 of a row
// and every row's threads sit in one wavefront (D/4 divides 64), so a row's
// m and l are read by all of its lanes before any lane of that wave writes them.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "ra_kernels.h"

namespace ra {
namespace {

constexpr int kThreads = 256;

__global__ void __launch_bounds__(kThreads) state_init_kernel(float *__restrict__ m,
                                                              float *__restrict__ l,
                                                              float4 *__restrict__ o,
                                                              int64_t n_rows, int64_t n_o4) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int64_t i = gid; i < n_o4; i += stride) o[i] = z;
  for (int64_t i = gid; i < n_rows; i += stride) {
    m[i] = -INFINITY;
    l[i] = 0.f;
  }
}

// dst (+)= src per row.  Empty sides (m == -inf) are taken bit-exactly from
// the other side; exp(-inf - -inf) is never formed.
template <int D>
__global__ void __launch_bounds__(kThreads) state_merge_kernel(
    float *__restrict__ dm, float *__restrict__ dl, float4 *__restrict__ dO,
    const float *__restrict__ sm, const float *__restrict__ sl, const float4 *__restrict__ sO,
    int64_t n_rows) {
  constexpr int kLanesPerRow = D / 4;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = gid / kLanesPerRow;
  const int chunk = (int)(gid % kLanesPerRow);
  if (row >= n_rows) return;
  const float ma = dm[row], mb = sm[row];
  const float la = dl[row], lb = sl[row];
  const int64_t oi = row * kLanesPerRow + chunk;
  if (mb == -INFINITY) return;  // nothing to add
  float4 ob = sO[oi];
  float mn, ln;
  float4 on;
  if (ma == -INFINITY) {  // dst empty: take src as is
    mn = mb;
    ln = lb;
    on = ob;
  } else {
    mn = fmaxf(ma, mb);
    const float wa = expf(ma - mn), wb = expf(mb - mn);
    const float4 oa = dO[oi];
    ln = wa * la + wb * lb;
    on = make_float4(wa * oa.x + wb * ob.x, wa * oa.y + wb * ob.y, wa * oa.z + wb * ob.z,
                     wa * oa.w + wb * ob.w);
  }
  dO[oi] = on;
  if (chunk == 0) {
    dm[row] = mn;
    dl[row] = ln;
  }
}

__device__ inline uint32_t pack_bf16x2(float a, float b) {
  __bf16 ha = (__bf16)a, hb = (__bf16)b;  // round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) |
         ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

// out = O / l, lse = m + ln l; l == 0 gives 0 and -inf.
template <int D, bool kBf16>
__global__ void __launch_bounds__(kThreads) finalize_kernel(
    const float *__restrict__ m, const float *__restrict__ l, const float4 *__restrict__ o,
    void *__restrict__ o_out, float *__restrict__ lse, int64_t n_rows) {
  constexpr int kLanesPerRow = D / 4;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = gid / kLanesPerRow;
  const int chunk = (int)(gid % kLanesPerRow);
  if (row >= n_rows) return;
  const float lr = l[row];
  const int64_t oi = row * kLanesPerRow + chunk;
  float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
  if (lr > 0.f) {
    const float4 x = o[oi];
    r = make_float4(x.x / lr, x.y / lr, x.z / lr, x.w / lr);
  }
  if (o_out) {
    if constexpr (kBf16) {
      uint2 pk;
      pk.x = pack_bf16x2(r.x, r.y);
      pk.y = pack_bf16x2(r.z, r.w);
      reinterpret_cast<uint2 *>(o_out)[oi] = pk;
    } else {
      reinterpret_cast<float4 *>(o_out)[oi] = r;
    }
  }
  if (lse && chunk == 0) lse[row] = lr > 0.f ? m[row] + logf(lr) : -INFINITY;
}

// The reduction of partial states over disjoint key sets, finalized: for each
// output row the parts p = 0 .. parts-1 (state batches b*parts + p of output
// batch b) give m = max_p m_p, w_p = exp(m_p - m) (0 for a part that saw no
// key: exp(-inf - -inf) is never formed), l = sum_p w_p l_p,
// out = (sum_p w_p O_p) / l and lse = m + ln l; a row no part saw gives 0 and
// -inf.  hr = heads * rows (rows of one state batch).
template <int D, bool kBf16>
__global__ void __launch_bounds__(kThreads) merge_finalize_kernel(
    const float *__restrict__ m, const float *__restrict__ l, const float4 *__restrict__ o,
    void *__restrict__ o_out, float *__restrict__ lse, int64_t n_out_rows, int64_t hr,
    int parts) {
  constexpr int kLanesPerRow = D / 4;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = gid / kLanesPerRow;
  const int chunk = (int)(gid % kLanesPerRow);
  if (row >= n_out_rows) return;
  const int64_t b = row / hr, first = b * parts * hr + (row - b * hr);   // part 0's state row
  // Parts are taken kBatch at a time with every load of a batch issued
  // before any use, so a thread waits for one memory round trip per batch
  // rather than per part.
  constexpr int kBatch = 8;
  float mx = -INFINITY;
  for (int p0 = 0; p0 < parts; p0 += kBatch) {
    float mv[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      mv[u] = p0 + u < parts ? m[first + (int64_t)(p0 + u) * hr] : -INFINITY;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) mx = fmaxf(mx, mv[u]);
  }
  float ls = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (mx != -INFINITY) {
    for (int p0 = 0; p0 < parts; p0 += kBatch) {
      float mv[kBatch], lv[kBatch];
      float4 ov[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const bool in = p0 + u < parts;
        const int64_t sr = first + (int64_t)(in ? p0 + u : 0) * hr;
        mv[u] = in ? m[sr] : -INFINITY;
        lv[u] = l[sr];
        ov[u] = o[sr * kLanesPerRow + chunk];
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (mv[u] == -INFINITY) continue;        // a part that saw no key adds nothing
        const float w = expf(mv[u] - mx);
        ls += w * lv[u];
        acc = make_float4(acc.x + w * ov[u].x, acc.y + w * ov[u].y, acc.z + w * ov[u].z,
                          acc.w + w * ov[u].w);
      }
    }
  }
  float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
  if (ls > 0.f) r = make_float4(acc.x / ls, acc.y / ls, acc.z / ls, acc.w / ls);
  const int64_t oi = row * kLanesPerRow + chunk;
  if (o_out) {
    if constexpr (kBf16) {
      uint2 pk;
      pk.x = pack_bf16x2(r.x, r.y);
      pk.y = pack_bf16x2(r.z, r.w);
      reinterpret_cast<uint2 *>(o_out)[oi] = pk;
    } else {
      reinterpret_cast<float4 *>(o_out)[oi] = r;
    }
  }
  if (lse && chunk == 0) lse[row] = ls > 0.f ? mx + logf(ls) : -INFINITY;
}

unsigned grid_for(int64_t threads) {
  int64_t b = (threads + kThreads - 1) / kThreads;
  return (unsigned)(b < 1 ? 1 : b);
}

}  // namespace

hipError_t launch_state_init(float *m, float *l, float *o, int64_t n_rows, int d,
                             hipStream_t s) {
  const int64_t n_o4 = n_rows * d / 4;
  int64_t blocks = (n_o4 + kThreads - 1) / kThreads;
  if (blocks > 65536) blocks = 65536;  // grid-stride beyond this
  if (blocks < 1) blocks = 1;
  state_init_kernel<<<dim3((unsigned)blocks), dim3(kThreads), 0, s>>>(
      m, l, reinterpret_cast<float4 *>(o), n_rows, n_o4);
  return hipGetLastError();
}

hipError_t launch_state_merge(float *dm, float *dl, float *dO, const float *sm, const float *sl,
                              const float *sO, int64_t n_rows, int d, hipStream_t s) {
  const dim3 grid(grid_for(n_rows * (d / 4)));
  if (d == 128)
    state_merge_kernel<128><<<grid, dim3(kThreads), 0, s>>>(
        dm, dl, reinterpret_cast<float4 *>(dO), sm, sl, reinterpret_cast<const float4 *>(sO),
        n_rows);
  else
    state_merge_kernel<64><<<grid, dim3(kThreads), 0, s>>>(
        dm, dl, reinterpret_cast<float4 *>(dO), sm, sl, reinterpret_cast<const float4 *>(sO),
        n_rows);
  return hipGetLastError();
}

hipError_t launch_finalize(const float *m, const float *l, const float *o, void *o_out,
                           bool out_bf16, float *lse, int64_t n_rows, int d, hipStream_t s) {
  const dim3 grid(grid_for(n_rows * (d / 4)));
  const float4 *o4 = reinterpret_cast<const float4 *>(o);
  if (d == 128) {
    if (out_bf16)
      finalize_kernel<128, true><<<grid, dim3(kThreads), 0, s>>>(m, l, o4, o_out, lse, n_rows);
    else
      finalize_kernel<128, false><<<grid, dim3(kThreads), 0, s>>>(m, l, o4, o_out, lse, n_rows);
  } else {
    if (out_bf16)
      finalize_kernel<64, true><<<grid, dim3(kThreads), 0, s>>>(m, l, o4, o_out, lse, n_rows);
    else
      finalize_kernel<64, false><<<grid, dim3(kThreads), 0, s>>>(m, l, o4, o_out, lse, n_rows);
  }
  return hipGetLastError();
}

hipError_t launch_merge_finalize(const float *m, const float *l, const float *o, void *o_out,
                                 bool out_bf16, float *lse, int64_t n_out_rows, int64_t hr,
                                 int parts, int d, hipStream_t s) {
  const dim3 grid(grid_for(n_out_rows * (d / 4)));
  const float4 *o4 = reinterpret_cast<const float4 *>(o);
  if (d == 128) {
    if (out_bf16)
      merge_finalize_kernel<128, true><<<grid, dim3(kThreads), 0, s>>>(m, l, o4, o_out, lse, n_out_rows, hr, parts);
    else
      merge_finalize_kernel<128, false><<<grid, dim3(kThreads), 0, s>>>(m, l, o4, o_out, lse, n_out_rows, hr, parts);
  } else {
    if (out_bf16)
      merge_finalize_kernel<64, true><<<grid, dim3(kThreads), 0, s>>>(m, l, o4, o_out, lse, n_out_rows, hr, parts);
    else
      merge_finalize_kernel<64, false><<<grid, dim3(kThreads), 0, s>>>(m, l, o4, o_out, lse, n_out_rows, hr, parts);
  }
  return hipGetLastError();
}

}  // namespace ra
