// bf16 ring-step kernel for gfx950: fold one visiting key/value block into the
// running softmax state of the rank's query block with the CDNA4 matrix cores.
//
// What one launch computes ("Ring Attention Paper Breakdown: Blockwise
// Distributed Transformers for Near-Infinite Context", section 3, steps 1-7):
// for every query row r of every (batch, head), over the keys t of block j
// that r may see,
//     m' = max(m, max_t s_rt),   s_rt = scale * q_r . k_t
//     l' = exp(m - m') l + sum_t exp(s_rt - m')
//     O' = exp(m - m') O + sum_t exp(s_rt - m') v_t
// with the diagonal block masked to t <= r ("Ring Attention：把超长序列沿设备环
// 流动", section "Causal Attention 让环不再完全对称").
//
// Design.  A workgroup is kW wavefronts of 32 query rows each, all of one
// (batch, head); two wavefronts share each SIMD.
//  * Q rows stay in registers for the whole block as the B operand of
//    v_mfma_f32_32x32x16_bf16; the O^T accumulator stays in registers too.
//  * Key/value tiles of 64 keys are copied from HBM straight into LDS by
//    buffer loads with an LDS destination (no staging registers), double
//    buffered: the loads of tile n+1 are issued before the matrix work of
//    tile n; one barrier per tile.  Rows past the block end are zero.
//  * Both tiles are row-major in LDS with the 16-byte chunks of each row
//    XOR-swizzled by the row index, so the fragment reads below hit distinct
//    banks without padding (a wavefront's LDS-destination load writes 1 KiB
//    contiguously, which rules padding out).
//  * Scores are produced transposed, S^T = K Q^T, so each lane holds one query
//    (lane % 32) and 32 of its keys.  K's LDS row rho holds key kappa(rho),
//    which swaps bits 2 and 3 of the key index within 32; this makes the 8
//    keys in each half of a lane's accumulator contiguous, so those registers
//    are directly the B operand of O^T += V^T P^T with no lane exchange and
//    the row statistics (max, sum, rescale factor) are per-lane values.
//  * The V^T operand comes from the row-major V tile through the transposing
//    LDS read ds_read_b64_tr_b16: within each 16-lane group, output lane i,
//    slot k receives element (i mod 4) of the 8 bytes addressed by lane
//    4k + i/4, so pointing lane j at V[key0 + j/4][d0 + 4(j mod 4)] gives lane
//    i the four keys key0..key0+3 of column d0 + i.
//  * The softmax works in base 2: p = exp2(s_raw * scale*log2(e) - m2), one
//    FMA and one v_exp_f32 per score.  The rescale of O is lazy: the reference
//    maximum only moves when a tile's maximum exceeds it by more than kTau (so
//    every p <= 2^kTau, safe in fp32 and bf16); the true running maximum is
//    tracked beside it and the state is rescaled to it once on exit, so the
//    stored state is canonical.
//  * Lanes l and l+32 hold the same query with disjoint keys: the row maximum
//    is combined with v_permlane32_swap, the partial row sums once at the end.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "ra_kernels.h"

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;

constexpr int kBN = 64;        // keys per tile
constexpr float kTau = 8.0f;   // lazy-rescale threshold, base-2 units
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963407f;

template <int D>
struct Tile {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kBytes = kBN * kRowBytes;          // one K (or V) tile
  static constexpr int kChunks = D / 8;                   // 16-byte chunks per row
  static constexpr int kRowsPerLoad = 1024 / kRowBytes;   // rows per wavefront load
  static constexpr int kLoads = kBytes / 1024;            // wavefront loads per tile
  static constexpr int kBufBytes = 2 * kBytes;            // K then V
  static constexpr size_t kLdsBytes = 2 * kBufBytes;      // double buffered
};

// Key held by LDS row rho of the K tile: bits 2 and 3 swapped within 32.
__device__ __forceinline__ int k_row_key(int rho) {
  return (rho & ~12) | ((rho & 4) << 1) | ((rho & 8) >> 1);
}
// 16-byte chunk swizzles of the K and V tiles.
__device__ __forceinline__ int k_swz(int rho) { return rho & 7; }
__device__ __forceinline__ int v_swz(int rho) { return 2 * (rho & 3); }

// Device-only helpers (the buffer resource type exists only for the GPU target).
#if defined(__HIP_DEVICE_COMPILE__)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, bytes, 0x00020000);
}

template <int D, int kW>
struct Stage {
  static constexpr int kPerWave = (Tile<D>::kLoads + kW - 1) / kW;
  uint32_t k[kPerWave];   // per-lane source byte offsets within a tile
  uint32_t v[kPerWave];
};

template <int D, int kW>
__device__ __forceinline__ Stage<D, kW> stage_offsets(int wave, int lane) {
  using T = Tile<D>;
  Stage<D, kW> so;
#pragma unroll
  for (int i = 0; i < Stage<D, kW>::kPerWave; ++i) {
    const int n = wave + i * kW;
    const int rho = n * T::kRowsPerLoad + lane / T::kChunks;
    const int chi = lane % T::kChunks;
    so.k[i] = (uint32_t)(k_row_key(rho) * T::kRowBytes + ((chi ^ k_swz(rho)) * 16));
    so.v[i] = (uint32_t)(rho * T::kRowBytes + ((chi ^ v_swz(rho)) * 16));
  }
  return so;
}

// Issue this wavefront's share of the HBM -> LDS copies of the tile at key k0.
template <int D, int kW>
__device__ __forceinline__ void issue_tile(char *buf, __amdgpu_buffer_rsrc_t rk,
                                           __amdgpu_buffer_rsrc_t rv, const Stage<D, kW> &so,
                                           int k0, int wave) {
  using T = Tile<D>;
  // The tile offset goes into the per-lane offset, which the buffer range
  // check covers (the scalar offset is not range checked).
  const uint32_t toff = (uint32_t)k0 * T::kRowBytes;
#pragma unroll
  for (int i = 0; i < Stage<D, kW>::kPerWave; ++i) {
    const int n = wave + i * kW;
    if (Stage<D, kW>::kPerWave * kW == T::kLoads || n < T::kLoads) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void *)(buf + n * 1024), 16, so.k[i] + toff, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void *)(buf + T::kBytes + n * 1024), 16,
                                               so.v[i] + toff, 0, 0, 0);
    }
  }
}

// Zero the LDS rows of a tile buffer whose keys lie at or past `n_valid` (only
// for the last tile of a block whose length is not a multiple of 64).  These
// rows are disjoint from the rows the copies write.
template <int D, int kW>
__device__ __forceinline__ void zero_tail(char *buf, int n_valid, int tid) {
  using T = Tile<D>;
  for (int e = tid; e < kBN * T::kChunks; e += 64 * kW) {
    const int rho = e / T::kChunks, chi = e % T::kChunks;
    const uint4 z = make_uint4(0, 0, 0, 0);
    if (k_row_key(rho) >= n_valid) *reinterpret_cast<uint4 *>(buf + rho * T::kRowBytes + chi * 16) = z;
    if (rho >= n_valid) *reinterpret_cast<uint4 *>(buf + T::kBytes + rho * T::kRowBytes + chi * 16) = z;
  }
}

#endif  // __HIP_DEVICE_COMPILE__

// max (sum) over lanes l and l^32, the two halves holding one query's keys.
__device__ __forceinline__ float half_swap_max(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Online-softmax bookkeeping of one lane's query.
struct RowState {
  float m_ref;   // reference maximum (base 2) the accumulators are relative to
  float m_run;   // true running maximum (base 2)
  float l;       // this lane's partial row sum
};

// Scores of the wavefront's 32 queries against the 64-key tile: lane (r, h)
// holds s[sb][i] for key 32sb + 16(i/8) + 8h + i%8 of the tile.

// Keys beyond `lim` (key_base = k0 + 8h) become -inf.
__device__ __forceinline__ void mask_tile(f32x16 (&s)[2], int key_base, int lim) {
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = key_base + sb * 32 + (i >> 3) * 16 + (i & 7);
      s[sb][i] = key > lim ? -INFINITY : s[sb][i];
    }
}

// Updates the row state and produces P as four bf16 B-operand fragments.
// Returns the O rescale factor; `rescale` is set when any lane of the
// wavefront needs it.
__device__ __forceinline__ float softmax_tile(const f32x16 (&s)[2], RowState &rs, bf16x8 (&pb)[4],
                                              float sl2, bool &rescale) {
  float mx = -INFINITY;
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[sb][i]);
  mx = half_swap_max(mx);
  const float mt = mx * sl2;
  rs.m_run = fmaxf(rs.m_run, mt);
  const bool need = mt > rs.m_ref + kTau;
  const float m_new = need ? mt : rs.m_ref;
  const float alpha = need ? __builtin_amdgcn_exp2f(rs.m_ref - m_new) : 1.f;
  rescale = __any(need);
  rs.m_ref = m_new;
  rs.l *= alpha;
  const float neg_m = (m_new == -INFINITY) ? 0.f : -m_new;
  float lsum[4] = {0.f, 0.f, 0.f, 0.f};   // four independent add chains
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[sb][half * 8 + j], sl2, neg_m));
        lsum[j & 3] += p;
        pb[sb * 2 + half][j] = (__bf16)p;
      }
  rs.l += (lsum[0] + lsum[1]) + (lsum[2] + lsum[3]);
  return alpha;
}

template <int D, bool kDiag, int kW>
__global__ void __launch_bounds__(64 * kW, 8 / kW) step_bf16_kernel(StepArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  using T = Tile<D>;
  constexpr int kBM = 32 * kW;  // query rows per workgroup
  constexpr int kQK = D / 16;   // k-chunks of the score product
  constexpr int kDB = D / 32;   // 32-row blocks of O^T
  extern __shared__ __attribute__((aligned(1024))) char lds[];

  const int rows = a.rows;
  const int n_qt = (rows + kBM - 1) / kBM;
  // Workgroup -> (head, query tile).  Consecutive workgroup ids go to
  // different XCDs; when the head count allows, give each XCD a contiguous
  // range of heads so that one head's key/value tiles stay in one L2.
  int bh, qi;
  {
    const int bid = blockIdx.x;
    if ((a.bh & 7) == 0) {
      const int per_xcd = (a.bh >> 3) * n_qt;
      const int logical = (bid & 7) * per_xcd + (bid >> 3);
      bh = logical / n_qt;
      qi = logical % n_qt;
    } else {
      bh = bid / n_qt;
      qi = bid % n_qt;
    }
  }
  // Diagonal blocks: heaviest query tiles first.
  const int qt = kDiag ? n_qt - 1 - qi : qi;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int r = lane & 31, h = lane >> 5;
  const int q0w = qt * kBM + wave * 32;
  const int row = q0w + r;
  const bool row_ok = row < rows;

  const size_t base = (size_t)bh * rows * D;
  const uint16_t *__restrict__ Q = static_cast<const uint16_t *>(a.q) + base;
  float *__restrict__ O = a.o + base;
  const uint32_t blk_bytes = (uint32_t)rows * T::kRowBytes;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(static_cast<const uint16_t *>(a.k) + base, blk_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(static_cast<const uint16_t *>(a.v) + base, blk_bytes);
  const Stage<D, kW> so = stage_offsets<D, kW>(wave, lane);

  const int kv_end = kDiag ? min(rows, qt * kBM + kBM) : rows;
  const int n_tiles = (kv_end + kBN - 1) / kBN;
  // A ragged last tile that is the first use of its LDS buffer must not see
  // uninitialised LDS past the block end: zero those rows.  A later buffer
  // use holds finite keys/values of an earlier full tile there, which the
  // mask (keys) and the zero probabilities (values) already neutralise.
  const int last = n_tiles - 1;
  if (last <= 1 && last * kBN + kBN > rows)
    zero_tail<D, kW>(lds + (last & 1) * T::kBufBytes, rows - last * kBN, tid);
  issue_tile<D, kW>(lds, rk, rv, so, 0, wave);

  // Q^T fragments: lane (r, h) holds q[row][16c + 8h .. 16c + 8h + 7].
  bf16x8 qf[kQK];
  // O^T accumulators: block b, entry i <-> column 32b + 8(i/4) + 4h + i%4.
  f32x16 oacc[kDB];
  RowState rs;
  {
    const size_t ro = (size_t)row * D;
#pragma unroll
    for (int c = 0; c < kQK; ++c) {
      uint4 u = row_ok ? *reinterpret_cast<const uint4 *>(Q + ro + c * 16 + h * 8)
                       : make_uint4(0, 0, 0, 0);
      qf[c] = __builtin_bit_cast(bf16x8, u);
    }
#pragma unroll
    for (int b = 0; b < kDB; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float4 x = row_ok ? *reinterpret_cast<const float4 *>(O + ro + b * 32 + g * 8 + h * 4)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
        oacc[b][4 * g + 0] = x.x;
        oacc[b][4 * g + 1] = x.y;
        oacc[b][4 * g + 2] = x.z;
        oacc[b][4 * g + 3] = x.w;
      }
    const size_t sr = (size_t)bh * rows + row;
    const float m_state = row_ok ? a.m[sr] * kLog2e : -INFINITY;
    rs.m_ref = m_state;
    rs.m_run = m_state;
    rs.l = (row_ok && h == 0) ? a.l[sr] : 0.f;
  }

  // Per-lane LDS byte offsets of the fragments within a tile buffer.
  //   K fragment (sb, c): row 32sb + r, chunk (2c + h) swizzled by the row.
  //   V^T fragment (b, c), transposed read rr: row 16c + 4rr + 8(g/2) + j/4,
  //   column 32b + 16(g%2) + 4(j%4), with g = lane/16 and j = lane%16.
  uint32_t koff[kQK];
#pragma unroll
  for (int c = 0; c < kQK; ++c)
    koff[c] = (uint32_t)(r * T::kRowBytes + (((2 * c + h) ^ k_swz(r)) * 16));
  uint32_t voff[kDB];
  {
    const int g = lane >> 4, j = lane & 15;
    const int vrow = 8 * (g >> 1) + (j >> 2);
#pragma unroll
    for (int b = 0; b < kDB; ++b) {
      const int chunk = 4 * b + 2 * (g & 1) + ((j & 3) >> 1);
      voff[b] = (uint32_t)(vrow * T::kRowBytes + ((chunk ^ v_swz(vrow)) * 16) + 8 * (j & 1));
    }
  }

  const float sl2 = a.scale_log2;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();   // tile 0 (and a zeroed tail) visible to every wavefront

#pragma clang loop unroll(disable)
  for (int t = 0; t < n_tiles; ++t) {
    const int k0 = t * kBN;
    const char *cur = lds + (t & 1) * T::kBufBytes;
    if (t + 1 < n_tiles) issue_tile<D, kW>(lds + ((t + 1) & 1) * T::kBufBytes, rk, rv, so, k0 + kBN, wave);

    // Whole tile beyond every row of this wavefront (diagonal only): skip.
    const bool wave_skip = kDiag && k0 > q0w + 31;
    const bool need_mask = (kDiag && k0 + kBN - 1 > q0w) || (k0 + kBN > rows);
    if (!wave_skip) {
      f32x16 s[2];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        s[sb] = f32x16{};
#pragma unroll
        for (int c = 0; c < kQK; ++c) {
          const bf16x8 kf = *(const lds_bf16x8 *)(cur + sb * 32 * T::kRowBytes + koff[c]);
          s[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[c], s[sb], 0, 0, 0);
        }
      }
      if (need_mask) mask_tile(s, k0 + h * 8, kDiag ? min(row, rows - 1) : rows - 1);
      bf16x8 pb[4];
      bool rescale;
      const float alpha = softmax_tile(s, rs, pb, sl2, rescale);
      if (rescale) {
#pragma unroll
        for (int b = 0; b < kDB; ++b) oacc[b] *= alpha;
      }
      const char *vt = cur + T::kBytes;
#pragma unroll
      for (int b = 0; b < kDB; ++b)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const char *p0 = vt + (16 * c) * T::kRowBytes + voff[b];
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p0);
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p0 + 4 * T::kRowBytes));
          const bf16x8 vf =
              __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          oacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[c], oacc[b], 0, 0, 0);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);   // this wavefront's copies of tile t+1 have landed
    __syncthreads();
  }

  // ---- back to the canonical state (m = true running maximum) --------------
  const float l_tot = half_swap_sum(rs.l);
  const float beta = (rs.m_run == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(rs.m_ref - rs.m_run);
  if (row_ok) {
    const size_t ro = (size_t)row * D;
#pragma unroll
    for (int b = 0; b < kDB; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float4 x = make_float4(oacc[b][4 * g + 0] * beta, oacc[b][4 * g + 1] * beta,
                               oacc[b][4 * g + 2] * beta, oacc[b][4 * g + 3] * beta);
        *reinterpret_cast<float4 *>(O + ro + b * 32 + g * 8 + h * 4) = x;
      }
    if (h == 0) {
      const size_t sr = (size_t)bh * rows + row;
      a.m[sr] = rs.m_run * kLn2;
      a.l[sr] = l_tot * beta;
    }
  }
#endif  // __HIP_DEVICE_COMPILE__
}

template <int D, bool kDiag, int kW>
hipError_t launch(const StepArgs &a, hipStream_t s) {
  constexpr int kBM = 32 * kW;
  const int n_qt = (a.rows + kBM - 1) / kBM;
  const dim3 grid((unsigned)((int64_t)a.bh * n_qt)), block(64 * kW);
  step_bf16_kernel<D, kDiag, kW><<<grid, block, Tile<D>::kLdsBytes, s>>>(a);
  return hipGetLastError();
}

// Full blocks: 8-wavefront workgroups (256 query rows share each key/value
// tile).  Diagonal blocks: 4-wavefront workgroups, whose finer query tiles
// waste less work on the masked triangle and balance better.
template <int D, bool kDiag>
hipError_t launch_d(const StepArgs &a, hipStream_t s) {
  if (kDiag) return launch<D, kDiag, 4>(a, s);
  return launch<D, kDiag, 8>(a, s);
}

}  // namespace

hipError_t launch_step_bf16(const StepArgs &a, int d, StepCase c, hipStream_t s) {
  const bool diag = c == StepCase::Diag;
  if (d == 128) return diag ? launch_d<128, true>(a, s) : launch_d<128, false>(a, s);
  return diag ? launch_d<64, true>(a, s) : launch_d<64, false>(a, s);
}

}  // namespace ra
