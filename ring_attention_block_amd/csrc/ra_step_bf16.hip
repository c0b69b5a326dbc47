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
// Design (one workgroup = 4 wavefronts = 128 query rows of one head):
//  * Each wavefront owns 32 query rows.  Its Q rows stay in VGPRs for the
//    whole block, as the B operand of v_mfma_f32_32x32x16_bf16.
//  * Key/value tiles of 64 keys are double-buffered in LDS.  The global loads
//    of tile n+1 are issued before the matrix work of tile n and written to
//    the other LDS buffer after it, so one barrier per tile suffices.  Keys
//    are stored row-major; values are stored transposed (d-major) so both
//    products read 16 contiguous bytes per lane.
//  * Scores are produced transposed, S^T = K Q^T, so each lane holds one
//    query (lane % 32) and 32 of its keys.  The LDS rows of K are read in the
//    permuted order pi(r) (bits 2 and 3 of r swapped), which makes the 8 keys
//    in each half of a lane's accumulator contiguous; those registers are then
//    directly the B operand of O^T += V^T P^T without any lane exchange, and
//    the row statistics (max, sum, rescale factor) are per-lane values.
//  * The softmax works in base 2: p = exp2(s_raw * scale*log2(e) - m2), one
//    FMA and one v_exp_f32 per score.  The rescale of O is lazy: the
//    reference maximum only moves when a tile's maximum exceeds it by more
//    than kTau (so every p <= 2^kTau, safe in fp32 and bf16), and the true
//    running maximum is tracked beside it.  On exit the state is rescaled
//    once to the true maximum, so the stored state is canonical.
//  * Lanes l and l+32 hold the same query with disjoint keys: their partial
//    row sums are added once at the end of the block.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "ra_kernels.h"

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 128;       // query rows per workgroup
constexpr int kBN = 64;        // keys per tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kTau = 8.0f;   // lazy-rescale threshold, base-2 units
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963407f;

template <int D>
struct Tile {
  static constexpr int kKS = D + 8;                 // K row stride in LDS (bf16)
  static constexpr int kVS = kBN + 8;               // V^T row stride in LDS (bf16)
  static constexpr int kKElems = kBN * kKS;
  static constexpr int kVElems = D * kVS;
  static constexpr int kKChunks = kBN * D / 8 / kThreads;   // 16-byte K loads per thread
  static constexpr int kDChunks = D / 8;                    // 8-column chunks per row
  static constexpr int kKeyGroups = kThreads / kDChunks;    // V: key groups per tile
  static constexpr int kKeysPerGroup = kBN / kKeyGroups;    // V: keys per thread
  static constexpr size_t kLdsBytes = 2 * (kKElems + kVElems) * sizeof(uint16_t);
  static_assert(kBN * D / 8 % kThreads == 0, "K tile must split evenly");
  static_assert(kKeysPerGroup == 2 || kKeysPerGroup == 4, "V packing assumes 2 or 4 keys");
};

// Row of the K tile that feeds MFMA row r (0..31): swap bits 2 and 3.
__device__ __forceinline__ int perm_row(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

template <int D>
struct Prefetch {
  uint4 k[Tile<D>::kKChunks];
  uint4 v[Tile<D>::kKeysPerGroup];
};

// Global -> registers for the tile starting at key k0 (rows past the block end
// are zero so that masked lanes never see NaN garbage).
template <int D>
__device__ __forceinline__ void load_tile(Prefetch<D> &pf, const uint16_t *__restrict__ K,
                                          const uint16_t *__restrict__ V, int k0, int rows,
                                          int tid) {
  using T = Tile<D>;
#pragma unroll
  for (int n = 0; n < T::kKChunks; ++n) {
    const int c = tid + n * kThreads;
    const int kr = c / T::kDChunks, cc = c % T::kDChunks;
    pf.k[n] = (k0 + kr < rows)
                  ? *reinterpret_cast<const uint4 *>(K + (size_t)(k0 + kr) * D + cc * 8)
                  : make_uint4(0, 0, 0, 0);
  }
  const int dc = tid % T::kDChunks, kg = tid / T::kDChunks;
#pragma unroll
  for (int n = 0; n < T::kKeysPerGroup; ++n) {
    const int kr = kg * T::kKeysPerGroup + n;
    pf.v[n] = (k0 + kr < rows)
                  ? *reinterpret_cast<const uint4 *>(V + (size_t)(k0 + kr) * D + dc * 8)
                  : make_uint4(0, 0, 0, 0);
  }
}

__device__ __forceinline__ uint32_t lo_pair(uint32_t a, uint32_t b) {
  return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t hi_pair(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xffff0000u);
}

// Registers -> LDS: K row-major, V transposed to [d][key].
template <int D>
__device__ __forceinline__ void store_tile(const Prefetch<D> &pf, uint16_t *__restrict__ ks,
                                           uint16_t *__restrict__ vts, int tid) {
  using T = Tile<D>;
#pragma unroll
  for (int n = 0; n < T::kKChunks; ++n) {
    const int c = tid + n * kThreads;
    const int kr = c / T::kDChunks, cc = c % T::kDChunks;
    *reinterpret_cast<uint4 *>(ks + kr * T::kKS + cc * 8) = pf.k[n];
  }
  const int dc = tid % T::kDChunks, kg = tid / T::kDChunks;
  const int key0 = kg * T::kKeysPerGroup;
  const uint32_t *w[T::kKeysPerGroup];
#pragma unroll
  for (int n = 0; n < T::kKeysPerGroup; ++n) w[n] = reinterpret_cast<const uint32_t *>(&pf.v[n]);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    uint16_t *dst = vts + (dc * 8 + e) * T::kVS + key0;
    const int wi = e >> 1;
    if constexpr (T::kKeysPerGroup == 4) {
      uint2 pk;
      pk.x = (e & 1) ? hi_pair(w[0][wi], w[1][wi]) : lo_pair(w[0][wi], w[1][wi]);
      pk.y = (e & 1) ? hi_pair(w[2][wi], w[3][wi]) : lo_pair(w[2][wi], w[3][wi]);
      *reinterpret_cast<uint2 *>(dst) = pk;
    } else {
      *reinterpret_cast<uint32_t *>(dst) =
          (e & 1) ? hi_pair(w[0][wi], w[1][wi]) : lo_pair(w[0][wi], w[1][wi]);
    }
  }
}

template <int D, bool kDiag>
__global__ void __launch_bounds__(kThreads, 2) step_bf16_kernel(StepArgs a) {
  using T = Tile<D>;
  constexpr int kQK = D / 16;   // k-chunks of the score product
  constexpr int kDB = D / 32;   // 32-row blocks of O^T
  extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
  // LDS: K tile buffers 0 and 1, then V^T tile buffers 0 and 1.
  auto ks_buf = [&](int i) { return lds + i * T::kKElems; };
  auto vt_buf = [&](int i) { return lds + 2 * T::kKElems + i * T::kVElems; };

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
  const int q0 = qt * kBM;
  const int q0w = q0 + wave * 32;
  const int row = q0w + r;
  const bool row_ok = row < rows;

  const size_t base = (size_t)bh * rows * D;
  const uint16_t *__restrict__ Q = static_cast<const uint16_t *>(a.q) + base;
  const uint16_t *__restrict__ K = static_cast<const uint16_t *>(a.k) + base;
  const uint16_t *__restrict__ V = static_cast<const uint16_t *>(a.v) + base;
  float *__restrict__ O = a.o + base;
  const size_t srow = (size_t)bh * rows + row;

  // Q^T fragments: lane (r, h) holds q[row][16c + 8h .. 16c + 8h + 7].
  bf16x8 qf[kQK];
#pragma unroll
  for (int c = 0; c < kQK; ++c) {
    uint4 u = row_ok ? *reinterpret_cast<const uint4 *>(Q + (size_t)row * D + c * 16 + h * 8)
                     : make_uint4(0, 0, 0, 0);
    qf[c] = __builtin_bit_cast(bf16x8, u);
  }

  // O^T accumulators: block b, entry i <-> column 32b + 8(i/4) + 4h + i%4.
  f32x16 oacc[kDB];
#pragma unroll
  for (int b = 0; b < kDB; ++b) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float4 x = row_ok
                     ? *reinterpret_cast<const float4 *>(O + (size_t)row * D + b * 32 + g * 8 + h * 4)
                     : make_float4(0.f, 0.f, 0.f, 0.f);
      oacc[b][4 * g + 0] = x.x;
      oacc[b][4 * g + 1] = x.y;
      oacc[b][4 * g + 2] = x.z;
      oacc[b][4 * g + 3] = x.w;
    }
  }
  const float m_state = row_ok ? a.m[srow] * kLog2e : -INFINITY;
  float m_ref = m_state;   // reference maximum the accumulators are relative to
  float m_run = m_state;   // true running maximum (base 2)
  float l_part = (row_ok && h == 0) ? a.l[srow] : 0.f;

  const int kv_end = kDiag ? min(rows, q0 + kBM) : rows;
  const int n_tiles = (kv_end + kBN - 1) / kBN;
  const float sl2 = a.scale_log2;

  Prefetch<D> pf;
  load_tile<D>(pf, K, V, 0, rows, tid);
  store_tile<D>(pf, ks_buf(0), vt_buf(0), tid);
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int k0 = t * kBN;
    const bool more = t + 1 < n_tiles;
    if (more) load_tile<D>(pf, K, V, k0 + kBN, rows, tid);

    const uint16_t *ks = ks_buf(t & 1);
    const uint16_t *vts = vt_buf(t & 1);
    // Whole tile beyond every row of this wave (diagonal only): nothing to do.
    const bool wave_skip = kDiag && k0 > q0w + 31;
    if (!wave_skip) {
      // ---- S^T = K Q^T for two 32-key halves -------------------------------
      f32x16 s[2];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        s[sb] = f32x16{};
        const uint16_t *kr = ks + (sb * 32 + perm_row(r)) * T::kKS + h * 8;
#pragma unroll
        for (int c = 0; c < kQK; ++c) {
          bf16x8 kf = *reinterpret_cast<const bf16x8 *>(kr + c * 16);
          s[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[c], s[sb], 0, 0, 0);
        }
      }
      // Lane (r, h), half sb, entry i <-> key k0 + 32sb + 16(i/8) + 8h + i%8.
      const bool need_mask = (kDiag && k0 + kBN - 1 > q0w) || (k0 + kBN > rows);
      if (need_mask) {
        const int lim = kDiag ? min(row, rows - 1) : rows - 1;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = k0 + sb * 32 + (i >> 3) * 16 + h * 8 + (i & 7);
            if (key > lim) s[sb][i] = -INFINITY;
          }
      }
      // ---- row maximum ------------------------------------------------------
      float mx = -INFINITY;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[sb][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mt = mx * sl2;
      m_run = fmaxf(m_run, mt);
      const bool need = mt > m_ref + kTau;
      if (__any(need)) {
        const float m_new = need ? mt : m_ref;
        const float alpha = need ? __builtin_amdgcn_exp2f(m_ref - m_new) : 1.f;
        m_ref = m_new;
        l_part *= alpha;
#pragma unroll
        for (int b = 0; b < kDB; ++b) oacc[b] *= alpha;
      }
      const float neg_m = (m_ref == -INFINITY) ? 0.f : -m_ref;
      // ---- p = exp2(s*scale*log2e - m), row sum, bf16 pack -----------------
      bf16x8 pb[4];
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float p = __builtin_amdgcn_exp2f(fmaf(s[sb][half * 8 + j], sl2, neg_m));
            l_part += p;
            pb[sb * 2 + half][j] = (__bf16)p;
          }
        }
      // ---- O^T += V^T P^T ---------------------------------------------------
#pragma unroll
      for (int b = 0; b < kDB; ++b) {
        const uint16_t *vr = vts + (b * 32 + r) * T::kVS + h * 8;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          bf16x8 vf = *reinterpret_cast<const bf16x8 *>(vr + c * 16);
          oacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[c], oacc[b], 0, 0, 0);
        }
      }
    }
    if (more) store_tile<D>(pf, ks_buf((t + 1) & 1), vt_buf((t + 1) & 1), tid);
    __syncthreads();
  }

  // ---- back to the canonical state (m = true running maximum) --------------
  const float l_tot = l_part + __shfl_xor(l_part, 32);
  const float beta = (m_run == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_run);
  if (row_ok) {
#pragma unroll
    for (int b = 0; b < kDB; ++b) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float4 x = make_float4(oacc[b][4 * g + 0] * beta, oacc[b][4 * g + 1] * beta,
                               oacc[b][4 * g + 2] * beta, oacc[b][4 * g + 3] * beta);
        *reinterpret_cast<float4 *>(O + (size_t)row * D + b * 32 + g * 8 + h * 4) = x;
      }
    }
    if (h == 0) {
      a.m[srow] = m_run * kLn2;
      a.l[srow] = l_tot * beta;
    }
  }
}

template <int D, bool kDiag>
hipError_t launch(const StepArgs &a, hipStream_t s) {
  const int n_qt = (a.rows + kBM - 1) / kBM;
  const dim3 grid((unsigned)((int64_t)a.bh * n_qt)), block(kThreads);
  step_bf16_kernel<D, kDiag><<<grid, block, Tile<D>::kLdsBytes, s>>>(a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_step_bf16(const StepArgs &a, int d, StepCase c, hipStream_t s) {
  const bool diag = c == StepCase::Diag;
  if (d == 128) return diag ? launch<128, true>(a, s) : launch<128, false>(a, s);
  return diag ? launch<64, true>(a, s) : launch<64, false>(a, s);
}

}  // namespace ra
