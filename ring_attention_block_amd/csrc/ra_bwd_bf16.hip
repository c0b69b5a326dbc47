// Backward of one ring step for bf16 inputs (head_dim 64 or 128) on the CDNA4
// matrix cores ("Ring Attention：把超长序列沿设备环流动", section "Backward
// 需要让梯度也沿环传播": the query owner accumulates dQ, the dK and dV of the
// visiting block accumulate while it travels; the probabilities are recomputed
// from the saved per-row log-sum-exp as in the FlashAttention backward):
//     P  = exp(scale q.k - LSE)          (0 where the causal mask hides the key)
//     dP = dO . v,   dS = P (dP - D),    D = rowsum(dO * O)
//     dQ += scale dS K,   dK += scale dS^T Q,   dV += P^T dO
//
// Two kernels per step, each owning its outputs (no atomics, so the result
// does not depend on the order workgroups run in):
//  * bwd_dq: query-stationary.  A wavefront holds 32 query rows of Q and dO in
//    registers and the dQ^T accumulator; 64-row key/value tiles stream through
//    LDS.  Per tile it forms S^T = K Q^T and dP^T = V dO^T (keys on the
//    register axis, queries on lanes, so LSE and D are per-lane values), then
//    dS^T and dQ^T += K^T dS^T.
//  * bwd_dkdv: key-stationary.  A wavefront holds 32 keys of K and V in
//    registers and the dK^T, dV^T accumulators; 64-row query tiles of Q, dO
//    (and their LSE and D) stream through LDS.  Per tile S = Q K^T and
//    dP = dO V^T (queries on the register axis, keys on lanes), then
//    dV^T += dO^T P and dK^T += Q^T dS.
// Each kernel recomputes S and dP; together they issue 7 products of the
// 64x64x128 tile shape where the gradients need 5.
//
// All products use v_mfma_f32_32x32x16_bf16 (lane l holds A[l%32][8(l/32)..]
// and B[8(l/32)..][l%32]; accumulator entry i of lane l is D[8(i/4) + 4(l/32)
// + i%4][l%32]).  Every streamed tile (64 rows x head_dim bf16) has the same LDS
// layout:
//  * physical row rho holds tile row kappa(rho), which swaps bits 2 and 3, so
//    accumulator entries 8(i/8)..8(i/8)+7 of a product whose A operand is
//    read row by row are 8 consecutive tile rows: they are directly the B
//    operand (or, transposed, the A operand) of the next product;
//  * the 16-byte chunks of each row are XOR-swizzled by
//    f(rho) = sigma(rho & 3) ^ ((rho >> 2) & 3), sigma = {0, 6, 10, 12} at
//    head_dim 128 (another f at 64, see swz), which
//    keeps both access patterns free of bank conflicts: 16-byte reads of 16
//    consecutive rows at one chunk (f is a permutation of 0..15 over them, and
//    of 0..7 modulo 8 over each aligned 8), and the transposing reads
//    ds_read_b64_tr_b16 of 4 consecutive rows x 64 bytes (the four rows land in
//    four different 64-byte quads, and in distinct halves of 128 bytes).
//  * tiles are copied HBM -> LDS by buffer loads with an LDS destination
//    (double buffered in bwd_dq, triple in bwd_dkdv), one barrier per tile.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "ra_kernels.h"

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) float4 lds_float4;

using NoMask = std::integral_constant<bool, false>;
using MayMask = std::integral_constant<bool, true>;

constexpr int kBT = 64;        // rows per streamed tile
constexpr int kWaves = 4;      // wavefronts per workgroup
constexpr float kLog2e = 1.442695040888963407f;

template <int D>
struct BTile {
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  static constexpr int kRowBytes = D * 2;
  static constexpr int kBytes = kBT * kRowBytes;
  static constexpr int kChunks = D / 8;
  static constexpr int kRowsPerLoad = 1024 / kRowBytes;
  static constexpr int kLoads = kBytes / 1024;
  static constexpr int kLoadsPerWave = kLoads / kWaves;
};

__device__ __forceinline__ int kappa(int rho) {
  return (rho & ~12) | ((rho & 4) << 1) | ((rho & 8) >> 1);
}
// 16-byte chunk swizzle of a tile row (see the layout notes above).  With
// head_dim 64 a row has 8 chunks (128 bytes, two rows per 256 bytes of banks):
// f(rho) = 2(rho & 3) ^ ((rho >> 2) & 3) is a permutation of 0..7 over every
// aligned 8 rows and over the even and the odd rows of every aligned 16 (the
// 16-byte reads), and over every aligned 4 rows f/2 takes four distinct values
// with bit 2 differing between rows two apart (the transposing reads).
template <int D>
__device__ __forceinline__ int swz(int rho) {
  const int x = rho & 3;
  if constexpr (D == 128) return (4 * x + 2 * ((x ^ (x >> 1)) & 1)) ^ ((rho >> 2) & 3);
  else return (2 * x) ^ ((rho >> 2) & 3);
}

// Workgroup -> (batch*head, tile): consecutive workgroup ids go to different
// XCDs; when the head count allows, each XCD gets a contiguous range of heads
// so that the tiles of one head stay in one L2.  Within an XCD workgroups
// start in id order; tile_major (diagonal blocks, whose tiles carry unequal
// work) walks tile 0 of every head, then tile 1, ..., so the heaviest tiles
// of all heads start first and the light ones fill in at the end; otherwise
// one head's tiles follow another's.
__device__ __forceinline__ void xcd_map(int bid, int n_bh, int n_t, bool tile_major, int &bh,
                                        int &ti) {
  if ((n_bh & 7) == 0) {
    const int heads8 = n_bh >> 3, k = bid >> 3, x = bid & 7;
    if (tile_major) {
      bh = x * heads8 + k % heads8;
      ti = k / heads8;
    } else {
      const int logical = x * heads8 * n_t + k;
      bh = logical / n_t;
      ti = logical % n_t;
    }
  } else if (tile_major) {
    bh = bid % n_bh;
    ti = bid / n_bh;
  } else {
    bh = bid / n_t;
    ti = bid % n_t;
  }
}

#if defined(__HIP_DEVICE_COMPILE__)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, bytes, 0x00020000);
}

// Per-lane source offsets (within a tile) of this wavefront's share of the
// copies: load n writes LDS bytes n*1024 + 16*lane, i.e. physical row
// 4n + lane/16, physical chunk lane%16, which holds tile row kappa(row) and
// logical chunk (lane%16) ^ f(row).
template <int D>
__device__ __forceinline__ void copy_offsets(uint32_t (&off)[BTile<D>::kLoadsPerWave], int wave, int lane) {
  using T = BTile<D>;
#pragma unroll
  for (int i = 0; i < T::kLoadsPerWave; ++i) {
    const int n = wave + i * kWaves;
    const int rho = n * T::kRowsPerLoad + lane / T::kChunks;
    const int chi = lane % T::kChunks;
    off[i] = (uint32_t)(kappa(rho) * T::kRowBytes + ((chi ^ swz<D>(rho)) * 16));
  }
}

// Copy tile rows row0 .. row0+63 into `buf`.  The tile offset is in the
// per-lane offset, which the buffer range check covers: rows past the end are
// not written.
template <int D>
__device__ __forceinline__ void issue_copy(char *buf, __amdgpu_buffer_rsrc_t rsrc,
                                           const uint32_t (&off)[BTile<D>::kLoadsPerWave], int row0,
                                           int wave) {
  using T = BTile<D>;
  const uint32_t toff = (uint32_t)row0 * T::kRowBytes;
#pragma unroll
  for (int i = 0; i < T::kLoadsPerWave; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void *)(buf + (wave + i * kWaves) * 1024), 16,
                                             off[i] + toff, 0, 0, 0);
}

// Zero the rows of two tile buffers that hold tile rows >= n_valid (the first
// use of a buffer by a ragged last tile; later uses hold finite stale rows,
// which the zero probabilities neutralise).
template <int D>
__device__ __forceinline__ void zero_tail(char *b0, char *b1, int n_valid, int tid) {
  using T = BTile<D>;
  for (int e = tid; e < kBT * T::kChunks; e += 64 * kWaves) {
    const int rho = e / T::kChunks, chi = e % T::kChunks;
    if (kappa(rho) >= n_valid) {
      const uint4 z = make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4 *>(b0 + rho * T::kRowBytes + chi * 16) = z;
      *reinterpret_cast<uint4 *>(b1 + rho * T::kRowBytes + chi * 16) = z;
    }
  }
}
#endif  // __HIP_DEVICE_COMPILE__

// Per-lane LDS offsets of the two fragment reads.
//  normal (A operand, tile rows as the M index, head_dim chunk c as K):
//    physical row r (+32 sb), logical chunk 2c + h.
//  transposed (A operand X^T: head_dim rows 32b.. as M, 16 tile rows of chunk
//    cc as K): two reads e = 0, 1 of physical rows 16cc + 8e + 4h + j/4
//    (tile rows 16cc + 8h + 4e + j/4), head_dim columns 32b + 16(g%2) + 4(j%4),
//    g = lane/16, j = lane%16; lane i of each 16 receives column 32b + 16(g%2)
//    + i of four consecutive tile rows.
template <int D>
struct FragOffsets {
  uint32_t nrm[D / 16];
  uint32_t tr[D / 32][2];
};

template <int D>
__device__ __forceinline__ FragOffsets<D> frag_offsets(int lane) {
  using T = BTile<D>;
  FragOffsets<D> fo;
  const int r = lane & 31, h = lane >> 5, g = lane >> 4, j = lane & 15;
#pragma unroll
  for (int c = 0; c < D / 16; ++c)
    fo.nrm[c] = (uint32_t)(r * T::kRowBytes + (((2 * c + h) ^ swz<D>(r)) * 16));
#pragma unroll
  for (int b = 0; b < D / 32; ++b)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int rho = 8 * e + 4 * h + (j >> 2);
      const int chunk = 4 * b + 2 * (g & 1) + ((j & 3) >> 1);
      fo.tr[b][e] = (uint32_t)(rho * T::kRowBytes + ((chunk ^ swz<D>(rho)) * 16) + 8 * (j & 1));
    }
  return fo;
}

template <int D>
__device__ __forceinline__ bf16x8 read_nrm(const char *buf, const FragOffsets<D> &fo, int sb, int c) {
  return *(const lds_bf16x8 *)(buf + sb * 32 * BTile<D>::kRowBytes + fo.nrm[c]);
}
template <int D>
__device__ __forceinline__ bf16x8 read_tr(const char *buf, const FragOffsets<D> &fo, int cc, int b) {
  const char *p = buf + cc * 16 * BTile<D>::kRowBytes;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p + fo.tr[b][0]));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p + fo.tr[b][1]));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ float neg_lse2(float lse) {
  return lse == -INFINITY ? -INFINITY : -lse * kLog2e;
}

// Add an accumulator X^T (entry i of block b <-> column 32b + 8(i/4) + 4h +
// i%4 of this lane's row) times `mul` into the fp32 row `dst`.
template <int D>
__device__ __forceinline__ void add_row(float *dst, const f32x16 (&acc)[D / 32], int h, float mul) {
#pragma unroll
  for (int b = 0; b < D / 32; ++b)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float4 *p = reinterpret_cast<float4 *>(dst + b * 32 + g * 8 + h * 4);
      float4 x = *p;
      x.x = fmaf(acc[b][4 * g + 0], mul, x.x);
      x.y = fmaf(acc[b][4 * g + 1], mul, x.y);
      x.z = fmaf(acc[b][4 * g + 2], mul, x.z);
      x.w = fmaf(acc[b][4 * g + 3], mul, x.w);
      *p = x;
    }
}

// ------------------------------------------------------------------ dQ ------
// Instruction order of one 32-key half of a dQ tile (one scheduling region):
// the fragment reads of the S/dP products issued eight ahead of the products
// that use them, then the softmax, then the dQ products with their
// transposing reads (two per product) issued four products ahead.  Without
// it the compiler reuses one register quad for every fragment and each
// product waits for its own read.  Masks: 0x008 MFMA, 0x100 LDS read, 0x402
// VALU and transcendental.
#define RA_DQ_INTERLEAVE(kQK_, kDB_)                                        \
  do {                                                                      \
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);                      \
    for (int i_ = 0; i_ < 2 * (kQK_) - 8; ++i_) {                           \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                    \
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                    \
    }                                                                       \
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);                      \
    __builtin_amdgcn_sched_group_barrier(0x402, 200, 0);                    \
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);                      \
    for (int i_ = 0; i_ < 2 * (kDB_) - 4; ++i_) {                           \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                    \
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);                    \
    }                                                                       \
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);                      \
    __builtin_amdgcn_sched_barrier(0);                                      \
  } while (0)
template <int D, bool kDiag, bool kMask>
__global__ void __launch_bounds__(64 * kWaves, 2) bwd_dq_bf16_kernel(BwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  using T = BTile<D>;
  constexpr int kBM = 32 * kWaves;
  constexpr int kQK = D / 16, kDB = D / 32;
  __shared__ __attribute__((aligned(1024))) char lds_k0[T::kBytes];
  __shared__ __attribute__((aligned(1024))) char lds_k1[T::kBytes];
  __shared__ __attribute__((aligned(1024))) char lds_v0[T::kBytes];
  __shared__ __attribute__((aligned(1024))) char lds_v1[T::kBytes];

  const int rows = a.rows;
  const int n_qt = (rows + kBM - 1) / kBM;
  int bh, qi;
  xcd_map(blockIdx.x, a.bh, n_qt, kDiag, bh, qi);
  const int qt = kDiag ? n_qt - 1 - qi : qi;   // diagonal: heaviest query tiles first

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 31, h = lane >> 5;
  const int q0w = qt * kBM + wave * 32;
  const int row = q0w + r;
  const bool row_ok = row < rows;
  const size_t base = (size_t)bh * rows * D;
  const uint32_t blk_bytes = (uint32_t)rows * T::kRowBytes;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(static_cast<const uint16_t *>(a.k) + base, blk_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(static_cast<const uint16_t *>(a.v) + base, blk_bytes);
  uint32_t coff[T::kLoadsPerWave];
  copy_offsets<D>(coff, wave, lane);

  const int kv_end = kDiag ? min(rows, qt * kBM + kBM) : rows;
  const int n_tiles = (kv_end + kBT - 1) / kBT;
  const int last = n_tiles - 1;
  if (last <= 1 && last * kBT + kBT > rows)
    zero_tail<D>((last & 1) ? lds_k1 : lds_k0, (last & 1) ? lds_v1 : lds_v0, rows - last * kBT, tid);
  issue_copy<D>(lds_k0, rk, coff, 0, wave);
  issue_copy<D>(lds_v0, rv, coff, 0, wave);

  // B operands: lane (r, h) holds q[row][16c + 8h ..] and do[row][16c + 8h ..].
  // Rows, LSE and D come through range-checked buffer loads (0 past the block
  // end), so no load sits under a branch (each would be waited for inside it)
  // and none is a flat access (which waits for the LDS copies before it).
  bf16x8 qf[kQK], of[kQK];
  float nl2, dd;
  {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(static_cast<const uint16_t *>(a.q) + base, blk_bytes);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(static_cast<const uint16_t *>(a.dout) + base, blk_bytes);
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(a.lse + (size_t)bh * rows, (uint32_t)rows * 4u);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(a.delta + (size_t)bh * rows, (uint32_t)rows * 4u);
#pragma unroll
    for (int c = 0; c < kQK; ++c) {
      const uint32_t off = (uint32_t)row * T::kRowBytes + (uint32_t)(c * 16 + h * 8) * 2;
      qf[c] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
      of[c] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(ro, off, 0, 0));
    }
    const float lse = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rl, (uint32_t)row * 4, 0, 0));
    const float del = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rd, (uint32_t)row * 4, 0, 0));
    nl2 = row_ok ? neg_lse2(lse) : -INFINITY;
    dd = row_ok ? del : 0.f;
  }
  f32x16 dq[kDB];
#pragma unroll
  for (int b = 0; b < kDB; ++b) dq[b] = f32x16{};
  const FragOffsets<D> fo = frag_offsets<D>(lane);
  const float sl2 = a.scale_log2;
  const int lim = kDiag ? min(row, rows - 1) : rows - 1;   // last key this row may see

  // may_mask (compile-time): the tile may need the element mask.
  auto body = [&](auto may_mask, int t, const char *kb, const char *vb) {
    constexpr bool kM = decltype(may_mask)::value;
    const bool masked = kM && ((kDiag && t * kBT + kBT - 1 > q0w) || (t * kBT + kBT > rows));
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int c = 0; c < kQK; ++c) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_nrm<D>(kb, fo, sb, c), qf[c], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_nrm<D>(vb, fo, sb, c), of[c], dp, 0, 0, 0);
      }
      // s[i], dp[i]: key t*64 + 32sb + 16(i/8) + 8h + i%8 of this lane's row.
      bf16x8 dsb[2];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float p = __builtin_amdgcn_exp2f(fmaf(s[i], sl2, nl2));
        if (masked) {
          const int key = t * kBT + sb * 32 + (i >> 3) * 16 + 8 * h + (i & 7);
          p = key > lim ? 0.f : p;
        }
        dsb[i >> 3][i & 7] = (__bf16)(p * (dp[i] - dd));
      }
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int b = 0; b < kDB; ++b)
          dq[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_tr<D>(kb, fo, 2 * sb + half, b), dsb[half],
                                                          dq[b], 0, 0, 0);
      if constexpr (!kM) RA_DQ_INTERLEAVE(kQK, kDB);
    }
  };
  auto iteration = [&](auto may_mask, int t, char *k_dst, char *v_dst, const char *k_src,
                       const char *v_src) {
    if (t + 1 < n_tiles) {
      issue_copy<D>(k_dst, rk, coff, (t + 1) * kBT, wave);
      issue_copy<D>(v_dst, rv, coff, (t + 1) * kBT, wave);
    }
    if (!(kDiag && t * kBT > q0w + 31)) body(may_mask, t, k_src, v_src);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  int t = 0;
  if constexpr (kMask) {
    // The tiles before the first that needs the element mask for this
    // wavefront (on the diagonal: keys before all of its rows; else the
    // ragged last tile) run without it.  Every wavefront runs n_tiles
    // iterations with one barrier each.
    const int first_diag = kDiag ? (q0w >= kBT - 1 ? (q0w - (kBT - 1)) / kBT + 1 : 0) : n_tiles;
    const int first_tail = rows >= kBT ? (rows - kBT) / kBT + 1 : 0;
    const int n_fast = min(min(first_diag, first_tail), n_tiles);
#pragma clang loop unroll(disable)
    for (; t + 1 < n_fast; t += 2) {
      iteration(NoMask{}, t, lds_k1, lds_v1, lds_k0, lds_v0);
      iteration(NoMask{}, t + 1, lds_k0, lds_v0, lds_k1, lds_v1);
    }
    if (t < n_fast) {
      iteration(NoMask{}, t, lds_k1, lds_v1, lds_k0, lds_v0);
      ++t;
      if (t < n_tiles) iteration(MayMask{}, t, lds_k0, lds_v0, lds_k1, lds_v1);
      ++t;
    }
#pragma clang loop unroll(disable)
    for (; t + 1 < n_tiles; t += 2) {
      iteration(MayMask{}, t, lds_k1, lds_v1, lds_k0, lds_v0);
      iteration(MayMask{}, t + 1, lds_k0, lds_v0, lds_k1, lds_v1);
    }
    if (t < n_tiles) iteration(MayMask{}, t, lds_k1, lds_v1, lds_k0, lds_v0);
  } else {
#pragma clang loop unroll(disable)
    for (; t + 1 < n_tiles; t += 2) {
      iteration(NoMask{}, t, lds_k1, lds_v1, lds_k0, lds_v0);
      iteration(NoMask{}, t + 1, lds_k0, lds_v0, lds_k1, lds_v1);
    }
    if (t < n_tiles) iteration(NoMask{}, t, lds_k1, lds_v1, lds_k0, lds_v0);
  }

  if (row_ok) add_row<D>(a.dq + base + (size_t)row * D, dq, h, a.scale);
#endif  // __HIP_DEVICE_COMPILE__
}

// ---------------------------------------------------------------- dK, dV ----
// The two halves of a dK/dV iteration are scheduled as separate regions: the
// compiler then interleaves each half's softmax with its products instead of
// hoisting work across the halves and raising register pressure.
#define RA_DKDV_HALF_END() __builtin_amdgcn_sched_barrier(0)
// One wavefront per SIMD (the dK^T and dV^T accumulators take 128 registers
// beside the 64 of K and V), so the work is software-pipelined by 32-query
// sub-tiles instead of relying on a second wavefront: while the matrix cores
// run the dV/dK products of sub-tile n and the S/dP products of sub-tile n+1,
// the vector unit turns the S/dP of sub-tile n into P and dS.  A tile is read
// from the iteration before it is current until the end of its own iteration,
// so query tiles are triple buffered: iteration u computes on tiles u and u+1
// while tile u+2 is copied in.
template <int D, bool kDiag>
__global__ void __launch_bounds__(64 * kWaves, D == 128 ? 1 : 2) bwd_dkdv_bf16_kernel(BwdArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  using T = BTile<D>;
  constexpr int kBK = 32 * kWaves;
  constexpr int kQK = D / 16, kDB = D / 32;
  __shared__ __attribute__((aligned(1024))) char lds_q0[T::kBytes];
  __shared__ __attribute__((aligned(1024))) char lds_q1[T::kBytes];
  __shared__ __attribute__((aligned(1024))) char lds_q2[T::kBytes];
  __shared__ __attribute__((aligned(1024))) char lds_o0[T::kBytes];
  __shared__ __attribute__((aligned(1024))) char lds_o1[T::kBytes];
  __shared__ __attribute__((aligned(1024))) char lds_o2[T::kBytes];
  // Per query of a tile: -LSE * log2(e) (-inf for a row past the end or one
  // that saw no key) and D.
  __shared__ __attribute__((aligned(16))) float lds_nl[3][kBT];
  __shared__ __attribute__((aligned(16))) float lds_dd[3][kBT];

  const int rows = a.rows;
  const int n_kt = (rows + kBK - 1) / kBK;
  int bh, kt;
  xcd_map(blockIdx.x, a.bh, n_kt, kDiag, bh, kt);   // diagonal: low keys (most queries) first

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 31, h = lane >> 5;
  const int k0w = kt * kBK + wave * 32;
  const int key = k0w + r;
  const bool key_ok = key < rows;
  const size_t base = (size_t)bh * rows * D;
  const size_t sbase = (size_t)bh * rows;
  const uint32_t blk_bytes = (uint32_t)rows * T::kRowBytes;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(static_cast<const uint16_t *>(a.q) + base, blk_bytes);
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(static_cast<const uint16_t *>(a.dout) + base, blk_bytes);
  uint32_t coff[T::kLoadsPerWave];
  copy_offsets<D>(coff, wave, lane);

  // Query tiles first .. first+n-1; tile first+u lives in buffer u % 3.
  const int first = kDiag ? (kt * kBK) / kBT : 0;   // earlier queries see none of the keys
  const int n = (rows + kBT - 1) / kBT - first;
  auto qbuf = [&](int i) { return i == 0 ? lds_q0 : (i == 1 ? lds_q1 : lds_q2); };
  auto obuf = [&](int i) { return i == 0 ? lds_o0 : (i == 1 ? lds_o1 : lds_o2); };
  {
    const int last = first + n - 1;
    if (n <= 3 && last * kBT + kBT > rows)
      zero_tail<D>(qbuf((n - 1) % 3), obuf((n - 1) % 3), rows - last * kBT, tid);
  }
  // Thread tid < 64 stages -LSE*log2(e) of query tid of a tile, 64 <= tid < 128
  // its D.  The load is branch-free (clamped row) and its value is used only
  // by the store at the end of the iteration, so that waiting for it does not
  // also wait for the tile copies issued before it.
  const float *stage_src = (tid < kBT ? a.lse : a.delta) + sbase;
  auto stage_load = [&](int tile) { return stage_src[min(tile * kBT + (tid & 63), rows - 1)]; };
  auto stage_store = [&](int buf, int tile, float raw) {
    const bool ok = tile * kBT + (tid & 63) < rows;
    if (tid < kBT) lds_nl[buf][tid] = ok ? neg_lse2(raw) : -INFINITY;
    else if (tid < 2 * kBT) lds_dd[buf][tid - kBT] = ok ? raw : 0.f;
  };
  issue_copy<D>(lds_q0, rq, coff, first * kBT, wave);
  issue_copy<D>(lds_o0, ro, coff, first * kBT, wave);
  stage_store(0, first, stage_load(first));
  if (n > 1) {
    issue_copy<D>(lds_q1, rq, coff, (first + 1) * kBT, wave);
    issue_copy<D>(lds_o1, ro, coff, (first + 1) * kBT, wave);
    stage_store(1, first + 1, stage_load(first + 1));
  }

  // B operands: lane (r, h) holds k[key][16c + 8h ..] and v[key][16c + 8h ..].
  bf16x8 kf[kQK], vf[kQK];
  {
    const uint16_t *K = static_cast<const uint16_t *>(a.k) + base + (size_t)key * D;
    const uint16_t *V = static_cast<const uint16_t *>(a.v) + base + (size_t)key * D;
#pragma unroll
    for (int c = 0; c < kQK; ++c) {
      const uint4 z = make_uint4(0, 0, 0, 0);
      kf[c] = __builtin_bit_cast(bf16x8, key_ok ? *reinterpret_cast<const uint4 *>(K + c * 16 + h * 8) : z);
      vf[c] = __builtin_bit_cast(bf16x8, key_ok ? *reinterpret_cast<const uint4 *>(V + c * 16 + h * 8) : z);
    }
  }
  f32x16 dk[kDB], dv[kDB];
#pragma unroll
  for (int b = 0; b < kDB; ++b) {
    dk[b] = f32x16{};
    dv[b] = f32x16{};
  }
  const FragOffsets<D> fo = frag_offsets<D>(lane);
  const float sl2 = a.scale_log2;

  // Sub-tile (tile t, half sb) covers queries 64t + 32sb .. +31.
  auto skipped = [&](int t, int sb) { return kDiag && t * kBT + sb * 32 + 31 < k0w; };
  auto needs_mask = [&](int t, int sb) { return kDiag && t * kBT + sb * 32 < k0w + 31; };
  // S = Q K^T and dP = dO V^T of a sub-tile: entry i of lane (key, h) is query
  // 32sb + 16(i/8) + 8h + i%8 of the tile.
  auto sdp = [&](const char *qb, const char *ob, int sb, f32x16 &s, f32x16 &dp) {
    s = f32x16{};
    dp = f32x16{};
#pragma unroll
    for (int c = 0; c < kQK; ++c) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_nrm<D>(qb, fo, sb, c), kf[c], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_nrm<D>(ob, fo, sb, c), vf[c], dp, 0, 0, 0);
    }
  };
  // P and dS of a sub-tile as the B operands of the gradient products.
  // may_mask (compile-time): the sub-tile may cross the diagonal.
  auto softmax = [&](auto may_mask, const f32x16 &s, const f32x16 &dp, int buf, int t, int sb,
                     bf16x8 (&pb)[2], bf16x8 (&dsb)[2]) {
    const bool masked = decltype(may_mask)::value && needs_mask(t, sb);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int q0 = sb * 32 + hh * 16 + 8 * h;
      const float4 n0 = *(const lds_float4 *)&lds_nl[buf][q0];
      const float4 n1 = *(const lds_float4 *)&lds_nl[buf][q0 + 4];
      const float4 d0 = *(const lds_float4 *)&lds_dd[buf][q0];
      const float4 d1 = *(const lds_float4 *)&lds_dd[buf][q0 + 4];
      const float nl[8] = {n0.x, n0.y, n0.z, n0.w, n1.x, n1.y, n1.z, n1.w};
      const float dl[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = hh * 8 + e;
        float p = __builtin_amdgcn_exp2f(fmaf(s[i], sl2, nl[e]));
        if (masked) p = t * kBT + q0 + e < key ? 0.f : p;
        pb[hh][e] = (__bf16)p;
        dsb[hh][e] = (__bf16)(p * (dp[i] - dl[e]));
      }
    }
  };
  // dV^T += dO^T P and dK^T += Q^T dS over the sub-tile's 32 queries.
  auto grads = [&](const char *qb, const char *ob, int sb, const bf16x8 (&pb)[2], const bf16x8 (&dsb)[2]) {
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int b = 0; b < kDB; ++b) {
        dv[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_tr<D>(ob, fo, 2 * sb + half, b), pb[half],
                                                        dv[b], 0, 0, 0);
        dk[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_tr<D>(qb, fo, 2 * sb + half, b), dsb[half],
                                                        dk[b], 0, 0, 0);
      }
  };

  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  f32x16 s0, dp0;   // S, dP of sub-tile (current tile, 0)
  if (!skipped(first, 0)) sdp(lds_q0, lds_o0, 0, s0, dp0);

  // Iteration u: tile t = first + u in buffer bc, tile t+1 in b1, copies of
  // tile t+2 into b2.
  // `generic` (compile-time): the tile may hold the diagonal of the
  // workgroup's keys (masked and skipped sub-tiles); otherwise the pipelined
  // block.
  auto iteration = [&](auto generic, int u, int bc, int b1, int b2, const char *qc, const char *oc,
                       const char *q1, const char *o1, char *q2, char *o2) {
    constexpr bool kGeneric = decltype(generic)::value;
    const int t = first + u;
    float staged = 0.f;
    if (u + 2 < n) {
      issue_copy<D>(q2, rq, coff, (t + 2) * kBT, wave);
      issue_copy<D>(o2, ro, coff, (t + 2) * kBT, wave);
      staged = stage_load(t + 2);
    }
    f32x16 s1, dp1;
    bf16x8 pb[2], dsb[2];
    if constexpr (!kGeneric) {
      // First half: P, dS of (t, 0); S, dP of (t, 1); gradients of (t, 0).
      softmax(NoMask{}, s0, dp0, bc, t, 0, pb, dsb);
      sdp(qc, oc, 1, s1, dp1);
      grads(qc, oc, 0, pb, dsb);
      RA_DKDV_HALF_END();
      // Second half: P, dS of (t, 1); S, dP of (t+1, 0) (stale and unused
      // after the last tile); gradients of (t, 1).
      softmax(NoMask{}, s1, dp1, bc, t, 1, pb, dsb);
      sdp(q1, o1, 0, s0, dp0);
      grads(qc, oc, 1, pb, dsb);
      RA_DKDV_HALF_END();
    } else {
      if (!skipped(t, 0)) softmax(MayMask{}, s0, dp0, bc, t, 0, pb, dsb);
      if (!skipped(t, 1)) sdp(qc, oc, 1, s1, dp1);
      if (!skipped(t, 0)) grads(qc, oc, 0, pb, dsb);
      if (!skipped(t, 1)) softmax(MayMask{}, s1, dp1, bc, t, 1, pb, dsb);
      if (u + 1 < n && !skipped(t + 1, 0)) sdp(q1, o1, 0, s0, dp0);
      if (!skipped(t, 1)) grads(qc, oc, 1, pb, dsb);
    }
    if (u + 2 < n) stage_store(b2, t + 2, staged);
    __builtin_amdgcn_s_waitcnt(0);   // this wavefront's copies of tile t+2 landed
    __syncthreads();
  };

  using Pipe = std::integral_constant<bool, false>;
  using Generic = std::integral_constant<bool, true>;
  int u = 0;
  if constexpr (!kDiag) {
#pragma clang loop unroll(disable)
    for (; u + 2 < n; u += 3) {
      iteration(Pipe{}, u, 0, 1, 2, lds_q0, lds_o0, lds_q1, lds_o1, lds_q2, lds_o2);
      iteration(Pipe{}, u + 1, 1, 2, 0, lds_q1, lds_o1, lds_q2, lds_o2, lds_q0, lds_o0);
      iteration(Pipe{}, u + 2, 2, 0, 1, lds_q2, lds_o2, lds_q0, lds_o0, lds_q1, lds_o1);
    }
    if (u < n) iteration(Pipe{}, u, 0, 1, 2, lds_q0, lds_o0, lds_q1, lds_o1, lds_q2, lds_o2);
    if (u + 1 < n) iteration(Pipe{}, u + 1, 1, 2, 0, lds_q1, lds_o1, lds_q2, lds_o2, lds_q0, lds_o0);
  } else {
    // The first two query tiles hold the diagonal of the workgroup's keys;
    // every later query follows every key, so those tiles take the pipelined
    // block (tile first+u stays in buffer u % 3).
    iteration(Generic{}, 0, 0, 1, 2, lds_q0, lds_o0, lds_q1, lds_o1, lds_q2, lds_o2);
    if (n > 1) iteration(Generic{}, 1, 1, 2, 0, lds_q1, lds_o1, lds_q2, lds_o2, lds_q0, lds_o0);
    u = 2;
#pragma clang loop unroll(disable)
    for (; u + 2 < n; u += 3) {
      iteration(Pipe{}, u, 2, 0, 1, lds_q2, lds_o2, lds_q0, lds_o0, lds_q1, lds_o1);
      iteration(Pipe{}, u + 1, 0, 1, 2, lds_q0, lds_o0, lds_q1, lds_o1, lds_q2, lds_o2);
      iteration(Pipe{}, u + 2, 1, 2, 0, lds_q1, lds_o1, lds_q2, lds_o2, lds_q0, lds_o0);
    }
    if (u < n) iteration(Pipe{}, u, 2, 0, 1, lds_q2, lds_o2, lds_q0, lds_o0, lds_q1, lds_o1);
    if (u + 1 < n) iteration(Pipe{}, u + 1, 0, 1, 2, lds_q0, lds_o0, lds_q1, lds_o1, lds_q2, lds_o2);
  }

  if (key_ok) {
    add_row<D>(a.dk + base + (size_t)key * D, dk, h, a.scale);
    add_row<D>(a.dv + base + (size_t)key * D, dv, h, 1.f);
  }
#endif  // __HIP_DEVICE_COMPILE__
}

template <int D, bool kDiag>
hipError_t launch_d(const BwdArgs &a, hipStream_t s, const LaunchTiming &t) {
  constexpr int kB = 32 * kWaves;
  const int n_t = (a.rows + kB - 1) / kB;
  const dim3 grid((unsigned)((int64_t)a.bh * n_t)), block(64 * kWaves);
  const hipError_t e = launch_one((kDiag || a.rows % kBT != 0) ? bwd_dq_bf16_kernel<D, kDiag, true>
                                                               : bwd_dq_bf16_kernel<D, kDiag, false>,
                                  grid, block, s, t.start, nullptr, a);
  if (e != hipSuccess) return e;
  return launch_one(bwd_dkdv_bf16_kernel<D, kDiag>, grid, block, s, nullptr, t.stop, a);
}

}  // namespace

hipError_t launch_bwd_step_bf16(const BwdArgs &a, int d, StepCase c, hipStream_t s,
                                const LaunchTiming &t) {
  const bool diag = c == StepCase::Diag;
  if (d == 128) return diag ? launch_d<128, true>(a, s, t) : launch_d<128, false>(a, s, t);
  if (d == 64) return diag ? launch_d<64, true>(a, s, t) : launch_d<64, false>(a, s, t);
  return hipErrorInvalidValue;
}

}  // namespace ra
