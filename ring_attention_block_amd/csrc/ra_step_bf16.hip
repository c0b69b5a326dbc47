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

#include <algorithm>
#include <type_traits>

#include "ra_kernels.h"

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
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
  static constexpr size_t kLdsBytes = 4 * kBytes;          // K and V, double buffered
};

// Key held by LDS row rho of the K tile: bits 2 and 3 swapped within 32.
__device__ __forceinline__ int k_row_key(int rho) {
  return (rho & ~12) | ((rho & 4) << 1) | ((rho & 8) >> 1);
}
// 16-byte chunk swizzles of the K and V tiles.  The fragment reads are
// conflict-free whether the LDS serves a 16-byte read in passes of 8 lanes
// over 32 banks or of 16 lanes over 64 banks (and an 8-byte read in passes of
// 16 or 32 lanes): K reads take 8/16 consecutive rows at one logical chunk;
// a transposed V read takes 4 consecutive rows at 32/64 contiguous bytes.
template <int D>
__device__ __forceinline__ int k_swz(int rho) {
  if constexpr (D == 128) return rho & 15;
  else return (rho & 7) ^ ((rho >> 3) & 1);
}
template <int D>
__device__ __forceinline__ int v_swz(int rho) {
  const int x = rho & 3;
  if constexpr (D == 128) return 4 * x + 2 * ((x ^ (x >> 1)) & 1);   // 0, 6, 10, 12
  else return 2 * x;
}

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
    so.k[i] = (uint32_t)(k_row_key(rho) * T::kRowBytes + ((chi ^ k_swz<D>(rho)) * 16));
    so.v[i] = (uint32_t)(rho * T::kRowBytes + ((chi ^ v_swz<D>(rho)) * 16));
  }
  return so;
}

// Issue this wavefront's share of the HBM -> LDS copies of one K (or V) tile
// starting at key k0 into `buf`.  The tile offset goes into the per-lane
// offset, which the buffer range check covers (the scalar offset is not range
// checked).
template <int D, int kW>
__device__ __forceinline__ void issue_copy(char *buf, __amdgpu_buffer_rsrc_t rsrc,
                                           const uint32_t (&off)[Stage<D, kW>::kPerWave], int k0,
                                           int wave) {
  using T = Tile<D>;
  const uint32_t toff = (uint32_t)k0 * T::kRowBytes;
#pragma unroll
  for (int i = 0; i < Stage<D, kW>::kPerWave; ++i) {
    const int n = wave + i * kW;
    if (Stage<D, kW>::kPerWave * kW == T::kLoads || n < T::kLoads)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void *)(buf + n * 1024), 16, off[i] + toff, 0,
                                               0, 0);
  }
}

// Zero the LDS rows of a K and a V tile buffer whose keys lie at or past
// `n_valid` (only for the last tile of a block whose length is not a multiple
// of 64).  These rows are disjoint from the rows the copies write.
template <int D, int kW>
__device__ __forceinline__ void zero_tail(char *kbuf, char *vbuf, int n_valid, int tid) {
  using T = Tile<D>;
  for (int e = tid; e < kBN * T::kChunks; e += 64 * kW) {
    const int rho = e / T::kChunks, chi = e % T::kChunks;
    const uint4 z = make_uint4(0, 0, 0, 0);
    if (k_row_key(rho) >= n_valid) *reinterpret_cast<uint4 *>(kbuf + rho * T::kRowBytes + chi * 16) = z;
    if (rho >= n_valid) *reinterpret_cast<uint4 *>(vbuf + rho * T::kRowBytes + chi * 16) = z;
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

// Row maximum of a score tile and the lazy-rescale decision.  `valid` false
// leaves the state untouched (a tile past the block end).  Updates the
// reference and true maxima, scales the partial row sum, and returns the
// factor the O accumulator must be scaled by; `rescale` is set when any lane
// of the wavefront needs it.
__device__ __forceinline__ float tile_max_update(const f32x16 (&s)[2], RowState &rs, float sl2,
                                                 bool valid, bool &rescale) {
  float m0 = fmaxf(s[0][0], s[0][1]), m1 = fmaxf(s[1][0], s[1][1]);   // two chains
#pragma unroll
  for (int i = 2; i < 16; ++i) {
    m0 = fmaxf(m0, s[0][i]);
    m1 = fmaxf(m1, s[1][i]);
  }
  const float mt = half_swap_max(fmaxf(m0, m1)) * sl2;
  rs.m_run = valid ? fmaxf(rs.m_run, mt) : rs.m_run;
  const bool need = valid && mt > rs.m_ref + kTau;
  const float m_new = need ? mt : rs.m_ref;
  const float alpha = need ? __builtin_amdgcn_exp2f(rs.m_ref - m_new) : 1.f;
  rescale = __any(need);
  rs.m_ref = m_new;
  rs.l *= alpha;
  return alpha;
}

// P = exp2(s * scale*log2(e) - m_ref) as four bf16 B-operand fragments, and
// the partial row sum of those bf16 values (the same weights the P V product
// uses), accumulated in fp32 two at a time by v_dot2c_f32_bf16 in two chains.
__device__ __forceinline__ void tile_exp(const f32x16 (&s)[2], RowState &rs, bf16x8 (&pb)[4],
                                         float sl2) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const float neg_m = (rs.m_ref == -INFINITY) ? 0.f : -rs.m_ref;
#pragma unroll
  for (int sb = 0; sb < 2; ++sb)
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        pb[sb * 2 + half][j] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[sb][half * 8 + j], sl2, neg_m));
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  float acc[2] = {0.f, 0.f};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    acc[0] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[c], pb[c], 0, 1), ones, acc[0], false);
    acc[1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[c], pb[c], 2, 3), ones, acc[1], false);
    acc[0] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[c], pb[c], 4, 5), ones, acc[0], false);
    acc[1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[c], pb[c], 6, 7), ones, acc[1], false);
  }
  rs.l += acc[0] + acc[1];
}

// kMask: some tile may need the element mask (diagonal block, or a block
// length that is not a multiple of 64).  kIdle: the query rows are not a
// multiple of the workgroup's, so some wavefronts may have no rows.  kCopy:
// the launch carries copies (StepCopies); without them the copy code compiles
// away and the kernel keeps its registers for the fold.
template <int D, bool kDiag, int kW, bool kMask, bool kIdle, bool kCopy>
__global__ void __launch_bounds__(64 * kW, 8 / kW) step_bf16_kernel(StepArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)
  using T = Tile<D>;
  constexpr int kBM = 32 * kW;  // query rows per workgroup
  constexpr int kQK = D / 16;   // k-chunks of the score product
  constexpr int kDB = D / 32;   // 32-row blocks of O^T
  // Four separate LDS objects (K and V, double buffered).  Being distinct
  // objects lets the compiler see that the HBM->LDS copies into one buffer do
  // not alias the reads of the other, so it does not make every LDS read wait
  // for the copies still in flight.
  __shared__ __attribute__((aligned(1024))) char lds_k0[T::kBytes];
  __shared__ __attribute__((aligned(1024))) char lds_k1[T::kBytes];
  __shared__ __attribute__((aligned(1024))) char lds_v0[T::kBytes];
  __shared__ __attribute__((aligned(1024))) char lds_v1[T::kBytes];

  const int rows = a.rows;         // query rows
  const int kv_rows = a.kv_rows;   // key/value rows (equal to rows on the diagonal)
  const int n_qt = (rows + kBM - 1) / kBM;
  // Workgroup -> (head, query tile).  Consecutive workgroup ids go to
  // different XCDs; when the head count allows, give each XCD a contiguous
  // range of heads so that one head's key/value tiles stay in one L2.  Within
  // an XCD, workgroups start in id order: full blocks walk one head's tiles
  // after another; diagonal blocks, whose tiles carry unequal work, walk the
  // tiles of all the XCD's heads from the heaviest down (largest work first,
  // so the light tiles fill in at the end).
  int bh, qi;
  {
    const int bid = blockIdx.x;
    if ((a.bh & 7) == 0) {
      const int heads8 = a.bh >> 3, k = bid >> 3, x = bid & 7;
      if (kDiag) {
        bh = x * heads8 + k % heads8;
        qi = k / heads8;
      } else {
        const int logical = x * heads8 * n_qt + k;
        bh = logical / n_qt;
        qi = logical % n_qt;
      }
    } else if (kDiag) {
      bh = bid % a.bh;
      qi = bid / a.bh;
    } else {
      bh = bid / n_qt;
      qi = bid % n_qt;
    }
  }
  // Diagonal blocks: qi 0 is the heaviest query tile (the last one).
  const int qt = kDiag ? n_qt - 1 - qi : qi;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int r = lane & 31, h = lane >> 5;
  const int q0w = qt * kBM + wave * 32;
  const int row = q0w + r;
  const bool row_ok = row < rows;

  const size_t srow0 = (size_t)bh * a.row_stride;   // first state row of this (batch, head)
  const size_t base = srow0 * D;
  const size_t kv_base = (size_t)bh * a.kv_stride * D;
  const int q_bh = bh < a.q_bh ? bh : bh % a.q_bh;   // a query block shared along the batch
  const uint16_t *__restrict__ Q = static_cast<const uint16_t *>(a.q) + (size_t)q_bh * a.row_stride * D;
  float *__restrict__ O = a.o + base;
  // The query rows and the state are read through buffer resources whose
  // range check returns 0 past the block end and, for the state, for every row
  // of a fresh step.  The loads then need no branch (a load under a branch is
  // waited for inside it, which serialised them).
  const bool fresh = (a.flags & kStepFresh) != 0;
  const uint32_t state_rows = fresh ? 0u : (uint32_t)rows;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q, (uint32_t)rows * T::kRowBytes);
  const __amdgpu_buffer_rsrc_t rso = make_rsrc(O, state_rows * (uint32_t)(D * 4));
  const __amdgpu_buffer_rsrc_t rsm = make_rsrc(a.m + srow0, state_rows * 4u);
  const __amdgpu_buffer_rsrc_t rsl = make_rsrc(a.l + srow0, state_rows * 4u);
  const uint32_t blk_bytes = (uint32_t)kv_rows * T::kRowBytes;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(static_cast<const uint16_t *>(a.k) + kv_base, blk_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(static_cast<const uint16_t *>(a.v) + kv_base, blk_bytes);
  const Stage<D, kW> so = stage_offsets<D, kW>(wave, lane);

  const int kv_end = kDiag ? min(kv_rows, qt * kBM + kBM) : kv_rows;
  const int n_tiles = (kv_end + kBN - 1) / kBN;
  // Tile n uses K and V buffer n % 2.

  // Carried copies (StepCopies): this workgroup's units are [u0, u0 + n_tiles)
  // in (batch-head, query tile) order; on the diagonal, query tile t holds
  // (t + 1) kBM / kBN key tiles (all but the last tile of the block are whole).
  // Each copy's slice is addressed through buffer resources based at its start
  // and bounded to its length, so lanes past its end load zeros and their
  // stores are dropped; both copies advance together, one 16-byte chunk per
  // thread and copy per tick.  A tick (one at the end of each key tile's
  // iteration) stores the chunks the previous tick loaded and loads the next
  // ones.  The state is uniform and set up once, so no kernel argument stays
  // live.  (Non-temporal accesses measured no better: 0.452 against 0.425 ms
  // for a 16-step ring of 8 heads x 2048 rows.)
  const uint32_t u0 = kDiag ? (uint32_t)bh * (uint32_t)((kBM / kBN) * (n_qt - 1) * n_qt / 2 +
                                                         (min(kv_rows, n_qt * kBM) + kBN - 1) / kBN) +
                                  (uint32_t)((kBM / kBN) * qt * (qt + 1) / 2)
                            : ((uint32_t)bh * (uint32_t)n_qt + (uint32_t)qt) * (uint32_t)n_tiles;
  constexpr int kCopyPolicy = 0;   // buffer access cache policy: default
  __amdgpu_buffer_rsrc_t cp_s0 = make_rsrc(nullptr, 0), cp_d0 = cp_s0, cp_s1 = cp_s0, cp_d1 = cp_s0;
  // cp_off starts past every slice (slices are below 2^31 bytes), so the first
  // tick's stores are out of range.
  uint32_t cp_ticks = 0, cp_t = 0, cp_off = 0x80000000u;
  u32x4 cp_v0 = {0u, 0u, 0u, 0u}, cp_v1 = cp_v0;
  if constexpr (kCopy) {
    uint32_t len_max = 0;
    auto slice = [&](uint64_t c, uint64_t pu, const void *src, void *dst, __amdgpu_buffer_rsrc_t &rs,
                     __amdgpu_buffer_rsrc_t &rd) {
      const uint64_t lo = min((uint64_t)u0 * pu, c), hi = min((uint64_t)(u0 + n_tiles) * pu, c);
      const uint32_t len = (uint32_t)(hi - lo);
      rs = make_rsrc(static_cast<const char *>(src) + lo * 16, len * 16u);
      rd = make_rsrc(static_cast<char *>(dst) + lo * 16, len * 16u);
      len_max = max(len_max, len);
    };
    slice(a.cp.chunks[0], a.cp.per_unit[0], a.cp.src[0], a.cp.dst[0], cp_s0, cp_d0);
    if (a.cp.n > 1) slice(a.cp.chunks[1], a.cp.per_unit[1], a.cp.src[1], a.cp.dst[1], cp_s1, cp_d1);
    cp_ticks = (len_max + 64u * kW - 1) / (64u * kW);
  }
  // The end of an iteration: the copy tick, then the wait for this
  // wavefront's tile copies (and its LDS accesses) before the barrier.  While
  // the slices last (one uniform test), the tick stores both slots' previous
  // chunks and loads both next ones without further branches: accesses that
  // fall outside a slice (before the first load, past the last chunk, a second
  // copy that does not exist) are out of range, so they load zeros and store
  // nothing.  Its four accesses are the last vector memory accesses issued,
  // and those complete in issue order, so vmcnt(4) leaves exactly them in
  // flight: no tile waits for a copy's memory latency.  Once the slices are
  // done the iteration ends as without copies (issuing the out-of-range
  // accesses in every iteration cost 2% of the step).
  auto close = [&]() {
    if constexpr (kCopy) {
      if (cp_t <= cp_ticks) {
        __builtin_amdgcn_raw_buffer_store_b128(cp_v0, cp_d0, cp_off, 0, kCopyPolicy);
        __builtin_amdgcn_raw_buffer_store_b128(cp_v1, cp_d1, cp_off, 0, kCopyPolicy);
        cp_off = (cp_t * 64u * kW + (uint32_t)tid) * 16u;
        cp_v0 = __builtin_amdgcn_raw_buffer_load_b128(cp_s0, cp_off, 0, kCopyPolicy);
        cp_v1 = __builtin_amdgcn_raw_buffer_load_b128(cp_s1, cp_off, 0, kCopyPolicy);
        ++cp_t;
        __builtin_amdgcn_s_waitcnt(4 | (7 << 4));   // vmcnt(4) lgkmcnt(0)
        return;
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
  };

  // A ragged last tile that is the first use of its LDS buffers must not see
  // uninitialised LDS past the block end: zero those rows.  A later use of a
  // buffer holds finite keys/values of an earlier full tile there, which the
  // mask (keys) and the zero probabilities (values) already neutralise.
  const int last = n_tiles - 1;
  if (last <= 1 && last * kBN + kBN > kv_rows)
    zero_tail<D, kW>((last & 1) ? lds_k1 : lds_k0, (last & 1) ? lds_v1 : lds_v0, kv_rows - last * kBN,
                     tid);
  issue_copy<D, kW>(lds_k0, rk, so.k, 0, wave);
  issue_copy<D, kW>(lds_v0, rv, so.v, 0, wave);
  if (n_tiles > 1) issue_copy<D, kW>(lds_k1, rk, so.k, kBN, wave);

  // Q^T fragments: lane (r, h) holds q[row][16c + 8h .. 16c + 8h + 7].
  bf16x8 qf[kQK];
  // O^T accumulators: block b, entry i <-> column 32b + 8(i/4) + 4h + i%4.
  f32x16 oacc[kDB];
  RowState rs;
#pragma unroll
  for (int c = 0; c < kQK; ++c) {
    const uint32_t off = (uint32_t)row * T::kRowBytes + (uint32_t)(c * 16 + h * 8) * 2;
    qf[c] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
  }
  // m and l are used only after the first barrier (below).
  const float m_ld = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsm, (uint32_t)row * 4, 0, 0));
  const float l_ld = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsl, (uint32_t)row * 4, 0, 0));

  // Per-lane LDS byte offsets of the fragments within a tile buffer.
  //   K fragment (sb, c): row 32sb + r, chunk (2c + h) swizzled by the row.
  //   V^T fragment (b, c), transposed read rr: row 16c + 4rr + 8(g/2) + j/4,
  //   column 32b + 16(g%2) + 4(j%4), with g = lane/16 and j = lane%16.
  uint32_t koff[kQK];
#pragma unroll
  for (int c = 0; c < kQK; ++c)
    koff[c] = (uint32_t)(r * T::kRowBytes + (((2 * c + h) ^ k_swz<D>(r)) * 16));
  uint32_t voff[kDB];
  {
    const int g = lane >> 4, j = lane & 15;
    const int vrow = 8 * (g >> 1) + (j >> 2);
#pragma unroll
    for (int b = 0; b < kDB; ++b) {
      const int chunk = 4 * b + 2 * (g & 1) + ((j & 3) >> 1);
      voff[b] = (uint32_t)(vrow * T::kRowBytes + ((chunk ^ v_swz<D>(vrow)) * 16) + 8 * (j & 1));
    }
  }

  const float sl2 = a.scale_log2;
  const int lim = kDiag ? min(row, kv_rows - 1) : kv_rows - 1;   // last key this row may see

  // S^T = K Q^T for the tile in K buffer `kb`.
  auto scores = [&](f32x16 (&s)[2], const char *kb) {
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      s[sb] = f32x16{};
#pragma unroll
      for (int c = 0; c < kQK; ++c) {
        const bf16x8 kf = *(const lds_bf16x8 *)(kb + sb * 32 * T::kRowBytes + koff[c]);
        s[sb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[c], s[sb], 0, 0, 0);
      }
    }
  };
  // V^T fragment (b, c) of the tile in V buffer `vb`: two transposed reads.
  auto read_v = [&](const char *vb, int c, int b) {
    const char *p0 = vb + (16 * c) * T::kRowBytes + voff[b];
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p0);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p0 + 4 * T::kRowBytes));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // O^T += V^T P^T for the tile in V buffer `vb`.  Key chunk outermost: the
  // kDB accumulators of one chunk are independent, and the V reads of the
  // next chunk overlap this chunk's MFMAs.
  auto accumulate = [&](const bf16x8 (&pb)[4], const char *vb) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int b = 0; b < kDB; ++b)
        oacc[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_v(vb, c, b), pb[c], oacc[b], 0, 0, 0);
  };
  // Tile t: nothing for this wavefront (diagonal only: every key after every
  // row of the wavefront) / needs the element mask.
  auto skip_tile = [&](int t) { return kDiag && t * kBN > q0w + 31; };
  auto mask_needed = [&](int t) {
    return (kDiag && t * kBN + kBN - 1 > q0w) || (t * kBN + kBN > kv_rows);
  };

  // The previous O state.  The state update is linear in it: the new O is
  // exp2(m_state - m_ref) O_state + (the P V products relative to m_ref).
  // Launches with the element mask load it into the accumulators up front:
  // the loads are issued last before the first barrier, which waits only for
  // the copies and the loads issued before them (vmcnt counts in issue
  // order), and are first waited for at the P V product of tile 0 (the
  // scheduling barrier keeps every earlier load ahead of them).  Unmasked
  // launches start from zero and add the state after the last tile, whose
  // iteration issues its loads (last_tile below): no tile waits for them.
  __builtin_amdgcn_sched_barrier(0);
  auto load_state_o = [&](f32x4 (&ol)[kDB * 4]) {
#pragma unroll
    for (int b = 0; b < kDB; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t off = ((uint32_t)row * D + (uint32_t)(b * 32 + g * 8 + h * 4)) * 4;
        // (Cast the whole vector: a scalar bit cast of one element of the
        // loaded vector was compiled as a cast of element 0.)
        ol[b * 4 + g] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rso, off, 0, 0));
      }
  };
  if constexpr (kMask) {
    f32x4 ol[kDB * 4];
    load_state_o(ol);
#pragma unroll
    for (int b = 0; b < kDB; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) oacc[b][4 * g + e] = ol[b * 4 + g][e];
    constexpr int kOLoads = kDB * 4;
    __builtin_amdgcn_s_waitcnt((kOLoads & 15) | ((kOLoads >> 4) << 14) | (7 << 4));  // vmcnt(kOLoads) lgkmcnt(0)
  } else {
#pragma unroll
    for (int b = 0; b < kDB; ++b) oacc[b] = f32x16{};
    __builtin_amdgcn_s_waitcnt(0);
  }
  __syncthreads();   // K(0), V(0), K(1) (and a zeroed tail) visible to all
  const bool read_state = row_ok && !fresh;
  const float m_state = read_state ? m_ld * kLog2e : -INFINITY;   // base 2
  rs.m_ref = m_state;
  rs.m_run = m_state;
  rs.l = (read_state && h == 0) ? l_ld : 0.f;
  // Software pipeline, one tile ahead.  Iteration t issues the copies of
  // K(t+2) and V(t+1), and in one branch-free block computes the scores of
  // tile t+1, the exponentials of tile t, the P V product of tile t and the
  // row maximum of tile t+1; the rare rescale of O for tile t+1 follows.
  // K(t+2) reuses the buffer of K(t), read one iteration earlier; V(t+1)
  // reuses that of V(t-1).
  // kIdle: some wavefront's rows may all lie past the block end (a short
  // query block, as in decoding); such a wavefront only issues its share of
  // the copies and takes the barriers.  Without kIdle the test compiles away
  // (the kernel without it is scheduled better).
  const bool wave_active = !kIdle || q0w < rows;
  f32x16 s_cur[2];
  if (wave_active) {
    scores(s_cur, lds_k0);   // tile 0 is never skipped
    if (kMask && mask_needed(0)) mask_tile(s_cur, h * 8, lim);
    bool rescale;
    const float alpha = tile_max_update(s_cur, rs, sl2, true, rescale);
    if (rescale) {
#pragma unroll
      for (int b = 0; b < kDB; ++b) oacc[b] *= alpha;
    }
  }
  __syncthreads();   // every wavefront is done with K buffer 0

  // Iteration t.  The buffers are passed explicitly (unrolled by two below)
  // so that every LDS access names one static buffer:
  //   copies: K(t+2) -> k_dst (= K buffer t%2), V(t+1) -> v_dst (V buffer (t+1)%2)
  //   reads:  K(t+1) <- k_src (K buffer (t+1)%2), V(t) <- v_src (V buffer t%2)
  // `fast` (a compile-time flag): tiles t and t+1 need no mask, so the
  // iteration is the interleaved block; otherwise the general masked one.
  auto iteration = [&](auto fast, int t, char *k_dst, char *v_dst, const char *k_src,
                       const char *v_src) {
    constexpr bool kFast = decltype(fast)::value;
    if (t + 2 < n_tiles) issue_copy<D, kW>(k_dst, rk, so.k, (t + 2) * kBN, wave);
    if (t + 1 < n_tiles) issue_copy<D, kW>(v_dst, rv, so.v, (t + 1) * kBN, wave);
    const bool has_next = t + 1 < n_tiles;

    if (wave_active) {
      f32x16 s_nxt[2];
      bf16x8 pb[4];
      bool rescale = false;
      float alpha = 1.f;
      if constexpr (kFast) {
        // The scores of the tile after the last one read a stale K buffer;
        // has_next = false keeps them out of the state.
        scores(s_nxt, k_src);
        tile_exp(s_cur, rs, pb, sl2);
        accumulate(pb, v_src);
        alpha = tile_max_update(s_nxt, rs, sl2, has_next, rescale);
        // Interleave: per score MFMA one LDS read and four vector instructions
        // (exponentials of tile t), then per P V MFMA two LDS reads and up to
        // four vector instructions (the rest of the exponentials, then the row
        // maximum of tile t+1).  The slots cover every vector instruction of
        // the block, so none is left for a serial tail after the last MFMA.
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int i = 0; i < 2 * kQK; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x402, 4, 0);
        }
#pragma unroll
        for (int i = 0; i < 4 * kDB; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x402, 4, 0);
        }
      } else {
        const bool run_next = has_next && !skip_tile(t + 1);
        if (run_next) scores(s_nxt, k_src);
        if (!skip_tile(t)) {
          tile_exp(s_cur, rs, pb, sl2);
          accumulate(pb, v_src);
        }
        if (run_next) {
          if (mask_needed(t + 1)) mask_tile(s_nxt, (t + 1) * kBN + h * 8, lim);
          alpha = tile_max_update(s_nxt, rs, sl2, true, rescale);
        }
      }
      if (rescale) {
#pragma unroll
        for (int b = 0; b < kDB; ++b) oacc[b] *= alpha;
      }
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) s_cur[sb] = s_nxt[sb];
    }
    close();   // this wavefront's copies of K(t+2), V(t+1) landed
    __syncthreads();
  };

  // The last tile of an unmasked launch: no next tile to score and no copies.
  // The O-state loads go out once the tile's exponentials have freed the
  // score registers, ahead of its P V product; the state is added after it.
  auto last_tile = [&](const char *v_src) {
    bf16x8 pb[4];
    if (wave_active) tile_exp(s_cur, rs, pb, sl2);
    __builtin_amdgcn_sched_barrier(0);
    f32x4 ol[kDB * 4];
    load_state_o(ol);
    __builtin_amdgcn_sched_barrier(0);
    if (wave_active) accumulate(pb, v_src);
    // m_ref only grows from m_state, so the factor is at most 1 (0 for an
    // empty state, whose loads read zeros).
    const float a_old = m_state == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_state - rs.m_ref);
#pragma unroll
    for (int b = 0; b < kDB; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) oacc[b][4 * g + e] = fmaf(a_old, ol[b * 4 + g][e], oacc[b][4 * g + e]);
  };

  using Fast = std::integral_constant<bool, true>;
  using Masked = std::integral_constant<bool, false>;
  int t = 0;
  if constexpr (!kMask) {
    // Tiles 0 .. n_tiles-2 take the interleaved block (tile t uses K and V
    // buffers t % 2), the last one last_tile (n_tiles >= 1: empty blocks
    // launch nothing).
#pragma clang loop unroll(disable)
    for (; t + 2 < n_tiles; t += 2) {
      iteration(Fast{}, t, lds_k0, lds_v1, lds_k1, lds_v0);
      iteration(Fast{}, t + 1, lds_k1, lds_v0, lds_k0, lds_v1);
    }
    if (t + 1 < n_tiles) {
      iteration(Fast{}, t, lds_k0, lds_v1, lds_k1, lds_v0);
      ++t;
    }
    // One call site (two inlined copies raised the register count); no copy
    // is in flight, so the selected buffer cannot alias one being written.
    last_tile((t & 1) ? lds_v1 : lds_v0);
  } else {
    // head_dim 64, and 8-wavefront workgroups: the tiles before the first one
    // that needs the element mask (on the diagonal: keys before every row of
    // the wavefront) run the interleaved block as long as the following tile
    // needs no mask either; the rest the masked one.  Every wavefront runs n_tiles iterations with
    // one barrier each, whichever block it takes.  (At head_dim 128 with four
    // wavefronts per workgroup the two blocks in one kernel leave too few
    // registers, and the masked block alone is faster; with eight they fit.)
    if constexpr (D == 64 || kW == 8) {
      const int first_diag = kDiag ? (q0w >= kBN - 1 ? (q0w - (kBN - 1)) / kBN + 1 : 0) : n_tiles;
      const int first_tail = kv_rows >= kBN ? (kv_rows - kBN) / kBN + 1 : 0;
      const int n_fast = max(0, min(min(first_diag, first_tail) - 1, n_tiles - 1));
#pragma clang loop unroll(disable)
      for (; t + 1 < n_fast; t += 2) {
        iteration(Fast{}, t, lds_k0, lds_v1, lds_k1, lds_v0);
        iteration(Fast{}, t + 1, lds_k1, lds_v0, lds_k0, lds_v1);
      }
      if (t < n_fast) {
        iteration(Fast{}, t, lds_k0, lds_v1, lds_k1, lds_v0);
        ++t;
        if (t < n_tiles) iteration(Masked{}, t, lds_k1, lds_v0, lds_k0, lds_v1);
        ++t;
      }
    }
#pragma clang loop unroll(disable)
    for (; t + 1 < n_tiles; t += 2) {
      iteration(Masked{}, t, lds_k0, lds_v1, lds_k1, lds_v0);
      iteration(Masked{}, t + 1, lds_k1, lds_v0, lds_k0, lds_v1);
    }
    if (t < n_tiles) iteration(Masked{}, t, lds_k0, lds_v1, lds_k1, lds_v0);
  }

  // ---- back to the canonical state (m = true running maximum) --------------
  const float l_tot = half_swap_sum(rs.l);
  const float beta = (rs.m_run == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(rs.m_ref - rs.m_run);
  if (row_ok && !(a.flags & kStepFinalize)) {
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
      const size_t sr = srow0 + row;
      a.m[sr] = rs.m_run * kLn2;
      a.l[sr] = l_tot * beta;
    }
  } else if (row_ok) {
    // Finalize in place of the store: out = O / l and LSE = m + ln l of the
    // state the branch above would store (l == 0 gives 0 and -inf).
    const float lr = l_tot * beta;
    const size_t oe = base + (size_t)row * D;
    if (a.o_out) {
#pragma unroll
      for (int b = 0; b < kDB; ++b)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = lr > 0.f ? (oacc[b][4 * g + e] * beta) / lr : 0.f;
          const size_t at = oe + b * 32 + g * 8 + h * 4;
          if (a.out_bf16) {
            typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
            const bf16x4 pk = {(__bf16)y[0], (__bf16)y[1], (__bf16)y[2], (__bf16)y[3]};
            *reinterpret_cast<bf16x4 *>(static_cast<uint16_t *>(a.o_out) + at) = pk;
          } else {
            *reinterpret_cast<float4 *>(static_cast<float *>(a.o_out) + at) =
                make_float4(y[0], y[1], y[2], y[3]);
          }
        }
    }
    if (h == 0 && a.lse_out) {
      // m is rounded to fp32 before the add, as the stored state is.
#pragma clang fp contract(off)
      const float m_nat = rs.m_run * kLn2;
      a.lse_out[srow0 + row] = lr > 0.f ? m_nat + logf(lr) : -INFINITY;
    }
  }
  // The rest of this workgroup's slices of the carried copies (a workgroup
  // with fewer key tiles than its slices need iterations).
  if constexpr (kCopy) {
    while (cp_t <= cp_ticks) close();
    __builtin_amdgcn_raw_buffer_store_b128(cp_v0, cp_d0, cp_off, 0, kCopyPolicy);
    __builtin_amdgcn_raw_buffer_store_b128(cp_v1, cp_d1, cp_off, 0, kCopyPolicy);
  }
#endif  // __HIP_DEVICE_COMPILE__
}

template <int D, bool kDiag, int kW>
hipError_t launch(StepArgs a, hipStream_t s, const LaunchTiming &t) {
  constexpr int kBM = 32 * kW;
  const int n_qt = (a.rows + kBM - 1) / kBM;
  const dim3 grid((unsigned)((int64_t)a.bh * n_qt)), block(64 * kW);
  if (a.cp.n > 0) {
    // Units of the launch (key tiles summed over its workgroups), counted as
    // the kernel counts each workgroup's (u0 and n_tiles there).
    const int64_t per = kBM / kBN;
    const int64_t units =
        kDiag ? (int64_t)a.bh * (per * (n_qt - 1) * n_qt / 2 +
                                 (std::min<int64_t>(a.kv_rows, (int64_t)n_qt * kBM) + kBN - 1) / kBN)
              : (int64_t)a.bh * n_qt * ((a.kv_rows + kBN - 1) / kBN);
    for (int k = 0; k < a.cp.n; ++k)
      a.cp.per_unit[k] = (uint32_t)(((int64_t)a.cp.chunks[k] + units - 1) / units);
  }
  auto go = [&](void (*plain)(StepArgs), void (*copying)(StepArgs)) {
    return launch_one(a.cp.n > 0 ? copying : plain, grid, block, s, t.start, t.stop, a);
  };
  if constexpr (kDiag)
    return go(step_bf16_kernel<D, true, kW, true, false, false>, step_bf16_kernel<D, true, kW, true, false, true>);
  const bool mask = a.kv_rows % kBN != 0, idle = a.rows % kBM != 0;
  if (mask) {
    return idle ? go(step_bf16_kernel<D, false, kW, true, true, false>, step_bf16_kernel<D, false, kW, true, true, true>)
                : go(step_bf16_kernel<D, false, kW, true, false, false>,
                     step_bf16_kernel<D, false, kW, true, false, true>);
  }
  return idle ? go(step_bf16_kernel<D, false, kW, false, true, false>, step_bf16_kernel<D, false, kW, false, true, true>)
              : go(step_bf16_kernel<D, false, kW, false, false, false>,
                   step_bf16_kernel<D, false, kW, false, false, true>);
}

// Full blocks: 8-wavefront workgroups (256 query rows share each key/value
// tile), unless that gives fewer workgroups than the chip has compute units
// (256 on MI355X); then 4-wavefront workgroups, twice as many (measured at 8
// heads x 2048 rows: 35 us against 50 us; at 32 heads x 4096 rows the
// 8-wavefront grid is faster).  Diagonal blocks at head_dim 128: 8-wavefront
// workgroups, which have the registers to run their tiles before the diagonal
// through the interleaved block (32 heads x 4096 rows: 137 us against 153 us
// with 4-wavefront workgroups, which must take the masked block throughout),
// unless that grid leaves compute units idle as above (8 heads x 2048 rows:
// 43 us with 4-wavefront workgroups against 49 us); at head_dim 64:
// 4-wavefront workgroups, whose finer query tiles waste less work on the
// masked triangle.  Query blocks of at most 64 rows (decoding: one wavefront
// has rows, the others only share the tile copies) take 4-wavefront workgroups
// whatever the grid (16 new rows against 8 x 4096 keys x 32 heads: the fold
// 96.7 us against 98.7 us with 8 wavefronts).
constexpr int64_t kComputeUnits = 256;

template <int D, bool kDiag>
hipError_t launch_d(const StepArgs &a, hipStream_t s, const LaunchTiming &t) {
  if constexpr (kDiag) {
    if (D == 64 || (int64_t)a.bh * ((a.rows + 255) / 256) < kComputeUnits) return launch<D, kDiag, 4>(a, s, t);
    return launch<D, kDiag, 8>(a, s, t);
  } else {
    if ((int64_t)a.bh * ((a.rows + 255) / 256) < kComputeUnits || a.rows <= 64) return launch<D, kDiag, 4>(a, s, t);
    return launch<D, kDiag, 8>(a, s, t);
  }
}

}  // namespace

hipError_t launch_step_bf16(const StepArgs &a, int d, StepCase c, hipStream_t s,
                            const LaunchTiming &t) {
  const bool diag = c == StepCase::Diag;
  if (d == 128) return diag ? launch_d<128, true>(a, s, t) : launch_d<128, false>(a, s, t);
  return diag ? launch_d<64, true>(a, s, t) : launch_d<64, false>(a, s, t);
}

}  // namespace ra
