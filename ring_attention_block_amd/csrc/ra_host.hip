// C ABI of the ring-step library: argument checks, causal case selection and
// kernel dispatch.  Nothing here allocates or synchronises; every check runs
// before anything is enqueued, so a rejected call leaves the state untouched.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <hip/hip_runtime.h>

#include "../../include/ra.h"
#include "ra_kernels.h"

namespace {

thread_local char g_err[512];

ra_status fail(ra_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

ra_status ok() {
  g_err[0] = '\0';
  return RA_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }

// A byte range of one tensor argument, for the overlap checks.
struct Span {
  const void *p;
  int64_t bytes;
  const char *name;
};

bool overlap(const Span &a, const Span &b) {
  if (!a.p || !b.p || a.bytes <= 0 || b.bytes <= 0) return false;
  const uintptr_t x = (uintptr_t)a.p, y = (uintptr_t)b.p;
  return x < y + (uintptr_t)b.bytes && y < x + (uintptr_t)a.bytes;
}

// Rows of a state (batch * heads * rows) or -1 on a malformed shape.
// Shape rules shared by every entry point: rows >= 0, head_dim 64 or 128, and
// the row count bounded so that element offsets fit comfortably in 64 bits.
ra_status check_shape(int32_t batch, int32_t heads, int32_t rows, int32_t head_dim,
                      const char *name, int64_t *n_rows) {
  if (batch < 0 || heads < 0 || rows < 0)
    return fail(RA_ERR_INVALID_ARG, "%s: negative shape (batch=%d heads=%d rows=%d)", name,
                batch, heads, rows);
  if (head_dim <= 0)
    return fail(RA_ERR_INVALID_ARG, "%s: head_dim=%d must be positive", name, head_dim);
  if (head_dim != 64 && head_dim != 128)
    return fail(RA_ERR_UNSUPPORTED, "%s: head_dim=%d (supported: 64, 128)", name, head_dim);
  const int64_t bh = (int64_t)batch * heads;
  if (bh > INT32_MAX) return fail(RA_ERR_INVALID_ARG, "%s: batch*heads exceeds 2^31-1", name);
  const int64_t n = bh * rows;
  if (n > ((int64_t)1 << 40) / head_dim)
    return fail(RA_ERR_INVALID_ARG, "%s: %lld rows is too large", name, (long long)n);
  *n_rows = n;
  return RA_OK;
}

ra_status check_state(const ra_state *st, const char *name, int64_t *n_rows) {
  if (!st) return fail(RA_ERR_INVALID_ARG, "%s: state pointer is NULL", name);
  int64_t n = 0;
  const ra_status s = check_shape(st->batch, st->heads, st->rows, st->head_dim, name, &n);
  if (s != RA_OK) return s;
  if (n > 0) {
    if (!st->m || !st->l || !st->o)
      return fail(RA_ERR_INVALID_ARG, "%s: NULL m, l or o with %lld rows", name, (long long)n);
    if (!aligned4(st->m) || !aligned4(st->l) || !aligned16(st->o))
      return fail(RA_ERR_INVALID_ARG, "%s: o must be 16-byte aligned, m and l 4-byte aligned", name);
    const Span parts[] = {{st->m, n * 4, "state m"}, {st->l, n * 4, "state l"},
                          {st->o, n * st->head_dim * 4, "state o"}};
    for (int i = 0; i < 3; ++i)
      for (int j = i + 1; j < 3; ++j)
        if (overlap(parts[i], parts[j]))
          return fail(RA_ERR_INVALID_ARG, "%s: %s and %s overlap", name, parts[i].name, parts[j].name);
  }
  *n_rows = n;
  return RA_OK;
}

// The bf16 kernels address a (batch, head) block, and its fp32 O state (twice
// the bytes), through buffer resources whose byte range and offsets are 32-bit.
bool bf16_block_too_long(int64_t rows, int32_t head_dim) {
  return rows * head_dim * 2 >= ((int64_t)1 << 31);
}

ra_status hip_status(hipError_t e, const char *what) {
  if (e != hipSuccess)
    return fail(RA_ERR_HIP, "%s: %s (%s)", what, hipGetErrorName(e), hipGetErrorString(e));
  return ok();
}

// Every buffer a call writes must be disjoint from every other buffer it
// touches (the kernels read and write through __restrict__ pointers, and
// different workgroups own different rows, so any overlap is a race).
template <size_t NW, size_t NR>
ra_status check_disjoint(const char *name, const Span (&w)[NW], const Span (&r)[NR]) {
  for (size_t i = 0; i < NW; ++i) {
    for (size_t j = i + 1; j < NW; ++j)
      if (overlap(w[i], w[j]))
        return fail(RA_ERR_INVALID_ARG, "%s: %s and %s overlap", name, w[i].name, w[j].name);
    for (size_t j = 0; j < NR; ++j)
      if (overlap(w[i], r[j]))
        return fail(RA_ERR_INVALID_ARG, "%s: %s and %s overlap", name, w[i].name, r[j].name);
  }
  return RA_OK;
}

}  // namespace

extern "C" {

const char *ra_status_string(ra_status s) {
  switch (s) {
    case RA_OK: return "RA_OK";
    case RA_ERR_INVALID_ARG: return "RA_ERR_INVALID_ARG";
    case RA_ERR_UNSUPPORTED: return "RA_ERR_UNSUPPORTED";
    case RA_ERR_HIP: return "RA_ERR_HIP";
  }
  return "RA_UNKNOWN_STATUS";
}

const char *ra_last_error(void) { return g_err; }

int32_t ra_step_case(int32_t q_block, int32_t kv_block, int32_t num_blocks, int32_t causal) {
  if (num_blocks < 1) return fail(RA_ERR_INVALID_ARG, "num_blocks=%d must be >= 1", num_blocks);
  if (q_block < 0 || q_block >= num_blocks || kv_block < 0 || kv_block >= num_blocks)
    return fail(RA_ERR_INVALID_ARG, "block indices (q_block=%d, kv_block=%d) outside [0, %d)",
                q_block, kv_block, num_blocks);
  if (causal != 0 && causal != 1)
    return fail(RA_ERR_INVALID_ARG, "causal=%d must be 0 or 1", causal);
  if (!causal) return RA_CASE_FULL;
  if (kv_block > q_block) return RA_CASE_SKIP;
  if (kv_block == q_block) return RA_CASE_DIAG;
  return RA_CASE_FULL;
}

ra_status ra_state_init(ra_state *st, hipStream_t stream) {
  int64_t n = 0;
  ra_status s = check_state(st, "ra_state_init", &n);
  if (s != RA_OK) return s;
  if (n == 0) return ok();
  (void)hipGetLastError();
  return hip_status(ra::launch_state_init(st->m, st->l, st->o, n, st->head_dim, stream),
                    "ra_state_init launch");
}

namespace {

// ra_step and ra_step_ex: every check before anything is enqueued.
static_assert(RA_MAX_STEP_COPIES == ra::kMaxStepCopies, "one copy limit for the ABI and the kernel");

// The copies a staged step carries: each one's own rules, then every
// destination disjoint from every other range the call touches and every
// source disjoint from what the call writes (`writes`), and the launch's work
// units countable in 31 bits (the kernel cuts the copies by them).
ra_status check_copies(const char *name, const ra_copy *copies, int32_t n_copies,
                       const Span *writes, int nw, const Span *reads, int nr, int64_t units_bound) {
  if (n_copies < 0 || n_copies > RA_MAX_STEP_COPIES)
    return fail(RA_ERR_INVALID_ARG, "%s: n_copies=%d (0 to %d)", name, n_copies, RA_MAX_STEP_COPIES);
  if (n_copies > 0 && !copies) return fail(RA_ERR_INVALID_ARG, "%s: NULL copies", name);
  for (int32_t i = 0; i < n_copies; ++i) {
    const ra_copy &c = copies[i];
    if (c.bytes == 0) continue;
    if (!c.dst || !c.src) return fail(RA_ERR_INVALID_ARG, "%s: copy %d has a NULL pointer", name, i);
    if (!aligned16(c.dst) || !aligned16(c.src) || c.bytes % 16 != 0)
      return fail(RA_ERR_INVALID_ARG, "%s: copy %d: pointers must be 16-byte aligned and bytes a multiple of 16",
                  name, i);
    if (c.bytes >= ((size_t)1 << 31))
      return fail(RA_ERR_INVALID_ARG, "%s: copy %d: %zu bytes (below 2^31 per copy)", name, i, c.bytes);
    if (units_bound >= ((int64_t)1 << 31))
      return fail(RA_ERR_UNSUPPORTED, "%s: the step is too large to carry copies", name);
    const Span d{c.dst, (int64_t)c.bytes, "a copy destination"};
    for (int32_t j = 0; j < n_copies; ++j) {
      if (copies[j].bytes == 0) continue;
      const Span sj{copies[j].src, (int64_t)copies[j].bytes, "a copy source"};
      const Span dj{copies[j].dst, (int64_t)copies[j].bytes, "another copy destination"};
      if (overlap(d, sj) || (j != i && overlap(d, dj)))
        return fail(RA_ERR_INVALID_ARG, "%s: copy %d's destination overlaps %s", name, i,
                    overlap(d, sj) ? sj.name : dj.name);
    }
    const Span src{c.src, (int64_t)c.bytes, "a copy source"};
    for (int j = 0; j < nw; ++j)
      if (overlap(d, writes[j]) || overlap(src, writes[j]))
        return fail(RA_ERR_INVALID_ARG, "%s: copy %d overlaps %s", name, i, writes[j].name);
    for (int j = 0; j < nr; ++j)
      if (overlap(d, reads[j]))
        return fail(RA_ERR_INVALID_ARG, "%s: copy %d's destination overlaps %s", name, i, reads[j].name);
  }
  return RA_OK;
}

// Enqueue the copies as full-chip copy kernels (a step that folds nothing, or
// an fp32 step).
ra_status launch_copies_alone(const char *name, const ra_copy *copies, int32_t n_copies,
                              hipStream_t stream) {
  for (int32_t i = 0; i < n_copies; ++i) {
    if (copies[i].bytes == 0) continue;
    (void)hipGetLastError();
    const ra_status s = hip_status(ra::launch_stage_copy(copies[i].dst, copies[i].src, copies[i].bytes,
                                                         true, stream), name);
    if (s != RA_OK) return s;
  }
  return ok();
}

ra_status step_impl(const char *name, ra_state *st, const void *q, const void *k, const void *v,
                    ra_dtype in_dtype, int32_t kv_rows, int32_t q_block, int32_t kv_block,
                    int32_t num_blocks, int32_t causal, float scale, uint32_t flags, void *o_out,
                    ra_dtype out_dtype, float *lse_out, hipEvent_t start, hipEvent_t stop,
                    hipStream_t stream, const ra_copy *copies = nullptr, int32_t n_copies = 0,
                    int64_t row_stride = -1, int64_t kv_row_stride = -1) {
  // row_stride, kv_row_stride: rows between consecutive (batch, head) entries
  // of q / the state / the outputs and of k / v; -1 = packed (rows, kv_rows).
  int64_t n = 0;
  ra_status s = check_state(st, name, &n);
  if (s != RA_OK) return s;
  const bool strided = row_stride >= 0 || kv_row_stride >= 0;
  const int64_t rs = row_stride < 0 ? st->rows : row_stride;
  const int64_t kvs = kv_row_stride < 0 ? (kv_rows > 0 ? kv_rows : 0) : kv_row_stride;
  if (rs < st->rows)
    return fail(RA_ERR_INVALID_ARG, "%s: row_stride=%lld is below rows=%d", name, (long long)rs, st->rows);
  if (kvs < kv_rows)
    return fail(RA_ERR_INVALID_ARG, "%s: kv_row_stride=%lld is below kv_rows=%d", name,
                (long long)kvs, kv_rows);
  const int64_t n_bh = (int64_t)st->batch * st->heads;
  if (n_bh * (rs > kvs ? rs : kvs) > ((int64_t)1 << 40) / st->head_dim)
    return fail(RA_ERR_INVALID_ARG, "%s: strided extent is too large", name);
  // Rows from the first row of the first (batch, head) entry to the end of the
  // last one: the extent of each buffer that the overlap checks compare.
  const int64_t ext = n_bh > 0 ? (n_bh - 1) * rs + st->rows : 0;
  const int32_t c = ra_step_case(q_block, kv_block, num_blocks, causal);
  if (c < 0) return (ra_status)c;
  if (in_dtype != RA_F32 && in_dtype != RA_BF16)
    return fail(RA_ERR_INVALID_ARG, "%s: in_dtype=%d is not RA_F32 or RA_BF16", name, (int)in_dtype);
  if (kv_rows < 0) return fail(RA_ERR_INVALID_ARG, "%s: kv_rows=%d is negative", name, kv_rows);
  if (kv_rows != st->rows && causal)
    return fail(RA_ERR_UNSUPPORTED,
                "%s: kv_rows=%d differs from rows=%d under the causal mask (equal blocks only)", name,
                kv_rows, st->rows);
  if ((int64_t)st->batch * st->heads * kv_rows > ((int64_t)1 << 40) / st->head_dim)
    return fail(RA_ERR_INVALID_ARG, "%s: key/value block of %d rows is too large", name, kv_rows);
  if (in_dtype == RA_BF16 && bf16_block_too_long(st->rows > kv_rows ? st->rows : kv_rows, st->head_dim))
    return fail(RA_ERR_UNSUPPORTED, "%s: bf16 blocks must stay below 2^31 bytes per (batch, head)", name);
  if (!(scale > 0.f) || !isfinite(scale))
    return fail(RA_ERR_INVALID_ARG, "%s: scale=%g must be finite and > 0", name, (double)scale);
  if (flags & ~(uint32_t)(RA_STEP_FRESH | RA_STEP_FINALIZE | RA_STEP_Q_BROADCAST))
    return fail(RA_ERR_INVALID_ARG, "%s: unknown flags 0x%x", name, (unsigned)flags);
  if (flags & RA_STEP_FINALIZE) {
    if (out_dtype != RA_F32 && out_dtype != RA_BF16)
      return fail(RA_ERR_INVALID_ARG, "%s: out_dtype=%d is not RA_F32 or RA_BF16", name, (int)out_dtype);
    if ((o_out && !aligned16(o_out)) || (lse_out && !aligned4(lse_out)))
      return fail(RA_ERR_INVALID_ARG, "%s: o_out must be 16-byte aligned, lse_out 4-byte aligned", name);
  }
  if (n > 0) {
    if (!q) return fail(RA_ERR_INVALID_ARG, "%s: NULL q", name);
    if (!aligned16(q)) return fail(RA_ERR_INVALID_ARG, "%s: q must be 16-byte aligned", name);
    if (kv_rows > 0) {
      if (!k || !v) return fail(RA_ERR_INVALID_ARG, "%s: NULL k or v", name);
      if (!aligned16(k) || !aligned16(v))
        return fail(RA_ERR_INVALID_ARG, "%s: k and v must be 16-byte aligned", name);
    }
    const int64_t es = in_dtype == RA_BF16 ? 2 : 4, d = st->head_dim;
    const int64_t q_rows = (flags & RA_STEP_Q_BROADCAST) ? (st->heads - 1) * rs + st->rows : ext;
    const int64_t kv_n = kv_rows > 0 ? (n_bh - 1) * kvs + kv_rows : 0;
    const Span in[] = {{q, q_rows * d * es, "q"}, {k, kv_n * d * es, "k"}, {v, kv_n * d * es, "v"}};
    const Span state[] = {{st->m, ext * 4, "state m"}, {st->l, ext * 4, "state l"},
                          {st->o, ext * d * 4, "state o"}};
    const Span out[] = {{o_out, ext * d * (out_dtype == RA_BF16 ? 2 : 4), "o_out"},
                        {lse_out, ext * 4, "lse_out"}};
    if (strided) {
      for (int i = 0; i < 3; ++i)
        for (int j = i + 1; j < 3; ++j)
          if (overlap(state[i], state[j]))
            return fail(RA_ERR_INVALID_ARG, "%s: %s and %s overlap", name, state[i].name, state[j].name);
    }
    if (flags & RA_STEP_FINALIZE) {
      const Span rd[] = {in[0], in[1], in[2], state[0], state[1], state[2]};
      s = check_disjoint(name, out, rd);
    } else {
      s = check_disjoint(name, state, in);
    }
    if (s != RA_OK) return s;
    if (n_copies != 0) {
      const bool fin = (flags & RA_STEP_FINALIZE) != 0;
      const Span w[] = {state[0], state[1], state[2], fin ? out[0] : Span{nullptr, 0, ""},
                        fin ? out[1] : Span{nullptr, 0, ""}};
      const int64_t units = (int64_t)st->batch * st->heads * ((st->rows + 127) / 128) *
                            ((kv_rows + 63) / 64);
      s = check_copies(name, copies, n_copies, w, 5, in, 3, units);
      if (s != RA_OK) return s;
    }
  } else if (n_copies != 0) {
    s = check_copies(name, copies, n_copies, nullptr, 0, nullptr, 0, 0);
    if (s != RA_OK) return s;
  }
  if (n == 0 || c == RA_CASE_SKIP || kv_rows == 0) {
    // Nothing to fold: the flags still take effect through the state kernels,
    // and the timing events bracket whatever they enqueue.
    if (n > 0 && strided && rs != st->rows && (flags & (RA_STEP_FRESH | RA_STEP_FINALIZE)))
      return fail(RA_ERR_UNSUPPORTED,
                  "%s: RA_STEP_FRESH or RA_STEP_FINALIZE on a strided state that folds nothing", name);
    if (start) {
      (void)hipGetLastError();
      const hipError_t e = hipEventRecord(start, stream);
      if (e != hipSuccess) return hip_status(e, name);
    }
    if (n > 0 && (flags & RA_STEP_FRESH)) {
      s = ra_state_init(st, stream);
      if (s != RA_OK) return s;
    }
    if (n > 0 && (flags & RA_STEP_FINALIZE)) {
      s = ra_finalize(st, o_out, out_dtype, lse_out, stream);
      if (s != RA_OK) return s;
    }
    if (stop) {
      (void)hipGetLastError();
      const hipError_t e = hipEventRecord(stop, stream);
      if (e != hipSuccess) return hip_status(e, name);
    }
    return launch_copies_alone(name, copies, n_copies, stream);
  }

  ra::StepArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.m = st->m;
  a.l = st->l;
  a.o = st->o;
  a.rows = st->rows;
  a.kv_rows = kv_rows;
  a.row_stride = (int32_t)rs;
  a.kv_stride = (int32_t)kvs;
  a.bh = st->batch * st->heads;
  a.q_bh = (flags & RA_STEP_Q_BROADCAST) ? st->heads : a.bh;
  a.scale_log2 = scale * 1.442695040888963407f;
  a.flags = (flags & RA_STEP_FRESH ? ra::kStepFresh : 0u) | (flags & RA_STEP_FINALIZE ? ra::kStepFinalize : 0u);
  a.o_out = (flags & RA_STEP_FINALIZE) ? o_out : nullptr;
  a.lse_out = (flags & RA_STEP_FINALIZE) ? lse_out : nullptr;
  a.out_bf16 = out_dtype == RA_BF16;
  const ra::StepCase sc = c == RA_CASE_DIAG ? ra::StepCase::Diag : ra::StepCase::Full;
  if (in_dtype == RA_BF16) {
    for (int32_t i = 0; i < n_copies; ++i) {
      if (copies[i].bytes == 0) continue;
      const int c = a.cp.n++;
      a.cp.src[c] = copies[i].src;
      a.cp.dst[c] = copies[i].dst;
      a.cp.chunks[c] = (uint32_t)(copies[i].bytes / 16);
    }
  }
  (void)hipGetLastError();
  const ra::LaunchTiming t{start, stop};
  const hipError_t e = in_dtype == RA_BF16 ? ra::launch_step_bf16(a, st->head_dim, sc, stream, t)
                                           : ra::launch_step_f32(a, st->head_dim, sc, stream, t);
  const ra_status r = hip_status(e, name);
  if (r != RA_OK || in_dtype == RA_BF16) return r;
  return launch_copies_alone(name, copies, n_copies, stream);
}

}  // namespace

ra_status ra_step(ra_state *st, const void *q, const void *k, const void *v, ra_dtype in_dtype,
                  int32_t kv_rows, int32_t q_block, int32_t kv_block, int32_t num_blocks,
                  int32_t causal, float scale, hipStream_t stream) {
  return step_impl("ra_step", st, q, k, v, in_dtype, kv_rows, q_block, kv_block, num_blocks, causal,
                   scale, 0u, nullptr, RA_F32, nullptr, nullptr, nullptr, stream);
}

ra_status ra_step_ex(ra_state *st, const void *q, const void *k, const void *v, ra_dtype in_dtype,
                     int32_t kv_rows, int32_t q_block, int32_t kv_block, int32_t num_blocks,
                     int32_t causal, float scale, uint32_t flags, void *o_out, ra_dtype out_dtype,
                     float *lse_out, hipStream_t stream) {
  return step_impl("ra_step_ex", st, q, k, v, in_dtype, kv_rows, q_block, kv_block, num_blocks,
                   causal, scale, flags, o_out, out_dtype, lse_out, nullptr, nullptr, stream);
}

ra_status ra_step_timed(ra_state *st, const void *q, const void *k, const void *v,
                        ra_dtype in_dtype, int32_t kv_rows, int32_t q_block, int32_t kv_block,
                        int32_t num_blocks, int32_t causal, float scale, uint32_t flags,
                        void *o_out, ra_dtype out_dtype, float *lse_out, hipEvent_t start,
                        hipEvent_t stop, hipStream_t stream) {
  return step_impl("ra_step_timed", st, q, k, v, in_dtype, kv_rows, q_block, kv_block, num_blocks,
                   causal, scale, flags, o_out, out_dtype, lse_out, start, stop, stream);
}

ra_status ra_step_staged(ra_state *st, const void *q, const void *k, const void *v,
                         ra_dtype in_dtype, int32_t kv_rows, int32_t q_block, int32_t kv_block,
                         int32_t num_blocks, int32_t causal, float scale, uint32_t flags,
                         void *o_out, ra_dtype out_dtype, float *lse_out, const ra_copy *copies,
                         int32_t n_copies, hipEvent_t start, hipEvent_t stop, hipStream_t stream) {
  if (n_copies < 0 || n_copies > RA_MAX_STEP_COPIES)
    return fail(RA_ERR_INVALID_ARG, "ra_step_staged: n_copies=%d (0 to %d)", n_copies, RA_MAX_STEP_COPIES);
  if (n_copies > 0 && !copies) return fail(RA_ERR_INVALID_ARG, "ra_step_staged: NULL copies");
  return step_impl("ra_step_staged", st, q, k, v, in_dtype, kv_rows, q_block, kv_block, num_blocks,
                   causal, scale, flags, o_out, out_dtype, lse_out, start, stop, stream, copies,
                   n_copies);
}

ra_status ra_step_strided(ra_state *st, int32_t row_stride, const void *q, const void *k,
                          const void *v, ra_dtype in_dtype, int32_t kv_rows, int32_t kv_row_stride,
                          int32_t q_block, int32_t kv_block, int32_t num_blocks, int32_t causal,
                          float scale, uint32_t flags, void *o_out, ra_dtype out_dtype,
                          float *lse_out, const ra_copy *copies, int32_t n_copies, hipEvent_t start,
                          hipEvent_t stop, hipStream_t stream) {
  if (row_stride < 0 || kv_row_stride < 0)
    return fail(RA_ERR_INVALID_ARG, "ra_step_strided: negative row stride (%d, %d)", row_stride,
                kv_row_stride);
  if (n_copies < 0 || n_copies > RA_MAX_STEP_COPIES)
    return fail(RA_ERR_INVALID_ARG, "ra_step_strided: n_copies=%d (0 to %d)", n_copies, RA_MAX_STEP_COPIES);
  if (n_copies > 0 && !copies) return fail(RA_ERR_INVALID_ARG, "ra_step_strided: NULL copies");
  return step_impl("ra_step_strided", st, q, k, v, in_dtype, kv_rows, q_block, kv_block, num_blocks,
                   causal, scale, flags, o_out, out_dtype, lse_out, start, stop, stream, copies,
                   n_copies, row_stride, kv_row_stride);
}

ra_status ra_lse_merge(ra_state *dst, const ra_state *src, hipStream_t stream) {
  int64_t nd = 0, ns = 0;
  ra_status s = check_state(dst, "ra_lse_merge dst", &nd);
  if (s != RA_OK) return s;
  s = check_state(src, "ra_lse_merge src", &ns);
  if (s != RA_OK) return s;
  if (dst->batch != src->batch || dst->heads != src->heads || dst->rows != src->rows ||
      dst->head_dim != src->head_dim)
    return fail(RA_ERR_INVALID_ARG, "ra_lse_merge: dst and src shapes differ");
  if (nd == 0) return ok();
  const int64_t d = dst->head_dim;
  const Span w[] = {{dst->m, nd * 4, "dst m"}, {dst->l, nd * 4, "dst l"}, {dst->o, nd * d * 4, "dst o"}};
  const Span r[] = {{src->m, ns * 4, "src m"}, {src->l, ns * 4, "src l"}, {src->o, ns * d * 4, "src o"}};
  s = check_disjoint("ra_lse_merge", w, r);
  if (s != RA_OK) return s;
  (void)hipGetLastError();
  return hip_status(ra::launch_state_merge(dst->m, dst->l, dst->o, src->m, src->l, src->o, nd,
                                           dst->head_dim, stream),
                    "ra_lse_merge launch");
}

ra_status ra_finalize(const ra_state *st, void *o_out, ra_dtype out_dtype, float *lse_out,
                      hipStream_t stream) {
  int64_t n = 0;
  ra_status s = check_state(st, "ra_finalize", &n);
  if (s != RA_OK) return s;
  if (out_dtype != RA_F32 && out_dtype != RA_BF16)
    return fail(RA_ERR_INVALID_ARG, "ra_finalize: out_dtype=%d is not RA_F32 or RA_BF16",
                (int)out_dtype);
  if (n == 0 || (!o_out && !lse_out)) return ok();
  if ((o_out && !aligned16(o_out)) || (lse_out && !aligned4(lse_out)))
    return fail(RA_ERR_INVALID_ARG, "ra_finalize: o_out must be 16-byte aligned, lse_out 4-byte aligned");
  {
    const int64_t d = st->head_dim;
    const Span w[] = {{o_out, n * d * (out_dtype == RA_BF16 ? 2 : 4), "o_out"}, {lse_out, n * 4, "lse_out"}};
    const Span r[] = {{st->m, n * 4, "state m"}, {st->l, n * 4, "state l"}, {st->o, n * d * 4, "state o"}};
    s = check_disjoint("ra_finalize", w, r);
    if (s != RA_OK) return s;
  }
  (void)hipGetLastError();
  return hip_status(ra::launch_finalize(st->m, st->l, st->o, o_out, out_dtype == RA_BF16,
                                        lse_out, n, st->head_dim, stream),
                    "ra_finalize launch");
}

ra_status ra_merge_finalize(const ra_state *st, int32_t parts, void *o_out, ra_dtype out_dtype,
                            float *lse_out, hipStream_t stream) {
  int64_t n = 0;
  ra_status s = check_state(st, "ra_merge_finalize", &n);
  if (s != RA_OK) return s;
  if (out_dtype != RA_F32 && out_dtype != RA_BF16)
    return fail(RA_ERR_INVALID_ARG, "ra_merge_finalize: out_dtype=%d is not RA_F32 or RA_BF16",
                (int)out_dtype);
  if (parts < 1 || st->batch % parts != 0)
    return fail(RA_ERR_INVALID_ARG, "ra_merge_finalize: parts=%d must be >= 1 and divide batch=%d",
                (int)parts, (int)st->batch);
  if (n == 0 || (!o_out && !lse_out)) return ok();
  if ((o_out && !aligned16(o_out)) || (lse_out && !aligned4(lse_out)))
    return fail(RA_ERR_INVALID_ARG, "ra_merge_finalize: o_out must be 16-byte aligned, lse_out 4-byte aligned");
  {
    const int64_t d = st->head_dim, no = n / parts;
    const Span w[] = {{o_out, no * d * (out_dtype == RA_BF16 ? 2 : 4), "o_out"}, {lse_out, no * 4, "lse_out"}};
    const Span r[] = {{st->m, n * 4, "state m"}, {st->l, n * 4, "state l"}, {st->o, n * d * 4, "state o"}};
    s = check_disjoint("ra_merge_finalize", w, r);
    if (s != RA_OK) return s;
  }
  const int64_t hr = (int64_t)st->heads * st->rows;
  (void)hipGetLastError();
  return hip_status(ra::launch_merge_finalize(st->m, st->l, st->o, o_out, out_dtype == RA_BF16,
                                              lse_out, n / parts, hr, parts, st->head_dim, stream),
                    "ra_merge_finalize launch");
}

ra_status ra_bwd_prepare(int32_t batch, int32_t heads, int32_t rows, int32_t head_dim,
                         const void *o, ra_dtype o_dtype, const void *dout, ra_dtype do_dtype,
                         float *delta, float *dq, hipStream_t stream) {
  int64_t n = 0;
  ra_status s = check_shape(batch, heads, rows, head_dim, "ra_bwd_prepare", &n);
  if (s != RA_OK) return s;
  if ((o_dtype != RA_F32 && o_dtype != RA_BF16) || (do_dtype != RA_F32 && do_dtype != RA_BF16))
    return fail(RA_ERR_INVALID_ARG, "ra_bwd_prepare: o_dtype and do_dtype must be RA_F32 or RA_BF16");
  if (n == 0) return ok();
  if (!o || !dout || !delta || !aligned16(o) || !aligned16(dout) || !aligned16(delta))
    return fail(RA_ERR_INVALID_ARG,
                "ra_bwd_prepare: o, dout and delta must be non-NULL and 16-byte aligned");
  if (dq && !aligned16(dq))
    return fail(RA_ERR_INVALID_ARG, "ra_bwd_prepare: dq must be 16-byte aligned");
  {
    const int64_t d = head_dim;
    const Span w[] = {{delta, n * 4, "delta"}, {dq, n * d * 4, "dq"}};
    const Span r[] = {{o, n * d * (o_dtype == RA_BF16 ? 2 : 4), "o"},
                      {dout, n * d * (do_dtype == RA_BF16 ? 2 : 4), "dout"}};
    s = check_disjoint("ra_bwd_prepare", w, r);
    if (s != RA_OK) return s;
  }
  (void)hipGetLastError();
  return hip_status(ra::launch_bwd_prepare(o, o_dtype == RA_BF16, dout, do_dtype == RA_BF16, delta,
                                           dq, n, head_dim, stream),
                    "ra_bwd_prepare launch");
}

static ra_status bwd_impl(const char *name, int32_t batch, int32_t heads, int32_t rows,
                          int32_t head_dim, const void *q, const void *dout, const float *lse,
                          const float *delta, const void *k, const void *v, ra_dtype in_dtype,
                          float *dq, float *dk, float *dv, int32_t q_block, int32_t kv_block,
                          int32_t num_blocks, int32_t causal, float scale, hipEvent_t start,
                          hipEvent_t stop, hipStream_t stream) {
  int64_t n = 0;
  ra_status s = check_shape(batch, heads, rows, head_dim, name, &n);
  if (s != RA_OK) return s;
  const int32_t c = ra_step_case(q_block, kv_block, num_blocks, causal);
  if (c < 0) return (ra_status)c;
  if (in_dtype != RA_F32 && in_dtype != RA_BF16)
    return fail(RA_ERR_INVALID_ARG, "%s: in_dtype=%d is not RA_F32 or RA_BF16", name, (int)in_dtype);
  if (in_dtype == RA_BF16 && bf16_block_too_long(rows, head_dim))
    return fail(RA_ERR_UNSUPPORTED, "%s: bf16 blocks must stay below 2^31 bytes per (batch, head)", name);
  if (!(scale > 0.f) || !isfinite(scale))
    return fail(RA_ERR_INVALID_ARG, "%s: scale=%g must be finite and > 0", name, (double)scale);
  if (n > 0) {
    const void *ptrs[] = {q, dout, lse, delta, k, v, dq, dk, dv};
    for (const void *p : ptrs)
      if (!p || !aligned16(p))
        return fail(RA_ERR_INVALID_ARG,
                    "%s: q, dout, lse, delta, k, v, dq, dk, dv must be non-NULL and 16-byte aligned", name);
    const int64_t d = head_dim, es = in_dtype == RA_BF16 ? 2 : 4;
    const Span w[] = {{dq, n * d * 4, "dq"}, {dk, n * d * 4, "dk"}, {dv, n * d * 4, "dv"}};
    const Span r[] = {{q, n * d * es, "q"}, {dout, n * d * es, "dout"}, {lse, n * 4, "lse"},
                      {delta, n * 4, "delta"}, {k, n * d * es, "k"}, {v, n * d * es, "v"}};
    s = check_disjoint(name, w, r);
    if (s != RA_OK) return s;
  }
  if (c == RA_CASE_SKIP || n == 0) {
    // Nothing to add: the timing events are recorded back to back.
    for (hipEvent_t ev : {start, stop}) {
      if (!ev) continue;
      (void)hipGetLastError();
      const hipError_t e = hipEventRecord(ev, stream);
      if (e != hipSuccess) return hip_status(e, name);
    }
    return ok();
  }
  ra::BwdArgs a;
  a.q = q;
  a.dout = dout;
  a.k = k;
  a.v = v;
  a.lse = lse;
  a.delta = delta;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.rows = rows;
  a.bh = batch * heads;
  a.scale = scale;
  a.scale_log2 = scale * 1.442695040888963407f;
  const ra::StepCase sc = c == RA_CASE_DIAG ? ra::StepCase::Diag : ra::StepCase::Full;
  (void)hipGetLastError();
  const ra::LaunchTiming t{start, stop};
  const hipError_t e = in_dtype == RA_BF16
                          ? ra::launch_bwd_step_bf16(a, head_dim, sc, stream, t)
                          : ra::launch_bwd_step_simple(a, head_dim, false, sc, stream, t);
  return hip_status(e, name);
}

ra_status ra_bwd_step(int32_t batch, int32_t heads, int32_t rows, int32_t head_dim, const void *q,
                      const void *dout, const float *lse, const float *delta, const void *k,
                      const void *v, ra_dtype in_dtype, float *dq, float *dk, float *dv,
                      int32_t q_block, int32_t kv_block, int32_t num_blocks, int32_t causal,
                      float scale, hipStream_t stream) {
  return bwd_impl("ra_bwd_step", batch, heads, rows, head_dim, q, dout, lse, delta, k, v, in_dtype,
                  dq, dk, dv, q_block, kv_block, num_blocks, causal, scale, nullptr, nullptr, stream);
}

ra_status ra_bwd_step_timed(int32_t batch, int32_t heads, int32_t rows, int32_t head_dim,
                            const void *q, const void *dout, const float *lse, const float *delta,
                            const void *k, const void *v, ra_dtype in_dtype, float *dq, float *dk,
                            float *dv, int32_t q_block, int32_t kv_block, int32_t num_blocks,
                            int32_t causal, float scale, hipEvent_t start, hipEvent_t stop,
                            hipStream_t stream) {
  return bwd_impl("ra_bwd_step_timed", batch, heads, rows, head_dim, q, dout, lse, delta, k, v,
                  in_dtype, dq, dk, dv, q_block, kv_block, num_blocks, causal, scale, start, stop,
                  stream);
}



static ra_status stage_impl(const char *name, void *dst, const void *src, size_t bytes, uint32_t flags,
                            hipStream_t stream) {
  if (flags & ~(uint32_t)RA_STAGE_ALONE) return fail(RA_ERR_INVALID_ARG, "%s: unknown flags 0x%x", name, flags);
  if (bytes == 0) return ok();
  if (!dst || !src) return fail(RA_ERR_INVALID_ARG, "%s: NULL pointer", name);
  const uintptr_t d = (uintptr_t)dst, s = (uintptr_t)src;
  if (d < s + bytes && s < d + bytes)
    return fail(RA_ERR_INVALID_ARG, "%s: source and destination overlap", name);
  if (!aligned16(dst) || !aligned16(src) || bytes % 16 != 0)
    return fail(RA_ERR_INVALID_ARG, "%s: pointers must be 16-byte aligned and bytes a multiple of 16", name);
  (void)hipGetLastError();
  return hip_status(ra::launch_stage_copy(dst, src, bytes, (flags & RA_STAGE_ALONE) != 0, stream), name);
}

ra_status ra_stage_block(void *dst, const void *src, size_t bytes, hipStream_t stream) {
  return stage_impl("ra_stage_block", dst, src, bytes, 0, stream);
}

ra_status ra_stage_block_ex(void *dst, const void *src, size_t bytes, uint32_t flags, hipStream_t stream) {
  return stage_impl("ra_stage_block_ex", dst, src, bytes, flags, stream);
}

}  // extern "C"
