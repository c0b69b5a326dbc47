// Internal launchers shared by the C-ABI layer (ra_host.hip) and the kernel
// translation units.  Callers have validated every argument; launchers only
// enqueue and return the hipError_t of the launch.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ra {

// Copies a bf16 step launch carries out beside its fold (a ring's next key and
// value blocks, staged while the current one is folded).  The launch's work is
// counted in units of one key tile of one workgroup; copy k is cut into
// consecutive slices of per_unit[k] 16-byte chunks per unit, and each
// workgroup copies the slices of its own units, one chunk per thread and copy
// between two of its key tiles (and whatever is left after its last tile).
constexpr int kMaxStepCopies = 2;
struct StepCopies {
  const void *src[kMaxStepCopies];
  void *dst[kMaxStepCopies];
  uint32_t chunks[kMaxStepCopies];     // 16-byte chunks of each copy
  uint32_t per_unit[kMaxStepCopies];   // set by the launcher from its grid
  int32_t n;                           // copies (0: none)
};

// Arguments of one ring-step kernel launch.  Tensors are [bh, rows, D].
struct StepArgs {
  const void *q, *k, *v;  // bf16 (uint16 storage) or fp32, per launcher
  float *m, *l, *o;       // state
  int32_t rows;           // query rows of the block
  int32_t kv_rows;        // key/value rows of the visiting block (== rows for a diagonal block)
  int32_t row_stride;     // rows between consecutive (batch, head) entries of q, the state and
                          // the outputs (>= rows; rows for packed tensors)
  int32_t kv_stride;      // the same for k and v (>= kv_rows)
  int32_t bh;             // batch * heads
  int32_t q_bh;           // (batch, head) entries of q: q entry of bh is bh % q_bh
  float scale_log2;       // score scale * log2(e): kernels work in base 2
  uint32_t flags;         // kStepFresh, kStepFinalize
  void *o_out;            // kStepFinalize: O / l ([bh, rows, D], fp32 or bf16), may be NULL
  float *lse_out;         // kStepFinalize: m + ln l ([bh, rows]), may be NULL
  int32_t out_bf16;       // kStepFinalize: o_out is bf16
  StepCopies cp;          // bf16 launches only (the fp32 launcher ignores it)
};

// The state is not read: the step starts from the empty state (m = -inf,
// l = 0, O = 0), as after state init.
constexpr uint32_t kStepFresh = 1u;
// The step writes the finalized O / l and LSE = m + ln l (exactly as the
// finalize kernel would from the state it would have stored) instead of the
// state, which keeps its previous contents.
constexpr uint32_t kStepFinalize = 2u;

enum class StepCase : int { Diag = 1, Full = 2 };

// Arguments of one backward-step launch.  Tensors are [bh, rows, D]; the query
// side (q, dout, lse, delta, dq) belongs to block i, the key side (k, v, dk,
// dv) to block j.  dq, dk, dv are fp32 accumulators.
struct BwdArgs {
  const void *q, *dout, *k, *v;  // bf16 (uint16 storage) or fp32, per launcher
  const float *lse, *delta;      // per query row: natural-log LSE, rowsum(dO * O)
  float *dq, *dk, *dv;
  int32_t rows;
  int32_t bh;
  float scale;                   // score scale
  float scale_log2;              // scale * log2(e)
};

// Timestamps of a launch for a caller that times it: the events (either may
// be null) take the begin and the end of the kernel's own dispatch packet, so
// timing adds no marker to the stream.
struct LaunchTiming {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

// kernel(arg) on s, with start and stop (may be null) bound to the dispatch.
template <typename Arg>
hipError_t launch_one(void (*kernel)(Arg), dim3 grid, dim3 block, hipStream_t s, hipEvent_t start,
                      hipEvent_t stop, Arg arg) {
  void *args[] = {&arg};
  return hipExtLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, args, 0, s, start,
                            stop, 0);
}

hipError_t launch_state_init(float *m, float *l, float *o, int64_t n_rows, int d,
                             hipStream_t s);
hipError_t launch_state_merge(float *dm, float *dl, float *dO, const float *sm, const float *sl,
                              const float *sO, int64_t n_rows, int d, hipStream_t s);
hipError_t launch_finalize(const float *m, const float *l, const float *o, void *o_out,
                           bool out_bf16, float *lse, int64_t n_rows, int d, hipStream_t s);
// Reduce `parts` partial states per output row (state batches b*parts + p of
// output batch b) and finalize; hr = heads * rows.
hipError_t launch_merge_finalize(const float *m, const float *l, const float *o, void *o_out,
                                 bool out_bf16, float *lse, int64_t n_out_rows, int64_t hr,
                                 int parts, int d, hipStream_t s);
hipError_t launch_step_bf16(const StepArgs &a, int d, StepCase c, hipStream_t s,
                            const LaunchTiming &t = {});
hipError_t launch_step_f32(const StepArgs &a, int d, StepCase c, hipStream_t s,
                           const LaunchTiming &t = {});
// bytes a multiple of 16, both pointers 16-byte aligned, no overlap.
hipError_t launch_stage_copy(void *dst, const void *src, size_t bytes, bool alone, hipStream_t s);
hipError_t launch_bwd_prepare(const void *o, bool o_bf16, const void *dout, bool do_bf16,
                              float *delta, float *dq, int64_t n_rows, int d, hipStream_t s);
hipError_t launch_bwd_step_simple(const BwdArgs &a, int d, bool bf16, StepCase c, hipStream_t s,
                                  const LaunchTiming &t = {});
// Matrix-core backward step (bf16, head_dim 64 or 128): two kernels; t.start
// is bound to the first, t.stop to the second.
hipError_t launch_bwd_step_bf16(const BwdArgs &a, int d, StepCase c, hipStream_t s,
                                const LaunchTiming &t = {});

}  // namespace ra
