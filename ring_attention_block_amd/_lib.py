"""ctypes binding of the C ABI in include/ra.h (argument marshalling only).

Torch tensors supply device pointers (``data_ptr()``) and HIP stream handles
(``torch.cuda.Stream.cuda_stream``); every step of the path runs in libra.so.
The library is loaded on first use from this package directory; if it is
missing the call raises, there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libra.so")

RA_OK, RA_ERR_INVALID_ARG, RA_ERR_UNSUPPORTED, RA_ERR_HIP = 0, -1, -2, -3
RA_F32, RA_BF16 = 0, 1
RA_CASE_SKIP, RA_CASE_DIAG, RA_CASE_FULL = 0, 1, 2
RA_STAGE_ALONE = 1

# Every symbol include/ra.h declares.
EXPORTS = ("ra_state_init", "ra_step_case", "ra_step", "ra_step_ex", "ra_step_timed", "ra_step_staged",
           "ra_step_strided", "ra_lse_merge",
           "ra_finalize", "ra_merge_finalize", "ra_stage_block", "ra_stage_block_ex", "ra_bwd_prepare", "ra_bwd_step",
           "ra_bwd_step_timed",
           "ra_status_string", "ra_last_error")


class RaState(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("rows", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("m", ctypes.c_void_p), ("l", ctypes.c_void_p),
                ("o", ctypes.c_void_p)]


class RaCopy(ctypes.Structure):
    _fields_ = [("dst", ctypes.c_void_p), ("src", ctypes.c_void_p), ("bytes", ctypes.c_size_t)]


RA_MAX_STEP_COPIES = 2


class RaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{_status_name(status)}: {detail}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libra.so (loads it on first call)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m ring_attention_block_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
        sp = ctypes.POINTER(RaState)
        sig = {
            "ra_state_init": (ctypes.c_int, [sp, vp]),
            "ra_step_case": (i32, [i32, i32, i32, i32]),
            "ra_step": (ctypes.c_int, [sp, vp, vp, vp, ctypes.c_int, i32, i32, i32, i32, i32, f32, vp]),
            "ra_step_ex": (ctypes.c_int, [sp, vp, vp, vp, ctypes.c_int, i32, i32, i32, i32, i32, f32,
                                          ctypes.c_uint32, vp, ctypes.c_int, vp, vp]),
            "ra_step_timed": (ctypes.c_int, [sp, vp, vp, vp, ctypes.c_int, i32, i32, i32, i32, i32,
                                             f32, ctypes.c_uint32, vp, ctypes.c_int, vp, vp, vp, vp]),
            "ra_step_staged": (ctypes.c_int, [sp, vp, vp, vp, ctypes.c_int, i32, i32, i32, i32, i32,
                                              f32, ctypes.c_uint32, vp, ctypes.c_int, vp,
                                              ctypes.POINTER(RaCopy), i32, vp, vp, vp]),
            "ra_step_strided": (ctypes.c_int, [sp, i32, vp, vp, vp, ctypes.c_int, i32, i32, i32, i32,
                                               i32, i32, f32, ctypes.c_uint32, vp, ctypes.c_int, vp,
                                               ctypes.POINTER(RaCopy), i32, vp, vp, vp]),
            "ra_lse_merge": (ctypes.c_int, [sp, sp, vp]),
            "ra_finalize": (ctypes.c_int, [sp, vp, ctypes.c_int, vp, vp]),
            "ra_merge_finalize": (ctypes.c_int, [sp, i32, vp, ctypes.c_int, vp, vp]),
            "ra_stage_block": (ctypes.c_int, [vp, vp, ctypes.c_size_t, vp]),
            "ra_stage_block_ex": (ctypes.c_int, [vp, vp, ctypes.c_size_t, ctypes.c_uint32, vp]),
            "ra_bwd_prepare": (ctypes.c_int, [i32, i32, i32, i32, vp, ctypes.c_int, vp, ctypes.c_int,
                                              vp, vp, vp]),
            "ra_bwd_step": (ctypes.c_int, [i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, ctypes.c_int,
                                           vp, vp, vp, i32, i32, i32, i32, f32, vp]),
            "ra_bwd_step_timed": (ctypes.c_int, [i32, i32, i32, i32, vp, vp, vp, vp, vp, vp,
                                                 ctypes.c_int, vp, vp, vp, i32, i32, i32, i32, f32,
                                                 vp, vp, vp]),
            "ra_status_string": (ctypes.c_char_p, [ctypes.c_int]),
            "ra_last_error": (ctypes.c_char_p, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _status_name(s: int) -> str:
    return lib().ra_status_string(s).decode()


def last_error() -> str:
    return lib().ra_last_error().decode()


def _check(status: int) -> int:
    if status < 0:
        raise RaError(status, last_error())
    return status


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


_IO_DTYPES = (torch.float32, torch.bfloat16)
_F32 = (torch.float32,)


# Every wrapper below validates each caller-supplied tensor before any call
# into the library, so a wrong buffer never reaches a kernel: first the layout
# of every tensor (shape, dtype, contiguity), then that all of them are GPU
# tensors (_on_gpu).

def _check_buf(name: str, t, shape, dtypes) -> None:
    """A tensor that a kernel reads or writes: contiguous, exactly `shape`,
    one of `dtypes`."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor, got {type(t).__name__}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must be one of {[str(d) for d in dtypes]}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_input(name: str, t) -> None:
    """A q, k, v, o or dout operand: contiguous (shapes and dtypes are checked
    by the caller against the other operands)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor, got {type(t).__name__}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_gpu(**tensors) -> None:
    """Every named tensor (None: absent) lives in GPU memory."""
    for name, t in tensors.items():
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor, got device {t.device}")


def _check_state(st: "State", name: str = "state") -> None:
    b, h, r, d = st.shape
    _check_buf(f"{name}.m", st.m, (b, h, r), _F32)
    _check_buf(f"{name}.l", st.l, (b, h, r), _F32)
    _check_buf(f"{name}.o", st.o, (b, h, r, d), _F32)
    _on_gpu(**{f"{name}.m": st.m, f"{name}.l": st.l, f"{name}.o": st.o})


def _event(ev) -> int | None:
    """A hipEvent_t from an event object with a .handle, a raw handle, or None."""
    if ev is None:
        return None
    return ev.handle if hasattr(ev, "handle") else ev


class State:
    """Caller-owned running state (m, l, O) as fp32 torch tensors.

    m, l: [batch, heads, rows]; o: [batch, heads, rows, head_dim].
    """

    def __init__(self, batch: int, heads: int, rows: int, head_dim: int, device="cuda"):
        self.m = torch.empty((batch, heads, rows), dtype=torch.float32, device=device)
        self.l = torch.empty((batch, heads, rows), dtype=torch.float32, device=device)
        self.o = torch.empty((batch, heads, rows, head_dim), dtype=torch.float32, device=device)
        self.c = RaState(batch, heads, rows, head_dim, self.m.data_ptr(), self.l.data_ptr(),
                         self.o.data_ptr())

    @property
    def shape(self):
        return (self.c.batch, self.c.heads, self.c.rows, self.c.head_dim)

    def row_slice(self, start: int, count: int) -> "State":
        """The state of rows [start, start + count) of every (batch, head)
        entry, sharing memory: a strided state for step_strided."""
        b, h, r, d = self.shape
        if start < 0 or count < 0 or start + count > r:
            raise ValueError(f"row slice [{start}, {start + count}) outside [0, {r})")
        view = State.__new__(State)
        view.m = self.m[:, :, start:start + count]
        view.l = self.l[:, :, start:start + count]
        view.o = self.o[:, :, start:start + count]
        view.c = RaState(b, h, count, d, view.m.data_ptr(), view.l.data_ptr(), view.o.data_ptr())
        return view

    def batch_slice(self, start: int, count: int) -> "State":
        """The state of batch entries [start, start + count), sharing memory."""
        b, h, r, d = self.shape
        if start < 0 or count < 0 or start + count > b:
            raise ValueError(f"batch slice [{start}, {start + count}) outside [0, {b})")
        view = State.__new__(State)
        view.m = self.m[start:start + count]
        view.l = self.l[start:start + count]
        view.o = self.o[start:start + count]
        view.c = RaState(count, h, r, d, view.m.data_ptr(), view.l.data_ptr(), view.o.data_ptr())
        return view


def step_case(q_block: int, kv_block: int, num_blocks: int, causal: bool) -> int:
    return _check(lib().ra_step_case(q_block, kv_block, num_blocks, int(causal)))


def state_init(st: State, stream=None) -> None:
    _check_state(st)
    _check(lib().ra_state_init(ctypes.byref(st.c), _stream(stream)))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return RA_BF16
    if t.dtype == torch.float32:
        return RA_F32
    raise TypeError(f"unsupported input dtype {t.dtype}")


RA_STEP_FRESH, RA_STEP_FINALIZE, RA_STEP_Q_BROADCAST = 1, 2, 4


def check_step(st: State, q, k, v, flags: int = 0, o_out=None, lse_out=None) -> None:
    """The checks step() makes before any library call: operand layouts,
    dtypes and shapes against the state, the finalize outputs, GPU memory."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_input(name, t)
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share one dtype")
    q_batch = 1 if flags & RA_STEP_Q_BROADCAST else k.shape[0]
    if k.shape != v.shape or k.dim() != 4 or q.dim() != 4 or \
            (q.shape[0], q.shape[1], q.shape[3]) != (q_batch, k.shape[1], k.shape[3]):
        raise ValueError(f"q, k, v shapes do not fit: {tuple(q.shape)} {tuple(k.shape)} {tuple(v.shape)}")
    if (k.shape[0], *q.shape[1:]) != st.shape:
        raise ValueError(f"q shape {tuple(q.shape)} does not match the state {st.shape}")
    b, h, r, d = st.shape
    if flags & RA_STEP_FINALIZE:
        if o_out is not None:
            _check_buf("o_out", o_out, (b, h, r, d), _IO_DTYPES)
        if lse_out is not None:
            _check_buf("lse_out", lse_out, (b, h, r), _F32)
    _on_gpu(q=q, k=k, v=v, o_out=o_out, lse_out=lse_out)
    _check_state(st)


def step(st: State, q, k, v, q_block: int, kv_block: int, num_blocks: int, causal: bool,
         scale: float, stream=None, flags: int = 0, o_out=None, lse_out=None, start=None,
         stop=None) -> int:
    """Fold block kv_block into st; returns the causal case (0 skip, 1 diag, 2 full).

    flags (ra_step_ex): RA_STEP_FRESH starts from the empty state without
    reading st; RA_STEP_FINALIZE writes o_out (fp32 or bf16) and lse_out
    instead of st, as finalize would.  start, stop (ra_step_timed): timing
    events (objects with a .handle, or raw hipEvent_t values) that take the
    begin and end of the step kernel's dispatch.
    """
    check_step(st, q, k, v, flags, o_out, lse_out)
    return step_checked(st, q, k, v, q_block, kv_block, num_blocks, causal, scale, stream, flags,
                        o_out, lse_out, start, stop)


def step_checked(st: State, q, k, v, q_block: int, kv_block: int, num_blocks: int, causal: bool,
                 scale: float, stream=None, flags: int = 0, o_out=None, lse_out=None, start=None,
                 stop=None) -> int:
    """step() without its Python checks, for a caller that ran check_step()
    on tensors of exactly these shapes, dtypes and devices (the ring driver:
    its own receive buffers, and each ring's first block).  The library still
    makes its own checks (pointers, alignment, overlaps, sizes)."""
    if flags == 0 and start is None and stop is None:
        _check(lib().ra_step(ctypes.byref(st.c), q.data_ptr(), k.data_ptr(), v.data_ptr(), _dtype_code(q),
                             k.shape[2], q_block, kv_block, num_blocks, int(causal), float(scale),
                             _stream(stream)))
    else:
        out_code = RA_BF16 if o_out is not None and o_out.dtype == torch.bfloat16 else RA_F32
        args = (ctypes.byref(st.c), q.data_ptr(), k.data_ptr(), v.data_ptr(), _dtype_code(q), k.shape[2],
                q_block, kv_block, num_blocks, int(causal), float(scale), int(flags), _ptr(o_out),
                out_code, _ptr(lse_out))
        if start is None and stop is None:
            _check(lib().ra_step_ex(*args, _stream(stream)))
        else:
            _check(lib().ra_step_timed(*args, _event(start), _event(stop), _stream(stream)))
    return step_case(q_block, kv_block, num_blocks, causal)


def check_copies(copies) -> None:
    """The checks step_staged() makes on its (dst, src) tensor pairs: at most
    RA_MAX_STEP_COPIES, contiguous GPU tensors, equal byte sizes per pair."""
    if len(copies) > RA_MAX_STEP_COPIES:
        raise ValueError(f"at most {RA_MAX_STEP_COPIES} copies per step, got {len(copies)}")
    for n, (dst, src) in enumerate(copies):
        _check_input(f"copy {n} dst", dst)
        _check_input(f"copy {n} src", src)
        _on_gpu(dst=dst, src=src)
        if dst.numel() * dst.element_size() != src.numel() * src.element_size():
            raise ValueError(f"copy {n}: sizes differ")


def _copy_array(copies):
    arr = (RaCopy * max(1, len(copies)))()
    for n, (dst, src) in enumerate(copies):
        arr[n].dst, arr[n].src = dst.data_ptr(), src.data_ptr()
        arr[n].bytes = src.numel() * src.element_size()
    return arr


def step_staged(st: State, q, k, v, q_block: int, kv_block: int, num_blocks: int, causal: bool,
                scale: float, copies=(), stream=None, flags: int = 0, o_out=None, lse_out=None,
                start=None, stop=None) -> int:
    """step() that also copies each (dst, src) of `copies` inside the step's
    launch (ra_step_staged: the next block's staging carried by the fold of
    the current one).  Returns the causal case."""
    check_step(st, q, k, v, flags, o_out, lse_out)
    check_copies(copies)
    return step_staged_checked(st, q, k, v, q_block, kv_block, num_blocks, causal, scale, copies,
                               stream, flags, o_out, lse_out, start, stop)


def step_staged_checked(st: State, q, k, v, q_block: int, kv_block: int, num_blocks: int,
                        causal: bool, scale: float, copies=(), stream=None, flags: int = 0,
                        o_out=None, lse_out=None, start=None, stop=None) -> int:
    """step_staged() without its Python checks, for a caller that ran
    check_step() and check_copies() on tensors of exactly these shapes, dtypes
    and devices.  The library still makes its own checks."""
    out_code = RA_BF16 if o_out is not None and o_out.dtype == torch.bfloat16 else RA_F32
    _check(lib().ra_step_staged(ctypes.byref(st.c), q.data_ptr(), k.data_ptr(), v.data_ptr(), _dtype_code(q),
                                k.shape[2], q_block, kv_block, num_blocks, int(causal), float(scale),
                                int(flags), _ptr(o_out), out_code, _ptr(lse_out), _copy_array(copies),
                                len(copies), _event(start), _event(stop), _stream(stream)))
    return step_case(q_block, kv_block, num_blocks, causal)


def _row_stride(name: str, t, shape, dtypes) -> int:
    """Rows between consecutive (batch, head) entries of t, a [batch, heads,
    rows] or [batch, heads, rows, head_dim] tensor of exactly `shape` whose
    rows are packed within each entry and whose entries are evenly spaced
    (a packed tensor, or a row range of a longer one); raises otherwise."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor, got {type(t).__name__}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must be one of {[str(d) for d in dtypes]}, got {t.dtype}")
    b, h, r = shape[:3]
    inner = shape[3] if len(shape) == 4 else 1
    st = t.stride()
    if len(shape) == 4 and inner > 1 and st[3] != 1:
        raise ValueError(f"{name}: elements of a row must be packed")
    if r > 1 and st[2] != inner:
        raise ValueError(f"{name}: rows of a (batch, head) entry must be packed")
    if h > 1:
        entry = st[1]
        if b > 1 and st[0] != h * entry:
            raise ValueError(f"{name}: (batch, head) entries must be evenly spaced")
    elif b > 1:
        entry = st[0]
    else:
        entry = r * inner
    if entry % inner or entry // inner < r:
        raise ValueError(f"{name}: (batch, head) entries overlap or are misaligned")
    return entry // inner


def check_step_strided(st: State, q, k, v, flags: int = 0, o_out=None, lse_out=None) -> tuple:
    """The checks step_strided() makes before any library call; returns
    (row_stride, kv_row_stride)."""
    b, h, r, d = st.shape
    rs = _row_stride("state.m", st.m, (b, h, r), _F32)
    for name, t in (("state.l", st.l), ("state.o", st.o)):
        if _row_stride(name, t, t.shape, _F32) != rs or tuple(t.shape[:3]) != (b, h, r):
            raise ValueError(f"{name} does not share the layout of state.m")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share one dtype")
    dts = (torch.bfloat16, torch.float32)
    q_batch = 1 if flags & RA_STEP_Q_BROADCAST else b
    if _row_stride("q", q, (q_batch, h, r, d), dts) != rs and q_batch * h > 1:
        raise ValueError("q must have the state's row stride")
    if k.dim() != 4 or tuple(k.shape) != tuple(v.shape) or (k.shape[0], k.shape[1], k.shape[3]) != (b, h, d):
        raise ValueError(f"k, v shapes do not fit the state: {tuple(k.shape)} {tuple(v.shape)}")
    kvs = _row_stride("k", k, k.shape, dts)
    if _row_stride("v", v, v.shape, dts) != kvs:
        raise ValueError("k and v must share one row stride")
    if flags & RA_STEP_FINALIZE:
        if o_out is not None and _row_stride("o_out", o_out, (b, h, r, d), _IO_DTYPES) != rs and b * h > 1:
            raise ValueError("o_out must have the state's row stride")
        if lse_out is not None and _row_stride("lse_out", lse_out, (b, h, r), _F32) != rs and b * h > 1:
            raise ValueError("lse_out must have the state's row stride")
    _on_gpu(q=q, k=k, v=v, o_out=o_out, lse_out=lse_out, m=st.m, l=st.l, o=st.o)
    return rs, kvs


def step_strided(st: State, q, k, v, q_block: int, kv_block: int, num_blocks: int, causal: bool,
                 scale: float, copies=(), stream=None, flags: int = 0, o_out=None, lse_out=None,
                 start=None, stop=None) -> int:
    """step_staged() on row ranges of longer blocks (ra_step_strided): q, the
    state (State.row_slice) and the outputs share one row stride, k and v
    another; every operand may also be packed.  Returns the causal case."""
    rs, kvs = check_step_strided(st, q, k, v, flags, o_out, lse_out)
    check_copies(copies)
    out_code = RA_BF16 if o_out is not None and o_out.dtype == torch.bfloat16 else RA_F32
    _check(lib().ra_step_strided(ctypes.byref(st.c), rs, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                 _dtype_code(q), k.shape[2], kvs, q_block, kv_block, num_blocks,
                                 int(causal), float(scale), int(flags), _ptr(o_out), out_code,
                                 _ptr(lse_out), _copy_array(copies), len(copies), _event(start),
                                 _event(stop), _stream(stream)))
    return step_case(q_block, kv_block, num_blocks, causal)


def lse_merge(dst: State, src: State, stream=None) -> None:
    _check_state(dst, "dst")
    _check_state(src, "src")
    _check(lib().ra_lse_merge(ctypes.byref(dst.c), ctypes.byref(src.c), _stream(stream)))


def finalize(st: State, out_dtype=torch.float32, stream=None, o_out=None, lse_out=None):
    """Return (O [B,H,rows,d] in out_dtype, LSE [B,H,rows] fp32)."""
    b, h, r, d = st.shape
    if o_out is None:
        o_out = torch.empty((b, h, r, d), dtype=out_dtype, device=st.o.device)
    if lse_out is None:
        lse_out = torch.empty((b, h, r), dtype=torch.float32, device=st.o.device)
    _check_buf("o_out", o_out, (b, h, r, d), _IO_DTYPES)
    _check_buf("lse_out", lse_out, (b, h, r), _F32)
    _on_gpu(o_out=o_out, lse_out=lse_out)
    _check_state(st)
    code = RA_BF16 if o_out.dtype == torch.bfloat16 else RA_F32
    _check(lib().ra_finalize(ctypes.byref(st.c), _ptr(o_out), code, _ptr(lse_out), _stream(stream)))
    return o_out, lse_out


def merge_finalize(st: State, parts: int, out_dtype=torch.float32, stream=None, o_out=None,
                   lse_out=None):
    """Reduce the `parts` partial states of each output batch (state batches
    b*parts .. b*parts+parts-1) and finalize.  Returns (O [B/parts,H,rows,d]
    in out_dtype, LSE [B/parts,H,rows] fp32)."""
    b, h, r, d = st.shape
    if parts < 1 or b % parts:
        raise ValueError(f"parts={parts} must divide the state batch {b}")
    if o_out is None:
        o_out = torch.empty((b // parts, h, r, d), dtype=out_dtype, device=st.o.device)
    if lse_out is None:
        lse_out = torch.empty((b // parts, h, r), dtype=torch.float32, device=st.o.device)
    _check_buf("o_out", o_out, (b // parts, h, r, d), _IO_DTYPES)
    _check_buf("lse_out", lse_out, (b // parts, h, r), _F32)
    _on_gpu(o_out=o_out, lse_out=lse_out)
    _check_state(st)
    code = RA_BF16 if o_out.dtype == torch.bfloat16 else RA_F32
    _check(lib().ra_merge_finalize(ctypes.byref(st.c), int(parts), _ptr(o_out), code, _ptr(lse_out),
                                   _stream(stream)))
    return o_out, lse_out


def stage_block(dst: torch.Tensor, src: torch.Tensor, stream=None, alone: bool = False) -> None:
    """Copy src into dst on `stream`; alone (ra_stage_block_ex with
    RA_STAGE_ALONE): no step runs beside the copy, which then takes the whole
    chip."""
    _check_input("dst", dst)
    _check_input("src", src)
    _on_gpu(dst=dst, src=src)
    if dst.numel() * dst.element_size() != src.numel() * src.element_size():
        raise ValueError("stage_block: sizes differ")
    n = src.numel() * src.element_size()
    if alone:
        _check(lib().ra_stage_block_ex(_ptr(dst), _ptr(src), n, RA_STAGE_ALONE, _stream(stream)))
    else:
        _check(lib().ra_stage_block(_ptr(dst), _ptr(src), n, _stream(stream)))


def stage_block_checked(dst: torch.Tensor, src: torch.Tensor, stream=None, alone: bool = False) -> None:
    """stage_block() without its Python checks, for a caller that checked
    both tensors (contiguous GPU tensors of one shape and dtype)."""
    n = src.numel() * src.element_size()
    if alone:
        _check(lib().ra_stage_block_ex(dst.data_ptr(), src.data_ptr(), n, RA_STAGE_ALONE, _stream(stream)))
    else:
        _check(lib().ra_stage_block(dst.data_ptr(), src.data_ptr(), n, _stream(stream)))


def bwd_prepare(o, dout, delta=None, stream=None, dq=None):
    """delta = rowsum(dout * o) [B,H,rows] fp32 (o: the forward output); dq, if
    given (fp32, o's shape), is set to zero in the same launch."""
    for name, t in (("o", o), ("dout", dout)):
        _check_input(name, t)
        if t.dim() != 4:
            raise ValueError(f"{name} must be a [B,H,rows,d] tensor")
    if o.shape != dout.shape:
        raise ValueError(f"o {tuple(o.shape)} and dout {tuple(dout.shape)} differ")
    b, h, r, d = o.shape
    if delta is None:
        delta = torch.empty((b, h, r), dtype=torch.float32, device=o.device)
    _check_buf("delta", delta, (b, h, r), _F32)
    if dq is not None:
        _check_buf("dq", dq, (b, h, r, d), _F32)
    _on_gpu(o=o, dout=dout, delta=delta, dq=dq)
    _check(lib().ra_bwd_prepare(b, h, r, d, _ptr(o), _dtype_code(o), _ptr(dout), _dtype_code(dout),
                                _ptr(delta), _ptr(dq), _stream(stream)))
    return delta


def bwd_step(q, dout, lse, delta, k, v, dq, dk, dv, q_block: int, kv_block: int,
             num_blocks: int, causal: bool, scale: float, stream=None, start=None,
             stop=None) -> int:
    """Add block kv_block's backward contribution: dq += ..., dk += ..., dv += ...
    start, stop (ra_bwd_step_timed): timing events bound to the step's first
    and last kernel dispatch.  Returns the causal case."""
    _check_input("q", q)
    if q.dim() != 4:
        raise ValueError("q must be a [B,H,rows,d] tensor")
    for name, t in (("dout", dout), ("k", k), ("v", v)):
        _check_buf(name, t, q.shape, (q.dtype,))
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check_buf(name, t, q.shape, _F32)
    b, h, r, d = q.shape
    for name, t in (("lse", lse), ("delta", delta)):
        _check_buf(name, t, (b, h, r), _F32)
    _on_gpu(q=q, dout=dout, lse=lse, delta=delta, k=k, v=v, dq=dq, dk=dk, dv=dv)
    args = (b, h, r, d, _ptr(q), _ptr(dout), _ptr(lse), _ptr(delta), _ptr(k), _ptr(v),
            _dtype_code(q), _ptr(dq), _ptr(dk), _ptr(dv), q_block, kv_block, num_blocks,
            int(causal), float(scale))
    if start is None and stop is None:
        _check(lib().ra_bwd_step(*args, _stream(stream)))
    else:
        _check(lib().ra_bwd_step_timed(*args, _event(start), _event(stop), _stream(stream)))
    return step_case(q_block, kv_block, num_blocks, causal)
