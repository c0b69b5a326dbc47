"""The Python binding rejects bad tensors before any call into the library:
wrong shape, dtype, layout or device never reaches a kernel.  CPU only: every
call below must raise on the host (CPU tensors stand in for device memory)."""
import pytest

torch = pytest.importorskip("torch")

from ring_attention_block_amd import _lib


def cpu_state(b=1, h=2, r=64, d=128):
    return _lib.State(b, h, r, d, device="cpu")


def test_state_on_host_memory_is_rejected():
    st = cpu_state()
    with pytest.raises(ValueError, match="GPU tensor"):
        _lib.state_init(st)
    with pytest.raises(ValueError, match="GPU tensor"):
        _lib.lse_merge(st, cpu_state())
    with pytest.raises(ValueError, match="GPU tensor"):
        _lib.finalize(st)


def test_finalize_checks_caller_outputs():
    st = cpu_state()
    o = torch.empty(1, 2, 64, 128)
    lse = torch.empty(1, 2, 64)
    with pytest.raises(ValueError, match="o_out must have shape"):
        _lib.finalize(st, o_out=torch.empty(1, 2, 63, 128), lse_out=lse)
    with pytest.raises(ValueError, match="lse_out must be one of"):
        _lib.finalize(st, o_out=o, lse_out=lse.to(torch.bfloat16))
    with pytest.raises(ValueError, match="o_out must be one of"):
        _lib.finalize(st, o_out=o.to(torch.float16), lse_out=lse)
    with pytest.raises(ValueError, match="contiguous"):
        _lib.finalize(st, o_out=torch.empty(1, 2, 128, 64).transpose(2, 3), lse_out=lse)
    with pytest.raises(ValueError, match="o_out must be a GPU tensor"):
        _lib.finalize(st, o_out=o, lse_out=lse)


def test_merge_finalize_checks_caller_outputs():
    st = cpu_state(b=4)
    o = torch.empty(2, 2, 64, 128)
    lse = torch.empty(2, 2, 64)
    with pytest.raises(ValueError, match="lse_out must have shape"):
        _lib.merge_finalize(st, 2, o_out=o, lse_out=torch.empty(4, 2, 64))
    with pytest.raises(ValueError, match="lse_out must be one of"):
        _lib.merge_finalize(st, 2, o_out=o, lse_out=lse.double())
    with pytest.raises(ValueError, match="contiguous"):
        _lib.merge_finalize(st, 2, o_out=o, lse_out=torch.empty(2, 64, 2).transpose(1, 2))
    with pytest.raises(ValueError, match="GPU tensor"):
        _lib.merge_finalize(st, 2, o_out=o, lse_out=lse)
    with pytest.raises(ValueError, match="divide"):
        _lib.merge_finalize(st, 3)


def test_step_checks_operands_and_outputs():
    st = cpu_state()
    q = torch.empty(1, 2, 64, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="q must be a GPU tensor"):
        _lib.step(st, q, q.clone(), q.clone(), 1, 0, 2, True, 0.1)
    with pytest.raises(ValueError, match="k must be contiguous"):
        _lib.step(st, q, torch.empty(1, 2, 128, 64, dtype=torch.bfloat16).transpose(2, 3), q, 1, 0,
                  2, True, 0.1)
    with pytest.raises(TypeError, match="torch tensor"):
        _lib.step(st, q, None, q, 1, 0, 2, True, 0.1)


def test_bwd_prepare_checks_delta_and_dq():
    o = torch.empty(1, 2, 64, 128)
    do = torch.empty(1, 2, 64, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="o must be a GPU tensor"):
        _lib.bwd_prepare(o, do)
    with pytest.raises(ValueError, match="delta must have shape"):
        _lib.bwd_prepare(o, do, delta=torch.empty(1, 2, 65))
    with pytest.raises(ValueError, match="delta must be one of"):
        _lib.bwd_prepare(o, do, delta=torch.empty(1, 2, 64, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="dq must be one of"):
        _lib.bwd_prepare(o, do, delta=torch.empty(1, 2, 64), dq=torch.empty(o.shape).double())
    with pytest.raises(ValueError, match="dq must have shape"):
        _lib.bwd_prepare(o, do, delta=torch.empty(1, 2, 64), dq=torch.empty(1, 2, 64, 64))


def test_bwd_step_checks_every_tensor():
    shp = (1, 2, 64, 128)
    bf = lambda: torch.empty(shp, dtype=torch.bfloat16)
    f32 = lambda: torch.empty(shp)
    lse, delta = torch.empty(1, 2, 64), torch.empty(1, 2, 64)
    args = lambda **kw: {**dict(q=bf(), dout=bf(), lse=lse, delta=delta, k=bf(), v=bf(), dq=f32(),
                                dk=f32(), dv=f32(), q_block=1, kv_block=0, num_blocks=2,
                                causal=True, scale=0.1), **kw}
    with pytest.raises(ValueError, match="dk must be one of"):
        _lib.bwd_step(**args(dk=bf()))
    with pytest.raises(ValueError, match="v must have shape"):
        _lib.bwd_step(**args(v=torch.empty(1, 2, 32, 128, dtype=torch.bfloat16)))
    with pytest.raises(ValueError, match="lse must have shape"):
        _lib.bwd_step(**args(lse=torch.empty(1, 2, 64, 1)))
    with pytest.raises(ValueError, match="GPU tensor"):
        _lib.bwd_step(**args())


def test_stage_block_needs_device_memory():
    with pytest.raises(ValueError, match="GPU tensor"):
        _lib.stage_block(torch.empty(16), torch.empty(16))
    with pytest.raises(ValueError, match="contiguous"):
        _lib.stage_block(torch.empty(4, 4).t(), torch.empty(16))


def test_row_stride_of_views():
    """_row_stride: packed tensors and row ranges of longer blocks are
    accepted with their entry spacing; other layouts are refused."""
    from ring_attention_block_amd._lib import _row_stride
    f32 = (torch.float32,)
    big = torch.empty(2, 3, 10, 4)
    assert _row_stride("t", big, (2, 3, 10, 4), f32) == 10
    assert _row_stride("t", big[:, :, 4:7], (2, 3, 3, 4), f32) == 10
    assert _row_stride("t", big[:1, :1, 4:7], (1, 1, 3, 4), f32) == 3     # one entry: its rows
    assert _row_stride("t", big[:, :1, 2:5], (2, 1, 3, 4), f32) == 30    # one head: batch spacing
    m = torch.empty(2, 3, 10)
    assert _row_stride("m", m[:, :, 5:], (2, 3, 5), f32) == 10
    with pytest.raises(ValueError):
        _row_stride("t", big[:, :, :, :2], (2, 3, 10, 2), f32)           # rows not packed
    with pytest.raises(ValueError):
        _row_stride("t", big[:, ::2], (2, 2, 10, 4), f32)                # heads 20 rows apart, batch 30
    with pytest.raises(ValueError):
        _row_stride("t", big.transpose(2, 3), (2, 3, 4, 10), f32)
    with pytest.raises(ValueError):
        _row_stride("t", big, (2, 3, 10, 4), (torch.bfloat16,))


def test_state_row_slice_shares_memory_and_stride():
    from ring_attention_block_amd._lib import _row_stride
    st = _lib.State(2, 3, 8, 64, device="cpu")
    view = st.row_slice(4, 4)
    assert view.shape == (2, 3, 4, 64)
    assert view.c.m == st.m.data_ptr() + 4 * 4 and view.c.o == st.o.data_ptr() + 4 * 64 * 4
    assert _row_stride("m", view.m, (2, 3, 4), (torch.float32,)) == 8
    assert _row_stride("o", view.o, (2, 3, 4, 64), (torch.float32,)) == 8
    with pytest.raises(ValueError):
        st.row_slice(6, 4)


def test_step_strided_refuses_mismatched_layouts_before_any_call():
    st = _lib.State(1, 2, 64, 128, device="cpu").row_slice(0, 32)
    q = torch.empty(1, 2, 64, 128, dtype=torch.bfloat16)
    k = torch.empty(1, 2, 64, 128, dtype=torch.bfloat16)
    # q packed at 32 rows while the state is spaced 64 apart
    with pytest.raises(ValueError):
        _lib.check_step_strided(st, q[:, :, :32].contiguous(), k, k)
    # k and v spaced differently
    with pytest.raises(ValueError):
        _lib.check_step_strided(st, q[:, :, :32], k[:, :, :16], k[:, :, :16].contiguous())
    # CPU tensors never reach the library
    with pytest.raises(ValueError, match="GPU"):
        _lib.check_step_strided(st, q[:, :, :32], k, k)
