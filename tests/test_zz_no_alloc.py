"""la_chunk_fwd_noalloc (the forward without a workspace, for callers that
cannot allocate device memory) through the C ABI, against la_chunk_fwd with
a workspace: the same kernels on the same plan, so the results must agree
bit for bit.  Two calls in a row share the library's fixed scratch array,
the second with a smaller input.  A plan beyond the array is rejected before
any HIP call and writes nothing.  Needs a gfx950 GPU."""
import pytest
import torch

from gpu_helpers import log, require_gpu
from long_sequence_causal_amd import linattn as la
from long_sequence_causal_amd.inputs import make_inputs, workload_inputs

pytestmark = pytest.mark.gpu

SCRATCH = 32 << 20  # LA_NOALLOC_SCRATCH_BYTES


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _pair(q, k, v, lam, S0, nseg=1, split=0):
    """(O, S_end) from la_chunk_fwd with a workspace and from
    la_chunk_fwd_noalloc into NaN-filled buffers, and the change of the
    device's free memory across the no-alloc call."""
    B, H, L, d = q.shape
    O_ref, S_ref = la.la_chunk_fwd(q, k, v, lam, S0=S0, nseg=nseg, split=split)
    O = torch.full_like(O_ref, float("nan"))
    S = torch.full_like(S_ref, float("nan"))
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    la.la_chunk_fwd_noalloc(q, k, v, lam, O, S, S0=S0, nseg=nseg, split=split)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    return O_ref, S_ref, O, S, free0 - free1


def test_noalloc_equals_the_workspace_call_on_two_calls_in_a_row():
    shape = la.make_shape(1, 32, 65536, 128, 128, 1, la.LA_BF16, 0)
    need = la.la_fwd_workspace_bytes(shape)
    log(f"no-alloc call 1: 64K tokens x 32 heads, d=128, S0 given; plan needs {need} B of "
        f"start states (array {SCRATCH} B)")
    assert 0 < need <= SCRATCH
    inp = workload_inputs("segment_64k", device="cuda")
    q, k, v, lam, S0 = inp["q"], inp["k"], inp["v"], inp["lam"], inp["S0"]
    O_ref, S_ref, O, S, used = _pair(q, k, v, lam, S0)
    # the first call on a device resolves the array's address
    # (hipGetSymbolAddress), and the runtime maps the array then: at most
    # its size in new device memory, once
    log(f"  free device memory change across the first call: {used} B")
    assert torch.equal(O, O_ref) and torch.equal(S, S_ref)
    assert used <= SCRATCH + (4 << 20)
    # the same call again: no device memory taken
    O2 = torch.full_like(O, float("nan"))
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    la.la_chunk_fwd_noalloc(q, k, v, lam, O2, S, S0=S0)
    torch.cuda.synchronize()
    used = free0 - torch.cuda.mem_get_info()[0]
    log(f"  free device memory change across the repeated call: {used} B")
    assert used == 0
    assert torch.equal(O2, O_ref)
    del inp, q, k, v, O_ref, O, O2
    # second call, smaller: 5000 tokens (ragged) x 6 heads, 3 segments, split 4
    B, H, L, D, nseg = 2, 3, 64 * 78 + 24, 128, 3
    L -= L % nseg
    inp = make_inputs(B, H, L, D, D, s0_std=0.3, nseg=nseg, seed=808, device="cuda")
    log(f"no-alloc call 2: B={B} H={H} L={L} nseg={nseg} split=4")
    O_ref, S_ref, O, S, used = _pair(inp["q"], inp["k"], inp["v"], inp["lam"], inp["S0"],
                                     nseg=nseg, split=4)
    assert la.la_fwd_workspace_bytes(la.make_shape(B, H, L, D, D, nseg, la.LA_BF16, 4)) > 0
    log(f"  free device memory change across the call: {used} B")
    assert torch.equal(O, O_ref) and torch.equal(S, S_ref)
    assert used == 0
    # fp32, state only, then the big shape once more after the small one
    inp = make_inputs(1, 2, 64 * 10, 64, 64, dtype="fp32", seed=809, device="cuda")
    S_ref = la.la_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["lam"], need_O=False, split=3)[1]
    S = torch.full_like(S_ref, float("nan"))
    la.la_chunk_fwd_noalloc(inp["q"], inp["k"], inp["v"], inp["lam"], None, S, split=3)
    torch.cuda.synchronize()
    assert torch.equal(S, S_ref)


def test_noalloc_rejects_a_plan_beyond_its_array_and_writes_nothing():
    B, H, L, D = 1, 16, 64 * 64, 128  # split 64: 16 x 63 start states of 64 KiB
    shape = la.make_shape(B, H, L, D, D, 1, la.LA_BF16, 64)
    assert la.la_fwd_workspace_bytes(shape) > SCRATCH
    inp = make_inputs(B, H, L, D, D, seed=810, device="cuda")
    O = torch.full((B, H, L, D), 7.0, dtype=torch.bfloat16, device="cuda")
    S = torch.full((B, H, 1, D, D), 7.0, device="cuda")
    with pytest.raises(la.LinAttnError) as ei:
        la.la_chunk_fwd_noalloc(inp["q"], inp["k"], inp["v"], inp["lam"], O, S, split=64)
    assert ei.value.status == la.LA_ERR_WORKSPACE
    log(f"  rejected: {ei.value}")
    torch.cuda.synchronize()
    assert bool((O.float() == 7.0).all()) and bool((S == 7.0).all())
    # argument errors come first, before any HIP call
    with pytest.raises(la.LinAttnError) as ei:
        la.la_chunk_fwd_noalloc(inp["q"], inp["k"], inp["v"], inp["lam"], None, None)
    assert ei.value.status == la.LA_ERR_INVALID_ARG
