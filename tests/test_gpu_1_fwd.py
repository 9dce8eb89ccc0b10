"""Forward parity of the HIP path (la_chunk_fwd through the C ABI) against the
CPU oracle, on seeded inputs that span several chunks and a ragged tail,
plus the method's invariants and edge cases.  Needs a gfx950 GPU."""
import math

import numpy as np
import pytest
import torch

from gpu_helpers import TOL, f64, log, rel_err, require_gpu
from long_sequence_causal_amd import linattn as la
from long_sequence_causal_amd.inputs import decay_schedule, make_inputs
from oracle import lao

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _lam(H, kind, device="cuda"):
    if kind == "schedule":
        return decay_schedule(H).to(device)
    if kind == "one":
        return torch.ones(H, dtype=torch.float32, device=device)
    if kind == "fast":  # fast decays exercise the masks and the powers
        vals = [0.5 + 0.5 * h / max(H - 1, 1) for h in range(H)]
        return torch.tensor(vals, dtype=torch.float32, device=device)
    raise ValueError(kind)


CASES = [
    # dtype, D, B, H, L, nseg, split, S0 std, lambda kind
    ("bf16", 128, 2, 3, 337, 1, 0, 0.5, "schedule"),
    ("bf16", 128, 2, 3, 337, 1, 1, 0.5, "fast"),
    ("bf16", 128, 1, 2, 64 * 9, 1, 4, 0.5, "schedule"),
    ("bf16", 128, 1, 2, 64 * 9 + 5, 1, 3, 0.0, "fast"),
    ("bf16", 64, 1, 4, 64 * 7, 1, 0, 0.5, "fast"),
    ("bf16", 64, 2, 1, 100, 1, 2, 0.5, "one"),
    ("bf16", 128, 1, 2, 64 * 6, 3, 2, 0.5, "fast"),
    ("fp32", 64, 1, 2, 1024, 1, 0, 0.0, "one"),
    ("fp32", 64, 2, 2, 130 * 4, 4, 2, 0.5, "fast"),
    ("fp32", 128, 1, 2, 200, 1, 2, 0.5, "schedule"),
    ("fp32", 128, 1, 1, 64, 1, 0, 0.5, "fast"),
    ("bf16", 128, 1, 1, 1, 1, 0, 0.5, "fast"),
    # 32 sequences of 72 (73) chunks: 8 sub-segments of 9 (10) chunks each
    ("bf16", 128, 2, 16, 64 * 72, 1, 0, 0.5, "schedule"),
    ("fp32", 64, 1, 32, 64 * 72 + 17, 1, 0, 0.5, "fast"),
]


@pytest.mark.parametrize("dtype,D,B,H,L,nseg,split,s0,lk", CASES)
def test_fwd_matches_oracle(dtype, D, B, H, L, nseg, split, s0, lk):
    log(f"fwd case dtype={dtype} D={D} B={B} H={H} L={L} nseg={nseg} split={split} s0={s0} lam={lk}")
    inp = make_inputs(B, H, L, D, D, dtype=dtype, s0_std=s0, nseg=nseg, seed=1000 + L + D,
                      device="cuda", lam=_lam(H, lk, "cpu"))
    q, k, v, lam, S0 = inp["q"], inp["k"], inp["v"], inp["lam"], inp["S0"]
    O, S_end = la.la_chunk_fwd(q, k, v, lam, S0=S0, nseg=nseg, split=split)
    torch.cuda.synchronize()
    O_ref, S_ref = lao.fwd(f64(q), f64(k), f64(v), f64(lam), S0=f64(S0), nseg=nseg)
    eo, es = rel_err(f64(O), O_ref), rel_err(f64(S_end), S_ref)
    log(f"  err O={eo:.3e} S_end={es:.3e}")
    assert eo <= TOL[dtype] and es <= TOL[dtype]


def test_state_only_mode_matches_oracle():
    inp = make_inputs(1, 3, 64 * 10 + 3, 128, 128, s0_std=0.3, seed=77, device="cuda",
                      lam=_lam(3, "fast", "cpu"))
    for split in (0, 1, 4):
        _, S_end = la.la_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["lam"], S0=inp["S0"],
                                   need_O=False, split=split)
        _, S_ref = lao.fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["lam"]),
                           S0=f64(inp["S0"]), need_O=False)
        assert rel_err(f64(S_end), S_ref) <= TOL["bf16"]


def test_split_variants_agree():
    """Any internal split gives the same result up to rounding."""
    inp = make_inputs(1, 2, 64 * 32, 128, 128, s0_std=0.1, seed=5, device="cuda")
    outs = []
    for split in (1, 2, 5, 16, 32):
        O, S = la.la_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["lam"], S0=inp["S0"], split=split)
        outs.append((f64(O), f64(S)))
    O_ref, S_ref = lao.fwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["lam"]),
                           S0=f64(inp["S0"]))
    for O, S in outs:
        assert rel_err(O, O_ref) <= TOL["bf16"] and rel_err(S, S_ref) <= TOL["bf16"]
        assert rel_err(O, outs[0][0]) <= 5e-3


def test_deterministic_bitwise():
    inp = make_inputs(1, 4, 64 * 20 + 7, 128, 128, s0_std=0.1, seed=6, device="cuda")
    a = la.la_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["lam"], S0=inp["S0"], split=3)
    b = la.la_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["lam"], S0=inp["S0"], split=3)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_outputs_fully_overwritten():
    inp = make_inputs(2, 2, 64 * 5 + 11, 64, 64, seed=8, device="cuda")
    O = torch.full((2, 2, 64 * 5 + 11, 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    S = torch.full((2, 2, 1, 64, 64), float("nan"), dtype=torch.float32, device="cuda")
    la.la_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["lam"], split=2, out=O, S_end_out=S)
    torch.cuda.synchronize()
    assert not torch.isnan(O).any() and not torch.isnan(S).any()


def test_invalid_call_writes_nothing():
    inp = make_inputs(1, 2, 128, 128, 128, seed=9, device="cuda")
    O = torch.full((1, 2, 128, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(la.LinAttnError) as ei:
        la.la_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["lam"], nseg=3, out=O)
    assert ei.value.status == la.LA_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert torch.all(O == 7.0)


def test_empty_sequence_returns_initial_state():
    B, H, D = 1, 3, 64
    S0 = torch.randn(B, H, 1, D, D, device="cuda")
    q = torch.empty(B, H, 0, D, dtype=torch.bfloat16, device="cuda")
    lam = decay_schedule(H).cuda()
    O, S_end = la.la_chunk_fwd(q, q, q, lam, S0=S0)
    torch.cuda.synchronize()
    assert O.numel() == 0 and torch.equal(S_end, S0)
    _, S_end = la.la_chunk_fwd(q, q, q, lam, S0=None)
    torch.cuda.synchronize()
    assert torch.all(S_end == 0)


def test_zero_keys_see_only_the_decayed_initial_state():
    inp = make_inputs(1, 2, 64 * 3 + 1, 128, 128, s0_std=0.5, seed=10, device="cuda",
                      lam=_lam(2, "fast", "cpu"))
    k0 = torch.zeros_like(inp["k"])
    O, S_end = la.la_chunk_fwd(inp["q"], k0, inp["v"], inp["lam"], S0=inp["S0"])
    O_ref, S_ref = lao.fwd(f64(inp["q"]), f64(k0), f64(inp["v"]), f64(inp["lam"]),
                           S0=f64(inp["S0"]))
    assert rel_err(f64(O), O_ref) <= TOL["bf16"] and rel_err(f64(S_end), S_ref) <= TOL["bf16"]


def test_tiny_decay_attends_to_the_current_token_only():
    inp = make_inputs(1, 2, 64 * 2 + 9, 64, 64, dtype="fp32", s0_std=0.5, seed=11, device="cuda",
                      lam=torch.full((2,), 1e-30))
    O, S_end = la.la_chunk_fwd(inp["q"], inp["k"], inp["v"], inp["lam"], S0=inp["S0"])
    q, k, v = f64(inp["q"]), f64(inp["k"]), f64(inp["v"])
    ref = np.sum(q * k, axis=-1, keepdims=True) * v
    assert rel_err(f64(O), ref) <= TOL["fp32"]
    S_last = np.einsum("bhi,bhj->bhij", k[:, :, -1], v[:, :, -1])
    assert rel_err(f64(S_end)[:, :, 0], S_last) <= TOL["fp32"]


def test_streaming_resume_equals_one_run():
    inp = make_inputs(1, 2, 64 * 12, 128, 128, s0_std=0.2, seed=12, device="cuda")
    q, k, v, lam, S0 = inp["q"], inp["k"], inp["v"], inp["lam"], inp["S0"]
    L1 = 64 * 5
    O, S = la.la_chunk_fwd(q, k, v, lam, S0=S0)
    O1, S1 = la.la_chunk_fwd(q[:, :, :L1].contiguous(), k[:, :, :L1].contiguous(),
                             v[:, :, :L1].contiguous(), lam, S0=S0)
    O2, S2 = la.la_chunk_fwd(q[:, :, L1:].contiguous(), k[:, :, L1:].contiguous(),
                             v[:, :, L1:].contiguous(), lam, S0=S1)
    assert rel_err(f64(torch.cat([O1, O2], dim=2)), f64(O)) <= 5e-3
    assert rel_err(f64(S2), f64(S)) <= 1e-4
