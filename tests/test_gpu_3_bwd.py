"""Backward parity of la_chunk_bwd (through the C ABI) against the CPU
oracle's backward, on seeded inputs spanning several chunks, ragged tails,
segments and internal splits.  Needs a gfx950 GPU."""
import ctypes

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


def _fast_lam(H):
    return torch.tensor([0.5 + 0.5 * h / max(H - 1, 1) for h in range(H)], dtype=torch.float32)


CASES = [
    # dtype, D, B, H, L, nseg, split, S0 std, dS_end std, fast decay
    ("bf16", 128, 1, 3, 337, 1, 0, 0.5, 0.5, False),
    ("bf16", 128, 2, 2, 64 * 8, 1, 3, 0.0, 0.0, True),
    ("bf16", 64, 1, 2, 64 * 5 + 30, 1, 2, 0.5, 1.0, True),
    ("bf16", 128, 1, 2, 64 * 6, 3, 2, 0.5, 0.5, False),
    ("fp32", 64, 1, 2, 1024, 1, 0, 0.0, 0.0, False),
    ("fp32", 64, 2, 2, 130 * 2, 2, 2, 0.5, 0.5, True),
    ("fp32", 128, 1, 1, 70, 1, 0, 0.5, 0.5, True),
    # a short last sub-segment ending in a partial chunk (the reverse sweeps
    # then start with it), fixed decay fast and slow
    ("bf16", 128, 1, 2, 64 * 7 + 5, 1, 3, 0.5, 0.5, True),
    ("bf16", 64, 2, 1, 64 * 10 + 40, 2, 4, 0.5, 1.0, False),
    # 32 sequences of 72 chunks: 8 sub-segments of 9 chunks in all three sweeps
    ("bf16", 128, 2, 16, 64 * 72, 1, 0, 0.5, 0.5, False),
]


@pytest.mark.parametrize("dtype,D,B,H,L,nseg,split,s0,dse,fast", CASES)
def test_bwd_matches_oracle(dtype, D, B, H, L, nseg, split, s0, dse, fast):
    log(f"bwd case dtype={dtype} D={D} B={B} H={H} L={L} nseg={nseg} split={split} s0={s0} dSe={dse}")
    inp = make_inputs(B, H, L, D, D, dtype=dtype, s0_std=s0, nseg=nseg, need_dO=True,
                      dS_end_std=dse, seed=2000 + L, device="cuda",
                      lam=_fast_lam(H) if fast else None)
    q, k, v, lam, S0, dO, dSe = (inp[x] for x in ("q", "k", "v", "lam", "S0", "dO", "dS_end"))
    dQ, dK, dV, dS0 = la.la_chunk_bwd(q, k, v, lam, dO, S0=S0, dS_end=dSe, nseg=nseg, split=split)
    torch.cuda.synchronize()
    ref = lao.bwd(f64(q), f64(k), f64(v), f64(lam), f64(dO), S0=f64(S0), dS_end=f64(dSe), nseg=nseg)
    errs = [rel_err(f64(x), r) for x, r in zip((dQ, dK, dV, dS0), ref)]
    log("  err dQ={:.3e} dK={:.3e} dV={:.3e} dS0={:.3e}".format(*errs))
    assert max(errs) <= TOL[dtype]


def test_bwd_without_dS0():
    inp = make_inputs(1, 2, 64 * 3, 64, 64, need_dO=True, seed=31, device="cuda")
    dQ, dK, dV, dS0 = la.la_chunk_bwd(inp["q"], inp["k"], inp["v"], inp["lam"], inp["dO"],
                                      need_dS0=False)
    ref = lao.bwd(f64(inp["q"]), f64(inp["k"]), f64(inp["v"]), f64(inp["lam"]), f64(inp["dO"]))
    assert dS0 is None
    for x, r in zip((dQ, dK, dV), ref[:3]):
        assert rel_err(f64(x), r) <= TOL["bf16"]


def test_bwd_deterministic_bitwise():
    inp = make_inputs(1, 2, 64 * 9 + 3, 128, 128, need_dO=True, s0_std=0.1, seed=32, device="cuda")
    a = la.la_chunk_bwd(inp["q"], inp["k"], inp["v"], inp["lam"], inp["dO"], S0=inp["S0"], split=3)
    b = la.la_chunk_bwd(inp["q"], inp["k"], inp["v"], inp["lam"], inp["dO"], S0=inp["S0"], split=3)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_euler_identities():
    """<dQ,Q> = <dO,O>; <dK,K> + <dS0,S0> = <dV,V> + <dS0,S0> = <dO,O> + <dS_end,S_end>
    (the loss is linear in Q and jointly linear in (K, S0) and in (V, S0))."""
    inp = make_inputs(1, 4, 64 * 16 + 5, 128, 128, need_dO=True, s0_std=0.3, dS_end_std=0.3,
                      seed=33, device="cuda")
    q, k, v, lam, S0, dO, dSe = (inp[x] for x in ("q", "k", "v", "lam", "S0", "dO", "dS_end"))
    O, S_end = la.la_chunk_fwd(q, k, v, lam, S0=S0)
    dQ, dK, dV, dS0 = la.la_chunk_bwd(q, k, v, lam, dO, S0=S0, dS_end=dSe)
    Q, K, V, G = f64(q), f64(k), f64(v), f64(dO)
    lo = np.sum(G * f64(O))
    l = lo + np.sum(f64(dSe) * f64(S_end))
    s0t = np.sum(f64(dS0) * f64(S0))
    t_q = np.sum(f64(dQ) * Q)
    t_k = np.sum(f64(dK) * K)
    t_v = np.sum(f64(dV) * V)
    scale = np.sum(np.abs(f64(dQ) * Q)) + np.sum(np.abs(f64(dS0) * f64(S0)))
    assert abs(t_q - lo) <= 1e-2 * np.sum(np.abs(f64(dQ) * Q))
    assert abs(t_k + s0t - l) <= 1e-2 * (np.sum(np.abs(f64(dK) * K)) + abs(s0t))
    assert abs(t_v + s0t - l) <= 1e-2 * (np.sum(np.abs(f64(dV) * V)) + abs(s0t))
    assert scale > 0


FROM_FWD_CASES = [
    # dtype, D, B, H, L, nseg, split, S0 std, dS_end std
    ("bf16", 128, 1, 4, 64 * 40 + 17, 1, 0, 0.5, 0.5),
    ("bf16", 128, 2, 3, 64 * 12, 2, 3, 0.5, 0.0),
    ("bf16", 64, 1, 2, 64 * 9, 1, 4, 0.0, 0.5),
    ("fp32", 64, 1, 2, 64 * 10 + 5, 1, 3, 0.5, 0.5),
]


@pytest.mark.parametrize("dtype,D,B,H,L,nseg,split,s0,dse", FROM_FWD_CASES)
def test_bwd_from_forward_states(dtype, D, B, H, L, nseg, split, s0, dse):
    """la_chunk_bwd_from_fwd with the workspace of the forward call just made
    matches the oracle and the plain backward."""
    log(f"bwd from fwd states dtype={dtype} D={D} B={B} H={H} L={L} nseg={nseg} split={split}")
    inp = make_inputs(B, H, L, D, D, dtype=dtype, s0_std=s0, nseg=nseg, need_dO=True,
                      dS_end_std=dse, seed=700 + L + D, device="cuda")
    q, k, v, lam, S0, dO, dSe = (inp[x] for x in ("q", "k", "v", "lam", "S0", "dO", "dS_end"))
    shape = la.make_shape(B, H, L, D, D, nseg, la._dtype_code(q.dtype), split)
    fws = torch.empty(max(la.la_fwd_workspace_bytes(shape), 16), dtype=torch.uint8, device="cuda")
    la.la_chunk_fwd(q, k, v, lam, S0=S0, nseg=nseg, split=split, workspace=fws)
    got = la.la_chunk_bwd(q, k, v, lam, dO, S0=S0, dS_end=dSe, nseg=nseg, split=split,
                          fwd_workspace=fws)
    plain = la.la_chunk_bwd(q, k, v, lam, dO, S0=S0, dS_end=dSe, nseg=nseg, split=split)
    torch.cuda.synchronize()
    ref = lao.bwd(f64(q), f64(k), f64(v), f64(lam), f64(dO), S0=f64(S0), dS_end=f64(dSe), nseg=nseg)
    errs = [rel_err(f64(x), r) for x, r in zip(got, ref)]
    diffs = [rel_err(f64(x), f64(y)) for x, y in zip(got, plain)]
    log("  err dQ={:.3e} dK={:.3e} dV={:.3e} dS0={:.3e}".format(*errs))
    log("  vs plain backward dQ={:.3e} dK={:.3e} dV={:.3e} dS0={:.3e}".format(*diffs))
    assert max(errs) <= TOL[dtype]
    # only dQ can differ (its start states); dK, dV, dS0 take the same path
    assert all(bool(torch.equal(x, y)) for x, y in zip(got[1:], plain[1:]))


def test_bwd_from_forward_states_requires_the_workspace():
    B, H, L, D = 1, 2, 64 * 8, 64
    inp = make_inputs(B, H, L, D, D, need_dO=True, seed=9, device="cuda")
    q, k, v, lam, dO = inp["q"], inp["k"], inp["v"], inp["lam"], inp["dO"]
    shape = la.make_shape(B, H, L, D, D, 1, la.LA_BF16, 4)
    ws = torch.empty(la.la_bwd_workspace_bytes(shape), dtype=torch.uint8, device="cuda")
    out = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)]
    st = la.lib().la_chunk_bwd_from_fwd(ctypes.byref(shape), la._ptr(q), la._ptr(k), la._ptr(v),
                                        la._ptr(lam), None, la._ptr(dO), None, None,
                                        la._ptr(out[0]), la._ptr(out[1]), la._ptr(out[2]), None,
                                        la._ptr(ws), ws.numel(), None)
    assert st == la.LA_ERR_INVALID_ARG


@pytest.mark.parametrize("lam0", [0.0, 1e-38, 1e-30])
@pytest.mark.parametrize("dtype,D,split", [("bf16", 128, 0), ("bf16", 128, 3), ("fp32", 64, 2)])
def test_tiny_and_zero_decay_forward_and_backward(lam0, dtype, D, split):
    """lambda = 0 (each token sees only itself; 0^0 = 1), a denormal fp32
    lambda (1e-38) and 1e-30, next to a slow head, with S0 and dS_end given:
    forward and backward match the oracle and stay finite.  The backward
    seeds its reverse sweeps with dS_end itself (never dS_end / lambda)."""
    B, H, L = 1, 2, 64 * 5 + 17
    lam = torch.tensor([lam0, 0.97], dtype=torch.float32)
    log(f"tiny decay case lambda0={float(lam[0]):.3e} dtype={dtype} D={D} split={split}")
    inp = make_inputs(B, H, L, D, D, dtype=dtype, s0_std=0.5, need_dO=True, dS_end_std=0.5,
                      seed=91, device="cuda", lam=lam)
    q, k, v, lam, S0, dO, dSe = (inp[x] for x in ("q", "k", "v", "lam", "S0", "dO", "dS_end"))
    O, S_end = la.la_chunk_fwd(q, k, v, lam, S0=S0, split=split)
    dQ, dK, dV, dS0 = la.la_chunk_bwd(q, k, v, lam, dO, S0=S0, dS_end=dSe, split=split)
    torch.cuda.synchronize()
    for t in (O, S_end, dQ, dK, dV, dS0):
        assert bool(torch.isfinite(t.float()).all())
    O_r, S_r = lao.fwd(f64(q), f64(k), f64(v), f64(lam), S0=f64(S0))
    ref = lao.bwd(f64(q), f64(k), f64(v), f64(lam), f64(dO), S0=f64(S0), dS_end=f64(dSe))
    errs = [rel_err(f64(O), O_r), rel_err(f64(S_end), S_r)]
    errs += [rel_err(f64(x), r) for x, r in zip((dQ, dK, dV, dS0), ref)]
    # the fast head on its own (its outputs are small next to the slow head's)
    own = [rel_err(f64(O[:, :1]), O_r[:, :1]), rel_err(f64(dK[:, :1]), ref[1][:, :1]),
           rel_err(f64(dS0[:, :1]), ref[3][:, :1])]
    log("  err O={:.3e} S_end={:.3e} dQ={:.3e} dK={:.3e} dV={:.3e} dS0={:.3e}".format(*errs)
        + "; fast head alone O={:.3e} dK={:.3e} dS0={:.3e}".format(*own))
    assert max(errs) <= TOL[dtype]
    assert max(own) <= TOL[dtype]
