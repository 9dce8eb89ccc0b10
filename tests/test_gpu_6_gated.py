"""Parity of the gated recurrence S_t = alpha_t S_{t-1} + k_t v_t^T (one
scalar gate per token and head) between the HIP path and the CPU oracle
(lao.fwd_gated, lao.scan_gated), through the C ABI.  Needs a gfx950 GPU."""
import numpy as np
import pytest
import torch

from gpu_helpers import gate_grad_err, TOL, WholeTensorErr, f64, log, rel_err, require_gpu
from long_sequence_causal_amd import linattn as la
from long_sequence_causal_amd.inputs import decay_schedule, gate_logs, make_inputs, workload_inputs
from oracle import lao

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _inputs(dtype, D, B, H, L, nseg, s0, seed):
    inp = make_inputs(B, H, L, D, D, dtype=dtype, s0_std=s0, nseg=nseg, seed=seed, device="cuda")
    G = gate_logs(decay_schedule(H, True), B, L, seed, device="cuda")
    return inp, G


CASES = [
    # dtype, D, B, H, L, nseg, split, S0 std
    ("bf16", 128, 2, 3, 337, 1, 0, 0.5),
    ("bf16", 128, 1, 2, 64 * 9, 1, 4, 0.5),
    ("bf16", 128, 1, 2, 64 * 9 + 5, 1, 3, 0.0),
    ("bf16", 64, 1, 4, 64 * 7, 1, 0, 0.5),
    ("bf16", 128, 1, 2, 64 * 6, 3, 2, 0.5),
    ("bf16", 128, 2, 16, 64 * 72, 1, 0, 0.5),
    ("fp32", 64, 1, 2, 1024, 1, 0, 0.0),
    ("fp32", 64, 2, 2, 130 * 4, 4, 2, 0.5),
    ("fp32", 128, 1, 2, 200, 1, 2, 0.5),
    ("bf16", 128, 1, 1, 1, 1, 0, 0.5),
]


@pytest.mark.parametrize("dtype,D,B,H,L,nseg,split,s0", CASES)
def test_gated_fwd_matches_oracle(dtype, D, B, H, L, nseg, split, s0):
    log(f"gated fwd dtype={dtype} D={D} B={B} H={H} L={L} nseg={nseg} split={split} s0={s0}")
    inp, G = _inputs(dtype, D, B, H, L, nseg, s0, 3000 + L + D)
    q, k, v, S0 = inp["q"], inp["k"], inp["v"], inp["S0"]
    O, S_end = la.la_chunk_fwd_gated(q, k, v, G, S0=S0, nseg=nseg, split=split)
    torch.cuda.synchronize()
    O_ref, S_ref = lao.fwd_gated(f64(q), f64(k), f64(v), f64(G), S0=f64(S0), nseg=nseg)
    eo, es = rel_err(f64(O), O_ref), rel_err(f64(S_end), S_ref)
    log(f"  err O={eo:.3e} S_end={es:.3e}")
    assert eo <= TOL[dtype] and es <= TOL[dtype]


def test_gated_constant_gate_matches_oracle_and_fixed_decay():
    B, H, L, D = 1, 4, 64 * 11 + 9, 128
    inp = make_inputs(B, H, L, D, D, dtype="bf16", s0_std=0.5, seed=31, device="cuda")
    q, k, v, lam, S0 = inp["q"], inp["k"], inp["v"], inp["lam"], inp["S0"]
    G = torch.log(lam.double()).float().view(1, H, 1).expand(B, H, L).contiguous()
    Og, Sg = la.la_chunk_fwd_gated(q, k, v, G, S0=S0)
    Of, Sf = la.la_chunk_fwd(q, k, v, lam, S0=S0)
    torch.cuda.synchronize()
    O_ref, S_ref = lao.fwd(f64(q), f64(k), f64(v), f64(lam), S0=f64(S0))
    errs = [rel_err(f64(Og), O_ref), rel_err(f64(Sg), S_ref), rel_err(f64(Og), f64(Of))]
    log("  constant gate: O err {:.3e}, S_end err {:.3e}, vs fixed-decay path {:.3e}".format(*errs))
    assert errs[0] <= TOL["bf16"] and errs[1] <= TOL["bf16"] and errs[2] <= 2 * TOL["bf16"]


def test_gated_extreme_and_unit_gates():
    """Gates that reset the state (log alpha = -30), that keep it (0) and
    everything between, mixed token by token: finite, and equal to the oracle."""
    B, H, L, D = 1, 2, 64 * 5 + 17, 128
    inp = make_inputs(B, H, L, D, D, dtype="bf16", s0_std=0.5, seed=32, device="cuda")
    q, k, v, S0 = inp["q"], inp["k"], inp["v"], inp["S0"]
    gen = torch.Generator(device="cuda").manual_seed(33)
    pick = torch.randint(0, 3, (B, H, L), generator=gen, device="cuda")
    G = torch.where(pick == 0, torch.full_like(pick, -30, dtype=torch.float32),
                    torch.where(pick == 1, torch.zeros_like(pick, dtype=torch.float32),
                                -torch.rand((B, H, L), generator=gen, device="cuda")))
    G = G.float().contiguous()
    O, S_end = la.la_chunk_fwd_gated(q, k, v, G, S0=S0)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(O.float()).all()) and bool(torch.isfinite(S_end).all())
    O_ref, S_ref = lao.fwd_gated(f64(q), f64(k), f64(v), f64(G), S0=f64(S0))
    eo, es = rel_err(f64(O), O_ref), rel_err(f64(S_end), S_ref)
    log(f"  extreme gates: err O={eo:.3e} S_end={es:.3e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


@pytest.mark.parametrize("P,reverse", [(1, False), (5, False), (7, True), (0, False)])
def test_gated_scan_matches_oracle(P, reverse):
    B, H, D = 2, 3, 64
    gen = torch.Generator(device="cuda").manual_seed(40 + P)
    dS = torch.randn((B, H, P, D, D), generator=gen, device="cuda")
    LD = -torch.rand((B, H, P), generator=gen, device="cuda") * 3.0
    S0 = torch.randn((B, H, D, D), generator=gen, device="cuda")
    st, en = la.la_state_scan_gated(dS, LD, S0=S0, reverse=reverse)
    torch.cuda.synchronize()
    st_ref, en_ref = lao.scan_gated(f64(dS), f64(LD), S0=f64(S0), reverse=reverse)
    if P:
        assert rel_err(f64(st), st_ref) <= TOL["fp32"]
    assert rel_err(f64(en), en_ref) <= TOL["fp32"]


def test_gated_segmented_flow_equals_monolithic():
    """Segment-local states from zero, combined by the gated scan with each
    segment's total log-gate, restart the segments exactly where one run
    over the whole sequence is."""
    B, H, P, Ls, D = 1, 4, 6, 64 * 5 + 32, 128
    L = P * Ls
    inp, G = _inputs("bf16", D, B, H, L, 1, 0.3, 41)
    q, k, v, S0 = inp["q"], inp["k"], inp["v"], inp["S0"]
    O_mono, S_mono = la.la_chunk_fwd_gated(q, k, v, G, S0=S0)
    _, dS = la.la_chunk_fwd_gated(q, k, v, G, nseg=P, need_O=False)
    LD = G.view(B, H, P, Ls).double().sum(-1).float().contiguous()
    S_start, S_end = la.la_state_scan_gated(dS, LD, S0=S0[:, :, 0].contiguous())
    O_seg, _ = la.la_chunk_fwd_gated(q, k, v, G, S0=S_start, nseg=P)
    torch.cuda.synchronize()
    e1 = rel_err(f64(O_seg), f64(O_mono))
    e2 = rel_err(f64(S_end), f64(S_mono[:, :, 0]))
    log(f"  segmented vs monolithic: O {e1:.3e}, S_end {e2:.3e}")
    assert e1 <= TOL["bf16"] and e2 <= TOL["bf16"]


def test_gated_invalid_call_writes_nothing():
    B, H, L, D = 1, 2, 128, 64
    inp, G = _inputs("bf16", D, B, H, L, 1, 0.0, 42)
    O = torch.full((B, H, L, D), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        la.la_chunk_fwd_gated(inp["q"], inp["k"], inp["v"], G[:, :, :-1].contiguous(), out=O)
    shape = la.make_shape(B, H, L, D, D, 1, la.LA_BF16, 0)
    st = la.lib().la_chunk_fwd_gated(shape, inp["q"].data_ptr(), inp["k"].data_ptr(),
                                     inp["v"].data_ptr(), None, None, O.data_ptr(), None,
                                     None, 0, None)
    assert st == la.LA_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert bool((O.float() == 7.0).all())


def test_gated_segment_64k_every_head():
    """The 64K-token, 32-head benchmark shape with gates, in the automatic
    launch configuration; the oracle checks every head, whole-tensor."""
    inp = workload_inputs("segment_64k", device="cuda")
    q, k, v, lam, S0 = inp["q"], inp["k"], inp["v"], inp["lam"], inp["S0"]
    B, H, L, D = q.shape
    G = gate_logs(lam, B, L, 3, device="cuda")
    O, S_end = la.la_chunk_fwd_gated(q, k, v, G, S0=S0)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(O.float()).all())
    acc = WholeTensorErr()
    for h0 in range(0, H, 8):
        hs = list(range(h0, min(H, h0 + 8)))
        sl = lambda t: f64(t[:, hs[0]:hs[-1] + 1])
        O_ref, S_ref = lao.fwd_gated(sl(q), sl(k), sl(v), sl(G), S0=sl(S0))
        acc.add("O", sl(O), O_ref, hs)
        acc.add("S_end", sl(S_end), S_ref, hs)
    errs = acc.report("gated segment_64k")
    assert max(errs.values()) <= TOL["bf16"]


def test_gated_empty_sequence_returns_initial_state():
    """No tokens (the log-gate tensor is empty and reaches the boundary as a
    null pointer): S_end is S0, and no gate or decay is read."""
    B, H, L, D, nseg = 1, 2, 0, 128, 1
    q = torch.empty((B, H, L, D), dtype=torch.bfloat16, device="cuda")
    G = torch.empty((B, H, L), dtype=torch.float32, device="cuda")
    S0 = torch.randn((B, H, nseg, D, D), device="cuda")
    _, S_end = la.la_chunk_fwd_gated(q, q, q, G, S0=S0, need_O=False)
    torch.cuda.synchronize()
    assert bool((S_end == S0).all())


BWD_CASES = [
    # dtype, D, B, H, L, nseg, split, S0 std, dS_end std
    ("bf16", 128, 1, 3, 337, 1, 0, 0.5, 0.5),
    ("bf16", 128, 2, 2, 64 * 8, 1, 3, 0.0, 0.0),
    ("bf16", 64, 1, 2, 64 * 5 + 30, 1, 2, 0.5, 1.0),
    ("bf16", 128, 1, 2, 64 * 6, 3, 2, 0.5, 0.5),
    ("bf16", 128, 2, 16, 64 * 20, 1, 0, 0.5, 0.5),
    ("fp32", 64, 1, 2, 1024 + 17, 1, 0, 0.0, 0.0),
    ("fp32", 64, 2, 2, 130 * 2, 2, 2, 0.5, 0.5),
    ("fp32", 128, 1, 1, 70, 1, 0, 0.5, 0.5),
    # several 1024-token sub-segments (ragged, segmented): anchored gate gradient
    ("bf16", 128, 1, 2, 5000, 1, 0, 0.5, 0.5),
    ("bf16", 64, 1, 2, 3 * 2100, 3, 0, 0.5, 0.5),
    ("fp32", 64, 1, 2, 4096 + 64, 1, 0, 0.5, 0.5),
    # sweeps walking several 1024-token blocks each from every step-th block
    # state (step 9, 5, 3), ragged in blocks and in chunks, forward and reverse
    ("bf16", 64, 1, 2, 3 * 8192 + 1037, 1, 3, 0.5, 0.5),
    ("bf16", 128, 1, 2, 2 * (2 * 4096 + 700), 2, 2, 0.5, 1.0),
    ("fp32", 64, 1, 1, 5000, 1, 2, 0.5, 0.5),
    # whole chunks (Ls % 64 == 0): the sweeps walk their own plan and write
    # the 1024-row states for the anchors themselves (joint dV/dK walk at
    # bf16 d = 128, separate walks otherwise), blocks ragged in the last
    # sub-segment
    ("bf16", 128, 1, 2, 3 * 8192 + 1024, 1, 3, 0.5, 0.5),
    ("bf16", 64, 2, 1, 2 * 4096, 2, 0, 0.5, 0.5),
    ("fp32", 128, 1, 1, 3072, 1, 2, 0.5, 1.0),
]


@pytest.mark.parametrize("dtype,D,B,H,L,nseg,split,s0,dse", BWD_CASES)
def test_gated_bwd_matches_oracle(dtype, D, B, H, L, nseg, split, s0, dse):
    log(f"gated bwd dtype={dtype} D={D} B={B} H={H} L={L} nseg={nseg} split={split} s0={s0} dSe={dse}")
    inp = make_inputs(B, H, L, D, D, dtype=dtype, s0_std=s0, nseg=nseg, need_dO=True,
                      dS_end_std=dse, seed=4000 + L + D, device="cuda")
    G = gate_logs(decay_schedule(H, True), B, L, 4000 + L, device="cuda")
    q, k, v, S0, dO, dSe = (inp[x] for x in ("q", "k", "v", "S0", "dO", "dS_end"))
    got = la.la_chunk_bwd_gated(q, k, v, G, dO, S0=S0, dS_end=dSe, nseg=nseg, split=split)
    torch.cuda.synchronize()
    ref = lao.bwd_gated(f64(q), f64(k), f64(v), f64(G), f64(dO), S0=f64(S0), dS_end=f64(dSe),
                        nseg=nseg)
    errs = [rel_err(f64(x), r) for x, r in zip(got, ref)]
    eg = gate_grad_err(f64(got[4]), ref[4], f64(q), f64(k), ref[0], ref[1], nseg)
    log("  err dQ={:.3e} dK={:.3e} dV={:.3e} dS0={:.3e} dlogalpha={:.3e} "
        "(against its terms' scale: {:.3e})".format(*errs, eg))
    assert max(errs[:4]) <= TOL[dtype]
    # dlog_alpha: fp32 on the plain measure; bf16 on the measure of a sum of
    # cancelling terms (gate_grad_err): a short-window head's gradient can be
    # a few hundred times smaller than its terms
    assert (errs[4] if dtype == "fp32" else eg) <= TOL[dtype]


FROM_FWD_CASES = [
    # dtype, D, B, H, L, nseg, split, log-gate gradient, whether the forward's states serve
    ("bf16", 128, 1, 2, 4096 * 3, 1, 3, True, True),    # 4096-token sub-segments
    ("bf16", 64, 2, 2, 1024 * 5, 1, 5, True, True),     # 1024-token sub-segments
    ("bf16", 128, 1, 2, 2 * 3072, 2, 3, True, True),    # two segments of 3 x 1024 tokens
    ("fp32", 64, 1, 2, 2048, 1, 2, True, True),         # the fp32 sweeps
    ("bf16", 128, 1, 2, 3 * 1024 - 5, 1, 3, False, True),  # ragged, no log-gate gradient
    ("bf16", 128, 1, 2, 5000, 1, 3, True, False),       # 1728-token sub-segments
    ("bf16", 128, 1, 2, 4096 + 17, 1, 2, True, False),  # ragged: the 1024-token plan
]


@pytest.mark.parametrize("dtype,D,B,H,L,nseg,split,dla,reuse", FROM_FWD_CASES)
def test_gated_bwd_from_the_forwards_states(dtype, D, B, H, L, nseg, split, dla, reuse):
    """la_chunk_bwd_gated_from_fwd right after la_chunk_fwd_gated on the same
    inputs: the oracle's gradients; la_chunk_bwd_gated's up to the rounding
    of the start states where the dQ sweep reads the forward's, bitwise where
    the plans differ and it forms its own."""
    log(f"gated bwd from fwd dtype={dtype} D={D} B={B} H={H} L={L} nseg={nseg} split={split}")
    inp = make_inputs(B, H, L, D, D, dtype=dtype, s0_std=0.5, nseg=nseg, need_dO=True,
                      dS_end_std=0.5, seed=4300 + L + D, device="cuda")
    G = gate_logs(decay_schedule(H, True), B, L, 4300 + L, device="cuda")
    q, k, v, S0, dO, dSe = (inp[x] for x in ("q", "k", "v", "S0", "dO", "dS_end"))
    shape = la.make_shape(B, H, L, D, D, nseg, la.LA_BF16 if dtype == "bf16" else la.LA_FP32,
                          split)
    fws = torch.empty(max(la.la_fwd_gated_workspace_bytes(shape), 16), dtype=torch.uint8,
                      device="cuda")
    la.la_chunk_fwd_gated(q, k, v, G, S0=S0, nseg=nseg, split=split, workspace=fws)
    got = la.la_chunk_bwd_gated(q, k, v, G, dO, S0=S0, dS_end=dSe, nseg=nseg, split=split,
                                need_dlog_alpha=dla, fwd_workspace=fws)
    own = la.la_chunk_bwd_gated(q, k, v, G, dO, S0=S0, dS_end=dSe, nseg=nseg, split=split,
                                need_dlog_alpha=dla)
    torch.cuda.synchronize()
    ref = lao.bwd_gated(f64(q), f64(k), f64(v), f64(G), f64(dO), S0=f64(S0), dS_end=f64(dSe),
                        nseg=nseg)
    n = 5 if dla else 4
    got, own, ref = got[:n], own[:n], ref[:n]
    errs = [rel_err(f64(x), r) for x, r in zip(got, ref)]
    if dla and dtype == "bf16":  # a sum of cancelling terms: gate_grad_err
        errs[4] = gate_grad_err(f64(got[4]), ref[4], f64(q), f64(k), ref[0], ref[1], nseg)
    diffs = [rel_err(f64(x), f64(y)) for x, y in zip(got, own)]
    log("  err dQ, dK, dV, dS0[, dlogalpha]: " + " ".join(f"{e:.3e}" for e in errs))
    log("  vs la_chunk_bwd_gated: " + " ".join(f"{d:.1e}" for d in diffs))
    assert max(errs) <= TOL[dtype]
    if reuse:
        assert max(diffs) <= TOL[dtype]
    else:
        assert all(torch.equal(x, y) for x, y in zip(got, own))


def test_gated_bwd_optional_outputs():
    """dS0 and the log-gate gradient may be skipped; the other gradients do
    not change."""
    B, H, L, D = 1, 2, 64 * 4 + 3, 128
    inp = make_inputs(B, H, L, D, D, dtype="bf16", s0_std=0.5, need_dO=True, dS_end_std=0.5,
                      seed=4100, device="cuda")
    G = gate_logs(decay_schedule(H, True), B, L, 4100, device="cuda")
    q, k, v, S0, dO, dSe = (inp[x] for x in ("q", "k", "v", "S0", "dO", "dS_end"))
    full = la.la_chunk_bwd_gated(q, k, v, G, dO, S0=S0, dS_end=dSe)
    part = la.la_chunk_bwd_gated(q, k, v, G, dO, S0=S0, dS_end=dSe, need_dS0=False,
                                 need_dlog_alpha=False)
    torch.cuda.synchronize()
    assert part[3] is None and part[4] is None
    for a, b in zip(full[:3], part[:3]):
        assert bool(torch.equal(a, b))


def test_gated_bwd_at_the_training_workload_every_head():
    """The 256K x 16 training workload with per-token gates, at full size in
    the launch configuration the benchmark times; the oracle checks every
    head (every token), the log-gate gradient included, whole-tensor.  Each
    head's error on its own scale is logged too: the short-window heads'
    log-gate gradients are small next to the terms of their suffix sums, so
    on their own scale they show errors of about 2 %."""
    from long_sequence_causal_amd.inputs import WORKLOADS
    w = WORKLOADS["train_256k"]
    inp = workload_inputs(w.name, device="cuda")
    q, k, v, lam, dO = inp["q"], inp["k"], inp["v"], inp["lam"], inp["dO"]
    G = gate_logs(lam, w.B, w.L, w.seed, device="cuda")
    log(f"gated bwd full size: {w.name} B={w.B} H={w.H} L={w.L}")
    got = la.la_chunk_bwd_gated(q, k, v, G, dO)
    # and from the gated forward's workspace, as a training step calls it
    shape = la.make_shape(w.B, w.H, w.L, w.d, w.d, 1, la.LA_BF16, 0)
    fws = torch.empty(max(la.la_fwd_gated_workspace_bytes(shape), 16), dtype=torch.uint8,
                      device="cuda")
    la.la_chunk_fwd_gated(q, k, v, G, need_O=False, workspace=fws)
    got_f = la.la_chunk_bwd_gated(q, k, v, G, dO, fwd_workspace=fws)
    torch.cuda.synchronize()
    names = ("dQ", "dK", "dV", "dS0", "dlogalpha")
    acc, acc_f = WholeTensorErr(), WholeTensorErr()
    for h0 in range(0, w.H, 8):
        hs = list(range(h0, min(w.H, h0 + 8)))
        sl = lambda t: f64(t[:, hs[0]:hs[-1] + 1])
        log(f"  oracle heads {hs}")
        ref = lao.bwd_gated(sl(q), sl(k), sl(v), sl(G), sl(dO))
        for n, x, xf, r in zip(names, got, got_f, ref):
            acc.add(n, sl(x), r, hs)
            acc_f.add(n, sl(xf), r, hs)
        del ref
    errs = acc.report("gated train_256k")
    errs_f = acc_f.report("gated train_256k from the forward's states")
    assert max(errs.values()) <= TOL["bf16"]
    assert max(errs_f.values()) <= TOL["bf16"]
    del q, k, v, dO, got, got_f, fws
