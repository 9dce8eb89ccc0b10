"""A second seeded random sweep, weighted towards segments of whole 64-token
chunks and segments across several 1024-token blocks (where the gated
backward's sweeps write the 1024-row states for the anchors themselves and the
row sums run in one pass), and towards the backward taking the forward's
workspace: per drawn configuration (dtype, d, batch, heads, segment length,
segments, internal split, S0, dS_end) one of the forward with the backward
from its workspace, the backward on its own, the gated backward (every other
one after the gated forward, from its workspace) or the decay gradient,
against the CPU oracle.  The draws are fixed by the seed, so a
failure names a reproducible case.  Needs a gfx950 GPU."""
import random

import pytest
import torch

from gpu_helpers import TOL, f64, gate_grad_err, log, rel_err, require_gpu
from long_sequence_causal_amd import linattn as la
from long_sequence_causal_amd.inputs import decay_schedule, gate_logs, make_inputs
from oracle import lao

pytestmark = pytest.mark.gpu

SEED = 20261203
NCASES = 40


def _draw_cases():
    rng = random.Random(SEED)
    cases = []
    for i in range(NCASES):
        dtype = rng.choice(["bf16", "bf16", "fp32"])
        D = rng.choice([64, 128, 128])
        B = rng.choice([1, 2])
        H = rng.choice([1, 2, 3])
        nseg = rng.choice([1, 1, 2, 3])
        Ls = rng.choice([rng.randint(1, 200), 64 * rng.randint(1, 12),
                         64 * rng.randint(1, 20) + rng.randint(1, 63),
                         1024 * rng.randint(1, 2) + 64 * rng.randint(0, 3)])
        split = rng.choice([0, 0, 1, 2, 3, 5])
        s0 = rng.choice([0.0, 0.5])
        dse = rng.choice([0.0, 0.5])
        what = ("fwd_bwd_from_fwd", "bwd", "gated_bwd", "decay_grad")[i % 4]
        cases.append((i, what, dtype, D, B, H, Ls * nseg, nseg, split, s0, dse))
    return cases


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("i,what,dtype,D,B,H,L,nseg,split,s0,dse", _draw_cases())
def test_random_shape_matches_oracle(i, what, dtype, D, B, H, L, nseg, split, s0, dse):
    log(f"case {i} {what} dtype={dtype} D={D} B={B} H={H} L={L} nseg={nseg} split={split} "
        f"s0={s0} dSe={dse}")
    inp = make_inputs(B, H, L, D, D, dtype=dtype, s0_std=s0, nseg=nseg, need_dO=True,
                      dS_end_std=dse, seed=10000 + i, device="cuda")
    q, k, v, lam, S0, dO, dSe = (inp[x] for x in ("q", "k", "v", "lam", "S0", "dO", "dS_end"))
    tol = TOL[dtype]
    if what == "fwd_bwd_from_fwd":
        shape = la.make_shape(B, H, L, D, D, nseg, la.LA_BF16 if dtype == "bf16" else la.LA_FP32,
                              split)
        fws = torch.empty(max(la.la_fwd_workspace_bytes(shape), 1), dtype=torch.uint8,
                          device="cuda")
        O, S_end = la.la_chunk_fwd(q, k, v, lam, S0=S0, nseg=nseg, split=split, workspace=fws)
        got = la.la_chunk_bwd(q, k, v, lam, dO, S0=S0, dS_end=dSe, nseg=nseg, split=split,
                              fwd_workspace=fws)
        torch.cuda.synchronize()
        ref_f = lao.fwd(f64(q), f64(k), f64(v), f64(lam), S0=f64(S0), nseg=nseg)
        ref_b = lao.bwd(f64(q), f64(k), f64(v), f64(lam), f64(dO), S0=f64(S0), dS_end=f64(dSe),
                        nseg=nseg)
        errs = [rel_err(f64(O), ref_f[0]), rel_err(f64(S_end), ref_f[1])]
        errs += [rel_err(f64(x), r) for x, r in zip(got, ref_b)]
        bounds = [tol] * len(errs)
    elif what == "bwd":
        got = la.la_chunk_bwd(q, k, v, lam, dO, S0=S0, dS_end=dSe, nseg=nseg, split=split)
        torch.cuda.synchronize()
        ref = lao.bwd(f64(q), f64(k), f64(v), f64(lam), f64(dO), S0=f64(S0), dS_end=f64(dSe),
                      nseg=nseg)
        errs = [rel_err(f64(x), r) for x, r in zip(got, ref)]
        bounds = [tol] * len(errs)
    elif what == "gated_bwd":
        G = gate_logs(decay_schedule(H, True), B, L, 10000 + i, device="cuda")
        errs = []
        fws = None
        if i % 8 == 6:  # every other one after the gated forward, from its workspace
            shape = la.make_shape(B, H, L, D, D, nseg,
                                  la.LA_BF16 if dtype == "bf16" else la.LA_FP32, split)
            fws = torch.empty(max(la.la_fwd_gated_workspace_bytes(shape), 16), dtype=torch.uint8,
                              device="cuda")
            O, S_end = la.la_chunk_fwd_gated(q, k, v, G, S0=S0, nseg=nseg, split=split,
                                             workspace=fws)
            torch.cuda.synchronize()
            ref_f = lao.fwd_gated(f64(q), f64(k), f64(v), f64(G), S0=f64(S0), nseg=nseg)
            errs = [rel_err(f64(O), ref_f[0]), rel_err(f64(S_end), ref_f[1])]
        got = la.la_chunk_bwd_gated(q, k, v, G, dO, S0=S0, dS_end=dSe, nseg=nseg, split=split,
                                    fwd_workspace=fws)
        torch.cuda.synchronize()
        ref = lao.bwd_gated(f64(q), f64(k), f64(v), f64(G), f64(dO), S0=f64(S0), dS_end=f64(dSe),
                            nseg=nseg)
        errs += [rel_err(f64(x), r) for x, r in zip(got, ref)]
        if dtype == "bf16":  # the log-gate gradient, a sum of cancelling terms
            errs[-1] = gate_grad_err(f64(got[4]), ref[4], f64(q), f64(k), ref[0], ref[1], nseg)
        bounds = [tol] * len(errs)
    else:
        got = la.la_decay_grad(q, k, v, lam, dO, S0=S0, dS_end=dSe, nseg=nseg, split=split)
        torch.cuda.synchronize()
        ref = lao.dlambda(f64(q), f64(k), f64(v), f64(lam), f64(dO), S0=f64(S0),
                          dS_end=f64(dSe), nseg=nseg)
        errs = [rel_err(f64(got), ref)]
        bounds = [tol]
    log("  errs " + " ".join(f"{e:.3e}" for e in errs))
    for e, b in zip(errs, bounds):
        assert e <= b
