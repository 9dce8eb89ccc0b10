"""Parity over randomly drawn small configurations (a fixed seed, so the
same cases every run): dtype, d, B, H, ragged L, segments, internal split,
initial state, upstream state gradient and decay schedule, for every entry
point against the CPU oracle.  Complements the hand-picked cases of the
other GPU tests.  Needs a gfx950 GPU."""
import numpy as np
import pytest
import torch

from gpu_helpers import TOL, f64, gate_grad_err, log, rel_err, require_gpu
from long_sequence_causal_amd import linattn as la
from long_sequence_causal_amd.inputs import gate_logs, make_inputs
from oracle import lao

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = "fp32" if rng.random() < 0.3 else "bf16"
        D = int(rng.choice([64, 128]))
        B = int(rng.integers(1, 3))
        H = int(rng.integers(1, 5))
        nseg = int(rng.choice([1, 1, 2, 3]))
        Ls = int(rng.integers(1, 700) if rng.random() < 0.7 else rng.integers(700, 2600))
        split = int(rng.choice([0, 0, 1, 2, 5]))
        s0 = float(rng.choice([0.0, 0.5]))
        dse = float(rng.choice([0.0, 0.5]))
        decay = bool(rng.random() < 0.8)
        out.append((i, dtype, D, B, H, Ls * nseg, nseg, split, s0, dse, decay))
    return out


CASES = _cases(24, 20261)


def _draw(dtype, D, B, H, L, nseg, s0, dse, decay, seed):
    return make_inputs(B, H, L, D, D, dtype=dtype, decay=decay, s0_std=s0, nseg=nseg,
                       need_dO=True, dS_end_std=dse, seed=seed, device="cuda")


@pytest.mark.parametrize("i,dtype,D,B,H,L,nseg,split,s0,dse,decay", CASES)
def test_random_shape_fixed_decay(i, dtype, D, B, H, L, nseg, split, s0, dse, decay):
    log(f"random case {i}: dtype={dtype} D={D} B={B} H={H} L={L} nseg={nseg} split={split} "
        f"s0={s0} dS_end={dse} decay={decay}")
    inp = _draw(dtype, D, B, H, L, nseg, s0, dse, decay, 9000 + i)
    q, k, v, lam, S0, dO, dSe = (inp[x] for x in ("q", "k", "v", "lam", "S0", "dO", "dS_end"))
    O, Se = la.la_chunk_fwd(q, k, v, lam, S0=S0, nseg=nseg, split=split)
    dQ, dK, dV, dS0 = la.la_chunk_bwd(q, k, v, lam, dO, S0=S0, dS_end=dSe, nseg=nseg, split=split)
    dlam = la.la_decay_grad(q, k, v, lam, dO, S0=S0, dS_end=dSe, nseg=nseg, split=split)
    torch.cuda.synchronize()
    a = [f64(x) for x in (q, k, v, lam, dO)]
    O_r, Se_r = lao.fwd(a[0], a[1], a[2], a[3], S0=f64(S0), nseg=nseg)
    g_r = lao.bwd(a[0], a[1], a[2], a[3], a[4], S0=f64(S0), dS_end=f64(dSe), nseg=nseg)
    dl_r = lao.dlambda(a[0], a[1], a[2], a[3], a[4], S0=f64(S0), dS_end=f64(dSe), nseg=nseg)
    errs = {"O": rel_err(f64(O), O_r), "S_end": rel_err(f64(Se), Se_r),
            "dQ": rel_err(f64(dQ), g_r[0]), "dK": rel_err(f64(dK), g_r[1]),
            "dV": rel_err(f64(dV), g_r[2]), "dS0": rel_err(f64(dS0), g_r[3]),
            "dlambda": rel_err(f64(dlam), dl_r)}
    log("  " + " ".join(f"{k2}={e:.2e}" for k2, e in errs.items()))
    assert max(errs.values()) <= TOL[dtype]


@pytest.mark.parametrize("i,dtype,D,B,H,L,nseg,split,s0,dse,decay", CASES[:12])
def test_random_shape_gated(i, dtype, D, B, H, L, nseg, split, s0, dse, decay):
    log(f"random gated case {i}: dtype={dtype} D={D} B={B} H={H} L={L} nseg={nseg} split={split}")
    inp = _draw(dtype, D, B, H, L, nseg, s0, dse, True, 9100 + i)
    q, k, v, lam, S0, dO, dSe = (inp[x] for x in ("q", "k", "v", "lam", "S0", "dO", "dS_end"))
    G = gate_logs(lam, B, L, 9100 + i, device="cuda")
    O, Se = la.la_chunk_fwd_gated(q, k, v, G, S0=S0, nseg=nseg, split=split)
    got = la.la_chunk_bwd_gated(q, k, v, G, dO, S0=S0, dS_end=dSe, nseg=nseg, split=split)
    torch.cuda.synchronize()
    a = [f64(x) for x in (q, k, v, G, dO)]
    O_r, Se_r = lao.fwd_gated(a[0], a[1], a[2], a[3], S0=f64(S0), nseg=nseg)
    g_r = lao.bwd_gated(a[0], a[1], a[2], a[3], a[4], S0=f64(S0), dS_end=f64(dSe), nseg=nseg)
    errs = [rel_err(f64(O), O_r), rel_err(f64(Se), Se_r)] + [rel_err(f64(x), r) for x, r in zip(got, g_r)]
    log("  err O={:.2e} S_end={:.2e} dQ={:.2e} dK={:.2e} dV={:.2e} dS0={:.2e} dlogalpha={:.2e}".format(*errs))
    if dtype == "bf16":  # the log-gate gradient, a sum of cancelling terms: gate_grad_err
        errs[-1] = gate_grad_err(f64(got[4]), g_r[4], a[0], a[1], g_r[0], g_r[1], nseg)
    assert max(errs) <= TOL[dtype]


@pytest.mark.parametrize("i,dtype,D,B,H,L,nseg,split,s0,dse,decay", CASES[:8])
def test_random_shape_decode_step(i, dtype, D, B, H, L, nseg, split, s0, dse, decay):
    inp = _draw(dtype, D, B, H, 1, 1, 0.5, 0.0, decay, 9200 + i)
    q, k, v, lam, S0 = (inp[x] for x in ("q", "k", "v", "lam", "S0"))
    S = S0[:, :, 0].contiguous()
    o, S1 = la.la_step(q[:, :, 0].contiguous(), k[:, :, 0].contiguous(), v[:, :, 0].contiguous(),
                       lam, S)
    torch.cuda.synchronize()
    o_r, S1_r = lao.step(f64(q[:, :, 0]), f64(k[:, :, 0]), f64(v[:, :, 0]), f64(lam), f64(S))
    eo, es = rel_err(f64(o), o_r), rel_err(f64(S1), S1_r)
    log(f"random step case {i}: dtype={dtype} D={D} B={B} H={H}: err o={eo:.2e} S'={es:.2e}")
    assert eo <= TOL[dtype] and es <= TOL["fp32"]
