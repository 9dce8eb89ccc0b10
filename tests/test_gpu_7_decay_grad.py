"""Parity of the decay gradient d l / d lambda_h (la_decay_grad, forward-mode
tangent walk) between the HIP path and the CPU oracle (lao.dlambda, the
gated backward with every gate at log lambda_h, pinned by finite
differences), through the C ABI.  Needs a gfx950 GPU."""
import numpy as np
import pytest
import torch

from gpu_helpers import TOL, f64, log, rel_err, require_gpu
from long_sequence_causal_amd import linattn as la
from long_sequence_causal_amd.inputs import make_inputs, workload_inputs
from oracle import lao

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


CASES = [
    # dtype, D, B, H, L, nseg, split, S0 std, dS_end std, decay
    ("fp32", 64, 2, 2, 200, 1, 0, 0.5, 0.5, True),
    ("fp32", 128, 1, 2, 64 * 6, 2, 3, 0.5, 0.5, True),
    ("fp32", 128, 1, 2, 64 * 5 + 23, 1, 2, 0.5, 0.5, True),  # ragged, no scratch spills
    ("fp32", 64, 1, 3, 1000, 1, 1, 0.0, 0.0, True),
    ("fp32", 64, 1, 2, 300, 1, 0, 0.5, 0.5, False),
    ("bf16", 128, 2, 3, 337, 1, 0, 0.5, 0.5, True),
    ("bf16", 128, 1, 4, 5000, 1, 0, 0.0, 0.5, True),
    ("bf16", 64, 1, 4, 64 * 7 + 3, 1, 0, 0.5, 0.0, True),
    ("bf16", 128, 1, 2, 64 * 6, 3, 2, 0.5, 0.5, True),
    ("bf16", 128, 2, 16, 64 * 72, 1, 0, 0.5, 0.5, True),
    ("bf16", 128, 1, 2, 2000, 1, 0, 0.5, 0.5, False),
    ("bf16", 128, 1, 1, 1, 1, 0, 0.5, 0.5, True),
]


@pytest.mark.parametrize("dtype,D,B,H,L,nseg,split,s0,dse,decay", CASES)
def test_decay_grad_matches_oracle(dtype, D, B, H, L, nseg, split, s0, dse, decay):
    log(f"decay grad dtype={dtype} D={D} B={B} H={H} L={L} nseg={nseg} split={split} "
        f"s0={s0} dS_end={dse} decay={decay}")
    inp = make_inputs(B, H, L, D, D, dtype=dtype, decay=decay, s0_std=s0, nseg=nseg,
                      need_dO=True, dS_end_std=dse, seed=4000 + L + D + H, device="cuda")
    q, k, v, lam, S0, dO, dSe = (inp[x] for x in ("q", "k", "v", "lam", "S0", "dO", "dS_end"))
    got = la.la_decay_grad(q, k, v, lam, dO, S0=S0, dS_end=dSe, nseg=nseg, split=split)
    torch.cuda.synchronize()
    ref = lao.dlambda(f64(q), f64(k), f64(v), f64(lam), f64(dO), S0=f64(S0), dS_end=f64(dSe),
                      nseg=nseg)
    e = rel_err(f64(got), ref)
    log(f"  dlambda {f64(got)} ref {ref} err {e:.3e}")
    assert e <= TOL[dtype]


def test_decay_grad_is_deterministic_and_split_independent():
    B, H, L, D = 1, 4, 64 * 40 + 17, 128
    inp = make_inputs(B, H, L, D, D, s0_std=0.5, need_dO=True, dS_end_std=0.5, seed=41,
                      device="cuda")
    args = (inp["q"], inp["k"], inp["v"], inp["lam"], inp["dO"])
    kw = dict(S0=inp["S0"], dS_end=inp["dS_end"])
    a = la.la_decay_grad(*args, **kw)
    b = la.la_decay_grad(*args, **kw)
    c = la.la_decay_grad(*args, split=1, **kw)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    e = rel_err(f64(a), f64(c))
    log(f"  split auto vs 1: err {e:.3e}")
    assert e <= TOL["bf16"]


@pytest.mark.parametrize("dtype,D,split", [("bf16", 128, 1), ("bf16", 128, 2), ("fp32", 64, 2),
                                           ("bf16", 64, 3), ("fp32", 128, 1)])
def test_decay_grad_for_decays_on_both_sides_of_one_half(dtype, D, split):
    """Heads with lambda below 1/2 (the walk scales its pair every chunk), at
    1/2 and above (the pair is kept divided by a power of lambda and scaled
    back every few chunks, the period the shorter the faster the decay: one
    chunk at 1/2 and 0.6, three at 0.8, the whole walk at 0.97 and 1), over
    eleven chunks and a ragged tail: each head against the oracle on its own
    scale."""
    lam = torch.tensor([0.3, 0.5, 0.6, 0.8, 0.97, 1.0], dtype=torch.float32)
    B, H, L = 1, lam.numel(), 64 * 11 + 9
    log(f"decay grad across one half: dtype={dtype} D={D} split={split} lambda={lam.tolist()}")
    inp = make_inputs(B, H, L, D, D, dtype=dtype, s0_std=0.5, nseg=1, need_dO=True,
                      dS_end_std=0.5, seed=4400 + D + split, device="cuda", lam=lam)
    q, k, v, lam_d, S0, dO, dSe = (inp[x] for x in ("q", "k", "v", "lam", "S0", "dO", "dS_end"))
    got = f64(la.la_decay_grad(q, k, v, lam_d, dO, S0=S0, dS_end=dSe, split=split))
    torch.cuda.synchronize()
    ref = lao.dlambda(f64(q), f64(k), f64(v), f64(lam_d), f64(dO), S0=f64(S0), dS_end=f64(dSe))
    own = np.abs(got - ref) / np.abs(ref)
    log("  per head on its own scale: " + " ".join(f"{x:.1e}" for x in own))
    assert own.max() <= TOL[dtype]


@pytest.mark.parametrize("dtype,D,B,H,L,nseg,split,s0,dse,decay,seed", [
    ("bf16", 128, 2, 1, 2176, 1, 0, 0.5, 0.0, True, 10011),
    ("bf16", 128, 1, 1, 1372, 2, 2, 0.0, 0.0, False, 9085),
])
def test_decay_grad_of_a_single_head_whose_gradient_is_small(dtype, D, B, H, L, nseg, split, s0,
                                                             dse, decay, seed):
    """Two single-head cases whose gradient is small next to its terms (72.7
    and -6381): with the U update's weighted V as one bf16 rounding they came
    out 8.5 % and 2.6 % off; as hi + lo, like every decayed operand, within
    1e-4."""
    inp = make_inputs(B, H, L, D, D, dtype=dtype, decay=decay, s0_std=s0, nseg=nseg,
                      need_dO=True, dS_end_std=dse, seed=seed, device="cuda")
    q, k, v, lam, S0, dO, dSe = (inp[x] for x in ("q", "k", "v", "lam", "S0", "dO", "dS_end"))
    ref = lao.dlambda(f64(q), f64(k), f64(v), f64(lam), f64(dO), S0=f64(S0), dS_end=f64(dSe),
                      nseg=nseg)
    for sp in (split, 1):
        got = la.la_decay_grad(q, k, v, lam, dO, S0=S0, dS_end=dSe, nseg=nseg, split=sp)
        torch.cuda.synchronize()
        e = rel_err(f64(got), ref)
        log(f"  split {sp}: dlambda {f64(got)} ref {ref} err {e:.3e}")
        assert e <= 1e-3


def _random_lambda_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        out.append((i, "bf16" if i % 3 else "fp32", int(rng.choice([64, 128])),
                    int(rng.choice([1, 2])), int(rng.choice([1, 2])), int(rng.integers(50, 3000)),
                    int(rng.choice([1, 2])), int(rng.choice([0, 1, 2, 3])),
                    [float(x) for x in rng.uniform(0.3, 1.0, 2)],
                    float(rng.choice([0.0, 0.5])), float(rng.choice([0.0, 0.5]))))
    return out


@pytest.mark.parametrize("i,dtype,D,B,H,Ls,nseg,split,lams,s0,dse", _random_lambda_cases(16, 4242))
def test_decay_grad_at_random_lambda_every_head_on_its_own_scale(i, dtype, D, B, H, Ls, nseg, split,
                                                                 lams, s0, dse):
    """Seeded random configurations with one or two heads at lambda drawn
    from [0.3, 1] (the eager and the lazy walk, periods of every length):
    each head's gradient against the oracle on its own scale, where a small
    gradient next to its terms shows any rounding that adds up."""
    lam = torch.tensor(lams[:H], dtype=torch.float32)
    inp = make_inputs(B, H, Ls * nseg, D, D, dtype=dtype, s0_std=s0, nseg=nseg, need_dO=True,
                      dS_end_std=dse, seed=30000 + i, device="cuda", lam=lam)
    q, k, v, lm, S0, dO, dSe = (inp[x] for x in ("q", "k", "v", "lam", "S0", "dO", "dS_end"))
    got = f64(la.la_decay_grad(q, k, v, lm, dO, S0=S0, dS_end=dSe, nseg=nseg, split=split))
    torch.cuda.synchronize()
    ref = lao.dlambda(f64(q), f64(k), f64(v), f64(lm), f64(dO), S0=f64(S0), dS_end=f64(dSe),
                      nseg=nseg)
    own = np.abs(got - ref) / np.abs(ref)
    log(f"case {i} {dtype} D={D} B={B} H={H} L={Ls * nseg} nseg={nseg} split={split} "
        f"lambda={lam.tolist()}: own-scale err " + " ".join(f"{x:.1e}" for x in own))
    assert own.max() <= TOL[dtype]


@pytest.mark.parametrize("B,L", [(1, 0), (0, 128)])
def test_decay_grad_of_empty_problem_is_zero(B, L):
    H, D = 3, 64
    q = torch.zeros((B, H, L, D), dtype=torch.bfloat16, device="cuda")
    lam = torch.full((H,), 0.9, dtype=torch.float32, device="cuda")
    S0 = torch.randn((B, H, 1, D, D), device="cuda")
    dSe = torch.randn((B, H, 1, D, D), device="cuda")
    out = torch.full((H,), float("nan"), device="cuda")
    la.la_decay_grad(q, q, q, lam, q, S0=S0, dS_end=dSe, out=out)
    torch.cuda.synchronize()
    assert torch.equal(out, torch.zeros_like(out))


@pytest.mark.parametrize("name,dse", [("segment_64k", 0.02), ("train_256k", 0.0)])
def test_decay_grad_at_full_size_every_head(name, dse):
    """The workloads at full size in the launch configuration the benchmark
    times; the oracle computes every head's gradient (every token), and the
    measure is taken over the whole [H] vector, with each head's own error
    logged."""
    inp = workload_inputs(name, device="cuda", need_dO=True, dS_end_std=dse)
    q, k, v, lam, S0, dO, dSe = (inp[x] for x in ("q", "k", "v", "lam", "S0", "dO", "dS_end"))
    H = q.shape[1]
    log(f"decay grad full size: {name}, {H} heads")
    got = f64(la.la_decay_grad(q, k, v, lam, dO, S0=S0, dS_end=dSe))
    torch.cuda.synchronize()
    ref = np.empty(H)
    for h0 in range(0, H, 8):
        hs = slice(h0, min(H, h0 + 8))
        sl = lambda t: None if t is None else f64(t[:, hs])
        ref[hs] = lao.dlambda(sl(q), sl(k), sl(v), f64(lam[hs]), sl(dO), S0=sl(S0),
                              dS_end=sl(dSe))
    e = rel_err(got, ref)
    own = np.abs(got - ref) / np.abs(ref)
    log(f"  whole-vector err {e:.3e}; per head on its own scale: "
        + " ".join(f"h{h}={x:.1e}" for h, x in enumerate(own)))
    assert e <= TOL["bf16"]
    # every head on its own scale as well
    assert own.max() <= 1e-2
    del q, k, v, dO
