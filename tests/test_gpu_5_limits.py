"""The longest sequence the boundary accepts: one segment of 2^24 - 64 tokens
at d = 128 in bf16, i.e. 4 GiB - 16 KiB per tensor (one chunk more is
rejected, because byte offsets inside a sequence are 32-bit; the CPU tests
cover the rejection).  With lambda = 0.5 a row of O (or dQ) depends on its
last ~60 tokens to within 2^-60 of its size, and a row of dK, dV on its next
~60, so the oracle checks sampled rows exactly on 128-token windows: at the
start, on both sides of byte offset 2^31, at sub-segment boundaries of the
automatic split, just below 2^32 bytes and at the end.  Needs a gfx950 GPU
and about 30 GiB of device memory."""
import numpy as np
import pytest
import torch

from gpu_helpers import TOL, f64, log, rel_err, require_gpu
from long_sequence_causal_amd import linattn as la
from oracle import lao

pytestmark = pytest.mark.gpu

D = 128
L = (1 << 24) - 64
W = 128  # oracle window; lambda^W = 2^-128
LAM = 0.5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    torch.cuda.empty_cache()


def _draw(gen, scale):
    """[1, 1, L, D] bf16 Gaussian drawn in slices (no fp32 copy of it all)."""
    t = torch.empty((1, 1, L, D), dtype=torch.bfloat16, device="cuda")
    step = 1 << 20
    for a in range(0, L, step):
        b = min(L, a + step)
        t[0, 0, a:b] = (torch.randn((b - a, D), generator=gen, device="cuda") * scale).to(torch.bfloat16)
    return t


def _rows():
    """Sampled token positions (sorted, unique)."""
    chunks = L // 64
    cps = -(-chunks // 256)  # automatic split for one sequence: 256 sub-segments
    Lp = 64 * cps
    pos = {0, 1, 63, 64, 127, 128, 1000,
           (1 << 23) - 1, 1 << 23, (1 << 23) + 1,          # byte offset 2^31
           Lp - 1, Lp, 255 * Lp - 1, 255 * Lp,            # sub-segment boundaries
           (1 << 24) - (1 << 12), L - 65, L - 64, L - 2, L - 1}
    return sorted(p for p in pos if 0 <= p < L)


def _win(t, a, b):
    return f64(t[:, :, a:b])


def test_forward_at_the_largest_segment():
    log(f"limits fwd: L={L} d={D} lambda={LAM}")
    gen = torch.Generator(device="cuda").manual_seed(77)
    q = _draw(gen, D ** -0.5)
    k = _draw(gen, D ** -0.5)
    v = _draw(gen, 1.0)
    lam = torch.full((1,), LAM, dtype=torch.float32, device="cuda")
    O, S_end = la.la_chunk_fwd(q, k, v, lam)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(O).all()) and bool(torch.isfinite(S_end).all())
    lam64 = np.array([LAM])
    got, ref = [], []
    for t in _rows():
        a = max(0, t - W + 1)
        Ow, _ = lao.fwd(_win(q, a, t + 1), _win(k, a, t + 1), _win(v, a, t + 1), lam64)
        got.append(f64(O[0, 0, t]))
        ref.append(Ow[0, 0, -1])
    e = rel_err(np.array(got), np.array(ref))
    _, Sw = lao.fwd(_win(q, L - W, L), _win(k, L - W, L), _win(v, L - W, L), lam64, need_O=False)
    es = rel_err(f64(S_end), Sw)
    log(f"  sampled rows err {e:.3e}, S_end err {es:.3e}")
    assert e <= TOL["bf16"] and es <= TOL["bf16"]
    del q, k, v, O


def test_backward_at_the_largest_segment():
    log(f"limits bwd: L={L} d={D} lambda={LAM}")
    gen = torch.Generator(device="cuda").manual_seed(78)
    q = _draw(gen, D ** -0.5)
    k = _draw(gen, D ** -0.5)
    v = _draw(gen, 1.0)
    dO = _draw(gen, 1.0)
    lam = torch.full((1,), LAM, dtype=torch.float32, device="cuda")
    dQ, dK, dV, dS0 = la.la_chunk_bwd(q, k, v, lam, dO)
    torch.cuda.synchronize()
    for t_ in (dQ, dK, dV, dS0):
        assert bool(torch.isfinite(t_).all())
    lam64 = np.array([LAM])
    gq, rq, gk, rk, gv, rv = [], [], [], [], [], []
    for t in _rows():
        # dq_t from the past window, dk_t and dv_t from the future window
        a = max(0, t - W + 1)
        w = [_win(x, a, t + 1) for x in (q, k, v, dO)]
        rQ, _, _, _ = lao.bwd(w[0], w[1], w[2], lam64, w[3])
        gq.append(f64(dQ[0, 0, t]))
        rq.append(rQ[0, 0, -1])
        b = min(L, t + W)
        w = [_win(x, t, b) for x in (q, k, v, dO)]
        _, rK, rV, _ = lao.bwd(w[0], w[1], w[2], lam64, w[3])
        gk.append(f64(dK[0, 0, t]))
        rk.append(rK[0, 0, 0])
        gv.append(f64(dV[0, 0, t]))
        rv.append(rV[0, 0, 0])
    w = [_win(x, 0, W) for x in (q, k, v, dO)]
    _, _, _, rS0 = lao.bwd(w[0], w[1], w[2], lam64, w[3])
    errs = [rel_err(np.array(g), np.array(r)) for g, r in ((gq, rq), (gk, rk), (gv, rv))]
    errs.append(rel_err(f64(dS0), rS0))
    log("  sampled rows err dQ={:.3e} dK={:.3e} dV={:.3e}, dS0={:.3e}".format(*errs))
    assert max(errs) <= TOL["bf16"]
    del q, k, v, dO, dQ, dK, dV
