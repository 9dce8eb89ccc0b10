"""Pins of the CPU oracle against facts that do not come from the oracle.

Each test checks the token recurrence in ``oracle/lao.c`` against something
fixed independently of it: a hand-worked example, a closed form evaluated with
numpy's matmul / cumsum, brute-force finite differences, exact invariants of
the mathematics (segment composition, streaming resume, Euler's identity for
homogeneous functions) or degenerate inputs.  All of this runs on the CPU.
"""
import json
import os

import numpy as np
import pytest

from oracle import lao

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.max(np.abs(b))
    return float(np.max(np.abs(a - b)) / (den if den > 0 else 1.0))


def quadratic_form(Q, K, V, lam, S0):
    """Closed form for one (b, h) sequence, 1-indexed tokens t, s:
         O = ((Q K^T) * D) V + diag(lam^t) Q S0,  D[t, s] = lam^(t-s) [s <= t]
         S_end = lam^L S0 + K^T diag(lam^(L-s)) V
    written with numpy matmul, independently of the recurrence."""
    L = Q.shape[0]
    t = np.arange(1, L + 1, dtype=np.float64)
    diff = t[:, None] - t[None, :]
    D = np.where(diff >= 0, lam ** np.maximum(diff, 0), 0.0)
    O = ((Q @ K.T) * D) @ V
    if S0 is not None:
        O = O + (lam ** t)[:, None] * (Q @ S0)
    w = lam ** (L - t)
    S_end = K.T @ (w[:, None] * V)
    if S0 is not None:
        S_end = S_end + lam ** L * S0
    return O, S_end


# --------------------------------------------------------------------------
# hand-worked examples


def test_hand_example_forward():
    g = json.load(open(os.path.join(GOLDEN, "hand_dk2_dv3.json")))
    Q = np.array(g["q"], float)[None, None]
    K = np.array(g["k"], float)[None, None]
    V = np.array(g["v"], float)[None, None]
    S0 = np.array(g["S0"], float)[None, None, None]
    O, S_end = lao.fwd(Q, K, V, np.array([g["lam"]]), S0=S0)
    # every value in the example is a dyadic rational: exact equality
    np.testing.assert_array_equal(O[0, 0], np.array(g["O"], float))
    np.testing.assert_array_equal(S_end[0, 0, 0], np.array(g["S_end"], float))


def test_hand_example_rows():
    g = json.load(open(os.path.join(GOLDEN, "hand_dk2_dv3.json")))
    Q = np.array(g["q"], float)[None, None]
    K = np.array(g["k"], float)[None, None]
    V = np.array(g["v"], float)[None, None]
    S0 = np.array(g["S0"], float)[None, None, None]
    rows = lao.fwd_rows(Q, K, V, np.array([g["lam"]]), [0, 0, 0], [0, 1, 2], S0=S0)
    np.testing.assert_array_equal(rows, np.array(g["O"], float))


def test_hand_example_scan():
    g = json.load(open(os.path.join(GOLDEN, "hand_scan.json")))
    dS = np.array(g["dS"], float).reshape(1, 1, 3, 1, 1)
    S0 = np.array([[[[g["S0"]]]]])
    for key, rev in (("forward", False), ("reverse", True)):
        st, en = lao.scan(dS, np.array([g["lam"]]), g["seg_len"], S0=S0, reverse=rev)
        np.testing.assert_array_equal(st.reshape(-1), np.array(g[key]["S_start"]))
        assert en.reshape(-1)[0] == g[key]["S_end"]


# --------------------------------------------------------------------------
# closed forms


@pytest.mark.parametrize("L,dk,dv", [(1, 4, 4), (77, 16, 24), (300, 64, 64), (512, 16, 16)])
def test_recurrence_equals_quadratic_form(L, dk, dv):
    rng = np.random.default_rng(100 + L)
    B, H = 2, 3
    Q = _rand(rng, B, H, L, dk) / np.sqrt(dk)
    K = _rand(rng, B, H, L, dk) / np.sqrt(dk)
    V = _rand(rng, B, H, L, dv)
    S0 = _rand(rng, B, H, 1, dk, dv)
    lam = rng.uniform(0.5, 1.0, H)
    lam[0] = 1.0
    O, S_end = lao.fwd(Q, K, V, lam, S0=S0)
    for b in range(B):
        for h in range(H):
            Oq, Sq = quadratic_form(Q[b, h], K[b, h], V[b, h], lam[h], S0[b, h, 0])
            assert _rel(O[b, h], Oq) < 1e-12
            assert _rel(S_end[b, h, 0], Sq) < 1e-12


def test_lambda_one_cumsum_closed_form():
    """lambda = 1: S_t = S0 + cumsum_s k_s v_s^T, O = tril(QK^T) V + Q S0."""
    rng = np.random.default_rng(7)
    L, dk, dv = 256, 8, 12
    Q = _rand(rng, 1, 1, L, dk)
    K = _rand(rng, 1, 1, L, dk)
    V = _rand(rng, 1, 1, L, dv)
    S0 = _rand(rng, 1, 1, 1, dk, dv)
    O, S_end = lao.fwd(Q, K, V, np.array([1.0]), S0=S0)
    outer = np.einsum("ti,tj->tij", K[0, 0], V[0, 0])
    S_t = S0[0, 0, 0][None] + np.cumsum(outer, axis=0)
    O_ref = np.einsum("ti,tij->tj", Q[0, 0], S_t)
    assert _rel(O[0, 0], O_ref) < 1e-12
    assert _rel(S_end[0, 0, 0], S_t[-1]) < 1e-12
    O_ref2 = np.tril(Q[0, 0] @ K[0, 0].T) @ V[0, 0] + Q[0, 0] @ S0[0, 0, 0]
    assert _rel(O[0, 0], O_ref2) < 1e-12


def test_lambda_one_workload_shape_closed_form():
    """The undecayed fp32 workload's shape (H=2, L=1024, d=64) at lambda = 1."""
    rng = np.random.default_rng(11)
    L, d = 1024, 64
    Q = _rand(rng, 1, 2, L, d) / 8
    K = _rand(rng, 1, 2, L, d) / 8
    V = _rand(rng, 1, 2, L, d)
    O, S_end = lao.fwd(Q, K, V, np.ones(2))
    for h in range(2):
        assert _rel(O[0, h], np.tril(Q[0, h] @ K[0, h].T) @ V[0, h]) < 1e-12
        assert _rel(S_end[0, h, 0], K[0, h].T @ V[0, h]) < 1e-12


def test_state_end_closed_form_long():
    """S_end = lam^L S0 + K^T diag(lam^(L-s)) V at a longer length."""
    rng = np.random.default_rng(5)
    L, d = 8192, 32
    lam = np.array([0.999, 0.97])
    Q = _rand(rng, 1, 2, L, d)
    K = _rand(rng, 1, 2, L, d) / np.sqrt(d)
    V = _rand(rng, 1, 2, L, d)
    S0 = _rand(rng, 1, 2, 1, d, d)
    _, S_end = lao.fwd(Q, K, V, lam, S0=S0, need_O=False)
    t = np.arange(1, L + 1)
    for h in range(2):
        w = lam[h] ** (L - t)
        ref = lam[h] ** L * S0[0, h, 0] + K[0, h].T @ (w[:, None] * V[0, h])
        assert _rel(S_end[0, h, 0], ref) < 1e-11


def test_rows_equal_recurrence():
    rng = np.random.default_rng(9)
    B, H, L, d = 1, 2, 200, 16
    Q, K, V = (_rand(rng, B, H, L, d) for _ in range(3))
    S0 = _rand(rng, B, H, 2, d, d)
    lam = np.array([0.9, 1.0])
    O, _ = lao.fwd(Q, K, V, lam, S0=S0, nseg=2)
    seq = np.array([0, 1, 2, 3, 3, 1])
    rows = np.array([0, 99, 50, 0, 99, 63])
    R = lao.fwd_rows(Q, K, V, lam, seq, rows, S0=S0, nseg=2)
    Of = O.reshape(B * H * 2, L // 2, d)
    assert _rel(R, Of[seq, rows]) < 1e-12


# --------------------------------------------------------------------------
# invariants


def test_segments_with_scanned_starts_equal_monolithic():
    """Local states from zero, scanned, then used as initial states of each
    segment, reproduce the monolithic run (ZeCO / LASP-2 abstracts)."""
    rng = np.random.default_rng(3)
    B, H, L, d, P = 1, 3, 768, 16, 6
    Q, K = (_rand(rng, B, H, L, d) / 4 for _ in range(2))
    V = _rand(rng, B, H, L, d)
    S0 = _rand(rng, B, H, 1, d, d)
    lam = np.array([0.95, 0.999, 1.0])
    O_mono, S_mono = lao.fwd(Q, K, V, lam, S0=S0)
    _, dS = lao.fwd(Q, K, V, lam, S0=None, nseg=P, need_O=False)
    S_start, S_end = lao.scan(dS, lam, L // P, S0=S0[:, :, 0])
    O_seg, S_seg_end = lao.fwd(Q, K, V, lam, S0=S_start, nseg=P)
    assert _rel(O_seg, O_mono) < 1e-12
    assert _rel(S_end, S_mono[:, :, 0]) < 1e-12
    # the end state of segment s is the start state of segment s + 1
    assert _rel(S_seg_end[:, :, :-1], S_start[:, :, 1:]) < 1e-12
    assert _rel(S_seg_end[:, :, -1], S_mono[:, :, 0]) < 1e-12


def test_scan_special_cases():
    rng = np.random.default_rng(4)
    B, H, P, d = 2, 2, 9, 5
    dS = _rand(rng, B, H, P, d, d)
    S0 = _rand(rng, B, H, d, d)
    # lambda^seg_len = 1: prefix sums
    st, en = lao.scan(dS, np.ones(H), 100, S0=S0)
    cs = np.cumsum(dS, axis=2)
    assert _rel(st[:, :, 1:], S0[:, :, None] + cs[:, :, :-1]) < 1e-13
    assert _rel(en, S0 + cs[:, :, -1]) < 1e-13
    # lambda = 0: every start is the previous local state
    st, en = lao.scan(dS, np.zeros(H), 4, S0=S0)
    np.testing.assert_array_equal(st[:, :, 1:], dS[:, :, :-1])
    np.testing.assert_array_equal(st[:, :, 0], S0)
    np.testing.assert_array_equal(en, dS[:, :, -1])
    # reverse scan = forward scan of the reversed segment order
    lam = np.array([0.9, 0.5])
    st_r, en_r = lao.scan(dS, lam, 3, S0=S0, reverse=True)
    st_f, en_f = lao.scan(dS[:, :, ::-1], lam, 3, S0=S0)
    np.testing.assert_array_equal(st_r, st_f[:, :, ::-1])
    np.testing.assert_array_equal(en_r, en_f)


def test_streaming_resume():
    """Running [1..L1] and then [L1+1..L] from the first part's end state
    equals one run (constant-memory inference, LASP-2 abstract)."""
    rng = np.random.default_rng(6)
    B, H, L, d, L1 = 1, 2, 500, 8, 173
    Q, K, V = (_rand(rng, B, H, L, d) for _ in range(3))
    S0 = _rand(rng, B, H, 1, d, d)
    lam = np.array([0.98, 0.7])
    O, S_end = lao.fwd(Q, K, V, lam, S0=S0)
    O1, S1 = lao.fwd(Q[:, :, :L1], K[:, :, :L1], V[:, :, :L1], lam, S0=S0)
    O2, S2 = lao.fwd(Q[:, :, L1:], K[:, :, L1:], V[:, :, L1:], lam, S0=S1)
    np.testing.assert_allclose(np.concatenate([O1, O2], axis=2), O, rtol=0, atol=1e-12)
    np.testing.assert_allclose(S2, S_end, rtol=0, atol=1e-12)


def test_degenerate_inputs():
    rng = np.random.default_rng(8)
    B, H, L, d = 1, 2, 64, 8
    Q = _rand(rng, B, H, L, d)
    S0 = _rand(rng, B, H, 1, d, d)
    lam = np.array([0.9, 0.6])
    t = np.arange(1, L + 1)
    # K = 0: only the decayed initial state is seen
    Z = np.zeros((B, H, L, d))
    O, S_end = lao.fwd(Q, Z, _rand(rng, B, H, L, d), lam, S0=S0)
    for h in range(H):
        ref = (lam[h] ** t)[:, None] * (Q[0, h] @ S0[0, h, 0])
        assert _rel(O[0, h], ref) < 1e-13
        assert _rel(S_end[0, h, 0], lam[h] ** L * S0[0, h, 0]) < 1e-13
    # L = 1
    K1, V1 = _rand(rng, B, H, 1, d), _rand(rng, B, H, 1, d)
    O, S_end = lao.fwd(Q[:, :, :1], K1, V1, lam, S0=S0)
    for h in range(H):
        S1 = lam[h] * S0[0, h, 0] + np.outer(K1[0, h, 0], V1[0, h, 0])
        assert _rel(S_end[0, h, 0], S1) < 1e-14
        assert _rel(O[0, h, 0], Q[0, h, 0] @ S1) < 1e-14
    # lambda -> 0: o_t = (q_t . k_t) v_t, S_end = k_L v_L^T
    K, V = _rand(rng, B, H, L, d), _rand(rng, B, H, L, d)
    O, S_end = lao.fwd(Q, K, V, np.array([1e-30, 1e-30]), S0=S0)
    ref = np.sum(Q * K, axis=-1, keepdims=True) * V
    assert _rel(O, ref) < 1e-13  # previous tokens weigh 1e-30: only rounding remains
    assert _rel(S_end[0, 0, 0], np.outer(K[0, 0, -1], V[0, 0, -1])) < 1e-13
    # L = 0 is an empty sequence: the end state is the initial state
    E = np.zeros((B, H, 0, d))
    O, S_end = lao.fwd(E, E, E, lam, S0=S0)
    assert O.shape == (B, H, 0, d)
    np.testing.assert_array_equal(S_end, S0)


# --------------------------------------------------------------------------
# backward


def _loss(Q, K, V, lam, S0, dO, dS_end):
    O, S_end = lao.fwd(Q, K, V, lam, S0=S0)
    return float(np.sum(O * dO) + np.sum(S_end * dS_end))


def test_backward_finite_differences():
    """Directional derivatives of <dO, O> + <dS_end, S_end> by central
    differences agree with the oracle backward (the loss is quadratic in the
    inputs, so the central difference is exact up to rounding)."""
    rng = np.random.default_rng(12)
    B, H, L, d = 1, 2, 40, 6
    Q, K, V, dO = (_rand(rng, B, H, L, d) for _ in range(4))
    S0, dS_end = _rand(rng, B, H, 1, d, d), _rand(rng, B, H, 1, d, d)
    lam = np.array([0.9, 0.99])
    dQ, dK, dV, dS0 = lao.bwd(Q, K, V, lam, dO, S0=S0, dS_end=dS_end)
    eps = 1e-3
    for name, X, G in (("Q", Q, dQ), ("K", K, dK), ("V", V, dV), ("S0", S0, dS0)):
        for trial in range(3):
            Dir = _rand(rng, *X.shape)
            args = dict(Q=Q, K=K, V=V, S0=S0)
            args[name] = X + eps * Dir
            lp = _loss(args["Q"], args["K"], args["V"], lam, args["S0"], dO, dS_end)
            args[name] = X - eps * Dir
            lm = _loss(args["Q"], args["K"], args["V"], lam, args["S0"], dO, dS_end)
            fd = (lp - lm) / (2 * eps)
            an = float(np.sum(G * Dir))
            assert abs(fd - an) <= 1e-8 * max(1.0, abs(an)), (name, fd, an)


def test_backward_closed_forms():
    """dQ = ((dO V^T) * D) K + diag(lam^t) dO S0^T
       dK = ((dO V^T) * D)^T Q + diag(lam^(L-s)) V dS_end^T
       dV = ((Q K^T) * D)^T dO + diag(lam^(L-s)) K dS_end
       dS0 = Q^T diag(lam^t) dO + lam^L dS_end"""
    rng = np.random.default_rng(13)
    B, H, L, dk, dv = 1, 2, 150, 12, 20
    Q, K = (_rand(rng, B, H, L, dk) for _ in range(2))
    V, dO = (_rand(rng, B, H, L, dv) for _ in range(2))
    S0, dS_end = _rand(rng, B, H, 1, dk, dv), _rand(rng, B, H, 1, dk, dv)
    lam = np.array([0.93, 1.0])
    dQ, dK, dV, dS0 = lao.bwd(Q, K, V, lam, dO, S0=S0, dS_end=dS_end)
    t = np.arange(1, L + 1, dtype=float)
    for h in range(H):
        l = lam[h]
        diff = t[:, None] - t[None, :]
        D = np.where(diff >= 0, l ** np.maximum(diff, 0), 0.0)
        q, k, v, g = Q[0, h], K[0, h], V[0, h], dO[0, h]
        s0, de = S0[0, h, 0], dS_end[0, h, 0]
        wt, wr = l ** t, l ** (L - t)
        assert _rel(dQ[0, h], ((g @ v.T) * D) @ k + wt[:, None] * (g @ s0.T)) < 1e-12
        assert _rel(dK[0, h], ((g @ v.T) * D).T @ q + wr[:, None] * (v @ de.T)) < 1e-12
        assert _rel(dV[0, h], ((q @ k.T) * D).T @ g + wr[:, None] * (k @ de)) < 1e-12
        assert _rel(dS0[0, h, 0], q.T @ (wt[:, None] * g) + l ** L * de) < 1e-12


def test_backward_matches_torch_autograd_on_quadratic_form():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(14)
    L, d = 70, 8
    lam = 0.95
    arrs = [_rand(rng, L, d) for _ in range(4)] + [_rand(rng, d, d), _rand(rng, d, d)]
    Q, K, V, dO, S0, dSe = arrs
    tq, tk, tv, ts = (torch.tensor(a, dtype=torch.float64, requires_grad=True)
                      for a in (Q, K, V, S0))
    t = torch.arange(1, L + 1, dtype=torch.float64)
    diff = t[:, None] - t[None, :]
    D = torch.where(diff >= 0, lam ** diff.clamp(min=0), torch.zeros_like(diff))
    O = ((tq @ tk.T) * D) @ tv + (lam ** t)[:, None] * (tq @ ts)
    Se = tk.T @ ((lam ** (L - t))[:, None] * tv) + lam ** L * ts
    loss = (O * torch.tensor(dO)).sum() + (Se * torch.tensor(dSe)).sum()
    loss.backward()
    dQ, dK, dV, dS0 = lao.bwd(Q[None, None], K[None, None], V[None, None], np.array([lam]),
                              dO[None, None], S0=S0[None, None, None],
                              dS_end=dSe[None, None, None])
    assert _rel(dQ[0, 0], tq.grad.numpy()) < 1e-12
    assert _rel(dK[0, 0], tk.grad.numpy()) < 1e-12
    assert _rel(dV[0, 0], tv.grad.numpy()) < 1e-12
    assert _rel(dS0[0, 0, 0], ts.grad.numpy()) < 1e-12


def test_backward_euler_identities():
    """l = <dO,O> + <dS_end,S_end> is linear in Q and jointly linear in
    (K, S0) and in (V, S0), so <dQ,Q> = <dO,O>, <dK,K> + <dS0,S0> = l and
    <dV,V> + <dS0,S0> = l."""
    rng = np.random.default_rng(15)
    B, H, L, d = 2, 2, 128, 8
    Q, K, V, dO = (_rand(rng, B, H, L, d) for _ in range(4))
    S0, dS_end = _rand(rng, B, H, 2, d, d), _rand(rng, B, H, 2, d, d)
    lam = np.array([0.97, 0.8])
    O, S_end = lao.fwd(Q, K, V, lam, S0=S0, nseg=2)
    dQ, dK, dV, dS0 = lao.bwd(Q, K, V, lam, dO, S0=S0, dS_end=dS_end, nseg=2)
    l_o = np.sum(dO * O)
    l = l_o + np.sum(dS_end * S_end)
    assert abs(np.sum(dQ * Q) - l_o) < 1e-10 * np.sum(np.abs(dQ * Q))
    assert abs(np.sum(dK * K) + np.sum(dS0 * S0) - l) < 1e-10 * (np.sum(np.abs(dK * K)) + np.sum(np.abs(dS0 * S0)))
    assert abs(np.sum(dV * V) + np.sum(dS0 * S0) - l) < 1e-10 * (np.sum(np.abs(dV * V)) + np.sum(np.abs(dS0 * S0)))


def test_backward_zero_state_inputs():
    """With S0 and dS_end absent (zero) the closed forms lose their state terms."""
    rng = np.random.default_rng(16)
    L, d = 96, 8
    Q, K, V, dO = (_rand(rng, 1, 1, L, d) for _ in range(4))
    lam = np.array([0.9])
    dQ, dK, dV, dS0 = lao.bwd(Q, K, V, lam, dO)
    t = np.arange(1, L + 1, dtype=float)
    diff = t[:, None] - t[None, :]
    D = np.where(diff >= 0, 0.9 ** np.maximum(diff, 0), 0.0)
    q, k, v, g = Q[0, 0], K[0, 0], V[0, 0], dO[0, 0]
    assert _rel(dQ[0, 0], ((g @ v.T) * D) @ k) < 1e-12
    assert _rel(dK[0, 0], ((g @ v.T) * D).T @ q) < 1e-12
    assert _rel(dV[0, 0], ((q @ k.T) * D).T @ g) < 1e-12
    assert _rel(dS0[0, 0, 0], q.T @ ((0.9 ** t)[:, None] * g)) < 1e-12


# --------------------------------------------------------------------------
# gated recurrence: S_t = alpha_t S_{t-1} + k_t v_t^T with a per-token gate


def gated_quadratic_form(Q, K, V, G, S0):
    """O and S_end of the gated recurrence in closed form (numpy matmul and
    cumsum): with c_t = sum_{u<=t} g_u,
      O = ((Q K^T) * D) V + diag(exp(c)) Q S0,   D_ts = exp(c_t - c_s) [s <= t]
      S_end = exp(c_L) S0 + K^T diag(exp(c_L - c)) V."""
    L = Q.shape[0]
    c = np.cumsum(G)
    Dm = np.tril(np.exp(c[:, None] - c[None, :]))
    O = ((Q @ K.T) * Dm) @ V
    S_end = np.zeros((K.shape[1], V.shape[1]))
    if S0 is not None:
        O = O + np.exp(c)[:, None] * (Q @ S0)
        S_end = np.exp(c[-1]) * S0
    S_end = S_end + K.T @ (np.exp(c[-1] - c)[:, None] * V) if L else S_end
    return O, S_end


def test_gated_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "hand_gated.json")))
    Q = np.array(g["q"], float)[None, None]
    K = np.array(g["k"], float)[None, None]
    V = np.array(g["v"], float)[None, None]
    S0 = np.array(g["S0"], float)[None, None, None]
    G = np.log(np.array(g["alpha"], float))[None, None]
    O, S_end = lao.fwd_gated(Q, K, V, G, S0=S0)
    # exp(log(alpha)) may differ from alpha in the last bit
    np.testing.assert_allclose(O[0, 0], np.array(g["O"], float), rtol=0, atol=1e-14)
    np.testing.assert_allclose(S_end[0, 0, 0], np.array(g["S_end"], float), rtol=0, atol=1e-14)


def test_gated_hand_example_scan():
    g = json.load(open(os.path.join(GOLDEN, "hand_gated.json")))["scan"]
    dS = np.array(g["dS"], float).reshape(1, 1, 3, 1, 1)
    LD = np.log(np.array(g["decay"], float)).reshape(1, 1, 3)
    S0 = np.array([[[[g["S0"]]]]], float)
    for key, rev in (("forward", False), ("reverse", True)):
        st, en = lao.scan_gated(dS, LD, S0=S0, reverse=rev)
        np.testing.assert_allclose(st.reshape(-1), np.array(g[key]["S_start"]), rtol=0, atol=1e-14)
        assert abs(en.reshape(-1)[0] - g[key]["S_end"]) <= 1e-14


@pytest.mark.parametrize("L,dk,dv", [(1, 4, 4), (77, 16, 24), (300, 64, 64)])
def test_gated_recurrence_equals_quadratic_form(L, dk, dv):
    rng = np.random.default_rng(100 + L)
    Q, K, V = _rand(rng, 1, 2, L, dk), _rand(rng, 1, 2, L, dk), _rand(rng, 1, 2, L, dv)
    G = -rng.uniform(0.0, 0.2, size=(1, 2, L))
    S0 = _rand(rng, 1, 2, 1, dk, dv)
    O, S_end = lao.fwd_gated(Q, K, V, G, S0=S0)
    for h in range(2):
        Or, Sr = gated_quadratic_form(Q[0, h], K[0, h], V[0, h], G[0, h], S0[0, h, 0])
        assert _rel(O[0, h], Or) < 1e-12
        assert _rel(S_end[0, h, 0], Sr) < 1e-12


def test_gated_unit_gate_is_a_cumulative_sum():
    rng = np.random.default_rng(7)
    L, dk, dv = 200, 8, 5
    Q, K, V = _rand(rng, 1, 1, L, dk), _rand(rng, 1, 1, L, dk), _rand(rng, 1, 1, L, dv)
    S0 = _rand(rng, 1, 1, 1, dk, dv)
    O, S_end = lao.fwd_gated(Q, K, V, np.zeros((1, 1, L)), S0=S0)
    S = S0[0, 0, 0] + np.cumsum(K[0, 0][:, :, None] * V[0, 0][:, None, :], axis=0)
    assert _rel(O[0, 0], np.einsum("tk,tkv->tv", Q[0, 0], S)) < 1e-12
    assert _rel(S_end[0, 0, 0], S[-1]) < 1e-12


def test_gated_constant_gate_is_the_fixed_decay():
    rng = np.random.default_rng(8)
    L, dk, dv, H = 150, 16, 16, 3
    Q, K, V = _rand(rng, 1, H, L, dk), _rand(rng, 1, H, L, dk), _rand(rng, 1, H, L, dv)
    lam = np.array([0.5, 0.9, 0.999])
    G = np.broadcast_to(np.log(lam)[None, :, None], (1, H, L)).copy()
    S0 = _rand(rng, 1, H, 1, dk, dv)
    O, S = lao.fwd_gated(Q, K, V, G, S0=S0)
    Or, Sr = quadratic_form(Q[0, 0], K[0, 0], V[0, 0], lam[0], S0[0, 0, 0])
    assert _rel(O[0, 0], Or) < 1e-12 and _rel(S[0, 0, 0], Sr) < 1e-12


def test_gated_segments_with_scanned_starts_equal_monolithic():
    rng = np.random.default_rng(9)
    P, Ls, dk, dv = 5, 40, 8, 6
    L = P * Ls
    Q, K, V = _rand(rng, 1, 2, L, dk), _rand(rng, 1, 2, L, dk), _rand(rng, 1, 2, L, dv)
    G = -rng.uniform(0.0, 0.1, size=(1, 2, L))
    S0 = _rand(rng, 1, 2, 1, dk, dv)
    O_ref, S_ref = lao.fwd_gated(Q, K, V, G, S0=S0)
    # local states of each segment from zero, combined with the product of
    # the gates over each segment
    _, dS = lao.fwd_gated(Q, K, V, G, nseg=P, need_O=False)
    LD = G.reshape(1, 2, P, Ls).sum(axis=-1)
    S_start, S_end = lao.scan_gated(dS, LD, S0=S0[:, :, 0])
    O, _ = lao.fwd_gated(Q, K, V, G, S0=S_start, nseg=P)
    assert _rel(O, O_ref) < 1e-12
    assert _rel(S_end, S_ref[:, :, 0]) < 1e-12


def _gated_loss(Q, K, V, G, dO, S0, dS_end, nseg=1):
    O, S = lao.fwd_gated(Q, K, V, G, S0=S0, nseg=nseg)
    return float((O * dO).sum() + (S * dS_end).sum())


@pytest.mark.parametrize("L", [1, 63, 64, 65, 150])
def test_gated_backward_finite_differences(L):
    rng = np.random.default_rng(200 + L)
    B, H, dk, dv = 1, 1, 8, 6
    Q, K, V, dO = (_rand(rng, B, H, L, d) for d in (dk, dk, dv, dv))
    G = -rng.uniform(0.0, 0.3, size=(B, H, L))
    S0, dSe = _rand(rng, B, H, 1, dk, dv), _rand(rng, B, H, 1, dk, dv)
    dQ, dK, dV, dS0, dG = lao.bwd_gated(Q, K, V, G, dO, S0=S0, dS_end=dSe)
    f = lambda **kw: _gated_loss(*(kw.get(n, x) for n, x in
                                   (("Q", Q), ("K", K), ("V", V), ("G", G), ("dO", dO),
                                    ("S0", S0), ("dS_end", dSe))))
    eps = 1e-6
    for t in sorted({0, L // 2, L - 1}):
        e = np.zeros_like(G)
        e[0, 0, t] = eps
        fd = (f(G=G + e) - f(G=G - e)) / (2 * eps)
        assert abs(dG[0, 0, t] - fd) <= 1e-6 * max(1.0, abs(fd))
        for name, X, dX in (("Q", Q, dQ), ("K", K, dK), ("V", V, dV)):
            e = np.zeros_like(X)
            e[0, 0, t, 1] = eps
            fd = (f(**{name: X + e}) - f(**{name: X - e})) / (2 * eps)
            assert abs(dX[0, 0, t, 1] - fd) <= 1e-6 * max(1.0, abs(fd))
    e = np.zeros_like(S0)
    e[0, 0, 0, 2, 3] = eps
    fd = (f(S0=S0 + e) - f(S0=S0 - e)) / (2 * eps)
    assert abs(dS0[0, 0, 0, 2, 3] - fd) <= 1e-6 * max(1.0, abs(fd))


def test_gated_backward_constant_gate_is_the_fixed_decay():
    rng = np.random.default_rng(210)
    B, H, L, dk, dv = 1, 2, 130, 16, 8
    Q, K, V, dO = (_rand(rng, B, H, L, d) for d in (dk, dk, dv, dv))
    lam = np.array([0.7, 0.99])
    G = np.broadcast_to(np.log(lam)[None, :, None], (B, H, L)).copy()
    S0, dSe = _rand(rng, B, H, 1, dk, dv), _rand(rng, B, H, 1, dk, dv)
    gated = lao.bwd_gated(Q, K, V, G, dO, S0=S0, dS_end=dSe)
    fixed = lao.bwd(Q, K, V, lam, dO, S0=S0, dS_end=dSe)
    for a, b in zip(gated[:4], fixed):
        assert _rel(a, b) < 1e-12


def test_gated_log_gate_gradient_identity():
    """g_t enters only through the cumulative log-gates, which multiply q_u
    by exp(c_u) and k_u by exp(-c_u) (u >= t) and S_end by exp(c_L), so
        dg_t = sum_{u >= t} (q_u . dq_u - k_u . dk_u) + <dS_end, S_end>
    within each segment; checked on segments of uneven content."""
    rng = np.random.default_rng(211)
    B, H, nseg, Ls, dk, dv = 1, 2, 3, 70, 8, 8
    L = nseg * Ls
    Q, K, V, dO = (_rand(rng, B, H, L, d) for d in (dk, dk, dv, dv))
    G = -rng.uniform(0.0, 0.5, size=(B, H, L))
    S0, dSe = _rand(rng, B, H, nseg, dk, dv), _rand(rng, B, H, nseg, dk, dv)
    dQ, dK, dV, dS0, dG = lao.bwd_gated(Q, K, V, G, dO, S0=S0, dS_end=dSe, nseg=nseg)
    _, S_end = lao.fwd_gated(Q, K, V, G, S0=S0, nseg=nseg, need_O=False)
    r = (Q * dQ).sum(-1) - (K * dK).sum(-1)
    for s in range(nseg):
        sl = slice(s * Ls, (s + 1) * Ls)
        tail = np.flip(np.cumsum(np.flip(r[..., sl], -1), -1), -1)
        ref = tail + (dSe[:, :, s] * S_end[:, :, s]).sum((-1, -2))[..., None]
        assert _rel(dG[..., sl], ref) < 1e-11


def test_decay_gradient_finite_differences():
    rng = np.random.default_rng(220)
    B, H, nseg, L, dk, dv = 2, 2, 2, 2 * 75, 8, 6
    Q, K, V, dO = (_rand(rng, B, H, L, d) for d in (dk, dk, dv, dv))
    lam = np.array([0.8, 0.97])
    S0, dSe = _rand(rng, B, H, nseg, dk, dv), _rand(rng, B, H, nseg, dk, dv)

    def loss(l):
        O, S = lao.fwd(Q, K, V, l, S0=S0, nseg=nseg)
        return float((O * dO).sum() + (S * dSe).sum())

    dl = lao.dlambda(Q, K, V, lam, dO, S0=S0, dS_end=dSe, nseg=nseg)
    for h in range(H):
        e = np.zeros(H)
        e[h] = 1e-7
        fd = (loss(lam + e) - loss(lam - e)) / 2e-7
        assert abs(dl[h] - fd) <= 1e-5 * max(1.0, abs(fd))


def test_step_closed_form_on_a_tiny_case():
    # dk = dv = 1: s' = lambda s + k v, o = q s'
    o, S1 = lao.step(np.array([[[2.0]]]), np.array([[[3.0]]]), np.array([[[5.0]]]),
                     np.array([0.5]), np.array([[[[4.0]]]]))
    assert S1[0, 0, 0, 0] == 0.5 * 4.0 + 3.0 * 5.0
    assert o[0, 0, 0] == 2.0 * 17.0
    # zero state: S' = k v^T exactly
    rng = np.random.default_rng(230)
    q, k = rng.standard_normal((1, 1, 3)), rng.standard_normal((1, 1, 3))
    v = rng.standard_normal((1, 1, 2))
    o, S1 = lao.step(q, k, v, np.array([0.9]))
    assert np.array_equal(S1[0, 0], np.outer(k[0, 0], v[0, 0]))


def test_a_chain_of_steps_is_the_forward_pass():
    # L steps from S0 reproduce the pinned C forward over the same L tokens
    rng = np.random.default_rng(231)
    B, H, L, dk, dv = 2, 3, 37, 5, 4
    Q, K, V = (_rand(rng, B, H, L, d) for d in (dk, dk, dv))
    S0 = _rand(rng, B, H, 1, dk, dv)
    lam = np.array([0.7, 0.95, 1.0])
    O, S_end = lao.fwd(Q, K, V, lam, S0=S0)
    S = S0[:, :, 0]
    for t in range(L):
        o, S = lao.step(Q[:, :, t], K[:, :, t], V[:, :, t], lam, S)
        assert _rel(o, O[:, :, t]) < 1e-13
    assert _rel(S, S_end[:, :, 0]) < 1e-13
