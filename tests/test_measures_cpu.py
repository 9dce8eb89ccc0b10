"""The test measures themselves (CPU): the log-gate gradient's measure of a
sum of cancelling terms, against a direct loop over tokens."""
import numpy as np

from gpu_helpers import gate_grad_err


def _scale_by_loop(q, k, dq, dk, nseg):
    B, H, L, _ = q.shape
    Ls = L // nseg
    a = np.abs(np.einsum("bhld,bhld->bhl", q, dq)) + np.abs(np.einsum("bhld,bhld->bhl", k, dk))
    T = 0.0
    for b in range(B):
        for h in range(H):
            for s in range(nseg):
                for t in range(Ls):
                    end = min(Ls, (t // 1024 + 1) * 1024)  # t's 1024-token block ends here
                    T = max(T, float(a[b, h, s * Ls + t:s * Ls + end].sum()))
    return T


def test_gate_grad_err_takes_the_larger_of_the_value_and_a_tenth_of_the_term_scale():
    rng = np.random.default_rng(5)
    B, H, L, D, nseg = 1, 2, 2 * 1100, 4, 2  # two segments of 1100 tokens: blocks of 1024 and 76
    q, k, dq, dk = (rng.standard_normal((B, H, L, D)) for _ in range(4))
    T = _scale_by_loop(q, k, dq, dk, nseg)
    ref = rng.standard_normal((B, H, L))
    got = ref.copy()
    got[0, 1, 7] += 0.5
    # the values are far smaller than a tenth of the terms' scale here
    assert np.abs(ref).max() < T / 10
    assert np.isclose(gate_grad_err(got, ref, q, k, dq, dk, nseg), 0.5 / (T / 10))
    # large values: the plain measure
    big = ref * 1e6
    gb = big.copy()
    gb[0, 0, 3] += 2.0
    assert np.isclose(gate_grad_err(gb, big, q, k, dq, dk, nseg), 2.0 / np.abs(big).max())
