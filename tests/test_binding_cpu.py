"""The Python binding refuses tensors whose extents do not match the call
before anything reaches the C ABI: the kernels index every buffer by the
sizes passed through it and cannot see tensor extents.  CPU only: the shape
is checked before the device, so these calls never need a GPU."""
import pytest
import torch

from long_sequence_causal_amd import linattn as la

B, H, L, D = 1, 2, 128, 64
bf = torch.bfloat16


def t(*shape, dtype=bf):
    return torch.zeros(shape, dtype=dtype)


def test_forward_checks_every_extent():
    q, v, lam = t(B, H, L, D), t(B, H, L, D), t(H, dtype=torch.float32)
    with pytest.raises(ValueError, match="k has shape"):
        la.la_chunk_fwd(q, t(B, H, L - 64, D), v, lam)
    with pytest.raises(ValueError, match="lam has shape"):
        la.la_chunk_fwd(q, q, v, t(H + 1, dtype=torch.float32))
    with pytest.raises(ValueError, match="S0 has shape"):
        la.la_chunk_fwd(q, q, v, lam, S0=t(B, H, 2, D, D, dtype=torch.float32))
    with pytest.raises(ValueError, match="out has shape"):
        la.la_chunk_fwd(q, q, v, lam, out=t(B, H, L // 2, D))
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        la.la_chunk_fwd(q, q, v, lam)  # right shapes: the device check comes next


def test_backward_and_gated_check_every_extent():
    q, lam = t(B, H, L, D), t(H, dtype=torch.float32)
    with pytest.raises(ValueError, match="dO has shape"):
        la.la_chunk_bwd(q, q, q, lam, t(B, H, L + 1, D))
    with pytest.raises(ValueError, match="dS_end has shape"):
        la.la_chunk_bwd(q, q, q, lam, q, dS_end=t(B, H, 1, D, D + 1, dtype=torch.float32))
    with pytest.raises(ValueError, match="log_alpha has shape"):
        la.la_chunk_fwd_gated(q, q, q, t(B, H, L - 1, dtype=torch.float32))
    with pytest.raises(ValueError, match="dlog_alpha has shape"):
        la.la_chunk_bwd_gated(q, q, q, t(B, H, L, dtype=torch.float32), q,
                              out=(q, q, q, None, t(B, H, 1, dtype=torch.float32)))


def test_decay_gradient_step_and_scan_check_every_extent():
    q, lam = t(B, H, L, D), t(H, dtype=torch.float32)
    with pytest.raises(ValueError, match="out has shape"):
        la.la_decay_grad(q, q, q, lam, q, out=t(H + 1, dtype=torch.float32))
    qs = t(B, H, D)
    with pytest.raises(ValueError, match="S has shape"):
        la.la_step(qs, qs, qs, lam, S=t(B, H, D, D // 2, dtype=torch.float32))
    with pytest.raises(ValueError, match="v has shape"):
        la.la_step(qs, qs, t(B, H + 1, D), lam)
    dS = t(B, H, 3, D, D, dtype=torch.float32)
    with pytest.raises(ValueError, match="S0 has shape"):
        la.la_state_scan(dS, lam, 64, S0=t(B, H, 1, D, D, dtype=torch.float32))
    with pytest.raises(ValueError, match="log_decay has shape"):
        la.la_state_scan_gated(dS, t(B, H, 4, dtype=torch.float32))
