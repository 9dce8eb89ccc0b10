"""Shared helpers of the GPU tests (no arithmetic of the method here)."""
import numpy as np
import torch

TOL = {"bf16": 1e-2, "fp32": 1e-4}


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("this test needs a gfx950 GPU")
    name = torch.cuda.get_device_properties(0).gcnArchName
    assert name.startswith("gfx950"), f"expected gfx950, found {name}"


def f64(t):
    if t is None:
        return None
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(x, ref):
    """max |x - ref| / max |ref| in fp64 (the graded measure)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(x - ref))) if ref.size else 0.0
    return num / den if den > 0 else num


def gate_grad_err(got, ref, q, k, dq_ref, dk_ref, nseg=1):
    """The measure of the log-gate gradient (bf16 paths): its value at t is an
    in-block suffix sum of q_u . dq_u - k_u . dk_u over 1024-token blocks of
    each segment, terms that cancel, so its attainable accuracy is set by the
    terms' magnitude T = max_t sum_{u >= t in t's block} (|q_u . dq_u| +
    |k_u . dk_u|) (from the oracle's dq, dk), not by max|ref| alone.  Returns
    max|got - ref| / max(max|ref|, T / 10): at most 1e-2 means an error below
    1e-2 of the largest value or below 1e-3 of T (half a bf16 unit roundoff
    of the terms), whichever is larger."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    q, k = np.asarray(q, np.float64), np.asarray(k, np.float64)
    B, H, L, _ = q.shape
    a = np.abs((q * np.asarray(dq_ref)).sum(-1)) + np.abs((k * np.asarray(dk_ref)).sum(-1))
    Ls = L // nseg
    nb = -(-Ls // 1024)
    pad = np.zeros((B, H, nseg, nb * 1024))
    pad[..., :Ls] = a.reshape(B, H, nseg, Ls)
    blk = pad.reshape(B, H, nseg, nb, 1024)
    T = float(np.flip(np.cumsum(np.flip(blk, -1), -1), -1).max()) if L else 0.0
    den = max(float(np.abs(ref).max()) if ref.size else 0.0, T / 10.0)
    num = float(np.abs(got - ref).max()) if ref.size else 0.0
    return num / den if den > 0 else num


class WholeTensorErr:
    """The graded measure max |X - X_ref| / max |X_ref| over whole tensors that
    are compared a slice of heads at a time: running maxima of the numerator
    and denominator per output name, and each head's own error for the log
    (a fast-decaying head's outputs are small next to the slow heads', so its
    error on its own scale is worth seeing even though it is not graded)."""

    def __init__(self):
        self.num, self.den, self.heads = {}, {}, {}

    def add(self, name, got, ref, heads):
        """got, ref: fp64 arrays [B, len(heads), ...] of the heads listed."""
        got = np.asarray(got, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        assert got.shape == ref.shape, (name, got.shape, ref.shape)
        for i, h in enumerate(heads):
            d = float(np.max(np.abs(got[:, i] - ref[:, i]))) if ref[:, i].size else 0.0
            r = float(np.max(np.abs(ref[:, i]))) if ref[:, i].size else 0.0
            self.num[name] = max(self.num.get(name, 0.0), d)
            self.den[name] = max(self.den.get(name, 0.0), r)
            self.heads.setdefault(name, {})[h] = d / r if r > 0 else d

    def err(self, name):
        n, d = self.num[name], self.den[name]
        return n / d if d > 0 else n

    def report(self, label):
        """Log the whole-tensor error of every output and each head's own
        error; return {name: whole-tensor error}."""
        out = {}
        for name in self.num:
            out[name] = self.err(name)
            ph = self.heads[name]
            worst = max(ph, key=ph.get)
            log(f"{label}: {name} whole-tensor err {out[name]:.3e} over {len(ph)} heads "
                f"(max |ref| {self.den[name]:.4g}); per head on its own scale: "
                + " ".join(f"h{h}={e:.2e}" for h, e in sorted(ph.items()))
                + f"; worst h{worst}")
        return out


def log(msg):
    print(msg, flush=True)
