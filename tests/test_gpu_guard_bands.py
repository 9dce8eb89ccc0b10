"""Guard bands: every output buffer and workspace is a view into a larger
allocation with 4 KiB before and after it filled with 0xFF bytes (a NaN
pattern in fp32 and bf16).  After each call through the C ABI the guard bytes
must be unchanged (nothing is written outside the buffers the call was given)
and no output may still hold the NaN pattern (outputs are fully
overwritten).  Covers every entry point, with ragged lengths, segments and a
split plan whose workspace is in use.  Needs a gfx950 GPU."""
import pytest
import torch

from gpu_helpers import log, require_gpu
from long_sequence_causal_amd import linattn as la
from long_sequence_causal_amd.inputs import gate_logs, make_inputs

pytestmark = pytest.mark.gpu

GUARD = 4096


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


class Guarded:
    """Buffers carved out of 0xFF-filled allocations with guard bands."""

    def __init__(self):
        self.bufs = []

    def new(self, shape, dtype):
        esz = torch.empty((), dtype=dtype).element_size()
        n = 1
        for x in shape:
            n *= int(x)
        nbytes = n * esz
        raw = torch.full((GUARD + nbytes + GUARD,), 0xFF, dtype=torch.uint8, device="cuda")
        view = raw[GUARD:GUARD + nbytes].view(dtype).view(*shape)
        self.bufs.append((raw, nbytes))
        return view

    def workspace(self, nbytes):
        return self.new((max(nbytes, 1),), torch.uint8)

    def check(self, label, outputs=()):
        torch.cuda.synchronize()
        for raw, nbytes in self.bufs:
            lo, hi = raw[:GUARD], raw[GUARD + nbytes:]
            assert bool((lo == 0xFF).all()), f"{label}: write below a buffer"
            assert bool((hi == 0xFF).all()), f"{label}: write above a buffer"
        for name, t in outputs:
            assert not bool(torch.isnan(t.float()).any()), f"{label}: {name} not fully written"
        log(f"guard bands intact: {label}")


CASES = [("bf16", 128, 1, 3, 64 * 9 + 21, 1, 3), ("bf16", 64, 2, 2, 64 * 6, 2, 2),
         ("fp32", 64, 1, 2, 64 * 4 + 5, 1, 2)]


@pytest.mark.parametrize("dtype,D,B,H,L,nseg,split", CASES)
def test_forward_backward_scan_stay_inside_their_buffers(dtype, D, B, H, L, nseg, split):
    log(f"guard case dtype={dtype} D={D} B={B} H={H} L={L} nseg={nseg} split={split}")
    inp = make_inputs(B, H, L, D, D, dtype=dtype, s0_std=0.3, nseg=nseg, need_dO=True,
                      dS_end_std=0.3, seed=505, device="cuda")
    q, k, v, lam, S0, dO, dSe = (inp[x] for x in ("q", "k", "v", "lam", "S0", "dO", "dS_end"))
    td = q.dtype
    shape = la.make_shape(B, H, L, D, D, nseg, la._dtype_code(td), split)
    g = Guarded()
    # forward
    O = g.new((B, H, L, D), td)
    S_end = g.new((B, H, nseg, D, D), torch.float32)
    ws = g.workspace(la.la_fwd_workspace_bytes(shape))
    la.la_chunk_fwd(q, k, v, lam, S0=S0, nseg=nseg, split=split, out=O, S_end_out=S_end,
                    workspace=ws)
    g.check("la_chunk_fwd", [("O", O), ("S_end", S_end)])
    # state-only forward
    S_only = g.new((B, H, nseg, D, D), torch.float32)
    la.la_chunk_fwd(q, k, v, lam, S0=S0, nseg=nseg, split=split, need_O=False, S_end_out=S_only,
                    workspace=ws)
    g.check("la_chunk_fwd state only", [("S_end", S_only)])
    # scan (out of place and in place)
    dS = torch.randn((B, H, 5, D, D), device="cuda")
    St = g.new((B, H, 5, D, D), torch.float32)
    Se = g.new((B, H, D, D), torch.float32)
    la.la_state_scan(dS, lam, 64, S0=S0[:, :, 0].contiguous(), out=St, S_end_out=Se)
    g.check("la_state_scan", [("S_start", St), ("S_end", Se)])
    # backward and backward from the forward's start states
    outs = (g.new((B, H, L, D), td), g.new((B, H, L, D), td), g.new((B, H, L, D), td),
            g.new((B, H, nseg, D, D), torch.float32))
    bws = g.workspace(la.la_bwd_workspace_bytes(shape))
    la.la_chunk_bwd(q, k, v, lam, dO, S0=S0, dS_end=dSe, nseg=nseg, split=split, out=outs,
                    workspace=bws)
    g.check("la_chunk_bwd", list(zip(("dQ", "dK", "dV", "dS0"), outs)))
    for t in outs:
        t.fill_(float("nan"))
    la.la_chunk_bwd(q, k, v, lam, dO, S0=S0, dS_end=dSe, nseg=nseg, split=split, out=outs,
                    workspace=bws, fwd_workspace=ws)
    g.check("la_chunk_bwd_from_fwd", list(zip(("dQ", "dK", "dV", "dS0"), outs)))
    # gated forward, scan and backward
    G = gate_logs(lam, B, L, 9, device="cuda")
    Og = g.new((B, H, L, D), td)
    Sg = g.new((B, H, nseg, D, D), torch.float32)
    gws = g.workspace(la.la_fwd_gated_workspace_bytes(shape))
    la.la_chunk_fwd_gated(q, k, v, G, S0=S0, nseg=nseg, split=split, out=Og, S_end_out=Sg,
                          workspace=gws)
    g.check("la_chunk_fwd_gated", [("O", Og), ("S_end", Sg)])
    LD = -torch.rand((B, H, 5), device="cuda")
    Stg = g.new((B, H, 5, D, D), torch.float32)
    Seg = g.new((B, H, D, D), torch.float32)
    la.la_state_scan_gated(dS, LD, S0=S0[:, :, 0].contiguous(), out=Stg, S_end_out=Seg)
    g.check("la_state_scan_gated", [("S_start", Stg), ("S_end", Seg)])
    gouts = (g.new((B, H, L, D), td), g.new((B, H, L, D), td), g.new((B, H, L, D), td),
             g.new((B, H, nseg, D, D), torch.float32), g.new((B, H, L), torch.float32))
    gbws = g.workspace(la.la_bwd_gated_workspace_bytes(shape))
    la.la_chunk_bwd_gated(q, k, v, G, dO, S0=S0, dS_end=dSe, nseg=nseg, split=split, out=gouts,
                          workspace=gbws)
    g.check("la_chunk_bwd_gated", list(zip(("dQ", "dK", "dV", "dS0", "dlog_alpha"), gouts)))
    for t in gouts:
        t.fill_(float("nan"))
    la.la_chunk_bwd_gated(q, k, v, G, dO, S0=S0, dS_end=dSe, nseg=nseg, split=split, out=gouts,
                          workspace=gbws, fwd_workspace=gws)
    g.check("la_chunk_bwd_gated_from_fwd",
            list(zip(("dQ", "dK", "dV", "dS0", "dlog_alpha"), gouts)))
    # decay gradient
    dl = g.new((H,), torch.float32)
    tws = g.workspace(la.la_decay_grad_workspace_bytes(shape))
    la.la_decay_grad(q, k, v, lam, dO, S0=S0, dS_end=dSe, nseg=nseg, split=split, out=dl,
                     workspace=tws)
    g.check("la_decay_grad", [("dlambda", dl)])


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("fp32", 64)])
def test_decode_step_stays_inside_its_buffers(dtype, D):
    B, H = 3, 5
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    gen = torch.Generator(device="cuda").manual_seed(3)
    q, k, v = (torch.randn((B, H, D), generator=gen, device="cuda").to(td) for _ in range(3))
    lam = torch.rand((H,), generator=gen, device="cuda") * 0.5 + 0.5
    S = torch.randn((B, H, D, D), generator=gen, device="cuda") * 0.1
    g = Guarded()
    o = g.new((B, H, D), td)
    So = g.new((B, H, D, D), torch.float32)
    la.la_step(q, k, v, lam, S, out=o, S_out=So)
    g.check("la_step", [("o", o), ("S_out", So)])
    la.la_step(q, k, v, lam, So, out=o, S_out=So)  # in place
    g.check("la_step in place", [("o", o), ("S_out", So)])
    G = -torch.rand((B, H), generator=gen, device="cuda")
    o.fill_(float("nan"))
    So.fill_(float("nan"))
    la.la_step_gated(q, k, v, G, S, out=o, S_out=So)
    g.check("la_step_gated", [("o", o), ("S_out", So)])
