"""The C ABI on the CPU: the library loads, exports every entry point the
header declares, and rejects bad arguments on the host before any HIP call
(so these run without a GPU).  No compute call is made here."""
import ctypes
import os
import re

import pytest

from long_sequence_causal_amd import linattn as la

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "linattn.h")

FAKE = 0x100000  # 16-byte aligned, never dereferenced: validation fails first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(la_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("la_chunk_fwd", "la_state_scan", "la_chunk_bwd",
                     "la_fwd_workspace_bytes", "la_bwd_workspace_bytes", "la_status_str"):
        assert required in names


def test_library_exports_every_declared_symbol():
    L = la.lib()
    for name in declared_functions():
        assert hasattr(L, name), f"{name} declared in linattn.h but not exported"
    assert set(la.EXPORTS) == set(declared_functions())


def test_version_and_status_strings():
    L = la.lib()
    assert L.la_version() == 1
    for code, name in enumerate(["LA_OK", "LA_ERR_INVALID_ARG", "LA_ERR_UNSUPPORTED",
                                 "LA_ERR_WORKSPACE", "LA_ERR_HIP"]):
        assert L.la_status_str(code).decode() == name


def _fwd(shape, Q=FAKE, K=FAKE, V=FAKE, lam=FAKE, S0=None, O=FAKE, S_end=None,
         ws=None, ws_bytes=0):
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    return la.lib().la_chunk_fwd(ctypes.byref(shape), v(Q), v(K), v(V), v(lam), v(S0), v(O),
                                 v(S_end), v(ws), ws_bytes, None)


def _shape(**kw):
    base = dict(B=1, H=2, L=128, dk=64, dv=64, nseg=1, dtype=la.LA_BF16, split=1)
    base.update(kw)
    return la.make_shape(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), la.LA_ERR_INVALID_ARG),
    (dict(L=-5), la.LA_ERR_INVALID_ARG),
    (dict(nseg=0), la.LA_ERR_INVALID_ARG),
    (dict(L=100, nseg=3), la.LA_ERR_INVALID_ARG),
    (dict(dtype=7), la.LA_ERR_INVALID_ARG),
    (dict(split=-1), la.LA_ERR_INVALID_ARG),
    (dict(dk=0), la.LA_ERR_INVALID_ARG),
    (dict(dk=64, dv=128), la.LA_ERR_UNSUPPORTED),
    (dict(dk=96, dv=96), la.LA_ERR_UNSUPPORTED),
    (dict(dk=256, dv=256), la.LA_ERR_UNSUPPORTED),
    # one segment of 2^24 tokens x 128 bf16 = 2^32 bytes: beyond 32-bit offsets
    (dict(L=1 << 24, dk=128, dv=128), la.LA_ERR_UNSUPPORTED),
    (dict(L=1 << 23, dk=128, dv=128, dtype=la.LA_FP32), la.LA_ERR_UNSUPPORTED),
])
def test_fwd_rejects_bad_shapes(kw, code):
    assert _fwd(_shape(**kw)) == code
    assert la.lib().la_last_error().decode().startswith(la.lib().la_status_str(code).decode())


def test_segment_size_limit_counts_one_segment():
    # Host-side query only: a valid shape with split=2 needs a workspace, a
    # rejected one reports 0.  2^24 tokens of d=128 bf16 in one segment is
    # 2^32 bytes (rejected); the same tokens as two segments, or one chunk
    # fewer, are accepted.
    assert la.la_fwd_workspace_bytes(_shape(L=1 << 24, dk=128, dv=128, split=2)) == 0
    assert la.la_fwd_workspace_bytes(_shape(L=1 << 24, dk=128, dv=128, nseg=2, split=2)) > 0
    assert la.la_fwd_workspace_bytes(_shape(L=(1 << 24) - 64, dk=128, dv=128, split=2)) > 0


def test_fwd_rejects_reserved_field():
    s = _shape()
    s.reserved = 1
    assert _fwd(s) == la.LA_ERR_INVALID_ARG


def test_fwd_rejects_null_and_misaligned_pointers():
    s = _shape()
    assert _fwd(s, Q=None) == la.LA_ERR_INVALID_ARG
    assert _fwd(s, V=None) == la.LA_ERR_INVALID_ARG
    assert _fwd(s, lam=None) == la.LA_ERR_INVALID_ARG
    assert _fwd(s, O=None, S_end=None) == la.LA_ERR_INVALID_ARG
    assert _fwd(s, K=FAKE + 8) == la.LA_ERR_INVALID_ARG
    assert _fwd(s, S0=FAKE + 4) == la.LA_ERR_INVALID_ARG


def test_fwd_workspace_rules():
    s = _shape(L=512, split=4)
    need = la.la_fwd_workspace_bytes(s)
    # B*H = 2 sequences, 4 sub-segments of 2 chunks: 3 scanned 64x64 fp32 states each
    assert need == 2 * 3 * 64 * 64 * 4
    assert _fwd(s, ws=None, ws_bytes=0) == la.LA_ERR_WORKSPACE
    assert _fwd(s, ws=FAKE, ws_bytes=need - 1) == la.LA_ERR_WORKSPACE
    assert la.la_fwd_workspace_bytes(_shape(split=1)) == 0


def test_workspace_bytes_of_invalid_shape_is_zero():
    assert la.la_fwd_workspace_bytes(_shape(dk=96, dv=96)) == 0
    assert la.la_bwd_workspace_bytes(_shape(nseg=0)) == 0


def test_plan_split_normalisation():
    # 128 tokens = 2 chunks: asking for more sub-segments than chunks gives 2
    s = _shape(L=128, split=16)
    assert la.la_fwd_workspace_bytes(s) == 2 * 1 * 64 * 64 * 4
    # 10 chunks in 3 sub-segments of 4, 4, 2 chunks
    s = _shape(L=640, split=3, B=1, H=1)
    assert la.la_fwd_workspace_bytes(s) == 1 * 2 * 64 * 64 * 4
    # automatic choice: 256 workgroups over B*H*nseg sequences
    s = la.make_shape(1, 32, 65536, 128, 128, 1, la.LA_BF16, 0)
    assert la.la_fwd_workspace_bytes(s) == 32 * 7 * 128 * 128 * 4


def test_automatic_plan_takes_a_second_round_only_for_long_walks():
    # the workspace holds the start states of sub-segments 1..split-1, so its
    # size gives the split the library chose
    state = 128 * 128 * 4

    def ws(B, H, L, nseg=1, split=0):
        return la.la_fwd_workspace_bytes(la.make_shape(B, H, L, 128, 128, nseg, la.LA_BF16, split))

    # 32 sequences of 64K tokens: 8 walks of 128 chunks each, one round of 256
    assert ws(1, 32, 65536) == 32 * 7 * state
    # 32 sequences of 16K tokens (walks of 32 chunks): one round
    assert ws(2, 16, 16384) == 32 * 7 * state
    # 16 sequences of 256K tokens: walks of 256 chunks at split 16 become
    # two rounds of 512 walks of 128 chunks
    assert ws(1, 16, 262144) == 16 * 31 * state
    # 16 sequences of 1M tokens: two rounds at most (512 walks)
    assert ws(1, 16, 1 << 20) == 16 * 31 * state
    # 1024 segments of 16K tokens fill the chip without a split
    assert ws(1, 16, 1 << 20, nseg=64) == 0
    # an explicit split is taken as given
    assert ws(1, 16, 262144, split=16) == 16 * 15 * state
    # the backward follows the same plan: two prepared states and three sets
    # of starts (dQ, dV and dK sweeps)
    s = la.make_shape(1, 16, 262144, 128, 128, 1, la.LA_BF16, 0)
    assert la.la_bwd_workspace_bytes(s) == 2 * 16 * 31 * state
    # the decay gradient's tangent walks keep one round: (S, U) starts and one
    # fp64 share per sub-segment
    # (its pre-pass walks each sub-segment as two pieces: two local pairs each)
    assert la.la_decay_grad_workspace_bytes(s) == 2 * 2 * 16 * 15 * state + 16 * 16 * 8


def test_scan_rejects_bad_arguments():
    L = la.lib()
    v = ctypes.c_void_p
    assert L.la_state_scan(-1, 1, 1, 4, 4, v(FAKE), v(FAKE), 1, None, v(FAKE), None, 0, None) == la.LA_ERR_INVALID_ARG
    assert L.la_state_scan(1, 1, -2, 4, 4, v(FAKE), v(FAKE), 1, None, v(FAKE), None, 0, None) == la.LA_ERR_INVALID_ARG
    assert L.la_state_scan(1, 1, 2, 0, 4, v(FAKE), v(FAKE), 1, None, v(FAKE), None, 0, None) == la.LA_ERR_INVALID_ARG
    assert L.la_state_scan(1, 1, 2, 4, 4, None, v(FAKE), 1, None, v(FAKE), None, 0, None) == la.LA_ERR_INVALID_ARG
    assert L.la_state_scan(1, 1, 2, 4, 4, v(FAKE), None, 1, None, v(FAKE), None, 0, None) == la.LA_ERR_INVALID_ARG
    assert L.la_state_scan(1, 1, 2, 4, 4, v(FAKE), v(FAKE), -1, None, v(FAKE), None, 0, None) == la.LA_ERR_INVALID_ARG
    assert L.la_state_scan(1, 1, 2, 4, 4, v(FAKE + 4), v(FAKE), 1, None, v(FAKE), None, 0, None) == la.LA_ERR_INVALID_ARG
    # nothing to do: no sequences
    assert L.la_state_scan(0, 3, 2, 4, 4, None, None, 1, None, None, None, 0, None) == la.LA_OK


def test_bwd_rejects_bad_arguments():
    L = la.lib()
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    s = _shape(split=2)

    def call(**kw):
        a = dict(Q=FAKE, K=FAKE, V=FAKE, lam=FAKE, S0=None, dO=FAKE, dSe=None, dQ=FAKE,
                 dK=FAKE, dV=FAKE, dS0=None, ws=None, nb=0)
        a.update(kw)
        return L.la_chunk_bwd(ctypes.byref(s), v(a["Q"]), v(a["K"]), v(a["V"]), v(a["lam"]),
                              v(a["S0"]), v(a["dO"]), v(a["dSe"]), v(a["dQ"]), v(a["dK"]),
                              v(a["dV"]), v(a["dS0"]), v(a["ws"]), a["nb"], None)

    assert call(dO=None) == la.LA_ERR_INVALID_ARG
    assert call(dK=None) == la.LA_ERR_INVALID_ARG
    assert call(dS0=FAKE + 2) == la.LA_ERR_INVALID_ARG
    # no workspace at split 1 (the sweeps read S0 and dS_end themselves,
    # transposed where they need it) ...
    assert la.la_bwd_workspace_bytes(_shape()) == 0
    # ... and two sets of sub-segment start states otherwise (dQ and dV
    # sweeps; the dK sweep reads the dV sweep's transposed)
    need = la.la_bwd_workspace_bytes(s)
    assert need == 2 * (2 * 1 * 64 * 64 * 4)
    assert call(ws=None) == la.LA_ERR_WORKSPACE
    assert call(ws=FAKE, nb=need - 16) == la.LA_ERR_WORKSPACE


def test_gated_entry_points_validate_on_the_host():
    L = la.lib()
    s = _shape(L=512, split=4)
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    call = lambda G, ws=None, nb=0, O=FAKE: L.la_chunk_fwd_gated(
        ctypes.byref(s), v(FAKE), v(FAKE), v(FAKE), v(G), None, v(O), None, v(ws), nb, None)
    assert call(None) == la.LA_ERR_INVALID_ARG          # log_alpha required
    assert call(FAKE + 4) == la.LA_ERR_INVALID_ARG      # misaligned
    assert call(FAKE) == la.LA_ERR_WORKSPACE            # split 4 needs a workspace
    need = la.la_fwd_gated_workspace_bytes(s)
    # start states of 3 sub-segments and their log-gates, per sequence
    assert need == la.la_fwd_workspace_bytes(s) + 256
    assert call(FAKE, FAKE, need - 1) == la.LA_ERR_WORKSPACE
    assert call(FAKE, O=None) == la.LA_ERR_INVALID_ARG  # O and S_end both NULL
    scan = lambda dS, LD, St, P=3: L.la_state_scan_gated(1, 2, P, 64, 64, v(dS), v(LD), None,
                                                         v(St), None, 0, None)
    assert scan(FAKE, None, FAKE) == la.LA_ERR_INVALID_ARG
    assert scan(None, FAKE, FAKE) == la.LA_ERR_INVALID_ARG
    assert scan(FAKE, FAKE + 8, FAKE) == la.LA_ERR_INVALID_ARG
    assert scan(FAKE, FAKE, FAKE, P=-1) == la.LA_ERR_INVALID_ARG
    # the backward from the forward's states: split 4 needs the forward's workspace
    bneed = la.la_bwd_gated_workspace_bytes(s)
    bwd = lambda fws: L.la_chunk_bwd_gated_from_fwd(
        ctypes.byref(s), v(FAKE), v(FAKE), v(FAKE), v(FAKE), None, v(FAKE), None, v(fws),
        v(FAKE), v(FAKE), v(FAKE), None, None, v(FAKE), bneed, None)
    assert bwd(None) == la.LA_ERR_INVALID_ARG
    assert bwd(FAKE + 8) == la.LA_ERR_INVALID_ARG


def test_gated_backward_workspace_follows_the_1024_token_plan():
    # L = 5000 -> 79 chunks -> 5 sub-segments of 1024 tokens whatever split asks;
    # d = 64: a state is 16 KiB.  Blocks (256-byte aligned): the 1024-row
    # states (4 each: forward, dV, dV transposed for the anchors), the forward
    # and dV start states on the sweeps' own plan (sub-segments of whole
    # 1024-token blocks covering the plan's sub-segment: split 0 or 40 -> 1024
    # tokens, 4 states; split 3 -> 1728 -> 2048 tokens, 2 states; split 1 ->
    # one sub-segment, none), the log-gates of both plans, the shifted gates,
    # the per-token q . dq, S_end and one anchor per block.
    DD4, nseq, Ls = 64 * 64 * 4, 2, 5000
    up = lambda x: -(-x // 256) * 256
    for split, coarse in ((0, 4), (1, 0), (3, 2), (40, 4)):
        want = (3 * up(nseq * 4 * DD4) + 2 * up(nseq * coarse * DD4)
                + up(nseq * 4 * 4) + up(nseq * coarse * 4) + 2 * up(nseq * Ls * 4)
                + up(nseq * DD4) + up(nseq * 5 * 4))
        assert la.la_bwd_gated_workspace_bytes(_shape(L=Ls, split=split)) == want, split


def test_decay_gradient_validates_on_the_host():
    L = la.lib()
    s = _shape(L=3000, split=4)
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    need = la.la_decay_grad_workspace_bytes(s)
    # start pairs (S, U) of the pre-pass's pieces (3 sub-segments of 768
    # tokens, two pieces of 384 each) and one fp64 share per sub-segment
    nseq, D = s.B * s.H, s.dk
    assert need == 2 * nseq * 2 * 3 * D * D * 4 + 256
    assert la.la_decay_grad_workspace_bytes(_shape(dk=96, dv=96)) == 0

    def call(Q=FAKE, K=FAKE, V=FAKE, lam=FAKE, S0=None, dO=FAKE, dSe=None, out=FAKE,
             ws=FAKE, nb=need):
        return L.la_decay_grad(ctypes.byref(s), v(Q), v(K), v(V), v(lam), v(S0), v(dO),
                               v(dSe), v(out), v(ws), nb, None)
    assert call(dO=None) == la.LA_ERR_INVALID_ARG
    assert call(V=None) == la.LA_ERR_INVALID_ARG
    assert call(lam=None) == la.LA_ERR_INVALID_ARG
    assert call(out=None) == la.LA_ERR_INVALID_ARG
    assert call(dSe=FAKE + 8) == la.LA_ERR_INVALID_ARG    # misaligned
    assert call(ws=None) == la.LA_ERR_WORKSPACE
    assert call(nb=need - 1) == la.LA_ERR_WORKSPACE


def test_decode_step_validates_on_the_host():
    L = la.lib()
    v = lambda x: None if x is None else ctypes.c_void_p(x)

    def call(B=2, H=3, dk=64, dv=64, dt=la.LA_BF16, q=FAKE, k=FAKE, vv=FAKE, lam=FAKE, S=None,
             So=FAKE + (1 << 24), o=FAKE):
        return L.la_step(B, H, dk, dv, dt, v(q), v(k), v(vv), v(lam), v(S), v(So), v(o), None)
    assert call(B=0, q=None, k=None, vv=None, lam=None, So=None) == la.LA_OK  # no-op
    assert call(q=None) == la.LA_ERR_INVALID_ARG
    assert call(So=None) == la.LA_ERR_INVALID_ARG
    assert call(B=-1) == la.LA_ERR_INVALID_ARG
    assert call(dt=7) == la.LA_ERR_INVALID_ARG
    assert call(dk=64, dv=128) == la.LA_ERR_UNSUPPORTED
    assert call(dk=96, dv=96) == la.LA_ERR_UNSUPPORTED
    assert call(k=FAKE + 4) == la.LA_ERR_INVALID_ARG
    # S_out overlapping S without being S
    assert call(S=FAKE + (1 << 24), So=FAKE + (1 << 24) + 4096) == la.LA_ERR_INVALID_ARG
    assert call(lam=None) == la.LA_ERR_INVALID_ARG

    def gcall(B=2, H=3, G=FAKE, S=None, So=FAKE + (1 << 24), dk=64):
        return L.la_step_gated(B, H, dk, dk, la.LA_BF16, v(FAKE), v(FAKE), v(FAKE), v(G), v(S),
                               v(So), v(FAKE), None)
    assert gcall(B=0, G=None, So=None) == la.LA_OK  # no-op
    assert gcall(G=None) == la.LA_ERR_INVALID_ARG      # log_alpha required
    assert gcall(G=FAKE + 4) == la.LA_ERR_INVALID_ARG  # misaligned
    assert gcall(So=None) == la.LA_ERR_INVALID_ARG
    assert gcall(dk=96) == la.LA_ERR_UNSUPPORTED
    assert gcall(S=FAKE + (1 << 24), So=FAKE + (1 << 24) + 4096) == la.LA_ERR_INVALID_ARG


def test_empty_problem_is_a_no_op():
    # B*H = 0: nothing to read or write, no HIP call needed
    assert _fwd(_shape(B=0), Q=None, K=None, V=None, lam=None) == la.LA_OK


def test_product_path_has_no_oracle_dependency():
    """The library and its binding never reference the CPU oracle."""
    pkg = os.path.join(ROOT, "long_sequence_causal_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), f
                assert "liblao" not in text and "lao_" not in text and "lao.c" not in text, f


def test_launch_grids_stay_within_32_bit_work_item_counts():
    """A launch covers at most 2^32 - 1 work-items.  Shapes whose launches
    would exceed that (one thread per state element of 2^18 states of
    128 x 128; one workgroup of 256 per 32-column slab of a decode state; a
    walk per 64-token sub-segment) are rejected on the host, before any HIP
    call, with LA_ERR_UNSUPPORTED -- never half-run."""
    L = la.lib()
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    # 2^18 sequences of 128 x 128 states: 2^32 state elements
    big = _shape(B=1 << 12, H=64, L=64, dk=128, dv=128, split=0)
    assert _fwd(big) == la.LA_ERR_UNSUPPORTED
    assert la.la_fwd_workspace_bytes(big) == 0
    assert la.la_bwd_workspace_bytes(big) == 0
    assert la.la_decay_grad_workspace_bytes(big) == 0
    ok = _shape(B=1 << 11, H=64, L=64, dk=128, dv=128, split=0)  # 2^17 sequences: fits
    assert la.la_decay_grad_workspace_bytes(ok) > 0  # a valid plan (its fp64 shares)
    assert L.la_state_scan(1 << 12, 64, 2, 128, 128, v(FAKE), v(FAKE), 64, None, v(FAKE), None,
                           0, None) == la.LA_ERR_UNSUPPORTED
    assert L.la_state_scan_gated(1 << 12, 64, 2, 128, 128, v(FAKE), v(FAKE), None, v(FAKE), None,
                                 0, None) == la.LA_ERR_UNSUPPORTED
    # decode: 2^21 sequences x 4 slabs x 256 threads = 2^31 fits; 2^22 x 4 x 256 does not
    step = lambda B: L.la_step(B, 1, 128, 128, la.LA_BF16, v(FAKE), v(FAKE), v(FAKE), v(FAKE),
                               None, v(FAKE), v(FAKE), None)
    assert step(1 << 23) == la.LA_ERR_UNSUPPORTED
    # many short sequences: 2^26 sequences of one chunk -> 2^26 walks x 512 threads
    many = _shape(B=1 << 20, H=64, L=64, dk=128, dv=128, split=1)
    assert _fwd(many) == la.LA_ERR_UNSUPPORTED
    # the gated backward's 1024-token blocks
    s = _shape(B=1 << 10, H=64, L=1 << 14, dk=128, dv=128, split=0)
    assert L.la_chunk_bwd_gated(ctypes.byref(s), v(FAKE), v(FAKE), v(FAKE), v(FAKE), None, v(FAKE),
                                None, v(FAKE), v(FAKE), v(FAKE), None, None, v(FAKE), 1 << 40,
                                None) == la.LA_ERR_UNSUPPORTED
