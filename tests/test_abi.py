"""The C ABI on the host: the library loads without a GPU, exports every symbol
include/kda.h declares, and rejects bad arguments on the host before any HIP
call (so these calls are safe with fake pointers and no device)."""
import ctypes
import re
from pathlib import Path

import pytest

import chunked_gated_delta_kda_amd as kda

HEADER = Path(__file__).resolve().parents[1] / "include" / "kda.h"
FAKE = ctypes.c_void_p(0x1000)  # 256-aligned, never dereferenced on these paths


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", HEADER.read_text(), flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return kda.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(kda.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), f"libkda.so does not export {n}"


def test_version_and_status_strings(lib):
    assert kda.version() == 100
    for code in range(5):
        assert kda.status_str(code)
    assert kda.status_str(99) == "unknown status"


def test_workspace_size_formula(lib):
    C = 32  # tokens per chunk
    rec = 3 * C * 128 * 2 + 2 * C * C * 2 + 128 * 4  # bytes per (chunk, head) at K=128
    B, T, H, N = 2, 2048, 32, 2
    al = lambda x: (x + 255) // 256 * 256
    meta = al(2 * 4 * (N + 1))
    slots = (B * T + C - 1) // C + N  # the packed-sequence bound covers both layouts
    bound = al(slots * H * 4)  # one fp32 transition bound per (chunk, head)
    want = meta + slots * H * rec + bound
    # the two-stage pass: 64 pairs x 4 blocks, no splitting
    assert kda.workspace_size(B, T, H, 128, 128, path="staged") == want
    assert kda.workspace_size(B, T, H, 128, 128, segment_chunks=-1, path="staged") == want
    # the single-launch pass: only the packed layout's tables (segments of
    # L = max(8, ceil(slots H / 512)) chunks, at most N + ceil(slots / L) of them)
    L = max(8, -(-slots * H // 512))
    nv = N + -(-slots // L)
    # sequence tables, segment tables and the longest-first dispatch order
    fused = meta + al(4 * (2 * (nv + 1) + nv + N + 1 + nv))
    assert kda.workspace_size(B, T, H, 128, 128) == fused
    assert fused < 4096 < want
    L = 16
    nv = N + -(-slots // L)
    assert kda.workspace_size(B, T, H, 128, 128, segment_chunks=L) == \
        meta + al(4 * (2 * (nv + 1) + nv + N + 1 + nv))
    for path in ("fused", "staged"):
        assert kda.workspace_size(1, 100, 1, 96, 128, path=path) == 0  # unsupported K
        assert kda.workspace_size(0, 100, 1, 128, 128, path=path) == 0


def _kda_call(lib, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, A_log=FAKE, dt_bias=FAKE, lb=-5.0,
             scale=0.088, h0=None, hT=None, cu=None, N=0, B=1, T=16, H=1, K=128, V=128, o=FAKE,
             ws=FAKE, wsb=1 << 30, stream=None)
    a.update(over)
    return lib.kda_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["A_log"], a["dt_bias"],
                       a["lb"], a["scale"], a["h0"], a["hT"], a["cu"], a["N"], a["B"], a["T"],
                       a["H"], a["K"], a["V"], a["o"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(g=None), 1),
    (dict(beta=None), 1), (dict(o=None), 1), (dict(A_log=None), 1), (dict(dt_bias=None), 1),
    (dict(B=0), 1), (dict(T=-1), 1), (dict(H=0), 1),
    (dict(lb=-5.5), 1), (dict(lb=0.5), 1), (dict(lb=float("nan")), 1),
    (dict(scale=float("inf")), 1),
    (dict(K=96), 2), (dict(V=256), 2),
    (dict(cu=FAKE, B=2, N=2), 1), (dict(cu=FAKE, N=0), 1),
    # packed sequences need the segment tables in the workspace
    (dict(cu=FAKE, N=2, ws=None), 3), (dict(cu=FAKE, N=2, wsb=100), 3),
    (dict(cu=FAKE, N=2, ws=ctypes.c_void_p(0x1010)), 3),
    (dict(q=ctypes.c_void_p(0x1002)), 1), (dict(dt_bias=ctypes.c_void_p(0x1008)), 1),
    (dict(o=ctypes.c_void_p(0x1008)), 1), (dict(h0=ctypes.c_void_p(0x1004)), 1),
    (dict(hT=ctypes.c_void_p(0x1008)), 1), (dict(beta=ctypes.c_void_p(0x1001)), 1),
    (dict(B=1 << 16, T=1 << 15), 1),
])
def test_kda_rejects_on_host(lib, over, code):
    assert _kda_call(lib, **over) == code


@pytest.mark.parametrize("over,code", [
    (dict(ws=None), 3), (dict(wsb=100), 3), (dict(ws=ctypes.c_void_p(0x1010)), 3),
    (dict(g=None), 1), (dict(K=96), 2),
])
def test_two_stage_rejects_on_host(lib, over, code):
    """kda_fwd_split keeps its record workspace for fixed-length batches too."""
    a = dict(g=FAKE, K=128, ws=FAKE, wsb=1 << 30)
    a.update(over)
    st = lib.kda_fwd_split(FAKE, FAKE, FAKE, a["g"], FAKE, FAKE, FAKE, -5.0, 0.088, None, None,
                           None, 0, 1, 16, 1, a["K"], 128, FAKE, a["ws"], a["wsb"], -1, None)
    assert st == code


def test_segmented_and_timed_check_like_kda_fwd(lib):
    base = [FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, -5.0, 0.088, None, None, None, 0, 1, 16,
            1, 128, 128, FAKE, FAKE, 1 << 30]
    assert lib.kda_fwd_segmented(*base, 4, None) == 1  # null g
    assert lib.kda_fwd_timed(*base, None, None, None) == 1
    base[3] = FAKE
    ev = ctypes.c_void_p(0x2000)
    assert lib.kda_fwd_timed(*base, None, ev, None) == 1  # one event of two
    assert lib.kda_fwd_timed(*base, None, None, ev) == 1
    base[16] = 32
    assert lib.kda_fwd_segmented(*base, 4, None) == 2
    gbase = [FAKE, FAKE, FAKE, None, FAKE, 0.1, None, None, None, 0, 1, 16, 1, 128, 128, FAKE,
             FAKE, 1 << 30]
    assert lib.gdn_fwd_segmented(*gbase, 4, None) == 1
    assert lib.gdn_fwd_timed(*gbase, None, None, None) == 1
    gbase[3] = FAKE
    assert lib.gdn_fwd_timed(*gbase, None, ev, None) == 1


def test_gdn_rejects_on_host(lib):
    args = [FAKE, FAKE, FAKE, None, FAKE, 0.1, None, None, None, 0, 1, 16, 1, 128, 128, FAKE,
            FAKE, 1 << 30, None]
    assert lib.gdn_fwd(*args) == 1  # null g
    args[3] = FAKE
    args[13] = 32
    assert lib.gdn_fwd(*args) == 2  # unsupported K
    args[13] = 128
    args[17] = 10
    assert lib.gdn_fwd_split(*args[:18], -1, None) == 3  # two-stage workspace too small
    args[8], args[9] = FAKE, 3
    assert lib.gdn_fwd(*args) == 3  # packed: segment tables do not fit


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError, match="missing"):
        kda.load(tmp_path / "nope.so")


def _decode_call(lib, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, A_log=FAKE, dt_bias=FAKE, lb=-5.0,
             scale=0.088, s_in=None, s_out=FAKE, N=2, H=4, K=128, V=128, o=FAKE, stream=None)
    a.update(over)
    return lib.kda_decode(a["q"], a["k"], a["v"], a["g"], a["beta"], a["A_log"], a["dt_bias"],
                          a["lb"], a["scale"], a["s_in"], a["s_out"], a["N"], a["H"], a["K"],
                          a["V"], a["o"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(g=None), 1),
    (dict(beta=None), 1), (dict(o=None), 1), (dict(s_out=None), 1), (dict(A_log=None), 1),
    (dict(dt_bias=None), 1), (dict(N=0), 1), (dict(H=0), 1), (dict(lb=-6.0), 1),
    (dict(scale=float("nan")), 1), (dict(K=32), 2), (dict(V=96), 2),
    (dict(s_in=ctypes.c_void_p(0x1004)), 1), (dict(q=ctypes.c_void_p(0x1008)), 1),
])
def test_kda_decode_rejects_on_host(lib, over, code):
    assert _decode_call(lib, **over) == code


def test_gdn_decode_rejects_on_host(lib):
    args = [FAKE, FAKE, FAKE, None, FAKE, 0.1, None, FAKE, 2, 4, 128, 128, FAKE, None]
    assert lib.gdn_decode(*args) == 1  # null g
    args[3] = FAKE
    args[10] = 48
    assert lib.gdn_decode(*args) == 2  # unsupported K
    args[10] = 128
    args[7] = None
    assert lib.gdn_decode(*args) == 1  # null state_out


def test_split_workspace_grows_with_segments(lib):
    """Explicit splitting adds the segment tables, flags, two [segments, H, K, V]
    state buffers and the [segments, H, K, K] transitions."""
    B, T, H, K, V = 1, 8192, 2, 128, 128
    plain = kda.workspace_size(B, T, H, K, V, segment_chunks=-1, path="staged")
    slots = (B * T + 31) // 32 + 1
    for L in (16, 64):
        nv = 1 + (slots + L - 1) // L
        extra = kda.workspace_size(B, T, H, K, V, segment_chunks=L, path="staged") - plain
        states = nv * H * K * V * 4
        assert extra >= 2 * states + nv * H * K * K * 4
        assert extra < 2 * states + nv * H * K * K * 4 + 4096
    # automatic: 2 heads x 4 column blocks is far too few workgroups, so it splits
    assert kda.workspace_size(B, T, H, K, V, path="staged") > plain


def _kda_bwd_call(lib, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, A_log=FAKE, dt_bias=FAKE, lb=-5.0,
             scale=0.088, h0=None, cu=None, N=0, B=1, T=16, H=1, K=128, V=128, do=FAKE,
             dfin=None, dq=FAKE, dk=FAKE, dv=FAKE, dg=FAKE, dbeta=FAKE, dA=FAKE, ddt=FAKE,
             dh0=None, ws=FAKE, wsb=1 << 30, stream=None)
    a.update(over)
    return lib.kda_bwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["A_log"], a["dt_bias"],
                       a["lb"], a["scale"], a["h0"], a["cu"], a["N"], a["B"], a["T"], a["H"],
                       a["K"], a["V"], a["do"], a["dfin"], a["dq"], a["dk"], a["dv"], a["dg"],
                       a["dbeta"], a["dA"], a["ddt"], a["dh0"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("over,code", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(g=None), 1),
    (dict(beta=None), 1), (dict(do=None), 1), (dict(dq=None), 1), (dict(dk=None), 1),
    (dict(dv=None), 1), (dict(dg=None), 1), (dict(dbeta=None), 1), (dict(dA=None), 1),
    (dict(ddt=None), 1), (dict(A_log=None), 1), (dict(B=0), 1), (dict(H=0), 1),
    (dict(lb=-7.0), 1), (dict(scale=float("nan")), 1), (dict(K=96), 2), (dict(V=32), 2),
    (dict(ws=None), 3), (dict(wsb=4096), 3),
    (dict(dq=ctypes.c_void_p(0x1002)), 1), (dict(dfin=ctypes.c_void_p(0x1004)), 1),
    (dict(dh0=ctypes.c_void_p(0x1008)), 1),
    # more (sequence, head) pairs than the recurrence grids can address
    (dict(cu=FAKE, N=1 << 27, H=16, wsb=1 << 62), 1),
])
def test_kda_bwd_rejects_on_host(lib, over, code):
    assert _kda_bwd_call(lib, **over) == code


def test_kda_bwd_needs_the_larger_workspace(lib):
    fwd = kda.workspace_size(1, 16, 1, 128, 128, path="staged")
    bwd = kda.bwd_workspace_size(1, 16, 1, 128, 128)
    assert bwd > fwd > 0
    # enough for the forward pass, not for the backward: rejected before any launch
    assert _kda_bwd_call(lib, wsb=fwd) == 3
    assert kda.bwd_workspace_size(1, 16, 1, 96, 128) == 0


def test_gdn_bwd_rejects_on_host(lib):
    def call(**over):
        a = dict(g=FAKE, K=128, wsb=1 << 30, dg=FAKE)
        a.update(over)
        return lib.gdn_bwd(FAKE, FAKE, FAKE, a["g"], FAKE, 0.088, None, None, 0, 1, 16, 1,
                           a["K"], 128, FAKE, None, FAKE, FAKE, FAKE, a["dg"], FAKE, None, FAKE,
                           a["wsb"], None)
    assert call(g=None) == 1
    assert call(dg=None) == 1
    assert call(K=32) == 2
    assert call(wsb=4096) == 3


@pytest.mark.parametrize("flag,value", [
    ("use_qk_l2norm_in_kernel", False), ("use_gate_in_kernel", False),
    ("use_beta_sigmoid_in_kernel", False), ("safe_gate", False),
    ("transpose_state_layout", True),
])
def test_chunk_kda_rejects_unsupported_variants(flag, value):
    import torch
    from chunked_gated_delta_kda_amd.autograd import chunk_kda
    x = torch.zeros(1, 4, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(NotImplementedError, match=flag):
        chunk_kda(x, x, x, x, torch.zeros(1, 4, 1, dtype=torch.bfloat16), torch.zeros(1),
                  torch.zeros(64), **{flag: value})


def test_fwd_save_needs_the_backward_workspace(lib):
    fwd = kda.workspace_size(1, 16, 1, 128, 128, path="staged")
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, -5.0, 0.088, None, None, None, 0, 1, 16, 1,
            128, 128, FAKE, FAKE, fwd, None]
    assert lib.kda_fwd_save(*args) == 3  # enough for kda_fwd only
    args[3] = None
    assert lib.kda_fwd_save(*args) == 1  # null g
    gargs = [FAKE, FAKE, FAKE, None, FAKE, 0.1, None, None, None, 0, 1, 16, 1, 128, 128, FAKE,
             FAKE, 1 << 30, None]
    assert lib.gdn_fwd_save(*gargs) == 1  # null g


def test_bwd_saved_checks_like_bwd(lib):
    for over, code in ((dict(dq=None), 1), (dict(K=96), 2), (dict(wsb=4096), 3)):
        a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, A_log=FAKE, dt_bias=FAKE, lb=-5.0,
                 scale=0.088, h0=None, cu=None, N=0, B=1, T=16, H=1, K=128, V=128, do=FAKE,
                 dfin=None, dq=FAKE, dk=FAKE, dv=FAKE, dg=FAKE, dbeta=FAKE, dA=FAKE, ddt=FAKE,
                 dh0=None, ws=FAKE, wsb=1 << 30, stream=None)
        a.update(over)
        assert lib.kda_bwd_saved(*a.values()) == code


def test_timed_stages_need_both_events_or_none(lib):
    """kda_prep_timed / kda_recur_timed: exactly one event handle is rejected on the
    host (before any HIP call); the other checks are those of the plain stages."""
    ev = ctypes.c_void_p(0x2000)
    prep = lambda s, e: lib.kda_prep_timed(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, -5.0, None, 0, 1,
                                           16, 1, 128, 128, FAKE, 1 << 30, None, s, e)
    recur = lambda s, e: lib.kda_recur_timed(FAKE, 0.088, None, None, 0, 0, 1, 16, 1, 128, 128,
                                             FAKE, FAKE, 1 << 30, None, s, e)
    for call in (prep, recur):
        assert call(ev, None) == 1
        assert call(None, ev) == 1
    # plain-stage checks still apply with both events given
    assert lib.kda_recur_timed(FAKE, 0.088, None, None, 0, 0, 1, 16, 1, 96, 128, FAKE, FAKE,
                               1 << 30, None, ev, ev) == 2
    assert lib.kda_prep_timed(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, -5.0, None, 0, 1, 16, 1, 128,
                              128, None, 1 << 30, None, ev, ev) == 3


def test_prep_grid_limit_checked_on_host(lib):
    """kda_prep's grid is one-dimensional over chunk slots x heads: a batch whose
    slots x heads exceeds 2^31 - 1 is rejected before any launch (2^19 slots x
    8192 heads here; the workspace size passed is large enough to get there)."""
    st = lib.kda_prep(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, -5.0, None, 0, 1, 1 << 24, 8192, 64,
                      64, FAKE, 1 << 62, None)
    assert st == 1


def test_noalloc_rejects_on_host(lib):
    """kda_fwd_noalloc: the checks of kda_fwd, and a packed batch whose tables
    exceed the library's scratch array rejected before any HIP call."""
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, -5.0, 0.088, None, None, FAKE, 1 << 20, 1,
            1 << 24, 4, 128, 128, FAKE, None]
    assert lib.kda_fwd_noalloc(*args) == 3  # 2^20 sequences: tables far beyond 4 MiB
    args[12], args[14] = 2, 64  # a small packed batch: the checks of kda_fwd
    args[3] = None
    assert lib.kda_fwd_noalloc(*args) == 1  # null g
    args[3] = FAKE
    args[16] = 96
    assert lib.kda_fwd_noalloc(*args) == 2  # unsupported K

