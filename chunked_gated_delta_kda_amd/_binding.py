"""ctypes binding of libkda (include/kda.h).

Argument marshalling only: dtype, shape and device checks, allocation of the
outputs and the workspace with torch, and the current HIP stream.  Every step
of the computation runs in the HIP kernels of libkda.so; if the library is
missing this module raises instead of computing anything elsewhere.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

PKG = Path(__file__).resolve().parent
LIB_PATH = PKG / "libkda.so"

_STATUS_NAMES = {0: "KDA_OK", 1: "KDA_ERR_INVALID_ARG", 2: "KDA_ERR_UNSUPPORTED",
                 3: "KDA_ERR_WORKSPACE", 4: "KDA_ERR_LAUNCH"}

# Every symbol include/kda.h declares.
EXPORTS = ("kda_fwd", "gdn_fwd", "kda_fwd_workspace_size", "gdn_fwd_workspace_size",
           "kda_fwd_segmented_workspace_size", "kda_fwd_segmented", "gdn_fwd_segmented",
           "kda_fwd_timed", "gdn_fwd_timed", "kda_fwd_noalloc",
           "kda_fwd_split_workspace_size", "kda_fwd_split", "gdn_fwd_split", "kda_prep",
           "gdn_prep", "kda_recur", "kda_prep_timed", "kda_recur_timed", "kda_decode", "gdn_decode", "kda_bwd_workspace_size",
           "kda_bwd", "gdn_bwd", "kda_fwd_save", "gdn_fwd_save", "kda_bwd_saved",
           "gdn_bwd_saved", "kda_status_str", "kda_version")


class LibKdaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None


def load(path: Path | str | None = None):
    """Load libkda.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = Path(path) if path else LIB_PATH
    if not p.exists():
        raise RuntimeError(f"{p} is missing: build it with "
                           f"`python -m chunked_gated_delta_kda_amd.build`")
    lib = ctypes.CDLL(str(p))
    vp, u16p, f32p, i32p = (ctypes.c_void_p,) * 4
    i32, f32, sz = ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    lib.kda_fwd.restype = ctypes.c_int
    lib.kda_fwd.argtypes = [u16p, u16p, u16p, u16p, u16p, f32p, f32p, f32, f32, f32p, f32p, i32p,
                            i32, i32, i32, i32, i32, i32, u16p, vp, sz, vp]
    lib.gdn_fwd.restype = ctypes.c_int
    lib.gdn_fwd.argtypes = [u16p, u16p, u16p, f32p, u16p, f32, f32p, f32p, i32p, i32, i32, i32,
                            i32, i32, i32, u16p, vp, sz, vp]
    lib.kda_fwd_split.restype = ctypes.c_int
    lib.kda_fwd_split.argtypes = [u16p, u16p, u16p, u16p, u16p, f32p, f32p, f32, f32, f32p, f32p,
                                  i32p, i32, i32, i32, i32, i32, i32, u16p, vp, sz, i32, vp]
    lib.gdn_fwd_split.restype = ctypes.c_int
    lib.gdn_fwd_split.argtypes = [u16p, u16p, u16p, f32p, u16p, f32, f32p, f32p, i32p, i32, i32,
                                  i32, i32, i32, i32, u16p, vp, sz, i32, vp]
    lib.kda_fwd_split_workspace_size.restype = ctypes.c_size_t
    lib.kda_fwd_split_workspace_size.argtypes = [i32] * 7
    lib.kda_fwd_segmented_workspace_size.restype = ctypes.c_size_t
    lib.kda_fwd_segmented_workspace_size.argtypes = [i32] * 7
    # the segmented forms take the segment length before the stream, the timed
    # forms two event handles after it
    lib.kda_fwd_segmented.restype = ctypes.c_int
    lib.kda_fwd_segmented.argtypes = lib.kda_fwd_split.argtypes
    lib.gdn_fwd_segmented.restype = ctypes.c_int
    lib.gdn_fwd_segmented.argtypes = lib.gdn_fwd_split.argtypes
    lib.kda_fwd_noalloc.restype = ctypes.c_int
    lib.kda_fwd_noalloc.argtypes = lib.kda_fwd.argtypes[:19] + [vp]
    lib.kda_fwd_timed.restype = ctypes.c_int
    lib.kda_fwd_timed.argtypes = lib.kda_fwd.argtypes + [vp, vp]
    lib.gdn_fwd_timed.restype = ctypes.c_int
    lib.gdn_fwd_timed.argtypes = lib.gdn_fwd.argtypes + [vp, vp]
    lib.kda_prep.restype = ctypes.c_int
    lib.kda_prep.argtypes = [u16p, u16p, u16p, u16p, f32p, f32p, f32, i32p, i32, i32, i32, i32,
                             i32, i32, vp, sz, vp]
    lib.gdn_prep.restype = ctypes.c_int
    lib.gdn_prep.argtypes = [u16p, u16p, f32p, u16p, i32p, i32, i32, i32, i32, i32, i32, vp, sz,
                             vp]
    lib.kda_recur.restype = ctypes.c_int
    lib.kda_recur.argtypes = [u16p, f32, f32p, f32p, i32, i32, i32, i32, i32, i32, i32, u16p, vp,
                              sz, vp]
    lib.kda_decode.restype = ctypes.c_int
    lib.kda_decode.argtypes = [u16p, u16p, u16p, u16p, u16p, f32p, f32p, f32, f32, f32p, f32p,
                               i32, i32, i32, i32, u16p, vp]
    lib.gdn_decode.restype = ctypes.c_int
    lib.gdn_decode.argtypes = [u16p, u16p, u16p, f32p, u16p, f32, f32p, f32p, i32, i32, i32, i32,
                               u16p, vp]
    lib.kda_bwd.restype = ctypes.c_int
    lib.kda_bwd.argtypes = [u16p, u16p, u16p, u16p, u16p, f32p, f32p, f32, f32, f32p, i32p,
                            i32, i32, i32, i32, i32, i32, u16p, f32p, u16p, u16p, u16p, u16p,
                            u16p, f32p, f32p, f32p, vp, sz, vp]
    lib.gdn_bwd.restype = ctypes.c_int
    lib.gdn_bwd.argtypes = [u16p, u16p, u16p, f32p, u16p, f32, f32p, i32p, i32, i32, i32, i32,
                            i32, i32, u16p, f32p, u16p, u16p, u16p, f32p, u16p, f32p, vp, sz, vp]
    # the measurement forms of the stages take two event handles more
    lib.kda_prep_timed.restype = ctypes.c_int
    lib.kda_prep_timed.argtypes = lib.kda_prep.argtypes + [vp, vp]
    lib.kda_recur_timed.restype = ctypes.c_int
    lib.kda_recur_timed.argtypes = lib.kda_recur.argtypes + [vp, vp]
    # the training pair shares the signatures of kda_fwd / gdn_fwd and kda_bwd / gdn_bwd
    for a, b in (("kda_fwd_save", "kda_fwd"), ("gdn_fwd_save", "gdn_fwd"),
                 ("kda_bwd_saved", "kda_bwd"), ("gdn_bwd_saved", "gdn_bwd")):
        getattr(lib, a).restype = ctypes.c_int
        getattr(lib, a).argtypes = getattr(lib, b).argtypes
    for name in ("kda_fwd_workspace_size", "gdn_fwd_workspace_size", "kda_bwd_workspace_size"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_size_t
        fn.argtypes = [i32] * 6
    lib.kda_status_str.restype = ctypes.c_char_p
    lib.kda_status_str.argtypes = [ctypes.c_int]
    lib.kda_version.restype = ctypes.c_int
    lib.kda_version.argtypes = []
    if path is None:
        _lib = lib
    return lib


def status_str(status: int) -> str:
    return load().kda_status_str(int(status)).decode()


def version() -> int:
    return int(load().kda_version())


def workspace_size(B, T, H, K, V, num_seqs=None, kind="kda", segment_chunks=None,
                   path="fused") -> int:
    """Workspace bytes of the single-launch forward pass (path "fused": kda_fwd,
    kda_fwd_segmented) or of the two-stage one (path "staged": kda_fwd_split;
    segment_chunks=-1 also sizes kda_prep / kda_recur).  0: unsupported sizes."""
    n = B if num_seqs is None else num_seqs
    seg = 0 if segment_chunks is None else int(segment_chunks)
    if path == "staged":
        return int(load().kda_fwd_split_workspace_size(B, T, H, K, V, n, seg))
    if path != "fused":
        raise ValueError(f"unknown path {path!r}")
    if segment_chunks is not None:
        return int(load().kda_fwd_segmented_workspace_size(B, T, H, K, V, n, seg))
    fn = load().kda_fwd_workspace_size if kind == "kda" else load().gdn_fwd_workspace_size
    return int(fn(B, T, H, K, V, n))


# ---------------------------------------------------------------- marshalling
def _torch():
    import torch

    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtype, shape=None, device=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _shapes(q, k, v, beta, scale, initial_state, cu_seqlens):
    """Checks of the forward inputs; returns (B, T, H, K, V, N, scale)."""
    torch = _torch()
    _need(q, "q", torch.bfloat16)
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, K]")
    dev = q.device
    B, T, H, K = q.shape
    _need(k, "k", torch.bfloat16, (B, T, H, K), dev)
    if v.dim() != 4:
        raise ValueError("v must be [B, T, H, V]")
    V = v.shape[3]
    _need(v, "v", torch.bfloat16, (B, T, H, V), dev)
    _need(beta, "beta", torch.bfloat16, (B, T, H), dev)
    N = B
    if cu_seqlens is not None:
        _need(cu_seqlens, "cu_seqlens", torch.int32, None, dev)
        if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
            raise ValueError("cu_seqlens must be 1-D with num_seqs + 1 entries")
        if B != 1:
            raise ValueError("cu_seqlens needs B == 1 (sequences packed along T)")
        N = cu_seqlens.numel() - 1
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32, (N, H, K, V), dev)
    if scale is None:
        scale = K ** -0.5
    return B, T, H, K, V, N, float(scale)


def _prepare(q, k, v, beta, scale, initial_state, output_final_state, cu_seqlens, workspace,
             kind, out=None, final_out=None, segment_chunks=None, path="fused"):
    torch = _torch()
    B, T, H, K, V, N, scale = _shapes(q, k, v, beta, scale, initial_state, cu_seqlens)
    dev = q.device
    if out is None:
        out = torch.empty((B, T, H, V), dtype=torch.bfloat16, device=dev)
    else:
        _need(out, "out", torch.bfloat16, (B, T, H, V), dev)
    o = out
    final = None
    if output_final_state:
        if final_out is None:
            final_out = torch.empty((N, H, K, V), dtype=torch.float32, device=dev)
        else:
            _need(final_out, "final_out", torch.float32, (N, H, K, V), dev)
        final = final_out
    need = workspace_size(B, T, H, K, V, N, kind, segment_chunks, path)
    if need == 0:
        raise LibKdaError(2, status_str(2))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    elif workspace.numel() * workspace.element_size() < need or workspace.device != dev:
        raise LibKdaError(3, status_str(3))
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    return dict(B=B, T=T, H=H, K=K, V=V, N=N, scale=float(scale), o=o, final=final,
                workspace=workspace, stream=stream)


def _kda_gate_checks(g, A_log, dt_bias, B, T, H, K, dev):
    torch = _torch()
    _need(g, "g", torch.bfloat16, (B, T, H, K), dev)
    _need(A_log, "A_log", torch.float32, (H,), dev)
    _need(dt_bias, "dt_bias", torch.float32, None, dev)
    if dt_bias.numel() != H * K:
        raise ValueError("dt_bias must hold H * K values ([H, K] or [H * K])")


def kda_fwd(q, k, v, g, beta, A_log, dt_bias, lower_bound=-5.0, scale=None, initial_state=None,
            output_final_state=True, cu_seqlens=None, workspace=None, out=None,
            final_out=None, segment_chunks=None, events=None):
    """KDA forward on the GPU (the single-launch pass).  q, k, g [B,T,H,K] bf16;
    v [B,T,H,V] bf16; beta logits [B,T,H] bf16; A_log [H] fp32; dt_bias [H,K] (or
    [H*K]) fp32; initial_state [N,H,K,V] fp32 or None; cu_seqlens int32 [N+1] or
    None (B must then be 1).  ``workspace``, ``out`` and ``final_out`` optionally
    supply preallocated device buffers.  ``segment_chunks`` (None: automatic)
    sets the sequence segments (kda_fwd_segmented); ``events`` = (start, stop)
    torch.cuda.Event records the kernel's own start and end (kda_fwd_timed).
    Returns (o [B,T,H,V] bf16, final_state [N,H,K,V] fp32 or None)."""
    a = _prepare(q, k, v, beta, scale, initial_state, output_final_state, cu_seqlens,
                 workspace, "kda", out, final_out, segment_chunks)
    B, T, H, K = a["B"], a["T"], a["H"], a["K"]
    _kda_gate_checks(g, A_log, dt_bias, B, T, H, K, q.device)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(A_log), _ptr(dt_bias),
            float(lower_bound), a["scale"], _ptr(initial_state), _ptr(a["final"]),
            _ptr(cu_seqlens), a["N"], B, T, H, K, a["V"], _ptr(a["o"]), _ptr(a["workspace"]),
            _nbytes(a["workspace"]))
    if events is not None:
        if segment_chunks is not None:
            raise ValueError("events time the automatic segments only")
        st = load().kda_fwd_timed(*args, a["stream"], *_events(events))
    elif segment_chunks is not None:
        st = load().kda_fwd_segmented(*args, int(segment_chunks), a["stream"])
    else:
        st = load().kda_fwd(*args, a["stream"])
    if st != 0:
        raise LibKdaError(st, status_str(st))
    return a["o"], a["final"]


NOALLOC_SCRATCH_BYTES = 4 << 20  # KDA_NOALLOC_SCRATCH_BYTES of include/kda.h


def kda_fwd_noalloc(q, k, v, g, beta, A_log, dt_bias, out, final_out=None, lower_bound=-5.0,
                    scale=None, initial_state=None, cu_seqlens=None):
    """kda_fwd through kda_fwd_noalloc: allocates nothing (no workspace, no
    outputs: ``out`` [B,T,H,V] bf16 and ``final_out`` [N,H,K,V] fp32 or None
    are written in place).  Packed batches keep their tables in the library's
    per-GPU scratch array; calls overlapping in time on one GPU race on it."""
    torch = _torch()
    B, T, H, K, V, N, scale = _shapes(q, k, v, beta, scale, initial_state, cu_seqlens)
    dev = q.device
    _need(out, "out", torch.bfloat16, (B, T, H, V), dev)
    if final_out is not None:
        _need(final_out, "final_out", torch.float32, (N, H, K, V), dev)
    _kda_gate_checks(g, A_log, dt_bias, B, T, H, K, dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    st = load().kda_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(A_log),
                                _ptr(dt_bias), float(lower_bound), float(scale),
                                _ptr(initial_state), _ptr(final_out), _ptr(cu_seqlens), N, B, T,
                                H, K, V, _ptr(out), stream)
    if st == 3 and cu_seqlens is not None:
        raise LibKdaError(st, f"the packed batch's tables need more than the "
                              f"{NOALLOC_SCRATCH_BYTES} bytes of the library's scratch array; "
                              f"use kda_fwd with a workspace")
    if st != 0:
        raise LibKdaError(st, status_str(st))
    return out, final_out


def gdn_fwd(q, k, v, g, beta, scale=None, initial_state=None, output_final_state=True,
            cu_seqlens=None, workspace=None, out=None, final_out=None, segment_chunks=None,
            events=None):
    """GDN forward on the GPU (the single-launch pass).  g is the fp32 log decay
    [B,T,H] (<= 0); beta are probabilities [B,T,H] bf16, used as given.  Other
    arguments as kda_fwd."""
    torch = _torch()
    a = _prepare(q, k, v, beta, scale, initial_state, output_final_state, cu_seqlens,
                 workspace, "gdn", out, final_out, segment_chunks)
    B, T, H = a["B"], a["T"], a["H"]
    _need(g, "g", torch.float32, (B, T, H), q.device)
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), a["scale"], _ptr(initial_state),
            _ptr(a["final"]), _ptr(cu_seqlens), a["N"], B, T, H, a["K"], a["V"], _ptr(a["o"]),
            _ptr(a["workspace"]), _nbytes(a["workspace"]))
    if events is not None:
        if segment_chunks is not None:
            raise ValueError("events time the automatic segments only")
        st = load().gdn_fwd_timed(*args, a["stream"], *_events(events))
    elif segment_chunks is not None:
        st = load().gdn_fwd_segmented(*args, int(segment_chunks), a["stream"])
    else:
        st = load().gdn_fwd(*args, a["stream"])
    if st != 0:
        raise LibKdaError(st, status_str(st))
    return a["o"], a["final"]


def kda_fwd_split(q, k, v, g, beta, A_log, dt_bias, lower_bound=-5.0, scale=None,
                  initial_state=None, output_final_state=True, cu_seqlens=None, workspace=None,
                  out=None, final_out=None, segment_chunks=0):
    """The two-stage KDA forward (kda_prep then kda_recur, records in the
    workspace) with its sequence splitting: segment_chunks < 0 never, 0
    automatic, > 0 segments of that many chunks.  Arguments as kda_fwd."""
    a = _prepare(q, k, v, beta, scale, initial_state, output_final_state, cu_seqlens,
                 workspace, "kda", out, final_out, segment_chunks, path="staged")
    B, T, H, K = a["B"], a["T"], a["H"], a["K"]
    _kda_gate_checks(g, A_log, dt_bias, B, T, H, K, q.device)
    st = load().kda_fwd_split(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(A_log),
                              _ptr(dt_bias), float(lower_bound), a["scale"], _ptr(initial_state),
                              _ptr(a["final"]), _ptr(cu_seqlens), a["N"], B, T, H, K, a["V"],
                              _ptr(a["o"]), _ptr(a["workspace"]), _nbytes(a["workspace"]),
                              int(segment_chunks), a["stream"])
    if st != 0:
        raise LibKdaError(st, status_str(st))
    return a["o"], a["final"]


def gdn_fwd_split(q, k, v, g, beta, scale=None, initial_state=None, output_final_state=True,
                  cu_seqlens=None, workspace=None, out=None, final_out=None, segment_chunks=0):
    """The two-stage GDN forward with its sequence splitting (see kda_fwd_split)."""
    torch = _torch()
    a = _prepare(q, k, v, beta, scale, initial_state, output_final_state, cu_seqlens,
                 workspace, "gdn", out, final_out, segment_chunks, path="staged")
    B, T, H = a["B"], a["T"], a["H"]
    _need(g, "g", torch.float32, (B, T, H), q.device)
    st = load().gdn_fwd_split(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), a["scale"],
                              _ptr(initial_state), _ptr(a["final"]), _ptr(cu_seqlens), a["N"],
                              B, T, H, a["K"], a["V"], _ptr(a["o"]), _ptr(a["workspace"]),
                              _nbytes(a["workspace"]), int(segment_chunks), a["stream"])
    if st != 0:
        raise LibKdaError(st, status_str(st))
    return a["o"], a["final"]


def _save_workspace(q, v, cu_seqlens, workspace):
    """A backward-sized workspace for the *_fwd_save calls (checked or allocated)."""
    torch = _torch()
    B, T, H, K = q.shape
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    need = bwd_workspace_size(B, T, H, K, v.shape[3], N)
    if need == 0:
        raise LibKdaError(2, status_str(2))
    if workspace is None:
        return torch.empty(need, dtype=torch.uint8, device=q.device)
    if _nbytes(workspace) < need or workspace.device != q.device:
        raise LibKdaError(3, status_str(3))
    return workspace


def kda_fwd_save(q, k, v, g, beta, A_log, dt_bias, lower_bound=-5.0, scale=None,
                 initial_state=None, output_final_state=True, cu_seqlens=None, workspace=None,
                 out=None, final_out=None):
    """kda_fwd that also leaves in ``workspace`` (backward-sized; allocated when
    None) what kda_bwd_saved needs.  Returns (o, final_state or None, workspace)."""
    torch = _torch()
    ws = _save_workspace(q, v, cu_seqlens, workspace)
    a = _prepare(q, k, v, beta, scale, initial_state, output_final_state, cu_seqlens, ws,
                 "kda", out, final_out, -1)
    B, T, H, K = a["B"], a["T"], a["H"], a["K"]
    _need(g, "g", torch.bfloat16, (B, T, H, K), q.device)
    _need(A_log, "A_log", torch.float32, (H,), q.device)
    _need(dt_bias, "dt_bias", torch.float32, None, q.device)
    if dt_bias.numel() != H * K:
        raise ValueError("dt_bias must hold H * K values ([H, K] or [H * K])")
    _check(load().kda_fwd_save(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(A_log),
                               _ptr(dt_bias), float(lower_bound), a["scale"], _ptr(initial_state),
                               _ptr(a["final"]), _ptr(cu_seqlens), a["N"], B, T, H, K, a["V"],
                               _ptr(a["o"]), _ptr(ws), _nbytes(ws), a["stream"]))
    return a["o"], a["final"], ws


def gdn_fwd_save(q, k, v, g, beta, scale=None, initial_state=None, output_final_state=True,
                 cu_seqlens=None, workspace=None, out=None, final_out=None):
    """gdn_fwd that also leaves in ``workspace`` what gdn_bwd_saved needs.
    Returns (o, final_state or None, workspace)."""
    torch = _torch()
    ws = _save_workspace(q, v, cu_seqlens, workspace)
    a = _prepare(q, k, v, beta, scale, initial_state, output_final_state, cu_seqlens, ws,
                 "gdn", out, final_out, -1)
    B, T, H = a["B"], a["T"], a["H"]
    _need(g, "g", torch.float32, (B, T, H), q.device)
    _check(load().gdn_fwd_save(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), a["scale"],
                               _ptr(initial_state), _ptr(a["final"]), _ptr(cu_seqlens), a["N"],
                               B, T, H, a["K"], a["V"], _ptr(a["o"]), _ptr(ws), _nbytes(ws),
                               a["stream"]))
    return a["o"], a["final"], ws


def _check(st):
    if st != 0:
        raise LibKdaError(st, status_str(st))


def _nbytes(t):
    return t.numel() * t.element_size()


def _events(events):
    """(start, stop) torch.cuda.Event pair (timing enabled, recorded once so the
    underlying events exist) -> two raw handles; None -> two NULLs."""
    if events is None:
        return ctypes.c_void_p(0), ctypes.c_void_p(0)
    start, stop = events
    if not start.cuda_event or not stop.cuda_event:
        raise ValueError("record() each event once before passing it (the handle is created then)")
    return ctypes.c_void_p(start.cuda_event), ctypes.c_void_p(stop.cuda_event)


def kda_prep(q, k, g, beta, A_log, dt_bias, lower_bound, workspace, cu_seqlens=None, V=None,
             events=None):
    """Token-parallel stage only: fills ``workspace`` (see kda_recur).  ``events``
    = (start, stop) torch.cuda.Event: the record kernel's own start and end are
    recorded into them (kda_prep_timed)."""
    B, T, H, K = q.shape
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    stream = ctypes.c_void_p(_torch().cuda.current_stream(q.device).cuda_stream)
    _check(load().kda_prep_timed(_ptr(q), _ptr(k), _ptr(g), _ptr(beta), _ptr(A_log),
                                 _ptr(dt_bias), float(lower_bound), _ptr(cu_seqlens), N, B, T, H,
                                 K, V or K, _ptr(workspace), _nbytes(workspace), stream,
                                 *_events(events)))


def gdn_prep(q, k, g, beta, workspace, cu_seqlens=None, V=None):
    B, T, H, K = q.shape
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    stream = ctypes.c_void_p(_torch().cuda.current_stream(q.device).cuda_stream)
    _check(load().gdn_prep(_ptr(q), _ptr(k), _ptr(g), _ptr(beta), _ptr(cu_seqlens), N, B, T, H,
                           K, V or K, _ptr(workspace), _nbytes(workspace), stream))


def kda_recur(v, K, scale, workspace, out, initial_state=None, final_out=None, num_seqs=None,
              events=None):
    """Head-parallel stage only: reads the workspace of the preceding prep call
    (same sizes and packing; ``num_seqs`` set for packed sequences).  ``events``
    as for kda_prep (kda_recur_timed: the recurrence kernel's start and end)."""
    B, T, H, V = v.shape
    varlen = num_seqs is not None
    N = num_seqs if varlen else B
    stream = ctypes.c_void_p(_torch().cuda.current_stream(v.device).cuda_stream)
    _check(load().kda_recur_timed(_ptr(v), float(scale), _ptr(initial_state), _ptr(final_out),
                                  1 if varlen else 0, N, B, T, H, K, V, _ptr(out),
                                  _ptr(workspace), _nbytes(workspace), stream,
                                  *_events(events)))


def _decode_prepare(q, k, v, beta, scale, state, state_out, out):
    torch = _torch()
    _need(q, "q", torch.bfloat16)
    if q.dim() != 3:
        raise ValueError("q must be [N, H, K]")
    dev = q.device
    N, H, K = q.shape
    _need(k, "k", torch.bfloat16, (N, H, K), dev)
    if v.dim() != 3:
        raise ValueError("v must be [N, H, V]")
    V = v.shape[2]
    _need(v, "v", torch.bfloat16, (N, H, V), dev)
    _need(beta, "beta", torch.bfloat16, (N, H), dev)
    if state is not None:
        _need(state, "state", torch.float32, (N, H, K, V), dev)
    if state_out is None:
        state_out = torch.empty((N, H, K, V), dtype=torch.float32, device=dev)
    else:
        _need(state_out, "state_out", torch.float32, (N, H, K, V), dev)
    if out is None:
        out = torch.empty((N, H, V), dtype=torch.bfloat16, device=dev)
    else:
        _need(out, "out", torch.bfloat16, (N, H, V), dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    return N, H, K, V, float(K ** -0.5 if scale is None else scale), state_out, out, stream


def kda_decode(q, k, v, g, beta, A_log, dt_bias, lower_bound=-5.0, scale=None, state=None,
               state_out=None, out=None):
    """One KDA step for N sequences: q, k, g [N,H,K] bf16; v [N,H,V] bf16; beta logits
    [N,H] bf16; state [N,H,K,V] fp32 or None (zeros).  ``state_out`` may be ``state``
    (update in place).  Returns (o [N,H,V] bf16, new state [N,H,K,V] fp32)."""
    torch = _torch()
    N, H, K, V, sc, so, o, stream = _decode_prepare(q, k, v, beta, scale, state, state_out, out)
    _need(g, "g", torch.bfloat16, (N, H, K), q.device)
    _need(A_log, "A_log", torch.float32, (H,), q.device)
    _need(dt_bias, "dt_bias", torch.float32, None, q.device)
    if dt_bias.numel() != H * K:
        raise ValueError("dt_bias must hold H * K values ([H, K] or [H * K])")
    _check(load().kda_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(A_log),
                             _ptr(dt_bias), float(lower_bound), sc, _ptr(state), _ptr(so), N, H,
                             K, V, _ptr(o), stream))
    return o, so


def gdn_decode(q, k, v, g, beta, scale=None, state=None, state_out=None, out=None):
    """One GDN step: g is the fp32 log decay [N,H]; beta probabilities [N,H] bf16."""
    torch = _torch()
    N, H, K, V, sc, so, o, stream = _decode_prepare(q, k, v, beta, scale, state, state_out, out)
    _need(g, "g", torch.float32, (N, H), q.device)
    _check(load().gdn_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), sc, _ptr(state),
                             _ptr(so), N, H, K, V, _ptr(o), stream))
    return o, so


# ---------------------------------------------------------------- backward
def bwd_workspace_size(B, T, H, K, V, num_seqs=None) -> int:
    return int(load().kda_bwd_workspace_size(B, T, H, K, V, B if num_seqs is None else num_seqs))


def _bwd_prepare(q, k, v, beta, do, scale, initial_state, dfinal, cu_seqlens, workspace,
                 need_dh0):
    torch = _torch()
    B, T, H, K, V, N, scale = _shapes(q, k, v, beta, scale, initial_state, cu_seqlens)
    a = dict(B=B, T=T, H=H, K=K, V=V, N=N, scale=scale,
             stream=ctypes.c_void_p(torch.cuda.current_stream(q.device).cuda_stream))
    dev = q.device
    _need(do, "do", torch.bfloat16, (B, T, H, V), dev)
    if dfinal is not None:
        _need(dfinal, "dfinal", torch.float32, (N, H, K, V), dev)
    need = bwd_workspace_size(B, T, H, K, V, N)
    if need == 0:
        raise LibKdaError(2, status_str(2))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    elif _nbytes(workspace) < need or workspace.device != dev:
        raise LibKdaError(3, status_str(3))
    out = {"dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
           "dbeta": torch.empty_like(beta),
           "dh0": torch.empty((N, H, K, V), dtype=torch.float32, device=dev) if need_dh0 else None}
    a.update(workspace=workspace, out=out)
    return a


def kda_bwd_saved(q, k, v, g, beta, A_log, dt_bias, do, workspace, lower_bound=-5.0, scale=None,
                  initial_state=None, dfinal=None, cu_seqlens=None, need_dh0=True):
    """kda_bwd reusing the ``workspace`` a kda_fwd_save call on the same inputs
    filled (its chunk records and states are not recomputed)."""
    return kda_bwd(q, k, v, g, beta, A_log, dt_bias, do, lower_bound, scale, initial_state,
                   dfinal, cu_seqlens, workspace, need_dh0, _saved=True)


def kda_bwd(q, k, v, g, beta, A_log, dt_bias, do, lower_bound=-5.0, scale=None,
            initial_state=None, dfinal=None, cu_seqlens=None, workspace=None, need_dh0=True,
            _saved=False):
    """Gradients of kda_fwd for dL/do = ``do`` [B,T,H,V] bf16 and dL/d(final state) =
    ``dfinal`` [N,H,K,V] fp32 (None: zero).  Returns a dict with dq, dk [B,T,H,K],
    dv [B,T,H,V], dg [B,T,H,K], dbeta [B,T,H] (bf16), dA_log [H], ddt_bias [H,K]
    and dh0 [N,H,K,V] (fp32; None unless ``need_dh0``)."""
    torch = _torch()
    a = _bwd_prepare(q, k, v, beta, do, scale, initial_state, dfinal, cu_seqlens, workspace,
                     need_dh0)
    B, T, H, K, V, N = (a[x] for x in "BTHKVN")
    dev = q.device
    _need(g, "g", torch.bfloat16, (B, T, H, K), dev)
    _need(A_log, "A_log", torch.float32, (H,), dev)
    _need(dt_bias, "dt_bias", torch.float32, None, dev)
    if dt_bias.numel() != H * K:
        raise ValueError("dt_bias must hold H * K values ([H, K] or [H * K])")
    o = a["out"]
    o["dg"] = torch.empty_like(g)
    o["dA_log"] = torch.empty((H,), dtype=torch.float32, device=dev)
    o["ddt_bias"] = torch.empty((H, K), dtype=torch.float32, device=dev)
    ws = a["workspace"]
    fn = load().kda_bwd_saved if _saved else load().kda_bwd
    _check(fn(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(A_log), _ptr(dt_bias),
              float(lower_bound), a["scale"], _ptr(initial_state), _ptr(cu_seqlens), N, B, T, H,
              K, V, _ptr(do), _ptr(dfinal), _ptr(o["dq"]), _ptr(o["dk"]), _ptr(o["dv"]),
              _ptr(o["dg"]), _ptr(o["dbeta"]), _ptr(o["dA_log"]), _ptr(o["ddt_bias"]),
              _ptr(o["dh0"]), _ptr(ws), _nbytes(ws), a["stream"]))
    return o


def gdn_bwd_saved(q, k, v, g, beta, do, workspace, scale=None, initial_state=None, dfinal=None,
                  cu_seqlens=None, need_dh0=True):
    """gdn_bwd reusing the ``workspace`` a gdn_fwd_save call on the same inputs filled."""
    return gdn_bwd(q, k, v, g, beta, do, scale, initial_state, dfinal, cu_seqlens, workspace,
                   need_dh0, _saved=True)


def gdn_bwd(q, k, v, g, beta, do, scale=None, initial_state=None, dfinal=None, cu_seqlens=None,
            workspace=None, need_dh0=True, _saved=False):
    """Gradients of gdn_fwd: dict with dq, dk, dv, dbeta (bf16), dg [B,T,H] and dh0
    (fp32).  Arguments as kda_bwd."""
    torch = _torch()
    a = _bwd_prepare(q, k, v, beta, do, scale, initial_state, dfinal, cu_seqlens, workspace,
                     need_dh0)
    B, T, H, K, V, N = (a[x] for x in "BTHKVN")
    _need(g, "g", torch.float32, (B, T, H), q.device)
    o = a["out"]
    o["dg"] = torch.empty_like(g)
    ws = a["workspace"]
    fn = load().gdn_bwd_saved if _saved else load().gdn_bwd
    _check(fn(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), a["scale"], _ptr(initial_state),
              _ptr(cu_seqlens), N, B, T, H, K, V, _ptr(do), _ptr(dfinal), _ptr(o["dq"]),
              _ptr(o["dk"]), _ptr(o["dv"]), _ptr(o["dg"]), _ptr(o["dbeta"]), _ptr(o["dh0"]),
              _ptr(ws), _nbytes(ws), a["stream"]))
    return o
