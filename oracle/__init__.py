"""fp64 CPU oracle for the gated delta-rule forward pass (KDA and GDN).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU library
never calls it, and it shares no code with the GPU library: the two meet only
through seeded inputs produced by ``chunked_gated_delta_kda_amd.inputs``.

``kda_oracle.c`` is the token-by-token recurrence (the definition).
``chunked.py`` is an independent fp64 NumPy implementation of the chunkwise
(WY / UT-transform) form, used to pin the recurrence and to serve as the
reference for chunk-level intermediates.

Parity status: pinned.  Every function here is checked in
``tests/test_oracle_pins.py`` against closed forms, invariants, brute force
and hand-worked examples (``tests/golden/``), and
``tests/test_oracle_mutants.py`` shows that planted mistakes in the C source
fail at least one of those pins.  No page prints numerical outputs, so there
is no page value to compare against.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import tempfile
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
SOURCE = _HERE / "kda_oracle.c"
BUILD_DIR = _HERE / "_build"
DEFAULT_LIB = BUILD_DIR / "libkda_oracle.so"


def build(src: Path = SOURCE, out: Path = DEFAULT_LIB, extra_flags=()) -> Path:
    """Compile the C oracle with gcc (fp64, OpenMP) into a shared library."""
    out = Path(out)
    out.parent.mkdir(parents=True, exist_ok=True)
    fd, tmp = tempfile.mkstemp(suffix=".so", dir=str(out.parent))
    os.close(fd)
    cmd = ["gcc", "-std=c99", "-O2", "-fopenmp", "-fPIC", "-shared", *extra_flags,
           str(src), "-o", tmp, "-lm"]
    try:
        subprocess.run(cmd, check=True, capture_output=True, text=True)
        os.replace(tmp, out)
    except subprocess.CalledProcessError as e:  # pragma: no cover - toolchain failure
        os.unlink(tmp)
        raise RuntimeError(f"oracle build failed: {' '.join(cmd)}\n{e.stderr}") from e
    return out


def _is_torch(x) -> bool:
    return type(x).__module__.startswith("torch")


def _f64(x, heads=None, axis=None):
    """Exact up-cast of a numpy array or torch tensor to contiguous float64,
    optionally keeping only the given head indices along ``axis``."""
    if x is None:
        return None
    if _is_torch(x):
        import torch

        t = x.detach()
        if heads is not None:
            t = t.index_select(axis, torch.as_tensor(heads, dtype=torch.long, device=t.device))
        return np.ascontiguousarray(t.to("cpu", torch.float64).numpy())
    a = np.asarray(x)
    if heads is not None:
        a = np.take(a, heads, axis=axis)
    return np.ascontiguousarray(a, dtype=np.float64)


def _i64(x):
    if x is None:
        return None
    if _is_torch(x):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(x), dtype=np.int64)


_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int64)


def _ptr(a, kind=_dp):
    return None if a is None else a.ctypes.data_as(kind)


class Oracle:
    """ctypes front end of one compiled copy of ``kda_oracle.c``."""

    def __init__(self, lib_path: Path | str | None = None):
        if lib_path is None:
            if not DEFAULT_LIB.exists() or DEFAULT_LIB.stat().st_mtime < SOURCE.stat().st_mtime:
                build()
            lib_path = DEFAULT_LIB
        self.lib = ctypes.CDLL(str(lib_path))
        f = self.lib.kda_oracle_forward
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.c_int, _dp, _dp, _dp, _dp, _dp, _dp, _dp, ctypes.c_double,
                      ctypes.c_double, _dp, _dp, _ip, ctypes.c_int64, ctypes.c_int64,
                      ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _dp,
                      ctypes.c_int]
        self.lib.kda_oracle_max_threads.restype = ctypes.c_int

    def max_threads(self) -> int:
        return int(self.lib.kda_oracle_max_threads())

    def _run(self, gdn, q, k, v, g, beta, A_log, dt_bias, lower_bound, scale, initial_state,
             output_final_state, cu_seqlens, heads, threads):
        q, k, v = _f64(q, heads, 2), _f64(k, heads, 2), _f64(v, heads, 2)
        g, beta = _f64(g, heads, 2), _f64(beta, heads, 2)
        A_log = None if gdn else _f64(A_log, heads, 0)
        if not gdn:
            # [H,K] and flat [H*K] name the same memory
            dt = _f64(dt_bias).reshape(-1, q.shape[-1])
            dt_bias = np.ascontiguousarray(dt if heads is None else dt[list(heads)])
        h0 = _f64(initial_state, heads, 1)
        cu = _i64(cu_seqlens)
        B, T, H, K = q.shape
        V = v.shape[-1]
        N = (len(cu) - 1) if cu is not None else B
        if scale is None:
            scale = K ** -0.5
        o = np.zeros((B, T, H, V), dtype=np.float64)
        hT = np.zeros((N, H, K, V), dtype=np.float64) if output_final_state else None
        rc = self.lib.kda_oracle_forward(
            1 if gdn else 0, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(A_log),
            _ptr(dt_bias), float(lower_bound), float(scale), _ptr(h0), _ptr(hT),
            _ptr(cu, _ip), N, B, T, H, K, V, _ptr(o), int(threads or 0))
        if rc != 0:
            raise ValueError("oracle rejected its arguments")
        return o, hT

    def kda(self, q, k, v, g, beta, A_log, dt_bias, lower_bound=-5.0, scale=None,
            initial_state=None, output_final_state=True, cu_seqlens=None, heads=None,
            threads=0):
        """KDA forward: g is the pre-activation gate [B,T,H,K], beta are logits.
        Returns (o [B,T,H',V], final_state [N,H',K,V] or None), H' = len(heads)."""
        return self._run(False, q, k, v, g, beta, A_log, dt_bias, lower_bound, scale,
                         initial_state, output_final_state, cu_seqlens, heads, threads)

    def gdn(self, q, k, v, g, beta, scale=None, initial_state=None, output_final_state=True,
            cu_seqlens=None, heads=None, threads=0):
        """GDN forward: g is the log-decay [B,T,H] (one scalar per head and token),
        beta are probabilities in (0,1) used as given."""
        return self._run(True, q, k, v, g, beta, None, None, 0.0, scale, initial_state,
                         output_final_state, cu_seqlens, heads, threads)


_default: Oracle | None = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def kda_fwd(*args, **kwargs):
    return default().kda(*args, **kwargs)


def gdn_fwd(*args, **kwargs):
    return default().gdn(*args, **kwargs)
