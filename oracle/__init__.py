"""Plain fp64 CPU oracle for the gated-delta SSM layer core.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, the smoke check and the
benchmark's CPU-baseline leg.  The HIP library and its Python binding never
import it, and it imports nothing from them.

The arithmetic lives in ``gdn_oracle.c`` (built with gcc into
``liboracle.so``); this module only widens fp32 arrays to fp64, converts the
GPU's transposed state layout, and calls the C functions through ctypes.
Each wrapper names the C function whose header comment cites the pages.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(verbose: bool = False) -> str:
    """Compile gdn_oracle.c with gcc (fp64, no fast-math, OpenMP)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-Wall", "-Wextra", "-o", LIB_PATH + ".tmp", _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        build()
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    I = ctypes.c_int
    L = ctypes.c_long
    D = ctypes.c_double
    lib.oracle_decay_gate.argtypes = [P, P, P, P, L, I]
    lib.oracle_conv1d_silu_l2norm.argtypes = [P, P, P, P, P, I, I, I, I, I, I, D]
    lib.oracle_recurrence_seq.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, D]
    lib.oracle_recurrence_chunked.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, D]
    lib.oracle_gated_rmsnorm.argtypes = [P, P, P, P, L, I, I, D]
    lib.oracle_mamba2_dt.argtypes = [P, P, P, L, I, D, D]
    lib.oracle_mamba2_ssd_seq.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I]
    lib.oracle_mamba2_ssd_chunked.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I]
    lib.oracle_max_threads.restype = I
    lib.oracle_set_threads.argtypes = [I]
    for f in (lib.oracle_decay_gate, lib.oracle_conv1d_silu_l2norm, lib.oracle_recurrence_seq,
              lib.oracle_recurrence_chunked, lib.oracle_gated_rmsnorm, lib.oracle_set_threads,
              lib.oracle_mamba2_dt, lib.oracle_mamba2_ssd_seq, lib.oracle_mamba2_ssd_chunked):
        f.restype = None
    _lib = lib
    return lib


def _f64(x) -> np.ndarray:
    """Widen to a C-contiguous fp64 copy (exact for fp32 inputs)."""
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def max_threads() -> int:
    return _load().oracle_max_threads()


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def decay_gate(alpha, dt, a) -> np.ndarray:
    """oracle_decay_gate: alpha [rows][H], dt [H], a [H] -> g [rows][H] (fp64)."""
    alpha, dt, a = _f64(alpha), _f64(dt), _f64(a)
    rows, H = alpha.shape
    g = np.empty((rows, H), np.float64)
    _load().oracle_decay_gate(_p(alpha), _p(dt), _p(a), _p(g), rows, H)
    return g


def conv1d_silu_l2norm(x, w, hist, qk_channels: int, head_dim: int, eps: float,
                       want_snap: bool = False):
    """oracle_conv1d_silu_l2norm.

    x [n_seq][n_tok][C], w [C][d], hist [n_seq][C][d-1] (not modified).
    Returns (out [n_seq][n_tok][C], new_hist, snap [n_seq][n_tok-1][C][d-1] or None).
    """
    x, w = _f64(x), _f64(w)
    hist = _f64(hist).copy()
    n_seq, n_tok, C = x.shape
    d = w.shape[1]
    out = np.empty_like(x)
    snap = np.zeros((n_seq, max(n_tok - 1, 0), C, d - 1)) if want_snap else None
    _load().oracle_conv1d_silu_l2norm(_p(x), _p(w), _p(hist), _p(out),
                                      _p(snap) if snap is not None else None,
                                      n_seq, n_tok, C, d, qk_channels, head_dim, float(eps))
    return out, hist, snap


def _state_to_kv(state_vk) -> np.ndarray:
    """[..][H][dv][dk] (the GPU's transposed layout) -> [..][H][dk][dv] fp64."""
    return np.ascontiguousarray(np.swapaxes(_f64(state_vk), -1, -2))


def recurrence_seq(state_vk, q, k, v, g, beta, scale: float, want_snap: bool = False):
    """oracle_recurrence_seq on the GPU layout.

    state_vk [n_seq][H][dv][dk]; q, k [n_seq][n_tok][Hk][dk]; v [n_seq][n_tok][H][dv];
    g, beta [n_seq][n_tok][H].  Returns (y [n_seq][n_tok][H][dv], new state in the
    same [dv][dk] layout, snap [n_seq][n_tok-1][H][dv][dk] or None).
    """
    S = _state_to_kv(state_vk)
    q, k, v, g, beta = _f64(q), _f64(k), _f64(v), _f64(g), _f64(beta)
    n_seq, n_tok, Hk, dk = q.shape
    H, dv = v.shape[2], v.shape[3]
    y = np.empty((n_seq, n_tok, H, dv))
    snap = np.zeros((n_seq, max(n_tok - 1, 0), H, dk, dv)) if want_snap else None
    _load().oracle_recurrence_seq(_p(S), _p(q), _p(k), _p(v), _p(g), _p(beta), _p(y),
                                  _p(snap) if snap is not None else None,
                                  n_seq, n_tok, H, Hk, dk, dv, float(scale))
    snap_vk = np.swapaxes(snap, -1, -2) if snap is not None else None
    return y, np.swapaxes(S, -1, -2), snap_vk


def recurrence_chunked(state_vk, q, k, v, g, beta, scale: float, chunk: int = 64):
    """oracle_recurrence_chunked on the GPU layout; returns (y, new state)."""
    S = _state_to_kv(state_vk)
    q, k, v, g, beta = _f64(q), _f64(k), _f64(v), _f64(g), _f64(beta)
    n_seq, n_tok, Hk, dk = q.shape
    H, dv = v.shape[2], v.shape[3]
    y = np.empty((n_seq, n_tok, H, dv))
    _load().oracle_recurrence_chunked(_p(S), _p(q), _p(k), _p(v), _p(g), _p(beta), _p(y),
                                      n_seq, n_tok, H, Hk, dk, dv, int(chunk), float(scale))
    return y, np.swapaxes(S, -1, -2)


def gated_rmsnorm(y, w, z, eps: float) -> np.ndarray:
    """oracle_gated_rmsnorm: y, z [rows][H][hd], w [hd] -> out [rows][H][hd]."""
    y, w, z = _f64(y), _f64(w), _f64(z)
    rows, H, hd = y.shape
    out = np.empty_like(y)
    _load().oracle_gated_rmsnorm(_p(y), _p(w), _p(z), _p(out), rows, H, hd, float(eps))
    return out


def mamba2_dt(dt_raw, dt_bias, dt_min: float, dt_max: float) -> np.ndarray:
    """oracle_mamba2_dt: dt_raw [rows][H], dt_bias [H] -> dt [rows][H] (fp64)."""
    dt_raw, dt_bias = _f64(dt_raw), _f64(dt_bias)
    shape = dt_raw.shape
    H = shape[-1]
    rows = dt_raw.size // H
    out = np.empty(shape, np.float64)
    _load().oracle_mamba2_dt(_p(dt_raw), _p(dt_bias), _p(out), rows, H, float(dt_min),
                             float(dt_max))
    return out


def _ssd_args(state, x, Bm, Cm, dt, A_log, D):
    st = _f64(state).copy()
    x, Bm, Cm, dt, D = _f64(x), _f64(Bm), _f64(Cm), _f64(dt), _f64(D)
    A = -np.exp(_f64(A_log))
    n_seq, T, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    return st, x, Bm, Cm, dt, A, D, n_seq, T, H, G, P, N


def mamba2_ssd_seq(state, x, Bm, Cm, dt, A_log, D):
    """oracle_mamba2_ssd_seq: state [n][H][P][N], x [n][T][H][P], Bm, Cm [n][T][G][N],
    dt [n][T][H] (already clamped), A_log, D [H].  Returns (y, new state), fp64."""
    st, x, Bm, Cm, dt, A, D, n_seq, T, H, G, P, N = _ssd_args(state, x, Bm, Cm, dt, A_log, D)
    y = np.empty_like(x)
    _load().oracle_mamba2_ssd_seq(_p(st), _p(x), _p(Bm), _p(Cm), _p(dt), _p(A), _p(D), _p(y),
                                  n_seq, T, H, G, P, N)
    return y, st


def mamba2_ssd_chunked(state, x, Bm, Cm, dt, A_log, D, chunk: int = 64):
    """oracle_mamba2_ssd_chunked: same arguments and results as mamba2_ssd_seq."""
    st, x, Bm, Cm, dt, A, D, n_seq, T, H, G, P, N = _ssd_args(state, x, Bm, Cm, dt, A_log, D)
    y = np.empty_like(x)
    _load().oracle_mamba2_ssd_chunked(_p(st), _p(x), _p(Bm), _p(Cm), _p(dt), _p(A), _p(D),
                                      _p(y), n_seq, T, H, G, P, N, int(chunk))
    return y, st
