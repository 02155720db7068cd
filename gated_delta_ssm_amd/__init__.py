"""Python binding of libgdn.so, the gfx950 gated-delta SSM layer core.

Argument marshalling only: each function below takes torch tensors that
already live on the GPU, checks dtype/device/layout, and passes raw device
pointers, element strides and the current HIP stream to the C entry point of
the same name (declared in include/gdn.h).  Every step of the computation runs
in the library's HIP kernels; there is no fallback.  Importing this module
fails loudly if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; "
                      "g.build()'` (or gated_delta_ssm_amd/_build.py) first")

_lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_I = ctypes.c_int
_L = ctypes.c_int64
_F = ctypes.c_float
_SZ = ctypes.c_size_t

_SIGS = {
    "gdn_strerror": (ctypes.c_char_p, [_I]),
    "gdn_version": (_I, []),
    "gdn_decay_gate": (_I, [_P, _P, _P, _P, _I, _I, _P]),
    "gdn_conv1d_silu_l2norm": (_I, [_P, _L, _L, _P, _P, _L, _P, _L, _L, _P, _L, _L,
                                    _I, _I, _I, _I, _I, _I, _F, _P]),
    "gdn_recurrence_decode": (_I, [_P, _L, _P, _P, _L, _L, _P, _L, _L, _P, _P, _P, _L, _L,
                                   _P, _L, _I, _I, _I, _I, _I, _F, _P]),
    "gdn_recurrence_chunked_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I, _I]),
    "gdn_recurrence_chunked": (_I, [_P, _L, _P, _P, _L, _L, _P, _L, _L, _P, _P, _P, _L, _L,
                                    _I, _I, _I, _I, _I, _F, _I, _P, _SZ, _P]),
    "gdn_prefill_chunked_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I, _I]),
    "gdn_prefill_chunked": (_I, [_P, _L, _P, _L, _L, _P, _P, _L, _P, _P, _P, _P, _P, _L, _L,
                                 _I, _I, _I, _I, _I, _I, _F, _F, _I, _P, _SZ, _P]),
    "gdn_recurrence_chunked_varlen_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I, _I]),
    "gdn_recurrence_chunked_varlen": (_I, [_P, _L, _P, _P, _L, _P, _L, _I, _P, _P, _P, _L,
                                           _P, _I, _I, _I, _I, _I, _F, _I, _P, _SZ, _P]),
    "gdn_mamba2_ssd_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I, _I]),
    "gdn_mamba2_ssd_chunked": (_I, [_P, _L, _P, _L, _L, _P, _P, _L, _L, _P, _L, _L, _P, _P, _P,
                                    _P, _L, _L, _I, _I, _I, _I, _I, _I, _F, _F, _I, _P, _SZ,
                                    _P]),
    "gdn_gated_rmsnorm": (_I, [_P, _L, _P, _P, _L, _P, _L, _I, _I, _I, _F, _P]),
    "gdn_stream_copy": (_I, [_P, _P, _SZ, _P]),
    "gdn_decode_fused": (_I, [_P, _L, _P, _P, _L, _L, _P, _L, _L, _P, _P, _P, _P, _P, _P, _L,
                              _L, _P, _L, _L, _P, _P, _L, _L, _P, _L, _I, _I, _I, _I, _I, _F,
                              _F, _P]),
    "gdn_decode_step_workspace_bytes": (_SZ, [_I, _I]),
    "gdn_decode_step": (_I, [_P, _L, _P, _L, _L, _P, _P, _L, _P, _L, _L, _P, _P, _P, _P, _P,
                             _P, _L, _L, _P, _L, _L, _P, _P, _L, _L, _P, _L, _I, _I, _I, _I,
                             _I, _I, _F, _F, _F, _P, _SZ, _P]),
    "gdn_decode_step_noalloc": (_I, [_P, _L, _P, _L, _L, _P, _P, _L, _P, _L, _L, _P, _P, _P, _P,
                                     _P, _P, _L, _L, _P, _L, _L, _P, _P, _L, _L, _P, _L, _I, _I,
                                     _I, _I, _I, _I, _F, _F, _F, _P]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTS = tuple(_SIGS)


class GdnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {_lib.gdn_strerror(status).decode()} (status {status})")


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise GdnError(fn, status)


def _ptr(t: torch.Tensor | None):
    return None if t is None else t.data_ptr()


# The raw-stream query skips building a torch Stream object on every call
# (about 3 us per launch); torch.cuda.current_stream is the documented route
# when the private query is absent.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream, like: torch.Tensor) -> int:
    """HIP stream handle: `stream` if given, else the current stream of the
    device that holds `like`."""
    if stream is None:
        if _raw_stream is not None:
            return _raw_stream(like.get_device())
        return torch.cuda.current_stream(like.device).cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


_F32 = torch.float32


def _dev_f32(name: str, t: torch.Tensor, inner_contig: int) -> None:
    """fp32 on a GPU, with the innermost `inner_contig` dims densely packed."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype is not _F32:
        raise TypeError(f"{name} must be float32, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    shape, stride = t.shape, t.stride()
    expect = 1
    for d in range(len(shape) - 1, len(shape) - 1 - inner_contig, -1):
        if shape[d] > 1 and stride[d] != expect:
            raise ValueError(f"{name}: innermost {inner_contig} dims must be dense, "
                             f"got strides {stride}")
        expect *= shape[d]


def version() -> int:
    return _lib.gdn_version()


def gdn_decay_gate(alpha: torch.Tensor, dt: torch.Tensor, a: torch.Tensor,
                   g: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """g[r][h] = a[h] * softplus(alpha[r][h] + dt[h]); alpha, g [rows][H] dense."""
    rows, H = alpha.shape
    if g is None:
        g = torch.empty_like(alpha)
    for n, t in (("alpha", alpha), ("dt", dt), ("a", a), ("g", g)):
        _dev_f32(n, t, t.dim())
    _check("gdn_decay_gate", _lib.gdn_decay_gate(_ptr(alpha), _ptr(dt), _ptr(a), _ptr(g),
                                                 rows, H, _stream(stream, g)))
    return g


def gdn_conv1d_silu_l2norm(x: torch.Tensor, w: torch.Tensor, conv_state: torch.Tensor,
                           out: torch.Tensor, *, qk_channels: int, head_dim: int,
                           l2_eps: float, snap: torch.Tensor | None = None,
                           stream=None) -> torch.Tensor:
    """Conv1d + SiLU (+ L2 on Q/K channels) over x [n_seq][n_tok][conv_dim] (any
    row strides), rolling conv_state [n_seq][conv_dim][d_conv-1] in place, into
    out [n_seq][n_tok][conv_dim]; snap [n_seq][n_tok-1][conv_dim][d_conv-1]."""
    n_seq, n_tok, C = out.shape
    D = w.shape[1]
    if x.shape != out.shape:
        raise ValueError(f"x {tuple(x.shape)} and out {tuple(out.shape)} differ")
    if w.shape[0] != C or tuple(conv_state.shape) != (n_seq, C, D - 1):
        raise ValueError("conv weight / state shape mismatch")
    _dev_f32("x", x, 1)
    _dev_f32("out", out, 1)
    _dev_f32("w", w, 2)
    _dev_f32("conv_state", conv_state, 2)
    sn_tok = sn_seq = 0
    if snap is not None:
        _dev_f32("snap", snap, 2)
        if tuple(snap.shape) != (n_seq, n_tok - 1, C, D - 1):
            raise ValueError("snap shape mismatch")
        sn_seq, sn_tok = snap.stride(0), snap.stride(1)
    _check("gdn_conv1d_silu_l2norm", _lib.gdn_conv1d_silu_l2norm(
        _ptr(x), x.stride(1), x.stride(0), _ptr(w), _ptr(conv_state), conv_state.stride(0),
        _ptr(out), out.stride(1), out.stride(0), _ptr(snap), sn_tok, sn_seq,
        n_seq, n_tok, C, D, qk_channels, head_dim, l2_eps, _stream(stream, out)))
    return out


def _recur_check(state, q, k, v, g, beta, y):
    n_seq, n_tok, Hk, S = q.shape
    H = v.shape[2]
    if tuple(state.shape) != (n_seq, H, S, S) or k.shape != q.shape:
        raise ValueError("state / q / k shape mismatch")
    if tuple(v.shape) != (n_seq, n_tok, H, S) or y.shape != v.shape:
        raise ValueError("v / y shape mismatch")
    if tuple(g.shape) != (n_seq, n_tok, H) or beta.shape != g.shape:
        raise ValueError("g / beta shape mismatch")
    _dev_f32("state", state, 3)
    for n, t in (("q", q), ("k", k), ("v", v), ("y", y)):
        _dev_f32(n, t, 2)
    if q.stride() != k.stride():
        raise ValueError("q and k must share strides")
    _dev_f32("g", g, 3)
    _dev_f32("beta", beta, 3)
    return n_seq, n_tok, H, Hk, S


def gdn_recurrence_decode(state: torch.Tensor, q: torch.Tensor, k: torch.Tensor,
                          v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
                          y: torch.Tensor, *, scale: float, snap: torch.Tensor | None = None,
                          stream=None) -> torch.Tensor:
    """Token-by-token recurrence.  state [n_seq][H][S][S] (value-major, updated
    in place), q, k [n_seq][n_tok][Hk][S], v, y [n_seq][n_tok][H][S], g, beta
    [n_seq][n_tok][H]; snap [n_seq][n_tok-1][H][S][S] or None."""
    n_seq, n_tok, H, Hk, S = _recur_check(state, q, k, v, g, beta, y)
    sn_seq = 0
    if snap is not None:
        _dev_f32("snap", snap, 4)
        if tuple(snap.shape) != (n_seq, n_tok - 1, H, S, S):
            raise ValueError("snap shape mismatch")
        sn_seq = snap.stride(0)
    _check("gdn_recurrence_decode", _lib.gdn_recurrence_decode(
        _ptr(state), state.stride(0), _ptr(q), _ptr(k), q.stride(1), q.stride(0),
        _ptr(v), v.stride(1), v.stride(0), _ptr(g), _ptr(beta), _ptr(y), y.stride(1),
        y.stride(0), _ptr(snap), sn_seq, n_seq, n_tok, H, Hk, S, scale, _stream(stream, y)))
    return y


def gdn_recurrence_chunked_workspace_bytes(n_seq: int, n_tok: int, n_v_heads: int,
                                           n_qk_heads: int, S: int, chunk: int = 64) -> int:
    return int(_lib.gdn_recurrence_chunked_workspace_bytes(n_seq, n_tok, n_v_heads,
                                                           n_qk_heads, S, chunk))


def gdn_recurrence_chunked(state: torch.Tensor, q: torch.Tensor, k: torch.Tensor,
                           v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
                           y: torch.Tensor, *, scale: float, chunk: int = 64,
                           workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Chunked (WY/UT) form of the recurrence; same layouts as decode.  If no
    workspace is given one is allocated here through torch."""
    n_seq, n_tok, H, Hk, S = _recur_check(state, q, k, v, g, beta, y)
    need = gdn_recurrence_chunked_workspace_bytes(n_seq, n_tok, H, Hk, S, chunk)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=state.device)
    _check("gdn_recurrence_chunked", _lib.gdn_recurrence_chunked(
        _ptr(state), state.stride(0), _ptr(q), _ptr(k), q.stride(1), q.stride(0),
        _ptr(v), v.stride(1), v.stride(0), _ptr(g), _ptr(beta), _ptr(y), y.stride(1),
        y.stride(0), n_seq, n_tok, H, Hk, S, scale, chunk, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream, y)))
    return y


def gdn_prefill_chunked_workspace_bytes(n_seq: int, n_tok: int, n_v_heads: int,
                                        n_qk_heads: int, S: int, chunk: int = 64) -> int:
    return int(_lib.gdn_prefill_chunked_workspace_bytes(n_seq, n_tok, n_v_heads, n_qk_heads, S,
                                                        chunk))


def gdn_prefill_chunked(state: torch.Tensor, x: torch.Tensor, conv_w: torch.Tensor,
                        conv_state: torch.Tensor, alpha: torch.Tensor, dt: torch.Tensor,
                        a: torch.Tensor, beta: torch.Tensor, y: torch.Tensor, *, scale: float,
                        l2_eps: float, chunk: int = 64, workspace: torch.Tensor | None = None,
                        stream=None) -> torch.Tensor:
    """Decay gate + conv1d/SiLU/L2 + chunked recurrence in two launches.
    state [n_seq][H][S][S] (in place); x [n_seq][n_tok][>= conv_dim] with
    conv_dim = (2*Hk + H)*S channels q | k | v; conv_w [conv_dim][d_conv];
    conv_state [n_seq][conv_dim][d_conv-1] rolled in place; alpha, beta
    [n_seq][n_tok][H]; dt, a [H]; y [n_seq][n_tok][H][S].  If no workspace
    is given one is allocated here through torch."""
    n_seq, H, S, _ = state.shape
    C, D = conv_w.shape
    if C % S or (C // S - H) < 2 or (C // S - H) % 2:
        raise ValueError(f"conv_dim {C} is not (2*Hk + H)*S for H={H}, S={S}")
    Hk = (C // S - H) // 2
    if x.dim() != 3 or x.shape[0] != n_seq or x.shape[2] < C:
        raise ValueError("x shape mismatch")
    n_tok = x.shape[1]
    if tuple(conv_state.shape) != (n_seq, C, D - 1):
        raise ValueError("conv_state shape mismatch")
    if tuple(alpha.shape) != (n_seq, n_tok, H) or beta.shape != alpha.shape:
        raise ValueError("alpha / beta shape mismatch")
    if tuple(dt.shape) != (H,) or tuple(a.shape) != (H,):
        raise ValueError("dt / a shape mismatch")
    if tuple(y.shape) != (n_seq, n_tok, H, S):
        raise ValueError("y shape mismatch")
    _dev_f32("state", state, 3)
    _dev_f32("x", x, 1)
    _dev_f32("conv_w", conv_w, 2)
    _dev_f32("conv_state", conv_state, 2)
    _dev_f32("y", y, 2)
    for n, t in (("alpha", alpha), ("beta", beta)):
        _dev_f32(n, t, 3)
    for n, t in (("dt", dt), ("a", a)):
        _dev_f32(n, t, 1)
    need = gdn_prefill_chunked_workspace_bytes(n_seq, n_tok, H, Hk, S, chunk)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=state.device)
    _check("gdn_prefill_chunked", _lib.gdn_prefill_chunked(
        _ptr(state), state.stride(0), _ptr(x), x.stride(1), x.stride(0), _ptr(conv_w),
        _ptr(conv_state), conv_state.stride(0), _ptr(alpha), _ptr(dt), _ptr(a), _ptr(beta),
        _ptr(y), y.stride(1), y.stride(0), n_seq, n_tok, H, Hk, S, D, scale, l2_eps, chunk,
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream, y)))
    return y


def gdn_recurrence_chunked_varlen_workspace_bytes(n_seq: int, total_tok: int, n_v_heads: int,
                                                  n_qk_heads: int, S: int,
                                                  chunk: int = 64) -> int:
    return int(_lib.gdn_recurrence_chunked_varlen_workspace_bytes(n_seq, total_tok, n_v_heads,
                                                                  n_qk_heads, S, chunk))


def gdn_recurrence_chunked_varlen(state: torch.Tensor, q: torch.Tensor, k: torch.Tensor,
                                  v: torch.Tensor, g: torch.Tensor, beta: torch.Tensor,
                                  y: torch.Tensor, cu_seqlens, *, scale: float, chunk: int = 64,
                                  workspace: torch.Tensor | None = None,
                                  stream=None) -> torch.Tensor:
    """Chunked recurrence over a packed batch of sequences of different lengths.
    state [n_seq][H][S][S] (updated in place), q, k [total][Hk][S], v, y
    [total][H][S], g, beta [total][H]; cu_seqlens: n_seq + 1 row offsets on the
    host (a list or a CPU integer tensor).  q, k, v are float32 or bfloat16
    (all three the same); everything else is float32.  If no workspace is
    given one is allocated here through torch."""
    cu = [int(c) for c in (cu_seqlens.tolist() if isinstance(cu_seqlens, torch.Tensor)
                           else cu_seqlens)]
    n_seq = len(cu) - 1
    total, Hk, S = q.shape
    H = v.shape[1]
    if n_seq < 1 or tuple(state.shape) != (n_seq, H, S, S) or k.shape != q.shape:
        raise ValueError("state / q / k / cu_seqlens shape mismatch")
    if tuple(v.shape) != (total, H, S) or y.shape != v.shape:
        raise ValueError("v / y shape mismatch")
    if tuple(g.shape) != (total, H) or beta.shape != g.shape:
        raise ValueError("g / beta shape mismatch")
    _dev_f32("state", state, 3)
    _dev_f32("y", y, 2)
    in_dtype = q.dtype
    if in_dtype not in (torch.float32, torch.bfloat16) or k.dtype != in_dtype or \
            v.dtype != in_dtype:
        raise TypeError(f"q, k, v must all be float32 or all bfloat16, got "
                        f"{q.dtype}, {k.dtype}, {v.dtype}")
    for n, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda:
            raise ValueError(f"{n} must be on the GPU")
        if (t.shape[2] > 1 and t.stride(2) != 1) or (t.shape[1] > 1 and t.stride(1) != t.shape[2]):
            raise ValueError(f"{n}: innermost 2 dims must be dense, got strides {t.stride()}")
    if q.stride() != k.stride():
        raise ValueError("q and k must share strides")
    _dev_f32("g", g, 2)
    _dev_f32("beta", beta, 2)
    dt_code = 1 if in_dtype == torch.bfloat16 else 0
    cu_arr = (ctypes.c_int32 * (n_seq + 1))(*cu)
    need = gdn_recurrence_chunked_varlen_workspace_bytes(n_seq, total, H, Hk, S, chunk)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=state.device)
    _check("gdn_recurrence_chunked_varlen", _lib.gdn_recurrence_chunked_varlen(
        _ptr(state), state.stride(0), _ptr(q), _ptr(k), q.stride(0), _ptr(v), v.stride(0),
        dt_code, _ptr(g), _ptr(beta), _ptr(y), y.stride(0), ctypes.cast(cu_arr, _P), n_seq,
        total, H,
        Hk, S, scale, chunk, _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream, y)))
    return y


def gdn_mamba2_ssd_workspace_bytes(n_seq: int, n_tok: int, n_heads: int, head_dim: int,
                                   d_state: int, chunk: int = 64) -> int:
    return int(_lib.gdn_mamba2_ssd_workspace_bytes(n_seq, n_tok, n_heads, head_dim, d_state,
                                                   chunk))


def gdn_mamba2_ssd_chunked(state: torch.Tensor, x: torch.Tensor, B: torch.Tensor,
                           C: torch.Tensor, dt_raw: torch.Tensor, A_log: torch.Tensor,
                           D: torch.Tensor, dt_bias: torch.Tensor, y: torch.Tensor, *,
                           dt_min: float, dt_max: float, chunk: int = 64,
                           workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Mamba-2 selective scan, chunked.  state [n_seq][H][P][N] (in place),
    x, y [n_seq][T][H][P], B, C [n_seq][T][G][N] (same strides), dt_raw
    [n_seq][T][H], A_log, D, dt_bias [H].  If no workspace is given one is
    allocated here through torch."""
    n_seq, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    if tuple(state.shape) != (n_seq, H, P, N) or y.shape != x.shape or C.shape != B.shape:
        raise ValueError("state / x / y / B / C shape mismatch")
    if tuple(B.shape[:2]) != (n_seq, T) or tuple(dt_raw.shape) != (n_seq, T, H):
        raise ValueError("B / dt_raw shape mismatch")
    for n, t in (("A_log", A_log), ("D", D), ("dt_bias", dt_bias)):
        if tuple(t.shape) != (H,):
            raise ValueError(f"{n} must have shape [H]")
        _dev_f32(n, t, 1)
    _dev_f32("state", state, 3)
    for n, t in (("x", x), ("y", y), ("B", B), ("C", C)):
        _dev_f32(n, t, 2)
    _dev_f32("dt_raw", dt_raw, 1)
    if B.stride() != C.stride():
        raise ValueError("B and C must share strides")
    need = gdn_mamba2_ssd_workspace_bytes(n_seq, T, H, P, N, chunk)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=state.device)
    _check("gdn_mamba2_ssd_chunked", _lib.gdn_mamba2_ssd_chunked(
        _ptr(state), state.stride(0), _ptr(x), x.stride(1), x.stride(0), _ptr(B), _ptr(C),
        B.stride(1), B.stride(0), _ptr(dt_raw), dt_raw.stride(1), dt_raw.stride(0),
        _ptr(A_log), _ptr(D), _ptr(dt_bias), _ptr(y), y.stride(1), y.stride(0), n_seq, T, H, G,
        P, N, dt_min, dt_max, chunk, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream, y)))
    return y


def gdn_gated_rmsnorm(y: torch.Tensor, w: torch.Tensor, z: torch.Tensor, out: torch.Tensor,
                      *, eps: float, stream=None) -> torch.Tensor:
    """out = ((y * rsqrt(mean(y^2) + eps)) * w) * silu(z) per (row, head);
    y, z, out [rows][H][head_dim] with dense heads and any row stride."""
    rows, H, hd = y.shape
    if z.shape != y.shape or out.shape != y.shape or tuple(w.shape) != (hd,):
        raise ValueError("norm shape mismatch")
    for n, t in (("y", y), ("z", z), ("out", out)):
        _dev_f32(n, t, 2)
    _dev_f32("w", w, 1)
    _check("gdn_gated_rmsnorm", _lib.gdn_gated_rmsnorm(
        _ptr(y), y.stride(0), _ptr(w), _ptr(z), z.stride(0), _ptr(out), out.stride(0),
        rows, H, hd, eps, _stream(stream, out)))
    return out


def gdn_decode_fused(state: torch.Tensor, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                     alpha: torch.Tensor, dt: torch.Tensor, a: torch.Tensor,
                     beta: torch.Tensor, norm_w: torch.Tensor, z: torch.Tensor,
                     out: torch.Tensor, *, scale: float, norm_eps: float,
                     g: torch.Tensor | None = None, y: torch.Tensor | None = None,
                     snap: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Decay gate -> recurrence -> gated RMSNorm in one launch.  Layouts as
    gdn_recurrence_decode; alpha, beta [n_seq][n_tok][H]; dt, a [H]; norm_w [S];
    z, out [n_seq][n_tok][H][S]; optional g [n_seq][n_tok][H] and pre-norm y
    [n_seq][n_tok][H][S] outputs; optional snap as gdn_recurrence_decode."""
    n_seq, n_tok, Hk, S = q.shape
    H = v.shape[2]
    if tuple(state.shape) != (n_seq, H, S, S) or k.shape != q.shape:
        raise ValueError("state / q / k shape mismatch")
    if tuple(v.shape) != (n_seq, n_tok, H, S) or out.shape != v.shape or z.shape != v.shape:
        raise ValueError("v / z / out shape mismatch")
    if tuple(alpha.shape) != (n_seq, n_tok, H) or beta.shape != alpha.shape:
        raise ValueError("alpha / beta shape mismatch")
    if tuple(dt.shape) != (H,) or tuple(a.shape) != (H,) or tuple(norm_w.shape) != (S,):
        raise ValueError("dt / a / norm_w shape mismatch")
    _dev_f32("state", state, 3)
    for n, t in (("q", q), ("k", k), ("v", v), ("z", z), ("out", out)):
        _dev_f32(n, t, 2)
    if q.stride() != k.stride():
        raise ValueError("q and k must share strides")
    for n, t in (("alpha", alpha), ("beta", beta)):
        _dev_f32(n, t, 3)
    for n, t in (("dt", dt), ("a", a), ("norm_w", norm_w)):
        _dev_f32(n, t, 1)
    y_tok = y_seq = 0
    if g is not None:
        _dev_f32("g", g, 3)
        if g.shape != alpha.shape:
            raise ValueError("g shape mismatch")
    if y is not None:
        _dev_f32("y", y, 2)
        if y.shape != v.shape:
            raise ValueError("y shape mismatch")
        y_seq, y_tok = y.stride(0), y.stride(1)
    sn_seq = 0
    if snap is not None:
        _dev_f32("snap", snap, 4)
        if tuple(snap.shape) != (n_seq, n_tok - 1, H, S, S):
            raise ValueError("snap shape mismatch")
        sn_seq = snap.stride(0)
    _check("gdn_decode_fused", _lib.gdn_decode_fused(
        _ptr(state), state.stride(0), _ptr(q), _ptr(k), q.stride(1), q.stride(0),
        _ptr(v), v.stride(1), v.stride(0), _ptr(alpha), _ptr(dt), _ptr(a), _ptr(beta),
        _ptr(norm_w), _ptr(z), z.stride(1), z.stride(0), _ptr(out), out.stride(1),
        out.stride(0), _ptr(g), _ptr(y), y_tok, y_seq, _ptr(snap), sn_seq, n_seq, n_tok, H,
        Hk, S, scale, norm_eps, _stream(stream, out)))
    return out


def gdn_decode_step_workspace_bytes(n_seq: int, n_qk_heads: int) -> int:
    return int(_lib.gdn_decode_step_workspace_bytes(n_seq, n_qk_heads))


def _step_args(state, x, conv_w, conv_state, alpha, dt, a, beta, norm_w, z, out, scale,
               l2_eps, norm_eps, g, y, snap, conv_snap):
    """Checks and the C arguments of the one-launch decode step up to (not
    including) its workspace arguments; also returns (n_seq, Hk)."""
    n_seq, H, S, _ = state.shape
    C, D = conv_w.shape
    if C % S or (C // S - H) < 2 or (C // S - H) % 2:
        raise ValueError(f"conv_dim {C} is not (2*Hk + H)*S for H={H}, S={S}")
    Hk = (C // S - H) // 2
    n_tok = x.shape[1]
    if x.dim() != 3 or x.shape[0] != n_seq or x.shape[2] < C:
        raise ValueError("x shape mismatch")
    if tuple(conv_state.shape) != (n_seq, C, D - 1):
        raise ValueError("conv_state shape mismatch")
    if tuple(out.shape) != (n_seq, n_tok, H, S) or z.shape != out.shape:
        raise ValueError("z / out shape mismatch")
    if tuple(alpha.shape) != (n_seq, n_tok, H) or beta.shape != alpha.shape:
        raise ValueError("alpha / beta shape mismatch")
    if tuple(dt.shape) != (H,) or tuple(a.shape) != (H,) or tuple(norm_w.shape) != (S,):
        raise ValueError("dt / a / norm_w shape mismatch")
    _dev_f32("state", state, 3)
    _dev_f32("x", x, 1)
    _dev_f32("conv_w", conv_w, 2)
    _dev_f32("conv_state", conv_state, 2)
    for n, t in (("z", z), ("out", out)):
        _dev_f32(n, t, 2)
    for n, t in (("alpha", alpha), ("beta", beta)):
        _dev_f32(n, t, 3)
    for n, t in (("dt", dt), ("a", a), ("norm_w", norm_w)):
        _dev_f32(n, t, 1)
    y_tok = y_seq = 0
    if g is not None:
        _dev_f32("g", g, 3)
        if g.shape != alpha.shape:
            raise ValueError("g shape mismatch")
    if y is not None:
        _dev_f32("y", y, 2)
        if y.shape != out.shape:
            raise ValueError("y shape mismatch")
        y_seq, y_tok = y.stride(0), y.stride(1)
    sn_seq = 0
    if snap is not None:
        _dev_f32("snap", snap, 4)
        if tuple(snap.shape) != (n_seq, n_tok - 1, H, S, S):
            raise ValueError("snap shape mismatch")
        sn_seq = snap.stride(0)
    cs_tok = cs_seq = 0
    if conv_snap is not None:
        _dev_f32("conv_snap", conv_snap, 2)
        if tuple(conv_snap.shape) != (n_seq, n_tok - 1, C, D - 1):
            raise ValueError("conv_snap shape mismatch")
        cs_seq, cs_tok = conv_snap.stride(0), conv_snap.stride(1)
    args = (_ptr(state), state.stride(0), _ptr(x), x.stride(1), x.stride(0), _ptr(conv_w),
            _ptr(conv_state), conv_state.stride(0), _ptr(conv_snap), cs_tok, cs_seq, _ptr(alpha),
            _ptr(dt), _ptr(a), _ptr(beta), _ptr(norm_w), _ptr(z), z.stride(1), z.stride(0),
            _ptr(out), out.stride(1), out.stride(0), _ptr(g), _ptr(y), y_tok, y_seq, _ptr(snap),
            sn_seq, n_seq, n_tok, H, Hk, S, D, scale, l2_eps, norm_eps)
    return args, n_seq, Hk


def gdn_decode_step(state: torch.Tensor, x: torch.Tensor, conv_w: torch.Tensor,
                    conv_state: torch.Tensor, alpha: torch.Tensor, dt: torch.Tensor,
                    a: torch.Tensor, beta: torch.Tensor, norm_w: torch.Tensor, z: torch.Tensor,
                    out: torch.Tensor, *, scale: float, l2_eps: float, norm_eps: float,
                    workspace: torch.Tensor | None = None, g: torch.Tensor | None = None,
                    y: torch.Tensor | None = None, snap: torch.Tensor | None = None,
                    conv_snap: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Conv1d + SiLU + L2 -> decay gate -> recurrence -> gated RMSNorm in one
    launch.  x [n_seq][n_tok][>= conv_dim] (any row strides) with conv_dim =
    (2*Hk + H)*S channels q | k | v; conv_w [conv_dim][d_conv]; conv_state
    [n_seq][conv_dim][d_conv-1] rolled in place; the other tensors as
    gdn_decode_fused; conv_snap [n_seq][n_tok-1][conv_dim][d_conv-1].
    workspace: int32 counters, zero before first use and left zero by every
    call (allocated zeroed here when None)."""
    args, n_seq, Hk = _step_args(state, x, conv_w, conv_state, alpha, dt, a, beta, norm_w, z,
                                 out, scale, l2_eps, norm_eps, g, y, snap, conv_snap)
    need = gdn_decode_step_workspace_bytes(n_seq, Hk)
    if workspace is None:
        workspace = torch.zeros(max(need, 4) // 4, dtype=torch.int32, device=state.device)
    _check("gdn_decode_step", _lib.gdn_decode_step(
        *args, _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream, out)))
    return out


NOALLOC_SCRATCH_BYTES = 65536   # GDN_NOALLOC_SCRATCH_BYTES


def gdn_decode_step_noalloc(state: torch.Tensor, x: torch.Tensor, conv_w: torch.Tensor,
                            conv_state: torch.Tensor, alpha: torch.Tensor, dt: torch.Tensor,
                            a: torch.Tensor, beta: torch.Tensor, norm_w: torch.Tensor,
                            z: torch.Tensor, out: torch.Tensor, *, scale: float, l2_eps: float,
                            norm_eps: float, g: torch.Tensor | None = None,
                            y: torch.Tensor | None = None, snap: torch.Tensor | None = None,
                            conv_snap: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """gdn_decode_step with its ticket counters in the library's own device
    array (no workspace, nothing allocated here or in the library); calls on
    one GPU share that array, so they must not overlap in time."""
    args, _, _ = _step_args(state, x, conv_w, conv_state, alpha, dt, a, beta, norm_w, z, out,
                            scale, l2_eps, norm_eps, g, y, snap, conv_snap)
    _check("gdn_decode_step_noalloc", _lib.gdn_decode_step_noalloc(*args, _stream(stream, out)))
    return out


def gdn_stream_copy(dst: torch.Tensor, src: torch.Tensor, stream=None) -> torch.Tensor:
    """Non-temporal device copy of src into dst (same byte size, 16-byte
    aligned): the achievable-bandwidth reference of the benchmark."""
    nb = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nb or not (src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("src and dst must be contiguous and of the same byte size")
    if not (src.is_cuda and dst.is_cuda):
        raise ValueError("src and dst must be on the GPU")
    _check("gdn_stream_copy", _lib.gdn_stream_copy(_ptr(dst), _ptr(src), nb, _stream(stream, dst)))
    return dst
