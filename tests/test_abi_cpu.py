"""CPU-side checks of the C ABI: the library loads, exports every entry point
include/gdn.h declares, and rejects invalid arguments on the host, before any
HIP call (so these run without a GPU; nothing here computes)."""
import ctypes
import os
import re

import pytest

import gated_delta_ssm_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("gdn.h", "gdn_measure.h")]

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUP, ERR_ALIAS, ERR_WS, ERR_SCRATCH = 0, -1, -2, -3, -4, -5, -7
FAKE = 0x10000            # never dereferenced: validation rejects first
L = gdn._lib


def declared():
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z0-9_]+)\s*\(", text)))


def test_header_declarations_all_exported():
    names = declared()
    assert "gdn_recurrence_decode" in names and len(names) >= 8
    for n in names:
        assert hasattr(L, n), f"{n} declared in gdn.h but not exported"
    assert set(names) == set(gdn.EXPORTS)


def test_strerror_and_version():
    for s in (0, -1, -2, -3, -4, -5, -6, -7):
        assert len(L.gdn_strerror(s)) >= 2
    assert L.gdn_version() >= 100


def F(p):
    return ctypes.c_void_p(p)


def gate(alpha=FAKE, dt=FAKE + 4096, a=FAKE + 8192, g=FAKE + 16384, rows=4, H=4):
    return L.gdn_decay_gate(alpha, dt, a, g, rows, H, None)


def test_gate_validation():
    assert gate(rows=-1) == ERR_SHAPE
    assert gate(H=0) == ERR_SHAPE
    assert gate(alpha=None) == ERR_NULL
    assert gate(g=FAKE + 4) == ERR_ALIAS           # shifted overlap of alpha
    assert gate(rows=0, alpha=None) == OK          # empty: nothing launched


def conv(**kw):
    a = dict(x=FAKE, xt=64, xs=64 * 8, w=FAKE + (1 << 20), st=FAKE + (2 << 20), ss=64 * 3,
             out=FAKE + (3 << 20), ot=64, os=64 * 8, snap=None, snt=0, sns=0,
             n_seq=2, n_tok=8, C=64, D=4, qk=32, hd=32, eps=1e-6)
    a.update(kw)
    return L.gdn_conv1d_silu_l2norm(a["x"], a["xt"], a["xs"], a["w"], a["st"], a["ss"], a["out"],
                                    a["ot"], a["os"], a["snap"], a["snt"], a["sns"], a["n_seq"],
                                    a["n_tok"], a["C"], a["D"], a["qk"], a["hd"], a["eps"], None)


def test_conv_validation():
    assert conv(D=1) == ERR_SHAPE and conv(D=9) == ERR_SHAPE          # 2..8 taps
    assert conv(n_tok=0) == ERR_SHAPE
    assert conv(qk=48) == ERR_SHAPE                                    # not a multiple of head_dim
    assert conv(qk=128) == ERR_SHAPE                                   # beyond conv_dim
    assert conv(hd=96, qk=0) != ERR_UNSUP                              # head_dim unused without Q/K
    assert conv(hd=96, qk=96, C=192) == ERR_UNSUP                      # multiple of 32, no kernel
    assert conv(x=None) == ERR_NULL
    assert conv(ot=32) == ERR_SHAPE                                    # output rows overlap
    assert conv(out=FAKE + 128) == ERR_ALIAS                           # out overlaps x
    assert conv(snap=FAKE + (2 << 20) + 16, snt=192, sns=192 * 8) == ERR_ALIAS


def recur(**kw):
    S, H, T, n = kw.pop("S", 32), kw.pop("H", 4), kw.pop("T", 2), kw.pop("n", 2)
    Hk = kw.pop("Hk", H)
    MB = 1 << 20
    a = dict(state=FAKE, sts=H * S * S, q=FAKE + 4 * MB, k=FAKE + 8 * MB, qkt=Hk * S,
             qks=T * Hk * S, v=FAKE + 12 * MB, vt=H * S, vs=T * H * S, g=FAKE + 16 * MB,
             beta=FAKE + 20 * MB, y=FAKE + 24 * MB, yt=H * S, ys=T * H * S, snap=None, sns=0)
    a.update(kw)
    return L.gdn_recurrence_decode(a["state"], a["sts"], a["q"], a["k"], a["qkt"], a["qks"], a["v"],
                                   a["vt"], a["vs"], a["g"], a["beta"], a["y"], a["yt"], a["ys"],
                                   a["snap"], a["sns"], n, T, H, Hk, S, 0.125, None)


def test_recurrence_validation():
    assert recur(S=48) == ERR_SHAPE                                    # not a multiple of 32
    assert recur(S=288) == ERR_SHAPE                                   # above 256
    assert recur(S=96) == ERR_UNSUP                                    # valid limit, no kernel
    assert recur(Hk=3) == ERR_SHAPE                                    # H % Hk
    assert recur(T=0) == ERR_SHAPE
    assert recur(q=None) == ERR_NULL
    assert recur(state=FAKE + 4) == ERR_SHAPE                          # misaligned float4 rows
    assert recur(sts=100) == ERR_SHAPE                                 # sequences overlap
    assert recur(y=FAKE + 4 * (1 << 20) + 64) == ERR_ALIAS             # y overlaps q
    assert recur(snap=FAKE + 256, sns=4 * 32 * 32) == ERR_ALIAS        # snap overlaps state


def test_chunked_validation_and_workspace_query():
    need = L.gdn_recurrence_chunked_workspace_bytes(1, 4096, 32, 16, 128, 64)
    assert need > 0
    assert L.gdn_recurrence_chunked_workspace_bytes(1, 4096, 32, 16, 96, 64) == 0
    assert L.gdn_recurrence_chunked_workspace_bytes(1, 4096, 32, 16, 128, 32) == 0
    MB = 1 << 20
    S, H, Hk, T = 128, 4, 2, 100
    base = [FAKE, H * S * S, FAKE + 4 * MB, FAKE + 8 * MB, Hk * S, T * Hk * S, FAKE + 12 * MB,
            H * S, T * H * S, FAKE + 16 * MB, FAKE + 20 * MB, FAKE + 24 * MB, H * S, T * H * S,
            1, T, H, Hk, S, 0.1, 64]
    ws_need = L.gdn_recurrence_chunked_workspace_bytes(1, T, H, Hk, S, 64)
    call = lambda args, ws, nb: L.gdn_recurrence_chunked(*args, ws, nb, None)
    assert call(base, None, ws_need) == ERR_WS
    assert call(base, FAKE + 64 * MB, ws_need - 1) == ERR_WS
    assert call(base, FAKE + 64 * MB + 16, ws_need) == ERR_WS          # not 256-byte aligned
    assert call(base, FAKE + 12 * MB, ws_need) == ERR_ALIAS            # workspace over v
    bad = list(base); bad[-1] = 32
    assert call(bad, FAKE + 64 * MB, ws_need) == ERR_UNSUP
    # S = 32 and 64 run the on-chip fp32 form: no workspace; S = 256 has no chunked kernel
    assert L.gdn_recurrence_chunked_workspace_bytes(1, 4096, 32, 16, 32, 64) == 0
    assert L.gdn_recurrence_chunked_workspace_bytes(1, 4096, 32, 16, 64, 64) == 0
    big = list(base); big[1] = H * 256 * 256; big[4] = Hk * 256; big[5] = T * Hk * 256
    big[7] = H * 256; big[8] = T * H * 256; big[12] = H * 256; big[13] = T * H * 256; big[18] = 256
    assert call(big, FAKE + 64 * MB, ws_need) == ERR_UNSUP


def test_chunked_varlen_validation_and_workspace_query():
    MB = 1 << 20
    S, H, Hk = 128, 4, 2
    lens = [100, 0, 64, 1]
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    T = cu[-1]
    ws_need = L.gdn_recurrence_chunked_varlen_workspace_bytes(len(lens), T, H, Hk, S, 64)
    # the bound covers the padded chunk count of this split: 2 + 0 + 2 + 2 chunks
    # (per_chunk: the bytes of one chunk position over all heads)
    per_chunk = L.gdn_recurrence_chunked_workspace_bytes(1, 64, H, Hk, S, 64) // 2
    assert ws_need >= 6 * per_chunk
    # and of the worst split of T positions into 4 sequences
    assert ws_need >= ((T + 63 * 4) // 64 + 4) * per_chunk
    assert L.gdn_recurrence_chunked_varlen_workspace_bytes(0, T, H, Hk, S, 64) == 0
    assert L.gdn_recurrence_chunked_varlen_workspace_bytes(257, T, H, Hk, S, 64) == 0
    assert L.gdn_recurrence_chunked_varlen_workspace_bytes(4, T, H, Hk, 64, 64) == 0

    def call(cu_list, n_seq=None, total=None, ws=FAKE + 64 * MB, nb=ws_need, state=FAKE,
             sts=H * S * S, y=FAKE + 24 * MB, S_=S, dtype=0, qkt=None, q=FAKE + 4 * MB):
        n = len(cu_list) - 1 if n_seq is None else n_seq
        arr = (ctypes.c_int32 * max(len(cu_list), 1))(*cu_list) if cu_list is not None else None
        return L.gdn_recurrence_chunked_varlen(
            state, sts, q, FAKE + 8 * MB, Hk * S_ if qkt is None else qkt, FAKE + 12 * MB,
            H * S_, dtype,
            FAKE + 16 * MB, FAKE + 20 * MB, y, H * S_,
            ctypes.cast(arr, ctypes.c_void_p) if arr is not None else None,
            n, T if total is None else total, H, Hk, S_, 0.1, 64, ws, nb, None)
    assert call(None, n_seq=4) == ERR_NULL
    assert call([1, 100, 100, 164, 165]) == ERR_SHAPE                 # cu[0] != 0
    assert call([0, 100, 99, 164, 165]) == ERR_SHAPE                  # decreasing
    assert call(cu, total=T + 1) == ERR_SHAPE                         # cu[n] != total
    assert call([0] * 258, n_seq=257, total=0) == ERR_SHAPE           # too many sequences
    assert call(cu, ws=None) == ERR_WS
    assert call(cu, nb=ws_need - 1) == ERR_WS
    assert call(cu, sts=100) == ERR_SHAPE                             # state rows overlap
    assert call(cu, state=FAKE + 12 * MB) == ERR_ALIAS                # a state over v
    assert call(cu, state=FAKE + 64 * MB) == ERR_ALIAS                # a state over the workspace
    assert call(cu, y=FAKE + 4 * MB + 64) == ERR_ALIAS                # y over q
    assert call([0, 0, 0], total=0) == OK                             # nothing to do
    assert call(cu, dtype=2) == ERR_UNSUP                             # unknown element type
    # bf16 q, k, v at S = 128: 16-byte rows (strides a multiple of 8 elements)
    assert call(cu, dtype=1, qkt=Hk * S + 4) == ERR_SHAPE
    assert call(cu, dtype=1, q=FAKE + 4 * MB + 8) == ERR_SHAPE


def test_mamba2_ssd_validation_and_workspace_query():
    MB = 1 << 20
    n, T, H, G, P, N = 2, 100, 4, 2, 64, 128
    need = L.gdn_mamba2_ssd_workspace_bytes(n, T, H, P, N, 64)
    assert need >= n * H * 2 * P * N * 4                     # two chunks of state blocks
    assert L.gdn_mamba2_ssd_workspace_bytes(n, T, H, 48, N, 64) == 0
    assert L.gdn_mamba2_ssd_workspace_bytes(n, T, H, P, 96, 64) == 0
    assert L.gdn_mamba2_ssd_workspace_bytes(n, T, H, P, N, 32) == 0

    def call(state=FAKE, sts=H * P * N, x=FAKE + 8 * MB, xt=H * P, B=FAKE + 16 * MB,
             C=FAKE + 24 * MB, bct=G * N, y=FAKE + 32 * MB, H_=H, G_=G, P_=P, N_=N,
             ws=FAKE + 64 * MB, nb=need, chunk=64):
        return L.gdn_mamba2_ssd_chunked(
            state, sts, x, xt, T * xt, B, C, bct, T * bct, FAKE + 40 * MB, H_, T * H_,
            FAKE + 41 * MB, FAKE + 42 * MB, FAKE + 43 * MB, y, H_ * P_, T * H_ * P_, n, T, H_,
            G_, P_, N_, 1e-3, 1e-1, chunk, ws, nb, None)
    assert call(G_=3) == ERR_SHAPE                           # H % G
    assert call(P_=48) == ERR_SHAPE
    assert call(P_=128) == ERR_UNSUP
    assert call(chunk=32) == ERR_UNSUP
    assert call(x=None) == ERR_NULL
    assert call(x=FAKE + 8 * MB + 4) == ERR_SHAPE            # misaligned 16-byte rows
    assert call(xt=H * P + 2) == ERR_SHAPE                   # stride not a multiple of 4
    assert call(sts=100) == ERR_SHAPE                        # state rows overlap
    assert call(ws=None) == ERR_WS
    assert call(nb=need - 1) == ERR_WS
    assert call(y=FAKE + 8 * MB + 64) == ERR_ALIAS           # y over x
    assert call(state=FAKE + 16 * MB) == ERR_ALIAS           # state over B
    assert call(ws=FAKE + 24 * MB) == ERR_ALIAS              # workspace over C


def test_norm_validation():
    MB = 1 << 20
    call = lambda y, ys, w, z, zs, o, os_, rows, H, hd: L.gdn_gated_rmsnorm(
        y, ys, w, z, zs, o, os_, rows, H, hd, 1e-6, None)
    assert call(FAKE, 256, FAKE + MB, FAKE + 2 * MB, 256, FAKE + 3 * MB, 256, 4, 2, 48) == ERR_SHAPE
    assert call(FAKE, 384, FAKE + MB, FAKE + 2 * MB, 384, FAKE + 3 * MB, 384, 4, 2, 192) == ERR_UNSUP
    assert call(FAKE, 256, None, FAKE + 2 * MB, 256, FAKE + 3 * MB, 256, 4, 2, 128) == ERR_NULL
    assert call(FAKE, 256, FAKE + MB, FAKE + 2 * MB, 256, FAKE + 2 * MB, 256, 4, 2, 128) == ERR_ALIAS
    assert call(FAKE, 256, FAKE + MB, FAKE + 2 * MB, 256, FAKE + 64, 256, 4, 2, 128) == ERR_ALIAS
    assert call(FAKE, 256, FAKE + MB, FAKE + 2 * MB, 256, FAKE + 3 * MB, 128, 4, 2, 128) == ERR_SHAPE


def fused(**kw):
    S, H, T, n = kw.pop("S", 32), 4, 2, 2
    MB = 1 << 20
    a = dict(state=FAKE, sts=H * S * S, q=FAKE + 4 * MB, k=FAKE + 8 * MB, qkt=H * S,
             qks=T * H * S, v=FAKE + 12 * MB, vt=H * S, vs=T * H * S, alpha=FAKE + 16 * MB,
             dt=FAKE + 17 * MB, a=FAKE + 18 * MB, beta=FAKE + 20 * MB, w=FAKE + 22 * MB,
             z=FAKE + 24 * MB, zt=H * S, zs=T * H * S, out=FAKE + 28 * MB, ot=H * S,
             os=T * H * S, g=None, y=None, yt=0, ys=0, snap=None, sns=0)
    a.update(kw)
    return L.gdn_decode_fused(a["state"], a["sts"], a["q"], a["k"], a["qkt"], a["qks"], a["v"],
                              a["vt"], a["vs"], a["alpha"], a["dt"], a["a"], a["beta"], a["w"],
                              a["z"], a["zt"], a["zs"], a["out"], a["ot"], a["os"], a["g"],
                              a["y"], a["yt"], a["ys"], a["snap"], a["sns"], n, T, H, H, S,
                              0.125, 1e-6, None)


def test_fused_validation():
    MB = 1 << 20
    assert fused(S=96) == ERR_UNSUP
    assert fused(dt=None) == ERR_NULL and fused(z=None) == ERR_NULL
    assert fused(out=FAKE + 28 * MB + 4) == ERR_SHAPE                  # out not 16-byte aligned
    assert fused(zt=4 * 32 + 2) == ERR_SHAPE                           # z stride not a multiple of 4
    assert fused(out=FAKE + 24 * MB + 64) == ERR_ALIAS                 # out overlaps z
    assert fused(g=FAKE + 16 * MB) == ERR_ALIAS                        # g overlaps alpha
    assert fused(y=FAKE + 28 * MB, yt=128, ys=256) == ERR_ALIAS        # y overlaps out
    assert fused(snap=FAKE + 22 * MB, sns=4 * 32 * 32) == ERR_ALIAS    # snapshot over norm_w


def step(**kw):
    S, H, Hk, n = 32, 4, 2, 2
    T = kw.pop("T", 2)
    MB = 1 << 20
    C = (2 * Hk + H) * S
    a = dict(state=FAKE, sts=H * S * S, x=FAKE + 4 * MB, xt=C, xs=2 * C, cw=FAKE + 5 * MB,
             hist=FAKE + 6 * MB, hs=3 * C, csnap=None, cst=0, css=0, alpha=FAKE + 16 * MB,
             dt=FAKE + 17 * MB, a=FAKE + 18 * MB, beta=FAKE + 20 * MB, w=FAKE + 22 * MB,
             z=FAKE + 24 * MB, zt=H * S, zs=2 * H * S, out=FAKE + 28 * MB, ot=H * S,
             os=2 * H * S, g=None, y=None, yt=0, ys=0, snap=None, sns=0, Hk=Hk, D=4,
             ws=FAKE + 40 * MB, wsb=n * Hk * 8)
    a.update(kw)
    if "hs" not in kw:
        a["hs"] = (a["D"] - 1) * C            # histories packed for the width asked for
    return L.gdn_decode_step(a["state"], a["sts"], a["x"], a["xt"], a["xs"], a["cw"], a["hist"],
                             a["hs"], a["csnap"], a["cst"], a["css"], a["alpha"], a["dt"],
                             a["a"], a["beta"], a["w"], a["z"], a["zt"], a["zs"], a["out"],
                             a["ot"], a["os"], a["g"], a["y"], a["yt"], a["ys"], a["snap"],
                             a["sns"], n, T, H, a["Hk"], S, a["D"], 0.125, 1e-6, 1e-6, a["ws"],
                             a["wsb"], None)


def test_step_validation_and_workspace_query():
    MB = 1 << 20
    assert L.gdn_decode_step_workspace_bytes(64, 16) == 64 * 16 * 2 * 4
    assert L.gdn_decode_step_workspace_bytes(0, 16) == 0
    # everything valid but a conv width without a kernel: the last check
    assert step(D=5) == ERR_UNSUP
    assert step(D=5, csnap=FAKE + 7 * MB, cst=4 * 256, css=4 * 256) == ERR_UNSUP
    assert step(D=9) == ERR_SHAPE and step(D=1) == ERR_SHAPE
    assert step(T=33) == ERR_SHAPE                                      # at most 32 positions
    assert step(Hk=3) == ERR_SHAPE                                      # H not a multiple of Hk
    assert step(x=None) == ERR_NULL and step(cw=None) == ERR_NULL and step(hist=None) == ERR_NULL
    assert step(ws=None) == ERR_WS and step(wsb=16) == ERR_WS
    assert step(ws=FAKE + 40 * MB + 2) == ERR_WS                        # counters misaligned
    assert step(x=FAKE + 4 * MB + 8) == ERR_SHAPE                       # x not 16-byte aligned
    assert step(xt=258, xs=516) == ERR_SHAPE                            # x stride not a multiple of 4
    assert step(xt=128, xs=256) == ERR_SHAPE                            # rows shorter than conv_dim
    assert step(hs=100) == ERR_SHAPE                                    # histories overlap each other
    assert step(hist=FAKE + 4 * MB + 64) == ERR_ALIAS                   # history over x
    assert step(ws=FAKE) == ERR_ALIAS                                   # counters over the state
    assert step(csnap=FAKE + 6 * MB + 256, cst=768, css=768) == ERR_ALIAS  # snapshot over history
    assert step(out=FAKE + 4 * MB + 512) == ERR_ALIAS                   # out over x


def step_noalloc(n=2, **kw):
    S, H, Hk = 32, 4, kw.pop("Hk", 2)
    MB = 1 << 20
    C = (2 * Hk + H) * S
    a = dict(state=FAKE, x=FAKE + 4 * MB, cw=FAKE + 5 * MB, hist=FAKE + 6 * MB,
             alpha=FAKE + 16 * MB, dt=FAKE + 17 * MB, a=FAKE + 18 * MB, beta=FAKE + 20 * MB,
             w=FAKE + 22 * MB, z=FAKE + 24 * MB, out=FAKE + 28 * MB, D=4, T=2)
    a.update(kw)
    return L.gdn_decode_step_noalloc(
        a["state"], H * S * S, a["x"], C, 2 * C, a["cw"], a["hist"], (a["D"] - 1) * C, None, 0, 0,
        a["alpha"], a["dt"], a["a"], a["beta"], a["w"], a["z"], H * S, 2 * H * S, a["out"],
        H * S, 2 * H * S, None, None, 0, 0, None, 0, n, a["T"], H, Hk, S, a["D"], 0.125, 1e-6,
        1e-6, None)


def test_step_noalloc_validation():
    # the fixed scratch array holds n_seq * n_qk_heads * 2 counters of 4 bytes
    m = re.search(r"#define GDN_NOALLOC_SCRATCH_BYTES (\d+)", open(HEADERS[0]).read())
    assert m and int(m.group(1)) == gdn.NOALLOC_SCRATCH_BYTES == 65536
    assert step_noalloc(n=4097, Hk=2) == ERR_SCRATCH                   # 8194 > 8192 pairs
    assert step_noalloc(n=4097, Hk=2, x=None) == ERR_SCRATCH            # the limit comes first
    # the workspace-free call keeps every other rule of gdn_decode_step
    assert step_noalloc(D=5) == ERR_UNSUP
    assert step_noalloc(T=33) == ERR_SHAPE and step_noalloc(Hk=3) == ERR_SHAPE
    assert step_noalloc(x=None) == ERR_NULL and step_noalloc(hist=None) == ERR_NULL
    assert step_noalloc(hist=FAKE + 4 * (1 << 20) + 64) == ERR_ALIAS


def prefill(**kw):
    """gdn_prefill_chunked on fake addresses, valid except for what kw changes
    (every case below fails a host check, so nothing is launched)."""
    MB = 1 << 20
    S, H, Hk, T = 128, 4, 2, 100
    C = (2 * Hk + H) * S
    a = dict(state=FAKE, sts=H * S * S, x=FAKE + 4 * MB, xt=C, xs=T * C, cw=FAKE + 8 * MB,
             hist=FAKE + 9 * MB, hs=3 * C, alpha=FAKE + 10 * MB, dt=FAKE + 11 * MB,
             a=FAKE + 12 * MB, beta=FAKE + 13 * MB, y=FAKE + 16 * MB, yt=H * S, ys=T * H * S,
             n=1, T=T, H=H, Hk=Hk, S=S, D=4, chunk=64, ws=FAKE + 64 * MB, wsb=None)
    a.update(kw)
    need = L.gdn_prefill_chunked_workspace_bytes(a["n"], a["T"], a["H"], a["Hk"], 128, 64)
    return L.gdn_prefill_chunked(
        a["state"], a["sts"], a["x"], a["xt"], a["xs"], a["cw"], a["hist"], a["hs"], a["alpha"],
        a["dt"], a["a"], a["beta"], a["y"], a["yt"], a["ys"], a["n"], a["T"], a["H"], a["Hk"],
        a["S"], a["D"], 0.088, 1e-6, a["chunk"], a["ws"], need if a["wsb"] is None else a["wsb"],
        None)


def test_prefill_validation_and_workspace_query():
    MB = 1 << 20
    assert (L.gdn_prefill_chunked_workspace_bytes(1, 4096, 32, 16, 128, 64) ==
            L.gdn_recurrence_chunked_workspace_bytes(1, 4096, 32, 16, 128, 64) > 0)
    assert L.gdn_prefill_chunked_workspace_bytes(1, 4096, 32, 16, 64, 64) == 0
    assert L.gdn_prefill_chunked_workspace_bytes(1, 4096, 32, 16, 128, 32) == 0
    assert prefill(D=3) == ERR_UNSUP and prefill(chunk=32) == ERR_UNSUP
    assert prefill(S=64, sts=4 * 64 * 64) == ERR_UNSUP
    assert prefill(D=9) == ERR_SHAPE and prefill(T=0) == ERR_SHAPE and prefill(Hk=3) == ERR_SHAPE
    for k in ("state", "x", "cw", "hist", "alpha", "dt", "a", "beta", "y"):
        assert prefill(**{k: None}) == ERR_NULL, k
    assert prefill(ws=None) == ERR_WS and prefill(wsb=16) == ERR_WS
    assert prefill(ws=FAKE + 64 * MB + 16) == ERR_WS                 # not 256-byte aligned
    assert prefill(x=FAKE + 4 * MB + 8) == ERR_SHAPE                 # x not 16-byte aligned
    assert prefill(xt=1026) == ERR_SHAPE                             # stride not a multiple of 4
    assert prefill(xt=512, xs=512 * 100) == ERR_SHAPE                # rows shorter than conv_dim
    assert prefill(n=2, hs=100) == ERR_SHAPE                         # histories overlap
    assert prefill(hist=FAKE + 4 * MB + 64) == ERR_ALIAS             # history over x
    assert prefill(y=FAKE + 12 * MB) == ERR_ALIAS                    # y over a
    assert prefill(ws=FAKE + 4 * MB) == ERR_ALIAS                    # workspace over x
    assert prefill(y=FAKE + 64 * MB) == ERR_ALIAS                    # y over the workspace


def test_stream_copy_validation():
    assert L.gdn_stream_copy(FAKE, FAKE + (1 << 20), 0, None) == OK            # nothing launched
    assert L.gdn_stream_copy(None, FAKE, 64, None) == ERR_NULL
    assert L.gdn_stream_copy(FAKE + 4, FAKE + (1 << 20), 64, None) == ERR_SHAPE  # misaligned
    assert L.gdn_stream_copy(FAKE, FAKE + (1 << 20), 60, None) == ERR_SHAPE      # not whole 16 B
    assert L.gdn_stream_copy(FAKE, FAKE + 32, 64, None) == ERR_ALIAS


def test_page_shape_limits_are_the_abi_limits():
    import json
    gold = json.load(open(os.path.join(ROOT, "tests", "golden", "page_constants.json")))
    assert recur(S=gold["max_state_size"]["value"] + 32) == ERR_SHAPE
    assert conv(D=gold["max_conv_kernel"]["value"] + 1) == ERR_SHAPE
    assert conv(D=gold["max_conv_kernel"]["value"], qk=0, x=None) == ERR_NULL   # 8 taps accepted
