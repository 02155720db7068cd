"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Error metric (the pages do not define "max rel err"): normwise-inf relative
error per output tensor, max|gpu - ref| / max|ref|, the final state and
snapshots counted as tensors of their own.  Tolerances: 1e-5 for the gate,
conv and norm; 1e-4 for the token-by-token recurrence; 2e-3 for the chunked
recurrence against the sequential scan.  Integer-like results (the conv
history, which only ever holds raw inputs) must match exactly, and the
multi-position paths must match their one-position equivalents bit for bit.

Every test runs at the workload's full size and launch configuration, on
inputs from gdn_inputs.make_inputs; the oracle sees the identical fp32 arrays.
"""
import functools
import math

import numpy as np
import pytest
import torch

import oracle
from gdn_inputs import WORKLOADS, make_inputs, make_mamba2_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
ALL = list(WORKLOADS)


def gdn():
    import gated_delta_ssm_amd
    return gated_delta_ssm_amd


def rel(x, r):
    x = x.detach().cpu().double().numpy() if isinstance(x, torch.Tensor) else np.asarray(x)
    r = np.asarray(r, np.float64)
    assert x.shape == r.shape, (x.shape, r.shape)
    assert np.all(np.isfinite(x)), "non-finite output"
    return float(np.max(np.abs(x - r)) / max(np.max(np.abs(r)), 1e-30))


def bits_equal(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.contiguous().view(torch.int32), b.contiguous().view(torch.int32))


@functools.lru_cache(maxsize=2)
def inputs(name):
    return make_inputs(name)


def on_dev(t):
    return t.to(DEV)


def oracle_g(inp):
    """g for the recurrence tests: the oracle's gate, rounded to fp32."""
    wl = inp["wl"]
    g = oracle.decay_gate(inp["alpha"], inp["dt"], inp["a"]).astype(np.float32)
    return torch.from_numpy(g).reshape(wl.n_seq, wl.n_tok, wl.H)


def log_case(name, **kw):
    print(f"[case] {name} " + " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


# ------------------------------------------------------------------------------------- gate

@pytest.mark.parametrize("name", ALL)
def test_gate(name):
    inp = inputs(name)
    log_case("gate", wl=name)
    g = gdn().gdn_decay_gate(on_dev(inp["alpha"]), on_dev(inp["dt"]), on_dev(inp["a"]))
    ref = oracle.decay_gate(inp["alpha"], inp["dt"], inp["a"])
    assert rel(g, ref) < 1e-5
    assert bool((g < 0).all())


def test_gate_guard_edges():
    log_case("gate_edges")
    v = torch.tensor([[-100.0, -20.0, 0.0, 19.999, 20.0, 20.001, 21.0, 1e4, 3e38]])
    H = v.shape[1]
    dt = torch.zeros(H)
    a = -torch.linspace(1.0, 16.0, H)
    g = gdn().gdn_decay_gate(on_dev(v), on_dev(dt), on_dev(a)).cpu()
    ref = oracle.decay_gate(v, dt, a)
    assert torch.isfinite(g[0, :-1]).all()
    # fp32 denormal results (v = -100) carry few significant bits: absolute slack there
    np.testing.assert_allclose(g[0, :-1].double().numpy(), ref[0, :-1], rtol=2e-6, atol=1e-37)
    assert g[0, 5] == (a[5] * v[0, 5])            # above the guard: a * v exactly


# ------------------------------------------------------------------------------------- conv

def run_conv(inp, x_rows=None, snap=False, n_tok=None, hist=None):
    wl = inp["wl"]
    C = wl.conv_dim
    x_full = on_dev(inp["x"] if x_rows is None else x_rows)
    T = x_full.shape[1] if n_tok is None else n_tok
    x = x_full[:, :T, :C]
    out_full = torch.full((wl.n_seq, T, wl.out_stride), float("nan"), device=DEV)
    out = out_full[..., :C]
    st = on_dev(inp["conv_hist"] if hist is None else hist).clone()
    sn = torch.full((wl.n_seq, T - 1, C, wl.d_conv - 1), float("nan"), device=DEV) if snap else None
    gdn().gdn_conv1d_silu_l2norm(x, on_dev(inp["conv_w"]), st, out, qk_channels=wl.qk_channels,
                                 head_dim=wl.head_dim, l2_eps=wl.l2_eps, snap=sn)
    return out, st, sn, out_full


@pytest.mark.parametrize("name", ALL)
def test_conv(name):
    inp = inputs(name)
    wl = inp["wl"]
    log_case("conv", wl=name, n_seq=wl.n_seq, n_tok=wl.n_tok, C=wl.conv_dim)
    x = inp["x"].clone()
    x[..., wl.conv_dim:] = float("nan")       # any read outside the conv channels poisons out
    out, st, sn, out_full = run_conv(inp, x_rows=x, snap=wl.n_tok > 1 and wl.n_tok <= 8)
    o_ref, h_ref, s_ref = oracle.conv1d_silu_l2norm(
        inp["x"][..., :wl.conv_dim], inp["conv_w"], inp["conv_hist"], wl.qk_channels,
        wl.head_dim, wl.l2_eps, want_snap=sn is not None)
    assert rel(out, o_ref) < 1e-5
    assert np.array_equal(st.cpu().double().numpy(), h_ref)
    if sn is not None:
        assert np.array_equal(sn.cpu().double().numpy(), s_ref)
    if wl.out_stride > wl.conv_dim:            # the gap between output rows is untouched
        assert torch.isnan(out_full[..., wl.conv_dim:]).all()


@pytest.mark.parametrize("head_dim,qk,d_conv,T", [(64, 128, 2, 37), (256, 512, 8, 70),
                                                  (32, 96, 3, 5), (128, 0, 4, 33)])
def test_conv_other_shapes(head_dim, qk, d_conv, T):
    C = 3 * max(qk, 64) + 32                      # a ragged last channel block
    inp = make_inputs("tiny", seed=11, conv_dim=C, qk_channels=qk, head_dim=head_dim,
                      d_conv=d_conv, n_tok=T, x_stride=C, out_stride=C, hist_std=1.0, n_seq=2)
    wl = inp["wl"]
    log_case("conv_shapes", hd=head_dim, qk=qk, d=d_conv, T=T, C=C)
    out, st, _, _ = run_conv(inp)
    o_ref, h_ref, _ = oracle.conv1d_silu_l2norm(inp["x"], inp["conv_w"], inp["conv_hist"],
                                                qk, head_dim, wl.l2_eps)
    assert rel(out, o_ref) < 1e-5
    assert np.array_equal(st.cpu().double().numpy(), h_ref)


@pytest.mark.parametrize("T", [1, 40])
def test_conv_unaligned_rows_bit_identical_to_aligned(T):
    # x and out one element off 16-byte alignment take the 4-byte-access path;
    # its arithmetic is the 16-byte path's, so the results agree bit for bit
    inp = make_inputs("tiny", seed=13, n_tok=T, n_seq=2, hist_std=1.0)
    wl = inp["wl"]
    C = wl.conv_dim
    log_case("conv_unaligned", T=T, C=C)
    out_a, st_a, _, _ = run_conv(inp)
    x_sh = torch.full((wl.n_seq, T, C + 1), float("nan"))
    x_sh[..., 1:] = inp["x"][..., :C]
    o_full = torch.full((wl.n_seq, T, C + 1), float("nan"), device=DEV)
    st = on_dev(inp["conv_hist"]).clone()
    gdn().gdn_conv1d_silu_l2norm(on_dev(x_sh)[..., 1:], on_dev(inp["conv_w"]), st,
                                 o_full[..., 1:], qk_channels=wl.qk_channels,
                                 head_dim=wl.head_dim, l2_eps=wl.l2_eps)
    assert bits_equal(o_full[..., 1:], out_a) and bits_equal(st, st_a)
    assert torch.isnan(o_full[..., 0]).all()


def test_conv_long_prompt_tiles():
    # more positions than 8-position tiles can put in the grid's y dimension
    # (65535 tiles): the launcher switches to 64-position tiles, same arithmetic
    T, C, D = 8 * 65535 + 40, 8, 4
    gen = torch.Generator("cpu").manual_seed(29)
    x = torch.randn(1, T, C, generator=gen)
    w = torch.randn(C, D, generator=gen) * 0.25
    hist = torch.randn(1, C, D - 1, generator=gen)
    log_case("conv_long_prompt", T=T, C=C)
    out = torch.full((1, T, C), float("nan"), device=DEV)
    st = on_dev(hist).clone()
    gdn().gdn_conv1d_silu_l2norm(on_dev(x), on_dev(w), st, out, qk_channels=0, head_dim=32,
                                 l2_eps=1e-6)
    o_ref, h_ref, _ = oracle.conv1d_silu_l2norm(x, w, hist, 0, 32, 1e-6)
    assert rel(out, o_ref) < 1e-5
    assert np.array_equal(st.cpu().double().numpy(), h_ref)


@pytest.mark.parametrize("C,qk,hd", [(222, 0, 32), (263, 128, 64)])
def test_conv_channels_not_multiple_of_4(C, qk, hd):
    # a last lane with fewer than 4 channels (scalar path), against the oracle
    T = 37
    inp = make_inputs("tiny", seed=17, conv_dim=C, qk_channels=qk, head_dim=hd, n_tok=T,
                      x_stride=C, out_stride=C, hist_std=1.0, n_seq=2)
    wl = inp["wl"]
    log_case("conv_ragged_channels", C=C, qk=qk, hd=hd)
    out, st, _, _ = run_conv(inp)
    o_ref, h_ref, _ = oracle.conv1d_silu_l2norm(inp["x"], inp["conv_w"], inp["conv_hist"],
                                                qk, hd, wl.l2_eps)
    assert rel(out, o_ref) < 1e-5
    assert np.array_equal(st.cpu().double().numpy(), h_ref)


@pytest.mark.parametrize("T", [100, 3])
def test_conv_token_parallel_bit_identical_to_steps(T):
    # the long-prompt kernel vs one-position calls, on the decode workload's channels
    inp = make_inputs("decode", seed=21, n_tok=T)
    wl = inp["wl"]
    log_case("conv_tp_vs_steps", T=T)
    out_all, st_all, _, _ = run_conv(inp)
    st = on_dev(inp["conv_hist"]).clone()
    outs = []
    for t in range(T):
        o = torch.empty(1, 1, wl.conv_dim, device=DEV)
        gdn().gdn_conv1d_silu_l2norm(on_dev(inp["x"])[:, t:t + 1, :wl.conv_dim],
                                     on_dev(inp["conv_w"]), st, o, qk_channels=wl.qk_channels,
                                     head_dim=wl.head_dim, l2_eps=wl.l2_eps)
        outs.append(o)
    assert bits_equal(out_all, torch.cat(outs, dim=1))
    assert bits_equal(st_all, st)


def test_conv_verify2_fused_equals_two_steps_and_rollback():
    inp = inputs("verify2")
    wl = inp["wl"]
    log_case("conv_verify2_bits")
    out2, st2, sn, _ = run_conv(inp, snap=True)
    st = on_dev(inp["conv_hist"]).clone()
    outs = []
    for t in range(2):
        o = torch.empty(wl.n_seq, 1, wl.conv_dim, device=DEV)
        gdn().gdn_conv1d_silu_l2norm(on_dev(inp["x"])[:, t:t + 1, :wl.conv_dim],
                                     on_dev(inp["conv_w"]), st, o, qk_channels=wl.qk_channels,
                                     head_dim=wl.head_dim, l2_eps=wl.l2_eps)
        outs.append(o)
        if t == 0:
            after0 = st.clone()
    assert bits_equal(out2, torch.cat(outs, 1)) and bits_equal(st2, st)
    assert bits_equal(sn[:, 0], after0)           # the rollback snapshot is position 0's window


# ------------------------------------------------------------------------------------- recurrence

def run_decode(inp, g3, state=None, snap=False, t0=0, t1=None):
    wl = inp["wl"]
    t1 = wl.n_tok if t1 is None else t1
    st = on_dev(inp["state"] if state is None else state).clone()
    sl = lambda a: on_dev(a[:, t0:t1]).contiguous()
    v = sl(inp["v"])
    y = torch.empty_like(v)
    sn = torch.full((wl.n_seq, t1 - t0 - 1, wl.H, wl.S, wl.S), float("nan"), device=DEV) \
        if snap else None
    gdn().gdn_recurrence_decode(st, sl(inp["q"]), sl(inp["k"]), v, sl(g3), sl(inp["beta"]), y,
                                scale=wl.scale, snap=sn)
    return y, st, sn


@pytest.mark.parametrize("name", ["tiny", "decode", "decode64", "verify2"])
def test_recurrence_decode(name):
    inp = inputs(name)
    wl = inp["wl"]
    log_case("recurrence_decode", wl=name, n_seq=wl.n_seq, n_tok=wl.n_tok, H=wl.H, S=wl.S)
    g3 = oracle_g(inp)
    snap = 1 < wl.n_tok <= 8
    y, st, sn = run_decode(inp, g3, snap=snap)
    y_ref, s_ref, sn_ref = oracle.recurrence_seq(inp["state"], inp["q"], inp["k"], inp["v"], g3,
                                                 inp["beta"], wl.scale, want_snap=snap)
    assert rel(y, y_ref) < 1e-4
    assert rel(st, s_ref) < 1e-4
    if snap:
        assert rel(sn, sn_ref) < 1e-4


@pytest.mark.parametrize("S,H,Hk,T,n_seq", [(64, 6, 3, 17, 3), (256, 2, 1, 5, 2), (32, 3, 1, 1, 5)])
def test_recurrence_decode_other_shapes(S, H, Hk, T, n_seq):
    inp = make_inputs("tiny", seed=31, S=S, H=H, Hk=Hk, n_tok=T, n_seq=n_seq, state_std=0.1)
    wl = inp["wl"]
    log_case("recurrence_shapes", S=S, H=H, Hk=Hk, T=T, n_seq=n_seq)
    g3 = oracle_g(inp)
    y, st, _ = run_decode(inp, g3)
    y_ref, s_ref, _ = oracle.recurrence_seq(inp["state"], inp["q"], inp["k"], inp["v"], g3,
                                            inp["beta"], wl.scale)
    assert rel(y, y_ref) < 1e-4 and rel(st, s_ref) < 1e-4


def test_recurrence_verify2_bit_identical_to_two_steps():
    inp = inputs("verify2")
    log_case("recurrence_verify2_bits")
    g3 = oracle_g(inp)
    y2, st2, sn = run_decode(inp, g3, snap=True)
    ya, sta, _ = run_decode(inp, g3, t0=0, t1=1)
    yb, stb, _ = run_decode(inp, g3, state=sta, t0=1, t1=2)
    assert bits_equal(y2, torch.cat([ya, yb], 1))
    assert bits_equal(st2, stb)
    assert bits_equal(sn[:, 0], sta)


@pytest.mark.parametrize("K", [4, 17])
def test_verify_k_positions_snapshots_and_steps(K):
    # K-position verify (batched speculative decoding): all K-1 rollback
    # snapshots, for the conv and the recurrence, against the oracle and
    # against K one-position calls
    inp = make_inputs("verify2", seed=81, n_tok=K, n_seq=4)
    wl = inp["wl"]
    log_case("verify_k", K=K, n_seq=wl.n_seq)
    g3 = oracle_g(inp)
    yK, stK, snK = run_decode(inp, g3, snap=True)
    y_ref, s_ref, sn_ref = oracle.recurrence_seq(inp["state"], inp["q"], inp["k"], inp["v"], g3,
                                                 inp["beta"], wl.scale, want_snap=True)
    assert rel(yK, y_ref) < 1e-4 and rel(stK, s_ref) < 1e-4 and rel(snK, sn_ref) < 1e-4
    st = on_dev(inp["state"]).clone()
    ys = []
    for t in range(K):
        y1, st, _ = run_decode(inp, g3, state=st, t0=t, t1=t + 1)
        ys.append(y1)
        if t < K - 1:
            assert bits_equal(snK[:, t], st)
    assert bits_equal(yK, torch.cat(ys, 1)) and bits_equal(stK, st)

    out, hist, sn, _ = run_conv(inp, snap=True)
    o_ref, h_ref, c_ref = oracle.conv1d_silu_l2norm(
        inp["x"][..., :wl.conv_dim], inp["conv_w"], inp["conv_hist"], wl.qk_channels,
        wl.head_dim, wl.l2_eps, want_snap=True)
    assert rel(out, o_ref) < 1e-5
    assert np.array_equal(hist.cpu().double().numpy(), h_ref)
    assert np.array_equal(sn.cpu().double().numpy(), c_ref)


def test_recurrence_strided_inputs_poisoned_gaps():
    # q/k/v/y rows inside wider buffers whose gaps hold NaN: a stray read or
    # write outside the declared rows shows up as NaN in y or a changed gap
    inp = make_inputs("tiny", seed=41, n_seq=3, n_tok=5, H=4, Hk=2, state_std=0.1)
    wl = inp["wl"]
    log_case("recurrence_strided")
    g3 = oracle_g(inp)

    def wide(a, pad):
        buf = torch.full((*a.shape[:-2], a.shape[-2] * a.shape[-1] + pad), float("nan"))
        buf[..., :a.shape[-2] * a.shape[-1]] = a.reshape(*a.shape[:-2], -1)
        return on_dev(buf)[..., :a.shape[-2] * a.shape[-1]].unflatten(-1, a.shape[-2:])

    qk_buf = torch.full((wl.n_seq, wl.n_tok, 2, wl.Hk * wl.S + 8), float("nan"))
    qk_buf[:, :, 0, :wl.Hk * wl.S] = inp["q"].reshape(wl.n_seq, wl.n_tok, -1)
    qk_buf[:, :, 1, :wl.Hk * wl.S] = inp["k"].reshape(wl.n_seq, wl.n_tok, -1)
    qk_dev = on_dev(qk_buf)
    q = qk_dev[:, :, 0, :wl.Hk * wl.S].unflatten(-1, (wl.Hk, wl.S))
    k = qk_dev[:, :, 1, :wl.Hk * wl.S].unflatten(-1, (wl.Hk, wl.S))
    v = wide(inp["v"], 12)
    y_buf = torch.full((wl.n_seq, wl.n_tok, wl.H * wl.S + 20), float("nan"), device=DEV)
    y = y_buf[..., :wl.H * wl.S].unflatten(-1, (wl.H, wl.S))
    st_buf = torch.full((wl.n_seq, wl.H * wl.S * wl.S + 64), float("nan"), device=DEV)
    st_buf[:, :wl.H * wl.S * wl.S] = on_dev(inp["state"]).reshape(wl.n_seq, -1)
    st = st_buf[:, :wl.H * wl.S * wl.S].unflatten(-1, (wl.H, wl.S, wl.S))
    gdn().gdn_recurrence_decode(st, q, k, v, on_dev(g3), on_dev(inp["beta"]), y, scale=wl.scale)
    y_ref, s_ref, _ = oracle.recurrence_seq(inp["state"], inp["q"], inp["k"], inp["v"], g3,
                                            inp["beta"], wl.scale)
    assert rel(y, y_ref) < 1e-4 and rel(st, s_ref) < 1e-4
    assert torch.isnan(y_buf[..., wl.H * wl.S:]).all()
    assert torch.isnan(st_buf[:, wl.H * wl.S * wl.S:]).all()


def test_recurrence_decode_deterministic():
    inp = inputs("decode64")
    log_case("recurrence_determinism")
    g3 = oracle_g(inp)
    ya, sa, _ = run_decode(inp, g3)
    yb, sb, _ = run_decode(inp, g3)
    assert bits_equal(ya, yb) and bits_equal(sa, sb)


# ------------------------------------------------------------------------------------- norm

@pytest.mark.parametrize("name", ALL)
def test_gated_rmsnorm(name):
    inp = inputs(name)
    wl = inp["wl"]
    log_case("norm", wl=name, rows=wl.rows, H=wl.H, hd=wl.head_dim)
    y = on_dev(inp["norm_y"])
    out = torch.empty_like(y)
    gdn().gdn_gated_rmsnorm(y, on_dev(inp["norm_w"]), on_dev(inp["z"]), out, eps=wl.norm_eps)
    ref = oracle.gated_rmsnorm(inp["norm_y"], inp["norm_w"], inp["z"], wl.norm_eps)
    assert rel(out, ref) < 1e-5


@pytest.mark.parametrize("hd,H", [(32, 5), (64, 3), (256, 2)])
@pytest.mark.parametrize("z_shift", [16, 17])
def test_gated_rmsnorm_z_offset_and_in_place(hd, H, z_shift):
    # z read at an offset inside a wider [Q|K|V|Z]-style row; out written over y.
    # A shift of 16 elements keeps z 16-byte aligned (the float4 kernel), 17
    # does not (the general kernel).
    rows = 7
    inp = make_inputs("tiny", seed=51, head_dim=hd, H=H, n_tok=rows)
    log_case("norm_offset_inplace", hd=hd, H=H, z_shift=z_shift)
    width = 3 * H * hd
    row = torch.full((rows, width), float("nan"))
    z_off = H * hd + z_shift
    row[:, z_off:z_off + H * hd] = inp["z"].reshape(rows, -1)
    row_dev = on_dev(row)
    z = row_dev[:, z_off:z_off + H * hd].unflatten(-1, (H, hd))
    y = on_dev(inp["norm_y"]).clone()
    gdn().gdn_gated_rmsnorm(y, on_dev(inp["norm_w"]), z, y, eps=1e-6)
    ref = oracle.gated_rmsnorm(inp["norm_y"], inp["norm_w"], inp["z"], 1e-6)
    assert rel(y, ref) < 1e-5


# ------------------------------------------------------------------------------------- chained

def test_tiny_chained_layer_core():
    # gate -> conv (Q|K|V channels) -> recurrence -> gated norm on one GPU,
    # against the same chain in the oracle with fp64 intermediates
    inp = inputs("tiny")
    wl = inp["wl"]
    log_case("chained_tiny")
    T, H, S = wl.n_tok, wl.H, wl.S
    g = gdn().gdn_decay_gate(on_dev(inp["alpha"]), on_dev(inp["dt"]), on_dev(inp["a"]))
    out, _, _, _ = run_conv(inp)
    qd = out[0, :, :H * S].reshape(1, T, H, S).contiguous()
    kd = out[0, :, H * S:2 * H * S].reshape(1, T, H, S).contiguous()
    vd = out[0, :, 2 * H * S:].reshape(1, T, H, S).contiguous()
    st = on_dev(inp["state"]).clone()
    y = torch.empty_like(vd)
    gdn().gdn_recurrence_decode(st, qd, kd, vd, g.reshape(1, T, H), on_dev(inp["beta"]), y,
                                scale=wl.scale)
    n = torch.empty(T, H, S, device=DEV)
    gdn().gdn_gated_rmsnorm(y.reshape(T, H, S), on_dev(inp["norm_w"]), on_dev(inp["z"]), n,
                            eps=wl.norm_eps)

    g_r = oracle.decay_gate(inp["alpha"], inp["dt"], inp["a"]).reshape(1, T, H)
    o_r, _, _ = oracle.conv1d_silu_l2norm(inp["x"], inp["conv_w"], inp["conv_hist"],
                                          wl.qk_channels, wl.head_dim, wl.l2_eps)
    q_r = o_r[0, :, :H * S].reshape(1, T, H, S)
    k_r = o_r[0, :, H * S:2 * H * S].reshape(1, T, H, S)
    v_r = o_r[0, :, 2 * H * S:].reshape(1, T, H, S)
    y_r, _, _ = oracle.recurrence_seq(inp["state"], q_r, k_r, v_r, g_r, inp["beta"], wl.scale)
    n_r = oracle.gated_rmsnorm(y_r.reshape(T, H, S), inp["norm_w"], inp["z"], wl.norm_eps)
    assert rel(n, n_r) < 1e-4


# ------------------------------------------------------------------------------------- fused decode

@pytest.mark.parametrize("name,opt,shape", [
    ("tiny", True, None), ("decode", True, None), ("decode", False, None),
    ("decode64", True, None), ("verify2", True, None),
    ("tiny", True, dict(S=64, head_dim=64, H=6, Hk=3, n_tok=3, n_seq=2)),
    ("tiny", True, dict(S=256, head_dim=256, H=2, Hk=1, n_tok=2, n_seq=2))])
def test_decode_fused_bit_identical_to_three_calls(name, opt, shape):
    # gate -> recurrence -> norm in one launch against the three separate calls
    # (bit for bit: same operations in the same order) and the fp64 oracle chain
    inp = inputs(name) if shape is None else make_inputs(name, seed=41, state_std=0.1, **shape)
    wl = inp["wl"]
    n, T, H, S = wl.n_seq, wl.n_tok, wl.H, wl.S
    assert wl.head_dim == S
    log_case("decode_fused", wl=name, n_seq=n, n_tok=T, H=H, S=S, optional_outputs=opt)
    snap = 1 < T <= 8
    d = {k: on_dev(inp[k]) for k in ("alpha", "dt", "a", "beta", "q", "k", "v", "norm_w", "z")}
    nan = float("nan")
    g3 = torch.empty(n * T, H, device=DEV)
    gdn().gdn_decay_gate(d["alpha"], d["dt"], d["a"], g3)
    st3 = on_dev(inp["state"]).clone()
    y3 = torch.empty(n, T, H, S, device=DEV)
    sn3 = torch.full((n, T - 1, H, S, S), nan, device=DEV) if snap else None
    gdn().gdn_recurrence_decode(st3, d["q"], d["k"], d["v"], g3.view(n, T, H), d["beta"], y3,
                                scale=wl.scale, snap=sn3)
    o3 = torch.empty(n * T, H, S, device=DEV)
    gdn().gdn_gated_rmsnorm(y3.view(n * T, H, S), d["norm_w"], d["z"], o3, eps=wl.norm_eps)

    stf = on_dev(inp["state"]).clone()
    of = torch.full((n, T, H, S), nan, device=DEV)
    gf = torch.full((n, T, H), nan, device=DEV) if opt else None
    yf = torch.full((n, T, H, S), nan, device=DEV) if opt else None
    snf = torch.full((n, T - 1, H, S, S), nan, device=DEV) if snap else None
    gdn().gdn_decode_fused(stf, d["q"], d["k"], d["v"], d["alpha"].view(n, T, H), d["dt"],
                           d["a"], d["beta"], d["norm_w"], d["z"].view(n, T, H, S), of,
                           scale=wl.scale, norm_eps=wl.norm_eps, g=gf, y=yf, snap=snf)
    assert bits_equal(of, o3.view(n, T, H, S))
    assert bits_equal(stf, st3)
    if opt:
        assert bits_equal(gf, g3.view(n, T, H)) and bits_equal(yf, y3)
    if snap:
        assert bits_equal(snf, sn3)

    g_ref = oracle.decay_gate(inp["alpha"], inp["dt"], inp["a"]).reshape(n, T, H)
    y_ref, s_ref, _ = oracle.recurrence_seq(inp["state"], inp["q"], inp["k"], inp["v"], g_ref,
                                            inp["beta"], wl.scale)
    o_ref = oracle.gated_rmsnorm(y_ref.reshape(n * T, H, S), inp["norm_w"], inp["z"],
                                 wl.norm_eps)
    assert rel(of.view(n * T, H, S), o_ref) < 1e-4
    assert rel(stf, s_ref) < 1e-4


# ------------------------------------------------------------------------------------- fused step

def step_shape(S, H, Hk, n_tok, n_seq, D=4, x_pad=0):
    """Workload overrides for a conv row laid out q | k | v (head width S)."""
    C = (2 * Hk + H) * S
    return dict(S=S, head_dim=S, H=H, Hk=Hk, n_tok=n_tok, n_seq=n_seq, d_conv=D, conv_dim=C,
                qk_channels=2 * Hk * S, x_stride=C + x_pad, out_stride=C, state_std=0.1,
                hist_std=1.0)


def step_two_ways(inp, opt=True, ws=None):
    """The decode step as one gdn_decode_step launch and as gdn_conv1d_silu_l2norm
    into a buffer followed by gdn_decode_fused; returns both results."""
    wl = inp["wl"]
    n, T, H, Hk, S, C, D = wl.n_seq, wl.n_tok, wl.H, wl.Hk, wl.S, wl.conv_dim, wl.d_conv
    nan = float("nan")
    d = {k: on_dev(inp[k]) for k in ("alpha", "dt", "a", "beta", "norm_w", "z", "x", "conv_w")}
    x = d["x"][:, :, :C]
    alpha3, z4 = d["alpha"].view(n, T, H), d["z"].view(n, T, H, S)
    snap = T > 1

    def outs():
        return dict(state=on_dev(inp["state"]).clone(), hist=on_dev(inp["conv_hist"]).clone(),
                    out=torch.full((n, T, H, S), nan, device=DEV),
                    g=torch.full((n, T, H), nan, device=DEV) if opt else None,
                    y=torch.full((n, T, H, S), nan, device=DEV) if opt else None,
                    snap=torch.full((n, T - 1, H, S, S), nan, device=DEV) if snap else None,
                    csnap=torch.full((n, T - 1, C, D - 1), nan, device=DEV) if snap else None)

    r = outs()
    cout = torch.full((n, T, C), nan, device=DEV)
    gdn().gdn_conv1d_silu_l2norm(x, d["conv_w"], r["hist"], cout, qk_channels=2 * Hk * S,
                                 head_dim=S, l2_eps=wl.l2_eps, snap=r["csnap"])
    q = cout[:, :, :Hk * S].unflatten(-1, (Hk, S))
    k = cout[:, :, Hk * S:2 * Hk * S].unflatten(-1, (Hk, S))
    v = cout[:, :, 2 * Hk * S:].unflatten(-1, (H, S))
    gdn().gdn_decode_fused(r["state"], q, k, v, alpha3, d["dt"], d["a"], d["beta"], d["norm_w"],
                           z4, r["out"], scale=wl.scale, norm_eps=wl.norm_eps, g=r["g"], y=r["y"],
                           snap=r["snap"])
    f = outs()
    if ws is None:
        ws = torch.zeros(gdn().gdn_decode_step_workspace_bytes(n, Hk) // 4, dtype=torch.int32,
                         device=DEV)
    gdn().gdn_decode_step(f["state"], x, d["conv_w"], f["hist"], alpha3, d["dt"], d["a"],
                          d["beta"], d["norm_w"], z4, f["out"], scale=wl.scale, l2_eps=wl.l2_eps,
                          norm_eps=wl.norm_eps, workspace=ws, g=f["g"], y=f["y"], snap=f["snap"],
                          conv_snap=f["csnap"])
    return r, f, ws


STEP_CASES = [("decode64", None), ("verify2", None), ("decode", None),
              ("tiny", dict(n_tok=4)),                                    # H == Hk: no tickets
              ("tiny", step_shape(32, 6, 2, 3, 2, D=2)),
              ("tiny", step_shape(64, 6, 3, 4, 2, D=3, x_pad=8)),
              ("tiny", step_shape(256, 4, 2, 2, 3)),
              ("tiny", step_shape(128, 4, 1, 8, 2)),                      # 8 positions, G = 4
              ("tiny", step_shape(128, 4, 2, 17, 2)),                     # K = 17 verify
              ("tiny", step_shape(256, 2, 1, 16, 2)),                     # most positions at S = 256
              ("tiny", step_shape(32, 6, 2, 32, 2, D=3)),                 # most positions
              ("tiny", step_shape(128, 4, 4, 2, 2))]


@pytest.mark.parametrize("name,shape", STEP_CASES)
def test_decode_step_bit_identical_to_conv_then_fused(name, shape):
    inp = inputs(name) if shape is None else make_inputs(name, seed=43, **shape)
    wl = inp["wl"]
    log_case("decode_step", wl=name, n_seq=wl.n_seq, n_tok=wl.n_tok, H=wl.H, Hk=wl.Hk, S=wl.S,
             D=wl.d_conv)
    r, f, ws = step_two_ways(inp)
    for key in r:
        if r[key] is not None:
            assert bits_equal(f[key], r[key]), key
    assert int(ws.abs().sum()) == 0          # the tickets are reset for the next call


def test_decode_step_twice_in_a_row():
    # state and conv history carried from one call to the next; the second call
    # reuses the first's workspace, which must have come back zero-filled
    inp = make_inputs("verify2", seed=47)
    wl = inp["wl"]
    log_case("decode_step_twice", n_seq=wl.n_seq, n_tok=wl.n_tok)
    r1, f1, ws = step_two_ways(inp, opt=False)
    assert bits_equal(f1["state"], r1["state"]) and bits_equal(f1["hist"], r1["hist"])
    inp2 = dict(inp)
    inp2["state"], inp2["conv_hist"] = r1["state"].cpu(), r1["hist"].cpu()
    inp2["x"] = make_inputs("verify2", seed=48)["x"]
    r2, f2, _ = step_two_ways(inp2, opt=False, ws=ws)
    for key in ("state", "hist", "out", "snap", "csnap"):
        assert bits_equal(f2[key], r2[key]), key
    assert int(ws.abs().sum()) == 0


def test_decode_step_verify_equals_two_single_steps():
    # K = 2 in one launch (snapshots inline) against two one-position launches:
    # outputs, final state and history bit for bit, and the position-0
    # snapshots equal to the state and history after the first one-position step
    inp = make_inputs("verify2", seed=53)
    wl = inp["wl"]
    n, T, H, Hk, S, C, D = wl.n_seq, wl.n_tok, wl.H, wl.Hk, wl.S, wl.conv_dim, wl.d_conv
    assert T == 2
    log_case("decode_step_verify_vs_steps", n_seq=n, H=H)
    d = {k: on_dev(inp[k]) for k in ("alpha", "dt", "a", "beta", "norm_w", "z", "x", "conv_w")}
    x = d["x"][:, :, :C]
    alpha3, z4 = d["alpha"].view(n, T, H), d["z"].view(n, T, H, S)
    nan = float("nan")
    ws = torch.zeros(gdn().gdn_decode_step_workspace_bytes(n, Hk) // 4, dtype=torch.int32,
                     device=DEV)
    kw = dict(scale=wl.scale, l2_eps=wl.l2_eps, norm_eps=wl.norm_eps, workspace=ws)

    st_k, hist_k = on_dev(inp["state"]).clone(), on_dev(inp["conv_hist"]).clone()
    out_k = torch.full((n, T, H, S), nan, device=DEV)
    snap = torch.full((n, 1, H, S, S), nan, device=DEV)
    csnap = torch.full((n, 1, C, D - 1), nan, device=DEV)
    gdn().gdn_decode_step(st_k, x, d["conv_w"], hist_k, alpha3, d["dt"], d["a"], d["beta"],
                          d["norm_w"], z4, out_k, snap=snap, conv_snap=csnap, **kw)

    st_1, hist_1 = on_dev(inp["state"]).clone(), on_dev(inp["conv_hist"]).clone()
    out_1 = torch.full((n, T, H, S), nan, device=DEV)
    for t in range(T):
        gdn().gdn_decode_step(st_1, x[:, t:t + 1], d["conv_w"], hist_1,
                              alpha3[:, t:t + 1].contiguous(), d["dt"], d["a"],
                              d["beta"][:, t:t + 1].contiguous(), d["norm_w"], z4[:, t:t + 1],
                              out_1[:, t:t + 1], **kw)
        if t == 0:
            assert bits_equal(snap[:, 0], st_1) and bits_equal(csnap[:, 0], hist_1)
    assert bits_equal(out_k, out_1)
    assert bits_equal(st_k, st_1) and bits_equal(hist_k, hist_1)
    assert int(ws.abs().sum()) == 0


def test_decode_step_against_oracle_chain():
    # conv -> gate -> recurrence -> norm in the fp64 oracle at the 64-sequence size
    inp = inputs("decode64")
    wl = inp["wl"]
    log_case("decode_step_oracle", n_seq=wl.n_seq, H=wl.H)
    n, T, H, Hk, S, C = wl.n_seq, wl.n_tok, wl.H, wl.Hk, wl.S, wl.conv_dim
    _, f, _ = step_two_ways(inp)
    o_r, hist_r, _ = oracle.conv1d_silu_l2norm(inp["x"][:, :, :C], inp["conv_w"],
                                               inp["conv_hist"], wl.qk_channels, wl.head_dim,
                                               wl.l2_eps)
    q_r = o_r[:, :, :Hk * S].reshape(n, T, Hk, S)
    k_r = o_r[:, :, Hk * S:2 * Hk * S].reshape(n, T, Hk, S)
    v_r = o_r[:, :, 2 * Hk * S:].reshape(n, T, H, S)
    g_r = oracle.decay_gate(inp["alpha"], inp["dt"], inp["a"]).reshape(n, T, H)
    y_r, s_r, _ = oracle.recurrence_seq(inp["state"], q_r, k_r, v_r, g_r, inp["beta"], wl.scale)
    n_r = oracle.gated_rmsnorm(y_r.reshape(n * T, H, S), inp["norm_w"], inp["z"], wl.norm_eps)
    assert rel(f["hist"], hist_r) == 0.0     # the history only holds raw inputs
    assert rel(f["out"].view(n * T, H, S), n_r) < 1e-4
    assert rel(f["state"], s_r) < 1e-4
    assert rel(f["g"], g_r) < 1e-5


# ------------------------------------------------------------------------------------- chunked

def run_chunked(inp, g3, state=None):
    wl = inp["wl"]
    st = on_dev(inp["state"] if state is None else state).clone()
    v = on_dev(inp["v"])
    y = torch.full_like(v, float("nan"))
    gdn().gdn_recurrence_chunked(st, on_dev(inp["q"]), on_dev(inp["k"]), v, on_dev(g3),
                                 on_dev(inp["beta"]), y, scale=wl.scale, chunk=64)
    return y, st


def test_chunked_prefill_full_size():
    inp = inputs("prefill")
    wl = inp["wl"]
    log_case("chunked_prefill", T=wl.n_tok, H=wl.H, Hk=wl.Hk)
    g3 = oracle_g(inp)
    y, st = run_chunked(inp, g3)
    y_ref, s_ref, _ = oracle.recurrence_seq(inp["state"], inp["q"], inp["k"], inp["v"], g3,
                                            inp["beta"], wl.scale)
    ey, es = rel(y, y_ref), rel(st, s_ref)
    print(f"[chunked prefill] rel err y {ey:.3e} state {es:.3e}", flush=True)
    assert ey < 2e-3 and es < 2e-3


@pytest.mark.parametrize("T,H,Hk,n_seq,g_scale", [(100, 4, 2, 2, 1.0), (37, 2, 2, 1, 1.0),
                                                  (64, 2, 1, 1, 1.0), (65, 2, 2, 3, 0.3),
                                                  (300, 2, 2, 1, 0.02)])
def test_chunked_ragged_and_weak_decay(T, H, Hk, n_seq, g_scale):
    # nonzero initial state; g_scale < 1 weakens the decay so the state carries
    # across many chunks (the inter-chunk path dominates)
    inp = make_inputs("prefill", seed=61, n_tok=T, H=H, Hk=Hk, n_seq=n_seq, state_std=0.05)
    wl = inp["wl"]
    log_case("chunked_ragged", T=T, H=H, Hk=Hk, n_seq=n_seq, g_scale=g_scale)
    g3 = (oracle_g(inp) * g_scale).float()
    y, st = run_chunked(inp, g3)
    y_ref, s_ref, _ = oracle.recurrence_seq(inp["state"], inp["q"], inp["k"], inp["v"], g3,
                                            inp["beta"], wl.scale)
    ey, es = rel(y, y_ref), rel(st, s_ref)
    print(f"[chunked] T={T} rel err y {ey:.3e} state {es:.3e}", flush=True)
    assert ey < 2e-3 and es < 2e-3


def degenerate_keys(T, Hk, S, gen):
    """Unit keys that stress the triangular solve: q/k head 0 repeats one key,
    head 1 alternates +k and -k, head 2 draws keys from a 3-dimensional
    subspace, any further head takes fresh random keys."""
    def unit(x):
        return x / x.norm(dim=-1, keepdim=True)
    k = unit(torch.randn(1, T, Hk, S, generator=gen, dtype=torch.float64))
    k0 = unit(torch.randn(S, generator=gen, dtype=torch.float64))
    k[0, :, 0] = k0
    if Hk > 1:
        sign = torch.tensor([1.0 if t % 2 == 0 else -1.0 for t in range(T)], dtype=torch.float64)
        k[0, :, 1] = sign[:, None] * k0[None, :]
    if Hk > 2:
        basis, _ = torch.linalg.qr(torch.randn(S, 3, generator=gen, dtype=torch.float64))
        k[0, :, 2] = unit(torch.randn(T, 3, generator=gen, dtype=torch.float64) @ basis.T)
    return k.float()


@pytest.mark.parametrize("S", [128, 64])
def test_chunked_degenerate_keys_no_decay(S):
    # the chunked form's contract (unit keys, beta |k|^2 <= 2, g <= 0) at its
    # edge: repeated, alternating and low-rank keys with beta = sigmoid(6) and
    # no decay at all, 4096 positions, against the sequential fp64 scan
    T, H, Hk = 4096, 6, 3
    inp = make_inputs("prefill", seed=79, n_tok=T, H=H, Hk=Hk, S=S, head_dim=S)
    wl = inp["wl"]
    log_case("chunked_degenerate", T=T, H=H, Hk=Hk, S=S)
    gen = torch.Generator("cpu").manual_seed(80)
    inp = dict(inp)
    inp["k"] = degenerate_keys(T, Hk, S, gen)
    inp["beta"] = torch.full_like(inp["beta"], float(1.0 / (1.0 + math.exp(-6.0))))
    g3 = torch.zeros(1, T, H)
    y, st = run_chunked(inp, g3)
    y_ref, s_ref, _ = oracle.recurrence_seq(inp["state"], inp["q"], inp["k"], inp["v"], g3,
                                            inp["beta"], wl.scale)
    ey, es = rel(y, y_ref), rel(st, s_ref)
    print(f"[chunked degenerate keys S={S}] rel err y {ey:.3e} state {es:.3e}", flush=True)
    assert ey < 2e-3 and es < 2e-3


@pytest.mark.parametrize("v_scale,state_std", [(3000.0, 100.0), (1e-3, 1e-4)])
def test_chunked_large_and_small_magnitudes(v_scale, state_std):
    # values far from 1: the scan's fp16 operand splits are scaled by powers of
    # two from a running norm bound, so neither large nor tiny states and
    # values lose range or precision; 1000 positions, paired and 8-wave scans
    for H, Hk in ((4, 2), (40, 8)):
        inp = make_inputs("prefill", seed=83, n_tok=1000, H=H, Hk=Hk, state_std=state_std)
        wl = inp["wl"]
        log_case("chunked_magnitudes", v_scale=v_scale, state_std=state_std, H=H)
        inp = dict(inp)
        inp["v"] = inp["v"] * v_scale
        g3 = oracle_g(inp) * 0.05
        y, st = run_chunked(inp, g3)
        y_ref, s_ref, _ = oracle.recurrence_seq(inp["state"], inp["q"], inp["k"], inp["v"], g3,
                                                inp["beta"], wl.scale)
        ey, es = rel(y, y_ref), rel(st, s_ref)
        print(f"[chunked magnitudes v x{v_scale} state {state_std}] H={H} rel err y {ey:.3e} "
              f"state {es:.3e}", flush=True)
        assert ey < 2e-3 and es < 2e-3


@pytest.mark.parametrize("T,H,Hk,n_seq", [(130, 33, 11, 1), (64, 20, 5, 2)])
def test_chunked_paired_scan_grid(T, H, Hk, n_seq):
    # more than 256 sequence x head x 16-column units, so the scan runs as
    # 16-wave workgroups over pairs of value blocks; 33 heads give a grid of
    # 132 workgroups, not a multiple of the 8 XCDs
    inp = make_inputs("prefill", seed=67, n_tok=T, H=H, Hk=Hk, n_seq=n_seq, state_std=0.05)
    wl = inp["wl"]
    log_case("chunked_paired", T=T, H=H, Hk=Hk, n_seq=n_seq)
    assert n_seq * H * 8 > 256
    g3 = oracle_g(inp)
    y, st = run_chunked(inp, g3)
    y_ref, s_ref, _ = oracle.recurrence_seq(inp["state"], inp["q"], inp["k"], inp["v"], g3,
                                            inp["beta"], wl.scale)
    ey, es = rel(y, y_ref), rel(st, s_ref)
    print(f"[chunked paired] H={H} rel err y {ey:.3e} state {es:.3e}", flush=True)
    assert ey < 2e-3 and es < 2e-3


def test_chunked_paired_scan_bit_identical():
    # heads are independent: one call over 48 heads (paired 16-wave scan) must
    # equal, bit for bit, two calls over 24 heads each (8-wave scan, 192
    # workgroups), since both forms run the same per-wave arithmetic
    n, T, H, Hk = 1, 200, 48, 16
    inp = make_inputs("prefill", seed=73, n_tok=T, H=H, Hk=Hk, n_seq=n, state_std=0.05)
    wl = inp["wl"]
    log_case("chunked_paired_bits", T=T, H=H, Hk=Hk)
    q, k, v, beta = (on_dev(inp[x]) for x in ("q", "k", "v", "beta"))
    g3 = on_dev(oracle_g(inp))
    st_full = on_dev(inp["state"]).clone()
    y_full = torch.full_like(v, float("nan"))
    gdn().gdn_recurrence_chunked(st_full, q, k, v, g3, beta, y_full, scale=wl.scale, chunk=64)
    st_half = on_dev(inp["state"]).clone()
    y_half = torch.full_like(v, float("nan"))
    hv, hk = H // 2, Hk // 2
    for i in range(2):
        vs, ks = slice(i * hv, (i + 1) * hv), slice(i * hk, (i + 1) * hk)
        gdn().gdn_recurrence_chunked(st_half[:, vs], q[:, :, ks], k[:, :, ks], v[:, :, vs],
                                     g3[:, :, vs].contiguous(), beta[:, :, vs].contiguous(),
                                     y_half[:, :, vs], scale=wl.scale, chunk=64)
    assert bits_equal(y_full, y_half)
    assert bits_equal(st_full, st_half)


@pytest.mark.parametrize("S,T,H,Hk,n_seq,g_scale", [(32, 64, 4, 4, 1, 1.0),      # the 64-token workload
                                                   (32, 100, 4, 2, 2, 1.0),
                                                   (64, 200, 3, 1, 2, 0.05),
                                                   (64, 37, 2, 2, 1, 1.0)])
def test_chunked_small_state(S, T, H, Hk, n_seq, g_scale):
    # S = 32 and 64: the one-pass fp32 chunked form, no workspace, against the
    # sequential scan; ragged last chunks, GQA, nonzero and weakly decaying state
    inp = make_inputs("tiny", seed=79, S=S, head_dim=S, n_tok=T, H=H, Hk=Hk, n_seq=n_seq,
                      state_std=0.1)
    wl = inp["wl"]
    log_case("chunked_small", S=S, T=T, H=H, Hk=Hk, n_seq=n_seq)
    assert gdn().gdn_recurrence_chunked_workspace_bytes(n_seq, T, H, Hk, S, 64) == 0
    g3 = (oracle_g(inp) * g_scale).float()
    st = on_dev(inp["state"]).clone()
    v = on_dev(inp["v"])
    y = torch.full_like(v, float("nan"))
    gdn().gdn_recurrence_chunked(st, on_dev(inp["q"]), on_dev(inp["k"]), v, on_dev(g3),
                                 on_dev(inp["beta"]), y, scale=wl.scale, chunk=64)
    y_ref, s_ref, _ = oracle.recurrence_seq(inp["state"], inp["q"], inp["k"], inp["v"], g3,
                                            inp["beta"], wl.scale)
    ey, es = rel(y, y_ref), rel(st, s_ref)
    print(f"[chunked S={S}] rel err y {ey:.3e} state {es:.3e}", flush=True)
    assert ey < 2e-3 and es < 2e-3


def pack_varlen(inp, lens, g3):
    """First lens[s] positions of every sequence, packed along one token axis."""
    take = lambda t: torch.cat([t[s, :n] for s, n in enumerate(lens)], 0)
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    return {"q": take(inp["q"]), "k": take(inp["k"]), "v": take(inp["v"]), "g": take(g3),
            "beta": take(inp["beta"]), "cu": cu}


@pytest.mark.parametrize("S,lens,H,Hk,g_scale", [
    (128, [100, 0, 64, 300, 1, 129], 4, 2, 1.0),                  # 8-wave scan grid
    (128, [64, 200, 37, 130, 0, 65, 3, 90, 150], 6, 3, 0.3),       # paired scan grid
    (128, [1000, 1500, 596, 1000], 32, 16, 1.0),                  # the 4096-token prompt, split
    (32, [64, 17, 0, 100], 4, 2, 1.0),
    (64, [37, 129, 5], 3, 1, 0.05)])
def test_chunked_varlen(S, lens, H, Hk, g_scale):
    # one packed call over sequences of different lengths from nonzero states:
    # every sequence bit for bit as a call on it alone, and within the chunked
    # tolerance of the sequential scan; empty sequences keep their state
    base = "prefill" if S == 128 else "tiny"
    inp = make_inputs(base, seed=83, S=S, head_dim=S, n_tok=max(lens), H=H, Hk=Hk,
                      n_seq=len(lens), state_std=0.05)
    wl = inp["wl"]
    log_case("chunked_varlen", S=S, lens=lens, H=H, Hk=Hk)
    g3 = (oracle_g(inp) * g_scale).float()
    pk = pack_varlen(inp, lens, g3)
    total = pk["cu"][-1]
    # v and y as strided views of wider rows; y poisoned
    vbuf = torch.full((total, H * S + 8), float("nan"), device=DEV)
    vbuf[:, :H * S] = on_dev(pk["v"]).reshape(total, H * S)
    v = vbuf[:, :H * S].unflatten(1, (H, S))
    ybuf = torch.full((total, H * S + 8), float("nan"), device=DEV)
    y = ybuf[:, :H * S].unflatten(1, (H, S))
    st = on_dev(inp["state"]).clone()
    gdn().gdn_recurrence_chunked_varlen(st, on_dev(pk["q"]), on_dev(pk["k"]), v, on_dev(pk["g"]),
                                        on_dev(pk["beta"]), y, pk["cu"], scale=wl.scale, chunk=64)
    assert torch.isnan(ybuf[:, H * S:]).all(), "write outside y's rows"
    for s, n in enumerate(lens):
        st1 = on_dev(inp["state"][s:s + 1]).clone()
        if n == 0:
            assert bits_equal(st[s:s + 1], st1)
            continue
        sl = slice(pk["cu"][s], pk["cu"][s + 1])
        y1 = torch.full((1, n, H, S), float("nan"), device=DEV)
        gdn().gdn_recurrence_chunked(st1, on_dev(pk["q"][sl])[None], on_dev(pk["k"][sl])[None],
                                     v[sl][None], on_dev(pk["g"][sl])[None],
                                     on_dev(pk["beta"][sl])[None], y1, scale=wl.scale, chunk=64)
        assert bits_equal(y[sl], y1[0]), f"sequence {s}: y differs from its own call"
        assert bits_equal(st[s:s + 1], st1), f"sequence {s}: state differs from its own call"
        y_ref, s_ref, _ = oracle.recurrence_seq(
            inp["state"][s:s + 1], pk["q"][sl][None], pk["k"][sl][None], pk["v"][sl][None],
            pk["g"][sl][None], pk["beta"][sl][None], wl.scale)
        ey, es = rel(y[sl][None], y_ref), rel(st[s:s + 1], s_ref)
        print(f"[chunked varlen S={S}] seq {s} len {n} rel err y {ey:.3e} state {es:.3e}",
              flush=True)
        assert ey < 2e-3 and es < 2e-3


@pytest.mark.parametrize("S", [128, 64])
def test_chunked_varlen_most_sequences(S):
    # the largest packed batch a call takes (256 sequences), lengths 0 .. 150
    # including empty ones and exact chunk multiples: every sequence bit for bit
    # as a call on it alone (on a sample of sequences), and the empty ones untouched
    n_seq, H, Hk = 256, 2, 1
    rng = np.random.default_rng(7)
    lens = [int(x) for x in rng.integers(0, 151, n_seq)]
    lens[:6] = [0, 64, 128, 1, 63, 65]
    base = "prefill" if S == 128 else "tiny"
    inp = make_inputs(base, seed=103, S=S, head_dim=S, n_tok=max(lens), H=H, Hk=Hk,
                      n_seq=n_seq, state_std=0.05)
    wl = inp["wl"]
    log_case("chunked_varlen_max", S=S, n_seq=n_seq, total=sum(lens))
    pk = pack_varlen(inp, lens, oracle_g(inp))
    st = on_dev(inp["state"]).clone()
    y = torch.full((pk["cu"][-1], H, S), float("nan"), device=DEV)
    gdn().gdn_recurrence_chunked_varlen(st, on_dev(pk["q"]), on_dev(pk["k"]), on_dev(pk["v"]),
                                        on_dev(pk["g"]), on_dev(pk["beta"]), y, pk["cu"],
                                        scale=wl.scale, chunk=64)
    assert not torch.isnan(y).any()
    for s in list(range(8)) + [100, 200, 255]:
        n = lens[s]
        st1 = on_dev(inp["state"][s:s + 1]).clone()
        if n == 0:
            assert bits_equal(st[s:s + 1], st1)
            continue
        sl = slice(pk["cu"][s], pk["cu"][s + 1])
        y1 = torch.empty((1, n, H, S), device=DEV)
        gdn().gdn_recurrence_chunked(st1, on_dev(pk["q"][sl])[None], on_dev(pk["k"][sl])[None],
                                     on_dev(pk["v"][sl])[None], on_dev(pk["g"][sl])[None],
                                     on_dev(pk["beta"][sl])[None], y1, scale=wl.scale, chunk=64)
        assert bits_equal(y[sl], y1[0]) and bits_equal(st[s:s + 1], st1), s
    for s in (3, 255):   # and against the sequential scan
        if lens[s] == 0:
            continue
        sl = slice(pk["cu"][s], pk["cu"][s + 1])
        y_ref, s_ref, _ = oracle.recurrence_seq(
            inp["state"][s:s + 1], pk["q"][sl][None], pk["k"][sl][None], pk["v"][sl][None],
            pk["g"][sl][None], pk["beta"][sl][None], wl.scale)
        assert rel(y[sl][None], y_ref) < 2e-3 and rel(st[s:s + 1], s_ref) < 2e-3


@pytest.mark.parametrize("S,H,Hk", [(128, 4, 2), (64, 3, 1), (32, 4, 4)])
def test_chunked_varlen_bf16_inputs(S, H, Hk):
    # bf16 q, k, v are widened exactly on load: the call must equal, bit for
    # bit, the fp32 call on the same (bf16-representable) values, and match the
    # sequential scan on them
    lens = [100, 0, 300, 65]
    base = "prefill" if S == 128 else "tiny"
    inp = make_inputs(base, seed=89, S=S, head_dim=S, n_tok=max(lens), H=H, Hk=Hk,
                      n_seq=len(lens), state_std=0.05)
    wl = inp["wl"]
    log_case("chunked_varlen_bf16", S=S, lens=lens, H=H, Hk=Hk)
    pk = pack_varlen(inp, lens, oracle_g(inp))
    qb, kb, vb = (on_dev(pk[x]).bfloat16() for x in ("q", "k", "v"))
    g, beta = on_dev(pk["g"]), on_dev(pk["beta"])
    st_b = on_dev(inp["state"]).clone()
    y_b = torch.full((pk["cu"][-1], H, S), float("nan"), device=DEV)
    gdn().gdn_recurrence_chunked_varlen(st_b, qb, kb, vb, g, beta, y_b, pk["cu"],
                                        scale=wl.scale, chunk=64)
    st_f = on_dev(inp["state"]).clone()
    y_f = torch.full_like(y_b, float("nan"))
    qf, kf, vf = qb.float(), kb.float(), vb.float()
    gdn().gdn_recurrence_chunked_varlen(st_f, qf, kf, vf, g, beta, y_f, pk["cu"],
                                        scale=wl.scale, chunk=64)
    assert bits_equal(y_b, y_f) and bits_equal(st_b, st_f)
    for s, n in enumerate(lens):
        if n == 0:
            continue
        sl = slice(pk["cu"][s], pk["cu"][s + 1])
        y_ref, s_ref, _ = oracle.recurrence_seq(
            inp["state"][s:s + 1], qf[sl].cpu()[None], kf[sl].cpu()[None], vf[sl].cpu()[None],
            pk["g"][sl][None], pk["beta"][sl][None], wl.scale)
        ey, es = rel(y_b[sl][None], y_ref), rel(st_b[s:s + 1], s_ref)
        assert ey < 2e-3 and es < 2e-3, (s, ey, es)


def test_chunked_deterministic():
    inp = make_inputs("prefill", seed=71, n_tok=512)
    log_case("chunked_determinism")
    g3 = oracle_g(inp)
    ya, sa = run_chunked(inp, g3)
    yb, sb = run_chunked(inp, g3)
    assert bits_equal(ya, yb) and bits_equal(sa, sb)


# ------------------------------------------------------------------------------- fused prefill

def prefill_two_ways(inp):
    """The prefill core as one gdn_prefill_chunked call and as gdn_decay_gate +
    gdn_conv1d_silu_l2norm into a buffer + gdn_recurrence_chunked on its q, k,
    v channels; returns both results (state, conv history, y)."""
    wl = inp["wl"]
    n, T, H, Hk, S, C = wl.n_seq, wl.n_tok, wl.H, wl.Hk, wl.S, wl.conv_dim
    nan = float("nan")
    d = {k: on_dev(inp[k]) for k in ("alpha", "dt", "a", "beta", "x", "conv_w")}
    x = d["x"][:, :, :C]

    def outs():
        return dict(state=on_dev(inp["state"]).clone(), hist=on_dev(inp["conv_hist"]).clone(),
                    y=torch.full((n, T, H, S), nan, device=DEV))

    r = outs()
    g = torch.full((n * T, H), nan, device=DEV)
    gdn().gdn_decay_gate(d["alpha"], d["dt"], d["a"], g)
    cout = torch.full((n, T, C), nan, device=DEV)
    gdn().gdn_conv1d_silu_l2norm(x, d["conv_w"], r["hist"], cout, qk_channels=2 * Hk * S,
                                 head_dim=S, l2_eps=wl.l2_eps)
    q = cout[:, :, :Hk * S].unflatten(-1, (Hk, S))
    k = cout[:, :, Hk * S:2 * Hk * S].unflatten(-1, (Hk, S))
    v = cout[:, :, 2 * Hk * S:].unflatten(-1, (H, S))
    gdn().gdn_recurrence_chunked(r["state"], q, k, v, g.view(n, T, H), d["beta"], r["y"],
                                 scale=wl.scale)
    f = outs()
    gdn().gdn_prefill_chunked(f["state"], x, d["conv_w"], f["hist"], d["alpha"].view(n, T, H),
                              d["dt"], d["a"], d["beta"], f["y"], scale=wl.scale,
                              l2_eps=wl.l2_eps)
    return r, f


PREFILL_CASES = [("prefill", None),                                     # 4096 x 32 / 16 heads
                 ("tiny", step_shape(128, 8, 4, 130, 2)),               # ragged, two sequences
                 ("tiny", step_shape(128, 4, 2, 1, 1)),                 # one position: history
                 ("tiny", step_shape(128, 4, 4, 2, 2)),                 # two positions, G = 1
                 ("tiny", step_shape(128, 6, 3, 67, 3, x_pad=8)),       # padded rows
                 ("tiny", step_shape(128, 4, 1, 64, 1)),                # one chunk, G = 4
                 ("tiny", step_shape(128, 24, 8, 200, 2))]              # the paired scan's grid


@pytest.mark.parametrize("name,shape", PREFILL_CASES)
def test_prefill_fused_bit_identical_to_three_calls(name, shape):
    inp = inputs(name) if shape is None else make_inputs(name, seed=47, **shape)
    wl = inp["wl"]
    log_case("prefill_fused", n_seq=wl.n_seq, n_tok=wl.n_tok, H=wl.H, Hk=wl.Hk)
    r, f = prefill_two_ways(inp)
    for key in r:
        assert bits_equal(f[key], r[key]), key


def test_prefill_fused_workspace_contents_and_graph_replay():
    # a NaN-filled workspace gives the zeroed workspace's bits; the two launches
    # captured in a HIP graph and replayed three times (eager work between the
    # replays) give the eager call's bits every time
    inp = make_inputs("tiny", seed=59, **step_shape(128, 4, 2, 150, 1))
    wl = inp["wl"]
    n, T, H, Hk, S, C = wl.n_seq, wl.n_tok, wl.H, wl.Hk, wl.S, wl.conv_dim
    log_case("prefill_fused_ws_graph", n_tok=T)
    d = {k: on_dev(inp[k]) for k in ("alpha", "dt", "a", "beta", "x", "conv_w")}
    x, a3 = d["x"][:, :, :C], d["alpha"].view(n, T, H)
    nb = gdn().gdn_prefill_chunked_workspace_bytes(n, T, H, Hk, S)

    def run(ws, st, hist, y):
        gdn().gdn_prefill_chunked(st, x, d["conv_w"], hist, a3, d["dt"], d["a"], d["beta"], y,
                                  scale=wl.scale, l2_eps=wl.l2_eps, workspace=ws)

    def fresh():
        return (on_dev(inp["state"]).clone(), on_dev(inp["conv_hist"]).clone(),
                torch.full((n, T, H, S), float("nan"), device=DEV))

    ref = fresh()
    run(torch.zeros(nb, dtype=torch.uint8, device=DEV), *ref)
    ws = torch.full((nb,), 255, dtype=torch.uint8, device=DEV)   # fp32 NaN patterns
    got = fresh()
    run(ws, *got)
    for a, b in zip(got, ref):
        assert bits_equal(a, b)
    st, hist, y = fresh()
    st0, hist0 = st.clone(), hist.clone()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(ws, st, hist, y)
    for _ in range(3):
        st.copy_(st0)
        hist.copy_(hist0)
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip((st, hist, y), ref):
            assert bits_equal(a, b)


def test_prefill_fused_against_oracle_chain():
    # conv -> gate -> sequential recurrence in the fp64 oracle, ragged, two
    # sequences with their own histories and states
    inp = make_inputs("tiny", seed=53, **step_shape(128, 4, 2, 100, 2))
    wl = inp["wl"]
    n, T, H, Hk, S, C = wl.n_seq, wl.n_tok, wl.H, wl.Hk, wl.S, wl.conv_dim
    log_case("prefill_fused_oracle", n_seq=n, n_tok=T)
    _, f = prefill_two_ways(inp)
    o_r, hist_r, _ = oracle.conv1d_silu_l2norm(inp["x"][:, :, :C], inp["conv_w"],
                                               inp["conv_hist"], wl.qk_channels, wl.head_dim,
                                               wl.l2_eps)
    q_r = o_r[:, :, :Hk * S].reshape(n, T, Hk, S)
    k_r = o_r[:, :, Hk * S:2 * Hk * S].reshape(n, T, Hk, S)
    v_r = o_r[:, :, 2 * Hk * S:].reshape(n, T, H, S)
    g_r = oracle.decay_gate(inp["alpha"], inp["dt"], inp["a"]).reshape(n, T, H)
    y_r, s_r, _ = oracle.recurrence_seq(inp["state"], q_r, k_r, v_r, g_r, inp["beta"], wl.scale)
    assert rel(f["hist"], hist_r) == 0.0     # the history only holds raw inputs
    ey, es = rel(f["y"], y_r), rel(f["state"], s_r)
    print(f"[prefill fused] rel err y {ey:.3e} state {es:.3e}", flush=True)
    assert ey < 2e-3 and es < 2e-3


# ------------------------------------------------------------------------------------- Mamba-2 SSD

def ssd_oracle(inp):
    n, T, H = inp["dt_raw"].shape
    dt = oracle.mamba2_dt(inp["dt_raw"].reshape(-1, H), inp["dt_bias"], inp["dt_min"],
                          inp["dt_max"]).reshape(n, T, H)
    return oracle.mamba2_ssd_seq(inp["state"], inp["x"], inp["B"], inp["C"], dt, inp["A_log"],
                                 inp["D"])


def run_ssd(inp, pad=0):
    """The GPU scan; with pad > 0, x, B, C, y are views into rows `pad` wider
    (y's gaps poisoned with NaN and checked afterwards)."""
    n, T, H, P = inp["x"].shape
    G, N = inp["B"].shape[2], inp["B"].shape[3]

    def wide(t, inner):
        buf = torch.full((n, T, inner + pad), float("nan"), device=DEV)
        buf[:, :, :inner] = on_dev(t).reshape(n, T, inner)
        return buf, buf[:, :, :inner]
    _, x = wide(inp["x"], H * P)
    _, Bm = wide(inp["B"], G * N)
    cbuf = torch.full((n, T, G * N + pad), float("nan"), device=DEV)
    cbuf[:, :, :G * N] = on_dev(inp["C"]).reshape(n, T, G * N)
    Cm = cbuf[:, :, :G * N]
    ybuf = torch.full((n, T, H * P + pad), float("nan"), device=DEV)
    y = ybuf[:, :, :H * P].unflatten(2, (H, P))
    st = on_dev(inp["state"]).clone()
    gdn().gdn_mamba2_ssd_chunked(st, x.unflatten(2, (H, P)), Bm.unflatten(2, (G, N)),
                                 Cm.unflatten(2, (G, N)), on_dev(inp["dt_raw"]),
                                 on_dev(inp["A_log"]), on_dev(inp["D"]), on_dev(inp["dt_bias"]),
                                 y, dt_min=inp["dt_min"], dt_max=inp["dt_max"])
    if pad:
        assert torch.isnan(ybuf[:, :, H * P:]).all(), "write outside y's rows"
    return y, st


@pytest.mark.parametrize("n,T,H,G,P,N,state_std,pad", [
    (1, 4096, 32, 1, 64, 128, 0.0, 0),       # a 4096-token prompt, 32 heads x 64, state 128
    (2, 100, 4, 2, 32, 64, 0.2, 8),
    (3, 1, 6, 3, 64, 64, 0.2, 0),
    (1, 65, 2, 1, 32, 128, 0.1, 4),
    (2, 200, 8, 4, 64, 128, 0.05, 0),
    (1, 1, 2, 1, 64, 128, 0.2, 0),           # the MFMA form: one position,
    (1, 65, 3, 3, 64, 128, 0.1, 0),          # a one-position last chunk,
    (2, 130, 4, 2, 64, 128, 0.2, 8)])        # strided rows with poisoned gaps
def test_mamba2_ssd_chunked(n, T, H, G, P, N, state_std, pad):
    inp = make_mamba2_inputs(n, T, H, G, P, N, seed=97, state_std=state_std)
    log_case("mamba2_ssd", n=n, T=T, H=H, G=G, P=P, N=N)
    y, st = run_ssd(inp, pad)
    y_ref, s_ref = ssd_oracle(inp)
    ey, es = rel(y, y_ref), rel(st, s_ref)
    print(f"[mamba2 ssd] T={T} rel err y {ey:.3e} state {es:.3e}", flush=True)
    assert ey < 1e-4 and es < 1e-4


def test_mamba2_ssd_deterministic():
    inp = make_mamba2_inputs(1, 300, 8, 2, 64, 128, seed=101, state_std=0.1)
    log_case("mamba2_ssd_determinism")
    ya, sa = run_ssd(inp)
    yb, sb = run_ssd(inp)
    assert bits_equal(ya, yb) and bits_equal(sa, sb)


def test_workspace_contents_do_not_matter():
    # every workspace value a chunked or Mamba-2 call reads is written earlier
    # in the same call (padding chunks and partial last chunks included): a
    # workspace filled with 0xFF bytes (NaN as fp32) gives, bit for bit, the
    # results of a zero-filled one
    log_case("workspace_contents")

    def both(call, nbytes):
        outs = []
        for fill in (0x00, 0xFF):
            ws = torch.full((max(nbytes, 1),), fill, dtype=torch.uint8, device=DEV)
            outs.append(call(ws))
        return outs

    # fixed-length chunked: 3 chunks per head, so the scan runs a padding chunk
    inp = make_inputs("prefill", seed=71, n_tok=130, H=4, Hk=2, n_seq=2, state_std=0.05)
    wl = inp["wl"]
    g3 = oracle_g(inp)

    def chunked(ws):
        st = on_dev(inp["state"]).clone()
        y = torch.full_like(on_dev(inp["v"]), float("nan"))
        gdn().gdn_recurrence_chunked(st, on_dev(inp["q"]), on_dev(inp["k"]), on_dev(inp["v"]),
                                     on_dev(g3), on_dev(inp["beta"]), y, scale=wl.scale,
                                     chunk=64, workspace=ws)
        return y, st
    (ya, sa), (yb, sb) = both(chunked, gdn().gdn_recurrence_chunked_workspace_bytes(
        2, 130, 4, 2, wl.S, 64))
    assert not torch.isnan(ya).any()
    assert bits_equal(ya, yb) and bits_equal(sa, sb)

    # packed prompts with an empty and a one-position sequence
    lens = [70, 0, 1, 129]
    inp = make_inputs("prefill", seed=73, n_tok=max(lens), H=4, Hk=2, n_seq=len(lens),
                      state_std=0.05)
    wl = inp["wl"]
    pk = pack_varlen(inp, lens, oracle_g(inp))

    def varlen(ws):
        st = on_dev(inp["state"]).clone()
        y = torch.full_like(on_dev(pk["v"]), float("nan"))
        gdn().gdn_recurrence_chunked_varlen(st, on_dev(pk["q"]), on_dev(pk["k"]), on_dev(pk["v"]),
                                            on_dev(pk["g"]), on_dev(pk["beta"]), y, pk["cu"],
                                            scale=wl.scale, chunk=64, workspace=ws)
        return y, st
    (ya, sa), (yb, sb) = both(varlen, gdn().gdn_recurrence_chunked_varlen_workspace_bytes(
        len(lens), pk["cu"][-1], 4, 2, wl.S, 64))
    assert not torch.isnan(ya).any()
    assert bits_equal(ya, yb) and bits_equal(sa, sb)

    # Mamba-2: a one-position last chunk, MFMA and VALU shapes
    for (H, G, P, N) in [(4, 2, 64, 128), (2, 1, 32, 64)]:
        mi = make_mamba2_inputs(2, 129, H, G, P, N, seed=79, state_std=0.1)

        def ssd(ws):
            st = on_dev(mi["state"]).clone()
            y = torch.full_like(on_dev(mi["x"]), float("nan"))
            gdn().gdn_mamba2_ssd_chunked(st, on_dev(mi["x"]), on_dev(mi["B"]), on_dev(mi["C"]),
                                         on_dev(mi["dt_raw"]), on_dev(mi["A_log"]),
                                         on_dev(mi["D"]), on_dev(mi["dt_bias"]), y,
                                         dt_min=mi["dt_min"], dt_max=mi["dt_max"], workspace=ws)
            return y, st
        (ya, sa), (yb, sb) = both(ssd, gdn().gdn_mamba2_ssd_workspace_bytes(2, 129, H, P, N, 64))
        assert not torch.isnan(ya).any()
        assert bits_equal(ya, yb) and bits_equal(sa, sb), (H, G, P, N)


# ------------------------------------------------------------------------------------- measurement aid

def test_stream_copy_exact():
    # the benchmark's bandwidth reference copies every byte, including a
    # ragged tail of the grid, and nothing else
    log_case("stream_copy")
    n = (1 << 20) + 12                                      # float4 count not a multiple of 256
    src = torch.randn(n * 4, device=DEV)
    dst = torch.full((n * 4 + 8,), float("nan"), device=DEV)
    gdn().gdn_stream_copy(dst[:n * 4], src)
    assert bits_equal(dst[:n * 4], src)
    assert torch.isnan(dst[n * 4:]).all()


# ------------------------------------------------------------------------------------- graph replay

def test_decode_step_graph_replay_matches_eager():
    # the decode step (gate -> conv -> recurrence -> norm) captured once into a
    # HIP graph and replayed several times, with eager work and synchronisation
    # between replays: every replay equals the eager step bit for bit
    inp = inputs("decode")
    wl = inp["wl"]
    log_case("graph_replay", wl="decode")
    n, T, H, Hk, S, C = wl.n_seq, wl.n_tok, wl.H, wl.Hk, wl.S, wl.conv_dim
    cu = {k: on_dev(v) for k, v in inp.items() if isinstance(v, torch.Tensor)}
    st = cu["state"].clone()
    hist = cu["conv_hist"].clone()
    conv_out = torch.empty(n, T, C, device=DEV)
    g = torch.empty(n * T, H, device=DEV)
    y = torch.empty(n, T, H, S, device=DEV)
    out = torch.empty(n * T, H, S, device=DEV)
    q = conv_out[..., :Hk * S].unflatten(-1, (Hk, S))
    k = conv_out[..., Hk * S:2 * Hk * S].unflatten(-1, (Hk, S))
    v = conv_out[..., 2 * Hk * S:].unflatten(-1, (H, S))

    def step():
        gdn().gdn_decay_gate(cu["alpha"], cu["dt"], cu["a"], g)
        gdn().gdn_conv1d_silu_l2norm(cu["x"][..., :C], cu["conv_w"], hist, conv_out,
                                     qk_channels=wl.qk_channels, head_dim=wl.head_dim,
                                     l2_eps=wl.l2_eps)
        gdn().gdn_recurrence_decode(st, q, k, v, g.view(n, T, H), cu["beta"], y, scale=wl.scale)
        gdn().gdn_gated_rmsnorm(y.view(n * T, H, S), cu["norm_w"], cu["z"], out,
                                eps=wl.norm_eps)

    def reset():
        st.copy_(cu["state"])
        hist.copy_(cu["conv_hist"])

    reset()
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, st, hist, g, y)]

    reset()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                    # warm up the allocator-free path
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    reset()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    for _ in range(3):
        reset()                                   # eager work between replays
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip((out, st, hist, g, y), ref):
            assert bits_equal(a, b)


def test_one_launch_step_graph_replay_matches_eager():
    # gdn_decode_step captured once into a HIP graph and replayed with eager
    # work between replays: every replay equals the eager call bit for bit and
    # leaves the ticket workspace at zero (two value heads share each q/k head)
    inp = inputs("decode")
    wl = inp["wl"]
    log_case("graph_replay_one_launch", wl="decode")
    n, T, H, Hk, S, C = wl.n_seq, wl.n_tok, wl.H, wl.Hk, wl.S, wl.conv_dim
    assert H > Hk
    cu = {k: on_dev(v) for k, v in inp.items() if isinstance(v, torch.Tensor)}
    st, hist = cu["state"].clone(), cu["conv_hist"].clone()
    out = torch.empty(n, T, H, S, device=DEV)
    ws = torch.zeros(gdn().gdn_decode_step_workspace_bytes(n, Hk) // 4, dtype=torch.int32,
                     device=DEV)

    def step():
        gdn().gdn_decode_step(st, cu["x"][..., :C], cu["conv_w"], hist,
                              cu["alpha"].view(n, T, H), cu["dt"], cu["a"], cu["beta"],
                              cu["norm_w"], cu["z"].view(n, T, H, S), out, scale=wl.scale,
                              l2_eps=wl.l2_eps, norm_eps=wl.norm_eps, workspace=ws)

    def reset():
        st.copy_(cu["state"])
        hist.copy_(cu["conv_hist"])

    reset()
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, st, hist)]
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        reset()
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    reset()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    for _ in range(3):
        reset()
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip((out, st, hist), ref):
            assert bits_equal(a, b)
        assert int(ws.abs().sum()) == 0


# ------------------------------------------------------------------------------------- degenerate cases

@pytest.mark.parametrize("path", ["decode", "chunked"])
def test_no_decay_no_update_keeps_state_bits(path):
    # g = 0 and beta = 0: S <- 1 * S and delta = 0, so the state must come back
    # bit for bit (chunked: A = 0, T = I, W = Ut = 0, e^{G_n} = 1), and y is the
    # readout of the unchanged state
    T = 3 if path == "decode" else 130
    inp = make_inputs("prefill", seed=91, n_tok=T, H=4, Hk=2, state_std=0.1)
    wl = inp["wl"]
    log_case("no_decay_no_update", path=path, T=T)
    g0 = torch.zeros(wl.n_seq, T, wl.H)
    b0 = torch.zeros(wl.n_seq, T, wl.H)
    st = on_dev(inp["state"]).clone()
    y = torch.empty(wl.n_seq, T, wl.H, wl.S, device=DEV)
    args = (st, on_dev(inp["q"]), on_dev(inp["k"]), on_dev(inp["v"]), on_dev(g0), on_dev(b0), y)
    if path == "decode":
        gdn().gdn_recurrence_decode(*args, scale=wl.scale)
    else:
        gdn().gdn_recurrence_chunked(*args, scale=wl.scale)
    assert bits_equal(st, on_dev(inp["state"]))
    y_ref, _, _ = oracle.recurrence_seq(inp["state"], inp["q"], inp["k"], inp["v"], g0, b0,
                                        wl.scale)
    assert rel(y, y_ref) < (1e-4 if path == "decode" else 2e-3)


@pytest.mark.parametrize("path", ["decode", "chunked"])
def test_total_decay_forgets_the_state(path):
    # g = -200: exp(g) underflows to 0 in fp32, so after a position the state
    # holds only that position's update, whatever it held before
    T = 2 if path == "decode" else 70
    inp = make_inputs("prefill", seed=93, n_tok=T, H=4, Hk=2, state_std=1.0)
    wl = inp["wl"]
    log_case("total_decay", path=path, T=T)
    g = torch.full((wl.n_seq, T, wl.H), -200.0)
    st = on_dev(inp["state"]).clone()
    y = torch.empty(wl.n_seq, T, wl.H, wl.S, device=DEV)
    args = (st, on_dev(inp["q"]), on_dev(inp["k"]), on_dev(inp["v"]), on_dev(g),
            on_dev(inp["beta"]), y)
    if path == "decode":
        gdn().gdn_recurrence_decode(*args, scale=wl.scale)
    else:
        gdn().gdn_recurrence_chunked(*args, scale=wl.scale)
    zero = np.zeros_like(inp["state"].numpy())
    y_ref, s_ref, _ = oracle.recurrence_seq(zero, inp["q"][:, -1:], inp["k"][:, -1:],
                                            inp["v"][:, -1:], g[:, -1:], inp["beta"][:, -1:],
                                            wl.scale)
    tol = 1e-4 if path == "decode" else 2e-3
    assert rel(st, s_ref) < tol
    assert rel(y[:, -1:], y_ref) < tol


def test_chunked_prefill_graph_replay_matches_eager():
    # a packed two-prompt chunked call (workspace passed in) and the Mamba-2
    # scan captured once into a HIP graph, replayed with eager work between
    # replays: every replay equals the eager calls bit for bit
    inp = make_inputs("prefill", seed=107, n_tok=200, H=4, Hk=2, n_seq=2, state_std=0.05)
    wl = inp["wl"]
    log_case("graph_replay_chunked")
    lens = [200, 77]
    pk = pack_varlen(inp, lens, oracle_g(inp))
    q, k, v, g, beta = (on_dev(pk[x]) for x in ("q", "k", "v", "g", "beta"))
    st0 = on_dev(inp["state"])
    st = st0.clone()
    y = torch.empty(sum(lens), wl.H, wl.S, device=DEV)
    ws = torch.empty(gdn().gdn_recurrence_chunked_varlen_workspace_bytes(2, sum(lens), wl.H,
                                                                       wl.Hk, wl.S, 64),
                     dtype=torch.uint8, device=DEV)
    mi = make_mamba2_inputs(1, 150, 4, 2, 64, 128, seed=109, state_std=0.1)
    mc = {kk: on_dev(vv) for kk, vv in mi.items() if isinstance(vv, torch.Tensor)}
    mst, my = mc["state"].clone(), torch.empty_like(mc["x"])
    mws = torch.empty(gdn().gdn_mamba2_ssd_workspace_bytes(1, 150, 4, 64, 128, 64),
                      dtype=torch.uint8, device=DEV)

    def run():
        gdn().gdn_recurrence_chunked_varlen(st, q, k, v, g, beta, y, pk["cu"], scale=wl.scale,
                                            chunk=64, workspace=ws)
        gdn().gdn_mamba2_ssd_chunked(mst, mc["x"], mc["B"], mc["C"], mc["dt_raw"], mc["A_log"],
                                     mc["D"], mc["dt_bias"], my, dt_min=mi["dt_min"],
                                     dt_max=mi["dt_max"], workspace=mws)

    def reset():
        st.copy_(st0)
        mst.copy_(mc["state"])

    reset()
    run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (y, st, my, mst)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        reset()
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    reset()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for _ in range(3):
        reset()
        y.fill_(float("nan"))
        my.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip((y, st, my, mst), ref):
            assert bits_equal(a, b)
