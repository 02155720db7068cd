"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Nothing here runs the HIP library.  Each test pins the oracle to something
other than itself: closed forms, a library routine with the same definition,
a brute-force evaluation, a second formula the pages give for the same step,
or an invariant.  Pages are cited by title and section:
  fm_kernel_ssm.h  (Foundry Metal kernels)
  ssm_mamba.rs     (spark_model layers/ops)
  scr_state.hpp    (regolith Metal engine scripts)
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.special import expit

import oracle
from gdn_inputs import WORKLOADS, make_inputs

RNG = np.random.default_rng(1234)


def rel_inf(x, r):
    x, r = np.asarray(x, np.float64), np.asarray(r, np.float64)
    return float(np.max(np.abs(x - r)) / max(np.max(np.abs(r)), 1e-300))


# --------------------------------------------------------------------------- gate
# fm_kernel_ssm.h, Decay gate section; scr_state.hpp, log_gate.

def test_gate_zero_argument_is_a_ln2():
    H = 5
    a = -np.exp(RNG.uniform(0, math.log(16), H))
    dt = RNG.uniform(0, 1, H)
    alpha = -dt[None, :].repeat(3, 0)          # alpha + dt == 0 exactly
    g = oracle.decay_gate(alpha, dt, a)
    np.testing.assert_allclose(g, np.broadcast_to(a * math.log(2.0), g.shape), rtol=1e-15)


def test_gate_above_guard_is_linear():
    # v > 20: softplus(v) is v itself, so g = a * v exactly.
    v = np.array([[20.5, 21.0, 100.0, 1e4]])
    a = np.array([-1.5, -2.0, -0.25, -16.0])
    g = oracle.decay_gate(v, np.zeros(4), a)
    assert np.array_equal(g, a * v)
    assert np.all(np.isfinite(g))


def test_gate_matches_library_softplus_threshold_20():
    v = RNG.uniform(-40, 60, size=(64, 8))
    v[0, :4] = [20.0, np.nextafter(20.0, 21.0), np.nextafter(20.0, 19.0), 0.0]  # the guard is strict
    a = -np.exp(RNG.uniform(0, math.log(16), 8))
    g = oracle.decay_gate(v, np.zeros(8), a)
    ref = a * F.softplus(torch.from_numpy(v), beta=1.0, threshold=20.0).numpy()
    np.testing.assert_allclose(g, ref, rtol=1e-14, atol=0)


def test_gate_softplus_reflection_identity():
    # softplus(v) - softplus(-v) = v for |v| <= 20 (both sides below the guard).
    v = RNG.uniform(-19.9, 19.9, size=(1, 200))
    a = -np.ones(200)
    gp = oracle.decay_gate(v, np.zeros(200), a)
    gm = oracle.decay_gate(-v, np.zeros(200), a)
    np.testing.assert_allclose(-(gp - gm), v, atol=1e-13)


def test_gate_negative_and_exp_in_unit_interval():
    v = np.concatenate([np.linspace(-700, 1e4, 4001), RNG.normal(size=1000)])[None, :]
    a = -np.exp(RNG.uniform(0, math.log(16), v.shape[1]))
    g = oracle.decay_gate(v, np.zeros(v.shape[1]), a)
    assert np.all(g < 0)
    # exp(g) in (0, 1): expm1 keeps the sign where exp(g) rounds to 1, and exp(g)
    # is representable (no fp64 underflow) wherever g > -745
    assert np.all(np.expm1(g) < 0)
    assert np.all(np.exp(g[g > -745]) > 0)


# --------------------------------------------------------------------------- conv
# fm_kernel_ssm.h, Causal depthwise conv1d + SiLU section;
# ssm_mamba.rs, conv1d_update_l2norm and gdn_verify_fused_conv_k2.

def _brute_conv(x, w, hist, qk_channels, head_dim, eps):
    """Cross-correlation of [history || x] with each channel's taps, via numpy."""
    n_seq, T, C = x.shape
    d = w.shape[1]
    out = np.empty((n_seq, T, C))
    for s in range(n_seq):
        for c in range(C):
            full = np.concatenate([hist[s, c], x[s, :, c]])
            out[s, :, c] = np.correlate(full, w[c], mode="valid")
    out = out * expit(out)
    for c0 in range(0, qk_channels, head_dim):
        blk = out[..., c0:c0 + head_dim]
        nrm = np.sqrt(np.sum(blk * blk, axis=-1, keepdims=True) + eps)
        out[..., c0:c0 + head_dim] = blk / nrm
    return out


@pytest.mark.parametrize("d", [2, 3, 4, 8])
def test_conv_brute_force(d):
    n_seq, T, C, hd = 2, 7, 8, 2
    x = RNG.normal(size=(n_seq, T, C))
    w = RNG.normal(size=(C, d)) * 0.5
    hist = RNG.normal(size=(n_seq, C, d - 1))
    out, new_hist, _ = oracle.conv1d_silu_l2norm(x, w, hist, 4, hd, 1e-6)
    ref = _brute_conv(x, w, hist, 4, hd, 1e-6)
    assert rel_inf(out, ref) < 1e-14
    full = np.concatenate([hist, np.swapaxes(x, 1, 2)], axis=2)
    np.testing.assert_array_equal(new_hist, full[:, :, -(d - 1):])


def test_conv_matches_torch_grouped_conv1d():
    T, C, d = 10, 6, 4
    x = RNG.normal(size=(1, T, C))
    w = RNG.normal(size=(C, d))
    hist = RNG.normal(size=(1, C, d - 1))
    out, _, _ = oracle.conv1d_silu_l2norm(x, w, hist, 0, 2, 1e-6)
    full = torch.from_numpy(np.concatenate([hist[0], x[0].T], axis=1))[None]
    ref = F.silu(F.conv1d(full, torch.from_numpy(w)[:, None, :], groups=C))[0].T.numpy()
    assert rel_inf(out[0], ref) < 1e-14


def test_conv_tap_order():
    T, C, d = 9, 3, 4
    x = RNG.normal(size=(1, T, C))
    hist = RNG.normal(size=(1, C, d - 1))
    silu = lambda t: t * expit(t)
    w_new = np.zeros((C, d)); w_new[:, d - 1] = 1.0     # newest tap only
    out, _, _ = oracle.conv1d_silu_l2norm(x, w_new, hist, 0, 1, 0.0)
    np.testing.assert_allclose(out[0], silu(x[0]), rtol=1e-15)
    w_old = np.zeros((C, d)); w_old[:, 0] = 1.0         # oldest tap only
    out, _, _ = oracle.conv1d_silu_l2norm(x, w_old, hist, 0, 1, 0.0)
    shifted = np.concatenate([hist[0].T, x[0]], axis=0)[:T]   # x delayed by d-1
    np.testing.assert_allclose(out[0], silu(shifted), rtol=1e-15)


def test_conv_l2_only_on_qk_channels_and_head_norm():
    T, C, d, hd, qk = 5, 12, 4, 4, 8
    x = RNG.normal(size=(1, T, C)) * 3
    w = RNG.normal(size=(C, d))
    hist = RNG.normal(size=(1, C, d - 1))
    eps = 1e-6
    out, _, _ = oracle.conv1d_silu_l2norm(x, w, hist, qk, hd, eps)
    raw, _, _ = oracle.conv1d_silu_l2norm(x, w, hist, 0, hd, eps)
    np.testing.assert_array_equal(out[..., qk:], raw[..., qk:])
    for c0 in range(0, qk, hd):
        n_raw = np.linalg.norm(raw[..., c0:c0 + hd], axis=-1)
        n_out = np.linalg.norm(out[..., c0:c0 + hd], axis=-1)
        np.testing.assert_allclose(n_out, n_raw / np.sqrt(n_raw ** 2 + eps), rtol=1e-13)


def test_conv_snapshot_is_window_after_each_position():
    T, C, d = 4, 5, 4
    x = RNG.normal(size=(2, T, C))
    w = RNG.normal(size=(C, d))
    hist = RNG.normal(size=(2, C, d - 1))
    _, last, snap = oracle.conv1d_silu_l2norm(x, w, hist, 0, 1, 0.0, want_snap=True)
    full = np.concatenate([hist, np.swapaxes(x, 1, 2)], axis=2)
    for t in range(T - 1):
        np.testing.assert_array_equal(snap[:, t], full[:, :, t + 1:t + d])
    np.testing.assert_array_equal(last, full[:, :, T:T + d - 1])


# --------------------------------------------------------------------------- recurrence
# fm_kernel_ssm.h, Delta-rule recurrence section; scr_state.hpp, GDN staleness.

def _rand_case(n_seq, T, H, Hk, dk, dv, g_scale=1.0, seed=0):
    r = np.random.default_rng(seed)
    q = r.normal(size=(n_seq, T, Hk, dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = r.normal(size=(n_seq, T, Hk, dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.normal(size=(n_seq, T, H, dv))
    g = -g_scale * r.uniform(0.01, 2.0, size=(n_seq, T, H))
    beta = expit(r.normal(size=(n_seq, T, H)))
    S0 = r.normal(size=(n_seq, H, dv, dk)) * 0.1          # GPU layout [dv][dk]
    return S0, q, k, v, g, beta


def test_recurrence_unit_key_beta_one_recalls_v():
    # beta = 1, |k| = 1, no decay: the updated state maps k to v exactly.
    dk = dv = 16
    S0, q, k, v, g, beta = _rand_case(1, 1, 3, 3, dk, dv)
    g[:] = 0.0
    beta[:] = 1.0
    _, S1, _ = oracle.recurrence_seq(S0, q, k, v, g, beta, 1.0)
    for h in range(3):
        Skv = S1[0, h].T                       # [dk][dv]
        np.testing.assert_allclose(Skv.T @ k[0, 0, h], v[0, 0, h], atol=1e-13)


def test_recurrence_beta_zero_is_pure_decay():
    dk, dv, T = 8, 12, 6
    S0, q, k, v, g, beta = _rand_case(1, T, 2, 2, dk, dv)
    beta[:] = 0.0
    y, S1, _ = oracle.recurrence_seq(S0, q, k, v, g, beta, 0.5)
    G = np.cumsum(g[0], axis=0)                # [T][H]
    for h in range(2):
        np.testing.assert_allclose(S1[0, h], np.exp(G[-1, h]) * S0[0, h], rtol=1e-13)
        for t in range(T):
            ref = 0.5 * np.exp(G[t, h]) * (S0[0, h] @ q[0, t, h])
            np.testing.assert_allclose(y[0, t, h], ref, rtol=1e-12, atol=1e-15)
    # and with g = 0 too, nothing changes at all
    g[:] = 0.0
    _, S2, _ = oracle.recurrence_seq(S0, q, k, v, g, beta, 0.5)
    np.testing.assert_array_equal(S2, S0)


def test_recurrence_single_token_from_zero():
    dk = dv = 8
    S0, q, k, v, g, beta = _rand_case(1, 1, 2, 2, dk, dv)
    S0[:] = 0.0
    y, S1, _ = oracle.recurrence_seq(S0, q, k, v, g, beta, 0.25)
    for h in range(2):
        b = beta[0, 0, h]
        np.testing.assert_allclose(S1[0, h], b * np.outer(v[0, 0, h], k[0, 0, h]), rtol=1e-14)
        ref_y = 0.25 * b * np.dot(k[0, 0, h], q[0, 0, h]) * v[0, 0, h]
        np.testing.assert_allclose(y[0, 0, h], ref_y, rtol=1e-13, atol=1e-16)


def test_recurrence_orthonormal_keys_exact_recall():
    # k_t = q_t = e_t, beta = 1, g = 0, zero state: every readout is scale * v_t.
    T, dk, dv = 10, 16, 6
    k = np.zeros((1, T, 1, dk))
    for t in range(T):
        k[0, t, 0, t] = 1.0
    v = RNG.normal(size=(1, T, 1, dv))
    g = np.zeros((1, T, 1)); beta = np.ones((1, T, 1))
    S0 = np.zeros((1, 1, dv, dk))
    y, S1, _ = oracle.recurrence_seq(S0, k, k, v, g, beta, 0.5)
    np.testing.assert_allclose(y[0, :, 0], 0.5 * v[0, :, 0], rtol=1e-15)
    yc, Sc = oracle.recurrence_chunked(S0, k, k, v, g, beta, 0.5, chunk=4)
    np.testing.assert_allclose(yc[0, :, 0], 0.5 * v[0, :, 0], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(Sc, S1, atol=1e-14)


def test_recurrence_matches_closed_form_transition():
    # scr_state.hpp gives each step as S' = gamma (I - b k k^T) S + b k v^T.
    T, H, dk, dv = 5, 2, 6, 9
    S0, q, k, v, g, beta = _rand_case(1, T, H, H, dk, dv)
    y, S1, _ = oracle.recurrence_seq(S0, q, k, v, g, beta, 0.7)
    for h in range(H):
        S = S0[0, h].T.copy()                               # [dk][dv]
        for t in range(T):
            kt = k[0, t, h]
            S = np.exp(g[0, t, h]) * (np.eye(dk) - beta[0, t, h] * np.outer(kt, kt)) @ S \
                + beta[0, t, h] * np.outer(kt, v[0, t, h])
            np.testing.assert_allclose(y[0, t, h], 0.7 * S.T @ q[0, t, h], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(S1[0, h].T, S, rtol=1e-12, atol=1e-14)


def test_recurrence_staleness_bound():
    # Two runs on the same inputs from different states: |D_T|_F <= exp(sum g) |D_0|_F.
    T, H, dk = 40, 3, 16
    S0, q, k, v, g, beta = _rand_case(1, T, H, H, dk, dk, g_scale=0.05)
    S0b = S0 + RNG.normal(size=S0.shape)
    _, Sa, _ = oracle.recurrence_seq(S0, q, k, v, g, beta, 1.0)
    _, Sb, _ = oracle.recurrence_seq(S0b, q, k, v, g, beta, 1.0)
    for h in range(H):
        lhs = np.linalg.norm(Sa[0, h] - Sb[0, h])
        rhs = np.exp(np.sum(g[0, :, h])) * np.linalg.norm(S0[0, h] - S0b[0, h])
        assert lhs <= rhs * (1 + 1e-12)
        assert lhs > 1e-6 * rhs                 # not vacuous


def test_recurrence_grouped_heads_use_contiguous_groups():
    T, H, Hk, dk = 4, 4, 2, 8
    S0, q, k, v, g, beta = _rand_case(1, T, H, Hk, dk, dk)
    y1, S1, _ = oracle.recurrence_seq(S0, q, k, v, g, beta, 1.0)
    rep = lambda a: np.repeat(a, H // Hk, axis=2)      # head h -> q/k head h // 2
    y2, S2, _ = oracle.recurrence_seq(S0, rep(q), rep(k), v, g, beta, 1.0)
    np.testing.assert_array_equal(y1, y2)
    np.testing.assert_array_equal(S1, S2)


def test_recurrence_snapshots_are_intermediate_states():
    T, H, dk = 3, 2, 8
    S0, q, k, v, g, beta = _rand_case(2, T, H, H, dk, dk)
    _, _, snap = oracle.recurrence_seq(S0, q, k, v, g, beta, 1.0, want_snap=True)
    for t in range(T - 1):
        _, St, _ = oracle.recurrence_seq(S0, q[:, :t + 1], k[:, :t + 1], v[:, :t + 1],
                                         g[:, :t + 1], beta[:, :t + 1], 1.0)
        np.testing.assert_array_equal(snap[:, t], St)


@pytest.mark.parametrize("T,dk,dv,chunk,H,Hk,g_scale", [
    (64, 32, 32, 64, 2, 2, 1.0),
    (100, 32, 32, 64, 2, 1, 1.0),
    (300, 64, 32, 64, 2, 2, 0.01),
    (130, 16, 48, 16, 4, 2, 0.1),
    (7, 8, 8, 64, 1, 1, 1.0),
])
def test_chunked_equals_sequential(T, dk, dv, chunk, H, Hk, g_scale):
    S0, q, k, v, g, beta = _rand_case(1, T, H, Hk, dk, dv, g_scale=g_scale, seed=T)
    y1, S1, _ = oracle.recurrence_seq(S0, q, k, v, g, beta, dk ** -0.5)
    y2, S2 = oracle.recurrence_chunked(S0, q, k, v, g, beta, dk ** -0.5, chunk=chunk)
    assert rel_inf(y2, y1) < 1e-12
    assert rel_inf(S2, S1) < 1e-12


def test_chunked_equals_sequential_workload_distribution():
    # the tiny workload's own draws, with the gate applied in the oracle
    inp = make_inputs("tiny")
    wl = inp["wl"]
    g = oracle.decay_gate(inp["alpha"], inp["dt"], inp["a"]).reshape(wl.n_seq, wl.n_tok, wl.H)
    S0 = np.random.default_rng(5).normal(size=(1, wl.H, wl.S, wl.S)) * 0.05
    y1, S1, _ = oracle.recurrence_seq(S0, inp["q"], inp["k"], inp["v"], g, inp["beta"], wl.scale)
    y2, S2 = oracle.recurrence_chunked(S0, inp["q"], inp["k"], inp["v"], g, inp["beta"],
                                       wl.scale, chunk=16)
    assert rel_inf(y2, y1) < 1e-12 and rel_inf(S2, S1) < 1e-12


# --------------------------------------------------------------------------- norm
# fm_kernel_ssm.h, Gated RMSNorm section.

def test_norm_constant_input_closed_form():
    rows, H, hd, eps = 3, 2, 32, 1e-6
    c = 0.37
    y = np.full((rows, H, hd), c)
    w = RNG.normal(size=hd)
    z = RNG.normal(size=(rows, H, hd))
    out = oracle.gated_rmsnorm(y, w, z, eps)
    ref = c / math.sqrt(c * c + eps) * w * (z * expit(z))
    np.testing.assert_allclose(out, ref, rtol=1e-14)


def test_norm_matches_library_rms_norm():
    rows, H, hd, eps = 4, 3, 64, 1e-6
    y = RNG.normal(size=(rows, H, hd))
    w = RNG.normal(size=hd)
    z = RNG.normal(size=(rows, H, hd))
    out = oracle.gated_rmsnorm(y, w, z, eps)
    t = lambda a: torch.from_numpy(a)
    ref = (F.rms_norm(t(y), (hd,), eps=eps) * t(w) * F.silu(t(z))).numpy()
    assert rel_inf(out, ref) < 1e-14


def test_norm_scale_invariant_without_eps():
    y = RNG.normal(size=(2, 2, 32))
    w = RNG.normal(size=32)
    z = RNG.normal(size=(2, 2, 32))
    np.testing.assert_allclose(oracle.gated_rmsnorm(7.5 * y, w, z, 0.0),
                               oracle.gated_rmsnorm(y, w, z, 0.0), rtol=1e-14)


# --------------------------------------------------------------------------- page constants

def test_workload_sizes_match_page_printed_layouts():
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")))
    wl = WORKLOADS["decode64"]
    assert wl.H * wl.S * wl.S * 4 == gold["gdn_state_bytes_per_layer"]["value"]
    assert wl.conv_dim * (wl.d_conv - 1) * 4 == gold["conv_history_bytes_per_layer"]["value"]
    d1 = WORKLOADS["decode"]
    assert 2 * d1.state_bytes == gold["decode_state_bytes_moved_mib"]["value"] * 2 ** 20


# --------------------------------------------------------------------------- Mamba-2 SSD
# ssm_mamba.rs, mamba2_ssm_prefill (its arguments: dt with bias and limits,
# A_log, D skip, groups) and the "Mamba-2 SSD chunked prefill scan" comment.

from gdn_inputs import make_mamba2_inputs  # noqa: E402


def test_mamba2_dt_matches_library_softplus_and_clamps():
    raw = np.concatenate([RNG.normal(0, 3, (50, 4)), [[25.0, 20.0, -40.0, 0.0]]])
    bias = RNG.uniform(-7, -2.3, 4)
    got = oracle.mamba2_dt(raw, bias, 1e-3, 1e-1)
    ref = F.softplus(torch.from_numpy(raw + bias[None, :]), threshold=20.0).clamp(1e-3, 1e-1)
    assert np.allclose(got, ref.numpy(), rtol=1e-14, atol=0)   # last-bit libm differences
    assert got.min() >= 1e-3 and got.max() <= 1e-1
    assert got[-1, 0] == 1e-1 and got[-1, 2] == 1e-3     # both limits reached


def ssd_case(n, T, H, G, P, N, seed, state_std=0.0):
    inp = make_mamba2_inputs(n, T, H, G, P, N, seed, state_std)
    dt = oracle.mamba2_dt(inp["dt_raw"].reshape(-1, H), inp["dt_bias"], inp["dt_min"],
                          inp["dt_max"]).reshape(n, T, H)
    return inp, dt


def test_mamba2_one_token_from_zero_closed_form():
    n, H, G, P, N = 2, 4, 2, 8, 16
    inp, dt = ssd_case(n, 1, H, G, P, N, 3)
    y, st = oracle.mamba2_ssd_seq(inp["state"], inp["x"], inp["B"], inp["C"], dt, inp["A_log"],
                                  inp["D"])
    x, B, C, D = (inp[k].double().numpy() for k in ("x", "B", "C", "D"))
    for b in range(n):
        for h in range(H):
            gi = h // (H // G)
            d = dt[b, 0, h]
            assert np.allclose(st[b, h], d * np.outer(x[b, 0, h], B[b, 0, gi]), rtol=1e-14,
                               atol=0)
            ref = d * (B[b, 0, gi] @ C[b, 0, gi]) * x[b, 0, h] + D[h] * x[b, 0, h]
            assert rel_inf(y[b, 0, h], ref) < 1e-13


def test_mamba2_pure_decay_closed_form():
    n, T, H, G, P, N = 1, 37, 3, 1, 4, 8
    inp, dt = ssd_case(n, T, H, G, P, N, 5, state_std=0.5)
    x0 = torch.zeros_like(inp["x"])
    y, st = oracle.mamba2_ssd_seq(inp["state"], x0, inp["B"], inp["C"], dt, inp["A_log"],
                                  inp["D"])
    A = -np.exp(inp["A_log"].double().numpy())
    h0 = inp["state"].double().numpy()
    C = inp["C"].double().numpy()
    cum = np.cumsum(dt[0], axis=0) * A[None, :]          # [T][H]
    for h in range(H):
        assert rel_inf(st[0, h], np.exp(cum[-1, h]) * h0[0, h]) < 1e-13
        ref = np.exp(cum[:, h])[:, None] * (C[0, :, 0] @ h0[0, h].T)
        assert rel_inf(y[0, :, h], ref) < 1e-13


def test_mamba2_d_skip_only_without_input_path():
    n, T, H, G, P, N = 1, 20, 4, 2, 8, 8
    inp, dt = ssd_case(n, T, H, G, P, N, 7)
    B = inp["B"].clone()
    B[:, :, 1] = 0.0                                     # group 1: heads 2, 3 see no input
    y, st = oracle.mamba2_ssd_seq(inp["state"], inp["x"], B, inp["C"], dt, inp["A_log"],
                                  inp["D"])
    x, D = inp["x"].double().numpy(), inp["D"].double().numpy()
    for h in (2, 3):
        assert np.array_equal(y[0, :, h], D[h] * x[0, :, h])
        assert not st[0, h].any()
    assert st[0, 0].any() and st[0, 1].any()


def test_mamba2_brute_force_quadratic_form():
    # the unrolled scan: y_t = sum_{s<=t} (C_t . B_s) exp(A sum_{s<r<=t} dt_r) dt_s x_s
    #                        + exp(A sum_{r<=t} dt_r) h0 C_t + D x_t
    n, T, H, G, P, N = 1, 11, 2, 1, 3, 5
    inp, dt = ssd_case(n, T, H, G, P, N, 9, state_std=0.3)
    y, st = oracle.mamba2_ssd_seq(inp["state"], inp["x"], inp["B"], inp["C"], dt, inp["A_log"],
                                  inp["D"])
    A = -np.exp(inp["A_log"].double().numpy())
    x, B, C, D = (inp[k].double().numpy() for k in ("x", "B", "C", "D"))
    h0 = inp["state"].double().numpy()
    for h in range(H):
        for t in range(T):
            ref = D[h] * x[0, t, h] + math.exp(A[h] * dt[0, :t + 1, h].sum()) * (h0[0, h] @ C[0, t, 0])
            for s_ in range(t + 1):
                decay = math.exp(A[h] * dt[0, s_ + 1:t + 1, h].sum())
                ref = ref + (C[0, t, 0] @ B[0, s_, 0]) * decay * dt[0, s_, h] * x[0, s_, h]
            assert rel_inf(y[0, t, h], ref) < 1e-12


@pytest.mark.parametrize("T,H,G,P,N,chunk,state_std", [(100, 4, 2, 8, 16, 16, 0.0),
                                                        (64, 2, 1, 16, 8, 64, 0.3),
                                                        (130, 3, 3, 4, 32, 64, 0.1),
                                                        (5, 2, 1, 4, 4, 64, 0.2)])
def test_mamba2_chunked_equals_sequential(T, H, G, P, N, chunk, state_std):
    inp, dt = ssd_case(2, T, H, G, P, N, 11, state_std)
    args = (inp["state"], inp["x"], inp["B"], inp["C"], dt, inp["A_log"], inp["D"])
    y_s, st_s = oracle.mamba2_ssd_seq(*args)
    y_c, st_c = oracle.mamba2_ssd_chunked(*args, chunk=chunk)
    assert rel_inf(y_c, y_s) < 1e-12 and rel_inf(st_c, st_s) < 1e-12
