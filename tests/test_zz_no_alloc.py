"""GPU check of gdn_decode_step_noalloc, the decode step whose ticket counters
live in the library's own device array: through the C ABI, against
gdn_decode_step (same kernels, caller-owned workspace) bit for bit, on two
calls in a row, the second with a smaller input (fewer sequences and q/k
groups, one position instead of two), so the second call meets the array as
the first left it."""
import pytest
import torch

from gdn_inputs import make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def bits_equal(a, b):
    return torch.equal(a.contiguous().view(torch.int32), b.contiguous().view(torch.int32))


def run_both(inp):
    import gated_delta_ssm_amd as gdn
    wl = inp["wl"]
    n, T, H, Hk, S, C, D = wl.n_seq, wl.n_tok, wl.H, wl.Hk, wl.S, wl.conv_dim, wl.d_conv
    print(f"[case] noalloc n_seq={n} n_tok={T} H={H} Hk={Hk} S={S}", flush=True)
    d = {k: inp[k].to(DEV) for k in ("alpha", "dt", "a", "beta", "norm_w", "z", "x", "conv_w")}
    x = d["x"][:, :, :C]
    alpha3, z4 = d["alpha"].view(n, T, H), d["z"].view(n, T, H, S)
    nan = float("nan")

    def outs():
        return dict(state=inp["state"].to(DEV).clone(), hist=inp["conv_hist"].to(DEV).clone(),
                    out=torch.full((n, T, H, S), nan, device=DEV),
                    g=torch.full((n, T, H), nan, device=DEV),
                    y=torch.full((n, T, H, S), nan, device=DEV),
                    snap=torch.full((n, T - 1, H, S, S), nan, device=DEV) if T > 1 else None,
                    csnap=torch.full((n, T - 1, C, D - 1), nan, device=DEV) if T > 1 else None)

    kw = dict(scale=wl.scale, l2_eps=wl.l2_eps, norm_eps=wl.norm_eps)
    ref = outs()
    ws = torch.zeros(gdn.gdn_decode_step_workspace_bytes(n, Hk) // 4, dtype=torch.int32,
                     device=DEV)
    gdn.gdn_decode_step(ref["state"], x, d["conv_w"], ref["hist"], alpha3, d["dt"], d["a"],
                        d["beta"], d["norm_w"], z4, ref["out"], workspace=ws, g=ref["g"],
                        y=ref["y"], snap=ref["snap"], conv_snap=ref["csnap"], **kw)
    got = outs()
    gdn.gdn_decode_step_noalloc(got["state"], x, d["conv_w"], got["hist"], alpha3, d["dt"],
                                d["a"], d["beta"], d["norm_w"], z4, got["out"], g=got["g"],
                                y=got["y"], snap=got["snap"], conv_snap=got["csnap"], **kw)
    torch.cuda.synchronize()
    for key in ref:
        if ref[key] is not None:
            assert bits_equal(got[key], ref[key]), key
    assert torch.isfinite(got["out"]).all()


def test_noalloc_step_twice_second_smaller():
    # first call: 16 sequences x 2 positions, 32 value / 16 q-k heads (groups of
    # two value heads share a ticket counter); second call: 4 sequences x 1
    # position, 8 value / 4 q-k heads, on the counters the first call left
    run_both(make_inputs("verify2", seed=61))
    S, H, Hk = 128, 8, 4
    C = (2 * Hk + H) * S
    run_both(make_inputs("verify2", seed=62, n_seq=4, n_tok=1, H=H, Hk=Hk, conv_dim=C,
                         qk_channels=2 * Hk * S, x_stride=C, out_stride=C))


def test_noalloc_limit_rejected_before_launch():
    import gated_delta_ssm_amd as gdn
    inp = make_inputs("tiny", seed=63, n_tok=1)
    wl = inp["wl"]
    H, S, C = wl.H, wl.S, wl.conv_dim
    assert C == (2 * wl.Hk + H) * S
    # a state batch whose counters exceed the fixed array: refused on the host
    big = 8192 // wl.Hk + 1
    st = torch.zeros(big, H, S, S, device=DEV)
    x = torch.zeros(big, 1, C, device=DEV)
    hist = torch.zeros(big, C, wl.d_conv - 1, device=DEV)
    ab = torch.zeros(big, 1, H, device=DEV)
    z = torch.zeros(big, 1, H, S, device=DEV)
    out = torch.zeros_like(z)
    with pytest.raises(gdn.GdnError) as e:
        gdn.gdn_decode_step_noalloc(st, x, inp["conv_w"].to(DEV), hist, ab, inp["dt"].to(DEV),
                                    inp["a"].to(DEV), ab.clone(), inp["norm_w"].to(DEV), z, out,
                                    scale=wl.scale, l2_eps=wl.l2_eps, norm_eps=wl.norm_eps)
    assert e.value.status == -7
