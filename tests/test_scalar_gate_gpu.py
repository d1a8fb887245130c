"""Scalar-gate entry points (one log-decay per token and head, shared by the key
channels; none at all for the plain delta rule) against the fp64 oracle, which
receives the same gate repeated over the d_k channels (or zeros).  The oracle's
own scalar-gate reduction is pinned on the CPU against an independent
scalar-decay loop.

Tolerances: relative Frobenius error <= 1e-4 (fp32 storage), <= 5e-3 (bf16).
"""
import numpy as np
import pytest
import torch

import kda_workloads as W
import oracle
from kda_harness import TOL, assert_close, cu_list, oracle_prefill, rel_err, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_80_amd as K
    K.lib()


def inputs(H=2, T=300, B=1, d=128, dtype="bf16", lengths=None, seed=31, z=(2.0, 9.0)):
    inp = W.make_prefill(H=H, dk=d, dv=d, dtype=dtype, z_range=z, seed=seed, B=B, T=T,
                         lengths=lengths, s0_std=0.05)
    gs = inp["g"][..., 0].contiguous()                       # [B, T, H]: one gate per token-head
    return inp, gs


def with_gate(inp, g_full):
    out = dict(inp)
    out["g"] = g_full
    return out


def run_scalar(inp, gs, chunk):
    import gated_delta_rule_80_amd as K
    d = to_dev(inp)
    o, fs = K.chunk_fwd_scalar_gate(d["q"], d["k"], d["v"], None if gs is None else gs.cuda(),
                                    d["beta"], scale=d["scale"],
                                    initial_state=d["initial_state"],
                                    cu_seqlens=d["cu_seqlens"], chunk_size=chunk)
    torch.cuda.synchronize()
    o64 = o.double().cpu().numpy()
    return o64.reshape(-1, *o64.shape[2:]), fs.double().cpu().numpy()


def check(inp, gs, chunk):
    g_full = (torch.zeros_like(inp["g"]) if gs is None
              else gs[..., None].expand_as(inp["g"]).contiguous())
    o, fs = run_scalar(inp, gs, chunk)
    o_ref, s_ref = oracle_prefill(with_gate(inp, g_full))
    assert_close(o, o_ref, fs, s_ref, cu_list(inp), TOL[inp["dtype"]], label="scalar gate")


@pytest.mark.parametrize("T,B", [(300, 2), (64, 1), (1000, 1)])
def test_scalar_gate_prefill(T, B):
    inp, gs = inputs(T=T, B=B)
    check(inp, gs, 64)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_no_gate_prefill_is_deltanet(dtype):
    inp, _ = inputs(T=500, dtype=dtype)
    check(inp, None, 64)


def test_scalar_gate_packed_sequences():
    inp, gs = inputs(H=3, lengths=[0, 65, 1, 300, 129])
    check(inp, gs, 64)


@pytest.mark.parametrize("d,C", [(16, 16), (32, 32), (64, 64), (128, 64)])
def test_scalar_gate_fp32_path(d, C):
    inp, gs = inputs(d=d, dtype="f32", T=3 * C + 5)
    check(inp, gs, C)


def test_scalar_gate_kernel_matches_the_per_channel_kernel_on_a_repeated_gate():
    """bf16 storage: the scalar gate has an intra-chunk kernel of its own (the
    C x C decay mask on K K^T and Q K^T); fed the same gate on every channel,
    the per-channel kernel computes the same operator by another route.  Both
    meet the oracle's tolerance, and they agree with each other to within it."""
    import gated_delta_rule_80_amd as K
    inp, gs = inputs(T=700, B=2)
    d = to_dev(inp)
    g_full = gs[..., None].expand_as(inp["g"]).contiguous()
    o1, s1 = K.chunk_fwd_scalar_gate(d["q"], d["k"], d["v"], gs.cuda(), d["beta"],
                                     initial_state=d["initial_state"])
    o2, s2 = K.chunk_fwd(d["q"], d["k"], d["v"], g_full.cuda(), d["beta"],
                         initial_state=d["initial_state"])
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_prefill(with_gate(inp, g_full))
    for o, st in ((o1, s1), (o2, s2)):
        o64 = o.double().cpu().numpy()
        assert_close(o64.reshape(-1, *o64.shape[2:]), o_ref, st.double().cpu().numpy(), s_ref,
                     cu_list(inp), TOL["bf16"], label="scalar vs per-channel kernel")
    assert rel_err(o1.double().cpu(), o2.double().cpu()) <= TOL["bf16"]
    assert rel_err(s1.double().cpu(), s2.double().cpu()) <= TOL["bf16"]


@pytest.mark.parametrize("d", [32, 128])
def test_scalar_gate_fp32_equals_repeated_per_channel_gate_bitwise(d):
    """fp32 storage: one path serves both gate layouts (at d = 128 the MFMA
    chunk factors, below it one VALU kernel), so a scalar gate gives exactly
    the bits of the per-channel entry point fed it on every channel."""
    import gated_delta_rule_80_amd as K
    inp, gs = inputs(d=d, dtype="f32", T=150, B=2)
    d = to_dev(inp)
    g_full = gs[..., None].expand_as(inp["g"]).contiguous().cuda()
    o1, s1 = K.chunk_fwd_scalar_gate(d["q"], d["k"], d["v"], gs.cuda(), d["beta"],
                                     initial_state=d["initial_state"], chunk_size=32)
    o2, s2 = K.chunk_fwd(d["q"], d["k"], d["v"], g_full, d["beta"],
                         initial_state=d["initial_state"], chunk_size=32)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


@pytest.mark.parametrize("lo,hi", [(-0.4, 0.0), (-5.0, 0.0), (-30.0, -5.0)])
def test_scalar_gate_strong_decays_and_minus_inf(lo, hi):
    """Scalar log-decays from weak to far below the floor of -10, with -inf on
    some tokens, over packed sequences with ragged tails: the mask factors
    e^{G_i - G_j} are at most 1 whatever the decay."""
    inp, _ = inputs(H=2, lengths=[70, 1, 200, 64, 17, 130])
    gen = torch.Generator().manual_seed(73)
    gs = (lo + (hi - lo) * torch.rand(inp["beta"].shape, generator=gen,
                                      dtype=torch.float64)).to(torch.float32)
    gs[:, [5, 71, 150, 300], :] = float("-inf")
    check(inp, gs.contiguous(), 64)


@pytest.mark.parametrize("gated", [True, False])
@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (32, "f32")])
def test_scalar_gate_decode(gated, d, dtype):
    import gated_delta_rule_80_amd as K
    w = W.Workload(3, "decode", "decode", H=4, dk=d, dv=d, dtype=dtype, z_range=(2.0, 9.0),
                   n_sessions=6, steps=3, state_std=0.05)
    st = W.make_decode_state(w)
    st_dev = st.cuda()
    ref = W.to64(st)
    o_gpu, o_ref = [], []
    for s in range(w.steps):
        tok = W.make_decode_step(s, w)
        gs = tok["g"][..., 0].contiguous()                   # [N, H]
        dd = to_dev(tok)
        o = K.decode_step_scalar_gate(dd["q"], dd["k"], dd["v"], gs.cuda() if gated else None,
                                      dd["beta"], st_dev, scale=w.scale)
        o_gpu.append(o.double().cpu().numpy())
        g_full = (np.repeat(W.to64(gs)[..., None], d, axis=-1) if gated
                  else np.zeros(tuple(tok["g"].shape)))
        orr, ref = oracle.decode_step(W.to64(tok["q"]), W.to64(tok["k"]), W.to64(tok["v"]),
                                      g_full, W.to64(tok["beta"]), w.scale, ref)
        o_ref.append(orr)
    torch.cuda.synchronize()
    eo = rel_err(np.stack(o_gpu), np.stack(o_ref))
    es = rel_err(st_dev.double().cpu().numpy(), ref)
    print("scalar gate decode err o %.3e S %.3e" % (eo, es))
    assert eo <= TOL[dtype] and es <= TOL[dtype]
