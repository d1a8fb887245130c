"""Inputs given in a layer's form (q, k to be L2-normalised, logit gates, logit
beta) and the output stage (RMS norm x weight x sigmoid gate), through the C
ABI, against the fp64 oracle: oracle/layer.py maps the same stored inputs to
the plain form, then the recurrence oracle runs.

Tolerances: relative Frobenius error <= 1e-4 (fp32 storage), <= 5e-3 (bf16).
"""
import numpy as np
import pytest
import torch

import kda_workloads as W
import oracle
from oracle import layer as L
from kda_harness import TOL, assert_close, cu_list, rel_err

pytestmark = pytest.mark.gpu

STORE = {"bf16": torch.bfloat16, "f32": torch.float32}


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_80_amd as K
    K.lib()


def raw_inputs(gate, H=2, T=300, B=1, d=128, dtype="bf16", lengths=None, seed=41):
    """Seeded inputs in the layer's form: q, k with per-row scales (not unit),
    decay logits z ~ U(2, 9) (per channel or per token-head), beta logits ~ N(0, 1)."""
    inp = W.make_prefill(H=H, dk=d, dv=d, dtype=dtype, z_range=(2.0, 9.0), seed=seed, B=B, T=T,
                         lengths=lengths, s0_std=0.05)
    rng = np.random.default_rng([seed, 77])
    rows = inp["q"].shape[:3]
    for name in ("q", "k"):
        f = torch.from_numpy(rng.uniform(0.3, 3.0, size=rows + (1,)).astype(np.float32))
        inp[name] = (inp[name].float() * f).to(STORE[dtype])
    gshape = rows + (d,) if gate == "per_channel" else rows
    inp["g"] = (None if gate == "none"
                else torch.from_numpy(rng.uniform(2.0, 9.0, size=gshape).astype(np.float32)))
    inp["beta"] = torch.from_numpy(rng.standard_normal(size=rows).astype(np.float32))
    return inp


def oracle_form(inp, gate, **form):
    d = inp["q"].shape[-1]
    flat = lambda t: None if t is None else W.to64(t).reshape(-1, *t.shape[2:])  # noqa: E731
    q, k, g, b = L.inputs_in_plain_form(flat(inp["q"]), flat(inp["k"]), flat(inp["g"]),
                                        flat(inp["beta"]), d_k=d, gate=gate, **form)
    return oracle.prefill(q, k, flat(inp["v"]), g, b, inp["scale"], W.to64(inp["initial_state"]),
                          cu_list(inp))


def gpu_form(inp, gate, chunk, **form):
    import gated_delta_rule_80_amd as K
    dev = lambda t: None if t is None else t.cuda()  # noqa: E731
    o, fs = K.chunk_fwd_ex(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), dev(inp["g"]),
                           dev(inp["beta"]), gate=gate, scale=inp["scale"],
                           initial_state=dev(inp["initial_state"]),
                           cu_seqlens=dev(inp["cu_seqlens"]), chunk_size=chunk, **form)
    torch.cuda.synchronize()
    o64 = o.double().cpu().numpy()
    return o64.reshape(-1, *o64.shape[2:]), fs.double().cpu().numpy()


ALL = dict(gate_is_logit=True, beta_is_logit=True, l2norm_qk=True, eps=1e-6)


def check(inp, gate, chunk, form):
    o, fs = gpu_form(inp, gate, chunk, **form)
    o_ref, s_ref = oracle_form(inp, gate, **form)
    assert_close(o, o_ref, fs, s_ref, cu_list(inp), TOL[inp["dtype"]],
                 label="form %s %s" % (gate, form))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("gate", ["per_channel", "scalar", "none"])
def test_prefill_with_every_input_step(gate, dtype):
    inp = raw_inputs(gate, T=300, B=2, dtype=dtype)
    form = dict(ALL)
    if gate == "none":
        form.pop("gate_is_logit")
    check(inp, gate, 64, form)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("gate", ["per_channel", "scalar"])
def test_logit_gate_down_to_minus_50(gate, dtype):
    """Decay logits anywhere in [-50, 9]: log sigmoid(x) is about x below -10,
    where the bf16 MFMA path floors the log-decay at -10 and the fp32 path
    keeps the exact factors; outputs stay finite and within the tolerance of
    the exact recurrence on the same logits."""
    inp = raw_inputs(gate, T=260, B=1, seed=43, dtype=dtype)
    rng = np.random.default_rng([43, 78])
    inp["g"] = torch.from_numpy(rng.uniform(-50.0, 9.0, size=inp["g"].shape).astype(np.float32))
    check(inp, gate, 64, dict(ALL))


@pytest.mark.parametrize("form", [dict(l2norm_qk=True, eps=1e-6), dict(gate_is_logit=True),
                                  dict(beta_is_logit=True)])
def test_prefill_one_step_at_a_time(form):
    inp = raw_inputs("per_channel", T=200)
    base = W.make_prefill(H=2, dk=128, dv=128, dtype="bf16", z_range=(2.0, 9.0), seed=41, B=1,
                          T=200, s0_std=0.05)
    if "l2norm_qk" not in form:      # without the in-kernel norm, q and k must already be unit
        inp["q"], inp["k"] = base["q"], base["k"]
    if "gate_is_logit" not in form:  # without it, g must already be a log-decay
        inp["g"] = base["g"]
    if "beta_is_logit" not in form:  # without it, beta must already be a write strength
        inp["beta"] = base["beta"]
    check(inp, "per_channel", 64, form)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_forms_packed_sequences(dtype):
    inp = raw_inputs("scalar", H=3, lengths=[0, 65, 1, 300, 129], dtype=dtype)
    check(inp, "scalar", 64, ALL)


@pytest.mark.parametrize("d,C", [(16, 16), (32, 32), (64, 64), (128, 64)])
def test_prefill_forms_fp32_path(d, C):
    inp = raw_inputs("per_channel", d=d, dtype="f32", T=3 * C + 7)
    check(inp, "per_channel", C, ALL)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_plain_form_is_the_plain_entry_point_bitwise(dtype):
    import gated_delta_rule_80_amd as K
    inp = W.make_prefill(H=2, dk=128, dv=128, dtype=dtype, z_range=(2.0, 9.0), seed=43, B=2,
                         T=500, s0_std=0.05)
    d = {k_: (v_.cuda() if isinstance(v_, torch.Tensor) else v_) for k_, v_ in inp.items()}
    o1, s1 = K.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"],
                         initial_state=d["initial_state"])
    o2, s2 = K.chunk_fwd_ex(d["q"], d["k"], d["v"], d["g"], d["beta"],
                            initial_state=d["initial_state"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


@pytest.mark.parametrize("gate", ["per_channel", "scalar", "none"])
@pytest.mark.parametrize("d,dtype", [(128, "bf16"), (16, "f32")])
def test_decode_with_every_input_step(gate, d, dtype):
    import gated_delta_rule_80_amd as K
    N, H, steps = 5, 3, 3
    rng = np.random.default_rng([51, d])
    st = torch.from_numpy((rng.standard_normal((N, H, d, d)) * 0.05).astype(np.float32))
    ref = W.to64(st)
    st_dev = st.cuda()
    form = dict(ALL)
    if gate == "none":
        form.pop("gate_is_logit")
    errs = []
    for s in range(steps):
        q = torch.from_numpy(rng.standard_normal((N, H, d)).astype(np.float32)).to(STORE[dtype])
        k = torch.from_numpy(rng.standard_normal((N, H, d)).astype(np.float32)).to(STORE[dtype])
        v = torch.from_numpy(rng.standard_normal((N, H, d)).astype(np.float32)).to(STORE[dtype])
        gshape = (N, H, d) if gate == "per_channel" else (N, H)
        g = (None if gate == "none"
             else torch.from_numpy(rng.uniform(2.0, 9.0, gshape).astype(np.float32)))
        b = torch.from_numpy(rng.standard_normal((N, H)).astype(np.float32))
        o = K.decode_step_ex(q.cuda(), k.cuda(), v.cuda(), None if g is None else g.cuda(),
                             b.cuda(), st_dev, gate=gate, scale=d ** -0.5, **form)
        q64, k64, g64, b64 = L.inputs_in_plain_form(W.to64(q), W.to64(k), W.to64(g), W.to64(b),
                                                    d_k=d, gate=gate, **form)
        o_ref, ref = oracle.decode_step(q64, k64, W.to64(v), g64, b64, d ** -0.5, ref)
        errs.append((o.double().cpu().numpy(), o_ref))
    torch.cuda.synchronize()
    eo = rel_err(np.stack([e[0] for e in errs]), np.stack([e[1] for e in errs]))
    es = rel_err(st_dev.double().cpu().numpy(), ref)
    print("decode form err o %.3e S %.3e" % (eo, es))
    assert eo <= TOL[dtype] and es <= TOL[dtype]


@pytest.mark.parametrize("dv", [16, 128, 256])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_output_rmsnorm_gate(dv, dtype):
    import gated_delta_rule_80_amd as K
    rng = np.random.default_rng([61, dv])
    rows = 1000 + 37                    # not a multiple of the rows per workgroup
    o = torch.from_numpy(rng.standard_normal((rows, dv)).astype(np.float32)).to(STORE[dtype])
    z = torch.from_numpy(rng.standard_normal((rows, dv)).astype(np.float32)).to(STORE[dtype])
    w = torch.from_numpy(rng.uniform(0.5, 1.5, dv).astype(np.float32))
    out = K.output_rmsnorm_gate(o.cuda(), z.cuda(), w.cuda(), eps=1e-6)
    inplace = o.cuda()
    K.output_rmsnorm_gate(inplace, z.cuda(), w.cuda(), eps=1e-6, out=inplace)
    torch.cuda.synchronize()
    ref = L.output_rmsnorm_gate(W.to64(o), W.to64(z), W.to64(w), 1e-6)
    err = rel_err(out.double().cpu().numpy(), ref)
    print("output stage err %.3e" % err)
    assert err <= TOL[dtype]
    assert torch.equal(out, inplace)
