"""The GPU backward (kda_chunk_bwd, fp32 storage) against the fp64
autograd oracle of the recurrence (oracle/backward.py, pinned to finite
differences), through the C ABI.  Tolerance: relative Frobenius error <= 1e-4
on every gradient, as for the fp32 forward."""
import numpy as np
import pytest
import torch

import oracle
from kda_harness import rel_err

pytestmark = pytest.mark.gpu
TOL = 1e-4


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_80_amd as K
    K.lib()


def make(B, T, H, d, seed, lengths=None, g_range=(-1.0, 0.0), s0=True, dfin=True):
    rng = np.random.default_rng(seed)
    rows = 1 if lengths else B
    tot = sum(lengths) if lengths else T
    n = len(lengths) if lengths else B
    shp = (rows, tot, H, d)
    q = rng.normal(size=shp)
    k = rng.normal(size=shp)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    x = dict(q=q, k=k, v=rng.normal(size=shp), g=rng.uniform(*g_range, size=shp),
             beta=rng.uniform(0.05, 0.95, size=shp[:3]), do=rng.normal(size=shp))
    x = {n_: a.astype(np.float32) for n_, a in x.items()}
    x["s0"] = (0.1 * rng.normal(size=(n, H, d, d))).astype(np.float32) if s0 else None
    x["dfin"] = rng.normal(size=(n, H, d, d)).astype(np.float32) if dfin else None
    x["cu"] = (np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32) if lengths else None)
    return x


def to_bf16(x):
    """q, k, v and do rounded to bf16 (RNE); the oracle gets the rounded values."""
    x = dict(x)
    for n in ("q", "k", "v", "do"):
        x[n] = torch.from_numpy(x[n]).to(torch.bfloat16).float().numpy()
    x["_bf16"] = True
    return x


def check(x, chunk):
    import gated_delta_rule_80_amd as K
    bf16 = x.pop("_bf16", False)
    dev = {n: (torch.from_numpy(a).cuda() if a is not None else None) for n, a in x.items()}
    if bf16:
        for n in ("q", "k", "v", "do"):
            dev[n] = dev[n].to(torch.bfloat16)   # exact: the values are bf16 already
    got = K.chunk_bwd(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], dev["do"],
                      initial_state=dev["s0"], cu_seqlens=dev["cu"], d_final_state=dev["dfin"],
                      chunk_size=chunk)
    torch.cuda.synchronize()
    flat = lambda a: None if a is None else a.reshape(-1, *a.shape[2:]).astype(np.float64)  # noqa
    rows, T, _, d = x["q"].shape
    # B equal rows are B sequences for the oracle
    cu = x["cu"].tolist() if x["cu"] is not None else list(range(0, rows * T + 1, T))
    ref = oracle.backward.recurrent_grads(flat(x["q"]), flat(x["k"]), flat(x["v"]), flat(x["g"]),
                                          x["beta"].reshape(-1, x["beta"].shape[-1]),
                                          1.0 / np.sqrt(d), flat(x["do"]), x["s0"], x["dfin"], cu)
    errs = {}
    for name in ("dq", "dk", "dv", "dg", "dbeta"):
        assert got[name].dtype == torch.float32
        a = got[name].double().cpu().numpy()
        errs[name] = rel_err(a.reshape(-1, *a.shape[2:]), ref[name])
    if x["s0"] is not None:
        errs["dinitial_state"] = rel_err(got["dinitial_state"].double().cpu().numpy(),
                                         ref["dinitial_state"])
    print("backward errors: " + "  ".join("%s %.2e" % kv for kv in errs.items()), flush=True)
    for name, e in errs.items():
        assert np.isfinite(e) and e <= TOL, (name, e)


@pytest.mark.parametrize("d,C,T", [(16, 16, 70), (16, 64, 150), (32, 16, 47), (32, 32, 100),
                                   (64, 16, 40), (64, 32, 65), (128, 16, 40)])
def test_backward_shapes(d, C, T):
    check(make(2, T, 2, d, seed=100 + d + C), C)


def test_backward_packed_sequences_with_an_empty_one():
    check(make(1, 0, 2, 32, seed=201, lengths=[17, 0, 43, 40]), 32)


def test_backward_strong_decays():
    check(make(1, 90, 2, 16, seed=202, g_range=(-5.0, 0.0)), 16)


def test_backward_without_states():
    check(make(1, 80, 3, 16, seed=203, s0=False, dfin=False), 32)


def test_backward_d128_packed_sequences():
    check(make(1, 0, 2, 128, seed=204, lengths=[33, 0, 17, 30]), 16)


def test_backward_d128_strong_decays_without_initial_state():
    check(make(1, 37, 1, 128, seed=205, g_range=(-5.0, 0.0), s0=False), 16)


def test_backward_d128_pairs_not_filling_groups_of_eight():
    """9 (sequence, head) pairs: the chain kernel's last group of 8 pairs is
    partly empty; 70 tokens are 5 chunks with a ragged tail."""
    check(make(3, 70, 3, 128, seed=206), 16)


def test_backward_d128_odd_and_even_chunk_counts_without_final_gradient():
    check(make(1, 0, 3, 128, seed=207, lengths=[49, 16, 0, 33], dfin=False), 16)


def test_backward_d128_rebuilt_states_along_long_sequences():
    """At d = 128, chunk 16, the chain stores S at even chunks and dS' at odd
    ones and the last; the gradient kernel rebuilds the rest.  Sequences of
    11 (ragged), 2, 1, 6 and 2 (ragged) chunks put the last chunk at both
    parities, full and ragged, and chain rebuilds over many chunks."""
    check(make(1, 0, 2, 128, seed=208, lengths=[161, 32, 15, 96, 17]), 16)
    check(to_bf16(make(1, 0, 2, 128, seed=209, lengths=[17, 15, 160])), 16)


@pytest.mark.parametrize("chunk", [32, 64])
def test_backward_d128_requested_chunks_run_as_16_token_chunks(chunk):
    """At d = 128 a requested chunk of 32 or 64 tokens (the forward's) gives
    the gradients of the 16-token computation, bit for bit, and so within the
    tolerance of the oracle."""
    import gated_delta_rule_80_amd as K
    x = make(1, 0, 2, 128, seed=213, lengths=[150, 0, 47])
    check(dict(x), chunk)
    dev = {n: (torch.from_numpy(a).cuda() if a is not None else None) for n, a in x.items()}
    run = lambda c: K.chunk_bwd(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], dev["do"],  # noqa: E731
                                initial_state=dev["s0"], cu_seqlens=dev["cu"],
                                d_final_state=dev["dfin"], chunk_size=c)
    a, b = run(16), run(chunk)
    torch.cuda.synchronize()
    for name in a:
        assert torch.equal(a[name], b[name]), name


def test_backward_d128_pairwise_and_factored_decay_paths():
    """At d = 128, chunk 16, a wave whose 16 channels all decay by at most 40
    over a chunk forms the decay-weighted sums as matrix products between
    row scalings; any other wave takes the pairwise factors.  Channels 0-47
    decay by 3-4 per token (spans of 45-60 over a full chunk), 48-127 weakly,
    so waves 0-2 take the pairwise factors and waves 3-7 the products,
    except in the short last chunk.  The prep kernel makes that choice for
    all 128 channels of a chunk at once (K~ and H), so here it takes the
    pairwise factors except in the last chunk."""
    x = make(1, 70, 2, 128, seed=210)
    rng = np.random.default_rng(211)
    x["g"][..., :48] = rng.uniform(-4.0, -3.0, size=x["g"][..., :48].shape).astype(np.float32)
    check(x, 16)


@pytest.mark.parametrize("d,C,T", [(128, 16, 45), (64, 32, 70), (16, 64, 130)])
def test_backward_bf16_storage(d, C, T):
    check(to_bf16(make(2, T, 2, d, seed=300 + d)), C)


def test_backward_bf16_packed_sequences():
    check(to_bf16(make(1, 0, 2, 128, seed=305, lengths=[20, 0, 37])), 16)


@pytest.mark.parametrize("storage", ["bf16", "f32"])
def test_backward_bench_workload_sampled_heads(storage):
    """The backward at the benchmark's size and launch shape: B = 1, H = 32,
    T = 8192, d = 128, chunk 16, bf16 (as benchmarked) or fp32 q, k, v and dO,
    log-decays U(-0.05, 0).
    The chain kernel walks 512 chunks each way in the same 256 workgroups (its
    prefetch wave included), and the gradient kernel rebuilds every other
    state.  Heads are independent, so three of the 32 are compared in full
    with the oracle's chunkwise backward (pinned to autograd of the
    recurrence to 1e-10 in the CPU tests)."""
    import gated_delta_rule_80_amd as K
    T, H, d, C = 8192, 32, 128, 16
    rng = np.random.default_rng(212)
    shp = (1, T, H, d)
    dt = torch.bfloat16 if storage == "bf16" else torch.float32
    bf = lambda a: torch.from_numpy(a).to(dt)  # noqa: E731
    q = rng.standard_normal(size=shp, dtype=np.float32)
    k = rng.standard_normal(size=shp, dtype=np.float32)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    x = dict(q=bf(q), k=bf(k), v=bf(rng.standard_normal(size=shp, dtype=np.float32)),
             do=bf(rng.standard_normal(size=shp, dtype=np.float32)))
    del q, k
    g = (-0.05 * rng.random(size=shp, dtype=np.float32))
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal(size=shp[:3])))).astype(np.float32)
    s0 = (0.1 * rng.standard_normal(size=(1, H, d, d))).astype(np.float32)
    dfin = rng.standard_normal(size=(1, H, d, d)).astype(np.float32)
    got = K.chunk_bwd(x["q"].cuda(), x["k"].cuda(), x["v"].cuda(), torch.from_numpy(g).cuda(),
                      torch.from_numpy(beta).cuda(), x["do"].cuda(),
                      initial_state=torch.from_numpy(s0).cuda(),
                      d_final_state=torch.from_numpy(dfin).cuda(), chunk_size=C)
    torch.cuda.synchronize()
    got = {n: t.cpu().numpy() for n, t in got.items()}
    for hh in (0, 13, 31):
        one = lambda a: a[0, :, hh:hh + 1].astype(np.float64)  # noqa: E731
        ref = oracle.backward.chunkwise_grads(
            one(x["q"].float().numpy()), one(x["k"].float().numpy()),
            one(x["v"].float().numpy()), one(g), beta[0, :, hh:hh + 1].astype(np.float64),
            1.0 / np.sqrt(d), C, one(x["do"].float().numpy()), s0[:, hh:hh + 1],
            dfin[:, hh:hh + 1], [0, T])
        errs = {n: rel_err(got[n][0, :, hh:hh + 1], ref[n]) for n in ("dq", "dk", "dv", "dg")}
        errs["dbeta"] = rel_err(got["dbeta"][0, :, hh:hh + 1], ref["dbeta"])
        errs["dinitial_state"] = rel_err(got["dinitial_state"][:, hh:hh + 1],
                                         ref["dinitial_state"])
        print("head %d backward errors: " % hh + "  ".join("%s %.2e" % kv for kv in errs.items()),
              flush=True)
        for name, e in errs.items():
            assert np.isfinite(e) and e <= TOL, (hh, name, e)
