"""The entry points inside HIP graphs (torch.cuda.graph capture on the caller's
stream): every replay must give exactly the eager result.  The library
enqueues only kernels (no memset or allocation), so its calls can be
captured; replays are separated by eager work and synchronisations."""
import pytest
import torch

import kda_workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_80_amd as K
    K.lib()


def test_decode_steps_replayed_from_a_graph():
    import gated_delta_rule_80_amd as K
    w = W.Workload(3, "decode", "decode", H=8, dk=128, dv=128, dtype="bf16", z_range=(2.0, 9.0),
                   n_sessions=16, steps=4, state_std=0.05)
    state0 = W.make_decode_state(w).cuda()
    toks = [{k_: (v_.cuda() if isinstance(v_, torch.Tensor) else v_)
             for k_, v_ in W.make_decode_step(s, w).items()} for s in range(w.steps)]

    def run_steps(state, outs):
        for s, t in enumerate(toks):
            K.decode_step(t["q"], t["k"], t["v"], t["g"], t["beta"], state, scale=w.scale,
                          out=outs[s])

    # eager reference
    st_ref = state0.clone()
    o_ref = [torch.empty((w.n_sessions, w.H, w.dv), dtype=torch.bfloat16, device="cuda")
             for _ in toks]
    run_steps(st_ref, o_ref)
    torch.cuda.synchronize()

    st = state0.clone()
    outs = [torch.empty_like(o) for o in o_ref]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):        # warm up outside the capture
        run_steps(state0.clone(), [torch.empty_like(o) for o in o_ref])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run_steps(st, outs)
    for replay in range(3):
        st.copy_(state0)                 # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(st, st_ref), "replay %d state" % replay
        for s in range(w.steps):
            assert torch.equal(outs[s], o_ref[s]), "replay %d step %d" % (replay, s)


@pytest.mark.parametrize("varlen,wide", [(False, False), (True, False), (True, True)])
def test_prefill_replayed_from_a_graph(varlen, wide):
    """wide: enough (sequence, head) pairs that the chain kernel takes its
    32-column value tiles (more 16-column chains than CUs)."""
    import gated_delta_rule_80_amd as K
    if varlen:
        lengths = [0, 130, 64, 257]
        n_cu = torch.cuda.get_device_properties(0).multi_processor_count
        H = -(-(n_cu // 8 + 1) // len(lengths)) if wide else 2
        inp = W.make_prefill(H=H, dk=128, dv=128, dtype="bf16", z_range=(2.0, 9.0), seed=71,
                             lengths=lengths, s0_std=0.05)
    else:
        inp = W.make_prefill(H=2, dk=128, dv=128, dtype="bf16", z_range=(2.0, 9.0), seed=71,
                             B=2, T=400, s0_std=0.05)
    d = {k_: (v_.cuda() if isinstance(v_, torch.Tensor) else v_) for k_, v_ in inp.items()}
    B, T, H, dk = d["q"].shape
    N = inp["n_seqs"]
    ws = torch.empty(K.workspace_bytes(B, T, H, dk, 128, 64, N), dtype=torch.uint8,
                     device="cuda")

    def call(o, fs):
        K.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], scale=d["scale"],
                    initial_state=d["initial_state"], cu_seqlens=d["cu_seqlens"], workspace=ws,
                    out=o, final_state=fs)

    o_ref = torch.empty((B, T, H, 128), dtype=torch.bfloat16, device="cuda")
    fs_ref = torch.empty((N, H, dk, 128), dtype=torch.float32, device="cuda")
    call(o_ref, fs_ref)
    torch.cuda.synchronize()

    o = torch.empty_like(o_ref)
    fs = torch.empty_like(fs_ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(torch.empty_like(o_ref), torch.empty_like(fs_ref))
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(o, fs)
    for replay in range(3):
        o.zero_()
        fs.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(fs, fs_ref), "replay %d" % replay


def test_backward_replayed_from_a_graph():
    import gated_delta_rule_80_amd as K
    gen = torch.Generator(device="cuda").manual_seed(73)
    B, T, H, d = 1, 150, 2, 32
    rnd = lambda *s: torch.randn(*s, generator=gen, device="cuda")  # noqa: E731
    q = torch.nn.functional.normalize(rnd(B, T, H, d), dim=-1).contiguous()
    k = torch.nn.functional.normalize(rnd(B, T, H, d), dim=-1).contiguous()
    v, do = rnd(B, T, H, d), rnd(B, T, H, d)
    g = (-0.5 * torch.rand(B, T, H, d, generator=gen, device="cuda")).contiguous()
    beta = torch.sigmoid(rnd(B, T, H)).contiguous()
    s0, dfin = 0.1 * rnd(1, H, d, d), rnd(1, H, d, d)
    ws = torch.empty(1 << 22, dtype=torch.uint8, device="cuda")

    def call():
        return K.chunk_bwd(q, k, v, g, beta, do, initial_state=s0, d_final_state=dfin,
                           chunk_size=32, workspace=ws)

    ref = call()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = call()
    for replay in range(3):
        for t in out.values():
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name in ref:
            assert torch.equal(out[name], ref[name]), "replay %d %s" % (replay, name)
