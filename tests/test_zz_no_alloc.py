"""kda_chunk_fwd_noalloc through the C ABI: the prefill on the library's own
device buffer gives the bits of kda_chunk_fwd with a caller workspace, on two
calls in a row (the second smaller, so the buffer holds stale records of the
first), for packed and equal-length sequences; problems too large for the
buffer are refused before anything is enqueued; the fp32 path (no workspace)
also goes through it.  Both entry points run the same kernels."""
import ctypes

import numpy as np
import pytest
import torch

import kda_workloads as W
from kda_harness import TOL, cu_list, oracle_prefill, rel_err, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_80_amd as K
    K.lib()


def _shape(inp):
    import gated_delta_rule_80_amd as K
    B, T, H, dk = inp["q"].shape
    dv = inp["v"].shape[-1]
    code = K.KDA_BF16 if inp["q"].dtype == torch.bfloat16 else K.KDA_F32
    return K.make_shape(B, T, H, dk, dv, 64 if dk == 128 else 16, inp["n_seqs"], code), (B, T, H,
                                                                                        dk, dv)


def _outputs(inp, dims):
    B, T, H, dk, dv = dims
    o = torch.full((B, T, H, dv), float("nan"), dtype=inp["q"].dtype, device="cuda")
    fs = torch.full((inp["n_seqs"], H, dk, dv), float("nan"), dtype=torch.float32, device="cuda")
    return o, fs


def _args(d):
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    return [p(d["q"]), p(d["k"]), p(d["v"]), p(d["g"]), p(d["beta"]), ctypes.c_float(d["scale"]),
            p(d["initial_state"]), p(d["cu_seqlens"])]


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def run_both(inp):
    """(o, final) from kda_chunk_fwd with a torch workspace, then from
    kda_chunk_fwd_noalloc, both through ctypes on the current stream."""
    import gated_delta_rule_80_amd as K
    L = K.lib()
    sh, dims = _shape(inp)
    d = to_dev(inp)
    need = L.kda_chunk_fwd_workspace_bytes(ctypes.byref(sh))
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    o1, f1 = _outputs(inp, dims)
    st = L.kda_chunk_fwd(ctypes.byref(sh), *_args(d), ctypes.c_void_p(o1.data_ptr()),
                         ctypes.c_void_p(f1.data_ptr()), ctypes.c_void_p(ws.data_ptr()),
                         ctypes.c_size_t(ws.numel()), _stream())
    assert st == 0, L.kda_last_error()
    o2, f2 = _outputs(inp, dims)
    st = L.kda_chunk_fwd_noalloc(ctypes.byref(sh), *_args(d), ctypes.c_void_p(o2.data_ptr()),
                                 ctypes.c_void_p(f2.data_ptr()), _stream())
    assert st == 0, L.kda_last_error()
    torch.cuda.synchronize()
    return (o1, f1), (o2, f2)


def _check(inp):
    (o1, f1), (o2, f2) = run_both(inp)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)
    # and both within the tolerance of the fp64 oracle
    o_ref, s_ref = oracle_prefill(inp)
    o64 = o2.double().cpu().numpy()
    eo = rel_err(o64.reshape(-1, *o64.shape[2:]), o_ref)
    es = rel_err(f2.double().cpu().numpy(), s_ref)
    print("noalloc err o %.3e S %.3e" % (eo, es), flush=True)
    assert eo <= TOL[inp["dtype"]] and es <= TOL[inp["dtype"]]


def test_noalloc_matches_the_workspace_entry_point_then_a_smaller_call():
    big = W.make_prefill(H=6, dk=128, dv=128, dtype="bf16", z_range=(2.0, 9.0), seed=91,
                         lengths=[700, 0, 1300, 65, 1], s0_std=0.05)
    small = W.make_prefill(H=2, dk=128, dv=128, dtype="bf16", z_range=(2.0, 9.0), seed=92,
                           B=2, T=150, s0_std=None)
    assert sum(cu_list(small)) < sum(cu_list(big))
    _check(big)
    _check(small)


def test_noalloc_fp32_path_and_refusal_of_oversize_problems():
    import gated_delta_rule_80_amd as K
    L = K.lib()
    _check(W.make_prefill(H=2, dk=16, dv=16, dtype="f32", z_range=(2.0, 9.0), seed=93, B=1, T=77,
                          s0_std=0.05))
    # fp32 at d = 128: the chunk factors fit the buffer, so the same MFMA path
    _check(W.make_prefill(H=2, dk=128, dv=128, dtype="f32", z_range=(2.0, 9.0), seed=94,
                          lengths=[150, 0, 33], s0_std=0.05))
    # 32 heads x 131072 tokens need about 4.7 GB of records: refused, nothing run
    sh = K.make_shape(1, 131072, 32, 128, 128, 64, 1, K.KDA_BF16)
    assert L.kda_chunk_fwd_workspace_bytes(ctypes.byref(sh)) > (256 << 20)
    sentinel = torch.full((4,), 7.0, device="cuda")
    st = L.kda_chunk_fwd_noalloc(ctypes.byref(sh), *([ctypes.c_void_p(sentinel.data_ptr())] * 5),
                                 ctypes.c_float(0.1), None, None,
                                 ctypes.c_void_p(sentinel.data_ptr() + 256), None, _stream())
    assert st == 3 and b"kda_chunk_fwd with a workspace" in L.kda_last_error()
    torch.cuda.synchronize()
    assert torch.equal(sentinel, torch.full((4,), 7.0, device="cuda"))


def test_noalloc_binding_reuses_caller_outputs():
    import gated_delta_rule_80_amd as K
    inp = W.make_prefill(H=2, dk=128, dv=128, dtype="bf16", z_range=(2.0, 9.0), seed=94, B=1,
                         T=300, s0_std=0.05)
    d = to_dev(inp)
    o = torch.empty((1, 300, 2, 128), dtype=torch.bfloat16, device="cuda")
    fs = torch.empty((1, 2, 128, 128), dtype=torch.float32, device="cuda")
    o_b, f_b = K.chunk_fwd_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"],
                                   initial_state=d["initial_state"], out=o, final_state=fs)
    o_r, f_r = K.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"],
                           initial_state=d["initial_state"])
    torch.cuda.synchronize()
    assert o_b.data_ptr() == o.data_ptr() and f_b.data_ptr() == fs.data_ptr()
    assert torch.equal(o_b, o_r) and torch.equal(f_b, f_r)
    assert np.isfinite(o_b.float().cpu().numpy()).all()


@pytest.mark.gpu
@pytest.mark.parametrize("varlen", [False, True], ids=["rows", "packed"])
def test_noalloc_replayed_from_a_graph(varlen):
    """kda_chunk_fwd_noalloc captured in a HIP graph (the callers it is for):
    every replay gives the eager result bit for bit, also after an eager call
    on another problem has overwritten the shared device buffer in between."""
    import gated_delta_rule_80_amd as K
    if varlen:
        inp = W.make_prefill(H=2, dk=128, dv=128, dtype="bf16", z_range=(2.0, 9.0), seed=95,
                             lengths=[0, 130, 64, 257], s0_std=0.05)
    else:
        inp = W.make_prefill(H=2, dk=128, dv=128, dtype="bf16", z_range=(2.0, 9.0), seed=95,
                             B=2, T=400, s0_std=0.05)
    other = to_dev(W.make_prefill(H=3, dk=128, dv=128, dtype="bf16", z_range=(2.0, 9.0),
                                  seed=96, B=1, T=700, s0_std=0.05))
    d = to_dev(inp)
    B, T, H, dk = d["q"].shape
    N = inp["n_seqs"]

    def call(o, fs):
        K.chunk_fwd_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], scale=d["scale"],
                            initial_state=d["initial_state"], cu_seqlens=d["cu_seqlens"],
                            out=o, final_state=fs)

    o_ref = torch.empty((B, T, H, 128), dtype=torch.bfloat16, device="cuda")
    fs_ref = torch.empty((N, H, dk, 128), dtype=torch.float32, device="cuda")
    call(o_ref, fs_ref)
    torch.cuda.synchronize()
    o, fs = torch.empty_like(o_ref), torch.empty_like(fs_ref)
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
        K.chunk_fwd_noalloc(other["q"], other["k"], other["v"], other["g"], other["beta"],
                            initial_state=other["initial_state"])
        o.zero_()
        fs.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(fs, fs_ref), "replay %d" % replay
