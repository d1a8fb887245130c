"""The overlapped prefill order (kda_set_prefill_overlap): the chain kernel runs
beside the intra-chunk kernel and takes each chunk's factors as they are
published, through the L2 of the XCD both kernels place the head on.  Both
orders run the same arithmetic on the same factors, so they must give the same
bits; every comparison here is exact.  The workspace is filled with NaN bytes
before each overlapped call, so a record read before it was written would show
up in o.  The first word of the workspace tells whether a call needed the
repair pass (the chain refused a record and reran in the serial order): the
fast path must not need it, and modes 2 and 3 force it.

This file runs before the other GPU tests on purpose: the library's side stream
is created by the first overlapped call, and a process has only a few hardware
queues (4 here).  Created after other tests have made streams of their own, the
side stream may share the caller's queue; then the intra-chunk kernel cannot
start before the chain ends, every chain gives up after 250 us, and each call
takes the repair pass (correct, but not the path these tests are about)."""
import contextlib

import pytest
import torch

import gated_delta_rule_80_amd as K
import kda_harness as Hn
import kda_workloads as W


@contextlib.contextmanager
def prefill_order(mode):
    prev = K.set_prefill_overlap(mode)
    try:
        yield
    finally:
        K.set_prefill_overlap(prev)


def same(a, b):
    """Bitwise equality of two tensors of one dtype (NaN equal to itself)."""
    view = torch.int32 if a.dtype == torch.float32 else torch.int16
    return a.dtype == b.dtype and torch.equal(a.view(view), b.view(view))


def _inputs(B, H, T, seed, z_range=(2.0, 9.0)):
    return Hn.to_dev(W.make_prefill(H=H, dk=128, dv=128, dtype="bf16", z_range=z_range, seed=seed,
                                    B=B, T=T, s0_std=0.01))


def _call(d, mode, fill=0xFF, fn=None, **kw):
    """One prefill in the given order with a caller-owned workspace filled with
    `fill` bytes first; returns (o, final state, the workspace's first word)."""
    fn = fn or K.chunk_fwd
    B, T, H = d["q"].shape[:3]
    n = K.workspace_bytes(B, T, H, 128, 128, 64, B)
    ws = torch.full((n,), fill, dtype=torch.uint8, device="cuda")
    with prefill_order(mode):
        o, fs = fn(d["q"], d["k"], d["v"], d["g"], d["beta"], scale=d["scale"],
                   initial_state=d["initial_state"], chunk_size=64, workspace=ws, **kw)
    torch.cuda.synchronize()
    words = ws[:24].view(torch.int32).tolist()
    _call.detail = words[:6]
    return o, fs, words[0]


# Rows of at least 128 chunks take the overlapped order; two have a ragged tail.
SHAPES = [(1, 32, 16384), (1, 8, 8192), (2, 16, 8192), (1, 32, 8130), (4, 8, 8200)]


@pytest.mark.gpu
@pytest.mark.parametrize("B,H,T", SHAPES, ids=["B1_H32_T16384", "B1_H8_T8192", "B2_H16_T8192",
                                               "B1_H32_T8130_ragged", "B4_H8_T8200_ragged"])
def test_overlapped_order_gives_the_serial_bits(B, H, T):
    print("overlapped vs serial prefill B=%d H=%d T=%d" % (B, H, T), flush=True)
    d = _inputs(B, H, T, seed=600 + T % 97)
    o0, s0, _ = _call(d, 0)
    o1, s1, st = _call(d, 1)
    # status[1..5]: why (1 not seen in time, 2 another XCD), flag, XCD, chunk, head
    assert st == 0, "the overlapped call needed its repair pass: %s" % _call.detail
    assert same(o1, o0) and same(s1, s0)


@pytest.mark.gpu
def test_overlapped_order_reads_this_calls_records():
    # Two problems through one workspace: the second call's chain must read the
    # records its own intra-chunk kernel writes, not the first call's.
    print("overlapped prefill, two problems through one workspace", flush=True)
    a = _inputs(1, 32, 8192, seed=611)
    b = _inputs(1, 32, 8192, seed=612, z_range=(-5.0, 0.0))
    n = K.workspace_bytes(1, 8192, 32, 128, 128, 64, 1)
    ws = torch.full((n,), 0xFF, dtype=torch.uint8, device="cuda")
    outs = []
    with prefill_order(1):
        for d in (a, b, a):
            o, fs = K.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], scale=d["scale"],
                                initial_state=d["initial_state"], chunk_size=64, workspace=ws)
            torch.cuda.synchronize()
            assert int(ws[:4].view(torch.int32).item()) == 0
            outs.append((o.clone(), fs.clone()))
    for d, (o, fs) in zip((a, b, a), outs):
        o0, s0, _ = _call(d, 0)
        assert same(o, o0) and same(fs, s0)


@pytest.mark.gpu
@pytest.mark.parametrize("B,H,T", [(1, 32, 8192), (2, 8, 8192)], ids=["B1_H32_T8192", "B2_H8_T8192"])
def test_repair_pass_gives_the_serial_bits(B, H, T):
    # Mode 2: the chain accepts no record, runs on whatever the workspace holds
    # (NaN bytes or records being written) and marks the call; the repair pass
    # then reruns the chain after both kernels have ended.
    print("repair pass B=%d H=%d T=%d" % (B, H, T), flush=True)
    d = _inputs(B, H, T, seed=620 + H)
    o0, s0, _ = _call(d, 0)
    o2, s2, st = _call(d, 2)
    assert st != 0
    assert same(o2, o0) and same(s2, s0)


@pytest.mark.gpu
@pytest.mark.parametrize("B,H,T", [(1, 32, 8192), (4, 8, 8200)], ids=["B1_H32_T8192", "B4_H8_T8200"])
def test_chains_that_give_up_at_the_start(B, H, T):
    # Mode 3: a chain whose first records are not yet published gives up at
    # once (as after 250 us when the intra-chunk kernel is queued behind it);
    # whatever mix of chains gave up, the results are the serial ones.
    print("chains giving up at the start B=%d H=%d T=%d" % (B, H, T), flush=True)
    d = _inputs(B, H, T, seed=650 + H)
    o0, s0, _ = _call(d, 0)
    for _ in range(3):
        o3, s3, _ = _call(d, 3)
        assert same(o3, o0) and same(s3, s0)


@pytest.mark.gpu
def test_overlapped_scalar_gate_and_input_forms():
    print("overlapped prefill: scalar gate and the _ex input forms", flush=True)
    d = _inputs(1, 16, 8192, seed=631)
    gs = d["g"][..., 0].contiguous()
    res = {}
    for mode in (0, 1):
        with prefill_order(mode):
            o_sg, s_sg = K.chunk_fwd_scalar_gate(d["q"], d["k"], d["v"], gs, d["beta"],
                                                 scale=d["scale"], initial_state=d["initial_state"])
            # beta as a logit keeps the overlapped order; the logit gate and the
            # norms make the intra-chunk work as long as the chain: serial order
            o_b, s_b = K.chunk_fwd_ex(d["q"], d["k"], d["v"], d["g"], d["beta"] * 4.0 - 2.0,
                                      scale=d["scale"], initial_state=d["initial_state"],
                                      beta_is_logit=True)
            o_ex, s_ex = K.chunk_fwd_ex(d["q"], d["k"], d["v"], -d["g"] * 50.0, d["beta"],
                                        scale=d["scale"], initial_state=d["initial_state"],
                                        gate_is_logit=True, beta_is_logit=True, l2norm_qk=True)
        torch.cuda.synchronize()
        res[mode] = (o_sg, s_sg, o_b, s_b, o_ex, s_ex)
    for x0, x1 in zip(res[0], res[1]):
        assert same(x0, x1)


@pytest.mark.gpu
def test_serial_order_where_overlap_does_not_apply():
    # In-place continuation (final state over the initial state), H not a
    # multiple of 8, more pairs than half the CUs and short rows take the
    # serial order; their results must still be the serial ones.
    print("prefill orders: cases that stay serial", flush=True)
    d = _inputs(1, 8, 4096, seed=644)   # 64 chunks per row
    o0, s0, _ = _call(d, 0)
    o1, s1, st = _call(d, 1, fill=0)
    assert st == 0 and same(o1, o0) and same(s1, s0)
    d = _inputs(1, 12, 8192, seed=641)
    o0, s0, _ = _call(d, 0)
    o1, s1, _ = _call(d, 1)
    assert same(o1, o0) and same(s1, s0)
    d = _inputs(2, 32, 8192, seed=643)   # 64 pairs: 32-column chains would fill every CU
    o0, s0, _ = _call(d, 0)
    o1, s1, _ = _call(d, 1)
    assert same(o1, o0) and same(s1, s0)
    d = _inputs(1, 32, 8192, seed=642)
    ref_o, ref_s, _ = _call(d, 0)
    st = d["initial_state"].clone()
    with prefill_order(1):
        o, fs = K.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], scale=d["scale"],
                            initial_state=st, chunk_size=64, final_state=st)
    torch.cuda.synchronize()
    assert same(o, ref_o) and same(st, ref_s)


def test_overlap_mode_setter_rejects_unknown_modes():
    prev = K.set_prefill_overlap(1)
    try:
        with pytest.raises(ValueError):
            K.set_prefill_overlap(4)
        with pytest.raises(ValueError):
            K.set_prefill_overlap(-1)
        assert K.set_prefill_overlap(0) == 1
        assert K.set_prefill_overlap(1) == 0
    finally:
        K.set_prefill_overlap(prev)
