"""HIP path vs the fp64 oracle, through the C ABI, on the standard workloads
and on the edge cases of the method (ragged tails, empty and length-1
sequences, NULL / aliased states, chunk-boundary continuation).

Tolerances: relative Frobenius error <= 1e-4 for fp32 storage, <= 5e-3 for
bf16 storage, on o and on the final state.
"""
import numpy as np
import pytest
import torch

import kda_workloads as W
import oracle
from kda_harness import TOL, check_prefill, gpu_prefill, oracle_prefill, rel_err, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_80_amd as K
    K.lib()


def small(H=2, T=200, dk=128, dv=128, dtype="bf16", z=(2.0, 9.0), seed=5, B=1, lengths=None,
          s0_std=0.05):
    return W.make_prefill(H=H, dk=dk, dv=dv, dtype=dtype, z_range=z, seed=seed, B=B, T=T,
                          lengths=lengths, s0_std=s0_std)


# ---------------------------------------------------------------- standard workloads
def test_workload1_tiny_fp32():
    inp = W.make_workload(1)
    check_prefill(inp, 16)


def test_workload2_prefill_full():
    inp = W.make_workload(2)
    check_prefill(inp, 64)


def test_workload4_varlen_full():
    """Every head, sequence and value column of the packed workload, with the
    per-(sequence, head) and per-chunk maxima."""
    inp = W.make_workload(4)
    check_prefill(inp, 64)


# Four columns of every 16-column value tile, at a different place in each tile,
# so every chain workgroup of the long workload is compared.
WORKLOAD5_COLS = sorted(16 * t + a for t in range(8) for a in {t % 16, (5 * t + 3) % 16,
                                                                 (11 * t + 7) % 16, 15 - t})


def test_workload5_long_all_heads():
    """All 32 heads of the T = 131072 workload on a column subset (columns of
    the value space are independent, so the subset is exact), with the
    per-head and per-chunk maxima over all 2048 chunks of every head."""
    assert len({c // 16 for c in WORKLOAD5_COLS}) == 8
    inp = W.make_workload(5)
    check_prefill(inp, 64, cols=WORKLOAD5_COLS)


# Sixteen value columns, one from each group of eight (the decode kernel's
# threads own four columns each), at varied places in the group.
DECODE_COLS = [8 * i + (3 * i) % 8 for i in range(16)]


def test_workload3_decode_256_steps_all_pairs():
    """All 128 x 32 (session, head) pairs at every one of the 256 steps, on a
    column subset: o stacked over the steps and the state after step 256, as a
    whole and per pair."""
    import gated_delta_rule_80_amd as K
    from kda_harness import state_pair_errors
    w = W.WORKLOADS[3]
    cols = DECODE_COLS
    state = W.make_decode_state(w)
    ref_state = W.to64(state[..., cols])
    st_dev = state.to("cuda")
    del state
    o_gpu, o_ref = [], []
    for s in range(w.steps):
        tok = W.make_decode_step(s, w)
        d = to_dev(tok)
        o = K.decode_step(d["q"], d["k"], d["v"], d["g"], d["beta"], st_dev, scale=w.scale)
        o_gpu.append(o[..., cols].double().cpu().numpy())
        orr, ref_state = oracle.decode_step(W.to64(tok["q"]), W.to64(tok["k"]),
                                            W.to64(tok["v"])[..., cols], W.to64(tok["g"]),
                                            W.to64(tok["beta"]), w.scale, ref_state)
        o_ref.append(orr)
    torch.cuda.synchronize()
    st = st_dev[..., cols].double().cpu().numpy()
    og, orf = np.stack(o_gpu), np.stack(o_ref)           # [steps, N, H, cols]
    eo, es = rel_err(og, orf), rel_err(st, ref_state)
    pair_o = np.sqrt(((og - orf) ** 2).sum(axis=(0, 3)) / (orf ** 2).sum(axis=(0, 3)))
    pair_s = state_pair_errors(st, ref_state)
    print("decode err o %.3e S %.3e  per pair max o %.3e S %.3e"
          % (eo, es, pair_o.max(), pair_s.max()), flush=True)
    tol = TOL["bf16"]
    assert np.all(np.isfinite(og)) and np.all(np.isfinite(st))
    assert eo <= tol and es <= tol and pair_o.max() <= tol and pair_s.max() <= tol


# ---------------------------------------------------------------- MFMA path edge cases
@pytest.mark.parametrize("T", [1, 37, 64, 65, 100, 130, 256])
def test_ragged_lengths(T):
    check_prefill(small(T=T), 64)


@pytest.mark.parametrize("T,B,s0", [(529, 1, True), (1000, 2, False), (4100, 1, True),
                                    (8192 + 33, 1, True)])
def test_multi_chunk_rows(T, B, s0):
    """Rows of 9 to 129 chunks, with and without an initial state, one or two rows."""
    check_prefill(small(T=T, B=B, H=2, s0_std=0.05 if s0 else None), 64)


def test_in_place_state_and_no_final_on_a_long_row():
    import gated_delta_rule_80_amd as K
    inp = small(T=1500, H=2)
    d = to_dev(inp)
    o_ref, s_ref = oracle_prefill(inp)
    st = d["initial_state"].clone()
    o, _ = K.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], initial_state=st,
                       final_state=st)
    o2, none = K.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"],
                           initial_state=d["initial_state"], output_final_state=False)
    torch.cuda.synchronize()
    assert none is None
    o64 = o.double().cpu().numpy().reshape(-1, 2, 128)
    assert rel_err(o64, o_ref) <= TOL["bf16"]
    assert rel_err(st.double().cpu().numpy(), s_ref) <= TOL["bf16"]
    assert torch.equal(o, o2)


def test_back_to_back_calls_reuse_workspace():
    """Consecutive calls on one stream share a workspace: the second call's
    intra-chunk work must not overwrite records the first call still reads."""
    import gated_delta_rule_80_amd as K
    a, b = small(T=2000, H=2, seed=21), small(T=2000, H=2, seed=22)
    da, db = to_dev(a), to_dev(b)
    ws = torch.empty(K.workspace_bytes(1, 2000, 2, 128, 128, 64, 1), dtype=torch.uint8,
                     device="cuda")
    outs = []
    for _ in range(3):
        for dd in (da, db):
            o, f = K.chunk_fwd(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"],
                               initial_state=dd["initial_state"], workspace=ws)
            outs.append((o, f))
    torch.cuda.synchronize()
    for i in range(2, 6):
        assert torch.equal(outs[i][0], outs[i % 2][0]) and torch.equal(outs[i][1], outs[i % 2][1])
    o_ref, s_ref = oracle_prefill(a)
    assert rel_err(outs[0][0].double().cpu().numpy().reshape(-1, 2, 128), o_ref) <= TOL["bf16"]


def test_equal_rows_batch():
    check_prefill(small(B=3, T=150, H=2), 64)


def test_varlen_with_empty_and_unit_sequences():
    inp = small(H=3, lengths=[0, 1, 130, 0, 64, 7, 200, 1], s0_std=0.05)
    o, fs = gpu_prefill(inp, 64)
    check_prefill(inp, 64)
    # zero-length sequences return their initial state exactly
    s0 = inp["initial_state"].double().numpy()
    assert np.array_equal(fs[0], s0[0]) and np.array_equal(fs[3], s0[3])


def test_null_initial_state():
    check_prefill(small(T=150, s0_std=None), 64)


def test_no_final_state():
    inp = small(T=100)
    o, fs = gpu_prefill(inp, 64, output_final_state=False)
    assert fs is None
    o_ref, _ = oracle_prefill(inp)
    assert rel_err(o, o_ref) <= TOL["bf16"]


def test_in_place_continuation_and_split_invariance():
    """final_state may alias initial_state; running T1 then T2 from the carried
    state matches one run over T1 + T2 (the state is all that crosses)."""
    import gated_delta_rule_80_amd as K
    inp = small(T=300, H=2)
    d = to_dev(inp)
    o_all, s_all = K.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"],
                               initial_state=d["initial_state"])
    st = d["initial_state"].clone()
    outs = []
    for a, b in [(0, 100), (100, 300)]:
        sl = lambda x: x[:, a:b].contiguous()  # noqa: E731
        o, _ = K.chunk_fwd(sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["g"]), sl(d["beta"]),
                           initial_state=st, final_state=st)
        outs.append(o)
    torch.cuda.synchronize()
    o_split = torch.cat(outs, dim=1)
    assert rel_err(o_split.double().cpu(), o_all.double().cpu()) <= 2e-3
    assert rel_err(st.double().cpu(), s_all.double().cpu()) <= 2e-3


def test_bitwise_deterministic():
    inp = small(T=200, H=2)
    o1, s1 = gpu_prefill(inp, 64)
    o2, s2 = gpu_prefill(inp, 64)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)


def test_varlen_equals_separate_calls():
    lengths = [70, 0, 129, 3]
    inp = small(H=2, lengths=lengths)
    o, fs = gpu_prefill(inp, 64)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    for n in range(len(lengths)):
        a, b = cu[n], cu[n + 1]
        if b == a:
            continue
        sub = dict(inp)
        for name in ("q", "k", "v", "g", "beta"):
            sub[name] = inp[name][:, a:b].contiguous()
        sub["initial_state"] = inp["initial_state"][n:n + 1].contiguous()
        sub["cu_seqlens"] = None
        o1, s1 = gpu_prefill(sub, 64)
        # the same kernels on the same chunks: identical bits
        assert np.array_equal(o1, o[a:b]) and np.array_equal(s1[0], fs[n])


def test_wide_value_tiles_match_narrow_bitwise():
    """With more (sequence, head) chains than CUs the chain kernel runs 32-column
    value tiles instead of 16-column ones; every column sees the same operations
    in the same order, so a packed call that takes the wide tiles gives the bits
    of per-sequence calls that take the narrow ones."""
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    lengths = [70, 0, 129, 3, 64, 200, 1, 65]
    H = -(-(n_cu // 8 + 1) // len(lengths))   # 8 H x 8 value tiles > n_cu chains
    inp = small(H=H, lengths=lengths)
    o, fs = gpu_prefill(inp, 64)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    for n in range(len(lengths)):
        a, b = cu[n], cu[n + 1]
        sub = dict(inp)
        for name in ("q", "k", "v", "g", "beta"):
            sub[name] = inp[name][:, a:b].contiguous()
        sub["initial_state"] = inp["initial_state"][n:n + 1].contiguous()
        sub["cu_seqlens"] = None
        if b == a:
            assert np.array_equal(fs[n], W.to64(inp["initial_state"][n]).astype(fs.dtype))
            continue
        o1, s1 = gpu_prefill(sub, 64)
        assert np.array_equal(o1, o[a:b]) and np.array_equal(s1[0], fs[n]), n
    check_prefill(inp, 64)


def test_moderate_decay_near_the_old_chunk_bound():
    # per-token log-decay about -0.23: a chunk's cumulative decay near -15,
    # where a single reference row per chunk would already leave fp16's range
    inp = small(T=256, z=(1.2, 1.5), s0_std=0.05)
    per_chunk = inp["g"].reshape(1, 4, 64, 2, 128).sum(dim=2)
    assert float(per_chunk.min()) < -14.0
    check_prefill(inp, 64)


def _strong_gate(inp, lo, hi, seed, mixed=False):
    """Replaces the log-decays by U(lo, hi) draws; with ``mixed`` every other
    channel keeps its weak decay, so long and short memories share a head."""
    gen = torch.Generator().manual_seed(seed)
    g = lo + (hi - lo) * torch.rand(inp["g"].shape, generator=gen, dtype=torch.float64)
    g = g.to(torch.float32)
    if mixed:
        g[..., 0::2] = inp["g"][..., 0::2]
    inp["g"] = g.contiguous()
    return inp


@pytest.mark.parametrize("lo,hi,mixed", [(-5.0, 0.0, False), (-5.0, -4.0, False),
                                         (-10.0, -9.0, False), (-10.0, 0.0, True)])
def test_strong_decay_sub_chunks(lo, hi, mixed):
    """Per-token log-decays down to -10 (the pages' layer bounds them at -5): a
    chunk's cumulative decay reaches -640, far outside any single-reference
    range, and the 16-token sub-chunks keep every factor finite."""
    inp = _strong_gate(small(T=333, H=2, s0_std=0.05), lo, hi, seed=61, mixed=mixed)
    check_prefill(inp, 64)


@pytest.mark.parametrize("lo,hi", [(-20.0, -10.0), (-100.0, -20.0), (-12.0, 0.0)])
def test_decay_below_the_floor(lo, hi):
    """Per-token log-decays below -10, which the MFMA path floors at -10 (a
    retention of e^-10 instead of less): the outputs stay finite and within the
    tolerance of the exact recurrence."""
    inp = _strong_gate(small(T=333, H=2, s0_std=0.05), lo, hi, seed=68)
    check_prefill(inp, 64)


def test_decay_minus_inf_on_channels_and_tokens():
    """log a = -inf (a channel that forgets everything in one token) on 5% of
    the (token, channel) entries, on every channel of some tokens, and on a
    whole channel of a head, among the workload's weak decays; packed
    sequences with ragged tails."""
    inp = small(H=2, lengths=[70, 1, 200, 64, 17, 130], s0_std=0.05, seed=69)
    g = inp["g"].clone()
    gen = torch.Generator().manual_seed(70)
    g[torch.rand(g.shape, generator=gen) < 0.05] = float("-inf")
    g[:, [3, 100, 101, 250], :, :] = float("-inf")
    g[:, :, 1, 77] = float("-inf")
    inp["g"] = g.contiguous()
    check_prefill(inp, 64)


def test_sub_chunk_edges_in_ragged_sequences():
    """Lengths that end inside, on and just past 16-token sub-chunk boundaries,
    with strong decays (each sub-chunk of a chunk has its own split point)."""
    lengths = [1, 15, 16, 17, 31, 33, 63, 65, 130]
    inp = _strong_gate(small(H=2, lengths=lengths, s0_std=0.05), -8.0, 0.0, seed=64)
    check_prefill(inp, 64)


def test_weak_and_strong_channel_blocks_in_one_head():
    """Channels 0-63 decay weakly and 64-127 strongly: the waves owning the
    first two 32-channel blocks take the fp16 path for the diagonal sub-chunk
    blocks, the other two the split-bf16 path, and their shares are summed."""
    inp = small(T=200, H=2, s0_std=0.05)
    weak = inp["g"][..., :64].clone()
    inp = _strong_gate(inp, -7.0, -1.0, seed=65)
    inp["g"][..., :64] = weak
    check_prefill(inp, 64)


@pytest.mark.parametrize("lo,hi", [(-0.40, -0.30), (-0.36, -0.34), (-0.19, -0.16)])
def test_decay_at_the_fp16_diagonal_threshold(lo, hi):
    """Sub-chunk decays near 2^-8 (about -0.35 per token), where a wave's choice
    between fp16 and split-bf16 diagonal operands flips from chunk to chunk;
    and whole-chunk decays near 2^-16 (about -0.17 per token), where its choice
    between one split point per chunk and sub-chunk splits flips."""
    inp = _strong_gate(small(T=320, H=2, s0_std=0.05), lo, hi, seed=66)
    check_prefill(inp, 64)


def test_strong_decay_varlen_and_scalar_gate():
    import gated_delta_rule_80_amd as K
    inp = _strong_gate(small(H=2, lengths=[70, 1, 200, 64, 17], s0_std=0.05), -6.0, 0.0,
                       seed=62)
    check_prefill(inp, 64)
    # one value per (token, head) through the scalar-gate entry point
    gs = inp["g"][..., 0].contiguous()
    inp["g"] = gs[..., None].expand(*gs.shape, 128).contiguous()
    o_ref, s_ref = oracle_prefill(inp, None, None)
    d = to_dev(inp)
    o, fs = K.chunk_fwd_scalar_gate(d["q"], d["k"], d["v"], gs.cuda(), d["beta"],
                                    scale=d["scale"], initial_state=d["initial_state"],
                                    cu_seqlens=d["cu_seqlens"])
    torch.cuda.synchronize()
    o64 = o.double().cpu().numpy()
    eo = rel_err(o64.reshape(-1, *o64.shape[2:]), o_ref)
    es = rel_err(fs.double().cpu().numpy(), s_ref)
    print("scalar gate, strong decay: err o %.3e  S %.3e" % (eo, es), flush=True)
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_strong_decay_fp32_path():
    inp = _strong_gate(small(T=150, H=2, dk=64, dv=64, dtype="f32"), -10.0, 0.0, seed=63)
    check_prefill(inp, 32)


# ---------------------------------------------------------------- degenerate cases of the method
def test_no_decay_is_deltanet():
    """a = 1 (g = 0): the delta rule without forgetting, through the same kernels."""
    inp = small(T=300, H=2)
    inp["g"] = torch.zeros_like(inp["g"])
    check_prefill(inp, 64)


def test_scalar_gate_per_head():
    """One decay value shared by every channel of a head (a scalar gate)."""
    inp = small(T=300, H=2, B=2)
    inp["g"] = inp["g"][..., :1].expand_as(inp["g"]).contiguous()
    check_prefill(inp, 64)


def test_zero_beta_is_pure_decay():
    """beta = 0: no writes, so S_T = Diag(e^{sum g}) S_0 and o_t reads the decayed S_0."""
    inp = small(T=200, H=2)
    inp["beta"] = torch.zeros_like(inp["beta"])
    check_prefill(inp, 64)
    _, fs = gpu_prefill(inp, 64)
    decay = np.exp(W.to64(inp["g"])[0].sum(axis=0))        # [H, d_k]
    expect = decay[:, :, None] * W.to64(inp["initial_state"])[0]
    assert rel_err(fs[0], expect) <= TOL["bf16"]


def test_zero_keys_leave_state_decaying_only():
    """k = 0 on every token: A, W, U's coupling and every write vanish."""
    inp = small(T=130, H=2)
    inp["k"] = torch.zeros_like(inp["k"])
    check_prefill(inp, 64)


# ---------------------------------------------------------------- shapes
@pytest.mark.parametrize("H,B,T", [(5, 2, 300), (1, 1, 64), (3, 4, 1), (12, 1, 513)])
def test_head_and_batch_shapes(H, B, T):
    """Head counts that do not fill the inter kernel's groups of 8 pairs, single
    tokens, and rows that are exactly one chunk."""
    check_prefill(small(H=H, B=B, T=T), 64)


def test_many_short_packed_sequences():
    lengths = np.random.default_rng(77).integers(0, 150, size=40).tolist()
    check_prefill(small(H=3, lengths=lengths), 64)


def test_thousands_of_packed_sequences():
    """More sequences than the chunk-table kernel has threads (1024): each
    thread of its scans then takes several sequences; many are empty."""
    lengths = np.random.default_rng(78).integers(0, 9, size=1500).tolist()
    check_prefill(small(H=2, lengths=lengths), 64)


def test_packed_position_does_not_change_a_sequence_bitwise():
    """Each packed sequence is chunked from its own first token and the chain
    kernel starts the longest sequences first, whatever their place in the
    pack: the same sequences packed in another order, each with its own
    initial state, give bitwise the same outputs and final states."""
    import gated_delta_rule_80_amd as K
    lengths = [40, 300, 0, 129, 64, 300, 1, 200]
    inp = small(H=3, lengths=lengths, s0_std=0.05, seed=81)
    d = to_dev(inp)
    o, fs = K.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], scale=d["scale"],
                        initial_state=d["initial_state"], cu_seqlens=d["cu_seqlens"])
    perm = [5, 2, 7, 0, 3, 6, 1, 4]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    rows = torch.cat([torch.arange(int(cu[n]), int(cu[n + 1])) for n in perm]).cuda()
    lp = [lengths[n] for n in perm]
    cu_p = torch.tensor(np.concatenate([[0], np.cumsum(lp)]).astype(np.int32)).cuda()
    take = lambda t: t[:, rows].contiguous()  # noqa: E731
    o2, fs2 = K.chunk_fwd(take(d["q"]), take(d["k"]), take(d["v"]), take(d["g"]),
                          take(d["beta"]), scale=d["scale"],
                          initial_state=d["initial_state"][perm].contiguous(), cu_seqlens=cu_p)
    torch.cuda.synchronize()
    assert torch.equal(o[:, rows], o2)
    assert torch.equal(fs[perm], fs2)


def test_chain_launches_split_over_pair_batches():
    """16,500 packed sequences x 32 heads = 528,000 (sequence, head) pairs, more
    than one chain launch takes (2^19 pairs, to stay within 2^32 threads), so
    the chain goes out in two launches.  Sequences on both sides of the split
    are checked one by one against the oracle (all heads, o and final state)."""
    import gated_delta_rule_80_amd as K
    H, N = 32, 16500
    split = (1 << 19) // H                       # first sequence of the second launch
    lengths = np.random.default_rng(79).integers(0, 5, size=N)
    lengths[[0, split - 1, split, N - 1]] = [3, 4, 2, 4]
    inp = small(H=H, lengths=lengths.tolist(), s0_std=None)
    d = to_dev(inp)
    o, fs = K.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], scale=d["scale"],
                        cu_seqlens=d["cu_seqlens"])
    torch.cuda.synchronize()
    cu = np.concatenate([[0], np.cumsum(lengths)])
    picks = [0, 1, 777, split - 2, split - 1, split, split + 1, split + 50, N - 1]
    errs = []
    for n in picks:
        t0, t1 = int(cu[n]), int(cu[n + 1])
        args = [W.to64(inp[x])[0, t0:t1] for x in ("q", "k", "v", "g", "beta")]
        o_ref, s_ref = oracle.prefill(*args, inp["scale"], None, [0, t1 - t0])
        got_s = fs[n].double().cpu().numpy()
        if t1 > t0:
            errs.append(rel_err(o[0, t0:t1].double().cpu().numpy(), o_ref))
            errs.append(rel_err(got_s, s_ref[0]))
        else:
            assert not got_s.any()               # no tokens, no initial state: zeros
    print("pair-batch split: max err %.3e over %d sequences" % (max(errs), len(picks)), flush=True)
    assert max(errs) <= TOL["bf16"]


# ---------------------------------------------------------------- fp32 path
@pytest.mark.parametrize("d,C,T", [(16, 16, 64), (16, 32, 77), (16, 64, 130), (32, 16, 50),
                                   (32, 32, 96), (32, 64, 150), (64, 16, 40), (64, 64, 129)])
def test_fp32_path(d, C, T):
    check_prefill(small(H=2, T=T, dk=d, dv=d, dtype="f32"), C)


def test_fp32_d128_prefill_workload2_shape():
    """fp32 storage at d_k = d_v = 128, C = 64 on the shape of workload 2
    (B = 2, H = 8, T = 2048, S0 ~ N(0, 0.01^2)): the fp32 path, 1e-4."""
    inp = W.make_prefill(H=8, dk=128, dv=128, dtype="f32", z_range=(2.0, 9.0), seed=1002, B=2,
                         T=2048, s0_std=0.01)
    check_prefill(inp, 64)


def test_fp32_d128_packed_ragged_strong_decay():
    """fp32 at d = 128, C = 64: packed sequences with ragged tails (and an
    empty one), log-decays in [-10, 0] on every other channel among weak ones."""
    inp = small(H=3, dk=128, dv=128, dtype="f32", lengths=[1, 63, 64, 65, 0, 200, 333],
                s0_std=0.05, seed=71)
    inp = _strong_gate(inp, -10.0, 0.0, seed=72, mixed=True)
    check_prefill(inp, 64)


@pytest.mark.parametrize("C", [16, 32])
def test_fp32_d128_smaller_chunks(C):
    check_prefill(small(H=2, T=150, dk=128, dv=128, dtype="f32"), C)


def test_fp32_varlen():
    check_prefill(small(H=2, dk=16, dv=16, dtype="f32", lengths=[5, 0, 33, 16, 1]), 16)


# ---------------------------------------------------------------- decode variants
@pytest.mark.parametrize("d,dtype", [(16, "f32"), (32, "bf16"), (64, "f32"), (128, "f32")])
def test_decode_shapes(d, dtype):
    import gated_delta_rule_80_amd as K
    w = W.Workload(3, "decode", "decode", H=3, dk=d, dv=d, dtype=dtype, z_range=(2.0, 9.0),
                   n_sessions=5, steps=4, state_std=0.05)
    state = W.make_decode_state(w)
    ref = W.to64(state)
    st = state.to("cuda")
    for s in range(w.steps):
        tok = W.make_decode_step(s, w)
        dd = to_dev(tok)
        o = K.decode_step(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], st, scale=w.scale)
        o_ref, ref = oracle.decode_step(*(W.to64(tok[n]) for n in ("q", "k", "v", "g", "beta")),
                                        w.scale, ref)
        torch.cuda.synchronize()
        tol = TOL[dtype]
        assert rel_err(o.double().cpu().numpy(), o_ref) <= tol
    assert rel_err(st.double().cpu().numpy(), ref) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_with_strong_decays(dtype):
    """Per-token log-decays in [-10, 0] (and exactly -inf for one channel: a
    channel that forgets everything) through the decode step: it scales the
    state by e^g directly, so any log-decay is in range."""
    import gated_delta_rule_80_amd as K
    w = W.Workload(3, "decode", "decode", H=3, dk=128, dv=128, dtype=dtype, z_range=(2.0, 9.0),
                   n_sessions=6, steps=5, state_std=0.05)
    state = W.make_decode_state(w)
    ref = W.to64(state)
    st = state.to("cuda")
    gen = torch.Generator().manual_seed(67)
    outs, refs = [], []
    for s in range(w.steps):
        tok = W.make_decode_step(s, w)
        tok["g"] = (-10.0 * torch.rand(tok["g"].shape, generator=gen,
                                       dtype=torch.float64)).to(torch.float32)
        tok["g"][..., 5] = float("-inf")
        dd = to_dev(tok)
        outs.append(K.decode_step(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], st,
                                  scale=w.scale).double().cpu().numpy())
        o_ref, ref = oracle.decode_step(*(W.to64(tok[n]) for n in ("q", "k", "v", "g", "beta")),
                                        w.scale, ref)
        refs.append(o_ref)
    torch.cuda.synchronize()
    eo = rel_err(np.stack(outs), np.stack(refs))
    es = rel_err(st.double().cpu().numpy(), ref)
    print("decode, strong decays: err o %.3e  S %.3e" % (eo, es), flush=True)
    assert np.isfinite(eo) and eo <= TOL[dtype] and es <= TOL[dtype]


def test_decode_steps_match_prefill():
    """T decode steps on one session equal a T-token prefill (both on the GPU)."""
    import gated_delta_rule_80_amd as K
    inp = small(H=2, T=40)
    d = to_dev(inp)
    o_p, s_p = K.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"],
                           initial_state=d["initial_state"])
    st = d["initial_state"].clone()
    outs = []
    for t in range(40):
        outs.append(K.decode_step(d["q"][:, t].contiguous(), d["k"][:, t].contiguous(),
                                  d["v"][:, t].contiguous(), d["g"][:, t].contiguous(),
                                  d["beta"][:, t].contiguous(), st))
    torch.cuda.synchronize()
    o_d = torch.stack(outs, dim=1)
    assert rel_err(o_d.double().cpu(), o_p.double().cpu()) <= 3e-3
    assert rel_err(st.double().cpu(), s_p.double().cpu()) <= 3e-3
