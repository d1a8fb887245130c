"""The record handoff a fused prefill would need, run on the GPU
(tests/handoff_gpu/ring_probe.hip; protocol modelled on the CPU in
tests/handoff_model/).  Producers stream records through a ring; R consumers
per stream check every word.  Every wait in the kernel is bounded by a poll
count and by a wall-clock deadline and polls a shared abort word, so each run
ends on its own; the abort path is exercised by streams whose producer the
host leaves out.  Mode 2 keeps each stream's roles on one XCD and hands the
records over through its L2 alone; the tests check the placement the kernel
reports as well as every word.
"""
import ctypes
import os
import time

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "handoff_gpu", "libringprobe.so")


def _lib():
    if not os.path.exists(LIB):
        raise RuntimeError("%s is not built; run __graft_entry__.build()" % LIB)
    lib = ctypes.CDLL(LIB)
    f = lib.ring_probe_launch
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p] * 7 + [ctypes.c_int] * 6 + [ctypes.c_uint32, ctypes.c_double,
                                                               ctypes.c_int, ctypes.c_void_p]
    return lib


def test_probe_library_exports_and_validates_on_the_host():
    f = _lib().ring_probe_launch
    fake = ctypes.c_void_p(0x100000)   # never dereferenced: validation fails first
    args = [fake] * 7 + [4, 8, 4, 16, 1024, 4, 1000, 1.0, 0, None]
    assert f(*([None] + args[1:])) == -1                       # null buffer
    # P = 0, R = 17, S = 65, 24-byte records, more producers than streams,
    # bounds of 0 and 11 s, mode 2 with P = 4 (not a multiple of 8), mode 3
    for i, bad in [(7, 0), (8, 17), (9, 65), (11, 24), (12, 5), (14, 0.0), (14, 11.0), (15, 2),
                   (15, 3)]:
        a = list(args)
        a[i] = bad
        assert f(*a) == -1, (i, bad)


def _run(P, R, S, n, rec_bytes, active, spin, max_s, mode=0):
    import torch
    dev = torch.device("cuda:0")
    ring = torch.zeros(P * S * rec_bytes // 4, dtype=torch.int32, device=dev)
    ready = torch.zeros(P * S, dtype=torch.int32, device=dev)
    done = torch.zeros(P * S, dtype=torch.int32, device=dev)
    words = torch.zeros(2, dtype=torch.int32, device=dev)      # abort, bad
    progress = torch.full((P * (1 + R),), -1, dtype=torch.int32, device=dev)
    xcc = torch.full((P * (1 + R),), -1, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream().cuda_stream
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.time()
    e0.record()
    rc = _lib().ring_probe_launch(ring.data_ptr(), ready.data_ptr(), done.data_ptr(),
                                  words.data_ptr(), words.data_ptr() + 4, progress.data_ptr(),
                                  xcc.data_ptr(), P, R, S, n, rec_bytes, active, spin, max_s, mode, st)
    e1.record()
    torch.cuda.synchronize()
    wall = time.time() - t0
    assert rc == 0
    _run.xcc = xcc.cpu().tolist()
    return (int(words[0]), int(words[1]), progress.cpu().tolist(), e0.elapsed_time(e1), wall)


def _one_xcd_per_stream(P, R):
    """Every role of a stream ran on the XCD of its producer, and the streams
    spread over all 8 XCDs."""
    x = _run.xcc
    ok = all(x[P + p * R + r] == x[p] for p in range(P) for r in range(R))
    return ok and sorted(set(x[:P])) == list(range(8))


@pytest.mark.gpu
@pytest.mark.parametrize("mode", [0, 1, 2], ids=["acquire_polls", "one_fence", "one_xcd"])
def test_ring_handoff_delivers_every_record(mode):
    P, R, S, n = 8, 8, 4, 512
    print("ring handoff P=%d R=%d S=%d chunks=%d rec=61952 B mode %d" % (P, R, S, n, mode),
          flush=True)
    abort, bad, prog, ms, _ = _run(P, R, S, n, 61952, P, 1 << 22, 5.0, mode)
    assert abort == 0 and bad == 0
    assert prog == [n] * (P * (1 + R))
    if mode == 2:
        assert _one_xcd_per_stream(P, R), _run.xcc
    print("  %.3f ms, %.3f us per record per stream" % (ms, 1e3 * ms / n), flush=True)


@pytest.mark.gpu
def test_ring_handoff_abort_ends_every_wait():
    # Streams 2 and 3 have no producer: their consumers run out of polls, the
    # first stores its code in the abort word, and every other wait returns.
    P, R, S, n = 4, 8, 2, 64
    print("ring handoff abort path P=%d R=%d, producers of streams 2, 3 left out" % (P, R),
          flush=True)
    abort, bad, prog, ms, wall = _run(P, R, S, n, 4096, 2, 1000, 2.0)
    assert bad == 0
    assert P + 2 * R <= abort - 1 < P + 4 * R, abort            # a consumer of a dead stream
    assert all(prog[P + q] == 0 for q in range(2 * R, 4 * R))    # they got nothing
    assert prog[2] == prog[3] == 0                                # the absent producers
    assert wall < 5.0
    print("  aborted by block %d after %.3f ms" % (abort - 1, ms), flush=True)


@pytest.mark.gpu
@pytest.mark.parametrize("mode,rec,S", [(0, 61952, 4), (1, 61952, 4), (1, 1024, 4), (1, 1024, 16),
                                        (1, 61952, 16), (2, 61952, 4), (2, 1024, 4), (2, 61952, 16)],
                         ids=["acquire_polls", "one_fence", "one_fence_1KB", "one_fence_1KB_16slots",
                              "one_fence_16slots", "one_xcd", "one_xcd_1KB", "one_xcd_16slots"])
def test_ring_handoff_at_the_prefill_shape(mode, rec, S):
    # 32 streams (heads) x 8 consumers (value tiles) x 2048 records of the
    # prefill's record size (and of 1 KB, for the round trip alone), 4 or 16
    # ring slots per stream: the rate at which the handoff by itself moves records.
    P, R, n = 32, 8, 2048
    print("ring handoff P=%d R=%d S=%d chunks=%d rec=%d B mode %d" % (P, R, S, n, rec, mode),
          flush=True)
    abort, bad, prog, ms, _ = _run(P, R, S, n, rec, P, 1 << 22, 8.0, mode)
    assert abort == 0 and bad == 0
    assert prog == [n] * (P * (1 + R))
    if mode == 2:
        assert _one_xcd_per_stream(P, R), _run.xcc
    print("  %.3f ms, %.3f us per record per stream, %.1f GB/s written, %.1f GB/s read"
          % (ms, 1e3 * ms / n, P * n * rec / ms / 1e6, R * P * n * rec / ms / 1e6), flush=True)
