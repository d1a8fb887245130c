"""The C ABI library on the host: it loads, exports every declared symbol, and
rejects bad arguments before touching the GPU (no compute call is made)."""
import ctypes
import os
import re
import subprocess

import pytest
import torch  # noqa: F401  (load torch's HIP runtime first, as the binding does)

import gated_delta_rule_80_amd as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("kda_chunk_fwd", "kda_decode_step", "kda_chunk_fwd_workspace_bytes",
              "kda_status_string", "kda_abi_version", "kda_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", K.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    lib = K.lib()
    for n in declared_functions():
        assert getattr(lib, n) is not None


def test_abi_version_and_status_strings():
    lib = K.lib()
    assert lib.kda_abi_version() == 6
    for code, name in K.STATUS.items():
        assert lib.kda_status_string(code).decode() == name


def shape(**kw):
    base = dict(batch=1, seqlen=2048, heads=32, d_k=128, d_v=128, chunk_size=64, num_seqs=1,
                dtype_code=K.KDA_BF16)
    base.update(kw)
    return K.make_shape(base["batch"], base["seqlen"], base["heads"], base["d_k"], base["d_v"],
                        base["chunk_size"], base["num_seqs"], base["dtype_code"])


def ws(sh):
    return K.lib().kda_chunk_fwd_workspace_bytes(ctypes.byref(sh))


def test_workspace_query():
    # records of 61952 bytes per (chunk, head) plus chunk table and offsets
    n = ws(shape())
    assert n >= 32 * (2048 // 64) * 61952
    assert ws(shape(seqlen=131072)) >= 32 * 2048 * 61952
    assert ws(shape(d_k=64)) == 0                       # unsupported
    assert ws(shape(batch=0)) == 0                      # invalid
    assert ws(shape(d_k=16, d_v=16, chunk_size=16, dtype_code=K.KDA_F32)) == 0  # fp32 path: none
    # varlen bound T/C + N chunks never below B * ceil(T/C)
    for B, T in [(1, 1), (3, 65), (2, 64), (5, 127)]:
        assert ws(shape(batch=B, seqlen=T, num_seqs=B)) >= B * ((T + 63) // 64) * 32 * 61952


FAKE = ctypes.c_void_p(0x100000)   # aligned, never dereferenced: validation fails first


def call_chunk(sh, **over):
    args = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, scale=ctypes.c_float(0.1), s0=None,
                cu=None, o=ctypes.c_void_p(0x200000), fs=None, ws=ctypes.c_void_p(0x300000),
                wsb=ctypes.c_size_t(1 << 40), stream=None)
    args.update(over)
    return K.lib().kda_chunk_fwd(ctypes.byref(sh) if sh is not None else None, args["q"],
                                 args["k"], args["v"], args["g"], args["beta"], args["scale"],
                                 args["s0"], args["cu"], args["o"], args["fs"], args["ws"],
                                 args["wsb"], args["stream"])


def test_chunk_fwd_rejects_bad_arguments():
    lib = K.lib()
    assert call_chunk(None) == 1
    assert call_chunk(shape(heads=0)) == 1
    assert call_chunk(shape(d_k=96, d_v=96)) == 2
    assert call_chunk(shape(chunk_size=32)) == 2
    assert call_chunk(shape(dtype_code=7)) == 1
    assert call_chunk(shape(batch=2, num_seqs=3)) == 1                 # N must equal B
    assert call_chunk(shape(batch=2, num_seqs=2), cu=FAKE) == 1        # varlen needs B == 1
    assert call_chunk(shape(), q=None) == 1
    assert call_chunk(shape(), q=ctypes.c_void_p(0x100004)) == 1       # misaligned
    assert call_chunk(shape(), o=FAKE) == 1                            # o aliases an input
    assert call_chunk(shape(), ws=None) == 1
    assert call_chunk(shape(), ws=ctypes.c_void_p(0x300010)) == 1      # workspace alignment
    assert call_chunk(shape(), wsb=ctypes.c_size_t(1024)) == 3
    assert b"workspace" in lib.kda_last_error()


def test_decode_rejects_bad_arguments():
    lib = K.lib()
    P = ctypes.c_void_p(0x100000)
    O = ctypes.c_void_p(0x200000)
    f = ctypes.c_float(0.1)
    assert lib.kda_decode_step(0, 32, 128, 128, K.KDA_BF16, P, P, P, P, P, f, P, O, None) == 1
    assert lib.kda_decode_step(4, 32, 96, 96, K.KDA_BF16, P, P, P, P, P, f, P, O, None) == 2
    assert lib.kda_decode_step(4, 32, 128, 64, K.KDA_BF16, P, P, P, P, P, f, P, O, None) == 2
    assert lib.kda_decode_step(4, 32, 128, 128, 5, P, P, P, P, P, f, P, O, None) == 1
    assert lib.kda_decode_step(4, 32, 128, 128, K.KDA_BF16, None, P, P, P, P, f, P, O, None) == 1
    assert lib.kda_decode_step(4, 32, 128, 128, K.KDA_BF16, P, P, P, P, P, f, P, P, None) == 1
    assert lib.kda_decode_step(4, 32, 128, 128, K.KDA_BF16, P, P, P, P, P, f, P,
                               ctypes.c_void_p(0x200008), None) == 1
    assert b"aligned" in lib.kda_last_error()


def test_decode_grid_above_32_bit_threads_is_an_error_not_a_launch():
    """2^20 sessions x 2047 heads fits the pair count but not one launch's 2^32
    threads at d = 128: the call reports it before launching anything."""
    lib = K.lib()
    P, O, f = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000), ctypes.c_float(0.1)
    assert lib.kda_decode_step(1 << 20, 2047, 128, 128, K.KDA_BF16, P, P, P, P, P, f, P, O,
                               None) == 4
    assert b"2^32" in lib.kda_last_error()


def test_last_error_is_cleared_on_entry():
    lib = K.lib()
    call_chunk(shape(heads=0))
    assert lib.kda_last_error() != b""
    # a call that fails later in validation overwrites the message
    call_chunk(shape(d_k=96, d_v=96))
    assert b"no kernel" in lib.kda_last_error()


def test_binding_refuses_host_tensors():
    q = torch.zeros(1, 64, 1, 16)
    with pytest.raises(ValueError):
        K.chunk_fwd(q, q, q, q.float(), torch.zeros(1, 64, 1), chunk_size=16)


def call_chunk_sg(sh, **over):
    args = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, scale=ctypes.c_float(0.1), s0=None,
                cu=None, o=ctypes.c_void_p(0x200000), fs=None, ws=ctypes.c_void_p(0x300000),
                wsb=ctypes.c_size_t(1 << 40), stream=None)
    args.update(over)
    return K.lib().kda_chunk_fwd_scalar_gate(
        ctypes.byref(sh) if sh is not None else None, args["q"], args["k"], args["v"],
        args["g"], args["beta"], args["scale"], args["s0"], args["cu"], args["o"], args["fs"],
        args["ws"], args["wsb"], args["stream"])


def test_scalar_gate_entry_points_validate_like_the_others():
    lib = K.lib()
    P, O, f = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000), ctypes.c_float(0.1)
    assert call_chunk_sg(shape(heads=0)) == 1
    assert call_chunk_sg(shape(d_k=96, d_v=96)) == 2
    assert call_chunk_sg(shape(), q=None) == 1
    assert call_chunk_sg(shape(), g=ctypes.c_void_p(0x100002)) == 1       # 4-byte alignment
    assert b"scalar gate" in lib.kda_last_error()
    assert call_chunk_sg(shape(), wsb=ctypes.c_size_t(1024)) == 3
    # a NULL gate (no decay) passes validation up to the workspace check
    assert call_chunk_sg(shape(), g=None, wsb=ctypes.c_size_t(1024)) == 3
    # the per-channel entry still needs its gate
    assert call_chunk(shape(), g=None) == 1
    dsg = lib.kda_decode_step_scalar_gate
    assert dsg(0, 32, 128, 128, K.KDA_BF16, P, P, P, P, P, f, P, O, None) == 1
    assert dsg(4, 32, 96, 96, K.KDA_BF16, P, P, P, P, P, f, P, O, None) == 2
    assert dsg(4, 32, 128, 128, K.KDA_BF16, P, P, P, ctypes.c_void_p(0x100001), P, f, P, O,
               None) == 1
    assert lib.kda_decode_step(4, 32, 128, 128, K.KDA_BF16, P, P, P, None, P, f, P, O, None) == 1


def test_binding_scalar_gate_shape_checks():
    q = torch.zeros(1, 64, 2, 16)
    with pytest.raises(ValueError):     # per-channel gate shape given to the scalar entry
        K.chunk_fwd_scalar_gate(q, q, q, q.float(), torch.zeros(1, 64, 2), chunk_size=16)


# ---------------------------------------------------------------- backward
def call_bwd(sh, **kw):
    lib = K.lib()
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first
    args = dict(q=fake, k=fake, v=fake, g=fake, beta=fake, s0=None, cu=None, do=fake, dfin=None,
                dq=ctypes.c_void_p(0x2000), dk=ctypes.c_void_p(0x3000), dv=ctypes.c_void_p(0x4000),
                dg=ctypes.c_void_p(0x5000), db=ctypes.c_void_p(0x6000), ds0=None,
                ws=ctypes.c_void_p(0x10000), wsb=ctypes.c_size_t(1 << 40))
    args.update(kw)
    return lib.kda_chunk_bwd(ctypes.byref(sh), args["q"], args["k"], args["v"], args["g"],
                             args["beta"], ctypes.c_float(0.25), args["s0"], args["cu"], args["do"],
                             args["dfin"], args["dq"], args["dk"], args["dv"], args["dg"],
                             args["db"], args["ds0"], args["ws"], args["wsb"], None)


def test_backward_workspace_at_d128_is_that_of_16_token_chunks():
    """At d = 128 the backward runs 16-token chunks for a requested 16, 32 or
    64, so the workspace it asks for is the same."""
    sizes = {C: K.workspace_bytes_bwd(1, 4096, 8, 128, C, 1) for C in (16, 32, 64)}
    assert sizes[16] > 0 and sizes[16] == sizes[32] == sizes[64]
    assert K.workspace_bytes_bwd(1, 4096, 8, 128, 48, 1) == 0


def test_backward_rejects_unsupported_problems():
    f32 = dict(d_k=32, d_v=32, chunk_size=32, dtype_code=K.KDA_F32, seqlen=64, heads=2)
    assert call_bwd(shape(**dict(f32, dtype_code=5))) == 2                # unknown dtype
    assert call_bwd(shape(**dict(f32, d_k=128, d_v=128, chunk_size=48))) == 2   # not 16/32/64
    assert call_bwd(shape(**dict(f32, d_k=128, d_v=128, chunk_size=8))) == 2
    assert call_bwd(shape(**dict(f32, d_k=96, d_v=96, chunk_size=16))) == 2
    assert call_bwd(shape(**dict(f32, d_k=64, d_v=32, chunk_size=16))) == 2
    assert call_bwd(shape(**dict(f32, chunk_size=64))) == 2
    assert call_bwd(shape(**f32), dq=None) == 1
    assert call_bwd(shape(**f32), dq=ctypes.c_void_p(0x1000)) == \
        1   # aliases an input
    assert call_bwd(shape(**f32), ws=None) == 1
    assert call_bwd(shape(**f32), wsb=ctypes.c_size_t(16)) == \
        3


def test_backward_workspace_query():
    sh = shape(d_k=16, d_v=16, chunk_size=16, dtype_code=K.KDA_F32, seqlen=100, heads=3)
    # (T / C + N + 1) chunk slots per head, each with the chunk-start state and
    # the end-state gradient (d x d), Z, dZ, R, Kbar, Qbar (C x d), T, K~, H
    # (C x C) and e^{G_C} (d), fp32
    per_slot = lambda d, C: 2 * d * d + 5 * C * d + 3 * C * C + d  # noqa: E731
    slots = 100 // 16 + 1 + 1
    assert K.lib().kda_chunk_bwd_workspace_bytes(ctypes.byref(sh)) == slots * 3 * per_slot(16, 16) * 4
    sh = shape(d_k=128, d_v=128, chunk_size=16, dtype_code=K.KDA_F32, seqlen=4096, heads=2)
    assert K.lib().kda_chunk_bwd_workspace_bytes(ctypes.byref(sh)) == \
        (4096 // 16 + 2) * 2 * per_slot(128, 16) * 4


def test_noalloc_refuses_before_touching_the_gpu():
    """kda_chunk_fwd_noalloc validates like kda_chunk_fwd and refuses problems
    whose workspace exceeds its buffer before any HIP call."""
    lib = K.lib()
    P = ctypes.c_void_p(0x100000)
    O = ctypes.c_void_p(0x200000)
    f = ctypes.c_float(0.1)

    def call(sh, o=O):
        return lib.kda_chunk_fwd_noalloc(ctypes.byref(sh) if sh is not None else None, P, P, P,
                                         P, P, f, None, None, o, None, None)
    big = shape(seqlen=131072)
    assert ws(big) > (256 << 20)
    assert call(big) == 3
    assert b"kda_chunk_fwd with a workspace" in lib.kda_last_error()
    assert call(None) == 1
    assert call(shape(d_k=96, d_v=96)) == 2
    assert call(shape(), o=P) == 1                     # o aliases an input


@pytest.mark.parametrize("hip_first", [True, False])
def test_header_compiles_as_c_next_to_the_hip_headers(tmp_path, hip_first):
    """kda.h is plain C99, and a hipStream_t passes as its stream argument
    whichever header is included first."""
    if not os.path.exists("/opt/rocm/include/hip/hip_runtime_api.h"):
        pytest.skip("HIP headers not available")
    inc = ['#include <hip/hip_runtime_api.h>', '#include "kda.h"']
    src = "\n".join(inc if hip_first else inc[::-1]) + """
kda_status f(hipStream_t s) {
    return kda_decode_step(1, 1, 128, 128, KDA_BF16, 0, 0, 0, 0, 0, 1.f, 0, 0, s);
}
"""
    c = tmp_path / "use.c"
    c.write_text(src)
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                        "-D__HIP_PLATFORM_AMD__", "-isystem", "/opt/rocm/include", "-I" + ROOT + "/include",
                        "-c", str(c), "-o", str(tmp_path / "use.o")], capture_output=True,
                       text=True)
    assert r.returncode == 0, r.stderr
