"""Kimi Delta Attention (KDA) forward pass on MI355X (gfx950).

A thin binding over the C ABI of ``libkda.so`` (declared in ``include/kda.h``).
Every step of the computation runs in the library's HIP kernels; this module
only checks shapes, allocates outputs and workspace with torch, and passes
device pointers and the current HIP stream.  There is no fallback: if the
library is missing or cannot be loaded, every call raises.

  chunk_fwd(q, k, v, g, beta, ...)      chunkwise prefill  -> (o, final_state)
  chunk_fwd_noalloc(...)                the same on the library's own device
                                        buffer (no workspace allocation)
  decode_step(q, k, v, g, beta, state)  one recurrent step -> o (state in place)
  chunk_fwd_scalar_gate, decode_step_scalar_gate
                                        the same with one log-decay per (token,
                                        head) shared by all key channels, or
                                        g=None for no decay
  chunk_fwd_ex, decode_step_ex          any gate layout, and the layer's last
                                        elementwise input steps (q/k L2 norm,
                                        logit gates, logit beta) done in-kernel
  output_rmsnorm_gate(o, gate, weight)  RMS norm x weight x sigmoid gate
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

__all__ = ["chunk_fwd", "chunk_fwd_noalloc", "decode_step", "chunk_fwd_scalar_gate", "decode_step_scalar_gate",
           "chunk_fwd_ex", "decode_step_ex", "output_rmsnorm_gate", "chunk_bwd", "workspace_bytes",
           "workspace_bytes_bwd", "lib", "KdaError", "LIB_PATH"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkda.so")

KDA_F32, KDA_BF16 = 0, 1
STATUS = {0: "KDA_OK", 1: "KDA_ERR_INVALID_ARGUMENT", 2: "KDA_ERR_UNSUPPORTED",
          3: "KDA_ERR_WORKSPACE_TOO_SMALL", 4: "KDA_ERR_HIP"}


class KdaError(RuntimeError):
    """A non-OK status from the C ABI."""

    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (STATUS.get(status, status), message))
        self.status = status


class KdaShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seqlen", ctypes.c_int32),
                ("num_heads", ctypes.c_int32), ("d_k", ctypes.c_int32),
                ("d_v", ctypes.c_int32), ("chunk_size", ctypes.c_int32),
                ("num_seqs", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class KdaInputsForm(ctypes.Structure):
    _fields_ = [("gate_layout", ctypes.c_int32), ("gate_is_logit", ctypes.c_int32),
                ("beta_is_logit", ctypes.c_int32), ("l2norm_qk", ctypes.c_int32),
                ("eps", ctypes.c_float)]


GATE_LAYOUTS = {"per_channel": 0, "scalar": 1, "none": 2}

_lib = None


def lib():
    """The loaded ``libkda.so`` (ctypes), with argument types declared."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libkda.so is not built (%s); run __graft_entry__.build() or "
                          "python gated_delta_rule_80_amd/build.py" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    vp, fp, ip = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
    L.kda_abi_version.restype = ctypes.c_int
    L.kda_abi_version.argtypes = []
    L.kda_set_prefill_overlap.restype = ctypes.c_int
    L.kda_set_prefill_overlap.argtypes = [ctypes.c_int]
    L.kda_status_string.restype = ctypes.c_char_p
    L.kda_status_string.argtypes = [ctypes.c_int]
    L.kda_last_error.restype = ctypes.c_char_p
    L.kda_last_error.argtypes = []
    L.kda_chunk_fwd_workspace_bytes.restype = ctypes.c_size_t
    L.kda_chunk_fwd_workspace_bytes.argtypes = [ctypes.POINTER(KdaShape)]
    L.kda_chunk_fwd.restype = ctypes.c_int
    L.kda_chunk_fwd.argtypes = [ctypes.POINTER(KdaShape), vp, vp, vp, fp, fp, ctypes.c_float,
                                fp, ip, vp, fp, vp, ctypes.c_size_t, vp]
    L.kda_chunk_fwd_noalloc.restype = ctypes.c_int
    L.kda_chunk_fwd_noalloc.argtypes = [ctypes.POINTER(KdaShape), vp, vp, vp, fp, fp,
                                        ctypes.c_float, fp, ip, vp, fp, vp]
    L.kda_chunk_fwd_scalar_gate.restype = ctypes.c_int
    L.kda_chunk_fwd_scalar_gate.argtypes = L.kda_chunk_fwd.argtypes
    L.kda_decode_step.restype = ctypes.c_int
    L.kda_decode_step.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                  ctypes.c_int32, ctypes.c_int, vp, vp, vp, fp, fp,
                                  ctypes.c_float, fp, vp, vp]
    L.kda_decode_step_scalar_gate.restype = ctypes.c_int
    L.kda_decode_step_scalar_gate.argtypes = L.kda_decode_step.argtypes
    L.kda_chunk_fwd_ex.restype = ctypes.c_int
    L.kda_chunk_fwd_ex.argtypes = [ctypes.POINTER(KdaShape), ctypes.POINTER(KdaInputsForm), vp, vp,
                                   vp, fp, fp, ctypes.c_float, fp, ip, vp, fp, vp, ctypes.c_size_t,
                                   vp]
    L.kda_decode_step_ex.restype = ctypes.c_int
    L.kda_decode_step_ex.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_int32, ctypes.c_int, ctypes.POINTER(KdaInputsForm),
                                     vp, vp, vp, fp, fp, ctypes.c_float, fp, vp, vp]
    L.kda_chunk_bwd_workspace_bytes.restype = ctypes.c_size_t
    L.kda_chunk_bwd_workspace_bytes.argtypes = [ctypes.POINTER(KdaShape)]
    L.kda_chunk_bwd.restype = ctypes.c_int
    L.kda_chunk_bwd.argtypes = [ctypes.POINTER(KdaShape), fp, fp, fp, fp, fp, ctypes.c_float, fp,
                                ip, fp, fp, fp, fp, fp, fp, fp, fp, vp, ctypes.c_size_t, vp]
    L.kda_output_rmsnorm_gate.restype = ctypes.c_int
    L.kda_output_rmsnorm_gate.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int, vp, vp, fp,
                                          ctypes.c_float, vp, vp]
    _lib = L
    return L


def _check(status: int):
    if status != 0:
        raise KdaError(status, lib().kda_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError("q, k, v must be bfloat16 or float32, got %s" % t.dtype)


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _on_device(ref: torch.Tensor, **tensors):
    """Every given tensor lives on ref's device, which is the current one (the
    library launches on the current device's current stream)."""
    _need(ref.is_cuda, "tensors must be on a HIP device")
    _need(ref.device.index == torch.cuda.current_device(),
          "tensors are on %s but the current device is %d" % (ref.device,
                                                               torch.cuda.current_device()))
    for name, t in tensors.items():
        _need(t is None or t.device == ref.device, "%s must be on %s" % (name, ref.device))


def _check_out(name: str, t: Optional[torch.Tensor], shape, dtype):
    """A caller-supplied output buffer must be exactly what the kernels write."""
    _need(t is None or (tuple(t.shape) == tuple(shape) and t.dtype == dtype and t.is_cuda
                        and t.is_contiguous()),
          "%s must be a contiguous %s device tensor %s" % (name, dtype, list(shape)))


def _check_workspace(t: Optional[torch.Tensor]):
    _need(t is None or (t.dtype == torch.uint8 and t.dim() == 1 and t.is_cuda
                        and t.is_contiguous()),
          "workspace must be a contiguous 1-D uint8 device tensor")


def make_shape(batch, seqlen, heads, d_k, d_v, chunk_size, num_seqs, dtype_code) -> KdaShape:
    return KdaShape(batch, seqlen, heads, d_k, d_v, chunk_size, num_seqs, dtype_code)


def workspace_bytes(batch, seqlen, heads, d_k, d_v, chunk_size, num_seqs,
                    dtype=torch.bfloat16) -> int:
    """Workspace kda_chunk_fwd needs for this problem (0 if unsupported)."""
    code = KDA_BF16 if dtype == torch.bfloat16 else KDA_F32
    sh = make_shape(batch, seqlen, heads, d_k, d_v, chunk_size, num_seqs, code)
    return int(lib().kda_chunk_fwd_workspace_bytes(ctypes.byref(sh)))


def workspace_bytes_bwd(batch, seqlen, heads, d, chunk_size, num_seqs,
                        dtype=torch.float32) -> int:
    """Workspace kda_chunk_bwd needs for this problem (0 if unsupported)."""
    code = KDA_BF16 if dtype == torch.bfloat16 else KDA_F32
    sh = make_shape(batch, seqlen, heads, d, d, chunk_size, num_seqs, code)
    return int(lib().kda_chunk_bwd_workspace_bytes(ctypes.byref(sh)))


def _prefill(entry, gate, q, k, v, g, beta, scale, initial_state, cu_seqlens,
             chunk_size, output_final_state, workspace, out, final_state, form=None,
             noalloc=False):
    _need(q.dim() == 4 and k.shape == q.shape and v.dim() == 4 and v.shape[:3] == q.shape[:3],
          "q, k must be [B, T, H, d_k] and v [B, T, H, d_v]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if gate == "scalar":
        _need(g is None or (g.shape == (B, T, H) and g.dtype == torch.float32),
              "g must be fp32 [B, T, H] or None")
    elif gate == "none":
        _need(g is None, "g must be None without a gate")
    else:
        _need(g is not None and g.shape == q.shape and g.dtype == torch.float32,
              "g must be fp32 [B, T, H, d_k]")
    _need(beta.shape == (B, T, H) and beta.dtype == torch.float32, "beta must be fp32 [B, T, H]")
    _need(q.dtype == k.dtype == v.dtype, "q, k, v must share one dtype")
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta)):
        _need(t is None or (t.is_cuda and t.is_contiguous()),
              "%s must be a contiguous device tensor" % name)
    code = _dtype_code(q)
    if cu_seqlens is not None:
        _need(cu_seqlens.dtype == torch.int32 and cu_seqlens.is_cuda and cu_seqlens.dim() == 1,
              "cu_seqlens must be an int32 device tensor [N+1]")
        _need(B == 1, "cu_seqlens needs batch 1")
        N = cu_seqlens.numel() - 1
    else:
        N = B
    if initial_state is not None:
        _need(initial_state.shape == (N, H, dk, dv) and initial_state.dtype == torch.float32
              and initial_state.is_cuda and initial_state.is_contiguous(),
              "initial_state must be a contiguous fp32 device tensor [N, H, d_k, d_v]")
    _check_out("out", out, (B, T, H, dv), q.dtype)
    _check_out("final_state", final_state, (N, H, dk, dv), torch.float32)
    _check_workspace(workspace)
    _on_device(q, k=k, v=v, g=g, beta=beta, initial_state=initial_state, cu_seqlens=cu_seqlens,
               out=out, final_state=final_state, workspace=workspace)
    scale = 1.0 / math.sqrt(dk) if scale is None else float(scale)
    sh = make_shape(B, T, H, dk, dv, chunk_size, N, code)
    if not noalloc:
        need = int(lib().kda_chunk_fwd_workspace_bytes(ctypes.byref(sh)))
        if workspace is None or workspace.numel() < need:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    o = out if out is not None else torch.empty((B, T, H, dv), dtype=q.dtype, device=q.device)
    fs = None
    if output_final_state:
        fs = final_state if final_state is not None else torch.empty(
            (N, H, dk, dv), dtype=torch.float32, device=q.device)
    extra = () if form is None else (ctypes.byref(form),)
    ws_args = () if noalloc else (_ptr(workspace), ctypes.c_size_t(workspace.numel()))
    st = entry(ctypes.byref(sh), *extra, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
               ctypes.c_float(scale), _ptr(initial_state), _ptr(cu_seqlens), _ptr(o), _ptr(fs),
               *ws_args, _stream())
    _check(st)
    return o, fs


def set_prefill_overlap(mode: int) -> int:
    """Process-wide order of the bf16 prefill's two kernels
    (``kda_set_prefill_overlap``): 1 overlapped where it applies (the default),
    0 one after the other, 2 overlapped with every chunk's factors refused by
    the chain, 3 overlapped with chains that give up at once when their first
    chunks are not ready (2 and 3 make the repair pass run; for tests).
    Returns the previous mode."""
    prev = lib().kda_set_prefill_overlap(int(mode))
    if prev < 0:
        raise ValueError("unknown prefill order %r (0, 1, 2 or 3)" % (mode,))
    return prev


def chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
              beta: torch.Tensor, scale: Optional[float] = None,
              initial_state: Optional[torch.Tensor] = None,
              cu_seqlens: Optional[torch.Tensor] = None, chunk_size: int = 64,
              output_final_state: bool = True, workspace: Optional[torch.Tensor] = None,
              out: Optional[torch.Tensor] = None, final_state: Optional[torch.Tensor] = None
              ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunkwise KDA prefill (``kda_chunk_fwd``).

    q, k: [B, T, H, d_k]; v: [B, T, H, d_v] (bf16 or fp32, same dtype);
    g: [B, T, H, d_k] fp32 per-token log-decay; beta: [B, T, H] fp32;
    initial_state: [N, H, d_k, d_v] fp32 or None; cu_seqlens: [N+1] int32 on
    the device (then B == 1) or None.  Returns (o [B, T, H, d_v], final_state
    [N, H, d_k, d_v] fp32 or None).
    """
    return _prefill(lib().kda_chunk_fwd, "per_channel", q, k, v, g, beta, scale, initial_state,
                    cu_seqlens, chunk_size, output_final_state, workspace, out, final_state)


def chunk_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                      beta: torch.Tensor, scale: Optional[float] = None,
                      initial_state: Optional[torch.Tensor] = None,
                      cu_seqlens: Optional[torch.Tensor] = None, chunk_size: int = 64,
                      output_final_state: bool = True, out: Optional[torch.Tensor] = None,
                      final_state: Optional[torch.Tensor] = None
                      ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """``chunk_fwd`` through ``kda_chunk_fwd_noalloc``: the library's own
    device buffer (``KDA_NOALLOC_SCRATCH_BYTES`` per device) is the workspace,
    so the call allocates no device memory when ``out`` (and ``final_state``,
    if wanted) are given.  Problems whose workspace would exceed that buffer
    raise ``KdaError`` (KDA_ERR_WORKSPACE_TOO_SMALL)."""
    return _prefill(lib().kda_chunk_fwd_noalloc, "per_channel", q, k, v, g, beta, scale,
                    initial_state, cu_seqlens, chunk_size, output_final_state, None, out,
                    final_state, noalloc=True)


def chunk_fwd_scalar_gate(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                          g: Optional[torch.Tensor], beta: torch.Tensor,
                          scale: Optional[float] = None,
                          initial_state: Optional[torch.Tensor] = None,
                          cu_seqlens: Optional[torch.Tensor] = None, chunk_size: int = 64,
                          output_final_state: bool = True,
                          workspace: Optional[torch.Tensor] = None,
                          out: Optional[torch.Tensor] = None,
                          final_state: Optional[torch.Tensor] = None
                          ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunkwise prefill with a scalar gate (``kda_chunk_fwd_scalar_gate``):
    g is [B, T, H] fp32, one log-decay per (token, head) for all key channels,
    or None for no decay.  Everything else as ``chunk_fwd``."""
    return _prefill(lib().kda_chunk_fwd_scalar_gate, "scalar", q, k, v, g, beta, scale,
                    initial_state, cu_seqlens, chunk_size, output_final_state, workspace, out,
                    final_state)


def _form(gate, gate_is_logit, beta_is_logit, l2norm_qk, eps):
    _need(gate in GATE_LAYOUTS, "gate must be one of %s" % sorted(GATE_LAYOUTS))
    return KdaInputsForm(GATE_LAYOUTS[gate], int(bool(gate_is_logit)), int(bool(beta_is_logit)),
                         int(bool(l2norm_qk)), float(eps))


def chunk_fwd_ex(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: Optional[torch.Tensor],
                 beta: torch.Tensor, *, gate: str = "per_channel", gate_is_logit: bool = False,
                 beta_is_logit: bool = False, l2norm_qk: bool = False, eps: float = 1e-6,
                 scale: Optional[float] = None, initial_state: Optional[torch.Tensor] = None,
                 cu_seqlens: Optional[torch.Tensor] = None, chunk_size: int = 64,
                 output_final_state: bool = True, workspace: Optional[torch.Tensor] = None,
                 out: Optional[torch.Tensor] = None, final_state: Optional[torch.Tensor] = None
                 ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunkwise prefill with the inputs in a stated form (``kda_chunk_fwd_ex``).

    gate: "per_channel" (g [B, T, H, d_k]), "scalar" (g [B, T, H]) or "none"
    (g None).  gate_is_logit: g holds logits x and log a = log sigmoid(x).
    beta_is_logit: beta = sigmoid(beta).  l2norm_qk: q and k are divided by
    sqrt(sum of squares + eps) per (token, head) inside the kernel.
    """
    f = _form(gate, gate_is_logit, beta_is_logit, l2norm_qk, eps)
    return _prefill(lib().kda_chunk_fwd_ex, gate, q, k, v, g, beta, scale, initial_state,
                    cu_seqlens, chunk_size, output_final_state, workspace, out, final_state,
                    form=f)


def _decode(entry, gate, q, k, v, g, beta, state, scale, out, form=None):
    _need(q.dim() == 3 and k.shape == q.shape and v.dim() == 3 and v.shape[:2] == q.shape[:2],
          "q, k must be [N, H, d_k] and v [N, H, d_v]")
    N, H, dk = q.shape
    dv = v.shape[-1]
    if gate == "scalar":
        _need(g is None or (g.shape == (N, H) and g.dtype == torch.float32),
              "g must be fp32 [N, H] or None")
    elif gate == "none":
        _need(g is None, "g must be None without a gate")
    else:
        _need(g is not None and g.shape == q.shape and g.dtype == torch.float32,
              "g must be fp32 [N, H, d_k]")
    _need(beta.shape == (N, H) and beta.dtype == torch.float32, "beta must be fp32 [N, H]")
    _need(state.shape == (N, H, dk, dv) and state.dtype == torch.float32,
          "state must be fp32 [N, H, d_k, d_v]")
    _need(q.dtype == k.dtype == v.dtype, "q, k, v must share one dtype")
    for name, t in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta), ("state", state)):
        _need(t is None or (t.is_cuda and t.is_contiguous()),
              "%s must be a contiguous device tensor" % name)
    code = _dtype_code(q)
    _check_out("out", out, (N, H, dv), q.dtype)
    _on_device(q, k=k, v=v, g=g, beta=beta, state=state, out=out)
    scale = 1.0 / math.sqrt(dk) if scale is None else float(scale)
    o = out if out is not None else torch.empty((N, H, dv), dtype=q.dtype, device=q.device)
    extra = () if form is None else (ctypes.byref(form),)
    st = entry(N, H, dk, dv, code, *extra, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
               ctypes.c_float(scale), _ptr(state), _ptr(o), _stream())
    _check(st)
    return o


def decode_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                beta: torch.Tensor, state: torch.Tensor, scale: Optional[float] = None,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One recurrent KDA step (``kda_decode_step``); ``state`` [N, H, d_k, d_v]
    fp32 is updated in place.

    q, k: [N, H, d_k]; v: [N, H, d_v] (bf16 or fp32); g: [N, H, d_k] fp32;
    beta: [N, H] fp32.  Returns o [N, H, d_v] in the dtype of v.
    """
    return _decode(lib().kda_decode_step, "per_channel", q, k, v, g, beta, state, scale, out)


def decode_step_scalar_gate(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                            g: Optional[torch.Tensor], beta: torch.Tensor, state: torch.Tensor,
                            scale: Optional[float] = None,
                            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One recurrent step with a scalar gate (``kda_decode_step_scalar_gate``):
    g is [N, H] fp32 or None for no decay.  Everything else as ``decode_step``."""
    return _decode(lib().kda_decode_step_scalar_gate, "scalar", q, k, v, g, beta, state, scale,
                   out)


def decode_step_ex(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: Optional[torch.Tensor],
                   beta: torch.Tensor, state: torch.Tensor, *, gate: str = "per_channel",
                   gate_is_logit: bool = False, beta_is_logit: bool = False,
                   l2norm_qk: bool = False, eps: float = 1e-6, scale: Optional[float] = None,
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One recurrent step with the inputs in a stated form (``kda_decode_step_ex``);
    the form arguments are those of ``chunk_fwd_ex`` (g [N, H, d_k], [N, H] or None)."""
    f = _form(gate, gate_is_logit, beta_is_logit, l2norm_qk, eps)
    return _decode(lib().kda_decode_step_ex, gate, q, k, v, g, beta, state, scale, out, form=f)


def output_rmsnorm_gate(o: torch.Tensor, gate: torch.Tensor, weight: torch.Tensor,
                        eps: float = 1e-6, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out = o / sqrt(mean(o^2 over d_v) + eps) * weight * sigmoid(gate)
    (``kda_output_rmsnorm_gate``).  o, gate: [..., d_v] bf16 or fp32 (same);
    weight: [d_v] fp32.  ``out`` may be ``o`` (in place)."""
    _need(o.shape == gate.shape and o.dtype == gate.dtype, "o and gate must match")
    dv = o.shape[-1]
    _need(weight.shape == (dv,) and weight.dtype == torch.float32, "weight must be fp32 [d_v]")
    for name, t in (("o", o), ("gate", gate), ("weight", weight)):
        _need(t.is_cuda and t.is_contiguous(), "%s must be a contiguous device tensor" % name)
    code = _dtype_code(o)
    _check_out("out", out, o.shape, o.dtype)
    _on_device(o, gate=gate, weight=weight, out=out)
    res = out if out is not None else torch.empty_like(o)
    st = lib().kda_output_rmsnorm_gate(o.numel() // dv, dv, code, _ptr(o), _ptr(gate), _ptr(weight),
                                       ctypes.c_float(eps), _ptr(res), _stream())
    _check(st)
    return res


def chunk_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
              beta: torch.Tensor, d_o: torch.Tensor, scale: Optional[float] = None,
              initial_state: Optional[torch.Tensor] = None,
              cu_seqlens: Optional[torch.Tensor] = None,
              d_final_state: Optional[torch.Tensor] = None, chunk_size: int = 32,
              workspace: Optional[torch.Tensor] = None) -> dict:
    """Gradients of ``chunk_fwd`` (``kda_chunk_bwd``) for L = <o, d_o> +
    <final states, d_final_state>: a dict with dq, dk, dv, dg, dbeta and, when
    an initial state is given, dinitial_state.  q, k, v and d_o in fp32 or
    bf16 (one dtype), g, beta and the states fp32; the gradients are fp32.
    d_k = d_v = d with (d, chunk_size) in {(16, 16|32|64), (32, 16|32),
    (64, 16|32), (128, 16|32|64)}; at d = 128 the gradients are formed over
    16-token chunks whatever chunk_size is (it changes only the rounding)."""
    _need(q.dim() == 4 and k.shape == q.shape and v.shape == q.shape and g.shape == q.shape,
          "q, k, v, g must be [B, T, H, d] (d_k = d_v)")
    B, T, H, d = q.shape
    _need(beta.shape == (B, T, H) and d_o.shape == q.shape, "beta must be [B, T, H], d_o like v")
    _need(q.dtype in (torch.float32, torch.bfloat16) and
          q.dtype == k.dtype == v.dtype == d_o.dtype, "q, k, v, d_o must share fp32 or bf16")
    for name, t in (("q", q), ("k", k), ("v", v), ("d_o", d_o)):
        _need(t.is_cuda and t.is_contiguous(), "%s must be a contiguous device tensor" % name)
    for name, t in (("g", g), ("beta", beta)):
        _need(t.dtype == torch.float32 and t.is_cuda and t.is_contiguous(),
              "%s must be a contiguous fp32 device tensor" % name)
    if cu_seqlens is not None:
        _need(cu_seqlens.dtype == torch.int32 and cu_seqlens.is_cuda and cu_seqlens.dim() == 1,
              "cu_seqlens must be an int32 device tensor [N+1]")
        _need(B == 1, "cu_seqlens needs batch 1")
        N = cu_seqlens.numel() - 1
    else:
        N = B
    for name, t in (("initial_state", initial_state), ("d_final_state", d_final_state)):
        _need(t is None or (t.shape == (N, H, d, d) and t.dtype == torch.float32 and t.is_cuda
                            and t.is_contiguous()),
              "%s must be a contiguous fp32 device tensor [N, H, d, d]" % name)
    _check_workspace(workspace)
    _on_device(q, k=k, v=v, g=g, beta=beta, d_o=d_o, initial_state=initial_state,
               cu_seqlens=cu_seqlens, d_final_state=d_final_state, workspace=workspace)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    sh = make_shape(B, T, H, d, d, chunk_size, N, _dtype_code(q))
    need = int(lib().kda_chunk_bwd_workspace_bytes(ctypes.byref(sh)))
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    out = {n: torch.empty(t.shape, dtype=torch.float32, device=q.device)
           for n, t in (("dq", q), ("dk", k), ("dv", v), ("dg", g), ("dbeta", beta))}
    ds0 = None
    if initial_state is not None:
        ds0 = torch.empty_like(initial_state)
        out["dinitial_state"] = ds0
    st = lib().kda_chunk_bwd(ctypes.byref(sh), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                             ctypes.c_float(scale), _ptr(initial_state), _ptr(cu_seqlens),
                             _ptr(d_o), _ptr(d_final_state), _ptr(out["dq"]), _ptr(out["dk"]),
                             _ptr(out["dv"]), _ptr(out["dg"]), _ptr(out["dbeta"]), _ptr(ds0),
                             _ptr(workspace), ctypes.c_size_t(workspace.numel()), _stream())
    _check(st)
    return out
