"""Thin ctypes binding of the C ABI in ``include/gdn.h`` (libgdn.so).

Argument marshalling only: every step of the computation runs in the gfx950
kernels of ``libgdn.so``.  PyTorch supplies device memory (tensors,
workspace) and the stream.  There is no fallback: if the library is not built,
or a tensor is not on a ROCm device, the call raises.

The Python functions carry the C names:
  gdn_chunk_fwd, gdn_chunk_fwd_profiled, gdn_chunk_fwd_noalloc, gdn_recurrent_step,
  gdn_chunk_fwd_workspace_bytes, gdn_chunk_fwd_supported, gdn_status_string,
  gdn_mamba2_chunk_fwd, gdn_gla_chunk_fwd, gdn_rule_chunk_fwd_profiled,
  gdn_rule_workspace_bytes, gdn_rule_supported, gdn_chunk_fwd_split, gdn_chunk_fwd_auto_span_chunks,
  gdn_chunk_fwd_split_workspace_bytes.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch  # imported before the library so that both share torch's HIP runtime

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_F32 = 0
GDN_BF16 = 1
GDN_RULE_DELTA = 0
GDN_RULE_MAMBA2 = 1
GDN_RULE_GLA = 2
_DT = {torch.float32: GDN_F32, torch.bfloat16: GDN_BF16}

_lib = None


class GdnError(RuntimeError):
    """A non-zero gdn_status returned by the library."""

    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: status {code} ({gdn_status_string(code)})")


def load_library() -> ctypes.CDLL:
    """Load libgdn.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run gated_delta_rule_16_amd.build.build() "
                           "(or __graft_entry__.build()) first")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.gdn_chunk_fwd_supported.argtypes = [I, I, I, I]
    lib.gdn_chunk_fwd_supported.restype = I
    lib.gdn_chunk_fwd_workspace_bytes.argtypes = [I, I, I, I, I, I, I, I]
    lib.gdn_chunk_fwd_workspace_bytes.restype = SZ
    lib.gdn_chunk_fwd.argtypes = [P, P, P, P, P, P, P, I, P, P, I, I, I, I, I, I, I, P, SZ, P]
    lib.gdn_chunk_fwd.restype = I
    lib.gdn_chunk_fwd_profiled.argtypes = lib.gdn_chunk_fwd.argtypes + [P]
    lib.gdn_chunk_fwd_profiled.restype = I
    lib.gdn_chunk_fwd_noalloc.argtypes = [P, P, P, P, P, P, P, I, P, P, I, I, I, I, I, I, I, P]
    lib.gdn_chunk_fwd_noalloc.restype = I
    lib.gdn_mamba2_chunk_fwd.argtypes = lib.gdn_chunk_fwd.argtypes
    lib.gdn_mamba2_chunk_fwd.restype = I
    lib.gdn_gla_chunk_fwd.argtypes = lib.gdn_chunk_fwd.argtypes
    lib.gdn_gla_chunk_fwd.restype = I
    lib.gdn_chunk_fwd_split_workspace_bytes.argtypes = [I, I, I, I, I, I, I, I]
    lib.gdn_chunk_fwd_split_workspace_bytes.restype = SZ
    lib.gdn_chunk_fwd_auto_span_chunks.argtypes = [I, I, I, I, I, I, I, I]
    lib.gdn_chunk_fwd_auto_span_chunks.restype = I
    lib.gdn_chunk_fwd_split.argtypes = [P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, P, SZ, P, P]
    lib.gdn_chunk_fwd_split.restype = I
    lib.gdn_rule_chunk_fwd_profiled.argtypes = [I] + lib.gdn_chunk_fwd.argtypes + [P]
    lib.gdn_rule_chunk_fwd_profiled.restype = I
    lib.gdn_rule_supported.argtypes = [I, I, I, I, I]
    lib.gdn_rule_supported.restype = I
    lib.gdn_rule_workspace_bytes.argtypes = [I, I, I, I, I, I, I, I, I]
    lib.gdn_rule_workspace_bytes.restype = SZ
    lib.gdn_recurrent_step.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, P]
    lib.gdn_recurrent_step.restype = I
    lib.gdn_status_string.argtypes = [I]
    lib.gdn_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def gdn_status_string(code: int) -> str:
    return load_library().gdn_status_string(int(code)).decode()


def gdn_chunk_fwd_supported(Dk: int, Dv: int, C: int, dtype: torch.dtype) -> bool:
    return bool(load_library().gdn_chunk_fwd_supported(Dk, Dv, C, _DT[dtype]))


def gdn_chunk_fwd_workspace_bytes(B: int, T: int, H: int, Dk: int, Dv: int, C: int,
                                  n_seqs: int, dtype: torch.dtype) -> int:
    return int(load_library().gdn_chunk_fwd_workspace_bytes(B, T, H, Dk, Dv, C, n_seqs,
                                                            _DT[dtype]))


def gdn_rule_supported(rule: int, Dk: int, Dv: int, C: int, dtype: torch.dtype) -> bool:
    return bool(load_library().gdn_rule_supported(rule, Dk, Dv, C, _DT[dtype]))


def gdn_rule_workspace_bytes(rule: int, B: int, T: int, H: int, Dk: int, Dv: int, C: int,
                             n_seqs: int, dtype: torch.dtype) -> int:
    return int(load_library().gdn_rule_workspace_bytes(rule, B, T, H, Dk, Dv, C, n_seqs,
                                                       _DT[dtype]))


def _ptr(t: Optional[torch.Tensor], name: str, device=None, dtype=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(device, stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _chunk_fwd(profiled: bool, q, k, v, log_alpha, beta, S0, cu_seqlens, chunk_size, O, S_T,
               output_final_state, workspace, stream, rule=GDN_RULE_DELTA):
    lib = load_library()
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError("q, k must be [B,T,H,Dk] and v [B,T,H,Dv]")
    B, T, H, Dk = q.shape
    Dv = v.shape[3]
    dev, dt = q.device, q.dtype
    if dt not in _DT:
        raise ValueError(f"unsupported dtype {dt}")
    n_seqs = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    N = B if cu_seqlens is None else n_seqs
    if beta is not None and beta.shape != (B, T, H):
        raise ValueError("beta must be [B,T,H]")
    la_shape = (B, T, H, Dk) if rule == GDN_RULE_GLA else (B, T, H)
    if log_alpha is not None and log_alpha.shape != la_shape:
        raise ValueError(f"log_alpha must be {list(la_shape)}")
    if S0 is not None and S0.shape != (N, H, Dv, Dk):
        raise ValueError("S0 must be [N,H,Dv,Dk]")
    if O is None:
        O = torch.empty(B, T, H, Dv, device=dev, dtype=dt)
    if S_T is None and output_final_state:
        S_T = torch.empty(N, H, Dv, Dk, device=dev, dtype=torch.float32)
    need = lib.gdn_rule_workspace_bytes(rule, B, T, H, Dk, Dv, chunk_size, n_seqs, _DT[dt])
    if workspace is None:
        workspace = torch.empty(max(int(need), 1), device=dev, dtype=torch.uint8)
    args = [
        _ptr(q, "q", dev, dt), _ptr(k, "k", dev, dt), _ptr(v, "v", dev, dt),
        _ptr(log_alpha, "log_alpha", dev, torch.float32), _ptr(beta, "beta", dev, torch.float32),
        _ptr(S0, "S0", dev, torch.float32), _ptr(cu_seqlens, "cu_seqlens", dev, torch.int32),
        n_seqs, _ptr(O, "O", dev, dt), _ptr(S_T, "S_T", dev, torch.float32),
        B, T, H, Dk, Dv, chunk_size, _DT[dt],
        _ptr(workspace, "workspace", dev), workspace.numel() * workspace.element_size(),
        _stream(dev, stream)]
    if profiled:
        ms = (ctypes.c_float * 4)()
        rc = lib.gdn_rule_chunk_fwd_profiled(rule, *args, ms)
        if rc != 0:
            raise GdnError(rc, "gdn_rule_chunk_fwd_profiled")
        return O, S_T, [float(x) for x in ms]
    fn, name = {GDN_RULE_DELTA: (lib.gdn_chunk_fwd, "gdn_chunk_fwd"),
                GDN_RULE_MAMBA2: (lib.gdn_mamba2_chunk_fwd, "gdn_mamba2_chunk_fwd"),
                GDN_RULE_GLA: (lib.gdn_gla_chunk_fwd, "gdn_gla_chunk_fwd")}[rule]
    rc = fn(*args)
    if rc != 0:
        raise GdnError(rc, name)
    return O, S_T


def gdn_chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                  log_alpha: Optional[torch.Tensor], beta: torch.Tensor,
                  S0: Optional[torch.Tensor] = None, cu_seqlens: Optional[torch.Tensor] = None,
                  *, chunk_size: int = 64, O: Optional[torch.Tensor] = None,
                  S_T: Optional[torch.Tensor] = None, output_final_state: bool = True,
                  workspace: Optional[torch.Tensor] = None,
                  stream: Optional[torch.cuda.Stream] = None
                  ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunkwise gated delta rule forward (see include/gdn.h, gdn_chunk_fwd).

    q, k [B,T,H,Dk]; v [B,T,H,Dv] (fp32 or bf16, same dtype); log_alpha (or
    None: alpha = 1) and beta [B,T,H] fp32; S0 [N,H,Dv,Dk] fp32 or None;
    cu_seqlens int32 [N+1] on the device for a packed batch (B = 1).
    Returns (O [B,T,H,Dv], S_T [N,H,Dv,Dk] or None).  Outputs and the
    workspace are allocated here unless passed in."""
    return _chunk_fwd(False, q, k, v, log_alpha, beta, S0, cu_seqlens, chunk_size, O, S_T,
                      output_final_state, workspace, stream)


def gdn_chunk_fwd_profiled(q, k, v, log_alpha, beta, S0=None, cu_seqlens=None, *,
                           chunk_size: int = 64, O=None, S_T=None, output_final_state=True,
                           workspace=None, stream=None):
    """As gdn_chunk_fwd, and also returns the device milliseconds of each
    kernel [table, prep, scan, output]; blocks until the call has finished."""
    return _chunk_fwd(True, q, k, v, log_alpha, beta, S0, cu_seqlens, chunk_size, O, S_T,
                      output_final_state, workspace, stream)


def gdn_mamba2_chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                         log_alpha: Optional[torch.Tensor], beta: Optional[torch.Tensor],
                         S0: Optional[torch.Tensor] = None,
                         cu_seqlens: Optional[torch.Tensor] = None, *, chunk_size: int = 64,
                         O: Optional[torch.Tensor] = None, S_T: Optional[torch.Tensor] = None,
                         output_final_state: bool = True,
                         workspace: Optional[torch.Tensor] = None,
                         stream: Optional[torch.cuda.Stream] = None
                         ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunked forward of S_t = alpha_t S_{t-1} + beta_t v_t k_t^T, o_t = S_t q_t
    (include/gdn.h, gdn_mamba2_chunk_fwd).  Arguments as gdn_chunk_fwd; beta may
    be None (beta = 1), and log_alpha None (alpha = 1) gives linear attention."""
    return _chunk_fwd(False, q, k, v, log_alpha, beta, S0, cu_seqlens, chunk_size, O, S_T,
                      output_final_state, workspace, stream, rule=GDN_RULE_MAMBA2)


def gdn_gla_chunk_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                      log_alpha: Optional[torch.Tensor], beta: Optional[torch.Tensor],
                      S0: Optional[torch.Tensor] = None,
                      cu_seqlens: Optional[torch.Tensor] = None, *, chunk_size: int = 64,
                      O: Optional[torch.Tensor] = None, S_T: Optional[torch.Tensor] = None,
                      output_final_state: bool = True,
                      workspace: Optional[torch.Tensor] = None,
                      stream: Optional[torch.cuda.Stream] = None
                      ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunked forward of S_t = S_{t-1} diag(alpha_t) + beta_t v_t k_t^T,
    o_t = S_t q_t with one gate per key channel (include/gdn.h,
    gdn_gla_chunk_fwd).  log_alpha [B,T,H,Dk] (each <= 0) or None; beta
    [B,T,H] or None (beta = 1); the rest as gdn_chunk_fwd."""
    return _chunk_fwd(False, q, k, v, log_alpha, beta, S0, cu_seqlens, chunk_size, O, S_T,
                      output_final_state, workspace, stream, rule=GDN_RULE_GLA)


def gdn_rule_chunk_fwd_profiled(rule: int, q, k, v, log_alpha, beta, S0=None, cu_seqlens=None,
                                *, chunk_size: int = 64, O=None, S_T=None,
                                output_final_state=True, workspace=None, stream=None):
    """The forward of ``rule`` (GDN_RULE_DELTA, GDN_RULE_MAMBA2 or GDN_RULE_GLA),
    also returning each kernel's device milliseconds [table, per-chunk
    preparation, scan, unused]."""
    return _chunk_fwd(True, q, k, v, log_alpha, beta, S0, cu_seqlens, chunk_size, O, S_T,
                      output_final_state, workspace, stream, rule=rule)


def gdn_chunk_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                          log_alpha: Optional[torch.Tensor], beta: torch.Tensor,
                          S0: Optional[torch.Tensor], cu_seqlens: Optional[torch.Tensor],
                          O: torch.Tensor, S_T: Optional[torch.Tensor], *, chunk_size: int = 64,
                          stream: Optional[torch.cuda.Stream] = None) -> None:
    """gdn_chunk_fwd on the library's static scratch buffer (include/gdn.h,
    gdn_chunk_fwd_noalloc): no workspace, and the caller passes the outputs
    O [B,T,H,Dv] and S_T [N,H,Dv,Dk] (or None), so that nothing is allocated."""
    lib = load_library()
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError("q, k must be [B,T,H,Dk] and v [B,T,H,Dv]")
    B, T, H, Dk = q.shape
    Dv = v.shape[3]
    dev, dt = q.device, q.dtype
    if dt not in _DT:
        raise ValueError(f"unsupported dtype {dt}")
    n_seqs = 0 if cu_seqlens is None else cu_seqlens.numel() - 1
    N = B if cu_seqlens is None else n_seqs
    for name, t in (("beta", beta), ("log_alpha", log_alpha)):
        if t is not None and t.shape != (B, T, H):
            raise ValueError(f"{name} must be [B,T,H]")
    if S0 is not None and S0.shape != (N, H, Dv, Dk):
        raise ValueError("S0 must be [N,H,Dv,Dk]")
    if O.shape != (B, T, H, Dv) or (S_T is not None and S_T.shape != (N, H, Dv, Dk)):
        raise ValueError("O must be [B,T,H,Dv] and S_T [N,H,Dv,Dk]")
    rc = lib.gdn_chunk_fwd_noalloc(
        _ptr(q, "q", dev, dt), _ptr(k, "k", dev, dt), _ptr(v, "v", dev, dt),
        _ptr(log_alpha, "log_alpha", dev, torch.float32), _ptr(beta, "beta", dev, torch.float32),
        _ptr(S0, "S0", dev, torch.float32), _ptr(cu_seqlens, "cu_seqlens", dev, torch.int32),
        n_seqs, _ptr(O, "O", dev, dt), _ptr(S_T, "S_T", dev, torch.float32),
        B, T, H, Dk, Dv, chunk_size, _DT[dt], _stream(dev, stream))
    if rc != 0:
        raise GdnError(rc, "gdn_chunk_fwd_noalloc")


def gdn_chunk_fwd_split_workspace_bytes(B: int, T: int, H: int, Dk: int, Dv: int, C: int,
                                        span_chunks: int, dtype: torch.dtype) -> int:
    return int(load_library().gdn_chunk_fwd_split_workspace_bytes(B, T, H, Dk, Dv, C, span_chunks,
                                                                  _DT[dtype]))


def gdn_chunk_fwd_auto_span_chunks(B: int, T: int, H: int, Dk: int, Dv: int, C: int,
                                   n_seqs: int, dtype: torch.dtype) -> int:
    """Span length gdn_chunk_fwd splits these sizes into on the current device,
    or 0 for the plain scan (include/gdn.h)."""
    return int(load_library().gdn_chunk_fwd_auto_span_chunks(B, T, H, Dk, Dv, C, n_seqs, _DT[dtype]))


def gdn_chunk_fwd_split(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                        log_alpha: Optional[torch.Tensor], beta: torch.Tensor,
                        S0: Optional[torch.Tensor] = None, *, span_chunks: int,
                        chunk_size: int = 64, O: Optional[torch.Tensor] = None,
                        S_T: Optional[torch.Tensor] = None, output_final_state: bool = True,
                        workspace: Optional[torch.Tensor] = None,
                        stream: Optional[torch.cuda.Stream] = None, profiled: bool = False):
    """gdn_chunk_fwd of a fixed-length batch with each sequence split into spans
    of ``span_chunks`` chunks (include/gdn.h, gdn_chunk_fwd_split).  Returns
    (O, S_T), and with ``profiled`` also the device milliseconds of
    [prep, pass 1, pass 2, pass 3] (the call then blocks)."""
    lib = load_library()
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError("q, k must be [B,T,H,Dk] and v [B,T,H,Dv]")
    B, T, H, Dk = q.shape
    Dv = v.shape[3]
    dev, dt = q.device, q.dtype
    if dt not in _DT:
        raise ValueError(f"unsupported dtype {dt}")
    for name, t in (("beta", beta), ("log_alpha", log_alpha)):
        if t is not None and t.shape != (B, T, H):
            raise ValueError(f"{name} must be [B,T,H]")
    if S0 is not None and S0.shape != (B, H, Dv, Dk):
        raise ValueError("S0 must be [B,H,Dv,Dk]")
    if O is None:
        O = torch.empty(B, T, H, Dv, device=dev, dtype=dt)
    if S_T is None and output_final_state:
        S_T = torch.empty(B, H, Dv, Dk, device=dev, dtype=torch.float32)
    need = lib.gdn_chunk_fwd_split_workspace_bytes(B, T, H, Dk, Dv, chunk_size, span_chunks, _DT[dt])
    if workspace is None:
        workspace = torch.empty(max(int(need), 1), device=dev, dtype=torch.uint8)
    ms = (ctypes.c_float * 4)() if profiled else None
    rc = lib.gdn_chunk_fwd_split(
        _ptr(q, "q", dev, dt), _ptr(k, "k", dev, dt), _ptr(v, "v", dev, dt),
        _ptr(log_alpha, "log_alpha", dev, torch.float32), _ptr(beta, "beta", dev, torch.float32),
        _ptr(S0, "S0", dev, torch.float32), _ptr(O, "O", dev, dt), _ptr(S_T, "S_T", dev, torch.float32),
        B, T, H, Dk, Dv, chunk_size, _DT[dt], span_chunks,
        _ptr(workspace, "workspace", dev), workspace.numel() * workspace.element_size(),
        _stream(dev, stream), ms)
    if rc != 0:
        raise GdnError(rc, "gdn_chunk_fwd_split")
    if profiled:
        return O, S_T, [float(x) for x in ms]
    return O, S_T


def gdn_recurrent_step(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                       log_alpha: Optional[torch.Tensor], beta: torch.Tensor, S: torch.Tensor,
                       *, o: Optional[torch.Tensor] = None,
                       stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """One token per sequence; S [N,H,Dv,Dk] fp32 is updated in place.
    q, k [N,H,Dk]; v [N,H,Dv]; log_alpha (or None), beta [N,H].  Returns o [N,H,Dv]."""
    lib = load_library()
    N, H, Dk = q.shape
    Dv = v.shape[2]
    dev, dt = q.device, q.dtype
    if dt not in _DT:
        raise ValueError(f"unsupported dtype {dt}")
    if S.shape != (N, H, Dv, Dk):
        raise ValueError("S must be [N,H,Dv,Dk]")
    if o is None:
        o = torch.empty(N, H, Dv, device=dev, dtype=dt)
    rc = lib.gdn_recurrent_step(
        _ptr(q, "q", dev, dt), _ptr(k, "k", dev, dt), _ptr(v, "v", dev, dt),
        _ptr(log_alpha, "log_alpha", dev, torch.float32), _ptr(beta, "beta", dev, torch.float32),
        _ptr(S, "S", dev, torch.float32), _ptr(o, "o", dev, dt), N, H, Dk, Dv, _DT[dt],
        _stream(dev, stream))
    if rc != 0:
        raise GdnError(rc, "gdn_recurrent_step")
    return o
