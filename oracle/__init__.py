"""fp64 CPU oracle of the gated delta rule -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It never imports the product package's
compute path (only its seeded input generator is shared, and that holds no
arithmetic of the method), and the product path never imports it.

Contents
  forward(...)      token-by-token recurrence in C (``gdn_oracle.c``), threaded
                    over independent (sequence, head) units: the gated delta
                    rule, its no-erase (Mamba2) form, each with a scalar or a
                    per-channel (vector) gate.
  wy_vectors(...)   the w recursion of the WY representation (numpy, tiny sizes).
  u_vectors(...)    the gated u recursion (numpy, tiny sizes).

Every function states the passage it follows; see each docstring.
Parity status: forward, wy_vectors and u_vectors are pinned by the CPU tests
(identities and closed forms of the pages, brute force on tiny inputs).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "libgdn_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (-O2, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _bind(path: str):
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.gdn_oracle_forward.argtypes = [P, P, P, P, P, P, P, I64, I64, I64, I64, I64, I64,
                                       P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.gdn_oracle_forward.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _lib = _bind(_LIB)
    return _lib



def default_threads() -> int:
    """Worker threads when none are asked for: GDN_ORACLE_THREADS if set, else
    min(cores, 16) -- the CPU share of one GPU on the measurement machines."""
    env = os.environ.get("GDN_ORACLE_THREADS")
    if env:
        return max(1, int(env))
    return max(1, min(os.cpu_count() or 1, 16))


def _f64(x) -> Optional[np.ndarray]:
    """Exact upcast of a CPU tensor / array (fp32 or bf16) to contiguous fp64."""
    if x is None:
        return None
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def forward(q, k, v, log_alpha, beta, S0=None, cu_seqlens=None, *,
            n_threads: int = 0, no_erase: bool = False, return_threads: bool = False,
            lib=None):
    """Run the gated delta rule token by token in fp64.

    Follows the Qiita Linear-Attention article, section "Gated-DeltaNet"
    (S_i = a_i S_{i-1}(I - b_i k_i k_i^T) + b_i v_i k_i^T, h_i = S_i q_i),
    token by token.  ``no_erase`` drops the prediction term (the same
    article's "Mamba2" update with a write strength).  A per-channel gate is
    selected by the shape of log_alpha, [B,T,H,Dk]: S~ = S diag(alpha_t) on
    the key side (the vector-gated GLA that LinearAttention系列解读(六),
    section 1, names), with or without the erase term.

    Shapes: q, k [B,T,H,Dk]; v [B,T,H,Dv]; log_alpha [B,T,H] (scalar gate)
    or [B,T,H,Dk] (per-channel gate) or None (alpha = 1); beta [B,T,H];
    S0 [N,H,Dv,Dk] or None; cu_seqlens [N+1] or None (then N = B).
    Returns (O [B,T,H,Dv], S_T [N,H,Dv,Dk]) as fp64 numpy arrays
    (and the thread count when ``return_threads``).
    ``lib`` substitutes another build of the same C source (the mutation
    tests use it to check that the pins reject planted mistakes).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    la, be, s0 = _f64(log_alpha), _f64(beta), _f64(S0)
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    assert k.shape == (B, T, H, Dk) and v.shape == (B, T, H, Dv)
    gate_vec = la is not None and la.ndim == 4
    assert be.shape == (B, T, H) and (la is None or la.shape in ((B, T, H), (B, T, H, Dk)))
    cu = None
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(
            cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens, dtype=np.int64))
        assert B == 1 and cu[0] == 0 and cu[-1] == T and np.all(np.diff(cu) >= 0)
        N = cu.size - 1
    else:
        N = B
    if s0 is not None:
        assert s0.shape == (N, H, Dv, Dk)
    O = np.zeros((B, T, H, Dv), dtype=np.float64)
    S_T = np.zeros((N, H, Dv, Dk), dtype=np.float64)
    if n_threads <= 0:
        n_threads = default_threads()
    rc = (lib or _load()).gdn_oracle_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(la), _ptr(be), _ptr(s0),
                                    _ptr(cu), N, B, T, H, Dk, Dv, _ptr(O), _ptr(S_T),
                                    int(n_threads), 1 if no_erase else 0, 1 if gate_vec else 0)
    if rc < 1:
        raise RuntimeError(f"gdn_oracle_forward failed with code {rc}")
    return (O, S_T, rc) if return_threads else (O, S_T)


def wy_vectors(K: np.ndarray, beta: np.ndarray) -> np.ndarray:
    """w vectors of the WY representation, by their defining recursion.

    Qiita Linear-Attention article, section "Gated-DeltaNet":
        w_1 = beta_1 k_1,   w_i = beta_i (k_i - sum_{t<i} (k_i^T k_t) w_t).
    K: [n, Dk] rows k_i; beta: [n].  Returns W: [n, Dk] rows w_i.
    Pure-Python loop: for tiny inputs only."""
    K = np.asarray(K, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    n = K.shape[0]
    W = np.zeros_like(K)
    for i in range(n):
        acc = K[i].copy()
        for t in range(i):
            acc -= (K[i] @ K[t]) * W[t]
        W[i] = beta[i] * acc
    return W


def u_vectors(K: np.ndarray, V: np.ndarray, beta: np.ndarray,
              log_alpha: Optional[np.ndarray]) -> np.ndarray:
    """u vectors of the gated WY form, by their defining recursion.

    Qiita Linear-Attention article, section "Gated-DeltaNet":
        u_1 = beta_1 v_1,
        u_i = beta_i (v_i - sum_{s<i} (gamma_i / gamma_s) (k_s^T k_i) u_s),
    with gamma_i = prod_{t<=i} alpha_t.  K: [n, Dk], V: [n, Dv], beta: [n],
    log_alpha: [n] or None (alpha = 1).  Returns U: [n, Dv] rows u_i."""
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    n = K.shape[0]
    la = np.zeros(n) if log_alpha is None else np.asarray(log_alpha, dtype=np.float64)
    lg = np.cumsum(la)                       # log gamma_i
    U = np.zeros_like(V)
    for i in range(n):
        acc = V[i].copy()
        for s in range(i):
            acc -= np.exp(lg[i] - lg[s]) * (K[s] @ K[i]) * U[s]
        U[i] = beta[i] * acc
    return U
