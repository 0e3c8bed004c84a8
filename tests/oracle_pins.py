"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each ``pin_*`` function takes the oracle's entry points as arguments and
raises AssertionError when a pinned property fails, so that the same pins
run both on the real oracle (tests/test_oracle_pins.py) and on builds with a
planted mistake (tests/test_oracle_mutants.py), where at least one must fail.

The closed forms here are written in the Qiita article's own column notation
(vectors are columns; K = [k_1 .. k_L] is Dk x L; H = [h_1 .. h_L]), not in
the row form the GPU kernels use, and they are evaluated with numpy dense
algebra (matrix products, explicit inverses, brute-force products).

Sources (cited by page title and section):
  [Q]  Qiita article by Nyysyyan on the Linear Attention lineage
       (sections "Linear attention", "Mamba2", "Gated-DeltaNet").
  [K]  kkkzoz blog post "linear-attention" (sections "Gated DeltaNet", "Workflow").
  [M]  LinearAttention系列解读(六)：DeltaNet的Chunkwise Form推导 (sections 1, 3 and 4).
"""
from __future__ import annotations

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

EXACT = 0.0          # bitwise equality
TIGHT = 1e-12        # fp64 closed forms vs the token loop, relative to max |ref|


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    scale = max(np.abs(b).max(), 1e-300)
    err = np.abs(a - b).max() / scale
    assert err <= tol, f"{what}: rel err {err:.3e} > {tol:.1e}"


def _orthonormal(rng, d, n):
    """n orthonormal vectors in R^d, as rows [n, d]."""
    qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    return qm[:, :n].T.copy()


def _one_unit(q, k, v, la, be, s0=None):
    """Shape a single (sequence, head) unit as [1, L, 1, D] arrays."""
    L = q.shape[0]
    return (q.reshape(1, L, 1, -1), k.reshape(1, L, 1, -1), v.reshape(1, L, 1, -1),
            None if la is None else la.reshape(1, L, 1), be.reshape(1, L, 1),
            None if s0 is None else s0.reshape(1, 1, *s0.shape))


def _run(forward, q, k, v, la, be, s0=None, **kw):
    O, S = forward(*_one_unit(q, k, v, la, be, s0), **kw)
    return O[0, :, 0, :], S[0, 0]


# ----------------------------------------------------------------------------
# Hand-worked example (tests/golden/gdn_2x2_worked.txt)
# ----------------------------------------------------------------------------
def load_golden(name="gdn_2x2_worked.txt"):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, rest = line.split(":", 1)
            vals[key.strip()] = np.array([float(x) for x in rest.split()])
    return vals


def pin_golden(forward, **_):
    """Worked example by hand from the update of [Q] "Gated-DeltaNet" in the
    step order of [K] "Workflow"; exact dyadic values."""
    g = load_golden()
    L, D = 3, 2
    q, k, v = g["q"].reshape(L, D), g["k"].reshape(L, D), g["v"].reshape(L, D)
    la, be, s0 = np.log(g["alpha"]), g["beta"], g["S0"].reshape(D, D)
    O, S = _run(forward, q, k, v, la, be, s0)
    _close(O, g["O"].reshape(L, D), 1e-15, "golden O")
    _close(S, g["S_T"].reshape(D, D), 1e-15, "golden S_T")
    _, S2 = _run(forward, q[:2], k[:2], v[:2], la[:2], be[:2], s0)
    _close(S2 @ k[1], g["S2_k2"], 1e-15, "golden S2 k2")


# ----------------------------------------------------------------------------
# P-1: alpha = 1, beta = 0 leaves the state unchanged ([Q] "Gated-DeltaNet").
# ----------------------------------------------------------------------------
def pin_identity_step(forward, rng=None, **_):
    rng = rng or np.random.default_rng(11)
    L, Dk, Dv = 9, 5, 4
    q, k, v = rng.standard_normal((L, Dk)), rng.standard_normal((L, Dk)), rng.standard_normal((L, Dv))
    s0 = rng.standard_normal((Dv, Dk))
    O, S = _run(forward, q, k, v, None, np.zeros(L), s0)
    assert np.array_equal(S, s0), "alpha=1, beta=0 changed the state"
    _close(O, q @ s0.T, 1e-15, "alpha=1, beta=0 output = S0 q")


# ----------------------------------------------------------------------------
# Retrieval identity of [Q] "Gated-DeltaNet" (stated for alpha = 1):
#   S_i k_i = (1 - beta_i |k_i|^2) S_{i-1} k_i + beta_i |k_i|^2 v_i,
# and its gated form, which follows from the same update by applying it to k_i:
#   S_i k_i = alpha_i (1 - beta_i |k_i|^2) S_{i-1} k_i + beta_i |k_i|^2 v_i.
# ----------------------------------------------------------------------------
def pin_retrieval_identity(forward, rng=None, **_):
    rng = rng or np.random.default_rng(12)
    L, Dk, Dv = 6, 4, 3
    q, k, v = rng.standard_normal((L, Dk)), 0.7 * rng.standard_normal((L, Dk)), rng.standard_normal((L, Dv))
    be = rng.uniform(0.1, 0.9, L)
    s0 = rng.standard_normal((Dv, Dk))
    for gated in (False, True):
        la = -rng.uniform(0.05, 1.0, L) if gated else None
        prev = s0
        for i in range(L):
            _, Si = _run(forward, q[:i + 1], k[:i + 1], v[:i + 1],
                         None if la is None else la[:i + 1], be[:i + 1], s0)
            a = 1.0 if la is None else np.exp(la[i])
            n2 = k[i] @ k[i]
            want = a * (1 - be[i] * n2) * (prev @ k[i]) + be[i] * n2 * v[i]
            _close(Si @ k[i], want, TIGHT, f"retrieval identity token {i} gated={gated}")
            prev = Si


# ----------------------------------------------------------------------------
# Mamba2 closed form of [Q] "Mamba2":  gamma_i = prod_{t<=i} alpha_t,
#   S_i = gamma_i S0 + sum_{s<=i} (gamma_i/gamma_s) v_s k_s^T   (write strength beta_s here)
#   H   = S0 Q D_gamma + V D_beta (Gamma o K^T Q),  Gamma_ij = gamma_j/gamma_i (i <= j).
# ----------------------------------------------------------------------------
def _mamba2_closed_form(Qc, Kc, Vc, be, la, s0):
    L = Qc.shape[1]
    gam = np.exp(np.cumsum(la))
    Gam = np.triu(gam[None, :] / gam[:, None])           # Gamma_ij = gamma_j / gamma_i, i <= j
    H = s0 @ Qc @ np.diag(gam) + (Vc @ np.diag(be)) @ (Gam * (Kc.T @ Qc))
    S = gam[-1] * s0 + sum((gam[-1] / gam[s]) * be[s] * np.outer(Vc[:, s], Kc[:, s]) for s in range(L))
    return H, S


def pin_mamba2_no_erase(forward, rng=None, **_):
    """(a) The test-only no-erase switch (prediction term dropped) gives the
    Mamba2 closed form on random gated inputs."""
    rng = rng or np.random.default_rng(13)
    L, Dk, Dv = 20, 6, 5
    q, k, v = rng.standard_normal((L, Dk)), rng.standard_normal((L, Dk)), rng.standard_normal((L, Dv))
    be, la = rng.uniform(0.1, 0.9, L), -rng.uniform(0.01, 0.5, L)
    s0 = rng.standard_normal((Dv, Dk))
    O, S = _run(forward, q, k, v, la, be, s0, no_erase=True)
    H, Sw = _mamba2_closed_form(q.T, k.T, v.T, be, la, s0)
    _close(O, H.T, TIGHT, "no-erase O vs Mamba2 closed form")
    _close(S, Sw, TIGHT, "no-erase S_T vs Mamba2 closed form")


def pin_mamba2_orthogonal_keys(forward, rng=None, **_):
    """(b) The unmodified recurrence reduces to the Mamba2 closed form when the
    keys are orthonormal and S0 annihilates every key: each prediction
    S~ k_i is then zero, so the delta term vanishes."""
    rng = rng or np.random.default_rng(14)
    L, Dk, Dv = 7, 10, 4
    k = _orthonormal(rng, Dk, L)
    q, v = rng.standard_normal((L, Dk)), rng.standard_normal((L, Dv))
    be, la = rng.uniform(0.1, 0.9, L), -rng.uniform(0.01, 0.5, L)
    s0 = rng.standard_normal((Dv, Dk)) @ (np.eye(Dk) - k.T @ k)
    O, S = _run(forward, q, k, v, la, be, s0)
    H, Sw = _mamba2_closed_form(q.T, k.T, v.T, be, la, s0)
    _close(O, H.T, TIGHT, "orthogonal-key O vs Mamba2 closed form")
    _close(S, Sw, TIGHT, "orthogonal-key S_T vs Mamba2 closed form")


# ----------------------------------------------------------------------------
# Exact retrieval ([Q] "Gated-DeltaNet", beta |k|^2 = 1 overwrites fully):
# orthonormal keys, beta = 1, alpha = 1, any S0  =>  S_T k_i = v_i;
# gated: later tokens with orthogonal keys only scale it, S_T k_i = (prod_{t>i} alpha_t) v_i.
# ----------------------------------------------------------------------------
def pin_exact_retrieval(forward, rng=None, **_):
    rng = rng or np.random.default_rng(15)
    L, Dk, Dv = 8, 8, 5
    k = _orthonormal(rng, Dk, L)
    q, v = rng.standard_normal((L, Dk)), rng.standard_normal((L, Dv))
    s0 = rng.standard_normal((Dv, Dk))
    _, S = _run(forward, q, k, v, None, np.ones(L), s0)
    _close(S @ k.T, v.T, TIGHT, "S_T k_i = v_i")
    la = -rng.uniform(0.01, 0.5, L)
    _, S = _run(forward, q, k, v, la, np.ones(L), s0)
    tail = np.exp(np.cumsum(la[::-1])[::-1] - la)        # prod_{t>i} alpha_t
    _close(S @ k.T, v.T * tail[None, :], TIGHT, "gated S_T k_i")


# ----------------------------------------------------------------------------
# P-4: WY identity of [Q] "Gated-DeltaNet":  I - sum_{t<=i} w_t k_t^T = A_1 ... A_i,
# A_t = I - beta_t k_t k_t^T, checked by brute-force matrix products.
# ----------------------------------------------------------------------------
def pin_wy_identity(wy_vectors, rng=None, **_):
    rng = rng or np.random.default_rng(16)
    n, Dk = 8, 5
    k, be = 0.8 * rng.standard_normal((n, Dk)), rng.uniform(0.1, 0.9, n)
    W = wy_vectors(k, be)
    P = np.eye(Dk)
    for i in range(n):
        P = P @ (np.eye(Dk) - be[i] * np.outer(k[i], k[i]))
        _close(np.eye(Dk) - W[:i + 1].T @ k[:i + 1], P, TIGHT, f"WY identity i={i + 1}")


# ----------------------------------------------------------------------------
# P-5: product form of [Q] "Gated-DeltaNet" with the w and u recursions:
#   S_i = gamma_i S0 (I - W_i K_i^T) + sum_{s<=i} (gamma_i/gamma_s) u_s k_s^T
# against the token loop, at every prefix.
# ----------------------------------------------------------------------------
def pin_product_form(forward, wy_vectors, u_vectors, rng=None, **_):
    rng = rng or np.random.default_rng(17)
    L, Dk, Dv = 10, 6, 4
    q, k, v = rng.standard_normal((L, Dk)), 0.6 * rng.standard_normal((L, Dk)), rng.standard_normal((L, Dv))
    be, la = rng.uniform(0.1, 0.9, L), -rng.uniform(0.01, 0.5, L)
    s0 = rng.standard_normal((Dv, Dk))
    W, U = wy_vectors(k, be), u_vectors(k, v, be, la)
    lg = np.cumsum(la)
    for i in range(1, L + 1):
        _, S = _run(forward, q[:i], k[:i], v[:i], la[:i], be[:i], s0)
        G = sum(np.exp(lg[i - 1] - lg[s]) * np.outer(U[s], k[s]) for s in range(i))
        want = np.exp(lg[i - 1]) * s0 @ (np.eye(Dk) - W[:i].T @ k[:i]) + G
        _close(S, want, TIGHT, f"product form prefix {i}")


# ----------------------------------------------------------------------------
# P-6: full-sequence parallel form of [Q] "Gated-DeltaNet":
#   H = S0 (Q - W (M^T o K^T Q)) D_gamma + U (Gamma o K^T Q)
#   W = K D_beta (I + (M^u o K^T K) D_beta)^-1
#   U = V D_beta (I + (Gamma^u o K^T K) D_beta)^-1
# M^u and Gamma^u keep only the STRICTLY upper part (the recursions sum over
# s < i; the printed text calls Gamma o K^T K strictly upper although Gamma
# has a diagonal -- the strict reading is the one the recursion implies).
# The inverses are dense numpy inverses, not substitution.
# ----------------------------------------------------------------------------
def parallel_form(Qc, Kc, Vc, be, la, s0):
    L = Qc.shape[1]
    lg = np.cumsum(la)
    gam = np.exp(lg)
    Mu = np.triu(np.ones((L, L)), 1)
    M = np.tril(np.ones((L, L)))
    Gam = np.triu(np.exp(lg[None, :] - lg[:, None]))
    Db = np.diag(be)
    KK = Kc.T @ Kc
    W = Kc @ Db @ np.linalg.inv(np.eye(L) + (Mu * KK) @ Db)
    U = Vc @ Db @ np.linalg.inv(np.eye(L) + (Mu * Gam * KK) @ Db)
    KQ = Kc.T @ Qc
    return s0 @ (Qc - W @ (M.T * KQ)) @ np.diag(gam) + U @ (Gam * KQ)


def pin_parallel_form(forward, rng=None, **_):
    rng = rng or np.random.default_rng(18)
    for (L, Dk, Dv) in [(48, 8, 6), (64, 16, 16)]:
        q, k, v = rng.standard_normal((L, Dk)), rng.standard_normal((L, Dk)), rng.standard_normal((L, Dv))
        k /= np.linalg.norm(k, axis=1, keepdims=True)
        be, la = rng.uniform(0.05, 0.95, L), -rng.uniform(0.005, 0.2, L)
        s0 = rng.standard_normal((Dv, Dk))
        O, _ = _run(forward, q, k, v, la, be, s0)
        H = parallel_form(q.T, k.T, v.T, be, la, s0)
        _close(O, H.T, 1e-10, f"parallel form L={L}")


# ----------------------------------------------------------------------------
# P-7: linear attention of [Q] "Linear attention": with orthonormal keys,
# beta = 1, alpha = 1 and S0 = 0 every prediction is zero and
#   H = V (M^T o K^T Q).
# ----------------------------------------------------------------------------
def pin_linear_attention(forward, rng=None, **_):
    rng = rng or np.random.default_rng(19)
    L, Dk, Dv = 12, 16, 7
    k = _orthonormal(rng, Dk, L)
    q, v = rng.standard_normal((L, Dk)), rng.standard_normal((L, Dv))
    O, _ = _run(forward, q, k, v, None, np.ones(L), None)
    M = np.tril(np.ones((L, L)))
    H = v.T @ (M.T * (k @ q.T))
    _close(O, H.T, TIGHT, "linear attention")


# ----------------------------------------------------------------------------
# Structure: units are independent ([Q] "Gated-DeltaNet": each (sequence,
# head) carries its own state), rows of S evolve independently (feature
# permutation), the state is the resume point ([Q] "Chunk Computation": the
# next chunk starts from the previous chunk's last state), packed sequences
# equal separate calls, and the thread count does not change a bit.
# ----------------------------------------------------------------------------
def pin_structure(forward, rng=None, **_):
    rng = rng or np.random.default_rng(20)
    B, T, H, Dk, Dv = 2, 23, 3, 5, 4
    q, k, v = rng.standard_normal((B, T, H, Dk)), rng.standard_normal((B, T, H, Dk)), rng.standard_normal((B, T, H, Dv))
    be, la = rng.uniform(0.1, 0.9, (B, T, H)), -rng.uniform(0.01, 0.5, (B, T, H))
    s0 = rng.standard_normal((B, H, Dv, Dk))
    O, S = forward(q, k, v, la, be, s0)
    O1, S1 = forward(q, k, v, la, be, s0, n_threads=1)
    assert np.array_equal(O, O1) and np.array_equal(S, S1), "thread count changed the result"
    for b in range(B):
        for h in range(H):
            Ou, Su = forward(q[b:b + 1, :, h:h + 1], k[b:b + 1, :, h:h + 1], v[b:b + 1, :, h:h + 1],
                             la[b:b + 1, :, h:h + 1], be[b:b + 1, :, h:h + 1], s0[b:b + 1, h:h + 1])
            assert np.array_equal(Ou[0, :, 0], O[b, :, h]), "units not independent (O)"
            assert np.array_equal(Su[0, 0], S[b, h]), "units not independent (S)"
    perm = rng.permutation(Dv)
    Op, Sp = forward(q, k, v[..., perm], la, be, s0[:, :, perm, :])
    assert np.array_equal(Op, O[..., perm]) and np.array_equal(Sp, S[:, :, perm, :]), "Dv permutation"
    T1 = 9
    Oa, Sa = forward(q[:, :T1], k[:, :T1], v[:, :T1], la[:, :T1], be[:, :T1], s0)
    Ob, Sb = forward(q[:, T1:], k[:, T1:], v[:, T1:], la[:, T1:], be[:, T1:], Sa)
    assert np.array_equal(np.concatenate([Oa, Ob], 1), O) and np.array_equal(Sb, S), "resume"
    # packed: the two batch rows as two sequences of one packed row, plus an empty one
    cu = np.array([0, T, T, 2 * T], dtype=np.int64)
    cat = lambda x: np.concatenate([x[0:1], x[1:2]], axis=1)
    s0p = np.stack([s0[0], rng.standard_normal((H, Dv, Dk)), s0[1]])
    Op, Sp = forward(cat(q), cat(k), cat(v), cat(la), cat(be), s0p, cu)
    assert np.array_equal(Op[0, :T], O[0]) and np.array_equal(Op[0, T:], O[1]), "packed O"
    assert np.array_equal(Sp[0], S[0]) and np.array_equal(Sp[2], S[1]), "packed S_T"
    assert np.array_equal(Sp[1], s0p[1]), "empty sequence must return its S0"


# ----------------------------------------------------------------------------
# Per-channel (vector) gate: the gate of token t is D_t = diag(alpha_t) on the
# key side of the state, S~ = S D_t ([M] section 1: the vector-gated GLA's
# transition is a diagonal matrix that scales each state element on its own).
# log_alpha of shape [B,T,H,Dk] selects it.
# ----------------------------------------------------------------------------
def _run_vec(forward, q, k, v, la, be, s0=None, **kw):
    L = q.shape[0]
    O, S = forward(q.reshape(1, L, 1, -1), k.reshape(1, L, 1, -1), v.reshape(1, L, 1, -1),
                   la.reshape(1, L, 1, -1), be.reshape(1, L, 1),
                   None if s0 is None else s0.reshape(1, 1, *s0.shape), **kw)
    return O[0, :, 0, :], S[0, 0]


def pin_vector_gate_golden(forward, **_):
    """Hand-worked 3-token example with per-channel gates, with and without the
    erase term (tests/golden/gla_vector_gate_2x2_worked.txt); exact dyadic values."""
    g = load_golden("gla_vector_gate_2x2_worked.txt")
    L, D = 3, 2
    q, k, v = g["q"].reshape(L, D), g["k"].reshape(L, D), g["v"].reshape(L, D)
    la, be, s0 = np.log(g["alpha"]).reshape(L, D), g["beta"], g["S0"].reshape(D, D)
    for mode, no_erase in (("no_erase", True), ("erase", False)):
        O, S = _run_vec(forward, q, k, v, la, be, s0, no_erase=no_erase)
        _close(O, g[f"O_{mode}"].reshape(L, D), 1e-15, f"vector-gate golden O ({mode})")
        _close(S, g[f"S_T_{mode}"].reshape(D, D), 1e-15, f"vector-gate golden S_T ({mode})")


def pin_vector_gate_scalar_reduction(forward, rng=None, **_):
    """Every channel of alpha_t equal: the per-channel gate is the scalar gate,
    to the last bit (the same doubles multiply the same entries), in both modes."""
    rng = rng or np.random.default_rng(21)
    B, T, H, Dk, Dv = 2, 17, 2, 5, 3
    q, k, v = rng.standard_normal((B, T, H, Dk)), rng.standard_normal((B, T, H, Dk)), rng.standard_normal((B, T, H, Dv))
    be, la = rng.uniform(0.1, 0.9, (B, T, H)), -rng.uniform(0.01, 0.5, (B, T, H))
    s0 = rng.standard_normal((B, H, Dv, Dk))
    lav = np.repeat(la[..., None], Dk, axis=-1)
    for no_erase in (False, True):
        Os, Ss = forward(q, k, v, la, be, s0, no_erase=no_erase)
        Ov, Sv = forward(q, k, v, lav, be, s0, no_erase=no_erase)
        assert np.array_equal(Os, Ov) and np.array_equal(Ss, Sv), \
            f"equal channels differ from the scalar gate (no_erase={no_erase})"


def gla_closed_form(q, k, v, la, be, s0):
    """Unrolled no-erase recurrence with a per-channel gate (row form, one unit):
    with b_i = sum_{t<=i} log alpha_t (a vector over key channels),
        S_i = S0 diag(e^{b_i}) + sum_{s<=i} beta_s v_s (k_s o e^{b_i - b_s})^T,
        o_i = S0 (q_i o e^{b_i}) + sum_{s<=i} beta_s v_s sum_d q_id k_sd e^{b_id - b_sd}.
    Evaluated densely with numpy (the exponent of every (i, s, d) formed
    explicitly, masked to s <= i)."""
    L = q.shape[0]
    b = np.cumsum(la, axis=0)                               # [L, Dk]
    E = np.exp(b[:, None, :] - b[None, :, :])               # [i, s, d]
    mask = np.tril(np.ones((L, L)))[:, :, None]
    P = np.einsum("id,sd,isd->is", q, k, E * mask)          # [i, s]
    O = (q * np.exp(b)) @ s0.T + P @ (be[:, None] * v)
    S = s0 * np.exp(b[-1])[None, :] + (be[:, None] * v).T @ (k * np.exp(b[-1] - b))
    return O, S


def pin_gla_closed_form(forward, rng=None, **_):
    """The no-erase mode with a per-channel gate equals its unrolled closed
    form (the diagonal transitions commute, so the decay between tokens s and
    i of channel d is e^{b_id - b_sd})."""
    rng = rng or np.random.default_rng(22)
    L, Dk, Dv = 24, 6, 4
    q, k, v = rng.standard_normal((L, Dk)), rng.standard_normal((L, Dk)), rng.standard_normal((L, Dv))
    be, la = rng.uniform(0.1, 0.9, L), -rng.uniform(0.01, 0.6, (L, Dk))
    s0 = rng.standard_normal((Dv, Dk))
    O, S = _run_vec(forward, q, k, v, la, be, s0, no_erase=True)
    Ow, Sw = gla_closed_form(q, k, v, la, be, s0)
    _close(O, Ow, TIGHT, "GLA closed form O")
    _close(S, Sw, TIGHT, "GLA closed form S_T")


def pin_vector_gate_coordinate_retrieval(forward, rng=None, **_):
    """Erase mode, keys = distinct coordinate vectors e_{c_i}, beta = 1, any S0:
    token i overwrites column c_i with v_i, later tokens (other columns) only
    scale it by their gate of channel c_i, so S_T e_{c_i} = (prod_{t>i}
    alpha_t[c_i]) v_i.  (A diagonal gate keeps coordinate keys orthogonal.)"""
    rng = rng or np.random.default_rng(23)
    L, Dk, Dv = 6, 9, 4
    cols = rng.permutation(Dk)[:L]
    k = np.zeros((L, Dk))
    k[np.arange(L), cols] = 1.0
    q, v = rng.standard_normal((L, Dk)), rng.standard_normal((L, Dv))
    la = -rng.uniform(0.01, 0.7, (L, Dk))
    s0 = rng.standard_normal((Dv, Dk))
    _, S = _run_vec(forward, q, k, v, la, np.ones(L), s0)
    for i in range(L):
        tail = np.exp(la[i + 1:, cols[i]].sum())
        _close(S[:, cols[i]], tail * v[i], TIGHT, f"coordinate retrieval token {i}")


def pin_vector_gate_key_permutation(forward, rng=None, **_):
    """Renaming the key channels (the same permutation applied to q, k, the
    per-channel gate and the columns of S0) leaves O unchanged and permutes the
    columns of S_T, in both modes: each channel's gate travels with it."""
    rng = rng or np.random.default_rng(24)
    L, Dk, Dv = 15, 7, 3
    q, k, v = rng.standard_normal((L, Dk)), 0.5 * rng.standard_normal((L, Dk)), rng.standard_normal((L, Dv))
    be, la = rng.uniform(0.1, 0.9, L), -rng.uniform(0.01, 0.6, (L, Dk))
    s0 = rng.standard_normal((Dv, Dk))
    perm = rng.permutation(Dk)
    for no_erase in (False, True):
        O, S = _run_vec(forward, q, k, v, la, be, s0, no_erase=no_erase)
        Op, Sp = _run_vec(forward, q[:, perm], k[:, perm], v, la[:, perm], be, s0[:, perm],
                          no_erase=no_erase)
        _close(Op, O, TIGHT, f"key permutation O (no_erase={no_erase})")
        _close(Sp, S[:, perm], TIGHT, f"key permutation S_T (no_erase={no_erase})")


ALL_PINS = [pin_golden, pin_identity_step, pin_retrieval_identity, pin_mamba2_no_erase,
            pin_mamba2_orthogonal_keys, pin_exact_retrieval, pin_wy_identity,
            pin_product_form, pin_parallel_form, pin_linear_attention, pin_structure,
            pin_vector_gate_golden, pin_vector_gate_scalar_reduction, pin_gla_closed_form,
            pin_vector_gate_coordinate_retrieval, pin_vector_gate_key_permutation]
