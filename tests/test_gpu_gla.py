"""Parity of gdn_gla_chunk_fwd (per-channel gate, no erase term) with the fp64
oracle, on the GPU, through the C ABI.

The recurrence is S_t = S_{t-1} diag(alpha_t) + beta_t v_t k_t^T, o_t = S_t q_t
with one gate per key channel: the vector-gated GLA that
LinearAttention系列解读(六), section 1, names, with a write strength.  The
oracle's per-channel no-erase mode is pinned by tests/oracle_pins.py
(pin_vector_gate_golden, pin_gla_closed_form, pin_vector_gate_scalar_reduction,
pin_vector_gate_key_permutation).  Tolerances as for the delta rule: max
relative error 1e-4 (fp32) and 2e-2 (bf16 inputs, fp32 accumulation).
"""
import os
import sys

import numpy as np
import pytest
import torch

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import oracle  # noqa: E402
import gated_delta_rule_16_amd as gdn  # noqa: E402
from gated_delta_rule_16_amd.inputs import make_inputs, workload_inputs  # noqa: E402
from test_gpu_parity import TOL, rel, rel_elem, say  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.load_library()


def run(inp, C=64, beta_none=False):
    d = inp.to(DEV)
    O, S = gdn.gdn_gla_chunk_fwd(d.q, d.k, d.v, d.log_alpha, None if beta_none else d.beta,
                                 d.S0, d.cu_seqlens, chunk_size=C)
    torch.cuda.synchronize()
    return O.double().cpu().numpy(), S.double().cpu().numpy()


def check(inp, dtype, C=64, beta_none=False, tag=""):
    say(f"[gpu] gla {tag} q={tuple(inp.q.shape)} v={tuple(inp.v.shape)} {dtype} C={C} "
        f"seed={inp.meta.get('seed')} beta={'1' if beta_none else 'drawn'}")
    O, S = run(inp, C, beta_none)
    be = torch.ones_like(inp.beta) if beta_none else inp.beta
    Or, Sr = oracle.forward(inp.q, inp.k, inp.v, inp.log_alpha, be, inp.S0, inp.cu_seqlens,
                            no_erase=True)
    eo, es = rel(O, Or), rel(S, Sr)
    say(f"      max rel err O {eo:.3e}  S_T {es:.3e}  (tol {TOL[dtype]:.0e}); element-wise "
        f"O {rel_elem(O, Or):.3e}  S_T {rel_elem(S, Sr):.3e}")
    assert eo <= TOL[dtype] and es <= TOL[dtype], (eo, es)
    return O, S


def test_gla_f32_b2_h4_t1024_d64():
    check(workload_inputs("gdn_f32_b2_h4_t1024_d64", gate_channels=True), "f32",
          tag="fp32 B2 H4 T1024 D64")


def test_gla_bf16_b4_h16_t4096_d128():
    check(workload_inputs("gdn_bf16_b4_h16_t4096_d128", gate_channels=True), "bf16",
          tag="bf16 B4 H16 T4096 D128")


def test_gla_bf16_varlen_dv256():
    check(workload_inputs("gdn_bf16_varlen_65536_h16_dk128_dv256", gate_channels=True), "bf16",
          tag="packed 65536 tokens Dv256")


@pytest.mark.parametrize("dtype,Dk,Dv,C", [("f32", 16, 16, 16), ("f32", 64, 64, 64),
                                           ("bf16", 128, 128, 64), ("bf16", 128, 256, 64)])
@pytest.mark.parametrize("T", [1, 5, 64, 300])
def test_gla_ragged(dtype, Dk, Dv, C, T):
    inp = make_inputs(B=2, T=T, H=3, Dk=Dk, Dv=Dv, dtype=dtype, gated=True, s0=True,
                      seed=2500 + T + Dv, gate_channels=True)
    check(inp, dtype, C=C, tag="ragged")


@pytest.mark.parametrize("dtype,D", [("f32", 64), ("bf16", 128)])
def test_gla_beta_one_and_ungated(dtype, D):
    inp = make_inputs(B=2, T=200, H=2, Dk=D, Dv=D, dtype=dtype, gated=True, s0=True, seed=710,
                      gate_channels=True)
    check(inp, dtype, beta_none=True, tag="beta=1")
    inp = make_inputs(B=2, T=200, H=2, Dk=D, Dv=D, dtype=dtype, gated=False, s0=True, seed=711)
    check(inp, dtype, beta_none=True, tag="alpha=1 (linear attention)")


@pytest.mark.parametrize("dtype,D", [("f32", 64), ("bf16", 128)])
def test_gla_equal_channels_match_scalar_rule(dtype, D):
    # every channel of the gate equal: the per-channel rule is the scalar one, so
    # gdn_gla_chunk_fwd and gdn_mamba2_chunk_fwd agree (to rounding: their
    # kernels group the decays differently), and both match the oracle
    inp = make_inputs(B=2, T=300, H=2, Dk=D, Dv=D, dtype=dtype, gated=True, s0=True, seed=720)
    vec = make_inputs(B=2, T=300, H=2, Dk=D, Dv=D, dtype=dtype, gated=True, s0=True, seed=720)
    vec.log_alpha = inp.log_alpha[..., None].expand(-1, -1, -1, D).contiguous()
    O1, S1 = check(vec, dtype, tag="equal channels")
    d = inp.to(DEV)
    O2, S2 = gdn.gdn_mamba2_chunk_fwd(d.q, d.k, d.v, d.log_alpha, d.beta, d.S0)
    torch.cuda.synchronize()
    assert rel(O1, O2.double().cpu().numpy()) <= TOL[dtype]
    assert rel(S1, S2.double().cpu().numpy()) <= TOL[dtype]


@pytest.mark.parametrize("case", ["decay30", "resets", "mixed_channels", "chunk_decay_61",
                                  "chunk_decay_67"])
@pytest.mark.parametrize("dtype,D", [("f32", 64), ("bf16", 128)])
def test_gla_degenerate_gates(case, dtype, D):
    # decay30: log alpha = -30 on every channel and token (every diagonal block
    # of P~ takes the term-by-term path); resets: -80 every 37 tokens on every
    # channel; mixed: half the channels at -30, the others drawn;
    # chunk_decay_61 / _67: -0.95 / -1.05 on every channel and token, a decay of
    # e^-60.8 / e^-67.2 over a 64-token chunk, on either side of the bound of
    # e^-64 below which a chunk leaves the whole-chunk form (Q~ and K e^-b) for
    # the blocked one (full chunks; the last, partial chunk decays less)
    inp = make_inputs(B=2, T=200, H=2, Dk=D, Dv=D, dtype=dtype, gated=True, s0=True, seed=730,
                      gate_channels=True)
    if case == "decay30":
        inp.log_alpha = torch.full_like(inp.log_alpha, -30.0)
    elif case == "resets":
        inp.log_alpha = torch.zeros_like(inp.log_alpha)
        inp.log_alpha[:, 5::37] = -80.0
    elif case == "chunk_decay_61":
        inp.log_alpha = torch.full_like(inp.log_alpha, -0.95)
    elif case == "chunk_decay_67":
        inp.log_alpha = torch.full_like(inp.log_alpha, -1.05)
    else:
        inp.log_alpha[..., ::2] = -30.0
    check(inp, dtype, tag=f"gates {case}")


def test_gla_varlen_short_and_empty():
    lengths = [0, 1, 63, 64, 65, 200, 0, 7, 130]
    inp = make_inputs(B=1, T=sum(lengths), H=2, Dk=128, Dv=256, dtype="bf16", gated=True,
                      s0=True, seed=740, lengths=lengths, gate_channels=True)
    check(inp, "bf16", tag=f"varlen {lengths}")


def test_gla_profiled_matches_plain_call():
    inp = make_inputs(B=2, T=300, H=4, Dk=128, Dv=128, dtype="bf16", gated=True, s0=True,
                      seed=750, gate_channels=True)
    d = inp.to(DEV)
    O1, S1 = gdn.gdn_gla_chunk_fwd(d.q, d.k, d.v, d.log_alpha, d.beta, d.S0)
    O2, S2, ms = gdn.gdn_rule_chunk_fwd_profiled(gdn.GDN_RULE_GLA, d.q, d.k, d.v, d.log_alpha,
                                                 d.beta, d.S0)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(S1, S2)
    assert ms[1] > 0 and ms[2] > 0


def test_gla_wide_slices():
    # bf16 calls with more 32-column slices than CUs take 64-column slices
    inp = make_inputs(B=8, T=300, H=32, Dk=128, Dv=128, dtype="bf16", gated=True, s0=True,
                      seed=420, gate_channels=True)
    check(inp, "bf16", tag="64-column slices")
