"""The split scan (gdn_chunk_fwd_split: span maps, chained span starts, outputs
per span) against the fp64 oracle and against gdn_chunk_fwd, on the GPU.

Tolerance: max relative error per tensor, 2e-2 for bf16 inputs with fp32
accumulation, 1e-4 for the fp32 path.
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


def check(inp, span_chunks, tag="", dtype="bf16"):
    say(f"[gpu] split {tag} q={tuple(inp.q.shape)} span_chunks={span_chunks} seed={inp.meta.get('seed')}")
    d = inp.to(DEV)
    O, S = gdn.gdn_chunk_fwd_split(d.q, d.k, d.v, d.log_alpha, d.beta, d.S0, span_chunks=span_chunks)
    Op, Sp = gdn.gdn_chunk_fwd(d.q, d.k, d.v, d.log_alpha, d.beta, d.S0)
    torch.cuda.synchronize()
    O, S = O.double().cpu().numpy(), S.double().cpu().numpy()
    Or, Sr = oracle.forward(inp.q, inp.k, inp.v, inp.log_alpha, inp.beta, inp.S0)
    eo, es = rel(O, Or), rel(S, Sr)
    say(f"      max rel err O {eo:.3e}  S_T {es:.3e}  (tol {TOL[dtype]:.0e}); element-wise O "
        f"{rel_elem(O, Or):.3e} S_T {rel_elem(S, Sr):.3e}; vs unsplit O "
        f"{rel(O, Op.double().cpu().numpy()):.3e} S_T {rel(S, Sp.double().cpu().numpy()):.3e}")
    assert eo <= TOL[dtype] and es <= TOL[dtype], (eo, es)


def test_split_long_workload_all_heads():
    # the long-context workload, 512 chunks per sequence in 8 spans of 64 (256
    # span-head units: the span maps run in 128-column slices, the output pass
    # in 64-column ones)
    check(workload_inputs("gdn_bf16_long_b1_h32_t32768_d128"), 64, tag="workload 4")


def test_split_output_pass_in_wide_slices_ragged():
    # 16 heads x 2 sequences x 8 spans of one chunk, the last one ragged: the
    # output pass has more 32-column slices than CUs and runs 64-column ones,
    # the span maps more 64-column slices than CUs and run 128-column ones
    inp = make_inputs(B=2, T=64 * 7 + 5, H=16, Dk=128, Dv=128, dtype="bf16", gated=True, s0=True,
                      seed=3050)
    check(inp, 1, tag="wide output pass")


@pytest.mark.parametrize("T,span_chunks", [(1, 1), (64, 1), (300, 2), (64 * 7 + 5, 3), (1000, 100)])
def test_split_ragged_spans(T, span_chunks):
    # partial last chunk, a last span shorter than the others, one span (P = 1)
    inp = make_inputs(B=2, T=T, H=3, Dk=128, Dv=128, dtype="bf16", gated=True, s0=True,
                      seed=3000 + T)
    check(inp, span_chunks, tag=f"T={T}")


def test_split_few_heads_long():
    # the shape the split is for: few (sequence, head) units, long sequences
    inp = make_inputs(B=1, T=8192, H=2, Dk=128, Dv=128, dtype="bf16", gated=True, s0=True, seed=3100)
    check(inp, 16, tag="B1 H2 T8192")


def test_split_weak_gate_carries_state_across_spans():
    # a weak gate (log alpha = -5e-4 per token: e^-0.26 over a span of 8 chunks),
    # so that the span maps are far from zero and every span's outputs depend on
    # the state chained from the spans before it
    inp = make_inputs(B=1, T=4096, H=2, Dk=128, Dv=128, dtype="bf16", gated=True, s0=True, seed=3150)
    inp.log_alpha = torch.full_like(inp.log_alpha, -5e-4)
    check(inp, 8, tag="weak gate")


def test_split_weak_gate_long_chain():
    # 32 spans of 4 chunks under a weak gate: the chained start states (bf16
    # split products on MFMA) carry the state through every span
    inp = make_inputs(B=1, T=8192, H=2, Dk=128, Dv=128, dtype="bf16", gated=True, s0=True, seed=3160)
    inp.log_alpha = torch.full_like(inp.log_alpha, -2e-4)
    check(inp, 4, tag="weak gate, 32 spans")


def test_split_deltanet_and_zero_state():
    inp = make_inputs(B=1, T=2000, H=2, Dk=128, Dv=128, dtype="bf16", gated=False, s0=False, seed=3200)
    check(inp, 4, tag="alpha=1, S0=0")


@pytest.mark.parametrize("Dk,T,span_chunks", [(64, 1024, 4), (64, 64 * 9 + 17, 2), (64, 1000, 100),
                                                (128, 64 * 11 + 3, 3)])
def test_split_f32(Dk, T, span_chunks):
    # the fp32 instantiations (Dk = Dv = 64 and 128, C = 64), ragged last chunk
    # and last span, against the oracle at the fp32 tolerance; a weak gate so
    # that the chained states matter
    inp = make_inputs(B=2, T=T, H=4, Dk=Dk, Dv=Dk, dtype="f32", gated=True, s0=True, seed=3500 + Dk + T)
    inp.log_alpha = inp.log_alpha * 0.05
    check(inp, span_chunks, tag=f"f32 D{Dk} T={T}", dtype="f32")


def test_split_f32_workload_2():
    # the fp32 Dk = Dv = 64 workload (B2 H4 T1024: 16 chunks per sequence) in spans of 4
    check(workload_inputs("gdn_f32_b2_h4_t1024_d64"), 4, tag="workload 2", dtype="f32")


def test_split_in_place_state_and_profiled():
    inp = make_inputs(B=2, T=700, H=4, Dk=128, Dv=128, dtype="bf16", gated=True, s0=True, seed=3300)
    d = inp.to(DEV)
    O1, S1 = gdn.gdn_chunk_fwd_split(d.q, d.k, d.v, d.log_alpha, d.beta, d.S0, span_chunks=3)
    S = d.S0.clone()
    O2, _ = gdn.gdn_chunk_fwd_split(d.q, d.k, d.v, d.log_alpha, d.beta, S, span_chunks=3, S_T=S)
    O3, S3, ms = gdn.gdn_chunk_fwd_split(d.q, d.k, d.v, d.log_alpha, d.beta, d.S0, span_chunks=3,
                                         profiled=True)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(S1, S) and torch.equal(O1, O3) and torch.equal(S1, S3)
    assert all(x > 0 for x in ms), ms


def test_gdn_chunk_fwd_takes_the_split_for_few_long_units():
    # B1 H2 T8192 (128 chunks per sequence, 2 units): gdn_chunk_fwd splits it
    # by itself, with the span length gdn_chunk_fwd_auto_span_chunks reports on
    # this device: bitwise what gdn_chunk_fwd_split gives with that span length,
    # and within tolerance of the plain scan (the profiled call) and the oracle
    inp = make_inputs(B=1, T=8192, H=2, Dk=128, Dv=128, dtype="bf16", gated=True, s0=True, seed=3400)
    L = gdn.gdn_chunk_fwd_auto_span_chunks(1, 8192, 2, 128, 128, 64, 0, torch.bfloat16)
    assert 8 <= L <= 64, L
    # the headline keeps the plain scan; the long workload (32 units of 512
    # chunks) is split into spans of 128 chunks
    assert gdn.gdn_chunk_fwd_auto_span_chunks(4, 4096, 16, 128, 128, 64, 0, torch.bfloat16) == 0
    assert gdn.gdn_chunk_fwd_auto_span_chunks(1, 32768, 32, 128, 128, 64, 0, torch.bfloat16) == 128
    d = inp.to(DEV)
    O, S = gdn.gdn_chunk_fwd(d.q, d.k, d.v, d.log_alpha, d.beta, d.S0)
    Os, Ss = gdn.gdn_chunk_fwd_split(d.q, d.k, d.v, d.log_alpha, d.beta, d.S0, span_chunks=L)
    Op, Sp, _ = gdn.gdn_chunk_fwd_profiled(d.q, d.k, d.v, d.log_alpha, d.beta, d.S0)
    torch.cuda.synchronize()
    assert torch.equal(O, Os) and torch.equal(S, Ss)
    assert rel(O.double().cpu().numpy(), Op.double().cpu().numpy()) <= 2e-2
    Or, Sr = oracle.forward(inp.q, inp.k, inp.v, inp.log_alpha, inp.beta, inp.S0)
    assert rel(O.double().cpu().numpy(), Or) <= 2e-2 and rel(S.double().cpu().numpy(), Sr) <= 2e-2


def test_gdn_chunk_fwd_takes_the_split_for_the_f32_workload():
    # the fp32 D64 workload (B2 H4 T1024, 16 chunks per sequence) is split by
    # gdn_chunk_fwd itself; bitwise the explicit split, within 1e-4 of the oracle
    inp = workload_inputs("gdn_f32_b2_h4_t1024_d64")
    L = gdn.gdn_chunk_fwd_auto_span_chunks(2, 1024, 4, 64, 64, 64, 0, torch.float32)
    assert L > 0, L
    d = inp.to(DEV)
    O, S = gdn.gdn_chunk_fwd(d.q, d.k, d.v, d.log_alpha, d.beta, d.S0)
    Os, Ss = gdn.gdn_chunk_fwd_split(d.q, d.k, d.v, d.log_alpha, d.beta, d.S0, span_chunks=L)
    torch.cuda.synchronize()
    assert torch.equal(O, Os) and torch.equal(S, Ss)
    Or, Sr = oracle.forward(inp.q, inp.k, inp.v, inp.log_alpha, inp.beta, inp.S0)
    eo, es = rel(O.double().cpu().numpy(), Or), rel(S.double().cpu().numpy(), Sr)
    say(f"      f32 workload 2 auto split L={L}: max rel err O {eo:.3e}  S_T {es:.3e}")
    assert eo <= TOL["f32"] and es <= TOL["f32"], (eo, es)
