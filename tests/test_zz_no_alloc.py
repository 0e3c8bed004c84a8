"""gdn_chunk_fwd_noalloc (the allocation-free variant, on the library's static
scratch buffer) through the C ABI, against gdn_chunk_fwd with a workspace.

Two calls in a row on the same GPU, the second with a smaller input, so that
the second runs on a buffer that still holds the first call's intermediates.
The two entry points run the same kernels, so their outputs must agree bit
for bit; the oracle check keeps the comparison anchored to the definition.
"""
import ctypes
import os
import sys

import numpy as np
import pytest
import torch

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import oracle  # noqa: E402
import gated_delta_rule_16_amd as gdn  # noqa: E402
from gated_delta_rule_16_amd.inputs import make_inputs  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _noalloc_raw(d, C, O, S_T):
    """Call the C entry point directly with ctypes (outputs preallocated here)."""
    lib = gdn.load_library()
    B, T, H, Dk = d.q.shape
    Dv = d.v.shape[3]
    n = 0 if d.cu_seqlens is None else d.cu_seqlens.numel() - 1
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    dt = gdn.GDN_BF16 if d.q.dtype == torch.bfloat16 else gdn.GDN_F32
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return lib.gdn_chunk_fwd_noalloc(P(d.q), P(d.k), P(d.v), P(d.log_alpha), P(d.beta), P(d.S0),
                                     P(d.cu_seqlens), n, P(O), P(S_T), B, T, H, Dk, Dv, C, dt,
                                     stream)


def _rel(x, r):
    return float(np.abs(x - r).max() / max(np.abs(r).max(), 1e-30))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.load_library()


def test_noalloc_matches_workspace_entry_two_calls():
    cases = [
        # (inputs, C, dtype tolerance): each smaller than the one before; the
        # first has enough units for the scan's 64-column slices
        (make_inputs(B=8, T=300, H=32, Dk=128, Dv=128, dtype="bf16", gated=True, s0=True,
                     seed=900), 64, 2e-2),
        (make_inputs(B=2, T=700, H=8, Dk=128, Dv=128, dtype="bf16", gated=True, s0=True,
                     seed=901), 64, 2e-2),
        (make_inputs(B=1, T=150, H=4, Dk=128, Dv=128, dtype="bf16", gated=True, s0=True,
                     seed=902), 64, 2e-2),
    ]
    for i, (inp, C, tol) in enumerate(cases):
        print(f"[gpu] noalloc call {i}: q={tuple(inp.q.shape)} C={C}", flush=True)
        d = inp.to(DEV)
        O_ref, S_ref = gdn.gdn_chunk_fwd(d.q, d.k, d.v, d.log_alpha, d.beta, d.S0, d.cu_seqlens,
                                         chunk_size=C)
        O = torch.full_like(O_ref, float("nan"))
        S_T = torch.full_like(S_ref, float("nan"))
        rc = _noalloc_raw(d, C, O, S_T)
        torch.cuda.synchronize()
        assert rc == 0, gdn.gdn_status_string(rc)
        assert torch.equal(O, O_ref) and torch.equal(S_T, S_ref), f"call {i} differs"
        Or, Sr = oracle.forward(inp.q, inp.k, inp.v, inp.log_alpha, inp.beta, inp.S0)
        eo = _rel(O.double().cpu().numpy(), Or)
        es = _rel(S_T.double().cpu().numpy(), Sr)
        print(f"      max rel err O {eo:.3e}  S_T {es:.3e}", flush=True)
        assert eo <= tol and es <= tol


def test_noalloc_packed_and_binding():
    # a packed batch (chunk table in the scratch buffer too), through the binding
    lengths = [0, 33, 130, 64]
    inp = make_inputs(B=1, T=sum(lengths), H=3, Dk=128, Dv=256, dtype="bf16", gated=True,
                      s0=True, seed=903, lengths=lengths)
    d = inp.to(DEV)
    O_ref, S_ref = gdn.gdn_chunk_fwd(d.q, d.k, d.v, d.log_alpha, d.beta, d.S0, d.cu_seqlens)
    O = torch.empty_like(O_ref)
    S_T = torch.empty_like(S_ref)
    gdn.gdn_chunk_fwd_noalloc(d.q, d.k, d.v, d.log_alpha, d.beta, d.S0, d.cu_seqlens, O, S_T)
    torch.cuda.synchronize()
    assert torch.equal(O, O_ref) and torch.equal(S_T, S_ref)


def test_noalloc_refuses_sizes_past_its_buffer():
    d = make_inputs(B=1, T=32768, H=32, Dk=128, Dv=128, dtype="bf16", seed=904, device=DEV)
    O = torch.empty(1, 32768, 32, 128, device=DEV, dtype=torch.bfloat16)
    with pytest.raises(gdn.GdnError) as e:
        gdn.gdn_chunk_fwd_noalloc(d.q, d.k, d.v, d.log_alpha, d.beta, d.S0, None, O, None)
    assert e.value.code == 7
