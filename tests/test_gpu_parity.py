"""Parity of the HIP path (through the C ABI) with the fp64 oracle, on the GPU.

Tolerances (max relative error per tensor, ||x - r||_inf / ||r||_inf, O and
S_T separately): 1e-4 for the fp32 path, 2e-2 for bf16 inputs with fp32
accumulation and state.
"""
import os
import sys

import numpy as np
import pytest
import torch

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import oracle  # noqa: E402
import gated_delta_rule_16_amd as gdn  # noqa: E402
from gated_delta_rule_16_amd.inputs import WORKLOADS, make_inputs, workload_inputs  # noqa: E402

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
DEV = "cuda:0"


def rel(x, r):
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    assert x.shape == r.shape, (x.shape, r.shape)
    if x.size == 0:
        return 0.0
    return float(np.abs(x - r).max() / max(np.abs(r).max(), 1e-30))


def rel_elem(x, r, floor=1e-3):
    """Element-wise relative error, max_i |x_i - r_i| / max(|r_i|, floor ||r||_inf):
    reported beside the norm-wise error (not a pass/fail bound)."""
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if x.size == 0:
        return 0.0
    den = np.maximum(np.abs(r), floor * max(np.abs(r).max(), 1e-30))
    return float((np.abs(x - r) / den).max())


def say(*a):
    print(*a, flush=True)


def run_gpu(inp, C=None, **kw):
    d = inp.to(DEV)
    O, S = gdn.gdn_chunk_fwd(d.q, d.k, d.v, d.log_alpha, d.beta, d.S0, d.cu_seqlens,
                             chunk_size=C or inp.C, **kw)
    torch.cuda.synchronize()
    return O.double().cpu().numpy(), None if S is None else S.double().cpu().numpy()


def run_oracle(inp, heads=None):
    """Oracle outputs; ``heads`` restricts it to a sample of heads (units are independent)."""
    sl = (lambda t: t) if heads is None else (lambda t: None if t is None else t[:, :, heads])
    s0 = inp.S0 if (heads is None or inp.S0 is None) else inp.S0[:, heads]
    return oracle.forward(sl(inp.q), sl(inp.k), sl(inp.v), sl(inp.log_alpha), sl(inp.beta), s0,
                          inp.cu_seqlens)


def check(inp, dtype, C=None, heads=None, tag=""):
    say(f"[gpu] {tag} shape q={tuple(inp.q.shape)} v={tuple(inp.v.shape)} dtype={dtype} "
        f"C={C or inp.C} seed={inp.meta.get('seed')}")
    O, S = run_gpu(inp, C)
    Or, Sr = run_oracle(inp, heads)
    if heads is not None:
        O, S = O[:, :, heads], S[:, heads]
    eo, es = rel(O, Or), rel(S, Sr)
    say(f"      max rel err O {eo:.3e}  S_T {es:.3e}  (tol {TOL[dtype]:.0e}); element-wise "
        f"(floor 1e-3 max|r|) O {rel_elem(O, Or):.3e}  S_T {rel_elem(S, Sr):.3e}")
    assert eo <= TOL[dtype] and es <= TOL[dtype], (eo, es)
    return eo, es


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    gdn.load_library()


# ---------------------------------------------------------------------------
# the five workloads at full size
# ---------------------------------------------------------------------------
def test_workload_deltanet_f32_t128_d16():
    check(workload_inputs("deltanet_f32_b1_h1_t128_d16"), "f32", tag="workload 1")


def test_workload_gdn_f32_b2_h4_t1024_d64():
    check(workload_inputs("gdn_f32_b2_h4_t1024_d64"), "f32", tag="workload 2")


def test_workload_gdn_f32_b2_h4_t1024_d64_plain_scan():
    # gdn_chunk_fwd splits this workload (few units); the plain scan on the same
    # inputs through the profiled call, which always runs it
    inp = workload_inputs("gdn_f32_b2_h4_t1024_d64")
    d = inp.to(DEV)
    O, S, _ = gdn.gdn_chunk_fwd_profiled(d.q, d.k, d.v, d.log_alpha, d.beta, d.S0)
    torch.cuda.synchronize()
    Or, Sr = run_oracle(inp)
    eo, es = rel(O.double().cpu().numpy(), Or), rel(S.double().cpu().numpy(), Sr)
    say(f"      workload 2, plain scan: max rel err O {eo:.3e}  S_T {es:.3e}")
    assert eo <= TOL["f32"] and es <= TOL["f32"], (eo, es)


def test_workload_gdn_bf16_b4_h16_t4096_d128():
    check(workload_inputs("gdn_bf16_b4_h16_t4096_d128"), "bf16", tag="workload 3")


def test_workload_gdn_bf16_long_t32768():
    check(workload_inputs("gdn_bf16_long_b1_h32_t32768_d128"), "bf16", tag="workload 4")


def test_workload_gdn_bf16_varlen_dv256():
    inp = workload_inputs("gdn_bf16_varlen_65536_h16_dk128_dv256")
    check(inp, "bf16", tag="workload 5")


def test_second_seed_headline():
    check(workload_inputs("gdn_bf16_b4_h16_t4096_d128", seed=103), "bf16", heads=[1, 14],
          tag="workload 3 seed 103")


# ---------------------------------------------------------------------------
# shapes: several tiles, ragged tails, short and empty sequences
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,Dk,Dv,C", [("f32", 16, 16, 16), ("f32", 64, 64, 16),
                                           ("f32", 64, 64, 64), ("f32", 128, 128, 64),
                                           ("f32", 128, 256, 64), ("bf16", 128, 128, 64),
                                           ("bf16", 128, 256, 64)])
@pytest.mark.parametrize("T", [1, 5, 64, 300])
def test_ragged(dtype, Dk, Dv, C, T):
    inp = make_inputs(B=2, T=T, H=3, Dk=Dk, Dv=Dv, dtype=dtype, gated=True, s0=True,
                      seed=1000 + T + Dv)
    check(inp, dtype, C=C, tag="ragged")


@pytest.mark.parametrize("C", [16, 64])
def test_f32_d64_two_column_waves(C):
    # fp32 Dk = Dv = 64 with enough (sequence, head) units that every CU gets a
    # 32-column slice: the scan with two column waves per workgroup (smaller
    # batches take the 16-column one)
    inp = make_inputs(B=4, T=200, H=64, Dk=64, Dv=64, dtype="f32", gated=True, s0=True,
                      seed=400 + C)
    check(inp, "f32", C=C, tag="fp32 D64 32-column slices")


@pytest.mark.parametrize("B,H,T,Dv", [(8, 32, 300, 128), (4, 32, 200, 256), (3, 32, 130, 128)])
def test_wide_slices(B, H, T, Dv):
    # bf16 calls whose 32-column slices would need more than one workgroup per
    # CU take 64-column slices (four column waves, one output helper per query
    # block); ragged last chunks, every head against the oracle
    inp = make_inputs(B=B, T=T, H=H, Dk=128, Dv=Dv, dtype="bf16", gated=True, s0=True,
                      seed=410 + B)
    check(inp, "bf16", tag="64-column slices")


def test_wide_slices_varlen():
    # packed batch in 64-column slices: empty, one-token, chunk-edge and
    # several-chunk sequences over 32 heads
    lengths = [0, 1, 63, 64, 65, 200, 0, 7, 130, 129, 2]
    inp = make_inputs(B=1, T=sum(lengths), H=32, Dk=128, Dv=128, dtype="bf16", gated=True,
                      s0=True, seed=415, lengths=lengths)
    check(inp, "bf16", tag="varlen 64-column slices")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_largest_accepted_sizes(dtype):
    # the largest token tensors gdn_chunk_fwd accepts (one token more passes
    # 2^31 - 1 elements): byte offsets past 2^31 (bf16) and past 2^32 (fp32).
    # Drawn on the device, checked by the oracle on the first, a middle and the
    # last head
    B, T, H, D = 1, 1023, 16384, 128
    assert B * T * H * D <= 2**31 - 1 < B * (T + 1) * H * D
    say(f"[gpu] largest sizes B={B} T={T} H={H} D={D} {dtype} C=64 seed=91")
    d = make_inputs(B, T, H, D, D, dtype=dtype, seed=91, device=DEV)
    O, S = gdn.gdn_chunk_fwd(d.q, d.k, d.v, d.log_alpha, d.beta, d.S0, None, chunk_size=64)
    torch.cuda.synchronize()
    heads = [0, H // 2 - 1, H - 1]
    sub = lambda t: t[:, :, heads].cpu()
    Or, Sr = oracle.forward(sub(d.q), sub(d.k), sub(d.v), sub(d.log_alpha), sub(d.beta),
                            d.S0[:, heads].cpu(), None)
    eo = rel(O[:, :, heads].double().cpu().numpy(), Or)
    es = rel(S[:, heads].double().cpu().numpy(), Sr)
    say(f"      max rel err O {eo:.3e}  S_T {es:.3e}  (tol {TOL[dtype]:.0e})")
    assert eo <= TOL[dtype] and es <= TOL[dtype], (eo, es)
    del d, O, S
    torch.cuda.empty_cache()


@pytest.mark.parametrize("case", ["beta0", "beta1", "decay30", "resets"])
@pytest.mark.parametrize("dtype,D", [("f32", 64), ("bf16", 128)])
def test_degenerate_gates(case, dtype, D):
    # beta = 0: nothing is written, the state only decays; beta = 1: each
    # write replaces the state's value along k; log alpha = -30 on every token:
    # the state is forgotten from one token to the next and the in-chunk
    # decays underflow; log alpha alternating 0 and -80: resets inside chunks,
    # so that exp(g) underflows to zero part-way through a chunk
    inp = make_inputs(B=2, T=200, H=2, Dk=D, Dv=D, dtype=dtype, gated=True, s0=True,
                      seed=300 + D, beta_fill={"beta0": 0.0, "beta1": 1.0}.get(case))
    if case == "decay30":
        inp.log_alpha = torch.full_like(inp.log_alpha, -30.0)
    elif case == "resets":
        inp.log_alpha = torch.zeros_like(inp.log_alpha)
        inp.log_alpha[:, 5::37] = -80.0
    check(inp, dtype, C=64, tag=f"gates {case}")   # a NaN or inf anywhere fails the bound


@pytest.mark.parametrize("dtype,D", [("f32", 64), ("bf16", 128)])
def test_deltanet_alpha_one_with_state(dtype, D):
    inp = make_inputs(B=1, T=257, H=2, Dk=D, Dv=D, dtype=dtype, gated=False, s0=True, seed=5)
    check(inp, dtype, C=64, tag="alpha=1")


def test_zero_length_sequence_returns_initial_state():
    inp = make_inputs(B=2, T=0, H=2, Dk=64, Dv=64, dtype="f32", gated=True, s0=True, seed=3)
    O, S = run_gpu(inp, 64)
    assert O.shape == (2, 0, 2, 64)
    assert np.array_equal(S, inp.S0.double().numpy())


@pytest.mark.parametrize("dtype,Dk,Dv", [("f32", 64, 64), ("bf16", 128, 256), ("bf16", 128, 128)])
def test_varlen_packed(dtype, Dk, Dv):
    lengths = [0, 1, 63, 64, 65, 200, 0, 7, 130]
    inp = make_inputs(B=1, T=sum(lengths), H=2, Dk=Dk, Dv=Dv, dtype=dtype, gated=True, s0=True,
                      seed=77, lengths=lengths)
    check(inp, dtype, C=64, tag=f"varlen {lengths}")


@pytest.mark.parametrize("dtype,D,C", [("f32", 16, 16), ("bf16", 128, 64)])
def test_varlen_many_sequences(dtype, D, C):
    # more sequences than the chunk table's workgroup covers in one pass (1024),
    # so its running maximum, chunk-count prefix sum and slot search carry
    # across passes; every third sequence is empty and most are shorter than
    # a chunk
    rng = np.random.default_rng(2500 + D)
    lengths = [int(x) for x in rng.integers(1, 40, size=2500)]
    for i in range(0, len(lengths), 3):
        lengths[i] = 0
    lengths[1], lengths[2047] = 300, 5 * C + 3   # several chunks with a ragged tail
    inp = make_inputs(B=1, T=sum(lengths), H=2, Dk=D, Dv=D, dtype=dtype, gated=True, s0=True,
                      seed=79, lengths=lengths)
    check(inp, dtype, C=C, tag=f"varlen {len(lengths)} sequences")


def test_varlen_longest_first_order_edges():
    # the scan dispatches packed sequences by chunk count, longest first (a
    # counting sort over 4096 bins, counts of 4095 chunks and more sharing the
    # first bin): sequences longer than that (4100 and 4300 chunks of 16), equal
    # lengths, ascending and descending runs and empty ones, all against the
    # oracle
    C = 16
    lengths = [4100 * C - 3, 5, 5, 0, 4300 * C, 17, 33, 64, 0, 65, 300, 299, 3, 1, 5]
    inp = make_inputs(B=1, T=sum(lengths), H=1, Dk=16, Dv=16, dtype="f32", gated=True, s0=True,
                      seed=81, lengths=lengths)
    check(inp, "f32", C=C, tag="varlen order edges")


def test_varlen_equals_separate_calls():
    lengths = [100, 37, 256]
    inp = make_inputs(B=1, T=sum(lengths), H=4, Dk=128, Dv=128, dtype="bf16", gated=True,
                      s0=True, seed=78, lengths=lengths)
    O, S = run_gpu(inp)
    off = 0
    for i, n in enumerate(lengths):
        sub = make_inputs(B=1, T=n, H=4, Dk=128, Dv=128, dtype="bf16", seed=0)
        sub.q, sub.k, sub.v = (t[:, off:off + n].contiguous() for t in (inp.q, inp.k, inp.v))
        sub.beta = inp.beta[:, off:off + n].contiguous()
        sub.log_alpha = inp.log_alpha[:, off:off + n].contiguous()
        sub.S0 = inp.S0[i:i + 1].contiguous()
        Oi, Si = run_gpu(sub)
        assert np.array_equal(Oi[0], O[0, off:off + n]), f"sequence {i} O"
        assert np.array_equal(Si[0], S[i]), f"sequence {i} S_T"
        off += n


# ---------------------------------------------------------------------------
# invariants: determinism, chunk-size invariance, resume, in-place state
# ---------------------------------------------------------------------------
def test_bitwise_deterministic():
    inp = workload_inputs("gdn_bf16_b4_h16_t4096_d128")
    O1, S1 = run_gpu(inp)
    O2, S2 = run_gpu(inp)
    assert np.array_equal(O1, O2) and np.array_equal(S1, S2)


def test_bitwise_deterministic_wide_slices_and_split():
    # the 64-column slices (B8 H32) and the automatic split (B1 H4 T8192)
    for inp in (make_inputs(B=8, T=300, H=32, Dk=128, Dv=128, dtype="bf16", seed=417),
                make_inputs(B=1, T=8192, H=4, Dk=128, Dv=128, dtype="bf16", seed=418)):
        O1, S1 = run_gpu(inp)
        O2, S2 = run_gpu(inp)
        assert np.array_equal(O1, O2) and np.array_equal(S1, S2)


def test_workspace_reused_across_inputs():
    """One workspace, filled with 0xff bytes first, serves calls on different
    inputs in turn: each call's results match the oracle, so nothing a previous
    call left there (Tb, gates) reaches the next one."""
    ins = [make_inputs(B=2, T=700, H=8, Dk=128, Dv=128, dtype="bf16", gated=True, s0=True, seed=s)
           for s in (81, 82)]
    nbytes = gdn.gdn_chunk_fwd_workspace_bytes(2, 700, 8, 128, 128, 64, 0, torch.bfloat16)
    ws = torch.full((nbytes,), 255, dtype=torch.uint8, device=DEV)
    refs = [run_oracle(x) for x in ins]
    for i in (0, 1, 0):
        d = ins[i].to(DEV)
        O, S = gdn.gdn_chunk_fwd(d.q, d.k, d.v, d.log_alpha, d.beta, d.S0, chunk_size=64, workspace=ws)
        torch.cuda.synchronize()
        eo, es = rel(O.double().cpu().numpy(), refs[i][0]), rel(S.double().cpu().numpy(), refs[i][1])
        say(f"[gpu] workspace reuse, inputs {i}: O {eo:.3e}  S_T {es:.3e}")
        assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_chunk_size_invariance_f32():
    inp = make_inputs(B=2, T=333, H=2, Dk=64, Dv=64, dtype="f32", gated=True, s0=True, seed=9)
    O16, S16 = run_gpu(inp, 16)
    O64, S64 = run_gpu(inp, 64)
    assert rel(O16, O64) <= 1e-5 and rel(S16, S64) <= 1e-5


@pytest.mark.parametrize("dtype,D", [("f32", 64), ("bf16", 128)])
def test_resume_from_state(dtype, D):
    inp = make_inputs(B=2, T=500, H=2, Dk=D, Dv=D, dtype=dtype, gated=True, s0=True, seed=21)
    Or, Sr = run_oracle(inp)
    T1 = 211
    a = make_inputs(B=2, T=T1, H=2, Dk=D, Dv=D, dtype=dtype, seed=0)
    b = make_inputs(B=2, T=500 - T1, H=2, Dk=D, Dv=D, dtype=dtype, seed=0)
    for part, sl in ((a, slice(0, T1)), (b, slice(T1, 500))):
        part.q, part.k, part.v = (t[:, sl].contiguous() for t in (inp.q, inp.k, inp.v))
        part.beta, part.log_alpha = (t[:, sl].contiguous() for t in (inp.beta, inp.log_alpha))
    a.S0 = inp.S0
    Oa, Sa = run_gpu(a, 64)
    b.S0 = torch.from_numpy(Sa).float()
    Ob, Sb = run_gpu(b, 64)
    assert rel(np.concatenate([Oa, Ob], 1), Or) <= TOL[dtype]
    assert rel(Sb, Sr) <= TOL[dtype]


def test_state_in_place_and_optional_final_state():
    inp = make_inputs(B=2, T=190, H=2, Dk=128, Dv=128, dtype="bf16", gated=True, s0=True, seed=31)
    d = inp.to(DEV)
    O_ref, S_ref = gdn.gdn_chunk_fwd(d.q, d.k, d.v, d.log_alpha, d.beta, d.S0)
    S = d.S0.clone()
    O_ip, _ = gdn.gdn_chunk_fwd(d.q, d.k, d.v, d.log_alpha, d.beta, S, S_T=S)
    O_no, S_no = gdn.gdn_chunk_fwd(d.q, d.k, d.v, d.log_alpha, d.beta, d.S0,
                                   output_final_state=False)
    torch.cuda.synchronize()
    assert S_no is None
    assert torch.equal(O_ip, O_ref) and torch.equal(S, S_ref) and torch.equal(O_no, O_ref)


def test_side_stream():
    inp = make_inputs(B=1, T=130, H=2, Dk=64, Dv=64, dtype="f32", gated=True, s0=True, seed=41)
    d = inp.to(DEV)
    ref = gdn.gdn_chunk_fwd(d.q, d.k, d.v, d.log_alpha, d.beta, d.S0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        out = gdn.gdn_chunk_fwd(d.q, d.k, d.v, d.log_alpha, d.beta, d.S0, stream=s)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(out[0], ref[0]) and torch.equal(out[1], ref[1])


# ---------------------------------------------------------------------------
# single-token step and prefill -> decode
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,Dk,Dv", [("f32", 16, 16), ("f32", 64, 64), ("bf16", 128, 128),
                                         ("bf16", 128, 256), ("f32", 128, 256)])
@pytest.mark.parametrize("gated", [False, True])
def test_recurrent_step(dtype, Dk, Dv, gated):
    inp = make_inputs(B=3, T=1, H=4, Dk=Dk, Dv=Dv, dtype=dtype, gated=gated, s0=True, seed=51)
    Or, Sr = run_oracle(inp)
    d = inp.to(DEV)
    S = d.S0.clone()
    o = gdn.gdn_recurrent_step(d.q[:, 0].contiguous(), d.k[:, 0].contiguous(), d.v[:, 0].contiguous(),
                               None if d.log_alpha is None else d.log_alpha[:, 0].contiguous(),
                               d.beta[:, 0].contiguous(), S)
    torch.cuda.synchronize()
    assert rel(o.double().cpu().numpy(), Or[:, 0]) <= TOL[dtype]
    assert rel(S.double().cpu().numpy(), Sr) <= 1e-5


def test_recurrent_step_largest_state():
    # the largest state gdn_recurrent_step accepts: N = 65535 sequences (the
    # grid limit), H = 2, Dk = Dv = 128, just under 2^31 fp32 elements (byte
    # offsets past 2^32). Drawn on the device, checked by the oracle on the
    # first, a middle and the last sequence
    N, H, D = 65535, 2, 128
    assert N * H * D * D <= 2**31 - 1 < N * (H + 1) * D * D
    say(f"[gpu] largest step state N={N} H={H} D={D} bf16 seed=93")
    d = make_inputs(B=N, T=1, H=H, Dk=D, Dv=D, dtype="bf16", seed=93, device=DEV)
    seqs = [0, N // 2, N - 1]
    sub = lambda t: t[seqs].cpu()
    Or, Sr = oracle.forward(sub(d.q), sub(d.k), sub(d.v), sub(d.log_alpha), sub(d.beta),
                            d.S0[seqs].cpu(), None)
    o = gdn.gdn_recurrent_step(d.q[:, 0].contiguous(), d.k[:, 0].contiguous(),
                               d.v[:, 0].contiguous(), d.log_alpha[:, 0].contiguous(),
                               d.beta[:, 0].contiguous(), d.S0)
    torch.cuda.synchronize()
    eo = rel(o[seqs].double().cpu().numpy(), Or[:, 0])
    es = rel(d.S0[seqs].double().cpu().numpy(), Sr)
    say(f"      max rel err o {eo:.3e}  S {es:.3e}")
    assert eo <= TOL["bf16"] and es <= 1e-5, (eo, es)
    del d, o
    torch.cuda.empty_cache()


def test_recurrent_step_decode_batch():
    """The decode batch that bench.py --recurrent 64 times: N = 64 sequences, H = 16,
    Dk = Dv = 128, bf16, every workgroup of the launch."""
    inp = make_inputs(B=64, T=1, H=16, Dk=128, Dv=128, dtype="bf16", gated=True, s0=True, seed=71)
    Or, Sr = run_oracle(inp)
    d = inp.to(DEV)
    S = d.S0.clone()
    o = gdn.gdn_recurrent_step(d.q[:, 0].contiguous(), d.k[:, 0].contiguous(), d.v[:, 0].contiguous(),
                               d.log_alpha[:, 0].contiguous(), d.beta[:, 0].contiguous(), S)
    torch.cuda.synchronize()
    eo, es = rel(o.double().cpu().numpy(), Or[:, 0]), rel(S.double().cpu().numpy(), Sr)
    say(f"[gpu] decode batch 64x16 D128 bf16: o {eo:.3e}  S {es:.3e}")
    assert eo <= TOL["bf16"] and es <= 1e-5


@pytest.mark.parametrize("dtype,D", [("f32", 64), ("bf16", 128)])
def test_prefill_then_decode(dtype, D):
    T = 150
    inp = make_inputs(B=2, T=T + 3, H=2, Dk=D, Dv=D, dtype=dtype, gated=True, s0=True, seed=61)
    Or, Sr = run_oracle(inp)
    d = inp.to(DEV)
    O, S = gdn.gdn_chunk_fwd(d.q[:, :T].contiguous(), d.k[:, :T].contiguous(),
                             d.v[:, :T].contiguous(), d.log_alpha[:, :T].contiguous(),
                             d.beta[:, :T].contiguous(), d.S0)
    outs = [O.double().cpu().numpy()]
    for t in range(T, T + 3):
        o = gdn.gdn_recurrent_step(d.q[:, t].contiguous(), d.k[:, t].contiguous(),
                                   d.v[:, t].contiguous(), d.log_alpha[:, t].contiguous(),
                                   d.beta[:, t].contiguous(), S)
        outs.append(o.double().cpu().numpy()[:, None])
    torch.cuda.synchronize()
    assert rel(np.concatenate(outs, 1), Or) <= TOL[dtype]
    assert rel(S.double().cpu().numpy(), Sr) <= TOL[dtype]
