"""Throughput of the chunkwise gated delta rule forward on one MI355X.

One step = one gdn_chunk_fwd call (prep and scan kernels) over the
whole batch of the headline workload: B=4, H=16, T=4096, Dk=Dv=128, chunk 64,
bf16 q/k/v/O, fp32 gates and state, S0 = 0, seeded synthetic inputs already
resident in HBM.  Prints ONE JSON line.

  value         tokens/s = B*T / (mean device time of one step)
  roofline      the whole call (every kernel of one gdn_chunk_fwd): the method's
                algorithmic bytes (or flops) per call over the mean HIP-event
                duration of a call, against MI355X's published peak; traffic is
                the sum of the call's kernels' measured HBM bytes
  roofline_dominant  the same for the longest kernel alone (its own algorithmic
                bytes over its mean duration, timed inside the library)
  kernels       per-kernel mean duration and roofline fraction
  cpu_baseline  the fp64 oracle on the host cores over a bounded sample of the
                same inputs, threaded and single-threaded

Options: --gpus (only 1), --steps, --warmup, --workload, --no-flush,
--profile-steps, --cpu-sample (heads per batch row the oracle runs on, 0 = skip),
--rule (delta: gdn_chunk_fwd, the default; mamba2: gdn_mamba2_chunk_fwd, the
scalar-gated rule without the erase term; gla: gdn_gla_chunk_fwd, one gate per
key channel and no erase term, the gate drawn per channel; each on the same
workload shape),
--split L (delta rule, fixed-length workloads: gdn_chunk_fwd_split with spans of
L chunks instead of gdn_chunk_fwd; its kernels are prep, the span-map scan,
the span chaining and the output scan), --heads H (override the workload's head
count, e.g. to measure the split where there are few units),
--recurrent N (instead: the single-token step, gdn_recurrent_step, over a decode
batch of N sequences with the workload's H, Dk, Dv and dtype; its own JSON line).
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # bytes/s, MI355X HBM3E
MFMA_PEAK = {"bf16": 2.5e15, "f32": 157.3e12}   # dense flop/s
METRIC = "tokens/sec gated-DeltaNet chunk fwd (H=16,T=4096,D=128,bf16); % roofline"
BASELINE_NOTE = ("the pages that define the method quote no throughput and no hardware, "
                 "so there is no published figure to compare with (vs_baseline null)")


def per_kernel_work(B, T, H, Dk, Dv, C, s_in, n_seqs, has_s0, gated, rule="delta"):
    """Algorithmic bytes and flops of each kernel and of the whole call.

    Bytes count only the operation's own inputs and outputs that a kernel
    touches (q, k, v, gates, O, S0, S_T); per-chunk intermediates (g and
    T diag(beta), written by prep and read by scan) are implementation traffic
    and are not counted.  Flops count dense 16x16 tiles of every product.
    The path's flops are the method's count per token-head,
    6 Dk Dv + 2C (3 Dk + 2 Dv) + C^2 / 3 (K K^T, W, Q K^T; U, P V'; inverse).
    The no-erase rule (mamba2) has no prediction and no inverse: its path is
    4 Dk Dv + 2C (Dk + Dv) per token-head (Q S^T, the state update, Q K^T, P V),
    and its per-chunk kernel ("prep" here: the gates kernel) reads only the
    gates.  The per-channel rule (gla) has the same flops; its gate is Dk fp32
    values per token-head, and its per-chunk kernel (the GLA prep) reads q, k
    and the gates and forms Q K^T."""
    th = B * T * H                      # token-heads
    gate_b = 4 + (4 if gated else 0)    # beta (+ log alpha), fp32
    state_b = n_seqs * H * Dv * Dk * 4 * (2 if has_s0 else 1)
    prep_b = th * (Dk * s_in + gate_b)
    scan_b = th * (2 * Dk + 2 * Dv) * s_in + state_b
    path_b = th * ((2 * Dk + 2 * Dv) * s_in + gate_b) + state_b
    prep_f = th * (2 * C * Dk + C * C / 3)
    scan_f = th * (6 * Dk * Dv + 2 * C * (Dk + 2 * Dv))
    path_f = th * (6 * Dk * Dv + 2 * C * (3 * Dk + 2 * Dv) + C * C / 3)
    if rule == "mamba2":
        prep_b, prep_f = th * gate_b, th * 8
        scan_f = th * (4 * Dk * Dv + 2 * C * (Dk + Dv))
        path_f = scan_f + prep_f
    elif rule == "gla":
        gate_b = 4 + (4 * Dk if gated else 0)
        path_b = th * ((2 * Dk + 2 * Dv) * s_in + gate_b) + state_b
        prep_b = th * (2 * Dk * s_in + gate_b)
        prep_f = th * (2 * C * Dk + 4 * Dk)
        scan_f = th * (4 * Dk * Dv + 2 * C * Dv)
        path_f = scan_f + prep_f
    return {"prep": (prep_b, prep_f), "scan": (scan_b, scan_f), "path": (path_b, path_f)}


TRAFFIC_DIR = os.path.join(ROOT, "profiles")


def kernel_sources_sha256():
    import hashlib
    d = os.path.join(ROOT, "gated_delta_rule_16_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        if f.endswith((".h", ".hip")):
            h.update(f.encode())
            with open(os.path.join(d, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload, kernel):
    """HBM bytes per launch of ``kernel`` from the committed FETCH_SIZE / WRITE_SIZE
    counter record for ``workload``, each counter scaled by what it read for a
    plain copy of known size; None when there is no record or the kernel sources
    changed since it was taken."""
    path = os.path.join(TRAFFIC_DIR, f"traffic_{workload.replace('gdn_', '', 1)}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("sources_sha256") != kernel_sources_sha256() or kernel not in rec.get("kernels", {}):
        return None
    cal = rec["copy_calibration"]
    f_fetch = cal["read_bytes"] / (cal["fetch_kib"] * 1024.0)
    f_write = cal["write_bytes"] / (cal["write_kib"] * 1024.0)
    k = rec["kernels"][kernel]
    return int(k["fetch_kib"] * 1024.0 * f_fetch + k["write_kib"] * 1024.0 * f_write)


def roofline(name, bytes_, flops, seconds, dtype):
    t_hbm, t_mma = bytes_ / HBM_PEAK, flops / MFMA_PEAK[dtype]
    if t_hbm >= t_mma:
        ach = bytes_ / seconds / 1e9
        return {"kernel": name, "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK / 1e9,
                "unit": "GB/s", "frac": round(ach / (HBM_PEAK / 1e9), 4), "traffic": None,
                "alg_bytes": int(bytes_), "alg_flops": int(flops), "ms": round(seconds * 1e3, 4)}
    ach = flops / seconds / 1e12
    return {"kernel": name, "bound": "mfma", "achieved": round(ach, 2),
            "peak": MFMA_PEAK[dtype] / 1e12, "unit": "TFLOP/s",
            "frac": round(ach / (MFMA_PEAK[dtype] / 1e12), 4), "traffic": None,
            "alg_bytes": int(bytes_), "alg_flops": int(flops), "ms": round(seconds * 1e3, 4)}


def usable_cores() -> int:
    """Host cores this process may run on (its CPU affinity set)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_baseline(inp, heads_per_row: int, single_heads: int = 2, no_erase: bool = False):
    """The fp64 oracle timed on the host cores over a bounded sample: every
    batch row, the first ``heads_per_row`` heads, all tokens (threaded over
    (sequence, head) units), and again on one thread over the first
    ``single_heads`` of those heads."""
    import numpy as np
    import oracle
    H = inp.q.shape[2]
    tokens = inp.q.shape[0] * inp.q.shape[1]

    def run(nh, n_threads):
        hs = list(range(min(nh, H)))
        sl = lambda t: None if t is None else t[:, :, hs].contiguous()
        q, k, v, la, be = (sl(t) for t in (inp.q, inp.k, inp.v, inp.log_alpha, inp.beta))
        s0 = None if inp.S0 is None else inp.S0[:, hs].contiguous()
        q, k, v = (np.ascontiguousarray(t.double().numpy()) for t in (q, k, v))
        la = None if la is None else np.ascontiguousarray(la.double().numpy())
        be = np.ascontiguousarray(be.double().numpy())
        t0 = time.perf_counter()
        _, _, nt = oracle.forward(q, k, v, la, be, s0, inp.cu_seqlens, n_threads=n_threads,
                                  return_threads=True, no_erase=no_erase)
        return len(hs), nt, time.perf_counter() - t0

    nh, nt, dt = run(heads_per_row, 0)
    nh1, _, dt1 = run(single_heads, 1)
    # scale to the full workload's tokens/s: a sample of nh heads of H
    return {"value": round(tokens * nh / H / dt, 1), "unit": "tokens/s", "cores": nt,
            "kind": "oracle",
            "sample": f"fp64 token recurrence over all {inp.q.shape[0]}x{inp.q.shape[1]} tokens "
                      f"of heads 0..{nh - 1} of {H} ({tokens * nh} token-heads, "
                      f"{dt:.2f} s wall on {nt} threads); tokens/s scaled by {nh}/{H}",
            "host_cores": usable_cores(),
            "single_thread": {"value": round(tokens * nh1 / H / dt1, 1), "unit": "tokens/s",
                              "seconds": round(dt1, 3),
                              "sample": f"heads 0..{nh1 - 1} of {H}, all tokens, one thread; "
                                        f"tokens/s scaled by {nh1}/{H}"}}


def bench_recurrent(args, w):
    """Tokens/s of the single-token step over a decode batch: N sequences of one
    token, H heads, the state read and written in place each step (HBM-bound:
    2 Dv Dk 4 bytes of state per sequence-head and token)."""
    import torch
    import gated_delta_rule_16_amd as gdn
    from gated_delta_rule_16_amd.inputs import make_inputs
    N, H = args.recurrent, w.H
    inp = make_inputs(B=N, T=1, H=H, Dk=w.Dk, Dv=w.Dv, dtype=w.dtype, gated=True, s0=True, seed=71)
    dev = torch.device("cuda:0")
    d = inp.to(dev)
    q, k, v = (t[:, 0].contiguous() for t in (d.q, d.k, d.v))
    la, be = d.log_alpha[:, 0].contiguous(), d.beta[:, 0].contiguous()
    S = d.S0.clone()
    o = torch.empty(N, H, w.Dv, device=dev, dtype=q.dtype)
    flush = None if args.no_flush else torch.zeros(512 << 18, device=dev, dtype=torch.float32)
    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        if flush is not None:
            flush.sum()
        gdn.gdn_recurrent_step(q, k, v, la, be, S, o=o, stream=stream)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        if flush is not None:
            flush.sum()
        starts[i].record(stream)
        gdn.gdn_recurrent_step(q, k, v, la, be, S, o=o, stream=stream)
        ends[i].record(stream)
    torch.cuda.synchronize()
    step_ms = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    ms = statistics.mean(step_ms)
    s_in = 2 if w.dtype == "bf16" else 4
    nbytes = N * H * (2 * w.Dv * w.Dk * 4 + (2 * w.Dk + 2 * w.Dv) * s_in + 8)
    flops = N * H * 8 * w.Dv * w.Dk
    rl = roofline("recurrent_step", nbytes, flops, ms / 1e3, w.dtype)
    out = {
        "metric": "tokens/sec gated-DeltaNet single-token step (decode)", "value": round(N / (ms / 1e3), 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": f"decode_n{N}_h{H}_dk{w.Dk}_dv{w.Dv}", "N": N, "H": H, "Dk": w.Dk,
                   "Dv": w.Dv, "state": "fp32", "flush_l2_mall": flush is not None},
        "roofline": rl,
        "step_ms": {"median": round(statistics.median(step_ms), 5), "min": round(min(step_ms), 5),
                    "max": round(max(step_ms), 5)},
        "cpu_baseline": None,
        "baseline_note": BASELINE_NOTE,
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gdn_bf16_b4_h16_t4096_d128")
    ap.add_argument("--no-flush", action="store_true",
                    help="do not overwrite a 512 MB buffer (L2 + MALL) before each step")
    ap.add_argument("--profile-steps", type=int, default=20)
    ap.add_argument("--cpu-sample", type=int, default=16,
                    help="heads per batch row for the oracle baseline (0 = skip)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MB",
                    help="after timing, copy an MB-megabyte buffer a few times (a plain copy "
                         "kernel of known traffic, the scale for hardware byte counters)")
    ap.add_argument("--rule", choices=["delta", "mamba2", "gla"], default="delta",
                    help="update rule: delta (gdn_chunk_fwd), mamba2 (gdn_mamba2_chunk_fwd) "
                         "or gla (gdn_gla_chunk_fwd)")
    ap.add_argument("--split", type=int, default=0, metavar="L",
                    help="delta rule: gdn_chunk_fwd_split with spans of L chunks")
    ap.add_argument("--heads", type=int, default=0, help="override the workload's head count")
    ap.add_argument("--recurrent", type=int, default=0, metavar="N",
                    help="time gdn_recurrent_step over N sequences instead (one token each)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only; --gpus {args.gpus} is not supported "
              "(the (sequence, head) units shard across GPUs with no communication, see the "
              "design notes)", file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_delta_rule_16_amd as gdn
    from gated_delta_rule_16_amd.inputs import WORKLOADS, workload_inputs

    assert torch.cuda.is_available(), "bench.py needs a ROCm GPU"
    w = WORKLOADS[args.workload]
    if args.recurrent > 0:
        bench_recurrent(args, w)
        return
    if args.heads > 0:
        import dataclasses
        w = dataclasses.replace(w, H=args.heads)
        from gated_delta_rule_16_amd.inputs import make_inputs
        inp = make_inputs(w.B, w.T, w.H, w.Dk, w.Dv, dtype=w.dtype, gated=w.gated, s0=w.s0,
                          seed=w.seed, C=w.C, gate_channels=args.rule == "gla")
    else:
        inp = workload_inputs(args.workload, gate_channels=args.rule == "gla")
    dev = torch.device("cuda:0")
    d = inp.to(dev)
    B, T, H = inp.q.shape[:3]
    N = inp.n_seqs
    tdt = inp.q.dtype
    O = torch.empty(B, T, H, w.Dv, device=dev, dtype=tdt)
    S_T = torch.empty(N, H, w.Dv, w.Dk, device=dev, dtype=torch.float32)
    rule = {"delta": gdn.GDN_RULE_DELTA, "mamba2": gdn.GDN_RULE_MAMBA2,
            "gla": gdn.GDN_RULE_GLA}[args.rule]
    fwd = {"delta": gdn.gdn_chunk_fwd, "mamba2": gdn.gdn_mamba2_chunk_fwd,
           "gla": gdn.gdn_gla_chunk_fwd}[args.rule]
    # span length of the split scan: --split, else what gdn_chunk_fwd takes by
    # itself for these sizes (0: the plain scan), so that the per-kernel times
    # below come from the path the timed steps ran
    auto_split = 0
    if args.rule == "delta" and args.split == 0:
        auto_split = gdn.gdn_chunk_fwd_auto_span_chunks(B, T, H, w.Dk, w.Dv, w.C,
                                                        0 if inp.cu_seqlens is None else N, tdt)
    span = args.split or auto_split
    if args.split > 0:
        assert args.rule == "delta" and inp.cu_seqlens is None, "--split: delta rule, fixed length"
        n_ws = gdn.gdn_chunk_fwd_split_workspace_bytes(B, T, H, w.Dk, w.Dv, w.C, args.split, tdt)
    else:
        n_ws = gdn.gdn_rule_workspace_bytes(rule, B, T, H, w.Dk, w.Dv, w.C,
                                            0 if inp.cu_seqlens is None else N, tdt)
    ws = torch.empty(n_ws, device=dev, dtype=torch.uint8)
    # Cache eviction between steps: one pass reading 512 MB (twice the MALL)
    # leaves L2 and MALL holding clean lines of this buffer, so every step reads
    # its inputs from HBM without paying write-backs that belong to other work.
    # fp32, so that the sum is one read pass with no widened temporary (an int32
    # sum would first write a 1 GB int64 copy, whose dirty lines land in the
    # timed kernels)
    flush = None if args.no_flush else torch.zeros(512 << 18, device=dev, dtype=torch.float32)

    def evict():
        if flush is not None:
            flush.sum()
    stream = torch.cuda.current_stream(dev)

    def step():
        if args.split > 0:
            gdn.gdn_chunk_fwd_split(d.q, d.k, d.v, d.log_alpha, d.beta, d.S0, span_chunks=args.split,
                                    chunk_size=w.C, O=O, S_T=S_T, workspace=ws, stream=stream)
        else:
            fwd(d.q, d.k, d.v, d.log_alpha, d.beta, d.S0, d.cu_seqlens, chunk_size=w.C,
                O=O, S_T=S_T, workspace=ws, stream=stream)

    for _ in range(args.warmup):
        evict()
        step()
    torch.cuda.synchronize()

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        evict()                 # every step reads its inputs from HBM
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    ms = statistics.mean(step_ms)
    tokens = B * T
    value = tokens / (ms / 1e3)

    # per-kernel device time (HIP events on the launch stream, inside the library)
    if span > 0:
        kms = {"prep": [], "span_maps": [], "span_chain": [], "scan": []}
    else:
        kms = {"table": [], "prep": [], "scan": [], "unused": []}
    for _ in range(args.profile_steps):
        evict()
        if span > 0:
            _, _, t = gdn.gdn_chunk_fwd_split(d.q, d.k, d.v, d.log_alpha, d.beta, d.S0,
                                              span_chunks=span, chunk_size=w.C, O=O,
                                              S_T=S_T, workspace=ws, stream=stream, profiled=True)
        else:
            _, _, t = gdn.gdn_rule_chunk_fwd_profiled(rule, d.q, d.k, d.v, d.log_alpha, d.beta,
                                                      d.S0, d.cu_seqlens, chunk_size=w.C, O=O,
                                                      S_T=S_T, workspace=ws, stream=stream)
        for key, x in zip(kms, t):
            kms[key].append(x)
    kms.pop("unused", None)
    kmean = {k_: (statistics.mean(v_) if v_ else 0.0) for k_, v_ in kms.items()}

    s_in = 2 if w.dtype == "bf16" else 4
    work = per_kernel_work(B, T, H, w.Dk, w.Dv, w.C, s_in, N, inp.S0 is not None,
                           inp.log_alpha is not None, args.rule)
    dom = max((k_ for k_ in ("prep", "scan") if k_ in kmean), key=lambda k_: kmean[k_])
    rl_dom = roofline(dom, *work[dom], kmean[dom] / 1e3, w.dtype)
    tkey = args.workload if args.rule == "delta" else f"{args.rule}_{args.workload}"
    if args.heads > 0:   # the counter records hold the workloads' own head counts
        tkey = f"{tkey}_h{args.heads}"
    rl_dom["traffic"] = measured_traffic(tkey, dom)
    # the metric is the call's % roofline: the whole call is the headline
    rl = roofline("call (" + " + ".join(k_ for k_ in kms if kmean[k_] > 0) + ")", *work["path"],
                  ms / 1e3, w.dtype)
    parts = [measured_traffic(tkey, k_) for k_ in kms if kmean[k_] > 0]
    rl["traffic"] = None if any(p is None for p in parts) else sum(parts)
    kernels = {k_: {"ms": round(kmean[k_], 4),
                    **({"frac": roofline(k_, *work[k_], kmean[k_] / 1e3, w.dtype)["frac"]}
                       if k_ in work and kmean[k_] > 0 else {})}
               for k_ in kms}

    if args.copy_calibration > 0:
        nbytes = args.copy_calibration << 20
        src = torch.ones(nbytes // 4, device=dev, dtype=torch.float32)
        dst = torch.empty_like(src)
        for _ in range(3):
            evict()
            torch.mul(src, 1.0, out=dst)      # an elementwise kernel: reads and writes nbytes
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if args.cpu_sample > 0:
        cpu = cpu_baseline(inp, args.cpu_sample, no_erase=args.rule != "delta")

    headline = (args.workload == ap.get_default("workload") and args.rule == "delta"
                and args.split == 0 and args.heads == 0)
    metric = METRIC if headline else f"tokens/sec gated-DeltaNet chunk fwd ({args.workload})"
    if args.rule == "mamba2":
        metric = f"tokens/sec Mamba2 (scalar gate, no erase) chunk fwd ({args.workload})"
    elif args.rule == "gla":
        metric = f"tokens/sec GLA (per-channel gate, no erase) chunk fwd ({args.workload})"
    out = {
        "metric": metric,
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": args.workload + (f"_h{H}" if args.heads > 0 else ""),
                   "rule": args.rule, "split_span_chunks": span or None,
                   "split": "forced" if args.split else ("auto" if auto_split else None), "B": B, "T": T, "H": H,
                   "Dk": w.Dk, "Dv": w.Dv,
                   "chunk": w.C, "state": "fp32", "S0": inp.S0 is not None,
                   "flush_l2_mall": flush is not None},
        "roofline": rl, "roofline_dominant": rl_dom, "kernels": kernels,
        "step_ms": {"median": round(statistics.median(step_ms), 4), "min": round(min(step_ms), 4),
                    "max": round(max(step_ms), 4)},
        "wall_s_timed_loop": round(wall, 4),
        "cpu_baseline": cpu,
        "baseline_note": BASELINE_NOTE,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
