"""The C ABI library on the CPU: it loads, exports every declared symbol, and
rejects bad arguments on the host before touching the GPU (no compute call
is made here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

GDN_OK, GDN_ERR_NULL, GDN_ERR_SHAPE, GDN_ERR_UNSUPPORTED, GDN_ERR_WORKSPACE = 0, 1, 2, 3, 4
F32, BF16 = 0, 1


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    import gated_delta_rule_16_amd as gdn
    if not os.path.exists(gdn.LIB_PATH):
        pytest.fail("libgdn.so is not built (run __graft_entry__.build())")
    return gdn.load_library()


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("gdn_chunk_fwd", "gdn_recurrent_step", "gdn_chunk_fwd_workspace_bytes",
              "gdn_status_string", "gdn_chunk_fwd_supported"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, f"not exported: {missing}"


def test_status_strings(lib):
    for code in range(8):
        s = lib.gdn_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.gdn_status_string(99).decode() == "unknown status"


def test_supported_instantiations(lib):
    yes = [(16, 16, 16, F32), (64, 64, 16, F32), (64, 64, 64, F32), (128, 128, 64, BF16),
           (128, 256, 64, BF16), (128, 128, 64, F32), (128, 256, 64, F32)]
    for a in yes:
        assert lib.gdn_chunk_fwd_supported(*a) == 1, a
    for a in [(128, 128, 32, BF16), (64, 64, 64, BF16), (96, 96, 64, F32), (128, 128, 64, 7)]:
        assert lib.gdn_chunk_fwd_supported(*a) == 0, a


def test_rule_queries(lib):
    RULE_DELTA, RULE_MAMBA2 = 0, 1
    for a in [(128, 128, 64, BF16), (128, 256, 64, BF16), (64, 64, 64, F32), (16, 16, 16, F32)]:
        assert lib.gdn_rule_supported(RULE_MAMBA2, *a) == 1, a
        assert lib.gdn_rule_supported(RULE_DELTA, *a) == lib.gdn_chunk_fwd_supported(*a)
    assert lib.gdn_rule_supported(RULE_MAMBA2, 64, 64, 16, F32) == 0
    RULE_GLA = 2
    for a in [(128, 128, 64, BF16), (128, 256, 64, BF16), (64, 64, 64, F32), (16, 16, 16, F32)]:
        assert lib.gdn_rule_supported(RULE_GLA, *a) == 1, a
    # GLA: e^{b_n} per key channel, P~ blocks, and decayed copies of q and k
    g = lib.gdn_rule_workspace_bytes(RULE_GLA, 4, 4096, 16, 128, 128, 64, 0, BF16)
    assert g >= 4 * 64 * 16 * (128 * 4 + 6 * 1024) + 2 * 4 * 4096 * 16 * 128 * 2
    assert lib.gdn_rule_supported(9, 128, 128, 64, BF16) == 0
    f = lib.gdn_rule_workspace_bytes
    assert f(RULE_DELTA, 4, 4096, 16, 128, 128, 64, 0, BF16) == \
        lib.gdn_chunk_fwd_workspace_bytes(4, 4096, 16, 128, 128, 64, 0, BF16)
    # no-erase: four fp32 gate rows per chunk and no Tb
    slots, H, C = 4 * 64, 16, 64
    assert f(RULE_MAMBA2, 4, 4096, 16, 128, 128, 64, 0, BF16) == slots * H * 4 * C * 4
    assert f(9, 4, 4096, 16, 128, 128, 64, 0, BF16) == 0


def test_mamba2_argument_errors(lib):
    p = ctypes.c_void_p(1 << 20)

    def call(**kw):
        a = dict(q=p, k=p, v=p, la=None, beta=p, S0=None, cu=None, n=0, O=p, S_T=None,
                 B=1, T=128, H=1, Dk=16, Dv=16, C=16, dt=F32, ws=p, wsb=0, st=None)
        a.update(kw)
        return lib.gdn_mamba2_chunk_fwd(a["q"], a["k"], a["v"], a["la"], a["beta"], a["S0"],
                                        a["cu"], a["n"], a["O"], a["S_T"], a["B"], a["T"],
                                        a["H"], a["Dk"], a["Dv"], a["C"], a["dt"], a["ws"],
                                        a["wsb"], a["st"])
    assert call(q=None) == GDN_ERR_NULL
    assert call(ws=None, wsb=1 << 30) == GDN_ERR_NULL
    assert call(wsb=16) == GDN_ERR_WORKSPACE          # beta NULL is allowed, the size is not
    assert call(beta=None, wsb=16) == GDN_ERR_WORKSPACE
    assert call(Dk=64, Dv=64, C=16) == GDN_ERR_UNSUPPORTED
    assert call(B=0) == GDN_ERR_SHAPE
    ms = (ctypes.c_float * 4)()
    args = [p, p, p, None, p, None, None, 0, p, None, 1, 128, 1, 16, 16, 16, F32, p, 16, None]
    assert lib.gdn_rule_chunk_fwd_profiled(7, *args, ms) == GDN_ERR_UNSUPPORTED
    assert lib.gdn_rule_chunk_fwd_profiled(1, *args, None) == GDN_ERR_NULL


def test_workspace_bytes(lib):
    f = lib.gdn_chunk_fwd_workspace_bytes
    a = f(4, 4096, 16, 128, 128, 64, 0, BF16)
    b = f(4, 4096, 16, 128, 128, 64, 0, F32)
    assert a > 0 and b > a
    # at least the per-chunk intermediates: g, exp(g), exp(g_n - g) (fp32) and
    # the lower block triangle of T diag(beta) (bf16: six 1 KB operand blocks
    # for a 64-token chunk)
    slots, H, C = 4 * 64, 16, 64
    assert a >= slots * H * (3 * C * 4 + 6 * 1024)
    assert f(1, 1000, 16, 128, 256, 64, 5, BF16) > 0          # packed batch
    assert f(1, 0, 4, 64, 64, 64, 0, F32) >= 0                # empty sequence
    assert f(0, 128, 1, 16, 16, 16, 0, F32) == 0              # bad B
    assert f(2, 128, 1, 16, 16, 16, 3, F32) == 0              # packed needs B = 1
    assert f(1, 128, 1, 96, 96, 64, 0, F32) == 0              # unsupported size
    assert f(1, 1 << 30, 16, 128, 128, 64, 0, BF16) == 0      # > 2^31 elements


def _fwd(lib, **kw):
    """gdn_chunk_fwd with fake, never dereferenced pointers (argument checks
    return before any HIP call)."""
    p = ctypes.c_void_p(1 << 20)       # 16-byte aligned dummy address
    a = dict(q=p, k=p, v=p, la=None, beta=p, S0=None, cu=None, n=0, O=p, S_T=None,
             B=1, T=128, H=1, Dk=16, Dv=16, C=16, dt=F32, ws=p, wsb=1 << 40, st=None)
    a.update(kw)
    return lib.gdn_chunk_fwd(a["q"], a["k"], a["v"], a["la"], a["beta"], a["S0"], a["cu"], a["n"],
                             a["O"], a["S_T"], a["B"], a["T"], a["H"], a["Dk"], a["Dv"], a["C"],
                             a["dt"], a["ws"], a["wsb"], a["st"])


def test_chunk_fwd_argument_errors(lib):
    for name in ("q", "k", "v", "beta", "O", "ws"):
        assert _fwd(lib, **{name: None}) == GDN_ERR_NULL, name
    assert _fwd(lib, B=0) == GDN_ERR_SHAPE
    assert _fwd(lib, H=0) == GDN_ERR_SHAPE
    assert _fwd(lib, T=-1) == GDN_ERR_SHAPE
    assert _fwd(lib, cu=ctypes.c_void_p(1 << 20), n=0) == GDN_ERR_SHAPE     # packed, no sequences
    assert _fwd(lib, cu=ctypes.c_void_p(1 << 20), n=2, B=2) == GDN_ERR_SHAPE
    assert _fwd(lib, Dk=32, Dv=32) == GDN_ERR_UNSUPPORTED
    assert _fwd(lib, C=32) == GDN_ERR_UNSUPPORTED
    assert _fwd(lib, dt=BF16) == GDN_ERR_UNSUPPORTED          # (16, 16, 16) exists in fp32 only
    assert _fwd(lib, dt=5) == GDN_ERR_UNSUPPORTED
    assert _fwd(lib, wsb=16) == GDN_ERR_WORKSPACE
    assert _fwd(lib, q=ctypes.c_void_p((1 << 20) + 4)) == GDN_ERR_SHAPE      # misaligned
    assert _fwd(lib, S0=ctypes.c_void_p((1 << 20) + 4)) == GDN_ERR_SHAPE
    assert _fwd(lib, S_T=ctypes.c_void_p((1 << 20) + 8)) == GDN_ERR_SHAPE
    need = lib.gdn_chunk_fwd_workspace_bytes(1, 128, 1, 16, 16, 16, 0, F32)
    assert _fwd(lib, wsb=need - 1) == GDN_ERR_WORKSPACE
    # one past the size limits: a token tensor of 2^31 elements; a chunk of one
    # tensor (C * H * Dv * element size) past 2^31 - 1 bytes
    big = dict(B=1, T=1024, H=16384, Dk=128, Dv=128, C=64, dt=BF16)
    assert _fwd(lib, **big) == GDN_ERR_SHAPE
    assert lib.gdn_chunk_fwd_workspace_bytes(1, 1024, 16384, 128, 128, 64, 0, BF16) == 0
    assert _fwd(lib, B=1, T=1, H=65535, Dk=128, Dv=256, C=64, dt=F32) == GDN_ERR_SHAPE


def test_noalloc_argument_errors(lib):
    """gdn_chunk_fwd_noalloc checks its arguments, and its scratch limit, on the
    host before any HIP call (fake, never dereferenced pointers)."""
    GDN_ERR_SCRATCH_LIMIT = 7
    p = ctypes.c_void_p(1 << 20)

    def call(**kw):
        a = dict(q=p, k=p, v=p, la=None, beta=p, S0=None, cu=None, n=0, O=p, S_T=None,
                 B=1, T=128, H=1, Dk=16, Dv=16, C=16, dt=F32, st=None)
        a.update(kw)
        return lib.gdn_chunk_fwd_noalloc(a["q"], a["k"], a["v"], a["la"], a["beta"], a["S0"],
                                         a["cu"], a["n"], a["O"], a["S_T"], a["B"], a["T"],
                                         a["H"], a["Dk"], a["Dv"], a["C"], a["dt"], a["st"])
    assert call(q=None) == GDN_ERR_NULL
    assert call(B=0) == GDN_ERR_SHAPE
    assert call(Dk=32, Dv=32) == GDN_ERR_UNSUPPORTED
    assert call(O=ctypes.c_void_p((1 << 20) + 4)) == GDN_ERR_SHAPE
    # the long-context shape needs about 113 MB of intermediates: above the 64 MiB buffer
    long = dict(B=1, T=32768, H=32, Dk=128, Dv=128, C=64, dt=BF16)
    assert lib.gdn_chunk_fwd_workspace_bytes(1, 32768, 32, 128, 128, 64, 0, BF16) > 64 << 20
    assert call(**long) == GDN_ERR_SCRATCH_LIMIT
    assert "scratch" in lib.gdn_status_string(GDN_ERR_SCRATCH_LIMIT).decode()


def test_workspace_holds_the_automatic_split(lib):
    # The automatic split's choices on a device of 256 CUs (the count assumed
    # when no device answers), from the cost model in gdn_api.hip: few long
    # units split, into the span lengths measured best; many units, or
    # sequences too short for the three extra kernels to pay, do not
    auto = lib.gdn_chunk_fwd_auto_span_chunks
    assert auto(1, 32768, 4, 128, 128, 64, 0, BF16) == 32
    # 8 heads: spans of 32 chunks give 128 span-units, whose span maps run in
    # 128-column slices (one round of the device); spans of 64 give 64, in
    # 64-column ones
    assert auto(1, 32768, 8, 128, 128, 64, 0, BF16) == 32
    assert auto(1, 32768, 16, 128, 128, 64, 0, BF16) == 64
    assert auto(1, 4096, 4, 128, 128, 64, 0, BF16) == 8
    # the long workload: 256 plain workgroups fill the device, but each of its
    # 512 chunk steps then costs more than with few workgroups
    assert auto(1, 32768, 32, 128, 128, 64, 0, BF16) == 128
    # half as long: spans of 64 (measured 0.315 ms against 0.338 for the plain
    # scan, 0.371 at spans of 32 or 128); a quarter as long: not worth it
    assert auto(1, 16384, 32, 128, 128, 64, 0, BF16) == 64
    assert auto(1, 8192, 32, 128, 128, 64, 0, BF16) == 0
    assert auto(4, 4096, 16, 128, 128, 64, 0, BF16) == 0       # the headline workload
    assert auto(1, 2048, 16, 128, 128, 64, 0, BF16) == 0       # 32 chunks, 16 heads
    assert auto(2, 1024, 4, 64, 64, 64, 0, F32) == 2           # the fp32 D64 workload
    assert auto(1, 2048, 32, 64, 64, 64, 0, F32) == 0
    assert auto(1, 8192, 2, 128, 128, 64, 3, BF16) == 0        # packed batches never split
    assert auto(1, 8192, 2, 128, 128, 64, 0, F32) == 8         # fp32 D128 (16-column slices only)
    assert auto(1, 4096, 16, 128, 128, 64, 0, F32) == 0
    assert auto(1, 8192, 2, 100, 128, 64, 0, BF16) == 0        # unsupported sizes
    # gdn_chunk_fwd's workspace query is then the split scan's, equal to
    # gdn_chunk_fwd_split_workspace_bytes with that span length; otherwise the
    # plain layout, below any split's
    L = auto(1, 8192, 2, 128, 128, 64, 0, BF16)
    assert L > 0
    few = lib.gdn_chunk_fwd_workspace_bytes(1, 8192, 2, 128, 128, 64, 0, BF16)
    assert few == lib.gdn_chunk_fwd_split_workspace_bytes(1, 8192, 2, 128, 128, 64, L, BF16)
    P = -(-128 // L)
    assert few >= P * 2 * (256 + 128) * 128 * 4                 # span maps and starts, fp32
    many = lib.gdn_chunk_fwd_workspace_bytes(4, 4096, 16, 128, 128, 64, 0, BF16)
    assert many < lib.gdn_chunk_fwd_split_workspace_bytes(4, 4096, 16, 128, 128, 64, 64, BF16)
    # the scalar-gate and per-channel rules never split
    assert lib.gdn_rule_workspace_bytes(1, 1, 8192, 2, 128, 128, 64, 0, BF16) < few


def test_split_queries_and_errors(lib):
    f = lib.gdn_chunk_fwd_split_workspace_bytes
    n = f(1, 32768, 32, 128, 128, 64, 64, BF16)
    # prep's per-chunk data, the span maps [8 spans][32][256][128] and the span
    # starts [8][32][128][128], fp32
    assert n >= 8 * 32 * 256 * 128 * 4 + 8 * 32 * 128 * 128 * 4
    assert f(1, 32768, 32, 64, 64, 64, 64, F32) > 0           # fp32 Dk = Dv = 64, C = 64
    assert f(1, 32768, 32, 128, 128, 64, 64, F32) > 0         # fp32 Dk = Dv = 128
    assert f(1, 32768, 32, 128, 256, 64, 64, BF16) == 0       # not compiled: Dv = 256
    assert f(1, 32768, 32, 64, 64, 16, 64, F32) == 0          # not compiled: C = 16
    assert f(1, 32768, 32, 128, 128, 64, 0, BF16) == 0        # span_chunks >= 1
    p = ctypes.c_void_p(1 << 20)
    g = lib.gdn_chunk_fwd_split
    args = [p, p, p, None, p, None, p, None, 1, 128, 1, 128, 128, 64, BF16, 1, p, 1 << 40, None, None]
    bad = list(args); bad[0] = None
    assert g(*bad) == GDN_ERR_NULL
    bad = list(args); bad[15] = 0
    assert g(*bad) == GDN_ERR_SHAPE
    bad = list(args); bad[12] = 256
    assert g(*bad) == GDN_ERR_UNSUPPORTED
    bad = list(args); bad[17] = 16
    assert g(*bad) == GDN_ERR_WORKSPACE


def test_recurrent_step_argument_errors(lib):
    p = ctypes.c_void_p(1 << 20)
    f = lib.gdn_recurrent_step
    assert f(None, p, p, None, p, p, p, 1, 1, 16, 16, F32, None) == GDN_ERR_NULL
    assert f(p, p, p, None, None, p, p, 1, 1, 16, 16, F32, None) == GDN_ERR_NULL
    assert f(p, p, p, None, p, None, p, 1, 1, 16, 16, F32, None) == GDN_ERR_NULL
    assert f(p, p, p, None, p, p, p, 0, 1, 16, 16, F32, None) == GDN_ERR_SHAPE
    assert f(p, p, p, None, p, p, p, 1, 1, 48, 16, F32, None) == GDN_ERR_UNSUPPORTED
    assert f(p, p, p, None, p, p, p, 1, 1, 16, 16, 9, None) == GDN_ERR_UNSUPPORTED
    assert f(p, p, p, None, p, ctypes.c_void_p((1 << 20) + 4), p, 1, 1, 16, 16, F32, None) == GDN_ERR_SHAPE


def test_python_binding_fails_loudly_without_gpu_tensors(lib):
    import torch
    import gated_delta_rule_16_amd as gdn
    x = torch.zeros(1, 16, 1, 16)
    b = torch.zeros(1, 16, 1)
    with pytest.raises(ValueError):
        gdn.gdn_chunk_fwd(x, x, x, None, b, chunk_size=16, workspace=None,
                          O=torch.zeros(1, 16, 1, 16), S_T=torch.zeros(1, 1, 16, 16))


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus above 1 exits with status 2 and says so
    (before touching any device)."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
