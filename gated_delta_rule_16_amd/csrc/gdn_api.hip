// gdn_api.hip -- the C ABI of include/gdn.h: argument validation, workspace
// carving, the packed-batch chunk table and the kernel launches.
//
// Data flow of gdn_chunk_fwd (all on the caller's stream):
//   [packed batches only] chunk table  <- cu_seqlens
//   prep  (chunk slot, head)            g, Tb = T diag(beta)   (independent chunks)
//   scan  (Dv slice, head, sequence)    O, S_T                 (serial over chunks)
// gdn_mamba2_chunk_fwd (the no-erase rule) replaces prep by the gates kernel
// (g and beta per chunk; the scan's 64-column and fp32 slices form them
// themselves instead) and runs the same scan without the prediction step.
// gdn_gla_chunk_fwd (per-channel gate) replaces it by the GLA prep kernel
// (Q~, K^, P~ and the chunk decay per chunk) and runs the scan on those.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <iterator>
#include <cstdlib>
#include <cstring>

#include "../../include/gdn.h"
#include "gdn_device.h"
#include "gdn_gla_prep.h"
#include "gdn_prep.h"
#include "gdn_scan_cols.h"
#include "gdn_span.h"
#include "gdn_step.h"

namespace gdn {
namespace {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool debug_sync() {
    static const bool on = [] {
        const char* e = std::getenv("GDN_DEBUG_SYNC");
        return e && e[0] && e[0] != '0';
    }();
    return on;
}

gdn_status check_launch(hipStream_t stream) {
    if (hipGetLastError() != hipSuccess) return GDN_ERR_HIP;
    if (debug_sync()) {
        if (hipStreamSynchronize(stream) != hipSuccess) return GDN_ERR_HIP;
        if (hipGetLastError() != hipSuccess) return GDN_ERR_HIP;
    }
    return GDN_OK;
}

struct FwdArgs {
    const void *q, *k, *v;
    const float *log_alpha, *beta, *S0;
    const int32_t* cu;
    int n_seqs;
    void* O;
    float* S_T;
    int B, T, H, Dk, Dv, C;
    gdn_dtype dt;
    unsigned char* ws;
    hipStream_t stream;
};

// Workspace regions, in order; every region starts on a 256-byte boundary.
struct Layout {
    int64_t slots, N;
    size_t g, Tb, qt, kh, bounds, seq_slot, table, order, total;
};

Layout make_layout(int rule, int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv, int64_t C,
                   bool varlen, int64_t n_seqs, size_t es) {
    Layout L{};
    const int64_t cps = (T + C - 1) / C;
    L.N = varlen ? n_seqs : B;
    L.slots = varlen ? cps + n_seqs : B * cps;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t at = off; off = align_up(off + bytes); return at; };
    const size_t u = (size_t)(L.slots * H);
    // g, exp(g), exp(g_n - g) (and beta for kNoErase) per chunk; kGla: e^{b_n}
    L.g = take(u * gate_floats(rule, (int)C, (int)Dk) * sizeof(float));
    // Tb (delta rule) or P~ (kGla) blocks per chunk
    L.Tb = take(rule != kNoErase ? u * (size_t)tb_blocks((int)C, es == 2) * 1024 : 0);
    // kGla: Q~ and K^, token-major like q and k
    const size_t tok = (size_t)(varlen ? T : B * T) * H * Dk * es;
    L.qt = take(rule == kGla ? tok : 0);
    L.kh = take(rule == kGla ? tok : 0);
    if (varlen) {
        L.bounds = take((size_t)(n_seqs + 1) * sizeof(int));
        L.seq_slot = take((size_t)(n_seqs + 1) * sizeof(int));
        L.table = take((size_t)L.slots * 4 * sizeof(int));
        L.order = take((size_t)n_seqs * sizeof(int));
    }
    L.total = off;
    return L;
}

// Per-device caches of launch queries, safe for calls from several host
// threads (a value is the same whichever thread stores it); devices past the
// table are queried on every call.
constexpr int kMaxCachedDevices = 64;
int current_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    return dev;
}

// Compute units of the current device.
int device_cu_count() {
    static std::atomic<int> cached[kMaxCachedDevices] = {};
    const int dev = current_device();
    int n = dev < kMaxCachedDevices ? cached[dev].load(std::memory_order_relaxed) : 0;
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        if (dev < kMaxCachedDevices) cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Raises the dynamic LDS limit of one kernel instantiation once (gfx950
// allows up to 160 KB per workgroup).
template <auto Kernel>
void allow_smem(size_t bytes) {
    static const bool done = [bytes] {
        (void)hipFuncSetAttribute(reinterpret_cast<const void*>(Kernel),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
        return true;
    }();
    (void)done;
}

// Workgroups of `threads` threads and `smem` bytes of LDS that one CU holds at
// once (occupancy query, cached per kernel and device; at least 1).
template <auto Kernel>
int resident_per_cu(int threads, size_t smem) {
    static std::atomic<int> cached[kMaxCachedDevices] = {};
    const int dev = current_device();
    int nb = dev < kMaxCachedDevices ? cached[dev].load(std::memory_order_relaxed) : 0;
    if (nb <= 0) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, reinterpret_cast<const void*>(Kernel), threads, smem) !=
                hipSuccess ||
            nb < 1)
            nb = 1;
        if (dev < kMaxCachedDevices) cached[dev].store(nb, std::memory_order_relaxed);
    }
    return nb;
}

// Optional per-kernel timing: events recorded on the launch stream around each
// kernel (table, prep, scan).
struct KernelTimer {
    hipEvent_t ev[8];
    int n = 0;
    bool on = false;
    void mark(hipStream_t s) {
        if (on && n < 8) (void)hipEventRecord(ev[n++], s);
    }
};

// The column-wave scan over n_seqs sequences (or spans) of every head, with 32
// state columns per workgroup where that fits in LDS and still gives every CU
// a workgroup, else 16; 64 (bf16 outputs) where 32 would need more than one
// workgroup per CU.
template <typename T, int DK, int DV, int C, int RULE>
gdn_status launch_scan(const T* q, const T* k, const T* v, const float* S0, const SeqGeom& geom,
                       int H, int64_t n_seqs, const float* g_ws, const T* Tb_ws, T* O, float* S_T,
                       ScanRows rows, hipStream_t stream, KernelTimer* tm, RawGates raw = RawGates{}) {
    using C32 = ColCfg<T, DK, DV, C, (DV >= 32 ? 32 : 16), RULE>;
    using C16 = ColCfg<T, DK, DV, C, 16, RULE>;
    constexpr bool fit32 = DV >= 32 && C32::FITS, fit16 = C16::FITS;
    const int64_t units = (int64_t)H * n_seqs;
    auto launch_cols = [&](auto cfg_tag) -> gdn_status {
        using CC = decltype(cfg_tag);
        if constexpr (CC::FITS) {
            constexpr int DVT = CC::NVW * 16;
            constexpr auto ks = gdn_scan_cols_kernel<T, DK, DV, C, DVT, RULE>;
            if constexpr (RULE == kNoErase && !CC::GATES_INLINE) {
                // the gate rows of every chunk, before a scan that stages them
                constexpr int WPB = kThreads / 64;
                const int64_t gu = raw.slots * H;
                tm->mark(stream);
                if (gu > 0) {
                    hipLaunchKernelGGL(gdn_gates_kernel<C>, dim3((unsigned)((gu + WPB - 1) / WPB)), dim3(kThreads),
                                       0, stream, raw.log_alpha, raw.beta, geom, H, (int)gu,
                                       const_cast<float*>(g_ws));
                    if (gdn_status s = check_launch(stream)) return s;
                }
                tm->mark(stream);
            }
            allow_smem<ks>(CC::SMEM);
            tm->mark(stream);
            hipLaunchKernelGGL(ks, dim3(DV / DVT, H, (unsigned)n_seqs), dim3(CC::NTHR), CC::SMEM, stream,
                               q, k, v, S0, geom, H, g_ws, Tb_ws, O, S_T, rows, raw);
            if (gdn_status s = check_launch(stream)) return s;
            tm->mark(stream);
            return GDN_OK;
        } else {
            return GDN_ERR_INTERNAL;
        }
    };
    static_assert(fit32 || fit16, "no column-scan configuration fits the LDS of one CU");
    // 64-column slices (bf16, C = 64) where 32-column ones would take more
    // than one workgroup per CU: a wide workgroup's chunk step is about 1.45
    // times a 32-column one's, against two narrow workgroups in turn
    if constexpr (sizeof(T) == 2 && C == 64 && DV % 64 == 0) {
        using C64 = ColCfg<T, DK, DV, C, 64, RULE>;
        if constexpr (C64::FITS) {
            if (units * (DV / 32) > device_cu_count())
                return launch_cols(C64{});
        }
    }
    if (fit32 && (!fit16 || units * (DV / 32) >= device_cu_count())) return launch_cols(C32{});
    return launch_cols(C16{});
}

// Whether the split scan's span maps over n span-units run 128-column slices
// (bf16, C = 64): where 64-column ones would need more than one round of the
// device.  Those slices write no outputs, so eight column waves take the place
// of the output helpers and each workgroup covers twice the columns.
template <typename T, int DK, int DV, int C>
constexpr bool kMaps128 = sizeof(T) == 2 && C == 64 && (DK + DV) % 128 == 0 &&
                          ColCfg<T, DK, DK + DV, C, 128, kDelta>::FITS;

bool maps128_pays(int64_t span_units, int cols) {
    return span_units * (cols / 64) > device_cu_count();
}

// The split scan's first pass: every span from identity state rows (DK of
// them, zero values) and from zero for the DV value rows; no outputs.
template <typename T, int DK, int DV, int C>
gdn_status launch_maps(const T* q, const T* k, const T* v, const SeqGeom& geom, int H, int64_t n_seqs,
                       const float* g_ws, const T* Tb_ws, float* maps, hipStream_t stream, KernelTimer* tm) {
    if constexpr (kMaps128<T, DK, DV, C>) {
        if (maps128_pays(n_seqs * H, DK + DV)) {
            using CM = ColCfg<T, DK, DK + DV, C, 128, kDelta>;
            constexpr auto ks = gdn_scan_cols_kernel<T, DK, DK + DV, C, 128, kDelta>;
            allow_smem<ks>(CM::SMEM);
            tm->mark(stream);
            hipLaunchKernelGGL(ks, dim3((DK + DV) / 128, H, (unsigned)n_seqs), dim3(CM::NTHR), CM::SMEM, stream,
                               q, k, v, (const float*)nullptr, geom, H, g_ws, Tb_ws, (T*)nullptr, maps,
                               ScanRows{DK, DV}, RawGates{});
            if (gdn_status s = check_launch(stream)) return s;
            tm->mark(stream);
            return GDN_OK;
        }
    }
    return launch_scan<T, DK, DK + DV, C, kDelta>(q, k, v, nullptr, geom, H, n_seqs, g_ws, Tb_ws, nullptr, maps,
                                                  ScanRows{DK, DV}, stream, tm);
}

template <typename T, int DK, int DV, int C, int RULE>
gdn_status launch_fwd(const FwdArgs& a, KernelTimer* tm) {
    const bool varlen = a.cu != nullptr;
    const Layout L = make_layout(RULE, a.B, a.T, a.H, DK, DV, C, varlen, a.n_seqs, sizeof(T));
    float* g_ws = reinterpret_cast<float*>(a.ws + L.g);
    T* Tb_ws = reinterpret_cast<T*>(a.ws + L.Tb);

    SeqGeom geom{};
    geom.C = C;
    geom.T = a.T;
    geom.chunks_per_seq = (a.T + C - 1) / C;
    if (varlen) {
        int* bounds = reinterpret_cast<int*>(a.ws + L.bounds);
        int* seq_slot = reinterpret_cast<int*>(a.ws + L.seq_slot);
        int* table = reinterpret_cast<int*>(a.ws + L.table);
        int* order = reinterpret_cast<int*>(a.ws + L.order);
        tm->mark(a.stream);
        hipLaunchKernelGGL(gdn_chunk_table_kernel, dim3(1), dim3(kTableThreads), 0, a.stream,
                           a.cu, a.n_seqs, a.T, C, (int)L.slots, bounds, seq_slot, table, order);
        if (gdn_status s = check_launch(a.stream)) return s;
        tm->mark(a.stream);
        geom.table = table;
        geom.seq_slot = seq_slot;
        geom.bounds = bounds;
        geom.order = order;
    }
    const T* q = static_cast<const T*>(a.q);
    const T* k = static_cast<const T*>(a.k);
    const T* v = static_cast<const T*>(a.v);
    if constexpr (RULE == kGla) {
        using P = GlaPrepCfg<T, DK, C>;
        constexpr auto kp = gdn_gla_prep_kernel<T, DK, C>;
        allow_smem<kp>(P::SMEM);
        const int64_t units = L.slots * a.H;
        T* qt = reinterpret_cast<T*>(a.ws + L.qt);
        T* kh = reinterpret_cast<T*>(a.ws + L.kh);
        // persistent: as many workgroups as are resident at once, each walking
        // units with a stride of the grid
        const int64_t resident = (int64_t)device_cu_count() * resident_per_cu<kp>(P::THREADS, P::SMEM);
        const unsigned grid = (unsigned)(units < resident ? units : resident);
        tm->mark(a.stream);
        if (units > 0) {
            hipLaunchKernelGGL(kp, dim3(grid), dim3(P::THREADS), P::SMEM, a.stream, q, k,
                               a.log_alpha, a.beta, geom, a.H, (int)units, g_ws, Tb_ws, qt, kh);
            if (gdn_status s = check_launch(a.stream)) return s;
        }
        tm->mark(a.stream);
        // the scan runs on the decayed operands
        q = qt;
        k = kh;
    }

    if constexpr (RULE == kDelta) if (L.slots > 0) {
        using P = PrepCfg<T, DK, C>;
        constexpr auto kp = gdn_prep_kernel<T, DK, C>;
        allow_smem<kp>(P::SMEM);
        // persistent: as many workgroups as are resident on the device at once,
        // each wave walking units (slot, head) with a stride of all waves
        const int64_t units = L.slots * a.H;
        const int64_t resident = (int64_t)device_cu_count() * resident_per_cu<kp>(kThreads, P::SMEM);
        const int64_t need = (units + P::WAVES - 1) / P::WAVES;
        const unsigned grid = (unsigned)(need < resident ? need : resident);
        tm->mark(a.stream);
        hipLaunchKernelGGL(kp, dim3(grid), dim3(kThreads), P::SMEM, a.stream,
                           k, a.log_alpha, a.beta, geom, a.H, (int)units, g_ws, Tb_ws);
        if (gdn_status s = check_launch(a.stream)) return s;
        tm->mark(a.stream);
    }
    // the no-erase rule: its gate rows (formed by the scan itself, or by the
    // gates kernel launch_scan runs first)
    const RawGates raw = RULE == kNoErase ? RawGates{a.log_alpha, a.beta, L.slots} : RawGates{};
    return launch_scan<T, DK, DV, C, RULE>(q, k, v, a.S0, geom, a.H, L.N, g_ws, Tb_ws,
                                           static_cast<T*>(a.O), a.S_T, ScanRows{0, DV}, a.stream,
                                           tm, raw);
}

// ---------------------------------------------------------------------------
// Split scan: the sequences of a fixed-length batch cut into spans of L
// chunks; (1) the scan of every span from identity rows gives its map (M, b),
// (2) gdn_span_chain_kernel chains the maps into each span's start state,
// (3) the scan of every span from its start state writes O.  Compiled for
// the shapes of kSplitVariants.
// ---------------------------------------------------------------------------
struct SplitLayout {
    int64_t P, slots;
    size_t g, Tb, maps, sin, total;
};

SplitLayout make_split_layout(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv, int64_t C,
                              int64_t L, size_t es) {
    SplitLayout S{};
    const int64_t cps = (T + C - 1) / C;
    S.P = cps > 0 ? (cps + L - 1) / L : 1;   // spans per sequence
    S.slots = B * cps;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t at = off; off = align_up(off + bytes); return at; };
    const size_t u = (size_t)(S.slots * H);
    S.g = take(u * gate_rows(kDelta) * C * sizeof(float));
    S.Tb = take(u * (size_t)tb_blocks((int)C, es == 2) * 1024);
    S.maps = take((size_t)(B * S.P * H) * (Dk + Dv) * Dk * sizeof(float));
    S.sin = take((size_t)(B * S.P * H) * Dv * Dk * sizeof(float));
    S.total = off;
    return S;
}

template <typename T, int DK, int DV, int C>
gdn_status launch_split(const FwdArgs& a, int L, KernelTimer* tm) {
    const SplitLayout S = make_split_layout(a.B, a.T, a.H, DK, DV, C, L, sizeof(T));
    float* g_ws = reinterpret_cast<float*>(a.ws + S.g);
    T* Tb_ws = reinterpret_cast<T*>(a.ws + S.Tb);
    float* maps = reinterpret_cast<float*>(a.ws + S.maps);
    float* sin = reinterpret_cast<float*>(a.ws + S.sin);
    const T* q = static_cast<const T*>(a.q);
    const T* k = static_cast<const T*>(a.k);
    const T* v = static_cast<const T*>(a.v);
    SeqGeom geom{};
    geom.C = C;
    geom.T = a.T;
    geom.chunks_per_seq = (a.T + C - 1) / C;
    // prep over every chunk: the chunk slots are the same split or not
    tm->mark(a.stream);
    if (S.slots > 0) {
        using P = PrepCfg<T, DK, C>;
        constexpr auto kp = gdn_prep_kernel<T, DK, C>;
        allow_smem<kp>(P::SMEM);
        const int64_t units = S.slots * a.H;
        const int64_t resident = (int64_t)device_cu_count() * resident_per_cu<kp>(kThreads, P::SMEM);
        const int64_t need = (units + P::WAVES - 1) / P::WAVES;
        const unsigned grid = (unsigned)(need < resident ? need : resident);
        hipLaunchKernelGGL(kp, dim3(grid), dim3(kThreads), P::SMEM, a.stream,
                           k, a.log_alpha, a.beta, geom, a.H, (int)units, g_ws, Tb_ws);
        if (gdn_status s = check_launch(a.stream)) return s;
    }
    tm->mark(a.stream);
    SeqGeom sg = geom;
    sg.span_chunks = L;
    sg.spans = (int)S.P;
    const int64_t NS = a.B * S.P;
    // (1) span maps: DK identity rows with zero values, then the DV value rows
    // from zero; no outputs
    if (gdn_status s = launch_maps<T, DK, DV, C>(q, k, v, sg, a.H, NS, g_ws, Tb_ws, maps, a.stream, tm)) return s;
    // (2) each span's start state, and S_T: on MFMA for bf16 inputs (split
    // products), on fp32 FMAs for fp32 ones
    if constexpr (sizeof(T) == 2 && DK % 64 == 0 && DV % 16 == 0) {
        using SC = SpanMfmaCfg<DK, DV>;
        constexpr auto kc = gdn_span_chain_mfma_kernel<DK, DV>;
        allow_smem<kc>(SC::SMEM);
        tm->mark(a.stream);
        hipLaunchKernelGGL(kc, dim3(a.H, DV / SC::ROWS, a.B), dim3(SC::THREADS), SC::SMEM, a.stream,
                           maps, a.S0, (int)S.P, a.H, sin, a.S_T);
        if (gdn_status s = check_launch(a.stream)) return s;
        tm->mark(a.stream);
    } else {
        using SC = SpanCfg<DK, DV>;
        constexpr auto kc = gdn_span_chain_kernel<DK, DV>;
        allow_smem<kc>(SC::SMEM);
        tm->mark(a.stream);
        hipLaunchKernelGGL(kc, dim3(a.H, DV / SC::ROWS, a.B), dim3(SC::THREADS), SC::SMEM, a.stream,
                           maps, a.S0, (int)S.P, a.H, sin, a.S_T);
        if (gdn_status s = check_launch(a.stream)) return s;
        tm->mark(a.stream);
    }
    // (3) the outputs of every span from its start state
    return launch_scan<T, DK, DV, C, kDelta>(q, k, v, sin, sg, a.H, NS, g_ws, Tb_ws,
                                             static_cast<T*>(a.O), nullptr, ScanRows{0, DV}, a.stream, tm);
}

// compiled instantiations of the split scan (the first pass runs the scan
// with Dk + Dv state columns)
typedef gdn_status (*SplitFn)(const FwdArgs&, int, KernelTimer*);
struct SplitVariant {
    int dk, dv, c;
    gdn_dtype dt;
    SplitFn fn;
};
const SplitVariant kSplitVariants[] = {
    {64, 64, 64, GDN_F32, launch_split<float, 64, 64, 64>},
    {128, 128, 64, GDN_F32, launch_split<float, 128, 128, 64>},
    {128, 128, 64, GDN_BF16, launch_split<bf16, 128, 128, 64>},
};
const SplitVariant* find_split(int dk, int dv, int c, gdn_dtype dt) {
    for (const SplitVariant& v : kSplitVariants)
        if (v.dk == dk && v.dv == dv && v.c == c && v.dt == dt) return &v;
    return nullptr;
}

typedef gdn_status (*FwdFn)(const FwdArgs&, KernelTimer*);
struct Variant {
    int dk, dv, c;
    gdn_dtype dt;
    FwdFn fn;
};

// compiled instantiations of each rule
const Variant kVariants[] = {
    {16, 16, 16, GDN_F32, launch_fwd<float, 16, 16, 16, kDelta>},
    {64, 64, 16, GDN_F32, launch_fwd<float, 64, 64, 16, kDelta>},
    {64, 64, 64, GDN_F32, launch_fwd<float, 64, 64, 64, kDelta>},
    {128, 128, 64, GDN_F32, launch_fwd<float, 128, 128, 64, kDelta>},
    {128, 256, 64, GDN_F32, launch_fwd<float, 128, 256, 64, kDelta>},
    {128, 128, 64, GDN_BF16, launch_fwd<bf16, 128, 128, 64, kDelta>},
    {128, 256, 64, GDN_BF16, launch_fwd<bf16, 128, 256, 64, kDelta>},
};
const Variant kVariantsNoErase[] = {
    {16, 16, 16, GDN_F32, launch_fwd<float, 16, 16, 16, kNoErase>},
    {64, 64, 64, GDN_F32, launch_fwd<float, 64, 64, 64, kNoErase>},
    {128, 128, 64, GDN_BF16, launch_fwd<bf16, 128, 128, 64, kNoErase>},
    {128, 256, 64, GDN_BF16, launch_fwd<bf16, 128, 256, 64, kNoErase>},
};
const Variant kVariantsGla[] = {
    {16, 16, 16, GDN_F32, launch_fwd<float, 16, 16, 16, kGla>},
    {64, 64, 64, GDN_F32, launch_fwd<float, 64, 64, 64, kGla>},
    {128, 128, 64, GDN_BF16, launch_fwd<bf16, 128, 128, 64, kGla>},
    {128, 256, 64, GDN_BF16, launch_fwd<bf16, 128, 256, 64, kGla>},
};
static_assert(GDN_RULE_DELTA == kDelta && GDN_RULE_MAMBA2 == kNoErase && GDN_RULE_GLA == kGla,
              "rule numbering");

bool valid_rule(int rule) {
    return rule == GDN_RULE_DELTA || rule == GDN_RULE_MAMBA2 || rule == GDN_RULE_GLA;
}

const Variant* find_variant(int rule, int dk, int dv, int c, gdn_dtype dt) {
    auto scan = [&](const Variant* b, const Variant* e) -> const Variant* {
        for (const Variant* v = b; v != e; ++v)
            if (v->dk == dk && v->dv == dv && v->c == c && v->dt == dt) return v;
        return nullptr;
    };
    if (rule == GDN_RULE_DELTA) return scan(std::begin(kVariants), std::end(kVariants));
    if (rule == GDN_RULE_MAMBA2) return scan(std::begin(kVariantsNoErase), std::end(kVariantsNoErase));
    if (rule == GDN_RULE_GLA) return scan(std::begin(kVariantsGla), std::end(kVariantsGla));
    return nullptr;
}

size_t elem_size(gdn_dtype dt) { return dt == GDN_BF16 ? 2 : 4; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kMaxElems = 0x7fffffffLL;

// Host-side checks shared by the size query and the forward call.
gdn_status check_sizes(int rule, int B, int T, int H, int Dk, int Dv, int C, bool varlen,
                       int n_seqs, gdn_dtype dt) {
    if (dt != GDN_F32 && dt != GDN_BF16) return GDN_ERR_UNSUPPORTED;
    if (!valid_rule(rule)) return GDN_ERR_UNSUPPORTED;
    if (B < 1 || T < 0 || H < 1 || H > 65535 || Dk < 1 || Dv < 1 || C < 1) return GDN_ERR_SHAPE;
    if (varlen && (B != 1 || n_seqs < 1 || n_seqs > 65535)) return GDN_ERR_SHAPE;
    if (!varlen && B > 65535) return GDN_ERR_SHAPE;
    const int64_t tokens = (int64_t)B * T;
    const int64_t dmax = Dk > Dv ? Dk : Dv;
    if (tokens * H * dmax > kMaxElems) return GDN_ERR_SHAPE;
    const int64_t N = varlen ? n_seqs : B;
    if (N * H * (int64_t)Dv * Dk > kMaxElems) return GDN_ERR_SHAPE;
    // the scan addresses one chunk of one token tensor with 31-bit byte offsets
    if ((int64_t)C * H * dmax * elem_size(dt) > kMaxElems) return GDN_ERR_SHAPE;
    // ... and the GLA prep one chunk of the per-channel gate (fp32, Dk per token)
    if (rule == GDN_RULE_GLA && (int64_t)C * H * Dk * 4 > kMaxElems) return GDN_ERR_SHAPE;
    if (!find_variant(rule, Dk, Dv, C, dt)) return GDN_ERR_UNSUPPORTED;
    return GDN_OK;
}

// Span length of gdn_chunk_fwd's automatic split (0: no split), from a cost
// model of the two paths with per-step costs measured on MI355X.  The plain
// scan runs each (sequence, head) unit's chunks one after another, so with few
// units most CUs idle; the split runs three kernels more (the span maps over
// Dk + Dv state columns, the chain of the maps, the output pass) over P times
// the workgroups:
//   plain    = f + chunks * s_plain
//   split(P) = 3 f + L (s1 r1 + s3 r3) + P (c0 + c1 units),  L = ceil(chunks / P),
// with s_plain rising from its few-workgroup value to s_full as the plain
// scan's workgroups go from half the CUs to all of them,
// with r1, r3 the rounds of workgroups each pass needs on the device (32-column
// slices where they fill it, else 16-column ones; bf16: 64-column slices, at
// their own step cost, where 32-column ones would need more than one round;
// the span maps on 128-column slices where 64-column ones would) and f a
// kernel's fixed cost.  The split is taken at the best P when it is under a
// share of the plain estimate (bf16 0.90, fp32 0.95).  Measured (ms per call,
// sums of the kernels' device times, plain -> split at the chosen span
// length): bf16 D128 T = 32768: 2 heads 0.49 -> 0.125, 4 heads 0.51 -> 0.14,
// 8 heads 0.53 -> 0.18, 16 heads 0.59 -> 0.32, 32 heads 0.66 -> 0.53; 4 heads
// T = 4096 0.077 -> 0.063; 32 heads T = 16384 0.338 -> 0.315, T = 8192 0.168
// (split 0.180: not taken); 16 heads T = 2048 0.057 (split 0.073: not taken);
// fp32 D64 B2 H4 T = 1024 0.078 -> 0.055; fp32 D128 B1 H2 T = 8192 0.693 ->
// 0.206, 16 heads T = 4096 0.368 (split 0.568: not taken).  Packed batches
// always run the plain scan.
struct SplitModel {
    int dk, dv, c;
    gdn_dtype dt;
    bool w32;                         // both passes have a 32-column slice that fits the LDS
    double s_plain, s_full, s1, s3, c0, c1;   // microseconds
    double s1w, s3w;                          // 64-column slices (0: none)
    double s1m;                               // span maps on 128-column slices (0: none)
    double take;                              // the split is taken under this share of plain
};
const SplitModel kSplitModels[] = {
    {128, 128, 64, GDN_BF16, true, 1.05, 1.25, 0.95, 1.40, 2.5, 0.10, 1.05, 1.95, 1.50, 0.90},
    {64, 64, 64, GDN_F32, true, 3.30, 3.30, 4.00, 4.00, 0.8, 0.04, 0.0, 0.0, 0.0, 0.95},
    {128, 128, 64, GDN_F32, false, 5.00, 5.00, 5.00, 5.00, 2.0, 0.05, 0.0, 0.0, 0.0, 0.95},
};
constexpr double kKernelFixedUs = 6.0;

int auto_span_chunks(int B, int T, int H, int Dk, int Dv, int C, gdn_dtype dt, bool varlen) {
    if (varlen || T <= 0) return 0;
    const SplitModel* m = nullptr;
    for (const SplitModel& x : kSplitModels)
        if (x.dk == Dk && x.dv == Dv && x.c == C && x.dt == dt) m = &x;
    if (!m || !find_split(Dk, Dv, C, dt)) return 0;
    const int64_t cps = ((int64_t)T + C - 1) / C;
    const int64_t cus = device_cu_count();
    const int64_t units = (int64_t)B * H;
    if (cps < 2 || units * (Dv / 16) > cus) return 0;   // the plain scan already fills the device
    const int64_t wp = m->w32 && units * (Dv / 32) >= cus ? units * (Dv / 32) : units * (Dv / 16);
    const double fill = std::min(1.0, std::max(0.0, 2.0 * (double)wp / (double)cus - 1.0));
    const double plain = kKernelFixedUs + (double)cps * (m->s_plain + fill * (m->s_full - m->s_plain));
    // time of one chunk step of a pass over n span-units: rounds of workgroups
    // times the step cost of the slice width the scan takes (launch_scan)
    auto step = [&](int64_t n, int cols, double s, double sw) {
        const int64_t w32 = n * cols / 32;
        if (sw > 0 && cols % 64 == 0 && w32 > cus) return sw * (double)((n * cols / 64 + cus - 1) / cus);
        const int64_t w = m->w32 && w32 >= cus ? w32 : n * cols / 16;
        return s * (double)((w + cus - 1) / cus);
    };
    // the span maps: 128-column slices where 64-column ones need more than one
    // round (launch_maps)
    auto step_maps = [&](int64_t n) {
        const int cols = Dk + Dv;
        if (m->s1m > 0 && n * (cols / 64) > cus) return m->s1m * (double)((n * cols / 128 + cus - 1) / cus);
        return step(n, cols, m->s1, m->s1w);
    };
    double best = m->take * plain;
    int best_l = 0;
    for (int64_t P = 2; P <= cps && P <= 64; ++P) {
        const int64_t L = (cps + P - 1) / P, Pe = (cps + L - 1) / L;
        const int64_t n = units * Pe;
        if ((int64_t)B * Pe > 65535) break;   // spans of the batch: the scan grid's third dimension
        const double cost = 3 * kKernelFixedUs + (double)L * (step_maps(n) + step(n, Dv, m->s3, m->s3w)) +
                            (double)Pe * (m->c0 + m->c1 * (double)units);
        if (cost < best) {
            best = cost;
            best_l = (int)L;
        }
    }
    return best_l;
}

}  // namespace
}  // namespace gdn

using namespace gdn;

extern "C" int gdn_rule_supported(gdn_rule rule, int Dk, int Dv, int C, gdn_dtype dt) {
    return find_variant(rule, Dk, Dv, C, dt) ? 1 : 0;
}

extern "C" int gdn_chunk_fwd_supported(int Dk, int Dv, int C, gdn_dtype dt) {
    return gdn_rule_supported(GDN_RULE_DELTA, Dk, Dv, C, dt);
}

extern "C" size_t gdn_rule_workspace_bytes(gdn_rule rule, int B, int T, int H, int Dk, int Dv,
                                           int C, int n_seqs, gdn_dtype dt) {
    const bool varlen = n_seqs > 0;
    if (check_sizes(rule, B, T, H, Dk, Dv, C, varlen, n_seqs, dt) != GDN_OK) return 0;
    const size_t plain = make_layout(rule, B, T, H, Dk, Dv, C, varlen, n_seqs, elem_size(dt)).total;
    if (rule == GDN_RULE_DELTA) {   // room for the automatic split where gdn_chunk_fwd takes it
        const int L = auto_span_chunks(B, T, H, Dk, Dv, C, dt, varlen);
        if (L > 0) {
            const size_t split = make_split_layout(B, T, H, Dk, Dv, C, L, elem_size(dt)).total;
            return split > plain ? split : plain;
        }
    }
    return plain;
}

extern "C" int gdn_chunk_fwd_auto_span_chunks(int B, int T, int H, int Dk, int Dv, int C,
                                              int n_seqs, gdn_dtype dt) {
    const bool varlen = n_seqs > 0;
    if (check_sizes(GDN_RULE_DELTA, B, T, H, Dk, Dv, C, varlen, n_seqs, dt) != GDN_OK) return 0;
    return auto_span_chunks(B, T, H, Dk, Dv, C, dt, varlen);
}

extern "C" size_t gdn_chunk_fwd_workspace_bytes(int B, int T, int H, int Dk, int Dv, int C,
                                                int n_seqs, gdn_dtype dt) {
    return gdn_rule_workspace_bytes(GDN_RULE_DELTA, B, T, H, Dk, Dv, C, n_seqs, dt);
}

// ---------------------------------------------------------------------------
// Static scratch buffer of gdn_chunk_fwd_noalloc: the per-chunk intermediates
// of one call, in device memory the library owns (one copy per GPU, from the
// library's load until the process ends), for callers that cannot allocate.
// In host code `scratch` names a host-side stand-in, not a device address: its
// device address is looked up once per device with hipGetSymbolAddress and
// only that pointer is ever handed to a kernel.
// ---------------------------------------------------------------------------
namespace {
constexpr size_t kScratchBytes = (size_t)64 << 20;
static_assert(kScratchBytes == (size_t)GDN_NOALLOC_SCRATCH_BYTES, "header and library disagree");
}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
// Device address of `scratch` on the current device (looked up on the first
// call with that device current, then cached); NULL if the lookup fails.
void* scratch_device_ptr() {
    static std::atomic<void*> cached[kMaxCachedDevices] = {};
    const int dev = current_device();
    void* p = dev < kMaxCachedDevices ? cached[dev].load(std::memory_order_acquire) : nullptr;
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return nullptr;
        }
        if (dev < kMaxCachedDevices) cached[dev].store(p, std::memory_order_release);
    }
    return p;
}

// use_scratch: run on the static scratch buffer instead of `workspace`;
// tm == NULL: only the host-side argument checks (no HIP call is made)
gdn_status chunk_fwd_impl(int rule, const void* q, const void* k, const void* v,
                          const float* log_alpha, const float* beta, const float* S0,
                          const int32_t* cu_seqlens, int n_seqs, void* O, float* S_T, int B,
                          int T, int H, int Dk, int Dv, int C, gdn_dtype dt, void* workspace,
                          size_t workspace_bytes, bool use_scratch, void* stream,
                          KernelTimer* tm) {
    const bool varlen = cu_seqlens != nullptr;
    // with no tokens the token tensors are never read (empty tensors may be
    // NULL); beta may be NULL (beta = 1) for the no-erase rules only
    const bool has_tokens = T > 0;
    if (has_tokens && (!q || !k || !v || (!beta && rule == GDN_RULE_DELTA) || !O)) return GDN_ERR_NULL;
    if (gdn_status s = check_sizes(rule, B, T, H, Dk, Dv, C, varlen, n_seqs, dt)) return s;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(O) || !aligned16(S0) ||
        !aligned16(S_T))
        return GDN_ERR_SHAPE;
    const Layout L = make_layout(rule, B, T, H, Dk, Dv, C, varlen, n_seqs, elem_size(dt));
    if (use_scratch) {
        if (L.total > kScratchBytes) return GDN_ERR_SCRATCH_LIMIT;
        if (!tm) return GDN_OK;
        workspace = scratch_device_ptr();
        if (!workspace) return GDN_ERR_HIP;
        workspace_bytes = kScratchBytes;
    }
    if (!aligned16(workspace)) return GDN_ERR_SHAPE;
    if (L.total > 0 && !workspace) return GDN_ERR_NULL;
    if (workspace_bytes < L.total) return GDN_ERR_WORKSPACE;
    if (!tm) return GDN_OK;
    FwdArgs a{q, k, v, log_alpha, beta, S0, cu_seqlens, varlen ? n_seqs : B, O, S_T,
              B, T, H, Dk, Dv, C, dt, static_cast<unsigned char*>(workspace),
              static_cast<hipStream_t>(stream)};
    (void)hipGetLastError();   // report only errors raised by this call's launches
    // the automatic split (plain, unprofiled calls of the delta rule with room
    // for it in the workspace)
    if (rule == GDN_RULE_DELTA && !use_scratch && !tm->on) {
        const int Ls = auto_span_chunks(B, T, H, Dk, Dv, C, dt, varlen);
        if (Ls > 0 && workspace_bytes >= make_split_layout(B, T, H, Dk, Dv, C, Ls, elem_size(dt)).total)
            return find_split(Dk, Dv, C, dt)->fn(a, Ls, tm);
    }
    return find_variant(rule, Dk, Dv, C, dt)->fn(a, tm);
}
}  // namespace

extern "C" gdn_status gdn_chunk_fwd(const void* q, const void* k, const void* v,
                                    const float* log_alpha, const float* beta, const float* S0,
                                    const int32_t* cu_seqlens, int n_seqs, void* O, float* S_T,
                                    int B, int T, int H, int Dk, int Dv, int C, gdn_dtype dt,
                                    void* workspace, size_t workspace_bytes, void* stream) {
    try {
        KernelTimer off;
        return chunk_fwd_impl(GDN_RULE_DELTA, q, k, v, log_alpha, beta, S0, cu_seqlens, n_seqs,
                              O, S_T, B, T, H, Dk, Dv, C, dt, workspace, workspace_bytes, false,
                              stream, &off);
    } catch (...) {
        return GDN_ERR_INTERNAL;
    }
}

extern "C" gdn_status gdn_chunk_fwd_noalloc(const void* q, const void* k, const void* v,
                                            const float* log_alpha, const float* beta,
                                            const float* S0, const int32_t* cu_seqlens,
                                            int n_seqs, void* O, float* S_T, int B, int T, int H,
                                            int Dk, int Dv, int C, gdn_dtype dt, void* stream) {
    try {
        KernelTimer off;
        return chunk_fwd_impl(GDN_RULE_DELTA, q, k, v, log_alpha, beta, S0, cu_seqlens, n_seqs,
                              O, S_T, B, T, H, Dk, Dv, C, dt, nullptr, 0, true, stream, &off);
    } catch (...) {
        return GDN_ERR_INTERNAL;
    }
}

extern "C" gdn_status gdn_mamba2_chunk_fwd(const void* q, const void* k, const void* v,
                                           const float* log_alpha, const float* beta,
                                           const float* S0, const int32_t* cu_seqlens,
                                           int n_seqs, void* O, float* S_T, int B, int T, int H,
                                           int Dk, int Dv, int C, gdn_dtype dt, void* workspace,
                                           size_t workspace_bytes, void* stream) {
    try {
        KernelTimer off;
        return chunk_fwd_impl(GDN_RULE_MAMBA2, q, k, v, log_alpha, beta, S0, cu_seqlens, n_seqs,
                              O, S_T, B, T, H, Dk, Dv, C, dt, workspace, workspace_bytes, false,
                              stream, &off);
    } catch (...) {
        return GDN_ERR_INTERNAL;
    }
}

extern "C" gdn_status gdn_gla_chunk_fwd(const void* q, const void* k, const void* v,
                                        const float* log_alpha, const float* beta, const float* S0,
                                        const int32_t* cu_seqlens, int n_seqs, void* O, float* S_T,
                                        int B, int T, int H, int Dk, int Dv, int C, gdn_dtype dt,
                                        void* workspace, size_t workspace_bytes, void* stream) {
    try {
        KernelTimer off;
        return chunk_fwd_impl(GDN_RULE_GLA, q, k, v, log_alpha, beta, S0, cu_seqlens, n_seqs, O,
                              S_T, B, T, H, Dk, Dv, C, dt, workspace, workspace_bytes, false,
                              stream, &off);
    } catch (...) {
        return GDN_ERR_INTERNAL;
    }
}

extern "C" gdn_status gdn_rule_chunk_fwd_profiled(gdn_rule rule, const void* q, const void* k,
                                                  const void* v, const float* log_alpha,
                                                  const float* beta, const float* S0,
                                                  const int32_t* cu_seqlens, int n_seqs, void* O,
                                                  float* S_T, int B, int T, int H, int Dk, int Dv,
                                                  int C, gdn_dtype dt, void* workspace,
                                                  size_t workspace_bytes, void* stream,
                                                  float* kernel_ms) {
    if (!kernel_ms) return GDN_ERR_NULL;
    for (int i = 0; i < 4; ++i) kernel_ms[i] = 0.f;
    try {
        // argument errors before any HIP call
        if (gdn_status s = chunk_fwd_impl(rule, q, k, v, log_alpha, beta, S0, cu_seqlens, n_seqs,
                                          O, S_T, B, T, H, Dk, Dv, C, dt, workspace,
                                          workspace_bytes, false, stream, nullptr))
            return s;
        KernelTimer tm;
        tm.on = true;
        for (int i = 0; i < 8; ++i) {
            if (hipEventCreate(&tm.ev[i]) != hipSuccess) {
                for (int j = 0; j < i; ++j) (void)hipEventDestroy(tm.ev[j]);
                return GDN_ERR_HIP;
            }
        }
        gdn_status s = chunk_fwd_impl(rule, q, k, v, log_alpha, beta, S0, cu_seqlens, n_seqs, O,
                                      S_T, B, T, H, Dk, Dv, C, dt, workspace, workspace_bytes,
                                      false, stream, &tm);
        if (s == GDN_OK && hipEventSynchronize(tm.ev[tm.n - 1]) != hipSuccess) s = GDN_ERR_HIP;
        if (s == GDN_OK) {
            // pairs of marks: [table], [prep or gates], scan (prep absent when
            // there are no chunks)
            const bool varlen = cu_seqlens != nullptr;
            const bool has_chunks = tm.n >= (varlen ? 6 : 4);
            int slot[4] = {-1, -1, -1, -1};
            int m = 0;
            if (varlen) slot[0] = m++;
            if (has_chunks) slot[1] = m++;
            slot[2] = m++;
            for (int i = 0; i < 4; ++i) {
                if (slot[i] < 0) continue;
                float ms = 0.f;
                if (hipEventElapsedTime(&ms, tm.ev[2 * slot[i]], tm.ev[2 * slot[i] + 1]) != hipSuccess)
                    s = GDN_ERR_HIP;
                kernel_ms[i] = ms;
            }
        }
        for (int i = 0; i < 8; ++i) (void)hipEventDestroy(tm.ev[i]);
        return s;
    } catch (...) {
        return GDN_ERR_INTERNAL;
    }
}

namespace {
gdn_status check_split(int B, int T, int H, int Dk, int Dv, int C, gdn_dtype dt, int span_chunks) {
    if (gdn_status s = check_sizes(GDN_RULE_DELTA, B, T, H, Dk, Dv, C, false, 0, dt)) return s;
    if (!find_split(Dk, Dv, C, dt)) return GDN_ERR_UNSUPPORTED;
    if (span_chunks < 1) return GDN_ERR_SHAPE;
    const SplitLayout S = make_split_layout(B, T, H, Dk, Dv, C, span_chunks, elem_size(dt));
    // the span maps, [B P][H][Dk + Dv][Dk], and the span grid
    if (B * S.P * H * (int64_t)(Dk + Dv) * Dk > kMaxElems || B * S.P > 65535) return GDN_ERR_SHAPE;
    return GDN_OK;
}
}  // namespace

extern "C" size_t gdn_chunk_fwd_split_workspace_bytes(int B, int T, int H, int Dk, int Dv, int C,
                                                      int span_chunks, gdn_dtype dt) {
    if (check_split(B, T, H, Dk, Dv, C, dt, span_chunks) != GDN_OK) return 0;
    return make_split_layout(B, T, H, Dk, Dv, C, span_chunks, elem_size(dt)).total;
}

extern "C" gdn_status gdn_chunk_fwd_split(const void* q, const void* k, const void* v,
                                          const float* log_alpha, const float* beta,
                                          const float* S0, void* O, float* S_T, int B, int T,
                                          int H, int Dk, int Dv, int C, gdn_dtype dt,
                                          int span_chunks, void* workspace,
                                          size_t workspace_bytes, void* stream,
                                          float* kernel_ms) {
    try {
        if (T > 0 && (!q || !k || !v || !beta || !O)) return GDN_ERR_NULL;
        if (gdn_status s = check_split(B, T, H, Dk, Dv, C, dt, span_chunks)) return s;
        if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(O) || !aligned16(S0) ||
            !aligned16(S_T) || !aligned16(workspace))
            return GDN_ERR_SHAPE;
        const size_t need = make_split_layout(B, T, H, Dk, Dv, C, span_chunks, elem_size(dt)).total;
        if (!workspace) return GDN_ERR_NULL;
        if (workspace_bytes < need) return GDN_ERR_WORKSPACE;
        FwdArgs a{q, k, v, log_alpha, beta, S0, nullptr, B, O, S_T, B, T, H, Dk, Dv, C, dt,
                  static_cast<unsigned char*>(workspace), static_cast<hipStream_t>(stream)};
        KernelTimer tm;
        tm.on = kernel_ms != nullptr;
        int created = 0;
        if (tm.on) {
            for (int i = 0; i < 4; ++i) kernel_ms[i] = 0.f;
            for (; created < 8; ++created)
                if (hipEventCreate(&tm.ev[created]) != hipSuccess) break;
            if (created < 8) {
                for (int j = 0; j < created; ++j) (void)hipEventDestroy(tm.ev[j]);
                return GDN_ERR_HIP;
            }
        }
        (void)hipGetLastError();
        gdn_status s = find_split(Dk, Dv, C, dt)->fn(a, span_chunks, &tm);
        if (tm.on) {
            // marks: prep, pass 1, chain, pass 3
            if (s == GDN_OK && hipEventSynchronize(tm.ev[tm.n - 1]) != hipSuccess) s = GDN_ERR_HIP;
            for (int i = 0; s == GDN_OK && i < 4 && 2 * i + 1 < tm.n; ++i)
                if (hipEventElapsedTime(&kernel_ms[i], tm.ev[2 * i], tm.ev[2 * i + 1]) != hipSuccess)
                    s = GDN_ERR_HIP;
            for (int i = 0; i < 8; ++i) (void)hipEventDestroy(tm.ev[i]);
        }
        return s;
    } catch (...) {
        return GDN_ERR_INTERNAL;
    }
}

extern "C" gdn_status gdn_chunk_fwd_profiled(const void* q, const void* k, const void* v,
                                             const float* log_alpha, const float* beta,
                                             const float* S0, const int32_t* cu_seqlens,
                                             int n_seqs, void* O, float* S_T, int B, int T,
                                             int H, int Dk, int Dv, int C, gdn_dtype dt,
                                             void* workspace, size_t workspace_bytes,
                                             void* stream, float* kernel_ms) {
    return gdn_rule_chunk_fwd_profiled(GDN_RULE_DELTA, q, k, v, log_alpha, beta, S0, cu_seqlens,
                                       n_seqs, O, S_T, B, T, H, Dk, Dv, C, dt, workspace,
                                       workspace_bytes, stream, kernel_ms);
}

namespace gdn {
namespace {
template <typename T, int DK, int DV>
gdn_status launch_step(const void* q, const void* k, const void* v, const float* la,
                       const float* beta, float* S, void* o, int N, int H, hipStream_t st) {
    hipLaunchKernelGGL((gdn_step_kernel<T, DK, DV>), dim3(DV / StepCfg<DK, DV>::RPW, H, N), dim3(64), 0, st,
                       static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v),
                       la, beta, S, static_cast<T*>(o), H);
    return check_launch(st);
}

typedef gdn_status (*StepFn)(const void*, const void*, const void*, const float*, const float*,
                             float*, void*, int, int, hipStream_t);

template <typename T, int DK>
StepFn pick_dv(int dv) {
    switch (dv) {
        case 16: return launch_step<T, DK, 16>;
        case 64: return launch_step<T, DK, 64>;
        case 128: return launch_step<T, DK, 128>;
        case 256: return launch_step<T, DK, 256>;
        default: return nullptr;
    }
}

template <typename T>
StepFn pick_step(int dk, int dv) {
    switch (dk) {
        case 16: return pick_dv<T, 16>(dv);
        case 64: return pick_dv<T, 64>(dv);
        case 128: return pick_dv<T, 128>(dv);
        case 256: return pick_dv<T, 256>(dv);
        default: return nullptr;
    }
}
}  // namespace
}  // namespace gdn

extern "C" gdn_status gdn_recurrent_step(const void* q, const void* k, const void* v,
                                         const float* log_alpha, const float* beta, float* S,
                                         void* o, int N, int H, int Dk, int Dv, gdn_dtype dt,
                                         void* stream) {
    try {
        if (!q || !k || !v || !beta || !S || !o) return GDN_ERR_NULL;
        if (dt != GDN_F32 && dt != GDN_BF16) return GDN_ERR_UNSUPPORTED;
        if (N < 1 || N > 65535 || H < 1 || H > 65535 || Dk < 1 || Dv < 1) return GDN_ERR_SHAPE;
        if ((int64_t)N * H * Dv * Dk > kMaxElems || !aligned16(S)) return GDN_ERR_SHAPE;
        StepFn fn = dt == GDN_BF16 ? pick_step<bf16>(Dk, Dv) : pick_step<float>(Dk, Dv);
        if (!fn) return GDN_ERR_UNSUPPORTED;
        (void)hipGetLastError();
        return fn(q, k, v, log_alpha, beta, S, o, N, H, static_cast<hipStream_t>(stream));
    } catch (...) {
        return GDN_ERR_INTERNAL;
    }
}

extern "C" const char* gdn_status_string(gdn_status s) {
    switch (s) {
        case GDN_OK: return "success";
        case GDN_ERR_NULL: return "a required pointer is NULL";
        case GDN_ERR_SHAPE: return "inconsistent, out-of-range or misaligned sizes";
        case GDN_ERR_UNSUPPORTED: return "no compiled kernel for this (Dk, Dv, chunk, dtype)";
        case GDN_ERR_WORKSPACE: return "workspace is smaller than required";
        case GDN_ERR_HIP: return "a HIP launch or runtime call failed";
        case GDN_ERR_INTERNAL: return "internal error";
        case GDN_ERR_SCRATCH_LIMIT:
            return "these sizes need more than the library's static scratch buffer holds";
    }
    return "unknown status";
}
