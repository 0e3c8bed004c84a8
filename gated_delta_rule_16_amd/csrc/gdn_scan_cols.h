// gdn_scan_cols.h -- serial inter-chunk state scan with the chunk outputs fused
// in, one wave per 16 state columns.
//
// Per chunk (row form, S = state at the chunk start, Dv x Dk; gamma_i =
// exp(g_i); Tb = T diag(beta) from the prep kernel):
//   Y  = K S^T,   X = V - diag(gamma) Y,   V' = Tb X
//   O^T = Z^T diag(gamma) + V'^T P^T,  Z^T = S Q^T, P = (Q K^T) o Gamma o M
//   S^T <- gamma_n S^T + K^T diag(gamma_n / gamma) V'
// (Qiita, the Linear Attention lineage, section "Gated-DeltaNet" and "Chunk
// Computation"; LinearAttention系列解读(六), sections 4.4 and 4.5).
//
// Rule kNoErase (the same article's "Mamba2" update with a write strength,
// S_t = alpha_t S_{t-1} + beta_t v_t k_t^T, in the chunk form of its "Chunk
// Computation" section): there is no prediction to remove, so Y and Tb drop
// out and V' = diag(beta) V; the output and the state update are unchanged.
//
// Rule kGla (per-channel gate, S_t = S_{t-1} diag(alpha_t) + beta_t v_t k_t^T;
// LinearAttention系列解读(六), section 1: the diagonal transition is split onto
// both sides of the mask): the GLA prep kernel hands over the chunk with its
// decays folded in, and the same pipeline runs on those operands:
//   Q -> Q~ = Q o e^b,  K -> K^ = diag(beta) K o e^(b_n - b),
//   Tb slot -> P~ = ((Q o e^b)(K o e^-b)^T o M) diag(beta)  (formed there with
//              bounded exponents), gates -> e^(b_n) per key channel,
// with b_i the in-chunk cumulative log-gate of each channel, so that
//   O^T = S Q~^T + V^T P~^T,   S^T <- diag(e^(b_n)) S^T + K^^T V.
// The column waves scale each state row by its channel's decay and take
// V' = V; the output helpers read P~ instead of forming P.
//
// Work split.  A workgroup owns a DVT-column slice of one (sequence, head):
//  - column waves (DVT / 16): wave vb holds all Dk rows of columns vb*16 ..
//    vb*16 + 15 of S^T in MFMA accumulators and runs the recurrence alone --
//    Y, X, V' and the state update never leave the wave, so there is no
//    synchronisation inside a chunk.  At the end of a chunk it leaves V' and
//    the new state (as MFMA operands in the input dtype) in LDS;
//  - two output helpers, each owning half of the chunk's query blocks, form
//    P^T = ((Q K^T) o Gamma o M)^T and Z^T = S Q^T for them in registers, and
//    one step later, when V' of that chunk is published, the output
//    O^T = Z^T diag(gamma) + V'^T P^T, which they leave in LDS;
//  - two staging waves: one loads the chunks straight into LDS (K, Tb, the V
//    slice and the gates two chunks ahead) and Q one chunk ahead through its
//    registers (where Q does not fit in LDS, the output helpers load it into
//    theirs, three chunks ahead), the other writes the output slices
//    out as whole 16-byte pieces of their rows (apart, so that the loader's
//    wait for its loads does not also wait for stores).
// With waves dealt to the four SIMDs in turn, the column waves and the output
// helpers get a SIMD each; the staging waves, which issue little, share the
// column waves' SIMDs.  One barrier per chunk.
//
// Wide slices (DVT = 64, bf16, for calls with more slices than CUs): a chunk's
// K, Q, Tb and gates are staged once per CU whatever the slice width, so a
// 64-column slice halves those bytes per state column.  Four column waves,
// four output helpers (one query block each) and the two staging waves: ten
// waves, three on two of the SIMDs, so every wave keeps to 168 registers.
// For that the helpers load Q into registers (there is no room for it in LDS
// beside three staging buffers), read their K, Q and state operands at the
// start of each contraction step rather than a step ahead, read V' at the
// output and form the decay factors after the products; the column waves keep
// two contraction steps of K fragments in flight instead of four.
//
// Span-map slices (DVT = 128, bf16): the first pass of the split scan writes
// no outputs, so where its 64-column slices would need more than one round of
// the device it runs 128-column ones: eight column waves and the two staging
// waves, no output helpers and no hand-over buffers, half the workgroups.
//
// State tile layout.  Column wave vb keeps Dk / 16 tiles; lane (g, n) of tile i
// holds S^T[drow(i, 4g + r)][vb*16 + n], r = 0..3.  bf16: tile 2m + h covers
// d = 32m + 8a + 4h + r for its rows 4a + r, so that the lane values of tiles
// 2m and 2m + 1 concatenate to d = 32m + 8g .. 32m + 8g + 7, the order of a
// 16-byte row fragment of K or Q; one 16x16x32 MFMA then contracts 32 d.
// fp32: tile i covers d = 16 i + rho (four 16x16x4 MFMAs per tile).
#pragma once

#include "gdn_ops.h"

namespace gdn {

template <typename T, int DK, int DV, int C, int DVT, int RULE = kDelta>
struct ColCfg {
    static constexpr bool BF = sizeof(T) == 2;
    static constexpr bool ERASE = RULE == kDelta;          // delta rule: Y, X and Tb
    static constexpr bool GLA = RULE == kGla;              // per-channel gate: P~ handed in
    static constexpr bool HAS_TB = RULE != kNoErase;       // Tb (delta) or P~ (GLA) staged
    static constexpr int GF = gate_floats(RULE, C, DK);    // fp32 gate values per chunk
    static constexpr int ES = sizeof(T);
    static constexpr int NW = C / 16;                      // 16-token blocks of a chunk
    static constexpr int NVW = DVT / 16;                   // column waves
    // 128-column slices (eight column waves) serve the split scan's span maps,
    // which write no outputs: no output helpers and no hand-over buffers
    static constexpr bool MAPS = NVW == 8;
    static constexpr bool WIDE = NVW > 2;                  // four or eight column waves
    static constexpr int NPP = MAPS ? 0 : WIDE ? NW : 2;   // helper waves: the first NPP
    static constexpr int NPW = NPP + 2;                    // form the output, the others
    static constexpr int NWG = NVW + NPW, NTHR = NWG * 64; // stage chunks and write out O
    // launch bound: the narrow slices keep the register budget of six waves
    static constexpr int BOUND = NTHR > 384 ? NTHR : 384;
    static constexpr int NF = NPW - NPP;                   // staging waves: NLD load
    static constexpr int NLD = NF - 1;                     // chunks, the last writes out O
    static constexpr int EV = 16 / ES;                     // elements per 16 bytes
    // staged rows: bf16 unpadded with XOR swizzles (K: kind 4 for rows of 16+
    // blocks, else 1; V: kind 5 for rows of 4 blocks, 2 for longer ones), fp32
    // padded by one block; Tb arrives as its lane-linear operand blocks
    static constexpr int KB = DK / EV, VB = DVT / EV;
    static constexpr int KP = BF ? KB : KB + 1, VP = BF ? VB : VB + 1;
    static constexpr int KSW = BF ? (KB >= 16 ? 4 : 1) : 0;
    static constexpr int VSW = BF && VB == 4 ? 5 : BF && VB > 4 ? 2 : 0;
    static constexpr int LDK = KP * EV, LDV = VP * EV;
    static constexpr int NDB = DK / 16;                    // state tiles per column wave
    static constexpr int NP = (NW + 1) / 2;                // pairs of token blocks
    static constexpr int KS = Step<T>::KS, NKK = DK / KS;  // contraction steps over d
    // staging buffer: regions K | Tb | V slice | gates, in whole 1 KB blocks,
    // each one direct-to-LDS load of 16 bytes per lane; block i is loaded by
    // loading wave i % NLD, as its load i / NLD
    static constexpr int blocks(int bytes) { return (bytes + 1023) / 1024; }
    static constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }
    static constexpr int NIK = blocks(C * LDK * ES), NIV = blocks(C * LDV * ES);
    static constexpr int NIT = HAS_TB ? tb_blocks(C, BF) : 0, NIG = blocks(GF * 4);
    static constexpr int BT = NIK, BV = BT + NIT, BG = BV + NIV, NI = BG + NIG;
    static constexpr size_t SZ_STAGE = (size_t)NI * 1024;
    static constexpr size_t OFF_T = (size_t)BT * 1024, OFF_V = (size_t)BV * 1024, OFF_G = (size_t)BG * 1024;
    // column-wave hand-over, lane by lane in MFMA operand form (one tile is 64
    // lanes of 4 values): the state at the next chunk's start (NDB tiles per
    // column wave) and V' (NW tiles per column wave); two buffers each (chunk
    // parity)
    static constexpr int TILE = 64 * 4 * ES;
    static constexpr size_t SZ_SB = MAPS ? 0 : (size_t)NVW * NDB * TILE, SZ_VO = MAPS ? 0 : (size_t)NVW * NW * TILE;
    // the chunk's output slice, handed from the output helpers to the staging
    // waves: rows of DVT values padded by 16 bytes; two buffers (chunk parity)
    static constexpr int LDO = DVT * ES + 16;                  // row pitch (bytes)
    static constexpr int OPR = DVT * ES / 16;                  // 16-byte pieces per row
    static constexpr int NOPL = cdiv(C * OPR, 64);             // pieces per writing lane
    // cache policy of the output stores: a slice row of less than a 128-byte
    // line leaves the rest of the line to the neighbouring slices, so its
    // stores stay in L2 (which holds a unit's slices) until the line is whole;
    // whole lines stream past the caches (nontemporal)
    static constexpr int OAUX = DVT * ES < 128 ? 0 : 2;
    static constexpr size_t SZ_O = MAPS ? 0 : (size_t)C * LDO;
    // Q of a chunk: staged by the loader one chunk ahead in two LDS buffers
    // (rows as K's) where that fits next to three staging buffers (QLDS), else
    // loaded by the output helpers straight into registers, NQS chunks ahead
    static constexpr size_t SZ_Q = (size_t)NIK * 1024;
    static constexpr size_t SZ_REST = 2 * SZ_SB + 2 * SZ_VO + 2 * SZ_O;
    // ns staging buffers (loads run ns - 1 chunks ahead), with or without the Q
    // buffers; the loader's wait for all but its newest ns - 2 chunks must stay
    // within the vmcnt range
    static constexpr bool fits(int ns, bool q) {
        return ns * SZ_STAGE + SZ_REST + (q ? 2 * SZ_Q : 0) <= 160 * 1024 && cdiv(NI, NLD) * (ns - 2) < 64;
    }
    static constexpr bool QLDS = !MAPS && fits(3, true);
    // The no-erase rule's gate rows: where the writing wave stages no Q (no
    // QLDS) it forms them itself in each chunk's staging buffer from log alpha
    // and beta (RawGates), and the loaders stage only the blocks before the
    // gate region; with QLDS, for fp32 and C = 64, the loading wave forms them
    // (GATES_BY_LOADER); elsewhere a per-chunk kernel writes them before the
    // scan.  Next to its Q pipeline the writing wave's loads would not keep
    // their order; for bf16 the loading wave's reads of the gates (a line per
    // token, in every column slice of a unit) cost the scan more than the
    // gates kernel takes, while fp32's longer chunk step absorbs them.
    static constexpr bool GATES_BY_LOADER = RULE == kNoErase && QLDS && C == 64 && !BF;
    static constexpr bool GATES_INLINE = RULE == kNoErase && (!QLDS || GATES_BY_LOADER);
    static constexpr int NIL = GATES_INLINE ? BG : NI;    // blocks loaded per chunk
    static constexpr int NL = cdiv(NIL, NLD);              // loads per loading lane per chunk
    // loads loading wave f issues per chunk
    static constexpr int nload(int f) { return NIL / NLD + (f < NIL % NLD ? 1 : 0); }
    static constexpr int NSTG = QLDS ? 3 : fits(4, false) ? 4 : fits(3, false) ? 3 : 2;
    static constexpr int DIST = NSTG - 1;                  // chunks staged ahead
    static constexpr size_t OFF_QB = NSTG * SZ_STAGE, OFF_SB = OFF_QB + (QLDS ? 2 * SZ_Q : 0);
    static constexpr size_t OFF_VO = OFF_SB + 2 * SZ_SB;
    static constexpr size_t OFF_O = OFF_VO + 2 * SZ_VO;
    // the no-erase rule's raw gates (log alpha, beta) where the loading wave
    // forms the gate rows: three slots of 2 C floats
    static constexpr size_t OFF_RG = OFF_O + 2 * SZ_O;
    static constexpr size_t SMEM = OFF_RG + (GATES_BY_LOADER ? 3 * 2 * C * 4 : 0);
    static constexpr bool FITS = SMEM <= 160 * 1024;
    // output helper of query block qb: 0 takes blocks 0 and NW - 1, 1 the middle
    // ones (wide slices: helper qb)
    static constexpr int pwave(int qb) {
        return NPP == 0 ? 0 : NPP >= NW ? qb : (qb < NW - 1 - qb ? qb : NW - 1 - qb) % NPP;
    }
    // the query blocks of helper hw, and how many
    static constexpr int nmine(int hw) {
        int c = 0;
        for (int qb = 0; qb < NW; ++qb) c += pwave(qb) == hw;
        return c;
    }
    static constexpr int mine(int hw, int j) {
        for (int qb = 0; qb < NW; ++qb)
            if (pwave(qb) == hw && j-- == 0) return qb;
        return 0;
    }
    static constexpr int NQB = NPP >= NW ? 1 : (NW + 1) / 2;   // query blocks per helper, at most
    // Q register sets without QLDS: three where a set takes at most 32 registers,
    // two below 64, else one (fp32 with Dk = 128: two sets would spill); the
    // wide slices one (with three, their ten-wave budget of 168 registers
    // spilled loop invariants, and each reload waited for every load in flight)
    static constexpr int NQS = WIDE ? 1 : NQB * NKK * 16 <= 128 ? 3 : NQB * NKK * 16 < 256 ? 2 : 1;
    static_assert(C % 16 == 0 && NW >= 1 && NW <= 4 && NVW >= 1 && (NVW <= 4 || MAPS) && NPP <= 4, "tile counts");
    static_assert(DV % DVT == 0 && DVT % 16 == 0 && DK % KS == 0 && DK % 16 == 0, "tile shapes");
    static_assert(!BF || (C % 32 == 0 && KB % 8 == 0 && (VB % 4 == 0 || VB == 2) && DK % 32 == 0),
                  "bf16 swizzles and tile pairs");
};

// logical d of row rho of state tile i
template <typename Cfg>
__device__ __forceinline__ constexpr int drow(int i, int rho) {
    if constexpr (Cfg::BF) return 32 * (i / 2) + 8 * (rho / 4) + 4 * (i % 2) + rho % 4;
    else return 16 * i + rho;
}

// region of staging load j of loading wave f: 0 K, 2 Tb, 3 V, 4 gates, 5 none
template <typename Cfg>
__device__ __forceinline__ constexpr int col_region(int j, int f) {
    const int i = j * Cfg::NLD + f;
    return i < Cfg::BT ? 0 : i < Cfg::BV ? 2 : i < Cfg::BG ? 3 : i < Cfg::NI ? 4 : 5;
}
// byte offset, relative to the chunk's first row, of lane l's 16 bytes of
// staging load j of loading wave f (kOutOfRange for padding)
template <typename Cfg>
__device__ __forceinline__ uint32_t col_stage_offset(int j, int f, int l, int64_t rs_k, int64_t rs_v) {
    constexpr int C = Cfg::NW * 16;
    const int i = j * Cfg::NLD + f;
    int64_t off = -1;
    auto region = [&](int s, int P, int B, int W, int64_t row_bytes) {
        const int r = s / P, p = s - r * P;
        if (r >= C || p >= B) return (int64_t)-1;
        int x = p;
        if (W == 1) x ^= swz<1>(r);
        else if (W == 2) x ^= swz<2>(r);
        else if (W == 3) x ^= swz<3>(r);
        else if (W == 4) x ^= swz<4>(r);
        else if (W == 5) x ^= swz<5>(r);
        return r * row_bytes + (int64_t)(x * 16);
    };
    switch (col_region<Cfg>(j, f)) {
        case 0: off = region(i * 64 + l, Cfg::KP, Cfg::KB, Cfg::KSW, rs_k); break;
        case 2: off = (int64_t)((i - Cfg::BT) * 64 + l) * 16; break;
        case 3: off = region((i - Cfg::BV) * 64 + l, Cfg::VP, Cfg::VB, Cfg::VSW, rs_v); break;
        case 4: {
            const int s = (i - Cfg::BG) * 64 + l;
            off = s < Cfg::GF / 4 ? (int64_t)s * 16 : -1;
            break;
        }
        default: break;
    }
    return (off < 0 || off >= (int64_t)kOutOfRange) ? kOutOfRange : (uint32_t)off;
}

// element (r, c) of the staged K (swizzled 16-byte blocks)
template <typename Cfg>
__device__ __forceinline__ int ckidx(int r, int c) { return sidx<Cfg, Cfg::KP, Cfg::KSW>(r, c); }

// K^T as the A operand of token block kb for state tile i: lane (g, n) gets
// K[kb*16 + 4g + e][drow(i, n)] (bf16: one transposing read -- lane s of group g
// supplies row kb*16 + 4g + s/4 at the 4-run of d holding drow(i, 4 (s%4));
// fp32: a gather)
template <typename Cfg, typename T>
__device__ __forceinline__ typename K16<T>::op kT_tile(const T* sK, int kb, int i) {
    const int l = lane_id(), g = l >> 4, n = l & 15;
    if constexpr (Cfg::BF) {
        return tr_read(sK + ckidx<Cfg>(kb * 16 + 4 * g + (n >> 2), drow<Cfg>(i, 4 * (n & 3))));
    } else {
        const T* p = sK + ckidx<Cfg>(kb * 16 + 4 * g, drow<Cfg>(i, n));
        return f32x4{p[0], p[Cfg::LDK], p[2 * Cfg::LDK], p[3 * Cfg::LDK]};
    }
}

// Rows of the scan's state beyond the plain forward (span maps):
//  vz   the first vz state rows start at the identity (row r = e_r) and take
//       zero values; row vz + j takes value column j of v.  After a span of
//       chunks those rows hold the product of the chunk maps S -> S M_c + B_c,
//       and the rest (from a zero start) hold the span's offset.
//  vld  elements per (token, head) row of v and O (DV - vz).
// O == NULL: no outputs; the output helpers and the writer only keep step.
struct ScanRows {
    int vz, vld;
};

// Per-token gates of the no-erase rule: log_alpha (NULL: 0) and beta (NULL:
// 1), [tokens][H] fp32, and the call's chunk slots.  Where the scan's
// configuration forms the gate rows itself (ColCfg::GATES_INLINE), its writing
// wave (or, with GATES_BY_LOADER, its loading wave) reads them; elsewhere the
// launcher runs the per-chunk gates kernel first.
struct RawGates {
    const float *log_alpha, *beta;
    int64_t slots;
};

template <typename T, int DK, int DV, int C, int DVT, int RULE>
__global__ __launch_bounds__((ColCfg<T, DK, DV, C, DVT, RULE>::BOUND)) void gdn_scan_cols_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* S0, SeqGeom geom, int H,
    const float* __restrict__ g_ws, const T* __restrict__ Tb_ws,
    T* __restrict__ O, float* S_T, ScanRows rows, RawGates raw) {   // S_T may alias S0
    using Cfg = ColCfg<T, DK, DV, C, DVT, RULE>;
    static_assert(Cfg::FITS, "scan workgroup exceeds the LDS of one CU");
    using St16 = Step<T>;
    using Frag = typename St16::frag;
    using KO = K16<T>;
    using Op = typename KO::op;
    constexpr int NW = Cfg::NW, NDB = Cfg::NDB, KS = Cfg::KS, NP = Cfg::NP, NKK = Cfg::NKK;
    constexpr int NVW = Cfg::NVW, ES = Cfg::ES;
    extern __shared__ __align__(16) unsigned char smem[];

    // Workgroups are dealt to the 8 XCDs round-robin by linear id; renumber them
    // so that the DV / DVT column slices of one (sequence, head) share an XCD and
    // its L2 serves their common K, Q, Tb and gate reads.
    int v0, h, seq;
    {
        constexpr int NS = DV / DVT;
        const int U = H * (int)gridDim.z;
        const int L = (int)(blockIdx.x + NS * (blockIdx.y + gridDim.y * blockIdx.z));
        const int lfull = (U / 8) * 8 * NS;
        int u, vs;
        if (L < lfull) {
            const int r = L >> 3;
            vs = r % NS;
            u = (L & 7) + 8 * (r / NS);
        } else {
            u = (U / 8) * 8 + (L - lfull) / NS;
            vs = (L - lfull) % NS;
        }
        v0 = vs * DVT;
        h = u % H;
        seq = geom.order ? geom.order[u / H] : u / H;   // packed batches: longest first
    }
    const int l = lane_id(), w = wave_id();
    const int n = l & 15, g4 = 4 * (l >> 4);

    int ts, te, first;
    if (geom.table) {
        ts = geom.bounds[seq];
        te = geom.bounds[seq + 1];
        first = geom.seq_slot[seq];
    } else if (geom.span_chunks > 0) {
        const int b = seq / geom.spans, p = seq - b * geom.spans;
        ts = b * geom.T + p * geom.span_chunks * C;
        te = min(ts + geom.span_chunks * C, (b + 1) * geom.T);
        first = b * geom.chunks_per_seq + p * geom.span_chunks;
    } else {
        ts = seq * geom.T;
        te = ts + geom.T;
        first = seq * geom.chunks_per_seq;
    }
    const int count = (te - ts + C - 1) / C;
    const int64_t sbase = ((int64_t)seq * H + h) * DV * DK;
    // token strides (bytes); v and O rows hold vld values, column v0 - vz
    const int64_t rs_k = (int64_t)H * DK * ES, rs_v = (int64_t)H * rows.vld * ES;
    const bool vzero = v0 < rows.vz;           // whole slice in the identity rows
    const int vc0 = v0 - rows.vz;              // first value column of the slice
    const bool no_out = Cfg::MAPS || O == nullptr;   // 128-column slices: span maps only

    auto barrier = [&]() __attribute__((always_inline)) {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    struct Staged {
        const T *K, *V, *Tb;
        const float *g, *gam, *dec, *beta;
    };
    auto staged = [&](int cc) __attribute__((always_inline)) {
        const unsigned char* sb = smem + (cc % Cfg::NSTG) * Cfg::SZ_STAGE;
        Staged st;
        st.K = reinterpret_cast<const T*>(sb);
        st.V = reinterpret_cast<const T*>(sb + Cfg::OFF_V);
        st.Tb = reinterpret_cast<const T*>(sb + Cfg::OFF_T);
        st.g = reinterpret_cast<const float*>(sb + Cfg::OFF_G);
        st.gam = st.g + C;
        st.dec = st.g + 2 * C;
        st.beta = st.g + 3 * C;   // kNoErase only
        return st;
    };
    // staged Q of chunk cd
    auto qbuf = [&](int cd) __attribute__((always_inline)) { return smem + Cfg::OFF_QB + (cd & 1) * Cfg::SZ_Q; };
    // hand-over tiles: tile i of column wave vb, this lane's 4 values
    auto sb_tile = [&](int cd, int vb, int i) __attribute__((always_inline)) {
        return reinterpret_cast<Op*>(smem + Cfg::OFF_SB + (cd & 1) * Cfg::SZ_SB + (vb * NDB + i) * Cfg::TILE) + l;
    };
    auto vo_tile = [&](int cd, int vb, int jb) __attribute__((always_inline)) {
        return reinterpret_cast<Op*>(smem + Cfg::OFF_VO + (cd & 1) * Cfg::SZ_VO + (vb * NW + jb) * Cfg::TILE) + l;
    };
    // output slice of chunk cd
    auto obuf = [&](int cd) __attribute__((always_inline)) { return smem + Cfg::OFF_O + (cd & 1) * Cfg::SZ_O; };

    // ---- column wave vb
    auto run_col = [&](auto vb_const) __attribute__((always_inline)) {
        constexpr int vb = decltype(vb_const)::value;
        const int vcol = v0 + vb * 16 + n;                 // this lane's state column
        f32x4 St[NDB];
#pragma unroll
        for (int i = 0; i < NDB; ++i) {
            if (vcol < rows.vz) {   // identity row: 1 at d = vcol
                const int d0 = drow<Cfg>(i, g4);
                St[i] = f32x4{d0 == vcol ? 1.f : 0.f, d0 + 1 == vcol ? 1.f : 0.f, d0 + 2 == vcol ? 1.f : 0.f,
                              d0 + 3 == vcol ? 1.f : 0.f};
            } else {
                St[i] = S0 ? *reinterpret_cast<const f32x4*>(S0 + sbase + (int64_t)vcol * DK + drow<Cfg>(i, g4))
                           : zero4();
            }
        }
        // the state slice as MFMA operands (input dtype), for this wave's Y and
        // for the output helpers' Z^T of chunk 0
        Op Sb[NDB];
#pragma unroll
        for (int i = 0; i < NDB; ++i) {
            Sb[i] = KO::tile(St[i]);
            if constexpr (!Cfg::MAPS) *sb_tile(0, vb, i) = Sb[i];
        }
        __syncthreads();

        // One chunk.  All K fragments of Y and the chunk's Tb rows, gates and V
        // values are requested as it starts, the K^T operands of the state
        // update right after the Y instructions.
        // K fragments in flight: all contraction steps of Y where they take at
        // most 64 registers, else a ring of that many
        constexpr int KPF = Cfg::WIDE ? 2 : NKK * NW * (int)sizeof(Frag) <= 256 ? NKK : 256 / (NW * (int)sizeof(Frag));
        auto step = [&](const int cc) __attribute__((always_inline)) {
            const Staged st = staged(cc);
            float4 dec4[NW];
            f32x4 vv[NW], Vp[NW];
            Op kt[NDB][NW];   // K^T operands of the state update
            const float gamma_n = Cfg::GLA ? 1.f : st.gam[C - 1];
            if constexpr (Cfg::ERASE) {
                Frag fk[KPF][NW];
#pragma unroll
                for (int kk = 0; kk < KPF; ++kk)
#pragma unroll
                    for (int tb = 0; tb < NW; ++tb) fk[kk][tb] = kfrag_rows<Cfg>(st.K, tb * 16, kk * KS);
                float4 gam4[NW];
                typedef typename std::conditional<Cfg::BF, bf16x8, f32x4>::type TFrag;
                constexpr int NTP = Cfg::BF ? NP : NW;
                TFrag ta[NW][NTP];
#pragma unroll
                for (int tb = 0; tb < NW; ++tb) {
                    gam4[tb] = *reinterpret_cast<const float4*>(st.gam + tb * 16 + g4);
                    dec4[tb] = *reinterpret_cast<const float4*>(st.dec + tb * 16 + g4);
                    vv[tb] = vcol4<Cfg>(st.V, tb, vb);
                }
#pragma unroll
                for (int ib = 0; ib < NW; ++ib)
#pragma unroll
                    for (int p = 0; p < NTP; ++p)
                        if ((Cfg::BF ? 2 * p : p) <= ib)
                            ta[ib][p] = *reinterpret_cast<const TFrag*>(reinterpret_cast<const unsigned char*>(st.Tb) +
                                                                        tb_block(ib, p, Cfg::BF) * 1024 + l * 16);
                // Y = K S^T (A: K rows; B: the state tiles) for every token block
                f32x4 Y[NW];
#pragma unroll
                for (int tb = 0; tb < NW; ++tb) Y[tb] = zero4();
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
                    for (int tb = 0; tb < NW; ++tb) {
                        if constexpr (Cfg::BF) Y[tb] = KO::mma2p(fk[kk % KPF][tb], Sb[2 * kk], Sb[2 * kk + 1], Y[tb]);
                        else Y[tb] = St16::mma(fk[kk % KPF][tb], Sb[kk], Y[tb]);
                    }
                    if (kk + KPF < NKK) {
#pragma unroll
                        for (int tb = 0; tb < NW; ++tb) fk[kk % KPF][tb] = kfrag_rows<Cfg>(st.K, tb * 16, (kk + KPF) * KS);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < NDB; ++i)
#pragma unroll
                    for (int kb = 0; kb < NW; ++kb) kt[i][kb] = kT_tile<Cfg>(st.K, kb, i);
                // X = V - diag(gamma) Y, as the B operand of V' = Tb X
                Op Xo[NW];
#pragma unroll
                for (int tb = 0; tb < NW; ++tb)
                    Xo[tb] = KO::tile(f32x4{vv[tb][0] - gam4[tb].x * Y[tb][0], vv[tb][1] - gam4[tb].y * Y[tb][1],
                                            vv[tb][2] - gam4[tb].z * Y[tb][2], vv[tb][3] - gam4[tb].w * Y[tb][3]});
                // V' = Tb X (A: Tb rows, token pairs as X)
#pragma unroll
                for (int ib = 0; ib < NW; ++ib) {
                    f32x4 acc = zero4();
                    if constexpr (Cfg::BF) {
#pragma unroll
                        for (int p = 0; p < NP; ++p)
                            if (2 * p <= ib) acc = KO::mma2p(ta[ib][p], Xo[2 * p], Xo[2 * p + 1], acc);
                    } else {
#pragma unroll
                        for (int jb = 0; jb <= ib; ++jb) acc = KO::mma1(ta[ib][jb], Xo[jb], acc);
                    }
                    Vp[ib] = acc;
                }
            } else if constexpr (Cfg::GLA) {
                // the decays and beta are in K^: V' = V
#pragma unroll
                for (int i = 0; i < NDB; ++i)
#pragma unroll
                    for (int kb = 0; kb < NW; ++kb) kt[i][kb] = kT_tile<Cfg>(st.K, kb, i);
#pragma unroll
                for (int tb = 0; tb < NW; ++tb) {
                    dec4[tb] = float4{1.f, 1.f, 1.f, 1.f};
                    vv[tb] = vcol4<Cfg>(st.V, tb, vb);
                    Vp[tb] = vv[tb];
                }
            } else {
                // no prediction to remove: V' = diag(beta) V
#pragma unroll
                for (int i = 0; i < NDB; ++i)
#pragma unroll
                    for (int kb = 0; kb < NW; ++kb) kt[i][kb] = kT_tile<Cfg>(st.K, kb, i);
#pragma unroll
                for (int tb = 0; tb < NW; ++tb) {
                    dec4[tb] = *reinterpret_cast<const float4*>(st.dec + tb * 16 + g4);
                    const float4 b4 = *reinterpret_cast<const float4*>(st.beta + tb * 16 + g4);
                    vv[tb] = vcol4<Cfg>(st.V, tb, vb);
                    Vp[tb] = f32x4{vv[tb][0] * b4.x, vv[tb][1] * b4.y, vv[tb][2] * b4.z, vv[tb][3] * b4.w};
                }
            }
            // gamma_n S^T while V' completes (kGla: e^(b_n) of each row's key channel)
            if constexpr (Cfg::GLA) {
#pragma unroll
                for (int i = 0; i < NDB; ++i) {
                    const float4 e4 = *reinterpret_cast<const float4*>(st.g + drow<Cfg>(i, g4));
                    St[i] = f32x4{St[i][0] * e4.x, St[i][1] * e4.y, St[i][2] * e4.z, St[i][3] * e4.w};
                }
            } else {
#pragma unroll
                for (int i = 0; i < NDB; ++i) St[i] *= gamma_n;
            }
            // S^T <- gamma_n S^T + K^T diag(gamma_n / gamma) V'
            Op Vd[NW];
#pragma unroll
            for (int jb = 0; jb < NW; ++jb)
                Vd[jb] = KO::tile(f32x4{Vp[jb][0] * dec4[jb].x, Vp[jb][1] * dec4[jb].y, Vp[jb][2] * dec4[jb].z,
                                        Vp[jb][3] * dec4[jb].w});
            // V' for the output helpers (A operand of O^T = V'^T P^T)
            if constexpr (!Cfg::MAPS) {
#pragma unroll
                for (int jb = 0; jb < NW; ++jb) *vo_tile(cc, vb, jb) = KO::tile(Vp[jb]);
            }
#pragma unroll
            for (int p = 0; p < NP; ++p)
#pragma unroll
                for (int i = 0; i < NDB; ++i) {
                    if (2 * p + 1 < NW)
                        St[i] = KO::mma2(kt[i][2 * p], kt[i][2 * p + 1], Vd[2 * p], Vd[2 * p + 1], St[i]);
                    else
                        St[i] = KO::mma1(kt[i][2 * p], Vd[2 * p], St[i]);
                }
            // the next chunk's state as operands, here and for the output helpers
#pragma unroll
            for (int i = 0; i < NDB; ++i) {
                Sb[i] = KO::tile(St[i]);
                if constexpr (!Cfg::MAPS) *sb_tile(cc + 1, vb, i) = Sb[i];
            }
            wait_vm_lgkm0<63>();
            barrier();
        };
        for (int cc = 0; cc < count; ++cc) step(cc);
        __syncthreads();   // the output helpers form the last output slice, the staging waves write it

        if (S_T) {
#pragma unroll
            for (int i = 0; i < NDB; ++i)
                *reinterpret_cast<f32x4*>(S_T + sbase + (int64_t)vcol * DK + drow<Cfg>(i, g4)) = St[i];
        }
    };

    // ---- output helper hw: P^T and Z^T of its query blocks for chunk cc in
    // step cc (kept in registers), their output in step cc + 1
    auto run_out = [&](auto hw_const) __attribute__((always_inline)) {
        constexpr int hw = decltype(hw_const)::value;
        if (no_out) {   // (uniform) no outputs: keep step with the other waves
            __syncthreads();
            for (int cc = 0; cc < count; ++cc) barrier();
            __syncthreads();
            return;
        }
        constexpr int NM = Cfg::nmine(hw);
        // without QLDS: Q rows of this helper's query blocks straight into
        // registers, lane (g, n) getting Q[qb*16 + n][kk*KS + g*EV ..] (rows past
        // the chunk end read as zeros)
        auto q_load = [&](Frag (*qr)[NKK], int cd) __attribute__((always_inline)) {
            const int t0 = ts + cd * C, len = min(C, te - t0);
            const __amdgpu_buffer_rsrc_t rq =
                make_rsrc(q + ((int64_t)t0 * H + h) * DK, (len - 1) * rs_k + DK * ES);
#pragma unroll
            for (int j = 0; j < NM; ++j)
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk)
                    qr[j][kk] = __builtin_bit_cast(
                        Frag, __builtin_amdgcn_raw_buffer_load_b128(
                                  rq, (uint32_t)((Cfg::mine(hw, j) * 16 + n) * rs_k) + kk * KS * ES + (l >> 4) * 16, 0, 0));
        };
        // P^T pairs (bf16: key blocks 2p, 2p + 1 in one operand) or tiles, and
        // Z^T diag(gamma) of the pending chunk
        constexpr int NPQ = Cfg::BF ? NP : NW;
        typedef typename std::conditional<Cfg::BF, s16x8, f32x4>::type PFrag;
        PFrag pp[Cfg::NQB][NPQ];
        f32x4 zp[Cfg::NQB][NVW];
        // output of chunk cd (its V' published by the last barrier, read into vo)
        auto out = [&](int cd, const Op (*vo_in)[NW]) __attribute__((always_inline)) {
            unsigned char* ob = obuf(cd) + n * Cfg::LDO + g4 * ES;
#pragma unroll
            for (int vb = 0; vb < NVW; ++vb) {
                Op vw[NW];   // V' tiles of column wave vb (wide slices: read here)
#pragma unroll
                for (int jb = 0; jb < NW; ++jb) {
                    if constexpr (Cfg::WIDE) vw[jb] = *vo_tile(cd, vb, jb);
                    else vw[jb] = vo_in[vb][jb];
                }
#pragma unroll
                for (int j = 0; j < NM; ++j) {
                    const int qb = Cfg::mine(hw, j);
                    f32x4 acc = zp[j][vb];
                    if constexpr (Cfg::BF) {
#pragma unroll
                        for (int p = 0; p < NP; ++p)
                            if (2 * p <= qb)
                                acc = KO::mma2(vw[2 * p], vw[2 * p + 1], __builtin_shufflevector(pp[j][p], pp[j][p], 0, 1, 2, 3),
                                               __builtin_shufflevector(pp[j][p], pp[j][p], 4, 5, 6, 7), acc);
                    } else {
#pragma unroll
                        for (int jb = 0; jb < NW; ++jb)
                            if (jb <= qb) acc = KO::mma1(vw[jb], pp[j][jb], acc);
                    }
                    store4(reinterpret_cast<T*>(ob + qb * 16 * Cfg::LDO + vb * 16 * ES), acc[0], acc[1], acc[2], acc[3]);
                }
            }
        };
        constexpr int QMAX = Cfg::mine(hw, NM - 1);   // the largest query block
        auto step = [&](const int cc, Frag (*qcur)[NKK]) __attribute__((always_inline)) {
            const Staged st = staged(cc);
            const T* sQ = reinterpret_cast<const T*>(qbuf(cc));
            // K and Q fragments and state tiles of one contraction step,
            // requested a step ahead of their use (two register sets; wide
            // slices: one set, requested as the step starts)
            Frag kf[Cfg::WIDE ? 1 : 2][NW], qf[Cfg::WIDE ? 1 : 2][Cfg::NQB];
            Op sbk[Cfg::WIDE ? 1 : 2][NVW][2];
            auto fetch = [&](int kk, int s) __attribute__((always_inline)) {
                if constexpr (!Cfg::GLA) {   // kGla: P~ arrives formed
#pragma unroll
                    for (int jb = 0; jb <= QMAX; ++jb) kf[s][jb] = kfrag_rows<Cfg>(st.K, jb * 16, kk * KS);
                }
#pragma unroll
                for (int j = 0; j < NM; ++j)
                    qf[s][j] = Cfg::QLDS ? kfrag_rows<Cfg>(sQ, Cfg::mine(hw, j) * 16, kk * KS) : qcur[j][kk];
                if constexpr (!Cfg::WIDE) {
#pragma unroll
                    for (int vb = 0; vb < NVW; ++vb) {
                        sbk[s][vb][0] = *sb_tile(cc, vb, Cfg::BF ? 2 * kk : kk);
                        if constexpr (Cfg::BF) sbk[s][vb][1] = *sb_tile(cc, vb, 2 * kk + 1);
                    }
                }
            };
            // the first contraction step's operands and V' of the pending chunk
            // (whose output goes out after the first step's instructions)
            if constexpr (!Cfg::WIDE) fetch(0, 0);
            Op vo[Cfg::WIDE ? 1 : NVW][NW];
            if (!Cfg::WIDE && cc > 0) {
#pragma unroll
                for (int vb = 0; vb < NVW; ++vb)
#pragma unroll
                    for (int jb = 0; jb < NW; ++jb) vo[vb][jb] = *vo_tile(cc - 1, vb, jb);
            }
            float gq[Cfg::NQB], gamq[Cfg::NQB];
#pragma unroll
            for (int j = 0; j < NM; ++j) {
                gq[j] = Cfg::GLA ? 0.f : st.g[Cfg::mine(hw, j) * 16 + n];
                gamq[j] = Cfg::GLA ? 1.f : st.gam[Cfg::mine(hw, j) * 16 + n];
            }
            // decay factors of the P^T tiles of key block jb (zero above the
            // diagonal), formed between the instructions of a contraction step
            f32x4 dfac[Cfg::NQB][NW];
            auto decay = [&](int jb) __attribute__((always_inline)) {
                const float4 gj = *reinterpret_cast<const float4*>(st.g + jb * 16 + g4);
                const int j0 = jb * 16 + g4;
#pragma unroll
                for (int j = 0; j < NM; ++j) {
                    const int cq = Cfg::mine(hw, j) * 16 + n;
                    if (jb <= Cfg::mine(hw, j))
                        dfac[j][jb] = f32x4{j0 + 0 <= cq ? __expf(gq[j] - gj.x) : 0.f, j0 + 1 <= cq ? __expf(gq[j] - gj.y) : 0.f,
                                            j0 + 2 <= cq ? __expf(gq[j] - gj.z) : 0.f, j0 + 3 <= cq ? __expf(gq[j] - gj.w) : 0.f};
                }
            };
            // P^T tiles (rows: key tokens) and Z^T (rows: state columns) of this
            // helper's query blocks
            f32x4 Pt[Cfg::NQB][NW], Zt[Cfg::NQB][NVW];
#pragma unroll
            for (int j = 0; j < Cfg::NQB; ++j) {
#pragma unroll
                for (int jb = 0; jb < NW; ++jb) Pt[j][jb] = zero4();
#pragma unroll
                for (int vb = 0; vb < NVW; ++vb) Zt[j][vb] = zero4();
            }
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                const int s = kk & 1;
                const int ss = Cfg::WIDE ? 0 : s;
                if constexpr (Cfg::WIDE) {
#pragma unroll
                    for (int vb = 0; vb < NVW; ++vb) {
                        sbk[0][vb][0] = *sb_tile(cc, vb, Cfg::BF ? 2 * kk : kk);
                        if constexpr (Cfg::BF) sbk[0][vb][1] = *sb_tile(cc, vb, 2 * kk + 1);
                    }
                }
                if constexpr (Cfg::WIDE) fetch(kk, 0);
                else if (kk + 1 < NKK) fetch(kk + 1, s ^ 1);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int j = 0; j < NM; ++j) {
                    const int qb = Cfg::mine(hw, j);
                    if constexpr (!Cfg::GLA) {
#pragma unroll
                        for (int jb = 0; jb <= qb; ++jb) Pt[j][jb] = St16::mma(kf[ss][jb], qf[ss][j], Pt[j][jb]);
                    }
#pragma unroll
                    for (int vb = 0; vb < NVW; ++vb) {
                        if constexpr (Cfg::BF) {
                            const s16x8 qs = __builtin_bit_cast(s16x8, qf[ss][j]);
                            Zt[j][vb] = KO::mma2(sbk[ss][vb][0], sbk[ss][vb][1], __builtin_shufflevector(qs, qs, 0, 1, 2, 3),
                                                 __builtin_shufflevector(qs, qs, 4, 5, 6, 7), Zt[j][vb]);
                        } else {
                            Zt[j][vb] = St16::mma(sbk[ss][vb][0], qf[ss][j], Zt[j][vb]);
                        }
                    }
                }
                if constexpr (!Cfg::GLA && !Cfg::WIDE) {
#pragma unroll
                    for (int jb = kk; jb < NW; jb += NKK) decay(jb);
                    if (kk == NKK - 1) {
#pragma unroll
                        for (int jb = NKK; jb < NW; ++jb) decay(jb);
                    }
                }
                if (kk == 0 && cc > 0) out(cc - 1, Cfg::WIDE ? nullptr : vo);
                __builtin_amdgcn_sched_barrier(0);
            }
            // decay and mask P^T, scale Z^T by gamma at the query token; keep both
            if constexpr (!Cfg::GLA && Cfg::WIDE) {
#pragma unroll
                for (int jb = 0; jb < NW; ++jb) decay(jb);
            }
#pragma unroll
            for (int j = 0; j < NM; ++j) {
                const int qb = Cfg::mine(hw, j);
#pragma unroll
                for (int vb = 0; vb < NVW; ++vb) zp[j][vb] = Zt[j][vb] * gamq[j];
                if constexpr (Cfg::GLA) {
                    // P~ of this query block from the staged operand blocks
                    const unsigned char* pb = reinterpret_cast<const unsigned char*>(st.Tb) + l * 16;
#pragma unroll
                    for (int p = 0; p < NPQ; ++p)
                        if ((Cfg::BF ? 2 * p : p) <= qb)
                            pp[j][p] = *reinterpret_cast<const PFrag*>(pb + tb_block(qb, p, Cfg::BF) * 1024);
                } else {
#pragma unroll
                    for (int jb = 0; jb <= qb; ++jb) Pt[j][jb] *= dfac[j][jb];
                    if constexpr (Cfg::BF) {
#pragma unroll
                        for (int p = 0; p < NP; ++p)
                            if (2 * p <= qb)
                                pp[j][p] = __builtin_shufflevector(KO::tile(Pt[j][2 * p]),
                                                                   KO::tile(2 * p + 1 < NW ? Pt[j][2 * p + 1] : zero4()),
                                                                   0, 1, 2, 3, 4, 5, 6, 7);
                    } else {
#pragma unroll
                        for (int jb = 0; jb <= qb; ++jb) pp[j][jb] = Pt[j][jb];
                    }
                }
            }
            if constexpr (!Cfg::QLDS) q_load(qcur, min(cc + Cfg::NQS, count - 1));   // refill the set just used
            wait_vm_lgkm0<63>();
            barrier();
        };
        if constexpr (Cfg::QLDS) {
            __syncthreads();
            for (int cc = 0; cc < count; ++cc) step(cc, nullptr);
        } else {
            constexpr int NQS = Cfg::NQS;
            Frag qs[NQS][Cfg::NQB][NKK];
            if (count > 0) {
#pragma unroll
                for (int d = 0; d < NQS; ++d) q_load(qs[d], min(d, count - 1));
            }
            __syncthreads();
            int cc = 0;
            for (; cc + NQS <= count; cc += NQS) {
#pragma unroll
                for (int i = 0; i < NQS; ++i) step(cc + i, qs[i]);
            }
#pragma unroll
            for (int i = 0; i < NQS - 1; ++i)
                if (cc + i < count) step(cc + i, qs[i]);
        }
        if (count > 0) {   // its V' was published by the last barrier
            Op vo[NVW][NW];
#pragma unroll
            for (int vb = 0; vb < NVW; ++vb)
#pragma unroll
                for (int jb = 0; jb < NW; ++jb) vo[vb][jb] = *vo_tile(count - 1, vb, jb);
            out(count - 1, Cfg::WIDE ? nullptr : vo);
        }
        __syncthreads();
    };

    // ---- staging waves: wave f < NF - 1 loads its share of each chunk (so that
    // its vmcnt counts these loads alone), the last one writes out the output
    // slices
    auto run_stage = [&](auto f_const) __attribute__((always_inline)) {
        constexpr int f = decltype(f_const)::value;
        constexpr bool LOADER = f < Cfg::NLD;
        // staging: chunk cd's K, Tb, V slice and gates straight into the staging
        // buffer of cd % NSTG (rows past the chunk end fall outside the buffer
        // ranges and land as zeros); ND loads per call
        constexpr int ND = LOADER ? Cfg::nload(f) : 0;
        uint32_t soff[Cfg::NL];
#pragma unroll
        for (int j = 0; j < Cfg::NL; ++j) soff[j] = col_stage_offset<Cfg>(j, f, l, rs_k, rs_v);
        auto stage = [&](int cd) __attribute__((always_inline)) {
            const int t0 = ts + cd * C, len = min(C, te - t0);
            const int64_t unit = (int64_t)(first + cd) * H + h;
            const T* kb = k + ((int64_t)t0 * H + h) * DK;
            const T* vb_ = v + ((int64_t)t0 * H + h) * rows.vld + (vzero ? 0 : vc0);
            const T* tb = Tb_ws + unit * (Cfg::NIT * 1024 / ES);
            const float* gb = g_ws + unit * Cfg::GF;
            const int nk = (int)((len - 1) * rs_k + DK * ES), nv = vzero ? 0 : (int)((len - 1) * rs_v + DVT * ES);
            unsigned char* dst = smem + (cd % Cfg::NSTG) * Cfg::SZ_STAGE + f * 1024;
#pragma unroll
            for (int j = 0; j < Cfg::NL; ++j) {
                const int r = col_region<Cfg>(j, f);
                if (r == 5) continue;
                const void* base = r == 0 ? (const void*)kb : r == 2 ? (const void*)tb : r == 3 ? (const void*)vb_
                                 : (const void*)gb;
                const int nrec = r == 0 ? nk : r == 2 ? Cfg::NIT * 1024 : r == 3 ? nv : Cfg::GF * 4;
                lds_load16(make_rsrc(base, nrec), dst + j * Cfg::NLD * 1024, soff[j]);
            }
        };
        // chunk cd's Q into the Q buffer of its parity (the K blocks' offsets and
        // swizzle, as the loader lays out K), through registers: q_issue loads
        // into one of two register sets, q_commit writes LDS once the loads are
        // in.  The writing wave does it: step cc writes Q of chunk cc + 1, which
        // it requested two steps before, and requests Q of chunk cc + 3 into the
        // set just written from -- the loads have two steps to land, as the
        // staging loads do (with one step they did not: the wait for them set
        // the chunk step).  The loader then issues only its direct-to-LDS
        // staging loads.  (Through registers measured 3 to 5 us faster over the
        // headline than direct-to-LDS loads for Q, one chunk ahead.)  The LDS
        // writes are inline assembly so that the compiler inserts no wait for
        // unrelated memory operations before them.
        constexpr bool QW = !LOADER && Cfg::QLDS;
        u32x4 qreg[2][Cfg::NL];
        uint32_t qoff[Cfg::NL];
#pragma unroll
        for (int j = 0; j < Cfg::NL; ++j) qoff[j] = QW ? col_stage_offset<Cfg>(j, 0, l, rs_k, rs_v) : 0u;
        auto q_issue = [&](u32x4* qr, int cd) __attribute__((always_inline)) {
            const int t0 = ts + cd * C, len = min(C, te - t0);
            const __amdgpu_buffer_rsrc_t rq =
                make_rsrc(q + ((int64_t)t0 * H + h) * DK, (int)((len - 1) * rs_k + DK * ES));
#pragma unroll
            for (int j = 0; j < Cfg::NL; ++j)
                if (col_region<Cfg>(j, 0) == 0) qr[j] = __builtin_amdgcn_raw_buffer_load_b128(rq, qoff[j], 0, 0);
        };
        auto q_commit = [&](const u32x4* qr, int cd) __attribute__((always_inline)) {
            typedef __attribute__((address_space(3))) unsigned char lds_u8;
            const uint32_t base = (uint32_t)(uintptr_t)(lds_u8*)(qbuf(cd)) + l * 16;
#pragma unroll
            for (int j = 0; j < Cfg::NL; ++j)
                if (col_region<Cfg>(j, 0) == 0)
                    asm volatile("ds_write_b128 %0, %1" ::"v"(base + j * Cfg::NLD * 1024), "v"(qr[j]) : "memory");
        };
        // chunk cd's output slice from LDS to memory, 16 bytes per lane, rows
        // past the chunk end dropped by the buffer range (cache policy OAUX)
        auto write_out = [&](int cd) __attribute__((always_inline)) {
            const int t0 = ts + cd * C, len = min(C, te - t0);
            const __amdgpu_buffer_rsrc_t ro =
                make_rsrc(O + ((int64_t)t0 * H + h) * rows.vld + vc0, (len - 1) * rs_v + DVT * ES);
            const unsigned char* ob = obuf(cd);
#pragma unroll
            for (int j = 0; j < Cfg::NOPL; ++j) {
                const int piece = j * 64 + l;
                if (Cfg::NOPL * 64 == C * Cfg::OPR || piece < C * Cfg::OPR) {
                    const int r = piece / Cfg::OPR, b = piece - r * Cfg::OPR;
                    const u32x4 d = *reinterpret_cast<const u32x4*>(ob + r * Cfg::LDO + b * 16);
                    __builtin_amdgcn_raw_buffer_store_b128(d, ro, (uint32_t)(r * rs_v) + b * 16, 0, Cfg::OAUX);
                }
            }
        };
        // Loader: step cc stages K .. gates of chunk cc + DIST into the buffer
        // whose readers passed the previous barrier; before its closing barrier
        // it waits for all but the newest DIST - 1 chunks of staging loads, i.e.
        // for everything chunk cc + 1 needs (loads complete in issue order).
        // Writer: step cc writes Q of chunk cc + 1 (register set (cc + 1) & 1),
        // requests Q of chunk cc + 3 into that set and writes out the output
        // slice of chunk cc - 2; before the barrier it waits for its LDS writes.
        // (Q requested before the stores: the wait for Q's loads, which count in
        // vmcnt with the stores, leaves the newer stores in flight.)  Past the
        // end the last chunk is re-read (the same values).
        static_assert(ND * (Cfg::DIST - 1) < 64, "vmcnt range");
        // no-erase rule: the writing wave forms chunk cd's gate rows (g, e^g,
        // e^(g_n - g), beta; lane = token, rows past the chunk end as tokens with
        // log alpha = 0 and beta = 0) in its staging buffer, from the inputs it
        // requested a step before (gate_issue).  The loads take no branch (a
        // NULL input reads as an empty range), so that the waits the compiler
        // places for them and for the Q register sets count exactly.
        constexpr bool GW = Cfg::GATES_INLINE && (Cfg::GATES_BY_LOADER ? LOADER : !LOADER);
        float g_la = 0.f, g_be = 0.f;
        auto gate_issue = [&](int cd) __attribute__((always_inline)) {
            const int t0 = ts + cd * C, len = min(C, te - t0);
            const int64_t row0 = (int64_t)t0 * H + h;
            const int gbytes = ((len - 1) * H + 1) * 4;
            const uint32_t goff = l < C ? (uint32_t)(l * H * 4) : kOutOfRange;
            const float* la = raw.log_alpha ? raw.log_alpha + row0 : nullptr;
            const float* be = raw.beta ? raw.beta + row0 : nullptr;
            g_la = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(la, la ? gbytes : 0), goff, 0, 0));
            g_be = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(be, be ? gbytes : 0), goff, 0, 0));
        };
        // beta of lane l in chunk cd: as loaded, or 1 inside the chunk where
        // beta is NULL (chosen where the rows are written, so that no wait for
        // the load is placed where it is issued)
        auto gate_beta = [&](int cd, float b) __attribute__((always_inline)) {
            const int len = min(C, te - (ts + cd * C));
            return raw.beta ? b : (l < len ? 1.f : 0.f);
        };
        auto gate_commit = [&](int cd) __attribute__((always_inline)) {
            float gs = g_la;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(gs, off, 64);
                if (l >= off) gs += y;
            }
            const float glast = __shfl(gs, C - 1, 64);
            float* gb = reinterpret_cast<float*>(smem + (cd % Cfg::NSTG) * Cfg::SZ_STAGE + Cfg::OFF_G);
            if (l < C) {
                gb[l] = gs;
                gb[C + l] = __expf(gs);
                gb[2 * C + l] = __expf(glast - gs);
                gb[3 * C + l] = gate_beta(cd, g_be);
            }
        };
        // the same rows formed by the loading wave, which has direct-to-LDS loads
        // in flight (the compiler waits for all of them before any LDS access it
        // knows of): log alpha and beta arrive direct-to-LDS too, 4 bytes per
        // lane, in one of three slots (chunk index mod 3: a chunk's inputs are
        // requested while those of the two before it may be unread), and the
        // rows are formed from them with inline-assembly LDS reads and writes
        // and a DPP prefix sum (row shifts, then row broadcasts).  C = 64: one
        // lane per token.
        auto rg_slot = [&](int x) __attribute__((always_inline)) { return smem + Cfg::OFF_RG + (x % 3) * (2 * C * 4); };
        auto rg_issue = [&](int cd, int x) __attribute__((always_inline)) {
            const int t0 = ts + cd * C, len = min(C, te - t0);
            const int64_t row0 = (int64_t)t0 * H + h;
            const int gbytes = ((len - 1) * H + 1) * 4;
            const uint32_t goff = l < C ? (uint32_t)(l * H * 4) : kOutOfRange;
            const float* la = raw.log_alpha ? raw.log_alpha + row0 : nullptr;
            const float* be = raw.beta ? raw.beta + row0 : nullptr;
            lds_load4(make_rsrc(la, la ? gbytes : 0), rg_slot(x), goff);
            lds_load4(make_rsrc(be, be ? gbytes : 0), rg_slot(x) + C * 4, goff);
        };
        auto rg_commit = [&](int cd, int x) __attribute__((always_inline)) {
            static_assert(!GW || !LOADER || C == 64, "one lane per token");
            typedef __attribute__((address_space(3))) unsigned char lds_u8;
            const uint32_t ra = (uint32_t)(uintptr_t)(lds_u8*)rg_slot(x) + l * 4;
            float gs, b;
            asm volatile("ds_read_b32 %0, %2\n\tds_read_b32 %1, %2 offset:256\n\ts_waitcnt lgkmcnt(0)"
                         : "=&v"(gs), "=&v"(b) : "v"(ra) : "memory");
            auto dpp = [](float v, auto ctrl, auto rmask) __attribute__((always_inline)) {
                return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                             decltype(ctrl)::value, decltype(rmask)::value, 0xf, true));
            };
            gs += dpp(gs, std::integral_constant<int, 0x111>{}, std::integral_constant<int, 0xf>{});   // row_shr:1
            gs += dpp(gs, std::integral_constant<int, 0x112>{}, std::integral_constant<int, 0xf>{});   // row_shr:2
            gs += dpp(gs, std::integral_constant<int, 0x114>{}, std::integral_constant<int, 0xf>{});   // row_shr:4
            gs += dpp(gs, std::integral_constant<int, 0x118>{}, std::integral_constant<int, 0xf>{});   // row_shr:8
            gs += dpp(gs, std::integral_constant<int, 0x142>{}, std::integral_constant<int, 0xa>{});   // row_bcast:15
            gs += dpp(gs, std::integral_constant<int, 0x143>{}, std::integral_constant<int, 0xc>{});   // row_bcast:31
            const float glast = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, gs), C - 1));
            const uint32_t a0 = (uint32_t)(uintptr_t)(lds_u8*)(smem + (cd % Cfg::NSTG) * Cfg::SZ_STAGE + Cfg::OFF_G) + l * 4;
            const float ge = __expf(gs), gd = __expf(glast - gs), bv = gate_beta(cd, b);
            asm volatile("ds_write_b32 %0, %1" ::"v"(a0), "v"(gs) : "memory");
            asm volatile("ds_write_b32 %0, %1" ::"v"(a0 + C * 4), "v"(ge) : "memory");
            asm volatile("ds_write_b32 %0, %1" ::"v"(a0 + 2 * C * 4), "v"(gd) : "memory");
            asm volatile("ds_write_b32 %0, %1" ::"v"(a0 + 3 * C * 4), "v"(bv) : "memory");
        };
        if (count > 0) {
            if constexpr (LOADER && GW) {
                // the loads in the order of the steps (the raw gates of chunk
                // x + 2 ahead of the staging of chunk x + 1), then the rows of
                // chunks 0 and 1
                static_assert(Cfg::DIST == 2 && 2 * ND + 2 < 64, "staging two chunks ahead, vmcnt range");
                rg_issue(0, 0);
                rg_issue(min(1, count - 1), 1);
                stage(0);
                rg_issue(min(2, count - 1), 2);
                stage(min(1, count - 1));
                wait_vm_lgkm0<2 * ND + 2>();   // the raw gates of chunks 0 and 1
                rg_commit(0, 0);
                rg_commit(min(1, count - 1), 1);
                wait_vm_lgkm0<ND + 2>();       // chunk 0's staging
            } else if constexpr (GW) {
                gate_issue(0);
                gate_commit(0);
                gate_issue(min(1, count - 1));
            }
            if constexpr (LOADER && !GW) {
#pragma unroll
                for (int d = 0; d < Cfg::DIST; ++d) stage(min(d, count - 1));
                wait_vm_lgkm0<ND * (Cfg::DIST - 1)>();
            } else if constexpr (!LOADER && QW) {
                if (!no_out) {
                    q_issue(qreg[0], 0);
                    q_commit(qreg[0], 0);
                    q_issue(qreg[1], min(1, count - 1));
                    q_issue(qreg[0], min(2, count - 1));
                    wait_vm_lgkm0<63>();
                }
            }
        }
        __syncthreads();
        auto writer_step = [&](int cc, u32x4* qr) __attribute__((always_inline)) {
            // past the end the last chunk's gates are formed again (the same values)
            if constexpr (GW) {
                gate_commit(min(cc + 1, count - 1));
                gate_issue(min(cc + 2, count - 1));
            }
            if constexpr (QW) {
                if (!no_out) {
                    q_commit(qr, min(cc + 1, count - 1));
                    q_issue(qr, min(cc + 3, count - 1));
                }
            }
            if (cc >= 2 && !no_out) write_out(cc - 2);       // formed by the output helpers last step
            wait_vm_lgkm0<63>();
            barrier();
        };
        if constexpr (LOADER && GW) {
            // step cc: the raw gates of chunk cc + 3 and the staging of chunk
            // cc + 2; then chunk cc + 2's rows from its raw gates (requested a
            // step before, ahead of chunk cc + 1's staging, so the wait does not
            // hang on that) into its staging buffer, free since the last barrier
            for (int cc = 0; cc < count; ++cc) {
                rg_issue(min(cc + 3, count - 1), cc + 3);
                stage(min(cc + 2, count - 1));
                wait_vm_lgkm0<2 * ND + 2>();
                rg_commit(min(cc + 2, count - 1), cc + 2);
                wait_vm_lgkm0<ND + 2>();   // chunk cc + 1's staging
                barrier();
            }
        } else if constexpr (LOADER) {
            for (int cc = 0; cc < count; ++cc) {
                stage(min(cc + Cfg::DIST, count - 1));
                wait_vm_lgkm0<ND * (Cfg::DIST - 1)>();
                barrier();
            }
        } else {
            // two steps per iteration, so that each register set is a fixed one
            for (int cc = 0; cc < count; cc += 2) {
                writer_step(cc, qreg[1]);
                if (cc + 1 < count) writer_step(cc + 1, qreg[0]);
            }
        }
        wait_vm_lgkm0<0>();   // no load still writing LDS when the workgroup ends
        __syncthreads();      // the output helpers have formed the last output slice
        if constexpr (!LOADER) {
            if (count >= 2 && !no_out) write_out(count - 2);
            if (count >= 1 && !no_out) write_out(count - 1);
        }
    };

    // waves: the column waves, the output helpers, the loader, the writer
    if constexpr (Cfg::MAPS) {
        static_assert(NVW == 8 && Cfg::NPP == 0, "span-map slices: eight column waves, no helpers");
        switch (w) {
            case 0: run_col(std::integral_constant<int, 0>{}); break;
            case 1: run_col(std::integral_constant<int, 1>{}); break;
            case 2: run_col(std::integral_constant<int, 2>{}); break;
            case 3: run_col(std::integral_constant<int, 3>{}); break;
            case 4: run_col(std::integral_constant<int, 4>{}); break;
            case 5: run_col(std::integral_constant<int, 5>{}); break;
            case 6: run_col(std::integral_constant<int, 6>{}); break;
            case 7: run_col(std::integral_constant<int, 7>{}); break;
            case 8: run_stage(std::integral_constant<int, 0>{}); break;
            default: run_stage(std::integral_constant<int, 1>{}); break;
        }
    } else if constexpr (!Cfg::WIDE) {
        if (w < NVW) {
            if (w == 0) run_col(std::integral_constant<int, 0>{});
            else if constexpr (NVW > 1) run_col(std::integral_constant<int, (NVW > 1 ? 1 : 0)>{});
        } else {
            switch (w - NVW) {
                case 0: run_out(std::integral_constant<int, 0>{}); break;
                case 1: run_out(std::integral_constant<int, 1>{}); break;
                case 2: run_stage(std::integral_constant<int, 0>{}); break;
                default: run_stage(std::integral_constant<int, 1>{}); break;
            }
        }
    } else {
        static_assert(NVW == 4 && Cfg::NPP == 4, "wide slices: four column waves and four helpers");
        switch (w) {
            case 0: run_col(std::integral_constant<int, 0>{}); break;
            case 1: run_col(std::integral_constant<int, 1>{}); break;
            case 2: run_col(std::integral_constant<int, 2>{}); break;
            case 3: run_col(std::integral_constant<int, 3>{}); break;
            case 4: run_out(std::integral_constant<int, 0>{}); break;
            case 5: run_out(std::integral_constant<int, 1>{}); break;
            case 6: run_out(std::integral_constant<int, 2>{}); break;
            case 7: run_out(std::integral_constant<int, 3>{}); break;
            case 8: run_stage(std::integral_constant<int, 0>{}); break;
            default: run_stage(std::integral_constant<int, 1>{}); break;
        }
    }
}

}  // namespace gdn
