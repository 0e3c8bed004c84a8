// gdn_scan.h -- serial inter-chunk state scan with the chunk outputs fused in.
//
// One workgroup owns a DVT-column slice of the state of one (sequence, head)
// and walks that sequence's chunks in order, holding its slice of S^T
// (Dk x DVT, fp32) in MFMA accumulators for the whole sequence.  Rows of S
// evolve independently (the update of the Qiita article on the Linear
// Attention lineage, section "Gated-DeltaNet", writes row r of S only from
// v_t[r] and k_t), so slicing Dv needs no communication between workgroups.
//
// Per chunk (row form, S = state at the chunk start, Dv x Dk; gamma_i = exp(g_i);
// Tb = T diag(beta) from the prep kernel):
//   Y  = K S^T,   X = V - diag(gamma) Y            prediction errors vs. the gated start state
//   V' = Tb X     (= U - W S^T)                    corrected for the chunk's earlier writes
//   O^T = Z^T diag(gamma) + V'^T P^T,  Z^T = S Q^T, P = (Q K^T) o Gamma o M
//   S^T <- gamma_n S^T + K^T diag(gamma_n / gamma) V'
// Sources: the same Qiita section (product form of S_i with I - sum w k^T =
// A_1..A_i and the G_i identity; parallel form H = S0 (Q - W (M^T o K^T Q)) D_gamma
// + U (Gamma o K^T Q) restricted to one chunk) and its section "Chunk
// Computation" (chunk j starts from chunk j-1's last state);
// LinearAttention系列解读(六)：DeltaNet的Chunkwise Form推导, section 4.4 (U - W S^T is
// each token's prediction error against the chunk-start state, corrected by the
// triangular solve) and section 4.5 (T, W, U do not depend on S).
//
// Work split: one wave per (token block cb, 16-column block vb) tile, NW x NVB
// waves (8 for a 64-token chunk and a 32-column slice, two per SIMD).  Per chunk:
//  phase A  each wave computes its tile of Y and Z^T and the P^T tiles of its
//           token block, and writes its tile of X (transposed) to LDS; barrier;
//  phase B  each wave computes V' for all token blocks of its column block
//           from X^T and Tb (that small redundancy keeps V' in registers for
//           both O and the state update), its O tile, and its two tiles of the
//           new state (d-blocks cb, cb + NW), whose copy goes to LDS; barrier.
// Register tiles feed MFMAs directly: a 16x16 accumulator tile (lane (g, n):
// rows 4g..4g+3 of column n) is, per lane, an operand of a 16-deep contraction
// block -- B when its rows are the contraction index, A of its transpose when
// its columns are -- and two such blocks form one 16x16x32 bf16 operand,
// provided A and B pair the same blocks.
//
// Data movement:
//  - K, Q, the V slice, Tb and the gates of chunk cc + 2 are loaded into
//    registers at the start of step cc (range-checked buffer loads: rows past
//    the chunk end read as zeros) and written to the free one of two LDS
//    staging buffers at the end of step cc + 1.
//  - O leaves through range-checked buffer stores, so the padded rows of a
//    last chunk are dropped without a branch.
//  - LDS pitches and XOR swizzles keep each access pattern free of bank
//    conflicts on 32 banks; on bf16, columns of row-major K and V are read with
//    the transposing LDS load, which hands each lane 4 rows of one column.
#pragma once

#include <type_traits>

#include "gdn_device.h"

namespace gdn {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// s_waitcnt with vmcnt <= vm and lgkmcnt = 0 (expcnt not waited on)
template <int VM>
__device__ __forceinline__ void wait_vm_lgkm0() {
    static_assert(VM >= 0 && VM < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | ((VM >> 4) << 14));
}

// Operand of one 16-deep contraction block: lane (g, n) holds k = 4g .. 4g+3
// for row / column n of the other dimension.  A 16x16 accumulator tile has
// exactly this layout, with k = its row.
template <typename T> struct K16;
template <> struct K16<bf16> {
    typedef s16x4 op;
    __device__ __forceinline__ static op tile(f32x4 t) {
        const bf16x4 v = {(bf16)t[0], (bf16)t[1], (bf16)t[2], (bf16)t[3]};
        return __builtin_bit_cast(s16x4, v);
    }
    __device__ __forceinline__ static f32x4 mma1(op a, op b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
    }
    // blocks (a0, b0) and (a1, b1) in one 16x16x32 instruction
    __device__ __forceinline__ static f32x4 mma2(op a0, op a1, op b0, op b1, f32x4 c) {
        const s16x8 a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
        return mma2p(__builtin_bit_cast(bf16x8, a), b0, b1, c);
    }
    // the A pair already packed (a0 in elements 0..3, a1 in 4..7)
    __device__ __forceinline__ static f32x4 mma2p(bf16x8 a, op b0, op b1, f32x4 c) {
        const s16x8 b = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};
template <> struct K16<float> {
    typedef f32x4 op;
    __device__ __forceinline__ static op tile(f32x4 t) { return t; }
    __device__ __forceinline__ static f32x4 mma1(op a, op b, f32x4 c) {
#pragma unroll
        for (int r = 0; r < 4; ++r) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[r], b[r], c, 0, 0, 0);
        return c;
    }
    __device__ __forceinline__ static f32x4 mma2(op a0, op a1, op b0, op b1, f32x4 c) {
        return mma1(a1, b1, mma1(a0, b0, c));
    }
};

__device__ __forceinline__ float bf16_bits_to_f32(short x) {
    return __builtin_bit_cast(float, (unsigned)(unsigned short)x << 16);
}

// Transposing 64-bit LDS read (ds_read_b64_tr_b16): within each 16-lane group,
// lane s supplies the address of 4 consecutive 16-bit values; lane j receives
// value j % 4 of lane 4e + j / 4 as its element e.
__device__ __forceinline__ s16x4 tr_read(const void* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

// 4 consecutive values of one lane, rounded to T, as one 8- or 16-byte LDS store
template <typename T>
__device__ __forceinline__ void store4(T* p, float a, float b, float c, float d) {
    if constexpr (sizeof(T) == 2) {
        const bf16x4 v = {(bf16)a, (bf16)b, (bf16)c, (bf16)d};
        *reinterpret_cast<bf16x4*>(p) = v;
    } else {
        *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
    }
}

template <typename T, int DK, int DV, int C, int DVT>
struct ScanCfg {
    static constexpr bool BF = sizeof(T) == 2;
    static constexpr int ES = sizeof(T);
    static constexpr int NW = C / 16;                      // 16-token blocks = waves of each role
    static constexpr int NVB = DVT / 16;                   // 16-column blocks of the slice (each wave: all)
    static constexpr int NTHR = 2 * NW * 64;               // state waves, then output waves
    static constexpr int EV = 16 / ES;                     // elements per 16 bytes
    // Staged regions.  bf16: unpadded rows with XOR swizzles that make every
    // access of the loop conflict-free on 32 banks -- 16-byte row reads of K and
    // Tb (8 lanes, 8 consecutive rows, one column block) and the transposing
    // reads of K and V (16 lanes, 4 consecutive rows, 2 adjacent blocks);
    // fp32: rows padded by one block (pitch = 4 words mod 32).
    static constexpr int KB = DK / EV, VB = DVT / EV, TB = C / EV;     // data blocks per row
    static constexpr int KP = BF ? KB : KB + 1, VP = BF ? VB : VB + 1, TP = BF ? TB : TB + 1;
    static constexpr int KSW = BF ? 1 : 0, VSW = BF && VB >= 4 ? 2 : 0, TSW = BF ? 3 : 0;
    static constexpr int LDK = KP * EV, LDV = VP * EV, LDC = TP * EV;   // pitches (elements)
    static constexpr int LDS = DK + EV;                    // state copy S[v][d]
    // X^T exchange buffer: DVT rows of C tokens (bf16: the token order within
    // each 32-token group pairs runs 4g.. and 16+4g.., see xcol; rows swizzled
    // like Tb); fp32: plain rows padded by one block
    static constexpr int XP = BF ? TB : TB + 1, XSW = BF ? 3 : 0;
    static constexpr int NDB = DK / 16, NDBW = NDB / NW;   // d-blocks of the state per wave
    static constexpr int NP = (NW + 1) / 2;                // pairs of token blocks
    static constexpr int KS = Step<T>::KS, NQ = DK / KS;   // Q fragments per lane
    // staging buffer: regions K | Tb | V slice | gates, each a whole number of
    // 1 KB blocks; block i is filled by output wave i % NW (64 lanes x 16 bytes)
    static constexpr int blocks(int bytes) { return (bytes + 1023) / 1024; }
    static constexpr int NIK = blocks(C * LDK * ES), NIV = blocks(C * LDV * ES);
    static constexpr int NIT = blocks(C * LDC * ES), NIG = blocks(3 * C * 4);
    static constexpr size_t SZ_SB = ((size_t)DVT * LDS * ES + 15) / 16 * 16;
    static constexpr size_t SZ_X = (size_t)DVT * XP * 16;
    // V' of the chunk in MFMA operand order, handed from the state waves to the
    // output waves: per (pair of token blocks p, column block vb) and lane, the
    // lane's 4 values of token block 2p then those of 2p + 1
    static constexpr size_t SZ_VP = (size_t)NP * NVB * 64 * 8 * ES;
    static constexpr size_t LDS_MAX = 160 * 1024;
    // Batches: batch j holds LDS blocks j*NW .. j*NW + NW - 1, block j*NW + w
    // filled by wave w (one 16-byte load per lane).  Regions start on batch
    // boundaries, so a batch belongs to one region -- K, Tb -- except the last,
    // which holds V then the gates when both fit in one batch.
    static constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }
    static constexpr bool VG1 = NIV + NIG <= NW;
    static constexpr int NBK = cdiv(NIK, NW), NBT = cdiv(NIT, NW);
    static constexpr int NBVG = VG1 ? 1 : cdiv(NIV, NW) + cdiv(NIG, NW);
    static constexpr int NL = NBK + NBT + NBVG;            // batches = staging loads per lane per chunk
    static constexpr int JT = NBK, JV = JT + NBT;          // first batch of each region
    static constexpr int JG = VG1 ? JV : JV + cdiv(NIV, NW);
    static constexpr int BG0 = VG1 ? JV * NW + NIV : JG * NW;   // first block of the gates
    static constexpr size_t SZ_STAGE = (size_t)NL * NW * 1024;
    static constexpr size_t OFF_T = (size_t)JT * NW * 1024;
    static constexpr size_t OFF_V = (size_t)JV * NW * 1024, OFF_G = (size_t)BG0 * 1024;
    static constexpr int NSTAGE = 2;                       // chunk cc in cc % 2; cc + 1 staged meanwhile
    static constexpr size_t OFF_SB = NSTAGE * SZ_STAGE, OFF_X = OFF_SB + SZ_SB, OFF_VP = OFF_X + SZ_X;
    static constexpr size_t SMEM = OFF_VP + SZ_VP;
    static constexpr bool FITS = SMEM <= LDS_MAX;
    static_assert(C % 16 == 0 && NW >= 1 && NW <= 4 && NVB >= 1 && NVB <= 2, "tile counts");
    static_assert(DV % DVT == 0 && DVT % 16 == 0 && NDB % NW == 0, "tile shapes");
    static_assert(DK % KS == 0 && DK % EV == 0 && DVT % EV == 0 && C % EV == 0, "whole 16-byte steps");
    static_assert(!BF || (C % 32 == 0 && KB % 8 == 0 && (VB % 4 == 0 || VB == 2) && TB % 8 == 0),
                  "bf16 swizzles: Tb and X^T in 32-column groups, K / V / Tb rows of 8 / 2 or 4k / 8 blocks");
};

// element (r, c) of a staged region (pitch P blocks, swizzle kind W)
template <typename Cfg, int P, int W>
__device__ __forceinline__ int sidx(int r, int c) {
    return (r * P + ((c / Cfg::EV) ^ swz<W>(r))) * Cfg::EV + (c % Cfg::EV);
}
template <typename Cfg>
__device__ __forceinline__ int kidx(int r, int c) { return sidx<Cfg, Cfg::KP, Cfg::KSW>(r, c); }
template <typename Cfg>
__device__ __forceinline__ int vidx(int r, int c) { return sidx<Cfg, Cfg::VP, Cfg::VSW>(r, c); }
template <typename Cfg>
__device__ __forceinline__ int tidx(int r, int c) { return sidx<Cfg, Cfg::TP, Cfg::TSW>(r, c); }
// X^T: row v, physical column c
template <typename Cfg>
__device__ __forceinline__ int xidx(int v, int c) { return sidx<Cfg, Cfg::XP, Cfg::XSW>(v, c); }
// physical column of token t in a bf16 row of Tb or X^T: within each 32-token
// group, the 4-token runs are stored in the order 0, 16, 4, 20, 8, 24, 12, 28
template <typename Cfg>
__device__ __forceinline__ int xcol(int t) {
    if constexpr (Cfg::BF) return (t & ~31) + (((t >> 2) & 3) << 3) + (((t >> 4) & 1) << 2) + (t & 3);
    else return t;
}

// Byte offset, relative to the chunk's first row, of the 16 bytes that lane l
// brings in for LDS block i (slot l of it), or kOutOfRange for padding.
// rs_k / rs_v: bytes between consecutive tokens of K / V.
template <typename Cfg, int P, int B, int W>
__device__ __forceinline__ int64_t region_offset(int s, int64_t row_bytes) {
    const int r = s / P, p = s - r * P;
    if (r >= Cfg::NW * 16 || p >= B) return -1;
    return r * row_bytes + (int64_t)((p ^ swz<W>(r)) * 16);
}
// region of staging batch j for wave w: 0 K, 2 Tb, 3 V, 4 gates, 5 padding
template <typename Cfg>
__device__ __forceinline__ int stage_region(int j, int w) {
    if (j < Cfg::JT) return 0;
    if (j < Cfg::JV) return 2;
    const int i = j * Cfg::NW + w;                       // LDS block
    if (i < Cfg::JV * Cfg::NW + Cfg::NIV) return 3;
    if (i >= Cfg::BG0 && i < Cfg::BG0 + Cfg::NIG) return 4;
    return 5;
}
template <typename Cfg>
__device__ __forceinline__ uint32_t stage_offset(int j, int w, int l, int64_t rs_k, int64_t rs_v) {
    constexpr int C = Cfg::NW * 16;
    const int i = j * Cfg::NW + w;
    int64_t off = -1;
    switch (stage_region<Cfg>(j, w)) {
        case 0: off = region_offset<Cfg, Cfg::KP, Cfg::KB, Cfg::KSW>(i * 64 + l, rs_k); break;
        case 2: off = region_offset<Cfg, Cfg::TP, Cfg::TB, Cfg::TSW>((i - Cfg::JT * Cfg::NW) * 64 + l,
                                                                  (int64_t)C * Cfg::ES); break;
        case 3: off = region_offset<Cfg, Cfg::VP, Cfg::VB, Cfg::VSW>((i - Cfg::JV * Cfg::NW) * 64 + l, rs_v); break;
        case 4: {
            const int s = (i - Cfg::BG0) * 64 + l;
            off = s < 3 * C / 4 ? (int64_t)s * 16 : -1;
            break;
        }
        default: break;
    }
    return (off < 0 || off >= (int64_t)kOutOfRange) ? kOutOfRange : (uint32_t)off;
}

// Step fragment (16 bytes) of the swizzled K chunk: K[row0 + n][k0 + g*EV ...]
template <typename Cfg, typename T>
__device__ __forceinline__ typename Step<T>::frag kfrag_rows(const T* sK, int row0, int k0) {
    const int l = lane_id();
    return *reinterpret_cast<const typename Step<T>::frag*>(
        sK + kidx<Cfg>(row0 + (l & 15), k0 + (l >> 4) * Cfg::EV));
}
// Step fragment of a plain row-major LDS tile
template <typename T>
__device__ __forceinline__ typename Step<T>::frag frag16(const T* p, int ld, int row0, int k0) {
    const int l = lane_id();
    return *reinterpret_cast<const typename Step<T>::frag*>(p + (row0 + (l & 15)) * ld + k0 +
                                                             (l >> 4) * (16 / sizeof(T)));
}

// K^T as the A operand of token block kb: lane (g, n) gets K[kb*16 + 4g + e][d0 + n]
// (bf16: one transposing read -- lane s of group g supplies row kb*16 + 4g + s/4,
// columns d0 + 4 (s%4) .. +3; fp32: a gather)
template <typename Cfg, typename T>
__device__ __forceinline__ typename K16<T>::op kT16(const T* sK, int kb, int d0) {
    const int l = lane_id(), g = l >> 4, n = l & 15;
    if constexpr (Cfg::BF) {
        return tr_read(sK + kidx<Cfg>(kb * 16 + 4 * g + (n >> 2), d0 + 4 * (n & 3)));
    } else {
        const T* p = sK + kidx<Cfg>(kb * 16 + 4 * g, d0 + n);        // fp32 rows are not swizzled
        return f32x4{p[0], p[Cfg::LDK], p[2 * Cfg::LDK], p[3 * Cfg::LDK]};
    }
}
// V rows jb*16 + 4g + e, column vb*16 + n, as fp32
template <typename Cfg, typename T>
__device__ __forceinline__ f32x4 vcol4(const T* sV, int jb, int vb) {
    const int l = lane_id(), g = l >> 4, n = l & 15;
    if constexpr (Cfg::BF) {
        const s16x4 x = tr_read(sV + vidx<Cfg>(jb * 16 + 4 * g + (n >> 2), vb * 16 + 4 * (n & 3)));
        return f32x4{bf16_bits_to_f32(x[0]), bf16_bits_to_f32(x[1]), bf16_bits_to_f32(x[2]),
                     bf16_bits_to_f32(x[3])};
    } else {
        const T* p = sV + vidx<Cfg>(jb * 16 + 4 * g, vb * 16 + n);   // fp32 rows are not swizzled
        return f32x4{p[0], p[Cfg::LDV], p[2 * Cfg::LDV], p[3 * Cfg::LDV]};
    }
}

template <typename T, int DK, int DV, int C, int DVT>
__global__ __launch_bounds__(512) void gdn_scan_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* S0, SeqGeom geom, int H,
    const float* __restrict__ g_ws, const T* __restrict__ Tb_ws,
    T* __restrict__ O, float* S_T) {   // S_T may alias S0
    using Cfg = ScanCfg<T, DK, DV, C, DVT>;
    static_assert(Cfg::FITS, "scan workgroup exceeds the LDS of one CU");
    using St16 = Step<T>;
    using Frag = typename St16::frag;
    using KO = K16<T>;
    using Op = typename KO::op;
    constexpr int NW = Cfg::NW, NVB = Cfg::NVB, NDBW = Cfg::NDBW, KS = Cfg::KS, NP = Cfg::NP;
    constexpr int ES = Cfg::ES;
    extern __shared__ __align__(16) unsigned char smem[];

    // Workgroups are dealt to the 8 XCDs round-robin by linear id; renumber them
    // so that the DV / DVT column slices of one (sequence, head) share an XCD and
    // its L2 serves their common K, Q, Tb and gate reads.
    int v0, h, seq;
    {
        constexpr int NS = DV / DVT;
        const int U = H * (int)gridDim.z;                       // (sequence, head) units
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
        seq = u / H;
    }
    const int l = lane_id(), w = wave_id();
    const int n = l & 15, g4 = 4 * (l >> 4);

    // this sequence's tokens [ts, te) and first chunk slot, read once; chunk cc
    // covers tokens ts + cc C .. min(ts + (cc + 1) C, te) - 1 in slot first + cc
    int ts, te, first;
    if (geom.table) {
        ts = geom.bounds[seq];
        te = geom.bounds[seq + 1];
        first = geom.seq_slot[seq];
    } else {
        ts = seq * geom.T;
        te = ts + geom.T;
        first = seq * geom.chunks_per_seq;
    }
    const int count = (te - ts + C - 1) / C;
    const int64_t sbase = ((int64_t)seq * H + h) * DV * DK;
    const int64_t rs_k = (int64_t)H * DK * ES, rs_v = (int64_t)H * DV * ES;   // token strides (bytes)
    T* sS = reinterpret_cast<T*>(smem + Cfg::OFF_SB);     // state copy S[v][d] (input dtype)
    T* sX = reinterpret_cast<T*>(smem + Cfg::OFF_X);      // X^T of the current chunk
    T* sVp = reinterpret_cast<T*>(smem + Cfg::OFF_VP);    // V' of the current chunk

    auto barrier = [&]() __attribute__((always_inline)) {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    // staged chunk cc: K, Tb, V slice, gates (g, gamma = e^g, gamma_n / gamma)
    struct Staged {
        const T *K, *V, *Tb;
        const float *g, *gam, *dec;
    };
    auto staged = [&](int cc) __attribute__((always_inline)) {
        const unsigned char* sb = smem + (cc & 1) * Cfg::SZ_STAGE;
        Staged st;
        st.K = reinterpret_cast<const T*>(sb);
        st.V = reinterpret_cast<const T*>(sb + Cfg::OFF_V);
        st.Tb = reinterpret_cast<const T*>(sb + Cfg::OFF_T);
        st.g = reinterpret_cast<const float*>(sb + Cfg::OFF_G);
        st.gam = st.g + C;
        st.dec = st.g + 2 * C;
        return st;
    };

    // ---- state waves: the recurrence.  Wave cb owns the tiles (d-block
    // db = cb + NW i, column block vb) of S^T; lane (g, n) of tile (i, vb) holds
    // S^T[db*16 + 4g + r][vb*16 + n].  Per chunk: Y = K S^T and X = V - diag(gamma) Y
    // for token block cb (X^T to LDS); barrier; V' = Tb X for every token block,
    // V' of block cb to LDS for the output waves, and the state update with the
    // new state's copy S[v][d] (input dtype) to LDS; barrier.
    auto run_state = [&](auto cb_const) __attribute__((always_inline)) {
        constexpr int cb = decltype(cb_const)::value;
        f32x4 St[NDBW][NVB];
#pragma unroll
        for (int i = 0; i < NDBW; ++i)
#pragma unroll
            for (int vb = 0; vb < NVB; ++vb) {
                const int db = cb + NW * i, vv = vb * 16 + n, d = db * 16 + g4;
                St[i][vb] = S0 ? *reinterpret_cast<const f32x4*>(S0 + sbase + (int64_t)(v0 + vv) * DK + d) : zero4();
                store4(sS + vv * Cfg::LDS + d, St[i][vb][0], St[i][vb][1], St[i][vb][2], St[i][vb][3]);
            }
        __syncthreads();

        auto step = [&](const int cc) __attribute__((always_inline)) {
            const Staged st = staged(cc);
            // phase A: Y and X for token block cb
            f32x4 Y[NVB];
#pragma unroll
            for (int vb = 0; vb < NVB; ++vb) Y[vb] = zero4();
#pragma unroll
            for (int kk = 0; kk < DK; kk += KS) {
                const Frag ak = kfrag_rows<Cfg>(st.K, cb * 16, kk);
#pragma unroll
                for (int vb = 0; vb < NVB; ++vb) Y[vb] = St16::mma(ak, frag16(sS, Cfg::LDS, vb * 16, kk), Y[vb]);
            }
            {
                const float4 gam4 = *reinterpret_cast<const float4*>(st.gam + cb * 16 + g4);
#pragma unroll
                for (int vb = 0; vb < NVB; ++vb) {
                    const f32x4 vv = vcol4<Cfg>(st.V, cb, vb);
                    // lane (g, n): X[cb*16 + 4g + r][vb*16 + n], 4 consecutive tokens of X^T row vb*16 + n
                    store4(sX + xidx<Cfg>(vb * 16 + n, xcol<Cfg>(cb * 16 + g4)), vv[0] - gam4.x * Y[vb][0],
                           vv[1] - gam4.y * Y[vb][1], vv[2] - gam4.z * Y[vb][2], vv[3] - gam4.w * Y[vb][3]);
                }
            }
            wait_vm_lgkm0<63>();   // the X^T stores are visible after the barrier
            barrier();

            // phase B: V' = Tb X for every token block (A: Tb rows, shared by the
            // column blocks; B: X^T rows; bf16 keeps both as 16-byte block pairs)
            f32x4 Vp[NVB][NW];
            {
                typename St16::frag xb[NVB][NP];
                Op x0[NVB][NP], x1[NVB][NP];
#pragma unroll
                for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
                    for (int p = 0; p < NP; ++p) {
                        if constexpr (Cfg::BF) {
                            xb[vb][p] = *reinterpret_cast<const bf16x8*>(sX + xidx<Cfg>(vb * 16 + n, 32 * p + 2 * g4));
                        } else {
                            x0[vb][p] = *reinterpret_cast<const f32x4*>(sX + xidx<Cfg>(vb * 16 + n, 32 * p + g4));
                            if (2 * p + 1 < NW)
                                x1[vb][p] = *reinterpret_cast<const f32x4*>(sX + xidx<Cfg>(vb * 16 + n, 32 * p + 16 + g4));
                        }
                    }
#pragma unroll
                for (int ib = 0; ib < NW; ++ib) {
                    const int ar = ib * 16 + n;
                    f32x4 acc[NVB];
#pragma unroll
                    for (int vb = 0; vb < NVB; ++vb) acc[vb] = zero4();
#pragma unroll
                    for (int p = 0; p < NP; ++p) {
                        if (2 * p > ib) continue;
                        if constexpr (Cfg::BF) {
                            const bf16x8 ta = *reinterpret_cast<const bf16x8*>(st.Tb + tidx<Cfg>(ar, 32 * p + 2 * g4));
#pragma unroll
                            for (int vb = 0; vb < NVB; ++vb) acc[vb] = St16::mma(ta, xb[vb][p], acc[vb]);
                        } else {
                            const f32x4 a0 = *reinterpret_cast<const f32x4*>(st.Tb + tidx<Cfg>(ar, 32 * p + g4));
                            if (2 * p + 1 < NW) {
                                const f32x4 a1 = *reinterpret_cast<const f32x4*>(st.Tb + tidx<Cfg>(ar, 32 * p + 16 + g4));
#pragma unroll
                                for (int vb = 0; vb < NVB; ++vb) acc[vb] = KO::mma2(a0, a1, x0[vb][p], x1[vb][p], acc[vb]);
                            } else {
#pragma unroll
                                for (int vb = 0; vb < NVB; ++vb) acc[vb] = KO::mma1(a0, x0[vb][p], acc[vb]);
                            }
                        }
                    }
#pragma unroll
                    for (int vb = 0; vb < NVB; ++vb) Vp[vb][ib] = acc[vb];
                }
            }
            // V' of token block cb, in the operand order of the output waves
#pragma unroll
            for (int vb = 0; vb < NVB; ++vb)
                store4(sVp + (((cb / 2) * NVB + vb) * 64 + l) * 8 + (cb & 1) * 4, Vp[vb][cb][0], Vp[vb][cb][1],
                       Vp[vb][cb][2], Vp[vb][cb][3]);

            // S^T <- gamma_n S^T + K^T diag(gamma_n / gamma) V' for the own tiles;
            // the new state's copy replaces the old one (its readers are past the
            // barrier above)
            const float gamma_n = st.gam[C - 1];
#pragma unroll
            for (int jb = 0; jb < NW; ++jb) {
                const float4 dec4 = *reinterpret_cast<const float4*>(st.dec + jb * 16 + g4);
#pragma unroll
                for (int vb = 0; vb < NVB; ++vb) {
                    Vp[vb][jb][0] *= dec4.x;
                    Vp[vb][jb][1] *= dec4.y;
                    Vp[vb][jb][2] *= dec4.z;
                    Vp[vb][jb][3] *= dec4.w;
                }
            }
#pragma unroll
            for (int i = 0; i < NDBW; ++i) {
                const int db = cb + NW * i;
                Op kt[NW];
#pragma unroll
                for (int kb = 0; kb < NW; ++kb) kt[kb] = kT16<Cfg>(st.K, kb, db * 16);
#pragma unroll
                for (int vb = 0; vb < NVB; ++vb) {
                    f32x4 s = St[i][vb] * gamma_n;
#pragma unroll
                    for (int p = 0; p < NP; ++p) {
                        if (2 * p + 1 < NW)
                            s = KO::mma2(kt[2 * p], kt[2 * p + 1], KO::tile(Vp[vb][2 * p]), KO::tile(Vp[vb][2 * p + 1]), s);
                        else
                            s = KO::mma1(kt[2 * p], KO::tile(Vp[vb][2 * p]), s);
                    }
                    St[i][vb] = s;
                    store4(sS + (vb * 16 + n) * Cfg::LDS + db * 16 + g4, s[0], s[1], s[2], s[3]);
                }
            }
            wait_vm_lgkm0<63>();   // the state copy and V' are visible after the barrier
            barrier();
        };
        int cc = 0;
        for (; cc + 2 <= count; cc += 2) {
            step(cc);
            step(cc + 1);
        }
        if (cc < count) step(cc);

        if (S_T) {
#pragma unroll
            for (int i = 0; i < NDBW; ++i)
#pragma unroll
                for (int vb = 0; vb < NVB; ++vb) {
                    const int db = cb + NW * i;
                    *reinterpret_cast<f32x4*>(S_T + sbase + (int64_t)(v0 + vb * 16 + n) * DK + db * 16 + g4) = St[i][vb];
                }
        }
    };

    // ---- output waves: staging and the outputs, one chunk behind the state
    // waves.  Wave cb stages its share of each chunk, computes Z^T = S Q^T
    // (scaled by gamma) and P^T = ((Q K^T) o Gamma o M)^T for query block cb of
    // chunk cc, and, in the next step, O^T = Z^T + V'^T P^T from the V' the
    // state waves left in LDS.
    auto run_out = [&](auto cb_const) __attribute__((always_inline)) {
        constexpr int cb = decltype(cb_const)::value;
        const int wf = cb;   // filler index of this wave
        // this lane's staging loads: LDS block i = wf + NW j, slot l
        uint32_t soff[Cfg::NL];
#pragma unroll
        for (int j = 0; j < Cfg::NL; ++j) soff[j] = stage_offset<Cfg>(j, wf, l, rs_k, rs_v);
        const uint32_t ooff = (uint32_t)((cb * 16 + n) * rs_v) + g4 * ES;
        const uint32_t qoff = (uint32_t)((cb * 16 + n) * rs_k) + (l >> 4) * 16;

        // chunk cd's K, Tb, V slice and gates into registers (rows past the
        // chunk end fall outside the buffer ranges and read as zeros) ...
        auto stage_load = [&](u32x4* R, int cd) __attribute__((always_inline)) {
            const int t0 = ts + cd * C, len = min(C, te - t0);
            const int64_t unit = (int64_t)(first + cd) * H + h;
            const T* kb = k + ((int64_t)t0 * H + h) * DK;
            const T* vb_ = v + ((int64_t)t0 * H + h) * DV + v0;
            const T* tb = Tb_ws + unit * C * C;
            const float* gb = g_ws + unit * 3 * C;
            const int nk = (int)((len - 1) * rs_k + DK * ES), nv = (int)((len - 1) * rs_v + DVT * ES);
#pragma unroll
            for (int j = 0; j < Cfg::NL; ++j) {
                // the region of batch j is fixed except in the shared V / gates batch
                const void* base;
                int nrec;
                if (j < Cfg::JT) { base = kb; nrec = nk; }
                else if (j < Cfg::JV) { base = tb; nrec = C * C * ES; }
                else {
                    const int r = stage_region<Cfg>(j, wf);
                    base = r == 3 ? (const void*)vb_ : (const void*)gb;
                    nrec = r == 3 ? nv : r == 4 ? 3 * C * 4 : 0;
                }
                R[j] = __builtin_amdgcn_raw_buffer_load_b128(make_rsrc(base, nrec), soff[j], 0, 0);
            }
        };
        // ... and from there into the staging buffer of chunk cd
        auto stage_store = [&](const u32x4* R, int cd) __attribute__((always_inline)) {
            unsigned char* base = smem + (cd & 1) * Cfg::SZ_STAGE + (wf * 64 + l) * 16;
#pragma unroll
            for (int j = 0; j < Cfg::NL; ++j) *reinterpret_cast<u32x4*>(base + j * Cfg::NW * 1024) = R[j];
        };
        // this wave's Q fragments of chunk cd (token block cb)
        auto q_in = [&](Frag* dst, int cd) __attribute__((always_inline)) {
            const int t0 = ts + cd * C, len = min(C, te - t0);
            const __amdgpu_buffer_rsrc_t rq =
                make_rsrc(q + ((int64_t)t0 * H + h) * DK, (len - 1) * rs_k + DK * ES);
#pragma unroll
            for (int j = 0; j < Cfg::NQ; ++j)
                dst[j] = __builtin_bit_cast(Frag, __builtin_amdgcn_raw_buffer_load_b128(rq, qoff + j * 64, 0, 0));
        };

        // two register sets take turns: step cc writes the one holding chunk
        // cc + 1 to LDS as it starts and refills it with chunk cc + 3; Q is read
        // straight into registers, two chunks ahead
        u32x4 ra[Cfg::NL], rb[Cfg::NL];
        Frag qa[Cfg::NQ], qb[Cfg::NQ];
        if (count > 0) {
            stage_load(ra, 0);
            stage_load(rb, min(1, count - 1));
            q_in(qa, 0);
            q_in(qb, min(1, count - 1));
            stage_store(ra, 0);
            stage_load(ra, min(2, count - 1));
        }
        __syncthreads();

        // Z^T (scaled) and P^T of the previous chunk, consumed by its output
        f32x4 Zt[NVB], Pt[NW];
        // O^T = Z^T + V'^T P^T for tiles (cb, vb) of chunk cd (A: the V' tiles as
        // V'^T, from LDS; B: the P^T tiles); lane (g, n) stores
        // O[token cb*16 + n][v0 + vb*16 + 4g .. + 3].  bf16 pairs a last odd block
        // with the (zero) P^T tile of the next one: every bf16 accumulation chain
        // then stays on one MFMA shape, since a 16x16x16 MFMA that accumulates
        // onto a 16x16x32 result has been seen to read a stale accumulator when
        // the compiler keeps it in VGPRs.
        auto output = [&](int cd) __attribute__((always_inline)) {
            const int t0 = ts + cd * C, len = min(C, te - t0);
            const __amdgpu_buffer_rsrc_t ro =
                make_rsrc(O + ((int64_t)t0 * H + h) * DV + v0, (len - 1) * rs_v + DVT * ES);
#pragma unroll
            for (int vb = 0; vb < NVB; ++vb) {
                f32x4 acc = Zt[vb];
#pragma unroll
                for (int p = 0; p < NP; ++p) {
                    if (2 * p > cb) continue;
                    const T* src = sVp + ((p * NVB + vb) * 64 + l) * 8;
                    if constexpr (Cfg::BF) {
                        const bf16x8 a = *reinterpret_cast<const bf16x8*>(src);
                        acc = KO::mma2p(a, KO::tile(Pt[2 * p]), KO::tile(Pt[2 * p + 1]), acc);
                    } else {
                        const f32x4 a0 = *reinterpret_cast<const f32x4*>(src);
                        if (2 * p + 1 <= cb)
                            acc = KO::mma2(a0, *reinterpret_cast<const f32x4*>(src + 4), Pt[2 * p], Pt[2 * p + 1], acc);
                        else
                            acc = KO::mma1(a0, Pt[2 * p], acc);
                    }
                }
                if constexpr (Cfg::BF) {
                    const bf16x4 o4 = {(bf16)acc[0], (bf16)acc[1], (bf16)acc[2], (bf16)acc[3]};
                    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, o4), ro, ooff + vb * 16 * ES, 0, 0);
                } else {
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc), ro, ooff + vb * 16 * ES, 0, 0);
                }
            }
        };

        auto step = [&](const int cc, u32x4* rnext, Frag* qcur) __attribute__((always_inline)) {
            // chunk cc + 1 into the other staging buffer (its last readers are
            // past the previous barrier); the next barrier publishes it
            stage_store(rnext, cc + 1);
            stage_load(rnext, min(cc + 3, count - 1));   // past the end: re-read, unused
            const Staged st = staged(cc);

            // phase A: the previous chunk's output (its V' was published by the
            // last barrier), then Z^T = S Q^T of this chunk while S is in LDS
            if (cc > 0) output(cc - 1);
#pragma unroll
            for (int vb = 0; vb < NVB; ++vb) Zt[vb] = zero4();
#pragma unroll
            for (int kk = 0; kk < DK; kk += KS)
#pragma unroll
                for (int vb = 0; vb < NVB; ++vb)
                    Zt[vb] = St16::mma(frag16(sS, Cfg::LDS, vb * 16, kk), qcur[kk / KS], Zt[vb]);
            wait_vm_lgkm0<63>();   // the staged chunk is visible after the barrier
            barrier();

            // phase B: P^T tiles of query block cb (rows: key tokens), decayed
            // and masked; Z^T columns scaled by gamma
#pragma unroll
            for (int jb = 0; jb < NW; ++jb) Pt[jb] = zero4();
#pragma unroll
            for (int kk = 0; kk < DK; kk += KS)
#pragma unroll
                for (int jb = 0; jb <= cb; ++jb)
                    Pt[jb] = St16::mma(kfrag_rows<Cfg>(st.K, jb * 16, kk), qcur[kk / KS], Pt[jb]);
            q_in(qcur, min(cc + 2, count - 1));   // this chunk's Q is consumed
            const int cq = cb * 16 + n;
            const float gq = st.g[cq], gamq = st.gam[cq];
#pragma unroll
            for (int vb = 0; vb < NVB; ++vb) Zt[vb] *= gamq;
#pragma unroll
            for (int jb = 0; jb <= cb; ++jb) {
                const float4 gj = *reinterpret_cast<const float4*>(st.g + jb * 16 + g4);
                const int j0 = jb * 16 + g4;
                Pt[jb][0] = j0 + 0 <= cq ? Pt[jb][0] * __expf(gq - gj.x) : 0.f;
                Pt[jb][1] = j0 + 1 <= cq ? Pt[jb][1] * __expf(gq - gj.y) : 0.f;
                Pt[jb][2] = j0 + 2 <= cq ? Pt[jb][2] * __expf(gq - gj.z) : 0.f;
                Pt[jb][3] = j0 + 3 <= cq ? Pt[jb][3] * __expf(gq - gj.w) : 0.f;
            }
            wait_vm_lgkm0<63>();   // all reads of this chunk's staging buffer are done
            barrier();
        };
        int cc = 0;
        for (; cc + 2 <= count; cc += 2) {
            step(cc, rb, qa);
            step(cc + 1, ra, qb);
        }
        if (cc < count) step(cc, rb, qa);
        if (count > 0) output(count - 1);   // its V' was published by the last barrier
    };

    switch (w) {
        case 0: run_state(std::integral_constant<int, 0>{}); break;
        case 1: if constexpr (NW > 1) run_state(std::integral_constant<int, (NW > 1 ? 1 : 0)>{}); break;
        case 2: if constexpr (NW > 2) run_state(std::integral_constant<int, (NW > 2 ? 2 : 0)>{}); break;
        case 3: if constexpr (NW > 3) run_state(std::integral_constant<int, (NW > 3 ? 3 : 0)>{}); break;
        default: break;
    }
    switch (w - NW) {
        case 0: run_out(std::integral_constant<int, 0>{}); break;
        case 1: if constexpr (NW > 1) run_out(std::integral_constant<int, (NW > 1 ? 1 : 0)>{}); break;
        case 2: if constexpr (NW > 2) run_out(std::integral_constant<int, (NW > 2 ? 2 : 0)>{}); break;
        case 3: if constexpr (NW > 3) run_out(std::integral_constant<int, (NW > 3 ? 3 : 0)>{}); break;
        default: break;
    }
}

}  // namespace gdn
