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
//   phase A   Y = K S^T,  Z^T = S Q^T,  P^T = K Q^T      (all read only S)
//             X = V - diag(gamma) Y                       prediction errors vs. the gated start state
//   phase B   V' = Tb X   (= U - W S^T)                   corrected for the chunk's earlier writes
//   phase C   O^T = Z^T diag(gamma) + V'^T P^T            P = (Q K^T) o Gamma o M
//             S^T <- gamma_n S^T + K^T diag(gamma_n / gamma) V'
// Sources: the same Qiita section (product form of S_i with I - sum w k^T =
// A_1..A_i and the G_i identity; parallel form H = S0 (Q - W (M^T o K^T Q)) D_gamma
// + U (Gamma o K^T Q) restricted to one chunk) and its section "Chunk
// Computation" (chunk j starts from chunk j-1's last state);
// LinearAttention系列解读(六)：DeltaNet的Chunkwise Form推导, section 4.4 (U - W S^T is
// each token's prediction error against the chunk-start state, corrected by the
// triangular solve) and section 4.5 (T, W, U do not depend on S).
//
// Work split: wave w owns token block w (16 tokens) for Y, Z, P, V' and O, and
// d-blocks w, w + NW, ... of the state.  Operands are reused from registers
// where the MFMA layouts allow it:
//  - the Q fragments of a wave come straight from global memory (no LDS);
//  - P^T and Z^T stay in the registers of the wave that computes them and feed
//    the output product directly (a 16x16 accumulator tile has the lane layout
//    of a 16-deep B operand);
//  - S^T, X, V' go through LDS once per chunk, with 8-byte stores.
// K is staged in LDS with 16-byte blocks XOR-swizzled by row group, which keeps
// both its row reads and its column gathers free of bank conflicts (32 banks).
// The chunks' state-independent inputs are fetched into a ring of register
// sets NPF chunks ahead, with unconditional loads so that the compiler waits
// only for the oldest set.
#pragma once

#include <type_traits>

#include "gdn_device.h"

namespace gdn {

typedef short s16x4 __attribute__((ext_vector_type(4)));

// acc += A[m0 + m][k0 + k] * B[k][n] over one 16-deep k block, where B is a 16x16
// accumulator tile held in the MFMA D layout (lane (g, n): rows 4g..4g+3 of column n)
// and A is read from LDS (row-major, leading dimension lda).
template <typename T> struct RegB;
template <> struct RegB<bf16> {
    __device__ __forceinline__ static f32x4 mma(const bf16* A, int lda, int m0, int k0, f32x4 b,
                                                f32x4 acc) {
        const int l = lane_id();
        const s16x4 a = *reinterpret_cast<const s16x4*>(A + (m0 + (l & 15)) * lda + k0 + 4 * (l >> 4));
        const bf16x4 bb = {(bf16)b[0], (bf16)b[1], (bf16)b[2], (bf16)b[3]};
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, __builtin_bit_cast(s16x4, bb), acc, 0, 0, 0);
    }
};
template <> struct RegB<float> {
    __device__ __forceinline__ static f32x4 mma(const float* A, int lda, int m0, int k0, f32x4 b,
                                                f32x4 acc) {
        const int l = lane_id();
        const float* a = A + (m0 + (l & 15)) * lda + k0 + 4 * (l >> 4);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[r], b[r], acc, 0, 0, 0);
        return acc;
    }
};

// 4 consecutive values of one lane, rounded to T, as one 8- or 16-byte store
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
    static constexpr int NW = C / 16, NTHR = NW * 64;      // one wave per 16-token block (<= 256 threads)
    static constexpr int EV = 16 / sizeof(T);              // elements per 16 bytes
    static constexpr int LDK = DK + EV, LDC = C + EV, LDV = DVT + EV;
    static constexpr int NVB = DVT / 16, NDB = DK / 16, NDBW = NDB / NW;
    static constexpr int KS = Mfma<T>::KS, NQ = DK / KS;   // Q fragments per lane
    static constexpr int VK = C * DK / EV, PK = (VK + NTHR - 1) / NTHR;
    static constexpr int VV = C * DVT / EV, PV = (VV + NTHR - 1) / NTHR;
    static constexpr int VT = C * C / EV, PT = (VT + NTHR - 1) / NTHR;
    static constexpr int VG = 3 * C / 4;                   // g, exp(g), exp(g_n - g)
    static constexpr int PG = (VG + NTHR - 1) / NTHR;
    static constexpr int NPF = 2;                          // chunks fetched ahead
    static constexpr size_t SZ_K = sizeof(T) * C * LDK;
    static constexpr size_t SZ_REST = sizeof(T) * C * LDV + sizeof(T) * C * LDC +
                                      sizeof(T) * DVT * LDK + 3 * sizeof(T) * DVT * LDC +
                                      sizeof(float) * 3 * C;
    static constexpr size_t LDS_MAX = 160 * 1024;
    static constexpr int KBUF = (2 * SZ_K + SZ_REST <= LDS_MAX) ? 2 : 1;
    static constexpr size_t OFF_K = 0;
    static constexpr size_t OFF_V = OFF_K + KBUF * SZ_K;
    static constexpr size_t OFF_TB = OFF_V + sizeof(T) * C * LDV;
    static constexpr size_t OFF_SB = OFF_TB + sizeof(T) * C * LDC;
    static constexpr size_t OFF_XT = OFF_SB + sizeof(T) * DVT * LDK;
    static constexpr size_t OFF_VPT = OFF_XT + sizeof(T) * DVT * LDC;
    static constexpr size_t OFF_VDT = OFF_VPT + sizeof(T) * DVT * LDC;
    static constexpr size_t OFF_G = OFF_VDT + sizeof(T) * DVT * LDC;
    static constexpr size_t SMEM = OFF_G + sizeof(float) * 3 * C;
    static_assert(SMEM <= LDS_MAX, "scan workgroup exceeds the LDS of one CU");
    static_assert(C % 16 == 0 && NW >= 1 && NW <= 4, "one to four 16-token blocks");
    static_assert(DV % DVT == 0 && DVT % 16 == 0 && NDB % NW == 0, "tile shapes");
    static_assert(C % KS == 0 && DK % KS == 0, "whole MFMA steps");
};

// Element (r, c) of the staged K chunk: 16-byte block c / EV of row r is stored
// at block (c / EV) ^ swz(r); swz(r) only flips block-index bits that stay below
// DK / EV, so every row keeps its own blocks.
template <typename Cfg>
__device__ __forceinline__ int kswz(int r) {
    constexpr int NBLK = Cfg::LDK / Cfg::EV - 1;      // blocks per row (DK / EV)
    return NBLK >= 8 ? (((r >> 3) & 3) << 1) : 0;
}
template <typename Cfg>
__device__ __forceinline__ int kidx(int r, int c) {
    return r * Cfg::LDK + (((c / Cfg::EV) ^ kswz<Cfg>(r)) * Cfg::EV) + (c % Cfg::EV);
}

// x32 (bf16) / x4 (fp32) fragment of swizzled K with the contraction along d
// (rows = tokens): element (row0 + n, k0 + g*KPL + e)
template <typename Cfg, typename T>
__device__ __forceinline__ typename Mfma<T>::frag kfrag_rows(const T* sK, int row0, int k0) {
    const int l = lane_id();
    const int r = row0 + (l & 15);
    const T* p = sK + kidx<Cfg>(r, k0 + (l >> 4) * Mfma<T>::KPL);
    if constexpr (Mfma<T>::KPL == 8) return *reinterpret_cast<const bf16x8*>(p);
    else return *p;
}
// fragment of swizzled K with the contraction along tokens: element
// (d = d0 + n, token k0 + g*KPL + e), i.e. K^T, gathered
template <typename Cfg, typename T>
__device__ __forceinline__ typename Mfma<T>::frag kfrag_cols(const T* sK, int k0, int d0) {
    const int l = lane_id();
    const int d = d0 + (l & 15), r0 = k0 + (l >> 4) * Mfma<T>::KPL;
    if constexpr (Mfma<T>::KPL == 8) {
        bf16x8 f;
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = sK[kidx<Cfg>(r0 + e, d)];
        return f;
    } else {
        return sK[kidx<Cfg>(r0, d)];
    }
}

// Register-staged copy of one chunk's state-independent inputs: K, the V slice,
// Tb and the gate rows for LDS, and this wave's Q fragments (token block w).
template <typename Cfg, typename T, int DK, int DV, int C, int DVT>
struct ChunkFetch {
    u32x4 k[Cfg::PK], v[Cfg::PV], tb[Cfg::PT], g[Cfg::PG];
    typename Mfma<T>::frag q[Cfg::NQ];

    // Every lane issues every load, unmasked (rows past the chunk end read row 0
    // of the chunk); store() and the Q consumer zero those rows.
    __device__ __forceinline__ void load(const T* __restrict__ kg, const T* __restrict__ qg,
                                         const T* __restrict__ vg, const float* __restrict__ g_ws,
                                         const T* __restrict__ Tb_ws, int t0, int len,
                                         int64_t unit, int H, int h, int v0) {
        const int tid = threadIdx.x, l = lane_id(), w = wave_id();
        constexpr int RK = DK / Cfg::EV, RV = DVT / Cfg::EV;
#pragma unroll
        for (int m = 0; m < Cfg::PK; ++m) {
            const int i = (tid + Cfg::NTHR * m) % Cfg::VK;
            const int r = i / RK, c = (i - r * RK) * Cfg::EV;
            k[m] = *reinterpret_cast<const u32x4*>(kg + ((int64_t)(t0 + (r < len ? r : 0)) * H + h) * DK + c);
        }
#pragma unroll
        for (int m = 0; m < Cfg::PV; ++m) {
            const int i = (tid + Cfg::NTHR * m) % Cfg::VV;
            const int r = i / RV, c = (i - r * RV) * Cfg::EV;
            v[m] = *reinterpret_cast<const u32x4*>(
                vg + ((int64_t)(t0 + (r < len ? r : 0)) * H + h) * DV + v0 + c);
        }
#pragma unroll
        for (int m = 0; m < Cfg::PT; ++m) {
            const int i = (tid + Cfg::NTHR * m) % Cfg::VT;
            tb[m] = *reinterpret_cast<const u32x4*>(Tb_ws + unit * C * C + (int64_t)i * Cfg::EV);
        }
#pragma unroll
        for (int m = 0; m < Cfg::PG; ++m) {
            const int i = (tid + Cfg::NTHR * m) % Cfg::VG;
            g[m] = *reinterpret_cast<const u32x4*>(g_ws + unit * 3 * C + 4 * i);
        }
        const int qr = w * 16 + (l & 15);
        const T* qrow = qg + ((int64_t)(t0 + (qr < len ? qr : 0)) * H + h) * DK + (l >> 4) * Mfma<T>::KPL;
#pragma unroll
        for (int j = 0; j < Cfg::NQ; ++j) {
            if constexpr (Mfma<T>::KPL == 8) q[j] = *reinterpret_cast<const bf16x8*>(qrow + j * Cfg::KS);
            else q[j] = qrow[j * Cfg::KS];
        }
    }

    __device__ __forceinline__ void store(T* sK, T* sV, T* sTb, float* sg, int len) const {
        const int tid = threadIdx.x;
        const u32x4 z = {0u, 0u, 0u, 0u};
        constexpr int RK = DK / Cfg::EV, RV = DVT / Cfg::EV, RT = C / Cfg::EV;
#pragma unroll
        for (int m = 0; m < Cfg::PK; ++m) {
            const int i = tid + Cfg::NTHR * m;
            const int r = i / RK, c = (i - r * RK) * Cfg::EV;
            if (i < Cfg::VK) *reinterpret_cast<u32x4*>(sK + kidx<Cfg>(r, c)) = r < len ? k[m] : z;
        }
#pragma unroll
        for (int m = 0; m < Cfg::PV; ++m) {
            const int i = tid + Cfg::NTHR * m;
            const int r = i / RV, c = (i - r * RV) * Cfg::EV;
            if (i < Cfg::VV) *reinterpret_cast<u32x4*>(sV + r * Cfg::LDV + c) = r < len ? v[m] : z;
        }
#pragma unroll
        for (int m = 0; m < Cfg::PT; ++m) {
            const int i = tid + Cfg::NTHR * m;
            const int r = i / RT, c = (i - r * RT) * Cfg::EV;
            if (i < Cfg::VT) *reinterpret_cast<u32x4*>(sTb + r * Cfg::LDC + c) = tb[m];
        }
#pragma unroll
        for (int m = 0; m < Cfg::PG; ++m) {
            const int i = tid + Cfg::NTHR * m;
            if (i < Cfg::VG) *reinterpret_cast<u32x4*>(sg + 4 * i) = g[m];
        }
    }
};

template <typename T, int DK, int DV, int C, int DVT>
__global__ __launch_bounds__(256) void gdn_scan_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* S0, SeqGeom geom, int H,
    const float* __restrict__ g_ws, const T* __restrict__ Tb_ws,
    T* __restrict__ O, float* S_T) {   // S_T may alias S0
    using Cfg = ScanCfg<T, DK, DV, C, DVT>;
    using M = Mfma<T>;
    using Frag = typename M::frag;
    constexpr int NW = Cfg::NW, NVB = Cfg::NVB, NDBW = Cfg::NDBW, KS = Cfg::KS;
    extern __shared__ __align__(16) unsigned char smem[];
    T* sK0 = reinterpret_cast<T*>(smem + Cfg::OFF_K);
    T* sV = reinterpret_cast<T*>(smem + Cfg::OFF_V);
    T* sTb = reinterpret_cast<T*>(smem + Cfg::OFF_TB);
    T* sSb = reinterpret_cast<T*>(smem + Cfg::OFF_SB);
    T* sXt = reinterpret_cast<T*>(smem + Cfg::OFF_XT);
    T* sVpt = reinterpret_cast<T*>(smem + Cfg::OFF_VPT);
    T* sVdt = reinterpret_cast<T*>(smem + Cfg::OFF_VDT);
    float* sg = reinterpret_cast<float*>(smem + Cfg::OFF_G);     // [g | exp(g) | exp(g_n - g)]

    const int v0 = blockIdx.x * DVT, h = blockIdx.y, seq = blockIdx.z;
    const int l = lane_id(), w = wave_id();
    const int n = l & 15, g4 = 4 * (l >> 4);

    // Each wave runs its own copy of the loop, specialised on its token block
    // cb (a compile-time constant there), so that no branch on the wave index
    // remains inside the chunk loop.
    auto run = [&](auto cb_const) __attribute__((always_inline)) {
    constexpr int cb = decltype(cb_const)::value;

    // state slice S^T (Dk x DVT): wave w owns d-blocks db = w + NW i, all v-blocks;
    // lane (g, n) of tile (i, vb) holds S^T[db*16 + 4g + r][vb*16 + n]
    f32x4 St[NDBW][NVB];
    const int64_t sbase = ((int64_t)seq * H + h) * DV * DK;
#pragma unroll
    for (int i = 0; i < NDBW; ++i) {
#pragma unroll
        for (int vb = 0; vb < NVB; ++vb) {
            const int db = w + NW * i, vv = vb * 16 + n, d = db * 16 + g4;
            St[i][vb] = S0 ? *reinterpret_cast<const f32x4*>(S0 + sbase + (int64_t)(v0 + vv) * DK + d)
                           : zero4();
            store4(sSb + vv * Cfg::LDK + d, St[i][vb][0], St[i][vb][1], St[i][vb][2], St[i][vb][3]);
        }
    }

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
    auto fetch = [&](auto& dst, int cc) __attribute__((always_inline)) {
        const int t0 = ts + cc * C;
        dst.load(k, q, v, g_ws, Tb_ws, t0, min(C, te - t0), (int64_t)(first + cc) * H + h, H, h, v0);
    };
    using Fetch = ChunkFetch<Cfg, T, DK, DV, C, DVT>;
    static_assert(Cfg::NPF == 2 || Cfg::NPF == 3, "ring of two or three register sets");
    Fetch pf0, pf1, pf2;                   // pf2 unused when NPF == 2
    Frag qcur[Cfg::NQ];                    // Q fragments of the current chunk
    if (count > 0) {
        fetch(pf0, 0);
        pf0.store(sK0, sV, sTb, sg, min(C, te - ts));
#pragma unroll
        for (int j = 0; j < Cfg::NQ; ++j) qcur[j] = pf0.q[j];
        fetch(pf1, min(1, count - 1));
        if constexpr (Cfg::NPF == 3) {
            fetch(pf2, min(2, count - 1));
            fetch(pf0, min(3, count - 1));
        } else {
            fetch(pf0, min(2, count - 1));
        }
    }
    __syncthreads();

    auto chunk_step = [&](const int cc, Fetch& nxt) __attribute__((always_inline)) {
        const int t0 = ts + cc * C;
        const int len = min(C, te - t0);
        const T* sK = sK0 + (Cfg::KBUF == 2 ? (cc & 1) : 0) * (Cfg::SZ_K / sizeof(T));
        const float* sgam = sg + C;
        const float* sdec = sg + 2 * C;

        // ---- phase A: Y = K S^T, Z^T = S Q^T, P^T = K Q^T for token block cb
        const int cq = cb * 16 + n;        // this lane's token as a column of Z^T, P^T, O^T
        const bool qok = cq < len;
        f32x4 Y[NVB], Zt[NVB], Pt[NW];
#pragma unroll
        for (int vb = 0; vb < NVB; ++vb) Y[vb] = Zt[vb] = zero4();
#pragma unroll
        for (int jb = 0; jb < NW; ++jb) Pt[jb] = zero4();
#pragma unroll
        for (int kk = 0; kk < DK; kk += KS) {
            const Frag aq = qok ? qcur[kk / KS] : Frag{};
            const Frag ak = kfrag_rows<Cfg>(sK, cb * 16, kk);
#pragma unroll
            for (int vb = 0; vb < NVB; ++vb) {
                const Frag bs = frag_kc(sSb, Cfg::LDK, vb * 16, kk);
                Y[vb] = M::mma(ak, bs, Y[vb]);
                Zt[vb] = M::mma(bs, aq, Zt[vb]);
            }
#pragma unroll
            for (int jb = 0; jb < NW; ++jb) {
                if (jb < cb) Pt[jb] = M::mma(kfrag_rows<Cfg>(sK, jb * 16, kk), aq, Pt[jb]);
                else if (jb == cb) Pt[jb] = M::mma(ak, aq, Pt[jb]);
            }
        }
        // X = V - diag(gamma) Y  ->  X^T in LDS (4 consecutive tokens per lane)
        const float4 gam4 = *reinterpret_cast<const float4*>(sgam + cb * 16 + g4);
#pragma unroll
        for (int vb = 0; vb < NVB; ++vb) {
            const int vv = vb * 16 + n, c = cb * 16 + g4;
            const float x0 = to_f32(sV[(c + 0) * Cfg::LDV + vv]) - gam4.x * Y[vb][0];
            const float x1 = to_f32(sV[(c + 1) * Cfg::LDV + vv]) - gam4.y * Y[vb][1];
            const float x2 = to_f32(sV[(c + 2) * Cfg::LDV + vv]) - gam4.z * Y[vb][2];
            const float x3 = to_f32(sV[(c + 3) * Cfg::LDV + vv]) - gam4.w * Y[vb][3];
            store4(sXt + vv * Cfg::LDC + c, x0, x1, x2, x3);
        }
        // Z^T columns scaled by gamma_c; P = (Q K^T) o Gamma o M, kept as P^T tiles
        const float gq = sg[cq];
        const float gamq = sgam[cq];
#pragma unroll
        for (int vb = 0; vb < NVB; ++vb) Zt[vb] *= gamq;
#pragma unroll
        for (int jb = 0; jb < NW; ++jb) {
            if (jb <= cb) {
                const float4 gj = *reinterpret_cast<const float4*>(sg + jb * 16 + g4);
                const int j0 = jb * 16 + g4;
                Pt[jb][0] = j0 + 0 <= cq ? Pt[jb][0] * __expf(gq - gj.x) : 0.f;
                Pt[jb][1] = j0 + 1 <= cq ? Pt[jb][1] * __expf(gq - gj.y) : 0.f;
                Pt[jb][2] = j0 + 2 <= cq ? Pt[jb][2] * __expf(gq - gj.z) : 0.f;
                Pt[jb][3] = j0 + 3 <= cq ? Pt[jb][3] * __expf(gq - gj.w) : 0.f;
            }
        }
        const float gamma_n = sgam[C - 1];
        __syncthreads();

        // ---- phase B: V' = Tb X for token block cb (plain and decayed copies, transposed)
        {
            const int kend = ((cb + 1) * 16 + KS - 1) / KS * KS;
            const float4 dec4 = *reinterpret_cast<const float4*>(sdec + cb * 16 + g4);
#pragma unroll
            for (int vb = 0; vb < NVB; ++vb) {
                f32x4 acc = zero4();
                for (int kk = 0; kk < kend; kk += KS)
                    acc = M::mma(frag_kc(sTb, Cfg::LDC, cb * 16, kk), frag_kc(sXt, Cfg::LDC, vb * 16, kk), acc);
                const int vv = vb * 16 + n, c = cb * 16 + g4;
                store4(sVpt + vv * Cfg::LDC + c, acc[0], acc[1], acc[2], acc[3]);
                store4(sVdt + vv * Cfg::LDC + c, acc[0] * dec4.x, acc[1] * dec4.y, acc[2] * dec4.z,
                       acc[3] * dec4.w);
            }
        }
        __syncthreads();

        // ---- phase C: O^T = Z^T + V'^T P^T (token block cb);  S^T update (own d-blocks)
#pragma unroll
        for (int vb = 0; vb < NVB; ++vb) {
            f32x4 acc = Zt[vb];
#pragma unroll
            for (int jb = 0; jb < NW; ++jb)
                if (jb <= cb) acc = RegB<T>::mma(sVpt, Cfg::LDC, vb * 16, jb * 16, Pt[jb], acc);
            // lane (g, n): O[token cb*16 + n][v0 + vb*16 + 4g .. + 3]
            if (qok)
                store4(O + ((int64_t)(t0 + cq) * H + h) * DV + v0 + vb * 16 + g4, acc[0], acc[1], acc[2],
                       acc[3]);
        }
        {
            Frag bvd[NVB][C / KS];
#pragma unroll
            for (int vb = 0; vb < NVB; ++vb)
#pragma unroll
                for (int kk = 0; kk < C; kk += KS) bvd[vb][kk / KS] = frag_kc(sVdt, Cfg::LDC, vb * 16, kk);
#pragma unroll
            for (int i = 0; i < NDBW; ++i) {
                const int db = w + NW * i;
#pragma unroll
                for (int vb = 0; vb < NVB; ++vb) St[i][vb] *= gamma_n;
#pragma unroll
                for (int kk = 0; kk < C; kk += KS) {
                    const Frag a = kfrag_cols<Cfg>(sK, kk, db * 16);
#pragma unroll
                    for (int vb = 0; vb < NVB; ++vb) St[i][vb] = M::mma(a, bvd[vb][kk / KS], St[i][vb]);
                }
#pragma unroll
                for (int vb = 0; vb < NVB; ++vb)
                    store4(sSb + (vb * 16 + n) * Cfg::LDK + db * 16 + g4, St[i][vb][0], St[i][vb][1],
                           St[i][vb][2], St[i][vb][3]);
            }
        }
        if (cc + 1 < count) {
            if constexpr (Cfg::KBUF == 1) __syncthreads();   // the update above still reads sK
            T* sKn = sK0 + (Cfg::KBUF == 2 ? ((cc + 1) & 1) : 0) * (Cfg::SZ_K / sizeof(T));
            nxt.store(sKn, sV, sTb, sg, min(C, te - (t0 + C)));
#pragma unroll
            for (int j = 0; j < Cfg::NQ; ++j) qcur[j] = nxt.q[j];
        }
        // refill this register set (past the end: re-read the last chunk, unused)
        fetch(nxt, min(cc + 1 + Cfg::NPF, count - 1));
        __syncthreads();
    };

    // chunk c + 1 sits in set (c + 1) % NPF
    int base = 0;
    if constexpr (Cfg::NPF == 3) {
        for (; base + 3 <= count; base += 3) {
            chunk_step(base, pf1);
            chunk_step(base + 1, pf2);
            chunk_step(base + 2, pf0);
        }
        if (base < count) chunk_step(base, pf1);
        if (base + 1 < count) chunk_step(base + 1, pf2);
    } else {
        for (; base + 2 <= count; base += 2) {
            chunk_step(base, pf1);
            chunk_step(base + 1, pf0);
        }
        if (base < count) chunk_step(base, pf1);
    }


    if (S_T) {
#pragma unroll
        for (int i = 0; i < NDBW; ++i)
#pragma unroll
            for (int vb = 0; vb < NVB; ++vb) {
                const int db = w + NW * i;
                *reinterpret_cast<f32x4*>(S_T + sbase + (int64_t)(v0 + vb * 16 + n) * DK + db * 16 + g4) =
                    St[i][vb];
            }
    }
    };
    switch (w) {
        case 0: run(std::integral_constant<int, 0>{}); break;
        case 1: if constexpr (NW > 1) run(std::integral_constant<int, (NW > 1 ? 1 : 0)>{}); break;
        case 2: if constexpr (NW > 2) run(std::integral_constant<int, (NW > 2 ? 2 : 0)>{}); break;
        default: if constexpr (NW > 3) run(std::integral_constant<int, (NW > 3 ? 3 : 0)>{}); break;
    }
}

}  // namespace gdn
