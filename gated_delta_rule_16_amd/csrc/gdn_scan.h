// gdn_scan.h -- serial inter-chunk state scan with the chunk outputs fused in.
//
// One workgroup (8 waves) owns a DVT-row slice of the state of one (sequence,
// head) and walks that sequence's chunks in order, keeping its slice of S in
// MFMA accumulators (fp32) for the whole sequence.  Rows of S evolve
// independently (the update of the Qiita article on the Linear Attention
// lineage, section "Gated-DeltaNet", writes row r of S only from v_t[r] and
// k_t), so slicing Dv needs no communication between workgroups.
//
// Per chunk (row form; S = state at the chunk start, Dv x Dk; gamma_i = exp(g_i);
// Tb = T diag(beta) from the prep kernel):
//   phase A   Y = K S^T,  Z = Q S^T                  (both read only S)
//             X = V - diag(gamma) Y                  prediction errors vs. the gated start state
//   phase B   V' = Tb X  (= U - W S^T)               corrected for the chunk's earlier writes
//             P  = (Q K^T) o Gamma o M               intra-chunk decayed causal scores
//   phase C   O  = diag(gamma) Z + P V'              the chunk's outputs
//             S <- gamma_n S + V'^T diag(gamma_n / gamma) K
// Sources: the same Qiita section (product form of S_i with I - sum w k^T =
// A_1..A_i and the G_i identity; parallel form H = S0 (Q - W (M^T o K^T Q)) D_gamma
// + U (Gamma o K^T Q) restricted to one chunk) and its section "Chunk
// Computation" (chunk j starts from chunk j-1's last state);
// LinearAttention系列解读(六)：DeltaNet的Chunkwise Form推导, section 4.4 (U - W S^T is
// each token's prediction error against the chunk-start state, corrected by the
// triangular solve) and section 4.5 (T, W, U do not depend on S).
//
// The chunks' inputs (K, Q, the V slice, Tb, g) do not depend on S: they are
// fetched into a ring of register sets NPF chunks ahead and written to LDS at
// the end of the previous chunk's phase C, so global-memory latency overlaps
// the serial work.
#pragma once

#include "gdn_device.h"

namespace gdn {

constexpr int kScanThreads = 512;   // 8 waves

template <typename T, int DK, int DV, int C, int DVT>
struct ScanCfg {
    static constexpr int NW = kScanThreads / 64, NTHR = kScanThreads;
    static constexpr int PAD = 16 / sizeof(T);
    static constexpr int LDK = DK + PAD, LDC = C + PAD, LDV = DVT + PAD;
    static constexpr int NCB = C / 16, NVB = DVT / 16, NDB = DK / 16;
    static constexpr int NTO = NCB * NVB, TPO = (NTO + NW - 1) / NW;   // output tiles
    static constexpr int NTS = NVB * NDB, TPS = (NTS + NW - 1) / NW;   // state tiles
    static constexpr int NTP = NCB * (NCB + 1) / 2;                    // lower tiles of P
    static constexpr int EV = 16 / sizeof(T);                          // elements per 16 B
    static constexpr int VK = C * DK / EV, PK = (VK + NTHR - 1) / NTHR;
    static constexpr int VV = C * DVT / EV, PV = (VV + NTHR - 1) / NTHR;
    static constexpr int VT = C * C / EV, PT = (VT + NTHR - 1) / NTHR;
    static constexpr int VG = C / 4;
    static constexpr int NPF = sizeof(T) == 2 ? 3 : 2;   // chunks fetched ahead, in registers
    static constexpr size_t SZ_K = sizeof(T) * C * LDK;
    static constexpr size_t SZ_REST = SZ_K                       // Q
                                    + sizeof(T) * C * LDV        // V slice
                                    + 2 * sizeof(T) * C * LDC    // Tb, P
                                    + sizeof(T) * DVT * LDK      // S (operand copy)
                                    + 3 * sizeof(T) * DVT * LDC  // X^T, V'^T, decayed V'^T
                                    + sizeof(float) * C;         // g
    static constexpr size_t LDS_MAX = 160 * 1024;
    static constexpr int KBUF = (2 * SZ_K + SZ_REST <= LDS_MAX) ? 2 : 1;   // K double buffer
    static constexpr size_t OFF_K = 0;
    static constexpr size_t OFF_Q = OFF_K + KBUF * SZ_K;
    static constexpr size_t OFF_V = OFF_Q + SZ_K;
    static constexpr size_t OFF_TB = OFF_V + sizeof(T) * C * LDV;
    static constexpr size_t OFF_P = OFF_TB + sizeof(T) * C * LDC;
    static constexpr size_t OFF_SB = OFF_P + sizeof(T) * C * LDC;
    static constexpr size_t OFF_XT = OFF_SB + sizeof(T) * DVT * LDK;
    static constexpr size_t OFF_VPT = OFF_XT + sizeof(T) * DVT * LDC;
    static constexpr size_t OFF_VDT = OFF_VPT + sizeof(T) * DVT * LDC;
    static constexpr size_t OFF_G = OFF_VDT + sizeof(T) * DVT * LDC;
    static constexpr size_t SMEM = OFF_G + sizeof(float) * C;
    static_assert(SMEM <= LDS_MAX, "scan workgroup exceeds the LDS of one CU");
    static_assert(DV % DVT == 0 && DVT % 16 == 0 && C % 16 == 0 && C <= 64, "tile shapes");
    static_assert(C % Mfma<T>::KS == 0, "chunk must cover whole MFMA steps");
};

// Register-staged copy of one chunk's state-independent inputs.
template <typename Cfg, typename T, int DK, int DV, int C, int DVT>
struct ChunkFetch {
    u32x4 k[Cfg::PK], q[Cfg::PK], v[Cfg::PV], tb[Cfg::PT], g;

    // Every lane issues every load, unmasked (rows past the chunk end read row
    // 0 of the chunk): nothing consumes the registers until store(), so the
    // compiler waits only for the oldest register set.  store() zeroes the
    // rows past the end.
    __device__ __forceinline__ void load(const T* __restrict__ kg, const T* __restrict__ qg,
                                         const T* __restrict__ vg, const float* __restrict__ g_ws,
                                         const T* __restrict__ Tb_ws, int t0, int len,
                                         int64_t unit, int H, int h, int v0) {
        const int tid = threadIdx.x;
        constexpr int RK = DK / Cfg::EV, RV = DVT / Cfg::EV;
#pragma unroll
        for (int m = 0; m < Cfg::PK; ++m) {
            const int i = (tid + Cfg::NTHR * m) % Cfg::VK;
            const int r = i / RK, c = (i - r * RK) * Cfg::EV;
            const int64_t off = ((int64_t)(t0 + (r < len ? r : 0)) * H + h) * DK + c;
            k[m] = *reinterpret_cast<const u32x4*>(kg + off);
            q[m] = *reinterpret_cast<const u32x4*>(qg + off);
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
        g = *reinterpret_cast<const u32x4*>(g_ws + unit * C + 4 * (tid % Cfg::VG));
    }

    __device__ __forceinline__ void store(T* sK, T* sQ, T* sV, T* sTb, float* sg, int len) const {
        const int tid = threadIdx.x;
        const u32x4 z = {0u, 0u, 0u, 0u};
        constexpr int RK = DK / Cfg::EV, RV = DVT / Cfg::EV, RT = C / Cfg::EV;
#pragma unroll
        for (int m = 0; m < Cfg::PK; ++m) {
            const int i = tid + Cfg::NTHR * m;
            const int r = i / RK, c = (i - r * RK) * Cfg::EV;
            if (i < Cfg::VK) {
                *reinterpret_cast<u32x4*>(sK + r * Cfg::LDK + c) = r < len ? k[m] : z;
                *reinterpret_cast<u32x4*>(sQ + r * Cfg::LDK + c) = r < len ? q[m] : z;
            }
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
        if (tid < Cfg::VG) *reinterpret_cast<u32x4*>(sg + 4 * tid) = g;
    }
};

__device__ __forceinline__ void lower_tile(int t, int& cb, int& jb) {
    cb = 0;
    while (t > cb) { t -= cb + 1; ++cb; }
    jb = t;
}

template <typename T, int DK, int DV, int C, int DVT>
__global__ __launch_bounds__(kScanThreads) void gdn_scan_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* S0, SeqGeom geom, int H,
    const float* __restrict__ g_ws, const T* __restrict__ Tb_ws,
    T* __restrict__ O, float* S_T) {   // S_T may alias S0
    using Cfg = ScanCfg<T, DK, DV, C, DVT>;
    using M = Mfma<T>;
    constexpr int NW = Cfg::NW;
    extern __shared__ __align__(16) unsigned char smem[];
    T* sK0 = reinterpret_cast<T*>(smem + Cfg::OFF_K);
    T* sQ = reinterpret_cast<T*>(smem + Cfg::OFF_Q);
    T* sV = reinterpret_cast<T*>(smem + Cfg::OFF_V);
    T* sTb = reinterpret_cast<T*>(smem + Cfg::OFF_TB);
    T* sP = reinterpret_cast<T*>(smem + Cfg::OFF_P);
    T* sSb = reinterpret_cast<T*>(smem + Cfg::OFF_SB);
    T* sXt = reinterpret_cast<T*>(smem + Cfg::OFF_XT);
    T* sVpt = reinterpret_cast<T*>(smem + Cfg::OFF_VPT);
    T* sVdt = reinterpret_cast<T*>(smem + Cfg::OFF_VDT);
    float* sg = reinterpret_cast<float*>(smem + Cfg::OFF_G);

    const int v0 = blockIdx.x * DVT, h = blockIdx.y, seq = blockIdx.z;
    const int tid = threadIdx.x, l = lane_id(), w = wave_id();
    const int n = l & 15, g4 = 4 * (l >> 4);

    // upper tiles of P stay zero (the P V' contraction may span them)
    for (int i = tid; i < C * C; i += Cfg::NTHR) {
        const int r = i / C, c = i - r * C;
        if (c / 16 > r / 16) sP[r * Cfg::LDC + c] = from_f32<T>(0.f);
    }

    // state slice: wave w owns state tiles t = w + NW m, rows (t / NDB) * 16 + g4 + r,
    // columns (t % NDB) * 16 + n; its bf16/fp32 operand copy lives in sSb.
    f32x4 S[Cfg::TPS];
    const int64_t sbase = ((int64_t)seq * H + h) * DV * DK;
#pragma unroll
    for (int m = 0; m < Cfg::TPS; ++m) {
        const int t = w + NW * m;
        S[m] = zero4();
        if (t < Cfg::NTS) {
            const int vr = (t / Cfg::NDB) * 16 + g4, dc = (t % Cfg::NDB) * 16 + n;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if (S0) S[m][r] = S0[sbase + (int64_t)(v0 + vr + r) * DK + dc];
                sSb[(vr + r) * Cfg::LDK + dc] = from_f32<T>(S[m][r]);
            }
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
        const int len = min(C, te - t0);
        dst.load(k, q, v, g_ws, Tb_ws, t0, len, (int64_t)(first + cc) * H + h, H, h, v0);
    };
    // register ring: chunk j of the sequence is fetched into set j % NPF,
    // NPF chunks before it is needed, and written to LDS one chunk ahead
    using Fetch = ChunkFetch<Cfg, T, DK, DV, C, DVT>;
    static_assert(Cfg::NPF == 2 || Cfg::NPF == 3, "ring of two or three register sets");
    Fetch pf0, pf1, pf2;   // pf2 unused when NPF == 2
    if (count > 0) {
        fetch(pf0, 0);
        pf0.store(sK0, sQ, sV, sTb, sg, min(C, te - ts));
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
            ChunkInfo ci;
            ci.t0 = ts + cc * C;
            ci.len = min(C, te - ci.t0);
            T* sK = sK0 + (Cfg::KBUF == 2 ? (cc & 1) : 0) * (Cfg::SZ_K / sizeof(T));

            // ---- phase A: Y = K S^T and Z = Q S^T; X = V - diag(gamma) Y (to LDS, transposed)
            const float gn = sg[C - 1];
            f32x4 Zr[Cfg::TPO];
#pragma unroll
            for (int m = 0; m < Cfg::TPO; ++m) {
                const int t = w + NW * m;
                Zr[m] = zero4();
                if (t < Cfg::NTO) {
                    const int cb = t / Cfg::NVB, vb = t - cb * Cfg::NVB;
                    f32x4 accY = zero4(), accZ = zero4();
#pragma unroll
                    for (int kk = 0; kk < DK; kk += M::KS) {
                        const auto bS = frag_kc(sSb, Cfg::LDK, vb * 16, kk);
                        accY = M::mma(frag_kc(sK, Cfg::LDK, cb * 16, kk), bS, accY);
                        accZ = M::mma(frag_kc(sQ, Cfg::LDK, cb * 16, kk), bS, accZ);
                    }
                    const int vv = vb * 16 + n;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int c = cb * 16 + g4 + r;
                        const float gam = __expf(sg[c]);
                        sXt[vv * Cfg::LDC + c] = from_f32<T>(to_f32(sV[c * Cfg::LDV + vv]) - gam * accY[r]);
                        Zr[m][r] = gam * accZ[r];
                    }
                }
            }
            __syncthreads();

            // ---- phase B: V' = Tb X (plain and decayed copies, transposed); P
#pragma unroll
            for (int m = 0; m < Cfg::TPO; ++m) {
                const int t = w + NW * m;
                if (t < Cfg::NTO) {
                    const int cb = t / Cfg::NVB, vb = t - cb * Cfg::NVB;
                    const int kend = ((cb + 1) * 16 + M::KS - 1) / M::KS * M::KS;
                    f32x4 acc = zero4();
                    for (int kk = 0; kk < kend; kk += M::KS)
                        acc = M::mma(frag_kc(sTb, Cfg::LDC, cb * 16, kk), frag_kc(sXt, Cfg::LDC, vb * 16, kk), acc);
                    const int vv = vb * 16 + n;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int c = cb * 16 + g4 + r;
                        sVpt[vv * Cfg::LDC + c] = from_f32<T>(acc[r]);
                        sVdt[vv * Cfg::LDC + c] = from_f32<T>(acc[r] * __expf(gn - sg[c]));
                    }
                }
            }
            for (int t = w; t < Cfg::NTP; t += NW) {
                int cb, jb;
                lower_tile(t, cb, jb);
                f32x4 acc = zero4();
#pragma unroll
                for (int kk = 0; kk < DK; kk += M::KS)
                    acc = M::mma(frag_kc(sQ, Cfg::LDK, cb * 16, kk), frag_kc(sK, Cfg::LDK, jb * 16, kk), acc);
                const int j = jb * 16 + n;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int i = cb * 16 + g4 + r;
                    sP[i * Cfg::LDC + j] = from_f32<T>(j <= i ? acc[r] * __expf(sg[i] - sg[j]) : 0.f);
                }
            }
            const float gamma_n = __expf(gn);
            __syncthreads();

            // ---- phase C: O = diag(gamma) Z + P V';  S <- gamma_n S + V'd^T K
#pragma unroll
            for (int m = 0; m < Cfg::TPO; ++m) {
                const int t = w + NW * m;
                if (t < Cfg::NTO) {
                    const int cb = t / Cfg::NVB, vb = t - cb * Cfg::NVB;
                    const int kend = ((cb + 1) * 16 + M::KS - 1) / M::KS * M::KS;
                    f32x4 acc = Zr[m];
                    for (int kk = 0; kk < kend; kk += M::KS)
                        acc = M::mma(frag_kc(sP, Cfg::LDC, cb * 16, kk), frag_kc(sVpt, Cfg::LDC, vb * 16, kk), acc);
                    const int vv = v0 + vb * 16 + n;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int c = cb * 16 + g4 + r;
                        if (c < ci.len) O[((int64_t)(ci.t0 + c) * H + h) * DV + vv] = from_f32<T>(acc[r]);
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < Cfg::TPS; ++m) {
                const int t = w + NW * m;
                if (t < Cfg::NTS) {
                    const int vb = t / Cfg::NDB, db = t - vb * Cfg::NDB;
                    f32x4 acc = S[m] * gamma_n;
#pragma unroll
                    for (int kk = 0; kk < C; kk += M::KS)
                        acc = M::mma(frag_kc(sVdt, Cfg::LDC, vb * 16, kk), frag_ks(sK, Cfg::LDK, kk, db * 16), acc);
                    S[m] = acc;
                    const int vr = vb * 16 + g4, dc = db * 16 + n;
#pragma unroll
                    for (int r = 0; r < 4; ++r) sSb[(vr + r) * Cfg::LDK + dc] = from_f32<T>(acc[r]);
                }
            }
            if (cc + 1 < count) {
                if constexpr (Cfg::KBUF == 1) __syncthreads();   // the update above still reads sK
                T* sKn = sK0 + (Cfg::KBUF == 2 ? ((cc + 1) & 1) : 0) * (Cfg::SZ_K / sizeof(T));
                nxt.store(sKn, sQ, sV, sTb, sg, min(C, te - (ci.t0 + C)));
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
        for (int m = 0; m < Cfg::TPS; ++m) {
            const int t = w + NW * m;
            if (t < Cfg::NTS) {
                const int vr = (t / Cfg::NDB) * 16 + g4, dc = (t % Cfg::NDB) * 16 + n;
#pragma unroll
                for (int r = 0; r < 4; ++r) S_T[sbase + (int64_t)(v0 + vr + r) * DK + dc] = S[m][r];
            }
        }
    }
}

}  // namespace gdn
