// gdn_scan.h -- serial inter-chunk state scan.
//
// One workgroup owns a DVT-row slice of the state of one (sequence, head) and
// walks that sequence's chunks in order.  Rows of S evolve independently (the
// update of the Qiita article, section "Gated-DeltaNet", writes row r of S only
// from v_t[r] and k_t), so slicing Dv needs no communication.
//
// For each chunk, with S the state at the chunk start (row form, S is Dv x Dk):
//   h  = S                                    stored for the output kernel
//   V' = U - W S^T                            per-token prediction error against S
//   S <- gamma_n S + V'^T diag(gamma_n / gamma) K
// V' and the state recursion follow from that article's product form
// S_i = gamma_i S0 A_1..A_i + sum_s (gamma_i/gamma_s) u_s k_s^T A_{s+1}..A_i with
// I - sum w k^T = A_1..A_i and the G_i identity, taken over one chunk; the
// next chunk starts from the previous chunk's last state (section "Chunk
// Computation").  LinearAttention系列解读(六), section 4.4: U - W S^T is each
// token's prediction error against the chunk-start state, corrected for the
// writes of the earlier tokens of the chunk.
#pragma once

#include "gdn_device.h"

namespace gdn {

template <typename T, int DK, int DV, int C, int DVT>
struct ScanCfg {
    static constexpr int PAD = 16 / sizeof(T);
    static constexpr int LDK = DK + PAD;
    static constexpr int LDU = DVT + PAD;
    static constexpr int LDC = C + PAD;
    static constexpr int NVB = DVT / 16, NDB = DK / 16, NT = NVB * NDB;
    static constexpr int TPW = (NT + 3) / 4;           // state tiles per wave
    static constexpr size_t OFF_W = 0;
    static constexpr size_t OFF_K = OFF_W + sizeof(T) * C * LDK;
    static constexpr size_t OFF_U = OFF_K + sizeof(T) * C * LDK;
    static constexpr size_t OFF_S = OFF_U + sizeof(T) * C * LDU;
    static constexpr size_t OFF_VD = OFF_S + sizeof(T) * DVT * LDK;
    static constexpr size_t OFF_G = OFF_VD + sizeof(T) * DVT * LDC;
    static constexpr size_t SMEM = OFF_G + sizeof(float) * C;
    static_assert(DV % DVT == 0 && DVT % 16 == 0, "state slice must be whole 16-row tiles");
};

template <typename T, int DK, int DV, int C, int DVT>
__global__ __launch_bounds__(kThreads) void gdn_scan_kernel(
    const T* __restrict__ k, const float* S0, SeqGeom geom, int H,
    const float* __restrict__ g_ws, const T* __restrict__ W_ws, const T* __restrict__ U_ws,
    T* __restrict__ Vp_ws, T* __restrict__ h_ws, float* S_T) {  // S_T may alias S0
    using Cfg = ScanCfg<T, DK, DV, C, DVT>;
    using M = Mfma<T>;
    extern __shared__ __align__(16) unsigned char smem[];
    T* sW = reinterpret_cast<T*>(smem + Cfg::OFF_W);
    T* sK = reinterpret_cast<T*>(smem + Cfg::OFF_K);
    T* sU = reinterpret_cast<T*>(smem + Cfg::OFF_U);
    T* sS = reinterpret_cast<T*>(smem + Cfg::OFF_S);
    T* sVd = reinterpret_cast<T*>(smem + Cfg::OFF_VD);
    float* sg = reinterpret_cast<float*>(smem + Cfg::OFF_G);

    const int v0 = blockIdx.x * DVT, h = blockIdx.y, seq = blockIdx.z;
    const int l = lane_id(), w = wave_id();
    const int n = l & 15, g4 = 4 * (l >> 4);

    // state slice in MFMA accumulator layout: tile m of this wave is tile
    // index t = w + 4m, rows (t / NDB) * 16 + g4 + r, columns (t % NDB) * 16 + n.
    f32x4 S[Cfg::TPW];
    const int64_t sbase = ((int64_t)seq * H + h) * DV * DK;
#pragma unroll
    for (int m = 0; m < Cfg::TPW; ++m) {
        const int t = w + 4 * m;
        S[m] = zero4();
        if (t < Cfg::NT && S0) {
            const int vr = (t / Cfg::NDB) * 16 + g4, dc = (t % Cfg::NDB) * 16 + n;
#pragma unroll
            for (int r = 0; r < 4; ++r) S[m][r] = S0[sbase + (int64_t)(v0 + vr + r) * DK + dc];
        }
    }

    int first, count;
    seq_slots(geom, seq, first, count);
    for (int cc = 0; cc < count; ++cc) {
        const int slot = first + cc;
        const ChunkInfo ci = chunk_info(geom, slot);
        const int64_t unit = (int64_t)slot * H + h;
        stage_dense<T, DK>(sW, Cfg::LDK, W_ws + unit * C * DK, DK, C);
        stage_tokens<T, DK>(sK, Cfg::LDK, k, ci.t0, ci.len, C, H, h);
        stage_dense<T, DVT>(sU, Cfg::LDU, U_ws + unit * C * DV + v0, DV, C);
        if (threadIdx.x < C) sg[threadIdx.x] = g_ws[unit * C + threadIdx.x];
        // chunk-start state: MFMA operand copy in LDS and the stored h
        T* hout = h_ws + (unit * DV + v0) * DK;
#pragma unroll
        for (int m = 0; m < Cfg::TPW; ++m) {
            const int t = w + 4 * m;
            if (t < Cfg::NT) {
                const int vr = (t / Cfg::NDB) * 16 + g4, dc = (t % Cfg::NDB) * 16 + n;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const T s = from_f32<T>(S[m][r]);
                    sS[(vr + r) * Cfg::LDK + dc] = s;
                    hout[(int64_t)(vr + r) * DK + dc] = s;
                }
            }
        }
        __syncthreads();

        // V' = U - W S^T  (C x DVT), then V'^T to the workspace and the
        // decayed copy diag(gamma_n / gamma) V' (transposed) to LDS.
        const float gl = sg[C - 1];
        T* vpout = Vp_ws + (unit * DV + v0) * C;
        for (int t = w; t < (C / 16) * Cfg::NVB; t += 4) {
            const int cb = t / Cfg::NVB, vb = t - cb * Cfg::NVB;
            f32x4 acc = zero4();
#pragma unroll
            for (int kk = 0; kk < DK; kk += M::KS)
                acc = M::mma(frag_kc(sW, Cfg::LDK, cb * 16, kk), frag_kc(sS, Cfg::LDK, vb * 16, kk), acc);
            const int vv = vb * 16 + n;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int c = cb * 16 + g4 + r;
                const float vp = to_f32(sU[c * Cfg::LDU + vv]) - acc[r];
                vpout[(int64_t)vv * C + c] = from_f32<T>(vp);
                sVd[vv * Cfg::LDC + c] = from_f32<T>(vp * __expf(gl - sg[c]));
            }
        }
        __syncthreads();

        // S <- gamma_n S + (decayed V')^T K
        const float gn = __expf(gl);
#pragma unroll
        for (int m = 0; m < Cfg::TPW; ++m) {
            const int t = w + 4 * m;
            if (t < Cfg::NT) {
                const int vb = t / Cfg::NDB, db = t % Cfg::NDB;
                f32x4 acc = S[m] * gn;
#pragma unroll
                for (int kk = 0; kk < C; kk += M::KS)
                    acc = M::mma(frag_kc(sVd, Cfg::LDC, vb * 16, kk), frag_ks(sK, Cfg::LDK, kk, db * 16), acc);
                S[m] = acc;
            }
        }
        __syncthreads();
    }

    if (S_T) {
#pragma unroll
        for (int m = 0; m < Cfg::TPW; ++m) {
            const int t = w + 4 * m;
            if (t < Cfg::NT) {
                const int vr = (t / Cfg::NDB) * 16 + g4, dc = (t % Cfg::NDB) * 16 + n;
#pragma unroll
                for (int r = 0; r < 4; ++r) S_T[sbase + (int64_t)(v0 + vr + r) * DK + dc] = S[m][r];
            }
        }
    }
}

}  // namespace gdn
