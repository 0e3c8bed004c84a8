// gdn_prep.h -- per-chunk preparation kernel (independent across chunks).
//
// For one chunk of n <= C tokens of one head (row form: K is n x Dk, token i is
// row i):
//   g_i  = sum_{t<=i} log alpha_t              in-chunk inclusive cumulative log-gate
//   A    = strict_lower( diag(beta) (K K^T o Gamma) ),   Gamma_ij = exp(g_i - g_j)
//   T    = (I + A)^-1                           unit lower triangular
//   Tb   = T diag(beta)                         stored (input dtype; bf16 rows with the
//                                               column order described at the store), with
//                                               g, exp(g), exp(g_n - g) (fp32, [3][C] per chunk)
// The scan kernel applies Tb to the chunk's prediction errors:
//   V' = Tb (V - diag(gamma) K S^T) = U - W S^T,  U = T diag(beta) V,
//   W = T diag(beta o gamma) K,  gamma_i = exp(g_i).
// Sources: Qiita article on the Linear Attention lineage, section
// "Gated-DeltaNet": the w and u recursions and their triangular systems
// (I + (strictly triangular part of K^T K, gated by gamma_i/gamma_s) D_beta)^-1;
// LinearAttention系列解读(六)：DeltaNet的Chunkwise Form推导, sections 4.2 and 4.5:
// the inverse is a small unit-lower-triangular one, and T depends on the chunk's
// keys and gates only, never on the state, so every chunk is prepared in parallel.
// Gating: I + A = D_gamma (I + A_0) D_gamma^-1 with A_0 the ungated matrix, so
// T diag(beta o gamma) K is diag(gamma) times the ungated W of that section.
//
// Padding: rows i >= n act as tokens with k = 0, beta = 0, log alpha = 0, which
// makes their rows and columns of Tb zero.
#pragma once

#include "gdn_device.h"

namespace gdn {

template <typename T, int DK, int C>
struct PrepCfg {
    static constexpr int PAD = 16 / sizeof(T);           // keeps 16-byte row alignment
    static constexpr int LDK = DK + PAD;
    static constexpr int LDA = C + 4;                     // fp32 A and T
    static constexpr int LDR = 16 + 4;                    // fp32 16x16 scratch per wave
    static constexpr int NB = C / 16;                     // 16-row diagonal blocks
    static constexpr size_t SZ_K = sizeof(T) * C * LDK;
    static constexpr size_t SZ_T = sizeof(float) * C * LDA;
    static constexpr size_t OFF_K = 0;                    // K, then T (K is dead by then)
    static constexpr size_t OFF_A = OFF_K + (SZ_K > SZ_T ? SZ_K : SZ_T);
    static constexpr size_t OFF_R = OFF_A + sizeof(float) * C * LDA;
    static constexpr size_t OFF_G = OFF_R + sizeof(float) * 4 * 16 * LDR;
    static constexpr size_t OFF_B = OFF_G + sizeof(float) * C;
    static constexpr size_t SMEM = OFF_B + sizeof(float) * C;
    static_assert(C <= 64 && C % 16 == 0, "at most four 16-row blocks");
};

template <typename T, int DK, int C>
__global__ __launch_bounds__(kThreads) void gdn_prep_kernel(
    const T* __restrict__ k, const float* __restrict__ log_alpha,
    const float* __restrict__ beta, SeqGeom geom, int H,
    float* __restrict__ g_ws, T* __restrict__ Tb_ws) {
    using Cfg = PrepCfg<T, DK, C>;
    using M = Mfma<T>;
    extern __shared__ __align__(16) unsigned char smem[];
    T* sK = reinterpret_cast<T*>(smem + Cfg::OFF_K);
    float* sA = reinterpret_cast<float*>(smem + Cfg::OFF_A);
    float* sg = reinterpret_cast<float*>(smem + Cfg::OFF_G);
    float* sb = reinterpret_cast<float*>(smem + Cfg::OFF_B);

    const int slot = blockIdx.x, h = blockIdx.y;
    const ChunkInfo ci = chunk_info(geom, slot);
    if (ci.len <= 0) return;
    const int l = lane_id(), w = wave_id();
    const int64_t unit = (int64_t)slot * H + h;

    // gates: inclusive prefix sum of log alpha inside the chunk (wave 0)
    if (w == 0) {
        float la = 0.f, b = 0.f;
        if (l < C && l < ci.len) {
            const int64_t x = (int64_t)(ci.t0 + l) * H + h;
            la = log_alpha ? log_alpha[x] : 0.f;
            b = beta[x];
        }
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(la, off, 64);
            if (l >= off) la += y;
        }
        const float glast = __shfl(la, C - 1, 64);
        if (l < C) {
            sg[l] = la;
            sb[l] = b;
            float* gout = g_ws + unit * 3 * C;
            gout[l] = la;                            // g_i
            gout[C + l] = __expf(la);                // gamma_i = exp(g_i)
            gout[2 * C + l] = __expf(glast - la);    // gamma_n / gamma_i
        }
    }
    stage_tokens<T, DK, kThreads>(sK, Cfg::LDK, k, ci.t0, ci.len, C, H, h);
    __syncthreads();

    // A = strict_lower(diag(beta) (K K^T o Gamma)) on MFMA, lower tiles only
    constexpr int NT = C / 16;
    for (int t = w; t < NT * NT; t += kThreads / 64) {
        const int ti = t / NT, tj = t - ti * NT;
        if (tj > ti) continue;
        f32x4 acc = zero4();
#pragma unroll
        for (int kk = 0; kk < DK; kk += M::KS)
            acc = M::mma(frag_kc(sK, Cfg::LDK, ti * 16, kk), frag_kc(sK, Cfg::LDK, tj * 16, kk), acc);
        const int j = tj * 16 + (l & 15);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = ti * 16 + 4 * (l >> 4) + r;
            sA[i * Cfg::LDA + j] = (j < i) ? sb[i] * acc[r] * __expf(sg[i] - sg[j]) : 0.f;
        }
    }
    __syncthreads();

    // T = (I + A)^-1, blocked by 16 rows.  Diagonal blocks by forward
    // substitution (wave 0, lane = 16 b + column); then, one block diagonal
    // at a time, T_ij = -T_ii (sum_{j<=m<i} A_im T_mj) on fp32 MFMA.
    float* sT = reinterpret_cast<float*>(smem + Cfg::OFF_K);
    float* sR = reinterpret_cast<float*>(smem + Cfg::OFF_R) + w * 16 * Cfg::LDR;
    using MF = Mfma<float>;
    if (w == 0 && l < C) {
        const int b = l >> 4, c = l & 15;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float* arow = sA + (16 * b + i) * Cfg::LDA + 16 * b;
            float acc = (i == c) ? 1.f : 0.f;
#pragma unroll
            for (int j = 0; j < i; ++j) acc -= arow[j] * x[j];
            x[i] = acc;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sT[(16 * b + i) * Cfg::LDA + 16 * b + c] = x[i];
    }
    __syncthreads();
#pragma unroll
    for (int d = 1; d < Cfg::NB; ++d) {
        const int j = w, i = w + d;          // wave w builds block (j + d, j)
        const bool mine = w < Cfg::NB - d;
        if (mine) {
            f32x4 acc = zero4();
            for (int kk = 16 * j; kk < 16 * i; kk += MF::KS)
                acc = MF::mma(frag_kc(sA, Cfg::LDA, 16 * i, kk), frag_ks(sT, Cfg::LDA, kk, 16 * j), acc);
#pragma unroll
            for (int r = 0; r < 4; ++r) sR[(4 * (l >> 4) + r) * Cfg::LDR + (l & 15)] = acc[r];
        }
        __syncthreads();
        if (mine) {
            f32x4 acc = zero4();
#pragma unroll
            for (int kk = 0; kk < 16; kk += MF::KS)
                acc = MF::mma(frag_kc(sT, Cfg::LDA, 16 * i, 16 * i + kk), frag_ks(sR, Cfg::LDR, kk, 0), acc);
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sT[(16 * i + 4 * (l >> 4) + r) * Cfg::LDA + 16 * j + (l & 15)] = -acc[r];
        }
        __syncthreads();
    }

    // Tb = T diag(beta), zero above the diagonal; 16-byte stores.  fp32 rows are
    // plain; a bf16 row stores each 32-column group as the 4-column runs
    // (0-3, 16-19, 4-7, 20-23, 8-11, 24-27, 12-15, 28-31), so that the 16 bytes at
    // group offset 8g are the operand of a 16-deep block pair (4g .. 4g+3 of both)
    constexpr int EV = 16 / sizeof(T), VPR = C / EV;
    static_assert(sizeof(T) == 4 || C % 32 == 0, "bf16 Tb groups of 32 columns");
    T* out = Tb_ws + unit * C * C;
    for (int idx = threadIdx.x; idx < C * VPR; idx += kThreads) {
        const int i = idx / VPR, c0 = (idx - i * VPR) * EV;
        union { uint4 u; T e[EV]; } pk;
#pragma unroll
        for (int e = 0; e < EV; ++e) {
            const int c = sizeof(T) == 4 ? c0 + e : (c0 & ~31) + 16 * (e >> 2) + ((c0 & 31) >> 1) + (e & 3);
            const bool lower = (c >> 4) < (i >> 4) || ((c >> 4) == (i >> 4) && c <= i);
            pk.e[e] = from_f32<T>(lower ? sT[i * Cfg::LDA + c] * sb[c] : 0.f);
        }
        *reinterpret_cast<uint4*>(out + i * C + c0) = pk.u;
    }
}

}  // namespace gdn
