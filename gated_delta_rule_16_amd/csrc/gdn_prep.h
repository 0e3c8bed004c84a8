// gdn_prep.h -- per-chunk preparation kernel (independent across chunks).
//
// For one chunk of n <= C tokens of one head (row form: K is n x Dk, token i is
// row i):
//   g_i  = sum_{t<=i} log alpha_t              in-chunk inclusive cumulative log-gate
//   A    = strict_lower( diag(beta) (K K^T o Gamma) ),   Gamma_ij = exp(g_i - g_j)
//   T    = (I + A)^-1                           unit lower triangular
//   Tb   = T diag(beta)                         stored (input dtype), with g (fp32)
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
    static constexpr int LDA = C + 4;                     // fp32 A
    static constexpr size_t OFF_K = 0;
    static constexpr size_t OFF_A = OFF_K + sizeof(T) * C * LDK;
    static constexpr size_t OFF_G = OFF_A + sizeof(float) * C * LDA;
    static constexpr size_t OFF_B = OFF_G + sizeof(float) * C;
    static constexpr size_t SMEM = OFF_B + sizeof(float) * C;
    static_assert(C <= 64 && C % 16 == 0, "one wave solves the chunk's triangular system");
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
        if (l < C) {
            sg[l] = la;
            sb[l] = b;
            g_ws[unit * C + l] = la;
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

    // T = (I + A)^-1 by forward substitution; lane c owns column c of T and
    // writes column c of Tb = T diag(beta) (each row store is contiguous).
    if (w == 0) {
        const int c = l;
        float x[C];
#pragma unroll
        for (int i = 0; i < C; ++i) {
            float acc = (i == c) ? 1.f : 0.f;
            const float* arow = sA + i * Cfg::LDA;
#pragma unroll
            for (int j = 0; j < (i & ~3); j += 4) {
                const float4 a4 = *reinterpret_cast<const float4*>(arow + j);
                acc -= a4.x * x[j] + a4.y * x[j + 1] + a4.z * x[j + 2] + a4.w * x[j + 3];
            }
#pragma unroll
            for (int j = (i & ~3); j < i; ++j) acc -= arow[j] * x[j];
            x[i] = acc;
        }
        if (c < C) {
            const float bc = sb[c];
            T* out = Tb_ws + unit * C * C + c;
#pragma unroll
            for (int i = 0; i < C; ++i) out[i * C] = from_f32<T>(x[i] * bc);
        }
    }
}

}  // namespace gdn
