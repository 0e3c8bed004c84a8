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
//
// The kernel is persistent: each workgroup walks units (chunk slot, head)
// u = blockIdx.x, blockIdx.x + gridDim.x, ... and loads the next unit's keys
// and gates into registers while it works on the current one, so that the
// loads' latency overlaps computation.
#pragma once

#include "gdn_device.h"

namespace gdn {

template <typename T, int DK, int C>
struct PrepCfg {
    static constexpr bool BF = sizeof(T) == 2;
    static constexpr int ES = sizeof(T), EV = 16 / ES;
    static constexpr int NB = C / 16;                     // 16-row blocks
    static constexpr int NT = NB * (NB + 1) / 2;          // lower 16x16 tiles of A
    // K rows: bf16 unpadded with the XOR swizzle of kind 1 (16-byte row reads of
    // 8 consecutive rows hit disjoint banks); fp32 padded by one block
    static constexpr int KB = DK / EV, KP = BF ? KB : KB + 1, KSW = BF ? 1 : 0;
    static constexpr int LDK = KP * EV;
    static constexpr int LDA = C + 4;                     // fp32 A and T rows
    static constexpr int NL = (C * KB + kThreads - 1) / kThreads;   // 16-byte K loads per lane
    static constexpr size_t SZ_K = (size_t)C * LDK * ES;
    static constexpr size_t SZ_T = sizeof(float) * C * LDA;
    static constexpr size_t OFF_K = 0;                    // K, then T (K is dead by then)
    static constexpr size_t OFF_A = ((SZ_K > SZ_T ? SZ_K : SZ_T) + 15) / 16 * 16;
    static constexpr size_t OFF_G = OFF_A + SZ_T;
    static constexpr size_t OFF_B = OFF_G + sizeof(float) * C;
    static constexpr size_t SMEM = OFF_B + sizeof(float) * C;
    static_assert(C <= 64 && C % 16 == 0, "at most four 16-row blocks");
    static_assert(!BF || KB % 8 == 0, "bf16 K rows of at least 8 blocks");
};

// c += A B over one 16-deep block with fp32 MFMA: lane (g, n) holds a = A[n][4g .. 4g+3]
// and b = B[4g .. 4g+3][n] (the 16x16 accumulator layout of B)
__device__ __forceinline__ f32x4 mma16_f32(f32x4 a, f32x4 b, f32x4 c) {
#pragma unroll
    for (int r = 0; r < 4; ++r) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[r], b[r], c, 0, 0, 0);
    return c;
}

template <typename T, int DK, int C>
__global__ __launch_bounds__(kThreads) void gdn_prep_kernel(
    const T* __restrict__ k, const float* __restrict__ log_alpha,
    const float* __restrict__ beta, SeqGeom geom, int H, int units,
    float* __restrict__ g_ws, T* __restrict__ Tb_ws) {
    using Cfg = PrepCfg<T, DK, C>;
    using M = Mfma<T>;
    using MF = Mfma<float>;
    extern __shared__ __align__(16) unsigned char smem[];
    T* sK = reinterpret_cast<T*>(smem + Cfg::OFF_K);
    float* sT = reinterpret_cast<float*>(smem + Cfg::OFF_K);
    float* sA = reinterpret_cast<float*>(smem + Cfg::OFF_A);
    float* sg = reinterpret_cast<float*>(smem + Cfg::OFF_G);
    float* sb = reinterpret_cast<float*>(smem + Cfg::OFF_B);

    const int tid = threadIdx.x, l = lane_id(), w = wave_id();
    const int64_t rs_k = (int64_t)H * DK * Cfg::ES;

    // this lane's K loads: slot s = tid + kThreads j is row s / KB, block s % KB
    uint32_t koff[Cfg::NL];
    int kdst[Cfg::NL];
#pragma unroll
    for (int j = 0; j < Cfg::NL; ++j) {
        const int s = tid + kThreads * j, r = s / Cfg::KB, b = s - r * Cfg::KB;
        const bool ok = r < C;
        koff[j] = ok ? (uint32_t)(r * rs_k + b * 16) : kOutOfRange;
        kdst[j] = ok ? (r * Cfg::KP + (b ^ swz<Cfg::KSW>(r))) * 16 : -1;
    }
    auto kidx = [](int r, int c) __attribute__((always_inline)) {
        return (r * Cfg::KP + ((c / Cfg::EV) ^ swz<Cfg::KSW>(r))) * Cfg::EV + (c % Cfg::EV);
    };

    // keys and gates of unit u into registers (rows past the chunk end read as 0)
    u32x4 kv[Cfg::NL];
    float la_n = 0.f, be_n = 0.f;
    ChunkInfo ci_n{};
    auto fetch = [&](int u) __attribute__((always_inline)) {
        const int slot = u / H, h = u - slot * H;
        ci_n = chunk_info(geom, slot);
        const int len = ci_n.len;
        const int64_t row0 = (int64_t)ci_n.t0 * H + h;
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + row0 * DK, len > 0 ? (len - 1) * rs_k + DK * Cfg::ES : 0);
#pragma unroll
        for (int j = 0; j < Cfg::NL; ++j) kv[j] = __builtin_amdgcn_raw_buffer_load_b128(rk, koff[j], 0, 0);
        if (w == 0) {   // wave 0 takes the gates: lane l holds token l's
            const int64_t gbytes = len > 0 ? ((int64_t)(len - 1) * H + 1) * 4 : 0;
            const uint32_t goff = l < C ? (uint32_t)(l * H * 4) : kOutOfRange;
            be_n = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(beta + row0, gbytes),
                                                                                  goff, 0, 0));
            la_n = log_alpha ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                   make_rsrc(log_alpha + row0, gbytes), goff, 0, 0))
                             : 0.f;
        }
    };

    int u = blockIdx.x;
    if (u < units) fetch(u);
    for (; u < units; u += gridDim.x) {
        const ChunkInfo ci = ci_n;
        const int slot = u / H, h = u - slot * H;
        const int64_t unit = (int64_t)slot * H + h;
        // this unit's keys into LDS and its gates into registers, then start the next unit's loads
#pragma unroll
        for (int j = 0; j < Cfg::NL; ++j)
            if (kdst[j] >= 0) *reinterpret_cast<u32x4*>(smem + Cfg::OFF_K + kdst[j]) = kv[j];
        float la = la_n;
        const float be = be_n;
        if (u + (int)gridDim.x < units) fetch(u + gridDim.x);
        if (ci.len <= 0) continue;   // unused packed-batch slot (uniform)

        // gates: inclusive prefix sum of log alpha inside the chunk (wave 0)
        if (w == 0) {
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float y = __shfl_up(la, off, 64);
                if (l >= off) la += y;
            }
            const float glast = __shfl(la, C - 1, 64);
            if (l < C) {
                sg[l] = la;
                sb[l] = be;
                float* gout = g_ws + unit * 3 * C;
                gout[l] = la;                            // g_i
                gout[C + l] = __expf(la);                // gamma_i = exp(g_i)
                gout[2 * C + l] = __expf(glast - la);    // gamma_n / gamma_i
            }
        }
        __syncthreads();

        // A = strict_lower(diag(beta) (K K^T o Gamma)) on MFMA: lower tile t = w, w + 4, ...
        for (int t = w; t < Cfg::NT; t += kThreads / 64) {
            const int ti = t >= 6 ? 3 : t >= 3 ? 2 : t >= 1 ? 1 : 0;
            const int tj = t - ti * (ti + 1) / 2;
            f32x4 acc = zero4();
#pragma unroll
            for (int kk = 0; kk < DK; kk += M::KS) {
                const int c = kk + (l >> 4) * M::KPL;
                typename M::frag a, b;
                if constexpr (M::KPL == 8) {
                    a = *reinterpret_cast<const bf16x8*>(sK + kidx(ti * 16 + (l & 15), c));
                    b = *reinterpret_cast<const bf16x8*>(sK + kidx(tj * 16 + (l & 15), c));
                } else {
                    a = sK[kidx(ti * 16 + (l & 15), c)];
                    b = sK[kidx(tj * 16 + (l & 15), c)];
                }
                acc = M::mma(a, b, acc);
            }
            const int j = tj * 16 + (l & 15), i0 = ti * 16 + 4 * (l >> 4);
            const float gj = sg[j];
            const float4 gi = *reinterpret_cast<const float4*>(sg + i0);
            const float4 bi = *reinterpret_cast<const float4*>(sb + i0);
            sA[(i0 + 0) * Cfg::LDA + j] = (j < i0 + 0) ? bi.x * acc[0] * __expf(gi.x - gj) : 0.f;
            sA[(i0 + 1) * Cfg::LDA + j] = (j < i0 + 1) ? bi.y * acc[1] * __expf(gi.y - gj) : 0.f;
            sA[(i0 + 2) * Cfg::LDA + j] = (j < i0 + 2) ? bi.z * acc[2] * __expf(gi.z - gj) : 0.f;
            sA[(i0 + 3) * Cfg::LDA + j] = (j < i0 + 3) ? bi.w * acc[3] * __expf(gi.w - gj) : 0.f;
        }
        __syncthreads();

        // T = (I + A)^-1, blocked by 16 rows.  Diagonal blocks by forward
        // substitution (wave 0, lane = 16 b + column); then, one block diagonal
        // at a time, T_ij = -T_ii (sum_{j<=m<i} A_im T_mj) on fp32 MFMA.
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
            if (w < Cfg::NB - d) {
                // R = sum_m A_im T_mj (accumulator layout), then T_ij = -T_ii R with R
                // as the B operand straight from the accumulators
                f32x4 acc = zero4();
                for (int kk = 16 * j; kk < 16 * i; kk += MF::KS)
                    acc = MF::mma(frag_kc(sA, Cfg::LDA, 16 * i, kk), frag_ks(sT, Cfg::LDA, kk, 16 * j), acc);
                const f32x4 tii = *reinterpret_cast<const f32x4*>(sT + (16 * i + (l & 15)) * Cfg::LDA + 16 * i +
                                                                   4 * (l >> 4));
                const f32x4 tij = mma16_f32(tii, acc, zero4());
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    sT[(16 * i + 4 * (l >> 4) + r) * Cfg::LDA + 16 * j + (l & 15)] = -tij[r];
            }
            __syncthreads();
        }

        // Tb = T diag(beta), zero above the diagonal; 16-byte stores.  fp32 rows are
        // plain; a bf16 row stores each 32-column group as the 4-column runs
        // (0-3, 16-19, 4-7, 20-23, 8-11, 24-27, 12-15, 28-31), so that the 16 bytes at
        // group offset 8g are the operand of a 16-deep block pair (4g .. 4g+3 of both).
        // Blocks above the diagonal block are not computed (masked); inside a
        // diagonal block the substitution leaves exact zeros above the diagonal.
        static_assert(sizeof(T) == 4 || C % 32 == 0, "bf16 Tb groups of 32 columns");
        constexpr int EV = Cfg::EV, VPR = C / EV;
        T* out = Tb_ws + unit * C * C;
        for (int idx = tid; idx < C * VPR; idx += kThreads) {
            const int i = idx / VPR, c0 = (idx - i * VPR) * EV;
            if constexpr (sizeof(T) == 4) {
                const bool keep = (c0 >> 4) <= (i >> 4);
                const f32x4 t4 = *reinterpret_cast<const f32x4*>(sT + i * Cfg::LDA + c0);
                const float4 b4 = *reinterpret_cast<const float4*>(sb + c0);
                const f32x4 o = keep ? f32x4{t4[0] * b4.x, t4[1] * b4.y, t4[2] * b4.z, t4[3] * b4.w} : zero4();
                *reinterpret_cast<f32x4*>(out + i * C + c0) = o;
            } else {
                const int lc = (c0 & ~31) + ((c0 & 31) >> 1);   // logical columns lc .. lc+3, lc+16 .. lc+19
                const bool keep0 = (lc >> 4) <= (i >> 4), keep1 = ((lc + 16) >> 4) <= (i >> 4);
                const f32x4 t0 = *reinterpret_cast<const f32x4*>(sT + i * Cfg::LDA + lc);
                const f32x4 t1 = *reinterpret_cast<const f32x4*>(sT + i * Cfg::LDA + lc + 16);
                const float4 b0 = *reinterpret_cast<const float4*>(sb + lc);
                const float4 b1 = *reinterpret_cast<const float4*>(sb + lc + 16);
                bf16x8 o;
                o[0] = (bf16)(keep0 ? t0[0] * b0.x : 0.f);
                o[1] = (bf16)(keep0 ? t0[1] * b0.y : 0.f);
                o[2] = (bf16)(keep0 ? t0[2] * b0.z : 0.f);
                o[3] = (bf16)(keep0 ? t0[3] * b0.w : 0.f);
                o[4] = (bf16)(keep1 ? t1[0] * b1.x : 0.f);
                o[5] = (bf16)(keep1 ? t1[1] * b1.y : 0.f);
                o[6] = (bf16)(keep1 ? t1[2] * b1.z : 0.f);
                o[7] = (bf16)(keep1 ? t1[3] * b1.w : 0.f);
                *reinterpret_cast<bf16x8*>(out + i * C + c0) = o;
            }
        }
        __syncthreads();   // the next unit's keys overwrite T
    }
}

}  // namespace gdn
