// gdn_output.h -- chunk output kernel (independent across chunks).
//
// For one chunk of one head, a DVO-wide slice of the outputs (row form):
//   O = diag(gamma) Q h^T + ((Q K^T) o Gamma o M) V'
// with h the state at the chunk start, V' the corrected prediction errors of
// the scan, gamma_i = exp(g_i), Gamma_ij = exp(g_i - g_j) and M the causal mask
// with its diagonal (o_t reads the state after token t's own write).
// Source: the Qiita article on the Linear Attention lineage, section
// "Gated-DeltaNet": H = S0 (Q - W (M^T o K^T Q)) D_gamma + U (Gamma o K^T Q),
// restricted to one chunk and regrouped as S0 Q D_gamma + (U - W S0^T ...)
// terms; section "Chunk Computation": each chunk reads the previous chunk's
// last state as its S0.  The mask includes the diagonal (causal mask M of
// the "Causal attention" section; the read h_i = S_i q_i).
#pragma once

#include "gdn_device.h"

namespace gdn {

template <typename T, int DK, int DV, int C, int DVO>
struct OutCfg {
    static constexpr int PAD = 16 / sizeof(T);
    static constexpr int LDK = DK + PAD;
    static constexpr int LDC = C + PAD;
    static constexpr size_t OFF_Q = 0;
    static constexpr size_t OFF_K = OFF_Q + sizeof(T) * C * LDK;
    static constexpr size_t OFF_H = OFF_K + sizeof(T) * C * LDK;
    static constexpr size_t OFF_VP = OFF_H + sizeof(T) * DVO * LDK;
    static constexpr size_t OFF_P = OFF_VP + sizeof(T) * DVO * LDC;
    static constexpr size_t OFF_G = OFF_P + sizeof(T) * C * LDC;
    static constexpr size_t SMEM = OFF_G + sizeof(float) * C;
    static_assert(DV % DVO == 0 && DVO % 16 == 0, "output slice must be whole 16-column tiles");
};

template <typename T, int DK, int DV, int C, int DVO>
__global__ __launch_bounds__(kThreads) void gdn_output_kernel(
    const T* __restrict__ q, const T* __restrict__ k, SeqGeom geom, int H,
    const float* __restrict__ g_ws, const T* __restrict__ Vp_ws, const T* __restrict__ h_ws,
    T* __restrict__ O) {
    using Cfg = OutCfg<T, DK, DV, C, DVO>;
    using M = Mfma<T>;
    extern __shared__ __align__(16) unsigned char smem[];
    T* sQ = reinterpret_cast<T*>(smem + Cfg::OFF_Q);
    T* sK = reinterpret_cast<T*>(smem + Cfg::OFF_K);
    T* sH = reinterpret_cast<T*>(smem + Cfg::OFF_H);
    T* sVp = reinterpret_cast<T*>(smem + Cfg::OFF_VP);
    T* sP = reinterpret_cast<T*>(smem + Cfg::OFF_P);
    float* sg = reinterpret_cast<float*>(smem + Cfg::OFF_G);

    const int slot = blockIdx.x, h = blockIdx.y, v0 = blockIdx.z * DVO;
    const ChunkInfo ci = chunk_info(geom, slot);
    if (ci.len <= 0) return;
    const int l = lane_id(), w = wave_id();
    const int n = l & 15, g4 = 4 * (l >> 4);
    const int64_t unit = (int64_t)slot * H + h;

    stage_tokens<T, DK>(sQ, Cfg::LDK, q, ci.t0, ci.len, C, H, h);
    stage_tokens<T, DK>(sK, Cfg::LDK, k, ci.t0, ci.len, C, H, h);
    stage_dense<T, DK>(sH, Cfg::LDK, h_ws + (unit * DV + v0) * DK, DK, DVO);
    stage_dense<T, C>(sVp, Cfg::LDC, Vp_ws + (unit * DV + v0) * C, C, DVO);
    if (threadIdx.x < C) sg[threadIdx.x] = g_ws[unit * C + threadIdx.x];
    __syncthreads();

    // P = (Q K^T) o Gamma o M, lower tiles on MFMA, upper tiles zero
    constexpr int NT = C / 16;
    for (int t = w; t < NT * NT; t += 4) {
        const int ti = t / NT, tj = t - ti * NT;
        const int j = tj * 16 + n;
        if (tj > ti) {
#pragma unroll
            for (int r = 0; r < 4; ++r) sP[(ti * 16 + g4 + r) * Cfg::LDC + j] = from_f32<T>(0.f);
            continue;
        }
        f32x4 acc = zero4();
#pragma unroll
        for (int kk = 0; kk < DK; kk += M::KS)
            acc = M::mma(frag_kc(sQ, Cfg::LDK, ti * 16, kk), frag_kc(sK, Cfg::LDK, tj * 16, kk), acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = ti * 16 + g4 + r;
            sP[i * Cfg::LDC + j] = from_f32<T>((j <= i) ? acc[r] * __expf(sg[i] - sg[j]) : 0.f);
        }
    }
    __syncthreads();

    // O = diag(gamma) Q h^T + P V'
    constexpr int NVB = DVO / 16;
    for (int t = w; t < NT * NVB; t += 4) {
        const int cb = t / NVB, vb = t - cb * NVB;
        f32x4 acc = zero4();
#pragma unroll
        for (int kk = 0; kk < DK; kk += M::KS)
            acc = M::mma(frag_kc(sQ, Cfg::LDK, cb * 16, kk), frag_kc(sH, Cfg::LDK, vb * 16, kk), acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] *= __expf(sg[cb * 16 + g4 + r]);
        const int kend = ((cb + 1) * 16 + M::KS - 1) / M::KS * M::KS;
        for (int kk = 0; kk < kend; kk += M::KS)
            acc = M::mma(frag_kc(sP, Cfg::LDC, cb * 16, kk), frag_kc(sVp, Cfg::LDC, vb * 16, kk), acc);
        const int vv = v0 + vb * 16 + n;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int c = cb * 16 + g4 + r;
            if (c < ci.len) O[((int64_t)(ci.t0 + c) * H + h) * DV + vv] = from_f32<T>(acc[r]);
        }
    }
}

}  // namespace gdn
