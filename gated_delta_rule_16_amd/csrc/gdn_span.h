// gdn_span.h -- second level of the split scan: chains the span maps of each
// sequence.
//
// Over a span of chunks the state map of the chunked forward is affine and the
// same for every row of S: S_out = S_in M + b, M (Dk x Dk), b (Dv x Dk).  This
// follows from the chunk update (Qiita article on the Linear Attention lineage,
// section "Gated-DeltaNet": S_i = gamma_i S_0 (I - W K^T) + sum (gamma_i /
// gamma_s) u_s k_s^T is affine in S_0, and section "Chunk Computation": each
// chunk starts from the previous chunk's last state).  The first pass of the
// split scan forms (M, b) of every span (the scan run with identity rows); this
// kernel walks the spans of a sequence in order,
//     S_in(0) = S0,   S_in(p + 1) = S_in(p) M_p + b_p,   S_T = S_in(P),
// writing each span's start state for the last pass, all in fp32.
//
// A workgroup owns 4 rows of one (sequence, head) state, so that short
// batches still spread over the CUs; M_{p+1} is loaded into registers while
// the product with M_p runs from LDS.
#pragma once

#include "gdn_device.h"

namespace gdn {

template <int DK, int DV>
struct SpanCfg {
    static constexpr int ROWS = 4;                     // state rows per workgroup
    static constexpr int THREADS = 256;
    static constexpr int TPR = THREADS / ROWS;         // threads per row
    static constexpr int CPT = DK / TPR;               // columns per thread
    static constexpr int LM = DK + 4;                  // M row pitch (floats)
    static constexpr int NM4 = DK * DK / 4 / THREADS;  // float4 pieces of M per thread
    static constexpr size_t SMEM = (size_t)(DK * LM + ROWS * DK) * 4;
    static_assert(DV % ROWS == 0 && DK % TPR == 0 && CPT <= 4 && (DK * DK / 4) % THREADS == 0,
                  "tile shapes");
};

// maps: [N * P][H][DK + DV][DK] (rows 0 .. DK-1: M_p, rows DK .. DK+DV-1: b_p);
// S0 (nullable, zeros) and S_T (nullable): [N][H][DV][DK]; S_in: [N * P][H][DV][DK].
// Grid (DV / 4, H, N); S_T may alias S0 (each workgroup reads its rows of S0
// before it writes the same rows of S_T).
template <int DK, int DV>
__global__ __launch_bounds__(256, 2) void gdn_span_chain_kernel(const float* __restrict__ maps,
                                                             const float* S0, int P, int H,
                                                             float* __restrict__ S_in, float* S_T) {
    using Cfg = SpanCfg<DK, DV>;
    constexpr int CPT = Cfg::CPT, LM = Cfg::LM, NM4 = Cfg::NM4;
    extern __shared__ __align__(16) unsigned char smem[];
    float* sM = reinterpret_cast<float*>(smem);       // [DK][LM]
    float* sS = sM + DK * LM;                          // [ROWS][DK]
    const int tid = (int)threadIdx.x;
    const int r = tid / Cfg::TPR, c0 = (tid % Cfg::TPR) * CPT;
    const int row = (int)blockIdx.x * Cfg::ROWS + r, h = (int)blockIdx.y, n = (int)blockIdx.z;
    const int64_t srow = (((int64_t)n * H + h) * DV + row) * DK + c0;
    const int64_t mstride = (int64_t)H * (DK + DV) * DK;                 // between spans
    const float* m0 = maps + ((int64_t)n * P * H + h) * (int64_t)(DK + DV) * DK;   // span 0
    float s[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) s[j] = S0 ? S0[srow + j] : 0.f;
    // M of the next span in registers: piece i of this thread is float4 number
    // tid + i THREADS of the row-major DK x DK block
    float4 mr[NM4];
#pragma unroll
    for (int i = 0; i < NM4; ++i) mr[i] = P > 0 ? reinterpret_cast<const float4*>(m0)[tid + i * Cfg::THREADS] : float4{0.f, 0.f, 0.f, 0.f};
    for (int p = 0; p < P; ++p) {
        const float* mp = m0 + p * mstride;
        float* sin = S_in + ((((int64_t)n * P + p) * H + h) * DV + row) * (int64_t)DK + c0;
        const float* bp = mp + (int64_t)(DK + row) * DK + c0;
        float acc[CPT];
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            sin[j] = s[j];
            sS[r * DK + c0 + j] = s[j];
            acc[j] = bp[j];
        }
#pragma unroll
        for (int i = 0; i < NM4; ++i) {
            const int x = tid + i * Cfg::THREADS;
            *reinterpret_cast<float4*>(sM + (x / (DK / 4)) * LM + (x % (DK / 4)) * 4) = mr[i];
        }
        __syncthreads();
        {   // M of the next span lands while this product runs (past the end: this span's again)
            const float* mn = p + 1 < P ? mp + mstride : mp;
#pragma unroll
            for (int i = 0; i < NM4; ++i)
                mr[i] = reinterpret_cast<const float4*>(mn)[tid + i * Cfg::THREADS];
        }
        // S_in(p + 1) row = S_in(p) row  M_p + b_p row
#pragma unroll 8
        for (int d = 0; d < DK; ++d) {
            const float sv = sS[r * DK + d];
#pragma unroll
            for (int j = 0; j < CPT; ++j) acc[j] += sv * sM[d * LM + c0 + j];
        }
#pragma unroll
        for (int j = 0; j < CPT; ++j) s[j] = acc[j];
        __syncthreads();   // before the next span overwrites sM and sS
    }
    if (S_T) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) S_T[srow + j] = s[j];
    }
}

}  // namespace gdn
