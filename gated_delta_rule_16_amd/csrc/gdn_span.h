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
// fp32 inputs (gdn_span_chain_kernel): a workgroup owns 4 rows of one
// (sequence, head) state, so that short batches still spread over the CUs;
// M_{p+1} is loaded into registers while the product with M_p runs from LDS,
// on fp32 FMAs.  bf16 inputs (gdn_span_chain_mfma_kernel, below): 16 rows per
// workgroup, the product on bf16 MFMAs with split operands.
//
// Both grids put the head first (H, row blocks, sequences): workgroups go to
// the 8 XCDs round-robin by linear id, so the row blocks of one head, H ids
// apart, share an XCD when H is a multiple of 8 (two XCDs for H = 4), and its
// L2 fetches each span's map once for all of them.
#pragma once

#include "gdn_ops.h"

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
// Grid (H, DV / 4, N); S_T may alias S0 (each workgroup reads its rows of S0
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
    const int row = (int)blockIdx.y * Cfg::ROWS + r, h = (int)blockIdx.x, n = (int)blockIdx.z;
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

// The same chain on MFMA, for bf16 inputs (whose tolerance leaves room for
// products of split operands): S_in(p + 1)^T = M_p^T S_in(p)^T + b_p^T, one
// workgroup per 16 state rows of one (sequence, head), so that each M is read
// by DV / 16 workgroups instead of DV / 4.  Per span, wave w forms output tile
// t = w (columns 16 t .. 16 t + 15 of the 16 rows) with 16x16x16 bf16 MFMAs
// over the DK / 16 blocks of d:
//   A (lane (g, n)): M^T[16 t + n][16 kt + 4 g + r] = M[16 kt + 4 g + r][16 t + n]
//   B (lane (g, n)): S^T[16 kt + 4 g + r][n], the accumulator layout of the
//   previous span's tile kt (all waves' tiles pass through LDS),
// each operand split as x = hi + lo (hi = bf16(x), lo = bf16(x - hi)) and the
// product taken as hi hi + hi lo + lo hi, in three separate fp32 accumulation
// chains per tile (about 2^-16 of relative error per product, fp32 sums).
// Each wave loads its share of M_{p+3} and its lanes' piece of b_{p+3} into
// one of two register sets at the end of span p, two spans before they are
// needed, and writes the other set (M_{p+1}) to the free one of two LDS
// buffers after the span's products; one barrier per span.
template <int DK, int DV>
struct SpanMfmaCfg {
    static constexpr int ROWS = 16;
    static constexpr int NT = DK / 16;             // 16-column tiles of a state row block
    static constexpr int WAVES = NT, THREADS = WAVES * 64;   // one output tile per wave
    static constexpr int MB = DK * DK * 4;         // bytes of one M (fp32)
    static constexpr int NLD = MB / 1024 / WAVES;  // 16-byte loads per lane per span
    static constexpr int SXB = NT * 1024;          // one exchange buffer of S^T tiles
    static constexpr size_t OFF_SX = 2 * (size_t)MB;
    static constexpr size_t OFF_B = OFF_SX + 2 * (size_t)SXB;   // b_p, 16 bytes per lane
    static constexpr size_t SMEM = OFF_B + 2 * (size_t)THREADS * 16;
    static_assert(DK % 64 == 0 && (MB / 1024) % WAVES == 0 && DV % ROWS == 0 && THREADS <= 1024, "tile shapes");
    static_assert(SMEM <= 160 * 1024, "LDS of one CU");
};

// LDS image of M (row-major, DK floats per row): 16-byte chunk j of row d sits
// at chunk j ^ (4 ((d / 4) mod 4)), so that the 64 lanes of an A read (16
// columns of four rows d = 4 g + r) fall in 64 different banks
__device__ __forceinline__ int span_mchunk(int d, int j) { return j ^ (((d >> 2) & 3) << 2); }

// maps, S0, S_in, S_T as for gdn_span_chain_kernel.  Grid (H, DV / 16, N).
template <int DK, int DV>
__global__ __launch_bounds__((SpanMfmaCfg<DK, DV>::THREADS)) void gdn_span_chain_mfma_kernel(
    const float* __restrict__ maps, const float* S0, int P, int H, float* __restrict__ S_in, float* S_T) {
    using Cfg = SpanMfmaCfg<DK, DV>;
    using KO = K16<bf16>;
    typedef typename KO::op Op;
    constexpr int NT = Cfg::NT, NLD = Cfg::NLD;
    extern __shared__ __align__(16) unsigned char smem[];
    const int l = lane_id(), w = wave_id();
    const int n = l & 15, g = l >> 4;
    const int t = w;   // this wave's output tile
    const int row0 = (int)blockIdx.y * Cfg::ROWS, h = (int)blockIdx.x, sq = (int)blockIdx.z;
    const int64_t mstride = (int64_t)H * (DK + DV) * DK;                      // between spans
    const float* m0 = maps + ((int64_t)sq * P * H + h) * (int64_t)(DK + DV) * DK;   // span 0
    // this lane's piece of tile t (row row0 + n, columns 16 t + 4 g .. + 3)
    // inside a [DV][DK] state
    const int64_t soff = (int64_t)(row0 + n) * DK + 16 * t + 4 * g;
    const int64_t st_base = (((int64_t)sq * H + h) * DV) * DK;
    auto sin_at = [&](int p) __attribute__((always_inline)) {
        return reinterpret_cast<f32x4*>(S_in + ((((int64_t)sq * P + p) * H + h) * DV) * DK + soff);
    };

    // M in registers: piece i of the set is the 16-byte chunk q = (w NLD + i) 64 + l
    // of M; piece NLD is this lane's piece of b (the first accumulator of its
    // tile).  One set, loaded a span ahead and used only to fill LDS (b too):
    // with two sets, or with b kept in a register, the compiler moved the
    // newest loads between registers at the loop head, and those moves waited
    // for loads issued just before the barrier.
    f32x4 mr[NLD + 1];
    auto m_load = [&](f32x4* mr, int p) __attribute__((always_inline)) {
        const float* mp = m0 + p * mstride;
        mr[NLD] = *reinterpret_cast<const f32x4*>(mp + (int64_t)DK * DK + soff);
#pragma unroll
        for (int i = 0; i < NLD; ++i) mr[i] = reinterpret_cast<const f32x4*>(mp)[(w * NLD + i) * 64 + l];
    };
    auto m_store = [&](const f32x4* mr, int buf) __attribute__((always_inline)) {
        float* sm = reinterpret_cast<float*>(smem + (size_t)buf * Cfg::MB);
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int q = (w * NLD + i) * 64 + l, d = q / (DK / 4), j = q % (DK / 4);
            *reinterpret_cast<f32x4*>(sm + d * DK + 4 * span_mchunk(d, j)) = mr[i];
        }
        reinterpret_cast<f32x4*>(smem + Cfg::OFF_B + (size_t)buf * Cfg::THREADS * 16)[w * 64 + l] = mr[NLD];
    };
    auto sx = [&](int buf, int tt) __attribute__((always_inline)) {
        return reinterpret_cast<f32x4*>(smem + Cfg::OFF_SX + (size_t)buf * Cfg::SXB + tt * 1024) + l;
    };
    auto split = [&](f32x4 x, Op& hi, Op& lo) __attribute__((always_inline)) {
        hi = KO::tile(x);
        const bf16x4 hb = __builtin_bit_cast(bf16x4, hi);
        lo = KO::tile(f32x4{x[0] - (float)hb[0], x[1] - (float)hb[1], x[2] - (float)hb[2], x[3] - (float)hb[3]});
    };

    // S_in(0) = S0 (zeros if NULL): this wave's tile to the exchange buffer and,
    // when there is a span, to the first span's start state
    {
        const f32x4 s = S0 ? *reinterpret_cast<const f32x4*>(S0 + st_base + soff) : zero4();
        *sx(0, t) = s;
        if (P > 0) *sin_at(0) = s;
        else if (S_T) *reinterpret_cast<f32x4*>(S_T + st_base + soff) = s;
    }
    if (P > 0) {
        m_load(mr, 0);
        m_store(mr, 0);
        m_load(mr, min(1, P - 1));
    }
    __syncthreads();

    // span p from LDS buffer p & 1 (the products of this wave's tile)
    auto product = [&](int p) __attribute__((always_inline)) {
        const float* sm = reinterpret_cast<const float*>(smem + (size_t)(p & 1) * Cfg::MB);
        // b_p row row0 + n, columns 16 t + 4 g .. + 3 starts the first chain
        f32x4 acc0 = reinterpret_cast<const f32x4*>(smem + Cfg::OFF_B + (size_t)(p & 1) * Cfg::THREADS * 16)[w * 64 + l];
        f32x4 acc1 = zero4(), acc2 = zero4();
        // the operands of step kt + 1 are requested before the products of
        // step kt, so that their LDS latency overlaps those
        f32x4 sv[2], av[2];
        auto fetch = [&](int kt, int s) __attribute__((always_inline)) {
            sv[s] = *sx(p & 1, kt);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int d = 16 * kt + 4 * g + r, c = 16 * t + n;
                av[s][r] = sm[d * DK + 4 * span_mchunk(d, c >> 2) + (c & 3)];
            }
        };
        fetch(0, 0);
#pragma unroll
        for (int kt = 0; kt < NT; ++kt) {
            if (kt + 1 < NT) fetch(kt + 1, (kt + 1) & 1);
            Op bh, bl, ah, al;
            split(sv[kt & 1], bh, bl);
            split(av[kt & 1], ah, al);
            acc0 = KO::mma1(ah, bh, acc0);
            acc1 = KO::mma1(ah, bl, acc1);
            acc2 = KO::mma1(al, bh, acc2);
        }
        return acc0 + (acc1 + acc2);
    };
    // a span with a successor: S_in(p + 1) out, M_{p+1} from the registers to
    // the other LDS buffer (its M_{p-1} was read before the last barrier), the
    // next map into the registers (past the end: the last one again)
    auto mid = [&](int p) __attribute__((always_inline)) {
        const f32x4 s = product(p);
        *sx((p + 1) & 1, t) = s;
        *sin_at(p + 1) = s;
        m_store(mr, (p + 1) & 1);
        m_load(mr, min(p + 2, P - 1));
        __syncthreads();
    };
    // the last span: S_T
    auto last = [&](int p) __attribute__((always_inline)) {
        const f32x4 s = product(p);
        if (S_T) *reinterpret_cast<f32x4*>(S_T + st_base + soff) = s;
    };
    for (int p = 0; p + 1 < P; ++p) mid(p);
    if (P > 0) last(P - 1);
}

}  // namespace gdn
