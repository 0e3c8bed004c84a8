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
// Work split: one wave prepares one unit (chunk slot, head) at a time, with no
// synchronisation beyond the wave.  Waves are persistent: wave w of workgroup
// b walks units b*4 + w, then that plus 4 gridDim, ...  At least two waves
// share each SIMD (the register budget is held to half the file), so that one
// computes while another waits for its unit's keys -- this measured faster
// than one wave per SIMD with the next unit's keys prefetched into registers.
// Per unit:
//  - the keys arrive as MFMA row fragments (lane (g, n): row 16b + n, 16 bytes
//    at contraction offset 16 g of each step), so K K^T needs no LDS;
//  - tile (i, m) of K K^T is formed as K_m K_i^T, whose accumulator layout is
//    the A operand layout of tile (i, m) -- lane (g, n) holds row 16i + n,
//    columns 16m + 4g .. + 3 -- and gated and masked there into A;
//  - each diagonal 16 x 16 block of T is found by forward substitution in
//    registers (lane (b, c): column c of block b) from the block's columns of
//    A in LDS; the blocks below the diagonal follow one block diagonal at a
//    time, T_ij = -T_ii sum_{j <= m < i} A_im T_mj, on MFMA (fp32, or bf16
//    products for bf16 inputs) straight from registers (the diagonal blocks
//    of T pass through LDS once, for the two
//    operand layouts they serve in), each block also formed in row layout as
//    T_ij^T = -R^T T_ii^T;
//  - Tb = T diag(beta) leaves from that row layout as lane-linear 1 KB blocks
//    of MFMA operands, the blocks above the diagonal omitted (tb_block).
#pragma once

#include "gdn_device.h"

namespace gdn {

template <typename T, int DK, int C>
struct PrepCfg {
    static constexpr bool BF = sizeof(T) == 2;
    static constexpr int ES = sizeof(T), EV = 16 / ES;
    static constexpr int NB = C / 16;                      // 16-row blocks
    static constexpr int KS = Step<T>::KS, NKK = DK / KS;  // contraction steps over d
    static constexpr int WAVES = kThreads / 64;
    static constexpr int MIN_WAVES_SIMD = 2;               // register budget: 512 / this per wave
    // per-wave LDS (bytes): g, beta; the diagonal blocks of A and of T, both
    // column-major
    static constexpr int OFF_G = 0, OFF_B = 4 * C, OFF_AD = 8 * C;
    static constexpr int OFF_TD = OFF_AD + NB * 1024;
    static constexpr int WAVE_LDS = OFF_TD + NB * 1024;
    static constexpr size_t SMEM = (size_t)WAVES * WAVE_LDS;
    static_assert(C <= 64 && C % 16 == 0 && DK % KS == 0, "at most four 16-row blocks");
    static_assert(!BF || C % 32 == 0, "bf16 Tb in 32-column groups");
};

// Exchange point between lanes of one wave that pass values through LDS: the
// hardware keeps one wave's LDS accesses in order, so it is enough that the
// compiler does not move memory accesses across this point (no wait is
// issued, which leaves outstanding global loads and stores in flight)
__device__ __forceinline__ void wave_lds_sync() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
}

// c += A B over one 16-deep block with fp32 MFMA: lane (g, n) holds a = A[n][4g .. 4g+3]
// and b = B[4g .. 4g+3][n] (the 16x16 accumulator layout of B)
__device__ __forceinline__ f32x4 mma16_f32(f32x4 a, f32x4 b, f32x4 c) {
#pragma unroll
    for (int r = 0; r < 4; ++r) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[r], b[r], c, 0, 0, 0);
    return c;
}

// c += A B over one 16-deep block on bf16 products (operands rounded to bf16,
// fp32 accumulation), layouts as for mma16_f32
typedef short p16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ p16x4 to_bf16x4(f32x4 x) {
    const bf16x4 h = {(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
    return __builtin_bit_cast(p16x4, h);
}
__device__ __forceinline__ f32x4 mma16_bf16(p16x4 a, p16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

template <typename T, int DK, int C>
__global__ __launch_bounds__(kThreads, (PrepCfg<T, DK, C>::MIN_WAVES_SIMD)) void gdn_prep_kernel(
    const T* __restrict__ k, const float* __restrict__ log_alpha,
    const float* __restrict__ beta, SeqGeom geom, int H, int units,
    float* __restrict__ g_ws, T* __restrict__ Tb_ws) {
    using Cfg = PrepCfg<T, DK, C>;
    using St = Step<T>;
    using Frag = typename St::frag;
    constexpr int NB = Cfg::NB, NKK = Cfg::NKK, KS = Cfg::KS, ES = Cfg::ES;
    extern __shared__ __align__(16) unsigned char smem[];
    const int l = lane_id(), w = wave_id();
    const int n = l & 15, g = l >> 4;
    unsigned char* wl = smem + w * Cfg::WAVE_LDS;
    float* sg = reinterpret_cast<float*>(wl + Cfg::OFF_G);
    float* sb = reinterpret_cast<float*>(wl + Cfg::OFF_B);
    float* sAd = reinterpret_cast<float*>(wl + Cfg::OFF_AD);   // [b][col][row]
    float* sTd = reinterpret_cast<float*>(wl + Cfg::OFF_TD);   // [b][col][row]
    const int64_t rs_k = (int64_t)H * DK * ES;
    const int stride = (int)gridDim.x * Cfg::WAVES;

    // gates and keys of unit u into registers (rows past the chunk end read as
    // 0); the gates first, so that their prefix sum is done by the time the
    // keys have landed
    float la_n = 0.f, be_n = 0.f;
    ChunkInfo ci_n{};
    auto fetch = [&](Frag (*dst)[NKK], int u) __attribute__((always_inline)) {
        const int slot = u / H, h = u - slot * H;
        ci_n = chunk_info(geom, slot);
        const int len = ci_n.len;
        const int64_t row0 = (int64_t)ci_n.t0 * H + h;
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + row0 * DK, len > 0 ? (len - 1) * rs_k + DK * ES : 0);
        {
            const int64_t gbytes = len > 0 ? ((int64_t)(len - 1) * H + 1) * 4 : 0;
            const uint32_t goff = l < C ? (uint32_t)(l * H * 4) : kOutOfRange;
            be_n = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(beta + row0, gbytes), goff, 0, 0));
            la_n = log_alpha ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                   make_rsrc(log_alpha + row0, gbytes), goff, 0, 0))
                             : 0.f;
        }
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk)
                dst[b][kk] = __builtin_bit_cast(
                    Frag, __builtin_amdgcn_raw_buffer_load_b128(
                              rk, (uint32_t)((b * 16 + n) * rs_k) + kk * KS * ES + g * 16, 0, 0));
    };

    // block (ti, q) of a unit's Tb at out: this lane's 16 bytes
    typedef typename std::conditional<Cfg::BF, bf16x8, f32x4>::type HFrag;
    constexpr int NHQ = Cfg::BF ? NB / 2 : NB;
    auto tb_store = [&](T* out, int ti, int q, HFrag v) __attribute__((always_inline)) {
        *reinterpret_cast<HFrag*>(reinterpret_cast<unsigned char*>(out) + tb_block(ti, q, Cfg::BF) * 1024 + l * 16) = v;
    };

    // one unit: keys, gates and geometry by fetch, then the chain below
    auto process = [&](int u, Frag (*cur)[NKK]) __attribute__((always_inline)) {
        fetch(cur, u);
        const ChunkInfo ci = ci_n;
        float la = la_n;
        const float be = be_n;
        if (ci.len <= 0) return;   // unused packed-batch slot (uniform)
        const int slot = u / H, h = u - slot * H;
        const int64_t unit = (int64_t)slot * H + h;

        // gates: inclusive prefix sum of log alpha inside the chunk (lane = token)
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(la, off, 64);
            if (l >= off) la += y;
        }
        const float glast = __shfl(la, C - 1, 64);
        if (l < C) {
            sg[l] = la;
            sb[l] = be;
        }
        {
            // g_i, gamma_i = exp(g_i), gamma_n / gamma_i
            float* gout = g_ws + unit * 3 * C;
            const float g3[3] = {la, __expf(la), __expf(glast - la)};
            if (l < C) {
                gout[l] = g3[0];
                gout[C + l] = g3[1];
                gout[2 * C + l] = g3[2];
            }
        }
        wave_lds_sync();

        // A = strict_lower(diag(beta) (K K^T o Gamma)).  Tile (i, m), m < i, in A
        // operand layout: lane (g, n) holds A[16i + n][16m + 4g + r]; the product
        // K_m K_i^T puts exactly those entries of K K^T in the lane.  Diagonal
        // tiles in accumulator layout -- lane (g, n) holds A[16b + 4g + r][16b + n]
        // (K K^T is symmetric) -- go to LDS as the columns of the block.
        f32x4 A[NB][NB];
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int row = 16 * i + n;
            const float gr = sg[row], br = sb[row];
#pragma unroll
            for (int m = 0; m <= i; ++m) {
                f32x4 acc = zero4();
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) acc = St::mma(cur[m][kk], cur[i][kk], acc);
                const int c0 = 16 * m + 4 * g;
                const float4 gc = *reinterpret_cast<const float4*>(sg + c0);
                if (m < i) {
                    A[i][m][0] = br * acc[0] * __expf(gr - gc.x);
                    A[i][m][1] = br * acc[1] * __expf(gr - gc.y);
                    A[i][m][2] = br * acc[2] * __expf(gr - gc.z);
                    A[i][m][3] = br * acc[3] * __expf(gr - gc.w);
                } else {
                    // rows c0 + r, column row: A = beta_rows S exp(g_rows - g_col) below the diagonal
                    const float4 bc = *reinterpret_cast<const float4*>(sb + c0);
                    f32x4 d;
                    d[0] = c0 + 0 > row ? bc.x * acc[0] * __expf(gc.x - gr) : 0.f;
                    d[1] = c0 + 1 > row ? bc.y * acc[1] * __expf(gc.y - gr) : 0.f;
                    d[2] = c0 + 2 > row ? bc.z * acc[2] * __expf(gc.z - gr) : 0.f;
                    d[3] = c0 + 3 > row ? bc.w * acc[3] * __expf(gc.w - gr) : 0.f;
                    *reinterpret_cast<f32x4*>(sAd + i * 256 + n * 16 + 4 * g) = d;   // column n, rows 4g..
                }
            }
        }
        wave_lds_sync();

        // diagonal blocks of T = (I + A)^-1: lane (b, c) solves (I + A_bb) x = e_c
        // right-looking -- once x_j is known, it leaves the rows below -- so the
        // dependent chain is one FMA per row
        if (g < NB) {
            const float* ab = sAd + g * 256;   // column j of the block at ab + 16 j
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] = i == n ? 1.f : 0.f;
            // the rows below the diagonal of column j, requested two columns ahead
            float4 col[3][4];
            auto ldcol = [&](int j) __attribute__((always_inline)) {
#pragma unroll
                for (int i4 = (j + 1) / 4; i4 < 4; ++i4)
                    col[j % 3][i4] = *reinterpret_cast<const float4*>(ab + j * 16 + 4 * i4);
            };
            ldcol(0);
            ldcol(1);
#pragma unroll
            for (int j = 0; j < 15; ++j) {
                if (j + 2 < 15) ldcol(j + 2);
                const float xj = x[j];
#pragma unroll
                for (int i4 = (j + 1) / 4; i4 < 4; ++i4) {
                    const float4 a4 = col[j % 3][i4];
                    if (4 * i4 + 0 > j) x[4 * i4 + 0] -= a4.x * xj;
                    if (4 * i4 + 1 > j) x[4 * i4 + 1] -= a4.y * xj;
                    if (4 * i4 + 2 > j) x[4 * i4 + 2] -= a4.z * xj;
                    if (4 * i4 + 3 > j) x[4 * i4 + 3] -= a4.w * xj;
                }
            }
            float* tc = sTd + g * 256 + n * 16;
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4)
                *reinterpret_cast<f32x4*>(tc + 4 * i4) = f32x4{x[4 * i4], x[4 * i4 + 1], x[4 * i4 + 2], x[4 * i4 + 3]};
        }
        wave_lds_sync();   // the columns of T, and the columns of A read above, are settled
        // the diagonal blocks of T as B operands (T_bb[4g + r][n]) and as A
        // operands (T_bb[n][4g + r], also the row layout of the output)
        f32x4 Tb_op[NB], Ta_op[NB];
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            Tb_op[b] = *reinterpret_cast<const f32x4*>(sTd + b * 256 + n * 16 + 4 * g);
#pragma unroll
            for (int r = 0; r < 4; ++r) Ta_op[b][r] = sTd[b * 256 + (4 * g + r) * 16 + n];
        }
        // blocks below the diagonal, one block diagonal at a time.  To (bf16: Tos):
        // accumulator layout (T[16i + 4g + r][16j + n]) for the blocks later levels
        // take as B operands; Tr: row layout (T[16i + n][16j + 4g + r]), from
        // T_ij^T = -R^T T_ii^T, for the output
        // (bf16 inputs: on bf16 products -- Tb leaves rounded to bf16 anyway, and
        // the outputs measured the same to three digits as with products of
        // fp32 accuracy)
        f32x4 To[NB][NB], Tr[NB][NB];
        if constexpr (Cfg::BF) {
            p16x4 As[NB][NB], Tbs[NB], Tas[NB], Tos[NB][NB];
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                Tbs[b] = to_bf16x4(Tb_op[b]);
                Tas[b] = to_bf16x4(Ta_op[b]);
#pragma unroll
                for (int m = 0; m < b; ++m) As[b][m] = to_bf16x4(A[b][m]);
            }
#pragma unroll
            for (int d = 1; d < NB; ++d)
#pragma unroll
                for (int j = 0; j + d < NB; ++j) {
                    const int i = j + d;
                    f32x4 R = zero4();
#pragma unroll
                    for (int m = j; m < i; ++m) R = mma16_bf16(As[i][m], m == j ? Tbs[j] : Tos[m][j], R);
                    const p16x4 Rb = to_bf16x4(R);
                    if (i < NB - 1) Tos[i][j] = to_bf16x4(-mma16_bf16(Tas[i], Rb, zero4()));
                    Tr[i][j] = -mma16_bf16(Rb, Tas[i], zero4());
                }
        } else {
#pragma unroll
            for (int d = 1; d < NB; ++d)
#pragma unroll
                for (int j = 0; j + d < NB; ++j) {
                    const int i = j + d;
                    f32x4 R = zero4();
#pragma unroll
                    for (int m = j; m < i; ++m) R = mma16_f32(A[i][m], m == j ? Tb_op[j] : To[m][j], R);
                    if (i < NB - 1) To[i][j] = -mma16_f32(Ta_op[i], R, zero4());
                    Tr[i][j] = -mma16_f32(R, Ta_op[i], zero4());
                }
        }

        // Tb = T diag(beta) straight from the row layout, in the block layout of
        // tb_block: lane (g, n) holds row 16 ti + n at columns 4g .. 4g+3 of each
        // 16-column tile (bf16: tiles 2q and 2q + 1 in one 16-byte piece).
        T* out = Tb_ws + unit * (tb_blocks(C, Cfg::BF) * 1024 / ES);
        auto trow = [&](int ti, int tj) __attribute__((always_inline)) {
            const f32x4 t = tj < ti ? Tr[ti][tj] : tj == ti ? Ta_op[ti] : zero4();
            const float4 b4 = *reinterpret_cast<const float4*>(sb + 16 * tj + 4 * g);
            return f32x4{t[0] * b4.x, t[1] * b4.y, t[2] * b4.z, t[3] * b4.w};
        };
#pragma unroll
        for (int ti = 0; ti < NB; ++ti) {
#pragma unroll
            for (int q = 0; q < NHQ; ++q) {
                if ((Cfg::BF ? 2 * q : q) > ti) continue;   // above the diagonal: not stored
                HFrag o;
                if constexpr (Cfg::BF) {
                    const f32x4 t0 = trow(ti, 2 * q), t1 = trow(ti, 2 * q + 1);
                    o = bf16x8{(bf16)t0[0], (bf16)t0[1], (bf16)t0[2], (bf16)t0[3],
                               (bf16)t1[0], (bf16)t1[1], (bf16)t1[2], (bf16)t1[3]};
                } else {
                    o = trow(ti, q);
                }
                tb_store(out, ti, q, o);
            }
        }
        wave_lds_sync();   // before the next unit overwrites what was read
    };

    Frag kf[NB][NKK];
    for (int u = blockIdx.x * Cfg::WAVES + w; u < units; u += stride) process(u, kf);
}

// Per-chunk gates of the no-erase rule, the only per-chunk preparation it
// needs (the chunk form of the Qiita article's "Chunk Computation" section,
// Mamba2 case, uses the in-chunk decays only): for every (chunk slot, head)
// unit, g_i = sum_{t<=i} log alpha_t, exp(g_i), exp(g_n - g_i) and beta_i, as
// four fp32 rows of C.  One wave per unit, lane = token; beta NULL means
// beta = 1; rows past the chunk end act as tokens with log alpha = 0, beta = 0.
template <int C>
__global__ __launch_bounds__(kThreads) void gdn_gates_kernel(const float* __restrict__ log_alpha,
                                                             const float* __restrict__ beta, SeqGeom geom,
                                                             int H, int units, float* __restrict__ g_ws) {
    static_assert(C <= 64, "one lane per token");
    const int l = lane_id();
    const int u = (int)blockIdx.x * (kThreads / 64) + wave_id();
    if (u >= units) return;
    const int slot = u / H, h = u - slot * H;
    const ChunkInfo ci = chunk_info(geom, slot);
    if (ci.len <= 0) return;   // unused packed-batch slot
    const bool in = l < ci.len;
    const int64_t x = ((int64_t)ci.t0 + (in ? l : 0)) * H + h;
    float g = in && log_alpha ? log_alpha[x] : 0.f;
    const float be = in ? (beta ? beta[x] : 1.f) : 0.f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(g, off, 64);
        if (l >= off) g += y;
    }
    const float glast = __shfl(g, C - 1, 64);
    if (l < C) {
        float* out = g_ws + (int64_t)u * gate_rows(kNoErase) * C;
        out[l] = g;
        out[C + l] = __expf(g);
        out[2 * C + l] = __expf(glast - g);
        out[3 * C + l] = be;
    }
}

}  // namespace gdn
