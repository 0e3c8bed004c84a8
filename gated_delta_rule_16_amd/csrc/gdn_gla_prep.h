// gdn_gla_prep.h -- per-chunk preparation of the per-channel (vector) gate rule
// (independent across chunks).
//
// The rule: S_t = S_{t-1} diag(alpha_t) + beta_t v_t k_t^T,  o_t = S_t q_t, with
// alpha_t in (0, 1]^Dk acting on the key channels of S = [Dv][Dk].  The pages
// name it without formulas (LinearAttention系列解读(六)：DeltaNet的Chunkwise
// Form推导, section 1: the vector-gated GLA's transition is a diagonal matrix
// that scales each state element on its own, by an amount fixed by the gate,
// so in the chunk form the scaling is split onto both sides of the mask).
// Unrolling the recurrence inside a chunk that starts from S, with
// b_i = sum_{t<=i} log alpha_t (one value per key channel):
//   o_i = S (q_i o e^{b_i}) + sum_{s<=i} beta_s v_s sum_d q_id k_sd e^{b_id - b_sd}
//   S  <- S diag(e^{b_n}) + sum_s beta_s v_s (k_s o e^{b_n - b_s})^T
// so in row form, with P_is = sum_d q_id k_sd e^{b_id - b_sd} (s <= i):
//   O = Q~ S^T + P~ V,   S^T <- diag(e^{b_n}) S^T + K^^T V,
//   Q~ = Q o e^b,  K^ = diag(beta) K o e^{b_n - b},  P~ = P diag(beta).
// This kernel forms Q~ and K^ (input dtype, token-major like q and k), P~ (the
// lower block triangle as MFMA operand blocks, the layout of the delta rule's
// Tb: tb_block) and e^{b_n} (fp32, Dk values) for each (chunk slot, head), one
// at a time per workgroup (persistent workgroups, the next unit's loads in
// flight while the current one's P~ is formed); the scan runs the same
// pipeline on them.
//
// Bounded exponents.  e^{b_id - b_sd} is formed as a product of factors that
// are each at most 1: for query block I (tokens 16I .. 16I+15) and key block
// J <= I (ending at token e_J = 16J + 15),
//   Q^_i = q_i o e^{b_i - b_16I} (<= |q_i|),  K~_s = k_s o e^{b_eJ - b_s} (<= |k_s|),
//   P_IJ = Q^_I (K~_J o c_IJ)^T,  c_IJ = e^{b_16I - b_eJ}
// where c_IJ <= 1 for J < I.  On the diagonal (J = I) c_II = e^{b_16I - b_eI} >= 1
// is the decay across the block; while it stays below e^64 on every channel
// the same product is used, else that block is formed term by term (exact for
// any gate, slow; only extreme gates take it).
// Whole-chunk fast path.  When every channel decays by less than e^64 over the
// whole chunk (b_n > -64), e^{b_id - b_sd} = e^{b_id} e^{-b_sd} with both
// factors between e^-64 and e^64, so P = Q~ K'^T with K' = K o e^{-b}: each
// tile is one MFMA chain over the operands as they are, with no per-tile
// scaling, and K^ = diag(beta) K' diag(e^{b_n}).  Chunks with a stronger decay
// on some channel take the blocked form above.
// Padding: rows past the chunk end act as tokens with q = k = 0, beta = 0,
// log alpha = 0.
#pragma once

#include "gdn_device.h"

namespace gdn {

template <typename T, int DK, int C>
struct GlaPrepCfg {
    static constexpr bool BF = sizeof(T) == 2;
    static constexpr int ES = sizeof(T), EV = 16 / ES;    // elements per 16 bytes
    static constexpr int NB = C / 16;                      // 16-token blocks
    static constexpr int KS = Step<T>::KS, NKK = DK / KS;  // contraction steps over d
    static constexpr int THREADS = 256, WAVES = THREADS / 64;
    static constexpr int NPAIR = NB * (NB + 1) / 2;        // (I, J <= I) block pairs
    static constexpr int NBLK = tb_blocks(C, BF);          // P~ operand blocks
    static constexpr int PARTS = THREADS / DK;             // cumsum: token ranges per channel
    static constexpr int TPP = C / PARTS;                  // tokens per range
    static constexpr float kMaxDiagLog = 64.f;             // diagonal fast path: c_II < e^64
    static constexpr float kMaxChunkLog = 64.f;            // whole-chunk fast path: -b_n < 64
    static constexpr int FLAG_SLOW_CHUNK = 15;             // sflag slot: the chunk takes the blocked form
    // LDS: b [C][LB] fp32; Q^, K~ [C][DK] in T; c_IJ [NPAIR][DK], e^{b_16I} and
    // e^{b_n - b_eI} [NB][DK] fp32; beta [C]; per-block slow-path flags
    static constexpr int LB = DK + 4;                      // b row pitch (floats)
    static constexpr int LQ = DK + EV;                     // Q^ / K~ row pitch: 16 lanes of a
                                                           // fragment read hit distinct banks
    static constexpr size_t OFF_B = 0;
    static constexpr size_t OFF_QH = OFF_B + (size_t)C * LB * 4;
    static constexpr size_t OFF_KT = OFF_QH + (size_t)C * LQ * ES;
    static constexpr size_t OFF_C = OFF_KT + (size_t)C * LQ * ES;
    static constexpr size_t OFF_ES = OFF_C + (size_t)NPAIR * DK * 4;
    static constexpr size_t OFF_EE = OFF_ES + (size_t)NB * DK * 4;
    static constexpr size_t OFF_BETA = OFF_EE + (size_t)NB * DK * 4;
    static constexpr size_t OFF_FLAG = OFF_BETA + (size_t)C * 4;
    static constexpr size_t SMEM = OFF_FLAG + 16 * 4;
    static_assert(C % 16 == 0 && C <= 64 && DK % KS == 0 && DK % EV == 0, "tile shapes");
    static_assert(THREADS % DK == 0 && C % PARTS == 0, "cumsum split");
    static_assert(!BF || C % 32 == 0, "bf16 P~ in 32-column groups");
    static_assert(SMEM <= 160 * 1024, "LDS");
};

// index of block pair (I, J), J <= I
__device__ __forceinline__ constexpr int gla_pair(int I, int J) { return I * (I + 1) / 2 + J; }

template <typename T, int DK, int C>
__global__ __launch_bounds__(256, 2) void gdn_gla_prep_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const float* __restrict__ log_alpha,
    const float* __restrict__ beta, SeqGeom geom, int H, int units, float* __restrict__ bn_ws,
    T* __restrict__ pt_ws, T* __restrict__ qt_ws, T* __restrict__ kh_ws) {
    using Cfg = GlaPrepCfg<T, DK, C>;
    using St = Step<T>;
    using Frag = typename St::frag;
    constexpr int NB = Cfg::NB, KS = Cfg::KS, NKK = Cfg::NKK, EV = Cfg::EV, LB = Cfg::LB, LQ = Cfg::LQ;
    extern __shared__ __align__(16) unsigned char smem[];
    float* sb = reinterpret_cast<float*>(smem + Cfg::OFF_B);
    T* sqh = reinterpret_cast<T*>(smem + Cfg::OFF_QH);
    T* skt = reinterpret_cast<T*>(smem + Cfg::OFF_KT);
    float* sc = reinterpret_cast<float*>(smem + Cfg::OFF_C);
    float* ses = reinterpret_cast<float*>(smem + Cfg::OFF_ES);
    float* see = reinterpret_cast<float*>(smem + Cfg::OFF_EE);
    float* sbeta = reinterpret_cast<float*>(smem + Cfg::OFF_BETA);
    int* sflag = reinterpret_cast<int*>(smem + Cfg::OFF_FLAG);

    const int tid = (int)threadIdx.x, l = lane_id(), w = wave_id();
    constexpr int NPC = C * (DK / EV);                     // 16-byte pieces of a chunk's q
    constexpr int NV = (NPC + Cfg::THREADS - 1) / Cfg::THREADS;
    const int64_t rs = (int64_t)H * DK;                    // elements between tokens
    const int cd = tid % DK, cp0 = (tid / DK) * Cfg::TPP;  // cumsum: channel, first token

    // The workgroup walks units u = blockIdx.x, + gridDim.x, ...  All loads of a
    // unit are issued up front into registers -- this thread's 16-byte pieces of
    // q and k (piece x = (token, 16 bytes of channels)) and its range of the
    // log-gate (channel cd, tokens cp0 .. cp0 + TPP - 1); rows past the chunk end
    // read as zero -- and those of the next unit are issued as soon as this
    // unit's are used, so that they land while its P~ tiles are formed.
    u32x4 qv[NV], kv[NV];
    float la[Cfg::TPP];
    // (buffer loads: one resource per tensor and unit, 32-bit offsets whose
    // per-piece parts are wave-uniform; out-of-range pieces read as zero)
    const int i_lane = tid / (DK / EV), d_lane = (tid % (DK / EV)) * EV;   // piece of j = 0
    constexpr int TOK_J = Cfg::THREADS / (DK / EV);                      // tokens between j and j + 1
    auto prefetch = [&](const ChunkInfo& ci, int h) __attribute__((always_inline)) {
        const int len = ci.len;
        const int64_t row0 = (int64_t)ci.t0 * H + h;
        const int nb = len > 0 ? (int)(((int64_t)(len - 1) * rs + DK) * Cfg::ES) : 0;
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + row0 * DK, nb);
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + row0 * DK, nb);
        const uint32_t lane_off = (uint32_t)((i_lane * rs + d_lane) * Cfg::ES);
#pragma unroll
        for (int j = 0; j < NV; ++j) {
            const bool ok = tid + j * Cfg::THREADS < NPC && i_lane + j * TOK_J < len;
            const uint32_t off = ok ? lane_off + (uint32_t)(j * TOK_J * rs * Cfg::ES) : kOutOfRange;
            qv[j] = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
            kv[j] = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
        }
        const int nl = log_alpha && len > 0 ? (int)(((int64_t)(len - 1) * rs + DK) * 4) : 0;
        const __amdgpu_buffer_rsrc_t rl =
            make_rsrc(log_alpha ? (const void*)(log_alpha + row0 * DK) : (const void*)q, nl);
        const uint32_t l_off = (uint32_t)((cp0 * rs + cd) * 4);
#pragma unroll
        for (int t = 0; t < Cfg::TPP; ++t)
            la[t] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                  rl, cp0 + t < len ? l_off + (uint32_t)(t * rs * 4) : kOutOfRange, 0, 0));
    };
    auto unit_info = [&](int uu) __attribute__((always_inline)) {
        ChunkInfo ci{0, 0, 0};
        if (uu < units) ci = chunk_info(geom, uu / H);
        return ci;
    };
    int u = (int)blockIdx.x;
    ChunkInfo ci_next = unit_info(u);
    if (ci_next.len > 0) prefetch(ci_next, u % H);
    for (; u < units; u += (int)gridDim.x) {
        const int slot = u / H, h = u - slot * H;
        const ChunkInfo ci = ci_next;
        const int len = ci.len;   // 0: unused packed-batch slot (uniform)
        const int64_t row0 = (int64_t)ci.t0 * H + h;   // (token, head) row of the chunk's first token
        const int un = u + (int)gridDim.x;
        ci_next = unit_info(un);
        if (len > 0) {
            if (tid < C) sbeta[tid] = tid < len ? (beta ? beta[(row0 + (int64_t)tid * H)] : 1.f) : 0.f;
            if (tid < 16) sflag[tid] = 0;

            // ---- the per-channel cumulative log-gate b: each range summed in
            // registers, then offset by the totals of the ranges before it
            {
                float acc = 0.f;
#pragma unroll
                for (int t = 0; t < Cfg::TPP; ++t) {
                    acc += la[t];
                    la[t] = acc;
                }
                sb[(cp0 + Cfg::TPP - 1) * LB + cd] = acc;
                __syncthreads();
                float off = 0.f;
                for (int r0 = 0; r0 < cp0; r0 += Cfg::TPP) off += sb[(r0 + Cfg::TPP - 1) * LB + cd];
                __syncthreads();
#pragma unroll
                for (int t = 0; t < Cfg::TPP; ++t) sb[(cp0 + t) * LB + cd] = la[t] + off;
                __syncthreads();
            }

            // ---- the path: fast unless some channel decays by e^64 or more
            if (tid < DK && !(sb[(C - 1) * LB + tid] > -Cfg::kMaxChunkLog)) sflag[Cfg::FLAG_SLOW_CHUNK] = 1;
            __syncthreads();
        }
        const bool fast = len > 0 && sflag[Cfg::FLAG_SLOW_CHUNK] == 0;   // (uniform)
        if (fast) {
            // ---- e^{b_n} per channel, then Q~, K^ out (valid rows), Q~ and K' into LDS
            for (int d = tid; d < DK; d += Cfg::THREADS) {
                const float en = __expf(sb[(C - 1) * LB + d]);
                ses[d] = en;
                bn_ws[(int64_t)u * DK + d] = en;
            }
            __syncthreads();
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                const int x = tid + j * Cfg::THREADS, i = x / (DK / EV), d0 = (x % (DK / EV)) * EV;
                if (x >= NPC) break;
                const T* qp = reinterpret_cast<const T*>(&qv[j]);
                const T* kp = reinterpret_cast<const T*>(&kv[j]);
                T qo[EV], ko[EV], kq[EV];
                const float be = sbeta[i];
#pragma unroll
                for (int e = 0; e < EV; ++e) {
                    const int d = d0 + e;
                    const float bi = sb[i * LB + d];
                    const float qt = to_f32(qp[e]) * __expf(bi);     // q e^{b_i}
                    const float kq_ = to_f32(kp[e]) * __expf(-bi);   // k e^{-b_i} (< e^64 |k|)
                    qo[e] = from_f32<T>(qt);
                    kq[e] = from_f32<T>(kq_);
                    ko[e] = from_f32<T>(be * kq_ * ses[d]);          // beta k e^{b_n - b_i}
                }
                *reinterpret_cast<u32x4*>(sqh + i * LQ + d0) = *reinterpret_cast<const u32x4*>(qo);
                *reinterpret_cast<u32x4*>(skt + i * LQ + d0) = *reinterpret_cast<const u32x4*>(kq);
                if (i < len) {
                    *reinterpret_cast<u32x4*>(qt_ws + (row0 * DK + (int64_t)i * rs + d0)) =
                        *reinterpret_cast<const u32x4*>(qo);
                    *reinterpret_cast<u32x4*>(kh_ws + (row0 * DK + (int64_t)i * rs + d0)) =
                        *reinterpret_cast<const u32x4*>(ko);
                }
            }
            __syncthreads();
        } else if (len > 0) {
            // ---- per-channel block factors: e^{b_16I}, e^{b_n - b_eI}, c_IJ, e^{b_n};
            // diagonal blocks whose decay reaches e^64 on some channel take the slow path
            for (int x = tid; x < DK * (2 * NB + Cfg::NPAIR + 1); x += Cfg::THREADS) {
                const int d = x % DK, y = x / DK;
                const float bn = sb[(C - 1) * LB + d];
                if (y < NB) {
                    ses[y * DK + d] = __expf(sb[16 * y * LB + d]);
                } else if (y < 2 * NB) {
                    const int I = y - NB;
                    see[I * DK + d] = __expf(bn - sb[(16 * I + 15) * LB + d]);
                } else if (y < 2 * NB + Cfg::NPAIR) {
                    int pr = y - 2 * NB, I = 0;
                    while (pr > I) pr -= ++I;      // pair index -> (I, J = pr)
                    const float e = sb[16 * I * LB + d] - sb[(16 * pr + 15) * LB + d];
                    sc[gla_pair(I, pr) * DK + d] = __expf(e);
                    if (pr == I && e >= Cfg::kMaxDiagLog) sflag[I] = 1;   // same value from every writer
                } else {
                    bn_ws[(int64_t)u * DK + d] = __expf(bn);
                }
            }
            __syncthreads();

            // ---- Q~, K^ out (valid rows), Q^ and K~ into LDS, from the pieces loaded above
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                const int x = tid + j * Cfg::THREADS, i = x / (DK / EV), d0 = (x % (DK / EV)) * EV, I = i / 16;
                if (x >= NPC) break;
                const bool in = i < len;
                const T* qp = reinterpret_cast<const T*>(&qv[j]);
                const T* kp = reinterpret_cast<const T*>(&kv[j]);
                T qo[EV], ko[EV], qh[EV], kt[EV];
                const float be = sbeta[i];
#pragma unroll
                for (int e = 0; e < EV; ++e) {
                    const int d = d0 + e;
                    const float qf = to_f32(qp[e]), kf = to_f32(kp[e]);
                    const float bi = sb[i * LB + d];
                    const float fq = __expf(bi - sb[16 * I * LB + d]);          // e^{b_i - b_16I} <= 1
                    const float fk = __expf(sb[(16 * I + 15) * LB + d] - bi);   // e^{b_eI - b_i} <= 1
                    const float qhv = qf * fq, ktv = kf * fk;
                    qh[e] = from_f32<T>(qhv);
                    kt[e] = from_f32<T>(ktv);
                    qo[e] = from_f32<T>(qhv * ses[I * DK + d]);                 // q e^{b_i}
                    ko[e] = from_f32<T>(be * ktv * see[I * DK + d]);           // beta k e^{b_n - b_i}
                }
                *reinterpret_cast<u32x4*>(sqh + i * LQ + d0) = *reinterpret_cast<const u32x4*>(qh);
                *reinterpret_cast<u32x4*>(skt + i * LQ + d0) = *reinterpret_cast<const u32x4*>(kt);
                if (in) {
                    *reinterpret_cast<u32x4*>(qt_ws + (row0 * DK + (int64_t)i * rs + d0)) =
                        *reinterpret_cast<const u32x4*>(qo);
                    *reinterpret_cast<u32x4*>(kh_ws + (row0 * DK + (int64_t)i * rs + d0)) =
                        *reinterpret_cast<const u32x4*>(ko);
                }
            }
            __syncthreads();
        }
        // the next unit's loads, now that this unit's registers are used
        if (ci_next.len > 0) prefetch(ci_next, un % H);
        if (len > 0) {
            // ---- P~ tiles: P^T_IJ = (K~_J o c_IJ) Q^_I^T, so that lane (g, n) holds
            // P[16I + n][16J + 4g + r] (the operand layout of the Tb blocks); then the
            // mask s <= i and the column scale beta_s.  Operand blocks go round-robin
            // to the waves.
            const int n = l & 15, g = l >> 4;
            auto tile = [&](int I, int J) __attribute__((always_inline)) -> f32x4 {
                if (J > I) return zero4();
                f32x4 acc = zero4();
                const bool slow = !fast && J == I && sflag[I] != 0;
                if (fast) {
#pragma unroll
                    for (int kk = 0; kk < NKK; ++kk) {
                        Frag a, b;
                        if constexpr (Cfg::BF) {
                            const int dd = kk * KS + g * EV;
                            a = *reinterpret_cast<const Frag*>(skt + (16 * J + n) * LQ + dd);
                            b = *reinterpret_cast<const Frag*>(sqh + (16 * I + n) * LQ + dd);
                        } else {
                            const int d4 = kk * KS + 4 * g;
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                a[r] = skt[(16 * J + n) * LQ + d4 + r];
                                b[r] = sqh[(16 * I + n) * LQ + d4 + r];
                            }
                        }
                        acc = St::mma(a, b, acc);
                    }
                } else if (!slow) {
                    const float* cp = sc + gla_pair(I, J) * DK;
#pragma unroll
                    for (int kk = 0; kk < NKK; ++kk) {
                        const int dd = kk * KS + g * EV;   // this lane's contraction values
                        Frag a, b;
                        if constexpr (Cfg::BF) {
                            const T* kr = skt + (16 * J + n) * LQ + dd;
                            const T* qr = sqh + (16 * I + n) * LQ + dd;
#pragma unroll
                            for (int e = 0; e < EV; ++e) {
                                a[e] = from_f32<T>(to_f32(kr[e]) * cp[dd + e]);
                                b[e] = qr[e];
                            }
                        } else {
                            // fp32 16x16x4 steps: value r of the fragment is contraction index 4g + r
                            const int d4 = kk * KS + 4 * g;
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                a[r] = skt[(16 * J + n) * LQ + d4 + r] * cp[d4 + r];
                                b[r] = sqh[(16 * I + n) * LQ + d4 + r];
                            }
                        }
                        acc = St::mma(a, b, acc);
                    }
                } else {
                    // term by term, from the inputs: P_is = sum_d q_id k_sd e^{b_id - b_sd}
                    const int i = 16 * I + n;
#pragma unroll 1
                    for (int r = 0; r < 4; ++r) {
                        const int s = 16 * J + 4 * g + r;
                        float sum = 0.f;
                        if (s <= i && i < len) {
                            const T* qp = q + (row0 + (int64_t)i * H) * DK;
                            const T* kp = k + (row0 + (int64_t)s * H) * DK;
#pragma unroll 1
                            for (int d = 0; d < DK; ++d)
                                sum += to_f32(qp[d]) * to_f32(kp[d]) * __expf(sb[i * LB + d] - sb[s * LB + d]);
                        }
                        acc[r] = sum;
                    }
                }
                // mask and beta: entry r is P[16I + n][16J + 4g + r]
                const int i = 16 * I + n;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int s = 16 * J + 4 * g + r;
                    acc[r] = s <= i ? acc[r] * sbeta[s] : 0.f;
                }
                return acc;
            };
            T* out = pt_ws + (int64_t)u * (Cfg::NBLK * 1024 / Cfg::ES);
            for (int blk = w; blk < Cfg::NBLK; blk += Cfg::WAVES) {
                // block -> (row block ti, column group qq), as tb_block numbers them
                int ti = 0, qq = blk;
                while (qq >= (Cfg::BF ? ti / 2 + 1 : ti + 1)) {
                    qq -= Cfg::BF ? ti / 2 + 1 : ti + 1;
                    ++ti;
                }
                unsigned char* dst = reinterpret_cast<unsigned char*>(out) + blk * 1024 + l * 16;
                if constexpr (Cfg::BF) {
                    const f32x4 t0 = tile(ti, 2 * qq), t1 = tile(ti, 2 * qq + 1);
                    const bf16x8 o = {(bf16)t0[0], (bf16)t0[1], (bf16)t0[2], (bf16)t0[3],
                                      (bf16)t1[0], (bf16)t1[1], (bf16)t1[2], (bf16)t1[3]};
                    *reinterpret_cast<bf16x8*>(dst) = o;
                } else {
                    *reinterpret_cast<f32x4*>(dst) = tile(ti, qq);
                }
            }
        }
        __syncthreads();   // before the next unit overwrites the LDS read above
    }
}

}  // namespace gdn
