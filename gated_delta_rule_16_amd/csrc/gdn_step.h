// gdn_step.h -- single-token recurrent step (decoding) and the packed-batch
// chunk table.
//
// Step, per (sequence, head), S of shape Dv x Dk updated in place:
//   S~ = alpha S;  p = S~ k;  S = S~ + beta (v - p) k^T;  o = S q
// Qiita article on the Linear Attention lineage, section "Gated-DeltaNet"
// (S_i = alpha_i S_{i-1}(I - beta_i k_i k_i^T) + beta_i v_i k_i^T, h_i = S_i q_i);
// a step needs only the previous state and the token's q, k, v (section
// "Linear attention": the state replaces the KV cache).
#pragma once

#include "gdn_device.h"

namespace gdn {

// One wave per state row; ROWS rows per workgroup.  Lanes stride over Dk.
template <typename T, int DK, int DV>
__global__ __launch_bounds__(kThreads) void gdn_step_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ beta,
    float* __restrict__ S, T* __restrict__ o, int H) {
    constexpr int ROWS_PER_WAVE = 4;
    constexpr int ROWS = 4 * ROWS_PER_WAVE;
    constexpr int PER_LANE = (DK + 63) / 64;
    static_assert(DV % ROWS == 0, "Dv must be a multiple of 16");
    const int h = blockIdx.y, seq = blockIdx.z;
    const int l = lane_id(), w = wave_id();
    const int64_t x = (int64_t)seq * H + h;
    const float a = log_alpha ? __expf(log_alpha[x]) : 1.f;
    const float b = beta[x];
    float kr[PER_LANE], qr[PER_LANE];
#pragma unroll
    for (int j = 0; j < PER_LANE; ++j) {
        const int d = l + 64 * j;
        kr[j] = d < DK ? to_f32(k[x * DK + d]) : 0.f;
        qr[j] = d < DK ? to_f32(q[x * DK + d]) : 0.f;
    }
    for (int rr = 0; rr < ROWS_PER_WAVE; ++rr) {
        const int row = blockIdx.x * ROWS + w * ROWS_PER_WAVE + rr;
        float* Srow = S + (x * DV + row) * DK;
        float s[PER_LANE];
        float p = 0.f;
#pragma unroll
        for (int j = 0; j < PER_LANE; ++j) {
            const int d = l + 64 * j;
            s[j] = d < DK ? a * Srow[d] : 0.f;
            p += s[j] * kr[j];
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) p += __shfl_xor(p, off, 64);
        const float e = b * (to_f32(v[x * DV + row]) - p);
        float ov = 0.f;
#pragma unroll
        for (int j = 0; j < PER_LANE; ++j) {
            const int d = l + 64 * j;
            s[j] += e * kr[j];
            ov += s[j] * qr[j];
            if (d < DK) Srow[d] = s[j];
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) ov += __shfl_xor(ov, off, 64);
        if (l == 0) o[x * DV + row] = from_f32<T>(ov);
    }
}

// Packed batch -> chunk table.  One workgroup of 1024 threads.
//  c'_i = min(T, max(0, max_{j<=i} cu[j]))   (monotone clamp; equals cu when valid)
//  sequence i = tokens c'_i .. c'_{i+1}-1, split into ceil(len / C) chunks;
//  seq_slot[i] = first slot of sequence i (exclusive prefix sum of chunk counts);
//  table[s] = {seq, t0, len, 0}; slots past the last chunk get len = 0.
// Scratch: bounds[N+1] holds c'.
constexpr int kTableThreads = 1024;

__global__ __launch_bounds__(kTableThreads) void gdn_chunk_table_kernel(
    const int* __restrict__ cu, int n_seqs, int T, int C, int max_slots,
    int* __restrict__ bounds, int* __restrict__ seq_slot, int* __restrict__ table) {
    __shared__ int sbuf[kTableThreads];
    __shared__ int carry;
    const int tid = threadIdx.x;
    // phase 1: running max of cu, clamped to [0, T]
    if (tid == 0) carry = 0;
    __syncthreads();
    for (int base = 0; base <= n_seqs; base += kTableThreads) {
        const int i = base + tid;
        int x = (i <= n_seqs) ? cu[i] : 0;
        x = x < 0 ? 0 : (x > T ? T : x);
        sbuf[tid] = x;
        __syncthreads();
        for (int off = 1; off < kTableThreads; off <<= 1) {
            const int y = tid >= off ? sbuf[tid - off] : 0;
            __syncthreads();
            if (y > sbuf[tid]) sbuf[tid] = y;
            __syncthreads();
        }
        const int c0 = carry;
        const int val = sbuf[tid] > c0 ? sbuf[tid] : c0;
        if (i <= n_seqs) bounds[i] = val;
        __syncthreads();
        if (tid == kTableThreads - 1) carry = val;
        __syncthreads();
    }
    // phase 2: exclusive prefix sum of per-sequence chunk counts
    if (tid == 0) carry = 0;
    __syncthreads();
    for (int base = 0; base < n_seqs; base += kTableThreads) {
        const int i = base + tid;
        const int cnt = (i < n_seqs) ? (bounds[i + 1] - bounds[i] + C - 1) / C : 0;
        sbuf[tid] = cnt;
        __syncthreads();
        for (int off = 1; off < kTableThreads; off <<= 1) {
            const int y = tid >= off ? sbuf[tid - off] : 0;
            __syncthreads();
            sbuf[tid] += y;
            __syncthreads();
        }
        const int c0 = carry;
        if (i < n_seqs) seq_slot[i] = c0 + sbuf[tid] - cnt;
        __syncthreads();
        if (tid == kTableThreads - 1) carry = c0 + sbuf[tid];
        __syncthreads();
    }
    if (tid == 0) seq_slot[n_seqs] = carry;
    __syncthreads();
    const int total = carry;
    // phase 3: fill the table
    int4* tab = reinterpret_cast<int4*>(table);
    for (int i = tid; i < n_seqs; i += kTableThreads) {
        const int s0 = seq_slot[i], t0 = bounds[i], t1 = bounds[i + 1];
        for (int c = 0; t0 + c * C < t1; ++c) {
            const int st = t0 + c * C;
            const int len = (t1 - st) < C ? (t1 - st) : C;
            tab[s0 + c] = make_int4(i, st, len, 0);
        }
    }
    for (int s = total + tid; s < max_slots; s += kTableThreads) tab[s] = make_int4(0, 0, 0, 0);
}

}  // namespace gdn
