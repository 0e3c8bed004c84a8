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

// Layout of the step: a workgroup is one wave and owns RPW consecutive rows of
// one state.  A row of Dk fp32 values is LPR lanes of 16 bytes, so one load
// instruction reads RPI = 64 / LPR whole rows (contiguous, as rows are), and a
// wave issues all NI loads of its rows before it uses any: NI KB in flight per
// wave, the step being a stream through the state.
template <int DK, int DV>
struct StepCfg {
    static constexpr int LPR = DK / 4;                  // lanes per row
    static constexpr int RPI = 64 / LPR;                // rows per load instruction
    static constexpr int NI = DV / RPI < 8 ? DV / RPI : 8;
    static constexpr int RPW = NI * RPI;                // rows per wave (= per workgroup)
    static_assert(DK % 4 == 0 && 64 % LPR == 0 && NI >= 1 && DV % RPW == 0, "step tiling");
};

template <typename T, int DK, int DV>
__global__ __launch_bounds__(64) void gdn_step_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ log_alpha, const float* __restrict__ beta,
    float* __restrict__ S, T* __restrict__ o, int H) {
    using Cfg = StepCfg<DK, DV>;
    constexpr int LPR = Cfg::LPR, RPI = Cfg::RPI, NI = Cfg::NI;
    const int h = blockIdx.y, seq = blockIdx.z;
    const int l = lane_id();
    const int ri = l / LPR, c4 = (l % LPR) * 4;         // row within an instruction, first d
    const int64_t x = (int64_t)seq * H + h;
    const int row0 = blockIdx.x * Cfg::RPW + ri;
    float* Sx = S + x * DV * DK + c4;
    // the rows first: NI loads of 16 bytes per lane
    f32x4 s[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) s[i] = *reinterpret_cast<const f32x4*>(Sx + (int64_t)(row0 + i * RPI) * DK);
    float vr[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) vr[i] = to_f32(v[x * DV + row0 + i * RPI]);
    const float a = log_alpha ? __expf(log_alpha[x]) : 1.f;
    const float b = beta[x];
    f32x4 kr, qr;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        kr[e] = to_f32(k[x * DK + c4 + e]);
        qr[e] = to_f32(q[x * DK + c4 + e]);
    }
    // p = (a S) k over the LPR lanes of each row
    float p[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        s[i] *= a;
        p[i] = s[i][0] * kr[0] + s[i][1] * kr[1] + s[i][2] * kr[2] + s[i][3] * kr[3];
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1)
#pragma unroll
        for (int i = 0; i < NI; ++i) p[i] += __shfl_xor(p[i], off, 64);
    // S = a S + beta (v - p) k^T, then o = S q
    float ov[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const float e = b * (vr[i] - p[i]);
        s[i] += e * kr;
        ov[i] = s[i][0] * qr[0] + s[i][1] * qr[1] + s[i][2] * qr[2] + s[i][3] * qr[3];
        *reinterpret_cast<f32x4*>(Sx + (int64_t)(row0 + i * RPI) * DK) = s[i];
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1)
#pragma unroll
        for (int i = 0; i < NI; ++i) ov[i] += __shfl_xor(ov[i], off, 64);
    if (l % LPR == 0) {
#pragma unroll
        for (int i = 0; i < NI; ++i) o[x * DV + row0 + i * RPI] = from_f32<T>(ov[i]);
    }
}

// Packed batch -> chunk table.  One workgroup of 1024 threads.
//  c'_i = min(T, max(0, max_{j<=i} cu[j]))   (monotone clamp; equals cu when valid)
//  sequence i = tokens c'_i .. c'_{i+1}-1, split into ceil(len / C) chunks;
//  seq_slot[i] = first slot of sequence i (exclusive prefix sum of chunk counts);
//  table[s] = {seq, t0, len, 0}; slots past the last chunk get len = 0.
// Scratch: bounds[N+1] holds c'.
constexpr int kTableThreads = 1024;

// Inclusive scan over the workgroup (max when MAX, else sum): each wave by
// shuffles, then the 16 wave totals by the first wave; wsum holds 16 ints.
template <bool MAX>
__device__ __forceinline__ int block_scan(int x, int* wsum) {
    const int l = lane_id(), w = threadIdx.x >> 6;
    auto op = [](int a, int b) { return MAX ? (a > b ? a : b) : a + b; };
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        if (l >= off) x = op(x, y);
    }
    if (l == 63) wsum[w] = x;
    __syncthreads();
    if (w == 0) {
        int t = l < kTableThreads / 64 ? wsum[l] : 0;
#pragma unroll
        for (int off = 1; off < kTableThreads / 64; off <<= 1) {
            const int y = __shfl_up(t, off, 64);
            if (l >= off) t = op(t, y);
        }
        if (l < kTableThreads / 64) wsum[l] = t;
    }
    __syncthreads();
    if (w > 0) x = op(x, wsum[w - 1]);
    __syncthreads();   // wsum free for the next scan
    return x;
}

// Order of the sequences for the scan, by chunk count, longest first: a
// counting sort over kOrderBins bins (counts of kOrderBins - 1 chunks and more
// share the first bin); equal counts in no fixed order.  With the longest
// sequences' workgroups dispatched first, a CU that frees up takes shorter
// work last, which shortens the scan's makespan over a mixed batch.
constexpr int kOrderBins = 4096;
static_assert(kOrderBins % kTableThreads == 0, "bins per thread");

__global__ __launch_bounds__(kTableThreads) void gdn_chunk_table_kernel(
    const int* __restrict__ cu, int n_seqs, int T, int C, int max_slots,
    int* __restrict__ bounds, int* __restrict__ seq_slot, int* __restrict__ table,
    int* __restrict__ order) {
    __shared__ int wsum[kTableThreads / 64];
    __shared__ int carry;
    __shared__ int bins[kOrderBins];
    const int tid = threadIdx.x;
    // phase 1: running max of cu, clamped to [0, T] (values are >= 0, so 0 is
    // the identity of the max)
    if (tid == 0) carry = 0;
    __syncthreads();
    for (int base = 0; base <= n_seqs; base += kTableThreads) {
        const int i = base + tid;
        int x = (i <= n_seqs) ? cu[i] : 0;
        x = x < 0 ? 0 : (x > T ? T : x);
        x = block_scan<true>(x, wsum);
        const int c0 = carry;
        const int val = x > c0 ? x : c0;
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
        const int inc = block_scan<false>(cnt, wsum);
        const int c0 = carry;
        if (i < n_seqs) seq_slot[i] = c0 + inc - cnt;
        __syncthreads();
        if (tid == kTableThreads - 1) carry = c0 + inc;
        __syncthreads();
    }
    if (tid == 0) seq_slot[n_seqs] = carry;
    __syncthreads();
    const int total = carry;
    // phase 3: fill the table, one slot per thread: its sequence is the last i
    // with seq_slot[i] <= slot (binary search; empty sequences own no slot)
    int4* tab = reinterpret_cast<int4*>(table);
    for (int s = tid; s < max_slots; s += kTableThreads) {
        if (s >= total) {
            tab[s] = make_int4(0, 0, 0, 0);
            continue;
        }
        int lo = 0, hi = n_seqs - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (seq_slot[mid] <= s) lo = mid;
            else hi = mid - 1;
        }
        const int st = bounds[lo] + (s - seq_slot[lo]) * C;
        const int len = (bounds[lo + 1] - st) < C ? (bounds[lo + 1] - st) : C;
        tab[s] = make_int4(lo, st, len, 0);
    }
    // phase 4: order, longest first.  Bin b holds the sequences of
    // kOrderBins - 1 - b chunks (the first bin also longer ones).
    constexpr int BPT = kOrderBins / kTableThreads;
    auto bin_of = [&](int i) {
        const int cnt = seq_slot[i + 1] - seq_slot[i];
        return kOrderBins - 1 - (cnt < kOrderBins - 1 ? cnt : kOrderBins - 1);
    };
#pragma unroll
    for (int j = 0; j < BPT; ++j) bins[tid * BPT + j] = 0;
    __syncthreads();
    for (int i = tid; i < n_seqs; i += kTableThreads) atomicAdd(&bins[bin_of(i)], 1);
    __syncthreads();
    // exclusive prefix sum over the bins (thread tid owns BPT consecutive ones)
    int loc[BPT], sum = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
        loc[j] = sum;
        sum += bins[tid * BPT + j];
    }
    const int before = block_scan<false>(sum, wsum) - sum;
#pragma unroll
    for (int j = 0; j < BPT; ++j) bins[tid * BPT + j] = before + loc[j];   // first position of the bin
    __syncthreads();
    for (int i = tid; i < n_seqs; i += kTableThreads) order[atomicAdd(&bins[bin_of(i)], 1)] = i;
}

}  // namespace gdn
