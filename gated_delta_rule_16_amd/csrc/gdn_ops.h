// gdn_ops.h -- MFMA operand helpers shared by the scan kernels: operand
// layouts of one 16-deep contraction block, transposing LDS reads, swizzled
// staged rows and the waits that order LDS hand-overs.
#pragma once

#include <type_traits>

#include "gdn_device.h"

namespace gdn {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// s_waitcnt with vmcnt <= vm and lgkmcnt = 0 (expcnt not waited on)
template <int VM>
__device__ __forceinline__ void wait_vm_lgkm0() {
    static_assert(VM >= 0 && VM < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | ((VM >> 4) << 14));
}

// Operand of one 16-deep contraction block: lane (g, n) holds k = 4g .. 4g+3
// for row / column n of the other dimension.  A 16x16 accumulator tile has
// exactly this layout, with k = its row.
template <typename T> struct K16;
template <> struct K16<bf16> {
    typedef s16x4 op;
    __device__ __forceinline__ static op tile(f32x4 t) {
        const bf16x4 v = {(bf16)t[0], (bf16)t[1], (bf16)t[2], (bf16)t[3]};
        return __builtin_bit_cast(s16x4, v);
    }
    __device__ __forceinline__ static f32x4 mma1(op a, op b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
    }
    // blocks (a0, b0) and (a1, b1) in one 16x16x32 instruction
    __device__ __forceinline__ static f32x4 mma2(op a0, op a1, op b0, op b1, f32x4 c) {
        const s16x8 a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
        return mma2p(__builtin_bit_cast(bf16x8, a), b0, b1, c);
    }
    // the A pair already packed (a0 in elements 0..3, a1 in 4..7)
    __device__ __forceinline__ static f32x4 mma2p(bf16x8 a, op b0, op b1, f32x4 c) {
        const s16x8 b = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};
template <> struct K16<float> {
    typedef f32x4 op;
    __device__ __forceinline__ static op tile(f32x4 t) { return t; }
    __device__ __forceinline__ static f32x4 mma1(op a, op b, f32x4 c) {
#pragma unroll
        for (int r = 0; r < 4; ++r) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[r], b[r], c, 0, 0, 0);
        return c;
    }
    __device__ __forceinline__ static f32x4 mma2(op a0, op a1, op b0, op b1, f32x4 c) {
        return mma1(a1, b1, mma1(a0, b0, c));
    }
};

__device__ __forceinline__ float bf16_bits_to_f32(short x) {
    return __builtin_bit_cast(float, (unsigned)(unsigned short)x << 16);
}

// Transposing 64-bit LDS read (ds_read_b64_tr_b16): within each 16-lane group,
// lane s supplies the address of 4 consecutive 16-bit values; lane j receives
// value j % 4 of lane 4e + j / 4 as its element e.
__device__ __forceinline__ s16x4 tr_read(const void* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

// 4 consecutive values of one lane, rounded to T, as one 8- or 16-byte LDS store
template <typename T>
__device__ __forceinline__ void store4(T* p, float a, float b, float c, float d) {
    if constexpr (sizeof(T) == 2) {
        const bf16x4 v = {(bf16)a, (bf16)b, (bf16)c, (bf16)d};
        *reinterpret_cast<bf16x4*>(p) = v;
    } else {
        *reinterpret_cast<f32x4*>(p) = f32x4{a, b, c, d};
    }
}

// element (r, c) of a staged region (pitch P blocks, swizzle kind W)
template <typename Cfg, int P, int W>
__device__ __forceinline__ int sidx(int r, int c) {
    return (r * P + ((c / Cfg::EV) ^ swz<W>(r))) * Cfg::EV + (c % Cfg::EV);
}
template <typename Cfg>
__device__ __forceinline__ int kidx(int r, int c) { return sidx<Cfg, Cfg::KP, Cfg::KSW>(r, c); }
template <typename Cfg>
__device__ __forceinline__ int vidx(int r, int c) { return sidx<Cfg, Cfg::VP, Cfg::VSW>(r, c); }

// Step fragment (16 bytes) of the swizzled K chunk: K[row0 + n][k0 + g*EV ...]
template <typename Cfg, typename T>
__device__ __forceinline__ typename Step<T>::frag kfrag_rows(const T* sK, int row0, int k0) {
    const int l = lane_id();
    return *reinterpret_cast<const typename Step<T>::frag*>(
        sK + kidx<Cfg>(row0 + (l & 15), k0 + (l >> 4) * Cfg::EV));
}

// V rows jb*16 + 4g + e, column vb*16 + n, as fp32
template <typename Cfg, typename T>
__device__ __forceinline__ f32x4 vcol4(const T* sV, int jb, int vb) {
    const int l = lane_id(), g = l >> 4, n = l & 15;
    if constexpr (Cfg::BF) {
        const s16x4 x = tr_read(sV + vidx<Cfg>(jb * 16 + 4 * g + (n >> 2), vb * 16 + 4 * (n & 3)));
        return f32x4{bf16_bits_to_f32(x[0]), bf16_bits_to_f32(x[1]), bf16_bits_to_f32(x[2]),
                     bf16_bits_to_f32(x[3])};
    } else {
        const T* p = sV + vidx<Cfg>(jb * 16 + 4 * g, vb * 16 + n);   // fp32 rows are not swizzled
        return f32x4{p[0], p[Cfg::LDV], p[2 * Cfg::LDV], p[3 * Cfg::LDV]};
    }
}

}  // namespace gdn
