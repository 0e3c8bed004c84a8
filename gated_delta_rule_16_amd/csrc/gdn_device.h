// gdn_device.h -- device-side building blocks shared by the gfx950 kernels:
// element types, 16x16 MFMA contraction steps, buffer resources, LDS swizzles,
// the Tb block layout and chunk metadata.
//
// MFMA tile conventions (wave64, 16x16 output tile):
//   lane l = 0..63, column/row index inside the tile  n = l & 15,  lane group g = l >> 4.
//   A fragment: A[m0 + n][k0 + g*KPL + e], e < KPL   (KPL contraction values per lane)
//   B fragment: B[k0 + g*KPL + e][n0 + n]
//   D (4 fp32 per lane): D[4g + r][n], r = 0..3
// bf16 uses v_mfma_f32_16x16x32_bf16 (KPL = 8), fp32 uses v_mfma_f32_16x16x4_f32
// (KPL = 1, four per 16-deep step).  A and B fragments assign contraction
// indices to (g, e) the same way, so the product does not depend on how the
// hardware orders them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));   // 16 raw bytes

constexpr int kThreads = 256;   // 4 waves per workgroup (prep)

// Update rules the chunk kernels evaluate (the C ABI's gdn_rule values):
//  kDelta    S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
//  kNoErase  S_t = alpha_t S_{t-1} + beta_t v_t k_t^T   (Mamba2 with a write strength)
//  kGla      S_t = S_{t-1} diag(alpha_t) + beta_t v_t k_t^T   (per-channel gate)
enum : int { kDelta = 0, kNoErase = 1, kGla = 2 };
// fp32 rows per chunk of the gate values handed to the scan: g, exp(g),
// exp(g_n - g), and for kNoErase beta as a fourth row
constexpr int gate_rows(int rule) { return rule == kDelta ? 3 : 4; }
// fp32 gate values per chunk handed to the scan: the rows above, or for kGla
// the decay of the whole chunk per key channel, exp(b_n) (Dk values)
constexpr int gate_floats(int rule, int C, int DK) { return rule == kGla ? DK : gate_rows(rule) * C; }

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }
// wave index, known to the compiler to be uniform across the wave
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// One 16-byte step of a contraction along the rows of two row-major operands:
// lane (g, n) holds elements [k0 + g*EV, k0 + (g+1)*EV) of row n (EV = 16 / sizeof(T)).
// bf16: one 16x16x32 MFMA; fp32: four 16x16x4 MFMAs, step r contracting
// k0 + 4g + r (the same assignment on both operands).
template <typename T> struct Step;
template <> struct Step<bf16> {
    static constexpr int KS = 32;
    typedef bf16x8 frag;
    __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct Step<float> {
    static constexpr int KS = 16;
    typedef f32x4 frag;
    __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
#pragma unroll
        for (int r = 0; r < 4; ++r) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[r], b[r], c, 0, 0, 0);
        return c;
    }
};

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // RNE

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Word 3 of a raw buffer resource: 32-bit untyped data, range-checked against
// the record count (out-of-range loads return 0, stores are dropped).
constexpr int kRsrcWord3 = 0x00020000;
constexpr uint32_t kOutOfRange = 0x80000000u;   // a byte offset past every record count

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

// 16 bytes per lane from a buffer straight into LDS: lane l's bytes land at
// lds + 16 l (lds must be the same for the whole wave); out-of-range offsets
// land as zeros.  Completion is counted by vmcnt, like any other load.
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, unsigned char* lds, uint32_t voff) {
    typedef __attribute__((address_space(3))) void lds_void;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, 0, 0, 0);
}

// 4 bytes per lane from a buffer straight into LDS (lane l's at lds + 4 l);
// otherwise as lds_load16
__device__ __forceinline__ void lds_load4(__amdgpu_buffer_rsrc_t r, unsigned char* lds, uint32_t voff) {
    typedef __attribute__((address_space(3))) void lds_void;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 4, voff, 0, 0, 0);
}

// XOR swizzles of 16-byte blocks in LDS rows: data block b of row r sits at
// block b ^ swz(r).  Kinds: 0 none; 1 (K / Q rows of 8+ blocks) 2 (r mod 4) +
// (r / 4 mod 2); 2 (V rows of 4+ blocks) 2 (r / 2 mod 2); 3 (Tb / X^T rows of 8+
// blocks) r mod 8; 4 (K / Q rows of 16+ blocks) 2 (r mod 8); 5 (V rows of 4
// blocks) 2 (r / 4 mod 2).
//
// Kinds 4 and 5 follow the LDS of gfx950 as measured with its bank-conflict
// counter: 64 banks of 4 bytes; a 16-byte read serves 16 lanes per cycle, the
// lanes with equal (lane / 32, parity of bits 2..4 of the lane); 8-byte reads
// (plain or transposing) serve lanes 0-31, then 32-63.  With 256-byte K rows,
// kind 4 makes the 16-byte row reads of an MFMA operand conflict-free and the
// transposing K^T reads take two passes, the least for rows of whole 16-byte
// blocks; kind 5 makes the transposing reads of 64-byte V rows conflict-free.
template <int KIND>
__device__ __forceinline__ constexpr int swz(int r) {
    if constexpr (KIND == 1) return 2 * (r & 3) + ((r >> 2) & 1);
    else if constexpr (KIND == 2) return ((r >> 1) & 1) << 1;
    else if constexpr (KIND == 3) return r & 7;
    else if constexpr (KIND == 4) return 2 * (r & 7);
    else if constexpr (KIND == 5) return ((r >> 2) & 1) << 1;
    else return 0;
}


// Tb = T diag(beta) of one chunk, as handed from the prep kernel to the scan:
// whole 1 KB blocks of MFMA operands (16 bytes per lane, lane-linear), only the
// blocks of the lower block triangle.  bf16: block (ti, q), 2q <= ti, gives
// lane (g, n) row 16 ti + n at columns 4g .. 4g+3 of 16-column tiles 2q and
// 2q + 1 (the A operand of a 16x16x32 instruction over token pair (2q, 2q + 1));
// fp32: block (ti, tj), tj <= ti, gives lane (g, n) row 16 ti + n at columns
// 16 tj + 4g .. + 3.  Blocks are numbered row block by row block.
constexpr int tb_block(int ti, int q, bool bf) {
    int s = 0;
    for (int t = 0; t < ti; ++t) s += bf ? t / 2 + 1 : t + 1;
    return s + q;
}
constexpr int tb_blocks(int C, bool bf) { return tb_block(C / 16, 0, bf); }

// ---------------------------------------------------------------------------
// Chunk metadata.  A chunk slot is one chunk of one sequence (shared by all
// heads).  Fixed-length batches compute it; packed batches read a table
// built on the device from cu_seqlens.
// ---------------------------------------------------------------------------
struct ChunkInfo {
    int seq;    // sequence index
    int t0;     // first token, flat index into the [B*T] token axis
    int len;    // valid tokens in this chunk (0 = unused slot)
};

struct SeqGeom {
    const int* table;        // varlen: [slots][4] = {seq, t0, len, pad}; NULL for fixed length
    const int* seq_slot;     // varlen: [N+1] first slot of each sequence
    const int* bounds;       // varlen: [N+1] clamped token offsets of the sequences
    const int* order;        // varlen: [N] sequences by chunk count, longest first (the
                             // scan's dispatch order); NULL: in index order
    int T;                   // fixed: tokens per sequence
    int chunks_per_seq;      // fixed: ceil(T / C)
    int C;
    // fixed length, split into spans of span_chunks chunks (0: not split): the
    // scan's sequence index s is then span s % spans of sequence s / spans
    int span_chunks, spans;
};

__device__ __forceinline__ ChunkInfo chunk_info(const SeqGeom& g, int slot) {
    ChunkInfo ci;
    if (g.table) {
        const int4 e = reinterpret_cast<const int4*>(g.table)[slot];
        ci.seq = e.x; ci.t0 = e.y; ci.len = e.z;
    } else {
        const int s = slot / g.chunks_per_seq, c = slot - s * g.chunks_per_seq;
        ci.seq = s;
        ci.t0 = s * g.T + c * g.C;
        const int rem = g.T - c * g.C;
        ci.len = rem < g.C ? rem : g.C;
    }
    return ci;
}

}  // namespace gdn
