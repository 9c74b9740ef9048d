// Device-side building blocks shared by the gfx950 decode kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla {

constexpr int kDqk = 576;          // latent 512 + RoPE 64
constexpr int kDv = 512;
constexpr int kBlock = 64;         // cache page = KV tile, in tokens
constexpr int kHeadsPerWG = 128;   // query heads per workgroup
constexpr int kWaves = 8;          // two per SIMD
constexpr int kThreads = kWaves * 64;
constexpr int kSubTok = 32;        // tokens per compute tile (half a page)
constexpr int kRowBytes = kDqk * 2;          // 1152
constexpr int kRowChunks = kRowBytes / 16;   // 72 chunks of 16 B
constexpr int kTileBytes = kBlock * kRowBytes;  // 73728
constexpr int kFp8RowBytes = 656;
constexpr int kMetaHeader = 8;
constexpr int kMetaRec = 5;
constexpr int32_t kMetaMagic = 0x4D4C4131;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef const __attribute__((address_space(1))) void gbl_void_t;

// LDS tile layout (32 tokens x 72 chunks of 16 bytes): chunk c of token t
// lives at chunk index 32c + (t ^ f(c)), f(c) = 4(c & 1) + 8((c >> 1) & 1),
// i.e. column-major with an XOR on the token.  Consequences:
//  - a direct-to-LDS load instruction writes 64 consecutive chunks = columns
//    2k and 2k+1, so lane l reads token (l & 31) ^ f(2k + (l >> 5)) and its
//    source offset is a per-lane constant plus 32k bytes;
//  - 16 lanes reading one column for 16 consecutive tokens (the K operand)
//    touch 16 distinct 16-byte bank slots;
//  - the transposed V read (4 tokens x 2 columns per 16 lanes, the next 16
//    lanes two columns further) touches 16 distinct slots per 32 lanes.
__device__ __forceinline__ int col_xor(int c) { return 4 * (c & 1) + 8 * ((c >> 1) & 1); }
__device__ __forceinline__ int lds_chunk(int t, int c) { return 32 * c + (t ^ col_xor(c)); }

// Load of a wave-uniform value through the constant address space: a scalar
// load (s_load, counted by lgkmcnt), so waiting for it never waits for the
// vector loads that stream KV tiles.  Only for memory the kernel never writes.
template <class T>
__device__ __forceinline__ T sload(const T* p) {
    return *(const __attribute__((address_space(4))) T*)(p);
}

// A field of the kernel's argument struct (which sits at offset 0 of the
// kernarg segment), loaded where it is used: the asm hides the pointer from
// the optimiser, so the load is not hoisted to the kernel's start and the
// value holds no scalar register across the kernel's main loop.
template <class T>
__device__ __forceinline__ T kernarg_at(size_t off) {
    const __attribute__((address_space(4))) char* p =
        (const __attribute__((address_space(4))) char*)__builtin_amdgcn_kernarg_segment_ptr();
    __asm__ volatile("" : "+s"(p));
    return *(const __attribute__((address_space(4))) T*)(p + off);
}
#define MLA_LATE_ARG(Struct, field) mla::kernarg_at<decltype(Struct::field)>(offsetof(Struct, field))

__host__ __device__ __forceinline__ int visible_len(int L, int s_q, int i, int causal) {
    if (!causal) return L;
    int v = L - s_q + 1 + i;
    return v < 0 ? 0 : (v > L ? L : v);
}

// Clamp a cache length read from device memory to what the block table holds.
__host__ __device__ __forceinline__ int clamp_len(int L, int max_blocks) {
    int cap = max_blocks * kBlock;
    return L < 0 ? 0 : (L > cap ? cap : L);
}

// Physical cache row of a KV slot, or -1 if the slot is masked.
// Dense: slot = logical token of request b, read through its page table; a
// page id outside [0, num_blocks) masks its whole page.  Sparse: slot = top-k
// entry holding page*64 + offset; entries < 0 or >= num_rows are masked.
__device__ __forceinline__ bool page_ok(int page, int64_t num_rows) {
    return page >= 0 && (int64_t)page * kBlock < num_rows;
}
__device__ __forceinline__ int64_t row_in_page(int page, int tok, int tok_valid, int64_t num_rows) {
    return (tok < tok_valid && page_ok(page, num_rows)) ? (int64_t)page * kBlock + tok : -1;
}
__device__ __forceinline__ int64_t sparse_entry_row(int64_t r, int64_t num_rows) {
    return (r < 0 || r >= num_rows) ? -1 : r;
}

// Top-k slots item j attends to: its first topk_length[j] entries (clamped to
// [0, topk]), or all topk without a length array.
__host__ __device__ __forceinline__ int topk_slots(int len, int topk) {
    return len < 0 ? 0 : (len > topk ? topk : len);
}

struct RowResolver {
    const int32_t* block_table;    // dense
    const int32_t* lengths;        // dense: cache_seqlens [batch]; sparse: topk_length [batch*s_q] or null
    const int32_t* indices;        // sparse
    int s_q, max_blocks, topk, causal;
    int64_t num_rows;

    // number of KV slots of item j (dense: causal-visible tokens; sparse: topk
    // or the item's top-k length)
    __device__ __forceinline__ int slots(int j) const {
        if (topk > 0) return lengths ? topk_slots(lengths[j], topk) : topk;
        int b = j / s_q, i = j - b * s_q;
        return visible_len(clamp_len(lengths[b], max_blocks), s_q, i, causal);
    }
    __device__ __forceinline__ int page(int j, int tile) const {
        return block_table[(int64_t)(j / s_q) * max_blocks + tile];
    }
    // wave-uniform variants (scalar loads)
    __device__ __forceinline__ int slots_uniform(int j) const {
        if (topk > 0) return lengths ? topk_slots(sload(lengths + j), topk) : topk;
        int b = j / s_q, i = j - b * s_q;
        return visible_len(clamp_len(sload(lengths + b), max_blocks), s_q, i, causal);
    }
    __device__ __forceinline__ int page_uniform(int j, int tile) const {
        return sload(block_table + (int64_t)(j / s_q) * max_blocks + tile);
    }
    __device__ __forceinline__ int64_t row(int j, int slot, int nslots) const {
        if (slot >= nslots) return -1;
        if (topk > 0) return sparse_entry_row(indices[(int64_t)j * topk + slot], num_rows);
        return row_in_page(page(j, slot >> 6), slot & 63, nslots - (slot & ~63), num_rows);
    }
};

// max(a, b, c) as one v_max3_f32.  Written as assembly because the compiler
// would first quiet signalling NaNs in every input with an extra max(x, x);
// scores out of MFMAs hold no signalling NaN.
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
    float r;
    __asm__("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

__device__ __forceinline__ float wave_max_pair(float x) {
    // lanes l and l^32 hold one head's two halves; after the swap both lanes
    // see both values
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float wave_sum_pair(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace mla
