// Split-KV partial-attention kernel for absorbed-MLA decode on gfx950: the
// top-k (sparse) calls and the quantised caches (656-, 528- and 288-byte
// records).  Dense decode over a bf16 cache runs the 64-heads-per-workgroup
// kernel of decode64.hip instead.
//
// One workgroup = 128 query heads x one scheduler partition (a contiguous run
// of 64-token KV pages, possibly spanning several items), so every cache page
// is read from HBM once per query token.  Eight waves, two per SIMD, 256
// registers each; wave w owns head block hb = w >> 1 (32 heads) and half
// kh = w & 1.  Each page is computed as two 32-token tiles:
//
//   fill   tiles are copied global -> LDS with 16-byte loads that write LDS
//          directly (three LDS buffers: the tile being multiplied, the
//          previous one for PV, the next one landing).  Quantised records
//          (FP8, FP4) are copied raw and dequantised in place in LDS by the
//          waves that copied them.  Masked tokens fall outside the buffer
//          range (or read a zero row) and land as zeros;
//   QK     the two waves of a head block split the 576 dims: wave kh runs
//          S^T = K Q^T over latent dims 256*kh.. and half of the RoPE dims
//          with v_mfma_f32_32x32x16_bf16 (Q in registers, RoPE part of Q in
//          LDS), then the pair adds its partial S^T through LDS.  Tokens sit
//          on the MFMA rows, so each lane holds one head's scores;
//   soft   both waves of a head block run the same exact online softmax
//          (running max updated on every increase, p = exp2(s*c - m) in fp32,
//          l sums the fp32 p, P rounded to bf16 for the PV product) and
//          rescale their part of O;
//   PV     wave kh accumulates O^T for dims 256*kh.. of its 32 heads; the
//          transposed V operand is read straight from the row-major LDS tile
//          with ds_read_b64_tr_b16 and P^T is the wave's own S^T registers.
//
// The waves form two groups (0-3 and 4-7, one wave of each per SIMD) that run
// the same step sequence one step apart: while one group issues the MFMAs of
// PV and QK, the other runs the softmax, so the matrix and vector units of a
// SIMD work at the same time.
//
// Items whose KV range sits in one partition write out/lse directly; split
// items write normalised partials for the combine kernel: float32 when the
// output is float32, otherwise float16 scaled per lane by a power of two.

#include "common.h"
#include "kernels.h"
#include "wave_sched.h"

namespace mla {

constexpr int kSubBytes = kSubTok * kRowBytes;   // 36864
constexpr int kNBuf = 3;

template <int V>
struct IntC {
    static constexpr int value = V;
};

// The small arrays come first: LDS instructions encode at most a 16-bit
// immediate offset, so arrays addressed with many constant offsets must sit
// below 64 KiB to share one address register.
struct __attribute__((aligned(16))) Smem {
    f32x4 xs[4][2][4][64];                  // partial S^T [head block][dim half][register quad][lane]
    bf16x8 qr[4][4][64];                    // RoPE part of Q as B fragments [head block][k-step][lane]
    int rows[4][kSubTok];                   // sparse: row ids of upcoming tiles (ring of 4)
    float f8scale[8][64];                   // FP8: per-wave scales of the tile being converted (lanes 32.. pad)
    int seg_tab[kMaxFusedItems];            // fused schedule: item j's split count << 16 | first split slot
    unsigned char tile[kNBuf][kSubBytes];   // 32-token KV tiles (bf16, swizzled)
};

__device__ __forceinline__ bf16x4 tr_read(const unsigned char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(p));
}

// Byte offset of LDS tile buffer ``idx``, hidden from the optimiser so that it
// does not precompute one set of lane addresses per buffer (addresses above
// 64 KiB cannot use the instruction's immediate offset and would each hold a
// register); each step adds the uniform offset to a few lane bases instead.
__device__ __forceinline__ int opaque_tile_offset(int idx) {
    int off = idx * (kSubTok * kRowBytes);
    __asm__ volatile("" : "+s"(off));
    return off;
}

// Lane id recomputed where it is used (bit count of an all-ones mask below
// this lane).  The mask goes through an empty asm statement so that the
// compiler cannot hoist the result out of a loop and hold (or spill) it.
__device__ __forceinline__ int lane_id() {
    unsigned m = ~0u;
    __asm__ volatile("" : "+s"(m));
    return (int)__builtin_amdgcn_mbcnt_hi(m, __builtin_amdgcn_mbcnt_lo(m, 0u));
}

__device__ __forceinline__ bf16x8 pack8(const float* v) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (__bf16)v[e];
    return r;
}

// Buffer resource for untyped loads: base, stride (bytes, struct loads only),
// num_records (bytes for raw loads, records for struct loads; accesses beyond
// it return zeros), 32-bit data format.  Built from uniform values, so it
// lives in scalar registers.
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, int stride, int num_records) {
    const uint64_t p = (uint64_t)base;
    i32x4 r;
    r[0] = (int)(uint32_t)p;
    r[1] = (int)(((uint32_t)(p >> 32) & 0xffffu) | ((uint32_t)stride << 16));
    r[2] = num_records;
    r[3] = 0x00020000;
    return r;
}

// 16-byte-per-lane global -> LDS copies (one wave instruction writes 1 KiB of
// LDS at M0).  They are issued through inline assembly so that the compiler
// does not treat them as pending LDS stores: it would otherwise wait for every
// in-flight tile load before the next LDS read of any other tile.  The kernel
// orders them itself: s_waitcnt vmcnt(0) by each wave that issued copies, then a workgroup
// barrier, before a filled tile is read.
// The immediate offset moves both the global source and the LDS destination
// (LDS address = M0 + offset + 16 * lane), so M0 is set to the destination
// minus the immediate.
template <int IMM>
__device__ __forceinline__ void dma_raw_x4(const i32x4& rs, int voff, int lds) {
    __asm__ volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen offset:%3 lds"
                     :: "s"(lds - IMM), "v"(voff), "s"(rs), "i"(IMM) : "memory", "m0");
}

// Gathered (sparse) rows are copied with a 64-bit address per lane, so caches
// beyond 4 GiB are reached (a buffer offset is 32-bit).  As for the buffer
// copies, the immediate offset moves both the source and the LDS destination
// (LDS address = M0 + offset + 16 * lane for x4, 4 * lane for x1).  An invalid
// row reads the zero row below instead, so it lands as zeros like an
// out-of-range buffer load.
__device__ __align__(16) unsigned char g_zero_row[kRowBytes];   // never written
template <int IMM>
__device__ __forceinline__ void dma_global_x4(const unsigned char* src, int lds) {
    __asm__ volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off offset:%2"
                     :: "s"(lds - IMM), "v"(src), "i"(IMM) : "memory", "m0");
}
__device__ __forceinline__ void dma_global_x1(const unsigned char* src, int lds) {
    __asm__ volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off"
                     :: "s"(lds), "v"(src) : "memory", "m0");
}
__device__ __forceinline__ const unsigned char* bf16_row_addr(const unsigned char* kv, int row, int off) {
    return (row >= 0 ? kv + (int64_t)row * kRowBytes : g_zero_row) + off;
}

// ---- bf16 tile fill: 36 pieces of 1 KB = LDS columns 2k, 2k+1; wave w issues
// pieces w, w+8, w+16, w+24 and, for w < 4, 32+w.  All pieces of a wave have
// k & 1 = w & 1, so lane l always reads token ft = (l & 31) ^ (4 half + 8 (w & 1))
// and column 2k + half: source offset ft*1152 + 16 half + 32k.

// dense: the tile is one half of a 64-token page; tokens >= tok_valid are masked
// ``dst`` is the LDS byte address of the tile buffer.
__device__ __forceinline__ void fill_dense(int dst, const unsigned char* kv, int page, int sub,
                                           int tok_valid, int64_t num_rows, int fbase, int wave) {
    const bool ok = page_ok(page, num_rows);
    int nvalid = tok_valid < kSubTok ? tok_valid : kSubTok;
    if (!ok || nvalid < 0) nvalid = 0;
    const unsigned char* base = kv + (ok ? (int64_t)page * kTileBytes + sub * kSubBytes : 0);
    const i32x4 rs = buffer_rsrc(base, 0, nvalid * kRowBytes);
    const int l0 = dst + wave * 1024;
    dma_raw_x4<0>(rs, fbase + 32 * wave, l0);
    dma_raw_x4<256>(rs, fbase + 32 * wave, l0 + 8 * 1024);
    dma_raw_x4<512>(rs, fbase + 32 * wave, l0 + 16 * 1024);
    dma_raw_x4<768>(rs, fbase + 32 * wave, l0 + 24 * 1024);
    if (wave < 4) dma_raw_x4<0>(rs, fbase + 32 * (32 + wave), l0 + 32 * 1024);
}

// sparse: the lane's row id from the LDS ring (-1 = masked -> index out of range)
// sparse: ``src`` is this lane's source (row start + 16 half + 32 wave)
__device__ __forceinline__ void fill_sparse(int dst, const unsigned char* src, int wave) {
    const int l0 = dst + wave * 1024;
    dma_global_x4<0>(src, l0);
    dma_global_x4<256>(src, l0 + 8 * 1024);
    dma_global_x4<512>(src, l0 + 16 * 1024);
    dma_global_x4<768>(src, l0 + 24 * 1024);
    if (wave < 4) dma_global_x4<1024>(src, l0 + 32 * 1024);
}

// ---- FP8 tile fill: the raw 656-B records are copied into the tile buffer
// and dequantised there.  The 32 code bytes of part p (latent dims
// 32p..32p+31) of every token land in LDS columns 4p+2 and 4p+3, two of the
// four chunks their bf16 values end in; the RoPE bytes (already bf16) land in
// columns 64..71, their final place; the scale of dims 128s.. lands in a
// per-wave array.  Wave w copies and converts parts 2w and 2w+1 of all 32
// tokens, so every raw byte is read by the lane that copied it, after that
// wave's own vmcnt wait, and overwritten only by that lane.
template <int IMM>
__device__ __forceinline__ void dma_raw_x1(const i32x4& rs, int voff, int lds) {
    __asm__ volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen offset:%3 lds"
                     :: "s"(lds - IMM), "v"(voff), "s"(rs), "i"(IMM) : "memory", "m0");
}
// ``rec``: record bytes (656, or 528 for the 512-wide head)
__device__ __forceinline__ const unsigned char* fp8_row_addr(const unsigned char* kv, int row, int off, int rec) {
    return (row >= 0 ? kv + (int64_t)row * rec : g_zero_row) + off;
}

// LDS token slot of lane l in a copy of columns (c, c+1): column c + (l >> 5),
// slot l & 31, token = slot ^ col_xor(column)
__device__ __forceinline__ int fp8_code_token(int l) { return (l & 31) ^ (8 + 4 * (l >> 5)); }   // c = 4p+2
__device__ __forceinline__ int fp8_rope_token(int l, int w) { return (l & 31) ^ (4 * (l >> 5) + 8 * (w & 1)); }

// 288-byte FP4 record: wave w copies the code chunks of parts 2w, 2w+1 (16 B,
// 32 e2m1 values each) into columns 8w+3 and 8w+4 with one instruction, so
// lane l reads token (l & 31) ^ col_xor(8w + 3 + (l >> 5)).
__device__ __forceinline__ int fp4_code_token(int l) { return (l & 31) ^ ((l >> 5) ? 0 : 12); }

// e2m1 pairs -> fp32 (exact: the conversion with scale 1, the even-indexed
// value from the low nibble), x the e4m3 scale of its group of 16 (exact), ->
// bf16 (exact: at most five significant bits), in place: lane l of wave w
// converts part p = 2w + (l >> 5) of token l & 31, whose code chunk sits in
// column 4p + 3 (half 0) or 4p (half 1) and is read before any write.  The
// scale word of a token holds the e4m3 scales of groups 4w..4w+3.
__device__ __forceinline__ void fp4_convert(unsigned char* dst, const float* scales, int w, int l) {
    const int t = l & 31, half = l >> 5, p = 2 * w + half;
    const i32x4 raw = *(const i32x4*)(dst + lds_chunk(t, half ? 4 * p : 4 * p + 3) * 16);
    const int sw = (int)(__float_as_uint(scales[t]) >> (16 * half));
    const auto sc = __builtin_amdgcn_cvt_pk_f32_fp8(sw, false);      // scales of values 0..15, 16..31
#pragma unroll
    for (int h = 0; h < 4; ++h) {                                     // output chunk h: values 8h..8h+7
        const float s = sc[h >> 1];
        const auto f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(raw[h], 1.0f, 0);
        const auto f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(raw[h], 1.0f, 1);
        const auto f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(raw[h], 1.0f, 2);
        const auto f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(raw[h], 1.0f, 3);
        float v[8] = {f0[0] * s, f0[1] * s, f1[0] * s, f1[1] * s, f2[0] * s, f2[1] * s, f3[0] * s, f3[1] * s};
        *(bf16x8*)(dst + lds_chunk(t, 4 * p + h) * 16) = pack8(v);
    }
}

// e4m3fn -> fp32 (exact), x scale in fp32, -> bf16 (round to nearest even), in
// place: lane l of wave w converts part 2w + (l >> 5) of token l & 31.  The
// scale word of a token holds one float32 (656-byte record: dims 128s..) or,
// for the 528-byte record, four e8m0 bytes of parts 4s..4s+3 (32 dims each).
template <bool E8M0>
__device__ __forceinline__ void fp8_convert(unsigned char* dst, const float* scales, int w, int l) {
    const int t = l & 31, p = 2 * w + (l >> 5);
    const i32x4 raw[2] = {*(const i32x4*)(dst + lds_chunk(t, 4 * p + 2) * 16),
                          *(const i32x4*)(dst + lds_chunk(t, 4 * p + 3) * 16)};
    if constexpr (E8M0) {
        // A power-of-two scale: the scaled conversion takes the scale's exponent
        // field (e << 23 as a float: 2^(e-127), e = 0 meaning 2^-127 and e = 255
        // NaN) and gives fp8 x 2^(e-127) rounded to bf16, two values per
        // instruction; it equals the three-step path below bit for bit for every
        // code and exponent (checked exhaustively on the hardware).
        const float sce = __uint_as_float(((__float_as_uint(scales[t]) >> (8 * (p & 3))) & 0xFFu) << 23);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            bf16x8 o[2];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const auto lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[h][q], sce, false);
                const auto hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[h][q], sce, true);
                o[q >> 1][4 * (q & 1) + 0] = lo[0];
                o[q >> 1][4 * (q & 1) + 1] = lo[1];
                o[q >> 1][4 * (q & 1) + 2] = hi[0];
                o[q >> 1][4 * (q & 1) + 3] = hi[1];
            }
            *(bf16x8*)(dst + lds_chunk(t, 4 * p + 2 * h) * 16) = o[0];
            *(bf16x8*)(dst + lds_chunk(t, 4 * p + 2 * h + 1) * 16) = o[1];
        }
        return;
    }
    const float sc = scales[t];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        float v[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int word = raw[h][q];
            auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(word, false);
            auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(word, true);
            v[4 * q + 0] = lo[0] * sc;
            v[4 * q + 1] = lo[1] * sc;
            v[4 * q + 2] = hi[0] * sc;
            v[4 * q + 3] = hi[1] * sc;
        }
        *(bf16x8*)(dst + lds_chunk(t, 4 * p + 2 * h) * 16) = pack8(v);
        *(bf16x8*)(dst + lds_chunk(t, 4 * p + 2 * h + 1) * 16) = pack8(v + 8);
    }
}

// Workgroup barrier for LDS traffic only.  __syncthreads() also orders global
// memory, which makes the compiler wait for every in-flight tile load
// (vmcnt(0)) at each barrier; here each wave first waits for its own LDS
// stores (lgkmcnt(0)) and the tile loads are waited for explicitly.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt, expcnt untouched
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

// Instruction order of the MFMA step, pinned for the scheduler: the LDS
// reads of the first kMstepLookahead operations, then each MFMA followed by
// the reads of the operation kMstepLookahead ahead (two for a PV step or a
// RoPE step, one for a latent QK step), then the four stores of the partial
// scores.
constexpr int kSchedMfma = 0x008, kSchedDsRead = 0x100, kSchedDsWrite = 0x200;
constexpr int kMstepLookahead = 3;   // operations whose operands are in flight
constexpr int mstep_reads(int i) { return (i < 16 || i >= 32) ? 2 : 1; }

template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(IntC<B>{});
        static_for<B + 1, E>(f);
    }
}

template <int I, int I1>
__device__ __forceinline__ void mstep_schedule() {
    if constexpr (I < I1) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        if constexpr (I + kMstepLookahead < I1)
            __builtin_amdgcn_sched_group_barrier(kSchedDsRead, mstep_reads(I + kMstepLookahead), 0);
        mstep_schedule<I + 1, I1>();
    }
}

template <int I, int I1>
constexpr int mstep_first_reads() {
    if constexpr (I < I1) return mstep_reads(I) + mstep_first_reads<I + 1, (I1 < I + kMstepLookahead ? I1 : I + kMstepLookahead)>();
    else return 0;
}

template <int I0, int I1, bool QK>
__device__ __forceinline__ void mstep_schedule_all() {
    constexpr int first = mstep_first_reads<I0, (I1 < I0 + kMstepLookahead ? I1 : I0 + kMstepLookahead)>();
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, first, 0);
    mstep_schedule<I0, I1>();
    if constexpr (QK) __builtin_amdgcn_sched_group_barrier(kSchedDsWrite, 4, 0);
}

// The same order when a tile-copy piece follows each of the first
// kMstepPieces operations.  Each piece (inline assembly) is fenced by
// scheduling barriers, without which the MFMAs, having no memory operands,
// drift across it and the reads lose their lookahead; the pins are then given
// region by region.  Region 0 holds the first reads and operation 0, region
// i < kMstepPieces operation i, the last region the remaining operations and
// the score stores.
constexpr int kMstepPieces = 4;   // pieces of each tile copy issued in the MFMA step (of nine)
template <int I>
__device__ __forceinline__ void mstep_schedule_region() {
    if constexpr (I == 0)
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, mstep_first_reads<0, kMstepLookahead>(), 0);
    mstep_schedule<I, I + 1>();
}
template <int I1>
__device__ __forceinline__ void mstep_schedule_tail() {
    mstep_schedule<kMstepPieces, I1>();
    __builtin_amdgcn_sched_group_barrier(kSchedDsWrite, 4, 0);
}

// A tile copy to be issued piecewise: buffer resource, sparse row id, lane
// source offset and LDS address of the wave's first piece.
struct FillCtx {
    bool on;
    i32x4 rs;                    // dense: buffer over the tile's page
    const unsigned char* src;    // sparse: this lane's source
    int vo, l0;
};

// KVF: cache format, 0 = bf16 rows of 576, 1 = 656-byte FP8 records, 2 =
// 528-byte FP8 records of the 512-wide head (K = V = all 512 dims, no RoPE part).
// DFUSED (dense calls): the schedule is computed in the kernel; a separate
// instantiation, so that the dense kernel that reads the metadata carries no
// code of the other path.  Sparse calls choose at run time (a.fused).
template <bool SPARSE, int KVF, bool DFUSED = false>
__global__ void __launch_bounds__(kThreads, 1) decode_kernel(const DecodeArgs a) {
    constexpr bool FP8 = KVF != 0;                            // quantised cache (copied raw, dequantised in LDS)
    constexpr bool FP4 = KVF == 3;
    constexpr bool D512 = KVF >= 2;                           // 512-wide head, K = V
    constexpr int kQRow = D512 ? 1024 : kRowBytes;            // q row bytes
    constexpr int kRec = FP4 ? 288 : D512 ? 528 : kFp8RowBytes;   // record bytes
    static_assert(!D512 || SPARSE, "the 528- and 288-byte records are read through top-k indices");
    __shared__ Smem sm;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // Two groups of four waves run the same step sequence one step apart
    // (group 1 lags).  The dispatcher puts wave w on SIMD w % 4, so every SIMD
    // hosts one wave of each group: while one runs MFMA work the other runs
    // VALU work.  Waves w and w^1 (same group, different SIMDs) share head
    // block hb and exchange partial scores.
    const int grp = wave >> 2;
    const int hb = wave >> 1;         // head block: heads 32*hb .. +31 of the workgroup
    const int kh = wave & 1;          // half: QK dims and PV output dims
    const int l32 = lane & 31;
    const int half = lane >> 5;

    // workgroup -> (partition, head block).  The dispatcher deals workgroups to
    // the 8 XCDs round-robin; give each XCD a contiguous run of partitions so
    // neighbouring partitions (same item, or the causal tokens of one request)
    // share an L2.
    int part, hblk;
    {
        const int G = a.num_parts * a.n_hblk;
        const int x = blockIdx.x & 7, k = blockIdx.x >> 3;
        const int q8 = G >> 3, r8 = G & 7;
        const int lin = x * q8 + min(x, r8) + k;
        part = lin / a.n_hblk;
        hblk = lin - part * a.n_hblk;
    }

    const int32_t* rec = a.meta + kMetaHeader + kMetaRec * part;
    // split offsets, read once per segment from a pointer loaded there
    auto so_at = [&](int k) __attribute__((always_inline)) -> int {
        return sload(MLA_LATE_ARG(DecodeArgs, meta) + kMetaHeader + kMetaRec * MLA_LATE_ARG(DecodeArgs, num_parts) + k);
    };
    const int N = a.batch * a.s_q;
    // This partition's record: read from the scheduler's metadata, or (fused)
    // computed by every wave from the lengths (top-k lengths, or the cache
    // lengths of a dense call) with the scheduler's arithmetic.  Fused, wave 0
    // also writes the schedule back and keeps each item's split count and first
    // split slot in LDS for the segments' epilogues.
    const bool fused = SPARSE ? a.fused != 0 : DFUSED;
    int jb, tbeg, je, tend, slot0;
    if (fused) {
        const int ln = lane_id();
        const int R = N <= 64 ? 1 : N <= 128 ? 2 : 4;
        WaveSched ws;
        wave_schedule_any(a, SPARSE ? a.topk_length : a.cache_seqlens, N, part, ln, R, ws);
        // uniform by construction; readfirstlane makes that visible to the compiler
        jb = __builtin_amdgcn_readfirstlane(ws.jb);
        tbeg = __builtin_amdgcn_readfirstlane(ws.tbeg);
        je = __builtin_amdgcn_readfirstlane(ws.je);
        tend = __builtin_amdgcn_readfirstlane(ws.tend);
        slot0 = __builtin_amdgcn_readfirstlane(ws.slot0);
        if (wave == 0) {
            wave_schedule_store(a, N, part, ln, R, ws, hblk == 0, blockIdx.x == 0);
            // entries past N (at most 64 * 4 = kMaxFusedItems in all) are never read
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (u < R) sm.seg_tab[ln * R + u] = (ws.NS[u] << 16) | ws.SO[u];
        }
    } else {
        jb = sload(rec + 0); tbeg = sload(rec + 1); je = sload(rec + 2); tend = sload(rec + 3);
        slot0 = sload(rec + 4);
    }
    const int H = a.h_q;
    const float c = a.scale_log2;
    const unsigned char* kv = (const unsigned char*)a.kv;

    RowResolver rr{a.block_table, SPARSE ? a.topk_length : a.cache_seqlens, a.indices, a.s_q, a.max_blocks,
                   SPARSE ? a.topk : 0,
                   a.causal, a.num_rows};

    const int head = hblk * kHeadsPerWG + hb * 32 + l32;   // this lane's head
    const bool head_ok = head < H;

    // bf16 fill: the token a lane copies, its dense source offset (+32k) and its
    // sparse column offset (+32k), rebuilt from the lane id where used so that
    // they are not held across the tile loop
    auto ftok = [&]() __attribute__((always_inline)) -> int {
        const int ln = lane_id();
        return (ln & 31) ^ (4 * (ln >> 5) + 8 * (wave & 1));
    };
    auto fbase = [&]() __attribute__((always_inline)) -> int { return ftok() * kRowBytes + 16 * (lane_id() >> 5); };
    auto fcol = [&]() __attribute__((always_inline)) -> int { return 16 * (lane_id() >> 5); };

    // LDS byte offsets inside a tile (see lds_chunk).  K operand: token l32,
    // column 32kh + 2kk + half -> kb[kk & 1] + 1024 kk + 16384 kh.  V^T
    // operand (transposed read): source token 16 j2 + 4 (gq >> 1) + (i16 >> 2)
    // (+8 for the second read), column 32kh + 4d + 2 (gq & 1) + ((i16 & 3) >> 1)
    // -> vb[second] + 256 j2 + 2048 d + 16384 kh.
    int kb[2], vb[2];
    {
#pragma unroll
        for (int p = 0; p < 2; ++p) kb[p] = 16 * (l32 ^ (4 * half + 8 * p)) + 512 * half;
        const int gq = lane >> 4, i16 = lane & 15;
        const int cl = 2 * (gq & 1) + ((i16 & 3) >> 1);
        const int f = 4 * ((i16 >> 1) & 1) + 8 * (gq & 1);
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int t = 4 * (gq >> 1) + (i16 >> 2) + 8 * r;
            vb[r] = 512 * cl + 16 * (t ^ f) + 8 * (i16 & 1);
        }
    }

    for (int j = jb; j <= je && j < N; ++j) {
        // the item's length, read with s_q loaded here (a divisor held across the
        // tile loop would keep its reciprocal in scalar registers)
        const int sq_s = MLA_LATE_ARG(DecodeArgs, s_q);
        const RowResolver rrs{nullptr, SPARSE ? MLA_LATE_ARG(DecodeArgs, topk_length) : MLA_LATE_ARG(DecodeArgs, cache_seqlens),
                              nullptr, sq_s, a.max_blocks, SPARSE ? a.topk : 0, a.causal, a.num_rows};
        const int nslots = rrs.slots_uniform(j);
        const int ntile_j = (nslots + 63) >> 6;
        const int t0 = (j == jb && tbeg > 0) ? tbeg : 0;
        int t1 = (j == je) ? tend : ntile_j;
        if (t1 > ntile_j) t1 = ntile_j;
        if (t0 >= t1) continue;
        const int g0 = 2 * t0;                                    // first 32-token tile
        const int gend = min(2 * t1, (nslots + kSubTok - 1) / kSubTok);
        const int ns = gend - g0;

        // ---- prologue: page ids, Q and tile 0 are requested together ----
        // dense: page ids of 64 consecutive pages of item j, one per lane, read
        // with v_readlane.  A scalar load here would be waited for with
        // lgkmcnt(0), which also drains every outstanding LDS operation.
        const int b_item = j / sq_s;
        const int npages_item = (nslots + kBlock - 1) / kBlock;
        int pt_base = g0 >> 1, pt_v = 0;
        auto load_pages = [&](int first) __attribute__((always_inline)) {
            pt_base = first;
            const int pi = first + lane;
            pt_v = pi < npages_item ? MLA_LATE_ARG(DecodeArgs, block_table)[(int64_t)b_item * a.max_blocks + pi] : 0;
            // waited for here, so that no later read of pt_v waits for other loads
            __builtin_amdgcn_s_waitcnt(0x0F70);
        };
        if (!SPARSE) load_pages(g0 >> 1);
        auto page_of = [&](int g) __attribute__((always_inline)) {
            return __builtin_amdgcn_readlane(pt_v, (g >> 1) - pt_base);
        };

        // Q: latent dims 256*kh.. in registers, RoPE part to LDS.  The lane
        // terms of the addresses are rebuilt from the lane id (mbcnt), so that
        // they are not kept (or spilled) across the item loop.
        bf16x8 qf[16], qrv[2];
        {
            const int tid_o = wave * 64 + lane_id();
            const int head_o = hblk * kHeadsPerWG + hb * 32 + (tid_o & 31);
            const int half_o = (tid_o >> 5) & 1;
            const bf16x8* qp = (const bf16x8*)((const unsigned char*)MLA_LATE_ARG(DecodeArgs, q) +
                                               ((int64_t)j * H + (head_o < H ? head_o : 0)) * kQRow);
#pragma unroll
            for (int kk = 0; kk < 16; ++kk) {
                bf16x8 v = qp[32 * kh + 2 * kk + half_o];
                if (!head_ok) v = bf16x8{};
                qf[kk] = v;
            }
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int idx = tid_o + kThreads * e;        // 0..1023 = [hb2][kr][lane]
                const int ln = idx & 63, kr = (idx >> 6) & 3, hb2 = idx >> 8;
                const int hq = hblk * kHeadsPerWG + hb2 * 32 + (ln & 31);
                bf16x8 v = {};
                if (!D512 && hq < H)
                    v = ((const bf16x8*)((const unsigned char*)MLA_LATE_ARG(DecodeArgs, q) + ((int64_t)j * H + hq) * kQRow))[64 + 2 * kr + (ln >> 5)];
                qrv[e] = v;
            }
        }

        f32x16 acc[8];
#pragma unroll
        for (int d = 0; d < 8; ++d) acc[d] = f32x16{};
        // cm_run: the running max of the scores times c (c > 0), as rounded in
        // the step that raised it.  When the max does not rise the exponent of
        // alpha is exactly 0 and alpha exactly 1, which lets the rescale be
        // skipped.
        float cm_run = -INFINITY, l_run = 0.f;

        int pg0 = 0, pg1 = 0, pg2 = 0;
        if (!SPARSE) {
            pg0 = page_of(g0);
            pg1 = ns > 1 ? page_of(g0 + 1) : 0;
            pg2 = ns > 2 ? page_of(g0 + 2) : 0;
        }
        if (SPARSE && wave == 0 && lane < kSubTok) {
#pragma unroll
            for (int u = 0; u < 2; ++u)
                if (u < ns) sm.rows[u][lane] = (int)rr.row(j, (g0 + u) * kSubTok + lane, nslots);
        }
        if (SPARSE || FP8) lds_barrier();   // row ids of tiles 0 and 1 for every wave

        auto issue_fill = [&](int it, int page) __attribute__((always_inline)) {
            const int g = g0 + it;
            const int dst = (int)(size_t)(lds_void_t*)&sm.tile[0][0] + opaque_tile_offset(it % kNBuf);
            if (SPARSE) fill_sparse(dst, bf16_row_addr(kv, sm.rows[it & 3][ftok()], fcol() + 32 * wave), wave);
            else {
                const int ln = lane_id();
                const int fb = ((ln & 31) ^ (4 * (ln >> 5) + 8 * (wave & 1))) * kRowBytes + 16 * (ln >> 5);
                fill_dense(dst, kv, page, g & 1, nslots - g * kSubTok, a.num_rows, fb, wave);
            }
        };
        // FP8: copy the raw records of tile it (page ``page``) into its buffer.
        // With it >= ns the copies run on an empty range and write zeros into
        // that buffer, which no step reads any more.
        auto fp8_copy = [&](int it, int page) __attribute__((always_inline)) {
            const int g = g0 + it;
            const int l = lane_id();
            const int dst = (int)(size_t)(lds_void_t*)&sm.tile[0][0] + opaque_tile_offset(it % kNBuf);
            const int sdst = (int)(size_t)(lds_void_t*)&sm.f8scale[wave][0];
            const int tc = FP4 ? fp4_code_token(l) : fp8_code_token(l), tr = fp8_rope_token(l, wave);
            const int wr = wave & 3;                       // waves w and w+4 copy the same RoPE columns
            const int code_off = FP4 ? 16 * (2 * wave + (l >> 5)) : 64 * wave + 16 * (l >> 5);
            const int rope_off = 528 + 16 * (2 * wr + (l >> 5));
            const int scale_off = FP4 ? 256 + 4 * wave : 512 + 4 * (wave >> 1);
            const int code_lds = dst + (8 * wave + (FP4 ? 3 : 2)) * 512, rope_lds = dst + (64 + 2 * wr) * 512;
            if (SPARSE) {
                const bool live = it < ns;
                const int rc = live ? sm.rows[it & 3][tc] : -1;
                const int rr_ = live ? sm.rows[it & 3][tr] : -1;
                const int rs_ = (live && l < kSubTok) ? sm.rows[it & 3][l] : -1;
                dma_global_x4<0>(fp8_row_addr(kv, rc, code_off, kRec), code_lds);
                if (!FP4) dma_global_x4<0>(fp8_row_addr(kv, rc, code_off + 32, kRec), code_lds + 2048);
                if (!D512) dma_global_x4<0>(fp8_row_addr(kv, rr_, rope_off, kRec), rope_lds);
                dma_global_x1(fp8_row_addr(kv, rs_, scale_off, kRec), sdst);
            } else {
                const bool ok = it < ns && page_ok(page, a.num_rows);
                int nvalid = min(nslots - g * kSubTok, kSubTok);
                if (!ok || nvalid < 0) nvalid = 0;
                const i32x4 rs = buffer_rsrc(kv + (ok ? ((int64_t)page * kBlock + (g & 1) * kSubTok) * kFp8RowBytes : 0),
                                             0, nvalid * kFp8RowBytes);
                dma_raw_x4<0>(rs, tc * kFp8RowBytes + code_off, code_lds);
                dma_raw_x4<32>(rs, tc * kFp8RowBytes + code_off, code_lds + 2048);
                dma_raw_x4<0>(rs, tr * kFp8RowBytes + rope_off, rope_lds);
                dma_raw_x1<0>(rs, l < kSubTok ? l * kFp8RowBytes + scale_off : 0x40000000, sdst);
            }
        };
        auto fp8_dequant = [&](int it) __attribute__((always_inline)) {
            if constexpr (FP4) fp4_convert(sm.tile[0] + opaque_tile_offset(it % kNBuf), sm.f8scale[wave], wave, lane_id());
            else fp8_convert<D512>(sm.tile[0] + opaque_tile_offset(it % kNBuf), sm.f8scale[wave], wave, lane_id());
        };
        // tile 0 lands before step 0
        if (FP8) {
            fp8_copy(0, pg0);
            __builtin_amdgcn_s_waitcnt(0x0F70);
            fp8_dequant(0);
        } else {
            issue_fill(0, pg0);
        }
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int idx = wave * 64 + lane_id() + kThreads * e;   // lane term rebuilt here, not held
            if (!D512) sm.qr[idx >> 8][(idx >> 6) & 3][idx & 63] = qrv[e];
        }
        if (!FP8) __builtin_amdgcn_s_waitcnt(0x0F70);
        lds_barrier();

        // ---- step pipeline ----
        // Per tile t a wave runs an MFMA step M(t) = PV(t-1), QK(t) and a VALU
        // step V(t) = partner exchange, online softmax of tile t and rescale of O;
        // M(ns) is the last PV alone.  Group 0 runs M(t), V(t) in steps 2t,
        // 2t+1; group 1 runs V(t-1), M(t), so on every SIMD one wave issues
        // MFMAs while the other runs the softmax.  Tile t is read in steps
        // 2t..2t+3.  Both groups copy parts of tile t+1 into the buffer of tile
        // t-2 during step 2t; every wave waits for its copies at the end of step
        // 2t+1.  Every step ends with a workgroup barrier.  The
        // group is a compile-time constant so that each wave's step sequence is
        // straight-line code.
        f32x16 s = {};
        bf16x8 p0 = {}, p1 = {};

        // Copy of tile t+1 into the buffer of tile t-2 in step 2t, as nine 1-KiB
        // pieces per wave (wave w of a group copies the pieces w + 4i).  Group 0
        // issues pieces 0..kMstepPieces-1, one after each of its first MFMAs;
        // group 1 issues the rest spread over its softmax step.  Each issuing
        // cost lands on a wave with slack, and group 0's share starts early.
        // In step 0 group 1, which has no other work, issues all nine.
        // With no tile left to copy the pieces still run, on an empty buffer
        // range: they write zeros into the buffer of tile t-2, which no step
        // reads any more.  Keeping them unconditional keeps the softmax step one
        // basic block (a branch around each piece makes the compiler wait for
        // every outstanding copy before the next one).
        auto fill_prepare = [&](int t) __attribute__((always_inline)) -> FillCtx {
            FillCtx f{true, {0, 0, 0, 0}, nullptr, 0, 0};
            const int g = g0 + t + 1;
            const int w = wave & 3;
            const bool live = t + 1 < ns;
            f.l0 = (int)(size_t)(lds_void_t*)&sm.tile[0][0] + opaque_tile_offset((t + 1) % kNBuf) + 1024 * w;
            if (SPARSE) {
                f.src = bf16_row_addr(kv, live ? sm.rows[(t + 1) & 3][ftok()] : -1, fcol() + 32 * w);
            } else if (!live) {
                f.rs = buffer_rsrc(kv, 0, 0);
                f.vo = fbase() + 32 * w;
            } else {
                const bool ok = page_ok(pg1, a.num_rows);
                int nvalid = min(nslots - g * kSubTok, kSubTok);
                if (!ok || nvalid < 0) nvalid = 0;
                f.rs = buffer_rsrc(kv + (ok ? (int64_t)pg1 * kTileBytes + (g & 1) * kSubBytes : 0), 0,
                                   nvalid * kRowBytes);
                f.vo = fbase() + 32 * w;
            }
            return f;
        };
        auto fill_piece = [&](const FillCtx& f, auto i_c) __attribute__((always_inline)) {
            constexpr int i = decltype(i_c)::value;
            if (f.on) {
                if (SPARSE) dma_global_x4<128 * i>(f.src, f.l0 + 4096 * i);
                else dma_raw_x4<128 * i>(f.rs, f.vo, f.l0 + 4096 * i);
            }
        };
        const FillCtx nofill{false, {0, 0, 0, 0}, nullptr, 0, 0};
        // the pieces group 1 issues in its softmax step
        auto fill_soft = [&](const FillCtx& f, auto i_c) __attribute__((always_inline)) {
            if constexpr (decltype(i_c)::value >= kMstepPieces) fill_piece(f, i_c);
        };
        // MFMA step body: PV(t-1) (16 MFMAs) then QK(t) (18 MFMAs), as one
        // sequence of operations whose LDS operands are fetched kMstepLookahead
        // ahead.  Operation i < 16 is PV k-step i/8 for output block i%8; operation 16 + k is
        // QK k-step k (k < 16 latent dims of this half, then two RoPE k-steps
        // whose Q fragment also comes from LDS).  P and S are never live
        // together.
        auto mstep = [&](int t, auto pv_c, auto qk_c, const FillCtx& fc, auto fill_c) __attribute__((always_inline)) {
            constexpr bool DO_PV = decltype(pv_c)::value != 0;
            constexpr bool DO_QK = decltype(qk_c)::value != 0;
            // copy pieces after the first MFMAs (full steady-state step only)
            constexpr bool FILL = decltype(fill_c)::value != 0 && DO_PV && DO_QK && !FP8;
            constexpr int I0 = DO_PV ? 0 : 16;
            constexpr int I1 = DO_QK ? (D512 ? 32 : 34) : 16;   // the 512-wide head has no RoPE steps
            const unsigned char* Tp = sm.tile[0] + opaque_tile_offset((t + kNBuf - 1) % kNBuf) + 16384 * kh;  // t-1
            const unsigned char* T = sm.tile[0] + opaque_tile_offset(t % kNBuf);                               // t
            auto fetch = [&](int i, bf16x8& A, bf16x8& B) __attribute__((always_inline)) {
                if (i < 16) {
                    const unsigned char* Tv = Tp + 256 * (i >> 3) + 2048 * (i & 7);
                    const bf16x4 v0 = tr_read(Tv + vb[0]);
                    const bf16x4 v1 = tr_read(Tv + vb[1]);
                    A = bf16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
                } else if (i < 32) {
                    const int kk = i - 16;
                    A = *(const bf16x8*)(T + 16384 * kh + kb[kk & 1] + 1024 * kk);
                } else {
                    const int kr = 2 * kh + (i - 32);    // RoPE column 64 + 2kr + half
                    A = *(const bf16x8*)(T + 32768 + kb[kr & 1] + 1024 * kr);
                    B = sm.qr[hb][kr][lane];
                }
            };
            constexpr int LA = kMstepLookahead;
            bf16x8 opA[LA + 1], opB[LA + 1];
#pragma unroll
            for (int i = I0; i < I0 + LA && i < I1; ++i) fetch(i, opA[i % (LA + 1)], opB[i % (LA + 1)]);
            static_for<0, 34>([&](auto i_c) __attribute__((always_inline)) {
                constexpr int i = decltype(i_c)::value;
                if constexpr (i >= I0 && i < I1) {
                    if (i + LA < I1) fetch(i + LA, opA[(i + LA) % (LA + 1)], opB[(i + LA) % (LA + 1)]);
                    constexpr int r = i % (LA + 1);
                    if constexpr (i < 16) {
                        acc[i & 7] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opA[r], (i < 8) ? p0 : p1, acc[i & 7],
                                                                            0, 0, 0);
                    } else if constexpr (i == 16) {
                        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opA[r], qf[0], f32x16{}, 0, 0, 0);
                    } else if constexpr (i < 32) {
                        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opA[r], qf[i - 16], s, 0, 0, 0);
                    } else {
                        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opA[r], opB[r], s, 0, 0, 0);
                    }
                    if constexpr (FILL && i < kMstepPieces) {
                        mstep_schedule_region<i>();
                        __builtin_amdgcn_sched_barrier(0);
                        fill_piece(fc, IntC<i>{});
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            });
            if (DO_QK) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sm.xs[hb][kh][i][lane] = f32x4{s[4 * i], s[4 * i + 1], s[4 * i + 2], s[4 * i + 3]};
            }
            if constexpr (FILL) mstep_schedule_tail<I1>();
            else mstep_schedule_all<I0, I1, DO_QK>();
        };
        // full scores, mask, exact online softmax.  Register r holds token
        // 8(r/4) + 4*half + r%4 of the tile.  Scores stay unscaled; c > 0 is
        // folded into the exponent.
        auto soft = [&](int t, const FillCtx& fc_in, auto fill_c) __attribute__((always_inline)) {
            // ``on`` is a compile-time constant here, so the pieces are straight-line code
            FillCtx fc = fc_in;
            fc.on = decltype(fill_c)::value != 0 && !FP8;
            // The softmax wave is issue-bound on VALU while the other wave of
            // the SIMD needs one issue slot per MFMA: give the softmax wave the
            // higher issue priority for the duration of the step.
            __builtin_amdgcn_s_setprio(2);
            const int g = g0 + t;
            const int tv = nslots - g * kSubTok;
            const int pg_t = SPARSE ? 0 : page_of(g);
            const bool full = SPARSE ? false : (page_ok(pg_t, a.num_rows) && tv >= kSubTok);
            f32x4 xo[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) xo[i] = sm.xs[hb][kh ^ 1][i][lane];
            fill_soft(fc, IntC<0>{});
            fill_soft(fc, IntC<1>{});
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int e = 0; e < 4; ++e) s[4 * i + e] += xo[i][e];
            }
            if (!full) {
                // token 8(r/4) + 4 half + r%4 is valid iff 4 half < tv - 8(r/4) - r%4:
                // one per-lane value against a uniform limit per register
                const int tv_ok = SPARSE ? 0 : (page_ok(pg_t, a.num_rows) ? tv : 0);
                const int h4 = 4 * half;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int c_r = 8 * (r >> 2) + (r & 3);
                    const bool valid = SPARSE ? (sm.rows[t & 3][h4 + c_r] >= 0) : (h4 < tv_ok - c_r);
                    if (!valid) s[r] = -INFINITY;
                }
            }
            // tile max in v_max3 (the scores hold no signalling NaN, so no
            // quieting max(x, x) per input), then across the lane pair
            float mx = max3_raw(max3_raw(s[0], s[1], s[2]), max3_raw(s[3], s[4], s[5]), max3_raw(s[6], s[7], s[8]));
            mx = max3_raw(mx, max3_raw(s[9], s[10], s[11]), max3_raw(s[12], s[13], s[14]));
            mx = max3_raw(mx, s[15], s[15]);
            {
                auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
                mx = max3_raw(__uint_as_float(r[0]), __uint_as_float(r[1]), __uint_as_float(r[1]));
            }
            fill_soft(fc, IntC<2>{});
            fill_soft(fc, IntC<3>{});
            // Running max: raised to the tile max only when that exceeds it by
            // more than tau in log2 units (tau = 0: whenever it is larger,
            // the exact running max).  From -inf any finite max is taken.
            const float cmx = c * mx;
            const bool keep = cmx - cm_run <= a.rescale_tau;
            const float cm_new = keep ? cm_run : fmaxf(cm_run, cmx);
            // while every score so far is masked, m_new = -inf: alpha 1, p = exp2(-inf) = 0
            const float alpha = cm_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(cm_run - cm_new);
            const float cm = cm_new == -INFINITY ? 0.f : cm_new;
            float psum = 0.f;
            static_for<0, 16>([&](auto r_c) __attribute__((always_inline)) {
                constexpr int r = decltype(r_c)::value;
                s[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -cm));
                psum += s[r];
                if constexpr (r == 5) fill_soft(fc, IntC<4>{});
                if constexpr (r == 10) fill_soft(fc, IntC<5>{});
                if constexpr (r == 15) fill_soft(fc, IntC<6>{});
            });
            psum = wave_sum_pair(psum);
            // rescale O (lane l holds head l%32); skipped when no head's max rose.
            // O is zero until the first finite max, so it needs no rescale then.
            const uint32_t rose = (uint32_t)__builtin_amdgcn_ballot_w64(alpha != 1.f);
            if (rose != 0 && __builtin_amdgcn_ballot_w64(cm_run != -INFINITY) != 0) {
#pragma unroll
                for (int dd = 0; dd < 8; ++dd)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[dd][r] *= alpha;
            }
            fill_soft(fc, IntC<7>{});
            l_run = l_run * alpha + psum;
            cm_run = cm_new;
#pragma unroll
            for (int e = 0; e < 8; ++e) { p0[e] = (__bf16)s[e]; p1[e] = (__bf16)s[8 + e]; }
            fill_soft(fc, IntC<8>{});
            __builtin_amdgcn_s_setprio(0);
        };
        // step 2t: FP8 tile t+1 to registers; sparse row ids of tile t+2
        auto step_even_begin = [&](int t) __attribute__((always_inline)) -> int {
            int next_row = -1;
            if (SPARSE && wave == 0 && lane < kSubTok && t + 2 < ns)
                next_row = (int)rr.row(j, (g0 + t + 2) * kSubTok + lane, nslots);
            if (FP8) fp8_copy(t + 1, pg1);
            return next_row;
        };
        auto step_even_end = [&](int t, int next_row) __attribute__((always_inline)) {
            if (SPARSE && wave == 0 && lane < kSubTok && t + 2 < ns) sm.rows[(t + 2) & 3][lane] = next_row;
            lds_barrier();
        };
        // end of step 2t+1: tile t+1 has landed
        auto step_odd_end = [&](int t) __attribute__((always_inline)) {
            if (t + 1 < ns) {
                if (FP8) {
                    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's copies of tile t+1
                    fp8_dequant(t + 1);
                }
                else if (t > 0 || grp == 1) __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's tile copies
            }
            if (!SPARSE) {
                if (((g0 + t + 3) >> 1) - pt_base >= 64) load_pages((g0 + t) >> 1);
                pg1 = pg2;
                pg2 = t + 3 < ns ? page_of(g0 + t + 3) : 0;
            }
            lds_barrier();
        };

        auto run = [&](auto grp_c) __attribute__((always_inline)) {
            constexpr int G = decltype(grp_c)::value;
            const IntC<0> no;
            const IntC<1> yes;
            // steps 0, 1
            int nr = step_even_begin(0);
            if (G == 0) {
                mstep(0, no, yes, nofill, no);
            } else {
                if (!FP8) {
                    const FillCtx fc = fill_prepare(0);
                    static_for<0, 9>([&](auto i_c) __attribute__((always_inline)) { fill_piece(fc, i_c); });
                }
            }
            step_even_end(0, nr);
            if (G == 0) soft(0, nofill, no);
            else mstep(0, no, yes, nofill, no);
            step_odd_end(0);
            // steady state: steps 2t, 2t+1
            for (int t = 1; t < ns; ++t) {
                nr = step_even_begin(t);
                if (G == 0) mstep(t, yes, yes, fill_prepare(t), yes);
                else soft(t - 1, fill_prepare(t), yes);
                step_even_end(t, nr);
                if (G == 0) soft(t, nofill, no);
                else mstep(t, yes, yes, nofill, no);
                step_odd_end(t);
            }
            // drain: steps 2ns, 2ns+1 (the last tile's PV)
            if (G == 0) mstep(ns, yes, no, nofill, no);
            else soft(ns - 1, nofill, no);
            lds_barrier();
            if (G == 1) mstep(ns, yes, no, nofill, no);
            lds_barrier();
        };
        if (grp == 0) run(IntC<0>{});
        else run(IntC<1>{});

        // ---- epilogue: both waves of a head block hold the same m, l ----
        // acc[d] register r, lane l: head 32-block base + l%32, dim 256 kh + 32 d +
        // (r/4)*8 + 4*(l/32) + r%4 (four consecutive dims per register quad).
        // lane-dependent indices rebuilt from the lane id here, so that no
        // 64-bit lane offset is kept live across the tile loop
        const int ln_e = lane_id();
        int wave_e = wave;
        __asm__ volatile("" : "+s"(wave_e));       // wave-derived offsets rebuilt here too
        const int kh_e = wave_e & 1, hb_e = wave_e >> 1;
        const int H_e = MLA_LATE_ARG(DecodeArgs, h_q), sq_e = MLA_LATE_ARG(DecodeArgs, s_q);
        const int head_e = hblk * kHeadsPerWG + hb_e * 32 + (ln_e & 31);
        const int half_e = ln_e >> 5;
        const bool head_ok_e = head_e < H_e;
        // the item's split count and this partition's output slot (fused: the
        // LDS table, written before the segment's first barrier)
        int nsplit, slot;
        if (fused) {
            const int e = __builtin_amdgcn_readfirstlane(sm.seg_tab[j]);
            nsplit = e >> 16;
            slot = (j == jb) ? slot0 : (e & 0xffff);
        } else {
            nsplit = so_at(j + 1) - so_at(j);
            slot = (j == jb) ? slot0 : so_at(j);
        }
        const bool final_out = (nsplit == 1);
        const int b = j / sq_e, iq = j - b * sq_e;
        if (final_out || (slot >= 0 && slot < MLA_LATE_ARG(DecodeArgs, max_slots))) {
            // l = 0: nothing visible (lse -inf, weight 0 in the merge); l NaN (a NaN
            // in q or the cache): lse NaN, so the merge propagates it
            const float lse_v = l_run > 0.f ? (cm_run + log2f(l_run)) * 0.69314718055994531f
                                             : (l_run == 0.f ? -INFINITY : __builtin_nanf(""));
            float inv = l_run > 0.f ? 1.f / l_run : 0.f;
            // attention sink: a final output is scaled by exp(lse) / (exp(lse) + exp(sink));
            // a row that saw nothing stays 0 (with lse = sink = -inf the factor would be NaN)
            const float* attn_sink = MLA_LATE_ARG(DecodeArgs, attn_sink);
            if (final_out && attn_sink && head_ok_e && l_run > 0.f)
                inv *= 1.f / (1.f + __expf(attn_sink[head_e] - lse_v));
            // Split partials in float16 (when the output is bf16): each lane scales
            // its 128 values by 2^-E, E from the exponent of their largest
            // magnitude, so they lie in [-1, 1) and cannot overflow; E is stored
            // in the head's exponent bytes 2 q + h of the dims d it holds
            // (q = d / 128 in {2 kh, 2 kh + 1}, h = d % 8 / 4, the lane's half).
            const bool part16 = !final_out && MLA_LATE_ARG(DecodeArgs, part_fp16);
            int E = 0;
            if (part16 && head_ok_e) {
                float amax = 0.f;
#pragma unroll
                for (int dd = 0; dd < 8; ++dd)
#pragma unroll
                    for (int r = 0; r < 16; ++r) amax = fmaxf(amax, fabsf(acc[dd][r]));
                amax *= inv;
                const int be = (int)((__float_as_uint(amax) >> 23) & 0xff);   // biased exponent
                E = amax > 0.f ? (be == 0 ? -125 : be - 126) : 0;              // amax * 2^-E < 1
                E = E > 127 ? 127 : E;
                // the lane's dims span quarters 2 kh and 2 kh + 1 of the head
                MLA_LATE_ARG(DecodeArgs, o_exp8)[((int64_t)slot * H_e + head_e) * 8 + 4 * kh_e + half_e] = (unsigned char)(signed char)E;
                MLA_LATE_ARG(DecodeArgs, o_exp8)[((int64_t)slot * H_e + head_e) * 8 + 4 * kh_e + 2 + half_e] = (unsigned char)(signed char)E;
            }
            if (head_ok_e) {
#pragma unroll
                for (int dd = 0; dd < 8; ++dd) {
#pragma unroll
                    for (int rq = 0; rq < 4; ++rq) {
                        const int dim = 256 * kh_e + 32 * dd + 8 * rq + 4 * half_e;
                        const float v0 = acc[dd][4 * rq + 0] * inv, v1 = acc[dd][4 * rq + 1] * inv;
                        const float v2 = acc[dd][4 * rq + 2] * inv, v3 = acc[dd][4 * rq + 3] * inv;
                        if (part16) {
                            const int64_t o = ((int64_t)slot * H_e + head_e) * kDv + dim;
                            typedef __attribute__((__vector_size__(4 * sizeof(_Float16)))) _Float16 f16x4;
                            *(f16x4*)((_Float16*)MLA_LATE_ARG(DecodeArgs, o_part) + o) = f16x4{(_Float16)ldexpf(v0, -E), (_Float16)ldexpf(v1, -E),
                                                                         (_Float16)ldexpf(v2, -E), (_Float16)ldexpf(v3, -E)};
                        } else if (final_out) {
                            const int64_t o = ((int64_t)j * H_e + head_e) * kDv + dim;
                            if (MLA_LATE_ARG(DecodeArgs, out_fp32)) {
                                *(f32x4*)((float*)MLA_LATE_ARG(DecodeArgs, out) + o) = f32x4{v0, v1, v2, v3};
                            } else {
                                const bf16x4 w = {(__bf16)v0, (__bf16)v1, (__bf16)v2, (__bf16)v3};
                                *(bf16x4*)((__bf16*)MLA_LATE_ARG(DecodeArgs, out) + o) = w;
                            }
                        } else {
                            const int64_t o = ((int64_t)slot * H_e + head_e) * kDv + dim;
                            *(f32x4*)(MLA_LATE_ARG(DecodeArgs, o_part) + o) = f32x4{v0, v1, v2, v3};
                        }
                    }
                }
            }
            if (kh_e == 0 && ln_e < 32 && head_ok_e) {
                if (final_out) MLA_LATE_ARG(DecodeArgs, lse)[((int64_t)b * H_e + head_e) * sq_e + iq] = lse_v;
                else MLA_LATE_ARG(DecodeArgs, lse_part)[(int64_t)slot * H_e + head_e] = lse_v;
            }
        }
        lds_barrier();
    }
}

hipError_t launch_decode(const DecodeArgs& a, bool sparse, int kvf, hipStream_t stream) {
    const dim3 grid(a.num_parts * a.n_hblk), block(kThreads);
    if (sparse) {
        if (kvf == 3) hipLaunchKernelGGL((decode_kernel<true, 3>), grid, block, 0, stream, a);
        else if (kvf == 2) hipLaunchKernelGGL((decode_kernel<true, 2>), grid, block, 0, stream, a);
        else if (kvf == 1) hipLaunchKernelGGL((decode_kernel<true, 1>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((decode_kernel<true, 0>), grid, block, 0, stream, a);
    } else {
        // the dense bf16 cache runs decode64_kernel
        if (kvf != 1) return hipErrorInvalidValue;
        if (a.fused) hipLaunchKernelGGL((decode_kernel<false, 1, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((decode_kernel<false, 1>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace mla
