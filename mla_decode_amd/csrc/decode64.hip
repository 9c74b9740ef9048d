// Split-KV partial-attention kernel for absorbed-MLA decode on gfx950, bf16
// cache (dense pages or top-k rows): 64 query heads per workgroup, waves split
// by role.
//
// A workgroup computes 64 heads of one scheduler partition (a contiguous run
// of 32-token KV tiles, possibly spanning several items).  The two workgroups
// that hold the two head blocks of a partition are placed on the same XCD, so
// the second read of every KV tile is served by that XCD's L2.  Halving the
// heads per workgroup halves the fixed register state (the fp32 output
// accumulator and Q), which is what lets every role below run without
// spilling and with deep operand prefetch.
//
// Eight waves, two per SIMD (the dispatcher puts wave w on SIMD w % 4):
//   QK waves (2, 3)     head block hb = w - 2 (32 heads).  Q for all 576 dims
//                       lives in registers (144 VGPRs), so the full scores
//                       S^T = K Q^T of a tile are one wave's MFMA chain (two
//                       alternating accumulators) and need no exchange with
//                       another wave.  While the MFMAs of tile k+1 run, the
//                       same wave does the exact online softmax of tile k:
//                       running max raised whenever the tile holds a larger
//                       score, p = exp2(s c - m c), l sums the fp32 p, P is
//                       rounded to bf16 and handed to the PV waves in LDS
//                       with the rescale factor alpha.
//   PV waves (0, 1, 4, 5)  output dims 128 q .. 128 q + 127 of all 64 heads
//                       (q = 0, 1, 2, 3): acc O^T += V^T P^T, the V^T operand
//                       read straight from the row-major tile with
//                       ds_read_b64_tr_b16, each fragment feeding the MFMAs of
//                       both head blocks.  Before a block of O takes its MFMAs
//                       it is rescaled by alpha (skipped when no head's max
//                       rose), so the multiplies of one block overlap the MFMAs
//                       of the previous one.
//   copy waves (6, 7)   stage tiles global -> registers -> LDS: 16-byte
//                       buffer loads two steps ahead into one of two register
//                       sets, ds_write_b128 when the tile's LDS buffer is
//                       free, and publish which tokens of each tile are valid.
//                       Dense: a page's tokens past the valid count fall
//                       outside the buffer range and load as zeros; the count
//                       is published.  Top-k: each lane loads its token's
//                       index one step before the row (so the index wait
//                       never waits on the tile in flight), rows are gathered
//                       through one buffer over the whole cache, an invalid
//                       entry (-1, out of range, past the item's top-k
//                       length) reads past its end as zeros, and a 32-bit mask
//                       of valid tokens is published.
//
// Step k (one workgroup barrier per step, LDS ring of four 32-token tiles):
//   QK waves     softmax(k) and QK(k+1)        reads tile k+1
//   PV waves     rescale and PV(k-1)           reads tile k-1
//   copy waves   write tile k+2, load tile k+4  writes the buffer of tile k-2
// so every SIMD has MFMA and vector work from two waves at once.
//
// Items whose KV range sits in one partition write out/lse directly; split
// items write normalised partials (float16 scaled per lane by a power of two
// when the output is bf16, float32 otherwise) for the combine kernel.

#include "common.h"
#include "kernels.h"
#include "wave_sched.h"

namespace mla {

namespace {

constexpr int kH = 64;                          // query heads per workgroup
constexpr int kT = 512;                         // threads (8 waves)
constexpr int kTileB = kSubTok * kRowBytes;     // 36864 bytes per 32-token tile
constexpr int kRing = 4;                        // LDS tile buffers
constexpr int kQkLA = 6;                        // K fragments in flight (QK waves)
constexpr int kPvLA = 4;                        // V fragments in flight (PV waves)
constexpr int kXRow = 2 * kDv + 16;             // epilogue staging: bytes per head row (16 bytes of bank skew)

typedef __attribute__((__vector_size__(4 * sizeof(_Float16)))) _Float16 f16x4;

// Small arrays first: LDS instructions encode at most a 16-bit immediate
// offset, so arrays addressed with constant offsets must sit below 64 KiB.
struct __attribute__((aligned(16))) Smem64 {
    bf16x8 p[2][2][2][64];          // P(k) as B fragments [k & 1][head block][k-step][lane]
    float alpha[2][2][32];          // rescale factor of O for tile k [k & 1][head block][head]
    float fin_inv[kH];              // epilogue: output scale 1/l (times the sink factor)
    float fin_pad[kH];
    int valid[kRing];               // dense: valid tokens of the tile in each buffer
    int vmask[kRing][2];            // top-k: valid-token bits of each buffer's tile [copy wave]
    int seg[2];                     // the current segment's output slot and (split count == 1)
    int pad[2];
    unsigned char tile[kRing][kTileB];   // 32-token tiles (bf16, swizzled columns, see lds_chunk)
};

// LDS layout of a 32-token tile (72 columns of 16 bytes per token): 36
// blocks of 1 KiB, block 4 (c / 8) + t / 8 holding the 128-byte line c / 8 of
// tokens 8 (t / 8) .. + 7; inside a block token t sits at chunk 8 (t % 8) +
// ((c % 8) ^ swz(t)), swz(t) = (t % 8) ^ ((t / 8) % 2).  A copy instruction then
// reads eight whole lines, and 16 consecutive tokens of one column fall on 16
// distinct 16-byte bank groups (64 banks of 4 bytes).  Returns the chunk index
// within the tile (for c < 64; RoPE columns 64..71 likewise).
__device__ __forceinline__ int tile_chunk(int t, int c) {
    const int swz = (t & 7) ^ ((t >> 3) & 1);
    return 64 * (4 * (c >> 3) + (t >> 3)) + 8 * (t & 7) + ((c & 7) ^ swz);
}

__device__ __forceinline__ bf16x4 tr_read64(const unsigned char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(p));
}

// Uniform byte offset of tile buffer ``idx``, hidden from the optimiser so
// that it adds it to a few lane bases instead of keeping one set of lane
// addresses per buffer.
__device__ __forceinline__ int ring_offset(int idx) {
    int off = idx * kTileB;
    __asm__ volatile("" : "+s"(off));
    return off;
}

__device__ __forceinline__ int lane_id64() {
    unsigned m = ~0u;
    __asm__ volatile("" : "+s"(m));
    return (int)__builtin_amdgcn_mbcnt_hi(m, __builtin_amdgcn_mbcnt_lo(m, 0u));
}

__device__ __forceinline__ void barrier_only() {
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

__device__ __forceinline__ void barrier_lds() {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt, expcnt untouched
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

constexpr int kGrpMfma = 0x008, kGrpValu = 0x002, kGrpDsRead = 0x100, kGrpDsWrite = 0x200;

template <int V>
struct Int {
    static constexpr int value = V;
};
template <int B, int E, class F>
__device__ __forceinline__ void unroll(F&& f) {
    if constexpr (B < E) {
        f(Int<B>{});
        unroll<B + 1, E>(f);
    }
}

}  // namespace

template <bool FUSED, bool SPARSE>
__global__ void __launch_bounds__(kT, 1) decode64_kernel(const DecodeArgs a) {
    __shared__ Smem64 sm;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // roles
    const bool is_qk = wave == 2 || wave == 3;
    const bool is_copy = wave >= 6;
    const int hbq = wave - 2;                                   // QK waves: head block
    const int dq = (wave & 1) + 2 * (wave >> 2);                // PV waves 0, 1, 4, 5 -> dim quarter 0, 1, 2, 3
    const int cw = wave - 6;                                    // copy waves: 0, 1

    // workgroup -> (partition, head block): each XCD (blockIdx % 8) gets a
    // contiguous run of linear indices, so the head blocks of a partition and
    // neighbouring partitions share an L2.
    int part, hblk;
    {
        const int G = a.num_parts * a.n_hblk;
        const int x = blockIdx.x & 7, k = blockIdx.x >> 3;
        const int q8 = G >> 3, r8 = G & 7;
        const int lin = x * q8 + min(x, r8) + k;
        part = lin / a.n_hblk;
        hblk = lin - part * a.n_hblk;
    }
    const int N = a.batch * a.s_q;
    const int32_t* rec = a.meta + kMetaHeader + kMetaRec * part;
    const int32_t* so = a.meta + kMetaHeader + kMetaRec * a.num_parts;
    // This partition's record: read from the scheduler's metadata, or (fused)
    // computed here by every wave from the cache lengths with the scheduler's
    // arithmetic (item costs, their prefix sum cut into equal runs, split
    // counts and offsets), items ln * fR + u held by lane ln.
    int jb, tbeg, je, tend, slot0;
    WaveSched ws;
    int fR = 1;
    // uniform read of item j's entry of a lane-distributed array (R items per lane)
    auto item_at = [&](const int (&v)[4], int j) __attribute__((always_inline)) -> int {
        const int u = j & (fR - 1);
        const int x = u == 0 ? v[0] : u == 1 ? v[1] : u == 2 ? v[2] : v[3];
        return __builtin_amdgcn_readlane(x, j >> (fR >> 1));
    };
    if constexpr (FUSED) {
        const int ln = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
        fR = N <= 64 ? 1 : N <= 128 ? 2 : 4;
        wave_schedule_any(a, SPARSE ? a.topk_length : a.cache_seqlens, N, part, ln, fR, ws);
        jb = ws.jb; tbeg = ws.tbeg; je = ws.je; tend = ws.tend; slot0 = ws.slot0;
        // the schedule written back: each partition's record by its first head
        // block, header and split offsets by workgroup 0 (copy wave 0 of each)
        if (is_copy && cw == 0) wave_schedule_store(a, N, part, ln, fR, ws, hblk == 0, blockIdx.x == 0);
    } else {
        jb = sload(rec + 0), tbeg = sload(rec + 1), je = sload(rec + 2), tend = sload(rec + 3);
        slot0 = sload(rec + 4);
    }
    const int H = a.h_q;
    const float c = a.scale_log2;
    const unsigned char* kv = (const unsigned char*)a.kv;
    RowResolver rr{a.block_table, SPARSE ? a.topk_length : a.cache_seqlens, a.indices, a.s_q, a.max_blocks,
                   SPARSE ? a.topk : 0, a.causal, a.num_rows};


    // One segment = the tiles of item j that this partition holds.  Every role
    // walks the same segments and passes the same barriers (n + 6 per segment).
    // The copy waves look up its output slot and split count and publish them
    // in LDS before the segment's first barrier; the other roles read them at
    // the segment's end.
    struct Seg {
        int nslots, g0, n, slot, b, iq;
        bool final_out, write_ok;
    };
    auto segment = [&](int j, Seg& sg) __attribute__((always_inline)) -> bool {
        sg.nslots = rr.slots_uniform(j);
        const int ntile_j = (sg.nslots + 63) >> 6;
        const int t0 = (j == jb && tbeg > 0) ? tbeg : 0;
        int t1 = (j == je) ? tend : ntile_j;
        if (t1 > ntile_j) t1 = ntile_j;
        if (t0 >= t1) return false;
        sg.g0 = 2 * t0;                                                     // first 32-token tile
        sg.n = min(2 * t1, (sg.nslots + kSubTok - 1) / kSubTok) - sg.g0;   // tiles of this segment
        sg.b = j / a.s_q;
        sg.iq = j - sg.b * a.s_q;
        return true;
    };
    // copy waves: slot and split count of segment j
    auto seg_split = [&](int j, Seg& sg) __attribute__((always_inline)) {
        int nsplit;
        if constexpr (FUSED) {
            nsplit = item_at(ws.NS, j);
            sg.slot = (j == jb) ? slot0 : item_at(ws.SO, j);
        } else {
            nsplit = sload(so + j + 1) - sload(so + j);
            sg.slot = (j == jb) ? slot0 : sload(so + j);
        }
        sg.final_out = nsplit == 1;
        sg.write_ok = sg.final_out || (sg.slot >= 0 && sg.slot < a.max_slots);
    };
    // QK and PV waves, after the segment's first barrier
    auto seg_read = [&](Seg& sg) __attribute__((always_inline)) {
        sg.slot = __builtin_amdgcn_readfirstlane(sm.seg[0]);
        sg.final_out = __builtin_amdgcn_readfirstlane(sm.seg[1]) != 0;
        sg.write_ok = sg.final_out || (sg.slot >= 0 && sg.slot < a.max_slots);
    };

    if (is_copy) {
        // -------------------------------------------------------------------- copy waves
        for (int j = jb; j <= je && j < N; ++j) {
            Seg sg;
            if (!segment(j, sg)) continue;
            seg_split(j, sg);
            sm.seg[0] = sg.slot;
            sm.seg[1] = sg.final_out ? 1 : 0;
            const int npages_item = (sg.nslots + kBlock - 1) / kBlock;
            int pt_base = 0, pt_v = 0;
            auto load_pages = [&](int first) __attribute__((always_inline)) {
                pt_base = first;
                const int pi = first + lane_id64();
                pt_v = pi < npages_item ? a.block_table[(int64_t)sg.b * a.max_blocks + pi] : 0;
                __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
            };
            if constexpr (!SPARSE) load_pages(sg.g0 >> 1);
            // A tile is copied as 36 blocks of 1 KiB, block 4 cg + tg holding the
            // 128-byte line cg (columns 8 cg .. 8 cg + 7) of tokens 8 tg .. 8 tg + 7,
            // so that every copy instruction reads eight whole lines (see
            // tile_chunk).  Copy wave cw copies token groups 2 cw and 2 cw + 1
            // (18 blocks): one wave sustains about 1 KiB of direct-to-LDS loads
            // per 90 cycles, so both copy waves share every tile.  Lane l copies
            // token 8 tg + l / 8, column 8 cg + ((l % 8) ^ swz(token)); the byte
            // count of the buffer of token group tg stops at the valid tokens,
            // so the rest land as zeros.
            // The 18 blocks of a tile are loaded into registers two steps before
            // they are written to LDS (ds_write_b128 to the address a direct copy
            // would fill), so each tile has two steps to arrive from HBM and two
            // tiles are in flight per workgroup; tile it uses register set it % 2.
            i32x4 st[2][18];
            int nvs[2] = {0, 0};
            const int ln = lane_id64();
            const int tq = ln >> 3, sl = ln & 7;
            const int fbe = tq * kRowBytes + 16 * (sl ^ tq);         // even token groups: swz = tq
            const int fbo = tq * kRowBytes + 16 * (sl ^ tq ^ 1);     // odd token groups: swz = tq ^ 1
            // top-k: lane's token is slot 32 g + 8 tg + tq of the item; its
            // index for tile it sits in ix[it % 2][u], loaded a step ahead
            int ix[2][2] = {{-1, -1}, {-1, -1}};
            int msk[2] = {0, 0};
            const int64_t ibase = (int64_t)j * a.topk;
            const uint32_t nrec = (uint32_t)a.num_rows * (uint32_t)kRowBytes;   // < 2^32 - 2 rows: host-checked
            auto load_idx = [&](auto s_c, int it) __attribute__((always_inline)) {
                constexpr int S = decltype(s_c)::value;
                unroll<0, 2>([&](auto u_c) __attribute__((always_inline)) {
                    constexpr int u = decltype(u_c)::value;
                    const int slot = (sg.g0 + it) * kSubTok + 8 * (2 * cw + u) + tq;
                    int v = -1;
                    if (it < sg.n && slot < sg.nslots) v = a.indices[ibase + slot];
                    ix[S][u] = v;
                });
            };
            auto load_tile = [&](auto s_c, int it) __attribute__((always_inline)) {
                constexpr int S = decltype(s_c)::value;
                if constexpr (SPARSE) {
                    // one buffer over the whole cache; an invalid row's offset
                    // starts at its end, so its 16-byte loads return zeros
                    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)kv, 0, (int)nrec, 0x00020000);
                    uint32_t m = 0;
                    unroll<0, 2>([&](auto u_c) __attribute__((always_inline)) {
                        constexpr int u = decltype(u_c)::value;
                        const int64_t r = sparse_entry_row(ix[S][u], a.num_rows);
                        const bool ok = r >= 0;
                        const uint32_t vo = (ok ? (uint32_t)r * (uint32_t)kRowBytes : nrec) +
                                            (uint32_t)(16 * (sl ^ tq ^ u));
                        // token 8 tg + t is valid when lane 8 t of the group is
                        const uint64_t bal = __builtin_amdgcn_ballot_w64(ok);
#pragma unroll
                        for (int t = 0; t < 8; ++t) m |= (uint32_t)((bal >> (8 * t)) & 1u) << (8 * (2 * cw + u) + t);
                        unroll<0, 9>([&](auto cg_c) __attribute__((always_inline)) {
                            constexpr int cg = decltype(cg_c)::value;
                            st[S][9 * u + cg] = __builtin_bit_cast(
                                i32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(vo + 128 * cg), 0, 0));
                        });
                    });
                    msk[S] = (int)m;
                    return;
                }
                const int g = sg.g0 + it;
                if (((g >> 1) - pt_base) >= 64) load_pages(g >> 1);
                const int page = __builtin_amdgcn_readlane(pt_v, (g >> 1) - pt_base);
                const bool ok = page_ok(page, a.num_rows);
                int nvalid = min(sg.nslots - g * kSubTok, kSubTok);
                if (!ok || nvalid < 0) nvalid = 0;
                nvs[S] = nvalid;
                const unsigned char* base = kv + (ok ? (int64_t)page * kTileBytes + (g & 1) * kTileB : 0);
                unroll<0, 2>([&](auto u_c) __attribute__((always_inline)) {
                    constexpr int u = decltype(u_c)::value;
                    const int tg = 2 * cw + u;
                    // base and byte count are uniform by construction; readfirstlane
                    // lets the compiler see it (no per-lane descriptor loop)
                    const uint64_t pb = (uint64_t)(base + 8 * tg * kRowBytes);
                    const uint64_t pu = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(pb >> 32)) << 32) |
                                        (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)pb);
                    const int nr = __builtin_amdgcn_readfirstlane(min(max(nvalid - 8 * tg, 0), 8) * kRowBytes);
                    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)pu, 0, nr, 0x00020000);
                    unroll<0, 9>([&](auto cg_c) __attribute__((always_inline)) {
                        constexpr int cg = decltype(cg_c)::value;
                        st[S][9 * u + cg] = __builtin_bit_cast(
                            i32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (u ? fbo : fbe) + 128 * cg, 0, 0));
                    });
                });
            };
            auto write_tile = [&](auto s_c, int it) __attribute__((always_inline)) {
                constexpr int S = decltype(s_c)::value;
                unsigned char* dst = sm.tile[0] + ring_offset(it % kRing) + 16 * ln;
                unroll<0, 2>([&](auto u_c) __attribute__((always_inline)) {
                    constexpr int u = decltype(u_c)::value;
                    const int tg = 2 * cw + u;
                    unroll<0, 9>([&](auto cg_c) __attribute__((always_inline)) {
                        constexpr int cg = decltype(cg_c)::value;
                        *(i32x4*)(dst + 1024 * (4 * cg + tg)) = st[S][9 * u + cg];
                    });
                });
                if constexpr (SPARSE) sm.vmask[it % kRing][cw] = msk[S];
                else if (cw == 0) sm.valid[it % kRing] = nvs[S];
            };
            // Step k writes tile k + 2 (set k % 2) and loads tile k + 4 into the
            // same set.  The steps that load (k + 4 < n) run in a loop of their
            // own, unrolled by two, so that the loads are unconditional there and
            // the compiler's waits before the writes leave the newer set in flight.
            auto step_load = [&](auto s_c, int k) __attribute__((always_inline)) {
                constexpr int S = decltype(s_c)::value;
                write_tile(s_c, k + 2);
                // top-k: the index of tile k + 5 is requested before the rows of
                // tile k + 4, so the next step's wait for it leaves those rows
                // in flight
                if constexpr (SPARSE) load_idx(Int<1 - S>{}, k + 5);
                load_tile(s_c, k + 4);
                barrier_lds();
            };
            auto step_tail = [&](auto s_c, int k) __attribute__((always_inline)) {
                if (k + 2 < sg.n) write_tile(s_c, k + 2);
                barrier_lds();
            };
            if constexpr (SPARSE) {
                load_idx(Int<0>{}, 0);
                load_idx(Int<1>{}, 1);
                load_tile(Int<0>{}, 0);
                load_idx(Int<0>{}, 2);
                if (1 < sg.n) load_tile(Int<1>{}, 1);
                load_idx(Int<1>{}, 3);
            } else {
                load_tile(Int<0>{}, 0);
                if (1 < sg.n) load_tile(Int<1>{}, 1);
            }
            write_tile(Int<0>{}, 0);
            if (2 < sg.n) load_tile(Int<0>{}, 2);
            barrier_lds();   // tile 0 has landed
            int k = -1;
            for (; k + 5 < sg.n; k += 2) {   // steps k and k + 1 both load
                step_load(Int<1>{}, k);
                step_load(Int<0>{}, k + 1);
            }
            if (k + 4 < sg.n) {              // one more loading step (set 1)
                step_load(Int<1>{}, k);
                ++k;
                for (; k <= sg.n; k += 2) {
                    step_tail(Int<0>{}, k);
                    if (k + 1 <= sg.n) step_tail(Int<1>{}, k + 1);
                }
            } else {
                for (; k <= sg.n; k += 2) {
                    step_tail(Int<1>{}, k);
                    if (k + 1 <= sg.n) step_tail(Int<0>{}, k + 1);
                }
            }
            __builtin_amdgcn_s_waitcnt(0x0F70);   // every load of this wave has written LDS
            barrier_lds();   // epilogue
            barrier_lds();   // epilogue: rows staged in LDS
            barrier_lds();   // the next segment reuses every LDS array
        }
    } else if (is_qk) {
        // -------------------------------------------------------------------- QK waves
        for (int j = jb; j <= je && j < N; ++j) {
            Seg sg;
            if (!segment(j, sg)) continue;
            const int ln = lane_id64();
            const int h32 = ln & 31, hf = ln >> 5;
            const int head = hblk * kH + hbq * 32 + h32;
            const bool head_ok = head < H;
            bf16x8 qf[36];
            {
                const bf16x8* qp = (const bf16x8*)((const unsigned char*)a.q +
                                                   ((int64_t)j * H + (head_ok ? head : 0)) * kRowBytes);
#pragma unroll
                for (int kk = 0; kk < 36; ++kk) {
                    bf16x8 v = qp[2 * kk + hf];
                    if (!head_ok) v = bf16x8{};
                    qf[kk] = v;
                }
            }
            // cm_run = c m_run as rounded in the step that raised m_run: when the
            // max does not rise the exponent of alpha is then exactly 0 and alpha
            // exactly 1, which lets the PV waves skip the rescale
            float m_run = -INFINITY, cm_run = -INFINITY, l_run = 0.f;
            f32x16 s = {}, sa = {}, sb = {};
            barrier_lds();   // tile 0 has landed

            // Softmax of the tile whose scores are in s, in stages that run
            // between the MFMAs of the next tile's QK (stage st after MFMA st +
            // kSoftOffset, so that the step's first MFMAs issue back to back
            // while their K fragments arrive):
            // tile max, the exact running max (raised when the tile max exceeds
            // it by more than tau in log2 units; tau = 0: whenever it is
            // larger), alpha, p = exp2(s c - m c) one score per stage, l, then
            // P rounded to bf16 and published with alpha.
            float mxa = 0.f, mxb = 0.f, m_new = 0.f, cm = 0.f, alpha = 0.f, psum = 0.f;
            bf16x8 p0 = {}, p1 = {};
            constexpr int kSoftStages = 27, kSoftOffset = 3;
            static_assert(kSoftStages + kSoftOffset <= 36, "every softmax stage follows a QK MFMA");
            auto soft_stage = [&](auto st_c, int tslot) __attribute__((always_inline)) {
                constexpr int st = decltype(st_c)::value;
                if constexpr (st == 0) {
                    mxa = max3_raw(max3_raw(s[0], s[1], s[2]), max3_raw(s[3], s[4], s[5]), max3_raw(s[6], s[7], s[7]));
                } else if constexpr (st == 1) {
                    mxb = max3_raw(max3_raw(s[8], s[9], s[10]), max3_raw(s[11], s[12], s[13]), max3_raw(s[14], s[15], s[15]));
                } else if constexpr (st == 2) {
                    // the two lanes of a head hold disjoint tokens
                    const float m2 = max3_raw(mxa, mxb, mxb);
                    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(m2), __float_as_uint(m2), false, false);
                    mxa = max3_raw(__uint_as_float(r[0]), __uint_as_float(r[1]), __uint_as_float(r[1]));
                } else if constexpr (st == 3) {
                    const bool keep = c * (mxa - m_run) <= a.rescale_tau;
                    m_new = keep ? m_run : fmaxf(m_run, mxa);
                    cm = keep ? cm_run : c * m_new;
                } else if constexpr (st == 4) {
                    // no score seen yet (cm = -inf): O and l are still 0, alpha 1
                    alpha = cm == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(cm_run - cm);
                    cm = cm == -INFINITY ? 0.f : cm;
                } else if constexpr (st >= 5 && st < 21) {
                    constexpr int r = st - 5;
                    s[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -cm));
                } else if constexpr (st == 21) {
                    psum = ((s[0] + s[1]) + (s[2] + s[3])) + ((s[4] + s[5]) + (s[6] + s[7]));
                } else if constexpr (st == 22) {
                    psum += ((s[8] + s[9]) + (s[10] + s[11])) + ((s[12] + s[13]) + (s[14] + s[15]));
                } else if constexpr (st == 23) {
                    psum = wave_sum_pair(psum);
                    l_run = l_run * alpha + psum;
                    m_run = m_new;
                    cm_run = m_new == -INFINITY ? -INFINITY : cm;
                } else if constexpr (st == 24) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) p0[e] = (__bf16)s[e];
                } else if constexpr (st == 25) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) p1[e] = (__bf16)s[8 + e];
                } else if constexpr (st == 26) {
                    const int l = lane_id64();
                    sm.p[tslot][hbq][0][l] = p0;
                    sm.p[tslot][hbq][1][l] = p1;
                    sm.alpha[tslot][hbq][l & 31] = alpha;   // both lanes of a head write the same value
                }
            };
            // QK(t): S^T = K Q^T over 36 k-steps, even k-steps into sa and odd
            // ones into sb, K fragments read kQkLA ahead.  The order is fixed
            // with scheduling fences: MFMA i, the read of fragment i + kQkLA,
            // then softmax stage i - kSoftOffset of the previous tile when SOFT.
            auto qk = [&](int t, auto soft_c, int tslot, auto&& pre) __attribute__((always_inline)) {
                constexpr bool SOFT = decltype(soft_c)::value != 0;
                // K operand of k-step kk: token l % 32, column 2 kk + half; its
                // byte offset is 4096 (kk / 4) plus a lane term kb[kk % 4]
                const unsigned char* T = sm.tile[0] + ring_offset(t % kRing);
                int kb[4];
                {
                    const int l = lane_id64();
                    const int tk = l & 31, hl = l >> 5;
#pragma unroll
                    for (int m = 0; m < 4; ++m) kb[m] = tile_chunk(tk, 2 * m + hl) * 16;
                }
                bf16x8 fr[kQkLA + 1];
#pragma unroll
                for (int i = 0; i < kQkLA; ++i) fr[i] = *(const bf16x8*)(T + 4096 * (i >> 2) + kb[i & 3]);
                __builtin_amdgcn_sched_barrier(0);
                pre();   // runs while the first fragments are in flight
                __builtin_amdgcn_sched_barrier(0);
                unroll<0, 36>([&](auto i_c) __attribute__((always_inline)) {
                    constexpr int i = decltype(i_c)::value;
                    const bf16x8 A = fr[i % (kQkLA + 1)];
                    if constexpr (i == 0) sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, qf[0], f32x16{}, 0, 0, 0);
                    else if constexpr (i == 1) sb = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, qf[1], f32x16{}, 0, 0, 0);
                    else if constexpr (i & 1) sb = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, qf[i], sb, 0, 0, 0);
                    else sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, qf[i], sa, 0, 0, 0);
                    if constexpr (i + kQkLA < 36)
                        fr[(i + kQkLA) % (kQkLA + 1)] = *(const bf16x8*)(T + 4096 * ((i + kQkLA) >> 2) + kb[(i + kQkLA) & 3]);
                    if constexpr (SOFT && i >= kSoftOffset && i - kSoftOffset < kSoftStages)
                        soft_stage(Int<i - kSoftOffset>{}, tslot);
                    __builtin_amdgcn_sched_barrier(0);
                });
            };
            // the scores of a tile into s, masked tokens (8 (r / 4) + 4 half + r % 4)
            // at -inf; nv = its valid token count
            auto scores = [&](int nv) __attribute__((always_inline)) {
#pragma unroll
                for (int r = 0; r < 16; ++r) s[r] = sa[r] + sb[r];
                if constexpr (SPARSE) {
                    // nv: bit t set when token t of the tile is valid
                    if (nv != -1) {
                        const int h4 = 4 * (lane_id64() >> 5);
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int tok = 8 * (r >> 2) + h4 + (r & 3);
                            if (!(((uint32_t)nv >> tok) & 1u)) s[r] = -INFINITY;
                        }
                    }
                } else if (nv < kSubTok) {
                    const int h4 = 4 * (lane_id64() >> 5);
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int c_r = 8 * (r >> 2) + (r & 3);
                        if (!(h4 < nv - c_r)) s[r] = -INFINITY;
                    }
                }
            };
            // The valid token count of tile k is written with its copy in step
            // k - 2; step k - 1 asks for it with its first fragment reads and
            // uses it at its end, so the read's latency is hidden.
            // step -1: QK(0)
            int nv_raw = 0;
            // a tile's validity: its token count (dense) or token bits (top-k)
            auto valid_of = [&](int b) __attribute__((always_inline)) -> int {
                if constexpr (SPARSE) return sm.vmask[b][0] | sm.vmask[b][1];
                else return sm.valid[b];
            };
            qk(0, Int<0>{}, 0, [&] { nv_raw = valid_of(0); });
            int nv = __builtin_amdgcn_readfirstlane(nv_raw);
            barrier_lds();
            // steps 0 .. n-2: softmax(k) and QK(k+1)
            for (int k = 0; k + 1 < sg.n; ++k) {
                qk(k + 1, Int<1>{}, k & 1, [&] { scores(nv); nv_raw = valid_of((k + 1) % kRing); });
                nv = __builtin_amdgcn_readfirstlane(nv_raw);
                barrier_lds();
            }
            // step n-1: the last softmax, then the output scale and lse
            {
                const int k = sg.n - 1;
                seg_read(sg);
                scores(nv);
                unroll<0, kSoftStages>([&](auto st_c) __attribute__((always_inline)) { soft_stage(st_c, k & 1); });
                const int l = lane_id64();
                const int hd = hblk * kH + hbq * 32 + (l & 31);
                const float lse_v = l_run > 0.f ? (c * m_run + log2f(l_run)) * 0.69314718055994531f
                                                 : (l_run == 0.f ? -INFINITY : __builtin_nanf(""));
                float inv = l_run > 0.f ? 1.f / l_run : 0.f;
                // attention sink on a final output; a row that saw nothing stays 0
                // (with lse = sink = -inf the factor would be NaN)
                if (sg.final_out && a.attn_sink && hd < H && l_run > 0.f)
                    inv *= 1.f / (1.f + __expf(a.attn_sink[hd] - lse_v));
                sm.fin_inv[hbq * 32 + (l & 31)] = inv;
                if (l < 32 && hd < H && sg.write_ok) {
                    if (sg.final_out) a.lse[((int64_t)sg.b * H + hd) * a.s_q + sg.iq] = lse_v;
                    else a.lse_part[(int64_t)sg.slot * H + hd] = lse_v;
                }
                barrier_lds();
            }
            barrier_lds();   // step n
            barrier_lds();   // epilogue
            barrier_lds();   // epilogue: rows staged in LDS
            barrier_lds();   // the next segment reuses every LDS array
        }
    } else {
        // -------------------------------------------------------------------- PV waves
        for (int j = jb; j <= je && j < N; ++j) {
            Seg sg;
            if (!segment(j, sg)) continue;
            // acc[hb][d], register r, lane l: head 32 hb + l % 32, dim 128 dq +
            // 32 d + 8 (r / 4) + 4 half + r % 4
            f32x16 acc[2][4];
#pragma unroll
            for (int hb = 0; hb < 2; ++hb)
#pragma unroll
                for (int d = 0; d < 4; ++d) acc[hb][d] = f32x16{};
            barrier_lds();   // tile 0 has landed
            barrier_lds();   // step -1
            // V^T operand (transposed read): lane (gq = l / 16, i16 = l % 16)
            // reads 8 bytes (byte 8 (i16 % 2) of the 16-byte chunk) of token
            // 16 ks + 8 r + 4 (gq / 2) + i16 / 4 and column 16 dq + 4 d + 2 (gq % 2)
            // + (i16 % 4) / 2, r = 0, 1 for the two reads of a fragment.  The
            // byte offset is 8192 dq + 4096 (d / 2) + 2048 ks plus a lane term
            // vb[d % 2][r].
            int vb[2][2];
            {
                const int l = lane_id64();
                const int gq = l >> 4, i16 = l & 15;
                const int x = 2 * (gq & 1) + ((i16 & 3) >> 1);
                const int tq = 4 * (gq >> 1) + (i16 >> 2);
#pragma unroll
                for (int e = 0; e < 2; ++e)
#pragma unroll
                    for (int r = 0; r < 2; ++r) vb[e][r] = tile_chunk(8 * r + tq, 4 * e + x) * 16 + 8 * (i16 & 1);
            }
            // fragment i = (dim block i / 2, k-step i % 2) of tile t, ring slot i % (kPvLA + 1)
            bf16x8 fr[kPvLA + 1];
            auto fetch = [&](int t, int i) __attribute__((always_inline)) -> bf16x8 {
                const int d = i >> 1, ks = i & 1;
                const unsigned char* Tv = sm.tile[0] + ring_offset(t % kRing) + 8192 * dq + 4096 * (d >> 1) + 2048 * ks;
                const bf16x4 v0 = tr_read64(Tv + vb[d & 1][0]);
                const bf16x4 v1 = tr_read64(Tv + vb[d & 1][1]);
                return bf16x8{v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
            };
            // the first fragments of tile t, read in the step before its PV (tile t
            // is resident from step t - 1 to step t + 1)
            auto prefetch = [&](int t) __attribute__((always_inline)) {
#pragma unroll
                for (int i = 0; i < kPvLA; ++i) fr[i] = fetch(t, i);
            };
            // PV(t): O^T += V^T P^T for the four 32-dim blocks of this wave's
            // quarter and both head blocks; each block is rescaled by alpha
            // before its first MFMA, the multiplies of block d + 1 placed between
            // the MFMAs of block d.  V fragments are read kPvLA ahead; the order
            // is fixed with scheduling fences.
            auto pv = [&](int t, float al0, float al1, bool rs0, bool rs1, const bf16x8 (&P)[2][2]) __attribute__((always_inline)) {
                if (rs0) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[0][0][r] *= al0;
                }
                if (rs1) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[1][0][r] *= al1;
                }
                __builtin_amdgcn_sched_barrier(0);
                unroll<0, 8>([&](auto i_c) __attribute__((always_inline)) {
                    constexpr int i = decltype(i_c)::value;
                    constexpr int d = i >> 1, ks = i & 1;
                    const bf16x8 A = fr[i % (kPvLA + 1)];
                    const bool rs = ks ? rs1 : rs0;
                    acc[0][d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, P[0][ks], acc[0][d], 0, 0, 0);
                    if constexpr (d + 1 < 4) {
                        if (rs) {
#pragma unroll
                            for (int r = 0; r < 8; ++r) acc[ks][d + 1][r] *= ks ? al1 : al0;
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    acc[1][d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, P[1][ks], acc[1][d], 0, 0, 0);
                    if constexpr (d + 1 < 4) {
                        if (rs) {
#pragma unroll
                            for (int r = 8; r < 16; ++r) acc[ks][d + 1][r] *= ks ? al1 : al0;
                        }
                    }
                    if constexpr (i + kPvLA < 8) fr[(i + kPvLA) % (kPvLA + 1)] = fetch(t, i + kPvLA);
                    __builtin_amdgcn_sched_barrier(0);
                });
            };
            prefetch(0);
            barrier_lds();   // step 0
            for (int k = 1; k <= sg.n; ++k) {
                const int t = k - 1, ts = t & 1;
                const int l = lane_id64();
                bf16x8 P[2][2];
#pragma unroll
                for (int hb = 0; hb < 2; ++hb)
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) P[hb][ks] = sm.p[ts][hb][ks][l];
                const float al0 = sm.alpha[ts][0][l & 31], al1 = sm.alpha[ts][1][l & 31];
                // a head block's rescale is skipped when none of its heads' max rose
                // (alpha = 1 for all 32)
                const bool rs0 = __builtin_amdgcn_ballot_w64(al0 != 1.f) != 0;
                const bool rs1 = __builtin_amdgcn_ballot_w64(al1 != 1.f) != 0;
                pv(t, al0, al1, rs0, rs1, P);
                if (k < sg.n) prefetch(k);
                // the prefetch reads stay in flight across the barrier: this wave
                // writes no LDS, and tile k is not overwritten before step k + 2
                barrier_only();
            }
            barrier_lds();   // epilogue: fin_inv was written in step n - 1
            seg_read(sg);
            // ---- epilogue: normalise and store.  Two-byte outputs (float16
            // partials, bf16 output) go through LDS as a row-major 64 x 512
            // tile, so that every store instruction writes one head's whole
            // 1 KiB row; the accumulator layout would otherwise spread a store
            // over 32 rows in 16-byte pieces.  Each format has its own
            // straight-line code, which keeps the code fetched once per launch
            // short.
            const bool part16 = !sg.final_out && a.part_fp16;
            const bool staged = part16 || (sg.final_out && !a.out_fp32);
            unsigned char* X = sm.tile[0];
            const int l = lane_id64();
            const int hf = l >> 5;
            // rows of head block hb into X, scaled by sc (per lane: one head)
            auto stage = [&](auto f16_c, int hb, float sc) __attribute__((always_inline)) {
                constexpr bool F16 = decltype(f16_c)::value != 0;
                unsigned char* xp = X + (hb * 32 + (l & 31)) * kXRow + 2 * (128 * dq + 4 * hf);
#pragma unroll
                for (int d = 0; d < 4; ++d) {
#pragma unroll
                    for (int rq = 0; rq < 4; ++rq) {
                        const float v0 = acc[hb][d][4 * rq + 0] * sc, v1 = acc[hb][d][4 * rq + 1] * sc;
                        const float v2 = acc[hb][d][4 * rq + 2] * sc, v3 = acc[hb][d][4 * rq + 3] * sc;
                        if constexpr (F16) *(f16x4*)(xp + 2 * (32 * d + 8 * rq)) = f16x4{(_Float16)v0, (_Float16)v1, (_Float16)v2, (_Float16)v3};
                        else *(bf16x4*)(xp + 2 * (32 * d + 8 * rq)) = bf16x4{(__bf16)v0, (__bf16)v1, (__bf16)v2, (__bf16)v3};
                    }
                }
            };
            if (sg.write_ok && part16) {
#pragma unroll
                for (int hb = 0; hb < 2; ++hb) {
                    const int head = hblk * kH + hb * 32 + (l & 31);
                    const float inv = sm.fin_inv[hb * 32 + (l & 31)];
                    float amax = 0.f;
#pragma unroll
                    for (int d = 0; d < 4; ++d)
#pragma unroll
                        for (int r = 0; r < 16; ++r) amax = fmaxf(amax, fabsf(acc[hb][d][r]));
                    amax *= inv;
                    const int be = (int)((__float_as_uint(amax) >> 23) & 0xff);
                    int E = amax > 0.f ? (be == 0 ? -125 : be - 126) : 0;        // amax * 2^-E < 1
                    E = E > 127 ? 127 : E;
                    if (head < H) a.o_exp8[((int64_t)sg.slot * H + head) * 8 + 2 * dq + hf] = (unsigned char)(signed char)E;
                    stage(Int<1>{}, hb, ldexpf(inv, -E));
                }
            } else if (sg.write_ok && staged) {
#pragma unroll
                for (int hb = 0; hb < 2; ++hb) stage(Int<0>{}, hb, sm.fin_inv[hb * 32 + (l & 31)]);
            } else if (sg.write_ok) {
                // float32 output or partials: stored from the accumulator layout
#pragma unroll
                for (int hb = 0; hb < 2; ++hb) {
                    const int head = hblk * kH + hb * 32 + (l & 31);
                    if (head >= H) continue;
                    const float inv = sm.fin_inv[hb * 32 + (l & 31)];
                    float* base = sg.final_out ? (float*)a.out + ((int64_t)j * H + head) * kDv
                                               : a.o_part + ((int64_t)sg.slot * H + head) * kDv;
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
#pragma unroll
                        for (int rq = 0; rq < 4; ++rq) {
                            const int dim = 128 * dq + 32 * d + 8 * rq + 4 * hf;
                            *(f32x4*)(base + dim) = f32x4{acc[hb][d][4 * rq + 0] * inv, acc[hb][d][4 * rq + 1] * inv,
                                                          acc[hb][d][4 * rq + 2] * inv, acc[hb][d][4 * rq + 3] * inv};
                        }
                    }
                }
            }
            barrier_lds();   // the staged rows are in LDS
            if (sg.write_ok && staged) {
                // wave dq stores rows 16 dq .. 16 dq + 15, lane l bytes 16 l .. 16 l + 15
                const int h0 = hblk * kH + 16 * dq;
                const int64_t row0 = (part16 ? (int64_t)sg.slot : (int64_t)j) * H + h0;
                unsigned char* gp = (unsigned char*)a.o_part + 0;
                if (!part16) gp = (unsigned char*)a.out;
                gp += row0 * (2 * kDv) + 16 * l;
                const unsigned char* xp = X + 16 * dq * kXRow + 16 * l;
                if (h0 + 16 <= H) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) *(i32x4*)(gp + i * (2 * kDv)) = *(const i32x4*)(xp + i * kXRow);
                } else {
#pragma unroll 1
                    for (int i = 0; i < H - h0; ++i) *(i32x4*)(gp + i * (2 * kDv)) = *(const i32x4*)(xp + i * kXRow);
                }
            }
            barrier_lds();   // the next segment reuses every LDS array
        }
    }
}

hipError_t launch_decode64(const DecodeArgs& a, hipStream_t stream) {
    const dim3 grid(a.num_parts * a.n_hblk), block(kT);
    if (a.topk > 0) {
        if (a.fused) hipLaunchKernelGGL((decode64_kernel<true, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((decode64_kernel<false, true>), grid, block, 0, stream, a);
    } else {
        if (a.fused) hipLaunchKernelGGL((decode64_kernel<true, false>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((decode64_kernel<false, false>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace mla
