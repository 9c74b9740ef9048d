// Split-KV partial-attention kernel for absorbed-MLA decode on gfx950.
//
// One workgroup = 128 query heads x one scheduler partition (a contiguous run
// of 64-token KV pages, possibly spanning several items), so every cache page
// is read from HBM once per query token.  Eight waves, two per SIMD, 256
// registers each; wave w owns head block hb = w & 3 (32 heads) and half
// kh = w >> 2.  Each page is computed as two 32-token tiles:
//
//   fill   tiles are copied global -> LDS with 16-byte buffer loads that
//          write LDS directly (bf16 cache; two tiles in flight, three LDS
//          buffers), or loaded to registers, dequantised and stored (FP8
//          cache).  Masked tokens fall outside the buffer range and land as
//          zeros;
//   QK     the two waves of a head block split the 576 dims: wave kh runs
//          S^T = K Q^T over latent dims 256*kh.. and half of the RoPE dims
//          with v_mfma_f32_32x32x16_bf16 (Q in registers, RoPE part of Q in
//          LDS), then the pair adds its partial S^T through LDS.  Tokens sit
//          on the MFMA rows, so each lane holds one head's scores;
//   soft   both waves of a head block run the same exact online softmax
//          (running max updated on every increase, p = exp2(s*c - m) in fp32,
//          l sums the fp32 p, P rounded to bf16 for the PV product);
//   PV     wave kh accumulates O^T for dims 256*kh.. of its 32 heads; the
//          transposed V operand is read straight from the row-major LDS tile
//          with ds_read_b64_tr_b16 and P^T is the wave's own S^T registers.
//
// Items whose KV range sits in one partition write out/lse directly; split
// items write normalised fp32 partials for the combine kernel.

#include "common.h"
#include "kernels.h"

namespace mla {

constexpr int kSubBytes = kSubTok * kRowBytes;   // 36864
constexpr int kNBuf = 3;

struct __attribute__((aligned(16))) Smem {
    unsigned char tile[kNBuf][kSubBytes];   // 32-token KV tiles (bf16, swizzled)
    f32x4 xs[4][2][4][64];                  // partial S^T [head block][dim half][register quad][lane]
    bf16x8 qr[4][4][64];                    // RoPE part of Q as B fragments [head block][k-step][lane]
    int rows[4][kSubTok];                   // sparse: row ids of upcoming tiles (ring of 4)
};

__device__ __forceinline__ bf16x4 tr_read(const unsigned char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(p));
}

__device__ __forceinline__ bf16x8 pack8(const float* v) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (__bf16)v[e];
    return r;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int stride, int num_records) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)stride, num_records, 0x00020000);
}

// ---- bf16 tile fill: 36 pieces of 1 KB = LDS columns 2k, 2k+1; wave w issues
// pieces w, w+8, w+16, w+24 and, for w < 4, 32+w.  All pieces of a wave have
// k & 1 = w & 1, so lane l always reads token ft = (l & 31) ^ (4 half + 8 (w & 1))
// and column 2k + half: source offset ft*1152 + 16 half + 32k.
__device__ __forceinline__ int fill_loads(int wave) { return wave < 4 ? 5 : 4; }

// dense: the tile is one half of a 64-token page; tokens >= tok_valid are masked
__device__ __forceinline__ void fill_dense(unsigned char* dst, const unsigned char* kv, int page, int sub,
                                           int tok_valid, int64_t num_rows, int fbase, int wave) {
    const bool ok = page_ok(page, num_rows);
    int nvalid = tok_valid < kSubTok ? tok_valid : kSubTok;
    if (!ok || nvalid < 0) nvalid = 0;
    const unsigned char* base = kv + (ok ? (int64_t)page * kTileBytes + sub * kSubBytes : 0);
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(base, 0, nvalid * kRowBytes);
#pragma unroll
    for (int i = 0; i < 5; ++i) {
        if (i == 4 && wave >= 4) break;
        const int k = i < 4 ? wave + 8 * i : 32 + wave;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(dst + k * 1024), 16, fbase + 32 * k, 0, 0, 0);
    }
}

// sparse: the lane's row id from the LDS ring (-1 = masked -> index out of range)
__device__ __forceinline__ void fill_sparse(unsigned char* dst, __amdgpu_buffer_rsrc_t rs, int row, int fcol,
                                            int wave) {
#pragma unroll
    for (int i = 0; i < 5; ++i) {
        if (i == 4 && wave >= 4) break;
        const int k = i < 4 ? wave + 8 * i : 32 + wave;
        __builtin_amdgcn_struct_ptr_buffer_load_lds(rs, (lds_void_t*)(dst + k * 1024), 16, (unsigned)row,
                                                    fcol + 32 * k, 0, 0, 0);
    }
}

// ---- FP8 tile fill: thread (token t = tid/16, part p = tid%16) owns latent
// dims 32p..32p+31 (one scale tile) and, for p < 8, RoPE chunk p.
struct Fp8Regs {
    i32x4 codes[2];
    float scale;
    i32x4 rope;
};

__device__ __forceinline__ void fp8_load(Fp8Regs& r, const unsigned char* kv, int64_t row, int p) {
    const i32x4 z = {0, 0, 0, 0};
    r.codes[0] = z;
    r.codes[1] = z;
    r.scale = 0.f;
    r.rope = z;
    if (row >= 0) {
        const unsigned char* base = kv + row * kFp8RowBytes;
        r.codes[0] = *(const i32x4*)(base + 32 * p);
        r.codes[1] = *(const i32x4*)(base + 32 * p + 16);
        r.scale = *(const float*)(base + 512 + 4 * (p >> 2));
        if (p < 8) r.rope = *(const i32x4*)(base + 528 + 16 * p);
    }
}

// e4m3fn -> fp32 (exact), x scale in fp32, -> bf16 (round to nearest even)
__device__ __forceinline__ void fp8_store(unsigned char* dst, const Fp8Regs& r, int t, int p) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        float v[16];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const int word = r.codes[h][w];
            auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(word, false);
            auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(word, true);
            v[4 * w + 0] = lo[0] * r.scale;
            v[4 * w + 1] = lo[1] * r.scale;
            v[4 * w + 2] = hi[0] * r.scale;
            v[4 * w + 3] = hi[1] * r.scale;
        }
        *(bf16x8*)(dst + lds_chunk(t, 4 * p + 2 * h) * 16) = pack8(v);
        *(bf16x8*)(dst + lds_chunk(t, 4 * p + 2 * h + 1) * 16) = pack8(v + 8);
    }
    if (p < 8) *(i32x4*)(dst + lds_chunk(t, 64 + p) * 16) = r.rope;
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

// s_waitcnt vmcnt(n) for a wave-uniform n in {0, 4, 5}
__device__ __forceinline__ void wait_vm(int n) {
    if (n >= 5) __builtin_amdgcn_s_waitcnt(0x0F75);
    else if (n == 4) __builtin_amdgcn_s_waitcnt(0x0F74);
    else __builtin_amdgcn_s_waitcnt(0x0F70);
}

template <bool SPARSE, bool FP8>
__global__ void __launch_bounds__(kThreads, 1) decode_kernel(const DecodeArgs a) {
    __shared__ Smem sm;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hb = wave & 3;          // head block: heads 32*hb .. +31 of the workgroup
    const int kh = wave >> 2;         // half: QK dims and PV output dims
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
    const int32_t* so = a.meta + kMetaHeader + kMetaRec * a.num_parts;
    const int jb = sload(rec + 0), tbeg = sload(rec + 1), je = sload(rec + 2), tend = sload(rec + 3);
    const int slot0 = sload(rec + 4);
    const int N = a.batch * a.s_q;
    const int H = a.h_q;
    const float c = a.scale_log2;
    const unsigned char* kv = (const unsigned char*)a.kv;

    RowResolver rr{a.block_table, a.cache_seqlens, a.indices, a.s_q, a.max_blocks, SPARSE ? a.topk : 0,
                   a.causal, a.num_rows};

    const int head = hblk * kHeadsPerWG + hb * 32 + l32;   // this lane's head
    const bool head_ok = head < H;

    const __amdgpu_buffer_rsrc_t srs = buffer_rsrc(kv, kRowBytes, (int)a.num_rows);
    const int f8_tok = tid >> 4, f8_p = tid & 15;    // FP8 fill role
    const int nload = fill_loads(wave);
    const int ftok = l32 ^ (4 * half + 8 * (wave & 1));   // bf16 fill: token this lane copies
    const int fbase = ftok * kRowBytes + 16 * half;       // dense fill source offset (+32k)
    const int fcol = 16 * half;                            // sparse fill column offset (+32k)

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
        const int nslots = rr.slots_uniform(j);
        const int ntile_j = (nslots + 63) >> 6;
        const int t0 = (j == jb && tbeg > 0) ? tbeg : 0;
        int t1 = (j == je) ? tend : ntile_j;
        if (t1 > ntile_j) t1 = ntile_j;
        if (t0 >= t1) continue;
        const int nsplit = sload(so + j + 1) - sload(so + j);
        const int slot = (j == jb) ? slot0 : sload(so + j);
        const int g0 = 2 * t0;                                    // first 32-token tile
        const int gend = min(2 * t1, (nslots + kSubTok - 1) / kSubTok);
        const int ns = gend - g0;

        // ---- Q: latent dims 256*kh.. in registers, RoPE part to LDS ----
        bf16x8 qf[16];
        {
            const bf16x8* qp = (const bf16x8*)((const unsigned char*)a.q +
                                               ((int64_t)j * H + (head_ok ? head : 0)) * kRowBytes);
#pragma unroll
            for (int kk = 0; kk < 16; ++kk) {
                bf16x8 v = qp[32 * kh + 2 * kk + half];
                if (!head_ok) v = bf16x8{};
                qf[kk] = v;
            }
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int idx = tid + kThreads * e;          // 0..1023 = [hb2][kr][lane]
                const int ln = idx & 63, kr = (idx >> 6) & 3, hb2 = idx >> 8;
                const int hq = hblk * kHeadsPerWG + hb2 * 32 + (ln & 31);
                bf16x8 v = {};
                if (hq < H)
                    v = ((const bf16x8*)((const unsigned char*)a.q + ((int64_t)j * H + hq) * kRowBytes))[64 + 2 * kr + (ln >> 5)];
                sm.qr[hb2][kr][ln] = v;
            }
        }

        f32x16 acc[8];
#pragma unroll
        for (int d = 0; d < 8; ++d) acc[d] = f32x16{};
        float m_run = -INFINITY, l_run = 0.f;

        // dense: page ids of tiles it, it+1, it+2 (one 64-token page = two tiles)
        auto page_of = [&](int g) { return rr.page_uniform(j, g >> 1); };
        int pg0 = 0, pg1 = 0, pg2 = 0;
        if (!SPARSE) {
            pg0 = page_of(g0);
            pg1 = ns > 1 ? page_of(g0 + 1) : 0;
            pg2 = ns > 2 ? page_of(g0 + 2) : 0;
        }
        if (SPARSE && wave == 0 && lane < kSubTok) {
#pragma unroll
            for (int u = 0; u < 3; ++u)
                if (u < ns) sm.rows[u][lane] = (int)rr.row(j, (g0 + u) * kSubTok + lane, nslots);
        }
        lds_barrier();

        auto issue_fill = [&](int it, int page) {
            const int g = g0 + it;
            unsigned char* dst = sm.tile[it % kNBuf];
            if (SPARSE) fill_sparse(dst, srs, sm.rows[it & 3][ftok], fcol, wave);
            else fill_dense(dst, kv, page, g & 1, nslots - g * kSubTok, a.num_rows, fbase, wave);
        };
        Fp8Regs f8;
        auto fp8_row = [&](int it, int page) -> int64_t {
            const int g = g0 + it;
            if (SPARSE) return sm.rows[it & 3][f8_tok];
            return row_in_page(page, (g & 1) * kSubTok + f8_tok, nslots - (g & ~1) * kSubTok, a.num_rows);
        };
        if (FP8) {
            fp8_load(f8, kv, fp8_row(0, pg0), f8_p);
            fp8_store(sm.tile[0], f8, f8_tok, f8_p);
        } else {
            issue_fill(0, pg0);
            if (ns > 1) issue_fill(1, pg1);
        }

        for (int it = 0; it < ns; ++it) {
            const int g = g0 + it;
            const unsigned char* T = sm.tile[it % kNBuf];
            if (!FP8) wait_vm(it + 1 < ns ? nload : 0);
            lds_barrier();                                 // tile it ready; tile it-1 finished everywhere

            // sparse: row ids of tile it+3 (issued before the fills so that waiting
            // for them never waits for a tile)
            int next_row = -1;
            if (SPARSE && wave == 0 && lane < kSubTok && it + 3 < ns)
                next_row = (int)rr.row(j, (g + 3) * kSubTok + lane, nslots);
            // keep the pipeline full: tile it+2 (bf16) or it+1 (FP8) in flight
            if (FP8) {
                if (it + 1 < ns) fp8_load(f8, kv, fp8_row(it + 1, pg1), f8_p);
            } else if (it + 2 < ns) {
                issue_fill(it + 2, pg2);
            }
            const int pg_cur = pg0;
            if (!SPARSE) {
                pg0 = pg1;
                pg1 = pg2;
                pg2 = it + 3 < ns ? page_of(g + 3) : 0;
            }

            // ---- QK: partial S^T[32 tokens x 32 heads] over this wave's dims ----
            f32x16 s = {};
            const unsigned char* Tk = T + 16384 * kh;
#pragma unroll
            for (int kk = 0; kk < 16; ++kk) {
                const bf16x8 kf = *(const bf16x8*)(Tk + kb[kk & 1] + 1024 * kk);
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], s, 0, 0, 0);
            }
#pragma unroll
            for (int r2 = 0; r2 < 2; ++r2) {
                const int kr = 2 * kh + r2;     // RoPE column 64 + 2kr + half
                const bf16x8 kf = *(const bf16x8*)(T + 32768 + kb[kr & 1] + 1024 * kr);
                const bf16x8 qv = sm.qr[hb][kr][lane];
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qv, s, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) sm.xs[hb][kh][i][lane] = f32x4{s[4 * i], s[4 * i + 1], s[4 * i + 2], s[4 * i + 3]};
            lds_barrier();

            // ---- full scores: own + partner partial; mask; scale (in place) ----
            // register r -> token 8(r/4) + 4*half + r%4 of the tile
            {
                const int tv = nslots - g * kSubTok;
                const bool pg = SPARSE ? true : page_ok(pg_cur, a.num_rows);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const f32x4 o = sm.xs[hb][kh ^ 1][i][lane];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int tok = 8 * i + 4 * half + e;
                        const bool valid = SPARSE ? (sm.rows[it & 3][tok] >= 0) : (pg && tok < tv);
                        s[4 * i + e] = valid ? (s[4 * i + e] + o[e]) * c : -INFINITY;
                    }
                }
            }

            // ---- exact online softmax over the tile's 32 tokens ----
            float mx = -INFINITY;
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
            mx = wave_max_pair(mx);
            const float m_new = fmaxf(m_run, mx);
            float alpha = 1.f, psum = 0.f;
            if (m_new == -INFINITY) {
                s = f32x16{};
            } else {
                alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    s[r] = __builtin_amdgcn_exp2f(s[r] - m_new);
                    psum += s[r];
                }
            }
            psum = wave_sum_pair(psum);
            l_run = l_run * alpha + psum;
            m_run = m_new;
            bf16x8 p0, p1;
#pragma unroll
            for (int e = 0; e < 8; ++e) { p0[e] = (__bf16)s[e]; p1[e] = (__bf16)s[8 + e]; }

            // ---- PV: O^T[dims 256kh + 32d .., heads] = alpha O^T + V^T P^T ----
            if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {
#pragma unroll
                for (int d = 0; d < 8; ++d) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[d][r] *= alpha;
                }
            }
#pragma unroll
            for (int j2 = 0; j2 < 2; ++j2) {
                const bf16x8 pf = j2 == 0 ? p0 : p1;
                const unsigned char* Tv = T + 256 * j2 + 16384 * kh;
#pragma unroll
                for (int d = 0; d < 8; ++d) {
                    const bf16x4 v0 = tr_read(Tv + vb[0] + 2048 * d);
                    const bf16x4 v1 = tr_read(Tv + vb[1] + 2048 * d);
                    const bf16x8 vf = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
                    acc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, acc[d], 0, 0, 0);
                }
            }

            if (FP8 && it + 1 < ns) fp8_store(sm.tile[(it + 1) % kNBuf], f8, f8_tok, f8_p);
            if (SPARSE && wave == 0 && lane < kSubTok && it + 3 < ns) sm.rows[(it + 3) & 3][lane] = next_row;
        }

        // ---- epilogue: both waves of a head block hold the same m, l ----
        const bool final_out = (nsplit == 1);
        const int b = j / a.s_q, iq = j - b * a.s_q;
        if (head_ok && (final_out || (slot >= 0 && slot < a.max_slots))) {
            const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
            for (int d = 0; d < 8; ++d) {
#pragma unroll
                for (int rq = 0; rq < 4; ++rq) {
                    const int dim = 256 * kh + 32 * d + 8 * rq + 4 * half;
                    const float v0 = acc[d][4 * rq + 0] * inv, v1 = acc[d][4 * rq + 1] * inv;
                    const float v2 = acc[d][4 * rq + 2] * inv, v3 = acc[d][4 * rq + 3] * inv;
                    if (final_out) {
                        const int64_t o = ((int64_t)j * H + head) * kDv + dim;
                        if (a.out_fp32) {
                            *(f32x4*)((float*)a.out + o) = f32x4{v0, v1, v2, v3};
                        } else {
                            const bf16x4 w = {(__bf16)v0, (__bf16)v1, (__bf16)v2, (__bf16)v3};
                            *(bf16x4*)((__bf16*)a.out + o) = w;
                        }
                    } else {
                        const int64_t o = ((int64_t)slot * H + head) * kDv + dim;
                        *(f32x4*)(a.o_part + o) = f32x4{v0, v1, v2, v3};
                    }
                }
            }
            if (kh == 0 && lane < 32) {
                const float lse_v = l_run > 0.f ? (m_run + log2f(l_run)) * 0.69314718055994531f : -INFINITY;
                if (final_out) a.lse[((int64_t)b * H + head) * a.s_q + iq] = lse_v;
                else a.lse_part[(int64_t)slot * H + head] = lse_v;
            }
        }
        lds_barrier();
    }
}

hipError_t launch_decode(const DecodeArgs& a, bool sparse, bool fp8, hipStream_t stream) {
    const dim3 grid(a.num_parts * a.n_hblk), block(kThreads);
    if (sparse) {
        if (fp8) hipLaunchKernelGGL((decode_kernel<true, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((decode_kernel<true, false>), grid, block, 0, stream, a);
    } else {
        if (fp8) hipLaunchKernelGGL((decode_kernel<false, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((decode_kernel<false, false>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace mla
