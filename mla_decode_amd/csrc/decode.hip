// Split-KV partial-attention kernel for absorbed-MLA decode on gfx950.
//
// One workgroup = 64 query heads of one head block x one scheduler partition
// (a contiguous run of 64-token KV tiles, possibly spanning several items).
// Four waves, one per SIMD, 512 registers each.  Per KV tile:
//
//   fill   the next tile is copied global -> LDS with direct-to-LDS 16-byte
//          loads (bf16 cache) or loaded to registers, dequantised and stored
//          (FP8 cache), while the current tile is computed (double buffer);
//   QK     wave (tb, hq) computes S^T = K Q^T for tokens 32*tb.. and heads
//          32*hq.. with v_mfma_f32_32x32x16_bf16; K comes from LDS, Q stays in
//          registers for the whole segment.  Putting tokens on the MFMA rows
//          leaves one head per lane, so the row max and row sum over tokens
//          are in-register plus one permlane32 swap;
//   soft   exact running max (the pair of waves sharing a head block swaps
//          tile maxima through LDS), p = exp2(s*c - m) in fp32, l accumulates
//          the fp32 p, P is rounded to bf16 for the PV product;
//   PV     wave w accumulates O^T for dims 128*w.. and all 64 heads; the
//          transposed V operand comes straight from the row-major LDS tile
//          with ds_read_b64_tr_b16, and the bf16 P fragments are exactly the
//          QK accumulator registers, exchanged through 8 KB of LDS.
//
// Items whose KV range sits in one partition write out/lse directly; split
// items write normalised fp32 partials for the combine kernel.

#include "common.h"
#include "kernels.h"

namespace mla {

struct __attribute__((aligned(16))) Smem {
    unsigned char tile[2][kTileBytes];   // double-buffered KV tile (bf16, swizzled)
    unsigned char p[4 * 2 * 64 * 16];    // P^T fragments [kstep][head half][lane]
    float red_max[2][2][32];             // tile maxima [head half][token half][head]
    float alpha[2][32];                  // rescale factors [head half][head]
    float lsum[2][2][32];                // final row sums [head half][token half][head]
    int rows[4][64];                     // sparse: row ids of upcoming tiles (ring)
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

// ---- tile fill, bf16 cache: 72 direct-to-LDS buffer loads of 1 KB per workgroup ----
// Lane ``lane`` of piece k = wave + 4i writes LDS chunk s = 64k + lane, i.e. token
// t = s / 72 and source chunk (s % 72) ^ swz(t).  For pieces i and i + 9 the
// chunk is the same and the token is 32 further, so nine precomputed offsets
// serve all eighteen loads.  Masked tokens read out of the buffer's range and
// land as zeros.
struct FillPlan {
    int voff[9];     // dense: t*1152 + chunk*16 ; sparse: chunk*16
    int tok[9];      // token of piece i (i < 9); piece i + 9 holds tok + 32
};

__device__ __forceinline__ void make_fill_plan(FillPlan& fp, int wave, int lane, bool sparse) {
#pragma unroll
    for (int i = 0; i < 9; ++i) {
        const int s = 64 * (wave + 4 * i) + lane;
        const int t = s / kRowChunks;
        const int cch = (s - t * kRowChunks) ^ swz(t);
        fp.tok[i] = t;
        fp.voff[i] = sparse ? cch * 16 : t * kRowBytes + cch * 16;
    }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int stride, int num_records) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)stride, num_records, 0x00020000);
}

// dense: one page = one tile, contiguous 73728 bytes; tokens >= tok_valid are masked
__device__ __forceinline__ void fill_dense(unsigned char* dst, const unsigned char* kv, int page, int tok_valid,
                                           int64_t num_rows, const FillPlan& fp, int wave) {
    int nvalid = tok_valid < kBlock ? tok_valid : kBlock;
    if (!page_ok(page, num_rows) || nvalid < 0) nvalid = 0;
    const unsigned char* base = kv + (page_ok(page, num_rows) ? (int64_t)page * kTileBytes : 0);
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(base, 0, nvalid * kRowBytes);
#pragma unroll
    for (int i = 0; i < 18; ++i) {
        const int k = wave + 4 * i;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(dst + k * 1024), 16, fp.voff[i % 9],
                                                 i < 9 ? 0 : 32 * kRowBytes, 0, 0);
    }
}

// sparse: rows come from the LDS ring (-1 = masked -> index out of range)
__device__ __forceinline__ void fill_sparse(unsigned char* dst, __amdgpu_buffer_rsrc_t rs, const int* rows,
                                            const FillPlan& fp, int wave) {
#pragma unroll
    for (int i = 0; i < 18; ++i) {
        const int k = wave + 4 * i;
        const int r = rows[fp.tok[i % 9] + (i < 9 ? 0 : 32)];
        __builtin_amdgcn_struct_ptr_buffer_load_lds(rs, (lds_void_t*)(dst + k * 1024), 16, (unsigned)r,
                                                    fp.voff[i % 9], 0, 0, 0);
    }
}

// ---- tile fill, FP8 cache: thread (token t, quarter q) owns code chunks q, q+4, ...
struct Fp8Regs {
    i32x4 codes[8];   // 8 x 16 e4m3 codes
    f32x4 scales;     // the token's four tile scales
    i32x4 rope[2];    // 16 RoPE values (bf16)
};

__device__ __forceinline__ void fp8_load(Fp8Regs& r, const unsigned char* kv, int64_t row, int q) {
    if (row >= 0) {
        const unsigned char* base = kv + row * kFp8RowBytes;
#pragma unroll
        for (int i = 0; i < 8; ++i) r.codes[i] = *(const i32x4*)(base + 16 * (q + 4 * i));
        r.scales = *(const f32x4*)(base + 512);
        r.rope[0] = *(const i32x4*)(base + 528 + 32 * q);
        r.rope[1] = *(const i32x4*)(base + 528 + 32 * q + 16);
    } else {
        const i32x4 z = {0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 8; ++i) r.codes[i] = z;
        r.scales = f32x4{0.f, 0.f, 0.f, 0.f};
        r.rope[0] = z;
        r.rope[1] = z;
    }
}

// e4m3fn -> fp32 (exact, hardware OCP conversion), x scale in fp32, -> bf16 (RNE)
__device__ __forceinline__ void fp8_store(unsigned char* dst, const Fp8Regs& r, int t, int q) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int cc = q + 4 * i;                 // 16-code chunk index = dims 16*cc ..
        const float sc = r.scales[cc >> 3];
        float v[16];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const int word = r.codes[i][w];
            auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(word, false);
            auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(word, true);
            v[4 * w + 0] = lo[0] * sc;
            v[4 * w + 1] = lo[1] * sc;
            v[4 * w + 2] = hi[0] * sc;
            v[4 * w + 3] = hi[1] * sc;
        }
        *(bf16x8*)(dst + lds_chunk(t, 2 * cc) * 16) = pack8(v);
        *(bf16x8*)(dst + lds_chunk(t, 2 * cc + 1) * 16) = pack8(v + 8);
    }
    *(i32x4*)(dst + lds_chunk(t, 64 + 2 * q) * 16) = r.rope[0];
    *(i32x4*)(dst + lds_chunk(t, 64 + 2 * q + 1) * 16) = r.rope[1];
}

template <bool SPARSE, bool FP8>
__global__ void __launch_bounds__(kThreads, 1) decode_kernel(const DecodeArgs a) {
    __shared__ Smem sm;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tb = wave & 1;          // QK role: token half of the tile
    const int hq = wave >> 1;         // QK role: head half of the workgroup
    const int l32 = lane & 31;
    const int half = lane >> 5;

    // workgroup -> (partition, head block); the head blocks of one partition
    // get ids 8 apart, which the dispatcher places on the same XCD (same L2)
    const int wg = blockIdx.x;
    const int grp = wg / (8 * a.n_hblk);
    const int rem = wg - grp * 8 * a.n_hblk;
    const int gsz = min(8, a.num_parts - grp * 8);
    const int hb = rem / gsz;
    const int part = grp * 8 + (rem - hb * gsz);

    const int32_t* rec = a.meta + kMetaHeader + kMetaRec * part;
    const int32_t* so = a.meta + kMetaHeader + kMetaRec * a.num_parts;
    const int jb = rec[0], tbeg = rec[1], je = rec[2], tend = rec[3], slot0 = rec[4];
    const int N = a.batch * a.s_q;
    const int H = a.h_q;
    const float c = a.scale_log2;
    const unsigned char* kv = (const unsigned char*)a.kv;

    RowResolver rr{a.block_table, a.cache_seqlens, a.indices, a.s_q, a.max_blocks, SPARSE ? a.topk : 0,
                   a.causal, a.num_rows};

    const int head_qk = hb * kHeadsPerWG + hq * 32 + l32;   // this lane's head in the QK role

    FillPlan fp;
    if (!FP8) make_fill_plan(fp, wave, lane, SPARSE);
    const __amdgpu_buffer_rsrc_t srs = buffer_rsrc(kv, kRowBytes, (int)a.num_rows);
    const int f8_tok = tid >> 2, f8_q = tid & 3;   // FP8 fill role: token and quarter

    for (int j = jb; j <= je && j < N; ++j) {
        const int nslots = rr.slots(j);
        const int ntile_j = (nslots + 63) >> 6;
        const int t0 = (j == jb && tbeg > 0) ? tbeg : 0;
        int t1 = (j == je) ? tend : ntile_j;
        if (t1 > ntile_j) t1 = ntile_j;
        if (t0 >= t1) continue;
        const int nsplit = so[j + 1] - so[j];
        const int slot = (j == jb) ? slot0 : so[j];
        const int ntiles = t1 - t0;

        // ---- Q fragments: B operand of S^T = K Q^T (head = lane, 8 dims) ----
        bf16x8 qf[36];
        {
            const bool ok = head_qk < H;
            const bf16x8* qp = (const bf16x8*)((const unsigned char*)a.q +
                                               ((int64_t)j * H + (ok ? head_qk : 0)) * kRowBytes) + half;
#pragma unroll
            for (int kk = 0; kk < 36; ++kk) {
                bf16x8 v = qp[2 * kk];
                if (!ok) v = bf16x8{};
                qf[kk] = v;
            }
        }

        f32x16 acc[4][2];
#pragma unroll
        for (int d = 0; d < 4; ++d) { acc[d][0] = f32x16{}; acc[d][1] = f32x16{}; }
        float m_run = -INFINITY, l_run = 0.f;

        // dense: page ids of the current and next tile (prefetched one tile ahead)
        int pg_cur = SPARSE ? 0 : rr.page(j, t0);
        int pg_next = (!SPARSE && ntiles > 1) ? rr.page(j, t0 + 1) : 0;

        // ---- prologue: first tile ----
        if (SPARSE) {
            if (wave == 0) {
                sm.rows[0][lane] = (int)rr.row(j, t0 * 64 + lane, nslots);
                if (ntiles > 1) sm.rows[1][lane] = (int)rr.row(j, (t0 + 1) * 64 + lane, nslots);
            }
            __syncthreads();
        }
        Fp8Regs f8;
        if (FP8) {
            const int64_t row = SPARSE ? (int64_t)sm.rows[0][f8_tok]
                                       : row_in_page(pg_cur, f8_tok, nslots - t0 * 64, a.num_rows);
            fp8_load(f8, kv, row, f8_q);
            fp8_store(sm.tile[0], f8, f8_tok, f8_q);
        } else if (SPARSE) {
            fill_sparse(sm.tile[0], srs, sm.rows[0], fp, wave);
        } else {
            fill_dense(sm.tile[0], kv, pg_cur, nslots - t0 * 64, a.num_rows, fp, wave);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();

        for (int it = 0; it < ntiles; ++it) {
            const int cur = it & 1;
            const int tile = t0 + it;
            const bool more = it + 1 < ntiles;
            // next tile in flight while this one is computed
            if (more) {
                if (FP8) {
                    const int64_t row = SPARSE ? (int64_t)sm.rows[(it + 1) & 3][f8_tok]
                                               : row_in_page(pg_next, f8_tok, nslots - (tile + 1) * 64, a.num_rows);
                    fp8_load(f8, kv, row, f8_q);
                } else if (SPARSE) {
                    fill_sparse(sm.tile[cur ^ 1], srs, sm.rows[(it + 1) & 3], fp, wave);
                } else {
                    fill_dense(sm.tile[cur ^ 1], kv, pg_next, nslots - (tile + 1) * 64, a.num_rows, fp, wave);
                }
            }
            int next_row = -1;
            if (SPARSE && wave == 0 && it + 2 < ntiles) next_row = (int)rr.row(j, (tile + 2) * 64 + lane, nslots);
            int pg_after = 0;
            if (!SPARSE && it + 2 < ntiles) pg_after = rr.page(j, tile + 2);

            const unsigned char* T = sm.tile[cur];

            // ---- QK: S^T[32 tokens x 32 heads] over 576 dims ----
            f32x16 s = {};
            {
                const int tq = 32 * tb + l32;
#pragma unroll
                for (int kk = 0; kk < 36; ++kk) {
                    const bf16x8 kf = *(const bf16x8*)(T + lds_chunk(tq, 2 * kk + half) * 16);
                    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], s, 0, 0, 0);
                }
            }

            // ---- mask, scale, tile max (register r -> token 32tb + 8(r/4) + 4half + r%4) ----
            float x[16];
            float mx = -INFINITY;
            {
                const int tv = nslots - tile * 64;   // dense: valid tokens in this tile
                const bool pg = SPARSE ? true : page_ok(pg_cur, a.num_rows);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int tok = 32 * tb + 8 * (r >> 2) + 4 * half + (r & 3);
                    const bool valid = SPARSE ? (sm.rows[it & 3][tok] >= 0) : (pg && tok < tv);
                    x[r] = valid ? s[r] * c : -INFINITY;
                    mx = fmaxf(mx, x[r]);
                }
            }
            mx = wave_max_pair(mx);
            if (lane < 32) sm.red_max[hq][tb][lane] = mx;
            __syncthreads();

            // ---- exact online softmax ----
            const float m_tile = fmaxf(mx, sm.red_max[hq][tb ^ 1][l32]);
            const float m_new = fmaxf(m_run, m_tile);
            float alpha;
            float psum = 0.f;
            if (m_new == -INFINITY) {
                alpha = 1.f;
#pragma unroll
                for (int r = 0; r < 16; ++r) x[r] = 0.f;
            } else {
                alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    x[r] = __builtin_amdgcn_exp2f(x[r] - m_new);
                    psum += x[r];
                }
            }
            psum = wave_sum_pair(psum);
            l_run = l_run * alpha + psum;
            m_run = m_new;
            *(bf16x8*)(sm.p + (((2 * tb + 0) * 2 + hq) * 64 + lane) * 16) = pack8(x);
            *(bf16x8*)(sm.p + (((2 * tb + 1) * 2 + hq) * 64 + lane) * 16) = pack8(x + 8);
            if (tb == 0 && lane < 32) sm.alpha[hq][lane] = alpha;
            __syncthreads();

            // ---- PV: O^T[dims 128w + 32d .. , heads] += V^T P^T ----
            {
                const float a0 = sm.alpha[0][l32], a1 = sm.alpha[1][l32];
#pragma unroll
                for (int d = 0; d < 4; ++d) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) { acc[d][0][r] *= a0; acc[d][1][r] *= a1; }
                }
                const int g = lane >> 4, i16 = lane & 15;
#pragma unroll
                for (int j4 = 0; j4 < 4; ++j4) {
                    const bf16x8 p0 = *(const bf16x8*)(sm.p + ((j4 * 2 + 0) * 64 + lane) * 16);
                    const bf16x8 p1 = *(const bf16x8*)(sm.p + ((j4 * 2 + 1) * 64 + lane) * 16);
                    const int tokA = 16 * j4 + 4 * (g >> 1) + (i16 >> 2);
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
                        const int dim0 = 128 * wave + 32 * d + 16 * (g & 1) + 4 * (i16 & 3);
                        const int boff = (dim0 & 7) * 2;
                        const bf16x4 v0 = tr_read(T + lds_chunk(tokA, dim0 >> 3) * 16 + boff);
                        const bf16x4 v1 = tr_read(T + lds_chunk(tokA + 8, dim0 >> 3) * 16 + boff);
                        const bf16x8 vf = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
                        acc[d][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, p0, acc[d][0], 0, 0, 0);
                        acc[d][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, p1, acc[d][1], 0, 0, 0);
                    }
                }
            }

            if (FP8 && more) fp8_store(sm.tile[cur ^ 1], f8, f8_tok, f8_q);
            if (SPARSE && wave == 0 && it + 2 < ntiles) sm.rows[(it + 2) & 3][lane] = next_row;
            pg_cur = pg_next;
            pg_next = pg_after;
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }

        // ---- epilogue ----
        if (lane < 32) sm.lsum[hq][tb][lane] = l_run;
        __syncthreads();
        const bool final_out = (nsplit == 1);
        const int b = j / a.s_q, iq = j - b * a.s_q;
        if (final_out || (slot >= 0 && slot < a.max_slots)) {
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const int head = hb * kHeadsPerWG + h2 * 32 + l32;
                const float lt = sm.lsum[h2][0][l32] + sm.lsum[h2][1][l32];
                const float inv = lt > 0.f ? 1.f / lt : 0.f;
                if (head < H) {
#pragma unroll
                    for (int d = 0; d < 4; ++d) {
#pragma unroll
                        for (int rq = 0; rq < 4; ++rq) {
                            const int dim = 128 * wave + 32 * d + 8 * rq + 4 * half;
                            const float v0 = acc[d][h2][4 * rq + 0] * inv, v1 = acc[d][h2][4 * rq + 1] * inv;
                            const float v2 = acc[d][h2][4 * rq + 2] * inv, v3 = acc[d][h2][4 * rq + 3] * inv;
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
                }
            }
            if (tb == 0 && lane < 32 && head_qk < H) {
                const float lt = sm.lsum[hq][0][lane] + sm.lsum[hq][1][lane];
                const float lse_v = lt > 0.f ? (m_run + log2f(lt)) * 0.69314718055994531f : -INFINITY;
                if (final_out) a.lse[((int64_t)b * H + head_qk) * a.s_q + iq] = lse_v;
                else a.lse_part[(int64_t)slot * H + head_qk] = lse_v;
            }
        }
        __syncthreads();
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
