// LSE merge of split partials, plus the debug gather of cache row ids.
//
// Combine: one workgroup per (item, 4 heads); 64 lanes x 8 dims cover the 512
// output dims of a head.  With m* = max_k lse_k and w_k = exp(lse_k - m*):
// out = sum_k w_k o_k / sum_k w_k and lse = m* + ln sum_k w_k, which is the
// pairwise split merge applied to all partials at once (computed a chunk of
// splits at a time with a running maximum).

#include "common.h"
#include "kernels.h"

namespace mla {

__global__ void __launch_bounds__(256) combine_kernel(const CombineArgs a) {
    const int item = blockIdx.x;
    const int h = blockIdx.y * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (h >= a.h_q) return;
    // split offsets, lse and the float16 scales are uniform per wave: scalar
    // loads, so the vector loads of the partials are the only memory round trip
    const int s0 = sload(a.split_offsets + item), s1 = sload(a.split_offsets + item + 1);
    const int n = s1 - s0;
    if (a.skip_single && n == 1) return;
    const int H = a.h_q;
    const int qd = lane >> 4;   // dims 8 lane .. 8 lane + 7 lie in quarter qd of the head's 512 dims
    // Splits are merged kSplitChunk at a time, every load of a chunk issued
    // before any is used; across chunks the merge is online (running max m).
    // Two per chunk: most split items have two or three splits, and the
    // registers of a larger chunk cost occupancy.
    constexpr int kSplitChunk = 2;
    float m = -INFINITY, wsum = 0.f;
    float o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    bool nan_lse = false;   // a split whose softmax sum was NaN (a NaN in q or the cache) makes the row NaN
    for (int k0 = s0; k0 < s1; k0 += kSplitChunk) {
        float lk[kSplitChunk];
        float x[kSplitChunk][8];
#pragma unroll
        for (int c = 0; c < kSplitChunk; ++c) {
            const int k = k0 + c;
            lk[c] = -INFINITY;
#pragma unroll
            for (int e = 0; e < 8; ++e) x[c][e] = 0.f;
            if (k < s1) {
                const int64_t row = (int64_t)k * H + h;
                lk[c] = sload(a.lse_part + row);
                if (a.part_fp16) {
                    // float16 partial scaled by 2^-E; dims lane*8 + 0..3 use byte
                    // 2 qd, dims + 4..7 byte 2 qd + 1 of the head's exponents
                    typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
                    const f16x8 v = *(const f16x8*)((const _Float16*)a.o_part + row * kDv + lane * 8);
                    const uint32_t* ew = (const uint32_t*)(a.o_exp8 + row * 8);
                    const uint32_t w0 = sload(ew), w1 = sload(ew + 1);
                    const uint32_t wq = (qd & 2) ? w1 : w0;
                    const int e0 = (int)(signed char)(wq >> (16 * (qd & 1)));
                    const int e1 = (int)(signed char)(wq >> (16 * (qd & 1) + 8));
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        x[c][e] = ldexpf((float)v[e], e0);
                        x[c][e + 4] = ldexpf((float)v[e + 4], e1);
                    }
                } else {
                    const f32x4* src = (const f32x4*)(a.o_part + row * kDv + lane * 8);
                    const f32x4 u = src[0], w = src[1];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        x[c][e] = u[e];
                        x[c][e + 4] = w[e];
                    }
                }
            }
        }
        float mc = m;
#pragma unroll
        for (int c = 0; c < kSplitChunk; ++c) {
            mc = fmaxf(mc, lk[c]);
            nan_lse |= lk[c] != lk[c];
        }
        if (mc == -INFINITY) continue;                       // nothing finite yet
        const float sc = m == -INFINITY ? 0.f : __expf(m - mc);
        wsum *= sc;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] *= sc;
#pragma unroll
        for (int c = 0; c < kSplitChunk; ++c) {
            const float w = lk[c] == -INFINITY ? 0.f : __expf(lk[c] - mc);
            wsum += w;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] += w * x[c][e];
        }
        m = mc;
    }
    float lse_v = -INFINITY;
    if (n > 0 && m != -INFINITY) {
        const float inv = 1.f / wsum;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] *= inv;
        lse_v = m + __logf(wsum);
        // attention sink: out is scaled by exp(lse) / (exp(lse) + exp(sink))
        if (a.attn_sink) {
            const float f = 1.f / (1.f + __expf(a.attn_sink[h] - lse_v));
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] *= f;
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = 0.f;
    }
    if (nan_lse) {
        lse_v = __builtin_nanf("");
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = lse_v;
    }
    const int64_t off = ((int64_t)item * H + h) * kDv + lane * 8;
    if (a.out_fp32) {
        f32x4* dst = (f32x4*)((float*)a.out + off);
        dst[0] = f32x4{o[0], o[1], o[2], o[3]};
        dst[1] = f32x4{o[4], o[5], o[6], o[7]};
    } else {
        bf16x8 w;
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = (__bf16)o[e];
        *(bf16x8*)((__bf16*)a.out + off) = w;
    }
    if (lane == 0) {
        const int b = item / a.s_q, i = item - b * a.s_q;
        a.lse[((int64_t)b * H + h) * a.s_q + i] = lse_v;
    }
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
    const dim3 grid(a.num_items, (a.h_q + 3) / 4), block(256);
    hipLaunchKernelGGL(combine_kernel, grid, block, 0, stream, a);
    return hipGetLastError();
}

// Test hook: the rows the decode kernels read, through the same resolver.
__global__ void __launch_bounds__(256) gather_kernel(const GatherArgs a) {
    const int j = blockIdx.x;
    const bool sparse = a.topk > 0;
    RowResolver rr{sparse ? nullptr : a.table_or_indices, a.cache_seqlens, sparse ? a.table_or_indices : nullptr,
                   a.s_q, a.max_blocks, a.topk, a.causal, a.num_rows};
    const int nslots = rr.slots(j);
    const int ntiles = (nslots + 63) >> 6;
    for (int t = threadIdx.x; t < ntiles * 64 && t < a.row_stride; t += blockDim.x)
        a.rows_out[(int64_t)j * a.row_stride + t] = (int32_t)rr.row(j, t, nslots);
}

hipError_t launch_gather(const GatherArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(gather_kernel, dim3(a.batch * a.s_q), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace mla
