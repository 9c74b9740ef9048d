// Split-KV tile scheduler, one workgroup, integer arithmetic only.
//
// Items are query tokens (j = b*s_q + i) with n_j KV tiles of 64 tokens
// (dense: causal-visible length; sparse: topk, or the item's top-k length
// clamped to [0, topk]).  Each item costs n_j + F;
// the prefix sum C_j of the costs is cut into P equal runs of q = ceil(T/P)
// cost units and every partition records the (item, tile) range it covers.
// The first F cost units of an item carry no tile: they stand for the item's
// fixed set-up and epilogue work.  num_splits[j] counts the partitions holding
// tiles of item j; split_offsets is its exclusive prefix sum.

#include "common.h"
#include "kernels.h"

namespace mla {

constexpr int kSchedThreads = 1024;

// inclusive block scan of one value per thread (1024 threads, wave64)
__device__ __forceinline__ int block_scan_incl(int v, int* tmp) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(v, o, 64);
        if (lane >= o) v += u;
    }
    if (lane == 63) tmp[w] = v;
    __syncthreads();
    if (w == 0) {
        int t = lane < (kSchedThreads / 64) ? tmp[lane] : 0;
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
            const int u = __shfl_up(t, o, 64);
            if (lane >= o) t += u;
        }
        if (lane < (kSchedThreads / 64)) tmp[lane] = t;
    }
    __syncthreads();
    const int add = w > 0 ? tmp[w - 1] : 0;
    __syncthreads();
    return v + add;
}

__global__ void __launch_bounds__(kSchedThreads) metadata_kernel(const MetaArgs a) {
    __shared__ int C[kMaxMetaItems + 1];    // exclusive prefix sum of item cost
    __shared__ int SO[kMaxMetaItems + 1];   // split offsets
    __shared__ int tmp[kSchedThreads / 64];
    __shared__ int carry_s;
    const int N = a.batch * a.s_q;
    const int F = a.fixed_overhead;
    const int P = a.num_parts;
    const int tid = threadIdx.x;

    auto tiles_of = [&](int j) -> int {
        if (a.topk > 0) return ((a.cache_seqlens ? topk_slots(a.cache_seqlens[j], a.topk) : a.topk) + 63) >> 6;
        const int b = j / a.s_q, i = j - b * a.s_q;
        return (visible_len(clamp_len(a.cache_seqlens[b], a.max_blocks), a.s_q, i, a.causal) + 63) >> 6;
    };

    // S1-S2: C_j and T
    if (tid == 0) { C[0] = 0; carry_s = 0; }
    __syncthreads();
    for (int base = 0; base < N; base += kSchedThreads) {
        const int j = base + tid;
        const int cost = j < N ? tiles_of(j) + F : 0;
        const int incl = block_scan_incl(cost, tmp);
        const int carry = carry_s;
        if (j < N) C[j + 1] = carry + incl;
        __syncthreads();
        if (tid == kSchedThreads - 1) carry_s = carry + incl;
        __syncthreads();
    }
    const int T = C[N];
    const int q = T > 0 ? (T + P - 1) / P : 1;

    // S5: num_splits and split_offsets
    if (tid == 0) { SO[0] = 0; carry_s = 0; }
    __syncthreads();
    for (int base = 0; base < N; base += kSchedThreads) {
        const int j = base + tid;
        int ns = 0;
        if (j < N) {
            const int n = C[j + 1] - C[j] - F;
            const int first = C[j] + F;
            ns = n > 0 ? (first + n - 1) / q - first / q + 1 : 0;
        }
        const int incl = block_scan_incl(ns, tmp);
        const int carry = carry_s;
        if (j < N) SO[j + 1] = carry + incl;
        __syncthreads();
        if (tid == kSchedThreads - 1) carry_s = carry + incl;
        __syncthreads();
    }

    int32_t* out = a.meta;
    int32_t* recs = out + kMetaHeader;
    int32_t* so = recs + kMetaRec * P;
    for (int j = tid; j <= N; j += kSchedThreads) so[j] = SO[j];

    // S3-S4: partition records
    auto item_of = [&](int x) -> int {   // last j in [0, N) with C[j] <= x
        int lo = 0, hi = N;              // invariant: C[lo] <= x, answer in [lo, hi)
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (C[mid] <= x) lo = mid; else hi = mid;
        }
        return lo;
    };
    for (int p = tid; p < P; p += kSchedThreads) {
        const int64_t lo64 = (int64_t)p * q;
        const int64_t hi64 = lo64 + q < T ? lo64 + q : T;
        int32_t* r = recs + kMetaRec * p;
        if (lo64 >= hi64) {
            r[0] = N; r[1] = 0; r[2] = N; r[3] = 0; r[4] = 0;
            continue;
        }
        const int lo = (int)lo64, hi = (int)hi64;
        const int jb = item_of(lo);
        int tb = lo - C[jb] - F;
        if (tb < 0) tb = 0;
        const int je = item_of(hi - 1);
        const int n_je = C[je + 1] - C[je] - F;
        int te = hi - C[je] - F;
        te = te < 0 ? 0 : (te > n_je ? n_je : te);
        const int n_jb = C[jb + 1] - C[jb] - F;
        const int first_end = (je == jb) ? te : n_jb;
        const int slot0 = tb < first_end ? SO[jb] + p - (C[jb] + F) / q : 0;
        r[0] = jb; r[1] = tb; r[2] = je; r[3] = te; r[4] = slot0;
    }
    if (tid == 0) {
        out[0] = kMetaMagic; out[1] = P; out[2] = N; out[3] = F;
        out[4] = q; out[5] = T; out[6] = a.s_q; out[7] = T - N * F;
    }
}

hipError_t launch_metadata(const MetaArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL(metadata_kernel, dim3(1), dim3(kSchedThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace mla
