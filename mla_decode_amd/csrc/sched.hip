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
//
// The kernel runs once per step ahead of the decode kernel, so its latency is
// on the step's critical path: four waves, each thread owning a contiguous
// run of items, and two block scans (wave shuffles plus one LDS exchange).

#include "common.h"
#include "kernels.h"

namespace mla {

constexpr int kSchedThreads = 256;

// inclusive scan of one value per thread over the workgroup (4 waves)
__device__ __forceinline__ int block_scan_incl(int v, int* tmp) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(v, o, 64);
        if (lane >= o) v += u;
    }
    if (lane == 63) tmp[w] = v;
    __syncthreads();
    int add = 0;
    for (int i = 0; i < w; ++i) add += tmp[i];
    __syncthreads();
    return v + add;
}

__global__ void __launch_bounds__(kSchedThreads) metadata_kernel(const MetaArgs a) {
    __shared__ int C[kMaxMetaItems + 1];    // exclusive prefix sum of item cost
    __shared__ int SO[kMaxMetaItems + 1];   // split offsets
    const int N = a.batch * a.s_q;
    const int F = a.fixed_overhead;
    const int P = a.num_parts;
    const int tid = threadIdx.x;
    __shared__ int tmp[kSchedThreads / 64];

    auto tiles_of = [&](int j) -> int {
        if (a.topk > 0) return ((a.cache_seqlens ? topk_slots(a.cache_seqlens[j], a.topk) : a.topk) + 63) >> 6;
        const int b = j / a.s_q, i = j - b * a.s_q;
        return (visible_len(clamp_len(a.cache_seqlens[b], a.max_blocks), a.s_q, i, a.causal) + 63) >> 6;
    };
    // thread tid owns items [tid * per, tid * per + per)
    const int per = (N + kSchedThreads - 1) / kSchedThreads;
    const int j0 = tid * per;

    // S1-S2: C_j and T
    int own = 0;
    for (int u = 0; u < per; ++u) {
        const int j = j0 + u;
        if (j < N) {
            const int cost = tiles_of(j) + F;
            C[j + 1] = cost;
            own += cost;
        }
    }
    int run = block_scan_incl(own, tmp) - own;
    if (tid == 0) C[0] = 0;
    for (int u = 0; u < per; ++u) {
        const int j = j0 + u;
        if (j < N) {
            run += C[j + 1];
            C[j + 1] = run;
        }
    }
    __syncthreads();
    const int T = C[N];
    const int q = T > 0 ? (T + P - 1) / P : 1;

    // S5: num_splits and split_offsets
    own = 0;
    for (int u = 0; u < per; ++u) {
        const int j = j0 + u;
        if (j < N) {
            const int n = C[j + 1] - C[j] - F;
            const int first = C[j] + F;
            const int ns = n > 0 ? (first + n - 1) / q - first / q + 1 : 0;
            SO[j + 1] = ns;
            own += ns;
        }
    }
    run = block_scan_incl(own, tmp) - own;
    if (tid == 0) SO[0] = 0;
    for (int u = 0; u < per; ++u) {
        const int j = j0 + u;
        if (j < N) {
            run += SO[j + 1];
            SO[j + 1] = run;
        }
    }
    __syncthreads();

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
