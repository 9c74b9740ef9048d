// Wave-level form of the split-KV scheduler, for decode kernels that compute
// their own schedule: every wave of a workgroup derives its partition's
// record from the lengths with the scheduler kernel's arithmetic (the same
// results word for word), without a separate launch.
#pragma once

#include "common.h"
#include "kernels.h"

namespace mla {

// Inclusive prefix sum of one int per lane over the wave, in DPP moves (no
// LDS): within rows of 16 lanes by shifts of 1, 2, 4 and 8, then the last
// lane of row 0 into row 1 and of row 2 into row 3, then lane 31 into rows 2
// and 3.  Lanes a move has no source for keep the identity 0.
__device__ __forceinline__ int wave_scan_incl(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);   // row_bcast:15 into rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);   // row_bcast:31 into rows 2, 3
    return v;
}

// x / d for 0 <= x < 2^31 and 0 < d, given rd = 1 / d in double precision:
// the estimate is within one of the quotient and is corrected once.
__device__ __forceinline__ int div_rd(int x, int d, double rd) {
    int y = (int)((double)x * rd);
    y -= y * d > x ? 1 : 0;
    y += (y + 1) * d <= x ? 1 : 0;
    return y;
}

// The scheduler's arithmetic for partition ``part``, computed by one wave:
// lane ln holds items ln * R + u (u < R) -- their tile counts Tl, the
// exclusive prefix sum C of item cost (tiles + F), split counts NS and split
// offsets SO -- and every lane gets the partition's record and the header
// values T (total cost), q (cost per partition) and total (split slots).
// Item j's tiles: the 64-token pages of its causal-visible length (dense,
// lengths = cache_seqlens [batch]) or of its top-k slots (sparse, topk > 0,
// lengths = topk_length [batch * s_q] or null for all topk).
struct WaveSched {
    int C[4], Tl[4], NS[4], SO[4];
    int jb, tbeg, je, tend, slot0, T, q, total;
};

template <int R>
__device__ __forceinline__ void wave_schedule(const DecodeArgs& a, const int32_t* lengths, int N, int part, int ln,
                                              WaveSched& w) {
    const int F = a.fixed_overhead, P = a.num_parts;
    const double rs = 1.0 / (double)a.s_q;
    int own = 0;
#pragma unroll
    for (int u = 0; u < R; ++u) {
        const int j = ln * R + u;
        w.Tl[u] = 0;
        if (j < N) {
            if (a.topk > 0) {
                w.Tl[u] = ((lengths ? topk_slots(lengths[j], a.topk) : a.topk) + 63) >> 6;
            } else {
                const int b = div_rd(j, a.s_q, rs), i = j - b * a.s_q;
                w.Tl[u] = (visible_len(clamp_len(lengths[b], a.max_blocks), a.s_q, i, a.causal) + 63) >> 6;
            }
            own += w.Tl[u] + F;
        }
    }
    int incl = wave_scan_incl(own);
    w.T = __builtin_amdgcn_readlane(incl, 63);
    int run = incl - own;
#pragma unroll
    for (int u = 0; u < R; ++u) {
        w.C[u] = run;
        if (ln * R + u < N) run += w.Tl[u] + F;
    }
    w.q = w.T > 0 ? div_rd(w.T + P - 1, P, 1.0 / (double)P) : 1;
    const double rq = 1.0 / (double)w.q;
    own = 0;
#pragma unroll
    for (int u = 0; u < R; ++u) {
        const int n = w.Tl[u], first = w.C[u] + F;
        w.NS[u] = (ln * R + u < N && n > 0) ? div_rd(first + n - 1, w.q, rq) - div_rd(first, w.q, rq) + 1 : 0;
        own += w.NS[u];
    }
    incl = wave_scan_incl(own);
    w.total = __builtin_amdgcn_readlane(incl, 63);
    run = incl - own;
#pragma unroll
    for (int u = 0; u < R; ++u) {
        w.SO[u] = run;
        run += w.NS[u];
    }
    // last item j with C[j] <= x: the C[j] are non-decreasing, so count them
    auto item_of = [&](int x) __attribute__((always_inline)) -> int {
        int cnt = 0;
#pragma unroll
        for (int u = 0; u < R; ++u) cnt += __builtin_popcountll(__builtin_amdgcn_ballot_w64(ln * R + u < N && w.C[u] <= x));
        return cnt - 1;
    };
    auto at = [&](const int (&v)[4], int j) __attribute__((always_inline)) -> int {
        const int u = j % R;
        const int x = R == 1 ? v[0] : (u == 0 ? v[0] : u == 1 ? v[1] : u == 2 ? v[2] : v[3]);
        return __builtin_amdgcn_readlane(x, j / R);
    };
    const int64_t lo64 = (int64_t)part * w.q;
    const int64_t hi64 = lo64 + w.q < w.T ? lo64 + w.q : w.T;
    if (lo64 >= hi64) {
        w.jb = N; w.tbeg = 0; w.je = N; w.tend = 0; w.slot0 = 0;
        return;
    }
    const int lo = (int)lo64, hi = (int)hi64;
    w.jb = item_of(lo);
    w.je = item_of(hi - 1);
    const int Cjb = at(w.C, w.jb), njb = at(w.Tl, w.jb);
    const int Cje = at(w.C, w.je), nje = at(w.Tl, w.je);
    w.tbeg = lo - Cjb - F;
    if (w.tbeg < 0) w.tbeg = 0;
    w.tend = hi - Cje - F;
    w.tend = w.tend < 0 ? 0 : (w.tend > nje ? nje : w.tend);
    const int first_end = w.je == w.jb ? w.tend : njb;
    w.slot0 = w.tbeg < first_end ? at(w.SO, w.jb) + part - div_rd(Cjb + F, w.q, rq) : 0;
}


// Dispatch on items per lane (batch * s_q <= 64, 128 or 256).
__device__ __forceinline__ void wave_schedule_any(const DecodeArgs& a, const int32_t* lengths, int N, int part,
                                                  int ln, int R, WaveSched& w) {
    if (R == 1) wave_schedule<1>(a, lengths, N, part, ln, w);
    else if (R == 2) wave_schedule<2>(a, lengths, N, part, ln, w);
    else wave_schedule<4>(a, lengths, N, part, ln, w);
}

// The schedule written back in the scheduler's layout (header, records, split
// offsets).  ``rec_writer``: this wave writes partition ``part``'s record;
// ``all_writer``: this wave writes the header and every split offset.
__device__ __forceinline__ void wave_schedule_store(const DecodeArgs& a, int N, int part, int ln, int R,
                                                    const WaveSched& w, bool rec_writer, bool all_writer) {
    int32_t* mo = a.meta_out;
    if (rec_writer && ln == 0) {
        int32_t* r = mo + kMetaHeader + kMetaRec * part;
        r[0] = w.jb; r[1] = w.tbeg; r[2] = w.je; r[3] = w.tend; r[4] = w.slot0;
    }
    if (all_writer) {
        int32_t* so_o = mo + kMetaHeader + kMetaRec * a.num_parts;
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (u < R && ln * R + u < N) so_o[ln * R + u] = w.SO[u];
        if (ln == 0) {
            const int F = a.fixed_overhead;
            so_o[N] = w.total;
            mo[0] = kMetaMagic; mo[1] = a.num_parts; mo[2] = N; mo[3] = F;
            mo[4] = w.q; mo[5] = w.T; mo[6] = a.s_q; mo[7] = w.T - N * F;
        }
    }
}

}  // namespace mla
