// Host-side validation of the arrays a decode call reads: the scheduler's
// metadata words, cache lengths, page ids, top-k indices and top-k lengths.
// mla_check_inputs runs it on host arrays; with MLA_DEBUG=1 in the
// environment every entry point copies its device arrays to the host and runs
// it before launching (a debug mode: it synchronises the stream).

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/mla_decode.h"
#include "check.h"
#include "common.h"

namespace mla {
namespace {

struct Msg {
    char* buf;
    size_t len;
    mla_status_t fail(const char* fmt, ...) {
        if (buf && len) {
            va_list ap;
            va_start(ap, fmt);
            vsnprintf(buf, len, fmt, ap);
            va_end(ap);
        }
        return MLA_ERR_INVALID_ARG;
    }
};

// KV tiles of item j, from the host copies of the length arrays (the rule the
// scheduler and the kernels apply: dense lengths clamped to the block table,
// causal visibility within the item's query group; sparse: topk, or the item's
// top-k length clamped to [0, topk]).
int64_t item_tiles(const mla_problem_t* p, const int32_t* seqlens, const int32_t* topk_length, int64_t j) {
    if (p->topk > 0) return ((topk_length ? topk_slots(topk_length[j], p->topk) : p->topk) + 63) / 64;
    const int64_t b = j / p->s_q, i = j - b * p->s_q;
    return (visible_len(clamp_len(seqlens[b], p->max_blocks_per_seq), p->s_q, (int)i, p->causal) + 63) / 64;
}

// The schedule in `w` covers every tile of every item exactly once, in item
// order, with partition boundaries, split counts and first split slots that
// agree with each other and with the current lengths.
mla_status_t check_words(const mla_problem_t* p, const mla_metadata_t* m, const int32_t* w,
                         const std::vector<int64_t>& tiles, Msg& e) {
    const int64_t N = (int64_t)p->batch * p->s_q;
    const int64_t P = m->num_partitions, F = m->fixed_overhead;
    int64_t T = 0;
    for (int64_t j = 0; j < N; ++j) T += tiles[j] + F;
    const int64_t q = T > 0 ? (T + P - 1) / P : 1;
    if (w[0] != kMetaMagic) return e.fail("metadata word 0 is 0x%08x, not the schedule's magic", (unsigned)w[0]);
    if (w[1] != P || w[2] != N || w[3] != F || w[6] != p->s_q)
        return e.fail("metadata header (P=%d N=%d F=%d s_q=%d) is not this plan's (P=%lld N=%lld F=%lld s_q=%d)",
                      w[1], w[2], w[3], w[6], (long long)P, (long long)N, (long long)F, p->s_q);
    if (w[5] != T || w[4] != q || w[7] != T - N * F)
        return e.fail("metadata totals (T=%d q=%d) do not match the current lengths (T=%lld q=%lld): stale metadata?",
                      w[5], w[4], (long long)T, (long long)q);
    const int32_t* recs = w + kMetaHeader;
    const int32_t* so = recs + kMetaRec * P;
    if (so[0] != 0) return e.fail("split_offsets[0] = %d, not 0", so[0]);
    for (int64_t j = 0; j < N; ++j)
        if (so[j + 1] < so[j]) return e.fail("split_offsets decrease at item %lld", (long long)j);
    if (so[N] > m->max_splits) return e.fail("split_offsets[N] = %d exceeds max_splits %d", so[N], m->max_splits);

    std::vector<int64_t> G(N + 1, 0);   // tiles before item j
    for (int64_t j = 0; j < N; ++j) G[j + 1] = G[j] + tiles[j];
    std::vector<int32_t> seen(N, 0);
    int64_t g = 0;                      // next tile to be covered
    for (int64_t k = 0; k < P; ++k) {
        const int32_t* r = recs + kMetaRec * k;
        const int64_t jb = r[0], tb = r[1], je = r[2], te = r[3], slot0 = r[4];
        if (jb == N) {
            if (tb != 0 || je != N || te != 0 || slot0 != 0)
                return e.fail("partition %lld: malformed empty record", (long long)k);
            continue;
        }
        if (jb < 0 || jb > je || je >= N || tb < 0 || tb > tiles[jb] || te < 0 || te > tiles[je])
            return e.fail("partition %lld: record (%lld,%lld)-(%lld,%lld) outside the items' tiles", (long long)k,
                          (long long)jb, (long long)tb, (long long)je, (long long)te);
        const int64_t gs = G[jb] + tb, ge = G[je] + te;
        if (gs > ge) return e.fail("partition %lld: range ends before it starts", (long long)k);
        if (gs < ge) {
            if (gs != g)
                return e.fail("partition %lld starts at tile %lld, the previous one ended at %lld", (long long)k,
                              (long long)gs, (long long)g);
            g = ge;
        }
        for (int64_t j = jb; j <= je; ++j) {
            const int64_t lo = j == jb ? tb : 0, hi = j == je ? te : tiles[j];
            if (lo >= hi) continue;
            if (j == jb ? slot0 != so[j] + seen[j] : seen[j] != 0)
                return e.fail("partition %lld: split slot of item %lld is inconsistent", (long long)k, (long long)j);
            if (seen[j] >= so[j + 1] - so[j])
                return e.fail("item %lld has more partitions than its %d splits", (long long)j, so[j + 1] - so[j]);
            ++seen[j];
        }
    }
    if (g != G[N]) return e.fail("the partitions cover %lld of %lld tiles", (long long)g, (long long)G[N]);
    for (int64_t j = 0; j < N; ++j)
        if (seen[j] != so[j + 1] - so[j])
            return e.fail("item %lld: %d splits recorded, %d partitions hold its tiles", (long long)j,
                          so[j + 1] - so[j], seen[j]);
    return MLA_OK;
}

mla_status_t check_host(const mla_problem_t* p, const mla_metadata_t* m, const int32_t* words,
                        const int32_t* seqlens, const int32_t* toi, const int32_t* topk_length, int64_t num_rows,
                        Msg& e) {
    if (words && (!m || m->num_partitions < 1 || m->sig.batch != p->batch || m->sig.s_q != p->s_q))
        return e.fail("the metadata words need the plan they were made from");
    const int64_t N = (int64_t)p->batch * p->s_q;
    if (num_rows <= 0) num_rows = (int64_t)p->num_blocks * kBlock;
    if (p->topk == 0) {
        if (!seqlens) return e.fail("cache_seqlens is required for a dense problem");
        const int64_t cap = (int64_t)p->max_blocks_per_seq * kBlock;
        for (int64_t b = 0; b < p->batch; ++b)
            if (seqlens[b] < 0 || seqlens[b] > cap)
                return e.fail("cache_seqlens[%lld] = %d is outside [0, %lld]", (long long)b, seqlens[b],
                              (long long)cap);
        if (toi)
            for (int64_t b = 0; b < p->batch; ++b)
                for (int64_t k = 0; k < (seqlens[b] + kBlock - 1) / kBlock; ++k) {
                    const int32_t page = toi[b * p->max_blocks_per_seq + k];
                    if (page < 0 || page >= p->num_blocks)
                        return e.fail("block_table[%lld, %lld] = %d is outside [0, %d)", (long long)b,
                                      (long long)k, page, p->num_blocks);
                }
    } else {
        if (topk_length)
            for (int64_t j = 0; j < N; ++j)
                if (topk_length[j] < 0 || topk_length[j] > p->topk)
                    return e.fail("topk_length[%lld] = %d is outside [0, %d]", (long long)j, topk_length[j],
                                  p->topk);
        if (toi)
            for (int64_t j = 0; j < N; ++j) {
                const int64_t n = topk_length ? topk_slots(topk_length[j], p->topk) : p->topk;
                for (int64_t t = 0; t < n; ++t) {
                    const int32_t r = toi[j * p->topk + t];
                    if (r < -1 || r >= num_rows)
                        return e.fail("indices[%lld, %lld] = %d is neither -1 nor a row in [0, %lld)",
                                      (long long)j, (long long)t, r, (long long)num_rows);
                }
            }
    }
    if (words) {
        std::vector<int64_t> tiles(N);
        for (int64_t j = 0; j < N; ++j) tiles[j] = item_tiles(p, seqlens, topk_length, j);
        return check_words(p, m, words, tiles, e);
    }
    return MLA_OK;
}

template <class T>
bool fetch(std::vector<T>& host, const T* dev, size_t n) {
    host.resize(n);
    return n == 0 || hipMemcpy(host.data(), dev, n * sizeof(T), hipMemcpyDeviceToHost) == hipSuccess;
}

}  // namespace

mla_status_t check_host_arrays(const mla_problem_t* p, const mla_metadata_t* m, const int32_t* words,
                               const int32_t* seqlens, const int32_t* toi, const int32_t* topk_length,
                               int64_t num_rows, char* msg, size_t msg_len) {
    if (msg && msg_len) msg[0] = 0;
    Msg e{msg, msg_len};
    return check_host(p, m, words, seqlens, toi, topk_length, num_rows, e);
}

bool debug_enabled() {
    const char* v = std::getenv("MLA_DEBUG");
    return v && std::strcmp(v, "1") == 0;
}

mla_status_t debug_check_call(const mla_problem_t* p, const mla_metadata_t* m, bool check_words_too,
                              const int32_t* seqlens, const int32_t* toi, const int32_t* topk_length,
                              int64_t num_rows, hipStream_t stream, const char* entry) {
    char buf[256] = {0};
    Msg e{buf, sizeof buf};
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return MLA_ERR_HIP;
    mla_status_t st = MLA_OK;
    if (cs != hipStreamCaptureStatusNone) {
        st = e.fail("the stream is capturing a graph; MLA_DEBUG=1 needs eager calls");
    } else {
        if (hipStreamSynchronize(stream) != hipSuccess) return MLA_ERR_HIP;
        const int64_t N = (int64_t)p->batch * p->s_q;
        std::vector<int32_t> w, sl, ti, tl;
        bool ok = true;
        if (check_words_too && m && m->dev) ok = ok && fetch(w, (const int32_t*)m->dev, m->bytes / sizeof(int32_t));
        if (p->topk == 0 && seqlens) ok = ok && fetch(sl, seqlens, (size_t)p->batch);
        if (toi)
            ok = ok && fetch(ti, toi, (size_t)(p->topk > 0 ? N * p->topk : (int64_t)p->batch * p->max_blocks_per_seq));
        if (p->topk > 0 && topk_length) ok = ok && fetch(tl, topk_length, (size_t)N);
        if (!ok) return MLA_ERR_HIP;
        st = check_host(p, m, w.empty() ? nullptr : w.data(), sl.empty() ? nullptr : sl.data(),
                        ti.empty() ? nullptr : ti.data(), tl.empty() ? nullptr : tl.data(), num_rows, e);
    }
    if (st != MLA_OK) std::fprintf(stderr, "MLA_DEBUG: %s: %s\n", entry, buf);
    return st;
}

mla_status_t debug_check_offsets(const int32_t* split_offsets, int32_t num_items, hipStream_t stream) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return MLA_ERR_HIP;
    if (cs != hipStreamCaptureStatusNone) {
        std::fprintf(stderr, "MLA_DEBUG: mla_combine: the stream is capturing a graph\n");
        return MLA_ERR_INVALID_ARG;
    }
    if (hipStreamSynchronize(stream) != hipSuccess) return MLA_ERR_HIP;
    std::vector<int32_t> so;
    if (!fetch(so, split_offsets, (size_t)num_items + 1)) return MLA_ERR_HIP;
    for (int32_t j = 0; j < num_items; ++j)
        if (so[0] != 0 || so[j + 1] < so[j]) {
            std::fprintf(stderr, "MLA_DEBUG: mla_combine: split_offsets are not a prefix sum from 0 (item %d)\n", j);
            return MLA_ERR_INVALID_ARG;
        }
    return MLA_OK;
}

}  // namespace mla
