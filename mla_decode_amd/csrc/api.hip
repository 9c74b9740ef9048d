// Host side of the C ABI: validation, planning and launches.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/mla_decode.h"
#include "check.h"
#include "common.h"
#include "kernels.h"

namespace {

using mla::kBlock;

constexpr int kFixedOverhead = 0;
constexpr int kMaxDevices = 64;

int g_cu_count[kMaxDevices];
std::mutex g_cu_mu;

// Scratch memory of mla_decode_step_noalloc: the schedule's metadata words,
// then the split partials.  Each device holds its own copy for the life of
// the process.  Host code never names the array itself (on the host it is
// only a stand-in for the symbol): it uses the device address that
// hipGetSymbolAddress returns for the current device.
constexpr size_t kScratchBytes = size_t(128) << 20;
constexpr size_t kScratchMetaBytes = size_t(64) << 10;   // metadata words, at the start
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

void* g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

mla_status_t device_scratch(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MLA_ERR_HIP;
    std::lock_guard<std::mutex> g(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MLA_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return MLA_OK;
}

mla_status_t device_cus(int32_t* out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MLA_ERR_HIP;
    std::lock_guard<std::mutex> g(g_cu_mu);
    if (g_cu_count[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            return MLA_ERR_HIP;
        g_cu_count[dev] = n;
    }
    *out = g_cu_count[dev];
    return MLA_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Calls over a bf16 cache run the 64-heads-per-workgroup kernel: dense ones
// always, top-k ones when every row offset of the cache, and one row past its
// end, fits the 32-bit offsets of a buffer load (the kernel gathers rows
// through one buffer over the whole cache).  The quantised formats and larger
// top-k caches run the 128-heads-per-workgroup kernel.
bool uses_decode64(const mla_problem_t* p) {
    if (p->kv_format != MLA_KV_BF16_576) return false;
    return p->topk == 0 || ((int64_t)p->num_blocks * kBlock + 2) * 1152 < ((int64_t)1 << 32);
}
int32_t heads_per_block(const mla_problem_t* p) { return uses_decode64(p) ? 64 : mla::kHeadsPerWG; }

mla_status_t validate(const mla_problem_t* p) {
    if (!p) return MLA_ERR_INVALID_ARG;
    if (p->batch < 1 || p->s_q < 1 || p->h_q < 1 || p->num_blocks < 1) return MLA_ERR_INVALID_ARG;
    if (p->topk < 0 || p->max_blocks_per_seq < 0) return MLA_ERR_INVALID_ARG;
    if (p->causal != 0 && p->causal != 1) return MLA_ERR_INVALID_ARG;
    if (p->kv_format != MLA_KV_BF16_576 && p->kv_format != MLA_KV_FP8_656 && p->kv_format != MLA_KV_FP8_528 &&
        p->kv_format != MLA_KV_FP4_288)
        return MLA_ERR_INVALID_ARG;
    if (p->out_dtype != MLA_OUT_BF16 && p->out_dtype != MLA_OUT_FP32) return MLA_ERR_INVALID_ARG;
    if (!std::isfinite(p->softmax_scale) || !(p->softmax_scale > 0.f)) return MLA_ERR_INVALID_ARG;
    if (!(p->rescale_threshold >= 0.f && p->rescale_threshold <= 30.f)) return MLA_ERR_INVALID_ARG;
    // the 528- and 288-byte records carry the 512-wide head (K = V), read through top-k indices
    const bool d512 = p->kv_format == MLA_KV_FP8_528 || p->kv_format == MLA_KV_FP4_288;
    const int d_qk = d512 ? 512 : mla::kDqk;
    if (p->h_kv != 1 || p->d_qk != d_qk || p->d_v != mla::kDv || p->block_size != kBlock)
        return MLA_ERR_UNSUPPORTED;
    if (d512 && p->topk < 1) return MLA_ERR_UNSUPPORTED;
    if (p->topk == 0 && p->max_blocks_per_seq < 1) return MLA_ERR_INVALID_ARG;
    if (p->topk > 0 && p->causal) return MLA_ERR_UNSUPPORTED;
    const int64_t items = (int64_t)p->batch * p->s_q;
    if (items > mla::kMaxMetaItems) return MLA_ERR_UNSUPPORTED;
    const int64_t tiles = p->topk > 0 ? ((int64_t)p->topk + 63) / 64 : (int64_t)p->max_blocks_per_seq;
    if (items * (tiles + kFixedOverhead) >= ((int64_t)1 << 31)) return MLA_ERR_UNSUPPORTED;
    if ((int64_t)p->num_blocks * kBlock >= ((int64_t)1 << 31)) return MLA_ERR_UNSUPPORTED;
    if ((int64_t)items * p->h_q * mla::kDv >= ((int64_t)1 << 40)) return MLA_ERR_UNSUPPORTED;
    return MLA_OK;
}

bool same_problem(const mla_problem_t& a, const mla_problem_t& b) {
    return a.batch == b.batch && a.s_q == b.s_q && a.h_q == b.h_q && a.h_kv == b.h_kv && a.d_qk == b.d_qk &&
           a.d_v == b.d_v && a.block_size == b.block_size && a.num_blocks == b.num_blocks &&
           a.max_blocks_per_seq == b.max_blocks_per_seq && a.topk == b.topk && a.causal == b.causal &&
           a.kv_format == b.kv_format && a.out_dtype == b.out_dtype && a.softmax_scale == b.softmax_scale;
}

size_t meta_bytes(int64_t parts, int64_t items) {
    return (size_t)(mla::kMetaHeader + mla::kMetaRec * parts + items + 1) * sizeof(int32_t);
}

mla_status_t check_meta(const mla_problem_t* p, const mla_metadata_t* m) {
    if (!m || !m->dev || !aligned16(m->dev)) return MLA_ERR_INVALID_ARG;
    if (!same_problem(m->sig, *p)) return MLA_ERR_METADATA_MISMATCH;
    const int64_t items = (int64_t)p->batch * p->s_q;
    if (m->num_partitions < 1 || m->num_head_blocks != (p->h_q + heads_per_block(p) - 1) / heads_per_block(p) ||
        m->fixed_overhead != kFixedOverhead || m->max_splits != items + m->num_partitions ||
        m->bytes < meta_bytes(m->num_partitions, items))
        return MLA_ERR_METADATA_MISMATCH;
    return MLA_OK;
}

// Top-k items all cost ceil(topk/64) + F scheduler units, so the plan alone
// fixes the schedule.  When the partition size q = ceil(T/P) is a multiple of
// that cost, every partition boundary falls on an item boundary: no item is
// split and the decode kernel writes every output itself.  (A sufficient
// condition; otherwise the combine runs and merges whatever was split.)
bool sparse_items_whole(const mla_problem_t* p, const mla_metadata_t* m) {
    if (p->topk <= 0) return false;
    const int64_t cost = ((int64_t)p->topk + 63) / 64 + m->fixed_overhead;
    const int64_t total = (int64_t)p->batch * p->s_q * cost;
    const int64_t q = total > 0 ? (total + m->num_partitions - 1) / m->num_partitions : 1;
    return q % cost == 0;
}

// Problems whose decode call computes its own schedule (up to four items per
// lane of one wave): every cache format, dense or sparse.
bool step_fusable(const mla_problem_t* p) {
    return (int64_t)p->batch * p->s_q <= mla::kMaxFusedItems;
}

mla_status_t run_decode(const mla_problem_t* p, bool sparse, const void* q, const void* kv,
                        const int32_t* block_table, const int32_t* cache_seqlens, const int32_t* indices,
                        const int32_t* topk_length, const float* attn_sink, const mla_metadata_t* meta,
                        void* ws, size_t ws_bytes, void* out, float* lse, void* stream, bool run_combine = true,
                        int64_t num_rows = 0, bool production_partials = true, bool fused = false) {
    mla_status_t st = validate(p);
    if (st != MLA_OK) return st;
    if (sparse != (p->topk > 0)) return MLA_ERR_INVALID_ARG;
    if (!q || !kv || !out || !lse || !aligned16(q) || !aligned16(kv) || !aligned16(out))
        return MLA_ERR_INVALID_ARG;
    if (sparse ? !indices : (!block_table || !cache_seqlens)) return MLA_ERR_INVALID_ARG;
    st = check_meta(p, meta);
    if (st != MLA_OK) return st;
    const size_t need = mla_workspace_bytes(meta);
    if (!ws || !aligned16(ws)) return need == 0 ? MLA_ERR_INVALID_ARG : MLA_ERR_WORKSPACE_TOO_SMALL;
    if (ws_bytes < need) return MLA_ERR_WORKSPACE_TOO_SMALL;

    hipStream_t s = (hipStream_t)stream;
    if (mla::debug_enabled()) {
        // a fused call writes the schedule itself: its inputs are checked here,
        // the schedule after the partial kernel
        st = mla::debug_check_call(p, meta, !fused, cache_seqlens, sparse ? indices : block_table, topk_length,
                                   num_rows, s, fused ? "mla_decode_step" : sparse ? "sparse decode" : "mla_decode_fwd");
        if (st != MLA_OK) return st;
    }

    const int64_t slots = meta->max_splits;
    mla::DecodeArgs a{};
    a.q = q;
    a.kv = kv;
    a.block_table = block_table;
    a.cache_seqlens = cache_seqlens;
    a.indices = indices;
    a.topk_length = sparse ? topk_length : nullptr;
    a.attn_sink = attn_sink;
    a.meta = (const int32_t*)meta->dev;
    a.o_part = (float*)ws;
    a.lse_part = (float*)ws + slots * p->h_q * mla::kDv;
    // With a bf16 output the split partials travel as scaled float16 (half the
    // bytes of the partial write and of the combine's read), their scales in
    // the second half of the float32 partial area; the test hook keeps float32
    // partials unless it is asked for the decode call's own format.
    a.part_fp16 = production_partials && p->out_dtype != MLA_OUT_FP32;
    a.o_exp8 = (unsigned char*)ws + slots * p->h_q * mla::kDv * 2;
    a.out = out;
    a.lse = lse;
    a.num_rows = num_rows > 0 ? num_rows : (int64_t)p->num_blocks * kBlock;   // rows a valid index may name
    a.batch = p->batch;
    a.s_q = p->s_q;
    a.h_q = p->h_q;
    a.max_blocks = p->max_blocks_per_seq;
    a.topk = p->topk;
    a.causal = p->causal;
    a.out_fp32 = p->out_dtype == MLA_OUT_FP32;
    a.num_parts = meta->num_partitions;
    a.n_hblk = meta->num_head_blocks;
    a.max_slots = (int)slots;
    a.scale_log2 = p->softmax_scale * 1.4426950408889634f;
    a.rescale_tau = p->rescale_threshold;
    a.fused = fused ? 1 : 0;
    a.meta_out = fused ? (int32_t*)meta->dev : nullptr;
    a.fixed_overhead = meta->fixed_overhead;
    const hipError_t e = uses_decode64(p) ? mla::launch_decode64(a, s) : mla::launch_decode(a, sparse, p->kv_format, s);
    if (e != hipSuccess) return MLA_ERR_HIP;
    if (fused && mla::debug_enabled()) {
        st = mla::debug_check_call(p, meta, true, cache_seqlens, sparse ? indices : block_table, topk_length, num_rows,
                                   s, "mla_decode_step");
        if (st != MLA_OK) return st;
    }

    mla::CombineArgs c{};
    c.o_part = a.o_part;
    c.lse_part = a.lse_part;
    c.o_exp8 = a.o_exp8;
    c.part_fp16 = a.part_fp16;
    c.split_offsets = a.meta + mla::kMetaHeader + mla::kMetaRec * meta->num_partitions;
    c.attn_sink = attn_sink;
    c.out = out;
    c.lse = lse;
    c.num_items = p->batch * p->s_q;
    c.h_q = p->h_q;
    c.s_q = p->s_q;
    c.out_fp32 = a.out_fp32;
    c.skip_single = 1;
    const bool skip = sparse && !topk_length && sparse_items_whole(p, meta);
    if (run_combine && !skip && mla::launch_combine(c, s) != hipSuccess) return MLA_ERR_HIP;
    return MLA_OK;
}

}  // namespace

extern "C" {

int32_t mla_abi_version(void) { return MLA_DECODE_ABI_VERSION; }

const char* mla_status_string(mla_status_t s) {
    switch (s) {
        case MLA_OK: return "ok";
        case MLA_ERR_INVALID_ARG: return "invalid argument";
        case MLA_ERR_UNSUPPORTED: return "unsupported problem";
        case MLA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case MLA_ERR_METADATA_MISMATCH: return "metadata was planned for another problem";
        case MLA_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

mla_status_t mla_plan(const mla_problem_t* problem, int32_t num_cus, mla_metadata_t* meta) {
    if (!meta || num_cus < 0) return MLA_ERR_INVALID_ARG;
    mla_status_t st = validate(problem);
    if (st != MLA_OK) return st;
    if (num_cus == 0) {
        st = device_cus(&num_cus);
        if (st != MLA_OK) return st;
    }
    const int32_t hblk = (problem->h_q + heads_per_block(problem) - 1) / heads_per_block(problem);
    int32_t parts = num_cus / hblk;
    if (parts < 1) parts = 1;
    const int64_t items = (int64_t)problem->batch * problem->s_q;
    meta->sig = *problem;
    meta->num_partitions = parts;
    meta->num_head_blocks = hblk;
    meta->fixed_overhead = kFixedOverhead;
    meta->max_splits = (int32_t)(items + parts);
    meta->dev = nullptr;
    meta->bytes = meta_bytes(parts, items);
    return MLA_OK;
}

size_t mla_workspace_bytes(const mla_metadata_t* meta) {
    if (!meta) return 0;
    return (size_t)meta->max_splits * (size_t)meta->sig.h_q * (mla::kDv + 1) * sizeof(float);
}

mla_status_t mla_get_decode_metadata(const mla_problem_t* problem, const int32_t* cache_seqlens,
                                     const int32_t* topk_length, mla_metadata_t* meta, void* stream) {
    mla_status_t st = validate(problem);
    if (st != MLA_OK) return st;
    st = check_meta(problem, meta);
    if (st != MLA_OK) return st;
    if (problem->topk == 0 && !cache_seqlens) return MLA_ERR_INVALID_ARG;
    const bool debug = mla::debug_enabled();
    hipStream_t s = (hipStream_t)stream;
    if (debug) {
        st = mla::debug_check_call(problem, meta, false, cache_seqlens, nullptr, topk_length, 0, s,
                                   "mla_get_decode_metadata");
        if (st != MLA_OK) return st;
    }
    mla::MetaArgs a{};
    a.cache_seqlens = problem->topk > 0 ? topk_length : cache_seqlens;
    a.meta = (int32_t*)meta->dev;
    a.batch = problem->batch;
    a.s_q = problem->s_q;
    a.max_blocks = problem->max_blocks_per_seq;
    a.topk = problem->topk;
    a.causal = problem->causal;
    a.num_parts = meta->num_partitions;
    a.fixed_overhead = meta->fixed_overhead;
    if (mla::launch_metadata(a, s) != hipSuccess) return MLA_ERR_HIP;
    // debug mode: the schedule just written is checked as well
    return debug ? mla::debug_check_call(problem, meta, true, cache_seqlens, nullptr, topk_length, 0, s,
                                         "mla_get_decode_metadata")
                 : MLA_OK;
}

mla_status_t mla_decode_fwd(const mla_problem_t* problem, const void* q, const void* kv_cache,
                            const int32_t* block_table, const int32_t* cache_seqlens, const float* attn_sink,
                            const mla_metadata_t* meta, void* workspace, size_t workspace_bytes, void* out,
                            float* lse, void* stream) {
    return run_decode(problem, false, q, kv_cache, block_table, cache_seqlens, nullptr, nullptr, attn_sink, meta,
                      workspace, workspace_bytes, out, lse, stream);
}

mla_status_t mla_sparse_decode_fwd(const mla_problem_t* problem, const void* q, const void* kv_cache,
                                   const int32_t* indices, const int32_t* topk_length, const float* attn_sink,
                                   const mla_metadata_t* meta, void* workspace, size_t workspace_bytes, void* out,
                                   float* lse, void* stream) {
    return run_decode(problem, true, q, kv_cache, nullptr, nullptr, indices, topk_length, attn_sink, meta,
                      workspace, workspace_bytes, out, lse, stream);
}

mla_status_t mla_sparse_prefill_fwd(const mla_problem_t* problem, int32_t s_kv, const void* q, const void* kv,
                                    const int32_t* indices, const int32_t* topk_length, const float* attn_sink,
                                    const mla_metadata_t* meta, void* workspace, size_t workspace_bytes, void* out,
                                    float* lse, void* stream) {
    if (!problem || problem->batch != 1 || problem->topk < 1) return MLA_ERR_INVALID_ARG;
    if (s_kv < 1 || (int64_t)s_kv > (int64_t)problem->num_blocks * kBlock) return MLA_ERR_INVALID_ARG;
    return run_decode(problem, true, q, kv, nullptr, nullptr, indices, topk_length, attn_sink, meta, workspace,
                      workspace_bytes, out, lse, stream, true, s_kv);
}

mla_status_t mla_combine(int32_t num_items, int32_t h_q, int32_t s_q, const float* o_part, const float* lse_part,
                         const int32_t* split_offsets, const float* attn_sink, int32_t out_dtype, void* out,
                         float* lse, void* stream) {
    if (num_items < 1 || h_q < 1 || s_q < 1 || num_items % s_q != 0) return MLA_ERR_INVALID_ARG;
    if (!o_part || !lse_part || !split_offsets || !out || !lse) return MLA_ERR_INVALID_ARG;
    if (!aligned16(o_part) || !aligned16(out)) return MLA_ERR_INVALID_ARG;
    if (out_dtype != MLA_OUT_BF16 && out_dtype != MLA_OUT_FP32) return MLA_ERR_INVALID_ARG;
    if ((int64_t)num_items * h_q >= ((int64_t)1 << 31) / 4) return MLA_ERR_UNSUPPORTED;
    if (mla::debug_enabled()) {
        const mla_status_t st = mla::debug_check_offsets(split_offsets, num_items, (hipStream_t)stream);
        if (st != MLA_OK) return st;
    }
    mla::CombineArgs c{};
    c.o_part = o_part;
    c.lse_part = lse_part;
    c.split_offsets = split_offsets;
    c.attn_sink = attn_sink;
    c.out = out;
    c.lse = lse;
    c.num_items = num_items;
    c.h_q = h_q;
    c.s_q = s_q;
    c.out_fp32 = out_dtype == MLA_OUT_FP32;
    c.skip_single = 0;
    return mla::launch_combine(c, (hipStream_t)stream) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status_t mla_debug_decode_partial(const mla_problem_t* problem, const void* q, const void* kv_cache,
                                      const int32_t* table_or_indices, const int32_t* cache_seqlens,
                                      const int32_t* topk_length, const float* attn_sink,
                                      const mla_metadata_t* meta, void* workspace, size_t workspace_bytes,
                                      void* out, float* lse, int32_t partial_format, void* stream) {
    if (!problem || partial_format < 0 || partial_format > 2) return MLA_ERR_INVALID_ARG;
    const bool sparse = problem->topk > 0;
    const bool fused = partial_format == 2 && validate(problem) == MLA_OK && step_fusable(problem);
    return run_decode(problem, sparse, q, kv_cache, sparse ? nullptr : table_or_indices,
                      sparse ? nullptr : cache_seqlens, sparse ? table_or_indices : nullptr, topk_length,
                      attn_sink, meta, workspace, workspace_bytes, out, lse, stream, false, 0, partial_format >= 1,
                      fused);
}

mla_status_t mla_debug_gather_rows(const mla_problem_t* problem, const int32_t* table_or_indices,
                                   const int32_t* cache_seqlens, const int32_t* topk_length, int32_t* rows_out,
                                   void* stream) {
    mla_status_t st = validate(problem);
    if (st != MLA_OK) return st;
    if (!table_or_indices || !rows_out || (problem->topk == 0 && !cache_seqlens)) return MLA_ERR_INVALID_ARG;
    if (mla::debug_enabled()) {
        st = mla::debug_check_call(problem, nullptr, false, cache_seqlens, table_or_indices, topk_length, 0,
                                   (hipStream_t)stream, "mla_debug_gather_rows");
        if (st != MLA_OK) return st;
    }
    mla::GatherArgs g{};
    g.table_or_indices = table_or_indices;
    g.cache_seqlens = problem->topk > 0 ? topk_length : cache_seqlens;
    g.rows_out = rows_out;
    g.num_rows = (int64_t)problem->num_blocks * kBlock;
    g.batch = problem->batch;
    g.s_q = problem->s_q;
    g.max_blocks = problem->max_blocks_per_seq;
    g.topk = problem->topk;
    g.causal = problem->causal;
    g.row_stride = problem->topk > 0 ? 64 * ((problem->topk + 63) / 64) : 64 * problem->max_blocks_per_seq;
    return mla::launch_gather(g, (hipStream_t)stream) == hipSuccess ? MLA_OK : MLA_ERR_HIP;
}

mla_status_t mla_decode_step(const mla_problem_t* problem, const void* q, const void* kv_cache,
                             const int32_t* table_or_indices, const int32_t* cache_seqlens,
                             const int32_t* topk_length, const float* attn_sink, const mla_metadata_t* meta,
                             void* workspace, size_t workspace_bytes, void* out, float* lse, void* stream) {
    mla_status_t st = validate(problem);
    if (st != MLA_OK) return st;
    const bool sparse = problem->topk > 0;
    if (!table_or_indices || (!sparse && !cache_seqlens)) return MLA_ERR_INVALID_ARG;
    if (step_fusable(problem))
        return run_decode(problem, sparse, q, kv_cache, sparse ? nullptr : table_or_indices,
                          sparse ? nullptr : cache_seqlens, sparse ? table_or_indices : nullptr,
                          sparse ? topk_length : nullptr, attn_sink, meta, workspace, workspace_bytes, out, lse,
                          stream, true, 0, true, true);
    st = mla_get_decode_metadata(problem, sparse ? nullptr : cache_seqlens, sparse ? topk_length : nullptr,
                                 (mla_metadata_t*)meta, stream);
    if (st != MLA_OK) return st;
    return run_decode(problem, sparse, q, kv_cache, sparse ? nullptr : table_or_indices,
                      sparse ? nullptr : cache_seqlens, sparse ? table_or_indices : nullptr,
                      sparse ? topk_length : nullptr, attn_sink, meta, workspace, workspace_bytes, out, lse, stream);
}

mla_status_t mla_decode_step_noalloc(const mla_problem_t* problem, int32_t num_cus, const void* q,
                                     const void* kv_cache, const int32_t* table_or_indices,
                                     const int32_t* cache_seqlens, const int32_t* topk_length,
                                     const float* attn_sink, void* out, float* lse, void* stream) {
    mla_metadata_t m{};
    mla_status_t st = mla_plan(problem, num_cus, &m);
    if (st != MLA_OK) return st;
    // sizes are checked before the device is touched
    if (m.bytes > kScratchMetaBytes || mla_workspace_bytes(&m) > kScratchBytes - kScratchMetaBytes)
        return MLA_ERR_WORKSPACE_TOO_SMALL;
    const bool sparse = problem->topk > 0;
    if (!table_or_indices || (!sparse && !cache_seqlens)) return MLA_ERR_INVALID_ARG;
    void* base = nullptr;
    st = device_scratch(&base);
    if (st != MLA_OK) return st;
    m.dev = base;
    return mla_decode_step(problem, q, kv_cache, table_or_indices, cache_seqlens, topk_length, attn_sink, &m,
                           (unsigned char*)base + kScratchMetaBytes, kScratchBytes - kScratchMetaBytes, out, lse,
                           stream);
}

mla_status_t mla_check_inputs(const mla_problem_t* problem, const mla_metadata_t* meta, const int32_t* meta_words,
                              const int32_t* cache_seqlens, const int32_t* table_or_indices,
                              const int32_t* topk_length, int64_t num_rows, char* msg, size_t msg_len) {
    if (msg && msg_len) msg[0] = 0;
    mla_status_t st = validate(problem);
    if (st != MLA_OK) return st;
    if (meta_words) {
        if (!meta) return MLA_ERR_INVALID_ARG;
        if (!same_problem(meta->sig, *problem) || meta->num_partitions < 1 ||
            meta->num_head_blocks != (problem->h_q + heads_per_block(problem) - 1) / heads_per_block(problem) ||
            meta->max_splits != (int64_t)problem->batch * problem->s_q + meta->num_partitions)
            return MLA_ERR_METADATA_MISMATCH;
    }
    if (num_rows < 0 || num_rows > (int64_t)problem->num_blocks * kBlock) return MLA_ERR_INVALID_ARG;
    return mla::check_host_arrays(problem, meta, meta_words, cache_seqlens, table_or_indices, topk_length, num_rows,
                                  msg, msg_len);
}

}  // extern "C"
