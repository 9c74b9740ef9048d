// Launch interfaces between the host API and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

struct DecodeArgs {
    const void* q;               // bf16 [B, S, H, 576]
    const void* kv;              // bf16 rows of 1152 B or fp8 rows of 656 B
    const int32_t* block_table;  // dense
    const int32_t* cache_seqlens;
    const int32_t* indices;      // sparse
    const int32_t* topk_length;  // sparse: [B*S] top-k entries used per query token, or null (all)
    const float* attn_sink;      // [H] per-head sink logits, or null
    const int32_t* meta;         // scheduler metadata (device)
    float* o_part;               // [max_slots, H, 512] float32, or float16 when part_fp16
    float* lse_part;             // [max_slots, H]
    unsigned char* o_exp8;       // part_fp16: [max_slots, H, 8] int8 power-of-two exponents; byte 2 q + h
                                 // scales dims d with d / 128 = q and (d % 8) / 4 = h
    int part_fp16;               // split partials stored as scaled float16 (see the decode epilogues)
    void* out;                   // [B, S, H, 512]
    float* lse;                  // [B, H, S]
    int64_t num_rows;            // num_blocks * 64
    int batch, s_q, h_q, max_blocks, topk, causal, out_fp32;
    int num_parts, n_hblk, max_slots;
    float scale_log2;            // softmax_scale * log2(e)
    float rescale_tau;           // running-max threshold in log2 units (0 = exact running max)
    int32_t* meta_out;           // fused: the schedule computed in the kernel is written here (same layout)
    int fused;                   // decode64: compute the schedule in the kernel instead of reading meta
    int fixed_overhead;          // fused: the scheduler's per-item cost F
};

struct MetaArgs {
    const int32_t* cache_seqlens;   // dense: [batch]; sparse: topk_length [batch*s_q] or null
    int32_t* meta;
    int batch, s_q, max_blocks, topk, causal, num_parts, fixed_overhead;
};

struct CombineArgs {
    const float* o_part;         // float32, or float16 with o_exp8 exponents when part_fp16
    const float* lse_part;
    const unsigned char* o_exp8;
    int part_fp16;
    const int32_t* split_offsets;
    const float* attn_sink;      // [H] or null
    void* out;
    float* lse;
    int num_items, h_q, s_q, out_fp32, skip_single;
};

struct GatherArgs {
    const int32_t* table_or_indices;
    const int32_t* cache_seqlens;   // dense: [batch]; sparse: topk_length [batch*s_q] or null
    int32_t* rows_out;
    int64_t num_rows;
    int batch, s_q, max_blocks, topk, causal, row_stride;
};

// kvf: 0 = bf16 rows of 576, 1 = 656-byte FP8 records, 2 = 528-byte FP8 records, 3 = 288-byte FP4 records
// (2 and 3: 512-wide head, sparse only)
hipError_t launch_decode(const DecodeArgs& a, bool sparse, int kvf, hipStream_t stream);
// dense bf16 cache, 64 heads per workgroup (num_head_blocks = ceil(h_q / 64))
hipError_t launch_decode64(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_metadata(const MetaArgs& a, hipStream_t stream);
hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);
hipError_t launch_gather(const GatherArgs& a, hipStream_t stream);

constexpr int kMaxMetaItems = 16384;   // batch * s_q handled by the one-workgroup scheduler
constexpr int kMaxFusedItems = 256;    // batch * s_q the decode64 kernel schedules itself (4 per lane)

}  // namespace mla
