// Host-side validation of the arrays a decode call reads (check.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mla_decode.h"

namespace mla {

// Checks host copies of the metadata words (NULL: skipped), cache_seqlens
// (dense), block table or top-k indices (NULL: skipped) and top-k lengths
// (NULL: none); writes the first failure into msg.  Returns OK or INVALID_ARG.
mla_status_t check_host_arrays(const mla_problem_t* p, const mla_metadata_t* m, const int32_t* words,
                               const int32_t* seqlens, const int32_t* toi, const int32_t* topk_length,
                               int64_t num_rows, char* msg, size_t msg_len);

// MLA_DEBUG=1 in the environment.
bool debug_enabled();

// Debug mode of an entry point: synchronises ``stream``, copies the device
// arrays the call reads to the host and checks them (the metadata words too
// when check_words_too); prints the first failure to stderr.  Refuses streams
// that are capturing a graph.
mla_status_t debug_check_call(const mla_problem_t* p, const mla_metadata_t* m, bool check_words_too,
                              const int32_t* seqlens, const int32_t* toi, const int32_t* topk_length,
                              int64_t num_rows, hipStream_t stream, const char* entry);

// Debug mode of mla_combine: split_offsets is a prefix sum starting at 0.
mla_status_t debug_check_offsets(const int32_t* split_offsets, int32_t num_items, hipStream_t stream);

}  // namespace mla
