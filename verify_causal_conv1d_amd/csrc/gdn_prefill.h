// Internal declarations of libgdn's chunked prompt pass.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

struct PrefillArgs {
    int32_t hk, hv, dk, dv, C;
    int32_t n_seqs, total_rows, max_len;
    const int32_t *seq_start;
    const uint16_t *qkv, *a, *b;
    const float *conv_w, *a_log, *dt_bias;
    uint16_t *conv_tail;
    float *state;
    float *out;
    void *workspace;
};

bool prefill_supported(int hk, int hv, int dk, int dv);
size_t prefill_workspace_bytes(int hk, int hv, int dk, int dv, int n_seqs, int total_rows);
hipError_t launch_prefill(const PrefillArgs &P, hipStream_t stream);

}  // namespace gdn
