// Internal declarations of libgdn's chunked prompt pass.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

constexpr int kChunk = 64;   // rows of a chunk (chunks never cross prompts)

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

// Byte offsets of the workspace arrays.  Per chunk (dense index over the
// prompts' chunks, at most T/64 + n_seqs) and value head, the sweep's
// matrix-core operands, each already in the lane order the sweep's MFMAs read:
//   blk  bf16 [NC][hv][kBlockElems]  W, U~ and P (40 KB)
//   gv   f32  [NC][hv][132]          e^{gamma_L}, e^gamma, e^{gamma_L - gamma}
// and per chunk and key head, what its value heads share (64 KB):
//   frag u32x4 [NC][hk][4][16][64]   K K^T, Q K^T, k^ and q^ fragments
struct PrefillLayout {
    size_t blk, gv, frag, total;
    int max_chunks_total;
};

PrefillLayout prefill_layout(int hk, int hv, int dk, int dv, int n_seqs, int total_rows);
bool prefill_supported(int hk, int hv, int dk, int dv);
size_t prefill_workspace_bytes(int hk, int hv, int dk, int dv, int n_seqs, int total_rows);
hipError_t launch_prefill(const PrefillArgs &P, hipStream_t stream);

}  // namespace gdn
