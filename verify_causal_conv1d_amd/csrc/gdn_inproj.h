// Internal declarations of libgdn's affine 4-bit in-projection.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

struct InprojArgs {
    int32_t rows, hidden, group;   // hidden % 128 == 0; group in {32, 64, 128}
    int32_t channels, hv;          // output features: [qkv (channels) | a (hv) | b (hv)]
    const uint16_t *x;             // [rows][hidden] bf16
    const uint32_t *wq;            // [features][hidden / 8] packed 4-bit codes
    const uint16_t *scales;        // [features][hidden / group] bf16
    const uint16_t *biases;        // [features][hidden / group] bf16
    uint16_t *qkv;                 // [rows][channels] bf16
    uint16_t *a, *b;               // [rows][hv] bf16
};

hipError_t launch_inproj(const InprojArgs &A, hipStream_t stream);

}  // namespace gdn
