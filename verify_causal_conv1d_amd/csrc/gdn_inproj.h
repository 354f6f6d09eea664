// Internal declarations of libgdn's affine 4-bit in-projection.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

struct InprojArgs {
    int32_t rows, hidden, group;   // hidden % 128 == 0; group in {32, 64, 128}
    int32_t channels, hv;          // output features: [qkv (channels) | a (hv) | b (hv)]
    const uint16_t *x;             // [rows][hidden] bf16
    const uint32_t *wq;            // tiled codes [blocks][hidden / 128][64][4]
    const uint16_t *scales;        // tiled [blocks][hidden / group][16] bf16
    const uint16_t *biases;        // tiled [blocks][hidden / group][16] bf16
    uint16_t *qkv;                 // [rows][channels] bf16
    uint16_t *a, *b;               // [rows][hv] bf16
};

// MLX layout ([features][hidden / 8] words, [features][hidden / group]
// scales and biases) -> the tiled layout, blocks = ceil(features / 16).
struct InprojPackArgs {
    int32_t hidden, group, channels, hv, blocks;
    const uint32_t *wq;
    const uint16_t *scales, *biases;
    uint32_t *wq_tiled;
    uint16_t *scales_tiled, *biases_tiled;
};

hipError_t launch_inproj(const InprojArgs &A, hipStream_t stream);
hipError_t launch_inproj_pack(const InprojPackArgs &P, hipStream_t stream);

}  // namespace gdn
