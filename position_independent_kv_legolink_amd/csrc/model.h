// Launchers of the decoder-layer kernels (model.hip). Internal to the library.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace piclink {

enum LinearEpilogue : int {
    kStore = 0,      // out[0] = A W^T
    kResidual = 1,   // out[0] = A W^T + residual ([M][N], may alias out[0])
    kSwiGlu = 2,     // W rows alternate 32 gate and 32 up rows; out[0] [M][N/2] = SiLU(gate) * up
    kSplit3 = 3,     // columns [0, split0) -> out[0], [split0, split0 + split1) -> out[1], rest -> out[2]
};

// C = A W^T over bf16 operands with fp32 accumulation: A [m][k], W [n][k] (both row-major, k
// contiguous); n a multiple of 128, k a multiple of 64 (kSplit3: split0 and split1 multiples of 64).
// n a multiple of 256 runs the kernel whose operand tiles are loaded straight into LDS.
struct LinearCall {
    const void *a;
    const void *w;
    int m, n, k;
    int epilogue;
    void *out[3];
    int ld_out[3];
    int split0, split1;
    const void *residual;
};

hipError_t launch_linear(const LinearCall &c, hipStream_t stream);

// y [rows][dm] = x / sqrt(mean(x^2) + eps) * w, bf16 in and out (dm a multiple of 8, at most 8,192).
hipError_t launch_rmsnorm(const void *x, const void *w, void *y, int rows, int dm, float eps, hipStream_t stream);

}  // namespace piclink
