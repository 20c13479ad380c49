// Internal interface between the C-ABI layer (api.cpp) and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace detred {

enum { EPI_STORE = 0, EPI_COMBINE = 1, EPI_ATOMIC = 2 };
enum { TILE_S16 = 0, TILE_M64 = 1, TILE_L128 = 2 };

struct GemmArgs {
    const uint16_t* X;
    long ldx;
    const uint16_t* W;
    long ldw;
    float* Y;             // output (EPI_STORE: slice z writes Y + z*out_z_stride)
    long ldy;
    long out_z_stride;
    float* part;          // EPI_COMBINE: S fp32 [M][N] partial planes
    unsigned* counters;   // EPI_COMBINE: one arrival counter per output tile
    int M, N, K;
    int Kc;               // chunk width
    int slices;           // grid slices along K
    int tiles_m, tiles_n;
};

void tile_shape(int tile, int* bm, int* bn);
// Launch the slice GEMM for a tile family; TILE_L128 uses the LDS-DMA engine
// whenever it supports the shape, else the register-staged engine.
hipError_t launch_slice_gemm(int tile, int epi, const GemmArgs& g, int cps, hipStream_t s);
hipError_t launch_reg_gemm(int tile, int epi, const GemmArgs& g, int cps, hipStream_t s);
bool lds_engine_supports(const GemmArgs& g, int cps);
hipError_t launch_lds_gemm(int epi, const GemmArgs& g, int cps, hipStream_t s);
hipError_t launch_tree_combine(const float* parts, size_t stride, int count, float* Y, size_t n,
                               hipStream_t s);
hipError_t launch_fill_zero(float* Y, long ld, int M, int N, hipStream_t s);
hipError_t launch_cast_bf16(const float* x, uint16_t* y, size_t n, hipStream_t s);

hipError_t launch_rmsnorm(const uint16_t* x, const uint16_t* gamma, float* y, int rows,
                          int hidden, float eps, hipStream_t s);
hipError_t launch_log_softmax(const float* x, float* y, int rows, int cols, hipStream_t s);
hipError_t launch_mean(const float* x, float* y, int rows, int cols, hipStream_t s);

}  // namespace detred
