// Internal interface between the C-ABI layer (api.cpp) and the HIP kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace detred {

// A kernel's dynamic-LDS limit is raised once per device: `done` (one
// static per kernel) has bit d set once device d has it.  Devices past 63
// set it on every launch.
inline hipError_t ensure_lds_limit(std::atomic<unsigned long long>& done, const void* fn,
                                   int bytes)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    const unsigned long long bit = dev < 64 ? (1ull << dev) : 0ull;
    if (bit && (done.load(std::memory_order_acquire) & bit))
        return hipSuccess;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && bit)
        done.fetch_or(bit, std::memory_order_acq_rel);
    return e;
}

enum { EPI_STORE = 0, EPI_COMBINE = 1, EPI_ATOMIC = 2 };
enum { TILE_S16 = 0, TILE_M64 = 1, TILE_L128 = 2, TILE_L256 = 3, TILE_D64 = 4, TILE_W256 = 5 };

struct GemmArgs {
    const uint16_t* X;
    long ldx;
    const uint16_t* W;
    long ldw;
    // wt == 0: W is [K][N] (element (k, n) at W[k*ldw + n]); wt == 1: W is
    // given transposed, [N][K] (element (k, n) at W[n*ldw + k]).  The
    // products and their order are the same, so are the bits.
    int wt;
    float* Y;             // output (EPI_STORE: slice z writes Y + z*out_z_stride)
    long ldy;
    long out_z_stride;
    float* part;          // EPI_COMBINE: S fp32 [M][N] partial planes
    unsigned* counters;   // EPI_COMBINE: one arrival counter per output tile
    int M, N, K;
    int Kc;               // chunk width
    int slices;           // grid slices along K
    int tiles_m, tiles_n;
    // Output epilogue (the addmm entry point), applied only where the final
    // value p of an element of Y is written, never to partials or shard
    // roots: y = beta*C[row][col] + alpha*p (y = alpha*p when C is null),
    // each product and the sum rounded as written; stored as bf16 (nearest
    // even) when out_bf16, else fp32.  epi == 0: y = p as fp32.
    int epi;
    const float* C;
    long ldc;             // 0: C is one row, broadcast to every row
    float alpha, beta;
    int out_bf16;
    // 256x256 root tile only: store the roots straight from the MFMA
    // registers (4-byte stores) instead of through LDS
    int direct_roots;
};

void tile_shape(int tile, int* bm, int* bn);
// Launch the slice GEMM for a tile family; TILE_L128 uses the LDS-DMA engine
// whenever it supports the shape, else the register-staged engine; TILE_L256
// (one-chunk slices storing their roots) and TILE_D64 (at most 64 rows)
// exist in the LDS-DMA engine only, and are chosen only where that engine
// supports the shape.
hipError_t launch_slice_gemm(int tile, int epi, const GemmArgs& g, int cps, hipStream_t s);
hipError_t launch_reg_gemm(int tile, int epi, const GemmArgs& g, int cps, hipStream_t s);
bool lds_engine_supports(int tile, const GemmArgs& g, int cps);
hipError_t launch_lds_gemm(int tile, int epi, const GemmArgs& g, int cps, hipStream_t s);
hipError_t launch_tree_combine(const float* parts, size_t stride, int count, float* Y, size_t n,
                               hipStream_t s);
// The same for [M][N] planes (g.M, g.N) into g.Y at row stride g.ldy, with
// the addmm epilogue of g when g.epi (N % 4 == 0).
hipError_t launch_tree_combine_rows(const float* parts, size_t stride, int count,
                                    const GemmArgs& g, hipStream_t s);
hipError_t launch_fill_zero(float* Y, long ld, int M, int N, hipStream_t s);
hipError_t launch_cast_bf16(const float* x, uint16_t* y, size_t n, hipStream_t s);

// Scratch of det_splitk_gemm_noalloc (noalloc.hip): a file-scope device
// array per device.  Counters at offset 0 (zero at rest), the partials
// after them.
constexpr size_t kNoallocScratchBytes = (size_t)32 << 20;
constexpr size_t kNoallocCounterBytes = (size_t)64 << 10;
// The device address of the current device's scratch; the first call on a
// device looks it up and zeroes its counters on stream s.
hipError_t noalloc_scratch(hipStream_t s, void** ptr);

hipError_t launch_rmsnorm(const uint16_t* x, const uint16_t* gamma, float* y, int rows,
                          int hidden, float eps, hipStream_t s);
hipError_t launch_rmsnorm_bf16(const uint16_t* x, const uint16_t* gamma, uint16_t* y, int rows,
                               int hidden, float eps, hipStream_t s);
// y = epilogue(p = 0) over an M x N output: the addmm of an empty product
hipError_t launch_epilogue_only(const GemmArgs& g, hipStream_t s);
// Decode attention (attention.hip).  q [B][Hq][D] bf16; k, v bf16 with D
// contiguous, element strides sb, sh, st for sequence, KV head, position;
// lens [B] int32 on the device; out [B][Hq][D] fp32.  part_o / part_ml:
// the per-chunk results, [B*Hq][nch][D] and [B*Hq][nch][2] fp32.
struct AttnArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    long sb, sh, st;
    const int* lens;
    float* out;
    float* part_o;
    float* part_ml;
    int B, Hq, Hkv, G, D, max_len, nch;
    float scale;
};
int attention_chunk();
hipError_t launch_decode_attention(const AttnArgs& a, hipStream_t s);

hipError_t launch_log_softmax(const float* x, float* y, int rows, int cols, hipStream_t s);
hipError_t launch_log_softmax_mean(const float* x, float* y, float* mu, int rows, int cols,
                                   hipStream_t s);
hipError_t launch_mean(const float* x, float* y, int rows, int cols, hipStream_t s);

}  // namespace detred
