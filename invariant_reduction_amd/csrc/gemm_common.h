// Pieces shared by the two slice-GEMM engines (register-staged and
// LDS-DMA): tile bookkeeping, the fold of a chunk into the fixed tree, and
// the three epilogues (direct store, last-arriver tree combine, atomics).
//
// The reduction every engine implements (see include/detred.h): K is cut
// into P chunks; a chunk is a chain of v_mfma_f32_16x16x32_bf16 steps over
// its k in increasing order from +0; the chunk values are added by the
// binary tree ((c0+c1)+(c2+c3))+((c4+c5)+(c6+c7)).  A workgroup folds the
// chunks of its slice with a binary counter: after chunk c the running
// value is added to the stored left sibling once per trailing one bit of c,
// which evaluates exactly the subtree over the slice's chunks.  Sources:
// "Reproducible LoRA Inference Through Deterministic Split-K Reduction"
// (Highlights; Q&A) and arXiv 2511.17826 (Abstract: one hierarchical binary
// tree for intra- and inter-GPU reduction orders).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bf16.h"
#include "kernels.h"

namespace detred {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int N>
struct Log2 { static constexpr int value = 1 + Log2<N / 2>::value; };
template <>
struct Log2<1> { static constexpr int value = 0; };

// Map the hardware workgroup id to a logical one so that consecutive logical
// tiles land on the same XCD (workgroups are dispatched round-robin over the
// 8 XCDs, each with its own L2).  A bijection on [0, G).
__device__ __forceinline__ int xcd_remap(int b, int G)
{
    const int xcd = b & 7, local = b >> 3;
    const int per = G >> 3, rem = G & 7;
    return xcd * per + (xcd < rem ? xcd : rem) + local;
}

// Output tile and slice of this workgroup.  Within a slice plane, tiles are
// walked in groups of GROUP_M tile rows: rows vary fastest inside a group,
// then columns, then groups.  The 32 workgroups an XCD runs at once then
// cover an 8 x 4 block of tiles, whose operands overlap in that XCD's L2.
constexpr int GROUP_M = 8;

struct TileCoord {
    int z;          // slice (or shard) index
    int tl;         // tile index within the slice plane
    int row0, col0; // first output row / column of the tile
};

__device__ __forceinline__ TileCoord tile_coord(const GemmArgs& g, int bm, int bn)
{
    const int G = g.tiles_m * g.tiles_n * g.slices;
    const int lid = xcd_remap(blockIdx.x, G);
    const int tiles = g.tiles_m * g.tiles_n;
    TileCoord t;
    t.z = lid / tiles;
    const int l = lid % tiles;
    const int per_group = GROUP_M * g.tiles_n;
    const int first_m = (l / per_group) * GROUP_M;
    const int rows_in_group = (g.tiles_m - first_m) < GROUP_M ? (g.tiles_m - first_m) : GROUP_M;
    const int in_group = l % per_group;
    const int tm = first_m + in_group % rows_in_group;
    const int tn = in_group / rows_in_group;
    t.tl = tn * g.tiles_m + tm;  // counter slot of the tile
    t.row0 = tm * bm;
    t.col0 = tn * bn;
    return t;
}

// Device-scope coherence bit (sc1) of the cache-policy operand of buffer
// loads and stores on gfx950.
constexpr int CPOL_SC1 = 16;
// Non-temporal bit (nt): the line is not kept in the caches after the
// store, so large outputs do not evict the operands still being read.
constexpr int CPOL_NT = 2;
// Raw buffer descriptor word 3: 32-bit data format, no swizzle.
constexpr int RAW_BUFFER_FLAGS = 0x00020000;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// s_waitcnt vmcnt(0): every vector-memory access of this wave has completed.
__device__ __forceinline__ void wait_vm_all()
{
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
}

// Store (or atomically add) a wave's FM x FN block of 16x16 MFMA results.
// Register q of a lane holds row 4*(lane/16)+q, column lane%16 of its tile.
// COHERENT stores are relaxed device-scope atomic stores: they are written
// through to the level every XCD reads, so a workgroup on another XCD can
// read them with device-coherent loads once they have completed.
template <int FM, int FN, bool COHERENT = false>
__device__ __forceinline__ void store_tile(const f32x4 (&acc)[FM][FN], float* out, long ld,
                                           int M, int N, int wrow0, int wcol0, int lane,
                                           bool atomic)
{
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int row = wrow0 + fm * 16 + 4 * (lane >> 4) + q;
                const int col = wcol0 + fn * 16 + (lane & 15);
                if (row < M && col < N) {
                    float* p = out + (size_t)row * ld + col;
                    if (atomic)
                        unsafeAtomicAdd(p, acc[fm][fn][q]);
                    else if (COHERENT)
                        __hip_atomic_store(p, acc[fm][fn][q], __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                    else
                        *p = acc[fm][fn][q];
                }
            }
}

// Fold chunk c (0-based within the slice) into the subtree.  Levels below
// REG_LEVELS are held in registers (stk); a level at or above REG_LEVELS is
// parked in this lane's slots of an LDS region (lds_top, one f32x4 per
// 16x16 tile, 64 lanes apart).
template <int FM, int FN, int LOG, int REG_LEVELS, int NSTK>
__device__ __forceinline__ void fold_chunk(int c, f32x4 (&acc)[FM][FN],
                                           f32x4 (&stk)[NSTK][FM][FN], f32x4* lds_top)
{
#pragma unroll
    for (int L = 0; L < LOG; ++L) {
        const bool in_lds = (L >= REG_LEVELS);
        if (c & (1 << L)) {
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) {
                    const f32x4 left = in_lds ? lds_top[(fm * FN + fn) * 64]
                                              : stk[in_lds ? 0 : L][fm][fn];
                    acc[fm][fn] = left + acc[fm][fn];
                }
        } else {
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) {
                    if (in_lds)
                        lds_top[(fm * FN + fn) * 64] = acc[fm][fn];
                    else
                        stk[in_lds ? 0 : L][fm][fn] = acc[fm][fn];
                }
            break;
        }
    }
}

// The final value of output element(s) under the epilogue of g (g.epi set):
// y = beta*c + alpha*p, or alpha*p without C; each operation rounds.
__device__ __forceinline__ float epi_value(const GemmArgs& g, float p, float c)
{
    const float ap = g.alpha * p;
    return g.C ? g.beta * c + ap : ap;
}

// Write the final value of element (row, col) of Y from its product p.
__device__ __forceinline__ void write_final1(const GemmArgs& g, int row, int col, float p)
{
    if (!g.epi) {
        g.Y[(size_t)row * g.ldy + col] = p;
        return;
    }
    const float c = g.C ? g.C[(size_t)row * g.ldc + col] : 0.0f;
    const float y = epi_value(g, p, c);
    if (g.out_bf16)
        reinterpret_cast<uint16_t*>(g.Y)[(size_t)row * g.ldy + col] = (uint16_t)f32_to_bf16_bits(y);
    else
        g.Y[(size_t)row * g.ldy + col] = y;
}

// The same for elements (row, col .. col+3), all inside M x N.
__device__ __forceinline__ void write_final4(const GemmArgs& g, int row, int col, float4 p)
{
    if (!g.epi) {
        *reinterpret_cast<float4*>(g.Y + (size_t)row * g.ldy + col) = p;
        return;
    }
    float4 c = make_float4(0.f, 0.f, 0.f, 0.f);
    if (g.C)
        c = *reinterpret_cast<const float4*>(g.C + (size_t)row * g.ldc + col);
    const float4 y = make_float4(epi_value(g, p.x, c.x), epi_value(g, p.y, c.y),
                                 epi_value(g, p.z, c.z), epi_value(g, p.w, c.w));
    if (g.out_bf16) {
        uint2 o;
        o.x = f32_to_bf16_bits(y.x) | (f32_to_bf16_bits(y.y) << 16);
        o.y = f32_to_bf16_bits(y.z) | (f32_to_bf16_bits(y.w) << 16);
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(g.Y) + (size_t)row * g.ldy + col) = o;
    } else {
        *reinterpret_cast<float4*>(g.Y + (size_t)row * g.ldy + col) = y;
    }
}

// Arrival and combine of EPI_COMBINE, after this workgroup has issued the
// stores of its partial (plane z of g.part) with device-coherent stores:
// count the arrival on the tile's counter and let the last slice to arrive
// add the S = 8/CPS partials in the fixed tree order, write Y and reset the
// counter.
//
// Ordering without whole-cache maintenance: each wave waits until its
// partial stores have completed before the workgroup barrier that precedes
// the counter update, so every partial of the S-1 earlier arrivals is
// complete before the last arriver's update returns.  The last arriver
// issues its loads only after that update has returned, and reads with
// device-coherent loads.  No L2 write-back or invalidate is issued, so the
// other workgroups of the XCD keep their cached operands.  Requires
// (BM-1)*N + BN < 2^29 (32-bit buffer offsets within a tile's rows).
template <int BM, int BN, int THREADS, int CPS>
__device__ __forceinline__ void arrive_and_combine(const GemmArgs& g, const TileCoord& tc,
                                                   int tid, int* s_last)
{
    wait_vm_all();
    __syncthreads();
    constexpr int S = 8 / CPS;  // a combine only exists when K has 8 chunks
    if (tid == 0) {
        const unsigned prev = __hip_atomic_fetch_add(g.counters + tc.tl, 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        *s_last = (prev == (unsigned)(S - 1));
    }
    __syncthreads();
    if (!*s_last)
        return;

    // one descriptor per partial plane, based at the tile's first element
    const size_t plane = (size_t)g.M * g.N;
    __amdgpu_buffer_rsrc_t rs[S];
#pragma unroll
    for (int s = 0; s < S; ++s)
        rs[s] = __builtin_amdgcn_make_buffer_rsrc(
            g.part + (size_t)s * plane + (size_t)tc.row0 * g.N + tc.col0, 0, 0x7fffffff,
            RAW_BUFFER_FLAGS);

    // each thread combines VPT float4 vectors of the tile; all S*VPT loads
    // are issued before the first addition
    constexpr int VEC = BM * BN / 4;
    constexpr int VPT = (VEC / THREADS) < 2 ? 1 : 2;
    for (int v0 = tid; v0 < VEC; v0 += VPT * THREADS) {
        float4 vals_all[VPT][S];
        bool ok[VPT];
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            const int v = v0 + u * THREADS;
            const int r = v / (BN / 4), cc = 4 * (v % (BN / 4));
            ok[u] = (v < VEC) && tc.row0 + r < g.M && tc.col0 + cc < g.N;
            const int off = (r * g.N + cc) * 4;
#pragma unroll
            for (int s = 0; s < S; ++s) {
                float4 t = make_float4(0.f, 0.f, 0.f, 0.f);
                if (ok[u]) {
                    const u32x4 q = __builtin_amdgcn_raw_buffer_load_b128(rs[s], off, 0, CPOL_SC1);
                    t = make_float4(__uint_as_float(q.x), __uint_as_float(q.y),
                                    __uint_as_float(q.z), __uint_as_float(q.w));
                }
                vals_all[u][s] = t;
            }
        }
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
            if (!ok[u])
                continue;
            const int v = v0 + u * THREADS;
            const int r = v / (BN / 4), cc = 4 * (v % (BN / 4));
            float4(&vals)[S] = vals_all[u];
            // top levels of the tree over the S slice roots, adjacent pairs
#pragma unroll
            for (int w = S; w > 1; w >>= 1)
#pragma unroll
                for (int i = 0; i < (w >> 1); ++i) {
                    vals[i].x = vals[2 * i].x + vals[2 * i + 1].x;
                    vals[i].y = vals[2 * i].y + vals[2 * i + 1].y;
                    vals[i].z = vals[2 * i].z + vals[2 * i + 1].z;
                    vals[i].w = vals[2 * i].w + vals[2 * i + 1].w;
                }
            write_final4(g, tc.row0 + r, tc.col0 + cc, vals[0]);
        }
    }
    if (tid == 0)
        g.counters[tc.tl] = 0u;  // leave the counter ready for the next call
}

// Epilogue of a slice with per-lane stores.  EPI_STORE: write the subtree
// root to Y + z*out_z_stride (through the output epilogue when g.epi, which
// only single-slice calls set).  EPI_ATOMIC: atomically add it into Y.
// EPI_COMBINE: write it to partial plane z with device-coherent stores, then
// arrive_and_combine.
template <int BM, int BN, int THREADS, int CPS, int EPI, int FM, int FN>
__device__ __forceinline__ void finish_slice(const f32x4 (&acc)[FM][FN], const GemmArgs& g,
                                             const TileCoord& tc, int wrow0, int wcol0,
                                             int lane, int tid, int* s_last)
{
    if (EPI == EPI_STORE) {
        if (g.epi) {
            // the final product of a single-slice addmm
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int row = wrow0 + fm * 16 + 4 * (lane >> 4) + q;
                        const int col = wcol0 + fn * 16 + (lane & 15);
                        if (row < g.M && col < g.N)
                            write_final1(g, row, col, acc[fm][fn][q]);
                    }
            return;
        }
        store_tile<FM, FN>(acc, g.Y + (size_t)tc.z * g.out_z_stride, g.ldy, g.M, g.N, wrow0,
                           wcol0, lane, false);
        return;
    }
    if (EPI == EPI_ATOMIC) {
        store_tile<FM, FN>(acc, g.Y, g.ldy, g.M, g.N, wrow0, wcol0, lane, true);
        return;
    }
    store_tile<FM, FN, true>(acc, g.part + (size_t)tc.z * g.M * g.N, g.N, g.M, g.N, wrow0,
                             wcol0, lane, false);
    arrive_and_combine<BM, BN, THREADS, CPS>(g, tc, tid, s_last);
}

}  // namespace detred
