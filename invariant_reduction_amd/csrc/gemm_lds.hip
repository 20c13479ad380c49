// LDS-DMA slice GEMM engine for gfx950: the wide-output workgroup tiles,
// 128x128 (eight waves of 64x32, any chunk count; four of 64x64 for
// one-chunk root stores), 256x256 (eight waves of 128x64, one-chunk slices
// only: its accumulators leave no registers for a subtree) and 64x128 for
// products of at most 64 rows (eight waves of 32x32).  Same reduction
// order and output values as the register-staged engine (gemm_common.h);
// split products on these tiles write their subtree roots and are
// combined by a second launch, so no last-arriver combine lives here.  The
// data movement differs:
//
//  * global -> LDS with buffer_load_dwordx4 ... lds (no register staging),
//    STAGES K blocks of 64 in flight (two to four, see Stages); the
//    buffer descriptors' record counts turn rows past M into zeros.  These
//    loads are issued from inline assembly (they have no register result)
//    and waited for explicitly with s_waitcnt vmcnt + s_barrier: issued
//    through the compiler builtin, they make every later ds_read_b64_tr_b16
//    wait for all outstanding loads, which would leave one stage in flight;
//  * A (X, K-contiguous) is stored [m][k] and read as one 16-byte
//    ds_read_b128 per MFMA operand;
//  * B (W, N-contiguous) is stored [k][n] as loaded and read with
//    ds_read_b64_tr_b16, which hands each lane four consecutive k of one
//    column; two such reads form one MFMA operand.  A W given transposed
//    ([N][K], the layout of a linear layer's weight) is stored [n][k] and
//    read like A;
//  * both layouts XOR-swizzle 16-byte chunks within a row so that the
//    fragment reads spread over the LDS banks (the DMA writes each wave's
//    1 KiB contiguously, so the swizzle is chosen by which global chunk
//    each lane fetches);
//  * the finished tile goes out through the stage buffers as whole 16-byte
//    row pieces (store_tile_via_lds; the 256x256 tile in two halves), with
//    the addmm epilogue applied on the way when the call asks for it.
//
// Requires every 32-wide MFMA step to lie inside K (K % 32 == 0 when K is
// one chunk; always true with 8 chunks), so no step needs zero padding.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gemm_common.h"

namespace detred {

namespace lds {

constexpr int BK = 64;
constexpr int KSTEPS = BK / 32;
constexpr int BUFFER_DWORD3 = 0x00020000;     // raw buffer, 32-bit data format

// Workgroup tile: WAVES_M x WAVES_N waves, each a TM x TN block of 16x16
// MFMA tiles; a stage holds one 64-wide K block of A and of B.
template <int BM_, int BN_, int WAVES_M_, int WAVES_N_>
struct LdsTile {
    static constexpr int BM = BM_, BN = BN_;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int WAVES = WAVES_M * WAVES_N, THREADS = 64 * WAVES;
    static constexpr int TM = BM / WAVES_M, TN = BN / WAVES_N;
    static constexpr int FM = TM / 16, FN = TN / 16;
    static constexpr int A_BYTES = BM * BK * 2;
    static constexpr int B_BYTES = BK * BN * 2;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    // 16-byte loads per lane of a stage's A and B blocks
    static constexpr int LOADS_A = A_BYTES / (THREADS * 16);
    static constexpr int LOADS_B = B_BYTES / (THREADS * 16);
    static constexpr int B_ROW_CHUNKS = BN / 8;              // 16-byte chunks per k-row of B
    static constexpr int PARK_BYTES = WAVES * FM * FN * 64 * 16;  // one subtree level
    static_assert(LOADS_A >= 1 && LOADS_A * THREADS * 16 == A_BYTES &&
                      LOADS_B * THREADS * 16 == B_BYTES,
                  "A and B blocks take whole numbers of loads per lane");
};
// Eight waves (two per SIMD) rather than four of 64x64: the second wave of
// each SIMD issues while the first waits on LDS or on its loads (dense
// 256x14336x4096 54.8 -> 51.7 us, 4096 rows 672 -> 628 us, one row at
// 8 slices 35.3 -> 31.0 us on MI355X; same bits).
using Tile128 = LdsTile<128, 128, 2, 4>;
// Four waves of 64x64 for one-chunk slices that store their roots (shards
// not on the 256x256 tile): there the eight-wave form is slower (8 shards
// of 512x8192x8192: 104 vs 112 us; 4096x4096x4096: 238 vs 245 us).
using Tile128x4 = LdsTile<128, 128, 2, 2>;
using Tile256 = LdsTile<256, 256, 2, 4>;
// Products of at most 64 rows (decode and small batches): 64x128, eight
// waves of 32x32.  The A block shrinks to 8 KiB, so the LDS holds more
// weight blocks in flight (64 rows of 4096x14336 at 8 slices, weights from
// HBM: 41.0 -> 32.6 us against 128x128; a 32x128 tile was no faster
// below 32 rows).
using TileD64 = LdsTile<64, 128, 2, 4>;
// Eight-chunk products of 1024 rows or more: 192x128, eight waves of 96x32
// (two per SIMD).  Half again the rows of the 128x128 tile per workgroup,
// so each weight block in LDS serves 1.5 times the MFMAs and the LDS bytes
// per MFMA drop by a fifth; the cost is 48 more accumulator registers per
// saved subtree level, which fit because the top level waits in the
// workgroup's own output tile of Y between chunk 3 and chunk 7 (the call
// needs no workspace).  Measured on MI355X against the 128x128 tile: 1024
// rows of 4096x14336 205 -> 195 us, 4096 rows 635 -> 621 us.
using TileW = LdsTile<192, 128, 2, 4>;

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
#define DETRED_LDS __attribute__((address_space(3)))

// s_waitcnt with only vmcnt limited (expcnt and lgkmcnt left at maximum).
template <int VM>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(VM >= 0 && VM < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | (15 << 8) | ((VM >> 4) << 14));
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor: 48-bit base, stride 0, record count in bytes.
__device__ __forceinline__ i32x4 buffer_desc(const void* base, uint32_t bytes)
{
    const uint64_t a = (uint64_t)base;
    i32x4 d;
    d.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    d.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xffff);
    d.z = __builtin_amdgcn_readfirstlane((int)bytes);
    d.w = BUFFER_DWORD3;
    return d;
}

// One 16-byte-per-lane load from the buffer at byte offset voff into LDS at
// lds_base + 16*lane (lds_base wave-uniform).  Offsets at or past the record
// count load zeros.  Completion is tracked by vmcnt only.
__device__ __forceinline__ void dma16(uint32_t lds_base, uint32_t voff, const i32x4& desc)
{
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    // m0 is written here; no compiler-generated code in these kernels
    // keeps a value in m0 across this statement
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds"
        :
        : "s"(lds_base), "v"(voff), "s"(desc)
        : "memory", "m0");
#pragma clang diagnostic pop
}


// dma16 with a wave-uniform part of the offset in an SGPR: the load reads
// the buffer at voff + soff.
__device__ __forceinline__ void dma16s(uint32_t lds_base, uint32_t voff, uint32_t soff,
                                       const i32x4& desc)
{
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen lds"
        :
        : "s"(lds_base), "v"(voff), "s"(desc), "s"(soff)
        : "memory", "m0");
#pragma clang diagnostic pop
}

// dma16s through a buffer resource value (as made by
// __builtin_amdgcn_make_buffer_rsrc), non-temporal: for data read once,
// which should not push reused operand blocks out of the L2.
__device__ __forceinline__ void dma16r(uint32_t lds_base, uint32_t voff, uint32_t soff,
                                       __amdgpu_buffer_rsrc_t rs)
{
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen nt lds"
        :
        : "s"(lds_base), "v"(voff), "s"(rs), "s"(soff)
        : "memory", "m0");
#pragma clang diagnostic pop
}

// s_waitcnt lgkmcnt(0): every LDS read of this wave has returned.
__device__ __forceinline__ void wait_lgkmcnt0()
{
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}

// MFMA I of N followed by its share of the READS reads, PER at most.
template <int I, int N, int READS, int PER>
__device__ __forceinline__ void spread_reads()
{
    if constexpr (I < N) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        constexpr int left = READS - I * PER;
        constexpr int here = left < PER ? (left > 0 ? left : 0) : PER;
        if constexpr (here > 0)
            __builtin_amdgcn_sched_group_barrier(0x100, here, 0);
        spread_reads<I + 1, N, READS, PER>();
    }
}

// Scheduling hint for one k step: alternate its 16 MFMAs with the LDS
// reads of the next k step (4 A and 8 transposed B reads, or 4 + 4 when W
// comes transposed).
template <class T, bool WT>
__device__ __forceinline__ void interleave_reads_with_mfma()
{
    constexpr int READS = WT ? T::FM + T::FN : T::FM + 2 * T::FN;
    constexpr int MFMAS = T::FM * T::FN;
    if constexpr (READS <= MFMAS) {
#pragma unroll
        for (int i = 0; i < READS; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, MFMAS - READS, 0);
    } else {
        // small wave tiles: more reads than MFMAs, spread over them
        spread_reads<0, MFMAS, READS, (READS + MFMAS - 1) / MFMAS>();
    }
}

// Swizzle of the B tile: k-row k keeps its 16 chunks of 8 columns, with the
// chunk index XORed by 2*h(k).  The 16 rows one transposed read touches
// (k0 + 8g + r, r < 4, g < 4) then hit 8 distinct bank windows, twice each.
__device__ __forceinline__ int b_swz(int k) { return 2 * ((k & 3) + 4 * ((k >> 3) & 1)); }

// Fragments of one k step: A as 16-byte reads, B as two transposed reads
// (k0..k0+3 and k0+4..k0+7 of the lane's column).
template <class T>
__device__ __forceinline__ void load_frags(bf16x8 (&af)[T::FM], bf16x8 (&bfr)[T::FN],
                                           const uint8_t* st, uint32_t a_addr,
                                           const uint32_t (&b_addr)[T::FN], int ks)
{
    constexpr int ROW = T::BN * 2;  // bytes per k-row of B
#pragma unroll
    for (int fm = 0; fm < T::FM; ++fm)
        af[fm] = *reinterpret_cast<const bf16x8*>(st + a_addr + fm * 16 * 8 * 16);
#pragma unroll
    for (int fn = 0; fn < T::FN; ++fn) {
        const uint8_t* pb = st + b_addr[fn] + ks * 32 * ROW;
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DETRED_LDS v4i16*)(pb));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DETRED_LDS v4i16*)(pb + 4 * ROW));
        const v8i16 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        bfr[fn] = __builtin_bit_cast(bf16x8, both);
    }
}

// Fragments of one k step when W comes transposed: B is stored [n][k] like
// A and read the same way, one 16-byte read per operand.
template <class T>
__device__ __forceinline__ void load_frags_wt(bf16x8 (&af)[T::FM], bf16x8 (&bfr)[T::FN],
                                              const uint8_t* st, uint32_t a_addr,
                                              uint32_t bt_addr)
{
#pragma unroll
    for (int fm = 0; fm < T::FM; ++fm)
        af[fm] = *reinterpret_cast<const bf16x8*>(st + a_addr + fm * 16 * 8 * 16);
#pragma unroll
    for (int fn = 0; fn < T::FN; ++fn)
        bfr[fn] = *reinterpret_cast<const bf16x8*>(st + T::A_BYTES + bt_addr + fn * 16 * 8 * 16);
}

template <class T>
__device__ __forceinline__ void mma_step(f32x4 (&acc)[T::FM][T::FN], const bf16x8 (&af)[T::FM],
                                         const bf16x8 (&bfr)[T::FN])
{
#pragma unroll
    for (int fm = 0; fm < T::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < T::FN; ++fn)
            acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[fm], bfr[fn], acc[fm][fn], 0,
                                                                  0, 0);
}

// Epilogue store through LDS.  The MFMA layout gives a lane four rows of
// one column, so direct stores are 4-byte scatters.  Instead the
// workgroup's fp32 tile is written to the (now idle) stage buffers
// row-major, with the 16-column group of each element XORed by (row/4)%4 so
// that the four row groups of a 16 x 16 result land in different banks;
// then every thread stores whole 16-byte row pieces.  A tile larger than
// the stage buffers goes in PASSES row halves, each written by the waves
// that own those rows.
// Subtree roots (several planes, out_z_stride set) go out with plain
// stores, as the combine reads them next; final outputs non-temporally (a
// large output would push out the operands still being read).
template <class T, int STAGES, bool EPI_OK = true>
__device__ __forceinline__ void store_tile_via_lds(const f32x4 (&acc)[T::FM][T::FN],
                                                   const GemmArgs& g, float* out, int ld, int row0,
                                                   int col0, int wm, int wn, int lane, int tid,
                                                   uint8_t* smem)
{
    constexpr int BN = T::BN;
    constexpr int PASSES = (T::BM * BN * 4 > STAGES * T::STAGE_BYTES) ? 2 : 1;
    constexpr int HR = T::BM / PASSES;  // rows per pass
    static_assert(HR * BN * 4 <= STAGES * T::STAGE_BYTES && HR % T::TM == 0,
                  "a pass fits the stage buffers and holds whole wave rows");
    const int M = g.M, N = g.N;
    float* t = reinterpret_cast<float*>(smem);
    // Stores (and epilogue loads of C) go through raw buffers based at the
    // tile's first element; a piece outside M x N gets an offset past the
    // record count, and the hardware drops the store (a load returns
    // zeros), so the loops have no branch and the reads stay batched.
    constexpr int OOB = (int)0x80000000u;
    // A thread's row pieces of a pass are read in groups of GROUP, each
    // group before its first store: the whole pass for a one-pass tile; 8
    // at a time when the other half's accumulators are still live.
    constexpr int ITER = HR * BN / 4 / T::THREADS;
    constexpr int GROUP = PASSES > 1 ? 8 : ITER;
    static_assert(ITER * T::THREADS * 4 == HR * BN && ITER % GROUP == 0,
                  "whole float4 pieces per thread, whole groups");
#pragma unroll
    for (int h = 0; h < PASSES; ++h) {
        __syncthreads();  // every wave is done with the stage buffers
        if (wm * T::TM / HR == h) {
#pragma unroll
            for (int fm = 0; fm < T::FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < T::FN; ++fn)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int r = wm * T::TM - h * HR + fm * 16 + 4 * (lane >> 4) + q;
                        const int c = wn * T::TN + fn * 16 + (lane & 15);
                        t[r * BN + (c ^ (16 * ((r >> 2) & 3)))] = acc[fm][fn][q];
                    }
        }
        __syncthreads();
        const int prow0 = row0 + h * HR;  // first output row of this pass
#pragma unroll
        for (int i0 = 0; i0 < ITER; i0 += GROUP) {
            u32x4 val[GROUP];
#pragma unroll
            for (int i = 0; i < GROUP; ++i) {
                const int v = tid + (i0 + i) * T::THREADS;
                const int r = v / (BN / 4), c4 = v % (BN / 4);
                val[i] = *reinterpret_cast<const u32x4*>(t + r * BN + 4 * (c4 ^ (4 * ((r >> 2) & 3))));
            }
            if (!EPI_OK || !g.epi) {
                const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                    out + (size_t)prow0 * ld + col0, 0, 0x7fffffff, RAW_BUFFER_FLAGS);
                auto put = [&](auto policy) {
#pragma unroll
                    for (int i = 0; i < GROUP; ++i) {
                        const int v = tid + (i0 + i) * T::THREADS;
                        const int r = v / (BN / 4), c4 = v % (BN / 4);
                        const bool in = (prow0 + r < M) && (col0 + 4 * c4 < N);
                        const int off = in ? (r * ld + 4 * c4) * 4 : OOB;
                        __builtin_amdgcn_raw_buffer_store_b128(val[i], rs, off, 0,
                                                               decltype(policy)::value);
                    }
                };
                if (g.out_z_stride)
                    put(std::integral_constant<int, 0>());
                else
                    put(std::integral_constant<int, CPOL_NT>());
                continue;
            }
            if constexpr (EPI_OK) {
            // the final product of a single-slice addmm: y = beta*C + alpha*p
            __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<float*>(g.C ? g.C : g.Y) + (size_t)prow0 * g.ldc + col0, 0,
                0x7fffffff, RAW_BUFFER_FLAGS);
            void* ybase =
                g.out_bf16 ? (void*)(reinterpret_cast<uint16_t*>(g.Y) + (size_t)prow0 * g.ldy + col0)
                           : (void*)(g.Y + (size_t)prow0 * g.ldy + col0);
            const __amdgpu_buffer_rsrc_t ry =
                __builtin_amdgcn_make_buffer_rsrc(ybase, 0, 0x7fffffff, RAW_BUFFER_FLAGS);
            u32x4 cv[GROUP];
#pragma unroll
            for (int i = 0; i < GROUP; ++i) {
                const int v = tid + (i0 + i) * T::THREADS;
                const int r = v / (BN / 4), c4 = v % (BN / 4);
                const bool in = (prow0 + r < M) && (col0 + 4 * c4 < N);
                cv[i] = u32x4{0u, 0u, 0u, 0u};
                if (g.C)
                    cv[i] = __builtin_amdgcn_raw_buffer_load_b128(
                        rc, in ? (int)((r * g.ldc + 4 * c4) * 4) : OOB, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < GROUP; ++i) {
                const int v = tid + (i0 + i) * T::THREADS;
                const int r = v / (BN / 4), c4 = v % (BN / 4);
                const bool in = (prow0 + r < M) && (col0 + 4 * c4 < N);
                float y[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    y[e] = epi_value(g, __uint_as_float(val[i][e]), __uint_as_float(cv[i][e]));
                if (g.out_bf16) {
                    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
                    const u32x2 o = {f32_to_bf16_bits(y[0]) | (f32_to_bf16_bits(y[1]) << 16),
                                     f32_to_bf16_bits(y[2]) | (f32_to_bf16_bits(y[3]) << 16)};
                    __builtin_amdgcn_raw_buffer_store_b64(
                        o, ry, in ? (int)((r * g.ldy + 4 * c4) * 2) : OOB, 0, CPOL_NT);
                } else {
                    const u32x4 o = {__float_as_uint(y[0]), __float_as_uint(y[1]),
                                     __float_as_uint(y[2]), __float_as_uint(y[3])};
                    __builtin_amdgcn_raw_buffer_store_b128(
                        o, ry, in ? (int)((r * g.ldy + 4 * c4) * 4) : OOB, 0, CPOL_NT);
                }
            }
            }
        }
    }
}

// Roots of the 256x256 tile straight from the MFMA layout: a lane holds four
// rows of one column per 16x16 block, so each store is 4 bytes and one
// instruction writes four 64-byte row pieces.  No LDS pass and no barrier:
// a wave stores as soon as its K loop ends.  Plain stores (the combine
// reads the roots next); pieces outside M x N are dropped by the buffer's
// range check.
template <class T>
__device__ __forceinline__ void store_roots_direct(const f32x4 (&acc)[T::FM][T::FN], float* out,
                                                   int ld, int M, int N, int wrow0, int wcol0,
                                                   int lane)
{
    constexpr int OOB = (int)0x80000000u;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        out + (size_t)wrow0 * ld + wcol0, 0, 0x7fffffff, RAW_BUFFER_FLAGS);
    // the lane index made opaque here, so that the 128 store offsets are
    // computed where they are used rather than hoisted into the K loop
    int l = lane;
    asm volatile("" : "+v"(l));
#pragma unroll
    for (int fm = 0; fm < T::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < T::FN; ++fn)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int r = fm * 16 + 4 * (l >> 4) + q, c = fn * 16 + (l & 15);
                const bool in = (wrow0 + r < M) && (wcol0 + c < N);
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[fm][fn][q]), rs,
                                                      in ? (r * ld + c) * 4 : OOB, 0, 0);
            }
}

// The top subtree level parked in the workgroup's own output tile of Y
// (PARK == 2): written once after chunk 3 and read back once after chunk 7,
// by the lane that wrote it.  A tile that lies wholly inside M x N holds
// the level as whole 16-byte pieces in an order of its own (lane slot s of
// block (fm, fn) of wave w, s = ((w*FM + fm)*FN + fn)*64 + lane, at tile
// row s/(BN/4), column 4*(s%(BN/4))); an edge tile keeps every value at
// its own element, and the buffer's range check drops (and reads as zero)
// the ones outside M x N, which no later step uses.  The final store
// overwrites the whole tile.
template <class T>
struct ParkOut {
    __amdgpu_buffer_rsrc_t rs;  // based at the tile's first element of Y
    bool full;                  // the tile lies wholly inside M x N
    int ld;                     // Y's row stride in elements
    int rows_left, cols_left;   // M - row0, N - col0
    int wave, wrow, wcol;       // wave index, its first row and column in the tile
};

template <class T>
__device__ __forceinline__ void park_out_store(const ParkOut<T>& po, const f32x4 (&v)[T::FM][T::FN],
                                               int lane_in)
{
    constexpr int OOB = (int)0x80000000u;
    // the lane index made opaque, so that the store offsets are computed
    // here rather than hoisted out of the K loops (where they would hold
    // registers for the whole kernel).  Full-tile slots take plain stores:
    // their read-back is non-temporal (4096x14336x4096: 569 -> 560 us
    // against non-temporal stores).
    int lane = lane_in;
    asm volatile("" : "+v"(lane));
#pragma unroll
    for (int fm = 0; fm < T::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < T::FN; ++fn) {
            if (po.full) {
                const int sl = ((po.wave * T::FM + fm) * T::FN + fn) * 64 + lane;
                const int off = ((sl / (T::BN / 4)) * po.ld + 4 * (sl % (T::BN / 4))) * 4;
                const u32x4 q = {__float_as_uint(v[fm][fn][0]), __float_as_uint(v[fm][fn][1]),
                                 __float_as_uint(v[fm][fn][2]), __float_as_uint(v[fm][fn][3])};
                __builtin_amdgcn_raw_buffer_store_b128(q, po.rs, off, 0, 0);
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int r = po.wrow + fm * 16 + 4 * (lane >> 4) + q;
                    const int c = po.wcol + fn * 16 + (lane & 15);
                    const bool in = r < po.rows_left && c < po.cols_left;
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[fm][fn][q]), po.rs,
                                                          in ? (r * po.ld + c) * 4 : OOB, 0,
                                                          CPOL_NT);
                }
            }
        }
}

// acc = parked + acc, element by element (the tree node's left operand is
// the parked level)
template <class T>
__device__ __forceinline__ void park_out_add(const ParkOut<T>& po, f32x4 (&acc)[T::FM][T::FN],
                                             int lane_in)
{
    constexpr int OOB = (int)0x80000000u;
    int lane = lane_in;  // opaque, as in park_out_store
    asm volatile("" : "+v"(lane));
#pragma unroll
    for (int fm = 0; fm < T::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < T::FN; ++fn) {
            f32x4 left;
            if (po.full) {
                const int sl = ((po.wave * T::FM + fm) * T::FN + fn) * 64 + lane;
                const int off = ((sl / (T::BN / 4)) * po.ld + 4 * (sl % (T::BN / 4))) * 4;
                const u32x4 q = __builtin_amdgcn_raw_buffer_load_b128(po.rs, off, 0, 0);
                left = f32x4{__uint_as_float(q.x), __uint_as_float(q.y), __uint_as_float(q.z),
                             __uint_as_float(q.w)};
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int r = po.wrow + fm * 16 + 4 * (lane >> 4) + q;
                    const int c = po.wcol + fn * 16 + (lane & 15);
                    const bool in = r < po.rows_left && c < po.cols_left;
                    left[q] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                        po.rs, in ? (r * po.ld + c) * 4 : OOB, 0, 0));
                }
            }
            acc[fm][fn] = left + acc[fm][fn];
        }
}

template <class T, int STAGES, int CPS, int EPI, bool PARK, bool WT>
__global__ __launch_bounds__(T::THREADS) void lds_gemm_kernel(GemmArgs g)
{
    constexpr int BM = T::BM, BN = T::BN, TM = T::TM, TN = T::TN, FM = T::FM, FN = T::FN;
    constexpr int LOADS_A = T::LOADS_A, LOADS_B = T::LOADS_B;
    constexpr int A_BYTES = T::A_BYTES, STAGE_BYTES = T::STAGE_BYTES;
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    constexpr int LOG = Log2<CPS>::value;
    constexpr int REG_LEVELS = PARK ? LOG - 1 : LOG;
    constexpr int NSTK = REG_LEVELS > 0 ? REG_LEVELS : 1;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / T::WAVES_N, wn = wave % T::WAVES_N;
    const TileCoord tc = tile_coord(g, BM, BN);
    const int row0 = tc.row0, col0 = tc.col0;
    const int wrow0 = row0 + wm * TM, wcol0 = col0 + wn * TN;
    // a wave whose whole block lies past M or N skips the MFMAs
    const bool active = (wrow0 < g.M) && (wcol0 < g.N);

    // Buffer descriptors over the tile's rows of X and columns of W.  Reads
    // past the record count return zeros (rows >= M, the last row's
    // columns >= N).
    // With W transposed the descriptor covers the tile's rows of W (columns
    // >= N read zeros, like rows >= M of X).
    const int rows_valid = (g.M - row0) < BM ? (g.M - row0) : BM;
    const int cols_valid = (g.N - col0) < BN ? (g.N - col0) : BN;
    const uint16_t* xa = g.X + (size_t)row0 * g.ldx;
    const uint16_t* wb = WT ? g.W + (size_t)col0 * g.ldw : g.W + col0;
    const uint32_t a_bytes = (uint32_t)(((size_t)(rows_valid - 1) * g.ldx + g.K) * 2);
    const uint32_t b_bytes =
        WT ? (uint32_t)(((size_t)(cols_valid - 1) * g.ldw + g.K) * 2)
           : (uint32_t)(((size_t)(g.K - 1) * g.ldw + (g.N - col0)) * 2);
    const i32x4 ra = buffer_desc(xa, a_bytes);
    const i32x4 rb = buffer_desc(wb, b_bytes);
    const uint32_t smem_lds = (uint32_t)(uintptr_t)((DETRED_LDS uint8_t*)smem);

    // Per-lane byte offsets of its LOADS_A chunks of A and LOADS_B chunks of
    // B inside a block; a wave's load i fills 16-byte slots
    // (wave * LOADS + i) * 64 + lane of the block.
    uint32_t offa[LOADS_A], offb[LOADS_B];
#pragma unroll
    for (int i = 0; i < LOADS_A; ++i) {
        const int s = (wave * LOADS_A + i) * 64 + lane;
        const int r = s >> 3, ca = (s & 7) ^ (r & 7);       // A: row r, k-chunk ca
        offa[i] = (uint32_t)((r * g.ldx + 8 * ca) * 2);
    }
#pragma unroll
    for (int i = 0; i < LOADS_B; ++i) {
        const int s = (wave * LOADS_B + i) * 64 + lane;
        if (WT) {
            const int n = s >> 3, cn = (s & 7) ^ (n & 7);  // B: row n, k-chunk cn
            offb[i] = (uint32_t)((n * g.ldw + 8 * cn) * 2);
        } else {
            const int k = s / T::B_ROW_CHUNKS;              // B: k-row k, n-chunk cb
            const int cb = (s % T::B_ROW_CHUNKS) ^ b_swz(k);
            offb[i] = (uint32_t)((k * g.ldw + 8 * cb) * 2);
        }
    }

    const int kslice = tc.z * CPS * g.Kc;
    const int nb = (g.Kc + BK - 1) / BK;
    const int total = CPS * nb;
    const uint32_t ldw_bytes = (uint32_t)g.ldw * 2;

    auto block_k = [&](int t) { return kslice + (t / nb) * g.Kc + (t % nb) * BK; };
    // LDS load of block t into stage buffer t % STAGES: LOADS_PER_ISSUE
    // vector-memory loads per lane.
    auto issue = [&](int t) {
        const int kb = block_k(t);
        const uint32_t st = smem_lds + (uint32_t)((t % STAGES) * STAGE_BYTES);
#pragma unroll
        for (int i = 0; i < LOADS_A; ++i)
            dma16(st + (uint32_t)((wave * LOADS_A + i) * 1024), offa[i] + (uint32_t)kb * 2, ra);
#pragma unroll
        for (int i = 0; i < LOADS_B; ++i)
            dma16(st + (uint32_t)(A_BYTES + (wave * LOADS_B + i) * 1024),
                  offb[i] + (WT ? (uint32_t)kb * 2 : (uint32_t)kb * ldw_bytes), rb);
    };
    constexpr int LOADS_PER_ISSUE = LOADS_A + LOADS_B;

    // Fragment addresses inside a stage.  A: row r = wm*TM + fm*16 + lane%16,
    // k-chunk 4*ks + lane/16, swizzled by r%8 (= lane%8).  B: lane j of each
    // 16-lane group addresses k-row k0 + j/4 (k0 = 32ks + 8g + 4q) at
    // columns 4*(j%4) .. +3 of 16-column tile fn.
    const int gq = lane >> 4, j = lane & 15;
    uint32_t a_addr[KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
        const int r = wm * TM + j;
        a_addr[ks] = (uint32_t)((r * 8 + ((4 * ks + gq) ^ (lane & 7))) * 16);
    }
    // transposed W: row n = wn*TN + fn*16 + lane%16, k-chunk as for A
    uint32_t bt_addr[KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
        const int n = wn * TN + j;
        bt_addr[ks] = (uint32_t)((n * 8 + ((4 * ks + gq) ^ (lane & 7))) * 16);
    }
    uint32_t b_addr[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
        const int rr = j >> 2, p = j & 3;
        const int k = 8 * gq + rr;                          // + 32ks + 4q added below
        const int n = wn * TN + fn * 16 + 4 * p;
        const int chunk = (n >> 3) ^ (2 * (rr + 4 * (gq & 1)));
        b_addr[fn] = (uint32_t)(A_BYTES + (k * T::B_ROW_CHUNKS + chunk) * 16 + ((n >> 2) & 1) * 8);
    }

    f32x4 acc[FM][FN];
    f32x4 stk[NSTK][FM][FN];
    f32x4* lds_top = reinterpret_cast<f32x4*>(smem + STAGES * STAGE_BYTES) +
                     wave * (FM * FN * 64) + lane;

    // Software pipeline over the K blocks of the slice.  Iteration t:
    //   first half:  MFMAs of block t, step 0 (fragments read earlier)
    //                while step 1's fragments are read from stage t;
    //   then:        every wave is done with stage t (lgkmcnt 0), block
    //                t+1's loads are complete (vmcnt), barrier, and block
    //                t+STAGES starts loading into stage t's buffer;
    //   second half: MFMAs of block t, step 1 while step 0's fragments of
    //                block t+1 are read.
    // The MFMA order along k is unchanged: step 0 then step 1 of each block.
#pragma unroll
    for (int p = 0; p < STAGES; ++p)
        if (p < total)
            issue(p);
    if (STAGES - 1 < total)
        wait_vmcnt<(STAGES - 1) * LOADS_PER_ISSUE>();
    else
        wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);

    bf16x8 fa0[FM], fb0[FN], fa1[FM], fb1[FN];
    auto frags = [&](bf16x8(&af)[FM], bf16x8(&bfr)[FN], const uint8_t* st, int ks) {
        if constexpr (WT)
            load_frags_wt<T>(af, bfr, st, a_addr[ks], bt_addr[ks]);
        else
            load_frags<T>(af, bfr, st, a_addr[ks], b_addr, ks);
    };
    if (active)
        frags(fa0, fb0, smem, 0);

#pragma unroll
    for (int c = 0; c < CPS; ++c) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                acc[fm][fn] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int cend = kslice + (c + 1) * g.Kc;
        for (int b = 0; b < nb; ++b) {
            const int t = c * nb + b;
            const int kb = block_k(t);
            const bool two_steps = (cend - kb) > 32;
            const uint8_t* st = smem + (t % STAGES) * STAGE_BYTES;
            const uint8_t* st_next = smem + ((t + 1) % STAGES) * STAGE_BYTES;
            __builtin_amdgcn_sched_barrier(0);
            if (active) {
                frags(fa1, fb1, st, 1);
                mma_step<T>(acc, fa0, fb0);
                interleave_reads_with_mfma<T, WT>();
            }
            __builtin_amdgcn_sched_barrier(0);
            wait_lgkmcnt0();
            if (t + STAGES - 1 < total)
                wait_vmcnt<(STAGES - 2) * LOADS_PER_ISSUE>();
            else
                wait_vmcnt<0>();
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            if (t + STAGES < total)
                issue(t + STAGES);
            __builtin_amdgcn_sched_barrier(0);
            if (active) {
                // the next block's reads are harmless after the last block
                if (two_steps) {
                    frags(fa0, fb0, st_next, 0);
                    mma_step<T>(acc, fa1, fb1);
                    interleave_reads_with_mfma<T, WT>();
                } else {
                    frags(fa0, fb0, st_next, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        fold_chunk<FM, FN, LOG, REG_LEVELS, NSTK>(c, acc, stk, lds_top);
    }
    if constexpr (EPI == EPI_ATOMIC) {
        store_tile<FM, FN>(acc, g.Y, g.ldy, g.M, g.N, wrow0, wcol0, lane, true);
    } else {
        // EPI_STORE: the final product, or slice tc.z's subtree root in its
        // own plane (out_z_stride)
        float* out = g.Y + (size_t)tc.z * g.out_z_stride;
        if constexpr (T::BM == 256 && T::BN == 256) {
            // the root tile: plain roots only, never an addmm epilogue (the
            // direct form only with a row-major W: beside the transposed
            // operand's addressing it would not fit the registers)
            if constexpr (!WT) {
                if (g.direct_roots) {
                    store_roots_direct<T>(acc, out, g.ldy, g.M, g.N, wrow0, wcol0, lane);
                    return;
                }
            }
            store_tile_via_lds<T, STAGES, false>(acc, g, out, g.ldy, row0, col0, wm, wn, lane,
                                                 tid, smem);
        } else {
            store_tile_via_lds<T, STAGES>(acc, g, out, g.ldy, row0, col0, wm, wn, lane, tid, smem);
        }
    }
}

// Eight-chunk product on the 192x128 tile (TileW).  The same chunk chains
// and tree as lds_gemm_kernel, arranged for the larger wave tile:
//  * one MFMA target (acc) and two saved subtree levels (keep0, keep1):
//    after chunk c the running value is added to the saved left siblings
//    and saved, the binary counter of fold_chunk written out for eight
//    chunks, with level 2 ((c0+c1)+(c2+c3)) parked in the output tile
//    (ParkOut) from chunk 3 to chunk 7; each chunk has a K loop of its own;
//  * A fragments rolled: the register of row fm takes the next k step's row
//    fm right after its last MFMA of this step; B fragments double-buffered;
//  * the LDS-DMA loads take their wave-uniform offset in a scalar register,
//    so a lane keeps three offset registers instead of one per load;
//  * no per-wave activity test and two k steps in every block (Kc % 64 ==
//    0): the K loops have no branch around their MFMAs.
template <class T, int STAGES, bool WT>
__global__ __launch_bounds__(T::THREADS) void wide_gemm_kernel(GemmArgs g)
{
    constexpr int BM = T::BM, BN = T::BN, TM = T::TM, TN = T::TN, FM = T::FM, FN = T::FN;
    constexpr int LOADS_A = T::LOADS_A, LOADS_B = T::LOADS_B;
    constexpr int A_BYTES = T::A_BYTES, STAGE_BYTES = T::STAGE_BYTES;
    constexpr int CPS = 8;
    static_assert(FN <= FM, "B fragment reads ride on the first FN rows");
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / T::WAVES_N, wn = wave % T::WAVES_N;
    const TileCoord tc = tile_coord(g, BM, BN);
    const int row0 = tc.row0, col0 = tc.col0;

    const int rows_valid = (g.M - row0) < BM ? (g.M - row0) : BM;
    const int cols_valid = (g.N - col0) < BN ? (g.N - col0) : BN;
    const uint16_t* xa = g.X + (size_t)row0 * g.ldx;
    const uint16_t* wb = WT ? g.W + (size_t)col0 * g.ldw : g.W + col0;
    const uint32_t a_bytes = (uint32_t)(((size_t)(rows_valid - 1) * g.ldx + g.K) * 2);
    const uint32_t b_bytes =
        WT ? (uint32_t)(((size_t)(cols_valid - 1) * g.ldw + g.K) * 2)
           : (uint32_t)(((size_t)(g.K - 1) * g.ldw + (g.N - col0)) * 2);
    const i32x4 ra = buffer_desc(xa, a_bytes);
    const i32x4 rb = buffer_desc(wb, b_bytes);
    const uint32_t smem_lds = (uint32_t)(uintptr_t)((DETRED_LDS uint8_t*)smem);

    // Per-lane load offsets, as in lds_gemm_kernel, split into a per-lane
    // part (in at most three registers) and a wave-uniform part passed as
    // the scalar offset.  Load i of wave w fills 16-byte slots
    // (w*LOADS + i)*64 + lane of the block:
    //  A (and a transposed W): row (w*LOADS + i)*8 + lane/8, 16-byte chunk
    //    (lane%8) ^ ((lane/8)%8) -- the row's low three bits come from lane;
    //  W: k-row (w*LOADS_B + i)*4 + lane/16, chunk (lane%16) ^ b_swz(k), whose
    //    bit ((w*LOADS_B + i)/2)%2 (wave-uniform) picks one of two per-lane
    //    parts.
    static_assert(T::B_ROW_CHUNKS == 16 && LOADS_B % 2 == 0, "B layout of the 128-wide tile");
    const uint32_t va = (uint32_t)((((lane >> 3) * g.ldx) + 8 * ((lane & 7) ^ ((lane >> 3) & 7))) * 2);
    uint32_t vb0, vb1;
    if constexpr (WT) {
        vb0 = vb1 = (uint32_t)((((lane >> 3) * g.ldw) + 8 * ((lane & 7) ^ ((lane >> 3) & 7))) * 2);
    } else {
        const int q = lane >> 4;
        vb0 = (uint32_t)((q * g.ldw + 8 * ((lane & 15) ^ (2 * q))) * 2);
        vb1 = (uint32_t)((q * g.ldw + 8 * ((lane & 15) ^ (2 * (q + 4)))) * 2);
    }
    const uint32_t lda_bytes = (uint32_t)g.ldx * 2, ldw_bytes = (uint32_t)g.ldw * 2;

    // one slice, chunks of a whole number of K blocks: block t starts at k = 64 t
    const int nb = g.Kc / BK;
    const int total = CPS * nb;
    auto issue = [&](int t) {
        const uint32_t kb = (uint32_t)(t * BK);
        const uint32_t st = smem_lds + (uint32_t)((t % STAGES) * STAGE_BYTES);
#pragma unroll
        for (int i = 0; i < LOADS_A; ++i)
            dma16s(st + (uint32_t)((wave * LOADS_A + i) * 1024), va,
                   (uint32_t)((wave * LOADS_A + i) * 8) * lda_bytes + kb * 2, ra);
#pragma unroll
        for (int i = 0; i < LOADS_B; ++i) {
            const uint32_t so =
                WT ? (uint32_t)((wave * LOADS_B + i) * 8) * ldw_bytes + kb * 2
                   : ((uint32_t)((wave * LOADS_B + i) * 4) + kb) * ldw_bytes;
            dma16s(st + (uint32_t)(A_BYTES + (wave * LOADS_B + i) * 1024),
                   (((wave * LOADS_B + i) >> 1) & 1) ? vb1 : vb0, so, rb);
        }
    };
    constexpr int LOADS_PER_ISSUE = LOADS_A + LOADS_B;

    // fragment addresses inside a stage, as in lds_gemm_kernel
    const int gq = lane >> 4, j = lane & 15;
    uint32_t a_addr[KSTEPS], bt_addr[KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
        a_addr[ks] = (uint32_t)(((wm * TM + j) * 8 + ((4 * ks + gq) ^ (lane & 7))) * 16);
        bt_addr[ks] = (uint32_t)(A_BYTES + ((wn * TN + j) * 8 + ((4 * ks + gq) ^ (lane & 7))) * 16);
    }
    uint32_t b_addr[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
        const int rr = j >> 2, p = j & 3;
        const int k = 8 * gq + rr;
        const int n = wn * TN + fn * 16 + 4 * p;
        const int chunk = (n >> 3) ^ (2 * (rr + 4 * (gq & 1)));
        b_addr[fn] = (uint32_t)(A_BYTES + (k * T::B_ROW_CHUNKS + chunk) * 16 + ((n >> 2) & 1) * 8);
    }
    constexpr int ROW = BN * 2;  // bytes per k-row of a [k][n] B block
    auto read_a = [&](const uint8_t* st, int ks, int fm) {
        return *reinterpret_cast<const bf16x8*>(st + a_addr[ks] + fm * 16 * 8 * 16);
    };
    auto read_b = [&](const uint8_t* st, int ks, int fn) {
        if constexpr (WT) {
            return *reinterpret_cast<const bf16x8*>(st + bt_addr[ks] + fn * 16 * 8 * 16);
        } else {
            const uint8_t* pb = st + b_addr[fn] + ks * 32 * ROW;
            const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DETRED_LDS v4i16*)(pb));
            const v4i16 hi =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16((DETRED_LDS v4i16*)(pb + 4 * ROW));
            return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
    };
    // One k step: the MFMAs of the fragments in af/bc, row by row; after row
    // fm, af[fm] takes row fm of the next step (st_n, ks_n) and, for the
    // first FN rows, bn[fm] column fm.
    auto row = [&](f32x4(&acc)[FM][FN], bf16x8(&af)[FM], const bf16x8(&bc)[FN], int fm) {
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
            acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[fm], bc[fn], acc[fm][fn], 0,
                                                                  0, 0);
    };
    auto kstep = [&](f32x4(&acc)[FM][FN], bf16x8(&af)[FM], const bf16x8(&bc)[FN],
                     bf16x8(&bn)[FN], const uint8_t* st_n, int ks_n) {
        // rows with a B column read beside the A row (WT: 2 reads, else 3
        // with the two transposed halves), then rows with the A read only;
        // each row's MFMAs are issued before its reads
#pragma unroll
        for (int fm = 0; fm < FN; ++fm) {
            row(acc, af, bc, fm);
            af[fm] = read_a(st_n, ks_n, fm);
            bn[fm] = read_b(st_n, ks_n, fm);
            __builtin_amdgcn_sched_group_barrier(0x008, FN, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, WT ? 2 : 3, 0);
        }
#pragma unroll
        for (int fm = FN; fm < FM; ++fm) {
            row(acc, af, bc, fm);
            af[fm] = read_a(st_n, ks_n, fm);
            __builtin_amdgcn_sched_group_barrier(0x008, FN, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
    };

    ParkOut<T> po;
    po.rs = __builtin_amdgcn_make_buffer_rsrc(g.Y + (size_t)row0 * g.ldy + col0, 0, 0x7fffffff,
                                              RAW_BUFFER_FLAGS);
    po.full = (row0 + BM <= g.M) && (col0 + BN <= g.N);
    po.ld = (int)g.ldy;
    po.rows_left = g.M - row0;
    po.cols_left = g.N - col0;
    po.wave = wave;
    po.wrow = wm * TM;
    po.wcol = wn * TN;

    // acc: the MFMA target of every chunk; keep0, keep1: the saved subtree
    // levels below the parked one
    f32x4 acc[FM][FN], keep0[FM][FN], keep1[FM][FN];
#pragma unroll
    for (int p = 0; p < STAGES; ++p)
        if (p < total)
            issue(p);
    if (STAGES - 1 < total)
        wait_vmcnt<(STAGES - 1) * LOADS_PER_ISSUE>();
    else
        wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);

    // Every wave runs its MFMAs, also one whose rows or columns lie wholly
    // past M or N (edge tiles): its operands read as zeros and its results
    // are dropped by the stores' range checks, and the loop has no branch.
    bf16x8 af[FM], b0[FN], b1[FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
        af[fm] = read_a(smem, 0, fm);
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
        b0[fn] = read_b(smem, 0, fn);

    auto zero = [&](f32x4(&v)[FM][FN]) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                v[fm][fn] = f32x4{0.f, 0.f, 0.f, 0.f};
    };
    // acc = left + acc, element by element (the node's left operand first)
    auto add_left = [&](const f32x4(&left)[FM][FN]) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                acc[fm][fn] = left[fm][fn] + acc[fm][fn];
    };
    auto keep = [&](f32x4(&dst)[FM][FN]) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
                dst[fm][fn] = acc[fm][fn];
    };

    // Read-back of the parked level on a full tile: each wave's FM*FN
    // 16-byte slots per lane (one per accumulator, slot i = fm*FN + fn) are
    // loaded by LDS-DMA into the stage buffers that the last blocks free,
    // while those blocks are still multiplied: the first PARK_A slots into
    // stage 0 after block total-4, the next PARK_A into stage 1 after
    // total-3, the rest into stage 2 after total-2 (total = 8 nb, so block
    // total-4 sat in stage 0).  Each lane loads only the slots it stored
    // itself, so its own vmcnt is the only wait; a wave's region in stage p
    // is PARK_A (p < 2) or PARK_C slots wide.
    constexpr int SLOTS = FM * FN;
    constexpr int PARK_A = STAGE_BYTES / 1024 / T::WAVES, PARK_C = SLOTS - 2 * PARK_A;
    static_assert(STAGE_BYTES % (1024 * T::WAVES) == 0 && PARK_C >= 0 && PARK_C <= PARK_A &&
                      STAGES == 4,
                  "park read-back layout of the 192x128 tile");
    auto park_lds = [&](int i) -> uint32_t {
        const int p = i < PARK_A ? 0 : (i < 2 * PARK_A ? 1 : 2);
        const int k = i - PARK_A * p;
        return (uint32_t)(p * STAGE_BYTES + (wave * (p < 2 ? PARK_A : PARK_C) + k) * 1024);
    };
    const uint32_t ldy_bytes = (uint32_t)g.ldy * 4;
    auto park_part = [&](int first, int count) {
        // slot i covers tile rows 2(SLOTS wave + i) and the next, 16 bytes a lane
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const uint32_t pv = (uint32_t)(ln >> 5) * ldy_bytes + (uint32_t)(ln & 31) * 16;
        for (int k = 0; k < count; ++k) {
            const int i = first + k;
            dma16r(smem_lds + park_lds(i), pv, (uint32_t)((wave * SLOTS + i) * 2) * ldy_bytes, po.rs);
        }
    };
    const bool pf = po.full;

    // chunk c into acc: its MFMA chain from +0 over the chunk's K blocks
    // (every block holds two k steps: Kc % 64 == 0 on this tile).  The
    // vmcnt waits before each barrier admit exactly the loads issued after
    // block t+1: two blocks in the steady state, then the last block and
    // the read-back parts already in flight.
    auto chunk = [&](int c) {
        zero(acc);
        for (int b = 0; b < nb; ++b) {
            const int t = c * nb + b;
            const uint8_t* st = smem + (t % STAGES) * STAGE_BYTES;
            const uint8_t* st_next = smem + ((t + 1) % STAGES) * STAGE_BYTES;
            __builtin_amdgcn_sched_barrier(0);
            kstep(acc, af, b0, b1, st, 1);
            __builtin_amdgcn_sched_barrier(0);
            wait_lgkmcnt0();
            if (t + STAGES - 1 < total) {
                wait_vmcnt<(STAGES - 2) * LOADS_PER_ISSUE>();
            } else if (t == total - 3) {
                if (pf)
                    wait_vmcnt<LOADS_PER_ISSUE + PARK_A>();
                else
                    wait_vmcnt<LOADS_PER_ISSUE>();
            } else if (t == total - 2) {
                if (pf)
                    wait_vmcnt<2 * PARK_A>();
                else
                    wait_vmcnt<0>();
            }
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            if (t + STAGES < total) {
                issue(t + STAGES);
            } else if (pf) {
                if (t == total - 4)
                    park_part(0, PARK_A);
                else if (t == total - 3)
                    park_part(PARK_A, PARK_A);
                else if (t == total - 2)
                    park_part(2 * PARK_A, PARK_C);
            }
            __builtin_amdgcn_sched_barrier(0);
            // the next block's reads are harmless after the last block
            kstep(acc, af, b1, b0, st_next, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    chunk(0);
    keep(keep0);                     // c0
    chunk(1);
    add_left(keep0);                 // c0 + c1
    keep(keep1);
    chunk(2);
    keep(keep0);                     // c2
    chunk(3);
    add_left(keep0);                 // c2 + c3
    add_left(keep1);                 // (c0 + c1) + (c2 + c3)
    __builtin_amdgcn_sched_barrier(0);
    park_out_store<T>(po, acc, lane);
    chunk(4);
    keep(keep0);                     // c4
    chunk(5);
    add_left(keep0);                 // c4 + c5
    keep(keep1);
    chunk(6);
    keep(keep0);                     // c6
    chunk(7);
    // chunk 7
    add_left(keep0);                 // c6 + c7
    add_left(keep1);                 // (c4 + c5) + (c6 + c7)
    __builtin_amdgcn_sched_barrier(0);
    // the left half + the right half
    if (pf) {
        wait_vmcnt<0>();
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const f32x4 left =
                    *reinterpret_cast<const f32x4*>(smem + park_lds(fm * FN + fn) + lane * 16);
                acc[fm][fn] = left + acc[fm][fn];
            }
    } else {
        park_out_add<T>(po, acc, lane);
    }

    // the final product through the stage buffers (addmm epilogue on the way)
    store_tile_via_lds<T, STAGES>(acc, g, g.Y, (int)g.ldy, row0, col0, wm, wn, lane, tid, smem);
}

template <bool WT>
hipError_t launch_wide(const GemmArgs& g, hipStream_t s)
{
    // four stages fill the 160 KiB of LDS (3 -> 4 on MI355X: 4096x14336x4096
    // 637 -> 621 us, 1024 rows 201 -> 195 us; three weight blocks in flight)
    constexpr int ST = 4;
    auto fn = wide_gemm_kernel<TileW, ST, WT>;
    constexpr int bytes = ST * TileW::STAGE_BYTES;
    static_assert(bytes <= 160 * 1024, "LDS of one workgroup");
    static std::atomic<unsigned long long> lds_set{0};
    const hipError_t attr = ensure_lds_limit(lds_set, reinterpret_cast<const void*>(fn), bytes);
    if (attr != hipSuccess)
        return attr;
    const unsigned grid = (unsigned)(g.tiles_m * g.tiles_n * g.slices);
    hipLaunchKernelGGL(fn, dim3(grid), dim3(TileW::THREADS), bytes, s, g);
    return hipGetLastError();
}

// Stage counts.  With 8 chunks per slice the top subtree level is parked in
// LDS where four copies of a wave's accumulators would not fit in registers,
// beside three stages (see the measurements at launch()).  Otherwise the
// depth follows the grid: a grid of at most 256 workgroups leaves one per
// CU, and four stages keep three weight blocks in flight (weights from HBM:
// 256x4096x4096 at 4 slices 32.0 -> 28.8 us, 256x4096x14336 69.5 -> 54.6
// us, 1024x1024x8192 48.6 -> 40.7 us on MI355X); a larger grid keeps two,
// so that two workgroups share each CU (512x4096x4096 at 4 slices: 42 us
// with two stages, 54 with four), unless the kernel's registers leave room
// for only one workgroup per CU anyway (four chunks per slice on 128x128):
// then it takes four (1024x8192x8192 at 2 slices, weights from HBM: 266 ->
// 217 us).
template <class T, int CPS>
struct Stages {
    static constexpr bool park = (CPS == 8) && (T::FM * T::FN >= 8);
    static constexpr int shallow = park ? 3 : 2;
    static constexpr int deep =
        (!park && 4 * T::STAGE_BYTES + 16 <= 160 * 1024) ? 4 : shallow;
};

template <class T, int ST, int CPS, int EPI, bool WT>
hipError_t launch_st(const GemmArgs& g, hipStream_t s)
{
    constexpr bool PK = Stages<T, CPS>::park;
    auto fn = lds_gemm_kernel<T, ST, CPS, EPI, PK, WT>;
    // + the last-arriver flag of a combine (never with 8 chunks per slice)
    constexpr int bytes = ST * T::STAGE_BYTES + (PK ? T::PARK_BYTES : 0);
    static_assert(bytes <= 160 * 1024, "LDS of one workgroup");
    static std::atomic<unsigned long long> lds_set{0};
    const hipError_t attr = ensure_lds_limit(lds_set, reinterpret_cast<const void*>(fn), bytes);
    if (attr != hipSuccess)
        return attr;
    const unsigned grid = (unsigned)(g.tiles_m * g.tiles_n * g.slices);
    hipLaunchKernelGGL(fn, dim3(grid), dim3(T::THREADS), bytes, s, g);
    return hipGetLastError();
}

// Eight-chunk slices (parked level, 96 + 64 KiB) keep three stages: two
// weight blocks in flight per workgroup, which is what a product whose
// weights come from HBM needs (256x14336x4096 with the weights not cached:
// 67.5 -> 53.4 us, 1024 rows 234 -> 185 us on MI355X), at a few percent on
// repeated calls whose weights stay in the MALL.
template <class T, int CPS, int EPI, bool WT>
hipError_t launch(const GemmArgs& g, hipStream_t s)
{
    using St = Stages<T, CPS>;
    if constexpr (St::deep != St::shallow) {
        // Deep also where a CU holds only one workgroup of the shallow form
        // anyway (its registers allow no second one): the extra stages then
        // cost no occupancy.
        static const int per_cu = [] {
            constexpr bool PK = St::park;
            constexpr int bytes = St::shallow * T::STAGE_BYTES + (PK ? T::PARK_BYTES : 0);
            int n = 0;
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
                    &n, lds_gemm_kernel<T, St::shallow, CPS, EPI, PK, WT>, T::THREADS, bytes) !=
                hipSuccess)
                n = 0;
            return n;
        }();
        const long wgs = (long)g.tiles_m * g.tiles_n * g.slices;
        if (wgs <= 256 || per_cu == 1)
            return launch_st<T, St::deep, CPS, EPI, WT>(g, s);
    }
    return launch_st<T, St::shallow, CPS, EPI, WT>(g, s);
}

// T1: the tile of one-chunk slices; T: the tile of the others.
template <class T1, class T, int EPI, bool WT>
hipError_t launch_cps(const GemmArgs& g, int cps, hipStream_t s)
{
    switch (cps) {
    case 1: return launch<T1, 1, EPI, WT>(g, s);
    case 2: return launch<T, 2, EPI, WT>(g, s);
    case 4: return launch<T, 4, EPI, WT>(g, s);
    case 8: return launch<T, 8, EPI, WT>(g, s);
    }
    return hipErrorInvalidValue;
}

template <int EPI>
hipError_t launch_layout(int tile, const GemmArgs& g, int cps, hipStream_t s)
{
    if (tile == TILE_L256) {
        // one-chunk slices writing their roots (shards) only
        if (cps != 1 || EPI != EPI_STORE)
            return hipErrorInvalidValue;
        if constexpr (EPI == EPI_STORE)
            return g.wt ? launch<Tile256, 1, EPI, true>(g, s) : launch<Tile256, 1, EPI, false>(g, s);
    }
    if (tile == TILE_W256) {
        // eight-chunk workgroups writing the final product only
        if (cps != 8 || EPI != EPI_STORE)
            return hipErrorInvalidValue;
        if constexpr (EPI == EPI_STORE)
            return g.wt ? launch_wide<true>(g, s) : launch_wide<false>(g, s);
    }
    if (tile == TILE_D64)
        return g.wt ? launch_cps<TileD64, TileD64, EPI, true>(g, cps, s)
                    : launch_cps<TileD64, TileD64, EPI, false>(g, cps, s);
    using T1 = std::conditional_t<EPI == EPI_STORE, Tile128x4, Tile128>;
    return g.wt ? launch_cps<T1, Tile128, EPI, true>(g, cps, s)
                : launch_cps<T1, Tile128, EPI, false>(g, cps, s);
}

}  // namespace lds

bool lds_engine_supports(int tile, const GemmArgs& g, int cps)
{
    // every MFMA step inside K, and byte offsets of the tile's X rows, W
    // columns and output rows within the 31-bit record range of a buffer
    // descriptor; the 256x256 tile for one-chunk slices only
    if (g.Kc % 32 != 0 ||
        (tile != TILE_L128 && tile != TILE_L256 && tile != TILE_D64 && tile != TILE_W256))
        return false;
    if (tile == TILE_L256 && cps != 1)
        return false;
    // the output-parked tile: eight chunks, a final fp32 output that the
    // park may use (not slice roots, not bf16)
    if (tile == TILE_W256 &&
        (cps != 8 || g.Kc % 64 != 0 || g.out_z_stride != 0 || (g.epi && g.out_bf16)))
        return false;
    const size_t BM = tile == TILE_L256 ? lds::Tile256::BM
                      : tile == TILE_W256 ? lds::TileW::BM
                      : tile == TILE_D64 ? lds::TileD64::BM : lds::Tile128::BM;
    const size_t BN = tile == TILE_L256 ? lds::Tile256::BN
                      : tile == TILE_W256 ? lds::TileW::BN
                      : tile == TILE_D64 ? lds::TileD64::BN : lds::Tile128::BN;
    const size_t xbytes = ((BM - 1) * g.ldx + g.K) * 2;
    const size_t wbytes = g.wt ? ((BN - 1) * g.ldw + g.K) * 2 : ((size_t)g.K * g.ldw) * 2;
    // output rows of the tile (Y at ldy, partial planes at N, C at ldc)
    // likewise
    size_t ld = (size_t)(g.ldy > g.N ? g.ldy : g.N);
    if (g.epi && g.C && (size_t)g.ldc > ld)
        ld = (size_t)g.ldc;
    const size_t ybytes = ((BM - 1) * ld + BN) * 4;
    return xbytes < 0x7fffffffu && wbytes < 0x7fffffffu && ybytes < 0x7fffffffu;
}

hipError_t launch_lds_gemm(int tile, int epi, const GemmArgs& g, int cps, hipStream_t s)
{
    switch (epi) {
    case EPI_STORE: return lds::launch_layout<EPI_STORE>(tile, g, cps, s);
    case EPI_ATOMIC: return lds::launch_layout<EPI_ATOMIC>(tile, g, cps, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace detred
