// Register-staged slice GEMM engine for gfx950 (every tile shape and every
// K, including one-chunk K with a zero-padded last MFMA step), plus the tree
// combine, zero fill and bf16 cast kernels the GEMM entry points need.
// The reduction order and the epilogues are shared with the LDS-DMA engine
// through gemm_common.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_common.h"

namespace detred {

// Workgroup tile description.  Waves form a WAVES_M x WAVES_N grid; each
// wave owns a (BM/WAVES_M) x (BN/WAVES_N) block of 16x16 MFMA tiles.  K is
// staged through LDS in BK-wide blocks.  In LDS, A is kept [m][k] and B
// transposed to [n][k] so that both MFMA operands are read as 16 contiguous
// bytes per lane.
template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int BK_>
struct Tile {
    static constexpr int BM = BM_, BN = BN_, BK = BK_;
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
    static constexpr int WAVES = WAVES_M * WAVES_N;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int TM = BM / WAVES_M, TN = BN / WAVES_N;
    static constexpr int FM = TM / 16, FN = TN / 16;
    static constexpr int KSTEPS = BK / 32;
    static constexpr int LDK = BK + 8;  // LDS row length in bf16 (16-byte pad)
    static constexpr int A_ELEMS = BM * LDK, B_ELEMS = BN * LDK;
    static constexpr int STAGE_ELEMS = A_ELEMS + B_ELEMS;
    static constexpr int LDS_BYTES = 2 * STAGE_ELEMS * 2;
    static constexpr int A_VECS = BM * BK / 8;             // 16-byte vectors
    static constexpr int A_PER_THREAD = (A_VECS + THREADS - 1) / THREADS;
    static constexpr int B_SUBS = (BK / 4) * (BN / 8);     // 4k x 8n blocks
    static constexpr int B_PER_THREAD = (B_SUBS + THREADS - 1) / THREADS;
    static constexpr int BT_VECS = BN * BK / 8;            // transposed W: 16-byte vectors
    static constexpr int BT_PER_THREAD = (BT_VECS + THREADS - 1) / THREADS;
    static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be 16-aligned");
    static_assert(BK % 32 == 0, "K block must hold whole MFMA steps");
};

// The narrow tile stages 256-wide K blocks: a LoRA slice (512 k) is then
// two global-load round trips instead of eight (shrink at 8 slices, M = 1:
// 10.8 -> 8.0 us).  The block width never changes the bits.
using TileS16 = Tile<64, 16, 4, 1, 256>;
using TileM64 = Tile<64, 64, 2, 2, 64>;
using TileL128 = Tile<128, 128, 2, 2, 64>;


// Whether the top level of an 8-chunk subtree is parked in LDS (large wave
// tiles only, where four register copies of the accumulators do not fit).
template <class T, int CPS>
struct TopLevelInLds {
    static constexpr bool value = (CPS == 8) && (T::FM * T::FN >= 16);
};

template <class T, int CPS>
constexpr int lds_bytes()
{
    return T::LDS_BYTES + (TopLevelInLds<T, CPS>::value ? T::WAVES * T::FM * T::FN * 64 * 16 : 0);
}

// WT: W is given transposed ([N][K], K contiguous); its rows then load like
// the rows of X and go to LDS unchanged.
template <class T, bool WT>
struct Prefetch {
    uint4 a[T::A_PER_THREAD];
    uint4 b[WT ? T::BT_PER_THREAD : T::B_PER_THREAD][WT ? 1 : 4];
};

// Global -> registers for one K block [kb, kb+BK) clipped to the chunk end ce.
template <class T, bool WT>
__device__ __forceinline__ void load_block(Prefetch<T, WT>& pf, const GemmArgs& g,
                                           int row0, int col0, int kb, int ce, int tid)
{
#pragma unroll
    for (int i = 0; i < T::A_PER_THREAD; ++i) {
        const int v = tid + i * T::THREADS;
        uint4 val = make_uint4(0, 0, 0, 0);
        if (v < T::A_VECS) {
            const int r = v / (T::BK / 8), kv = v % (T::BK / 8);
            const int grow = row0 + r, gk = kb + 8 * kv;
            if (grow < g.M && gk < ce)
                val = *reinterpret_cast<const uint4*>(g.X + (size_t)grow * g.ldx + gk);
        }
        pf.a[i] = val;
    }
    if constexpr (WT) {
#pragma unroll
        for (int i = 0; i < T::BT_PER_THREAD; ++i) {
            const int v = tid + i * T::THREADS;
            uint4 val = make_uint4(0, 0, 0, 0);
            if (v < T::BT_VECS) {
                const int n = v / (T::BK / 8), kv = v % (T::BK / 8);
                const int gn = col0 + n, gk = kb + 8 * kv;
                if (gn < g.N && gk < ce)
                    val = *reinterpret_cast<const uint4*>(g.W + (size_t)gn * g.ldw + gk);
            }
            pf.b[i][0] = val;
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < T::B_PER_THREAD; ++i) {
        const int s = tid + i * T::THREADS;
        const int kq = s / (T::BN / 8), nq = s % (T::BN / 8);
        const int n = col0 + 8 * nq;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint4 val = make_uint4(0, 0, 0, 0);
            const int k = kb + 4 * kq + j;
            if (s < T::B_SUBS && k < ce && n < g.N)
                val = *reinterpret_cast<const uint4*>(g.W + (size_t)k * g.ldw + n);
            pf.b[i][j] = val;
        }
    }
}

// Registers -> LDS stage.  A is copied as is; each 4k x 8n block of B is
// transposed to 8 rows (one per n) of 4 consecutive k.
template <class T, bool WT>
__device__ __forceinline__ void store_block(const Prefetch<T, WT>& pf, uint16_t* stage, int tid)
{
    uint16_t* sA = stage;
    uint16_t* sB = stage + T::A_ELEMS;
#pragma unroll
    for (int i = 0; i < T::A_PER_THREAD; ++i) {
        const int v = tid + i * T::THREADS;
        if (v < T::A_VECS) {
            const int r = v / (T::BK / 8), kv = v % (T::BK / 8);
            *reinterpret_cast<uint4*>(sA + r * T::LDK + 8 * kv) = pf.a[i];
        }
    }
    if constexpr (WT) {
#pragma unroll
        for (int i = 0; i < T::BT_PER_THREAD; ++i) {
            const int v = tid + i * T::THREADS;
            if (v < T::BT_VECS) {
                const int n = v / (T::BK / 8), kv = v % (T::BK / 8);
                *reinterpret_cast<uint4*>(sB + n * T::LDK + 8 * kv) = pf.b[i][0];
            }
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < T::B_PER_THREAD; ++i) {
        const int s = tid + i * T::THREADS;
        if (s < T::B_SUBS) {
            const int kq = s / (T::BN / 8), nq = s % (T::BN / 8);
            const uint32_t r0[4] = {pf.b[i][0].x, pf.b[i][0].y, pf.b[i][0].z, pf.b[i][0].w};
            const uint32_t r1[4] = {pf.b[i][1].x, pf.b[i][1].y, pf.b[i][1].z, pf.b[i][1].w};
            const uint32_t r2[4] = {pf.b[i][2].x, pf.b[i][2].y, pf.b[i][2].z, pf.b[i][2].w};
            const uint32_t r3[4] = {pf.b[i][3].x, pf.b[i][3].y, pf.b[i][3].z, pf.b[i][3].w};
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                // column 2d: low halves; column 2d+1: high halves
                uint2 even, odd;
                even.x = (r0[d] & 0xffffu) | (r1[d] << 16);
                even.y = (r2[d] & 0xffffu) | (r3[d] << 16);
                odd.x = (r0[d] >> 16) | (r1[d] & 0xffff0000u);
                odd.y = (r2[d] >> 16) | (r3[d] & 0xffff0000u);
                *reinterpret_cast<uint2*>(sB + (8 * nq + 2 * d) * T::LDK + 4 * kq) = even;
                *reinterpret_cast<uint2*>(sB + (8 * nq + 2 * d + 1) * T::LDK + 4 * kq) = odd;
            }
        }
    }
}

// MFMA over the first nks 32-wide k steps of one LDS stage, increasing k.
// FULL: every 16x16 tile of the wave is inside M and N; otherwise tiles
// past fm_act / fn_act are skipped (rows and columns are independent, so
// skipping them never changes a kept element).
template <class T, bool FULL>
__device__ __forceinline__ void mma_block(f32x4 (&acc)[T::FM][T::FN], const uint16_t* stage,
                                          int nks, int wm, int wn, int lane,
                                          int fm_act, int fn_act)
{
    const uint16_t* sA = stage + (wm * T::TM + (lane & 15)) * T::LDK + 8 * (lane >> 4);
    const uint16_t* sB = stage + T::A_ELEMS + (wn * T::TN + (lane & 15)) * T::LDK + 8 * (lane >> 4);
#pragma unroll
    for (int ks = 0; ks < T::KSTEPS; ++ks) {
        if (ks < nks) {
            bf16x8 af[T::FM], bfr[T::FN];
#pragma unroll
            for (int fm = 0; fm < T::FM; ++fm)
                if (FULL || fm < fm_act)
                    af[fm] = *reinterpret_cast<const bf16x8*>(sA + fm * 16 * T::LDK + 32 * ks);
#pragma unroll
            for (int fn = 0; fn < T::FN; ++fn)
                if (FULL || fn < fn_act)
                    bfr[fn] = *reinterpret_cast<const bf16x8*>(sB + fn * 16 * T::LDK + 32 * ks);
#pragma unroll
            for (int fm = 0; fm < T::FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < T::FN; ++fn)
                    if (FULL || (fm < fm_act && fn < fn_act))
                        acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            af[fm], bfr[fn], acc[fm][fn], 0, 0, 0);
        }
    }
}

template <class T, int CPS, int EPI, bool WT>
__global__ __launch_bounds__(T::THREADS) void slice_gemm_kernel(GemmArgs g)
{
    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
    __shared__ int s_last;
    constexpr int LOG = Log2<CPS>::value;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / T::WAVES_N, wn = wave % T::WAVES_N;
    const TileCoord tc = tile_coord(g, T::BM, T::BN);
    const int row0 = tc.row0, col0 = tc.col0;

    const int wrow0 = row0 + wm * T::TM, wcol0 = col0 + wn * T::TN;
    int fm_act = (g.M - wrow0 + 15) / 16;
    fm_act = fm_act < 0 ? 0 : (fm_act > T::FM ? T::FM : fm_act);
    int fn_act = (g.N - wcol0 + 15) / 16;
    fn_act = fn_act < 0 ? 0 : (fn_act > T::FN ? T::FN : fn_act);
    const bool full = (fm_act == T::FM) && (fn_act == T::FN);

    const int kslice = tc.z * CPS * g.Kc;         // first k of this slice
    const int nb = (g.Kc + T::BK - 1) / T::BK;     // K blocks per chunk
    const int total = CPS * nb;

    f32x4 acc[T::FM][T::FN];
    // Subtree values waiting for their right sibling.  With 8 chunks per
    // slice and large wave tiles the top level (held from chunk 3 to chunk
    // 7) is parked in this wave's own LDS region, past the two stages.
    constexpr int REG_LEVELS = TopLevelInLds<T, CPS>::value ? LOG - 1 : LOG;
    constexpr int NSTK = REG_LEVELS > 0 ? REG_LEVELS : 1;
    f32x4 stk[NSTK][T::FM][T::FN];
    f32x4* lds_top = reinterpret_cast<f32x4*>(smem + 2 * T::STAGE_ELEMS) +
                     wave * (T::FM * T::FN * 64) + lane;
    Prefetch<T, WT> pf;

    load_block<T, WT>(pf, g, row0, col0, kslice, kslice + g.Kc, tid);
    store_block<T, WT>(pf, smem, tid);
    __syncthreads();

#pragma unroll
    for (int c = 0; c < CPS; ++c) {
#pragma unroll
        for (int fm = 0; fm < T::FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < T::FN; ++fn)
                acc[fm][fn] = f32x4{0.f, 0.f, 0.f, 0.f};

        const int cbeg = kslice + c * g.Kc, cend = cbeg + g.Kc;
        for (int b = 0; b < nb; ++b) {
            const int t = c * nb + b;
            const bool more = (t + 1 < total);
            if (more) {
                // next block: the following K block of this chunk, or the
                // first block of the next chunk
                const int nc = (b + 1 < nb) ? c : c + 1;
                const int nbi = (b + 1 < nb) ? b + 1 : 0;
                const int nbeg = kslice + nc * g.Kc;
                load_block<T, WT>(pf, g, row0, col0, nbeg + nbi * T::BK, nbeg + g.Kc, tid);
            }
            const int kb = cbeg + b * T::BK;
            int nks = (cend - kb + 31) / 32;
            nks = nks > T::KSTEPS ? T::KSTEPS : nks;
            const uint16_t* stage = smem + (t & 1) * T::STAGE_ELEMS;
            if (full)
                mma_block<T, true>(acc, stage, nks, wm, wn, lane, fm_act, fn_act);
            else if (fm_act > 0 && fn_act > 0)
                mma_block<T, false>(acc, stage, nks, wm, wn, lane, fm_act, fn_act);
            if (more)
                store_block<T, WT>(pf, smem + ((t + 1) & 1) * T::STAGE_ELEMS, tid);
            __syncthreads();
        }
        fold_chunk<T::FM, T::FN, LOG, REG_LEVELS, NSTK>(c, acc, stk, lds_top);
    }
    // acc now holds the root of this slice's subtree.
    finish_slice<T::BM, T::BN, T::THREADS, CPS, EPI>(acc, g, tc, wrow0, wcol0, lane, tid,
                                                     &s_last);
}

// Y[e] = fixed tree over count arrays (count in {1,2,4,8}); 4 elements per
// thread, grid-stride.
template <int COUNT>
__global__ __launch_bounds__(256) void tree_combine_kernel(const float* __restrict__ parts,
                                                           size_t stride,
                                                           float* __restrict__ Y, size_t n4)
{
    for (size_t v = (size_t)blockIdx.x * blockDim.x + threadIdx.x; v < n4;
         v += (size_t)gridDim.x * blockDim.x) {
        float4 vals[COUNT];
#pragma unroll
        for (int s = 0; s < COUNT; ++s)
            vals[s] = reinterpret_cast<const float4*>(parts + (size_t)s * stride)[v];
#pragma unroll
        for (int w = COUNT; w > 1; w >>= 1)
#pragma unroll
            for (int i = 0; i < (w >> 1); ++i) {
                vals[i].x = vals[2 * i].x + vals[2 * i + 1].x;
                vals[i].y = vals[2 * i].y + vals[2 * i + 1].y;
                vals[i].z = vals[2 * i].z + vals[2 * i + 1].z;
                vals[i].w = vals[2 * i].w + vals[2 * i + 1].w;
            }
        reinterpret_cast<float4*>(Y)[v] = vals[0];
    }
}

// The same tree into g.Y with its row stride and, when g.epi, the addmm
// epilogue (beta*C + alpha*p, fp32 or bf16) applied to the combined value:
// element (r, c) of each part plane at r*N + c; 4 columns per thread.
template <int COUNT>
__global__ __launch_bounds__(256) void tree_combine_rows_kernel(const float* __restrict__ parts,
                                                                size_t stride, GemmArgs g)
{
    const size_t per_row = (size_t)g.N / 4;
    const size_t total4 = per_row * (size_t)g.M;
    for (size_t v = (size_t)blockIdx.x * blockDim.x + threadIdx.x; v < total4;
         v += (size_t)gridDim.x * blockDim.x) {
        const size_t r = v / per_row, c = 4 * (v % per_row);
        float4 vals[COUNT];
#pragma unroll
        for (int s = 0; s < COUNT; ++s)
            vals[s] = *reinterpret_cast<const float4*>(parts + (size_t)s * stride + r * g.N + c);
#pragma unroll
        for (int w = COUNT; w > 1; w >>= 1)
#pragma unroll
            for (int i = 0; i < (w >> 1); ++i) {
                vals[i].x = vals[2 * i].x + vals[2 * i + 1].x;
                vals[i].y = vals[2 * i].y + vals[2 * i + 1].y;
                vals[i].z = vals[2 * i].z + vals[2 * i + 1].z;
                vals[i].w = vals[2 * i].w + vals[2 * i + 1].w;
            }
        write_final4(g, (int)r, (int)c, vals[0]);
    }
}

// Y[r][0..N) = +0 for r < M (row stride ld); N % 4 == 0.
__global__ __launch_bounds__(256) void fill_zero_kernel(float* Y, long ld, int M, int N)
{
    const size_t per_row = (size_t)N / 4;
    const size_t total = per_row * (size_t)M;
    for (size_t v = (size_t)blockIdx.x * blockDim.x + threadIdx.x; v < total;
         v += (size_t)gridDim.x * blockDim.x) {
        const size_t r = v / per_row, c = 4 * (v % per_row);
        *reinterpret_cast<float4*>(Y + r * ld + c) = make_float4(0.f, 0.f, 0.f, 0.f);
    }
}

__global__ __launch_bounds__(256) void cast_bf16_kernel(const float* __restrict__ x,
                                                        uint16_t* __restrict__ y, size_t n8)
{
    for (size_t v = (size_t)blockIdx.x * blockDim.x + threadIdx.x; v < n8;
         v += (size_t)gridDim.x * blockDim.x) {
        const float4 a = reinterpret_cast<const float4*>(x)[2 * v];
        const float4 b = reinterpret_cast<const float4*>(x)[2 * v + 1];
        uint4 o;
        o.x = f32_to_bf16_bits(a.x) | (f32_to_bf16_bits(a.y) << 16);
        o.y = f32_to_bf16_bits(a.z) | (f32_to_bf16_bits(a.w) << 16);
        o.z = f32_to_bf16_bits(b.x) | (f32_to_bf16_bits(b.y) << 16);
        o.w = f32_to_bf16_bits(b.z) | (f32_to_bf16_bits(b.w) << 16);
        reinterpret_cast<uint4*>(y)[v] = o;
    }
}

// The addmm of an empty product (K = 0): every element is the epilogue of
// p = +0.  One thread per element, grid-stride.
__global__ __launch_bounds__(256) void epilogue_only_kernel(GemmArgs g)
{
    const size_t n = (size_t)g.M * g.N;
    for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < n;
         e += (size_t)gridDim.x * blockDim.x)
        write_final1(g, (int)(e / g.N), (int)(e % g.N), 0.0f);
}

// ---------------------------------------------------------------- launches

template <class T, int CPS, int EPI, bool WT>
static hipError_t launch_t(const GemmArgs& g, hipStream_t s)
{
    auto fn = slice_gemm_kernel<T, CPS, EPI, WT>;
    constexpr int lds = lds_bytes<T, CPS>();
    static std::atomic<unsigned long long> lds_set{0};
    const hipError_t attr = ensure_lds_limit(lds_set, reinterpret_cast<const void*>(fn), lds);
    if (attr != hipSuccess)
        return attr;
    const unsigned grid = (unsigned)(g.tiles_m * g.tiles_n * g.slices);
    hipLaunchKernelGGL(fn, dim3(grid), dim3(T::THREADS), lds, s, g);
    return hipGetLastError();
}

template <class T, int EPI, bool WT>
static hipError_t launch_cps(const GemmArgs& g, int cps, hipStream_t s)
{
    switch (cps) {
    case 1: return launch_t<T, 1, EPI, WT>(g, s);
    case 2: return launch_t<T, 2, EPI, WT>(g, s);
    case 4: return launch_t<T, 4, EPI, WT>(g, s);
    case 8:
        if constexpr (EPI == EPI_COMBINE)  // a single slice never needs a combine
            return hipErrorInvalidValue;
        else
            return launch_t<T, 8, EPI, WT>(g, s);
    }
    return hipErrorInvalidValue;
}

template <int EPI>
static hipError_t launch_tile(int tile, const GemmArgs& g, int cps, hipStream_t s)
{
    if (g.wt) {
        switch (tile) {
        case TILE_S16: return launch_cps<TileS16, EPI, true>(g, cps, s);
        case TILE_M64: return launch_cps<TileM64, EPI, true>(g, cps, s);
        case TILE_L128: return launch_cps<TileL128, EPI, true>(g, cps, s);
        }
        return hipErrorInvalidValue;
    }
    switch (tile) {
    case TILE_S16: return launch_cps<TileS16, EPI, false>(g, cps, s);
    case TILE_M64: return launch_cps<TileM64, EPI, false>(g, cps, s);
    case TILE_L128: return launch_cps<TileL128, EPI, false>(g, cps, s);
    }
    return hipErrorInvalidValue;
}

void tile_shape(int tile, int* bm, int* bn)
{
    switch (tile) {
    case TILE_S16: *bm = TileS16::BM; *bn = TileS16::BN; return;
    case TILE_M64: *bm = TileM64::BM; *bn = TileM64::BN; return;
    case TILE_L256: *bm = 256; *bn = 256; return;
    case TILE_D64: *bm = 64; *bn = 128; return;
    case TILE_W256: *bm = 192; *bn = 128; return;
    default: *bm = TileL128::BM; *bn = TileL128::BN; return;
    }
}

hipError_t launch_slice_gemm(int tile, int epi, const GemmArgs& g, int cps, hipStream_t s)
{
    if ((tile == TILE_L128 || tile == TILE_L256 || tile == TILE_D64 || tile == TILE_W256) &&
        lds_engine_supports(tile, g, cps))
        return launch_lds_gemm(tile, epi, g, cps, s);
    if (tile == TILE_L256 || tile == TILE_D64 || tile == TILE_W256)
        return hipErrorInvalidValue;
    return launch_reg_gemm(tile, epi, g, cps, s);
}

hipError_t launch_reg_gemm(int tile, int epi, const GemmArgs& g, int cps, hipStream_t s)
{
    switch (epi) {
    case EPI_STORE: return launch_tile<EPI_STORE>(tile, g, cps, s);
    case EPI_COMBINE: return launch_tile<EPI_COMBINE>(tile, g, cps, s);
    case EPI_ATOMIC: return launch_tile<EPI_ATOMIC>(tile, g, cps, s);
    }
    return hipErrorInvalidValue;
}

static unsigned grid_for(size_t work, unsigned block)
{
    size_t g = (work + block - 1) / block;
    if (g > 8192) g = 8192;
    if (g < 1) g = 1;
    return (unsigned)g;
}

hipError_t launch_tree_combine(const float* parts, size_t stride, int count, float* Y, size_t n,
                               hipStream_t s)
{
    const size_t n4 = n / 4;
    const dim3 grid(grid_for(n4, 256)), block(256);
    switch (count) {
    case 1: hipLaunchKernelGGL(tree_combine_kernel<1>, grid, block, 0, s, parts, stride, Y, n4); break;
    case 2: hipLaunchKernelGGL(tree_combine_kernel<2>, grid, block, 0, s, parts, stride, Y, n4); break;
    case 4: hipLaunchKernelGGL(tree_combine_kernel<4>, grid, block, 0, s, parts, stride, Y, n4); break;
    case 8: hipLaunchKernelGGL(tree_combine_kernel<8>, grid, block, 0, s, parts, stride, Y, n4); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_tree_combine_rows(const float* parts, size_t stride, int count,
                                    const GemmArgs& g, hipStream_t s)
{
    const size_t total4 = (size_t)g.M * (g.N / 4);
    const dim3 grid(grid_for(total4, 256)), block(256);
    switch (count) {
    case 1: hipLaunchKernelGGL(tree_combine_rows_kernel<1>, grid, block, 0, s, parts, stride, g); break;
    case 2: hipLaunchKernelGGL(tree_combine_rows_kernel<2>, grid, block, 0, s, parts, stride, g); break;
    case 4: hipLaunchKernelGGL(tree_combine_rows_kernel<4>, grid, block, 0, s, parts, stride, g); break;
    case 8: hipLaunchKernelGGL(tree_combine_rows_kernel<8>, grid, block, 0, s, parts, stride, g); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_fill_zero(float* Y, long ld, int M, int N, hipStream_t s)
{
    hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for((size_t)M * (N / 4), 256)), dim3(256), 0,
                       s, Y, ld, M, N);
    return hipGetLastError();
}

hipError_t launch_epilogue_only(const GemmArgs& g, hipStream_t s)
{
    const size_t n = (size_t)g.M * g.N;
    hipLaunchKernelGGL(epilogue_only_kernel, dim3(grid_for(n, 256)), dim3(256), 0, s, g);
    return hipGetLastError();
}

hipError_t launch_cast_bf16(const float* x, uint16_t* y, size_t n, hipStream_t s)
{
    const size_t n8 = n / 8;
    hipLaunchKernelGGL(cast_bf16_kernel, dim3(grid_for(n8, 256)), dim3(256), 0, s, x, y, n8);
    return hipGetLastError();
}

}  // namespace detred
