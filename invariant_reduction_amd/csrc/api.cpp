// C-ABI layer of libdetred: argument checks, the locked policy, workspace
// layout and kernel launches.  Declarations and the contract of every entry
// point are in include/detred.h.
#include "detred.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

using namespace detred;

namespace {

constexpr int kChunks = 8;          // chunks of K when K allows them
constexpr int kChunkGranule = 256;  // K must be a multiple of this for 8 chunks

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned256(const void* p) { return ((uintptr_t)p & 255u) == 0; }
bool pow2_le8(int v) { return v == 1 || v == 2 || v == 4 || v == 8; }

// ceil(a / b) for a >= 0, b > 0, without overflowing int on the way
int cdiv(int a, int b) { return (int)(((long)a + b - 1) / b); }

int chunk_count(int K) { return (K >= kChunkGranule && K % kChunkGranule == 0) ? kChunks : 1; }

// The locked reduction (P, Kc: a function of K alone, they fix the bits)
// and the tile family for N.  The tile a call launches and its split also
// follow M (plan, narrow_for_decode, widen_for_rows, widen_for_roots,
// auto_split): the tile decides speed, the chunk tree decides the bits.
struct Policy {
    int P, Kc, tile, bm, bn, default_split;
};

Policy policy_for(int N, int K)
{
    Policy p;
    p.P = chunk_count(K);
    p.Kc = K / p.P;
    if (N <= 16) {
        p.tile = TILE_S16;
        p.default_split = p.P;   // skinny outputs: parallelise over K
    } else if (N <= 64 || p.P == 1) {
        p.tile = TILE_M64;
        p.default_split = N <= 64 ? p.P : 1;
    } else {
        p.tile = TILE_L128;
        p.default_split = 1;
    }
    tile_shape(p.tile, &p.bm, &p.bn);
    return p;
}

// The tile for an M-row product: the policy's, except that narrow outputs
// (N <= 64) take 64x16 tiles while 64x64 tiles would leave fewer than 256
// workgroups (LoRA shrink on MI355X at 8 slices: 256x64x4096 14.7 -> 12.1 us,
// M = 1 13.3 -> 10.7 us; at M = 4096 the wider tile stays, 20.1 vs 28.2 us).
// Like the split, the tile never changes the bits.
Policy plan(int M, int N, int K)
{
    Policy p = policy_for(N, K);
    if (p.tile == TILE_M64 && N <= 64) {
        const long wgs = (long)cdiv(M, p.bm) * cdiv(N, p.bn) * p.default_split;
        if (wgs < 256) {
            p.tile = TILE_S16;
            tile_shape(p.tile, &p.bm, &p.bn);
        }
    }
    return p;
}

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

size_t partial_bytes(int M, int N, int S) { return round_up((size_t)S * M * N * sizeof(float), 256); }

size_t counter_bytes(const Policy& p, int M, int N)
{
    const size_t tm = (size_t)cdiv(M, p.bm), tn = (size_t)cdiv(N, p.bn);
    return round_up(tm * tn * sizeof(unsigned), 256);
}

detred_status hip_status(hipError_t e) { return e == hipSuccess ? DETRED_OK : DETRED_EHIP; }

// Checks shared by the GEMM entry points (wt: W given transposed, [N][K]
// with rows ldw apart).
detred_status check_gemm(const uint16_t* X, int ldx, const uint16_t* W, int ldw, const float* Y,
                         int ldy, int M, int N, int K, bool wt = false)
{
    if (M < 0 || N < 0 || K < 0)
        return DETRED_EINVAL;
    if (ldx < K || ldw < (wt ? K : N) || ldy < N || ldx < 0 || ldw < 0 || ldy < 0)
        return DETRED_EINVAL;
    if (M == 0 || N == 0)
        return DETRED_OK;
    if (!Y || !aligned16(Y) || (ldy % 4) != 0)
        return DETRED_EINVAL;
    if (K > 0) {
        if (!X || !W || !aligned16(X) || !aligned16(W) || (ldx % 8) != 0 || (ldw % 8) != 0)
            return DETRED_EINVAL;
    }
    if ((K % 8) != 0 || (N % 8) != 0)
        return DETRED_EUNSUPPORTED;
    return DETRED_OK;
}

GemmArgs make_args(const Policy& p, const uint16_t* X, int ldx, const uint16_t* W, int ldw,
                   float* Y, int ldy, int M, int N, int K, int slices)
{
    GemmArgs g;
    g.X = X;
    g.ldx = ldx;
    g.W = W;
    g.ldw = ldw;
    g.wt = 0;
    g.Y = Y;
    g.ldy = ldy;
    g.out_z_stride = 0;
    g.part = nullptr;
    g.counters = nullptr;
    g.M = M;
    g.N = N;
    g.K = K;
    g.Kc = p.Kc;
    g.slices = slices;
    g.tiles_m = cdiv(M, p.bm);
    g.tiles_n = cdiv(N, p.bn);
    g.epi = 0;
    g.C = nullptr;
    g.ldc = 0;
    g.alpha = 1.0f;
    g.beta = 1.0f;
    g.out_bf16 = 0;
    g.direct_roots = 0;
    return g;
}

// Subtree roots of one-chunk slices (the tree-TP shards) on the 256x256
// tile: it halves the operand traffic into LDS per product, and at chunks of
// 1024 or more its longer prologue and two-pass epilogue pay off (8 shards
// of 512x8192x8192 on MI355X: 104 -> 93 us; 1024 rows: 236 -> 192 us; with
// chunks of 512, 4096x4096x4096 at 8 shards, the 128x128 tile stays ahead,
// 242 vs 248 us).  Taken only where the grid still has 256 workgroups.  The
// tile never changes the bits.
void widen_for_roots(Policy& p, GemmArgs& g, int cps)
{
    if (p.tile != TILE_L128 || cps != 1 || p.Kc < 1024 || g.M < 256)
        return;
    GemmArgs w = g;
    w.tiles_m = cdiv(g.M, 256);
    w.tiles_n = cdiv(g.N, 256);
    if ((long)w.tiles_m * w.tiles_n * w.slices < 256 || !lds_engine_supports(TILE_L256, w, 1))
        return;
    // Roots that fit the 256 MiB MALL go out straight from the registers:
    // 8 shards of 512x8192x8192 (134 MB) 83 -> 79 us, 1024 rows 183 -> 179
    // us; a larger output keeps the staged row pieces (4096 rows: 730 vs
    // 754 us), whose whole 128-byte lines suit HBM better.
    w.direct_roots = (size_t)w.slices * w.M * w.N * sizeof(float) <= ((size_t)256 << 20);
    p.tile = TILE_L256;
    tile_shape(p.tile, &p.bm, &p.bn);
    g = w;
}

// Products of at most 64 rows on the 64x128 tile: the same tile count as
// 128x128 (one tile row either way, so the split, the workspace and the
// arrival counters are unchanged), but half the A block, so more stages of
// weights are in flight.  The tile never changes the bits.
void narrow_for_decode(Policy& p, GemmArgs& g, int cps)
{
    if (p.tile != TILE_L128 || g.M > 64)
        return;
    GemmArgs w = g;
    w.tiles_m = 1;
    if (!lds_engine_supports(TILE_D64, w, cps))
        return;
    p.tile = TILE_D64;
    tile_shape(p.tile, &p.bm, &p.bn);
    g = w;
}

// Unsplit eight-chunk products on the 192x128 tile, whose top subtree level
// waits in the product's own output rows of Y (so the output must be fp32
// and hold nothing the call still reads: no bf16 output, and a C that
// overlaps Y keeps the 128x128 tile), where it takes fewer rounds of
// workgroups: each CU holds one workgroup of either tile, and a 192x128 tile
// takes about 1.25 times as long as a 128x128 one (1.5 times the outputs at
// a sixth less time per output), so it is taken when 1.25 x its rounds over
// the 256 CUs do not exceed the 128x128 tile's.  On MI355X this picks the
// faster tile on all 40 shapes of a sweep of M in 512..4096, N in
// {4096, 8192, 14336}, K in {4096, 8192, 14336} (768x8192x8192 167 -> 111
// us, 1280x4096x14336 283 -> 158 us, 4096x14336x4096 618 -> 539 us; the
// 128x128 tile kept at 1024x4096x4096 47 vs 55 us, 512x8192x8192 99 vs 104
// us).  The tile never changes the bits.
constexpr long kComputeUnits = 256;

bool overlaps(const void* a, size_t na, const void* b, size_t nb)
{
    const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
    return pa < pb + nb && pb < pa + na;
}

void widen_for_rows(Policy& p, GemmArgs& g, int cps)
{
    if (p.tile != TILE_L128 || cps != 8 || g.out_z_stride != 0)
        return;
    if (g.epi && g.out_bf16)
        return;
    if (g.epi && g.C) {
        const size_t ybytes = ((size_t)(g.M - 1) * g.ldy + g.N) * sizeof(float);
        const size_t cbytes =
            (g.ldc == 0 ? (size_t)g.N : (size_t)(g.M - 1) * g.ldc + g.N) * sizeof(float);
        if (overlaps(g.Y, ybytes, g.C, cbytes))
            return;
    }
    GemmArgs w = g;
    int bm = 0, bn = 0;
    tile_shape(TILE_W256, &bm, &bn);
    w.tiles_m = cdiv(g.M, bm);
    w.tiles_n = cdiv(g.N, bn);
    const long rounds = ((long)g.tiles_m * g.tiles_n + kComputeUnits - 1) / kComputeUnits;
    const long rounds_w = ((long)w.tiles_m * w.tiles_n + kComputeUnits - 1) / kComputeUnits;
    if (5 * rounds_w > 4 * rounds || !lds_engine_supports(TILE_W256, w, cps))
        return;
    p.tile = TILE_W256;
    p.bm = bm;
    p.bn = bn;
    g = w;
}

// The split for split_k = 0.  The split only decides how many workgroups
// share the chunk tree, never the bits.  Narrow outputs keep the policy's
// split (one slice per chunk).  A wide product is sized against the 256 CUs,
// the LDS engine's stage depth (four stages for a grid of at most 256
// workgroups) and the cost of its slice roots, which a second launch
// combines (t = output tiles of 128 x 128, Kc = chunk width):
//  - 257 <= t <= 447 and the unsplit product fits one round of 192 x 128
//    tiles (eight chunks of whole 64-wide K blocks, ceil(M/192) x
//    ceil(N/128) <= 256, and a call that may take that tile: wide): unsplit;
//  - Kc >= 1536 with at least 256 rows and t >= 96: 8 slices (one chunk
//    each, on the 256x256 root tile: the long chunks amortise its
//    prologue and epilogue);
//  - t <= 128: the most slices that keep the grid at or under 256
//    workgroups, except 4 rather than 2 for products of at most 16 rows;
//  - 129 <= t <= 192: 4 slices for Kc >= 1024, else unsplit (at t = 192
//    with chunks of 1024, cold: 320x8192x8192 97 -> 82 us, 700x4096x8192
//    86 -> 82 us);
//  - t > 192: unsplit, except for 257..447 tiles (1.0-1.75 waves of
//    workgroups unsplit): 4 slices for Kc >= 1024, 2 for shorter chunks.
// Measured on MI355X with the weights coming from HBM over M in 1..2560,
// N in 1024..14336, K in {4096, 8192, 14336}, S in {1, 2, 4, 8}; e.g.
// 128x14336x4096 45.2 -> 38.2 us (2 slices, not 4), 768x1024x4096 33.5 ->
// 29.2 us (4, not 8), 384x8192x14336 at 8 slices 27 % faster than unsplit;
// the first rule (unsplit on one round of 192x128 tiles) against the split
// the others give there: 384x14336x4096 85 -> 66 us, 768x8192x8192 140 ->
// 105 us, 1280x4096x4096 86 -> 62 us, 6144x1024x4096 87 -> 64 us,
// 384x14336x14336 216 -> 194 us (640x8192x14336 175 vs 177 us).
bool fits_one_wide_round(const Policy& p, int M, int N)
{
    return p.P == 8 && p.Kc % 64 == 0 && (long)cdiv(M, 192) * cdiv(N, 128) <= kComputeUnits;
}

int auto_split(const Policy& p, int M, int N, bool wide = true)
{
    if (p.tile != TILE_L128)
        return p.default_split;
    const long tiles = (long)cdiv(M, p.bm) * cdiv(N, p.bn);
    const bool long_chunks = p.Kc >= 1024;
    const bool band = tiles > 256 && tiles < 448;
    int S = 1;
    if (band && wide && fits_one_wide_round(p, M, N)) {
        S = 1;
    } else if (p.Kc >= 1536 && M >= 256 && tiles >= 96) {
        S = 8;
    } else if (tiles > 192) {
        if (band)
            S = long_chunks ? 4 : 2;
    } else if (tiles > 128) {
        S = long_chunks ? 4 : 1;
    } else {
        while (S < p.P && tiles * S * 2 <= 256)
            S *= 2;
        if (S == 2 && M <= 16)
            S = 4;
    }
    return S < p.P ? S : p.P;
}

// Resolve split_k / tp_shards against the policy; 0 means auto_split.
detred_status resolve_split(const Policy& p, int split, int M, int N, int* out,
                            bool wide = true)
{
    if (split == 0)
        split = auto_split(p, M, N, wide);
    if (!pow2_le8(split) || split > p.P)
        return DETRED_EUNSUPPORTED;
    *out = split;
    return DETRED_OK;
}

}  // namespace

extern "C" {

const char* detred_status_string(detred_status status)
{
    switch (status) {
    case DETRED_OK: return "DETRED_OK";
    case DETRED_EINVAL: return "DETRED_EINVAL: invalid argument";
    case DETRED_EUNSUPPORTED: return "DETRED_EUNSUPPORTED: shape or split not supported";
    case DETRED_EWORKSPACE: return "DETRED_EWORKSPACE: workspace missing or too small";
    case DETRED_EHIP: return "DETRED_EHIP: HIP runtime error";
    }
    return "DETRED_UNKNOWN_STATUS";
}

int detred_version(void) { return 100; }

detred_status detred_policy(int N, int K, int* chunks, int* chunk_k, int* tile_m, int* tile_n,
                            int* default_split)
{
    if (N < 0 || K < 0)
        return DETRED_EINVAL;
    const Policy p = policy_for(N, K);
    if (chunks) *chunks = p.P;
    if (chunk_k) *chunk_k = p.Kc;
    if (tile_m) *tile_m = p.bm;
    if (tile_n) *tile_n = p.bn;
    if (default_split) *default_split = p.default_split;
    return DETRED_OK;
}

int detred_auto_split(int M, int N, int K)
{
    if (M < 0 || N < 0 || K < 0)
        return 0;
    return auto_split(plan(M, N, K), M, N);
}

size_t detred_gemm_workspace_bytes(int M, int N, int K, int split_or_shards)
{
    if (M < 0 || N < 0 || K < 0)
        return 0;
    const Policy p = plan(M, N, K);
    // split 0: enough for the split any call picks, also an addmm that
    // cannot take the 192x128 tile (a bf16 output, or C overlapping Y)
    if (split_or_shards == 0) {
        const int a = auto_split(p, M, N, true), b = auto_split(p, M, N, false);
        const size_t na = detred_gemm_workspace_bytes(M, N, K, a);
        const size_t nb = detred_gemm_workspace_bytes(M, N, K, b);
        return na > nb ? na : nb;
    }
    // no workspace for one slice, none for a split the calls reject
    if (!pow2_le8(split_or_shards) || split_or_shards == 1 || split_or_shards > p.P)
        return 0;
    return partial_bytes(M, N, split_or_shards) + counter_bytes(p, M, N);
}

detred_status detred_workspace_init(void* ws, size_t ws_bytes, detred_stream s)
{
    if (ws_bytes == 0)
        return DETRED_OK;
    if (!ws)
        return DETRED_EINVAL;
    return hip_status(hipMemsetAsync(ws, 0, ws_bytes, (hipStream_t)s));
}

}  // extern "C"

namespace {

// The deterministic product (and its epilogue, when g.epi) with S slices:
// one launch; with S > 1 the partials and counters live in ws.
// S subtree roots into S planes [S][M][N] at ws (plain stores, one launch),
// then the top log2(S) tree levels into Y (a second, streaming launch).
// The bits are those of the one-launch last-arriver combine.
detred_status run_roots_then_combine(Policy p, GemmArgs g, int S, float* ws, hipStream_t hs)
{
    const GemmArgs out = g;  // Y, ldy and the epilogue of the combined value
    g.Y = ws;
    g.epi = 0;
    g.out_bf16 = 0;
    g.C = nullptr;
    g.ldy = g.N;
    g.out_z_stride = (long)g.M * g.N;
    g.part = nullptr;
    g.counters = nullptr;
    widen_for_roots(p, g, p.P / S);
    narrow_for_decode(p, g, p.P / S);
    if (launch_slice_gemm(p.tile, EPI_STORE, g, p.P / S, hs) != hipSuccess)
        return DETRED_EHIP;
    const size_t plane = (size_t)g.M * g.N;
    if (!out.epi && out.ldy == g.N)
        return hip_status(launch_tree_combine(ws, plane, S, out.Y, plane, hs));
    return hip_status(launch_tree_combine_rows(ws, plane, S, out, hs));
}

// Which combine a split product takes.  Two launches (roots, then one
// streaming pass over them) wherever the 128x128 policy tile runs (the wide
// engine's roots go out with plain stores at full rate, where the last
// arriver of each tile would read S partial tiles at the end of its own
// work) and for outputs of at least kTwoPhaseMinElems elements; the
// one-launch last-arriver combine for narrow outputs below that, where a
// second launch costs more than it saves.  Measured on MI355X, same bits
// either way: 4096x4096x4096 at 8 slices 662 -> 385 us and 512x8192x8192 at
// 8 158 -> 108 us in two launches; kernel time (rocprofv3) of the LoRA
// shrink 256x64x4096 at 8 slices 7.96 us in two launches against 7.59 in
// one (the atomic control: 7.4), at 4 slices 10.3 against 8.7 (atomic 9.7).
constexpr size_t kTwoPhaseMinElems = 65536;

// counters: where the arrival counters of a last-arriver combine live when
// not in ws after the partials (the no-allocation entry point keeps them at
// a fixed place in its scratch, so that they stay zero between calls).
detred_status run_det(const Policy& p0, GemmArgs g, int S, void* ws, size_t ws_bytes,
                      hipStream_t hs, unsigned* counters = nullptr)
{
    Policy p = p0;
    if (g.K == 0)
        return hip_status(g.epi ? launch_epilogue_only(g, hs)
                                : launch_fill_zero(g.Y, g.ldy, g.M, g.N, hs));
    if (S == 1) {
        narrow_for_decode(p, g, p.P);
        widen_for_rows(p, g, p.P);
        return hip_status(launch_slice_gemm(p.tile, EPI_STORE, g, p.P, hs));
    }
    // the last-arriver combine addresses a tile's rows with 32-bit offsets
    if ((size_t)(p.bm - 1) * g.N + p.bn >= ((size_t)1 << 29))
        return DETRED_EUNSUPPORTED;
    const size_t need = partial_bytes(g.M, g.N, S) + (counters ? 0 : counter_bytes(p, g.M, g.N));
    if (!ws || !aligned256(ws) || ws_bytes < need)
        return DETRED_EWORKSPACE;
    if (p.tile == TILE_L128 || (size_t)g.M * g.N >= kTwoPhaseMinElems)
        return run_roots_then_combine(p, g, S, (float*)ws, hs);
    g.part = (float*)ws;
    g.counters = counters ? counters : (unsigned*)((char*)ws + partial_bytes(g.M, g.N, S));
    narrow_for_decode(p, g, p.P / S);
    return hip_status(launch_slice_gemm(p.tile, EPI_COMBINE, g, p.P / S, hs));
}

// Validation of det_splitk_gemm / det_splitk_addmm that would otherwise
// only happen in run_det (so a composite call can check before launching).
detred_status check_det(const Policy& p, int M, int N, int K, int S, const void* ws,
                        size_t ws_bytes)
{
    if (K == 0 || S == 1)
        return DETRED_OK;
    if ((size_t)(p.bm - 1) * N + p.bn >= ((size_t)1 << 29))
        return DETRED_EUNSUPPORTED;
    if (!ws || !aligned256(ws) || ws_bytes < partial_bytes(M, N, S) + counter_bytes(p, M, N))
        return DETRED_EWORKSPACE;
    return DETRED_OK;
}

detred_status check_epilogue(const float* C, int ldc, int N, int y_dtype)
{
    if (y_dtype != DETRED_F32 && y_dtype != DETRED_BF16)
        return DETRED_EINVAL;
    if (C && (!aligned16(C) || ldc < 0 || (ldc != 0 && (ldc < N || ldc % 4 != 0))))
        return DETRED_EINVAL;
    return DETRED_OK;
}

// Byte layout of the det_lora_forward workspace.
struct LoraLayout {
    size_t base, zb, ws_base, ws_z, total;
    size_t ws_base_bytes, ws_z_bytes;
    int s_base, s_z;
};

LoraLayout lora_layout(int M, int N, int K, int r)
{
    LoraLayout l;
    l.s_base = auto_split(plan(M, N, K), M, N);
    l.s_z = auto_split(plan(M, r, K), M, r);
    l.ws_base_bytes = detred_gemm_workspace_bytes(M, N, K, l.s_base);
    l.ws_z_bytes = detred_gemm_workspace_bytes(M, r, K, l.s_z);
    l.base = 0;
    l.zb = l.base + round_up((size_t)M * N * sizeof(float), 256);
    l.ws_base = l.zb + round_up((size_t)M * r * sizeof(uint16_t), 256);
    l.ws_z = l.ws_base + round_up(l.ws_base_bytes, 256);
    l.total = l.ws_z + round_up(l.ws_z_bytes, 256);
    return l;
}

}  // namespace

namespace {

detred_status det_gemm_impl(const uint16_t* X, int ldx, const uint16_t* W, int ldw, bool wt,
                            float* Y, int ldy, int M, int N, int K, int split_k, void* ws,
                            size_t ws_bytes, detred_stream s)
{
    detred_status st = check_gemm(X, ldx, W, ldw, Y, ldy, M, N, K, wt);
    if (st != DETRED_OK || M == 0 || N == 0)
        return st;
    const Policy p = plan(M, N, K);
    int S = 0;
    if ((st = resolve_split(p, split_k, M, N, &S)) != DETRED_OK)
        return st;
    GemmArgs g = make_args(p, X, ldx, W, ldw, Y, ldy, M, N, K, S);
    g.wt = wt;
    return run_det(p, g, S, ws, ws_bytes, (hipStream_t)s);
}

detred_status det_addmm_impl(const uint16_t* X, int ldx, const uint16_t* W, int ldw, bool wt,
                             const float* C, int ldc, float alpha, float beta, void* Y, int ldy,
                             int y_dtype, int M, int N, int K, int split_k, void* ws,
                             size_t ws_bytes, detred_stream s)
{
    detred_status st = check_epilogue(C, ldc, N, y_dtype);
    if (st != DETRED_OK)
        return st;
    st = check_gemm(X, ldx, W, ldw, (const float*)Y, ldy, M, N, K, wt);
    if (st != DETRED_OK || M == 0 || N == 0)
        return st;
    const Policy p = plan(M, N, K);
    int S = 0;
    // the 192x128 tile (and so the automatic split that counts on it) needs
    // an fp32 output that holds nothing the call still reads
    bool wide = y_dtype != DETRED_BF16;
    if (wide && C) {
        const size_t ybytes = ((size_t)(M - 1) * ldy + N) * sizeof(float);
        const size_t cbytes = (ldc == 0 ? (size_t)N : (size_t)(M - 1) * ldc + N) * sizeof(float);
        wide = !overlaps(Y, ybytes, C, cbytes);
    }
    if ((st = resolve_split(p, split_k, M, N, &S, wide)) != DETRED_OK)
        return st;
    GemmArgs g = make_args(p, X, ldx, W, ldw, (float*)Y, ldy, M, N, K, S);
    g.wt = wt;
    g.epi = 1;
    g.C = C;
    g.ldc = ldc;
    g.alpha = alpha;
    g.beta = beta;
    g.out_bf16 = (y_dtype == DETRED_BF16);
    return run_det(p, g, S, ws, ws_bytes, (hipStream_t)s);
}

}  // namespace

extern "C" {

detred_status det_splitk_gemm(const uint16_t* X, int ldx, const uint16_t* W, int ldw, float* Y,
                              int ldy, int M, int N, int K, int split_k, void* ws, size_t ws_bytes,
                              detred_stream s)
{
    return det_gemm_impl(X, ldx, W, ldw, false, Y, ldy, M, N, K, split_k, ws, ws_bytes, s);
}

detred_status det_splitk_gemm_wt(const uint16_t* X, int ldx, const uint16_t* Wt, int ldwt, float* Y,
                                 int ldy, int M, int N, int K, int split_k, void* ws,
                                 size_t ws_bytes, detred_stream s)
{
    return det_gemm_impl(X, ldx, Wt, ldwt, true, Y, ldy, M, N, K, split_k, ws, ws_bytes, s);
}

static_assert(kNoallocScratchBytes - kNoallocCounterBytes == DETRED_NOALLOC_PARTIAL_BYTES,
              "the header states the no-allocation limit");

detred_status det_splitk_gemm_noalloc(const uint16_t* X, int ldx, const uint16_t* W, int ldw,
                                      float* Y, int ldy, int M, int N, int K, int split_k,
                                      detred_stream s)
{
    detred_status st = check_gemm(X, ldx, W, ldw, Y, ldy, M, N, K);
    if (st != DETRED_OK || M == 0 || N == 0)
        return st;
    const Policy p = plan(M, N, K);
    int S = 0;
    if ((st = resolve_split(p, split_k, M, N, &S)) != DETRED_OK)
        return st;
    hipStream_t hs = (hipStream_t)s;
    const GemmArgs g = make_args(p, X, ldx, W, ldw, Y, ldy, M, N, K, S);
    if (K == 0 || S == 1)
        return run_det(p, g, S, nullptr, 0, hs);  // no scratch involved
    if (partial_bytes(M, N, S) > kNoallocScratchBytes - kNoallocCounterBytes ||
        counter_bytes(p, M, N) > kNoallocCounterBytes)
        return DETRED_EWORKSPACE;
    if ((size_t)(p.bm - 1) * N + p.bn >= ((size_t)1 << 29))
        return DETRED_EUNSUPPORTED;
    void* scratch = nullptr;
    if (noalloc_scratch(hs, &scratch) != hipSuccess)
        return DETRED_EHIP;
    char* base = static_cast<char*>(scratch);
    return run_det(p, g, S, base + kNoallocCounterBytes,
                   kNoallocScratchBytes - kNoallocCounterBytes, hs,
                   reinterpret_cast<unsigned*>(base));
}

detred_status det_splitk_addmm(const uint16_t* X, int ldx, const uint16_t* W, int ldw,
                               const float* C, int ldc, float alpha, float beta, void* Y, int ldy,
                               int y_dtype, int M, int N, int K, int split_k, void* ws,
                               size_t ws_bytes, detred_stream s)
{
    return det_addmm_impl(X, ldx, W, ldw, false, C, ldc, alpha, beta, Y, ldy, y_dtype, M, N, K,
                          split_k, ws, ws_bytes, s);
}

detred_status det_splitk_addmm_wt(const uint16_t* X, int ldx, const uint16_t* Wt, int ldwt,
                                  const float* C, int ldc, float alpha, float beta, void* Y,
                                  int ldy, int y_dtype, int M, int N, int K, int split_k, void* ws,
                                  size_t ws_bytes, detred_stream s)
{
    return det_addmm_impl(X, ldx, Wt, ldwt, true, C, ldc, alpha, beta, Y, ldy, y_dtype, M, N, K,
                          split_k, ws, ws_bytes, s);
}

size_t det_lora_workspace_bytes(int M, int N, int K, int r)
{
    if (M < 0 || N < 0 || K < 0 || r <= 0)
        return 0;
    return lora_layout(M, N, K, r).total;
}

detred_status det_lora_forward(const uint16_t* X, int ldx, const uint16_t* W, int ldw,
                               const uint16_t* A, int lda, const uint16_t* B, int ldb, float scale,
                               uint16_t* Y, int ldy, int M, int N, int K, int r, void* ws,
                               size_t ws_bytes, detred_stream s)
{
    if (M < 0 || N < 0 || K < 0 || r <= 0)
        return DETRED_EINVAL;
    if (r % 8 != 0)
        return DETRED_EUNSUPPORTED;
    if (M == 0 || N == 0)
        return DETRED_OK;
    const LoraLayout l = lora_layout(M, N, K, r);
    if (!ws || !aligned256(ws) || ws_bytes < l.total)
        return DETRED_EWORKSPACE;
    char* w = (char*)ws;
    float* base = (float*)(w + l.base);
    uint16_t* zb = (uint16_t*)(w + l.zb);
    const Policy pb = plan(M, N, K), pz = plan(M, r, K), pe = plan(M, N, r);
    // every check before the first launch
    detred_status st;
    if ((st = check_gemm(X, ldx, W, ldw, base, N, M, N, K)) != DETRED_OK ||
        (st = check_gemm(X, ldx, A, lda, (const float*)zb, r, M, r, K)) != DETRED_OK ||
        (st = check_gemm(zb, r, B, ldb, (const float*)Y, ldy, M, N, r)) != DETRED_OK ||
        (st = check_det(pb, M, N, K, l.s_base, w + l.ws_base, l.ws_base_bytes)) != DETRED_OK ||
        (st = check_det(pz, M, r, K, l.s_z, w + l.ws_z, l.ws_z_bytes)) != DETRED_OK)
        return st;
    hipStream_t hs = (hipStream_t)s;
    const GemmArgs gb = make_args(pb, X, ldx, W, ldw, base, N, M, N, K, l.s_base);
    if ((st = run_det(pb, gb, l.s_base, w + l.ws_base, l.ws_base_bytes, hs)) != DETRED_OK)
        return st;
    // the shrink rounds its final values to bf16 in its own epilogue (alpha
    // = 1, no C): the bits of casting its fp32 result, one launch fewer
    GemmArgs gz = make_args(pz, X, ldx, A, lda, (float*)zb, r, M, r, K, l.s_z);
    gz.epi = 1;
    gz.out_bf16 = 1;
    if ((st = run_det(pz, gz, l.s_z, w + l.ws_z, l.ws_z_bytes, hs)) != DETRED_OK)
        return st;
    GemmArgs ge = make_args(pe, zb, r, B, ldb, (float*)Y, ldy, M, N, r, 1);
    ge.epi = 1;
    ge.C = base;
    ge.ldc = N;
    ge.alpha = scale;
    ge.beta = 1.0f;
    ge.out_bf16 = 1;
    return run_det(pe, ge, 1, nullptr, 0, hs);
}

detred_status atomic_splitk_gemm(const uint16_t* X, int ldx, const uint16_t* W, int ldw, float* Y,
                                 int ldy, int M, int N, int K, int split_k, detred_stream s)
{
    detred_status st = check_gemm(X, ldx, W, ldw, Y, ldy, M, N, K);
    if (st != DETRED_OK || M == 0 || N == 0)
        return st;
    const Policy p = plan(M, N, K);
    int S = 0;
    if ((st = resolve_split(p, split_k, M, N, &S)) != DETRED_OK)
        return st;
    hipStream_t hs = (hipStream_t)s;
    hipError_t e = launch_fill_zero(Y, ldy, M, N, hs);
    if (e != hipSuccess || K == 0)
        return hip_status(e);
    GemmArgs g = make_args(p, X, ldx, W, ldw, Y, ldy, M, N, K, S);
    Policy pa = p;
    narrow_for_decode(pa, g, p.P / S);
    return hip_status(launch_slice_gemm(pa.tile, EPI_ATOMIC, g, p.P / S, hs));
}

}  // extern "C"

namespace {

detred_status tree_tp_impl(const uint16_t* X, int ldx, const uint16_t* W, int ldw, bool wt,
                           float* Y, int ldy, int M, int N, int K, int tp_shards, void* ws,
                           size_t ws_bytes, detred_stream s)
{
    detred_status st = check_gemm(X, ldx, W, ldw, Y, ldy, M, N, K, wt);
    if (st != DETRED_OK || M == 0 || N == 0)
        return st;
    Policy p = plan(M, N, K);
    if (!pow2_le8(tp_shards) || tp_shards > p.P)
        return DETRED_EUNSUPPORTED;
    const int T = tp_shards;
    hipStream_t hs = (hipStream_t)s;
    if (K == 0)
        return hip_status(launch_fill_zero(Y, ldy, M, N, hs));
    GemmArgs g = make_args(p, X, ldx, W, ldw, Y, ldy, M, N, K, T);
    g.wt = wt;
    if (T == 1) {
        narrow_for_decode(p, g, p.P);
        widen_for_rows(p, g, p.P);
        return hip_status(launch_slice_gemm(p.tile, EPI_STORE, g, p.P, hs));
    }
    if (!ws || !aligned256(ws) || ws_bytes < partial_bytes(M, N, T))
        return DETRED_EWORKSPACE;
    // phase 1: every shard writes its subtree root to its own buffer; phase
    // 2: the top log2(T) tree levels (the cross-rank reduction)
    return run_roots_then_combine(p, g, T, (float*)ws, hs);
}

detred_status tree_tp_shards_impl(const uint16_t* X, int ldx, const uint16_t* W, int ldw, bool wt,
                                  float* P, int M, int N, int K, int tp_shards, detred_stream s)
{
    detred_status st = check_gemm(X, ldx, W, ldw, P, N, M, N, K, wt);
    if (st != DETRED_OK || M == 0 || N == 0)
        return st;
    Policy p = plan(M, N, K);
    if (!pow2_le8(tp_shards) || tp_shards > p.P)
        return DETRED_EUNSUPPORTED;
    hipStream_t hs = (hipStream_t)s;
    if (K == 0) {
        const hipError_t e = launch_fill_zero(P, N, M * tp_shards, N, hs);
        return hip_status(e);
    }
    GemmArgs g = make_args(p, X, ldx, W, ldw, P, N, M, N, K, tp_shards);
    g.wt = wt;
    g.out_z_stride = (long)M * N;
    widen_for_roots(p, g, p.P / tp_shards);
    narrow_for_decode(p, g, p.P / tp_shards);
    return hip_status(launch_slice_gemm(p.tile, EPI_STORE, g, p.P / tp_shards, hs));
}

detred_status tree_tp_shard_impl(const uint16_t* Xt, int ldx, const uint16_t* Wt, int ldw, bool wt,
                                 float* Pt, int ldp, int M, int N, int Kt, int tp_shards,
                                 detred_stream s)
{
    if (!pow2_le8(tp_shards) || Kt < 0)
        return DETRED_EINVAL;
    const long Kl = (long)Kt * tp_shards;
    if (Kl > 0x7fffffffL)
        return DETRED_EINVAL;
    const int K = (int)Kl;
    detred_status st = check_gemm(Xt, ldx, Wt, ldw, Pt, ldp, M, N, Kt, wt);
    if (st != DETRED_OK || M == 0 || N == 0)
        return st;
    Policy p = plan(M, N, K);
    if (tp_shards > p.P)
        return DETRED_EUNSUPPORTED;
    hipStream_t hs = (hipStream_t)s;
    if (Kt == 0)
        return hip_status(launch_fill_zero(Pt, ldp, M, N, hs));
    // the shard's own K range is chunks [0, P/T) of width K/P
    GemmArgs g = make_args(p, Xt, ldx, Wt, ldw, Pt, ldp, M, N, Kt, 1);
    g.wt = wt;
    widen_for_roots(p, g, p.P / tp_shards);
    narrow_for_decode(p, g, p.P / tp_shards);
    return hip_status(launch_slice_gemm(p.tile, EPI_STORE, g, p.P / tp_shards, hs));
}

}  // namespace

extern "C" {

detred_status tree_tp_gemm(const uint16_t* X, int ldx, const uint16_t* W, int ldw, float* Y,
                           int ldy, int M, int N, int K, int tp_shards, void* ws, size_t ws_bytes,
                           detred_stream s)
{
    return tree_tp_impl(X, ldx, W, ldw, false, Y, ldy, M, N, K, tp_shards, ws, ws_bytes, s);
}

detred_status tree_tp_gemm_wt(const uint16_t* X, int ldx, const uint16_t* Wt, int ldwt, float* Y,
                              int ldy, int M, int N, int K, int tp_shards, void* ws,
                              size_t ws_bytes, detred_stream s)
{
    return tree_tp_impl(X, ldx, Wt, ldwt, true, Y, ldy, M, N, K, tp_shards, ws, ws_bytes, s);
}

detred_status tree_tp_shards_gemm(const uint16_t* X, int ldx, const uint16_t* W, int ldw, float* P,
                                  int M, int N, int K, int tp_shards, detred_stream s)
{
    return tree_tp_shards_impl(X, ldx, W, ldw, false, P, M, N, K, tp_shards, s);
}

detred_status tree_tp_shards_gemm_wt(const uint16_t* X, int ldx, const uint16_t* Wt, int ldwt,
                                     float* P, int M, int N, int K, int tp_shards, detred_stream s)
{
    return tree_tp_shards_impl(X, ldx, Wt, ldwt, true, P, M, N, K, tp_shards, s);
}

detred_status tree_tp_shard_gemm(const uint16_t* Xt, int ldx, const uint16_t* Wt, int ldw,
                                 float* Pt, int ldp, int M, int N, int Kt, int tp_shards,
                                 detred_stream s)
{
    return tree_tp_shard_impl(Xt, ldx, Wt, ldw, false, Pt, ldp, M, N, Kt, tp_shards, s);
}

detred_status tree_tp_shard_gemm_wt(const uint16_t* Xt, int ldx, const uint16_t* Wtt, int ldwt,
                                    float* Pt, int ldp, int M, int N, int Kt, int tp_shards,
                                    detred_stream s)
{
    return tree_tp_shard_impl(Xt, ldx, Wtt, ldwt, true, Pt, ldp, M, N, Kt, tp_shards, s);
}

detred_status tree_combine_f32(const float* parts, size_t part_stride, int count, float* Y,
                               size_t n, detred_stream s)
{
    if (!pow2_le8(count))
        return DETRED_EUNSUPPORTED;
    if (n == 0)
        return DETRED_OK;
    if (!parts || !Y || !aligned16(parts) || !aligned16(Y) || (n % 4) != 0 ||
        (part_stride % 4) != 0 || (count > 1 && part_stride < n))
        return DETRED_EINVAL;
    return hip_status(launch_tree_combine(parts, part_stride, count, Y, n, (hipStream_t)s));
}

detred_status detred_f32_to_bf16(const float* x, uint16_t* y, size_t n, detred_stream s)
{
    if (n == 0)
        return DETRED_OK;
    if (!x || !y || !aligned16(x) || !aligned16(y))
        return DETRED_EINVAL;
    if ((n % 8) != 0)
        return DETRED_EUNSUPPORTED;
    return hip_status(launch_cast_bf16(x, y, n, (hipStream_t)s));
}

detred_status inv_rmsnorm(const uint16_t* x, const uint16_t* gamma, float* y, int rows, int hidden,
                          float eps, detred_stream s)
{
    if (rows < 0 || hidden < 0)
        return DETRED_EINVAL;
    if (rows == 0)
        return DETRED_OK;
    if (!x || !gamma || !y || !aligned16(x) || !aligned16(gamma) || !aligned16(y))
        return DETRED_EINVAL;
    if (hidden == 0 || hidden % 8 != 0 || hidden > 65536)
        return DETRED_EUNSUPPORTED;
    return hip_status(launch_rmsnorm(x, gamma, y, rows, hidden, eps, (hipStream_t)s));
}

detred_status inv_rmsnorm_bf16(const uint16_t* x, const uint16_t* gamma, uint16_t* y, int rows,
                               int hidden, float eps, detred_stream s)
{
    if (rows < 0 || hidden < 0)
        return DETRED_EINVAL;
    if (rows == 0)
        return DETRED_OK;
    if (!x || !gamma || !y || !aligned16(x) || !aligned16(gamma) || !aligned16(y))
        return DETRED_EINVAL;
    if (hidden == 0 || hidden % 8 != 0 || hidden > 65536)
        return DETRED_EUNSUPPORTED;
    return hip_status(launch_rmsnorm_bf16(x, gamma, y, rows, hidden, eps, (hipStream_t)s));
}

detred_status inv_log_softmax(const float* x, float* y, int rows, int cols, detred_stream s)
{
    if (rows < 0 || cols < 0)
        return DETRED_EINVAL;
    if (rows == 0)
        return DETRED_OK;
    if (!x || !y || !aligned16(x) || !aligned16(y))
        return DETRED_EINVAL;
    if (cols == 0 || cols % 4 != 0)
        return DETRED_EUNSUPPORTED;
    return hip_status(launch_log_softmax(x, y, rows, cols, (hipStream_t)s));
}

detred_status inv_log_softmax_mean(const float* x, float* y, float* mu, int rows, int cols,
                                   detred_stream s)
{
    if (rows < 0 || cols < 0)
        return DETRED_EINVAL;
    if (rows == 0)
        return DETRED_OK;
    if (!x || !y || !mu || !aligned16(x) || !aligned16(y) || ((uintptr_t)mu & 3u))
        return DETRED_EINVAL;
    if (cols == 0 || cols % 4 != 0)
        return DETRED_EUNSUPPORTED;
    return hip_status(launch_log_softmax_mean(x, y, mu, rows, cols, (hipStream_t)s));
}

detred_status inv_mean(const float* x, float* y, int rows, int cols, detred_stream s)
{
    if (rows < 0 || cols < 0)
        return DETRED_EINVAL;
    if (rows == 0)
        return DETRED_OK;
    if (!x || !y || !aligned16(x))
        return DETRED_EINVAL;
    if (cols == 0 || cols % 4 != 0)
        return DETRED_EUNSUPPORTED;
    return hip_status(launch_mean(x, y, rows, cols, (hipStream_t)s));
}

size_t inv_decode_attention_workspace_bytes(int B, int Hq, int D, int max_len)
{
    if (B < 0 || Hq <= 0 || D <= 0 || max_len < 0)
        return 0;
    const size_t nch = ((size_t)max_len + attention_chunk() - 1) / attention_chunk();
    const size_t rows = (size_t)B * Hq * nch;
    return round_up(rows * D * sizeof(float), 256) + round_up(rows * 2 * sizeof(float), 256);
}

detred_status inv_decode_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                   long kv_stride_b, long kv_stride_h, long kv_stride_t,
                                   const int* lens, float* out, int B, int Hq, int Hkv, int D,
                                   int max_len, float scale, void* ws, size_t ws_bytes,
                                   detred_stream s)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || max_len < 0 || Hq % Hkv != 0)
        return DETRED_EINVAL;
    if (D != 64 && D != 128)
        return DETRED_EUNSUPPORTED;
    if (Hq / Hkv > 16)
        return DETRED_EUNSUPPORTED;
    if (B == 0)
        return DETRED_OK;
    if (!q || !k || !v || !lens || !out || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
        ((uintptr_t)lens & 3u) != 0 || ((uintptr_t)q & 1u) != 0)
        return DETRED_EINVAL;
    if (kv_stride_b < 0 || kv_stride_h < 0 || kv_stride_t < 0 || kv_stride_b % 8 != 0 ||
        kv_stride_h % 8 != 0 || kv_stride_t % 8 != 0)
        return DETRED_EINVAL;
    const int chunk = attention_chunk();
    const size_t nch = ((size_t)max_len + chunk - 1) / chunk;
    if ((size_t)B * Hkv * nch >= ((size_t)1 << 31) || (size_t)B * Hq >= ((size_t)1 << 31))
        return DETRED_EUNSUPPORTED;
    const size_t need = inv_decode_attention_workspace_bytes(B, Hq, D, max_len);
    if (!ws || !aligned256(ws) || ws_bytes < need)
        return DETRED_EWORKSPACE;
    AttnArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.sb = kv_stride_b;
    a.sh = kv_stride_h;
    a.st = kv_stride_t;
    a.lens = lens;
    a.out = out;
    a.part_o = (float*)ws;
    a.part_ml = (float*)((char*)ws + round_up((size_t)B * Hq * nch * D * sizeof(float), 256));
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = Hq / Hkv;
    a.D = D;
    a.max_len = max_len;
    a.nch = (int)nch;
    a.scale = scale;
    return hip_status(launch_decode_attention(a, (hipStream_t)s));
}

}  // extern "C"
