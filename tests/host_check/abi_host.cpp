// Host-only check of the C-ABI layer (csrc/api.cpp), built with g++ and
// AddressSanitizer + UndefinedBehaviorSanitizer against stub launchers: no
// GPU code runs.  Every launcher the ABI layer calls is replaced by one
// that records what it was asked to launch, so the checks cover
//  * argument validation of every entry point (the status of each bad call,
//    and that a rejected call launches nothing);
//  * the planner: which tile, chunks per slice and grid a call would
//    launch, including where the tile and the split change with M;
//  * the workspace layout: partial planes and arrival counters inside the
//    caller's buffer, for the split products, the LoRA layer and the
//    no-allocation entry point;
//  * size arithmetic at very large dimensions (UBSan traps on overflow).
// Exit status 0 when every check passes; the failures are printed.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <string>
#include <vector>

#include "detred.h"
#include "kernels.h"

using namespace detred;

// ---- recording stubs -------------------------------------------------------

struct Launch {
    std::string kind;
    int tile = -1, epi = -1, cps = 0, count = 0;
    GemmArgs g{};
    const void* a = nullptr;  // first buffer argument (parts, x, ...)
    const void* b = nullptr;  // output
    size_t n = 0;
};
static std::vector<Launch> launches;
static const int kScratchFake = 0x40000000;  // stand-in device address of the no-alloc scratch

namespace detred {

void tile_shape(int tile, int* bm, int* bn)
{
    switch (tile) {
    case TILE_S16: *bm = 64; *bn = 16; return;
    case TILE_M64: *bm = 64; *bn = 64; return;
    case TILE_L256: *bm = 256; *bn = 256; return;
    case TILE_D64: *bm = 64; *bn = 128; return;
    case TILE_W256: *bm = 192; *bn = 128; return;
    default: *bm = 128; *bn = 128; return;
    }
}
bool lds_engine_supports(int tile, const GemmArgs& g, int cps)
{
    if (g.Kc % 32 != 0)
        return false;
    if (tile == TILE_L256 && cps != 1)
        return false;
    if (tile == TILE_W256 && (cps != 8 || g.Kc % 64 != 0 || g.out_z_stride != 0 ||
                              (g.epi && g.out_bf16)))
        return false;
    return true;
}
hipError_t launch_slice_gemm(int tile, int epi, const GemmArgs& g, int cps, hipStream_t)
{
    Launch l;
    l.kind = "gemm";
    l.tile = tile;
    l.epi = epi;
    l.cps = cps;
    l.g = g;
    launches.push_back(l);
    return hipSuccess;
}
hipError_t launch_tree_combine(const float* parts, size_t stride, int count, float* Y, size_t n,
                               hipStream_t)
{
    Launch l;
    l.kind = "combine";
    l.a = parts;
    l.b = Y;
    l.n = n;
    l.count = count;
    (void)stride;
    launches.push_back(l);
    return hipSuccess;
}
hipError_t launch_tree_combine_rows(const float* parts, size_t, int count, const GemmArgs& g,
                                    hipStream_t)
{
    Launch l;
    l.kind = "combine_rows";
    l.a = parts;
    l.count = count;
    l.g = g;
    launches.push_back(l);
    return hipSuccess;
}
hipError_t launch_fill_zero(float* Y, long, int M, int N, hipStream_t)
{
    Launch l;
    l.kind = "fill";
    l.b = Y;
    l.n = (size_t)M * N;
    launches.push_back(l);
    return hipSuccess;
}
hipError_t launch_cast_bf16(const float* x, uint16_t* y, size_t n, hipStream_t)
{
    Launch l;
    l.kind = "cast";
    l.a = x;
    l.b = y;
    l.n = n;
    launches.push_back(l);
    return hipSuccess;
}
hipError_t noalloc_scratch(hipStream_t, void** ptr)
{
    *ptr = (void*)(uintptr_t)kScratchFake;
    return hipSuccess;
}
static hipError_t rec(const char* kind)
{
    Launch l;
    l.kind = kind;
    launches.push_back(l);
    return hipSuccess;
}
hipError_t launch_rmsnorm(const uint16_t*, const uint16_t*, float*, int, int, float, hipStream_t)
{
    return rec("rmsnorm");
}
hipError_t launch_rmsnorm_bf16(const uint16_t*, const uint16_t*, uint16_t*, int, int, float,
                               hipStream_t)
{
    return rec("rmsnorm_bf16");
}
hipError_t launch_epilogue_only(const GemmArgs&, hipStream_t) { return rec("epilogue"); }
int attention_chunk() { return 256; }
hipError_t launch_decode_attention(const AttnArgs&, hipStream_t) { return rec("attention"); }
hipError_t launch_log_softmax(const float*, float*, int, int, hipStream_t)
{
    return rec("log_softmax");
}
hipError_t launch_log_softmax_mean(const float*, float*, float*, int, int, hipStream_t)
{
    return rec("log_softmax_mean");
}
hipError_t launch_mean(const float*, float*, int, int, hipStream_t) { return rec("mean"); }

}  // namespace detred

extern "C" hipError_t hipMemsetAsync(void*, int, size_t, hipStream_t) { return rec("memset"); }

// ---- checks ----------------------------------------------------------------

static int failures = 0;
#define CHECK(cond)                                                              \
    do {                                                                         \
        if (!(cond)) {                                                           \
            printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);               \
            ++failures;                                                          \
        }                                                                        \
    } while (0)

// Fake, 256-byte aligned device addresses; never dereferenced.
static const uint16_t* X = (const uint16_t*)(uintptr_t)0x100000;
static const uint16_t* W = (const uint16_t*)(uintptr_t)0x200000;
static float* Y = (float*)(uintptr_t)0x300000;
static const uint16_t* MIS = (const uint16_t*)(uintptr_t)0x100002;

static int det(int M, int N, int K, int S, void* ws = nullptr, size_t nws = 0, int ldx = -1,
               int ldw = -1, int ldy = -1)
{
    return det_splitk_gemm(X, ldx < 0 ? K : ldx, W, ldw < 0 ? N : ldw, Y, ldy < 0 ? N : ldy, M, N,
                           K, S, ws, nws, nullptr);
}

// the single GEMM launch of an unsplit det call
static Launch plan1(int M, int N, int K)
{
    launches.clear();
    CHECK(det(M, N, K, 1) == DETRED_OK);
    CHECK(launches.size() == 1);
    return launches.empty() ? Launch() : launches[0];
}

static void check_validation()
{
    // det_splitk_gemm: every rejection launches nothing
    struct Case {
        int M, N, K, S, ldx, ldw, ldy;
        const uint16_t* x;
        detred_status want;
    } cases[] = {
        {-1, 16, 512, 8, 512, 16, 16, X, DETRED_EINVAL},
        {16, 16, -8, 8, 512, 16, 16, X, DETRED_EINVAL},
        {16, 16, 512, 8, 100, 16, 16, X, DETRED_EINVAL},   // ldx < K
        {16, 16, 512, 8, 512, 8, 16, X, DETRED_EINVAL},    // ldw < N
        {16, 16, 512, 8, 512, 16, 8, X, DETRED_EINVAL},    // ldy < N
        {16, 16, 512, 8, 512, 16, 16, nullptr, DETRED_EINVAL},
        {16, 16, 512, 8, 512, 16, 16, MIS, DETRED_EINVAL},
        {16, 16, 512, 8, 516, 16, 16, X, DETRED_EINVAL},   // ldx % 8
        {16, 16, 500, 8, 504, 16, 16, X, DETRED_EUNSUPPORTED},  // K % 8
        {16, 12, 512, 8, 512, 16, 16, X, DETRED_EUNSUPPORTED},  // N % 8
        {16, 16, 512, 3, 512, 16, 16, X, DETRED_EUNSUPPORTED},
        {16, 16, 512, 16, 512, 16, 16, X, DETRED_EUNSUPPORTED},
        {16, 16, 264, 2, 264, 16, 16, X, DETRED_EUNSUPPORTED},  // one chunk
        {16, 16, 512, 8, 512, 16, 16, X, DETRED_EWORKSPACE},    // no workspace
    };
    for (const Case& c : cases) {
        launches.clear();
        const detred_status st = det_splitk_gemm(c.x, c.ldx, W, c.ldw, Y, c.ldy, c.M, c.N, c.K,
                                                 c.S, nullptr, 0, nullptr);
        if (st != c.want)
            printf("  case M=%d N=%d K=%d S=%d ld=%d/%d/%d: got %d want %d\n", c.M, c.N, c.K, c.S,
                   c.ldx, c.ldw, c.ldy, (int)st, (int)c.want);
        CHECK(st == c.want);
        CHECK(launches.empty());
    }
    // a workspace too small, or not 256-byte aligned
    const size_t need = detred_gemm_workspace_bytes(16, 16, 512, 8);
    CHECK(need >= 8 * 16 * 16 * 4 + 4 && need % 256 == 0);
    launches.clear();
    CHECK(det(16, 16, 512, 8, (void*)(uintptr_t)0x400000, need - 1) == DETRED_EWORKSPACE);
    CHECK(det(16, 16, 512, 8, (void*)(uintptr_t)0x400010, need) == DETRED_EWORKSPACE);
    CHECK(launches.empty());
    // empty problems launch nothing; K == 0 writes zeros
    launches.clear();
    CHECK(det_splitk_gemm(nullptr, 8, nullptr, 8, nullptr, 8, 0, 8, 8, 8, nullptr, 0, nullptr) ==
          DETRED_OK);
    CHECK(launches.empty());
    CHECK(det(16, 16, 0, 1) == DETRED_OK);
    CHECK(launches.size() == 1 && launches[0].kind == "fill");

    // the other entry points
    float* f = Y;
    CHECK(atomic_splitk_gemm(X, 512, W, 16, Y, 16, 16, 16, 512, 5, nullptr) ==
          DETRED_EUNSUPPORTED);
    CHECK(tree_tp_gemm(X, 512, W, 16, Y, 16, 16, 16, 512, 3, nullptr, 0, nullptr) ==
          DETRED_EUNSUPPORTED);
    CHECK(tree_tp_gemm(X, 512, W, 16, Y, 16, 16, 16, 512, 4, nullptr, 0, nullptr) ==
          DETRED_EWORKSPACE);
    CHECK(tree_tp_shards_gemm(nullptr, 512, W, 16, Y, 16, 16, 512, 2, nullptr) == DETRED_EINVAL);
    CHECK(tree_tp_shard_gemm(X, 64, W, 16, Y, 16, 16, 16, 64, 6, nullptr) == DETRED_EINVAL);
    CHECK(tree_tp_shard_gemm(X, 40, W, 16, Y, 16, 16, 16, 40, 2, nullptr) == DETRED_EUNSUPPORTED);
    CHECK(tree_combine_f32(f, 16, 3, f + 1024, 16, nullptr) == DETRED_EUNSUPPORTED);
    CHECK(tree_combine_f32(f, 8, 2, f + 1024, 16, nullptr) == DETRED_EINVAL);
    CHECK(detred_f32_to_bf16(f, (uint16_t*)X, 12, nullptr) == DETRED_EUNSUPPORTED);
    CHECK(inv_rmsnorm(X, W, f, 4, 4100, 1e-6f, nullptr) == DETRED_EUNSUPPORTED);
    CHECK(inv_rmsnorm(X, nullptr, f, 4, 4096, 1e-6f, nullptr) == DETRED_EINVAL);
    CHECK(inv_log_softmax(f, f, 4, 6, nullptr) == DETRED_EUNSUPPORTED);
    CHECK(inv_mean(nullptr, f, 4, 8, nullptr) == DETRED_EINVAL);
    CHECK(inv_log_softmax_mean(f, f, (float*)((char*)f + 2), 4, 8, nullptr) == DETRED_EINVAL);
    CHECK(det_splitk_addmm(X, 512, W, 16, f, 16, 1.f, 1.f, Y, 16, 2, 16, 16, 512, 1, nullptr, 0,
                           nullptr) == DETRED_EINVAL);
    CHECK(det_splitk_addmm(X, 512, W, 16, f, 8, 1.f, 1.f, Y, 16, DETRED_F32, 16, 16, 512, 1,
                           nullptr, 0, nullptr) == DETRED_EINVAL);  // ldc < N
    CHECK(det_lora_forward(X, 512, W, 64, W, 16, W, 64, 1.f, (uint16_t*)Y, 64, 16, 64, 512, 12,
                           nullptr, 0, nullptr) == DETRED_EUNSUPPORTED);  // r % 8
    CHECK(det_lora_forward(X, 512, W, 64, W, 16, W, 64, 1.f, (uint16_t*)Y, 64, 16, 64, 512, 16,
                           nullptr, 0, nullptr) == DETRED_EWORKSPACE);
    CHECK(inv_decode_attention(X, W, W, 0, 0, 0, (const int*)f, f, 2, 8, 2, 96, 100, 1.f, nullptr,
                               0, nullptr) == DETRED_EUNSUPPORTED);  // D
    CHECK(detred_workspace_init(nullptr, 16, nullptr) == DETRED_EINVAL);
    CHECK(strcmp(detred_status_string(DETRED_OK), "DETRED_OK") == 0);
    CHECK(strncmp(detred_status_string((detred_status)99), "DETRED_UNKNOWN", 14) == 0);
}

static void check_planner()
{
    // decode / small batches: the 64x128 tile up to 64 rows, then 128x128
    Launch l = plan1(64, 4096, 4096);
    CHECK(l.tile == TILE_D64 && l.cps == 8 && l.g.tiles_m == 1);
    l = plan1(65, 4096, 4096);
    CHECK(l.tile == TILE_L128 && l.g.tiles_m == 1);
    // an unsplit eight-chunk product takes the 192x128 tile where 1.25 x its
    // rounds of workgroups over 256 CUs do not exceed the 128x128 tile's:
    // 512 rows of 14336 columns take 2 rounds either way, 513 take 3 on
    // 128x128 and 2 on 192x128; 1024 rows of 4096 take 1 either way, 1025
    // take 2 and 1
    l = plan1(512, 14336, 4096);
    CHECK(l.tile == TILE_L128 && l.g.tiles_m == 4 && l.g.tiles_n == 112);
    l = plan1(513, 14336, 4096);
    CHECK(l.tile == TILE_W256 && l.g.tiles_m == 3 && l.g.tiles_n == 112 && l.cps == 8);
    l = plan1(1024, 4096, 4096);
    CHECK(l.tile == TILE_L128 && l.g.tiles_m == 8 && l.g.tiles_n == 32);
    l = plan1(1025, 4096, 4096);
    CHECK(l.tile == TILE_W256 && l.g.tiles_m == 6 && l.g.tiles_n == 32);
    l = plan1(1280, 14336, 4096);   // 5 rounds on 128x128, 4 on 192x128: 5 <= 5
    CHECK(l.tile == TILE_W256 && l.g.tiles_m == 7);
    l = plan1(4096, 14336, 4096);
    CHECK(l.tile == TILE_W256 && l.g.tiles_m == 22);
    // ...but not for one-chunk K, nor for a bf16 addmm output, nor when C
    // overlaps Y
    l = plan1(2048, 4096, 264);
    CHECK(l.tile != TILE_W256 && l.cps == 1);
    launches.clear();
    CHECK(det_splitk_addmm(X, 4096, W, 4096, nullptr, 0, 1.f, 0.f, Y, 4096, DETRED_BF16, 1280,
                           4096, 4096, 1, nullptr, 0, nullptr) == DETRED_OK);
    CHECK(launches.size() == 1 && launches[0].tile == TILE_L128);
    launches.clear();
    CHECK(det_splitk_addmm(X, 4096, W, 4096, Y, 4096, 1.f, 1.f, Y, 4096, DETRED_F32, 1280, 4096,
                           4096, 1, nullptr, 0, nullptr) == DETRED_OK);
    CHECK(launches.size() == 1 && launches[0].tile == TILE_L128);
    launches.clear();
    CHECK(det_splitk_addmm(X, 4096, W, 4096, Y + 1280 * 4096, 4096, 1.f, 1.f, Y, 4096, DETRED_F32,
                           1280, 4096, 4096, 1, nullptr, 0, nullptr) == DETRED_OK);
    CHECK(launches.size() == 1 && launches[0].tile == TILE_W256);
    // narrow outputs: 64x16 while 64x64 would leave fewer than 256
    // workgroups, else 64x64
    static char ws_buf[1 << 16] __attribute__((aligned(256)));
    launches.clear();
    const size_t nws = detred_gemm_workspace_bytes(256, 64, 4096, 8);
    CHECK(det(256, 64, 4096, 8, ws_buf, nws) == DETRED_OK);
    CHECK(!launches.empty() && launches[0].tile == TILE_S16);
    // the automatic split keeps one slice where the 128x128 grid would take
    // 1.0-1.75 rounds and one round of 192x128 tiles holds the product
    // (384 x 14336: 336 tiles of 128x128, 224 of 192x128); an addmm into
    // bf16 cannot take that tile and keeps 2 slices, which the workspace of
    // split 0 covers
    {
        void* big = (void*)(uintptr_t)0x40000000;
        const size_t nbig = detred_gemm_workspace_bytes(384, 14336, 4096, 0);
        CHECK(nbig == detred_gemm_workspace_bytes(384, 14336, 4096, 2));
        CHECK(detred_auto_split(384, 14336, 4096) == 1);
        launches.clear();
        CHECK(det(384, 14336, 4096, 0, big, nbig) == DETRED_OK);
        CHECK(launches.size() == 1 && launches[0].tile == TILE_W256 && launches[0].cps == 8);
        launches.clear();
        CHECK(det_splitk_addmm(X, 4096, W, 14336, nullptr, 0, 1.f, 0.f, Y, 14336, DETRED_BF16, 384,
                               14336, 4096, 0, big, nbig, nullptr) == DETRED_OK);
        CHECK(!launches.empty() && launches[0].tile == TILE_L128 && launches[0].cps == 4 &&
              launches[0].g.slices == 2);
    }
    // the automatic split: 8 slices for chunks of 1792 with 256+ rows (on
    // the 256x256 root tile), none at 4096 x 14336 x 4096
    CHECK(detred_auto_split(256, 8192, 14336) == 8);
    CHECK(detred_auto_split(255, 8192, 14336) != 8);
    CHECK(detred_auto_split(4096, 14336, 4096) == 1);
    // shard roots of one-chunk slices: 256x256 from 256 rows at chunks of
    // 1024 or more, 128x128 below
    launches.clear();
    CHECK(tree_tp_shards_gemm(X, 8192, W, 8192, Y, 256, 8192, 8192, 8, nullptr) == DETRED_OK);
    CHECK(launches.size() == 1 && launches[0].tile == TILE_L256 && launches[0].cps == 1 &&
          launches[0].g.slices == 8);
    launches.clear();
    CHECK(tree_tp_shards_gemm(X, 8192, W, 8192, Y, 255, 8192, 8192, 8, nullptr) == DETRED_OK);
    CHECK(launches.size() == 1 && launches[0].tile == TILE_L128);
}

static void check_workspace_layout()
{
    // two-launch split: S root planes at ws, then a combine over them
    static char big[(8 << 20) + 4096] __attribute__((aligned(256)));
    const size_t nws = detred_gemm_workspace_bytes(64, 4096, 4096, 4);
    CHECK(nws > 0 && nws <= sizeof(big));
    launches.clear();
    CHECK(det(64, 4096, 4096, 4, big, nws) == DETRED_OK);
    CHECK(launches.size() == 2 && launches[1].kind == "combine" && launches[1].count == 4);
    if (launches.size() == 2) {
        const Launch& r = launches[0];
        CHECK(r.epi == EPI_STORE && r.cps == 2 && (char*)r.g.Y == big &&
              r.g.out_z_stride == 64L * 4096);
        CHECK((char*)r.g.Y + 4 * r.g.out_z_stride * sizeof(float) <= big + nws);
    }
    // one-launch split of a small narrow output: partials then counters,
    // both inside ws
    const size_t n2 = detred_gemm_workspace_bytes(16, 16, 512, 8);
    launches.clear();
    CHECK(det(16, 16, 512, 8, big, n2) == DETRED_OK);
    CHECK(launches.size() == 1 && launches[0].epi == EPI_COMBINE);
    if (launches.size() == 1) {
        const GemmArgs& g = launches[0].g;
        CHECK((char*)g.part == big);
        CHECK((char*)g.counters >= big + 8 * 16 * 16 * 4 &&
              (char*)(g.counters + g.tiles_m * g.tiles_n) <= big + n2);
    }
    // the no-allocation entry point: counters at the scratch's start, the
    // partials after them
    launches.clear();
    CHECK(det_splitk_gemm_noalloc(X, 512, W, 16, Y, 16, 16, 16, 512, 8, nullptr) == DETRED_OK);
    CHECK(launches.size() == 1 && launches[0].epi == EPI_COMBINE);
    if (launches.size() == 1) {
        CHECK((uintptr_t)launches[0].g.counters == (uintptr_t)kScratchFake);
        CHECK((uintptr_t)launches[0].g.part == (uintptr_t)kScratchFake + 65536);
    }
    launches.clear();
    CHECK(det_splitk_gemm_noalloc(X, 4096, W, 4096, Y, 4096, 4096, 4096, 4096, 8, nullptr) ==
          DETRED_EWORKSPACE);
    CHECK(launches.empty());
    // the LoRA layer: every launch's buffers inside its workspace
    const size_t nl = det_lora_workspace_bytes(64, 1024, 4096, 16);
    CHECK(nl > 0 && nl <= sizeof(big));
    launches.clear();
    CHECK(det_lora_forward(X, 4096, W, 1024, W, 16, W, 1024, 2.f, (uint16_t*)Y, 1024, 64, 1024,
                           4096, 16, big, nl, nullptr) == DETRED_OK);
    CHECK(launches.size() >= 3);
    for (const Launch& l : launches) {
        if (l.kind != "gemm")
            continue;
        const char* p = (const char*)l.g.part;
        if (p)
            CHECK(p >= big && p < big + nl);
        if (l.g.out_z_stride)
            CHECK((const char*)l.g.Y >= big && (const char*)l.g.Y < big + nl);
    }
}

static void check_large_sizes()
{
    // sizes far past any buffer: the arithmetic stays in size_t (UBSan
    // traps signed overflow), and nothing launches for what is rejected
    const size_t b = detred_gemm_workspace_bytes(1 << 30, 1 << 20, 4096, 8);
    CHECK(b >= (size_t)8 * ((size_t)1 << 30) * ((size_t)1 << 20) * 4);
    CHECK(detred_gemm_workspace_bytes(0x7fffffff, 0x7ffffff8, 4096, 2) > 0);
    CHECK(det_lora_workspace_bytes(1 << 30, 1 << 20, 4096, 64) > 0);
    CHECK(inv_decode_attention_workspace_bytes(1 << 20, 128, 128, 1 << 30) > 0);
    launches.clear();
    // a split whose tile rows do not fit 32-bit offsets
    CHECK(det(16, 1 << 24, 4096, 8, (void*)(uintptr_t)0x1000000000, (size_t)1 << 40) ==
          DETRED_EUNSUPPORTED);
    CHECK(launches.empty());
}

int main()
{
    check_validation();
    check_planner();
    check_workspace_layout();
    check_large_sizes();
    if (failures) {
        printf("%d check(s) failed\n", failures);
        return 1;
    }
    printf("host ABI checks passed\n");
    return 0;
}
