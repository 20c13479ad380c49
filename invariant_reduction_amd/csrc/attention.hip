// Batch-invariant decode attention for gfx950 with a fixed-size KV split.
//
// Attention reduces over the KV cache, and a split of that reduction whose
// pieces depend on the batch (or on the number of CUs) changes the order of
// the sums; a split into pieces of one fixed size keeps it ("Restoring AI
// Reproducibility: Thinking Machines Lab's Challenge to Overcome
// Nondeterminism", 2-3 and 3-2).  Here the positions of every sequence are
// cut into chunks of CHUNK = 256, fixed; nothing else enters the order:
//
//   chunk pass, one workgroup per (sequence b, KV head h, chunk j), for the
//   G = Hq/Hkv query heads of h:
//     s_t   = (sum over d of q_d * k_td) * scale: per position, D/8 lanes
//             each take 8 consecutive d in a fused multiply-add chain, then
//             a fixed tree of DPP adds over those lanes, read from the first;
//     m_j   = max of s_t over the chunk (exact);
//     p_t   = exp(s_t - m_j);   l_j = sum of p_t (per lane 4 positions in
//             order, then a wave butterfly);
//     o_j,d = sum of p_t * v_td (per lane its positions in increasing order,
//             then butterflies over the lanes of a wave, then
//             (w0 + w1) + (w2 + w3) over the four waves);
//   fold pass, one workgroup per (b, query head): the chunk results in
//     chunk order, (M, L, O) <- (max(M, m_j), L*a + l_j*c, O*a + o_j*c) with
//     a = exp(M - max), c = exp(m_j - max); out = O / L.
//
// Decode attention reads every key and value once for a handful of query
// rows, so it is bound by HBM, not by arithmetic: the products run on fp32
// VALU lanes (no MFMA reshaping), and each key or value row is read as
// 16-byte pieces by consecutive lanes.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "kernels.h"

namespace detred {
namespace attn {

constexpr int CHUNK = 256;
constexpr int THREADS = 256;
static_assert(CHUNK == 4 * 64, "the softmax pass gives each lane four positions");

__device__ __forceinline__ float bf16_f32(uint32_t bits) { return __uint_as_float(bits << 16); }

// Cross-lane moves within a row of 16 lanes (DPP): a rotation of the row,
// a mirror of each half row, and two quad permutations.
template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int DPP_ROW_ROR8 = 0x128, DPP_ROW_ROR4 = 0x124, DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_QUAD_XOR2 = 0x4e, DPP_QUAD_XOR1 = 0xb1;

// Sum over the DG consecutive lanes holding one position's pieces (DG = 16:
// a row; DG = 8: a half row), a fixed tree; the first lane of the group
// holds the result.  16 lanes: ror 8, ror 4, then lanes xor 2, xor 1;
// 8 lanes: mirror, then xor 2, xor 1.
template <int DG>
__device__ __forceinline__ float group_sum(float v)
{
    static_assert(DG == 8 || DG == 16, "8 or 16 lanes per position");
    if constexpr (DG == 16) {
        v = v + dpp<DPP_ROW_ROR8>(v);
        v = v + dpp<DPP_ROW_ROR4>(v);
    } else {
        v = v + dpp<DPP_ROW_HALF_MIRROR>(v);
    }
    v = v + dpp<DPP_QUAD_XOR2>(v);
    v = v + dpp<DPP_QUAD_XOR1>(v);
    return v;
}

__device__ __forceinline__ void unpack8(const uint4 q, float (&f)[8])
{
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}

// GM: the query-head group size rounded up to 4, 8 or 16 (heads g >= G of
// the group are skipped).
template <int D, int GM>
__global__ __launch_bounds__(THREADS) void chunk_kernel(AttnArgs a)
{
    constexpr int DG = D / 8;          // 16-byte pieces per key/value row
    constexpr int TPI = THREADS / DG;  // positions per pass over the workgroup
    constexpr int ITER = CHUNK / TPI;
    static_assert(DG <= 64 && 64 % DG == 0, "a position's pieces lie in one wave");
    __shared__ float qs[GM][D];
    __shared__ float sc[GM][CHUNK];
    __shared__ float red[THREADS / 64][GM][D];
    __shared__ float mls[GM][2];

    const int j = blockIdx.x % a.nch;
    const int bh = blockIdx.x / a.nch;
    const int b = bh / a.Hkv, h = bh % a.Hkv;
    int len = a.lens[b];
    len = len < a.max_len ? len : a.max_len;
    const int t0 = j * CHUNK;
    if (t0 >= len)
        return;  // a chunk past the sequence (the whole workgroup leaves)
    const int nv = (len - t0) < CHUNK ? (len - t0) : CHUNK;
    const int G = a.G;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    for (int e = tid; e < GM * D; e += THREADS) {
        const int g = e / D, d = e % D;
        qs[g][d] = g < G ? bf16_f32(a.q[((size_t)b * a.Hq + (size_t)h * G + g) * D + d]) : 0.0f;
    }
    __syncthreads();

    const size_t base = (size_t)b * a.sb + (size_t)h * a.sh + (size_t)t0 * a.st;
    const uint16_t* kb = a.k + base;
    const uint16_t* vb = a.v + base;
    const int dg = tid % DG, tl = tid / DG;

    // this thread's 8 query dimensions of every head, in registers when
    // they fit
    constexpr bool QREG = GM <= 8;
    float qr[QREG ? GM : 1][8];
    if constexpr (QREG) {
#pragma unroll
        for (int g = 0; g < GM; ++g)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                qr[g][e] = qs[g][dg * 8 + e];
    }
    // scores, in two batches: all key pieces of a batch are loaded before
    // its products
    constexpr int IB = ITER / 2;
#pragma unroll
    for (int h0 = 0; h0 < ITER; h0 += IB) {
        uint4 kq[IB];
#pragma unroll
        for (int r = 0; r < IB; ++r) {
            const int t = (h0 + r) * TPI + tl;
            kq[r] = t < nv ? *reinterpret_cast<const uint4*>(kb + (size_t)t * a.st + dg * 8)
                           : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int r = 0; r < IB; ++r) {
            const int t = (h0 + r) * TPI + tl;
            float kf[8];
            unpack8(kq[r], kf);
            float part[GM];
#pragma unroll
            for (int g = 0; g < GM; ++g) {
                float s = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    s = fmaf(QREG ? qr[QREG ? g : 0][e] : qs[g][dg * 8 + e], kf[e], s);
                part[g] = group_sum<DG>(s);
            }
            if (dg == 0) {
#pragma unroll
                for (int g = 0; g < GM; ++g)
                    sc[g][t] = t < nv ? part[g] * a.scale : -INFINITY;
            }
        }
    }
    __syncthreads();

    // softmax of the chunk: wave w takes heads w, w+4, ...
    for (int g = wave; g < G; g += THREADS / 64) {
        float s4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            s4[i] = sc[g][lane + 64 * i];
        float m = fmaxf(fmaxf(s4[0], s4[1]), fmaxf(s4[2], s4[3]));
#pragma unroll
        for (int off = 32; off > 0; off >>= 1)
            m = fmaxf(m, __shfl_xor(m, off, 64));
        float ls = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float p = expf(s4[i] - m);  // exp(-inf) = 0 past the sequence
            sc[g][lane + 64 * i] = p;
            ls = ls + p;
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1)
            ls = ls + __shfl_xor(ls, off, 64);
        if (lane == 0) {
            mls[g][0] = m;
            mls[g][1] = ls;
        }
    }
    __syncthreads();

    // weighted sum of the value rows
    float acc[GM][8];
#pragma unroll
    for (int g = 0; g < GM; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc[g][e] = 0.0f;
    uint4 vq[ITER];
#pragma unroll
    for (int r = 0; r < ITER; ++r) {
        const int t = r * TPI + tl;
        vq[r] = t < nv ? *reinterpret_cast<const uint4*>(vb + (size_t)t * a.st + dg * 8)
                       : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int r = 0; r < ITER; ++r) {
        const int t = r * TPI + tl;
        float vf[8];
        unpack8(vq[r], vf);
#pragma unroll
        for (int g = 0; g < GM; ++g) {
            const float p = sc[g][t];  // 0 past the sequence
#pragma unroll
            for (int e = 0; e < 8; ++e)
                acc[g][e] = fmaf(p, vf[e], acc[g][e]);
        }
    }
    // lanes of a wave holding the same 8 dimensions: butterfly
#pragma unroll
    for (int off = DG; off < 64; off <<= 1)
#pragma unroll
        for (int g = 0; g < GM; ++g)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                acc[g][e] = acc[g][e] + __shfl_xor(acc[g][e], off, 64);
    if (lane < DG) {
#pragma unroll
        for (int g = 0; g < GM; ++g)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                red[wave][g][dg * 8 + e] = acc[g][e];
    }
    __syncthreads();

    const size_t row0 = (size_t)b * a.Hq + (size_t)h * G;  // first query head of the group
    for (int e = tid; e < G * D; e += THREADS) {
        const int g = e / D, d = e % D;
        const float o = (red[0][g][d] + red[1][g][d]) + (red[2][g][d] + red[3][g][d]);
        a.part_o[((row0 + g) * a.nch + j) * D + d] = o;
    }
    if (tid < G) {
        a.part_ml[((row0 + tid) * a.nch + j) * 2] = mls[tid][0];
        a.part_ml[((row0 + tid) * a.nch + j) * 2 + 1] = mls[tid][1];
    }
}

// One workgroup of D threads per (sequence, query head): fold the chunk
// results in chunk order and divide.
template <int D>
__global__ __launch_bounds__(D) void fold_kernel(AttnArgs a)
{
    const size_t bh = blockIdx.x;
    const int b = (int)(bh / a.Hq);
    int len = a.lens[b];
    len = len < a.max_len ? len : a.max_len;
    const int n = len > 0 ? (len + CHUNK - 1) / CHUNK : 0;
    const int d = threadIdx.x;
    if (n == 0) {
        a.out[bh * D + d] = 0.0f;
        return;
    }
    const float* ml = a.part_ml + bh * a.nch * 2;
    const float* po = a.part_o + bh * a.nch * D + d;
    float M = ml[0], L = ml[1], O = po[0];
    // FB chunks' results are loaded before they are folded, in chunk order
    constexpr int FB = 8;
    for (int j0 = 1; j0 < n; j0 += FB) {
        float mj[FB], lj[FB], oj[FB];
#pragma unroll
        for (int u = 0; u < FB; ++u) {
            const int jj = j0 + u < n ? j0 + u : n - 1;
            mj[u] = ml[2 * jj];
            lj[u] = ml[2 * jj + 1];
            oj[u] = po[(size_t)jj * D];
        }
#pragma unroll
        for (int u = 0; u < FB; ++u) {
            if (j0 + u < n) {
                const float Mn = fmaxf(M, mj[u]);
                const float ca = expf(M - Mn), cb = expf(mj[u] - Mn);
                L = L * ca + lj[u] * cb;
                O = O * ca + oj[u] * cb;
                M = Mn;
            }
        }
    }
    a.out[bh * D + d] = O / L;
}

template <int D, int GM>
hipError_t launch_chunks(const AttnArgs& a, hipStream_t s)
{
    const unsigned grid = (unsigned)((size_t)a.B * a.Hkv * a.nch);
    hipLaunchKernelGGL((chunk_kernel<D, GM>), dim3(grid), dim3(THREADS), 0, s, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const AttnArgs& a, hipStream_t s)
{
    if (a.nch > 0 && a.B > 0) {
        hipError_t e;
        if (a.G <= 4)
            e = launch_chunks<D, 4>(a, s);
        else if (a.G <= 8)
            e = launch_chunks<D, 8>(a, s);
        else
            e = launch_chunks<D, 16>(a, s);
        if (e != hipSuccess)
            return e;
    }
    if (a.B > 0)
        hipLaunchKernelGGL(fold_kernel<D>, dim3((unsigned)((size_t)a.B * a.Hq)), dim3(D), 0, s, a);
    return hipGetLastError();
}

}  // namespace attn

int attention_chunk() { return attn::CHUNK; }

hipError_t launch_decode_attention(const AttnArgs& a, hipStream_t s)
{
    return a.D == 64 ? attn::launch_d<64>(a, s) : attn::launch_d<128>(a, s);
}

}  // namespace detred
