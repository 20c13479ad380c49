// Batch-invariant row reductions for gfx950: RMSNorm, log_softmax, mean.
//
// One workgroup owns one row ("Restoring AI Reproducibility: Thinking
// Machines Lab's Challenge to Overcome Nondeterminism", 3-1: each batch
// element handled by one core and reduced in one consistent order).  The
// order of every reduction depends only on the row length:
//   1. thread t visits the 16-byte vectors t, t+NT, t+2NT, ... of the row in
//      that order and the elements of each vector left to right, keeping
//      one running binary32 value;
//   2. the 64 lanes of a wave are combined by a butterfly (xor 32,16,..,1);
//      addition is commutative, so every lane ends with the same bits;
//   3. the per-wave values are combined through LDS by a fixed butterfly.
// The batch size, the row's position and the launch never enter.
//
// Operations: RMSNorm (the article, 2-3); log_softmax and mean ("Batch
// Invariant Ops" project summary, Highlighted Details).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "bf16.h"
#include "kernels.h"

namespace detred {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1)
        v = v + __shfl_xor(v, off, 64);
    return v;
}

// Sum of one value per wave, identical on every thread of the block.
template <int NW>
__device__ __forceinline__ float block_sum(float v, float* red)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = wave_sum(v);
    if (lane == 0)
        red[wave] = v;
    __syncthreads();
    float t = (lane < NW) ? red[lane] : 0.0f;
#pragma unroll
    for (int off = NW / 2; off > 0; off >>= 1)
        t = t + __shfl_xor(t, off, 64);
    const float total = __shfl(t, 0, 64);
    __syncthreads();
    return total;
}

// ------------------------------------------------------------------ RMSNorm
constexpr int RMS_THREADS = 256;
// 16-byte vectors per thread kept in registers between RMSNorm's two passes
// (repeated 4096x4096: 21.6 -> 20.3 us, with x coming from HBM 26.0 -> 24.4
// us on MI355X)
constexpr int RMS_KEEP = 4;

// OutT float: fp32 output; OutT uint16_t: the same fp32 values rounded to
// bf16 (nearest even) as they are stored.
template <class OutT>
__global__ __launch_bounds__(RMS_THREADS) void rmsnorm_kernel(const uint16_t* __restrict__ x,
                                                              const uint16_t* __restrict__ gamma,
                                                              OutT* __restrict__ y, int hidden,
                                                              float eps)
{
    __shared__ float red[RMS_THREADS / 64];
    const size_t row = blockIdx.x;
    const uint4* xr = reinterpret_cast<const uint4*>(x + row * hidden);
    const int nv = hidden / 8;

    // A thread's first RMS_KEEP vectors (the whole row up to 8192 wide) stay
    // in registers for the second pass; the rest is read again.
    uint4 keep[RMS_KEEP];
    float ss = 0.0f;
    auto square_sum = [&](const uint4 q) {
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float a = bf16_lo(w[i]), b = bf16_hi(w[i]);
            ss = ss + a * a;
            ss = ss + b * b;
        }
    };
#pragma unroll
    for (int i = 0; i < RMS_KEEP; ++i) {
        const int v = threadIdx.x + i * RMS_THREADS;
        keep[i] = v < nv ? xr[v] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int i = 0; i < RMS_KEEP; ++i)
        if (threadIdx.x + i * RMS_THREADS < nv)
            square_sum(keep[i]);
    for (int v = threadIdx.x + RMS_KEEP * RMS_THREADS; v < nv; v += RMS_THREADS)
        square_sum(xr[v]);
    ss = block_sum<RMS_THREADS / 64>(ss, red);
    const float inv = 1.0f / sqrtf(ss / (float)hidden + eps);

    const uint4* gr = reinterpret_cast<const uint4*>(gamma);
    auto emit = [&](int v, const uint4 q) {
        const uint4 gq = gr[v];
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
        const uint32_t gw[4] = {gq.x, gq.y, gq.z, gq.w};
        float o[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = (bf16_lo(w[i]) * inv) * bf16_lo(gw[i]);
            o[2 * i + 1] = (bf16_hi(w[i]) * inv) * bf16_hi(gw[i]);
        }
        if constexpr (sizeof(OutT) == 4) {
            float4* yr = reinterpret_cast<float4*>(y + row * hidden);
            yr[2 * v] = make_float4(o[0], o[1], o[2], o[3]);
            yr[2 * v + 1] = make_float4(o[4], o[5], o[6], o[7]);
        } else {
            uint4 b;
            b.x = f32_to_bf16_bits(o[0]) | (f32_to_bf16_bits(o[1]) << 16);
            b.y = f32_to_bf16_bits(o[2]) | (f32_to_bf16_bits(o[3]) << 16);
            b.z = f32_to_bf16_bits(o[4]) | (f32_to_bf16_bits(o[5]) << 16);
            b.w = f32_to_bf16_bits(o[6]) | (f32_to_bf16_bits(o[7]) << 16);
            reinterpret_cast<uint4*>(y + row * hidden)[v] = b;
        }
    };
#pragma unroll
    for (int i = 0; i < RMS_KEEP; ++i) {
        const int v = threadIdx.x + i * RMS_THREADS;
        if (v < nv)
            emit(v, keep[i]);
    }
    for (int v = threadIdx.x + RMS_KEEP * RMS_THREADS; v < nv; v += RMS_THREADS)
        emit(v, xr[v]);
}

// -------------------------------------------------------------- log_softmax
// The row is read in the first pass and needed again in the second.  Most of
// it stays on chip in between: a thread keeps its first LSM_REG vectors in
// registers and its next LSM_LDS vectors in LDS (with 512 threads that is
// 40 + 18 vectors, 464 KiB of a row, 78% of a 151936-wide row); only the
// rest is read from memory a second time.  The visit order is that of
// every row kernel here (thread t: vectors t, t+NT, t+2NT, ...).
constexpr int UNROLL = 4;          // 16-byte loads in flight per thread
constexpr int LSM_THREADS = 512;
constexpr int LSM_REG = 40;
constexpr int LSM_LDS = 18;
constexpr int LSM_LDS_BYTES = LSM_LDS * LSM_THREADS * 16;

// (m, s) stands for s * exp(m): a running maximum and the sum of exp(x - m)
// of the elements seen.  Merging is commutative bit for bit: the operand
// with the larger maximum is the one rescaled by 1, and for equal maxima
// the two sums are added.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2)
{
    if (m > m2) {
        s = s + s2 * expf(m2 - m);
    } else if (m2 > m) {
        s = s2 + s * expf(m - m2);
        m = m2;
    } else {
        s = s + s2;
    }
}

// y = (x - m) - ls.  The output is written once and not read back here, so
// it is stored non-temporally: it does not push the logits (or other data
// that is read again) out of the caches.
__device__ __forceinline__ void store_shifted(float4* p, const float4 q, float m, float ls)
{
    f32x4 r = {(q.x - m) - ls, (q.y - m) - ls, (q.z - m) - ls, (q.w - m) - ls};
    __builtin_nontemporal_store(r, reinterpret_cast<f32x4*>(p));
}

// MEAN: the row mean is taken in the same pass (mu[row]), with the order,
// thread count and tree of mean_kernel, so its bits are inv_mean's.
template <bool MEAN>
__global__ __launch_bounds__(LSM_THREADS) void log_softmax_kernel(const float* x, float* y,
                                                                  float* mu, int cols)
{
    extern __shared__ float4 cache[];  // LSM_LDS vectors per thread
    __shared__ float red_m[LSM_THREADS / 64], red_s[LSM_THREADS / 64];
    __shared__ float red_sum[LSM_THREADS / 64];
    constexpr int NT = LSM_THREADS;
    const int tid = threadIdx.x;
    const size_t row = blockIdx.x;
    const float4* xr = reinterpret_cast<const float4*>(x + row * cols);
    float4* yr = reinterpret_cast<float4*>(y + row * cols);
    const int nv = cols / 4;
    const int lane = tid & 63, wave = tid >> 6;

    // exp of an element: the hardware base-2 exponential of (x - m)*log2(e)
    // (__expf), relative error about 2e-6 for |x - m| <= 30, a fixed
    // function like any other; the rescales of the running sum use expf
    float m = -INFINITY, s = 0.0f, sum = 0.0f;
    auto visit = [&](const float4 q) {
        if (MEAN) {
            sum = sum + q.x;
            sum = sum + q.y;
            sum = sum + q.z;
            sum = sum + q.w;
        }
        const float mx = fmaxf(fmaxf(q.x, q.y), fmaxf(q.z, q.w));
        if (mx > m) {
            s = s * expf(m - mx);
            m = mx;
        }
        s = s + __expf(q.x - m);
        s = s + __expf(q.y - m);
        s = s + __expf(q.z - m);
        s = s + __expf(q.w - m);
    };

    // vectors 0 .. LSM_REG-1 of the thread: all loads issued, then visited
    float4 rc[LSM_REG];
#pragma unroll
    for (int i = 0; i < LSM_REG; ++i) {
        const int v = tid + i * NT;
        rc[i] = (v < nv) ? xr[v] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int i = 0; i < LSM_REG; ++i)
        if (tid + i * NT < nv)
            visit(rc[i]);
    // the next LSM_LDS vectors, kept in LDS, UNROLL loads in flight
#pragma unroll
    for (int i0 = 0; i0 < LSM_LDS; i0 += UNROLL) {
        float4 q[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int v = tid + (LSM_REG + i0 + u) * NT;
            if (i0 + u < LSM_LDS && v < nv)
                q[u] = xr[v];
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int v = tid + (LSM_REG + i0 + u) * NT;
            if (i0 + u < LSM_LDS && v < nv) {
                cache[(i0 + u) * NT + tid] = q[u];
                visit(q[u]);
            }
        }
    }
    // the rest of the row, streamed
    constexpr int CACHED = LSM_REG + LSM_LDS;
    int v = tid + CACHED * NT;
    for (; v + (UNROLL - 1) * NT < nv; v += UNROLL * NT) {
        float4 q[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
            q[u] = xr[v + u * NT];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
            visit(q[u]);
    }
    for (; v < nv; v += NT)
        visit(xr[v]);

#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float m2 = __shfl_xor(m, off, 64), s2 = __shfl_xor(s, off, 64);
        lse_merge(m, s, m2, s2);
    }
    if (lane == 0) {
        red_m[wave] = m;
        red_s[wave] = s;
    }
    __syncthreads();
    constexpr int NW = LSM_THREADS / 64;
    m = (lane < NW) ? red_m[lane] : -INFINITY;
    s = (lane < NW) ? red_s[lane] : 0.0f;
#pragma unroll
    for (int off = NW / 2; off > 0; off >>= 1) {
        const float m2 = __shfl_xor(m, off, 64), s2 = __shfl_xor(s, off, 64);
        lse_merge(m, s, m2, s2);
    }
    m = __shfl(m, 0, 64);
    s = __shfl(s, 0, 64);
    const float ls = logf(s);
    if constexpr (MEAN) {
        const float total = block_sum<LSM_THREADS / 64>(sum, red_sum);
        if (tid == 0)
            mu[row] = total / (float)cols;
    }

    // second pass: cached vectors from registers and LDS, the rest re-read
#pragma unroll
    for (int i = 0; i < LSM_REG; ++i) {
        const int w = tid + i * NT;
        if (w < nv)
            store_shifted(yr + w, rc[i], m, ls);
    }
#pragma unroll
    for (int i = 0; i < LSM_LDS; ++i) {
        const int w = tid + (LSM_REG + i) * NT;
        if (w < nv)
            store_shifted(yr + w, cache[i * NT + tid], m, ls);
    }
    v = tid + CACHED * NT;
    for (; v + (UNROLL - 1) * NT < nv; v += UNROLL * NT) {
        float4 q[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
            q[u] = xr[v + u * NT];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
            store_shifted(yr + v + u * NT, q[u], m, ls);
    }
    for (; v < nv; v += NT)
        store_shifted(yr + v, xr[v], m, ls);
}

// --------------------------------------------------------------------- mean
// The thread count, per-thread visit order and tree of log_softmax's first
// pass, so the mean fused into log_softmax has the same bits; MEAN_UNROLL
// loads in flight per thread.
constexpr int ROW_THREADS = LSM_THREADS;
constexpr int MEAN_UNROLL = 8;

__global__ __launch_bounds__(ROW_THREADS) void mean_kernel(const float* __restrict__ x,
                                                           float* __restrict__ y, int cols)
{
    __shared__ float red[ROW_THREADS / 64];
    const size_t row = blockIdx.x;
    const float4* xr = reinterpret_cast<const float4*>(x + row * cols);
    const int nv = cols / 4;
    float s = 0.0f;
    auto visit = [&](const float4 q) {
        s = s + q.x;
        s = s + q.y;
        s = s + q.z;
        s = s + q.w;
    };
    int v = threadIdx.x;
    for (; v + (MEAN_UNROLL - 1) * ROW_THREADS < nv; v += MEAN_UNROLL * ROW_THREADS) {
        float4 q[MEAN_UNROLL];
#pragma unroll
        for (int u = 0; u < MEAN_UNROLL; ++u)
            q[u] = xr[v + u * ROW_THREADS];
#pragma unroll
        for (int u = 0; u < MEAN_UNROLL; ++u)
            visit(q[u]);
    }
    for (; v < nv; v += ROW_THREADS)
        visit(xr[v]);
    s = block_sum<ROW_THREADS / 64>(s, red);
    if (threadIdx.x == 0)
        y[row] = s / (float)cols;
}

hipError_t launch_rmsnorm(const uint16_t* x, const uint16_t* gamma, float* y, int rows,
                          int hidden, float eps, hipStream_t s)
{
    hipLaunchKernelGGL(rmsnorm_kernel<float>, dim3(rows), dim3(RMS_THREADS), 0, s, x, gamma, y,
                       hidden, eps);
    return hipGetLastError();
}

hipError_t launch_rmsnorm_bf16(const uint16_t* x, const uint16_t* gamma, uint16_t* y, int rows,
                               int hidden, float eps, hipStream_t s)
{
    hipLaunchKernelGGL(rmsnorm_kernel<uint16_t>, dim3(rows), dim3(RMS_THREADS), 0, s, x, gamma, y,
                       hidden, eps);
    return hipGetLastError();
}

template <bool MEAN>
static hipError_t launch_lsm(const float* x, float* y, float* mu, int rows, int cols,
                             hipStream_t s)
{
    static std::atomic<unsigned long long> lds_set{0};
    const hipError_t attr = ensure_lds_limit(
        lds_set, reinterpret_cast<const void*>(log_softmax_kernel<MEAN>), LSM_LDS_BYTES);
    if (attr != hipSuccess)
        return attr;
    hipLaunchKernelGGL(log_softmax_kernel<MEAN>, dim3(rows), dim3(LSM_THREADS), LSM_LDS_BYTES, s,
                       x, y, mu, cols);
    return hipGetLastError();
}

hipError_t launch_log_softmax(const float* x, float* y, int rows, int cols, hipStream_t s)
{
    return launch_lsm<false>(x, y, nullptr, rows, cols, s);
}

hipError_t launch_log_softmax_mean(const float* x, float* y, float* mu, int rows, int cols,
                                   hipStream_t s)
{
    return launch_lsm<true>(x, y, mu, rows, cols, s);
}

hipError_t launch_mean(const float* x, float* y, int rows, int cols, hipStream_t s)
{
    hipLaunchKernelGGL(mean_kernel, dim3(rows), dim3(ROW_THREADS), 0, s, x, y, cols);
    return hipGetLastError();
}

}  // namespace detred
