/*
 * CPU oracle for the deterministic-reduction hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: it is used by the tests, by the smoke check and by the
 * CPU-baseline leg of the benchmark, and nowhere else.  It shares no code,
 * header, table or helper with the HIP library.
 *
 * Every function is the plain definition of what the method computes, in
 * fp64 where the result is a real-valued sum, with no blocking, fusion or
 * reordering beyond the definition.  Sources (page title, then section):
 *
 *  - "Reproducible LoRA Inference Through Deterministic Split-K Reduction"
 *    (Highlights; Q&A): the LoRA shrink X*A whose FP32 outputs are compared,
 *    and split-K partial results combined either by atomics or in a fixed
 *    order.
 *  - arXiv 2511.17826 "Deterministic Inference across Tensor Parallel Sizes
 *    That Eliminates Training-Inference Mismatch" (Abstract): matrix
 *    multiplication and reduction whose intra- and inter-GPU partial sums
 *    are combined by one hierarchical binary tree.
 *  - "Restoring AI Reproducibility: Thinking Machines Lab's Challenge to
 *    Overcome Nondeterminism" (sections 2-2, 2-3, 3-1): RMSNorm and MatMul
 *    as reductions whose per-row result must not depend on batch size.
 *  - "Batch Invariant Ops" project summary (Highlighted Details): the
 *    supported operations mm, addmm, log_softmax and mean.
 *  - "Restoring AI Reproducibility..." (2-3, 3-2): attention is a reduction
 *    over the KV cache whose result must not depend on how it is split;
 *    the decode-attention oracle is the softmax-weighted sum itself.
 *
 * Pins (see tests/test_oracle_pins.py): exact rational brute force on tiny
 * shapes, integer-valued inputs with exact integer results, closed forms for
 * constant and +-1 rows, torch/numpy fp64 library routines, and the fp32
 * non-associativity example.
 */
#include <math.h>
#include <omp.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* A bf16 value is the upper half of an IEEE binary32 value, so widening it
 * to binary32 and then to binary64 is exact. */
static double bf16_bits_to_f64(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

void oracle_bf16_to_f64(const uint16_t *x, double *y, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        y[i] = bf16_bits_to_f64(x[i]);
}

/*
 * Matrix product Y = X W (the LoRA shrink X*A, the expand, the dense
 * projection and every tensor-parallel shard of it).
 *   X: M x K bf16 bits, row-major with leading dimension ldx.
 *   W: K x N bf16 bits, row-major with leading dimension ldw.
 *   Y: M x N fp64, Y[i][j] = sum_{k=0..K-1} x[i][k] * w[k][j], k increasing.
 *   Amag (optional): M x N fp64, Amag[i][j] = sum_k |x[i][k] * w[k][j]|,
 *   the magnitude sum the parity tolerance is scaled by.
 * The product of two bf16 values is exact in fp64 (8+8 significant bits),
 * so the only rounding is in the fp64 running sum.
 */
void oracle_gemm_f64(const uint16_t *X, long ldx, const uint16_t *W, long ldw,
                     double *Y, double *Amag, int M, int N, int K)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < M; ++i) {
        double *y = Y + (size_t)i * N;
        double *a = Amag ? Amag + (size_t)i * N : NULL;
        for (int j = 0; j < N; ++j) {
            y[j] = 0.0;
            if (a) a[j] = 0.0;
        }
        for (int k = 0; k < K; ++k) {
            double xv = bf16_bits_to_f64(X[(size_t)i * ldx + k]);
            const uint16_t *w = W + (size_t)k * ldw;
            if (a) {
                for (int j = 0; j < N; ++j) {
                    double p = xv * bf16_bits_to_f64(w[j]);
                    y[j] += p;
                    a[j] += fabs(p);
                }
            } else {
                for (int j = 0; j < N; ++j)
                    y[j] += xv * bf16_bits_to_f64(w[j]);
            }
        }
    }
}

/*
 * RMSNorm of each row (Thinking Machines article, 2-3 and 3-1):
 *   y[j] = gamma[j] * x[j] / sqrt( (1/H) sum_l x[l]^2 + eps ).
 * x: rows x H bf16 bits, gamma: H bf16 bits, y: rows x H fp64.
 */
void oracle_rmsnorm_f64(const uint16_t *x, const uint16_t *gamma, double *y,
                        int rows, int H, double eps)
{
#pragma omp parallel for schedule(static)
    for (int r = 0; r < rows; ++r) {
        const uint16_t *xr = x + (size_t)r * H;
        double ss = 0.0;
        for (int l = 0; l < H; ++l) {
            double v = bf16_bits_to_f64(xr[l]);
            ss += v * v;
        }
        double denom = sqrt(ss / (double)H + eps);
        for (int j = 0; j < H; ++j)
            y[(size_t)r * H + j] =
                bf16_bits_to_f64(gamma[j]) * bf16_bits_to_f64(xr[j]) / denom;
    }
}

/*
 * log_softmax over the last dimension (Batch Invariant Ops, Highlighted
 * Details):  y[j] = (x[j] - m) - ln sum_l exp(x[l] - m),  m = max_l x[l].
 */
void oracle_log_softmax_f64(const float *x, double *y, int rows, int cols)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < rows; ++r) {
        const float *xr = x + (size_t)r * cols;
        double m = -INFINITY;
        for (int l = 0; l < cols; ++l)
            if ((double)xr[l] > m) m = (double)xr[l];
        double s = 0.0;
        for (int l = 0; l < cols; ++l)
            s += exp((double)xr[l] - m);
        double ls = log(s);
        for (int j = 0; j < cols; ++j)
            y[(size_t)r * cols + j] = ((double)xr[j] - m) - ls;
    }
}

/* mean over the last dimension (Batch Invariant Ops, Highlighted Details):
 * y[r] = (sum_j x[r][j]) / cols. */
void oracle_mean_f64(const float *x, double *y, int rows, int cols)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < rows; ++r) {
        const float *xr = x + (size_t)r * cols;
        double s = 0.0;
        for (int j = 0; j < cols; ++j)
            s += (double)xr[j];
        y[r] = s / (double)cols;
    }
}

/*
 * The fixed binary reduction tree in binary32 (split-K paper, Q&A: partial
 * results combined in a fixed order; TBIK abstract: one hierarchical binary
 * tree).  P holds S partial arrays of n floats each (S a power of two); the
 * tree adds neighbours pairwise, level by level:
 *   S=2: p0+p1;  S=4: (p0+p1)+(p2+p3);
 *   S=8: ((p0+p1)+(p2+p3))+((p4+p5)+(p6+p7)).
 * Each node is one IEEE binary32 addition, rounded to nearest even.
 * Returns 0, or -1 if S is not a power of two in 1..64.
 */
int oracle_tree_sum_f32(const float *P, int S, size_t n, float *Y)
{
    if (S < 1 || S > 64 || (S & (S - 1)) != 0)
        return -1;
    for (size_t e = 0; e < n; ++e) {
        volatile float v[64];
        for (int s = 0; s < S; ++s)
            v[s] = P[(size_t)s * n + e];
        for (int width = S; width > 1; width /= 2)
            for (int i = 0; i < width / 2; ++i) {
                float a = v[2 * i], b = v[2 * i + 1];
                v[i] = a + b;
            }
        Y[e] = v[0];
    }
    return 0;
}

/* Sequential left-to-right binary32 sum (((v0+v1)+v2)+...), the order an
 * unsplit reduction or a single accumulator uses. */
float oracle_fold_sum_f32(const float *v, int n)
{
    volatile float acc = 0.0f;
    for (int i = 0; i < n; ++i) {
        float t = acc + v[i];
        acc = t;
    }
    return acc;
}

/*
 * binary32 -> bf16 with round to nearest, ties to even: the explicit cast
 * that turns the fp32 shrink output into the bf16 input of the expand.
 * Written from the definition: of the two bf16 neighbours of x (truncation
 * toward zero and one bf16 ulp further from zero) take the nearer one,
 * comparing distances exactly in fp64; on a tie take the one whose last
 * significand bit is 0.  NaN maps to a quiet NaN of the same sign;
 * values beyond the largest bf16 round to infinity as IEEE prescribes.
 */
void oracle_f32_to_bf16_rne(const float *x, uint16_t *y, size_t n)
{
    for (size_t i = 0; i < n; ++i) {
        uint32_t u;
        memcpy(&u, &x[i], sizeof u);
        if ((u & 0x7f800000u) == 0x7f800000u) {            /* inf or nan */
            if (u & 0x007fffffu)
                y[i] = (uint16_t)((u >> 16) | 0x0040u);      /* quiet nan */
            else
                y[i] = (uint16_t)(u >> 16);
            continue;
        }
        uint16_t lo = (uint16_t)(u >> 16);          /* toward zero */
        uint16_t hi = (uint16_t)(lo + 1);           /* away from zero (may reach inf) */
        double xv = (double)x[i];
        double dlo = fabs(xv - bf16_bits_to_f64(lo));
        double dhi;
        if ((hi & 0x7f80u) == 0x7f80u && (hi & 0x7fu) == 0) {
            /* hi is infinity: distance measured to 2^128, the value the
             * first unrepresentable binade would start at. */
            dhi = fabs(fabs(xv) - ldexp(1.0, 128));
        } else {
            dhi = fabs(xv - bf16_bits_to_f64(hi));
        }
        if (dlo < dhi)
            y[i] = lo;
        else if (dhi < dlo)
            y[i] = hi;
        else
            y[i] = (lo & 1u) ? hi : lo;
    }
}

/* Number of OpenMP threads the oracle's parallel loops use. */
int oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
    return n;
}

/*
 * Decode attention, one new query token per sequence ("Restoring AI
 * Reproducibility...", 2-3 and 3-2: attention over the KV cache).  For
 * sequence b and query head hq (KV head h = hq / G, G = Hq / Hkv):
 *   sigma_t = scale * sum_d q[b][hq][d] * k[b][h][t][d],   t < len_b
 *   w_t     = exp(sigma_t - max_t sigma_t)
 *   out[d]  = sum_t w_t v[b][h][t][d] / sum_t w_t
 * all in fp64.  Also, per output element, A = sum_t w_t |v_td| / sum_t w_t
 * (the magnitude the tolerance scales with) and, per (b, hq),
 * S = max_t scale * sum_d |q_d k_td| (the score magnitude).  q is [B][Hq][D]
 * bf16; k and v are bf16 with D contiguous and strides (in elements)
 * sb, sh, st for sequence, KV head and position.  len_b <= 0 gives zeros.
 */
void oracle_decode_attention_f64(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                                 long sb, long sh, long st, const int *lens, double *out,
                                 double *amag, double *smag, int B, int Hq, int Hkv, int D,
                                 double scale)
{
    const int G = Hq / Hkv;
#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < B * Hq; ++bh) {
        const int b = bh / Hq, hq = bh % Hq, h = hq / G;
        const int len = lens[b];
        double *o = out + (size_t)bh * D, *a = amag + (size_t)bh * D;
        for (int d = 0; d < D; ++d)
            o[d] = a[d] = 0.0;
        smag[bh] = 0.0;
        if (len <= 0)
            continue;
        const uint16_t *qv = q + (size_t)bh * D;
        double *sig = (double *)malloc(sizeof(double) * (size_t)len);
        double mx = -INFINITY, smax = 0.0;
        for (int t = 0; t < len; ++t) {
            const uint16_t *kt = k + b * sb + h * sh + t * st;
            double acc = 0.0, accabs = 0.0;
            for (int d = 0; d < D; ++d) {
                const double p = bf16_bits_to_f64(qv[d]) * bf16_bits_to_f64(kt[d]);
                acc += p;
                accabs += fabs(p);
            }
            sig[t] = scale * acc;
            if (sig[t] > mx)
                mx = sig[t];
            if (fabs(scale) * accabs > smax)
                smax = fabs(scale) * accabs;
        }
        double l = 0.0;
        for (int t = 0; t < len; ++t) {
            const double w = exp(sig[t] - mx);
            l += w;
            const uint16_t *vt = v + b * sb + h * sh + t * st;
            for (int d = 0; d < D; ++d) {
                const double x = bf16_bits_to_f64(vt[d]);
                o[d] += w * x;
                a[d] += w * fabs(x);
            }
        }
        for (int d = 0; d < D; ++d) {
            o[d] /= l;
            a[d] /= l;
        }
        smag[bh] = smax;
        free(sig);
    }
}
