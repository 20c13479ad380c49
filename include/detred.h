/*
 * detred.h -- deterministic, batch-invariant and tensor-parallel-invariant
 * reductions for MI355X (gfx950).
 *
 * C ABI.  All tensor arguments are DEVICE pointers allocated and owned by the
 * caller; the library keeps no pointer after a call returns and allocates no
 * device memory on any compute call.  bf16 tensors are passed as their 16-bit
 * patterns (uint16_t).  Every matrix is row-major with an explicit leading
 * dimension (elements between the starts of consecutive rows).
 *
 * Calls are asynchronous on the given stream (a hipStream_t passed as void*,
 * NULL = the null stream).  Validation is synchronous: a return value other
 * than DETRED_OK means nothing was launched.
 *
 * Which operations and why
 * ------------------------
 * Split-K parallelises a matrix product over its reduction dimension K: K is
 * cut into slices, each slice produces an fp32 partial result, and the
 * partials are summed.  Summing them with floating-point atomics makes the
 * order, and so the rounding, depend on timing ("Reproducible LoRA Inference
 * Through Deterministic Split-K Reduction", Highlights and Q&A); summing them
 * in a fixed order removes that.  Using one hierarchical binary tree for the
 * partial sums inside a GPU and across GPUs makes the bits independent of the
 * tensor-parallel size as well (arXiv 2511.17826, "Deterministic Inference
 * across Tensor Parallel Sizes...", Abstract).  Row reductions such as RMSNorm
 * must likewise reduce each row in an order that does not depend on the batch
 * ("Restoring AI Reproducibility: Thinking Machines Lab's Challenge to
 * Overcome Nondeterminism", sections 2-2 to 3-2); mm, addmm, log_softmax and
 * mean are the operations the "Batch Invariant Ops" project makes batch
 * invariant (Highlighted Details).
 *
 * The canonical reduction of a product (every GEMM entry point)
 * -------------------------------------------------------------
 * For a reduction length K the library fixes, from K alone:
 *   P  = 8 chunks if K >= 256 and K % 256 == 0, else P = 1;
 *   Kc = K / P, chunk c covers k in [c*Kc, (c+1)*Kc).
 * Output element (i,j) is
 *   chunk_c(i,j) = a chain of v_mfma_f32_16x16x32_bf16 steps over the chunk's
 *                  k in increasing order, starting from +0.0f, 32 k per step
 *                  (a step that runs past K uses exact zeros for the missing
 *                  k; this only happens when P = 1);
 *   Y(i,j)       = the fixed binary tree over the P chunk values:
 *                  ((c0+c1)+(c2+c3))+((c4+c5)+(c6+c7)), one binary32
 *                  round-to-nearest-even addition per node.
 * A split into S slices (S | P) gives slice s the chunks
 * [s*P/S, (s+1)*P/S), which form a complete subtree; the slices' partials are
 * then combined by the top log2(S) levels of the same tree.  The same holds
 * for T tensor-parallel shards.  Hence Y's bits do not depend on the batch
 * size M, on a row's position in the batch, on S, on T, on the tile shape, on
 * the stream or on replay.  atomic_splitk_gemm is the only exception: it is
 * the nondeterministic control.
 *
 * What is locked and what follows M.  P and Kc (the bits) depend on K only.
 * The workgroup tile a call launches and the split that split_k = 0 picks
 * are chosen for speed and DO depend on M (and on N and K): at most 64 rows
 * run 64 x 128 tiles, an eight-chunk product at one slice runs 192 x 128
 * tiles where 1.25 times their rounds of workgroups over the 256 compute
 * units do not exceed those of 128 x 128 tiles (e.g. from 513 rows of a
 * 14336-column output, from 1025 rows of a 4096-column one), one-chunk
 * shard roots with 256 rows or more (chunks of 1024 or more) run 256 x 256
 * tiles, outputs of at most 64 columns run 64 x 16 tiles while 64 x 64 ones
 * would leave fewer than 256 workgroups, and detred_auto_split keys on M as
 * described there.  None of
 * these choices changes a bit: every tile evaluates the same chunk chains
 * with the same MFMA k-slot layout and the same tree, and an output
 * element's MFMA result does not depend on the row's place in the tile.
 *
 * Requirements shared by the GEMM entry points (else the status shown):
 *   M, N, K >= 0; ldx >= K, ldw >= N, ldy >= N                   (EINVAL)
 *   X, W, Y 16-byte aligned; ldx, ldw multiples of 8; ldy of 4    (EINVAL)
 *   K % 8 == 0 and N % 8 == 0                                  (EUNSUPPORTED)
 *   split_k / tp_shards in {1,2,4,8} and <= P                  (EUNSUPPORTED)
 * M == 0 or N == 0 launches nothing and returns DETRED_OK; K == 0 writes
 * +0.0f to Y.  Y must not overlap X, W or the workspace.
 */
#ifndef DETRED_H
#define DETRED_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DETRED_OK = 0,
    DETRED_EINVAL = 1,       /* null/misaligned pointer, bad dims or ld   */
    DETRED_EUNSUPPORTED = 2, /* valid but outside what the kernels cover  */
    DETRED_EWORKSPACE = 3,   /* workspace missing or too small            */
    DETRED_EHIP = 4          /* the HIP runtime reported an error         */
} detred_status;

typedef void *detred_stream; /* hipStream_t; NULL = null stream */

/* Element type of an output that may be fp32 or bf16. */
enum { DETRED_F32 = 0, DETRED_BF16 = 1 };

/* Human-readable name of a status code (static storage; never NULL). */
const char *detred_status_string(detred_status status);

/* Library version as 10000*major + 100*minor + patch. */
int detred_version(void);

/*
 * The locked reduction for reduction length K and the tile family for N
 * output columns.  Writes, where the pointer is non-NULL:
 *   chunks   = P (1 or 8) and chunk_k = Kc: these alone fix the bits;
 *   tile_m, tile_n = the family's workgroup output tile (128 x 128 for wide
 *                    outputs, 64 x 64 or 64 x 16 for narrow ones); the tile
 *                    a call launches also follows M (see "What is locked
 *                    and what follows M" above), never changing the bits;
 *   default_split  = the split split_k = 0 picks once M is large enough to
 *                    give every CU an output tile (detred_auto_split).
 * Returns EINVAL for N < 0 or K < 0.
 */
detred_status detred_policy(int N, int K, int *chunks, int *chunk_k, int *tile_m,
                            int *tile_n, int *default_split);

/*
 * The split that split_k = 0 selects for an M x N x K product.  The split
 * only decides how many workgroups share the chunk tree; the bits of the
 * result never depend on it (nor on M).  Outputs of at most 64 columns use
 * one slice per chunk (S = P).  For wider ones, with t = the number of
 * 128 x 128 output tiles and Kc = K / P:
 *   257 <= t <= 447, P = 8, Kc % 64 == 0 and ceil(M/192) * ceil(N/128) <=
 *                   256 (one round of 192 x 128 tiles on the 256 compute
 *                   units): S = 1;
 *   else Kc >= 1536, M >= 256 and t >= 96: S = 8;
 *   else t <= 128:  the largest S (<= P) with t*S <= 256, but 4 instead of
 *                   2 for products of at most 16 rows;
 *   129 <= t <= 192: S = 4 if Kc >= 1024, else 1;
 *   t > 192:        S = 1, but for 257 <= t <= 447 S = 4 if Kc >= 1024,
 *                   else 2.
 * This is the split of det_splitk_gemm and of an fp32 det_splitk_addmm
 * whose C does not overlap Y.  An addmm into bf16, or with C overlapping Y,
 * cannot run the 192 x 128 tile and skips the first rule.
 * Returns 0 for invalid arguments.
 */
int detred_auto_split(int M, int N, int K);

/*
 * Workspace size in bytes that det_splitk_gemm (split_k = S) or tree_tp_gemm
 * (tp_shards = S) needs for an M x N output with reduction length K:
 * S fp32 partial arrays of M*N elements plus one 32-bit counter per output
 * tile, rounded up to 256 bytes.  S = 0 means the split a call with
 * split_k = 0 picks: detred_auto_split(M, N, K), or, where larger, the split
 * of an addmm that cannot run the 192 x 128 tile (see there).
 * 0 when S == 1 (no workspace is used), and 0 for a split the products reject
 * (S not in {1,2,4,8}, or S > P) and for invalid arguments.
 */
size_t detred_gemm_workspace_bytes(int M, int N, int K, int split_or_shards);

/*
 * Zero a workspace's counters (the whole buffer) on stream s.  Call once
 * after allocating a workspace.  The arrival counters are read only by the
 * one-launch combine (split products of at most 64 columns with fewer than
 * 65536 output elements); they must be zero when such a call starts, and
 * every such call leaves them zero when it completes.  A workspace that was
 * never zeroed, or that anything else has written since (another call's
 * partials included, when the buffer is shared between shapes), gives
 * those calls undefined results: the tree combine may run before every
 * slice has arrived, or not at all.  The library does not detect this.
 * One workspace serves one call in flight at a time.
 */
detred_status detred_workspace_init(void *ws, size_t ws_bytes, detred_stream s);

/*
 * Deterministic split-K product Y[M,N] (fp32) = X[M,K] W[K,N] (bf16), the
 * fixed-order split-K of the split-K paper (Highlights, Q&A) with the
 * canonical tree above.  split_k = S in {1,2,4,8} (S <= P), or 0 for
 * detred_auto_split(M, N, K).  With S > 1 each slice writes its fp32
 * subtree root into the workspace as S row-major [M][N] arrays (ld N) at
 * byte offset 0, and the top log2(S) levels of the tree add them into Y:
 * in a second launch that streams over the S arrays when N > 64 or
 * M*N >= 65536, otherwise (small narrow outputs) by the last slice of each
 * output tile to finish, in the same launch.  Either way the bits are the
 * same.  ws may be NULL when S == 1.
 * ws must be 256-byte aligned and at least detred_gemm_workspace_bytes()
 * large (EWORKSPACE otherwise), and its counters zero (detred_workspace_init).
 * With S > 1, N must stay below about 4.1 million (the combine addresses a
 * tile's rows with 32-bit offsets; EUNSUPPORTED otherwise).
 * The bits of Y do not depend on S.
 */
detred_status det_splitk_gemm(const uint16_t *X, int ldx, const uint16_t *W,
                              int ldw, float *Y, int ldy, int M, int N, int K,
                              int split_k, void *ws, size_t ws_bytes,
                              detred_stream s);

/*
 * Deterministic addmm, the form of torch.addmm that the "Batch Invariant Ops"
 * project makes batch invariant (Highlighted Details), with an optional bf16
 * output:
 *   p = the canonical product of X[M,K] and W[K,N] (the bits det_splitk_gemm
 *       writes, for any split_k);
 *   y = beta*C[i][j] + alpha*p   (C == NULL: y = alpha*p), each product and
 *       the sum rounded to binary32 as written (alpha = beta = 1 makes both
 *       products exact);
 *   Y[i][j] = y as fp32 (y_dtype DETRED_F32) or rounded to bf16, nearest
 *       even (DETRED_BF16; NaN stays NaN).
 * C is fp32, 16-byte aligned; ldc = 0 broadcasts one row of N values (a
 * bias) to every row, otherwise ldc >= N and ldc % 4 == 0.  Y is 16-byte
 * aligned, ldy % 4 == 0, in elements of y_dtype.  The epilogue is applied
 * where the final value of an element is written (in the tree combine when
 * split_k > 1), so it adds no pass over Y.  split_k, ws and errors as
 * det_splitk_gemm; EINVAL for a bad y_dtype, C or ldc.  K == 0 gives
 * y = beta*C + alpha*(+0).  Row i of Y depends only on row i of X (and of C).
 */
detred_status det_splitk_addmm(const uint16_t *X, int ldx, const uint16_t *W,
                               int ldw, const float *C, int ldc, float alpha,
                               float beta, void *Y, int ldy, int y_dtype, int M,
                               int N, int K, int split_k, void *ws, size_t ws_bytes,
                               detred_stream s);

/*
 * det_splitk_gemm and det_splitk_addmm with the weight given transposed:
 * Wt is [N,K] bf16, K contiguous, rows ldwt elements apart (ldwt >= K,
 * ldwt % 8 == 0, 16-byte aligned) -- the layout in which a linear layer
 * keeps its weight ([out, in]), so y = x W^T needs no transposed copy when
 * the kernels stand in for mm/addmm under an unchanged model ("Batch
 * Invariant Ops", How It Works).  Element (k, n) of the
 * product's right operand is Wt[n*ldwt + k].  The products, the chunk tree
 * and the split rules are those of the untransposed calls, so the output
 * bits equal theirs for W = Wt^T; workspace, errors and asynchrony as there
 * (EINVAL also for ldwt < K).
 */
detred_status det_splitk_gemm_wt(const uint16_t *X, int ldx, const uint16_t *Wt,
                                 int ldwt, float *Y, int ldy, int M, int N, int K,
                                 int split_k, void *ws, size_t ws_bytes,
                                 detred_stream s);
detred_status det_splitk_addmm_wt(const uint16_t *X, int ldx, const uint16_t *Wt,
                                  int ldwt, const float *C, int ldc, float alpha,
                                  float beta, void *Y, int ldy, int y_dtype, int M,
                                  int N, int K, int split_k, void *ws,
                                  size_t ws_bytes, detred_stream s);

/*
 * det_splitk_gemm for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * The same product, split rules and output bits as det_splitk_gemm, with no
 * workspace argument: the S slice partials and the arrival counters live in
 * a scratch array the library holds on each device it runs on (32 MiB,
 * kept until the process ends).  The first call on a device looks the
 * array up with that device current and zeroes its counters with a kernel
 * on s; no call allocates or frees memory (no hipMalloc, hipFree or
 * allocating library routine).
 * Limit: with S > 1 the partials, S*M*N*4 bytes, must not exceed
 * DETRED_NOALLOC_PARTIAL_BYTES (EWORKSPACE otherwise, nothing launched).
 * S == 1 and K == 0 use no scratch.  Every call on a device shares its
 * scratch: calls that overlap on one device (other streams, other host
 * threads) race and give undefined results; calls ordered on one stream, or
 * synchronised, do not.  Other arguments and errors as det_splitk_gemm.
 */
#define DETRED_NOALLOC_PARTIAL_BYTES ((size_t)33488896) /* 32 MiB - 64 KiB */
detred_status det_splitk_gemm_noalloc(const uint16_t *X, int ldx,
                                      const uint16_t *W, int ldw, float *Y,
                                      int ldy, int M, int N, int K, int split_k,
                                      detred_stream s);

/*
 * Workspace of det_lora_forward for an M x N layer output with input width K
 * and LoRA rank r: the fp32 base product, the bf16 shrink output and the
 * split-K workspaces of the base product and the shrink, each 256-byte
 * aligned.  0 for invalid arguments.
 */
size_t det_lora_workspace_bytes(int M, int N, int K, int r);

/*
 * A LoRA-adapted linear layer in one call, every step in a fixed order
 * (split-K paper, Highlights and Q&A: the base product, the shrink X*A and
 * the expand of its bf16 cast by B):
 *   base = det_splitk_gemm(X, W)              fp32 [M,N], policy split;
 *   zb   = det_splitk_addmm(X, A, no C, alpha = 1, bf16 output)
 *                                             bf16 [M,r], policy split (8):
 *          the bits of detred_f32_to_bf16(det_splitk_gemm(X, A)), the
 *          rounding done in the shrink's own epilogue;
 *   Y    = det_splitk_addmm(zb, B, C = base, alpha = scale, beta = 1,
 *                           bf16 output)      bf16 [M,N]
 * i.e. Y = bf16(base + scale*(zb*B)).  X [M,K] ld ldx, W [K,N] ld ldw,
 * A [K,r] ld lda, B [r,N] ld ldb, all bf16; Y bf16 ld ldy.  r % 8 == 0,
 * K % 8 == 0, N % 8 == 0.  ws: det_lora_workspace_bytes(M,N,K,r) bytes,
 * 256-byte aligned, zeroed once with detred_workspace_init.  Three to five
 * launches on s (a split base product or shrink adds its combine launch).
 * The bits of Y do not depend on M.
 */
detred_status det_lora_forward(const uint16_t *X, int ldx, const uint16_t *W,
                               int ldw, const uint16_t *A, int lda,
                               const uint16_t *B, int ldb, float scale, uint16_t *Y,
                               int ldy, int M, int N, int K, int r, void *ws,
                               size_t ws_bytes, detred_stream s);

/*
 * The nondeterministic control: the same slice products as det_splitk_gemm,
 * but Y is zero-filled on the stream and every slice adds its partial into Y
 * with fp32 atomic additions, so the summation order follows the order in
 * which slices finish (split-K paper, Q&A: partial results combined with
 * floating-point atomic additions).  split_k as above (0 = automatic).  The
 * zero fill is part of the call.  Results agree with the oracle to the same
 * tolerance but are not bit-reproducible.
 */
detred_status atomic_splitk_gemm(const uint16_t *X, int ldx, const uint16_t *W,
                                 int ldw, float *Y, int ldy, int M, int N, int K,
                                 int split_k, detred_stream s);

/*
 * Tree-based TP-invariant product on one GPU (TBIK, arXiv 2511.17826,
 * Abstract): K is cut into tp_shards = T contiguous shards (T in {1,2,4,8},
 * T <= P); shard t reduces chunks [t*P/T, (t+1)*P/T) to its subtree root and
 * writes it to its own fp32 [M][N] buffer (the value rank t of a T-way
 * row-parallel group would hold before the all-reduce); the buffers are then
 * added by the top log2(T) levels of the same tree into Y (the step the
 * inter-GPU reduction performs).  Two launches for T > 1, one for T == 1.
 * ws: T*M*N fp32 shard buffers (detred_gemm_workspace_bytes(M,N,K,T));
 * may be NULL when T == 1.  Y's bits equal det_splitk_gemm's for every T.
 */
detred_status tree_tp_gemm(const uint16_t *X, int ldx, const uint16_t *W, int ldw,
                           float *Y, int ldy, int M, int N, int K, int tp_shards,
                           void *ws, size_t ws_bytes, detred_stream s);

/*
 * Phase 1 of tree_tp_gemm on its own: all T shards in one launch, shard t's
 * subtree root written to P + t*M*N as a row-major [M][N] fp32 array (ld N).
 * P must hold T*M*N floats, 16-byte aligned.  tree_combine_f32(P, M*N, T,
 * Y, M*N) is phase 2 (the cross-rank reduction) for a contiguous Y.
 */
detred_status tree_tp_shards_gemm(const uint16_t *X, int ldx, const uint16_t *W,
                                  int ldw, float *P, int M, int N, int K,
                                  int tp_shards, detred_stream s);

/*
 * One shard of tree_tp_gemm at its own share shape: what rank t of a
 * T-way row-parallel group computes locally.  Xt is the rank's [M, Kt]
 * activation shard, Wt its [Kt, N] weight shard, Kt = K / T, and Pt
 * (fp32 [M][N], ld ldp) receives the root of the shard's subtree: its
 * P/T chunks of width K/8 each.  Requires Kt*T to satisfy the P = 8 rule
 * (Kt*T >= 256, Kt*T % 256 == 0) when T > 1.
 */
detred_status tree_tp_shard_gemm(const uint16_t *Xt, int ldx, const uint16_t *Wt,
                                 int ldw, float *Pt, int ldp, int M, int N, int Kt,
                                 int tp_shards, detred_stream s);

/*
 * The three tree-TP calls with the weight given transposed, as a
 * row-parallel linear layer keeps its shard ([out, in] = [N, K], or [N, Kt]
 * for one rank), K contiguous, rows ldwt elements apart (ldwt >= K, resp.
 * Kt; ldwt % 8 == 0; 16-byte aligned).  Element (k, n) of the product's
 * right operand is Wt[n*ldwt + k].  Shards, tree, workspace, errors and
 * asynchrony as in the untransposed calls, and the same output bits.
 */
detred_status tree_tp_gemm_wt(const uint16_t *X, int ldx, const uint16_t *Wt,
                              int ldwt, float *Y, int ldy, int M, int N, int K,
                              int tp_shards, void *ws, size_t ws_bytes,
                              detred_stream s);
detred_status tree_tp_shards_gemm_wt(const uint16_t *X, int ldx, const uint16_t *Wt,
                                     int ldwt, float *P, int M, int N, int K,
                                     int tp_shards, detred_stream s);
detred_status tree_tp_shard_gemm_wt(const uint16_t *Xt, int ldx,
                                    const uint16_t *Wtt, int ldwt, float *Pt,
                                    int ldp, int M, int N, int Kt, int tp_shards,
                                    detred_stream s);

/*
 * The fixed binary tree over `count` fp32 arrays of n elements each
 * (count in {1,2,4,8}): parts + i*part_stride (elements) is array i;
 * Y[e] = ((p0+p1)+(p2+p3))+... as in the canonical tree's top levels.
 * parts and Y 16-byte aligned, part_stride and n multiples of 4.
 * Y may not overlap the parts.
 */
detred_status tree_combine_f32(const float *parts, size_t part_stride, int count,
                               float *Y, size_t n, detred_stream s);

/*
 * The explicit binary32 -> bf16 cast (round to nearest, ties to even) that
 * turns the fp32 LoRA shrink output into the bf16 input of the expand
 * (split-K paper, Q&A: shrink, then expand).  n elements; x, y 16-byte
 * aligned, n % 8 == 0.  NaN stays NaN.
 */
detred_status detred_f32_to_bf16(const float *x, uint16_t *y, size_t n,
                                 detred_stream s);

/*
 * Batch-invariant RMSNorm (Thinking Machines article, 2-3 and 3-1: each row
 * handled by one workgroup and reduced in one fixed order):
 *   y[r][j] = (x[r][j] * inv) * gamma[j],  inv = 1 / sqrt(ss/hidden + eps),
 *   ss = sum_j x[r][j]^2 in binary32 in a fixed order that depends only on
 *   hidden.
 * x bf16 [rows][hidden], gamma bf16 [hidden], y fp32 [rows][hidden], all
 * contiguous and 16-byte aligned; hidden % 8 == 0, 0 < hidden <= 65536
 * (EUNSUPPORTED otherwise).  rows == 0 launches nothing.
 */
detred_status inv_rmsnorm(const uint16_t *x, const uint16_t *gamma, float *y,
                          int rows, int hidden, float eps, detred_stream s);

/*
 * inv_rmsnorm with a bf16 output: the same binary32 values, each rounded to
 * bf16 (nearest even) as it is stored.  y bf16 [rows][hidden], 16-byte
 * aligned; other arguments and errors as inv_rmsnorm.
 */
detred_status inv_rmsnorm_bf16(const uint16_t *x, const uint16_t *gamma,
                               uint16_t *y, int rows, int hidden, float eps,
                               detred_stream s);

/*
 * Batch-invariant log_softmax over the last dimension (Batch Invariant Ops,
 * Highlighted Details): y[r][j] = (x[r][j] - m) - log(s), with m the row
 * maximum and s = sum_j exp(x[r][j] - m), both reduced by one workgroup per
 * row in a fixed order that depends only on cols.  x, y fp32 [rows][cols]
 * contiguous, 16-byte aligned, cols % 4 == 0 and cols > 0 (EUNSUPPORTED
 * otherwise).  x and y may be the same buffer.
 */
detred_status inv_log_softmax(const float *x, float *y, int rows, int cols,
                              detred_stream s);

/*
 * Batch-invariant mean over the last dimension (Batch Invariant Ops,
 * Highlighted Details): y[r] = (sum_j x[r][j]) / cols, the sum in binary32
 * in a fixed order that depends only on cols, then one IEEE division.
 * x fp32 [rows][cols] contiguous, 16-byte aligned, cols % 4 == 0, cols > 0;
 * y fp32 [rows].
 */
detred_status inv_mean(const float *x, float *y, int rows, int cols,
                       detred_stream s);

/*
 * inv_log_softmax and inv_mean of the same rows in one pass over x: y as
 * inv_log_softmax gives it and mu[r] as inv_mean gives it, bit for bit (the
 * mean takes the order and tree inv_mean uses), with x read once instead of
 * twice: two of the operations the "Batch Invariant Ops" project makes
 * batch invariant (Highlighted Details) in one kernel.  mu fp32 [rows],
 * 4-byte aligned; other arguments and errors as inv_log_softmax (x and y may
 * be the same buffer).
 */
detred_status inv_log_softmax_mean(const float *x, float *y, float *mu, int rows,
                                   int cols, detred_stream s);

/*
 * Workspace of inv_decode_attention: the per-chunk results of B*Hq query
 * rows over ceil(max_len/256) chunks (D + 2 floats each), 256-byte aligned
 * sections.  0 for invalid arguments.
 */
size_t inv_decode_attention_workspace_bytes(int B, int Hq, int D, int max_len);

/*
 * Batch-invariant decode attention: one new query token per sequence
 * attends to its KV cache, with the reduction over positions split into
 * chunks of a fixed size, 256 positions, whatever the batch ("Restoring AI
 * Reproducibility: Thinking Machines Lab's Challenge to Overcome
 * Nondeterminism", 2-3 and 3-2: attention needs a fixed-size split of the
 * KV cache to keep its order independent of the batch).  For sequence b and
 * query head hq (KV head h = hq / G, G = Hq / Hkv):
 *   out[b][hq][:] = sum_t softmax_t(scale * q[b][hq] . k[b][h][t]) v[b][h][t]
 * over t < min(lens[b], max_len) (zeros when that is <= 0).  Order: within
 * a chunk of 256 positions, scores from 8-term fused multiply-add chains
 * and a 16-lane butterfly, the chunk maximum, weights exp(s - max), and the
 * chunk's weight sum and weighted value sum in a fixed lane and wave order;
 * across chunks a left-to-right fold in chunk order; then one division.
 * Row (b, hq) of out depends only on q[b][hq], sequence b's cache and
 * lens[b]: not on B, on the other sequences, on max_len or on the layout.
 *   q    bf16 [B][Hq][D], contiguous;
 *   k, v bf16, element (b, h, t, d) at b*kv_stride_b + h*kv_stride_h +
 *        t*kv_stride_t + d (D contiguous; "bhtd" and "bthd" caches are both
 *        expressible), 16-byte aligned, strides multiples of 8;
 *   lens int32 [B] in device memory;  out fp32 [B][Hq][D], contiguous.
 * D in {64, 128}; Hq % Hkv == 0 and G <= 16 (EUNSUPPORTED / EINVAL
 * otherwise).  ws: inv_decode_attention_workspace_bytes(B, Hq, D, max_len)
 * bytes, 256-byte aligned (EWORKSPACE).  Two launches on s.
 */
detred_status inv_decode_attention(const uint16_t *q, const uint16_t *k,
                                   const uint16_t *v, long kv_stride_b,
                                   long kv_stride_h, long kv_stride_t,
                                   const int *lens, float *out, int B, int Hq,
                                   int Hkv, int D, int max_len, float scale,
                                   void *ws, size_t ws_bytes, detred_stream s);

#ifdef __cplusplus
}
#endif

#endif /* DETRED_H */
