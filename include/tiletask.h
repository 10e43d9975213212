/*
 * tiletask.h -- C ABI of libtiletask: a GPT2 training step written as tile
 * tasks on one AMD Instinct MI355X (gfx950).
 *
 * Method. The pith.science review of NNTile ("What carries the argument")
 * describes the mechanism this library implements: every tensor is split
 * into tiles along all of its axes; every layer (embedding, linear, layer
 * norm, softmax, attention, cross-entropy, Adam update) becomes tasks that
 * read and write a few tiles, forward and backward; tasks are submitted in
 * program order (sequential task flow) and a runtime infers the ordering
 * between them from the tiles they touch, then maps ready tasks onto the
 * hardware and moves tiles between GPU and CPU memory on its own. The NNTile
 * arXiv index page ("Abstract") adds that the runtime, not the user, decides
 * where each task runs and when data moves. The NNTile README ("Minimal
 * working GPT example") gives the tile flags (batch, seq, embd, inner and
 * head tiles; seq, head and batch tiles must divide their axis, embd and
 * inner tiles need not) and the optimiser settings (fused AdamW, eps 1e-8,
 * weight decay 0.1, lr 3e-4, mean loss over the batch's tokens).
 *
 * Three layers of entry points:
 *   1. tile ops   -- tile_* : one kernel launch on raw device pointers;
 *   2. tasks      -- tt_ctx / tt_tensor / tt_submit_* : tiled tensors and the
 *                    sequential-task-flow executor;
 *   3. the model  -- tt_gpt2_* : the whole fwd + bwd + AdamW step.
 *
 * Conventions (all entry points):
 *   - Every function returns int: TT_OK (0) or a negative TT_ERR_* code;
 *     tt_last_error() returns a thread-local message for the last failure.
 *     Nothing throws across the ABI.
 *   - All floating point is IEEE fp32 (no TF32/xf32/bf16 anywhere).
 *   - "device" pointers are HIP device memory on the current device;
 *     "host" pointers are ordinary host memory. Streams are hipStream_t
 *     passed as void* (NULL = the default stream).
 *   - Tile ops are asynchronous on their stream; they validate arguments on
 *     the host (TT_ERR_ARG / TT_ERR_SHAPE) before launching and return
 *     TT_ERR_HIP if the launch fails. Size 0 problems are no-ops.
 *   - Matrices are row-major with an explicit leading dimension (elements).
 */
#ifndef TILETASK_H
#define TILETASK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---------------------------------------------------------------- errors */
#define TT_OK             0
#define TT_ERR_ARG       -1  /* null pointer, bad enum, negative size       */
#define TT_ERR_SHAPE     -2  /* tile/shape rule violated                     */
#define TT_ERR_OOM       -3  /* device or pinned-host allocation failed      */
#define TT_ERR_HIP       -4  /* a HIP call failed (launch, copy, event)      */
#define TT_ERR_STATE     -5  /* use after destroy, or a latched async fault  */
#define TT_ERR_UNSUPPORTED -6

const char* tt_last_error(void);
/* Library version string, e.g. "tiletask 0.1 gfx950". */
const char* tt_version(void);

/* tt_probe_mfma_f32 -- device peak probe, not part of the step: `blocks`
 * workgroups of 4 waves each issue `iters` x 4 independent fp32 matrix-core
 * products (32x32x2, 4096 flops each) with no memory traffic, so the launch
 * time gives the fp32 matrix throughput the GEMM and attention tiles are
 * measured against (published MI355X figure: 157.3 TFLOP/s). *flops (host,
 * may be NULL) receives blocks * 4 * iters * 4 * 4096. out: DEVICE float
 * [blocks * 256] (one sum per lane, so the work is not optimised away).
 * TT_ERR_ARG for blocks outside 1..65535, iters outside 1..2^24 or a null
 * out. Asynchronous on `stream`. */
int tt_probe_mfma_f32(void* stream, int64_t blocks, int64_t iters, float* out, double* flops);
/* tt_probe_hbm -- device bandwidth probe, not part of the step: one
 * grid-stride pass of `blocks` workgroups (256 threads, 16-byte accesses)
 * over n floats. mode TT_PROBE_READ sums src (n floats) and writes one sum
 * per thread to dst (blocks * 256 floats); TT_PROBE_WRITE fills dst (n
 * floats) with a constant; TT_PROBE_COPY copies src to dst (n floats each).
 * | TT_PROBE_NONTEMPORAL makes the loads and stores non-temporal. *bytes (host, may be
 * NULL) receives the bytes moved: 4n, or 8n for a copy. The launch time
 * gives the practical HBM rate of each traffic mix (published MI355X
 * figure: 8 TB/s). TT_ERR_ARG for an unknown mode, n not a multiple of 4,
 * blocks outside 1..65535, a null or misaligned buffer. Asynchronous on
 * `stream`. */
#define TT_PROBE_READ  0
#define TT_PROBE_WRITE 1
#define TT_PROBE_COPY  2
#define TT_PROBE_NONTEMPORAL 4
int tt_probe_hbm(void* stream, int mode, const float* src, float* dst, int64_t n, int64_t blocks,
                 double* bytes);

/* ============================================================ 1. tile ops */

/* tile_gemm -- the linear layer's tile task (forward Y = X W + b and its
 * backward dX = dY W^T, dW += X^T dY), and the tied LM head's z = n wte^T.
 * Layer list: pith.science review of NNTile, "What carries the argument".
 *
 *   acc = alpha * op(A) * op(B) + beta * S          (S = C, or aux for GELU)
 *   op(A) is m x k: A[i*lda + p] (transA = 0) or A[p*lda + i] (transA = 1)
 *   op(B) is k x n: B[p*ldb + j] (transB = 0) or B[j*ldb + p] (transB = 1)
 * Epilogue flags (bitwise or):
 *   TT_EPI_BIAS     acc += bias[j]                  (bias: n floats)
 *   TT_EPI_RES      acc += res[i*ldr + j]           (residual add)
 *   TT_EPI_GELU     S = aux; aux[i*ldaux+j] = acc; C = gelu_tanh(acc)
 *                   (the MLP activation, stored with its pre-activation)
 *   TT_EPI_GELU_BWD C = acc * gelu_tanh'(aux[i*ldaux+j])
 * When beta == 0, S is not read (it may hold NaNs). C, A, B must not alias
 * except that res may equal C (each element is read before it is written).
 * Arbitrary (ragged) m, n, k; any leading dimensions >= the row length.
 * Accumulation is fp32 on the matrix cores (MFMA). Deterministic.
 */
#define TT_EPI_NONE      0
#define TT_EPI_BIAS      1
#define TT_EPI_RES       2
#define TT_EPI_GELU      4
#define TT_EPI_GELU_BWD  8
#define TT_EPI_XSTATS   16  /* cross-entropy statistics: tile_gemm_batch_xstats and its task op only */
int tile_gemm(void* stream, int transA, int transB, int64_t m, int64_t n, int64_t k,
              float alpha, const float* A, int64_t lda, const float* B, int64_t ldb,
              float beta, float* C, int64_t ldc, int epilogue, const float* bias,
              const float* res, int64_t ldr, float* aux, int64_t ldaux);
/* tile_gemm with a device workspace (caller-owned, not used concurrently by
 * another launch). When C has too few 128x128 blocks to fill the GPU and K
 * is long, the K range is split over workgroups that write partial sums to
 * the workspace; a second kernel adds them in a fixed order (same result
 * on every run). tile_gemm_workspace(m, n, k) is the size that enables the
 * full split; smaller workspaces split less (0 bytes = no split). */
int tile_gemm_ws(void* stream, int transA, int transB, int64_t m, int64_t n, int64_t k,
                 float alpha, const float* A, int64_t lda, const float* B, int64_t ldb,
                 float beta, float* C, int64_t ldc, int epilogue, const float* bias,
                 const float* res, int64_t ldr, float* aux, int64_t ldaux,
                 void* workspace, size_t workspace_bytes);
size_t tile_gemm_workspace(int64_t m, int64_t n, int64_t k);
/* tile_gemm_ksum -- a sum of products into one tile:
 *   C = alpha * sum_{t < count} A_t op(B_t) + beta * C
 * with A_t [m x k[t]] (A_t[i*lda[t] + p]) and op(B_t) [k[t] x n]: B_t[p*ldb[t] + j]
 * (transB = 0) or B_t[j*ldb[t] + p] (transB = 1) -- a linear layer's input
 * gradient summed over tiles of its output axis: the LM head's dnf = sum over
 * vocab tiles of dz_v wte_v, and dX = sum_t dY_t W_t^T of the attention block's
 * q, k, v projections (tiled linear layer backward; pith.science review,
 * "What carries the argument"). A, B, k, lda, ldb are HOST arrays of `count`
 * entries (A[t], B[t] DEVICE pointers; read before the call returns). Runs of
 * pairs that share lda and ldb, with k[t] a multiple of the K step, 16-byte
 * aligned operands and m, n multiples of the block size go through one
 * long-K launch each (up to 96 pairs); any other pair runs on its own
 * through tile_gemm, accumulating. The pairs are summed in list order: same
 * result on every run. k[t] = 0 contributes nothing; count = 0 gives
 * C = beta*C. TT_ERR_ARG for negative sizes, a null array, or a pair with a
 * null operand or a leading dimension below its row length. */
int tile_gemm_ksum(void* stream, int count, int transB, int64_t m, int64_t n, const int64_t* k, float alpha,
                   const float* const* A, const int64_t* lda, const float* const* B, const int64_t* ldb,
                   float beta, float* C, int64_t ldc);
/* tile_gemm_ksum_ex -- the same sum followed by tile_gemm's epilogue on the
 * whole of it (TT_EPI_BIAS, TT_EPI_RES, TT_EPI_GELU with its pre-activation
 * in aux, TT_EPI_GELU_BWD; the arguments as in tile_gemm): a linear layer
 * whose input features are split over several tiles, e.g. the MLP's first
 * layer g = gelu(sum over embd tiles of n2_e W_e + b) as one long-K launch
 * instead of a chain of accumulating GEMMs (layer list: pith.science
 * review, "What carries the argument"). With an epilogue every pair must go
 * through the one long-K launch (as described above, at most 96 pairs with
 * equal leading dimensions): TT_ERR_UNSUPPORTED otherwise, before anything
 * is launched. epilogue = 0 is tile_gemm_ksum. */
int tile_gemm_ksum_ex(void* stream, int count, int transB, int64_t m, int64_t n, const int64_t* k, float alpha,
                      const float* const* A, const int64_t* lda, const float* const* B, const int64_t* ldb,
                      float beta, float* C, int64_t ldc, int epilogue, const float* bias, const float* res,
                      int64_t ldr, float* aux, int64_t ldaux);
/* tile_gemm_ksum_ws -- tile_gemm_ksum_ex with a DEVICE workspace (16-byte
 * aligned; null with 0 bytes = none). An output of at most 128 blocks
 * of 128 x 128 (m and n multiples of 128) then splits the concatenated K
 * steps of each long-K launch into up to 16 slices that run side by side
 * (about 512 workgroups), each summing its slice into its own m x n region
 * of the workspace; a second kernel adds the slices in slice order and
 * applies alpha, beta and the epilogue. Deterministic: same result on every
 * run. tile_gemm_ksum_workspace(m, n) is the size that allows the widest
 * split (0 where none applies); a smaller workspace splits less. TT_ERR_ARG
 * also for a null or misaligned workspace with nonzero bytes. */
size_t tile_gemm_ksum_workspace(int64_t m, int64_t n);
int tile_gemm_ksum_ws(void* stream, int count, int transB, int64_t m, int64_t n, const int64_t* k, float alpha,
                      const float* const* A, const int64_t* lda, const float* const* B, const int64_t* ldb,
                      float beta, float* C, int64_t ldc, int epilogue, const float* bias, const float* res,
                      int64_t ldr, float* aux, int64_t ldaux, void* workspace, size_t workspace_bytes);
/* tile_gemm_batch -- independent products in one launch:
 *   C_t = alpha * op(A_t) op(B_t) + beta * C_t,   t < count
 * op() as in tile_gemm; the products share transA, transB, k, alpha and
 * beta; each has its own m[t], n[t] and leading dimensions lda[t], ldb[t],
 * ldc[t]. The tied LM head runs one such product per vocab tile (forward
 * z_v = n wte_v^T and weight gradient dwte_v = dz_v^T n, the last vocab tile
 * ragged; tiled linear layer, pith.science review, "What carries the
 * argument"); the batch fills the GPU where each product alone would not.
 * m, n, A, lda, B, ldb, C, ldc are HOST arrays of `count` entries (device
 * pointers in A, B, C; read before the call returns). C_t must not overlap
 * C_u (u != t) or any A_u, B_u. Arbitrary (ragged) sizes; an operand whose
 * leading dimension is a multiple of 4 and whose base is 16-byte aligned is
 * loaded 16 bytes at a time, any other 4 (per product and operand);
 * products with a 4-byte operand are scheduled first. No epilogue, no
 * split-K. When beta == 0, C_t is not read. Up to 72 products
 * per launch (more make several launches). Deterministic. Products with
 * m[t] or n[t] = 0 are skipped; count = 0 does nothing. TT_ERR_ARG for a
 * negative size, a null array or operand, or a leading dimension below its
 * row length (or above 2^31 - 1). */
int tile_gemm_batch(void* stream, int count, int transA, int transB, const int64_t* m, const int64_t* n,
                    int64_t k, float alpha, const float* const* A, const int64_t* lda,
                    const float* const* B, const int64_t* ldb, float beta, float* const* C,
                    const int64_t* ldc);
/* tile_gemm_batch with a device workspace (caller-owned, not used
 * concurrently by another launch): when the products together have few
 * 128x128 blocks (at most 144) and K is long (>= 2048) -- the attention
 * block's q, k and v weight gradients, K = tokens -- K is split over
 * workgroups that write partial sums to the workspace, and one more kernel
 * adds them in slice order for every product (same result on every run).
 * tile_gemm_batch_workspace(count, m, n, k) is the size that enables the
 * split (0 = never splits); a smaller workspace disables it. */
int tile_gemm_batch_ws(void* stream, int count, int transA, int transB, const int64_t* m, const int64_t* n,
                       int64_t k, float alpha, const float* const* A, const int64_t* lda,
                       const float* const* B, const int64_t* ldb, float beta, float* const* C,
                       const int64_t* ldc, void* workspace, size_t workspace_bytes);
size_t tile_gemm_batch_workspace(int count, const int64_t* m, const int64_t* n, int64_t k);
/* tile_gemm_batch_xstats -- the tied LM head's logits with the statistics of
 * the cross-entropy in the epilogue (pith.science review, "What carries the
 * argument": the head and the loss are tile tasks; the softmax statistics
 * are taken from the logits while they are in registers instead of a second
 * pass over them). Product t: C_t = alpha A_t op(B_t) + beta C_t (A_t m x k,
 * transA = 0, op() as in tile_gemm), C_t holding vocab columns
 * v_off0 + t*v_tile .. + n[t] - 1 (n[t] <= v_tile) of m rows. Then, for every
 * row i and 64-column group q of C_t, with x the stored values of the
 * group's columns inside C_t:
 *   parts + t*part_stride + (q*m + i)*3 = { max x, sum exp(x - max x),
 *     x[labels[i] - v_off0 - t*v_tile - 64q] if that column is in the group, else 0 }
 * labels: DEVICE int32 [m]; parts: DEVICE, part_stride >= ceil(max n / 64)*m*3
 * floats. Always 128x128 blocks, no split; deterministic. The groups merge
 * with tile_xentropy_merge_groups. TT_ERR_ARG for null arrays, n[t] outside
 * 1..v_tile, a short part_stride, or more than 32767 products. */
int tile_gemm_batch_xstats(void* stream, int count, int transB, int64_t m, const int64_t* n, int64_t k,
                           float alpha, const float* const* A, const int64_t* lda, const float* const* B,
                           const int64_t* ldb, float beta, float* const* C, const int64_t* ldc,
                           const int32_t* labels, int64_t v_off0, int64_t v_tile, float* parts,
                           int64_t part_stride);

/* tile_layernorm_fwd -- layer norm over the embedding axis, split into
 * feature tiles (layer list: pith.science review, "What carries the
 * argument"; definition after the "Layer Normalization" paper the arXiv
 * index page lists under "Builds on"): y = (x - mean) * rstd * gamma + beta,
 * rstd = 1/sqrt(var + eps), var biased. Rows are tokens, columns a feature
 * tile of width cols starting at feature col_offset of a row of n_total.
 * Phases:
 *   TT_LN_PARTIAL  parts[r*3 + {0,1,2}] = (count, mean, M2) of this tile's row r
 *   TT_LN_MERGE    merges n_parts partial buffers (part i at parts + i*part_stride)
 *                  pairwise in order (Chan et al. update) -> stats[r*2 + {0,1}] =
 *                  (mean, rstd). x, gamma, beta, y unused.
 *   TT_LN_APPLY    y = (x - mean) * rstd * gamma + beta using stats
 *   TT_LN_FUSED    the row fits this tile (cols == n_total): computes stats
 *                  and y in one pass.
 * gamma/beta point at this tile's cols entries. x/y: rows x cols, ld ldx/ldy.
 */
#define TT_LN_PARTIAL 0
#define TT_LN_MERGE   1
#define TT_LN_APPLY   2
#define TT_LN_FUSED   3
int tile_layernorm_fwd(void* stream, int phase, int64_t rows, int64_t cols,
                       const float* x, int64_t ldx, const float* gamma, const float* beta,
                       float* parts, int64_t n_parts, int64_t part_stride,
                       float* stats, float* y, int64_t ldy, float eps);

/* tile_layernorm_bwd -- gradient of tile_layernorm_fwd.
 * With xhat = (x - mean) * rstd and dxhat = dy * gamma:
 *   TT_LN_PARTIAL  parts[r*2 + {0,1}] = (sum dxhat, sum dxhat*xhat) over this tile
 *   TT_LN_APPLY    sums the n_parts partials (part i at parts + i*part_stride) in
 *                  order and writes dx = rstd*(dxhat - S1/n_total - xhat*S2/n_total);
 *                  if dx_acc != 0, dx is added to the existing contents of dx
 *                  (the residual-stream gradient).
 *   TT_LN_FUSED    cols == n_total: PARTIAL and APPLY in one pass.
 * APPLY and FUSED also accumulate dgamma[c] += sum_r dy*xhat and
 * dbeta[c] += sum_r dy (deterministic two-stage column sums through
 * `workspace`, which must hold tile_layernorm_bwd_workspace(rows, cols)
 * bytes and must not be used concurrently by another launch).
 */
int tile_layernorm_bwd(void* stream, int phase, int64_t rows, int64_t cols, int64_t n_total,
                       const float* dy, int64_t lddy, const float* x, int64_t ldx,
                       const float* gamma, const float* stats,
                       float* parts, int64_t n_parts, int64_t part_stride,
                       float* dx, int64_t lddx, int dx_acc, float* dgamma, float* dbeta,
                       void* workspace);
size_t tile_layernorm_bwd_workspace(int64_t rows, int64_t cols);

/* tile_layernorm_fwd_multi / tile_layernorm_bwd_multi -- the layer norm of
 * one block of rows whose features are split over `count` tiles (2..16),
 * in one pass over the tiles instead of the partial / merge / apply phases
 * (layer list: pith.science review, "What carries the argument";
 * definition after the "Layer Normalization" paper on the arXiv index
 * page). Tile t is rows x cols[t] floats, row-major with leading dimension
 * cols[t], at x[t] (dy[t], y[t], dx[t]); gamma[t], beta[t], dgamma[t],
 * dbeta[t] hold cols[t] floats. x, gamma, beta, dy, y, dx and the workspace
 * are DEVICE memory aligned to 16 bytes; the pointer arrays and cols are
 * HOST arrays read before the call returns. Every tile is as wide as the
 * first except the last, which may be narrower; widths are multiples of 4
 * and sum to at most 16384 (TT_ERR_SHAPE otherwise).
 *   forward:  stats[r*2 + {0,1}] = (mean, rstd) of row r over all the tiles'
 *             features; y = (x - mean) * rstd * gamma + beta.
 *   backward: dx = rstd*(dxhat - mean(dxhat) - xhat*mean(dxhat*xhat)) with
 *             dxhat = dy*gamma, added to dx's contents when dx_acc != 0;
 *             dgamma += sum_rows dy*xhat, dbeta += sum_rows dy, in a fixed
 *             order through `workspace` (at least
 *             tile_layernorm_bwd_multi_workspace(rows, sum of cols) bytes,
 *             not used concurrently by another launch).
 * Same arithmetic as the single-tile FUSED phase up to summation order. */
int tile_layernorm_fwd_multi(void* stream, int count, int64_t rows, const int64_t* cols, const float* const* x,
                             const float* const* gamma, const float* const* beta, float* stats, float* const* y,
                             float eps);
int tile_layernorm_bwd_multi(void* stream, int count, int64_t rows, const int64_t* cols, const float* const* dy,
                             const float* const* x, const float* const* gamma, const float* stats, float* const* dx,
                             int dx_acc, float* const* dgamma, float* const* dbeta, void* workspace,
                             size_t workspace_bytes);
size_t tile_layernorm_bwd_multi_workspace(int64_t rows, int64_t total_cols);

/* tile_rmsnorm_fwd / tile_rmsnorm_bwd -- the LLaMA block's normalisation
 * (RMSNorm: the published LLaMA architecture; the NNTile README's notebook
 * list names LLaMa as its second model) over one block of rows whose
 * features are split over `count` tiles (1..16), with the tile layout and
 * pointer conventions of tile_layernorm_fwd_multi above (widths multiples
 * of 4, equal but for a narrower last tile, at most 16384 in all; DEVICE
 * data aligned to 16 bytes; HOST pointer arrays and cols).
 *   forward:  rstd[r] = 1 / sqrt(mean over the row's features of x^2 + eps);
 *             y = x * rstd * gamma (no mean, no shift).
 *   backward: with n = x * rstd and dn = dy * gamma,
 *             dx = rstd * (dn - n * mean(dn * n)), added to dx's contents
 *             when dx_acc != 0; dgamma += sum_rows dy * n in a fixed order
 *             through `workspace` (at least tile_rmsnorm_bwd_workspace(rows,
 *             sum of cols) bytes, not used concurrently by another launch).
 * TT_ERR_ARG / TT_ERR_SHAPE for bad arguments, before anything runs. */
int tile_rmsnorm_fwd(void* stream, int count, int64_t rows, const int64_t* cols, const float* const* x,
                     const float* const* gamma, float* rstd, float* const* y, float eps);
int tile_rmsnorm_bwd(void* stream, int count, int64_t rows, const int64_t* cols, const float* const* dy,
                     const float* const* x, const float* const* gamma, const float* rstd, float* const* dx,
                     int dx_acc, float* const* dgamma, void* workspace, size_t workspace_bytes);
size_t tile_rmsnorm_bwd_workspace(int64_t rows, int64_t total_cols);

/* tile_rope_table / tile_rope -- rotary position embedding of q and k (the
 * published LLaMA architecture; the README's notebook list names LLaMa).
 * tile_rope_table fills table[t*hd + i] = cos(t * base^(-2i/hd)) and
 * table[t*hd + hd/2 + i] = sin(same) for t < seq, i < hd/2 (DEVICE float
 * [seq, hd], angles and functions in double precision, rounded once).
 * tile_rope rotates, in place, the pair (x_i, x_{i+hd/2}) of every head of
 * every row of a q or k tile: x is DEVICE [rows, heads, hd] (rows = batch
 * x length of the tile, row-major, 16-byte aligned); row r has position
 * pos_off + r % seq_len, which must lie below table_rows. inverse != 0
 * applies the transposed rotation (the backward). hd in {16, 32, 64, 128}.
 * TT_ERR_ARG / TT_ERR_SHAPE for bad arguments, TT_ERR_ARG also for more
 * work than one launch covers (2^31 workgroups of 256 threads). */
int tile_rope_table(void* stream, int64_t seq, int64_t hd, double base, float* table);
int tile_rope(void* stream, float* x, int64_t rows, int64_t heads, int64_t hd, int64_t seq_len,
              int64_t pos_off, const float* table, int64_t table_rows, int inverse);
/* tile_rope_multi -- tile_rope on 1..4 tiles of equal shape in one launch
 * (a q and a k tile); x is a HOST array of DEVICE pointers. */
int tile_rope_multi(void* stream, int count, float* const* x, int64_t rows, int64_t heads, int64_t hd,
                    int64_t seq_len, int64_t pos_off, const float* table, int64_t table_rows, int inverse);
/* tile_swiglu_fwd / tile_swiglu_bwd -- the LLaMA MLP's gate over n
 * contiguous DEVICE floats: h = silu(a) * b, silu(a) = a / (1 + exp(-a));
 * backward da = dh * b * silu'(a), db = dh * silu(a). da and db may be a
 * and b themselves (in place). TT_ERR_ARG for n < 0, null pointers or more
 * elements than one launch covers (2^31 workgroups of 1024). */
int tile_swiglu_fwd(void* stream, int64_t n, const float* a, const float* b, float* h);
int tile_swiglu_bwd(void* stream, int64_t n, const float* dh, const float* a, const float* b, float* da,
                    float* db);

/* tile_layernorm_bwd_noalloc -- for callers that cannot allocate (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): tile_layernorm_bwd with the same arguments and results except
 * the workspace, whose column partials live in a device array of the
 * library instead (16 MiB per device, held until the process ends;
 * tile_layernorm_bwd_noalloc_max_bytes() returns the size). The array's
 * device address is looked up on the first call on each device, so make
 * that call outside a graph capture. Calls no allocating routine. Every
 * call on one device uses the same array: calls that overlap on a device
 * (on two streams at once) race, calls in stream order do not. TT_ERR_ARG
 * when tile_layernorm_bwd_workspace(rows, cols) exceeds the array, before
 * anything is launched; otherwise as tile_layernorm_bwd. */
int tile_layernorm_bwd_noalloc(void* stream, int phase, int64_t rows, int64_t cols, int64_t n_total,
                               const float* dy, int64_t lddy, const float* x, int64_t ldx, const float* gamma,
                               const float* stats, float* parts, int64_t n_parts, int64_t part_stride, float* dx,
                               int64_t lddx, int dx_acc, float* dgamma, float* dbeta);
size_t tile_layernorm_bwd_noalloc_max_bytes(void);

/* tile_softmax -- row softmax of a tile whose columns are one tile of a
 * longer row (layer list: pith.science review, "What carries the argument").
 * Element (r, c) of the tile is logit x = scale * X[r*ldx + c] at global
 * column col_offset + c; with causal != 0 it is masked (-inf) when
 * col_offset + c > row_offset + r.
 *   TT_SM_STATS  parts[r*3 + {0,1,2}] = (row max, sum exp(x - max), picked)
 *                where picked = x at column labels[r] if labels != NULL and the
 *                label falls in this tile, else 0. Fully masked rows give
 *                (-inf, 0, 0).
 *   TT_SM_MERGE  lse[r] = logsumexp over the n_parts partials (part i at
 *                parts + i*part_stride), merged in order by rescaling to the
 *                larger max; if row_loss != NULL also row_loss[r] =
 *                lse[r] - sum_i picked_i (the cross-entropy of row r).
 *   TT_SM_APPLY  Y = (exp(x - lse[r]) - [labels && col == labels[r]]) * grad_scale;
 *                Y may equal X (in place).
 */
#define TT_SM_STATS 0
#define TT_SM_MERGE 1
#define TT_SM_APPLY 2
int tile_softmax(void* stream, int phase, int64_t rows, int64_t cols,
                 int64_t row_offset, int64_t col_offset, float scale, int causal,
                 const float* X, int64_t ldx, const int32_t* labels,
                 float* parts, int64_t n_parts, int64_t part_stride,
                 float* lse, float* row_loss, float* Y, int64_t ldy, float grad_scale);

/* tile_xentropy -- mean cross-entropy over all tokens of the batch (NNTile
 * README, "Minimal working GPT example": the reported loss is the mean over
 * the batch's tokens). Builds on tile_softmax's STATS/MERGE/APPLY:
 *   TT_XE_LOSS  loss[0] = (accumulate ? loss[0] : 0) + inv_n * sum_r row_loss[r]
 *               over `rows` rows, summed in a fixed order (deterministic).
 *   TT_XE_GRAD  logits (rows x v_len tile at vocab offset v_off, ld ldz) are
 *               replaced in place by dz = (softmax - onehot(labels)) * inv_n.
 */
#define TT_XE_LOSS 0
#define TT_XE_GRAD 1
int tile_xentropy(void* stream, int phase, int64_t rows, int64_t v_len, int64_t v_off,
                  const int32_t* labels, float* logits, int64_t ldz, const float* lse,
                  const float* row_loss, float* loss, int accumulate, float inv_n);
/* tile_xentropy_multi -- the cross-entropy sweeps over several vocab tiles
 * of one token tile in one launch (the LM head's logits, one tile per vocab
 * tile; NNTile README, "Minimal working GPT example": mean loss over the
 * batch's tokens). Alone, each tile is a few microseconds of HBM traffic,
 * too little to fill the GPU.
 *   TT_XE_STATS parts[t*part_stride + r*3 + {0,1,2}] = (row max, sum of
 *               exp(z - max), z[r][labels[r] - v_off[t]] when that column is
 *               in tile t else 0): tile_softmax(TT_SM_STATS) of each tile,
 *               ready for TT_SM_MERGE
 *   TT_XE_GRAD  each tile replaced in place by (softmax - onehot(labels)) *
 *               inv_n, given lse from TT_SM_MERGE: tile_xentropy(TT_XE_GRAD)
 *               of each tile
 * Tile t is rows x v_len[t] floats at logits[t] with leading dimension
 * ldz[t] and vocab offset v_off[t]; v_len, v_off, logits, ldz are HOST
 * arrays of `count` entries (device pointers in logits, read before the
 * call returns). v_len[t] in [1, 2048], rows <= 65535, up to 64 tiles per
 * launch (more make several launches). Same results as the per-tile calls.
 * TT_ERR_ARG / TT_ERR_SHAPE for bad arguments. */
#define TT_XE_STATS 2
int tile_xentropy_multi(void* stream, int phase, int count, int64_t rows, const int64_t* v_len,
                        const int64_t* v_off, const int32_t* labels, float* const* logits,
                        const int64_t* ldz, float* parts, int64_t part_stride, const float* lse,
                        float inv_n);
/* tile_xentropy_merge_groups -- lse and per-row loss from group partials
 * (tile_gemm_batch_xstats): tile t holds ceil(v_len[t] / group) partials
 * of rows x 3 floats at parts + t*part_stride (group-major), each (max, sum
 * exp(x - max), picked target logit). lse[r] = logsumexp over all of them,
 * row_loss[r] (may be NULL) = lse[r] - sum of the picked logits. One wave
 * per row, each lane merging every 64th partial in order, then a fixed xor
 * tree: deterministic. v_len: HOST array of `count` entries. TT_ERR_ARG for
 * null pointers, rows > 65535, group < 1 or v_len[t] < 1. */
int tile_xentropy_merge_groups(void* stream, int64_t rows, int count, const int64_t* v_len, int group,
                               const float* parts, int64_t part_stride, float* lse, float* row_loss);

/* tile_attention_fwd -- causal multi-head scaled dot-product attention for
 * one (query tile, key tile) pair (layer list: pith.science review; the
 * "Attention Is All You Need" paper listed under "Builds on"; the README's
 * flash-attention flag reorders work to save memory, which this online
 * softmax does). Q/O tiles hold batch x q_len tokens x heads x hd, K/V
 * tiles batch x k_len x heads x hd, token-major:
 *   Q[((b*q_len + t)*heads + h)*hd + e]       (row stride heads*hd)
 * Query t has global position q_off + t, key s position k_off + s; keys
 * with k_off + s > q_off + t are masked. scale is usually 1/sqrt(hd).
 * State carried across the key tiles of one query tile:
 *   O   unnormalised accumulator (same layout as Q),
 *   ml  running (max, sum) per (b, h, t): ml[((b*heads + h)*q_len + t)*2 + {0,1}],
 *   lse logsumexp per (b, h, t):          lse[(b*heads + h)*q_len + t].
 * first != 0 starts from (max = -inf, sum = 0, O = 0); last != 0 finishes:
 * O /= sum and lse = max + log(sum). A single key tile uses first = last = 1.
 * hd must be 16, 32, 64 or 128.
 */
int tile_attention_fwd(void* stream, int64_t batch, int64_t heads, int64_t q_len, int64_t k_len,
                       int64_t hd, int64_t q_off, int64_t k_off, const float* Q, const float* K,
                       const float* V, float* O, float* ml, float* lse, int first, int last,
                       float scale);

/* tile_attention_bwd -- gradient of tile_attention_fwd for one tile pair.
 *   TT_ATT_PREP  Dvec[(b*heads+h)*q_len + t] = sum_e dO*O over the query tile
 *                (K, V, dQ, dK, dV unused).
 *   TT_ATT_GRAD  with P = exp(scale*Q K^T - lse) (masked causally):
 *                dV += P^T dO; dS = P * (dO V^T - Dvec); dQ += scale * dS K;
 *                dK += scale * dS^T Q.
 *                acc_dq / acc_dkv = 0 overwrite dQ / (dK, dV) instead of adding.
 * Layouts as tile_attention_fwd. Deterministic (no atomics).
 */
#define TT_ATT_PREP 0
#define TT_ATT_GRAD 1
int tile_attention_bwd(void* stream, int phase, int64_t batch, int64_t heads, int64_t q_len,
                       int64_t k_len, int64_t hd, int64_t q_off, int64_t k_off,
                       const float* Q, const float* K, const float* V, const float* O,
                       const float* dO, const float* lse, float* Dvec,
                       float* dQ, float* dK, float* dV, int acc_dq, int acc_dkv, float scale);

/* tile_attention_bwd_ws -- tile_attention_bwd with a caller-owned device
 * workspace of at least tile_attention_bwd_workspace(batch, heads, q_len,
 * k_len) bytes, 16-byte aligned. TT_ATT_GRAD then computes S, dP and dS once
 * per 32 x 32 block of the pair (dK/dV kernel), stores dS there and forms
 * dQ += scale * dS K from it (dQ kernel): five matrix products per block
 * instead of the seven of the recomputing form. Same results up to rounding
 * order; deterministic. A null, misaligned or short workspace selects the
 * recomputing form. The workspace holds no state between calls; calls that
 * share one must be ordered (same stream).
 */
size_t tile_attention_bwd_workspace(int64_t batch, int64_t heads, int64_t q_len, int64_t k_len);
int tile_attention_bwd_ws(void* stream, int phase, int64_t batch, int64_t heads, int64_t q_len,
                          int64_t k_len, int64_t hd, int64_t q_off, int64_t k_off,
                          const float* Q, const float* K, const float* V, const float* O,
                          const float* dO, const float* lse, float* Dvec,
                          float* dQ, float* dK, float* dV, int acc_dq, int acc_dkv, float scale,
                          void* workspace, size_t workspace_bytes);

/* tile_fused_adamw -- one decoupled-weight-decay Adam step over one
 * parameter tile, one pass over p, g, m, v (NNTile README, "Minimal working
 * GPT example": fused AdamW; the "Decoupled Weight Decay Regularization"
 * paper listed on the arXiv index page under "Builds on"):
 *   p *= 1 - lr*wd;  m = b1 m + (1-b1) g;  v = b2 v + (1-b2) g^2;
 *   p -= lr * (m / bc[0]) / (sqrt(v / bc[1]) + eps)
 * bias_corr is DEVICE memory holding bc = {1 - b1^t, 1 - b2^t} (so a
 * captured step stays valid as t advances; see tile_adamw_advance).
 */
int tile_fused_adamw(void* stream, int64_t n, float* p, const float* g, float* m, float* v,
                     float lr, float beta1, float beta2, float eps, float weight_decay,
                     const float* bias_corr);
/* tile_fused_adamw_multi -- the same update on `count` tiles (0 <= count <=
 * TT_ADAMW_MAX_TILES) in one launch: tile i has n[i] elements at p[i],
 * g[i], m[i], v[i]. The pointer arrays and n are HOST arrays of DEVICE
 * pointers, read before the call returns. Each element gets exactly the
 * arithmetic of tile_fused_adamw. TT_ERR_ARG for a count out of range, a
 * negative size or a null pointer of a non-empty tile. */
#define TT_ADAMW_MAX_TILES 16
int tile_fused_adamw_multi(void* stream, int count, float* const* p, const float* const* g,
                           float* const* m, float* const* v, const int64_t* n, float lr, float beta1,
                           float beta2, float eps, float weight_decay, const float* bias_corr);
/* tile_sgd -- plain stochastic-gradient step on one tile (the pith.science
 * review's "What carries the argument" lists Adam and SGD as the tile-wise
 * updates; the README's --optimizer flag picks one): p[i] -= lr * g[i] for
 * i < n. p and g are DEVICE arrays (16-byte aligned ones take the float4
 * path). No momentum, no weight decay. TT_ERR_ARG for n < 0 or a null
 * pointer with n > 0. */
int tile_sgd(void* stream, int64_t n, float* p, const float* g, float lr);
/* tile_sgd_multi -- the same step on `count` tiles (0 <= count <=
 * TT_SGD_MAX_TILES) in one launch: tile i has n[i] elements at p[i], g[i]
 * (HOST arrays of DEVICE pointers, read before the call returns); each
 * element gets exactly tile_sgd's arithmetic. TT_ERR_ARG for a count out of
 * range, a negative size or a null pointer of a non-empty tile. */
#define TT_SGD_MAX_TILES 16
int tile_sgd_multi(void* stream, int count, float* const* p, const float* const* g, const int64_t* n, float lr);
/* tile_adamw_advance -- device-side step counter: t = ++(*step) and
 * bias_corr = {1 - beta1^t, 1 - beta2^t} (step: device int32, bias_corr: device
 * float[2]). One tiny launch per optimiser step. */
int tile_adamw_advance(void* stream, int32_t* step, float* bias_corr, float beta1, float beta2);

/* ---- auxiliary tile ops of the embedding layer and the linear backward ---- */

/* tile_embedding_fwd -- token + position embedding for one (token tile, embd
 * tile): out[r*ldo + c] = wte[(ids[r] - v_off)*ld_wte + c] + wpe[pos_r*ld_wpe + c]
 * with pos_r = pos_offset + (r % seq_len), for the rows whose id lies in
 * [v_off, v_off + v_len); wte points at that [v_len x cols] slab of the table
 * (one vocab tile, or with v_off = 0 and v_len = vocab a whole embd tile
 * column of the tiled table, which is contiguous) and wpe at a
 * [positions x cols] slab. Other rows are left untouched, except that rows
 * whose id is outside [0, vocab) get NaN when v_off == 0 -- ids are checked
 * on the device and never read out of bounds. wpe may be NULL: no position
 * term (a model without a position table; ld_wpe is then ignored). */
int tile_embedding_fwd(void* stream, int64_t rows, int64_t cols, const int32_t* ids, int64_t vocab,
                       int64_t v_off, int64_t v_len, const float* wte, int64_t ld_wte, const float* wpe,
                       int64_t ld_wpe, int64_t seq_len, int64_t pos_offset, float* out, int64_t ldo);

/* tile_embedding_index -- stable sort of one token tile's ids: sorted_ids
 * ascending and perm (original row of each sorted entry), ties in row order.
 * rows <= 65536. Used by tile_embedding_bwd for a deterministic scatter-add. */
int tile_embedding_index(void* stream, int64_t rows, const int32_t* ids, int32_t* sorted_ids,
                         int32_t* perm);

/* tile_embedding_bwd -- dwte rows of one vocab tile [v_off, v_off + v_len):
 * dwte[(id - v_off)*ld_dwte + c] += sum of dh[r*lddh + c] over rows r with
 * ids[r] == id, added in row order (from tile_embedding_index's output).
 * TT_EMB_POS phase instead accumulates the position gradient of one
 * (batch tile x seq tile) token tile: dwpe[t*ld + c] += sum_b dh[(b*seq_len + t)*lddh + c]
 * for batch = rows / seq_len. */
#define TT_EMB_TOKEN 0
#define TT_EMB_POS   1
int tile_embedding_bwd(void* stream, int phase, int64_t rows, int64_t cols,
                       const int32_t* sorted_ids, const int32_t* perm,
                       int64_t v_off, int64_t v_len, int64_t seq_len,
                       const float* dh, int64_t lddh, float* dst, int64_t ld_dst);

/* tile_reduce_rows -- bias gradient of the linear layer:
 * out[c] = (beta ? out[c] : 0) + sum_r X[r*ldx + c], in a fixed order
 * (two-stage through `workspace` of tile_reduce_rows_workspace(rows, cols)
 * bytes). */
int tile_reduce_rows(void* stream, int64_t rows, int64_t cols, const float* X, int64_t ldx,
                     float* out, int beta, void* workspace);
size_t tile_reduce_rows_workspace(int64_t rows, int64_t cols);
/* tile_reduce_rows_multi -- tile_reduce_rows of up to 16 tiles that share
 * the row count, in one pair of launches (the attention block's q, k and v
 * bias gradients: one column sum per tile, each alone a few microseconds):
 * out_t[c] = (beta ? out_t[c] : 0) + sum_r X_t[r*ldx[t] + c], c < cols[t].
 * cols, X, ldx, out are HOST arrays of `count` entries (device pointers in X
 * and out). The workspace holds every tile's partial rows: at least
 * sum_t tile_reduce_rows_workspace(rows, cols[t]) bytes (TT_ERR_ARG when
 * smaller). Same result as the per-tile calls (fixed order, deterministic). */
int tile_reduce_rows_multi(void* stream, int count, int64_t rows, const int64_t* cols, const float* const* X,
                           const int64_t* ldx, float* const* out, int beta, void* workspace,
                           size_t workspace_bytes);

/* tile_fill -- dst[i] = value for i < n. tile_split_tokens -- from a window
 * array tokens[b*(seq+1) + t] (int32), ids[b*seq + t] = tokens[b*(seq+1)+t]
 * and labels[b*seq + t] = tokens[b*(seq+1)+t+1] for b < batch, t < seq. */
int tile_fill(void* stream, int64_t n, float* dst, float value);
/* tile_fill_multi -- the same on `count` tiles (0 <= count <=
 * TT_FILL_MAX_TILES) in one launch: dst[i][0..n[i]) = value. dst and n are
 * HOST arrays (dst of DEVICE pointers), read before the call returns.
 * TT_ERR_ARG for a count out of range, a negative size or a null pointer of
 * a non-empty tile. */
#define TT_FILL_MAX_TILES 16
int tile_fill_multi(void* stream, int count, float* const* dst, const int64_t* n, float value);
int tile_split_tokens(void* stream, int64_t batch, int64_t seq, const int32_t* tokens,
                      int32_t* ids, int32_t* labels);

/* ================================================= 2. tensors and tasks */

typedef struct tt_ctx tt_ctx;
typedef struct tt_tensor tt_tensor;

#define TT_MAX_DIMS 6
#define TT_F32 0
#define TT_I32 1
#define TT_HOME_DEVICE      0   /* tiles live in HBM */
#define TT_HOME_PINNED_HOST 1   /* tiles live in pinned host RAM, staged on use */
#define TT_HOME_PINNED_STATE 2  /* tt_gpt2_create / tt_llama_create param_home only: parameters and
                                   AdamW moments pinned host, gradients in HBM */
#define TT_DEVICE_DRYRUN   -1   /* tt_ctx_create: no GPU, tasks recorded only */

/* Context: owns n_streams HIP streams (default priority), their events and
 * per-stream workspaces, and the device arena of its tensors. device =
 * TT_DEVICE_DRYRUN builds a context that runs nothing: tensors get no
 * memory, submitted tasks are recorded with their inferred dependencies and
 * stream choice and can be dumped (tt_dump_dag); this is how the executor's
 * dependency inference is tested without a GPU. device_budget_bytes is the
 * size of the device arena that holds copies of tiles whose home is pinned
 * host (0 = half of the free device memory at first use). Such a tile is
 * copied in (copy stream, H2D) before a task that reads it runs, and the
 * tiles the next 4 tasks read are prefetched; when the arena is full the
 * least recently used tile that the launching task does not access is
 * evicted, written back first if a task changed it. Results do not depend
 * on the budget. TT_ERR_OOM (latched, reported by the submit or wait that
 * launches it) when the tiles of one task do not fit.
 * window = number of submitted tasks held before they are launched
 * (0 = default 512); a larger window gives the stream assignment more
 * look-ahead. One submitting thread per context. */
int tt_ctx_create(int device, int n_streams, int window, size_t device_budget_bytes, tt_ctx** out);
/* tt_ctx_create_on_streams -- tt_ctx_create whose tasks run on n_streams
 * HIP streams the caller owns (a HOST array of hipStream_t handles, e.g.
 * torch streams) of that device: the context does not create, and on
 * destruction does not destroy, them; they must stay valid until
 * tt_ctx_destroy returns. Work
 * the caller queues on them interleaves with the tasks in stream order
 * (use tt_ctx_wait_stream / tt_ctx_join_stream for other streams). The
 * context still creates its own copy streams for pinned-host tiles.
 * TT_ERR_ARG for the dry-run device, a null array, a null (legacy
 * default) stream, or the same stream twice. */
int tt_ctx_create_on_streams(int device, int n_streams, void* const* streams, int window,
                             size_t device_budget_bytes, tt_ctx** out);
int tt_ctx_destroy(tt_ctx* ctx);
/* hipStream_t of executor stream i (for callers that want to order their own
 * work after the context's). */
int tt_ctx_stream(tt_ctx* ctx, int i, void** stream);
/* Launch the tasks submitted from now on on streams 0..n-1 only (1 <= n <=
 * n_streams; TT_ERR_ARG otherwise). n = 1 runs the task graph in submission
 * order on one stream, so every kernel has the GPU to itself (per-task
 * timing); results do not depend on n. */
int tt_ctx_streams_active(tt_ctx* ctx, int n);
/* Heavy lane (min_flops > 0, with at least 2 active streams): tasks whose
 * flop estimate (GEMM 2mnk, attention 4·hd per visible pair forward, 10·hd
 * backward) is at least min_flops run in submission order on stream 0,
 * every other task on streams 1..n-1. A kernel that fills every CU gains
 * nothing from sharing the GPU with another one; the light memory-bound
 * tasks still overlap with it. 0 = off (default). Results do not change. */
int tt_ctx_heavy_lane(tt_ctx* ctx, double min_flops);
/* Critical-path priorities (whole-iteration scheduling, which the
 * pith.science review's "Reading between the lines" names as the lever):
 * with on != 0, each window of submitted tasks is launched as a list
 * schedule instead of in submission order: among the tasks whose
 * dependencies have been launched, the one with the costliest chain of
 * flops to the end of the window goes first (memory-bound tasks count as
 * 1 MFLOP). The order stays topological and the kernels are the same, so
 * results do not change; with several streams, the critical path reaches
 * the GPU first. Contexts with pinned-host tensors keep submission order
 * (their staging plan follows it). Off by default. Dry-run DAG dumps list
 * tasks in launch order. */
int tt_ctx_priorities(tt_ctx* ctx, int on);
/* Keep (on != 0) or drop the per-task records tt_dump_dag writes; dry-run
 * contexts record by default, device contexts do not. */
int tt_ctx_record(tt_ctx* ctx, int on);

/* Tiled tensor: shape[d] split into tiles of tile_shape[d] (the last tile of
 * an axis is ragged when tile_shape[d] does not divide shape[d]). Storage is
 * tile-major: each tile is one contiguous row-major block of its own extent;
 * tiles are laid out in grid order with the FIRST grid axis varying fastest,
 * so for a matrix all tiles of one tile-column form one contiguous row-major
 * slab. Memory is owned by the tensor (home = TT_HOME_*). */
int tt_tensor_create(tt_ctx* ctx, int ndim, const int64_t* shape, const int64_t* tile_shape,
                     int dtype, int home, tt_tensor** out);
/* Same, over caller-owned device memory of tt_tensor_bytes() bytes laid out
 * as above; the memory must outlive the tensor. */
int tt_tensor_wrap(tt_ctx* ctx, int ndim, const int64_t* shape, const int64_t* tile_shape,
                   int dtype, void* device_base, tt_tensor** out);
int tt_tensor_destroy(tt_tensor* t);
/* Matrix view of every tile: rows = product of the tile's extents over the
 * first k axes, cols = product over the rest (0 <= k <= ndim; default
 * ndim - 1). Token-major activations with a head axis, [B, T, H, hd] tiled
 * [bt, st, ht, hd], take k = 2 so that a tile is the [bt*st, ht*hd] matrix a
 * linear layer writes. Set it before the tensor's first task. TT_ERR_ARG for
 * k out of range. */
int tt_tensor_set_matrix_split(tt_tensor* t, int k);
int64_t tt_tensor_bytes(const tt_tensor* t);
/* Number of tiles along axis d, and the total. */
int tt_tensor_grid(const tt_tensor* t, int64_t* grid_out /* ndim */, int64_t* ntiles);
/* Device pointer and extent of one tile, after waiting for every submitted
 * task. TT_ERR_UNSUPPORTED for a tensor whose home is pinned host: its
 * device copy lives in the context's arena only while tasks use it. */
int tt_tensor_tile(tt_tensor* t, const int64_t* tile_idx, void** dev_ptr, int64_t* extent);
/* Dense row-major host array <-> tiled tensor (synchronous; waits for the
 * tensor's pending tasks). */
int tt_tensor_copy_in(tt_tensor* t, const void* dense_host);
int tt_tensor_copy_out(tt_tensor* t, void* dense_host);

/* Task submission in sequential task flow order. Each call records the
 * task's tile accesses, derives read-after-write, write-after-read and
 * write-after-write edges against earlier tasks, and queues the task; tasks
 * are launched in submission order onto the context's streams, with event
 * waits for edges that cross streams. */
#define TT_R  1
#define TT_W  2
#define TT_RW 3
typedef struct {
    tt_tensor* tensor;
    int64_t tile[TT_MAX_DIMS];
    int mode;            /* TT_R, TT_W or TT_RW */
} tt_access;
/* TT_W promises that the task overwrites EVERY element of the tile: for a
 * pinned-host tile no copy-in precedes it. A task that updates part of a
 * tile declares TT_RW. Accesses of one task to the same tile merge (any
 * write makes the merged access a write). */
/* A task that only declares accesses (runs nothing); label <= 31 chars. */
int tt_submit_nop(tt_ctx* ctx, const char* label, const tt_access* acc, int n_acc);
/* C(ic) = alpha op(A(ia)) op(B(ib)) + beta C(ic) on 2-D tiles (extents must
 * agree after transposition; TT_ERR_SHAPE otherwise). Accesses: A R, B R,
 * C W when beta == 0 else RW. */
int tt_submit_gemm(tt_ctx* ctx, int transA, int transB, float alpha,
                   tt_tensor* A, const int64_t* ia, tt_tensor* B, const int64_t* ib,
                   float beta, tt_tensor* C, const int64_t* ic);
/* Every element of tile idx = value (access W). */
int tt_submit_fill(tt_ctx* ctx, tt_tensor* t, const int64_t* idx, float value);
/* ---- generic task submission: every tile op as a task over tiled tensors
 *
 * The pith.science review of NNTile ("What carries the argument") describes
 * the programming model: every layer of the network is expressed as tasks
 * that read and write a few tiles, submitted in program order; the runtime
 * derives the ordering from those reads and writes. tt_submit is that
 * interface for every tile op of this library: `op` names the operation,
 * `tiles` lists the tiles it touches in the order given below, `scalars`
 * points at the op's scalar struct (scalars_size = its sizeof; NULL and 0
 * for ops without one). The access mode of each tile (read, write, update)
 * is implied by the op and its scalars, as listed; the executor turns them
 * into read-after-write, write-after-read and write-after-write edges.
 *
 * Tiles are addressed by tensor and tile index. A 2-D "matrix view" of a
 * tile is rows x cols where rows is the product of the tile's extents over
 * all axes but the last and cols the last extent (for a tensor created with
 * tt_tensor_create). Shapes are checked at submit time (TT_ERR_SHAPE), the
 * argument list and dtypes too (TT_ERR_ARG); errors of the launch itself
 * latch in the context and are reported by the next submit or tt_wait.
 * Ops that need scratch memory use the context's per-stream workspace,
 * enlarged at submit time when needed (this drains the context first, so
 * the first submit of a larger op may block).
 */
typedef struct {
    tt_tensor* tensor;
    int64_t tile[TT_MAX_DIMS];
} tt_tile;

/* TT_OP_FILL: tiles d_0..d_{n-1} (1 <= n <= TT_FILL_MAX_TILES, f32), each
 * written (W) with `value`. Scalars tt_op_fill. */
#define TT_OP_FILL 1
typedef struct { float value; } tt_op_fill;

/* TT_OP_GEMM -- one tile of a linear layer (tile_gemm; layer list: review,
 * "What carries the argument"): C = alpha op(A) op(B) + beta C, then the
 * epilogue. tiles: A, B, C, then bias (if epilogue & TT_EPI_BIAS; n
 * elements), res (if & TT_EPI_RES; m x n), aux (if & (TT_EPI_GELU |
 * TT_EPI_GELU_BWD); m x n), in that order. Accesses: A, B, bias, res read;
 * C written (beta == 0 or GELU) else updated; aux updated by GELU when
 * beta != 0, written when beta == 0, read by GELU_BWD. split_k != 0 lets a
 * launch with few output blocks and a long K split K over the workspace
 * (deterministic). Scalars tt_op_gemm.
 * TT_OP_GEMM_BATCH -- independent products sharing K and the scalars
 * (tile_gemm_batch; the tied head's per-vocab-tile products): tiles A_0,
 * B_0, C_0, A_1, B_1, C_1, ... (one or more products; more than 72 make
 * several launches); epilogue 0. C_t written (beta == 0) or updated.
 * With epilogue TT_EPI_XSTATS (tile_gemm_batch_xstats; transA = 0): the
 * triples, then labels (i32, >= m elements), then one partials tile per
 * product (>= ceil(v_tile / 64) * m * 3 floats, equally spaced in memory);
 * the C tiles are consecutive tiles along the last axis of one tensor (the
 * logits), whose tile index times tile size gives each product's vocab
 * offset; labels read, partials written.
 * TT_OP_GEMM_KSUM -- a sum of products into one tile (tile_gemm_ksum_ex: a
 * linear layer whose contraction axis is split over several tiles, forward
 * or backward): tiles C, then bias / res / aux as the epilogue requires (as
 * for TT_OP_GEMM), then A_0, B_0, A_1, B_1, ... (one or more pairs; more
 * than 96 make several launches); C = epilogue(alpha sum_t A_t op(B_t) +
 * beta C) with transA = 0. Accesses as TT_OP_GEMM. split_k != 0 lets an
 * output of few blocks split K over the stream's workspace
 * (tile_gemm_ksum_ws; the op enlarges it as needed). Where one long-K launch
 * cannot take every pair (shapes not multiples of its blocks, misaligned
 * tiles, more than 96 pairs), the task runs a chain of products instead:
 * the same result up to the order of the additions. */
#define TT_OP_GEMM       2
#define TT_OP_GEMM_BATCH 3
#define TT_OP_GEMM_KSUM  4
typedef struct {
    int transA, transB, epilogue;
    float alpha, beta;
    int split_k;
} tt_op_gemm;

/* TT_OP_LAYERNORM_FWD -- layer norm of one block of rows whose features are
 * split over n tiles (review, "What carries the argument"; definition after
 * the "Layer Normalization" paper on the arXiv index page): tiles x_0..x_{n-1}
 * (rows x c_i), gamma_0..gamma_{n-1} (c_i), beta_0..beta_{n-1} (c_i), stats
 * (>= 2*rows floats: mean, rstd per row), y_0..y_{n-1} (rows x c_i) -- 4n+1
 * tiles. Reads x, gamma, beta; writes stats and y. Statistics over all
 * sum(c_i) features, biased variance, eps inside the square root.
 * Scalars tt_op_layernorm (eps).
 * TT_OP_LAYERNORM_BWD -- its gradient: tiles dy_0.., x_0.., gamma_0..,
 * stats, dx_0.., dgamma_0.., dbeta_0.. -- 6n+1 tiles. Reads dy, x, gamma,
 * stats; writes dx (updates it, adding, when dx_acc != 0); updates
 * dgamma += sum_rows dy*xhat and dbeta += sum_rows dy (fixed order). */
#define TT_OP_LAYERNORM_FWD 5
#define TT_OP_LAYERNORM_BWD 6
typedef struct {
    float eps;
    int dx_acc;
} tt_op_layernorm;

/* TT_OP_ATTENTION_FWD -- causal attention of one (query tile, key tile)
 * pair (tile_attention_fwd; "Attention Is All You Need", arXiv index page
 * "Builds on"): tiles Q, K, V, O, ml, lse. Q and O are 4-D tiles [batch,
 * q_len, heads, hd], K and V [batch, k_len, heads, hd] (same batch, heads,
 * hd); ml holds >= 2*batch*heads*q_len floats, lse >= batch*heads*q_len.
 * Reads Q, K, V; O written when first, else updated; ml written (first) or
 * updated, not touched when first && last; lse written when last, else not
 * touched. Scalars tt_op_attention (q_off, k_off: global positions of the
 * tiles' first query and key; scale usually 1/sqrt(hd)).
 * TT_OP_ATTENTION_PREP -- tiles O, dO, Dvec: Dvec = rowsum(dO * O) per
 * (b, h, query) (reads O, dO; writes Dvec).
 * TT_OP_ATTENTION_BWD -- tiles Q, K, V, dO, lse, Dvec, dQ, dK, dV:
 * dQ += , dK += , dV += the pair's gradient (tile_attention_bwd
 * TT_ATT_GRAD); reads the first six; dQ written unless acc_dq (then
 * updated), dK and dV written unless acc_dkv. dS passes through the
 * stream's workspace (tile_attention_bwd_ws), which the op enlarges to
 * tile_attention_bwd_workspace of the pair when needed. */
#define TT_OP_ATTENTION_FWD  7
#define TT_OP_ATTENTION_PREP 8
#define TT_OP_ATTENTION_BWD  9
typedef struct {
    int64_t q_off, k_off;
    int first, last;
    int acc_dq, acc_dkv;
    float scale;
} tt_op_attention;

/* Cross-entropy over vocab tiles (NNTile README, "Minimal working GPT
 * example": the loss is the mean over the batch's tokens), rows = tokens of
 * one token tile. The vocab offset of a logits tile is its tile index along
 * the tensor's last axis times that axis's tile size.
 * TT_OP_XENTROPY_STATS -- tiles labels (i32, rows), z_0..z_{n-1} (rows x
 * v_j, v_j <= 2048), parts_0..parts_{n-1} (>= 3*rows floats each, equally
 * spaced in memory, e.g. consecutive tiles of one tensor): per tile the
 * (row max, sum exp, picked target logit). Reads labels, z; writes parts.
 * TT_OP_XENTROPY_MERGE -- tiles lse (rows), row_loss (rows),
 * parts_0..parts_{n-1}: lse = merged logsumexp, row_loss = lse - target
 * logit. Reads parts; writes lse and row_loss. No scalars: one partial per
 * tile (from TT_OP_XENTROPY_STATS). Scalars tt_op_xe_groups: tile j holds
 * the column-group partials of vocab tile j (of vocab / v_tile tiles,
 * rounded up; from the head's TT_EPI_XSTATS epilogue), merged by
 * tile_xentropy_merge_groups.
 * TT_OP_XENTROPY_LOSS -- tiles row_loss, loss (1 float): loss =
 * (accumulate ? loss : 0) + inv_n * sum row_loss. Reads row_loss; loss
 * written, or updated when accumulate.
 * TT_OP_XENTROPY_GRAD -- tiles labels, lse, z_0..z_{n-1}: every z_j replaced
 * in place by (softmax - onehot(label)) * inv_n. Reads labels, lse; updates
 * z. Scalars tt_op_xentropy. */
#define TT_OP_XENTROPY_STATS 10
#define TT_OP_XENTROPY_MERGE 11
#define TT_OP_XENTROPY_LOSS  12
#define TT_OP_XENTROPY_GRAD  13
typedef struct {
    int accumulate;
    float inv_n;
} tt_op_xentropy;
typedef struct {
    int64_t vocab, v_tile;
    int group;            /* 64 for the TT_EPI_XSTATS partials */
} tt_op_xe_groups;

/* Optimiser steps (NNTile README, "Minimal working GPT example": fused
 * AdamW; the review's "What carries the argument" lists the Adam/SGD
 * update as tile tasks). Scalars tt_op_optim.
 * TT_OP_ADAMW -- tiles bias_corr (2 floats, from TT_OP_ADAMW_ADVANCE), then
 * p_i, g_i, m_i, v_i for i < n (1 <= n <= TT_ADAMW_MAX_TILES): the update of
 * tile_fused_adamw on each. Reads bias_corr and g; updates p, m, v.
 * TT_OP_ADAMW_ADVANCE -- tiles step (i32, 1 element), bias_corr (2 floats):
 * t = ++step, bias_corr = {1 - beta1^t, 1 - beta2^t}. Updates step, writes
 * bias_corr.
 * TT_OP_SGD -- tiles p_i, g_i (1 <= n <= TT_SGD_MAX_TILES pairs): p -= lr g.
 * Reads g; updates p. */
#define TT_OP_ADAMW         14
#define TT_OP_ADAMW_ADVANCE 15
#define TT_OP_SGD           16
typedef struct {
    float lr, beta1, beta2, eps, weight_decay;
} tt_op_optim;

/* Embedding layer (review, "What carries the argument"). Scalars
 * tt_op_embedding: seq_len = rows per sequence in the token tile (row r has
 * position r % seq_len within the wpe tile).
 * TT_OP_EMBEDDING_FWD -- tiles ids (i32, rows), wpe (positions x cols), out
 * (rows x cols), wte_0..wte_{n-1}: all vocab tiles of one embd tile column of
 * the token table, in vocab order. out = wte[id] + wpe[pos]; an id outside
 * [0, vocab) gives a NaN row. Reads ids, wpe, wte; writes out.
 * TT_OP_EMBEDDING_INDEX -- tiles ids, sorted, perm (i32, rows <= 65536):
 * stable sort of the ids. Reads ids; writes sorted, perm.
 * TT_OP_EMBEDDING_BWD -- tiles dh (rows x cols), sorted, perm,
 * dwte_0..dwte_{n-1}: consecutive vocab tiles of one embd tile column of the
 * table's gradient, in vocab order (all of them, or a run: ids outside the
 * run are skipped): dwte[id] += sum of the dh rows with that id, in row
 * order. Reads dh, sorted, perm; updates dwte.
 * TT_OP_EMBEDDING_POS_BWD -- tiles dh, dwpe: dwpe[pos] += sum over the
 * tile's sequences of dh. Reads dh; updates dwpe. */
#define TT_OP_EMBEDDING_FWD     17
#define TT_OP_EMBEDDING_INDEX   18
#define TT_OP_EMBEDDING_BWD     19
#define TT_OP_EMBEDDING_POS_BWD 20
typedef struct { int64_t seq_len; } tt_op_embedding;

/* TT_OP_REDUCE_ROWS -- bias gradients of a linear layer (column sums):
 * tiles X_0, out_0, X_1, out_1, ... (1..16 pairs, equal row counts):
 * out_t = (beta ? out_t : 0) + sum_rows X_t in a fixed order. Reads X;
 * out written, or updated when beta. Scalars tt_op_reduce. */
#define TT_OP_REDUCE_ROWS 21
typedef struct { int beta; } tt_op_reduce;

/* TT_OP_SPLIT_TOKENS -- the token batch (NNTile README, "Minimal working
 * GPT example": windows of a token stream): tiles tokens (i32 [B, T+1] in a
 * single tile), ids, labels (tile (bi, si) of i32 [B, T] tensors tiled [bt,
 * st]): ids = windows bi*bt.. at positions si*st.., labels the same shifted
 * by one. Reads tokens; writes ids and labels. No scalars.
 * TT_OP_COPY_IN -- tiles dst: dst = tile_bytes(dst) bytes copied from the
 * DEVICE address src (device to device). The source is read when the task
 * runs, which can be after tt_submit returns: it must stay allocated and
 * unchanged until then (tt_wait, or work ordered after the context with
 * tt_ctx_join_stream). Writes dst. Scalars tt_op_copy. */
#define TT_OP_SPLIT_TOKENS 22
#define TT_OP_COPY_IN      23
typedef struct { const void* src; } tt_op_copy;

/* Ops of the LLaMA block (the README's notebook list names LLaMa as its
 * second model; definitions after the published LLaMA architecture).
 * TT_OP_RMSNORM_FWD -- tiles x_0..x_{n-1} (rows x c_i), gamma_0..gamma_{n-1},
 * rstd (>= rows floats), y_0..y_{n-1}: tile_rmsnorm_fwd over the row block
 * (3n+1 tiles, n <= 16). Reads x, gamma; writes rstd and y. Scalars
 * tt_op_layernorm (eps).
 * TT_OP_RMSNORM_BWD -- tiles dy_0.., x_0.., gamma_0.., rstd, dx_0..,
 * dgamma_0.. (5n+1 tiles): tile_rmsnorm_bwd. Reads dy, x, gamma, rstd;
 * writes dx (updates it when dx_acc); updates dgamma. Scalars
 * tt_op_layernorm (dx_acc).
 * TT_OP_ROPE -- tiles x_0..x_{n-1} (1..4 tiles [batch, len, heads, hd] of
 * equal shape, e.g. a q and a k tile), then table ([>= positions, hd],
 * from TT_OP_ROPE_TABLE): tile_rope in place on each x (updated; table
 * read). Row r of a tile has position pos_off + r % len. Scalars tt_op_rope.
 * TT_OP_ROPE_TABLE -- tiles table [seq, hd]: tile_rope_table (written).
 * Scalars tt_op_rope (base; pos_off and inverse unused).
 * TT_OP_SWIGLU_FWD -- tiles a_0, b_0, h_0, a_1, b_1, h_1, ... (equal element
 * counts per triple, 1..16 triples): h = silu(a) * b. Reads a, b; writes h.
 * TT_OP_SWIGLU_BWD -- tiles dh_0, a_0, b_0, ...: a_t <- dh * b * silu'(a),
 * b_t <- dh * silu(a), in place (a and b updated, dh read).
 * TT_OP_EMBEDDING_TOKEN_FWD -- tiles ids, out, wte_0..wte_{n-1}: as
 * TT_OP_EMBEDDING_FWD without the position term (out = wte[id]). Scalars
 * tt_op_embedding (seq_len = rows, or any divisor of them). */
#define TT_OP_RMSNORM_FWD         24
#define TT_OP_RMSNORM_BWD         25
#define TT_OP_ROPE                26
#define TT_OP_ROPE_TABLE          27
#define TT_OP_SWIGLU_FWD          28
#define TT_OP_SWIGLU_BWD          29
#define TT_OP_EMBEDDING_TOKEN_FWD 30
typedef struct {
    int64_t pos_off;
    int inverse;
    double base;
} tt_op_rope;

int tt_submit(tt_ctx* ctx, int op, const tt_tile* tiles, int ntiles, const void* scalars, size_t scalars_size);

/* Ordering against streams the context does not own (e.g. a framework's
 * current stream), on the device, without blocking the host:
 * tt_ctx_wait_stream -- tasks launched from now on run after the work
 *   queued on `stream` so far (an event recorded there, waited on by every
 *   executor stream);
 * tt_ctx_join_stream -- work queued on `stream` from now on runs after
 *   every task the context has launched so far (each executor stream's
 *   tail, waited on by `stream`). Tasks still held in the submit window are
 *   launched first. */
int tt_ctx_wait_stream(tt_ctx* ctx, void* stream);
int tt_ctx_join_stream(tt_ctx* ctx, void* stream);

/* Launch everything queued and wait for the GPU; returns the first latched
 * error, if any. */
int tt_wait(tt_ctx* ctx);
/* Write the recorded task graph as JSON lines: one object per task with
 * id, label, stream, cost (the task's flop estimate, 0 for memory-bound
 * tasks), deps and accesses (dry-run and real contexts). */
int tt_dump_dag(tt_ctx* ctx, const char* path);

/* Per-task GPU timing. Tasks whose label equals label_filter ("*" = every
 * task, NULL = off) are bracketed by a pair of timing events on their
 * stream; the durations are aggregated per label when the context drains.
 * tt_ctx_profile first waits for the work already queued.
 * tt_profile_read waits, fills up to max_entries entries (one per label,
 * *n_entries = number of labels seen) and clears the aggregate. Timing
 * events add a little GPU time per bracketed task, so narrow filters are
 * the ones to use inside a timed region. */
typedef struct {
    char label[32];
    int64_t count;            /* launches timed                             */
    double total_ms, min_ms, max_ms;
} tt_profile_entry;
int tt_ctx_profile(tt_ctx* ctx, const char* label_filter);
int tt_profile_read(tt_ctx* ctx, tt_profile_entry* out, int max_entries, int* n_entries);
/* Time only every `every`-th matching task (1 = all, the default): each
 * event pair costs a few microseconds of queue time, so a timed region
 * samples. Counting restarts at every tt_ctx_profile call. TT_ERR_ARG for
 * every < 1. */
int tt_ctx_profile_every(tt_ctx* ctx, int every);
/* GPU occupancy of the timed tasks: tt_ctx_profile drains the context and
 * records a reference event; every task timed since has a [start, end]
 * interval against it. tt_profile_busy waits and returns the length of the
 * union of those intervals (*busy_ms: time at least one timed task was on
 * the GPU), the time from the first start to the last end (*span_ms) and
 * the number of intervals, then clears them. With the filter "*" and every
 * = 1, 1 - busy/span is the fraction of the span the GPU had no task of the
 * context running (the gaps between dependent tasks and launch latency not
 * hidden by other streams); the timing events add a few microseconds per
 * task to that span. */
int tt_profile_busy(tt_ctx* ctx, double* busy_ms, double* span_ms, int64_t* n_tasks);

typedef struct {
    int64_t tasks;            /* tasks submitted since creation / reset     */
    int64_t edges;            /* dependency edges inferred                  */
    int64_t cross_stream_waits;
    int64_t events_recorded;
    double  submit_seconds;   /* host time spent in submit + launch         */
    int64_t h2d_bytes, d2h_bytes;  /* residency traffic                      */
    int64_t evictions, prefetches;
} tt_stats;
int tt_get_stats(tt_ctx* ctx, tt_stats* out);
int tt_reset_stats(tt_ctx* ctx);

/* ====================================================== 3. the GPT2 step */

typedef struct tt_gpt2 tt_gpt2;
typedef struct {
    int n_layer, vocab, n_embd, n_head, n_inner, seq, batch;
    float ln_eps;             /* 1e-5 */
} tt_gpt2_config;
typedef struct {              /* README tile flags; vocab has no flag there */
    int batch, seq, embd, inner, head, vocab;
} tt_gpt2_tiles;
/* Optimiser settings of the NNTile README's GPT example (fused AdamW, eps,
 * weight decay, lr) plus its warm-up flags: update 1 uses start_lr, update
 * full_lr_iter and later ones lr, linearly in between; full_lr_iter <= 1
 * uses lr throughout. Updates are counted per tt_gpt2 from its creation.
 * optimizer (the README's --optimizer flag): TT_OPT_ADAMW, or TT_OPT_SGD
 * for the plain step p -= lr*g on every parameter (beta1, beta2, eps and
 * weight_decay are then unused and the moments are left untouched). */
#define TT_OPT_ADAMW 0
#define TT_OPT_SGD 1
typedef struct {
    float lr, beta1, beta2, eps, weight_decay;
    float start_lr;
    int full_lr_iter;
    int optimizer;
} tt_adamw_hparams;

/* Allocates parameters, gradients, AdamW moments (zeroed) and activations
 * as tiled tensors. Parameters are in the order: wte [V,d], wpe [T,d], then
 * per block ln1_g, ln1_b, w_qkv [d,3d], b_qkv, w_o [d,d], b_o, ln2_g, ln2_b,
 * w_fc [d,I], b_fc, w_p [I,d], b_p, then lnf_g, lnf_b (GPT2 with a tied
 * head). TT_ERR_SHAPE if seq, head or batch tiles do not divide their axis
 * or n_embd % n_head != 0. param_home = TT_HOME_PINNED_HOST keeps
 * parameters, gradients and moments in pinned host RAM (out-of-core);
 * TT_HOME_PINNED_STATE keeps parameters and moments there and the
 * gradients, which are made and consumed within a step, in HBM (no link
 * traffic for them). */
int tt_gpt2_create(tt_ctx* ctx, const tt_gpt2_config* cfg, const tt_gpt2_tiles* tiles,
                   int param_home, tt_gpt2** out);
/* The LLaMA-style model (the NNTile README's notebook list names LLaMa
 * next to GPT2; the pith.science review's "Editorial extensions" notes the
 * same tile tasks assemble other architectures): pre-RMSNorm blocks,
 * rotary embedding of q and k (base 10000, pairs (i, i + hd/2)), SwiGLU MLP
 * of width n_inner, no biases, no position table, an untied head. Built
 * from the same tile tasks as the GPT2 step; the handle is used with every
 * tt_gpt2_* call below (step, accumulation, loss, row losses, parameters).
 * cfg->ln_eps is the RMSNorm eps. Parameters, in order: wte [V,d], then per
 * block attn_norm_g [d], w_qkv [d,3d], w_o [d,d], mlp_norm_g [d], w_gate
 * [d,I], w_up [d,I], w_down [I,d], then norm_f_g [d], w_head [V,d].
 * Besides tt_gpt2_create's checks: TT_ERR_SHAPE unless n_embd and the embd
 * tile are multiples of 4. */
int tt_llama_create(tt_ctx* ctx, const tt_gpt2_config* cfg, const tt_gpt2_tiles* tiles,
                    int param_home, tt_gpt2** out);
int tt_gpt2_destroy(tt_gpt2* g);
int tt_gpt2_num_params(tt_gpt2* g, int* n);
/* Tensors of parameter `index`: value, gradient, first and second moment
 * (any output may be NULL). Dense layouts match the shapes listed above. */
int tt_gpt2_param(tt_gpt2* g, int index, tt_tensor** param, tt_tensor** grad,
                  tt_tensor** m, tt_tensor** v);
/* One training step, submitted as tile tasks: embedding, blocks, final
 * LayerNorm, tied head, cross-entropy, the backward of each, and (if
 * do_update) one AdamW step on every parameter tile. tokens: DEVICE int32
 * [batch, seq+1] windows (inputs = tokens[:, :seq], labels = tokens[:, 1:]),
 * ids in [0, vocab). The step is queued; tt_gpt2_loss waits and returns
 * the mean loss. */
int tt_gpt2_step(tt_gpt2* g, const int32_t* tokens, const tt_adamw_hparams* hp, int do_update);
/* One optimiser step over a batch of n_micro minibatches (the README's
 * batch / minibatch flags: gradients of the whole batch are collected
 * before the update). tokens: DEVICE int32 [n_micro * batch, seq + 1];
 * minibatch i is rows i*batch .. (i+1)*batch - 1. Forward and backward run
 * per minibatch, every gradient accumulating after the first; the loss and
 * its gradient are scaled by 1 / (n_micro * batch * seq), so the result is
 * the step on the whole batch with the mean loss. AdamW (if do_update) runs
 * once, after the last minibatch's backward. tt_gpt2_loss returns the batch
 * mean, tt_gpt2_row_losses the last minibatch's. n_micro = 1 is
 * tt_gpt2_step. TT_ERR_ARG for n_micro < 1. */
int tt_gpt2_step_accum(tt_gpt2* g, const int32_t* tokens, int n_micro, const tt_adamw_hparams* hp,
                       int do_update);
/* Graph replay (on != 0): the next tt_gpt2_step records its tasks into one
 * HIP graph (kernels, copies and cross-stream waits; nothing runs while
 * recording) and launches it; later steps with the same tokens pointer,
 * hyperparameters and do_update launch that graph again instead of
 * submitting the tasks one by one. The tokens buffer is read when the graph
 * runs, so its contents may change between steps; another pointer or other
 * hyperparameters record a new graph. The AdamW step count lives in device
 * memory, so replays advance it. Results are bitwise those of the task-by-
 * task step. TT_ERR_UNSUPPORTED for pinned-host parameters or a dry-run
 * context; per-task timing (tt_ctx_profile) is refused while recording.
 * CURRENTLY DISABLED: on != 0 always returns TT_ERR_UNSUPPORTED (the first
 * GPU run of a recorded step ended in a host-side fault not yet explained);
 * on = 0 is accepted. */
int tt_gpt2_set_replay(tt_gpt2* g, int on);
int tt_gpt2_loss(tt_gpt2* g, float* loss_host);
/* Per-token losses of the last step's forward, lse - z[label] for every
 * (b, t), written to host memory as float [batch, seq] row-major (the
 * caller owns out_host, batch*seq floats). Waits for the step. Their mean
 * is the loss. Position t depends only on tokens 0..t of its window
 * (causal attention), so a prefix of the window reproduces it. */
int tt_gpt2_row_losses(tt_gpt2* g, float* out_host);
/* Number of tasks the last step submitted. */
int tt_gpt2_task_count(tt_gpt2* g, int64_t* n);

#ifdef __cplusplus
}
#endif
#endif /* TILETASK_H */
