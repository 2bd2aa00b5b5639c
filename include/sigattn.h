/*
 * sigattn.h: C ABI of the padding-aware, non-causal sigmoid attention library
 * for AMD Instinct MI355X (gfx950).
 *
 * The operation comes from the summaries of "Better Models, Faster Training:
 * Sigmoid Attention for single-cell Foundation Models" (arXiv:2604.27124):
 *   rainbus.top summary, section "方法步骤详情" (method steps), steps 1-5;
 *   gist.science summary, section 2.A (the forward formula);
 *   paperlayer.ai summary, section 3 (the bias b = -log n).
 *
 *   S = alpha * Q K^T + b,  P = sigma(S) (elementwise, no row normalisation),
 *   O = P V.
 *   Keys j >= n_k[z] get weight exactly 0. Rows i >= n_q[z] of O are written 0.
 *   Backward, with P recomputed from Q and K:
 *     dS = P (1 - P) (dO V^T),
 *     dQ = alpha dS K,  dK = alpha dS^T Q,  dV = P^T dO.
 *   dQ rows i >= n_q and dK, dV rows j >= n_k are written 0. dO rows i >= n_q
 *   are never read.
 *
 * Conventions shared by every entry point:
 *  - Tensors are contiguous [Z, L, H, D] (batch, length, heads, head dim) with
 *    D fastest. Q, K, V, dO, O, dQ, dK and dV all share this shape, and
 *    queries and keys share L.
 *  - dtype SIGATTN_BF16: bf16 storage. The two contractions run on bf16 MFMA
 *    with fp32 accumulation. P and dS are rounded to bf16 (RNE) before they
 *    enter an MFMA, and outputs are rounded to bf16 (RNE).
 *    dtype SIGATTN_FP32: fp32 storage and fp32 arithmetic throughout (the
 *    validation build).
 *  - D must be 64 or 128.
 *  - Lengths are int32[Z] arrays in DEVICE memory, read by the kernels, so the
 *    host never synchronises. A value below 0 is treated as 0, and a value
 *    above L as L. Padding is a suffix: positions [0, n) are valid.
 *  - Padded input rows are never read, so their contents, NaN included, cannot
 *    change any output.
 *  - Every element of every output is written, padding included (in the
 *    packed layout: every row, under the offsets contract at sigattn_fwd_ex).
 *    The caller need not clear outputs.
 *  - All tensor pointers are DEVICE pointers owned by the caller. The library
 *    keeps no reference after the call returns and allocates no memory.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL means the
 *    null stream). Calls are reentrant and thread-safe. Overlapping calls that
 *    write the same output race, as any two kernels would.
 *  - A call with Z, L or H equal to 0 does nothing and returns SIGATTN_OK.
 *  - Return value: SIGATTN_OK (0) or a negative sigattn_status. No entry point
 *    throws, aborts or prints. sigattn_last_error() returns a message for the
 *    calling thread's most recent failure.
 *  - Optional tile counters (nullable device int32 buffers) record the
 *    skip decisions: for each tile, how many tiles it was paired with.
 */
#ifndef SIGATTN_H
#define SIGATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Every enum below carries a last enumerator of 0x7fffffff that names nothing:
 * it keeps the type int-sized and every int value in its range, so an unknown
 * value passed by a caller is rejected with a status, never undefined. */
typedef enum { SIGATTN_BF16 = 0, SIGATTN_FP32 = 1, SIGATTN_DTYPE_INT_RANGE_ = 0x7fffffff } sigattn_dtype;

typedef enum {
  SIGATTN_OK = 0,
  SIGATTN_EINVAL = -1,        /* null pointer, negative size, D not 64/128, misaligned
                                 pointer, non-finite alpha/bias, grid too large */
  SIGATTN_EUNSUPPORTED = -2,  /* unknown dtype */
  SIGATTN_EHIP = -3,          /* a HIP launch failed; see sigattn_last_error() */
  SIGATTN_EWORKSPACE = -4     /* workspace smaller than sigattn_softmax_bwd_workspace_size() */
} sigattn_status;

/* Where each sample's rows live (sigattn_fwd_ex, sigattn_bwd_ex).
 *  PADDED: tensors are [Z, L, H, D]; seq_q and seq_k are the lengths n_q[Z] and
 *          n_k[Z] (the convention of every other entry point).
 *  PACKED: tensors are [T, H, D], the samples' valid rows back to back with no
 *          padding; seq_q and seq_k are int32[Z + 1] cumulative offsets (sample
 *          z owns rows seq[z] .. seq[z+1] - 1, so n = seq[z+1] - seq[z]). L is an
 *          upper bound on every length (see the contract at sigattn_fwd_ex).
 *          Q, O, dO and dQ use seq_q; K, V, dK and dV use seq_k. T is implied
 *          by the offsets and never passed.
 * The pages fix per-sample lengths n_q, n_k (rainbus.top summary, 方法步骤详情
 * step 1) and say that cells are attended one by one, never split or
 * concatenated with other cells (paperlayer.ai summary, section 1). The packed
 * layout keeps exactly that per-sample attention: no score ever pairs rows of
 * two samples. Only the storage changes, the valid rows back to back without
 * padding rows; that storage variant is this library's own design, not the
 * pages'. */
typedef enum { SIGATTN_LAYOUT_PADDED = 0, SIGATTN_LAYOUT_PACKED = 1, SIGATTN_LAYOUT_INT_RANGE_ = 0x7fffffff } sigattn_layout;

/* The score bias (paperlayer.ai summary, section 3: b = -log n).
 *  CONSTANT:   b = bias for every sample.
 *  NEG_LOG_NK: b_z = bias - ln(n_k[z]) for sample z (ln 1 for n_k = 0). With
 *              bias = 0 this is the per-sample reading b = -log(n). */
typedef enum {
  SIGATTN_BIAS_CONSTANT = 0,
  SIGATTN_BIAS_NEG_LOG_NK = 1,
  SIGATTN_BIAS_INT_RANGE_ = 0x7fffffff
} sigattn_bias_mode;

/* Which kernel a tile configuration or a counter refers to. */
typedef enum {
  SIGATTN_KERNEL_FWD = 0,
  SIGATTN_KERNEL_DQ = 1,
  SIGATTN_KERNEL_DKDV = 2,
  SIGATTN_KERNEL_INT_RANGE_ = 0x7fffffff
} sigattn_kernel;

/*
 * Forward: o = sigma(alpha * q k^T + bias) v with padding (rainbus.top summary,
 * 方法步骤详情 steps 1-3; gist.science summary 2.A).
 *   q, k, v        [Z, L, H, D] inputs, read only on valid rows.
 *   o              [Z, L, H, D] output. Rows >= n_q[z] are written 0.
 *   seqlens_q/_k   int32[Z], device.
 *   alpha, bias    score scale and bias. The pages use 1/sqrt(D) and -log(n).
 *   dtype          SIGATTN_BF16 or SIGATTN_FP32; any other value gives
 *                  SIGATTN_EUNSUPPORTED.
 *   tile_counts    NULL, or int32[Z * H * ceil(L / BQ)], where BQ is the forward's
 *                  query tile from sigattn_tile_config. Entry (z, h, m) receives
 *                  the number of key tiles that query tile m computed. It is 0
 *                  when the tile lies wholly in padding and was skipped.
 * In bf16, sigma of a block of scores that all lie at or below -3.47 is taken
 * as t - t^2 with t = e^S (relative error t^2 <= 2^-10 before P's rounding to
 * bf16); every other block gets the exact 1 / (1 + e^-S). The result does not
 * depend on the padding, and is deterministic run to run.
 */
int sigattn_fwd(const void* q, const void* k, const void* v, void* o,
                const int32_t* seqlens_q, const int32_t* seqlens_k,
                int Z, int L, int H, int D, float alpha, float bias, sigattn_dtype dtype,
                int32_t* tile_counts, void* stream);

/*
 * Backward: dq, dk, dv from q, k, v and dout. P is recomputed, and neither O
 * nor any saved statistic is needed (rainbus.top summary, 方法步骤详情 steps
 * 4-5). Two independent kernels run on `stream`, one for dQ and one for dK/dV,
 * so there are no atomics and the results are bitwise deterministic.
 *   dout             [Z, L, H, D] upstream gradient. Rows >= n_q are not read.
 *   dq, dk, dv       [Z, L, H, D] outputs. dq rows >= n_q and dk, dv rows >= n_k
 *                    are written 0.
 *   tile_counts_dq   NULL or int32[Z * H * ceil(L / BQ_dq)]: key tiles per query tile.
 *   tile_counts_dkdv NULL or int32[Z * H * ceil(L / BK_dkdv)]: query tiles per key tile.
 * All other arguments are as for sigattn_fwd.
 */
int sigattn_bwd(const void* q, const void* k, const void* v, const void* dout,
                void* dq, void* dk, void* dv,
                const int32_t* seqlens_q, const int32_t* seqlens_k,
                int Z, int L, int H, int D, float alpha, float bias, sigattn_dtype dtype,
                int32_t* tile_counts_dq, int32_t* tile_counts_dkdv, void* stream);

/*
 * The two halves of sigattn_bwd, for callers that want to place or time them
 * separately (for example, on two streams). Each launches one kernel;
 * sigattn_bwd_dkdv's computes dk and dv together from one recomputed P.
 * sigattn_bwd_dkdv writes dk and dv. sigattn_bwd_dq writes dq. Arguments are as
 * for sigattn_bwd. Together they compute exactly what sigattn_bwd computes,
 * bit for bit.
 */
int sigattn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, void* dk, void* dv,
                     const int32_t* seqlens_q, const int32_t* seqlens_k,
                     int Z, int L, int H, int D, float alpha, float bias, sigattn_dtype dtype,
                     int32_t* tile_counts_dkdv, void* stream);
int sigattn_bwd_dq(const void* q, const void* k, const void* v, const void* dout, void* dq,
                   const int32_t* seqlens_q, const int32_t* seqlens_k,
                   int Z, int L, int H, int D, float alpha, float bias, sigattn_dtype dtype,
                   int32_t* tile_counts_dq, void* stream);

/*
 * dk alone and dv alone, each one kernel launch over the same key tiles as
 * sigattn_bwd_dkdv (rainbus.top summary, 方法步骤详情 step 5: dV = P^T dO and
 * dK = alpha dS^T Q are separate contractions over the recomputed P). dv needs
 * no v. Both write tile_counts_dkdv as sigattn_bwd_dkdv does, and their outputs
 * equal its dk and dv bit for bit. Together they cost more than
 * sigattn_bwd_dkdv: each recomputes the scores (and dk also dO V^T).
 */
int sigattn_bwd_dk(const void* q, const void* k, const void* v, const void* dout, void* dk,
                   const int32_t* seqlens_q, const int32_t* seqlens_k,
                   int Z, int L, int H, int D, float alpha, float bias, sigattn_dtype dtype,
                   int32_t* tile_counts_dkdv, void* stream);
int sigattn_bwd_dv(const void* q, const void* k, const void* dout, void* dv,
                   const int32_t* seqlens_q, const int32_t* seqlens_k,
                   int Z, int L, int H, int D, float alpha, float bias, sigattn_dtype dtype,
                   int32_t* tile_counts_dkdv, void* stream);

/*
 * sigattn_fwd and sigattn_bwd with a choice of layout and bias mode (see
 * sigattn_layout and sigattn_bias_mode). With SIGATTN_LAYOUT_PADDED and
 * SIGATTN_BIAS_CONSTANT they are exactly sigattn_fwd and sigattn_bwd. Tile
 * counters are indexed as in the padded layout, with ceil(L / tile) tiles per
 * (z, h).
 * Packed-layout contract, which the caller owns: the offsets live in device
 * memory and the host never reads them (that would need a synchronisation),
 * so they are not checked here. They must start at 0, never decrease, end at
 * or below the tensors' row count T, and give no sample more than L rows.
 * Under that contract every row of every output is written exactly once. A
 * sample longer than L is cut at L: its rows past L are neither read nor
 * written, so those output rows keep whatever they held. Offsets past T make
 * the kernels read and write outside the tensors. (The Python binding checks
 * all of this on the host before it calls in, and raises ValueError.)
 * Errors: as sigattn_fwd / sigattn_bwd, plus SIGATTN_EINVAL for an unknown
 * layout or bias mode.
 */
int sigattn_fwd_ex(const void* q, const void* k, const void* v, void* o,
                   const int32_t* seq_q, const int32_t* seq_k, sigattn_layout layout, sigattn_bias_mode bias_mode,
                   int Z, int L, int H, int D, float alpha, float bias, sigattn_dtype dtype,
                   int32_t* tile_counts, void* stream);
int sigattn_bwd_ex(const void* q, const void* k, const void* v, const void* dout,
                   void* dq, void* dk, void* dv,
                   const int32_t* seq_q, const int32_t* seq_k, sigattn_layout layout, sigattn_bias_mode bias_mode,
                   int Z, int L, int H, int D, float alpha, float bias, sigattn_dtype dtype,
                   int32_t* tile_counts_dq, int32_t* tile_counts_dkdv, void* stream);

/*
 * Padding-aware, non-causal SOFTMAX attention, the same padding design applied
 * to softmax (rainbus.top summary, "未来方向"; the softmax itself is the one
 * of the "前置知识" entries on self-attention and softmax normalisation):
 *   S = alpha * Q K^T over the keys j < n_k[z],
 *   P_ij = e^{S_ij} / sum_{j < n_k} e^{S_ij},  O = P V,
 *   LSE_i = log sum_{j < n_k} e^{S_ij}  (natural log).
 * A constant score bias cancels in the row normalisation, so there is no bias.
 * A row with no valid key (n_k[z] = 0) and every padded row (i >= n_q[z]) get
 * O = 0 and LSE = 0.
 * Backward, with P recomputed as e^{S - LSE}:
 *   dP = dO V^T,  Dvec_i = sum_d dO_id O_id,  dS = P (dP - Dvec),
 *   dQ = alpha dS K,  dK = alpha dS^T Q,  dV = P^T dO.
 *
 * Layout: `layout` as in sigattn_fwd_ex (PADDED with lengths, PACKED with
 * offsets). lse is fp32 [Z, L, H] (padded) or [T, H] (packed), one value per
 * query row and head, device memory owned by the caller. O, dO, dQ, dK and dV
 * follow Q, K and V in dtype and layout. alpha must be > 0: the kernels take
 * each row's running maximum of alpha q.k to keep e^x finite.
 * bf16: both contractions run on bf16 MFMA with fp32 accumulation; P and dS
 * are rounded to bf16 before an MFMA; the running maximum, the row sums and
 * LSE are fp32. fp32: fp32 throughout.
 *
 * sigattn_softmax_bwd takes the forward's O and lse unchanged, and a device
 * workspace of at least sigattn_softmax_bwd_workspace_size(rows_q, H) bytes,
 * rows_q being the number of query rows (Z * L padded, T packed). It holds
 * {LSE log2 e, Dvec} per query row and head between the backward's kernels,
 * and is written before it is read, so it need not be cleared. The padded
 * layout's size is checked; the packed layout's T lives in device memory and
 * is the caller's to respect.
 * Errors: as sigattn_fwd_ex, plus SIGATTN_EINVAL for alpha <= 0 or a NULL
 * lse or workspace, and SIGATTN_EWORKSPACE for a workspace that is too small.
 */
int sigattn_softmax_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                        const int32_t* seq_q, const int32_t* seq_k, sigattn_layout layout,
                        int Z, int L, int H, int D, float alpha, sigattn_dtype dtype, void* stream);
size_t sigattn_softmax_bwd_workspace_size(long long rows_q, int H);
int sigattn_softmax_bwd(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                        const int32_t* seq_q, const int32_t* seq_k, sigattn_layout layout,
                        int Z, int L, int H, int D, float alpha, sigattn_dtype dtype,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * sigattn_softmax_bwd without a workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc. The call allocates nothing. The row statistics
 * {LSE log2 e, Dvec} live instead in a fixed buffer inside the library of
 * SIGATTN_NOALLOC_ROWS float pairs (16 MiB), one per GPU, which each GPU the
 * library runs on holds until the process ends. The first call on a device
 * looks up that device's buffer address (hipGetSymbolAddress), once.
 * Limit: Z * L * H <= SIGATTN_NOALLOC_ROWS (both layouts: a packed batch within
 * its contract has at most Z * L query rows), else SIGATTN_EINVAL.
 * Every call on one GPU uses that GPU's buffer, and the buffer keeps the last
 * call's contents (each call writes every entry it reads before reading it):
 * calls that overlap on one GPU, on two streams or from two threads, race
 * and give wrong results. Arguments, errors and results are those of
 * sigattn_softmax_bwd, bit for bit.
 */
#define SIGATTN_NOALLOC_ROWS (1 << 21)
int sigattn_softmax_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                                const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                const int32_t* seq_q, const int32_t* seq_k, sigattn_layout layout,
                                int Z, int L, int H, int D, float alpha, sigattn_dtype dtype, void* stream);

/*
 * FP8 forward (OCP E4M3 operands on the gfx950 FP8 MFMA), the FP8 direction
 * the pages leave as future work (rainbus.top summary of arXiv:2604.27124,
 * "未来方向"; paperlayer.ai summary, section 5), on the sigmoid forward above.
 *
 * sigattn_quantize_fp8 turns a bf16 tensor (layout as `layout` says: padded
 * [Z, L, H, D] with lengths seq, or packed [T, H, D] with offsets seq) into
 * E4M3 codes x8 (one byte per element, same layout) and one scale byte per
 * (sample, head, tile of 64 rows counted from the sample's first row):
 * scales is uint8 [Z, H, ceil(L / 64)]. A tile's scale is 2^E with
 * E = floor(log2 amax) - 7 over its valid rows (E = 0 for an all-zero tile,
 * E >= -127), stored as the E8M0 byte E + 127; code = x * 2^-E rounded to
 * nearest-even E4M3 (it never overflows: |x| 2^-E < 256). Rows past the
 * length that lie inside the tensor get code 0; padded rows are not read.
 * Quantise Q and the query lengths, K and V with the key lengths.
 *
 * sigattn_fwd_fp8 computes O (bf16, layout of Q) = sigma(alpha Q K^T + b) V on
 * the dequantised operands, with P quantised per query row and 64-key tile:
 * 2^e * E4M3(P 2^-e), e = floor(log2 m) - 7, m the tile's largest P over its
 * valid keys. Both products run on the FP8 MFMA, which sums each group of 8
 * products on its own, every product cut toward zero to a multiple of
 * 2^(E - 13) (E the group's largest sum of the two operands' exponents), and
 * adds the groups in fp32: a score or an output element can differ from the
 * exact dot product of the dequantised operands by up to 2^-10 of each
 * group's largest product, before P's E4M3 rounding. Padding, bias modes and
 * lengths as for sigattn_fwd_ex. alpha must be > 0 and L <= 262144.
 * Errors: as sigattn_fwd_ex, plus SIGATTN_EINVAL for alpha <= 0, L > 262144
 * or a NULL scale array. Scale arrays need no alignment.
 */
int sigattn_quantize_fp8(const void* x, void* x8, uint8_t* scales, const int32_t* seq, sigattn_layout layout,
                         int Z, int L, int H, int D, void* stream);
int sigattn_fwd_fp8(const void* q8, const void* k8, const void* v8,
                    const uint8_t* sq, const uint8_t* sk, const uint8_t* sv, void* o,
                    const int32_t* seq_q, const int32_t* seq_k, sigattn_layout layout, sigattn_bias_mode bias_mode,
                    int Z, int L, int H, int D, float alpha, float bias, void* stream);

/* The tile sizes a kernel uses, for reading the tile counters. block_q is the
 * query tile and block_k the key tile. Returns SIGATTN_EINVAL for an unknown
 * kernel, D or dtype. */
int sigattn_tile_config(sigattn_kernel kernel, int D, sigattn_dtype dtype, int* block_q, int* block_k);

/* A static description of a status code. */
const char* sigattn_strerror(int status);

/* The calling thread's most recent error message ("" if none). */
const char* sigattn_last_error(void);

/* Library version string. */
const char* sigattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SIGATTN_H */
