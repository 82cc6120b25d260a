/*
 * spense.h - C interface of the Spense hybrid sparse-dense linear layer on
 * AMD Instinct MI355X (gfx950).
 *
 * The layer (SpenseGPT gist.science explainer, Technical Summary 2.A "The
 * Spense Format"): the input dimension K of a weight matrix W[N,K] is split
 * into a contiguous 2:4 semi-structured region and a contiguous dense region,
 * and the input-split form accumulates both products into one output,
 *
 *     Y[M,N] = X'[:, :K_s] . W_sparse^T + X'[:, K_s:] . W_dense^T,
 *
 * where X' = X[:, pi] and pi lists the sparse columns ascending, then the
 * dense columns ascending.  Which columns stay dense (Technical Summary 2.B
 * "Dense Index Selection Strategies"): the last p% of K (SpenseGPT), or any
 * chosen set moved into the dense block by that permutation (SpenseGPT+).
 * 2:4 means at most two nonzeros in every four consecutive weights (Technical
 * Summary 1 "Problem Statement"); here exactly two slots per group are kept,
 * the two with the largest magnitude, the lower position winning ties.
 *
 * General rules for every entry point:
 *   - All arguments are validated on the host before any HIP call or launch;
 *     a rejected call returns SPENSE_EINVAL / SPENSE_EUNSUPPORTED and has no
 *     side effect.
 *   - "device pointer" means memory the HIP runtime can access from the GPU
 *     current at the call (hipMalloc / torch CUDA tensors).  "host pointer" is
 *     ordinary CPU memory.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *   - Matrices are row-major; leading dimensions are in elements.
 *   - A HIP runtime failure returns SPENSE_EHIP; spense_last_hip_error()
 *     then returns the hipError_t value.  Faults inside a kernel surface at the
 *     caller's next synchronisation, as for any HIP launch.
 *   - The library is not thread-safe per handle: at most one spense_linear may
 *     be in flight on a handle at a time (its split-K and gather workspaces
 *     are shared).
 *   - spense_linear, spense_linear_w8a8 and spense_glu may be captured in a HIP
 *     graph once an eager call on the same handle at a batch size of at least
 *     the captured one has run (automatic split counts): a call that has to
 *     grow the handle's workspaces synchronises the stream and allocates, and
 *     sizes them for every batch size up to its own, whatever split count the
 *     planner picks there.  spense_linear_splits with a forced split count
 *     sizes them for that call only.  The calls record kernel launches only;
 *     the split-K hand-off counters are reset by the kernels.
 */
#ifndef SPENSE_H
#define SPENSE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPENSE_ABI_VERSION 6

/* Element types.  The numbering is fixed. */
typedef enum spense_dtype {
  SPENSE_F32 = 0,      /* IEEE binary32 */
  SPENSE_BF16 = 1,     /* bfloat16 */
  SPENSE_FP8_E4M3 = 2  /* OCP e4m3fn: bias 7, largest finite 448, no infinities */
} spense_dtype;

typedef enum spense_status {
  SPENSE_OK = 0,
  SPENSE_EINVAL = -1,       /* bad argument (null pointer, size, dense set, ...) */
  SPENSE_EUNSUPPORTED = -2, /* valid but unsupported combination of types */
  SPENSE_ENOMEM = -3,       /* device or host allocation failed */
  SPENSE_EHIP = -4,         /* a HIP runtime call failed */
  SPENSE_ESCRATCH = -5      /* spense_linear_noalloc: the call needs more than its fixed scratch */
} spense_status;

typedef struct spense_layer* spense_handle;

typedef struct spense_layer_info {
  int64_t N, K;           /* weight shape */
  int64_t K_s, K_d;       /* sparse / dense region lengths, K_s + K_d = K, K_s % 4 == 0 */
  int32_t wdtype;         /* spense_dtype of the stored weights */
  int32_t gather;         /* 1 when spense_linear gathers activation columns (pi not the identity
                             on a 128-aligned split), 0 when X is read in place */
  int64_t weight_bytes;   /* bytes the method must stream per call: kept values + 2-bit indices
                             + dense block = N*(K_s/2*b + K_s/8 + K_d*b), b = element bytes */
  int64_t device_bytes;   /* bytes of the device-resident packed form, padding included */
  int32_t split;          /* 0: input-split layer (spense_pack); 1: output-split (spense_pack_rows);
                             2: GLU block (spense_pack_glu) */
  int64_t N_s, N_d;       /* output-split: 2:4 rows / dense rows (input-split: N and 0); for an
                             output-split layer K_s = K when N_s > 0 and K_d = K when N_d > 0.
                             GLU block: N = K = H, N_s / N_d = 2:4 / dense intermediate indices,
                             K_s / K_d those of the down projection */
} spense_layer_info;

/*
 * spense_pack - choose the 2:4 mask and build the packed layer (once per weight).
 *
 * Defined by Technical Summary 2.A / 2.B of the SpenseGPT explainer: the dense
 * set is either `dense_cols` (SpenseGPT+ style, any columns, order irrelevant)
 * or, when dense_cols is NULL, the last K_d = round(dense_fraction*K) columns
 * (SpenseGPT style, rounding half away from zero).  In every group of four
 * consecutive sparse-region columns (in pi order) the two entries with the
 * largest magnitude are kept, magnitude being the stored bit pattern with the
 * sign bit cleared; the lower in-group position wins ties.
 *
 *   W          device pointer, [N, ldw] elements of `wdtype`; only [N, K] is read.
 *   wdtype     SPENSE_F32, SPENSE_BF16 or SPENSE_FP8_E4M3.
 *   N, K       N >= 1, K >= 1; ldw >= K.
 *   scales     device pointer, [N] float32 per-output-channel dequantisation scales;
 *              required (non-NULL) iff wdtype == SPENSE_FP8_E4M3, must be NULL otherwise.
 *              Y[m,n] is multiplied by scales[n].
 *   dense_cols host pointer to n_dense distinct int32 column indices in [0, K), or NULL.
 *   n_dense    number of entries in dense_cols (ignored when dense_cols is NULL).
 *   dense_fraction  used only when dense_cols is NULL; must lie in [0, 1].
 *   stream     stream the packing kernels run on.
 *   out        receives the new handle.
 *
 * K - K_d must be a multiple of 4 (SPENSE_EINVAL otherwise).  The call returns
 * after the packed form is complete (it synchronises `stream`), so W and
 * scales may be freed or overwritten once it returns.  The handle owns every
 * buffer it holds; release it with spense_free.
 */
int spense_pack(const void* W, int32_t wdtype, int64_t N, int64_t K, int64_t ldw, const float* scales,
                const int32_t* dense_cols, int64_t n_dense, double dense_fraction, void* stream,
                spense_handle* out);

/*
 * spense_pack_rows - build an output-split layer (once per weight).
 *
 * Output-split form (Technical Summary 2.A of the SpenseGPT explainer; the
 * page uses it for the GLU gate and up projections): the output rows are
 * split instead of the input columns.  Rows in the dense row set keep all
 * their weights; every other row is 2:4 along K, in groups of four
 * consecutive columns (natural column order), with the same magnitude rule
 * and tie-break as spense_pack.  The two row classes produce different output
 * columns, so nothing is accumulated across them.  The dense row set is
 * `dense_rows` (any rows, order irrelevant) or, when dense_rows is NULL, the
 * last N_d = round(dense_fraction*N) rows.  Arguments as for spense_pack,
 * with dense_rows / n_dense naming rows in [0, N).
 *
 * wdtype must be SPENSE_BF16 or SPENSE_FP8_E4M3 (SPENSE_EUNSUPPORTED for
 * SPENSE_F32).  K must be a multiple of 4 when any row is sparse
 * (SPENSE_EINVAL otherwise).  spense_linear, spense_linear_splits, spense_info
 * and spense_free accept the handle; both row classes run in one launch.
 * Synchronises `stream` before returning.
 */
int spense_pack_rows(const void* W, int32_t wdtype, int64_t N, int64_t K, int64_t ldw, const float* scales,
                     const int32_t* dense_rows, int64_t n_dense, double dense_fraction, void* stream,
                     spense_handle* out);

/*
 * spense_pack_glu - build a GLU MLP block (once per block).
 *
 * Technical Summary 2.A and 2.B of the SpenseGPT explainer: in a GLU MLP the
 * gate and up projections are output-split and the down projection is
 * input-split, over one dense set D of intermediate indices (rows D of gate
 * and up, columns D of down keep all their weights); permuting the
 * intermediate indices so that D becomes one contiguous block leaves the
 * block's output unchanged.  That permutation rho = [other indices ascending
 * | D ascending] is applied here at pack time, so spense_glu gathers nothing.
 * Gate/up rows outside D are 2:4 along the hidden dimension; down columns
 * outside D are 2:4 in groups of four consecutive indices of rho (same
 * magnitude rule and tie-break as spense_pack).  The gate nonlinearity is
 * SiLU (the pages do not name it; the GLU models they evaluate use it).
 *
 *   W_gu       device pointer, [2I, ld_gu] elements: rows [0, I) the gate
 *              projection, rows [I, 2I) the up projection, each [I, H].
 *   W_down     device pointer, [H, ld_down] elements: the down projection [H, I].
 *   wdtype     SPENSE_BF16 or SPENSE_FP8_E4M3 (SPENSE_EUNSUPPORTED for SPENSE_F32).
 *   H, I       hidden and intermediate sizes; ld_gu >= H, ld_down >= I.
 *   s_gu, s_down  device pointers, [2I] and [H] float32 per-row scales; required
 *              iff wdtype == SPENSE_FP8_E4M3, NULL otherwise.
 *   dense_idx  host pointer to n_dense distinct intermediate indices in [0, I), or
 *              NULL for the last round(dense_fraction*I) indices.
 * I - |D| must be a multiple of 4, and so must H when I - |D| > 0
 * (SPENSE_EINVAL otherwise).  Synchronises `stream` before returning.
 */
int spense_pack_glu(const void* W_gu, const void* W_down, int32_t wdtype, int64_t H, int64_t I, int64_t ld_gu,
                    int64_t ld_down, const float* s_gu, const float* s_down, const int32_t* dense_idx,
                    int64_t n_dense, double dense_fraction, void* stream, spense_handle* out);

/*
 * spense_glu - Y = down(silu(gate(X)) * up(X)), the GLU block forward.
 *
 *   X     device pointer, [M, ldx] bf16, ldx >= H.
 *   A     device pointer, [M, lda] bf16, lda >= I: caller-owned workspace for the
 *         intermediate silu(gate) * up, written in rho order (column j holds
 *         intermediate index rho[j]; rho from spense_info's split layout:
 *         the 2:4 indices ascending, then the dense ones ascending).
 *   Y     device pointer, [M, ldy] elements of ydtype (SPENSE_F32 or SPENSE_BF16), ldy >= H.
 * Two launches on `stream`: gate and up (both row classes in one grid, the
 * SiLU * up product in its epilogue, rounded to bf16 into A), then down.
 * Workspaces grow as for spense_linear.
 */
int spense_glu(spense_handle h, const void* X, int64_t M, int64_t ldx, void* A, int64_t lda, void* Y,
               int32_t ydtype, int64_t ldy, void* stream);

/*
 * spense_score_glu - SpenseGPT+ importance score of every intermediate index of a GLU block.
 *
 * Technical Summary 2.B of the SpenseGPT explainer: each weight scores
 * |W_ij| * sqrt(H_jj), H = X^T X over calibration inputs of its projection,
 * and the scores are aggregated per intermediate index over the gate, up and
 * down projections.  Here (the pages leave the aggregation open) it is the
 * plain sum over the weights attached to index i:
 *   score[i] = sum_j |Wg[i,j]| sqrt(Hx_jj) + sum_j |Wu[i,j]| sqrt(Hx_jj)
 *            + sum_n |Wd[n,i]| sqrt(Ha_ii),
 * |W| the dequantised magnitude (per-row scale included).
 *
 *   W_gu, W_down, wdtype, H, I, ld_gu, ld_down, s_gu, s_down: as for spense_pack_glu
 *              (bf16 or e4m3 weights, the unpruned block).
 *   X_cal      device pointer, [T, ld_x] bf16: calibration inputs of gate and up, ld_x >= H.
 *   A_cal      device pointer, [T, ld_a] bf16: calibration inputs of down (the block's
 *              intermediate activations), ld_a >= I.
 *   score      device pointer, [I] float32 output.
 * Reductions run in a fixed order (bitwise repeatable).  Offline step: it
 * allocates scratch (hipMalloc) and synchronises `stream`.
 */
int spense_score_glu(const void* W_gu, const void* W_down, int32_t wdtype, int64_t H, int64_t I, int64_t ld_gu,
                     int64_t ld_down, const float* s_gu, const float* s_down, const void* X_cal, int64_t T,
                     int64_t ld_x, const void* A_cal, int64_t ld_a, float* score, void* stream);

/*
 * spense_select_dense - the dense set: the k indices with the highest scores.
 *
 *   score      device pointer, [n] float32 (for example from spense_score_glu).
 *   dense_idx  host pointer, [k] int32 output, ascending; ready for spense_pack_glu.
 * Index i is selected iff fewer than k indices j have score[j] > score[i] or
 * score[j] == score[i] with j < i (ties go to the lower index).  0 <= k <= n.
 * Infinite scores take their place in that order; a NaN score has none, and
 * the call then returns SPENSE_EINVAL (dense_idx untouched).  Allocates
 * scratch (hipMalloc) and synchronises `stream`.
 */
int spense_select_dense(const float* score, int64_t n, int64_t k, int32_t* dense_idx, void* stream);

/*
 * spense_linear - Y = X . W_pruned^T (times the per-channel scales), the layer forward.
 *
 * Input-split execution (Technical Summary 2.A): the sparse region runs on the
 * structured-sparse SMFMAC matrix instructions, the dense region on the same
 * instruction with index words that select every position (a dense 16x64
 * block is two such products), both accumulating into the same fp32
 * accumulators; when the dense set is not a 128-aligned tail the activation
 * columns are gathered through pi, inside the layer kernel for small batches
 * or into a handle-owned workspace by a preceding kernel on the same stream.
 * Accumulation is fp32; products of bf16 activations with bf16 or e4m3
 * weights are exact.
 *
 *   h          handle from spense_pack.
 *   X          device pointer, [M, ldx] elements of `xdtype`, ldx >= K.
 *              xdtype must be SPENSE_F32 for fp32 weights and SPENSE_BF16 otherwise.
 *   M          number of activation rows, M >= 1.
 *   Y          device pointer, [M, ldy] elements of `ydtype`, ldy >= N; only [M, N] is written.
 *   ydtype     SPENSE_F32 (fp32 accumulators as they are) or SPENSE_BF16 (round to nearest even).
 *
 * Asynchronous on `stream`.  Deterministic: repeated calls give bitwise equal
 * Y (split-K partial sums are added in a fixed order).  The first call at a
 * larger M than before may synchronise `stream` and allocate a larger split-K
 * or gather workspace (hipMalloc); SPENSE_ENOMEM if that fails.
 */
int spense_linear(spense_handle h, const void* X, int32_t xdtype, int64_t M, int64_t ldx, void* Y, int32_t ydtype,
                  int64_t ldy, void* stream);

/*
 * spense_linear_splits - spense_linear with the split-K factor forced (tuning and tests).
 * splits == 0 picks automatically; otherwise 1 <= splits <= number of 128-column steps.
 */
int spense_linear_splits(spense_handle h, const void* X, int32_t xdtype, int64_t M, int64_t ldx, void* Y,
                         int32_t ydtype, int64_t ldy, int32_t splits, void* stream);

/*
 * spense_linear_noalloc - spense_linear that allocates nothing.
 *
 * For callers that cannot allocate device memory during the call: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, result and kernels as spense_linear (automatic split
 * count), bitwise equal to it; only the call's workspaces differ: the split-K
 * counters and partials and the gathered activations live in a fixed device
 * array of 32 MiB that the library holds on every GPU it runs on until the
 * process ends (64 KiB of it for counters), instead of the handle's own
 * workspaces.  Its first call on a device looks the array up and clears its
 * counters (a fill kernel on `stream`); every completed call leaves them
 * cleared.  No hipMalloc, hipFree or other allocating routine is called.
 *
 * A call whose workspaces exceed the array returns SPENSE_ESCRATCH before any
 * launch (for example a chosen dense set gathered for a large batch: M * K_p
 * * 2 bytes, K_p = K rounded up per region to 128 columns).  Every call on
 * one GPU shares that GPU's array, so two such calls that overlap in time on
 * one GPU (different streams, or different host threads) race and must be
 * ordered by the caller; calls on one stream are ordered by the stream.
 */
int spense_linear_noalloc(spense_handle h, const void* X, int32_t xdtype, int64_t M, int64_t ldx, void* Y,
                          int32_t ydtype, int64_t ldy, void* stream);

/*
 * spense_quantize_tokens - per-token e4m3 quantisation of bf16 activations.
 *
 * The SpenseGPT explainer runs its layers in FP8 (Technical Summary 4,
 * "Experimental Results"); the SlideSparse explainer quantises activations
 * per token online, ahead of the 2:4 GEMM (Methodology 2.B "Activation
 * Lifting", 2.C).  The scale rule is not given there; this library uses the
 * absmax rule:
 *   sx[m]     = max_k |X[m][k]| / 448 as an fp32 quotient (448 is the largest
 *               e4m3fn value), or 1 for an all-zero row;
 *   Xq[m][k]  = the e4m3fn code nearest to the fp32 quotient X[m][k] / sx[m],
 *               ties to the even code, sign kept (within range by construction).
 *
 *   X    device pointer, [M, ldx] bf16, finite values, ldx >= K.
 *   Xq   device pointer, [M, ldq] e4m3 codes (uint8), ldq >= K; written.
 *   sx   device pointer, [M] float32; written.
 * 1 <= M <= 2^24, K >= 1 (SPENSE_EINVAL otherwise).  Asynchronous on `stream`.
 */
int spense_quantize_tokens(const void* X, int64_t M, int64_t K, int64_t ldx, uint8_t* Xq, int64_t ldq, float* sx,
                           void* stream);

/*
 * spense_linear_w8a8 - Y = sx[m] * s[n] * sum_k Xq[m][k] * Wp[n][k]: the layer
 * with e4m3 weights and per-token e4m3 activations.
 *
 * The activations are quantised as spense_quantize_tokens does; the same pass
 * writes them in the layer's packed column order (the dense-set permutation
 * rides on the quantisation, as the SlideSparse explainer folds its activation
 * re-ordering into per-token quantisation), into the handle's workspace.
 * Products of two e4m3 values are exact in fp32; the sum runs in fp32 in a
 * fixed order (bitwise repeatable).
 *
 *   h      an input-split layer packed from SPENSE_FP8_E4M3 weights
 *          (SPENSE_EUNSUPPORTED for other weight types and for output-split
 *          layers and GLU blocks).
 *   X      device pointer, [M, ldx] bf16, finite values, ldx >= K.
 *   Y      device pointer, [M, ldy] of ydtype (SPENSE_F32 or SPENSE_BF16 RNE), ldy >= N.
 *   splits split-K factor as for spense_linear_splits (0: automatic).
 * Grows the handle's workspaces on first use at a larger M (synchronising
 * `stream`); otherwise asynchronous.  One call in flight per handle.
 */
int spense_linear_w8a8(spense_handle h, const void* X, int64_t M, int64_t ldx, void* Y, int32_t ydtype, int64_t ldy,
                       int32_t splits, void* stream);

/* spense_info - sizes of a packed layer (host-side, no synchronisation). */
int spense_info(spense_handle h, spense_layer_info* info);

/*
 * spense_export - write the packed layer in its canonical form (for bit-exact checks).
 *
 *   vals   device pointer, [N, K_s/2] elements of wdtype: the two kept values of each
 *          group, lower position first.
 *   meta   device pointer, [N, ceil(K_s/32)] uint32: group g's nibble (i0 | i1 << 2),
 *          i0 < i1 its kept in-group positions, sits at bits 4*(g%8) of word g/8;
 *          unused nibbles are 0.
 *   mask   device pointer, [N, K_s] uint8: 1 on kept slots (columns in pi order).
 *   dense  device pointer, [N, K_d] elements of wdtype: W[:, pi[K_s:]].
 *   pi     host pointer, [K] int32 column order.
 * Any pointer may be NULL to skip that part.  Synchronises `stream` before returning.
 */
int spense_export(spense_handle h, void* vals, uint32_t* meta, uint8_t* mask, void* dense, int32_t* pi,
                  void* stream);

/*
 * spense_export_rows - canonical form of an output-split layer (for bit-exact checks).
 *
 *   vals   device pointer, [N_s, K/2]: kept values of the 2:4 rows, in rho order.
 *   meta   device pointer, [N_s, ceil(K/32)] uint32, encoded as for spense_export.
 *   mask   device pointer, [N_s, K] uint8, 1 on kept positions.
 *   dense  device pointer, [N_d, K]: the dense rows, in rho order.
 *   rho    host pointer, [N] int32 row order: the 2:4 rows ascending, then the dense rows ascending.
 * Any pointer may be NULL to skip that part.  SPENSE_EINVAL for an input-split
 * handle (and spense_export returns SPENSE_EINVAL for an output-split one).
 * Synchronises `stream` before returning.
 */
int spense_export_rows(spense_handle h, void* vals, uint32_t* meta, uint8_t* mask, void* dense, int32_t* rho,
                       void* stream);

/* spense_free - release the handle and its device buffers (no launch may still use it). */
int spense_free(spense_handle h);

/* Human-readable text for a status code (static storage). */
const char* spense_strerror(int status);

/* hipError_t value of the most recent SPENSE_EHIP on the calling thread (0 if none). */
int spense_last_hip_error(void);

/* SPENSE_ABI_VERSION of the loaded library. */
int spense_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPENSE_H */
