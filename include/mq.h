/*
 * mq.h -- C ABI of the MI355X (gfx950) MosaicQuant library.
 *
 * The library computes the ZipperEngine path of MosaicQuant ("MosaicQuant:
 * Inlier-Outlier Disaggregation for Unified 4-Bit LLM Quantization", technical
 * summary on gist.science): a weight matrix W^ [N][K] (out x in) is decomposed as
 * W^ ~ Q(W^) + R (Methodology 1), a dense 4-bit base plus a 4-bit residual kept
 * only for the top-K (bn x bk) blocks ranked by a Hessian-guided Delta-score
 * (Methodology 2), and Y = Xq Q(W^)^T + Xq R^T is computed by one fused kernel
 * that walks the residual blocks inside the dense 4-bit GEMM (Methodology 3).
 *
 * Conventions shared by every call
 *   - Every pointer argument is a DEVICE pointer (HBM), owned and allocated by the
 *     caller; the library keeps no reference after the call returns.
 *   - `stream` is a hipStream_t (NULL = the default stream). Calls are
 *     asynchronous on it unless stated otherwise.
 *   - Inputs are read-only. Outputs are fully overwritten. Inputs and outputs
 *     must not overlap.
 *   - int4 codes (values in [-7, 7]) are packed eight to a little-endian 32-bit
 *     word, inputs k0..k0+7 with k0 a multiple of 8: nibble e of the word (bits
 *     4e..4e+3) holds |c_e| in its low three bits and, in its high bit, the sign
 *     of code (e - 1) mod 8 (1 = negative; zero has no sign). With this encoding
 *     word & 0x87878787 and rotr(word, 4) & 0x87878787 are the fp8 (e4m3) MFMA
 *     operand bytes of the even and the odd codes (value c * 2^-9, exact).
 *   - Packed layouts (G = K/128 groups, G4 = ceil(G/4)). Each is chosen so that one
 *     64-lane 16-byte load of the GEMM reads 1 KB of contiguous memory:
 *       xq  activations, group-major: the word at byte (g*M + m)*64 + 4i holds
 *           inputs 128g + 8i .. 128g + 8i + 7 of token m.
 *       wq  base codes, tiled by 16 rows x 1 group: row n, group g, byte j (0..63)
 *           of the row's 64-byte group chunk (words in input order) is at
 *             ((n/16)*G + g)*1024 + ((j/16)*16 + n%16)*16 + j%16.
 *       sw  fp16 group scales, four groups per row entry: scale (n, g) is element
 *             (((n/16)*G4 + g/4)*16 + n%16)*4 + g%4   of a u16 array of N*G4*4;
 *           entries of groups g >= G are zero.
 *       rq  residual codes of the chosen blocks, [nnz][bn][bk/2], rows contiguous
 *           (8 words of 8 codes per block row).
 *     Sizes: xq M*K/2 bytes, wq N*K/2 bytes, sw N*G4*4 u16, rq nnz*bn*bk/2 bytes.
 *   - Packed buffers (xq, wq, rq), the activations x and the fp32 w and h must be
 *     16-byte aligned; sw must be 8-byte aligned.
 *   - Argument checks happen before any launch and return MQ_ERR_INVALID_ARG or
 *     MQ_ERR_UNSUPPORTED with nothing written. A failed launch returns
 *     MQ_ERR_HIP; faults inside a kernel surface at the caller's next
 *     synchronisation of `stream`.
 *   - Shapes the GPU path supports: K % 128 == 0, K <= 65536, group == 128, bk == 64,
 *     bn in {64, 128}, N % bn == 0. M may be any value >= 0 (M == 0 is a no-op).
 *   - Inputs must be finite, and max|w| over a group must be below 7 * 65504
 *     (the fp16 scale must be finite); otherwise results are unspecified.
 */
#ifndef MQ_H
#define MQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MQ_OK = 0,
    MQ_ERR_INVALID_ARG = -1,  /* null pointer, bad size, misaligned buffer, k_blocks > NB */
    MQ_ERR_UNSUPPORTED = -2,  /* shape outside the supported set above */
    MQ_ERR_HIP = -3,          /* a HIP runtime call or launch failed */
    MQ_ERR_SCRATCH = -4       /* the shape needs more than the library's static scratch */
} mq_status;

typedef enum { MQ_F32 = 0, MQ_BF16 = 1 } mq_dtype;

/* Human-readable text for a status code (static storage). */
const char* mq_status_string(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int mq_version(void);

/*
 * Diagonal-Hessian estimate of the input channels (Methodology 2: the
 * "activation sensitivity" that weights the residual error in the Delta-score).
 *   h[k] = fp32( (sum over m = 0..M-1, in ascending order, of (double)x[m][k]^2) / M )
 * x: [M][K] fp32 or bf16 (x_dtype), h: fp32 [K]. M >= 1, K >= 1.
 */
int mq_hessian_diag(const void* x, int x_dtype, int64_t M, int64_t K, float* h, void* stream);

/*
 * Migration of activation outliers into the weights by an equivalent per-channel
 * transform (Methodology 1: the method starts by moving activation outliers into
 * the weight matrix, SmoothQuant being one such transform; the exponent is not
 * given, alpha = 1/2 here):
 *   a_k = max_m |x[m][k]|, b_k = max_n |w[n][k]|,
 *   s[k] = sqrtf(a_k) / sqrtf(b_k)  (fp32, correctly rounded), 1 when a_k or b_k is 0,
 *   r[k] = 1 / s[k].
 * The migrated layer is W^ = W diag(s) (mq_scale_columns) and X^ = X diag(r), which
 * the *_scaled calls below apply on the fly: X^ W^T = X W^T up to rounding.
 * x: [M][K] fp32 or bf16, w: fp32 [N][K], s and r: fp32 [K]. Asynchronous on `stream`.
 */
int mq_smooth_factors(const void* x, int x_dtype, int64_t M, int64_t K, const float* w, int64_t N,
                      float* s, float* r, void* stream);

/* w_hat[n][k] = fp32(w[n][k] * s[k]) (the migrated weights). K % 4 == 0; w, s and
 * w_hat 16-byte aligned; w_hat may equal w (in place). */
int mq_scale_columns(const float* w, int64_t N, int64_t K, const float* s, float* w_hat, void* stream);

/* mq_hessian_diag of the migrated activations x^[m][k] = fp32(x[m][k] * r[k]). */
int mq_hessian_diag_scaled(const void* x, int x_dtype, int64_t M, int64_t K, const float* r, float* h,
                           void* stream);

/* mq_quantize_act of the migrated activations x^[m][k] = fp32(x[m][k] * r[k]); the
 * per-call path of a migrated layer (r 16-byte aligned). */
int mq_quantize_act_scaled(const void* x, int x_dtype, int64_t M, int64_t K, const float* r, uint8_t* xq,
                           float* sx, void* stream);

/*
 * Per-token symmetric int4 activation quantization (the W4A4 setting of the
 * Experimental Results; "quantization" is the first stage of the ZipperEngine
 * pipeline, Methodology 3).
 *   sx[m] = fp32(max_k |x[m][k]| / 7)
 *   xq[m][k] = sx[m] == 0 ? 0 : clamp(rint(x[m][k] / sx[m]), -7, 7)   (ties to even)
 * x: [M][K] fp32 or bf16 (row-major, 16-byte aligned), xq: M*K/2 bytes in the
 * group-major layout above, sx: fp32 [M]. K % 128 == 0.
 */
int mq_quantize_act(const void* x, int x_dtype, int64_t M, int64_t K, uint8_t* xq, float* sx,
                    void* stream);

/*
 * Hessian-guided Delta-score of every (bn x bk) block and global top-k_blocks
 * selection (Methodology 2 "Block-wise Residual Allocation").
 * For element (n, k) of group g with fp16 base scale s (see mq_pack_weights):
 *   q = base code, E = w - s*q, s_r = fp32(s / 14), r = clamp(rint(E / s_r), -7, 7),
 *   E' = E - s_r*r (single rounding).
 *   Delta_b = sum over rows n of b (ascending) of
 *             [ sum over cols k of b (ascending) of (double)h[k] * (E^2 - E'^2) ]
 * every fp64 operation rounded separately. Blocks are ranked by (Delta descending,
 * id ascending), id = (n / bn) * (K / bk) + k / bk, and the first k_blocks are
 * chosen. Output is CSR over block rows:
 *   row_ptr: int32 [N/bn + 1], col_idx: int32 [k_blocks] (column-block index,
 *   ascending within a row), delta: fp64 [NB] with NB = (N/bn)*(K/bk).
 * w: fp32 [N][K], h: fp32 [K]. 0 <= k_blocks <= NB.
 * delta may be NULL (the scores are then kept in the workspace and not returned).
 * workspace: device scratch of at least mq_select_workspace_bytes(N, K, bn, bk) bytes,
 * 8-byte aligned (the per-block ranks, 4 * NB bytes, and when delta is NULL the
 * scores, 8 * NB more), or NULL: the call then takes a stream-ordered allocation
 * (hipMallocAsync) and releases it on the same stream. Calls sharing one
 * workspace must be ordered on one stream.
 */
int mq_select_blocks(const float* w, const float* h, int64_t N, int64_t K, int group, int bn,
                     int bk, int64_t k_blocks, int32_t* row_ptr, int32_t* col_idx,
                     double* delta, void* workspace, size_t workspace_bytes, void* stream);

/*
 * mq_select_blocks for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. Same
 * arguments, results and errors as mq_select_blocks without a workspace; its
 * scratch (select ranks, and the scores when delta is NULL) is a static device
 * array of MQ_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs
 * on until the process ends. The call makes no allocation of any kind.
 * Limit: 4 * NB bytes (rounded up to 8) plus 8 * NB when delta is NULL must fit,
 * i.e. NB <= 349525 with delta NULL, NB <= 1048576 otherwise; larger shapes
 * return MQ_ERR_SCRATCH with nothing launched. Every call on one GPU shares that
 * GPU's array: calls that overlap on one GPU (different streams, or threads
 * without ordering) race and give wrong results; order them on one stream.
 * The first call on a device looks up the array's address on that device
 * (hipGetSymbolAddress) with the device current.
 */
#define MQ_NOALLOC_SCRATCH_BYTES (4u << 20)
int mq_select_blocks_noalloc(const float* w, const float* h, int64_t N, int64_t K, int group,
                             int bn, int bk, int64_t k_blocks, int32_t* row_ptr,
                             int32_t* col_idx, double* delta, void* stream);

/* Workspace bytes mq_select_blocks needs for this shape with delta == NULL (12 * NB;
   4 * NB suffice when delta is given); 0 for an unsupported shape. */
size_t mq_select_workspace_bytes(int64_t N, int64_t K, int bn, int bk);

/*
 * Packs the dense 4-bit base for every group and the 4-bit residual payload for
 * the chosen blocks (Methodology 1: W^ ~ Q(W^) + R, both parts 4-bit).
 *   sw(n, g) = fp16_rne( fp32(max_{k in g} |w[n][k]|) / 7 )      (fp16 bits)
 *   wq(n, k) = s == 0 ? 0 : clamp(rint(w / s), -7, 7)  with s = fp32(sw(n, g))
 *   rq[p][i][c] = residual code r (see mq_select_blocks) of row (row_block*bn + i),
 *                 column (col_idx[p]*bk + c) for CSR entry p, in CSR order.
 * w: fp32 [N][K] row-major; row_ptr/col_idx as produced by mq_select_blocks (nnz
 * entries); wq, sw, rq in the packed layouts above (rq may be NULL if nnz == 0).
 * Entries with a column-block index outside [0, K/bk) are skipped.
 */
int mq_pack_weights(const float* w, int64_t N, int64_t K, int group, int bn, int bk,
                    const int32_t* row_ptr, const int32_t* col_idx, int64_t nnz,
                    uint8_t* wq, uint16_t* sw, uint8_t* rq, void* stream);

/*
 * The fused ZipperEngine GEMM (Methodology 3): one kernel streams the packed base
 * and, inside the same K-loop, the residual blocks listed for its rows; both
 * products are summed exactly per 128-group (integers; the fp8 MFMA returns them
 * scaled by 2^-18 without rounding), and the group sums are dequantized and
 * summed in fp32:
 *   T[m][n][g] = 14 * P + Pr,  P = sum_{k in g} xq*q,  Pr = sum over chosen blocks in g of xq*r
 *   y[m][n]    = sx[m] * sum_g ( groups with a chosen block in this row: s_r * T,
 *                                otherwise s * P )            (fp32; s_r = fp32(s/14))
 * which equals sx * sum_g (s*P + s_r*Pr) up to fp32 rounding.
 * xq, wq, sw, rq in the packed layouts above (rq NULL if nnz == 0), sx: fp32 [M],
 * row_ptr: int32 [N/bn+1], col_idx: int32 [nnz],
 * y: [M][N] fp32 or bf16 (y_dtype, bf16 rounded to nearest even).
 * acc_dump: NULL, or int32 [M][N][K/group] receiving T (a debug build of the same
 * kernel; production calls pass NULL). Indices outside the CSR ranges are ignored,
 * so a malformed list gives wrong values, never an out-of-bounds access.
 * The call allocates nothing and needs no scratch memory.
 */
int mq_gemm_w4a4_residual(const uint8_t* xq, const float* sx, const uint8_t* wq,
                          const uint16_t* sw, const int32_t* row_ptr, const int32_t* col_idx,
                          const uint8_t* rq, int64_t nnz, int64_t M, int64_t N, int64_t K,
                          int group, int bn, int bk, void* y, int y_dtype, int32_t* acc_dump,
                          void* stream);

/*
 * The dense block map of a selection (Methodology 3: the fused kernel finds each
 * 128-group's residual blocks in step with the K loop; with the map that lookup is
 * one coalesced load per wavefront instead of a walk of the block row's list):
 *   rmap[b][j] = p  if col_idx[p] == j for some p in [row_ptr[b], row_ptr[b+1]),
 *              = -1 otherwise,
 * for block rows b < N/bn and column blocks j < K/bk. rmap: int32 [N/bn][K/bk]
 * (device, 4-byte aligned), fully overwritten. Entries with a column-block index
 * outside [0, K/bk) are skipped; for a block listed twice in one row, one of its
 * positions is kept. Row pointers are clamped to [0, nnz]. Asynchronous.
 */
int mq_block_map(const int32_t* row_ptr, const int32_t* col_idx, int64_t nnz, int64_t N, int64_t K,
                 int bn, int bk, int32_t* rmap, void* stream);

/*
 * mq_gemm_w4a4_residual with the chosen blocks found through a block map
 * (mq_block_map of the CSR lists the payload was packed with) instead of the lists:
 * the same kernels and the same arithmetic, so y and acc_dump are bit-identical to
 * mq_gemm_w4a4_residual's. Map entries outside [0, nnz) mean "no block".
 * Requires nnz * bn * bk / 2 <= 2^31 (else MQ_ERR_UNSUPPORTED).
 */
int mq_gemm_w4a4_residual_mapped(const uint8_t* xq, const float* sx, const uint8_t* wq,
                                 const uint16_t* sw, const int32_t* rmap, const uint8_t* rq,
                                 int64_t nnz, int64_t M, int64_t N, int64_t K, int group, int bn,
                                 int bk, void* y, int y_dtype, int32_t* acc_dump, void* stream);

/*
 * The fused GEMM that also quantizes its activations (Methodology 3 schedules
 * quantization as a stage of the same pipeline as the dense and sparse products):
 * y = mq_gemm_w4a4_residual_mapped applied to mq_quantize_act(x), with xq and sx
 * written as mq_quantize_act writes them (same bits), and y bit-identical to the
 * two calls in sequence.
 * It runs either as one launch (M <= 32): its first M workgroups quantize one
 * token each while the output-column workgroups wait for them (counters in
 * `sync`) before reading any activation; or as two launches on `stream`,
 * mq_quantize_act and then the GEMM. `launch` picks: MQ_ACT_ONE_LAUNCH (M > 32
 * is then an invalid argument), MQ_ACT_TWO_LAUNCHES, or MQ_ACT_AUTO, which takes
 * one launch when mq_act_one_launch(M, N, K) says so and two otherwise. Both give
 * the same bits.
 * x: [M][K] fp32 or bf16 (x_dtype), 16-byte aligned; xq, sx: outputs as in
 * mq_quantize_act; rmap, rq, nnz: as in mq_gemm_w4a4_residual_mapped (rmap required).
 * sync (required when the one-launch form runs, else unused and may be null):
 * int32 [MQ_SYNC_WORDS] device array, all zero before the first call (e.g.
 * zero-filled once); every completed call leaves it zero again, so it needs no
 * clearing between calls and the call can be captured in a HIP graph. It holds the
 * count of quantized tokens, a check-in count and, in one 128-byte line per XCD
 * slot, a ready flag and a count of finished column workgroups. sync[2] becomes 1
 * if a workgroup ever gave up waiting (after well under a few seconds; never
 * expected) and stays 1 until the caller clears it. Calls that share one sync
 * array must not overlap (order them on one stream).
 */
#define MQ_SYNC_WORDS 544
#define MQ_ACT_AUTO 0
#define MQ_ACT_ONE_LAUNCH 1
#define MQ_ACT_TWO_LAUNCHES 2
/*
 * The MQ_ACT_AUTO rule of mq_gemm_w4a4_residual_act, for callers that need to know
 * beforehand whether the counters are required: 1 if the call takes one launch
 * for this shape, else 0 (also for M outside 1..32, and for shapes the GEMM does
 * not accept). Host only; no GPU call.
 * One launch when its per-token quantizing workgroups (the decode plan's waves)
 * are at least as wide as the stand-alone quantizer's, M = 1 and N >= 4096: where
 * it measured faster on MI355X.
 */
int mq_act_one_launch(int64_t M, int64_t N, int64_t K);
int mq_gemm_w4a4_residual_act(const void* x, int x_dtype, const uint8_t* wq, const uint16_t* sw,
                              const int32_t* rmap, const uint8_t* rq, int64_t nnz, int64_t M,
                              int64_t N, int64_t K, int group, int bn, int bk, uint8_t* xq,
                              float* sx, int32_t* sync, int launch, void* y, int y_dtype, void* stream);

/*
 * Measurement aid, not a step of the method: a plain streaming read of `bytes`
 * bytes at p (16-byte aligned, bytes a multiple of 16), the HBM read rate a kernel
 * reaches at that byte count. The decode GEMM streams its weights once, so this
 * is the ceiling its time is compared with (the Experimental Results measure
 * decode overheads against the dense kernel; this measures both against memory).
 * out: uint32 [MQ_READ_PROBE_WORDS] device array; each workgroup writes the XOR of
 * the words it read to one entry (the values mean nothing). Asynchronous.
 */
#define MQ_READ_PROBE_WORDS 8192
int mq_read_probe(const void* p, int64_t bytes, uint32_t* out, void* stream);

/*
 * Dense-only 4-bit GEMM: the same kernel with the residual path compiled out
 * (the "dense 4-bit GEMM kernel" the residual is fused into, Methodology 3).
 * y = sx * sum_g s * P. With nnz == 0 the fused call gives the same bits.
 * acc_dump (optional) receives T = 14 * P.
 */
int mq_gemm_w4a4_dense(const uint8_t* xq, const float* sx, const uint8_t* wq, const uint16_t* sw,
                       int64_t M, int64_t N, int64_t K, int group, void* y, int y_dtype,
                       int32_t* acc_dump, void* stream);

/*
 * The separate-kernel alternative that Methodology 3 argues against: the dense
 * kernel writes fp32 partial outputs to `ws` (fp32 [M][N], caller-allocated),
 * then a second kernel re-reads the activations, computes the residual product
 * block by block, merges it into the partial outputs and writes y.
 * y = sx * sum_g (s*P + s_r*Pr) up to fp32 rounding. Same arguments as the fused
 * call plus ws.
 */
int mq_gemm_residual_separate(const uint8_t* xq, const float* sx, const uint8_t* wq,
                              const uint16_t* sw, const int32_t* row_ptr, const int32_t* col_idx,
                              const uint8_t* rq, int64_t nnz, int64_t M, int64_t N, int64_t K,
                              int group, int bn, int bk, void* y, int y_dtype, float* ws,
                              void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MQ_H */
