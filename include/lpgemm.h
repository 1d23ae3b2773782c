/*
 * lpgemm: low-precision dense GEMM C = A.B for one AMD Instinct MI355X (gfx950).
 *
 * The operation is the one the PTX-vs-WMMA summary page (thecoregrid.dev,
 * "PTX Tensor-Core GEMM", paragraphs on FP16, INT8 and INT4 and on the s4 mma
 * shape) measures: a dense GEMM in FP16, INT8 and INT4.  Integer operands are
 * summed exactly in int32; FP16 operands are summed in FP32.  A fourth entry
 * point applies a per-row x per-column fp32 dequantisation to the exact int8
 * product, the step after the GEMM in quantised-LLM inference (the page's
 * closing recommendation on quantised LLM inference on one GPU).
 *
 * Layouts (fixed; there are no leading-dimension arguments):
 *   A  M x K, row-major (each row is K contiguous elements).
 *   B  K x N stored K-contiguous: N rows of K contiguous elements, i.e. the
 *      N x K row-major array B^T (the layout the page's ablation keeps;
 *      its variant with B transposed lost coalescing).
 *   C  M x N, row-major.
 *   INT4: two signed 4-bit values per byte along k; byte t of a row holds
 *      element 2t in its low nibble and element 2t+1 in its high nibble, each
 *      a two's-complement nibble (-8..7).  A_packed is M x K/2 bytes and
 *      B_packed is N x K/2 bytes.
 *   FP16: IEEE binary16 (bit-compatible with _Float16 / torch.float16).
 *   Scales: row_scale[M] and col_scale[N], fp32.
 *
 * Semantics: C is overwritten with A.B (no alpha/beta, no accumulation into
 * C).  The work is enqueued on `stream` (NULL = the default stream) and the
 * call returns after the enqueue, without synchronising.
 *
 * Ownership: every pointer is device memory owned by the caller, which must
 * keep it valid until the enqueued work completes.  The library allocates no
 * memory, keeps no per-call state and may be called from several host threads
 * (the split-K entry points keep per-tile counters in the caller's
 * workspace).
 * C must not overlap A, B or the scales.
 *
 * Degenerate sizes: M = 0 or N = 0 is an empty product; the call returns
 * LPGEMM_SUCCESS without enqueueing anything or reading any pointer.  K = 0
 * is an empty sum: C is filled with zeros, and A and B may then be NULL.
 *
 * Errors (checked on the host before any HIP call, in this order):
 *   LPGEMM_ERROR_INVALID_VALUE     M, N or K negative, or M or N above
 *                                  2^31 - 1.
 *   LPGEMM_ERROR_UNSUPPORTED_SHAPE K breaks the entry point's divisibility or
 *                                  range rule (each function says which).
 *   (M = 0 or N = 0 returns LPGEMM_SUCCESS here.)
 *   LPGEMM_ERROR_INVALID_VALUE     C, a scale array, or (for K > 0) A or B
 *                                  is NULL.
 *   LPGEMM_ERROR_MISALIGNED        A, B or C not 16-byte aligned (the scale
 *                                  arrays need only 4-byte alignment).
 * then, after selecting the current device:
 *   LPGEMM_ERROR_ARCH              the current device is not gfx950, or its
 *                                  properties could not be read.
 *   LPGEMM_ERROR_LAUNCH            the kernel launch was rejected.
 * Faults during execution are reported by the caller's next synchronisation
 * of the stream, as for any HIP kernel.  M and N need no divisibility: edge
 * tiles are masked.
 */
#ifndef LPGEMM_H
#define LPGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as HIP's own hipStream_t. */
typedef struct ihipStream_t *hipStream_t;

typedef enum lpgemm_status {
    LPGEMM_SUCCESS = 0,
    LPGEMM_ERROR_INVALID_VALUE = 1,
    LPGEMM_ERROR_MISALIGNED = 2,
    LPGEMM_ERROR_UNSUPPORTED_SHAPE = 3,
    LPGEMM_ERROR_ARCH = 4,
    LPGEMM_ERROR_LAUNCH = 5
} lpgemm_status;

/* Largest K of the integer entry points: with every product equal to
 * (-128)^2 = 2^14, the exact sum 2^14 * K still fits int32 for K <= 131071. */
#define LPGEMM_MAX_K_INT 131071
/* Largest K of the fp16 entry point: an operand panel of 256 rows then stays
 * well below 2 GiB, the reach of the 32-bit offsets the kernels' loads use. */
#define LPGEMM_MAX_K_F16 1048576

/* INT8: C[i][j] = sum_k A[i][k] * B[k][j], exact in int32.
 * A: M x K int8, B: N x K int8 (K-contiguous), C: M x N int32.
 * K must be a multiple of 16 and at most LPGEMM_MAX_K_INT. */
lpgemm_status lpgemm_i8(int64_t M, int64_t N, int64_t K, const int8_t *A, const int8_t *B,
                        int32_t *C, hipStream_t stream);

/* INT4: the same exact int32 product over signed 4-bit operands packed two
 * per byte (low nibble = even k).  A_packed: M x K/2 bytes, B_packed: N x K/2
 * bytes, C: M x N int32.  K counts 4-bit elements; it must be a multiple of
 * 32 and at most LPGEMM_MAX_K_INT. */
lpgemm_status lpgemm_i4(int64_t M, int64_t N, int64_t K, const uint8_t *A_packed,
                        const uint8_t *B_packed, int32_t *C, hipStream_t stream);

/* FP64 GEMM emulated with exact INT8 GEMMs (the FP64-emulation page of the
 * series, day 12: scale / exponent scan, residue quantisation, INT8 GEMM, mod
 * reduction, CRT reconstruction, undo scaling, write double).  C ~ A . B for
 * fp64 A (M x K, row-major) and B stored K-contiguous (N x K), fp64 C
 * (M x N).  `bits` (1..53) is the target: each row of A and each column of B
 * is scaled by a power of two to integers of at most `bits` bits (nearest,
 * ties to even), their exact product is formed through one int8 GEMM per
 * modulus (lpgemm_f64_emu_moduli tells how many) and the Chinese remainder
 * theorem, rounded once to double and scaled back.  The only error is that
 * scaling (plus the final rounding).  K must be a multiple of 16 and at most
 * LPGEMM_MAX_K_INT.  The caller provides `workspace` (256-byte aligned) of at
 * least lpgemm_f64_emu_workspace(M, N, K, bits) bytes; the library still
 * allocates nothing.  A, B, C 16-byte aligned.  Inputs must be finite; results
 * that fall below the normal range are rounded a second time.  Errors: as for
 * the GEMMs, plus INVALID_VALUE for bits outside 1..53 or a workspace that is
 * missing or too small. */
int lpgemm_f64_emu_moduli(int64_t K, int bits);
int64_t lpgemm_f64_emu_workspace(int64_t M, int64_t N, int64_t K, int bits);
lpgemm_status lpgemm_f64_emu(int64_t M, int64_t N, int64_t K, const double *A, const double *B,
                             double *C, int bits, void *workspace, int64_t workspace_bytes,
                             hipStream_t stream);

/* Largest workspace of lpgemm_f64_emu_noalloc: 64 MiB (M = N = K = 1024 at
 * 53 bits needs about 48 MiB). */
#define LPGEMM_F64_EMU_NOALLOC_MAX_WORKSPACE (64 * 1024 * 1024)

/* lpgemm_f64_emu for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same operation, arguments and result (bit for bit) as lpgemm_f64_emu, but
 * the intermediates live in a scratch array of
 * LPGEMM_F64_EMU_NOALLOC_MAX_WORKSPACE bytes that the library holds in the
 * device memory of each GPU it runs on, from the library's first use on that
 * GPU until the process ends; the call itself allocates nothing.  Shapes
 * whose workspace (lpgemm_f64_emu_workspace) exceeds that size return
 * LPGEMM_ERROR_UNSUPPORTED_SHAPE before anything is enqueued.  Every call on
 * one GPU shares its scratch, which keeps the last call's contents: calls
 * that overlap in time on one GPU (on different streams, or from several
 * host threads) race and give wrong results, so serialise them (for
 * instance on one stream).  Nothing needs clearing between calls: each call
 * writes every scratch byte it reads.  Errors as for lpgemm_f64_emu (without
 * the workspace cases), plus LPGEMM_ERROR_LAUNCH if the scratch's device
 * address cannot be obtained. */
lpgemm_status lpgemm_f64_emu_noalloc(int64_t M, int64_t N, int64_t K, const double *A, const double *B,
                                     double *C, int bits, hipStream_t stream);

/* INT8 with B stored K x N row-major (N contiguous; the "transposed" B of
 * the PTX-vs-WMMA summary page's layout ablation): C = A . B exactly in
 * int32, as lpgemm_i8.  A: M x K int8, B_kxn: K x N int8, C: M x N int32.
 * K must be a multiple of 16 and at most LPGEMM_MAX_K_INT; N a multiple of
 * 16 (every k-row starts 16-byte aligned) with K * N < 2^31.  Pointers
 * 16-byte aligned.  Errors and degenerate sizes as for lpgemm_i8. */
lpgemm_status lpgemm_i8_kxn(int64_t M, int64_t N, int64_t K, const int8_t *A, const int8_t *B_kxn,
                            int32_t *C, hipStream_t stream);

/* INT4 through FP6 E3M2 matrix cores, step 1 of 2: re-encode packed int4
 * rows (the layout of lpgemm_i4: two values per byte along k, low nibble =
 * even k, two's complement) as E3M2 operand rows.  Every value in [-8, 7] is
 * exact in E3M2; gfx950 multiplies FP6 operands at about twice its int8 rate
 * (a route to the PTX-vs-WMMA summary page's native 4-bit tensor-core path,
 * which this chip lacks for integers).  src_packed: rows x K/2 bytes;
 * dst: rows x K bytes, each group of 32 values becoming 24 bytes of six-bit
 * codes followed by 8 zero bytes (the codes in an order private to the
 * library; dst is meant only for lpgemm_i4_e3m2).  K must be a multiple of
 * 32 and at most LPGEMM_MAX_K_INT; both pointers 16-byte aligned.  rows = 0
 * or K = 0 is a no-op.  Weights that do not change need converting once. */
lpgemm_status lpgemm_i4_to_e3m2(int64_t rows, int64_t K, const uint8_t *src_packed, uint8_t *dst,
                                hipStream_t stream);

/* INT4 through FP6 E3M2, step 2 of 2: C = A . B exactly in int32 for int4
 * operands that lpgemm_i4_to_e3m2 has re-encoded (A_e3m2: M x K bytes,
 * B_e3m2: N x K bytes).  Products are at most 64 and the fp32 sums are
 * integers below 2^24 for K <= LPGEMM_MAX_K_INT, so the result equals
 * lpgemm_i4's bit for bit.  Shapes, alignment and errors as for lpgemm_i4. */
lpgemm_status lpgemm_i4_e3m2(int64_t M, int64_t N, int64_t K, const uint8_t *A_e3m2,
                             const uint8_t *B_e3m2, int32_t *C, hipStream_t stream);

/* FP16: C[i][j] = sum_k A[i][k] * B[k][j] with binary16 operands, products
 * and sums in binary32 (the summation order is unspecified).  A: M x K,
 * B: N x K (K-contiguous), C: M x N fp32.  The pointers have the bit layout of
 * binary16 (_Float16 or uint16_t storage).  K must be a multiple of 8 and at
 * most LPGEMM_MAX_K_F16. */
lpgemm_status lpgemm_f16(int64_t M, int64_t N, int64_t K, const void *A, const void *B,
                         float *C, hipStream_t stream);

/* INT8 with dequantisation: acc = the exact int32 product of lpgemm_i8, then
 * C[i][j] = ((float)acc * row_scale[i]) * col_scale[j], each multiplication
 * rounded to binary32 (nearest even) in that order.  C: M x N fp32.
 * K as for lpgemm_i8. */
lpgemm_status lpgemm_i8_dequant(int64_t M, int64_t N, int64_t K, const int8_t *A,
                                const int8_t *B, const float *row_scale,
                                const float *col_scale, float *C, hipStream_t stream);

/* Split-K variants of lpgemm_i8, lpgemm_i4, lpgemm_f16 and lpgemm_i8_dequant
 * for products with few output tiles and a long K, whose tiles alone would
 * leave most of the GPU idle (the PTX-vs-WMMA summary page's INT4 paragraph
 * picks the pipeline per problem size).  Same operation, arguments,
 * layouts, result and errors as the entry point without the suffix, plus a
 * caller-provided workspace in device memory:
 *   lpgemm_splitk_workspace(M, N) is the number of bytes the automatic
 *   choice may use for an M x N product on the current device, whatever K
 *   is (0 when that product never splits; -1 for sizes outside 0..2^31-1
 *   or when the device cannot be queried).
 * The automatic choice splits when M > 64, the product's 128 x 128 output
 * tiles number at most a quarter of the GPU's compute units, for M > 128
 * its 64 x 64 tiles number more than a quarter of them (below that the
 * unsplit kernel already splits K inside each workgroup), and each operand
 * row holds more than 31 x 256 bytes (int8 K >= 7952, fp16 K >= 3976, int4
 * K >= 15904); below 64 x 256 bytes only when the product's 128 x 64 tiles
 * number less than half the compute units or the kind is int4 (otherwise
 * the unsplit kernel was as fast).  The K dimension of each tile is then split
 * over 4 workgroups; each writes its partial sums to the workspace and the
 * last of a tile to finish adds them and writes C.
 * The integer results are exact and equal to the unsplit entry point's bit
 * for bit; the fp16 result adds the parts in a fixed order, so it is
 * deterministic and within the same error bound, but may differ from the
 * unsplit one in the last bits.  Any other shape, a null workspace, or one
 * smaller than lpgemm_splitk_workspace(M, N), runs the product unsplit.
 * The workspace must be 256-byte aligned and ZEROED ONCE before its first
 * use (for instance with hipMemset): its first 4 KiB hold one arrival
 * counter per tile, and every call leaves the counters at zero when it
 * completes, so the same workspace serves any number of later calls, of any
 * shape, without clearing (a product of more than 1024 tiles never
 * splits).  Calls that
 * share a workspace must not overlap in time (serialise them, for instance
 * on one stream).  Errors, after the unsuffixed entry point's argument
 * checks: INVALID_VALUE for workspace_bytes < 0, MISALIGNED for a workspace
 * that is not 256-byte aligned.  The workspace must not overlap A, B, C or
 * the scales. */
int64_t lpgemm_splitk_workspace(int64_t M, int64_t N);
lpgemm_status lpgemm_i8_splitk(int64_t M, int64_t N, int64_t K, const int8_t *A, const int8_t *B,
                               int32_t *C, void *workspace, int64_t workspace_bytes, hipStream_t stream);
lpgemm_status lpgemm_i4_splitk(int64_t M, int64_t N, int64_t K, const uint8_t *A_packed,
                               const uint8_t *B_packed, int32_t *C, void *workspace,
                               int64_t workspace_bytes, hipStream_t stream);
lpgemm_status lpgemm_f16_splitk(int64_t M, int64_t N, int64_t K, const void *A, const void *B, float *C,
                                void *workspace, int64_t workspace_bytes, hipStream_t stream);
lpgemm_status lpgemm_i8_dequant_splitk(int64_t M, int64_t N, int64_t K, const int8_t *A, const int8_t *B,
                                       const float *row_scale, const float *col_scale, float *C,
                                       void *workspace, int64_t workspace_bytes, hipStream_t stream);

/* Largest M of lpgemm_w8a8_fused: one band of 32 rows, the decode-sized
 * products it is meant for. */
#define LPGEMM_W8A8_FUSED_MAX_M 32

/* The W8A8 projection in one launch: C = the result of
 * lpgemm_quantize_rows_f16(X) followed by lpgemm_i8_dequant(Q, W, row_scale,
 * w_scale), bit for bit, without materialising Q or the row scales.  The
 * Day-12 page weighs a quantisation prologue inside the GEMM, which repeats
 * its work per tile, against a separate pass; this is the fused side of that
 * comparison: every workgroup rescans its rows for their absmax and rounds
 * each A fragment as it loads it.  X: M x K binary16 (row-major), W: N x K
 * int8 (K-contiguous), w_scale: N floats, C: M x N fp32.  1 <= M <=
 * LPGEMM_W8A8_FUSED_MAX_M (UNSUPPORTED_SHAPE otherwise); K as for
 * lpgemm_i8_dequant.  X, W, C 16-byte aligned, w_scale 4-byte aligned.  M = 0
 * or N = 0 is a no-op.  Errors as for lpgemm_i8_dequant; inf/NaN inputs are
 * outside the contract. */
lpgemm_status lpgemm_w8a8_fused(int64_t M, int64_t N, int64_t K, const void *X, const int8_t *W,
                                const float *w_scale, float *C, hipStream_t stream);

/* Largest K of lpgemm_quantize_rows_f16 (byte offsets within a row of X then
 * fit easily in the 32-bit offsets the kernels use). */
#define LPGEMM_MAX_K_QUANT 1048576

/* Per-row int8 quantisation of fp16 activations, the step in front of a W8A8
 * projection that lpgemm_i8_dequant then computes (the PTX-vs-WMMA summary
 * page's closing advice on quantised LLM inference; the pages leave the
 * quantisation rule open, and this is its plainest form):
 *   row_scale[i] = max_k |X[i][k]| / 127, in binary32;
 *   Q[i][k] = the nearest-even integer to X[i][k] / row_scale[i], in binary32,
 *             clamped to [-127, 127];  an all-zero row gets scale 0 and Q 0.
 * X: M x K binary16, row-major; Q: M x K int8; row_scale: M floats.
 * K must be a multiple of 8 and at most LPGEMM_MAX_K_QUANT.  X and Q must be
 * 16-byte aligned, row_scale 4-byte aligned; X and Q may be NULL when K = 0.
 * M = 0 is a no-op.  Errors as for the GEMM entry points; inf/NaN inputs are
 * outside the contract. */
lpgemm_status lpgemm_quantize_rows_f16(int64_t M, int64_t K, const void *X, int8_t *Q,
                                       float *row_scale, hipStream_t stream);

/* Static text for a status code ("unknown status" for other values). */
const char *lpgemm_status_string(lpgemm_status status);

/* Library version, major * 10000 + minor * 100 + patch. */
int lpgemm_version(void);

/* Ablation hook (the PTX-vs-WMMA summary page varies one kernel knob at a
 * time around its best kernel; this makes the same walk possible here).
 * lpgemm_config_count() is the number of kernel configurations the GEMM
 * entry points know.  lpgemm_force_config(c) pins configuration c
 * (0 <= c < lpgemm_config_count()) for every later GEMM call in the process,
 * or restores the automatic choice per shape for any other value (-1); it
 * returns the previous setting (-1 = automatic).  A configuration that an
 * entry point cannot run (for instance one without 128-byte stage rows for
 * lpgemm_i4_e3m2) leaves that entry point on its automatic choice.  The
 * environment variable LPGEMM_FORCE_CONFIG sets the initial value when the
 * library loads.  The setting is process-wide and not synchronised with
 * calls in flight on other host threads; results do not depend on it (every
 * configuration computes the same C), only the speed does. */
int lpgemm_config_count(void);
int lpgemm_force_config(int config);

/* The configuration the automatic choice per shape takes (whatever
 * lpgemm_force_config has pinned) for an M x N x K product on a device with
 * `cu_count` compute units, through the entry points without a workspace:
 * kind 0 lpgemm_i8, 1 lpgemm_i4, 2 lpgemm_f16, 3 lpgemm_i8_dequant.  Host
 * arithmetic only; no device is needed.  Returns -1 for another kind,
 * cu_count < 1, M or N <= 0 (nothing is launched), K < 0 or sizes above
 * 2^31 - 1.  The rules behind the choice are measured ones (the
 * PTX-vs-WMMA summary page's one-knob method, applied per shape), so the
 * value can change between library versions. */
int lpgemm_auto_config(int kind, int64_t M, int64_t N, int64_t K, int cu_count);

#ifdef __cplusplus
}
#endif

#endif /* LPGEMM_H */
