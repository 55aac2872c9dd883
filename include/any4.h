/*
 * any4.h -- C ABI of libany4.so, the MI355X (gfx950) any4 dequantize-GEMM
 * (with plain int4, the any2 and any3 variants and the any4 quantiser).
 *
 * any4 (the 10100.com any4 explainer, section 二) stores each weight of a
 * row as a 4-bit index into that row's 16-entry bf16 lookup table; each
 * contiguous group of g weights of a row also has a scale alpha and an offset
 * beta (step 1, "分组缩放": g = 128 typical, accuracy holds to g = 1024).  A
 * weight is w = alpha * LUT_row[idx] + beta.  The matmul y = x * W^T runs at
 * the decode batch sizes M = 1..16 that the same page's section 三 targets.
 *
 * Conventions shared by every call
 *   - All data pointers are DEVICE pointers owned by the caller.  The library
 *     allocates nothing, keeps no global state and may be called from several
 *     host threads.  Buffers must stay alive until the work on `stream`
 *     completes.
 *   - bf16 values travel as uint16_t bit patterns.  Dense row-major arrays:
 *         idx     [N][K]    uint8, values 0..15 (only the low 4 bits are read)
 *         lut     [N][16]   bf16, lut[n][i] is the value of index i in row n
 *         alpha   [N][K/g]  bf16, scale of weights k in [j*g, (j+1)*g) of row n
 *         beta    [N][K/g]  bf16, offset of the same group
 *         x       [M][K]    bf16 activations
 *         y       [M][N]    bf16 output
 *         w       [N][K]    bf16 dequantised weights
 *   - packed: the indices, two per byte, in tiles of 16 rows x 128 k
 *     (any4_packed_bytes(N, K) bytes; the tile layout is the library's, made
 *     so that one tile is one 16-byte load per lane of a 64-lane wave):
 *         tile (b, c) covers rows 16b..16b+15 and k 128c..128c+127 and starts
 *         at byte (b * K/128 + c) * 1024;
 *         byte 16*l + i of a tile (lane l = 0..63, i = 0..15) holds, for row
 *         n = 16b + (l % 16) and k = 128c + 32*(l / 16) + 2i,
 *             idx[n][k] in bits 0..3 and idx[n][k+1] in bits 4..7;
 *         rows n >= N (the last block when N % 16 != 0) are zero bytes.
 *     Equivalently: take the row-major nibble packing P[n][j] = idx[n][2j] |
 *     idx[n][2j+1] << 4, pad N up to a multiple of 16 with zero rows, view it
 *     as [N/16][16][K/128][4][16] and store it transposed to
 *     [N/16][K/128][4][16][16].
 *   - Calls are asynchronous on `stream` (0 = the default stream).  They
 *     return before the GPU work finishes; device faults show up at the
 *     caller's next synchronisation.
 *   - Arguments are checked before anything is launched.  On any error
 *     nothing is launched and every output is left untouched.
 *   - Outputs must not overlap inputs.  They are fully overwritten (no
 *     accumulate mode).
 *   - K must be a multiple of 128.  Group size: g must be a positive multiple
 *     of 128 that divides K (g = 128 .. 1024 are the sizes tested).  Every
 *     buffer must be smaller than 2 GiB.
 *   - Alignment: x, idx, packed and w need 16-byte aligned base pointers;
 *     lut needs 16 bytes for any4_gemm and 2 for any4_dequant; alpha, beta and
 *     y need 2 bytes, except that any4_gemm reads alpha and beta with 16-byte
 *     loads and needs them 16-byte aligned.
 */
#ifndef ANY4_H
#define ANY4_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum any4_status {
    ANY4_OK = 0,
    ANY4_E_NULL = 1,      /* a required pointer is NULL                               */
    ANY4_E_SHAPE = 2,     /* a size is negative, K is not a multiple of 128, g is not a
                             positive multiple of 128, K % g != 0, K/g > 512 or M > 65535*64 (any4_gemm*),
                             or a buffer would be 2 GiB or larger                     */
    ANY4_E_ALIGN = 3,     /* a base pointer misses the alignment stated above          */
    ANY4_E_WORKSPACE = 4, /* workspace smaller than any4_gemm_workspace_size()         */
    ANY4_E_HIP = 5        /* the HIP runtime refused a query or a launch               */
} any4_status;

/*
 * any4_packed_bytes -- size in bytes of the packed tiles of an N x K weight
 * matrix: ceil(N/16) * 16 * K/2.  Returns 0 when N < 0, K < 0 or K % 128 != 0.
 */
size_t any4_packed_bytes(int64_t N, int64_t K);

/*
 * any4_pack -- pack 4-bit indices two per byte into the tile layout above.
 * The offline step before inference, the counterpart of the "weights laid out
 * ahead of time" that the explainer's section 三 describes for its kernel.
 *   idx     device, [N][K] uint8, read-only; bits 4..7 of each byte are ignored.
 *   packed  device, any4_packed_bytes(N, K) bytes, written (padding included).
 *   N, K    N >= 0, K >= 0, K % 128 == 0.  N*K == 0 is a no-op.
 * Errors: ANY4_E_SHAPE, ANY4_E_NULL, ANY4_E_ALIGN (idx or packed not 16-byte
 * aligned), ANY4_E_HIP.
 */
any4_status any4_pack(const uint8_t* idx, uint8_t* packed, int64_t N, int64_t K,
                      hipStream_t stream);

/*
 * any4_dequant -- materialise the bf16 weights (the explainer, section 二:
 * a lookup in the row's table; step 1: group scale and offset):
 *     w[n][k] = bf16_rne( fp32( alpha[n][k/g] * lut[n][idx[n][k]] + beta[n][k/g] ) )
 * The bf16 x bf16 product is exact in fp32, so the inner value is one fp32
 * rounding (nearest even) of the exact sum; the result is then rounded to bf16
 * (nearest even).  Bit-exact: there is one correct answer.
 *   packed, lut, alpha, beta  device, read-only, layouts above.
 *   w                         device, [N][K] bf16, written.
 *   N >= 0, K >= 0, g as above.  N*K == 0 is a no-op.
 * Errors: ANY4_E_SHAPE, ANY4_E_NULL, ANY4_E_ALIGN, ANY4_E_HIP.
 */
any4_status any4_dequant(const uint8_t* packed, const uint16_t* lut, const uint16_t* alpha,
                         const uint16_t* beta, uint16_t* w, int64_t N, int64_t K, int64_t g,
                         hipStream_t stream);

/*
 * any4_gemm_workspace_size -- bytes of device workspace with which any4_gemm
 * may split K over several workgroups for this shape, or 0 when it does not
 * split.  It splits when the weights give each CU one or two 16-row blocks
 * (N/16 between 256 and 512 on the 256 CUs of an MI355X), K is at least
 * 12288, and the x rows the kernel loads (M rounded up to 1, 2, 4, 8 or 16)
 * exceed four per block of a CU (M = 5..16 with one block, M = 9..16 with
 * two): then x, which every workgroup reads for its whole K, would cost more
 * than the weights.  The workspace then holds S*M*N fp32
 * partial sums (S = 4 / blocks per CU), added up in a fixed order.  For
 * M >= 128 (prefill) it is N*K*2 bytes: room for the dequantised layer (see
 * any4_gemm).  Other shapes, and invalid ones, give 0.
 */
size_t any4_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int64_t g);

/*
 * any4_gemm -- y = x * W^T with W the any4 weights above.  Built for the
 * decode batches M = 1..16 of the explainer's section 三 (weights streamed
 * once, decoded in registers); larger M (prefill) also works: up to 48 rows
 * with the weights still streamed once (two or three 16-row slices of x per
 * decoded tile; for a few shapes, 16-row slices of x and y that each stream
 * the weights), beyond that a tiled matrix-core product over weight tiles
 * dequantised in on-chip memory.  From M = 128 on, given a workspace of
 * any4_gemm_workspace_size bytes, the layer is instead dequantised into the
 * workspace (the any4_dequant values exactly, w[n][k] at element n*K + k) and
 * y is one bf16 GEMM with fp32 accumulation from hipBLASLt (the library's
 * summation order; the bound below holds with its fp32 summation error);
 * should the library decline, the tiled kernel runs.  (That path uses the
 * library handle of the calling thread's current device: `stream` must belong
 * to it.)
 *     y[m][n] = bf16_rne( sum_k x[m][k] * w[n][k] )
 * Otherwise every weight is dequantised inside the kernel (the weights are
 * never written to memory) as bf16_rne(fp32(alpha * v + beta)), v the table value
 * as the kernel holds it: each table row is kept as f16 scaled by 2^-s, s
 * chosen so that the row's largest finite magnitude lies in [2^14, 2^15)
 * (and s >= -60).  A table value is therefore held exactly -- and w[n][k] is
 * exactly the any4_dequant value -- when it is 0, inf, NaN, or its binary
 * exponent is at least both (that of the row's largest finite magnitude) - 31
 * and -77.  Any other value v of the row (more than 2^31 below the row's
 * largest, or a bf16 subnormal) is rounded to the f16 grid of the scaled row,
 * an error of at most 2^(s-25) (values below that become 0).
 * The products are exact and the sum is fp32 (matrix-core accumulation), so,
 * for tables whose values are all held exactly, y differs from the fp64
 * product y_ref over the any4_dequant weights by the fp32 summation error and
 * y's own rounding to bf16 (at most 2^-8 * |y|); that is within
 *     |y - y_ref| <= 2e-3 * sum_k |x[m][k] * w[n][k]| + 1e-3
 * whenever |y| <= sum_k |x[m][k] * w[n][k]| / 2 (sums with cancellation, as
 * for activations and weights of both signs).  With values not held exactly,
 * each such weight adds at most |alpha| * 2^(s-25) to that error: negligible
 * where a row's small values are small in absolute terms (1.0 beside 2^-40 or
 * subnormals), not where a row's other values are needed beside a value
 * 2^39 times larger.  Runs are deterministic (same inputs, same bits): the
 * summation order depends only on the shape (on the prefill path, the
 * library GEMM's order, which this library does not control: its algorithm
 * is picked once per shape and process by timing the library's candidates
 * on the first eager call, so two processes may round differently;
 * environment ANY4_BLAS_TUNE=0 keeps the library's first choice).
 *   x                         device, [M][K] bf16, read-only.
 *   packed, lut, alpha, beta  device, read-only.
 *   y                         device, [M][N] bf16, written.
 *   M >= 0 (at most 65535*64), N >= 0, K >= 0 with K % g == 0 and K/g <= 512.
 *   M*N == 0 is a no-op; K == 0 writes y = 0 (x, packed, lut, alpha and beta
 *   may then be NULL).
 *   workspace, workspace_bytes  optional device scratch, 16-byte aligned,
 *       owned by the caller, contents need not be initialised.  With at least
 *       any4_gemm_workspace_size(M, N, K, g) bytes the call may split K over
 *       workgroups (a second kernel then adds the partial sums in split order,
 *       so results stay deterministic) or, for M >= 128, dequantise the layer
 *       into it; with NULL it uses kernels that need no scratch (same result
 *       bound, another summation order).  Calls that share one workspace
 *       must be ordered (e.g. one stream).
 * Errors: ANY4_E_SHAPE, ANY4_E_NULL, ANY4_E_ALIGN (also a misaligned
 * workspace), ANY4_E_WORKSPACE (a non-NULL workspace smaller than
 * any4_gemm_workspace_size), ANY4_E_HIP.
 */
any4_status any4_gemm(const uint16_t* x, const uint8_t* packed, const uint16_t* lut,
                      const uint16_t* alpha, const uint16_t* beta, uint16_t* y, int64_t M,
                      int64_t N, int64_t K, int64_t g, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/*
 * any4_gemm_noalloc -- any4_gemm for callers that cannot allocate device
 * memory (code under HIP graph capture, serving loops that must not call the
 * allocator, harnesses that forbid it): the same arguments without the
 * workspace, the same kernels and the same result, bit for bit, as any4_gemm
 * given a workspace of any4_gemm_workspace_size(M, N, K, g) bytes for
 * M <= 16 (for larger M: as any4_gemm with no workspace).  Where that size
 * is not 0 (K split over workgroups), the partial sums go to a
 * 4 MiB array of device memory inside the library, one per GPU, held until
 * the process ends; its device address is looked up on the first such call
 * on each GPU (with that GPU current: `stream` must belong to the current
 * device).  Nothing is allocated per call and nothing needs clearing (every
 * partial sum is written before it is read).  Calls on one GPU that use the
 * array and can overlap in time (other streams, other threads) race on it:
 * order them, e.g. on one stream.
 * Errors: as any4_gemm; ANY4_E_WORKSPACE if the shape would need more than
 * the array's 4 MiB (the splitting shapes need at most 1 MiB); ANY4_E_HIP if
 * the array's address cannot be looked up.
 */
any4_status any4_gemm_noalloc(const uint16_t* x, const uint8_t* packed, const uint16_t* lut,
                              const uint16_t* alpha, const uint16_t* beta, uint16_t* y,
                              int64_t M, int64_t N, int64_t K, int64_t g, hipStream_t stream);

/*
 * any4_gemv_dot -- the M = 1 product (y = x * W^T with one row of x) computed
 * on the vector ALUs with v_dot2_f32_bf16 instead of the matrix cores: the
 * GEMV form of the decode-batch product (the explainer's section 三, batch
 * 1), kept beside any4_gemm to compare the two; any4_gemm is the faster and
 * is what any4_gemm uses at M = 1.  Same decode and dequantisation as
 * any4_gemm (so the same exactness condition and bound), x [1][K], y [1][N].
 * Shapes whose x does not fit the kernel's on-chip staging (2*K bytes above
 * 64 KiB with the weights' tables) return ANY4_E_SHAPE.
 * Errors: ANY4_E_SHAPE, ANY4_E_NULL, ANY4_E_ALIGN, ANY4_E_HIP.
 */
any4_status any4_gemv_dot(const uint16_t* x, const uint8_t* packed, const uint16_t* lut,
                          const uint16_t* alpha, const uint16_t* beta, uint16_t* y, int64_t N,
                          int64_t K, int64_t g, hipStream_t stream);

/*
 * any4_gemm_int4 -- the same product for plain asymmetric int4 weights, the
 * baseline the explainer compares any4 against (section 二: int4 is the fixed
 * table 0..15, with the group scale and offset of step 1):
 *     w[n][k] = bf16_rne( fp32( alpha[n][k/g] * q[n][k] + beta[n][k/g] ) )
 *     y[m][n] = bf16_rne( sum_k x[m][k] * w[n][k] )
 * q[n][k] is the 4-bit code in `packed` (same tile layout), read as 0..15.
 * The result is bit-identical to any4_gemm with every table row 0, 1, .., 15
 * and the same workspace (given or NULL), and carries the same error bound.
 * Arguments, sizes, alignment, workspace and errors as any4_gemm, without
 * lut.
 */
any4_status any4_gemm_int4(const uint16_t* x, const uint8_t* packed, const uint16_t* alpha,
                           const uint16_t* beta, uint16_t* y, int64_t M, int64_t N, int64_t K,
                           int64_t g, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * any2 -- the 2-bit variant at 2 bits per stored weight (the paper's abstract
 * names any2): each weight is a 2-bit code into its row's table, of which
 * only entries 0..3 are read (a [N][16] bf16 table as everywhere else, e.g.
 * any4_quantize with bits = 2; entries 4..15 are ignored).  Codes are packed
 * four to a byte in tiles of 16 rows x 128 k (any2_packed_bytes(N, K)
 * bytes):
 *     tile (b, c) covers rows 16b..16b+15 and k 128c..128c+127 and starts at
 *     byte (b * K/128 + c) * 512;
 *     byte 8*l + i of a tile (lane l = 0..63, i = 0..7) holds, for row
 *     n = 16b + (l % 16) and k = 128c + 32*(l / 16) + 4i,
 *         code[n][k+s] in bits 2s..2s+1 (s = 0..3);
 *     rows n >= N are zero bytes.
 * Equivalently: row-major bytes P[n][j] = sum_s code[n][4j+s] << 2s, padded to
 * a multiple of 16 rows, viewed as [N/16][16][K/128][4][8] and stored as
 * [N/16][K/128][4][16][8].
 * any2_pack, any2_dequant and any2_gemm take the same arguments and follow
 * the same conventions, checks and errors as any4_pack, any4_dequant and
 * any4_gemm (the same optional workspace, sized by
 * any4_gemm_workspace_size), with idx read as codes 0..3 (bits above 1
 * ignored):
 *     w[n][k] = bf16_rne( fp32( alpha[n][k/g] * lut[n][code[n][k]] + beta[n][k/g] ) )
 *     y[m][n] = bf16_rne( sum_k x[m][k] * w[n][k] )   (same bound as any4_gemm)
 * Returns of any2_packed_bytes: ceil(N/16) * 16 * K/4, or 0 as any4_packed_bytes.
 */
size_t any2_packed_bytes(int64_t N, int64_t K);
any4_status any2_pack(const uint8_t* idx, uint8_t* packed, int64_t N, int64_t K,
                      hipStream_t stream);
any4_status any2_dequant(const uint8_t* packed, const uint16_t* lut, const uint16_t* alpha,
                         const uint16_t* beta, uint16_t* w, int64_t N, int64_t K, int64_t g,
                         hipStream_t stream);
any4_status any2_gemm(const uint16_t* x, const uint8_t* packed, const uint16_t* lut,
                      const uint16_t* alpha, const uint16_t* beta, uint16_t* y, int64_t M,
                      int64_t N, int64_t K, int64_t g, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/*
 * any3 -- the 3-bit variant at 3 bits per stored weight (the paper's abstract
 * names any3): each weight is a 3-bit code into its row's table, of which
 * only entries 0..7 are read (entries 8..15 are ignored; any4_quantize with
 * bits = 3 writes such tables).  Codes are stored in tiles of 16 rows x 128 k
 * (any3_packed_bytes(N, K) bytes):
 *     tile (b, c) covers rows 16b..16b+15 and k 128c..128c+127 and starts at
 *     byte (b * K/128 + c) * 768;
 *     the 12 bytes 12*l .. 12*l+11 of a tile (lane l = 0..63) hold row
 *     n = 16b + (l % 16), k = 128c + 32*(l / 16) + 0..31, as 16 pair indices
 *         P_i = code[n][k+2i] | code[n][k+2i+1] << 3      (i = 0..15);
 *     byte j (j = 0..11) holds P_j in bits 0-5, and in bits 6-7 the two bits
 *     2*(j/4), 2*(j/4)+1 of P_{12 + j%4};
 *     rows n >= N are zero bytes.
 * (So dwords 0-2 of a lane's 12 bytes carry the pair indices of its first
 * three 32-k MFMA operands one per byte, and the fourth operand's are
 * gathered from the bytes' top bits: one load of 12 bytes per lane.)
 * any3_pack, any3_dequant and any3_gemm take the same arguments and follow
 * the same conventions, checks and errors as any2_pack, any2_dequant and
 * any2_gemm, with idx read as codes 0..7 (bits above 2 ignored):
 *     w[n][k] = bf16_rne( fp32( alpha[n][k/g] * lut[n][code[n][k]] + beta[n][k/g] ) )
 *     y[m][n] = bf16_rne( sum_k x[m][k] * w[n][k] )   (same bound as any4_gemm)
 * Returns of any3_packed_bytes: ceil(N/16) * 16 * 3K/8, or 0 as any4_packed_bytes.
 */
size_t any3_packed_bytes(int64_t N, int64_t K);
any4_status any3_pack(const uint8_t* idx, uint8_t* packed, int64_t N, int64_t K,
                      hipStream_t stream);
any4_status any3_dequant(const uint8_t* packed, const uint16_t* lut, const uint16_t* alpha,
                         const uint16_t* beta, uint16_t* w, int64_t N, int64_t K, int64_t g,
                         hipStream_t stream);
any4_status any3_gemm(const uint16_t* x, const uint8_t* packed, const uint16_t* lut,
                      const uint16_t* alpha, const uint16_t* beta, uint16_t* y, int64_t M,
                      int64_t N, int64_t K, int64_t g, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/*
 * any4_quantize -- the any4 quantiser: turns weights into the idx, lut, alpha
 * and beta arrays above (the explainer, section 二: step 1, group scaling and
 * the calibration statistic E|x|; step 2, the E-step / M-step iteration that
 * learns each row's 16 table values, weighting each weight by alpha * E|x|).
 * bits = 3 or 2 gives any3 / any2 (the paper's abstract): Q = 8 or 4 table
 * values instead of Q = 16, stored in the first Q entries of the 16-entry
 * row (the rest zero), indices 0..Q-1, so such layers run through any4_pack,
 * any4_dequant and any4_gemm unchanged (at 4 bits per stored index).
 * Per row, in binary64 and in this order:
 *   1. per group of g weights: beta = bf16(min), alpha = bf16((max - min) /
 *      (Q - 1)) (the asymmetric range mapping that makes the start table
 *      0..Q-1 the plain uniform grid);
 *   2. ws = (w - beta) / alpha (0 where alpha == 0), wt = alpha * ex[k];
 *   3. L = 0, 1, .., Q-1, then `iters` rounds of: assign every weight to its
 *      nearest table value (ties: the lower index), then
 *      L[q] = sum(wt * ws) / sum(wt) over the members of q, summed in
 *      increasing k with products and sums rounded separately; a cluster
 *      without members keeps its value;
 *   4. lut = bf16(L), and idx = the nearest stored value for every weight.
 * The result is a deterministic function of the inputs.  One GPU thread
 * works through one row (the sums must run in k order), so this is an
 * offline step: milliseconds per layer.
 *   W      device, [N][K] fp32, read-only.
 *   ex     device, [K] fp32, E|x| of each input channel, read-only.
 *   idx    device, [N][K] uint8 (values 0..15), written; pack it with any4_pack.
 *   lut    device, [N][16] bf16, written.
 *   alpha, beta  device, [N][K/g] bf16, written.
 *   N >= 0, K >= 0, g > 0 with K % g == 0, iters >= 0, bits in 2..4,
 *   N*K < 2^31.  N*K == 0 is a no-op.
 * Errors: ANY4_E_SHAPE, ANY4_E_NULL, ANY4_E_ALIGN (W or ex not 4-byte aligned,
 * lut, alpha or beta not 2-byte aligned), ANY4_E_HIP.
 */
any4_status any4_quantize(const float* W, const float* ex, uint8_t* idx, uint16_t* lut,
                          uint16_t* alpha, uint16_t* beta, int64_t N, int64_t K, int64_t g,
                          int iters, int bits, hipStream_t stream);

/*
 * any4_read_probe -- a measurement aid, not part of the method: reads `bytes`
 * of device memory at `buf` once, with the GEMM kernels' loads (16 bytes per
 * lane, 1 KB per wave, non-temporal), one workgroup of 16 waves per CU, each
 * wave issuing its ceil(bytes / 4 MiB) loads (at most 16 at a time) at once,
 * and writes at most one word to `out`.  Its duration is the streaming-read
 * ceiling that the GEMM's bandwidth is compared with.  bytes: a multiple of
 * 1024, below 2 GiB (0: no-op).
 * Errors: ANY4_E_SHAPE, ANY4_E_NULL, ANY4_E_ALIGN (buf not 16-byte or out
 * not 4-byte aligned), ANY4_E_HIP.
 */
any4_status any4_read_probe(const void* buf, size_t bytes, uint32_t* out, hipStream_t stream);

/* A static, human-readable name for a status code (never NULL). */
const char* any4_status_string(any4_status s);

#ifdef __cplusplus
}
#endif

#endif /* ANY4_H */
