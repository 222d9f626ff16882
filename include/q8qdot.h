/*
 * q8qdot -- Q8_0 block-quantized contraction on AMD Instinct MI355X (gfx950).
 *
 * The operation ("Phobos Language Spec", section "Quantized built-ins",
 * Q8_0 table, row qdot_t; restated in "Quantized built-ins and formats",
 * section "Q8_0"):
 *
 *     C[i, j] = sum over blocks b of  AS[i, b] * WS[j, b] * P[i, j, b]
 *     P[i, j, b] = sum over t < 32 of  A[i, 32 b + t] * W[j, 32 b + t]
 *
 * with A, W signed bytes (sign-extended, "Phobos Language Spec", section
 * "Types"), AS, WS f32 block scales, one per 32 consecutive k, and the inner
 * block sum exact in int32 (|P| <= 32 * 128^2 = 2^19).
 *
 * Operand layout (row-major, densely packed, as the "Kernel ABI" page's
 * section "Memory layout and alignment" requires of every tensor):
 *
 *     A   int8  [M][K]        activations, Q8_0 bytes
 *     AS  f32   [M][K/32]     activation block scales
 *     W   int8  [N][K]        weights, Q8_0 bytes
 *     WS  f32   [N][K/32]     weight block scales (same orientation as AS,
 *                             the qdot_t form; not the transposed qmma_t form)
 *     C   f32   [M][N]        output, assigned (never read, never accumulated)
 *     P   int32 [M][N][K/32]  per-block integer partials (debug entry)
 *
 * Conventions shared by every entry point:
 *   - Every pointer is a DEVICE pointer owned by the caller.  The library
 *     allocates nothing, keeps no per-call state, never synchronizes and
 *     never reads an output.  Work is enqueued on `stream` (a hipStream_t;
 *     NULL means the null stream) and is asynchronous like a kernel launch.
 *   - Shapes: M, N, K >= 0 and K % 32 == 0.  M or N == 0 is an empty
 *     output: OK, nothing is launched and pointers are not inspected.
 *     K == 0 with M, N > 0 is the empty sum: C is filled with 0.0f and A,
 *     AS, W, WS may be NULL.  M and N need not be multiples of any tile:
 *     ragged edges are masked inside the kernels (the pages instead ask for
 *     whole tiles, "Kernel ABI", section "Entry checks").
 *   - Alignment: A, W (and Q of q8_quantize) must be 16-byte aligned, so
 *     every row (a multiple of 32 bytes long) can be read with 16-byte
 *     loads; the f32/int32 arrays must be 4-byte aligned.
 *   - Errors are detected on the host and returned BEFORE anything is
 *     enqueued (the pages instead trap at kernel entry and leave the context
 *     unusable, "Kernel ABI", section "Entry checks").  A size larger than a
 *     buffer cannot be detected and reads or writes past it, as on the pages.
 *     A fault inside a kernel surfaces at the caller's next synchronize.
 *   - Calls are reentrant; calls on different streams may overlap.
 *   - Numerics: int32 block sums are exact; C is within
 *     1e-5 * sum_b |AS * WS * P| + 1e-6 of the exact sum for finite inputs
 *     whose per-block products AS[i, b] * WS[j, b] and partial sums are
 *     finite in f32.  The M >= 8 kernels use a 2-operation epilogue whose
 *     bias product is finite for |WS| below about 2^104; a tile whose result
 *     comes out non-finite is recomputed in the plain order (AS * WS) * P,
 *     so any finite scales work.  That epilogue drops the two lowest
 *     mantissa bits of each weight scale: at most 3.6e-7 relative for a
 *     normal scale; for a subnormal one (below 2^-126) at most
 *     3 * 2^-149 * |AS * P| per block, below the absolute term of the bound
 *     unless |AS| exceeds about 10^26.
 */
#ifndef Q8QDOT_H
#define Q8QDOT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    Q8_OK = 0,
    Q8_EINVAL = -1,  /* M, N or K negative, or K % 32 != 0 */
    Q8_ENULL = -2,   /* a pointer the call must dereference is NULL */
    Q8_EALIGN = -3,  /* A/W/X/Q not 16-byte aligned, or W5 or another array not 4-byte aligned */
    Q8_ELAUNCH = -4, /* the HIP runtime rejected the launch (hipGetLastError) */
    Q8_ERANGE = -5   /* an extent product overflows 64-bit byte addressing, or
                        M >= 8 with 32 * K > 2^31 - 1 (32-bit tile offsets), or
                        q8_qmma with M >= 8 and (K/32) * N * 4 > 2^31 - 1, or
                        q8_qdot_noalloc on a shape whose split form needs
                        more than its static scratch */
} q8_status;

/*
 * C = qdot_t(A, AS, W, WS) on the null stream.  Dispatches on M like
 * q8_qdot_path.  Returns a q8_status.
 */
int q8_qdot(const int8_t *A, const float *AS, const int8_t *W, const float *WS,
            float *C, int M, int N, int K);

/* The same on an explicit HIP stream (hipStream_t passed as void*). */
int q8_qdot_stream(const int8_t *A, const float *AS, const int8_t *W, const float *WS,
                   float *C, int M, int N, int K, void *stream);

/*
 * C = qmma_t(A, AS, W, WST): the same sum with the weight scales stored
 * transposed ("Phobos Language Spec", section "Quantized built-ins", Q8_0
 * table, row qmma_t; "Quantized built-ins and formats", section "Q8_0"):
 *
 *     C[i, j] = sum over blocks b of  AS[i, b] * WST[b, j] * P[i, j, b]
 *
 *     WST  f32  [K/32][N]   weight block scales, block-major
 *
 * Everything else (A, AS, W, C, conventions, errors) as for q8_qdot_stream.
 * The pages ask for M and N multiples of 8 here; this library accepts any
 * M, N >= 0.  For M >= 8, (K/32) * N * 4 must be below 2^31 (32-bit offsets
 * into WST), else Q8_ERANGE.  The int32 partials do not involve the scales:
 * q8_qdot_partials serves both forms.
 */
int q8_qmma(const int8_t *A, const float *AS, const int8_t *W, const float *WST,
            float *C, int M, int N, int K, void *stream);

/*
 * Q5_0 weights ("Phobos Language Spec", section "Quantized built-ins", Q8_0
 * table, rows q50_qdot_t and q50_qmma_t; "Quantized built-ins and formats",
 * section "Q8_0"): the same contraction against a weight held as Q5_0 blocks
 * without their scale.
 *
 *     W5  uint8 [N][K/32 * 20]  per 32 values: the qh word (4 bytes,
 *                               little-endian), then 16 bytes; byte e holds
 *                               element e in its low nibble and element e+16
 *                               in its high nibble; the element is q - 16,
 *                               q = nibble + 16 * (bit e of qh)
 *
 * (The bit of qh that belongs to element e is not stated on the pages; this
 * library reads it as bit e of the little-endian word.)  W5 must be 4-byte
 * aligned; A 16-byte; AS, WS/WST, C, P 4-byte.  Scales as for q8_qdot_stream
 * (q8_q50_qdot: WS [N][K/32]) and q8_qmma (q8_q50_qmma: WST [K/32][N]).
 * M < 8 with K <= 16384 runs the Q5_0 matvec: a batch of 2..7 activation
 * rows that fits in LDS beside the weight staging areas (up to 7 rows of
 * K <= 8192, 6 of 12288, 5 of 14336, 4 of 16384) is taken in one pass that
 * reads the weights once, larger ones one activation row per pass
 * (q8_q50_partials: always one row per pass).  Anything else runs an MFMA
 * GEMM (for which 32 * K, and with WST (K/32) * N * 4, must be below 2^31,
 * else Q8_ERANGE): the 64 x 64-tile ring GEMM, decoding each stage's blocks
 * once in LDS, for shapes whose Q8_0 dispatch (q8_qdot_path) is 2 or 3 and
 * that have more 64 x 64 output tiles than the GPU has compute units, when
 * K/32 is a multiple of 4 and W5 is 16-byte aligned; else the K-split GEMM.
 * q8_q50_path reports which.  q8_q50_partials: P[i][j][b] =
 * sum over the block of A * (q - 16), int32 [M][N][K/32].
 */
int q8_q50_qdot(const int8_t *A, const float *AS, const uint8_t *W5, const float *WS,
                float *C, int M, int N, int K, void *stream);
int q8_q50_qmma(const int8_t *A, const float *AS, const uint8_t *W5, const float *WST,
                float *C, int M, int N, int K, void *stream);
int q8_q50_partials(const int8_t *A, const uint8_t *W5, int32_t *P, int M, int N, int K,
                    void *stream);

/*
 * The kernel the Q5_0 entries take for a shape, with a 16-byte aligned W5:
 * 0 = Q5_0 matvec, 1 = K-split MFMA GEMM, 3 = 64 x 64-tile ring GEMM (as
 * described above; a W5 that is only 4-byte aligned takes 1 instead of 3).
 * Q8_EINVAL for bad shapes.
 */
int q8_q50_path(int M, int N, int K);

/*
 * Debug entry: P[i][j][b] = the int32 block sum of the qdot_t definition,
 * int32 [M][N][K/32] row-major.  Runs the kernel q8_qdot runs for this
 * (M, N, K), with the same loads, the same integer-dot instructions and (in
 * the GEMMs) the same software-pipelined loop and accumulator seed, and
 * stores each block sum where q8_qdot applies the f32 block scales, so each
 * kernel's integer core can be checked bit for bit.  K == 0 is an empty P:
 * OK, nothing is launched.
 */
int q8_qdot_partials(const int8_t *A, const int8_t *W, int32_t *P,
                     int M, int N, int K, void *stream);

/*
 * The same contractions with a caller workspace (qdot_t / qmma_t as for
 * q8_qdot_stream and q8_qmma; "Phobos Language Spec", section "Quantized
 * built-ins", Q8_0 table).  For M >= 8 shapes with K >= 8192 whose 64 x 64
 * output tiles are too few to occupy the GPU (for example M = 32, N = 4096,
 * K = 14336), the contraction is split into slices of K/32 blocks across
 * workgroups; each writes its
 * partial f32 tile to the workspace and the last of a tile's workgroups to
 * finish adds the partial tiles in slice order (so the result does not
 * depend on the order in which they finish) and stores C.
 *
 *   q8_qdot_ws_size: *bytes = the workspace the split form needs for this
 *     shape on the current device, or 0 when the shape does not take it.
 *     Q8_ENULL if bytes is NULL; shape errors as for q8_qdot.
 *   q8_qdot_ws / q8_qmma_ws: workspace is a device pointer owned by the
 *     caller, 16-byte aligned, of ws_bytes bytes.  Its first 4096 bytes hold
 *     one counter per output tile and must be ZERO-FILLED before the first
 *     use; the kernel resets every counter it used, so they are zero again
 *     after each call, and one workspace serves calls of any shape in turn.
 *     The rest holds partial tiles (no initial value needed).  With a
 *     workspace of at least q8_qdot_ws_size bytes the shape takes the split
 *     form; with less (or NULL) the call is exactly q8_qdot_stream /
 *     q8_qmma.  Calls that share a workspace must not overlap (use one
 *     workspace per stream).  Everything else as for q8_qdot_stream /
 *     q8_qmma.
 *   q8_qdot_ws_partials: the int32 block sums of the kernel q8_qdot_ws runs
 *     for this shape (given a sufficient workspace), as q8_qdot_partials
 *     describes; it needs no workspace.
 */
int q8_qdot_ws_size(int M, int N, int K, size_t *bytes);
int q8_qdot_ws(const int8_t *A, const float *AS, const int8_t *W, const float *WS,
               float *C, int M, int N, int K, void *workspace, size_t ws_bytes, void *stream);
int q8_qmma_ws(const int8_t *A, const float *AS, const int8_t *W, const float *WST,
               float *C, int M, int N, int K, void *workspace, size_t ws_bytes, void *stream);
int q8_qdot_ws_partials(const int8_t *A, const int8_t *W, int32_t *P, int M, int N, int K,
                        void *stream);

/*
 * For callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid allocation): q8_qdot_ws without
 * a workspace argument.  Where q8_qdot_ws would split the contraction, the
 * workspace is a static device array inside the library (one per GPU, alive
 * until the process ends): 4 MiB of partial tiles plus 8 KiB of tile
 * counters, enough for every shape on a GPU of up to 256 compute units; a
 * shape that would need more returns Q8_ERANGE (nothing is enqueued).  Every
 * other shape runs exactly q8_qdot_stream.  The call allocates nothing and
 * needs no set-up; it finds its counters at zero (each call resets the
 * counters it used and zero-fills those the next call will use).  All calls
 * on one GPU share the array: calls that overlap on one GPU (different
 * streams, or threads) race and may return wrong results; serialize them.
 * Arguments, layout, ownership and the other errors as for q8_qdot_stream.
 */
int q8_qdot_noalloc(const int8_t *A, const float *AS, const int8_t *W, const float *WS,
                    float *C, int M, int N, int K, void *stream);

/*
 * The kernel a shape dispatches to: 0 = wave64 matvec (M < 8: with K <=
 * 16384 the 2..7 activation rows are staged together so the weights are read
 * once; longer rows take one activation row per grid row); for M >= 8 the
 * int8-MFMA block GEMM, 1 = one workgroup per
 * 32 x 32 output tile with the K/32 blocks split across its waves (few
 * tiles: small M or N), 2 = LDS-staged 128 x 224 workgroup tiles (large M
 * and N), 3 = one workgroup per 64 x 64 output tile over all of K, staged
 * through an LDS ring (medium shapes: too few 128 x 224 tiles to fill the
 * chip, but so many 32 x 32 tiles that one workgroup per 64 x 64 tile needs
 * far fewer rounds of workgroups; also shapes with one or two rounds of
 * 128 x 224 tiles but at most about four 64 x 64 tiles per compute unit
 * per round, where two of its workgroups per unit beat the staged GEMM;
 * the kernel of q8_qdot_ws's split form, with one slice and no workspace).
 * The debug entry q8_qdot_partials takes the same kernel.  Q5_0 weights
 * take 0 or 1.  Q8_EINVAL for bad shapes.
 */
int q8_qdot_path(int M, int N, int K);

/*
 * Q8_0 quantization of f32 rows on the GPU (the step that produces A and AS
 * from an f32 activation; "Quantized built-ins and formats", section "Q8_0":
 * activations are quantized like the weights, one scale per 32 values).
 * X f32 [rows][K] -> Q int8 [rows][K], D f32 [rows][K/32].  Per block:
 * d = f32(max|x| / 127), q = clamp(round-half-even(x / d), -127, 127) with an
 * IEEE f32 division, and d == 0 gives q == 0.  (The scale and rounding rule
 * are a reading: the pages do not state how Q8_0 values are produced.)
 * Inputs must be finite.  rows == 0 or K == 0 is OK (nothing launched).
 * X and Q must be 16-byte aligned (16-byte loads of X), D 4-byte aligned.
 */
int q8_quantize(const float *X, int8_t *Q, float *D, int rows, int K, void *stream);

/* Static text for a q8_status value ("unknown status" otherwise). */
const char *q8_strerror(int status);

/* Library version, MAJOR * 10000 + MINOR * 100 + PATCH. */
int q8_version(void);

#ifdef __cplusplus
}
#endif

#endif /* Q8QDOT_H */
