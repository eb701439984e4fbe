/*
 * w4a16.h — C ABI of the MI355X (gfx950) W4A16 library: group-wise asymmetric
 * int4 weight-only GEMM with 16-bit activations, and the one-time repack of
 * AWQ-packed weights into this library's GPU tile layout.
 *
 *   y[m, n] = sum_k x[m, k] * W[k, n],   W[k, n] = (q[k, n] - z[g, n]) * s[g, n],
 *   g = k div G  (G = group size: 128 in the common case, also 32, 64 or any
 *   multiple of 128 dividing K; -1 means G = K).
 *
 * Lifecycle, after the three phases of a quantised linear layer in the vLLM
 * note "Carga de capas cuantizadas: AWQ / GPTQ / Marlin / fp8" (section
 * "Responsabilidades": create_weights builds qweight / scales / qzeros,
 * process_weights_after_loading reorders once after loading, apply runs the
 * quantised GEMM in the forward):
 *   1. the caller holds the checkpoint tensors with the shapes of section
 *      "Flujo de datos": qweight int32 [K, N/8], qzeros int32 [K/G, N/8],
 *      scales fp16/bf16 [K/G, N];
 *   2. w4a16_repack writes them once into a packed buffer of
 *      w4a16_packed_bytes(K, N, G) bytes (the caller may free the three
 *      checkpoint tensors once the stream has passed the repack);
 *   3. w4a16_gemm runs the product from the packed buffer, as often as needed.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller. The library
 *     never allocates, frees or retains them after the call returns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). Work
 *     is enqueued asynchronously on it; nothing synchronises the host. The
 *     caller keeps every buffer alive until the stream has passed the call.
 *   - Every argument is validated on the host before anything is launched; an
 *     invalid call returns its status and touches no memory.
 *   - Calls on different streams touch only the buffers they are given, so
 *     they may run concurrently when their outputs do not overlap (except
 *     w4a16_gemm_noalloc, whose calls share one library-owned array per GPU).
 *   - Status codes are returned; nothing is thrown across the ABI.
 */
#ifndef W4A16_H
#define W4A16_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enumerations below end in two range members that are not values: they give each
 * type every 32-bit integer as a valid value, so an entry point can check and reject
 * any value a caller passes without undefined behaviour in the C++ implementation. */

typedef enum {
    W4A16_OK = 0,
    W4A16_ERR_NULL = 1,         /* a required pointer is NULL                       */
    W4A16_ERR_SHAPE = 2,        /* M < 0, K or N <= 0, K % 128 != 0, N % 8 != 0,
                                   K > 2^20, N > 2^28, K*N > 2^37 or M*K > 2^32       */
    W4A16_ERR_GROUP = 3,        /* group size not -1, 32, 64 or a multiple of 128 dividing K */
    W4A16_ERR_DTYPE = 4,        /* dtype is neither W4A16_FP16 nor W4A16_BF16        */
    W4A16_ERR_ALIGN = 5,        /* a pointer is not aligned as documented            */
    W4A16_ERR_BUFFER_SIZE = 6,  /* a caller buffer is smaller than required          */
    W4A16_ERR_DEVICE = 7,       /* the current device is not a gfx950 GPU            */
    W4A16_ERR_HIP = 8,          /* the HIP runtime reported an error at launch       */
    W4A16_ERR_PATH = 9,         /* unknown path, or the forced path cannot take M    */
    W4A16_ERR_LAYOUT = 10,      /* packed header bad, or from another layout version */
    W4A16_STATUS_RANGE_MIN_ = -0x7FFFFFFF - 1,
    W4A16_STATUS_RANGE_MAX_ = 0x7FFFFFFF
} w4a16_status;

typedef enum {
    W4A16_FP16 = 0,             /* IEEE binary16 activations, scales, bias, output  */
    W4A16_BF16 = 1,             /* bfloat16 activations, scales, bias, output       */
    W4A16_DTYPE_RANGE_MIN_ = -0x7FFFFFFF - 1,
    W4A16_DTYPE_RANGE_MAX_ = 0x7FFFFFFF
} w4a16_dtype;

typedef enum {
    W4A16_PATH_AUTO = 0,        /* M <= gemv_max_m: GEMV, otherwise MFMA GEMM      */
    W4A16_PATH_GEMV = 1,        /* weight-streaming split-K GEMV, M <= 16          */
    W4A16_PATH_MFMA = 2,        /* LDS-staged dequantise -> MFMA GEMM, any M       */
    W4A16_PATH_RANGE_MIN_ = -0x7FFFFFFF - 1,
    W4A16_PATH_RANGE_MAX_ = 0x7FFFFFFF
} w4a16_path;

/* Version of the packed tile layout. A buffer written by one version must not be
 * read by another; callers that persist packed buffers store this number with them. */
int w4a16_layout_version(void);

/* Bytes of the packed buffer for a K x N weight with group size `group_size`:
 * K*Np/2 (4-bit codes) + 4*UW*Np (one 32-bit scale/zero word per column per unit
 * of min(G, 128) rows), Np = N rounded up to a multiple of 16 and UW = K/min(G, 128)
 * rounded up to a multiple of 4. N must be a multiple of 8 (the AWQ and GPTQ pack factor); with
 * N % 16 == 8 the last 16-column block carries 8 zero columns that no entry point
 * reads into a result.
 * Returns 0 if the shape or group size is not supported. */
size_t w4a16_packed_bytes(int64_t K, int64_t N, int64_t group_size);

/* One-time repack of AWQ checkpoint tensors into the packed tile layout
 * ("process_weights_after_loading" of the vLLM note: the AWQ packing order along
 * the output dimension is undone and the codes are rewritten in the layout the
 * GEMM kernels read with 128-bit loads).
 *
 *   qweight  int32 [K, N/8], row-major. Word j of row k holds the 4-bit codes of
 *            columns 8j .. 8j+7; nibble slot s (bits 4s..4s+3) holds column
 *            8j + ORDER[s], ORDER = 0,2,4,6,1,3,5,7 (the AWQ interleave).
 *   qzeros   int32 [K/G, N/8], row-major, packed exactly like qweight.
 *   scales   [K/G, N] row-major, of `dtype`.
 *   packed   output, `packed_bytes` >= w4a16_packed_bytes(K, N, group_size).
 *            Only the first w4a16_packed_bytes(...) bytes are written.
 *
 * Alignment: qweight, qzeros 4 bytes; scales 2 bytes; packed 16 bytes.
 * The result is a pure function of the inputs (bit-for-bit reproducible). */
w4a16_status w4a16_repack(const int32_t* qweight, const int32_t* qzeros, const void* scales,
                          w4a16_dtype dtype, int64_t K, int64_t N, int64_t group_size,
                          void* packed, size_t packed_bytes, void* stream);

/* The same one-time repack from GPTQ-standard tensors. GPTQ-style packing runs
 * along the input dimension in standard bit order (vLLM note "Carga de capas
 * cuantizadas", section "Motivación de diseño": the Marlin kernel takes only that
 * style, so AWQ checkpoints are converted to it first). The packed buffer written
 * is byte-for-byte the one w4a16_repack writes for the same codes, zero points and
 * scales, so every other entry point reads it unchanged.
 *
 *   qweight  int32 [K/8, N], row-major. Word i of column n holds rows 8i .. 8i+7;
 *            nibble j (bits 4j..4j+3) holds row 8i + j.
 *   qzeros   int32 [K/G, N/8], row-major, packed along N in standard order:
 *            nibble j of word w holds the zero point of column 8w + j, used as is
 *            (w = (q - z) * s; no +1 offset is applied).
 *   scales   [K/G, N] row-major, of `dtype`.
 *   packed   output, `packed_bytes` >= w4a16_packed_bytes(K, N, group_size).
 *
 * Activation-order checkpoints (a g_idx permutation of K) are not supported: groups
 * are contiguous runs of G rows. Alignment as for w4a16_repack. */
w4a16_status w4a16_repack_gptq(const int32_t* qweight, const int32_t* qzeros, const void* scales,
                               w4a16_dtype dtype, int64_t K, int64_t N, int64_t group_size,
                               void* packed, size_t packed_bytes, void* stream);

/* Column-chunked repack, to bound the device-side copy of the checkpoint tensors
 * while loading (vllm-omni commit "cpu_int4: repack weights in n-blocks, to bound
 * the load-time peak": column blocks are independent, so the expansion can cover one
 * chunk at a time; the whole-matrix transient there was 1 GiB for the tied head).
 * The tensors hold columns [n0, n0 + nc) of the K x N weight, contiguous:
 *   w4a16_repack_columns:      qweight int32 [K, nc/8], qzeros int32 [K/G, nc/8]
 *                              (AWQ order), scales [K/G, nc];
 *   w4a16_repack_gptq_columns: qweight int32 [K/8, nc], qzeros int32 [K/G, nc/8]
 *                              (standard order), scales [K/G, nc].
 * They write exactly those columns' codes and metadata into `packed`, the buffer of
 * the whole K x N weight (packed_bytes >= w4a16_packed_bytes(K, N, G)); the other
 * columns' bytes are not touched. n0 % 16 == 0, nc % 8 == 0, n0 + nc <= N, and
 * nc % 16 == 0 unless the chunk ends at N. Repacking all chunks of a partition of
 * [0, N) gives the bytes w4a16_repack writes. Alignment as for w4a16_repack. */
w4a16_status w4a16_repack_columns(const int32_t* qweight, const int32_t* qzeros, const void* scales,
                                  w4a16_dtype dtype, int64_t K, int64_t N, int64_t group_size,
                                  int64_t n0, int64_t nc, void* packed, size_t packed_bytes, void* stream);
w4a16_status w4a16_repack_gptq_columns(const int32_t* qweight, const int32_t* qzeros, const void* scales,
                                       w4a16_dtype dtype, int64_t K, int64_t N, int64_t group_size,
                                       int64_t n0, int64_t nc, void* packed, size_t packed_bytes,
                                       void* stream);

/* Persisting a packed buffer, so a later load skips the repack (the AWQ-v2 PR
 * "feat(quantization): add AWQ-v2 64KB DMA page-aligned zero-repack loader and
 * specification", sections "Overview" and "Claims": weights stored pre-swizzled in
 * the kernel's layout, with the legacy path still available). A stored buffer starts
 * with this 64-byte header, host memory:
 *   bytes 0..7 "W4A16PK\0", 8..11 layout version (w4a16_layout_version), 12..15
 *   dtype, 16..23 K, 24..31 N, 32..39 group_size, 40..47 packed bytes (all
 *   little-endian), 48..55 FNV-1a 64-bit hash of bytes 0..47, 56..63 zero.
 * w4a16_packed_header fills `header` (header_bytes >= 64) for a valid shape.
 * w4a16_parse_packed_header checks it and returns the fields; W4A16_ERR_LAYOUT if the
 * magic, the hash, the reserved bytes, the fields or the layout version disagree (a
 * buffer of another version must be repacked from the checkpoint). Host only: no
 * device is touched. */
#define W4A16_PACKED_HEADER_BYTES 64
w4a16_status w4a16_packed_header(int64_t K, int64_t N, int64_t group_size, w4a16_dtype dtype,
                                 void* header, size_t header_bytes);
w4a16_status w4a16_parse_packed_header(const void* header, size_t header_bytes, int64_t* K, int64_t* N,
                                       int64_t* group_size, w4a16_dtype* dtype, size_t* packed_bytes);

/* Device workspace the GEMM needs for this shape, in bytes (0 for most shapes).
 * It is non-zero when the MFMA GEMM splits K over workgroups because the output has
 * too few tiles to fill the GPU (small N and M, long K); the split partial sums
 * (fp32) and one counter per output tile live there. Independent of the path that
 * w4a16_gemm_ex would choose: the value suffices for every path. The GEMV uses the
 * workspace too when one this large is passed, from M = 6 on outputs of at most 128
 * column blocks (N <= 2048) with K >= 6144, to split K over workgroups, where its
 * balanced variants do not take the shape (in practice from M = 9, or with groups of
 * 32 or 64 rows); with NULL it runs one workgroup per column block (same result
 * within the tolerance, not bit for bit).
 *
 * Layout: its first 512 bytes hold the tile counters for every shape (a split plan
 * has fewer than 128 output tiles), the partial sums follow.
 *
 * Contract: the workspace must be zero-filled before its first use and is left
 * zero-filled (in its counter part) by every call, so one zeroed allocation as large
 * as the largest requirement can be reused by consecutive calls of any shapes on one
 * stream, W4A8 calls included. Calls that overlap in time (different streams) need
 * different workspaces. 16-byte alignment. */
size_t w4a16_workspace_bytes(int64_t M, int64_t K, int64_t N, int64_t group_size);

/* y = x . dequant(W) (+ bias), from a buffer written by w4a16_repack
 * ("apply(layer, x, bias)" of the vLLM note, section "Flujo de datos").
 *
 *   x        [M, K] row-major, `dtype`. 16-byte aligned.
 *   packed   the repacked weight, `packed_bytes` >= w4a16_packed_bytes(K, N, G).
 *            16-byte aligned.
 *   y        [M, N] row-major, `dtype`, written in full. 16-byte aligned. Must not
 *            overlap x, packed or bias.
 *   bias     [N] of `dtype`, or NULL. 2-byte aligned. Added in fp32 before rounding.
 *   group_size must be the value the buffer was repacked with (checked for shape
 *            validity only: the metadata of the buffer carries the groups).
 *   workspace / workspace_bytes: at least w4a16_workspace_bytes(M, K, N, group_size)
 *            bytes under the contract stated there; may be NULL / 0 when that is 0.
 *
 * Products accumulate in fp32; the output is rounded to `dtype` once, to nearest
 * even. For fixed inputs and shape the result is bit-for-bit reproducible from run
 * to run. M = 0 is a valid no-op. */
w4a16_status w4a16_gemm(const void* x, const void* packed, size_t packed_bytes, w4a16_dtype dtype,
                        void* y, int64_t M, int64_t K, int64_t N, int64_t group_size,
                        const void* bias, void* workspace, size_t workspace_bytes, void* stream);

/* w4a16_gemm with the kernel choice exposed (tests, tuning). With
 * W4A16_PATH_AUTO, M <= gemv_max_m takes the GEMV (gemv_max_m in 0..16; a
 * negative value selects the default, which w4a16_gemm uses: 8, raised to 12 when
 * the codes (K*N/2 bytes) take at most 16 MiB and to 15 at most 4 MiB or when
 * N <= 2048 and K >= 2048, and to 16 on outputs of at least 512 16-column blocks that
 * the balanced matrix-core GEMV takes at M = 16 (at most 8 half blocks per compute
 * unit), for groups of 128 rows or more, where the GEMV was measured faster up to those
 * row counts).
 * W4A16_PATH_GEMV requires M <= 16. Both paths read the same packed buffer. */
w4a16_status w4a16_gemm_ex(const void* x, const void* packed, size_t packed_bytes, w4a16_dtype dtype,
                           void* y, int64_t M, int64_t K, int64_t N, int64_t group_size,
                           const void* bias, void* workspace, size_t workspace_bytes, void* stream,
                           w4a16_path path, int64_t gemv_max_m);

/* w4a16_gemm for callers that cannot allocate: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc. It takes no workspace: the K-split
 * partial sums and tile counters that w4a16_gemm keeps in the caller's workspace live
 * in a device array of W4A16_NOALLOC_SCRATCH_BYTES owned by the library (one copy per
 * GPU, held until the process ends). The call allocates nothing, on the host or the
 * device, and returns exactly what w4a16_gemm returns for the same arguments with a
 * large enough workspace (same plan, same kernels: bit-for-bit the same y).
 *
 *   Arguments, alignment, path choice and errors as for w4a16_gemm, plus:
 *   W4A16_ERR_BUFFER_SIZE when w4a16_workspace_bytes(M, K, N, group_size) exceeds
 *   W4A16_NOALLOC_SCRATCH_BYTES (4 MiB); nothing is launched then. Every call with
 *   M <= 32 fits (decode and the GEMV); larger M are rejected only when the output
 *   has too few tiles for the GPU and the MFMA GEMM splits a long K (e.g. M = 33,
 *   K = 16384, N = 512): such callers use w4a16_gemm with a workspace.
 *
 * Every call on one GPU shares that GPU's array: calls that may overlap in time on one
 * GPU (different streams, or different host threads without ordering) race on it and
 * must not be issued; calls queued on one stream are safe. The array's counters start
 * at zero (cleared by a small kernel on the first call on each device) and every call
 * leaves them at zero. */
#define W4A16_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)
w4a16_status w4a16_gemm_noalloc(const void* x, const void* packed, size_t packed_bytes, w4a16_dtype dtype,
                                void* y, int64_t M, int64_t K, int64_t N, int64_t group_size, const void* bias,
                                void* stream);

/* Tied-embedding gather from the packed head weight: a model whose input embedding
 * is tied to its output head keeps one quantised matrix for both (vllm-omni commit
 * "cpu_int4: repack weights in n-blocks, to bound the load-time peak": the
 * 131072 x 2048 embedding matrix doubles as the output head; commit "Add cpu_int4,
 * an asymmetric 4-bit weight path for vLLM's CPU backend": the quantised tied
 * embedding is checked end to end). With the head stored for y = x . W, W [K, N]
 * (K hidden, N vocabulary), the embedding of token t is column t of dequant(W):
 *
 *   out[i, k] = (q[k, ids[i]] - z[k div G, ids[i]]) * s[k div G, ids[i]]
 *
 * computed exactly and rounded once to `dtype` (nearest even): bit-for-bit the
 * correctly rounded value.
 *
 *   ids      int32 [T] token ids, device memory, 4-byte aligned. An id outside
 *            [0, N) yields a row of zeros (no error is reported for it).
 *   packed   the buffer w4a16_repack wrote for the head, `packed_bytes` >=
 *            w4a16_packed_bytes(K, N, G), 16-byte aligned; read only.
 *   out      [T, K] row-major, `dtype`, written in full, 16-byte aligned. Must not
 *            overlap ids or packed.
 *   T        number of tokens, 0 <= T < 2^31 (T = 0 is a valid no-op).
 *   dtype and group_size must be those the buffer was repacked with. */
w4a16_status w4a16_embedding(const int32_t* ids, int64_t T, const void* packed, size_t packed_bytes,
                             w4a16_dtype dtype, int64_t K, int64_t N, int64_t group_size, void* out,
                             void* stream);

/* ---------------------------------------------------------------- W4A8
 * The same packed int4 weights against fp8 (E4M3) activations. The vLLM note
 * "Carga de capas cuantizadas: AWQ / GPTQ / Marlin / fp8" (section "Límites y
 * fallos") describes the int4 Marlin kernel taking float8_e4m3fn activations, with
 * the scales multiplied by 512: a 4-bit code in the low nibble of an E4M3 byte reads
 * as code * 2^-9, and 512 restores the scale. Here the factor is applied as each
 * scale is read, so the buffer w4a16_repack wrote serves W4A16 and W4A8 alike.
 *
 * Two calls: w4a8_quantize turns 16-bit activations into the W4A8 activation
 * buffer, w4a8_gemm multiplies it by the packed weight. The product is
 *   y[m, n] = a[m] * sum_k e[m, k] * (q[k, n] - z[g, n]) * s[g, n]  (+ bias[n]),
 * a[m] the row scale and e the E4M3 code values, accumulated in fp32 and rounded
 * once to the output dtype (nearest even). */

/* Bytes of the W4A8 activation buffer for M rows of K (K % 128 == 0); 0 for an
 * invalid shape or M = 0. Layout, each part starting on a 256-byte boundary:
 *   codes      M*K bytes, E4M3 (OCP, no infinities, largest finite 448), row-major;
 *              within each 128-element block of a row, byte 32 h + 8 i + j holds
 *              element 32 i + 8 h + (0, 4, 1, 5, 2, 6, 3, 7)[j] (h, i = 0..3, j = 0..7):
 *              the order in which the fp8 matrix-core operands pair each activation
 *              with its weight code in the packed tiles;
 *   row scales M fp32, a[m];
 *   block sums M * K/128 fp32, row-major: the sum of the decoded codes of each
 *              128-element block (used for the zero points). */
size_t w4a8_activation_bytes(int64_t M, int64_t K);

/* Per-row dynamic quantisation: a[m] = max_k |x[m, k]| / 448 (fp32; 1 for a row of
 * zeros), codes e = RNE_E4M3(x[m, k] / a[m]) with the quotient in fp32 (correctly
 * rounded division), written with the row scales and block sums into `act`.
 *   x    [M, K] row-major, `dtype`, finite values. 16-byte aligned.
 *   act  at least w4a8_activation_bytes(M, K) bytes, 16-byte aligned, written in full
 *        (its padding excepted). Must not overlap x.
 * Bit-for-bit deterministic. M = 0 is a valid no-op. */
w4a16_status w4a8_quantize(const void* x, w4a16_dtype dtype, int64_t M, int64_t K, void* act, size_t act_bytes,
                           void* stream);

/* Workspace bytes w4a8_gemm needs for this shape (0 when it splits no K range, or for
 * an invalid shape), under the contract of w4a16_workspace_bytes: zero-filled before
 * first use, left zero by every call, not shared by calls that may overlap. */
size_t w4a8_workspace_bytes(int64_t M, int64_t K, int64_t N, int64_t group_size);

/* y = (W4A8 product above), from an activation buffer written by w4a8_quantize for
 * these M, K and a weight buffer written by w4a16_repack (any front end).
 *   act      `act_bytes` >= w4a8_activation_bytes(M, K). 16-byte aligned.
 *   packed   as for w4a16_gemm; group_size -1 or a multiple of 128 (one fp8 MFMA
 *            covers a 128-row block; 32 and 64 give W4A16_ERR_GROUP).
 *   dtype    the dtype of the scales the buffer holds, of bias and of y.
 *   y, bias, workspace: as for w4a16_gemm.
 * Bit-for-bit reproducible for fixed inputs and shape. M = 0 is a valid no-op. */
w4a16_status w4a8_gemm(const void* act, size_t act_bytes, const void* packed, size_t packed_bytes,
                       w4a16_dtype dtype, void* y, int64_t M, int64_t K, int64_t N, int64_t group_size,
                       const void* bias, void* workspace, size_t workspace_bytes, void* stream);

/* Static, NUL-terminated description of a status code ("unknown status" otherwise). */
const char* w4a16_status_str(w4a16_status status);

#ifdef __cplusplus
}
#endif

#endif /* W4A16_H */
