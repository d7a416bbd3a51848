/*
 * xq.h — C ABI of libxq, the quantized decode mat-vec for AMD MI355X (gfx950).
 *
 * Every entry point validates its arguments on the host, enqueues its kernel
 * on the caller's HIP stream and returns without synchronising ("25 — Writing
 * XPU Kernels", section 25.5: chain launches on one stream and wait once on
 * the read side). Faults during execution surface at the caller's next
 * synchronisation.
 *
 * Conventions shared by every entry point:
 *  - Pointers named as device buffers are device memory owned by the caller
 *    ("cajeta.xpu — one kernel, any device", section 2.2: buffers are the
 *    caller's allocations). The library allocates no memory and keeps no
 *    per-call state; it never synchronizes a stream or the device.
 *  - Three entry points need device scratch beyond their inputs and outputs
 *    (xq_gemm_q4k_small_m's split-K partials and arrival counters,
 *    xq_gemv_q4k_q8k's arrival counters, xq_gemm_q4k_id's expert map). The
 *    caller passes it as `workspace` (device memory, 256-byte aligned) and
 *    `workspace_bytes`; the matching *_workspace_bytes query gives the exact
 *    bytes a call needs (0: none, and then workspace may be NULL). The caller
 *    zeroes a workspace once before its first use; every call that completes
 *    leaves it ready for the next (its arrival counters back at zero), so one
 *    workspace serves any sequence of calls on one stream whose needs it
 *    covers. Calls that may run at the same time (different streams) need
 *    different workspaces. A NULL workspace where one is needed is refused
 *    with XQ_E_NULL, a short one with XQ_E_SHAPE, a misaligned one with
 *    XQ_E_ALIGN.
 *  - `stream` is a hipStream_t passed as void*; NULL means the null stream.
 *  - Outputs are fully overwritten, never accumulated into. Outputs must not
 *    alias inputs (documented, not checked).
 *  - A refused call returns a status other than XQ_OK, launches nothing and
 *    sets the thread-local text returned by xq_last_error() naming the gate
 *    that refused (section 25.6: a refusal answers with the gate that
 *    refused). There is no fallback kernel.
 *  - The gates run before any HIP call in this order: null pointers, shape,
 *    alignment, then the device (it must be gfx950).
 *
 * Byte layouts (all little-endian):
 *  q8_K block, 320 B per 256 activations (section 25.2, the integer-route
 *    bullet, and section 25.2.1): int8 codes at +0, eight int32 sums of 32
 *    consecutive codes at +256, the f32 scale at +288; bytes 292..319 are
 *    written as zero and carry no meaning. A q8_K tensor of R rows and K
 *    columns is [R][K/256] blocks, row-major.
 *  Q4_K super-block, 144 B per 256 weights ("cajeta.xpu — one kernel, any
 *    device", section 2.3, the alignment example: nibble group g at
 *    16 + 32*g): f16 d at +0, f16 dmin at +2, twelve bytes of packed 6-bit
 *    scales and mins at +4, 128 B of nibbles at +16. Group g's 32 bytes hold
 *    sub-block 2g in their low nibbles and sub-block 2g+1 in their high
 *    nibbles. Weight = d*sc_j*q - dmin*m_j. A matrix of N rows and K columns
 *    is [N][K/256] blocks, row-major.
 *  IQ4_NL resident row (section 25.2.1): the row's K/32 f16 block scales,
 *    padded to a multiple of 4 bytes, then K/32 payloads of 16 B; payload
 *    byte t gives weight t (low nibble) and weight t+16 (high nibble); a
 *    nibble selects an int8 from the 16-entry IQ4_NL codebook; weight =
 *    d_c * kv[nibble]. A matrix is N such rows back to back.
 */
#ifndef XQ_H
#define XQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t xq_status;

enum {
    XQ_OK = 0,
    XQ_E_NULL = 1,   /* a required pointer is NULL */
    XQ_E_SHAPE = 2,  /* a size is out of range or not a multiple it must be */
    XQ_E_ALIGN = 3,  /* a buffer base is short of the alignment its loads need */
    XQ_E_DEVICE = 4, /* no HIP device, or the current device is not gfx950 */
    XQ_E_LAUNCH = 5  /* the runtime refused the kernel launch */
};

/*
 * Quantize f32 activations to q8_K ("25 — Writing XPU Kernels", section 25.2,
 * the integer-route bullet: the activation is quantized once to q8_K).
 * Per 256-block: amax = max|x_i|; d = amax/127 as one IEEE f32 division;
 * code_i = x_i/d (IEEE f32 division) rounded to nearest, ties to even (0 when
 * d == 0); sum_j = sum of codes 32j..32j+31.
 *
 *  xq    device, out: rows*(K/256) q8_K blocks, 16-byte aligned.
 *  x     device, in: f32 [rows][K] row-major, 4-byte aligned (a 16-byte
 *        aligned x is read with 16-byte loads, any other with 4-byte loads;
 *        the bytes written are the same).
 *  rows  >= 1.  K >= 256, a multiple of 256.
 * Errors: XQ_E_NULL, XQ_E_SHAPE, XQ_E_ALIGN, XQ_E_DEVICE, XQ_E_LAUNCH.
 */
xq_status xq_quantize_q8k(void *xq, const float *x, int64_t rows, int64_t K, void *stream);

/*
 * Q4_K x q8_K decode mat-vec, batch 1 ("25 — Writing XPU Kernels", section
 * 25.2, and section 25.5 for the Q4_K mat-vec's 16-byte loads):
 *   y[r] = sum_b xs_b * (d_rb * S_rb - dmin_rb * M_rb),
 *   S_rb = sum_j sc_j * sum_{t<32} q * code   (exact int32),
 *   M_rb = sum_j m_j * s_j                    (exact int32; s_j the q8_K's stored
 *                                              sum of sub-block j's 32 codes),
 * which is the dot of the dequantized row with the dequantized activation.
 *
 *  y   device, out: f32 [N], 4-byte aligned.
 *  w   device, in: Q4_K [N][K/256], 16-byte aligned.
 *  xq  device, in: one q8_K row of K/256 blocks, 16-byte aligned.
 *  1 <= N <= 2^30.  K >= 256, a multiple of 256, K <= XQ_MAX_K.
 * Errors: XQ_E_NULL, XQ_E_SHAPE, XQ_E_ALIGN, XQ_E_DEVICE, XQ_E_LAUNCH.
 */
xq_status xq_gemv_q4k(float *y, const void *w, const void *xq, int64_t N, int64_t K, void *stream);

/*
 * Q4_K x q8_K mat-vec with its output quantized in the same launch ("25 —
 * Writing XPU Kernels", section 25.5: the FFN pair's fused tail; the up
 * product hands the down product its q8_K activation):
 *   y  = the result of xq_gemv_q4k(y, w, xq, N, K), bit for bit;
 *   yq = the bytes xq_quantize_q8k(yq, y, 1, N) writes, bytes 0..291 of every
 *        block bit for bit (292..319 zero).
 * The 256/(rows per workgroup) workgroups of each q8_K block of y count
 * their arrival on a counter; the last quantizes the block.
 *
 *  y   device, out: f32 [N], 4-byte aligned.
 *  yq  device, out: q8_K [N/256] blocks (xq_q8k_bytes(1, N)), 16-byte aligned.
 *  w, xq, K as xq_gemv_q4k.
 *  N a multiple of 256, 256 <= N <= 2^22.
 *  workspace  the block counters: xq_gemv_q4k_q8k_workspace_bytes(N) bytes
 *      (one 128-byte line per q8_K block of y), zeroed before first use; the
 *      last arrival at a counter resets it.
 * Errors: XQ_E_NULL, XQ_E_SHAPE, XQ_E_ALIGN, XQ_E_DEVICE, XQ_E_LAUNCH.
 */
xq_status xq_gemv_q4k_q8k(float *y, void *yq, const void *w, const void *xq, int64_t N, int64_t K,
                          void *workspace, size_t workspace_bytes, void *stream);
size_t xq_gemv_q4k_q8k_workspace_bytes(int64_t N);  /* N/256 * 128; 0 if N is invalid */

/*
 * IQ4_NL x q8_K decode mat-vec, batch 1 ("25 — Writing XPU Kernels", section
 * 25.2.1): y[r] = sum_c d_rc * xs_(c/8) * D_rc with D_rc = sum_{t<32}
 * kv[nibble_t] * code_(32c+t) (exact int32).
 *
 *  y   device, out: f32 [N], 4-byte aligned.
 *  w   device, in: N resident IQ4_NL rows (xq_iq4nl_bytes(N, K) bytes),
 *      16-byte aligned.
 *  xq  device, in: one q8_K row of K/256 blocks, 16-byte aligned.
 *  1 <= N <= 2^30.  K >= 256, a multiple of 256 (each 32-block must fall inside a
 *  q8_K block), K <= XQ_MAX_K.
 * Errors: XQ_E_NULL, XQ_E_SHAPE, XQ_E_ALIGN, XQ_E_DEVICE, XQ_E_LAUNCH.
 */
xq_status xq_gemv_iq4nl(float *y, const void *w, const void *xq, int64_t N, int64_t K,
                        void *stream);

/*
 * Q4_K x q8_K small-M product (multi-token prefill; "25 — Writing XPU
 * Kernels", section 25.3): Y[m][n] = sum_b xs_mb * (d_nb * S_mnb - dmin_nb *
 * M_mnb), with S and M the exact int32 block partials of xq_gemv_q4k taken
 * against token m's q8_K row.
 *
 *  y   device, out: f32 [M][N] row-major (token-major), 4-byte aligned.
 *  w   device, in: Q4_K [N][K/256], 16-byte aligned.
 *  xq  device, in: q8_K [M][K/256], 16-byte aligned.
 *  1 <= M <= 2^30.  1 <= N <= 2^30.  K >= 256, a multiple of 256. Each of
 *  xq and w below 2 GiB (the kernel's loads use 32-bit offsets).
 * A very short batch (M = 1; M <= 3; M = 4 when K <= 4096 or N*K <= 2^25,
 * M <= 6 when N*K <= 2^24, M <= 8 when N*K <= 2^23 or when K <= 4096 and
 * N*K <= 2^24, in each while the M q8_K rows fit 64 KB) is a weight stream
 * rather than a dense contraction: it runs on the mat-vec kernels, one pass
 * over the weights for all M tokens, and row m is then bit-identical to
 * xq_gemv_q4k on token m. Larger M runs on int8 MFMA: 5 to 16 tokens on
 * matrices of 8161 to 16384 rows and 8 to 16 super-blocks per row in
 * tiles of 32 rows whose four waves split K and sum their partial tiles in
 * a fixed order (no workspace); otherwise in tiles of 16 tokens up to M = 32
 * (64 when N*K <= 2^25 or N <= 4096, 96 when N*K <= 2^25, 128 when
 * N*K <= 2^24) and of 64 tokens beyond.
 * Shapes with at most 256 tiles of 16 or 64 tokens x 128 rows split K over
 * several workgroups (section 25.3: fill the device first); shapes with more
 * tiles than one round of resident workgroups run whole rounds of whole
 * tiles and may split the last, short round's tiles the same way. Splits
 * are summed in a fixed order, so results are bit-identical from call to
 * call and do not depend on the workspace's address.
 *  workspace  96 KiB of arrival counters (one 128-byte line per split tile,
 *      at the same place for every shape), then the split partials:
 *      xq_gemm_q4k_small_m_workspace_bytes(M, N, K) bytes, 0 when the shape
 *      splits no tile (at most 16 MiB + 96 KiB for any shape), zeroed
 *      before first use.
 * Errors: XQ_E_NULL, XQ_E_SHAPE, XQ_E_ALIGN, XQ_E_DEVICE, XQ_E_LAUNCH.
 */
xq_status xq_gemm_q4k_small_m(float *y, const void *w, const void *xq, int64_t M, int64_t N,
                              int64_t K, void *workspace, size_t workspace_bytes, void *stream);
size_t xq_gemm_q4k_small_m_workspace_bytes(int64_t M, int64_t N, int64_t K);  /* 0 if none, or
                                                                              if the shape is refused */

/*
 * xq_gemm_q4k_small_m without a workspace and without any allocation, for
 * callers that cannot allocate device memory or pass a workspace: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, results (bit for bit), gates and errors as
 * xq_gemm_q4k_small_m, except the workspace: the split-K partials and
 * arrival counters live in the library's own device array of
 * XQ_NOALLOC_SCRATCH_BYTES, one per GPU, held until the process ends. A shape
 * whose plan needs more scratch than that (xq_gemm_q4k_small_m_workspace_bytes
 * above it: some 64-token-tile shapes with split K) is refused with
 * XQ_E_SHAPE; every shape of up to 32 tokens fits. The first call on a GPU
 * looks the array up and clears its counters on the caller's stream; every
 * completed call leaves them at zero. All calls on one GPU share the array:
 * calls that overlap in time on one GPU (other streams, other threads) race
 * and must not be issued.
 */
#define XQ_NOALLOC_SCRATCH_BYTES (8u * 1024u * 1024u)
xq_status xq_gemm_q4k_small_m_noalloc(float *y, const void *w, const void *xq, int64_t M,
                                      int64_t N, int64_t K, void *stream);

/*
 * Grouped Q4_K x q8_K small-M product over an expert slab (mul_mat_id; "25 —
 * Writing XPU Kernels", section 25.3: a mixture-of-experts prefill is one
 * launch over an expert map, padded only to the finest tile, never one
 * product per expert). Token t's slot k uses expert e = ids[t][k]:
 *   y[t][k][n] = sum_b xs_b * (d_enb * S_b - dmin_enb * M_b)
 * with S, M the exact int32 block partials of expert e's row n against the
 * pair's q8_K row, which is row t of xq (x_per_slot = 0: the slots of a
 * token share its activation, as for up and gate) or row t * n_used + k
 * (x_per_slot = 1: each slot has its own, as for down).
 *
 *  y     device, out: f32 [n_tokens][n_used][rows], 4-byte aligned. The rows
 *        of a pair whose selection lies outside 0..n_experts-1 are NaN.
 *  slab  device, in: n_experts experts of rows x K Q4_K weights back to back
 *        (expert e's row n is row e * rows + n), 16-byte aligned.
 *  xq    device, in: q8_K [n_tokens or n_tokens * n_used][K/256], 16-byte aligned.
 *  ids   device, in: int32 [n_tokens][n_used], 4-byte aligned.
 *  1 <= n_tokens * n_used <= 2^20.  1 <= n_experts <= 1024.  1 <= rows <= 2^30.
 *  K >= 256, a multiple of 256. One expert's weights and all of xq below
 *  2 GiB (32-bit offsets).
 * A first kernel groups the pairs by expert into tiles of at most 64 pairs
 * (an expert's remainder of at most 32 pairs into tiles of at most 16); the
 * product then runs once over both lists. Every output is computed from its
 * own pair alone, so results do not depend on how pairs fall into tiles.
 *  workspace  the expert map (tile descriptors, the pairs grouped by
 *      expert, the tile counts): xq_gemm_q4k_id_workspace_bytes(n_tokens,
 *      n_used, n_experts) bytes (at most 4.3 MB), rewritten by every call.
 * Errors: XQ_E_NULL, XQ_E_SHAPE, XQ_E_ALIGN, XQ_E_DEVICE, XQ_E_LAUNCH.
 */
xq_status xq_gemm_q4k_id(float *y, const void *slab, const void *xq, const int32_t *ids,
                         int64_t n_tokens, int64_t n_used, int64_t n_experts, int64_t rows,
                         int64_t K, int64_t x_per_slot, void *workspace, size_t workspace_bytes,
                         void *stream);
size_t xq_gemm_q4k_id_workspace_bytes(int64_t n_tokens, int64_t n_used, int64_t n_experts);

/* Largest K the mat-vecs accept (the q8_K row is then 1.25 MiB). Rows of up
 * to 49152 columns stage the row in the workgroup's LDS (60 KiB at most);
 * longer rows read it from global memory, where every workgroup finds it in
 * L2. The small-M product (xq_gemm_q4k_small_m) takes any K. */
#define XQ_MAX_K 1048576

/* Byte sizes of the layouts above; 0 when the shape is invalid. */
size_t xq_q8k_bytes(int64_t rows, int64_t K);   /* rows*(K/256)*320 */
size_t xq_q4k_bytes(int64_t N, int64_t K);      /* N*(K/256)*144 */
size_t xq_iq4nl_bytes(int64_t N, int64_t K);    /* N*(ceil4(2*(K/32)) + 16*(K/32)) */

/* Static name of a status code ("XQ_OK", "XQ_E_SHAPE", ...). */
const char *xq_status_name(xq_status s);

/* Thread-local text of the last refusal on this thread ("" after success). */
const char *xq_last_error(void);

/*
 * Q4_0 x q8_K mat-vec: y[n] = sum_k w[n][k] * xhat[k] with w = d_c * (nibble - 8)
 * ("25 — Writing XPU Kernels", section 25.2: the Q4_0 twin of the IQ4_NL
 * kernel; its -8 rides on the activation's sum). The weight rows have the
 * IQ4_NL resident shape (K/32 f16 scales padded to a dword, then K/32 payloads
 * of 16 B; xq_iq4nl_bytes(N, K) bytes; xq_repack_iq4nl converts Q4_0 file
 * blocks too, they share the 18-byte shape); each 32-block's integer dot
 * sum(nibble*code) - 8*s uses the q8_K's stored sum s of its 32 codes.
 *  Same arguments, alignment and limits as xq_gemv_iq4nl.
 */
xq_status xq_gemv_q4_0(float *y, const void *w_q4_0, const void *xq, int64_t N, int64_t K,
                       void *stream);

/*
 * Expert-grouped mat-vecs ("25 — Writing XPU Kernels", section 25.2.2: one
 * launch over a bank of experts, the dot loop of the dense kernel unchanged;
 * the expert is picked on the device through a selection buffer, nothing is
 * read back). For each selection slot kk in 0..used-1 and row r in
 * 0..rows-1:
 *   y[kk*rows + r] = row (sel[kk]*rows + r) of `slab` . activation kk
 * where activation kk is the q8_K row starting x_stride_blocks*kk blocks into
 * `xq` (x_stride_blocks = 0: every slot reads the one token, as in decode;
 * = K/256: slot kk reads row kk of a [used][K/256] q8_K tensor).
 *  slab  [n_experts][rows] rows of the format (Q4_K: [.][K/256] blocks of
 *        144 B; IQ4_NL: resident rows), experts back to back, 16-byte aligned.
 *  sel   device int32[used], 4-byte aligned. A value outside
 *        0..n_experts-1 makes that slot's `rows` outputs NaN (nothing is
 *        read for it); the other slots are unaffected.
 *  y     f32[used][rows], slot-major.
 *  1 <= used <= 65535, 1 <= rows, n_experts*rows <= 2^30, K as for the
 *  dense entry point, x_stride_blocks in {0, K/256}.
 * Each slot's outputs are bit-identical to the dense entry point (xq_gemv_q4k
 * or xq_gemv_iq4nl) on that expert's rows and that activation.
 */
xq_status xq_gemv_q4k_id(float *y, const void *slab, const void *xq, const int32_t *sel,
                         int64_t n_experts, int64_t used, int64_t rows, int64_t K,
                         int64_t x_stride_blocks, void *stream);
xq_status xq_gemv_iq4nl_id(float *y, const void *slab, const void *xq, const int32_t *sel,
                           int64_t n_experts, int64_t used, int64_t rows, int64_t K,
                           int64_t x_stride_blocks, void *stream);

/*
 * Bind-time repack of IQ4_NL file blocks into resident rows ("25 — Writing XPU
 * Kernels", section 25.4: weights are converted once, at upload, into the one
 * resident layout the kernels read; section 25.4.1: each work item moves one
 * payload dword). A file block is 18 bytes: the f16 scale, then the 16 payload bytes
 * (byte t: weight t in the low nibble, weight t+16 in the high nibble).
 *  file_blocks  the chunk: n_blocks blocks back to back, global blocks
 *               block_base .. block_base + n_blocks - 1 of a matrix of bpr
 *               blocks per row (block g is block g % bpr of row g / bpr);
 *               2-byte aligned (16-byte aligned chunks are staged through LDS
 *               with 16-byte loads, the faster route; the bytes written are
 *               the same).
 *  resident     row 0 of the matrix in resident rows (xq_iq4nl_bytes per row
 *               for K = 32*bpr: bpr f16 scales, zero-padded to a multiple of
 *               4 bytes, then bpr payloads of 16 B); 4-byte aligned; must hold
 *               rows 0 .. (block_base + n_blocks - 1) / bpr. Only the bytes of
 *               the chunk's blocks are written (and a row's 2 pad bytes, when
 *               bpr is odd, by the chunk holding the row's last block).
 *  1 <= n_blocks <= 2^29, 0 <= block_base <= 2^40, 1 <= bpr <= 2^24.
 * One pass reads each source byte once. A chunk that starts and ends on row
 * boundaries writes its scale prefix as whole dwords; any other chunk writes
 * each scale as a 16-bit half. xq_repack_dword_prefix_launches() counts the
 * launches of the first route in this process (section 25.7.2: a test that
 * the route fires, and one that it does not).
 */
xq_status xq_repack_iq4nl(void *resident, const void *file_blocks, int64_t n_blocks,
                          int64_t block_base, int64_t bpr, void *stream);
int64_t xq_repack_dword_prefix_launches(void);

/*
 * Measurement helper, not part of the method: read `bytes` of device memory
 * once with 16-byte loads and fold them into one word per workgroup of
 * `sink` (sink must hold xq_bench_sink_words(bytes) uint32). Its duration
 * gives the streaming-read ceiling the mat-vecs are held against ("25 —
 * Writing XPU Kernels", section 25.1: measure the bandwidth once per device
 * with a streaming pass well past L2).
 *  buf 16-byte aligned, bytes a positive multiple of 16.
 */
xq_status xq_bench_stream_read(const void *buf, int64_t bytes, uint32_t *sink, void *stream);
int64_t xq_bench_sink_words(int64_t bytes);

#ifdef __cplusplus
}
#endif

#endif /* XQ_H */
