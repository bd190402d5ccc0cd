/*
 * mxcast.h -- C ABI of libmxcast: block-scaled quantisation of bf16 tensors
 * on MI355X (gfx950).
 *
 * The operations are the cast kernels that the pages measure:
 *   - MXFP8 cast, row-wise, column-wise (into the transposed layout) or both
 *     in one pass, optionally fused with a GELU / dGELU pre-op and a dbias
 *     column sum ("[Common] Fix pointer arithmatic to generate correct
 *     LDS/STS instructions", TransformerEngine PR 3291: tables "MXFP8 generic
 *     quantize kernel" and "MXFP8 specialized cast-only kernel
 *     (bidimensional)"; torchao PR 12 "Multiply with inverse scale in loop
 *     inside of dividing to improve perf": the dim1 cast and its inverse-scale
 *     multiply);
 *   - gated MXFP8 cast of act(gate) * linear with SwiGLU or GeGLU (PR 3291,
 *     table "MXFP8 gated (swiglu / geglu) kernel"), and the backward casts
 *     the same tables name: dSiLU (generic kernel) and dSwiGLU / dGeGLU
 *     (gated kernel);
 *   - NVFP4 quantize-transpose with 16-element or 16 x 16 blocks (PR 3291,
 *     the NVFP4 quantize-transpose kernels under "Important Files Changed",
 *     "Patched but not measurable" and table "NVFP4 2D quantize-transpose
 *     kernel");
 *   - grouped (per-expert) MXFP8 and NVFP4 casts of tensors stacked along
 *     rows (PR 3291, the grouped NVFP4 quantize-transpose row);
 *   - format, layout and shape extensions of the MXFP8 casts: E5M2 elements,
 *     the round-up scale rule, GEMM-ready scale tiles, any row count and row
 *     length (partial edge blocks).
 *
 * Numerics (the pages name these formats but do not define their
 * arithmetic; these are the readings the library implements bit-exactly):
 *   MXFP8 block of 32: amax = max|y|; scale byte (E8M0) = floor(log2 amax) - 8
 *     + 127 clamped to [0, 254]; element = E4M3(y * 2^(127 - byte)), round
 *     to nearest, ties to even code, saturating at +-448, sign kept.  A block
 *     holding Inf/NaN gets scale 0xFF and elements 0x7F.  (E5M2 and the
 *     round-up rule: see MX_ELEM_E5M2 / MX_SCALE_ROUND_UP.)
 *   Fused pre-ops: evaluated in fp32 (tanh-form GELU through
 *     0.5(1+tanh u) = 1/(1+e^-2u), the library's own exp), rounded once to
 *     bf16; that bf16 tensor y is what is quantised and what dbias sums.
 *   NVFP4: S_g = fl32(amax / 2688) (1 if amax = 0); per block of 16:
 *     s = E4M3(fl32(fl32(b/6)/S_g)), inv = fl32(1/fl32(decode(s)*S_g)) (0 if
 *     the product is 0), element = E2M1(fl32(x*inv)), nearest, ties to even,
 *     saturating at +-6.
 *
 * Conventions for every call:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the
 *     library never allocates, frees or synchronises.  Work is enqueued on
 *     `stream` (NULL = the default stream) and completes asynchronously.
 *     Scratch memory comes from the caller (a workspace argument), except
 *     for mx_quantize_noalloc, whose scratch is a static device array.
 *   - bf16 tensors are raw 16-bit patterns; E4M3, E8M0 and packed E2M1 are
 *     raw bytes.  Every tensor is row-major and contiguous.
 *   - Column-wise outputs are transposed: for x[M][K], q_col is [K][M] and
 *     s_col is [K][ceil(M/32)] (MXFP8, compact scales) or q_col
 *     [K][ceil(M/2)], s_col [K][ceil(M/16)] (NVFP4).
 *   - Every pointer must be 16-byte aligned (dbias: 4-byte).
 *   - Arguments are validated on the host before anything is enqueued; on a
 *     validation error nothing is written and a non-zero status returns.
 *     Launch failures return MX_ERR_HIP.  Device faults surface at the
 *     caller's next synchronisation.
 *   - Calls hold no state and are safe from several host threads (the one
 *     exception, mx_quantize_noalloc's shared scratch, is described there).
 */
#ifndef MXCAST_H
#define MXCAST_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MXCAST_ABI_VERSION 10

typedef enum mx_status {
    MX_OK = 0,
    MX_ERR_NULL = 1,        /* a required pointer is NULL                     */
    MX_ERR_ENUM = 2,        /* unknown axis mask, fusion or activation        */
    MX_ERR_SHAPE = 3,       /* non-positive or too large size                 */
    MX_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned               */
    MX_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required     */
    MX_ERR_ALIAS = 6,       /* an output overlaps an input or another output  */
    MX_ERR_HIP = 7,         /* the HIP runtime reported a launch error        */
    MX_ERR_UNSUPPORTED = 8  /* valid request this version does not implement  */
} mx_status;

/* axis_mask bits */
#define MX_ROWWISE 1u       /* blocks along K: q_row[M][K] and its scales    */
#define MX_COLWISE 2u       /* blocks along M, transposed outputs             */

/*
 * Format flags, OR-ed into the axis_mask of the three MXFP8 casts
 * (mx_quantize, mx_quantize_gated, mx_quantize_dgated; not NVFP4).  The
 * pages name the MXFP8 cast without fixing its element format or scale rule
 * (TransformerEngine PR 3291, table "MXFP8 generic quantize kernel"); the
 * default is E4M3 elements with the floor rule, and these select the other
 * choices of the OCP MX format family:
 *   MX_ELEM_E5M2       E5M2 elements (bias 15, max 57344, round to nearest
 *                      even, saturating) instead of E4M3 (max 448); the
 *                      floor rule becomes byte = floor(log2 amax) - 15 + 127.
 *   MX_SCALE_ROUND_UP  byte = ceil(log2(amax / max_elem)) + 127, the smallest
 *                      power-of-two scale under which no element saturates,
 *                      instead of floor(log2 amax) - emax + 127.
 * Bytes clamp to [0, 254]; a block holding Inf or NaN gets scale 0xFF and
 * elements 0x7F under every choice.  Output layouts are unchanged.
 */
#define MX_ELEM_E5M2 4u
#define MX_SCALE_ROUND_UP 8u

/*
 * MX_SCALE_TILED, OR-ed into the axis_mask of the MXFP8 casts: the scale
 * tensors are written in a GEMM-ready layout instead of compact row-major.
 * The pages only hint at consumer-ready scale shapes (the "fix scale shapes"
 * step of the torchao PR 12 stack); the layout is the one a gfx950
 * block-scaled 32x32x64 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4) reads: lane
 * L of a wave supplies the E8M0 scale of row L % 32 and 32-element K block
 * L / 32 of each 64-wide step (its operand bytes hold 16 K values of each of
 * the step's two blocks), from a byte of a 32-bit register that the
 * instruction's op_sel picks per step; a GPU test feeds the cast's outputs
 * to that instruction.  For a scale matrix S[R][C] (s_row: R = M rows,
 * C = K/32 blocks; s_col: R = K transposed rows, C = M/32 blocks):
 *   tile (rt, bt) = rows 32 rt .. 32 rt + 31, blocks 8 bt .. 8 bt + 7,
 *                   256 bytes at byte offset (bt * ceil(R/32) + rt) * 256;
 *   inside it, the 4-byte word of lane L holds in byte j (j = 0..3) the scale
 *                   of row 32 rt + L % 32, block 8 bt + 2j + L / 32, i.e. the
 *                   scale lane L uses in the j-th of four consecutive steps.
 * Blocks past C in the last block tile are 0.  Size: ceil(R/32) * ceil(C/8)
 * * 256 bytes (mx_scale_size).  Element tensors are unchanged.
 */
#define MX_SCALE_TILED 16u

/* fusion: a pre-op in the low bits, optionally OR-ed with MX_FUSE_DBIAS */
#define MX_FUSE_NONE 0
#define MX_FUSE_GELU 1      /* y = GELU(x)                                    */
#define MX_FUSE_DGELU 2     /* y = GELU'(x) * grad                            */
#define MX_FUSE_DSILU 3     /* y = SiLU'(x) * grad                            */
#define MX_FUSE_DBIAS 0x10  /* also write dbias[k] = sum_m y[m][k] (fp32)     */

/* gated activation */
#define MX_GATED_SWIGLU 1   /* y = silu(gate) * linear                        */
#define MX_GATED_GEGLU 2    /* y = gelu(gate) * linear                        */

/*
 * MXFP8 cast of x[M][K] (bf16), block size 32.  Element bytes are E4M3
 * unless axis_mask holds MX_ELEM_E5M2.  When 32 does not divide K (M), the
 * last block of each row (column) is partial: its scale and codes come from
 * its own elements, and the scale tensors have ceil(K/32) (ceil(M/32))
 * blocks per line.
 *   x        device, bf16 [M][K]
 *   grad     device, bf16 [M][K]; required for MX_FUSE_DGELU / DSILU, else
 *            ignored
 *   M, K     rows, columns: any M, K >= 1, each <= 2^23, M*K <= 2^40.  K a
 *            multiple of 8 (every row of x 16-byte aligned) takes the tiled
 *            kernel, for any M (with M not a multiple of 16 the rows of q_col
 *            start at any byte and it writes them through a two-tile stage,
 *            at a lower bandwidth); any other K takes a kernel for arbitrary
 *            row alignment (same results, lower bandwidth still)
 *   axis_mask  MX_ROWWISE, MX_COLWISE or both (one pass over x), optionally
 *            with the format flags MX_ELEM_E5M2 / MX_SCALE_ROUND_UP and the
 *            layout flag MX_SCALE_TILED (scale tensors then have
 *            mx_scale_size() bytes in the tile layout)
 *   fusion   MX_FUSE_NONE | GELU | DGELU | DSILU, optionally | MX_FUSE_DBIAS
 *   q_row, s_row  E4M3 [M][K] and E8M0 [M][ceil(K/32)]; required iff MX_ROWWISE
 *   q_col, s_col  E4M3 [K][M] and E8M0 [K][ceil(M/32)]; required iff MX_COLWISE
 *   dbias    fp32 [K]; required iff MX_FUSE_DBIAS
 *   workspace, workspace_bytes  device scratch of at least
 *            mx_quantize_workspace_size() bytes (0 unless MX_FUSE_DBIAS);
 *            its contents on entry are ignored and on exit are undefined
 *   stream   HIP stream
 * With MX_FUSE_DBIAS a second, small kernel reduces per-tile column partial
 * sums (fp32, fixed order) into dbias, so results are run-to-run identical.
 */
mx_status mx_quantize(const void *x, const void *grad, int64_t M, int64_t K,
                      unsigned axis_mask, int fusion,
                      uint8_t *q_row, uint8_t *s_row, uint8_t *q_col, uint8_t *s_col,
                      float *dbias, void *workspace, size_t workspace_bytes,
                      hipStream_t stream);

/* Bytes of workspace mx_quantize needs for these arguments (0 without dbias;
 * 0 also for invalid arguments). */
size_t mx_quantize_workspace_size(int64_t M, int64_t K, unsigned axis_mask, int fusion);

/*
 * mx_quantize for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same cast with the same arguments, minus the workspace: with MX_FUSE_DBIAS
 * the per-tile column partial sums go to a static device array of the
 * library, MX_NOALLOC_SCRATCH_BYTES per GPU, which each GPU the library runs
 * on holds until the process ends.  Outputs are bit-identical to
 * mx_quantize's (the same kernels and the same fixed summation order).
 *   - No device memory is allocated or freed, by the library or a library it
 *     calls.  Without MX_FUSE_DBIAS the scratch is not used at all.
 *   - A dbias cast whose workspace (mx_quantize_workspace_size) exceeds
 *     MX_NOALLOC_SCRATCH_BYTES returns MX_ERR_WORKSPACE and writes nothing.
 *   - Every call on one GPU shares that GPU's scratch, which keeps the last
 *     call's contents (every byte a call reads it has written first): calls
 *     with MX_FUSE_DBIAS that overlap on one GPU (on different streams, or
 *     from several host threads without ordering) race and may give wrong
 *     dbias values.  Calls ordered on one stream are safe.
 *   - The first call on each device looks up the scratch address (no
 *     allocation); the stream's device is made current for that lookup.
 * Other errors as for mx_quantize.
 */
#define MX_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)
mx_status mx_quantize_noalloc(const void *x, const void *grad, int64_t M, int64_t K,
                              unsigned axis_mask, int fusion,
                              uint8_t *q_row, uint8_t *s_row, uint8_t *q_col, uint8_t *s_col,
                              float *dbias, hipStream_t stream);

/*
 * Bytes of one scale tensor of an MXFP8 cast: the scales of a quantised
 * [rows][cols] tensor blocked along cols (s_row: rows = M, cols = K; s_col:
 * rows = K, cols = M; for the gated casts the quantised tensor's own sizes).
 * rows * ceil(cols/32) for the compact layout, ceil(rows/32) *
 * ceil(ceil(cols/32)/8) * 256 with MX_SCALE_TILED in axis_mask.  0 for a
 * non-positive size, a size above 2^23 or an invalid axis_mask.
 */
size_t mx_scale_size(int64_t rows, int64_t cols, unsigned axis_mask);

/*
 * Grouped (per-expert) MXFP8 cast: G tensors stacked along rows, cast in one
 * launch, each exactly as mx_quantize would cast it on its own.  The pages
 * name a grouped quantize-transpose (TransformerEngine PR 3291, the
 * group_quantize_transpose_nvfp4 row of its "Important Files Changed"
 * table) whose non-Hadamard path was not ready; this is that operation for
 * MXFP8.
 *   x, grad      device, bf16 [M][K], M = sum of group_rows; group g owns rows
 *                r_g .. r_g + group_rows[g] - 1, r_g = sum_{h<g} group_rows[h]
 *   group_rows   HOST array of G row counts, each >= 0 (an empty group is
 *                allowed); 1 <= G <= 64, 0 < M <= 2^23.  K a multiple of 8
 *                takes the tiled kernel, for any counts (counts that are not
 *                multiples of 16: as for an M that is not, in mx_quantize),
 *                any other K the any-shape kernel (same results)
 *   axis_mask, fusion  as for mx_quantize (format and layout flags included)
 *   q_row        [M][K]: the groups' row-wise elements (the stacked tensor's)
 *   s_row        the groups' row scales one after the other, group g's
 *                mx_scale_size(group_rows[g], K) bytes each (for the compact
 *                layout this is [M][ceil(K/32)])
 *   q_col        the groups' transposed elements one after the other: group
 *                g's [K][group_rows[g]] at byte K * r_g
 *   s_col        the groups' column scales one after the other, group g's
 *                mx_scale_size(K, group_rows[g]) bytes each
 *   dbias        fp32 [G][K], group g's column sums (0 for an empty group)
 *   workspace    mx_quantize_grouped_workspace_size() bytes with dbias
 * Errors as for mx_quantize; MX_ERR_SHAPE also for G out of range or a bad
 * group size.
 */
mx_status mx_quantize_grouped(const void *x, const void *grad, int64_t K,
                              const int64_t *group_rows, int G, unsigned axis_mask, int fusion,
                              uint8_t *q_row, uint8_t *s_row, uint8_t *q_col, uint8_t *s_col,
                              float *dbias, void *workspace, size_t workspace_bytes,
                              hipStream_t stream);

/* Workspace bytes of mx_quantize_grouped (0 without dbias or for invalid
 * arguments). */
size_t mx_quantize_grouped_workspace_size(int64_t K, const int64_t *group_rows, int G,
                                          unsigned axis_mask, int fusion);

/* Total bytes of the row scales (colwise = 0) or column scales (colwise = 1)
 * of mx_quantize_grouped (0 for invalid arguments). */
size_t mx_grouped_scale_size(int64_t K, const int64_t *group_rows, int G, unsigned axis_mask,
                             int colwise);

/*
 * Gated MXFP8 cast.  x is bf16 [M][2N] holding [gate | linear] (gate =
 * columns 0..N-1); the quantised tensor is y[M][N] = act(gate) * linear,
 * block size 32 (partial at the edges as for mx_quantize), any M, N >= 1
 * with M <= 2^23, 2N <= 2^23, M * 2N <= 2^40 (N a multiple of 8 takes the
 * tiled kernel, for any M, as in mx_quantize).  axis_mask as for mx_quantize
 * (format flags included).
 *   q_row, s_row  E4M3 [M][N], E8M0 [M][ceil(N/32)]   (iff MX_ROWWISE)
 *   q_col, s_col  E4M3 [N][M], E8M0 [N][ceil(M/32)]   (iff MX_COLWISE)
 */
mx_status mx_quantize_gated(const void *x, int64_t M, int64_t N, unsigned axis_mask, int act,
                            uint8_t *q_row, uint8_t *s_row, uint8_t *q_col, uint8_t *s_col,
                            hipStream_t stream);

/*
 * Gated backward MXFP8 cast (the dswiglu / dgeglu rows of the gated table).
 * grad is bf16 [M][N] (the gradient of act(gate) * linear), x the forward
 * input bf16 [M][2N] = [gate | linear].  With a = act(gate), a' = act'(gate)
 * (act = SiLU for MX_GATED_SWIGLU, GELU for MX_GATED_GEGLU), the quantised
 * tensor is dx[M][2N] = [d_gate | d_linear]:
 *   d_gate   = fl32(fl32(a' * grad) * linear),   d_linear = fl32(a * grad),
 * each rounded once to bf16; block size 32 along 2N (row-wise) and M.
 * Any M, N >= 1 with M <= 2^23, 2N <= 2^23, M * 2N <= 2^40 (partial blocks
 * at the edges as for mx_quantize; N a multiple of 8 takes the tiled kernel,
 * for any M).  axis_mask as for mx_quantize (format flags included).
 *   q_row, s_row  E4M3 [M][2N], E8M0 [M][ceil(2N/32)]   (iff MX_ROWWISE)
 *   q_col, s_col  E4M3 [2N][M], E8M0 [2N][ceil(M/32)]   (iff MX_COLWISE)
 * Errors as for mx_quantize_gated.
 */
mx_status mx_quantize_dgated(const void *grad, const void *x, int64_t M, int64_t N,
                             unsigned axis_mask, int act, uint8_t *q_row, uint8_t *s_row,
                             uint8_t *q_col, uint8_t *s_col, hipStream_t stream);

/*
 * Grouped gated casts (an MoE layer's experts in one launch): x is bf16
 * [M][2N] = [gate | linear] with the groups' rows stacked as for
 * mx_quantize_grouped (HOST group_rows, any counts >= 0, empty groups
 * allowed, 1 <= G <= 64); each group is cast exactly as mx_quantize_gated
 * (forward: quantised tensor [rows][N], W = N) or mx_quantize_dgated
 * (backward, grad bf16 [M][N]: quantised tensor [rows][2N], W = 2N) casts
 * it on its own.  q_row is [M][W]; q_col holds group g's [W][rows] at byte
 * W * r_g; s_row and s_col hold the groups' scale tensors one after the
 * other, group g's mx_scale_size(rows, W) and mx_scale_size(W, rows) bytes
 * (mx_grouped_scale_size(W, ...) in total).  axis_mask as for mx_quantize.
 * Errors as for mx_quantize_gated; MX_ERR_SHAPE also for G out of range or a
 * bad group size.
 */
mx_status mx_quantize_gated_grouped(const void *x, int64_t N, const int64_t *group_rows, int G,
                                    unsigned axis_mask, int act, uint8_t *q_row, uint8_t *s_row,
                                    uint8_t *q_col, uint8_t *s_col, hipStream_t stream);
mx_status mx_quantize_dgated_grouped(const void *grad, const void *x, int64_t N,
                                     const int64_t *group_rows, int G, unsigned axis_mask, int act,
                                     uint8_t *q_row, uint8_t *s_row, uint8_t *q_col,
                                     uint8_t *s_col, hipStream_t stream);

/*
 * The fused elementwise values alone, as bf16: y = pre-op(x[, grad]) for
 * op = MX_FUSE_GELU / MX_FUSE_DGELU / MX_FUSE_DSILU (x, grad and y are
 * [M][K]), the gated value for op = 0x100 | MX_GATED_SWIGLU / MX_GATED_GEGLU
 * (x is [M][2K], y is [M][K]), or the gated backward for op = 0x200 |
 * MX_GATED_SWIGLU / MX_GATED_GEGLU (x is [M][2K], grad [M][K], y [M][2K]).
 * This is the exact tensor the fused casts quantise; it is exposed so that
 * the pre-op arithmetic can be checked on its own.  Any M, K >= 1, each
 * <= 2^23 (2K <= 2^23 for gated ops), M * K <= 2^40.
 */
#define MX_OP_GATED 0x100
#define MX_OP_DGATED 0x200
mx_status mx_fused_values(const void *x, const void *grad, int64_t M, int64_t K, int op,
                          void *y, hipStream_t stream);

/*
 * Tensor absmax for NVFP4: *amax = max |x_i| over n bf16 elements, as fp32
 * (exact); a NaN when an element is NaN, else +Inf when one is infinite.
 * amax is a device pointer to one float; it is first cleared and then
 * combined with integer atomic max, so the result does not depend on
 * scheduling.  n > 0, n <= 2^40, x 16-byte aligned.
 */
mx_status mx_absmax_bf16(const void *x, int64_t n, float *amax, hipStream_t stream);

/*
 * NVFP4 quantize-transpose of x[M][K] (bf16), block size 16, any M, K >= 1,
 * each <= 2^23, M*K <= 2^40.  When 16 does not divide K (M), the last block
 * of each row (column) is partial: its scale and codes come from its own
 * elements, and a line of n codes packs into ceil(n/2) bytes, the high nibble
 * of an odd line's last byte 0.  K a multiple of 16 takes the tiled kernel,
 * for any M (with the transpose and M not a multiple of 16, its rows start
 * at any byte and a variant of the kernel writes them through a two-pair
 * stage); other K a kernel for arbitrary row alignment (same results).
 *   amax     device, one fp32: the tensor absmax the global scale is built
 *            from, as mx_absmax_bf16 computes it (on the same stream).  With
 *            a NaN or infinite amax (a tensor holding a NaN or an Inf) there
 *            is no usable global scale: every scale byte is 0x7F (the E4M3
 *            NaN), every element code 0, and S_g = amax / 2688 stays NaN or
 *            Inf.  An amax other than the tensor's absmax is outside the
 *            contract.
 *   q_row, s_row  packed E2M1 [M][ceil(K/2)] (element 2j in the low nibble
 *            of byte j), E4M3 [M][ceil(K/16)]        (iff MX_ROWWISE)
 *   q_col, s_col  the same for the transpose: [K][ceil(M/2)],
 *            [K][ceil(M/16)]                        (iff MX_COLWISE)
 *   global_scale_out  device, one fp32 receiving S_g; may be NULL
 */
mx_status nvfp4_quantize_transpose(const void *x, int64_t M, int64_t K, const float *amax,
                                   unsigned axis_mask,
                                   uint8_t *q_row, uint8_t *s_row, uint8_t *q_col, uint8_t *s_col,
                                   float *global_scale_out, hipStream_t stream);

/*
 * NVFP4 quantize-transpose with 2D scaling (the "nvfp42d" rows of the
 * quantize-transpose table): one E4M3 scale per 16 x 16 block of x (partial
 * at the right and bottom edges), from the block's amax over its elements by
 * the same chain as above; every element is coded with its block's
 * multiplier.  Arguments, layouts and errors exactly as for
 * nvfp4_quantize_transpose: the block's scale is written for each of its
 * rows in s_row and for each of its columns in s_col, so a consumer of the
 * 1D layouts reads 2D-scaled data unchanged.
 */
mx_status nvfp4_quantize_transpose_2d(const void *x, int64_t M, int64_t K, const float *amax,
                                      unsigned axis_mask,
                                      uint8_t *q_row, uint8_t *s_row, uint8_t *q_col,
                                      uint8_t *s_col, float *global_scale_out, hipStream_t stream);

/* Static string naming a status code. */
/*
 * Per-group tensor absmax for the grouped NVFP4 cast: amax[g] = max |x| over
 * the rows of group g (0 for an empty group), as fp32.  x, group_rows, G as
 * for nvfp4_quantize_transpose_grouped; amax is a device array of G floats.
 */
mx_status mx_absmax_bf16_grouped(const void *x, int64_t K, const int64_t *group_rows, int G,
                                 float *amax, hipStream_t stream);

/*
 * Grouped NVFP4 quantize-transpose: G tensors stacked along rows (the
 * operation of the group_quantize_transpose_nvfp4 row of TransformerEngine PR
 * 3291's "Important Files Changed" table, without the Hadamard transform),
 * each quantised in one launch exactly as nvfp4_quantize_transpose (or, with
 * scaling_2d = 1, nvfp4_quantize_transpose_2d) quantises a tensor of its own:
 * with its own tensor amax and global scale.
 *   x            device, bf16 [M][K], M = sum of group_rows; group g owns rows
 *                r_g .. r_g + group_rows[g] - 1
 *   group_rows   HOST array of G row counts, each >= 0; 1 <= G <= 64,
 *                0 < M <= 2^23; any K >= 1.  K a multiple of 16 takes the
 *                tiled kernel, for any counts (counts that are not multiples
 *                of 16: through its variant for transposed rows at any byte,
 *                as for nvfp4_quantize_transpose), any other K the any-shape
 *                kernel (same results)
 *   amax         device, fp32 [G]: each group's tensor amax (for example from
 *                mx_absmax_bf16_grouped)
 *   q_row, s_row [M][ceil(K/2)], [M][ceil(K/16)]: the groups' rows (the
 *                stacked layout)
 *   q_col, s_col group g's [K][ceil(rows/2)] and [K][ceil(rows/16)], the
 *                groups one after the other
 *   global_scale_out  device fp32 [G] or NULL: each group's global scale
 *                (1 for an empty group)
 * Errors as for nvfp4_quantize_transpose; MX_ERR_ENUM also for scaling_2d not
 * 0 or 1, MX_ERR_SHAPE for G out of range or a bad group size.
 */
mx_status nvfp4_quantize_transpose_grouped(const void *x, int64_t K, const int64_t *group_rows,
                                           int G, const float *amax, int scaling_2d,
                                           unsigned axis_mask, uint8_t *q_row, uint8_t *s_row,
                                           uint8_t *q_col, uint8_t *s_col,
                                           float *global_scale_out, hipStream_t stream);

const char *mx_status_str(int status);

/* MXCAST_ABI_VERSION of the built library. */
int mx_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MXCAST_H */
