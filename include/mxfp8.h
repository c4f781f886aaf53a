/*
 * mxfp8.h -- C ABI of the MI355X (gfx950) MXFP8 training cast and MXFP8 scaled
 * grouped GEMM.
 *
 * The operations are the ones the pages turn on:
 *   - the MXFP8 training cast: bf16 in, 1x32 blocks, an E8M0 scale per block
 *     rounded up ("RCEIL"), E4M3 data, with scales written straight into the
 *     layout the GEMM reads ("blocked E8M0 scales", no rearrange pass)
 *     [torchtitan PR 5334, body; ao fork PR 10 "[moe training] Add
 *     backward_override to the MXFP8 grouped GEMM", Design notes];
 *     a rowwise (dim0) and a columnwise (dim1) form [same ao page, Summary and
 *     Test plan] and a 32x32 weight-scale form [torchtitan PR 5334, body and
 *     review];
 *   - the MXFP8 scaled grouped GEMM over per-group row offsets `offs`, with
 *     offs = NULL for a dense layer ("a single API for dense and grouped",
 *     "offs=None") [torchtitan PR 5334, body], in forward, dgrad and wgrad
 *     [ao fork PR 10, Summary; pytorch/ao PR 4705 "Wire MoE and MXFP8Linear
 *     training paths to CuTeDSL by default", body].
 * The numerics follow the OCP Microscaling (MX) definition:
 *   scale exponent s = ceil(log2(amax / 448)) clamped to [-127, 127], stored as
 *   the byte s + 127; each element is encoded as E4M3 (OCP E4M3FN: bias 7, max
 *   448, NaN = S.1111.111) of x / 2^s, round-to-nearest-even, saturating. A zero
 *   block gets scale byte 0. The sign of zero is kept.
 *
 * CONVENTIONS (every entry point)
 *   - Pointers are device pointers unless stated; the caller allocates and frees
 *     every buffer, workspaces included. The library never allocates device
 *     memory and keeps no state beyond a per-device architecture check,
 *     per-process launch settings (both set up thread-safely) and the fixed
 *     per-device scratch of mx_grouped_mm_wgrad_noalloc (part of the code object).
 *   - bf16 data is passed as uint16_t bit patterns; E4M3 codes and E8M0 scales
 *     as uint8_t; `stream` is a hipStream_t (NULL = the default stream).
 *   - Work is enqueued asynchronously on `stream`. No call copies device memory
 *     to the host, reads `offs` on the host or synchronises the host, and no call
 *     records a memset, so sequences of calls can be captured into a HIP graph
 *     as they are (no warm-up call needed).
 *   - Arguments are validated on the host before anything is launched. On any
 *     error nothing is launched, a negative status is returned and
 *     mx_last_error() describes the problem (thread-local string).
 *   - Inputs must be finite. NaN or Inf input gives unspecified codes/scales.
 *   - All pointers must be 16-byte aligned; all row pitches are in elements and
 *     must make every row 16-byte aligned.
 *
 * SCALE LAYOUT ("MFMA-blocked"), used by every scale buffer below
 *   A quantized matrix Q [R x C] (C = the blocked, contiguous axis, a multiple
 *   of 32) has logical scales S [R x KB], KB = C / 32. Physically they are stored
 *   in tiles of 32 rows x 8 blocks, 256 bytes per tile, tiles ordered row-band
 *   major:
 *       KT     = ceil(KB / 8)
 *       offset(r, kb) = ((r / 32) * KT + kb / 8) * 256
 *                       + (kb % 2) * 128 + (r % 32) * 4 + (kb % 8) / 2
 *   Buffer size = mx_scale_bytes(R, C) = ceil(R / 32) * KT * 256 bytes. Bytes
 *   that no (r, kb) maps to are written as 0x7F (scale 1.0) by the casts.
 *   Why: the gfx950 block-scaled MFMA (32x32x64, fp8) takes the scale of output
 *   row r and of the k-block b (0 or 1) of one 64-wide k-step from lane r + 32*b,
 *   and a byte selector picks one byte of that lane's 32-bit scale register. With
 *   this layout lane l loads the dword at tile offset 4*l and it serves four
 *   consecutive k-steps (256 contraction elements) through bytes 0..3.
 */
#ifndef MXFP8_H_
#define MXFP8_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int mx_status;

#define MX_OK 0
#define MX_E_NULL (-1)    /* a required pointer is NULL */
#define MX_E_SHAPE (-2)   /* a size is negative, too large, or not a required multiple */
#define MX_E_ALIGN (-3)   /* a pointer or row pitch breaks the 16-byte alignment rule */
#define MX_E_LAYOUT (-4)  /* a row pitch is smaller than the row length */
#define MX_E_DTYPE (-5)   /* unknown output dtype, cast form or scale rule */
#define MX_E_DEVICE (-6)  /* no HIP device, or the current device is not gfx950 */
#define MX_E_LAUNCH (-7)  /* the kernel launch failed (see mx_last_error) */

#define MX_OUT_F32 0  /* GEMM output as float32 */
#define MX_OUT_BF16 1 /* GEMM output as bf16 (round-to-nearest-even of the fp32 sum) */

/* Bytes of the MFMA-blocked scale buffer for a [rows x cols] quantized matrix
 * (cols = the blocked axis). Returns -1 if rows < 0 or cols is not a
 * non-negative multiple of 32. Host function, no device access. */
int64_t mx_scale_bytes(int64_t rows, int64_t cols);

/* Status code as text, e.g. "MX_E_SHAPE". */
const char* mx_status_string(mx_status s);

/* Description of the last error raised on the calling thread ("" if none). */
const char* mx_last_error(void);

/* 1x32 rowwise ("dim0") cast [torchtitan PR 5334, body: 1x32 RCEIL casts
 * with blocked E8M0 scales; ao fork PR 10, Design notes].
 *   x      [rows x cols] bf16, row pitch ld_x elements (ld_x >= cols, ld_x % 8 == 0)
 *   q      [rows x cols] E4M3 codes, row pitch cols (written)
 *   scale  mx_scale_bytes(rows, cols) bytes, MFMA-blocked layout (written)
 * Blocks are 32 consecutive elements of a row. cols % 32 == 0; rows >= 0 (any
 * value). A 3D tensor [G, N, K] is cast as rows = G*N. */
mx_status mx_quantize_dim0(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, uint8_t* q,
                           uint8_t* scale, void* stream);

/* 32x1 columnwise ("dim1") cast, written transposed [ao fork PR 10, Summary
 * and Test plan: dim1-cast wgrad operands; pytorch/ao PR 4705, ghstack list:
 * 32x1 quantization].
 *   x        batch x [rows x cols] bf16; batch b starts at x + b*rows*ld_x;
 *            row pitch ld_x (ld_x >= cols, ld_x % 8 == 0)
 *   q_t      batch x [cols x rows] E4M3 codes (the transpose: blocks of 32
 *            consecutive input rows become 32 contiguous bytes), written
 *   scale_t  mx_scale_bytes(batch*cols, rows) bytes: the scales of the stacked
 *            [batch*cols x rows] matrix q_t, MFMA-blocked (written)
 * rows % 32 == 0, cols % 32 == 0, batch >= 1. Identity: dim1(X) == dim0(X^T). */
mx_status mx_quantize_dim1(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, int64_t ld_x,
                           uint8_t* q_t, uint8_t* scale_t, void* stream);

/* dim0 and dim1 in one pass: reads x once and writes both casts, exactly as
 * mx_quantize_dim0 on the stacked [batch*rows x cols] matrix plus mx_quantize_dim1
 * would [torchtitan PR 5334, body: the fused dense rowwise/columnwise cast].
 * 4.0625 bytes of HBM traffic per element instead of 2 x 3.03125.
 *   x        batch x [rows x cols] bf16; batch b starts at x + b*rows*ld_x; row
 *            pitch ld_x (ld_x >= cols, ld_x % 8 == 0)
 *   q        [batch*rows x cols] codes, row pitch cols (written)
 *   scale    mx_scale_bytes(batch*rows, cols) bytes (written)
 *   q_t      batch x [cols x rows] codes, transposed (written)
 *   scale_t  mx_scale_bytes(batch*cols, rows) bytes (written)
 * rows % 32 == 0, cols % 32 == 0, batch >= 1; ld_x < 2^25 and rows < 2^29 (the
 * kernel addresses a 32-row sub-tile through 32-bit offsets), else MX_E_SHAPE. */
mx_status mx_quantize_dim0_dim1(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, int64_t ld_x,
                                uint8_t* q, uint8_t* scale, uint8_t* q_t, uint8_t* scale_t, void* stream);

/* Forms and scale rules of mx_quantize_ex. */
#define MX_FORM_DIM0 1
#define MX_FORM_DIM1 2
#define MX_FORM_STREAM_T 4 /* with both forms: write the transposed codes with non-temporal
                              stores, for a q_t that is read only after much other traffic
                              (a weight's q_t read by dgrad, the tokens' by wgrad): the
                              caches then keep the row-wise codes the next GEMM reads.
                              Results are identical; only where the bytes are cached differs */
#define MX_SCALE_RCEIL 0 /* ceil(log2(amax / 448)): the rule of the other casts */
#define MX_SCALE_FLOOR 1 /* floor(log2(amax)) - 8 (the OCP default): the block maximum
                            can exceed 448 after scaling and saturates to 448 */

/* Casts with a choice of form and scale rule [ao fork PR 10, Known follow-ups:
 * FLOOR is reachable next to RCEIL]. forms = MX_FORM_DIM0, MX_FORM_DIM1 or both
 * (the one-pass cast), optionally with MX_FORM_STREAM_T; arguments as mx_quantize_dim0 (on the stacked
 * [batch*rows x cols] matrix), mx_quantize_dim1 and mx_quantize_dim0_dim1. Outputs
 * of a form not requested may be NULL. rows % 32 == 0 when MX_FORM_DIM1 is
 * requested; cols % 32 == 0 always; both forms at once take the one-pass cast's
 * limits (ld_x < 2^25, rows < 2^29). With MX_SCALE_RCEIL the results equal those of
 * the other entry points. An unknown forms or scale_mode value, or MX_FORM_STREAM_T
 * without both forms, is MX_E_DTYPE. */
mx_status mx_quantize_ex(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, int64_t ld_x, int forms,
                         int scale_mode, uint8_t* q, uint8_t* scale, uint8_t* q_t, uint8_t* scale_t, void* stream);

/* 32x32 weight cast: one scale per 32x32 tile [torchtitan PR 5334, body
 * ("32x32 RCEIL weight-scale policy") and review (the square weight kernel is
 * RCEIL-only)]. One set of codes, quantized with the tile scale, is written
 * in both orientations (the rowwise and columnwise copies of one weight).
 *   w          batch x [n x k] bf16, row pitch ld_w (ld_w >= k, ld_w % 8 == 0)
 *   q          batch x [n x k] codes (written)
 *   q_t        batch x [k x n] the same codes transposed (written; may be NULL)
 *   scale_row  mx_scale_bytes(batch*n, k): scales of q, tile byte repeated over
 *              the tile's 32 rows (written)
 *   scale_col  mx_scale_bytes(batch*k, n): scales of q_t (written; NULL iff q_t
 *              is NULL)
 * n % 32 == 0, k % 32 == 0, batch >= 1. */
mx_status mx_quantize_weight_32x32(const uint16_t* w, int64_t batch, int64_t n, int64_t k, int64_t ld_w,
                                   uint8_t* q, uint8_t* q_t, uint8_t* scale_row, uint8_t* scale_col,
                                   void* stream);

/* Grouped GEMM forward: out[r, :] = deq(a)[r, :] . deq(b_g)^T for r in group g
 * [ao fork PR 10, Summary (the MXFP8 grouped GEMM); torchtitan PR 5334, body
 * (offs=None for dense)].
 *   a, a_s    [m x k] codes + mx_scale_bytes(m, k) scales (dim0 of the tokens)
 *   b, b_s    [groups*n x k] codes (group g's [n x k] weight at rows g*n) +
 *             mx_scale_bytes(groups*n, k) scales
 *   offs      device int32[groups]: inclusive cumulative group ends; group g is
 *             rows [offs[g-1], offs[g]) with offs[-1] = 0. NULL = one dense group
 *             (groups must be 1). Caller precondition (not checked on the host, offs
 *             stays on the device; mx_check_offs tests it on the device):
 *             non-decreasing, every entry % 32 == 0, offs[G-1] <= m.
 *             Rows past offs[G-1] belong to no group and are left unwritten (the
 *             buffers of mx_pad_token_groups end with such rows). The kernel reads
 *             the ends as their running maximum clamped into [0, m], so an
 *             out-of-contract offs gives unspecified output rows but no access
 *             outside a, b, their scales and out (the same holds for dgrad, wgrad,
 *             whose token ranges are clamped into [0, m], the padded calls and the
 *             bf16 calls).
 *   out       [m x n], float32 or bf16 per out_dtype, row pitch n (written)
 * k % 32 == 0 (k need not be a multiple of 128: the tail is zero-padded inside
 * the kernel); m >= 0; n >= 1; if groups > 1, n % 32 == 0. fp32 accumulation.
 * A buffer that holds no element (a, a_s, out when m == 0; for wgrad the two
 * operands when the contraction m == 0, whose dw is then all zeros) may be NULL;
 * the same holds for every other call's empty buffers.
 * Extent limits (all three GEMM calls, MX_E_SHAPE otherwise): the contraction
 * length (k here, n for dgrad, m for wgrad) is at most 2^22, and each operand's
 * scale buffer (mx_scale_bytes of its rows and the contraction) is below 2^31
 * bytes; the kernels address operands with 32-bit buffer offsets. */
mx_status mx_grouped_mm_fwd(const uint8_t* a, const uint8_t* a_s, const uint8_t* b, const uint8_t* b_s,
                            const int32_t* offs, int32_t groups, int64_t m, int64_t n, int64_t k, void* out,
                            int out_dtype, void* stream);

/* Grouped GEMM dgrad: dx[r, :] = deq(dy)[r, :] . deq(W_g) for r in group g
 * [ao fork PR 10, Summary: dgrad from the dim0-cast grad_out].
 *   dy, dy_s     [m x n] codes + mx_scale_bytes(m, n) (dim0 of grad_out)
 *   w_t, w_t_s   [groups*k x n]: W_g^T per group (the dim1 cast of the
 *                [groups, n, k] weight, or q_t of the 32x32 cast) +
 *                mx_scale_bytes(groups*k, n)
 *   offs, groups as for mx_grouped_mm_fwd
 *   dx           [m x k] (written)
 * n % 32 == 0 (the contraction); if groups > 1, k % 32 == 0. */
mx_status mx_grouped_mm_dgrad(const uint8_t* dy, const uint8_t* dy_s, const uint8_t* w_t, const uint8_t* w_t_s,
                              const int32_t* offs, int32_t groups, int64_t m, int64_t n, int64_t k, void* dx,
                              int out_dtype, void* stream);

/* Grouped GEMM wgrad: dw[g] = deq(dy_t)[:, rows_g] . deq(x_t)[:, rows_g]^T; an
 * empty group gives zeros [ao fork PR 10, Summary and Test plan: wgrad from
 * dim1 casts of grad_out and input; pytorch/ao PR 4705, ghstack list: K-groups].
 *   dy_t, dy_t_s  [n x m] codes (dim1 of grad_out) + mx_scale_bytes(n, m)
 *   x_t, x_t_s    [k x m] codes (dim1 of the input) + mx_scale_bytes(k, m)
 *   offs, groups  group g contracts over rows [offs[g-1], offs[g]) of m; NULL =
 *                 one group over all m. Same caller preconditions as fwd; rows
 *                 past offs[G-1] are not read.
 *   dw            [groups x n x k] (written, every element)
 *   workspace, workspace_bytes  caller memory (16-byte aligned; NULL, 0 allowed)
 *                 for split contractions, below
 * m % 32 == 0 (the contraction), n >= 1, k >= 1.
 * Split contraction: when the output has fewer 256 x 256 tiles than the device
 * has compute units (narrow layers), each group's contraction can be split at
 * 256-token window boundaries into S parts (enough to fill the device once, at
 * most 16): fp32 partials go to the workspace and a second kernel sums them in
 * split order, so results are deterministic. It needs
 * mx_grouped_mm_wgrad_workspace_bytes(groups, m, n, k, 0) bytes (S * groups * n
 * * k * 4, rounded up to 16); with a smaller workspace, or none, the contraction
 * runs unsplit (same sums up to the fp32 rounding of the partials; slower on
 * narrow outputs). The workspace is in use until the call's work on `stream`
 * has finished: calls that may overlap need workspaces of their own. */
mx_status mx_grouped_mm_wgrad(const uint8_t* dy_t, const uint8_t* dy_t_s, const uint8_t* x_t, const uint8_t* x_t_s,
                              const int32_t* offs, int32_t groups, int64_t m, int64_t n, int64_t k, void* dw,
                              int out_dtype, void* workspace, int64_t workspace_bytes, void* stream);

/* mx_grouped_mm_wgrad for callers that cannot allocate memory (code under HIP
 * graph capture that must not allocate, tight serving loops, harnesses that forbid
 * allocation): the same arguments without a workspace, the same results as
 * mx_grouped_mm_wgrad with a workspace of mx_grouped_mm_wgrad_workspace_bytes
 * (bit for bit). A split contraction keeps its fp32 partials in a fixed scratch
 * array inside the library, MX_WGRAD_NOALLOC_SCRATCH_BYTES (64 MiB) per device,
 * held until the process ends: the most any split can need (at most one round of
 * 256 output tiles of 256 x 256 fp32 partials), so no valid call is refused; a
 * call needing more would return MX_E_SHAPE. Every call on one device shares that
 * device's scratch:
 * calls whose work may overlap (different streams, no event between them) race, so
 * the caller orders them. Nothing is allocated, synchronised or cleared. */
#define MX_WGRAD_NOALLOC_SCRATCH_BYTES (64 * 1024 * 1024)
mx_status mx_grouped_mm_wgrad_noalloc(const uint8_t* dy_t, const uint8_t* dy_t_s, const uint8_t* x_t,
                                      const uint8_t* x_t_s, const int32_t* offs, int32_t groups, int64_t m, int64_t n,
                                      int64_t k, void* dw, int out_dtype, void* stream);

/* Workspace bytes with which mx_grouped_mm_wgrad (bf16_operands = 0) or
 * mx_grouped_mm_bf16_wgrad (bf16_operands = 1) splits its contraction; 0 when the
 * call does not split (enough output tiles, or too short a contraction). Host
 * function, no device access; -1 for arguments outside the calls' limits. */
int64_t mx_grouped_mm_wgrad_workspace_bytes(int32_t groups, int64_t m, int64_t n, int64_t k, int bf16_operands);

/* ---- Backward override arms ----
 * The backward of the MXFP8 grouped GEMM may take its gradients from elsewhere
 * while the quantized forward is kept [ao fork PR 10, Design notes]: the
 * high-precision arm from the saved bf16 input and weight, the dequantized arm
 * from the forward's quantized operands dequantized to bf16 (with their logical,
 * pre-blocking scales), both through bf16 grouped GEMMs (fp32 accumulation):
 *   dX = dY . W_g per row group          -> mx_grouped_mm_bf16_dgrad(dy, W_g^T)
 *   dW_g = dY_g^T . X_g per group        -> mx_grouped_mm_bf16_wgrad(dy^T, X^T)
 * Every GEMM operand is contraction-contiguous; the transposed operands come from
 * mx_transpose_bf16 (saved bf16 tensors) or mx_dequantize(transpose = 1) (codes). */

/* Dequantizes codes to bf16: out = value(code) * 2^(byte - 127) rounded to
 * nearest even in bf16 (exact unless below 2^-126 or at 2^128 and above, which
 * gives infinity; NaN codes give a bf16 NaN).
 *   q, scale  [batch*rows x cols] codes (row pitch cols) and their
 *             mx_scale_bytes(batch*rows, cols) MFMA-blocked scales (a dim0 cast)
 *   transpose 0: out [batch*rows x cols]; 1: out [batch][cols][rows] (each
 *             batch's matrix transposed; rows % 8 == 0)
 *   out       bf16 bit patterns (written)
 * cols % 32 == 0. */
mx_status mx_dequantize(const uint8_t* q, const uint8_t* scale, int64_t batch, int64_t rows, int64_t cols,
                        int transpose, uint16_t* out, void* stream);

/* Logical view of MFMA-blocked scales: logical[r * (cols/32) + kb] = the byte
 * of row r, block kb (the dequantized arm needs pre-blocking scales [ao fork
 * PR 10, Design notes]). cols % 32 == 0. */
mx_status mx_scales_to_logical(const uint8_t* scale, int64_t rows, int64_t cols, uint8_t* logical, void* stream);

/* bf16 transpose: x [batch][rows][cols] (row pitch ld_x, batches contiguous at
 * rows * ld_x) -> out [batch][cols][rows]. rows % 8 == 0, cols % 8 == 0. */
mx_status mx_transpose_bf16(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols, int64_t ld_x, uint16_t* out,
                            void* stream);

/* bf16 grouped GEMMs: the same three calls as the MXFP8 ones with bf16 operands
 * (bit patterns, no scales) and fp32 accumulation; out_dtype as there.
 *   fwd:   out [m x n] = a [m x k] . b_g [n x k]^T for the rows of group g
 *   dgrad: dx [m x k] = dy [m x n] . (w_t_g [k x n])^T, w_t = [groups*k x n]
 *   wgrad: dw [groups x n x k], dw[g] = dy_t[:, rows_g] . x_t[:, rows_g]^T,
 *          dy_t [n x m], x_t [k x m]; an empty group gives zeros
 * offs as for the MXFP8 calls but with no alignment: any non-decreasing ends with
 * offs[G-1] <= m (group edges inside a 16-byte chunk of the contraction are
 * masked element by element). The contraction (k, n, m respectively) is a
 * multiple of 8 and at most 2^21. The wgrad takes a workspace as
 * mx_grouped_mm_wgrad does (size from mx_grouped_mm_wgrad_workspace_bytes with
 * bf16_operands = 1). */
mx_status mx_grouped_mm_bf16_fwd(const uint16_t* a, const uint16_t* b, const int32_t* offs, int32_t groups, int64_t m,
                                 int64_t n, int64_t k, void* out, int out_dtype, void* stream);
mx_status mx_grouped_mm_bf16_dgrad(const uint16_t* dy, const uint16_t* w_t, const int32_t* offs, int32_t groups,
                                   int64_t m, int64_t n, int64_t k, void* dx, int out_dtype, void* stream);
mx_status mx_grouped_mm_bf16_wgrad(const uint16_t* dy_t, const uint16_t* x_t, const int32_t* offs, int32_t groups,
                                   int64_t m, int64_t n, int64_t k, void* dw, int out_dtype, void* workspace,
                                   int64_t workspace_bytes, void* stream);

/* ---- Token-group padding (group sizes that are not multiples of 32) ----
 * The grouped GEMM needs every group to start on a 32-row boundary (its scales
 * and its wgrad blocks run in 32-row units). Padding moves each token group to
 * such a boundary before the casts and unpadding gathers the GEMM outputs back
 * [pytorch/ao PR 4705, ghstack list: pad/unpad kernels; ao fork PR 10, Known
 * follow-ups: padded token groups feed padded offsets to the grouped GEMM].
 * Group g's rows [offs[g-1], offs[g]) move, in order, to the run starting at
 * offs_pad[g-1], offs_pad[g] = sum over j <= g of (size_j rounded up to 32);
 * every other row of the padded buffer is zero. The padded buffer's size depends
 * only on (rows, groups), so nothing is read back to the host.
 *
 * offs here may hold any non-decreasing ends with offs[G-1] <= rows (no 32-row
 * alignment needed). The kernels clamp each end into [0, rows] and make the
 * sequence non-decreasing while reading it, so an out-of-contract offs moves the
 * wrong rows but never addresses memory outside the buffers. groups <= 1024.
 * A row buffer with zero rows may be NULL. */

/* Device check of offs for the grouped calls (a debugging aid for callers whose
 * offs come from elsewhere; the GEMMs themselves never read offs on the host).
 *   offs      device int32[groups], groups >= 1
 *   m         rows (M-grouped calls) or tokens (wgrad) the ends must stay within
 *   multiple  required divisor of every end: 32 for the MXFP8 calls, 1 for the
 *             bf16 calls and the padding calls
 *   result    device int32[2] (written, asynchronously on `stream`): result[0] =
 *             OR of MX_OFFS_DECREASING, MX_OFFS_NOT_MULTIPLE, MX_OFFS_OUT_OF_RANGE
 *             over all groups (0 = offs meets the preconditions), result[1] = the
 *             first group with a violation, or -1.
 * A group's end is compared with the previous end (0 before group 0). Errors:
 * MX_E_SHAPE (groups < 1, m outside [0, 2^31], multiple < 1), MX_E_NULL,
 * MX_E_ALIGN (a pointer not 4-byte aligned). */
#define MX_OFFS_DECREASING 1    /* an end below the previous one */
#define MX_OFFS_NOT_MULTIPLE 2  /* an end that is not a multiple of `multiple` */
#define MX_OFFS_OUT_OF_RANGE 4  /* an end below 0 or above m */
mx_status mx_check_offs(const int32_t* offs, int32_t groups, int64_t m, int32_t multiple, int32_t* result,
                        void* stream);

/* Measurement aid, not part of the computation: a register-only loop of the
 * block-scaled MFMA (v_mfma_scale_f32_32x32x64_f8f6f4, fixed pseudo-random E4M3
 * operands, unit scales) on every SIMD, so a caller can time the MXFP8 rate this
 * part sustains and report the GEMMs against it beside the nominal peak.
 *   iters  loop trips, 1 <= iters < 2^31; one call performs iters * 2^30 flops
 *   sink   device float[256] (written with checksums; keeps the loop)
 * Errors: MX_E_SHAPE, MX_E_NULL, MX_E_ALIGN (sink not 4-byte aligned). */
mx_status mx_probe_mfma(int64_t iters, float* sink, void* stream);

/* Measurement aid, not part of the computation: ONE block-scaled MFMA of either
 * full-rate form on caller-given operands, so tests can pin the instruction's
 * arithmetic (which sets how closely the GEMMs can match an exact fp32 sum).
 *   form     MX_PROBE_32X32X64 (v_mfma_scale_f32_32x32x64_f8f6f4: R = 32, K = 64)
 *            or MX_PROBE_16X16X128 (v_mfma_scale_f32_16x16x128_f8f6f4: R = 16,
 *            K = 128), optionally | MX_PROBE_SWAP (b is the instruction's first
 *            operand, the order the GEMM kernels use)
 *   a, b     device [R x K] E4M3 codes, row-major
 *   a_scale, b_scale  device [R x K/32] E8M0 bytes, row-major (block kb of row r)
 *   c        device [R x R] float32 accumulator input, row-major
 *   d        device [R x R] float32 (written): d[i][j] = c[i][j] + the
 *            instruction's dot product of row i of a with row j of b
 * One wave; asynchronous on `stream`. Errors: MX_E_DTYPE (form), MX_E_NULL,
 * MX_E_ALIGN (c or d not 4-byte aligned). */
#define MX_PROBE_32X32X64 0
#define MX_PROBE_16X16X128 1
#define MX_PROBE_SWAP 2
mx_status mx_probe_mfma_dot(int form, const uint8_t* a, const uint8_t* a_scale, const uint8_t* b,
                            const uint8_t* b_scale, const float* c, float* d, void* stream);

/* Rows of the padded buffer for any split of `rows` rows into `groups` groups:
 * rows + 31 * groups rounded up to a multiple of 256 (a group grows by at most 31
 * rows; the rounding keeps the token axis, which is the row pitch of the dim1
 * codes fed to wgrad, a whole number of 256-byte windows, so no GEMM load
 * straddles cache lines). -1 if rows < 0, rows > 2^31 or groups < 1. */
int64_t mx_padded_rows(int64_t rows, int32_t groups);

/* Pads bf16 token rows.
 *   x         [rows x cols] bf16, row pitch ld_x (ld_x % 8 == 0), cols % 8 == 0
 *   offs      device int32[groups], unpadded group ends (see above)
 *   x_pad     [rows_pad x cols] bf16, row pitch cols (written, every row)
 *   rows_pad  >= mx_padded_rows(rows, groups), < 2^31
 *   offs_pad  device int32[groups] (written): padded group ends, each % 32 == 0,
 *             offs_pad[G-1] <= rows_pad; pass it as `offs` to the casts' users
 *             (the grouped GEMM calls) with m = rows_pad.
 * rows + 31 * groups < 2^31. */
mx_status mx_pad_token_groups(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, const int32_t* offs,
                              int32_t groups, uint16_t* x_pad, int64_t rows_pad, int32_t* offs_pad, void* stream);

/* Unpads rows (the inverse gather): y[offs[g-1] + i] = y_pad[offs_pad[g-1] + i]
 * for every row of group g, offs_pad being recomputed from offs as above.
 *   y_pad     [rows_pad x cols], row pitch ld_pad, element type `dtype`
 *             (MX_OUT_F32 or MX_OUT_BF16): e.g. a grouped GEMM output
 *   offs      the same unpadded group ends given to mx_pad_token_groups
 *   y         [rows x cols], row pitch ld_y (rows of the groups written; rows
 *             past offs[G-1] untouched)
 * cols * element size and both pitches * element size multiples of 16 bytes;
 * rows_pad >= mx_padded_rows(rows, groups). */
mx_status mx_unpad_token_groups(const void* y_pad, int64_t rows_pad, int64_t cols, int64_t ld_pad,
                                const int32_t* offs, int32_t groups, void* y, int64_t rows, int64_t ld_y, int dtype,
                                void* stream);

/* The padding fused into the casts and the GEMM outputs: no padded bf16 copy of the
 * tokens or grad_out is written, and the forward / dgrad outputs come out unpadded.
 *
 * One-pass dim0 + dim1 cast of the padded rows: the codes and scales are those of
 * mx_quantize_dim0_dim1 applied to the output of mx_pad_token_groups(x, offs), and
 * offs_pad is written as there.
 *   x         [rows x cols] bf16 (pitch ld_x), offs the unpadded group ends
 *   q, scale  [rows_pad x cols] + mx_scale_bytes(rows_pad, cols) (written)
 *   q_t, scale_t  [cols x rows_pad] + mx_scale_bytes(cols, rows_pad) (written)
 * rows_pad >= mx_padded_rows(rows, groups), a multiple of 32; cols % 32 == 0;
 * ld_x < 2^25 and rows_pad < 2^29 as for mx_quantize_dim0_dim1. */
mx_status mx_pad_quantize_dim0_dim1(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x,
                                    const int32_t* offs, int32_t groups, int64_t rows_pad, uint8_t* q,
                                    uint8_t* scale, uint8_t* q_t, uint8_t* scale_t, int32_t* offs_pad,
                                    void* stream);

/* mx_pad_quantize_dim0_dim1 with flags: 0, or MX_FORM_STREAM_T to write the transposed
 * codes with non-temporal stores (as for mx_quantize_ex; identical results). Any other
 * flags value is MX_E_DTYPE. */
mx_status mx_pad_quantize_ex(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld_x, const int32_t* offs,
                             int32_t groups, int64_t rows_pad, int flags, uint8_t* q, uint8_t* scale, uint8_t* q_t,
                             uint8_t* scale_t, int32_t* offs_pad, void* stream);

/* Forward / dgrad on padded token rows with unpadded outputs: the result equals
 * mx_unpad_token_groups of mx_grouped_mm_fwd(..., offs_pad, m = m_pad, ...) (resp.
 * dgrad): row offs_pad[g-1] + i of group g is written to row offs[g-1] + i of out
 * [m x n] (dx [m x k]) for i < offs[g] - offs[g-1]; no other row is written.
 *   offs_pad  padded group ends (from mx_pad_quantize_dim0_dim1 or
 *             mx_pad_token_groups); offs the unpadded ends; m <= m_pad
 * Other arguments and conditions as for mx_grouped_mm_fwd / mx_grouped_mm_dgrad
 * with m = m_pad for the operands. */
mx_status mx_grouped_mm_fwd_padded(const uint8_t* a, const uint8_t* a_s, const uint8_t* b, const uint8_t* b_s,
                                   const int32_t* offs_pad, const int32_t* offs, int32_t groups, int64_t m_pad,
                                   int64_t m, int64_t n, int64_t k, void* out, int out_dtype, void* stream);
mx_status mx_grouped_mm_dgrad_padded(const uint8_t* dy, const uint8_t* dy_s, const uint8_t* w_t, const uint8_t* w_t_s,
                                     const int32_t* offs_pad, const int32_t* offs, int32_t groups, int64_t m_pad,
                                     int64_t m, int64_t n, int64_t k, void* dx, int out_dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MXFP8_H_ */
