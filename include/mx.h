/*
 * libmxfp4 — OCP MX v1.0 MXFP4 quantizer and block-scaled GEMMs for MI355X (gfx950).
 *
 * C ABI.  Every pointer argument marked "device" is a device (HBM) pointer that
 * the caller owns; the library never allocates, frees or synchronizes.  Every
 * call only validates its arguments on the host and enqueues kernels on
 * `stream` (a hipStream_t; NULL = the null stream), so it returns before the
 * GPU work finishes.  On an invalid argument a call returns a non-zero
 * mx_status, records a message for mx_last_error() and launches nothing; a
 * launch failure reported by the HIP runtime returns MX_ERR_HIP.  No C++
 * exception crosses this interface.
 *
 * Data format ("MXFP4", AI Wiki, §Format specification; §Use in models /
 * gpt-oss):
 *   - a block is 32 elements sharing one E8M0 scale byte (value 2^(s-127),
 *     s = 0xFF is NaN and poisons the whole block);
 *   - elements are 4-bit E2M1 codes (bit 3 sign, 2 exponent bits, 1 mantissa
 *     bit, bias 1: magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6);
 *   - an MX operand is K-major: `codes` is [rows, K/2] bytes with element 2j of
 *     a row in the low nibble of byte j and element 2j+1 in the high nibble;
 *     `scales` is stored apart, [rows, K/32] bytes for 1-D blocks (32
 *     consecutive elements of a row) or [rows/32, K/32] bytes for 2-D blocks
 *     (32x32 tiles of 32 rows by 32 elements).
 *   136 bits per 1-D block: 4.25 bits per value.
 *
 * The other MX v1.0 element types ("MXFP4", AI Wiki, §Place in the MX family:
 * MXFP8 with FP8 E4M3 or E5M2 elements, MXFP6 with FP6 E2M3 or E3M2, all with
 * 32-element blocks and an E8M0 scale) are selected per operand by
 * mx_tensor.elem.  Their codes follow the OCP element definitions (bias
 * 2^(e-1)-1, subnormals; E4M3 has no Inf and S.1111.111 is NaN, largest
 * normal 448; E5M2 is IEEE-like, largest normal 57344; FP6 has no Inf/NaN,
 * largest normals 7.5 (E2M3) and 28 (E3M2)).  Storage is K-major like MXFP4:
 * FP8 rows are K bytes (byte k = element k); FP6 rows are 3K/4 bytes with
 * element k at bits 6k .. 6k+5 of the row, little-endian (a block fills 24
 * bytes); scales are laid out as for MXFP4.
 */
#ifndef LIBMXFP4_MX_H
#define LIBMXFP4_MX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MX_OK = 0,
  MX_ERR_INVALID_ARG = 1,  /* bad shape, stride, pointer, alignment or enum */
  MX_ERR_UNSUPPORTED = 2,  /* valid request this build does not implement   */
  MX_ERR_HIP = 3           /* the HIP runtime reported an error             */
} mx_status;

typedef enum { MX_DT_F32 = 0, MX_DT_BF16 = 1 } mx_dtype;

/* Blocking axis of the SOURCE tensor [R, C] given to mx_quantize. */
typedef enum {
  MX_AXIS_LAST = 0,  /* blocks along C: output [R, C], K = C                      */
  MX_AXIS_DIM0 = 1   /* blocks along R: output is the quantized transpose [C, R], K = R */
} mx_axis;

typedef enum { MX_BLOCK_1D = 0, MX_BLOCK_2D = 1 } mx_block;

/* Element type of an MX operand (mx_tensor.elem). */
typedef enum {
  MX_ELEM_E2M1 = 0,  /* FP4, MXFP4 (the default)   */
  MX_ELEM_E4M3 = 1,  /* FP8, MXFP8                 */
  MX_ELEM_E5M2 = 2,  /* FP8, MXFP8                 */
  MX_ELEM_E2M3 = 3,  /* FP6, MXFP6                 */
  MX_ELEM_E3M2 = 4   /* FP6, MXFP6                 */
} mx_elem;

typedef enum {
  MX_ROUND_RNE = 0,  /* round to nearest, ties to even mantissa bit, saturate at +-6 */
  MX_ROUND_SR = 1,   /* stochastic rounding with 16 Philox4x32-10 bits per element   */
  MX_ROUND_SR8 = 2   /* stochastic rounding with 8 bits per element (a cheaper option;
                        rounds up with probability ceil(256 f) / 256, a bias of less
                        than 2^-8 of the step): element p takes byte (p & 3) of word
                        ((p >> 2) & 3) of the Philox call with q = p >> 4 and rounds up
                        iff that byte r satisfies r < f * 2^8                         */
} mx_round;

/*
 * Block scale rule.  The shared exponent of a block with largest magnitude
 * amax (after the optional transform):
 *   MX_SCALE_FLOOR        floor(log2 amax) - 2, the reference rule ("MXFP4",
 *                         AI Wiki, §Conversion rules); the scaled block maximum
 *                         lies in [4, 8) and values scaling into (6, 8) clip to
 *                         6 (§Clipping in the reference algorithm).
 *   MX_SCALE_ROUND_UP     ceil(log2(amax / 6)): the decode scale rounded up to
 *                         the next power of two so that nothing saturates (the
 *                         alternative §Clipping in the reference algorithm
 *                         attributes to NVIDIA's NVFP4 pretraining report); the
 *                         scaled maximum lies in (3, 6].  Computed exactly as
 *                         floor(log2 amax) - 2 + (mantissa of amax > 1.5).
 *   MX_SCALE_PRESCALE_3_4 the reference rule's scale, taken from the block as
 *                         given; every element is then multiplied by 0.75 (one
 *                         float32 multiply, after the transform) before it is
 *                         divided by that scale, so the scaled maximum lies in
 *                         [3, 6) and no element clips (Tseng, Yu, Park,
 *                         "Training LLMs with MXFP4", in the table of "MXFP4",
 *                         AI Wiki, §Training with MXFP4).  The operand then
 *                         encodes 0.75 x; a product of two such operands is
 *                         9/16 of x.y and the caller rescales.
 * All rules clamp the exponent to [-127, 127]; NaN/Inf blocks take 0xFF.
 */
typedef enum { MX_SCALE_FLOOR = 0, MX_SCALE_ROUND_UP = 1, MX_SCALE_PRESCALE_3_4 = 2 } mx_scale_mode;

/* One MX operand, K-major (see the format notes above).  All fields are
 * read-only to the library; the buffers are the caller's. */
typedef struct {
  uint8_t* codes;     /* device; [rows, K*bits/8] bytes (MXFP4: K/2), row stride ld_codes bytes */
  uint8_t* scales;    /* device; 1-D: [rows, K/32]; 2-D: [rows/32, K/32]; row stride ld_scales bytes */
  int64_t rows;       /* logical rows (M or N of a GEMM)                            */
  int64_t K;          /* logical elements per row, a multiple of 32                  */
  int64_t ld_codes;   /* bytes between rows of codes, >= K*bits/8                    */
  int64_t ld_scales;  /* bytes between rows of scales, >= K/32                       */
  int32_t block;      /* mx_block                                                    */
  int32_t elem;       /* mx_elem (0: MXFP4); codes rows hold K * bits / 8 bytes       */
} mx_tensor;

/* Quantizer settings. */
typedef struct {
  int32_t axis;            /* mx_axis                                             */
  int32_t block;           /* mx_block                                            */
  int32_t rounding;        /* mx_round                                            */
  int32_t use_rht;         /* 1: apply the 32-point randomized Hadamard transform */
  uint32_t rht_sign_mask;  /* bit i set: negate element i of every block first   */
  uint32_t scale_mode;     /* mx_scale_mode (0: the reference rule)               */
  uint64_t philox_seed;    /* SR: Philox key = (seed mod 2^32, seed >> 32)        */
  uint64_t philox_offset;  /* SR: counter words 2,3 = (offset mod 2^32, offset >> 32) */
} mx_quant_cfg;

/*
 * mx_quantize — MX conversion of a bf16/fp32 tensor (MXFP4 by default; the
 * element type is out->elem).
 *
 * Follows "MXFP4", AI Wiki, §Conversion rules and §Clipping in the reference
 * algorithm: per block, the shared exponent is floor(log2(amax)) - 2 clamped
 * to [-127, 127] (scale byte = exponent + 127; amax = 0 gives byte 0; a block
 * holding NaN or Inf gets byte 0xFF and all-zero codes); each element is
 * divided by the scale with one float32 multiply and rounded to E2M1 by RNE
 * (ties to the even mantissa bit, saturating to +-6, sign of zero kept) or by
 * stochastic rounding.  Options from "MXFP4", AI Wiki, §Training with MXFP4
 * and "Training an MoE LLM in MXFP4" (summary): the 32-point randomized
 * Hadamard transform y = c*H32*(d.x) (Sylvester order, d from rht_sign_mask,
 * c = float32(1/sqrt(32)), float32 stages h = 1,2,4,8,16 then the multiply by
 * c), stochastic rounding (element p = row_out*K + k of the output uses the
 * 16-bit half (p & 1) of word ((p >> 1) & 3) of Philox4x32-10 with counter
 * (q mod 2^32, q >> 32, offset mod 2^32, offset >> 32), q = p >> 3, and rounds
 * up iff those bits r satisfy r < f*2^16 for the fraction f of the way from
 * the lower to the upper grid point), and 1-D or 2-D (32x32) blocks.
 *
 *   src      device; R x C elements of src_dtype (mx_dtype), row stride ld_src
 *            ELEMENTS (>= C); blocks along the last dim: 16-byte aligned base,
 *            ld_src a multiple of 8; along dim 0: any element-aligned base
 *            and stride.
 *   cfg      host; quantizer settings.
 *   out      host struct describing device buffers the caller allocated:
 *            rows = R (LAST) or C (DIM0), K = C (LAST) or R (DIM0),
 *            block = cfg->block, ld_codes >= K/2, ld_scales >= K/32,
 *            codes 16-byte aligned with ld_codes a multiple of 16.
 *   Requires K % 32 == 0; 2-D blocks need rows % 32 == 0.  R = 0 or C = 0 is
 *   a no-op.  Reads only src, writes only out's buffers.  Size limits (else
 *   MX_ERR_UNSUPPORTED, nothing launched): last dim at most 2^32 - 256
 *   blocks; dim-0 at most 65535*128 source rows and 32 source rows spanning
 *   < 4 GiB.
 *   Other element types (out->elem != MX_ELEM_E2M1): the same steps with that
 *   type's grid: the shared exponent is floor(log2(amax)) - emax, emax the
 *   exponent of the type's largest power of two (8 E4M3, 15 E5M2, 2 E2M3,
 *   4 E3M2, per §Conversion rules), elements round to nearest even (or
 *   stochastically, the same 16-bit draws) and saturate at the largest
 *   normal; the round-up rule uses the largest normal in place of 6.  1-D or
 *   2-D blocks, either axis; ld_codes >= K*bits/8.
 */
mx_status mx_quantize(const void* src, int32_t src_dtype, int64_t R, int64_t C, int64_t ld_src,
                      const mx_quant_cfg* cfg, const mx_tensor* out, void* stream);

/*
 * mx_quantize_gather — mx_quantize of rows gathered by index, 1-D blocks along
 * the last dim: output row i is the quantization of source row rows[i].  This
 * is the front end of an MoE layer ("Training an MoE LLM in MXFP4", summary;
 * "MXFP4", AI Wiki, §Use in models): the routed rows (each token once per
 * expert it is sent to, grouped by expert) are quantized straight from the
 * token activations, so the routed bf16 copy is never stored.  The result
 * equals mx_quantize of the gathered tensor, stochastic-rounding draws
 * included (they follow the output element index row_out*K + k).
 *
 *   src      device; R_src x C elements of src_dtype, row stride ld_src
 *            elements (>= C), 16-byte aligned, ld_src a multiple of 8.
 *   rows     device; int32 [rows_out], the source row of each output row.  An
 *            index outside [0, R_src) gives that output row NaN blocks (scale
 *            byte 0xFF, codes 0); it is never dereferenced.
 *   cfg      host; axis must be MX_AXIS_LAST and block MX_BLOCK_1D
 *            (else MX_ERR_UNSUPPORTED); the other settings as in mx_quantize.
 *   out      host struct of device buffers: rows = rows_out, K = C, 1-D,
 *            MXFP4 (other element types return MX_ERR_UNSUPPORTED).
 *   Requires C % 32 == 0; rows_out = 0 or C = 0 is a no-op; at most
 *   2^32 - 256 blocks per call.  Reads only src and rows, writes only out.
 */
mx_status mx_quantize_gather(const void* src, int32_t src_dtype, int64_t R_src, int64_t C, int64_t ld_src,
                             const int32_t* rows, int64_t rows_out, const mx_quant_cfg* cfg,
                             const mx_tensor* out, void* stream);

/*
 * mx_quantize_scatter — the same MoE front end driven from the token side:
 * each source row is quantized once (1-D blocks along the last dim, RNE) and
 * its codes and scale bytes are stored to each of its k destination rows
 * dest[t*k + j].  A row's RNE codes do not depend on its destination, so when
 * every output row is some dest entry this equals mx_quantize_gather with the
 * inverse index, while reading each token row once instead of k times
 * ("MXFP4", AI Wiki, §Use in models: MoE weights and activations in MXFP4).
 *
 *   src      device; R x C elements of src_dtype, as in mx_quantize_gather.
 *   dest     device; int32 [R * k], the destinations of row t at t*k .. t*k+k-1;
 *            entries outside [0, out->rows) are skipped.  Output rows named by
 *            no entry are left untouched; a row named twice gets one of the
 *            writes (both hold the same bytes only if they come from the same
 *            source row).
 *   k        destinations per row (>= 0).
 *   cfg      host; MX_AXIS_LAST, MX_BLOCK_1D and MX_ROUND_RNE (stochastic
 *            rounding draws follow the destination element index, so SR
 *            returns MX_ERR_UNSUPPORTED: use mx_quantize_gather); transform and
 *            scale mode as in mx_quantize.
 *   out      host struct of device buffers: K = C, 1-D, MXFP4.
 *   Requires C % 32 == 0; R, C, k or out->rows = 0 is a no-op; at most
 *   2^32 - 256 source blocks per call.
 */
mx_status mx_quantize_scatter(const void* src, int32_t src_dtype, int64_t R, int64_t C, int64_t ld_src,
                              const int32_t* dest, int32_t k, const mx_quant_cfg* cfg, const mx_tensor* out,
                              void* stream);

/*
 * mx_dequantize — decode an MX operand: value = element(code) * 2^(scale-127)
 * ("MXFP4", AI Wiki, §Format specification: X times P_i; NaN scale makes the
 * whole block NaN; any element type: NaN and Inf element codes decode as
 * such).  With inverse_rht = 1 the 32-point transform is undone per
 * block along K in float32: the stages h = 1,2,4,8,16, the multiply by c, then
 * the sign flips of rht_sign_mask.
 *
 *   in       host struct of device buffers (any 1-D/2-D operand).
 *   dst      device; [in->rows, in->K] of dst_dtype, row stride ld_dst elements
 *            (>= K), 16-byte aligned, ld_dst a multiple of 8.  bf16 output is
 *            rounded to nearest even from the float32 value.
 */
mx_status mx_dequantize(const mx_tensor* in, int32_t inverse_rht, uint32_t rht_sign_mask,
                        void* dst, int32_t dst_dtype, int64_t ld_dst, void* stream);

/*
 * mx_transpose — the exact transpose of an operand quantized with 2-D (32x32)
 * blocks: out[c, r] = in[r, c] code for code, and the scale of out's tile
 * (c/32, r/32) is the scale of in's tile (r/32, c/32).  A 32x32 tile shares
 * one scale in either orientation, so nothing is re-rounded and the result is
 * bit-exact whatever rounding produced the input: one 2-D quantization of a
 * weight serves the forward product and, transposed, the data-gradient
 * product (dX = dY W needs W blocked along the other axis), the reason for 2-D
 * weight blocks in the hybrid 1D/2D recipe ("Training an MoE LLM in MXFP4:
 * How We Closed the Gap to BF16", summary).  A transform applied along the
 * input's K stays along the output's rows.
 *
 *   in    host struct of device buffers; block must be MX_BLOCK_2D ([R, C],
 *         R and C multiples of 32); any element type.
 *   out   host struct of device buffers; block MX_BLOCK_2D, rows == in->K and
 *         K == in->rows, the same element type; must not overlap in.
 * 1-D operands return MX_ERR_UNSUPPORTED (their blocks run along K only and
 * cannot be transposed without re-quantizing).  Empty operands are a no-op.
 */
mx_status mx_transpose(const mx_tensor* in, const mx_tensor* out, void* stream);

/*
 * mx_gemm — C[m, n] = sum_k A[m, k] * B[n, k] for MX operands A [M, K] and
 * B [N, K] (both K-major), per "MXFP4", AI Wiki, §Conversion rules: each block
 * pair contributes X(A) X(B) sum_i P_i(A) P_i(B) and a long dot product is the
 * sum of block dot products, accumulated in float32 (the order of that float32
 * sum is the library's); groups of 32 run along the contraction dimension
 * ("MXFP4", AI Wiki, §Hardware support: scales applied inside the matrix
 * instruction, float32 or bf16 output).  Runs on gfx950's scaled f8f6f4 MFMA:
 * A and B may each be any element type (MXFP4, MXFP6, MXFP8, mixed).  With an
 * FP8 or FP6 operand the instruction's internal sum of its 64 products keeps
 * about 14 binades below the largest product (measured; the spec leaves
 * internal precision to the implementation).
 *
 *   A, B       host structs of device buffers; A->K == B->K; either may use
 *              1-D or 2-D scales (2-D requires rows % 32 == 0).
 *   C          device; [M, N] of c_dtype, row stride ldc elements (>= N).
 *   workspace  device scratch of ws_bytes bytes, needed only when
 *              mx_gemm_workspace_size(M, N, K) > 0 (split-K partial sums;
 *              256-byte aligned, contract at mx_gemm_workspace_size) and
 *              the problem takes the MXFP4 256 x 256 kernels; otherwise may
 *              be NULL.  A missing, short or misaligned workspace for a split
 *              shape returns MX_ERR_INVALID_ARG without launching.
 *   M, N or K = 0: C is left untouched (K = 0 writes zeros).
 */
mx_status mx_gemm(const mx_tensor* A, const mx_tensor* B, void* C, int32_t c_dtype, int64_t ldc,
                  void* workspace, size_t ws_bytes, void* stream);

/*
 * mx_gemm_quantize — the product C = A B^T of mx_gemm, quantized in the GEMM's
 * epilogue into an MXFP4 operand blocked along N, so the float32 product never
 * reaches memory: the fused output quantization of a low-precision linear
 * layer ("MXFP4", AI Wiki, §Conversion rules for the block step; "Training an
 * MoE LLM in MXFP4: How We Closed the Gap to BF16" for MXFP4 GEMM outputs that
 * feed the next MXFP4 GEMM).  Each 32 consecutive outputs of a row form a
 * block quantized from their float32 values exactly as mx_quantize does with
 * RNE, no transform and the given scale mode: the result equals mx_gemm with
 * float32 output followed by mx_quantize of that output along its last dim.
 *
 *   A, B        host structs of device buffers, A->K == B->K, 1-D or 2-D
 *               scales: both MXFP4 (E2M1; scale rows 16-byte aligned with a
 *               stride that is a multiple of 16; codes under 2 GiB), or both
 *               MXFP8 / MXFP6 of any pair of E4M3, E5M2, E2M3, E3M2 ("MXFP4",
 *               AI Wiki, §Place in the MX family; scale rows 4-byte aligned
 *               with a stride that is a multiple of 4, 256 code rows under
 *               2 GiB); one MXFP4 and one other type: MX_ERR_UNSUPPORTED.
 *   scale_mode  an mx_scale_mode.
 *   out         host struct of device buffers: rows = M = A->rows, K = N =
 *               B->rows (a multiple of 32), MX_BLOCK_1D, MX_ELEM_E2M1; codes
 *               [M, N/2], scales [M, N/32] with their row strides (ld_codes a
 *               multiple of 16, as every mx_tensor).
 *   M, N >= 256 (the epilogue exists on the 256 x 256 pipeline only); other
 *   shapes or layouts return MX_ERR_UNSUPPORTED without launching.
 *   M or N = 0: nothing is written.  K = 0: the product is zero, so every
 *   block gets scale byte 0 and zero codes.  Row padding of out is untouched.
 */
mx_status mx_gemm_quantize(const mx_tensor* A, const mx_tensor* B, int32_t scale_mode, mx_tensor* out,
                           void* stream);

/*
 * mx_gemm_fused_quant_a — C = Q(A) B^T with the A operand handed over in bf16
 * and quantized to MXFP4 inside the GEMM's operand load, so the quantized A
 * is never written to memory (the fusion of the quantizer into the GEMM that
 * "Training an MoE LLM in MXFP4: How We Closed the Gap to BF16", summary,
 * and "MXFP4", AI Wiki, §Training with MXFP4 motivate: MXFP4 GEMMs fed by
 * activations quantized on the fly).  Each 32-element block of a row of A
 * along K is quantized exactly as mx_quantize does (same scale rule, RNE,
 * optional transform), so C equals mx_gemm of mx_quantize(A) and B whenever
 * both accumulate in K order one 64-deep step at a time (every shape that
 * mx_gemm_workspace_size does not split).  Every output tile re-reads and
 * re-quantizes its rows of A: the quantization work is repeated once per
 * 256 columns of C.
 *
 *   a, a_dtype  device; M x K elements, row stride lda elements (>= K, a
 *               multiple of 8), 16-byte aligned.  a_dtype must be
 *               MX_DT_BF16 (MX_DT_F32 returns MX_ERR_UNSUPPORTED).
 *   cfg         host; axis MX_AXIS_LAST, block MX_BLOCK_1D and rounding
 *               MX_ROUND_RNE (else MX_ERR_UNSUPPORTED); use_rht,
 *               rht_sign_mask and scale_mode as in mx_quantize.
 *   B           host struct of device buffers: MXFP4 [N, K], 1-D or 2-D.
 *   C           device; [M, N] of c_dtype, row stride ldc elements (>= N).
 *   Requires K % 32 == 0.  M or N = 0: nothing is written; K = 0 writes
 *   zeros (A is not read and may be NULL).
 */
mx_status mx_gemm_fused_quant_a(const void* a, int32_t a_dtype, int64_t M, int64_t K, int64_t lda,
                                const mx_quant_cfg* cfg, const mx_tensor* B, void* C, int32_t c_dtype, int64_t ldc,
                                void* stream);

/*
 * mx_gemm_workspace_size — bytes of device workspace mx_gemm needs for an
 * M x N x K problem (0 if none).  Problems with too few 256 x 256 output tiles
 * to fill the GPU, or a K longer than one float32 accumulator may sum while
 * keeping 1e-5 sum|a b| ("MXFP4", AI Wiki, §Conversion rules: the long dot
 * product is a sum of block dot products accumulated in float32), are split
 * along K: each output is accumulated in float32 over K segments of at most
 * 10240 (each tile walks its K range from a start fixed by the shape,
 * wrapping around once) and the segment sums are added in that walk's order,
 * fixed by the shape alone (the result is the same bit for bit on every
 * run).  With one
 * rounding per 64-deep step the error of an output is at most
 * (n - 1 + S - 1) 2^-24 sum|a b| to first order, n the 64-deep steps of its
 * longest segment (<= 160) and S its segments (<= 8): 8.6e-6 sum|a b| for the
 * weight gradient 2880 x 2880 x 16384 (n = 144, S <= 3).
 * Workspace contract: zero-filled before its first use (e.g. by a
 * hipMemsetAsync right after allocating it); every call leaves it fit for
 * the next call of any shape (its tile counters back at zero); calls that
 * share a workspace must not run concurrently.  Layout: 64 KiB of tile
 * counters, then the float32 partial tiles (256 KiB each).
 */
size_t mx_gemm_workspace_size(int64_t M, int64_t N, int64_t K);

/*
 * mx_gemm_noalloc — mx_gemm for callers that cannot allocate (code under HIP
 * graph capture, serving loops, harnesses that forbid allocation): the same
 * product and the same kernels, with the split-K workspace taken from the
 * library's own device array (64 KiB + 128 MiB per GPU the library runs on,
 * held until the process ends) instead of a caller buffer.  Allocates and
 * frees nothing.  Every call on a GPU shares that GPU's array, so calls that
 * overlap on one GPU (concurrent streams, other threads) race; the array's
 * counters start at zero and every call leaves them so.  Shapes whose split
 * would need more than the array holds (more than 256 workers, see
 * mx_gemm_workspace_size) return MX_ERR_UNSUPPORTED without launching.  Other
 * arguments and errors as mx_gemm.
 */
mx_status mx_gemm_noalloc(const mx_tensor* A, const mx_tensor* B, void* C, int32_t c_dtype, int64_t ldc,
                          void* stream);

/*
 * mx_grouped_gemm — the MoE expert GEMM over rows grouped by expert ("MXFP4",
 * AI Wiki, §Software support and §Use in models: MoE weights stored in
 * MXFP4): rows [off[e], off[e+1]) of A and of C belong to expert e, and
 * C[r, n] = sum_k A[r, k] * B_e[n, k], with the same block arithmetic as
 * mx_gemm.
 *
 *   A                host struct; A->rows is the capacity (rows of A and C).
 *   d_group_offsets  device; int32 [E+1], off[0] = 0, non-decreasing, read on
 *                    the device (no host synchronization).  Offsets above
 *                    A->rows are clamped to A->rows; rows past off[E] are not
 *                    written.
 *   E                number of experts (>= 1).
 *   B                host struct for expert 0: rows = N, K, block, strides;
 *                    expert e's codes start at B->codes + e*expert_stride_codes
 *                    bytes and its scales at B->scales + e*expert_stride_scales.
 *                    A and B may be any element types (MXFP4 runs on the
 *                    256x256 pipeline, other types on the C++ kernel).
 *   C                device; [A->rows, N] of c_dtype, row stride ldc.
 */
mx_status mx_grouped_gemm(const mx_tensor* A, const int32_t* d_group_offsets, int32_t E,
                          const mx_tensor* B, int64_t expert_stride_codes,
                          int64_t expert_stride_scales, void* C, int32_t c_dtype, int64_t ldc,
                          void* stream);

/*
 * mx_grouped_gemm_quantize — the product of mx_grouped_gemm quantized in the
 * GEMM epilogue into an MXFP4 operand blocked along N, as mx_gemm_quantize
 * does for the dense product (the expert outputs never reach memory in
 * float32 or bf16).  Equal to mx_grouped_gemm with float32 output followed by
 * mx_quantize of the rows it writes (RNE, no transform, the given scale mode).
 *
 *   A, d_group_offsets, E, B, expert strides: as mx_grouped_gemm; N =
 *               B->rows >= 256 and a multiple of 32, E <= 960; both operands
 *               MXFP4 (scale rows 16-byte aligned with strides, and the expert
 *               scale stride, a multiple of 16), or both MXFP8 / MXFP6 of any
 *               pair of E4M3, E5M2, E2M3, E3M2 (the same with 4 for 16).
 *   scale_mode  an mx_scale_mode.
 *   out         host struct of device buffers: rows = A->rows, K = N, 1-D,
 *               MXFP4.  Rows past off[E] are not written.
 *   Other shapes or layouts return MX_ERR_UNSUPPORTED without launching.
 */
mx_status mx_grouped_gemm_quantize(const mx_tensor* A, const int32_t* d_group_offsets, int32_t E,
                                   const mx_tensor* B, int64_t expert_stride_codes, int64_t expert_stride_scales,
                                   int32_t scale_mode, mx_tensor* out, void* stream);

/*
 * mx_clip_count — clipping statistic of a quantization.  "MXFP4", AI Wiki,
 * §Clipping in the reference algorithm: under the reference scale rule a
 * block's maximum can scale to just below twice the element type's largest
 * power of two, and every element scaling above the largest normal (6 for
 * E2M1, 448 E4M3, 57344 E5M2, 7.5 E2M3, 28 E3M2) saturates to it; the page
 * estimates ~3 % of entries on typical matrices.  This adds to *count the
 * number of elements of src that saturate when src is quantized with cfg and
 * element type elem: those whose value after the optional sign flips and
 * transform, the optional 3/4 prescale and the multiply by the inverse block
 * scale (exactly the quantizer's steps) has a magnitude above the largest
 * normal.  cfg->rounding is ignored (every mode saturates the same elements);
 * blocks holding NaN or Inf count nothing.  With MX_SCALE_ROUND_UP or
 * MX_SCALE_PRESCALE_3_4 the count is 0 by construction.
 *
 *   src, src_dtype, R, C, ld_src, cfg  as in mx_quantize (the same alignment
 *            rules; axis, block, use_rht, rht_sign_mask and scale_mode used).
 *   elem     an mx_elem.
 *   count    device; one 64-bit counter, ADDED to (atomically; the caller
 *            zeroes it, and calls on one stream accumulate).
 *   Requires K % 32 == 0 (K = C for MX_AXIS_LAST, R for MX_AXIS_DIM0); 2-D
 *   blocks need rows_out % 32 == 0.  R = 0 or C = 0 adds nothing.  Reads only
 *   src; allocates nothing.
 */
mx_status mx_clip_count(const void* src, int32_t src_dtype, int64_t R, int64_t C, int64_t ld_src,
                        const mx_quant_cfg* cfg, int32_t elem, uint64_t* count, void* stream);

/* Message describing the last failed call on this thread ("" if none). */
const char* mx_last_error(void);

/* Library version string. */
const char* mx_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBMXFP4_MX_H */
