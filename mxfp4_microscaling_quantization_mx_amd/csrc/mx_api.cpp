// C-ABI entry points of libmxfp4: argument validation, error reporting and
// dispatch to the kernel launchers.  Declarations and the contract of every
// entry point are in include/mx.h.
#include "../../include/mx.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "mx_launch.h"

namespace {

thread_local char g_err[512] = "";

mx_status fail(mx_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

mx_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MX_OK;
  return fail(MX_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Validate one MX operand description; `what` names it in messages.
// Bits per element of an mx_elem (0 for an unknown value).
int elem_bits(int32_t e) {
  switch (e) {
    case MX_ELEM_E2M1: return 4;
    case MX_ELEM_E4M3:
    case MX_ELEM_E5M2: return 8;
    case MX_ELEM_E2M3:
    case MX_ELEM_E3M2: return 6;
    default: return 0;
  }
}

mx_status check_tensor(const mx_tensor* t, const char* what) {
  if (!t) return fail(MX_ERR_INVALID_ARG, "%s: null mx_tensor", what);
  if (t->rows < 0 || t->K < 0) return fail(MX_ERR_INVALID_ARG, "%s: negative shape", what);
  if (t->K % 32) return fail(MX_ERR_INVALID_ARG, "%s: K=%lld is not a multiple of 32", what, (long long)t->K);
  if (t->block != MX_BLOCK_1D && t->block != MX_BLOCK_2D)
    return fail(MX_ERR_INVALID_ARG, "%s: unknown block kind %d", what, t->block);
  if (elem_bits(t->elem) == 0) return fail(MX_ERR_INVALID_ARG, "%s: unknown element type %d", what, t->elem);
  if (t->block == MX_BLOCK_2D && t->rows % 32)
    return fail(MX_ERR_INVALID_ARG, "%s: 2-D blocks need rows %% 32 == 0 (rows=%lld)", what, (long long)t->rows);
  if (t->rows == 0 || t->K == 0) return MX_OK;
  if (!t->codes || !t->scales) return fail(MX_ERR_INVALID_ARG, "%s: null codes/scales pointer", what);
  if (t->ld_codes < t->K * elem_bits(t->elem) / 8 || t->ld_scales < t->K / 32)
    return fail(MX_ERR_INVALID_ARG, "%s: row strides too small (ld_codes=%lld, ld_scales=%lld)", what,
                (long long)t->ld_codes, (long long)t->ld_scales);
  if (!aligned(t->codes, 16) || t->ld_codes % 16)
    return fail(MX_ERR_INVALID_ARG, "%s: codes must be 16-byte aligned with ld_codes %% 16 == 0", what);
  return MX_OK;
}

mx::MxOperand operand(const mx_tensor* t) {
  return mx::MxOperand{t->codes, t->scales, t->ld_codes, t->ld_scales};
}

// The C++ kernels for MXFP8 / MXFP6 operands (and the operand-load
// quantizing GEMM) address one 256-row tile of an operand, of its scales and
// of C with 32-bit buffer offsets.
bool tile_offsets_fit(const mx_tensor* t, int64_t ldc_bytes) {
  const int64_t lim = (int64_t)1 << 31;
  return (t == nullptr || (256 * t->ld_codes < lim && 256 * t->ld_scales < lim)) && 256 * ldc_bytes < lim;
}

}  // namespace

extern "C" {

const char* mx_last_error(void) { return g_err; }

const char* mx_version(void) { return "libmxfp4 0.1.0 (gfx950)"; }

mx_status mx_quantize(const void* src, int32_t src_dtype, int64_t R, int64_t C, int64_t ld_src,
                      const mx_quant_cfg* cfg, const mx_tensor* out, void* stream) {
  g_err[0] = '\0';
  if (!cfg || !out) return fail(MX_ERR_INVALID_ARG, "mx_quantize: null cfg or out");
  if (src_dtype != MX_DT_F32 && src_dtype != MX_DT_BF16)
    return fail(MX_ERR_INVALID_ARG, "mx_quantize: unknown source dtype %d", src_dtype);
  if (cfg->axis != MX_AXIS_LAST && cfg->axis != MX_AXIS_DIM0)
    return fail(MX_ERR_INVALID_ARG, "mx_quantize: unknown axis %d", cfg->axis);
  if (cfg->rounding != MX_ROUND_RNE && cfg->rounding != MX_ROUND_SR && cfg->rounding != MX_ROUND_SR8)
    return fail(MX_ERR_INVALID_ARG, "mx_quantize: unknown rounding %d", cfg->rounding);
  if (cfg->block != MX_BLOCK_1D && cfg->block != MX_BLOCK_2D)
    return fail(MX_ERR_INVALID_ARG, "mx_quantize: unknown block kind %d", cfg->block);
  if (cfg->use_rht != 0 && cfg->use_rht != 1)
    return fail(MX_ERR_INVALID_ARG, "mx_quantize: use_rht must be 0 or 1");
  if (cfg->scale_mode > MX_SCALE_PRESCALE_3_4)
    return fail(MX_ERR_INVALID_ARG, "mx_quantize: unknown scale_mode %u", cfg->scale_mode);
  if (R < 0 || C < 0) return fail(MX_ERR_INVALID_ARG, "mx_quantize: negative shape");
  const bool dim0 = cfg->axis == MX_AXIS_DIM0;
  const int64_t rows_out = dim0 ? C : R;
  const int64_t K = dim0 ? R : C;
  if (K % 32) return fail(MX_ERR_INVALID_ARG, "mx_quantize: blocking dimension %lld is not a multiple of 32", (long long)K);
  if (out->rows != rows_out || out->K != K)
    return fail(MX_ERR_INVALID_ARG, "mx_quantize: out is [%lld, %lld], expected [%lld, %lld]",
                (long long)out->rows, (long long)out->K, (long long)rows_out, (long long)K);
  if (out->block != cfg->block) return fail(MX_ERR_INVALID_ARG, "mx_quantize: out->block differs from cfg->block");
  mx_status st = check_tensor(out, "mx_quantize: out");
  if (st != MX_OK) return st;
  if (R == 0 || C == 0) return MX_OK;
  if (!src) return fail(MX_ERR_INVALID_ARG, "mx_quantize: null src");
  if (ld_src < C) return fail(MX_ERR_INVALID_ARG, "mx_quantize: ld_src=%lld < C=%lld", (long long)ld_src, (long long)C);
  // along the last dim the kernels read 16-byte pieces of a row; along dim 0
  // one element per lane, so any element-aligned base and row stride will do
  if (dim0 ? !aligned(src, src_dtype == MX_DT_BF16 ? 2 : 4) : (!aligned(src, 16) || ld_src % 8))
    return fail(MX_ERR_INVALID_ARG,
                dim0 ? "mx_quantize: src must be aligned to its element size"
                     : "mx_quantize: src must be 16-byte aligned with ld_src %% 8 == 0 (blocks along the last dim)");
  if (dim0 && (R + 127) / 128 > 65535)
    return fail(MX_ERR_UNSUPPORTED, "mx_quantize: dim-0 blocking supports at most 65535*128 source rows");
  if (dim0 && (31 * ld_src + C) * (src_dtype == MX_DT_BF16 ? 2 : 4) > (int64_t)0xFFFFFFFF)
    return fail(MX_ERR_UNSUPPORTED, "mx_quantize: dim-0 blocking needs 32 source rows to span < 4 GiB");
  if (!dim0 && R * (C / 32) > (int64_t)0xFFFFFF00)
    return fail(MX_ERR_UNSUPPORTED, "mx_quantize: at most 2^32 - 256 blocks per call");

  mx::QuantArgs a{};
  a.src = src;
  a.R = R;
  a.C = C;
  a.ld_src = ld_src;
  a.bf16 = src_dtype == MX_DT_BF16;
  a.dim0 = dim0;
  a.two_d = cfg->block == MX_BLOCK_2D;
  a.rht = cfg->use_rht == 1;
  a.sr = cfg->rounding == MX_ROUND_SR ? 1 : cfg->rounding == MX_ROUND_SR8 ? 2 : 0;
  a.mask = cfg->rht_sign_mask;
  a.seed = cfg->philox_seed;
  a.offset = cfg->philox_offset;
  a.scale_mode = (int)cfg->scale_mode;
  a.codes = out->codes;
  a.ld_codes = out->ld_codes;
  a.scales = out->scales;
  a.ld_scales = out->ld_scales;
  a.elem = out->elem;
  return hip_status(mx::launch_quantize(a, static_cast<hipStream_t>(stream)), "mx_quantize");
}

mx_status mx_clip_count(const void* src, int32_t src_dtype, int64_t R, int64_t C, int64_t ld_src,
                        const mx_quant_cfg* cfg, int32_t elem, uint64_t* count, void* stream) {
  g_err[0] = '\0';
  if (!cfg) return fail(MX_ERR_INVALID_ARG, "mx_clip_count: null cfg");
  if (src_dtype != MX_DT_F32 && src_dtype != MX_DT_BF16)
    return fail(MX_ERR_INVALID_ARG, "mx_clip_count: unknown source dtype %d", src_dtype);
  if (cfg->axis != MX_AXIS_LAST && cfg->axis != MX_AXIS_DIM0)
    return fail(MX_ERR_INVALID_ARG, "mx_clip_count: unknown axis %d", cfg->axis);
  if (cfg->block != MX_BLOCK_1D && cfg->block != MX_BLOCK_2D)
    return fail(MX_ERR_INVALID_ARG, "mx_clip_count: unknown block kind %d", cfg->block);
  if (cfg->use_rht != 0 && cfg->use_rht != 1)
    return fail(MX_ERR_INVALID_ARG, "mx_clip_count: use_rht must be 0 or 1");
  if (cfg->scale_mode > MX_SCALE_PRESCALE_3_4)
    return fail(MX_ERR_INVALID_ARG, "mx_clip_count: unknown scale_mode %u", cfg->scale_mode);
  if (elem < MX_ELEM_E2M1 || elem > MX_ELEM_E3M2)
    return fail(MX_ERR_INVALID_ARG, "mx_clip_count: unknown element type %d", elem);
  if (R < 0 || C < 0) return fail(MX_ERR_INVALID_ARG, "mx_clip_count: negative shape");
  const bool dim0 = cfg->axis == MX_AXIS_DIM0;
  const int64_t rows_out = dim0 ? C : R;
  const int64_t K = dim0 ? R : C;
  if (K % 32) return fail(MX_ERR_INVALID_ARG, "mx_clip_count: blocking dimension %lld is not a multiple of 32", (long long)K);
  if (cfg->block == MX_BLOCK_2D && rows_out % 32)
    return fail(MX_ERR_INVALID_ARG, "mx_clip_count: 2-D blocks need rows_out %% 32 == 0 (got %lld)", (long long)rows_out);
  if (!count) return fail(MX_ERR_INVALID_ARG, "mx_clip_count: null count");
  if (!aligned(count, 8)) return fail(MX_ERR_INVALID_ARG, "mx_clip_count: count must be 8-byte aligned");
  if (R == 0 || C == 0) return MX_OK;
  if (!src) return fail(MX_ERR_INVALID_ARG, "mx_clip_count: null src");
  if (ld_src < C) return fail(MX_ERR_INVALID_ARG, "mx_clip_count: ld_src=%lld < C=%lld", (long long)ld_src, (long long)C);
  // (along dim 0 the kernel reads one element per lane, as the quantizer does)
  if (dim0 ? !aligned(src, src_dtype == MX_DT_BF16 ? 2 : 4) : (!aligned(src, 16) || ld_src % 8))
    return fail(MX_ERR_INVALID_ARG,
                dim0 ? "mx_clip_count: src must be aligned to its element size"
                     : "mx_clip_count: src must be 16-byte aligned with ld_src %% 8 == 0 (blocks along the last dim)");
  mx::ClipArgs a{};
  a.src = src;
  a.R = R;
  a.C = C;
  a.ld_src = ld_src;
  a.bf16 = src_dtype == MX_DT_BF16;
  a.dim0 = dim0;
  a.two_d = cfg->block == MX_BLOCK_2D;
  a.rht = cfg->use_rht == 1;
  a.mask = cfg->rht_sign_mask;
  a.scale_mode = (int)cfg->scale_mode;
  a.elem = elem;
  a.count = reinterpret_cast<unsigned long long*>(count);
  return hip_status(mx::launch_clip_count(a, static_cast<hipStream_t>(stream)), "mx_clip_count");
}

mx_status mx_quantize_scatter(const void* src, int32_t src_dtype, int64_t R, int64_t C, int64_t ld_src,
                              const int32_t* dest, int32_t k, const mx_quant_cfg* cfg, const mx_tensor* out,
                              void* stream) {
  g_err[0] = '\0';
  if (!cfg || !out) return fail(MX_ERR_INVALID_ARG, "mx_quantize_scatter: null cfg or out");
  if (src_dtype != MX_DT_F32 && src_dtype != MX_DT_BF16)
    return fail(MX_ERR_INVALID_ARG, "mx_quantize_scatter: unknown source dtype %d", src_dtype);
  if (cfg->axis != MX_AXIS_LAST || cfg->block != MX_BLOCK_1D)
    return fail(MX_ERR_UNSUPPORTED, "mx_quantize_scatter: only 1-D blocks along the last dim");
  if (cfg->rounding != MX_ROUND_RNE)
    return fail(MX_ERR_UNSUPPORTED, "mx_quantize_scatter: RNE only (SR draws depend on the destination row)");
  if (cfg->use_rht != 0 && cfg->use_rht != 1)
    return fail(MX_ERR_INVALID_ARG, "mx_quantize_scatter: use_rht must be 0 or 1");
  if (cfg->scale_mode > MX_SCALE_PRESCALE_3_4)
    return fail(MX_ERR_INVALID_ARG, "mx_quantize_scatter: unknown scale_mode %u", cfg->scale_mode);
  if (R < 0 || C < 0 || k < 0) return fail(MX_ERR_INVALID_ARG, "mx_quantize_scatter: negative shape or k");
  if (C % 32) return fail(MX_ERR_INVALID_ARG, "mx_quantize_scatter: C=%lld is not a multiple of 32", (long long)C);
  if (out->K != C)
    return fail(MX_ERR_INVALID_ARG, "mx_quantize_scatter: out.K=%lld != C=%lld", (long long)out->K, (long long)C);
  if (out->block != MX_BLOCK_1D) return fail(MX_ERR_INVALID_ARG, "mx_quantize_scatter: out must hold 1-D blocks");
  mx_status st = check_tensor(out, "mx_quantize_scatter: out");
  if (st != MX_OK) return st;
  if (out->elem != MX_ELEM_E2M1) return fail(MX_ERR_UNSUPPORTED, "mx_quantize_scatter: MXFP4 output only");
  if (R == 0 || C == 0 || k == 0 || out->rows == 0) return MX_OK;
  if (!dest || !aligned(dest, 4)) return fail(MX_ERR_INVALID_ARG, "mx_quantize_scatter: null or unaligned dest");
  if (!src) return fail(MX_ERR_INVALID_ARG, "mx_quantize_scatter: null src");
  if (ld_src < C)
    return fail(MX_ERR_INVALID_ARG, "mx_quantize_scatter: ld_src=%lld < C=%lld", (long long)ld_src, (long long)C);
  if (!aligned(src, 16) || ld_src % 8)
    return fail(MX_ERR_INVALID_ARG, "mx_quantize_scatter: src must be 16-byte aligned with ld_src %% 8 == 0");
  if (R * (C / 32) > (int64_t)0xFFFFFF00)
    return fail(MX_ERR_UNSUPPORTED, "mx_quantize_scatter: at most 2^32 - 256 blocks per call");
  mx::QuantArgs a{};
  a.src = src;
  a.R = R;
  a.C = C;
  a.ld_src = ld_src;
  a.bf16 = src_dtype == MX_DT_BF16;
  a.rht = cfg->use_rht == 1;
  a.mask = cfg->rht_sign_mask;
  a.scale_mode = (int)cfg->scale_mode;
  a.codes = out->codes;
  a.ld_codes = out->ld_codes;
  a.scales = out->scales;
  a.ld_scales = out->ld_scales;
  return hip_status(mx::launch_quantize_scatter(a, dest, k, out->rows, static_cast<hipStream_t>(stream)),
                    "mx_quantize_scatter");
}

mx_status mx_quantize_gather(const void* src, int32_t src_dtype, int64_t R_src, int64_t C, int64_t ld_src,
                             const int32_t* rows, int64_t rows_out, const mx_quant_cfg* cfg,
                             const mx_tensor* out, void* stream) {
  g_err[0] = '\0';
  if (!cfg || !out) return fail(MX_ERR_INVALID_ARG, "mx_quantize_gather: null cfg or out");
  if (src_dtype != MX_DT_F32 && src_dtype != MX_DT_BF16)
    return fail(MX_ERR_INVALID_ARG, "mx_quantize_gather: unknown source dtype %d", src_dtype);
  if (cfg->axis != MX_AXIS_LAST || cfg->block != MX_BLOCK_1D)
    return fail(MX_ERR_UNSUPPORTED, "mx_quantize_gather: only 1-D blocks along the last dim");
  if (cfg->rounding != MX_ROUND_RNE && cfg->rounding != MX_ROUND_SR && cfg->rounding != MX_ROUND_SR8)
    return fail(MX_ERR_INVALID_ARG, "mx_quantize_gather: unknown rounding %d", cfg->rounding);
  if (cfg->use_rht != 0 && cfg->use_rht != 1)
    return fail(MX_ERR_INVALID_ARG, "mx_quantize_gather: use_rht must be 0 or 1");
  if (cfg->scale_mode > MX_SCALE_PRESCALE_3_4)
    return fail(MX_ERR_INVALID_ARG, "mx_quantize_gather: unknown scale_mode %u", cfg->scale_mode);
  if (R_src < 0 || C < 0 || rows_out < 0) return fail(MX_ERR_INVALID_ARG, "mx_quantize_gather: negative shape");
  if (C % 32) return fail(MX_ERR_INVALID_ARG, "mx_quantize_gather: C=%lld is not a multiple of 32", (long long)C);
  if (out->rows != rows_out || out->K != C)
    return fail(MX_ERR_INVALID_ARG, "mx_quantize_gather: out is [%lld, %lld], expected [%lld, %lld]",
                (long long)out->rows, (long long)out->K, (long long)rows_out, (long long)C);
  if (out->block != MX_BLOCK_1D) return fail(MX_ERR_INVALID_ARG, "mx_quantize_gather: out must hold 1-D blocks");
  mx_status st = check_tensor(out, "mx_quantize_gather: out");
  if (st != MX_OK) return st;
  if (out->elem != MX_ELEM_E2M1) return fail(MX_ERR_UNSUPPORTED, "mx_quantize_gather: MXFP4 output only");
  if (rows_out == 0 || C == 0) return MX_OK;
  if (!rows || !aligned(rows, 4)) return fail(MX_ERR_INVALID_ARG, "mx_quantize_gather: null or unaligned rows");
  if (R_src > 0) {
    if (!src) return fail(MX_ERR_INVALID_ARG, "mx_quantize_gather: null src");
    if (ld_src < C)
      return fail(MX_ERR_INVALID_ARG, "mx_quantize_gather: ld_src=%lld < C=%lld", (long long)ld_src, (long long)C);
    if (!aligned(src, 16) || ld_src % 8)
      return fail(MX_ERR_INVALID_ARG, "mx_quantize_gather: src must be 16-byte aligned with ld_src %% 8 == 0");
  }
  if (rows_out * (C / 32) > (int64_t)0xFFFFFF00)
    return fail(MX_ERR_UNSUPPORTED, "mx_quantize_gather: at most 2^32 - 256 blocks per call");

  mx::QuantArgs a{};
  a.src = src;
  a.R = rows_out;
  a.C = C;
  a.ld_src = ld_src;
  a.bf16 = src_dtype == MX_DT_BF16;
  a.rht = cfg->use_rht == 1;
  a.sr = cfg->rounding == MX_ROUND_SR ? 1 : cfg->rounding == MX_ROUND_SR8 ? 2 : 0;
  a.mask = cfg->rht_sign_mask;
  a.seed = cfg->philox_seed;
  a.offset = cfg->philox_offset;
  a.scale_mode = (int)cfg->scale_mode;
  a.codes = out->codes;
  a.ld_codes = out->ld_codes;
  a.scales = out->scales;
  a.ld_scales = out->ld_scales;
  a.gather = rows;
  a.R_src = R_src;
  return hip_status(mx::launch_quantize(a, static_cast<hipStream_t>(stream)), "mx_quantize_gather");
}

mx_status mx_dequantize(const mx_tensor* in, int32_t inverse_rht, uint32_t rht_sign_mask, void* dst,
                        int32_t dst_dtype, int64_t ld_dst, void* stream) {
  g_err[0] = '\0';
  mx_status st = check_tensor(in, "mx_dequantize: in");
  if (st != MX_OK) return st;
  if (dst_dtype != MX_DT_F32 && dst_dtype != MX_DT_BF16)
    return fail(MX_ERR_INVALID_ARG, "mx_dequantize: unknown destination dtype %d", dst_dtype);
  if (inverse_rht != 0 && inverse_rht != 1)
    return fail(MX_ERR_INVALID_ARG, "mx_dequantize: inverse_rht must be 0 or 1");
  if (in->rows == 0 || in->K == 0) return MX_OK;
  if (!dst) return fail(MX_ERR_INVALID_ARG, "mx_dequantize: null dst");
  if (ld_dst < in->K || ld_dst % 8 || !aligned(dst, 16))
    return fail(MX_ERR_INVALID_ARG, "mx_dequantize: dst must be 16-byte aligned with ld_dst >= K and ld_dst %% 8 == 0");
  mx::DequantArgs a{};
  a.codes = in->codes;
  a.scales = in->scales;
  a.rows = in->rows;
  a.K = in->K;
  a.ld_codes = in->ld_codes;
  a.ld_scales = in->ld_scales;
  a.two_d = in->block == MX_BLOCK_2D;
  a.inverse_rht = inverse_rht == 1;
  a.mask = rht_sign_mask;
  a.dst = dst;
  a.out_bf16 = dst_dtype == MX_DT_BF16;
  a.ld_dst = ld_dst;
  a.elem = in->elem;
  return hip_status(mx::launch_dequantize(a, static_cast<hipStream_t>(stream)), "mx_dequantize");
}

mx_status mx_transpose(const mx_tensor* in, const mx_tensor* out, void* stream) {
  g_err[0] = '\0';
  mx_status st = check_tensor(in, "mx_transpose: in");
  if (st != MX_OK) return st;
  st = check_tensor(out, "mx_transpose: out");
  if (st != MX_OK) return st;
  if (in->block != MX_BLOCK_2D || out->block != MX_BLOCK_2D)
    return fail(MX_ERR_UNSUPPORTED, "mx_transpose: only operands with 2-D (32x32) blocks transpose exactly");
  if (in->elem != out->elem)
    return fail(MX_ERR_INVALID_ARG, "mx_transpose: in and out element types differ");
  if (out->rows != in->K || out->K != in->rows)
    return fail(MX_ERR_INVALID_ARG, "mx_transpose: out is [%lld, %lld], expected [%lld, %lld]", (long long)out->rows,
                (long long)out->K, (long long)in->K, (long long)in->rows);
  if (in->rows == 0 || in->K == 0) return MX_OK;
  if (((in->rows + 127) / 128) * ((in->K + 127) / 128) > (int64_t)0x7FFFFFFF)
    return fail(MX_ERR_UNSUPPORTED, "mx_transpose: at most 2^31 - 1 tiles of 128 x 128");
  mx::TransposeArgs a{};
  a.in_codes = in->codes;
  a.in_scales = in->scales;
  a.R = in->rows;
  a.C = in->K;
  a.ld_in = in->ld_codes;
  a.ld_sin = in->ld_scales;
  a.out_codes = out->codes;
  a.out_scales = out->scales;
  a.ld_out = out->ld_codes;
  a.ld_sout = out->ld_scales;
  a.bits = elem_bits(in->elem);
  return hip_status(mx::launch_transpose(a, static_cast<hipStream_t>(stream)), "mx_transpose");
}

size_t mx_gemm_workspace_size(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  return mx::gemm_splitk_workspace(M, N, K);
}

namespace {

// Validate an mx_gemm call and describe it; M = 0 or N = 0 leaves a.M or a.N 0.
mx_status gemm_args(const mx_tensor* A, const mx_tensor* B, void* C, int32_t c_dtype, int64_t ldc,
                    const char* what, mx::GemmArgs& a) {
  char name[64];
  std::snprintf(name, sizeof(name), "%s: A", what);
  mx_status st = check_tensor(A, name);
  if (st != MX_OK) return st;
  std::snprintf(name, sizeof(name), "%s: B", what);
  st = check_tensor(B, name);
  if (st != MX_OK) return st;
  if (A->K != B->K)
    return fail(MX_ERR_INVALID_ARG, "%s: A.K=%lld != B.K=%lld", what, (long long)A->K, (long long)B->K);
  if (c_dtype != MX_DT_F32 && c_dtype != MX_DT_BF16)
    return fail(MX_ERR_INVALID_ARG, "%s: unknown output dtype %d", what, c_dtype);
  const int64_t M = A->rows, N = B->rows;
  a = mx::GemmArgs{};
  a.M = M;
  a.N = N;
  if (M == 0 || N == 0) return MX_OK;
  if (!C) return fail(MX_ERR_INVALID_ARG, "%s: null C", what);
  if (ldc < N) return fail(MX_ERR_INVALID_ARG, "%s: ldc=%lld < N=%lld", what, (long long)ldc, (long long)N);
  if ((M + 127) / 128 > 65535) return fail(MX_ERR_UNSUPPORTED, "%s: M too large", what);
  a.A = operand(A);
  a.B = operand(B);
  a.a_2d = A->block == MX_BLOCK_2D;
  a.b_2d = B->block == MX_BLOCK_2D;
  a.K = A->K;
  a.C = C;
  a.ldc = ldc;
  a.out_bf16 = c_dtype == MX_DT_BF16;
  a.a_elem = A->elem;
  a.b_elem = B->elem;
  if ((a.a_elem != 0 || a.b_elem != 0) &&
      !(tile_offsets_fit(A, ldc * (a.out_bf16 ? 2 : 4)) && tile_offsets_fit(B, 0)))
    return fail(MX_ERR_UNSUPPORTED, "%s: row strides too large for the MXFP8/MXFP6 kernels", what);
  return MX_OK;
}

}  // namespace

mx_status mx_gemm(const mx_tensor* A, const mx_tensor* B, void* C, int32_t c_dtype, int64_t ldc,
                  void* workspace, size_t ws_bytes, void* stream) {
  g_err[0] = '\0';
  mx::GemmArgs a;
  const mx_status st = gemm_args(A, B, C, c_dtype, ldc, "mx_gemm", a);
  if (st != MX_OK || a.M == 0 || a.N == 0) return st;
  if (a.K > 0 && mx::gemm_splitk_applies(a)) {
    const size_t need = mx::gemm_splitk_workspace(a.M, a.N, a.K);
    if (!workspace || ws_bytes < need || !aligned(workspace, 256))
      return fail(MX_ERR_INVALID_ARG,
                  "mx_gemm: this shape is split along K and needs a 256-byte aligned workspace of %zu bytes "
                  "(got %zu bytes at %p)",
                  need, ws_bytes, workspace);
    return hip_status(mx::launch_gemm_splitk(a, workspace, static_cast<hipStream_t>(stream)), "mx_gemm");
  }
  return hip_status(mx::launch_gemm(a, static_cast<hipStream_t>(stream)), "mx_gemm");
}

mx_status mx_gemm_noalloc(const mx_tensor* A, const mx_tensor* B, void* C, int32_t c_dtype, int64_t ldc,
                          void* stream) {
  g_err[0] = '\0';
  mx::GemmArgs a;
  const mx_status st = gemm_args(A, B, C, c_dtype, ldc, "mx_gemm_noalloc", a);
  if (st != MX_OK || a.M == 0 || a.N == 0) return st;
  if (a.K > 0 && mx::gemm_splitk_applies(a)) {
    const size_t need = mx::gemm_splitk_workspace(a.M, a.N, a.K);
    if (need > mx::gemm_splitk_scratch_bytes())
      return fail(MX_ERR_UNSUPPORTED,
                  "mx_gemm_noalloc: this shape's split-K workspace (%zu bytes) exceeds the library's scratch "
                  "(%zu bytes); use mx_gemm with a workspace",
                  need, mx::gemm_splitk_scratch_bytes());
    void* scratch = nullptr;
    const hipError_t e = mx::gemm_splitk_scratch(&scratch);
    if (e != hipSuccess) return hip_status(e, "mx_gemm_noalloc: scratch address");
    return hip_status(mx::launch_gemm_splitk(a, scratch, static_cast<hipStream_t>(stream)), "mx_gemm_noalloc");
  }
  return hip_status(mx::launch_gemm(a, static_cast<hipStream_t>(stream)), "mx_gemm_noalloc");
}

mx_status mx_gemm_fused_quant_a(const void* a, int32_t a_dtype, int64_t M, int64_t K, int64_t lda,
                                const mx_quant_cfg* cfg, const mx_tensor* B, void* C, int32_t c_dtype, int64_t ldc,
                                void* stream) {
  g_err[0] = '\0';
  const char* what = "mx_gemm_fused_quant_a";
  if (!cfg || !B) return fail(MX_ERR_INVALID_ARG, "%s: null cfg or B", what);
  if (a_dtype != MX_DT_F32 && a_dtype != MX_DT_BF16)
    return fail(MX_ERR_INVALID_ARG, "%s: unknown A dtype %d", what, a_dtype);
  if (a_dtype != MX_DT_BF16) return fail(MX_ERR_UNSUPPORTED, "%s: A must be bf16", what);
  if (cfg->axis != MX_AXIS_LAST || cfg->block != MX_BLOCK_1D || cfg->rounding != MX_ROUND_RNE)
    return fail(MX_ERR_UNSUPPORTED, "%s: A is quantized along K with 1-D blocks and RNE only", what);
  if (cfg->use_rht != 0 && cfg->use_rht != 1) return fail(MX_ERR_INVALID_ARG, "%s: use_rht must be 0 or 1", what);
  if (cfg->scale_mode > MX_SCALE_PRESCALE_3_4)
    return fail(MX_ERR_INVALID_ARG, "%s: unknown scale_mode %u", what, cfg->scale_mode);
  mx_status st = check_tensor(B, "mx_gemm_fused_quant_a: B");
  if (st != MX_OK) return st;
  if (B->elem != MX_ELEM_E2M1) return fail(MX_ERR_UNSUPPORTED, "%s: B must be MXFP4", what);
  if (M < 0 || K < 0) return fail(MX_ERR_INVALID_ARG, "%s: negative shape", what);
  if (K % 32) return fail(MX_ERR_INVALID_ARG, "%s: K=%lld is not a multiple of 32", what, (long long)K);
  if (B->K != K) return fail(MX_ERR_INVALID_ARG, "%s: K=%lld != B.K=%lld", what, (long long)K, (long long)B->K);
  if (c_dtype != MX_DT_F32 && c_dtype != MX_DT_BF16)
    return fail(MX_ERR_INVALID_ARG, "%s: unknown output dtype %d", what, c_dtype);
  const int64_t N = B->rows;
  if (M == 0 || N == 0) return MX_OK;
  if (!C) return fail(MX_ERR_INVALID_ARG, "%s: null C", what);
  if (ldc < N) return fail(MX_ERR_INVALID_ARG, "%s: ldc=%lld < N=%lld", what, (long long)ldc, (long long)N);
  if (K > 0) {
    if (!a) return fail(MX_ERR_INVALID_ARG, "%s: null A", what);
    if (lda < K) return fail(MX_ERR_INVALID_ARG, "%s: lda=%lld < K=%lld", what, (long long)lda, (long long)K);
    if (!aligned(a, 16) || lda % 8)
      return fail(MX_ERR_INVALID_ARG, "%s: A must be 16-byte aligned with lda %% 8 == 0", what);
  }
  if ((M + 255) / 256 > 65535) return fail(MX_ERR_UNSUPPORTED, "%s: M too large", what);
  if (256 * lda * 2 >= ((int64_t)1 << 31) || !tile_offsets_fit(B, ldc * (c_dtype == MX_DT_BF16 ? 2 : 4)))
    return fail(MX_ERR_UNSUPPORTED, "%s: row strides too large", what);
  mx::GemmQaArgs q{};
  q.a = a;
  q.lda = lda;
  q.rht = cfg->use_rht == 1;
  q.mask = cfg->rht_sign_mask;
  q.scale_mode = (int)cfg->scale_mode;
  q.B = operand(B);
  q.b_2d = B->block == MX_BLOCK_2D;
  q.M = M;
  q.N = N;
  q.K = K;
  q.C = C;
  q.ldc = ldc;
  q.out_bf16 = c_dtype == MX_DT_BF16;
  return hip_status(mx::launch_gemm_qa(q, static_cast<hipStream_t>(stream)), what);
}

mx_status mx_gemm_quantize(const mx_tensor* A, const mx_tensor* B, int32_t scale_mode, mx_tensor* out,
                           void* stream) {
  g_err[0] = '\0';
  mx_status st = check_tensor(A, "mx_gemm_quantize: A");
  if (st != MX_OK) return st;
  st = check_tensor(B, "mx_gemm_quantize: B");
  if (st != MX_OK) return st;
  st = check_tensor(out, "mx_gemm_quantize: out");
  if (st != MX_OK) return st;
  if (A->K != B->K)
    return fail(MX_ERR_INVALID_ARG, "mx_gemm_quantize: A.K=%lld != B.K=%lld", (long long)A->K, (long long)B->K);
  if (scale_mode < MX_SCALE_FLOOR || scale_mode > MX_SCALE_PRESCALE_3_4)
    return fail(MX_ERR_INVALID_ARG, "mx_gemm_quantize: unknown scale mode %d", scale_mode);
  const int64_t M = A->rows, N = B->rows;
  if (out->rows != M || out->K != N)
    return fail(MX_ERR_INVALID_ARG, "mx_gemm_quantize: out is [%lld, %lld], the product is [%lld, %lld]",
                (long long)out->rows, (long long)out->K, (long long)M, (long long)N);
  if (out->elem != MX_ELEM_E2M1) return fail(MX_ERR_UNSUPPORTED, "mx_gemm_quantize: the output is MXFP4");
  if ((A->elem == MX_ELEM_E2M1) != (B->elem == MX_ELEM_E2M1))
    return fail(MX_ERR_UNSUPPORTED, "mx_gemm_quantize: both operands MXFP4, or both MXFP8 / MXFP6");
  if (out->block != MX_BLOCK_1D)
    return fail(MX_ERR_UNSUPPORTED, "mx_gemm_quantize: the output uses 1-D blocks");
  if (M == 0 || N == 0) return MX_OK;
  mx::GemmQuantArgs a{};
  a.A = operand(A);
  a.B = operand(B);
  a.a_2d = A->block == MX_BLOCK_2D;
  a.b_2d = B->block == MX_BLOCK_2D;
  a.M = M;
  a.N = N;
  a.K = A->K;
  a.codes = out->codes;
  a.scales = out->scales;
  a.ld_codes = out->ld_codes;
  a.ld_scales = out->ld_scales;
  a.scale_mode = scale_mode;
  a.a_elem = A->elem;
  a.b_elem = B->elem;
  if (!mx::gemm_quantize_supported(a))
    return fail(MX_ERR_UNSUPPORTED,
                "mx_gemm_quantize: needs M, N >= 256, operand scale rows 16-byte aligned with strides %% 16 == 0, "
                "operands under 2 GiB, out code rows 4-byte aligned");
  return hip_status(mx::launch_gemm_quantize(a, static_cast<hipStream_t>(stream)), "mx_gemm_quantize");
}

mx_status mx_grouped_gemm_quantize(const mx_tensor* A, const int32_t* d_group_offsets, int32_t E,
                                   const mx_tensor* B, int64_t expert_stride_codes, int64_t expert_stride_scales,
                                   int32_t scale_mode, mx_tensor* out, void* stream) {
  g_err[0] = '\0';
  mx_status st = check_tensor(A, "mx_grouped_gemm_quantize: A");
  if (st != MX_OK) return st;
  st = check_tensor(B, "mx_grouped_gemm_quantize: B");
  if (st != MX_OK) return st;
  st = check_tensor(out, "mx_grouped_gemm_quantize: out");
  if (st != MX_OK) return st;
  if (A->block != MX_BLOCK_1D) return fail(MX_ERR_UNSUPPORTED, "mx_grouped_gemm_quantize: A must use 1-D blocks");
  if (A->K != B->K)
    return fail(MX_ERR_INVALID_ARG, "mx_grouped_gemm_quantize: A.K=%lld != B.K=%lld", (long long)A->K,
                (long long)B->K);
  if (E < 1) return fail(MX_ERR_INVALID_ARG, "mx_grouped_gemm_quantize: E=%d < 1", E);
  if (!d_group_offsets) return fail(MX_ERR_INVALID_ARG, "mx_grouped_gemm_quantize: null group offsets");
  if (scale_mode < MX_SCALE_FLOOR || scale_mode > MX_SCALE_PRESCALE_3_4)
    return fail(MX_ERR_INVALID_ARG, "mx_grouped_gemm_quantize: unknown scale mode %d", scale_mode);
  if (expert_stride_codes < 0 || expert_stride_scales < 0 || expert_stride_codes % 16)
    return fail(MX_ERR_INVALID_ARG, "mx_grouped_gemm_quantize: expert strides must be >= 0 (codes stride %% 16 == 0)");
  const int64_t M = A->rows, N = B->rows;
  if (out->rows != M || out->K != N)
    return fail(MX_ERR_INVALID_ARG, "mx_grouped_gemm_quantize: out is [%lld, %lld], the product is [%lld, %lld]",
                (long long)out->rows, (long long)out->K, (long long)M, (long long)N);
  if (out->elem != MX_ELEM_E2M1) return fail(MX_ERR_UNSUPPORTED, "mx_grouped_gemm_quantize: the output is MXFP4");
  if ((A->elem == MX_ELEM_E2M1) != (B->elem == MX_ELEM_E2M1))
    return fail(MX_ERR_UNSUPPORTED, "mx_grouped_gemm_quantize: both operands MXFP4, or both MXFP8 / MXFP6");
  if (out->block != MX_BLOCK_1D)
    return fail(MX_ERR_UNSUPPORTED, "mx_grouped_gemm_quantize: the output uses 1-D blocks");
  if (M == 0 || N == 0) return MX_OK;
  mx::GroupedQuantArgs q{};
  q.g.A = operand(A);
  q.g.B = operand(B);
  q.g.a_2d = false;
  q.g.b_2d = B->block == MX_BLOCK_2D;
  q.g.M_cap = M;
  q.g.N = N;
  q.g.K = A->K;
  q.g.offsets = d_group_offsets;
  q.g.E = E;
  q.g.stride_codes = expert_stride_codes;
  q.g.stride_scales = expert_stride_scales;
  q.codes = out->codes;
  q.scales = out->scales;
  q.ld_codes = out->ld_codes;
  q.ld_scales = out->ld_scales;
  q.scale_mode = scale_mode;
  q.g.a_elem = A->elem;
  q.g.b_elem = B->elem;
  if (!mx::grouped_quantize_supported(q))
    return fail(MX_ERR_UNSUPPORTED,
                "mx_grouped_gemm_quantize: needs N >= 256, 16-byte aligned scale rows with strides %% 16 == 0 (and "
                "expert scale stride), E <= 960, operands under 2 GiB");
  return hip_status(mx::launch_grouped_gemm_quantize(q, static_cast<hipStream_t>(stream)),
                    "mx_grouped_gemm_quantize");
}

mx_status mx_grouped_gemm(const mx_tensor* A, const int32_t* d_group_offsets, int32_t E,
                          const mx_tensor* B, int64_t expert_stride_codes,
                          int64_t expert_stride_scales, void* C, int32_t c_dtype, int64_t ldc,
                          void* stream) {
  g_err[0] = '\0';
  mx_status st = check_tensor(A, "mx_grouped_gemm: A");
  if (st != MX_OK) return st;
  st = check_tensor(B, "mx_grouped_gemm: B");
  if (st != MX_OK) return st;
  if (A->block != MX_BLOCK_1D)
    return fail(MX_ERR_UNSUPPORTED, "mx_grouped_gemm: A must use 1-D blocks (expert boundaries are arbitrary rows)");
  if (A->K != B->K)
    return fail(MX_ERR_INVALID_ARG, "mx_grouped_gemm: A.K=%lld != B.K=%lld", (long long)A->K, (long long)B->K);
  if (E < 1) return fail(MX_ERR_INVALID_ARG, "mx_grouped_gemm: E=%d < 1", E);
  if (!d_group_offsets) return fail(MX_ERR_INVALID_ARG, "mx_grouped_gemm: null group offsets");
  if (c_dtype != MX_DT_F32 && c_dtype != MX_DT_BF16)
    return fail(MX_ERR_INVALID_ARG, "mx_grouped_gemm: unknown output dtype %d", c_dtype);
  if (expert_stride_codes < 0 || expert_stride_scales < 0 || expert_stride_codes % 16)
    return fail(MX_ERR_INVALID_ARG, "mx_grouped_gemm: expert strides must be >= 0 (codes stride %% 16 == 0)");
  const int64_t M = A->rows, N = B->rows;
  if (M == 0 || N == 0) return MX_OK;
  if (!C) return fail(MX_ERR_INVALID_ARG, "mx_grouped_gemm: null C");
  if (ldc < N) return fail(MX_ERR_INVALID_ARG, "mx_grouped_gemm: ldc=%lld < N=%lld", (long long)ldc, (long long)N);
  if ((M + 127) / 128 + E > 65535) return fail(MX_ERR_UNSUPPORTED, "mx_grouped_gemm: too many row tiles");
  if (((M + 255) / 256 + E) * ((N + 255) / 256) > 0x7FFFFFFF)
    return fail(MX_ERR_UNSUPPORTED, "mx_grouped_gemm: too many tiles");
  mx::GroupedGemmArgs a{};
  a.A = operand(A);
  a.B = operand(B);
  a.a_2d = false;
  a.b_2d = B->block == MX_BLOCK_2D;
  a.M_cap = M;
  a.N = N;
  a.K = A->K;
  a.offsets = d_group_offsets;
  a.E = E;
  a.stride_codes = expert_stride_codes;
  a.stride_scales = expert_stride_scales;
  a.C = C;
  a.ldc = ldc;
  a.out_bf16 = c_dtype == MX_DT_BF16;
  a.a_elem = A->elem;
  a.b_elem = B->elem;
  if ((a.a_elem != 0 || a.b_elem != 0) &&
      !(tile_offsets_fit(A, ldc * (a.out_bf16 ? 2 : 4)) && tile_offsets_fit(B, 0)))
    return fail(MX_ERR_UNSUPPORTED, "mx_grouped_gemm: row strides too large for the MXFP8/MXFP6 kernels");
  return hip_status(mx::launch_grouped_gemm(a, static_cast<hipStream_t>(stream)), "mx_grouped_gemm");
}

}  // extern "C"
