// Internal launch interface between the C-ABI layer (mx_api.cpp) and the
// kernel translation units.  Arguments are validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

struct QuantArgs {
  const void* src;
  int64_t R, C, ld_src;       // source [R, C], row stride in elements
  bool bf16;                  // else float32
  bool dim0;                  // blocks along dim 0 (output = quantized transpose)
  bool two_d;                 // 32x32 tiles
  bool rht;
  int sr;                     // stochastic rounding: 0 none, 1 16-bit draws, 2 8-bit draws
  uint32_t mask;
  uint64_t seed, offset;
  uint8_t* codes;
  int64_t ld_codes;
  uint8_t* scales;
  int64_t ld_scales;
  int scale_mode = 0;                // 0 reference rule, 1 round up, 2 prescale by 3/4
  const int32_t* gather = nullptr;   // device [R]: source row of each output row (last dim, 1-D only)
  int64_t R_src = 0;                 // source rows when gathering
  int elem = 0;                      // mx_elem of the output (0: FP4 E2M1)
};

struct DequantArgs {
  const uint8_t* codes;
  const uint8_t* scales;
  int64_t rows, K, ld_codes, ld_scales;
  bool two_d;
  bool inverse_rht;
  uint32_t mask;
  void* dst;
  bool out_bf16;
  int64_t ld_dst;
  int elem = 0;
};

// One MX operand as the GEMM kernels see it.
struct MxOperand {
  const uint8_t* codes;
  const uint8_t* scales;
  int64_t ld_codes, ld_scales;
};

struct GemmArgs {
  MxOperand A, B;
  bool a_2d, b_2d;
  int64_t M, N, K;
  void* C;
  int64_t ldc;
  bool out_bf16;
  int a_elem = 0, b_elem = 0;  // mx_elem of A and B
};

// C = A B^T quantized along N (MXFP4, 1-D blocks, RNE) in the GEMM epilogue.
struct GemmQuantArgs {
  MxOperand A, B;
  bool a_2d, b_2d;
  int64_t M, N, K;
  uint8_t* codes;
  uint8_t* scales;
  int64_t ld_codes, ld_scales;
  int scale_mode;
  int a_elem = 0, b_elem = 0;  // mx_elem of A and B (E2M1, or both MXFP8 / MXFP6)
};

// C = Q(A) B^T with A bf16 [M, K] (row stride lda elements) quantized to
// MXFP4 in the GEMM's operand load (RNE, 1-D blocks along K, optional
// transform with sign mask `mask`, scale_mode as mx_quantize); B MXFP4.
struct GemmQaArgs {
  const void* a;
  int64_t lda;
  bool rht;
  uint32_t mask;
  int scale_mode;
  MxOperand B;
  bool b_2d;
  int64_t M, N, K;
  void* C;
  int64_t ldc;
  bool out_bf16;
};

struct GroupedGemmArgs {
  MxOperand A, B;             // B = expert 0
  bool a_2d, b_2d;
  int64_t M_cap, N, K;
  const int32_t* offsets;     // device, E+1
  int32_t E;
  int64_t stride_codes, stride_scales;
  void* C;
  int64_t ldc;
  bool out_bf16;
  int a_elem = 0, b_elem = 0;  // mx_elem of A and B
};

// The grouped product quantized along N (MXFP4, 1-D blocks, RNE) in the
// epilogue: g describes the product (its C, ldc and out_bf16 are unused).
struct GroupedQuantArgs {
  GroupedGemmArgs g;
  uint8_t* codes;
  uint8_t* scales;
  int64_t ld_codes, ld_scales;
  int scale_mode;
};

struct TransposeArgs {
  const uint8_t* in_codes;
  const uint8_t* in_scales;
  int64_t R, C;               // input [R, C] elements, both multiples of 32
  int64_t ld_in, ld_sin;
  uint8_t* out_codes;
  uint8_t* out_scales;
  int64_t ld_out, ld_sout;
  int bits = 4;               // bits per element code (4, 6 or 8)
};

hipError_t launch_quantize(const QuantArgs& a, hipStream_t st);

// Clipping statistic: the elements that saturate when src is quantized with
// these settings, added to *count.
struct ClipArgs {
  const void* src;
  int64_t R, C, ld_src;       // source [R, C], row stride in elements
  bool bf16, dim0, two_d, rht;
  uint32_t mask;
  int scale_mode;
  int elem;
  unsigned long long* count;  // device
};
hipError_t launch_clip_count(const ClipArgs& a, hipStream_t st);
// MXFP4 RNE quantization of the a.R source rows, row t stored to output rows
// dest[t * k + j], j < k (those in [0, M)).
hipError_t launch_quantize_scatter(const QuantArgs& a, const int32_t* dest, int k, int64_t M, hipStream_t st);
hipError_t launch_transpose(const TransposeArgs& a, hipStream_t st);
hipError_t launch_dequantize(const DequantArgs& a, hipStream_t st);
hipError_t launch_gemm(const GemmArgs& a, hipStream_t st);
hipError_t launch_gemm_qa(const GemmQaArgs& a, hipStream_t st);
// Whether the 256x256 MXFP4 pipeline takes this problem's layout (16-byte
// scale rows, operands and output under 2 GiB, M and N >= 256).
bool gemm256_layout_ok(const GemmArgs& a);
// Split-K form of the 256x256 MXFP4 GEMM (gemm_splitk.hip): the workspace it
// needs for an M x N x K problem (0 when that shape is not split), whether it
// takes this problem, and its launch (workspace of that many bytes, 256-byte
// aligned, zero-filled before its first use and left so by every launch).
size_t gemm_splitk_workspace(int64_t M, int64_t N, int64_t K);
bool gemm_splitk_applies(const GemmArgs& a);
hipError_t launch_gemm_splitk(const GemmArgs& a, void* workspace, hipStream_t st);
// The library's own split-K workspace on the current device (a static device
// array, resolved once per device): its size and its device address.
size_t gemm_splitk_scratch_bytes();
hipError_t gemm_splitk_scratch(void** ptr);
// Whether the 256x256 pipeline (the only kernel with the quantizing epilogue)
// takes this problem; launch_gemm_quantize requires it.
bool gemm_quantize_supported(const GemmQuantArgs& a);
hipError_t launch_gemm_quantize(const GemmQuantArgs& a, hipStream_t st);
hipError_t launch_grouped_gemm(const GroupedGemmArgs& a, hipStream_t st);
// Whether the 256x256 grouped pipeline (the only grouped kernel with the
// quantizing epilogue) takes this problem; launch_grouped_gemm_quantize
// requires it.
bool grouped_quantize_supported(const GroupedQuantArgs& a);
hipError_t launch_grouped_gemm_quantize(const GroupedQuantArgs& a, hipStream_t st);

}  // namespace mx
