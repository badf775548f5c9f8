// MXFP4 dequantizer for gfx950: value = E2M1(code) * 2^(scale - 127), with a
// NaN scale poisoning its whole block ("MXFP4", AI Wiki, §Format
// specification), and an optional inverse 32-point Hadamard transform.
//
// A quad of 4 lanes owns one 32-element block (8 codes = one 32-bit word per
// lane); the inverse transform runs stages 1/2/4 in-lane and 8/16 across the
// quad, then multiplies by c and applies the sign flips.
#include "mx_device.h"
#include "mx_launch.h"

namespace mx {
namespace {

// The 8 codes of one lane (elements col0 .. col0+7 of a row): E2M1 one 32-bit
// word of nibbles, FP8 8 bytes, FP6 6 bytes (element e at bits 6e).
template <int ELEM>
__device__ __forceinline__ void load_codes8(const uint8_t* p, uint32_t c[8]) {
  if constexpr (ELEM == 0) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = (w >> (4 * i)) & 15u;
  } else if constexpr (ElemT<ELEM>::BITS == 8) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = ((i < 4 ? w.x : w.y) >> (8 * (i & 3))) & 0xFFu;
  } else {
    const uint16_t* h = reinterpret_cast<const uint16_t*>(p);      // 6 bytes, 2-byte aligned
    const uint64_t w = (uint64_t)h[0] | ((uint64_t)h[1] << 16) | ((uint64_t)h[2] << 32);
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = (uint32_t)(w >> (6 * i)) & 0x3Fu;
  }
}

template <int ELEM>
__device__ __forceinline__ float code_value(uint32_t c) {
  if constexpr (ELEM == 0) return e2m1_value(c);
  else return elem_value<ELEM>(c);
}

template <bool OUT_BF16, bool IRHT, bool TWO_D, int ELEM>
__global__ __launch_bounds__(256) void k_dequant(const uint8_t* __restrict__ codes, int64_t ld_codes,
                                                 const uint8_t* __restrict__ scales,
                                                 int64_t ld_scales, int64_t rows, int64_t K,
                                                 void* __restrict__ dst, int64_t ld_dst,
                                                 uint32_t mask) {
  const int64_t lanes_per_row = K >> 3;
  const int64_t total = rows * lanes_per_row;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const uint32_t ql = threadIdx.x & 3u;
  const float c = __uint_as_float(kRhtCBits);
  for (int64_t l = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; l < total; l += stride) {
    const int64_t row = l / lanes_per_row;
    const int64_t col0 = (l - row * lanes_per_row) << 3;
    constexpr int BITS = elem_bits<ELEM>();
    uint32_t cd[8];
    load_codes8<ELEM>(codes + row * ld_codes + col0 * BITS / 8, cd);
    const uint32_t s = scales[(TWO_D ? (row >> 5) : row) * ld_scales + (col0 >> 5)];
    const float sv = scale_value(s);
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = code_value<ELEM>(cd[i]) * sv;
    if (IRHT) {
      fwht8_inlane(x);
      fwht_cross_quad(x, ql);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float y = x[i] * c;
        x[i] = __uint_as_float(__float_as_uint(y) ^ (((mask >> (8 * ql + i)) & 1u) << 31));
      }
    }
    if (OUT_BF16) {
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = f32_to_bf16_rne(x[2 * i]) | (f32_to_bf16_rne(x[2 * i + 1]) << 16);
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(dst) + row * ld_dst + col0) =
          make_uint4(w[0], w[1], w[2], w[3]);
    } else {
      float4* p = reinterpret_cast<float4*>(static_cast<float*>(dst) + row * ld_dst + col0);
      p[0] = make_float4(x[0], x[1], x[2], x[3]);
      p[1] = make_float4(x[4], x[5], x[6], x[7]);
    }
  }
}

template <int ELEM>
hipError_t launch_dequantize_elem(const DequantArgs& a, hipStream_t st) {
  const int64_t lanes = a.rows * (a.K / 8);
  int64_t blocks = (lanes + 255) / 256;
  if (blocks > 256 * 64) blocks = 256 * 64;
#define MX_DQ(B_, I_, T_)                                                                   \
  hipLaunchKernelGGL((k_dequant<B_, I_, T_, ELEM>), dim3((unsigned)blocks), dim3(256), 0, st, a.codes, \
                     a.ld_codes, a.scales, a.ld_scales, a.rows, a.K, a.dst, a.ld_dst, a.mask)
  if (a.out_bf16) {
    if (a.inverse_rht) { if (a.two_d) MX_DQ(true, true, true); else MX_DQ(true, true, false); }
    else { if (a.two_d) MX_DQ(true, false, true); else MX_DQ(true, false, false); }
  } else {
    if (a.inverse_rht) { if (a.two_d) MX_DQ(false, true, true); else MX_DQ(false, true, false); }
    else { if (a.two_d) MX_DQ(false, false, true); else MX_DQ(false, false, false); }
  }
#undef MX_DQ
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dequantize(const DequantArgs& a, hipStream_t st) {
  if (a.rows == 0 || a.K == 0) return hipSuccess;
  switch (a.elem) {
    case 1: return launch_dequantize_elem<1>(a, st);
    case 2: return launch_dequantize_elem<2>(a, st);
    case 3: return launch_dequantize_elem<3>(a, st);
    case 4: return launch_dequantize_elem<4>(a, st);
    default: return launch_dequantize_elem<0>(a, st);
  }
}

}  // namespace mx
