// MXFP4 dequantizer for gfx950: value = E2M1(code) * 2^(scale - 127), with a
// NaN scale poisoning its whole block ("MXFP4", AI Wiki, §Format
// specification), and an optional inverse 32-point Hadamard transform.
//
// Without the inverse transform a quad of 4 lanes owns one 32-element block
// (8 codes = one 32-bit word per lane for E2M1); with it one lane owns the
// block and runs all five butterfly stages in registers, then multiplies by c
// and applies the sign flips.
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

template <bool OUT_BF16, bool IRHT, bool TWO_D, int ELEM, class IDX>
__global__ __launch_bounds__(256) void k_dequant(const uint8_t* __restrict__ codes, int64_t ld_codes,
                                                 const uint8_t* __restrict__ scales,
                                                 int64_t ld_scales, int64_t rows, int64_t K,
                                                 void* __restrict__ dst, int64_t ld_dst,
                                                 uint32_t mask) {
  // lanes are counted in IDX (32 bits unless rows * K / 8 comes near 2^32:
  // a 64-bit division per lane is a long VALU sequence)
  const IDX lanes_per_row = (IDX)(K >> 3);
  const IDX total = (IDX)(rows * (K >> 3));
  const IDX stride = (IDX)gridDim.x * blockDim.x;
  const uint32_t ql = threadIdx.x & 3u;
  const float c = __uint_as_float(kRhtCBits);
  constexpr int BITS = elem_bits<ELEM>();
  if constexpr (!IRHT) {
    // two positions per pass, l and l + stride, both loads issued first
    auto where = [&](IDX l, int64_t& row, int64_t& col0) {
      const IDX r = l / lanes_per_row;
      row = (int64_t)r;
      col0 = (int64_t)(l - r * lanes_per_row) << 3;
    };
    auto finish = [&](const uint32_t cd[8], uint32_t s, int64_t row, int64_t col0) {
      const float sv = scale_value(s);
      float x[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = code_value<ELEM>(cd[i]) * sv;
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
    };
    for (IDX l = (IDX)blockIdx.x * blockDim.x + threadIdx.x; l < total; l += 2 * stride) {
      int64_t row0, c00, row1 = 0, c01 = 0;
      where(l, row0, c00);
      const bool two = l + stride < total;
      uint32_t cd0[8], cd1[8], s1 = 0;
      load_codes8<ELEM>(codes + row0 * ld_codes + c00 * BITS / 8, cd0);
      const uint32_t s0 = scales[(TWO_D ? (row0 >> 5) : row0) * ld_scales + (c00 >> 5)];
      if (two) {
        where(l + stride, row1, c01);
        load_codes8<ELEM>(codes + row1 * ld_codes + c01 * BITS / 8, cd1);
        s1 = scales[(TWO_D ? (row1 >> 5) : row1) * ld_scales + (c01 >> 5)];
      }
      finish(cd0, s0, row0, c00);
      if (two) finish(cd1, s1, row1, c01);
    }
    return;
  }
  for (IDX l = (IDX)blockIdx.x * blockDim.x + threadIdx.x; l < total; l += stride) {
    const IDX r = l / lanes_per_row;
    const int64_t row = (int64_t)r;
    const int64_t col0 = (int64_t)(l - r * lanes_per_row) << 3;
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

// With the inverse transform: one lane per 32-element block, its codes in
// one (E2M1), two (FP8) or three (FP6) wide loads, the transform wholly in
// registers (the same stages, sums and rounding as the quad form, so the same
// bits) and its 32 outputs in 16-byte stores.  No cross-lane exchanges; a few
// per cent faster than the quad form there, a little slower without the
// transform, where the quad form's fully contiguous stores win.
template <int ELEM>
__device__ __forceinline__ void load_codes32(const uint8_t* p, uint32_t c[32]) {
  if constexpr (ELEM == 0) {
    const uint4 w = *reinterpret_cast<const uint4*>(p);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 32; ++i) c[i] = (ww[i >> 3] >> (4 * (i & 7))) & 15u;
  } else if constexpr (ElemT<ELEM>::BITS == 8) {
    const uint4 w0 = *reinterpret_cast<const uint4*>(p);
    const uint4 w1 = *reinterpret_cast<const uint4*>(p + 16);
    const uint32_t ww[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
    for (int i = 0; i < 32; ++i) c[i] = (ww[i >> 2] >> (8 * (i & 3))) & 0xFFu;
  } else {
    const uint2 w0 = *reinterpret_cast<const uint2*>(p);
    const uint2 w1 = *reinterpret_cast<const uint2*>(p + 8);
    const uint2 w2 = *reinterpret_cast<const uint2*>(p + 16);
    const uint32_t ww[6] = {w0.x, w0.y, w1.x, w1.y, w2.x, w2.y};
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int bit = 6 * i;
      uint32_t v = ww[bit >> 5] >> (bit & 31);
      if ((bit & 31) > 26) v |= ww[(bit >> 5) + 1] << (32 - (bit & 31));
      c[i] = v & 0x3Fu;
    }
  }
}

template <bool OUT_BF16, bool IRHT, bool TWO_D, int ELEM>
__global__ __launch_bounds__(256) void k_dequant32(const uint8_t* __restrict__ codes, int64_t ld_codes,
                                                   const uint8_t* __restrict__ scales, int64_t ld_scales,
                                                   uint32_t nkb, uint32_t nblocks, void* __restrict__ dst,
                                                   int64_t ld_dst, uint32_t mask) {
  const uint32_t g = blockIdx.x * 256u + threadIdx.x;
  if (g >= nblocks) return;
  const uint32_t r = g / nkb, kb = g - r * nkb;
  const int64_t row = r;
  constexpr int BB = elem_bits<ELEM>() * 4;                   // code bytes per block
  uint32_t cd[32];
  load_codes32<ELEM>(codes + row * ld_codes + (int64_t)kb * BB, cd);
  const float sv = scale_value(scales[(TWO_D ? (row >> 5) : row) * ld_scales + kb]);
  float x[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) x[i] = code_value<ELEM>(cd[i]) * sv;
  if (IRHT) {
    const float c = __uint_as_float(kRhtCBits);
    fwht32_inlane(x);
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = __uint_as_float(__float_as_uint(x[i] * c) ^ (((mask >> i) & 1u) << 31));
  }
  const int64_t col0 = (int64_t)kb * 32;
  if (OUT_BF16) {
    uint4* p = reinterpret_cast<uint4*>(static_cast<uint16_t*>(dst) + row * ld_dst + col0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = f32_to_bf16_rne(x[8 * q + 2 * i]) | (f32_to_bf16_rne(x[8 * q + 2 * i + 1]) << 16);
      p[q] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  } else {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(dst) + row * ld_dst + col0);
#pragma unroll
    for (int q = 0; q < 8; ++q) p[q] = make_float4(x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]);
  }
}

template <int ELEM>
hipError_t launch_dequantize_elem(const DequantArgs& a, hipStream_t st) {
  const int64_t nblocks = a.rows * (a.K / 32);
  if (a.inverse_rht && nblocks < (1ll << 32) - 256) {
    const unsigned grid = (unsigned)((nblocks + 255) / 256);
#define MX_DQ32(B_, I_, T_)                                                                                    \
    hipLaunchKernelGGL((k_dequant32<B_, I_, T_, ELEM>), dim3(grid), dim3(256), 0, st, a.codes, a.ld_codes,      \
                       a.scales, a.ld_scales, (uint32_t)(a.K / 32), (uint32_t)nblocks, a.dst, a.ld_dst, a.mask)
    if (a.out_bf16) {
      if (a.inverse_rht) { if (a.two_d) MX_DQ32(true, true, true); else MX_DQ32(true, true, false); }
      else { if (a.two_d) MX_DQ32(true, false, true); else MX_DQ32(true, false, false); }
    } else {
      if (a.inverse_rht) { if (a.two_d) MX_DQ32(false, true, true); else MX_DQ32(false, true, false); }
      else { if (a.two_d) MX_DQ32(false, false, true); else MX_DQ32(false, false, false); }
    }
#undef MX_DQ32
    return hipGetLastError();
  }
  // the quad form: a grid of at most 32 workgroups per CU striding over the
  // lanes, two positions per lane and pass without the transform (16384 x
  // 2880 to bf16: 37.8 us with 64 workgroups per CU and one position per
  // pass, 36.7 with 32, 35.6 with 32 and two; 16 and two 36.2), with 32-bit
  // lane indices while the loop cannot wrap (total + 2 stride < 2^32)
  const int64_t lanes = a.rows * (a.K / 8);
  int64_t blocks = (lanes + 255) / 256;
  if (blocks > 256 * 32) blocks = 256 * 32;
  const bool small = lanes < (1ll << 32) - 2ll * 256 * 32 * 256;   // l + 2 stride cannot wrap
  // (with the transform this path only sees more than 2^32 - 256 blocks, so
  // never 32-bit indices)
#define MX_DQ(B_, I_, T_)                                                                                   \
  if (!(I_) && small)                                                                                       \
    hipLaunchKernelGGL((k_dequant<B_, false, T_, ELEM, uint32_t>), dim3((unsigned)blocks), dim3(256), 0, st, \
                       a.codes, a.ld_codes, a.scales, a.ld_scales, a.rows, a.K, a.dst, a.ld_dst, a.mask);   \
  else                                                                                                      \
    hipLaunchKernelGGL((k_dequant<B_, I_, T_, ELEM, int64_t>), dim3((unsigned)blocks), dim3(256), 0, st,    \
                       a.codes, a.ld_codes, a.scales, a.ld_scales, a.rows, a.K, a.dst, a.ld_dst, a.mask)
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
