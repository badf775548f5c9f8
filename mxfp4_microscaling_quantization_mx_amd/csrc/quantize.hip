// MXFP4 quantizer kernels for gfx950.
//
// Method ("MXFP4", AI Wiki, §Conversion rules and §Clipping in the reference
// algorithm; options from §Training with MXFP4 and "Training an MoE LLM in
// MXFP4", summary): per 32-element block (or 32x32 tile) take amax, set the
// E8M0 exponent to floor(log2 amax) - 2, divide by the scale with one float32
// multiply, round to E2M1 by RNE or stochastic rounding, saturate at +-6, and
// optionally rotate each block by the 32-point randomized Hadamard transform
// first.  The kernels are bound by HBM bandwidth: 2 bytes in (bf16) and 0.53
// bytes out per element.
//
// Two kernel families:
//  * k_quant_rows_1d — blocks along the contiguous dim, one lane per block:
//    four 16-byte loads per lane, the whole 32-point transform and the amax in
//    registers, one 16-byte code store per lane.
//  * k_quant_tile — one lane per block, fed from an LDS tile.  Used for blocks
//    along dim 0 (the transposed output that wgrad and K x N weights need) and
//    for 2-D 32x32 tiles, whose amax is a reduction over 32 lanes.
#include "mx_device.h"
#include "mx_launch.h"

namespace mx {

namespace {

// ------------------------------------------------------------------ loads
// 8 consecutive source elements widened to float32, with the Hadamard sign
// flips applied as an XOR of the sign bits (exact).  sgn8 must be uniform
// across the wave.
template <bool BF16>
__device__ __forceinline__ void load8(const void* __restrict__ src, int64_t idx, float x[8],
                                      uint32_t sgn8) {
  if (BF16) {
    const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + idx);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // bit 15 flips the even element, bit 31 the odd one (sgn8 is the same
      // in every lane; one scalar register per word keeps it a single XOR)
      const uint32_t flip = __builtin_amdgcn_readfirstlane(
          (((sgn8 >> (2 * i)) & 1u) << 15) | (((sgn8 >> (2 * i + 1)) & 1u) << 31));
      const uint32_t v = ww[i] ^ flip;
      x[2 * i] = bf16lo(v);
      x[2 * i + 1] = bf16hi(v);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(src) + idx);
    const float4 a = p[0], b = p[1];
    const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = __uint_as_float(__float_as_uint(f[i]) ^ (((sgn8 >> i) & 1u) << 31));
  }
}

template <bool BF16>
__device__ __forceinline__ float load1(const void* __restrict__ src, int64_t idx) {
  if (BF16) return bf16lo(static_cast<const uint16_t*>(src)[idx]);
  return static_cast<const float*>(src)[idx];
}

// ------------------------------------------------------------------ rows, 1-D
// One lane per 32-element block: the lane reads its 64 contiguous source bytes
// (bf16) with four 16-byte loads, so a wave covers 4 KiB of consecutive input
// and writes 1 KiB of consecutive codes (one 16-byte store per lane) and 64
// consecutive scale bytes.  The whole 32-point transform stays in registers.
template <bool BF16>
__device__ __forceinline__ void load32(const void* __restrict__ src, int64_t idx, float x[32],
                                       uint32_t mask) {
#pragma unroll
  for (int j = 0; j < 4; ++j) load8<BF16>(src, idx + 8 * j, x + 8 * j, (mask >> (8 * j)) & 0xFFu);
}

// Quantize one block held in registers (x already sign-flipped when RHT).
// Returns the scale byte and writes the 16 code bytes to `packed`.
template <bool RHT, bool SR>
__device__ __forceinline__ uint32_t quantize_block32(float x[32], uint32_t packed[4], uint64_t p0,
                                                     uint64_t seed, uint64_t offset) {
  const float c = __uint_as_float(kRhtCBits);
  if (RHT) fwht32_inlane(x);
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) m = max(m, __float_as_uint(x[i]) & 0x7FFFFFFFu);
  if (RHT) {
    m = __float_as_uint(c * __uint_as_float(m));      // max |c t_i| = c max |t_i|
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = c * x[i];
  }
  const uint32_t s = scale_code_from_absmax_bits(m);
  packed[0] = packed[1] = packed[2] = packed[3] = 0u;
  if (s == 0xFFu) return s;
  if (SR) {
    const float inv = inv_scale_from_code(s);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint32_t w[4];
      sr_words((p0 >> 3) + g, seed, offset, w);
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = x[8 * g + i] * inv;
      packed[g] = pack8_sr(v, w);
    }
  } else {
    float sc = scale_f32_normal(s);
    if (s == 0u) {
      // scale 2^-127 is a float32 subnormal: multiply by 2^127 instead and
      // convert at scale 1 (the same single rounding)
#pragma unroll
      for (int i = 0; i < 32; ++i) x[i] = x[i] * __uint_as_float(0x7F000000u);
      sc = 1.0f;
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) packed[g] = pack8_rne(x + 8 * g, sc);
  }
  return s;
}

template <bool BF16, bool RHT, bool SR>
__global__ __launch_bounds__(256) void k_quant_rows_1d(const void* __restrict__ src, uint32_t nblocks,
                                                       uint32_t nkb, int64_t ld_src,
                                                       uint8_t* __restrict__ codes, int64_t ld_codes,
                                                       uint8_t* __restrict__ scales,
                                                       int64_t ld_scales, uint32_t mask,
                                                       uint64_t seed, uint64_t offset) {
  const uint32_t g = blockIdx.x * 256u + threadIdx.x;
  if (g >= nblocks) return;
  const uint32_t row = g / nkb;
  const uint32_t kb = g - row * nkb;
  float x[32];
  load32<BF16>(src, (int64_t)row * ld_src + 32 * kb, x, RHT ? mask : 0u);
  uint32_t packed[4];
  const uint64_t p0 = ((uint64_t)row * nkb + kb) * 32u;         // row * K + 32 kb
  const uint32_t s = quantize_block32<RHT, SR>(x, packed, p0, seed, offset);
  *reinterpret_cast<uint4*>(codes + (int64_t)row * ld_codes + 16 * kb) =
      make_uint4(packed[0], packed[1], packed[2], packed[3]);
  scales[(int64_t)row * ld_scales + kb] = (uint8_t)s;
}

// ------------------------------------------------------------------ LDS tiles
// TRANS: source tile of 128 rows x 64 columns; output rows are source columns
//        (lane -> column), K runs along source rows (wave w -> K-block w).
// !TRANS: source tile of 64 rows x 128 columns; lane -> row, wave w -> K-block w.
template <bool TRANS>
struct TileShape {
  static constexpr int TR = TRANS ? 128 : 64;   // source rows per tile
  static constexpr int TC = TRANS ? 64 : 128;   // source cols per tile
  static constexpr int LD = TRANS ? 64 : 129;   // LDS row pitch in floats (bank-conflict free reads)
};

template <bool TRANS, bool TWO_D, bool BF16, bool RHT, bool SR>
__global__ __launch_bounds__(256) void k_quant_tile(const void* __restrict__ src, int64_t R,
                                                    int64_t C, int64_t ld_src,
                                                    uint8_t* __restrict__ codes, int64_t ld_codes,
                                                    uint8_t* __restrict__ scales,
                                                    int64_t ld_scales, uint32_t mask,
                                                    uint64_t seed, uint64_t offset) {
  using S = TileShape<TRANS>;
  __shared__ float tile[S::TR * S::LD];

  const int64_t r0 = (int64_t)blockIdx.y * S::TR;
  const int64_t c0 = (int64_t)blockIdx.x * S::TC;

  // Stage the tile: 8 consecutive columns per load, TC/8 loads per row.
  constexpr int CHUNKS = S::TR * S::TC / 8;
#pragma unroll
  for (int it = 0; it < CHUNKS / 256; ++it) {
    const int id = threadIdx.x + 256 * it;
    const int tr = id / (S::TC / 8);
    const int tc = (id % (S::TC / 8)) * 8;
    const int64_t gr = r0 + tr, gc = c0 + tc;
    float x[8];
    if (gr < R && gc + 8 <= C) {
      load8<BF16>(src, gr * ld_src + gc, x, 0u);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        x[i] = (gr < R && gc + i < C) ? load1<BF16>(src, gr * ld_src + gc + i) : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) tile[tr * S::LD + tc + i] = x[i];
  }
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  // Output coordinates of this lane's block.
  const int64_t K = TRANS ? R : C;
  const int64_t orow = TRANS ? c0 + lane : r0 + lane;
  const int64_t kb = (TRANS ? r0 : c0) / 32 + w;
  const bool valid = (TRANS ? (orow < C) : (orow < R)) && (kb * 32 < K);

  float x[32];
#pragma unroll
  for (int i = 0; i < 32; ++i)
    x[i] = TRANS ? tile[(w * 32 + i) * S::LD + lane] : tile[lane * S::LD + w * 32 + i];
  const float c = __uint_as_float(kRhtCBits);
  if (RHT) {
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = __uint_as_float(__float_as_uint(x[i]) ^ (((mask >> i) & 1u) << 31));
    fwht32_inlane(x);
  }
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) m = max(m, __float_as_uint(x[i]) & 0x7FFFFFFFu);
  if (RHT) m = __float_as_uint(c * __uint_as_float(m));     // max |c t_i| = c max |t_i|
  if (!valid) m = 0;
  if (TWO_D) {
    // amax over the 32x32 tile = over the 32 lanes of this half-wave.
#pragma unroll
    for (int d = 1; d < 32; d <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, d, 32));
  }
  if (!valid) return;
  if (RHT) {
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = c * x[i];
  }
  const uint32_t s = scale_code_from_absmax_bits(m);
  uint32_t packed[4] = {0u, 0u, 0u, 0u};
  if (s != 0xFFu) {
    if (SR) {
      const float inv = inv_scale_from_code(s);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint32_t w[4];
        sr_words((uint64_t)(orow * K + kb * 32) / 8 + g, seed, offset, w);
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = x[8 * g + i] * inv;
        packed[g] = pack8_sr(v, w);
      }
    } else {
      float sc = scale_f32_normal(s);
      if (s == 0u) {
#pragma unroll
        for (int i = 0; i < 32; ++i) x[i] = x[i] * __uint_as_float(0x7F000000u);
        sc = 1.0f;
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) packed[g] = pack8_rne(x + 8 * g, sc);
    }
  }
  *reinterpret_cast<uint4*>(codes + orow * ld_codes + kb * 16) =
      make_uint4(packed[0], packed[1], packed[2], packed[3]);
  if (!TWO_D) {
    scales[orow * ld_scales + kb] = (uint8_t)s;
  } else if ((orow & 31) == 0) {
    scales[(orow >> 5) * ld_scales + kb] = (uint8_t)s;
  }
}

template <bool TRANS, bool TWO_D, bool BF16>
hipError_t launch_tile(const QuantArgs& a, hipStream_t st) {
  using S = TileShape<TRANS>;
  dim3 grid((unsigned)((a.C + S::TC - 1) / S::TC), (unsigned)((a.R + S::TR - 1) / S::TR));
#define MX_TILE(RHT_, SR_)                                                                   \
  hipLaunchKernelGGL((k_quant_tile<TRANS, TWO_D, BF16, RHT_, SR_>), grid, dim3(256), 0, st, \
                     a.src, a.R, a.C, a.ld_src, a.codes, a.ld_codes, a.scales, a.ld_scales,  \
                     a.mask, a.seed, a.offset)
  if (a.rht) {
    if (a.sr) MX_TILE(true, true); else MX_TILE(true, false);
  } else {
    if (a.sr) MX_TILE(false, true); else MX_TILE(false, false);
  }
#undef MX_TILE
  return hipGetLastError();
}

template <bool BF16>
hipError_t launch_rows_1d(const QuantArgs& a, hipStream_t st) {
  const uint32_t nkb = (uint32_t)(a.C / 32);
  const uint32_t nblocks = (uint32_t)(a.R * nkb);
  const unsigned grid = (nblocks + 255u) / 256u;
#define MX_ROWS(RHT_, SR_)                                                                   \
  hipLaunchKernelGGL((k_quant_rows_1d<BF16, RHT_, SR_>), dim3(grid), dim3(256), 0, st, a.src, \
                     nblocks, nkb, a.ld_src, a.codes, a.ld_codes, a.scales, a.ld_scales, a.mask, \
                     a.seed, a.offset)
  if (a.rht) {
    if (a.sr) MX_ROWS(true, true); else MX_ROWS(true, false);
  } else {
    if (a.sr) MX_ROWS(false, true); else MX_ROWS(false, false);
  }
#undef MX_ROWS
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize(const QuantArgs& a, hipStream_t st) {
  if (a.R == 0 || a.C == 0) return hipSuccess;
  if (!a.dim0 && !a.two_d) return a.bf16 ? launch_rows_1d<true>(a, st) : launch_rows_1d<false>(a, st);
  if (a.dim0) {
    if (a.two_d) return a.bf16 ? launch_tile<true, true, true>(a, st) : launch_tile<true, true, false>(a, st);
    return a.bf16 ? launch_tile<true, false, true>(a, st) : launch_tile<true, false, false>(a, st);
  }
  return a.bf16 ? launch_tile<false, true, true>(a, st) : launch_tile<false, true, false>(a, st);
}

}  // namespace mx
