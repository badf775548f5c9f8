// MXFP4 quantizer kernels for gfx950.
//
// Method ("MXFP4", AI Wiki, §Conversion rules and §Clipping in the reference
// algorithm; options from §Training with MXFP4 and "Training an MoE LLM in
// MXFP4", summary): per 32-element block (or 32x32 tile) take amax, set the
// E8M0 exponent to floor(log2 amax) - 2, divide by the scale with one float32
// multiply, round to E2M1 by RNE or stochastic rounding, saturate at +-6, and
// optionally rotate each block by the 32-point randomized Hadamard transform
// first.  Without stochastic rounding the kernels are bound by HBM bandwidth
// (2 bytes in (bf16) and 0.53 bytes out per element); with it, by the VALU
// work of the Philox draws.
//
// Four kernels, each with one lane per 32-element block and the whole block
// (transform, amax, rounding) in registers:
//  * k_quant_rows_1d — blocks along the contiguous dim: four 16-byte loads per
//    lane, one 16-byte code store per lane; optionally of rows gathered by
//    index.
//  * k_quant_cols — blocks along dim 0 (the transposed output that wgrad and
//    K x N weights need), 1-D or 2-D: lane = source column, 32 loads of one
//    element per lane, each reading 64 consecutive columns across the wave.
//  * k_quant_rows_2d — 2-D 32x32 tiles along the contiguous dim: a half-wave
//    per tile, lane l the block of its row l, loaded as in the row kernel.
//  * k_quant_rows_scatter — the row kernel's block step once per source row,
//    stored to each of the row's k destination rows (MoE routing, RNE).
// For 2-D tiles the amax is a reduction over the 32 lanes of a half-wave.
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

// The same block step for the other MX element types (ELEM = mx_elem 1..4,
// FP8 or FP6): scale from the type's largest power of two, elements rounded
// (RNE: the hardware converts; SR: in software by elem_code with the same
// Philox draws as E2M1) and packed: FP8 one byte per element (8 words), FP6
// element e at bits 6e of the block's 192 bits (6 words).  Returns the scale
// byte.
template <int ELEM, bool RHT, int SR, bool TWO_D = false>
__device__ __forceinline__ uint32_t quantize_block32_elem(float x[32], uint32_t out[8], uint64_t p0, uint64_t seed,
                                                          uint64_t offset, int scale_mode) {
  using T = ElemT<ELEM>;
  const float c = __uint_as_float(kRhtCBits);
  if (RHT) fwht32_inlane(x);
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) m = max(m, __float_as_uint(x[i]) & 0x7FFFFFFFu);
  if (RHT) {
    m = __float_as_uint(c * __uint_as_float(m));
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = c * x[i];
  }
  if (TWO_D) {
#pragma unroll
    for (int d = 1; d < 32; d <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, d, 32));
  }
  const uint32_t s = elem_scale_code<ELEM>(m, scale_mode == 1);
#pragma unroll
  for (int j = 0; j < 8; ++j) out[j] = 0u;
  if (s == 0xFFu) return s;
  if (scale_mode == 2) {
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = 0.75f * x[i];
  }
  if constexpr (!SR) {
    // RNE through the hardware converts (pack4_fp8 / pack32_fp6), which
    // divide by the scale themselves; scale byte 0 (2^-127, a float32
    // subnormal) goes in as x 2^127 at scale 1, the same single rounding.
    float sc = scale_f32_normal(s);
    if (s == 0u) {
#pragma unroll
      for (int i = 0; i < 32; ++i) x[i] = x[i] * __uint_as_float(0x7F000000u);
      sc = 1.0f;
    }
    const float lim = __uint_as_float(T::MAXBITS) * sc;
    if constexpr (T::BITS == 8) {
#pragma unroll
      for (int j = 0; j < 8; ++j) out[j] = pack4_fp8<ELEM>(x + 4 * j, sc, lim);
    } else {
      pack32_fp6<ELEM>(x, sc, lim, out);
    }
    return s;
  }
  const float inv = inv_scale_from_code(s);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if constexpr (SR == 2) sr_words((p0 >> 4) + (g >> 1), seed, offset, w);
    else if constexpr (SR == 1) sr_words((p0 >> 3) + g, seed, offset, w);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = 8 * g + i;
      // 16-bit draws: half (i & 1) of word i >> 1; 8-bit: byte (i16 & 3) of
      // word i16 >> 2 of the call's 16 elements, as the 16-bit draw 256 b
      const int i16 = 8 * (g & 1) + i;
      const uint32_t r16 = SR == 2 ? ((w[i16 >> 2] >> (8 * (i16 & 3))) & 0xFFu) << 8
                           : SR ? (w[i >> 1] >> (16 * (i & 1))) & 0xFFFFu : 0u;
      const uint32_t code = elem_code<ELEM, (SR != 0)>(x[e] * inv, r16);
      if (T::BITS == 8) {
        out[e >> 2] |= code << (8 * (e & 3));
      } else {
        const int bit = 6 * e;
        out[bit >> 5] |= code << (bit & 31);
        if ((bit & 31) > 26) out[(bit >> 5) + 1] |= code >> (32 - (bit & 31));
      }
    }
  }
  return s;
}

// Store one block's codes (E2M1: 16 bytes, FP6: 24, FP8: 32) at dst, which is
// aligned to the block size's power-of-two part.
template <int ELEM>
__device__ __forceinline__ void store_block(uint8_t* dst, const uint32_t w[8]) {
  if constexpr (ELEM == 0) {
    *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
  } else if constexpr (ElemT<ELEM>::BITS == 8) {
    *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
    *reinterpret_cast<uint4*>(dst + 16) = make_uint4(w[4], w[5], w[6], w[7]);
  } else {
    *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
    *reinterpret_cast<uint2*>(dst + 8) = make_uint2(w[2], w[3]);
    *reinterpret_cast<uint2*>(dst + 16) = make_uint2(w[4], w[5]);
  }
}

// Code bytes of one 32-element block.
template <int ELEM>
constexpr int block_bytes() {
  return 4 * elem_bits<ELEM>();
}

// Quantize one block of element type ELEM (E2M1 through the hardware-convert
// path above) and store its codes at dst; returns the scale byte.
template <int ELEM, bool RHT, int SR, bool TWO_D = false>
__device__ __forceinline__ uint32_t quantize_store(float x[32], uint8_t* dst, uint64_t p0, uint64_t seed,
                                                   uint64_t offset, int scale_mode) {
  uint32_t w[8];
  uint32_t s;
  if constexpr (ELEM == 0) {
    s = quantize_block32<RHT, SR, TWO_D>(x, w, p0, seed, offset, scale_mode);
  } else {
    s = quantize_block32_elem<ELEM, RHT, SR, TWO_D>(x, w, p0, seed, offset, scale_mode);
  }
  store_block<ELEM>(dst, w);
  return s;
}

// GATHER: output row r quantizes source row gidx[r] (the routed rows of an MoE
// layer read straight from the token activations); an index outside
// [0, R_src) gives the row NaN blocks (scale byte 0xFF, codes 0).
template <bool BF16, bool RHT, int SR, bool GATHER, int ELEM>
__global__ __launch_bounds__(256) void k_quant_rows_1d(const void* __restrict__ src, uint32_t nblocks,
                                                       uint32_t nkb, int64_t ld_src,
                                                       uint8_t* __restrict__ codes, int64_t ld_codes,
                                                       uint8_t* __restrict__ scales,
                                                       int64_t ld_scales, uint32_t mask,
                                                       uint64_t seed, uint64_t offset, int scale_mode,
                                                       const int32_t* __restrict__ gidx, int64_t R_src) {
  const uint32_t g = blockIdx.x * 256u + threadIdx.x;
  if (g >= nblocks) return;
  const uint32_t row = g / nkb;
  const uint32_t kb = g - row * nkb;
  int64_t srow = row;
  if (GATHER) {
    srow = gidx[row];
    if (srow < 0 || srow >= R_src) {
      *reinterpret_cast<uint4*>(codes + (int64_t)row * ld_codes + 16 * kb) = make_uint4(0u, 0u, 0u, 0u);
      scales[(int64_t)row * ld_scales + kb] = 0xFFu;
      return;
    }
  }
  float x[32];
  load32<BF16>(src, srow * ld_src + 32 * kb, x, RHT ? mask : 0u);
  const uint64_t p0 = ((uint64_t)row * nkb + kb) * 32u;         // output row * K + 32 kb
  const uint32_t s = quantize_store<ELEM, RHT, SR>(
      x, codes + (int64_t)row * ld_codes + block_bytes<ELEM>() * kb, p0, seed, offset, scale_mode);
  scales[(int64_t)row * ld_scales + kb] = (uint8_t)s;
}

// ------------------------------------------------------------------ rows, 2-D
// 32x32 tiles along the last dim straight from global memory: each half-wave
// takes one tile and lane l of it the block of tile row l (its 32 source
// elements in four 16-byte loads for bf16, as in the 1-D row kernel), so the
// tile's amax is a reduction over the 32 lanes of the half-wave (the same
// register path as the dim-0 2-D kernel).  Consecutive half-waves take
// consecutive K-blocks of the same 32 rows, so a wave reads whole 128-byte
// pieces of each row.  The rows are a multiple of 32 (2-D blocks).
template <bool BF16, bool RHT, int SR, int ELEM>
__global__ __launch_bounds__(256) void k_quant_rows_2d(const void* __restrict__ src, uint32_t ntiles, uint32_t nkb,
                                                       int64_t ld_src, uint8_t* __restrict__ codes, int64_t ld_codes,
                                                       uint8_t* __restrict__ scales, int64_t ld_scales, uint32_t mask,
                                                       uint64_t seed, uint64_t offset, int scale_mode) {
  const uint32_t t = blockIdx.x * 8u + (threadIdx.x >> 5);   // this half-wave's tile
  if (t >= ntiles) return;                                   // whole half-waves leave together
  const uint32_t tr = t / nkb, kb = t - tr * nkb;
  const int64_t row = (int64_t)tr * 32 + (threadIdx.x & 31);
  float x[32];
  load32<BF16>(src, row * ld_src + 32 * (int64_t)kb, x, RHT ? mask : 0u);
  const uint64_t p0 = ((uint64_t)row * nkb + kb) * 32u;      // output row * K + 32 kb
  const uint32_t s = quantize_store<ELEM, RHT, SR, true>(x, codes + row * ld_codes + block_bytes<ELEM>() * kb, p0,
                                                          seed, offset, scale_mode);
  if ((threadIdx.x & 31) == 0) scales[(int64_t)tr * ld_scales + kb] = (uint8_t)s;
}

// ------------------------------------------------------------------ columns (blocks along dim 0)
// Blocks along dim 0 without an LDS input tile: lane = source column (= output
// row); the COLS_KB waves of a workgroup take the K-blocks
// [COLS_KB y, COLS_KB (y + 1)) of its 64 columns, one each (two blocks per wave in turn
// measured 5-12 % slower: half the loads in flight).  Each of the 32 loads of a block
// reads one element per lane; across the wave it reads 64 consecutive columns
// of one source row.  The blocks go through the same register path as a row
// block.  Their codes and scale bytes are gathered in LDS, so that each output
// row's COLS_KB blocks (MXFP4, 16 blocks: 256 contiguous code bytes, two cache
// lines, and 16 scale bytes) leave as whole 16-byte pieces from consecutive lanes, instead
// of every store instruction putting one 16-byte piece into each of 64 rows
// (the bytes written drop from 1.63x to 1.06x the output).  2-D: a half-wave
// holds one 32x32 tile (output rows are a multiple of 32, so half-waves are
// whole or past the end).
// COLS_KB K-blocks per workgroup, one per wave: 16, or 8 where 16 would give
// fewer than 4 workgroups per CU (a 5760 x 2880 weight: 540 workgroups of 16
// waves took 15.1 us after a cache-evicting read, 1080 of 8 waves 13.7 us, 2160
// of 4 waves no better; the 16384 x 2880 activations run 0.4-1.4 us faster
// with 16).
template <int COLS_KB, bool TWO_D, bool BF16, bool RHT, int SR, int ELEM>
__global__ __launch_bounds__(64 * COLS_KB) void k_quant_cols(const void* __restrict__ src, int64_t R, int64_t C,
                                                    int64_t ld_src, uint8_t* __restrict__ codes,
                                                    int64_t ld_codes, uint8_t* __restrict__ scales,
                                                    int64_t ld_scales, uint32_t mask, uint64_t seed,
                                                    uint64_t offset, int scale_mode) {
  constexpr int COLS_THREADS = 64 * COLS_KB;
  constexpr int BB = block_bytes<ELEM>();
  constexpr int RB = COLS_KB * BB;           // code bytes of one output row here (a multiple of 16)
  constexpr int PITCH = RB + 16;             // LDS row pitch: rows start in different banks
  __shared__ __attribute__((aligned(16))) uint8_t lc[64 * PITCH];
  __shared__ uint8_t ls[64 * COLS_KB];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t col0 = (int64_t)blockIdx.x * 64;
  const int64_t col = col0 + lane;
  const int64_t kb0 = (int64_t)blockIdx.y * COLS_KB;
  const int64_t nkb = R / 32;
  constexpr int ES = BF16 ? 2 : 4;
  // lanes past the last column read the last column (their blocks are never
  // stored; for 2-D they form whole half-waves of their own)
  const uint32_t voff = (uint32_t)((col < C ? col : C - 1) * ES);
  const int kl = w;                          // this wave's K-block
  const int64_t kb = kb0 + kl;
  if (kb < nkb) {                            // wave-uniform
    // a raw buffer over the block's 32 source rows: per-lane column offset,
    // wave-uniform row offsets
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(static_cast<const uint8_t*>(src) + kb * 32 * ld_src * ES), 0,
        (uint32_t)(31 * ld_src * ES + C * ES), 0x00020000);
    float x[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t soff = (uint32_t)(i * ld_src * ES);
      uint32_t b = BF16 ? ((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rs, voff, soff, 0) << 16)
                        : __builtin_amdgcn_raw_buffer_load_b32(rs, voff, soff, 0);
      if (RHT) b ^= ((mask >> i) & 1u) << 31;
      x[i] = __uint_as_float(b);
    }
    const uint64_t p0 = (uint64_t)col * (uint64_t)R + (uint64_t)kb * 32u;   // output row * K + 32 kb
    ls[lane * COLS_KB + kl] =
        (uint8_t)quantize_store<ELEM, RHT, SR, TWO_D>(x, lc + lane * PITCH + kl * BB, p0, seed, offset, scale_mode);
  }
  __syncthreads();
  const int nvalid = (int)(nkb - kb0 < COLS_KB ? nkb - kb0 : COLS_KB);
  const int vbytes = nvalid * BB;            // a multiple of 8
  constexpr int PIECES = RB / 16;
#pragma unroll
  for (int i = threadIdx.x; i < 64 * PIECES; i += COLS_THREADS) {
    const int r = i / PIECES, off = 16 * (i - r * PIECES);
    const int64_t orow = col0 + r;
    if (orow < C && off < vbytes) {
      uint8_t* g = codes + orow * ld_codes + kb0 * BB + off;
      const uint4 v = *reinterpret_cast<const uint4*>(lc + r * PITCH + off);
      if (off + 16 <= vbytes) *reinterpret_cast<uint4*>(g) = v;
      else *reinterpret_cast<uint2*>(g) = make_uint2(v.x, v.y);   // an FP6 row ending mid-piece
    }
  }
  if (!TWO_D) {
#pragma unroll
    for (int i = threadIdx.x; i < 64 * COLS_KB; i += COLS_THREADS) {
      const int r = i / COLS_KB, k = i - r * COLS_KB;
      if (col0 + r < C && k < nvalid) scales[(col0 + r) * ld_scales + kb0 + k] = ls[i];
    }
  } else if (threadIdx.x < 2 * COLS_KB) {
    const int r = 32 * (threadIdx.x / COLS_KB), k = threadIdx.x % COLS_KB;
    if (col0 + r < C && k < nvalid) scales[((col0 + r) >> 5) * ld_scales + kb0 + k] = ls[r * COLS_KB + k];
  }
}

// Launch M_ with the stochastic-rounding variant of a.sr (0 none, 1 16-bit
// draws, 2 8-bit draws).
#define MX_SR3(M_, RHT_)  \
  if (a.sr == 2)          \
    M_(RHT_, 2);          \
  else if (a.sr == 1)     \
    M_(RHT_, 1);          \
  else                    \
    M_(RHT_, 0)

template <int KB, bool TWO_D, bool BF16, int ELEM>
hipError_t launch_cols_kb(const QuantArgs& a, hipStream_t st) {
  dim3 grid((unsigned)((a.C + 63) / 64), (unsigned)((a.R + 32 * KB - 1) / (32 * KB)));
#define MX_COLS(RHT_, SR_)                                                                                      \
  hipLaunchKernelGGL((k_quant_cols<KB, TWO_D, BF16, RHT_, SR_, ELEM>), grid, dim3(64 * KB), 0, st, a.src, a.R, a.C, \
                     a.ld_src, a.codes, a.ld_codes, a.scales, a.ld_scales, a.mask, a.seed, a.offset, a.scale_mode)
  if (a.rht) {
    MX_SR3(MX_COLS, true);
  } else {
    MX_SR3(MX_COLS, false);
  }
#undef MX_COLS
  return hipGetLastError();
}

template <bool TWO_D, bool BF16, int ELEM>
hipError_t launch_cols(const QuantArgs& a, hipStream_t st) {
  const int64_t wg16 = ((a.C + 63) / 64) * ((a.R + 511) / 512);
  return wg16 < 4 * 256 ? launch_cols_kb<8, TWO_D, BF16, ELEM>(a, st) : launch_cols_kb<16, TWO_D, BF16, ELEM>(a, st);
}

template <bool BF16, int ELEM>
hipError_t launch_tile(const QuantArgs& a, hipStream_t st) {
  const uint32_t nkb = (uint32_t)(a.C / 32);
  const uint32_t ntiles = (uint32_t)(a.R / 32) * nkb;
  const unsigned grid = (ntiles + 7u) / 8u;
#define MX_R2D(RHT_, SR_)                                                                                    \
  hipLaunchKernelGGL((k_quant_rows_2d<BF16, RHT_, SR_, ELEM>), dim3(grid), dim3(256), 0, st, a.src, ntiles, nkb,   \
                     a.ld_src, a.codes, a.ld_codes, a.scales, a.ld_scales, a.mask, a.seed, a.offset, a.scale_mode)
  if (a.rht) {
    MX_SR3(MX_R2D, true);
  } else {
    MX_SR3(MX_R2D, false);
  }
#undef MX_R2D
  return hipGetLastError();
}

template <bool BF16, bool GATHER, int ELEM>
hipError_t launch_rows_1d(const QuantArgs& a, hipStream_t st) {
  const uint32_t nkb = (uint32_t)(a.C / 32);
  const uint32_t nblocks = (uint32_t)(a.R * nkb);
  const unsigned grid = (nblocks + 255u) / 256u;
#define MX_ROWS(RHT_, SR_)                                                                            \
  hipLaunchKernelGGL((k_quant_rows_1d<BF16, RHT_, SR_, GATHER, ELEM>), dim3(grid), dim3(256), 0, st, a.src, \
                     nblocks, nkb, a.ld_src, a.codes, a.ld_codes, a.scales, a.ld_scales, a.mask,    \
                     a.seed, a.offset, a.scale_mode, a.gather, a.R_src)
  if (a.rht) {
    MX_SR3(MX_ROWS, true);
  } else {
    MX_SR3(MX_ROWS, false);
  }
#undef MX_ROWS
  return hipGetLastError();
}

// Kernel choice for one element type: gather and 1-D last-dim blocks by rows,
// dim 0 by columns (1-D or 2-D), 2-D last-dim tiles by half-waves.
template <int ELEM>
hipError_t launch_quantize_elem(const QuantArgs& a, hipStream_t st) {
  if (a.gather) {
    if constexpr (ELEM == 0)
      return a.bf16 ? launch_rows_1d<true, true, 0>(a, st) : launch_rows_1d<false, true, 0>(a, st);
    return hipErrorInvalidValue;                 // validated by the caller: MXFP4 only
  }
  if (a.dim0) {
    if (a.two_d) return a.bf16 ? launch_cols<true, true, ELEM>(a, st) : launch_cols<true, false, ELEM>(a, st);
    return a.bf16 ? launch_cols<false, true, ELEM>(a, st) : launch_cols<false, false, ELEM>(a, st);
  }
  if (a.two_d) return a.bf16 ? launch_tile<true, ELEM>(a, st) : launch_tile<false, ELEM>(a, st);
  return a.bf16 ? launch_rows_1d<true, false, ELEM>(a, st) : launch_rows_1d<false, false, ELEM>(a, st);
}

// Scatter form (MXFP4, RNE): one lane per block of a source row, quantized
// once and stored to each of the row's k destination rows dest[t * k + j]
// (destinations outside [0, M) are skipped).  With RNE a row's codes do not
// depend on where it goes, so this equals quantizing the gathered copy.
template <bool BF16, bool RHT>
__global__ __launch_bounds__(256) void k_quant_rows_scatter(const void* __restrict__ src, uint32_t nblocks,
                                                            uint32_t nkb, int64_t ld_src, uint8_t* __restrict__ codes,
                                                            int64_t ld_codes, uint8_t* __restrict__ scales,
                                                            int64_t ld_scales, uint32_t mask, int scale_mode,
                                                            const int32_t* __restrict__ dest, int k, int64_t M) {
  const uint32_t g = blockIdx.x * 256u + threadIdx.x;
  if (g >= nblocks) return;
  const uint32_t row = g / nkb;
  const uint32_t kb = g - row * nkb;
  float x[32];
  load32<BF16>(src, (int64_t)row * ld_src + 32 * kb, x, RHT ? mask : 0u);
  uint32_t packed[4];
  const uint32_t s = quantize_block32<RHT, 0>(x, packed, 0u, 0u, 0u, scale_mode);
  const uint4 v = make_uint4(packed[0], packed[1], packed[2], packed[3]);
  for (int j = 0; j < k; ++j) {
    const int64_t d = dest[(int64_t)row * k + j];
    if (d < 0 || d >= M) continue;
    *reinterpret_cast<uint4*>(codes + d * ld_codes + 16 * kb) = v;
    scales[d * ld_scales + kb] = (uint8_t)s;
  }
}

}  // namespace

hipError_t launch_quantize_scatter(const QuantArgs& a, const int32_t* dest, int k, int64_t M, hipStream_t st) {
  if (a.R == 0 || a.C == 0 || k == 0) return hipSuccess;
  const uint32_t nkb = (uint32_t)(a.C / 32);
  const uint32_t nblocks = (uint32_t)(a.R * nkb);
  const unsigned grid = (nblocks + 255u) / 256u;
#define MX_SC(BF_, RHT_)                                                                                   \
  hipLaunchKernelGGL((k_quant_rows_scatter<BF_, RHT_>), dim3(grid), dim3(256), 0, st, a.src, nblocks, nkb, \
                     a.ld_src, a.codes, a.ld_codes, a.scales, a.ld_scales, a.mask, a.scale_mode, dest, k, M)
  if (a.bf16) {
    if (a.rht) MX_SC(true, true); else MX_SC(true, false);
  } else {
    if (a.rht) MX_SC(false, true); else MX_SC(false, false);
  }
#undef MX_SC
  return hipGetLastError();
}

hipError_t launch_quantize(const QuantArgs& a, hipStream_t st) {
  if (a.R == 0 || a.C == 0) return hipSuccess;
  switch (a.elem) {
    case 1: return launch_quantize_elem<1>(a, st);
    case 2: return launch_quantize_elem<2>(a, st);
    case 3: return launch_quantize_elem<3>(a, st);
    case 4: return launch_quantize_elem<4>(a, st);
    default: return launch_quantize_elem<0>(a, st);
  }
}

}  // namespace mx
