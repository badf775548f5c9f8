// Exact transpose of an MX operand quantized with 32x32 (2-D) blocks, for
// gfx950 (MXFP4 below; MXFP8 / MXFP6 in k_transpose_2d_bytes).  A 32x32 tile has one shared scale, so the transposed tile is the
// same block: its codes are the tile's codes transposed and its scale byte is
// unchanged.  This is what lets one 2-D quantization of a weight serve both
// the forward product and, transposed, the data-gradient product (the hybrid
// 1D/2D block quantization of "Training an MoE LLM in MXFP4: How We Closed the
// Gap to BF16", summary).  Nothing is re-rounded, so the result is bit-exact
// whatever rounding produced the input.
//
// A 256-thread workgroup owns a 128 x 128 element tile of the input (128 rows
// x 64 code bytes): 16-byte loads into LDS, then each thread transposes one
// 8 x 8 block of nibbles in registers (three rounds of masked swaps: the 4 x 4
// quadrants, then 2 x 2 sub-blocks, then single nibbles) and writes its 8
// words to an output tile in LDS, from which the 128 output rows leave as
// 16-byte stores.  The 4 x 4 scale bytes of the tile are copied transposed by
// 16 threads.
#include "mx_launch.h"

namespace mx {
namespace {

constexpr int TT = 128;        // tile edge in elements
constexpr int IP = 18;         // input tile row pitch in words (16 + 2: conflict-free block reads)
constexpr int OP = 17;         // output tile row pitch in words

// Tile origin (r0, c0) of this workgroup.  Workgroups go to the 8 XCDs in
// turn by launch index, so launch index L takes tile (L mod 8) * q + L / 8 of
// the row-major tile order (q tiles per XCD, the first n mod 8 XCDs one
// more): neighbouring tiles of a tile row, which read the two halves of the
// same 128-byte input lines (MXFP4), then run on one XCD at about the same
// time and share its L2, instead of each XCD fetching whole lines for half
// of them.
__device__ __forceinline__ void tile_origin(int64_t gx, int64_t n, int64_t& r0, int64_t& c0) {
  const int64_t L = blockIdx.x, x = L & 7, base = n >> 3, rem = n & 7;
  const int64_t T = x * base + (x < rem ? x : rem) + (L >> 3);
  r0 = (T / gx) * TT;
  c0 = (T % gx) * TT;
}

__global__ __launch_bounds__(256) void k_transpose_2d(const uint8_t* __restrict__ in_codes, int64_t ld_in,
                                                      const uint8_t* __restrict__ in_scales, int64_t ld_sin,
                                                      int64_t R, int64_t C, uint8_t* __restrict__ out_codes,
                                                      int64_t ld_out, uint8_t* __restrict__ out_scales,
                                                      int64_t ld_sout, int64_t gx, int64_t ntiles) {
  __shared__ uint32_t tin[TT * IP];
  __shared__ uint32_t tout[TT * OP];
  int64_t r0, c0;
  tile_origin(gx, ntiles, r0, c0);
  const int t = threadIdx.x;
  // 128 input rows x 4 chunks of 16 bytes (32 elements each); chunks past the
  // matrix read as zeros (R and C are multiples of 32)
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int id = t + 256 * it;
    const int row = id >> 2, ch = id & 3;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (r0 + row < R && c0 + 32 * ch < C)
      v = *reinterpret_cast<const uint4*>(in_codes + (r0 + row) * ld_in + (c0 >> 1) + 16 * ch);
    uint32_t* d = tin + row * IP + 4 * ch;
    *reinterpret_cast<uint2*>(d) = make_uint2(v.x, v.y);
    *reinterpret_cast<uint2*>(d + 2) = make_uint2(v.z, v.w);
  }
  __syncthreads();
  // 8 x 8 nibble block (br: input rows 8br.., bc: input columns 8bc..): word i
  // holds input row 8br+i, nibble j its column 8bc+j; afterwards word j holds
  // input column 8bc+j with nibble i from input row 8br+i.
  const int br = t >> 4, bc = t & 15;
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = tin[(8 * br + i) * IP + bc];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t x = ((w[i] >> 16) ^ w[i + 4]) & 0x0000FFFFu;
    w[i] ^= x << 16;
    w[i + 4] ^= x;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = (q & 1) + 4 * (q >> 1);   // 0, 1, 4, 5
    const uint32_t x = ((w[i] >> 8) ^ w[i + 2]) & 0x00FF00FFu;
    w[i] ^= x << 8;
    w[i + 2] ^= x;
  }
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    const uint32_t x = ((w[i] >> 4) ^ w[i + 1]) & 0x0F0F0F0Fu;
    w[i] ^= x << 4;
    w[i + 1] ^= x;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) tout[(8 * bc + j) * OP + br] = w[j];
  __syncthreads();
  // 128 output rows (input columns) x 4 chunks of 16 bytes (32 input rows each)
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int id = t + 256 * it;
    const int row = id >> 2, ch = id & 3;
    if (c0 + row < C && r0 + 32 * ch < R) {
      const uint32_t* s = tout + row * OP + 4 * ch;
      *reinterpret_cast<uint4*>(out_codes + (c0 + row) * ld_out + (r0 >> 1) + 16 * ch) =
          make_uint4(s[0], s[1], s[2], s[3]);
    }
  }
  // scale bytes: input tile (r0/32 + b, c0/32 + a) -> output (c0/32 + a, r0/32 + b)
  if (t < 16) {
    const int a = t >> 2, b = t & 3;
    const int64_t ib = (r0 >> 5) + b, jb = (c0 >> 5) + a;
    if (ib * 32 < R && jb * 32 < C) out_scales[jb * ld_sout + ib] = in_scales[ib * ld_sin + jb];
  }
}

// The other element types (FP8: one byte per code; FP6: 4 codes per 3 bytes,
// element k at bits 6k of the row): the 128 x 128 tile is unpacked to one byte
// per code in LDS, transposed by reading it column-wise, and packed again.
// Thread t unpacks / packs groups of 4 codes (3 bytes for FP6, 4 for FP8).
template <int BITS>
__global__ __launch_bounds__(256) void k_transpose_2d_bytes(const uint8_t* __restrict__ in_codes, int64_t ld_in,
                                                            const uint8_t* __restrict__ in_scales, int64_t ld_sin,
                                                            int64_t R, int64_t C, uint8_t* __restrict__ out_codes,
                                                            int64_t ld_out, uint8_t* __restrict__ out_scales,
                                                            int64_t ld_sout, int64_t gx, int64_t ntiles) {
  constexpr int GB = BITS / 2;                     // bytes per group of 4 codes
  constexpr int PITCH = TT + 4;                    // LDS bytes per row
  __shared__ uint8_t tile[TT * PITCH];
  int64_t r0, c0;
  tile_origin(gx, ntiles, r0, c0);
  const int t = threadIdx.x;
  // unpack: 128 rows x 32 groups
  for (int id = t; id < TT * (TT / 4); id += 256) {
    const int row = id >> 5, g = id & 31;
    uint32_t w = 0;
    if (r0 + row < R && c0 + 4 * g < C) {
      const uint8_t* p = in_codes + (r0 + row) * ld_in + (c0 / 4 + g) * GB;
#pragma unroll
      for (int b = 0; b < GB; ++b) w |= (uint32_t)p[b] << (8 * b);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      tile[row * PITCH + 4 * g + j] = (uint8_t)((w >> (BITS * j)) & ((1u << BITS) - 1u));
  }
  __syncthreads();
  // pack: output row o (input column c0 + o), 32 groups of 4 input rows
  for (int id = t; id < TT * (TT / 4); id += 256) {
    const int o = id >> 5, g = id & 31;
    if (c0 + o >= C || r0 + 4 * g >= R) continue;
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) w |= (uint32_t)tile[(4 * g + j) * PITCH + o] << (BITS * j);
    uint8_t* p = out_codes + (c0 + o) * ld_out + (r0 / 4 + g) * GB;
#pragma unroll
    for (int b = 0; b < GB; ++b) p[b] = (uint8_t)(w >> (8 * b));
  }
  if (t < 16) {
    const int a = t >> 2, b = t & 3;
    const int64_t ib = (r0 >> 5) + b, jb = (c0 >> 5) + a;
    if (ib * 32 < R && jb * 32 < C) out_scales[jb * ld_sout + ib] = in_scales[ib * ld_sin + jb];
  }
}

}  // namespace

hipError_t launch_transpose(const TransposeArgs& a, hipStream_t st) {
  if (a.R == 0 || a.C == 0) return hipSuccess;
  const int64_t gx = (a.C + TT - 1) / TT, n = gx * ((a.R + TT - 1) / TT);
  if (n > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)n);
  if (a.bits == 8) {
    hipLaunchKernelGGL(k_transpose_2d_bytes<8>, grid, dim3(256), 0, st, a.in_codes, a.ld_in, a.in_scales, a.ld_sin,
                       a.R, a.C, a.out_codes, a.ld_out, a.out_scales, a.ld_sout, gx, n);
  } else if (a.bits == 6) {
    hipLaunchKernelGGL(k_transpose_2d_bytes<6>, grid, dim3(256), 0, st, a.in_codes, a.ld_in, a.in_scales, a.ld_sin,
                       a.R, a.C, a.out_codes, a.ld_out, a.out_scales, a.ld_sout, gx, n);
  } else {
    hipLaunchKernelGGL(k_transpose_2d, grid, dim3(256), 0, st, a.in_codes, a.ld_in, a.in_scales, a.ld_sin, a.R,
                       a.C, a.out_codes, a.ld_out, a.out_scales, a.ld_sout, gx, n);
  }
  return hipGetLastError();
}

}  // namespace mx
