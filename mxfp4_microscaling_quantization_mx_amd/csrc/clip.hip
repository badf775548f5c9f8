// Clipping statistic of a quantization ("MXFP4", AI Wiki, §Clipping in the
// reference algorithm): under the reference scale rule a block's maximum can
// scale to just below 2 x the element type's largest power of two, and the
// elements that land above the largest normal (6 for E2M1) saturate.  This
// counts them for a given set of quantizer settings, with the quantizer's
// own steps up to the division by the scale: the sign flips and the 32-point
// transform (float32, the same stage order), the block (1-D) or 32x32 tile
// (2-D) maximum, the scale byte of the chosen rule, the optional 3/4
// prescale, and the multiply by the inverse scale.  An element counts iff its
// scaled magnitude is above the largest normal; the rounding mode does not
// enter (every mode saturates the same elements), and blocks holding NaN or
// Inf count nothing.
//
// One lane per block, with the block-to-lane maps below chosen so that a
// wave's loads are contiguous; per-lane counts are summed per workgroup and
// added to the 64-bit total with one atomic.
#include "mx_device.h"
#include "mx_launch.h"

namespace mx {
namespace {

// Workgroup sizes and grid caps: every workgroup ends in one 64-bit atomic
// add on the same address, and those serialize (8192 of them took ~80 us), so
// the grids are capped near the CU count, with large workgroups for the
// streaming kernels (measured at 16384 x 2880 bf16: 1-D rows 22-25 us, dim 0
// 25-28 us) and 4 workgroups of 256 per CU for the 2-D tile kernel, whose
// barrier per unit favours smaller groups (29-31 us).
constexpr int CLIP_STREAM_THREADS = 1024, CLIP_STREAM_GROUPS = 256;
// the 1-D row kernel: 2 workgroups per CU (16384 x 2880 with the transform
// 23.7 -> 22.5 us against 1 per CU; two blocks per lane and pass with both
// loads first measured 28.5 us)
constexpr int CLIP_ROWS_GROUPS = 512;
constexpr int CLIP_TILE_THREADS = 256, CLIP_TILE_GROUPS = 1024;

template <bool BF16>
__device__ __forceinline__ float clip_load1(const void* __restrict__ src, int64_t i) {
  if (BF16) return bf16lo(static_cast<const uint16_t*>(src)[i]);
  return static_cast<const float*>(src)[i];
}

// 8 consecutive elements from a 16-byte aligned index (rows axis)
template <bool BF16>
__device__ __forceinline__ void clip_load8(const void* __restrict__ src, int64_t i, float x[8]) {
  if (BF16) {
    const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src) + i);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = bf16lo(ww[j]);
      x[2 * j + 1] = bf16hi(ww[j]);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(src) + i);
    const float4 a = p[0], b = p[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

// Scale byte of a block with largest magnitude bits m under the rule
// (0 reference, 1 round up, 2 reference: the prescale does not change it).
template <int ELEM>
__device__ __forceinline__ uint32_t clip_scale_code(uint32_t m, int scale_mode) {
  if constexpr (ELEM == 0) return scale_mode == 1 ? scale_code_round_up(m) : scale_code_from_absmax_bits(m);
  else return elem_scale_code<ELEM>(m, scale_mode == 1);
}

template <int ELEM>
constexpr uint32_t clip_top_bits() {
  if constexpr (ELEM == 0) return 0x40C00000u;   // 6
  else return ElemT<ELEM>::MAXBITS;
}

// The block's values after the optional sign flips, transform and constant
// (in place), and the float32 bits of its largest magnitude.
template <bool RHT>
__device__ __forceinline__ uint32_t clip_prepare(float x[32], uint32_t mask) {
  uint32_t m = 0;
  if (RHT) {
    const float c = __uint_as_float(kRhtCBits);
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = __uint_as_float(__float_as_uint(x[i]) ^ (((mask >> i) & 1u) << 31));
    fwht32_inlane(x);
#pragma unroll
    for (int i = 0; i < 32; ++i) m = max(m, __float_as_uint(x[i]) & 0x7FFFFFFFu);
    m = __float_as_uint(c * __uint_as_float(m));   // max |c t_i| = c max |t_i| (rounding is monotone)
#pragma unroll
    for (int i = 0; i < 32; ++i) x[i] = c * x[i];
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) m = max(m, __float_as_uint(x[i]) & 0x7FFFFFFFu);
  }
  return m;
}

// Elements of a prepared block that saturate, given the largest magnitude m
// of its block (1-D) or tile (2-D).
template <int ELEM>
__device__ __forceinline__ uint32_t clip_block(const float x[32], uint32_t m, int scale_mode) {
  const uint32_t s = clip_scale_code<ELEM>(m, scale_mode);
  if (s == 0xFFu) return 0;
  const float top = __uint_as_float(clip_top_bits<ELEM>());
  const float inv = inv_scale_from_code(s);   // 2^(127 - s), a normal float for s <= 253
  uint32_t n = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float y = scale_mode == 2 ? 0.75f * x[i] : x[i];
    n += fabsf(y * inv) > top ? 1u : 0u;
  }
  return n;
}

// Sum the lanes' counts of a workgroup of T threads and add them to the total.
template <int T>
__device__ __forceinline__ void clip_commit(uint32_t n, uint32_t* wsum, unsigned long long* count) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) n += (uint32_t)__shfl_xor((int)n, d, 64);
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = n;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long tot = 0;
#pragma unroll
    for (int w = 0; w < T / 64; ++w) tot += wsum[w];
    if (tot) atomicAdd(count, tot);
  }
}

// Blocks along the rows, 1-D: lane t takes block t of the row-major block
// order, so a wave reads 64 consecutive blocks (4 KiB of bf16) of a row.
template <int ELEM, bool BF16, bool RHT, class IDX>
__global__ __launch_bounds__(CLIP_STREAM_THREADS) void k_clip_rows(const void* __restrict__ src, int64_t ld,
                                                                   int64_t rows, int64_t nkb_, uint32_t mask,
                                                                   int scale_mode, unsigned long long* count) {
  constexpr int T = CLIP_STREAM_THREADS;
  __shared__ uint32_t wsum[T / 64];
  uint32_t n = 0;
  // block indices in IDX: 32 bits while total + stride < 2^32 (a 64-bit
  // division per block is a long VALU sequence)
  const IDX nkb = (IDX)nkb_;
  const IDX total = (IDX)(rows * nkb_), stride = (IDX)gridDim.x * T;
  for (IDX b = (IDX)blockIdx.x * T + threadIdx.x; b < total; b += stride) {
    const IDX rq = b / nkb;
    const int64_t r = rq, kb = b - rq * nkb;
    float x[32];
#pragma unroll
    for (int j = 0; j < 4; ++j) clip_load8<BF16>(src, r * ld + 32 * kb + 8 * j, x + 8 * j);
    const uint32_t m = clip_prepare<RHT>(x, mask);
    n += clip_block<ELEM>(x, m, scale_mode);
  }
  clip_commit<T>(n, wsum, count);
}

// Blocks along the rows, 2-D (32x32 tiles): a workgroup takes 32 rows x KB
// K-blocks at a time, thread (row rr = t / KB, block kk = t % KB), so a wave
// reads runs of KB consecutive blocks of a row; the tile maxima go through LDS.
template <int ELEM, bool BF16, bool RHT>
__global__ __launch_bounds__(CLIP_TILE_THREADS) void k_clip_rows_2d(const void* __restrict__ src, int64_t ld,
                                                                    int64_t rows, int64_t nkb, uint32_t mask,
                                                                    int scale_mode, unsigned long long* count) {
  constexpr int T = CLIP_TILE_THREADS;
  constexpr int KB = T / 32;                  // K-blocks per unit
  __shared__ uint32_t wsum[T / 64];
  __shared__ uint32_t bm[32][KB + 1];
  const int rr = threadIdx.x / KB, kk = threadIdx.x % KB;
  const int64_t groups_k = (nkb + KB - 1) / KB, units = rows / 32 * groups_k;
  uint32_t n = 0;
  for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
    const int64_t tr = u / groups_k, kg = u - tr * groups_k;
    const int64_t r = 32 * tr + rr, kb = KB * kg + kk;
    const bool valid = kb < nkb;
    float x[32];
    if (valid) {
#pragma unroll
      for (int j = 0; j < 4; ++j) clip_load8<BF16>(src, r * ld + 32 * kb + 8 * j, x + 8 * j);
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) x[i] = 0.0f;
    }
    bm[rr][kk] = clip_prepare<RHT>(x, mask);
    __syncthreads();
    uint32_t m = 0;
#pragma unroll 8
    for (int q = 0; q < 32; ++q) m = max(m, bm[q][kk]);
    if (valid) n += clip_block<ELEM>(x, m, scale_mode);
    __syncthreads();                          // bm is rewritten by the next unit
  }
  clip_commit<T>(n, wsum, count);
}

// Blocks along dim 0: lanes 32 g .. 32 g + 31 take 32 consecutive source
// columns (output rows) of one K-block, each reading its column's 32 elements
// (consecutive lanes, consecutive addresses); a 2-D tile's maximum is a
// 32-lane reduction.
template <int ELEM, bool BF16, bool TWO_D, bool RHT>
__global__ __launch_bounds__(CLIP_STREAM_THREADS) void k_clip_dim0(const void* __restrict__ src, int64_t ld,
                                                                   int64_t rows_out, int64_t nkb, int64_t lanes,
                                                                   uint32_t mask, int scale_mode,
                                                                   unsigned long long* count) {
  constexpr int T = CLIP_STREAM_THREADS;
  __shared__ uint32_t wsum[T / 64];
  uint32_t n = 0;
  const int64_t stride = (int64_t)gridDim.x * T;
  // `lanes` is a multiple of 32 and so is the stride: the 32 lanes of a tile
  // row are in or out of the loop together (the 2-D reduction needs all 32)
  for (int64_t t = (int64_t)blockIdx.x * T + threadIdx.x; t < lanes; t += stride) {
    const int64_t g = t >> 5;
    const int64_t tr = g / nkb, kb = g - tr * nkb;
    const int64_t r = 32 * tr + (t & 31);
    const bool valid = r < rows_out;
    float x[32];
    if (valid) {
#pragma unroll
      for (int i = 0; i < 32; ++i) x[i] = clip_load1<BF16>(src, (32 * kb + i) * ld + r);
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) x[i] = 0.0f;
    }
    uint32_t m = clip_prepare<RHT>(x, mask);
    if (TWO_D) {
#pragma unroll
      for (int d = 1; d < 32; d <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, d, 32));
    }
    if (valid) n += clip_block<ELEM>(x, m, scale_mode);
  }
  clip_commit<T>(n, wsum, count);
}

template <int ELEM, bool BF16, bool RHT>
hipError_t launch_clip3(const ClipArgs& a, hipStream_t st) {
  const int64_t rows_out = a.dim0 ? a.C : a.R, K = a.dim0 ? a.R : a.C;
  const int64_t nkb = K / 32;
  auto grid_for = [](int64_t work, int cap) { return (unsigned)(work < cap ? (work > 0 ? work : 1) : cap); };
  constexpr int TS = CLIP_STREAM_THREADS, TT = CLIP_TILE_THREADS;
  if (!a.dim0 && !a.two_d) {
    const unsigned grid = grid_for((rows_out * nkb + TS - 1) / TS, CLIP_ROWS_GROUPS);
    if (rows_out * nkb < (1ll << 32) - (int64_t)CLIP_ROWS_GROUPS * TS)
      hipLaunchKernelGGL((k_clip_rows<ELEM, BF16, RHT, uint32_t>), dim3(grid), dim3(TS), 0, st, a.src, a.ld_src,
                         rows_out, nkb, a.mask, a.scale_mode, a.count);
    else
      hipLaunchKernelGGL((k_clip_rows<ELEM, BF16, RHT, int64_t>), dim3(grid), dim3(TS), 0, st, a.src, a.ld_src,
                         rows_out, nkb, a.mask, a.scale_mode, a.count);
  } else if (!a.dim0) {
    hipLaunchKernelGGL((k_clip_rows_2d<ELEM, BF16, RHT>),
                       dim3(grid_for(rows_out / 32 * ((nkb + TT / 32 - 1) / (TT / 32)), CLIP_TILE_GROUPS)), dim3(TT),
                       0, st, a.src, a.ld_src, rows_out, nkb, a.mask, a.scale_mode, a.count);
  } else {
    const int64_t lanes = (rows_out + 31) / 32 * nkb * 32;
    const unsigned grid = grid_for((lanes + TS - 1) / TS, CLIP_STREAM_GROUPS);
    if (a.two_d)
      hipLaunchKernelGGL((k_clip_dim0<ELEM, BF16, true, RHT>), dim3(grid), dim3(TS), 0, st, a.src, a.ld_src,
                         rows_out, nkb, lanes, a.mask, a.scale_mode, a.count);
    else
      hipLaunchKernelGGL((k_clip_dim0<ELEM, BF16, false, RHT>), dim3(grid), dim3(TS), 0, st, a.src, a.ld_src,
                         rows_out, nkb, lanes, a.mask, a.scale_mode, a.count);
  }
  return hipGetLastError();
}

template <int ELEM>
hipError_t launch_clip_elem(const ClipArgs& a, hipStream_t st) {
  if (a.bf16) return a.rht ? launch_clip3<ELEM, true, true>(a, st) : launch_clip3<ELEM, true, false>(a, st);
  return a.rht ? launch_clip3<ELEM, false, true>(a, st) : launch_clip3<ELEM, false, false>(a, st);
}

}  // namespace

hipError_t launch_clip_count(const ClipArgs& a, hipStream_t st) {
  switch (a.elem) {
    case 1: return launch_clip_elem<1>(a, st);
    case 2: return launch_clip_elem<2>(a, st);
    case 3: return launch_clip_elem<3>(a, st);
    case 4: return launch_clip_elem<4>(a, st);
    default: return launch_clip_elem<0>(a, st);
  }
}

}  // namespace mx
