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
// One lane per block: lanes 32 g .. 32 g + 31 take the 32 output rows of one
// tile row and one K-block, so a 2-D tile's maximum is a 32-lane reduction.
// Rows-axis blocks are read as four 16-byte loads per lane, dim-0 blocks one
// element per load (consecutive lanes, consecutive columns).  Per-lane counts
// are summed per workgroup and added to the 64-bit total with one atomic.
#include "mx_device.h"
#include "mx_launch.h"

namespace mx {
namespace {

constexpr int CLIP_THREADS = 256;
constexpr int CLIP_MAX_GROUPS = 8192;

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

template <int ELEM, bool BF16, bool DIM0, bool TWO_D, bool RHT>
__global__ __launch_bounds__(CLIP_THREADS) void k_clip_count(const void* __restrict__ src, int64_t ld,
                                                             int64_t rows_out, int64_t nkb, int64_t lanes,
                                                             uint32_t mask, int scale_mode,
                                                             unsigned long long* count) {
  __shared__ uint32_t wsum[CLIP_THREADS / 64];
  const float top = __uint_as_float(clip_top_bits<ELEM>());
  const float c = __uint_as_float(kRhtCBits);
  uint32_t n = 0;
  const int64_t stride = (int64_t)gridDim.x * CLIP_THREADS;
  // `lanes` is a multiple of 32 and so is the stride: the 32 lanes of a tile
  // row are in or out of the loop together (the 2-D reduction needs all 32)
  for (int64_t t = (int64_t)blockIdx.x * CLIP_THREADS + threadIdx.x; t < lanes; t += stride) {
    const int64_t g = t >> 5;
    const int64_t tr = g / nkb, kb = g - tr * nkb;
    const int64_t r = 32 * tr + (t & 31);
    const bool valid = r < rows_out;
    float x[32];
    if (!valid) {
#pragma unroll
      for (int i = 0; i < 32; ++i) x[i] = 0.0f;
    } else if (DIM0) {
#pragma unroll
      for (int i = 0; i < 32; ++i) x[i] = clip_load1<BF16>(src, (32 * kb + i) * ld + r);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) clip_load8<BF16>(src, r * ld + 32 * kb + 8 * j, x + 8 * j);
    }
    uint32_t m = 0;
    if (RHT) {
#pragma unroll
      for (int i = 0; i < 32; ++i) x[i] = __uint_as_float(__float_as_uint(x[i]) ^ (((mask >> i) & 1u) << 31));
      fwht32_inlane(x);
#pragma unroll
      for (int i = 0; i < 32; ++i) m = max(m, __float_as_uint(x[i]) & 0x7FFFFFFFu);
      m = __float_as_uint(c * __uint_as_float(m));
#pragma unroll
      for (int i = 0; i < 32; ++i) x[i] = c * x[i];
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) m = max(m, __float_as_uint(x[i]) & 0x7FFFFFFFu);
    }
    if (TWO_D) {
#pragma unroll
      for (int d = 1; d < 32; d <<= 1) m = max(m, (uint32_t)__shfl_xor((int)m, d, 32));
    }
    const uint32_t s = clip_scale_code<ELEM>(m, scale_mode);
    if (valid && s != 0xFFu) {
      const float inv = inv_scale_from_code(s);   // 2^(127 - s), a normal float for s <= 253
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const float y = scale_mode == 2 ? 0.75f * x[i] : x[i];
        n += fabsf(y * inv) > top ? 1u : 0u;
      }
    }
  }
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) n += (uint32_t)__shfl_xor((int)n, d, 64);
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = n;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long tot = 0;
#pragma unroll
    for (int w = 0; w < CLIP_THREADS / 64; ++w) tot += wsum[w];
    if (tot) atomicAdd(count, tot);
  }
}

template <int ELEM, bool BF16, bool DIM0, bool TWO_D>
hipError_t launch_clip4(const ClipArgs& a, hipStream_t st) {
  const int64_t rows_out = a.dim0 ? a.C : a.R, K = a.dim0 ? a.R : a.C;
  const int64_t nkb = K / 32;
  const int64_t lanes = (rows_out + 31) / 32 * nkb * 32;
  const int64_t groups = (lanes + CLIP_THREADS - 1) / CLIP_THREADS;
  const unsigned grid = (unsigned)(groups < CLIP_MAX_GROUPS ? groups : CLIP_MAX_GROUPS);
  if (a.rht)
    hipLaunchKernelGGL((k_clip_count<ELEM, BF16, DIM0, TWO_D, true>), dim3(grid), dim3(CLIP_THREADS), 0, st, a.src,
                       a.ld_src, rows_out, nkb, lanes, a.mask, a.scale_mode, a.count);
  else
    hipLaunchKernelGGL((k_clip_count<ELEM, BF16, DIM0, TWO_D, false>), dim3(grid), dim3(CLIP_THREADS), 0, st, a.src,
                       a.ld_src, rows_out, nkb, lanes, a.mask, a.scale_mode, a.count);
  return hipGetLastError();
}

template <int ELEM>
hipError_t launch_clip_elem(const ClipArgs& a, hipStream_t st) {
  if (a.bf16) {
    if (a.dim0) return a.two_d ? launch_clip4<ELEM, true, true, true>(a, st) : launch_clip4<ELEM, true, true, false>(a, st);
    return a.two_d ? launch_clip4<ELEM, true, false, true>(a, st) : launch_clip4<ELEM, true, false, false>(a, st);
  }
  if (a.dim0) return a.two_d ? launch_clip4<ELEM, false, true, true>(a, st) : launch_clip4<ELEM, false, true, false>(a, st);
  return a.two_d ? launch_clip4<ELEM, false, false, true>(a, st) : launch_clip4<ELEM, false, false, false>(a, st);
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
