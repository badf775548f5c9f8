// Block-scaled MXFP4 GEMM and grouped (MoE) GEMM for gfx950.
//
// C[m, n] = sum_kb 2^(sa[m,kb]-127) 2^(sb[n,kb]-127) sum_{j<32} P_a P_b
// ("MXFP4", AI Wiki, §Conversion rules: block dot products X(A) X(B) sum P P,
// summed over blocks; §Hardware support: 32-element groups along the
// contraction dimension, scales applied inside the matrix instruction, float32
// accumulation).  The inner products run on V_MFMA_SCALE_F32_32X32X64_F8F6F4
// with both operands in FP4 (E2M1) and one E8M0 scale per lane:
//   lane l holds row (l % 32) of A (column of B) and the 32 K-elements
//   [32*(l/32), 32*(l/32)+32) of the 64-deep step, i.e. exactly one MX block,
//   16 bytes; its scale byte is picked from a 32-bit register by op_sel;
//   the 32x32 float32 result: lane l, register r holds
//   row 8*(r/4) + 4*(l/32) + (r%4), column l % 32.
//
// Tiling: a 256-thread workgroup computes a 128x128 tile with 4 waves (2x2),
// each wave 64x64 = 2x2 MFMA tiles.  Per 128-deep K stage the workgroup stages
// 128 rows x 64 bytes of A and of B codes in LDS (row pitch 80 bytes) plus one
// 32-bit word of 4 scale bytes per row.  Rows past M/N and K past the end are
// zero codes with scale 1.0, so they add exact zeros (a NaN scale there would
// otherwise poison the sums).
// The 256x256 pipeline in its two MFMA operand orders (see gemm_tile256.h).
#define MX_T256_NS t256
#define MX_T256_SWAP 0
#include "gemm_tile256.h"
#undef MX_T256_NS
#undef MX_T256_SWAP
#define MX_T256_NS t256s
#define MX_T256_SWAP 1
#include "gemm_tile256.h"
#undef MX_T256_NS
#undef MX_T256_SWAP
#include "mx_device.h"
#include "mx_launch.h"

namespace mx {
namespace {

// ---------------------------------------------------------------- 256x256 tiles
// Persistent kernels: one workgroup per CU (G workgroups).  Workgroup b runs
// on XCD b % 8, so XCD x holds the step_x workgroups b = x, x+8, ...  The
// tiles, in the grouped order below, are cut into 8 contiguous ranges sized
// in proportion to step_x, one per XCD, and the XCD's workgroups take its
// range round-robin: the tiles one XCD works on at a time are consecutive,
// and each operand panel is fetched into one XCD's L2 rather than into all.
struct XcdShare {
  int first, n, step, k;                   // tiles first + k + j*step < first + n
  __device__ XcdShare(int b, int G, int T) {
    const int x = b % 8;
    step = G / 8 + (x < G % 8 ? 1 : 0);
    k = b / 8;
    // workgroups on the XCDs before x and up to x
    const int64_t w0 = (int64_t)x * (G / 8) + (x < G % 8 ? x : G % 8);
    const int64_t w1 = w0 + step;
    first = (int)(w0 * T / G);
    n = (int)(w1 * T / G) - first;
  }
  __device__ int count() const { return k < n ? (n - k + step - 1) / step : 0; }
  __device__ int tile(int j) const { return first + k + j * step; }
};

// Tile order (t256c::group_order): groups of GM M-tiles, each walked N-tile
// by N-tile (GM = 8 for the dense GEMM; 2 for the grouped one, whose row tiles
// belong to different experts' weights, measured ~3 % faster there).
using t256c::group_order;

constexpr int GW = t256::WAVES;

struct DenseSched {
  static constexpr bool UNITS = false;
  const uint8_t *a_codes, *a_scales, *b_codes, *b_scales;
  int M, N, tiles_m, tiles_n;
  XcdShare share;
  __device__ int count() const { return share.count(); }
  __device__ t256::TileInfo tile(int j) const {
    int tm, tn;
    group_order<8>(share.tile(j), tiles_m, tiles_n, tm, tn);
    t256::TileInfo ti;
    ti.a_codes = a_codes;
    ti.a_scales = a_scales;
    ti.b_codes = b_codes;
    ti.b_scales = b_scales;
    ti.m0 = tm * t256::TM;
    ti.n0 = tn * t256::TN;
    ti.M = M;
    ti.N = N;
    ti.c_row0 = ti.m0;
    return ti;
  }
};

template <bool A2D, bool B2D, bool OUT_BF16>
__global__ __launch_bounds__(64 * GW, 1) void k_gemm256(MxOperand A, MxOperand B, int M, int N, int K, void* C,
                                                        int64_t ldc, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[t256::LDS_BYTES];
  const DenseSched sc{A.codes, A.scales, B.codes, B.scales, M, N, tiles_m, tiles_n,
                      XcdShare((int)blockIdx.x, (int)gridDim.x, tiles_m * tiles_n)};
  const t256::Strides sd{(int)A.ld_codes, (int)A.ld_scales, (int)B.ld_codes, (int)B.ld_scales};
  t256::run_tiles<A2D, B2D, OUT_BF16 ? t256::OUT_BF16_ : t256::OUT_F32, true>(sc, sd, K, C, ldc, lds);
}

// The dense kernel with the quantizing epilogue (the pipeline with swapped
// MFMA operands): C = A B^T is never stored; each tile leaves as MXFP4 codes
// and scale bytes along N.
template <bool A2D, bool B2D>
__global__ __launch_bounds__(64 * GW, 1) void k_gemm256_q(MxOperand A, MxOperand B, int M, int N, int K,
                                                          t256::QOut qo, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[t256s::LDS_BYTES];
  const DenseSched sc{A.codes, A.scales, B.codes, B.scales, M, N, tiles_m, tiles_n,
                      XcdShare((int)blockIdx.x, (int)gridDim.x, tiles_m * tiles_n)};
  const t256::Strides sd{(int)A.ld_codes, (int)A.ld_scales, (int)B.ld_codes, (int)B.ld_scales};
  t256s::run_tiles<A2D, B2D, t256s::OUT_MX, true>(sc, sd, K, nullptr, 0, lds, qo);
}

// Grouped (MoE) GEMM.  A row tile ("slot") never straddles two experts: the
// slots of expert e are the ceil(rows_e / 256) tiles of its rows, numbered in
// expert order.  Each workgroup first builds, in LDS, the clamped row range of
// every expert and the exclusive prefix count of slots, from the device
// offsets (so the schedule needs no host synchronization); a tile's expert is
// then found by one wave-wide comparison against that prefix.
constexpr int GG_EMAX = 960;                // experts the LDS table holds (it fits beside the ring)

__device__ __forceinline__ int lds_i32(const int* p) {
  int v;
  const uint32_t a = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
  // an asm read that waits only for itself (not for loads in flight to LDS)
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v) : "v"(a) : "memory");
  return v;
}

// Per-launch parameters of the grouped GEMM, kept in LDS and read back per
// tile (holding them in scalar registers across the pipeline would spill).
struct alignas(16) GroupedParams {
  const uint8_t *a_codes, *a_scales, *b_codes, *b_scales;
  int64_t stride_codes, stride_scales;      // between experts of B
  int lda, ldsa, N, tiles_n, E, total_slots, pad0, pad1;
};
static_assert(sizeof(GroupedParams) == 80, "five 16-byte LDS reads");

// Read a wave-uniform GroupedParams from LDS with one wait.
__device__ __forceinline__ GroupedParams load_params(const GroupedParams* p) {
  typedef int v4i_ __attribute__((ext_vector_type(4)));
  v4i_ q[5];
  const uint32_t a = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
  asm volatile(
      "ds_read_b128 %0, %5\n\t"
      "ds_read_b128 %1, %5 offset:16\n\t"
      "ds_read_b128 %2, %5 offset:32\n\t"
      "ds_read_b128 %3, %5 offset:48\n\t"
      "ds_read_b128 %4, %5 offset:64\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(q[0]), "=&v"(q[1]), "=&v"(q[2]), "=&v"(q[3]), "=&v"(q[4])
      : "v"(a)
      : "memory");
  int w[20];
#pragma unroll
  for (int i = 0; i < 5; ++i)
#pragma unroll
    for (int k = 0; k < 4; ++k) w[4 * i + k] = __builtin_amdgcn_readfirstlane(q[i][k]);
  return __builtin_bit_cast(GroupedParams, w);
}

// Two LDS words at per-lane addresses, one wait.
__device__ __forceinline__ void lds_i32x2(const int* p0, const int* p1, int& v0, int& v1) {
  const uint32_t a0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p0;
  const uint32_t a1 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p1;
  asm volatile("ds_read_b32 %0, %2\n\tds_read_b32 %1, %3\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(v0), "=&v"(v1)
               : "v"(a0), "v"(a1)
               : "memory");
}

struct GroupedSched {
  static constexpr bool UNITS = false;
  const GroupedParams* prm;                 // LDS
  const int* tab;                           // LDS: pre [E+1] exclusive prefix of slots, lo [E], hi [E]
  XcdShare share;
  __device__ int count() const { return share.count(); }
  __device__ t256::TileInfo tile(int j) const {
    const GroupedParams P = load_params(prm);
    int slot, tn;
    group_order<2>(share.tile(j), P.total_slots, P.tiles_n, slot, tn);
    const int* pre = tab;
    const int* lo = tab + GG_EMAX + 1;
    const int* hi = lo + GG_EMAX;
    const int lane = threadIdx.x & 63;
    int ex = P.E - 1;
    for (int base = 0; base < P.E; base += 64) {
      const int e = base + lane < P.E ? base + lane : P.E - 1;
      int p0, p1;
      lds_i32x2(pre + e, pre + e + 1, p0, p1);
      const unsigned long long m = __ballot(base + lane < P.E && slot >= p0 && slot < p1);
      if (m) {
        ex = base + __ffsll((long long)m) - 1;
        break;
      }
    }
    ex = __builtin_amdgcn_readfirstlane(ex);
    int l0, p0, h0;
    lds_i32x2(lo + ex, pre + ex, l0, p0);
    h0 = lds_i32(hi + ex);
    const int row0 = __builtin_amdgcn_readfirstlane(l0 + (slot - p0) * t256::TM);
    const int end = __builtin_amdgcn_readfirstlane(h0);
    const int rows = end - row0 < t256::TM ? end - row0 : t256::TM;
    t256::TileInfo ti;
    ti.a_codes = P.a_codes + (int64_t)row0 * P.lda;
    ti.a_scales = P.a_scales + (int64_t)row0 * P.ldsa;
    ti.b_codes = P.b_codes + (int64_t)ex * P.stride_codes;
    ti.b_scales = P.b_scales + (int64_t)ex * P.stride_scales;
    ti.m0 = 0;
    ti.n0 = tn * t256::TN;
    ti.M = rows;
    ti.N = P.N;
    ti.c_row0 = row0;
    return ti;
  }
};

// Fill the LDS expert table: pre [E+1] exclusive prefix of row tiles,
// lo [E] and hi [E] the clamped row range of each expert (wave 0 computes it;
// ends with a workgroup barrier).
__device__ __forceinline__ void build_expert_table(const int32_t* __restrict__ offsets, int E, int64_t M_cap,
                                                   int* tab) {
  int* pre = tab;
  int* lo = tab + GG_EMAX + 1;
  int* hi = lo + GG_EMAX;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int carry = 0;
    for (int base = 0; base < E; base += 64) {
      const int e = base + lane;
      int64_t l0 = 0, h0 = 0;
      if (e < E) {
        l0 = offsets[e];
        h0 = offsets[e + 1];
        l0 = l0 < 0 ? 0 : (l0 > M_cap ? M_cap : l0);
        h0 = h0 < l0 ? l0 : (h0 > M_cap ? M_cap : h0);
      }
      const int tiles = (int)((h0 - l0 + t256::TM - 1) / t256::TM);
      int incl = tiles;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int v = __shfl_up(incl, d, 64);
        if (lane >= d) incl += v;
      }
      if (e < E) {
        pre[e] = carry + incl - tiles;
        lo[e] = (int)l0;
        hi[e] = (int)h0;
      }
      carry += __shfl(incl, 63, 64);
    }
    if (lane == 0) pre[E] = carry;
  }
  __syncthreads();
}

template <bool B2D, bool OUT_BF16>
__global__ __launch_bounds__(64 * GW, 1) void k_grouped_gemm256(MxOperand A, MxOperand B, int64_t M_cap, int N,
                                                                int K, const int32_t* __restrict__ offsets, int E,
                                                                int64_t stride_codes, int64_t stride_scales,
                                                                void* C, int64_t ldc, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[t256::LDS_BYTES];
  __shared__ int tab[3 * GG_EMAX + 1];
  __shared__ GroupedParams prm;
  build_expert_table(offsets, E, M_cap, tab);   // ends with a barrier
  const int total_slots = tab[E];
  if (threadIdx.x == 0)
    prm = GroupedParams{A.codes, A.scales, B.codes, B.scales, stride_codes, stride_scales, (int)A.ld_codes,
                        (int)A.ld_scales, N, tiles_n, E, total_slots, 0, 0};
  __syncthreads();
  const GroupedSched sc{&prm, tab, XcdShare((int)blockIdx.x, (int)gridDim.x, total_slots * tiles_n)};
  const t256::Strides sd{(int)A.ld_codes, (int)A.ld_scales, (int)B.ld_codes, (int)B.ld_scales};
  t256::run_tiles<false, B2D, OUT_BF16 ? t256::OUT_BF16_ : t256::OUT_F32, true>(sc, sd, K, C, ldc, lds);
}

// The grouped kernel with the quantizing epilogue (swapped MFMA operands): the
// rows of each expert's product leave as MXFP4 codes and scale bytes along N.
template <bool B2D>
__global__ __launch_bounds__(64 * GW, 1) void k_grouped_gemm256_q(MxOperand A, MxOperand B, int64_t M_cap, int N,
                                                                int K, const int32_t* __restrict__ offsets, int E,
                                                                int64_t stride_codes, int64_t stride_scales,
                                                                t256::QOut qo, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[t256s::LDS_BYTES];
  __shared__ int tab[3 * GG_EMAX + 1];
  __shared__ GroupedParams prm;
  build_expert_table(offsets, E, M_cap, tab);   // ends with a barrier
  const int total_slots = tab[E];
  if (threadIdx.x == 0)
    prm = GroupedParams{A.codes, A.scales, B.codes, B.scales, stride_codes, stride_scales, (int)A.ld_codes,
                        (int)A.ld_scales, N, tiles_n, E, total_slots, 0, 0};
  __syncthreads();
  const GroupedSched sc{&prm, tab, XcdShare((int)blockIdx.x, (int)gridDim.x, total_slots * tiles_n)};
  const t256::Strides sd{(int)A.ld_codes, (int)A.ld_scales, (int)B.ld_codes, (int)B.ld_scales};
  t256s::run_tiles<false, B2D, t256s::OUT_MX, true>(sc, sd, K, nullptr, 0, lds, qo);
}

// ---------------------------------------------------------------- 128x128 tiles

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128;
constexpr int BK = 128;                 // K elements per LDS stage
constexpr int ROWB = BK / 2;            // code bytes per row per stage
constexpr int PITCH = ROWB + 16;        // LDS row pitch in bytes

struct Smem {
  uint8_t a[BM * PITCH];
  uint8_t b[BN * PITCH];
  uint32_t sa[BM];
  uint32_t sb[BN];
};

// Stage rows [r0, r0 + 128) x K-stage k0 of one operand into LDS.
template <bool TWO_D>
__device__ __forceinline__ void stage_operand(const MxOperand& op, int64_t r0, int64_t rows,
                                              int64_t k0, int64_t K, uint8_t* lds_codes,
                                              uint32_t* lds_scales, int tid, int stid) {
  // 128 rows x 4 chunks of 16 bytes: 2 chunks per thread.
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int id = tid + 256 * it;
    const int r = id >> 2, ch = id & 3;
    const int64_t gr = r0 + r;
    const int64_t kk = k0 + 32 * ch;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (gr < rows && kk < K)
      v = *reinterpret_cast<const uint4*>(op.codes + gr * op.ld_codes + (kk >> 1));
    *reinterpret_cast<uint4*>(lds_codes + r * PITCH + ch * 16) = v;
  }
  // Threads with stid in [0, 128) fetch the 4 scale bytes of one row each.
  if (stid >= 0 && stid < 128) {
    const int64_t gr = r0 + stid;
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t kb = (k0 >> 5) + j;
      uint32_t s = 127u;
      if (gr < rows && kb * 32 < K) s = op.scales[(TWO_D ? (gr >> 5) : gr) * op.ld_scales + kb];
      w |= s << (8 * j);
    }
    lds_scales[stid] = w;
  }
}

template <bool A2D, bool B2D, bool OUT_BF16>
__device__ __forceinline__ void gemm_tile(const MxOperand& A, const MxOperand& B, int64_t M,
                                          int64_t N, int64_t K, int64_t m0, int64_t n0, void* C,
                                          int64_t ldc, Smem& sm) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int l32 = lane & 31, hi = lane >> 5;

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  for (int64_t k0 = 0; k0 < K; k0 += BK) {
    stage_operand<A2D>(A, m0, M, k0, K, sm.a, sm.sa, tid, tid);
    stage_operand<B2D>(B, n0, N, k0, K, sm.b, sm.sb, tid, tid - 128);
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      v8i a[2], b[2];
      int sa[2], sb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = wm * 64 + i * 32 + l32;
        const uint4 v = *reinterpret_cast<const uint4*>(sm.a + r * PITCH + 32 * ks + 16 * hi);
        a[i] = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
        sa[i] = (int)(sm.sa[r] >> (8 * hi));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = wn * 64 + j * 32 + l32;
        const uint4 v = *reinterpret_cast<const uint4*>(sm.b + r * PITCH + 32 * ks + 16 * hi);
        b[j] = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
        sb[j] = (int)(sm.sb[r] >> (8 * hi));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if (ks == 0)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], 4, 4, 0,
                                                                         sa[i], 0, sb[j]);
          else
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], 4, 4, 2,
                                                                         sa[i], 2, sb[j]);
        }
    }
    __syncthreads();
  }

  // Epilogue: lane holds column l32; register r holds row 8*(r/4) + 4*hi + r%4.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = n0 + wn * 64 + j * 32 + l32;
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
        if (row < M) {
          if (OUT_BF16)
            static_cast<uint16_t*>(C)[row * ldc + col] = (uint16_t)f32_to_bf16_rne(acc[i][j][r]);
          else
            static_cast<float*>(C)[row * ldc + col] = acc[i][j][r];
        }
      }
    }
}

template <bool A2D, bool B2D, bool OUT_BF16>
__global__ __launch_bounds__(256) void k_gemm(MxOperand A, MxOperand B, int64_t M, int64_t N,
                                              int64_t K, void* C, int64_t ldc) {
  __shared__ Smem sm;
  const int64_t m0 = (int64_t)blockIdx.y * BM;
  const int64_t n0 = (int64_t)blockIdx.x * BN;
  gemm_tile<A2D, B2D, OUT_BF16>(A, B, M, N, K, m0, n0, C, ldc, sm);
}

// Grouped GEMM: the flat grid enumerates (m-tile slot, n-tile); each
// workgroup maps its slot to (expert, m-tile within the expert) from the
// device offsets, so the schedule needs no host synchronization.  Slots past
// the total number of tiles exit.
template <bool B2D, bool OUT_BF16>
__global__ __launch_bounds__(256) void k_grouped_gemm(MxOperand A, MxOperand B, int64_t M_cap,
                                                      int64_t N, int64_t K,
                                                      const int32_t* __restrict__ offsets, int E,
                                                      int64_t stride_codes, int64_t stride_scales,
                                                      void* C, int64_t ldc) {
  __shared__ Smem sm;
  __shared__ int s_expert, s_row0, s_rows;
  const int64_t slot = blockIdx.y;
  const int64_t n0 = (int64_t)blockIdx.x * BN;
  if (threadIdx.x == 0) {
    int64_t acc_tiles = 0;
    int ex = -1, r0 = 0, nr = 0;
    for (int e = 0; e < E; ++e) {
      int64_t lo = offsets[e], hi = offsets[e + 1];
      lo = lo < 0 ? 0 : (lo > M_cap ? M_cap : lo);
      hi = hi < lo ? lo : (hi > M_cap ? M_cap : hi);
      const int64_t tiles = (hi - lo + BM - 1) / BM;
      if (slot < acc_tiles + tiles) {
        ex = e;
        r0 = (int)(lo + (slot - acc_tiles) * BM);
        nr = (int)(hi - r0 < BM ? hi - r0 : BM);
        break;
      }
      acc_tiles += tiles;
    }
    s_expert = ex;
    s_row0 = r0;
    s_rows = nr;
  }
  __syncthreads();
  const int ex = s_expert;
  if (ex < 0) return;
  MxOperand Ae = A;
  Ae.codes = A.codes + (int64_t)s_row0 * A.ld_codes;
  Ae.scales = A.scales + (int64_t)s_row0 * A.ld_scales;
  MxOperand Be = B;
  Be.codes = B.codes + (int64_t)ex * stride_codes;
  Be.scales = B.scales + (int64_t)ex * stride_scales;
  void* Ce = OUT_BF16 ? (void*)(static_cast<uint16_t*>(C) + (int64_t)s_row0 * ldc)
                      : (void*)(static_cast<float*>(C) + (int64_t)s_row0 * ldc);
  gemm_tile<false, B2D, OUT_BF16>(Ae, Be, s_rows, N, K, 0, n0, Ce, ldc, sm);
}

// ---------------------------------------------------------------- other element types
// The same scaled MFMA with FP8 or FP6 operands (MXFP8, MXFP6; either operand
// may be any MX element type): a 256x256 tile per 8-wave workgroup (64x128 per
// wave), or 128x128 per 4 waves for small problems, staged through LDS per
// 128-deep K stage in 16-byte units.  Operand registers per lane and 64-deep step (the
// instruction's layout, checked by the probe tests): FP4 and FP6 take K-block
// l/32 of the step whole (16 or 24 bytes); FP8 takes the 16-element halves
// [16g, 16g+16) and [32+16g, 48+16g), g = l/32 (2 x 16 bytes).  Scale bytes are
// per K-block as for FP4.

// MFMA operand-format field of mx_elem F.
template <int F>
constexpr int mfma_fmt() {
  if constexpr (F == 0) return 4;
  else return ElemT<F>::MFMA;
}

// One stage (ROWS rows x 128 K-elements) of an operand of element type F held
// in registers between its global fetch and its LDS store, so that the next
// stage's loads are in flight while the current one is multiplied: N 16-byte
// units per thread of a THREADS-thread workgroup (a row stage is RB bytes)
// and, for threads stid in [0, ROWS), the row's word of 4 scale bytes.
template <int F, int ROWS, int THREADS>
struct MxStage {
  static constexpr int RB = 128 * elem_bits<F>() / 8;
  static constexpr int U = RB / 16;
  static constexpr int N = ROWS * U / THREADS;
  static_assert(ROWS * U % THREADS == 0, "whole units per thread");
  uint4 v[N];
  uint32_t sc;
};

// Bytes past K or rows past `rows` read as zeros and their scales as 1.0 (an
// FP6 row may end half-way through a 16-byte unit).  Raw buffer loads over
// the tile's rows, with out-of-range lanes pointed past the end (they return
// zeros), so no load sits behind a branch and all of them are in flight at
// once.
constexpr uint32_t MX_OOB = 0x80000000u;

template <int F, int ROWS, int THREADS>
__device__ __forceinline__ void fetch_mx(MxStage<F, ROWS, THREADS>& f, const MxOperand& op, bool two_d, int64_t r0,
                                         int64_t rows, int64_t k0, int64_t K, int stid) {
  using S = MxStage<F, ROWS, THREADS>;
  const int64_t kbytes = K * elem_bits<F>() / 8;
  const int64_t kb0 = k0 * elem_bits<F>() / 8;
  int64_t nrows = rows - r0;
  nrows = nrows < 0 ? 0 : (nrows > ROWS ? ROWS : nrows);
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(op.codes + r0 * op.ld_codes), 0, (uint32_t)(nrows * op.ld_codes), 0x00020000);
#pragma unroll
  for (int it = 0; it < S::N; ++it) {
    const int id = threadIdx.x + THREADS * it;
    const int r = id / S::U, u = id - r * S::U;
    const int64_t off = kb0 + 16 * u;
    const uint32_t voff = (r < nrows && off < kbytes) ? (uint32_t)(r * op.ld_codes + off) : MX_OOB;
    uint4 v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rc, voff, 0, 0));
    if (off + 16 > kbytes) v.z = v.w = 0u;     // an FP6 row ending 8 bytes into this unit
    f.v[it] = v;
  }
  f.sc = 0x7F7F7F7Fu;
  if (stid >= 0 && stid < ROWS) {             // wave-uniform
    const int64_t gr = r0 + stid;
    const int64_t s0 = two_d ? (r0 >> 5) : r0;
    const int64_t srows = two_d ? ROWS / 32 + 1 : ROWS;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(op.scales + s0 * op.ld_scales), 0, (uint32_t)(srows * op.ld_scales), 0x00020000);
    const int64_t srow = (two_d ? (gr >> 5) : gr) - s0;
    const int64_t kb0s = k0 >> 5;               // a multiple of 4
    // blocks of this stage below K (the rest of the word is row padding or
    // the next row, replaced by scale 1.0)
    const int64_t nk = (K >> 5) - kb0s;
    uint32_t w = 0;
    if ((op.ld_scales & 3) == 0 && ((uintptr_t)op.scales & 3) == 0) {   // uniform: one 4-byte load per row
      const uint32_t v = __builtin_amdgcn_raw_buffer_load_b32(
          rs, gr < rows ? (uint32_t)(srow * op.ld_scales + kb0s) : MX_OOB, 0, 0);
#pragma unroll
      for (int j = 0; j < 4; ++j) w |= (gr < rows && j < nk ? (v >> (8 * j)) & 0xFFu : 127u) << (8 * j);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool valid = gr < rows && j < nk;
        const uint32_t b = __builtin_amdgcn_raw_buffer_load_b8(
            rs, valid ? (uint32_t)(srow * op.ld_scales + kb0s + j) : MX_OOB, 0, 0);
        w |= (valid ? b : 127u) << (8 * j);
      }
    }
    f.sc = w;
  }
}

template <int F, int ROWS, int THREADS>
__device__ __forceinline__ void put_mx(const MxStage<F, ROWS, THREADS>& f, uint8_t* lds, int pitch,
                                       uint32_t* lds_scales, int stid) {
  using S = MxStage<F, ROWS, THREADS>;
#pragma unroll
  for (int it = 0; it < S::N; ++it) {
    const int id = threadIdx.x + THREADS * it;
    const int r = id / S::U, u = id - r * S::U;
    *reinterpret_cast<uint4*>(lds + r * pitch + 16 * u) = f.v[it];
  }
  if (stid >= 0 && stid < ROWS) lds_scales[stid] = f.sc;
}

// This lane's operand registers for 64-deep step ks from its LDS row.
template <int F>
__device__ __forceinline__ v8i read_mx(const uint8_t* row, int ks, int hi) {
  if constexpr (F == 0) {
    const uint4 v = *reinterpret_cast<const uint4*>(row + 32 * ks + 16 * hi);
    return v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
  } else if constexpr (elem_bits<F>() == 8) {
    const uint4 v0 = *reinterpret_cast<const uint4*>(row + 64 * ks + 16 * hi);
    const uint4 v1 = *reinterpret_cast<const uint4*>(row + 64 * ks + 32 + 16 * hi);
    return v8i{(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w, (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
  } else {
    const uint2* p = reinterpret_cast<const uint2*>(row + 48 * ks + 24 * hi);
    const uint2 a = p[0], b = p[1], c = p[2];
    return v8i{(int)a.x, (int)a.y, (int)b.x, (int)b.y, (int)c.x, (int)c.y, 0, 0};
  }
}

// ------------------------------------------ A quantized in the operand load
// The A operand may arrive as bf16 [M, K] and be quantized to MXFP4 on its way
// into LDS (RNE, 1-D blocks along K, optionally the 32-point transform with
// sign mask `mask`), by the same block step the quantizer kernels use, so the
// codes and scale bytes the MFMAs read are those mx_quantize writes.  A
// 256-row, 128-deep stage is 64 KiB of bf16: thread t of the 512 holds half a
// row, row t/2 and blocks 2(t%2), 2(t%2)+1 (128 contiguous bytes, eight
// 16-byte loads).  Rows past M and blocks past K load as zeros (zero codes).
struct QaSrc {
  const uint16_t* a;
  int64_t lda;          // elements
  uint32_t mask;
  int scale_mode;
};

struct QaStage {
  uint4 v[8];
};

__device__ __forceinline__ void fetch_qa(QaStage& f, const QaSrc& q, int64_t m0, int64_t M, int64_t k0, int64_t K) {
  const int r = threadIdx.x >> 1, h = threadIdx.x & 1;
  int64_t nrows = M - m0;
  nrows = nrows < 0 ? 0 : (nrows > 256 ? 256 : nrows);
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(q.a + m0 * q.lda), 0, (uint32_t)(nrows * q.lda * 2), 0x00020000);
  const int64_t kk = k0 + 64 * h;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    // K % 32 == 0: a block is whole or absent; absent blocks and rows past M read zeros
    const bool live = r < nrows && kk + 32 * b < K;
    const uint32_t base = live ? (uint32_t)((r * q.lda + kk + 32 * b) * 2) : 0x80000000u;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      f.v[4 * b + u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rc, base + 16 * u, 0, 0));
  }
}

// Quantize the thread's two blocks and store their codes (16 bytes each, at
// byte 16 j of the row for block j) and scale bytes (byte j of the row's
// scale word) to LDS.
template <bool RHT>
__device__ __forceinline__ void put_qa(const QaStage& f, const QaSrc& q, uint8_t* la, int pitch, uint32_t* lsa) {
  const int r = threadIdx.x >> 1, h = threadIdx.x & 1;
  uint32_t sbytes = 0;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    float x[32];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t w[4] = {f.v[4 * b + u].x, f.v[4 * b + u].y, f.v[4 * b + u].z, f.v[4 * b + u].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = 8 * u + 2 * i;        // element index in the block
        uint32_t v = w[i];
        if (RHT) v ^= (((q.mask >> e) & 1u) << 15) | (((q.mask >> (e + 1)) & 1u) << 31);
        x[e] = bf16lo(v);
        x[e + 1] = bf16hi(v);
      }
    }
    uint32_t packed[4];
    const uint32_t s = quantize_block32<RHT, 0>(x, packed, 0u, 0u, 0u, q.scale_mode);
    *reinterpret_cast<uint4*>(la + r * pitch + 32 * h + 16 * b) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    sbytes |= s << (8 * b);
  }
  reinterpret_cast<uint16_t*>(lsa + r)[h] = (uint16_t)sbytes;
}

// Tile BM x BN per workgroup; each wave owns TI x TJ MFMA tiles of 32x32
// (waves laid out BM/(32 TI) x BN/(32 TJ)).
template <int FA, int FB, int BM_, int BN_, int TI, int TJ>
constexpr int mx_threads() {
  return 64 * (BM_ / (32 * TI)) * (BN_ / (32 * TJ));
}

// The output tile [m0, m0 + BM_) x [n0, n0 + BN_) of C = A B^T (rows past M
// or N are neither read nor written).
// QA (1: plain, 2: with the transform): A comes from bf16 through qa and is
// quantized in the load (FA must be MXFP4, 256-row tiles of 512 threads).
template <int FA, int FB, int BM_, int BN_, int TI, int TJ, int QA = 0>
__device__ __forceinline__ void gemm_mx_tile(const MxOperand& A, const MxOperand& B, int64_t M, int64_t N,
                                             int64_t K, int64_t m0, int64_t n0, void* C, int64_t ldc, int a_2d,
                                             int b_2d, int out_bf16, const QaSrc& qa = QaSrc{}) {
  constexpr int WN = BN_ / (32 * TJ);
  constexpr int THREADS = mx_threads<FA, FB, BM_, BN_, TI, TJ>();
  static_assert(THREADS >= BM_ && THREADS >= BN_, "one A and one B scale row per thread");
  // scale rows: with fewer threads than BM_ + BN_ rows, thread t takes A row t and B row t
  constexpr int BSTID_OFF = THREADS >= BM_ + BN_ ? BM_ : 0;
  static_assert(QA == 0 || (FA == 0 && BM_ == 256 && THREADS == 512), "two threads per A row of the stage");
  constexpr int PA = 128 * elem_bits<FA>() / 8 + 16, PB = 128 * elem_bits<FB>() / 8 + 16;
  constexpr int FMA = mfma_fmt<FA>(), FMB = mfma_fmt<FB>();
  // two LDS buffers, so one barrier per stage: stage s + 1 (fetched into
  // registers during stage s - 1) is written to buffer (s + 1) % 2, the loads
  // of stage s + 2 are issued, and the MFMAs of stage s read buffer s % 2
  __shared__ __attribute__((aligned(16))) uint8_t la[2][BM_ * PA];
  __shared__ __attribute__((aligned(16))) uint8_t lb[2][BN_ * PB];
  __shared__ uint32_t lsa[2][BM_], lsb[2][BN_];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int wm = w / WN, wn = w % WN;
  const int l32 = lane & 31, hi = lane >> 5;
  v16f acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  MxStage<FA, BM_, THREADS> fa;
  QaStage fq;
  MxStage<FB, BN_, THREADS> fb;
  auto fetch = [&](int64_t k0) {
    if constexpr (QA) fetch_qa(fq, qa, m0, M, k0, K);
    else fetch_mx(fa, A, a_2d != 0, m0, M, k0, K, tid);
    fetch_mx(fb, B, b_2d != 0, n0, N, k0, K, tid - BSTID_OFF);
  };
  auto put = [&](int buf) {
    if constexpr (QA) put_qa<QA == 2>(fq, qa, la[buf], PA, lsa[buf]);
    else put_mx(fa, la[buf], PA, lsa[buf], tid);
    put_mx(fb, lb[buf], PB, lsb[buf], tid - BSTID_OFF);
  };
  const int64_t nst = (K + 127) / 128;
  if (nst > 0) {
    fetch(0);
    put(0);
    if (nst > 1) fetch(128);
    __syncthreads();
  }
  for (int64_t st = 0; st < nst; ++st) {
    const int cur = (int)(st & 1);
    // the other buffer was last read in stage st - 1, before the last barrier
    if (st + 1 < nst) put(cur ^ 1);
    if (st + 2 < nst) fetch((st + 2) * 128);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      v8i a[TI], b[TJ];
      int sa[TI], sb[TJ];
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const int r = wm * 32 * TI + i * 32 + l32;
        a[i] = read_mx<FA>(la[cur] + r * PA, ks, hi);
        sa[i] = (int)(lsa[cur][r] >> (8 * hi));
      }
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int r = wn * 32 * TJ + j * 32 + l32;
        b[j] = read_mx<FB>(lb[cur] + r * PB, ks, hi);
        sb[j] = (int)(lsb[cur][r] >> (8 * hi));
      }
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
          if (ks == 0)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], FMA, FMB, 0,
                                                                         sa[i], 0, sb[j]);
          else
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], FMA, FMB, 2,
                                                                         sa[i], 2, sb[j]);
        }
    }
    __syncthreads();
  }
  // lane holds column l32; register r holds row 8*(r/4) + 4*hi + r%4.  Buffer
  // stores through a resource that ends after the tile's last valid row and
  // column: lanes past N point past the end, rows past M fall past it.
  constexpr int ES = 4;
  const int64_t mrows = (M - m0) < BM_ ? (M - m0) : BM_, ncols = (N - n0) < BN_ ? (N - n0) : BN_;
  if (mrows <= 0 || ncols <= 0) return;
  const int es = out_bf16 ? 2 : ES;
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
      static_cast<uint8_t*>(C) + (m0 * ldc + n0) * es, 0, (uint32_t)(((mrows - 1) * ldc + ncols) * es), 0x00020000);
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int col = wn * 32 * TJ + j * 32 + l32;
      const uint32_t voff = col < ncols ? (uint32_t)((4 * hi * ldc + col) * es) : MX_OOB;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t soff = (uint32_t)((wm * 32 * TI + i * 32 + 8 * (r >> 2) + (r & 3)) * ldc * es);
        if (out_bf16)
          __builtin_amdgcn_raw_buffer_store_b16((unsigned short)f32_to_bf16_rne(acc[i][j][r]), rc, voff, soff, 0);
        else
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][r]), rc, voff, soff, 0);
      }
    }
}

template <int FA, int FB, int BM_, int BN_, int TI, int TJ>
__global__ __launch_bounds__((mx_threads<FA, FB, BM_, BN_, TI, TJ>())) void k_gemm_mx(
    MxOperand A, MxOperand B, int64_t M, int64_t N, int64_t K, void* C, int64_t ldc, int a_2d, int b_2d,
    int out_bf16) {
  gemm_mx_tile<FA, FB, BM_, BN_, TI, TJ>(A, B, M, N, K, (int64_t)blockIdx.y * BM_, (int64_t)blockIdx.x * BN_, C,
                                         ldc, a_2d, b_2d, out_bf16);
}

// C = Q(A) B^T with A bf16, quantized in the operand load (QA as above); B
// MXFP4; 256x256 tiles, blockIdx.x the N tile, so the workgroups in flight
// at once share an A panel.
template <int QA>
__global__ __launch_bounds__(512) void k_gemm_qa(QaSrc qa, MxOperand B, int64_t M, int64_t N, int64_t K, void* C,
                                                  int64_t ldc, int b_2d, int out_bf16) {
  gemm_mx_tile<0, 0, 256, 256, 2, 4, QA>(MxOperand{}, B, M, N, K, (int64_t)blockIdx.y * 256,
                                         (int64_t)blockIdx.x * 256, C, ldc, 0, b_2d, out_bf16, qa);
}

// Grouped (MoE) form: blockIdx.y is a row-tile slot, mapped to (expert, rows)
// from the device offsets by one thread, as in the MXFP4 grouped kernel.
template <int FA, int FB, int BM_, int BN_, int TI, int TJ>
__global__ __launch_bounds__((mx_threads<FA, FB, BM_, BN_, TI, TJ>())) void k_grouped_gemm_mx(
    MxOperand A, MxOperand B, int64_t M_cap, int64_t N, int64_t K, const int32_t* __restrict__ offsets, int E,
    int64_t stride_codes, int64_t stride_scales, void* C, int64_t ldc, int b_2d, int out_bf16) {
  __shared__ int s_expert, s_row0, s_rows;
  const int64_t slot = blockIdx.y;
  if (threadIdx.x == 0) {
    int64_t acc_tiles = 0;
    int ex = -1, r0 = 0, nr = 0;
    for (int e = 0; e < E; ++e) {
      int64_t lo = offsets[e], hi = offsets[e + 1];
      lo = lo < 0 ? 0 : (lo > M_cap ? M_cap : lo);
      hi = hi < lo ? lo : (hi > M_cap ? M_cap : hi);
      const int64_t tiles = (hi - lo + BM_ - 1) / BM_;
      if (slot < acc_tiles + tiles) {
        ex = e;
        r0 = (int)(lo + (slot - acc_tiles) * BM_);
        nr = (int)(hi - r0 < BM_ ? hi - r0 : BM_);
        break;
      }
      acc_tiles += tiles;
    }
    s_expert = ex;
    s_row0 = r0;
    s_rows = nr;
  }
  __syncthreads();
  const int ex = s_expert;
  if (ex < 0) return;
  MxOperand Ae = A;
  Ae.codes = A.codes + (int64_t)s_row0 * A.ld_codes;
  Ae.scales = A.scales + (int64_t)s_row0 * A.ld_scales;
  MxOperand Be = B;
  Be.codes = B.codes + (int64_t)ex * stride_codes;
  Be.scales = B.scales + (int64_t)ex * stride_scales;
  void* Ce = out_bf16 ? (void*)(static_cast<uint16_t*>(C) + (int64_t)s_row0 * ldc)
                      : (void*)(static_cast<float*>(C) + (int64_t)s_row0 * ldc);
  gemm_mx_tile<FA, FB, BM_, BN_, TI, TJ>(Ae, Be, s_rows, N, K, 0, (int64_t)blockIdx.x * BN_, Ce, ldc, 0, b_2d,
                                         out_bf16);
}

// ------------------------------------ MXFP8 / MXFP6 operands, loads straight to LDS
// 256x256 tiles of 8 waves (4 along M x 2 along N, 64x128 each as 2 x 4
// MFMA tiles) over 128-deep stages: 4 blocks, 128 code bytes per row for an
// FP8 operand (one cache line) and 96 for FP6, and 4 scale bytes.  Each stage
// goes global -> LDS with direct-to-LDS buffer loads into one of two slots
// while the stage in the other slot is multiplied, so the codes never pass
// through VGPRs: per wave and stage, 8 loads of 1 KiB (4 of A, 4 of B: 8
// rows each, a 16-byte chunk per lane; an FP6 row's chunks 6 and 7 read as
// zeros) and one 4-byte scale load (A rows for waves 0-3, B rows for 4-7).
// LDS rows are 128 bytes with XOR-swizzled 16-byte chunks (chunk c of row r
// sits at c ^ ((r >> 1) & 7)), so the operand reads of consecutive rows fall
// in different banks.  The two slots are separate LDS arrays and the stage
// loop is unrolled by two, and the LDS reads are asm blocks that wait only
// for themselves: the compiler would otherwise wait for the loads in flight
// into the other slot before every read.  FP8 lanes read 2 x 16 bytes per
// 64-deep step (K-elements [16 g, 16 g + 16) and [32 + 16 g, 48 + 16 g) of
// the step, g = lane / 32), FP6 lanes 3 x 8 bytes (their whole 24-byte
// block).
namespace f8 {
constexpr int ROWB = 128;                  // LDS bytes per row and stage
constexpr int OPB = 256 * ROWB;            // one operand's stage (32 KiB)
constexpr int SLOT = 2 * OPB;              // A then B
constexpr int SWORDS = 512;                // scale words of a stage: A rows, then B rows
typedef __attribute__((address_space(3))) void* lds_t;
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
template <int F>
constexpr int gbytes() { return elem_bits<F>() == 8 ? 128 : 96; }   // global code bytes of a stage row
}

struct F8Lane {
  __amdgpu_buffer_rsrc_t ra, rb, rs;
  uint32_t va[4], vb[4];                   // code offsets of this lane's 8 loads (stage 0)
  int c[4];                                // their K chunk (16-byte unit of the stage row)
  uint32_t so;                             // scale offset of this lane's row (stage 0)
};

// Issue the loads of stage s into the slot (codes) and sl (scale words).
// Load t of the wave covers rows 8 (4 wave + t) + lane / 8 and puts this
// lane's 16 bytes at LDS chunk lane % 8 of its row, which holds the row's
// K chunk c = (lane % 8) ^ ((row / 2) % 8).  Chunks past the stage row (FP6:
// 6 and 7) or past K read zeros; an FP6 chunk that K ends half-way through
// brings 8 bytes of the next block, whose scale byte compute() clears.
template <int FA, int FB>
__device__ __forceinline__ void f8_issue(const F8Lane& L, int s, int K, uint8_t* slot, uint32_t* sl, int wave) {
  constexpr int RA = f8::gbytes<FA>(), RB = f8::gbytes<FB>();
  const int ka = RA * s, kbb = RB * s;
  const int kbytes_a = K * elem_bits<FA>() / 8, kbytes_b = K * elem_bits<FB>() / 8;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int c16 = 16 * L.c[t];
    const bool ina = c16 < RA && ka + c16 < kbytes_a, inb = c16 < RB && kbb + c16 < kbytes_b;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(L.ra, (f8::lds_t)(slot + 1024 * (4 * wave + t)), 16,
                                             ina ? L.va[t] : MX_OOB, (uint32_t)ka, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(L.rb, (f8::lds_t)(slot + f8::OPB + 1024 * (4 * wave + t)), 16,
                                             inb ? L.vb[t] : MX_OOB, (uint32_t)kbb, 0, 0);
  }
  __builtin_amdgcn_raw_ptr_buffer_load_lds(L.rs, (f8::lds_t)(sl + 64 * wave), 4, L.so, (uint32_t)(4 * s), 0, 0);
}

// This lane's operands of 64-deep step ks for NT row tiles (4096 LDS bytes
// apart) starting at LDS row address `row` (key = the row's chunk swizzle),
// in one asm block that waits for itself only.
template <int F, int NT>
__device__ __forceinline__ void f8_read(uint32_t row, int key, int ks, int hi, v8i out[NT]) {
  if constexpr (elem_bits<F>() == 8) {
    const uint32_t q0 = row + 16 * ((4 * ks + hi) ^ key), q1 = row + 16 * ((4 * ks + 2 + hi) ^ key);
    f8::v4i x[NT], y[NT];
    if constexpr (NT == 2) {
      asm volatile(
          "ds_read_b128 %0, %4\n\t"
          "ds_read_b128 %2, %5\n\t"
          "ds_read_b128 %1, %4 offset:4096\n\t"
          "ds_read_b128 %3, %5 offset:4096\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(x[0]), "=&v"(x[1]), "=&v"(y[0]), "=&v"(y[1])
          : "v"(q0), "v"(q1)
          : "memory");
    } else {
      asm volatile(
          "ds_read_b128 %0, %8\n\t"
          "ds_read_b128 %4, %9\n\t"
          "ds_read_b128 %1, %8 offset:4096\n\t"
          "ds_read_b128 %5, %9 offset:4096\n\t"
          "ds_read_b128 %2, %8 offset:8192\n\t"
          "ds_read_b128 %6, %9 offset:8192\n\t"
          "ds_read_b128 %3, %8 offset:12288\n\t"
          "ds_read_b128 %7, %9 offset:12288\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(y[0]), "=&v"(y[1]), "=&v"(y[2]), "=&v"(y[3])
          : "v"(q0), "v"(q1)
          : "memory");
    }
#pragma unroll
    for (int i = 0; i < NT; ++i) out[i] = __builtin_shufflevector(x[i], y[i], 0, 1, 2, 3, 4, 5, 6, 7);
  } else {
    // the lane's block: bytes 48 ks + 24 hi + [0, 24) of the stage row, as
    // three 8-byte reads (each inside one 16-byte chunk)
    const int o = 48 * ks + 24 * hi;
    const uint32_t q0 = row + 16 * ((o >> 4) ^ key) + (o & 15);
    const uint32_t q1 = row + 16 * (((o + 8) >> 4) ^ key) + ((o + 8) & 15);
    const uint32_t q2 = row + 16 * (((o + 16) >> 4) ^ key) + ((o + 16) & 15);
    f8::v2i x[NT], y[NT], z[NT];
    if constexpr (NT == 2) {
      asm volatile(
          "ds_read_b64 %0, %6\n\t"
          "ds_read_b64 %2, %7\n\t"
          "ds_read_b64 %4, %8\n\t"
          "ds_read_b64 %1, %6 offset:4096\n\t"
          "ds_read_b64 %3, %7 offset:4096\n\t"
          "ds_read_b64 %5, %8 offset:4096\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(x[0]), "=&v"(x[1]), "=&v"(y[0]), "=&v"(y[1]), "=&v"(z[0]), "=&v"(z[1])
          : "v"(q0), "v"(q1), "v"(q2)
          : "memory");
    } else {
      asm volatile(
          "ds_read_b64 %0, %12\n\t"
          "ds_read_b64 %4, %13\n\t"
          "ds_read_b64 %8, %14\n\t"
          "ds_read_b64 %1, %12 offset:4096\n\t"
          "ds_read_b64 %5, %13 offset:4096\n\t"
          "ds_read_b64 %9, %14 offset:4096\n\t"
          "ds_read_b64 %2, %12 offset:8192\n\t"
          "ds_read_b64 %6, %13 offset:8192\n\t"
          "ds_read_b64 %10, %14 offset:8192\n\t"
          "ds_read_b64 %3, %12 offset:12288\n\t"
          "ds_read_b64 %7, %13 offset:12288\n\t"
          "ds_read_b64 %11, %14 offset:12288\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(y[0]), "=&v"(y[1]), "=&v"(y[2]), "=&v"(y[3]),
            "=&v"(z[0]), "=&v"(z[1]), "=&v"(z[2]), "=&v"(z[3])
          : "v"(q0), "v"(q1), "v"(q2)
          : "memory");
    }
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const f8::v4i xy = __builtin_shufflevector(x[i], y[i], 0, 1, 2, 3);
      const f8::v4i zz = {z[i][0], z[i][1], 0, 0};   // an FP6 operand is 6 dwords; the rest zero
      out[i] = __builtin_shufflevector(xy, zz, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  }
}

// Multiply the stage held in (slot, sl: LDS byte addresses of its codes and
// scale words): 2 steps of 8 MFMAs per wave.  SWAP issues every MFMA with the
// operands (and their formats and scales) exchanged, so that tile (i, j)
// accumulates its transpose: each lane then holds 16 columns of one output
// row, the layout of the quantizing epilogue.
template <int FA, int FB, bool SWAP = false>
__device__ __forceinline__ void f8_compute(v16f acc[2][4], uint32_t slot, uint32_t sl, int s, int K, int wm, int wn,
                                           int l32, int hi) {
  // blocks of this stage below K; the scale bytes of the others (row padding)
  // are cleared to 0, a finite scale: their codes are zero, or for an FP6 row
  // that K ends inside a chunk, 8 bytes whose products with a scale of 2^-127
  // on both sides vanish in float32
  const int nk = (K >> 5) - 4 * s;
  const uint32_t keep = nk >= 4 ? 0xFFFFFFFFu : (1u << (8 * nk)) - 1u;
  // the scale words through an asm read (waiting for itself only)
  const uint32_t wa = sl + 4 * (wm * 64 + l32);
  const uint32_t wb = sl + 4 * (256 + wn * 128 + l32);
  uint32_t q[6];
  asm volatile(
      "ds_read_b32 %0, %6\n\t"
      "ds_read_b32 %1, %6 offset:128\n\t"
      "ds_read_b32 %2, %7\n\t"
      "ds_read_b32 %3, %7 offset:128\n\t"
      "ds_read_b32 %4, %7 offset:256\n\t"
      "ds_read_b32 %5, %7 offset:384\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(q[0]), "=&v"(q[1]), "=&v"(q[2]), "=&v"(q[3]), "=&v"(q[4]), "=&v"(q[5])
      : "v"(wa), "v"(wb)
      : "memory");
  int sa[2], sb[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) sa[i] = (int)((q[i] & keep) >> (8 * hi));
#pragma unroll
  for (int j = 0; j < 4; ++j) sb[j] = (int)((q[2 + j] & keep) >> (8 * hi));
  const int key = (l32 >> 1) & 7;
  const uint32_t ra = slot + (wm * 64 + l32) * f8::ROWB;
  const uint32_t rb = slot + f8::OPB + (wn * 128 + l32) * f8::ROWB;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    v8i a[2], b[4];
    f8_read<FA, 2>(ra, key, ks, hi, a);
    f8_read<FB, 4>(rb, key, ks, hi, b);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (SWAP) {
          if (ks == 0)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b[j], a[i], acc[i][j], mfma_fmt<FB>(),
                                                                         mfma_fmt<FA>(), 0, sb[j], 0, sa[i]);
          else
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b[j], a[i], acc[i][j], mfma_fmt<FB>(),
                                                                         mfma_fmt<FA>(), 2, sb[j], 2, sa[i]);
        } else {
          if (ks == 0)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], mfma_fmt<FA>(),
                                                                         mfma_fmt<FB>(), 0, sa[i], 0, sb[j]);
          else
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], mfma_fmt<FA>(),
                                                                         mfma_fmt<FB>(), 2, sa[i], 2, sb[j]);
        }
      }
  }
}

// Persistent: one workgroup per CU walks its list of tiles (Sched: the dense
// XCD-contiguous ranges in groups of 8 M-tiles, or the grouped GEMM's expert
// row tiles), and the stage sequence runs on across tiles: the next tile's
// first stage loads into the free slot while the current tile's last stage is
// multiplied and its result stored.
// OUT: 0 float32, 1 bf16, 2 the quantizing epilogue (MXFP4 codes and scale
// bytes along N into qo, from the swapped-operand accumulators).
template <int FA, int FB, int OUT, class Sched>
__device__ __forceinline__ void run_f8(const Sched& sc, const MxOperand& A, const MxOperand& B, int K, void* C,
                                       int64_t ldc, int a_2d, int b_2d, uint8_t* slots, uint32_t* sws,
                                       const t256::QOut& qo = t256::QOut{}) {
  constexpr bool OUT_BF16 = OUT == 1;
  constexpr bool SWAP = OUT == 2;
  const int ntiles = sc.count();
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, hi = lane >> 5;
  // this lane's K chunks (one per load) and its scale row
  int crow[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int row = 8 * (4 * wave + t) + (lane >> 3);
    crow[t] = (lane & 7) ^ ((row >> 1) & 7);               // the K chunk this lane's LDS chunk holds
  }
  const bool sA = wave < 4;
  const int srow = 64 * (wave & 3) + lane;                    // this lane's scale row within the tile
  const bool s2d = sA ? a_2d != 0 : b_2d != 0;
  const int64_t lds_s = sA ? A.ld_scales : B.ld_scales;
  // Tile j of this workgroup: the lane's load state, and the tile's output
  // origin (row of C, column) and extent.
  auto setup = [&](int j, F8Lane& L, int64_t& crow0, int& n0, int& mlim, int& nlim) {
    const t256::TileInfo ti = sc.tile(j);
    mlim = ti.M - ti.m0;
    nlim = ti.N - ti.n0;
    const int arows = mlim < 256 ? mlim : 256, brows = nlim < 256 ? nlim : 256;
    L.ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(ti.a_codes) + (int64_t)ti.m0 * A.ld_codes, 0,
                                             (uint32_t)(arows * A.ld_codes), 0x00020000);
    L.rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(ti.b_codes) + (int64_t)ti.n0 * B.ld_codes, 0,
                                             (uint32_t)(brows * B.ld_codes), 0x00020000);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int row = 8 * (4 * wave + t) + (lane >> 3);
      L.c[t] = crow[t];
      L.va[t] = row < arows ? (uint32_t)(row * A.ld_codes + 16 * crow[t]) : MX_OOB;
      L.vb[t] = row < brows ? (uint32_t)(row * B.ld_codes + 16 * crow[t]) : MX_OOB;
    }
    const int r0 = sA ? ti.m0 : ti.n0, rows = sA ? arows : brows;
    const uint8_t* sbase = (sA ? ti.a_scales : ti.b_scales) + (int64_t)(s2d ? (r0 >> 5) : r0) * lds_s;
    L.rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(sbase), 0, (uint32_t)((s2d ? 8 : 256) * lds_s),
                                             0x00020000);
    L.so = srow < rows ? (uint32_t)((s2d ? (srow >> 5) : srow) * lds_s) : MX_OOB;
    crow0 = ti.c_row0;
    n0 = ti.n0;
  };
  const int nst = (K + 127) / 128;
  const uint32_t a_slots = (uint32_t)(uintptr_t)(f8::lds_t)slots, a_sws = (uint32_t)(uintptr_t)(f8::lds_t)sws;
  F8Lane L;
  int64_t c0 = 0, c0n = 0;
  int n0 = 0, mlim = 0, nlim = 0, n0n = 0, mln = 0, nln = 0;
  if (ntiles > 0) setup(0, L, c0, n0, mlim, nlim);
  if (ntiles > 0 && nst > 0) f8_issue<FA, FB>(L, 0, K, slots, sws, wave);
  int g = 0;                                                  // stages multiplied so far (slot g & 1)
  for (int j = 0; j < ntiles; ++j) {
    t256::Acc acc;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc.t[i][jj][r] = 0.0f;
    for (int s = 0; s < nst; ++s, ++g) {
      // stage s of tile j is in slot g & 1; the other slot takes the next stage
      __builtin_amdgcn_s_waitcnt(0x0F70);      // vmcnt(0): this wave's loads of stage s landed
      __syncthreads();                         // ... every wave's; every wave is done with the other slot
      const int nx = (g + 1) & 1;
      if (s + 1 < nst) {
        f8_issue<FA, FB>(L, s + 1, K, slots + nx * f8::SLOT, sws + nx * f8::SWORDS, wave);
      } else if (j + 1 < ntiles) {
        // tile j issues nothing more: its load state becomes tile j + 1's
        setup(j + 1, L, c0n, n0n, mln, nln);
        f8_issue<FA, FB>(L, 0, K, slots + nx * f8::SLOT, sws + nx * f8::SWORDS, wave);
      }
      f8_compute<FA, FB, SWAP>(acc.t, a_slots + (uint32_t)((g & 1) * f8::SLOT),
                               a_sws + (uint32_t)((g & 1) * 4 * f8::SWORDS), s, K, wm, wn, l32, hi);
    }
    // epilogue: the 256x256 kernels' bounds-checked store path (same wave
    // layout and MFMA tiles), or their quantizing epilogue
    if constexpr (SWAP) {
      t256s::Acc q;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) q.t[i][jj] = acc.t[i][jj];
      t256s::store_tile_mx(q, qo, (int)c0, n0, mlim, nlim);
    } else {
      constexpr int ES = OUT_BF16 ? 2 : 4;
      t256::store_tile<OUT_BF16>(acc, static_cast<uint8_t*>(C) + (c0 * ldc + n0) * ES, (int)ldc, mlim, nlim);
    }
    if (j + 1 < ntiles) {
      if (nst == 0) setup(j + 1, L, c0n, n0n, mln, nln);
      c0 = c0n;
      n0 = n0n;
      mlim = mln;
      nlim = nln;
    }
  }
}

template <int FA, int FB, bool OUT_BF16>
__global__ __launch_bounds__(512, 1) void k_gemm_f8(MxOperand A, MxOperand B, int M, int N, int K, void* C,
                                                   int64_t ldc, int a_2d, int b_2d, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) uint8_t slots[2 * f8::SLOT];
  __shared__ __attribute__((aligned(16))) uint32_t sws[2 * f8::SWORDS];
  const DenseSched sc{A.codes, A.scales, B.codes, B.scales, M, N, tiles_m, tiles_n,
                      XcdShare((int)blockIdx.x, (int)gridDim.x, tiles_m * tiles_n)};
  run_f8<FA, FB, OUT_BF16>(sc, A, B, K, C, ldc, a_2d, b_2d, slots, sws);
}

// The dense MXFP8 / MXFP6 product quantized along N in the epilogue (MXFP4
// codes and scale bytes; the operands swapped in every MFMA).
template <int FA, int FB>
__global__ __launch_bounds__(512, 1) void k_gemm_f8_q(MxOperand A, MxOperand B, int M, int N, int K, t256::QOut qo,
                                                     int a_2d, int b_2d, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) uint8_t slots[2 * f8::SLOT];
  __shared__ __attribute__((aligned(16))) uint32_t sws[2 * f8::SWORDS];
  const DenseSched sc{A.codes, A.scales, B.codes, B.scales, M, N, tiles_m, tiles_n,
                      XcdShare((int)blockIdx.x, (int)gridDim.x, tiles_m * tiles_n)};
  run_f8<FA, FB, 2>(sc, A, B, K, nullptr, 0, a_2d, b_2d, slots, sws, qo);
}

// Grouped (MoE) form: the expert table and the schedule of the MXFP4 grouped
// kernel (row tiles never straddle experts), A with 1-D scales.
template <int FA, int FB, bool OUT_BF16>
__global__ __launch_bounds__(512, 1) void k_grouped_gemm_f8(MxOperand A, MxOperand B, int64_t M_cap, int N, int K,
                                                           const int32_t* __restrict__ offsets, int E,
                                                           int64_t stride_codes, int64_t stride_scales, void* C,
                                                           int64_t ldc, int b_2d, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) uint8_t slots[2 * f8::SLOT];
  __shared__ __attribute__((aligned(16))) uint32_t sws[2 * f8::SWORDS];
  __shared__ int tab[3 * GG_EMAX + 1];
  __shared__ GroupedParams prm;
  build_expert_table(offsets, E, M_cap, tab);   // ends with a barrier
  const int total_slots = tab[E];
  if (threadIdx.x == 0)
    prm = GroupedParams{A.codes, A.scales, B.codes, B.scales, stride_codes, stride_scales, (int)A.ld_codes,
                        (int)A.ld_scales, N, tiles_n, E, total_slots, 0, 0};
  __syncthreads();
  const GroupedSched sc{&prm, tab, XcdShare((int)blockIdx.x, (int)gridDim.x, total_slots * tiles_n)};
  run_f8<FA, FB, OUT_BF16>(sc, A, B, K, C, ldc, 0, b_2d, slots, sws);
}

// The grouped MXFP8 / MXFP6 product quantized along N in the epilogue.
template <int FA, int FB>
__global__ __launch_bounds__(512, 1) void k_grouped_gemm_f8_q(MxOperand A, MxOperand B, int64_t M_cap, int N, int K,
                                                             const int32_t* __restrict__ offsets, int E,
                                                             int64_t stride_codes, int64_t stride_scales,
                                                             t256::QOut qo, int b_2d, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) uint8_t slots[2 * f8::SLOT];
  __shared__ __attribute__((aligned(16))) uint32_t sws[2 * f8::SWORDS];
  __shared__ int tab[3 * GG_EMAX + 1];
  __shared__ GroupedParams prm;
  build_expert_table(offsets, E, M_cap, tab);   // ends with a barrier
  const int total_slots = tab[E];
  if (threadIdx.x == 0)
    prm = GroupedParams{A.codes, A.scales, B.codes, B.scales, stride_codes, stride_scales, (int)A.ld_codes,
                        (int)A.ld_scales, N, tiles_n, E, total_slots, 0, 0};
  __syncthreads();
  const GroupedSched sc{&prm, tab, XcdShare((int)blockIdx.x, (int)gridDim.x, total_slots * tiles_n)};
  run_f8<FA, FB, 2>(sc, A, B, K, nullptr, 0, 0, b_2d, slots, sws, qo);
}

template <int FA, int FB>
hipError_t launch_grouped_gemm_mx(const GroupedGemmArgs& a, hipStream_t st, int cus) {
  if constexpr (FA >= 1 && FA <= 4 && FB >= 1 && FB <= 4) {
    // MXFP8 / MXFP6 operands: the persistent direct-to-LDS kernel when the
    // scale rows are whole 32-bit words and the tile offsets fit 32 bits
    const bool words = a.A.ld_scales % 4 == 0 && a.B.ld_scales % 4 == 0 && a.stride_scales % 4 == 0 &&
                       (uintptr_t)a.A.scales % 4 == 0 && (uintptr_t)a.B.scales % 4 == 0;
    const bool small = 256 * a.A.ld_codes < (1ll << 31) && 256 * a.B.ld_codes < (1ll << 31) &&
                       256 * a.ldc * 4 < (1ll << 31) && a.N < (1ll << 31) && a.K < (1ll << 30) &&
                       a.A.ld_codes < (1ll << 31) && a.A.ld_scales < (1ll << 31);
    const int64_t slot_bound = (a.M_cap + 255) / 256 + a.E;
    const int tiles_n = (int)((a.N + 255) / 256);
    if (a.N >= 256 && words && small && a.E <= GG_EMAX && slot_bound * tiles_n < (1ll << 31)) {
      const int64_t tiles = slot_bound * tiles_n;
      const unsigned nwg = (unsigned)(tiles < cus ? tiles : cus);
      if (a.out_bf16)
        hipLaunchKernelGGL((k_grouped_gemm_f8<FA, FB, true>), dim3(nwg), dim3(512), 0, st, a.A, a.B, a.M_cap,
                           (int)a.N, (int)a.K, a.offsets, a.E, a.stride_codes, a.stride_scales, a.C, a.ldc,
                           (int)a.b_2d, tiles_n);
      else
        hipLaunchKernelGGL((k_grouped_gemm_f8<FA, FB, false>), dim3(nwg), dim3(512), 0, st, a.A, a.B, a.M_cap,
                           (int)a.N, (int)a.K, a.offsets, a.E, a.stride_codes, a.stride_scales, a.C, a.ldc,
                           (int)a.b_2d, tiles_n);
      return hipGetLastError();
    }
  }
  if (a.N >= 256) {
    const int64_t slots = (a.M_cap + 255) / 256 + a.E;
    const dim3 grid((unsigned)((a.N + 255) / 256), (unsigned)slots);
    hipLaunchKernelGGL((k_grouped_gemm_mx<FA, FB, 256, 256, 2, 4>), grid, dim3(512), 0, st, a.A, a.B, a.M_cap, a.N,
                       a.K, a.offsets, a.E, a.stride_codes, a.stride_scales, a.C, a.ldc, (int)a.b_2d,
                       (int)a.out_bf16);
  } else {
    const int64_t slots = (a.M_cap + 127) / 128 + a.E;
    const dim3 grid((unsigned)((a.N + 127) / 128), (unsigned)slots);
    hipLaunchKernelGGL((k_grouped_gemm_mx<FA, FB, 128, 128, 2, 2>), grid, dim3(256), 0, st, a.A, a.B, a.M_cap, a.N,
                       a.K, a.offsets, a.E, a.stride_codes, a.stride_scales, a.C, a.ldc, (int)a.b_2d,
                       (int)a.out_bf16);
  }
  return hipGetLastError();
}

template <int FA>
hipError_t launch_grouped_gemm_mx_b(const GroupedGemmArgs& a, hipStream_t st, int cus) {
  switch (a.b_elem) {
    case 1: return launch_grouped_gemm_mx<FA, 1>(a, st, cus);
    case 2: return launch_grouped_gemm_mx<FA, 2>(a, st, cus);
    case 3: return launch_grouped_gemm_mx<FA, 3>(a, st, cus);
    case 4: return launch_grouped_gemm_mx<FA, 4>(a, st, cus);
    default: return launch_grouped_gemm_mx<FA, 0>(a, st, cus);
  }
}


// 256x256 tiles (8 waves of 64x128) when both dimensions fill them, else
// 128x128 (4 waves of 64x64).
template <int FA, int FB>
hipError_t launch_gemm_mx(const GemmArgs& a, hipStream_t st, int cus) {
  if constexpr (FA >= 1 && FA <= 4 && FB >= 1 && FB <= 4) {
    // MXFP8 / MXFP6 operands with whole 256x256 tiles available, 4-byte
    // aligned scale rows and 32-bit tile offsets: the direct-to-LDS kernel
    const bool words = a.A.ld_scales % 4 == 0 && a.B.ld_scales % 4 == 0 && (uintptr_t)a.A.scales % 4 == 0 &&
                       (uintptr_t)a.B.scales % 4 == 0;
    const bool small = 256 * a.A.ld_codes < (1ll << 31) && 256 * a.B.ld_codes < (1ll << 31) &&
                       256 * a.ldc * 4 < (1ll << 31) && a.M < (1ll << 31) && a.N < (1ll << 31) && a.K < (1ll << 30);
    if (a.M >= 256 && a.N >= 256 && words && small) {
      const int tiles_m = (int)((a.M + 255) / 256), tiles_n = (int)((a.N + 255) / 256);
      const int tiles = tiles_m * tiles_n;
      const unsigned nwg = (unsigned)(tiles < cus ? tiles : cus);
      if (a.out_bf16)
        hipLaunchKernelGGL((k_gemm_f8<FA, FB, true>), dim3(nwg), dim3(512), 0, st, a.A, a.B, (int)a.M, (int)a.N,
                           (int)a.K, a.C, a.ldc, (int)a.a_2d, (int)a.b_2d, tiles_m, tiles_n);
      else
        hipLaunchKernelGGL((k_gemm_f8<FA, FB, false>), dim3(nwg), dim3(512), 0, st, a.A, a.B, (int)a.M, (int)a.N,
                           (int)a.K, a.C, a.ldc, (int)a.a_2d, (int)a.b_2d, tiles_m, tiles_n);
      return hipGetLastError();
    }
  }
  if (a.M >= 256 && a.N >= 256) {
    const dim3 grid((unsigned)((a.N + 255) / 256), (unsigned)((a.M + 255) / 256));
    hipLaunchKernelGGL((k_gemm_mx<FA, FB, 256, 256, 2, 4>), grid, dim3(512), 0, st, a.A, a.B, a.M, a.N, a.K, a.C,
                       a.ldc, (int)a.a_2d, (int)a.b_2d, (int)a.out_bf16);
  } else {
    const dim3 grid((unsigned)((a.N + 127) / 128), (unsigned)((a.M + 127) / 128));
    hipLaunchKernelGGL((k_gemm_mx<FA, FB, 128, 128, 2, 2>), grid, dim3(256), 0, st, a.A, a.B, a.M, a.N, a.K, a.C,
                       a.ldc, (int)a.a_2d, (int)a.b_2d, (int)a.out_bf16);
  }
  return hipGetLastError();
}

template <int FA>
hipError_t launch_gemm_mx_b(const GemmArgs& a, hipStream_t st, int cus) {
  switch (a.b_elem) {
    case 1: return launch_gemm_mx<FA, 1>(a, st, cus);
    case 2: return launch_gemm_mx<FA, 2>(a, st, cus);
    case 3: return launch_gemm_mx<FA, 3>(a, st, cus);
    case 4: return launch_gemm_mx<FA, 4>(a, st, cus);
    default: return launch_gemm_mx<FA, 0>(a, st, cus);
  }
}

}  // namespace

// Compute units of the current device (cached per device).
static int cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

// 256x256 tiles: scale rows are fetched 16 bytes at a time (16-byte aligned
// rows), and the operands are addressed with 32-bit offsets.
bool gemm256_layout_ok(const GemmArgs& a) {
  const bool words = (a.A.ld_scales % 16 == 0) && (a.B.ld_scales % 16 == 0) &&
                     ((uintptr_t)a.A.scales % 16 == 0) && ((uintptr_t)a.B.scales % 16 == 0);
  const bool small = a.M * a.A.ld_codes < (1ll << 31) && a.N * a.B.ld_codes < (1ll << 31) &&
                     a.M * a.ldc * (a.out_bf16 ? 2 : 4) < (1ll << 31) && a.K < (1ll << 31);
  return a.M >= 256 && a.N >= 256 && words && small;
}

hipError_t launch_gemm(const GemmArgs& a, hipStream_t st) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  if (a.a_elem != 0 || a.b_elem != 0) {
    const int cus = cu_count();
    switch (a.a_elem) {
      case 1: return launch_gemm_mx_b<1>(a, st, cus);
      case 2: return launch_gemm_mx_b<2>(a, st, cus);
      case 3: return launch_gemm_mx_b<3>(a, st, cus);
      case 4: return launch_gemm_mx_b<4>(a, st, cus);
      default: return launch_gemm_mx_b<0>(a, st, cus);
    }
  }
  if (gemm256_layout_ok(a)) {
    const int tiles_m = (int)((a.M + 255) / 256), tiles_n = (int)((a.N + 255) / 256);
    const int tiles = tiles_m * tiles_n;
    const int cus = cu_count();
    const unsigned nwg = (unsigned)(tiles < cus ? tiles : cus);
#define MX_G256(A_, B_, O_)                                                                        \
  hipLaunchKernelGGL((k_gemm256<A_, B_, O_>), dim3(nwg), dim3(64 * GW), 0, st, a.A, a.B, (int)a.M, \
                     (int)a.N, (int)a.K, a.C, a.ldc, tiles_m, tiles_n)
    if (a.out_bf16) {
      if (a.a_2d) { if (a.b_2d) MX_G256(true, true, true); else MX_G256(true, false, true); }
      else { if (a.b_2d) MX_G256(false, true, true); else MX_G256(false, false, true); }
    } else {
      if (a.a_2d) { if (a.b_2d) MX_G256(true, true, false); else MX_G256(true, false, false); }
      else { if (a.b_2d) MX_G256(false, true, false); else MX_G256(false, false, false); }
    }
#undef MX_G256
    return hipGetLastError();
  }
  dim3 grid((unsigned)((a.N + BN - 1) / BN), (unsigned)((a.M + BM - 1) / BM));
#define MX_G(A_, B_, O_) \
  hipLaunchKernelGGL((k_gemm<A_, B_, O_>), grid, dim3(256), 0, st, a.A, a.B, a.M, a.N, a.K, a.C, a.ldc)
  if (a.out_bf16) {
    if (a.a_2d) { if (a.b_2d) MX_G(true, true, true); else MX_G(true, false, true); }
    else { if (a.b_2d) MX_G(false, true, true); else MX_G(false, false, true); }
  } else {
    if (a.a_2d) { if (a.b_2d) MX_G(true, true, false); else MX_G(true, false, false); }
    else { if (a.b_2d) MX_G(false, true, false); else MX_G(false, false, false); }
  }
#undef MX_G
  return hipGetLastError();
}

hipError_t launch_gemm_qa(const GemmQaArgs& a, hipStream_t st) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  const dim3 grid((unsigned)((a.N + 255) / 256), (unsigned)((a.M + 255) / 256));
  const QaSrc q{static_cast<const uint16_t*>(a.a), a.lda, a.rht ? a.mask : 0u, a.scale_mode};
  if (a.rht)
    hipLaunchKernelGGL((k_gemm_qa<2>), grid, dim3(512), 0, st, q, a.B, a.M, a.N, a.K, a.C, a.ldc, (int)a.b_2d,
                       (int)a.out_bf16);
  else
    hipLaunchKernelGGL((k_gemm_qa<1>), grid, dim3(512), 0, st, q, a.B, a.M, a.N, a.K, a.C, a.ldc, (int)a.b_2d,
                       (int)a.out_bf16);
  return hipGetLastError();
}

template <int FA, int FB>
hipError_t launch_gemm_f8_q(const GemmQuantArgs& a, const t256::QOut& qo, unsigned nwg, int tiles_m, int tiles_n,
                            hipStream_t st) {
  hipLaunchKernelGGL((k_gemm_f8_q<FA, FB>), dim3(nwg), dim3(512), 0, st, a.A, a.B, (int)a.M, (int)a.N, (int)a.K, qo,
                     (int)a.a_2d, (int)a.b_2d, tiles_m, tiles_n);
  return hipGetLastError();
}

template <int FA>
hipError_t launch_gemm_f8_q_b(const GemmQuantArgs& a, const t256::QOut& qo, unsigned nwg, int tiles_m, int tiles_n,
                              hipStream_t st) {
  switch (a.b_elem) {
    case 1: return launch_gemm_f8_q<FA, 1>(a, qo, nwg, tiles_m, tiles_n, st);
    case 2: return launch_gemm_f8_q<FA, 2>(a, qo, nwg, tiles_m, tiles_n, st);
    case 3: return launch_gemm_f8_q<FA, 3>(a, qo, nwg, tiles_m, tiles_n, st);
    case 4: return launch_gemm_f8_q<FA, 4>(a, qo, nwg, tiles_m, tiles_n, st);
    default: return hipErrorNotSupported;
  }
}

hipError_t launch_gemm_f8_q_a(const GemmQuantArgs& a, const t256::QOut& qo, unsigned nwg, int tiles_m, int tiles_n,
                              hipStream_t st) {
  switch (a.a_elem) {
    case 1: return launch_gemm_f8_q_b<1>(a, qo, nwg, tiles_m, tiles_n, st);
    case 2: return launch_gemm_f8_q_b<2>(a, qo, nwg, tiles_m, tiles_n, st);
    case 3: return launch_gemm_f8_q_b<3>(a, qo, nwg, tiles_m, tiles_n, st);
    case 4: return launch_gemm_f8_q_b<4>(a, qo, nwg, tiles_m, tiles_n, st);
    default: return hipErrorNotSupported;
  }
}

bool gemm_quantize_supported(const GemmQuantArgs& a) {
  const bool out_ok = a.M >= 256 && a.N >= 256 && a.N % 32 == 0 && a.ld_codes % 4 == 0 &&
                      (uintptr_t)a.codes % 4 == 0 && 256 * a.ld_codes < (1ll << 31) &&
                      256 * a.ld_scales < (1ll << 31) && a.ld_codes >= a.N / 2 && a.ld_scales >= a.N / 32;
  if (a.a_elem != 0 || a.b_elem != 0) {
    // MXFP8 / MXFP6 operands (both): the direct-to-LDS kernel's conditions
    const bool types = a.a_elem >= 1 && a.a_elem <= 4 && a.b_elem >= 1 && a.b_elem <= 4;
    const bool words = a.A.ld_scales % 4 == 0 && a.B.ld_scales % 4 == 0 && (uintptr_t)a.A.scales % 4 == 0 &&
                       (uintptr_t)a.B.scales % 4 == 0;
    const bool small = 256 * a.A.ld_codes < (1ll << 31) && 256 * a.B.ld_codes < (1ll << 31) &&
                       a.M < (1ll << 31) && a.N < (1ll << 31) && a.K < (1ll << 30);
    return out_ok && types && words && small;
  }
  if (a.K == 0) return out_ok;   // the operands are never read
  return out_ok && a.A.ld_scales % 16 == 0 && a.B.ld_scales % 16 == 0 && (uintptr_t)a.A.scales % 16 == 0 &&
         (uintptr_t)a.B.scales % 16 == 0 && a.M * a.A.ld_codes < (1ll << 31) && a.N * a.B.ld_codes < (1ll << 31) &&
         a.K < (1ll << 31);
}

hipError_t launch_gemm_quantize(const GemmQuantArgs& a, hipStream_t st) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  if (!gemm_quantize_supported(a)) return hipErrorNotSupported;
  const int tiles_m = (int)((a.M + 255) / 256), tiles_n = (int)((a.N + 255) / 256);
  const int tiles = tiles_m * tiles_n;
  const int cus = cu_count();
  const unsigned nwg = (unsigned)(tiles < cus ? tiles : cus);
  const t256::QOut qo{a.codes, a.scales, (int)a.ld_codes, (int)a.ld_scales, a.scale_mode};
  if (a.a_elem != 0 || a.b_elem != 0) return launch_gemm_f8_q_a(a, qo, nwg, tiles_m, tiles_n, st);
#define MX_GQ(A_, B_)                                                                                   \
  hipLaunchKernelGGL((k_gemm256_q<A_, B_>), dim3(nwg), dim3(64 * GW), 0, st, a.A, a.B, (int)a.M, (int)a.N, \
                     (int)a.K, qo, tiles_m, tiles_n)
  if (a.a_2d) { if (a.b_2d) MX_GQ(true, true); else MX_GQ(true, false); }
  else { if (a.b_2d) MX_GQ(false, true); else MX_GQ(false, false); }
#undef MX_GQ
  return hipGetLastError();
}

template <int FA, int FB>
hipError_t launch_grouped_f8_q(const GroupedQuantArgs& q, const t256::QOut& qo, unsigned nwg, int tiles_n,
                               hipStream_t st) {
  const GroupedGemmArgs& a = q.g;
  hipLaunchKernelGGL((k_grouped_gemm_f8_q<FA, FB>), dim3(nwg), dim3(512), 0, st, a.A, a.B, a.M_cap, (int)a.N,
                     (int)a.K, a.offsets, a.E, a.stride_codes, a.stride_scales, qo, (int)a.b_2d, tiles_n);
  return hipGetLastError();
}

template <int FA>
hipError_t launch_grouped_f8_q_b(const GroupedQuantArgs& q, const t256::QOut& qo, unsigned nwg, int tiles_n,
                                 hipStream_t st) {
  switch (q.g.b_elem) {
    case 1: return launch_grouped_f8_q<FA, 1>(q, qo, nwg, tiles_n, st);
    case 2: return launch_grouped_f8_q<FA, 2>(q, qo, nwg, tiles_n, st);
    case 3: return launch_grouped_f8_q<FA, 3>(q, qo, nwg, tiles_n, st);
    case 4: return launch_grouped_f8_q<FA, 4>(q, qo, nwg, tiles_n, st);
    default: return hipErrorNotSupported;
  }
}

bool grouped_quantize_supported(const GroupedQuantArgs& q) {
  const GroupedGemmArgs& a = q.g;
  if (a.a_elem != 0 || a.b_elem != 0) {
    // MXFP8 / MXFP6 operands (both): the grouped direct-to-LDS kernel's conditions
    const bool types = a.a_elem >= 1 && a.a_elem <= 4 && a.b_elem >= 1 && a.b_elem <= 4;
    const bool words = a.A.ld_scales % 4 == 0 && a.B.ld_scales % 4 == 0 && a.stride_scales % 4 == 0 &&
                       (uintptr_t)a.A.scales % 4 == 0 && (uintptr_t)a.B.scales % 4 == 0;
    const bool small = 256 * a.A.ld_codes < (1ll << 31) && 256 * a.B.ld_codes < (1ll << 31) && a.N < (1ll << 31) &&
                       a.K < (1ll << 30) && a.A.ld_codes < (1ll << 31) && a.A.ld_scales < (1ll << 31);
    const int64_t slot_bound = (a.M_cap + 255) / 256 + a.E;
    return types && words && small && !a.a_2d && a.N >= 256 && a.N % 32 == 0 && a.E <= GG_EMAX &&
           slot_bound * ((a.N + 255) / 256) < (1ll << 31) && q.ld_codes % 4 == 0 && (uintptr_t)q.codes % 4 == 0 &&
           256 * q.ld_codes < (1ll << 31) && 256 * q.ld_scales < (1ll << 31) && q.ld_codes >= a.N / 2 &&
           q.ld_scales >= a.N / 32;
  }
  const bool words = (a.A.ld_scales % 16 == 0) && (a.B.ld_scales % 16 == 0) && (a.stride_scales % 16 == 0) &&
                     ((uintptr_t)a.A.scales % 16 == 0) && ((uintptr_t)a.B.scales % 16 == 0);
  const int64_t slot_bound = (a.M_cap + 255) / 256 + a.E;
  return a.a_elem == 0 && a.b_elem == 0 && !a.a_2d && a.N >= 256 && a.N % 32 == 0 && words && a.E <= GG_EMAX &&
         256 * a.A.ld_codes < (1ll << 31) && a.N * a.B.ld_codes < (1ll << 31) && a.K < (1ll << 31) &&
         slot_bound * ((a.N + 255) / 256) < (1ll << 31) && q.ld_codes % 4 == 0 && (uintptr_t)q.codes % 4 == 0 &&
         256 * q.ld_codes < (1ll << 31) && 256 * q.ld_scales < (1ll << 31) && q.ld_codes >= a.N / 2 &&
         q.ld_scales >= a.N / 32;
}

hipError_t launch_grouped_gemm_quantize(const GroupedQuantArgs& q, hipStream_t st) {
  const GroupedGemmArgs& a = q.g;
  if (a.M_cap == 0 || a.N == 0) return hipSuccess;
  if (!grouped_quantize_supported(q)) return hipErrorNotSupported;
  const int64_t slot_bound = (a.M_cap + 255) / 256 + a.E;
  const int tiles_n = (int)((a.N + 255) / 256);
  const int64_t tiles = slot_bound * tiles_n;
  const int cus = cu_count();
  const unsigned nwg = (unsigned)(tiles < cus ? tiles : cus);
  const t256::QOut qo{q.codes, q.scales, (int)q.ld_codes, (int)q.ld_scales, q.scale_mode};
  if (a.a_elem != 0 || a.b_elem != 0) {
    switch (a.a_elem) {
      case 1: return launch_grouped_f8_q_b<1>(q, qo, nwg, tiles_n, st);
      case 2: return launch_grouped_f8_q_b<2>(q, qo, nwg, tiles_n, st);
      case 3: return launch_grouped_f8_q_b<3>(q, qo, nwg, tiles_n, st);
      case 4: return launch_grouped_f8_q_b<4>(q, qo, nwg, tiles_n, st);
      default: return hipErrorNotSupported;
    }
  }
  if (a.b_2d)
    hipLaunchKernelGGL((k_grouped_gemm256_q<true>), dim3(nwg), dim3(64 * GW), 0, st, a.A, a.B, a.M_cap, (int)a.N,
                       (int)a.K, a.offsets, a.E, a.stride_codes, a.stride_scales, qo, tiles_n);
  else
    hipLaunchKernelGGL((k_grouped_gemm256_q<false>), dim3(nwg), dim3(64 * GW), 0, st, a.A, a.B, a.M_cap, (int)a.N,
                       (int)a.K, a.offsets, a.E, a.stride_codes, a.stride_scales, qo, tiles_n);
  return hipGetLastError();
}

hipError_t launch_grouped_gemm(const GroupedGemmArgs& a, hipStream_t st) {
  if (a.M_cap == 0 || a.N == 0) return hipSuccess;
  if (a.a_elem != 0 || a.b_elem != 0) {
    const int cus = cu_count();
    switch (a.a_elem) {
      case 1: return launch_grouped_gemm_mx_b<1>(a, st, cus);
      case 2: return launch_grouped_gemm_mx_b<2>(a, st, cus);
      case 3: return launch_grouped_gemm_mx_b<3>(a, st, cus);
      case 4: return launch_grouped_gemm_mx_b<4>(a, st, cus);
      default: return launch_grouped_gemm_mx_b<0>(a, st, cus);
    }
  }
  const bool words = (a.A.ld_scales % 16 == 0) && (a.B.ld_scales % 16 == 0) && (a.stride_scales % 16 == 0) &&
                     ((uintptr_t)a.A.scales % 16 == 0) && ((uintptr_t)a.B.scales % 16 == 0);
  const bool small = 256 * a.A.ld_codes < (1ll << 31) && a.N * a.B.ld_codes < (1ll << 31) &&
                     256 * a.ldc * (a.out_bf16 ? 2 : 4) < (1ll << 31) && a.K < (1ll << 31);
  // upper bound on row tiles: each expert adds at most one partial tile
  const int64_t slot_bound = (a.M_cap + 255) / 256 + a.E;
  const int tiles_n = (int)((a.N + 255) / 256);
  if (a.N >= 256 && words && small && a.E <= GG_EMAX && slot_bound * tiles_n < (1ll << 31)) {
    const int64_t tiles = slot_bound * tiles_n;
    const int cus = cu_count();
    const unsigned nwg = (unsigned)(tiles < cus ? tiles : cus);
#define MX_GG256(B_, O_)                                                                                  \
  hipLaunchKernelGGL((k_grouped_gemm256<B_, O_>), dim3(nwg), dim3(64 * GW), 0, st, a.A, a.B, a.M_cap,     \
                     (int)a.N, (int)a.K, a.offsets, a.E, a.stride_codes, a.stride_scales, a.C, a.ldc, tiles_n)
    if (a.out_bf16) {
      if (a.b_2d) MX_GG256(true, true); else MX_GG256(false, true);
    } else {
      if (a.b_2d) MX_GG256(true, false); else MX_GG256(false, false);
    }
#undef MX_GG256
    return hipGetLastError();
  }
  // Upper bound on m-tiles over all experts: each expert adds at most one partial tile.
  const int64_t slots = (a.M_cap + BM - 1) / BM + a.E;
  dim3 grid((unsigned)((a.N + BN - 1) / BN), (unsigned)slots);
#define MX_GG(B_, O_)                                                                          \
  hipLaunchKernelGGL((k_grouped_gemm<B_, O_>), grid, dim3(256), 0, st, a.A, a.B, a.M_cap, a.N, a.K, \
                     a.offsets, a.E, a.stride_codes, a.stride_scales, a.C, a.ldc)
  if (a.out_bf16) {
    if (a.b_2d) MX_GG(true, true); else MX_GG(false, true);
  } else {
    if (a.b_2d) MX_GG(true, false); else MX_GG(false, false);
  }
#undef MX_GG
  return hipGetLastError();
}

}  // namespace mx
