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

// Tile order: groups of GM M-tiles, each walked N-tile by N-tile, so that a
// run of consecutive tiles shares a few A and B panels (GM = 8 for the dense
// GEMM; 2 for the grouped one, whose row tiles belong to different experts'
// weights, measured ~3 % faster there).
template <int GM>
__device__ __forceinline__ void group_order(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int group = t / (GM * tiles_n);
  const int first_m = group * GM;
  const int gm = (tiles_m - first_m) < GM ? (tiles_m - first_m) : GM;
  const int in = t - group * GM * tiles_n;
  tm = first_m + in % gm;
  tn = in / gm;
}

constexpr int GW = t256::WAVES;

struct DenseSched {
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
// FP6 row may end half-way through a 16-byte unit).
template <int F, int ROWS, int THREADS>
__device__ __forceinline__ void fetch_mx(MxStage<F, ROWS, THREADS>& f, const MxOperand& op, bool two_d, int64_t r0,
                                         int64_t rows, int64_t k0, int64_t K, int stid) {
  using S = MxStage<F, ROWS, THREADS>;
  const int64_t kbytes = K * elem_bits<F>() / 8;
  const int64_t kb0 = k0 * elem_bits<F>() / 8;
#pragma unroll
  for (int it = 0; it < S::N; ++it) {
    const int id = threadIdx.x + THREADS * it;
    const int r = id / S::U, u = id - r * S::U;
    const int64_t gr = r0 + r, off = kb0 + 16 * u;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (gr < rows) {
      const uint8_t* p = op.codes + gr * op.ld_codes + off;
      if (off + 16 <= kbytes) {
        v = *reinterpret_cast<const uint4*>(p);
      } else if (off < kbytes) {
        const uint2 h = *reinterpret_cast<const uint2*>(p);
        v = make_uint4(h.x, h.y, 0u, 0u);
      }
    }
    f.v[it] = v;
  }
  f.sc = 0x7F7F7F7Fu;
  if (stid >= 0 && stid < ROWS) {
    const int64_t gr = r0 + stid;
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t kb = (k0 >> 5) + j;
      uint32_t sc = 127u;
      if (gr < rows && kb * 32 < K) sc = op.scales[(two_d ? (gr >> 5) : gr) * op.ld_scales + kb];
      w |= sc << (8 * j);
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

// Tile BM x BN per workgroup; each wave owns TI x TJ MFMA tiles of 32x32
// (waves laid out BM/(32 TI) x BN/(32 TJ)).
template <int FA, int FB, int BM_, int BN_, int TI, int TJ>
constexpr int mx_threads() {
  return 64 * (BM_ / (32 * TI)) * (BN_ / (32 * TJ));
}

// The output tile [m0, m0 + BM_) x [n0, n0 + BN_) of C = A B^T (rows past M
// or N are neither read nor written).
template <int FA, int FB, int BM_, int BN_, int TI, int TJ>
__device__ __forceinline__ void gemm_mx_tile(const MxOperand& A, const MxOperand& B, int64_t M, int64_t N,
                                             int64_t K, int64_t m0, int64_t n0, void* C, int64_t ldc, int a_2d,
                                             int b_2d, int out_bf16) {
  constexpr int WN = BN_ / (32 * TJ);
  constexpr int THREADS = mx_threads<FA, FB, BM_, BN_, TI, TJ>();
  static_assert(THREADS >= BM_ + BN_, "one scale row per thread");
  constexpr int PA = 128 * elem_bits<FA>() / 8 + 16, PB = 128 * elem_bits<FB>() / 8 + 16;
  constexpr int FMA = mfma_fmt<FA>(), FMB = mfma_fmt<FB>();
  __shared__ __attribute__((aligned(16))) uint8_t la[BM_ * PA];
  __shared__ __attribute__((aligned(16))) uint8_t lb[BN_ * PB];
  __shared__ uint32_t lsa[BM_], lsb[BN_];
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
  MxStage<FB, BN_, THREADS> fb;
  if (K > 0) {
    fetch_mx(fa, A, a_2d != 0, m0, M, 0, K, tid);
    fetch_mx(fb, B, b_2d != 0, n0, N, 0, K, tid - BM_);
  }
  for (int64_t k0 = 0; k0 < K; k0 += 128) {
    put_mx(fa, la, PA, lsa, tid);
    put_mx(fb, lb, PB, lsb, tid - BM_);
    __syncthreads();
    if (k0 + 128 < K) {                 // the next stage's loads fly during this stage's MFMAs
      fetch_mx(fa, A, a_2d != 0, m0, M, k0 + 128, K, tid);
      fetch_mx(fb, B, b_2d != 0, n0, N, k0 + 128, K, tid - BM_);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      v8i a[TI], b[TJ];
      int sa[TI], sb[TJ];
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const int r = wm * 32 * TI + i * 32 + l32;
        a[i] = read_mx<FA>(la + r * PA, ks, hi);
        sa[i] = (int)(lsa[r] >> (8 * hi));
      }
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int r = wn * 32 * TJ + j * 32 + l32;
        b[j] = read_mx<FB>(lb + r * PB, ks, hi);
        sb[j] = (int)(lsb[r] >> (8 * hi));
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
  // lane holds column l32; register r holds row 8*(r/4) + 4*hi + r%4
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int64_t col = n0 + wn * 32 * TJ + j * 32 + l32;
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 32 * TI + i * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
        if (row < M) {
          if (out_bf16)
            static_cast<uint16_t*>(C)[row * ldc + col] = (uint16_t)f32_to_bf16_rne(acc[i][j][r]);
          else
            static_cast<float*>(C)[row * ldc + col] = acc[i][j][r];
        }
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

template <int FA, int FB>
hipError_t launch_grouped_gemm_mx(const GroupedGemmArgs& a, hipStream_t st) {
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
hipError_t launch_grouped_gemm_mx_b(const GroupedGemmArgs& a, hipStream_t st) {
  switch (a.b_elem) {
    case 1: return launch_grouped_gemm_mx<FA, 1>(a, st);
    case 2: return launch_grouped_gemm_mx<FA, 2>(a, st);
    case 3: return launch_grouped_gemm_mx<FA, 3>(a, st);
    case 4: return launch_grouped_gemm_mx<FA, 4>(a, st);
    default: return launch_grouped_gemm_mx<FA, 0>(a, st);
  }
}

// 256x256 tiles (8 waves of 64x128) when both dimensions fill them, else
// 128x128 (4 waves of 64x64).
template <int FA, int FB>
hipError_t launch_gemm_mx(const GemmArgs& a, hipStream_t st) {
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
hipError_t launch_gemm_mx_b(const GemmArgs& a, hipStream_t st) {
  switch (a.b_elem) {
    case 1: return launch_gemm_mx<FA, 1>(a, st);
    case 2: return launch_gemm_mx<FA, 2>(a, st);
    case 3: return launch_gemm_mx<FA, 3>(a, st);
    case 4: return launch_gemm_mx<FA, 4>(a, st);
    default: return launch_gemm_mx<FA, 0>(a, st);
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

hipError_t launch_gemm(const GemmArgs& a, hipStream_t st) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  if (a.a_elem != 0 || a.b_elem != 0) {
    switch (a.a_elem) {
      case 1: return launch_gemm_mx_b<1>(a, st);
      case 2: return launch_gemm_mx_b<2>(a, st);
      case 3: return launch_gemm_mx_b<3>(a, st);
      case 4: return launch_gemm_mx_b<4>(a, st);
      default: return launch_gemm_mx_b<0>(a, st);
    }
  }
  // 256x256 tiles: scale rows are fetched 16 bytes at a time (16-byte aligned
  // rows), and the operands are addressed with 32-bit offsets.
  const bool words = (a.A.ld_scales % 16 == 0) && (a.B.ld_scales % 16 == 0) &&
                     ((uintptr_t)a.A.scales % 16 == 0) && ((uintptr_t)a.B.scales % 16 == 0);
  const bool small = a.M * a.A.ld_codes < (1ll << 31) && a.N * a.B.ld_codes < (1ll << 31) &&
                     a.M * a.ldc * (a.out_bf16 ? 2 : 4) < (1ll << 31) && a.K < (1ll << 31);
  if (a.M >= 256 && a.N >= 256 && words && small) {
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

bool gemm_quantize_supported(const GemmQuantArgs& a) {
  const bool out_ok = a.M >= 256 && a.N >= 256 && a.N % 32 == 0 && a.ld_codes % 4 == 0 &&
                      (uintptr_t)a.codes % 4 == 0 && 256 * a.ld_codes < (1ll << 31) &&
                      256 * a.ld_scales < (1ll << 31) && a.ld_codes >= a.N / 2 && a.ld_scales >= a.N / 32;
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
#define MX_GQ(A_, B_)                                                                                   \
  hipLaunchKernelGGL((k_gemm256_q<A_, B_>), dim3(nwg), dim3(64 * GW), 0, st, a.A, a.B, (int)a.M, (int)a.N, \
                     (int)a.K, qo, tiles_m, tiles_n)
  if (a.a_2d) { if (a.b_2d) MX_GQ(true, true); else MX_GQ(true, false); }
  else { if (a.b_2d) MX_GQ(false, true); else MX_GQ(false, false); }
#undef MX_GQ
  return hipGetLastError();
}

bool grouped_quantize_supported(const GroupedQuantArgs& q) {
  const GroupedGemmArgs& a = q.g;
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
    switch (a.a_elem) {
      case 1: return launch_grouped_gemm_mx_b<1>(a, st);
      case 2: return launch_grouped_gemm_mx_b<2>(a, st);
      case 3: return launch_grouped_gemm_mx_b<3>(a, st);
      case 4: return launch_grouped_gemm_mx_b<4>(a, st);
      default: return launch_grouped_gemm_mx_b<0>(a, st);
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
