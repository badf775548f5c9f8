// 256x256-tile mainloop of the MXFP4 GEMMs for gfx950 (shared by the dense and
// grouped kernels).
//
// Work split: a workgroup of W waves (4 or 8) owns a 256x256 output tile; the
// waves form a (W/2) x 2 grid and each owns TI x TJ tiles of
// V_MFMA_SCALE_F32_32X32X64_F8F6F4 (FP4 x FP4, one E8M0 scale per lane and
// operand, float32 accumulators in AGPRs).  With 8 waves two waves share each
// SIMD, so one wave's LDS waits and barrier are covered by the other's matrix
// work.  Operand lane layout of that instruction: lane l supplies row l % 32
// and the 32 K-elements [32*(l/32), 32*(l/32)+32) of the 64-deep step (one
// whole MX block, 16 bytes) with that block's scale byte; result register r of
// lane l is row 8*(r/4) + 4*(l/32) + r%4, column l % 32.
//
// Data movement per 128-deep K stage: A and B codes (256 rows x 64 bytes each)
// and the 4 scale bytes of each row (one aligned 32-bit word: scale rows must
// have a stride that is a multiple of 4 bytes) go global -> LDS with
// direct-to-LDS buffer loads (no VGPR round trip) into a ring of NS stages,
// so NS - 1 stages of loads are in flight while one is multiplied.  Each
// 64-byte LDS code row is XOR-swizzled in 16-byte chunks so the 128-bit LDS
// reads of consecutive rows hit different bank groups.  The operand reads
// from LDS are issued from asm blocks (each waits for its own reads), so the
// compiler does not make them wait for the direct-to-LDS loads still in
// flight into the other ring slots; the ring's own vmcnt waits and barriers
// order the slots.  Raw buffer addressing returns zeros past the end of an
// operand, so rows past M (or N) read as zeros and are never stored; in the
// last, partial K stage the missing chunks are pointed past the end (zero
// codes) and their scale bytes are cleared to 0 (a finite scale), so they add
// exact zeros.
#pragma once

#include <type_traits>

#include "mx_device.h"
#include "mx_launch.h"

namespace mx {
namespace t256 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int TM = 256, TN = 256;
constexpr int TK = 128;                    // K elements per stage
constexpr int ROWB = TK / 2;               // code bytes per row per stage
constexpr int OPB = 256 * ROWB;            // code bytes per operand per stage (16 KiB)
constexpr int SCB = 256 * 4;               // scale bytes per operand per stage (1 KiB)
constexpr int STAGE_BYTES = 2 * OPB + 2 * SCB;
constexpr int NS = 4;                      // stages in the LDS ring
constexpr int LDS_BYTES = NS * STAGE_BYTES;

template <int W>
struct Cfg {
  static_assert(W == 4 || W == 8, "4 or 8 waves");
  static constexpr int WN = 2;                           // waves along N
  static constexpr int WM = W / WN;                      // waves along M
  static constexpr int TI = TM / WM / 32;                // 32-row MFMA tiles per wave along M
  static constexpr int TJ = TN / WN / 32;                // ... along N
  static constexpr int DMA = 16 / W;                     // 1 KiB code loads per wave and operand
  static constexpr int SC_LOADS = (W == 4) ? 2 : 1;      // scale-word loads per wave
  static constexpr int LOADS = 2 * DMA + SC_LOADS;       // loads per wave and stage
};

// 16-byte chunk swizzle inside a 64-byte LDS row: with f = (b2, b1 ^ b3) of
// the row number, any 8 consecutive rows (and any 16 consecutive rows) reading
// the same logical chunk hit distinct 16-byte bank groups of a 128-byte (and
// 256-byte) bank window.
__device__ __forceinline__ int swz(int row, int chunk) {
  return chunk ^ ((((row >> 2) & 1) << 1) | (((row >> 1) ^ (row >> 3)) & 1));
}

// Raw buffer resource over [base, base + bytes): loads past the end return 0
// and stores past the end are dropped (gfx9 raw buffer addressing).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
constexpr uint32_t OOB = 0x80000000u;        // an offset past any operand (validated < 2 GiB)

// Per-lane 32-bit byte offsets, computed once per tile.
template <int W>
struct LaneOffsets {
  uint32_t dma_a[Cfg<W>::DMA], dma_b[Cfg<W>::DMA];   // code chunk of each code load
  int chunk[Cfg<W>::DMA];                           // its logical chunk (K-block within the stage)
  uint32_t sc_a, sc_b;                              // this lane's scale row word
};

template <int W, bool A2D, bool B2D>
__device__ __forceinline__ void lane_offsets(const MxOperand& A, const MxOperand& B, int M, int N,
                                             int m0, int n0, int wave, int lane, LaneOffsets<W>& o) {
#pragma unroll
  for (int t = 0; t < Cfg<W>::DMA; ++t) {
    const int row = 16 * (wave * Cfg<W>::DMA + t) + (lane >> 2);
    const int c = swz(row, lane & 3);
    o.chunk[t] = c;
    o.dma_a[t] = (m0 + row < M) ? (uint32_t)(m0 + row) * (uint32_t)A.ld_codes + 16u * c : OOB;
    o.dma_b[t] = (n0 + row < N) ? (uint32_t)(n0 + row) * (uint32_t)B.ld_codes + 16u * c : OOB;
  }
  // 4 waves: every wave loads 64 A and 64 B scale rows; 8 waves: waves 0-3
  // load the A rows, waves 4-7 the B rows.
  const int r = 64 * (wave & 3) + lane;
  const int ra = m0 + r, rb = n0 + r;
  o.sc_a = ra < M ? (uint32_t)(A2D ? (ra >> 5) : ra) * (uint32_t)A.ld_scales : OOB;
  o.sc_b = rb < N ? (uint32_t)(B2D ? (rb >> 5) : rb) * (uint32_t)B.ld_scales : OOB;
}

// Issue one stage's loads: 256 rows x 64 code bytes of each operand as 16
// direct-to-LDS loads of 1 KiB, and the 32-bit scale word of each row.  In the
// partial last stage, chunks at or past K point past the end and read as zeros.
template <int W, bool TAIL>
__device__ __forceinline__ void issue_stage(__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                            __amdgpu_buffer_rsrc_t rsa, __amdgpu_buffer_rsrc_t rsb,
                                            const LaneOffsets<W>& o, int st, int kchunks,
                                            uint8_t* stage, int wave) {
  const uint32_t cs = (uint32_t)st * (TK / 2), ss = (uint32_t)st * (TK / 32);
  uint8_t* la = stage;
  uint8_t* lb = stage + OPB;
#pragma unroll
  for (int t = 0; t < Cfg<W>::DMA; ++t) {
    const uint32_t va = (TAIL && o.chunk[t] >= kchunks) ? OOB : o.dma_a[t];
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(la + 1024 * (wave * Cfg<W>::DMA + t)), 16,
                                             va, cs, 0, 0);
  }
#pragma unroll
  for (int t = 0; t < Cfg<W>::DMA; ++t) {
    const uint32_t vb = (TAIL && o.chunk[t] >= kchunks) ? OOB : o.dma_b[t];
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(lb + 1024 * (wave * Cfg<W>::DMA + t)), 16,
                                             vb, cs, 0, 0);
  }
  uint8_t* sa = stage + 2 * OPB + 256 * (wave & 3);
  if (W == 4) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_ptr_t)sa, 4, o.sc_a, ss, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_ptr_t)(sa + SCB), 4, o.sc_b, ss, 0, 0);
  } else if (wave < 4) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_ptr_t)sa, 4, o.sc_a, ss, 0, 0);
  } else {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_ptr_t)(sa + SCB), 4, o.sc_b, ss, 0, 0);
  }
}

template <int W>
struct Acc {
  v16f t[Cfg<W>::TI][Cfg<W>::TJ];
};

// ---------------------------------------------------------------- LDS reads
// The operand reads from LDS sit in asm blocks that wait for their own reads
// (outputs are early-clobber: a read may land before a later read of the
// block has taken its address).  Written in asm because the compiler cannot
// tell these reads from the direct-to-LDS loads still in flight into other
// ring slots and would otherwise wait for all of those first.
// Row tiles of one operand are 2048 code bytes / 128 scale-word bytes apart.

// 4 A + 4 B operand chunks of one K step.
__device__ __forceinline__ void lds_read_k(uint32_t ada, uint32_t adb, v4i a[4], v4i b[4]) {
  asm volatile(
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %8 offset:2048\n\t"
      "ds_read_b128 %2, %8 offset:4096\n\t"
      "ds_read_b128 %3, %8 offset:6144\n\t"
      "ds_read_b128 %4, %9\n\t"
      "ds_read_b128 %5, %9 offset:2048\n\t"
      "ds_read_b128 %6, %9 offset:4096\n\t"
      "ds_read_b128 %7, %9 offset:6144\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3]), "=&v"(b[0]), "=&v"(b[1]), "=&v"(b[2]),
        "=&v"(b[3])
      : "v"(ada), "v"(adb)
      : "memory");
}

// 2 A + 4 B operand chunks of one K step.
__device__ __forceinline__ void lds_read_k(uint32_t ada, uint32_t adb, v4i a[2], v4i b[4], int) {
  asm volatile(
      "ds_read_b128 %0, %6\n\t"
      "ds_read_b128 %1, %6 offset:2048\n\t"
      "ds_read_b128 %2, %7\n\t"
      "ds_read_b128 %3, %7 offset:2048\n\t"
      "ds_read_b128 %4, %7 offset:4096\n\t"
      "ds_read_b128 %5, %7 offset:6144\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(a[0]), "=&v"(a[1]), "=&v"(b[0]), "=&v"(b[1]), "=&v"(b[2]), "=&v"(b[3])
      : "v"(ada), "v"(adb)
      : "memory");
}

// Scale words of 4 A + 4 B row tiles.
__device__ __forceinline__ void lds_read_scales(uint32_t ada, uint32_t adb, uint32_t sa[4], uint32_t sb[4]) {
  asm volatile(
      "ds_read_b32 %0, %8\n\t"
      "ds_read_b32 %1, %8 offset:128\n\t"
      "ds_read_b32 %2, %8 offset:256\n\t"
      "ds_read_b32 %3, %8 offset:384\n\t"
      "ds_read_b32 %4, %9\n\t"
      "ds_read_b32 %5, %9 offset:128\n\t"
      "ds_read_b32 %6, %9 offset:256\n\t"
      "ds_read_b32 %7, %9 offset:384\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(sa[0]), "=&v"(sa[1]), "=&v"(sa[2]), "=&v"(sa[3]), "=&v"(sb[0]), "=&v"(sb[1]),
        "=&v"(sb[2]), "=&v"(sb[3])
      : "v"(ada), "v"(adb)
      : "memory");
}

// Scale words of 2 A + 4 B row tiles.
__device__ __forceinline__ void lds_read_scales(uint32_t ada, uint32_t adb, uint32_t sa[2], uint32_t sb[4],
                                                int) {
  asm volatile(
      "ds_read_b32 %0, %6\n\t"
      "ds_read_b32 %1, %6 offset:128\n\t"
      "ds_read_b32 %2, %7\n\t"
      "ds_read_b32 %3, %7 offset:128\n\t"
      "ds_read_b32 %4, %7 offset:256\n\t"
      "ds_read_b32 %5, %7 offset:384\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(sa[0]), "=&v"(sa[1]), "=&v"(sb[0]), "=&v"(sb[1]), "=&v"(sb[2]), "=&v"(sb[3])
      : "v"(ada), "v"(adb)
      : "memory");
}

template <int W>
__device__ __forceinline__ void read_k(uint32_t ada, uint32_t adb, v4i* a, v4i* b) {
  if constexpr (Cfg<W>::TI == 4) lds_read_k(ada, adb, a, b);
  else lds_read_k(ada, adb, a, b, 0);
}
template <int W>
__device__ __forceinline__ void read_scales(uint32_t ada, uint32_t adb, uint32_t* sa, uint32_t* sb) {
  if constexpr (Cfg<W>::TI == 4) lds_read_scales(ada, adb, sa, sb);
  else lds_read_scales(ada, adb, sa, sb, 0);
}

// Multiply one stage held in LDS at byte address `stage`.  Scale word of a
// row = 4 scale bytes of the stage's 4 K-blocks; lane l of a K step ks needs
// K-block 2*ks + l/32, so the word is shifted right by 8*(l/32) and op_sel
// picks byte 2*ks.  `keep` masks the bytes of K-blocks that exist (all of them
// except in a partial last stage, whose missing blocks get scale byte 0, a
// finite scale; their codes are 0).
template <int W>
__device__ __forceinline__ void compute_stage(uint32_t stage, int wm, int wn, int lane, uint32_t keep,
                                              Acc<W>& acc) {
  constexpr int TI = Cfg<W>::TI, TJ = Cfg<W>::TJ;
  const int l32 = lane & 31, kh = lane >> 5;
  const int rowa = wm * TI * 32 + l32, rowb = wn * TJ * 32 + l32;   // row tile 0
  uint32_t wa[TI], wb[TJ];
  read_scales<W>(stage + 2 * OPB + 4 * rowa, stage + 2 * OPB + SCB + 4 * rowb, wa, wb);
  int sa[TI], sb[TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i) sa[i] = (int)((wa[i] & keep) >> (8 * kh));
#pragma unroll
  for (int j = 0; j < TJ; ++j) sb[j] = (int)((wb[j] & keep) >> (8 * kh));
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    // the chunk swizzle depends on bits 1..3 of the row only, equal for all tiles
    v4i av[TI], bv[TJ];
    read_k<W>(stage + rowa * ROWB + 16 * swz(rowa, 2 * ks + kh),
              stage + OPB + rowb * ROWB + 16 * swz(rowb, 2 * ks + kh), av, bv);
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const v8i a = v8i{av[i].x, av[i].y, av[i].z, av[i].w, 0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const v8i b = v8i{bv[j].x, bv[j].y, bv[j].z, bv[j].w, 0, 0, 0, 0};
        if (ks == 0)
          acc.t[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc.t[i][j], 4, 4, 0, sa[i], 0,
                                                                       sb[j]);
        else
          acc.t[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc.t[i][j], 4, 4, 2, sa[i], 2,
                                                                       sb[j]);
      }
    }
  }
}

// Wait until at most `stages_ahead` stages of this wave's vector-memory loads
// are outstanding (0, 1 or 2 stages).
template <int W>
__device__ __forceinline__ void wait_vmcnt(int stages_ahead) {
  // s_waitcnt encoding (gfx9): vmcnt bits [3:0] and [15:14]; expcnt and
  // lgkmcnt left at their maxima (no wait).
#define MX_VMCNT(N_) (((N_) & 0xF) | (((N_) >> 4) << 14) | (0x7 << 4) | (0xF << 8))
  constexpr int L = Cfg<W>::LOADS;
  switch (stages_ahead) {
    case 0: __builtin_amdgcn_s_waitcnt(MX_VMCNT(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(MX_VMCNT(L)); break;
    default: __builtin_amdgcn_s_waitcnt(MX_VMCNT(2 * L)); break;
  }
#undef MX_VMCNT
}

// C tile (rows m0.., cols n0..) = A[m0:m0+256] * B[n0:n0+256]^T over all K.
// Operand rows past M/N read as zeros; the caller's epilogue stores only
// valid rows and columns.  Byte extents of the operands must be < 2 GiB.
// `lds` holds the NS ring slots back to back.
template <int W, bool A2D, bool B2D>
__device__ __forceinline__ void mainloop(const MxOperand& A, const MxOperand& B, int M, int N, int K,
                                         int m0, int n0, uint8_t* lds, Acc<W>& acc) {
  static_assert(NS == 4, "wait_vmcnt assumes at most 2 stages queued behind the current one");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int i = 0; i < Cfg<W>::TI; ++i)
#pragma unroll
    for (int j = 0; j < Cfg<W>::TJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc.t[i][j][r] = 0.0f;

  const int nstages = (K + TK - 1) / TK;
  const int nfull = K / TK;                 // stages without a K tail
  if (nstages == 0) return;
  const __amdgpu_buffer_rsrc_t ra = rsrc(A.codes, (uint32_t)(M * A.ld_codes));
  const __amdgpu_buffer_rsrc_t rb = rsrc(B.codes, (uint32_t)(N * B.ld_codes));
  const __amdgpu_buffer_rsrc_t rsa = rsrc(A.scales, (uint32_t)((A2D ? M / 32 : M) * A.ld_scales));
  const __amdgpu_buffer_rsrc_t rsb = rsrc(B.scales, (uint32_t)((B2D ? N / 32 : N) * B.ld_scales));
  LaneOffsets<W> o;
  lane_offsets<W, A2D, B2D>(A, B, M, N, m0, n0, wave, lane, o);
  const int kchunks = (K - nfull * TK) / 32;          // K-blocks in the tail stage (0 if none)
  const uint32_t tail_keep = (1u << (8 * kchunks)) - 1u;
  const uint32_t lds_addr = (uint32_t)(uintptr_t)(lds_ptr_t)lds;   // LDS byte address of slot 0

  auto issue = [&](int p) {
    uint8_t* slot = lds + (p % NS) * STAGE_BYTES;
    if (p < nfull) issue_stage<W, false>(ra, rb, rsa, rsb, o, p, 4, slot, wave);
    else if (p < nstages) issue_stage<W, true>(ra, rb, rsa, rsb, o, p, kchunks, slot, wave);
  };
#pragma unroll
  for (int p = 0; p < NS - 1; ++p) issue(p);
  for (int s = 0; s < nstages; ++s) {
    // loads of the stages after s that are already issued stay in flight
    const int ahead = (nstages - 1 - s) < (NS - 2) ? (nstages - 1 - s) : (NS - 2);
    wait_vmcnt<W>(ahead);                   // this wave's stage-s loads landed
    // every wave's did, and the slot of stage s-1 is free.  A bare barrier:
    // __syncthreads() would add a fence that waits for all loads in flight.
    // The empty asm statements keep the compiler from moving memory
    // operations (the next loads into the freed slot) across it.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    issue(s + NS - 1);
    compute_stage<W>(lds_addr + (uint32_t)((s % NS) * STAGE_BYTES), wm, wn, lane,
                     s < nfull ? 0xFFFFFFFFu : tail_keep, acc);
  }
  __syncthreads();                          // LDS may be reused by the caller
}

// Store the wave's part of the tile with bounds-checked buffer stores: the
// resource ends after row mlim (relative to the tile origin C), and lanes
// whose column is >= nlim point past it, so nothing outside the matrix is
// written.  Row offsets are wave-uniform (scalar), column offsets per lane.
template <int W, bool OUT_BF16>
__device__ __forceinline__ void store_tile(const Acc<W>& acc, void* C, int ldc, int mlim, int nlim) {
  constexpr int TI = Cfg<W>::TI, TJ = Cfg<W>::TJ;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, kh = lane >> 5;
  constexpr int ES = OUT_BF16 ? 2 : 4;
  const int rows = mlim < 256 ? mlim : 256;
  const __amdgpu_buffer_rsrc_t r = rsrc(C, (uint32_t)((rows - 1) * ldc * ES + (nlim < 256 ? nlim : 256) * ES));
#pragma unroll
  for (int j = 0; j < TJ; ++j) {
    const int col = wn * TJ * 32 + 32 * j + l32;
    const uint32_t voff = col < nlim ? (uint32_t)(((wm * TI * 32 + 4 * kh) * ldc + col) * ES) : OOB;
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t soff = (uint32_t)((32 * i + 8 * r4 + q) * ldc * ES);
          const float v = acc.t[i][j][4 * r4 + q];
          if (OUT_BF16)
            __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (__bf16)v), r, voff,
                                                  soff, 0);
          else
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, voff, soff, 0);
        }
  }
}

}  // namespace t256
}  // namespace mx
