// Four-wave variant of the 256x256-tile MXFP4 GEMM mainloop for gfx950.
//
// Same tile, stage, LDS layout and persistent schedule as the eight-wave
// mainloop (gemm_tile256.h), with a different split of the work inside the
// workgroup: 4 waves, one per SIMD, in a 2 x 2 grid, each owning 128 x 128
// of the tile = 4 x 4 tiles of V_MFMA_SCALE_F32_32X32X64_F8F6F4 with the
// float32 accumulators in AGPRs (256 per wave).  Per 64-deep K step a wave
// reads 4 A and 4 B operand chunks for 16 MFMAs (eight waves read 2 + 4 for
// 8), so LDS read traffic is a third lower, and the arch VGPRs hold four
// steps of operands, a whole stage.
//
// Pipeline of stage g (steps 0-3), one barrier per stage:
//   step 0: MFMAs on step 0's operands; read step 2's operands of stage g
//   step 1: MFMAs on step 1's; read step 3's of stage g
//   -- stage g+1 landed (this wave's loads, then every wave's, by the
//      barrier); every wave has also finished reading stage g from LDS --
//   step 2: MFMAs on step 2's; read step 0's of stage g+1; issue the 8 A
//           code loads of stage g+2 into stage g's slot
//   step 3: MFMAs on step 3's; read step 1's of stage g+1 and its scale
//           bytes; issue the 8 B code loads of stage g+2
// so a stage's loads are spread over two steps (32 MFMAs) and have four
// steps to land.  The accumulators of a finished tile are stored while the
// next tile's first stages load.
#pragma once

#include "gemm_tile256.h"

namespace mx {
namespace t4 {

using t256::LDS_BYTES;
using t256::OOB;
using t256::OPB;
using t256::ROWB;
using t256::SROWB;
using t256::SSLOT;
using t256::STAGE_BYTES;
using t256::Strides;
using t256::TileInfo;
using t256::TK;
using t256::TM;
using t256::TN;
using t256::lds_ptr_t;
using t256::rsrc;
using t256::swz;
using t256::v16f;
using t256::v2u;
using t256::v4i;

constexpr int WAVES = 4;                   // 2 along M x 2 along N
constexpr int TI = 4, TJ = 4;              // 32x32 MFMA tiles per wave along M, N

struct Acc {
  v16f t[TI][TJ];
};

// One step's operands: the 16-byte chunk of each of the wave's 4 A and 4 B
// row tiles.
struct Ops {
  v4i a[TI], b[TJ];
};

// This wave's code loads of a tile: load t (0..7) of an operand covers rows
// 8*(8*wave+t) .. +8, lane l the swizzled chunk of row l/8 of those.  The
// row of load t is base_row + 8t with base_row = 64*wave + l/8, and its
// chunk depends only on the parity of t.
__device__ __forceinline__ int load_chunk(int wave, int lane, int t) {
  return swz(8 * (wave * 8 + t) + (lane >> 3), lane & 7);
}

// Per-tile state of one operand's loads: the byte offset of this lane's row
// of load 0 and the number of rows of that operand left below its limit,
// counted from that row (loads of rows at or past the limit read zeros).
struct LoadBase {
  uint32_t off;                  // (first row + base_row) * ld
  int rows_left;                 // limit - (first row + base_row)
};

__device__ __forceinline__ LoadBase load_base(int first, int limit, int ld, int wave, int lane) {
  const int r = first + 64 * wave + (lane >> 3);
  return {(uint32_t)r * (uint32_t)ld, limit - r};
}

// The 8 load offsets of stage s of one operand (tail stage: chunks at or
// past K read zeros).
__device__ __forceinline__ void load_offsets(const LoadBase& lb, int ld, int s, int nfull, int kchunks, int wave,
                                             int lane, uint32_t v[8]) {
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int c = load_chunk(wave, lane, t);
    const bool live = (s < nfull || c < kchunks) && 8 * t < lb.rows_left;
    v[t] = live ? lb.off + (uint32_t)(8 * t * ld) + 16u * c : OOB;
  }
}

// Scale rows of a tile loaded by this wave: waves 0 and 1 load A rows
// 128*wave + 64*u + lane, waves 2 and 3 B rows 128*(wave-2) + 64*u + lane.
template <bool A2D, bool B2D>
__device__ __forceinline__ void scale_offsets(const TileInfo& ti, const Strides& sd, int wave, int lane,
                                              uint32_t off[2]) {
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int r = 128 * (wave & 1) + 64 * u + lane;
    if (wave < 2) {
      const int ra = ti.m0 + r;
      off[u] = ra < ti.M ? (uint32_t)(A2D ? (ra >> 5) : ra) * (uint32_t)sd.ldsa : OOB;
    } else {
      const int rb = ti.n0 + r;
      off[u] = rb < ti.N ? (uint32_t)(B2D ? (rb >> 5) : rb) * (uint32_t)sd.ldsb : OOB;
    }
  }
}

template <bool A2D, bool B2D>
__device__ __forceinline__ void tile_rsrc(const TileInfo& ti, const Strides& sd, int wave, __amdgpu_buffer_rsrc_t& ra,
                                          __amdgpu_buffer_rsrc_t& rb, __amdgpu_buffer_rsrc_t& rs) {
  ra = rsrc(ti.a_codes, (uint32_t)(ti.M * sd.lda));
  rb = rsrc(ti.b_codes, (uint32_t)(ti.N * sd.ldb));
  rs = wave < 2 ? rsrc(ti.a_scales, (uint32_t)((A2D ? ti.M / 32 : ti.M) * sd.ldsa))
                : rsrc(ti.b_scales, (uint32_t)((B2D ? ti.N / 32 : ti.N) * sd.ldsb));
}

// Scale loads of stages 2q and 2q+1 of a tile into `sslot` (16 bytes per row).
__device__ __forceinline__ void issue_scales(__amdgpu_buffer_rsrc_t rs, const uint32_t off[2], int q, uint8_t* sslot,
                                             int wave) {
  uint8_t* dst = sslot + (wave < 2 ? 0 : 256 * SROWB) + 128 * SROWB * (wave & 1);
#pragma unroll
  for (int u = 0; u < 2; ++u)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(dst + 64 * SROWB * u), 16, off[u], (uint32_t)q * SROWB,
                                             0, 0);
}

// Code loads of one stage with the compiler's builtin (before the pipeline runs).
__device__ __forceinline__ void issue_codes(__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb, const uint32_t va[8],
                                            const uint32_t vb[8], uint32_t cs, uint8_t* slot, int wave) {
#pragma unroll
  for (int t = 0; t < 8; ++t)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(slot + 1024 * (wave * 8 + t)), 16, va[t], cs, 0, 0);
#pragma unroll
  for (int t = 0; t < 8; ++t)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(slot + OPB + 1024 * (wave * 8 + t)), 16, vb[t], cs, 0,
                                             0);
}

// ------------------------------------------------------------ asm K steps
// Row tiles are 4096 code bytes and 512 scale bytes apart in a slot.  op_sel
// picks byte 0 (even step) or 2 (odd step) of each lane's scale word, which
// is already shifted right by 8 * (l / 32).
#define MX4_LO "0,0,0"
#define MX4_HI "1,1,0"
#define MX4_MFMA(I, J, OPSEL)                                                                          \
  "v_mfma_scale_f32_32x32x64_f8f6f4 %[c" #I #J "], %[a" #I "], %[b" #J "], %[c" #I #J "], %[sa" #I \
  "], %[sb" #J "] op_sel_hi:[" OPSEL "] cbsz:4 blgp:4\n\t"
#define MX4_ACC(c)                                                                                           \
  [c00] "+a"(c.t[0][0]), [c01] "+a"(c.t[0][1]), [c02] "+a"(c.t[0][2]), [c03] "+a"(c.t[0][3]),             \
      [c10] "+a"(c.t[1][0]), [c11] "+a"(c.t[1][1]), [c12] "+a"(c.t[1][2]), [c13] "+a"(c.t[1][3]),         \
      [c20] "+a"(c.t[2][0]), [c21] "+a"(c.t[2][1]), [c22] "+a"(c.t[2][2]), [c23] "+a"(c.t[2][3]),         \
      [c30] "+a"(c.t[3][0]), [c31] "+a"(c.t[3][1]), [c32] "+a"(c.t[3][2]), [c33] "+a"(c.t[3][3])
#define MX4_OUT(n)                                                                                           \
  [na0] "=&v"(n.a[0]), [na1] "=&v"(n.a[1]), [na2] "=&v"(n.a[2]), [na3] "=&v"(n.a[3]), [nb0] "=&v"(n.b[0]), \
      [nb1] "=&v"(n.b[1]), [nb2] "=&v"(n.b[2]), [nb3] "=&v"(n.b[3])
#define MX4_IN(x, sa, sb)                                                                                    \
  [a0] "v"(x.a[0]), [a1] "v"(x.a[1]), [a2] "v"(x.a[2]), [a3] "v"(x.a[3]), [b0] "v"(x.b[0]),                \
      [b1] "v"(x.b[1]), [b2] "v"(x.b[2]), [b3] "v"(x.b[3]), [sa0] "v"(sa[0]), [sa1] "v"(sa[1]),             \
      [sa2] "v"(sa[2]), [sa3] "v"(sa[3]), [sb0] "v"(sb[0]), [sb1] "v"(sb[1]), [sb2] "v"(sb[2]),             \
      [sb3] "v"(sb[3])
// The 8 operand reads of one step (A tiles at ada, B tiles at adb).
#define MX4_R0 "ds_read_b128 %[na0], %[ada]\n\t"
#define MX4_R1 "ds_read_b128 %[na1], %[ada] offset:4096\n\t"
#define MX4_R2 "ds_read_b128 %[na2], %[ada] offset:8192\n\t"
#define MX4_R3 "ds_read_b128 %[na3], %[ada] offset:12288\n\t"
#define MX4_R4 "ds_read_b128 %[nb0], %[adb]\n\t"
#define MX4_R5 "ds_read_b128 %[nb1], %[adb] offset:4096\n\t"
#define MX4_R6 "ds_read_b128 %[nb2], %[adb] offset:8192\n\t"
#define MX4_R7 "ds_read_b128 %[nb3], %[adb] offset:12288\n\t"
// 16 MFMAs with the 8 reads after the first 8 of them; X0..X7 go after the
// odd-numbered MFMAs.
#define MX4_BODY(OPSEL, X0, X1, X2, X3, X4, X5, X6, X7)                                                   \
  "s_nop 1\n\t" MX4_MFMA(0, 0, OPSEL) MX4_R0 MX4_MFMA(0, 1, OPSEL) MX4_R1 X0 MX4_MFMA(0, 2, OPSEL) MX4_R2 \
      MX4_MFMA(0, 3, OPSEL) MX4_R3 X1 MX4_MFMA(1, 0, OPSEL) MX4_R4 MX4_MFMA(1, 1, OPSEL) MX4_R5 X2        \
          MX4_MFMA(1, 2, OPSEL) MX4_R6 MX4_MFMA(1, 3, OPSEL) MX4_R7 X3 MX4_MFMA(2, 0, OPSEL)              \
              MX4_MFMA(2, 1, OPSEL) X4 MX4_MFMA(2, 2, OPSEL) MX4_MFMA(2, 3, OPSEL) X5                     \
                  MX4_MFMA(3, 0, OPSEL) MX4_MFMA(3, 1, OPSEL) X6 MX4_MFMA(3, 2, OPSEL)                    \
                      MX4_MFMA(3, 3, OPSEL) X7 "s_waitcnt lgkmcnt(0)"

// A step that only reads the next operands (steps 0 and 1).
template <bool ODD>
__device__ __forceinline__ void step_rd(Acc& c, const Ops& x, const int sa[TI], const int sb[TJ], uint32_t ada,
                                        uint32_t adb, Ops& n) {
  if constexpr (!ODD)
    asm volatile(MX4_BODY(MX4_LO, "", "", "", "", "", "", "", "")
                 : MX4_ACC(c), MX4_OUT(n)
                 : MX4_IN(x, sa, sb), [ada] "v"(ada), [adb] "v"(adb)
                 : "memory");
  else
    asm volatile(MX4_BODY(MX4_HI, "", "", "", "", "", "", "", "")
                 : MX4_ACC(c), MX4_OUT(n)
                 : MX4_IN(x, sa, sb), [ada] "v"(ada), [adb] "v"(adb)
                 : "memory");
}

#define MX4_LD(V) "buffer_load_dwordx4 %[" #V "], %[rc], %[cs] offen lds\n\ts_add_u32 m0, m0, 0x400\n\t"

// Step 2: also issues 8 code loads (LDS addresses m0, m0+1024, ...) at
// per-lane offsets v[] plus the stage offset cs, through resource rc.
__device__ __forceinline__ void step_ld(Acc& c, const Ops& x, const int sa[TI], const int sb[TJ], uint32_t ada,
                                        uint32_t adb, Ops& n, uint32_t m0, const uint32_t v[8],
                                        __amdgpu_buffer_rsrc_t rc, uint32_t cs) {
  asm volatile(MX4_BODY(MX4_LO, MX4_LD(v0), MX4_LD(v1), MX4_LD(v2), MX4_LD(v3), MX4_LD(v4), MX4_LD(v5), MX4_LD(v6),
                        MX4_LD(v7))
               : MX4_ACC(c), MX4_OUT(n), [m0] "+{m0}"(m0)
               : MX4_IN(x, sa, sb), [ada] "v"(ada), [adb] "v"(adb), [v0] "v"(v[0]), [v1] "v"(v[1]), [v2] "v"(v[2]),
                 [v3] "v"(v[3]), [v4] "v"(v[4]), [v5] "v"(v[5]), [v6] "v"(v[6]), [v7] "v"(v[7]), [rc] "s"(rc),
                 [cs] "s"(cs)
               : "memory");
}

// Step 3: as step 2, and reads the next stage's 8 scale bytes per row tile
// (adsa, adsb) into wa, wb.
#define MX4_S(W, AD, OFF) "ds_read_b64 %[" #W "], %[" #AD "]" OFF "\n\t"
__device__ __forceinline__ void step_last(Acc& c, const Ops& x, const int sa[TI], const int sb[TJ], uint32_t ada,
                                          uint32_t adb, uint32_t adsa, uint32_t adsb, Ops& n, v2u wa[TI], v2u wb[TJ],
                                          uint32_t m0, const uint32_t v[8], __amdgpu_buffer_rsrc_t rc, uint32_t cs) {
  asm volatile(MX4_BODY(MX4_HI, MX4_LD(v0) MX4_S(wa0, adsa, ""), MX4_LD(v1) MX4_S(wa1, adsa, " offset:512"),
                        MX4_LD(v2) MX4_S(wa2, adsa, " offset:1024"), MX4_LD(v3) MX4_S(wa3, adsa, " offset:1536"),
                        MX4_LD(v4) MX4_S(wb0, adsb, ""), MX4_LD(v5) MX4_S(wb1, adsb, " offset:512"),
                        MX4_LD(v6) MX4_S(wb2, adsb, " offset:1024"), MX4_LD(v7) MX4_S(wb3, adsb, " offset:1536"))
               : MX4_ACC(c), MX4_OUT(n), [wa0] "=&v"(wa[0]), [wa1] "=&v"(wa[1]), [wa2] "=&v"(wa[2]),
                 [wa3] "=&v"(wa[3]), [wb0] "=&v"(wb[0]), [wb1] "=&v"(wb[1]), [wb2] "=&v"(wb[2]), [wb3] "=&v"(wb[3]),
                 [m0] "+{m0}"(m0)
               : MX4_IN(x, sa, sb), [ada] "v"(ada), [adb] "v"(adb), [adsa] "v"(adsa), [adsb] "v"(adsb),
                 [v0] "v"(v[0]), [v1] "v"(v[1]), [v2] "v"(v[2]), [v3] "v"(v[3]), [v4] "v"(v[4]), [v5] "v"(v[5]),
                 [v6] "v"(v[6]), [v7] "v"(v[7]), [rc] "s"(rc), [cs] "s"(cs)
               : "memory");
}

// The first stage's step 0 and 1 operands and scale bytes.
__device__ __forceinline__ void read_first(uint32_t ada0, uint32_t adb0, uint32_t ada1, uint32_t adb1, uint32_t adsa,
                                           uint32_t adsb, Ops& x0, Ops& x1, v2u wa[TI], v2u wb[TJ]) {
  asm volatile(
      "ds_read_b128 %[x0a0], %[ada0]\n\t"
      "ds_read_b128 %[x0a1], %[ada0] offset:4096\n\t"
      "ds_read_b128 %[x0a2], %[ada0] offset:8192\n\t"
      "ds_read_b128 %[x0a3], %[ada0] offset:12288\n\t"
      "ds_read_b128 %[x0b0], %[adb0]\n\t"
      "ds_read_b128 %[x0b1], %[adb0] offset:4096\n\t"
      "ds_read_b128 %[x0b2], %[adb0] offset:8192\n\t"
      "ds_read_b128 %[x0b3], %[adb0] offset:12288\n\t"
      "ds_read_b128 %[x1a0], %[ada1]\n\t"
      "ds_read_b128 %[x1a1], %[ada1] offset:4096\n\t"
      "ds_read_b128 %[x1a2], %[ada1] offset:8192\n\t"
      "ds_read_b128 %[x1a3], %[ada1] offset:12288\n\t"
      "ds_read_b128 %[x1b0], %[adb1]\n\t"
      "ds_read_b128 %[x1b1], %[adb1] offset:4096\n\t"
      "ds_read_b128 %[x1b2], %[adb1] offset:8192\n\t"
      "ds_read_b128 %[x1b3], %[adb1] offset:12288\n\t"
      "s_waitcnt lgkmcnt(0)\n\t"
      "ds_read_b64 %[wa0], %[adsa]\n\t"
      "ds_read_b64 %[wa1], %[adsa] offset:512\n\t"
      "ds_read_b64 %[wa2], %[adsa] offset:1024\n\t"
      "ds_read_b64 %[wa3], %[adsa] offset:1536\n\t"
      "ds_read_b64 %[wb0], %[adsb]\n\t"
      "ds_read_b64 %[wb1], %[adsb] offset:512\n\t"
      "ds_read_b64 %[wb2], %[adsb] offset:1024\n\t"
      "ds_read_b64 %[wb3], %[adsb] offset:1536\n\t"
      "s_waitcnt lgkmcnt(0)"
      : [x0a0] "=&v"(x0.a[0]), [x0a1] "=&v"(x0.a[1]), [x0a2] "=&v"(x0.a[2]), [x0a3] "=&v"(x0.a[3]),
        [x0b0] "=&v"(x0.b[0]), [x0b1] "=&v"(x0.b[1]), [x0b2] "=&v"(x0.b[2]), [x0b3] "=&v"(x0.b[3]),
        [x1a0] "=&v"(x1.a[0]), [x1a1] "=&v"(x1.a[1]), [x1a2] "=&v"(x1.a[2]), [x1a3] "=&v"(x1.a[3]),
        [x1b0] "=&v"(x1.b[0]), [x1b1] "=&v"(x1.b[1]), [x1b2] "=&v"(x1.b[2]), [x1b3] "=&v"(x1.b[3]),
        [wa0] "=&v"(wa[0]), [wa1] "=&v"(wa[1]), [wa2] "=&v"(wa[2]), [wa3] "=&v"(wa[3]), [wb0] "=&v"(wb[0]),
        [wb1] "=&v"(wb[1]), [wb2] "=&v"(wb[2]), [wb3] "=&v"(wb[3])
      : [ada0] "v"(ada0), [adb0] "v"(adb0), [ada1] "v"(ada1), [adb1] "v"(adb1), [adsa] "v"(adsa), [adsb] "v"(adsb)
      : "memory");
}

// Wait states between the last MFMA and any later access to the accumulators.
__device__ __forceinline__ void drain(Acc& c) { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : MX4_ACC(c)); }

#undef MX4_S
#undef MX4_LD
#undef MX4_BODY
#undef MX4_R0
#undef MX4_R1
#undef MX4_R2
#undef MX4_R3
#undef MX4_R4
#undef MX4_R5
#undef MX4_R6
#undef MX4_R7
#undef MX4_IN
#undef MX4_OUT
#undef MX4_ACC
#undef MX4_MFMA
#undef MX4_LO
#undef MX4_HI

__device__ __forceinline__ void zero(Acc& acc) {
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc.t[i][j][r] = 0.0f;
}

// Store the wave's 128 x 128 part of the tile (bounds as in the eight-wave
// epilogue: the resource ends after row mlim, lanes past column nlim point
// past it).
template <bool OUT_BF16>
__device__ __forceinline__ void store_tile(const Acc& acc, void* C, int ldc, int mlim, int nlim) {
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
    for (int i = 0; i < TI; ++i) {
      // read this MFMA tile's accumulators out of the AGPRs only here (the
      // empty asm pins them), not all 256 at once
      v16f t = acc.t[i][j];
      asm volatile("" : "+v"(t));
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t soff = (uint32_t)((32 * i + 8 * r4 + q) * ldc * ES);
          const float v = t[4 * r4 + q];
          if (OUT_BF16)
            __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (__bf16)v), r, voff, soff, 0);
          else
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, voff, soff, 0);
        }
    }
  }
}

// Run this workgroup's tiles (see t256::run_tiles for the stage sequence,
// slot and scale-pair numbering; here 4 waves and the pipeline above).
template <bool A2D, bool B2D, bool OUT_BF16, class Sched>
__device__ __forceinline__ void run_tiles(const Sched& sc, const Strides& sd, int K, void* C, int64_t ldc,
                                          uint8_t* lds) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int ntiles = sc.count();
  if (ntiles <= 0) return;
  Acc acc;
  t4::zero(acc);
  constexpr int ES = OUT_BF16 ? 2 : 4;
  auto store = [&](const TileInfo& ti) {
    t4::store_tile<OUT_BF16>(acc, static_cast<uint8_t*>(C) + (ti.c_row0 * ldc + ti.n0) * ES, (int)ldc,
                             ti.M - ti.m0, ti.N - ti.n0);
  };
  const int nst = (K + TK - 1) / TK;
  if (nst == 0) {
    for (int j = 0; j < ntiles; ++j) store(sc.tile(j));
    return;
  }
  const int nfull = K / TK;
  const int kchunks = (K - nfull * TK) / 32;
  const int npairs = (nst + 1) / 2;
  const int gtotal = ntiles * nst;
  const uint32_t tail_lo = kchunks >= 4 ? 0xFFFFFFFFu : (1u << (8 * kchunks)) - 1u;
  const uint32_t tail_hi = kchunks <= 4 ? 0u : (1u << (8 * (kchunks - 4))) - 1u;
  uint8_t* const sslots = lds + 2 * STAGE_BYTES;
  const uint32_t lds_addr = (uint32_t)(uintptr_t)(lds_ptr_t)lds;
  const uint32_t sl_addr = lds_addr + 2 * STAGE_BYTES;

  // LDS read offsets of step ks inside a slot: row tile 0 of A and of B, XOR
  // 32*ks (the swizzled chunk 2*ks + l/32 of a row).
  auto sslot_of = [&](int j, int s) { return ((j * npairs + (s >> 1)) & 1) * SSLOT; };

  // Prefetch position (tile j2, stage s2) and its tile's load state.
  int j2 = 0, s2 = 0;
  TileInfo t2 = sc.tile(0);
  __amdgpu_buffer_rsrc_t ra2, rb2, rs2;
  LoadBase la, lb;
  uint32_t psc[2];
  auto load_tile = [&]() {
    t4::tile_rsrc<A2D, B2D>(t2, sd, wave, ra2, rb2, rs2);
    la = t4::load_base(t2.m0, t2.M, sd.lda, wave, lane);
    lb = t4::load_base(t2.n0, t2.N, sd.ldb, wave, lane);
    t4::scale_offsets<A2D, B2D>(t2, sd, wave, lane, psc);
  };
  auto advance = [&]() {
    if (++s2 == nst) {
      s2 = 0;
      if (++j2 < ntiles) {
        t2 = sc.tile(j2);
        load_tile();
      }
    }
  };
  auto stage_offsets = [&](const LoadBase& b, int ld, uint32_t* v) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    t4::load_offsets(b, ld, s2, nfull, kchunks, wave, ln, v);
  };
  load_tile();

#pragma unroll
  for (int g = 0; g < 2; ++g) {
    if (g >= gtotal) break;
    if (!(s2 & 1)) t4::issue_scales(rs2, psc, s2 >> 1, sslots + sslot_of(j2, s2), wave);
    uint32_t va[8], vb[8];
    stage_offsets(la, sd.lda, va);
    stage_offsets(lb, sd.ldb, vb);
    t4::issue_codes(ra2, rb2, va, vb, (uint32_t)s2 * ROWB, lds + (g & 1) * STAGE_BYTES, wave);
    advance();
  }
  t256::wait_vmcnt(0);                      // both prologue stages landed (this wave's loads)
  t256::bare_barrier();                     // ... and every wave's
  Ops x0, x1, x2, x3;
  v2u wa[TI], wb[TJ];
  {
    const int l32 = lane & 31, kh = lane >> 5;
    const int rowa = wm * TI * 32 + l32, rowb = wn * TJ * 32 + l32;
    const uint32_t ra0 = rowa * ROWB + 16 * swz(rowa, kh);
    const uint32_t rb0 = OPB + rowb * ROWB + 16 * swz(rowb, kh);
    const uint32_t s_a = rowa * SROWB, s_b = 256 * SROWB + rowb * SROWB;
    t4::read_first(lds_addr + ra0, lds_addr + rb0, lds_addr + (ra0 ^ 32u), lds_addr + (rb0 ^ 32u), sl_addr + s_a,
             sl_addr + s_b, x0, x1, wa, wb);
  }

  int s = 0, j = 0;
  int s1 = 1 % nst, j1 = 1 / nst;
  for (int g = 0; g < gtotal; ++g) {
    // The per-lane offsets are cheap to recompute; an opaque copy of the lane
    // index keeps the compiler from holding all of them in registers across
    // the loop (the 4 operand sets already take half of the arch VGPRs).
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int l32 = ln & 31, kh = ln >> 5;
    const int rowa = wm * TI * 32 + l32, rowb = wn * TJ * 32 + l32;
    const uint32_t ra0 = rowa * ROWB + 16 * swz(rowa, kh);
    const uint32_t rb0 = OPB + rowb * ROWB + 16 * swz(rowb, kh);
    const uint32_t s_a = rowa * SROWB, s_b = 256 * SROWB + rowb * SROWB;
    const int sh = 8 * kh;
    const uint32_t slot = lds_addr + (uint32_t)((g & 1) * STAGE_BYTES);
    const uint32_t keep_lo = s < nfull ? 0xFFFFFFFFu : tail_lo;
    const uint32_t keep_hi = s < nfull ? 0xFFFFFFFFu : tail_hi;
    int sa[TI], sb[TJ], sa2[TI], sb2[TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      sa[i] = (int)((wa[i].x & keep_lo) >> sh);
      sa2[i] = (int)((wa[i].y & keep_hi) >> sh);
    }
#pragma unroll
    for (int jj = 0; jj < TJ; ++jj) {
      sb[jj] = (int)((wb[jj].x & keep_lo) >> sh);
      sb2[jj] = (int)((wb[jj].y & keep_hi) >> sh);
    }
    t4::step_rd<false>(acc, x0, sa, sb, slot + (ra0 ^ 64u), slot + (rb0 ^ 64u), x2);
    t4::step_rd<true>(acc, x1, sa, sb, slot + (ra0 ^ 96u), slot + (rb0 ^ 96u), x3);
    // Stage g+1 landed (this wave's loads, then every wave's); every wave has
    // read all of stage g, so its slot takes stage g+2.
    t256::wait_vmcnt(0);
    t256::bare_barrier();
    // Stage g+2's loads (past the last stage: every load points past the end).
    const bool more = g + 2 < gtotal;
    if (more && !(s2 & 1)) t4::issue_scales(rs2, psc, s2 >> 1, sslots + sslot_of(j2, s2), wave);
    const uint32_t cs2 = (uint32_t)s2 * ROWB;
    const uint32_t m0a = slot + 1024u * (wave * 8);
    const uint32_t next = lds_addr + (uint32_t)(((g + 1) & 1) * STAGE_BYTES);
    const uint32_t snext = sl_addr + (uint32_t)(sslot_of(j1, s1) + 8 * (s1 & 1));
    {
      uint32_t va[8];
      stage_offsets(la, sd.lda, va);
      if (!more) {
#pragma unroll
        for (int t = 0; t < 8; ++t) va[t] = OOB;
      }
      t4::step_ld(acc, x2, sa2, sb2, next + ra0, next + rb0, x0, m0a, va, ra2, cs2);
    }
    {
      uint32_t vb[8];
      stage_offsets(lb, sd.ldb, vb);
      if (!more) {
#pragma unroll
        for (int t = 0; t < 8; ++t) vb[t] = OOB;
      }
      t4::step_last(acc, x3, sa2, sb2, next + (ra0 ^ 32u), next + (rb0 ^ 32u), snext + s_a, snext + s_b, x1, wa,
                    wb, m0a + OPB, vb, rb2, cs2);
    }
    if (more) advance();
    if (++s1 == nst) {
      s1 = 0;
      ++j1;
    }
    if (++s == nst) {
      t4::drain(acc);
      store(sc.tile(j));
      t4::zero(acc);
      s = 0;
      ++j;
    }
  }
  __syncthreads();
}

}  // namespace t4
}  // namespace mx
