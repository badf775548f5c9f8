// 256x256-tile mainloop of the MXFP4 GEMMs for gfx950 (shared by the dense and
// grouped kernels).
//
// Work split: a workgroup of 8 waves (two per SIMD) owns a 256x256 output
// tile; the waves form a 4 x 2 grid and each owns 2 x 4 tiles of
// V_MFMA_SCALE_F32_32X32X64_F8F6F4 (FP4 x FP4, one E8M0 scale per lane and
// operand, float32 accumulators).  Operand lane layout of that instruction:
// lane l supplies row l % 32 and the 32 K-elements [32*(l/32), 32*(l/32)+32)
// of the 64-deep step (one whole MX block, 16 bytes) with that block's scale
// byte; result register r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column
// l % 32.
//
// Data movement: a stage is 256 K (four 64-deep steps).  Its A and B codes
// (256 rows x 128 bytes each) go global -> LDS with direct-to-LDS buffer loads
// (no VGPR round trip) into a ring of two slots; each load instruction covers
// 8 whole 128-byte row segments, the request size at which this path runs
// fastest.  Scale bytes travel the same way, 16 bytes (16 MX blocks, two
// stages) per row per load, into a ring of two scale slots; scale rows must be
// 16-byte aligned with a stride that is a multiple of 16 bytes.  Each 128-byte
// LDS code row is XOR-swizzled in 16-byte chunks so that the 128-bit LDS
// reads of 16 consecutive rows hit 16 different bank groups.  Raw buffer
// addressing returns zeros past the end of an operand, so rows past M (or N)
// read as zeros and are never stored; in the last, partial stage the missing
// chunks are pointed past the end (zero codes) and their scale bytes are
// cleared to 0 (a finite scale), so they add exact zeros.
//
// Software pipeline inside a wave: the operands of the next step are read from
// LDS into a second register set while the 8 MFMAs of the current step run,
// so the LDS latency is hidden behind matrix work.  Each step is one asm block
// that issues its MFMAs with the next step's LDS reads interleaved and waits
// for those reads at its end.  (The compiler can neither be told that these
// reads do not touch the ring slot the direct-to-LDS loads are filling, which
// would make it wait for every load in flight, nor be made to keep the
// interleaving.)  The hazards it would otherwise cover are handled here: two
// wait states between a VALU write of an operand and the MFMA that reads it
// (an s_nop at the start of each block) and wait states between the last MFMA
// and the first read of its result (after the loop).  One barrier per stage,
// before its last step: every wave has then read the stage's codes, so its
// slot is refilled with the stage two ahead: its 8 code loads per wave go
// out one per MFMA of the last step, or (SPLIT, used by the dense and grouped
// kernels) the A half there and the B half in the next stage's first step, so
// that the load unit never receives a whole stage's loads at once.
//
// Persistent schedule: one workgroup per CU walks its list of tiles, and the
// stage sequence runs on across tile boundaries: the first two stages of the
// next tile are loaded while the last stage of the current one is multiplied
// and its result stored, so neither the pipeline fill nor the epilogue leaves
// the load path idle.
//
// The file is included twice, with MX_T256_NS naming the namespace and
// MX_T256_SWAP choosing the MFMA operand order: 0 multiplies A-row x B-row
// (lane = output column, registers = output rows: the layout of the float32 /
// bf16 stores), 1 issues every MFMA with the operands and their scales
// swapped, so that each lane holds 16 columns of one output row (the layout
// of the quantizing epilogue, which then finds a block's 32 values in two
// lanes).
#if !defined(MX_T256_NS) || !defined(MX_T256_SWAP)
#error "define MX_T256_NS and MX_T256_SWAP before including gemm_tile256.h"
#endif

#include "mx_device.h"
#include "mx_launch.h"

#ifndef MX_T256_SHARED_TYPES
#define MX_T256_SHARED_TYPES
namespace mx {
namespace t256c {
// One 256x256 output tile: A rows [m0, m0+256) (valid below M) of the
// operand at a_codes/a_scales, B rows [n0, n0+256) (valid below N), and the
// output row of its first row.  All fields are wave-uniform.
struct TileInfo {
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const uint8_t* b_codes;
  const uint8_t* b_scales;
  int m0, n0, M, N;
  int64_t c_row0;
  // Schedules that split K (Sched::UNITS) hand out units = a range of stages
  // [k0, k0 + ns) of one tile, k0 even; the others always run whole tiles.
  int k0, ns;
};

// Row strides (bytes) shared by all tiles of a launch.
struct Strides {
  int lda, ldsa, ldb, ldsb;
};

// Tile order: groups of GM M-tiles, each walked N-tile by N-tile, so that a
// run of consecutive tiles shares a few A and B panels.
template <int GM>
__device__ __forceinline__ void group_order(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int group = t / (GM * tiles_n);
  const int first_m = group * GM;
  const int gm = (tiles_m - first_m) < GM ? (tiles_m - first_m) : GM;
  const int in = t - group * GM * tiles_n;
  tm = first_m + in % gm;
  tn = in / gm;
}

// Destination of the quantizing epilogue: the float32 tile quantized along N
// into MXFP4 blocks of 32 (RNE), codes [M, N/2] and scale bytes [M, N/32]
// with these row strides; scale_mode as in mx_quantize.
struct QOut {
  uint8_t* codes;
  uint8_t* scales;
  int ld_codes, ld_scales, scale_mode;
};
}  // namespace t256c
}  // namespace mx
#endif

namespace mx {
namespace MX_T256_NS {

using t256c::QOut;
using t256c::Strides;
using t256c::TileInfo;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int WAVES = 8;                   // 4 along M x 2 along N
constexpr int TM = 256, TN = 256;
constexpr int TK = 256;                    // K elements per stage
constexpr int ROWB = TK / 2;               // code bytes per row per stage (128)
constexpr int OPB = 256 * ROWB;            // code bytes per operand per stage (32 KiB)
constexpr int STAGE_BYTES = 2 * OPB;       // one code slot
constexpr int SROWB = 16;                  // scale bytes per row per scale slot (two stages)
constexpr int SSLOT = 2 * 256 * SROWB;     // one scale slot: A rows, then B rows (8 KiB)
constexpr int DUMMY_BYTES = 4096;          // target of loads that must not land in a live slot
constexpr int LDS_BYTES = 2 * STAGE_BYTES + 2 * SSLOT + DUMMY_BYTES;
constexpr int TI = 2, TJ = 4;              // 32x32 MFMA tiles per wave along M, N
constexpr int CODE_LOADS = 8;              // 1 KiB code loads per wave and stage (4 A + 4 B)

// 16-byte chunk swizzle inside a 128-byte LDS row: chunk c of row r sits at
// c ^ ((r >> 1) & 7).  Rows r and r+1 are 128 bytes apart, so 16 consecutive
// rows reading one logical chunk land in 16 distinct 16-byte bank groups of
// the 256-byte bank window.
__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

// Raw buffer resource over [base, base + bytes): loads past the end return 0
// and stores past the end are dropped (gfx9 raw buffer addressing).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
constexpr uint32_t OOB = 0x80000000u;        // an offset past any operand (validated < 2 GiB)

// Per-lane global offsets of this wave's 8 code loads of a tile (stage 0):
// load t of each operand covers rows 8*(4*wave+t) .. +8, lane l the swizzled
// chunk of row l/8 (load_chunk: its K-block within the stage); rows past the
// limits point past the end (zeros).
__device__ __forceinline__ int load_chunk(int wave, int lane, int t) {
  return swz(8 * (wave * 4 + t) + (lane >> 3), lane & 7);
}

__device__ __forceinline__ void code_offsets(const TileInfo& ti, const Strides& sd, int wave, int lane, uint32_t va[4],
                                             uint32_t vb[4]) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int row = 8 * (wave * 4 + t) + (lane >> 3);
    const int c = load_chunk(wave, lane, t);
    va[t] = (ti.m0 + row < ti.M) ? (uint32_t)(ti.m0 + row) * (uint32_t)sd.lda + 16u * c : OOB;
    vb[t] = (ti.n0 + row < ti.N) ? (uint32_t)(ti.n0 + row) * (uint32_t)sd.ldb + 16u * c : OOB;
  }
}

// This lane's scale-row offset for the scale loads of a tile (A rows for
// waves 0-3, B rows for 4-7), past the end for rows past the limits.
template <bool A2D, bool B2D>
__device__ __forceinline__ uint32_t scale_offset(const TileInfo& ti, const Strides& sd, int wave, int lane) {
  const int r = 64 * (wave & 3) + lane;
  if (wave < 4) {
    const int ra = ti.m0 + r;
    return ra < ti.M ? (uint32_t)(A2D ? (ra >> 5) : ra) * (uint32_t)sd.ldsa : OOB;
  }
  const int rb = ti.n0 + r;
  return rb < ti.N ? (uint32_t)(B2D ? (rb >> 5) : rb) * (uint32_t)sd.ldsb : OOB;
}

template <bool A2D, bool B2D>
__device__ __forceinline__ void tile_rsrc(const TileInfo& ti, const Strides& sd, int wave, __amdgpu_buffer_rsrc_t& ra,
                                          __amdgpu_buffer_rsrc_t& rb, __amdgpu_buffer_rsrc_t& rs) {
  ra = rsrc(ti.a_codes, (uint32_t)(ti.M * sd.lda));
  rb = rsrc(ti.b_codes, (uint32_t)(ti.N * sd.ldb));
  rs = wave < 4 ? rsrc(ti.a_scales, (uint32_t)((A2D ? ti.M / 32 : ti.M) * sd.ldsa))
                : rsrc(ti.b_scales, (uint32_t)((B2D ? ti.N / 32 : ti.N) * sd.ldsb));
}

// Issue the scale loads of stages 2q and 2q+1 of a tile into `sslot`: 16
// bytes per row at this lane's row offset `off`, 64 rows per wave (A rows for
// waves 0-3, B rows for 4-7).
__device__ __forceinline__ void issue_scales(__amdgpu_buffer_rsrc_t rs, uint32_t off, int q, uint8_t* sslot,
                                             int wave) {
  uint8_t* dst = sslot + (wave < 4 ? 0 : 256 * SROWB) + 64 * SROWB * (wave & 3);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)dst, 16, off, (uint32_t)q * SROWB, 0, 0);
}

// Issue the 8 code loads of one stage with the compiler's load builtin (used
// before the pipeline runs; inside it the loads sit in the last step's asm).
__device__ __forceinline__ void issue_codes(__amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb, const uint32_t va[4],
                                            const uint32_t vb[4], uint32_t cs, uint8_t* slot, int wave) {
#pragma unroll
  for (int t = 0; t < 4; ++t)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)(slot + 1024 * (wave * 4 + t)), 16, va[t], cs, 0, 0);
#pragma unroll
  for (int t = 0; t < 4; ++t)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)(slot + OPB + 1024 * (wave * 4 + t)), 16, vb[t], cs, 0,
                                             0);
}

struct Acc {
  v16f t[TI][TJ];
};

// ------------------------------------------------------------ asm K steps
// Row tiles of one operand are 32 x 128 = 4096 code bytes and 32 x 16 = 512
// scale bytes apart in a slot.  Each lane's 32-bit scale word holds the bytes
// of 4 consecutive K-blocks, already shifted right by 8 * (l / 32); op_sel_hi
// [0,0,0] then picks the lane's block of an even step, [1,1,0] of an odd step.
#define MX_OPSEL_LO "0,0,0"
#define MX_OPSEL_HI "1,1,0"
#if MX_T256_SWAP
#define MX_MFMA(C, A, B, SA, SB, OPSEL)                                                                    \
  "v_mfma_scale_f32_32x32x64_f8f6f4 %[" #C "], %[" #B "], %[" #A "], %[" #C "], %[" #SB "], %[" #SA \
  "] op_sel_hi:[" OPSEL "] cbsz:4 blgp:4\n\t"
#else
#define MX_MFMA(C, A, B, SA, SB, OPSEL)                                                                    \
  "v_mfma_scale_f32_32x32x64_f8f6f4 %[" #C "], %[" #A "], %[" #B "], %[" #C "], %[" #SA "], %[" #SB \
  "] op_sel_hi:[" OPSEL "] cbsz:4 blgp:4\n\t"
#endif
#define MX_ACC_OPERANDS(c)                                                                                 \
  [c00] "+v"(c.t[0][0]), [c01] "+v"(c.t[0][1]), [c02] "+v"(c.t[0][2]), [c03] "+v"(c.t[0][3]),           \
      [c10] "+v"(c.t[1][0]), [c11] "+v"(c.t[1][1]), [c12] "+v"(c.t[1][2]), [c13] "+v"(c.t[1][3])
#define MX_NEXT_OPERANDS                                                                                   \
  [na0] "=&v"(na[0]), [na1] "=&v"(na[1]), [nb0] "=&v"(nb[0]), [nb1] "=&v"(nb[1]), [nb2] "=&v"(nb[2]),    \
      [nb3] "=&v"(nb[3])
#define MX_CUR_OPERANDS                                                                                    \
  [a0] "v"(a[0]), [a1] "v"(a[1]), [b0] "v"(b[0]), [b1] "v"(b[1]), [b2] "v"(b[2]), [b3] "v"(b[3]),         \
      [sa0] "v"(sa[0]), [sa1] "v"(sa[1]), [sb0] "v"(sb[0]), [sb1] "v"(sb[1]), [sb2] "v"(sb[2]),           \
      [sb3] "v"(sb[3])
// 8 MFMAs of one step with the 6 operand reads of the next one interleaved.
#define MX_STEP_BODY(OPSEL)                                   \
  "s_nop 1\n\t"                                              \
  MX_MFMA(c00, a0, b0, sa0, sb0, OPSEL)                       \
  "ds_read_b128 %[na0], %[ada]\n\t"                          \
  "ds_read_b128 %[na1], %[ada] offset:4096\n\t"              \
  MX_MFMA(c01, a0, b1, sa0, sb1, OPSEL)                       \
  "ds_read_b128 %[nb0], %[adb]\n\t"                          \
  "ds_read_b128 %[nb1], %[adb] offset:4096\n\t"              \
  MX_MFMA(c02, a0, b2, sa0, sb2, OPSEL)                       \
  "ds_read_b128 %[nb2], %[adb] offset:8192\n\t"              \
  "ds_read_b128 %[nb3], %[adb] offset:12288\n\t"             \
  MX_MFMA(c03, a0, b3, sa0, sb3, OPSEL)

// One step on operands a, b; reads the next step's operands (LDS byte
// addresses ada, adb of its row tile 0) into na, nb.
template <bool ODD>
__device__ __forceinline__ void step(Acc& c, const v4i a[TI], const v4i b[TJ], const int sa[TI],
                                     const int sb[TJ], uint32_t ada, uint32_t adb, v4i na[TI], v4i nb[TJ]) {
  if constexpr (!ODD) {
    asm volatile(MX_STEP_BODY(MX_OPSEL_LO)
                 MX_MFMA(c10, a1, b0, sa1, sb0, MX_OPSEL_LO)
                 MX_MFMA(c11, a1, b1, sa1, sb1, MX_OPSEL_LO)
                 MX_MFMA(c12, a1, b2, sa1, sb2, MX_OPSEL_LO)
                 MX_MFMA(c13, a1, b3, sa1, sb3, MX_OPSEL_LO)
                 "s_waitcnt lgkmcnt(0)"
                 : MX_ACC_OPERANDS(c), MX_NEXT_OPERANDS
                 : MX_CUR_OPERANDS, [ada] "v"(ada), [adb] "v"(adb)
                 : "memory");
  } else {
    asm volatile(MX_STEP_BODY(MX_OPSEL_HI)
                 MX_MFMA(c10, a1, b0, sa1, sb0, MX_OPSEL_HI)
                 MX_MFMA(c11, a1, b1, sa1, sb1, MX_OPSEL_HI)
                 MX_MFMA(c12, a1, b2, sa1, sb2, MX_OPSEL_HI)
                 MX_MFMA(c13, a1, b3, sa1, sb3, MX_OPSEL_HI)
                 "s_waitcnt lgkmcnt(0)"
                 : MX_ACC_OPERANDS(c), MX_NEXT_OPERANDS
                 : MX_CUR_OPERANDS, [ada] "v"(ada), [adb] "v"(adb)
                 : "memory");
  }
}

// The first step of a stage with 4 code loads interleaved: the B half of the
// loads of the stage two ahead (issued one step after its A half, so that a
// stage's loads are spread over two steps), to LDS addresses m0, m0+1024, ...
// at per-lane offsets v plus the stage offset cs through resource rc.
__device__ __forceinline__ void step0_ld(Acc& c, const v4i a[TI], const v4i b[TJ], const int sa[TI],
                                         const int sb[TJ], uint32_t ada, uint32_t adb, v4i na[TI], v4i nb[TJ],
                                         uint32_t m0, const uint32_t v[4], __amdgpu_buffer_rsrc_t rc, uint32_t cs) {
  asm volatile(MX_STEP_BODY(MX_OPSEL_LO)
               "buffer_load_dwordx4 %[v0], %[rc], %[cs] offen lds\n\t"
               "s_add_u32 m0, m0, 0x400\n\t"
               MX_MFMA(c10, a1, b0, sa1, sb0, MX_OPSEL_LO)
               "buffer_load_dwordx4 %[v1], %[rc], %[cs] offen lds\n\t"
               "s_add_u32 m0, m0, 0x400\n\t"
               MX_MFMA(c11, a1, b1, sa1, sb1, MX_OPSEL_LO)
               "buffer_load_dwordx4 %[v2], %[rc], %[cs] offen lds\n\t"
               "s_add_u32 m0, m0, 0x400\n\t"
               MX_MFMA(c12, a1, b2, sa1, sb2, MX_OPSEL_LO)
               "buffer_load_dwordx4 %[v3], %[rc], %[cs] offen lds\n\t"
               MX_MFMA(c13, a1, b3, sa1, sb3, MX_OPSEL_LO)
               "s_waitcnt lgkmcnt(0)"
               : MX_ACC_OPERANDS(c), MX_NEXT_OPERANDS, [m0] "+{m0}"(m0)
               : MX_CUR_OPERANDS, [ada] "v"(ada), [adb] "v"(adb), [v0] "v"(v[0]), [v1] "v"(v[1]), [v2] "v"(v[2]),
                 [v3] "v"(v[3]), [rc] "s"(rc), [cs] "s"(cs)
               : "memory");
}

// The last (odd) step of a stage; reads the next stage's first-step operands
// (ada, adb) and its 8 scale bytes per row tile (adsa, adsb) into wa, wb, and
// issues this wave's 4 A code loads of the stage two ahead, one after every
// other MFMA, to LDS addresses m0, m0+1024, m0+2048, m0+3072 at per-lane
// offsets va plus the stage offset cs (the B half follows in the next step).
__device__ __forceinline__ void step_last(Acc& c, const v4i a[TI], const v4i b[TJ], const int sa[TI],
                                          const int sb[TJ], uint32_t ada, uint32_t adb, uint32_t adsa,
                                          uint32_t adsb, v4i na[TI], v4i nb[TJ], v2u wa[TI], v2u wb[TJ],
                                          uint32_t m0, const uint32_t va[4], __amdgpu_buffer_rsrc_t ra, uint32_t cs) {
  asm volatile(
      "s_nop 1\n\t"
      MX_MFMA(c00, a0, b0, sa0, sb0, MX_OPSEL_HI)
      "ds_read_b128 %[na0], %[ada]\n\t"
      "ds_read_b128 %[na1], %[ada] offset:4096\n\t"
      "buffer_load_dwordx4 %[va0], %[ra], %[cs] offen lds\n\t"
      "s_add_u32 m0, m0, 0x400\n\t"
      MX_MFMA(c01, a0, b1, sa0, sb1, MX_OPSEL_HI)
      "ds_read_b128 %[nb0], %[adb]\n\t"
      "ds_read_b128 %[nb1], %[adb] offset:4096\n\t"
      MX_MFMA(c02, a0, b2, sa0, sb2, MX_OPSEL_HI)
      "ds_read_b128 %[nb2], %[adb] offset:8192\n\t"
      "ds_read_b128 %[nb3], %[adb] offset:12288\n\t"
      "buffer_load_dwordx4 %[va1], %[ra], %[cs] offen lds\n\t"
      "s_add_u32 m0, m0, 0x400\n\t"
      MX_MFMA(c03, a0, b3, sa0, sb3, MX_OPSEL_HI)
      "ds_read_b64 %[wa0], %[adsa]\n\t"
      "ds_read_b64 %[wa1], %[adsa] offset:512\n\t"
      MX_MFMA(c10, a1, b0, sa1, sb0, MX_OPSEL_HI)
      "ds_read_b64 %[wb0], %[adsb]\n\t"
      "ds_read_b64 %[wb1], %[adsb] offset:512\n\t"
      "buffer_load_dwordx4 %[va2], %[ra], %[cs] offen lds\n\t"
      "s_add_u32 m0, m0, 0x400\n\t"
      MX_MFMA(c11, a1, b1, sa1, sb1, MX_OPSEL_HI)
      "ds_read_b64 %[wb2], %[adsb] offset:1024\n\t"
      "ds_read_b64 %[wb3], %[adsb] offset:1536\n\t"
      MX_MFMA(c12, a1, b2, sa1, sb2, MX_OPSEL_HI)
      "buffer_load_dwordx4 %[va3], %[ra], %[cs] offen lds\n\t"
      MX_MFMA(c13, a1, b3, sa1, sb3, MX_OPSEL_HI)
      "s_waitcnt lgkmcnt(0)"
      : MX_ACC_OPERANDS(c), MX_NEXT_OPERANDS, [wa0] "=&v"(wa[0]), [wa1] "=&v"(wa[1]),
        [wb0] "=&v"(wb[0]), [wb1] "=&v"(wb[1]), [wb2] "=&v"(wb[2]), [wb3] "=&v"(wb[3]), [m0] "+{m0}"(m0)
      : MX_CUR_OPERANDS, [ada] "v"(ada), [adb] "v"(adb), [adsa] "v"(adsa), [adsb] "v"(adsb),
        [va0] "v"(va[0]), [va1] "v"(va[1]), [va2] "v"(va[2]), [va3] "v"(va[3]), [ra] "s"(ra), [cs] "s"(cs)
      : "memory");
}

// step_last without its MFMAs, for a tail stage whose fourth 64-deep step
// lies past K: the same loads of the stage two ahead and reads of the next
// stage's first operands and scale bytes.
__device__ __forceinline__ void step_last_nm(uint32_t ada, uint32_t adb, uint32_t adsa, uint32_t adsb, v4i na[TI],
                                             v4i nb[TJ], v2u wa[TI], v2u wb[TJ], uint32_t m0, const uint32_t va[4],
                                             __amdgpu_buffer_rsrc_t ra, uint32_t cs) {
  asm volatile(
      "ds_read_b128 %[na0], %[ada]\n\t"
      "ds_read_b128 %[na1], %[ada] offset:4096\n\t"
      "buffer_load_dwordx4 %[va0], %[ra], %[cs] offen lds\n\t"
      "s_add_u32 m0, m0, 0x400\n\t"
      "ds_read_b128 %[nb0], %[adb]\n\t"
      "ds_read_b128 %[nb1], %[adb] offset:4096\n\t"
      "ds_read_b128 %[nb2], %[adb] offset:8192\n\t"
      "ds_read_b128 %[nb3], %[adb] offset:12288\n\t"
      "buffer_load_dwordx4 %[va1], %[ra], %[cs] offen lds\n\t"
      "s_add_u32 m0, m0, 0x400\n\t"
      "ds_read_b64 %[wa0], %[adsa]\n\t"
      "ds_read_b64 %[wa1], %[adsa] offset:512\n\t"
      "ds_read_b64 %[wb0], %[adsb]\n\t"
      "ds_read_b64 %[wb1], %[adsb] offset:512\n\t"
      "buffer_load_dwordx4 %[va2], %[ra], %[cs] offen lds\n\t"
      "s_add_u32 m0, m0, 0x400\n\t"
      "ds_read_b64 %[wb2], %[adsb] offset:1024\n\t"
      "ds_read_b64 %[wb3], %[adsb] offset:1536\n\t"
      "buffer_load_dwordx4 %[va3], %[ra], %[cs] offen lds\n\t"
      "s_waitcnt lgkmcnt(0)"
      : MX_NEXT_OPERANDS, [wa0] "=&v"(wa[0]), [wa1] "=&v"(wa[1]), [wb0] "=&v"(wb[0]), [wb1] "=&v"(wb[1]),
        [wb2] "=&v"(wb[2]), [wb3] "=&v"(wb[3]), [m0] "+{m0}"(m0)
      : [ada] "v"(ada), [adb] "v"(adb), [adsa] "v"(adsa), [adsb] "v"(adsb), [va0] "v"(va[0]), [va1] "v"(va[1]),
        [va2] "v"(va[2]), [va3] "v"(va[3]), [ra] "s"(ra), [cs] "s"(cs)
      : "memory");
}

// As step_last, but issuing all 8 code loads of the stage two ahead (4 A
// loads at m0, m0+1024, ..., then 4 B loads OPB further), one after each MFMA.
__device__ __forceinline__ void step_last8(Acc& c, const v4i a[TI], const v4i b[TJ], const int sa[TI],
                                           const int sb[TJ], uint32_t ada, uint32_t adb, uint32_t adsa,
                                           uint32_t adsb, v4i na[TI], v4i nb[TJ], v2u wa[TI], v2u wb[TJ],
                                           uint32_t m0, const uint32_t va[4], const uint32_t vb[4],
                                           __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb, uint32_t cs) {
  static_assert(OPB - 3072 == 0x7400, "B loads start OPB after the A loads");
  asm volatile(
      "s_nop 1\n\t"
      MX_MFMA(c00, a0, b0, sa0, sb0, MX_OPSEL_HI)
      "ds_read_b128 %[na0], %[ada]\n\t"
      "ds_read_b128 %[na1], %[ada] offset:4096\n\t"
      "buffer_load_dwordx4 %[va0], %[ra], %[cs] offen lds\n\t"
      "s_add_u32 m0, m0, 0x400\n\t"
      MX_MFMA(c01, a0, b1, sa0, sb1, MX_OPSEL_HI)
      "ds_read_b128 %[nb0], %[adb]\n\t"
      "ds_read_b128 %[nb1], %[adb] offset:4096\n\t"
      "buffer_load_dwordx4 %[va1], %[ra], %[cs] offen lds\n\t"
      "s_add_u32 m0, m0, 0x400\n\t"
      MX_MFMA(c02, a0, b2, sa0, sb2, MX_OPSEL_HI)
      "ds_read_b128 %[nb2], %[adb] offset:8192\n\t"
      "ds_read_b128 %[nb3], %[adb] offset:12288\n\t"
      "buffer_load_dwordx4 %[va2], %[ra], %[cs] offen lds\n\t"
      "s_add_u32 m0, m0, 0x400\n\t"
      MX_MFMA(c03, a0, b3, sa0, sb3, MX_OPSEL_HI)
      "ds_read_b64 %[wa0], %[adsa]\n\t"
      "ds_read_b64 %[wa1], %[adsa] offset:512\n\t"
      "buffer_load_dwordx4 %[va3], %[ra], %[cs] offen lds\n\t"
      "s_add_u32 m0, m0, 0x7400\n\t"
      MX_MFMA(c10, a1, b0, sa1, sb0, MX_OPSEL_HI)
      "ds_read_b64 %[wb0], %[adsb]\n\t"
      "ds_read_b64 %[wb1], %[adsb] offset:512\n\t"
      "buffer_load_dwordx4 %[vb0], %[rb], %[cs] offen lds\n\t"
      "s_add_u32 m0, m0, 0x400\n\t"
      MX_MFMA(c11, a1, b1, sa1, sb1, MX_OPSEL_HI)
      "ds_read_b64 %[wb2], %[adsb] offset:1024\n\t"
      "ds_read_b64 %[wb3], %[adsb] offset:1536\n\t"
      "buffer_load_dwordx4 %[vb1], %[rb], %[cs] offen lds\n\t"
      "s_add_u32 m0, m0, 0x400\n\t"
      MX_MFMA(c12, a1, b2, sa1, sb2, MX_OPSEL_HI)
      "buffer_load_dwordx4 %[vb2], %[rb], %[cs] offen lds\n\t"
      "s_add_u32 m0, m0, 0x400\n\t"
      MX_MFMA(c13, a1, b3, sa1, sb3, MX_OPSEL_HI)
      "buffer_load_dwordx4 %[vb3], %[rb], %[cs] offen lds\n\t"
      "s_waitcnt lgkmcnt(0)"
      : MX_ACC_OPERANDS(c), MX_NEXT_OPERANDS, [wa0] "=&v"(wa[0]), [wa1] "=&v"(wa[1]),
        [wb0] "=&v"(wb[0]), [wb1] "=&v"(wb[1]), [wb2] "=&v"(wb[2]), [wb3] "=&v"(wb[3]), [m0] "+{m0}"(m0)
      : MX_CUR_OPERANDS, [ada] "v"(ada), [adb] "v"(adb), [adsa] "v"(adsa), [adsb] "v"(adsb),
        [va0] "v"(va[0]), [va1] "v"(va[1]), [va2] "v"(va[2]), [va3] "v"(va[3]), [vb0] "v"(vb[0]),
        [vb1] "v"(vb[1]), [vb2] "v"(vb[2]), [vb3] "v"(vb[3]), [ra] "s"(ra), [rb] "s"(rb), [cs] "s"(cs)
      : "memory");
}

// The first stage's first-step operands and scale bytes.
__device__ __forceinline__ void read_first(uint32_t ada, uint32_t adb, uint32_t adsa, uint32_t adsb,
                                           v4i a[TI], v4i b[TJ], v2u wa[TI], v2u wb[TJ]) {
  asm volatile(
      "ds_read_b128 %[a0], %[ada]\n\t"
      "ds_read_b128 %[a1], %[ada] offset:4096\n\t"
      "ds_read_b128 %[b0], %[adb]\n\t"
      "ds_read_b128 %[b1], %[adb] offset:4096\n\t"
      "ds_read_b128 %[b2], %[adb] offset:8192\n\t"
      "ds_read_b128 %[b3], %[adb] offset:12288\n\t"
      "ds_read_b64 %[wa0], %[adsa]\n\t"
      "ds_read_b64 %[wa1], %[adsa] offset:512\n\t"
      "ds_read_b64 %[wb0], %[adsb]\n\t"
      "ds_read_b64 %[wb1], %[adsb] offset:512\n\t"
      "ds_read_b64 %[wb2], %[adsb] offset:1024\n\t"
      "ds_read_b64 %[wb3], %[adsb] offset:1536\n\t"
      "s_waitcnt lgkmcnt(0)"
      : [a0] "=&v"(a[0]), [a1] "=&v"(a[1]), [b0] "=&v"(b[0]), [b1] "=&v"(b[1]), [b2] "=&v"(b[2]),
        [b3] "=&v"(b[3]), [wa0] "=&v"(wa[0]), [wa1] "=&v"(wa[1]), [wb0] "=&v"(wb[0]), [wb1] "=&v"(wb[1]),
        [wb2] "=&v"(wb[2]), [wb3] "=&v"(wb[3])
      : [ada] "v"(ada), [adb] "v"(adb), [adsa] "v"(adsa), [adsb] "v"(adsb)
      : "memory");
}

// Wait states between the last MFMA and any later instruction that reads or
// writes the accumulators (more than the 16-pass requirement).
__device__ __forceinline__ void drain(Acc& c) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : MX_ACC_OPERANDS(c));
}

#undef MX_STEP_BODY
#undef MX_CUR_OPERANDS
#undef MX_NEXT_OPERANDS
#undef MX_ACC_OPERANDS
#undef MX_MFMA
#undef MX_OPSEL_LO
#undef MX_OPSEL_HI

// Wait until at most n of this wave's vector-memory loads are outstanding
// (n = 0, the code loads of one stage, or those plus one scale load).
__device__ __forceinline__ void wait_vmcnt(int n) {
  // s_waitcnt encoding (gfx9): vmcnt bits [3:0] and [15:14]; expcnt and
  // lgkmcnt left at their maxima (no wait).
#define MX_VMCNT(N_) (((N_) & 0xF) | (((N_) >> 4) << 14) | (0x7 << 4) | (0xF << 8))
  if (n >= CODE_LOADS + 1) __builtin_amdgcn_s_waitcnt(MX_VMCNT(CODE_LOADS + 1));
  else if (n >= CODE_LOADS) __builtin_amdgcn_s_waitcnt(MX_VMCNT(CODE_LOADS));
  else __builtin_amdgcn_s_waitcnt(MX_VMCNT(0));
#undef MX_VMCNT
}

// Workgroup barrier without the fence of __syncthreads() (which would wait for
// every load in flight).  The empty asm statements keep the compiler from
// moving memory operations across it.
__device__ __forceinline__ void bare_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ void zero(Acc& acc) {
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc.t[i][j][r] = 0.0f;
}

template <bool OUT_BF16>
__device__ __forceinline__ void store_tile(const Acc& acc, void* C, int ldc, int mlim, int nlim);

template <bool OUT_BF16, class Sched>
__device__ __forceinline__ void store_unit(Acc& acc, const Sched& sc, int j, void* C, int64_t ldc);

// Output kinds of run_tiles: float32, bf16, or the quantizing epilogue
// (MX_T256_SWAP = 1 only).
constexpr int OUT_F32 = 0, OUT_BF16_ = 1, OUT_MX = 2;

__device__ __forceinline__ void store_tile_mx(const Acc& acc, const QOut& q, int m0, int n0, int mlim, int nlim);

// Run this workgroup's tiles: C tile = A[m0:m0+256] * B[n0:n0+256]^T over all
// K for each tile sc.tile(j), j < sc.count().  The stage sequence g = j * nst
// + s (s < nst stages of tile j) is pipelined across tiles: code slot g & 1,
// scale slot P & 1 for the scale pair P = j * npairs + s / 2.  Operand rows
// past the limits read as zeros and are never stored.  Byte extents of the
// operands must be < 2 GiB.  `lds` holds LDS_BYTES: the two code slots, the
// two scale slots and a dummy region.
//
// With Sched::UNITS the schedule hands out units instead of whole tiles: unit
// j covers stages [k0, k0 + ns) of its tile, k0 and ns even (a tile with an
// odd stage count gets one more stage, past K, whose codes read as zeros and
// whose scale bytes are masked to 0, adding exact zeros).  The stage sequence
// runs through the units back to back; with every unit an even number of
// stages, global stage g uses scale pair g / 2.  Each unit ends in
// store_unit (the split-K epilogue) instead of a plain store.
template <bool A2D, bool B2D, int OUT, bool SPLIT, class Sched>
__device__ __forceinline__ void run_tiles(const Sched& sc, const Strides& sd, int K, void* C, int64_t ldc,
                                          uint8_t* lds, const QOut& qo = QOut{}) {
  static_assert((OUT == OUT_MX) == (MX_T256_SWAP != 0), "the quantizing epilogue needs the swapped operand order");
  constexpr bool UNITS = Sched::UNITS;
  static_assert(!UNITS || OUT != OUT_MX, "units end in the split-K epilogue, which stores float32 or bf16");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int ntiles = sc.count();
  if (ntiles <= 0) return;
  Acc acc;
  zero(acc);
  constexpr int ES = OUT == OUT_BF16_ ? 2 : 4;
  auto store = [&](const TileInfo& ti) {
    if constexpr (OUT == OUT_MX)
      store_tile_mx(acc, qo, (int)ti.c_row0, ti.n0, ti.M - ti.m0, ti.N - ti.n0);
    else
      store_tile<OUT == OUT_BF16_>(acc, static_cast<uint8_t*>(C) + (ti.c_row0 * ldc + ti.n0) * ES, (int)ldc,
                                   ti.M - ti.m0, ti.N - ti.n0);
  };
  const int nst = (K + TK - 1) / TK;
  if (nst == 0) {                           // K = 0: every tile is zero
    for (int j = 0; j < ntiles; ++j) store(sc.tile(j));
    return;
  }
  const int nfull = K / TK;                 // stages without a K tail
  const int kchunks = (K - nfull * TK) / 32;          // K-blocks in the tail stage (0 if none)
  const int npairs = (nst + 1) / 2;
  int gtotal;
  if constexpr (UNITS) gtotal = sc.total_stages();
  else gtotal = ntiles * nst;
  // scale bytes of the tail stage's blocks: low word blocks 0-3, high word 4-7
  const uint32_t tail_lo = kchunks >= 4 ? 0xFFFFFFFFu : (1u << (8 * kchunks)) - 1u;
  const uint32_t tail_hi = kchunks <= 4 ? 0u : (1u << (8 * (kchunks - 4))) - 1u;
  uint8_t* const sslots = lds + 2 * STAGE_BYTES;
  const uint32_t lds_addr = (uint32_t)(uintptr_t)(lds_ptr_t)lds;   // LDS byte address of code slot 0
  const uint32_t sl_addr = lds_addr + 2 * STAGE_BYTES;             // ... of scale slot 0

  // This lane's LDS read offsets inside a slot (the chunk swizzle depends on
  // bits 1..3 of the row only, equal for all row tiles of the wave).
  const int l32 = lane & 31, kh = lane >> 5;
  const int rowa = wm * TI * 32 + l32, rowb = wn * TJ * 32 + l32;
  uint32_t ra_k[4], rb_k[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    ra_k[ks] = rowa * ROWB + 16 * swz(rowa, 2 * ks + kh);
    rb_k[ks] = OPB + rowb * ROWB + 16 * swz(rowb, 2 * ks + kh);
  }
  const uint32_t s_a = rowa * SROWB, s_b = 256 * SROWB + rowb * SROWB;
  const int sh = 8 * kh;

  // The stage whose loads are issued next ("prefetch" position j2, s2) and
  // its tile's load state, refreshed once per tile.  For units, kb2 is the
  // first stage of unit j2 within its tile and ns2 its stage count.
  int j2 = 0, s2 = 0;
  TileInfo t2 = sc.tile(0);
  int kb2 = 0, ns2 = nst;
  if constexpr (UNITS) {
    kb2 = t2.k0;
    ns2 = t2.ns;
  }
  __amdgpu_buffer_rsrc_t ra2, rb2, rs2;
  uint32_t pa[4], pb[4], psc;
  auto load_tile = [&]() {
    tile_rsrc<A2D, B2D>(t2, sd, wave, ra2, rb2, rs2);
    code_offsets(t2, sd, wave, lane, pa, pb);
    psc = scale_offset<A2D, B2D>(t2, sd, wave, lane);
  };
  auto advance = [&]() {
    if (++s2 == ns2) {
      s2 = 0;
      if (++j2 < ntiles) {
        t2 = sc.tile(j2);
        if constexpr (UNITS) {
          kb2 = t2.k0;
          ns2 = t2.ns;
        }
        load_tile();
      }
    }
  };
  // Code offsets of the prefetch stage (the tail stage masks the chunks past
  // K; a unit's padding stage past the tail masks all of them).
  auto stage_offsets = [&](uint32_t va[4], uint32_t vb[4]) {
    const int k = (kb2 + s2);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      bool live;
      if constexpr (UNITS) live = k < nfull || (k == nfull && load_chunk(wave, lane, t) < kchunks);
      else live = k < nfull || load_chunk(wave, lane, t) < kchunks;
      va[t] = live ? pa[t] : OOB;
      vb[t] = live ? pb[t] : OOB;
    }
  };
  // scale slot of global stage gs at prefetch position (j2, s2)
  auto sslot2 = [&](int gs) {
    if constexpr (UNITS) return ((gs >> 1) & 1) * SSLOT;
    else return ((j2 * npairs + (s2 >> 1)) & 1) * SSLOT;
  };
  load_tile();

  // Prologue: global stages 0 and 1 with the compiler's load builtins.
  int loads1 = 0;                           // loads of stage 1
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    if (g >= gtotal) break;
    if (!(s2 & 1)) issue_scales(rs2, psc, (kb2 + s2) >> 1, sslots + sslot2(g), wave);
    uint32_t va[4], vb[4];
    stage_offsets(va, vb);
    issue_codes(ra2, rb2, va, vb, (uint32_t)(kb2 + s2) * ROWB, lds + (g & 1) * STAGE_BYTES, wave);
    if (g == 1) loads1 = CODE_LOADS + ((s2 & 1) ? 0 : 1);
    advance();
  }
  wait_vmcnt(loads1);                       // this wave's stage-0 loads landed
  bare_barrier();                           // ... and every wave's
  v4i a[TI], b[TJ], na[TI], nb[TJ];
  v2u wa[TI], wb[TJ];
  read_first(lds_addr + ra_k[0], lds_addr + rb_k[0], sl_addr + s_a, sl_addr + s_b, a, b, wa, wb);

  int s = 0, j = 0;                         // stage s of tile j is multiplied
  int kb = 0, ns = nst;                     // (units: first stage and stage count of unit j)
  int s1 = 1 % nst, j1 = 1 / nst;           // the stage after it (whole tiles)
  if constexpr (UNITS) {
    const TileInfo t0 = sc.tile(0);
    kb = t0.k0;
    ns = t0.ns;
  }
  // scale slot and word offset of the stage after global stage g
  auto snext_off = [&](int g) {
    if constexpr (UNITS) return (((g + 1) >> 1) & 1) * SSLOT + 8 * ((g + 1) & 1);
    else return ((j1 * npairs + (s1 >> 1)) & 1) * SSLOT + 8 * (s1 & 1);
  };
  // Pending B-half loads; none before the first stage: those 4 loads point
  // past the end and land in the dummy region (slots 0 and 1 are live).
  uint32_t pend_vb[4] = {OOB, OOB, OOB, OOB};
  __amdgpu_buffer_rsrc_t pend_rb = rb2;
  uint32_t pend_cs = 0, pend_m0 = lds_addr + 2 * STAGE_BYTES + 2 * SSLOT;
  for (int g = 0; g < gtotal; ++g) {
    const uint32_t slot = lds_addr + (uint32_t)((g & 1) * STAGE_BYTES);
    const int kc = kb + s;                  // the K stage multiplied now
    uint32_t keep_lo = kc < nfull ? 0xFFFFFFFFu : tail_lo;
    uint32_t keep_hi = kc < nfull ? 0xFFFFFFFFu : tail_hi;
    if constexpr (UNITS) {
      if (kc > nfull) keep_lo = keep_hi = 0u;   // a padding stage past the tail
    }
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
    // 64-deep steps of this stage that hold K-blocks below K: all four except
    // in the tail stage (none in a unit's padding stage, whose first step
    // still runs on masked scales to carry its loads)
    const int live = kc < nfull ? 4 : (kc == nfull ? (kchunks + 1) >> 1 : 0);
    // the B half of stage g+1's loads (issued by the previous iteration's
    // prefetch position; dummy loads past the end in the first iteration)
    if constexpr (SPLIT)
      step0_ld(acc, a, b, sa, sb, slot + ra_k[1], slot + rb_k[1], na, nb, pend_m0, pend_vb, pend_rb, pend_cs);
    else
      step<false>(acc, a, b, sa, sb, slot + ra_k[1], slot + rb_k[1], na, nb);
    if (live >= 2) step<true>(acc, na, nb, sa, sb, slot + ra_k[2], slot + rb_k[2], a, b);
    if (live >= 3) step<false>(acc, a, b, sa2, sb2, slot + ra_k[3], slot + rb_k[3], na, nb);
    // Stage g+2 (the prefetch position): its code offsets.  Past the last
    // stage every code load points past the end (zeros into the free slot).
    const bool more = g + 2 < gtotal;
    uint32_t va[4], vb[4];
    stage_offsets(va, vb);
    if (!more) {
#pragma unroll
      for (int t = 0; t < 4; ++t) va[t] = vb[t] = OOB;
    }
    // Stage g+1: this wave's loads landed, then every wave's.  Every wave has
    // also read all of stage g (codes and scales), so its slots take stage g+2.
    wait_vmcnt(0);
    bare_barrier();
    if (more && !(s2 & 1)) issue_scales(rs2, psc, (kb2 + s2) >> 1, sslots + sslot2(g + 2), wave);
    // The next stage's first-step operands and scale bytes (in the very last
    // stage these reads of unused slots are harmless).
    const uint32_t next = lds_addr + (uint32_t)(((g + 1) & 1) * STAGE_BYTES);
    const uint32_t snext = sl_addr + (uint32_t)snext_off(g);
    if constexpr (SPLIT) {
      if (live == 4)
        step_last(acc, na, nb, sa2, sb2, next + ra_k[0], next + rb_k[0], snext + s_a, snext + s_b, a, b, wa, wb,
                  slot + 4096u * wave, va, ra2, (uint32_t)(kb2 + s2) * ROWB);
      else
        step_last_nm(next + ra_k[0], next + rb_k[0], snext + s_a, snext + s_b, a, b, wa, wb, slot + 4096u * wave,
                     va, ra2, (uint32_t)(kb2 + s2) * ROWB);
      // the B half goes out in the next iteration's first step
#pragma unroll
      for (int t = 0; t < 4; ++t) pend_vb[t] = vb[t];
      pend_rb = rb2;
      pend_cs = (uint32_t)(kb2 + s2) * ROWB;
      pend_m0 = slot + OPB + 4096u * wave;
    } else {
      static_assert(!UNITS, "units need the split load issue");
      step_last8(acc, na, nb, sa2, sb2, next + ra_k[0], next + rb_k[0], snext + s_a, snext + s_b, a, b, wa, wb,
                 slot + 4096u * wave, va, vb, ra2, rb2, (uint32_t)(kb2 + s2) * ROWB);
    }
    if (more) advance();
    if constexpr (!UNITS) {
      if (++s1 == nst) {
        s1 = 0;
        ++j1;
      }
    }
    if (++s == ns) {                        // tile (unit) j is complete
      drain(acc);
      if constexpr (UNITS) {
        store_unit<OUT == OUT_BF16_>(acc, sc, j, C, ldc);
        if (j + 1 < ntiles) {
          const TileInfo tn = sc.tile(j + 1);
          kb = tn.k0;
          ns = tn.ns;
        }
      } else {
        store(sc.tile(j));
      }
      zero(acc);
      s = 0;
      ++j;
    }
  }
  __syncthreads();                          // LDS may be reused by the caller
}

// Output stores are bounds-checked buffer stores: the resource ends after row
// mlim (relative to the tile origin C), and lanes whose columns are >= nlim
// point past it, so nothing outside the matrix is written.  Row offsets are
// wave-uniform (scalar), column offsets per lane.  (In the accumulator layout
// each store instruction writes two 32-lane row segments; gathering 4 columns
// of 4 rows per lane for wider stores measured slower, whole-line bf16 stores
// below 1-2 % faster.)
//
// Buffer resource of the output tile at C: it ends after row mlim (relative
// to the tile origin) and column nlim of that row.
template <bool OUT_BF16>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_out_rsrc(void* C, int ldc, int mlim, int nlim) {
  constexpr int ES = OUT_BF16 ? 2 : 4;
  const int rows = mlim < 256 ? mlim : 256;
  return rsrc(C, (uint32_t)((rows - 1) * ldc * ES + (nlim < 256 ? nlim : 256) * ES));
}

// Store 32x32 MFMA tile (i, j) of the wave's part (values x in the
// accumulator layout) through the resource r of the output tile.
template <bool OUT_BF16>
__device__ __forceinline__ void store_subtile(const v16f& x, int i, int j, __amdgpu_buffer_rsrc_t r, int ldc,
                                              int nlim) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, kh = lane >> 5;
  constexpr int ES = OUT_BF16 ? 2 : 4;
  const int col = wn * TJ * 32 + 32 * j + l32;
  const uint32_t voff = col < nlim ? (uint32_t)(((wm * TI * 32 + 4 * kh) * ldc + col) * ES) : OOB;
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t soff = (uint32_t)((32 * i + 8 * r4 + q) * ldc * ES);
      const float v = x[4 * r4 + q];
      if (OUT_BF16)
        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (__bf16)v), r, voff, soff, 0);
      else
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, voff, soff, 0);
    }
}

// bf16 tile stores in whole 128-byte lines.  In the accumulator layout a
// store instruction covers two rows of 32 columns, 64 bytes each: half lines.
// Exchanging the upper half-wave of MFMA tile j with the lower half-wave of
// tile j + 1 (v_permlane32_swap) gives registers holding one row of 64
// columns across the wave; converting two such rows to bf16 pairs and trading
// halves with the neighbouring lane (a DPP swap and a byte permute) leaves an
// even lane with columns (l, l + 1) of the first row and an odd lane with
// columns (l - 1, l) of the second.  One 4-byte store per lane then writes
// two whole lines, half as many store instructions as the plain layout.
// Needs an even ldc and nlim and a 4-byte aligned tile origin (so a lane's
// pair of columns is either wholly inside the matrix or wholly outside).
__device__ __forceinline__ void store_bf16_rows(float x0, float x1, __amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                uint32_t soff, uint32_t sel) {
  const uint32_t p = (uint32_t)__builtin_bit_cast(unsigned short, (__bf16)x0) |
                     ((uint32_t)__builtin_bit_cast(unsigned short, (__bf16)x1) << 16);
  const uint32_t q = (uint32_t)__builtin_amdgcn_mov_dpp((int)p, 0xB1, 0xF, 0xF, false);   // lane l ^ 1
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_amdgcn_perm(q, p, sel), r, voff, soff, 0);
}

__device__ __forceinline__ void store_tile_bf16_lines(const Acc& acc, __amdgpu_buffer_rsrc_t r, int ldc, int nlim) {
  static_assert(TJ % 2 == 0, "tiles are paired along N");
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int odd = lane & 1;
  // even lane: bytes 0-1 of its own pair, then bytes 0-1 of its neighbour's;
  // odd lane: bytes 2-3 of the neighbour's, then its own bytes 2-3
  const uint32_t sel = odd ? 0x03020706u : 0x05040100u;
#pragma unroll
  for (int jp = 0; jp < TJ; jp += 2) {
    const int col = wn * TJ * 32 + 32 * jp + (lane & ~1);
    const uint32_t voff = col < nlim ? (uint32_t)(((wm * TI * 32 + odd) * ldc + col) * 2) : OOB;
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
        for (int qp = 0; qp < 4; qp += 2) {
          const auto s0 = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc.t[i][jp][4 * r4 + qp]),
                                                           __float_as_uint(acc.t[i][jp + 1][4 * r4 + qp]), false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc.t[i][jp][4 * r4 + qp + 1]),
                                                           __float_as_uint(acc.t[i][jp + 1][4 * r4 + qp + 1]), false,
                                                           false);
          // s?[0]: row 32 i + 8 r4 + q (the lower half-wave's row), 64 columns;
          // s?[1]: row 32 i + 8 r4 + 4 + q (the upper half-wave's row)
          const int row = 32 * i + 8 * r4 + qp;
          store_bf16_rows(__uint_as_float(s0[0]), __uint_as_float(s1[0]), r, voff, (uint32_t)(row * ldc * 2), sel);
          store_bf16_rows(__uint_as_float(s0[1]), __uint_as_float(s1[1]), r, voff, (uint32_t)((row + 4) * ldc * 2),
                          sel);
        }
  }
}

// Store the wave's part of the tile.
template <bool OUT_BF16>
__device__ __forceinline__ void store_tile(const Acc& acc, void* C, int ldc, int mlim, int nlim) {
  const __amdgpu_buffer_rsrc_t r = tile_out_rsrc<OUT_BF16>(C, ldc, mlim, nlim);
  if constexpr (OUT_BF16) {
    if (((ldc | nlim) & 1) == 0 && ((uintptr_t)C & 3) == 0) {
      store_tile_bf16_lines(acc, r, ldc, nlim);
      return;
    }
  }
#pragma unroll
  for (int j = 0; j < TJ; ++j)
#pragma unroll
    for (int i = 0; i < TI; ++i) store_subtile<OUT_BF16>(acc.t[i][j], i, j, r, ldc, nlim);
}

// ------------------------------------------------------------ split-K epilogue
// A unit that covers only part of its tile's K range ends here.  The tile's
// segments (its K range cut at the unit boundaries, segment 0 first in the
// tile's pair order) each hold a float32 partial product; the tile is their
// sum taken in segment
// order, ((p_0 + p_1) + p_2) + ..., each addition rounded to float32, so the
// result does not depend on which workgroup gets there last.  No workgroup
// waits for another: each segment first reads the tile's counter; if every
// other segment has already published its partial (counter = S - 1) this one
// is the last and sums; otherwise it writes its partial to its workspace slot,
// makes it visible at device scope and increments the counter, and the
// segment that sees S - 1 come back from that increment sums.  The summing
// segment resets the counter to 0, so the workspace is left as it was found.
// The summing segment takes its own partial from its accumulators and the
// others from their slots.
// Partial slots hold the 256x256 floats in the accumulator layout: float4 q
// (= 4 (TJ i + j) + r4) of thread tid at float4 index q * 512 + tid.
constexpr int SLOT_BYTES = TM * TN * 4;    // one partial tile

// The partials pass between workgroups on different XCDs, whose L2 caches are
// not kept coherent with each other for plain accesses: they are stored and
// loaded at system scope (cache policy SC0 | SC1), which writes through to
// memory and reads from it.
constexpr int CPOL_SYSTEM = 1 | 16;

// A wave-uniform 64-bit address (so buffer resources built from it stay in
// scalar registers instead of being looped over lane by lane).
__device__ __forceinline__ float* uniform_ptr(float* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (float*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// Partial slot `slot` as a buffer resource (one lane offset, the float4 index
// in the scalar offset, so no per-load 64-bit addresses are held).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slot_rsrc(float* parts, int slot) {
  return rsrc(uniform_ptr(parts + (size_t)__builtin_amdgcn_readfirstlane(slot) * (SLOT_BYTES / 4)),
              (uint32_t)SLOT_BYTES);
}

// Write this workgroup's accumulators to partial slot `slot`.
__device__ __forceinline__ void put_partial(const Acc& acc, float* parts, int slot) {
  constexpr int NT = 64 * WAVES;
  const __amdgpu_buffer_rsrc_t r = slot_rsrc(parts, slot);
  const uint32_t voff = 16u * threadIdx.x;
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int jj = 0; jj < TJ; ++jj)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const v16f& x = acc.t[i][jj];
        const v4u w = {__float_as_uint(x[4 * r4]), __float_as_uint(x[4 * r4 + 1]), __float_as_uint(x[4 * r4 + 2]),
                       __float_as_uint(x[4 * r4 + 3])};
        __builtin_amdgcn_raw_buffer_store_b128(w, r, voff, (uint32_t)(((i * TJ + jj) * 4 + r4) * NT * 16),
                                               CPOL_SYSTEM);
      }
}

// Publish this workgroup's partial: every wave's stores complete (they write
// through at system scope, so completion means visible to every XCD), then
// one increment of the counter; returns the counter's value before it (the
// same in every thread).  No fence is needed on either side: the partials
// never pass through a cache that another XCD could read stale (the summing
// segment loads them at system scope too), and the compiler's agent-scope
// fences (a write-back and an invalidate of the whole L2) measured ~70 us on
// the weight-gradient shape.
__device__ __forceinline__ int publish(const Acc& acc, float* parts, int slot, int* cnt, volatile int* flag) {
  put_partial(acc, parts, slot);
  __builtin_amdgcn_s_waitcnt(0x0F70);     // vmcnt(0): this wave's stores are complete
  __syncthreads();
  if (threadIdx.x == 0) {
    *flag = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  return *flag;
}

template <bool OUT_BF16, class Sched>
__device__ __forceinline__ void store_unit(Acc& acc, const Sched& sc, int j, void* C, int64_t ldc) {
  constexpr int ES = OUT_BF16 ? 2 : 4;
  const TileInfo ti = sc.tile(j);
  uint8_t* const ct = static_cast<uint8_t*>(C) + (ti.c_row0 * ldc + ti.n0) * ES;
  const auto sg = sc.segment(j);
  if (sg.S == 1) {
    store_tile<OUT_BF16>(acc, ct, (int)ldc, ti.M - ti.m0, ti.N - ti.n0);
    return;
  }
  int* const cnt = sc.counter(sg.t);
  volatile int* const aux = sc.aux();      // LDS: [0] counter value
  float* const parts = sc.parts();
  __syncthreads();
  if (threadIdx.x == 0) aux[0] = __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (aux[0] != sg.S - 1 && publish(acc, parts, sg.slot, cnt, aux) != sg.S - 1) return;
  // the last segment: every other partial is published

  // Sum each 32x32 MFMA tile over the segments in order into temporaries (the
  // accumulators are only read: rewriting all 128 of them on this path would
  // leave the register allocator two versions to merge) and store it.
  constexpr int NT = 64 * WAVES;
  const __amdgpu_buffer_rsrc_t out = tile_out_rsrc<OUT_BF16>(ct, (int)ldc, ti.M - ti.m0, ti.N - ti.n0);
  const __amdgpu_buffer_rsrc_t whole = rsrc(uniform_ptr(parts), 0xFFFFFFFFu);
  const uint32_t voff = 16u * threadIdx.x;
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int jj = 0; jj < TJ; ++jj) {
      v16f r;
#pragma unroll 1
      for (int q = 0; q < sg.S; ++q) {
        v16f p;
        if (q == sg.k) {
          p = acc.t[i][jj];
        } else {
          const uint32_t base = (uint32_t)__builtin_amdgcn_readfirstlane(sg.slot_of(q)) * (uint32_t)SLOT_BYTES +
                                (uint32_t)((i * TJ + jj) * 4 * NT * 16);
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const v4u v =
                __builtin_amdgcn_raw_buffer_load_b128(whole, voff, base + (uint32_t)(r4 * NT * 16), CPOL_SYSTEM);
#pragma unroll
            for (int e = 0; e < 4; ++e) p[4 * r4 + e] = __uint_as_float(v[e]);
          }
        }
        if (q == 0) {
          r = p;
        } else {
#pragma unroll
          for (int e = 0; e < 16; ++e) r[e] = r[e] + p[e];
        }
      }
      store_subtile<OUT_BF16>(r, i, jj, out, (int)ldc, ti.N - ti.n0);
    }
  if (threadIdx.x == 0) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

#if MX_T256_SWAP
// ------------------------------------------------------------ quantizing epilogue
// With the operands swapped, accumulator register r of MFMA tile (i, j) holds
// in lane (kh = lane / 32, l = lane % 32) the output at row 32i + l and column
// 32j + 8(r/4) + 4kh + r%4 of the wave's 64 x 128 region: a block of 32
// columns of one row lies in lanes l and l + 32, 16 values each.  Per block:
// amax of the sign-cleared bits over the lane's 16 values, then with the
// partner lane; the scale by the mode's rule (NaN/Inf -> 0xFF with zero
// codes); the 3/4 prescale after the scale; the hardware RNE convert at the
// power-of-two scale (for the lowest byte, whose 2^-127 is a float32
// subnormal, the values are multiplied by 2^127 first, exactly, and converted
// at scale 1, as the row quantizer does).  Each lane converts its 16 values into two words of
// code bytes, trades one word with its partner, and stores 8 of the block's
// 16 code bytes; lane kh = 0 stores the scale byte.  The same arithmetic as
// the row quantizer without the transform.
__device__ __forceinline__ void store_tile_mx(const Acc& acc, const QOut& q, int m0, int n0, int mlim, int nlim) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, kh = lane >> 5;
  const int rows = mlim < 256 ? mlim : 256;
  const __amdgpu_buffer_rsrc_t rc = rsrc(q.codes + (int64_t)m0 * q.ld_codes, (uint32_t)(rows * q.ld_codes));
  const __amdgpu_buffer_rsrc_t rs = rsrc(q.scales + (int64_t)m0 * q.ld_scales, (uint32_t)(rows * q.ld_scales));
  const int partner = (lane ^ 32) << 2;            // ds_bpermute byte address of lane ^ 32
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    const int row = wm * TI * 32 + 32 * i + l32;
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int cb = wn * TJ + j;                   // block column in the tile
      const v16f& x = acc.t[i][j];
      uint32_t m = 0;
#pragma unroll
      for (int r = 0; r < 16; r += 2)
        m = max(m, max(__float_as_uint(x[r]) & 0x7FFFFFFFu, __float_as_uint(x[r + 1]) & 0x7FFFFFFFu));
      m = max(m, (uint32_t)__builtin_amdgcn_ds_bpermute(partner, (int)m));
      const uint32_t s = q.scale_mode == 1 ? scale_code_round_up(m) : scale_code_from_absmax_bits(m);
      float sc = __uint_as_float(s << 23);
      float v[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) v[r] = q.scale_mode == 2 ? 0.75f * x[r] : x[r];
      if (s == 0u) {
#pragma unroll
        for (int r = 0; r < 16; ++r) v[r] = v[r] * __uint_as_float(0x7F000000u);
        sc = 1.0f;
      }
      // words p0 (columns 4kh + 0..3 and 8 + 4kh + 0..3) and p1 (16 + ..., 24 + ...)
      uint32_t p0 = 0u, p1 = 0u;
      p0 = cvt_pk_fp4<0>(p0, v[0], v[1], sc);
      p0 = cvt_pk_fp4<1>(p0, v[2], v[3], sc);
      p0 = cvt_pk_fp4<2>(p0, v[4], v[5], sc);
      p0 = cvt_pk_fp4<3>(p0, v[6], v[7], sc);
      p1 = cvt_pk_fp4<0>(p1, v[8], v[9], sc);
      p1 = cvt_pk_fp4<1>(p1, v[10], v[11], sc);
      p1 = cvt_pk_fp4<2>(p1, v[12], v[13], sc);
      p1 = cvt_pk_fp4<3>(p1, v[14], v[15], sc);
      // lane kh = 0 stores block bytes 0..7 (its p0 with the partner's p0),
      // lane kh = 1 bytes 8..15 (the partner's p1 with its p1)
      const uint32_t mine = kh ? p1 : p0;
      const uint32_t other = (uint32_t)__builtin_amdgcn_ds_bpermute(partner, (int)(kh ? p0 : p1));
      const uint32_t lo = kh ? other : mine, hi = kh ? mine : other;
      uint32_t w0 = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
      uint32_t w1 = __builtin_amdgcn_perm(hi, lo, 0x07060302u);
      if (s == 0xFFu) w0 = w1 = 0u;
      const bool colok = 32 * cb < nlim;
      const uint32_t coff = colok ? (uint32_t)(row * q.ld_codes + (n0 >> 1) + 16 * cb + 8 * kh) : OOB;
      __builtin_amdgcn_raw_buffer_store_b64(v2u{w0, w1}, rc, coff, 0, 0);
      if (kh == 0) {
        const uint32_t soff = colok ? (uint32_t)(row * q.ld_scales + (n0 >> 5) + cb) : OOB;
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)s, rs, soff, 0, 0);
      }
    }
  }
}
#endif

}  // namespace MX_T256_NS
}  // namespace mx
