// Split-K ("stream-K") form of the 256x256 MXFP4 GEMM, for problems with too
// few output tiles to fill the chip (the weight gradient: 2880 x 2880 is 144
// tiles) or too long a K for one float32 accumulator per output.
//
// "MXFP4", AI Wiki, §Conversion rules: a long dot product is the sum of block
// dot products accumulated in float32, with the order of that sum left to the
// implementation.  Here each output is accumulated in float32 over K ranges
// ("segments") of at most SK_MAX_PAIRS x 512 K, and the segment results are
// added in segment order (gemm_tile256.h, store_unit; the segments follow the
// tile's rotated pair order below), so the order is fixed by the problem shape
// alone and the result is the same bit for bit on every run.
//
// Work split: the tiles' K ranges, in units of 512 K (two 256-deep stages, the
// granule of the scale loads), are laid end to end (tile after tile in the
// grouped tile order) and cut into W equal contiguous ranges, one per
// persistent workgroup ("worker"): U pairs in all, worker w takes pairs
// [floor(w U / W), floor((w + 1) U / W)).  Each tile walks its pairs from a
// rotated start (SplitSched::rotation), so that the workers run in step along
// K and share operand slices in L2.  A tile cut by these ranges is summed by
// its last segment to finish; a tile inside one range is stored as in the
// plain kernel.  W is a multiple of 256 chosen from the shape only (not
// from the device), so the cuts, and with them the rounding, are the same on
// any GPU.  Worker w runs as workgroup b with b % 8 = its XCD and consecutive
// workers on one XCD, so the workers that share a tile mostly share an L2.
#define MX_T256_NS t256k
#define MX_T256_SWAP 0
#include "gemm_tile256.h"
#undef MX_T256_NS
#undef MX_T256_SWAP
#include "mx_launch.h"

#include <mutex>

namespace mx {

namespace {

constexpr int SK_ROUND = 256;     // workers per round of the split
constexpr int SK_MAX_PAIRS = 20;  // longest K range of one segment, in 512-K pairs (10240 K)
constexpr int SK_MIN_PAIRS = 4;   // shortest worker range worth a partial tile
constexpr int SK_SEG_MAX = 8;     // most segments per tile (the summing segment reads S - 1 partials)
constexpr int SK_MAX_TILES = 16384;                               // tiles the counter region holds
constexpr size_t SK_COUNTER_BYTES = (size_t)SK_MAX_TILES * 4;     // (the workspace layout is below)

struct SkPlan {
  int tiles_m, tiles_n, T, nst, P, W;
  int64_t U;
};

__host__ __device__ inline int64_t sk_cut(int64_t w, int64_t U, int W) { return w * U / W; }
// The worker whose range holds pair g: the largest w with sk_cut(w) <= g.
__host__ __device__ inline int sk_worker(int64_t g, int64_t U, int W) { return (int)(((g + 1) * W - 1) / U); }

// The split of an M x N x K problem, or false when the whole-tile kernel is
// the better choice: split when a tile's K is longer than one segment may be,
// or when the whole-tile schedule's longest queue (ceil(T / 256) tiles of P
// pairs per workgroup) is more than 15 % longer than the split's.
bool sk_plan(int64_t M, int64_t N, int64_t K, SkPlan& p) {
  p.tiles_m = (int)((M + 255) / 256);
  p.tiles_n = (int)((N + 255) / 256);
  p.T = p.tiles_m * p.tiles_n;
  p.nst = (int)((K + 255) / 256);
  p.P = (p.nst + 1) / 2;
  p.U = (int64_t)p.T * p.P;
  if (p.P < 2 || M <= 0 || N <= 0 || p.T > SK_MAX_TILES) return false;
  int64_t W = SK_ROUND;
  while ((p.U + W - 1) / W > SK_MAX_PAIRS) W += SK_ROUND;
  if (p.U / W < SK_MIN_PAIRS) W = p.U / SK_MIN_PAIRS > 1 ? p.U / SK_MIN_PAIRS : 1;
  // cuts at least floor(U / W) pairs apart: at most ceil(P / that) + 1 segments per tile
  while (W > 1 && (p.P + p.U / W - 1) / (p.U / W) + 1 > SK_SEG_MAX) --W;
  p.W = (int)W;
  // partial slots are addressed with 32-bit byte offsets
  if (W <= 1 || (int64_t)2 * W * t256k::SLOT_BYTES >= (int64_t)1 << 32) return false;
  const int64_t whole = (int64_t)p.P * ((p.T + SK_ROUND - 1) / SK_ROUND);
  const int64_t split = (p.U + W - 1) / W * ((W + SK_ROUND - 1) / SK_ROUND);
  return p.P > SK_MAX_PAIRS || whole * 100 > split * 115;
}

// Workspace: a fixed region of tile counters (int32, at most SK_MAX_TILES of
// them) and after it two partial slots per worker (its first and its last
// unit may each be part of a tile).  The counter region has the same place
// and size for every shape, so a workspace shared by calls of different
// shapes never finds one call's partials where another keeps its counters:
// each call leaves its counters at 0 and touches no other counter bytes.
size_t sk_workspace_bytes(const SkPlan& p) {
  return SK_COUNTER_BYTES + (size_t)2 * p.W * t256k::SLOT_BYTES;
}

// Per-launch parameters of a worker, kept in LDS and read back at unit
// boundaries (the pipeline leaves no scalar registers to hold them).
struct alignas(16) SkParams {
  const uint8_t *a_codes, *a_scales, *b_codes, *b_scales;
  float* parts;
  int* counters;
  int64_t U, c0, c1;       // total pairs; this worker's pairs [c0, c1)
  int M, N, tiles_m, tiles_n, nst, P, W, t0, n, pad0;
};
static_assert(sizeof(SkParams) == 112, "seven 16-byte LDS reads");

__device__ __forceinline__ SkParams load_sk(const SkParams* p) {
  typedef int v4i_ __attribute__((ext_vector_type(4)));
  v4i_ q[7];
  const uint32_t a = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
  // an asm read that waits only for itself (not for loads in flight to LDS)
  asm volatile(
      "ds_read_b128 %0, %7\n\t"
      "ds_read_b128 %1, %7 offset:16\n\t"
      "ds_read_b128 %2, %7 offset:32\n\t"
      "ds_read_b128 %3, %7 offset:48\n\t"
      "ds_read_b128 %4, %7 offset:64\n\t"
      "ds_read_b128 %5, %7 offset:80\n\t"
      "ds_read_b128 %6, %7 offset:96\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(q[0]), "=&v"(q[1]), "=&v"(q[2]), "=&v"(q[3]), "=&v"(q[4]), "=&v"(q[5]), "=&v"(q[6])
      : "v"(a)
      : "memory");
  int w[28];
#pragma unroll
  for (int i = 0; i < 7; ++i)
#pragma unroll
    for (int k = 0; k < 4; ++k) w[4 * i + k] = __builtin_amdgcn_readfirstlane(q[i][k]);
  return __builtin_bit_cast(SkParams, w);
}

struct SplitSched {
  static constexpr bool UNITS = true;
  struct Seg {
    int t, S, k, slot;   // tile, its segment count, this unit's segment index, its partial slot
    int w0, slot0;       // the worker of segment 0 and that segment's slot
    __device__ int slot_of(int i) const { return i == 0 ? slot0 : 2 * (w0 + i); }
  };
  const SkParams* prm;   // LDS
  int* aux_;             // LDS: one int (the counter value every thread acts on)
  int n;                 // units of this worker

  __device__ int count() const { return n; }
  // Pair range [lo, hi) of unit j within its tile t.
  __device__ static void range(const SkParams& P, int j, int& t, int& lo, int& hi) {
    t = P.t0 + j;
    const int64_t tp = (int64_t)t * P.P;
    lo = (int)((P.c0 > tp ? P.c0 : tp) - tp);
    hi = (int)((P.c1 < tp + P.P ? P.c1 : tp + P.P) - tp);
  }
  __device__ t256k::TileInfo tile(int j) const {
    const SkParams P = load_sk(prm);
    int t, lo, hi;
    range(P, j, t, lo, hi);
    int tm, tn;
    t256c::group_order<8>(t, P.tiles_m, P.tiles_n, tm, tn);
    t256k::TileInfo ti;
    ti.a_codes = P.a_codes;
    ti.a_scales = P.a_scales;
    ti.b_codes = P.b_codes;
    ti.b_scales = P.b_scales;
    ti.m0 = tm * t256k::TM;
    ti.n0 = tn * t256k::TN;
    ti.M = P.M;
    ti.N = P.N;
    ti.c_row0 = ti.m0;
    // even; a tile with an odd stage count runs one padding stage (K stages
    // [k0, k0 + ns) lie inside [0, 2P): lo + rot < P, or rot = 0)
    ti.k0 = 2 * ((lo + rotation(P, t)) % P.P);
    ti.ns = 2 * (hi - lo);
    return ti;
  }
  // Tile t walks its pairs from pair rot: local pair l (the l-th of the
  // tile's range in the laid-end-to-end order) is K pair (l + rot) mod P.
  // rot moves the first cut inside the tile (the start of worker w1 + 1, at
  // local pair o) to K pair 0, so no unit wraps past the tile's last pair,
  // and the worker starting there is at K pair 0 when it starts, like every
  // worker whose range starts inside a tile.  The worker ending in the tile
  // (local pairs [0, o), K pairs [P - o, P)) is then at K pair P - L, L the
  // range length, when it gets there: at any moment the workers are in a few
  // K phases, so the workers of an XCD read the same few 512-K slices of their
  // operand panels and find them in L2.  A tile without a cut inside keeps
  // rot = 0.
  __device__ static int rotation(const SkParams& P, int t) {
    const int64_t tp = (int64_t)t * P.P;
    const int64_t c = sk_cut(sk_worker(tp, P.U, P.W) + 1, P.U, P.W);
    return c > tp && c < tp + P.P ? (int)(tp + P.P - c) : 0;
  }
  __device__ int total_stages() const {
    const SkParams P = load_sk(prm);
    return (int)(2 * (P.c1 - P.c0));
  }
  // Tile t's segments in closed form.  With wk(g) the worker holding pair g,
  // the cuts strictly inside the tile are those of workers wk(tP) + 1 ..
  // wk(tP + P - 1), so S = wk(tP + P - 1) - wk(tP) + 1; segment i >= 1 starts
  // at the cut of worker w0 + i (w0 = wk(tP)) and is that worker's first unit
  // (slot 2 (w0 + i)); segment 0 starts at tP, the first unit of w0 when its
  // cut is tP (slot 2 w0), else its last (slot 2 w0 + 1).
  __device__ Seg segment(int j) const {
    const SkParams P = load_sk(prm);
    int t, lo, hi;
    range(P, j, t, lo, hi);
    const int64_t tp = (int64_t)t * P.P;
    const int w0 = sk_worker(tp, P.U, P.W);
    const int w = sk_worker(P.c0, P.U, P.W);
    Seg s;
    s.t = t;
    s.S = sk_worker(tp + P.P - 1, P.U, P.W) - w0 + 1;
    s.k = sk_worker(tp + lo, P.U, P.W) - w0;
    s.slot = 2 * w + (j == 0 ? 0 : 1);
    s.w0 = w0;
    s.slot0 = 2 * w0 + (sk_cut(w0, P.U, P.W) == tp ? 0 : 1);
    return s;
  }
  __device__ float* parts() const { return load_sk(prm).parts; }
  __device__ int* counter(int t) const { return load_sk(prm).counters + t; }
  __device__ volatile int* aux() const { return aux_; }
};

template <bool A2D, bool B2D, bool OUT_BF16>
__global__ __launch_bounds__(64 * t256k::WAVES, 1) void k_gemm256_sk(MxOperand A, MxOperand B, int M, int N, int K,
                                                                     void* C, int64_t ldc, SkPlan plan,
                                                                     float* parts, int* counters) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[t256k::LDS_BYTES];
  __shared__ SkParams prm;
  __shared__ int aux[1];
  if (threadIdx.x == 0) {
    const int G = plan.W, b = (int)blockIdx.x, x = b % 8;
    const int w = x * (G / 8) + (x < G % 8 ? x : G % 8) + b / 8;
    SkParams P;
    P.a_codes = A.codes;
    P.a_scales = A.scales;
    P.b_codes = B.codes;
    P.b_scales = B.scales;
    P.parts = parts;
    P.counters = counters;
    P.U = plan.U;
    P.c0 = sk_cut(w, plan.U, plan.W);
    P.c1 = sk_cut(w + 1, plan.U, plan.W);
    P.M = M;
    P.N = N;
    P.tiles_m = plan.tiles_m;
    P.tiles_n = plan.tiles_n;
    P.nst = plan.nst;
    P.P = plan.P;
    P.W = plan.W;
    P.t0 = (int)(P.c0 / plan.P);
    P.n = P.c1 > P.c0 ? (int)((P.c1 - 1) / plan.P) - P.t0 + 1 : 0;
    P.pad0 = 0;
    prm = P;
  }
  __syncthreads();
  const SplitSched sc{&prm, aux, __builtin_amdgcn_readfirstlane(prm.n)};
  const t256k::Strides sd{(int)A.ld_codes, (int)A.ld_scales, (int)B.ld_codes, (int)B.ld_scales};
  t256k::run_tiles<A2D, B2D, OUT_BF16 ? t256k::OUT_BF16_ : t256k::OUT_F32, true>(sc, sd, K, C, ldc, lds);
}

// The workspace of the allocation-free entry point (mx_gemm_noalloc): the
// counter region and 2 x 256 partial slots, enough for every plan with at most
// 256 workers (all shapes whose tiles' K ranges fit 256 x SK_MAX_PAIRS pairs,
// the weight gradient among them).  Zero at load; every call leaves its
// counters at zero again.  In host code `scratch` names a host-side stand-in:
// only the address hipGetSymbolAddress returns for the current device is
// passed to kernels.
constexpr size_t SK_SCRATCH_BYTES = SK_COUNTER_BYTES + (size_t)2 * SK_ROUND * t256k::SLOT_BYTES;
static __device__ __align__(256) uint8_t scratch[SK_SCRATCH_BYTES];

}  // namespace

size_t gemm_splitk_scratch_bytes() { return SK_SCRATCH_BYTES; }

hipError_t gemm_splitk_scratch(void** ptr) {
  static std::mutex mu;
  static void* addr[64] = {nullptr};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

size_t gemm_splitk_workspace(int64_t M, int64_t N, int64_t K) {
  SkPlan p;
  return sk_plan(M, N, K, p) ? sk_workspace_bytes(p) : 0;
}

bool gemm_splitk_applies(const GemmArgs& a) {
  SkPlan p;
  return a.a_elem == 0 && a.b_elem == 0 && gemm256_layout_ok(a) && sk_plan(a.M, a.N, a.K, p);
}

hipError_t launch_gemm_splitk(const GemmArgs& a, void* workspace, hipStream_t st) {
  SkPlan p;
  if (!sk_plan(a.M, a.N, a.K, p)) return hipErrorInvalidValue;
  int* counters = static_cast<int*>(workspace);
  float* parts = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + SK_COUNTER_BYTES);
#define MX_SK(A_, B_, O_)                                                                                  \
  hipLaunchKernelGGL((k_gemm256_sk<A_, B_, O_>), dim3(p.W), dim3(64 * t256k::WAVES), 0, st, a.A, a.B,       \
                     (int)a.M, (int)a.N, (int)a.K, a.C, a.ldc, p, parts, counters)
  if (a.out_bf16) {
    if (a.a_2d) { if (a.b_2d) MX_SK(true, true, true); else MX_SK(true, false, true); }
    else { if (a.b_2d) MX_SK(false, true, true); else MX_SK(false, false, true); }
  } else {
    if (a.a_2d) { if (a.b_2d) MX_SK(true, true, false); else MX_SK(true, false, false); }
    else { if (a.b_2d) MX_SK(false, true, false); else MX_SK(false, false, false); }
  }
#undef MX_SK
  return hipGetLastError();
}

}  // namespace mx
