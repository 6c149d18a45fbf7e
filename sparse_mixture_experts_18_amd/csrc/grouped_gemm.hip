// Grouped expert GEMMs over the ragged expert segments of the dispatch.
//
// One launch covers every expert (and the shared expert as one more
// segment): running one GEMM per expert instead is what the pages name as
// the throughput killer ("MoE architecture in practice", expert-parallelism
// section: contiguous per-expert segments let a grouped GEMM finish all
// experts at once).  Each expert is a SwiGLU FFN, E(x) = W2 (silu(Wg x) *
// (Wu x)); the shared expert is always on ("shared expert" section).
//
// GEMM1: h[s, c] = silu(x_t . Wg_e[c]) * (x_t . Wu_e[c])   t = perm[s] / k
// GEMM2: y_perm[s, n] = h[s] . W2_e[n]
//
// MFMA path (bf16: v_mfma_f32_32x32x16_bf16; MXFP8: the block-scaled
// v_mfma_scale_f32_32x32x64_f8f6f4), fp32 accumulation, work items of up to
// 384 (gate/up) or 256 (down) rows x 256 weight rows (64 x 128 and 64 x 256
// for layers with few rows per expert),
// both operands K-contiguous (weights in nn.Linear [out, in] layout), staged
// through LDS by direct buffer DMA with an XOR swizzle of the 16-byte chunks.
// The work list (segment, row block, column tile) is built on the device
// from the dispatch offsets, so no host synchronisation is needed.
// Persistent blocks, one per CU: each XCD walks its own contiguous,
// cost-balanced run of the list (whole experts, dealt to the XCDs by cost),
// so sibling row blocks that share a weight slab run close together on one
// L2.  The same
// kernels run the dense products of the LatentMoE layer over a one-segment
// list.  An fp32 VALU path serves fp32 layers.
#include <atomic>
#include <type_traits>
#include <utility>

#include "moe_internal.h"
#include "route_device.h"

namespace moe {
namespace {
// one group of the explicit instruction order of a scheduling region: N
// instructions of the classes in MASK (0x008 MFMA, 0x020 vector-memory read,
// 0x100 LDS read); nothing for N = 0
template <int MASK, int N>
__device__ __forceinline__ void sched() {
  if constexpr (N > 0) __builtin_amdgcn_sched_group_barrier(MASK, N, 0);
}
constexpr int kSchedMfma = 0x008, kSchedVmemRead = 0x020, kSchedLdsRead = 0x100;
// f(integral_constant<int, I>) for I = 0 .. N-1, in order
template <int... I, class F>
__device__ __forceinline__ void static_for_impl(std::integer_sequence<int, I...>, F&& f) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(std::make_integer_sequence<int, N>{}, f);
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// work-list construction
// ---------------------------------------------------------------------------
// The two work lists of an expert projection pair (one block per list), or
// the one or two lists of dense products.
__global__ __launch_bounds__(1024) void plan_kernel(PlanArgs a) { plan_device(a, blockIdx.x); }

// Non-persistent item index (fp32 path): block b runs on XCD b % 8; XCD x takes
// the contiguous range [x*per, (x+1)*per).  -1 for blocks without work.
__device__ __forceinline__ int xcd_item(int count) {
  const int per = (count + 7) >> 3;
  const int b = blockIdx.x;
  const int local = b >> 3, x = b & 7;
  if (local >= per) return -1;
  const int item = x * per + local;
  return item < count ? item : -1;
}

// Operands are addressed in bytes: bf16 elements are 2 bytes, MXFP8 codes 1.
// MXFP8 operands carry their scales in separate arrays, one byte per row per
// 32 values of the reduction axis.
struct GemmArgs {
  const unsigned char* a_routed;  // GEMM1: x [T, d]       GEMM2: h [T*k, d_ff]
  const unsigned char* a_shared;  // GEMM1: x [T, d]       GEMM2: h_shared [T, d_ffs]
  const int32_t* perm;            // GEMM1: row -> token via perm[row] / k; GEMM2: null
  int k;
  const unsigned char* b_routed;  // GEMM1: w1 [N][2*d_ff][d]  GEMM2: w2 [N][d][d_ff]
  const unsigned char* b_shared;
  unsigned char* c_routed;        // GEMM1: h              GEMM2: y_perm (bf16)
  unsigned char* c_shared;        // GEMM1: h_shared       GEMM2: y_shared (bf16)
  // MXFP8 only: scale bytes [rows][K/32] of A and B, and of the GEMM1 output
  const unsigned char* as_routed;
  const unsigned char* as_shared;
  const unsigned char* bs_routed;
  const unsigned char* bs_shared;
  unsigned char* cs_routed;
  unsigned char* cs_shared;
  int K_r, K_s;                   // reduction length (elements)
  int Nout_r, Nout_s;             // output columns (h columns for GEMM1)
  long long b_stride;             // elements per routed expert weight matrix
  int N;
  const WorkItem* items;
  int32_t* hdr;
  // plain (non-gated) products only: bf16 [rows, Nout] added to the fp32
  // result before the final rounding (NULL: nothing added)
  const unsigned char* addend;
  int a_rows_r, a_rows_s;  // MXFP8: rows of the A matrices (bounds of their scale arrays)
};

// ---------------------------------------------------------------------------
// MFMA grouped GEMM (bf16, or MXFP8 with per-32 block scales).
//
// Block tile: up to BM rows (assignments) x BNW weight rows, k-slices of BK
// bf16 per row (64-byte or 128-byte rows) or 128 MXFP8 values (128-byte
// rows).  RG x CG waves: wave (rg, cg)
// owns the weight rows of column group cg (GATED: gate rows 32cg..32cg+31 and
// the matching up rows, i.e. 32 h columns, so SwiGLU is applied in
// registers; plain: 64 output columns) and the 32-row MFMA sub-tiles i with
// i % RG == rg.  An item with few rows costs MFMA work in proportion to
// ceil(rows/32), not to the full tile.
//
// Operands move global -> LDS with the direct buffer-to-LDS load
// (buffer_load_dwordx4 ... lds, 16 bytes per lane, one 1 KiB block of rows per
// wave instruction) into rings of SA (rows) and SB (weights) buffers, so
// SA-1 / SB-1 k-slices are in flight while the MFMAs consume one.  Each wave
// waits only on its own loads (vmcnt); one s_barrier per slice
// publishes the slice to all waves and retires the buffer that the next DMA
// overwrites.  Inside an LDS row the 16-byte chunk c of row r sits at position
// c ^ swz(r), swz(r) = (r / rows-per-256-bytes) % chunks-per-row: the 32 rows
// of an MFMA fragment read then hit 64 distinct banks per 16 lanes.  The DMA
// lane -> LDS position map is fixed, so each lane fetches the chunk that
// belongs at its position.
//
// MXFP8: v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 x E4M3, fp32 accumulation),
// two 64-deep k-steps per slice.  Lane (r, h) of a fragment holds row r and
// k 16h..16h+15 and 32+16h..32+16h+15 of the step, and gives the scale of
// row r for the step's 32-value block h.  The scale bytes travel in groups
// of four slices (16 bytes per row): one 16-byte DMA per lane every fourth
// slice, rows of A first, then the weight rows.
// ---------------------------------------------------------------------------
template <int RG_, int CG_, int NTW_, int BK_, int SA_, int SB_, int MSW_ = 4, int LDS_KIB_ = 160,
          int MAXS_ = 4>
struct GCfg {
  static constexpr int RG = RG_, CG = CG_, NTW = NTW_, BK = BK_;
  static constexpr int SA = SA_, SB = SB_;      // LDS ring depth of A and of B
  static constexpr int WAVES = RG * CG, THREADS = WAVES * 64;
  static constexpr int MSW = MSW_;            // max 32-row sub-tiles per wave
  static constexpr int BM = RG * MSW * 32;    // rows per work item
  static constexpr int BNW = CG * NTW * 32;   // weight rows per work item
  static constexpr int ROWB = BK * 2;         // bytes per LDS row
  static constexpr int CPR = BK / 8;          // 16-byte chunks per row
  static constexpr int RP = 256 / ROWB;       // rows per 256-byte bank line
  static constexpr int DROWS = 1024 / ROWB;   // rows per wave DMA instruction
  static constexpr int A_BYTES = BM * ROWB, B_BYTES = BNW * ROWB;
  static constexpr int A_LOADS = A_BYTES / 1024 / WAVES, B_LOADS = B_BYTES / 1024 / WAVES;
  static constexpr int SGB = WAVES * 64 * 16;  // MXFP8 scale bytes of a 4-slice group
  // LDS per block; items with few rows use it for deeper rings.  160 KiB is
  // the whole CU (one block per CU); 80 KiB lets two blocks share a CU.
  static constexpr int LDS_BYTES = LDS_KIB_ * 1024;
  static constexpr int BLOCKS_PER_CU = 160 / LDS_KIB_;
  static constexpr int MAXS = MAXS_;  // deepest ring that items with few rows get
  static_assert(A_LOADS * 1024 * WAVES == A_BYTES && B_LOADS * 1024 * WAVES == B_BYTES, "");
  // the full-height tile needs at least two stages of each operand (shorter
  // items take the configured depths, or deeper rings, when they fit)
  static_assert(2 * A_BYTES + 2 * B_BYTES <= LDS_BYTES, "LDS");
  static_assert(SA >= 2 && SB >= 2 && (SB == SA || SA == SB + 1),
                "equal rings, or A one slice deeper than B");
  static_assert(ROWB == 128 || ROWB == 64, "k-slices are 64 or 128 bytes per row");
  // row sub-tiles per wave come in multiples of MSQ, so that an A stage is a
  // whole number of 1 KiB DMA blocks per wave
  static constexpr int MSQ = (RG * 32 * ROWB >= 1024 * WAVES) ? 1 : 1024 * WAVES / (RG * 32 * ROWB);
  static_assert((RG * 32 * ROWB * MSQ) % (1024 * WAVES) == 0 && MSW % MSQ == 0, "A stage DMA");
  __device__ static __forceinline__ int swz(int r) { return (r / RP) % CPR; }
};

// bf16 wide tiles.  Gate/up: up to 384 rows x 256 weight rows (six 32-row
// sub-tiles per wave), so an expert of up to 384 rows streams its weights
// once and each k-slice carries 1.5x the MFMA work per byte of 256-row
// tiles; items of up to 256 rows take three A stages and two B stages
// (160 KiB: the gathered token rows get one more slice of lead than the
// weight rows), taller ones two of each.  Down: 256 x 256, three A and two
// B stages (its bf16 output tile is staged through LDS, which a 384-row
// tile would not fit).
using Cfg1 = GCfg<2, 4, 2, 64, 3, 2, 6>;
using Cfg2 = GCfg<2, 4, 2, 64, 3, 2>;
// MXFP8 layers (the scale DMA needs BM + BNW <= 64 * WAVES)
using Cfg1x = GCfg<2, 4, 2, 64, 2, 2>;
using Cfg2x = GCfg<2, 4, 2, 64, 2, 2>;
// Layers with few rows per expert (decode batches) stream the weights with
// short items and the LDS spent on a four-deep ring.  Gate/up: 64 rows x 128
// weight rows on four waves -- twice as many items as weight slabs of 256
// rows spread the touched experts' weights over every CU.  Down: 64 rows x
// 256 weight rows on eight waves -- its reduction is only d_ff long, so the
// wider slice (twice the bytes in flight per CU) and half the items (each
// with its own ring fill and epilogue) pay more than the finer spread.  The
// k order of every output is the same as with the wide tiles, so the choice
// never changes a result.
using Cfg1n = GCfg<2, 2, 2, 64, 2, 2, 1, 160, 4>;
using Cfg2n = GCfg<2, 4, 2, 64, 2, 2, 1, 160, 4>;
using Cfg1nx = GCfg<2, 2, 2, 64, 2, 2, 1, 160, 4>;
using Cfg2nx = GCfg<2, 4, 2, 64, 2, 2, 1, 160, 4>;
// Row blocks of the dense (one-segment) lists are sized by the plain
// configurations and also run on the gated ones; a work item may never be
// taller than the tile that runs it.
static_assert(Cfg2::BM <= Cfg1::BM && Cfg2n::BM <= Cfg1n::BM, "dense row blocks fit both tiles");

// mean rows per expert at or below which the small-row tiles are used
constexpr int kNarrowRows = 64;

typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

// Operand fragments of one k-step from an LDS stage: this wave's A sub-tiles
// (rows a_row[j]) and weight rows b_row[0..NTW).  bf16 (16-k steps): 16-byte
// chunk 2ks + h of each row.  MXFP8 (64-k steps): chunks 4ks + h and
// 4ks + 2 + h.
template <bool MX>
struct Frag;
template <>
struct Frag<false> {
  typedef bf16x8_t T;
  __device__ static __forceinline__ T read(const unsigned char* row, int ks, int fh, int sw) {
    return *reinterpret_cast<const bf16x8_t*>(row + (((2 * ks + fh) ^ sw) << 4));
  }
};
template <>
struct Frag<true> {
  typedef i32x8_t T;
  __device__ static __forceinline__ T read(const unsigned char* row, int ks, int fh, int sw) {
    const i32x4_t lo = *reinterpret_cast<const i32x4_t*>(row + (((4 * ks + fh) ^ sw) << 4));
    const i32x4_t hi = *reinterpret_cast<const i32x4_t*>(row + (((4 * ks + 2 + fh) ^ sw) << 4));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
};

template <bool MX, class C, int MS>
__device__ __forceinline__ void load_frags(const unsigned char* As, const unsigned char* Bs,
                                           const int (&a_row)[MS], const int (&b_row)[C::NTW],
                                           int fh, int ks, typename Frag<MX>::T (&af)[MS],
                                           typename Frag<MX>::T (&bf)[C::NTW]) {
#pragma unroll
  for (int j = 0; j < C::NTW; ++j)
    bf[j] = Frag<MX>::read(Bs + b_row[j] * C::ROWB, ks, fh, C::swz(b_row[j]));
#pragma unroll
  for (int i = 0; i < MS; ++i)
    af[i] = Frag<MX>::read(As + a_row[i] * C::ROWB, ks, fh, C::swz(a_row[i]));
}

// acc += weight fragment x row fragment (the accumulator holds the tile
// transposed); MXFP8 scales are E8M0 bytes in bits 0..7 of sb / sa
__device__ __forceinline__ f32x16_t mma(const bf16x8_t& b, const bf16x8_t& a, const f32x16_t& c,
                                        int, int) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16_t mma(const i32x8_t& b, const i32x8_t& a, const f32x16_t& c,
                                        int sb, int sa) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c, 0, 0, 0, sb, 0, sa);
}

// main loop + epilogue for items whose waves hold MS row sub-tiles (the last
// one only if `last` is set for this wave)
template <bool GATED, bool MX, class C, int MS>
__device__ __forceinline__ void gemm_body(const GemmArgs& g, const WorkItem& it,
                                          unsigned char* lds, int msub) {
  typedef typename Frag<MX>::T FT;
  static_assert(!MX || C::BM + C::BNW <= C::WAVES * 64, "one scale DMA per wave covers every row");
  static_assert(!MX || C::ROWB == 128, "MXFP8 slices are two 64-deep k-steps");
  constexpr int ES = MX ? 1 : 2;         // bytes per element
  constexpr int KSTEPS = MX ? 2 : C::ROWB / 32;  // k-steps per slice: 64-deep / 16-deep
  const bool shared = it.seg == g.N;
  const int K = shared ? g.K_s : g.K_r;
  const int Kb = K * ES;                 // bytes per operand row
  const int Nout = shared ? g.Nout_s : g.Nout_r;
  const unsigned char* A = shared ? g.a_shared : g.a_routed;
  const unsigned char* B =
      shared ? g.b_shared : g.b_routed + (long long)it.seg * g.b_stride * ES;
  unsigned char* Cm = shared ? g.c_shared : g.c_routed;
  const int n0 = it.nt * (GATED ? C::BNW / 2 : C::BNW);

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int rg = w / C::CG, cg = w % C::CG;
  // this wave's last row sub-tile is live iff (MS-1)*RG + rg < msub
  const bool last = (MS - 1) * C::RG + rg < msub;

  // DMA geometry: wave load q covers tile rows DROWS*q .. +DROWS-1; lane ->
  // tile row DROWS*q + lane/CPR at LDS position lane%CPR, so it fetches global
  // chunk (lane%CPR) ^ swz(row)
  const int drow = lane / C::CPR, dpos = lane % C::CPR;
  // only the rows of the MS*RG live sub-tiles are fetched
  constexpr int AL = C::RG * MS * 32 * C::ROWB / 1024 / C::WAVES;
  static_assert(AL * 1024 * C::WAVES == C::RG * MS * 32 * C::ROWB, "A rows per wave load");
  auto a_src = [&](int tr) {  // source row of tile row tr (clamped to the item)
    int src = it.row0 + min(tr, it.nrows - 1);
    if (g.perm && !shared) src = g.perm[src] / g.k;
    return src;
  };
  auto b_src = [&](int r) {  // weight row of tile weight row r (clamped)
    if (GATED)
      return r < C::BNW / 2 ? min(n0 + r, Nout - 1) : Nout + min(n0 + r - C::BNW / 2, Nout - 1);
    return min(n0 + r, Nout - 1);
  };
  uint32_t a_off[AL], b_off[C::B_LOADS];
#pragma unroll
  for (int j = 0; j < AL; ++j) {
    const int tr = (w * AL + j) * C::DROWS + drow;
    a_off[j] = (uint32_t)a_src(tr) * (uint32_t)Kb + (dpos ^ C::swz(tr)) * 16;
  }
#pragma unroll
  for (int j = 0; j < C::B_LOADS; ++j) {
    const int r = (w * C::B_LOADS + j) * C::DROWS + drow;
    b_off[j] = (uint32_t)b_src(r) * (uint32_t)Kb + (dpos ^ C::swz(r)) * 16;
  }
  // MXFP8 scales travel in groups of four slices: every fourth iteration
  // lane gl = 64w + lane fetches 16 bytes -- the scale bytes of those four
  // slices -- of tile row gl (gl < BM) or weight row gl - BM (gl < BM +
  // BNW); the remaining lanes repeat weight row 0 into slots nobody reads.
  // BM is a multiple of 64, so each wave reads from one array (a uniform
  // base).  The buffer ends at the array's end: the bytes a short last
  // group reads past it come back as 0 and are never used.
  const unsigned char* s_base = nullptr;
  uint32_t s_off = 0, s_bytes = 0;
  if (MX) {
    static_assert(C::BM % 64 == 0, "");
    const int gl = w * 64 + lane;
    const int kb = K / kMxBlock;  // scale bytes per row
    if (w * 64 < C::BM) {
      s_base = shared ? g.as_shared : g.as_routed;
      s_off = (uint32_t)a_src(gl) * (uint32_t)kb;
      s_bytes = (uint32_t)(shared ? g.a_rows_s : g.a_rows_r) * (uint32_t)kb;
    } else {
      const int r = gl - C::BM < C::BNW ? gl - C::BM : 0;
      s_base = shared ? g.bs_shared : g.bs_routed + (long long)it.seg * (g.b_stride / kMxBlock);
      s_off = (uint32_t)b_src(r) * (uint32_t)kb;
      s_bytes = (uint32_t)(GATED ? 2 * Nout : Nout) * (uint32_t)kb;
    }
  }

  // LDS: SA buffers of the A slice (only the live rows), then SB buffers of
  // the B slice, then (MXFP8) two scale-group buffers.  Items with fewer rows
  // have smaller A slices and get deeper rings (their short MFMA phase hides
  // less latency per slice).
  constexpr int A_SL = C::RG * MS * 32 * C::ROWB;  // bytes of one A stage
  constexpr int SGL = MX ? 2 * C::SGB : 0;         // scale-group buffers
  constexpr int RING = C::LDS_BYTES - SGL;
  constexpr int SDEEP = (RING / (A_SL + C::B_BYTES)) < C::MAXS
                            ? (RING / (A_SL + C::B_BYTES)) : C::MAXS;
  constexpr bool CFG_FITS = C::SA * A_SL + C::SB * C::B_BYTES <= RING;
  constexpr int SA = SDEEP > C::SA ? SDEEP : (CFG_FITS ? C::SA : SDEEP);
  constexpr int SB = SDEEP > C::SB ? SDEEP : (CFG_FITS ? C::SB : SDEEP);
  static_assert(SA * A_SL + SB * C::B_BYTES <= RING, "LDS");
  static_assert((SB == SA || (!MX && SA == SB + 1)) && (!MX || SA <= 4),
                "MXFP8: equal rings, and a window of SA-2 iterations holds at most one group load");
  unsigned char* const Abuf = lds;
  unsigned char* const Bbuf = lds + SA * A_SL;
  unsigned char* const Gbuf = lds + RING;
  const int nk = Kb / C::ROWB;
  const int ng = (nk + 3) >> 2;  // scale groups
  const rsrc_t ra = make_rsrc(A), rb = make_rsrc(B);
  const rsrc_t rs = make_rsrc(MX ? s_base : A, MX ? s_bytes : 0xFFFFFFFFu);
  auto issue_g = [&](int gi) {  // scale group gi (slices 4gi .. 4gi+3)
    if (MX) dma16(rs, s_off + 16 * gi, 0, Gbuf + (gi & 1) * C::SGB + w * 1024);
  };
  auto issue_a = [&](int kt) {
    unsigned char* st = Abuf + (kt % SA) * A_SL;
    const uint32_t k0 = kt * C::ROWB;
#pragma unroll
    for (int j = 0; j < AL; ++j) dma16(ra, a_off[j], k0, st + (w * AL + j) * 1024);
  };
  auto issue_b = [&](int kt) {
    unsigned char* st = Bbuf + (kt % SB) * C::B_BYTES;
    const uint32_t k0 = kt * C::ROWB;
    // weights as streaming data, so that they leave L2 and the MALL before
    // the rows they multiply: in the gate/up projection (the token rows
    // are re-read by every column tile of their row block; mixtral -4 %,
    // switch -16 %, dsv3 unchanged) and in the small-row tiles (one 32-row
    // sub-tile per wave, each weight byte read about once).  The dsv3 down
    // projection, whose sibling row blocks share their weight slabs in L2,
    // loses 3.5 % with it.
    constexpr int aux = (GATED || C::MSW == 1) ? kNonTemporal : 0;
#pragma unroll
    for (int j = 0; j < C::B_LOADS; ++j)
      dma16<aux>(rb, b_off[j], k0, st + (w * C::B_LOADS + j) * 1024);
  };


  constexpr int NT = C::NTW, HT = NT / 2;  // weight tiles per wave; GATED: gate tiles
  f32x16_t acc[MS][NT];
#pragma unroll
  for (int i = 0; i < MS; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // GATED: tiles 0..HT-1 are gate rows cg*HT*32 + 32j, tiles HT..NT-1 the
  // matching up rows (same h columns); plain: NT consecutive tiles
  const int fr = lane & 31, fh = lane >> 5;
  int a_row[MS], b_row[NT];
#pragma unroll
  for (int i = 0; i < MS; ++i) a_row[i] = (i * C::RG + rg) * 32 + fr;
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    if (GATED)
      b_row[j] = (j < HT ? 0 : C::BNW / 2) + (cg * HT + (j % HT)) * 32 + fr;
    else
      b_row[j] = (cg * NT + j) * 32 + fr;
  }

  // Issue order: iteration j issues (MXFP8, j a multiple of 4: scale group
  // j/4 + 1,) A(j+SA-1), then B(j+SB-1); the prologue plays iterations
  // -(SB-1) .. -1 after scale group 0.  Vector-memory loads retire in order,
  // so at iteration kt the loads of slice kt are complete once no more than
  // the younger ones are outstanding: A/B(kt+1 .. kt+SA-2), and the scale
  // group loaded in one of those iterations.  A scale group is loaded three
  // or more iterations before its first slice, so it is complete by then.
  //
  // With an A ring one slice deeper than the B ring (bf16), iteration j
  // issues B(j+SB-1) first, then A(j+SA-1) = A(j+SB): the younger loads at
  // iteration kt are A(kt+1) and A/B of iterations kt-SB+2 .. kt-1.
  constexpr bool BFIRST = SA > SB;
  constexpr int YOUNGER = BFIRST ? AL + (SB - 2) * (AL + C::B_LOADS)
                                 : (SA - 2) * (AL + C::B_LOADS);
  constexpr int SMAX = SA > SB ? SA : SB;
  issue_g(0);
#pragma unroll
  for (int j = -(SMAX - 1); j < 0; ++j) {
    if (BFIRST && j + SB - 1 >= 0 && j + SB - 1 < nk) issue_b(j + SB - 1);
    if (j + SA - 1 >= 0 && j + SA - 1 < nk) issue_a(j + SA - 1);
    if (!BFIRST && j + SB - 1 >= 0 && j + SB - 1 < nk) issue_b(j + SB - 1);
  }

  if constexpr (!MX) {
    // bf16: the k-loop in two parts -- steady iterations that refill the
    // ring, then the last SA-1 that do not -- and the live-row test of the
    // wave's last sub-tile taken once per item, so the body of a slice is
    // one straight-line block whose LDS reads and MFMAs are interleaved
    // explicitly: each fragment is read at least one MFMA pair before it is
    // used, instead of being read into the register its previous use has
    // just released.
    // Refill of the ring in a steady iteration, in the issue order the wait
    // counts assume (with a deeper A ring, B first).  The gate/up projection
    // issues both operands at k-step 0, as early as the barrier allows (its
    // long reduction is bound by load latency: dsv3 -2.4 %, mixtral -5 %,
    // switch -13 %); the down projection issues the second operand one
    // k-step later, so the fragment reads of k-step 0 do not queue behind a
    // burst of loads (issuing both at once costs it 2.5-11 %).
    auto refill_second = [&](int kt) {
      if (BFIRST) issue_a(kt + SA - 1);
      else issue_b(kt + SB - 1);
    };
    constexpr int FIRST_LOADS = BFIRST ? C::B_LOADS : AL;
    constexpr int REFILL0 = GATED ? AL + C::B_LOADS : FIRST_LOADS;
    auto refill_first = [&](int kt) {
      if (BFIRST) issue_b(kt + SB - 1);
      else issue_a(kt + SA - 1);
      if (GATED) refill_second(kt);
    };
    auto slice = [&](int kt, auto issue_tag, auto last_tag) {
      constexpr bool ISSUE = decltype(issue_tag)::value;
      constexpr bool LAST = decltype(last_tag)::value;
      constexpr int MSL = LAST ? MS : MS - 1;  // live row sub-tiles
      const unsigned char* As = Abuf + (kt % SA) * A_SL;
      const unsigned char* Bs = Bbuf + (kt % SB) * C::B_BYTES;
      if constexpr (MS * NT * 16 + 2 * (MS + NT) * 4 > 224) {
        // tall tiles: weight fragments double-buffered across k-steps, row
        // fragments in a two-register rotation one sub-tile ahead
        FT bf[2][NT], ar[2];
#pragma unroll
        for (int j = 0; j < NT; ++j)
          bf[0][j] = Frag<MX>::read(Bs + b_row[j] * C::ROWB, 0, fh, C::swz(b_row[j]));
        ar[0] = Frag<MX>::read(As + a_row[0] * C::ROWB, 0, fh, C::swz(a_row[0]));
        sched<kSchedLdsRead, NT + 1>();
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
          const int cb = ks & 1;
          const bool more = ks + 1 < KSTEPS;
          if (ISSUE && ks == 0) refill_first(kt);
          if (ISSUE && ks == 1 && !GATED) refill_second(kt);
#pragma unroll
          for (int i = 0; i < MSL; ++i) {
            const int q = (ks * MSL + i) & 1;  // rotation slot of sub-tile i
            if (i + 1 < MSL) {
              ar[q ^ 1] = Frag<MX>::read(As + a_row[i + 1] * C::ROWB, ks, fh, C::swz(a_row[i + 1]));
            } else if (more) {
              ar[q ^ 1] = Frag<MX>::read(As + a_row[0] * C::ROWB, ks + 1, fh, C::swz(a_row[0]));
#pragma unroll
              for (int j = 0; j < NT; ++j)
                bf[cb ^ 1][j] =
                    Frag<MX>::read(Bs + b_row[j] * C::ROWB, ks + 1, fh, C::swz(b_row[j]));
            }
#pragma unroll
            for (int j = 0; j < NT; ++j) acc[i][j] = mma(bf[cb][j], ar[q], acc[i][j], 0, 0);
          }
        }
        // order: per sub-tile, the next fragment read(s), then its MFMAs
        static_for<KSTEPS>([&](auto ks_c) {
          constexpr int ks = decltype(ks_c)::value;
          if constexpr (ISSUE && ks == 0) sched<kSchedVmemRead, REFILL0>();
          if constexpr (ISSUE && ks == 1 && !GATED)
            sched<kSchedVmemRead, (BFIRST ? AL : C::B_LOADS)>();
          static_for<MSL>([&](auto i_c) {
            constexpr int i = decltype(i_c)::value;
            sched<kSchedLdsRead, (i + 1 < MSL ? 1 : (ks + 1 < KSTEPS ? NT + 1 : 0))>();
            sched<kSchedMfma, NT>();
          });
        });
      } else {
        // fragments of k-step ks+1 are read while the MFMAs of k-step ks
        // run (two register sets), one read after each MFMA
        FT bf[2][NT], af[2][MS];
        load_frags<MX, C, MS>(As, Bs, a_row, b_row, fh, 0, af[0], bf[0]);
        sched<kSchedLdsRead, MS + NT>();
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
          const int cur = ks & 1;
          if (ISSUE && ks == 0) refill_first(kt);
          if (ISSUE && ks == 1 && !GATED) refill_second(kt);
          if (ks + 1 < KSTEPS)
            load_frags<MX, C, MS>(As, Bs, a_row, b_row, fh, ks + 1, af[cur ^ 1], bf[cur ^ 1]);
#pragma unroll
          for (int i = 0; i < MSL; ++i)
#pragma unroll
            for (int j = 0; j < NT; ++j)
              acc[i][j] = mma(bf[cur][j], af[cur][i], acc[i][j], 0, 0);
        }
        static_for<KSTEPS>([&](auto ks_c) {
          constexpr int ks = decltype(ks_c)::value;
          if constexpr (ISSUE && ks == 0) sched<kSchedVmemRead, REFILL0>();
          if constexpr (ISSUE && ks == 1 && !GATED)
            sched<kSchedVmemRead, (BFIRST ? AL : C::B_LOADS)>();
          constexpr int NM = MSL * NT;
          constexpr int NR = ks + 1 < KSTEPS ? MS + NT : 0;
          static_for<NM>([&](auto m_c) {
            constexpr int m = decltype(m_c)::value;
            sched<kSchedMfma, 1>();
            sched<kSchedLdsRead, (m < NR ? 1 : 0)>();
          });
          sched<kSchedLdsRead, (NR > NM ? NR - NM : 0)>();
        });
      }
    };
    auto run = [&](auto last_tag) {
      int kt = 0;
      for (; kt < nk - (SA - 1); ++kt) {
        wait_vm<YOUNGER>();
        __builtin_amdgcn_s_barrier();
        slice(kt, std::true_type{}, last_tag);
      }
      for (; kt < nk; ++kt) {
        if (kt + SMAX - 2 < nk) wait_vm<YOUNGER>();
        else wait_vm<0>();
        __builtin_amdgcn_s_barrier();
        if (BFIRST && kt + SB - 1 < nk) issue_b(kt + SB - 1);
        slice(kt, std::false_type{}, last_tag);
      }
    };
    if (last) run(std::true_type{});
    else run(std::false_type{});
  } else {
    // MXFP8: the same two-part k-loop and straight-line slices.  Fragments
    // are twice as wide and each MFMA four times as long as in bf16: each
    // row fragment is re-read for the next k-step right after its MFMAs,
    // and the weight fragments of the next k-step are read into a second
    // set at the start of this one.  The gate/up projection refills both
    // operands at k-step 0, the down projection the weights at k-step 1.
    auto slice = [&](int kt, auto issue_tag, auto last_tag) {
      constexpr bool ISSUE = decltype(issue_tag)::value;
      constexpr bool LAST = decltype(last_tag)::value;
      constexpr int MSL = LAST ? MS : MS - 1;
      const unsigned char* As = Abuf + (kt % SA) * A_SL;
      const unsigned char* Bs = Bbuf + (kt % SB) * C::B_BYTES;
      // scales of this slice: word kt % 4 of a row's 16 bytes in its group
      // buffer; byte b of the word is block b of the slice; the lane of half
      // h takes block 2ks + h into bits 0..7
      const uint32_t* sc =
          reinterpret_cast<const uint32_t*>(Gbuf + ((kt >> 2) & 1) * C::SGB) + (kt & 3);
      uint32_t sa_w[MS], sb_w[NT];
#pragma unroll
      for (int i = 0; i < MS; ++i) sa_w[i] = sc[4 * a_row[i]] >> (8 * fh);
#pragma unroll
      for (int j = 0; j < NT; ++j) sb_w[j] = sc[4 * (C::BM + b_row[j])] >> (8 * fh);
      FT bf[2][NT], af[MS];
      load_frags<MX, C, MS>(As, Bs, a_row, b_row, fh, 0, af, bf[0]);
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const int cb = ks & 1;
        const bool more = ks + 1 < KSTEPS;
        if (ISSUE && ks == 0) {
          issue_a(kt + SA - 1);
          if (GATED) issue_b(kt + SB - 1);
        }
        if (ISSUE && ks == 1 && !GATED) issue_b(kt + SB - 1);
        if (more) {
#pragma unroll
          for (int j = 0; j < NT; ++j)
            bf[cb ^ 1][j] = Frag<MX>::read(Bs + b_row[j] * C::ROWB, ks + 1, fh, C::swz(b_row[j]));
        }
        const int sh = 16 * ks;  // block 2ks + h sits 16 ks bits up
#pragma unroll
        for (int i = 0; i < MSL; ++i) {
#pragma unroll
          for (int j = 0; j < NT; ++j)
            acc[i][j] = mma(bf[cb][j], af[i], acc[i][j], (int)(sb_w[j] >> sh), (int)(sa_w[i] >> sh));
          if (more) af[i] = Frag<MX>::read(As + a_row[i] * C::ROWB, ks + 1, fh, C::swz(a_row[i]));
        }
      }
      // order: the scale words and k-step 0's fragments, then per k-step
      // the loads, the next weight fragments, and per sub-tile its MFMAs
      // followed by the re-read of its row fragment
      sched<kSchedLdsRead, 3 * (MS + NT)>();
      static_for<KSTEPS>([&](auto ks_c) {
        constexpr int ks = decltype(ks_c)::value;
        constexpr bool more = ks + 1 < KSTEPS;
        if constexpr (ISSUE && ks == 0) sched<kSchedVmemRead, GATED ? AL + C::B_LOADS : AL>();
        if constexpr (ISSUE && ks == 1 && !GATED) sched<kSchedVmemRead, C::B_LOADS>();
        sched<kSchedLdsRead, (more ? 2 * NT : 0)>();
        static_for<MSL>([&](auto) {
          sched<kSchedMfma, NT>();
          sched<kSchedLdsRead, (more ? 2 : 0)>();
        });
      });
    };
    // a scale group among the younger loads at iteration kt: one of
    // iterations kt-SA+2 .. kt-1 was a multiple of 4 that issued one
    auto wait_for = [&](int kt) {
      bool grp = false;
#pragma unroll
      for (int i = 1; i <= SA - 2; ++i) {
        const int it2 = kt - i;
        grp = grp || (it2 >= 0 && (it2 & 3) == 0 && (it2 >> 2) + 1 < ng);
      }
      if (kt + SMAX - 2 < nk) {  // every younger load was issued
        if (grp) wait_vm<YOUNGER + 1>();
        else wait_vm<YOUNGER>();
      } else {
        wait_vm<0>();
      }
    };
    auto run = [&](auto last_tag) {
      int kt = 0;
      // every wave's part of slice kt is in LDS after the wait, and every
      // wave is done with slice kt-1, whose buffers the refill overwrites,
      // after the barrier
      for (; kt < nk - (SA - 1); ++kt) {
        wait_for(kt);
        __builtin_amdgcn_s_barrier();
        if ((kt & 3) == 0 && (kt >> 2) + 1 < ng) issue_g((kt >> 2) + 1);
        slice(kt, std::true_type{}, last_tag);
      }
      for (; kt < nk; ++kt) {
        wait_for(kt);
        __builtin_amdgcn_s_barrier();
        if ((kt & 3) == 0 && (kt >> 2) + 1 < ng) issue_g((kt >> 2) + 1);
        slice(kt, std::false_type{}, last_tag);
      }
    };
    if (last) run(std::true_type{});
    else run(std::false_type{});
  }

  // epilogue.  32x32 accumulator layout of the transposed tile: lane l holds
  // token row l & 31 of the sub-tile; register r holds output column
  // 8*(r/4) + 4*(l/32) + r%4 of the 32-column weight tile, so each group of
  // four registers is four consecutive columns: one 8-byte bf16 store, or
  // one 4-byte store of MXFP8 codes.  An MXFP8 output (GEMM1) is quantised
  // per 32 columns: the two lanes l and l^32 hold the 32 columns of a row.
  constexpr int OT = GATED ? HT : NT;  // output tiles per wave
  constexpr bool QOUT = MX && GATED;   // h is stored as MXFP8
  // bf16 outputs go through LDS (the ring is free once every wave is past
  // the last slice): each wave writes its tiles there, then the block stores
  // whole rows, 16 bytes per lane with consecutive lanes on consecutive
  // chunks, so each store instruction writes full cache lines instead of 16
  // bytes of 32 different rows.  Rows are padded by 16 bytes (bank spread).
  constexpr int OC = GATED ? C::BNW / 2 : C::BNW;  // output columns of an item
  constexpr int RSB = OC * 2 + 16;                 // bytes per staged row
  constexpr bool STAGE = !QOUT && C::BM * RSB <= C::LDS_BYTES;
  if (STAGE) __builtin_amdgcn_s_barrier();
#pragma unroll
  for (int i = 0; i < MS; ++i) {
    if (i == MS - 1 && !last) continue;
    const int row = (i * C::RG + rg) * 32 + fr;
    const bool live = row < it.nrows;
    const size_t orow = (size_t)(it.row0 + row);
#pragma unroll
    for (int j = 0; j < OT; ++j) {
      const int c0 = n0 + (cg * OT + j) * 32;  // Nout is a multiple of 32
      if (c0 >= Nout) continue;
      float v[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float gv = acc[i][j][r];
        if (GATED) {
          const float uv = acc[i][j + HT][r];
          v[r] = gv / (1.0f + expf(-gv)) * uv;
        } else {
          v[r] = gv;
        }
      }
      if (QOUT) {
        float amax = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float a = fabsf(v[r]);
          amax = a > amax ? a : amax;
        }
        const float o = __shfl_xor(amax, 32, 64);
        amax = o > amax ? o : amax;
        const int X = mx_shared_exp(amax);
        if (live) {
          unsigned char* crow = Cm + orow * Nout;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t pk = e4m3_code(v[4 * q], X) | (e4m3_code(v[4 * q + 1], X) << 8) |
                                (e4m3_code(v[4 * q + 2], X) << 16) |
                                (e4m3_code(v[4 * q + 3], X) << 24);
            *reinterpret_cast<uint32_t*>(crow + c0 + 8 * q + 4 * fh) = pk;
          }
          if (fh == 0)
            (shared ? g.cs_shared : g.cs_routed)[orow * (Nout / kMxBlock) + c0 / kMxBlock] =
                (unsigned char)(X + 127);
        }
      } else if (STAGE || live) {
        bf16_t* crow = reinterpret_cast<bf16_t*>(Cm) + orow * Nout;
        if (!GATED && g.addend && live) {
          const bf16_t* arow = reinterpret_cast<const bf16_t*>(g.addend) + orow * Nout;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const u32x2_t ad = *reinterpret_cast<const u32x2_t*>(arow + c0 + 8 * q + 4 * fh);
            v[4 * q] += __uint_as_float(ad[0] << 16);
            v[4 * q + 1] += __uint_as_float(ad[0] & 0xFFFF0000u);
            v[4 * q + 2] += __uint_as_float(ad[1] << 16);
            v[4 * q + 3] += __uint_as_float(ad[1] & 0xFFFF0000u);
          }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          u32x2_t pk;
          pk[0] = (uint32_t)f32_to_bf16(v[4 * q]) | ((uint32_t)f32_to_bf16(v[4 * q + 1]) << 16);
          pk[1] = (uint32_t)f32_to_bf16(v[4 * q + 2]) | ((uint32_t)f32_to_bf16(v[4 * q + 3]) << 16);
          if (STAGE)
            *reinterpret_cast<u32x2_t*>(lds + row * RSB + ((c0 - n0) + 8 * q + 4 * fh) * 2) = pk;
          else
            *reinterpret_cast<u32x2_t*>(crow + c0 + 8 * q + 4 * fh) = pk;
        }
      }
    }
  }
  if (STAGE) {
    __syncthreads();
    constexpr int CH = OC / 8;  // 16-byte chunks per staged row
    const int live_ch = min(OC, Nout - n0) / 8;
    const int nch = it.nrows * CH;
    for (int q = tid; q < nch; q += C::THREADS) {
      const int r = q / CH, ch = q - r * CH;
      if (ch < live_ch) {
        const i32x4_t v = *reinterpret_cast<const i32x4_t*>(lds + r * RSB + ch * 16);
        *reinterpret_cast<i32x4_t*>(Cm + ((size_t)(it.row0 + r) * Nout + n0 + ch * 8) * 2) = v;
      }
    }
  }
}

// Work distribution.  Block b runs on XCD b % 8 (the hardware deals blocks
// round-robin over the XCDs).  One block per CU takes items of its XCD's
// equal-cost range from a per-XCD counter, so siblings that share a weight
// slab or a row block run close together on one L2; an item's result does
// not depend on which block computes it.

template <bool GATED, bool MX, class C>
__device__ __forceinline__ void gemm_item(const GemmArgs& g, int item, unsigned char* lds) {
  // the item is the same for the whole block: keep its fields (and every
  // base pointer derived from them) in scalar registers
  const WorkItem ld = g.items[item];
  const WorkItem it{__builtin_amdgcn_readfirstlane(ld.seg), __builtin_amdgcn_readfirstlane(ld.row0),
                    __builtin_amdgcn_readfirstlane(ld.nrows), __builtin_amdgcn_readfirstlane(ld.nt)};
  const int msub = (it.nrows + 31) >> 5;  // live 32-row sub-tiles
  const int ms = (msub + C::RG - 1) / C::RG;  // sub-tiles of the busiest wave
  // instances with 1, 2, 3 and MSW sub-tiles per wave, rounded up to MSQ
  constexpr int Q = C::MSQ;
  constexpr int M1 = Q, M2 = C::MSW < 2 ? C::MSW : (2 + Q - 1) / Q * Q;
  constexpr int M3 = C::MSW < 3 ? C::MSW : (3 + Q - 1) / Q * Q;
  constexpr int M4 = C::MSW < 4 ? C::MSW : (4 + Q - 1) / Q * Q;
  constexpr int M5 = C::MSW < 5 ? C::MSW : (5 + Q - 1) / Q * Q;
  if (ms <= 1) gemm_body<GATED, MX, C, M1>(g, it, lds, msub);
  else if (ms <= 2) gemm_body<GATED, MX, C, M2>(g, it, lds, msub);
  else if (ms <= 3) gemm_body<GATED, MX, C, M3>(g, it, lds, msub);
  else if (C::MSW > 4 && ms <= 4) gemm_body<GATED, MX, C, M4>(g, it, lds, msub);
  else if (C::MSW > 5 && ms <= 5) gemm_body<GATED, MX, C, M5>(g, it, lds, msub);
  else gemm_body<GATED, MX, C, C::MSW>(g, it, lds, msub);
}

template <bool GATED, bool MX, class C>
__global__ __launch_bounds__(C::THREADS)
__attribute__((amdgpu_waves_per_eu(C::WAVES * C::BLOCKS_PER_CU / 4 > 0 ? C::WAVES * C::BLOCKS_PER_CU / 4 : 1))) void gemm_mfma_kernel(
    GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[C::LDS_BYTES];
  int& s_item = *reinterpret_cast<int*>(lds);  // LDS is idle between items
  const int x = blockIdx.x & 7;
  const int beg = g.hdr[kHdrStart + x], end = g.hdr[kHdrStart + x + 1];
  for (;;) {
    __syncthreads();  // every wave is done with the previous item's LDS
    if (threadIdx.x == 0) s_item = beg + atomicAdd(&g.hdr[kHdrCtr + x], 1);
    __syncthreads();
    const int item = __builtin_amdgcn_readfirstlane(s_item);
    __syncthreads();  // read before the next DMA overwrites it
    if (item >= end) break;
    gemm_item<GATED, MX, C>(g, item, lds);
  }
  // the last block out re-arms the item counters, so the same work list can
  // be launched again without rebuilding it (every other block has already
  // drawn its final item)
  if (threadIdx.x == 0 && atomicAdd(&g.hdr[kHdrDone], 1) == (int)gridDim.x - 1) {
    for (int i = 0; i < 8; ++i) atomicExch(&g.hdr[kHdrCtr + i], 0);
    atomicExch(&g.hdr[kHdrDone], 0);
  }
}

// ---------------------------------------------------------------------------
// fp32 VALU grouped GEMM (fp32 layers): 32 rows x 32 columns per work item.
// ---------------------------------------------------------------------------
struct GemmArgsF {
  const float* a_routed;
  const float* a_shared;
  const int32_t* perm;
  int k;
  const float* b_routed;
  const float* b_shared;
  float* c_routed;
  float* c_shared;
  int K_r, K_s, Nout_r, Nout_s;
  long long b_stride;
  int N;
  const WorkItem* items;
  const int32_t* hdr;
  const float* addend;  // plain products: [rows, Nout] added to the result (or NULL)
};

template <bool GATED>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgsF g) {
  constexpr int BK = 32;
  __shared__ float As[kBMf][BK + 1];
  __shared__ float Bg[kBNf][BK + 1];
  __shared__ float Bu[kBNf][BK + 1];
  const int item_id = xcd_item(g.hdr[0]);
  if (item_id < 0) return;
  const WorkItem it = g.items[item_id];
  const bool shared = it.seg == g.N;
  const int K = shared ? g.K_s : g.K_r;
  const int Nout = shared ? g.Nout_s : g.Nout_r;
  const float* A = shared ? g.a_shared : g.a_routed;
  const float* B = shared ? g.b_shared : g.b_routed + (long long)it.seg * g.b_stride;
  float* Cm = shared ? g.c_shared : g.c_routed;
  const int n0 = it.nt * kBNf;
  const int tid = threadIdx.x;
  const int lr = tid >> 3, lk = (tid & 7) * 4;
  int src = it.row0 + min(lr, it.nrows - 1);
  if (g.perm && !shared) src = g.perm[src] / g.k;
  const float* ap = A + (size_t)src * K + lk;
  const int wcol = min(n0 + lr, Nout - 1);
  const float* bgp = B + (size_t)wcol * K + lk;
  const float* bup = B + (size_t)(Nout + wcol) * K + lk;
  const int r = tid >> 3, cq = (tid & 7) * 4;
  float ag[4] = {}, au[4] = {};
  for (int k0 = 0; k0 < K; k0 += BK) {
    float4 a4 = *reinterpret_cast<const float4*>(ap + k0);
    float4 g4 = *reinterpret_cast<const float4*>(bgp + k0);
    As[lr][lk] = a4.x; As[lr][lk + 1] = a4.y; As[lr][lk + 2] = a4.z; As[lr][lk + 3] = a4.w;
    Bg[lr][lk] = g4.x; Bg[lr][lk + 1] = g4.y; Bg[lr][lk + 2] = g4.z; Bg[lr][lk + 3] = g4.w;
    if (GATED) {
      float4 u4 = *reinterpret_cast<const float4*>(bup + k0);
      Bu[lr][lk] = u4.x; Bu[lr][lk + 1] = u4.y; Bu[lr][lk + 2] = u4.z; Bu[lr][lk + 3] = u4.w;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < BK; ++kk) {
      const float a = As[r][kk];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        ag[c] = fmaf(a, Bg[cq + c][kk], ag[c]);
        if (GATED) au[c] = fmaf(a, Bu[cq + c][kk], au[c]);
      }
    }
    __syncthreads();
  }
  if (r < it.nrows) {
    float* crow = Cm + (size_t)(it.row0 + r) * Nout;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int col = n0 + cq + c;
      if (col >= Nout) continue;
      crow[col] = GATED ? ag[c] / (1.0f + expf(-ag[c])) * au[c]
                        : ag[c] + (g.addend ? g.addend[(size_t)(it.row0 + r) * Nout + col] : 0.f);
    }
  }
}

inline int cdiv(long long a, long long b) { return (int)((a + b - 1) / b); }

// persistent blocks: per compute unit, a multiple of the 8 XCDs.  The CU
// count of a device is read once and kept in an atomic (every thread that
// races on the first call stores the same value)
int persistent_grid(int per_cu) {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    n = (cus + 7) / 8 * 8;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n * per_cu;
}

template <bool GATED, bool MX, class C>
void launch_mfma(const GemmArgs& g, int64_t cap, hipStream_t st) {
  (void)cap;
  const int grid = persistent_grid(C::BLOCKS_PER_CU);
  gemm_mfma_kernel<GATED, MX, C><<<grid, C::THREADS, 0, st>>>(g);
}

bool narrow_tiles(const moe_shape& s) {
  return s.dtype != MOE_DTYPE_F32 && s.T * s.top_k <= (long long)kNarrowRows * s.n_experts &&
         s.d_ff_shared == 0;
}

typedef const unsigned char* cbytes;
typedef unsigned char* bytes;
inline cbytes cb(const void* p) { return static_cast<cbytes>(p); }
inline bytes mb(void* p) { return static_cast<bytes>(p); }
// scale bytes of a packed MX matrix with `elems` codes (NULL stays NULL)
inline cbytes mx_sc(const void* p, size_t elems) { return p ? cb(p) + elems : nullptr; }
inline bytes mx_sc(void* p, size_t elems) { return p ? mb(p) + elems : nullptr; }

template <bool GATED, bool MX>
void launch_tiles(bool narrow, const GemmArgs& g, int64_t cap, hipStream_t st) {
  using Wide = typename std::conditional<MX, typename std::conditional<GATED, Cfg1x, Cfg2x>::type,
                                         typename std::conditional<GATED, Cfg1, Cfg2>::type>::type;
  using Narrow =
      typename std::conditional<MX, typename std::conditional<GATED, Cfg1nx, Cfg2nx>::type,
                                typename std::conditional<GATED, Cfg1n, Cfg2n>::type>::type;
  if (narrow)
    launch_mfma<GATED, MX, Narrow>(g, cap, st);
  else
    launch_mfma<GATED, MX, Wide>(g, cap, st);
}

struct PlanGeom {
  int bm1, bm2, nt1_r, nt1_s, nt2_r, nt2_s;
};

// row-block size and column-tile counts of the two work lists
PlanGeom plan_geom(const moe_shape& s) {
  const bool bf = s.dtype != MOE_DTYPE_F32;  // bf16 or MXFP8 MFMA tiles
  const bool nar = narrow_tiles(s);
  const bool mx = s.dtype == MOE_DTYPE_MXFP8;
  const int bm1 = bf ? (nar ? (mx ? Cfg1nx::BM : Cfg1n::BM) : mx ? Cfg1x::BM : Cfg1::BM) : kBMf;
  const int bm2 = bf ? (nar ? (mx ? Cfg2nx::BM : Cfg2n::BM) : mx ? Cfg2x::BM : Cfg2::BM) : kBMf;
  const int bn1 =
      bf ? (nar ? (mx ? Cfg1nx::BNW : Cfg1n::BNW) : mx ? Cfg1x::BNW : Cfg1::BNW) / 2 : kBNf;
  const int bn2 = bf ? (nar ? (mx ? Cfg2nx::BNW : Cfg2n::BNW) : mx ? Cfg2x::BNW : Cfg2::BNW) : kBNf;
  const bool sh = s.d_ff_shared > 0;
  return PlanGeom{bm1, bm2, cdiv(s.d_ff, bn1), sh ? cdiv(s.d_ff_shared, bn1) : 0,
                  cdiv(s.d_model, bn2), sh ? cdiv(s.d_model, bn2) : 0};
}

}  // namespace

PlanArgs plan_args(const moe_shape& s, const int32_t* offsets, const Workspace& w) {
  const int fs = s.d_ff_shared;
  const PlanGeom pg = plan_geom(s);
  return PlanArgs{offsets, s.n_experts, (int)s.T, fs > 0 ? 1 : 0, pg.bm1, pg.bm2, pg.nt1_r,
                  pg.nt1_s, pg.nt2_r, pg.nt2_s, s.d_model, s.d_model, s.d_ff, fs > 0 ? fs : 64,
                  w.plan1, w.plan1_hdr, w.plan2, w.plan2_hdr, narrow_tiles(s) ? 0 : 1};
}

hipError_t launch_plan(const moe_shape& s, const int32_t* offsets, const Workspace& w,
                       hipStream_t st) {
  plan_kernel<<<2, 1024, 0, st>>>(plan_args(s, offsets, w));
  return hipGetLastError();
}

// h = silu(x W_gate^T) * (x W_up^T) over the work list built by launch_plan.
// MXFP8 layers: x is quantised into the workspace first, w1 / w1s / h / hs
// are packed MX matrices (codes, then scales).
hipError_t launch_gemm1(const moe_shape& s, const void* x, const int32_t* perm, const void* w1,
                        const void* w1s, void* h, void* hs, const Workspace& w,
                        hipStream_t st) {
  const int N = s.n_experts, d = s.d_model, f = s.d_ff, fs = s.d_ff_shared;
  const size_t T = (size_t)s.T, A = T * s.top_k;
  if (s.dtype == MOE_DTYPE_BF16) {
    GemmArgs g1{cb(x), cb(x), perm, s.top_k, cb(w1), cb(w1s), mb(h), mb(hs),
                nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                d, d, f, fs, (long long)2 * f * d, N, w.plan1, w.plan1_hdr};
    launch_tiles<true, false>(narrow_tiles(s), g1, w.plan1_cap, st);
  } else if (s.dtype == MOE_DTYPE_MXFP8) {
    hipError_t e = launch_mx_quantize(x, MOE_DTYPE_BF16, s.T, d, w.xq, w.xq + T * d, st);
    if (e != hipSuccess) return e;
    const unsigned char* xs = w.xq + T * d;
    GemmArgs g1{w.xq, w.xq, perm, s.top_k, cb(w1), cb(w1s), mb(h), mb(hs),
                xs, xs, mx_sc(w1, (size_t)N * 2 * f * d), mx_sc(w1s, (size_t)2 * fs * d),
                mx_sc(h, A * f), mx_sc(hs, T * fs),
                d, d, f, fs, (long long)2 * f * d, N, w.plan1, w.plan1_hdr, nullptr,
                (int)T, (int)T};
    launch_tiles<true, true>(narrow_tiles(s), g1, w.plan1_cap, st);
  } else {
    GemmArgsF g1{static_cast<const float*>(x), static_cast<const float*>(x), perm, s.top_k,
                 static_cast<const float*>(w1), static_cast<const float*>(w1s),
                 static_cast<float*>(h), static_cast<float*>(hs), d, d, f, fs,
                 (long long)2 * f * d, N, w.plan1, w.plan1_hdr};
    gemm_f32_kernel<true><<<(int)((w.plan1_cap + 7) / 8 * 8), 256, 0, st>>>(g1);
  }
  return hipGetLastError();
}

// y_perm = h W2^T (and y_shared = h_shared W2s^T) over the second work list
hipError_t launch_gemm2(const moe_shape& s, const void* h, const void* hs, const void* w2,
                        const void* w2s, void* y_perm, void* y_shared, const Workspace& w,
                        hipStream_t st) {
  const int N = s.n_experts, d = s.d_model, f = s.d_ff, fs = s.d_ff_shared;
  const size_t T = (size_t)s.T, A = T * s.top_k;
  if (s.dtype != MOE_DTYPE_F32) {
    const bool mx = s.dtype == MOE_DTYPE_MXFP8;
    GemmArgs g2{cb(h), cb(hs), nullptr, s.top_k, cb(w2), cb(w2s), mb(y_perm), mb(y_shared),
                mx ? mx_sc(h, A * f) : nullptr, mx ? mx_sc(hs, T * fs) : nullptr,
                mx ? mx_sc(w2, (size_t)N * d * f) : nullptr,
                mx ? mx_sc(w2s, (size_t)d * fs) : nullptr, nullptr, nullptr,
                f, fs, d, d, (long long)d * f, N, w.plan2, w.plan2_hdr, nullptr,
                (int)A, (int)T};
    if (mx)
      launch_tiles<false, true>(narrow_tiles(s), g2, w.plan2_cap, st);
    else
      launch_tiles<false, false>(narrow_tiles(s), g2, w.plan2_cap, st);
  } else {
    GemmArgsF g2{static_cast<const float*>(h), static_cast<const float*>(hs), nullptr,
                 s.top_k, static_cast<const float*>(w2), static_cast<const float*>(w2s),
                 static_cast<float*>(y_perm), static_cast<float*>(y_shared), f, fs, d, d,
                 (long long)d * f, N, w.plan2, w.plan2_hdr};
    gemm_f32_kernel<false><<<(int)((w.plan2_cap + 7) / 8 * 8), 256, 0, st>>>(g2);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Dense products over all T rows (the LatentMoE projections and a shared
// expert run on its own): one segment in the shared-expert slot of the work
// lists (N = 0), the same kernels as the expert projections.
// ---------------------------------------------------------------------------
namespace {
bool dense_narrow(const moe_shape& s) { return s.dtype != MOE_DTYPE_F32 && s.T <= kNarrowRows; }
int dense_bm(const moe_shape& s) {
  if (s.dtype == MOE_DTYPE_F32) return kBMf;
  return dense_narrow(s) ? Cfg2n::BM : Cfg2::BM;
}
// output columns per item of a gated / plain product
int dense_bn(const moe_shape& s, bool gated) {
  if (s.dtype == MOE_DTYPE_F32) return kBNf;
  const bool n = dense_narrow(s);
  return gated ? (n ? Cfg1n::BNW : Cfg1::BNW) / 2 : (n ? Cfg2n::BNW : Cfg2::BNW);
}
}  // namespace

int64_t dense_plan_cap(const moe_shape& s, int Nout, bool gated) {
  return (int64_t)cdiv(s.T, dense_bm(s)) * cdiv(Nout, dense_bn(s, gated));
}

// list 1 (gated or plain, Nout1 columns, reduction K1) and, when p2 is given,
// list 2 (plain, Nout2 columns, reduction K2) of dense products over T rows
hipError_t launch_dense_plan(const moe_shape& s, bool gated1, int K1, int Nout1, WorkItem* p1,
                             int32_t* h1, int K2, int Nout2, WorkItem* p2, int32_t* h2,
                             hipStream_t st) {
  const int bm = dense_bm(s);
  const int n1 = cdiv(Nout1, dense_bn(s, gated1));
  const int n2 = p2 ? cdiv(Nout2, dense_bn(s, false)) : 0;
  plan_kernel<<<p2 ? 2 : 1, 1024, 0, st>>>(PlanArgs{nullptr, 0, (int)s.T, 1, bm, bm, 0, n1, 0,
                                                    n2, K1, K1, p2 ? K2 : 64, p2 ? K2 : 64, p1,
                                                    h1, p2, h2, 0});
  return hipGetLastError();
}

// C [T, Nout] = A [T, K] B^T (gated: SwiGLU of the gate and up halves of B,
// Nout h columns; plain: plus `addend` when given), over a list built by
// launch_dense_plan with the same geometry
hipError_t launch_dense(const moe_shape& s, bool gated, const void* a, const void* b, void* c,
                        const void* addend, int K, int Nout, const WorkItem* plan, int32_t* hdr,
                        int64_t cap, hipStream_t st) {
  if (s.dtype == MOE_DTYPE_F32) {
    GemmArgsF g{static_cast<const float*>(a), static_cast<const float*>(a), nullptr, 1,
                static_cast<const float*>(b), static_cast<const float*>(b),
                static_cast<float*>(c), static_cast<float*>(c), K, K, Nout, Nout, 0, 0, plan,
                hdr, static_cast<const float*>(addend)};
    if (gated)
      gemm_f32_kernel<true><<<(int)((cap + 7) / 8 * 8), 256, 0, st>>>(g);
    else
      gemm_f32_kernel<false><<<(int)((cap + 7) / 8 * 8), 256, 0, st>>>(g);
    return hipGetLastError();
  }
  if (s.dtype != MOE_DTYPE_BF16) return hipErrorInvalidValue;
  GemmArgs g{cb(a), cb(a), nullptr, 1, cb(b), cb(b), mb(c), mb(c),
             nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
             K, K, Nout, Nout, 0, 0, plan, hdr, cb(addend)};
  if (gated)
    launch_tiles<true, false>(dense_narrow(s), g, cap, st);
  else
    launch_tiles<false, false>(dense_narrow(s), g, cap, st);
  return hipGetLastError();
}

// work-list capacities for a shape (upper bounds of the plan sizes)
void plan_caps(const moe_shape& s, int64_t& cap1, int64_t& cap2) {
  const PlanGeom pg = plan_geom(s);
  const int64_t A = s.T * s.top_k;
  const int64_t mt1 = (A + pg.bm1 - 1) / pg.bm1 + s.n_experts;
  const int64_t mt2 = (A + pg.bm2 - 1) / pg.bm2 + s.n_experts;
  const int64_t ms1 = s.d_ff_shared > 0 ? (s.T + pg.bm1 - 1) / pg.bm1 : 0;
  const int64_t ms2 = s.d_ff_shared > 0 ? (s.T + pg.bm2 - 1) / pg.bm2 : 0;
  cap1 = mt1 * pg.nt1_r + ms1 * pg.nt1_s;
  cap2 = mt2 * pg.nt2_r + ms2 * pg.nt2_s;
}

}  // namespace moe
