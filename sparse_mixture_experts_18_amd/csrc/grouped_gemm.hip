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
// bf16 path: v_mfma_f32_32x32x16_bf16, fp32 accumulation, 128-row work items,
// both operands K-contiguous (weights in nn.Linear [out, in] layout), staged
// through LDS with an XOR swizzle of the 16-byte chunks.  The work list
// (segment, row block, column tile) is built on the device from the dispatch
// offsets, so no host synchronisation is needed; blocks are mapped so that
// each XCD walks a contiguous run of the list (same expert, same weight
// slab), which keeps that slab in the XCD's L2 across the row blocks.
#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// work-list construction
// ---------------------------------------------------------------------------
__device__ __forceinline__ void block_exclusive_scan2(int* sh0, int* sh1, int v0, int v1,
                                                      int& ex0, int& ex1, int& tot0,
                                                      int& tot1) {
  const int i = threadIdx.x, n = blockDim.x;
  sh0[i] = v0;
  sh1[i] = v1;
  __syncthreads();
  for (int o = 1; o < n; o <<= 1) {
    int a = i >= o ? sh0[i - o] : 0;
    int b = i >= o ? sh1[i - o] : 0;
    __syncthreads();
    sh0[i] += a;
    sh1[i] += b;
    __syncthreads();
  }
  ex0 = sh0[i] - v0;
  ex1 = sh1[i] - v1;
  tot0 = sh0[n - 1];
  tot1 = sh1[n - 1];
}

__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* __restrict__ offsets, int N,
                                                    int T, int has_shared, int bm, int nt1_r,
                                                    int nt1_s, int nt2_r, int nt2_s,
                                                    WorkItem* __restrict__ plan1,
                                                    int32_t* __restrict__ count1,
                                                    WorkItem* __restrict__ plan2,
                                                    int32_t* __restrict__ count2) {
  __shared__ int sh0[1024], sh1[1024];
  const int s = threadIdx.x;
  const int S = N + has_shared;
  int rows = 0, rbase = 0, n1t = 0, n2t = 0;
  if (s < N) {
    rbase = offsets[s];
    rows = offsets[s + 1] - rbase;
    n1t = nt1_r;
    n2t = nt2_r;
  } else if (s < S) {
    rows = T;
    n1t = nt1_s;
    n2t = nt2_s;
  }
  const int mt = (rows + bm - 1) / bm;
  int st1, st2, tot1, tot2;
  block_exclusive_scan2(sh0, sh1, mt * n1t, mt * n2t, st1, st2, tot1, tot2);
  for (int nt = 0; nt < n1t; ++nt)
    for (int m = 0; m < mt; ++m)
      plan1[st1 + nt * mt + m] = WorkItem{s, rbase + m * bm, min(bm, rows - m * bm), nt};
  for (int nt = 0; nt < n2t; ++nt)
    for (int m = 0; m < mt; ++m)
      plan2[st2 + nt * mt + m] = WorkItem{s, rbase + m * bm, min(bm, rows - m * bm), nt};
  if (s == 0) {
    *count1 = tot1;
    *count2 = tot2;
  }
}

// XCD-aware item index: the hardware deals blocks round-robin over the 8
// XCDs, so block b runs on XCD b % 8.  Give XCD x the contiguous item range
// [x*per, (x+1)*per).  Returns -1 for blocks without work.
__device__ __forceinline__ int xcd_item(int count) {
  const int per = (count + 7) >> 3;
  const int b = blockIdx.x;
  const int local = b >> 3, x = b & 7;
  if (local >= per) return -1;
  const int item = x * per + local;
  return item < count ? item : -1;
}

struct GemmArgs {
  const bf16_t* a_routed;  // GEMM1: x [T, d]       GEMM2: h [T*k, d_ff]
  const bf16_t* a_shared;  // GEMM1: x [T, d]       GEMM2: h_shared [T, d_ffs]
  const int32_t* perm;     // GEMM1: row -> token via perm[row] / k; GEMM2: null
  int k;
  const bf16_t* b_routed;  // GEMM1: w1 [N][2*d_ff][d]  GEMM2: w2 [N][d][d_ff]
  const bf16_t* b_shared;
  bf16_t* c_routed;        // GEMM1: h              GEMM2: y_perm
  bf16_t* c_shared;        // GEMM1: h_shared       GEMM2: y_shared
  int K_r, K_s;            // reduction length
  int Nout_r, Nout_s;      // output columns (h columns for GEMM1)
  long long b_stride;      // elements per routed expert weight matrix
  int N;
  const WorkItem* items;
  const int32_t* count;
};

// ---------------------------------------------------------------------------
// bf16 MFMA grouped GEMM.  Block tile 128 rows x 256 weight rows x 64 k,
// 4 waves in 2x2, each wave 64 rows x 4 column tiles of 32 (GATED: 2 gate +
// 2 up tiles covering the same 64 h columns).
// ---------------------------------------------------------------------------
constexpr int G_BM = 128, G_BNW = 256, G_BK = 64;

__device__ __forceinline__ void gload_tile(u32x4_t (&ra)[4], u32x4_t (&rb)[8],
                                           const bf16_t* __restrict__ A,
                                           const bf16_t* __restrict__ B,
                                           const uint32_t (&a_off)[4],
                                           const uint32_t (&b_off)[8], int k0) {
#pragma unroll
  for (int i = 0; i < 4; ++i) ra[i] = *reinterpret_cast<const u32x4_t*>(A + a_off[i] + k0);
#pragma unroll
  for (int i = 0; i < 8; ++i) rb[i] = *reinterpret_cast<const u32x4_t*>(B + b_off[i] + k0);
}

// one BK slice of the block tile: 4 k-steps of 16, 2 x 4 MFMA 32x32x16 per wave
__device__ __forceinline__ void mma_tile(f32x16_t (&acc)[2][4], const unsigned char* As,
                                         const unsigned char* Bs, const int (&a_row)[2],
                                         const int (&b_row)[4], int fh) {
#pragma unroll
  for (int ks = 0; ks < G_BK / 16; ++ks) {
    const int ch = 2 * ks + fh;
    bf16x8_t af[2], bf[4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
      af[i] = *reinterpret_cast<const bf16x8_t*>(As + a_row[i] * (G_BK * 2) +
                                                 ((ch ^ (a_row[i] & 7)) << 4));
#pragma unroll
    for (int j = 0; j < 4; ++j)
      bf[j] = *reinterpret_cast<const bf16x8_t*>(Bs + b_row[j] * (G_BK * 2) +
                                                 ((ch ^ (b_row[j] & 7)) << 4));
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
  }
}

__device__ __forceinline__ void lstore_tile(const u32x4_t (&ra)[4], const u32x4_t (&rb)[8],
                                            unsigned char* As, unsigned char* Bs, int lds_off) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *reinterpret_cast<u32x4_t*>(As + lds_off + i * 32 * G_BK * 2) = ra[i];
#pragma unroll
  for (int i = 0; i < 8; ++i)
    *reinterpret_cast<u32x4_t*>(Bs + lds_off + i * 32 * G_BK * 2) = rb[i];
}

template <bool GATED>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[(G_BM + G_BNW) * G_BK * 2];
  unsigned char* As = lds;
  unsigned char* Bs = lds + G_BM * G_BK * 2;

  const int item_id = xcd_item(*g.count);
  if (item_id < 0) return;
  const WorkItem it = g.items[item_id];
  const bool shared = it.seg == g.N;
  const int K = shared ? g.K_s : g.K_r;
  const int Nout = shared ? g.Nout_s : g.Nout_r;
  const bf16_t* A = shared ? g.a_shared : g.a_routed;
  const bf16_t* B = shared ? g.b_shared : g.b_routed + (long long)it.seg * g.b_stride;
  bf16_t* Cm = shared ? g.c_shared : g.c_routed;
  const int n0 = it.nt * (GATED ? G_BNW / 2 : G_BNW);

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;

  // loader geometry: rows (tid>>3) + 32 i, 16-byte chunk tid&7
  const int lrow = tid >> 3, lcc = tid & 7;
  const int lds_off = lrow * (G_BK * 2) + ((lcc ^ (lrow & 7)) << 4);
  uint32_t a_off[4], b_off[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int r = min(lrow + 32 * i, it.nrows - 1);
    int src = it.row0 + r;
    if (g.perm && !shared) src = g.perm[src] / g.k;
    a_off[i] = (uint32_t)src * (uint32_t)K + lcc * 8;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int r = lrow + 32 * i;
    int wrow;
    if (GATED) {
      wrow = r < G_BNW / 2 ? min(n0 + r, Nout - 1) : Nout + min(n0 + r - G_BNW / 2, Nout - 1);
    } else {
      wrow = min(n0 + r, Nout - 1);
    }
    b_off[i] = (uint32_t)wrow * (uint32_t)K + lcc * 8;
  }

  f32x16_t acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  u32x4_t ra[4], rb[8];
  // fragment geometry: row (lane & 31) of a 32-row tile, chunk 2*ks + (lane >> 5)
  const int fr = lane & 31, fh = lane >> 5;
  int a_row[2], b_row[4];
#pragma unroll
  for (int i = 0; i < 2; ++i) a_row[i] = wm * 64 + i * 32 + fr;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (GATED)
      b_row[j] = (j < 2 ? wn * 64 + j * 32 : G_BNW / 2 + wn * 64 + (j - 2) * 32) + fr;
    else
      b_row[j] = wn * 128 + j * 32 + fr;
  }

  const int nk = K / G_BK;
  gload_tile(ra, rb, A, B, a_off, b_off, 0);
  lstore_tile(ra, rb, As, Bs, lds_off);
  __syncthreads();
  for (int kt = 1; kt < nk; ++kt) {
    gload_tile(ra, rb, A, B, a_off, b_off, kt * G_BK);  // in flight during the MFMAs
    mma_tile(acc, As, Bs, a_row, b_row, fh);
    __syncthreads();
    lstore_tile(ra, rb, As, Bs, lds_off);
    __syncthreads();
  }
  mma_tile(acc, As, Bs, a_row, b_row, fh);

  // epilogue.  32x32 accumulator layout: column = lane & 31,
  // row = 8*(r/4) + 4*(lane/32) + r%4 for register r.
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * fh + (r & 3);
      if (row >= it.nrows) continue;
      bf16_t* crow = Cm + (size_t)(it.row0 + row) * Nout;
      if (GATED) {
#pragma unroll
        for (int jn = 0; jn < 2; ++jn) {
          const int col = n0 + wn * 64 + jn * 32 + fr;
          const float gv = acc[i][jn][r], uv = acc[i][jn + 2][r];
          const float hv = gv / (1.0f + expf(-gv)) * uv;
          if (col < Nout) crow[col] = f32_to_bf16(hv);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = n0 + wn * 128 + j * 32 + fr;
          if (col < Nout) crow[col] = f32_to_bf16(acc[i][j][r]);
        }
      }
    }
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
  const int32_t* count;
};

template <bool GATED>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgsF g) {
  constexpr int BK = 32;
  __shared__ float As[kBMf][BK + 1];
  __shared__ float Bg[kBNf][BK + 1];
  __shared__ float Bu[kBNf][BK + 1];
  const int item_id = xcd_item(*g.count);
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
      crow[col] = GATED ? ag[c] / (1.0f + expf(-ag[c])) * au[c] : ag[c];
    }
  }
}

inline int cdiv(long long a, long long b) { return (int)((a + b - 1) / b); }

}  // namespace

hipError_t launch_expert_ffn(const moe_shape& s, const void* x, const int32_t* perm,
                             const int32_t* offsets, const void* w1, const void* w2,
                             const void* w1s, const void* w2s, void* y_perm, void* y_shared,
                             const Workspace& w, hipStream_t st) {
  const int T = (int)s.T, N = s.n_experts, d = s.d_model, f = s.d_ff, fs = s.d_ff_shared;
  const bool bf = s.dtype == MOE_DTYPE_BF16;
  const int has_shared = fs > 0 ? 1 : 0;
  const int bm = bf ? G_BM : kBMf;
  const int bn1 = bf ? G_BNW / 2 : kBNf, bn2 = bf ? G_BNW : kBNf;
  const int nt1_r = cdiv(f, bn1), nt1_s = has_shared ? cdiv(fs, bn1) : 0;
  const int nt2_r = cdiv(d, bn2), nt2_s = has_shared ? cdiv(d, bn2) : 0;
  plan_kernel<<<1, 1024, 0, st>>>(offsets, N, T, has_shared, bm, nt1_r, nt1_s, nt2_r, nt2_s,
                                  w.plan1, w.plan1_count, w.plan2, w.plan2_count);
  const int grid1 = (int)((w.plan1_cap + 7) / 8 * 8), grid2 = (int)((w.plan2_cap + 7) / 8 * 8);
  if (bf) {
    GemmArgs g1{static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(x), perm, s.top_k,
                static_cast<const bf16_t*>(w1), static_cast<const bf16_t*>(w1s),
                static_cast<bf16_t*>(w.h), static_cast<bf16_t*>(w.h_shared), d, d, f, fs,
                (long long)2 * f * d, N, w.plan1, w.plan1_count};
    gemm_bf16_kernel<true><<<grid1, 256, 0, st>>>(g1);
    GemmArgs g2{static_cast<const bf16_t*>(w.h), static_cast<const bf16_t*>(w.h_shared),
                nullptr, s.top_k, static_cast<const bf16_t*>(w2),
                static_cast<const bf16_t*>(w2s), static_cast<bf16_t*>(y_perm),
                static_cast<bf16_t*>(y_shared), f, fs, d, d, (long long)d * f, N, w.plan2,
                w.plan2_count};
    gemm_bf16_kernel<false><<<grid2, 256, 0, st>>>(g2);
  } else {
    GemmArgsF g1{static_cast<const float*>(x), static_cast<const float*>(x), perm, s.top_k,
                 static_cast<const float*>(w1), static_cast<const float*>(w1s),
                 static_cast<float*>(w.h), static_cast<float*>(w.h_shared), d, d, f, fs,
                 (long long)2 * f * d, N, w.plan1, w.plan1_count};
    gemm_f32_kernel<true><<<grid1, 256, 0, st>>>(g1);
    GemmArgsF g2{static_cast<const float*>(w.h), static_cast<const float*>(w.h_shared),
                 nullptr, s.top_k, static_cast<const float*>(w2),
                 static_cast<const float*>(w2s), static_cast<float*>(y_perm),
                 static_cast<float*>(y_shared), f, fs, d, d, (long long)d * f, N, w.plan2,
                 w.plan2_count};
    gemm_f32_kernel<false><<<grid2, 256, 0, st>>>(g2);
  }
  return hipGetLastError();
}

// work-list capacities for a shape (upper bounds of the plan sizes)
void plan_caps(const moe_shape& s, int64_t& cap1, int64_t& cap2) {
  const bool bf = s.dtype == MOE_DTYPE_BF16;
  const int64_t A = s.T * s.top_k;
  const int bm = bf ? G_BM : kBMf;
  const int bn1 = bf ? G_BNW / 2 : kBNf, bn2 = bf ? G_BNW : kBNf;
  const int64_t mt_r = (A + bm - 1) / bm + s.n_experts;
  const int64_t mt_s = s.d_ff_shared > 0 ? (s.T + bm - 1) / bm : 0;
  cap1 = mt_r * ((s.d_ff + bn1 - 1) / bn1) +
         mt_s * (s.d_ff_shared > 0 ? (s.d_ff_shared + bn1 - 1) / bn1 : 0);
  cap2 = mt_r * ((s.d_model + bn2 - 1) / bn2) + mt_s * ((s.d_model + bn2 - 1) / bn2);
}

}  // namespace moe
