// Router: affinity GEMM (fp32) and per-token scores + top-k selection.
//
// Affinity l = x W_r^T with a bias-free gate ("MoE architecture in
// practice", routing-math section; llm-compass MoE page, gate equation).
// Scores: softmax over experts, or an independent sigmoid per expert
// ("MoE common taste of open models", section 7).  Selection on
// key = fl32(s + b) with weights from the raw score (llm-compass MoE page,
// aux-loss-free section; the article's BiasBalancedRouter), optional group
// limit ("MoE industrial evolution", section 4), top-k with ties to the lower
// expert index, renormalised gates.
#include <type_traits>

#include "moe_internal.h"
#include "route_device.h"

namespace moe {
namespace {

// ---------------------------------------------------------------------------
// K1 (fp32 layers): logits[T,N] = x[T,d] . W_r[N,d]^T, fp32 FMA.  Each output is a single
// FMA chain over k = 0..d-1 in order, so a token's logits do not depend on
// the batch it is in.
// ---------------------------------------------------------------------------
constexpr int RT_BM = 64, RT_BN = 64, RT_BK = 16;

__device__ __forceinline__ void load4(const float* p, float* o) {
  float4 v = *reinterpret_cast<const float4*>(p);
  o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
}

__global__ __launch_bounds__(256) void router_gemm_kernel(const float* __restrict__ x,
                                                          const float* __restrict__ w,
                                                          float* __restrict__ logits,
                                                          int T, int N, int d) {
  __shared__ float As[RT_BK][RT_BM + 4];
  __shared__ float Bs[RT_BK][RT_BN + 4];
  const int tid = threadIdx.x;
  const int m0 = blockIdx.x * RT_BM, n0 = blockIdx.y * RT_BN;
  const int lr = tid >> 2, lk = (tid & 3) * 4;  // loader: row, k quad
  const int ty = tid >> 4, tx = tid & 15;       // compute: 4x4 outputs
  const int am = min(m0 + lr, T - 1), bn = min(n0 + lr, N - 1);
  const float* xa = x + (size_t)am * d + lk;
  const float* wb = w + (size_t)bn * d + lk;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < d; k0 += RT_BK) {
    float a4[4], b4[4];
    load4(xa + k0, a4);
    load4(wb + k0, b4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      As[lk + i][lr] = a4[i];
      Bs[lk + i][lr] = b4[i];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < RT_BK; ++kk) {
      float4 a = *reinterpret_cast<const float4*>(&As[kk][ty * 4]);
      float4 b = *reinterpret_cast<const float4*>(&Bs[kk][tx * 4]);
      float av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int m = m0 + ty * 4 + i;
    if (m >= T) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int n = n0 + tx * 4 + j;
      if (n < N) logits[(size_t)m * N + n] = acc[i][j];
    }
  }
}

// ---------------------------------------------------------------------------
// K1, bf16 activations: the same fp32 GEMM on the matrix cores.  x is exactly
// bf16; W_r (fp32) is split into three bf16 terms w = w1 + w2 + w3 with
// w1 = bf16(w), w2 = bf16(w - w1), w3 = bf16(w - w1 - w2), which represent w
// to within 2^-27 |w|.  Every product x*wi is exact in fp32; the three partial
// GEMMs accumulate in fp32 and are summed smallest first (Henry, Tang &
// Heinecke 2019, "Leveraging the bfloat16 AI datatype for higher-precision
// computations").  The k order of every output is fixed, so a token's logits
// do not depend on the batch.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void split3_kernel(const float* __restrict__ w,
                                                     bf16_t* __restrict__ ws, long long n) {
  for (long long i = blockIdx.x * 256LL + threadIdx.x; i < n; i += (long long)gridDim.x * 256) {
    const float v = w[i];
    const bf16_t h1 = f32_to_bf16(v);
    const float r1 = v - bf16_to_f32(h1);
    const bf16_t h2 = f32_to_bf16(r1);
    const float r2 = r1 - bf16_to_f32(h2);
    ws[i] = h1;
    ws[n + i] = h2;
    ws[2 * n + i] = f32_to_bf16(r2);
  }
}

// block: 64 tokens x 64 experts, 4 waves of 32 x 32; k-slices of 64 through
// LDS (rows of 128 bytes, 16-byte chunk c of row r at c ^ ((r >> 1) & 7))
constexpr int RM_BM = 64, RM_BN = 64, RM_BK = 64;

__device__ __forceinline__ int rswz(int r) { return (r >> 1) & 7; }

// The k range is cut into chunks of RM_KC: each chunk's three partial GEMMs
// start from zero, are summed smallest first, and the chunk results are added
// in chunk order.  A block either walks all chunks (out = logits) or, for
// small batches, one chunk (out = partials [chunk][T][N], summed in chunk order
// by the top-k kernel as it reads them): the same fp32 operations in the same order either
// way, so the logits of a token never depend on the batch size.
constexpr int RM_KC = 512;

__global__ __launch_bounds__(256) void router_mfma_kernel(const bf16_t* __restrict__ x,
                                                          const bf16_t* __restrict__ ws,
                                                          float* __restrict__ out, int T,
                                                          int N, int d, int chunks_per_block) {
  __shared__ __attribute__((aligned(16))) unsigned char As[RM_BM * 128];
  __shared__ __attribute__((aligned(16))) unsigned char Bs[3][RM_BN * 128];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int m0 = blockIdx.x * RM_BM, n0 = blockIdx.y * RM_BN;
  const long long plane = (long long)N * d;
  const int nkc = (d + RM_KC - 1) / RM_KC;
  const int c_begin = blockIdx.z * chunks_per_block;
  const int c_end = min(nkc, c_begin + chunks_per_block);
  // loader: 64 rows x 8 chunks = 512 chunks per tile, 2 per thread
  const int lr = tid >> 3, lc = tid & 7;
  const bf16_t* ap[2];
  const bf16_t* bp[2];
  int lofs[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = lr + 32 * i;
    ap[i] = x + (size_t)min(m0 + r, T - 1) * d + lc * 8;
    bp[i] = ws + (size_t)min(n0 + r, N - 1) * d + lc * 8;
    lofs[i] = r * 128 + ((lc ^ rswz(r)) << 4);
  }
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  const int wm = w >> 1, wn = w & 1, fr = lane & 31, fh = lane >> 5;
  const int ar = wm * 32 + fr, br = wn * 32 + fr;
  f32x16_t tot;
  for (int c = c_begin; c < c_end; ++c) {
    f32x16_t acc[3];
#pragma unroll
    for (int t = 0; t < 3; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
    const int k_end = min(d, (c + 1) * RM_KC);
    for (int k0 = c * RM_KC; k0 < k_end; k0 += RM_BK) {
      u32x4_t va[2], vb[3][2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        va[i] = *reinterpret_cast<const u32x4_t*>(ap[i] + k0);
#pragma unroll
        for (int t = 0; t < 3; ++t)
          vb[t][i] = *reinterpret_cast<const u32x4_t*>(bp[i] + t * plane + k0);
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        *reinterpret_cast<u32x4_t*>(As + lofs[i]) = va[i];
#pragma unroll
        for (int t = 0; t < 3; ++t) *reinterpret_cast<u32x4_t*>(Bs[t] + lofs[i]) = vb[t][i];
      }
      __syncthreads();
#pragma unroll
      for (int ks = 0; ks < RM_BK / 16; ++ks) {
        const int ch = 2 * ks + fh;
        const bf16x8_t af =
            *reinterpret_cast<const bf16x8_t*>(As + ar * 128 + ((ch ^ rswz(ar)) << 4));
#pragma unroll
        for (int t = 0; t < 3; ++t) {
          const bf16x8_t bf =
              *reinterpret_cast<const bf16x8_t*>(Bs[t] + br * 128 + ((ch ^ rswz(br)) << 4));
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf, acc[t], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = (acc[2][r] + acc[1][r]) + acc[0][r];
      tot[r] = c == c_begin ? p : tot[r] + p;
    }
  }
  // 32x32 accumulator layout: column = lane & 31, row = 8*(r/4) + 4*(lane/32) + r%4
  float* o = out + (size_t)blockIdx.z * T * N;
  const int col = n0 + wn * 32 + fr;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = m0 + wm * 32 + 8 * (r >> 2) + 4 * fh + (r & 3);
    if (row < T && col < N) o[(size_t)row * N + col] = tot[r];
  }
}

// Small batches: one block per 32 x 32 tile of logits and 512-wide k-chunk
// (the k split), reading the fp32 router weights directly.  The block loads
// the chunk's x rows (32 KiB) and fp32 weights (64 KiB) in one round of
// 16-byte loads, forms the three bf16 parts of each weight with the same
// arithmetic as split3_kernel, and waves 0, 1, 2 each run the MFMA chain of
// one part over the chunk's k-steps in order -- the three accumulators of
// router_mfma_kernel, computed side by side -- so the partial planes are bit
// for bit the ones of the other router kernels.
constexpr int RS_T = 32;  // tile rows and columns
// Each token tile of this kernel splits the weight chunk it uses again, so it
// serves batches of at most two tiles; larger k-split batches split the
// weights once (split3_kernel) and run router_mfma_kernel per chunk (the
// same partial planes).
constexpr int kRouterSmallMaxT = 2 * RS_T;
constexpr int RS_THREADS = 1024;  // sixteen waves: the weight split spread thin
__global__ __launch_bounds__(RS_THREADS) void router_small_kernel(const bf16_t* __restrict__ x,
                                                                  const float* __restrict__ w,
                                                                  float* __restrict__ out, int T,
                                                                  int N, int d) {
  constexpr int SLW = RM_KC / 64;  // 64-wide slices per chunk
  constexpr int XL = RS_T * 64 / RS_THREADS, WL = RS_T * 128 / RS_THREADS;  // loads per thread
  __shared__ __attribute__((aligned(16))) unsigned char As[SLW][RS_T * 128];
  __shared__ __attribute__((aligned(16))) unsigned char Bs[3][SLW][RS_T * 128];
  __shared__ __attribute__((aligned(16))) float red[2][RS_T * RS_T];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int m0 = blockIdx.x * RS_T, n0 = blockIdx.y * RS_T;
  const int c = blockIdx.z;
  const int k0 = c * RM_KC;
  const int nsl = min(SLW, (d - k0) / 64);  // 64-wide slices in this chunk (d % 64 == 0)
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  // coalesced loads: load i of thread t takes 16-byte chunk i * RS_THREADS + t
  // of the tile (x: 32 rows x 64 chunks of 8 bf16; weights: 32 rows x 128
  // chunks of 4 fp32), so a wave reads 1 KiB of one row per instruction
  u32x4_t xa[XL];
  f32x4_t wb[WL];
#pragma unroll
  for (int i = 0; i < XL; ++i) {
    const int g = i * RS_THREADS + tid, r = g >> 6, ch = g & 63;
    const bf16_t* xp = x + (size_t)min(m0 + r, T - 1) * d + k0;
    xa[i] = ch / 8 < nsl ? *reinterpret_cast<const u32x4_t*>(xp + ch * 8) : u32x4_t{0, 0, 0, 0};
  }
#pragma unroll
  for (int i = 0; i < WL; ++i) {
    const int g = i * RS_THREADS + tid, r = g >> 7, ch = g & 127;
    const float* wp = w + (size_t)min(n0 + r, N - 1) * d + k0;
    wb[i] = ch / 16 < nsl ? *reinterpret_cast<const f32x4_t*>(wp + ch * 4) : f32x4_t{0, 0, 0, 0};
  }
#pragma unroll
  for (int i = 0; i < XL; ++i) {
    const int g = i * RS_THREADS + tid, r = g >> 6, ch = g & 63, sl = ch / 8, c8 = ch % 8;
    *reinterpret_cast<u32x4_t*>(&As[sl][r * 128 + ((c8 ^ rswz(r)) << 4)]) = xa[i];
  }
#pragma unroll
  for (int i = 0; i < WL; ++i) {
    const int g = i * RS_THREADS + tid, r = g >> 7, ch = g & 127;
    const int sl = ch / 16, c16 = ch % 16;  // half of a 16-byte bf16 chunk
    const int pos = (((c16 >> 1) ^ rswz(r)) << 4) + (c16 & 1) * 8;
    uint32_t h[3][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      uint32_t part[3][2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float v = wb[i][2 * u + e];
        const bf16_t h1 = f32_to_bf16(v);
        const float r1 = v - bf16_to_f32(h1);
        const bf16_t h2 = f32_to_bf16(r1);
        const float r2 = r1 - bf16_to_f32(h2);
        part[0][e] = h1;
        part[1][e] = h2;
        part[2][e] = f32_to_bf16(r2);
      }
#pragma unroll
      for (int t = 0; t < 3; ++t) h[t][u] = part[t][0] | (part[t][1] << 16);
    }
#pragma unroll
    for (int t = 0; t < 3; ++t)
      *reinterpret_cast<uint2*>(&Bs[t][sl][r * 128 + pos]) = make_uint2(h[t][0], h[t][1]);
  }
  __syncthreads();
  const int fr = lane & 31, fh = lane >> 5;
  f32x16_t acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  if (wv < 3) {
    // the chunk's k-steps in order; the fragments of step q+1 are read while
    // the MFMA of step q runs
    const int nq = nsl * (RM_BK / 16);
    auto frag = [&](const unsigned char* base, int q) {
      const int ch = 2 * (q & 3) + fh;
      return *reinterpret_cast<const bf16x8_t*>(base + (q >> 2) * RS_T * 128 + fr * 128 +
                                                ((ch ^ rswz(fr)) << 4));
    };
    const unsigned char* Ab = &As[0][0];
    const unsigned char* Bb = &Bs[wv][0][0];
    bf16x8_t af = frag(Ab, 0), bf = frag(Bb, 0);
    for (int q = 0; q < nq; ++q) {
      const int qn = q + 1 < nq ? q + 1 : q;
      const bf16x8_t an = frag(Ab, qn), bn = frag(Bb, qn);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf, acc, 0, 0, 0);
      af = an;
      bf = bn;
    }
  }
  // parts 1 and 2 to LDS, part 0's wave adds them smallest first
  if (wv == 1 || wv == 2) {
#pragma unroll
    for (int i = 0; i < 16; ++i) red[wv - 1][i * 64 + lane] = acc[i];
  }
  __syncthreads();
  if (wv == 0) {
    float* o = out + (size_t)c * T * N;
    const int col = n0 + fr;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = m0 + 8 * (i >> 2) + 4 * fh + (i & 3);
      const float p = (red[1][i * 64 + lane] + red[0][i * 64 + lane]) + acc[i];
      if (row < T && col < N) o[(size_t)row * N + col] = p;
    }
  }
}

// The same product for batches that take no k split: 128 tokens x 64
// experts per block, eight waves of 32 x 32 (x the three planes), k-slices of
// 64 through a four-stage LDS ring filled by direct DMA (two slices in
// flight while one is consumed), and an XCD-aware tile order: blocks of XCD
// x take the x-th eighth of the tiles in column-major order, so an XCD works
// on one or two expert tiles and keeps their 2.75 MB of weight planes in its
// L2.  Every logit is computed by the same MFMA sequence as in
// router_mfma_kernel (same operand order, k-steps in order, chunk sums
// formed and added the same way), so the two kernels agree bit for bit.
constexpr int R2_BM = 128, R2_BN = 64, R2_ST = 4;
constexpr int R2_A = R2_BM * 128, R2_B = 3 * R2_BN * 128, R2_STAGE = R2_A + R2_B;

__global__ __launch_bounds__(512) void router_mfma2_kernel(const bf16_t* __restrict__ x,
                                                           const bf16_t* __restrict__ ws,
                                                           float* __restrict__ out, int T, int N,
                                                           int d) {
  __shared__ __attribute__((aligned(1024))) unsigned char lds[R2_ST * R2_STAGE];
  const int ntm = (T + R2_BM - 1) / R2_BM, ntn = (N + R2_BN - 1) / R2_BN;
  const int Q = ntm * ntn, per = (Q + 7) / 8;
  const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
  const int q = xcd * per + local;
  if (local >= per || q >= Q) return;  // uniform over the block
  const int m0 = (q % ntm) * R2_BM, n0 = (q / ntm) * R2_BN;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // DMA: a wave load covers 8 rows of 128 bytes; lane -> row lane / 8 at LDS
  // chunk position lane % 8, fetching the global chunk that belongs there
  const int drow = lane >> 3, dpos = lane & 7;
  const size_t plane = (size_t)N * d;
  uint32_t a_off[2], b_off[3];
#pragma unroll
  for (int j = 0; j < 2; ++j) {  // A rows (w*2 + j)*8 + drow of 128
    const int tr = (w * 2 + j) * 8 + drow;
    a_off[j] = (uint32_t)((size_t)min(m0 + tr, T - 1) * d * 2) + ((dpos ^ rswz(tr)) << 4);
  }
#pragma unroll
  for (int j = 0; j < 3; ++j) {  // B rows (w*3 + j)*8 + drow of 3 x 64 (plane-major)
    const int br = (w * 3 + j) * 8 + drow;
    const int t = br / R2_BN, e = br % R2_BN;
    b_off[j] = (uint32_t)((t * plane + (size_t)min(n0 + e, N - 1) * d) * 2) +
               ((dpos ^ rswz(br)) << 4);
  }
  const rsrc_t ra = make_rsrc(reinterpret_cast<const unsigned char*>(x));
  const rsrc_t rb = make_rsrc(reinterpret_cast<const unsigned char*>(ws));
  const int nk = d / 64;
  auto issue = [&](int kt) {
    unsigned char* st = lds + (kt % R2_ST) * R2_STAGE;
    const uint32_t k0 = (uint32_t)kt * 128;
#pragma unroll
    for (int j = 0; j < 2; ++j) dma16(ra, a_off[j], k0, st + (w * 2 + j) * 1024);
#pragma unroll
    for (int j = 0; j < 3; ++j) dma16(rb, b_off[j], k0, st + R2_A + (w * 3 + j) * 1024);
  };
#pragma unroll
  for (int kt = 0; kt < R2_ST - 1; ++kt)
    if (kt < nk) issue(kt);

  const int wm = w & 3, wn = w >> 2, fr = lane & 31, fh = lane >> 5;
  const int ar = wm * 32 + fr, br = wn * 32 + fr;
  constexpr int SL = RM_KC / 64;  // slices per chunk
  f32x16_t acc[3], tot;
#pragma unroll
  for (int t = 0; t < 3; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
  for (int kt = 0; kt < nk; ++kt) {
    // slice kt is complete once only the loads of slices kt+1, kt+2 remain
    if (kt + R2_ST - 2 < nk) wait_vm<(R2_ST - 2) * 5>();
    else wait_vm<0>();
    __builtin_amdgcn_s_barrier();  // ... in every wave; slice kt-1 is free
    if (kt + R2_ST - 1 < nk) issue(kt + R2_ST - 1);
    const unsigned char* As = lds + (kt % R2_ST) * R2_STAGE;
    const unsigned char* Bs = As + R2_A;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int ch = 2 * ks + fh;
      const bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(As + ar * 128 + ((ch ^ rswz(ar)) << 4));
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        const int rr = t * R2_BN + br;
        const bf16x8_t bfr =
            *reinterpret_cast<const bf16x8_t*>(Bs + rr * 128 + ((ch ^ rswz(rr)) << 4));
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bfr, acc[t], 0, 0, 0);
      }
    }
    if ((kt + 1) % SL == 0 || kt + 1 == nk) {  // end of a chunk
      const bool first = kt < SL;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = (acc[2][r] + acc[1][r]) + acc[0][r];
        tot[r] = first ? p : tot[r] + p;
      }
#pragma unroll
      for (int t = 0; t < 3; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
    }
  }
  const int col = n0 + wn * 32 + fr;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = m0 + wm * 32 + 8 * (r >> 2) + 4 * fh + (r & 3);
    if (row < T && col < N) out[(size_t)row * N + col] = tot[r];
  }
}

// ---------------------------------------------------------------------------
// K2: one wavefront per token.  Lane l holds experts [l*P, l*P+P).
// ---------------------------------------------------------------------------

template <int P>
__global__ __launch_bounds__(256) void topk_kernel(
    const float* __restrict__ logits, int nparts, float* __restrict__ logits_out,
    const float* __restrict__ logit_add, int logits_are_scores, const float* __restrict__ bias,
    float* __restrict__ scores_out, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    int T, int N, int k, int score_fn, int renorm, int n_groups, int topk_groups) {
  __shared__ float keys_lds[TK_WAVES][512];
  __shared__ float gsc[TK_WAVES][64];
  __shared__ int gsel[TK_WAVES][64];
  const int wv = threadIdx.x >> 6;
  topk_token<P>(blockIdx.x * TK_WAVES + wv, keys_lds[wv], gsc[wv], gsel[wv], logits, nparts,
                logits_out, logit_add, logits_are_scores, bias, scores_out, topk_idx, topk_w,
                T, N, k, score_fn, renorm, n_groups, topk_groups);
}

}  // namespace

// chunks of the split router GEMM for small batches (0: one pass per block)
int router_split_chunks(const moe_shape& s) {
  if (!act_bf16(s)) return 0;
  const long long blocks = ((s.T + RM_BM - 1) / RM_BM) * ((s.n_experts + RM_BN - 1) / RM_BN);
  const int nkc = (s.d_model + RM_KC - 1) / RM_KC;
  return (blocks < 128 && nkc > 1) ? nkc : 0;
}

// writes x W_r^T to `logits`, or, when the k-split is taken, its per-chunk
// partial sums to the workspace (launch_topk adds them up); returns the number
// of partial-sum planes that launch_topk must read (1: `logits` holds sums)
hipError_t launch_router_gemm(const moe_shape& s, const void* x, const float* w_router,
                              float* logits, const Workspace& w, hipStream_t st, int* nparts) {
  const int T = (int)s.T, N = s.n_experts, d = s.d_model;
  *nparts = 1;
  if (act_bf16(s)) {
    const long long n = (long long)N * d;
    const int nkc = router_split_chunks(s);
    if (nkc && T <= kRouterSmallMaxT) {
      dim3 grid((T + RS_T - 1) / RS_T, (N + RS_T - 1) / RS_T, nkc);
      router_small_kernel<<<grid, RS_THREADS, 0, st>>>(static_cast<const bf16_t*>(x), w_router,
                                                w.router_part, T, N, d);
      *nparts = nkc;
      return hipGetLastError();
    }
    split3_kernel<<<(int)min((n + 255) / 256, 2048LL), 256, 0, st>>>(w_router, w.wsplit, n);
    if (nkc) {
      dim3 grid((T + RM_BM - 1) / RM_BM, (N + RM_BN - 1) / RM_BN, nkc);
      router_mfma_kernel<<<grid, 256, 0, st>>>(static_cast<const bf16_t*>(x), w.wsplit,
                                               w.router_part, T, N, d, 1);
      *nparts = nkc;
    } else if ((size_t)T * d * 2 < (1ull << 31) && (size_t)3 * N * d * 2 < (1ull << 31)) {
      // (32-bit buffer offsets)
      const int Q = ((T + R2_BM - 1) / R2_BM) * ((N + R2_BN - 1) / R2_BN);
      router_mfma2_kernel<<<8 * ((Q + 7) / 8), 512, 0, st>>>(static_cast<const bf16_t*>(x),
                                                              w.wsplit, logits, T, N, d);
    } else {
      dim3 grid((T + RM_BM - 1) / RM_BM, (N + RM_BN - 1) / RM_BN, 1);
      router_mfma_kernel<<<grid, 256, 0, st>>>(static_cast<const bf16_t*>(x), w.wsplit, logits,
                                               T, N, d, (d + RM_KC - 1) / RM_KC);
    }
  } else {
    dim3 grid((T + RT_BM - 1) / RT_BM, (N + RT_BN - 1) / RT_BN);
    router_gemm_kernel<<<grid, 256, 0, st>>>(static_cast<const float*>(x), w_router,
                                                     logits, T, N, d);
  }
  return hipGetLastError();
}

template <int P>
static void launch_topk_p(dim3 grid, hipStream_t st, const float* logits, int nparts,
                          float* logits_out, const float* logit_add, bool logits_are_scores,
                          const float* bias, float* scores_out, int32_t* topk_idx,
                          float* topk_w, int T, const moe_shape& s) {
  topk_kernel<P><<<grid, 256, 0, st>>>(logits, nparts, logits_out, logit_add,
                                       logits_are_scores ? 1 : 0, bias, scores_out, topk_idx,
                                       topk_w, T, s.n_experts, s.top_k, s.score_fn,
                                       s.renormalize, s.n_groups, s.topk_groups);
}

hipError_t launch_topk(const moe_shape& s, const float* logits, int nparts, float* logits_out,
                       const float* logit_add, bool logits_are_scores, const float* bias,
                       float* scores_out, int32_t* topk_idx, float* topk_w, hipStream_t st) {
  const int T = (int)s.T, N = s.n_experts;
  dim3 grid((T + TK_WAVES - 1) / TK_WAVES);
  const int P = (N + 63) / 64;
  auto run = [&](auto tag) {
    launch_topk_p<decltype(tag)::value>(grid, st, logits, nparts, logits_out, logit_add,
                                        logits_are_scores, bias, scores_out, topk_idx, topk_w,
                                        T, s);
  };
  if (P <= 1) run(std::integral_constant<int, 1>());
  else if (P <= 2) run(std::integral_constant<int, 2>());
  else if (P <= 4) run(std::integral_constant<int, 4>());
  else run(std::integral_constant<int, 8>());
  return hipGetLastError();
}

}  // namespace moe
