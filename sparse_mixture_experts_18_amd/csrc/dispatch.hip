// Dispatch: per-expert histogram, prefix scan and stable permutation with
// deterministic capacity drops.
//
// Assignments are numbered token-major, a = t*k + j, and grouped by expert
// keeping that order ("MoE architecture in practice", expert-parallelism
// section: flatten to [T*k], stable group-by-expert so one grouped GEMM
// covers all experts).  An assignment's arrival position is the number of
// earlier assignments to the same expert; the earliest C arrivals keep their
// slot, the rest are dropped (same article, routing-math and capacity
// sections; llm-compass MoE page, capacity = capacity_factor * tokens / N).
//
// Three launches, none of whose results depends on atomic ordering:
//   rank   one wavefront per chunk of 512 assignments: position inside the
//          chunk (wave-wide equality counting, 64 lanes at a time) and the
//          chunk's per-expert histogram
//   scan   per expert, a running sum over chunks -> chunk base positions and
//          pre-drop counts; kept = min(count, C); offsets = exclusive scan
//   place  pos = base + rank; slot / perm
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int RK_WAVES = 4;

__global__ __launch_bounds__(256) void rank_kernel(const int32_t* __restrict__ topk_idx,
                                                   int32_t* __restrict__ rank,
                                                   int32_t* __restrict__ hist, int A, int N,
                                                   int nchunks) {
  __shared__ int cnt[RK_WAVES][512];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int c = blockIdx.x * RK_WAVES + wv;
  if (c >= nchunks) return;  // wave-uniform; no block barrier in this kernel
  int* my = cnt[wv];
  for (int e = lane; e < N; e += kWave) my[e] = 0;
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_wave_barrier();
  for (int step = 0; step < kDispatchChunk / kWave; ++step) {
    const int a = c * kDispatchChunk + step * kWave + lane;
    int e = a < A ? topk_idx[a] : -1;
    if (e >= N) e = -1;  // out-of-range ids are not placed
    int r = 0;
    bool last = true;
    for (int j = 0; j < kWave; ++j) {
      const int ej = __shfl(e, j, kWave);
      if (ej == e) {
        r += j < lane;
        last = last && !(j > lane);
      }
    }
    int base = 0;
    if (e >= 0) base = my[e];
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
    if (e >= 0) {
      rank[a] = base + r;
      if (last) my[e] = base + r + 1;
    }
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_wave_barrier();
  }
  for (int e = lane; e < N; e += kWave) hist[(size_t)c * N + e] = my[e];
}

__global__ __launch_bounds__(512) void scan_kernel(const int32_t* __restrict__ hist,
                                                   int32_t* __restrict__ base,
                                                   int32_t* __restrict__ counts,
                                                   int32_t* __restrict__ offsets,
                                                   int32_t* __restrict__ nkd, int A, int N,
                                                   int nchunks, long long C) {
  __shared__ int sh[512];
  const int e = threadIdx.x;
  int run = 0;
  if (e < N) {
    for (int c = 0; c < nchunks; ++c) {
      const int h = hist[(size_t)c * N + e];
      base[(size_t)c * N + e] = run;
      run += h;
    }
    counts[e] = run;
  }
  int kept = e < N ? (C < 0 ? run : (int)min((long long)run, C)) : 0;
  // inclusive Hillis-Steele scan over 512 entries (integer: exact)
  sh[e] = kept;
  __syncthreads();
  for (int o = 1; o < 512; o <<= 1) {
    int v = e >= o ? sh[e - o] : 0;
    __syncthreads();
    sh[e] += v;
    __syncthreads();
  }
  if (e < N) offsets[e] = sh[e] - kept;
  if (e == 0) {
    const int R = sh[511];
    offsets[N] = R;
    nkd[0] = R;
    nkd[1] = A - R;
  }
}

__global__ __launch_bounds__(256) void place_kernel(const int32_t* __restrict__ topk_idx,
                                                    const int32_t* __restrict__ rank,
                                                    const int32_t* __restrict__ base,
                                                    const int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ slot,
                                                    int32_t* __restrict__ perm, int A, int N,
                                                    long long C) {
  for (int a = blockIdx.x * blockDim.x + threadIdx.x; a < A; a += gridDim.x * blockDim.x) {
    const int e = topk_idx[a];
    int s = -1;
    if (e >= 0 && e < N) {
      const int pos = base[(size_t)(a / kDispatchChunk) * N + e] + rank[a];
      if (C < 0 || pos < C) {
        s = offsets[e] + pos;
        perm[s] = a;
      }
    }
    slot[a] = s;
  }
}

}  // namespace

hipError_t launch_dispatch(const moe_shape& s, const int32_t* topk_idx, int32_t* counts,
                           int32_t* offsets, int32_t* slot, int32_t* perm, int32_t* nkd,
                           const Workspace& w, hipStream_t st) {
  const int A = (int)(s.T * s.top_k), N = s.n_experts;
  const int nchunks = (A + kDispatchChunk - 1) / kDispatchChunk;
  const long long C = capacity_of(s);
  rank_kernel<<<(nchunks + RK_WAVES - 1) / RK_WAVES, 256, 0, st>>>(topk_idx, w.rank, w.hist, A,
                                                                   N, nchunks);
  scan_kernel<<<1, 512, 0, st>>>(w.hist, w.base, counts, offsets, nkd, A, N, nchunks, C);
  const int blocks = min((A + 255) / 256, 4096);
  place_kernel<<<blocks, 256, 0, st>>>(topk_idx, w.rank, w.base, offsets, slot, perm, A, N, C);
  return hipGetLastError();
}

}  // namespace moe
