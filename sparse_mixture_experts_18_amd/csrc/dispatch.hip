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
// Three launches (one when all assignments fit one chunk), none of whose
// results depends on atomic ordering:
//   rank   one block per chunk of 512 assignments: position inside the chunk
//          (wave-wide equality counting per 64 assignments, then a prefix over
//          the chunk's 8 waves) and the chunk's per-expert histogram
//   scan   per expert, a running sum over chunks -> chunk base positions and
//          pre-drop counts; kept = min(count, C); offsets = exclusive scan
//   place  pos = base + rank; slot / perm
#include "moe_internal.h"
#include "route_device.h"

namespace moe {
namespace {

constexpr int RK_WAVES = kDispatchChunk / kWave;  // 8 waves, one per 64 assignments

// one block per chunk of 512 assignments; wave w ranks assignments 64w..64w+63
// of the chunk (wave-wide equality counting), then a per-expert prefix over
// the 8 waves turns those into positions inside the chunk
__global__ __launch_bounds__(kDispatchChunk) void rank_kernel(const int32_t* __restrict__ topk_idx,
                                                              int32_t* __restrict__ rank,
                                                              int32_t* __restrict__ hist, int A,
                                                              int N, int nchunks) {
  __shared__ int cnt[RK_WAVES][512];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int c = blockIdx.x;
  for (int i = tid; i < RK_WAVES * 512; i += kDispatchChunk) (&cnt[0][0])[i] = 0;
  __syncthreads();
  const int a = c * kDispatchChunk + tid;
  int e = a < A ? topk_idx[a] : -1;
  if (e >= N || e < 0) e = -1;  // out-of-range ids are not placed
  int r = 0;
  bool last = true;
  for (int j = 0; j < kWave; ++j) {
    const int ej = __builtin_amdgcn_readlane(e, j);
    if (ej == e) {
      r += j < lane;
      last = last && !(j > lane);
    }
  }
  if (e >= 0 && last) cnt[wv][e] = r + 1;  // this wave's count of expert e
  __syncthreads();
  for (int x = tid; x < N; x += kDispatchChunk) {
    int run = 0;
#pragma unroll
    for (int w = 0; w < RK_WAVES; ++w) {
      const int v = cnt[w][x];
      cnt[w][x] = run;
      run += v;
    }
    hist[(size_t)c * N + x] = run;
  }
  __syncthreads();
  if (e >= 0) rank[a] = cnt[wv][e] + r;
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
    // per expert, a running sum over the chunks; loads batched so that 16 are
    // in flight at a time
    constexpr int BATCH = 16;
    for (int c0 = 0; c0 < nchunks; c0 += BATCH) {
      int v[BATCH];
#pragma unroll
      for (int i = 0; i < BATCH; ++i) v[i] = c0 + i < nchunks ? hist[(size_t)(c0 + i) * N + e] : 0;
#pragma unroll
      for (int i = 0; i < BATCH; ++i) {
        if (c0 + i < nchunks) base[(size_t)(c0 + i) * N + e] = run;
        run += v[i];
      }
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

__global__ __launch_bounds__(kDispatchChunk) void dispatch_one_chunk_kernel(
    const int32_t* __restrict__ topk_idx, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ slot, int32_t* __restrict__ perm,
    int32_t* __restrict__ nkd, int A, int N, long long C) {
  dispatch_one_chunk(topk_idx, counts, offsets, slot, perm, nkd, A, N, C);
}

}  // namespace

hipError_t launch_dispatch(const moe_shape& s, const int32_t* topk_idx, int32_t* counts,
                           int32_t* offsets, int32_t* slot, int32_t* perm, int32_t* nkd,
                           const Workspace& w, hipStream_t st) {
  const int A = (int)(s.T * s.top_k), N = s.n_experts;
  const int nchunks = (A + kDispatchChunk - 1) / kDispatchChunk;
  const long long C = capacity_of(s);
  if (nchunks <= 1) {
    dispatch_one_chunk_kernel<<<1, kDispatchChunk, 0, st>>>(topk_idx, counts, offsets, slot,
                                                            perm, nkd, A, N, C);
    return hipGetLastError();
  }
  rank_kernel<<<nchunks, kDispatchChunk, 0, st>>>(topk_idx, w.rank, w.hist, A, N, nchunks);
  scan_kernel<<<1, 512, 0, st>>>(w.hist, w.base, counts, offsets, nkd, A, N, nchunks, C);
  const int blocks = min((A + 255) / 256, 4096);
  place_kernel<<<blocks, 256, 0, st>>>(topk_idx, w.rank, w.base, offsets, slot, perm, A, N, C);
  return hipGetLastError();
}

}  // namespace moe
