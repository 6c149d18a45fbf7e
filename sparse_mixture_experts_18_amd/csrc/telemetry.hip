// Router telemetry and the per-sequence balancing step.
//
// Telemetry: the indicators "MoE architecture in practice" lists as the
// minimum MoE observability (section on scale drift between experts: drop
// ratio, per-expert load, per-expert output mean / std / max, bias magnitude,
// gate entropy; its checklist: drop ratio logged per expert) and the "MoE
// landscape" page's first-class indicators (dead experts, usage CV, token
// drop, router bias norm).  Every reduction runs in fp64 in a fixed order, so
// the numbers are reproducible bit for bit.
//
// Per-sequence balancing step: the same article's update_bias (load-balancing
// section), which averages loads over sequences so that long sequences do not
// dominate; the load of expert i in sequence s is its share c_si / (k L_s).
#include <math.h>

#include "moe_internal.h"

namespace moe {
namespace {

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ double wave_max_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o, kWave));
  return v;
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// the values of one 16-byte chunk of a row
template <typename XT>
struct Chunk;
template <>
struct Chunk<float> {
  static constexpr int n = 4;
  __device__ static __forceinline__ void get(const u32x4_t& v, float* o) {
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = __uint_as_float(v[i]);
  }
};
template <>
struct Chunk<bf16_t> {
  static constexpr int n = 8;
  __device__ static __forceinline__ void get(const u32x4_t& v, float* o) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(v[i] << 16);
      o[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
  }
};

// one wave per output row: fp64 sum, sum of squares, max and max |.| of the
// row's d values -> part[row][4]; rows from *nrows_dev on (dropped slots of
// y_perm) are skipped when nrows_dev is given
template <typename XT>
__global__ __launch_bounds__(256) void row_stats_kernel(const XT* __restrict__ y, int rows,
                                                        const int32_t* __restrict__ nrows_dev,
                                                        int d, double* __restrict__ part) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows || (nrows_dev && row >= *nrows_dev)) return;
  // 16-byte chunks (d is a multiple of 32 elements, rows 16-byte aligned)
  const u32x4_t* p = reinterpret_cast<const u32x4_t*>(y + (size_t)row * d);
  constexpr int E = Chunk<XT>::n;
  const int nch = d / E;
  double s = 0.0, q = 0.0, mx = -INFINITY, ma = 0.0;
  for (int c = lane; c < nch; c += kWave) {
    float f[E];
    Chunk<XT>::get(__builtin_nontemporal_load(p + c), f);  // each row is read once
#pragma unroll
    for (int i = 0; i < E; ++i) {
      const double v = (double)f[i];
      s += v;
      q += v * v;
      mx = fmax(mx, v);
      ma = fmax(ma, fabs(v));
    }
  }
  s = wave_sum_d(s);
  q = wave_sum_d(q);
  mx = wave_max_d(mx);
  ma = wave_max_d(ma);
  if (lane == 0) {
    double* o = part + (size_t)row * 4;
    o[0] = s;
    o[1] = q;
    o[2] = mx;
    o[3] = ma;
  }
}

// one block per expert (blockIdx.x == N: the shared expert's T rows):
// load / kept / dropped / drop ratio and the output moments of its rows
__global__ __launch_bounds__(256) void expert_stats_kernel(
    const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
    const double* __restrict__ part, const double* __restrict__ part_shared, int N, int T,
    int d, int has_routed_rows, int has_shared, double* __restrict__ per) {
  __shared__ double sh[4][256];
  const int e = blockIdx.x, tid = threadIdx.x;
  int r0 = 0, r1 = 0, has_rows = has_routed_rows;
  const double* src = part;
  if (e < N) {
    r0 = offsets[e];
    r1 = offsets[e + 1];
  } else if (has_shared) {
    r1 = T;
    src = part_shared;
    has_rows = 1;
  } else {  // no shared expert: an all-zero row
    if (tid < 8) per[(size_t)N * 8 + tid] = 0.0;
    return;
  }
  double s = 0.0, q = 0.0, mx = -INFINITY, ma = 0.0;
  if (has_rows)
    for (int r = r0 + tid; r < r1; r += 256) {
      const double* o = src + (size_t)r * 4;
      s += o[0];
      q += o[1];
      mx = fmax(mx, o[2]);
      ma = fmax(ma, o[3]);
    }
  sh[0][tid] = s;
  sh[1][tid] = q;
  sh[2][tid] = mx;
  sh[3][tid] = ma;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if (tid < h) {
      sh[0][tid] += sh[0][tid + h];
      sh[1][tid] += sh[1][tid + h];
      sh[2][tid] = fmax(sh[2][tid], sh[2][tid + h]);
      sh[3][tid] = fmax(sh[3][tid], sh[3][tid + h]);
    }
    __syncthreads();
  }
  if (tid == 0) {
    double* o = per + (size_t)e * 8;
    const int load = e < N ? counts[e] : T;
    const int kept = r1 - r0;
    o[0] = load;
    o[1] = kept;
    o[2] = load - kept;
    o[3] = load > 0 ? (double)(load - kept) / (double)load : 0.0;
    const double n = (double)kept * (double)d;
    if (has_rows && kept > 0) {
      const double m = sh[0][0] / n;
      const double var = sh[1][0] / n - m * m;
      o[4] = m;
      o[5] = sqrt(var > 0.0 ? var : 0.0);
      o[6] = sh[2][0];
      o[7] = sh[3][0];
    } else {
      o[4] = o[5] = o[6] = o[7] = 0.0;
    }
  }
}

// entropy of a non-negative vector normalised to sum 1, over a wave's lanes
__device__ __forceinline__ double wave_entropy(const float* v, int n) {
  const int lane = threadIdx.x & 63;
  double tot = 0.0;
  for (int i = lane; i < n; i += kWave) tot += (double)v[i];
  tot = wave_sum_d(tot);
  if (!(tot > 0.0)) return 0.0;
  double h = 0.0;
  for (int i = lane; i < n; i += kWave) {
    const double p = (double)v[i] / tot;
    if (p > 0.0) h -= p * log(p);
  }
  return wave_sum_d(h);
}

// one wave per token: entropy of its k gates and of its N scores
__global__ __launch_bounds__(256) void entropy_kernel(const float* __restrict__ topk_w,
                                                      const float* __restrict__ scores, int T,
                                                      int N, int k, double* __restrict__ ent) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const double hg = wave_entropy(topk_w + (size_t)t * k, k);
  const double hs = scores ? wave_entropy(scores + (size_t)t * N, N) : 0.0;
  if ((threadIdx.x & 63) == 0) {
    ent[2 * (size_t)t] = hg;
    ent[2 * (size_t)t + 1] = hs;
  }
}

// one block: the global indicators
__global__ __launch_bounds__(512) void stats_final_kernel(const int32_t* __restrict__ counts,
                                                          const float* __restrict__ bias,
                                                          const double* __restrict__ ent,
                                                          const double* __restrict__ per,
                                                          int N, int T, int k,
                                                          double* __restrict__ glob) {
  __shared__ double sh[6][512];
  const int tid = threadIdx.x;
  const double mean = (double)T * k / N;
  double dv = 0.0, dead = 0.0, drop = 0.0, b2 = 0.0, ba = 0.0;
  for (int e = tid; e < N; e += 512) {
    const double c = counts[e];
    dv += (c - mean) * (c - mean);
    dead += counts[e] == 0 ? 1.0 : 0.0;
    drop += per[(size_t)e * 8 + 2];
    if (bias) {
      const double b = bias[e];
      b2 += b * b;
      ba = fmax(ba, fabs(b));
    }
  }
  double hg = 0.0, hs = 0.0;
  for (int t = tid; t < T; t += 512) {
    hg += ent[2 * (size_t)t];
    hs += ent[2 * (size_t)t + 1];
  }
  sh[0][tid] = dv;
  sh[1][tid] = dead;
  sh[2][tid] = drop;
  sh[3][tid] = b2;
  sh[4][tid] = hg;
  sh[5][tid] = hs;
  __syncthreads();
  for (int h = 256; h > 0; h >>= 1) {
    if (tid < h)
      for (int j = 0; j < 6; ++j) sh[j][tid] += sh[j][tid + h];
    __syncthreads();
  }
  // max |b| separately (a max, not a sum)
  __shared__ double shm[512];
  shm[tid] = ba;
  __syncthreads();
  for (int h = 256; h > 0; h >>= 1) {
    if (tid < h) shm[tid] = fmax(shm[tid], shm[tid + h]);
    __syncthreads();
  }
  if (tid == 0) {
    glob[0] = T;
    glob[1] = (double)T * k;
    glob[2] = sh[2][0];
    glob[3] = sh[2][0] / ((double)T * k);
    glob[4] = sqrt(sh[0][0] / N) / mean;
    glob[5] = sh[1][0];
    glob[6] = sqrt(sh[3][0]);
    glob[7] = shm[0];
    glob[8] = sh[4][0] / T;
    glob[9] = sh[5][0] / T;
    for (int i = 10; i < 16; ++i) glob[i] = 0.0;
  }
}

// ---- per-sequence balancing step ----

// block per sequence: its per-expert counts (integer adds in LDS: exact in any
// order) -> cnt[s][N]
__global__ __launch_bounds__(256) void seq_count_kernel(const int32_t* __restrict__ topk_idx,
                                                        const int32_t* __restrict__ seq_off,
                                                        int N, int k, int T,
                                                        int32_t* __restrict__ cnt) {
  __shared__ int h[512];
  const int s = blockIdx.x, tid = threadIdx.x;
  for (int i = tid; i < N; i += 256) h[i] = 0;
  __syncthreads();
  // offsets are checked by the step kernel; here they are only kept in
  // [0, T] so that malformed ones cannot reach outside topk_idx
  const int t0 = min(max(seq_off[s], 0), T), t1 = min(max(seq_off[s + 1], t0), T);
  const int a0 = t0 * k, a1 = t1 * k;
  for (int a = a0 + tid; a < a1; a += 256) {
    const int e = topk_idx[a];
    if (e >= 0 && e < N) atomicAdd(&h[e], 1);
  }
  __syncthreads();
  for (int i = tid; i < N; i += 256) cnt[(size_t)s * N + i] = h[i];
}

// one block, thread per expert: score_i = sum_s c_si / (k L_s) in sequence
// order, / S; mean = sum_i score_i / N in expert order (one thread); then
// b_i <- fl32(b_i + fl32(step * sign(mean - score_i))), clamped.  Every fp64
// operation is a single IEEE add, divide or compare, in that order.
__global__ __launch_bounds__(512) void seq_bias_step_kernel(
    const int32_t* __restrict__ cnt, const int32_t* __restrict__ seq_off, int S, int N, int k,
    int T, float step, float clamp, float* __restrict__ bias, int32_t* __restrict__ err) {
  __shared__ double score[512];
  __shared__ double mean_s;
  __shared__ int bad;
  const int i = threadIdx.x;
  if (i == 0) {
    int b = seq_off[0] != 0 || seq_off[S] != T;
    for (int s = 0; s < S && !b; ++s) b = seq_off[s + 1] <= seq_off[s];
    bad = b;
  }
  __syncthreads();
  if (bad) {
    if (i == 0 && err) err[0] = 1;
    return;
  }
  if (i < N) {
    double sc = 0.0;
    for (int s = 0; s < S; ++s) {
      const double den = (double)((long long)k * (seq_off[s + 1] - seq_off[s]));
      sc = __dadd_rn(sc, __ddiv_rn((double)cnt[(size_t)s * N + i], den));
    }
    score[i] = __ddiv_rn(sc, (double)S);
  }
  __syncthreads();
  if (i == 0) {
    double tot = 0.0;
    for (int e = 0; e < N; ++e) tot = __dadd_rn(tot, score[e]);
    mean_s = __ddiv_rn(tot, (double)N);
    if (err) err[0] = 0;
  }
  __syncthreads();
  if (i < N) {
    const double m = mean_s;
    const float sg = m > score[i] ? 1.0f : (m < score[i] ? -1.0f : 0.0f);
    float nb = bias[i] + step * sg;
    if (clamp > 0.0f) nb = fminf(fmaxf(nb, -clamp), clamp);
    bias[i] = nb;
  }
}

}  // namespace

hipError_t launch_router_stats(const moe_shape& s, const int32_t* counts, const int32_t* offsets,
                               const float* topk_w, const float* scores, const float* bias,
                               const void* y_perm, const void* y_shared, double* stats,
                               const Workspace& w, hipStream_t st) {
  const int T = (int)s.T, N = s.n_experts, k = s.top_k, d = s.d_model;
  const bool bf = act_bf16(s);
  double* part = w.stats_rows;                       // [T*k][4]
  double* part_sh = w.stats_rows + (size_t)T * k * 4;  // [T][4]
  if (y_perm) {
    // the kept rows [0, R) of y_perm, R = offsets[N]
    const int rows = T * k;
    if (bf)
      row_stats_kernel<bf16_t><<<(rows + 3) / 4, 256, 0, st>>>(
          static_cast<const bf16_t*>(y_perm), rows, offsets + N, d, part);
    else
      row_stats_kernel<float><<<(rows + 3) / 4, 256, 0, st>>>(
          static_cast<const float*>(y_perm), rows, offsets + N, d, part);
  }
  if (y_shared) {
    if (bf)
      row_stats_kernel<bf16_t><<<(T + 3) / 4, 256, 0, st>>>(
          static_cast<const bf16_t*>(y_shared), T, nullptr, d, part_sh);
    else
      row_stats_kernel<float><<<(T + 3) / 4, 256, 0, st>>>(static_cast<const float*>(y_shared),
                                                           T, nullptr, d, part_sh);
  }
  double* per = stats + 16;
  expert_stats_kernel<<<N + 1, 256, 0, st>>>(counts, offsets, part, part_sh, N, T, d,
                                             y_perm ? 1 : 0, y_shared ? 1 : 0, per);
  entropy_kernel<<<(T + 3) / 4, 256, 0, st>>>(topk_w, scores, T, N, k, w.stats_ent);
  stats_final_kernel<<<1, 512, 0, st>>>(counts, bias, w.stats_ent, per, N, T, k, stats);
  return hipGetLastError();
}

hipError_t launch_bias_update_seq(const moe_shape& s, const int32_t* topk_idx,
                                  const int32_t* seq_off, int n_seq, float step, float clamp,
                                  float* bias, int32_t* err, const Workspace& w, hipStream_t st) {
  const int N = s.n_experts, k = s.top_k;
  int32_t* cnt = reinterpret_cast<int32_t*>(w.logits);  // [S][N] ints, S <= T
  seq_count_kernel<<<n_seq, 256, 0, st>>>(topk_idx, seq_off, N, k, (int)s.T, cnt);
  seq_bias_step_kernel<<<1, 512, 0, st>>>(cnt, seq_off, n_seq, N, k, (int)s.T, step, clamp, bias,
                                          err);
  return hipGetLastError();
}

}  // namespace moe
