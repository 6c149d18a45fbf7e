// Gate-weighted combine and the balancing step.
//
// Combine: y_t = sum_{kept j} g_tj E_{e_tj}(x_t) + S(x_t) (llm-compass MoE
// page, output equation; "MoE architecture in practice", shared-expert
// section: the shared output is added).  A dropped assignment contributes
// nothing (same article, capacity section: its FFN branch output is zero).
// fp32 accumulation in ascending j, then the shared term; one pass, no
// atomics, so the result is bitwise reproducible.
//
// Balancing step (same article, load-balancing section: BiasBalancedRouter
// update and the f_i P_i statistic; llm-compass MoE page, aux-loss-free and
// aux-loss equations).
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int CB_THREADS = 256;
typedef unsigned int u4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void unpack8(const uint4& v, float* o) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = __uint_as_float(w[i] << 16);
    o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

__device__ __forceinline__ uint4 pack8(const float* f) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = (uint32_t)f32_to_bf16(f[2 * i]) | ((uint32_t)f32_to_bf16(f[2 * i + 1]) << 16);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// one block per token; threads walk the row in 16-byte vectors.  All of a
// vector's k expert rows are loaded before the first is added (KM >= k
// slots, unrolled), so the loads are in flight together; the sum still runs
// in ascending j.
template <int KM>
__global__ __launch_bounds__(CB_THREADS) void combine_bf16_kernel(
    const bf16_t* __restrict__ y_perm, const bf16_t* __restrict__ y_shared,
    const int32_t* __restrict__ slot, const float* __restrict__ topk_w, bf16_t* __restrict__ y,
    int d, int k) {
  const int t = blockIdx.x;
  __shared__ int s_slot[16];
  __shared__ float s_w[16];
  if (threadIdx.x < k) {
    s_slot[threadIdx.x] = slot[(size_t)t * k + threadIdx.x];
    s_w[threadIdx.x] = topk_w[(size_t)t * k + threadIdx.x];
  }
  __syncthreads();
  int sl[KM];
  float gw[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    sl[j] = j < k ? s_slot[j] : -1;
    gw[j] = j < k ? s_w[j] : 0.f;
  }
  const int nv = d / 8;
  for (int v = threadIdx.x; v < nv; v += CB_THREADS) {
    uint4 raw[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j)
      if (sl[j] >= 0) {
        // each expert row is read once: non-temporal loads keep it from
        // displacing reusable lines in the caches
        const u4v t = __builtin_nontemporal_load(
            reinterpret_cast<const u4v*>(y_perm + (size_t)sl[j] * d) + v);
        raw[j] = make_uint4(t[0], t[1], t[2], t[3]);
      }
    uint4 rs = make_uint4(0, 0, 0, 0);
    if (y_shared) rs = reinterpret_cast<const uint4*>(y_shared + (size_t)t * d)[v];
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if (sl[j] < 0) continue;  // beyond k, or a dropped assignment
      float e[8];
      unpack8(raw[j], e);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += gw[j] * e[i];
    }
    if (y_shared) {
      float e[8];
      unpack8(rs, e);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += e[i];
    }
    reinterpret_cast<uint4*>(y + (size_t)t * d)[v] = pack8(acc);
  }
}

__global__ __launch_bounds__(CB_THREADS) void combine_f32_kernel(
    const float* __restrict__ y_perm, const float* __restrict__ y_shared,
    const int32_t* __restrict__ slot, const float* __restrict__ topk_w, float* __restrict__ y,
    int d, int k) {
  const int t = blockIdx.x;
  __shared__ int s_slot[16];
  __shared__ float s_w[16];
  if (threadIdx.x < k) {
    s_slot[threadIdx.x] = slot[(size_t)t * k + threadIdx.x];
    s_w[threadIdx.x] = topk_w[(size_t)t * k + threadIdx.x];
  }
  __syncthreads();
  for (int c = threadIdx.x; c < d; c += CB_THREADS) {
    float acc = 0.f;
    for (int j = 0; j < k; ++j) {
      const int sl = s_slot[j];
      if (sl < 0) continue;
      acc += s_w[j] * y_perm[(size_t)sl * d + c];
    }
    if (y_shared) acc += y_shared[(size_t)t * d + c];
    y[(size_t)t * d + c] = acc;
  }
}

// P_i = mean_t s_ti, one block per expert, fp64 partial sums in a fixed tree
__global__ __launch_bounds__(256) void score_mean_kernel(const float* __restrict__ scores,
                                                         double* __restrict__ P, int T, int N) {
  __shared__ double sh[256];
  const int e = blockIdx.x;
  double acc = 0.0;
  for (int t = threadIdx.x; t < T; t += 256) acc += (double)scores[(size_t)t * N + e];
  sh[threadIdx.x] = acc;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) sh[threadIdx.x] += sh[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) P[e] = sh[0] / (double)T;
}

__global__ __launch_bounds__(512) void bias_step_kernel(const int32_t* __restrict__ counts,
                                                        const double* __restrict__ P,
                                                        float* __restrict__ bias,
                                                        float* __restrict__ aux_out,
                                                        long long T, int N, int k, float step,
                                                        float clamp) {
  __shared__ double sh[512];
  const int e = threadIdx.x;
  double fp = 0.0;
  if (e < N) {
    const long long c = counts[e];
    const long long diff = (long long)N * c - T * (long long)k;  // sign of load - mean load
    const float sg = diff > 0 ? 1.f : (diff < 0 ? -1.f : 0.f);
    float b = bias[e] - step * sg;
    if (clamp > 0.f) b = fminf(fmaxf(b, -clamp), clamp);
    bias[e] = b;
    if (P) fp = ((double)c / (double)T) * P[e];
  }
  if (!aux_out) return;  // uniform
  sh[e] = fp;
  __syncthreads();
  for (int o = 256; o > 0; o >>= 1) {
    if (e < o) sh[e] += sh[e + o];
    __syncthreads();
  }
  if (e == 0) aux_out[0] = (float)((double)N * sh[0]);
}

}  // namespace

hipError_t launch_combine(const moe_shape& s, const void* y_perm, const void* y_shared,
                          const int32_t* slot, const float* topk_w, void* y, hipStream_t st) {
  const int T = (int)s.T, d = s.d_model, k = s.top_k;
  if (act_bf16(s) && k <= 8)
    combine_bf16_kernel<8><<<T, CB_THREADS, 0, st>>>(
        static_cast<const bf16_t*>(y_perm), static_cast<const bf16_t*>(y_shared), slot, topk_w,
        static_cast<bf16_t*>(y), d, k);
  else if (act_bf16(s))
    combine_bf16_kernel<16><<<T, CB_THREADS, 0, st>>>(
        static_cast<const bf16_t*>(y_perm), static_cast<const bf16_t*>(y_shared), slot, topk_w,
        static_cast<bf16_t*>(y), d, k);
  else
    combine_f32_kernel<<<T, CB_THREADS, 0, st>>>(static_cast<const float*>(y_perm),
                                                 static_cast<const float*>(y_shared), slot,
                                                 topk_w, static_cast<float*>(y), d, k);
  return hipGetLastError();
}

hipError_t launch_bias_update(const moe_shape& s, const int32_t* counts, const float* scores,
                              float step, float clamp, float* bias, float* aux_out,
                              double* p_scratch, hipStream_t st) {
  const int N = s.n_experts;
  const bool aux = scores && aux_out;
  if (aux) score_mean_kernel<<<N, 256, 0, st>>>(scores, p_scratch, (int)s.T, N);
  bias_step_kernel<<<1, 512, 0, st>>>(counts, aux ? p_scratch : nullptr, bias,
                                      aux ? aux_out : nullptr, s.T, N, s.top_k, step, clamp);
  return hipGetLastError();
}

}  // namespace moe
