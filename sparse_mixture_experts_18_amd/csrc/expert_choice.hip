// Expert-choice routing: every expert takes its top-C tokens ("MoE
// architecture in practice", routing-math section: each expert takes the
// top-C tokens its capacity allows; perfectly balanced, no overflow, not
// causal; "MoE landscape" page: the capacity constraint moves into the
// routing).  The scores are the token-choice scores (softmax or sigmoid);
// the raw score s[t, e] is the gate of a chosen pair; a token no expert took
// gets only the shared expert.
//
//   transpose  scores [T,N] -> order keys [N,T] (NaN lowest, -0 == +0)
//   select     one block per expert: radix select of the C-th largest key
//              (four 8-bit passes over LDS histograms), ties at that key to
//              the lower token index, then the expert's segment in ascending
//              token order -> perm (t*k), row_of [T,N], offsets
//   combine    one block per token: the experts that took it, ascending
//
// Integer counts only: every result is exact and independent of scheduling.
#include "moe_internal.h"

namespace moe {
namespace {

// same total order as the token-choice selection: NaN lowest (1), -0 == +0,
// numbers mapped monotonically above it
__device__ __forceinline__ uint32_t ec_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 1u;  // NaN
  if (u == 0x80000000u) u = 0u;
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return u == 0xffffffffu ? u : u + 1u;
}

// keys[e][t] = ec_key(scores[t][e]) through 32 x 32 LDS tiles
__global__ __launch_bounds__(256) void ec_transpose_kernel(const float* __restrict__ scores,
                                                           uint32_t* __restrict__ keys, int T,
                                                           int N) {
  __shared__ uint32_t tile[32][33];
  const int t0 = blockIdx.x * 32, e0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  for (int r = ty; r < 32; r += 8) {
    const int t = t0 + r, e = e0 + tx;
    if (t < T && e < N) tile[r][tx] = ec_key(scores[(size_t)t * N + e]);
  }
  __syncthreads();
  for (int r = ty; r < 32; r += 8) {
    const int e = e0 + r, t = t0 + tx;
    if (t < T && e < N) keys[(size_t)e * T + t] = tile[tx][r];
  }
}

constexpr int EC_THREADS = 1024;

// exclusive prefix sum over the block (NT threads, a multiple of 64, at most
// 1024) of one int per thread
template <int NT = EC_THREADS>
__device__ __forceinline__ int ec_block_scan(int v, int* sh, int& total) {
  const int i = threadIdx.x, lane = i & 63, w = i >> 6, nw = NT / 64;
  int a = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(a, o, 64);
    if (lane >= o) a += t;
  }
  __syncthreads();
  if (lane == 63) sh[w] = a;
  __syncthreads();
  if (w == 0) {
    int c = lane < nw ? sh[lane] : 0;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const int t = __shfl_up(c, o, 64);
      if (lane >= o) c += t;
    }
    if (lane < nw) sh[32 + lane] = c;
  }
  __syncthreads();
  total = sh[32 + nw - 1];
  return (w ? sh[32 + w - 1] : 0) + a - v;
}

// one block per expert e: the Cp = min(C, T) tokens with the largest keys,
// ties to the lower token index; its segment rows [e*Cp, (e+1)*Cp) hold them
// in ascending token order
__global__ __launch_bounds__(EC_THREADS) void ec_select_kernel(
    const uint32_t* __restrict__ keys, int T, int N, int Cp, int k, int32_t* __restrict__ perm,
    int32_t* __restrict__ row_of, int32_t* __restrict__ counts, int32_t* __restrict__ offsets) {
  __shared__ int hist[256];
  __shared__ int sh[64];
  __shared__ uint32_t s_prefix;
  __shared__ int s_remaining;
  const int e = blockIdx.x, tid = threadIdx.x;
  const uint32_t* key = keys + (size_t)e * T;
  // radix select: prefix of the Cp-th largest key, 8 bits at a time
  uint32_t prefix = 0, mask = 0;
  int remaining = Cp;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += EC_THREADS) hist[i] = 0;
    __syncthreads();
    for (int t = tid; t < T; t += EC_THREADS) {
      const uint32_t v = key[t];
      if ((v & mask) == prefix) atomicAdd(&hist[(v >> shift) & 255u], 1);
    }
    __syncthreads();
    if (tid == 0) {
      int above = 0, b = 255;
      for (; b > 0; --b) {
        if (above + hist[b] >= remaining) break;
        above += hist[b];
      }
      s_prefix = prefix | ((uint32_t)b << shift);
      s_remaining = remaining - above;
    }
    __syncthreads();
    prefix = s_prefix;
    remaining = s_remaining;
    mask |= 255u << shift;
    __syncthreads();
  }
  // prefix is the Cp-th largest key; `remaining` of the tokens holding it are
  // taken, the first ones in token order.  Each thread owns a contiguous run
  // of tokens, so token order is thread order.
  const int per = (T + EC_THREADS - 1) / EC_THREADS;
  const int t0 = min(T, tid * per), t1 = min(T, t0 + per);
  int eq = 0;
  for (int t = t0; t < t1; ++t) eq += key[t] == prefix;
  int tot;
  int eq_before = ec_block_scan(eq, sh, tot);
  int taken = 0;
  for (int t = t0; t < t1; ++t) {
    const uint32_t v = key[t];
    if (v > prefix) ++taken;
    else if (v == prefix && eq_before++ < remaining) ++taken;
  }
  int pos = ec_block_scan(taken, sh, tot);
  eq_before = ec_block_scan(eq, sh, tot);  // again, for the second walk
  const int base = e * Cp;
  for (int t = t0; t < t1; ++t) {
    const uint32_t v = key[t];
    bool take = v > prefix;
    if (v == prefix) take = eq_before++ < remaining;
    if (take) {
      perm[base + pos] = t * k;
      row_of[(size_t)t * N + e] = base + pos;
      ++pos;
    } else {
      row_of[(size_t)t * N + e] = -1;
    }
  }
  if (tid == 0) {
    counts[e] = Cp;
    offsets[e] = base;
    if (e == N - 1) offsets[N] = N * Cp;
  }
}

// one block per token: y_t = sum over the experts that took t, ascending e,
// of s[t, e] * y_perm[row] (+ y_shared_t), fp32 accumulation
constexpr int ECC_THREADS = 256;

template <typename XT>
__device__ __forceinline__ void ec_load8(const XT* p, float* o);
template <>
__device__ __forceinline__ void ec_load8<float>(const float* p, float* o) {
  const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}
template <>
__device__ __forceinline__ void ec_load8<bf16_t>(const bf16_t* p, float* o) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = __uint_as_float(w[i] << 16);
    o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
template <typename XT>
__device__ __forceinline__ void ec_store8(XT* p, const float* f);
template <>
__device__ __forceinline__ void ec_store8<float>(float* p, const float* f) {
  reinterpret_cast<float4*>(p)[0] = make_float4(f[0], f[1], f[2], f[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(f[4], f[5], f[6], f[7]);
}
template <>
__device__ __forceinline__ void ec_store8<bf16_t>(bf16_t* p, const float* f) {
  uint4 v;
  v.x = (uint32_t)f32_to_bf16(f[0]) | ((uint32_t)f32_to_bf16(f[1]) << 16);
  v.y = (uint32_t)f32_to_bf16(f[2]) | ((uint32_t)f32_to_bf16(f[3]) << 16);
  v.z = (uint32_t)f32_to_bf16(f[4]) | ((uint32_t)f32_to_bf16(f[5]) << 16);
  v.w = (uint32_t)f32_to_bf16(f[6]) | ((uint32_t)f32_to_bf16(f[7]) << 16);
  *reinterpret_cast<uint4*>(p) = v;
}

template <typename XT>
__global__ __launch_bounds__(ECC_THREADS) void ec_combine_kernel(
    const XT* __restrict__ y_perm, const XT* __restrict__ y_shared,
    const int32_t* __restrict__ row_of, const float* __restrict__ scores, XT* __restrict__ y,
    int N, int d) {
  __shared__ int s_row[512];
  __shared__ float s_g[512];
  __shared__ int s_n;
  const int t = blockIdx.x, tid = threadIdx.x;
  __shared__ int sh[64];
  // the experts that took t, compacted in ascending order (N <= 512: two
  // experts per thread)
  int r[2], f = 0;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int e = 2 * tid + i;
    r[i] = e < N ? row_of[(size_t)t * N + e] : -1;
    f += r[i] >= 0;
  }
  int total;
  int pos = ec_block_scan<ECC_THREADS>(f, sh, total);
#pragma unroll
  for (int i = 0; i < 2; ++i)
    if (r[i] >= 0) {
      s_row[pos] = r[i];
      s_g[pos] = scores[(size_t)t * N + 2 * tid + i];
      ++pos;
    }
  if (tid == 0) s_n = total;
  __syncthreads();
  const int n = s_n;
  for (int c = tid * 8; c < d; c += ECC_THREADS * 8) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < n; ++j) {
      float v[8];
      ec_load8<XT>(y_perm + (size_t)s_row[j] * d + c, v);
      const float g = s_g[j];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += g * v[i];
    }
    if (y_shared) {
      float v[8];
      ec_load8<XT>(y_shared + (size_t)t * d + c, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    ec_store8<XT>(y + (size_t)t * d + c, acc);
  }
}

}  // namespace

int64_t ec_capacity(const moe_shape& s) {
  const int64_t C = capacity_of(s);
  if (C <= 0) return C;
  return C < s.T ? C : s.T;
}

hipError_t launch_ec_select(const moe_shape& s, const float* scores, int32_t* counts,
                            int32_t* offsets, int32_t* perm, int32_t* row_of, const Workspace& w,
                            hipStream_t st) {
  const int T = (int)s.T, N = s.n_experts;
  uint32_t* keys = reinterpret_cast<uint32_t*>(w.logits);  // [N][T]
  dim3 tg((T + 31) / 32, (N + 31) / 32);
  ec_transpose_kernel<<<tg, 256, 0, st>>>(scores, keys, T, N);
  ec_select_kernel<<<N, EC_THREADS, 0, st>>>(keys, T, N, (int)ec_capacity(s), s.top_k, perm,
                                             row_of, counts, offsets);
  return hipGetLastError();
}

hipError_t launch_ec_combine(const moe_shape& s, const void* y_perm, const void* y_shared,
                             const int32_t* row_of, const float* scores, void* y,
                             hipStream_t st) {
  const int T = (int)s.T, N = s.n_experts, d = s.d_model;
  if (act_bf16(s))
    ec_combine_kernel<bf16_t><<<T, ECC_THREADS, 0, st>>>(
        static_cast<const bf16_t*>(y_perm), static_cast<const bf16_t*>(y_shared), row_of, scores,
        static_cast<bf16_t*>(y), N, d);
  else
    ec_combine_kernel<float><<<T, ECC_THREADS, 0, st>>>(
        static_cast<const float*>(y_perm), static_cast<const float*>(y_shared), row_of, scores,
        static_cast<float*>(y), N, d);
  return hipGetLastError();
}

}  // namespace moe
