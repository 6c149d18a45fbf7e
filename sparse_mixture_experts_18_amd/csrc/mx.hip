// MXFP8 quantisation (OCP Microscaling Formats v1.0): every block of 32
// consecutive values of a row gets one E8M0 power-of-two scale 2^X with
// X = floor(log2 max|v|) - 8, and every value the E4M3 code of v / 2^X
// (nearest, ties to even, saturating).  Used for the expert weights (once,
// when they are loaded) and for the token rows of a layer with MXFP8
// experts; the SwiGLU intermediate is quantised in the grouped GEMM's
// epilogue with the same rule.  MXFP8 expert compute with the router kept
// in fp32: "MoE common taste of open models", section 2 and the closing
// recipe table; "MoE architecture in practice", precision section.
//
// Packed layout of an MX matrix of R rows and K values per row: R*K code
// bytes (row-major), then R*K/32 scale bytes (row-major, X + 127).
#include "moe_internal.h"

namespace moe {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <typename IN>
__device__ __forceinline__ void load32(const IN* p, float (&v)[32]);

template <>
__device__ __forceinline__ void load32<bf16_t>(const bf16_t* p, float (&v)[32]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const u32x4_t w = reinterpret_cast<const u32x4_t*>(p)[q];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[8 * q + 2 * e] = __uint_as_float(w[e] << 16);
      v[8 * q + 2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
  }
}

template <>
__device__ __forceinline__ void load32<float>(const float* p, float (&v)[32]) {
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const u32x4_t w = reinterpret_cast<const u32x4_t*>(p)[q];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[4 * q + e] = __uint_as_float(w[e]);
  }
}

// one thread per block of 32 values; the blocks of a row-major matrix whose
// row length is a multiple of 32 are its consecutive runs of 32 elements
template <typename IN>
__global__ __launch_bounds__(256) void mx_quantize_kernel(const IN* __restrict__ in,
                                                          long long nblocks,
                                                          unsigned char* __restrict__ codes,
                                                          unsigned char* __restrict__ scales) {
  for (long long b = (long long)blockIdx.x * 256 + threadIdx.x; b < nblocks;
       b += (long long)gridDim.x * 256) {
    float v[32];
    load32<IN>(in + b * kMxBlock, v);
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float a = fabsf(v[i]);
      amax = a > amax ? a : amax;  // NaN never wins
    }
    const int X = mx_shared_exp(amax);
    u32x4_t w0, w1;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      w0[q] = e4m3_code(v[4 * q], X) | (e4m3_code(v[4 * q + 1], X) << 8) |
              (e4m3_code(v[4 * q + 2], X) << 16) | (e4m3_code(v[4 * q + 3], X) << 24);
      w1[q] = e4m3_code(v[16 + 4 * q], X) | (e4m3_code(v[16 + 4 * q + 1], X) << 8) |
              (e4m3_code(v[16 + 4 * q + 2], X) << 16) | (e4m3_code(v[16 + 4 * q + 3], X) << 24);
    }
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(codes + b * kMxBlock);
    dst[0] = w0;
    dst[1] = w1;
    scales[b] = (unsigned char)(X + 127);
  }
}

}  // namespace

hipError_t launch_mx_quantize(const void* in, int in_dtype, int64_t rows, int64_t cols,
                              unsigned char* codes, unsigned char* scales, hipStream_t st) {
  const long long nblocks = rows * cols / kMxBlock;
  if (nblocks <= 0) return hipSuccess;
  long long grid = (nblocks + 255) / 256;
  if (grid > 8192) grid = 8192;
  if (in_dtype == MOE_DTYPE_F32)
    mx_quantize_kernel<float><<<(int)grid, 256, 0, st>>>(static_cast<const float*>(in), nblocks,
                                                         codes, scales);
  else
    mx_quantize_kernel<bf16_t><<<(int)grid, 256, 0, st>>>(static_cast<const bf16_t*>(in),
                                                          nblocks, codes, scales);
  return hipGetLastError();
}

}  // namespace moe
