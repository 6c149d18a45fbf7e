// Internal declarations shared by the HIP translation units of libmoe.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

typedef unsigned short bf16_t;  // raw bf16 bits in memory

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v) << 16);
}

// round to nearest even; NaN stays a quiet NaN
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

// ---- MXFP8 (OCP Microscaling v1.0: E4M3 elements, one E8M0 scale per 32
// consecutive values along the reduction axis) ----
constexpr int kMxBlock = 32;

// shared exponent X of a block from its largest magnitude (NaN excluded by
// the caller): floor(log2(amax)) - 8, 8 being the exponent of the top E4M3
// binade, clamped to [-127, 127]; zero (and any fp32 subnormal maximum)
// gives -127, an infinite maximum 127.  Stored as the E8M0 byte X + 127.
__device__ __forceinline__ int mx_shared_exp(float amax) {
  const uint32_t u = __float_as_uint(amax);
  if (u >= 0x7f800000u) return 127;
  const int X = (int)(u >> 23) - 127 - 8;
  return ((u >> 23) == 0 || X < -127) ? -127 : X;
}

// E4M3 code of v / 2^X: nearest, ties to the even mantissa, saturating at
// 448; NaN gives the NaN code; the sign bit is kept.  The scaling by 2^-X is
// exact except for results far below the smallest code (which round to 0).
__device__ __forceinline__ uint32_t e4m3_code(float v, int X) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  if (!(a == a)) return sign | 0x7Fu;
  const float s = ldexpf(a, -X);
  if (!(s < 448.0f)) return sign | 0x7Eu;
  if (s < 0.015625f) return sign | (uint32_t)rintf(s * 512.0f);  // subnormals: 2^-9 steps
  // round the fp32 mantissa to 3 bits at bit 20 (ties to even); a carry
  // moves into the exponent, which is what the next binade's code needs
  const uint32_t us = __float_as_uint(s);
  const uint32_t r = us + 0x7FFFFu + ((us >> 20) & 1u);
  return sign | ((r >> 20) - (120u << 3));
}

constexpr int kWave = 64;
constexpr int kDispatchChunk = 512;  // assignments ranked by one block

// Grouped-GEMM tile geometry of the fp32 path (VALU tiles); the bf16 tile
// families are defined with their kernel.
constexpr int kBMf = 32;
constexpr int kBNf = 32;

// activations (x, y, y_perm, y_shared) are bf16 in bf16 and MXFP8 layers
inline bool act_bf16(const moe_shape& s) { return s.dtype != MOE_DTYPE_F32; }

// one unit of grouped-GEMM work: rows [row0, row0+nrows) of segment `seg`
// (seg < N: routed expert, seg == N: shared expert), output column tile `nt`
struct WorkItem {
  int seg, row0, nrows, nt;
};

struct Workspace {
  float* logits;
  float* scores;
  int32_t* topk_idx;
  float* topk_w;
  int32_t* counts;
  int32_t* offsets;
  int32_t* slot;
  int32_t* perm;
  int32_t* nkd;
  int32_t* rank;
  int32_t* hist;
  int32_t* base;
  int32_t* plan1_hdr;
  WorkItem* plan1;
  int32_t* plan2_hdr;
  WorkItem* plan2;
  void* h;         // routed h [T*k, d_ff], then shared h [T, d_ff_shared]
  void* h_shared;
  void* y_perm;    // [T*k, d]
  void* y_shared;  // [T, d]
  double* pmean;   // [N] mean score per expert (balancing step)
  bf16_t* wsplit;  // [3][N][d] bf16 terms of the fp32 router weight (bf16 layers)
  float* router_part;  // [chunks][T][N] partial logits of the split router GEMM
  double* stats_rows;  // [T*k + T][4] per-row output moments (telemetry)
  double* stats_ent;   // [T][2] per-token gate / score entropy (telemetry)
  int32_t* ec_row;     // [T][N] row of each (token, expert) pair, expert choice
  unsigned char* xq;   // MXFP8 layers: x as a packed MX matrix [T, d]
  size_t total;
  int64_t plan1_cap, plan2_cap;
};

// Carve `ws` (may be NULL to only compute sizes) for a validated shape.
Workspace layout_workspace(const moe_shape& s, void* ws);

// LatentMoE: the routing regions of the full shape, the expert regions of the
// latent shape (d_model = d_latent, no shared expert), the latent rows z and
// y_lat, the shared expert's h and output, and the dense work lists
struct LatentWorkspace {
  Workspace w;
  void *z, *y_lat, *h_sh, *y_sh;
  WorkItem *plan_sh1, *plan_down, *plan_up;
  int32_t *hdr_sh1, *hdr_down, *hdr_up;
  int64_t cap_sh1, cap_down, cap_up;
  size_t total;
};
moe_shape latent_expert_shape(const moe_shape& s, int d_latent);
LatentWorkspace layout_latent(const moe_shape& s, int d_latent, void* ws);

int64_t capacity_of(const moe_shape& s);  // -1 = dropless

constexpr int kStatsGlobal = 16;   // doubles of global indicators
constexpr int kStatsPerExpert = 8; // doubles per expert row (N routed + 1 shared)

// ---- launchers (validated arguments; return hipError_t of the launch) ----
hipError_t launch_router_gemm(const moe_shape& s, const void* x, const float* w_router,
                              float* logits, const Workspace& w, hipStream_t st, int* nparts);
// logits: x W_r^T (nparts == 1) or nparts k-chunk partial-sum planes [nparts][T][N]
// to be added in chunk order; logits_out (optional) receives the summed x W_r^T
hipError_t launch_topk(const moe_shape& s, const float* logits, int nparts, float* logits_out,
                       const float* logit_add, bool logits_are_scores, const float* bias,
                       float* scores_out, int32_t* topk_idx, float* topk_w, hipStream_t st);
hipError_t launch_dispatch(const moe_shape& s, const int32_t* topk_idx, int32_t* counts,
                           int32_t* offsets, int32_t* slot, int32_t* perm, int32_t* nkd,
                           const Workspace& w, hipStream_t st);
hipError_t launch_plan(const moe_shape& s, const int32_t* offsets, const Workspace& w,
                       hipStream_t st);
hipError_t launch_gemm1(const moe_shape& s, const void* x, const int32_t* perm, const void* w1,
                        const void* w1s, void* h, void* hs, const Workspace& w,
                        hipStream_t st);
hipError_t launch_gemm2(const moe_shape& s, const void* h, const void* hs, const void* w2,
                        const void* w2s, void* y_perm, void* y_shared, const Workspace& w,
                        hipStream_t st);
hipError_t launch_combine(const moe_shape& s, const void* y_perm, const void* y_shared,
                          const int32_t* slot, const float* topk_w, void* y, hipStream_t st);
hipError_t launch_bias_update(const moe_shape& s, const int32_t* counts, const float* scores,
                              float step, float clamp, float* bias, float* aux_out,
                              double* p_scratch, hipStream_t st);
void plan_caps(const moe_shape& s, int64_t& cap1, int64_t& cap2);
int router_split_chunks(const moe_shape& s);  // 0: router GEMM not split

hipError_t launch_router_stats(const moe_shape& s, const int32_t* counts, const int32_t* offsets,
                               const float* topk_w, const float* scores, const float* bias,
                               const void* y_perm, const void* y_shared, double* stats,
                               const Workspace& w, hipStream_t st);
hipError_t launch_bias_update_seq(const moe_shape& s, const int32_t* topk_idx,
                                  const int32_t* seq_off, int n_seq, float step, float clamp,
                                  float* bias, int32_t* err, const Workspace& w, hipStream_t st);

// dense products over the T rows of a shape (one work-list segment)
int64_t dense_plan_cap(const moe_shape& s, int Nout, bool gated);
hipError_t launch_dense_plan(const moe_shape& s, bool gated1, int K1, int Nout1, WorkItem* p1,
                             int32_t* h1, int K2, int Nout2, WorkItem* p2, int32_t* h2,
                             hipStream_t st);
hipError_t launch_dense(const moe_shape& s, bool gated, const void* a, const void* b, void* c,
                        const void* addend, int K, int Nout, const WorkItem* plan, int32_t* hdr,
                        int64_t cap, hipStream_t st);

// MXFP8 quantisation of a [rows, cols] bf16/fp32 matrix (cols % 32 == 0)
hipError_t launch_mx_quantize(const void* in, int in_dtype, int64_t rows, int64_t cols,
                              unsigned char* codes, unsigned char* scales, hipStream_t st);

// expert choice: per-expert capacity min(C, T) (-1 without a capacity)
int64_t ec_capacity(const moe_shape& s);
hipError_t launch_ec_select(const moe_shape& s, const float* scores, int32_t* counts,
                            int32_t* offsets, int32_t* perm, int32_t* row_of, const Workspace& w,
                            hipStream_t st);
hipError_t launch_ec_combine(const moe_shape& s, const void* y_perm, const void* y_shared,
                             const int32_t* row_of, const float* scores, void* y,
                             hipStream_t st);

// Direct global -> LDS loads through a buffer resource: the base address
// sits in scalar registers, each lane supplies a 32-bit offset and a
// uniform offset (a k-slice) goes in the scalar soffset, so a load costs one
// VGPR.  Lane i of a wave writes its 16 bytes to lds_wave_base + 16 i.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const unsigned char* base,
                                            uint32_t bytes = 0xFFFFFFFFu) {
  // raw buffer (stride 0) of `bytes` bytes; reads past the end return 0;
  // gfx9 dword 3
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(base), (short)0,
                                           (int)bytes, 0x00020000);
}
// cache-policy bits of a buffer load (the aux operand): nt, streaming data
constexpr int kNonTemporal = 2;
template <int AUX = 0>
__device__ __forceinline__ void dma16(rsrc_t r, uint32_t voff, uint32_t soff,
                                      unsigned char* lds_wave_base) {
  typedef __attribute__((address_space(3))) void* lptr_t;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lptr_t)(lds_wave_base), 16, voff, soff, 0, AUX);
}

// wait until at most n vector-memory ops of this wave are outstanding (they
// retire in order)
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

}  // namespace moe
