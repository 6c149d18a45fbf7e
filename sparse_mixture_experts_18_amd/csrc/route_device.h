// Device-side pieces of the routing and work-list steps, shared by their
// own kernels and by the fused small-batch routing tail (router.hip): the
// per-token score and top-k selection of one wave, the one-block dispatch of
// up to 512 assignments, and the work-list builder.
#pragma once

#include "moe_internal.h"

namespace moe {

// exclusive prefix sums of two values over the block (blockDim.x a multiple
// of 64, at most 1024): scans inside each wave with lane shuffles, then one
// wave scans the wave totals; integer, so exact
__device__ __forceinline__ void block_exclusive_scan2(int* sh0, int* sh1, int v0, int v1,
                                                      int& ex0, int& ex1, int& tot0,
                                                      int& tot1) {
  const int i = threadIdx.x, lane = i & 63, w = i >> 6, nw = blockDim.x >> 6;
  int a = v0, b = v1;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int ta = __shfl_up(a, o, 64), tb = __shfl_up(b, o, 64);
    if (lane >= o) {
      a += ta;
      b += tb;
    }
  }
  __syncthreads();  // the scratch may still be read by a previous call
  if (lane == 63) {
    sh0[w] = a;
    sh1[w] = b;
  }
  __syncthreads();
  if (w == 0) {
    int ca = lane < nw ? sh0[lane] : 0, cb = lane < nw ? sh1[lane] : 0;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const int ta = __shfl_up(ca, o, 64), tb = __shfl_up(cb, o, 64);
      if (lane >= o) {
        ca += ta;
        cb += tb;
      }
    }
    if (lane < nw) {
      sh0[32 + lane] = ca;  // inclusive wave prefixes
      sh1[32 + lane] = cb;
    }
  }
  __syncthreads();
  const int pa = w ? sh0[32 + w - 1] : 0, pb = w ? sh1[32 + w - 1] : 0;
  ex0 = pa + a - v0;
  ex1 = pb + b - v1;
  tot0 = sh0[32 + nw - 1];
  tot1 = sh1[32 + nw - 1];
}

// Cost of an item for the XCD split: (live 32-row sub-tiles + a fixed part for
// the weight slice every item streams) x k-slices.
constexpr int kCostFixed = 2;

// Work-list header (int32): [0] item count, [1..9] XCD range starts
// (xcd x owns items [hdr[1+x], hdr[2+x])), [16..23] per-XCD item counters.
constexpr int kHdrStart = 1, kHdrCtr = 16, kHdrDone = 24;  // header: 32 ints

struct PlanArgs {
  const int32_t* offsets;  // [N+1] segment offsets (NULL: no routed segments)
  int N, T, has_shared, bm1, bm2, nt1_r, nt1_s, nt2_r, nt2_s, k1_r, k1_s, k2_r, k2_s;
  WorkItem* plan1;
  int32_t* hdr1;
  WorkItem* plan2;
  int32_t* hdr2;
  int deal;
};

// the work-list arguments of a shape's expert projections (grouped_gemm.hip)
PlanArgs plan_args(const moe_shape& s, const int32_t* offsets, const Workspace& w);

// Builds work list `pass` (0: GEMM1, 1: GEMM2) for a block of up to 1024
// threads (a multiple of 64, at least N + has_shared of them).
__device__ __forceinline__ void plan_device(const PlanArgs& a, int pass) {
  const int32_t* offsets = a.offsets;
  const int N = a.N, T = a.T, has_shared = a.has_shared, bm1 = a.bm1, bm2 = a.bm2;
  const int nt1_r = a.nt1_r, nt1_s = a.nt1_s, nt2_r = a.nt2_r, nt2_s = a.nt2_s;
  const int k1_r = a.k1_r, k1_s = a.k1_s, k2_r = a.k2_r, k2_s = a.k2_s;
  WorkItem* plan1 = a.plan1;
  int32_t* hdr1 = a.hdr1;
  WorkItem* plan2 = a.plan2;
  int32_t* hdr2 = a.hdr2;
  const int deal = a.deal;
  __shared__ int sh0[64], sh1[64];
  __shared__ int st1s[1025], st2s[1025], mt1s[1024], mt2s[1024], rbases[1024], rowss[1024];
  __shared__ long long ucost[1024];
  __shared__ int uslot[1024];
  const int s = threadIdx.x, nthr = blockDim.x;
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
  const int mt1 = (rows + bm1 - 1) / bm1, mt2 = (rows + bm2 - 1) / bm2;
  int st1, st2, tot1, tot2;
  block_exclusive_scan2(sh0, sh1, mt1 * n1t, mt2 * n2t, st1, st2, tot1, tot2);
  st1s[s] = st1;
  st2s[s] = st2;
  mt1s[s] = mt1;
  mt2s[s] = mt2;
  rbases[s] = rbase;
  rowss[s] = rows;
  if (s == 0) {
    st1s[nthr] = tot1;
    st2s[nthr] = tot2;
  }
  __syncthreads();
  {
    const int* st = pass ? st2s : st1s;
    const int* mts = pass ? mt2s : mt1s;
    const int kr = (pass ? k2_r : k1_r) / 64, ks = (pass ? k2_s : k1_s) / 64;
    WorkItem* plan = pass ? plan2 : plan1;
    int32_t* hdr = pass ? hdr2 : hdr1;
    const int tot = pass ? tot2 : tot1;
    // Lists of routed experts on the wide tiles.  Units: each routed expert
    // (all its column tiles) and each column tile of the shared expert.  A
    // unit's cost is the sum of its items' costs (32-row sub-tiles plus a
    // fixed part, times k-slices).  Units are ranked by cost (descending,
    // ties by index) and dealt to the 8 XCDs in snake order (ranks 0..7 to
    // XCDs 0..7, ranks 8..15 to XCDs 7..0, ...): every XCD gets the same
    // total and a similar mix, and a unit never straddles two XCDs, so a
    // list of about one item per CU leaves no CU with two.  Each XCD's range
    // takes its units alternately from the large and the small end of its
    // share (largest, smallest, second largest, ...), so compute-bound and
    // weight-bound items run side by side; inside a unit, column tile then
    // row block, so sibling row blocks of one weight slab are drawn in a
    // row.  The small-row tiles stream the weights at a cost that hardly
    // depends on the rows, so their lists keep the plain order and an
    // equal-cost cut at item granularity.
    const int nrt = pass ? nt2_r : nt1_r, nst = pass ? nt2_s : nt1_s;
    const int U = N + (has_shared ? nst : 0);
    if (deal && N > 0 && U + 8 <= nthr) {
      long long c = -1;  // threads without a unit rank after every unit
      int useg = 0, t0 = 0, t1 = 0;
      if (s < U) {
        useg = s < N ? s : N;
        t0 = s < N ? 0 : s - N;
        t1 = s < N ? nrt : t0 + 1;
        const int R = rowss[useg], mt = mts[useg];
        c = 0;
        if (mt > 0) {
          // row blocks as in the walk below: mt - 1 blocks of `part` rows
          const int part = ((R + mt - 1) / mt + 31) / 32 * 32;
          const long long sub = (long long)(mt - 1) * (part / 32) + (R - (mt - 1) * part + 31) / 32;
          c = (long long)(t1 - t0) * (sub + (long long)kCostFixed * mt) * (useg < N ? kr : ks);
        }
      }
      ucost[s] = c;
      uslot[s] = -1;
      __syncthreads();
      const int R8 = (U + 7) >> 3;
      if (s < U) {
        int rank = 0;
        for (int v = 0; v < U; ++v) {
          const long long cv = ucost[v];
          rank += (cv > c) || (cv == c && v < s);
        }
        const int rd = rank >> 3, p = rank & 7;
        const int x = (rd & 1) ? 7 - p : p;
        // position of round rd in the XCD's order 0, R8-1, 1, R8-2, ...
        const int j = rd <= (R8 - 1) / 2 ? 2 * rd : 2 * (R8 - 1 - rd) + 1;
        uslot[x * R8 + j] = s;
      }
      __syncthreads();
      // thread q lays out slot q: XCD q / R8, position q % R8
      const int u = uslot[s];
      int useg2 = 0, u0 = 0, u1 = 0, mt = 0;
      if (u >= 0) {
        useg2 = u < N ? u : N;
        u0 = u < N ? 0 : u - N;
        u1 = u < N ? nrt : u0 + 1;
        mt = mts[useg2];
      }
      int base, dummy_ex, total, dummy_tot;
      block_exclusive_scan2(sh0, sh1, mt * (u1 - u0), 0, base, dummy_ex, total, dummy_tot);
      if (s == 0) {
        hdr[0] = total;
        hdr[kHdrStart + 8] = total;
        for (int x = 0; x < 8; ++x) hdr[kHdrCtr + x] = 0;
        hdr[kHdrDone] = 0;
      }
      if (s < 8 * R8 && s % R8 == 0) hdr[kHdrStart + s / R8] = base;
      if (total <= 64 * U) {  // a few items per unit: each slot's thread writes its own
        if (u >= 0 && mt > 0) {
          const int R = rowss[useg2];
          const int part = ((R + mt - 1) / mt + 31) / 32 * 32;
          int i = base;
          for (int nt = u0; nt < u1; ++nt)
            for (int m = 0; m < mt; ++m)
              plan[i++] = WorkItem{useg2, rbases[useg2] + m * part, min(part, R - m * part), nt};
        }
        return;
      }
      // many items per unit (few experts with many column tiles: one thread
      // writing an expert's hundreds of items took most of the 24 us of
      // mixtral's plan): the block writes them together; item i belongs to
      // the last slot whose base is <= i (slots without items have the next
      // slot's base)
      st1s[s] = base;  // (the segment starts are no longer needed)
      if (s == 0) st1s[nthr] = total;
      __syncthreads();
      for (int i = s; i < total; i += nthr) {
        int lo = 0, hi = nthr - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (st1s[mid] <= i) lo = mid;
          else hi = mid - 1;
        }
        const int v = uslot[lo];
        const int sg = v < N ? v : N;
        const int t0v = v < N ? 0 : v - N;
        const int mtv = mts[sg], R = rowss[sg];
        const int part = ((R + mtv - 1) / mtv + 31) / 32 * 32;
        const int loc = i - st1s[lo], m = loc % mtv, nt = t0v + loc / mtv;
        plan[i] = WorkItem{sg, rbases[sg] + m * part, min(part, R - m * part), nt};
      }
      return;
    }
    // Otherwise (one-segment dense lists): items in segment-major, then column
    // tile, then row block order.  Thread s fills a contiguous chunk of the
    // list; the list is then cut into 8 ranges of equal cost, one per XCD.
    const int chunk = (tot + nthr - 1) / nthr;
    const int i0 = min(tot, s * chunk), i1 = min(tot, i0 + chunk);
    // segment of item i0: the last segment with st[seg] <= i0 (empty ones skipped)
    int seg0 = 0;
    {
      int lo = 0, hi = nthr - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (st[mid] <= i0) lo = mid;
        else hi = mid - 1;
      }
      seg0 = lo;
    }
    // walk the chunk: (segment, column tile, row block) advance incrementally
    auto walk = [&](auto&& visit) {
      int seg = seg0;
      int loc = i0 - st[seg];
      int mt = max(mts[seg], 1);
      int m = loc % mt, nt = loc / mt;
      for (int i = i0; i < i1; ++i) {
        while (i >= st[seg + 1]) {  // next non-empty segment
          ++seg;
          mt = max(mts[seg], 1);
          m = 0;
          nt = 0;
        }
        // a segment's rows are cut into mt near-equal, 32-aligned row blocks,
        // so the row blocks that share a weight slab run at the same pace
        const int part = ((rowss[seg] + mt - 1) / mt + 31) / 32 * 32;
        const int nr = min(part, rowss[seg] - m * part);
        const int cost = (((nr + 31) >> 5) + kCostFixed) * (seg < N ? kr : ks);
        visit(i, WorkItem{seg, rbases[seg] + m * part, nr, nt}, cost);
        if (++m == mt) {
          m = 0;
          ++nt;
        }
      }
    };
    int local = 0;
    walk([&](int i, const WorkItem& it, int c) {
      plan[i] = it;
      local += c;
    });
    int pre, dummy_ex, total, dummy_tot;
    block_exclusive_scan2(sh0, sh1, local, 0, pre, dummy_ex, total, dummy_tot);
    // boundary x = first item i with 8 * cost(items < i) >= x * total
    if (s == 0) {
      hdr[0] = tot;
      hdr[kHdrStart] = 0;
      hdr[kHdrStart + 8] = tot;
      for (int x = 0; x < 8; ++x) hdr[kHdrCtr + x] = 0;
      hdr[kHdrDone] = 0;
      if (total == 0)
        for (int x = 1; x < 8; ++x) hdr[kHdrStart + x] = 0;
    }
    if (total > 0) {
      long long cum = pre;
      walk([&](int i, const WorkItem&, int c) {
        for (int x = 1; x < 8; ++x) {
          const long long tgt = (long long)x * total;
          if (8 * cum < tgt && tgt <= 8 * (cum + c)) hdr[kHdrStart + x] = i + 1;
        }
        cum += c;
      });
    }
  }
}


// ---------------------------------------------------------------------------
// scores and top-k selection: one wavefront per token, lane l holding experts
// [l*P, l*P+P)
// ---------------------------------------------------------------------------
// total order used for selection: NaN lowest, -0 == +0; 0 is reserved for
// "not a candidate"
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 1u;  // NaN
  if (u == 0x80000000u) u = 0u;
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return u + 1u;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
constexpr int TK_WAVES = 4;

// One wavefront selects for token t_raw (a token >= T computes on token T-1
// and writes nothing).  keys_lds: 512 floats, gsc / gsel: 64 entries, all
// private to the wave; with n_groups > 1 the calls __syncthreads(), so every
// wave of the block must make the call.
template <int P>
__device__ __forceinline__ void topk_token(
    int t_raw, float* keys_w, float* gsc_w, int* gsel_w, const float* __restrict__ logits,
    int nparts, float* __restrict__ logits_out, const float* __restrict__ logit_add,
    int logits_are_scores, const float* __restrict__ bias, float* __restrict__ scores_out,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_w, int T, int N, int k,
    int score_fn, int renorm, int n_groups, int topk_groups) {
  const int lane = threadIdx.x & 63;
  const bool valid = t_raw < T;  // tail waves compute on token T-1, write nothing
  const int t = valid ? t_raw : T - 1;
  const float* lrow = logits + (size_t)t * N;
  float s[P];
  uint32_t ok[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    int e = lane * P + p;
    float v = -INFINITY;
    if (e < N) {
      v = lrow[e];
      // partial sums of a k-split router GEMM: added in chunk order, the
      // order a single pass over the chunks uses
      for (int c = 1; c < nparts; ++c) v += lrow[(size_t)c * T * N + e];
      if (logits_out && valid) logits_out[(size_t)t * N + e] = v;
      if (logit_add && !logits_are_scores) v += logit_add[(size_t)t * N + e];
    }
    s[p] = v;
  }
  if (!logits_are_scores) {
    if (score_fn == MOE_SCORE_SOFTMAX) {
      float m = s[0];
#pragma unroll
      for (int p = 1; p < P; ++p) m = fmaxf(m, s[p]);
      m = wave_max(m);
      float sum = 0.f;
#pragma unroll
      for (int p = 0; p < P; ++p) {
        int e = lane * P + p;
        s[p] = e < N ? expf(s[p] - m) : 0.f;
        sum += s[p];
      }
      sum = wave_sum(sum);
      const float inv = 1.0f / sum;
#pragma unroll
      for (int p = 0; p < P; ++p) s[p] = s[p] * inv;
    } else {
#pragma unroll
      for (int p = 0; p < P; ++p) s[p] = 1.0f / (1.0f + expf(-s[p]));
    }
  }
#pragma unroll
  for (int p = 0; p < P; ++p) {
    int e = lane * P + p;
    if (e < N) {
      if (scores_out && valid) scores_out[(size_t)t * N + e] = s[p];
      float key = bias ? s[p] + bias[e] : s[p];
      ok[p] = order_key(key);
      keys_w[e] = key;
    } else {
      ok[p] = 0u;
    }
  }
  if (n_groups > 1) {  // uniform across the block
    // group score: fl32 sum of the best m keys of the group, best first
    const int gsz = N / n_groups, m = k / topk_groups;
    // groups of whole lanes (gsz = lpg * P, lpg a power of two) with m <= 2:
    // the group's best two (key, index) pairs by a shuffle reduction over its
    // lpg lanes.  A pair is the 64-bit (order key, ~index), so the larger one
    // is the larger key, then the lower index -- the order of the serial scan
    // below, which serves every other shape.
    const int lpg = gsz / P;
    const bool whole = m <= 2 && gsz == lpg * P && lpg <= 64 && (lpg & (lpg - 1)) == 0;
    if (whole) {
      uint64_t b1 = 0, b2 = 0;  // this lane's best two (0: none)
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int e = lane * P + p;
        const uint64_t c = e < N ? ((uint64_t)ok[p] << 32) | (uint32_t)~(uint32_t)e : 0ull;
        if (c > b1) {
          b2 = b1;
          b1 = c;
        } else if (c > b2) {
          b2 = c;
        }
      }
      for (int off = 1; off < lpg; off <<= 1) {
        const uint64_t o1 = ((uint64_t)(uint32_t)__shfl_xor((int)(b1 >> 32), off, 64) << 32) |
                            (uint32_t)__shfl_xor((int)(uint32_t)b1, off, 64);
        const uint64_t o2 = ((uint64_t)(uint32_t)__shfl_xor((int)(b2 >> 32), off, 64) << 32) |
                            (uint32_t)__shfl_xor((int)(uint32_t)b2, off, 64);
        const uint64_t n1 = b1 > o1 ? b1 : o1;
        const uint64_t lo = b1 > o1 ? o1 : b1, hi2 = b2 > o2 ? b2 : o2;
        b2 = lo > hi2 ? lo : hi2;
        b1 = n1;
      }
      const int g = lane / lpg;
      if (lane % lpg == 0 && g < n_groups) {
        const float v1 = keys_w[~(uint32_t)b1];
        gsc_w[g] = m == 1 ? v1 : v1 + keys_w[~(uint32_t)b2];
      }
    }
    __syncthreads();
    if (!whole && lane < n_groups) {
      const float* gk = &keys_w[lane * gsz];
      float acc = 0.f;
      uint32_t prev_o = 0xffffffffu;
      int prev_i = -1;
      for (int r = 0; r < m; ++r) {
        // next key after (prev_o, prev_i) in the order (key desc, index asc)
        uint32_t bo = 0u;
        int bi = -1;
        float bv = 0.f;
        for (int i = 0; i < gsz; ++i) {
          uint32_t o = order_key(gk[i]);
          bool after = (o < prev_o) || (o == prev_o && i > prev_i);
          if (after && (bi < 0 || o > bo)) {
            bo = o;
            bi = i;
            bv = gk[i];
          }
        }
        acc = (r == 0) ? bv : acc + bv;
        prev_o = bo;
        prev_i = bi;
      }
      gsc_w[lane] = acc;
    }
    __syncthreads();
    if (lane < n_groups) {
      uint32_t mine = order_key(gsc_w[lane]);
      int rank = 0;
      for (int g = 0; g < n_groups; ++g) {
        uint32_t o = order_key(gsc_w[g]);
        rank += (o > mine) || (o == mine && g < lane);
      }
      gsel_w[lane] = rank < topk_groups;
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < P; ++p) {
      int e = lane * P + p;
      if (e < N && !gsel_w[e / gsz]) ok[p] = 0u;
    }
  }
  // Selection: the k largest (key, -index) pairs among the candidates
  // (ok > 0; a valid shape has at least k).  tau, the k-th largest order key,
  // is found bit by bit from wave ballots; every key above tau is taken, then
  // the ties at tau in ascending expert order.  Lane j then receives the pick
  // of rank j (key descending, index ascending): the order in which k rounds
  // of arg-max would take them.
  uint32_t tau = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t cand = tau | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int p = 0; p < P; ++p) cnt += __popcll(__ballot(ok[p] >= cand));
    if (cnt >= k) tau = cand;
  }
  int need = k;  // ties at tau to take
  int below = 0;  // ties at tau in the lanes below this one
#pragma unroll
  for (int p = 0; p < P; ++p) {
    need -= __popcll(__ballot(ok[p] > tau));
    const uint64_t tm = __ballot(ok[p] == tau);
    below += __builtin_amdgcn_mbcnt_hi((uint32_t)(tm >> 32),
                                       __builtin_amdgcn_mbcnt_lo((uint32_t)tm, 0u));
  }
  uint64_t selm[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const bool tie = ok[p] == tau;
    selm[p] = __ballot(ok[p] > tau || (tie && below < need));
    below += tie;
  }
  int my_e = 0;
  float my_s = 0.f;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    for (uint64_t m = selm[p]; m; m &= m - 1) {
      const int l = __builtin_ctzll(m);
      const uint32_t okm = __builtin_amdgcn_readlane(ok[p], l);
      const float sm = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s[p]), l));
      const int em = l * P + p;
      int rank = 0;
#pragma unroll
      for (int q = 0; q < P; ++q)
        rank += __popcll(__ballot(ok[q] > okm || (ok[q] == okm && lane * P + q < em)));
      if (lane == rank) {
        my_e = em;
        my_s = sm;
      }
    }
  }
  // renormalise: fp32 sum in ascending j
  float sum = 0.f;
  for (int j = 0; j < k; ++j)
    sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_s), j));
  if (valid && lane < k) {
    topk_idx[(size_t)t * k + lane] = my_e;
    topk_w[(size_t)t * k + lane] = renorm ? my_s / sum : my_s;
  }
}


// ---------------------------------------------------------------------------
// dispatch of one chunk of up to kDispatchChunk assignments in one block
// ---------------------------------------------------------------------------
constexpr int kDispatchWaves = kDispatchChunk / kWave;

// the three steps in one block when all assignments fit one chunk (decode
// batches): the chunk base positions are all zero, so the chunk's histogram
// is the expert counts; same integer results as the three launches
// (a block of exactly kDispatchChunk threads)
__device__ __forceinline__ void dispatch_one_chunk(
    const int32_t* __restrict__ topk_idx, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ slot, int32_t* __restrict__ perm,
    int32_t* __restrict__ nkd, int A, int N, long long C) {
  __shared__ int cnt[kDispatchWaves][512];
  __shared__ int sh[512];
  __shared__ int off[512];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int i = tid; i < kDispatchWaves * 512; i += kDispatchChunk) (&cnt[0][0])[i] = 0;
  __syncthreads();
  const int a = tid;
  int e = a < A ? topk_idx[a] : -1;
  if (e >= N || e < 0) e = -1;
  int r = 0;
  bool last = true;
  for (int j = 0; j < kWave; ++j) {
    const int ej = __builtin_amdgcn_readlane(e, j);
    if (ej == e) {
      r += j < lane;
      last = last && !(j > lane);
    }
  }
  if (e >= 0 && last) cnt[wv][e] = r + 1;
  __syncthreads();
  int kept = 0;
  if (tid < N) {
    int run = 0;
#pragma unroll
    for (int w = 0; w < kDispatchWaves; ++w) {
      const int v = cnt[w][tid];
      cnt[w][tid] = run;
      run += v;
    }
    counts[tid] = run;
    kept = C < 0 ? run : (int)min((long long)run, C);
  }
  sh[tid] = kept;
  __syncthreads();
  for (int o = 1; o < 512; o <<= 1) {
    int v = tid >= o ? sh[tid - o] : 0;
    __syncthreads();
    sh[tid] += v;
    __syncthreads();
  }
  off[tid] = sh[tid] - kept;
  if (tid < N) offsets[tid] = sh[tid] - kept;
  if (tid == 0) {
    const int R = sh[511];
    offsets[N] = R;
    nkd[0] = R;
    nkd[1] = A - R;
  }
  __syncthreads();
  if (a < A) {
    int sl = -1;
    if (e >= 0) {
      const int pos = cnt[wv][e] + r;
      if (C < 0 || pos < C) {
        sl = off[e] + pos;
        perm[sl] = a;
      }
    }
    slot[a] = sl;
  }
}


}  // namespace moe
