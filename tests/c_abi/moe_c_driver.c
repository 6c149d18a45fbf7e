/* Drives the MoE library through its C ABI alone (no Python, no PyTorch):
 * reads a layer from a binary file, runs moe_forward on the GPU and writes
 * the outputs.  Used by the tests to show that include/moe.h is consumable
 * from plain C with device pointers from the HIP runtime.
 *
 *   moe_c_driver <in.bin> <out.bin>
 *
 * in.bin: moe_shape (as laid out in moe.h), then int32 has_bias, has_shared,
 * then x, w_router, bias (if any), w1, w2, w1_shared, w2_shared (if any),
 * each as raw bytes of the sizes moe.h documents.
 * out.bin: y, scores [T,N] fp32, topk_idx [T,k] int32, topk_w [T,k] fp32,
 * counts [N], offsets [N+1], slot [T*k], n_kept_dropped [2] int32. */
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "moe.h"

#define CHECK(cond, msg)                                      \
  do {                                                        \
    if (!(cond)) {                                            \
      fprintf(stderr, "moe_c_driver: %s\n", msg);             \
      return 1;                                               \
    }                                                         \
  } while (0)

static void* load(FILE* f, size_t bytes) {
  void* h = malloc(bytes ? bytes : 1);
  if (h && bytes && fread(h, 1, bytes, f) != bytes) {
    free(h);
    return NULL;
  }
  return h;
}

static void* to_device(const void* h, size_t bytes) {
  void* d = NULL;
  if (hipMalloc(&d, bytes ? bytes : 1) != hipSuccess) return NULL;
  if (bytes && hipMemcpy(d, h, bytes, hipMemcpyHostToDevice) != hipSuccess) return NULL;
  return d;
}

int main(int argc, char** argv) {
  CHECK(argc == 3, "usage: moe_c_driver <in.bin> <out.bin>");
  FILE* f = fopen(argv[1], "rb");
  CHECK(f, "cannot open input");
  moe_shape s;
  int32_t flags[2];
  CHECK(fread(&s, sizeof s, 1, f) == 1 && fread(flags, sizeof flags, 1, f) == 1, "short header");
  CHECK(moe_check_shape(&s) == MOE_OK, "shape rejected");
  const size_t T = (size_t)s.T, d = (size_t)s.d_model, N = (size_t)s.n_experts;
  const size_t k = (size_t)s.top_k, ff = (size_t)s.d_ff, fs = (size_t)s.d_ff_shared;
  const size_t es = s.dtype == MOE_DTYPE_F32 ? 4 : 2;
  CHECK(s.dtype != MOE_DTYPE_MXFP8, "this driver takes fp32 or bf16 layers");
  const size_t bx = T * d * es, bwr = N * d * 4, bb = flags[0] ? N * 4 : 0;
  const size_t bw1 = N * 2 * ff * d * es, bw2 = N * d * ff * es;
  const size_t bw1s = flags[1] ? 2 * fs * d * es : 0, bw2s = flags[1] ? d * fs * es : 0;
  void *hx = load(f, bx), *hwr = load(f, bwr), *hb = load(f, bb), *hw1 = load(f, bw1),
       *hw2 = load(f, bw2), *hw1s = load(f, bw1s), *hw2s = load(f, bw2s);
  fclose(f);
  CHECK(hx && hwr && hb && hw1 && hw2 && hw1s && hw2s, "short input");

  void *x = to_device(hx, bx), *wr = to_device(hwr, bwr), *w1 = to_device(hw1, bw1),
       *w2 = to_device(hw2, bw2);
  void* b = flags[0] ? to_device(hb, bb) : NULL;
  void* w1s = flags[1] ? to_device(hw1s, bw1s) : NULL;
  void* w2s = flags[1] ? to_device(hw2s, bw2s) : NULL;
  CHECK(x && wr && w1 && w2 && (!flags[0] || b) && (!flags[1] || (w1s && w2s)), "hipMalloc");
  const size_t by = T * d * es, bsc = T * N * 4, bk = T * k * 4;
  void *y, *sc, *ti, *tw, *cn, *of, *sl, *nkd, *ws;
  const size_t wsb = moe_workspace_bytes(&s);
  CHECK(wsb > 0, "workspace size");
  CHECK(hipMalloc(&y, by) == hipSuccess && hipMalloc(&sc, bsc) == hipSuccess &&
            hipMalloc(&ti, bk) == hipSuccess && hipMalloc(&tw, bk) == hipSuccess &&
            hipMalloc(&cn, N * 4) == hipSuccess && hipMalloc(&of, (N + 1) * 4) == hipSuccess &&
            hipMalloc(&sl, bk) == hipSuccess && hipMalloc(&nkd, 8) == hipSuccess &&
            hipMalloc(&ws, wsb) == hipSuccess,
        "hipMalloc outputs");

  moe_status st = moe_forward(&s, x, (const float*)wr, NULL, (const float*)b, w1, w2, w1s, w2s,
                              y, (float*)sc, (int32_t*)ti, (float*)tw, (int32_t*)cn,
                              (int32_t*)of, (int32_t*)sl, (int32_t*)nkd, ws, wsb, NULL);
  if (st != MOE_OK) {
    fprintf(stderr, "moe_c_driver: %s\n", moe_status_string(st));
    return 1;
  }
  CHECK(hipDeviceSynchronize() == hipSuccess, "kernel failure");

  FILE* o = fopen(argv[2], "wb");
  CHECK(o, "cannot open output");
  const void* dev[8] = {y, sc, ti, tw, cn, of, sl, nkd};
  const size_t sz[8] = {by, bsc, bk, bk, N * 4, (N + 1) * 4, bk, 8};
  for (int i = 0; i < 8; ++i) {
    void* h = malloc(sz[i]);
    CHECK(h && hipMemcpy(h, dev[i], sz[i], hipMemcpyDeviceToHost) == hipSuccess, "copy back");
    CHECK(fwrite(h, 1, sz[i], o) == sz[i], "write");
    free(h);
  }
  fclose(o);
  printf("moe_c_driver: ok (T=%zu N=%zu k=%zu)\n", T, N, k);
  return 0;
}
