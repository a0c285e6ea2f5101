/*
 * One MoE-layer forward through include/moe.h from plain C: no PyTorch, the
 * HIP runtime API only for device memory, copies and one stream.  Used by
 * tests/test_gpu_c_abi.py, which writes the inputs, runs this program as a
 * child process and checks its outputs against the CPU oracle.
 *
 *   forward <in.bin> <out.bin>
 *
 * in.bin:  int32 T, H, E, K, h_exp, h_shared, dtype (MOE_BF16), flags;
 *          float capacity_factor;
 *          then the activation-dtype tensors x [T,H], w_router [H,E],
 *          w1 [E,H,h_exp], w2 [E,h_exp,H] (h_shared must be 0).
 * out.bin: logits [T,E] f32, topk_ids [T,K] i32, topk_w [T,K] f32,
 *          counts [E], kept [E], offsets [E+1], row_of [T,K], n_dropped [1]
 *          (int32), aux [1] f32, y [T,H] in the activation dtype.
 *
 * Exit status 0 on success; on any failure it prints the failing call and
 * its status or HIP error and exits with 1.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "moe.h"

#define HIP_OK(call)                                                       \
  do {                                                                     \
    hipError_t e_ = (call);                                                \
    if (e_ != hipSuccess) {                                                \
      fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));           \
      exit(1);                                                             \
    }                                                                      \
  } while (0)
#define MOE_OK_(call)                                                      \
  do {                                                                     \
    int s_ = (call);                                                       \
    if (s_ != MOE_OK) {                                                    \
      fprintf(stderr, "%s: %s\n", #call, moe_status_string(s_));           \
      exit(1);                                                             \
    }                                                                      \
  } while (0)

static void* read_dev(FILE* f, size_t bytes) {
  void* host = malloc(bytes ? bytes : 1);
  void* dev = NULL;
  if (!host || fread(host, 1, bytes, f) != bytes) {
    fprintf(stderr, "short input file\n");
    exit(1);
  }
  HIP_OK(hipMalloc(&dev, bytes ? bytes : 1));
  HIP_OK(hipMemcpy(dev, host, bytes, hipMemcpyHostToDevice));
  free(host);
  return dev;
}

static void* dev_alloc(size_t bytes) {
  void* dev = NULL;
  HIP_OK(hipMalloc(&dev, bytes ? bytes : 1));
  return dev;
}

static void write_dev(FILE* f, const void* dev, size_t bytes) {
  void* host = malloc(bytes ? bytes : 1);
  if (!host) exit(1);
  HIP_OK(hipMemcpy(host, dev, bytes, hipMemcpyDeviceToHost));
  if (fwrite(host, 1, bytes, f) != bytes) {
    fprintf(stderr, "write failed\n");
    exit(1);
  }
  free(host);
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s <in.bin> <out.bin>\n", argv[0]);
    return 2;
  }
  FILE* in = fopen(argv[1], "rb");
  if (!in) {
    perror(argv[1]);
    return 1;
  }
  int32_t hdr[8];
  float cf;
  if (fread(hdr, sizeof hdr, 1, in) != 1 || fread(&cf, sizeof cf, 1, in) != 1) {
    fprintf(stderr, "bad header\n");
    return 1;
  }
  moe_shape s = {0};
  s.T = hdr[0];
  s.H = hdr[1];
  s.E = hdr[2];
  s.K = hdr[3];
  s.h_exp = hdr[4];
  s.h_shared = hdr[5];
  s.dtype = hdr[6];
  s.flags = (uint32_t)hdr[7];
  s.capacity_factor = cf;
  MOE_OK_(moe_check_shape(&s));
  if (s.h_shared != 0) {
    fprintf(stderr, "this example runs without a shared expert\n");
    return 1;
  }
  const size_t b = s.dtype == MOE_BF16 ? 2 : 4;
  const size_t T = (size_t)s.T, H = (size_t)s.H, E = (size_t)s.E, K = (size_t)s.K;
  const size_t h = (size_t)s.h_exp;
  const size_t rows = (size_t)moe_max_rows(&s);

  void* x = read_dev(in, T * H * b);
  void* w_r = read_dev(in, H * E * b);
  void* w1 = read_dev(in, E * H * h * b);
  void* w2 = read_dev(in, E * h * H * b);
  fclose(in);

  float* logits = (float*)dev_alloc(T * E * 4);
  int32_t* topk_ids = (int32_t*)dev_alloc(T * K * 4);
  float* topk_w = (float*)dev_alloc(T * K * 4);
  int32_t* counts = (int32_t*)dev_alloc(E * 4);
  int32_t* kept = (int32_t*)dev_alloc(E * 4);
  int32_t* offsets = (int32_t*)dev_alloc((E + 1) * 4);
  int32_t* row_of = (int32_t*)dev_alloc(T * K * 4);
  int32_t* token_of = (int32_t*)dev_alloc(rows * 4);
  int32_t* n_dropped = (int32_t*)dev_alloc(4);
  float* aux = (float*)dev_alloc(4);
  void* xp = dev_alloc(rows * H * b);
  void* hbuf = dev_alloc(rows * h * b);
  void* out = dev_alloc(rows * H * b);
  void* y = dev_alloc(T * H * b);
  const size_t ws_bytes = moe_workspace_size(&s);
  void* ws = dev_alloc(ws_bytes);

  hipStream_t st;
  HIP_OK(hipStreamCreate(&st));
  MOE_OK_(moe_route(&s, x, w_r, NULL, logits, topk_ids, topk_w, ws, ws_bytes, st));
  MOE_OK_(moe_aux_loss(&s, ws, ws_bytes, aux, st));
  MOE_OK_(moe_permute(&s, x, topk_ids, ws, ws_bytes, counts, kept, offsets, row_of, token_of,
                      n_dropped, xp, st));
  MOE_OK_(moe_expert_ffn(&s, xp, offsets, w1, w2, hbuf, out, NULL, NULL, NULL, NULL, NULL, ws,
                         ws_bytes, st));
  MOE_OK_(moe_combine(&s, out, row_of, topk_w, NULL, y, st));
  HIP_OK(hipStreamSynchronize(st));
  HIP_OK(hipStreamDestroy(st));

  FILE* o = fopen(argv[2], "wb");
  if (!o) {
    perror(argv[2]);
    return 1;
  }
  write_dev(o, logits, T * E * 4);
  write_dev(o, topk_ids, T * K * 4);
  write_dev(o, topk_w, T * K * 4);
  write_dev(o, counts, E * 4);
  write_dev(o, kept, E * 4);
  write_dev(o, offsets, (E + 1) * 4);
  write_dev(o, row_of, T * K * 4);
  write_dev(o, n_dropped, 4);
  write_dev(o, aux, 4);
  write_dev(o, y, T * H * b);
  fclose(o);

  void* bufs[] = {x,  w_r,   w1,     w2,   logits, topk_ids, topk_w, counts, kept, offsets,
                  row_of, token_of, n_dropped, aux, xp, hbuf, out, y, ws};
  for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i) HIP_OK(hipFree(bufs[i]));
  printf("forward ok: T=%d H=%d E=%d K=%d h=%d\n", s.T, s.H, s.E, s.K, s.h_exp);
  return 0;
}
