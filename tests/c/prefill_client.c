/*
 * A plain C client of libtilemix (include/tilemix.h) and the HIP runtime C API: one routed
 * prefill (quantize Q and K, pack the route map, size the workspace, run the fused call) on
 * inputs read from files, output written to a file. Used by the test suite to show the
 * boundary is callable without Python; it allocates device memory with hipMalloc itself.
 *
 *   prefill_client DIR          run: reads DIR/{meta.txt,q.bin,k.bin,v.bin,route.bin,
 *                               cu_q.bin,cu_k.bin,cu_m.bin}, writes DIR/out.bin (fp32)
 *   prefill_client --validate   no GPU work: checks that bad arguments are rejected with the
 *                               documented status and a message
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "tilemix.h"

#define CHECK_HIP(x)                                                         \
  do {                                                                       \
    hipError_t e_ = (x);                                                     \
    if (e_ != hipSuccess) {                                                  \
      fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, hipGetErrorString(e_)); \
      return 1;                                                              \
    }                                                                        \
  } while (0)

#define CHECK_TM(x)                                                          \
  do {                                                                       \
    tilemix_status s_ = (x);                                                 \
    if (s_ != TILEMIX_OK) {                                                  \
      fprintf(stderr, "%s:%d: status %d: %s\n", __FILE__, __LINE__, (int)s_, \
              tilemix_last_error());                                         \
      return 1;                                                              \
    }                                                                        \
  } while (0)

static void* read_file(const char* dir, const char* name, size_t* bytes) {
  char path[1024];
  snprintf(path, sizeof(path), "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) return NULL;
  fseek(f, 0, SEEK_END);
  long n = ftell(f);
  fseek(f, 0, SEEK_SET);
  void* buf = malloc(n > 0 ? (size_t)n : 1);
  if (buf && n > 0 && fread(buf, 1, (size_t)n, f) != (size_t)n) {
    free(buf);
    buf = NULL;
  }
  fclose(f);
  *bytes = (size_t)n;
  return buf;
}

static int to_device(const void* host, size_t bytes, void** dev) {
  CHECK_HIP(hipMalloc(dev, bytes > 0 ? bytes : 16));
  if (bytes > 0) CHECK_HIP(hipMemcpy(*dev, host, bytes, hipMemcpyHostToDevice));
  return 0;
}

static int validate(void) {
  int fails = 0;
  tilemix_status s = tilemix_prefill_fwd(NULL, NULL);
  if (s != TILEMIX_EINVAL || strlen(tilemix_last_error()) == 0) ++fails;
  tilemix_fwd_params p;
  memset(&p, 0, sizeof(p));
  p.struct_size = sizeof(p);
  p.head_dim = 96;  /* unsupported */
  s = tilemix_prefill_fwd(&p, NULL);
  if (s != TILEMIX_EUNSUPPORTED) ++fails;
  p.struct_size = 4; /* wrong struct size */
  s = tilemix_prefill_fwd(&p, NULL);
  if (s != TILEMIX_EINVAL) ++fails;
  s = tilemix_pack_route_mask(NULL, 4, 100, NULL, 1, NULL); /* 100 groups do not fit one word */
  if (s != TILEMIX_EINVAL) ++fails;
  s = tilemix_quantize_qk(NULL, 0, 1, 0, 0, NULL, NULL, NULL, 0, 1, 0, 0, NULL, NULL, 80, NULL);
  if (s != TILEMIX_EUNSUPPORTED) ++fails;
  printf("validate: version %d, %d failure(s)\n", tilemix_version(), fails);
  return fails != 0;
}

int main(int argc, char** argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: %s DIR | --validate\n", argv[0]);
    return 2;
  }
  if (strcmp(argv[1], "--validate") == 0) return validate();
  const char* dir = argv[1];

  size_t nb = 0;
  char* meta = (char*)read_file(dir, "meta.txt", &nb);
  if (!meta) return 1;
  int batch, hq, hk, d, bm, bn, g, causal, t_mask, wpr, total_m, max_q, max_k;
  long long total_q, total_k;
  if (sscanf(meta, "%d %d %d %d %lld %lld %d %d %d %d %d %d %d %d %d", &batch, &hq, &hk, &d, &total_q, &total_k,
             &bm, &bn, &g, &causal, &t_mask, &wpr, &total_m, &max_q, &max_k) != 15) {
    fprintf(stderr, "bad meta.txt\n");
    return 1;
  }
  free(meta);

  size_t qb, kb, vb, rb, cqb, ckb, cmb;
  void* q = read_file(dir, "q.bin", &qb);
  void* k = read_file(dir, "k.bin", &kb);
  void* v = read_file(dir, "v.bin", &vb);
  void* route = read_file(dir, "route.bin", &rb);
  void* cu_q = read_file(dir, "cu_q.bin", &cqb);
  void* cu_k = read_file(dir, "cu_k.bin", &ckb);
  void* cu_m = read_file(dir, "cu_m.bin", &cmb);
  if (!q || !k || !v || !route || !cu_q || !cu_k || !cu_m) {
    fprintf(stderr, "missing input file\n");
    return 1;
  }

  void *dq, *dk, *dv, *droute, *dcu_q, *dcu_k, *dcu_m;
  if (to_device(q, qb, &dq) || to_device(k, kb, &dk) || to_device(v, vb, &dv) || to_device(route, rb, &droute) ||
      to_device(cu_q, cqb, &dcu_q) || to_device(cu_k, ckb, &dcu_k) || to_device(cu_m, cmb, &dcu_m))
    return 1;
  void *dq8, *dqs, *dk8, *dks, *dwords, *dout, *dws;
  CHECK_HIP(hipMalloc(&dq8, (size_t)total_q * hq * d));
  CHECK_HIP(hipMalloc(&dqs, (size_t)total_q * hq * 4));
  CHECK_HIP(hipMalloc(&dk8, (size_t)total_k * hk * d));
  CHECK_HIP(hipMalloc(&dks, (size_t)total_k * hk * 4));
  CHECK_HIP(hipMalloc(&dwords, (size_t)hk * total_m * wpr * 8));
  CHECK_HIP(hipMalloc(&dout, (size_t)total_q * hq * d * 4));

  hipStream_t stream;
  CHECK_HIP(hipStreamCreate(&stream));
  CHECK_TM(tilemix_quantize_qk(dq, total_q, hq, (int64_t)hq * d, d, (int8_t*)dq8, (float*)dqs, dk, total_k, hk,
                               (int64_t)hk * d, d, (int8_t*)dk8, (float*)dks, d, stream));
  CHECK_TM(tilemix_pack_route_mask((const uint8_t*)droute, (int64_t)hk * total_m, t_mask, (uint64_t*)dwords, wpr,
                                   stream));

  tilemix_fwd_params p;
  memset(&p, 0, sizeof(p));
  p.struct_size = sizeof(p);
  p.batch = batch;
  p.hq = hq;
  p.hkv = hk;
  p.head_dim = d;
  p.total_q = total_q;
  p.total_k = total_k;
  p.max_seqlen_q = max_q;
  p.max_seqlen_k = max_k;
  p.cu_seqlens_q = (const int32_t*)dcu_q;
  p.cu_seqlens_k = (const int32_t*)dcu_k;
  p.cu_mtiles = (const int32_t*)dcu_m;
  p.total_mtiles = total_m;
  p.q = dq;
  p.q_stride_tok = (int64_t)hq * d;
  p.q_stride_head = d;
  p.k = dk;
  p.k_stride_tok = (int64_t)hk * d;
  p.k_stride_head = d;
  p.v = dv;
  p.v_stride_tok = (int64_t)hk * d;
  p.v_stride_head = d;
  p.q8 = (const int8_t*)dq8;
  p.q_scale = (const float*)dqs;
  p.k8 = (const int8_t*)dk8;
  p.k_scale = (const float*)dks;
  p.route_words = (const uint64_t*)dwords;
  p.words_per_row = wpr;
  p.route_block_m = bm;
  p.route_block_n = bn;
  p.route_group = g;
  p.causal = causal;
  p.softmax_scale = 0.0f;
  p.out = dout;
  p.out_dtype = 1;
  int64_t ws_bytes = 0;
  CHECK_TM(tilemix_prefill_workspace_size(&p, &ws_bytes));
  CHECK_HIP(hipMalloc(&dws, ws_bytes > 0 ? (size_t)ws_bytes : 256));
  p.workspace = dws;
  p.workspace_bytes = ws_bytes;
  CHECK_TM(tilemix_prefill_fwd(&p, stream));
  CHECK_HIP(hipStreamSynchronize(stream));

  size_t ob = (size_t)total_q * hq * d * 4;
  float* out = (float*)malloc(ob);
  CHECK_HIP(hipMemcpy(out, dout, ob, hipMemcpyDeviceToHost));
  char path[1024];
  snprintf(path, sizeof(path), "%s/out.bin", dir);
  FILE* f = fopen(path, "wb");
  if (!f || fwrite(out, 1, ob, f) != ob) return 1;
  fclose(f);
  printf("prefill_client: %lld query rows x %d heads written (workspace %lld bytes)\n", total_q, hq,
         (long long)ws_bytes);

  hipFree(dq); hipFree(dk); hipFree(dv); hipFree(droute); hipFree(dcu_q); hipFree(dcu_k); hipFree(dcu_m);
  hipFree(dq8); hipFree(dqs); hipFree(dk8); hipFree(dks); hipFree(dwords); hipFree(dout); hipFree(dws);
  hipStreamDestroy(stream);
  free(q); free(k); free(v); free(route); free(cu_q); free(cu_k); free(cu_m); free(out);
  return 0;
}
