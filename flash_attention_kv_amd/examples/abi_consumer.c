/*
 * abi_consumer.c -- the library used from plain C through include/fakv.h,
 * with no Python: HIP allocations, seeded bf16 inputs, one causal GQA ring
 * prefill (ring_attn_fwd) and one split-KV decode step (splitkv_decode), all
 * on one stream.  Writes the inputs and outputs as raw bf16 to the file named
 * on the command line, so they can be compared with any other caller of the
 * same entry points:
 *   int32 header {T, h_q, h_kv, d, C, B, S, n_chunks}, then prefill q, k, v,
 *   decode q, k, v, prefill o, decode o (each tensor contiguous, token-major).
 * Exit status 0 on success; any failing call prints fakv_last_error().
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "fakv.h"

/* bf16 bits of a value in [-2, 2) from a 32-bit mix of (seed, i) */
static uint16_t gen(uint32_t seed, uint32_t i) {
  uint32_t x = seed * 0x9E3779B9u ^ (i + 0x7F4A7C15u);
  x ^= x >> 16; x *= 0x85EBCA6Bu; x ^= x >> 13; x *= 0xC2B2AE35u; x ^= x >> 16;
  union { float f; uint32_t u; } cv;
  cv.f = (float)(x >> 8) * (4.0f / 16777216.0f) - 2.0f;
  return (uint16_t)((cv.u + 0x7FFFu + ((cv.u >> 16) & 1u)) >> 16);   /* round to nearest even */
}

#define CHECK_HIP(e) do { hipError_t err_ = (e); if (err_ != hipSuccess) { \
  fprintf(stderr, "HIP error %d at line %d\n", (int)err_, __LINE__); return 1; } } while (0)
#define CHECK_FAKV(e) do { fakv_status st_ = (e); if (st_ != FAKV_OK) { \
  fprintf(stderr, "fakv error %d: %s\n", (int)st_, fakv_last_error()); return 1; } } while (0)

static int upload(uint16_t** dev, size_t n, uint32_t seed, FILE* out) {
  uint16_t* h = (uint16_t*)malloc(n * 2);
  if (!h) return 1;
  for (size_t i = 0; i < n; ++i) h[i] = gen(seed, (uint32_t)i);
  CHECK_HIP(hipMalloc((void**)dev, n * 2));
  CHECK_HIP(hipMemcpy(*dev, h, n * 2, hipMemcpyHostToDevice));
  fwrite(h, 2, n, out);
  free(h);
  return 0;
}

static int download(const uint16_t* dev, size_t n, FILE* out) {
  uint16_t* h = (uint16_t*)malloc(n * 2);
  if (!h) return 1;
  CHECK_HIP(hipMemcpy(h, dev, n * 2, hipMemcpyDeviceToHost));
  fwrite(h, 2, n, out);
  free(h);
  return 0;
}

int main(int argc, char** argv) {
  if (argc != 2) { fprintf(stderr, "usage: %s OUTPUT_FILE\n", argv[0]); return 2; }
  /* same major version, at least the minor version this file was written for */
  if (fakv_abi_version() / 100 != 1 || fakv_abi_version() < 101) {
    fprintf(stderr, "unexpected ABI version\n");
    return 1;
  }
  const int32_t T = 300, h_q = 8, h_kv = 2, d = 128, C = 3;      /* prefill: T % C == 0 */
  const int32_t B = 2, S = 1000, n_chunks = 7;                   /* decode */
  FILE* out = fopen(argv[1], "wb");
  if (!out) return 1;
  const int32_t hdr[8] = {T, h_q, h_kv, d, C, B, S, n_chunks};
  fwrite(hdr, 4, 8, out);
  hipStream_t s;
  CHECK_HIP(hipStreamCreate(&s));

  uint16_t *q, *k, *v, *o;
  if (upload(&q, (size_t)T * h_q * d, 1, out) || upload(&k, (size_t)T * h_kv * d, 2, out) ||
      upload(&v, (size_t)T * h_kv * d, 3, out))
    return 1;
  CHECK_HIP(hipMalloc((void**)&o, (size_t)T * h_q * d * 2));
  /* a dense batch needs no workspace */
  if (ring_attn_workspace_bytes(T, T, h_q, h_kv, d, C, 1, 1, 0, FAKV_BF16) != 0) return 1;
  CHECK_FAKV(ring_attn_fwd(q, k, v, o, T, T, h_q, h_kv, d, C, 1, NULL, 1, FAKV_BF16, NULL, 0, s));

  uint16_t *dq, *dk, *dv, *dout;
  if (upload(&dq, (size_t)B * h_q * d, 4, out) || upload(&dk, (size_t)B * S * h_kv * d, 5, out) ||
      upload(&dv, (size_t)B * S * h_kv * d, 6, out))
    return 1;
  CHECK_HIP(hipMalloc((void**)&dout, (size_t)B * h_q * d * 2));
  const size_t wsb = splitkv_decode_workspace_bytes(B, h_q, d, n_chunks);
  void* ws = NULL;
  CHECK_HIP(hipMalloc(&ws, wsb));
  CHECK_FAKV(splitkv_decode(dq, dk, dv, dout, B, h_q, h_kv, d, S, n_chunks, FAKV_BF16, ws, wsb, s));
  /* an invalid call is refused with a message and enqueues nothing */
  if (ring_attn_fwd(q, k, v, o, T, T, 3, 2, d, C, 1, NULL, 1, FAKV_BF16, NULL, 0, s) != FAKV_EINVAL) return 1;

  CHECK_HIP(hipStreamSynchronize(s));
  if (download(o, (size_t)T * h_q * d, out) || download(dout, (size_t)B * h_q * d, out)) return 1;
  fclose(out);
  hipFree(q); hipFree(k); hipFree(v); hipFree(o);
  hipFree(dq); hipFree(dk); hipFree(dv); hipFree(dout); hipFree(ws);
  hipStreamDestroy(s);
  printf("abi_consumer ok\n");
  return 0;
}
