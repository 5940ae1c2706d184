/* Drives every libdllm entry point through its argument-validation and error
 * paths (no device work is ever enqueued): NULL pointers, out-of-range and
 * inconsistent dimensions, and dllm_create on a host without a GPU.  Built
 * with the host code under AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_sanitize_cpu.py; exits non-zero on the first unexpected status. */
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "libdllm.h"

static int failures = 0;

#define EXPECT(call, want)                                                                     \
  do {                                                                                         \
    const dllm_status got_ = (call);                                                           \
    if (got_ != (want)) {                                                                      \
      fprintf(stderr, "%s:%d %s -> %d, expected %d (%s)\n", __FILE__, __LINE__, #call, got_,     \
              (want), dllm_last_error());                                                      \
      ++failures;                                                                              \
    }                                                                                          \
  } while (0)

static dllm_dims dims(void) {
  dllm_dims d;
  memset(&d, 0, sizeof d);
  d.n_layers = 2; d.d_model = 256; d.n_q_heads = 4; d.n_kv_heads = 4; d.head_dim = 64; d.d_ffn = 1024;
  d.vocab = 1024; d.max_batch = 1; d.seq_len = 128; d.block_len = 32; d.proxy_rank = 16; d.dtype = DLLM_FP32;
  d.rms_eps = 1e-5f; d.rope_theta = 1e4f;
  return d;
}

int main(int argc, char** argv) {
  const int has_gpu = argc > 1 && strcmp(argv[1], "gpu") == 0;
  dllm_model* m = NULL;
  dllm_dims d;

  /* dimension checks */
  EXPECT(dllm_create(NULL, &m), DLLM_E_ARG);
  d = dims(); EXPECT(dllm_create(&d, NULL), DLLM_E_ARG);
  d = dims(); d.head_dim = 63; EXPECT(dllm_create(&d, &m), DLLM_E_SHAPE);
  d = dims(); d.head_dim = 288; EXPECT(dllm_create(&d, &m), DLLM_E_SHAPE);
  d = dims(); d.d_model = 8224; EXPECT(dllm_create(&d, &m), DLLM_E_SHAPE);
  d = dims(); d.n_q_heads = 6; EXPECT(dllm_create(&d, &m), DLLM_E_SHAPE);
  d = dims(); d.seq_len = 9000; EXPECT(dllm_create(&d, &m), DLLM_E_SHAPE);
  d = dims(); d.seq_len = 130; EXPECT(dllm_create(&d, &m), DLLM_E_SHAPE);
  d = dims(); d.block_len = 65; EXPECT(dllm_create(&d, &m), DLLM_E_SHAPE);
  d = dims(); d.proxy_rank = 129; EXPECT(dllm_create(&d, &m), DLLM_E_SHAPE);
  d = dims(); d.dtype = 7; EXPECT(dllm_create(&d, &m), DLLM_E_ARG);
  d = dims(); d.n_layers = 0; EXPECT(dllm_create(&d, &m), DLLM_E_ARG);
  d = dims(); d.vocab = 1; EXPECT(dllm_create(&d, &m), DLLM_E_ARG);
  d = dims(); d.d_model = 250; EXPECT(dllm_create(&d, &m), DLLM_E_SHAPE);
  d = dims(); d.rms_eps = -1.0f; EXPECT(dllm_create(&d, &m), DLLM_E_ARG);
  d = dims(); d.rope_theta = NAN; EXPECT(dllm_create(&d, &m), DLLM_E_ARG);
  d = dims(); d.dtype = DLLM_BF16; d.vocab = 1000; EXPECT(dllm_create(&d, &m), DLLM_E_SHAPE);
  d = dims(); d.dtype = DLLM_BF16; d.n_q_heads = 1; d.n_kv_heads = 1; d.head_dim = 32;
  EXPECT(dllm_create(&d, &m), DLLM_E_SHAPE);
  if (m != NULL) { fprintf(stderr, "model set on failure\n"); ++failures; }
  if (dllm_last_error()[0] == '\0') { fprintf(stderr, "no error text\n"); ++failures; }

  /* a valid shape: with no GPU the HIP runtime's failure comes back as DLLM_E_HIP */
  if (!has_gpu) {
    d = dims();
    EXPECT(dllm_create(&d, &m), DLLM_E_HIP);
    if (m != NULL) { fprintf(stderr, "model set on failure\n"); ++failures; }
    if (strncmp(dllm_last_error(), "hipGetDevice: ", 14) != 0) {
      fprintf(stderr, "unexpected error text: %s\n", dllm_last_error());
      ++failures;
    }
  }

  /* NULL model / state / parameter checks of every entry point */
  EXPECT(dllm_destroy(NULL), DLLM_OK);
  EXPECT(dllm_init_layer(NULL, 0, NULL, NULL), DLLM_E_ARG);
  EXPECT(dllm_init_head(NULL, NULL, NULL, NULL, NULL), DLLM_E_ARG);
  EXPECT(dllm_derive_proxy_basis(NULL, NULL, 1, NULL, NULL), DLLM_E_ARG);
  EXPECT(dllm_derive_proxy_basis_noalloc(NULL, NULL, 1, NULL, NULL), DLLM_E_ARG);
  EXPECT(dllm_embed(NULL, NULL, NULL, NULL, NULL), DLLM_E_ARG);
  EXPECT(dllm_drift_score(NULL, 0, NULL, NULL, NULL, 0, NULL), DLLM_E_ARG);
  EXPECT(dllm_select(NULL, 0, NULL, NULL, NULL, 0.1, NULL, NULL, NULL), DLLM_E_ARG);
  EXPECT(dllm_sparse_layer(NULL, 0, NULL, NULL, NULL, 0, NULL), DLLM_E_ARG);
  EXPECT(dllm_lm_head(NULL, NULL, NULL, NULL, NULL), DLLM_E_ARG);
  EXPECT(dllm_commit(NULL, NULL, 0.9, 2.0, NULL), DLLM_E_ARG);
  EXPECT(dllm_commit_ce(NULL, NULL, NULL, NULL, 0.9, 2.0, NULL), DLLM_E_ARG);
  EXPECT(dllm_polestar_drift(NULL, 0, NULL, NULL, NULL, NULL), DLLM_E_ARG);
  EXPECT(dllm_polestar_select(NULL, 0, NULL, NULL, NULL, NULL, NULL, NULL), DLLM_E_ARG);
  EXPECT(dllm_polestar_commit(NULL, NULL, NULL, NULL, 0.9, 2.0, NULL), DLLM_E_ARG);
  EXPECT(dllm_forced_set(NULL, NULL, DLLM_FORCED_BLOCK, 0, NULL, NULL), DLLM_E_ARG);
  EXPECT(dllm_step(NULL, NULL, NULL, NULL, NULL), DLLM_E_ARG);
  EXPECT(dllm_profile(NULL, 0), DLLM_E_ARG);
  EXPECT(dllm_profile_read(NULL, NULL), DLLM_E_ARG);
  {
    double g = 0.0;
    EXPECT(dllm_stream_probe(NULL, 0, NULL, 1, &g, NULL), DLLM_E_ARG);
    char buf[16];
    EXPECT(dllm_stream_probe(buf, sizeof buf, buf, 1, &g, NULL), DLLM_E_ARG); /* < 256 MiB */
    EXPECT(dllm_stream_probe(buf, (size_t)1 << 30, buf, 0, &g, NULL), DLLM_E_ARG); /* reps < 1 */
  }
  if (failures) {
    fprintf(stderr, "%d unexpected statuses\n", failures);
    return 1;
  }
  printf("all validation paths as documented\n");
  return 0;
}
