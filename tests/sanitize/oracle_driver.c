/*
 * Driver of the oracle (oracle/gdn_oracle.c) for its AddressSanitizer /
 * UndefinedBehaviorSanitizer build.  Usage: oracle_driver IN OUT
 *
 * IN:  int32 T, S, D, io_dtype, beta_mode, has_state, threads; then q, k, v
 *      (T*S*D elements of 4, 2 or 1 bytes each), gamma and beta (T float32
 *      each), and state_in (D*D float64) when has_state.
 * OUT: out (T*S*D float64), state_out (D*D float64), norms (T float64).
 *
 * Before the case it runs the oracle's argument checks on invalid calls and
 * fails (exit 3) if one of them is accepted.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_gdn_head(int T, int S, int D, int io_dtype, int beta_mode, const void* q, const void* k,
                    const void* v, const float* gamma, const float* beta, const double* state_in, double* out,
                    double* state_out, double* norms, int threads);

static void* read_n(FILE* f, size_t n) {
  void* p = malloc(n ? n : 1);
  if (!p || fread(p, 1, n, f) != n) {
    fprintf(stderr, "short input\n");
    exit(2);
  }
  return p;
}

int main(int argc, char** argv) {
  if (argc != 3) return 2;
  float g1 = 1.0f, b1 = 0.5f;
  uint16_t x1 = 0x3f80;
  double s1 = 0.0;
  /* invalid calls: each must be refused */
  if (oracle_gdn_head(-1, 1, 1, 1, 0, &x1, &x1, &x1, &g1, &b1, NULL, NULL, &s1, NULL, 1) == 0 ||
      oracle_gdn_head(1, 0, 1, 1, 0, &x1, &x1, &x1, &g1, &b1, NULL, NULL, &s1, NULL, 1) == 0 ||
      oracle_gdn_head(1, 1, 0, 1, 0, &x1, &x1, &x1, &g1, &b1, NULL, NULL, &s1, NULL, 1) == 0 ||
      oracle_gdn_head(1, 1, 1, 3, 0, &x1, &x1, &x1, &g1, &b1, NULL, NULL, &s1, NULL, 1) == 0 ||
      oracle_gdn_head(1, 1, 1, 1, 2, &x1, &x1, &x1, &g1, &b1, NULL, NULL, &s1, NULL, 1) == 0 ||
      oracle_gdn_head(1, 1, 1, 1, 0, NULL, &x1, &x1, &g1, &b1, NULL, NULL, &s1, NULL, 1) == 0) {
    fprintf(stderr, "an invalid call was accepted\n");
    return 3;
  }
  FILE* f = fopen(argv[1], "rb");
  if (!f) return 2;
  int32_t h[7];
  if (fread(h, sizeof h, 1, f) != 1) return 2;
  const int T = h[0], S = h[1], D = h[2], io = h[3], mode = h[4], has_state = h[5], threads = h[6];
  const size_t esz = io == 0 ? 4 : io == 1 ? 2 : 1;
  const size_t n = (size_t)T * S * D;
  void* q = read_n(f, n * esz);
  void* k = read_n(f, n * esz);
  void* v = read_n(f, n * esz);
  float* gamma = (float*)read_n(f, (size_t)T * sizeof(float));
  float* beta = (float*)read_n(f, (size_t)T * sizeof(float));
  double* sin = has_state ? (double*)read_n(f, (size_t)D * D * sizeof(double)) : NULL;
  fclose(f);
  double* out = (double*)malloc((n ? n : 1) * sizeof(double));
  double* sout = (double*)malloc((size_t)D * D * sizeof(double));
  double* norms = (double*)malloc((T ? (size_t)T : 1) * sizeof(double));
  const int rc = oracle_gdn_head(T, S, D, io, mode, q, k, v, gamma, beta, sin, out, sout, norms, threads);
  if (rc != 0) {
    fprintf(stderr, "oracle_gdn_head returned %d\n", rc);
    return 4;
  }
  FILE* o = fopen(argv[2], "wb");
  if (!o) return 2;
  fwrite(out, sizeof(double), n, o);
  fwrite(sout, sizeof(double), (size_t)D * D, o);
  fwrite(norms, sizeof(double), (size_t)T, o);
  fclose(o);
  free(q); free(k); free(v); free(gamma); free(beta); free(sin); free(out); free(sout); free(norms);
  return 0;
}
