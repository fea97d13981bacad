/*
 * Oracle for the frame-wise Gated DeltaNet (GDN) forward recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the package's smoke check and the CPU
 * baseline leg of the benchmark use it.  It shares no code, header, table or
 * helper with the HIP library.
 *
 * What it computes (plain double precision, one head at a time):
 *
 *   Source: "NVIDIA Apresenta SANA-WM: Um Modelo de Mundo de Larga Escala de
 *   2.6 Bilhoes de Parametros ..." (acheiumaia.com.br), section
 *   "1. Atencao Linear Hibrida com Gated DeltaNet (GDN)": SANA-WM replaces
 *   most attention blocks by a GDN that takes one whole latent frame per
 *   recurrent step; the update has a decay gate gamma that down-weights old
 *   frames and a delta-rule correction that writes only the residual between
 *   the target value and what the current state predicts; the state is a
 *   constant D x D matrix; keys are scaled by 1/sqrt(D*S) (D = head dim,
 *   S = spatial tokens per frame) so that the transition keeps a bounded
 *   spectral norm.
 *
 *   Readings of what the page leaves open (each one is listed, with its
 *   reason, in the design notes of the repository):
 *     - feature map phi = ReLU on Q and K, none on V;
 *     - key scale c = 1/sqrt(D*S) on K only; Q unscaled; no normaliser;
 *     - gamma_t, beta_t: one already-activated fp32 scalar per (head, frame);
 *     - decay is applied before the prediction;
 *     - the output reads the post-update state;
 *     - beta placement: ERASE (default) puts beta on the correction term,
 *       WRITE puts it on the whole written residual.
 *
 *   Per frame t (M is [key i][value j], D x D):
 *     Qf  = phi(Q_t)                      S x D
 *     Kf  = c * phi(K_t)                  S x D
 *     Md  = gamma_t * M                   decay
 *     P   = Kf * Md                       prediction of the values
 *     R   = V_t - beta_t * P              (ERASE)
 *     R   = beta_t * (V_t - P)            (WRITE)
 *     M   = Md + Kf^T * R                 delta-rule write
 *     O_t = Qf * M                        readout of the post-update state
 *
 * Every sum runs over its contraction index in natural order (0, 1, 2, ...),
 * whatever the thread count, so the result is bitwise reproducible.  Memory is
 * O(S*D + D*D) per head and does not grow with T.
 *
 * Inputs are read exactly: fp32 values, bf16 bit patterns widened to fp32
 * (exact) and then to double (exact), or OCP 8-bit E4M3 codes decoded from
 * the format's definition (see e4m3_value).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#else
static int omp_get_max_threads(void) { return 1; }
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_ARG 1
#define ORACLE_ERR_NOMEM 2

/* A planted-mistake build (-DORACLE_MUTANT=n) exists only so that a test can
 * show that the pins catch each kind of error; the normal build has 0. */
#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

/* OCP 8-bit float E4M3 ("fn" variant): sign bit, 4 exponent bits with bias 7,
 * 3 mantissa bits; exponent field 0 holds the subnormals m/8 * 2^-6; the
 * all-ones code (exponent 15, mantissa 7) is NaN; there is no infinity. */
static double e4m3_value(uint8_t b) {
  const int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
  double x;
  if (e == 15 && m == 7)
    x = NAN;
  else if (e == 0)
    x = ldexp((double)m, -9);
  else
    x = ldexp(1.0 + m / 8.0, e - 7);
  return s ? -x : x;
}

static double widen(const void* p, int io_dtype, size_t idx) {
  if (io_dtype == 0) return (double)((const float*)p)[idx];
  if (io_dtype == 2) return e4m3_value(((const uint8_t*)p)[idx]);
  uint32_t u = ((uint32_t)((const uint16_t*)p)[idx]) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double relu(double x) { return x > 0.0 ? x : 0.0; }

int oracle_abi_version(void) { return 1; }

/* The E4M3 decoder on its own, for the tests that pin it: n codes -> doubles. */
void oracle_e4m3_decode(const uint8_t* codes, double* out, int n) {
  for (int i = 0; i < n; ++i) out[i] = e4m3_value(codes[i]);
}

/*
 * One head.
 *   T, S, D      frames, tokens per frame, head dim (>= 1 each)
 *   io_dtype     0 = fp32 inputs, 1 = bf16 bit patterns (uint16), 2 = E4M3 codes (uint8)
 *   beta_mode    0 = ERASE, 1 = WRITE
 *   q, k, v      [T][S][D] for this head, row-major
 *   gamma, beta  [T] fp32
 *   state_in     [D][D] double or NULL (zeros)
 *   out          [T][S][D] double or NULL (skip the readout)
 *   state_out    [D][D] double or NULL
 *   norms        [T] double or NULL: Frobenius norm of the post-update state
 *   threads      OpenMP threads (<= 0: runtime default)
 */
int oracle_gdn_head(int T, int S, int D, int io_dtype, int beta_mode,
                    const void* q, const void* k, const void* v,
                    const float* gamma, const float* beta,
                    const double* state_in, double* out, double* state_out,
                    double* norms, int threads) {
  if (T < 0 || S < 1 || D < 1 || io_dtype < 0 || io_dtype > 2 ||
      (beta_mode != 0 && beta_mode != 1))
    return ORACLE_ERR_ARG;
  if (T > 0 && (!q || !k || !v || !gamma || !beta)) return ORACLE_ERR_ARG;

  const size_t SD = (size_t)S * D, DD = (size_t)D * D;
  double* M = (double*)calloc(DD, sizeof(double));
  double* Md = (double*)malloc(DD * sizeof(double));
  double* W = (double*)malloc(DD * sizeof(double));
  double* Qf = (double*)malloc(SD * sizeof(double));
  double* Kf = (double*)malloc(SD * sizeof(double));
  double* Vt = (double*)malloc(SD * sizeof(double));
  double* P = (double*)malloc(SD * sizeof(double));
  double* R = (double*)malloc(SD * sizeof(double));
  double* colsq = (double*)malloc((size_t)D * sizeof(double));
  if (!M || !Md || !W || !Qf || !Kf || !Vt || !P || !R || !colsq) {
    free(M); free(Md); free(W); free(Qf); free(Kf); free(Vt); free(P); free(R); free(colsq);
    return ORACLE_ERR_NOMEM;
  }
  if (state_in) memcpy(M, state_in, DD * sizeof(double));

#if ORACLE_MUTANT == 6
  const double c = 1.0 / sqrt((double)D);          /* planted: wrong key scale */
#else
  const double c = 1.0 / sqrt((double)D * (double)S);
#endif
  const int nt = threads > 0 ? threads : 0;

#pragma omp parallel num_threads(nt > 0 ? nt : omp_get_max_threads())
  {
    for (int t = 0; t < T; ++t) {
      const size_t fo = (size_t)t * SD;
      const double g = (double)gamma[t];
      const double b = (double)beta[t];

      /* feature maps and key scale */
#pragma omp for schedule(static)
      for (int s = 0; s < S; ++s)
        for (int i = 0; i < D; ++i) {
          const size_t x = (size_t)s * D + i;
#if ORACLE_MUTANT == 5
          Qf[x] = widen(q, io_dtype, fo + x);       /* planted: no ReLU on Q */
#else
          Qf[x] = relu(widen(q, io_dtype, fo + x));
#endif
          Kf[x] = c * relu(widen(k, io_dtype, fo + x));
          Vt[x] = widen(v, io_dtype, fo + x);
        }

      /* decay */
#pragma omp for schedule(static)
      for (int i = 0; i < D; ++i)
        for (int j = 0; j < D; ++j) {
#if ORACLE_MUTANT == 1
          Md[(size_t)i * D + j] = M[(size_t)i * D + j];   /* planted: no decay */
#else
          Md[(size_t)i * D + j] = g * M[(size_t)i * D + j];
#endif
        }

      /* prediction P = Kf * Md, then the residual */
#pragma omp for schedule(static)
      for (int s = 0; s < S; ++s) {
        double* prow = P + (size_t)s * D;
        for (int j = 0; j < D; ++j) prow[j] = 0.0;
        for (int i = 0; i < D; ++i) {
          const double kv = Kf[(size_t)s * D + i];
          const double* mrow = Md + (size_t)i * D;
          for (int j = 0; j < D; ++j) prow[j] += kv * mrow[j];
        }
        double* rrow = R + (size_t)s * D;
        const double* vrow = Vt + (size_t)s * D;
        for (int j = 0; j < D; ++j) {
#if ORACLE_MUTANT == 2
          rrow[j] = (beta_mode == 0) ? b * (vrow[j] - prow[j]) : vrow[j] - b * prow[j];  /* planted: modes swapped */
#elif ORACLE_MUTANT == 7
          rrow[j] = (beta_mode == 0) ? vrow[j] + b * prow[j] : b * (vrow[j] + prow[j]);  /* planted: sign */
#else
          rrow[j] = (beta_mode == 0) ? vrow[j] - b * prow[j] : b * (vrow[j] - prow[j]);
#endif
        }
      }

      /* delta-rule write M = Md + Kf^T * R (sum over tokens s in order) */
#pragma omp for schedule(static)
      for (int i = 0; i < D; ++i) {
        double* wrow = W + (size_t)i * D;
        for (int j = 0; j < D; ++j) wrow[j] = 0.0;
        for (int s = 0; s < S; ++s) {
#if ORACLE_MUTANT == 3
          /* planted: transposed key operand (reads Kf[i][s] as if D == S) */
          const double kv = Kf[((size_t)i * D + (size_t)s) % SD];
#else
          const double kv = Kf[(size_t)s * D + i];
#endif
          const double* rrow = R + (size_t)s * D;
          for (int j = 0; j < D; ++j) wrow[j] += kv * rrow[j];
        }
        double* mrow = M + (size_t)i * D;
        const double* mdrow = Md + (size_t)i * D;
        for (int j = 0; j < D; ++j) mrow[j] = mdrow[j] + wrow[j];
      }

      /* readout O_t = Qf * M (post-update state) */
      if (out) {
#if ORACLE_MUTANT == 4
        const double* Mread = Md;                    /* planted: pre-update state */
#else
        const double* Mread = M;
#endif
#pragma omp for schedule(static)
        for (int s = 0; s < S; ++s) {
          double* orow = out + fo + (size_t)s * D;
          for (int j = 0; j < D; ++j) orow[j] = 0.0;
          for (int i = 0; i < D; ++i) {
            const double qv = Qf[(size_t)s * D + i];
            const double* mrow = Mread + (size_t)i * D;
            for (int j = 0; j < D; ++j) orow[j] += qv * mrow[j];
          }
        }
      }

      /* Frobenius norm of the state: column sums in order i, then j */
      if (norms) {
#pragma omp for schedule(static)
        for (int j = 0; j < D; ++j) {
          double acc = 0.0;
          for (int i = 0; i < D; ++i) acc += M[(size_t)i * D + j] * M[(size_t)i * D + j];
          colsq[j] = acc;
        }
#pragma omp single
        {
          double tot = 0.0;
          for (int j = 0; j < D; ++j) tot += colsq[j];
          norms[t] = sqrt(tot);
        }
      }
#pragma omp barrier
    }
  }

  if (state_out) memcpy(state_out, M, DD * sizeof(double));
  free(M); free(Md); free(W); free(Qf); free(Kf); free(Vt); free(P); free(R); free(colsq);
  return ORACLE_OK;
}
