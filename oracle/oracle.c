/*
 * Oracle primitives for the chunked causal-conv video decoder. TEST INFRASTRUCTURE ONLY:
 * nothing on the product path may link, load or call this file; only the tests, the smoke
 * check and the bench's CPU-baseline leg use it.
 *
 * Plain, slow, obviously correct CPU code. Tensors are dense fp32 arrays in [C][T][H][W]
 * order (batch 1). Every sum is accumulated in double, in one fixed order per output
 * element, and rounded to fp32 once at the end of the op. A product of two fp32 values is
 * exact in double, so a fused multiply-add and a separate multiply and add give the same
 * bits here. The per-element summation order does not depend on the tensor's extent in
 * time, so a chunked evaluation and a one-shot evaluation of the same element agree bit for
 * bit. OpenMP splits the work over independent output elements only; there is no
 * cross-thread reduction, so results do not depend on the thread count.
 *
 * Source of the definitions: the FastVideo compare page "[perf] PAN2 sampling: Wan2.2 VAE
 * decode kernel, split decode, fused DiT kernels", its reference decoder (reference.py):
 * the docstring's part list and the functions causal_conv, rms_norm and the SiLU use in
 * residual_block. Each function below names the part it follows.
 *
 * Parity pins: see the header of oracle/__init__.py; every function here is pinned.
 */
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ROW_BLOCK 8

/*
 * Causal 3-D convolution (the page's causal conv part and its causal_conv function).
 * The conv is a cross-correlation with stride 1. In space it zero-pads kh/2 rows and
 * kw/2 columns on both sides. In time it places P = 2*(kt/2) frames in front of x: first
 * P - Th zero frames, then the Th history frames `hist` (oldest first), and no frame after.
 *
 *   y[o,t,h,w] = b[o] + sum_c sum_i sum_j sum_k  W[o,c,i,j,k] * xt[c, t+i, h+j-kh/2, w+k-kw/2]
 *
 * where xt is the padded sequence, and taps that fall on a zero (pad frame, pad row or
 * pad column) contribute nothing. The sum runs c outermost, then i, j, k.
 *
 * x    [C][T][H][W]       hist [C][Th][H][W] (NULL when Th == 0), Th <= P
 * w    [Co][C][kt][kh][kw] b   [Co] or NULL (zero bias)
 * y    [Co][T][H][W]
 * Returns 0, or -1 on an invalid argument.
 */
int orc_causal_conv3d(const float* x, int C, int T, int H, int W, const float* hist, int Th,
                      const float* w, int Co, int kt, int kh, int kw, const float* b, float* y) {
  const int P = 2 * (kt / 2);
  if (C <= 0 || T < 0 || H <= 0 || W <= 0 || Co <= 0 || kt <= 0 || kh <= 0 || kw <= 0) return -1;
  if (Th < 0 || Th > P || (Th > 0 && !hist)) return -1;
  if (T == 0) return 0;
  const int ph = kh / 2, pw = kw / 2;
  const int64_t plane = (int64_t)H * W;
  const int nhb = (H + ROW_BLOCK - 1) / ROW_BLOCK;
  const int64_t items = (int64_t)Co * T * nhb;

#pragma omp parallel
  {
    double* acc = (double*)malloc(sizeof(double) * ROW_BLOCK * (size_t)W);
#pragma omp for schedule(dynamic, 1)
    for (int64_t it = 0; it < items; ++it) {
      const int o = (int)(it / ((int64_t)T * nhb));
      const int t = (int)((it / nhb) % T);
      const int h0 = (int)(it % nhb) * ROW_BLOCK;
      const int nh = (h0 + ROW_BLOCK <= H) ? ROW_BLOCK : H - h0;
      const double bias = b ? (double)b[o] : 0.0;
      for (int r = 0; r < nh * W; ++r) acc[r] = bias;
      for (int c = 0; c < C; ++c) {
        for (int i = 0; i < kt; ++i) {
          /* padded frame index u = t + i; frames u < P are the front padding */
          const int u = t + i;
          const float* src;
          if (u >= P) {
            src = x + ((int64_t)c * T + (u - P)) * plane;
          } else if (u >= P - Th) {
            src = hist + ((int64_t)c * Th + (u - (P - Th))) * plane;
          } else {
            continue; /* zero frame */
          }
          for (int j = 0; j < kh; ++j) {
            for (int k = 0; k < kw; ++k) {
              const double wv = (double)w[((((int64_t)o * C + c) * kt + i) * kh + j) * kw + k];
              const int dx = k - pw;
              const int wlo = dx < 0 ? -dx : 0;
              const int whi = dx > 0 ? W - dx : W;
              for (int hh = 0; hh < nh; ++hh) {
                const int sh = h0 + hh + j - ph;
                if (sh < 0 || sh >= H) continue; /* zero row */
                const float* srow = src + (int64_t)sh * W + dx;
                double* arow = acc + (int64_t)hh * W;
                for (int ww = wlo; ww < whi; ++ww) arow[ww] += wv * (double)srow[ww];
              }
            }
          }
        }
      }
      float* dst = y + ((int64_t)o * T + t) * plane + (int64_t)h0 * W;
      for (int r = 0; r < nh * W; ++r) dst[r] = (float)acc[r];
    }
    free(acc);
  }
  return 0;
}

/*
 * RMS norm over channels (the page's RMS norm part), in the form
 *   y[c,p] = gamma[c] * x[c,p] / sqrt(mean_c x[c,p]^2 + eps)
 * at every position p of the P positions (P = T*H*W). The mean of squares is summed in
 * double in channel order; the quotient and the product are formed in double and rounded
 * once. x, y: [C][P]; gamma: [C]. y may alias x.
 */
int orc_rms_norm(const float* x, int C, int64_t P, const float* gamma, double eps, float* y) {
  if (C <= 0 || P < 0 || !gamma) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t p = 0; p < P; ++p) {
    double ss = 0.0;
    for (int c = 0; c < C; ++c) {
      const double v = (double)x[(int64_t)c * P + p];
      ss += v * v;
    }
    const double inv = 1.0 / sqrt(ss / (double)C + eps);
    for (int c = 0; c < C; ++c) {
      const int64_t idx = (int64_t)c * P + p;
      y[idx] = (float)((double)gamma[c] * ((double)x[idx] * inv));
    }
  }
  return 0;
}

/*
 * SiLU (the activation between norm and conv in the page's residual block part):
 * y = x / (1 + exp(-x)), in double, rounded once. y may alias x.
 */
int orc_silu(const float* x, int64_t n, float* y) {
  if (n < 0) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    const double v = (double)x[i];
    y[i] = (float)(v / (1.0 + exp(-v)));
  }
  return 0;
}

/* Thread count the OpenMP runtime will use (reported beside the oracle's timings). */
int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
