/*
 * ssim_oracle.c -- plain, slow, fp64 CPU oracle for the SSIM loss and its
 * gradients.
 *
 * THIS IS TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load it.  It shares no code, header,
 * table or constant with the HIP library: the Gaussian taps, the index maps,
 * the statistics, the SSIM formula, the partial derivatives and the adjoint
 * gather are all written out here again, from the definitions.
 *
 * What it follows (page titles as printed on the source pages):
 *   - "Fully Fused Differentiable SSIM" (fused-ssim README), opening section:
 *     the window is the 11x11 Gaussian of the original SSIM paper, separable
 *     and symmetric; channels are independent; one window serves the mean,
 *     the second moments and the cross moment.
 *   - same page, "Usage": padding "same" (default, output the size of the
 *     input) and "valid" (output shrinks by the window size minus one, the
 *     pytorch-msssim convention); "Constraints": images in [0,1], so the data
 *     range L is 1.
 *   - "TriSSIM -- A Highly Optimized Triton-based Fused SSIM Library",
 *     "How it works": the forward blurs five quantities (mu1, mu2, s11, s22,
 *     s12 = blur of img1, img2, img1^2, img2^2, img1*img2); the backward
 *     applies the adjoint of the blur to the five upstream gradients and
 *     combines them with the chain rule
 *         grad_img1 = B^T g_mu1 + 2 img1 B^T g_s11 + img2 B^T g_s12
 *         grad_img2 = B^T g_mu2 + 2 img2 B^T g_s22 + img1 B^T g_s12.
 *     "Usage": the training loss is 1 - SSIM (SSIM = mean of the map).
 *
 * Readings where the pages are silent: sigma = 1.5, taps sampled at integer
 * offsets and normalised to sum 1; C1 = (0.01 L)^2, C2 = (0.03 L)^2 with
 * L = 1; "same" pads with zeros; the mean runs over all N*C*Ho*Wo map
 * entries with equal weight; no clamping of negative variances.
 *
 * Everything is done the direct way: every windowed sum is a 121-term double
 * loop over the non-separable 11x11 window, and every gradient entry is a
 * direct gather over the (at most 121) map positions whose window covers the
 * input pixel.  No separable passes, no running sums, no fusion.
 *
 * Every function here is pinned by the CPU test suite (closed forms,
 * invariants, finite differences, scipy/torch special cases); none is
 * "parity unpinned".
 *
 * Build: gcc -O2 -fopenmp -fPIC -shared (no -ffast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define WIN 11      /* window side, "Fully Fused Differentiable SSIM" intro */
#define HALF 5      /* centre offset of the window */
#define SIGMA 1.5   /* reading: the original SSIM paper's Gaussian */
#define K1 0.01
#define K2 0.03
#define DATA_RANGE 1.0 /* images in [0,1]: fused-ssim "Constraints" */

#define PAD_VALID 0
#define PAD_SAME 1

/* ---------------------------------------------------------------------- */
/* Window                                                                  */
/* ---------------------------------------------------------------------- */

/* 1-D Gaussian taps g[k] ~ exp(-(k-5)^2 / (2 sigma^2)), k = 0..10, normalised
 * so that they sum to one.  The 2-D window is the outer product g g^T
 * (separable, symmetric: fused-ssim intro). */
void oracle_taps(double g[WIN]) {
  double s = 0.0;
  for (int k = 0; k < WIN; ++k) {
    double d = (double)(k - HALF);
    g[k] = exp(-(d * d) / (2.0 * SIGMA * SIGMA));
    s += g[k];
  }
  for (int k = 0; k < WIN; ++k) g[k] /= s;
}

static void window2d(double w[WIN][WIN]) {
  double g[WIN];
  oracle_taps(g);
  for (int a = 0; a < WIN; ++a)
    for (int b = 0; b < WIN; ++b) w[a][b] = g[a] * g[b];
}

double oracle_c1(void) { return (K1 * DATA_RANGE) * (K1 * DATA_RANGE); }
double oracle_c2(void) { return (K2 * DATA_RANGE) * (K2 * DATA_RANGE); }

/* ---------------------------------------------------------------------- */
/* Index map (fused-ssim "Usage": same / valid)                            */
/* ---------------------------------------------------------------------- */

/* Output extent for an H x W input.  valid: (H-10) x (W-10); same: H x W.
 * Returns 0 when the extent is empty (valid with H or W below 11). */
int oracle_out_shape(int64_t H, int64_t W, int padding, int64_t* Ho, int64_t* Wo) {
  if (padding == PAD_VALID) {
    *Ho = H - (WIN - 1);
    *Wo = W - (WIN - 1);
  } else {
    *Ho = H;
    *Wo = W;
  }
  return (*Ho > 0 && *Wo > 0);
}

/* Output (i, j) looks at inputs (i + a - off, j + b - off), a, b in [0, 10].
 * off = 0 for valid, 5 for same (window centred, zeros outside). */
static int offset_of(int padding) { return padding == PAD_VALID ? 0 : HALF; }

/* Input pixel with zero fill outside the image. */
static double pix(const double* img, int64_t H, int64_t W, int64_t r, int64_t c) {
  if (r < 0 || r >= H || c < 0 || c >= W) return 0.0;
  return img[r * W + c];
}

/* ---------------------------------------------------------------------- */
/* B and its adjoint, on their own (used by the adjoint-identity pin)      */
/* ---------------------------------------------------------------------- */

/* out = B(in): direct 121-term windowed sum at every output position. */
void oracle_blur(const double* in, int64_t H, int64_t W, int padding, double* out) {
  double w[WIN][WIN];
  window2d(w);
  int64_t Ho, Wo;
  if (!oracle_out_shape(H, W, padding, &Ho, &Wo)) return;
  const int off = offset_of(padding);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < Ho; ++i)
    for (int64_t j = 0; j < Wo; ++j) {
      double s = 0.0;
      for (int a = 0; a < WIN; ++a)
        for (int b = 0; b < WIN; ++b) s += w[a][b] * pix(in, H, W, i + a - off, j + b - off);
      out[i * Wo + j] = s;
    }
}

/* out = B^T(in): the adjoint of oracle_blur, written as a gather.  Input
 * pixel q = (u, v) collects w[a][b] * in[p] from every output p = (i, j)
 * with u = i + a - off and v = j + b - off ("full" correlation for valid,
 * TriSSIM "How it works"). */
void oracle_blur_adjoint(const double* in, int64_t H, int64_t W, int padding, double* out) {
  double w[WIN][WIN];
  window2d(w);
  int64_t Ho, Wo;
  if (!oracle_out_shape(H, W, padding, &Ho, &Wo)) return;
  const int off = offset_of(padding);
#pragma omp parallel for schedule(static)
  for (int64_t u = 0; u < H; ++u)
    for (int64_t v = 0; v < W; ++v) {
      double s = 0.0;
      for (int a = 0; a < WIN; ++a) {
        int64_t i = u - a + off;
        if (i < 0 || i >= Ho) continue;
        for (int b = 0; b < WIN; ++b) {
          int64_t j = v - b + off;
          if (j < 0 || j >= Wo) continue;
          s += w[a][b] * in[i * Wo + j];
        }
      }
      out[u * W + v] = s;
    }
}

/* ---------------------------------------------------------------------- */
/* SSIM at one output position                                             */
/* ---------------------------------------------------------------------- */

typedef struct {
  double mux, muy, sxx, syy, sxy; /* the five blurred quantities */
  double A1, A2, B1, B2, S;
} stats_t;

/* The five windowed sums at output (i, j) (TriSSIM "How it works": mu1, mu2,
 * s11, s22, s12, where s11 = B(img1^2) is the raw second moment), then the
 * SSIM of the original paper:
 *   sigma_x^2 = sxx - mux^2, sigma_y^2 = syy - muy^2, sigma_xy = sxy - mux muy
 *   S = (2 mux muy + C1)(2 sigma_xy + C2) / ((mux^2 + muy^2 + C1)(sigma_x^2 + sigma_y^2 + C2)) */
static stats_t stats_at(const double* x, const double* y, int64_t H, int64_t W, int off,
                        const double w[WIN][WIN], int64_t i, int64_t j) {
  stats_t s;
  double mux = 0, muy = 0, sxx = 0, syy = 0, sxy = 0;
  for (int a = 0; a < WIN; ++a)
    for (int b = 0; b < WIN; ++b) {
      double xv = pix(x, H, W, i + a - off, j + b - off);
      double yv = pix(y, H, W, i + a - off, j + b - off);
      double wv = w[a][b];
      mux += wv * xv;
      muy += wv * yv;
      sxx += wv * xv * xv;
      syy += wv * yv * yv;
      sxy += wv * xv * yv;
    }
  const double C1 = oracle_c1(), C2 = oracle_c2();
  double vx = sxx - mux * mux;
  double vy = syy - muy * muy;
  double cxy = sxy - mux * muy;
  s.mux = mux;
  s.muy = muy;
  s.sxx = sxx;
  s.syy = syy;
  s.sxy = sxy;
  s.A1 = 2.0 * mux * muy + C1;
  s.A2 = 2.0 * cxy + C2;
  s.B1 = mux * mux + muy * muy + C1;
  s.B2 = vx + vy + C2;
  s.S = (s.A1 * s.A2) / (s.B1 * s.B2);
  return s;
}

/* Partial derivatives of S with respect to the five blurred quantities,
 * obtained by differentiating the formula above term by term:
 *   dS/dsxy = 2 A1 / (B1 B2)
 *   dS/dsxx = dS/dsyy = -S / B2
 *   dS/dmux = 2 muy (A2 - A1) / (B1 B2) + 2 mux S (1/B2 - 1/B1)
 *   dS/dmuy = 2 mux (A2 - A1) / (B1 B2) + 2 muy S (1/B2 - 1/B1) */
static void partials(const stats_t* s, double d[5]) {
  double den = s->B1 * s->B2;
  d[0] = 2.0 * s->muy * (s->A2 - s->A1) / den + 2.0 * s->mux * s->S * (1.0 / s->B2 - 1.0 / s->B1);
  d[1] = 2.0 * s->mux * (s->A2 - s->A1) / den + 2.0 * s->muy * s->S * (1.0 / s->B2 - 1.0 / s->B1);
  d[2] = -s->S / s->B2;
  d[3] = -s->S / s->B2;
  d[4] = 2.0 * s->A1 / den;
}

/* ---------------------------------------------------------------------- */
/* Compensated summation for the mean (Neumaier)                           */
/* ---------------------------------------------------------------------- */

typedef struct {
  double s, c;
} ksum_t;

static void kadd(ksum_t* k, double v) {
  double t = k->s + v;
  if (fabs(k->s) >= fabs(v))
    k->c += (k->s - t) + v;
  else
    k->c += (v - t) + k->s;
  k->s = t;
}
static double kval(const ksum_t* k) { return k->s + k->c; }

/* ---------------------------------------------------------------------- */
/* One (n, c) plane                                                        */
/* ---------------------------------------------------------------------- */

/* SSIM map of one plane (Ho x Wo doubles). */
void oracle_ssim_map_plane(const double* x, const double* y, int64_t H, int64_t W, int padding,
                           double* S_out) {
  double w[WIN][WIN];
  window2d(w);
  int64_t Ho, Wo;
  if (!oracle_out_shape(H, W, padding, &Ho, &Wo)) return;
  const int off = offset_of(padding);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < Ho; ++i)
    for (int64_t j = 0; j < Wo; ++j) S_out[i * Wo + j] = stats_at(x, y, H, W, off, w, i, j).S;
}

/* Sum of the SSIM map of one plane (compensated, row order fixed so that
 * the result does not depend on the thread count), and -- when grad_x or
 * grad_y is non-NULL -- the gradient of  loss = 1 - (sum over all planes)/M
 * with respect to this plane's pixels, times dloss.
 *
 * Gradient (TriSSIM "How it works", chain rule above): with
 * g_q(p) = -(dloss/M) dS/dq at map position p for q in {mux, muy, sxx, syy,
 * sxy}, and B^T written as the gather over the outputs p whose window covers
 * the input pixel u,
 *   grad_x[u] = sum_p w(u - p) (g_mux(p) + 2 x[u] g_sxx(p) + y[u] g_sxy(p))
 *   grad_y[u] = sum_p w(u - p) (g_muy(p) + 2 y[u] g_syy(p) + x[u] g_sxy(p)).
 * Pixels outside the image (same padding) are constants and get nothing. */
double oracle_ssim_plane(const double* x, const double* y, int64_t H, int64_t W, int padding,
                         double M, double dloss, double* grad_x, double* grad_y) {
  double w[WIN][WIN];
  window2d(w);
  int64_t Ho, Wo;
  if (!oracle_out_shape(H, W, padding, &Ho, &Wo)) return 0.0;
  const int off = offset_of(padding);
  const int want_grad = (grad_x != NULL || grad_y != NULL);

  double* g[5] = {0, 0, 0, 0, 0};
  if (want_grad)
    for (int k = 0; k < 5; ++k) g[k] = (double*)malloc(sizeof(double) * (size_t)(Ho * Wo));
  double* rowsum = (double*)malloc(sizeof(double) * (size_t)Ho);

#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < Ho; ++i) {
    ksum_t acc = {0.0, 0.0};
    for (int64_t j = 0; j < Wo; ++j) {
      stats_t s = stats_at(x, y, H, W, off, w, i, j);
      kadd(&acc, s.S);
      if (want_grad) {
        double d[5];
        partials(&s, d);
        for (int k = 0; k < 5; ++k) g[k][i * Wo + j] = -(dloss / M) * d[k];
      }
    }
    rowsum[i] = kval(&acc);
  }
  ksum_t tot = {0.0, 0.0};
  for (int64_t i = 0; i < Ho; ++i) kadd(&tot, rowsum[i]);
  free(rowsum);

  if (want_grad) {
#pragma omp parallel for schedule(static)
    for (int64_t u = 0; u < H; ++u)
      for (int64_t v = 0; v < W; ++v) {
        double gx = 0.0, gy = 0.0;
        const double xu = x[u * W + v], yu = y[u * W + v];
        for (int a = 0; a < WIN; ++a) {
          int64_t i = u - a + off;
          if (i < 0 || i >= Ho) continue;
          for (int b = 0; b < WIN; ++b) {
            int64_t j = v - b + off;
            if (j < 0 || j >= Wo) continue;
            int64_t p = i * Wo + j;
            double wv = w[a][b];
            gx += wv * (g[0][p] + 2.0 * xu * g[2][p] + yu * g[4][p]);
            gy += wv * (g[1][p] + 2.0 * yu * g[3][p] + xu * g[4][p]);
          }
        }
        if (grad_x) grad_x[u * W + v] = gx;
        if (grad_y) grad_y[u * W + v] = gy;
      }
    for (int k = 0; k < 5; ++k) free(g[k]);
  }
  return kval(&tot);
}

/* ---------------------------------------------------------------------- */
/* Whole batch                                                             */
/* ---------------------------------------------------------------------- */

static void widen(const float* src, double* dst, int64_t n) {
  for (int64_t k = 0; k < n; ++k) dst[k] = (double)src[k];
}

/* loss = 1 - (1/M) sum over the N*C planes of the SSIM-map sums, with
 * M = N*C*Ho*Wo (TriSSIM "Usage": loss = 1 - fused_ssim).  Inputs are fp64
 * NCHW.  grad_x / grad_y (fp64 NCHW, nullable) receive dloss * dloss/dimg.
 * Returns 0 on success, -1 on an empty output extent, -2 on bad padding. */
int oracle_ssim_f64(const double* x, const double* y, int64_t N, int64_t C, int64_t H,
                    int64_t W, int padding, double dloss, double* loss, double* grad_x,
                    double* grad_y) {
  if (padding != PAD_VALID && padding != PAD_SAME) return -2;
  int64_t Ho, Wo;
  if (!oracle_out_shape(H, W, padding, &Ho, &Wo)) return -1;
  const double M = (double)N * (double)C * (double)Ho * (double)Wo;
  const int64_t plane = H * W;
  ksum_t tot = {0.0, 0.0};
  for (int64_t pc = 0; pc < N * C; ++pc) {
    double s = oracle_ssim_plane(x + pc * plane, y + pc * plane, H, W, padding, M, dloss,
                                 grad_x ? grad_x + pc * plane : NULL,
                                 grad_y ? grad_y + pc * plane : NULL);
    kadd(&tot, s);
  }
  *loss = 1.0 - kval(&tot) / M;
  return 0;
}

/* Same as oracle_ssim_f64 for fp32 inputs (the exact buffers a GPU run
 * consumes), widened to fp64 one plane at a time. */
int oracle_ssim_f32(const float* x, const float* y, int64_t N, int64_t C, int64_t H,
                    int64_t W, int padding, double dloss, double* loss, double* grad_x,
                    double* grad_y) {
  if (padding != PAD_VALID && padding != PAD_SAME) return -2;
  int64_t Ho, Wo;
  if (!oracle_out_shape(H, W, padding, &Ho, &Wo)) return -1;
  const double M = (double)N * (double)C * (double)Ho * (double)Wo;
  const int64_t plane = H * W;
  double* xd = (double*)malloc(sizeof(double) * (size_t)plane);
  double* yd = (double*)malloc(sizeof(double) * (size_t)plane);
  ksum_t tot = {0.0, 0.0};
  for (int64_t pc = 0; pc < N * C; ++pc) {
    widen(x + pc * plane, xd, plane);
    widen(y + pc * plane, yd, plane);
    double s = oracle_ssim_plane(xd, yd, H, W, padding, M, dloss,
                                 grad_x ? grad_x + pc * plane : NULL,
                                 grad_y ? grad_y + pc * plane : NULL);
    kadd(&tot, s);
  }
  free(xd);
  free(yd);
  *loss = 1.0 - kval(&tot) / M;
  return 0;
}

/* ---------------------------------------------------------------------- */
/* Point samples (for checks at sizes where whole gradients are too slow)  */
/* ---------------------------------------------------------------------- */

/* SSIM map value at output (i, j) of one fp32 plane. */
double oracle_sample_ssim_f32(const float* x, const float* y, int64_t H, int64_t W, int padding,
                              int64_t i, int64_t j) {
  double w[WIN][WIN];
  window2d(w);
  const int off = offset_of(padding);
  /* Widen the (at most) 11x11 neighbourhood into a local zero-padded patch. */
  double px[WIN * WIN], py[WIN * WIN];
  for (int a = 0; a < WIN; ++a)
    for (int b = 0; b < WIN; ++b) {
      int64_t r = i + a - off, c = j + b - off;
      int in = (r >= 0 && r < H && c >= 0 && c < W);
      px[a * WIN + b] = in ? (double)x[r * W + c] : 0.0;
      py[a * WIN + b] = in ? (double)y[r * W + c] : 0.0;
    }
  stats_t s = stats_at(px, py, WIN, WIN, 0, w, 0, 0);
  return s.S;
}

/* Gradient entries at input pixel (u, v) of one fp32 plane, for a loss whose
 * mean runs over M map entries in total, times dloss.  Same gather as
 * oracle_ssim_plane, with each needed map value computed on the spot. */
void oracle_sample_grad_f32(const float* x, const float* y, int64_t H, int64_t W, int padding,
                            double M, double dloss, int64_t u, int64_t v, double* gx,
                            double* gy) {
  double w[WIN][WIN];
  window2d(w);
  int64_t Ho, Wo;
  *gx = 0.0;
  *gy = 0.0;
  if (!oracle_out_shape(H, W, padding, &Ho, &Wo)) return;
  const int off = offset_of(padding);
  const double xu = (double)x[u * W + v], yu = (double)y[u * W + v];
  double sx = 0.0, sy = 0.0;
  for (int a = 0; a < WIN; ++a) {
    int64_t i = u - a + off;
    if (i < 0 || i >= Ho) continue;
    for (int b = 0; b < WIN; ++b) {
      int64_t j = v - b + off;
      if (j < 0 || j >= Wo) continue;
      double px[WIN * WIN], py[WIN * WIN];
      for (int aa = 0; aa < WIN; ++aa)
        for (int bb = 0; bb < WIN; ++bb) {
          int64_t r = i + aa - off, c = j + bb - off;
          int in = (r >= 0 && r < H && c >= 0 && c < W);
          px[aa * WIN + bb] = in ? (double)x[r * W + c] : 0.0;
          py[aa * WIN + bb] = in ? (double)y[r * W + c] : 0.0;
        }
      stats_t s = stats_at(px, py, WIN, WIN, 0, w, 0, 0);
      double d[5];
      partials(&s, d);
      double k = -(dloss / M) * w[a][b];
      sx += k * (d[0] + 2.0 * xu * d[2] + yu * d[4]);
      sy += k * (d[1] + 2.0 * yu * d[3] + xu * d[4]);
    }
  }
  *gx = sx;
  *gy = sy;
}

/* ---------------------------------------------------------------------- */
/* Volumes ("Fully Fused Differentiable SSIM", 3D data)                    */
/* ---------------------------------------------------------------------- */

/* The 3-D SSIM of the page's 3D section keeps the 2-D computation on each XY
 * slice and adds a Z-axis pass of the same window.  Reading: the window is
 * the outer product g g g of the same 11 taps (separable, so 2-D blur of each
 * slice followed by the Z blur is this window exactly); the same constants;
 * the map is over Do x Ho x Wo output voxels with the same valid/same rule on
 * every axis; the loss is 1 - the mean over all N*C*Do*Ho*Wo map entries;
 * gradients go to both volumes.  Volumes are NCDHW. */

static void window3d(double w[WIN][WIN][WIN]) {
  double g[WIN];
  oracle_taps(g);
  for (int a = 0; a < WIN; ++a)
    for (int b = 0; b < WIN; ++b)
      for (int c = 0; c < WIN; ++c) w[a][b][c] = g[a] * g[b] * g[c];
}

int oracle_out_shape3(int64_t D, int64_t H, int64_t W, int padding, int64_t* Do, int64_t* Ho,
                      int64_t* Wo) {
  if (padding == PAD_VALID) {
    *Do = D - (WIN - 1);
    *Ho = H - (WIN - 1);
    *Wo = W - (WIN - 1);
  } else {
    *Do = D;
    *Ho = H;
    *Wo = W;
  }
  return (*Do > 0 && *Ho > 0 && *Wo > 0);
}

/* Voxel with zero fill outside the volume. */
static double vox(const double* v, int64_t D, int64_t H, int64_t W, int64_t z, int64_t r,
                  int64_t c) {
  if (z < 0 || z >= D || r < 0 || r >= H || c < 0 || c >= W) return 0.0;
  return v[(z * H + r) * W + c];
}

/* out = B3(in): direct 1331-term windowed sum at every output voxel. */
void oracle_blur3(const double* in, int64_t D, int64_t H, int64_t W, int padding, double* out) {
  static double w[WIN][WIN][WIN];
  window3d(w);
  int64_t Do, Ho, Wo;
  if (!oracle_out_shape3(D, H, W, padding, &Do, &Ho, &Wo)) return;
  const int off = offset_of(padding);
#pragma omp parallel for schedule(static) collapse(2)
  for (int64_t k = 0; k < Do; ++k)
    for (int64_t i = 0; i < Ho; ++i)
      for (int64_t j = 0; j < Wo; ++j) {
        double s = 0.0;
        for (int a = 0; a < WIN; ++a)
          for (int b = 0; b < WIN; ++b)
            for (int c = 0; c < WIN; ++c)
              s += w[a][b][c] * vox(in, D, H, W, k + a - off, i + b - off, j + c - off);
        out[(k * Ho + i) * Wo + j] = s;
      }
}

/* The five windowed sums at output voxel (k, i, j) and the SSIM, exactly as
 * stats_at in 2-D with the 1331-term window. */
static stats_t stats_at3(const double* x, const double* y, int64_t D, int64_t H, int64_t W,
                         int off, const double w[WIN][WIN][WIN], int64_t k, int64_t i, int64_t j) {
  stats_t s;
  double mux = 0, muy = 0, sxx = 0, syy = 0, sxy = 0;
  for (int a = 0; a < WIN; ++a)
    for (int b = 0; b < WIN; ++b)
      for (int c = 0; c < WIN; ++c) {
        double xv = vox(x, D, H, W, k + a - off, i + b - off, j + c - off);
        double yv = vox(y, D, H, W, k + a - off, i + b - off, j + c - off);
        double wv = w[a][b][c];
        mux += wv * xv;
        muy += wv * yv;
        sxx += wv * xv * xv;
        syy += wv * yv * yv;
        sxy += wv * xv * yv;
      }
  const double C1 = oracle_c1(), C2 = oracle_c2();
  double vx = sxx - mux * mux;
  double vy = syy - muy * muy;
  double cxy = sxy - mux * muy;
  s.mux = mux;
  s.muy = muy;
  s.sxx = sxx;
  s.syy = syy;
  s.sxy = sxy;
  s.A1 = 2.0 * mux * muy + C1;
  s.A2 = 2.0 * cxy + C2;
  s.B1 = mux * mux + muy * muy + C1;
  s.B2 = vx + vy + C2;
  s.S = (s.A1 * s.A2) / (s.B1 * s.B2);
  return s;
}

/* Sum of the SSIM map of one volume and, when grad_x or grad_y is non-NULL,
 * dloss * d(1 - sum/M)/d(voxel), by the same chain rule and gather as the
 * 2-D plane (the adjoint of B3 gathers over the <= 1331 outputs whose window
 * covers the voxel). */
double oracle_ssim3_volume(const double* x, const double* y, int64_t D, int64_t H, int64_t W,
                           int padding, double M, double dloss, double* grad_x, double* grad_y) {
  static double w[WIN][WIN][WIN];
  window3d(w);
  int64_t Do, Ho, Wo;
  if (!oracle_out_shape3(D, H, W, padding, &Do, &Ho, &Wo)) return 0.0;
  const int off = offset_of(padding);
  const int want_grad = (grad_x != NULL || grad_y != NULL);
  const int64_t nout = Do * Ho * Wo;

  double* g[5] = {0, 0, 0, 0, 0};
  if (want_grad)
    for (int q = 0; q < 5; ++q) g[q] = (double*)malloc(sizeof(double) * (size_t)nout);
  double* rowsum = (double*)malloc(sizeof(double) * (size_t)(Do * Ho));

#pragma omp parallel for schedule(static) collapse(2)
  for (int64_t k = 0; k < Do; ++k)
    for (int64_t i = 0; i < Ho; ++i) {
      ksum_t acc = {0.0, 0.0};
      for (int64_t j = 0; j < Wo; ++j) {
        stats_t s = stats_at3(x, y, D, H, W, off, w, k, i, j);
        kadd(&acc, s.S);
        if (want_grad) {
          double d[5];
          partials(&s, d);
          for (int q = 0; q < 5; ++q) g[q][(k * Ho + i) * Wo + j] = -(dloss / M) * d[q];
        }
      }
      rowsum[k * Ho + i] = kval(&acc);
    }
  ksum_t tot = {0.0, 0.0};
  for (int64_t r = 0; r < Do * Ho; ++r) kadd(&tot, rowsum[r]);
  free(rowsum);

  if (want_grad) {
#pragma omp parallel for schedule(static) collapse(2)
    for (int64_t t = 0; t < D; ++t)
      for (int64_t u = 0; u < H; ++u)
        for (int64_t v = 0; v < W; ++v) {
          double gx = 0.0, gy = 0.0;
          const int64_t q0 = (t * H + u) * W + v;
          const double xu = x[q0], yu = y[q0];
          for (int a = 0; a < WIN; ++a) {
            int64_t k = t - a + off;
            if (k < 0 || k >= Do) continue;
            for (int b = 0; b < WIN; ++b) {
              int64_t i = u - b + off;
              if (i < 0 || i >= Ho) continue;
              for (int c = 0; c < WIN; ++c) {
                int64_t j = v - c + off;
                if (j < 0 || j >= Wo) continue;
                int64_t p = (k * Ho + i) * Wo + j;
                double wv = w[a][b][c];
                gx += wv * (g[0][p] + 2.0 * xu * g[2][p] + yu * g[4][p]);
                gy += wv * (g[1][p] + 2.0 * yu * g[3][p] + xu * g[4][p]);
              }
            }
          }
          if (grad_x) grad_x[q0] = gx;
          if (grad_y) grad_y[q0] = gy;
        }
    for (int q = 0; q < 5; ++q) free(g[q]);
  }
  return kval(&tot);
}

/* loss = 1 - (1/M) sum of the SSIM maps of the N*C volumes (fp32 NCDHW,
 * widened to fp64 one volume at a time), M = N*C*Do*Ho*Wo; gradients (fp64
 * NCDHW, nullable) times dloss.  Returns 0, -1 on an empty map, -2 on bad
 * padding. */
int oracle_ssim3_f32(const float* x, const float* y, int64_t N, int64_t C, int64_t D, int64_t H,
                     int64_t W, int padding, double dloss, double* loss, double* grad_x,
                     double* grad_y) {
  if (padding != PAD_VALID && padding != PAD_SAME) return -2;
  int64_t Do, Ho, Wo;
  if (!oracle_out_shape3(D, H, W, padding, &Do, &Ho, &Wo)) return -1;
  const double M = (double)N * (double)C * (double)Do * (double)Ho * (double)Wo;
  const int64_t vol = D * H * W;
  double* xd = (double*)malloc(sizeof(double) * (size_t)vol);
  double* yd = (double*)malloc(sizeof(double) * (size_t)vol);
  ksum_t tot = {0.0, 0.0};
  for (int64_t pc = 0; pc < N * C; ++pc) {
    widen(x + pc * vol, xd, vol);
    widen(y + pc * vol, yd, vol);
    double s = oracle_ssim3_volume(xd, yd, D, H, W, padding, M, dloss,
                                   grad_x ? grad_x + pc * vol : NULL,
                                   grad_y ? grad_y + pc * vol : NULL);
    kadd(&tot, s);
  }
  free(xd);
  free(yd);
  *loss = 1.0 - kval(&tot) / M;
  return 0;
}

/* Gradient entries at voxel (t, u, v) of one fp32 volume, for a loss whose
 * mean runs over M map entries in total, times dloss: the same gather, each
 * needed map value computed on the spot. */
void oracle_sample_grad3_f32(const float* x, const float* y, int64_t D, int64_t H, int64_t W,
                             int padding, double M, double dloss, int64_t t, int64_t u, int64_t v,
                             double* gx, double* gy) {
  static double w[WIN][WIN][WIN];
  window3d(w);
  int64_t Do, Ho, Wo;
  *gx = 0.0;
  *gy = 0.0;
  if (!oracle_out_shape3(D, H, W, padding, &Do, &Ho, &Wo)) return;
  const int off = offset_of(padding);
  const int64_t q0 = (t * H + u) * W + v;
  const double xu = (double)x[q0], yu = (double)y[q0];
  /* Every map voxel whose window covers (t, u, v) reads volume voxels within
   * 10 of it on each axis: copy that 21^3 neighbourhood, zero-filled outside
   * the volume, widened to fp64.  Patch origin: (t, u, v) - 10. */
  enum { P = 2 * WIN - 1 };
  double* px = (double*)malloc(sizeof(double) * P * P * P);
  double* py = (double*)malloc(sizeof(double) * P * P * P);
  const int64_t z0 = t - (WIN - 1), r0 = u - (WIN - 1), c0 = v - (WIN - 1);
  for (int a = 0; a < P; ++a)
    for (int b = 0; b < P; ++b)
      for (int c = 0; c < P; ++c) {
        const int64_t zz = z0 + a, rr = r0 + b, cc = c0 + c;
        const int in = (zz >= 0 && zz < D && rr >= 0 && rr < H && cc >= 0 && cc < W);
        px[(a * P + b) * P + c] = in ? (double)x[(zz * H + rr) * W + cc] : 0.0;
        py[(a * P + b) * P + c] = in ? (double)y[(zz * H + rr) * W + cc] : 0.0;
      }
  double sx = 0.0, sy = 0.0;
  for (int a = 0; a < WIN; ++a) {
    int64_t k = t - a + off;
    if (k < 0 || k >= Do) continue;
    for (int b = 0; b < WIN; ++b) {
      int64_t i = u - b + off;
      if (i < 0 || i >= Ho) continue;
      for (int c = 0; c < WIN; ++c) {
        int64_t j = v - c + off;
        if (j < 0 || j >= Wo) continue;
        /* map voxel (k, i, j) reads volume voxels (k + aa - off, ...), which
         * is patch voxel (k - off - z0 + aa, ...) */
        stats_t s = stats_at3(px, py, P, P, P, 0, w, k - off - z0, i - off - r0, j - off - c0);
        double d[5];
        partials(&s, d);
        double kk = -(dloss / M) * w[a][b][c];
        sx += kk * (d[0] + 2.0 * xu * d[2] + yu * d[4]);
        sy += kk * (d[1] + 2.0 * yu * d[3] + xu * d[4]);
      }
    }
  }
  free(px);
  free(py);
  *gx = sx;
  *gy = sy;
}

/* ---------------------------------------------------------------------- */
/* Threads                                                                 */
/* ---------------------------------------------------------------------- */

void oracle_set_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
