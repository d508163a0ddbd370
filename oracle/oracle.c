/*
 * CPU oracle for the fused forward NHWC convolution.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain reference that the
 * GPU path is checked against.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load it; the library itself never does,
 * and the two share no source, header, table or helper.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fno-fast-math -shared -fPIC
 * (-ffp-contract=off matters: the int8 epilogue below is specified step by
 * step, and a fused multiply-add that the compiler invents would change its
 * rounding.)
 *
 * What is computed, and where the pages define it:
 *
 *  - Output size and padding.  TensorFlow conv_ops_fused_int8.cc,
 *    LaunchFusedConv2DOpGpuInt8Helper, the SAME-padding comment and the
 *    padding_rows / padding_cols expressions: the total SAME padding is
 *    max(0, (Ho-1)*stride + R - H), half (rounded down) goes before, the rest
 *    after.  The output size itself is not printed for SAME; we read it as
 *    ceil(H / stride), the only value for which the Im2col size expression
 *    (TensorFlow conv_grad_filter_ops.cc, Im2col: (H + pt + pb - R)/stride + 1)
 *    returns the same Ho again.  VALID is zero padding, Ho = (H - R)/stride + 1.
 *
 *  - The contraction.  acc[n,ho,wo,k] = sum over r,s,c of
 *    X(n, ho*sh - pt + r, wo*sw - pl + s, c) * w[r,s,c,k], with X zero outside
 *    the image.  Input NHWC, filter HWIO (conv_ops_fused_int8.cc,
 *    LaunchFusedConv2DOpCpuInt8Helper: "input in NHWC and filter in HWIO");
 *    cross-correlation, no filter flip (MXNet cudnn_deconvolution-inl.h,
 *    InitDescriptors, CUDNN_CROSS_CORRELATION).  Two independent forms:
 *      oracle_conv_*_direct   seven nested loops;
 *      oracle_conv_i8_im2col  per image, the patch matrix of Im2col
 *                             (conv_grad_filter_ops.cc, Im2col: rows in (ho,wo)
 *                             order, columns in (r,s,c) order, zero outside the
 *                             image) times the filter viewed as [R*S*C, K].
 *    int8 products are summed exactly in int64 (then checked to fit int32);
 *    bf16 and fp32 products are exact in double and summed in double.
 *
 *  - The int8 epilogue.  conv_ops_fused_int8.cc, BiasActivationOutputKernel,
 *    the cuDNN 8 order: (1) t = acc * conv_input_scale, (2) unless the side
 *    input is absent or side_input_scale is zero, t = fmaf(side,
 *    side_input_scale, t), one rounding, (3) t = t + bias[k]; then round half
 *    to even, clip to [-128, 127] (lower bound 0 under ReLU), cast to int8.
 *    All in fp32; the accumulator is converted to fp32 first.
 *    Two variants from the same kernel: conv_input_scale may be a vector with
 *    one value per output channel (the scale tensor of more than one element,
 *    sliced at the output channel), and the cuDNN 7 order that the comment
 *    there names, whose first step is one fused multiply-add
 *    t = fmaf(acc, conv_input_scale, bias) and whose second is the same side
 *    step as above (read as fmaf(side, side_input_scale, t): the comment
 *    writes both orders' side step alike, and the cuDNN 8 code spells it that
 *    way), with no separate bias step.
 *
 *  - The weight gradient.  TensorFlow conv_grad_filter_ops.cc,
 *    Conv2DCustomBackpropFilterOp: per image, the Im2col patch matrix A
 *    ([Ho*Wo, R*S*C]) and the output gradient B ([Ho*Wo, K]); the filter
 *    gradient [R*S*C, K] (HWIO) is the sum over images of A^T B.  Written out
 *    here as the plain sum dW[r,s,c,k] = sum over n, ho, wo of
 *    X(n, ho*sh - pt + r, wo*sw - pl + s, c) * dY[n,ho,wo,k], in double.
 *
 *  - The float epilogue.  MIOpen "Using the fusion API": operators apply in
 *    the order they are added, and the supported-fusion tables list
 *    conv -> bias -> batch-norm inference -> activation (CBNA).  Batch-norm
 *    inference is the standard gamma * (t - mean) / sqrt(var + eps) + beta,
 *    evaluated here unfolded, in double.  The activation is ReLU or one of the
 *    other modes the same page's fusion tables list for these combinations:
 *    Leaky Relu, Clipped Relu and CLAMP, with the activation arguments alpha
 *    and beta (miopenSetOpArgsActivForward).  The page names them without
 *    formulas; read plainly: leaky t > 0 ? t : alpha * t; clipped
 *    min(max(t, 0), alpha); clamp min(max(t, alpha), beta).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARG -1
#define ORACLE_OVERFLOW -2
#define ORACLE_NO_MEMORY -3

/* ---------------------------------------------------------------- geometry */

/*
 * out[0..5] = Ho, Wo, pad_top, pad_bottom, pad_left, pad_right.
 * same != 0 selects SAME padding, otherwise VALID.  Returns ORACLE_BAD_ARG for
 * non-positive sizes or strides, or VALID with a filter larger than the input.
 */
int oracle_geometry(int H, int W, int R, int S, int sh, int sw, int same,
                    int out[6]) {
  if (H < 1 || W < 1 || R < 1 || S < 1 || sh < 1 || sw < 1) return ORACLE_BAD_ARG;
  int Ho, Wo, pt, pb, pl, pr;
  if (same) {
    Ho = (H + sh - 1) / sh;
    Wo = (W + sw - 1) / sw;
    int prow = (Ho - 1) * sh + R - H;
    int pcol = (Wo - 1) * sw + S - W;
    if (prow < 0) prow = 0;
    if (pcol < 0) pcol = 0;
    pt = prow / 2;
    pb = prow - pt;
    pl = pcol / 2;
    pr = pcol - pl;
  } else {
    if (H < R || W < S) return ORACLE_BAD_ARG;
    pt = pb = pl = pr = 0;
    Ho = (H - R) / sh + 1;
    Wo = (W - S) / sw + 1;
  }
  out[0] = Ho;
  out[1] = Wo;
  out[2] = pt;
  out[3] = pb;
  out[4] = pl;
  out[5] = pr;
  return ORACLE_OK;
}

/*
 * Shape block shared by every conv entry below, as a flat int array:
 *   d[0..8]  = N, H, W, C, K, R, S, stride_h, stride_w
 *   d[9..12] = pad_top, pad_bottom, pad_left, pad_right
 * The output size follows from the Im2col expression
 *   Ho = (H + pt + pb - R)/sh + 1,  Wo = (W + pl + pr - S)/sw + 1.
 */
typedef struct {
  long N, H, W, C, K, R, S, sh, sw, pt, pb, pl, pr, Ho, Wo;
} shape_t;

static int unpack_shape(const int* d, shape_t* s) {
  s->N = d[0]; s->H = d[1]; s->W = d[2]; s->C = d[3]; s->K = d[4];
  s->R = d[5]; s->S = d[6]; s->sh = d[7]; s->sw = d[8];
  s->pt = d[9]; s->pb = d[10]; s->pl = d[11]; s->pr = d[12];
  if (s->N < 0 || s->H < 1 || s->W < 1 || s->C < 1 || s->K < 1 || s->R < 1 ||
      s->S < 1 || s->sh < 1 || s->sw < 1 || s->pt < 0 || s->pb < 0 ||
      s->pl < 0 || s->pr < 0)
    return ORACLE_BAD_ARG;
  long hspan = s->H + s->pt + s->pb - s->R;
  long wspan = s->W + s->pl + s->pr - s->S;
  if (hspan < 0 || wspan < 0) return ORACLE_BAD_ARG;
  s->Ho = hspan / s->sh + 1;
  s->Wo = wspan / s->sw + 1;
  return ORACLE_OK;
}

int oracle_output_hw(const int* d, int hw[2]) {
  shape_t s;
  if (unpack_shape(d, &s) != ORACLE_OK) return ORACLE_BAD_ARG;
  hw[0] = (int)s.Ho;
  hw[1] = (int)s.Wo;
  return ORACLE_OK;
}

/* ------------------------------------------------- direct convolution, int8 */

/* acc is N x Ho x Wo x K int32.  Returns ORACLE_OVERFLOW if a sum leaves int32. */
int oracle_conv_i8_direct(const int8_t* x, const int8_t* w, const int* d,
                          int32_t* acc) {
  shape_t s;
  if (unpack_shape(d, &s) != ORACLE_OK) return ORACLE_BAD_ARG;
  int overflow = 0;
#pragma omp parallel for collapse(2) schedule(static) reduction(| : overflow)
  for (long n = 0; n < s.N; ++n) {
    for (long ho = 0; ho < s.Ho; ++ho) {
      for (long wo = 0; wo < s.Wo; ++wo) {
        for (long k = 0; k < s.K; ++k) {
          int64_t sum = 0;
          for (long r = 0; r < s.R; ++r) {
            long hi = ho * s.sh - s.pt + r;
            if (hi < 0 || hi >= s.H) continue; /* zero padding */
            for (long q = 0; q < s.S; ++q) {
              long wi = wo * s.sw - s.pl + q;
              if (wi < 0 || wi >= s.W) continue;
              for (long c = 0; c < s.C; ++c) {
                int64_t xv = x[((n * s.H + hi) * s.W + wi) * s.C + c];
                int64_t wv = w[((r * s.S + q) * s.C + c) * s.K + k];
                sum += xv * wv;
              }
            }
          }
          if (sum > INT32_MAX || sum < INT32_MIN) overflow = 1;
          acc[((n * s.Ho + ho) * s.Wo + wo) * s.K + k] = (int32_t)sum;
        }
      }
    }
  }
  return overflow ? ORACLE_OVERFLOW : ORACLE_OK;
}

/* ------------------------------------------ im2col + plain GEMM, int8 form */

/*
 * Patch matrix of one NHWC image: row (ho, wo), column (r, s, c); a tap that
 * falls outside the image contributes C zeros.
 */
static void patches_of_image(const int8_t* img, const shape_t* s, int8_t* cols) {
  long row_len = s->R * s->S * s->C;
  for (long ho = 0; ho < s->Ho; ++ho) {
    for (long wo = 0; wo < s->Wo; ++wo) {
      int8_t* dst = cols + (ho * s->Wo + wo) * row_len;
      for (long r = 0; r < s->R; ++r) {
        long hi = ho * s->sh - s->pt + r;
        for (long q = 0; q < s->S; ++q) {
          long wi = wo * s->sw - s->pl + q;
          int8_t* tap = dst + (r * s->S + q) * s->C;
          if (hi >= 0 && hi < s->H && wi >= 0 && wi < s->W)
            memcpy(tap, img + (hi * s->W + wi) * s->C, (size_t)s->C);
          else
            memset(tap, 0, (size_t)s->C);
        }
      }
    }
  }
}

int oracle_conv_i8_im2col(const int8_t* x, const int8_t* w, const int* d,
                          int32_t* acc) {
  shape_t s;
  if (unpack_shape(d, &s) != ORACLE_OK) return ORACLE_BAD_ARG;
  long rows = s.Ho * s.Wo;
  long depth = s.R * s.S * s.C; /* the filter seen as a [depth, K] matrix */
  int overflow = 0, nomem = 0;
#pragma omp parallel reduction(| : overflow, nomem)
  {
    /* One patch matrix per thread at a time, so memory stays bounded. */
    int8_t* cols = (int8_t*)malloc((size_t)(rows * depth > 0 ? rows * depth : 1));
    if (!cols) nomem = 1;
#pragma omp for schedule(static)
    for (long n = 0; n < s.N; ++n) {
      if (!cols) continue;
      patches_of_image(x + n * s.H * s.W * s.C, &s, cols);
      int32_t* out = acc + n * rows * s.K;
      for (long i = 0; i < rows; ++i) {
        for (long k = 0; k < s.K; ++k) {
          int64_t sum = 0;
          for (long j = 0; j < depth; ++j)
            sum += (int64_t)cols[i * depth + j] * (int64_t)w[j * s.K + k];
          if (sum > INT32_MAX || sum < INT32_MIN) overflow = 1;
          out[i * s.K + k] = (int32_t)sum;
        }
      }
    }
    free(cols);
  }
  if (nomem) return ORACLE_NO_MEMORY;
  return overflow ? ORACLE_OVERFLOW : ORACLE_OK;
}

/* --------------------------------------------- direct convolution, floats */

/* bf16 is the top half of an IEEE binary32; widening is exact. */
static float widen_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* Products of two floats are exact in double; the sum is taken in double. */
int oracle_conv_f32_direct(const float* x, const float* w, const int* d,
                           double* acc) {
  shape_t s;
  if (unpack_shape(d, &s) != ORACLE_OK) return ORACLE_BAD_ARG;
#pragma omp parallel for collapse(2) schedule(static)
  for (long n = 0; n < s.N; ++n) {
    for (long ho = 0; ho < s.Ho; ++ho) {
      for (long wo = 0; wo < s.Wo; ++wo) {
        for (long k = 0; k < s.K; ++k) {
          double sum = 0.0;
          for (long r = 0; r < s.R; ++r) {
            long hi = ho * s.sh - s.pt + r;
            if (hi < 0 || hi >= s.H) continue;
            for (long q = 0; q < s.S; ++q) {
              long wi = wo * s.sw - s.pl + q;
              if (wi < 0 || wi >= s.W) continue;
              for (long c = 0; c < s.C; ++c) {
                double xv = x[((n * s.H + hi) * s.W + wi) * s.C + c];
                double wv = w[((r * s.S + q) * s.C + c) * s.K + k];
                sum += xv * wv;
              }
            }
          }
          acc[((n * s.Ho + ho) * s.Wo + wo) * s.K + k] = sum;
        }
      }
    }
  }
  return ORACLE_OK;
}

int oracle_conv_bf16_direct(const uint16_t* x, const uint16_t* w, const int* d,
                            double* acc) {
  shape_t s;
  if (unpack_shape(d, &s) != ORACLE_OK) return ORACLE_BAD_ARG;
#pragma omp parallel for collapse(2) schedule(static)
  for (long n = 0; n < s.N; ++n) {
    for (long ho = 0; ho < s.Ho; ++ho) {
      for (long wo = 0; wo < s.Wo; ++wo) {
        for (long k = 0; k < s.K; ++k) {
          double sum = 0.0;
          for (long r = 0; r < s.R; ++r) {
            long hi = ho * s.sh - s.pt + r;
            if (hi < 0 || hi >= s.H) continue;
            for (long q = 0; q < s.S; ++q) {
              long wi = wo * s.sw - s.pl + q;
              if (wi < 0 || wi >= s.W) continue;
              for (long c = 0; c < s.C; ++c) {
                double xv = widen_bf16(x[((n * s.H + hi) * s.W + wi) * s.C + c]);
                double wv = widen_bf16(w[((r * s.S + q) * s.C + c) * s.K + k]);
                sum += xv * wv;
              }
            }
          }
          acc[((n * s.Ho + ho) * s.Wo + wo) * s.K + k] = sum;
        }
      }
    }
  }
  return ORACLE_OK;
}

/* ------------------------------------------------------------- epilogues */

/*
 * int8 epilogue over an M x K accumulator (M = N*Ho*Wo), cuDNN 8 order as the
 * TensorFlow output kernel spells it.  side may be NULL (no side input).
 * Every step is a separate fp32 operation; only step (2) is fused.
 */
/*
 * int8 epilogue.  scales == NULL: every channel uses conv_input_scale;
 * otherwise channel k uses scales[k].  order 8: cuDNN 8 order; order 7:
 * cuDNN 7 order (see the header).
 */
void oracle_epilogue_i8_ex(const int32_t* acc, long M, int K, float conv_input_scale,
                           const float* scales, const int8_t* side,
                           float side_input_scale, const float* bias, int relu,
                           int order, int8_t* y) {
  const float hi = 127.0f;
  const float lo = relu ? 0.0f : -128.0f;
  const int use_side = side != NULL && side_input_scale != 0.0f;
#pragma omp parallel for schedule(static)
  for (long m = 0; m < M; ++m) {
    for (int k = 0; k < K; ++k) {
      long i = m * K + k;
      const float cis = scales ? scales[k] : conv_input_scale;
      float t = (float)acc[i];          /* int32 -> fp32, round to nearest even */
      if (order == 7) {
        t = fmaf(t, cis, bias[k]);       /* scale and bias, single rounding */
        if (use_side) t = fmaf((float)side[i], side_input_scale, t);
      } else {
        t = t * cis;                     /* (1) scale */
        if (use_side)                    /* (2) side input, single rounding */
          t = fmaf((float)side[i], side_input_scale, t);
        t = t + bias[k];                 /* (3) bias */
      }
      t = nearbyintf(t);                 /* round half to even (default mode) */
      if (t < lo) t = lo;                /* clip; ReLU raises the lower bound */
      if (t > hi) t = hi;
      y[i] = (int8_t)t;
    }
  }
}

void oracle_epilogue_i8(const int32_t* acc, long M, int K, float conv_input_scale,
                        const int8_t* side, float side_input_scale,
                        const float* bias, int relu, int8_t* y) {
  oracle_epilogue_i8_ex(acc, M, K, conv_input_scale, NULL, side, side_input_scale, bias,
                        relu, 8, y);
}

/*
 * Weight gradient, in double: x [N][H][W][C], dy [N][Ho][Wo][K] (both as
 * double), dw [R][S][C][K].  d as for the convolutions.
 */
int oracle_wgrad_direct(const double* x, const double* dy, const int* d, double* dw) {
  shape_t s;
  if (unpack_shape(d, &s) != ORACLE_OK) return ORACLE_BAD_ARG;
#pragma omp parallel for collapse(2) schedule(static)
  for (long r = 0; r < s.R; ++r) {
    for (long q = 0; q < s.S; ++q) {
      for (long c = 0; c < s.C; ++c) {
        double* out = dw + ((r * s.S + q) * s.C + c) * s.K;
        for (long k = 0; k < s.K; ++k) out[k] = 0.0;
        for (long n = 0; n < s.N; ++n) {
          for (long ho = 0; ho < s.Ho; ++ho) {
            long hi = ho * s.sh - s.pt + r;
            if (hi < 0 || hi >= s.H) continue;
            for (long wo = 0; wo < s.Wo; ++wo) {
              long wi = wo * s.sw - s.pl + q;
              if (wi < 0 || wi >= s.W) continue;
              const double xv = x[((n * s.H + hi) * s.W + wi) * s.C + c];
              const double* g = dy + ((n * s.Ho + ho) * s.Wo + wo) * s.K;
              for (long k = 0; k < s.K; ++k) out[k] += xv * g[k];
            }
          }
        }
      }
    }
  }
  return ORACLE_OK;
}

/*
 * Float epilogue: bias, then batch-norm inference, then ReLU, each optional,
 * in that order, in double.  bias == NULL skips the bias; gamma == NULL skips
 * the batch norm (then beta/mean/var are ignored).
 */
/* Activation modes of the float epilogue. */
#define ORACLE_ACT_NONE 0
#define ORACLE_ACT_RELU 1
#define ORACLE_ACT_LEAKY 2
#define ORACLE_ACT_CLIPPED 3
#define ORACLE_ACT_CLAMP 4

void oracle_epilogue_float_ex(const double* acc, long M, int K, const float* bias,
                              const float* gamma, const float* beta,
                              const float* mean, const float* var, float eps,
                              int act, float alpha, float act_beta, double* y) {
#pragma omp parallel for schedule(static)
  for (long m = 0; m < M; ++m) {
    for (int k = 0; k < K; ++k) {
      long i = m * K + k;
      double t = acc[i];
      if (bias) t = t + (double)bias[k];
      if (gamma)
        t = (double)gamma[k] * (t - (double)mean[k]) /
                sqrt((double)var[k] + (double)eps) +
            (double)beta[k];
      switch (act) {
        case ORACLE_ACT_RELU:
          if (t < 0.0) t = 0.0;
          break;
        case ORACLE_ACT_LEAKY:
          if (!(t > 0.0)) t = (double)alpha * t;
          break;
        case ORACLE_ACT_CLIPPED:
          if (t < 0.0) t = 0.0;
          if (t > (double)alpha) t = (double)alpha;
          break;
        case ORACLE_ACT_CLAMP:
          if (t < (double)alpha) t = (double)alpha;
          if (t > (double)act_beta) t = (double)act_beta;
          break;
        default:
          break;
      }
      y[i] = t;
    }
  }
}

void oracle_epilogue_float(const double* acc, long M, int K, const float* bias,
                           const float* gamma, const float* beta,
                           const float* mean, const float* var, float eps,
                           int relu, double* y) {
  oracle_epilogue_float_ex(acc, M, K, bias, gamma, beta, mean, var, eps,
                           relu ? ORACLE_ACT_RELU : ORACLE_ACT_NONE, 0.0f, 0.0f, y);
}

/* Thread count of the OpenMP loops above (the baseline timing runs them on
 * one thread and on all host cores). */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  extern void omp_set_num_threads(int);
  omp_set_num_threads(n > 0 ? n : 1);
#else
  (void)n;
#endif
}

int oracle_num_threads(void) {
  int n = 1;
#pragma omp parallel
  {
#pragma omp single
    {
#ifdef _OPENMP
      extern int omp_get_num_threads(void);
      n = omp_get_num_threads();
#endif
    }
  }
  return n;
}
