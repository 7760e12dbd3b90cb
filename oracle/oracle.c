/*
 * Deformable-sampling CPU oracle — TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, fp64 loop nests that define what the GPU library must compute.
 * Only tests/, the smoke check and the bench's cpu_baseline leg may load this.
 * It shares no source, header, table or helper with the HIP library.
 *
 * Sources (page title, section):
 *  [P-DCNv1]  "用PyTorch实战DCNv1：从零构建可变形卷积与ROI池化模块"
 *             (Hands-on DCNv1 in PyTorch), section 1 (the deformable sum
 *             y(p0) = sum_n w(p_n) x(p0 + p_n + dp_n)) and section 2 (the
 *             bilinear kernel G(q,p) = g(qx,px) g(qy,py), g(a,b) = max(0,1-|a-b|);
 *             offsets laid out as interleaved (x, y) pairs per point).
 *  [P-DCNv2]  "DCNv2实战：在YOLOv5中替换普通卷积…" (DCNv2 in YOLOv5), section 1:
 *             each sampled value is additionally scaled by a modulation scalar.
 *  [P-DCNv3]  "DCNV3技术深度解析与高性能AI开发环境构建" (DCNv3 deep dive), the
 *             forward-kernel section: kernel points indexed row-major
 *             (k = ki*kernel_w + kj).
 *  [P-DCNv4]  lpnh.cn news 2795861 (DCNv4 in YOLOv11), section 1.1: channels
 *             split into groups with their own offsets and modulation; DCNv3
 *             normalises the modulation with a softmax over the points, DCNv4
 *             does not; section 3.2: channels-last input, offset_scale.
 *  [P-AGG]    mlqm.cn news 106099 (Sparse4D deformable_aggregation), sections
 *             2.1-2.2 (inputs: multi-camera multi-scale features flattened to
 *             [B, N*H*W, C], spatial shapes, scale start index, sampling
 *             locations, weights) and section 7 (softmax-normalised weights).
 *
 * Readings where the pages are silent:
 *  - zero outside the image, per corner;
 *  - grid base = out*stride - pad + tap*dilation;
 *  - offset pairs are (dx, dy), x first;
 *  - the scaled core offset is one fp32 quantity: fl32(offset_scale*delta);
 *  - aggregation pixel coordinate: x = fl32(u*W) - 0.5 (pixel centres at
 *    (i+1/2)/W), y likewise with v and H.
 *
 * Every function also returns, per output element, the sum of the absolute
 * values of all product terms ("absum"), used by the tests' error bound.
 *
 * oracle_dcn_core_backward (and oracle_dcn_v2_backward) is the derivative of
 * the forward sum,
 * written out by hand (the pages print no backward pass); its pins are
 * finite differences, adjoint identities and torch autograd of an
 * independent fp64 formulation.
 */
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

/* ---------------------------------------------------------------------- */
/* Bilinear sample, [P-DCNv1] section 2.                                   */
/* X(h, w) is X[(h*W + w) * cstride]; positions outside [0,H)x[0,W) give 0. */
/* The 4-corner form below equals the lattice sum over all q of G(q,p)X(q): */
/* g(q,p) is non-zero only for the two integers q bracketing p, with        */
/* weights 1-f and f.                                                       */
/* ---------------------------------------------------------------------- */
double oracle_bilinear(const double *X, int64_t H, int64_t W, int64_t cstride,
                       double y, double x, double *absum)
{
    double y0 = floor(y), x0 = floor(x);
    double fy = y - y0, fx = x - x0;
    double wy[2] = {1.0 - fy, fy};
    double wx[2] = {1.0 - fx, fx};
    double s = 0.0, a = 0.0;
    for (int dy = 0; dy < 2; ++dy) {
        for (int dx = 0; dx < 2; ++dx) {
            double qy = y0 + dy, qx = x0 + dx;
            double wq = wy[dy] * wx[dx];
            if (wq == 0.0) continue;
            if (qy < 0.0 || qy >= (double)H || qx < 0.0 || qx >= (double)W) continue;
            double v = X[((int64_t)qy * W + (int64_t)qx) * cstride];
            s += wq * v;
            a += fabs(wq * v);
        }
    }
    if (absum) *absum += a;
    return s;
}

/* fl32(s * d): the exact product of two fp32 values fits in a double, so one
 * conversion performs the single round-to-nearest-even. */
static double fl32_mul(float s, double d)
{
    return (double)(float)((double)s * d);
}

/* Softmax of n values in fp64, max-subtracted ([P-DCNv4] section 1.1 for
 * DCNv3's per-group normalisation; [P-AGG] section 7 for aggregation). */
static void softmax_d(const double *l, int64_t n, int64_t lstride, double *m)
{
    double mx = -INFINITY;
    for (int64_t i = 0; i < n; ++i)
        if (l[i * lstride] > mx) mx = l[i * lstride];
    double den = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        m[i] = exp(l[i * lstride] - mx);
        den += m[i];
    }
    for (int64_t i = 0; i < n; ++i) m[i] /= den;
}

void oracle_softmax(const double *l, int64_t n, double *m) { softmax_d(l, n, 1, m); }

/* Threads the parallel loops below run on (reported with timings). */
int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Set the thread count of the parallel loops (n >= 1; for single-thread timings). */
void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

static int64_t out_size(int64_t in, int64_t k, int64_t s, int64_t p, int64_t d)
{
    return (in + 2 * p - d * (k - 1) - 1) / s + 1;
}

/* ---------------------------------------------------------------------- */
/* DCNv3/v4 core, channels-last.                                            */
/*  x      [N, H, W, G*C]                                                   */
/*  offset [N, Ho, Wo, G, K, 2]  (dx, dy), K = kh*kw, k = i*kw + j         */
/*  mask   [N, Ho, Wo, G, K] or NULL (then every modulation is 1)           */
/*  out    [npix, G*C]  for the listed output pixels (pix = (n*Ho+ho)*Wo+wo)*/
/*         or [N*Ho*Wo, G*C] when pix == NULL.                              */
/* out[.., g*C+c] = sum_k m_k * bilinear(x[n,:,:,g*C+c], y_k, x_k) with     */
/* y_k = ho*sh - ph + i*dh + dy_k and x_k = wo*sw - pw + j*dw + dx_k         */
/* ([P-DCNv1] s1, [P-DCNv2] s1, [P-DCNv4] s1.1). With softmax != 0, m_k is  */
/* the softmax over k of the mask values of (n, ho, wo, g).                 */
/* ---------------------------------------------------------------------- */
int oracle_dcn_core(const double *x, const double *offset, const double *mask,
                    double *out, double *absum,
                    int64_t N, int64_t H, int64_t W, int64_t G, int64_t C,
                    int64_t kh, int64_t kw, int64_t sh, int64_t sw,
                    int64_t ph, int64_t pw, int64_t dh, int64_t dw,
                    float offset_scale, int softmax,
                    const int64_t *pix, int64_t npix)
{
    int64_t Ho = out_size(H, kh, sh, ph, dh), Wo = out_size(W, kw, sw, pw, dw);
    int64_t K = kh * kw, GC = G * C;
    if (Ho <= 0 || Wo <= 0) return 1;
    if (!pix) npix = N * Ho * Wo;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t t = 0; t < npix; ++t) {
        int64_t p = pix ? pix[t] : t;
        if (p < 0 || p >= N * Ho * Wo) { bad = 1; continue; }
        int64_t n = p / (Ho * Wo), ho = (p / Wo) % Ho, wo = p % Wo;
        double *m = (double *)malloc(sizeof(double) * (size_t)K);
        for (int64_t g = 0; g < G; ++g) {
            const double *om = offset + (p * G + g) * K * 2;
            const double *mm = mask ? mask + (p * G + g) * K : NULL;
            for (int64_t k = 0; k < K; ++k) m[k] = mm ? mm[k] : 1.0;
            if (softmax) softmax_d(mm ? mm : m, K, 1, m);
            for (int64_t c = 0; c < C; ++c) {
                const double *X = x + n * H * W * GC + g * C + c;
                double s = 0.0, a = 0.0;
                for (int64_t i = 0; i < kh; ++i) {
                    for (int64_t j = 0; j < kw; ++j) {
                        int64_t k = i * kw + j;
                        double yy = (double)(ho * sh - ph + i * dh) + fl32_mul(offset_scale, om[2 * k + 1]);
                        double xx = (double)(wo * sw - pw + j * dw) + fl32_mul(offset_scale, om[2 * k + 0]);
                        double ab = 0.0;
                        double b = oracle_bilinear(X, H, W, GC, yy, xx, &ab);
                        s += m[k] * b;
                        a += fabs(m[k]) * ab;
                    }
                }
                out[t * GC + g * C + c] = s;
                if (absum) absum[t * GC + g * C + c] = a;
            }
        }
        free(m);
    }
    return bad ? 2 : 0;
}

/* ---------------------------------------------------------------------- */
/* Gradients of the DCNv3/v4 core above (the derivative of its sum; no      */
/* page prints it). With G = grad_out[n,ho,wo,g*C+c] and, for tap k at      */
/* (y, x) = (y0 + fy, x0 + fx), corner values X_ab = x[n, y0+a, x0+b, .]    */
/* (0 outside the image) and bilinear weights                               */
/*   w_00 = (1-fy)(1-fx), w_01 = (1-fy)fx, w_10 = fy(1-fx), w_11 = fy fx:   */
/*   B    = sum_ab w_ab X_ab                                                 */
/*   dB/dy = (1-fx)(X_10 - X_00) + fx(X_11 - X_01)                           */
/*   dB/dx = (1-fy)(X_01 - X_00) + fy(X_11 - X_10)                           */
/* (derivatives taken from the right at integer positions, where floor()     */
/* moves), so that                                                          */
/*   grad_x[corner ab] += m_k w_ab G        (every corner inside the image)  */
/*   grad_m_k           = sum_c G B                                          */
/*   grad_offset[k]     = (s m_k sum_c G dB/dx, s m_k sum_c G dB/dy), s =    */
/*                        offset_scale (d fl32(s d)/dd taken as s)           */
/*   and with softmax, grad_logit_k = m_k (grad_m_k - sum_j m_j grad_m_j).   */
/* Outputs may be NULL. gx is overwritten (not accumulated into). The *_abs  */
/* arrays (NULL allowed) receive the matching sums of |product terms|.       */
/* ---------------------------------------------------------------------- */
int oracle_dcn_core_backward(const double *x, const double *offset, const double *mask,
                             const double *gout, double *gx, double *goff, double *gmask,
                             double *gx_abs, double *goff_abs, double *gmask_abs,
                             int64_t N, int64_t H, int64_t W, int64_t G, int64_t C,
                             int64_t kh, int64_t kw, int64_t sh, int64_t sw,
                             int64_t ph, int64_t pw, int64_t dh, int64_t dw,
                             float offset_scale, int softmax)
{
    int64_t Ho = out_size(H, kh, sh, ph, dh), Wo = out_size(W, kw, sw, pw, dw);
    int64_t K = kh * kw, GC = G * C;
    if (Ho <= 0 || Wo <= 0) return 1;
    double s = (double)offset_scale;
    if (gx) for (int64_t i = 0; i < N * H * W * GC; ++i) gx[i] = 0.0;
    if (gx_abs) for (int64_t i = 0; i < N * H * W * GC; ++i) gx_abs[i] = 0.0;
    /* one image per iteration: the scatter into gx never crosses images */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t n = 0; n < N; ++n) {
        double *m = (double *)malloc(sizeof(double) * (size_t)K * 4);
        double *gm = m + K, *gma = m + 2 * K, *unused = m + 3 * K;
        (void)unused;
        for (int64_t ho = 0; ho < Ho; ++ho)
        for (int64_t wo = 0; wo < Wo; ++wo)
        for (int64_t g = 0; g < G; ++g) {
            int64_t pg = ((n * Ho + ho) * Wo + wo) * G + g;  /* (pixel, group) pair */
            const double *om = offset + pg * K * 2;
            const double *mm = mask ? mask + pg * K : NULL;
            const double *Gv = gout + ((n * Ho + ho) * Wo + wo) * GC + g * C;
            for (int64_t k = 0; k < K; ++k) m[k] = mm ? mm[k] : 1.0;
            if (softmax) softmax_d(mm ? mm : m, K, 1, m);
            for (int64_t i = 0; i < kh; ++i)
            for (int64_t j = 0; j < kw; ++j) {
                int64_t k = i * kw + j;
                double yy = (double)(ho * sh - ph + i * dh) + fl32_mul(offset_scale, om[2 * k + 1]);
                double xx = (double)(wo * sw - pw + j * dw) + fl32_mul(offset_scale, om[2 * k + 0]);
                double y0 = floor(yy), x0 = floor(xx);
                double fy = yy - y0, fx = xx - x0;
                double w[2][2] = {{(1.0 - fy) * (1.0 - fx), (1.0 - fy) * fx},
                                  {fy * (1.0 - fx), fy * fx}};
                double dwy[2][2] = {{-(1.0 - fx), -fx}, {1.0 - fx, fx}};  /* d w_ab / d fy */
                double dwx[2][2] = {{-(1.0 - fy), 1.0 - fy}, {-fy, fy}};  /* d w_ab / d fx */
                int inside[2][2];
                int64_t idx[2][2];
                for (int a = 0; a < 2; ++a)
                    for (int b = 0; b < 2; ++b) {
                        double qy = y0 + a, qx = x0 + b;
                        inside[a][b] = !(qy < 0.0 || qy >= (double)H || qx < 0.0 || qx >= (double)W);
                        idx[a][b] = inside[a][b]
                                        ? ((n * H + (int64_t)qy) * W + (int64_t)qx) * GC + g * C
                                        : 0;
                    }
                double sb = 0.0, sba = 0.0, sy = 0.0, sya = 0.0, sx = 0.0, sxa = 0.0;
                for (int64_t c = 0; c < C; ++c) {
                    double gc = Gv[c];
                    for (int a = 0; a < 2; ++a)
                        for (int b = 0; b < 2; ++b) {
                            if (!inside[a][b]) continue;
                            double X = x[idx[a][b] + c];
                            sb += gc * w[a][b] * X;
                            sba += fabs(gc * w[a][b] * X);
                            sy += gc * dwy[a][b] * X;
                            sya += fabs(gc * dwy[a][b] * X);
                            sx += gc * dwx[a][b] * X;
                            sxa += fabs(gc * dwx[a][b] * X);
                            if (gx && w[a][b] != 0.0) gx[idx[a][b] + c] += m[k] * w[a][b] * gc;
                            if (gx_abs) gx_abs[idx[a][b] + c] += fabs(m[k] * w[a][b] * gc);
                        }
                }
                gm[k] = sb;
                gma[k] = sba;
                if (goff) {
                    goff[pg * K * 2 + 2 * k + 0] = s * m[k] * sx;
                    goff[pg * K * 2 + 2 * k + 1] = s * m[k] * sy;
                }
                if (goff_abs) {
                    goff_abs[pg * K * 2 + 2 * k + 0] = fabs(s * m[k]) * sxa;
                    goff_abs[pg * K * 2 + 2 * k + 1] = fabs(s * m[k]) * sya;
                }
            }
            if (gmask || gmask_abs) {
                double dot = 0.0, dota = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    dot += m[k] * gm[k];
                    dota += fabs(m[k]) * gma[k];
                }
                for (int64_t k = 0; k < K; ++k) {
                    double v = softmax ? m[k] * (gm[k] - dot) : gm[k];
                    double va = softmax ? fabs(m[k]) * (gma[k] + dota) : gma[k];
                    if (gmask) gmask[pg * K + k] = v;
                    if (gmask_abs) gmask_abs[pg * K + k] = va;
                }
            }
        }
        free(m);
    }
    return 0;
}

/* ---------------------------------------------------------------------- */
/* DCNv2 deform-im2col column for one output pixel, NCHW.                   */
/*  x      [N, Cin, H, W]                                                   */
/*  offset [N, dg*K*2, Ho, Wo]: channel (g*K + k)*2 + 0 is dx, +1 is dy      */
/*  mask   [N, dg*K, Ho, Wo] or NULL                                        */
/*  col    [Cin*K] for pixel p: col[ci*K + k] = m * bilinear(x[n,ci], pos)  */
/* Channel ci belongs to deformable group ci / (Cin/dg). With softmax != 0  */
/* the K modulation values of each deformable group are softmax-normalised. */
/* ---------------------------------------------------------------------- */
static void v2_column(const double *x, const double *offset, const double *mask,
                      double *col, double *colabs, int64_t p,
                      int64_t Cin, int64_t H, int64_t W, int64_t Ho, int64_t Wo,
                      int64_t kh, int64_t kw, int64_t sh, int64_t sw,
                      int64_t ph, int64_t pw, int64_t dh, int64_t dw,
                      int64_t dg, int softmax, double *m)
{
    int64_t K = kh * kw, HWo = Ho * Wo;
    int64_t n = p / HWo, r = p % HWo, ho = r / Wo, wo = r % Wo;
    int64_t cpg = Cin / dg;
    for (int64_t g = 0; g < dg; ++g) {
        for (int64_t k = 0; k < K; ++k)
            m[k] = mask ? mask[(n * dg * K + g * K + k) * HWo + r] : 1.0;
        if (softmax && mask)
            softmax_d(mask + (n * dg * K + g * K) * HWo + r, K, HWo, m);
        else if (softmax)
            for (int64_t k = 0; k < K; ++k) m[k] = 1.0 / (double)K;
        for (int64_t ci = g * cpg; ci < (g + 1) * cpg; ++ci) {
            const double *X = x + (n * Cin + ci) * H * W;
            for (int64_t i = 0; i < kh; ++i) {
                for (int64_t j = 0; j < kw; ++j) {
                    int64_t k = i * kw + j;
                    int64_t oc = (n * dg * K + g * K + k) * 2;
                    double dx = offset[(oc + 0) * HWo + r];
                    double dy = offset[(oc + 1) * HWo + r];
                    double yy = (double)(ho * sh - ph + i * dh) + dy;
                    double xx = (double)(wo * sw - pw + j * dw) + dx;
                    double ab = 0.0;
                    double b = oracle_bilinear(X, H, W, 1, yy, xx, &ab);
                    col[ci * K + k] = m[k] * b;
                    if (colabs) colabs[ci * K + k] = fabs(m[k]) * ab;
                }
            }
        }
    }
}

/* Deform-im2col of the listed pixels: cols [npix, Cin*K] (row t = column of
 * pixel pix[t], element ci*K + k). */
int oracle_dcn_v2_columns(const double *x, const double *offset, const double *mask,
                          double *cols,
                          int64_t N, int64_t Cin, int64_t H, int64_t W,
                          int64_t kh, int64_t kw, int64_t sh, int64_t sw,
                          int64_t ph, int64_t pw, int64_t dh, int64_t dw,
                          int64_t dg, int softmax, const int64_t *pix, int64_t npix)
{
    int64_t Ho = out_size(H, kh, sh, ph, dh), Wo = out_size(W, kw, sw, pw, dw);
    int64_t K = kh * kw;
    if (Ho <= 0 || Wo <= 0 || dg <= 0 || Cin % dg) return 1;
    if (!pix) npix = N * Ho * Wo;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t t = 0; t < npix; ++t) {
        int64_t p = pix ? pix[t] : t;
        if (p < 0 || p >= N * Ho * Wo) { bad = 1; continue; }
        double *m = (double *)malloc(sizeof(double) * (size_t)K);
        v2_column(x, offset, mask, cols + t * Cin * K, NULL, p, Cin, H, W, Ho, Wo,
                  kh, kw, sh, sw, ph, pw, dh, dw, dg, softmax, m);
        free(m);
    }
    return bad ? 2 : 0;
}

/* DCNv2 modulated deformable convolution ([P-DCNv2] s1), NCHW:
 *  weight [Cout, Cin, kh, kw]; out [npix, Cout] for the listed pixels, or
 *  [N*Ho*Wo, Cout] (pixel-major) when pix == NULL.
 *  out[p, co] = sum_{ci,k} weight[co, ci, k] * col_p[ci*K + k]. */
int oracle_dcn_v2(const double *x, const double *offset, const double *mask,
                  const double *weight, double *out, double *absum,
                  int64_t N, int64_t Cin, int64_t H, int64_t W, int64_t Cout,
                  int64_t kh, int64_t kw, int64_t sh, int64_t sw,
                  int64_t ph, int64_t pw, int64_t dh, int64_t dw,
                  int64_t dg, int softmax, const int64_t *pix, int64_t npix)
{
    int64_t Ho = out_size(H, kh, sh, ph, dh), Wo = out_size(W, kw, sw, pw, dw);
    int64_t K = kh * kw, R = Cin * K;
    if (Ho <= 0 || Wo <= 0 || dg <= 0 || Cin % dg) return 1;
    if (!pix) npix = N * Ho * Wo;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t t = 0; t < npix; ++t) {
        int64_t p = pix ? pix[t] : t;
        if (p < 0 || p >= N * Ho * Wo) { bad = 1; continue; }
        double *m = (double *)malloc(sizeof(double) * (size_t)K);
        double *col = (double *)malloc(sizeof(double) * (size_t)R);
        double *cab = (double *)malloc(sizeof(double) * (size_t)R);
        v2_column(x, offset, mask, col, cab, p, Cin, H, W, Ho, Wo,
                  kh, kw, sh, sw, ph, pw, dh, dw, dg, softmax, m);
        for (int64_t co = 0; co < Cout; ++co) {
            const double *wr = weight + co * R;
            double s = 0.0, a = 0.0;
            for (int64_t rr = 0; rr < R; ++rr) {
                s += wr[rr] * col[rr];
                a += fabs(wr[rr]) * cab[rr];
            }
            out[t * Cout + co] = s;
            if (absum) absum[t * Cout + co] = a;
        }
        free(cab);
        free(col);
        free(m);
    }
    return bad ? 2 : 0;
}

/* DCNv2 backward: the derivative of oracle_dcn_v2's sum (no page prints it).
 *  gout  [N, Cout, Ho, Wo]
 *  gx    [N, Cin, H, W]      gradient w.r.t. x
 *  goff  [N, dg*K*2, Ho, Wo] gradient w.r.t. the offsets (dx, dy channels)
 *  gmask [N, dg*K, Ho, Wo]   gradient w.r.t. the mask argument (the logits when
 *                            softmax != 0; with mask == NULL, w.r.t. the implied
 *                            modulation: ones, or zero logits with softmax)
 *  gw    [Cout, Cin, kh, kw] gradient w.r.t. the weight
 * and the matching sums of |product terms| (*_abs; any output may be NULL).
 * Three steps: the column gradient gc[p][ci*K + k] = sum_co weight[co,ci,k] *
 * gout[n,co,p]; the weight gradient sum_p gout[n,co,p] * col_p[ci*K + k]; the
 * sampling derivative of each column entry m_k * bilinear(x[n,ci], pos_k) with
 * upstream value gc (as oracle_dcn_core_backward, one upstream value per tap). */
int oracle_dcn_v2_backward(const double *x, const double *offset, const double *mask,
                           const double *weight, const double *gout,
                           double *gx, double *goff, double *gmask, double *gw,
                           double *gx_abs, double *goff_abs, double *gmask_abs, double *gw_abs,
                           int64_t N, int64_t Cin, int64_t H, int64_t W, int64_t Cout,
                           int64_t kh, int64_t kw, int64_t sh, int64_t sw,
                           int64_t ph, int64_t pw, int64_t dh, int64_t dw,
                           int64_t dg, int softmax)
{
    int64_t Ho = out_size(H, kh, sh, ph, dh), Wo = out_size(W, kw, sw, pw, dw);
    int64_t K = kh * kw, R = Cin * K, HWo = Ho * Wo, P = N * HWo;
    if (Ho <= 0 || Wo <= 0 || dg <= 0 || Cin % dg) return 1;
    int64_t cpg = Cin / dg;
    double *col = (double *)malloc(sizeof(double) * (size_t)(P * R > 0 ? P * R : 1));
    double *cab = (double *)malloc(sizeof(double) * (size_t)(P * R > 0 ? P * R : 1));
    double *gc = (double *)malloc(sizeof(double) * (size_t)(P * R > 0 ? P * R : 1));
    double *gca = (double *)malloc(sizeof(double) * (size_t)(P * R > 0 ? P * R : 1));
    if (!col || !cab || !gc || !gca) {
        free(col); free(cab); free(gc); free(gca);
        return 3;
    }
    /* forward columns and the column gradient, per output pixel */
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t p = 0; p < P; ++p) {
        int64_t n = p / HWo, r = p % HWo;
        double *m = (double *)malloc(sizeof(double) * (size_t)K);
        v2_column(x, offset, mask, col + p * R, cab + p * R, p, Cin, H, W, Ho, Wo,
                  kh, kw, sh, sw, ph, pw, dh, dw, dg, softmax, m);
        free(m);
        for (int64_t rr = 0; rr < R; ++rr) {
            double s = 0.0, a = 0.0;
            for (int64_t co = 0; co < Cout; ++co) {
                double go = gout[(n * Cout + co) * HWo + r];
                s += weight[co * R + rr] * go;
                a += fabs(weight[co * R + rr] * go);
            }
            gc[p * R + rr] = s;
            gca[p * R + rr] = a;
        }
    }
    /* weight gradient: one (co, ci*K + k) entry per iteration */
    if (gw || gw_abs) {
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t co = 0; co < Cout; ++co) {
            for (int64_t rr = 0; rr < R; ++rr) {
                double s = 0.0, a = 0.0;
                for (int64_t p = 0; p < P; ++p) {
                    double go = gout[((p / HWo) * Cout + co) * HWo + p % HWo];
                    s += go * col[p * R + rr];
                    a += fabs(go) * cab[p * R + rr];
                }
                if (gw) gw[co * R + rr] = s;
                if (gw_abs) gw_abs[co * R + rr] = a;
            }
        }
    }
    if (gx) for (int64_t i = 0; i < N * Cin * H * W; ++i) gx[i] = 0.0;
    if (gx_abs) for (int64_t i = 0; i < N * Cin * H * W; ++i) gx_abs[i] = 0.0;
    /* sampling derivative; one image per iteration (the scatter stays in it) */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t n = 0; n < N; ++n) {
        double *m = (double *)malloc(sizeof(double) * (size_t)K * 3);
        double *gm = m + K, *gma = m + 2 * K;
        for (int64_t r = 0; r < HWo; ++r) {
            int64_t p = n * HWo + r, ho = r / Wo, wo = r % Wo;
            for (int64_t g = 0; g < dg; ++g) {
                for (int64_t k = 0; k < K; ++k)
                    m[k] = mask ? mask[(n * dg * K + g * K + k) * HWo + r] : 1.0;
                if (softmax && mask)
                    softmax_d(mask + (n * dg * K + g * K) * HWo + r, K, HWo, m);
                else if (softmax)
                    for (int64_t k = 0; k < K; ++k) m[k] = 1.0 / (double)K;
                for (int64_t i = 0; i < kh; ++i)
                for (int64_t j = 0; j < kw; ++j) {
                    int64_t k = i * kw + j;
                    int64_t oc = (n * dg * K + g * K + k) * 2;
                    double dx = offset[(oc + 0) * HWo + r];
                    double dy = offset[(oc + 1) * HWo + r];
                    double yy = (double)(ho * sh - ph + i * dh) + dy;
                    double xx = (double)(wo * sw - pw + j * dw) + dx;
                    double y0 = floor(yy), x0 = floor(xx);
                    double fy = yy - y0, fx = xx - x0;
                    double w[2][2] = {{(1.0 - fy) * (1.0 - fx), (1.0 - fy) * fx},
                                      {fy * (1.0 - fx), fy * fx}};
                    double dwy[2][2] = {{-(1.0 - fx), -fx}, {1.0 - fx, fx}};  /* d w_ab / d fy */
                    double dwx[2][2] = {{-(1.0 - fy), 1.0 - fy}, {-fy, fy}};  /* d w_ab / d fx */
                    int inside[2][2];
                    int64_t q[2][2];
                    for (int a = 0; a < 2; ++a)
                        for (int b = 0; b < 2; ++b) {
                            double qy = y0 + a, qx = x0 + b;
                            inside[a][b] = !(qy < 0.0 || qy >= (double)H || qx < 0.0 || qx >= (double)W);
                            q[a][b] = inside[a][b] ? (int64_t)qy * W + (int64_t)qx : 0;
                        }
                    double sb = 0.0, sba = 0.0, sy = 0.0, sya = 0.0, sx = 0.0, sxa = 0.0;
                    for (int64_t ci = g * cpg; ci < (g + 1) * cpg; ++ci) {
                        double u = gc[p * R + ci * K + k], ua = gca[p * R + ci * K + k];
                        const double *X = x + (n * Cin + ci) * H * W;
                        for (int a = 0; a < 2; ++a)
                            for (int b = 0; b < 2; ++b) {
                                if (!inside[a][b]) continue;
                                double v = X[q[a][b]];
                                sb += u * w[a][b] * v;
                                sba += ua * fabs(w[a][b] * v);
                                sy += u * dwy[a][b] * v;
                                sya += ua * fabs(dwy[a][b] * v);
                                sx += u * dwx[a][b] * v;
                                sxa += ua * fabs(dwx[a][b] * v);
                                int64_t xi = (n * Cin + ci) * H * W + q[a][b];
                                if (gx && w[a][b] != 0.0) gx[xi] += m[k] * w[a][b] * u;
                                if (gx_abs) gx_abs[xi] += fabs(m[k] * w[a][b]) * ua;
                            }
                    }
                    gm[k] = sb;
                    gma[k] = sba;
                    if (goff) {
                        goff[(oc + 0) * HWo + r] = m[k] * sx;
                        goff[(oc + 1) * HWo + r] = m[k] * sy;
                    }
                    if (goff_abs) {
                        goff_abs[(oc + 0) * HWo + r] = fabs(m[k]) * sxa;
                        goff_abs[(oc + 1) * HWo + r] = fabs(m[k]) * sya;
                    }
                }
                if (gmask || gmask_abs) {
                    double dot = 0.0, dota = 0.0;
                    for (int64_t k = 0; k < K; ++k) {
                        dot += m[k] * gm[k];
                        dota += fabs(m[k]) * gma[k];
                    }
                    for (int64_t k = 0; k < K; ++k) {
                        double v = softmax ? m[k] * (gm[k] - dot) : gm[k];
                        double va = softmax ? fabs(m[k]) * (gma[k] + dota) : gma[k];
                        int64_t mi = (n * dg * K + g * K + k) * HWo + r;
                        if (gmask) gmask[mi] = v;
                        if (gmask_abs) gmask_abs[mi] = va;
                    }
                }
            }
        }
        free(m);
    }
    free(col); free(cab); free(gc); free(gca);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* Multi-camera multi-scale deformable aggregation ([P-AGG] s2.1-2.2, s7).  */
/*  feat   [B, P_total, G*Cg]; map (cam, s) occupies rows                    */
/*         scale_start[cam, s] + h*W_s + w, with (H_s, W_s) = spatial_shape  */
/*  loc    [B, A, pts, cams, 2] (u, v) normalised to the camera image        */
/*  weights[B, A, pts, cams, scales, G] (logits when softmax != 0)           */
/*  out    [nanch, G*Cg] for the listed (b*A + a) anchors, or [B*A, G*Cg].   */
/* Pixel coordinate: x = fl32(u*W_s) - 0.5, y = fl32(v*H_s) - 0.5.           */
/* ---------------------------------------------------------------------- */
int oracle_deform_agg(const double *feat, const int32_t *spatial_shape,
                      const int32_t *scale_start, const double *loc,
                      const double *weights, double *out, double *absum,
                      int64_t B, int64_t P_total, int64_t A, int64_t pts,
                      int64_t cams, int64_t scales, int64_t G, int64_t Cg,
                      int softmax, const int64_t *anch, int64_t nanch)
{
    int64_t GC = G * Cg, T = pts * cams * scales;
    for (int64_t cs = 0; cs < cams * scales; ++cs) {
        int64_t Hs = spatial_shape[2 * cs], Ws = spatial_shape[2 * cs + 1];
        if (Hs <= 0 || Ws <= 0 || scale_start[cs] < 0 || scale_start[cs] + Hs * Ws > P_total)
            return 1;
    }
    if (!anch) nanch = B * A;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t t = 0; t < nanch; ++t) {
        int64_t ba = anch ? anch[t] : t;
        if (ba < 0 || ba >= B * A) { bad = 1; continue; }
        int64_t b = ba / A;
        double *w = (double *)malloc(sizeof(double) * (size_t)T);
        for (int64_t g = 0; g < G; ++g) {
            /* weights of (b, a, g) over (p, cam, s) */
            const double *wl = weights + ba * T * G + g;
            if (softmax) {
                softmax_d(wl, T, G, w);
            } else {
                for (int64_t i = 0; i < T; ++i) w[i] = wl[i * G];
            }
            for (int64_t c = 0; c < Cg; ++c) {
                double s = 0.0, a = 0.0;
                for (int64_t p = 0; p < pts; ++p) {
                    for (int64_t cam = 0; cam < cams; ++cam) {
                        const double *uv = loc + ((ba * pts + p) * cams + cam) * 2;
                        for (int64_t sc = 0; sc < scales; ++sc) {
                            int64_t cs = cam * scales + sc;
                            int64_t Hs = spatial_shape[2 * cs], Ws = spatial_shape[2 * cs + 1];
                            double xx = (double)(float)(uv[0] * (double)Ws) - 0.5;
                            double yy = (double)(float)(uv[1] * (double)Hs) - 0.5;
                            const double *X = feat + (b * P_total + scale_start[cs]) * GC + g * Cg + c;
                            double ab = 0.0;
                            double v = oracle_bilinear(X, Hs, Ws, GC, yy, xx, &ab);
                            double wi = w[(p * cams + cam) * scales + sc];
                            s += wi * v;
                            a += fabs(wi) * ab;
                        }
                    }
                }
                out[t * GC + g * Cg + c] = s;
                if (absum) absum[t * GC + g * Cg + c] = a;
            }
        }
        free(w);
    }
    return bad ? 2 : 0;
}

/* ---------------------------------------------------------------------- */
/* Gradients of the aggregation above (its derivative; [AGG] section 2.1   */
/* names the gradients of the features, the sampling locations and the     */
/* weights). With G the group's grad_out, wt the (softmax-normalised)       */
/* weight of sample t = (p, cam, s) and B_t, dB_t/dy, dB_t/dx the bilinear  */
/* sample and its derivatives in the pixel position (from the right at     */
/* integer positions):                                                      */
/*   grad_feat[corner ab of t] += wt * w_ab * G         (inside the map)    */
/*   grad_w_t = sum_c G_c B_t,c  (softmax: wt (grad_w_t - sum_j wj grad_w_j))*/
/*   grad_u(p,cam) += wt * W_s * sum_c G_c dB_t/dx,c   over scales, groups  */
/*   grad_v(p,cam) += wt * H_s * sum_c G_c dB_t/dy,c                        */
/* (x = fl32(u*W_s) - 0.5, whose derivative in u is taken as W_s). Outputs  */
/* are overwritten; any may be NULL; the *_abs arrays (NULL allowed) get    */
/* the matching sums of |product terms|. One thread per group: the groups   */
/* write disjoint channels of grad_feat and grad_w; grad_loc sums the       */
/* groups' partials in group order.                                         */
/* ---------------------------------------------------------------------- */
int oracle_deform_agg_backward(const double *feat, const int32_t *spatial_shape,
                               const int32_t *scale_start, const double *loc,
                               const double *weights, const double *gout,
                               double *gfeat, double *gloc, double *gw,
                               double *gfeat_abs, double *gloc_abs, double *gw_abs,
                               int64_t B, int64_t P_total, int64_t A, int64_t pts,
                               int64_t cams, int64_t scales, int64_t G, int64_t Cg,
                               int softmax)
{
    int64_t GC = G * Cg, T = pts * cams * scales, NL = B * A * pts * cams * 2;
    for (int64_t cs = 0; cs < cams * scales; ++cs) {
        int64_t Hs = spatial_shape[2 * cs], Ws = spatial_shape[2 * cs + 1];
        if (Hs <= 0 || Ws <= 0 || scale_start[cs] < 0 || scale_start[cs] + Hs * Ws > P_total)
            return 1;
    }
    if (gfeat) for (int64_t i = 0; i < B * P_total * GC; ++i) gfeat[i] = 0.0;
    if (gfeat_abs) for (int64_t i = 0; i < B * P_total * GC; ++i) gfeat_abs[i] = 0.0;
    double *part = (double *)calloc((size_t)(G * NL * 2), sizeof(double)); /* loc partials, abs */
    if (!part) return 3;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t g = 0; g < G; ++g) {
        double *w = (double *)malloc(sizeof(double) * (size_t)T * 3);
        double *gt = w + T, *gta = w + 2 * T;
        double *pl = part + g * NL * 2, *pla = pl + NL;
        for (int64_t ba = 0; ba < B * A; ++ba) {
            int64_t b = ba / A;
            const double *wl = weights + ba * T * G + g;
            if (softmax) softmax_d(wl, T, G, w);
            else for (int64_t i = 0; i < T; ++i) w[i] = wl[i * G];
            const double *Gv = gout + ba * GC + g * Cg;
            for (int64_t p = 0; p < pts; ++p)
            for (int64_t cam = 0; cam < cams; ++cam) {
                const double *uv = loc + ((ba * pts + p) * cams + cam) * 2;
                double *lg = pl + ((ba * pts + p) * cams + cam) * 2;
                double *lga = pla + ((ba * pts + p) * cams + cam) * 2;
                for (int64_t sc = 0; sc < scales; ++sc) {
                    int64_t cs = cam * scales + sc, t = (p * cams + cam) * scales + sc;
                    int64_t Hs = spatial_shape[2 * cs], Ws = spatial_shape[2 * cs + 1];
                    double xx = (double)(float)(uv[0] * (double)Ws) - 0.5;
                    double yy = (double)(float)(uv[1] * (double)Hs) - 0.5;
                    double y0 = floor(yy), x0 = floor(xx), fy = yy - y0, fx = xx - x0;
                    double wb[2][2] = {{(1.0 - fy) * (1.0 - fx), (1.0 - fy) * fx},
                                       {fy * (1.0 - fx), fy * fx}};
                    double dwy[2][2] = {{-(1.0 - fx), -fx}, {1.0 - fx, fx}};
                    double dwx[2][2] = {{-(1.0 - fy), 1.0 - fy}, {-fy, fy}};
                    double sb = 0.0, sba = 0.0, sy = 0.0, sya = 0.0, sx = 0.0, sxa = 0.0;
                    for (int a = 0; a < 2; ++a)
                    for (int bb = 0; bb < 2; ++bb) {
                        double qy = y0 + a, qx = x0 + bb;
                        if (qy < 0.0 || qy >= (double)Hs || qx < 0.0 || qx >= (double)Ws) continue;
                        int64_t row = b * P_total + scale_start[cs] + (int64_t)qy * Ws + (int64_t)qx;
                        const double *X = feat + row * GC + g * Cg;
                        for (int64_t c = 0; c < Cg; ++c) {
                            double gx = Gv[c] * X[c];
                            sb += wb[a][bb] * gx;
                            sba += fabs(wb[a][bb] * gx);
                            sy += dwy[a][bb] * gx;
                            sya += fabs(dwy[a][bb] * gx);
                            sx += dwx[a][bb] * gx;
                            sxa += fabs(dwx[a][bb] * gx);
                            if (gfeat) gfeat[row * GC + g * Cg + c] += w[t] * wb[a][bb] * Gv[c];
                            if (gfeat_abs) gfeat_abs[row * GC + g * Cg + c] += fabs(w[t] * wb[a][bb] * Gv[c]);
                        }
                    }
                    gt[t] = sb;
                    gta[t] = sba;
                    lg[0] += w[t] * (double)Ws * sx;
                    lg[1] += w[t] * (double)Hs * sy;
                    lga[0] += fabs(w[t]) * (double)Ws * sxa;
                    lga[1] += fabs(w[t]) * (double)Hs * sya;
                }
            }
            double dot = 0.0, dota = 0.0;
            for (int64_t t = 0; t < T; ++t) {
                dot += w[t] * gt[t];
                dota += fabs(w[t]) * gta[t];
            }
            for (int64_t t = 0; t < T; ++t) {
                double v = softmax ? w[t] * (gt[t] - dot) : gt[t];
                double va = softmax ? fabs(w[t]) * (gta[t] + dota) : gta[t];
                if (gw) gw[(ba * T + t) * G + g] = v;
                if (gw_abs) gw_abs[(ba * T + t) * G + g] = va;
            }
        }
        free(w);
    }
    for (int64_t i = 0; i < NL; ++i) {
        double v = 0.0, va = 0.0;
        for (int64_t g = 0; g < G; ++g) {
            v += part[g * NL * 2 + i];
            va += part[g * NL * 2 + NL + i];
        }
        if (gloc) gloc[i] = v;
        if (gloc_abs) gloc_abs[i] = va;
    }
    free(part);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* Deformable RoI pooling ([P-DCNv1] section 3: per-bin offsets normalised  */
/* as dp_ij = gamma * dp^_ij o (w, h), bilinear sampling, pooling).         */
/* Readings where the page is silent: rois[r] = (batch, x1, y1, x2, y2) in  */
/* input coordinates, multiplied by spatial_scale; w = (x2 - x1)*scale,     */
/* h = (y2 - y1)*scale; bin (i, j) of a k x k grid averages S x S samples   */
/* at (y1s + (i + (sy + 1/2)/S) h/k + gamma*dy_ij*h,                        */
/*     x1s + (j + (sx + 1/2)/S) w/k + gamma*dx_ij*w)                        */
/* in pixel-index coordinates (pixel q at integer q), each read through the */
/* bilinear kernel with zero outside the image per corner; offsets are      */
/* [R, k, k, 2] (dx, dy) pairs, x first. x is channels-last [N, H, W, C],   */
/* out [R, k, k, C]. offset may be NULL (plain RoIAlign-style average       */
/* pooling).                                                                */
/*                                                                          */
/* The sample position is a fixed sequence of fp32 operations, each rounded */
/* once to nearest even (rois, offsets, spatial_scale and gamma are fp32    */
/* quantities; products are never fused with a following addition):        */
/*   x1s = fl(x1*s)            w  = fl(fl(x2 - x1)*s)     bw = fl(w/k)      */
/*   dx  = fl(fl(gamma*dx^)*w)                                              */
/*   tx  = fl((2(j*S + sx) + 1) / (2S))   (the sample's place in bin units) */
/*   px  = fl(fl(x1s + fl(tx*bw)) + dx)                                     */
/* and likewise for y. Everything after the position (the corner split and  */
/* the weighted sum) is exact fp64. Each fl() is evaluated as one fp64      */
/* operation on fp32 operands followed by a conversion to float: for +, -,  */
/* * and / the double rounding this implies equals a single fp32 rounding,  */
/* since 53 >= 2*24 + 2.                                                    */
/* ---------------------------------------------------------------------- */
static double fl32(double v) { return (double)(float)v; }

int oracle_deform_roi_pool(const double *x, const double *rois, const double *offset,
                           double *out, double *absum, int64_t N, int64_t H, int64_t W,
                           int64_t C, int64_t R, int64_t k, int64_t S, double spatial_scale,
                           double gamma)
{
    if (k <= 0 || S <= 0) return 1;
    const double s = fl32(spatial_scale), gm = fl32(gamma);
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t r = 0; r < R; ++r) {
        const double *ro = rois + r * 5;
        int64_t n = (int64_t)ro[0];
        if (n < 0 || n >= N) { bad = 1; continue; }
        const double rx1 = fl32(ro[1]), ry1 = fl32(ro[2]), rx2 = fl32(ro[3]), ry2 = fl32(ro[4]);
        double x1 = fl32(rx1 * s), y1 = fl32(ry1 * s);
        double w = fl32(fl32(rx2 - rx1) * s), h = fl32(fl32(ry2 - ry1) * s);
        double bw = fl32(w / (double)k), bh = fl32(h / (double)k);
        const double *X = x + n * H * W * C;
        for (int64_t i = 0; i < k; ++i)
        for (int64_t j = 0; j < k; ++j) {
            double dx = 0.0, dy = 0.0;
            if (offset) {
                dx = fl32(fl32(gm * fl32(offset[((r * k + i) * k + j) * 2 + 0])) * w);
                dy = fl32(fl32(gm * fl32(offset[((r * k + i) * k + j) * 2 + 1])) * h);
            }
            double *o = out + ((r * k + i) * k + j) * C;
            double *oa = absum ? absum + ((r * k + i) * k + j) * C : NULL;
            for (int64_t c = 0; c < C; ++c) {
                double sum = 0.0, sa = 0.0;
                for (int64_t sy = 0; sy < S; ++sy)
                for (int64_t sx = 0; sx < S; ++sx) {
                    double ty = fl32((double)(2 * (i * S + sy) + 1) / (double)(2 * S));
                    double tx = fl32((double)(2 * (j * S + sx) + 1) / (double)(2 * S));
                    double yy = fl32(fl32(y1 + fl32(ty * bh)) + dy);
                    double xx = fl32(fl32(x1 + fl32(tx * bw)) + dx);
                    double ab = 0.0;
                    sum += oracle_bilinear(X + c, H, W, C, yy, xx, &ab);
                    sa += ab;
                }
                o[c] = sum / (double)(S * S);
                if (oa) oa[c] = sa / (double)(S * S);
            }
        }
    }
    return bad ? 2 : 0;
}
