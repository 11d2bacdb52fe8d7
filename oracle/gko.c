/*
 * gko.c - plain CPU oracle for the GKDT parameter-free detection head.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load this library. It shares no code,
 * header, table or helper with the GPU library; the two only consume the
 * same seeded inputs.
 *
 * What it follows:
 *   - GKDT-L GGUF model card (huggingface.co/Asher-1/GKD_GGUF), section
 *     "Model": the head has no parameters; it upsamples the dense features
 *     4x bilinearly, L2-normalises each kernel row, applies the kernels as a
 *     1x1 convolution, and fuses the per-prompt heatmaps row by row under a
 *     mask, with prompt rows padded to 80; the output is the peak of each
 *     96x96 heatmap mapped to the crop's -1..1 frame plus a confidence score.
 *     Its "Prompts" bullet gives visual prompts as Gaussian pooling of
 *     support feature fibres at sigma = 14 px.
 *   - GKDT paper summary (agihunt.info, "GKDT: General Keypoint Detection
 *     Transformer"), pipeline paragraph: visual prototypes come from
 *     Gaussian heatmaps on the support image; kernels convolve the query
 *     features to give heatmaps directly.
 *   - Reading notes (paper.gecl.asia, section "Method"): the support
 *     features near the annotated point are aggregated into the visual
 *     prototype; the kernels and the query features meet in a normalised
 *     convolution.
 *
 * Everything is double precision and computed literally in the pages'
 * order: the query features are upsampled FIRST (the model card lists the
 * upsample before the convolution), then every heatmap value is a naive
 * dot product over channels, then the modalities are fused, then a linear
 * scan finds the first maximum. Readings where the pages are silent:
 *   - bilinear upsampling uses half-pixel centres with edge clamping (the
 *     align_corners=False convention); when both taps land on the same
 *     source row their weights are summed onto it;
 *   - only the kernels are normalised, k / max(||k||_2, 1e-12);
 *   - dual-prompt fusion is the mean over the modalities whose mask is set;
 *   - Gaussian pooling evaluates exp(-d^2 / (2 sigma^2)) at the stride-grid
 *     cell centres ((j + 1/2) * stride, (i + 1/2) * stride) over the whole
 *     grid and returns the weighted mean of the fibres;
 *   - the score is the raw heatmap value at the peak; the peak index p
 *     maps to x = (2 (p mod Wo) + 1) / Wo - 1, y = (2 (p div Wo) + 1) / Ho - 1;
 *     ties go to the lowest flat index.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define GKO_UP 4 /* 4x upsample (model card, "Model") */

int gko_version(void) { return 1; }

int gko_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Set the OpenMP thread count of the following calls (timing only). */
void gko_set_threads(int n)
{
    if (n > 0) omp_set_num_threads(n);
}

/* Round a double to the nearest bfloat16 value (8 significant bits,
 * float32 exponent range), ties to even. Finite inputs only; results
 * beyond the bfloat16 range become +-inf. */
double gko_round_bf16(double v)
{
    if (v == 0.0 || isnan(v) || isinf(v)) return v;
    const double min_normal = ldexp(1.0, -126);
    if (fabs(v) < min_normal) {
        /* subnormal bfloat16: fixed quantum 2^-133 */
        const double q = ldexp(1.0, -133);
        return nearbyint(v / q) * q;
    }
    int e;
    double m = frexp(v, &e);             /* v = m * 2^e, 0.5 <= |m| < 1 */
    double r = nearbyint(ldexp(m, 8));   /* 8 significant bits, RNE */
    double out = ldexp(r, e - 8);
    const double max_bf16 = ldexp(255.0, 120); /* (2 - 2^-7) * 2^127 */
    if (fabs(out) > max_bf16) return v > 0 ? INFINITY : -INFINITY;
    return out;
}

static double round_to(double v, int dtype)
{
    if (dtype == 0) return (double)(float)v; /* float32, round to nearest */
    if (dtype == 1) return gko_round_bf16(v);
    return v;                                /* 2: keep double */
}

/* ---------------------------------------------------------------------- */
/* Visual keypoint prototypes: Gaussian-weighted mean of support fibres.   */
/* support [B,C,H,W], kpts [B,R,2] (x,y in input px), valid [B,R].         */
/* protos [B,R,C]; rows with valid == 0 are not written.                   */
/* dtype: 0 round to float32, 1 round to bfloat16, 2 keep double.          */
/* ---------------------------------------------------------------------- */
int gko_vkp_pool(const double *support, const double *kpts,
                 const uint8_t *valid, int B, int C, int H, int W, int R,
                 double stride, double sigma, int dtype, double *protos)
{
    if (B < 0 || C < 1 || H < 1 || W < 1 || R < 0) return 2;
    if (!(stride > 0) || !(sigma > 0)) return 4;
    const long S = (long)H * W;
#pragma omp parallel for schedule(dynamic)
    for (long br = 0; br < (long)B * R; ++br) {
        if (!valid[br]) continue;
        const long b = br / R;
        const double x = kpts[2 * br + 0], y = kpts[2 * br + 1];
        double *w = (double *)malloc(sizeof(double) * S);
        double wsum = 0.0;
        for (int i = 0; i < H; ++i) {
            for (int j = 0; j < W; ++j) {
                const double cx = (j + 0.5) * stride, cy = (i + 0.5) * stride;
                const double d2 = (cx - x) * (cx - x) + (cy - y) * (cy - y);
                w[(long)i * W + j] = exp(-d2 / (2.0 * sigma * sigma));
                wsum += w[(long)i * W + j];
            }
        }
        for (int c = 0; c < C; ++c) {
            const double *f = support + ((long)b * C + c) * S;
            double acc = 0.0;
            for (long s = 0; s < S; ++s) acc += w[s] * f[s];
            protos[br * C + c] = round_to(acc / wsum, dtype);
        }
        free(w);
    }
    return 0;
}

/* ---------------------------------------------------------------------- */
/* 4x bilinear upsample, half-pixel centres, edge clamp; or with corners   */
/* the align_corners=True grid, whose first and last samples sit on the    */
/* first and last source samples: source position out (n - 1)/(4n - 1).   */
/* ---------------------------------------------------------------------- */
typedef struct {
    int n;       /* 1 or 2 taps */
    int idx[2];
    double a[2];
} taps_t;

static taps_t up_taps(int out, int n_in, int corners)
{
    double src;
    if (corners)
        src = n_in > 1 ? (double)out * (n_in - 1) / (GKO_UP * n_in - 1.0) : 0.0;
    else
        src = ((double)out + 0.5) / GKO_UP - 0.5;
    if (src < 0.0) src = 0.0;
    const int i0 = (int)floor(src);
    const int i1 = (i0 + 1 < n_in) ? i0 + 1 : n_in - 1;
    const double lam = src - i0;
    taps_t t;
    if (i1 == i0) { /* both weights land on the same source sample */
        t.n = 1;
        t.idx[0] = i0;
        t.a[0] = (1.0 - lam) + lam;
    } else {
        t.n = 2;
        t.idx[0] = i0;
        t.a[0] = 1.0 - lam;
        t.idx[1] = i1;
        t.a[1] = lam;
    }
    return t;
}

/* One upsampled value G[c, y, x] of the map f = F[c] (H x W). */
static double up_value(const double *f, int H, int W, int y, int x, int corners)
{
    const taps_t ty = up_taps(y, H, corners), tx = up_taps(x, W, corners);
    double g = 0.0;
    for (int a = 0; a < ty.n; ++a)
        for (int b = 0; b < tx.n; ++b)
            g += ty.a[a] * tx.a[b] * f[(long)ty.idx[a] * W + tx.idx[b]];
    return g;
}

/* F [C,H,W] -> G [C,4H,4W] */
int gko_upsample4(const double *F, int C, int H, int W, int corners, double *G)
{
    if (C < 1 || H < 1 || W < 1) return 2;
    const int Ho = GKO_UP * H, Wo = GKO_UP * W;
    for (int c = 0; c < C; ++c)
        for (int y = 0; y < Ho; ++y)
            for (int x = 0; x < Wo; ++x)
                G[((long)c * Ho + y) * Wo + x] =
                    up_value(F + (long)c * H * W, H, W, y, x, corners);
    return 0;
}

/* k_hat = k / max(||k||_2, 1e-12) */
static void l2_normalise(const double *k, int C, double *out)
{
    double ss = 0.0;
    for (int c = 0; c < C; ++c) ss += k[c] * k[c];
    double n = sqrt(ss);
    if (n < 1e-12) n = 1e-12;
    for (int c = 0; c < C; ++c) out[c] = k[c] / n;
}

/* ---------------------------------------------------------------------- */
/* Kernel heatmaps. query [B,C,H,W]; kern_vis/kern_txt [B,R,C] with masks  */
/* [B,R] (a NULL pair means that modality is absent). heat [B,R,4H,4W];    */
/* rows with no mask set are not written.                                  */
/* ---------------------------------------------------------------------- */
int gko_kernel_heatmap(const double *query, const double *kern_vis,
                       const uint8_t *mask_vis, const double *kern_txt,
                       const uint8_t *mask_txt, int B, int C, int H, int W,
                       int R, int corners, double *heat)
{
    if (B < 0 || C < 1 || H < 1 || W < 1 || R < 0) return 2;
    const int Ho = GKO_UP * H, Wo = GKO_UP * W;
    const long P = (long)Ho * Wo;
    /* upsampled features of one crop, channels-last [P][C] */
    double *G = (double *)malloc(sizeof(double) * P * C);
    double *kv = (double *)malloc(sizeof(double) * C);
    double *kt = (double *)malloc(sizeof(double) * C);
    if (!G || !kv || !kt) { free(G); free(kv); free(kt); return 6; }

    for (long b = 0; b < B; ++b) {
        int any = 0;
        for (int r = 0; r < R; ++r)
            any |= (mask_vis && mask_vis[b * R + r]) ||
                   (mask_txt && mask_txt[b * R + r]);
        if (!any) continue;

        /* 1. upsample first */
        const double *Fb = query + b * (long)C * H * W;
#pragma omp parallel for schedule(static)
        for (long p = 0; p < P; ++p) {
            const int y = (int)(p / Wo), x = (int)(p % Wo);
            for (int c = 0; c < C; ++c)
                G[p * C + c] = up_value(Fb + (long)c * H * W, H, W, y, x, corners);
        }

        for (int r = 0; r < R; ++r) {
            const int mv = mask_vis && mask_vis[b * R + r];
            const int mt = mask_txt && mask_txt[b * R + r];
            const int n = mv + mt;
            if (n == 0) continue;
            /* 2. normalise the kernels */
            if (mv) l2_normalise(kern_vis + (b * R + r) * (long)C, C, kv);
            if (mt) l2_normalise(kern_txt + (b * R + r) * (long)C, C, kt);
            double *out = heat + (b * R + r) * P;
            /* 3. naive dot product per output cell, 4. masked mean */
#pragma omp parallel for schedule(static)
            for (long p = 0; p < P; ++p) {
                const double *g = G + p * C;
                double sum = 0.0;
                if (mv) {
                    double m = 0.0;
                    for (int c = 0; c < C; ++c) m += kv[c] * g[c];
                    sum += m;
                }
                if (mt) {
                    double m = 0.0;
                    for (int c = 0; c < C; ++c) m += kt[c] * g[c];
                    sum += m;
                }
                out[p] = sum / n;
            }
        }
    }
    free(G);
    free(kv);
    free(kt);
    return 0;
}

/* ---------------------------------------------------------------------- */
/* Peak decode: first maximum by linear scan (strict >).                   */
/* heat [B,R,Ho,Wo]; row_valid [B,R] or NULL (all rows valid).             */
/* Invalid rows: idx -1, xy NaN, score -inf, gap NaN.                      */
/* gap = best - max over all other cells (+inf for a 1-cell map).          */
/* corners: the index maps to -1..1 with the first and last cell at -1 and */
/* +1 (the convention of align_corners=True grids; 0 for a 1-cell axis)     */
/* instead of the cell centres.                                            */
/* ---------------------------------------------------------------------- */
static double index_coord(long i, int n, int corners)
{
    if (!corners) return (2.0 * (double)i + 1.0) / n - 1.0;
    return n > 1 ? 2.0 * (double)i / (n - 1) - 1.0 : 0.0;
}

int gko_peak_decode(const double *heat, const uint8_t *row_valid, int B,
                    int R, int Ho, int Wo, int corners, int32_t *idx,
                    double *xy, double *score, double *gap)
{
    if (B < 0 || R < 0 || Ho < 1 || Wo < 1) return 2;
    const long P = (long)Ho * Wo;
#pragma omp parallel for schedule(static)
    for (long br = 0; br < (long)B * R; ++br) {
        if (row_valid && !row_valid[br]) {
            idx[br] = -1;
            xy[2 * br] = NAN;
            xy[2 * br + 1] = NAN;
            score[br] = -INFINITY;
            gap[br] = NAN;
            continue;
        }
        const double *h = heat + br * P;
        long best = 0;
        for (long p = 1; p < P; ++p)
            if (h[p] > h[best]) best = p;
        double second = -INFINITY;
        for (long p = 0; p < P; ++p)
            if (p != best && h[p] > second) second = h[p];
        idx[br] = (int32_t)best;
        xy[2 * br] = index_coord(best % Wo, Wo, corners);
        xy[2 * br + 1] = index_coord(best / Wo, Ho, corners);
        score[br] = h[best];
        gap[br] = (P > 1) ? h[best] - second : INFINITY;
    }
    return 0;
}

/* ---------------------------------------------------------------------- */
/* ROI stage either side of the head (model card, section "Model": the     */
/* Input bullet resizes the image so its longer side is the input size,    */
/* centre-pads it to a square with the mean colour (124, 116, 104) and     */
/* applies ImageNet normalisation; the Output bullet gives the keypoints   */
/* in the ROI's -1..1 frame. Top-down use crops each detector box first).  */
/*                                                                         */
/* Readings where the card is silent:                                      */
/*   - a box is an integer pixel rectangle (x0, y0, x1, y1), x1 and y1     */
/*     exclusive, clamped to the image; an empty box gives a canvas of     */
/*     pad colour and NaN back-projections;                                */
/*   - the resized size: the longer side becomes L, the shorter one is     */
/*     round(short * L / long), halves rounded up, at least 1 (integers);  */
/*   - the pad splits with the odd pixel on the right / bottom;            */
/*   - the resize is bilinear with half-pixel centres and edge clamping    */
/*     inside the crop (the convention of the head's own upsample), no     */
/*     antialiasing and no re-quantisation to 8 bits;                      */
/*   - ImageNet normalisation: (v / 255 - mean_c) / std_c with mean         */
/*     (0.485, 0.456, 0.406) and std (0.229, 0.224, 0.225), pad included;  */
/*   - a -1..1 coordinate spans the canvas edge to edge, and image          */
/*     coordinates are continuous (pixel i covers [i, i + 1)).             */
/* ---------------------------------------------------------------------- */
static const double roi_mean[3] = {0.485, 0.456, 0.406};
static const double roi_std[3] = {0.229, 0.224, 0.225};
static const double roi_pad[3] = {124.0, 116.0, 104.0};

typedef struct {
    int x0, y0, bw, bh;   /* clamped box; bw or bh 0 = empty */
    int nw, nh;           /* resized size */
    int px, py;           /* left / top pad */
} roi_geom;

static roi_geom roi_geometry(const int *box, int H, int W, int L)
{
    roi_geom g;
    int x0 = box[0], y0 = box[1], x1 = box[2], y1 = box[3];
    x0 = x0 < 0 ? 0 : (x0 > W ? W : x0);
    x1 = x1 < 0 ? 0 : (x1 > W ? W : x1);
    y0 = y0 < 0 ? 0 : (y0 > H ? H : y0);
    y1 = y1 < 0 ? 0 : (y1 > H ? H : y1);
    g.x0 = x0;
    g.y0 = y0;
    g.bw = x1 > x0 ? x1 - x0 : 0;
    g.bh = y1 > y0 ? y1 - y0 : 0;
    g.nw = g.nh = g.px = g.py = 0;
    if (g.bw == 0 || g.bh == 0) {
        g.bw = g.bh = 0;
        return g;
    }
    const long lng = g.bw > g.bh ? g.bw : g.bh;
    /* round(side * L / long), halves up, in exact integers */
    g.nw = (int)(((long)2 * g.bw * L + lng) / ((long)2 * lng));
    g.nh = (int)(((long)2 * g.bh * L + lng) / ((long)2 * lng));
    if (g.nw < 1) g.nw = 1;
    if (g.nh < 1) g.nh = 1;
    g.px = (L - g.nw) / 2;
    g.py = (L - g.nh) / 2;
    return g;
}

/* Source taps of output sample o when n_in samples are resized to n_out:
 * half-pixel centres, negative positions clamped to 0, upper tap clamped. */
static void resize_taps(int o, int n_in, int n_out, int *i0, int *i1, double *lam)
{
    double src = ((double)o + 0.5) * ((double)n_in / (double)n_out) - 0.5;
    if (src < 0.0) src = 0.0;
    int a = (int)floor(src);
    if (a > n_in - 1) a = n_in - 1;
    *i0 = a;
    *i1 = a + 1 < n_in ? a + 1 : n_in - 1;
    *lam = src - (double)a;
}

/* image [H,W,3] uint8 RGB, boxes [B,4]; out [B,3,L,L]. */
int gko_roi_preprocess(const uint8_t *image, int H, int W, const int *boxes,
                       int B, int L, double *out)
{
    if (H < 1 || W < 1 || B < 0 || L < 1) return 2;
    const long LL = (long)L * L;
#pragma omp parallel for schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        const roi_geom g = roi_geometry(boxes + 4 * b, H, W, L);
        /* 1. the canvas starts as the pad colour */
        double *canvas = malloc(sizeof(double) * 3 * LL);
        for (long p = 0; p < LL; ++p)
            for (int c = 0; c < 3; ++c) canvas[3 * p + c] = roi_pad[c];
        if (g.bw > 0) {
            /* 2. crop the box */
            double *crop = malloc(sizeof(double) * 3 * (long)g.bw * g.bh);
            for (int y = 0; y < g.bh; ++y)
                for (int x = 0; x < g.bw; ++x)
                    for (int c = 0; c < 3; ++c)
                        crop[3 * ((long)y * g.bw + x) + c] =
                            image[3 * ((long)(g.y0 + y) * W + g.x0 + x) + c];
            /* 3. resize it to nh x nw and paste it centred */
            for (int v = 0; v < g.nh; ++v) {
                int r0, r1;
                double ly;
                resize_taps(v, g.bh, g.nh, &r0, &r1, &ly);
                for (int u = 0; u < g.nw; ++u) {
                    int s0, s1;
                    double lx;
                    resize_taps(u, g.bw, g.nw, &s0, &s1, &lx);
                    for (int c = 0; c < 3; ++c) {
                        const double a = crop[3 * ((long)r0 * g.bw + s0) + c];
                        const double bq = crop[3 * ((long)r0 * g.bw + s1) + c];
                        const double cq = crop[3 * ((long)r1 * g.bw + s0) + c];
                        const double d = crop[3 * ((long)r1 * g.bw + s1) + c];
                        const double top = (1.0 - lx) * a + lx * bq;
                        const double bot = (1.0 - lx) * cq + lx * d;
                        canvas[3 * ((long)(g.py + v) * L + g.px + u) + c] =
                            (1.0 - ly) * top + ly * bot;
                    }
                }
            }
            free(crop);
        }
        /* 4. ImageNet normalisation, channels first */
        for (int c = 0; c < 3; ++c)
            for (long p = 0; p < LL; ++p)
                out[(long)b * 3 * LL + (long)c * LL + p] =
                    (canvas[3 * p + c] / 255.0 - roi_mean[c]) / roi_std[c];
        free(canvas);
    }
    return 0;
}

/* xy [B,R,2] in the canvas's -1..1 frame -> image coordinates [B,R,2]:
 * the canvas position (x + 1) L / 2, less the pad, scaled back by the
 * crop's size over the resized size, plus the box origin. */
int gko_roi_backproject(const double *xy, const int *boxes, int B, int R,
                        int H, int W, int L, double *out)
{
    if (H < 1 || W < 1 || B < 0 || R < 0 || L < 1) return 2;
    for (int b = 0; b < B; ++b) {
        const roi_geom g = roi_geometry(boxes + 4 * b, H, W, L);
        for (int r = 0; r < R; ++r) {
            const long o = 2 * ((long)b * R + r);
            if (g.bw == 0) {
                out[o] = out[o + 1] = NAN;
                continue;
            }
            const double xc = (xy[o] + 1.0) * L / 2.0;
            const double yc = (xy[o + 1] + 1.0) * L / 2.0;
            out[o] = g.x0 + (xc - g.px) * ((double)g.bw / g.nw);
            out[o + 1] = g.y0 + (yc - g.py) * ((double)g.bh / g.nh);
        }
    }
    return 0;
}
