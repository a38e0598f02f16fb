/*
 * Reference (oracle) forward 2-D convolution in float64.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library links, loads or
 * calls this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do. It shares no code with the HIP path.
 *
 * What it computes is the plain definition of the layer, not the im2win steps:
 *
 *   Ho = floor((H + 2p - KH) / s) + 1,   Wo = floor((W + 2p - KW) / s) + 1
 *   Y[n][co][ho][wo] = sum_{ci < Cin} sum_{kh < KH} sum_{kw < KW}
 *                      Xp[n][ci][ho*s + kh - p][wo*s + kw - p] * Wt[co][ci][kh][kw]
 *
 * where Xp equals X inside [0,H) x [0,W) and is zero outside.
 *
 * Sources: the direct convolution of "Enabling Memory-efficient Im2win
 * Convolution with Multi-precision Support on GPU CUDA and Tensor Cores",
 * Sec. III-A, Eq. (1) (written there 1-based, unit stride, unpadded; read here
 * 0-based with stride s and symmetric zero padding p); the seven nested loops
 * of "Unifying Convolutions and GEMM", Sec. 1, with the padded output extent
 * of its Sec. 5; the cross-correlation convention (no kernel flip) stated in
 * "im2col Expansion, FFT Convolution, and Winograd Transforms", FFT section.
 * Taps that fall in the padding are skipped, which is exactly the same as
 * multiplying by the padding zeros.
 *
 * All arrays are contiguous NCHW (x: [N][Cin][H][W], w: [Cout][Cin][KH][KW],
 * y: [N][Cout][Ho][Wo]) of double. Inputs stored as fp32/fp16/bf16 convert to
 * double exactly, and every product of two such values is exact in double.
 */
#include <stdint.h>
#include <stddef.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* floor((in + 2p - k) / s) + 1, or 0 when no window fits (or s < 1). */
int64_t oracle_out_extent(int64_t in, int64_t k, int64_t s, int64_t p)
{
    int64_t span = in + 2 * p - k;
    if (s < 1 || k < 1 || p < 0 || span < 0) return 0;
    return span / s + 1;
}

/* One output element by the direct sum. */
static double direct_sum(int64_t Cin, int64_t H, int64_t W, int64_t KH, int64_t KW,
                         int64_t s, int64_t p, const double *xn, const double *wco,
                         int64_t ho, int64_t wo)
{
    double acc = 0.0;
    for (int64_t ci = 0; ci < Cin; ++ci) {
        const double *xc = xn + ci * H * W;
        const double *wc = wco + ci * KH * KW;
        for (int64_t kh = 0; kh < KH; ++kh) {
            int64_t ih = ho * s + kh - p;
            if (ih < 0 || ih >= H) continue;          /* padding row: zero */
            for (int64_t kw = 0; kw < KW; ++kw) {
                int64_t iw = wo * s + kw - p;
                if (iw < 0 || iw >= W) continue;      /* padding column: zero */
                acc += xc[ih * W + iw] * wc[kh * KW + kw];
            }
        }
    }
    return acc;
}

static int bad_desc(int64_t N, int64_t Cin, int64_t H, int64_t W, int64_t Cout,
                    int64_t KH, int64_t KW, int64_t s, int64_t p)
{
    return N < 1 || Cin < 1 || H < 1 || W < 1 || Cout < 1 || KH < 1 || KW < 1 ||
           s < 1 || p < 0 || oracle_out_extent(H, KH, s, p) < 1 ||
           oracle_out_extent(W, KW, s, p) < 1;
}

/* Full output. Loop order n, co | ho, wo | ci, kh, kw; OpenMP over (n, co).
 * nthreads <= 0 uses the OpenMP default. Returns 0, or -1 on a bad shape. */
int oracle_conv2d_f64(int64_t N, int64_t Cin, int64_t H, int64_t W, int64_t Cout,
                      int64_t KH, int64_t KW, int64_t s, int64_t p,
                      const double *x, const double *w, double *y, int nthreads)
{
    if (bad_desc(N, Cin, H, W, Cout, KH, KW, s, p)) return -1;
    const int64_t Ho = oracle_out_extent(H, KH, s, p);
    const int64_t Wo = oracle_out_extent(W, KW, s, p);
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for collapse(2) schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t co = 0; co < Cout; ++co) {
            const double *xn = x + n * Cin * H * W;
            const double *wco = w + co * Cin * KH * KW;
            double *yp = y + (n * Cout + co) * Ho * Wo;
            for (int64_t ho = 0; ho < Ho; ++ho)
                for (int64_t wo = 0; wo < Wo; ++wo)
                    yp[ho * Wo + wo] = direct_sum(Cin, H, W, KH, KW, s, p, xn, wco, ho, wo);
        }
    }
    (void)nthreads;
    return 0;
}

/* Selected outputs only: idx[i] is a flat NCHW index into y; out[i] receives
 * that element. Used to check full-size layers on a sample of outputs.
 * Returns 0, -1 on a bad shape, -2 on an index out of range. */
int oracle_conv2d_f64_points(int64_t N, int64_t Cin, int64_t H, int64_t W, int64_t Cout,
                             int64_t KH, int64_t KW, int64_t s, int64_t p,
                             const double *x, const double *w,
                             const int64_t *idx, int64_t count, double *out, int nthreads)
{
    if (bad_desc(N, Cin, H, W, Cout, KH, KW, s, p)) return -1;
    const int64_t Ho = oracle_out_extent(H, KH, s, p);
    const int64_t Wo = oracle_out_extent(W, KW, s, p);
    const int64_t total = N * Cout * Ho * Wo;
    for (int64_t i = 0; i < count; ++i)
        if (idx[i] < 0 || idx[i] >= total) return -2;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(static) num_threads(nthreads)
#endif
    for (int64_t i = 0; i < count; ++i) {
        int64_t f = idx[i];
        int64_t wo = f % Wo; f /= Wo;
        int64_t ho = f % Ho; f /= Ho;
        int64_t co = f % Cout;
        int64_t n = f / Cout;
        out[i] = direct_sum(Cin, H, W, KH, KW, s, p, x + n * Cin * H * W,
                            w + co * Cin * KH * KW, ho, wo);
    }
    (void)nthreads;
    return 0;
}
