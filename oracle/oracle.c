/*
 * oracle.c - plain, slow CPU oracle for the transposed-convolution / pooling
 * path, in fp64.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The GPU library
 * never links, calls or includes anything from here, and this file includes
 * nothing from the GPU side.
 *
 * Sources (web pages on the POPCORNBENCH site, one problem each):
 *   [p50] "Kimi-K2.6 l2_p50": ConvTranspose3d(3->16, k3, s2, p1) -> x0.5 ->
 *         AvgPool3d(2) -> +bias -> x1.0 on a [128,3,16,32,32] input.
 *   [p46] "Kimi-K2.6 l1_p46": AvgPool3d(k3, s2, p1) on [16,32,128,128,256].
 *   [p74] "Kimi-K2.6 l1_p74": ConvTranspose1d(32->64, k5, s1, p0, dilation 3,
 *         no bias) on [32,32,131072].
 *
 * Every routine is the literal definition: transposed convolutions are
 * written in SCATTER form (each input element adds weight * value into the
 * outputs it reaches), pooling is a literal window loop.  Inputs are fp32 (the
 * values the GPU sees); all arithmetic and every output is fp64.  Nothing is
 * blocked, fused or reordered beyond the definition.  Work is split over
 * independent (batch, channel) slices with OpenMP; each slice is computed by
 * one thread in the definition's order, so results do not depend on the
 * thread count.
 *
 * Return value of every routine: 0 on success, -1 on an invalid geometry
 * (non-positive sizes, empty output), -2 when a scratch allocation fails.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* floor(a / b) for b > 0 and any sign of a. */
static int64_t floor_div(int64_t a, int64_t b)
{
    int64_t q = a / b;
    if ((a % b != 0) && (a < 0)) q -= 1;
    return q;
}

/*
 * Length of a transposed convolution's output along one axis:
 *   (in - 1) * stride - 2 * pad + dilation * (k - 1) + out_pad + 1.
 * [p50], passage deriving the ConvTranspose3d output shape (31/63/63 from
 * 16/32/32); [p74], opening passage deriving L_out = L + 12.
 */
int64_t oracle_convT_out_len(int64_t in, int64_t k, int64_t stride, int64_t pad,
                             int64_t out_pad, int64_t dilation)
{
    return (in - 1) * stride - 2 * pad + dilation * (k - 1) + out_pad + 1;
}

/*
 * Length of an average pool's output along one axis (ceil_mode off):
 *   floor((in + 2 * pad - k) / stride) + 1.
 * [p50], passage on the AvgPool3d(2) output shape (31 -> 15);
 * [p46], opening passage (128 -> 64, 256 -> 128).
 */
int64_t oracle_pool_out_len(int64_t in, int64_t k, int64_t stride, int64_t pad)
{
    return floor_div(in + 2 * pad - k, stride) + 1;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Scatter one output channel `co` of a 3D transposed convolution for one
 * batch item into y[Do][Ho][Wo] (which the caller zeroes):
 *   for every input (ci, id, ih, iw) and tap (kd, kh, kw), the value
 *   x[ci,id,ih,iw] * w[ci,co,kd,kh,kw] is added at
 *   (id*s - p + kd, ih*s - p + kh, iw*s - p + kw) when that lies inside the
 *   output.  [p50], passage stating how ConvTranspose3d places each input
 *   element into the output (output position = input * stride + k - pad).
 * x points at this batch item's [Cin][D][H][W] block; w is [Cin][Cout][k][k][k].
 */
static void scatter3d_channel(const float *x, const float *w, int64_t co,
                              int64_t Cin, int64_t D, int64_t H, int64_t W,
                              int64_t Cout, int64_t k, int64_t s, int64_t p,
                              int64_t Do, int64_t Ho, int64_t Wo, double *y)
{
    for (int64_t ci = 0; ci < Cin; ++ci) {
        const float *xc = x + ci * D * H * W;
        const float *wc = w + (ci * Cout + co) * k * k * k;
        for (int64_t id = 0; id < D; ++id)
        for (int64_t ih = 0; ih < H; ++ih)
        for (int64_t iw = 0; iw < W; ++iw) {
            double v = (double)xc[(id * H + ih) * W + iw];
            for (int64_t kd = 0; kd < k; ++kd) {
                int64_t od = id * s - p + kd;
                if (od < 0 || od >= Do) continue;
                for (int64_t kh = 0; kh < k; ++kh) {
                    int64_t oh = ih * s - p + kh;
                    if (oh < 0 || oh >= Ho) continue;
                    for (int64_t kw = 0; kw < k; ++kw) {
                        int64_t ow = iw * s - p + kw;
                        if (ow < 0 || ow >= Wo) continue;
                        y[(od * Ho + oh) * Wo + ow] +=
                            v * (double)wc[(kd * k + kh) * k + kw];
                    }
                }
            }
        }
    }
}

/*
 * Plain 3D transposed convolution (no pooling), scatter form, optional bias:
 *   y[n,co,...] = scatter of x with w, then + conv_bias[co] when given.
 * x [N,Cin,D,H,W], w [Cin,Cout,k,k,k], conv_bias [Cout] or NULL,
 * y [N,Cout,Do,Ho,Wo] with Do = oracle_convT_out_len(D, k, s, p, op, 1).
 */
int oracle_convT3d(const float *x, const float *w, const float *conv_bias,
                   int64_t N, int64_t Cin, int64_t D, int64_t H, int64_t W,
                   int64_t Cout, int64_t k, int64_t s, int64_t p, int64_t op,
                   double *y)
{
    if (N <= 0 || Cin <= 0 || D <= 0 || H <= 0 || W <= 0 || Cout <= 0 ||
        k <= 0 || s <= 0 || p < 0 || op < 0)
        return -1;
    int64_t Do = oracle_convT_out_len(D, k, s, p, op, 1);
    int64_t Ho = oracle_convT_out_len(H, k, s, p, op, 1);
    int64_t Wo = oracle_convT_out_len(W, k, s, p, op, 1);
    if (Do <= 0 || Ho <= 0 || Wo <= 0) return -1;
    int64_t plane = Do * Ho * Wo;

    #pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t n = 0; n < N; ++n)
    for (int64_t co = 0; co < Cout; ++co) {
        double *yc = y + (n * Cout + co) * plane;
        memset(yc, 0, (size_t)plane * sizeof(double));
        scatter3d_channel(x + n * Cin * D * H * W, w, co, Cin, D, H, W, Cout,
                          k, s, p, Do, Ho, Wo, yc);
        if (conv_bias)
            for (int64_t i = 0; i < plane; ++i) yc[i] += (double)conv_bias[co];
    }
    return 0;
}

/*
 * The fused chain of [p50] (its problem statement and the model's forward):
 *   1. Y = ConvTranspose3d(x; w, stride s, pad p, output_padding op) + conv_bias
 *   2. Y = Y * scale1
 *   3. P = AvgPool3d(Y; kernel pk, stride ps, pad 0, floor mode), i.e. the sum
 *      over each pk^3 window divided by pk^3
 *   4. P = P + bias[co]
 *   5. out = P * scale2
 * in exactly that order, each step applied elementwise over the whole
 * pre-pool volume of one (n, co) before the next.  conv_bias and bias may be
 * NULL (read as 0).  out is [N,Cout,Dp,Hp,Wp] with
 * Dp = oracle_pool_out_len(Do, pk, ps, 0).
 */
int oracle_convT3d_scale_pool_bias(const float *x, const float *w,
                                   const float *conv_bias, const float *bias,
                                   double scale1, double scale2,
                                   int64_t N, int64_t Cin, int64_t D, int64_t H,
                                   int64_t W, int64_t Cout, int64_t k,
                                   int64_t s, int64_t p, int64_t op,
                                   int64_t pk, int64_t ps, double *out)
{
    if (N <= 0 || Cin <= 0 || D <= 0 || H <= 0 || W <= 0 || Cout <= 0 ||
        k <= 0 || s <= 0 || p < 0 || op < 0 || pk <= 0 || ps <= 0)
        return -1;
    int64_t Do = oracle_convT_out_len(D, k, s, p, op, 1);
    int64_t Ho = oracle_convT_out_len(H, k, s, p, op, 1);
    int64_t Wo = oracle_convT_out_len(W, k, s, p, op, 1);
    if (Do <= 0 || Ho <= 0 || Wo <= 0) return -1;
    int64_t Dp = oracle_pool_out_len(Do, pk, ps, 0);
    int64_t Hp = oracle_pool_out_len(Ho, pk, ps, 0);
    int64_t Wp = oracle_pool_out_len(Wo, pk, ps, 0);
    if (Dp <= 0 || Hp <= 0 || Wp <= 0) return -1;
    int64_t plane = Do * Ho * Wo;
    int64_t pplane = Dp * Hp * Wp;
    double divisor = (double)(pk * pk * pk);
    int failed = 0;

    #pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t n = 0; n < N; ++n)
    for (int64_t co = 0; co < Cout; ++co) {
        double *Y = (double *)calloc((size_t)plane, sizeof(double));
        if (!Y) {
            #pragma omp atomic write
            failed = 1;
            continue;
        }
        /* step 1 */
        scatter3d_channel(x + n * Cin * D * H * W, w, co, Cin, D, H, W, Cout,
                          k, s, p, Do, Ho, Wo, Y);
        if (conv_bias)
            for (int64_t i = 0; i < plane; ++i) Y[i] += (double)conv_bias[co];
        /* step 2 */
        for (int64_t i = 0; i < plane; ++i) Y[i] *= scale1;
        /* steps 3-5 */
        double *o = out + (n * Cout + co) * pplane;
        for (int64_t dp = 0; dp < Dp; ++dp)
        for (int64_t hp = 0; hp < Hp; ++hp)
        for (int64_t wp = 0; wp < Wp; ++wp) {
            double sum = 0.0;
            for (int64_t a = 0; a < pk; ++a)
            for (int64_t b = 0; b < pk; ++b)
            for (int64_t c = 0; c < pk; ++c)
                sum += Y[((dp * ps + a) * Ho + (hp * ps + b)) * Wo + (wp * ps + c)];
            double v = sum / divisor;
            v = v + (bias ? (double)bias[co] : 0.0);
            o[(dp * Hp + hp) * Wp + wp] = v * scale2;
        }
        free(Y);
    }
    return failed ? -2 : 0;
}

/*
 * AvgPool3d over zero-padded input, floor mode.  [p46], opening passages:
 * out[d,h,w] = (sum over kd,kh,kw < k of x[d*s - p + kd, h*s - p + kh,
 * w*s - p + kw], where taps outside the input count as 0) / divisor, with
 * divisor = k^3 when count_include_pad is set (PyTorch's default, which the
 * page settles on), else the number of in-bounds taps.
 * x is NC independent [D][H][W] slices; out is NC slices of [Do][Ho][Wo].
 */
int oracle_avgpool3d(const float *x, int64_t NC, int64_t D, int64_t H,
                     int64_t W, int64_t k, int64_t s, int64_t p,
                     int count_include_pad, double *out)
{
    if (NC <= 0 || D <= 0 || H <= 0 || W <= 0 || k <= 0 || s <= 0 || p < 0)
        return -1;
    int64_t Do = oracle_pool_out_len(D, k, s, p);
    int64_t Ho = oracle_pool_out_len(H, k, s, p);
    int64_t Wo = oracle_pool_out_len(W, k, s, p);
    if (Do <= 0 || Ho <= 0 || Wo <= 0) return -1;

    #pragma omp parallel for schedule(dynamic)
    for (int64_t sl = 0; sl < NC; ++sl) {
        const float *xs = x + sl * D * H * W;
        double *os = out + sl * Do * Ho * Wo;
        for (int64_t od = 0; od < Do; ++od)
        for (int64_t oh = 0; oh < Ho; ++oh)
        for (int64_t ow = 0; ow < Wo; ++ow) {
            double sum = 0.0;
            int64_t cnt = 0;
            for (int64_t kd = 0; kd < k; ++kd)
            for (int64_t kh = 0; kh < k; ++kh)
            for (int64_t kw = 0; kw < k; ++kw) {
                int64_t id = od * s - p + kd;
                int64_t ih = oh * s - p + kh;
                int64_t iw = ow * s - p + kw;
                if (id < 0 || id >= D || ih < 0 || ih >= H || iw < 0 || iw >= W)
                    continue;
                sum += (double)xs[(id * H + ih) * W + iw];
                cnt += 1;
            }
            double div = count_include_pad ? (double)(k * k * k) : (double)cnt;
            os[(od * Ho + oh) * Wo + ow] = (cnt == 0 && !count_include_pad) ? 0.0 : sum / div;
        }
    }
    return 0;
}

/*
 * 1D transposed convolution, scatter form.  [p74], passages on the dilation
 * worked examples: input element i of channel ci adds x[n,ci,i] * w[ci,co,k]
 * at output position i*stride - pad + dilation*k, for every co and k, when that
 * position lies inside [0, L_out); then + bias[co] when given.
 * x [N,Cin,L], w [Cin,Cout,K], bias [Cout] or NULL, y [N,Cout,L_out].
 */
int oracle_convT1d(const float *x, const float *w, const float *bias,
                   int64_t N, int64_t Cin, int64_t L, int64_t Cout, int64_t K,
                   int64_t s, int64_t p, int64_t dil, int64_t op, double *y)
{
    if (N <= 0 || Cin <= 0 || L <= 0 || Cout <= 0 || K <= 0 || s <= 0 ||
        p < 0 || dil <= 0 || op < 0)
        return -1;
    int64_t Lo = oracle_convT_out_len(L, K, s, p, op, dil);
    if (Lo <= 0) return -1;

    #pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t n = 0; n < N; ++n)
    for (int64_t co = 0; co < Cout; ++co) {
        double *yc = y + (n * Cout + co) * Lo;
        memset(yc, 0, (size_t)Lo * sizeof(double));
        for (int64_t ci = 0; ci < Cin; ++ci) {
            const float *xc = x + (n * Cin + ci) * L;
            const float *wc = w + (ci * Cout + co) * K;
            for (int64_t i = 0; i < L; ++i) {
                double v = (double)xc[i];
                for (int64_t kk = 0; kk < K; ++kk) {
                    int64_t o = i * s - p + dil * kk;
                    if (o < 0 || o >= Lo) continue;
                    yc[o] += v * (double)wc[kk];
                }
            }
        }
        if (bias)
            for (int64_t o = 0; o < Lo; ++o) yc[o] += (double)bias[co];
    }
    return 0;
}
