// generic.hip - general-geometry kernels: any kernel size, stride, padding,
// output padding, pooling window and dtype the ABI accepts.  They gather each
// output directly from its definition on the vector ALUs; the specialised
// matrix-core kernels handle the pages' own geometry.
//
//  * Transposed convolution, gather form ([p50], passage placing input i at
//    output i*stride - pad + k; [p74], passage on the general-stride gather):
//      y[o] = sum_k x[(o + pad - dil*k) / stride] * w[k]
//    over taps whose division is exact and whose input index is in range.
//  * AvgPool ([p46], opening passages): window sum over zero padding divided
//    by k^3 (count_include_pad) or by the number of in-range taps.
//  * Fused chain ([p50], model forward): for a pooled voxel, S is the sum of
//    the transposed convolution over the pool window; the output is
//    ((S/pk^3 + conv_bias)*scale1 + bias)*scale2 (the conv bias passes
//    through the window mean unchanged).
// One thread per output element, consecutive threads along the innermost
// output axis (coalesced stores); grid-stride over 64-bit element counts.
#include "ct_internal.h"

namespace ct {
namespace {

constexpr int kThreads = 256;

template <typename T> __device__ __forceinline__ float ld(const T *p, int64_t i);
template <> __device__ __forceinline__ float ld<float>(const float *p, int64_t i) { return p[i]; }
template <> __device__ __forceinline__ float ld<uint16_t>(const uint16_t *p, int64_t i)
{
    return __uint_as_float(((unsigned)p[i]) << 16);   // bf16 -> fp32, exact
}

// Input index feeding output position o through tap k of a dilated 1D
// transposed convolution, or -1 when the division is inexact or the index
// falls outside [0, in).
__device__ __forceinline__ int in_index(int o, int k, int stride, int pad, int dil, int in)
{
    const int t = o + pad - dil * k;
    if (t < 0 || t % stride) return -1;
    const int i = t / stride;
    return i < in ? i : -1;
}

// Taps of one axis of a dilation-1 transposed convolution that feed output
// position o: tap k reaches o from input (o + pad - k) / stride when that
// division is exact, so the valid taps are k0, k0 + stride, ... with
// k0 = (o + pad) mod stride, and their inputs i0, i0 - 1, ...  The range is
// clipped to taps below k and inputs inside [0, in); n <= 0 means none.
struct Taps {
    int k0, i0, n;
};

__device__ __forceinline__ Taps axis_taps(int o, int k, int stride, int pad, int in)
{
    const int t = o + pad;
    const int k0 = t % stride, i0 = t / stride;
    const int jlo = i0 - (in - 1) > 0 ? i0 - (in - 1) : 0;   // input <= in - 1
    int jhi = k0 < k ? (k - 1 - k0) / stride : -1;          // tap < k
    if (jhi > i0) jhi = i0;                                 // input >= 0
    return {k0 + jlo * stride, i0 - jlo, jhi - jlo + 1};
}

// ConvTranspose3d value (without bias) at output (co, od, oh, ow) of one batch
// item; xn points at that item's [Cin][D][H][W] block.
template <typename T>
__device__ float convT3d_point(const T *__restrict__ xn, const T *__restrict__ w, int Cin,
                               int D, int H, int W, int Cout, int k, int s, int p, int co,
                               int od, int oh, int ow)
{
    float acc = 0.0f;
    const int64_t HW = (int64_t)H * W, DHW = (int64_t)D * HW, k3 = (int64_t)k * k * k;
    const int64_t wstride = (int64_t)Cout * k3;   // between input channels
    const Taps td = axis_taps(od, k, s, p, D), th = axis_taps(oh, k, s, p, H),
               tw = axis_taps(ow, k, s, p, W);
    for (int a = 0; a < td.n; ++a) {
        const int kd = td.k0 + a * s, id = td.i0 - a;
        for (int b = 0; b < th.n; ++b) {
            const int kh = th.k0 + b * s, ih = th.i0 - b;
            for (int c = 0; c < tw.n; ++c) {
                const int kw = tw.k0 + c * s, iw = tw.i0 - c;
                const int64_t xo = (int64_t)id * HW + (int64_t)ih * W + iw;
                const int64_t wo = (int64_t)co * k3 + ((int64_t)kd * k + kh) * k + kw;
                for (int ci = 0; ci < Cin; ++ci)
                    acc = __builtin_fmaf(ld(xn, ci * DHW + xo), ld(w, ci * wstride + wo), acc);
            }
        }
    }
    return acc;
}

template <typename T>
__global__ __launch_bounds__(kThreads)
void fused3d_generic_kernel(const T *__restrict__ x, const T *__restrict__ w,
                            const float *__restrict__ conv_bias, const float *__restrict__ bias,
                            float s1, float s2, float inv, int Cin, int D, int H, int W,
                            int Cout, int k, int s, int p, int pk, int ps, int Dp, int Hp,
                            int Wp, int64_t total, float *__restrict__ out)
{
    for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * kThreads) {
        int64_t t = e;
        const int wp = (int)(t % Wp); t /= Wp;
        const int hp = (int)(t % Hp); t /= Hp;
        const int dp = (int)(t % Dp); t /= Dp;
        const int co = (int)(t % Cout);
        const int64_t n = t / Cout;
        const T *xn = x + n * Cin * (int64_t)D * H * W;
        float S = 0.0f;
        for (int a = 0; a < pk; ++a)
            for (int b = 0; b < pk; ++b)
                for (int c = 0; c < pk; ++c)
                    S += convT3d_point(xn, w, Cin, D, H, W, Cout, k, s, p, co,
                                       dp * ps + a, hp * ps + b, wp * ps + c);
        float v = S * inv;
        v = (v + (conv_bias ? conv_bias[co] : 0.0f)) * s1;
        v = (v + (bias ? bias[co] : 0.0f)) * s2;
        out[e] = v;
    }
}

template <typename T>
__global__ __launch_bounds__(kThreads)
void convT3d_generic_kernel(const T *__restrict__ x, const T *__restrict__ w,
                            const float *__restrict__ bias, int Cin, int D, int H, int W,
                            int Cout, int k, int s, int p, int Do, int Ho, int Wo, int64_t total,
                            float *__restrict__ y)
{
    for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * kThreads) {
        int64_t t = e;
        const int ow = (int)(t % Wo); t /= Wo;
        const int oh = (int)(t % Ho); t /= Ho;
        const int od = (int)(t % Do); t /= Do;
        const int co = (int)(t % Cout);
        const int64_t n = t / Cout;
        const T *xn = x + n * Cin * (int64_t)D * H * W;
        y[e] = convT3d_point(xn, w, Cin, D, H, W, Cout, k, s, p, co, od, oh, ow) +
               (bias ? bias[co] : 0.0f);
    }
}

__global__ __launch_bounds__(kThreads)
void avgpool3d_generic_kernel(const float *__restrict__ x, int D, int H, int W, int k, int s,
                              int p, int include_pad, float kvol, int Do, int Ho, int Wo,
                              int64_t total, float *__restrict__ out)
{
    for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * kThreads) {
        int64_t t = e;
        const int ow = (int)(t % Wo); t /= Wo;
        const int oh = (int)(t % Ho); t /= Ho;
        const int od = (int)(t % Do);
        const int64_t sl = t / Do;
        const float *xs = x + sl * (int64_t)D * H * W;
        float sum = 0.0f;
        int cnt = 0;
        for (int kd = 0; kd < k; ++kd) {
            const int id = od * s - p + kd;
            if (id < 0 || id >= D) continue;
            for (int kh = 0; kh < k; ++kh) {
                const int ih = oh * s - p + kh;
                if (ih < 0 || ih >= H) continue;
                for (int kw = 0; kw < k; ++kw) {
                    const int iw = ow * s - p + kw;
                    if (iw < 0 || iw >= W) continue;
                    sum += xs[((int64_t)id * H + ih) * W + iw];
                    ++cnt;
                }
            }
        }
        out[e] = sum / (include_pad ? kvol : (float)cnt);
    }
}

template <typename T>
__global__ __launch_bounds__(kThreads)
void convT1d_generic_kernel(const T *__restrict__ x, const T *__restrict__ w,
                            const float *__restrict__ bias, int Cin, int L, int Cout, int K,
                            int s, int p, int dil, int Lo, int64_t total, float *__restrict__ y)
{
    for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < total;
         e += (int64_t)gridDim.x * kThreads) {
        const int o = (int)(e % Lo);
        int64_t t = e / Lo;
        const int co = (int)(t % Cout);
        const int64_t n = t / Cout;
        const T *xn = x + n * Cin * (int64_t)L;
        float acc = 0.0f;
        for (int kk = 0; kk < K; ++kk) {
            const int i = in_index(o, kk, s, p, dil, L);
            if (i < 0) continue;
            for (int ci = 0; ci < Cin; ++ci)
                acc = __builtin_fmaf(ld(xn, (int64_t)ci * L + i),
                                     ld(w, ((int64_t)ci * Cout + co) * K + kk), acc);
        }
        y[e] = acc + (bias ? bias[co] : 0.0f);
    }
}

// One thread per output up to 2^16 workgroups (256 per CU); larger problems
// loop over the grid.
unsigned grid_for(int64_t total)
{
    constexpr int64_t kMaxBlocks = 65536;
    const int64_t blocks = (total + kThreads - 1) / kThreads;
    return (unsigned)(blocks < kMaxBlocks ? blocks : kMaxBlocks);
}

}  // namespace

hipError_t launch_fused3d_generic(const void *x, const void *w, bool bf16,
                                  const float *conv_bias, const float *bias, float s1, float s2,
                                  int64_t N, int64_t Cin, int64_t D, int64_t H, int64_t W,
                                  int64_t Cout, int k, int s, int p, int op, int pk, int ps,
                                  float *out, hipStream_t stream)
{
    const int64_t Do = (D - 1) * s - 2 * p + k + op, Ho = (H - 1) * s - 2 * p + k + op,
                  Wo = (W - 1) * s - 2 * p + k + op;
    const int64_t Dp = (Do - pk) / ps + 1, Hp = (Ho - pk) / ps + 1, Wp = (Wo - pk) / ps + 1;
    const int64_t total = N * Cout * Dp * Hp * Wp;
    const float inv = (float)(1.0 / ((double)pk * pk * pk));
    if (bf16)
        hipLaunchKernelGGL(fused3d_generic_kernel<uint16_t>, dim3(grid_for(total)), dim3(kThreads), 0,
                           stream, (const uint16_t *)x, (const uint16_t *)w, conv_bias, bias, s1, s2,
                           inv, (int)Cin, (int)D, (int)H, (int)W, (int)Cout, k, s, p, pk, ps,
                           (int)Dp, (int)Hp, (int)Wp, total, out);
    else
        hipLaunchKernelGGL(fused3d_generic_kernel<float>, dim3(grid_for(total)), dim3(kThreads), 0,
                           stream, (const float *)x, (const float *)w, conv_bias, bias, s1, s2,
                           inv, (int)Cin, (int)D, (int)H, (int)W, (int)Cout, k, s, p, pk, ps,
                           (int)Dp, (int)Hp, (int)Wp, total, out);
    return hipGetLastError();
}

hipError_t launch_convT3d_generic(const void *x, const void *w, bool bf16, const float *bias,
                                  int64_t N, int64_t Cin, int64_t D, int64_t H, int64_t W,
                                  int64_t Cout, int k, int s, int p, int op, float *y,
                                  hipStream_t stream)
{
    const int64_t Do = (D - 1) * s - 2 * p + k + op, Ho = (H - 1) * s - 2 * p + k + op,
                  Wo = (W - 1) * s - 2 * p + k + op;
    const int64_t total = N * Cout * Do * Ho * Wo;
    if (bf16)
        hipLaunchKernelGGL(convT3d_generic_kernel<uint16_t>, dim3(grid_for(total)), dim3(kThreads), 0,
                           stream, (const uint16_t *)x, (const uint16_t *)w, bias, (int)Cin, (int)D,
                           (int)H, (int)W, (int)Cout, k, s, p, (int)Do, (int)Ho, (int)Wo, total, y);
    else
        hipLaunchKernelGGL(convT3d_generic_kernel<float>, dim3(grid_for(total)), dim3(kThreads), 0,
                           stream, (const float *)x, (const float *)w, bias, (int)Cin, (int)D,
                           (int)H, (int)W, (int)Cout, k, s, p, (int)Do, (int)Ho, (int)Wo, total, y);
    return hipGetLastError();
}

hipError_t launch_avgpool3d_generic(const float *x, int64_t NC, int64_t D, int64_t H, int64_t W,
                                    int k, int s, int p, int include_pad, float *out,
                                    hipStream_t stream)
{
    const int64_t Do = (D + 2 * p - k) / s + 1, Ho = (H + 2 * p - k) / s + 1,
                  Wo = (W + 2 * p - k) / s + 1;
    const int64_t total = NC * Do * Ho * Wo;
    hipLaunchKernelGGL(avgpool3d_generic_kernel, dim3(grid_for(total)), dim3(kThreads), 0, stream,
                       x, (int)D, (int)H, (int)W, k, s, p, include_pad, (float)k * k * k, (int)Do,
                       (int)Ho, (int)Wo, total, out);
    return hipGetLastError();
}

hipError_t launch_convT1d_generic(const void *x, const void *w, bool bf16, const float *bias,
                                  int64_t N, int64_t Cin, int64_t L, int64_t Cout, int K, int s,
                                  int p, int dil, int op, float *y, hipStream_t stream)
{
    const int64_t Lo = (L - 1) * s - 2 * p + dil * (K - 1) + op + 1;
    const int64_t total = N * Cout * Lo;
    if (bf16)
        hipLaunchKernelGGL(convT1d_generic_kernel<uint16_t>, dim3(grid_for(total)), dim3(kThreads), 0,
                           stream, (const uint16_t *)x, (const uint16_t *)w, bias, (int)Cin, (int)L,
                           (int)Cout, K, s, p, dil, (int)Lo, total, y);
    else
        hipLaunchKernelGGL(convT1d_generic_kernel<float>, dim3(grid_for(total)), dim3(kThreads), 0,
                           stream, (const float *)x, (const float *)w, bias, (int)Cin, (int)L,
                           (int)Cout, K, s, p, dil, (int)Lo, total, y);
    return hipGetLastError();
}

}  // namespace ct
