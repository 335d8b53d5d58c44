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
// output axis (coalesced stores), grid-stride.  Element indices are 32-bit
// when the output has fewer than 2^31 elements, and every division by a
// runtime size (index decode, stride) is then a multiply-high by a
// precomputed reciprocal instead of a software division loop.
#include "ct_internal.h"

namespace ct {
namespace {

constexpr int kThreads = 256;

// Unsigned division by a run-time constant d (1 <= d < 2^32), after
// Granlund and Montgomery, "Division by invariant integers using
// multiplication" (PLDI 1994): with l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, n / d = (umulhi(m, n) + n) >> l for
// every 32-bit n (the sum is formed in 64 bits).  64-bit dividends use the
// ordinary division.
struct Div {
    uint32_t d, m, l;
    __device__ __forceinline__ uint32_t q(uint32_t n) const
    {
        const uint32_t t = __umulhi(m, n);
        return (uint32_t)(((uint64_t)t + n) >> l);
    }
    __device__ __forceinline__ uint64_t q(uint64_t n) const { return n / d; }
};

Div make_div(uint32_t d)
{
    uint32_t l = 0;
    while (l < 32 && (uint64_t(1) << l) < d) ++l;
    const uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1;
    return {d, (uint32_t)m, l};
}

template <typename T> __device__ __forceinline__ float ld(const T *p, int64_t i);
template <> __device__ __forceinline__ float ld<float>(const float *p, int64_t i) { return p[i]; }
template <> __device__ __forceinline__ float ld<uint16_t>(const uint16_t *p, int64_t i)
{
    return __uint_as_float(((unsigned)p[i]) << 16);   // bf16 -> fp32, exact
}
// fp32 result -> element: as is, or rounded to the nearest bf16 (ties to even)
template <typename T, typename I> __device__ __forceinline__ void st(T *p, I i, float v);
template <typename I> __device__ __forceinline__ void st(float *p, I i, float v) { p[i] = v; }
template <typename I> __device__ __forceinline__ void st(uint16_t *p, I i, float v)
{
    p[i] = __builtin_bit_cast(uint16_t, (__bf16)v);
}

// Geometry of a 3D transposed convolution (dilation 1) and the pool after it.
struct Geo3 {
    int Cin, D, H, W, Cout, k, s, p, pk, ps;
};

// Taps of one axis that feed output position o: tap k reaches o from input
// (o + pad - k) / stride when that division is exact, so the valid taps are
// k0, k0 + stride, ... with k0 = (o + pad) mod stride, and their inputs
// i0, i0 - 1, ...  The range is clipped to taps below k and inputs inside
// [0, in); n <= 0 means none.
struct Taps {
    int k0, i0, n;
};

__device__ __forceinline__ Taps axis_taps(int o, int k, const Div &ds, int pad, int in)
{
    const uint32_t t = (uint32_t)(o + pad);
    const int i0 = (int)ds.q(t), k0 = (int)(t - (uint32_t)i0 * ds.d);
    const int jlo = i0 - (in - 1) > 0 ? i0 - (in - 1) : 0;          // input <= in - 1
    int jhi = k0 < k ? (int)ds.q((uint32_t)(k - 1 - k0)) : -1;      // tap < k
    if (jhi > i0) jhi = i0;                                         // input >= 0
    return {k0 + jlo * (int)ds.d, i0 - jlo, jhi - jlo + 1};
}

// ConvTranspose3d value (without bias) at output (co, od, oh, ow) of one batch
// item; xn points at that item's [Cin][D][H][W] block.
// acc + sum over ci < Cin of x[ci*xs + xo] * w[ci*ws + wo], one fma per
// channel in channel order.  Channels go four at a time: all eight loads of a
// group are issued before its fmas (a loop over a run-time count would wait
// on each pair), from clamped addresses that are always valid; a clamped
// duplicate's fma result is discarded by a select, so the sum and its NaN /
// infinity behaviour are those of the plain loop.  Used by the position-ordered 1D
// kernel; the 3D gather keeps the plain loop, which was faster with 3
// channels (1.4 against 2.2 ms).
template <int G = 4, typename T>
__device__ __forceinline__ float dot_ci(const T *__restrict__ xn, int64_t xs, int64_t xo,
                                        const T *__restrict__ w, int64_t ws, int64_t wo, int Cin,
                                        float acc)
{
    for (int ci = 0; ci < Cin; ci += G) {
        float xv[G], wv[G];
#pragma unroll
        for (int u = 0; u < G; ++u) {
            const int c = min(ci + u, Cin - 1);
            xv[u] = ld(xn, c * xs + xo);
            wv[u] = ld(w, c * ws + wo);
        }
#pragma unroll
        for (int u = 0; u < G; ++u) {
            const float f = __builtin_fmaf(xv[u], wv[u], acc);
            acc = ci + u < Cin ? f : acc;
        }
    }
    return acc;
}

template <typename T>
__device__ float convT3d_point(const T *__restrict__ xn, const T *__restrict__ w, const Geo3 &g,
                               const Div &ds, int co, int od, int oh, int ow)
{
    float acc = 0.0f;
    const int k = g.k, s = g.s;
    const int64_t HW = (int64_t)g.H * g.W, DHW = (int64_t)g.D * HW, k3 = (int64_t)k * k * k;
    const int64_t wstride = (int64_t)g.Cout * k3;   // between input channels
    const Taps td = axis_taps(od, k, ds, g.p, g.D), th = axis_taps(oh, k, ds, g.p, g.H),
               tw = axis_taps(ow, k, ds, g.p, g.W);
    for (int a = 0; a < td.n; ++a) {
        const int kd = td.k0 + a * s, id = td.i0 - a;
        for (int b = 0; b < th.n; ++b) {
            const int kh = th.k0 + b * s, ih = th.i0 - b;
            for (int c = 0; c < tw.n; ++c) {
                const int kw = tw.k0 + c * s, iw = tw.i0 - c;
                const int64_t xo = (int64_t)id * HW + (int64_t)ih * g.W + iw;
                const int64_t wo = (int64_t)co * k3 + ((int64_t)kd * k + kh) * k + kw;
                for (int ci = 0; ci < g.Cin; ++ci)
                    acc = __builtin_fmaf(ld(xn, ci * DHW + xo), ld(w, ci * wstride + wo), acc);
            }
        }
    }
    return acc;
}

// Splits a flat index into (rest, coordinate) for one axis of size d.
template <typename I>
__device__ __forceinline__ int peel(I &e, const Div &dv)
{
    const I q = dv.q(e);
    const int c = (int)(e - q * (I)dv.d);
    e = q;
    return c;
}

template <typename T, typename I>
__global__ __launch_bounds__(kThreads)
void fused3d_generic_kernel(const T *__restrict__ x, const T *__restrict__ w,
                            const float *__restrict__ conv_bias, const float *__restrict__ bias,
                            float s1, float s2, float inv, Geo3 g, Div dWp, Div dHp, Div dDp,
                            Div dCout, Div ds, I total, float *__restrict__ out)
{
    const int64_t xitem = (int64_t)g.Cin * g.D * g.H * g.W;
    for (I e = (I)blockIdx.x * kThreads + threadIdx.x; e < total; e += (I)gridDim.x * kThreads) {
        I t = e;
        const int wp = peel(t, dWp), hp = peel(t, dHp), dp = peel(t, dDp), co = peel(t, dCout);
        const T *xn = x + (int64_t)t * xitem;
        float S = 0.0f;
        for (int a = 0; a < g.pk; ++a)
            for (int b = 0; b < g.pk; ++b)
                for (int c = 0; c < g.pk; ++c)
                    S += convT3d_point(xn, w, g, ds, co, dp * g.ps + a, hp * g.ps + b,
                                       wp * g.ps + c);
        float v = S * inv;
        v = (v + (conv_bias ? conv_bias[co] : 0.0f)) * s1;
        v = (v + (bias ? bias[co] : 0.0f)) * s2;
        out[e] = v;
    }
}

// The page's geometry (k3, s2, p1, 2-pool) with any output padding, from the
// effective filter ([p50], passage grouping the 27 weight terms by input
// tap): a pooled voxel is sum_ci sum_{a,b,c} x[ci, d+a, h+b, w+c] *
// Weff[ci, co, abc] / 8, where input offset 0 along an axis pairs with taps
// {1, 2} and offset 1 with tap {0}.  Inputs past the far edge read 0, which
// is all that output_padding = 1 changes.  Weff is formed once per workgroup
// in LDS.  A thread takes one pooled voxel and a block of up to 16 output
// channels: it loads each input channel's 8 taps once (together, from clamped
// addresses, masking the ones past the edge with a select) and applies them
// to every channel of the block.
template <typename T, typename I>
__global__ __launch_bounds__(kThreads)
void fused3d_weff_kernel(const T *__restrict__ x, const T *__restrict__ w,
                         const float *__restrict__ conv_bias, const float *__restrict__ bias,
                         float s1, float s2, Geo3 g, int Dp, int Hp, int Wp, Div dWp, Div dHp,
                         Div dDp, Div dCb, I total, float *__restrict__ out)
{
    extern __shared__ float weff[];            // [Cin][Cout][8], tap = 4a + 2b + c
    const int nw = g.Cin * g.Cout * 8;
    for (int e = threadIdx.x; e < nw; e += kThreads) {
        const int tap = e & 7;
        const int a = tap >> 2, b = (tap >> 1) & 1, c = tap & 1;
        const T *wk = w + (int64_t)(e >> 3) * 27;   // w[ci][co][3][3][3]
        float sum = 0.0f;
        for (int kd = a ? 0 : 1; kd <= (a ? 0 : 2); ++kd)
            for (int kh = b ? 0 : 1; kh <= (b ? 0 : 2); ++kh)
                for (int kw = c ? 0 : 1; kw <= (c ? 0 : 2); ++kw)
                    sum += ld(wk, (kd * 3 + kh) * 3 + kw);
        weff[e] = sum;
    }
    __syncthreads();
    constexpr int kCB = 16;                    // output channels per thread
    const int64_t HW = (int64_t)g.H * g.W, DHW = (int64_t)g.D * HW, xitem = (int64_t)g.Cin * DHW;
    const int64_t pplane = (int64_t)Dp * Hp * Wp;
    for (I e = (I)blockIdx.x * kThreads + threadIdx.x; e < total; e += (I)gridDim.x * kThreads) {
        I t = e;
        const int wp = peel(t, dWp), hp = peel(t, dHp), dp = peel(t, dDp), cb = peel(t, dCb);
        const int co0 = cb * kCB;
        const T *xc = x + (int64_t)t * xitem + dp * HW + (int64_t)hp * g.W + wp;
        const bool vd = dp + 1 < g.D, vh = hp + 1 < g.H, vw = wp + 1 < g.W;
        const int64_t od = vd ? HW : 0, oh = vh ? g.W : 0, ow = vw ? 1 : 0;
        float S[kCB];
#pragma unroll
        for (int j = 0; j < kCB; ++j) S[j] = 0.0f;
        // input channels four at a time: all 32 tap loads go out before the fmas
        for (int ci0 = 0; ci0 < g.Cin; ci0 += 4) {
            float xv[4][8];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const T *xi = xc + min(ci0 + u, g.Cin - 1) * DHW;   // clamped: always valid
#pragma unroll
                for (int tp = 0; tp < 8; ++tp) {
                    const int a = tp >> 2, b = (tp >> 1) & 1, c = tp & 1;
                    const float v = ld(xi, (a ? od : 0) + (b ? oh : 0) + (c ? ow : 0));
                    xv[u][tp] = ((a && !vd) || (b && !vh) || (c && !vw)) ? 0.0f : v;
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (ci0 + u >= g.Cin) break;              // same for every lane
                // channels past Cout read the block's first channel (never stored)
                const float *wrow = weff + (int64_t)(ci0 + u) * g.Cout * 8;
#pragma unroll
                for (int j = 0; j < kCB; ++j) {
                    const float *wf = wrow + (co0 + j < g.Cout ? co0 + j : co0) * 8;
#pragma unroll
                    for (int tp = 0; tp < 8; ++tp) S[j] = __builtin_fmaf(xv[u][tp], wf[tp], S[j]);
                }
            }
        }
        float *ob = out + ((int64_t)t * g.Cout + co0) * pplane + ((int64_t)dp * Hp + hp) * Wp + wp;
#pragma unroll
        for (int j = 0; j < kCB; ++j) {
            if (co0 + j < g.Cout) {
                float v = S[j] * 0.125f;
                v = (v + (conv_bias ? conv_bias[co0 + j] : 0.0f)) * s1;
                v = (v + (bias ? bias[co0 + j] : 0.0f)) * s2;
                ob[(int64_t)j * pplane] = v;
            }
        }
    }
}

template <typename T, typename I>
__global__ __launch_bounds__(kThreads)
void convT3d_generic_kernel(const T *__restrict__ x, const T *__restrict__ w,
                            const float *__restrict__ bias, Geo3 g, Div dWo, Div dHo, Div dDo,
                            Div dCout, Div ds, I total, float *__restrict__ y)
{
    const int64_t xitem = (int64_t)g.Cin * g.D * g.H * g.W;
    for (I e = (I)blockIdx.x * kThreads + threadIdx.x; e < total; e += (I)gridDim.x * kThreads) {
        I t = e;
        const int ow = peel(t, dWo), oh = peel(t, dHo), od = peel(t, dDo), co = peel(t, dCout);
        const T *xn = x + (int64_t)t * xitem;
        y[e] = convT3d_point(xn, w, g, ds, co, od, oh, ow) + (bias ? bias[co] : 0.0f);
    }
}

// KC > 0: window size known at compile time; every tap is loaded from a
// clamped (always valid) address and masked, so that all KC^3 loads are in
// flight together.  KC == 0: run-time k, taps outside the input skipped.
template <int KC, typename T, typename I>
__global__ __launch_bounds__(kThreads)
void avgpool3d_generic_kernel(const T *__restrict__ x, int D, int H, int W, int k, int s,
                              int p, int include_pad, float kvol, Div dWo, Div dHo, Div dDo,
                              I total, T *__restrict__ out)
{
    for (I e = (I)blockIdx.x * kThreads + threadIdx.x; e < total; e += (I)gridDim.x * kThreads) {
        I t = e;
        const int ow = peel(t, dWo), oh = peel(t, dHo), od = peel(t, dDo);
        const T *xs = x + (int64_t)t * D * H * W;
        float sum = 0.0f;
        int cnt = 0;
        if constexpr (KC > 0) {
            int id[KC], ih[KC], iw[KC];
            bool vd[KC], vh[KC], vw[KC];
#pragma unroll
            for (int j = 0; j < KC; ++j) {
                const int d = od * s - p + j, h = oh * s - p + j, w = ow * s - p + j;
                vd[j] = d >= 0 && d < D;
                vh[j] = h >= 0 && h < H;
                vw[j] = w >= 0 && w < W;
                id[j] = vd[j] ? d : 0;
                ih[j] = vh[j] ? h : 0;
                iw[j] = vw[j] ? w : 0;
            }
#pragma unroll
            for (int a = 0; a < KC; ++a)
#pragma unroll
                for (int b = 0; b < KC; ++b)
#pragma unroll
                    for (int c = 0; c < KC; ++c) {
                        const float v = ld(xs, ((int64_t)id[a] * H + ih[b]) * W + iw[c]);
                        const bool in = vd[a] && vh[b] && vw[c];
                        sum += in ? v : 0.0f;
                        cnt += in;
                    }
        } else {
            for (int kd = 0; kd < k; ++kd) {
                const int id = od * s - p + kd;
                if (id < 0 || id >= D) continue;
                for (int kh = 0; kh < k; ++kh) {
                    const int ih = oh * s - p + kh;
                    if (ih < 0 || ih >= H) continue;
                    for (int kw = 0; kw < k; ++kw) {
                        const int iw = ow * s - p + kw;
                        if (iw < 0 || iw >= W) continue;
                        sum += ld(xs, ((int64_t)id * H + ih) * W + iw);
                        ++cnt;
                    }
                }
            }
        }
        st(out, e, sum / (include_pad ? kvol : (float)cnt));
    }
}

template <typename T, typename I>
__global__ __launch_bounds__(kThreads)
void convT1d_generic_kernel(const T *__restrict__ x, const T *__restrict__ w,
                            const float *__restrict__ bias, int Cin, int L, int Cout, int K,
                            int p, int dil, Div dLo, Div dCout, Div ds, I total,
                            float *__restrict__ y)
{
    for (I e = (I)blockIdx.x * kThreads + threadIdx.x; e < total; e += (I)gridDim.x * kThreads) {
        I t = e;
        const int o = peel(t, dLo), co = peel(t, dCout);
        const T *xn = x + (int64_t)t * Cin * L;
        float acc = 0.0f;
        for (int kk = 0; kk < K; ++kk) {
            // input (o + pad - dil*k) / stride when exact and inside [0, L)
            const int tt = o + p - dil * kk;
            if (tt < 0) break;                      // later taps only go lower
            const int i = (int)ds.q((uint32_t)tt);
            if (i * (int)ds.d != tt || i >= L) continue;
            acc = dot_ci(xn, (int64_t)L, (int64_t)i, w, (int64_t)Cout * K, (int64_t)co * K + kk, Cin, acc);
        }
        y[e] = acc + (bias ? bias[co] : 0.0f);
    }
}

// The same sum with a wave per (n, block of 16 output channels, residue r of
// o modulo the stride, 64 consecutive j): lane l computes o = r + s*(64*chunk
// + l) for the block's channels.  Every lane of a wave then has the same valid
// taps (o + p - dil*k is a multiple of s for all of them or for none), a tap's
// inputs are consecutive across the lanes, and each input load feeds 16
// channels.  The weights are staged once per workgroup in LDS as
// [ci][k][co], so a wave reads the same entries on every lane.  Consecutive
// waves take the next channel block, then the next residue, and the workgroup
// order is XCD-aware, so the input segment of a chunk is reused from one L2
// (ordered by output position instead, the large 1D shape re-read its input
// 67 times from HBM).  Sums run in the same order as in
// convT1d_generic_kernel.
template <typename T, typename I>
__global__ __launch_bounds__(kThreads)
void convT1d_residue_kernel(const T *__restrict__ x, const T *__restrict__ w,
                            const float *__restrict__ bias, int Cin, int L, int Cout, int K,
                            int p, int dil, int s, int Lo, Div dCb, Div dS, Div dChunks,
                            I total, float *__restrict__ y)
{
    constexpr int kCB = 16;
    extern __shared__ float wl[];              // [Cin][K][Cout]
    for (int e = threadIdx.x; e < Cin * K * Cout; e += kThreads) {
        const int co = e % Cout, ck = e / Cout;            // ck = ci*K + k
        const int ci = ck / K, kk = ck - ci * K;
        wl[e] = ld(w, ((int64_t)ci * Cout + co) * K + kk);
    }
    __syncthreads();
    // the grid stride is a multiple of 64, so e >> 6 is the same on every
    // lane of a wave and (block, r, chunk) are wave-uniform
    const I b = (I)xcd_remap(blockIdx.x, gridDim.x);
    for (I e = b * kThreads + threadIdx.x; e < total; e += (I)gridDim.x * kThreads) {
        const int lane = (int)(e & 63);
        I t = e >> 6;
        const int cb = __builtin_amdgcn_readfirstlane(peel(t, dCb));
        const int r = __builtin_amdgcn_readfirstlane(peel(t, dS));
        const int ch = __builtin_amdgcn_readfirstlane(peel(t, dChunks));
        const int co0 = cb * kCB;
        const int j = ch * 64 + lane;
        const int64_t o = (int64_t)r + (int64_t)s * j;
        const T *xn = x + (int64_t)t * Cin * L;
        float acc[kCB];
#pragma unroll
        for (int q = 0; q < kCB; ++q) acc[q] = 0.0f;
        for (int kk = 0; kk < K; ++kk) {
            // input (o + p - dil*kk) / s = c0/s + j when c0 = r + p - dil*kk
            // is a multiple of s (the same for every lane; |c0| < 2^31 is
            // checked by the launcher)
            const int c0 = r + p - dil * kk;
            if (c0 % s != 0) continue;
            const int64_t i = (int64_t)(c0 / s) + j;
            if (i < 0 || i >= L) continue;
            // eight channels' loads per wait
            for (int ci0 = 0; ci0 < Cin; ci0 += 8) {
                float xv[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) xv[u] = ld(xn, (int64_t)min(ci0 + u, Cin - 1) * L + i);
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    if (ci0 + u >= Cin) break;             // same for every lane
                    // channels past Cout read the block's first channel (never stored)
                    const float *wr = wl + ((ci0 + u) * K + kk) * Cout;
#pragma unroll
                    for (int q = 0; q < kCB; ++q)
                        acc[q] = __builtin_fmaf(xv[u], wr[co0 + q < Cout ? co0 + q : co0], acc[q]);
                }
            }
        }
        if (o < Lo) {
            float *yo = y + ((int64_t)t * Cout + co0) * Lo + o;
#pragma unroll
            for (int q = 0; q < kCB; ++q)
                if (co0 + q < Cout) yo[(int64_t)q * Lo] = acc[q] + (bias ? bias[co0 + q] : 0.0f);
        }
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

// 32-bit element indices when the grid-stride loop cannot wrap.
bool small_index(int64_t total) { return total < (int64_t(1) << 31); }

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
    const Geo3 g{(int)Cin, (int)D, (int)H, (int)W, (int)Cout, k, s, p, pk, ps};
    const Div dW = make_div((uint32_t)Wp), dH = make_div((uint32_t)Hp), dD = make_div((uint32_t)Dp),
              dC = make_div((uint32_t)Cout), dS = make_div((uint32_t)s);
    const dim3 grid(grid_for(total)), block(kThreads);
    if (k == 3 && s == 2 && p == 1 && pk == 2 && ps == 2 && Cin * Cout <= 1024) {
        const size_t lds = (size_t)Cin * Cout * 8 * sizeof(float);   // <= 32 KB
        // one thread per (n, channel block of 16, pooled voxel)
        const int64_t cblocks = (Cout + 15) / 16;
        const int64_t vtotal = N * cblocks * Dp * Hp * Wp;
        const Div dB = make_div((uint32_t)cblocks);
        const dim3 vgrid(grid_for(vtotal));
#define CT_WEFF(T, I)                                                                           \
        hipLaunchKernelGGL((fused3d_weff_kernel<T, I>), vgrid, block, lds, stream, (const T *)x,    \
                           (const T *)w, conv_bias, bias, s1, s2, g, (int)Dp, (int)Hp, (int)Wp,     \
                           dW, dH, dD, dB, (I)vtotal, out)
        if (bf16 && small_index(vtotal)) CT_WEFF(uint16_t, uint32_t);
        else if (bf16) CT_WEFF(uint16_t, uint64_t);
        else if (small_index(vtotal)) CT_WEFF(float, uint32_t);
        else CT_WEFF(float, uint64_t);
#undef CT_WEFF
        return hipGetLastError();
    }
#define CT_FUSED(T, I)                                                                          \
    hipLaunchKernelGGL((fused3d_generic_kernel<T, I>), grid, block, 0, stream, (const T *)x,    \
                       (const T *)w, conv_bias, bias, s1, s2, inv, g, dW, dH, dD, dC, dS,       \
                       (I)total, out)
    if (bf16 && small_index(total)) CT_FUSED(uint16_t, uint32_t);
    else if (bf16) CT_FUSED(uint16_t, uint64_t);
    else if (small_index(total)) CT_FUSED(float, uint32_t);
    else CT_FUSED(float, uint64_t);
#undef CT_FUSED
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
    const Geo3 g{(int)Cin, (int)D, (int)H, (int)W, (int)Cout, k, s, p, 1, 1};
    const Div dW = make_div((uint32_t)Wo), dH = make_div((uint32_t)Ho), dD = make_div((uint32_t)Do),
              dC = make_div((uint32_t)Cout), dS = make_div((uint32_t)s);
    const dim3 grid(grid_for(total)), block(kThreads);
#define CT_CONV(T, I)                                                                           \
    hipLaunchKernelGGL((convT3d_generic_kernel<T, I>), grid, block, 0, stream, (const T *)x,    \
                       (const T *)w, bias, g, dW, dH, dD, dC, dS, (I)total, y)
    if (bf16 && small_index(total)) CT_CONV(uint16_t, uint32_t);
    else if (bf16) CT_CONV(uint16_t, uint64_t);
    else if (small_index(total)) CT_CONV(float, uint32_t);
    else CT_CONV(float, uint64_t);
#undef CT_CONV
    return hipGetLastError();
}

hipError_t launch_avgpool3d_generic(const void *x, bool bf16, int64_t NC, int64_t D, int64_t H,
                                    int64_t W, int k, int s, int p, int include_pad, void *out,
                                    hipStream_t stream)
{
    const int64_t Do = (D + 2 * p - k) / s + 1, Ho = (H + 2 * p - k) / s + 1,
                  Wo = (W + 2 * p - k) / s + 1;
    const int64_t total = NC * Do * Ho * Wo;
    const Div dW = make_div((uint32_t)Wo), dH = make_div((uint32_t)Ho), dD = make_div((uint32_t)Do);
    const float kvol = (float)k * k * k;
    const dim3 grid(grid_for(total)), block(kThreads);
#define CT_POOL(KC, T, I)                                                                       \
    hipLaunchKernelGGL((avgpool3d_generic_kernel<KC, T, I>), grid, block, 0, stream,             \
                       (const T *)x, (int)D, (int)H, (int)W, k, s, p, include_pad, kvol, dW, dH, \
                       dD, (I)total, (T *)out)
#define CT_POOL_T(T)                                                                            \
    do {                                                                                        \
        if (k == 2 && small) CT_POOL(2, T, uint32_t);                                           \
        else if (k == 3 && small) CT_POOL(3, T, uint32_t);                                      \
        else if (small) CT_POOL(0, T, uint32_t);                                                \
        else CT_POOL(0, T, uint64_t);                                                           \
    } while (0)
    const bool small = small_index(total);
    if (bf16) CT_POOL_T(uint16_t);
    else CT_POOL_T(float);
#undef CT_POOL_T
#undef CT_POOL
    return hipGetLastError();
}

hipError_t launch_convT1d_generic(const void *x, const void *w, bool bf16, const float *bias,
                                  int64_t N, int64_t Cin, int64_t L, int64_t Cout, int K, int s,
                                  int p, int dil, int op, float *y, hipStream_t stream)
{
    const int64_t Lo = (L - 1) * s - 2 * p + (int64_t)dil * (K - 1) + op + 1;
    const dim3 block(kThreads);
    const size_t wbytes = (size_t)Cin * K * Cout * sizeof(float);
    if (s <= 8 && Lo >= 64 * (int64_t)s && p + (int64_t)dil * (K - 1) + s < (int64_t(1) << 31) &&
        wbytes <= 48 * 1024) {
        // waves over (n, chunk of 64 j, residue, block of 16 channels); at
        // most 63 idle lanes per (n, residue, block) with these bounds
        const int64_t chunks = ((Lo + s - 1) / s + 63) / 64;
        const int64_t cblocks = (Cout + 15) / 16;
        const int64_t total = N * chunks * s * cblocks * 64;
        const Div dB = make_div((uint32_t)cblocks), dS = make_div((uint32_t)s),
                  dK = make_div((uint32_t)chunks);
        const dim3 grid(grid_for(total));
#define CT_C1R(T, I)                                                                            \
        hipLaunchKernelGGL((convT1d_residue_kernel<T, I>), grid, block, wbytes, stream,            \
                           (const T *)x, (const T *)w, bias, (int)Cin, (int)L, (int)Cout, K, p,    \
                           dil, s, (int)Lo, dB, dS, dK, (I)total, y)
        if (bf16 && small_index(total)) CT_C1R(uint16_t, uint32_t);
        else if (bf16) CT_C1R(uint16_t, uint64_t);
        else if (small_index(total)) CT_C1R(float, uint32_t);
        else CT_C1R(float, uint64_t);
#undef CT_C1R
        return hipGetLastError();
    }
    const int64_t total = N * Cout * Lo;
    const Div dL = make_div((uint32_t)Lo), dC = make_div((uint32_t)Cout), dS = make_div((uint32_t)s);
    const dim3 grid(grid_for(total));
#define CT_C1D(T, I)                                                                            \
    hipLaunchKernelGGL((convT1d_generic_kernel<T, I>), grid, block, 0, stream, (const T *)x,    \
                       (const T *)w, bias, (int)Cin, (int)L, (int)Cout, K, p, dil, dL, dC, dS,  \
                       (I)total, y)
    if (bf16 && small_index(total)) CT_C1D(uint16_t, uint32_t);
    else if (bf16) CT_C1D(uint16_t, uint64_t);
    else if (small_index(total)) CT_C1D(float, uint32_t);
    else CT_C1D(float, uint64_t);
#undef CT_C1D
    return hipGetLastError();
}

}  // namespace ct
