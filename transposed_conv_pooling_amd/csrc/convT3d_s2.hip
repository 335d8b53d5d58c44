// convT3d_s2.hip - ConvTranspose3d(k3, stride 2, pad 1), output_padding 0 or
// 1, materialising its output: the first layer of the [p50] model on its own,
// as the unfused chain runs it.
//
// Parity rule ([p50], passages on which kernel taps reach an output under
// stride 2): along one axis, even output 2m takes only tap 1 from input m;
// odd output 2m + 1 takes tap 0 from input m + 1 and tap 2 from input m.  So
// the 2x2x2 output block at (2md, 2mh, 2mw) depends only on the 2x2x2 input
// block at (md, mh, mw), and per input channel its 8 outputs use each of the
// 27 weights exactly once (27 FMAs per channel and block).
//
// One thread per input block (lanes along w), so its 8 * Cin input loads
// coalesce and, per output channel, 27 FMAs per input channel produce all 8
// outputs with no wasted term.  A lane's 8 outputs form 4 pairs of adjacent
// columns; written directly, each store instruction would touch every other
// float of a 512-byte span.  Instead the wave stages each pair row in a
// wave-private 512-byte LDS row (lane l at columns 2l, 2l + 1) and reads it
// back so that lane l stores the l-th and (64 + l)-th floats: each store
// instruction then writes consecutive floats of one output row segment.  The
// output address and validity of the pair each lane stores are decoded once,
// before the output-channel loop.  With output_padding 0 the last block's odd
// outputs fall outside and are skipped.
#include "ct_internal.h"

namespace ct {
namespace {

constexpr int kThreads = 256;

template <typename T> __device__ __forceinline__ float ldf(const T *p, int64_t i);
template <> __device__ __forceinline__ float ldf<float>(const float *p, int64_t i) { return p[i]; }
template <> __device__ __forceinline__ float ldf<uint16_t>(const uint16_t *p, int64_t i)
{
    return __uint_as_float(((unsigned)p[i]) << 16);   // bf16 -> fp32, exact
}

constexpr int kWaves = kThreads / 64;

// Output offset of the first (even, even, even) output of input block b, and
// which of its odd d / h / w outputs exist.
struct BlockOut {
    int64_t off;
    bool d1, h1, w1;
};

__device__ __forceinline__ BlockOut block_out(int64_t b, int D, int H, int W, int Cout, int Do,
                                              int Ho, int Wo)
{
    const int mw = (int)(b % W);
    b /= W;
    const int mh = (int)(b % H);
    b /= H;
    const int md = (int)(b % D);
    const int64_t n = b / D;
    return {n * Cout * ((int64_t)Do * Ho * Wo) + ((int64_t)(2 * md) * Ho + 2 * mh) * Wo + 2 * mw,
            2 * md + 1 < Do, 2 * mh + 1 < Ho, 2 * mw + 1 < Wo};
}

template <typename T, int CIN>
__global__ __launch_bounds__(kThreads)
void convT3d_s2_kernel(const T *__restrict__ x, const T *__restrict__ w,
                       const float *__restrict__ bias, int D, int H, int W, int Cout, int Do,
                       int Ho, int Wo, int64_t nblocks, float *__restrict__ y)
{
    __shared__ float stage[kWaves][4][128];      // per wave: 4 pair rows of 64 lanes
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // XCD-aware: each XCD takes one contiguous range of workgroups, so the
    // partly written 128-byte lines at the seams between neighbouring
    // workgroups' output rows meet in one L2
    const int64_t wbase = xcd_remap(blockIdx.x, gridDim.x) * kThreads + wave * 64;
    if (wbase >= nblocks) return;                // whole wave idle
    const int64_t bown = wbase + lane < nblocks ? wbase + lane : nblocks - 1;   // clamped

    // this lane's own input block
    int64_t t = bown;
    const int mw = (int)(t % W); t /= W;
    const int mh = (int)(t % H); t /= H;
    const int md = (int)(t % D);
    const int64_t n = t / D;
    const int64_t HW = (int64_t)H * W, DHW = (int64_t)D * HW;
    const bool vd = md + 1 < D, vh = mh + 1 < H, vw = mw + 1 < W;
    const int64_t o000 = (int64_t)md * HW + (int64_t)mh * W + mw;
    const int64_t sd = vd ? HW : 0, sh = vh ? W : 0, sw = vw ? 1 : 0;   // clamped steps
    float xv[CIN][2][2][2];
    const T *xn = x + n * CIN * DHW;
#pragma unroll
    for (int ci = 0; ci < CIN; ++ci)
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    // unconditional loads from clamped (always valid)
                    // addresses, masked afterwards
                    const float v = ldf(xn, ci * DHW + o000 + a * sd + c * sh + e * sw);
                    const bool in = (!a || vd) && (!c || vh) && (!e || vw);
                    xv[ci][a][c][e] = in ? v : 0.0f;
                }

    // the two output pairs this lane stores: column (lane & 1) of the pairs of
    // lanes lane/2 and 32 + lane/2
    const int par = lane & 1;
    const int64_t bA = wbase + (lane >> 1), bB = wbase + 32 + (lane >> 1);
    const bool okA = bA < nblocks, okB = bB < nblocks;
    const BlockOut A = block_out(okA ? bA : bown, D, H, W, Cout, Do, Ho, Wo);
    const BlockOut B = block_out(okB ? bB : bown, D, H, W, Cout, Do, Ho, Wo);
    const bool colA = okA && (!par || A.w1), colB = okB && (!par || B.w1);
    const int64_t ostride_c = (int64_t)Do * Ho * Wo;
    float *yA = y + A.off + par, *yB = y + B.off + par;
    float(*st)[128] = stage[wave];

    for (int co = 0; co < Cout; ++co) {
        float acc[2][2][2] = {};
#pragma unroll
        for (int ci = 0; ci < CIN; ++ci) {
            const T *wc = w + ((int64_t)ci * Cout + co) * 27;
            // per axis: parity 0 <- (tap 1, offset 0); parity 1 <- (tap 0,
            // offset 1) and (tap 2, offset 0)
#pragma unroll
            for (int kd = 0; kd < 3; ++kd)
#pragma unroll
                for (int kh = 0; kh < 3; ++kh)
#pragma unroll
                    for (int kw = 0; kw < 3; ++kw) {
                        const float wv = ldf(wc, kd * 9 + kh * 3 + kw);
                        const int rd = kd != 1, rh = kh != 1, rw = kw != 1;
                        const int ad = kd == 0, ah = kh == 0, aw = kw == 0;
                        acc[rd][rh][rw] = __builtin_fmaf(xv[ci][ad][ah][aw], wv, acc[rd][rh][rw]);
                    }
        }
        const float bv = bias ? bias[co] : 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            st[r][2 * lane] = acc[r >> 1][r & 1][0] + bv;
            st[r][2 * lane + 1] = acc[r >> 1][r & 1][1] + bv;
        }
        __builtin_amdgcn_wave_barrier();
        const int64_t oc = co * ostride_c;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int rd = r >> 1, rh = r & 1;
            const float va = st[r][lane], vb = st[r][64 + lane];
            const int64_t ro = oc + ((int64_t)rd * Ho + rh) * Wo;
            if (colA && (!rd || A.d1) && (!rh || A.h1)) yA[ro] = va;
            if (colB && (!rd || B.d1) && (!rh || B.h1)) yB[ro] = vb;
        }
        __builtin_amdgcn_wave_barrier();
    }
}

template <typename T>
hipError_t launch_t(const T *x, const T *w, const float *bias, int64_t N, int64_t Cin, int64_t D,
                    int64_t H, int64_t W, int64_t Cout, int op, float *y, hipStream_t stream)
{
    const int64_t Do = 2 * D - 1 + op, Ho = 2 * H - 1 + op, Wo = 2 * W - 1 + op;
    const int64_t nblocks = N * D * H * W;
    const dim3 grid((unsigned)((nblocks + kThreads - 1) / kThreads)), block(kThreads);
#define CT_S2(C)                                                                                \
    case C:                                                                                     \
        hipLaunchKernelGGL((convT3d_s2_kernel<T, C>), grid, block, 0, stream, x, w, bias,      \
                           (int)D, (int)H, (int)W, (int)Cout, (int)Do, (int)Ho, (int)Wo,        \
                           nblocks, y);                                                         \
        break;
    switch (Cin) {
        CT_S2(1) CT_S2(2) CT_S2(3) CT_S2(4) CT_S2(5) CT_S2(6) CT_S2(7) CT_S2(8)
    default: return hipErrorInvalidValue;
    }
#undef CT_S2
    return hipGetLastError();
}

}  // namespace

hipError_t launch_convT3d_s2(const void *x, const void *w, bool bf16, const float *bias,
                             int64_t N, int64_t Cin, int64_t D, int64_t H, int64_t W,
                             int64_t Cout, int op, float *y, hipStream_t stream)
{
    if (bf16)
        return launch_t((const uint16_t *)x, (const uint16_t *)w, bias, N, Cin, D, H, W, Cout, op,
                        y, stream);
    return launch_t((const float *)x, (const float *)w, bias, N, Cin, D, H, W, Cout, op, y,
                    stream);
}

}  // namespace ct
