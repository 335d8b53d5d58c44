// fused3d_f32.hip - ConvTranspose3d(k3, s2, p1) -> *scale1 -> AvgPool3d(2)
// -> +bias -> *scale2 in one pass, fp32, on the gfx950 fp32 matrix cores.
//
// Method ([p50] "Kimi-K2.6 l2_p50"):
//  * Parity gather (passage on which input/kernel pairs reach each output of
//    a stride-2 transposed conv): pre-pool position 2d takes input d with
//    tap 1; position 2d+1 takes input d with tap 2 and input d+1 with tap 0.
//  * A pooled voxel (d,h,w) averages pre-pool positions {2d,2d+1} x
//    {2h,2h+1} x {2w,2w+1}, so it depends only on the 8 inputs
//    x[ci, d+a, h+b, w+c], a,b,c in {0,1} (passage grouping the 27 terms by
//    input tap), each input offset 0 pairing with taps {1,2} and offset 1
//    with tap {0}.  Pre-summing those weights gives the effective filter
//      Weff[ci,co,(a,b,c)] = sum_{kd in T(a)} sum_{kh in T(b)} sum_{kw in T(c)}
//                            w[ci,co,kd,kh,kw],  T(0) = {1,2}, T(1) = {0},
//    and  S[co,d,h,w] = sum_ci sum_{a,b,c} x[ci,d+a,h+b,w+c] * Weff[ci,co,abc]
//    is the sum of the 8 pre-pool values (27 products per ci, each weight
//    once).  Every tap is in bounds and the pooled size is D-1 (passage on
//    arbitrary input sizes).
//  * Epilogue in the model's order: ((S/8 + conv_bias)*scale1 + bias)*scale2
//    (passage on the epilogue algebra: the conv bias passes through the
//    average unchanged).
//
// MI355X mapping.  S is a dense contraction over kappa = ci*8 + tap
// (K = 8*Cin) for each (co, voxel), so it runs as v_mfma_f32_16x16x4_f32:
//   A (16 x 4)  = Weff^T rows co,      lane l supplies A[l%16][l/16]
//   B (4 x 16)  = X[kappa][voxel],     lane l supplies B[l/16][l%16]
//   D (16 x 16) = S[co][voxel],        lane l holds D[4*(l/16)+r][l%16]
// An M-block is 16 consecutive w of one pooled row (n, d, h); a 16-wide
// block of output channels is blockIdx.y.  Weff^T is built per workgroup in
// LDS in fragment order (conflict-free ds_read_b32).  Lanes 0..15 of each
// store write 16 consecutive w of one channel (64 contiguous bytes).
#include "ct_internal.h"

namespace ct {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kMbPerWave = 2;     // M-blocks each wave computes
constexpr int kChunk = 8;         // k-steps whose loads are issued together

__global__ __launch_bounds__(kThreads)
void fused3d_f32_kernel(const float *__restrict__ x, const float *__restrict__ w,
                        const float *__restrict__ conv_bias,
                        const float *__restrict__ bias, float s1, float s2,
                        int Cin, int D, int H, int W, int Cout,
                        int Dp, int Hp, int Wp, int wblocks, int nmblocks,
                        float *__restrict__ out)
{
    extern __shared__ float wfrag[];          // [ksteps][64]
    const int ksteps = 2 * Cin;               // K = 8*Cin, 4 per MFMA
    const int cob = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;

    // Effective filter, fragment order: wfrag[j][l] = Weff^T[co = l%16][kappa = 4j + l/16].
    for (int e = threadIdx.x; e < ksteps * 64; e += kThreads) {
        const int j = e >> 6, l = e & 63;
        const int co = cob * 16 + (l & 15);
        const int kap = 4 * j + (l >> 4);
        float v = 0.0f;
        if (co < Cout) {
            const int ci = kap >> 3, tap = kap & 7;
            const int a = tap >> 2, b = (tap >> 1) & 1, c = tap & 1;
            const float *wp = w + ((int64_t)ci * Cout + co) * 27;
            // offset 0 -> taps {1,2}; offset 1 -> tap {0}
            const int d0 = a ? 0 : 1, d1 = a ? 0 : 2;
            const int h0 = b ? 0 : 1, h1 = b ? 0 : 2;
            const int w0 = c ? 0 : 1, w1 = c ? 0 : 2;
            for (int kd = d0; kd <= d1; ++kd)
                for (int kh = h0; kh <= h1; ++kh)
                    for (int kw = w0; kw <= w1; ++kw)
                        v += wp[kd * 9 + kh * 3 + kw];
        }
        wfrag[e] = v;
    }
    __syncthreads();

    const int col = lane & 15;   // voxel (w offset) inside the M-block
    const int kq = lane >> 4;    // kappa offset inside a k-step / co group in D
    const int64_t HW = (int64_t)H * W;
    const int64_t DHW = (int64_t)D * HW;
    const int64_t pplane = (int64_t)Dp * Hp * Wp;

    // Per-lane epilogue constants for co = cob*16 + 4*kq + r.
    float cbv[4], bv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int co = cob * 16 + 4 * kq + r;
        cbv[r] = (conv_bias && co < Cout) ? conv_bias[co] : 0.0f;
        bv[r] = (bias && co < Cout) ? bias[co] : 0.0f;
    }

    const int64_t wg = xcd_remap(blockIdx.x, gridDim.x);
    const int mb0 = (int)((wg * kWaves + wave) * kMbPerWave);

#pragma unroll
    for (int m = 0; m < kMbPerWave; ++m) {
        const int mb = mb0 + m;
        if (mb >= nmblocks) break;                    // wave-uniform
        const int wb = mb % wblocks;
        int t = mb / wblocks;
        const int h = t % Hp;
        t /= Hp;
        const int d = t % Dp;
        const int n = t / Dp;
        const int wv = wb * 16 + col;
        const bool valid = wv < Wp;
        const float *xn = x + (int64_t)n * Cin * DHW + (int64_t)d * HW + (int64_t)h * W + wv;

        v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int j0 = 0; j0 < ksteps; j0 += kChunk) {
            float xv[kChunk];
#pragma unroll
            for (int jj = 0; jj < kChunk; ++jj) {
                const int kap = 4 * (j0 + jj) + kq;
                const int ci = kap >> 3, tap = kap & 7;
                const int a = tap >> 2, b = (tap >> 1) & 1, c = tap & 1;
                xv[jj] = (valid && j0 + jj < ksteps)
                    ? xn[(int64_t)ci * DHW + a * HW + b * W + c] : 0.0f;
            }
#pragma unroll
            for (int jj = 0; jj < kChunk; ++jj) {
                if (j0 + jj < ksteps)
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(
                        wfrag[(j0 + jj) * 64 + lane], xv[jj], acc, 0, 0, 0);
            }
        }

        if (valid) {
            float *on = out + (int64_t)n * Cout * pplane + ((int64_t)d * Hp + h) * Wp + wv;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int co = cob * 16 + 4 * kq + r;
                if (co < Cout) {
                    float v = acc[r] * 0.125f;
                    v = (v + cbv[r]) * s1;
                    v = (v + bv[r]) * s2;
                    on[(int64_t)co * pplane] = v;   // plain store: L2 merges the partial lines
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_fused3d_f32(const float *x, const float *w,
                              const float *conv_bias, const float *bias,
                              float s1, float s2, int64_t N, int64_t Cin,
                              int64_t D, int64_t H, int64_t W, int64_t Cout,
                              float *out, hipStream_t stream)
{
    const int Dp = (int)(D - 1), Hp = (int)(H - 1), Wp = (int)(W - 1);
    const int wblocks = (Wp + 15) / 16;
    const int64_t nmb = N * Dp * (int64_t)Hp * wblocks;   // < 2^31 (checked by the shim)
    const int64_t per_wg = (int64_t)kWaves * kMbPerWave;
    const unsigned gx = (unsigned)((nmb + per_wg - 1) / per_wg);
    const unsigned gy = (unsigned)((Cout + 15) / 16);
    const size_t lds = (size_t)(2 * Cin) * 64 * sizeof(float);
    hipLaunchKernelGGL(fused3d_f32_kernel, dim3(gx, gy), dim3(kThreads), lds, stream,
                       x, w, conv_bias, bias, s1, s2, (int)Cin, (int)D, (int)H, (int)W,
                       (int)Cout, Dp, Hp, Wp, wblocks, (int)nmb, out);
    return hipGetLastError();
}

}  // namespace ct
