// avgpool3d.hip - AvgPool3d(k3, s2, p1) with zero padding counted in the
// divisor (27), fp32, streaming each input byte from HBM about once.
//
// Method ([p46] "Kimi-K2.6 l1_p46"): out[d,h,w] is the sum of
// x[2d-1+kd, 2h-1+kh, 2w-1+kw] over kd,kh,kw < 3, out-of-range taps reading 0,
// divided by 27 (passages on padding and count_include_pad).  Each input
// lies in at most 2x2x2 windows (passage on reuse), so a kernel that reads
// every window from memory moves 27/8 times the input; this one reads each
// input row once per pass and forms the window sums in registers.
//
// The 3x3x3 box sum is separable, so it is evaluated as three 3-tap sums:
//   R[p][r][w] = x[p][r][2w-1] + x[p][r][2w] + x[p][r][2w+1]     (along W)
//   V[p][h][w] = R[p][2h-1][w] + R[p][2h][w] + R[p][2h+1][w]      (along H)
//   out[d][h][w] = (V[2d-1][h][w] + V[2d][h][w] + V[2d+1][h][w]) / 27
// A wave owns 4 output rows x 128 output columns of one (n, c) slice and
// walks a range of output planes; the odd input plane 2d+1 is carried in
// registers to the next output plane.
//
// Memory mapping on MI355X:
//  * lane l loads input columns 4l..4l+3 of a row as one 16-byte load (one
//    wave = one contiguous 1 KiB row segment); the column 4l-1 it also needs
//    comes from lane l-1 through a DPP wave shift, not from memory;
//  * per plane a wave loads the 9 input rows 2h0-1 .. 2h0+7 (contiguous in
//    memory), two planes per step, so 18 independent 16-byte loads per lane
//    are in flight.  The 7 rows only this wave reads are loaded
//    non-temporally; the first and last rows, which the neighbouring waves
//    read as well, are plain loads so the second read hits L2.  (Measured on
//    this read/write mix: non-temporal loads and stores together stream
//    faster than either alone.)
//  * 8 waves of a workgroup own 32 consecutive output rows (65 contiguous
//    input rows per plane) and walk 8 output planes; workgroups are remapped
//    so consecutive tiles share one XCD's L2;
//  * each lane stores its 2 outputs as one 8-byte non-temporal store (a wave
//    writes a contiguous 512-byte output row segment).
// Ragged W (not a multiple of 4, or a misaligned slice) takes the same path
// with element-wise masked loads.
#include "ct_internal.h"

namespace ct {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kTH = 4;            // output rows per wave
constexpr int kRows = 2 * kTH + 1; // input rows per plane
constexpr int kTD = 8;            // output planes per task
constexpr int kTW = 128;          // output columns per task (2 per lane)

struct f4 { float x, y, z, w; };
typedef float v2f __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float shr1(float v)
{
    // lane i <- lane i-1 of v; lane 0 <- 0
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x138, 0xf, 0xf, false));
}

template <bool kVec, bool kNT>
__device__ __forceinline__ f4 load_row4(const float *__restrict__ row, int c, int W)
{
    f4 v;
    if (kVec) {
        if (c + 3 < W) {
            const v4f *p = reinterpret_cast<const v4f *>(row + c);
            const v4f t = kNT ? __builtin_nontemporal_load(p) : *p;
            v.x = t.x; v.y = t.y; v.z = t.z; v.w = t.w;
        } else {
            v.x = v.y = v.z = v.w = 0.0f;   // W % 4 == 0: whole vector in or out
        }
    } else {
        v.x = (c + 0 < W) ? row[c + 0] : 0.0f;
        v.y = (c + 1 < W) ? row[c + 1] : 0.0f;
        v.z = (c + 2 < W) ? row[c + 2] : 0.0f;
        v.w = (c + 3 < W) ? row[c + 3] : 0.0f;
    }
    return v;
}

// Vertical 3-row sums of one input plane for the wave's kTH output rows.
// vs[i][0/1] = V[plane][h0+i][2 outputs of this lane].
template <bool kVec>
__device__ __forceinline__ void plane_sums(const float *__restrict__ xs, int plane,
                                           int D, int H, int W, int h0, int c,
                                           int lane, float vs[kTH][2])
{
    f4 v[kRows];
    const bool pok = plane >= 0 && plane < D;
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
        const int row = 2 * h0 - 1 + r;
        // rows 0 and kRows-1 are shared with the neighbouring waves
        if (pok && row >= 0 && row < H)
            v[r] = (r != 0 && r != kRows - 1)
                       ? load_row4<kVec, true>(xs + ((int64_t)plane * H + row) * W, c, W)
                       : load_row4<kVec, false>(xs + ((int64_t)plane * H + row) * W, c, W);
        else
            v[r].x = v[r].y = v[r].z = v[r].w = 0.0f;
    }
    float rs[kRows][2];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
        float left = shr1(v[r].w);
        if (lane == 0 && c > 0) {
            const int row = 2 * h0 - 1 + r;
            left = (pok && row >= 0 && row < H) ? xs[((int64_t)plane * H + row) * W + c - 1] : 0.0f;
        }
        rs[r][0] = left + v[r].x + v[r].y;
        rs[r][1] = v[r].y + v[r].z + v[r].w;
    }
#pragma unroll
    for (int i = 0; i < kTH; ++i) {
        vs[i][0] = rs[2 * i][0] + rs[2 * i + 1][0] + rs[2 * i + 2][0];
        vs[i][1] = rs[2 * i][1] + rs[2 * i + 1][1] + rs[2 * i + 2][1];
    }
}

template <bool kVec>
__global__ __launch_bounds__(kThreads)
void avgpool3d_k3s2p1_kernel(const float *__restrict__ x, float *__restrict__ out,
                             int D, int H, int W, int Do, int Ho, int Wo,
                             int hgroups, int dchunks, int wchunks)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    int64_t t = xcd_remap(blockIdx.x, gridDim.x);
    // tile order (slice, dchunk, wchunk, hgroup): consecutive tiles are
    // vertical neighbours that share a boundary input row.
    const int hg = (int)(t % hgroups); t /= hgroups;
    const int wc = (int)(t % wchunks); t /= wchunks;
    const int dc = (int)(t % dchunks); t /= dchunks;
    const int64_t sl = t;

    const int h0 = (hg * kWaves + wave) * kTH;
    if (h0 >= Ho) return;                       // no barriers in this kernel
    const int d0 = dc * kTD;
    const int d1 = min(d0 + kTD, Do);
    const int c = wc * (2 * kTW) + 4 * lane;    // first input column of this lane
    const int wo = wc * kTW + 2 * lane;         // first output column of this lane

    const float *xs = x + sl * (int64_t)D * H * W;
    float *os = out + sl * (int64_t)Do * Ho * Wo;

    float carry[kTH][2];
    plane_sums<kVec>(xs, 2 * d0 - 1, D, H, W, h0, c, lane, carry);
    const float inv27 = 1.0f / 27.0f;

    for (int d = d0; d < d1; ++d) {
        float va[kTH][2], vb[kTH][2];
        plane_sums<kVec>(xs, 2 * d, D, H, W, h0, c, lane, va);
        plane_sums<kVec>(xs, 2 * d + 1, D, H, W, h0, c, lane, vb);
#pragma unroll
        for (int i = 0; i < kTH; ++i) {
            const int h = h0 + i;
            const float o0 = (carry[i][0] + va[i][0] + vb[i][0]) * inv27;
            const float o1 = (carry[i][1] + va[i][1] + vb[i][1]) * inv27;
            if (h < Ho) {
                float *orow = os + ((int64_t)d * Ho + h) * Wo;
                if (kVec && wo + 1 < Wo) {
                    // Wo even here (W % 4 == 0), so wo is even and 8-byte aligned
                    const v2f pr = {o0, o1};
                    __builtin_nontemporal_store(pr, reinterpret_cast<v2f *>(orow + wo));
                } else {
                    if (wo < Wo) __builtin_nontemporal_store(o0, orow + wo);
                    if (wo + 1 < Wo) __builtin_nontemporal_store(o1, orow + wo + 1);
                }
            }
            carry[i][0] = vb[i][0];
            carry[i][1] = vb[i][1];
        }
    }
}

}  // namespace

hipError_t launch_avgpool3d_k3s2p1(const float *x, int64_t NC, int64_t D,
                                   int64_t H, int64_t W, float *out,
                                   hipStream_t stream)
{
    const int Do = (int)((D - 1) / 2 + 1);
    const int Ho = (int)((H - 1) / 2 + 1);
    const int Wo = (int)((W - 1) / 2 + 1);
    const int hgroups = (Ho + kWaves * kTH - 1) / (kWaves * kTH);
    const int dchunks = (Do + kTD - 1) / kTD;
    const int wchunks = (Wo + kTW - 1) / kTW;
    const int64_t nwg = NC * (int64_t)hgroups * dchunks * wchunks;
    const bool vec = (W % 4 == 0) && ((reinterpret_cast<uintptr_t>(x) & 15) == 0) &&
                     ((reinterpret_cast<uintptr_t>(out) & 7) == 0);
    if (vec)
        hipLaunchKernelGGL(avgpool3d_k3s2p1_kernel<true>, dim3((unsigned)nwg), dim3(kThreads), 0,
                           stream, x, out, (int)D, (int)H, (int)W, Do, Ho, Wo, hgroups,
                           dchunks, wchunks);
    else
        hipLaunchKernelGGL(avgpool3d_k3s2p1_kernel<false>, dim3((unsigned)nwg), dim3(kThreads), 0,
                           stream, x, out, (int)D, (int)H, (int)W, Do, Ho, Wo, hgroups,
                           dchunks, wchunks);
    return hipGetLastError();
}

}  // namespace ct
