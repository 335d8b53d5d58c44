// avgpool3d.hip - AvgPool3d(k3, s2, p1) with zero padding counted in the
// divisor (27), fp32, streaming each input byte from HBM about once.
//
// Method ([p46] "Kimi-K2.6 l1_p46"): out[d,h,w] is the sum of
// x[2d-1+kd, 2h-1+kh, 2w-1+kw] over kd,kh,kw < 3, out-of-range taps reading 0,
// divided by 27 (passages on padding and count_include_pad).  Each input
// lies in at most 2x2x2 windows (passage on reuse), so a kernel that reads
// every window from memory moves 27/8 times the input; these kernels read
// each input row once per pass and form the window sums in registers.
//
// The 3x3x3 box sum is separable, so it is evaluated as three 3-tap sums:
//   R[p][r][w] = x[p][r][2w-1] + x[p][r][2w] + x[p][r][2w+1]     (along W)
//   V[p][h][w] = R[p][2h-1][w] + R[p][2h][w] + R[p][2h+1][w]      (along H)
//   out[d][h][w] = (V[2d-1][h][w] + V[2d][h][w] + V[2d+1][h][w]) / 27
// A wave owns 4 output rows x 128 output columns of one (n, c) slice and
// walks a range of output planes; the odd input plane 2d+1 is carried in
// registers (as V) to the next output plane.
//
// Vector kernel (W a multiple of 4, 16-byte aligned x), memory mapping on MI355X:
//  * a workgroup of 16 waves owns 64 output rows x 128 output columns of a
//    slice, i.e. 128 consecutive input rows of every plane: per output plane
//    it reads input planes 2d and 2d+1 as one contiguous 256 KiB run (for
//    W = 256), each wave loading only its own 8 rows, 16 independent 16-byte
//    loads per lane in flight.  Long contiguous runs per workgroup measured
//    faster on HBM than the same bytes read as several shorter runs.
//  * the row above a wave's first row belongs to the previous wave: that
//    row's horizontal sums are passed through LDS (one barrier per output
//    plane), not read from memory again;
//  * loads and stores are buffer instructions with a fixed count: rows,
//    planes and lanes outside the tensor get an offset past the buffer's
//    range, which reads 0 and writes nothing, so the loop body has no branch
//    around a memory instruction and the memory counter waits stay exact;
//  * lane l loads input columns 4l..4l+3 of a row (one wave = one 1 KiB row
//    segment); the column 4l-1 comes from lane l-1 through a DPP wave shift;
//  * a workgroup walks as many output planes as keeps two workgroups per CU,
//    so that for the large case every slice is read by one workgroup from
//    its first plane to its last and no plane is read twice.
// Other inputs (ragged W, misaligned x) take the element kernel: one wave per
// 4 output rows, element-wise masked loads, same arithmetic.
#include "ct_internal.h"

namespace ct {
namespace {

constexpr int kTH = 4;             // output rows per wave
constexpr int kTW = 128;           // output columns per wave row (2 per lane)

typedef float v2f __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float shr1(float v)
{
    // lane i <- lane i-1 of v; lane 0 <- 0
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x138, 0xf, 0xf, false));
}

// ------------------------------------------------------------ vector kernel --
constexpr int kVWaves = 16;                  // waves per workgroup
constexpr int kVThreads = 64 * kVWaves;
constexpr int kOwn = 2 * kTH;                // input rows a wave owns per plane
constexpr int kGroupRows = kVWaves * kTH;    // output rows per workgroup
constexpr unsigned kOOB = 0x40000000u;       // past every buffer (planes < 2^30 bytes)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t plane_rsrc(const float *base, bool valid, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, 0, valid ? bytes : 0, 0x00020000);
}

// Own rows of one plane: 16-byte loads, plus (kWide) the column left of the
// wave's first column, which only lane 0 needs: lane r loads it for row r.
struct Rows {
    v4f v[kOwn];
    float lf;
};

template <bool kWide>
__device__ __forceinline__ void load_rows(Rows &R, __amdgpu_buffer_rsrc_t rs, int row0, int H, int W,
                                          int lane, unsigned laneoff, int c0w)
{
#pragma unroll
    for (int r = 0; r < kOwn; ++r) {
        const int row = row0 + r;
        const unsigned roff = row < H ? (unsigned)(row * W * 4) : kOOB;
        R.v[r] = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(roff + laneoff), 0, 2));
    }
    if (kWide) {
        const int row = row0 + lane;
        const unsigned loff = (lane < kOwn && row < H && c0w > 0)
                                  ? (unsigned)((row * W + c0w - 1) * 4) : kOOB;
        R.lf = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (int)loff, 0, 0));
    }
}

// Horizontal 3-tap sums of a row held as one float4 per lane; lf is the
// column left of lane 0's first column (used by lane 0 only).
template <bool kWide>
__device__ __forceinline__ v2f hsum(v4f v, float lf, int lane)
{
    float left = shr1(v.w);
    if (kWide && lane == 0) left += lf;
    return v2f{left + v.x + v.y, v.y + v.z + v.w};
}

// One output plane's worth of input: planes pa and pb (pb may be out of
// range), vertical sums of both for the wave's kTH output rows.  xs is the
// slice, lds[2 planes][waves][64] the exchange buffer of this step.
template <bool kWide>
__device__ __forceinline__ void plane_pair(const float *xs, int pa, int pb, int D, int H, int W,
                                           int rowbase, int wave, int lane, unsigned laneoff,
                                           int c0w, v2f *lds, float va[kTH][2], float vb[kTH][2])
{
    const int pbytes = H * W * 4;
    const bool oka = pa >= 0 && pa < D, okb = pb >= 0 && pb < D;
    const __amdgpu_buffer_rsrc_t ra = plane_rsrc(xs + (int64_t)(oka ? pa : 0) * H * W, oka, pbytes);
    const __amdgpu_buffer_rsrc_t rb = plane_rsrc(xs + (int64_t)(okb ? pb : 0) * H * W, okb, pbytes);
    const int row0 = rowbase + wave * kOwn;
    Rows A, B;
    load_rows<kWide>(A, ra, row0, H, W, lane, laneoff, c0w);
    load_rows<kWide>(B, rb, row0, H, W, lane, laneoff, c0w);

    v2f sa[kOwn + 1], sb[kOwn + 1];   // index 0: the row above the wave's first row
#pragma unroll
    for (int r = 0; r < kOwn; ++r) {
        const int la = kWide ? __builtin_amdgcn_readlane(__float_as_int(A.lf), r) : 0;
        const int lb = kWide ? __builtin_amdgcn_readlane(__float_as_int(B.lf), r) : 0;
        sa[r + 1] = hsum<kWide>(A.v[r], __int_as_float(la), lane);
        sb[r + 1] = hsum<kWide>(B.v[r], __int_as_float(lb), lane);
    }
    lds[wave * 64 + lane] = sa[kOwn];
    lds[(kVWaves + wave) * 64 + lane] = sb[kOwn];
    __syncthreads();
    if (wave > 0) {
        sa[0] = lds[(wave - 1) * 64 + lane];
        sb[0] = lds[(kVWaves + wave - 1) * 64 + lane];
    } else if (rowbase > 0) {
        // the row above belongs to the workgroup of the previous row group
        const unsigned roff = (unsigned)((rowbase - 1) * W * 4);
        const unsigned loff = (kWide && lane == 0 && c0w > 0) ? roff + (unsigned)((c0w - 1) * 4) : kOOB;
        const v4f a = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(ra, (int)(roff + laneoff), 0, 0));
        const v4f b = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(rb, (int)(roff + laneoff), 0, 0));
        float la = 0.0f, lb = 0.0f;
        if (kWide) {
            la = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ra, (int)loff, 0, 0));
            lb = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rb, (int)loff, 0, 0));
        }
        sa[0] = hsum<kWide>(a, la, lane);
        sb[0] = hsum<kWide>(b, lb, lane);
    } else {
        sa[0] = sb[0] = v2f{0.0f, 0.0f};   // row -1: padding
    }
#pragma unroll
    for (int i = 0; i < kTH; ++i) {
        const v2f a = sa[2 * i] + sa[2 * i + 1] + sa[2 * i + 2];
        const v2f b = sb[2 * i] + sb[2 * i + 1] + sb[2 * i + 2];
        va[i][0] = a.x; va[i][1] = a.y;
        vb[i][0] = b.x; vb[i][1] = b.y;
    }
}

// Grid: one workgroup per (slice, plane chunk of td output planes, column
// chunk, row group of kGroupRows output rows), row groups fastest.
template <bool kWide>
__global__ __launch_bounds__(kVThreads)
void avgpool3d_k3s2p1_vec_kernel(const float *__restrict__ x, float *__restrict__ out,
                                 int D, int H, int W, int Do, int Ho, int Wo,
                                 int hgroups, int dchunks, int wchunks, int td)
{
    __shared__ v2f lds[2][2 * kVWaves * 64];   // double-buffered by step
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int64_t t = xcd_remap(blockIdx.x, gridDim.x);
    const int hg = (int)(t % hgroups); t /= hgroups;
    const int wc = (int)(t % wchunks); t /= wchunks;
    const int dc = (int)(t % dchunks); t /= dchunks;
    const int64_t sl = t;

    const int rowbase = 2 * hg * kGroupRows;      // first input row of the workgroup
    const int h0 = hg * kGroupRows + wave * kTH;  // first output row of the wave
    const int d0 = dc * td;
    const int d1 = min(d0 + td, Do);
    const int c0w = wc * (2 * kTW);
    const int c = c0w + 4 * lane;
    const int wo = wc * kTW + 2 * lane;
    const unsigned laneoff = c < W ? (unsigned)(c * 4) : kOOB;

    const float *xs = x + sl * (int64_t)D * H * W;
    float *os = out + sl * (int64_t)Do * Ho * Wo;
    const int obytes = Ho * Wo * 4;

    float carry[kTH][2], vb[kTH][2];
    plane_pair<kWide>(xs, 2 * d0 - 1, -1, D, H, W, rowbase, wave, lane, laneoff, c0w, lds[0],
                      carry, vb);
    const float inv27 = 1.0f / 27.0f;
    for (int d = d0; d < d1; ++d) {
        float va[kTH][2];
        plane_pair<kWide>(xs, 2 * d, 2 * d + 1, D, H, W, rowbase, wave, lane, laneoff, c0w,
                          lds[(d - d0 + 1) & 1], va, vb);
        const __amdgpu_buffer_rsrc_t ro = plane_rsrc(os + (int64_t)d * Ho * Wo, true, obytes);
#pragma unroll
        for (int i = 0; i < kTH; ++i) {
            const int h = h0 + i;
            const v2f o = {(carry[i][0] + va[i][0] + vb[i][0]) * inv27,
                           (carry[i][1] + va[i][1] + vb[i][1]) * inv27};
            // Wo is even here (W % 4 == 0), so wo < Wo covers the pair
            const unsigned off = (h < Ho && wo < Wo) ? (unsigned)((h * Wo + wo) * 4) : kOOB;
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2i, o), ro, (int)off, 0, 2);
            carry[i][0] = vb[i][0];
            carry[i][1] = vb[i][1];
        }
    }
}

// ----------------------------------------------------------- element kernel --
constexpr int kEWaves = 8;
constexpr int kEThreads = 64 * kEWaves;
constexpr int kERows = 2 * kTH + 1;   // input rows per plane, halo included
constexpr int kETD = 8;               // output planes per workgroup

// Vertical 3-row sums of one input plane for the wave's kTH output rows,
// element-wise masked loads.  vs[i][0/1] = V[plane][h0+i][2 outputs of this lane].
__device__ __forceinline__ void plane_sums_elem(const float *__restrict__ xs, int plane, int D,
                                                int H, int W, int h0, int c, int lane,
                                                float vs[kTH][2])
{
    float rs[kERows][2];
    const bool pok = plane >= 0 && plane < D;
#pragma unroll
    for (int r = 0; r < kERows; ++r) {
        const int row = 2 * h0 - 1 + r;
        float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        float left = 0.0f;
        if (pok && row >= 0 && row < H) {
            const float *rp = xs + ((int64_t)plane * H + row) * W;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (c + j < W) v[j] = rp[c + j];
            if (lane == 0 && c > 0) left = rp[c - 1];
        }
        left += shr1(v[3]);
        rs[r][0] = left + v[0] + v[1];
        rs[r][1] = v[1] + v[2] + v[3];
    }
#pragma unroll
    for (int i = 0; i < kTH; ++i) {
        vs[i][0] = rs[2 * i][0] + rs[2 * i + 1][0] + rs[2 * i + 2][0];
        vs[i][1] = rs[2 * i][1] + rs[2 * i + 1][1] + rs[2 * i + 2][1];
    }
}

__global__ __launch_bounds__(kEThreads)
void avgpool3d_k3s2p1_elem_kernel(const float *__restrict__ x, float *__restrict__ out,
                                  int D, int H, int W, int Do, int Ho, int Wo,
                                  int hgroups, int dchunks, int wchunks)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    int64_t t = xcd_remap(blockIdx.x, gridDim.x);
    const int hg = (int)(t % hgroups); t /= hgroups;
    const int wc = (int)(t % wchunks); t /= wchunks;
    const int dc = (int)(t % dchunks); t /= dchunks;
    const int64_t sl = t;

    const int h0 = (hg * kEWaves + wave) * kTH;
    if (h0 >= Ho) return;                       // no barriers in this kernel
    const int d0 = dc * kETD;
    const int d1 = min(d0 + kETD, Do);
    const int c = wc * (2 * kTW) + 4 * lane;    // first input column of this lane
    const int wo = wc * kTW + 2 * lane;         // first output column of this lane

    const float *xs = x + sl * (int64_t)D * H * W;
    float *os = out + sl * (int64_t)Do * Ho * Wo;

    float carry[kTH][2];
    plane_sums_elem(xs, 2 * d0 - 1, D, H, W, h0, c, lane, carry);
    const float inv27 = 1.0f / 27.0f;
    for (int d = d0; d < d1; ++d) {
        float va[kTH][2], vb[kTH][2];
        plane_sums_elem(xs, 2 * d, D, H, W, h0, c, lane, va);
        plane_sums_elem(xs, 2 * d + 1, D, H, W, h0, c, lane, vb);
#pragma unroll
        for (int i = 0; i < kTH; ++i) {
            const int h = h0 + i;
            const float o0 = (carry[i][0] + va[i][0] + vb[i][0]) * inv27;
            const float o1 = (carry[i][1] + va[i][1] + vb[i][1]) * inv27;
            if (h < Ho) {
                float *orow = os + ((int64_t)d * Ho + h) * Wo;
                if (wo < Wo) __builtin_nontemporal_store(o0, orow + wo);
                if (wo + 1 < Wo) __builtin_nontemporal_store(o1, orow + wo + 1);
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
    const int wchunks = (Wo + kTW - 1) / kTW;
    const bool vec = (W % 4 == 0) && ((reinterpret_cast<uintptr_t>(x) & 15) == 0) &&
                     ((reinterpret_cast<uintptr_t>(out) & 7) == 0) && H * W * 4 < (int64_t)kOOB;
    if (vec) {
        const int hgroups = (Ho + kGroupRows - 1) / kGroupRows;
        // as few plane chunks as still give every CU two workgroups
        int cus = 256, dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            cus = 256;
        const int64_t base = NC * hgroups * wchunks;
        int64_t dchunks = (2 * (int64_t)cus + base - 1) / base;
        if (dchunks > Do) dchunks = Do;
        const int td = (int)((Do + dchunks - 1) / dchunks);
        dchunks = (Do + td - 1) / td;
        const int64_t nwg = base * dchunks;
        if (wchunks > 1)
            hipLaunchKernelGGL(avgpool3d_k3s2p1_vec_kernel<true>, dim3((unsigned)nwg),
                               dim3(kVThreads), 0, stream, x, out, (int)D, (int)H, (int)W, Do,
                               Ho, Wo, hgroups, (int)dchunks, wchunks, td);
        else
            hipLaunchKernelGGL(avgpool3d_k3s2p1_vec_kernel<false>, dim3((unsigned)nwg),
                               dim3(kVThreads), 0, stream, x, out, (int)D, (int)H, (int)W, Do,
                               Ho, Wo, hgroups, (int)dchunks, wchunks, td);
    } else {
        const int hgroups = (Ho + kEWaves * kTH - 1) / (kEWaves * kTH);
        const int dchunks = (Do + kETD - 1) / kETD;
        const int64_t nwg = NC * (int64_t)hgroups * dchunks * wchunks;
        hipLaunchKernelGGL(avgpool3d_k3s2p1_elem_kernel, dim3((unsigned)nwg), dim3(kEThreads), 0,
                           stream, x, out, (int)D, (int)H, (int)W, Do, Ho, Wo, hgroups, dchunks,
                           wchunks);
    }
    return hipGetLastError();
}

}  // namespace ct
