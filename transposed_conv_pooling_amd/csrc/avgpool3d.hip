// avgpool3d.hip - AvgPool3d(k3, s2, p1) with zero padding counted in the
// divisor (27) or, with count_include_pad off, a divisor of the window taps
// inside the input, streaming each input byte from HBM about once.  fp32
// data, or bf16 data with fp32 sums and each mean rounded to the nearest bf16.
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
//    slice, i.e. 128 consecutive input rows of every plane, and walks a range
//    of output planes;
//  * wave w loads rows w, w+16, w+32, ... of the workgroup's 128: one load
//    instruction across the 16 waves covers 16 consecutive rows, so the
//    requests of a workgroup reach HBM in address order (measured ~7% faster
//    than each wave loading its own 8 consecutive rows);
//  * each wave turns its rows into horizontal sums and writes them to an
//    LDS table of the workgroup's 128 rows; after a barrier it reads back
//    the 9 rows of its 4 output rows (the table is double-buffered by
//    plane, so one barrier per plane suffices);
//  * the next-but-one plane's loads are issued as soon as a plane's rows are
//    in the table, so two planes of loads (16 per lane) stay in flight while
//    the table is read and the outputs are formed;
//  * loads and stores are buffer instructions with a fixed count: rows,
//    planes and lanes outside the tensor get an offset past the buffer's
//    range, which reads 0 and writes nothing, so the loop body has no branch
//    around a memory instruction and the memory counter waits stay exact;
//  * lane l loads input columns 4l..4l+3 of a row (one wave = one 1 KiB row
//    segment); the column 4l-1 comes from lane l-1 through a DPP wave shift;
//  * a workgroup walks as many output planes as keeps two workgroups per CU,
//    so that for the large case every slice is read by one workgroup from
//    its first plane to its last and no plane is read twice (fp32); bf16
//    workgroups start at staggered plane offsets and wrap around, so that
//    the workgroups running together stream different offsets of their
//    slices, at the cost of one plane read twice.
// Planes of at most 4096 elements (a 64 x 64 plane, or 8 x 512) take the
// small-plane kernel below instead, which fills its workgroups with several
// slices.  Other inputs (ragged W, misaligned x or out, planes of 2^30 bytes
// or more) take the element kernel: one wave per 4 output rows,
// element-wise masked loads, same arithmetic.
#include <algorithm>

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

// Element type of the pooled tensor: fp32, or bf16 carried as its 16-bit
// pattern (widened exactly to fp32 for the sums; the mean is rounded to the
// nearest bf16, ties to even, by the hardware conversion).
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
template <typename E> struct Elem;
template <> struct Elem<float> {
    typedef v4f raw4;                        // 4 consecutive elements as loaded
    template <int kAux>
    static __device__ __forceinline__ raw4 load4(__amdgpu_buffer_rsrc_t r, unsigned off)
    {
        return __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kAux));
    }
    static __device__ __forceinline__ v4f widen(raw4 v) { return v; }
    static __device__ __forceinline__ float load1(__amdgpu_buffer_rsrc_t r, unsigned off)
    {
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
    }
    static __device__ __forceinline__ void store2(__amdgpu_buffer_rsrc_t r, unsigned off, int soff, float a, float b)
    {
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(v2i, v2f{a, b}), r, (int)off, soff, 2);
    }
    static __device__ __forceinline__ float to_f32(float v) { return v; }
    static __device__ __forceinline__ float from_f32(float v) { return v; }
};
template <> struct Elem<uint16_t> {
    typedef u32x2 raw4;                      // 4 bf16 in two dwords
    template <int kAux>
    static __device__ __forceinline__ raw4 load4(__amdgpu_buffer_rsrc_t r, unsigned off)
    {
        return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kAux);
    }
    static __device__ __forceinline__ v4f widen(raw4 v)
    {
        return v4f{__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                   __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u)};
    }
    static __device__ __forceinline__ float load1(__amdgpu_buffer_rsrc_t r, unsigned off)
    {
        return __uint_as_float((unsigned)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0) << 16);
    }
    static __device__ __forceinline__ uint16_t from_f32(float v) { return __builtin_bit_cast(uint16_t, (__bf16)v); }
    static __device__ __forceinline__ void store2(__amdgpu_buffer_rsrc_t r, unsigned off, int soff, float a, float b)
    {
        const unsigned u = (unsigned)from_f32(a) | ((unsigned)from_f32(b) << 16);
        __builtin_amdgcn_raw_buffer_store_b32(u, r, (int)off, soff, 2);
    }
    static __device__ __forceinline__ float to_f32(uint16_t v) { return __uint_as_float((unsigned)v << 16); }
};

// Taps of output q's window 2q-1 .. 2q+1 inside an axis of length n (1..3);
// with count_include_pad=False the mean divides by the product over the axes.
__device__ __forceinline__ int taps3(int q, int n) { return 3 - (q == 0) - (2 * q + 1 >= n); }

// ------------------------------------------------------------ vector kernel --
constexpr int kVWaves = 16;                  // waves per workgroup
constexpr int kVThreads = 64 * kVWaves;
constexpr int kOwn = 2 * kTH;                // input rows a wave loads per plane
constexpr int kGroupRows = kVWaves * kTH;    // output rows per workgroup
constexpr int kGroupIn = 2 * kGroupRows;     // input rows per workgroup
constexpr unsigned kOOB = 0x40000000u;       // past every buffer (planes < 2^30 bytes)
// The kernel's row table (2 planes x kGroupIn rows x 64 lanes x 8 bytes =
// 128 KiB of static LDS) leaves room for one workgroup per CU (160 KiB).
constexpr int kVTableBytes = 2 * kGroupIn * 64 * 8;
constexpr int kVPerCu = (160 * 1024) / kVTableBytes;
static_assert(kVPerCu >= 1, "row table must fit the LDS");

__device__ __forceinline__ __amdgpu_buffer_rsrc_t plane_rsrc(const void *base, bool valid, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, 0, valid ? bytes : 0, 0x00020000);
}

// Raw rows of one plane in flight: row rowbase + wave + kVWaves*k in v[k];
// (kWide) lane k also holds the element left of the wave's first column in
// that row.
template <typename E>
struct Rows {
    typename Elem<E>::raw4 v[kOwn];
    float lf;
};

// kG: column groups per workgroup; the kVWaves/kG waves of a group share its
// kGroupIn/kG input rows (wave wv of the group holds rows wv, wv + kVWaves/kG,
// ... of them).
template <typename E, bool kWide, int kG>
__device__ __forceinline__ void issue_plane(Rows<E> &R, const E *xs, int p, bool want, int D, int H,
                                            int W, int rowbase, int wave, int lane,
                                            unsigned laneoff, int c0w)
{
    constexpr int kNW = kVWaves / kG;
    const bool ok = want && p >= 0 && p < D;
    constexpr int ES = (int)sizeof(E);
    const __amdgpu_buffer_rsrc_t rs = plane_rsrc(xs + (int64_t)(ok ? p : 0) * H * W, ok, H * W * ES);
#pragma unroll
    for (int k = 0; k < kOwn; ++k) {
        const int row = rowbase + wave + kNW * k;
        const unsigned roff = row < H ? (unsigned)(row * W * ES) : kOOB;
        R.v[k] = Elem<E>::template load4<2>(rs, roff + laneoff);
    }
    if (kWide) {
        const int row = rowbase + wave + kNW * lane;
        const unsigned loff = (lane < kOwn && row < H && c0w > 0)
                                  ? (unsigned)((row * W + c0w - 1) * ES) : kOOB;
        R.lf = Elem<E>::load1(rs, loff);
    }
}

// Horizontal 3-tap sums of a row held as one float4 per lane; lf is the
// element left of lane 0's first column (used by lane 0 only).
template <bool kWide>
__device__ __forceinline__ v2f hsum(v4f v, float lf, int lane)
{
    float left = shr1(v.w);
    if (kWide && lane == 0) left += lf;
    return v2f{left + v.x + v.y, v.y + v.z + v.w};
}

// The wave's rows of one plane, as horizontal sums, into the row table.
template <typename E, bool kWide, int kG>
__device__ __forceinline__ void put_rows(const Rows<E> &R, v2f (*T)[64], int wave, int lane)
{
#pragma unroll
    for (int k = 0; k < kOwn; ++k) {
        const int lf = kWide ? __builtin_amdgcn_readlane(__float_as_int(R.lf), k) : 0;
        T[wave + (kVWaves / kG) * k][lane] = hsum<kWide>(Elem<E>::widen(R.v[k]), __int_as_float(lf), lane);
    }
}

// After the barrier: vertical sums of the wave's kTH output rows from table
// rows 8w-1 .. 8w+7.  Row -1 of the table is padding for the first row
// group and the last row of the previous group otherwise (read from memory).
template <typename E, bool kWide>
__device__ __forceinline__ void get_vsums(v2f (*T)[64], const E *xs, int p, int D, int H, int W,
                                          int rowbase, int wave, int lane, unsigned laneoff,
                                          int c0w, v2f vs[kTH])
{
    __syncthreads();
    v2f r[kOwn + 1];
#pragma unroll
    for (int k = 0; k < kOwn; ++k) r[k + 1] = T[kOwn * wave + k][lane];
    if (wave > 0) {
        r[0] = T[kOwn * wave - 1][lane];
    } else if (rowbase > 0 && p >= 0 && p < D) {
        constexpr int ES = (int)sizeof(E);
        const __amdgpu_buffer_rsrc_t rs = plane_rsrc(xs + (int64_t)p * H * W, true, H * W * ES);
        const unsigned roff = (unsigned)((rowbase - 1) * W * ES);
        const v4f a = Elem<E>::widen(Elem<E>::template load4<0>(rs, roff + laneoff));
        float lf = 0.0f;
        if (kWide) {
            const unsigned loff = (lane == 0 && c0w > 0) ? roff + (unsigned)((c0w - 1) * ES) : kOOB;
            lf = Elem<E>::load1(rs, loff);
        }
        r[0] = hsum<kWide>(a, lf, lane);
    } else {
        r[0] = v2f{0.0f, 0.0f};
    }
#pragma unroll
    for (int i = 0; i < kTH; ++i) vs[i] = r[2 * i] + r[2 * i + 1] + r[2 * i + 2];
}

// Grid: one workgroup per (slice, plane chunk of td output planes, column
// chunk, row group of kGroupRows/kG output rows), row groups fastest.  With
// kG > 1 (planes of fewer than kGroupIn rows) the workgroup's waves form kG
// groups, each with its own 256-column chunk (wchunks counts groups of kG
// chunks) and kGroupIn/kG input rows, in its own rows of the row table.
template <typename E, bool kWide, bool kIncl, int kG = 1>
__global__ __launch_bounds__(kVThreads)
void avgpool3d_k3s2p1_vec_kernel(const E *__restrict__ x, E *__restrict__ out,
                                 int D, int H, int W, int Do, int Ho, int Wo,
                                 int hgroups, int dchunks, int wchunks, int td)
{
    static_assert(kG == 1 || kWide, "column groups read the element left of their chunk");
    constexpr int kNW = kVWaves / kG;             // waves per column group
    __shared__ v2f T[2][kGroupIn][64];   // row table, double-buffered by plane
    static_assert(sizeof(T) == kVTableBytes, "row table size");
    const int lane = threadIdx.x & 63;
    const int wave0 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int grp = wave0 / kNW;                  // column group
    const int wave = wave0 - grp * kNW;           // wave within the group
    int64_t t = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t blk = t;
    const int hg = (int)(t % hgroups); t /= hgroups;
    const int wc = (int)(t % wchunks) * kG + grp; t /= wchunks;
    const int dc = (int)(t % dchunks); t /= dchunks;
    const int64_t sl = t;

    const int rowbase = hg * (kGroupIn / kG);     // first input row of the group
    const int h0 = hg * (kGroupRows / kG) + wave * kTH;   // first output row of the wave
    const int d0 = dc * td;
    const int d1 = min(d0 + td, Do);
    const int c0w = wc * (2 * kTW);
    const int c = c0w + 4 * lane;
    const int wo = wc * kTW + 2 * lane;
    // the group's rows of the row table
    v2f (*T0)[64] = T[0] + grp * (kGroupIn / kG);
    v2f (*T1)[64] = T[1] + grp * (kGroupIn / kG);
    constexpr int ES = (int)sizeof(E);
    const unsigned laneoff = c < W ? (unsigned)(c * ES) : kOOB;
    // Wo is even here (W % 4 == 0), so wo < Wo covers the lane's pair
    const unsigned wooff = wo < Wo ? (unsigned)(wo * ES) : kOOB;
    const E *xs = x + sl * (int64_t)D * H * W;
    E *os = out + sl * (int64_t)Do * Ho * Wo;
    const int obytes = Ho * Wo * ES;
    const float inv27 = 1.0f / 27.0f;
    // (count_include_pad=False) valid taps along W of the lane's two outputs
    const int cw0 = taps3(wo, W), cw1 = taps3(wo + 1, W);

    // Output planes [pa, pb): input planes go through T0, T1, T0, ...
    // starting with plane 2*pa-1
    auto run = [&](const int pa, const int pb) {
        Rows<E> A, B;
        v2f carry[kTH];
        issue_plane<E, kWide, kG>(A, xs, 2 * pa - 1, true, D, H, W, rowbase, wave, lane, laneoff, c0w);
        issue_plane<E, kWide, kG>(B, xs, 2 * pa, true, D, H, W, rowbase, wave, lane, laneoff, c0w);
        put_rows<E, kWide, kG>(A, T0, wave, lane);
        __builtin_amdgcn_sched_barrier(0);
        issue_plane<E, kWide, kG>(A, xs, 2 * pa + 1, true, D, H, W, rowbase, wave, lane, laneoff, c0w);
        // (an empty asm with a memory clobber after each issue keeps the loads
        // ahead of the barrier in get_vsums; without it the compiler sinks them
        // past the barrier and the LDS reads, delaying the next plane)
        asm volatile("" ::: "memory");
        get_vsums<E, kWide>(T0, xs, 2 * pa - 1, D, H, W, rowbase, wave, lane, laneoff, c0w, carry);
        // stores past the range, so that the memory-counter state entering the
        // loop matches the one at its back-edge
        const __amdgpu_buffer_rsrc_t none = plane_rsrc(os, false, 0);
#pragma unroll
        for (int i = 0; i < kTH; ++i) Elem<E>::store2(none, kOOB, 0, 0.0f, 0.0f);

        // invariant: B holds plane 2d and A plane 2d+1, both in flight
        for (int d = pa; d < pb; ++d) {
            const bool more = d + 1 < pb;
            v2f acc[kTH], v[kTH];
            put_rows<E, kWide, kG>(B, T1, wave, lane);
            __builtin_amdgcn_sched_barrier(0);
            issue_plane<E, kWide, kG>(B, xs, 2 * d + 2, more, D, H, W, rowbase, wave, lane, laneoff, c0w);
            asm volatile("" ::: "memory");
            get_vsums<E, kWide>(T1, xs, 2 * d, D, H, W, rowbase, wave, lane, laneoff, c0w, v);
#pragma unroll
            for (int i = 0; i < kTH; ++i) acc[i] = carry[i] + v[i];
            put_rows<E, kWide, kG>(A, T0, wave, lane);
            __builtin_amdgcn_sched_barrier(0);
            issue_plane<E, kWide, kG>(A, xs, 2 * d + 3, more, D, H, W, rowbase, wave, lane, laneoff, c0w);
            asm volatile("" ::: "memory");
            get_vsums<E, kWide>(T0, xs, 2 * d + 1, D, H, W, rowbase, wave, lane, laneoff, c0w, v);
            const __amdgpu_buffer_rsrc_t ro = plane_rsrc(os + (int64_t)d * Ho * Wo, true, obytes);
#pragma unroll
            for (int i = 0; i < kTH; ++i) {
                const int h = h0 + i;
                v2f o;
                if constexpr (kIncl) {
                    o = (acc[i] + v[i]) * inv27;
                } else {
                    const int cdh = taps3(d, D) * taps3(h, H);
                    const v2f sum = acc[i] + v[i];
                    o = v2f{sum.x * (1.0f / (float)(cdh * cw0)), sum.y * (1.0f / (float)(cdh * cw1))};
                }
                // the row (wave-uniform) in the scalar offset, the lane's
                // column in the vector offset; a row past the plane takes the
                // zero-size resource
                Elem<E>::store2(h < Ho ? ro : none, wooff, h < Ho ? h * Wo * ES : 0, o.x, o.y);
                carry[i] = v[i];
            }
        }
    };
    if constexpr (sizeof(E) == 4) {
        run(d0, d1);
    } else {
        // bf16: each workgroup starts at its own plane offset and wraps
        // around, so the workgroups running together stream different offsets
        // of their slices (one plane is read twice).  At [16,32,128,128,256]
        // this took 917 to 840 us; the same rotation made the fp32 kernel
        // 3-4% slower, so fp32 keeps one pass from the first plane.
        const int n = d1 - d0;
        const int r = n > 1 ? (int)((blk * 13 + 5) % n) : 0;
        if (r == 0) {
            run(d0, d1);
        } else {
            run(d0 + r, d1);
            __syncthreads();   // the second range's prologue rewrites T0
            run(d0, d0 + r);
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
template <typename E>
__device__ __forceinline__ void plane_sums_elem(const E *__restrict__ xs, int plane, int D,
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
            const E *rp = xs + ((int64_t)plane * H + row) * W;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (c + j < W) v[j] = Elem<E>::to_f32(rp[c + j]);
            if (lane == 0 && c > 0) left = Elem<E>::to_f32(rp[c - 1]);
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

template <typename E, bool kIncl>
__global__ __launch_bounds__(kEThreads)
void avgpool3d_k3s2p1_elem_kernel(const E *__restrict__ x, E *__restrict__ out,
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

    const E *xs = x + sl * (int64_t)D * H * W;
    E *os = out + sl * (int64_t)Do * Ho * Wo;

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
            const float s0 = carry[i][0] + va[i][0] + vb[i][0];
            const float s1 = carry[i][1] + va[i][1] + vb[i][1];
            float o0 = s0 * inv27, o1 = s1 * inv27;
            if constexpr (!kIncl) {
                const int cdh = taps3(d, D) * taps3(h, H);
                o0 = s0 * (1.0f / (float)(cdh * taps3(wo, W)));
                o1 = s1 * (1.0f / (float)(cdh * taps3(wo + 1, W)));
            }
            if (h < Ho) {
                E *orow = os + ((int64_t)d * Ho + h) * Wo;
                if (wo < Wo) __builtin_nontemporal_store(Elem<E>::from_f32(o0), orow + wo);
                if (wo + 1 < Wo) __builtin_nontemporal_store(Elem<E>::from_f32(o1), orow + wo + 1);
            }
            carry[i][0] = vb[i][0];
            carry[i][1] = vb[i][1];
        }
    }
}

// ------------------------------------------------------ small-plane kernel --
// Planes of at most kSElems elements whose bordered copy fits one LDS buffer.
// The kernels above give a wave 4 output rows x 128 output columns, which a
// small plane fills only in part (a 16 x 16 plane: 2 of 16 rows, 4 of 64
// lanes).  Here a workgroup takes S whole slices and walks output planes
// [d0, d1): each input plane of the S slices is loaded once (VW consecutive
// elements per load), widened into an LDS buffer with a zero border (one row
// above and below, one column left and right), and every output of the S
// slices sums its 3x3 window there, so no tap needs a bounds test.  Output
// plane d adds the window sums of input planes 2d-1, 2d and 2d+1; the last
// is carried to d+1.  The next plane's loads are in flight while a plane is
// summed; the buffer is double-buffered by plane, one barrier per plane.
constexpr int kSThreads = 256;
constexpr int kSElems = 4096;                // elements of one input plane of the S slices
constexpr int kSOut = 8;                     // outputs per work-item
constexpr int kSBufBytes = 24 * 1024;        // one LDS plane buffer

// LDS geometry of one slice's plane: rows -1 .. H (zero rows -1 and H),
// columns at +4 of their index (zero columns 3 and W + 4), so that a row's
// first element is 16-byte aligned.
__host__ __device__ constexpr int plane_pitch(int W) { return W + 8; }
__host__ __device__ constexpr int plane_floats(int H, int W) { return (H + 2) * plane_pitch(W); }

template <typename E, int VW>
struct Piece;
template <> struct Piece<float, 4> {
    typedef v4f raw;
    static __device__ __forceinline__ raw zero() { return v4f{0.0f, 0.0f, 0.0f, 0.0f}; }
    static __device__ __forceinline__ raw load(const float *p) { return *reinterpret_cast<const v4f *>(p); }
    static __device__ __forceinline__ void put(float *d, raw v) { *reinterpret_cast<v4f *>(d) = v; }
};
template <> struct Piece<uint16_t, 4> {
    typedef u32x2 raw;
    static __device__ __forceinline__ raw zero() { return u32x2{0u, 0u}; }
    static __device__ __forceinline__ raw load(const uint16_t *p) { return *reinterpret_cast<const u32x2 *>(p); }
    static __device__ __forceinline__ void put(float *d, raw v) { *reinterpret_cast<v4f *>(d) = Elem<uint16_t>::widen(v); }
};
template <typename E> struct Piece<E, 1> {
    typedef E raw;
    static __device__ __forceinline__ raw zero() { return (E)0; }
    static __device__ __forceinline__ raw load(const E *p) { return *p; }
    static __device__ __forceinline__ void put(float *d, raw v) { *d = Elem<E>::to_f32(v); }
};

template <typename E, int VW, bool kIncl>
__global__ __launch_bounds__(kSThreads)
void avgpool3d_k3s2p1_plane_kernel(const E *__restrict__ x, E *__restrict__ out, int64_t NC,
                                   int D, int H, int W, int Do, int Ho, int Wo, int S,
                                   int dchunks, int td)
{
    constexpr int kP = kSElems / VW / kSThreads;      // pieces per work-item
    typedef Piece<E, VW> PC;
    extern __shared__ float lds[];                   // [2][S][H + 2][pitch]
    const int tid = threadIdx.x;
    const int pitch = plane_pitch(W);
    const int pf = plane_floats(H, W);
    const int buf = S * pf;
    const int sg = (int)(blockIdx.x / dchunks), dc = (int)(blockIdx.x % dchunks);
    const int64_t s0 = (int64_t)sg * S;
    const int ns = (int)min((int64_t)S, NC - s0);
    const int d0 = dc * td, d1 = min(d0 + td, Do);
    const int64_t HW = (int64_t)H * W, DHW = (int64_t)D * HW;

    // both buffers start zero: the border is never written afterwards
    for (int i = tid; i < 2 * buf; i += kSThreads) lds[i] = 0.0f;

    // pieces: q = tid + 256*i -> slice q / pps, row r, first column c
    const int wv = W / VW, pps = H * wv;
    const E *src[kP];
    int loff[kP];
    bool pv[kP];
#pragma unroll
    for (int i = 0; i < kP; ++i) {
        const int q = tid + kSThreads * i;
        pv[i] = q < ns * pps;
        const int sl = pv[i] ? q / pps : 0, e = pv[i] ? q - sl * pps : 0;
        const int r = e / wv, c = (e - r * wv) * VW;
        src[i] = x + (s0 + sl) * DHW + (int64_t)r * W + c;
        loff[i] = sl * pf + (r + 1) * pitch + 4 + c;
    }
    // outputs: o = tid + 256*j -> slice, ho, wo; window top-left in LDS
    const int opp = Ho * Wo;
    E *dst[kSOut];
    int lb[kSOut];
    float chw[kSOut], acc[kSOut];
    bool ov[kSOut];
#pragma unroll
    for (int j = 0; j < kSOut; ++j) {
        const int o = tid + kSThreads * j;
        ov[j] = o < ns * opp;
        const int sl = ov[j] ? o / opp : 0, e = ov[j] ? o - sl * opp : 0;
        const int ho = e / Wo, wo = e - ho * Wo;
        dst[j] = out + (s0 + sl) * (int64_t)Do * opp + e;
        lb[j] = sl * pf + 2 * ho * pitch + 2 * wo + 3;
        chw[j] = (float)(taps3(ho, H) * taps3(wo, W));
        acc[j] = 0.0f;
    }

    typename PC::raw pre[kP];
    auto load = [&](int p) {
        const bool pok = p >= 0 && p < D;
        const int64_t po = pok ? (int64_t)p * HW : 0;
#pragma unroll
        for (int i = 0; i < kP; ++i) {
            const bool ok = pok && pv[i];
            const typename PC::raw v = PC::load(ok ? src[i] + po : x);
            pre[i] = ok ? v : PC::zero();
        }
    };
    const int pa = 2 * d0 - 1, pb = 2 * d1 - 1;
    load(pa);
    for (int p = pa; p <= pb; ++p) {
        const int k = p - pa;
        float *B = lds + (k & 1) * buf;
        // this buffer was last read two planes ago, before the previous
        // plane's barrier
#pragma unroll
        for (int i = 0; i < kP; ++i)
            if (pv[i]) PC::put(B + loff[i], pre[i]);
        if (p < pb) load(p + 1);
        // keeps the next plane's loads ahead of the barrier
        asm volatile("" ::: "memory");
        __syncthreads();
        const int d = d0 + (k - 2) / 2;               // output plane finished at even k >= 2
#pragma unroll
        for (int j = 0; j < kSOut; ++j) {
            if (!ov[j]) continue;
            const float *t = B + lb[j];
            const float s2 = (t[0] + t[1] + t[2]) + (t[pitch] + t[pitch + 1] + t[pitch + 2]) +
                             (t[2 * pitch] + t[2 * pitch + 1] + t[2 * pitch + 2]);
            if (k == 0) {
                acc[j] = s2;
            } else if (k & 1) {
                acc[j] += s2;
            } else {
                const float sum = acc[j] + s2;
                const float o = kIncl ? sum * (1.0f / 27.0f)
                                      : sum * (1.0f / ((float)taps3(d, D) * chw[j]));
                dst[j][(int64_t)d * opp] = Elem<E>::from_f32(o);
                acc[j] = s2;
            }
        }
    }
}

}  // namespace

namespace {
// Launch shape of the streaming kernels for one call.
struct PoolPlan {
    bool vec;          // vector kernel
    bool small;        // small-plane kernel (else, without vec, the element kernel)
    int Do, Ho, Wo, hgroups, wchunks, dchunks, td;
    int G;             // vector kernel: column groups per workgroup
    int S, vw;         // small-plane kernel: slices per workgroup, elements per load
    size_t lds;        // small-plane kernel: dynamic LDS bytes
    int64_t nwg;       // workgroups
    int threads;       // work-items per workgroup
};

PoolPlan plan_k3s2p1(int es, const void *x, const void *out, int64_t NC, int64_t D, int64_t H,
                     int64_t W)
{
    PoolPlan p;
    p.Do = (int)((D - 1) / 2 + 1);
    p.Ho = (int)((H - 1) / 2 + 1);
    p.Wo = (int)((W - 1) / 2 + 1);
    p.wchunks = (p.Wo + kTW - 1) / kTW;
    p.vec = false;
    p.small = H * W <= kSElems && plane_floats((int)H, (int)W) * 4 <= kSBufBytes &&
              (int64_t)p.Ho * p.Wo <= (int64_t)kSThreads * kSOut;
    if (p.small) {
        // slices per workgroup: as many as the LDS buffer, the loads (kSElems
        // elements) and the outputs (kSOut per work-item) allow
        int64_t S = kSBufBytes / (plane_floats((int)H, (int)W) * 4);
        S = std::min<int64_t>(S, kSElems / (H * W));
        S = std::min<int64_t>(S, (int64_t)kSThreads * kSOut / ((int64_t)p.Ho * p.Wo));
        S = std::min<int64_t>(S, NC);
        p.S = (int)S;
        p.vw = (W % 4 == 0 && (reinterpret_cast<uintptr_t>(x) % (4 * es)) == 0) ? 4 : 1;
        p.lds = (size_t)2 * p.S * plane_floats((int)H, (int)W) * sizeof(float);
        // plane chunks (each re-reads one halo plane) until the grid has about
        // four workgroups per CU, none shorter than two output planes
        const int64_t groups = (NC + p.S - 1) / p.S;
        const int64_t want = (int64_t)device_cus() * 4;
        int64_t dchunks = (want + groups - 1) / groups;
        if (dchunks > p.Do) dchunks = p.Do;
        int64_t td = (p.Do + dchunks - 1) / dchunks;
        if (td < 2) td = std::min<int64_t>(2, p.Do);
        p.td = (int)td;
        p.dchunks = (int)((p.Do + td - 1) / td);
        p.hgroups = 1;
        p.nwg = groups * p.dchunks;
        p.threads = kSThreads;
        return p;
    }
    // vector path: 4 elements per lane load, 2 per lane store, planes < 2^30 bytes
    p.vec = (W % 4 == 0) && ((reinterpret_cast<uintptr_t>(x) % (4 * es)) == 0) &&
            ((reinterpret_cast<uintptr_t>(out) % (2 * es)) == 0) && H * W * es < (int64_t)kOOB;
    p.G = 1;
    if (p.vec) {
        // planes of fewer than kGroupIn rows: split the waves into column
        // groups of kGroupIn/G rows each (G a power of two up to 8, no more
        // groups than column chunks)
        while (p.G < 8 && kGroupIn / (2 * p.G) >= H && p.G < p.wchunks) p.G *= 2;
        p.wchunks = (p.wchunks + p.G - 1) / p.G;
        p.hgroups = (p.Ho + kGroupRows / p.G - 1) / (kGroupRows / p.G);
        // as few plane chunks as still give every CU as many workgroups as fit
        // on it at once (one: the 128 KiB row table fills the LDS)
        const int64_t base = NC * p.hgroups * p.wchunks;
        const int64_t want = (int64_t)device_cus() * kVPerCu;
        int64_t dchunks = (want + base - 1) / base;
        if (dchunks > p.Do) dchunks = p.Do;
        p.td = (int)((p.Do + dchunks - 1) / dchunks);
        p.dchunks = (int)((p.Do + p.td - 1) / p.td);
        p.nwg = base * p.dchunks;
        p.threads = kVThreads;
    } else {
        p.hgroups = (p.Ho + kEWaves * kTH - 1) / (kEWaves * kTH);
        p.dchunks = (p.Do + kETD - 1) / kETD;
        p.td = kETD;
        p.nwg = NC * (int64_t)p.hgroups * p.dchunks * p.wchunks;
        p.threads = kEThreads;
    }
    return p;
}

template <typename E, bool kIncl>
hipError_t launch_k3s2p1(const E *x, int64_t NC, int64_t D, int64_t H, int64_t W, E *out,
                         hipStream_t stream)
{
    const PoolPlan p = plan_k3s2p1((int)sizeof(E), x, out, NC, D, H, W);
    if (p.nwg * p.threads > (int64_t)UINT32_MAX) return hipErrorInvalidConfiguration;
    if (p.small) {
        const void *fn = p.vw == 4 ? (const void *)avgpool3d_k3s2p1_plane_kernel<E, 4, kIncl>
                                   : (const void *)avgpool3d_k3s2p1_plane_kernel<E, 1, kIncl>;
        hipError_t e = allow_dynamic_lds(fn, p.lds);
        if (e != hipSuccess) return e;
        if (p.vw == 4)
            hipLaunchKernelGGL((avgpool3d_k3s2p1_plane_kernel<E, 4, kIncl>), dim3((unsigned)p.nwg),
                               dim3(kSThreads), p.lds, stream, x, out, NC, (int)D, (int)H, (int)W,
                               p.Do, p.Ho, p.Wo, p.S, p.dchunks, p.td);
        else
            hipLaunchKernelGGL((avgpool3d_k3s2p1_plane_kernel<E, 1, kIncl>), dim3((unsigned)p.nwg),
                               dim3(kSThreads), p.lds, stream, x, out, NC, (int)D, (int)H, (int)W,
                               p.Do, p.Ho, p.Wo, p.S, p.dchunks, p.td);
    } else if (p.vec) {
        const void *fn = p.G == 8   ? (const void *)avgpool3d_k3s2p1_vec_kernel<E, true, kIncl, 8>
                         : p.G == 4 ? (const void *)avgpool3d_k3s2p1_vec_kernel<E, true, kIncl, 4>
                         : p.G == 2 ? (const void *)avgpool3d_k3s2p1_vec_kernel<E, true, kIncl, 2>
                         : p.wchunks > 1 ? (const void *)avgpool3d_k3s2p1_vec_kernel<E, true, kIncl, 1>
                                         : (const void *)avgpool3d_k3s2p1_vec_kernel<E, false, kIncl, 1>;
        int iD = (int)D, iH = (int)H, iW = (int)W;
        int Do_ = p.Do, Ho_ = p.Ho, Wo_ = p.Wo, hg = p.hgroups, dch = p.dchunks, wch = p.wchunks, td = p.td;
        void *args[] = {(void *)&x, (void *)&out, &iD, &iH, &iW, &Do_, &Ho_, &Wo_, &hg, &dch, &wch, &td};
        return hipLaunchKernel(fn, dim3((unsigned)p.nwg), dim3(kVThreads), args, 0, stream);
    } else {
        hipLaunchKernelGGL((avgpool3d_k3s2p1_elem_kernel<E, kIncl>), dim3((unsigned)p.nwg),
                           dim3(kEThreads), 0, stream, x, out, (int)D, (int)H, (int)W, p.Do, p.Ho,
                           p.Wo, p.hgroups, p.dchunks, p.wchunks);
    }
    return hipGetLastError();
}
}  // namespace

bool avgpool3d_k3s2p1_fits(bool bf16, const void *x, const void *out, int64_t NC, int64_t D,
                           int64_t H, int64_t W)
{
    const PoolPlan p = plan_k3s2p1(bf16 ? 2 : 4, x, out, NC, D, H, W);
    return p.nwg * p.threads <= (int64_t)UINT32_MAX;
}

hipError_t launch_avgpool3d_k3s2p1(const void *x, bool bf16, bool include_pad, int64_t NC,
                                   int64_t D, int64_t H, int64_t W, void *out, hipStream_t stream)
{
    const uint16_t *xb = static_cast<const uint16_t *>(x);
    const float *xf = static_cast<const float *>(x);
    uint16_t *ob = static_cast<uint16_t *>(out);
    float *of = static_cast<float *>(out);
    if (bf16)
        return include_pad ? launch_k3s2p1<uint16_t, true>(xb, NC, D, H, W, ob, stream)
                           : launch_k3s2p1<uint16_t, false>(xb, NC, D, H, W, ob, stream);
    return include_pad ? launch_k3s2p1<float, true>(xf, NC, D, H, W, of, stream)
                       : launch_k3s2p1<float, false>(xf, NC, D, H, W, of, stream);
}

}  // namespace ct
