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
//  * Epilogue: the model's ((S/8 + conv_bias)*scale1 + bias)*scale2, which the
//    page folds to S*(scale1*scale2/8) + (conv_bias*scale1 + bias)*scale2
//    (passage on the epilogue algebra: the conv bias passes through the
//    average unchanged); the slab path evaluates the folded form as one fma
//    (within an ulp or two of the literal order), the direct path the literal
//    order.
//
// MI355X mapping.  S is a dense contraction over kappa = ci*8 + tap
// (K = 8*Cin) for each (co, voxel), so it runs as v_mfma_f32_16x16x4_f32:
//   A (16 x 4)  = Weff^T rows co,      lane l supplies A[l%16][l/16]
//   B (4 x 16)  = X[kappa][voxel],     lane l supplies B[l/16][l%16]
//   D (16 x 16) = S[co][voxel],        lane l holds D[4*(l/16)+r][l%16]
// An M-block is 16 consecutive w of one pooled row (n, d, h); a 16-wide
// block of output channels is blockIdx.y.  Lanes 0..15 of each store write 16
// consecutive w of one channel (64 contiguous bytes; plain stores so that L2
// merges the neighbouring blocks' partial lines).
//  * Weff^T is built once per workgroup in LDS in fragment order, then each
//    wave holds its fragments in registers (KS = 2*Cin k-steps, Cin <= 4).
//  * Waves are persistent: each walks a contiguous range of M-blocks (the
//    workgroup index is remapped so neighbouring ranges share an XCD's L2),
//    advancing (n, d, h, w-block) incrementally instead of dividing, with
//    the per-lane tap offsets ci*DHW + a*HW + b*W + c computed once.
//  * The next M-block's 8*Cin input taps are loaded before the current
//    block's MFMAs, so one block's load latency overlaps another's math.
// Cin > 4 takes the same structure with a runtime k-step loop and the
// fragments read from LDS.
#include "ct_internal.h"

namespace ct {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kMinMbPerWave = 4;  // do not split the work finer than this

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Weff^T fragments for output-channel block cob: wfrag[j*64 + l] =
// Weff[ci, co = cob*16 + l%16, tap] with kappa = 4j + l/16 = ci*8 + tap.
__device__ __forceinline__ void build_wfrag(const float *__restrict__ w, int Cout, int cob,
                                            int ksteps, float *wfrag)
{
    for (int e = threadIdx.x; e < ksteps * 64; e += kThreads) {
        const int j = e >> 6, l = e & 63;
        const int co = cob * 16 + (l & 15);
        const int kap = 4 * j + (l >> 4);
        // all 8 candidate taps are loaded unconditionally from valid addresses
        // (a conditional load would be waited on before the next one issues)
        const int ci = kap >> 3, tap = kap & 7;
        const int a = tap >> 2, b = (tap >> 1) & 1, c = tap & 1;
        const float *wp = w + ((int64_t)ci * Cout + min(co, Cout - 1)) * 27;
        // per axis: input offset 0 takes taps {1,2}, offset 1 takes tap {0}
        const int kd0 = a ? 0 : 1, nkd = a ? 1 : 2;
        const int kh0 = b ? 0 : 1, nkh = b ? 1 : 2;
        const int kw0 = c ? 0 : 1, nkw = c ? 1 : 2;
        float t8[8];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                for (int k = 0; k < 2; ++k)
                    t8[(i * 2 + jj) * 2 + k] = wp[(kd0 + i) * 9 + (kh0 + jj) * 3 + kw0 + k];
        float v = 0.0f;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                for (int k = 0; k < 2; ++k)
                    if (i < nkd && jj < nkh && k < nkw) v += t8[(i * 2 + jj) * 2 + k];
        if (co >= Cout) v = 0.0f;
        wfrag[e] = v;
    }
}

struct Pos {        // wave-uniform position of an M-block
    int n, d, h, wb;
};

__device__ __forceinline__ void advance(Pos &p, int wblocks, int Hp, int Dp)
{
    if (++p.wb == wblocks) {
        p.wb = 0;
        if (++p.h == Hp) {
            p.h = 0;
            if (++p.d == Dp) { p.d = 0; ++p.n; }
        }
    }
}

// KS > 0: 2*Cin k-steps known at compile time; KS == 0: runtime Cin.
template <int KS>
__global__ __launch_bounds__(kThreads)
void fused3d_f32_kernel(const float *__restrict__ x, const float *__restrict__ w,
                        const float *__restrict__ conv_bias,
                        const float *__restrict__ bias, float s1, float s2,
                        int Cin, int D, int H, int W, int Cout,
                        int Dp, int Hp, int Wp, int wblocks, int nmblocks, int mb_per_wave,
                        float *__restrict__ out)
{
    extern __shared__ float wfrag[];          // [ksteps][64]
    const int ksteps = KS > 0 ? KS : 2 * Cin;
    const int cob = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const int col = lane & 15;   // voxel (w offset) inside the M-block
    const int kq = lane >> 4;    // kappa offset inside a k-step / co group in D

    build_wfrag(w, Cout, cob, ksteps, wfrag);
    __syncthreads();

    const int HW = H * W;                      // per-item sizes < 2^31 (checked by the shim)
    const int DHW = D * HW;
    const int64_t pplane = (int64_t)Dp * Hp * Wp;

    // per-lane epilogue constants and output offsets, co = cob*16 + 4*kq + r
    float cbv[4], bv[4];
    int64_t co_off[4];
    bool co_ok[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int co = cob * 16 + 4 * kq + r;
        co_ok[r] = co < Cout;
        cbv[r] = (conv_bias && co_ok[r]) ? conv_bias[co] : 0.0f;
        bv[r] = (bias && co_ok[r]) ? bias[co] : 0.0f;
        co_off[r] = (int64_t)co * pplane;
    }

    // this wave's contiguous range of M-blocks
    const int64_t gw = xcd_remap(blockIdx.x, gridDim.x) * kWaves + wave;
    const int mb_begin = uniform((int)min<int64_t>(gw * mb_per_wave, nmblocks));
    const int mb_end = uniform((int)min<int64_t>((int64_t)mb_begin + mb_per_wave, nmblocks));
    if (mb_begin >= mb_end) return;           // after the only barrier
    Pos p;
    {
        int t = mb_begin;
        p.wb = uniform(t % wblocks); t /= wblocks;
        p.h = uniform(t % Hp); t /= Hp;
        p.d = uniform(t % Dp);
        p.n = uniform(t / Dp);
    }

    if constexpr (KS > 0) {
        float a[KS];
        int off[KS];
#pragma unroll
        for (int j = 0; j < KS; ++j) {
            a[j] = wfrag[j * 64 + lane];
            const int kap = 4 * j + kq;
            const int ci = kap >> 3, tap = kap & 7;
            off[j] = ci * DHW + (tap >> 2) * HW + ((tap >> 1) & 1) * W + (tap & 1);
        }
        auto load = [&](const Pos &q, float *v) {
            const int wv = min(q.wb * 16 + col, Wp - 1);   // masked lanes read a valid tap
            const float *xb = x + (int64_t)q.n * Cin * DHW + (int64_t)q.d * HW + q.h * W + wv;
#pragma unroll
            for (int j = 0; j < KS; ++j) v[j] = xb[off[j]];
        };
        float cur[KS], nxt[KS];
        load(p, cur);
        for (int mb = mb_begin; mb < mb_end; ++mb) {
            Pos q = p;
            advance(q, wblocks, Hp, Dp);
            if (mb + 1 < mb_end) load(q, nxt);
            v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int j = 0; j < KS; ++j)
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], cur[j], acc, 0, 0, 0);
            const int wv = p.wb * 16 + col;
            if (wv < Wp) {
                float *on = out + (int64_t)p.n * Cout * pplane + ((int64_t)p.d * Hp + p.h) * Wp + wv;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if (co_ok[r]) {
                        float v = acc[r] * 0.125f;
                        v = (v + cbv[r]) * s1;
                        v = (v + bv[r]) * s2;
                        on[co_off[r]] = v;
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < KS; ++j) cur[j] = nxt[j];
            p = q;
        }
    } else {
        constexpr int kChunk = 8;    // k-steps whose loads are issued together
        for (int mb = mb_begin; mb < mb_end; ++mb) {
            const int wv0 = p.wb * 16 + col;
            const int wv = min(wv0, Wp - 1);
            const float *xb = x + (int64_t)p.n * Cin * DHW + (int64_t)p.d * HW + p.h * W + wv;
            v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
            for (int j0 = 0; j0 < ksteps; j0 += kChunk) {
                float xv[kChunk];
#pragma unroll
                for (int jj = 0; jj < kChunk; ++jj) {
                    const int kap = 4 * (j0 + jj) + kq;
                    const int ci = kap >> 3, tap = kap & 7;
                    const int cic = min(ci, Cin - 1);          // valid address; masked below
                    const float v = xb[(int64_t)cic * DHW + (tap >> 2) * HW + ((tap >> 1) & 1) * W + (tap & 1)];
                    xv[jj] = (j0 + jj < ksteps) ? v : 0.0f;
                }
#pragma unroll
                for (int jj = 0; jj < kChunk; ++jj)
                    if (j0 + jj < ksteps)
                        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(
                            wfrag[(j0 + jj) * 64 + lane], xv[jj], acc, 0, 0, 0);
            }
            if (wv0 < Wp) {
                float *on = out + (int64_t)p.n * Cout * pplane + ((int64_t)p.d * Hp + p.h) * Wp + wv0;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if (co_ok[r]) {
                        float v = acc[r] * 0.125f;
                        v = (v + cbv[r]) * s1;
                        v = (v + bv[r]) * s2;
                        on[co_off[r]] = v;
                    }
                }
            }
            advance(p, wblocks, Hp, Dp);
        }
    }
}

// Main path for Cin <= 4: persistent workgroups walk contiguous ranges of
// tasks (n, d, TH pooled rows).  A task's input slab x[n, :, d..d+1,
// h0..h0+TH, :] is loaded two tasks ahead with coalesced VEC-wide loads into
// registers, written into the spare half of a double-buffered LDS slab one
// task ahead, and read from there as B fragments (16 consecutive w per lane
// group); one barrier per task.  The first slab's loads are issued before
// the filter build so the two latencies overlap.
constexpr int kSlabPrefetch = 4;   // slab pieces each thread keeps in flight

template <int VEC> struct Vec;
template <> struct Vec<4> { typedef float4 T; };
template <> struct Vec<1> { typedef float T; };

template <int KS, int VEC>
__global__ __launch_bounds__(kThreads)
void fused3d_f32_slab_kernel(const float *__restrict__ x, const float *__restrict__ w,
                             const float *__restrict__ conv_bias,
                             const float *__restrict__ bias, float s1, float s2,
                             int Cin, int D, int H, int W, int Cout,
                             int Dp, int Hp, int Wp, int TH, int hchunks, int ntasks,
                             int tasks_per_wg, float *__restrict__ out)
{
    typedef typename Vec<VEC>::T vec_t;
    extern __shared__ float lds[];
    const int R = TH + 1;                      // input rows per plane in a slab
    const int slab_floats = Cin * 2 * R * W;
    float *wfrag = lds;                        // [KS][64]
    float *slabs = lds + KS * 64;              // 2 x [Cin][2][R][W] (double buffer)
    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const int col = lane & 15;
    const int kq = lane >> 4;
    const int cob = blockIdx.y;
    const int HW = H * W, DHW = D * HW;        // per-item sizes < 2^31 (checked by the shim)
    const int64_t pplane = (int64_t)Dp * Hp * Wp;
    const int wblocks = (Wp + 15) / 16;

    // this workgroup's contiguous task range (n, d, hc), decoded once
    const int t_begin = uniform((int)min<int64_t>(xcd_remap(blockIdx.x, gridDim.x) * tasks_per_wg, ntasks));
    const int t_end = uniform(min(t_begin + tasks_per_wg, ntasks));
    int hc, d, n;
    {
        int t = t_begin;
        hc = uniform(t % hchunks); t /= hchunks;
        d = uniform(t % Dp);
        n = uniform(t / Dp);
    }

    // tile-invariant staging plan: piece q = ((ci*2 + a)*R + r)*(W/VEC) + v
    const int WV = W / VEC;
    const int npieces = Cin * 2 * R * WV;
    int src_off[kSlabPrefetch], dst_off[kSlabPrefetch], prow[kSlabPrefetch];
#pragma unroll
    for (int i = 0; i < kSlabPrefetch; ++i) {
        const int q = threadIdx.x + i * kThreads;
        const int v = q % WV, t = q / WV;
        const int r = t % R, ca = t / R;
        const int a = ca & 1, ci = ca >> 1;
        src_off[i] = ci * DHW + a * HW + r * W + v * VEC;
        dst_off[i] = (ca * R + r) * W + v * VEC;
        prow[i] = q < npieces ? r : 1 << 30;   // rows past H (or no piece) load nothing
    }
    vec_t pre[kSlabPrefetch];
    // loads are unconditional (rows past H read x[0..], a valid address) so
    // they all stay in flight; the zero fill is applied when they are stored
    auto fetch = [&](int n_, int d_, int hc_) {
        const int h0 = hc_ * TH;
        const float *xb = x + (int64_t)n_ * Cin * DHW + (int64_t)d_ * HW + (int64_t)h0 * W;
#pragma unroll
        for (int i = 0; i < kSlabPrefetch; ++i) {
            const float *src = (h0 + prow[i] < H) ? xb + src_off[i] : x;
            pre[i] = *reinterpret_cast<const vec_t *>(src);
        }
    };
    // writes the prefetched slab (plus any pieces beyond the prefetch plan) into buf
    auto put = [&](float *buf, int n_, int d_, int hc_) {
        const int h0 = hc_ * TH;
#pragma unroll
        for (int i = 0; i < kSlabPrefetch; ++i)
            if (prow[i] < (1 << 30))
                *reinterpret_cast<vec_t *>(buf + dst_off[i]) = (h0 + prow[i] < H) ? pre[i] : vec_t{};
        for (int q = threadIdx.x + kSlabPrefetch * kThreads; q < npieces; q += kThreads) {
            const int v = q % WV, tt = q / WV;
            const int r = tt % R, ca = tt / R;
            vec_t val = vec_t{};
            if (h0 + r < H)
                val = *reinterpret_cast<const vec_t *>(
                    x + (int64_t)n_ * Cin * DHW + (int64_t)d_ * HW + (int64_t)h0 * W +
                    (ca >> 1) * DHW + (ca & 1) * HW + r * W + v * VEC);
            *reinterpret_cast<vec_t *>(buf + (ca * R + r) * W + v * VEC) = val;
        }
    };
    // the first slab's loads fly while the filter is built
    if (t_begin < t_end) fetch(n, d, hc);

    build_wfrag(w, Cout, cob, KS, wfrag);

    float a[KS];
    int soff[KS];
#pragma unroll
    for (int j = 0; j < KS; ++j) {
        const int kap = 4 * j + kq;
        const int ci = kap >> 3, tap = kap & 7;
        soff[j] = ((ci * 2 + (tap >> 2)) * R + ((tap >> 1) & 1)) * W + (tap & 1);
    }
    // folded epilogue ((S/8 + cb)*s1 + b)*s2 = S*alpha + beta[co]
    const float alpha = 0.125f * s1 * s2;
    float beta[4];
    int co_off[4];            // per-item output offsets fit in int32 (checked by the shim)
    bool co_ok[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int co = cob * 16 + 4 * kq + r;
        co_ok[r] = co < Cout;
        const float cbv = (conv_bias && co_ok[r]) ? conv_bias[co] : 0.0f;
        const float bv = (bias && co_ok[r]) ? bias[co] : 0.0f;
        beta[r] = (cbv * s1 + bv) * s2;
        co_off[r] = co * (int)pplane;
    }

    // slab of the first task into buffer 0; then per task: put the next slab
    // into the other buffer, fetch the one after, compute, one barrier
    if (t_begin < t_end) put(slabs, n, d, hc);
    __syncthreads();                           // filter and first slab visible
#pragma unroll
    for (int j = 0; j < KS; ++j) a[j] = wfrag[j * 64 + lane];
    int hc2 = hc + 1, d2 = d, n2 = n;
    if (hc2 == hchunks) { hc2 = 0; if (++d2 == Dp) { d2 = 0; ++n2; } }
    if (t_begin + 1 < t_end) fetch(n2, d2, hc2);

    for (int t = t_begin; t < t_end; ++t) {
        const int buf = (t - t_begin) & 1;
        float *cur = slabs + buf * slab_floats;
        // next task's slab into the other buffer (its last readers finished
        // before the previous iteration's barrier), then the loads after it
        if (t + 1 < t_end) {
            put(slabs + (buf ^ 1) * slab_floats, n2, d2, hc2);
            int hc3 = hc2 + 1, d3 = d2, n3 = n2;
            if (hc3 == hchunks) { hc3 = 0; if (++d3 == Dp) { d3 = 0; ++n3; } }
            if (t + 2 < t_end) fetch(n3, d3, hc3);
            hc2 = hc3; d2 = d3; n2 = n3;
        }

        const int h0 = hc * TH;
        const int rows = min(TH, Hp - h0);
        float *ob = out + (int64_t)n * Cout * pplane + ((int64_t)d * Hp + h0) * Wp;
        // each wave takes rows hh = wave, wave + 4, ... two at a time (hh and
        // hh + 4); a row's w-blocks go in pairs, each block's K range split
        // over two accumulators: eight independent MFMA chains in flight, with
        // all their LDS reads issued first
        auto store_block = [&](float *orow, int wv, const v4f &p, const v4f &q) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (co_ok[r]) orow[co_off[r] + wv] = __builtin_fmaf(p[r] + q[r], alpha, beta[r]);
        };
        for (int hh = wave; hh < rows; hh += 2 * kWaves) {
            const int hh2 = hh + kWaves;
            const bool two = hh2 < rows;           // wave-uniform
            const float *srowA = cur + hh * W, *srowB = cur + (two ? hh2 : hh) * W;
            float *orowA = ob + hh * Wp, *orowB = ob + hh2 * Wp;
            for (int wb = 0; wb < wblocks; wb += 2) {
                const int wv0 = wb * 16 + col, wv1 = wv0 + 16;
                const int wc0 = min(wv0, Wp - 1), wc1 = min(wv1, Wp - 1);
                float a0[KS], a1[KS], b0[KS], b1[KS];
#pragma unroll
                for (int j = 0; j < KS; ++j) {
                    a0[j] = srowA[wc0 + soff[j]];
                    a1[j] = srowA[wc1 + soff[j]];
                    b0[j] = srowB[wc0 + soff[j]];
                    b1[j] = srowB[wc1 + soff[j]];
                }
                v4f pA0 = {0.0f, 0.0f, 0.0f, 0.0f}, qA0 = pA0, pA1 = pA0, qA1 = pA0;
                v4f pB0 = pA0, qB0 = pA0, pB1 = pA0, qB1 = pA0;
#pragma unroll
                for (int j = 0; j < KS; j += 2) {
                    pA0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], a0[j], pA0, 0, 0, 0);
                    pA1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], a1[j], pA1, 0, 0, 0);
                    pB0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b0[j], pB0, 0, 0, 0);
                    pB1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b1[j], pB1, 0, 0, 0);
                    qA0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j + 1], a0[j + 1], qA0, 0, 0, 0);
                    qA1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j + 1], a1[j + 1], qA1, 0, 0, 0);
                    qB0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j + 1], b0[j + 1], qB0, 0, 0, 0);
                    qB1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j + 1], b1[j + 1], qB1, 0, 0, 0);
                }
                const bool w1 = wb + 1 < wblocks && wv1 < Wp;
                if (wv0 < Wp) store_block(orowA, wv0, pA0, qA0);
                if (w1) store_block(orowA, wv1, pA1, qA1);
                if (two) {
                    if (wv0 < Wp) store_block(orowB, wv0, pB0, qB0);
                    if (w1) store_block(orowB, wv1, pB1, qB1);
                }
            }
        }
        __syncthreads();                       // next slab written; this one consumed
        if (++hc == hchunks) { hc = 0; if (++d == Dp) { d = 0; ++n; } }
    }
}

}  // namespace

constexpr size_t kSlabLdsMax = 48 * 1024;   // keep several workgroups resident per CU

template <int KS>
static hipError_t launch_ks(const float *x, const float *w, const float *conv_bias,
                            const float *bias, float s1, float s2, int64_t N, int64_t Cin,
                            int64_t D, int64_t H, int64_t W, int64_t Cout, float *out,
                            hipStream_t stream)
{
    const int Dp = (int)(D - 1), Hp = (int)(H - 1), Wp = (int)(W - 1);
    const int wblocks = (Wp + 15) / 16;
    int dev = 0, cus = 256, per_cu = 1;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 256;
    const unsigned gy = (unsigned)((Cout + 15) / 16);

    if constexpr (KS > 0) {
        // pooled rows per task: up to 16, as many as the LDS budget allows
        int TH = Hp < 16 ? Hp : 16;
        auto slab_bytes = [&](int th) { return (size_t)(KS * 64 + 2 * Cin * 2 * (th + 1) * W) * sizeof(float); };
        while (TH > 1 && slab_bytes(TH) > kSlabLdsMax) --TH;
        if (slab_bytes(TH) <= kSlabLdsMax) {
            const size_t lds = slab_bytes(TH);
            const int hchunks = (Hp + TH - 1) / TH;
            const int64_t ntasks = N * Dp * (int64_t)hchunks;
            const bool vec4 = (W % 4 == 0) && (((uintptr_t)x & 15) == 0);
            const void *fn = vec4 ? (const void *)fused3d_f32_slab_kernel<KS, 4>
                                  : (const void *)fused3d_f32_slab_kernel<KS, 1>;
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, lds) != hipSuccess ||
                per_cu < 1)
                per_cu = 1;
            int64_t wgs = (int64_t)cus * per_cu / gy;
            if (wgs < 1) wgs = 1;
            if (wgs > ntasks) wgs = ntasks;
            const int per = (int)((ntasks + wgs - 1) / wgs);
            const unsigned gx = (unsigned)((ntasks + per - 1) / per);
            if (vec4)
                hipLaunchKernelGGL((fused3d_f32_slab_kernel<KS, 4>), dim3(gx, gy), dim3(kThreads), lds,
                                   stream, x, w, conv_bias, bias, s1, s2, (int)Cin, (int)D, (int)H,
                                   (int)W, (int)Cout, Dp, Hp, Wp, TH, hchunks, (int)ntasks, per, out);
            else
                hipLaunchKernelGGL((fused3d_f32_slab_kernel<KS, 1>), dim3(gx, gy), dim3(kThreads), lds,
                                   stream, x, w, conv_bias, bias, s1, s2, (int)Cin, (int)D, (int)H,
                                   (int)W, (int)Cout, Dp, Hp, Wp, TH, hchunks, (int)ntasks, per, out);
            return hipGetLastError();
        }
    }
    // direct-load path (Cin > 4, or rows too wide for an LDS slab)
    const int64_t nmb = N * Dp * (int64_t)Hp * wblocks;   // < 2^31 (checked by the shim)
    const size_t lds = (size_t)(2 * Cin) * 64 * sizeof(float);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void *)fused3d_f32_kernel<KS>,
                                                     kThreads, lds) != hipSuccess || per_cu < 1)
        per_cu = 1;
    int64_t waves = (int64_t)cus * per_cu * kWaves / gy;
    const int64_t max_waves = (nmb + kMinMbPerWave - 1) / kMinMbPerWave;
    if (waves > max_waves) waves = max_waves;
    if (waves < kWaves) waves = kWaves;
    const int per = (int)((nmb + waves - 1) / waves);
    const unsigned gx = (unsigned)(((nmb + per - 1) / per + kWaves - 1) / kWaves);
    hipLaunchKernelGGL(fused3d_f32_kernel<KS>, dim3(gx, gy), dim3(kThreads), lds, stream, x, w,
                       conv_bias, bias, s1, s2, (int)Cin, (int)D, (int)H, (int)W, (int)Cout,
                       Dp, Hp, Wp, wblocks, (int)nmb, per, out);
    return hipGetLastError();
}

hipError_t launch_fused3d_f32(const float *x, const float *w,
                              const float *conv_bias, const float *bias,
                              float s1, float s2, int64_t N, int64_t Cin,
                              int64_t D, int64_t H, int64_t W, int64_t Cout,
                              float *out, hipStream_t stream)
{
    switch (Cin) {
    case 1: return launch_ks<2>(x, w, conv_bias, bias, s1, s2, N, Cin, D, H, W, Cout, out, stream);
    case 2: return launch_ks<4>(x, w, conv_bias, bias, s1, s2, N, Cin, D, H, W, Cout, out, stream);
    case 3: return launch_ks<6>(x, w, conv_bias, bias, s1, s2, N, Cin, D, H, W, Cout, out, stream);
    case 4: return launch_ks<8>(x, w, conv_bias, bias, s1, s2, N, Cin, D, H, W, Cout, out, stream);
    default: return launch_ks<0>(x, w, conv_bias, bias, s1, s2, N, Cin, D, H, W, Cout, out, stream);
    }
}

}  // namespace ct
