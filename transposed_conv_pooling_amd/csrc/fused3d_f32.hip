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
// fragments read from LDS.  This direct kernel also serves small calls with
// Cin <= 4; larger ones take the slab pipeline below.
#include "ct_internal.h"

namespace ct {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kMinMbPerWave = 4;  // do not split the work finer than this

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Weff^T fragments for output-channel block cob: wfrag[j*64 + l] =
// Weff[ci, co = cob*16 + l%16, tap] with kappa = 4j + l/16 = ci*8 + tap.
// A thread takes two entries per pass and issues both entries' 16 weight
// loads before summing, so with at most 2*kThreads entries (Cin <= 4) the
// whole filter costs one round trip to memory.
// One element of x or w as fp32: fp32 data as is, bf16 data (its 16-bit
// pattern) widened exactly.
__device__ __forceinline__ float ld_elem(const float *p) { return *p; }
__device__ __forceinline__ float ld_elem(const uint16_t *p) { return __uint_as_float((unsigned)*p << 16); }

template <typename E>
__device__ __forceinline__ void build_wfrag(const E *__restrict__ w, int Cout, int cob,
                                            int ksteps, float *wfrag)
{
    const int nent = ksteps * 64;
    for (int e0 = threadIdx.x; e0 < nent; e0 += 2 * kThreads) {
        float t8[2][8];
        int nk[2][3];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            // an entry past the end reads entry e0's weights (valid addresses,
            // so every load is unconditional) and is not written
            const int e = e0 + u * kThreads < nent ? e0 + u * kThreads : e0;
            const int j = e >> 6, l = e & 63;
            const int co = cob * 16 + (l & 15);
            const int kap = 4 * j + (l >> 4);
            const int ci = kap >> 3, tap = kap & 7;
            const int a = tap >> 2, b = (tap >> 1) & 1, c = tap & 1;
            const E *wp = w + ((int64_t)ci * Cout + min(co, Cout - 1)) * 27;
            // per axis: input offset 0 takes taps {1,2}, offset 1 takes tap {0}
            const int kd0 = a ? 0 : 1, kh0 = b ? 0 : 1, kw0 = c ? 0 : 1;
            nk[u][0] = a ? 1 : 2; nk[u][1] = b ? 1 : 2; nk[u][2] = c ? 1 : 2;
            // all 8 candidate taps of the 2x2x2 block starting at (kd0, kh0, kw0)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                    for (int k = 0; k < 2; ++k)
                        t8[u][(i * 2 + jj) * 2 + k] = ld_elem(wp + (kd0 + i) * 9 + (kh0 + jj) * 3 + kw0 + k);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int e = e0 + u * kThreads;
            if (e >= nent) continue;
            float v = 0.0f;
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                    for (int k = 0; k < 2; ++k)
                        if (i < nk[u][0] && jj < nk[u][1] && k < nk[u][2]) v += t8[u][(i * 2 + jj) * 2 + k];
            if (cob * 16 + (e & 15) >= Cout) v = 0.0f;
            wfrag[e] = v;
        }
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
// E: element type of x and w (fp32, or bf16 bit patterns widened exactly).
// OP: output padding 1: the pooled grid reaches the input's far edges
// (Dp = D, Hp = H, Wp = W) and a tap past an edge reads 0 ([p50]'s parity
// rule with the missing inputs taken as zero); without it every tap is in
// bounds and the loads carry no masks.
template <int KS, typename E, bool OP>
__global__ __launch_bounds__(kThreads)
void fused3d_f32_kernel(const E *__restrict__ x, const E *__restrict__ w,
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
    // which of a lane's taps (a, b, c) are past the far edges: the plane,
    // row and column offsets must stay below D, H and W
    auto tap_ok = [&](const Pos &q, int wv, int tap) {
        return !OP || (q.d + (tap >> 2) < D && q.h + ((tap >> 1) & 1) < H && wv + (tap & 1) < W);
    };

    if constexpr (KS > 0) {
        float a[KS];
        int off[KS], tp[KS];
#pragma unroll
        for (int j = 0; j < KS; ++j) {
            a[j] = wfrag[j * 64 + lane];
            const int kap = 4 * j + kq;
            const int ci = kap >> 3, tap = kap & 7;
            tp[j] = tap;
            off[j] = ci * DHW + (tap >> 2) * HW + ((tap >> 1) & 1) * W + (tap & 1);
        }
        auto load = [&](const Pos &q, float *v) {
            const int wv = min(q.wb * 16 + col, Wp - 1);   // masked lanes read a valid tap
            const E *xb = x + (int64_t)q.n * Cin * DHW + (int64_t)q.d * HW + q.h * W + wv;
#pragma unroll
            for (int j = 0; j < KS; ++j) {
                const bool ok = tap_ok(q, wv, tp[j]);
                const float t = ld_elem(ok ? xb + off[j] : x);
                v[j] = ok ? t : 0.0f;
            }
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
            const E *xb = x + (int64_t)p.n * Cin * DHW + (int64_t)p.d * HW + p.h * W + wv;
            v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
            for (int j0 = 0; j0 < ksteps; j0 += kChunk) {
                float xv[kChunk];
#pragma unroll
                for (int jj = 0; jj < kChunk; ++jj) {
                    const int kap = 4 * (j0 + jj) + kq;
                    const int ci = kap >> 3, tap = kap & 7;
                    const int cic = min(ci, Cin - 1);          // valid address; masked below
                    const bool ok = j0 + jj < ksteps && tap_ok(p, wv, tap);
                    const float v = ld_elem(ok ? xb + (int64_t)cic * DHW + (tap >> 2) * HW +
                                                     ((tap >> 1) & 1) * W + (tap & 1)
                                               : x);
                    xv[jj] = ok ? v : 0.0f;
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
// group).  The first slab's loads are issued before the filter build so the
// two latencies overlap.
//
// Output.  For one (n, co) the pooled outputs of all (d, h, w) form one
// contiguous stream of Dp*Hp*Wp floats, and consecutive tasks of a workgroup
// continue each of their 16 streams.  A task's results go to a staging row
// per channel in LDS, placed so that staging position p is the float at
// address line_base + 4p (line_base = the 128-byte line holding the task's
// first output of that stream).  The store phase then writes every complete
// 128-byte line with non-temporal 16-byte stores, and hands the unfinished
// last line (fewer than 32 floats) to the next task's staging row instead of
// writing it, so HBM sees whole lines; only a stream's first and last
// partial lines in a workgroup are written with plain stores (for L2 to
// merge with the neighbour's part).  Staging is double-buffered as well:
// one barrier per task separates a task's compute from its store phase.
constexpr int kSlabPrefetch = 4;   // slab pieces each loader lane keeps in flight
constexpr int kLine = 32;          // floats per 128-byte line
constexpr int kLineSlack = 2 * kLine;   // LDS floats after the staging sets (see the store waves)
// 4 compute waves, 2 loader waves, 2 store waves: 8 waves, so that three
// workgroups fit a CU's 32 wave slots (with at most 64 VGPRs a wave).  vmcnt counts a wave's
// loads and stores together and retires them in order, so a wave that both
// stores and prefetches would wait for its earlier stores before each slab;
// here only the loader waves load and only the store waves store.
constexpr int kLoadWaves = 2;
constexpr int kStoreWaves = 2;
constexpr int kRowsPerStoreWave = 16 / kStoreWaves;       // staging rows per store wave
constexpr int kLanesPerRow = 64 / kRowsPerStoreWave;      // lanes on one row (16 B each)
constexpr int kLinesPerStore = kLanesPerRow / 8;          // lines of a row per store instruction
constexpr int kLoadThreads = 64 * kLoadWaves;
constexpr int kSlabThreads = 64 * (kWaves + kLoadWaves + kStoreWaves);

template <int VEC> struct Vec;
template <> struct Vec<4> { typedef float4 T; };
template <> struct Vec<1> { typedef float T; };

// LDS layout sizes in floats (int64 so the host can size any geometry)
__host__ __device__ inline int64_t slab_floats(int64_t cin, int64_t th, int64_t w) { return cin * 2 * (th + 1) * w; }
// staging row stride: a leading partial line plus TH rows, a multiple of 4
// floats (16-byte aligned rows) plus 4 to spread the channels over banks
__host__ __device__ inline int64_t stage_stride(int64_t th, int64_t wp) { return ((kLine + th * wp + 3) & ~int64_t(3)) + 4; }
__host__ __device__ inline int64_t stage_offset(int64_t ks, int64_t cin, int64_t th, int64_t w)
{
    return (ks * 64 + 2 * slab_floats(cin, th, w) + 3) & ~int64_t(3);
}
// (plus two lines of slack: the store waves read whole pieces up to two lines
// past a staging row's end, for pieces they then do not store)
__host__ __device__ inline int64_t slab_lds_floats(int64_t ks, int64_t cin, int64_t th, int64_t w, int64_t wp)
{
    return stage_offset(ks, cin, th, w) + 2 * 16 * stage_stride(th, wp) + kLineSlack;
}

// GW > 0: the input width GW, the output padding GOP and the pooled rows per
// task GTH are compile-time constants (the page's geometries), so that row
// lengths, strides and trip counts fold into immediates; GW == 0: runtime.
template <int KS, int VEC, int GW = 0, int GTH = 0, int GOP = 0>
__global__ __launch_bounds__(kSlabThreads)
void fused3d_f32_slab_kernel(const float *__restrict__ x, const float *__restrict__ w,
                             const float *__restrict__ conv_bias,
                             const float *__restrict__ bias, float s1, float s2,
                             int Cin_, int D, int H, int W_, int SW_, int Cout,
                             int Dp, int Hp, int Wp_, int TH_, int hchunks, int ntasks,
                             int tasks_per_wg, float *__restrict__ out)
{
    static_assert(KS > 0, "the slab kernel has a compile-time channel count");
    (void)Cin_;                                // equal to KS / 2, passed for the launch record
    const int Cin = KS / 2;
    const int W = GW > 0 ? GW : W_;
    const int SW = GW > 0 ? GW + (GOP ? (VEC == 4 ? 4 : 1) : 0) : SW_;
    const int Wp = GW > 0 ? GW - 1 + GOP : Wp_;
    const int TH = GW > 0 ? GTH : TH_;
    typedef typename Vec<VEC>::T vec_t;
    extern __shared__ __attribute__((aligned(16))) float lds[];
    const int R = TH + 1;                      // input rows per plane in a slab
    const int sfl = (int)slab_floats(Cin, TH, SW);
    const int STR = (int)stage_stride(TH, Wp);
    float *wfrag = lds;                        // [KS][64]
    float *slabs = lds + KS * 64;              // 2 x [Cin][2][R][SW] (double buffer)
    float *stage = lds + stage_offset(KS, Cin, TH, SW);  // 2 x [16][STR]
    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const int cob = blockIdx.y;
    const int HW = H * W, DHW = D * HW;        // per-item sizes < 2^31 (checked by the shim)
    const int64_t pplane = (int64_t)Dp * Hp * Wp;

    // this workgroup's contiguous task range (n, d, hc), decoded once
    const int t_begin = uniform((int)min<int64_t>(xcd_remap(blockIdx.x, gridDim.x) * tasks_per_wg, ntasks));
    const int ntask = uniform(min(t_begin + tasks_per_wg, ntasks) - t_begin);
    int hc, d, n;
    {
        int t = t_begin;
        hc = uniform(t % hchunks); t /= hchunks;
        d = uniform(t % Dp);
        n = uniform(t / Dp);
    }
    auto next = [&](int &n_, int &d_, int &hc_) {
        if (++hc_ == hchunks) { hc_ = 0; if (++d_ == Dp) { d_ = 0; ++n_; } }
    };

    // With output_padding 1 the pooled grid reaches the input's far edges
    // (Dp = D, Hp = H, Wp = W): the taps x[d+1], x[h+1], x[w+1] past them
    // read 0 ([p50]'s parity rule with the missing inputs taken as zero).
    // Slab rows then carry SW - W >= 1 zero columns after the row, zeroed
    // here in both slab buffers (the loaders write only columns < W); rows
    // and planes past the input are zero-filled by the loaders.
    if (SW > W) {
        const int zc = SW - W;                 // zero columns per slab row
        for (int e = threadIdx.x; e < 2 * Cin * 2 * R * zc; e += kSlabThreads) {
            const int row = e / zc, c = e - row * zc;
            slabs[row * SW + W + c] = 0.0f;
        }
    }

    // Three roles, one pipeline stage per task, one barrier per stage (after
    // a first barrier that publishes the filter and the first slab).  In
    // stage s the loader waves put slab s+1 into LDS, the compute waves turn
    // slab s into staging row set s, and the store waves write staging set
    // s-1 to memory.  Each role runs its own loop over the same barriers, so
    // no role's registers are live in another's code.
    if (wave >= kWaves && wave < kWaves + kLoadWaves) {
        // ---- loader: slab pieces q = ((ci*2 + a)*R + r)*(W/VEC) + v --------
        const int ll = threadIdx.x - kThreads;  // 0 .. kLoadThreads-1
        const int WV = W / VEC;
        const int npieces = Cin * 2 * R * WV;
        // per piece: source offset, and destination offset * 256 + plane * 16
        // + slab row (a slab fits the LDS budget, so offsets are < 2^23, and
        // R <= 9); -1 marks "no piece"
        int src_off[kSlabPrefetch], dst_row[kSlabPrefetch];
#pragma unroll
        for (int i = 0; i < kSlabPrefetch; ++i) {
            const int q = ll + i * kLoadThreads;
            const int v = q % WV, t = q / WV;
            const int r = t % R, ca = t / R;
            const int a = ca & 1, ci = ca >> 1;
            src_off[i] = ci * DHW + a * HW + r * W + v * VEC;
            dst_row[i] = q < npieces ? (((ca * R + r) * SW + v * VEC) << 8) | (a << 4) | r : -1;
        }
        // Every fetch issues exactly kSlabPrefetch loads, all from valid
        // addresses (x[0..] for no piece, a row past H or a task past the
        // range), so the count of loads in flight is the same on every path
        // and each put waits only for its own batch.
        auto fetch = [&](vec_t *pre, int n_, int d_, int hc_, bool real) {
            const int h0 = hc_ * TH;
            const float *xb = x + (int64_t)n_ * Cin * DHW + (int64_t)d_ * HW + (int64_t)h0 * W;
#pragma unroll
            for (int i = 0; i < kSlabPrefetch; ++i) {
                const bool ok = real && dst_row[i] >= 0 && h0 + (dst_row[i] & 15) < H &&
                                d_ + ((dst_row[i] >> 4) & 1) < D;
                pre[i] = *reinterpret_cast<const vec_t *>(ok ? xb + src_off[i] : x);
            }
        };
        // writes a fetched slab (plus any pieces beyond the prefetch plan) into buf
        auto put = [&](float *buf, const vec_t *pre, int n_, int d_, int hc_) {
            const int h0 = hc_ * TH;
#pragma unroll
            for (int i = 0; i < kSlabPrefetch; ++i)
                if (dst_row[i] >= 0)
                    *reinterpret_cast<vec_t *>(buf + (dst_row[i] >> 8)) =
                        (h0 + (dst_row[i] & 15) < H && d_ + ((dst_row[i] >> 4) & 1) < D) ? pre[i] : vec_t{};
            for (int q = ll + kSlabPrefetch * kLoadThreads; q < npieces; q += kLoadThreads) {
                const int v = q % WV, tt = q / WV;
                const int r = tt % R, ca = tt / R;
                vec_t val = vec_t{};
                if (h0 + r < H && d_ + (ca & 1) < D)
                    val = *reinterpret_cast<const vec_t *>(
                        x + (int64_t)n_ * Cin * DHW + (int64_t)d_ * HW + (int64_t)h0 * W +
                        (ca >> 1) * DHW + (ca & 1) * HW + r * W + v * VEC);
                *reinterpret_cast<vec_t *>(buf + (ca * R + r) * SW + v * VEC) = val;
            }
        };
        vec_t pa[kSlabPrefetch], pb[kSlabPrefetch];
        // slab 0 now; slabs 1 and 2 in flight in registers
        int n1 = n, d1 = d, h1 = hc;
        fetch(pa, n1, d1, h1, ntask > 0);
        put(slabs, pa, n1, d1, h1);
        next(n1, d1, h1);
        fetch(pa, n1, d1, h1, ntask > 1);
        int n2 = n1, d2 = d1, h2 = h1;
        next(n2, d2, h2);
        fetch(pb, n2, d2, h2, ntask > 2);
        __syncthreads();
        // stage s: put slab s+1 (held in pa for even s, pb for odd s) into
        // buffer (s+1)&1, refill that register set with slab s+3
        for (int s = 0; s <= ntask; s += 2) {
            if (s + 1 < ntask) put(slabs + sfl, pa, n1, d1, h1);
            next(n1, d1, h1); next(n1, d1, h1);
            fetch(pa, n1, d1, h1, s + 3 < ntask);
            __syncthreads();
            if (s + 1 > ntask) break;
            if (s + 2 < ntask) put(slabs, pb, n2, d2, h2);
            next(n2, d2, h2); next(n2, d2, h2);
            fetch(pb, n2, d2, h2, s + 4 < ntask);
            __syncthreads();
        }
        return;
    }

    if (wave >= kWaves + kLoadWaves) {
        // ---- store waves: store wave k owns kRowsPerStoreWave staging rows;
        // lane l serves row k*kRowsPerStoreWave + l/kLanesPerRow with column
        // j = l%kLanesPerRow, so one store instruction writes kLinesPerStore
        // whole 128-byte lines of each of its rows and every per-row bound
        // is a per-lane value.  (Stores are spread over several waves: each
        // wave keeps at most 63 memory operations in flight, and
        // non-temporal stores are acknowledged late.)  `cont` says the lane's
        // row starts with a carried line head.  Task s-1 is stored in stage s.
        const int j = lane % kLanesPerRow;
        const int sc = (wave - kWaves - kLoadWaves) * kRowsPerStoreWave + lane / kLanesPerRow;
        const bool row_ok = cob * 16 + sc < Cout;
        // float offset of this row's channel plane within a batch item's output
        // (an item's output is below 2^31 bytes, checked by the shim)
        const int co_off = (cob * 16 + sc) * (int)pplane;
        const int item_bytes = Cout * (int)pplane * 4;
        // most store instructions a row needs: its whole lines, kLinesPerStore at a time
        const int kmax = ((kLine - 1 + TH * Wp) / kLine + kLinesPerStore - 1) / kLinesPerStore;
        constexpr int kTail = (kLine + kLanesPerRow - 1) / kLanesPerRow;
        constexpr int kStep = 4 * kLanesPerRow;                    // floats of a row per instruction
        constexpr unsigned kOff = 0x80000000u;                     // past any item: dropped
        bool cont = false;
        __syncthreads();
        __syncthreads();                       // stage 0: nothing to store yet
        int ns = n, ds = d, hs = hc;
        for (int s = 1; s <= ntask; ++s) {
            int nn = ns, dn = ds, hn = hs;
            next(nn, dn, hn);
            const bool next_same_n = s < ntask && nn == ns;  // task s continues the streams
            const int buf = (s - 1) & 1;
            const float *sr = stage + buf * 16 * STR + sc * STR;
            float *sn = stage + (buf ^ 1) * 16 * STR + sc * STR;
            const int h0 = hs * TH;
            const int len = min(TH, Hp - h0) * Wp;
            // stores go through a buffer resource over batch item ns's output;
            // a lane's row starts at float offset foff of the item
            const float *item = out + (int64_t)ns * Cout * pplane;
            const __amdgpu_buffer_rsrc_t rs =
                __builtin_amdgcn_make_buffer_rsrc((void *)item, 0, item_bytes, 0x00020000);
            const int foff = co_off + (ds * Hp + h0) * Wp;
            // staging positions [start, end) hold task s-1's outputs (and, if
            // continued, the carried line head [0, c0)); whole lines [lo, hi)
            // go out with non-temporal 16-byte stores, the partial head
            // [start, lo) with plain stores, the tail [hi, end) to the next
            // staging set or, where the stream ends here, to memory.  Position
            // p is the float at item offset gbase + p (gbase + p >= 0 for
            // every position that is stored: a carried head belongs to the
            // previous task of the same item).
            const int c0 = (int)((((uintptr_t)item >> 2) + (unsigned)foff) & (kLine - 1));
            const int gbase = foff - c0;                              // 128-byte aligned
            const int end = c0 + len;
            const int start = cont ? 0 : c0;
            const int lo = min((start + kLine - 1) & ~(kLine - 1), end);
            const int hi = max(lo, end & ~(kLine - 1));
            const int nf = row_ok ? (hi - lo) / 4 : 0;             // 16-byte pieces of whole lines
            // all reads go out before any store, so the wave waits for LDS once
            // (reads reach at most 2 lines past a staging row's data, for
            // pieces that are then not stored: the next row, or the slack at
            // the end of the LDS allocation)
            float tl[kTail];
#pragma unroll
            for (int u = 0; u < kTail; ++u) tl[u] = sr[hi + j + kLanesPerRow * u];
            // lo is a line boundary whenever nf > 0; (lo & ~3) keeps the 16-byte
            // reads aligned when nothing is stored
            const float *rb = sr + (lo & ~3) + 4 * j;
            const int ob = (gbase + lo + 4 * j) * 4;
            for (int k0 = 0; k0 < kmax; k0 += 4) {
                v4f v[4];
#pragma unroll
                for (int u = 0; u < 4; ++u)   // (pieces past kmax re-read the last one)
                    v[u] = *reinterpret_cast<const v4f *>(rb + min(k0 + u, kmax - 1) * kStep);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const bool ok = (k0 + u) * kLanesPerRow + j < nf;
                    __builtin_amdgcn_raw_buffer_store_b128(
                        __builtin_bit_cast(u32x4, v[u]), rs,
                        ok ? (unsigned)(ob + (k0 + u) * kStep * 4) : kOff, 0, 2 /* non-temporal */);
                }
            }
            if (row_ok)
                for (int p = start + j; p < lo; p += kLanesPerRow)       // head: partial line
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sr[p]), rs, (gbase + p) * 4, 0, 0);
            // tail [hi, end): fewer than 32 floats
#pragma unroll
            for (int u = 0; u < kTail; ++u) {
                const int p = hi + j + kLanesPerRow * u;
                if (p < end) {
                    if (next_same_n) sn[p - hi] = tl[u];                     // carried
                    else if (row_ok)                                           // partial line
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(tl[u]), rs, (gbase + p) * 4, 0, 0);
                }
            }
            // the next task's row starts with a carried line unless this
            // task's last line was written as a head
            cont = next_same_n && (hi < end || (end & (kLine - 1)) == 0);
            __syncthreads();
            ns = nn; ds = dn; hs = hn;
        }
        return;
    }

    // ---- compute waves: task s in stage s, MFMA into staging set s&1 ------
    const int col = lane & 15;
    const int kq = lane >> 4;
    const int wblocks = (Wp + 15) / 16;
    // The MFMA runs with the operands swapped, D = S^T (16 voxels x 16
    // channels): lane (kq, col) then holds voxels 4kq .. 4kq+3 of its block
    // for channel cob*16 + col, four consecutive outputs of one channel.
    // folded epilogue ((S/8 + cb)*s1 + b)*s2 = S*alpha + beta[co]; the bias
    // loads go out with the filter's, in the same round trip
    const float alpha = 0.125f * s1 * s2;
    const int co_l = cob * 16 + col;
    const bool co_ok = co_l < Cout;
    const float cbv = conv_bias && co_ok ? conv_bias[co_l] : 0.0f;
    const float bv = bias && co_ok ? bias[co_l] : 0.0f;
    build_wfrag(w, Cout, cob, KS, wfrag);
    const float beta = (cbv * s1 + bv) * s2;
    int soff[KS];
#pragma unroll
    for (int j = 0; j < KS; ++j) {
        const int kap = 4 * j + kq;
        const int ci = kap >> 3, tap = kap & 7;
        soff[j] = ((ci * 2 + (tap >> 2)) * R + ((tap >> 1) & 1)) * SW + (tap & 1);
    }
    const int co_off = co_l * (int)pplane;    // per-item output offsets fit in int32 (checked by the shim)
    __syncthreads();                           // filter and first slab visible
    float a[KS];
#pragma unroll
    for (int j = 0; j < KS; ++j) a[j] = wfrag[j * 64 + lane];

    for (int s = 0; s <= ntask; ++s) {
        if (s < ntask) {
            const int buf = s & 1;
            const float *cur = slabs + buf * sfl;
            float *stg = stage + buf * 16 * STR;
            const int h0 = hc * TH;
            const int rows = min(TH, Hp - h0);
            float *ob = out + (int64_t)n * Cout * pplane + ((int64_t)d * Hp + h0) * Wp;
            // staging row of channel co starts at its line base: the task's
            // first output sits at its float index within its 128-byte line
            float *srow = stg + col * STR + (int)(((uintptr_t)(ob + co_off) >> 2) & (kLine - 1)) + 4 * kq;
            // each wave takes rows hh = wave, wave + 4, ... one at a time; a
            // row's w-blocks go in pairs, each block's K range split over two
            // accumulators: four independent MFMA chains in flight, with all
            // their LDS reads issued first.  (One row, not two, per pass keeps
            // every role within 64 VGPRs: three 8-wave workgroups per CU.)
            // (block voxels 4kq+r at w = wv0 + r of the block start wv0)
            auto stage_block = [&](int hh, int wv0, const v4f &p, const v4f &q) {
                float *dst = srow + hh * Wp + wv0;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (co_ok && wv0 + 4 * kq + r < Wp) dst[r] = __builtin_fmaf(p[r] + q[r], alpha, beta);
            };
            for (int hh = wave; hh < rows; hh += kWaves) {
                const float *srowA = cur + hh * SW;
                for (int wb = 0; wb < wblocks; wb += 2) {
                    const int wv0 = wb * 16 + col, wv1 = wv0 + 16;
                    const int wc0 = min(wv0, Wp - 1), wc1 = min(wv1, Wp - 1);
                    float a0[KS], a1[KS];
#pragma unroll
                    for (int j = 0; j < KS; ++j) {
                        a0[j] = srowA[wc0 + soff[j]];
                        a1[j] = srowA[wc1 + soff[j]];
                    }
                    v4f pA0 = {0.0f, 0.0f, 0.0f, 0.0f}, qA0 = pA0, pA1 = pA0, qA1 = pA0;
#pragma unroll
                    for (int j = 0; j < KS; j += 2) {
                        pA0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a0[j], a[j], pA0, 0, 0, 0);
                        pA1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a1[j], a[j], pA1, 0, 0, 0);
                        qA0 = __builtin_amdgcn_mfma_f32_16x16x4f32(a0[j + 1], a[j + 1], qA0, 0, 0, 0);
                        qA1 = __builtin_amdgcn_mfma_f32_16x16x4f32(a1[j + 1], a[j + 1], qA1, 0, 0, 0);
                    }
                    stage_block(hh, wb * 16, pA0, qA0);
                    if (wb + 1 < wblocks) stage_block(hh, wb * 16 + 16, pA1, qA1);
                }
            }
            next(n, d, hc);
        }
        __syncthreads();
    }
}

}  // namespace

constexpr size_t kSlabLdsMax = 52 * 1024;   // three workgroups per CU (160 KB of LDS)

// Pooled rows per slab task and the slab row stride for a geometry, or
// TH = 0 when no slab fits the LDS budget.  Output padding 1 adds zero
// columns after each slab row (4, keeping rows 16-byte aligned, when the
// rows are loaded as float4).
static void slab_plan(int ks, int64_t Cin, int64_t H, int64_t W, int op, bool vec4, int *TH_out,
                      int *SW_out)
{
    const int Hp = (int)(H - 1 + op), Wp = (int)(W - 1 + op);
    const int SW = (int)W + (op ? (vec4 ? 4 : 1) : 0);
    int TH = Hp < 8 ? Hp : 8;
    auto bytes = [&](int th) { return (size_t)slab_lds_floats(ks, Cin, th, SW, Wp) * sizeof(float); };
    while (TH > 1 && bytes(TH) > kSlabLdsMax) --TH;
    *TH_out = bytes(TH) <= kSlabLdsMax ? TH : 0;
    *SW_out = SW;
}

static bool slab_vec4(int64_t W, const float *x) { return (W % 4 == 0) && (((uintptr_t)x & 15) == 0); }

// The direct kernel: waves walk contiguous ranges of 16-voxel blocks and
// load their taps straight from memory (Cin > 4, rows too wide for an LDS
// slab, a small call, or bf16 data the bf16 kernel does not take).
template <int KS, typename E>
static hipError_t launch_direct(const E *x, const E *w, const float *conv_bias, const float *bias,
                                float s1, float s2, int64_t N, int64_t Cin, int64_t D, int64_t H,
                                int64_t W, int64_t Cout, int op, float *out, hipStream_t stream)
{
    const void *fn = op ? (const void *)fused3d_f32_kernel<KS, E, true>
                        : (const void *)fused3d_f32_kernel<KS, E, false>;
    const int Dp = (int)(D - 1 + op), Hp = (int)(H - 1 + op), Wp = (int)(W - 1 + op);
    const int wblocks = (Wp + 15) / 16;
    const unsigned gy = (unsigned)((Cout + 15) / 16);
    const int64_t nmb = N * Dp * (int64_t)Hp * wblocks;   // < 2^31 (checked by the shim)
    const size_t lds = (size_t)(2 * Cin) * 64 * sizeof(float);
    const int per_cu = occupancy(fn, kThreads, lds);
    int64_t waves = (int64_t)device_cus() * per_cu * kWaves / gy;
    const int64_t max_waves = (nmb + kMinMbPerWave - 1) / kMinMbPerWave;
    if (waves > max_waves) waves = max_waves;
    if (waves < kWaves) waves = kWaves;
    const int per = (int)((nmb + waves - 1) / waves);
    const unsigned gx = (unsigned)(((nmb + per - 1) / per + kWaves - 1) / kWaves);
    int a_cin = (int)Cin, a_d = (int)D, a_h = (int)H, a_w = (int)W, a_cout = (int)Cout, a_dp = Dp,
        a_hp = Hp, a_wp = Wp, a_wb = wblocks, a_nmb = (int)nmb, a_per = per;
    void *args[] = {(void *)&x, (void *)&w, (void *)&conv_bias, (void *)&bias, &s1, &s2, &a_cin,
                    &a_d, &a_h, &a_w, &a_cout, &a_dp, &a_hp, &a_wp, &a_wb, &a_nmb, &a_per,
                    (void *)&out};
    return hipLaunchKernel(fn, dim3(gx, gy), dim3(kThreads), args, lds, stream);
}

template <int KS>
static hipError_t launch_ks(const float *x, const float *w, const float *conv_bias,
                            const float *bias, float s1, float s2, int64_t N, int64_t Cin,
                            int64_t D, int64_t H, int64_t W, int64_t Cout, int op, float *out,
                            hipStream_t stream)
{
    const int Dp = (int)(D - 1 + op), Hp = (int)(H - 1 + op), Wp = (int)(W - 1 + op);
    const int wblocks = (Wp + 15) / 16;
    const int cus = device_cus();
    int per_cu = 1;
    const unsigned gy = (unsigned)((Cout + 15) / 16);

    if constexpr (KS > 0) {
        const bool vec4 = slab_vec4(W, x);
        int TH, SW;
        slab_plan(KS, Cin, H, W, op, vec4, &TH, &SW);
        // Small calls (fewer than 48 blocks of 16 outputs x 16 channels per CU)
        // finish sooner on the direct kernel, which has no pipeline to fill:
        // the small page workload [2,3,8,16,16] takes 4.3 against 5.0 us per
        // call replayed from a graph, and the two meet near 48 blocks per CU.
        const int64_t blocks = N * Dp * (int64_t)Hp * wblocks * gy;
        const bool small = op == 0 && blocks < 48 * (int64_t)cus;
        if (TH > 0 && !small) {
            const size_t lds = (size_t)slab_lds_floats(KS, Cin, TH, SW, Wp) * sizeof(float);
            const int hchunks = (Hp + TH - 1) / TH;
            const int64_t ntasks = N * Dp * (int64_t)hchunks;
            // the page's geometries (W = 32, fp32 rows 16-byte aligned) take
            // instantiations with the geometry folded in
            const void *fn = vec4 ? (const void *)fused3d_f32_slab_kernel<KS, 4>
                                  : (const void *)fused3d_f32_slab_kernel<KS, 1>;
            if constexpr (KS == 6) {
                if (vec4 && W == 32 && op == 0 && TH == 8)
                    fn = (const void *)fused3d_f32_slab_kernel<KS, 4, 32, 8, 0>;
                else if (vec4 && W == 32 && op == 1 && TH == 7)
                    fn = (const void *)fused3d_f32_slab_kernel<KS, 4, 32, 7, 1>;
            }
            per_cu = occupancy(fn, kSlabThreads, lds);
            int64_t wgs = (int64_t)cus * per_cu / gy;
            if (wgs < 1) wgs = 1;
            if (wgs > ntasks) wgs = ntasks;
            const int per = (int)((ntasks + wgs - 1) / wgs);
            const unsigned gx = (unsigned)((ntasks + per - 1) / per);
            int a_cin = (int)Cin, a_d = (int)D, a_h = (int)H, a_w = (int)W, a_sw = SW,
                a_cout = (int)Cout, a_dp = Dp, a_hp = Hp, a_wp = Wp, a_th = TH, a_hc = hchunks,
                a_nt = (int)ntasks, a_per = per;
            void *args[] = {(void *)&x, (void *)&w, (void *)&conv_bias, (void *)&bias, &s1, &s2,
                            &a_cin, &a_d, &a_h, &a_w, &a_sw, &a_cout, &a_dp, &a_hp, &a_wp, &a_th,
                            &a_hc, &a_nt, &a_per, (void *)&out};
            return hipLaunchKernel(fn, dim3(gx, gy), dim3(kSlabThreads), args, lds, stream);
        }
    }
    return launch_direct<KS, float>(x, w, conv_bias, bias, s1, s2, N, Cin, D, H, W, Cout, op, out,
                                    stream);
}

hipError_t launch_fused3d_f32(const float *x, const float *w,
                              const float *conv_bias, const float *bias,
                              float s1, float s2, int64_t N, int64_t Cin,
                              int64_t D, int64_t H, int64_t W, int64_t Cout, int op,
                              float *out, hipStream_t stream)
{
    switch (Cin) {
    case 1: return launch_ks<2>(x, w, conv_bias, bias, s1, s2, N, Cin, D, H, W, Cout, op, out, stream);
    case 2: return launch_ks<4>(x, w, conv_bias, bias, s1, s2, N, Cin, D, H, W, Cout, op, out, stream);
    case 3: return launch_ks<6>(x, w, conv_bias, bias, s1, s2, N, Cin, D, H, W, Cout, op, out, stream);
    case 4: return launch_ks<8>(x, w, conv_bias, bias, s1, s2, N, Cin, D, H, W, Cout, op, out, stream);
    default: return launch_ks<0>(x, w, conv_bias, bias, s1, s2, N, Cin, D, H, W, Cout, op, out, stream);
    }
}

hipError_t launch_fused3d_direct_bf16(const uint16_t *x, const uint16_t *w,
                                      const float *conv_bias, const float *bias, float s1,
                                      float s2, int64_t N, int64_t Cin, int64_t D, int64_t H,
                                      int64_t W, int64_t Cout, int op, float *out,
                                      hipStream_t stream)
{
    switch (Cin) {
    case 1: return launch_direct<2>(x, w, conv_bias, bias, s1, s2, N, Cin, D, H, W, Cout, op, out, stream);
    case 2: return launch_direct<4>(x, w, conv_bias, bias, s1, s2, N, Cin, D, H, W, Cout, op, out, stream);
    case 3: return launch_direct<6>(x, w, conv_bias, bias, s1, s2, N, Cin, D, H, W, Cout, op, out, stream);
    case 4: return launch_direct<8>(x, w, conv_bias, bias, s1, s2, N, Cin, D, H, W, Cout, op, out, stream);
    default: return launch_direct<0>(x, w, conv_bias, bias, s1, s2, N, Cin, D, H, W, Cout, op, out, stream);
    }
}

}  // namespace ct
