// fused3d_bf16.hip - ConvTranspose3d(k3, s2, p1) -> *scale1 -> AvgPool3d(2)
// -> +bias -> *scale2 with bf16 x and w, fp32 accumulation and output, on the
// gfx950 bf16 matrix cores (v_mfma_f32_16x16x32_bf16).
//
// Method ([p50] "Kimi-K2.6 l2_p50"): as the fp32 kernel - each pooled voxel
// is S/8 with S = sum_ci sum_{a,b,c in {0,1}} x[ci,d+a,h+b,w+c] *
// Weff[ci,co,abc], Weff the per-tap sums of the 27 weights (passages on the
// stride-2 parity rule and on grouping the 27 terms by input tap), then the
// model's epilogue ((S/8 + conv_bias)*scale1 + bias)*scale2, evaluated in the
// folded form S*(scale1*scale2/8) + (conv_bias*scale1 + bias)*scale2 the page
// derives (one fma per output; within an ulp or two of the literal order).
//
// Precision.  Weff is summed in fp32 from the bf16 weights and split as
// Weff = hi + lo with hi = bf16(Weff), lo = bf16(Weff - hi); both halves go
// through the MFMA against the same bf16 x, so every product is exact in the
// fp32 accumulator and the filter is represented to ~2^-17 relative (a single
// bf16 rounding of Weff would cost 2^-9).
//
// MI355X mapping (16x16x32 MFMA, D = A * B):
//   A (16 x 32) = Weff^T: row co = l%16, 8 consecutive kappa per lane group
//   B (32 x 16) = X:      col voxel = l%16, the same 8 kappa per lane group
//   D (16 x 16) = S[co][voxel], lane l holds rows 4*(l/16)+r, column l%16
// with kappa = tap*Cin8 + ci (Cin8 = Cin rounded up to 8), so a lane group's
// 8 kappas are 8 consecutive channels at one tap: with the input slab held
// channels-last in LDS that is one 16-byte ds_read_b128.
//  * Workgroup = 8 waves, persistent, one 64-channel output group
//    (blockIdx.y).  Prologue: every thread forms Weff and its hi/lo split
//    for its (ci, co) pairs into a [half][tap][co][ci] table, from which each
//    wave loads its fragments (2 output-channel blocks x all k-steps x
//    hi/lo) into registers for the whole kernel.  With 25..32 input
//    channels, Cout a multiple of 64 and 16-byte aligned weights, the group's
//    weights are read as whole lines into an LDS copy (two 16-channel
//    halves) and the table is written in fragment order; with fewer input
//    channels and one 64-channel group a thread reads its pairs' 54 weights
//    straight into registers; otherwise the raw weights are staged in LDS in
//    16-channel chunks.
//  * Tile = (n, d, 8 pooled rows): the input slab x[n, :, d..d+1, h0..h0+8, :]
//    is transposed to [plane][row][w][ci] in a double-buffered LDS slab.  A
//    tile's loads are issued two tiles ahead into registers and written to
//    the spare buffer one tile ahead; one barrier per tile.
//  * Wave = (voxel-block slot s = w%4, channel pair p = w/4): each B read
//    feeds 4 MFMAs (2 channel blocks x hi/lo).
//  * Each workgroup walks a contiguous range of tiles in (n, row chunk, d)
//    order, so consecutive tiles share an input plane and its second read
//    hits the same XCD's L2; the workgroup index is remapped so that
//    neighbouring ranges also run on one XCD.
#include "ct_internal.h"

namespace ct {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kCoGroup = 64;          // output channels per workgroup
constexpr int kCiChunk = 16;          // input channels staged per prologue pass
constexpr int kPrefetch = 3;          // slab pieces (2 channels x 8 w) prefetched per thread

__device__ __forceinline__ float bf16_to_f32(unsigned short b)
{
    return __uint_as_float(((unsigned)b) << 16);
}

// round to nearest even (one v_cvt_pk_bf16_f32 on gfx950); NaN stays a NaN
__device__ __forceinline__ unsigned short f32_to_bf16(float f)
{
    return __builtin_bit_cast(unsigned short, (__bf16)f);
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Byte sizes of the LDS regions (shared with the launcher).
__host__ __device__ constexpr int raw_bytes() { return kCiChunk * kCoGroup * 27 * 2; }
__host__ __device__ constexpr int afrag_bytes(int ksteps) { return 2 * 8 * kCoGroup * (4 * ksteps + 8) * 2; }
// one slab: 2 planes x (th + 1) rows x W positions x cs channels (u16)
__host__ __device__ inline int slab_bytes(int th, int W, int cs) { return 2 * (th + 1) * W * cs * 2; }
// The epilogue constants sit after the larger of the prologue regions and the
// two slabs, so neither overwrites them.
__host__ __device__ inline int epi_offset(int th, int W, int cs)
{
    const int a = raw_bytes() + afrag_bytes(8), b = 2 * slab_bytes(th, W, cs);
    return ((a > b ? a : b) + 15) & ~15;
}

// kWB > 0: the output rows' 16-voxel block count (Wp + 15) / 16 known at
// compile time (2 for the page's W = 32), so a wave's voxel-block loop has a
// fixed trip count and every tile issues a fixed number of stores; 0: runtime.
template <int KSTEPS, int kTH, int kWB>
__global__ __launch_bounds__(kThreads)
void fused3d_bf16_kernel(const unsigned short *__restrict__ x,
                         const unsigned short *__restrict__ w,
                         const float *__restrict__ conv_bias,
                         const float *__restrict__ bias, float s1, float s2,
                         int Cin, int D, int H, int W, int Cout,
                         int Dp, int Hp, int Wp, int hpairs, int ntiles, int tiles_per_wg,
                         float *__restrict__ out)
{
    constexpr int Cin8 = 4 * KSTEPS;
    constexpr int CS = Cin8 + 8;              // channel stride of a slab position (u16)
    constexpr int kRows = kTH + 1;            // input rows per plane in a slab
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_bytes[];
    unsigned short *lds = reinterpret_cast<unsigned short *>(lds_bytes);
    unsigned short *raw = lds;                                // prologue: raw weights
    unsigned short *slab = lds;                               // main loop: input slab
    float *epi = reinterpret_cast<float *>(lds_bytes + epi_offset(kTH, W, CS));   // [64]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int g = lane >> 4;                 // lane group
    const int col = lane & 15;
    const int slot = wave & 3;               // voxel-block slot
    const int cp = wave >> 2;                // channel-block pair
    const int co0 = blockIdx.y * kCoGroup;
    const int ncog = min(kCoGroup, Cout - co0);
    const int HW = H * W, DHW = D * HW;      // per-item sizes < 2^31 (checked by the shim)
    const int64_t pplane = (int64_t)Dp * Hp * Wp;

    // ---- this workgroup's tiles, and the first slab's loads ---------------
    // workgroups of one XCD take consecutive ranges, so the input plane two
    // neighbouring ranges share is fetched into that XCD's L2 once
    const int t_begin = uniform((int)xcd_remap(blockIdx.x, gridDim.x) * tiles_per_wg);
    const int t_end = uniform(min(t_begin + tiles_per_wg, ntiles));
    int hp, d, n;
    {
        int t = t_begin;
        // tile order (n, row chunk, d), d fastest: a workgroup's consecutive
        // tiles share an input plane, whose second read then hits its L2
        d = uniform(t % Dp); t /= Dp;
        hp = uniform(t % hpairs);
        n = uniform(t / hpairs);
    }
    // tile-invariant staging plan: piece q = ((a*kRows + row)*W8 + w8)*(Cin8/2) + cpair
    // covers channels 2*cpair, 2*cpair+1 at x[.., d+a, h0+row, 8*w8 .. 8*w8+7]
    const int W8 = W >> 3;
    const int npieces = 2 * kRows * W8 * (Cin8 / 2);
    int src_off[kPrefetch], dst_off[kPrefetch], prow[kPrefetch], pci[kPrefetch];
#pragma unroll
    for (int i = 0; i < kPrefetch; ++i) {
        const int q = tid + i * kThreads;
        const int cpair = q % (Cin8 / 2);
        int t = q / (Cin8 / 2);
        const int w8 = t % W8;
        t /= W8;
        const int row = t % kRows, a = t / kRows;
        pci[i] = 2 * cpair;
        src_off[i] = 2 * cpair * DHW + a * HW + row * W + 8 * w8;
        dst_off[i] = ((a * kRows + row) * W + 8 * w8) * CS + 2 * cpair;
        prow[i] = q < npieces ? row : 1 << 30;
    }
    u16x8 pre0[kPrefetch], pre1[kPrefetch];
    int pok[kPrefetch];
    auto fetch = [&](int n_, int d_, int hp_) {
        const int h0 = kTH * hp_;
        const unsigned short *xb = x + (int64_t)n_ * Cin * DHW + (int64_t)d_ * HW + (int64_t)h0 * W;
        // unconditional loads from valid addresses (x[0..] for masked pieces) so
        // they all stay in flight; the zero fill happens in put()
#pragma unroll
        for (int i = 0; i < kPrefetch; ++i) {
            const bool rok = h0 + prow[i] < H;
            pre0[i] = *reinterpret_cast<const u16x8 *>((rok && pci[i] < Cin) ? xb + src_off[i] : x);
            pre1[i] = *reinterpret_cast<const u16x8 *>((rok && pci[i] + 1 < Cin) ? xb + src_off[i] + DHW : x);
            pok[i] = (rok ? 1 : 0) | ((rok && pci[i] < Cin) ? 2 : 0) | ((rok && pci[i] + 1 < Cin) ? 4 : 0);
        }
    };
    auto put = [&](unsigned short *buf, int off, u16x8 v0, u16x8 v1) {
        unsigned *dst = reinterpret_cast<unsigned *>(buf + off);     // 2 channels per dword
#pragma unroll
        for (int k = 0; k < 8; ++k)
            dst[k * (CS / 2)] = (unsigned)v0[k] | ((unsigned)v1[k] << 16);
    };
    // slab staging: all pieces of a tile into one slab buffer
    const int slab_u16 = slab_bytes(kTH, W, CS) / 2;
    const u16x8 z8 = {0, 0, 0, 0, 0, 0, 0, 0};
    auto put_all = [&](unsigned short *buf, int n_, int d_, int hp_) {
        const int h0 = kTH * hp_;
#pragma unroll
        for (int i = 0; i < kPrefetch; ++i)
            if (prow[i] < (1 << 30))
                put(buf, dst_off[i], (pok[i] & 2) ? pre0[i] : z8, (pok[i] & 4) ? pre1[i] : z8);
        for (int q = tid + kPrefetch * kThreads; q < npieces; q += kThreads) {
            const int cpair = q % (Cin8 / 2);
            int tt = q / (Cin8 / 2);
            const int w8 = tt % W8;
            tt /= W8;
            const int row = tt % kRows, a = tt / kRows;
            const int ci = 2 * cpair;
            const unsigned short *src = x + (int64_t)n_ * Cin * DHW + (int64_t)d_ * HW +
                                        (int64_t)h0 * W + ci * DHW + a * HW + row * W + 8 * w8;
            const bool rok = h0 + row < H;
            const u16x8 v0 = (rok && ci < Cin) ? *reinterpret_cast<const u16x8 *>(src) : z8;
            const u16x8 v1 = (rok && ci + 1 < Cin) ? *reinterpret_cast<const u16x8 *>(src + DHW) : z8;
            put(buf, ((a * kRows + row) * W + 8 * w8) * CS + ci, v0, v1);
        }
    };
    auto next_pos = [&](int &n_, int &d_, int &hp_) {
        if (++d_ == Dp) { d_ = 0; if (++hp_ == hpairs) { hp_ = 0; ++n_; } }
    };

    // ---- prologue: Weff hi/lo -------------------------------------------
    // weffT[h][tap][col][ci] (row stride Cin8 + 8 u16: rows 16-byte aligned
    // for the fragment reads)
    constexpr int WS = Cin8 + 8;
    unsigned short *weffT = lds + raw_bytes() / 2;
    // The 27 weights of pair (ci, col) -> Weff for the 8 input taps, split
    // into bf16 hi and lo.  Per axis, input offset 0 takes kernel taps {1,2}
    // and offset 1 takes tap {0}; the 3-D sum is done axis by axis.
    auto emit = [&](const float (&wv)[27], int cl, int ci) {
        float s1w[9][2];
#pragma unroll
        for (int r = 0; r < 9; ++r) {
            s1w[r][0] = wv[r * 3 + 1] + wv[r * 3 + 2];
            s1w[r][1] = wv[r * 3 + 0];
        }
        float s2w[3][2][2];
#pragma unroll
        for (int kd = 0; kd < 3; ++kd)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                s2w[kd][0][c] = s1w[kd * 3 + 1][c] + s1w[kd * 3 + 2][c];
                s2w[kd][1][c] = s1w[kd * 3 + 0][c];
            }
#pragma unroll
        for (int tap = 0; tap < 8; ++tap) {
            const int a = tap >> 2, b = (tap >> 1) & 1, c = tap & 1;
            const float we = a ? s2w[0][b][c] : (s2w[1][b][c] + s2w[2][b][c]);
            const unsigned short hi = f32_to_bf16(we);
            weffT[((0 * 8 + tap) * kCoGroup + cl) * WS + ci] = hi;
            weffT[((1 * 8 + tap) * kCoGroup + cl) * WS + ci] = f32_to_bf16(we - bf16_to_f32(hi));
        }
    };
    // Direct path (one 64-channel group, 4-byte aligned w): couple q holds the
    // pairs (ci, 2m) and (ci, 2m+1), q = 32*ci + m, whose 54 weights are the
    // 27 consecutive dwords q*27 .. q*27+26 of w.  Every thread loads its (at
    // most two) couples before the first slab's loads are issued, so the
    // weights return first; the filter is formed straight from registers.
    constexpr int kCouples = Cin8 * kCoGroup / 2;
    constexpr int kCouplesPerThread = (kCouples + kThreads - 1) / kThreads;
    // Line path (Cin8 = 32, Cout a multiple of 64, 16-byte aligned w): the
    // group's 32 x 64 x 27 weights are read as whole 128-byte lines (16 bytes
    // a lane, consecutive lanes consecutive pieces) in two halves of 16 input
    // channels, copied to LDS, and each thread forms Weff for input channels
    // (ci, ci+1) of one output channel from aligned dwords of that copy.  The
    // per-couple reads of the couple path below touch a 128-byte line per
    // lane and instruction, which held the prologue to ~4.6 us at the page's
    // wide workload; formed this way the filter is ready ~2 us sooner.  The
    // hi/lo halves go straight into fragment order, [cb][k-step][half][lane]
    // x 16 bytes, so each lane's fragments are consecutive 16-byte reads.
    constexpr bool kLinePath = (Cin8 == 32);
    constexpr int kRawRow = kCoGroup * 27 + 16;       // u16 per input channel in the copy (+16: banks)
    constexpr int kRawPieces = 16 * kCoGroup * 27 * 2 / 16;   // 16-byte pieces per half
    constexpr int kRawPR = (kRawPieces + kThreads - 1) / kThreads;
    constexpr int kTabBytes = 4 * 8 * 2 * 64 * 16;    // fragment-order table at LDS 0
    static_assert(!kLinePath || kTabBytes + 16 * kRawRow * 2 <= raw_bytes() + afrag_bytes(8),
                  "line-path prologue exceeds the prologue regions");
    const bool direct_w = kLinePath
                              ? (Cout % kCoGroup == 0) && ((((uintptr_t)w) & 15) == 0)
                              : (Cout == kCoGroup) && ((((uintptr_t)w) & 3) == 0);
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    unsigned wd[kLinePath ? 1 : kCouplesPerThread][27];
    u32x4 rw[kLinePath ? 2 : 1][kLinePath ? kRawPR : 1];
    if (direct_w) {
        if constexpr (kLinePath) {
            // piece p of half h: input channel 16h + p/216, bytes 16*(p%216)
            // of its 64*27 weights (contiguous: Cout is a multiple of 64)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int r = 0; r < kRawPR; ++r) {
                    const int p = tid + r * kThreads;
                    const int ci = 16 * h + p / 216;
                    const bool ok = p < kRawPieces && ci < Cin;
                    const unsigned short *src = ok ? w + ((int64_t)ci * Cout + co0) * 27 + 8 * (p % 216) : w;
                    rw[h][r] = *reinterpret_cast<const u32x4 *>(src);
                }
        } else {
            const unsigned *w32 = reinterpret_cast<const unsigned *>(w);
#pragma unroll
            for (int j = 0; j < kCouplesPerThread; ++j) {
                const int q = tid + j * kThreads;
                // unconditional loads (couples past Cin read couple 0, zeroed below)
                const unsigned *src = w32 + ((q < kCouples && (q >> 5) < Cin) ? q * 27 : 0);
#pragma unroll
                for (int k = 0; k < 27; ++k) wd[j][k] = src[k];
            }
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (t_begin < t_end) fetch(n, d, hp);
    int n2 = n, d2 = d, hp2 = hp;   // the next tile to stage
    const bool early_slab = !kLinePath && direct_w && slab_bytes(kTH, W, CS) <= raw_bytes();

    if (direct_w && kLinePath) {
        unsigned short *rawc = lds + kTabBytes / 2;
        unsigned *tab = reinterpret_cast<unsigned *>(lds);
        // forming thread: wave -> channel block fcb and input-channel quad
        // fcq; lane -> output channel 16*fcb + col, input channels
        // 16h + 8*fcq + 2*g + {0, 1}: dword g of the fragment of lane
        // (fcq + 2h, col) of block fcb
        const int fcb = wave & 3, fcq = wave >> 2;
        const int fco = 16 * fcb + col;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if (h == 1) __syncthreads();                       // half 0's copy consumed
#pragma unroll
            for (int r = 0; r < kRawPR; ++r) {
                const int p = tid + r * kThreads;
                if (p < kRawPieces) {
                    const u32x4 v = (16 * h + p / 216) < Cin ? rw[h][r] : u32x4{0u, 0u, 0u, 0u};
                    *reinterpret_cast<u32x4 *>(rawc + (p / 216) * kRawRow + 8 * (p % 216)) = v;
                }
            }
            __syncthreads();
            float we[2][8];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                // the record's 27 weights start at u16 ro (odd when fco is
                // odd): read the 14 aligned dwords around it and shift each
                // pair into place
                const int ro = (8 * fcq + 2 * g + e) * kRawRow + fco * 27;
                const unsigned *rd = reinterpret_cast<const unsigned *>(rawc) + (ro >> 1);
                const unsigned sh = 16u * (unsigned)(ro & 1);
                unsigned dw[14];
#pragma unroll
                for (int m = 0; m < 14; ++m) dw[m] = rd[m];
                float wv[27];
#pragma unroll
                for (int m = 0; m < 14; ++m) {
                    const unsigned pr = __builtin_amdgcn_alignbit(dw[m < 13 ? m + 1 : 13], dw[m], sh);
                    wv[2 * m] = __uint_as_float(pr << 16);
                    if (2 * m + 1 < 27) wv[2 * m + 1] = __uint_as_float(pr & 0xffff0000u);
                }
                // per axis, input offset 0 takes kernel taps {1,2} and offset
                // 1 takes tap {0}; the 3-D sums are formed axis by axis (the
                // same sums as emit() below)
                float s1w[9][2];
#pragma unroll
                for (int rr = 0; rr < 9; ++rr) {
                    s1w[rr][0] = wv[rr * 3 + 1] + wv[rr * 3 + 2];
                    s1w[rr][1] = wv[rr * 3 + 0];
                }
                float s2w[3][2][2];
#pragma unroll
                for (int kd = 0; kd < 3; ++kd)
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        s2w[kd][0][c] = s1w[kd * 3 + 1][c] + s1w[kd * 3 + 2][c];
                        s2w[kd][1][c] = s1w[kd * 3 + 0][c];
                    }
#pragma unroll
                for (int tap = 0; tap < 8; ++tap) {
                    const int a = tap >> 2, b = (tap >> 1) & 1, c = tap & 1;
                    we[e][tap] = a ? s2w[0][b][c] : (s2w[1][b][c] + s2w[2][b][c]);
                }
            }
            const int frag_lane = (fcq + 2 * h) * 16 + col;
#pragma unroll
            for (int tap = 0; tap < 8; ++tap) {
                const unsigned short h0v = f32_to_bf16(we[0][tap]), h1v = f32_to_bf16(we[1][tap]);
                const unsigned short l0v = f32_to_bf16(we[0][tap] - bf16_to_f32(h0v));
                const unsigned short l1v = f32_to_bf16(we[1][tap] - bf16_to_f32(h1v));
                tab[(((fcb * 8 + tap) * 2 + 0) * 64 + frag_lane) * 4 + g] = (unsigned)h0v | ((unsigned)h1v << 16);
                tab[(((fcb * 8 + tap) * 2 + 1) * 64 + frag_lane) * 4 + g] = (unsigned)l0v | ((unsigned)l1v << 16);
            }
        }
    } else if (direct_w) {
        if constexpr (!kLinePath) {
#pragma unroll
            for (int j = 0; j < kCouplesPerThread; ++j) {
                const int q = tid + j * kThreads;
                if (q < kCouples) {
                    const int ci = q >> 5, cl = 2 * (q & 31);
                    const bool ok = ci < Cin;
#pragma unroll
                    for (int half = 0; half < 2; ++half) {
                        float wv[27];
#pragma unroll
                        for (int k = 0; k < 27; ++k) {
                            const int e = 27 * half + k;   // u16 element of the couple
                            const unsigned u = (wd[j][e >> 1] >> (16 * (e & 1))) & 0xffffu;
                            wv[k] = ok ? bf16_to_f32((unsigned short)u) : 0.0f;
                        }
                        emit(wv, cl + half, ci);
                    }
                }
            }
            if (early_slab && t_begin < t_end) {
                // slab buffer 0 lies below the filter table here: stage the first
                // tile now and issue the second tile's loads before the fragments
                put_all(slab, n, d, hp);
                next_pos(n2, d2, hp2);
                if (t_begin + 1 < t_end) fetch(n2, d2, hp2);
            }
        }
    } else {
        // general path: raw weights of a 16-channel chunk staged in LDS as
        // raw[cil][col][27], zero beyond Cin and Cout
        constexpr int kChunks = (Cin8 + kCiChunk - 1) / kCiChunk;
        for (int ch = 0; ch < kChunks; ++ch) {
            const int c0 = ch * kCiChunk;
            const int nci = min(kCiChunk, Cin - c0);
            __syncthreads();                               // previous chunk's raw consumed
            const int run = ncog * 27;
            for (int cil = 0; cil < kCiChunk; ++cil) {
                unsigned short *rd = raw + cil * kCoGroup * 27;
                const int64_t base = ((int64_t)(c0 + cil) * Cout + co0) * 27;
                const int n_in = cil < nci ? run : 0;
                for (int e = tid; e < kCoGroup * 27; e += kThreads)
                    rd[e] = e < n_in ? w[base + e] : (unsigned short)0;
            }
            __syncthreads();
            // pairs (cil, col), output channel fastest: raw reads 27 u16 apart
            for (int pr = tid; pr < kCiChunk * kCoGroup; pr += kThreads) {
                const int cil = pr / kCoGroup, cl = pr % kCoGroup;
                const int ci = c0 + cil;
                if (ci >= Cin8) continue;
                float wv[27];
#pragma unroll
                for (int k = 0; k < 27; ++k) wv[k] = bf16_to_f32(raw[pr * 27 + k]);
                emit(wv, cl, ci);
            }
        }
    }
    __syncthreads();
    // A fragments: lane (g, l%16) of channel block cb, k-step j, half h holds
    // Weff_h[ci0 .. ci0+7][co][tap] with kappa = 32j + 8g = tap*Cin8 + ci0.
    // Tap 7 (input offsets 1,1,1) takes the single weight w[ci,co,0,0,0], so
    // its hi part is exact and its lo part zero: k-steps holding only tap 7
    // (the last Cin8/32 of them when Cin8 is a multiple of 32) skip the lo pass.
    constexpr int kLoSteps = (Cin8 % 32 == 0) ? KSTEPS - Cin8 / 32 : KSTEPS;
    bf16x8 A[2][KSTEPS][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < KSTEPS; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if (h == 1 && j >= kLoSteps) continue;
                const int cl = 16 * (2 * cp + i) + col;
                const int kap = 32 * j + 8 * g;
                const int tap = kap / Cin8, ci0 = kap % Cin8;
                // one 16-byte read: rows are 16-byte aligned (WS = Cin8 + 8),
                // and the 80-byte row stride spreads lanes over all banks; the
                // line path's table is in fragment order
                const unsigned short *src =
                    (kLinePath && direct_w)
                        ? lds + ((((2 * cp + i) * 8 + j) * 2 + h) * 64 + lane) * 8
                        : weffT + ((h * 8 + tap) * kCoGroup + cl) * WS + ci0;
                A[i][j][h] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8 *>(src));
            }
    // folded epilogue ((S/8 + cb)*s1 + b)*s2 = S*alpha + beta[co]
    const float alpha = 0.125f * s1 * s2;
    if (tid < kCoGroup) {
        const int co = co0 + tid;
        const float cbv = (conv_bias && co < Cout) ? conv_bias[co] : 0.0f;
        const float bv = (bias && co < Cout) ? bias[co] : 0.0f;
        epi[tid] = (cbv * s1 + bv) * s2;
    }
    // B-fragment slab offsets of this lane: kappa = 32j + 8g -> (tap, ci0)
    int boff[KSTEPS];
#pragma unroll
    for (int j = 0; j < KSTEPS; ++j) {
        const int kap = 32 * j + 8 * g;
        const int tap = kap / Cin8, ci0 = kap % Cin8;
        boff[j] = (((tap >> 2) * kRows + ((tap >> 1) & 1)) * W + (tap & 1)) * CS + ci0;
    }

    // ---- main loop over tiles (n, d, pooled row pair) --------------------
    const int wblocks = kWB > 0 ? kWB : (Wp + 15) / 16;
    const int nvb = kTH * wblocks;                // voxel blocks per tile
    // voxel blocks of this slot per tile (slot, slot+4, ...); a compile-time
    // count when kWB > 0 and the tile's blocks split evenly over the 4 slots
    const int nvb_slot = (kWB > 0 && (kTH * kWB) % 4 == 0) ? kTH * kWB / 4 : (nvb - slot + 3) / 4;
    int vb_hh0 = 0, vb_wb0 = slot;               // first voxel block of this slot
    while (vb_wb0 >= wblocks) { vb_wb0 -= wblocks; ++vb_hh0; }

    __syncthreads();              // every wave holds its fragments: the slabs may reuse that LDS
    if (!early_slab) {
        // first tile's slab into buffer 0 (its loads were issued before the
        // prologue), the second tile's loads into registers
        if (t_begin < t_end) {
            put_all(slab, n, d, hp);
            next_pos(n2, d2, hp2);
            if (t_begin + 1 < t_end) fetch(n2, d2, hp2);
        }
        __syncthreads();
    }

    // Per tile t: MFMA and stores of tile t, then slab t+1 into the spare
    // buffer and the loads of slab t+2, then the barrier.  Waiting for slab
    // t+1's loads (issued before tile t's stores; loads and stores retire in
    // order) then never waits for tile t's stores, and the wait sees the same
    // loads-then-stores sequence on the first tile as on every later one.
    for (int t = t_begin; t < t_end; ++t) {
        const int h0 = kTH * hp;
        unsigned short *cur = slab + ((t - t_begin) & 1) * slab_u16;

        // Stores go through a buffer resource over this batch item's output
        // (word 3 0x00020000: 32-bit data format; the host keeps an item's
        // output below 2^31 bytes); masked lanes store past the range, which
        // the hardware drops.  No store sits behind a branch, so every tile
        // issues the same number of stores, and the next tile's wait for the
        // slab loads issued before them (loads and stores retire in order)
        // does not wait for these stores.
        const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
            out + (int64_t)n * Cout * pplane, 0, (int)(Cout * pplane * 4), 0x00020000);
        const int obase = (d * Hp + h0) * Wp;       // per-item offsets fit in int32 (shim)
        int hh = vb_hh0, wb = vb_wb0;
        for (int it = 0; it < nvb_slot; ++it) {
            const int h = h0 + hh;
            const int wv = wb * 16 + col;
            const bool valid = (wv < Wp) && (h < Hp);
            const int wc = min(wv, Wp - 1);
            const unsigned short *sb = cur + (hh * W + wc) * CS;
            v4f a0h = {0.0f, 0.0f, 0.0f, 0.0f}, a1h = a0h, a0l = a0h, a1l = a0h;
#pragma unroll
            for (int j = 0; j < KSTEPS; ++j) {
                const bf16x8 B = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8 *>(sb + boff[j]));
                a0h = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[0][j][0], B, a0h, 0, 0, 0);
                a1h = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[1][j][0], B, a1h, 0, 0, 0);
                if (j < kLoSteps) {
                    a0l = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[0][j][1], B, a0l, 0, 0, 0);
                    a1l = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[1][j][1], B, a1l, 0, 0, 0);
                }
            }
            const int opos = obase + hh * Wp + wv;
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int cl = 16 * (2 * cp + i) + 4 * g + r;
                    const float sum = i ? (a1h[r] + a1l[r]) : (a0h[r] + a0l[r]);
                    const int off = (valid && co0 + cl < Cout) ? ((co0 + cl) * (int)pplane + opos) * 4
                                                               : 0x7ffffff0;   // past the range
                    __builtin_amdgcn_raw_buffer_store_b32(
                        __float_as_uint(__builtin_fmaf(sum, alpha, epi[cl])), orsrc, off, 0, 0);
                }
            wb += 4;
            while (wb >= wblocks) { wb -= wblocks; ++hh; }
        }
        if (t + 1 < t_end) {
            // the spare buffer's last readers finished before the previous barrier
            put_all(slab + (((t - t_begin) & 1) ^ 1) * slab_u16, n2, d2, hp2);
            next_pos(n2, d2, hp2);
            if (t + 2 < t_end) fetch(n2, d2, hp2);
        }
        __syncthreads();                           // next slab written; this one consumed
        next_pos(n, d, hp);
    }
}

}  // namespace

// Pooled rows per tile for a geometry: 8 when the double-buffered slab fits
// next to the prologue regions in LDS, else 2; 0 if nothing fits.
static int pick_th(int cin8, int64_t W)
{
    for (int th : {8, 2}) {
        const int64_t lds = (int64_t)epi_offset(th, (int)W, cin8 + 8) + kCoGroup * (int64_t)sizeof(float);
        if (lds <= 160 * 1024) return th;
    }
    return 0;
}

// LDS bytes for a geometry; 0 if Cin or W is outside the implemented range
// (Cin <= 32, W a multiple of 8, slab fits).
size_t fused3d_bf16_lds_bytes(int64_t Cin, int64_t W)
{
    if (Cin < 1 || Cin > 32 || W % 8 != 0 || W > 4096) return 0;
    const int cin8 = (int)((Cin + 7) & ~int64_t(7));
    const int th = pick_th(cin8, W);
    if (th == 0) return 0;
    return (size_t)epi_offset(th, (int)W, cin8 + 8) + kCoGroup * sizeof(float);
}

hipError_t launch_fused3d_bf16(const uint16_t *x, const uint16_t *w, const float *conv_bias,
                               const float *bias, float s1, float s2, int64_t N, int64_t Cin,
                               int64_t D, int64_t H, int64_t W, int64_t Cout, float *out,
                               hipStream_t stream)
{
    const int Dp = (int)(D - 1), Hp = (int)(H - 1), Wp = (int)(W - 1);
    const int cin8 = (int)((Cin + 7) & ~int64_t(7));
    const int ksteps = cin8 / 4;
    const int th = pick_th(cin8, W);
    const size_t lds = fused3d_bf16_lds_bytes(Cin, W);
    if (th == 0 || lds == 0) return hipErrorInvalidValue;
    const int hchunks = (Hp + th - 1) / th;
    const int64_t ntiles = N * Dp * (int64_t)hchunks;
    const int cus = device_cus();
    const unsigned gy = (unsigned)((Cout + kCoGroup - 1) / kCoGroup);
    int64_t gx = cus / (int64_t)gy;
    if (gx < 1) gx = 1;
    if (gx > ntiles) gx = ntiles;
    const int tpw = (int)((ntiles + gx - 1) / gx);
    gx = (ntiles + tpw - 1) / tpw;

#define CT_LAUNCH_BF16(KS, TH, WB)                                                            \
    do {                                                                                      \
        hipError_t e = allow_dynamic_lds((const void *)fused3d_bf16_kernel<KS, TH, WB>, lds);   \
        if (e != hipSuccess) return e;                                                        \
        hipLaunchKernelGGL((fused3d_bf16_kernel<KS, TH, WB>), dim3((unsigned)gx, gy),             \
                           dim3(kThreads), lds, stream, (const unsigned short *)x,            \
                           (const unsigned short *)w, conv_bias, bias, s1, s2, (int)Cin,      \
                           (int)D, (int)H, (int)W, (int)Cout, Dp, Hp, Wp, hchunks,            \
                           (int)ntiles, tpw, out);                                            \
    } while (0)

    if (ksteps == 8 && th == 8 && (Wp + 15) / 16 == 2) {
        CT_LAUNCH_BF16(8, 8, 2);          // the page's wide workload (Cin 25..32, W 18..32)
        return hipGetLastError();
    }
    switch (ksteps * 16 + th) {
    case 2 * 16 + 8: CT_LAUNCH_BF16(2, 8, 0); break;
    case 4 * 16 + 8: CT_LAUNCH_BF16(4, 8, 0); break;
    case 6 * 16 + 8: CT_LAUNCH_BF16(6, 8, 0); break;
    case 8 * 16 + 8: CT_LAUNCH_BF16(8, 8, 0); break;
    case 2 * 16 + 2: CT_LAUNCH_BF16(2, 2, 0); break;
    case 4 * 16 + 2: CT_LAUNCH_BF16(4, 2, 0); break;
    case 6 * 16 + 2: CT_LAUNCH_BF16(6, 2, 0); break;
    case 8 * 16 + 2: CT_LAUNCH_BF16(8, 2, 0); break;
    default: return hipErrorInvalidValue;
    }
#undef CT_LAUNCH_BF16
    return hipGetLastError();
}

}  // namespace ct
