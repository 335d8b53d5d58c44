// fused3d_bf16.hip - ConvTranspose3d(k3, s2, p1) -> *scale1 -> AvgPool3d(2)
// -> +bias -> *scale2 with bf16 x and w, fp32 accumulation and output, on the
// gfx950 bf16 matrix cores (v_mfma_f32_16x16x32_bf16).
//
// Method ([p50] "Kimi-K2.6 l2_p50"): as the fp32 kernel - each pooled voxel
// is S/8 with S = sum_ci sum_{a,b,c in {0,1}} x[ci,d+a,h+b,w+c] *
// Weff[ci,co,abc], Weff the per-tap sums of the 27 weights (passages on the
// stride-2 parity rule and on grouping the 27 terms by input tap), then the
// model's epilogue ((S/8 + conv_bias)*scale1 + bias)*scale2.
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
//    (blockIdx.y).  Prologue: stage the raw weights into LDS (coalesced),
//    form Weff and its hi/lo split once, write them in fragment order, and
//    load each wave's fragments (2 output-channel blocks x all k-steps x
//    hi/lo) into registers for the whole kernel.
//  * Tile = (n, d, 2 pooled rows): the input slab x[n, :, d..d+1, h0..h0+2, :]
//    is transposed to [plane][row][w][ci] in LDS; the next tile's slab is
//    prefetched into registers while the current one is computed.
//  * Wave = (voxel-block slot s = w%4, channel pair p = w/4): each B read
//    feeds 4 MFMAs (2 channel blocks x hi/lo).
//  * Each workgroup walks a contiguous range of tiles, so neighbouring tiles
//    (which share input rows) run on the same XCD and hit its L2.
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
constexpr int kTH = 2;                // pooled rows per tile
constexpr int kRows = kTH + 1;        // input rows per plane in a slab
constexpr int kPrefetch = 2;          // 16-byte slab pieces prefetched per thread

__device__ __forceinline__ float bf16_to_f32(unsigned short b)
{
    return __uint_as_float(((unsigned)b) << 16);
}

// round to nearest even; NaN stays a quiet NaN
__device__ __forceinline__ unsigned short f32_to_bf16(float f)
{
    unsigned u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (unsigned short)((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (unsigned short)(u >> 16);
}

// Byte sizes of the LDS regions (shared with the launcher).
__host__ __device__ inline int raw_bytes() { return kCiChunk * kCoGroup * 27 * 2; }
__host__ __device__ inline int afrag_bytes(int ksteps) { return 4 * ksteps * 2 * 512 * 2; }
__host__ __device__ inline int slab_bytes(int W, int cs) { return 2 * kRows * W * cs * 2; }
// The epilogue constants sit after the larger of the prologue regions and the
// slab, so neither overwrites them.
__host__ __device__ inline int epi_offset(int W, int cs)
{
    const int a = raw_bytes() + afrag_bytes(8), b = slab_bytes(W, cs);
    return ((a > b ? a : b) + 15) & ~15;
}

template <int KSTEPS>
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
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_bytes[];
    unsigned short *lds = reinterpret_cast<unsigned short *>(lds_bytes);
    unsigned short *raw = lds;                                // prologue: raw weights
    unsigned short *afrag = lds + raw_bytes() / 2;            // prologue: fragments
    unsigned short *slab = lds;                               // main loop: input slab

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = lane >> 4;                 // lane group
    const int col = lane & 15;
    const int slot = wave & 3;               // voxel-block slot
    const int cp = wave >> 2;                // channel-block pair
    const int co0 = blockIdx.y * kCoGroup;
    const int ncog = min(kCoGroup, Cout - co0);

    // ---- prologue: Weff hi/lo in fragment order ------------------------
    for (int c0 = 0; c0 < Cin8; c0 += kCiChunk) {
        const int nci = min(kCiChunk, Cin - c0);
        __syncthreads();
        for (int e = tid; e < kCiChunk * kCoGroup * 27; e += kThreads) {
            const int pr = e / 27, k = e - pr * 27;
            const int cil = pr / kCoGroup, col_ = pr - cil * kCoGroup;
            raw[e] = (cil < nci && col_ < ncog)
                ? w[((int64_t)(c0 + cil) * Cout + co0 + col_) * 27 + k] : (unsigned short)0;
        }
        __syncthreads();
        for (int pr = tid; pr < kCiChunk * kCoGroup; pr += kThreads) {
            const int cil = pr / kCoGroup, cl = pr - cil * kCoGroup;
            const int ci = c0 + cil;
            if (ci >= Cin8) continue;
            float wv[27];
#pragma unroll
            for (int k = 0; k < 27; ++k) wv[k] = bf16_to_f32(raw[pr * 27 + k]);
            // offset 0 pairs with taps {1,2}, offset 1 with tap {0}, per axis
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
                const unsigned short lo = f32_to_bf16(we - bf16_to_f32(hi));
                const int kap = tap * Cin8 + ci;
                const int j = kap >> 5, gg = (kap >> 3) & 3, e8 = kap & 7;
                const int cb = cl >> 4, l = gg * 16 + (cl & 15);
                const int base = ((cb * KSTEPS + j) * 2) * 512 + l * 8 + e8;
                afrag[base] = hi;
                afrag[base + 512] = lo;
            }
        }
    }
    __syncthreads();
    bf16x8 A[2][KSTEPS][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < KSTEPS; ++j)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int cb = 2 * cp + i;
                const u16x8 v = *reinterpret_cast<const u16x8 *>(
                    afrag + ((cb * KSTEPS + j) * 2 + h) * 512 + lane * 8);
                A[i][j][h] = __builtin_bit_cast(bf16x8, v);
            }
    // epilogue constants of this workgroup's channels, kept in LDS
    float *epi = reinterpret_cast<float *>(lds_bytes + epi_offset(W, CS));   // [2][64]
    if (tid < kCoGroup) {
        const int co = co0 + tid;
        epi[tid] = (conv_bias && co < Cout) ? conv_bias[co] : 0.0f;
        epi[kCoGroup + tid] = (bias && co < Cout) ? bias[co] : 0.0f;
    }

    // ---- main loop over tiles (n, d, pooled row pair) --------------------
    const int64_t HW = (int64_t)H * W;
    const int64_t DHW = (int64_t)D * HW;
    const int64_t pplane = (int64_t)Dp * Hp * Wp;
    const int W8 = W >> 3;                        // 8-element column groups (W % 8 == 0)
    const int nq = Cin8 * 2 * kRows * W8;         // 16-byte slab pieces per tile
    const int wblocks = (Wp + 15) / 16;
    const int nvb = kTH * wblocks;                // voxel blocks per tile
    const int t_begin = blockIdx.x * tiles_per_wg;
    const int t_end = min(t_begin + tiles_per_wg, ntiles);

    // piece q = ((ci*2 + a)*kRows + row)*W8 + w8 covers x[n, ci, d+a, 2*hp+row, 8*w8 .. 8*w8+7]
    auto piece_load = [&](int t, int q) -> u16x8 {
        const int hp = t % hpairs;
        const int nd = t / hpairs;
        const int d = nd % Dp, n = nd / Dp;
        const int w8 = q % W8;
        int r = q / W8;
        const int row = r % kRows;
        r /= kRows;
        const int a = r & 1, ci = r >> 1;
        const int h = 2 * hp + row;
        if (ci >= Cin || h >= H) return (u16x8){0, 0, 0, 0, 0, 0, 0, 0};
        return *reinterpret_cast<const u16x8 *>(
            x + (int64_t)n * Cin * DHW + (int64_t)ci * DHW + (int64_t)(d + a) * HW +
            (int64_t)h * W + 8 * w8);
    };
    auto piece_store = [&](int q, u16x8 v) {
        const int w8 = q % W8;
        int r = q / W8;
        const int row = r % kRows;
        r /= kRows;
        const int a = r & 1, ci = r >> 1;
        unsigned short *dst = slab + ((a * kRows + row) * W + 8 * w8) * CS + ci;
#pragma unroll
        for (int k = 0; k < 8; ++k) dst[k * CS] = v[k];
    };

    u16x8 pre[kPrefetch];
    if (t_begin < t_end) {
#pragma unroll
        for (int i = 0; i < kPrefetch; ++i) {
            const int q = tid + i * kThreads;
            if (q < nq) pre[i] = piece_load(t_begin, q);
        }
    }
    for (int t = t_begin; t < t_end; ++t) {
        __syncthreads();                           // previous slab consumed
#pragma unroll
        for (int i = 0; i < kPrefetch; ++i) {
            const int q = tid + i * kThreads;
            if (q < nq) piece_store(q, pre[i]);
        }
        for (int q = tid + kPrefetch * kThreads; q < nq; q += kThreads)
            piece_store(q, piece_load(t, q));
        __syncthreads();
        if (t + 1 < t_end) {
#pragma unroll
            for (int i = 0; i < kPrefetch; ++i) {
                const int q = tid + i * kThreads;
                if (q < nq) pre[i] = piece_load(t + 1, q);
            }
        }

        const int hp = t % hpairs;
        const int nd = t / hpairs;
        const int d = nd % Dp, n = nd / Dp;
        for (int vb = slot; vb < nvb; vb += 4) {
            const int hh = vb / wblocks, wb = vb - hh * wblocks;
            const int h = 2 * hp + hh;
            const int wv = wb * 16 + col;
            const bool valid = (wv < Wp) && (h < Hp);
            const int wc = min(wv, Wp - 1);
            v4f acc0 = {0.0f, 0.0f, 0.0f, 0.0f}, acc1 = acc0;
#pragma unroll
            for (int j = 0; j < KSTEPS; ++j) {
                const int kap = 32 * j + 8 * g;
                const int tap = kap / Cin8, ci0 = kap - tap * Cin8;
                const int a = tap >> 2, b = (tap >> 1) & 1, c = tap & 1;
                const u16x8 bvv = *reinterpret_cast<const u16x8 *>(
                    slab + ((a * kRows + hh + b) * W + wc + c) * CS + ci0);
                const bf16x8 B = __builtin_bit_cast(bf16x8, bvv);
                acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[0][j][0], B, acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[1][j][0], B, acc1, 0, 0, 0);
                acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[0][j][1], B, acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[1][j][1], B, acc1, 0, 0, 0);
            }
            if (valid) {
                float *on = out + (int64_t)n * Cout * pplane + ((int64_t)d * Hp + h) * Wp + wv;
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int cl = 16 * (2 * cp + i) + 4 * g + r;
                        if (co0 + cl < Cout) {
                            float v = (i ? acc1[r] : acc0[r]) * 0.125f;
                            v = (v + epi[cl]) * s1;
                            v = (v + epi[kCoGroup + cl]) * s2;
                            on[(int64_t)(co0 + cl) * pplane] = v;
                        }
                    }
            }
        }
    }
}

}  // namespace

// LDS bytes for a geometry; 0 if Cin or W is outside the implemented range
// (Cin <= 32, W a multiple of 8).
size_t fused3d_bf16_lds_bytes(int64_t Cin, int64_t W)
{
    if (Cin < 1 || Cin > 32 || W % 8 != 0 || W > 4096) return 0;
    const int cin8 = (int)((Cin + 7) & ~int64_t(7));
    const int ksteps = cin8 / 4;
    (void)ksteps;
    return (size_t)epi_offset((int)W, cin8 + 8) + 2 * kCoGroup * sizeof(float);
}

hipError_t launch_fused3d_bf16(const uint16_t *x, const uint16_t *w, const float *conv_bias,
                               const float *bias, float s1, float s2, int64_t N, int64_t Cin,
                               int64_t D, int64_t H, int64_t W, int64_t Cout, float *out,
                               hipStream_t stream)
{
    const int Dp = (int)(D - 1), Hp = (int)(H - 1), Wp = (int)(W - 1);
    const int hpairs = (Hp + kTH - 1) / kTH;
    const int64_t ntiles = N * Dp * (int64_t)hpairs;
    const int cin8 = (int)((Cin + 7) & ~int64_t(7));
    const int ksteps = cin8 / 4;
    const size_t lds = fused3d_bf16_lds_bytes(Cin, W);
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        cus = 256;
    const unsigned gy = (unsigned)((Cout + kCoGroup - 1) / kCoGroup);
    int64_t gx = cus / (int64_t)gy;
    if (gx < 1) gx = 1;
    if (gx > ntiles) gx = ntiles;
    const int tpw = (int)((ntiles + gx - 1) / gx);
    gx = (ntiles + tpw - 1) / tpw;

#define CT_LAUNCH_BF16(KS)                                                                   \
    do {                                                                                     \
        hipError_t e = hipFuncSetAttribute((const void *)fused3d_bf16_kernel<KS>,            \
                                           hipFuncAttributeMaxDynamicSharedMemorySize,       \
                                           (int)lds);                                        \
        if (e != hipSuccess) return e;                                                       \
        hipLaunchKernelGGL(fused3d_bf16_kernel<KS>, dim3((unsigned)gx, gy), dim3(kThreads),  \
                           lds, stream, (const unsigned short *)x, (const unsigned short *)w, \
                           conv_bias, bias, s1, s2, (int)Cin, (int)D, (int)H, (int)W,        \
                           (int)Cout, Dp, Hp, Wp, hpairs, (int)ntiles, tpw, out);            \
    } while (0)

    switch (ksteps) {
    case 2: CT_LAUNCH_BF16(2); break;
    case 4: CT_LAUNCH_BF16(4); break;
    case 6: CT_LAUNCH_BF16(6); break;
    case 8: CT_LAUNCH_BF16(8); break;
    default: return hipErrorInvalidValue;
    }
#undef CT_LAUNCH_BF16
    return hipGetLastError();
}

}  // namespace ct
