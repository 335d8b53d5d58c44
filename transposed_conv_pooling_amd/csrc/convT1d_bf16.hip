// convT1d_bf16.hip - dilated ConvTranspose1d (stride 1, any pad and output
// padding) with bf16 inputs and weights as an implicit GEMM on the gfx950
// bf16 matrix cores (fp32 accumulation and output).
//
// Method ([p74] "Kimi-K2.6 l1_p74"): with stride 1 and pad 0 the transposed
// convolution is the gather
//     y[n,co,o] = sum_ci sum_{k<K} x[n,ci,o - dil*k] * w[ci,co,k]
// over in-range input positions, weights unflipped (passages on the gather
// formula and the implicit-GEMM view).  Per batch item and tap k this is the
// product of the shifted input (positions x channels) with w[:, :, k]
// (channels x output channels), summed over the K taps.
//
// MI355X mapping (v_mfma_f32_16x16x32_bf16, 8 bf16 per lane per operand):
//  * A (16 x 32) = input: lane l supplies the 8 channels 8*(l/16) .. +7 at
//    output position o = l%16 of a 16-output block, shifted by -dil*k;
//    B (32 x 16) = weights: the same 8 channels for output channel l%16;
//    D (16 x 16): lane l holds D[o = 4*(l/16) + r][co = l%16], i.e. four
//    consecutive outputs of one channel -> one 16-byte store.
//  * The input strip of a tile (positions o0 - 80 .. o0 + 255, all 32
//    channels) is staged in LDS channels-last, two channels per dword, at a
//    row stride of 20 dwords: a fragment read is one ds_read_b128 per lane
//    and the 16 positions of a lane group cover all 64 banks once.
//  * The weights of the workgroup's 64 output channels are staged once in
//    LDS in B-fragment order for all K taps (workgroups are persistent).
//  * A workgroup (4 waves) owns 64 channels of a tile; each wave 80 outputs
//    x 64 channels = 20 accumulators and 20 MFMAs per tap.
//    The next tile's strip is loaded into registers while this one computes.
//  * The fp32 output dominates the traffic, so tiles are cut at 128-byte
//    lines of each output row rather than at multiples of 256 outputs:
//    a line written in two pieces by two workgroups costs far more HBM time
//    than one written whole (measured: 3.3 vs 5.0 TB/s for this output).
//    Each workgroup computes 320 outputs per tile (5 blocks of 16 per wave)
//    and stores, per channel row, the 256 of them that start on a line.
#include "ct_internal.h"

namespace ct {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTO = 256;              // outputs stored per tile and channel row
constexpr int kCO = 64;               // output channels per workgroup
constexpr int kCin = 32;              // input channels (one MFMA K step per tap)
constexpr int kCSW = 20;              // LDS dwords per strip position (16 used)

constexpr int kLead = 64;             // outputs computed before a tile's first stored one
constexpr int kOB = 5;                // 16-output blocks per wave: 4 * 5 * 16 = kLead + kTO

// H8: strip positions before a tile's first computed output, a multiple of 8
// (16-byte pieces): the halo DIL*(K-1) rounded up without padding; with a pad
// the strip is shifted by the pad rounded up to a multiple of 8 and needs up
// to 7 more.
template <int K, int DIL, int H8 = (DIL * (K - 1) + 7) / 8 * 8>
struct Geo1 {
    static constexpr int kHalo = DIL * (K - 1);
    static constexpr int kH8 = H8;
    static constexpr int kTS = kLead + kTO + kH8;             // strip positions
    static constexpr int kPieces = (kCin / 2) * (kTS / 8);   // (channel pair, 8 positions)
    static constexpr int kPPT = (kPieces + kThreads - 1) / kThreads;
    static constexpr int kLdsBytes = kTS * kCSW * 4;
};

// With a pad (stride 1) output o is output o + pad of the unpadded
// convolution (output padding only extends the window at the end): the strip
// of a tile starts shift = pad rounded up to a multiple of 8 positions later,
// and the lanes read it pad - shift positions back (H8 above the unpadded
// halo; the unpadded instantiation folds pad and shift to 0).
// RAGGED: output rows may start at any 4-byte boundary (Lo % 4 != 0 or y
// not 16-byte aligned); otherwise every row starts 16-byte aligned.
template <int K, int DIL, bool RAGGED, int H8 = (DIL * (K - 1) + 7) / 8 * 8>
__global__ __launch_bounds__(kThreads, 2)
void convT1d_bf16_kernel(const uint16_t *__restrict__ x, const uint16_t *__restrict__ w,
                         const float *__restrict__ bias, int L, int Cout, int Lo, int tiles_per_n,
                         int ntiles, int pad_arg, float *__restrict__ y)
{
    typedef Geo1<K, DIL, H8> G;
    static_assert(H8 % 8 == 0 && H8 >= DIL * (K - 1), "strip halo");
    const int pad = H8 == (DIL * (K - 1) + 7) / 8 * 8 ? 0 : pad_arg;
    const int shift = (pad + 7) & ~7;
    __shared__ __attribute__((aligned(16))) unsigned strip[G::kTS * kCSW];
    __shared__ __attribute__((aligned(16))) uint16_t wfrag[K * 4 * 64 * 8];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, col = lane & 15;
    const int cog = blockIdx.y;

    // B fragments in LDS, fragment order [k][cb][lane][8]: channels 8g .. 8g+7
    // of output channel cog*64 + 16cb + col at tap k (zero beyond Cout), so a
    // lane's fragment is one conflict-free ds_read_b128
    for (int e = tid; e < K * 4 * 64 * 8; e += kThreads) {
        const int j = e & 7, l = (e >> 3) & 63, cb = (e >> 9) & 3, k = e >> 11;
        const int co = cog * kCO + 16 * cb + (l & 15);
        const int ci = 8 * (l >> 4) + j;
        const uint16_t t = w[((int64_t)ci * Cout + (co < Cout ? co : 0)) * K + k];
        wfrag[e] = co < Cout ? t : (uint16_t)0;
    }
    float bv[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
        const int co = cog * kCO + 16 * cb + col;
        bv[cb] = (bias && co < Cout) ? bias[co] : 0.0f;
    }

    // strip piece q: channel pair cp = q % 16, positions s0 + 8*(q / 16) .. +7.
    // Loads are unconditional from clamped addresses (L % 8 == 0, so a piece
    // lies wholly inside [0, L) or wholly outside) and masked when stored.
    u16x8 pre0[G::kPPT], pre1[G::kPPT];
    bool pok[G::kPPT];
    auto fetch = [&](int tile) {
        const int n = tile / tiles_per_n;
        const int s0 = (tile - n * tiles_per_n) * kTO - kLead - G::kH8 + shift;
        const uint16_t *xn = x + (int64_t)n * kCin * L;
#pragma unroll
        for (int i = 0; i < G::kPPT; ++i) {
            const int q = tid + i * kThreads;
            const int cp = q & 15, pos = s0 + 8 * (q >> 4);
            const bool ok = q < G::kPieces && pos >= 0 && pos + 8 <= L;
            const uint16_t *src = xn + (int64_t)(2 * cp) * L + (ok ? pos : 0);
            pre0[i] = *reinterpret_cast<const u16x8 *>(src);
            pre1[i] = *reinterpret_cast<const u16x8 *>(src + L);
            pok[i] = ok;
        }
    };
    auto put = [&]() {
        const u16x8 z = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < G::kPPT; ++i) {
            const int q = tid + i * kThreads;
            if (q < G::kPieces) {
                const u16x8 a = pok[i] ? pre0[i] : z, b = pok[i] ? pre1[i] : z;
                unsigned *dst = strip + (8 * (q >> 4)) * kCSW + (q & 15);
#pragma unroll
                for (int j = 0; j < 8; ++j) dst[j * kCSW] = (unsigned)a[j] | ((unsigned)b[j] << 16);
            }
        }
    };

    if ((int)blockIdx.x < ntiles) fetch(blockIdx.x);
    // lane's A base: strip position kH8 - (shift - pad) + 80*wave + col
    // (input o + pad of output o = o0 - kLead + 80*wave + col), channels
    // 8g..8g+7
    const unsigned *al = strip + (G::kH8 - (shift - pad) + 16 * kOB * wave + col) * kCSW + 4 * g;
    const uint16_t *wl = wfrag + lane * 8;        // lane's B fragments
    const int64_t ybase = (int64_t)(((uintptr_t)y) >> 2);   // y in floats (y is 4-byte aligned)

    for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int n = tile / tiles_per_n;
        const int o0 = (tile - n * tiles_per_n) * kTO;
        __syncthreads();          // previous strip consumed
        put();
        __syncthreads();
        if (tile + (int)gridDim.x < ntiles) fetch(tile + gridDim.x);

        v4f acc[kOB][4];
#pragma unroll
        for (int ob = 0; ob < kOB; ++ob)
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) acc[ob][cb] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int k = 0; k < K; ++k) {
            bf16x8 A[kOB], B[4];
#pragma unroll
            for (int i = 0; i < kOB; ++i)
                A[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8 *>(al + (16 * i - DIL * k) * kCSW));
#pragma unroll
            for (int i = 0; i < 4; ++i)
                B[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8 *>(wl + (k * 4 + i) * 64 * 8));
#pragma unroll
            for (int ob = 0; ob < kOB; ++ob)
#pragma unroll
                for (int cb = 0; cb < 4; ++cb)
                    acc[ob][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[ob], B[cb], acc[ob][cb], 0, 0, 0);
        }

        // Row co of the tile is stored over [o0 - sh, o0 + 256 - sh), where sh
        // (below 32 floats) moves the segment's start onto a 128-byte line:
        // segments of neighbouring tiles then never share a line, so no
        // partly written line goes to memory.  The computed range
        // [o0 - kLead, o0 + 256) covers every such segment.
        float *yn = y + (int64_t)n * Cout * Lo;
        // vector stores go through a buffer resource over this item's output
        // (word 3 0x00020000: 32-bit data format, as gfx9-family raw buffers
        // need); the hardware drops a store whose offset lies past the range,
        // so masked lanes need no branch and the wait for the next strip's
        // loads does not cover these stores.  With 16-byte aligned rows sh is
        // a multiple of 4 and a lane's four outputs lie wholly inside or
        // outside the segment.  Ragged rows take 4-byte aligned 16-byte
        // stores (which gfx950's vector memory accepts; the compiler emits
        // them for 4-byte-aligned vectors) and store the 1-3 outputs of a
        // vector cut by a segment end one by one.
        const __amdgpu_buffer_rsrc_t yrs = __builtin_amdgcn_make_buffer_rsrc(yn, 0, Cout * Lo * 4, 0x00020000);
        const int ow = o0 - kLead + 16 * kOB * wave + 4 * g;   // lane's first output
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            const int co = cog * kCO + 16 * cb + col;
            int lo = o0, hi = o0 + kTO;
            if (co >= Cout) hi = lo;
            const int sh = (int)((ybase + ((int64_t)n * Cout + co) * Lo) & 31);
            lo -= sh;
            hi -= sh;
            lo = lo > 0 ? lo : 0;
            hi = hi < Lo ? hi : Lo;
#pragma unroll
            for (int ob = 0; ob < kOB; ++ob) {
                const int o = ow + 16 * ob;
                const v4f v = acc[ob][cb] + bv[cb];
                const bool whole = o >= lo && (RAGGED ? o + 4 <= hi : o < hi);
                const int off = whole ? (co * Lo + o) * 4 : 0x7ffffff0;
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), yrs, off, 0, 0);
                if (RAGGED && !whole && o < hi && o + 4 > lo) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (o + r >= lo && o + r < hi)
                            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[r]), yrs,
                                                                  (co * Lo + o + r) * 4, 0, 0);
                }
            }
        }
    }
}

template <int K, int DIL, bool RAGGED, int H8>
hipError_t launch_geo(const uint16_t *x, const uint16_t *w, const float *bias, int64_t N,
                      int64_t L, int64_t Cout, int64_t Lo, int pad, float *out, hipStream_t stream)
{
    // tiles of 256 stored outputs, each row segment shifted back by up to
    // 31 floats: one extra tile when Lo is within 31 of a multiple of 256
    const int tiles_per_n = (int)((Lo + 31 + kTO - 1) / kTO);
    const int64_t ntiles = N * tiles_per_n;
    const void *fn = (const void *)convT1d_bf16_kernel<K, DIL, RAGGED, H8>;
    const int cus = device_cus(), per_cu = occupancy(fn, kThreads, 0);
    const unsigned gy = (unsigned)((Cout + kCO - 1) / kCO);
    int64_t gx = (int64_t)cus * per_cu / gy;
    if (gx < 1) gx = 1;
    if (gx > ntiles) gx = ntiles;
    hipLaunchKernelGGL((convT1d_bf16_kernel<K, DIL, RAGGED, H8>), dim3((unsigned)gx, gy),
                       dim3(kThreads), 0, stream, x, w, bias, (int)L, (int)Cout, (int)Lo,
                       tiles_per_n, (int)ntiles, pad, out);
    return hipGetLastError();
}

}  // namespace

bool convT1d_bf16_supported(int64_t Cin, int K, int dilation, int64_t L, const void *x)
{
    return Cin == kCin && K == 5 && dilation == 3 && L >= 8 && L % 8 == 0 &&
           (((uintptr_t)x) & 15) == 0;
}

hipError_t launch_convT1d_bf16(const uint16_t *x, const uint16_t *w, const float *bias,
                               int64_t N, int64_t L, int64_t Cout, int K, int dilation, int pad,
                               int out_pad, float *out, hipStream_t stream)
{
    if (K != 5 || dilation != 3) return hipErrorInvalidValue;
    const int64_t Lo = L + (int64_t)dilation * (K - 1) - 2 * (int64_t)pad + out_pad;
    const bool ragged = Lo % 4 != 0 || (((uintptr_t)out) & 15) != 0;
    if (pad == 0)
        return ragged ? launch_geo<5, 3, true, 16>(x, w, bias, N, L, Cout, Lo, 0, out, stream)
                      : launch_geo<5, 3, false, 16>(x, w, bias, N, L, Cout, Lo, 0, out, stream);
    return ragged ? launch_geo<5, 3, true, 24>(x, w, bias, N, L, Cout, Lo, pad, out, stream)
                  : launch_geo<5, 3, false, 24>(x, w, bias, N, L, Cout, Lo, pad, out, stream);
}

}  // namespace ct
