// convT1d_f32.hip - dilated ConvTranspose1d (stride 1, pad 0) as an implicit
// GEMM on the gfx950 fp32 matrix cores.
//
// Method ([p74] "Kimi-K2.6 l1_p74"): with stride 1 and pad 0 the transposed
// convolution is the gather
//     y[n,co,o] = sum_ci sum_{k<K} x[n,ci,o - dil*k] * w[ci,co,k]
// over in-range input positions, weights unflipped (passages on the gather
// formula and the dilation worked examples).  For one batch item it is the
// GEMM  Y[co][o] = sum_kappa A[co][kappa] * B[kappa][o]  with
// kappa = (k, ci), A[co][(k,ci)] = w[ci,co,k] and B[(k,ci)][o] =
// x[ci, o - dil*k] (passage on the implicit-GEMM view, M = Cout,
// K = Cin*K); B is never materialised (no im2col).
//
// MI355X mapping:
//  * v_mfma_f32_16x16x4_f32 (full fp32 products and accumulation):
//      A (16x4):  lane l supplies A[co = l%16][kappa = l/16]
//      B (4x16):  lane l supplies B[kappa = l/16][o = l%16]
//      D (16x16): lane l holds D[co = 4*(l/16) + r][o = l%16]
//    kappa runs k-major with ci padded to a multiple of 4 (Cin4), so the 4
//    kappas of one MFMA share one tap k.
//  * General kernel (any Cin, K, dilation within the LDS limit): a
//    workgroup (4 waves) owns a 64-channel x 256-output tile; each wave
//    computes 64 channels x 64 outputs = 16 MFMA accumulators.  Workgroups
//    are persistent: they stage the weights once into LDS in fragment order
//    (lane-consecutive, conflict-free) and then walk tiles; per tile the
//    input strip x[n, :, o0-halo .. o0+255] (halo = dil*(K-1), zero outside
//    [0,L)) is staged in LDS once behind a workgroup barrier, and the K
//    shifted views of the gather are different LDS offsets into that strip,
//    read at a row stride of 16 mod 64 words so the four 16-lane groups of a
//    fragment read hit disjoint banks.
//  * Page's geometry (Cin 32, K 5, dilation 3): the same MFMA tiling with
//    everything known at compile time, but each wave owns its tiles and a
//    private strip, so no tile waits at a barrier (convT1d_f32_wave_kernel).
#include <type_traits>

#include "ct_internal.h"

namespace ct {
namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTO = 256;              // outputs per tile (64 per wave)
constexpr int kCO = 64;               // output channels per tile

__global__ __launch_bounds__(kThreads)
void convT1d_f32_kernel(const float *__restrict__ x, const float *__restrict__ w,
                        const float *__restrict__ bias, int Cin, int Cin4, int L,
                        int Cout, int K, int dil, int Lo, int tiles_per_n,
                        int ntiles, int xs_str, float *__restrict__ y)
{
    extern __shared__ float lds[];
    const int ksteps = (Cin4 * K) >> 2;
    float *wfrag = lds;                               // [4 m][ksteps][64]
    float *xs = lds + 4 * ksteps * 64;                // [Cin4][xs_str]
    const int halo = dil * (K - 1);
    const int ts = kTO + halo;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int cog = blockIdx.y;                       // 64-channel group

    // Weights in fragment order: wfrag[(m*ksteps + j)*64 + l] = A[co][kappa]
    // with co = cog*64 + 16m + l%16, kappa = 4j + l/16 = k*Cin4 + ci.
    for (int e = threadIdx.x; e < 4 * ksteps * 64; e += kThreads) {
        const int l = e & 63;
        const int j = (e >> 6) % ksteps;
        const int m = (e >> 6) / ksteps;
        const int co = cog * kCO + 16 * m + (l & 15);
        const int kap = 4 * j + (l >> 4);
        const int k = kap / Cin4, ci = kap - k * Cin4;
        wfrag[e] = (co < Cout && ci < Cin) ? w[((int64_t)ci * Cout + co) * K + k] : 0.0f;
    }

    float bv[4][4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int co = cog * kCO + 16 * m + 4 * (lane >> 4) + r;
            bv[m][r] = (bias && co < Cout) ? bias[co] : 0.0f;
        }

    const int kq = lane >> 4;
    const int col = lane & 15;

    for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
        const int n = tile / tiles_per_n;
        const int o0 = (tile - n * tiles_per_n) * kTO;
        __syncthreads();          // previous tile's strip fully consumed (and weights staged)
        // stage x[n, ci, o0 - halo + t], t < ts
        const float *xn = x + (int64_t)n * Cin * L;
        for (int e = threadIdx.x; e < Cin4 * ts; e += kThreads) {
            const int ci = e / ts, t = e - ci * ts;
            const int pos = o0 - halo + t;
            xs[ci * xs_str + t] = (ci < Cin && pos >= 0 && pos < L) ? xn[(int64_t)ci * L + pos] : 0.0f;
        }
        __syncthreads();

        v4f acc[4][4];
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int b = 0; b < 4; ++b) acc[m][b] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};

        // B row base for this lane: xs[ci][halo - dil*k + 64*wave + 16b + col]
        const int obase = halo + 64 * wave + col;
        for (int j = 0; j < ksteps; ++j) {
            const int kap = 4 * j + kq;
            const int k = kap / Cin4, ci = kap - k * Cin4;
            const float *xb = xs + ci * xs_str + obase - dil * k;
            float av[4], bvv[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) av[m] = wfrag[(m * ksteps + j) * 64 + lane];
#pragma unroll
            for (int b = 0; b < 4; ++b) bvv[b] = xb[16 * b];
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    acc[m][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[m], bvv[b], acc[m][b], 0, 0, 0);
        }

        float *yn = y + (int64_t)n * Cout * Lo;
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int co = cog * kCO + 16 * m + 4 * kq + r;
                if (co >= Cout) continue;
                float *yr = yn + (int64_t)co * Lo;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int o = o0 + 64 * wave + 16 * b + col;
                    if (o < Lo) yr[o] = acc[m][b][r] + bv[m][r];
                }
            }
    }
}

// Specialised path for the page's geometry: Cin4, K and the dilation known
// at compile time, so every LDS address is a per-lane base plus an immediate
// offset and the k-loop carries no index arithmetic.  Requires L % 4 == 0
// (whole float4 pieces of the strip are either inside or outside [0, L)) and
// a 16-byte aligned x; output rows may start at any 4-byte boundary.
// Wave-independent path for the same specialised geometry: a workgroup of
// WW waves shares one copy of the weight fragments (40 KiB of LDS, staged
// once behind the kernel's only barrier); each wave then walks its own
// contiguous range of 16*NB-output tiles with a wave-private input strip
// (positions o0 - halo .. o0 + 16*NB - 1), so no tile ever waits at a
// workgroup barrier.  Several waves per SIMD, out of phase with each other,
// keep the matrix pipe busy while any one of them stages its next strip or
// issues its stores.  Neighbouring tiles both read the strip halo.
// HP: strip positions before a tile's first output: DIL*(K-1) without
// padding; with a pad the strip is shifted by the pad rounded up to a
// multiple of 4 (so its float4 pieces stay aligned) and needs up to 3 more.
template <int CIN4, int K, int DIL, int NB, int WW, int HP = DIL * (K - 1)>
struct WaveGeom {
    static constexpr int kThreads = 64 * WW;
    static constexpr int kTW = 16 * NB;                             // outputs per wave tile
    static constexpr int kKsteps = CIN4 * K / 4;
    static constexpr int kHalo = HP;
    static constexpr int kTs = kTW + kHalo;                         // strip positions
    // row stride >= kTs with stride mod 64 in {16, 48} words: the four
    // 16-lane groups of a B-fragment read (rows kq = 0..3) hit disjoint banks
    static constexpr int kStr16 = kTs <= 16 ? 16 : (kTs - 16 + 63) / 64 * 64 + 16;
    static constexpr int kStr48 = kTs <= 48 ? 48 : (kTs - 48 + 63) / 64 * 64 + 48;
    static constexpr int kStr = kStr16 < kStr48 ? kStr16 : kStr48;
    static constexpr int kQ = CIN4 * kTs / 4;                       // float4 pieces per strip
    static constexpr int kQPerLane = (kQ + 63) / 64;
    static constexpr int kWfrag = 4 * kKsteps * 64;                 // floats
    static constexpr int kLdsFloats = kWfrag + kCO + WW * CIN4 * kStr;
};

// Stride 1 with padding: output o of the padded call is output o + pad of
// the unpadded one (output padding only extends the window at the end), so
// the kernel runs unchanged over tiles of o with the input strip of a tile
// starting at o0 + shift - HP, shift = pad rounded up to a multiple of 4
// (HP > DIL*(K-1) instantiations only; the unpadded one folds both to 0).
// RAGGED: Lo % 4 != 0 or y not 16-byte aligned (rows start at any 4-byte
// boundary); the aligned instantiation carries no tail stores.
template <int CIN4, int K, int DIL, int NB, int WW, int HP = DIL * (K - 1), bool RAGGED = false>
__global__ __launch_bounds__(64 * WW, 1)
void convT1d_f32_wave_kernel(const float *__restrict__ x, const float *__restrict__ w,
                             const float *__restrict__ bias, int Cin, int L, int Cout, int Lo,
                             int tiles_per_n, int ntiles, int pad_arg, float *__restrict__ y)
{
    typedef WaveGeom<CIN4, K, DIL, NB, WW, HP> G;
    static_assert(HP % 4 == 0 && HP >= DIL * (K - 1), "strip halo");
    const int pad = HP == DIL * (K - 1) ? 0 : pad_arg;
    const int shift = (pad + 3) & ~3;                        // strip offset, a multiple of 4
    static_assert(G::kStr >= G::kTs && (G::kStr % 64 == 16 || G::kStr % 64 == 48), "strip row stride");
    static_assert(G::kHalo % 4 == 0, "halo in whole float4 pieces");
    static_assert(G::kQPerLane <= 32, "piece mask");
    static_assert(G::kLdsFloats * 4 <= 160 * 1024, "LDS of one workgroup");
    typedef float v4f_ __attribute__((ext_vector_type(4)));
    extern __shared__ float lds[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    float *wfrag = lds;                                      // [j][lane][m]
    float *bsh = lds + G::kWfrag;                            // [64] bias of the channel block
    float *xs = bsh + kCO + wave * CIN4 * G::kStr;           // this wave's [CIN4][kStr]
    const int cog = blockIdx.y;
    const int kq = lane >> 4, col = lane & 15;

    for (int e = threadIdx.x; e < G::kWfrag; e += G::kThreads) {
        const int m = e & 3, l = (e >> 2) & 63, j = e >> 8;
        const int co = cog * kCO + 16 * m + (l & 15);
        const int kap = 4 * j + (l >> 4);
        const int k = kap / CIN4, ci = kap % CIN4;
        wfrag[e] = (co < Cout && ci < Cin) ? w[((int64_t)ci * Cout + co) * K + k] : 0.0f;
    }
    if (threadIdx.x < kCO) {
        const int co = cog * kCO + threadIdx.x;
        bsh[threadIdx.x] = (bias && co < Cout) ? bias[co] : 0.0f;
    }

    // this wave's contiguous tile range (workgroups in XCD-aware order)
    const int64_t gw = xcd_remap(blockIdx.x, gridDim.x) * WW + wave;
    const int64_t nw = (int64_t)gridDim.x * WW;
    const int per = (int)(ntiles / nw), rem = (int)(ntiles % nw);
    const int t_begin = (int)(gw * per + (gw < rem ? gw : rem));
    const int t_end = t_begin + per + (gw < rem ? 1 : 0);

    // strip piece q = ci * (kTs/4) + t4; unconditional loads from clamped
    // addresses (L % 4 == 0: a piece is wholly inside or outside [0, L)),
    // masked when written.  When a tile continues the previous tile of the
    // same batch item, its halo pieces (t4 < kHalo/4) are the previous
    // strip's last kHalo positions: they are copied inside LDS, not loaded
    // (their load slot reads x[0..], so every tile issues the same number of
    // loads), and the tile fetches only its own kTW positions per channel.
    v4f_ pre[G::kQPerLane];
    unsigned pok = 0;                                        // bit i: piece i is loaded data
    unsigned pput = 0;                                       // bit i: piece i is written
    auto fetch = [&](int tile, bool carry) {
        const int n = tile / tiles_per_n;
        const int o0 = (tile - n * tiles_per_n) * G::kTW;
        const float *xb = x + (int64_t)n * Cin * L + (o0 + shift - G::kHalo);
#pragma unroll
        for (int i = 0; i < G::kQPerLane; ++i) {
            const int q = lane + 64 * i;
            const int ci = q / (G::kTs / 4), t4 = q % (G::kTs / 4);
            const int pos = o0 + shift - G::kHalo + 4 * t4;
            const bool mine = q < G::kQ && !(carry && t4 < G::kHalo / 4);
            const bool ok = mine && ci < Cin && pos >= 0 && pos < L;
            pre[i] = *reinterpret_cast<const v4f_ *>(ok ? xb + ci * L + 4 * t4 : x);
            pok = ok ? pok | (1u << i) : pok & ~(1u << i);
            pput = mine ? pput | (1u << i) : pput & ~(1u << i);
        }
    };
    if (t_begin < t_end) fetch(t_begin, false);
    __syncthreads();                                         // weights and bias staged

    // lane's B base: strip index of input o + pad - DIL*k is
    // o - o0 + HP - (shift - pad) - DIL*k
    const float *xl = xs + kq * G::kStr + G::kHalo - (shift - pad) + col;
    const float *al = wfrag + lane * 4;                      // lane's A base
    for (int tile = t_begin; tile < t_end; ++tile) {
        const int n = tile / tiles_per_n;
        const int o0 = (tile - n * tiles_per_n) * G::kTW;
        // this wave alone reads and writes its strip, and a wave's LDS
        // operations complete in order: compiler-only fences suffice
        __builtin_amdgcn_wave_barrier();
        if (tile > t_begin && o0 > 0) {
            // halo = the previous strip's positions kTW .. kTW+kHalo-1, moved
            // to the front before the new pieces overwrite them
            constexpr int kHq = CIN4 * (G::kHalo / 4);      // halo pieces
            v4f_ hv[(kHq + 63) / 64];
#pragma unroll
            for (int i = 0; i < (kHq + 63) / 64; ++i) {
                const int q = lane + 64 * i;
                const int ci = q / (G::kHalo / 4), u = q % (G::kHalo / 4);
                hv[i] = *reinterpret_cast<const v4f_ *>(xs + min(ci, CIN4 - 1) * G::kStr + G::kTW + 4 * u);
            }
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int i = 0; i < (kHq + 63) / 64; ++i) {
                const int q = lane + 64 * i;
                const int ci = q / (G::kHalo / 4), u = q % (G::kHalo / 4);
                if (q < kHq) *reinterpret_cast<v4f_ *>(xs + ci * G::kStr + 4 * u) = hv[i];
            }
            __builtin_amdgcn_wave_barrier();
        }
#pragma unroll
        for (int i = 0; i < G::kQPerLane; ++i) {
            const int q = lane + 64 * i;
            if ((pput >> i) & 1) {
                const int ci = q / (G::kTs / 4), t4 = q % (G::kTs / 4);
                *reinterpret_cast<v4f_ *>(xs + ci * G::kStr + 4 * t4) =
                    ((pok >> i) & 1) ? pre[i] : (v4f_){0.0f, 0.0f, 0.0f, 0.0f};
            }
        }
        __builtin_amdgcn_wave_barrier();
        if (tile + 1 < t_end) {
            // the next tile continues this one when it is in the same batch item
            const int n1 = (tile + 1) / tiles_per_n;
            fetch(tile + 1, n1 == n);
        }

        // The MFMAs run with the operands swapped, D = Y^T (16 outputs x 16
        // channels): lane (kq, col) holds outputs 16b + 4kq .. +3 of channel
        // 16m + col, four consecutive floats of one output row.  Each
        // accumulator starts at its channel's bias.
        v4f acc[4][NB];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const float bc = bsh[16 * m + col];
            const v4f b4 = {bc, bc, bc, bc};
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[m][b] = b4;
        }
        // 40 k-steps fully unrolled, fragments double-buffered in registers:
        // step s+1's LDS reads are issued before step s's MFMAs (the
        // scheduling barriers keep that order), so the MFMAs never wait on
        // a read issued just before them
        constexpr int kSteps = K * (CIN4 / 4);
        v4f_ fa[2];
        float fb[2][NB];
        auto ldf = [&](int s, int buf) {
            const int k = s / (CIN4 / 4), c = s % (CIN4 / 4);
            fa[buf] = *reinterpret_cast<const v4f_ *>(al + s * 256);
#pragma unroll
            for (int b = 0; b < NB; ++b) fb[buf][b] = xl[-DIL * k + 4 * c * G::kStr + 16 * b];
        };
        ldf(0, 0);
#pragma unroll
        for (int s = 0; s < kSteps; ++s) {
            if (s + 1 < kSteps) ldf(s + 1, (s + 1) & 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    acc[m][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(fb[s & 1][b], fa[s & 1][m], acc[m][b], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }

        // 16-byte buffer stores over this batch item's output (word 3
        // 0x00020000: 32-bit data format) of every lane whose four outputs
        // lie wholly inside [0, Lo); masked lanes store past the range, which
        // the hardware drops, so no store sits behind a branch and every tile
        // issues the same number of stores (4*NB, well under the 63 memory
        // operations a wave can have in flight, so waiting for the next
        // strip's loads never waits for this tile's stores).  A row starts
        // 16-byte aligned only when Lo % 4 == 0 and y is; otherwise the
        // stores are 4-byte aligned, which gfx950's vector memory accepts
        // (the compiler emits such 16-byte stores for 4-byte-aligned
        // vectors).
        const __amdgpu_buffer_rsrc_t yr =
            __builtin_amdgcn_make_buffer_rsrc(y + (int64_t)n * Cout * Lo, 0, Cout * Lo * 4, 0x00020000);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int co = cog * kCO + 16 * m + col;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const int o = o0 + 16 * b + 4 * kq;
                const int off = (co < Cout && o + 4 <= Lo) ? (co * Lo + o) * 4 : 0x7ffffff0;   // past the range
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, acc[m][b]), yr, off, 0, 0);
            }
        }
        // Lo % 4 != 0: the last 1-3 outputs of each row belong to a lane
        // whose vector runs past Lo; only the tile holding the row end (a
        // wave-uniform test) stores them one by one
        if (RAGGED && (Lo & 3) != 0 && o0 + G::kTW > (Lo & ~3)) {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int co = cog * kCO + 16 * m + col;
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const int o = o0 + 16 * b + 4 * kq;
                    if (co < Cout && o < Lo && o + 4 > Lo) {
#pragma unroll
                        for (int r = 0; r < 3; ++r)
                            if (o + r < Lo)
                                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[m][b][r]), yr,
                                                                      (co * Lo + o + r) * 4, 0, 0);
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Strided transposed convolution as S stride-1 gathers ([p74], passage on
// the general-stride gather x[(o + pad - dil*k)/stride]): with o + pad =
// S*q + rho (0 <= rho < S), output o takes exactly the taps k with
// dil*k = rho (mod S), each from input i = q - delta_k,
// delta_k = (dil*k - rho)/S >= 0.  So residue class rho is a stride-1
// dilated gather over q with its own taps and shifts, every class reads the
// same inputs x[q - delta], and the taps of all classes together are the K
// taps once each.  On the matrix cores a wave tile is 16*NB consecutive q
// of one batch item and 64 output channels; for each class the same input
// strip x[n, :, q0 - HP .. q0 + 16*NB - 1] serves as the B operand at that
// class's shifts, so a tile runs K*CIN4/4 k-steps in all, as at stride 1.
// f(std::integral_constant<int, R>) for R = B .. E-1, in order
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

template <int K, int DIL, int S>
struct Poly {
    static constexpr int count(int rho)
    {
        int c = 0;
        for (int k = 0; k < K; ++k) c += ((DIL * k) % S == rho) ? 1 : 0;
        return c;
    }
    static constexpr int tap(int rho, int idx)        // idx-th tap of class rho
    {
        int c = 0;
        for (int k = 0; k < K; ++k)
            if ((DIL * k) % S == rho) {
                if (c == idx) return k;
                ++c;
            }
        return 0;
    }
    static constexpr int delta(int rho, int idx) { return (DIL * tap(rho, idx) - rho) / S; }
    static constexpr int first(int rho)               // taps of the classes before rho
    {
        int c = 0;
        for (int r = 0; r < rho; ++r) c += count(r);
        return c;
    }
    static constexpr int dmax()
    {
        int m = 0;
        for (int k = 0; k < K; ++k) {
            const int dd = (DIL * k - (DIL * k) % S) / S;
            m = dd > m ? dd : m;
        }
        return m;
    }
    static constexpr int kHalo = (dmax() + 3) / 4 * 4;  // strip positions before q0
};

template <int CIN4, int K, int DIL, int S, int NB, int WW>
struct PolyGeom {
    typedef Poly<K, DIL, S> P;
    static constexpr int kThreads = 64 * WW;
    static constexpr int kTQ = 16 * NB;                             // q per wave tile
    static constexpr int kKsteps = CIN4 * K / 4;
    static constexpr int kTs = kTQ + P::kHalo;                      // strip positions
    static constexpr int kStr16 = kTs <= 16 ? 16 : (kTs - 16 + 63) / 64 * 64 + 16;
    static constexpr int kStr48 = kTs <= 48 ? 48 : (kTs - 48 + 63) / 64 * 64 + 48;
    static constexpr int kStr = kStr16 < kStr48 ? kStr16 : kStr48;
    static constexpr int kQ = CIN4 * kTs / 4;                       // float4 pieces per strip
    static constexpr int kQPerLane = (kQ + 63) / 64;
    static constexpr int kWfrag = 4 * kKsteps * 64;                 // floats
    static constexpr int kLdsFloats = kWfrag + kCO + WW * CIN4 * kStr;
};

template <int CIN4, int K, int DIL, int S, int NB, int WW>
__global__ __launch_bounds__(64 * WW, 1)
void convT1d_f32_poly_kernel(const float *__restrict__ x, const float *__restrict__ w,
                             const float *__restrict__ bias, int Cin, int L, int Cout, int Lo,
                             int pad, int qa4, int tq_per_n, int ntiles, float *__restrict__ y)
{
    typedef PolyGeom<CIN4, K, DIL, S, NB, WW> G;
    typedef Poly<K, DIL, S> P;
    static_assert(G::kStr >= G::kTs && (G::kStr % 64 == 16 || G::kStr % 64 == 48), "strip row stride");
    static_assert(G::kQPerLane <= 32, "piece mask");
    static_assert(G::kLdsFloats * 4 <= 160 * 1024, "LDS of one workgroup");
    typedef float v4f_ __attribute__((ext_vector_type(4)));
    constexpr int HP = P::kHalo;
    extern __shared__ float lds[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    float *wfrag = lds;                                      // [js][lane][m]
    float *bsh = lds + G::kWfrag;                            // [64] bias of the channel block
    float *xs = bsh + kCO + wave * CIN4 * G::kStr;           // this wave's [CIN4][kStr]
    const int cog = blockIdx.y;
    const int kq = lane >> 4, col = lane & 15;

    // Fragments in class order: k-step js = (first(rho) + idx)*(CIN4/4) + c
    // holds A[co = 16m + l%16][kappa = l/16] = w[4c + l/16, co, tap(rho, idx)].
    for (int e = threadIdx.x; e < G::kWfrag; e += G::kThreads) {
        const int m = e & 3, l = (e >> 2) & 63, js = e >> 8;
        const int t = js / (CIN4 / 4), c = js % (CIN4 / 4);   // t-th tap in class order
        int k = 0;
#pragma unroll
        for (int rho = 0; rho < S; ++rho)
#pragma unroll
            for (int idx = 0; idx < P::count(rho); ++idx)
                if (P::first(rho) + idx == t) k = P::tap(rho, idx);
        const int co = cog * kCO + 16 * m + (l & 15);
        const int ci = 4 * c + (l >> 4);
        wfrag[e] = (co < Cout && ci < Cin) ? w[((int64_t)ci * Cout + co) * K + k] : 0.0f;
    }
    if (threadIdx.x < kCO) {
        const int co = cog * kCO + threadIdx.x;
        bsh[threadIdx.x] = (bias && co < Cout) ? bias[co] : 0.0f;
    }

    // this wave's contiguous tile range (workgroups in XCD-aware order)
    const int64_t gw = xcd_remap(blockIdx.x, gridDim.x) * WW + wave;
    const int64_t nw = (int64_t)gridDim.x * WW;
    const int per = (int)(ntiles / nw), rem = (int)(ntiles % nw);
    const int t_begin = (int)(gw * per + (gw < rem ? gw : rem));
    const int t_end = t_begin + per + (gw < rem ? 1 : 0);

    // byte offset of this lane's output row co = cog*64 + 4kq within a batch
    // item (an item's output is below 2^31 bytes; rows 16m + r further on
    // add a wave-uniform multiple of Lo) and the rows left in the block
    const int row0b = (cog * kCO + 4 * kq) * Lo * 4;
    const int rows_left = Cout - cog * kCO - 4 * kq;

    // strip piece q = ci * (kTs/4) + t4 covers inputs q0 - HP + 4*t4 .. +3
    // (L % 4 == 0 and q0 - HP = 0 mod 4: a piece is wholly inside or outside
    // [0, L)); as in the stride-1 kernel, a tile that continues the previous
    // one takes its halo from the previous strip inside LDS.
    v4f_ pre[G::kQPerLane];
    unsigned pok = 0, pput = 0;
    auto fetch = [&](int tile, bool carry) {
        const int n = tile / tq_per_n;
        const int q0 = qa4 + (tile - n * tq_per_n) * G::kTQ;
        const float *xn = x + (int64_t)n * Cin * L;
#pragma unroll
        for (int i = 0; i < G::kQPerLane; ++i) {
            const int qq = lane + 64 * i;
            const int ci = qq / (G::kTs / 4), t4 = qq % (G::kTs / 4);
            const int pos = q0 - HP + 4 * t4;
            const bool mine = qq < G::kQ && !(carry && t4 < HP / 4);
            const bool ok = mine && ci < Cin && pos >= 0 && pos < L;
            pre[i] = *reinterpret_cast<const v4f_ *>(ok ? xn + (int64_t)ci * L + pos : x);
            pok = ok ? pok | (1u << i) : pok & ~(1u << i);
            pput = mine ? pput | (1u << i) : pput & ~(1u << i);
        }
    };
    if (t_begin < t_end) fetch(t_begin, false);
    __syncthreads();                                         // weights and bias staged

    const float *xl = xs + kq * G::kStr + HP + col;         // lane's B base (q = q0 + col)
    const float *al = wfrag + lane * 4;                      // lane's A base
    for (int tile = t_begin; tile < t_end; ++tile) {
        const int n = tile / tq_per_n;
        const int q0 = qa4 + (tile - n * tq_per_n) * G::kTQ;
        __builtin_amdgcn_wave_barrier();
        if (HP > 0 && tile > t_begin && tile - n * tq_per_n > 0) {
            constexpr int kHq = CIN4 * (HP > 0 ? HP / 4 : 1);
            v4f_ hv[(kHq + 63) / 64];
#pragma unroll
            for (int i = 0; i < (kHq + 63) / 64; ++i) {
                const int qq = lane + 64 * i;
                const int ci = qq / (HP / 4), u = qq % (HP / 4);
                hv[i] = *reinterpret_cast<const v4f_ *>(xs + min(ci, CIN4 - 1) * G::kStr + G::kTQ + 4 * u);
            }
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int i = 0; i < (kHq + 63) / 64; ++i) {
                const int qq = lane + 64 * i;
                const int ci = qq / (HP / 4), u = qq % (HP / 4);
                if (qq < kHq) *reinterpret_cast<v4f_ *>(xs + ci * G::kStr + 4 * u) = hv[i];
            }
            __builtin_amdgcn_wave_barrier();
        }
#pragma unroll
        for (int i = 0; i < G::kQPerLane; ++i) {
            const int qq = lane + 64 * i;
            if ((pput >> i) & 1) {
                const int ci = qq / (G::kTs / 4), t4 = qq % (G::kTs / 4);
                *reinterpret_cast<v4f_ *>(xs + ci * G::kStr + 4 * t4) =
                    ((pok >> i) & 1) ? pre[i] : (v4f_){0.0f, 0.0f, 0.0f, 0.0f};
            }
        }
        __builtin_amdgcn_wave_barrier();
        if (tile + 1 < t_end) {
            const int n1 = (tile + 1) / tq_per_n;
            fetch(tile + 1, n1 == n);
        }

        const __amdgpu_buffer_rsrc_t yr =
            __builtin_amdgcn_make_buffer_rsrc(y + (int64_t)n * Cout * Lo, 0, Cout * Lo * 4, 0x00020000);
        // D[co][q] (operands not swapped): lane (kq, col) holds channel
        // 16m + 4kq + r at q = q0 + 16b + col; class rho's value there is
        // output o = S*q + rho - pad.
        v4f acc[S][4][NB];
        static_for<0, S>([&](auto rc) {
            constexpr int rho = decltype(rc)::value;
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float bc = bsh[16 * m + 4 * kq + r];
#pragma unroll
                    for (int b = 0; b < NB; ++b) acc[rho][m][b][r] = bc;
                }
            constexpr int kSteps = P::count(rho) * (CIN4 / 4);
            v4f_ fa[2];
            float fb[2][NB];
            auto ldf = [&](int st, int buf) {
                const int idx = st / (CIN4 / 4), c = st % (CIN4 / 4);
                const int dl = P::delta(rho, idx);
                fa[buf] = *reinterpret_cast<const v4f_ *>(al + ((P::first(rho) + idx) * (CIN4 / 4) + c) * 256);
#pragma unroll
                for (int b = 0; b < NB; ++b) fb[buf][b] = xl[-dl + 4 * c * G::kStr + 16 * b];
            };
            if constexpr (kSteps > 0) ldf(0, 0);     // a class without taps keeps the bias
#pragma unroll
            for (int st = 0; st < kSteps; ++st) {
                if (st + 1 < kSteps) ldf(st + 1, (st + 1) & 1);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int m = 0; m < 4; ++m)
#pragma unroll
                    for (int b = 0; b < NB; ++b)
                        acc[rho][m][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[st & 1][m], fb[st & 1][b], acc[rho][m][b], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        });

        // Stores.  Class rho at q is output S*q + rho - pad, so a lane's S
        // values at q are S consecutive outputs: one 8-, 12- or 16-byte store
        // for S = 2, 3 or 4 (two stores, 16 bytes and the rest, for S = 5 to
        // 8), and 16 lanes write 16*S contiguous floats of one channel.  The vector is 4-byte aligned when pad or
        // Lo is not a multiple of S (gfx950's vector memory accepts such
        // stores; the compiler emits them for 4-byte-aligned data).  Tiles
        // whose outputs reach past either end of the row take one 4-byte
        // store per output instead.
        const int olo = S * q0 - pad, ohi = S * (q0 + G::kTQ) - 1 - pad;   // tile's first, last output
        const bool grouped = olo >= 0 && ohi < Lo;
        if (grouped) {
            typedef int v2i_ __attribute__((ext_vector_type(2)));
            typedef int v3i_ __attribute__((ext_vector_type(3)));
            typedef int v4i_ __attribute__((ext_vector_type(4)));
            // byte offset of this lane's first group in row co = 16m + 4kq + r
            // of the channel block (row0b plus (16m + r) rows), and an offset
            // past the output for lanes that store nothing (with the
            // constant per-block offsets added it stays below 2^32 and above
            // the output's size)
            constexpr unsigned kOff = 0x80000000u;
            const int ob = (S * (q0 + col) - pad) * 4;
#pragma unroll
            for (int m = 0; m < 4; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const bool rowok = 16 * m + r < rows_left;
                    const int rowb = row0b + (16 * m + r) * Lo * 4;
                    const unsigned base = rowok ? (unsigned)(rowb + ob) : kOff;
#pragma unroll
                    for (int b = 0; b < NB; ++b) {
                        // identity DPP moves: the group goes out through
                        // VGPRs (taken straight from the accumulators, whose
                        // values are not adjacent registers, it made the
                        // compiler spill 85 registers)
                        int v[S];
                        static_for<0, S>([&](auto rc) {
                            constexpr int rho = decltype(rc)::value;
                            v[rho] = __builtin_amdgcn_update_dpp(
                                0, __float_as_int(acc[rho][m][b][r]), 0xE4, 0xf, 0xf, false);   // quad_perm:[0,1,2,3]
                        });
                        // 16 q = 16*S outputs per block; the group goes out
                        // in pieces of up to four values
                        static_for<0, (S + 3) / 4>([&](auto pc) {
                            constexpr int c = decltype(pc)::value, n = S - 4 * c < 4 ? S - 4 * c : 4;
                            const int boff = (int)(base + 64u * S * b + 16u * c);
                            if constexpr (n == 1)
                                __builtin_amdgcn_raw_buffer_store_b32(v[4 * c], yr, boff, 0, 0);
                            else if constexpr (n == 2)
                                __builtin_amdgcn_raw_buffer_store_b64((v2i_){v[4 * c], v[4 * c + 1]}, yr, boff, 0, 0);
                            else if constexpr (n == 3)
                                __builtin_amdgcn_raw_buffer_store_b96((v3i_){v[4 * c], v[4 * c + 1], v[4 * c + 2]}, yr, boff, 0, 0);
                            else
                                __builtin_amdgcn_raw_buffer_store_b128((v4i_){v[4 * c], v[4 * c + 1], v[4 * c + 2], v[4 * c + 3]}, yr, boff, 0, 0);
                        });
                    }
                }
        } else {
            static_for<0, S>([&](auto rc) {
                constexpr int rho = decltype(rc)::value;
#pragma unroll
                for (int m = 0; m < 4; ++m)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int co = cog * kCO + 16 * m + 4 * kq + r;
#pragma unroll
                        for (int b = 0; b < NB; ++b) {
                            const int o = S * (q0 + 16 * b + col) + rho - pad;
                            const int off = (co < Cout && o >= 0 && o < Lo) ? (co * Lo + o) * 4 : 0x7ffffff0;
                            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[rho][m][b][r]), yr, off, 0, 0);
                        }
                    }
            });
        }
    }
}

// The configuration the launcher uses for Cin 32, K 5, dilation 3: 64-output
// wave tiles, 8 waves (2 per SIMD) per workgroup.  Measured at the
// [32,32,131072] workload: 710 us, against 720 for 32-output tiles with 12
// or 16 waves and 743 for 256-output workgroup tiles behind barriers.
constexpr int kWaveNB = 4;
constexpr int kWaveWW = 8;

}  // namespace

// LDS bytes the kernel needs for a geometry (weights + input strip).
size_t convT1d_f32_lds_bytes(int64_t Cin, int K, int dilation)
{
    const int64_t cin4 = (Cin + 3) & ~int64_t(3);
    const int64_t ksteps = cin4 * K / 4;
    const int64_t ts = kTO + (int64_t)dilation * (K - 1);
    int64_t str = ((ts + 63) / 64) * 64 + 16;        // % 64 == 16
    if (str - 64 >= ts) str -= 64;
    return (size_t)(4 * ksteps * 64 + cin4 * str) * sizeof(float);
}

bool convT1d_f32_wave_supported(int64_t Cin, int K, int dilation, int64_t L, const void *x)
{
    return Cin == 32 && K == 5 && dilation == 3 && L % 4 == 0 && (((uintptr_t)x) & 15) == 0;
}

namespace {
template <int HP, bool RAGGED>
hipError_t launch_wave(const float *x, const float *w, const float *bias, int64_t N, int64_t Cin,
                       int64_t L, int64_t Cout, int64_t Lo, int pad, float *out, hipStream_t stream)
{
    typedef WaveGeom<32, 5, 3, kWaveNB, kWaveWW, HP> G;
    const void *fn = (const void *)convT1d_f32_wave_kernel<32, 5, 3, kWaveNB, kWaveWW, HP, RAGGED>;
    const size_t lds = (size_t)G::kLdsFloats * sizeof(float);
    hipError_t e = allow_dynamic_lds(fn, lds);
    if (e != hipSuccess) return e;
    const int cus = device_cus(), per_cu = occupancy(fn, G::kThreads, lds);
    const int wtiles_per_n = (int)((Lo + G::kTW - 1) / G::kTW);
    const int64_t wtiles = N * wtiles_per_n;
    const unsigned gy = (unsigned)((Cout + kCO - 1) / kCO);
    int64_t gx = (int64_t)cus * per_cu / gy;
    if (gx < 1) gx = 1;
    hipLaunchKernelGGL((convT1d_f32_wave_kernel<32, 5, 3, kWaveNB, kWaveWW, HP, RAGGED>), dim3((unsigned)gx, gy),
                       dim3(G::kThreads), lds, stream, x, w, bias, (int)Cin, (int)L, (int)Cout,
                       (int)Lo, wtiles_per_n, (int)wtiles, pad, out);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_convT1d_f32(const float *x, const float *w, const float *bias,
                              int64_t N, int64_t Cin, int64_t L, int64_t Cout,
                              int K, int dilation, int pad, int out_pad, float *out,
                              hipStream_t stream)
{
    const int cin4 = (int)((Cin + 3) & ~int64_t(3));
    const int64_t Lo = L + (int64_t)dilation * (K - 1) - 2 * (int64_t)pad + out_pad;
    if (convT1d_f32_wave_supported(Cin, K, dilation, L, x)) {
        const bool ragged = Lo % 4 != 0 || (((uintptr_t)out) & 15) != 0;
        if (pad == 0 && out_pad == 0)
            return ragged ? launch_wave<12, true>(x, w, bias, N, Cin, L, Cout, Lo, 0, out, stream)
                          : launch_wave<12, false>(x, w, bias, N, Cin, L, Cout, Lo, 0, out, stream);
        return ragged ? launch_wave<16, true>(x, w, bias, N, Cin, L, Cout, Lo, pad, out, stream)
                      : launch_wave<16, false>(x, w, bias, N, Cin, L, Cout, Lo, pad, out, stream);
    }
    if (pad != 0 || out_pad != 0) return hipErrorInvalidValue;   // the tile kernel has no shift
    const int tiles_per_n = (int)((Lo + kTO - 1) / kTO);
    const int64_t ntiles = N * tiles_per_n;
    const int64_t ts = kTO + (int64_t)dilation * (K - 1);
    int64_t str = ((ts + 63) / 64) * 64 + 16;
    if (str - 64 >= ts) str -= 64;
    const size_t lds = convT1d_f32_lds_bytes(Cin, K, dilation);
    hipError_t e = allow_dynamic_lds((const void *)convT1d_f32_kernel, lds);
    if (e != hipSuccess) return e;
    const int cus = device_cus();
    const int per_cu = lds <= 80 * 1024 ? 2 : 1;
    int64_t gx = (int64_t)cus * per_cu;
    if (gx > ntiles) gx = ntiles;
    const unsigned gy = (unsigned)((Cout + kCO - 1) / kCO);
    hipLaunchKernelGGL(convT1d_f32_kernel, dim3((unsigned)gx, gy), dim3(kThreads), lds, stream,
                       x, w, bias, (int)Cin, cin4, (int)L, (int)Cout, K, dilation, (int)Lo,
                       tiles_per_n, (int)ntiles, (int)str, out);
    return hipGetLastError();
}

bool convT1d_f32_poly_supported(int64_t Cin, int K, int stride, int dilation, int64_t L,
                                const void *x)
{
    return Cin == 32 && K == 5 && dilation == 3 && stride >= 2 && stride <= 8 && L % 4 == 0 &&
           (((uintptr_t)x) & 15) == 0;
}

namespace {
template <int S, int NB, int WW>
hipError_t launch_poly(const float *x, const float *w, const float *bias, int64_t N, int64_t Cin,
                       int64_t L, int64_t Cout, int K, int pad, int dilation, int out_pad,
                       float *out, hipStream_t stream)
{
    typedef PolyGeom<32, 5, 3, S, NB, WW> G;
    const int64_t Lo = (L - 1) * S - 2 * (int64_t)pad + (int64_t)dilation * (K - 1) + out_pad + 1;
    // q covers o + pad = S*q + rho for every output: q in [pad/S, ceil((Lo + pad)/S)),
    // started at a multiple of 4 so that strip pieces stay float4-aligned
    const int64_t qa4 = ((int64_t)pad / S) & ~int64_t(3);
    const int64_t qb = (Lo + pad + S - 1) / S;
    const int tq_per_n = (int)((qb - qa4 + G::kTQ - 1) / G::kTQ);
    const int64_t ntiles = N * tq_per_n;
    const void *fn = (const void *)convT1d_f32_poly_kernel<32, 5, 3, S, NB, WW>;
    const size_t lds = (size_t)G::kLdsFloats * sizeof(float);
    hipError_t e = allow_dynamic_lds(fn, lds);
    if (e != hipSuccess) return e;
    const int cus = device_cus(), per_cu = occupancy(fn, G::kThreads, lds);
    const unsigned gy = (unsigned)((Cout + kCO - 1) / kCO);
    int64_t gx = (int64_t)cus * per_cu / gy;
    if (gx < 1) gx = 1;
    hipLaunchKernelGGL((convT1d_f32_poly_kernel<32, 5, 3, S, NB, WW>), dim3((unsigned)gx, gy),
                       dim3(G::kThreads), lds, stream, x, w, bias, (int)Cin, (int)L, (int)Cout,
                       (int)Lo, pad, (int)qa4, tq_per_n, (int)ntiles, out);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_convT1d_f32_poly(const float *x, const float *w, const float *bias, int64_t N,
                                   int64_t Cin, int64_t L, int64_t Cout, int K, int stride,
                                   int pad, int dilation, int out_pad, float *out,
                                   hipStream_t stream)
{
    if (!convT1d_f32_poly_supported(Cin, K, stride, dilation, L, x)) return hipErrorInvalidValue;
    // 4-wave workgroups at one wave per SIMD, each wave's S classes x 4
    // channel blocks x NB 16-q blocks of accumulators (192 registers) in the
    // accumulation registers beside 256 vector registers.  Stride 2: 96-q
    // tiles (6 blocks); against 32-q tiles at two waves per SIMD (no room for
    // more accumulators) the larger tile spreads each tile's strip handling
    // and store setup over three times the MFMAs: 1.04 -> 0.91 ms at the
    // page's stride-2 shape.  Stride 3: 64-q tiles (4 blocks); stride 4: 48-q
    // tiles (3 blocks).
    if (stride == 2)
        return launch_poly<2, 6, 4>(x, w, bias, N, Cin, L, Cout, K, pad, dilation, out_pad, out,
                                    stream);
    if (stride == 3)
        return launch_poly<3, 4, 4>(x, w, bias, N, Cin, L, Cout, K, pad, dilation, out_pad, out,
                                    stream);
    if (stride == 4)
        return launch_poly<4, 3, 4>(x, w, bias, N, Cin, L, Cout, K, pad, dilation, out_pad, out,
                                    stream);
    // Strides 5 to 8: 32-q tiles, except 48-q at stride 5 and 16-q tiles
    // in 8-wave workgroups (two waves per SIMD) at stride 7, each 4-7% faster
    // than 32-q tiles at the page's size; the other choices measured slower.
    if (stride == 5)
        return launch_poly<5, 3, 4>(x, w, bias, N, Cin, L, Cout, K, pad, dilation, out_pad, out,
                                    stream);
    if (stride == 6)
        return launch_poly<6, 2, 4>(x, w, bias, N, Cin, L, Cout, K, pad, dilation, out_pad, out,
                                    stream);
    if (stride == 7)
        return launch_poly<7, 1, 8>(x, w, bias, N, Cin, L, Cout, K, pad, dilation, out_pad, out,
                                    stream);
    return launch_poly<8, 2, 4>(x, w, bias, N, Cin, L, Cout, K, pad, dilation, out_pad, out, stream);
}

}  // namespace ct
