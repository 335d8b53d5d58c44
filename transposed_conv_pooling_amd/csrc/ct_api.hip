// ct_api.hip - the extern "C" boundary declared in include/ct.h.
//
// Each entry point validates every argument on the host first (no HIP call
// happens before a request is accepted), then calls one launcher from the
// kernel files and maps a launch error to CT_EHIP.
#include <cstdarg>
#include <initializer_list>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "ct.h"
#include "ct_internal.h"

namespace ct {
size_t convT1d_f32_lds_bytes(int64_t Cin, int K, int dilation);
size_t fused3d_bf16_lds_bytes(int64_t Cin, int64_t W);
}

namespace {

constexpr int64_t kI32Max = 2147483647;
constexpr size_t kLdsMax = 160 * 1024;      // gfx950 LDS per workgroup

thread_local char g_err[512] = "";

ct_status fail(ct_status s, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

ct_status ok()
{
    g_err[0] = '\0';
    return CT_OK;
}

// a * b into *r; false on overflow or negative operands.
bool mul(int64_t a, int64_t b, int64_t *r)
{
    if (a < 0 || b < 0) return false;
    if (a != 0 && b > INT64_MAX / a) return false;
    *r = a * b;
    return true;
}

bool prod(std::initializer_list<int64_t> v, int64_t *r)
{
    int64_t p = 1;
    for (int64_t t : v)
        if (!mul(p, t, &p)) return false;
    *r = p;
    return true;
}

bool overlap(const void *a, int64_t abytes, const void *b, int64_t bbytes)
{
    if (!a || !b || abytes <= 0 || bbytes <= 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

int dtype_size(int dt) { return dt == CT_F32 ? 4 : dt == CT_BF16 ? 2 : 0; }

ct_status hip_status(hipError_t e, const char *what)
{
    if (e == hipSuccess) return ok();
    return fail(CT_EHIP, "%s: %s", what, hipGetErrorString(e));
}


// Limits of the general-geometry kernels: they index one axis in 32-bit
// arithmetic (o + pad - k, i * stride), so every length, pad and stride stays
// below 2^30 and the kernel / pool size below 2^10 (a window already holds
// 2^30 taps there).
constexpr int64_t kGenericMaxLen = int64_t(1) << 30;
constexpr int kGenericMaxTap = 1024;

// Checks shared by the fused chain and the standalone ConvTranspose3d:
// pointers, dtypes, sizes, PyTorch's rule out_pad < stride (dilation 1),
// non-empty convolution output (od[]), alignment of x, w and out, and the
// general kernel's index range.
ct_status check_convT3d(const char *fn, const void *x, int x_dtype, const void *w, int w_dtype,
                        int64_t N, int64_t Cin, int64_t D, int64_t H, int64_t W, int64_t Cout,
                        int k, int stride, int pad, int out_pad, const float *out, int *xs,
                        int *ws, int64_t od[3])
{
    if (!x || !w || !out) return fail(CT_EINVAL, "%s: x, w and out must be non-null", fn);
    *xs = dtype_size(x_dtype);
    *ws = dtype_size(w_dtype);
    if (!*xs || !*ws) return fail(CT_EINVAL, "%s: unknown dtype (%d, %d)", fn, x_dtype, w_dtype);
    if (N < 1 || Cin < 1 || D < 1 || H < 1 || W < 1 || Cout < 1)
        return fail(CT_EINVAL, "%s: sizes must be >= 1 (N=%lld Cin=%lld D=%lld H=%lld W=%lld Cout=%lld)",
                    fn, (long long)N, (long long)Cin, (long long)D, (long long)H, (long long)W,
                    (long long)Cout);
    if (k < 1 || stride < 1 || pad < 0 || out_pad < 0 || out_pad >= stride)
        return fail(CT_EINVAL, "%s: invalid geometry k=%d stride=%d pad=%d out_pad=%d "
                    "(out_pad must be < stride)", fn, k, stride, pad, out_pad);
    const int64_t in[3] = {D, H, W};
    for (int i = 0; i < 3; ++i) {
        od[i] = ct_convT_out_len(in[i], k, stride, pad, out_pad, 1);
        if (od[i] <= 0)
            return fail(CT_EINVAL, "%s: empty output along axis %d (input %lld -> conv %lld)", fn, i,
                        (long long)in[i], (long long)od[i]);
    }
    if (!aligned(x, *xs) || !aligned(w, *ws) || !aligned(out, 4))
        return fail(CT_EINVAL, "%s: misaligned pointer", fn);
    for (int i = 0; i < 3; ++i)
        if (in[i] > kGenericMaxLen || od[i] > kGenericMaxLen)
            return fail(CT_EUNSUPPORTED, "%s: lengths beyond %lld are not implemented", fn,
                        (long long)kGenericMaxLen);
    if (Cin > kGenericMaxLen || Cout > kGenericMaxLen || pad > kGenericMaxLen ||
        k > kGenericMaxTap)
        return fail(CT_EUNSUPPORTED, "%s: Cin, Cout or pad beyond %lld, or k beyond %d, is not "
                    "implemented", fn, (long long)kGenericMaxLen, kGenericMaxTap);
    return CT_OK;
}

}  // namespace

extern "C" {

// Both size formulas are evaluated in 128-bit arithmetic, where no product or
// sum of 64-bit operands overflows; a length outside int64 returns -1.
int64_t ct_convT_out_len(int64_t in, int64_t k, int64_t stride, int64_t pad,
                         int64_t out_pad, int64_t dilation)
{
    const __int128 r = (__int128)(in - (__int128)1) * stride - (__int128)2 * pad +
                       (__int128)dilation * (k - (__int128)1) + out_pad + 1;
    return (r > INT64_MAX || r < INT64_MIN) ? -1 : (int64_t)r;
}

int64_t ct_pool_out_len(int64_t in, int64_t k, int64_t stride, int64_t pad)
{
    if (stride == 0) stride = k;
    if (stride <= 0) return 0;
    const __int128 num = (__int128)in + (__int128)2 * pad - k;
    __int128 q = num / stride;
    if (num % stride != 0 && num < 0) --q;
    const __int128 r = q + 1;
    return (r > INT64_MAX || r < INT64_MIN) ? -1 : (int64_t)r;
}

const char *ct_status_str(int status)
{
    switch (status) {
    case CT_OK: return "CT_OK";
    case CT_EINVAL: return "CT_EINVAL";
    case CT_EUNSUPPORTED: return "CT_EUNSUPPORTED";
    case CT_EHIP: return "CT_EHIP";
    default: return "CT_UNKNOWN_STATUS";
    }
}

const char *ct_last_error(void) { return g_err; }

const char *ct_version(void) { return "transposed_conv_pooling_amd 0.1.0 (gfx950)"; }

ct_status ct_convT3d_scale_pool_bias(
    const void *x, int x_dtype, const void *w, int w_dtype,
    const float *conv_bias, const float *bias, float scale1, float scale2,
    int64_t N, int64_t Cin, int64_t D, int64_t H, int64_t W, int64_t Cout,
    int k, int stride, int pad, int out_pad, int pool_k, int pool_s,
    float *out, void *stream)
{
    const char *fn = "convT3d_scale_pool_bias";
    int xs, ws;
    int64_t od[3];
    ct_status st = check_convT3d(fn, x, x_dtype, w, w_dtype, N, Cin, D, H, W, Cout, k, stride,
                                 pad, out_pad, out, &xs, &ws, od);
    if (st != CT_OK) return st;
    if (pool_k < 1 || pool_s < 0)
        return fail(CT_EINVAL, "%s: invalid pool geometry pool_k=%d pool_s=%d", fn, pool_k, pool_s);
    const int ps = pool_s == 0 ? pool_k : pool_s;
    int64_t pd[3];
    for (int i = 0; i < 3; ++i) {
        pd[i] = ct_pool_out_len(od[i], pool_k, ps, 0);
        if (pd[i] <= 0)
            return fail(CT_EINVAL, "%s: empty output along axis %d (conv %lld -> pool %lld)", fn, i,
                        (long long)od[i], (long long)pd[i]);
    }
    if ((conv_bias && !aligned(conv_bias, 4)) || (bias && !aligned(bias, 4)))
        return fail(CT_EINVAL, "%s: misaligned pointer", fn);
    int64_t nx, nw, no;
    if (!prod({N, Cin, D, H, W, (int64_t)xs}, &nx) ||
        !prod({Cin, Cout, (int64_t)k, (int64_t)k, (int64_t)k, (int64_t)ws}, &nw) ||
        !prod({N, Cout, pd[0], pd[1], pd[2], 4}, &no))
        return fail(CT_EINVAL, "%s: tensor size overflows", fn);
    if (overlap(out, no, x, nx) || overlap(out, no, w, nw) ||
        overlap(out, no, conv_bias, Cout * 4) || overlap(out, no, bias, Cout * 4))
        return fail(CT_EINVAL, "%s: out overlaps an input", fn);
    if (x_dtype != w_dtype)
        return fail(CT_EUNSUPPORTED, "%s: x and w dtypes must match", fn);

    // The pages' geometry (k3 s2 p1, 2-pool; output padding 0 or 1) runs on
    // the matrix-core kernels when their index limits hold: fp32 on the slab
    // or direct fp32 kernel, bf16 on the bf16 kernel where it applies (no
    // output padding, Cin <= 32, W % 8 == 0, 16-byte aligned x) and on the
    // direct kernel with the taps widened to fp32 otherwise.  The bf16 kernel
    // works in 64-channel groups, so the first layer's own shape (Cin <= 4,
    // Cout <= 16) is faster on the direct kernel too (53 against 74 us at
    // [128,3,16,32,32] -> 16 channels).  Everything else runs on the general
    // kernels.
    bool page = k == 3 && stride == 2 && pad == 1 && pool_k == 2 && ps == 2 && out_pad <= 1;
    bool bf16_fast = false;
    if (page) {
        const int64_t wblocks = (pd[2] + 15) / 16;
        int64_t nmb, xitem, oitem;
        page = prod({N, pd[0], pd[1], wblocks}, &nmb) && nmb <= kI32Max / 8 &&
               prod({Cin, D, H, W}, &xitem) && xitem <= kI32Max &&
               prod({Cout, pd[0], pd[1], pd[2]}, &oitem) && oitem <= kI32Max &&
               Cout <= 65535 * 16 && Cin <= 128;
        if (page && x_dtype == CT_BF16 && out_pad == 0) {
            const size_t lb = ct::fused3d_bf16_lds_bytes(Cin, W);
            // (its buffer stores take 32-bit byte offsets within one batch item,
            // and masked lanes store at 2^31 - 16, which must lie past the item)
            bf16_fast = Cin <= 32 && W % 8 == 0 && aligned(x, 16) && lb != 0 && lb <= kLdsMax &&
                        oitem * 4 < (int64_t(1) << 31) - 64 && !(Cin <= 4 && Cout <= 16);
        }
    }
    hipError_t e;
    if (page && x_dtype == CT_F32) {
        e = ct::launch_fused3d_f32((const float *)x, (const float *)w, conv_bias, bias, scale1,
                                   scale2, N, Cin, D, H, W, Cout, out_pad, out, (hipStream_t)stream);
    } else if (bf16_fast) {
        e = ct::launch_fused3d_bf16((const uint16_t *)x, (const uint16_t *)w, conv_bias, bias,
                                    scale1, scale2, N, Cin, D, H, W, Cout, out,
                                    (hipStream_t)stream);
    } else if (page) {
        e = ct::launch_fused3d_direct_bf16((const uint16_t *)x, (const uint16_t *)w, conv_bias, bias,
                                           scale1, scale2, N, Cin, D, H, W, Cout, out_pad, out,
                                           (hipStream_t)stream);
    } else {
        if (pool_k > kGenericMaxTap)
            return fail(CT_EUNSUPPORTED, "%s: pool_k > %d is not implemented", fn, kGenericMaxTap);
        e = ct::launch_fused3d_generic(x, w, x_dtype == CT_BF16, conv_bias, bias, scale1, scale2,
                                       N, Cin, D, H, W, Cout, k, stride, pad, out_pad, pool_k, ps,
                                       out, (hipStream_t)stream);
    }
    return hip_status(e, "convT3d_scale_pool_bias launch");
}

ct_status ct_convT3d(const void *x, int x_dtype, const void *w, int w_dtype, const float *bias,
                     int64_t N, int64_t Cin, int64_t D, int64_t H, int64_t W, int64_t Cout,
                     int k, int stride, int pad, int out_pad, float *out, void *stream)
{
    const char *fn = "convT3d";
    int xs, ws;
    int64_t od[3];
    ct_status st = check_convT3d(fn, x, x_dtype, w, w_dtype, N, Cin, D, H, W, Cout, k, stride,
                                 pad, out_pad, out, &xs, &ws, od);
    if (st != CT_OK) return st;
    if (bias && !aligned(bias, 4)) return fail(CT_EINVAL, "%s: misaligned pointer", fn);
    int64_t nx, nw, no;
    if (!prod({N, Cin, D, H, W, (int64_t)xs}, &nx) ||
        !prod({Cin, Cout, (int64_t)k, (int64_t)k, (int64_t)k, (int64_t)ws}, &nw) ||
        !prod({N, Cout, od[0], od[1], od[2], 4}, &no))
        return fail(CT_EINVAL, "%s: tensor size overflows", fn);
    if (overlap(out, no, x, nx) || overlap(out, no, w, nw) || overlap(out, no, bias, Cout * 4))
        return fail(CT_EINVAL, "%s: out overlaps an input", fn);
    if (x_dtype != w_dtype) return fail(CT_EUNSUPPORTED, "%s: x and w dtypes must match", fn);
    // The pages' k3 s2 p1 layer with few input channels runs on the parity
    // kernel (one work-item per input voxel, a grid below the 2^32 work-items
    // of one dispatch); the rest on the general one.
    int64_t nvox;
    const bool parity = k == 3 && stride == 2 && pad == 1 && Cin <= 8 &&
                        prod({N, D, H, W}, &nvox) && nvox <= (int64_t)UINT32_MAX - 1024;
    hipError_t e;
    if (parity)
        e = ct::launch_convT3d_s2(x, w, x_dtype == CT_BF16, bias, N, Cin, D, H, W, Cout, out_pad,
                                  out, (hipStream_t)stream);
    else
        e = ct::launch_convT3d_generic(x, w, x_dtype == CT_BF16, bias, N, Cin, D, H, W, Cout, k,
                                       stride, pad, out_pad, out, (hipStream_t)stream);
    return hip_status(e, "convT3d launch");
}

namespace {
// ct_avgpool3d and ct_avgpool3d_bf16: x and out are fp32 (bf16 = false) or
// bf16 bit patterns (bf16 = true); es is the element size in bytes.
ct_status avgpool3d_impl(const char *fn, const void *x, bool bf16, int64_t N, int64_t C,
                         int64_t D, int64_t H, int64_t W, int k, int stride, int pad,
                         int count_include_pad, void *out, void *stream)
{
    const int es = bf16 ? 2 : 4;
    if (!x || !out) return fail(CT_EINVAL, "%s: x and out must be non-null", fn);
    if (N < 1 || C < 1 || D < 1 || H < 1 || W < 1)
        return fail(CT_EINVAL, "%s: sizes must be >= 1", fn);
    if (k < 1 || stride < 0 || pad < 0 || 2 * (int64_t)pad > k ||
        (count_include_pad != 0 && count_include_pad != 1))
        return fail(CT_EINVAL, "%s: invalid geometry k=%d stride=%d pad=%d count_include_pad=%d "
                    "(pad must be <= k/2)", fn, k, stride, pad, count_include_pad);
    const int s = stride == 0 ? k : stride;
    int64_t o[3];
    const int64_t in[3] = {D, H, W};
    for (int i = 0; i < 3; ++i) {
        o[i] = ct_pool_out_len(in[i], k, s, pad);
        if (o[i] <= 0)
            return fail(CT_EINVAL, "%s: empty output along axis %d", fn, i);
    }
    if (!aligned(x, es) || !aligned(out, es)) return fail(CT_EINVAL, "%s: misaligned pointer", fn);
    int64_t nx, no, slice;
    if (!prod({N, C, D, H, W, es}, &nx) || !prod({N, C, o[0], o[1], o[2], es}, &no) ||
        !prod({D, H, W}, &slice))
        return fail(CT_EINVAL, "%s: tensor size overflows", fn);
    if (overlap(out, no, x, nx)) return fail(CT_EINVAL, "%s: out overlaps x", fn);

    // k3 s2 p1 takes the streaming kernels with either divisor, as long as one
    // slice is below 2^31 elements and the grid fits one dispatch
    const bool fast = k == 3 && s == 2 && pad == 1 && slice <= kI32Max &&
                      ct::avgpool3d_k3s2p1_fits(bf16, x, out, N * C, D, H, W);
    hipError_t e;
    if (fast) {
        e = ct::launch_avgpool3d_k3s2p1(x, bf16, count_include_pad == 1, N * C, D, H, W, out,
                                        (hipStream_t)stream);
    } else {
        if (D > kGenericMaxLen || H > kGenericMaxLen || W > kGenericMaxLen || k > kGenericMaxTap ||
            s > kGenericMaxLen)
            return fail(CT_EUNSUPPORTED, "%s: sizes beyond the general kernel's index range "
                        "(lengths and stride <= %lld, k <= %d)", fn, (long long)kGenericMaxLen,
                        kGenericMaxTap);
        e = ct::launch_avgpool3d_generic(x, bf16, N * C, D, H, W, k, s, pad, count_include_pad,
                                         out, (hipStream_t)stream);
    }
    return hip_status(e, fn);
}
}  // namespace

ct_status ct_avgpool3d(const float *x, int64_t N, int64_t C, int64_t D, int64_t H, int64_t W,
                       int k, int stride, int pad, int count_include_pad, float *out,
                       void *stream)
{
    return avgpool3d_impl("avgpool3d", x, false, N, C, D, H, W, k, stride, pad,
                          count_include_pad, out, stream);
}

ct_status ct_avgpool3d_bf16(const uint16_t *x, int64_t N, int64_t C, int64_t D, int64_t H,
                            int64_t W, int k, int stride, int pad, int count_include_pad,
                            uint16_t *out, void *stream)
{
    return avgpool3d_impl("avgpool3d_bf16", x, true, N, C, D, H, W, k, stride, pad,
                          count_include_pad, out, stream);
}

ct_status ct_convT1d(const void *x, int x_dtype, const void *w, int w_dtype, const float *bias,
                     int64_t N, int64_t Cin, int64_t L, int64_t Cout, int K, int stride, int pad,
                     int dilation, int out_pad, float *out, void *stream)
{
    if (!x || !w || !out) return fail(CT_EINVAL, "convT1d: x, w and out must be non-null");
    const int xs = dtype_size(x_dtype), ws = dtype_size(w_dtype);
    if (!xs || !ws) return fail(CT_EINVAL, "convT1d: unknown dtype (%d, %d)", x_dtype, w_dtype);
    if (N < 1 || Cin < 1 || L < 1 || Cout < 1) return fail(CT_EINVAL, "convT1d: sizes must be >= 1");
    if (K < 1 || stride < 1 || pad < 0 || dilation < 1 || out_pad < 0 ||
        out_pad >= (stride > dilation ? stride : dilation))
        return fail(CT_EINVAL, "convT1d: invalid geometry K=%d stride=%d pad=%d dilation=%d out_pad=%d "
                    "(out_pad must be < max(stride, dilation))", K, stride, pad, dilation, out_pad);
    const int64_t Lo = ct_convT_out_len(L, K, stride, pad, out_pad, dilation);
    if (Lo <= 0) return fail(CT_EINVAL, "convT1d: empty output (L_out=%lld)", (long long)Lo);
    if (!aligned(x, xs) || !aligned(w, ws) || !aligned(out, 4) || (bias && !aligned(bias, 4)))
        return fail(CT_EINVAL, "convT1d: misaligned pointer");
    int64_t nx, nw, no, nb;
    if (!prod({N, Cin, L, (int64_t)xs}, &nx) || !prod({Cin, Cout, (int64_t)K, (int64_t)ws}, &nw) ||
        !prod({N, Cout, Lo, 4}, &no) || !prod({Cout, 4}, &nb))
        return fail(CT_EINVAL, "convT1d: tensor size overflows");
    if (overlap(out, no, x, nx) || overlap(out, no, w, nw) || overlap(out, no, bias, nb))
        return fail(CT_EINVAL, "convT1d: out overlaps an input");
    if (x_dtype != w_dtype) return fail(CT_EUNSUPPORTED, "convT1d: x and w dtypes must match");

    // Stride 1 in fp32 runs on the fp32 matrix-core kernels when their tiles
    // fit: without padding for any channels, taps and dilation, and with a pad
    // or output padding at the page's channels and taps (a shifted output
    // window); everything else not caught below on the general kernel.
    bool fast = x_dtype == CT_F32 && stride == 1 &&
                ((pad == 0 && out_pad == 0) ||
                 ct::convT1d_f32_wave_supported(Cin, K, dilation, L, x));
    if (fast) {
        const int64_t tiles = (Lo + 255) / 256;
        int64_t ntiles;
        fast = Lo <= kI32Max - 256 && L <= kI32Max - 1024 && prod({N, tiles}, &ntiles) &&
               ntiles <= kI32Max &&
               (Cout + 63) / 64 <= 65535 && Cin <= 4096 && K <= 4096 &&
               (int64_t)dilation * (K - 1) <= 65536 &&
               ct::convT1d_f32_lds_bytes(Cin, K, dilation) <= kLdsMax;
        int64_t item;           // one batch item's output within a 2 GiB buffer range
        fast = fast && prod({Cout, Lo, 4}, &item) && item < (int64_t(1) << 31) - 64;
    }
    // bf16 at the page's geometry, stride 1, runs on the bf16 matrix-core kernel.
    bool fast_bf16 = x_dtype == CT_BF16 && stride == 1 &&
                     ct::convT1d_bf16_supported(Cin, K, dilation, L, x);
    if (fast_bf16) {
        const int64_t tiles = (Lo + 31 + 255) / 256;
        int64_t ntiles;
        int64_t item;           // one batch item's output within a 2 GiB buffer range
        fast_bf16 = Lo <= kI32Max - 512 && L <= kI32Max - 1024 && prod({N, tiles}, &ntiles) &&
                    ntiles <= kI32Max &&
                    (Cout + 63) / 64 <= 65535 && prod({Cout, Lo, 4}, &item) &&
                    item < (int64_t(1) << 31) - 64;
    }
    // Stride 2 to 8 in fp32 at the page's channel and tap geometry runs as
    // stride-1 gathers over the residue classes of o + pad on the fp32
    // matrix cores.
    bool poly = x_dtype == CT_F32 && stride >= 2 && stride <= 8 &&
                ct::convT1d_f32_poly_supported(Cin, K, stride, dilation, L, x);
    if (poly) {
        const int64_t tq = ((Lo + pad + stride - 1) / stride + 16) / 16 + 1;   // 16-q tiles bound every stride's
        int64_t ntq, item;
        poly = Lo <= kI32Max / 2 && pad <= kGenericMaxLen && prod({N, tq}, &ntq) &&
               ntq <= kI32Max && (Cout + 63) / 64 <= 65535 && prod({Cout, Lo, 4}, &item) &&
               item < (int64_t(1) << 31) - 64;
    }
    hipError_t e;
    if (poly) {
        e = ct::launch_convT1d_f32_poly((const float *)x, (const float *)w, bias, N, Cin, L, Cout,
                                        K, stride, pad, dilation, out_pad, out,
                                        (hipStream_t)stream);
    } else if (fast) {
        e = ct::launch_convT1d_f32((const float *)x, (const float *)w, bias, N, Cin, L, Cout, K,
                                   dilation, pad, out_pad, out, (hipStream_t)stream);
    } else if (fast_bf16) {
        e = ct::launch_convT1d_bf16((const uint16_t *)x, (const uint16_t *)w, bias, N, L, Cout, K,
                                    dilation, pad, out_pad, out, (hipStream_t)stream);
    } else {
        if (Lo > kGenericMaxLen || L > kGenericMaxLen || Cin > kGenericMaxLen ||
            Cout > kGenericMaxLen || pad > kGenericMaxLen ||
            (int64_t)dilation * (K - 1) > kGenericMaxLen)
            return fail(CT_EUNSUPPORTED, "convT1d: sizes beyond the general kernel's index range "
                        "(lengths, pad and dilation*(K-1) <= %lld)", (long long)kGenericMaxLen);
        e = ct::launch_convT1d_generic(x, w, x_dtype == CT_BF16, bias, N, Cin, L, Cout, K, stride,
                                       pad, dilation, out_pad, out, (hipStream_t)stream);
    }
    return hip_status(e, "convT1d launch");
}

}  // extern "C"
