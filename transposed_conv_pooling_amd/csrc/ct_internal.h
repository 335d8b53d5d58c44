// ct_internal.h - launchers shared between the C-ABI shim (ct_api.hip) and
// the kernel files.  Every launcher assumes its arguments were validated by
// the shim: sizes positive, pointers non-null and aligned, geometry one the
// kernel implements, and all per-launch index ranges within int32 where the
// kernel says so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ct {

// Per-device facts, queried once per device and cached (device.hip):
// compute units of the current device; workgroups of `fn` that fit on one CU
// with `threads` threads and `lds` bytes of dynamic LDS (at least 1); and
// hipFuncSetAttribute(MaxDynamicSharedMemorySize) issued only when `lds`
// exceeds what this device already granted `fn`.
int current_device();
int device_cus();
int occupancy(const void *fn, int threads, size_t lds);
hipError_t allow_dynamic_lds(const void *fn, size_t lds);

// Fused ConvTranspose3d(k3, s2, p1, output_padding op) -> *s1 ->
// AvgPool3d(2) -> +bias -> *s2, fp32 x and w.  Output [N, Cout, D-1+op,
// H-1+op, W-1+op], op 0 or 1, Cin up to 128 (the slab kernel for Cin <= 4
// when an LDS slab fits and the call is not small, else the direct kernel).
hipError_t launch_fused3d_f32(const float *x, const float *w,
                              const float *conv_bias, const float *bias,
                              float s1, float s2, int64_t N, int64_t Cin,
                              int64_t D, int64_t H, int64_t W, int64_t Cout, int op,
                              float *out, hipStream_t stream);

// The direct fp32 kernel of the same chain for bf16 x and w, the taps
// widened exactly to fp32 (any Cin up to 128, output padding 0 or 1, no
// alignment beyond 2 bytes); the bf16 kernel below is the fast path.
hipError_t launch_fused3d_direct_bf16(const uint16_t *x, const uint16_t *w,
                                      const float *conv_bias, const float *bias, float s1,
                                      float s2, int64_t N, int64_t Cin, int64_t D, int64_t H,
                                      int64_t W, int64_t Cout, int op, float *out,
                                      hipStream_t stream);

// Same chain with bf16 x and w (fp32 accumulation and output).
hipError_t launch_fused3d_bf16(const uint16_t *x, const uint16_t *w,
                               const float *conv_bias, const float *bias,
                               float s1, float s2, int64_t N, int64_t Cin,
                               int64_t D, int64_t H, int64_t W, int64_t Cout,
                               float *out, hipStream_t stream);

// AvgPool3d(k3, s2, p1) over NC independent [D][H][W] slices, divisor 27
// (include_pad) or the number of window taps inside the slice; x and out
// fp32, or (bf16 = true) bf16 bit patterns with fp32 sums.
hipError_t launch_avgpool3d_k3s2p1(const void *x, bool bf16, bool include_pad, int64_t NC,
                                   int64_t D, int64_t H, int64_t W, void *out,
                                   hipStream_t stream);
// Whether that launch's grid (workgroups x work-items per workgroup) stays
// within the 32-bit work-item count of one dispatch; the streaming kernels
// have no grid-stride loop, so a larger call takes the general kernel.
bool avgpool3d_k3s2p1_fits(bool bf16, const void *x, const void *out, int64_t NC, int64_t D,
                           int64_t H, int64_t W);

// ConvTranspose1d, stride 1, fp32: pad 0 and no output padding for any K and
// dilation the LDS holds; with a pad or output padding only where
// convT1d_f32_wave_supported() holds (Cin 32, K 5, dilation 3, L a multiple
// of 4, x 16-byte aligned; any output length and 4-byte aligned out).
bool convT1d_f32_wave_supported(int64_t Cin, int K, int dilation, int64_t L, const void *x);
hipError_t launch_convT1d_f32(const float *x, const float *w,
                              const float *bias, int64_t N, int64_t Cin,
                              int64_t L, int64_t Cout, int K, int dilation, int pad,
                              int out_pad, float *out, hipStream_t stream);

// ConvTranspose1d with stride 2 (any pad and output padding) as two stride-1
// gathers on the fp32 matrix cores, where convT1d_f32_poly_supported() holds
// (fp32, Cin 32, K 5, dilation 3, L % 4 == 0, x 16-byte aligned); output
// items below 2^31 - 64 bytes.
bool convT1d_f32_poly_supported(int64_t Cin, int K, int stride, int dilation, int64_t L,
                                const void *x);
hipError_t launch_convT1d_f32_poly(const float *x, const float *w, const float *bias, int64_t N,
                                   int64_t Cin, int64_t L, int64_t Cout, int K, int stride,
                                   int pad, int dilation, int out_pad, float *out,
                                   hipStream_t stream);

// ConvTranspose1d, stride 1 with any pad and output padding, bf16 x and w
// (fp32 accumulation and output) on the bf16 matrix cores, for the
// geometries where convT1d_bf16_supported() holds (Cin 32, K 5, dilation 3,
// L a multiple of 8, x 16-byte aligned); L below 2^31 - 1024.
bool convT1d_bf16_supported(int64_t Cin, int K, int dilation, int64_t L, const void *x);
hipError_t launch_convT1d_bf16(const uint16_t *x, const uint16_t *w, const float *bias,
                               int64_t N, int64_t L, int64_t Cout, int K, int dilation, int pad,
                               int out_pad, float *out, hipStream_t stream);

// ConvTranspose3d(k3, s2, p1), output_padding 0 or 1, 1 <= Cin <= 8, output
// [N, Cout, 2D-1+op, 2H-1+op, 2W-1+op] materialised; x, w fp32 or bf16.
// Requires N*D*H*W < 2^31 * 256 and each output length below 2^31.
hipError_t launch_convT3d_s2(const void *x, const void *w, bool bf16, const float *bias,
                             int64_t N, int64_t Cin, int64_t D, int64_t H, int64_t W,
                             int64_t Cout, int op, float *y, hipStream_t stream);

// General-geometry kernels (generic.hip): one thread per output element,
// fp32 or bf16 (bf16 = true) x and w, fp32 accumulation and output.
hipError_t launch_fused3d_generic(const void *x, const void *w, bool bf16,
                                  const float *conv_bias, const float *bias, float s1, float s2,
                                  int64_t N, int64_t Cin, int64_t D, int64_t H, int64_t W,
                                  int64_t Cout, int k, int s, int p, int op, int pk, int ps,
                                  float *out, hipStream_t stream);
hipError_t launch_convT3d_generic(const void *x, const void *w, bool bf16, const float *bias,
                                  int64_t N, int64_t Cin, int64_t D, int64_t H, int64_t W,
                                  int64_t Cout, int k, int s, int p, int op, float *y,
                                  hipStream_t stream);
hipError_t launch_avgpool3d_generic(const void *x, bool bf16, int64_t NC, int64_t D, int64_t H,
                                    int64_t W, int k, int s, int p, int include_pad, void *out,
                                    hipStream_t stream);
hipError_t launch_convT1d_generic(const void *x, const void *w, bool bf16, const float *bias,
                                  int64_t N, int64_t Cin, int64_t L, int64_t Cout, int K, int s,
                                  int p, int dil, int op, float *y, hipStream_t stream);

// Workgroup index remapped so that each XCD (blocks are dealt to the 8 XCDs
// round-robin) works on one contiguous range of logical tiles: neighbouring
// tiles then share that XCD's L2.
__device__ __forceinline__ int64_t xcd_remap(int64_t bid, int64_t nblocks)
{
    constexpr int64_t kXcd = 8;
    const int64_t per = nblocks / kXcd;          // full rounds
    const int64_t rem = nblocks - per * kXcd;    // XCDs that get one extra
    const int64_t xcd = bid % kXcd;
    const int64_t idx = bid / kXcd;
    // XCD x owns logical tiles [start(x), start(x) + per + (x < rem))
    const int64_t start = xcd * per + (xcd < rem ? xcd : rem);
    return start + idx;
}

}  // namespace ct
