// One-wave GPU probes of the instruction lane images the library's kernels
// are built on (test infrastructure, not part of the library).  Each probe
// runs a single instruction through the library's own wrappers
// (device_common.hpp) on per-lane operands given by the host and returns
// what every lane received, so that the tests can check the images stated
// in device_common.hpp and layout.hpp against the hardware:
//   - the 16x16x32 16-bit MFMA: operand lanes, output registers;
//   - the block-scaled 16x16x128 MFMA for every pair of the formats the
//     kernels use (E4M3 0, E2M3 2, E3M2 3, E2M1 4): operand bytes / values,
//     scale lanes, the internal K index by which mixed formats meet;
//   - the transposing LDS read ds_read_b64_tr_b16.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"

using namespace mswz;

namespace {

__global__ void __launch_bounds__(64) k_mfma16(int bf16, const u32x4 *a, const u32x4 *b, f32x4 *out)
{
    const int l = threadIdx.x;
    out[l] = bf16 ? mfma_16x16x32<true>(a[l], b[l], f32x4{}) : mfma_16x16x32<false>(a[l], b[l], f32x4{});
}

template <int F1, int F2>
__global__ void __launch_bounds__(64) k_mfma_scale16(const i32x8 *a, const i32x8 *b, const int *sa,
                                                     const int *sb, f32x4 *out)
{
    const int l = threadIdx.x;
    out[l] = mfma_scale_16x16x128_fmt<F1, F2>(a[l], b[l], f32x4{}, sa[l], sb[l]);
}

constexpr int kTrLdsBytes = 32768;

__global__ void __launch_bounds__(64) k_read_tr16(const uint16_t *init, int n, const uint32_t *addrs, u32x2 *out)
{
    __shared__ __attribute__((aligned(16))) uint16_t lds[kTrLdsBytes / 2];
    for (int i = threadIdx.x; i < kTrLdsBytes / 2; i += 64)
        lds[i] = i < n ? init[i] : 0;
    __syncthreads();
    out[threadIdx.x] = lds_read_tr16(reinterpret_cast<const uint8_t *>(lds), addrs[threadIdx.x]);
}

// Copies `in` (in_bytes) to a fresh device buffer per input, runs `launch`
// with the device pointers, copies `out_bytes` back.
struct Dev {
    void *p = nullptr;
    ~Dev() { if (p) (void)hipFree(p); }
};

int up(Dev &d, const void *src, size_t bytes)
{
    if (hipMalloc(&d.p, bytes) != hipSuccess)
        return -1;
    return hipMemcpy(d.p, src, bytes, hipMemcpyHostToDevice) == hipSuccess ? 0 : -1;
}

int down(void *dst, const Dev &d, size_t bytes)
{
    if (hipDeviceSynchronize() != hipSuccess || hipGetLastError() != hipSuccess)
        return -1;
    return hipMemcpy(dst, d.p, bytes, hipMemcpyDeviceToHost) == hipSuccess ? 0 : -1;
}

template <int F1, int F2>
void launch_scale(const i32x8 *a, const i32x8 *b, const int *sa, const int *sb, f32x4 *out)
{
    k_mfma_scale16<F1, F2><<<1, 64>>>(a, b, sa, sb, out);
}

template <int F1>
int launch_scale_f2(int f2, const i32x8 *a, const i32x8 *b, const int *sa, const int *sb, f32x4 *out)
{
    switch (f2) {
    case 0: launch_scale<F1, 0>(a, b, sa, sb, out); return 0;
    case 2: launch_scale<F1, 2>(a, b, sa, sb, out); return 0;
    case 3: launch_scale<F1, 3>(a, b, sa, sb, out); return 0;
    case 4: launch_scale<F1, 4>(a, b, sa, sb, out); return 0;
    default: return -2;
    }
}

}  // namespace

extern "C" {

// a, b: 64 lanes x 4 registers; out: 64 lanes x 4 fp32.  0 or a negative error.
int probe_mfma16(int bf16, const uint32_t *a, const uint32_t *b, float *out)
{
    Dev da, db, dout;
    if (up(da, a, 64 * 16) || up(db, b, 64 * 16) || hipMalloc(&dout.p, 64 * 16) != hipSuccess)
        return -1;
    k_mfma16<<<1, 64>>>(bf16, static_cast<const u32x4 *>(da.p), static_cast<const u32x4 *>(db.p),
                        static_cast<f32x4 *>(dout.p));
    return down(out, dout, 64 * 16);
}

// f1, f2: format codes of the first and second operand (0, 2, 3 or 4);
// a, b: 64 lanes x 8 registers; sa, sb: one scale register per lane (byte 0
// used); out: 64 lanes x 4 fp32.
int probe_mfma_scale16(int f1, int f2, const uint32_t *a, const uint32_t *b, const int32_t *sa,
                       const int32_t *sb, float *out)
{
    Dev da, db, dsa, dsb, dout;
    if (up(da, a, 64 * 32) || up(db, b, 64 * 32) || up(dsa, sa, 64 * 4) || up(dsb, sb, 64 * 4) ||
        hipMalloc(&dout.p, 64 * 16) != hipSuccess)
        return -1;
    auto *pa = static_cast<const i32x8 *>(da.p);
    auto *pb = static_cast<const i32x8 *>(db.p);
    auto *psa = static_cast<const int *>(dsa.p);
    auto *psb = static_cast<const int *>(dsb.p);
    auto *po = static_cast<f32x4 *>(dout.p);
    int rc;
    switch (f1) {
    case 0: rc = launch_scale_f2<0>(f2, pa, pb, psa, psb, po); break;
    case 2: rc = launch_scale_f2<2>(f2, pa, pb, psa, psb, po); break;
    case 3: rc = launch_scale_f2<3>(f2, pa, pb, psa, psb, po); break;
    case 4: rc = launch_scale_f2<4>(f2, pa, pb, psa, psb, po); break;
    default: rc = -2;
    }
    if (rc)
        return rc;
    return down(out, dout, 64 * 16);
}

// init: n 16-bit values (n <= 16384) loaded into LDS from byte 0 (the rest
// zero); addrs: each lane's byte offset, 8-byte aligned, below 32768 - 7;
// out: 64 lanes x 2 registers (four 16-bit values).
int probe_read_tr16(const uint16_t *init, int n, const uint32_t *addrs, uint32_t *out)
{
    if (n < 0 || n > kTrLdsBytes / 2)
        return -2;
    for (int l = 0; l < 64; ++l)
        if ((addrs[l] & 7u) || addrs[l] > uint32_t(kTrLdsBytes - 8))
            return -2;
    Dev di, dad, dout;
    if (up(di, init, size_t(n > 0 ? n : 1) * 2) || up(dad, addrs, 64 * 4) || hipMalloc(&dout.p, 64 * 8) != hipSuccess)
        return -1;
    k_read_tr16<<<1, 64>>>(static_cast<const uint16_t *>(di.p), n, static_cast<const uint32_t *>(dad.p),
                           static_cast<u32x2 *>(dout.p));
    return down(out, dout, 64 * 8);
}

}  // extern "C"
