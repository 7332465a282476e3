// Pieces shared by the FP8 GEMM schedules (the large-M kernels in jetfp8_gemm.hip, the small-M kernel in
// jetfp8_decode.hip): the group product instruction, buffer descriptors, the group width and the device's
// compute-unit count.
#pragma once
#include <hip/hip_runtime.h>
#include <atomic>

namespace jetfp8 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// 16x16x128 FP8 (E4M3 x E4M3) matrix product with C = 0: D[i][j] = sum_k a[i][k] * b[j][k].  Lane l supplies
// row (l % 16) of a and of b, bytes k = 32 * (l / 16) .. +31; result element v of lane l is
// D[4 * (l / 16) + v][l % 16].
// The builtin is the scaled form (V_MFMA_SCALE_F32_16X16X128_F8F6F4); its trailing operands are the formats of
// a and b (0 = E4M3 for both) and the E8M0 block-scale operands with their byte selectors.  With the scale
// operands constant zero the compiler selects the plain, unscaled V_MFMA_F32_16X16X128_F8F6F4 (the only matrix
// opcode in the library's gfx950 assembly), so the result is the unscaled E4M3 x E4M3 product.
__device__ __forceinline__ v4f mfma_group(const v8i& a, const v8i& b) {
    const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 0, 0, 0);
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer descriptor over [base, base + bytes) (stride 0, range-checked: loads past the end return
// zero).  base and bytes must be block-uniform values (scalar registers); then so is the descriptor.
// bytes < 2^31 is guaranteed by the host-side shape limits (kMaxGemmBand).
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

constexpr int BK = 128;            // one quantization group along the contraction axis
// s_waitcnt immediate: lgkmcnt == 0 only (vmcnt and expcnt at their maxima)
constexpr int kWaitLgkm0 = 0xF | (7 << 4) | (3 << 14);

// Compute units of the current device (one persistent block per compute unit: a block's LDS ring
// takes most of a CU's LDS).  The per-device cache is atomic: concurrent first calls may both query the
// runtime, and they store the same value.
inline int device_cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

}  // namespace jetfp8
