// Q8_0 quantization of f32 rows on the GPU, a small fill kernel, and the
// cached compute-unit count that launch shapes use.
//
// Format: "Quantized built-ins and formats", section "Q8_0" -- signed bytes,
// one f32 scale per 32 consecutive values; activations use the same form
// (a_scales: one f32 per 32 elements, "Phobos Language Spec", section
// "Quantized built-ins").  The pages do not say how values are quantized;
// the rule here is the plainest one: d = f32(max|x| / 127) per block,
// q = clamp(round-half-even(x / d), -127, 127) with an IEEE f32 division
// (ties to even as the spec's round(), section "Elementwise"), and d == 0
// gives q == 0.
//
// Layout of the work: 8 lanes per 32-value block, 4 values (16 bytes) per
// lane, so one wave reads 1 KiB of contiguous f32 and writes 256 contiguous
// bytes of Q.  HBM-bound: 4 bytes in, 1 + 1/8 bytes out per value.
#include <atomic>

#include "q8_device.h"
#include "q8_launch.h"

namespace q8 {
namespace {

constexpr int kQuantThreads = 256;

__device__ __forceinline__ int quantize_one(float x, float d) {
    float v = rintf(x / d);  // IEEE f32 division, then ties-to-even
    v = fminf(fmaxf(v, -127.0f), 127.0f);
    return (int)v & 0xFF;
}

__global__ void __launch_bounds__(kQuantThreads)
quantize_kernel(const float4* __restrict__ X, uint32_t* __restrict__ Q, float* __restrict__ D,
                int64_t nblocks) {
    const int64_t nthreads = nblocks * 8;
    const int64_t stride = (int64_t)gridDim.x * kQuantThreads;
    // Uniform trip count across the wave: every lane reaches each shuffle.
    for (int64_t base = (int64_t)blockIdx.x * kQuantThreads; base < nthreads; base += stride) {
        const int64_t t = base + threadIdx.x;
        const bool ok = t < nthreads;
        const float4 x = ok ? X[t] : make_float4(0.f, 0.f, 0.f, 0.f);
        float m = fmaxf(fmaxf(fabsf(x.x), fabsf(x.y)), fmaxf(fabsf(x.z), fabsf(x.w)));
        // Max over the 8 lanes of the block (lanes 8g .. 8g+7 of the wave).
        m = fmaxf(m, __shfl_xor(m, 1, 8));
        m = fmaxf(m, __shfl_xor(m, 2, 8));
        m = fmaxf(m, __shfl_xor(m, 4, 8));
        const float d = m / 127.0f;
        uint32_t packed = 0;
        if (d != 0.0f) {
            packed = (uint32_t)quantize_one(x.x, d) | ((uint32_t)quantize_one(x.y, d) << 8) |
                     ((uint32_t)quantize_one(x.z, d) << 16) | ((uint32_t)quantize_one(x.w, d) << 24);
        }
        if (ok) {
            Q[t] = packed;
            if ((t & 7) == 0) D[t >> 3] = d;
        }
    }
}

__global__ void __launch_bounds__(256)
fill_zero_kernel(float* __restrict__ C, int64_t count) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < count; t += stride)
        C[t] = 0.0f;
}

}  // namespace

hipError_t launch_quantize(const float* X, int8_t* Q, float* D, int rows, int K,
                           hipStream_t stream) {
    const int64_t nblocks = (int64_t)rows * (K / kBlock);
    if (nblocks == 0) return hipSuccess;
    const int64_t need = (nblocks * 8 + kQuantThreads - 1) / kQuantThreads;
    const int64_t cap = 256 * 32;
    const unsigned grid = (unsigned)(need < cap ? need : cap);
    quantize_kernel<<<grid, kQuantThreads, 0, stream>>>(reinterpret_cast<const float4*>(X),
                                                        reinterpret_cast<uint32_t*>(Q), D, nblocks);
    return hipGetLastError();
}

hipError_t launch_fill_zero(float* C, int64_t count, hipStream_t stream) {
    if (count == 0) return hipSuccess;
    const int64_t need = (count + 255) / 256;
    const int64_t cap = 256 * 16;
    fill_zero_kernel<<<(unsigned)(need < cap ? need : cap), 256, 0, stream>>>(C, count);
    return hipGetLastError();
}

int device_cu_count() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cached[kMaxDevices];  // zero until queried
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
    return n;
}

}  // namespace q8
