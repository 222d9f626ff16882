// Host-side launch helpers behind the C-ABI (internal; not exported).
// Arguments are validated by the caller (q8qdot_api.cpp): non-negative
// shapes, K % 32 == 0, aligned non-null pointers.  Each helper only enqueues
// kernels on `stream` and returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace q8 {

// Raise `kernel`'s dynamic-LDS limit to `bytes` on the current device, once
// per device: the attribute is set per device, so `done` (one per kernel,
// owned by the caller) keeps a bit per device ordinal below 64 (others are
// set on every call).  Concurrent first calls only repeat the setting.
inline hipError_t set_dynamic_lds(const void* kernel, int bytes, std::atomic<uint64_t>& done) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = -1;
    const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t)1 << dev : 0;
    if (bit != 0 && (done.load(std::memory_order_relaxed) & bit) != 0) return hipSuccess;
    const hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess && bit != 0) done.fetch_or(bit, std::memory_order_relaxed);
    return e;
}

// Workgroups of `kernel` (`threads` each, `smem` bytes of dynamic LDS) that
// one compute unit holds at once, as the runtime computes it from the
// kernel's registers and LDS, at least 1.  `cache` (one per kernel and key,
// owned by the caller, zero-initialised) holds the answer per device
// ordinal below 64; concurrent first calls only repeat the query.
inline int wgs_per_cu(const void* kernel, int threads, size_t smem, std::atomic<int> (&cache)[64]) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = -1;
    if (dev >= 0) {
        const int v = cache[dev].load(std::memory_order_relaxed);
        if (v > 0) return v;
    }
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, smem) != hipSuccess || n < 1) n = 1;
    if (dev >= 0) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

// M < 8: wave64 matvec.  K <= 16 KiB: one kernel for one activation row or
// (2 <= M <= 7) for all rows at once, every weight row read once; longer
// rows: one activation row per grid row, taken in 16 KiB chunks.
// P == nullptr -> f32 output C; otherwise int32 partials P, C unused.
// ws_t: WS is stored transposed, [K/32][N] (the qmma_t form); else [N][K/32].
hipError_t launch_matvec(const int8_t* A, const float* AS, const int8_t* W, const float* WS,
                         float* C, int32_t* P, int M, int N, int K, bool ws_t, hipStream_t stream);

// M >= 8: int8-MFMA block GEMM.  Same P convention.
// qgemm_variant: 1 = one workgroup per 32 x 32 tile with the contraction
// split across its waves (few tiles), 2 = LDS-staged 128 x 224 workgroup
// tiles (large M and N).
int qgemm_variant(int M, int N, int K);
hipError_t launch_qgemm(const int8_t* A, const float* AS, const int8_t* W, const float* WS,
                        float* C, int32_t* P, int M, int N, int K, bool ws_t, hipStream_t stream);
hipError_t launch_qgemm_ksplit(const int8_t* A, const float* AS, const int8_t* W, const float* WS,
                               float* C, int32_t* P, int M, int N, int K, bool ws_t,
                               hipStream_t stream);

// M >= 8 with too few 64 x 64 output tiles to fill the chip: the contraction
// split into S slices of slice_blocks blocks across workgroups, reduced in a
// caller workspace of ws_bytes (zero-filled; left zero-filled).  false when
// the shape does not take this form.
bool splitk_plan(int M, int N, int K, int* S, int* slice_blocks, size_t* ws_bytes);
hipError_t launch_qgemm_splitk(const int8_t* A, const float* AS, const int8_t* W, const float* WS,
                               float* C, int32_t* P, int M, int N, int K, bool ws_t, int S,
                               int slice_blocks, void* workspace, hipStream_t stream);
// The same kernel over all of K (S = 1, slice_blocks = splitk_whole_k_blocks,
// no workspace): taken instead of the K-split GEMM where its 64 x 64 tiles
// need fewer rounds of workgroups (splitk_whole_k).
bool splitk_whole_k(int M, int N, int K);
// The LDS-staged GEMM's output tile (qgemm.hip: kBM rows, kStagedTN tiles
// of kTile columns), for the choice between that kernel and this one.
constexpr int kStagedTileM = 128;
constexpr int kStagedTileN = 224;
// Shapes the staged GEMM would take on which the 64 x 64-tile kernel over
// all of K is faster.
bool splitk_over_staged(int M, int N, int K);
// Whether the kernel over all of K has more 64 x 64 tiles than compute
// units (its two-workgroups-per-unit form).
bool splitk_shared(int M, int N);
// The same kernel over all of K for Q5_0 weights (W5: 20 bytes per 32
// values), decoding each stage's blocks into LDS once (the two-workgroups-
// per-unit form only).
hipError_t launch_qgemm_splitk_q50(const int8_t* A, const float* AS, const uint8_t* W5,
                                   const float* WS, float* C, int32_t* P, int M, int N, int K,
                                   bool ws_t, hipStream_t stream);
int splitk_whole_k_blocks(int K);
// The same with the library's file-scope scratch array as the workspace (no
// allocation); splitk_scratch_capacity() is the largest workspace it stands
// for.  Calls that overlap on one GPU race on it.
size_t splitk_scratch_capacity();
hipError_t launch_qgemm_splitk_scratch(const int8_t* A, const float* AS, const int8_t* W,
                                       const float* WS, float* C, int M, int N, int K, bool ws_t,
                                       int S, int slice_blocks, hipStream_t stream);

// Q5_0 weights (W5: 20 bytes per 32 values): one-row matvec for M < 8 with
// K <= 16 Ki values; otherwise the K-split MFMA GEMM decoding into LDS.
bool matvec_q50_fits(int K);
hipError_t launch_matvec_q50(const int8_t* A, const float* AS, const uint8_t* W5, const float* WS,
                             float* C, int32_t* P, int M, int N, int K, bool ws_t,
                             hipStream_t stream);
hipError_t launch_qgemm_ksplit_q50(const int8_t* A, const float* AS, const uint8_t* W5,
                                   const float* WS, float* C, int32_t* P, int M, int N, int K,
                                   bool ws_t, hipStream_t stream);

// Q8_0 quantization of f32 rows.
hipError_t launch_quantize(const float* X, int8_t* Q, float* D, int rows, int K,
                           hipStream_t stream);

// C[0 .. count) = 0.0f with a plain fill kernel (no memset node, so the
// call stays safe inside a captured graph).
hipError_t launch_fill_zero(float* C, int64_t count, hipStream_t stream);

// Compute units of the current device (queried once per device; 256 on
// MI355X).  Launch shapes that place one workgroup per compute unit use it.
int device_cu_count();

}  // namespace q8
