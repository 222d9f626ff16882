// Q8_0 block GEMM for M >= 8 (prompt projection) on CDNA4 int8 MFMA.
//
// What is computed: the qdot_t row of the Q8_0 table ("Phobos Language Spec",
// section "Quantized built-ins"); the pages' batched form qmma_t computes the
// same sum on integer tensor cores (same table).  One
// v_mfma_i32_32x32x32_i8 covers exactly one 32-wide Q8_0 block of a 32 x 32
// output tile, giving the exact int32 block sums P[i, j, b]; the block
// scales are applied in an f32 epilogue per block.
//
// MFMA lane layout relied on (32x32 family, wave64):
//   operand rows: lane l supplies row (l % 32) of its operand and the 16
//   bytes k in [16 (l / 32), +16) of the block -- both operands use the same
//   k split, so the product sums all 32 k of the block whatever order the
//   hardware uses inside a lane's 16 bytes;
//   result: lane l, register r holds D[m][n] with n = l % 32 and
//   m = 8 (r / 4) + 4 (l / 32) + (r % 4).
// With the activation tile as the first operand, m is the activation row i
// and n the weight row j: each lane owns one output column j and 16 rows.
#include "q8_device.h"
#include "q8_launch.h"

namespace q8 {
namespace {

constexpr int kTile = 32;
constexpr int kQgemmWaves = 4;  // waves per workgroup, side by side along N

__device__ __forceinline__ int tile_row(int r, int half) {
    return 8 * (r / 4) + 4 * half + (r % 4);
}

template <bool PARTIALS>
__global__ void __launch_bounds__(kQgemmWaves * kWave)
qgemm_simple_kernel(const int8_t* __restrict__ A, const float* __restrict__ AS,
                    const int8_t* __restrict__ W, const float* __restrict__ WS,
                    float* __restrict__ C, int32_t* __restrict__ P, int M, int N, int K,
                    int n_groups) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    const int i0 = (blockIdx.x / n_groups) * kTile;
    const int j0 = ((blockIdx.x % n_groups) * kQgemmWaves + wv) * kTile;
    if (j0 >= N) return;  // whole wave
    const int KB = K / kBlock;
    const int half = lane / 32;
    const int ra = i0 + (lane & 31);
    const int rw = j0 + (lane & 31);
    const bool a_ok = ra < M;
    const bool w_ok = rw < N;
    const int8_t* Ap = A + (int64_t)ra * K + 16 * half;
    const int8_t* Wp = W + (int64_t)rw * K + 16 * half;
    const v16i zero = {};

    float acc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;

    for (int b = 0; b < KB; ++b) {
        const v4i af = a_ok ? load16(Ap + (int64_t)kBlock * b) : v4i{0, 0, 0, 0};
        const v4i wf = w_ok ? load16(Wp + (int64_t)kBlock * b) : v4i{0, 0, 0, 0};
        const v16i d = __builtin_amdgcn_mfma_i32_32x32x32_i8(af, wf, zero, 0, 0, 0);
        if constexpr (PARTIALS) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = i0 + tile_row(r, half);
                if (i < M && w_ok) P[((int64_t)i * N + rw) * KB + b] = d[r];
            }
        } else {
            const float ws = w_ok ? WS[(int64_t)rw * KB + b] : 0.0f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = i0 + tile_row(r, half);
                const float as = i < M ? AS[(int64_t)i * KB + b] : 0.0f;
                acc[r] = fmaf(as * ws, (float)d[r], acc[r]);
            }
        }
    }
    if constexpr (!PARTIALS) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int i = i0 + tile_row(r, half);
            if (i < M && w_ok) C[(int64_t)i * N + rw] = acc[r];
        }
    }
}

}  // namespace

hipError_t launch_qgemm(const int8_t* A, const float* AS, const int8_t* W, const float* WS,
                        float* C, int32_t* P, int M, int N, int K, hipStream_t stream) {
    const int n_groups = (N + kTile * kQgemmWaves - 1) / (kTile * kQgemmWaves);
    const int64_t m_tiles = (M + kTile - 1) / kTile;
    const int64_t blocks = m_tiles * n_groups;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    dim3 grid((unsigned)blocks);
    if (P != nullptr)
        qgemm_simple_kernel<true><<<grid, kQgemmWaves * kWave, 0, stream>>>(A, AS, W, WS, C, P, M, N, K, n_groups);
    else
        qgemm_simple_kernel<false><<<grid, kQgemmWaves * kWave, 0, stream>>>(A, AS, W, WS, C, P, M, N, K, n_groups);
    return hipGetLastError();
}

}  // namespace q8
