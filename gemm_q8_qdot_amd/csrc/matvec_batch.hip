// Q8_0 matvec for a small batch of activation rows (2 <= M <= 7, decode of
// several sequences): every weight row is read from HBM once for all M rows.
//
// What is computed: the qdot_t (or, with transposed weight scales, qmma_t)
// row of the Q8_0 table ("Phobos Language Spec", section "Quantized
// built-ins"), with the inner block sums in integers ("Quantized built-ins
// and formats", section "Q8_0").
//
// Design: the single-row matvec's weight streaming (a wave owns R rows, lane
// l holds bytes [1024 s + 16 l, +16) of a row, lanes 2m and 2m+1 the two
// halves of one block, one DPP swap completes the int32 block sum), with the
// M activation rows and their scales staged once per workgroup in LDS (at
// most 7 x 16 KiB + scales).  Each 16-byte weight fragment is dotted with
// the M activation fragments read from LDS, so the weights cross the memory
// bus once instead of M times.  K <= 16 KiB; longer rows use the one-row
// kernel per activation row.
#include "q8_device.h"
#include "q8_launch.h"

namespace q8 {
namespace {

constexpr int kMbMaxM = 7;
constexpr int kMbStepBytes = kWave * 16;  // 1 KiB of a row per 16-byte lane load
constexpr int kMbMaxWaves = 256 * 32;

// WST: weight scales stored transposed, [K/32][N] (the qmma_t form).
// T: threads per workgroup (512 when the staged rows fill much of the LDS,
// so that one or two workgroups per CU still bring 8 or 16 waves).
template <int S, int R, bool PARTIALS, bool WST, int T>
__global__ void __launch_bounds__(T)
matvec_batch_kernel(const int8_t* __restrict__ A, const float* __restrict__ AS,
                    const int8_t* __restrict__ W, const float* __restrict__ WS,
                    float* __restrict__ C, int32_t* __restrict__ P, int M, int N, int K) {
    extern __shared__ __align__(16) int8_t mb_smem[];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = blockIdx.x * (T / kWave) + threadIdx.x / kWave;
    const int nwaves = gridDim.x * (T / kWave);
    const int KB = K / kBlock;
    const bool even = (lane & 1) == 0;
    int8_t* a_lds = mb_smem;                                            // [M][K]
    float* as_lds = reinterpret_cast<float*>(mb_smem + (int64_t)M * K);  // [M][K/32]

    // Stage the activation rows (contiguous: A is [M][K] dense) and scales.
    for (int idx = threadIdx.x * 16; idx < M * K; idx += T * 16)
        *reinterpret_cast<v4i*>(a_lds + idx) = load16(A + idx);
    if constexpr (!PARTIALS)
        for (int idx = threadIdx.x; idx < M * KB; idx += T) as_lds[idx] = AS[idx];
    __syncthreads();

    const int groups = (N + R - 1) / R;
    for (int g = wave; g < groups; g += nwaves) {
        const int j0 = g * R;
        v4i w[R][S];
        float ws[R][S];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int j = j0 + r;
            const int8_t* Wj = W + (int64_t)j * K;
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const int off = s * kMbStepBytes + lane * 16;
                const bool ok = j < N && off < K;
                w[r][s] = ok ? load16_stream(Wj + off) : v4i{0, 0, 0, 0};
                if constexpr (!PARTIALS) {
                    const int64_t widx = WST ? (int64_t)(off / kBlock) * N + j
                                             : (int64_t)j * KB + off / kBlock;
                    ws[r][s] = ok ? WS[widx] : 0.0f;
                }
            }
        }
        float acc[kMbMaxM][R];
#pragma unroll
        for (int m = 0; m < kMbMaxM; ++m)
#pragma unroll
            for (int r = 0; r < R; ++r) acc[m][r] = 0.0f;
#pragma unroll
        for (int m = 0; m < kMbMaxM; ++m) {
            if (m >= M) break;  // uniform
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const int off = s * kMbStepBytes + lane * 16;
                if (off >= K) continue;  // lanes past K: their weights are zero
                const v4i a = *reinterpret_cast<const v4i*>(a_lds + m * K + off);
                // the activation scale in even lanes only: each block counted once
                const float as = (!PARTIALS && even) ? as_lds[m * KB + off / kBlock] : 0.0f;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    int p = dot16(a, w[r][s], 0);
                    p += dpp_i32<kDppSwapPairs>(p);  // exact block sum in both lanes of the pair
                    if constexpr (PARTIALS) {
                        const int j = j0 + r;
                        if (even && j < N)
                            P[((int64_t)m * N + j) * KB + off / kBlock] = p;
                    } else {
                        acc[m][r] = fmaf(as * ws[r][s], (float)p, acc[m][r]);
                    }
                }
            }
        }
        if constexpr (!PARTIALS) {
#pragma unroll
            for (int m = 0; m < kMbMaxM; ++m) {
                if (m >= M) break;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float tot = wave_sum(acc[m][r]);
                    if (lane == 0 && j0 + r < N) C[(int64_t)m * N + j0 + r] = tot;
                }
            }
        }
    }
}

template <int S, bool PARTIALS, bool WST, int T>
hipError_t launch_mb_t(const int8_t* A, const float* AS, const int8_t* W, const float* WS,
                       float* C, int32_t* P, int M, int N, int K, size_t smem, hipStream_t stream) {
    constexpr int R = S <= 2 ? 2 : 1;  // short rows: two per wave
    auto kern = matvec_batch_kernel<S, R, PARTIALS, WST, T>;
    if (smem > 64 * 1024) {
        static bool attr_set = false;
        if (!attr_set) {
            hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               kMbMaxM * 16384 + kMbMaxM * 512 * 4);
            if (e != hipSuccess) return e;
            attr_set = true;
        }
    }
    const int groups = (N + R - 1) / R;
    const int waves = groups < kMbMaxWaves ? groups : kMbMaxWaves;
    const int wgs = (waves + T / kWave - 1) / (T / kWave);
    kern<<<dim3(wgs), T, smem, stream>>>(A, AS, W, WS, C, P, M, N, K);
    return hipGetLastError();
}

template <int S, bool PARTIALS, bool WST>
hipError_t launch_mb_s(const int8_t* A, const float* AS, const int8_t* W, const float* WS,
                       float* C, int32_t* P, int M, int N, int K, hipStream_t stream) {
    const size_t smem = (size_t)M * K + (PARTIALS ? 0 : (size_t)M * (K / kBlock) * 4);
    if (smem > 40 * 1024)  // at most three workgroups per CU: make them 8 waves
        return launch_mb_t<S, PARTIALS, WST, 512>(A, AS, W, WS, C, P, M, N, K, smem, stream);
    return launch_mb_t<S, PARTIALS, WST, 256>(A, AS, W, WS, C, P, M, N, K, smem, stream);
}

template <bool PARTIALS, bool WST>
hipError_t launch_mb(const int8_t* A, const float* AS, const int8_t* W, const float* WS,
                     float* C, int32_t* P, int M, int N, int K, hipStream_t stream) {
    const int steps = (K + kMbStepBytes - 1) / kMbStepBytes;
    switch (steps) {
#define Q8_MB_CASE(S_) \
    case S_: return launch_mb_s<S_, PARTIALS, WST>(A, AS, W, WS, C, P, M, N, K, stream);
        Q8_MB_CASE(1) Q8_MB_CASE(2) Q8_MB_CASE(3) Q8_MB_CASE(4)
        Q8_MB_CASE(5) Q8_MB_CASE(6) Q8_MB_CASE(7) Q8_MB_CASE(8)
        Q8_MB_CASE(9) Q8_MB_CASE(10) Q8_MB_CASE(11) Q8_MB_CASE(12)
        Q8_MB_CASE(13) Q8_MB_CASE(14) Q8_MB_CASE(15) Q8_MB_CASE(16)
#undef Q8_MB_CASE
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool matvec_batch_fits(int M, int K) { return M >= 2 && M <= kMbMaxM && K <= 16 * kMbStepBytes; }

hipError_t launch_matvec_batch(const int8_t* A, const float* AS, const int8_t* W, const float* WS,
                               float* C, int32_t* P, int M, int N, int K, bool ws_t,
                               hipStream_t stream) {
    if (!matvec_batch_fits(M, K)) return hipErrorInvalidValue;
    if (P != nullptr) return launch_mb<true, false>(A, AS, W, WS, C, P, M, N, K, stream);
    if (ws_t) return launch_mb<false, true>(A, AS, W, WS, C, P, M, N, K, stream);
    return launch_mb<false, false>(A, AS, W, WS, C, P, M, N, K, stream);
}

}  // namespace q8
