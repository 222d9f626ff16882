// C-ABI of the Q8_0 contraction library: host-side validation and dispatch.
// Declarations and the contract of every entry point: include/q8qdot.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "q8qdot.h"
#include "q8_launch.h"

#define Q8_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kVersion = 203;  // 0.2.3: Q5_0 weights on the 64 x 64-tile ring GEMM (q8_q50_path)
constexpr int kMatvecMaxM = 7;  // M < 8 -> matvec; the MFMA path needs 8+ rows to pay off

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int check_shape(int M, int N, int K) {
    if (M < 0 || N < 0 || K < 0 || K % 32 != 0) return Q8_EINVAL;
    return Q8_OK;
}

// Largest element offset any kernel forms must fit in int64 bytes.
int check_range(int64_t M, int64_t N, int64_t K, bool partials) {
    const int64_t lim = INT64_MAX / 8;
    if (M > 0 && K > lim / M) return Q8_ERANGE;
    if (N > 0 && K > lim / N) return Q8_ERANGE;
    if (M > 0 && N > lim / M) return Q8_ERANGE;
    if (partials && M > 0 && N > 0 && K / 32 > lim / (M * N)) return Q8_ERANGE;
    return Q8_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? Q8_OK : Q8_ELAUNCH; }

// The block GEMM a Q8_0 shape with M >= 8 takes (q8_qdot_path's numbers):
// 1 = K-split (32 x 32 tiles), 2 = LDS-staged (128 x 224 tiles), 3 = the
// 64 x 64-tile ring kernel over all of K (the split-K kernel's one-slice
// form), which takes over from either where it is faster.
int gemm_path(int M, int N, int K) {
    const int v = q8::qgemm_variant(M, N, K);
    if (v == 1) return q8::splitk_whole_k(M, N, K) ? 3 : 1;
    return q8::splitk_over_staged(M, N, K) ? 3 : v;
}

// ws_t: WS is the qmma_t form, stored transposed [K/32][N].  split: the
// workspace entries -- shapes with few output tiles take the split-K GEMM
// when `workspace` holds at least the bytes it needs (the debug entry needs
// none and passes split with a null workspace).
int run_qdot(const int8_t* A, const float* AS, const int8_t* W, const float* WS, float* C,
             int32_t* P, int M, int N, int K, bool ws_t, hipStream_t stream,
             bool split = false, void* workspace = nullptr, size_t ws_bytes = 0) {
    int st = check_shape(M, N, K);
    if (st != Q8_OK) return st;
    st = check_range(M, N, K, P != nullptr);
    if (st != Q8_OK) return st;
    if (M == 0 || N == 0) return Q8_OK;  // empty output
    const bool partials = P != nullptr;
    if (K == 0) {
        // Empty sum over blocks: C = 0; P has no elements.
        if (partials) return Q8_OK;
        if (C == nullptr) return Q8_ENULL;
        if (!aligned(C, 4)) return Q8_EALIGN;
        return status_of(q8::launch_fill_zero(C, (int64_t)M * N, stream));
    }
    // The block GEMMs address a 32-row operand tile, and the transposed
    // weight scales from a column to the end, with 32-bit offsets.
    if (M > kMatvecMaxM && (int64_t)K * 32 > INT32_MAX) return Q8_ERANGE;
    if (M > kMatvecMaxM && ws_t && (int64_t)(K / 32) * N * 4 > INT32_MAX) return Q8_ERANGE;
    if (A == nullptr || W == nullptr) return Q8_ENULL;
    if (!partials && (AS == nullptr || WS == nullptr || C == nullptr)) return Q8_ENULL;
    if (!aligned(A, 16) || !aligned(W, 16)) return Q8_EALIGN;
    if (partials) {
        if (!aligned(P, 4)) return Q8_EALIGN;
    } else if (!aligned(AS, 4) || !aligned(WS, 4) || !aligned(C, 4)) {
        return Q8_EALIGN;
    }
    if (split && M > kMatvecMaxM && q8::qgemm_variant(M, N, K) == 1) {
        int S = 0, sb = 0;
        size_t need = 0;
        if (q8::splitk_plan(M, N, K, &S, &sb, &need) &&
            (partials || (workspace != nullptr && ws_bytes >= need && aligned(workspace, 16))))
            return status_of(q8::launch_qgemm_splitk(A, AS, W, WS, C, P, M, N, K, ws_t, S, sb,
                                                     workspace, stream));
    }
    if (M > kMatvecMaxM && gemm_path(M, N, K) == 3)
        return status_of(q8::launch_qgemm_splitk(A, AS, W, WS, C, P, M, N, K, ws_t, 1,
                                                 q8::splitk_whole_k_blocks(K), nullptr, stream));
    hipError_t e = M <= kMatvecMaxM
                       ? q8::launch_matvec(A, AS, W, WS, C, P, M, N, K, ws_t, stream)
                       : q8::launch_qgemm(A, AS, W, WS, C, P, M, N, K, ws_t, stream);
    return status_of(e);
}

}  // namespace

Q8_API int q8_qdot_stream(const int8_t* A, const float* AS, const int8_t* W, const float* WS,
                          float* C, int M, int N, int K, void* stream) {
    return run_qdot(A, AS, W, WS, C, nullptr, M, N, K, false, static_cast<hipStream_t>(stream));
}

Q8_API int q8_qmma(const int8_t* A, const float* AS, const int8_t* W, const float* WST,
                   float* C, int M, int N, int K, void* stream) {
    return run_qdot(A, AS, W, WST, C, nullptr, M, N, K, true, static_cast<hipStream_t>(stream));
}

Q8_API int q8_qdot(const int8_t* A, const float* AS, const int8_t* W, const float* WS,
                   float* C, int M, int N, int K) {
    return run_qdot(A, AS, W, WS, C, nullptr, M, N, K, false, nullptr);
}

Q8_API int q8_qdot_partials(const int8_t* A, const int8_t* W, int32_t* P, int M, int N, int K,
                            void* stream) {
    if (P == nullptr) {
        int st = check_shape(M, N, K);
        if (st != Q8_OK) return st;
        if (M == 0 || N == 0 || K == 0) return Q8_OK;
        return Q8_ENULL;
    }
    return run_qdot(A, nullptr, W, nullptr, nullptr, P, M, N, K, false, static_cast<hipStream_t>(stream));
}

Q8_API int q8_qdot_ws_size(int M, int N, int K, size_t* bytes) {
    if (bytes == nullptr) return Q8_ENULL;
    *bytes = 0;
    int st = check_shape(M, N, K);
    if (st != Q8_OK) return st;
    st = check_range(M, N, K, false);
    if (st != Q8_OK) return st;
    if (M > kMatvecMaxM && K > 0 && N > 0 && q8::qgemm_variant(M, N, K) == 1) {
        int S = 0, sb = 0;
        size_t need = 0;
        if (q8::splitk_plan(M, N, K, &S, &sb, &need)) *bytes = need;
    }
    return Q8_OK;
}

Q8_API int q8_qdot_ws(const int8_t* A, const float* AS, const int8_t* W, const float* WS,
                      float* C, int M, int N, int K, void* workspace, size_t ws_bytes,
                      void* stream) {
    return run_qdot(A, AS, W, WS, C, nullptr, M, N, K, false, static_cast<hipStream_t>(stream),
                    true, workspace, ws_bytes);
}

Q8_API int q8_qmma_ws(const int8_t* A, const float* AS, const int8_t* W, const float* WST,
                      float* C, int M, int N, int K, void* workspace, size_t ws_bytes,
                      void* stream) {
    return run_qdot(A, AS, W, WST, C, nullptr, M, N, K, true, static_cast<hipStream_t>(stream),
                    true, workspace, ws_bytes);
}

Q8_API int q8_qdot_ws_partials(const int8_t* A, const int8_t* W, int32_t* P, int M, int N, int K,
                               void* stream) {
    if (P == nullptr) {
        int st = check_shape(M, N, K);
        if (st != Q8_OK) return st;
        if (M == 0 || N == 0 || K == 0) return Q8_OK;
        return Q8_ENULL;
    }
    return run_qdot(A, nullptr, W, nullptr, nullptr, P, M, N, K, false,
                    static_cast<hipStream_t>(stream), true);
}

// The no-allocation variant of q8_qdot_ws: the split form's workspace is
// the library's static scratch array; other shapes run exactly q8_qdot_stream.
Q8_API int q8_qdot_noalloc(const int8_t* A, const float* AS, const int8_t* W, const float* WS,
                           float* C, int M, int N, int K, void* stream) {
    int st = check_shape(M, N, K);
    if (st != Q8_OK) return st;
    st = check_range(M, N, K, false);
    if (st != Q8_OK) return st;
    int S = 0, sb = 0;
    size_t need = 0;
    const bool split = M > kMatvecMaxM && N > 0 && K > 0 && q8::qgemm_variant(M, N, K) == 1 &&
                       q8::splitk_plan(M, N, K, &S, &sb, &need);
    if (!split)
        return run_qdot(A, AS, W, WS, C, nullptr, M, N, K, false, static_cast<hipStream_t>(stream));
    if (need > q8::splitk_scratch_capacity()) return Q8_ERANGE;
    if ((int64_t)K * 32 > INT32_MAX) return Q8_ERANGE;
    if (A == nullptr || W == nullptr || AS == nullptr || WS == nullptr || C == nullptr) return Q8_ENULL;
    if (!aligned(A, 16) || !aligned(W, 16) || !aligned(AS, 4) || !aligned(WS, 4) || !aligned(C, 4))
        return Q8_EALIGN;
    return status_of(q8::launch_qgemm_splitk_scratch(A, AS, W, WS, C, M, N, K, false, S, sb,
                                                     static_cast<hipStream_t>(stream)));
}

// Q5_0 weights at M >= 8: the 64 x 64-tile ring GEMM (each stage's blocks
// decoded once in LDS) for the shapes whose Q8_0 GEMM is the staged one or
// that kernel -- there is no staged form for Q5_0 -- and that have more of
// its tiles than compute units (two workgroups per unit: with one, its
// per-stage decode and second barrier made it slower than the K-split GEMM),
// when its whole-piece loads of the weight rows are 16-byte aligned (K/32 a
// multiple of 4, and a 16-byte aligned W5, checked by the caller); else the
// K-split GEMM.
bool q50_ring(int M, int N, int K) {
    return M > kMatvecMaxM && (K / 32) % 4 == 0 && gemm_path(M, N, K) >= 2 && q8::splitk_shared(M, N);
}

// Q5_0 weights: W5 is [N][K/32 * 20] bytes, 4-byte aligned (dword loads).
static int run_q50(const int8_t* A, const float* AS, const uint8_t* W5, const float* WS, float* C,
            int32_t* P, int M, int N, int K, bool ws_t, hipStream_t stream) {
    int st = check_shape(M, N, K);
    if (st != Q8_OK) return st;
    st = check_range(M, N, K, P != nullptr);
    if (st != Q8_OK) return st;
    if (M == 0 || N == 0) return Q8_OK;
    const bool partials = P != nullptr;
    if (K == 0) {
        if (partials) return Q8_OK;
        if (C == nullptr) return Q8_ENULL;
        if (!aligned(C, 4)) return Q8_EALIGN;
        return status_of(q8::launch_fill_zero(C, (int64_t)M * N, stream));
    }
    // The matvec addresses the whole weight array with 32-bit offsets.
    const bool matvec = M <= kMatvecMaxM && q8::matvec_q50_fits(K) &&
                        (int64_t)N * (K / 32) * 20 < INT32_MAX - (1 << 20);
    if (!matvec && (int64_t)K * 32 > INT32_MAX) return Q8_ERANGE;
    if (!matvec && ws_t && (int64_t)(K / 32) * N * 4 > INT32_MAX) return Q8_ERANGE;
    if (A == nullptr || W5 == nullptr) return Q8_ENULL;
    if (!partials && (AS == nullptr || WS == nullptr || C == nullptr)) return Q8_ENULL;
    if (!aligned(A, 16) || !aligned(W5, 4)) return Q8_EALIGN;
    if (partials) {
        if (!aligned(P, 4)) return Q8_EALIGN;
    } else if (!aligned(AS, 4) || !aligned(WS, 4) || !aligned(C, 4)) {
        return Q8_EALIGN;
    }
    hipError_t e;
    if (matvec)
        e = q8::launch_matvec_q50(A, AS, W5, WS, C, P, M, N, K, ws_t, stream);
    else if (q50_ring(M, N, K) && aligned(W5, 16))
        e = q8::launch_qgemm_splitk_q50(A, AS, W5, WS, C, P, M, N, K, ws_t, stream);
    else
        e = q8::launch_qgemm_ksplit_q50(A, AS, W5, WS, C, P, M, N, K, ws_t, stream);
    return status_of(e);
}

Q8_API int q8_q50_qdot(const int8_t* A, const float* AS, const uint8_t* W5, const float* WS,
                       float* C, int M, int N, int K, void* stream) {
    return run_q50(A, AS, W5, WS, C, nullptr, M, N, K, false, static_cast<hipStream_t>(stream));
}

Q8_API int q8_q50_qmma(const int8_t* A, const float* AS, const uint8_t* W5, const float* WST,
                       float* C, int M, int N, int K, void* stream) {
    return run_q50(A, AS, W5, WST, C, nullptr, M, N, K, true, static_cast<hipStream_t>(stream));
}

Q8_API int q8_q50_partials(const int8_t* A, const uint8_t* W5, int32_t* P, int M, int N, int K,
                           void* stream) {
    if (P == nullptr) {
        int st = check_shape(M, N, K);
        if (st != Q8_OK) return st;
        if (M == 0 || N == 0 || K == 0) return Q8_OK;
        return Q8_ENULL;
    }
    return run_q50(A, nullptr, W5, nullptr, nullptr, P, M, N, K, false, static_cast<hipStream_t>(stream));
}

Q8_API int q8_qdot_path(int M, int N, int K) {
    int st = check_shape(M, N, K);
    if (st != Q8_OK) return st;
    return M <= kMatvecMaxM ? 0 : gemm_path(M, N, K);
}

Q8_API int q8_quantize(const float* X, int8_t* Q, float* D, int rows, int K, void* stream) {
    if (rows < 0 || K < 0 || K % 32 != 0) return Q8_EINVAL;
    if (rows > 0 && K > INT64_MAX / 8 / rows) return Q8_ERANGE;
    if (rows == 0 || K == 0) return Q8_OK;
    if (X == nullptr || Q == nullptr || D == nullptr) return Q8_ENULL;
    if (!aligned(X, 16) || !aligned(Q, 16) || !aligned(D, 4)) return Q8_EALIGN;
    return status_of(q8::launch_quantize(X, Q, D, rows, K, static_cast<hipStream_t>(stream)));
}

Q8_API const char* q8_strerror(int status) {
    switch (status) {
        case Q8_OK: return "ok";
        case Q8_EINVAL: return "invalid shape: M, N, K must be >= 0 and K a multiple of 32";
        case Q8_ENULL: return "null pointer for an operand the call must dereference";
        case Q8_EALIGN: return "misaligned pointer: A, W, X, Q need 16 bytes, Q5_0 weights and f32/int32 arrays 4";
        case Q8_ERANGE: return "shape out of range: an extent product overflows 64-bit addressing, a GEMM offset 32 bits, "
                               "or (q8_qdot_noalloc) the split form needs more than its 4 MiB static scratch";
        case Q8_ELAUNCH: return "HIP runtime rejected the kernel launch";
        default: return "unknown status";
    }
}

Q8_API int q8_q50_path(int M, int N, int K) {
    const int st = check_shape(M, N, K);
    if (st != Q8_OK) return st;
    if (M <= kMatvecMaxM && q8::matvec_q50_fits(K) && (int64_t)N * (K / 32) * 20 < INT32_MAX - (1 << 20))
        return 0;
    return q50_ring(M, N, K) ? 3 : 1;
}

Q8_API int q8_version(void) { return kVersion; }
