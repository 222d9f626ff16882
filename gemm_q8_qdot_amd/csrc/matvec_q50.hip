// Q5_0-weight matvec for small M (decode step): C[i, :] = q50_qdot_t (or,
// with transposed weight scales, q50_qmma_t) of activation row i.
//
// What is computed: the q50 rows of the Q8_0 table ("Phobos Language Spec",
// section "Quantized built-ins"): the Q8_0 contraction against a weight held
// as Q5_0 blocks without their scale -- per 32 values 20 bytes, the qh word
// then 16 bytes whose byte e holds element e (low nibble) and element e + 16
// (high nibble); element value q - 16, q the 5-bit number with bit e of qh
// (little-endian) as bit 4.  The 20 bytes per 32 values plus the 4-byte
// scale are all that is read of the weights; the codes are rebuilt in
// registers ("Quantized built-ins and formats", introduction).
//
// Design for CDNA4 wave64: lane l owns whole blocks b = l + 64 t of a row;
// the rows arrive as contiguous 1 KiB wave loads staged in LDS (see the
// kernel).  The lane's activation bytes for its blocks stay in VGPRs, with
// their block sums.  Per block: the 5-bit codes q are rebuilt
// as bytes (nibble | qh bit << 4; four qh bits are spread to four bytes by
// one 24-bit multiply), and eight v_dot4_i32_i8 chained from -16 * sum a
// (the block's activation sum, computed once) give sum a*(q - 16) exactly
// in int32.  A DPP fold sums
// the row over the wave.  A batch of 2..7 activation rows (MULTI) is staged
// in LDS once per workgroup and every decoded block is dotted with all of
// them, so the weights cross the bus once for the whole batch.
#include "q8_device.h"
#include "q8_launch.h"

namespace q8 {
namespace {

constexpr int kQ5Threads = 256;
constexpr int kQ5BatchThreads = 512;      // MULTI: eight waves share one staged batch
constexpr int kQ5BlockBytes = 20;
constexpr int kQ5MaxT = 8;               // K <= 64 * 8 blocks (16 Ki values) resident
constexpr int kQ5MaxBatch = 7;
constexpr int kQ5MaxLds = 160 * 1024;

// WST: weight scales stored transposed, [K/32][N] (q50_qmma_t).
// A wave reads its R weight rows as contiguous 16-byte pieces (lane l takes
// bytes [16 (l + 64 s), +16) of the rows' bytes: full 1 KiB transactions),
// parks them in its own LDS area, and each lane then reads back its whole
// 20-byte blocks (5-dword stride across lanes: no bank conflicts).  The
// weight array is read through a raw buffer resource, so pieces past its
// end read as zero.
//
// MULTI (2 <= M <= 7 activation rows, f32 outputs): the rows are staged in
// LDS after the weight staging areas, row m at m * K bytes, each block's
// two 16-byte halves in two regions ([KB][16] low halves, then the high
// halves) so that lanes reading consecutive blocks read consecutive 16-byte
// words; then one 8-byte record per row and block, {sum of the block's 32
// bytes, its scale}.  Each lane decodes a block once and dots it with every
// row; a row's arithmetic is exactly that of the one-row kernel.
template <int T, int R, bool PARTIALS, bool WST, bool MULTI, int NT>
__global__ void __launch_bounds__(NT)
matvec_q50_kernel(const int8_t* __restrict__ A, const float* __restrict__ AS,
                  const uint8_t* __restrict__ W5, const float* __restrict__ WS,
                  float* __restrict__ C, int32_t* __restrict__ P, int N, int K, int M) {
    static_assert(!(MULTI && PARTIALS), "the batch form computes f32 outputs only");
    extern __shared__ __align__(16) uint8_t q5_smem[];
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    const int wave = blockIdx.x * (NT / kWave) + wv;
    const int nwaves = gridDim.x * (NT / kWave);
    const int i = MULTI ? 0 : (int)blockIdx.y;
    const int KB = K / kBlock;
    const int row_bytes = KB * kQ5BlockBytes;
    const int group_bytes = R * row_bytes;            // this wave's rows, contiguous in W5
    const int pieces = (group_bytes + 15) / 16;       // 16-byte pieces of the group
    constexpr int kPieceRounds = (R * T * kWave * kQ5BlockBytes + kWave * 16 - 1) / (kWave * 16);
    uint8_t* area = q5_smem + (size_t)wv * kPieceRounds * kWave * 16;
    int8_t* a_lds = reinterpret_cast<int8_t*>(q5_smem + (size_t)(NT / kWave) * kPieceRounds * kWave * 16);
    float* as_lds = reinterpret_cast<float*>(a_lds + K);
    int2* sa_lds = reinterpret_cast<int2*>(a_lds + (MULTI ? M : 0) * K);  // MULTI: {-16 * block sum, scale bits}
    const __amdgpu_buffer_rsrc_t rW5 = buffer_rsrc(W5, (int64_t)N * row_bytes);

    const int groups = (N + R - 1) / R;
    // A group's bytes: contiguous 16-byte pieces (the resource zeroes pieces
    // past the array; pieces past the group are not needed).  The next
    // group's pieces are loaded into registers while this group, already
    // parked in LDS, is decoded and computed.
    // Rows of up to 256 blocks: the group's weight scales come with its
    // pieces, one group ahead too (loaded when the group is about to be
    // computed, their latency was exposed once per group: N=14336, K=4096
    // 9.9 -> 9.6 us, M=4 14.2 -> 13.3 us); longer rows load them with the
    // group (K=14336: 12.0 against 12.4 us ahead, where the extra registers
    // cost more).
    constexpr bool kWsAhead = T <= 4;
    v4i piece[kPieceRounds];
    float ws_next[R][T];
    // Transposed scales with R = 2 or 4 consecutive rows per group: a lane's
    // R scales of one block are adjacent (WST[b][j0 .. j0 + R - 1]) and come
    // as one 8- or 16-byte load when N is a multiple of R and WS is aligned
    // to it (else one 4-byte load per row and block, 64 cache lines per
    // instruction).
    const bool ws_vec = WST && (R == 2 || R == 4) && N % R == 0 &&
                        (reinterpret_cast<uintptr_t>(WS) & (4 * R - 1)) == 0;
    auto load_ws = [&](int g, float (&ws)[R][T]) {
        const int j0 = g * R;
        if constexpr (WST && (R == 2 || R == 4)) {
            if (ws_vec) {
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    const int b = lane + kWave * t;
                    const bool ok = j0 < N && b < KB;
                    const float* src = WS + (ok ? (int64_t)b * N + j0 : 0);
                    if constexpr (R == 4) {
                        const float4 v = ok ? *reinterpret_cast<const float4*>(src) : make_float4(0.f, 0.f, 0.f, 0.f);
                        ws[0][t] = v.x; ws[1][t] = v.y; ws[2][t] = v.z; ws[3][t] = v.w;
                    } else {
                        const float2 v = ok ? *reinterpret_cast<const float2*>(src) : make_float2(0.f, 0.f);
                        ws[0][t] = v.x; ws[1][t] = v.y;
                    }
                }
                return;
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const int j = j0 + r;
                const int b = lane + kWave * t;
                const int64_t widx = WST ? (int64_t)b * N + j : (int64_t)j * KB + b;
                ws[r][t] = (j < N && b < KB) ? WS[widx] : 0.0f;
            }
    };
    auto load_group = [&](int g) {
        const int gbase = g * R * row_bytes;
#pragma unroll
        for (int s = 0; s < kPieceRounds; ++s) {
            const int pc = lane + kWave * s;
            piece[s] = buffer_load16_nt(rW5, pc < pieces ? gbase + 16 * pc : kNoRead, 0);  // read once: streaming
        }
        if constexpr (!PARTIALS && kWsAhead) load_ws(g, ws_next);
    };
    // The first group's pieces are in flight while the activation row is
    // staged (its latency and theirs overlap).
    if (wave < groups) load_group(wave);

    // The activation row(s) and scales, read once per workgroup (not once
    // per wave) and shared through LDS.
    if constexpr (MULTI) {
        const int pieces_row = K / 16;
        for (int idx = threadIdx.x; idx < M * pieces_row; idx += NT) {
            const int m = idx / pieces_row, pc = idx % pieces_row;
            *reinterpret_cast<v4i*>(a_lds + m * K + (pc & 1) * KB * 16 + (pc >> 1) * 16) =
                load16(A + (int64_t)m * K + pc * 16);
        }
        __syncthreads();
        const v4i ones = v4i{0x01010101, 0x01010101, 0x01010101, 0x01010101};
        for (int idx = threadIdx.x; idx < M * KB; idx += NT) {
            const int m = idx / KB, b = idx % KB;
            const v4i lo = *reinterpret_cast<const v4i*>(a_lds + m * K + b * 16);
            const v4i hi = *reinterpret_cast<const v4i*>(a_lds + m * K + KB * 16 + b * 16);
            sa_lds[idx] = int2{-16 * dot16(hi, ones, dot16(lo, ones, 0)), __float_as_int(AS[(int64_t)m * KB + b])};
        }
    } else {
        for (int idx = threadIdx.x * 16; idx < K; idx += NT * 16)
            *reinterpret_cast<v4i*>(a_lds + idx) = load16(A + (int64_t)i * K + idx);
        if constexpr (!PARTIALS)
            for (int idx = threadIdx.x; idx < KB; idx += NT) as_lds[idx] = AS[(int64_t)i * KB + idx];
    }
    __syncthreads();

    // This lane's activation blocks b = lane + 64 t: bytes, block sums, scales.
    constexpr int TA = MULTI ? 1 : T;  // the batch form reads its rows from LDS
    v4i a_lo[TA], a_hi[TA];
    int a_c[TA];  // -16 * (sum of the block's activation bytes)
    float a_s[TA];
#pragma unroll
    for (int t = 0; t < (MULTI ? 0 : T); ++t) {
        const int b = lane + kWave * t;
        const bool ok = b < KB;
        const int8_t* Ab = a_lds + (ok ? b : 0) * kBlock;
        a_lo[t] = ok ? *reinterpret_cast<const v4i*>(Ab) : v4i{0, 0, 0, 0};
        a_hi[t] = ok ? *reinterpret_cast<const v4i*>(Ab + 16) : v4i{0, 0, 0, 0};
        if constexpr (!PARTIALS) a_s[t] = ok ? as_lds[b] : 0.0f;
        int s = dot16(a_lo[t], v4i{0x01010101, 0x01010101, 0x01010101, 0x01010101}, 0);
        a_c[t] = -16 * dot16(a_hi[t], v4i{0x01010101, 0x01010101, 0x01010101, 0x01010101}, s);
    }

    for (int g = wave; g < groups; g += nwaves) {
        const int j0 = g * R;
        float ws[R][T];
        if constexpr (!PARTIALS) {
            if constexpr (kWsAhead) {
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int t = 0; t < T; ++t) ws[r][t] = ws_next[r][t];
            } else {
                load_ws(g, ws);
            }
        }
        // The previous group's reads of this area are done (one wave, in order).
        asm volatile("" ::: "memory");
#pragma unroll
        for (int s = 0; s < kPieceRounds; ++s)
            *reinterpret_cast<v4i*>(area + 16 * (lane + kWave * s)) = piece[s];
        asm volatile("" ::: "memory");
        if (g + nwaves < groups) load_group(g + nwaves);

        if constexpr (MULTI) {
            float acc[kQ5MaxBatch][R];
#pragma unroll
            for (int m = 0; m < kQ5MaxBatch; ++m)
#pragma unroll
                for (int r = 0; r < R; ++r) acc[m][r] = 0.0f;
#pragma unroll
            for (int r = 0; r < R; ++r) {
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    const int b = lane + kWave * t;
                    const bool ok = b < KB;
                    const int bb = ok ? b : 0;
                    const uint32_t* blk = reinterpret_cast<const uint32_t*>(area + r * row_bytes + bb * kQ5BlockBytes);
                    const uint32_t qh = blk[0];
                    const v4i qs = v4i{(int)blk[1], (int)blk[2], (int)blk[3], (int)blk[4]};
                    uint32_t q[8];
                    q50_codes(qh, qs, q);
                    const v4i qlo = v4i{(int)q[0], (int)q[1], (int)q[2], (int)q[3]};
                    const v4i qhi = v4i{(int)q[4], (int)q[5], (int)q[6], (int)q[7]};
#pragma unroll
                    for (int m = 0; m < kQ5MaxBatch; ++m) {
                        if (m >= M) break;  // uniform
                        const v4i lo = *reinterpret_cast<const v4i*>(a_lds + m * K + bb * 16);
                        const v4i hi = *reinterpret_cast<const v4i*>(a_lds + m * K + KB * 16 + bb * 16);
                        const int2 sa = sa_lds[m * KB + bb];
                        // sum a * (q - 16) = sum a * q - 16 * sum a, exact
                        const int p = dot16(hi, qhi, dot16(lo, qlo, sa.x));
                        const float as_m = ok ? __int_as_float(sa.y) : 0.0f;
                        acc[m][r] = fmaf(as_m * ws[r][t], (float)p, acc[m][r]);
                    }
                }
            }
#pragma unroll
            for (int m = 0; m < kQ5MaxBatch; ++m) {
                if (m >= M) break;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float tot = wave_sum(acc[m][r]);
                    if (lane == 0 && j0 + r < N) C[(int64_t)m * N + j0 + r] = tot;
                }
            }
        } else {
            float acc[R];
#pragma unroll
            for (int r = 0; r < R; ++r) acc[r] = 0.0f;
#pragma unroll
            for (int r = 0; r < R; ++r) {
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    const int b = lane + kWave * t;
                    const uint32_t* blk = reinterpret_cast<const uint32_t*>(
                        area + r * row_bytes + (b < KB ? b : 0) * kQ5BlockBytes);
                    const uint32_t qh = blk[0];
                    const v4i qs = v4i{(int)blk[1], (int)blk[2], (int)blk[3], (int)blk[4]};
                    uint32_t q[8];
                    q50_codes(qh, qs, q);
                    // sum a * (q - 16) = sum a * q - 16 * sum a, exact
                    int p = dot16(a_lo[t], v4i{(int)q[0], (int)q[1], (int)q[2], (int)q[3]}, a_c[t]);
                    p = dot16(a_hi[t], v4i{(int)q[4], (int)q[5], (int)q[6], (int)q[7]}, p);
                    if constexpr (PARTIALS) {
                        if (j0 + r < N && b < KB) P[((int64_t)i * N + j0 + r) * KB + b] = p;
                    } else {
                        acc[r] = fmaf(a_s[t] * ws[r][t], (float)p, acc[r]);
                    }
                }
            }
            if constexpr (!PARTIALS) {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float tot = wave_sum(acc[r]);
                    if (lane == 0 && j0 + r < N) C[(int64_t)i * N + j0 + r] = tot;
                }
            }
        }
    }
}

template <int T, bool PARTIALS, bool WST>
hipError_t launch_q5_t(const int8_t* A, const float* AS, const uint8_t* W5, const float* WS,
                       float* C, int32_t* P, int M, int N, int K, hipStream_t stream) {
    // Launch shape, measured on MI355X (N=14336): rows of 2 KiB or less go
    // four to a wave group, eight waves per compute unit; rows of 65..192
    // blocks (K = 2080..6144) one per group, sixteen waves per compute unit
    // (K=4096: 11.0 -> 10.6 us against two rows per group and eight waves;
    // K=6144: 15.4 -> 14.2 us); longer rows one per group, eight waves (at
    // K=8192 sixteen tie, at K=14336 they are 12 % slower).
    // Rows per wave group: four for rows of 64 blocks or less; with
    // transposed scales also four for up to 192 blocks and two for up to 256
    // (so that a lane's scales of one block arrive as one vector load).
    constexpr int R = T == 1 ? 4 : (WST ? (T <= 3 ? 4 : (T == 4 ? 2 : 1)) : 1);
    // Waves per compute unit: sixteen for rows of 65..192 blocks (one row a
    // group), eight otherwise; twelve for the transposed-scale groups of two
    // or four longer rows (their registers allow three waves per SIMD;
    // measured N=14336, K=4096: 13.3 us against 13.7 with eight or sixteen,
    // 21.8 us with one row a group and per-row scale gathers).
    constexpr int kWavesPerCU = (WST && R > 1 && T > 1) ? 12 : ((T == 2 || T == 3) ? 16 : 8);
    constexpr int kPieceRounds = (R * T * kWave * kQ5BlockBytes + kWave * 16 - 1) / (kWave * 16);
    const int groups = (N + R - 1) / R;
    if constexpr (!PARTIALS) {
        // A batch of rows in one pass when the staged rows fit in LDS beside
        // eight waves' weight areas (else one grid row per activation row).
        constexpr int kWavesWG = kQ5BatchThreads / kWave;
        const size_t smem_b = (size_t)kWavesWG * kPieceRounds * kWave * 16 + (size_t)M * K +
                              (size_t)M * (K / kBlock) * 8;
        if (M >= 2 && M <= kQ5MaxBatch && smem_b <= (size_t)kQ5MaxLds) {
            auto kern = matvec_q50_kernel<T, R, false, WST, true, kQ5BatchThreads>;
            static std::atomic<uint64_t> lds_set{0};
            const hipError_t e = set_dynamic_lds(reinterpret_cast<const void*>(kern), kQ5MaxLds, lds_set);
            if (e != hipSuccess) return e;
            int wpc = kWavesPerCU / kWavesWG;  // workgroups per compute unit, as LDS allows
            const int fit = (int)((size_t)kQ5MaxLds / smem_b);
            if (wpc > fit) wpc = fit;
            const int max_wb = device_cu_count() * wpc * kWavesWG;
            const int waves_b = groups < max_wb ? groups : max_wb;
            const int wgs_b = (waves_b + kWavesWG - 1) / kWavesWG;
            kern<<<dim3(wgs_b, 1), kQ5BatchThreads, smem_b, stream>>>(A, AS, W5, WS, C, P, N, K, M);
            return hipGetLastError();
        }
    }
    // one activation row per grid row: per-wave weight staging areas, then
    // the row and its scales
    const size_t smem = (size_t)(kQ5Threads / kWave) * kPieceRounds * kWave * 16 + (size_t)K +
                        (size_t)(K / kBlock) * 4;
    const int max_waves = device_cu_count() * kWavesPerCU;
    const int waves = groups < max_waves ? groups : max_waves;
    const int wgs = (waves + kQ5Threads / kWave - 1) / (kQ5Threads / kWave);
    matvec_q50_kernel<T, R, PARTIALS, WST, false, kQ5Threads><<<dim3(wgs, M), kQ5Threads, smem, stream>>>(
        A, AS, W5, WS, C, P, N, K, M);
    return hipGetLastError();
}

template <bool PARTIALS, bool WST>
hipError_t launch_q5(const int8_t* A, const float* AS, const uint8_t* W5, const float* WS,
                     float* C, int32_t* P, int M, int N, int K, hipStream_t stream) {
    const int KB = K / kBlock;
    const int T = (KB + kWave - 1) / kWave;
    switch (T) {
#define Q8_Q5_CASE(T_) \
    case T_: return launch_q5_t<T_, PARTIALS, WST>(A, AS, W5, WS, C, P, M, N, K, stream);
        Q8_Q5_CASE(1) Q8_Q5_CASE(2) Q8_Q5_CASE(3) Q8_Q5_CASE(4)
        Q8_Q5_CASE(5) Q8_Q5_CASE(6) Q8_Q5_CASE(7) Q8_Q5_CASE(8)
#undef Q8_Q5_CASE
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool matvec_q50_fits(int K) { return K <= kQ5MaxT * kWave * kBlock; }

hipError_t launch_matvec_q50(const int8_t* A, const float* AS, const uint8_t* W5, const float* WS,
                             float* C, int32_t* P, int M, int N, int K, bool ws_t,
                             hipStream_t stream) {
    if (!matvec_q50_fits(K)) return hipErrorInvalidValue;
    if (P != nullptr) return launch_q5<true, false>(A, AS, W5, WS, C, P, M, N, K, stream);
    if (ws_t) return launch_q5<false, true>(A, AS, W5, WS, C, P, M, N, K, stream);
    return launch_q5<false, false>(A, AS, W5, WS, C, P, M, N, K, stream);
}

}  // namespace q8
