// Q8_0 matvec for small M (decode step): C[i, :] = qdot_t(A[i, :], AS[i, :], W, WS).
//
// What is computed: the qdot_t row of the Q8_0 table ("Phobos Language Spec",
// section "Quantized built-ins"); each block sum is an integer dot product
// ("Quantized built-ins and formats", section "Q8_0").  The weights come from
// HBM exactly as stored, one byte per value and one f32 scale per 32 values,
// and only the kernel turns them into products (same page, introduction).
//
// Prior art on the pages: the q8_qdot decode kernel (one activation row
// against 64 output columns per CTA, Q8_0 section) and lanes_matvec (one warp
// per row, lane-strided 4-element runs, a lane fold; "Uniform, warp-uniform
// and varying").  Design here, for CDNA4 wave64:
//   - a wave walks weight rows with a grid stride;
//   - lane l reads bytes [1024 s + 16 l, +16) of a row: each load instruction
//     covers 1 KiB of contiguous weight bytes, so W streams fully coalesced;
//   - lanes 2m and 2m+1 hold the two halves of block (1024 s)/32 + m: each
//     lane does 4 v_dot4_i32_i8, one DPP swap adds the partner's half, giving
//     the exact int32 block sum in both lanes; only the even lane scales and
//     accumulates it;
//   - the f32 accumulator is folded across the wave with DPP (no LDS).
// Two kernels share this scheme.  matvec_rows_kernel (K <= 16 KiB): one
// activation row held in VGPRs, or a batch of 2..7 rows staged once in LDS
// so that the weights are read once for all of them; row-sized buffer
// resources; one or two workgroups per compute unit.  matvec_kernel (rows
// longer than 16 KiB): one activation row per grid row, taken in 16 KiB
// chunks.  Either takes the weight scales as [N][K/32] or transposed
// ([K/32][N], the qmma_t form), which are staged through LDS.
// HBM-bound: algorithmic traffic is N*K weight bytes + N*K/8 scale bytes.
#include "q8_device.h"
#include "q8_launch.h"

namespace q8 {
namespace {

// Launch-shape knobs (compile-time; defaults are the tuned values).
#ifndef Q8_MV_THREADS
#define Q8_MV_THREADS 256
#endif
#ifndef Q8_MV_MAX_WAVES
#define Q8_MV_MAX_WAVES (256 * 32)      // short rows: about one row group per wave
#endif
#ifndef Q8_MV_MAX_WAVES_LONG
#define Q8_MV_MAX_WAVES_LONG (256 * 8)  // rows of 8+ KiB: a resident grid that walks rows
#endif
#ifndef Q8_MV_LOADS
#define Q8_MV_LOADS 4
#endif
#ifndef Q8_MV_NT
#define Q8_MV_NT 1
#endif

constexpr int kStepBytes = kWave * 16;  // one 16-byte load per lane = 1 KiB of a row
constexpr int kMatvecThreads = Q8_MV_THREADS;
constexpr int kMaxSteps = 16;           // activation row resident in VGPRs up to K = 16 KiB
constexpr int kMatvecMaxWaves = Q8_MV_MAX_WAVES;
constexpr int kMatvecMaxWavesLong = Q8_MV_MAX_WAVES_LONG;
constexpr int kLoadsInFlight = Q8_MV_LOADS;  // 16-byte weight loads per lane per row group

// WST: weight scales stored transposed, [K/32][N] (the qmma_t form).
template <int S, int R, bool PARTIALS, bool WST>
__global__ void __launch_bounds__(kMatvecThreads)
matvec_kernel(const int8_t* __restrict__ A, const float* __restrict__ AS,
              const int8_t* __restrict__ W, const float* __restrict__ WS,
              float* __restrict__ C, int32_t* __restrict__ P, int N, int K) {
    const int lane = threadIdx.x & (kWave - 1);
    const int waves_per_wg = kMatvecThreads / kWave;
    const int wave = blockIdx.x * waves_per_wg + (threadIdx.x / kWave);
    const int nwaves = gridDim.x * waves_per_wg;
    const int i = blockIdx.y;
    const int KB = K / kBlock;
    const int chunk = S * kStepBytes;
    const int nchunks = (K + chunk - 1) / chunk;
    const int groups = (N + R - 1) / R;
    const bool even = (lane & 1) == 0;
    const int8_t* Ai = A + (int64_t)i * K;

    v4i a[S];
    float as[S];
    auto load_a = [&](int c) {
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const int off = c * chunk + s * kStepBytes + lane * 16;
            const bool ok = off < K;
            a[s] = ok ? load16(Ai + off) : v4i{0, 0, 0, 0};
            if constexpr (!PARTIALS)
                as[s] = (ok && even) ? AS[(int64_t)i * KB + off / kBlock] : 0.0f;
        }
    };
    if (nchunks == 1) load_a(0);

    // Transposed weight scales: a workgroup's rows are consecutive in each
    // pass, so their scales of one block are consecutive in WS; the
    // workgroup stages them for the chunk in LDS ([block][row]) instead of
    // each lane gathering one scale per row (32 rows per load instruction).
    constexpr int kRowsWG = (kMatvecThreads / kWave) * R;
    __shared__ float ws_stage[WST ? S * (kStepBytes / kBlock) * kRowsWG : 1];

    // Every wave of a workgroup runs the same passes (the staging above
    // synchronizes the workgroup); a wave past the last row group computes
    // on masked (zero) rows and stores nothing.
    const int wg_passes = (groups + nwaves - 1) / nwaves;
    for (int pass = 0; pass < wg_passes; ++pass) {
        const int g = wave + pass * nwaves;
        if (!WST && g >= groups) break;
        const int j0 = g * R;
        float acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = 0.0f;

        for (int c = 0; c < nchunks; ++c) {
            if (nchunks > 1) load_a(c);
            // Transposed scales of this pass's rows for the chunk, loaded first
            // (consecutive threads read consecutive rows of one block).
            constexpr int kChunkBlocks = S * (kStepBytes / kBlock);
            constexpr int kStageN = kChunkBlocks * kRowsWG;
            constexpr int kStagePer = (kStageN + kMatvecThreads - 1) / kMatvecThreads;
            float wst_reg[WST ? kStagePer : 1];
            if constexpr (!PARTIALS && WST) {
                const int kb0 = c * kChunkBlocks;
                const int jw0 = (blockIdx.x * (kMatvecThreads / kWave) + pass * nwaves) * R;
#pragma unroll
                for (int t = 0; t < kStagePer; ++t) {
                    const int idx = threadIdx.x + t * kMatvecThreads;
                    const int kb = kb0 + idx / kRowsWG;
                    const int j = jw0 + idx % kRowsWG;
                    wst_reg[t] = (idx < kStageN && kb < KB && j < N) ? WS[(int64_t)kb * N + j] : 0.0f;
                }
            }
            v4i w[R][S];
            float ws[R][S];
            // Issue every load of the row group before the first use.
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int j = j0 + r;
                const bool row_ok = j < N;
                const int8_t* Wj = W + (int64_t)j * K;
#pragma unroll
                for (int s = 0; s < S; ++s) {
                    const int off = c * chunk + s * kStepBytes + lane * 16;
                    const bool ok = row_ok && off < K;
                    w[r][s] = ok ? (Q8_MV_NT ? load16_stream(Wj + off) : load16(Wj + off))
                                 : v4i{0, 0, 0, 0};
                    if constexpr (!PARTIALS && !WST)
                        ws[r][s] = ok ? WS[(int64_t)j * KB + off / kBlock] : 0.0f;
                }
            }
            if constexpr (!PARTIALS && WST) {
                // Barriers without a memory-wait on the weight loads in flight:
                // only this wave's LDS accesses must be complete.
                asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // chunk c-1 read
#pragma unroll
                for (int t = 0; t < kStagePer; ++t) {
                    const int idx = threadIdx.x + t * kMatvecThreads;
                    if (idx < kStageN) ws_stage[idx] = wst_reg[t];
                }
                asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
                const int wrow = (threadIdx.x / kWave) * R;
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int s = 0; s < S; ++s) {
                        const int kbl = (s * kStepBytes + lane * 16) / kBlock;  // block within the chunk
                        ws[r][s] = ws_stage[kbl * kRowsWG + wrow + r];
                    }
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int j = j0 + r;
#pragma unroll
                for (int s = 0; s < S; ++s) {
                    int p = dot16(a[s], w[r][s], 0);
                    p += dpp_i32<kDppSwapPairs>(p);  // exact block sum in both lanes of the pair
                    if constexpr (PARTIALS) {
                        const int off = c * chunk + s * kStepBytes + lane * 16;
                        if (even && j < N && off < K)
                            P[((int64_t)i * N + j) * KB + off / kBlock] = p;
                    } else {
                        acc[r] = fmaf(as[s] * ws[r][s], (float)p, acc[r]);
                    }
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

// ---- K <= 16 KiB: the decode kernel (one activation row, or a small batch).
// A wave walks weight rows with a grid stride.  Each row is read through a
// buffer resource built for that row alone (its base is wave-uniform, so the
// resource sits in SGPRs): a lane's offset past K, or a row past N, reads
// zero, so there are no lane masks and no 64-bit address arithmetic, and the
// whole wave fits in few VGPRs.  One activation row (MULTI false, the row is
// blockIdx.y): the lane's slice of it and of its scales stays in VGPRs.
// Several rows (MULTI, 2 <= M <= 7): the workgroup stages all of them and
// their scales in LDS once, and every 16-byte weight piece is dotted with
// the M activation pieces read back from LDS, so the weights cross the bus
// once for all rows.  Launch shape for one activation row, measured on
// MI355X: each wave has one weight row in flight; rows of up to 8 KiB run
// one 8-wave workgroup per compute unit, rows of 9..14 KiB one 4-wave
// workgroup (36..56 KiB in flight per compute unit), rows of 15 or 16 KiB
// one 8-wave workgroup.  Two rows in flight per wave (the next row's loads
// issued before the current row is computed) or eight waves on rows of
// 9..14 KiB streamed 3-4 % slower; fewer bytes in flight than this on short
// rows made the stream slower too.
// WST: weight scales stored transposed, [K/32][N] (qmma_t), staged through
// LDS per tile of rows (see below).
constexpr int kMaxBatch = 7;
// Rows per LDS tile of transposed scales (~32 KiB of scales, a whole number
// of rows per wave, at most 64), and that tile's static LDS bytes.
constexpr int wst_tile_rows(int S, int T) {
    const int rows_wg = T / kWave, kb = S * (kStepBytes / kBlock), t0 = 8192 / kb;
    return t0 < rows_wg ? rows_wg : (t0 > 64 ? 64 : t0 / rows_wg * rows_wg);
}
constexpr size_t wst_tile_bytes(int S, int T) { return (size_t)wst_tile_rows(S, T) * (S * (kStepBytes / kBlock) + 1) * 4; }
// LDS of a staged batch of M rows (S KiB each): the rows at a pitch of S
// KiB, then their scales at a pitch of S * 32 + 64 floats (whole 256-byte
// loads).
template <int S>
constexpr size_t batch_smem_bytes(int M, bool partials) {
    return (size_t)M * S * kStepBytes + (partials ? 0 : (size_t)M * (S * (kStepBytes / kBlock) + 64) * 4);
}

template <int S, bool PARTIALS, bool WST, bool MULTI, int T>
__global__ void __launch_bounds__(T)
matvec_rows_kernel(const int8_t* __restrict__ A, const float* __restrict__ AS,
                   const int8_t* __restrict__ W, const float* __restrict__ WS,
                   float* __restrict__ C, int32_t* __restrict__ P, int M, int N, int K) {
    extern __shared__ __align__(16) int8_t rows_smem[];
    const int lane = threadIdx.x & (kWave - 1);
    const int nwg = gridDim.x;
    // With WST, the workgroups of one XCD (workgroup b runs on XCD b mod 8)
    // take neighbouring row shares, so the scale lines they share stay in
    // that XCD's L2.
    const int wgx = (WST && nwg % 8 == 0) ? (blockIdx.x % 8) * (nwg / 8) + blockIdx.x / 8 : (int)blockIdx.x;
    // wave-uniform (readfirstlane), so the row resources live in SGPRs
    const int wave = __builtin_amdgcn_readfirstlane(wgx * (T / kWave) + (int)(threadIdx.x / kWave));
    const int nwaves = gridDim.x * (T / kWave);
    const int i = MULTI ? 0 : (int)blockIdx.y;
    const int KB = K / kBlock;
    const bool even = (lane & 1) == 0;
    const int lo = lane * 16;
    // MULTI: [M][S KiB] activation bytes, then [M][S * 32] f32 scales
    constexpr int kBatchPitch = S * kStepBytes;
    constexpr int kBatchSPitch = S * (kStepBytes / kBlock) + 64;  // whole 256-byte loads
    int8_t* a_lds = rows_smem;
    float* as_lds = reinterpret_cast<float*>(rows_smem + M * kBatchPitch);

    // One row: this lane's activation bytes [1024 s + 16 lane, +16) and, in
    // even lanes, the scale of their block (odd lanes hold 0: each block's
    // product is accumulated once).
    v4i a[MULTI ? 1 : S];
    float as[MULTI ? 1 : S];
    // (Offsets past the row's K bytes or K/32 scales read zero through the
    // buffer range check.)
    if constexpr (!MULTI) {
        const __amdgpu_buffer_rsrc_t rA = buffer_rsrc(A + (int64_t)i * K, K);
        const __amdgpu_buffer_rsrc_t rAS = buffer_rsrc(AS + (int64_t)i * KB, (int64_t)KB * 4);
#pragma unroll
        for (int s = 0; s < S; ++s) {
            a[s] = buffer_load16(rA, lo + s * kStepBytes, 0);
            if constexpr (!PARTIALS) {
                const float v = buffer_load_f32(rAS, (lo / kBlock) * 4 + s * kStepBytes / kBlock * 4, 0);
                as[s] = even ? v : 0.0f;
            }
        }
    }
    // Several rows: stage them (and their scales) in LDS with direct
    // global -> LDS loads (no VGPRs), 1 KiB (scales: 256 bytes) per wave
    // instruction, each row at a fixed pitch of S KiB (scales: S * 32
    // floats) so that every LDS read below is one base address plus a
    // constant; a row's bytes past K (scales past K/32) land as zeros.
    // Callers issue their first weight row before this, so it is in flight
    // meanwhile.
    auto stage_batch = [&]() {
        if constexpr (MULTI) {
            const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
            const uint32_t a_base = lds_addr(a_lds);
            for (int c = wv; c < M * S; c += T / kWave) {
                const int m = c / S, piece = c % S;
                const v4i dA = make_desc(A + (int64_t)m * K, K);
                dma16(dA, a_base + m * kBatchPitch + piece * kStepBytes, lo + piece * kStepBytes, 0);
            }
            if constexpr (!PARTIALS) {
                constexpr int kSPieces = (S * kStepBytes / kBlock * 4 + kWave * 4 - 1) / (kWave * 4);
                const uint32_t s_base = lds_addr(as_lds);
                for (int c = wv; c < M * kSPieces; c += T / kWave) {
                    const int m = c / kSPieces, piece = c % kSPieces;
                    const v4i dAS = make_desc(AS + (int64_t)m * KB, (int64_t)KB * 4);
                    dma4(dAS, s_base + m * kBatchSPitch * 4 + piece * kWave * 4, (piece * kWave + lane) * 4, 0);
                }
            }
            asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
        }
    };

    auto load_row = [&](int j, v4i (&w)[S], float (&ws)[S]) {
        const __amdgpu_buffer_rsrc_t rW = buffer_rsrc(W + (int64_t)j * K, K);
        const __amdgpu_buffer_rsrc_t rWS = buffer_rsrc(WS + (int64_t)j * KB, (int64_t)KB * 4);
#pragma unroll
        for (int s = 0; s < S; ++s) {
            w[s] = buffer_load16_nt(rW, lo + s * kStepBytes, 0);  // read once: streaming
            if constexpr (!PARTIALS && !WST)
                ws[s] = buffer_load_f32(rWS, (lo / kBlock) * 4 + s * kStepBytes / kBlock * 4, 0);
        }
    };
    auto compute_row = [&](int j, const v4i (&w)[S], const float (&ws)[S]) {
        constexpr int kM = MULTI ? kMaxBatch : 1;
#pragma unroll
        for (int m = 0; m < kM; ++m) {
            if (MULTI && m >= M) break;  // uniform
            const int row = MULTI ? m : i;
            int32_t* Prow = P + ((int64_t)row * N + j) * KB;  // (PARTIALS) this row's blocks
            float acc = 0.0f;
#pragma unroll
            for (int s = 0; s < S; ++s) {
                const int off = s * kStepBytes + lo;
                const v4i am = MULTI ? *reinterpret_cast<const v4i*>(a_lds + m * kBatchPitch + s * kStepBytes + lo) : a[s];
                int p = dot16(am, w[s], 0);
                p += dpp_i32<kDppSwapPairs>(p);  // exact block sum in both lanes of the pair
                if constexpr (PARTIALS) {
                    if (even && off < K) Prow[s * (kStepBytes / kBlock) + lane / 2] = p;
                } else {
                    const float asm_ = MULTI ? (even ? as_lds[m * kBatchSPitch + (s * kStepBytes + lo) / kBlock] : 0.0f) : as[s];
                    acc = fmaf(asm_ * ws[s], (float)p, acc);
                }
            }
            if constexpr (!PARTIALS) {
                const float tot = wave_sum(acc);
                if (lane == 0) C[(int64_t)row * N + j] = tot;
            }
            // one activation row's LDS reads at a time (else all M rows' pieces
            // would be read ahead into VGPRs)
            if constexpr (MULTI) asm volatile("" ::: "memory");
        }
    };

    if constexpr (WST) {
        // Workgroup wgx owns the rows [r_lo, r_hi) (a contiguous share) and
        // takes them in tiles of up to kTile rows.  The tile's scales of
        // every block are staged through LDS ([row][block], padded against
        // bank conflicts) by the whole workgroup from runs of WST that are
        // contiguous in the row index; each wave then takes the tile's rows
        // wv, wv + kRowsWG, ... with two rows in flight (one for rows over
        // 12 KiB).  The staging comes in two parts so that the first rows do
        // not wait for the whole tile: the scales of the first two rows of
        // every wave (the head) are requested first, then those rows, then
        // the scales of the rest of the tile, which are written to LDS after
        // each wave has finished its first two rows.  (Loads return in
        // order: a head row's data is usable once the head scales are in,
        // not the whole tile's.)  Every wave runs the same tiles and reaches
        // every barrier.  Rows past the tile's end are loaded through a
        // zero-length descriptor (no memory access), so that every wave
        // issues the same loads and each wait covers exactly the loads it
        // needs.
        constexpr int kRowsWG = T / kWave;
        constexpr int kKBMax = S * (kStepBytes / kBlock);
        constexpr int kPitch = kKBMax + 1;
        constexpr int kTile = wst_tile_rows(S, T);
        constexpr bool kTwo = S <= 12;  // two rows of 16 KiB would spill
        constexpr int kHead = kTwo ? (2 * kRowsWG < kTile ? 2 * kRowsWG : kTile) : kTile;
        constexpr int kRest = kTile - kHead;
        constexpr int kHeadPer = (kHead * kKBMax + T - 1) / T;
        constexpr int kRestPer = kRest > 0 ? (kRest * kKBMax + T - 1) / T : 1;
        static_assert(kTile % kRowsWG == 0, "a tile holds whole rounds of rows");
        __shared__ float ws_tile[kTile * kPitch];
        const __amdgpu_buffer_rsrc_t rWST = buffer_rsrc(WS, (int64_t)KB * N * 4);
        const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
        const int r_lo = (int)((int64_t)N * wgx / nwg);
        const int r_hi = (int)((int64_t)N * (wgx + 1) / nwg);
        float ws[S];
        // row j's weights, or zeros without a memory access when !valid
        auto load_row_or_zero = [&](int j, bool valid, v4i (&w)[S]) {
            const __amdgpu_buffer_rsrc_t rW = buffer_rsrc(W + (int64_t)(valid ? j : 0) * K, valid ? K : 0);
#pragma unroll
            for (int s = 0; s < S; ++s) w[s] = buffer_load16_nt(rW, lo + s * kStepBytes, 0);
        };
        stage_batch();
        for (int t0 = r_lo; t0 < r_hi; t0 += kTile) {
            const int t1 = t0 + kTile < r_hi ? t0 + kTile : r_hi;
            const int j0 = t0 + wv;
            // consecutive threads: consecutive rows of one block
            float sh[kHeadPer], sr[kRestPer];
#pragma unroll
            for (int u = 0; u < kHeadPer; ++u) {
                const int idx = threadIdx.x + u * T;
                const int b = idx / kHead, r = idx % kHead;
                sh[u] = buffer_load_f32(rWST, (b < KB && t0 + r < t1) ? (b * N + t0 + r) * 4 : kNoRead, 0);
            }
            v4i w0[S], w1[S];
            load_row_or_zero(j0, j0 < t1, w0);
            if constexpr (kTwo) load_row_or_zero(j0 + kRowsWG, j0 + kRowsWG < t1, w1);
            if constexpr (kRest > 0) {
#pragma unroll
                for (int u = 0; u < kRestPer; ++u) {
                    const int idx = threadIdx.x + u * T;
                    const int b = idx / kRest, r = kHead + idx % kRest;
                    sr[u] = buffer_load_f32(rWST, (b < KB && t0 + r < t1) ? (b * N + t0 + r) * 4 : kNoRead, 0);
                }
            }
            // the previous tile's reads of ws_tile are done (no wait on loads)
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
            for (int u = 0; u < kHeadPer; ++u) {
                const int idx = threadIdx.x + u * T;
                const int b = idx / kHead, r = idx % kHead;
                if (b < kKBMax) ws_tile[r * kPitch + b] = sh[u];
            }
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            auto tile_ws = [&](int jj) {
#pragma unroll
                for (int s = 0; s < S; ++s) ws[s] = ws_tile[(jj - t0) * kPitch + (s * kStepBytes + lo) / kBlock];
            };
            if constexpr (kTwo) {
                // the head rows; each row's compute is followed by the load
                // of the row two rounds ahead into its registers
                if (j0 < t1) { tile_ws(j0); compute_row(j0, w0, ws); }
                load_row_or_zero(j0 + 2 * kRowsWG, j0 + 2 * kRowsWG < t1, w0);
                if (j0 + kRowsWG < t1) { tile_ws(j0 + kRowsWG); compute_row(j0 + kRowsWG, w1, ws); }
                load_row_or_zero(j0 + 3 * kRowsWG, j0 + 3 * kRowsWG < t1, w1);
                if constexpr (kRest > 0) {
#pragma unroll
                    for (int u = 0; u < kRestPer; ++u) {
                        const int idx = threadIdx.x + u * T;
                        const int b = idx / kRest, r = kHead + idx % kRest;
                        if (b < kKBMax) ws_tile[r * kPitch + b] = sr[u];
                    }
                    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
                }
                for (int j = j0 + 2 * kRowsWG; j < t1; j += 2 * kRowsWG) {
                    const int j1 = j + kRowsWG;
                    tile_ws(j);
                    compute_row(j, w0, ws);
                    load_row_or_zero(j + 2 * kRowsWG, j + 2 * kRowsWG < t1, w0);
                    if (j1 >= t1) break;
                    tile_ws(j1);
                    compute_row(j1, w1, ws);
                    load_row_or_zero(j1 + 2 * kRowsWG, j1 + 2 * kRowsWG < t1, w1);
                }
            } else {
                for (int j = j0; j < t1; j += kRowsWG) {
                    if (j != j0) load_row_or_zero(j, true, w0);
                    tile_ws(j);
                    compute_row(j, w0, ws);
                }
            }
        }
    } else {
        v4i w[S];
        float ws[S];
        // A wave's rows: every nwaves-th; but for one activation row where
        // each wave has one or two rows (nwaves < N <= 2 nwaves), the two
        // neighbouring rows 2w and 2w + 1, which streams better (measured:
        // N=4096, K=4096 5.0-5.1 -> 4.73 us, K=6144 6.44 -> 6.21 us; N=3000,
        // K=4096 4.37 -> 4.30 us).  Runs of neighbouring rows were slower
        // with more rows per wave (N=14336, K=4096, eight a wave: 11.4 ->
        // 11.9 us) and in the batch form (M=4, N=14336: 14.2 -> 15.9 us).
        const bool pairs = !MULTI && N > nwaves && N <= 2 * nwaves;
        const int j0 = pairs ? 2 * wave : wave;
        const int jend = pairs ? (2 * wave + 2 < N ? 2 * wave + 2 : N) : N;
        const int step = pairs ? 1 : nwaves;
        if (j0 < jend) load_row(j0, w, ws);
        stage_batch();
        for (int j = j0; j < jend; j += step) {
            if (j != j0) load_row(j, w, ws);
            compute_row(j, w, ws);
        }
    }
}

template <int S, bool PARTIALS, bool WST, bool MULTI, int kT>
hipError_t launch_rows_t(const int8_t* A, const float* AS, const int8_t* W, const float* WS,
                         float* C, int32_t* P, int M, int N, int K, hipStream_t stream) {
    // workgroups per compute unit (one row, either scale layout: three for
    // rows of 1 KiB, two for rows of 2..3 KiB, else one; a batch: see below)
    int wpc = MULTI ? (!(WST && S > 4) ? 2 : 1) : (S == 1 ? 3 : (S <= 3 ? 2 : 1));
    auto kern = matvec_rows_kernel<S, PARTIALS, WST, MULTI, kT>;
    size_t smem = 0;
    if constexpr (MULTI) {
        smem = batch_smem_bytes<S>(M, PARTIALS);
        static std::atomic<uint64_t> lds_set{0};
        const hipError_t e = set_dynamic_lds(reinterpret_cast<const void*>(kern),
                                             (int)batch_smem_bytes<S>(kMaxBatch, PARTIALS), lds_set);
        if (e != hipSuccess) return e;
        if constexpr (!WST) {
            // As many workgroups per compute unit as registers and LDS allow,
            // up to four (32 waves); cached per batch size M.
            static std::atomic<int> occ[kMaxBatch + 1][64];
            const int n = wgs_per_cu(reinterpret_cast<const void*>(kern), kT, smem, occ[M]);
            wpc = n < 4 ? n : 4;
        }
    }
    if (MULTI && WST && wpc > 1 && (smem + wst_tile_bytes(S, kT)) * wpc > 160 * 1024) wpc = 1;
    const int cap = device_cu_count() * wpc * (kT / kWave);
    const int waves = N < cap ? N : cap;
    const int wgs = (waves + kT / kWave - 1) / (kT / kWave);
    kern<<<dim3(wgs, MULTI ? 1 : M), kT, smem, stream>>>(A, AS, W, WS, C, P, M, N, K);
    return hipGetLastError();
}

template <int S, bool PARTIALS, bool WST, bool MULTI>
hipError_t launch_rows(const int8_t* A, const float* AS, const int8_t* W, const float* WS,
                       float* C, int32_t* P, int M, int N, int K, hipStream_t stream) {
    // Launch shapes, measured on MI355X.  One row: rows of 1 KiB run three
    // 8-wave workgroups per compute unit and rows of 2..3 KiB two (N=14336:
    // K=1024 6.8 -> 4.7-5.2 us, K=2048 8.1 -> 6.9 us against one; with
    // transposed scales N=40000, K=1024 14.5 -> 9.8 us; rows this short keep
    // too few bytes in flight with eight waves); rows of 9..14
    // KiB run one 4-wave workgroup per compute unit; rows of 4..8 KiB one 7-wave
    // workgroup when seven waves per compute unit leave no more row slots
    // per compute unit than eight (N=14336, K=4096: 11.55 -> 11.3 us; at
    // N=4096 seven waves would leave some waves a third row), else one
    // 8-wave workgroup, as for shorter and longer rows.  A batch of rows
    // (more work per weight byte, so more waves to hide it): 8-wave
    // workgroups, as many per compute unit as registers and LDS allow, up
    // to four (M=4, N=14336, K=4096: 13.7 -> 13.2 us against two; M=7:
    // 19.0 -> 17.9 us; M=4, K=2048: 9.3 -> 8.4 us; one workgroup: 17.8 us
    // at M=4); with transposed scales two when their LDS fits, one on rows
    // over 4 KiB (whose scale tiles then split worse).
    if constexpr (!WST && !MULTI && S > 8 && S <= 14)
        return launch_rows_t<S, PARTIALS, WST, MULTI, 256>(A, AS, W, WS, C, P, M, N, K, stream);
    if constexpr (!WST && !MULTI && S >= 4 && S <= 8) {
        const int64_t cus = device_cu_count();
        const int64_t slots7 = ((int64_t)N + 7 * cus - 1) / (7 * cus) * 7;
        const int64_t slots8 = ((int64_t)N + 8 * cus - 1) / (8 * cus) * 8;
        if (slots7 <= slots8)
            return launch_rows_t<S, PARTIALS, WST, MULTI, 448>(A, AS, W, WS, C, P, M, N, K, stream);
    }
    return launch_rows_t<S, PARTIALS, WST, MULTI, 512>(A, AS, W, WS, C, P, M, N, K, stream);
}

template <bool PARTIALS, bool WST, bool MULTI>
hipError_t launch_rows_any(const int8_t* A, const float* AS, const int8_t* W, const float* WS,
                           float* C, int32_t* P, int M, int N, int K, hipStream_t stream) {
    switch ((K + kStepBytes - 1) / kStepBytes) {
#define Q8_ROWS_CASE(S_) \
    case S_: return launch_rows<S_, PARTIALS, WST, MULTI>(A, AS, W, WS, C, P, M, N, K, stream);
        Q8_ROWS_CASE(1) Q8_ROWS_CASE(2) Q8_ROWS_CASE(3) Q8_ROWS_CASE(4)
        Q8_ROWS_CASE(5) Q8_ROWS_CASE(6) Q8_ROWS_CASE(7) Q8_ROWS_CASE(8)
        Q8_ROWS_CASE(9) Q8_ROWS_CASE(10) Q8_ROWS_CASE(11) Q8_ROWS_CASE(12)
        Q8_ROWS_CASE(13) Q8_ROWS_CASE(14) Q8_ROWS_CASE(15) Q8_ROWS_CASE(16)
#undef Q8_ROWS_CASE
        default: return hipErrorInvalidValue;
    }
}

template <bool MULTI>
hipError_t launch_rows_mode(const int8_t* A, const float* AS, const int8_t* W, const float* WS,
                            float* C, int32_t* P, int M, int N, int K, bool ws_t, hipStream_t stream) {
    if (P != nullptr) return launch_rows_any<true, false, MULTI>(A, AS, W, WS, C, P, M, N, K, stream);
    if (ws_t) return launch_rows_any<false, true, MULTI>(A, AS, W, WS, C, P, M, N, K, stream);
    return launch_rows_any<false, false, MULTI>(A, AS, W, WS, C, P, M, N, K, stream);
}

template <int S, bool PARTIALS, bool WST>
hipError_t launch_s(const int8_t* A, const float* AS, const int8_t* W, const float* WS,
                    float* C, int32_t* P, int M, int N, int K, hipStream_t stream) {
    // Rows per wave: at least kLoadsInFlight 16-byte weight loads per lane
    // per row group (more rows only for short rows).  Measured on MI355X:
    // many light waves beat few heavy ones; long rows (K >= 8 KiB, large
    // VGPR footprint) prefer a grid that fits the chip at once.
    // With transposed weight scales, more rows per wave make the workgroup's
    // rows of one block's scales span whole cache lines (16 rows = 64 bytes).
    constexpr int R0w = kLoadsInFlight / S;
    // (launch_any caps S at 8 for them, so R = 2 stays within the VGPRs.)
    constexpr int R0 = WST ? (S <= 4 ? (R0w > 4 ? R0w : 4) : (R0w > 2 ? R0w : 2)) : R0w;
    constexpr int R = R0 >= 8 ? 8 : (R0 >= 4 ? 4 : (R0 >= 2 ? 2 : 1));
    constexpr int max_waves = S >= 8 ? kMatvecMaxWavesLong : kMatvecMaxWaves;
    if constexpr (WST && S > 8) {
        return hipErrorInvalidValue;  // never dispatched (steps capped at 8)
    } else {
        const int groups = (N + R - 1) / R;
        const int waves = groups < max_waves ? groups : max_waves;
        const int wgs = (waves + kMatvecThreads / kWave - 1) / (kMatvecThreads / kWave);
        dim3 grid(wgs, M);
        matvec_kernel<S, R, PARTIALS, WST><<<grid, kMatvecThreads, 0, stream>>>(A, AS, W, WS, C, P, N, K);
        return hipGetLastError();
    }
}

template <bool PARTIALS, bool WST>
hipError_t launch_any(const int8_t* A, const float* AS, const int8_t* W, const float* WS,
                      float* C, int32_t* P, int M, int N, int K, hipStream_t stream) {
    int steps = (K + kStepBytes - 1) / kStepBytes;
    if (steps > kMaxSteps) steps = kMaxSteps;
    if (WST && steps > 8) steps = 8;  // longer rows in chunks of 8 KiB
    switch (steps) {
#define Q8_MATVEC_CASE(S_) \
    case S_: return launch_s<S_, PARTIALS, WST>(A, AS, W, WS, C, P, M, N, K, stream);
        Q8_MATVEC_CASE(1) Q8_MATVEC_CASE(2) Q8_MATVEC_CASE(3) Q8_MATVEC_CASE(4)
        Q8_MATVEC_CASE(5) Q8_MATVEC_CASE(6) Q8_MATVEC_CASE(7) Q8_MATVEC_CASE(8)
        Q8_MATVEC_CASE(9) Q8_MATVEC_CASE(10) Q8_MATVEC_CASE(11) Q8_MATVEC_CASE(12)
        Q8_MATVEC_CASE(13) Q8_MATVEC_CASE(14) Q8_MATVEC_CASE(15) Q8_MATVEC_CASE(16)
#undef Q8_MATVEC_CASE
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_matvec(const int8_t* A, const float* AS, const int8_t* W, const float* WS,
                         float* C, int32_t* P, int M, int N, int K, bool ws_t, hipStream_t stream) {
    // K <= 16 KiB: the decode kernel, for one row or (2..7 rows) reading the
    // weights once for all of them.  Transposed scales are addressed with
    // 32-bit offsets over the whole [K/32][N] array.
    if (K <= kMaxSteps * kStepBytes && (!ws_t || (int64_t)(K / kBlock) * N * 4 < INT32_MAX)) {
        if (M == 1) return launch_rows_mode<false>(A, AS, W, WS, C, P, M, N, K, ws_t, stream);
        if (M <= kMaxBatch) return launch_rows_mode<true>(A, AS, W, WS, C, P, M, N, K, ws_t, stream);
    }
    if (P != nullptr) return launch_any<true, false>(A, AS, W, WS, C, P, M, N, K, stream);
    if (ws_t) return launch_any<false, true>(A, AS, W, WS, C, P, M, N, K, stream);
    return launch_any<false, false>(A, AS, W, WS, C, P, M, N, K, stream);
}

}  // namespace q8
