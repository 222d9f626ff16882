// Q8_0 block GEMM for few output tiles (small M, or small M x N) on CDNA4
// int8 MFMA: one workgroup per 32 x 32 output tile, the contraction split
// across the workgroup's waves.
//
// What is computed: the qdot_t row of the Q8_0 table ("Phobos Language Spec",
// section "Quantized built-ins"), C[i, j] = sum_b AS[i, b] WS[j, b] P[i, j, b],
// with P the exact int32 block sums ("Quantized built-ins and formats",
// section "Q8_0": the inner sum is taken in integers).
//
// Why this shape: with M = 64 and N = 4096 there are only 2 x 128 output
// tiles of 32 x 32, so a tile per wave leaves most SIMDs idle and makes each
// wave walk all K/32 blocks serially.  Here a workgroup of NW waves owns one
// tile and wave w takes the chunks of four Q8_0 blocks (128 k) numbered
// w, w + NW, w + 2 NW, ...  Per chunk a wave
//   - loads the tile's 32 A rows and 32 W rows, 128 contiguous bytes of each
//     (eight lanes per row, eight rows per 16-byte load instruction: the
//     MFMA operand layout itself would touch 32 rows per instruction, which
//     the memory pipeline serves about three times slower), and the 32 x 4
//     activation and weight scales (four lanes per row);
//   - writes them to its own LDS area (rows swizzled so that the fragment
//     reads are bank-conflict-free) and reads them back in MFMA layout: an
//     exchange inside one wave, ordered by the LDS queue of that wave;
//   - per block one v_mfma_i32_32x32x32_i8 (one Q8_0 block) seeded with the
//     f32 bias pattern, then the 2-op f32 epilogue of ws_pair, the
//     activation scale broadcast by DPP from one VGPR per chunk (as in the
//     staged GEMM) instead of sixteen LDS reads per block.
// Sixteen waves per workgroup (four per SIMD) while the tiles fit the
// compute units in one round; with more tiles than compute units, eight
// waves per workgroup (72 KB of LDS), so two workgroups share a compute unit
// and the second round of tiles runs beside the first (measured on MI355X,
// us, sixteen against eight waves: M=16, N=14336, K=4096 19.6 / 17.6; M=8
// 18.5 / 16.3; M=32 21.5 / 20.1; M=128, N=4096 18.6 / 16.4; M=96 18.1 /
// 15.9; M=512, N=1024 18.0 / 15.5; Q5_0 weights, M=16, N=14336 20.8 / 19.1;
// the one-round M=64, N=4096 workload within 1 % either way).  Measured on MI355X (M=64,
// N=4096, K=4096): each compute unit spends about 2 us bringing in its
// 256 KB and about 3 us in the epilogue; keeping two chunks in flight per
// wave (a VGPR double buffer, which fits once the wave index is scalar)
// measured 10.1-10.4 us against 10.2-10.7 us, eight waves with four chunks
// in flight 12.7 us, so one chunk at a time is kept.  At the end the NW
// partial tiles are summed in LDS in wave order (a fixed order: the result
// is deterministic) and stored.  Tiles sharing a W slab (the M tiles of one
// N tile) get consecutive launch slots of one XCD so the slab is read from
// HBM once.
#include "q8_device.h"
#include "q8_launch.h"

namespace q8 {
namespace {

#ifndef Q8_KS_WAVES
#define Q8_KS_WAVES 16
#endif

constexpr int kKsWaves = Q8_KS_WAVES;  // waves per workgroup (K split), one round of tiles
constexpr int kKsWavesShared = 8;      // more tiles than compute units: two workgroups per unit
constexpr int kKsBlocks = 4;           // Q8_0 blocks per chunk
constexpr int kKsSeg = kKsBlocks * kBlock;  // 128 bytes of a row per chunk

// One wave's staging area for one chunk.
struct KsStage {
    int8_t a[kTile * kKsSeg];       // [row][8 chunks of 16 B], swizzled
    int8_t w[kTile * kKsSeg];
    float as[kTile][kKsBlocks];     // [A row][block]
    float ws[kTile][kKsBlocks];     // [W row][block]
};

template <int NW>
constexpr size_t ksplit_smem_bytes() {
    // The partial tiles of the final reduction ([NW][16][64] floats) reuse
    // the staging areas once every wave is done with them.
    constexpr size_t stage = NW * sizeof(KsStage);
    constexpr size_t red = (size_t)NW * 16 * kWave * sizeof(float);
    return stage > red ? stage : red;
}

// A chunk's operands as loaded: lane l holds 16 bytes of rows 8q + l/8
// (q = 0..3), chunk l % 8, and the scales of rows l/4 and 16 + l/4,
// block l % 4.
// Q5_0 weights: lane l holds blocks (row (l + 64 h) / 4, block (l + 64 h) % 4)
// of the chunk, h = 0, 1: the qh word and the 16 nibble bytes.
struct KsRaw {
    v4i a[4], w[4];
    float as[2], ws[2];
    uint32_t qh[2];
    v4i qs[2];
};

// WST: weight scales stored transposed, [K/32][N] (the qmma_t form).
// Q5: W holds Q5_0 blocks (20 bytes per 32 values; the q50 rows of the
// Q8_0 table), decoded to signed bytes on their way into LDS.
// WNT: W rows loaded with the nontemporal bit (set when at most two M tiles
// read each W slab, so the slab is not wanted in the L2 afterwards).
template <int NW, bool PARTIALS, bool WST, bool Q5, bool WNT>
__global__ void __launch_bounds__(NW * kWave)
qgemm_ksplit_kernel(const int8_t* __restrict__ A, const float* __restrict__ AS,
                    const int8_t* __restrict__ W, const float* __restrict__ WS,
                    float* __restrict__ C, int32_t* __restrict__ P, int M, int N, int K,
                    int m_tiles, int tiles_total) {
    extern __shared__ __align__(16) int8_t ks_smem[];
    const int lane = threadIdx.x & (kWave - 1);
    // wave-uniform (readfirstlane): the chunk offsets derived from it go in
    // scalar registers (else every buffer load sits in a readfirstlane loop)
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    // The 8 XCDs take workgroups round-robin: consecutive tiles (the M tiles
    // of one N tile) go to consecutive slots of one XCD.
    int tile = blockIdx.x;
    if (tiles_total % 8 == 0) tile = (blockIdx.x % 8) * (tiles_total / 8) + blockIdx.x / 8;
    const int64_t i0 = (int64_t)(tile % m_tiles) * kTile;
    const int64_t j0 = (int64_t)(tile / m_tiles) * kTile;
    const int KB = K / kBlock;
    KsStage& st = reinterpret_cast<KsStage*>(ks_smem)[wv];

    // ---- load-side lane roles.  Raw buffer loads: rows past M or N fall
    // outside the resource and read as zero; the row part of every offset is
    // in the per-lane offset, the chunk's k offset in the scalar one.
    const int lrow = lane / 8;   // row within an 8-row load group
    const int lch = lane % 8;    // 16-byte chunk of the 128-byte segment
    const int srow = lane / 4;   // scale row (and 16 + srow)
    const int sblk = lane % 4;   // scale block within the chunk
    const int rows_a = M - i0 < kTile ? (int)(M - i0) : kTile;
    const int rows_w = N - j0 < kTile ? (int)(N - j0) : kTile;
    const __amdgpu_buffer_rsrc_t rA = buffer_rsrc(A + i0 * K, (int64_t)rows_a * K);
    const __amdgpu_buffer_rsrc_t rW = buffer_rsrc(Q5 ? W : W + j0 * K, Q5 ? 0 : (int64_t)rows_w * K);
    // (the debug entry passes no scales and reads none)
    const __amdgpu_buffer_rsrc_t rAS = buffer_rsrc(PARTIALS ? nullptr : AS + i0 * KB, (int64_t)rows_a * KB * 4);
    // Weight scales [N][K/32]: this tile's rows.  Transposed [K/32][N]: from
    // column j0 to the end of the array (columns past the tile belong to
    // other tiles or the next block row; they meet zero weights and are
    // never stored).
    const __amdgpu_buffer_rsrc_t rWS =
        buffer_rsrc(PARTIALS ? nullptr : WS + (WST ? j0 : j0 * KB),
                    WST ? ((int64_t)KB * N - j0) * 4 : (int64_t)rows_w * KB * 4);
    const int voff_ops = lrow * K + 16 * lch;             // + 8 q K for group q
    const int voff_sc = (srow * KB + sblk) * 4;           // + 16 k KB * 4 for half k
    const int voff_wst = (sblk * N + srow) * 4;           // + (kb0 N + 16 k) * 4

    // ---- MFMA-side lane roles
    const int half = lane / 32;
    const int r32 = lane & 31;
    const int as_row = tile_row(lane % 16, half);  // activation row whose scales this lane holds
    int frag_off[kKsBlocks];  // logical chunk 2 t + half of row r32
#pragma unroll
    for (int t = 0; t < kKsBlocks; ++t) frag_off[t] = r32 * kKsSeg + 16 * ((2 * t + half) ^ swz(r32));

    auto load_chunk = [&](KsRaw& raw, int c) {
        const int kb0 = c * kKsBlocks;
        // a lane whose 16 bytes lie past K reads nothing (zeros)
        const int vo = (kb0 + lch / 2 < KB) ? voff_ops : kNoRead;
        const int so = kb0 * kBlock;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int v = vo == kNoRead ? kNoRead : vo + 8 * q * K;
            raw.a[q] = buffer_load16(rA, v, so);
            if constexpr (!Q5) raw.w[q] = WNT ? buffer_load16_nt(rW, v, so) : buffer_load16(rW, v, so);
        }
        if constexpr (Q5) {
            // whole blocks per lane; rows past N and blocks past K load
            // nothing (their values meet no stored output / are skipped)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int idx = lane + kWave * h;
                const int64_t j = j0 + idx / 4;
                const int b = kb0 + idx % 4;
                const bool ok = j < N && b < KB;
                const int8_t* blk = W + (ok ? j * KB * 20 + (int64_t)b * 20 : 0);
                raw.qh[h] = ok ? *reinterpret_cast<const uint32_t*>(blk) : 0u;
                raw.qs[h] = ok ? load16_a4(blk + 4) : v4i{0, 0, 0, 0};
            }
        }
        if constexpr (!PARTIALS) {
            const bool blk_ok = kb0 + sblk < KB;
            const int vs = blk_ok ? voff_sc : kNoRead;
            // transposed: the whole offset in the range-checked lane offset
            const int vt = blk_ok ? voff_wst + kb0 * N * 4 : kNoRead;
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int v = vs == kNoRead ? kNoRead : vs + 16 * k * KB * 4;
                raw.as[k] = buffer_load_f32(rAS, v, kb0 * 4);
                if constexpr (WST)
                    raw.ws[k] = buffer_load_f32(rWS, vt == kNoRead ? kNoRead : vt + 16 * k * 4, 0);
                else
                    raw.ws[k] = buffer_load_f32(rWS, v, kb0 * 4);
            }
        }
    };

    // One seed for both modes: the debug entry issues the f32 path's MFMAs
    // and stores D - kBias, the exact block sum.
    v16i bias;
#pragma unroll
    for (int r = 0; r < 16; ++r) bias[r] = kBias;
    asm volatile("" : "+v"(bias));

    float acc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;

    // exact: the plain-order epilogue acc += (AS * WS) * p, taken when the
    // fast form's result is not finite (see below).
    auto stage_and_compute = [&](const KsRaw& raw, int c, bool exact) {
        // Lanes exchange data through this wave's LDS area: keep the compiler
        // from moving LDS accesses across the write/read boundaries (the LDS
        // queue itself serves one wave's accesses in order).
        asm volatile("" ::: "memory");
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int row = 8 * q + lrow;
            const int off = row * kKsSeg + 16 * (lch ^ swz(row));
            *reinterpret_cast<v4i*>(st.a + off) = raw.a[q];
            if constexpr (!Q5) *reinterpret_cast<v4i*>(st.w + off) = raw.w[q];
        }
        if constexpr (Q5) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int idx = lane + kWave * h;
                const int row = idx / 4, blk = idx % 4;
                uint32_t v[8];
                q50_values(raw.qh[h], raw.qs[h], v);
                // logical chunks 2 blk (values 0..15) and 2 blk + 1 (16..31)
                *reinterpret_cast<v4i*>(st.w + row * kKsSeg + 16 * ((2 * blk) ^ swz(row))) =
                    v4i{(int)v[0], (int)v[1], (int)v[2], (int)v[3]};
                *reinterpret_cast<v4i*>(st.w + row * kKsSeg + 16 * ((2 * blk + 1) ^ swz(row))) =
                    v4i{(int)v[4], (int)v[5], (int)v[6], (int)v[7]};
            }
        }
        if constexpr (!PARTIALS) {
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                st.as[16 * k + srow][sblk] = raw.as[k];
                st.ws[16 * k + srow][sblk] = raw.ws[k];
            }
        }
        asm volatile("" ::: "memory");
        const int kb0 = c * kKsBlocks;
        float4 ws4 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        float4 as4 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if constexpr (!PARTIALS) {
            ws4 = *reinterpret_cast<const float4*>(&st.ws[r32][0]);
            // the chunk's four scales of the activation row this lane serves
            // to its 16-lane row (see fmac_rowbcast8)
            as4 = *reinterpret_cast<const float4*>(&st.as[as_row][0]);
        }
        const float wsv[4] = {ws4.x, ws4.y, ws4.z, ws4.w};
        const float asv[4] = {as4.x, as4.y, as4.z, as4.w};
#pragma unroll
        for (int t = 0; t < kKsBlocks; ++t) {
            const int b = kb0 + t;
            if (b >= KB) continue;  // wave-uniform
            const v4i af = *reinterpret_cast<const v4i*>(st.a + frag_off[t]);
            const v4i wf = *reinterpret_cast<const v4i*>(st.w + frag_off[t]);
            const v16i d = __builtin_amdgcn_mfma_i32_32x32x32_i8(af, wf, bias, 0, 0, 0);
            if constexpr (PARTIALS) {
                const int64_t j = j0 + r32;
                if (j < N) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int64_t i = i0 + tile_row(r, half);
                        if (i < M) P[(i * N + j) * KB + b] = d[r] - kBias;
                    }
                }
            } else if (!exact) {
                // acc[r] += AS[row r] * round(ws_hi * p[r]), the activation
                // scale broadcast from lane r of the 16-lane row (DPP)
                const float2 wp = ws_pair(wsv[t]);
                float u[16];
#pragma unroll
                for (int r = 0; r < 8; ++r) u[r] = fmaf(wp.x, __int_as_float(d[r]), wp.y);
                fmac_rowbcast8<0>(acc, asv[t], u);
#pragma unroll
                for (int r = 8; r < 16; ++r) u[r] = fmaf(wp.x, __int_as_float(d[r]), wp.y);
                fmac_rowbcast8<8>(acc, asv[t], u);
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[r] = fmaf(st.as[tile_row(r, half)][t] * wsv[t], (float)(d[r] - kBias), acc[r]);
            }
        }
    };

    const int nchunks = (KB + kKsBlocks - 1) / kKsBlocks;
    // Wave w takes chunks w, w + NW, w + 2 NW, ...: at any moment the waves
    // of a workgroup read consecutive 128-byte segments of their rows
    // (measured against contiguous ranges per wave: M=32, N=4096, K=14336
    // 35.1 -> 30.6 us, M=127, N=300, K=4160 11.9 -> 10.5 us, the M=64,
    // N=4096, K=4096 workload unchanged within noise).
    const int n_mine = wv < nchunks ? (nchunks - wv + NW - 1) / NW : 0;
    auto chunk_of = [&](int n) { return wv + NW * n; };
    for (int n = 0; n < n_mine; ++n) {
        KsRaw r0;
        load_chunk(r0, chunk_of(n));
        stage_and_compute(r0, chunk_of(n), false);
    }
    if constexpr (!PARTIALS) {
        // The fast epilogue's bias product -12582912 ws is finite for |WS|
        // below about 2^104, and it forms ws * p before the activation scale:
        // a wave whose partial tile came out non-finite recomputes its chunks
        // in the plain order (AS * WS) * p (finite wherever AS * WS and the
        // sums are).
        bool bad = false;
#pragma unroll
        for (int r = 0; r < 16; ++r) bad |= !__builtin_isfinite(acc[r]);
        if (__builtin_amdgcn_ballot_w64(bad) != 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
            for (int n = 0; n < n_mine; ++n) {
                KsRaw r0;
                load_chunk(r0, chunk_of(n));
                stage_and_compute(r0, chunk_of(n), true);
            }
        }
    }

    if constexpr (!PARTIALS) {
        // Sum the NW partial tiles in wave order and store the tile.
        float* red = reinterpret_cast<float*>(ks_smem);  // [NW][16][64], over the stages
        __syncthreads();  // every wave is done with its staging area
#pragma unroll
        for (int r = 0; r < 16; ++r) red[(wv * 16 + r) * kWave + lane] = acc[r];
        __syncthreads();
        for (int o = threadIdx.x; o < 16 * kWave; o += NW * kWave) {
            float s = 0.0f;
#pragma unroll
            for (int w = 0; w < NW; ++w) s += red[w * 16 * kWave + o];
            const int r = o / kWave;
            const int l = o % kWave;
            const int64_t i = i0 + tile_row(r, l / 32);
            const int64_t j = j0 + (l & 31);
            if (i < M && j < N) C[i * N + j] = s;
        }
    }
}

template <int NW, bool PARTIALS, bool WST, bool Q5>
hipError_t launch_ks(const int8_t* A, const float* AS, const int8_t* W, const float* WS,
                     float* C, int32_t* P, int M, int N, int K, hipStream_t stream) {
    const int64_t m_tiles = (M + kTile - 1) / kTile;
    const int64_t n_tiles = (N + kTile - 1) / kTile;
    const int64_t total = m_tiles * n_tiles;
    if (total > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    constexpr size_t smem = ksplit_smem_bytes<NW>();
    static_assert(smem <= 160 * 1024, "LDS budget");
    // Q8_0 W rows stream with the nontemporal bit when at most two M tiles
    // (which run side by side on one XCD) read each W slab, measured on
    // MI355X: M=16, N=14336, K=4096 21.2 -> 18.9 us; M=64, N=4096: 10.9 ->
    // 10.5 us; with four M tiles it lost (M=127, N=300: 11.3 -> 12.9 us).
    bool wnt = false;
    auto kern = qgemm_ksplit_kernel<NW, PARTIALS, WST, Q5, false>;
    if constexpr (!Q5) {
        if (m_tiles <= 2) {
            wnt = true;
            kern = qgemm_ksplit_kernel<NW, PARTIALS, WST, Q5, true>;
        }
    }
    if (smem > 64 * 1024) {
        static std::atomic<uint64_t> lds_set[2] = {{0}, {0}};
        const hipError_t e = set_dynamic_lds(reinterpret_cast<const void*>(kern), (int)smem, lds_set[wnt]);
        if (e != hipSuccess) return e;
    }
    kern<<<dim3((unsigned)total), NW * kWave, smem, stream>>>(A, AS, W, WS, C, P, M, N, K,
                                                             (int)m_tiles, (int)total);
    return hipGetLastError();
}

// Waves per workgroup for a shape: kKsWaves while its 32 x 32 tiles fit the
// compute units in one round, else kKsWavesShared (two workgroups per unit).
template <bool Q5>
hipError_t launch_ks_any(const int8_t* A, const float* AS, const int8_t* W, const float* WS,
                         float* C, int32_t* P, int M, int N, int K, bool ws_t, hipStream_t stream) {
    const int64_t tiles = ((int64_t)M + kTile - 1) / kTile * (((int64_t)N + kTile - 1) / kTile);
    if (tiles > device_cu_count()) {
        if (P != nullptr) return launch_ks<kKsWavesShared, true, false, Q5>(A, AS, W, WS, C, P, M, N, K, stream);
        if (ws_t) return launch_ks<kKsWavesShared, false, true, Q5>(A, AS, W, WS, C, P, M, N, K, stream);
        return launch_ks<kKsWavesShared, false, false, Q5>(A, AS, W, WS, C, P, M, N, K, stream);
    }
    if (P != nullptr) return launch_ks<kKsWaves, true, false, Q5>(A, AS, W, WS, C, P, M, N, K, stream);
    if (ws_t) return launch_ks<kKsWaves, false, true, Q5>(A, AS, W, WS, C, P, M, N, K, stream);
    return launch_ks<kKsWaves, false, false, Q5>(A, AS, W, WS, C, P, M, N, K, stream);
}

}  // namespace

hipError_t launch_qgemm_ksplit(const int8_t* A, const float* AS, const int8_t* W, const float* WS,
                               float* C, int32_t* P, int M, int N, int K, bool ws_t,
                               hipStream_t stream) {
    return launch_ks_any<false>(A, AS, W, WS, C, P, M, N, K, ws_t, stream);
}

hipError_t launch_qgemm_ksplit_q50(const int8_t* A, const float* AS, const uint8_t* W5,
                                   const float* WS, float* C, int32_t* P, int M, int N, int K,
                                   bool ws_t, hipStream_t stream) {
    return launch_ks_any<true>(A, AS, reinterpret_cast<const int8_t*>(W5), WS, C, P, M, N, K, ws_t, stream);
}

}  // namespace q8
