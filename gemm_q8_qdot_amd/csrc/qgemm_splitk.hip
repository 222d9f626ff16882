// Q8_0 block GEMM for few output tiles with the contraction split across
// workgroups (prompt projections with small M), on CDNA4 int8 MFMA.
//
// What is computed: the qdot_t row of the Q8_0 table ("Phobos Language Spec",
// section "Quantized built-ins"), or qmma_t with the weight scales stored
// [K/32][N] (same table): C[i, j] = sum_b AS[i, b] WS[j, b] P[i, j, b], with
// P the exact int32 block sums ("Quantized built-ins and formats", section
// "Q8_0": the inner sum is taken in integers).
//
// Why: with a long contraction and few output tiles (M = 32, N = 4096,
// K = 14336: 128 tiles of 32 x 32) the one-tile-per-workgroup GEMM walks
// all of K in each workgroup, bringing in its 32 activation rows and 32
// weight rows over the whole of K (900 KB per compute unit here), and the
// per-unit ingest and the f32 epilogue run one after the other.  Here a
// workgroup owns a 64 x 64 output tile and one of S contiguous slices of the
// K/32 blocks (S chosen on the host so that there are about as many
// workgroups as compute units): per slice it brings in 64 activation rows
// and 64 weight rows of its k range only.  The split costs about 4 us of
// fixed reduction work, so it is taken for K >= 8192 only (see splitk_plan).
// With one slice (S = 1: no workspace, each workgroup stores its tile) the
// same kernel also serves the plain entries for medium shapes whose 32 x 32
// tiles would take the one-tile GEMM several rounds of workgroups (see
// splitk_whole_k).
//
//   - Staging: stages of 8 blocks (256 k); a 4-stage ring in LDS (36 KB a
//     stage) filled by direct global->LDS loads, three stages ahead.  Each
//     stage is 48 wave-wide load instructions (16 for the activation rows,
//     16 for the weight rows, 8 + 8 for the scales), three per wave, so every
//     wave waits for the same number of loads.  Row segments are stored with
//     their 16-byte chunks permuted (chunk c of row r at c ^ (r mod 16)) so
//     that the MFMA fragment reads are free of bank conflicts; the
//     permutation is applied by choosing which global chunk each lane loads.
//   - Math: 16 waves; wave w computes the 32 x 32 sub-tile w mod 4 on blocks
//     2 (w / 4) and 2 (w / 4) + 1 of every stage: one v_mfma_i32_32x32x32_i8
//     per block (one Q8_0 block), seeded with the f32 bias pattern, and the
//     2-operation epilogue of ws_pair with the activation scale broadcast by
//     DPP (see qgemm.hip).
//   - Reduction: the four waves of a sub-tile are summed in LDS in wave
//     order.  With S > 1 each workgroup writes its 64 x 64 partial tile to
//     the workspace, and the last of the tile's S workgroups to finish (an
//     atomic counter per tile) adds the S partial tiles in slice order
//     (0, 1, ..., S - 1, so the result does not depend on which finished
//     last) and stores C; it then resets the counter, so the workspace is
//     left zero-filled for the next call.
//   - The debug entry runs the same loads and MFMAs and stores each block
//     sum (D - bias) where the epilogue would run; it needs no workspace.
#include "q8_device.h"
#include "q8_launch.h"

namespace q8 {
namespace {

constexpr int kSkM = 64;                          // activation rows per tile
constexpr int kSkN = 64;                          // weight rows per tile
constexpr int kSkSB = 8;                          // Q8_0 blocks per stage
constexpr int kSkSeg = kSkSB * kBlock;            // 256 bytes of a row per stage
constexpr int kSkRing = 4;                        // stages in LDS
constexpr int kSkWaves = 16;
constexpr int kSkThreads = kSkWaves * kWave;
constexpr int kSkTileFloats = kSkM * kSkN;        // one partial tile
// Workspace layout: one 32-bit counter per output tile in a fixed area at
// the start (so that calls of any shape sharing a workspace find their
// counters at zero), then the partial tiles.
constexpr int kSkMaxTiles = 1024;
constexpr size_t kSkCounterBytes = kSkMaxTiles * sizeof(unsigned);

struct SkStage {
    int8_t a[kSkM * kSkSeg];          // [row][16 chunks of 16 B], permuted
    int8_t w[kSkN * kSkSeg];
    float as[kSkM * kSkSB];           // [row][block]
    float ws[kSkN * kSkSB];           // [row][block]; transposed scales: [block][column]
};
static_assert(sizeof(SkStage) == 36864, "stage layout");
constexpr size_t kSkSmem = sizeof(SkStage) * kSkRing;
static_assert(kSkSmem <= 160 * 1024, "LDS budget");
static_assert((size_t)kSkWaves * 16 * kWave * sizeof(float) <= kSkSmem, "reduction area");

// WST: weight scales stored [K/32][N] (qmma_t).  S > 1: cnt (one counter per
// tile) and part (tiles x S partial tiles) are the workspace; cnt_clear (or
// null) is a counter area this kernel zero-fills for a later call.
template <bool PARTIALS, bool WST>
__global__ void __launch_bounds__(kSkThreads, 1)
qgemm_splitk_kernel(const int8_t* __restrict__ A, const float* __restrict__ AS,
                    const int8_t* __restrict__ W, const float* __restrict__ WS,
                    float* __restrict__ C, int32_t* __restrict__ P, int M, int N, int K,
                    int tiles_m, int S, int slice_blocks, float* __restrict__ part,
                    unsigned* __restrict__ cnt, unsigned* __restrict__ cnt_clear) {
    extern __shared__ __align__(16) unsigned char sk_smem[];
    // The no-allocation entry's next call counts in the other counter area:
    // zero it now (this call does not use it).
    if (cnt_clear != nullptr && threadIdx.x < kWave) {
        for (int k = blockIdx.x * kWave + threadIdx.x; k < kSkMaxTiles; k += gridDim.x * kWave)
            __hip_atomic_store(&cnt_clear[k], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    SkStage* ring = reinterpret_cast<SkStage*>(sk_smem);
    __shared__ int last_flag;

    // The 8 XCDs take workgroups round-robin: consecutive ids (the S slices
    // of one tile, then the neighbouring tiles) go to one XCD.
    const int total = (int)gridDim.x;
    int id = blockIdx.x;
    if (total % 8 == 0) id = (blockIdx.x % 8) * (total / 8) + blockIdx.x / 8;
    const int tile = id / S;
    const int slice = id % S;
    const int i0 = (tile % tiles_m) * kSkM;
    const int j0 = (tile / tiles_m) * kSkN;
    const int KB = K / kBlock;
    const int kb_lo = slice * slice_blocks;
    const int kb_hi = min(KB, kb_lo + slice_blocks);
    const int nst = (kb_hi - kb_lo + kSkSB - 1) / kSkSB;

    const int lane = threadIdx.x & (kWave - 1);
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    const int half = lane / 32;
    const int col = lane & 31;
    const int rows_a = min(M - i0, kSkM);
    const int rows_w = min(N - j0, kSkN);

    // Descriptors of this tile's rows: reads past them return 0.
    const v4i dA = make_desc(A + (int64_t)i0 * K, (int64_t)rows_a * K);
    const v4i dW = make_desc(W + (int64_t)j0 * K, (int64_t)rows_w * K);
    const v4i dAS = make_desc(PARTIALS ? nullptr : AS + (int64_t)i0 * KB, (int64_t)rows_a * KB * 4);
    // Transposed weight scales: from column j0 to the end of the array
    // (columns past the tile meet zero weight rows and are never stored).
    const v4i dWS = make_desc(PARTIALS ? nullptr : WS + (WST ? (int64_t)j0 : (int64_t)j0 * KB),
                              WST ? ((int64_t)KB * N - j0) * 4 : (int64_t)rows_w * KB * 4);

    // Load jobs of stage st (three per wave).  Operand job q (wave q): rows
    // 4q .. 4q + 3; lane l fills physical chunk l % 16 of row 4q + l / 16,
    // i.e. loads logical chunk (l % 16) ^ (row % 16).  Scale job e: rows
    // 8e .. 8e + 7, block l % 8 of row 8e + l / 8 ([row][block]); transposed
    // weight scales: block e, column l ([block][column]).  A chunk or block
    // past the slice (or past K) reads nothing and lands as zeros; so does a
    // stage past the last one (its ring slot is not read again).
    const int op_row = 4 * wv + lane / 16;
    const int op_chunk = (lane % 16) ^ (op_row & 15);
    const int op_voff = op_row * K + 16 * op_chunk;
    const int sc_row = 8 * (wv & 7) + lane / 8;
    const int sc_blk = lane % 8;
    auto issue_stage = [&](int st) {
        SkStage& sg = ring[st % kSkRing];
        const int kbs = kb_lo + st * kSkSB;  // first block of the stage
        const bool in = st < nst;
        const int vo = (in && kbs + op_chunk / 2 < kb_hi) ? op_voff : kNoRead;
        dma16(dA, lds_addr(&sg.a[wv * 4 * kSkSeg]), vo, kbs * kBlock);
        dma16(dW, lds_addr(&sg.w[wv * 4 * kSkSeg]), vo, kbs * kBlock);
        if (wv < 8) {
            const bool ok = !PARTIALS && in && kbs + sc_blk < kb_hi;
            dma4(dAS, lds_addr(&sg.as[wv * kWave]), ok ? (sc_row * KB + kbs + sc_blk) * 4 : kNoRead, 0);
        } else if constexpr (WST) {
            const int e = wv - 8;
            const bool ok = !PARTIALS && in && kbs + e < kb_hi;
            dma4(dWS, lds_addr(&sg.ws[e * kWave]), ok ? ((kbs + e) * N + lane) * 4 : kNoRead, 0);
        } else {
            const bool ok = !PARTIALS && in && kbs + sc_blk < kb_hi;
            dma4(dWS, lds_addr(&sg.ws[(wv - 8) * kWave]), ok ? (sc_row * KB + kbs + sc_blk) * 4 : kNoRead, 0);
        }
    };

    // MFMA-side roles: sub-tile (sm, sn) of 32 x 32, blocks 2 kq, 2 kq + 1
    // of each stage.
    const int sub = wv & 3;
    const int sm = sub >> 1, sn = sub & 1;
    const int kq = wv >> 2;
    const int a_row = kSkM / 2 * sm + col;
    const int w_row = kSkN / 2 * sn + col;
    const int as_row = kSkM / 2 * sm + tile_row(lane % 16, half);  // row this lane serves by DPP
    int frag_a[2], frag_w[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int c = 2 * (2 * kq + t) + half;  // logical chunk of block 2 kq + t
        frag_a[t] = a_row * kSkSeg + 16 * (c ^ (a_row & 15));
        frag_w[t] = w_row * kSkSeg + 16 * (c ^ (w_row & 15));
    }

    v16i bias;
#pragma unroll
    for (int r = 0; r < 16; ++r) bias[r] = kBias;
    asm volatile("" : "+v"(bias));
    float acc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;

    auto compute_stage = [&](int st) {
        const SkStage& sg = ring[st % kSkRing];
        const int kbs = kb_lo + st * kSkSB + 2 * kq;
        float2 ws2 = make_float2(0.0f, 0.0f), as2 = make_float2(0.0f, 0.0f);
        if constexpr (!PARTIALS) {
            as2 = *reinterpret_cast<const float2*>(&sg.as[as_row * kSkSB + 2 * kq]);
            if constexpr (WST) ws2 = make_float2(sg.ws[(2 * kq) * kSkN + w_row], sg.ws[(2 * kq + 1) * kSkN + w_row]);
            else ws2 = *reinterpret_cast<const float2*>(&sg.ws[w_row * kSkSB + 2 * kq]);
        }
        const float wsv[2] = {ws2.x, ws2.y};
        const float asv[2] = {as2.x, as2.y};
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int b = kbs + t;
            if (b >= kb_hi) break;  // wave-uniform
            const v4i af = *reinterpret_cast<const v4i*>(sg.a + frag_a[t]);
            const v4i wf = *reinterpret_cast<const v4i*>(sg.w + frag_w[t]);
            const v16i d = __builtin_amdgcn_mfma_i32_32x32x32_i8(af, wf, bias, 0, 0, 0);
            if constexpr (PARTIALS) {
                const int j = j0 + w_row;
                if (j < N) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int i = i0 + kSkM / 2 * sm + tile_row(r, half);
                        if (i < M) P[((int64_t)i * N + j) * KB + b] = d[r] - kBias;
                    }
                }
            } else {
                const float2 wp = ws_pair(wsv[t]);
                float u[16];
#pragma unroll
                for (int r = 0; r < 8; ++r) u[r] = fmaf(wp.x, __int_as_float(d[r]), wp.y);
                fmac_rowbcast8<0>(acc, asv[t], u);
#pragma unroll
                for (int r = 8; r < 16; ++r) u[r] = fmaf(wp.x, __int_as_float(d[r]), wp.y);
                fmac_rowbcast8<8>(acc, asv[t], u);
            }
        }
    };

    // Prologue: the whole ring in flight.  In iteration st, once the wave's
    // own loads of stage st have landed and every wave has passed the
    // barrier (so all of stage st is in LDS and stage st - 1 is no longer
    // read), the slot of stage st - 1 is refilled with stage st - 1 + 4.
    // Loads complete in order: stage st has landed once at most the loads of
    // the stages issued after it (three per stage) are outstanding.
#pragma unroll
    for (int st = 0; st < kSkRing; ++st) issue_stage(st);
    for (int st = 0; st < nst; ++st) {
        if (st == 0) asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        if (st > 0) issue_stage(st - 1 + kSkRing);
        compute_stage(st);
    }
    // Every load (the ring's trailing stages included) has landed before
    // the LDS is used for the reduction.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if constexpr (PARTIALS) return;

    // The fast epilogue's bias product -12582912 ws is finite for |WS| below
    // about 2^104, and it forms ws * p before the activation scale: a wave
    // whose result came out non-finite recomputes its blocks in the plain
    // order (AS * WS) * p, straight from memory (no barriers).
    bool bad = false;
#pragma unroll
    for (int r = 0; r < 16; ++r) bad |= !__builtin_isfinite(acc[r]);
    if (__builtin_amdgcn_ballot_w64(bad) != 0) {
        const v16i zero = {};
        const int ia = i0 + a_row, jw = j0 + w_row;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
        for (int st = 0; st < nst; ++st) {
            for (int t = 0; t < 2; ++t) {
                const int b = kb_lo + st * kSkSB + 2 * kq + t;
                if (b >= kb_hi) break;
                const int ko = b * kBlock + 16 * half;
                const v4i af = ia < M ? load16(A + (int64_t)ia * K + ko) : v4i{0, 0, 0, 0};
                const v4i wf = jw < N ? load16(W + (int64_t)jw * K + ko) : v4i{0, 0, 0, 0};
                const v16i d = __builtin_amdgcn_mfma_i32_32x32x32_i8(af, wf, zero, 0, 0, 0);
                const float ws = jw < N ? (WST ? WS[(int64_t)b * N + jw] : WS[(int64_t)jw * KB + b]) : 0.0f;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int ir = i0 + kSkM / 2 * sm + tile_row(r, half);
                    const float as = ir < M ? AS[(int64_t)ir * KB + b] : 0.0f;
                    acc[r] = fmaf(as * ws, (float)d[r], acc[r]);
                }
            }
        }
    }

    // The four waves of each sub-tile, summed in wave order (kq = 0..3).
    float* red = reinterpret_cast<float*>(sk_smem);  // [16 waves][16][64]
#pragma unroll
    for (int r = 0; r < 16; ++r) red[(wv * 16 + r) * kWave + lane] = acc[r];
    __syncthreads();
    float tot[16];
    if (wv < 4) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float s = red[(wv * 16 + r) * kWave + lane];
            s += red[((wv + 4) * 16 + r) * kWave + lane];
            s += red[((wv + 8) * 16 + r) * kWave + lane];
            s += red[((wv + 12) * 16 + r) * kWave + lane];
            tot[r] = s;
        }
    }
    auto store_c = [&](const float (&v)[16]) {
        const int j = j0 + w_row;
        if (j < N) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = i0 + kSkM / 2 * sm + tile_row(r, half);
                if (i < M) C[(int64_t)i * N + j] = v[r];
            }
        }
    };
    if (S == 1) {
        if (wv < 4) store_c(tot);
        return;
    }

    // Split: publish this slice's partial tile; the tile's last workgroup
    // adds the S partial tiles in slice order.  The partial tiles and the
    // counters are accessed with device-coherent (agent-scope) loads and
    // stores, which bypass the per-XCD caches, instead of agent-scope
    // fences (an L2 write-back and invalidate per workgroup, which cost
    // more than the whole contraction here).  Each workgroup waits until
    // its partial-tile stores have completed before it increments the
    // counter, and the last one reads the partial tiles only after its
    // increment has returned S - 1, so it finds all of them in memory.
    float* mine = part + ((int64_t)tile * S + slice) * kSkTileFloats;
    if (wv < 4) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
            __hip_atomic_store(&mine[(wv * 16 + r) * kWave + lane], tot[r], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned prev = __hip_atomic_fetch_add(&cnt[tile], 1u, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT);
        last_flag = prev == (unsigned)(S - 1);
    }
    __syncthreads();
    if (!last_flag) return;
    if (wv < 4) {
        float sum[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) sum[r] = 0.0f;
        for (int s = 0; s < S; ++s) {
            const float* src = part + ((int64_t)tile * S + s) * kSkTileFloats;
#pragma unroll
            for (int r = 0; r < 16; ++r)
                sum[r] += s == slice ? tot[r]
                                     : __hip_atomic_load(&src[(wv * 16 + r) * kWave + lane],
                                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        store_c(sum);
    }
    if (threadIdx.x == 0) __hip_atomic_store(&cnt[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

bool splitk_plan(int M, int N, int K, int* S_out, int* slice_blocks_out, size_t* ws_bytes) {
    const int KB = K / kBlock;
    // Long contractions only: the split adds a fixed cost (an LDS reduction
    // of four waves, the partial tile written and read back through the
    // device-coherent level, the counter), about 4 us, against the one-tile
    // GEMM's serial walk over K.  Measured on MI355X (us, one-tile GEMM
    // against split): M=64, N=4096, K=4096: 10.7 / 14.5; K=8192: 20.1 /
    // 18.6; K=14336: 34.0 / 26.5; M=32, N=2048, K=14336: 33.4 / 19.6; M=8,
    // N=4096, K=4096: 9.0 / 13.8.
    if (M < 8 || KB < 256 || (int64_t)K * kSkM > INT32_MAX) return false;
    const int64_t tiles_m = ((int64_t)M + kSkM - 1) / kSkM;
    const int64_t tiles_n = ((int64_t)N + kSkN - 1) / kSkN;
    const int64_t tiles = tiles_m * tiles_n;
    const int cus = device_cu_count();
    // Only where the tiles alone cannot fill the chip: about one workgroup
    // per compute unit, slices of at least two stages.
    if (tiles >= cus || tiles > kSkMaxTiles) return false;
    int64_t S = cus / tiles;
    const int64_t max_s = (KB + 2 * kSkSB - 1) / (2 * kSkSB);
    if (S > max_s) S = max_s;
    if (S > 64) S = 64;
    if (S < 2) return false;
    int sb = (int)((KB + S - 1) / S);
    sb = (sb + kSkSB - 1) / kSkSB * kSkSB;
    S = (KB + sb - 1) / sb;
    if (S < 2) return false;
    *S_out = (int)S;
    *slice_blocks_out = sb;
    *ws_bytes = kSkCounterBytes + (size_t)tiles * S * kSkTileFloats * sizeof(float);
    return true;
}

// The kernel over all of K (one slice: no workspace, C stored directly)
// against the K-split GEMM (one 32 x 32 tile per workgroup), for the shapes
// that kernel would take.  Both place one workgroup per compute unit (their
// LDS), so their time goes with their rounds of workgroups: a 64 x 64 tile
// over all of K costs about 2.45 times a 32 x 32 one (it brings in twice the
// rows and computes four times the outputs, sharing each row four ways).
// Measured on MI355X (us, K-split against this kernel, K = 4096): 512 x
// 1792 (4 rounds against 1) 32.2 / 21.5; 256 x 4096 (4 / 1) 34.7 / 22.5;
// 300 x 2000 (3 / 1) 25.3 / 20.9; 128 x 4096 (2 / 1) 18.2 / 20.6; 96 x 4096
// (2 / 1) 17.6 / 20.2; 512 x 1024 (2 / 1) 17.2 / 20.3.
bool splitk_whole_k(int M, int N, int K) {
    if (M < 8 || N < 1 || K < kBlock || (int64_t)K * kSkM > INT32_MAX) return false;
    const int64_t cus = device_cu_count();
    const int64_t t32 = ((int64_t)M + kTile - 1) / kTile * (((int64_t)N + kTile - 1) / kTile);
    const int64_t t64 = ((int64_t)M + kSkM - 1) / kSkM * (((int64_t)N + kSkN - 1) / kSkN);
    if (t64 > 0x7FFFFFFF) return false;
    const int64_t r32 = (t32 + cus - 1) / cus;
    const int64_t r64 = (t64 + cus - 1) / cus;
    return 100 * r32 > 245 * r64;
}

int splitk_whole_k_blocks(int K) { return (K / kBlock + kSkSB - 1) / kSkSB * kSkSB; }

namespace {

hipError_t launch_splitk(const int8_t* A, const float* AS, const int8_t* W, const float* WS,
                         float* C, int32_t* P, int M, int N, int K, bool ws_t, int S,
                         int slice_blocks, unsigned* cnt, float* part, unsigned* cnt_clear,
                         hipStream_t stream) {
    const int64_t tiles_m = ((int64_t)M + kSkM - 1) / kSkM;
    const int64_t tiles_n = ((int64_t)N + kSkN - 1) / kSkN;
    const int64_t total = tiles_m * tiles_n * S;
    if (total > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    auto launch = [&](auto kern) -> hipError_t {
        static std::atomic<uint64_t> lds_set[2][2] = {{{0}, {0}}, {{0}, {0}}};
        const hipError_t e = set_dynamic_lds(reinterpret_cast<const void*>(kern), (int)kSkSmem,
                                             lds_set[P != nullptr][ws_t]);
        if (e != hipSuccess) return e;
        kern<<<dim3((unsigned)total), kSkThreads, kSkSmem, stream>>>(
            A, AS, W, WS, C, P, M, N, K, (int)tiles_m, S, slice_blocks, part, cnt, cnt_clear);
        return hipGetLastError();
    };
    if (P != nullptr) return launch(qgemm_splitk_kernel<true, false>);
    if (ws_t) return launch(qgemm_splitk_kernel<false, true>);
    return launch(qgemm_splitk_kernel<false, false>);
}

// ---- The no-allocation form: the workspace is this file-scope device
// array (one copy per GPU, alive until the process ends): two counter areas
// used alternately (each call zero-fills the one the next call counts in,
// besides resetting its own counters), then the partial tiles.  With one
// workgroup per compute unit the split form never needs more than
// (compute units) x 16 KiB of partial tiles: 4 MiB on MI355X.
constexpr size_t kSkScratchParts = (size_t)4 << 20;
constexpr size_t kSkScratchBytes = 2 * kSkCounterBytes + kSkScratchParts;
static __device__ __align__(256) unsigned char scratch[kSkScratchBytes];

// The scratch array's device address on the current device, looked up once
// per device (with that device current) and kept; null if the lookup fails.
// Host code must use this address: the array's own name is a host-side
// stand-in, not a device address.
unsigned char* scratch_on_device() {
    constexpr int kMaxDevices = 64;
    static std::atomic<unsigned char*> addr[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    unsigned char* p = addr[dev].load(std::memory_order_acquire);
    if (p != nullptr) return p;
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) return nullptr;
    addr[dev].store(static_cast<unsigned char*>(q), std::memory_order_release);
    return static_cast<unsigned char*>(q);
}

}  // namespace

hipError_t launch_qgemm_splitk(const int8_t* A, const float* AS, const int8_t* W, const float* WS,
                               float* C, int32_t* P, int M, int N, int K, bool ws_t, int S,
                               int slice_blocks, void* workspace, hipStream_t stream) {
    unsigned* cnt = static_cast<unsigned*>(workspace);
    float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) + kSkCounterBytes);
    return launch_splitk(A, AS, W, WS, C, P, M, N, K, ws_t, S, slice_blocks, cnt, part, nullptr,
                         stream);
}

size_t splitk_scratch_capacity() { return kSkCounterBytes + kSkScratchParts; }

hipError_t launch_qgemm_splitk_scratch(const int8_t* A, const float* AS, const int8_t* W,
                                       const float* WS, float* C, int M, int N, int K, bool ws_t,
                                       int S, int slice_blocks, hipStream_t stream) {
    unsigned char* base = scratch_on_device();
    if (base == nullptr) return hipErrorInvalidSymbol;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    static std::atomic<uint64_t> epoch[64];
    const uint64_t e = epoch[dev].fetch_add(1, std::memory_order_relaxed);
    unsigned* cnt = reinterpret_cast<unsigned*>(base + (e & 1) * kSkCounterBytes);
    unsigned* clear = reinterpret_cast<unsigned*>(base + ((e + 1) & 1) * kSkCounterBytes);
    float* part = reinterpret_cast<float*>(base + 2 * kSkCounterBytes);
    return launch_splitk(A, AS, W, WS, C, nullptr, M, N, K, ws_t, S, slice_blocks, cnt, part,
                         clear, stream);
}

}  // namespace q8
