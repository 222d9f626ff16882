// Q8_0 block GEMM for few output tiles with the contraction split across
// workgroups (prompt projections with small M), on CDNA4 int8 MFMA.
//
// What is computed: the qdot_t row of the Q8_0 table ("Phobos Language Spec",
// section "Quantized built-ins"), or qmma_t with the weight scales stored
// [K/32][N] (same table): C[i, j] = sum_b AS[i, b] WS[j, b] P[i, j, b], with
// P the exact int32 block sums ("Quantized built-ins and formats", section
// "Q8_0": the inner sum is taken in integers); and the q50 rows of the same
// table, W held as Q5_0 blocks (value = code - 16).
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
// splitk_whole_k), and for shapes of one or two rounds of the staged GEMM's
// tiles on which it is faster (see splitk_over_staged).  Launches with more
// workgroups than compute units take a half-width form (4-block stages,
// 8 waves, a 72 KB ring) so that two workgroups share a unit.
//
//   - Staging: stages of 8 blocks (256 k; 4 in the half-width form); a
//     4-stage ring in LDS (36 KB a stage; 18 KB) filled by direct
//     global->LDS loads, three stages ahead.  Each stage is 48 wave-wide
//     load instructions (16 for the activation rows, 16 for the weight rows,
//     8 + 8 for the scales; half of each in the half-width form), three per
//     wave, so every wave waits for the same number of loads.  Row segments
//     are stored with their 16-byte chunks permuted (chunk c of row r at
//     c ^ (r mod 16); 128-byte rows: c ^ swz(r)) so that the MFMA fragment
//     reads are free of bank conflicts; the permutation is applied by
//     choosing which global chunk each lane loads.
//   - Math: 16 waves (8); wave w computes the 32 x 32 sub-tile w mod 4 on
//     blocks 2 (w / 4) and 2 (w / 4) + 1 of every stage: one v_mfma_i32_32x32x32_i8
//     per block (one Q8_0 block), seeded with the f32 bias pattern, and the
//     2-operation epilogue of ws_pair with the activation scale broadcast by
//     DPP (see qgemm.hip).
//   - Reduction: the four (two) waves of a sub-tile are summed in LDS in
//     wave order.  With S > 1 each workgroup writes its 64 x 64 partial tile to
//     the workspace, and the last of the tile's S workgroups to finish (an
//     atomic counter per tile) adds the S partial tiles in slice order
//     (0, 1, ..., S - 1, so the result does not depend on which finished
//     last) and stores C; it then resets the counter, so the workspace is
//     left zero-filled for the next call.
//   - The debug entry runs the same loads and MFMAs and stores each block
//     sum (D - bias) where the epilogue would run; it needs no workspace.
//   - Q5_0 weights (half-width form, one slice): each stage's raw 20-byte
//     blocks are staged like the other operands and decoded once into a
//     signed-byte tile laid out like the activation tile, behind a second
//     barrier, before the same MFMA loop.
#include "q8_device.h"
#include "q8_launch.h"

#include <type_traits>

namespace q8 {
namespace {

constexpr int kSkM = 64;                          // activation rows per tile
constexpr int kSkN = 64;                          // weight rows per tile
constexpr int kSkSB = 8;                          // blocks per stage, one workgroup per CU
constexpr int kSkRing = 4;                        // stages in LDS
constexpr int kSkTileFloats = kSkM * kSkN;        // one partial tile
// Workspace layout: one 32-bit counter per output tile in a fixed area at
// the start (so that calls of any shape sharing a workspace find their
// counters at zero), then the partial tiles.
constexpr int kSkMaxTiles = 1024;
constexpr size_t kSkCounterBytes = kSkMaxTiles * sizeof(unsigned);

// Stage width SB (Q8_0 blocks per stage): 8 (16 waves, a 144 KB ring: one
// workgroup per compute unit) or 4 (8 waves, a 72 KB ring: two workgroups
// share a compute unit, for launches with more workgroups than units).
// Either way every wave computes one 32 x 32 sub-tile on two blocks of each
// stage and issues three loads per stage.
template <int SB>
struct SkShape {
    static constexpr int kSeg = SB * kBlock;          // bytes of a row per stage
    static constexpr int kChunks = kSeg / 16;         // 16-byte chunks of a row segment
    static constexpr int kWaves = 2 * SB;
    static constexpr int kThreads = kWaves * kWave;
    static constexpr int kJobRows = kWave / kChunks;  // rows of one 16-byte-per-lane load
};

// Q5_0 weights (Q5): the ring holds each stage's raw 20-byte blocks
// ([row][SB blocks]); after the stage lands the workgroup decodes them once
// into a signed-byte tile laid out like the activation tile (one area,
// reused every stage), and a 1 KB spare area takes the loads of waves that
// have no weight piece to fetch.
constexpr int kQ5Bytes = 20;  // qh word + 16 nibble bytes per 32 values
template <int SB, bool Q5>
struct SkStage {
    int8_t a[kSkM * SkShape<SB>::kSeg];                       // [row][chunks], permuted
    int8_t w[kSkN * (Q5 ? SB * kQ5Bytes : SkShape<SB>::kSeg)];  // Q5: raw blocks
    float as[kSkM * SB];                                      // [row][block]
    float ws[kSkN * SB];  // [row][block]; transposed scales: [block][column]
};
template <int SB, bool Q5>
constexpr size_t sk_ring_bytes() {
    return sizeof(SkStage<SB, Q5>) * kSkRing + (Q5 ? kSkN * SkShape<SB>::kSeg + 1024 : 0);
}
static_assert(sizeof(SkStage<8, false>) == 36864 && sizeof(SkStage<4, false>) == 18432 &&
              sizeof(SkStage<8, true>) == 30720 && sizeof(SkStage<4, true>) == 15360, "stage layout");
static_assert(sk_ring_bytes<8, false>() <= 160 * 1024 && 2 * sk_ring_bytes<4, false>() <= 160 * 1024 &&
              sk_ring_bytes<8, true>() <= 160 * 1024 && 2 * sk_ring_bytes<4, true>() <= 160 * 1024,
              "LDS budget");
static_assert((size_t)SkShape<8>::kWaves * 16 * kWave * sizeof(float) <= sk_ring_bytes<8, true>() &&
              (size_t)SkShape<4>::kWaves * 16 * kWave * sizeof(float) <= sk_ring_bytes<4, true>() &&
              (size_t)SkShape<8>::kWaves * 16 * kWave * sizeof(float) <= sk_ring_bytes<8, false>() &&
              (size_t)SkShape<4>::kWaves * 16 * kWave * sizeof(float) <= sk_ring_bytes<4, false>(),
              "reduction area");
// Raw Q5_0 pieces of a stage: 16 bytes per lane, whole pieces per row.
static_assert((8 * kQ5Bytes) % 16 == 0 && (4 * kQ5Bytes) % 16 == 0, "Q5_0 row segments in 16-byte pieces");
static_assert(kSkN * 8 * kQ5Bytes / 16 <= SkShape<8>::kWaves * kWave &&
              kSkN * 4 * kQ5Bytes / 16 <= SkShape<4>::kWaves * kWave, "one Q5_0 piece job per wave at most");

// Signed bytes of half h (values 16 h .. 16 h + 15) of a Q5_0 block: code
// nibble | (bit of qh) << 4, value code - 16 ("Quantized built-ins and
// formats", section "Q5_0").  The byte permute turns each bit into the
// value's sign bits (selector 0x0C gives 0x00, 0x0D gives 0xFF).
__device__ __forceinline__ v4i q50_half(uint32_t qh, const uint32_t (&qs)[4], int h) {
    v4i out;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t nib = (qs[d] >> (4 * h)) & 0x0F0F0F0Fu;
        const uint32_t sel = 0x0D0D0D0Du - spread4(__builtin_amdgcn_ubfe(qh, 16 * h + 4 * d, 4));
        out[d] = (int)((__builtin_amdgcn_perm(0u, 0u, sel) & 0xF0F0F0F0u) | nib);
    }
    return out;
}
static_assert(kSkM / SkShape<8>::kJobRows == SkShape<8>::kWaves &&
              kSkM / SkShape<4>::kJobRows == SkShape<4>::kWaves, "one operand job per wave");

// Chunk c of row r sits at physical chunk c ^ perm(r): sixteen consecutive
// rows read at one logical chunk hit sixteen distinct 16-byte bank groups,
// so the MFMA fragment reads are free of bank conflicts (256-byte rows:
// r mod 16; 128-byte rows: swz).
template <int SB>
__device__ __forceinline__ int sk_perm(int r) {
    if constexpr (SB == 8) return r & 15;
    else return swz(r);
}

// WST: weight scales stored [K/32][N] (qmma_t).  S > 1: cnt (one counter per
// tile) and part (tiles x S partial tiles) are the workspace; cnt_clear (or
// null) is a counter area this kernel zero-fills for a later call.
// Q5: W holds Q5_0 blocks (20 bytes per 32 values, rows of K/32 blocks).
template <bool PARTIALS, bool WST, int SB, bool Q5>
__global__ void __launch_bounds__(SkShape<SB>::kThreads, SB == kSkSB ? 1 : 2)
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
    using Sh = SkShape<SB>;
    SkStage<SB, Q5>* ring = reinterpret_cast<SkStage<SB, Q5>*>(sk_smem);
    // Q5: the decoded weight tile and the spare load target, after the ring
    int8_t* dec = reinterpret_cast<int8_t*>(sk_smem) + sizeof(SkStage<SB, Q5>) * kSkRing;
    int8_t* spare = dec + kSkN * Sh::kSeg;
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
    const int nst = (kb_hi - kb_lo + SB - 1) / SB;

    const int lane = threadIdx.x & (kWave - 1);
    const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    const int half = lane / 32;
    const int col = lane & 31;
    const int rows_a = min(M - i0, kSkM);
    const int rows_w = min(N - j0, kSkN);

    // Descriptors of this tile's rows: reads past them return 0.
    const v4i dA = make_desc(A + (int64_t)i0 * K, (int64_t)rows_a * K);
    const int64_t w_pitch = Q5 ? (int64_t)KB * kQ5Bytes : K;  // bytes per weight row
    const v4i dW = make_desc(W + (int64_t)j0 * w_pitch, (int64_t)rows_w * w_pitch);
    const v4i dAS = make_desc(PARTIALS ? nullptr : AS + (int64_t)i0 * KB, (int64_t)rows_a * KB * 4);
    // Transposed weight scales: from column j0 to the end of the array
    // (columns past the tile meet zero weight rows and are never stored).
    const v4i dWS = make_desc(PARTIALS ? nullptr : WS + (WST ? (int64_t)j0 : (int64_t)j0 * KB),
                              WST ? ((int64_t)KB * N - j0) * 4 : (int64_t)rows_w * KB * 4);

    // Load jobs of stage st (three per wave).  Operand job q (wave q): the
    // kJobRows rows from kJobRows q; lane l fills physical chunk
    // l % kChunks of row kJobRows q + l / kChunks, i.e. loads the logical
    // chunk (l % kChunks) ^ perm(row).  Scale job e (waves below SB: the
    // activation scales; the others: the weight scales): rows
    // (64 / SB) e + l / SB, block l % SB ([row][block]); transposed weight
    // scales: block e, column l ([block][column]).  A chunk or block past
    // the slice (or past K) reads nothing and lands as zeros; so does a
    // stage past the last one (its ring slot is not read again).
    const int op_row = Sh::kJobRows * wv + lane / Sh::kChunks;
    const int op_chunk = (lane % Sh::kChunks) ^ sk_perm<SB>(op_row);
    const int op_voff = op_row * K + 16 * op_chunk;
    constexpr int kQ5RowPieces = SB * kQ5Bytes / 16;            // 10 or 5
    constexpr int q5_jobs = kSkN * kQ5RowPieces / kWave;         // 10 or 5 waves load pieces
    const int q5_row = (wv * kWave + lane) / kQ5RowPieces;
    const int q5_part = (wv * kWave + lane) % kQ5RowPieces;
    const int q5_voff = q5_row * KB * kQ5Bytes + 16 * q5_part;
    const int sc_job = wv < SB ? wv : wv - SB;
    const int sc_row = kSkM / SB * sc_job + lane / SB;
    const int sc_blk = lane % SB;
    auto issue_stage = [&](int st) {
        SkStage<SB, Q5>& sg = ring[st % kSkRing];
        const int kbs = kb_lo + st * SB;  // first block of the stage
        const bool in = st < nst;
        const int vo = (in && kbs + op_chunk / 2 < kb_hi) ? op_voff : kNoRead;
        dma16(dA, lds_addr(&sg.a[wv * Sh::kJobRows * Sh::kSeg]), vo, kbs * kBlock);
        if constexpr (Q5) {
            // piece 64 wv + lane of the stage's raw rows ([row][SB * 20 bytes]):
            // row q5_row, bytes 16 q5_part ..; pieces whose first byte lies
            // past the slice read nothing
            const bool real = wv < q5_jobs;
            const int v5 = (real && in && kbs + q5_part * 16 / kQ5Bytes < kb_hi) ? q5_voff : kNoRead;
            dma16(dW, lds_addr(real ? (void*)&sg.w[wv * 1024] : (void*)spare), v5, kbs * kQ5Bytes);
        } else {
            dma16(dW, lds_addr(&sg.w[wv * Sh::kJobRows * Sh::kSeg]), vo, kbs * kBlock);
        }
        if (wv < SB) {
            const bool ok = !PARTIALS && in && kbs + sc_blk < kb_hi;
            dma4(dAS, lds_addr(&sg.as[sc_job * kWave]), ok ? (sc_row * KB + kbs + sc_blk) * 4 : kNoRead, 0);
        } else if constexpr (WST) {
            const bool ok = !PARTIALS && in && kbs + sc_job < kb_hi;
            dma4(dWS, lds_addr(&sg.ws[sc_job * kWave]), ok ? ((kbs + sc_job) * N + lane) * 4 : kNoRead, 0);
        } else {
            const bool ok = !PARTIALS && in && kbs + sc_blk < kb_hi;
            dma4(dWS, lds_addr(&sg.ws[sc_job * kWave]), ok ? (sc_row * KB + kbs + sc_blk) * 4 : kNoRead, 0);
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
        frag_a[t] = a_row * Sh::kSeg + 16 * (c ^ sk_perm<SB>(a_row));
        frag_w[t] = w_row * Sh::kSeg + 16 * (c ^ sk_perm<SB>(w_row));
    }

    v16i bias;
#pragma unroll
    for (int r = 0; r < 16; ++r) bias[r] = kBias;
    asm volatile("" : "+v"(bias));
    float acc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;

    // Q5: decode the stage's raw weight blocks into the signed-byte tile
    // (laid out like the activation tile).  Lane item 64 wv + lane takes
    // half item % 2 of block (item / 2) % SB of row item / (2 SB): the
    // workgroup's lanes cover the stage exactly once.  Neighbouring lanes
    // read neighbouring 20-byte blocks (distinct banks), and the writes of
    // a wave fill 1 KB of whole permuted rows.
    auto decode_stage = [&](int st) {
        const SkStage<SB, Q5>& sg = ring[st % kSkRing];
        const int item = wv * kWave + lane;
        const int r = item / (2 * SB), bb = (item / 2) % SB, h = item & 1;
        const uint32_t* wd = reinterpret_cast<const uint32_t*>(sg.w + r * (SB * kQ5Bytes) + kQ5Bytes * bb);
        const uint32_t qs[4] = {wd[1], wd[2], wd[3], wd[4]};
        *reinterpret_cast<v4i*>(dec + r * Sh::kSeg + 16 * ((2 * bb + h) ^ sk_perm<SB>(r))) =
            q50_half(wd[0], qs, h);
    };

    auto compute_stage = [&](int st) {
        const SkStage<SB, Q5>& sg = ring[st % kSkRing];
        const int kbs = kb_lo + st * SB + 2 * kq;
        float2 ws2 = make_float2(0.0f, 0.0f), as2 = make_float2(0.0f, 0.0f);
        if constexpr (!PARTIALS) {
            as2 = *reinterpret_cast<const float2*>(&sg.as[as_row * SB + 2 * kq]);
            if constexpr (WST) ws2 = make_float2(sg.ws[(2 * kq) * kSkN + w_row], sg.ws[(2 * kq + 1) * kSkN + w_row]);
            else ws2 = *reinterpret_cast<const float2*>(&sg.ws[w_row * SB + 2 * kq]);
        }
        const float wsv[2] = {ws2.x, ws2.y};
        const float asv[2] = {as2.x, as2.y};
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int b = kbs + t;
            if (b >= kb_hi) break;  // wave-uniform
            const v4i af = *reinterpret_cast<const v4i*>(sg.a + frag_a[t]);
            const v4i wf = *reinterpret_cast<const v4i*>((Q5 ? dec : sg.w) + frag_w[t]);
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
        if constexpr (Q5) {
            // every wave's decoded bytes are in LDS before any wave reads
            // them (no vmcnt wait: the later stages' loads stay in flight)
            decode_stage(st);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_s_barrier();
        }
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
                const int b = kb_lo + st * SB + 2 * kq + t;
                if (b >= kb_hi) break;
                const int ko = b * kBlock + 16 * half;
                const v4i af = ia < M ? load16(A + (int64_t)ia * K + ko) : v4i{0, 0, 0, 0};
                v4i wf = {0, 0, 0, 0};
                if (jw < N) {
                    if constexpr (Q5) {
                        const int8_t* blk = W + (int64_t)jw * w_pitch + (int64_t)b * kQ5Bytes;
                        const v4i q = load16_a4(blk + 4);
                        const uint32_t qs[4] = {(uint32_t)q.x, (uint32_t)q.y, (uint32_t)q.z, (uint32_t)q.w};
                        wf = q50_half(*reinterpret_cast<const uint32_t*>(blk), qs, half);
                    } else {
                        wf = load16(W + (int64_t)jw * K + ko);
                    }
                }
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

    // The waves of each sub-tile, summed in wave order (kq = 0, 1, ...).
    float* red = reinterpret_cast<float*>(sk_smem);  // [waves][16][64]
#pragma unroll
    for (int r = 0; r < 16; ++r) red[(wv * 16 + r) * kWave + lane] = acc[r];
    __syncthreads();
    float tot[16];
    if (wv < 4) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float s = red[(wv * 16 + r) * kWave + lane];
#pragma unroll
            for (int k = 1; k < Sh::kWaves / 4; ++k) s += red[((wv + 4 * k) * 16 + r) * kWave + lane];
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

// Shapes the LDS-staged GEMM would take (at least 128 of its 128 x 224
// tiles) on which this kernel, two workgroups per compute unit, is faster.
// The staged GEMM runs in rounds of one workgroup per unit, a round costing
// about as much as a full one even when partly filled; this kernel's time
// grows with its 64 x 64 tiles per unit (~0.07 us per tile per K/32 = 128
// blocks, i.e. ~18 us per tile per unit at K = 4096).  Measured on MI355X
// (us, staged against this kernel, K = 4096 unless noted; 64 x 64 tiles):
// 256 x 14336 (896) 77.1 / 69.0; 128 x 28672 (896) 78.2 / 73.3; 130 x 14336
// (672) 72.8 / 53.6; 256 x 16384 (1024) 80.8 / 72.1; 1024 x 4096 (1024)
// 78.6 / 70.8; 2048 x 4096 (2048, two staged rounds) 149.6 / 140.3;
// 256 x 14336 x 8192 139.9 / 123.3; K = 1024: 256 x 14336 25.9 / 26.2,
// 1024 x 4096 25.9 / 25.2.  And the other way: 320 x 14336 (1120) 79.1 /
// 85.2; 384 x 14336 (1344) 81.2 / 100.2; 1536 x 4096 (1536) 87.4 / 109.6;
// 512 x 14336 (1792) 90.9 / 123.8; 640 x 14336 (2240, two rounds) 151.5 /
// 148.4; 768 x 14336 (2688, two rounds) 151.3 / 171.0.  Rule: this kernel
// when its tiles number at most 4.1 per unit per staged round.
bool splitk_over_staged(int M, int N, int K) {
    if (M < 8 || N < 1 || K < kBlock || (int64_t)K * kSkM > INT32_MAX) return false;
    const int64_t cus = device_cu_count();
    const int64_t t64 = ((int64_t)M + kSkM - 1) / kSkM * (((int64_t)N + kSkN - 1) / kSkN);
    const int64_t ts = ((int64_t)M + kStagedTileM - 1) / kStagedTileM *
                       (((int64_t)N + kStagedTileN - 1) / kStagedTileN);
    if (t64 > 0x7FFFFFFF) return false;
    const int64_t rounds = (ts + cus - 1) / cus;
    return 10 * t64 <= 41 * cus * rounds;
}

bool splitk_shared(int M, int N) {
    const int64_t t64 = ((int64_t)M + kSkM - 1) / kSkM * (((int64_t)N + kSkN - 1) / kSkN);
    return t64 > device_cu_count();
}

int splitk_whole_k_blocks(int K) { return (K / kBlock + kSkSB - 1) / kSkSB * kSkSB; }

namespace {

template <bool Q5>
hipError_t launch_splitk(const int8_t* A, const float* AS, const int8_t* W, const float* WS,
                         float* C, int32_t* P, int M, int N, int K, bool ws_t, int S,
                         int slice_blocks, unsigned* cnt, float* part, unsigned* cnt_clear,
                         hipStream_t stream) {
    const int64_t tiles_m = ((int64_t)M + kSkM - 1) / kSkM;
    const int64_t tiles_n = ((int64_t)N + kSkN - 1) / kSkN;
    const int64_t total = tiles_m * tiles_n * S;
    if (total > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    // More workgroups than compute units: the 8-wave form with its 72 KB
    // ring, so that two workgroups share a unit and one's loads run under
    // the other's math.  Q5_0 weights always take that form (they are
    // dispatched here only for such launches).
    const bool shared = Q5 || total > device_cu_count();
    auto launch = [&](auto kern, auto sb_const) -> hipError_t {
        constexpr int SB = decltype(sb_const)::value;
        constexpr size_t smem = sk_ring_bytes<SB, Q5>();
        static std::atomic<uint64_t> lds_set[2][2] = {{{0}, {0}}, {{0}, {0}}};
        const hipError_t e = set_dynamic_lds(reinterpret_cast<const void*>(kern), (int)smem,
                                             lds_set[P != nullptr][ws_t]);
        if (e != hipSuccess) return e;
        kern<<<dim3((unsigned)total), SkShape<SB>::kThreads, smem, stream>>>(
            A, AS, W, WS, C, P, M, N, K, (int)tiles_m, S, slice_blocks, part, cnt, cnt_clear);
        return hipGetLastError();
    };
    using Wide = std::integral_constant<int, kSkSB>;
    using Narrow = std::integral_constant<int, kSkSB / 2>;
    if (shared) {
        if (P != nullptr) return launch(qgemm_splitk_kernel<true, false, Narrow::value, Q5>, Narrow{});
        if (ws_t) return launch(qgemm_splitk_kernel<false, true, Narrow::value, Q5>, Narrow{});
        return launch(qgemm_splitk_kernel<false, false, Narrow::value, Q5>, Narrow{});
    }
    if constexpr (!Q5) {
        if (P != nullptr) return launch(qgemm_splitk_kernel<true, false, Wide::value, false>, Wide{});
        if (ws_t) return launch(qgemm_splitk_kernel<false, true, Wide::value, false>, Wide{});
        return launch(qgemm_splitk_kernel<false, false, Wide::value, false>, Wide{});
    }
    return hipErrorInvalidValue;  // not reached
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
    return launch_splitk<false>(A, AS, W, WS, C, P, M, N, K, ws_t, S, slice_blocks, cnt, part, nullptr,
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
    return launch_splitk<false>(A, AS, W, WS, C, nullptr, M, N, K, ws_t, S, slice_blocks, cnt, part,
                                clear, stream);
}

hipError_t launch_qgemm_splitk_q50(const int8_t* A, const float* AS, const uint8_t* W5,
                                   const float* WS, float* C, int32_t* P, int M, int N, int K,
                                   bool ws_t, hipStream_t stream) {
    return launch_splitk<true>(A, AS, reinterpret_cast<const int8_t*>(W5), WS, C, P, M, N, K, ws_t, 1,
                               splitk_whole_k_blocks(K), nullptr, nullptr, nullptr, stream);
}

}  // namespace q8
