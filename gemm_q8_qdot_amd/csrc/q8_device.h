// Device-side helpers shared by the Q8_0 kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q8 {

constexpr int kBlock = 32;   // Q8_0 block: 32 consecutive k share one scale
constexpr int kWave = 64;    // CDNA wavefront width

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// DPP controls (GFX9 encoding).
constexpr int kDppSwapPairs = 0xB1;   // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kDppSwapHalves = 0x4E;  // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kDppRowHalfMirror = 0x141;  // lane k <- 7 - k within 8 lanes
constexpr int kDppRowMirror = 0x140;      // lane k <- 15 - k within 16 lanes

template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v) {
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Signed 4 x i8 dot product accumulated into an int32 (v_dot4_i32_i8): the
// "Phobos Language Spec" dp4a of section "Operators and conversions" -- acc
// plus the sum of the products of the four signed bytes of x and of y.
__device__ __forceinline__ int dot4(int x, int y, int acc) {
    return __builtin_amdgcn_sdot4(x, y, acc, false);
}

// Integer dot of 16 signed bytes.
__device__ __forceinline__ int dot16(v4i a, v4i w, int acc) {
    acc = dot4(a.x, w.x, acc);
    acc = dot4(a.y, w.y, acc);
    acc = dot4(a.z, w.z, acc);
    acc = dot4(a.w, w.w, acc);
    return acc;
}

// Sum over all 64 lanes; every lane gets the total.  Fixed order, so the
// result is deterministic: two DPP quad steps, two DPP mirror steps (each
// 16-lane row then holds its row sum), then the four row sums via readlane.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_f32<kDppSwapPairs>(v);
    v += dpp_f32<kDppSwapHalves>(v);
    v += dpp_f32<kDppRowHalfMirror>(v);
    v += dpp_f32<kDppRowMirror>(v);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ v4i load16(const int8_t* p) {
    return *reinterpret_cast<const v4i*>(p);
}

// 16 bytes from an address that is only 4-byte aligned (one dword-aligned
// 16-byte load: the hardware's unaligned-access mode serves it).
typedef int v4i_a4 __attribute__((ext_vector_type(4), aligned(4)));
__device__ __forceinline__ v4i load16_a4(const void* p) {
    const v4i_a4 v = *reinterpret_cast<const v4i_a4*>(p);
    return v4i{v.x, v.y, v.z, v.w};
}

__device__ __forceinline__ v4i load16_stream(const int8_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const v4i*>(p));
}

// ---- v_mfma_i32_32x32x32_i8 (one 32-wide Q8_0 block of a 32 x 32 tile) ----
// Lane l supplies row l % 32 of each operand and the 16 bytes
// k in [16 (l / 32), +16) of the block; register r of the result holds
// D[m][n] with n = l % 32 and m = tile_row(r, l / 32).
constexpr int kTile = 32;
constexpr int kBias = 0x4B400000;  // bits of 12582912.0f = 1.5 * 2^23
constexpr float kBiasF = 12582912.0f;

__device__ __forceinline__ int tile_row(int r, int half) {
    return 8 * (r / 4) + 4 * half + (r % 4);
}

// (ws_hi, -12582912 ws_hi): ws with its two low mantissa bits cleared, so
// that the product with the bias is exact.  With D = the MFMA result seeded
// with kBias (bits of the f32 12582912 + p), fma(ws_hi, D, -12582912 ws_hi)
// is ws_hi * p rounded once.
__device__ __forceinline__ float2 ws_pair(float ws) {
    const float hi = __int_as_float(__float_as_int(ws) & ~3);
    return make_float2(hi, hi * -kBiasF);
}

// acc[R0 + k] += as(lane 16 (l / 16) + R0 + k) * u[R0 + k] for k < 8: one
// v_fmac_f32 per element whose first factor comes through the DPP
// row_newbcast control, i.e. from lane R0 + k of the lane's 16-lane row.  A
// lane thus holds one scale per 16-lane row position instead of sixteen.
// The leading s_nop covers the two wait states a DPP source needs after a
// VALU write of it.
template <int R0>
__device__ __forceinline__ void fmac_rowbcast8(float (&acc)[16], float as, const float (&u)[16]) {
    asm("s_nop 1\n\t"
        "v_fmac_f32_dpp %0, %8, %9 row_newbcast:%17 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %1, %8, %10 row_newbcast:%18 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %2, %8, %11 row_newbcast:%19 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %3, %8, %12 row_newbcast:%20 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %4, %8, %13 row_newbcast:%21 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %5, %8, %14 row_newbcast:%22 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %6, %8, %15 row_newbcast:%23 row_mask:0xf bank_mask:0xf\n\t"
        "v_fmac_f32_dpp %7, %8, %16 row_newbcast:%24 row_mask:0xf bank_mask:0xf"
        : "+v"(acc[R0]), "+v"(acc[R0 + 1]), "+v"(acc[R0 + 2]), "+v"(acc[R0 + 3]),
          "+v"(acc[R0 + 4]), "+v"(acc[R0 + 5]), "+v"(acc[R0 + 6]), "+v"(acc[R0 + 7])
        : "v"(as), "v"(u[R0]), "v"(u[R0 + 1]), "v"(u[R0 + 2]), "v"(u[R0 + 3]), "v"(u[R0 + 4]),
          "v"(u[R0 + 5]), "v"(u[R0 + 6]), "v"(u[R0 + 7]),
          "n"(R0), "n"(R0 + 1), "n"(R0 + 2), "n"(R0 + 3), "n"(R0 + 4), "n"(R0 + 5), "n"(R0 + 6),
          "n"(R0 + 7));
}

// ---- raw buffer loads (SGPR resource + 32-bit per-lane offset) ----
// A load whose per-lane offset is at or past the resource's byte count
// returns zeros; kNoRead is such an offset for every resource here.
constexpr int kNoRead = 0x7FFFFFF0;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int64_t bytes) {
    const int n = bytes > 0x7FFFFFFF ? 0x7FFFFFFF : (int)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, 0x00020000);
}
__device__ __forceinline__ v4i buffer_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
// Streaming form for data read once: cache policy bit 1 (nt).
__device__ __forceinline__ v4i buffer_load16_nt(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 2));
}
__device__ __forceinline__ float buffer_load_f32(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}

// ---- Buffer loads straight into LDS (direct global -> LDS DMA).
typedef __attribute__((address_space(3))) char lds_char;
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit dwords (gfx9 family)

// Raw buffer descriptor (in SGPRs) for `bytes` bytes at `base`; reads whose
// offset is past the range return 0 (and write 0 to LDS).
__device__ __forceinline__ v4i make_desc(const void* base, int64_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const int n = bytes > 0x7FFFFFFF ? 0x7FFFFFFF : (int)bytes;
    v4i d;
    d.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    d.y = __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xFFFF));  // stride 0
    d.z = __builtin_amdgcn_readfirstlane(n);
    d.w = kRsrcWord3;
    return d;
}

// Lane l's 16 (dma16) or 4 (dma4) bytes from offset voff + soff land at
// LDS address lds + l * size.  Issued from inline assembly, so the compiler
// neither waits on them nor counts them: the caller waits (s_waitcnt vmcnt)
// before the data is read.  m0 carries the LDS address.
__device__ __forceinline__ void dma16(v4i desc, uint32_t lds, int voff, int soff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(lds), "v"(voff), "s"(desc), "s"(soff) : "memory", "m0");
}
__device__ __forceinline__ void dma4(v4i desc, uint32_t lds, int voff, int soff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                 :: "s"(lds), "v"(voff), "s"(desc), "s"(soff) : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    // wave-uniform: m0 is a scalar register
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)(const lds_char*)p);
}

// LDS tiles of 128-byte row segments (four Q8_0 blocks = eight 16-byte
// chunks per row): row r holds its chunks permuted, logical chunk c at
// physical chunk c ^ swz(r).  Sixteen consecutive rows read at the same
// logical chunk then hit sixteen distinct 16-byte bank groups (with 32 or 64
// four-byte banks), so the MFMA fragment reads are conflict-free.  swz only
// depends on r mod 16, so a lane's chunk is the same in every 16-row group.
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// ---- Q5_0 weight blocks: 20 bytes per 32 values, the qh word then 16
// bytes, byte e holding element e (low nibble) and element e + 16 (high);
// code q = nibble | (bit e of qh) << 4, value q - 16.
// Four bits of x (bits 0..3) to bit 0 of four bytes: x * (1 + 2^7 + 2^14 +
// 2^21) places bit i at bit 8 i with no overlapping copies (x < 16).  Both
// factors fit 24 bits: v_mul_u32_u24 (full rate; the compiler would pick the
// quarter-rate 32-bit multiply).
__device__ __forceinline__ uint32_t spread4(uint32_t x) {
    uint32_t r;
    asm("v_mul_u32_u24 %0, 0x204081, %1" : "=v"(r) : "v"(x));
    return r & 0x01010101u;
}

// The 32 codes q (0..31) of one block as 8 dwords of bytes: elements
// 4d..4d+3 in q[d], elements 16+4d.. in q[4+d].
__device__ __forceinline__ void q50_codes(uint32_t qh, const v4i& qs, uint32_t (&q)[8]) {
    const uint32_t w[4] = {(uint32_t)qs.x, (uint32_t)qs.y, (uint32_t)qs.z, (uint32_t)qs.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t lo = w[d] & 0x0F0F0F0Fu;
        const uint32_t hi = (w[d] >> 4) & 0x0F0F0F0Fu;
        q[d] = lo | (spread4(__builtin_amdgcn_ubfe(qh, 4 * d, 4)) << 4);
        q[4 + d] = hi | (spread4(__builtin_amdgcn_ubfe(qh, 16 + 4 * d, 4)) << 4);
    }
}

// The 32 values q - 16 of one block as 8 dwords of signed bytes (same
// order as q50_codes): value = nibble - 16 when the qh bit is clear, the
// nibble itself when it is set, i.e. the nibble with 0xF0 or'ed in where
// the bit is clear (v_perm_b32 selector 0x0C gives byte 0x00, 0x0D 0xFF).
__device__ __forceinline__ void q50_values(uint32_t qh, const v4i& qs, uint32_t (&v)[8]) {
    const uint32_t w[4] = {(uint32_t)qs.x, (uint32_t)qs.y, (uint32_t)qs.z, (uint32_t)qs.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t lo = w[d] & 0x0F0F0F0Fu;
        const uint32_t hi = (w[d] >> 4) & 0x0F0F0F0Fu;
        const uint32_t sl = 0x0D0D0D0Du - spread4(__builtin_amdgcn_ubfe(qh, 4 * d, 4));
        const uint32_t sh = 0x0D0D0D0Du - spread4(__builtin_amdgcn_ubfe(qh, 16 + 4 * d, 4));
        v[d] = (__builtin_amdgcn_perm(0u, 0u, sl) & 0xF0F0F0F0u) | lo;
        v[4 + d] = (__builtin_amdgcn_perm(0u, 0u, sh) & 0xF0F0F0F0u) | hi;
    }
}

}  // namespace q8
