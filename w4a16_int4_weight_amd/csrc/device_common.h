// Device-side definitions shared by the W4A16 kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Packed tile layout, version 2 (K x N weight, 128-row blocks, 16-column blocks):
//   weight plane: block (nb, kb) = 1024 bytes at 1024 * (nb * KB + kb); lane L owns
//   16 bytes = 4 words; word i of lane L holds column 16 nb + (L % 16), rows
//   128 kb + 32 i + 8 (L / 16) + e, e = 0..7; nibble slot s holds row e = tile_row_of_slot(s).
//   metadata plane (after K*N/2 bytes): word n * KBP + kb = scale bits | zero << 16
//   for column n over row block kb; KBP = KB rounded up to a multiple of 4, the
//   padding words are 0. One 16-byte load gives a column's words for 4 row blocks.
constexpr int kRowsPerBlock = 128;
constexpr int kColsPerBlock = 16;
constexpr int kBlockBytes = 1024;

__host__ __device__ constexpr int64_t padded_row_blocks(int64_t K) { return ((K / kRowsPerBlock) + 3) / 4 * 4; }
// Columns of the packed layout: N rounded up to whole 16-column blocks (N % 8 == 0;
// a last block of 8 real columns carries 8 zero columns, code 0 and metadata 0).
// Metadata words: one per unit of min(G, 128) rows, i.e. 128 / G per 128-row block
// for group sizes 32 and 64 (1 otherwise); per column, K / unit rows rounded up to 4.
__host__ __device__ constexpr int units_per_block(int64_t G) { return G < kRowsPerBlock ? (int)(kRowsPerBlock / G) : 1; }
__host__ __device__ constexpr int64_t padded_units(int64_t K, int64_t G) {
    return ((K / kRowsPerBlock) * units_per_block(G) + 3) / 4 * 4;
}
__host__ __device__ constexpr int64_t padded_cols(int64_t N) { return (N + kColsPerBlock - 1) / kColsPerBlock * kColsPerBlock; }

// Row e held by nibble slot s of a tile word: 0,2,4,6,1,3,5,7. Slots t and t+4
// hold rows 2t and 2t+1, so (word >> 4t) & 0x000F000F puts the pair (2t, 2t+1)
// in the low bits of the two 16-bit halves.
__host__ __device__ constexpr int tile_row_of_slot(int s) { return 2 * (s & 3) + (s >> 2); }

// AWQ: column 8j + t of an AWQ word sits in nibble slot awq_slot_of_column(t),
// the inverse of the interleave 0,2,4,6,1,3,5,7 (slot s holds column ORDER[s]).
__host__ __device__ constexpr int awq_slot_of_column(int t) { return (t >> 1) + 4 * (t & 1); }

// Workgroup ids go to the 8 XCDs in turn (the XCD of id is id % 8). Kernels that cut
// their work into n ordered shares give workgroup id share (id % 8) (n / 8) + id / 8,
// so that neighbouring shares run on one XCD; grids of other sizes keep share = id.
__device__ __forceinline__ int xcd_share(int id, int n) {
    return (n & 7) ? id : (id & 7) * (n >> 3) + (id >> 3);
}

// 16-bit "magic" encodings: OR-ing a code q (0..15) into the low mantissa bits
// gives the exact value base + q.
//   bf16 0x4300 = 128.0, mantissa step 1 on [128, 256)
//   fp16 0x6400 = 1024.0, mantissa step 1 on [1024, 2048)
template <bool kBF16> struct Magic;
template <> struct Magic<true> {
    static constexpr uint32_t kBase2 = 0x43004300u;   // (128, 128)
    static constexpr uint32_t kNegBase = 0xC300u;      // -128; OR z gives -(128 + z)
    static constexpr float kBase = 128.0f;
};
template <> struct Magic<false> {
    static constexpr uint32_t kBase2 = 0x64006400u;   // (1024, 1024)
    static constexpr uint32_t kNegBase = 0xE400u;      // -1024; OR z gives -(1024 + z)
    static constexpr float kBase = 1024.0f;
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
    _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)b);
    return (float)h;
}

template <bool kBF16>
__device__ __forceinline__ float half_bits_to_f32(uint32_t b) {
    return kBF16 ? bf16_bits_to_f32(b) : f16_bits_to_f32(b);
}

// fp32 -> 16-bit, round to nearest even.
template <bool kBF16>
__device__ __forceinline__ uint16_t f32_to_half_bits(float v) {
    if constexpr (kBF16) {
        return __builtin_bit_cast(uint16_t, (__bf16)v);
    } else {
        return __builtin_bit_cast(uint16_t, (_Float16)v);
    }
}

// Two fp32 -> packed pair of 16-bit values (lo = a, hi = b), round to nearest even.
template <bool kBF16>
__device__ __forceinline__ uint32_t pack2_rne(float a, float b) {
    if constexpr (kBF16) {
        f32x2 v = {a, b};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
    } else {
        f32x2 v = {a, b};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
    }
}

// Decode one tile word (8 codes of one column, rows in slot order) into 8 values
// (q - z) * s in row order: the B operand of a 16x16x32 MFMA, or 8 consecutive
// output rows of a dequantised column.
template <bool kBF16> struct Dequant;

template <> struct Dequant<true> {
    // bf16: codes -> fp32 with the byte converters, (q - z) * s = fma(q, s, -z*s) is
    // exact in fp32 (a 4-bit integer times an 8-bit significand), then one RNE
    // conversion per pair. Byte b of (d & 0x0F0F0F0F) is slot 2b and byte b of
    // (d >> 4) & 0x0F0F0F0F is slot 2b+1; slot -> row: 0,2,4,6,1,3,5,7.
    float s, nzs;
    Dequant() = default;
    __device__ __forceinline__ Dequant(uint32_t md) {
        s = bf16_bits_to_f32(md & 0xFFFFu);
        nzs = -(float)((md >> 16) & 0xFu) * s;
    }
    __device__ __forceinline__ uint4 operator()(uint32_t d) const {
        uint32_t lo = d & 0x0F0F0F0Fu;          // rows 0, 4, 1, 5 in bytes 0..3
        uint32_t hi = (d >> 4) & 0x0F0F0F0Fu;   // rows 2, 6, 3, 7 in bytes 0..3
        // hide the masks from the optimiser so each byte converts with one
        // v_cvt_f32_ubyteN instead of an extract and a convert
        asm volatile("" : "+v"(lo), "+v"(hi));
        const float r0 = fmaf((float)(lo & 0xFFu), s, nzs);
        const float r4 = fmaf((float)((lo >> 8) & 0xFFu), s, nzs);
        const float r1 = fmaf((float)((lo >> 16) & 0xFFu), s, nzs);
        const float r5 = fmaf((float)(lo >> 24), s, nzs);
        const float r2 = fmaf((float)(hi & 0xFFu), s, nzs);
        const float r6 = fmaf((float)((hi >> 8) & 0xFFu), s, nzs);
        const float r3 = fmaf((float)((hi >> 16) & 0xFFu), s, nzs);
        const float r7 = fmaf((float)(hi >> 24), s, nzs);
        return make_uint4(pack2_rne<true>(r0, r1), pack2_rne<true>(r2, r3),
                          pack2_rne<true>(r4, r5), pack2_rne<true>(r6, r7));
    }
};

template <> struct Dequant<false> {
    // fp16: OR-ing a pair of codes into 1024.0 gives (1024 + q) exactly; a packed
    // fp16 subtract of (1024 + z) gives q - z exactly; a packed multiply by s rounds
    // (q - z) * s once, to nearest even.
    f16x2 zz, ss;
    Dequant() = default;
    __device__ __forceinline__ Dequant(uint32_t md) {
        const _Float16 s = __builtin_bit_cast(_Float16, (uint16_t)(md & 0xFFFFu));
        const _Float16 zb = (_Float16)(1024.0f + (float)((md >> 16) & 0xFu));
        zz = f16x2{zb, zb};
        ss = f16x2{s, s};
    }
    __device__ __forceinline__ uint32_t pair(uint32_t bits) const {
        f16x2 v = __builtin_bit_cast(f16x2, bits | Magic<false>::kBase2);
        v = (v - zz) * ss;
        return __builtin_bit_cast(uint32_t, v);
    }
    __device__ __forceinline__ uint4 operator()(uint32_t d) const {
        return make_uint4(pair(d & 0x000F000Fu), pair((d >> 4) & 0x000F000Fu),
                          pair((d >> 8) & 0x000F000Fu), pair((d >> 12) & 0x000F000Fu));
    }
};

// Direct global -> LDS copies (global_load_lds): each lane's 4 or 16 bytes land at
// M0 + 4*lane or M0 + 16*lane, M0 being uniform over the wave. They count in vmcnt
// like loads but occupy no registers, so several k blocks can be in flight. They are
// issued through inline assembly so that the compiler does not guard every later LDS
// read with a wait for all of them: the kernel waits for exactly the copies it needs.
// Scalar-base form: a wave-uniform 64-bit base in SGPRs plus a loop-invariant 32-bit
// byte offset per lane. (With a 64-bit address per copy the compiler rebuilt every
// address in one VGPR pair, so each copy waited until the previous one had read it:
// ~55 cycles a copy, a sixth of the k loop.)
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// (readfirstlane returns int: each half goes through uint32_t so that a low half
// with bit 31 set is not sign-extended over the high half)
__device__ __forceinline__ const uint8_t* uniform_ptr(const void* p) {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<const uint8_t*>((hi << 32) | lo);
}
// M0 is written as an output operand bound to that register ("={m0}"), not listed as a
// clobber: the compiler then knows the statement defines M0 and keeps nothing of its
// own there across it (a clobber of a reserved register is not honoured).
__device__ __forceinline__ void dma16(const uint8_t* base, uint32_t voff, uint32_t lds) {
    uint32_t m0v;
    asm volatile("s_mov_b32 %0, %3\n\tglobal_load_lds_dwordx4 %1, %2" : "={m0}"(m0v) : "v"(voff), "s"(base), "s"(lds)
                 : "memory");
}
__device__ __forceinline__ void dma4(const uint8_t* base, uint32_t voff, uint32_t lds) {
    uint32_t m0v;
    asm volatile("s_mov_b32 %0, %3\n\tglobal_load_lds_dword %1, %2" : "={m0}"(m0v) : "v"(voff), "s"(base), "s"(lds)
                 : "memory");
}

// Workgroup barrier that is also a compiler barrier for memory operations, without
// the vmcnt(0) a full __syncthreads() fence would add.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" : : : "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" : : : "memory");
}

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt low bits [3:0], high
// bits [15:14], expcnt [6:4] = 7, lgkmcnt [11:8] = 15).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// One 16-byte output store: a streaming (nontemporal) store where `nt`, else an
// ordinary one. Tile GEMMs whose grid fits the CUs in one round write streaming (their
// output is read by nothing in the launch); those of several rounds write ordinary
// stores (the streaming ones measured slower on one box for the W4A8 LM head).
__device__ __forceinline__ void store_out16(void* dst, const uint4 v, bool nt) {
    typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
    if (nt) __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_t*>(dst));
    else *reinterpret_cast<uint4*>(dst) = v;
}

// s_waitcnt with only lgkmcnt constrained, to zero: this wave's LDS accesses have
// completed (vmcnt field at its maximum 63, expcnt 7).
__device__ __forceinline__ void wait_lgkmcnt0() {
    __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));
}

// D = A(16x32) * B(32x16) + C, fp32 accumulate. Operand layout for lane l:
// A row l%16 / B column l%16, eight consecutive k starting at 8*(l/16);
// C/D: rows 4*(l/16) + r (r = register 0..3), column l%16.
template <bool kBF16>
__device__ __forceinline__ f32x4 mfma16x16x32(uint4 a, uint4 b, f32x4 c) {
    if constexpr (kBF16) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    } else {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
}

}  // namespace w4a16
