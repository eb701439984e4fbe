// W4A8: the packed int4 weights of the W4A16 layer against fp8 (E4M3) activations,
// on the fp8 matrix cores.
//
// The vLLM note "Carga de capas cuantizadas: AWQ / GPTQ / Marlin / fp8" (section
// "Límites y fallos") describes the int4 Marlin kernel taking float8_e4m3fn
// activations: the weights get a one-time fp8 pre-processing and the scales are
// multiplied by 512. The factor has a plain reason on any hardware: a 4-bit code q
// in the low nibble of an E4M3 byte (exponent field 0 or 1, mantissa the low three
// bits) reads as q * 2^-9 exactly, so the packed codes become fp8 operands with two
// instructions per 8 codes (mask, shift-and-mask), and 2^9 restores the scale. Here
// the factor is applied to each scale as it is read, so one packed buffer (the W4A16
// layout, unchanged) serves both activation types.
//
// Activations are quantised per row: a = max |x| / 448, codes RNE(x / a), with the
// codes written in the order the MFMA operands take them and each 128-element block's
// code sum written beside them (quantize_kernel). The product is
//
//   y[m, n] = a[m] * sum_g ( 512 s[g, n] * D[g] - s[g, n] z[g, n] * X[m, g] ) + bias[n],
//   D[g] = sum_{k in block g} e[m, k] * (q[k, n] * 2^-9),  X[m, g] = sum_{k in g} e[m, k],
//
// one 16x16x128 fp8 MFMA per 16x16 output fragment and 128-row block giving D
// exactly (products of two E4M3 values are exact, the sum is fp32); 512 s scales it
// into the fp32 accumulators. The zero-point term, a [M x K/128] by [K/128 x N]
// product, runs after the loop on the fp32 matrix cores (16x16x4).
//
// Tiling, the three-stage ring of direct global -> LDS copies, the XCD-aware
// workgroup order and the K split are those of the 16-bit GEMM; the activation
// tile is half the size (one byte per element).
#include <stddef.h>

#include "device_common.h"
#include "launch.h"
#include "split_k.h"

namespace w4a16 {
namespace {

constexpr int kXcds = 8;
constexpr int kTilesPerRound = 256;       // one workgroup of the widest tile per CU
constexpr float kE4M3Max = 448.0f;

typedef int i32x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- quantisation

constexpr int kQuantThreads = 256;

// One workgroup per row. Pass 1: max |x|; pass 2: codes, in operand order (within each
// 128-element block, byte 32 h + 8 i + j holds element 32 i + 8 h + (0,4,1,5,2,6,3,7)[j]),
// and the block sums of the decoded codes. A thread keeps its first kQuantCached chunks
// of 16 bytes (all of them for K <= 8192) in registers between the passes, so pass 2
// reads nothing again.
constexpr int kQuantCached = 4;

template <bool kBF16>
__device__ __forceinline__ float chunk_absmax(const uint4 v, float amax) {
    const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        amax = fmaxf(amax, fabsf(half_bits_to_f32<kBF16>(wd[t] & 0xFFFFu)));
        amax = fmaxf(amax, fabsf(half_bits_to_f32<kBF16>(wd[t] >> 16)));
    }
    return amax;
}

// chunk c of the row (8 elements): block c / 16, rows 8 (c % 16) .. +7 of it = step i,
// lane group h. Its codes, and (by the first lane of its block's 16) the block's sum.
template <bool kBF16>
__device__ __forceinline__ void quantize_chunk(const uint4 v, int c, float scale, uint8_t* __restrict__ cr,
                                               float* __restrict__ bs) {
    const int kb = c >> 4, i = (c & 15) >> 2, h = c & 3;
    const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
    float q[8];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        q[2 * t] = half_bits_to_f32<kBF16>(wd[t] & 0xFFFFu) / scale;
        q[2 * t + 1] = half_bits_to_f32<kBF16>(wd[t] >> 16) / scale;
    }
    // bytes 0..3 = rows 0, 4, 1, 5; bytes 4..7 = rows 2, 6, 3, 7 (RNE, OCP E4M3)
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[4], 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[1], q[5], lo, true);
    int hi = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[6], 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(q[3], q[7], hi, true);
    *reinterpret_cast<uint2*>(cr + (size_t)kb * kRowsPerBlock + 32 * h + 8 * i) = make_uint2((uint32_t)lo, (uint32_t)hi);
    float s = __builtin_amdgcn_cvt_f32_fp8(lo, 0) + __builtin_amdgcn_cvt_f32_fp8(lo, 1);
    s += __builtin_amdgcn_cvt_f32_fp8(lo, 2) + __builtin_amdgcn_cvt_f32_fp8(lo, 3);
    s += __builtin_amdgcn_cvt_f32_fp8(hi, 0) + __builtin_amdgcn_cvt_f32_fp8(hi, 1);
    s += __builtin_amdgcn_cvt_f32_fp8(hi, 2) + __builtin_amdgcn_cvt_f32_fp8(hi, 3);
    // the 16 chunks of a block sit in 16 consecutive lanes (K / 8 is a multiple of 16,
    // so those lanes are all active or all idle together)
#pragma unroll
    for (int d = 8; d >= 1; d >>= 1) s += __shfl_xor(s, d, 16);
    if ((c & 15) == 0) bs[kb] = s;
}

template <bool kBF16>
__global__ __launch_bounds__(kQuantThreads) void quantize_kernel(const uint16_t* __restrict__ x,
                                                                  uint8_t* __restrict__ codes,
                                                                  float* __restrict__ row_scale,
                                                                  float* __restrict__ block_sum, int K) {
    __shared__ float wave_max[kQuantThreads / 64];
    const int m = blockIdx.x;
    const int tid = threadIdx.x;
    const uint16_t* xr = x + (size_t)m * K;
    const int chunks = K / 8;                  // 8 elements (16 bytes) each
    float amax = 0.f;
    uint4 cached[kQuantCached];
#pragma unroll
    for (int k = 0; k < kQuantCached; ++k) {
        const int c = tid + k * kQuantThreads;
        cached[k] = c < chunks ? *reinterpret_cast<const uint4*>(xr + 8 * c) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int k = 0; k < kQuantCached; ++k) amax = chunk_absmax<kBF16>(cached[k], amax);
    for (int c = tid + kQuantCached * kQuantThreads; c < chunks; c += kQuantThreads)
        amax = chunk_absmax<kBF16>(*reinterpret_cast<const uint4*>(xr + 8 * c), amax);
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) amax = fmaxf(amax, __shfl_xor(amax, d));
    if ((tid & 63) == 0) wave_max[tid >> 6] = amax;
    __syncthreads();
    amax = wave_max[0];
#pragma unroll
    for (int i = 1; i < kQuantThreads / 64; ++i) amax = fmaxf(amax, wave_max[i]);
    const float scale = amax > 0.f ? amax / kE4M3Max : 1.f;     // IEEE division, as are the quotients
    if (tid == 0) row_scale[m] = scale;

    uint8_t* cr = codes + (size_t)m * K;
    float* bs = block_sum + (size_t)m * (K / kRowsPerBlock);
#pragma unroll
    for (int k = 0; k < kQuantCached; ++k) {
        const int c = tid + k * kQuantThreads;
        if (c < chunks) quantize_chunk<kBF16>(cached[k], c, scale, cr, bs);
    }
    for (int c = tid + kQuantCached * kQuantThreads; c < chunks; c += kQuantThreads)
        quantize_chunk<kBF16>(*reinterpret_cast<const uint4*>(xr + 8 * c), c, scale, cr, bs);
}

// ---------------------------------------------------------------- GEMM

// One stage of the LDS ring: the fp8 activation tile of one 128-row block of K
// (16-byte chunk j of row r stored at chunk j ^ row_swizzle(r)) and the workgroup's
// blocks of packed codes.
template <int BM, int CBW, int W, bool kGroupMeta>
struct StageA8 {
    uint4 x[BM * 8];
    uint4 w[W * CBW * 64];
    uint32_t meta[kGroupMeta ? 1 : W * 64];  // per-stage metadata of small tiles (64 per wave)
};

// Metadata of 4 consecutive k blocks for the 16 CBW columns of one wave, per column its
// 4 words (contiguous in the packed layout): CBW 4-byte copies of 16 columns each, with
// the group's first stage, instead of one copy per k block touching a line per lane.
template <int CBW>
struct MetaGroupA8 {
    uint32_t words[16 * CBW * 4];           // [column of the wave][k block of the group]
};

// XOR applied to the chunk index of row r of the activation tile. A fragment read
// (16 rows, chunks 2h and 2h+1 of each) then meets no bank twice, whether the LDS
// serves 16 lanes per cycle from 64 banks or 32 lanes from 128: bits 1..3 of the row
// go to the chunk bits in the order (2, 1, 3), so rows 4 apart (one 512-byte bank
// span) and rows 2 apart (one 256-byte span) differ in chunk bits that the lane
// groups h do not use. (XOR with r % 8 measured one bank-conflict cycle per read
// cycle on gfx950.)
__device__ __forceinline__ int row_swizzle(int r) { return ((r >> 2) & 1) | (r & 2) | (((r >> 3) & 1) << 2); }

// v as two bf16 values (hi = v rounded to nearest even, lo = the rest rounded), packed
// (lo half = hi): exact wherever v has at most 16 significant bits around hi's exponent
__device__ __forceinline__ uint32_t bf16_split(float v) {
    const float hi = __uint_as_float(pack2_rne<true>(v, 0.f) << 16);
    return pack2_rne<true>(v, v - hi);
}
// v's two bf16 parts, each duplicated into both halves of a packed pair
__device__ __forceinline__ void bf16_split_dup(float v, uint32_t& hi2, uint32_t& lo2) {
    hi2 = pack2_rne<true>(v, v);
    const float hi = __uint_as_float(hi2 << 16);
    const float lo = v - hi;
    lo2 = pack2_rne<true>(lo, lo);
}

__device__ __forceinline__ f32x4 mfma_fp8(const i32x8& a, const i32x8& b) {
    // format 0 (E4M3) for both operands, no block scales: the plain 16x16x128 fp8 MFMA
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
}

// Workgroup tile 16*MR rows x 16*CBW*kWaves columns, waves side by side along N as in
// the 16-bit GEMM. MFMA operands: weights first, activations second, so each lane
// holds 4 adjacent output columns of one row (lane (c, h), register e -> row 16 r + c,
// column 16 j + 4 h + e).
template <bool kBF16, int MR, int CBW, int kWaves, bool kZpStaged>
__global__ __launch_bounds__(64 * kWaves) void w4a8_gemm_kernel(
    const uint8_t* __restrict__ act, const float* __restrict__ row_scale, const float* __restrict__ block_sum,
    const uint8_t* __restrict__ packed, const uint16_t* __restrict__ bias, uint16_t* __restrict__ y, int M, int K,
    int N, int tiles_m, int tiles_n, int splits, uint32_t* __restrict__ counters, float* __restrict__ partials,
    int nt_out) {
    constexpr int BM = 16 * MR;
    constexpr int kXBytes = BM * kRowsPerBlock;
    // 1 KiB copies (8 rows) when every wave gets at least one, else 256-byte ones (2 rows)
    constexpr bool kXSlabs = kXBytes >= kWaves * 1024;
    constexpr int kXCopyBytes = kXSlabs ? 1024 : 256;
    constexpr int kXPerWave = kXBytes / kXCopyBytes / kWaves;
    static_assert(kXPerWave >= 1 && kXPerWave * kXCopyBytes * kWaves == kXBytes, "x tile must split over the waves");
    // tiles of 8 or more fragments per wave copy their metadata 4 k blocks at a time
    // (LM head 182 -> 175-177 us); smaller ones one k block at a time (qkv 12.4 us
    // against 13.3-13.7 us grouped)
    constexpr bool kGroupMeta = MR * CBW >= 8;
    constexpr int kDmaPerStage = kXPerWave + CBW + (kGroupMeta ? 0 : 1);   // + kMetaDma in a group's first stage
    constexpr int kMetaDma = kGroupMeta ? CBW : 0;
    constexpr int kStages = 3;
    using StageT = StageA8<BM, CBW, kWaves, kGroupMeta>;
    __shared__ StageT ring[kStages];
    using MetaT = MetaGroupA8<CBW>;
    static_assert(!kGroupMeta || sizeof(MetaT) == (size_t)kMetaDma * 256, "a group is whole 4-byte copies");
    __shared__ MetaT mring[kGroupMeta ? 2 : 1][kGroupMeta ? kWaves : 1];  // group g in slot g % 2

    const int id = blockIdx.x;
    const int local = id / kXcds;
    const int m_tile = local % tiles_m;
    const int rest = local / tiles_m;
    const int split = rest % splits;
    const int n_tile = (rest / splits) * kXcds + id % kXcds;
    if (n_tile >= tiles_n) return;

    const int KB = K / kRowsPerBlock;
    const int UW = (int)padded_units(K, kRowsPerBlock);
    const int Np = (int)padded_cols(N);
    const int NB = Np / kColsPerBlock;
    const int kb_begin = (int)((int64_t)KB * split / splits);
    const int kb_end = (int)((int64_t)KB * (split + 1) / splits);
    const int nkb = kb_end - kb_begin;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int c = lane & 15;
    const int h = lane >> 4;
    const int m0 = m_tile * BM;
    const int nbw = (n_tile * kWaves + w) * CBW;

    // activation copies: copy p of this wave covers tile rows (8 or 2 per copy);
    // rows past M read row M-1 (their outputs are not written)
    const uint8_t* xbase = uniform_ptr(act + (size_t)m0 * K);
    uint32_t xoff[kXPerWave];
#pragma unroll
    for (int t = 0; t < kXPerWave; ++t) {
        const int piece = w * kXPerWave + t;
        const int row = kXSlabs ? 8 * piece + (lane >> 3) : 2 * piece + (lane >> 5);
        const int chunk = kXSlabs ? (lane & 7) : ((lane & 31) >> 2);
        const int sub = kXSlabs ? 0 : 4 * (lane & 3);
        const int m = m0 + row < M ? m0 + row : M - 1;
        xoff[t] = (uint32_t)(m - m0) * (uint32_t)K + 16u * (uint32_t)(chunk ^ row_swizzle(row)) + (uint32_t)sub;
    }
    const int nbw0 = nbw < NB ? nbw : NB - 1;
    const uint8_t* wbase = uniform_ptr(packed + (size_t)nbw0 * KB * kBlockBytes);
    uint32_t woff[CBW];
#pragma unroll
    for (int j = 0; j < CBW; ++j) {
        const int nbj = nbw + j < NB ? nbw + j : NB - 1;
        woff[j] = (uint32_t)(nbj - nbw0) * (uint32_t)KB * kBlockBytes + 16u * (uint32_t)lane;
    }
    const uint32_t* meta_plane = reinterpret_cast<const uint32_t*>(packed + (size_t)K * Np / 2);
    // metadata copies: word 64 i + lane of copy i is column (64 i + lane) / 4 of the
    // wave and k block (64 i + lane) % 4 of the group (16 columns, so 16 cache lines, per
    // copy; ordered k block first it would be 32 lines per copy with two column blocks
    // per wave, measured slower); columns past the last read the last, blocks past the
    // column's last word read that word
    const int col0 = nbw * kColsPerBlock < Np ? nbw * kColsPerBlock : Np - kColsPerBlock;
    const uint8_t* mbase = uniform_ptr(meta_plane + (size_t)col0 * UW);
    const uint32_t ring_base = lds_addr(&ring[0]);
    const uint32_t mring_base = lds_addr(&mring[0][kGroupMeta ? w : 0]);

    // Operands of the zero-point term (one batch of at most 16 k blocks: the tile rows'
    // block sums and the tile columns' metadata words, 16 per row and column) are
    // copied into the ring slot that the last k blocks leave free, two k blocks before
    // the end, so the term's loads do not wait a memory latency after the loop.
    constexpr int kBN = 16 * CBW * kWaves;
    constexpr int kSumCopies = BM * 16 / 64 / kWaves;      // 4-byte copies per wave
    constexpr int kZMetaCopies = 16 * CBW * 16 / 64;       // a wave's own columns
    static_assert(kSumCopies >= 1 && kSumCopies * 64 * kWaves == BM * 16, "block sums must split over the waves");
    constexpr int kRsCopies = (BM + 63) / 64;               // row scales: 4-byte copies, waves 0 ..
    static_assert(kRsCopies <= kWaves, "one row-scale copy per wave at most");
    static_assert((size_t)(BM + kBN) * 64 + (size_t)kRsCopies * 256 <= sizeof(StageT),
                  "the zero-point operands and row scales fit one ring slot");
    // kZpStaged: chosen by the host where every K split has 8 to 16 blocks (every
    // row's and column's 16 words are copied, so with fewer k blocks the wasted copies
    // cost more than the latency; the other instantiation keeps the loads after the
    // loop, and its loop free of the staging code: both measured 2-3% slower otherwise)
    constexpr bool zp_staged = kZpStaged;
    // Word u of row (or column) rho of the staged operands sits at 16 rho + (u ^ sw(rho)),
    // sw from bits 2..3 of rho: unswizzled, lanes c, c + 4, c + 8, c + 12 of the term's
    // reads (rows 16 r + c) met the same banks. The bf16 pass reads block pairs
    // 8 q + 2 h + (0, 1) (sw on bits 2..3), the fp32 pass block 4 h + u (sw on bits 0..1):
    // the 32 lanes served together then hit distinct banks, whether 64 or 128 of them.
    constexpr bool kZpBf16 = MR * CBW >= 16;
    auto zsw = [](int rho) {
        const int k = (rho >> 2) & 3;
        return kZpBf16 ? 4 * k : k;
    };
    const int zp_issue = nkb - 2;                           // step after whose barrier they are copied
    const int zp_slot = nkb % kStages;                      // that of step nkb - 3, free from then on
    const uint8_t* sbase = uniform_ptr(block_sum + (size_t)m0 * KB);
    auto issue_zp = [&]() {
        const uint32_t st = ring_base + (uint32_t)zp_slot * (uint32_t)sizeof(StageT);
        // the copies' offsets are computed here, in the loop's one step that issues
        // them (hoisted out of the loop they would hold 16 registers through it)
        int ln = lane;
        asm volatile("" : "+v"(ln));
        // block sums: word g = 16 r + u of [BM][16] is row m0 + r (rows past M read row
        // M - 1) and block kb_begin + u (blocks past the split's end read its last:
        // they are weighed 0)
#pragma unroll
        for (int i = 0; i < kSumCopies; ++i) {
            const int g = (w * kSumCopies + i) * 64 + ln;
            const int r = g >> 4, u = (g & 15) ^ zsw(g >> 4);
            const int m = m0 + r < M ? m0 + r : M - 1;
            const int kb = kb_begin + u < kb_end ? kb_begin + u : kb_end - 1;
            dma4(sbase, ((uint32_t)(m - m0) * (uint32_t)KB + (uint32_t)kb) * 4u,
                 st + (uint32_t)((w * kSumCopies + i) * 64) * 4u);
        }
        // metadata: word 16 cl + u of this wave's 16 CBW columns (past the last: the last)
#pragma unroll
        for (int i = 0; i < kZMetaCopies; ++i) {
            const int g = i * 64 + ln;
            const int cl = g >> 4, u = (g & 15) ^ zsw(cl);      // tile column 16 w CBW + cl
            const int n = nbw * kColsPerBlock + cl < Np ? nbw * kColsPerBlock + cl : Np - 1;
            const int kb = kb_begin + u < kb_end ? kb_begin + u : kb_end - 1;
            dma4(mbase, ((uint32_t)(n - col0) * (uint32_t)UW + (uint32_t)kb) * 4u,
                 st + (uint32_t)(BM * 64 + (w * 16 * CBW * 16 + i * 64) * 4));
        }
        // the tile rows' scales (rows past M read row M - 1), for the epilogue
        if (w < kRsCopies) {
            const int r = w * 64 + ln;
            const int m = m0 + r < M ? m0 + r : M - 1;
            dma4(uniform_ptr(row_scale), (uint32_t)m * 4u, st + (uint32_t)((BM + kBN) * 64 + w * 256));
        }
    };
    const int ncol = nbw * kColsPerBlock + (lane < 16 * CBW ? lane : 0);   // per-stage copies
    const uint32_t moff = (uint32_t)((ncol < Np ? ncol : Np - 1) - col0) * (uint32_t)UW * 4u;

    // stage t (k block kb_begin + t); a group's first stage also copies the group's
    // metadata into slot (t / 4) % 2
    auto issue = [&](int slot, int t) {
        const int kb = kb_begin + t;
        const uint32_t st = ring_base + (uint32_t)slot * (uint32_t)sizeof(StageT);
#pragma unroll
        for (int t = 0; t < kXPerWave; ++t) {
            const uint32_t dst = st + (uint32_t)offsetof(StageT, x) + (uint32_t)((w * kXPerWave + t) * kXCopyBytes);
            if constexpr (kXSlabs) dma16(xbase + (size_t)kb * kRowsPerBlock, xoff[t], dst);
            else dma4(xbase + (size_t)kb * kRowsPerBlock, xoff[t], dst);
        }
#pragma unroll
        for (int j = 0; j < CBW; ++j)
            dma16(wbase + (size_t)kb * kBlockBytes, woff[j],
                  st + (uint32_t)offsetof(StageT, w) + (uint32_t)(w * CBW + j) * 1024u);
        if constexpr (!kGroupMeta)
            dma4(mbase + (size_t)kb * 4, moff, st + (uint32_t)offsetof(StageT, meta) + (uint32_t)w * 256u);
        if (kGroupMeta && (t & 3) == 0) {
            const uint32_t dst = mring_base + (uint32_t)((t >> 2) & 1) * (uint32_t)(kWaves * sizeof(MetaT));
#pragma unroll
            for (int i = 0; i < kMetaDma; ++i) {
                const int wi = 64 * i + lane;
                const int cl = wi >> 2, u = wi & 3;
                const int n = nbw * kColsPerBlock + cl < Np ? nbw * kColsPerBlock + cl : Np - 1;
                const int ua = kb + u < UW ? kb + u : UW - 1;
                dma4(mbase, ((uint32_t)(n - col0) * (uint32_t)UW + (uint32_t)ua) * 4u, dst + (uint32_t)i * 256u);
            }
        }
    };

    f32x4 acc[MR][CBW];
#pragma unroll
    for (int r = 0; r < MR; ++r)
#pragma unroll
        for (int j = 0; j < CBW; ++j) acc[r][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (nkb > 0) issue(0, 0);
    if (nkb > 1) issue(1, 1);
    for (int t = 0; t < nkb; ++t) {
        // leave step t+1's copies in flight (its metadata copies too when it starts a
        // group); a group's metadata slot is refilled at step 4g + 6, after every wave
        // has passed the group's last step 4g + 3
        if (t + 1 >= nkb) wait_vmcnt<0>();
        else if (((t + 1) & 3) == 0) wait_vmcnt<kDmaPerStage + kMetaDma>();
        else wait_vmcnt<kDmaPerStage>();
        lds_barrier();
        if (t + 2 < nkb) issue((t + 2) % kStages, t + 2);
        else if constexpr (zp_staged) {
            if (t == zp_issue) issue_zp();
        }

        const StageT& st = ring[t % kStages];
        // 512 s for this lane's 4 columns of each column block
        float sc[CBW][4];
        i32x8 b[CBW];
#pragma unroll
        for (int j = 0; j < CBW; ++j) {
            if constexpr (kGroupMeta) {
                const uint32_t* mw = &mring[(t >> 2) & 1][w].words[(16 * j + 4 * h) * 4 + (t & 3)];
#pragma unroll
                for (int e = 0; e < 4; ++e) sc[j][e] = 512.f * half_bits_to_f32<kBF16>(mw[4 * e] & 0xFFFFu);
            } else {
                const uint4 md = *reinterpret_cast<const uint4*>(&st.meta[w * 64 + 16 * j + 4 * h]);
                sc[j][0] = 512.f * half_bits_to_f32<kBF16>(md.x & 0xFFFFu);
                sc[j][1] = 512.f * half_bits_to_f32<kBF16>(md.y & 0xFFFFu);
                sc[j][2] = 512.f * half_bits_to_f32<kBF16>(md.z & 0xFFFFu);
                sc[j][3] = 512.f * half_bits_to_f32<kBF16>(md.w & 0xFFFFu);
            }
            // codes -> E4M3 bytes q * 2^-9: word i gives bytes 8 i .. 8 i + 7 (rows 0,4,1,5 | 2,6,3,7)
            const uint4 wq = st.w[(w * CBW + j) * 64 + lane];
            b[j] = i32x8{(int)(wq.x & 0x0F0F0F0Fu), (int)((wq.x >> 4) & 0x0F0F0F0Fu),
                         (int)(wq.y & 0x0F0F0F0Fu), (int)((wq.y >> 4) & 0x0F0F0F0Fu),
                         (int)(wq.z & 0x0F0F0F0Fu), (int)((wq.z >> 4) & 0x0F0F0F0Fu),
                         (int)(wq.w & 0x0F0F0F0Fu), (int)((wq.w >> 4) & 0x0F0F0F0Fu)};
        }
#pragma unroll
        for (int r = 0; r < MR; ++r) {
            // row 16 r + c, bytes 32 h .. 32 h + 31 of the block: chunks 2h, 2h+1
            // (row_swizzle(16 r + c) = row_swizzle(c))
            const int row = 16 * r + c;
            const uint4 a0 = st.x[row * 8 + ((2 * h) ^ row_swizzle(c))];
            const uint4 a1 = st.x[row * 8 + ((2 * h + 1) ^ row_swizzle(c))];
            const i32x8 a = i32x8{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                                  (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
#pragma unroll
            for (int j = 0; j < CBW; ++j) {
                const f32x4 d = mfma_fp8(b[j], a);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[r][j][e] = fmaf(sc[j][e], d[e], acc[r][j][e]);
            }
        }
    }

    // zero-point term over this split's blocks: acc -= sum_kb (s z)[kb, n] * X[m, kb].
    // One batch of 8 to 16 blocks, its operands in the ring (copied during the loop,
    // landed by its last barrier). Tiles of 16 or more fragments per wave run it on the
    // bf16 matrix cores (smaller ones measured slower that way: qkv 11.6 -> 12.4 us, the
    // splitting outweighs the saved MFMA time, so they take the fp32 16x16x4 MFMA of
    // the unstaged path, on the staged operands): -s z has at most 12
    // significant bits (s 8 or 11, z 4), so it is exactly the sum of two bf16 values
    // (checked for every finite scale and zero point), and X is split the same way (the
    // rest, below 2^-17 of X, is dropped); a block then contributes the four exact
    // products of the parts, summed in fp32. In 16x16x32 MFMA q, lane group h takes
    // blocks 8 q + 2 h and 8 q + 2 h + 1, k = 4 (block) + 2 a + b holding X part a and
    // s z part b: two MFMAs per fragment instead of four fp32 16x16x4 ones, each of
    // which costs as much as four 16-bit ones.
    if constexpr (zp_staged && kZpBf16) {
        const uint8_t* zb = reinterpret_cast<const uint8_t*>(&ring[zp_slot]);
        const int sw = zsw(c);                               // rows 16 r + c, columns 16 j' + c
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int kb0 = 8 * q + 2 * h;                   // this lane's blocks kb0, kb0 + 1
            const int pos = kb0 ^ sw;                        // where the pair sits in its row
            uint4 av[CBW];                                   // per block (sz1, sz2, sz1, sz2)
#pragma unroll
            for (int j = 0; j < CBW; ++j) {
                const uint2 md = *reinterpret_cast<const uint2*>(zb + BM * 64 + ((16 * (w * CBW + j) + c) * 16 + pos) * 4);
                const float s0 = kb0 < nkb ? -half_bits_to_f32<kBF16>(md.x & 0xFFFFu) * (float)((md.x >> 16) & 0xFu) : 0.f;
                const float s1 = kb0 + 1 < nkb ? -half_bits_to_f32<kBF16>(md.y & 0xFFFFu) * (float)((md.y >> 16) & 0xFu) : 0.f;
                const uint32_t p0 = bf16_split(s0), p1 = bf16_split(s1);
                av[j] = make_uint4(p0, p0, p1, p1);
            }
#pragma unroll
            for (int r = 0; r < MR; ++r) {
                const float2 xv = *reinterpret_cast<const float2*>(zb + ((16 * r + c) * 16 + pos) * 4);
                uint32_t x1a, x2a, x1b, x2b;                 // per block (X1, X1) and (X2, X2)
                bf16_split_dup(xv.x, x1a, x2a);
                bf16_split_dup(xv.y, x1b, x2b);
                const uint4 bv = make_uint4(x1a, x2a, x1b, x2b);
#pragma unroll
                for (int j = 0; j < CBW; ++j) acc[r][j] = mfma16x16x32<true>(av[j], bv, acc[r][j]);
            }
        }
    }
    if constexpr (zp_staged && !kZpBf16) {
        // in 16x16x4 fp32 MFMA u, lane group h takes block 4 h + u
        const uint8_t* zb = reinterpret_cast<const uint8_t*>(&ring[zp_slot]);
        const int sw = zsw(c);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int kb = 4 * h + u;
            const int pos = kb ^ sw;
            float zs[CBW], xs[MR];
#pragma unroll
            for (int j = 0; j < CBW; ++j) {
                const uint32_t md = *reinterpret_cast<const uint32_t*>(zb + BM * 64 + ((16 * (w * CBW + j) + c) * 16 + pos) * 4);
                zs[j] = kb < nkb ? -half_bits_to_f32<kBF16>(md & 0xFFFFu) * (float)((md >> 16) & 0xFu) : 0.f;
            }
#pragma unroll
            for (int r = 0; r < MR; ++r) xs[r] = *reinterpret_cast<const float*>(zb + ((16 * r + c) * 16 + pos) * 4);
#pragma unroll
            for (int r = 0; r < MR; ++r)
#pragma unroll
                for (int j = 0; j < CBW; ++j)
                    acc[r][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(zs[j], xs[r], acc[r][j], 0, 0, 0);
        }
    }
    // More batches: from global memory. A lane's four blocks are consecutive, so where
    // they are 16-byte aligned its four block sums of a row and four metadata words of a
    // column come in one load each (18 loads per batch instead of 72 4-byte ones), all
    // issued before the batch's MFMAs.
    for (int t0 = kb_begin; !zp_staged && t0 < kb_end; t0 += 16) {
        const int kb4 = t0 + 4 * h;
        const bool vec = ((KB | kb4) & 3) == 0 && kb4 + 3 < kb_end;    // UW % 4 == 0 always
        float zs[4][CBW], xs[4][MR];
#pragma unroll
        for (int j = 0; j < CBW; ++j) {
            int n = (nbw + j) * kColsPerBlock + c;
            n = n < Np ? n : Np - 1;
            uint32_t md[4];
            if (vec) {
                const uint4 v = *reinterpret_cast<const uint4*>(meta_plane + (size_t)n * UW + kb4);
                md[0] = v.x; md[1] = v.y; md[2] = v.z; md[3] = v.w;
            } else {
#pragma unroll
                for (int u = 0; u < 4; ++u) md[u] = kb4 + u < kb_end ? meta_plane[(size_t)n * UW + kb4 + u] : 0u;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                zs[u][j] = kb4 + u < kb_end ? -half_bits_to_f32<kBF16>(md[u] & 0xFFFFu) * (float)((md[u] >> 16) & 0xFu) : 0.f;
        }
#pragma unroll
        for (int r = 0; r < MR; ++r) {
            const int m = m0 + 16 * r + c < M ? m0 + 16 * r + c : M - 1;
            if (vec) {
                const float4 v = *reinterpret_cast<const float4*>(block_sum + (size_t)m * KB + kb4);
                xs[0][r] = v.x; xs[1][r] = v.y; xs[2][r] = v.z; xs[3][r] = v.w;
            } else {
#pragma unroll
                for (int u = 0; u < 4; ++u) xs[u][r] = kb4 + u < kb_end ? block_sum[(size_t)m * KB + kb4 + u] : 0.f;
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int r = 0; r < MR; ++r)
#pragma unroll
                for (int j = 0; j < CBW; ++j)
                    acc[r][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(zs[u][j], xs[u][r], acc[r][j], 0, 0, 0);
    }

    // the row scales of this lane's rows: staged ones from the ring now, before the
    // epilogue writes its output tile over it (the others after the barrier below)
    float rs[MR];
    if constexpr (zp_staged) {
#pragma unroll
        for (int r = 0; r < MR; ++r)
            rs[r] = *reinterpret_cast<const float*>(reinterpret_cast<const uint8_t*>(&ring[zp_slot]) +
                                                    (BM + kBN) * 64 + (16 * r + c) * 4);
    }

    // (tiles of more than 16 fragments per wave are only planned for outputs that need no
    // K split: their reduction would not fit in registers)
    if constexpr (MR * CBW <= 16) {
        if (splits > 1 && !reduce_splits<MR, CBW, kWaves>(acc, counters, partials, m_tile * tiles_n + n_tile, split,
                                                           splits))
            return;
    }

    // Epilogue through LDS: the lanes write their rounded outputs (4 adjacent columns
    // of one row each) into the free ring as a row-major [BM][BN] tile, rows padded by
    // 16 bytes (16 rows of a fragment then fall on different banks), and the waves then
    // store whole rows, 16 bytes per lane and 1 KiB per instruction. (Stored straight
    // from the fragments, each wave wrote half of every 128-byte line it touched, and
    // lines evicted between the two halves were written twice: 1.49x the output
    // bytes on the LM head.)
    constexpr int BN = 16 * CBW * kWaves;
    constexpr int kRowBytes = BN * 2 + 16;
    static_assert((size_t)BM * kRowBytes <= kStages * sizeof(StageT), "the output tile fits in the ring");
    uint8_t* otile = reinterpret_cast<uint8_t*>(&ring[0]);
    lds_barrier();                           // every wave is done with the ring's operands
    if constexpr (!zp_staged) {
#pragma unroll
        for (int r = 0; r < MR; ++r) rs[r] = m0 + 16 * r + c < M ? row_scale[m0 + 16 * r + c] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < CBW; ++j) {
        const int col = 16 * (w * CBW + j) + 4 * h;        // in the tile
        const int n = (nbw + j) * kColsPerBlock + 4 * h;   // in y
        float bv[4] = {0.f, 0.f, 0.f, 0.f};
        if (bias && n < N) {
#pragma unroll
            for (int e = 0; e < 4; ++e) bv[e] = half_bits_to_f32<kBF16>(bias[n + e]);
        }
#pragma unroll
        for (int r = 0; r < MR; ++r) {
            const float a = rs[r];
            const f32x4 v = acc[r][j];
            const uint2 o = make_uint2(pack2_rne<kBF16>(fmaf(a, v[0], bv[0]), fmaf(a, v[1], bv[1])),
                                       pack2_rne<kBF16>(fmaf(a, v[2], bv[2]), fmaf(a, v[3], bv[3])));
            *reinterpret_cast<uint2*>(otile + (16 * r + c) * kRowBytes + 2 * col) = o;
        }
    }
    __syncthreads();
    // rows past M and columns past N (the zero padding of a last half block, whole
    // column blocks past the last) are not stored; N % 8 == 0, so a 16-byte chunk of 8
    // columns lies wholly inside or outside
    const int n0 = n_tile * BN;
    for (int q = tid; q < BM * (BN / 8); q += 64 * kWaves) {
        const int row = q / (BN / 8);
        const int ch = q - row * (BN / 8);
        const int m = m0 + row, n = n0 + 8 * ch;
        if (m < M && n < N)
            store_out16(y + (size_t)m * N + n, *reinterpret_cast<const uint4*>(otile + row * kRowBytes + 16 * ch), nt_out != 0);
    }
}

template <bool kBF16, int MR, int CBW, int W>
void launch_cfg(const GemmPlan& p, const W4A8Act& a, const uint8_t* packed, const uint16_t* bias, uint16_t* y,
                int M, int K, int N, uint32_t* counters, float* partials, hipStream_t stream) {
    const int tiles_n_pad = (p.tiles_n + kXcds - 1) / kXcds * kXcds;
    const dim3 grid((unsigned)(p.tiles_m * p.splits * tiles_n_pad));
    // zero-point operands staged in the ring where every split has 8 to 16 k blocks
    const int KB = K / kRowsPerBlock;
    const bool staged = KB / p.splits >= 8 && (KB + p.splits - 1) / p.splits <= 16;
    // streaming output stores when every workgroup runs in the first round (qkv 11.7 ->
    // 11.5 us, gate_up 24.6 -> 23.7 us; the LM head, 4 rounds, keeps ordinary stores)
    const int nt_out = (int64_t)p.tiles_m * p.tiles_n * p.splits <= 256 ? 1 : 0;
    if (staged)
        hipLaunchKernelGGL((w4a8_gemm_kernel<kBF16, MR, CBW, W, true>), grid, dim3(64 * W), 0, stream, a.codes,
                           a.row_scale, a.block_sum, packed, bias, y, M, K, N, p.tiles_m, p.tiles_n, p.splits, counters,
                           partials, nt_out);
    else
        hipLaunchKernelGGL((w4a8_gemm_kernel<kBF16, MR, CBW, W, false>), grid, dim3(64 * W), 0, stream, a.codes,
                           a.row_scale, a.block_sum, packed, bias, y, M, K, N, p.tiles_m, p.tiles_n, p.splits, counters,
                           partials, nt_out);
}

template <bool kBF16, int MR>
void launch_mr(const GemmPlan& p, const W4A8Act& a, const uint8_t* packed, const uint16_t* bias, uint16_t* y,
               int M, int K, int N, uint32_t* counters, float* partials, hipStream_t stream) {
    if constexpr (MR == 16) {
        launch_cfg<kBF16, 16, 2, 8>(p, a, packed, bias, y, M, K, N, counters, partials, stream);
    } else {
        if constexpr (MR >= 4) {
            if (p.waves == 8 && p.cbw == 1) {
                launch_cfg<kBF16, MR, 1, 8>(p, a, packed, bias, y, M, K, N, counters, partials, stream);
                return;
            }
        }
        if constexpr (MR >= 2) {
            if (p.waves == 8) {
                launch_cfg<kBF16, MR, 2, 8>(p, a, packed, bias, y, M, K, N, counters, partials, stream);
                return;
            }
        }
        if (p.cbw == 4) launch_cfg<kBF16, MR, 4, 4>(p, a, packed, bias, y, M, K, N, counters, partials, stream);
        else if (p.cbw == 2) launch_cfg<kBF16, MR, 2, 4>(p, a, packed, bias, y, M, K, N, counters, partials, stream);
        else launch_cfg<kBF16, MR, 1, 4>(p, a, packed, bias, y, M, K, N, counters, partials, stream);
    }
}

template <bool kBF16>
void launch_typed(const GemmPlan& p, const W4A8Act& a, const uint8_t* packed, const uint16_t* bias, uint16_t* y,
                  int M, int K, int N, uint32_t* counters, float* partials, hipStream_t stream) {
    if (p.mr == 1) launch_mr<kBF16, 1>(p, a, packed, bias, y, M, K, N, counters, partials, stream);
    else if (p.mr == 2) launch_mr<kBF16, 2>(p, a, packed, bias, y, M, K, N, counters, partials, stream);
    else if (p.mr == 4) launch_mr<kBF16, 4>(p, a, packed, bias, y, M, K, N, counters, partials, stream);
    else if (p.mr == 8) launch_mr<kBF16, 8>(p, a, packed, bias, y, M, K, N, counters, partials, stream);
    else launch_mr<kBF16, 16>(p, a, packed, bias, y, M, K, N, counters, partials, stream);
}

// The 16-bit GEMM's plan, except that outputs with at least two rounds of 256 x 256
// tiles over the CUs take that tile (8 waves of 16 fragments each): the activation
// and weight copies per output element, which bound this kernel (a run without the
// MFMA work takes ~85% of the full time on the LM head), drop by a quarter.
// Such outputs never split K.
GemmPlan plan_w4a8(int64_t M, int64_t K, int64_t N, int64_t G) {
    GemmPlan p = plan_gemm(M, K, N, G);
    const int64_t NB = padded_cols(N) / kColsPerBlock;
    const int64_t tm = (M + 255) / 256, tn = (NB + 15) / 16;
    if (tm * tn >= 2 * kTilesPerRound) {
        p.mr = 16;
        p.cbw = 2;
        p.waves = 8;
        p.tiles_m = (int)tm;
        p.tiles_n = (int)tn;
        p.splits = 1;
        p.workspace_bytes = 0;
    }
    return p;
}

}  // namespace

hipError_t launch_w4a8_quantize(const uint16_t* x, int64_t M, int64_t K, bool bf16, const W4A8Act& a,
                                hipStream_t stream) {
    const dim3 grid((unsigned)M), block(kQuantThreads);
    if (bf16)
        hipLaunchKernelGGL(quantize_kernel<true>, grid, block, 0, stream, x, a.codes, a.row_scale, a.block_sum, (int)K);
    else
        hipLaunchKernelGGL(quantize_kernel<false>, grid, block, 0, stream, x, a.codes, a.row_scale, a.block_sum, (int)K);
    return hipGetLastError();
}

hipError_t launch_w4a8_gemm(const W4A8Act& a, const uint8_t* packed, const uint16_t* bias, uint16_t* y, int64_t M,
                            int64_t K, int64_t N, int64_t G, bool bf16, void* workspace, hipStream_t stream) {
    const GemmPlan p = plan_w4a8(M, K, N, G);
    uint32_t* counters = static_cast<uint32_t*>(workspace);
    float* partials = nullptr;
    if (p.splits > 1) {
        partials = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + kSplitCounterBytes);
    }
    if (bf16) launch_typed<true>(p, a, packed, bias, y, (int)M, (int)K, (int)N, counters, partials, stream);
    else launch_typed<false>(p, a, packed, bias, y, (int)M, (int)K, (int)N, counters, partials, stream);
    return hipGetLastError();
}

}  // namespace w4a16
