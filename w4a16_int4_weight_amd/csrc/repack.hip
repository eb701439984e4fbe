// One-time repack of AWQ int32 nibble packing into the packed tile layout.
//
// The AWQ checkpoint stores codes packed along the output dimension, eight per
// int32 but not in ascending column order, and vLLM reorders them once after loading (note
// "Carga de capas cuantizadas: AWQ / GPTQ / Marlin / fp8", sections "Motivación de
// diseño" and "Flujo de datos"). Here that reorder is a single coalesced pass on the
// GPU: no int32 expansion of the codes is ever materialised (the CPU path of the
// vllm-omni commit "cpu_int4: repack weights in n-blocks ..." shows that transient
// reaching 1 GiB for a 131072 x 2048 head).
//
// The reorder is an 8 x 8 transpose of 4-bit elements. Eight AWQ words of one word
// column (8 output columns) and 8 consecutive rows hold nibble (row r, AWQ slot s);
// a tile word holds one column and 8 rows. Transposing the 8 words in registers
// (swap 16-bit halves, then bytes, then nibbles: three stages of pairwise swaps)
// gives word s = the 8 rows of the column in AWQ slot s. Both orders are folded in
// for free: feeding the rows in tile slot order makes nibble s' of every result hold
// row tile_row_of_slot(s'), and the column t result is result word
// awq_slot_of_column(t).
//
// Work split: workgroup = 128-row block kb x 64 AWQ words (512 columns); thread
// (word j, lane group h) transposes rows 32 i + 8 h + 0..7 for i = 0..3 and places,
// for each of its 8 columns, the 16-byte chunk of lane (column % 16) + 16 h in LDS;
// the workgroup then writes its 32 blocks whole. Wave h reads 64 consecutive words
// (256 bytes) of one row per load instruction. The tile's metadata rows are dealt
// to its row-block workgroups and written whole (1 KiB per wave store).
#include "device_common.h"
#include "launch.h"

namespace w4a16 {
namespace {

constexpr int kWordsPerTile = 64;                    // AWQ words (8 columns each) per workgroup
constexpr int kRepackThreads = kWordsPerTile * 4;    // x 4 lane groups

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Every checkpoint word is read once and every packed byte written once, so both
// streams are nontemporal: on the 131072 x 2048 head, nontemporal code stores took
// the AWQ repack from 61.6 to 57.0 us, nontemporal loads as well to 50.7 us
// (bit-identical output; the metadata rows gained nothing from it).
__device__ __forceinline__ uint32_t load_nt(const uint32_t* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void store_nt(uint4* p, const uint4 v) {
    __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(p));
}

// 8 x 8 transpose of nibbles: on return nibble r of word s = nibble s of word r on entry.
__device__ __forceinline__ void transpose8x8_nibbles(uint32_t (&v)[8]) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {            // 4x4 blocks: 16-bit halves
        const uint32_t a = v[r], b = v[r + 4];
        v[r] = (a & 0x0000FFFFu) | (b << 16);
        v[r + 4] = (a >> 16) | (b & 0xFFFF0000u);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {            // 2x2 blocks: bytes within halves
        const int r = (q & 1) + 4 * (q >> 1);
        const uint32_t a = v[r], b = v[r + 2];
        v[r] = (a & 0x00FF00FFu) | ((b & 0x00FF00FFu) << 8);
        v[r + 2] = ((a >> 8) & 0x00FF00FFu) | (b & 0xFF00FF00u);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {            // single nibbles within bytes
        const int r = 2 * q;
        const uint32_t a = v[r], b = v[r + 1];
        v[r] = (a & 0x0F0F0F0Fu) | ((b & 0x0F0F0F0Fu) << 4);
        v[r + 1] = ((a >> 4) & 0x0F0F0F0Fu) | (b & 0xF0F0F0F0u);
    }
}

// XOR applied to a chunk's lane index in the LDS staging of block b (b < 32, so the
// result stays in 0..63): the 32 blocks one store instruction touches then map a lane
// to 32 different 16-byte slots of a 512-byte bank span, two lanes per slot.
__device__ __forceinline__ int stage_swizzle(int b) { return b & 31; }

// Metadata rows of columns [c0, c0 + cols) of the input tensors (padding columns of
// a last half block included), written whole: the columns are dealt to the KB
// workgroups of row blocks kb = 0 .. KB-1 of one column tile, and a thread writes one
// 16-byte chunk (4 consecutive unit words: scale bits | zero << 16 per unit of
// min(G, 128) rows, zero past the last unit and for padding columns) of one column's
// row, so a wave stores 1 KiB of consecutive rows. (Rows written in 4- or 16-byte
// pieces strided over many lines left partial lines to HBM: ~12 us on the LM head.)
// kAwq: qzeros in AWQ slot order, else in standard order, both packed along N.
template <bool kAwq>
__device__ __forceinline__ void write_metadata_rows(const uint32_t* __restrict__ qzeros,
                                                    const uint16_t* __restrict__ scales, uint8_t* __restrict__ packed,
                                                    int64_t K, int64_t N, int64_t G, int64_t n0, int64_t Nt,
                                                    int64_t c0, int cols, int64_t kb, int tid, int nthreads) {
    const int64_t KB = K / kRowsPerBlock;
    const int sub = units_per_block(G);
    const int64_t Gu = kRowsPerBlock / sub;                       // rows per unit
    const int64_t U = KB * sub;
    const int cpr = (int)(padded_units(K, G) / 4);                // 16-byte chunks per row
    const int cpw = (int)((cols + KB - 1) / KB);                  // columns per workgroup
    const int c_begin = kb * cpw < cols ? (int)(kb * cpw) : cols;
    const int c_end = c_begin + cpw < cols ? c_begin + cpw : cols;
    uint4* meta4 = reinterpret_cast<uint4*>(packed + K * padded_cols(Nt) / 2);
    for (int q = tid; q < (c_end - c_begin) * cpr; q += nthreads) {
        const int r = q / cpr;
        const int p4 = q - r * cpr;
        const int64_t n = c0 + c_begin + r;                       // column of the input tensors
        const bool real = n < N;
        const int zshift = 4 * (kAwq ? awq_slot_of_column((int)(n & 7)) : (int)(n & 7));
        uint32_t word[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t b = 4 * p4 + e;
            word[e] = 0u;
            if (real && b < U) {
                const int64_t g = (b * Gu) / G;
                const uint32_t z = (qzeros[g * (N / 8) + (n >> 3)] >> zshift) & 0xFu;
                word[e] = (uint32_t)scales[g * N + n] | (z << 16);
            }
        }
        meta4[(n0 + n) * cpr + p4] = make_uint4(word[0], word[1], word[2], word[3]);
    }
}

// Input tensors hold columns [n0, n0 + N) of a K x Nt weight (the whole weight when
// n0 = 0 and N = Nt): qweight [K, N/8], qzeros [K/G, N/8], scales [K/G, N]. Output:
// those columns' blocks and metadata rows in the packed layout of the K x Nt weight.
__global__ __launch_bounds__(kRepackThreads) void repack_kernel(
    const uint32_t* __restrict__ qweight, const uint32_t* __restrict__ qzeros,
    const uint16_t* __restrict__ scales, uint8_t* __restrict__ packed,
    int64_t K, int64_t N, int64_t G, int64_t n0, int64_t Nt) {
    const int64_t KB = K / kRowsPerBlock;
    const int64_t words_per_row = N / 8;
    // row blocks vary fastest over the grid: the workgroups running together write
    // whole column blocks (each column block's K range is contiguous in the layout)
    const int64_t kb = blockIdx.x % KB;
    const int64_t j0 = (int64_t)(blockIdx.x / KB) * kWordsPerTile;     // first AWQ word of the tile
    const int tid = threadIdx.x;
    const int jl = tid & (kWordsPerTile - 1);
    const int h = tid / kWordsPerTile;                            // lane group (wave) 0..3
    const int64_t j = j0 + jl;
    const bool active = j < words_per_row;
    const int64_t jc = active ? j : words_per_row - 1;            // clamped: loads stay in bounds

    const int64_t tile_words = words_per_row - j0 < kWordsPerTile ? words_per_row - j0 : kWordsPerTile;
    const int nblk = (int)((tile_words + 1) / 2);                 // a last half block included

    // 1. rows 128 kb + 32 i + 8 h + e of word column jc, fed in tile slot order
    uint32_t t[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t* src = qweight + (kb * kRowsPerBlock + 32 * i + 8 * h) * words_per_row + jc;
#pragma unroll
        for (int s = 0; s < 8; ++s) t[i][s] = load_nt(src + (int64_t)tile_row_of_slot(s) * words_per_row);
    }
    // 2. transpose: t[i][s] = column in AWQ slot s, its 8 rows in tile slot order
#pragma unroll
    for (int i = 0; i < 4; ++i) transpose8x8_nibbles(t[i]);

    // 3. column 8 j + c8 -> block (j / 2), lane (8 (j % 2) + c8) + 16 h: words i = 0..3.
    //    The tile's 32 blocks are assembled in LDS and written out whole, each wave
    //    storing contiguous 1 KiB blocks.
    //    With N % 16 == 8 the last block has one word: its other 8 columns are zero.
    //    In LDS, chunk `lane` of block b sits at b * 64 + (lane ^ stage_swizzle(b)): the
    //    64 threads of one store instruction write one chunk into each of 32 blocks,
    //    1 KiB apart, which unswizzled would all fall on the same banks (32-way
    //    conflicts measured); the XOR spreads them over 32 different 16-byte bank
    //    groups, and each block stays a permutation of its own 64 chunks.
    __shared__ uint4 stage[kWordsPerTile / 2 * 64];
#pragma unroll
    for (int c8 = 0; c8 < 8; ++c8) {
        const int s = awq_slot_of_column(c8);
        const int b = jl >> 1;
        const int lane = 8 * (jl & 1) + c8 + 16 * h;
        stage[b * 64 + (lane ^ stage_swizzle(b))] =
            active ? make_uint4(t[0][s], t[1][s], t[2][s], t[3][s]) : make_uint4(0, 0, 0, 0);
    }
    __syncthreads();
    for (int q = tid; q < nblk * 64; q += kRepackThreads) {
        const int b = q >> 6;
        const int64_t nb = n0 / kColsPerBlock + (j0 >> 1) + b;
        store_nt(reinterpret_cast<uint4*>(packed + (nb * KB + kb) * kBlockBytes) + (q & 63),
                 stage[b * 64 + ((q & 63) ^ stage_swizzle(b))]);
    }

    // 4. the tile's metadata rows, dealt to its row-block workgroups
    write_metadata_rows<true>(qzeros, scales, packed, K, N, G, n0, Nt, j0 * 8, nblk * kColsPerBlock, kb, tid,
                              kRepackThreads);
}

// ---- GPTQ-standard input: codes packed along K ----
//
// GPTQ-style packing runs along the input dimension in standard bit order (vLLM
// note "Carga de capas cuantizadas", section "Motivación de diseño", on converting
// AWQ to the GPTQ style the Marlin kernel takes): qweight int32 [K/8, N], word
// (i, n) holding rows 8 i + j of column n in nibble j; qzeros int32 [K/G, N/8]
// packed along N, nibble j = column 8 w + j. A tile word holds the same 8 rows of
// one column (rows 32 w + 8 h + 0..7 of a row block, word w of lane c + 16 h), with
// row e in nibble slot s where e = tile_row_of_slot(s): even rows in the low half,
// odd rows in the high half. So each tile word is one GPTQ word with its nibbles
// unzipped, and no transpose is needed. The workgroup stages its row block's 16 GPTQ
// rows of its columns in LDS with 16-byte loads (on the 131072 x 2048 head 64.3 ->
// 53.0 us against each thread loading its 16 words with 4-byte loads), then each
// thread unzips one column's words and writes its 4 tile chunks.
constexpr int kGptqColumns = 256;    // columns per workgroup, one per thread

// nibbles 0,2,4,6 of v -> nibbles 0..3, nibbles 1,3,5,7 -> nibbles 4..7
__device__ __forceinline__ uint32_t unzip_nibbles(uint32_t v) {
    uint32_t e = v & 0x0F0F0F0Fu;            // even nibbles, one per byte
    uint32_t o = (v >> 4) & 0x0F0F0F0Fu;     // odd nibbles
    e = (e | (e >> 4)) & 0x00FF00FFu;
    o = (o | (o >> 4)) & 0x00FF00FFu;
    e = (e | (e >> 8)) & 0x0000FFFFu;
    o = (o | (o >> 8)) & 0x0000FFFFu;
    return e | (o << 16);
}

// Input columns [n0, n0 + N) of a K x Nt weight, as for repack_kernel: qweight
// [K/8, N], qzeros [K/G, N/8], scales [K/G, N].
__global__ __launch_bounds__(kGptqColumns) void repack_gptq_kernel(
    const uint32_t* __restrict__ qweight, const uint32_t* __restrict__ qzeros,
    const uint16_t* __restrict__ scales, uint8_t* __restrict__ packed,
    int64_t K, int64_t N, int64_t G, int64_t n0, int64_t Nt) {
    const int64_t KB = K / kRowsPerBlock;
    // column tiles vary fastest over the grid: the workgroups running together read
    // long stretches of the same GPTQ rows (the other order measured ~2% slower here)
    const int64_t tiles = (padded_cols(N) + kGptqColumns - 1) / kGptqColumns;
    const int64_t kb = blockIdx.x / tiles;
    const int64_t c0 = (int64_t)(blockIdx.x % tiles) * kGptqColumns;
    const int64_t n = c0 + threadIdx.x;
    const int64_t Np = padded_cols(N);
    // the row block's 16 GPTQ rows of the tile's columns, staged in LDS with 16-byte
    // loads (64 lanes read 1 KiB of one row); columns past N (a last half block's
    // padding) hold 0
    __shared__ __attribute__((aligned(16))) uint32_t rows[16][kGptqColumns];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int f = q * kGptqColumns + (int)threadIdx.x;
        const int r = f >> 6;
        const int cc = (f & 63) * 4;
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (c0 + cc < N)       // N % 8 == 0: the 4 columns lie wholly inside or outside
            v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(qweight + (16 * kb + r) * N + c0 + cc));
        *reinterpret_cast<u32x4*>(&rows[r][cc]) = v;
    }
    __syncthreads();
    if (n < Np) {
        const int64_t nb = (n0 + n) / kColsPerBlock;
        const int c = (int)(n % kColsPerBlock);
        uint4* blk = reinterpret_cast<uint4*>(packed + (nb * KB + kb) * kBlockBytes);
        // GPTQ word row i = 16 kb + 4 w + h: lane group h, word w of the tile
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            uint32_t t[4];
#pragma unroll
            for (int w = 0; w < 4; ++w) t[w] = unzip_nibbles(rows[4 * w + h][threadIdx.x]);
            store_nt(blk + c + 16 * h, make_uint4(t[0], t[1], t[2], t[3]));
        }
    }
    // the metadata rows of the workgroup's columns, dealt to its row-block workgroups
    const int cols = (int)(Np - c0 < kGptqColumns ? Np - c0 : kGptqColumns);
    write_metadata_rows<false>(qzeros, scales, packed, K, N, G, n0, Nt, c0, cols, kb, (int)threadIdx.x,
                               kGptqColumns);
}

}  // namespace

hipError_t launch_repack_gptq(const int32_t* qweight, const int32_t* qzeros, const uint16_t* scales,
                              uint8_t* packed, int64_t K, int64_t N, int64_t G, int64_t n0, int64_t Nt,
                              hipStream_t stream) {
    // one workgroup per (256-column tile, row block), tiles fastest: at most
    // K N / 2^15 <= 2^22 workgroups
    const dim3 grid((unsigned)(K / kRowsPerBlock * ((padded_cols(N) + kGptqColumns - 1) / kGptqColumns)));
    hipLaunchKernelGGL(repack_gptq_kernel, grid, dim3(kGptqColumns), 0, stream,
                       reinterpret_cast<const uint32_t*>(qweight), reinterpret_cast<const uint32_t*>(qzeros),
                       scales, packed, K, N, G, n0, Nt);
    return hipGetLastError();
}

hipError_t launch_repack(const int32_t* qweight, const int32_t* qzeros, const uint16_t* scales,
                         uint8_t* packed, int64_t K, int64_t N, int64_t G, int64_t n0, int64_t Nt,
                         hipStream_t stream) {
    const int64_t KB = K / kRowsPerBlock;
    const int64_t words = N / 8;
    // one workgroup per (row block, 64-word tile), row blocks fastest: at most
    // K N / 2^16 <= 2^21 workgroups
    const dim3 grid((unsigned)(KB * ((words + kWordsPerTile - 1) / kWordsPerTile)));
    hipLaunchKernelGGL(repack_kernel, grid, dim3(kRepackThreads), 0, stream,
                       reinterpret_cast<const uint32_t*>(qweight), reinterpret_cast<const uint32_t*>(qzeros),
                       scales, packed, K, N, G, n0, Nt);
    return hipGetLastError();
}

}  // namespace w4a16
