// One-time repack of AWQ int32 nibble packing into the packed tile layout.
//
// The AWQ checkpoint stores codes packed along the output dimension, eight per
// int32 in a non-standard order, and vLLM reorders them once after loading (note
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
// (256 bytes) of one row per load instruction. The workgroups of row block 0 also
// write the metadata rows of their 512 columns (one column's row is contiguous).
#include "device_common.h"
#include "launch.h"

namespace w4a16 {
namespace {

constexpr int kWordsPerTile = 64;                    // AWQ words (8 columns each) per workgroup
constexpr int kRepackThreads = kWordsPerTile * 4;    // x 4 lane groups

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

// Input tensors hold columns [n0, n0 + N) of a K x Nt weight (the whole weight when
// n0 = 0 and N = Nt): qweight [K, N/8], qzeros [K/G, N/8], scales [K/G, N]. Output:
// those columns' blocks and metadata rows in the packed layout of the K x Nt weight.
__global__ __launch_bounds__(kRepackThreads) void repack_kernel(
    const uint32_t* __restrict__ qweight, const uint32_t* __restrict__ qzeros,
    const uint16_t* __restrict__ scales, uint8_t* __restrict__ packed,
    int64_t K, int64_t N, int64_t G, int64_t n0, int64_t Nt) {
    const int64_t KB = K / kRowsPerBlock;
    const int64_t words_per_row = N / 8;
    const int64_t kb = blockIdx.y;
    const int64_t j0 = (int64_t)blockIdx.x * kWordsPerTile;     // first AWQ word of the tile
    const int tid = threadIdx.x;
    const int jl = tid & (kWordsPerTile - 1);
    const int h = tid / kWordsPerTile;                            // lane group (wave) 0..3
    const int64_t j = j0 + jl;
    const bool active = j < words_per_row;
    const int64_t jc = active ? j : words_per_row - 1;            // clamped: loads stay in bounds

    // 1. rows 128 kb + 32 i + 8 h + e of word column jc, fed in tile slot order
    uint32_t t[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t* src = qweight + (kb * kRowsPerBlock + 32 * i + 8 * h) * words_per_row + jc;
#pragma unroll
        for (int s = 0; s < 8; ++s) t[i][s] = src[(int64_t)tile_row_of_slot(s) * words_per_row];
    }
    // 2. transpose: t[i][s] = column in AWQ slot s, its 8 rows in tile slot order
#pragma unroll
    for (int i = 0; i < 4; ++i) transpose8x8_nibbles(t[i]);

    // 3. column 8 j + c8 -> block (j / 2), lane (8 (j % 2) + c8) + 16 h: words i = 0..3.
    //    The tile's 32 blocks are assembled in LDS and written out whole, each wave
    //    storing contiguous 1 KiB blocks.
    //    With N % 16 == 8 the last block has one word: its other 8 columns are zero.
    __shared__ uint4 stage[kWordsPerTile / 2 * 64];
#pragma unroll
    for (int c8 = 0; c8 < 8; ++c8) {
        const int s = awq_slot_of_column(c8);
        const int lane = 8 * (jl & 1) + c8 + 16 * h;
        stage[(jl >> 1) * 64 + lane] = active ? make_uint4(t[0][s], t[1][s], t[2][s], t[3][s]) : make_uint4(0, 0, 0, 0);
    }
    __syncthreads();
    const int64_t tile_words = words_per_row - j0 < kWordsPerTile ? words_per_row - j0 : kWordsPerTile;
    const int nblk = (int)((tile_words + 1) / 2);                 // a last half block included
    for (int q = tid; q < nblk * 64; q += kRepackThreads) {
        const int64_t nb = n0 / kColsPerBlock + (j0 >> 1) + (q >> 6);
        reinterpret_cast<uint4*>(packed + (nb * KB + kb) * kBlockBytes)[q & 63] = stage[q];
    }

    // 4. metadata: the workgroups of row block 0 write, for each column of their tile's
    //    blocks, its whole row of UW words (scale bits | zero << 16 per metadata unit of
    //    min(G, 128) rows, then zero padding; all zero for the padding columns of a last
    //    half block), 16 bytes at a time
    if (kb != 0) return;
    const int64_t UW = padded_units(K, G);
    const int64_t U = KB * units_per_block(G);
    const int64_t Gu = kRowsPerBlock / units_per_block(G);      // rows per unit
    uint32_t* meta = reinterpret_cast<uint32_t*>(packed + K * padded_cols(Nt) / 2);
    for (int q = tid; q < nblk * kColsPerBlock; q += kRepackThreads) {
        const int64_t n = j0 * 8 + q;                 // column of the input tensors
        const bool real = n < N;
        const int zshift = 4 * awq_slot_of_column((int)(n & 7));
        uint4* row = reinterpret_cast<uint4*>(meta + (n0 + n) * UW);
        for (int64_t p0 = 0; p0 < UW; p0 += 4) {
            uint32_t word[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t b = p0 + e;
                word[e] = 0u;
                if (real && b < U) {
                    const int64_t g = (b * Gu) / G;
                    const uint32_t z = (qzeros[g * words_per_row + (n >> 3)] >> zshift) & 0xFu;
                    word[e] = (uint32_t)scales[g * N + n] | (z << 16);
                }
            }
            row[p0 / 4] = make_uint4(word[0], word[1], word[2], word[3]);
        }
    }
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
// unzipped, and no transpose is needed.
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
    const int64_t kb = blockIdx.y;
    const int64_t n = (int64_t)blockIdx.x * kGptqColumns + threadIdx.x;
    if (n >= padded_cols(N)) return;
    const bool real = n < N;          // else a zero padding column of a last half block
    const int64_t nb = (n0 + n) / kColsPerBlock;
    const int c = (int)(n % kColsPerBlock);
    uint4* blk = reinterpret_cast<uint4*>(packed + (nb * KB + kb) * kBlockBytes);
    // GPTQ word row i = 16 kb + 4 w + h: lane group h, word w of the tile
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        uint32_t t[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) t[w] = real ? unzip_nibbles(qweight[(16 * kb + 4 * w + h) * N + n]) : 0u;
        blk[c + 16 * h] = make_uint4(t[0], t[1], t[2], t[3]);
    }
    if (kb != 0) return;
    // metadata row of column n: scale bits | zero << 16 per unit of min(G, 128) rows,
    // zero padding
    const int64_t UW = padded_units(K, G);
    const int64_t U = KB * units_per_block(G);
    const int64_t Gu = kRowsPerBlock / units_per_block(G);
    uint4* row = reinterpret_cast<uint4*>(packed + K * padded_cols(Nt) / 2 + (n0 + n) * UW * 4);
    for (int64_t p0 = 0; p0 < UW; p0 += 4) {
        uint32_t word[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t b = p0 + e;
            word[e] = 0u;
            if (real && b < U) {
                const int64_t g = (b * Gu) / G;
                const uint32_t z = (qzeros[g * (N / 8) + n / 8] >> (4 * (n % 8))) & 0xFu;
                word[e] = (uint32_t)scales[g * N + n] | (z << 16);
            }
        }
        row[p0 / 4] = make_uint4(word[0], word[1], word[2], word[3]);
    }
}

}  // namespace

hipError_t launch_repack_gptq(const int32_t* qweight, const int32_t* qzeros, const uint16_t* scales,
                              uint8_t* packed, int64_t K, int64_t N, int64_t G, int64_t n0, int64_t Nt,
                              hipStream_t stream) {
    const dim3 grid((unsigned)((padded_cols(N) + kGptqColumns - 1) / kGptqColumns), (unsigned)(K / kRowsPerBlock));
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
    dim3 grid((unsigned)((words + kWordsPerTile - 1) / kWordsPerTile), (unsigned)KB);
    hipLaunchKernelGGL(repack_kernel, grid, dim3(kRepackThreads), 0, stream,
                       reinterpret_cast<const uint32_t*>(qweight), reinterpret_cast<const uint32_t*>(qzeros),
                       scales, packed, K, N, G, n0, Nt);
    return hipGetLastError();
}

}  // namespace w4a16
