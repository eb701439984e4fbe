// LDS-staged dequantise -> MFMA GEMM for prefill-sized batches.
//
// A W4A16 product at hundreds of rows is a real dense contraction, so it runs on
// the matrix cores. What the CPU design of the vllm-omni cpu_int4 commits teaches
// carries over: a kernel that dequantises once per activation row is linear in the
// batch (the commit "Add cpu_int4 ..." measures such a kernel an order of magnitude
// behind a bf16 GEMM at 512 rows), and
// re-laying the weights out on every call halves prefill (commit "cpu_int4:
// dequantize prefill weights from the tinygemm layout, not a copy"). Here each
// weight is dequantised once per workgroup tile of up to 128 rows, straight from
// the packed layout, which is already in MFMA operand order: no per-call shuffle.
//
// Workgroup: 4 or 8 waves side by side along N, each owning CBW column blocks (16 CBW
// columns) and all 16*MR rows of the tile; the 256-column tile runs as 8 waves of
// 2 blocks and the 64 x 128 tile as 8 waves of one, two per SIMD, so that one
// computes while the other waits on its copies or the barrier. Per 128-row block of K:
//   * a 3-stage LDS ring holds, per k block, the activation tile [16*MR x 128]
//     (16-byte chunks XOR-swizzled by row, so the fragment reads of a wave spread
//     over all banks), the workgroup's blocks of packed codes and its metadata;
//     the ring is filled by direct global -> LDS copies, two k blocks ahead;
//   * per 32-row step a wave decodes one word per column block into 8 fp16/bf16
//     weights (q - z) * s, each rounded once to the dtype, and issues MR x CBW
//     MFMAs (16x16x32, fp32 accumulators). For bf16 the decoding of the next
//     operand is cut into single-instruction slices placed between the MFMAs of the
//     current one (a wave hides about two VALU instructions behind each MFMA, and
//     the decode is ~3 per MFMA at MR = 8: issued in a burst it stalled the matrix
//     cores);
//   * the MFMA is given the weights as its first operand and the activations as its
//     second, so it produces the transposed tile: each lane then holds 4 adjacent
//     output columns of one row and the epilogue writes 8 bytes per lane.
// Workgroups are numbered so that the M tiles of one N tile land on the same XCD
// (the hardware deals workgroup ids round-robin over the 8 XCDs), where they share
// the packed codes through that XCD's L2. A tile that holds one workgroup per CU runs
// persistent when there are more tiles than CUs: each workgroup takes a tile per
// round and copies the next tile's first k block while it writes the current output
// (same box, three runs each: the LM head at M = 512 270.7-274.4 -> 268.1-269.7 us,
// gate_up at M = 2048 129.0 -> 126.2 us).
// Epilogue: bias in fp32, one rounding to the dtype.
#include <stddef.h>

#include "device_common.h"
#include "launch.h"
#include "split_k.h"

namespace w4a16 {
namespace {

constexpr int kXcds = 8;

__device__ __forceinline__ uint32_t pick(const uint4 v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}


// One stage of the LDS ring: the activation tile of one 128-row block of K and the
// workgroup's blocks of packed codes (W waves x CBW).
template <int BM, int CBW, int W, int kSub>
struct Stage {
    // [BM rows][16 chunks of 16 bytes], chunk j of row r stored at chunk j ^ (r % 16)
    uint4 x[BM * 16];
    uint4 w[W * CBW * 64];                  // 1 KiB per block, as in global memory
};

// Metadata of 4 consecutive k blocks ("a group") for the 16 CBW columns of one wave:
// per column its 4 kSub unit words, which are contiguous in the packed layout, so the
// group is copied with CBW kSub 4-byte copies whose lanes cover 16 columns each (16
// cache lines per copy). (One copy per k block, each lane reading one word of its own
// column, touched 32 lines per copy for 256 useful bytes: dropping those copies alone
// made the LM-head GEMM ~8% faster.)
template <int CBW, int kSub>
struct MetaGroup {
    uint32_t words[16 * CBW * 4 * kSub];    // [column of the wave][unit of the group]
};

// Workgroup tile: 16*MR rows x 64*CBW columns, 4 waves side by side along N, each
// owning CBW column blocks and all rows. `splits` > 1 splits the K range over
// workgroups; their fp32 partial tiles meet in `workspace` and the last workgroup of
// a tile to finish adds them in split order (deterministic) and writes y.
template <bool kBF16, int MR, int CBW, int kWaves, int kSub, bool kPersist>
__global__ __launch_bounds__(64 * kWaves) void gemm_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ packed, const uint16_t* __restrict__ bias,
    uint16_t* __restrict__ y, int M, int K, int N, int tiles_m, int tiles_n, int splits,
    uint32_t* __restrict__ counters, float* __restrict__ partials, int nt_out, int total_ids) {
    constexpr int BM = 16 * MR;
    constexpr int kSlabsPerWave = BM / 4 / kWaves;      // 1 KiB slabs (4 rows) of the x tile per wave
    static_assert(kSlabsPerWave * 4 * kWaves == BM, "x tile must split over the waves");
    constexpr int kDmaPerStage = kSlabsPerWave + CBW;          // copies per wave per stage
    constexpr int kMetaDma = CBW * kSub;                        // + these in a group's first stage
    constexpr int kStages = 3;
    using StageT = Stage<BM, CBW, kWaves, kSub>;
    using MetaT = MetaGroup<CBW, kSub>;
    static_assert(sizeof(MetaT) == (size_t)kMetaDma * 256, "a group is whole 4-byte copies");
    __shared__ StageT ring[kStages];
    __shared__ MetaT mring[2][kWaves];       // group g of this split in slot g % 2

    const int KB = K / kRowsPerBlock;
    const int UW = (int)padded_units(K, kRowsPerBlock / kSub);     // metadata words per column
    const int Np = (int)padded_cols(N);                         // columns of the packed layout
    const int NB = Np / kColsPerBlock;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);    // wave index, uniform
    const int lane = tid & 63;
    const int c = lane & 15;
    const int h = lane >> 4;
    const uint32_t ring_base = lds_addr(&ring[0]);
    const uint32_t mring_base = lds_addr(&mring[0][w]);

    // Where one tile's copies come from: wave-uniform bases (k block kb adds kb * stride)
    // plus per-lane byte offsets.
    struct Src {
        int m_tile, n_tile, split, kb_begin, nkb, m0, nbw, col0;
        const uint8_t* xbase;
        const uint8_t* wbase;
        const uint8_t* mbase;
        uint32_t xoff[kSlabsPerWave];
        uint32_t woff[CBW];
    };
    // XCD-aware order: ids id, id+8, id+16, ... share an XCD; they take the M tiles and
    // the K splits of one N tile. Ids past the last N tile (grid padding) hold no tile.
    auto locate = [&](int id, Src& s) -> bool {
        const int local = id / kXcds;
        s.m_tile = local % tiles_m;
        const int rest = local / tiles_m;
        s.split = rest % splits;
        s.n_tile = (rest / splits) * kXcds + id % kXcds;
        if (s.n_tile >= tiles_n) return false;
        s.kb_begin = (int)((int64_t)KB * s.split / splits);
        s.nkb = (int)((int64_t)KB * (s.split + 1) / splits) - s.kb_begin;
        s.m0 = s.m_tile * BM;
        s.nbw = (s.n_tile * kWaves + w) * CBW;                 // first column block of this wave
        // x: slab `slab` covers tile rows 4 slab .. 4 slab + 3; lane (row 4 slab + lane/16,
        // stored chunk lane%16) fetches logical chunk (lane%16) ^ (row%16). Rows past M
        // read row M-1 and columns past N read column N-1: they only feed outputs that
        // are not written. Offsets from the tile's first row stay below 2^28 (128 rows of
        // at most 2^20 elements).
        s.xbase = uniform_ptr(x + (size_t)s.m0 * K);
#pragma unroll
        for (int t = 0; t < kSlabsPerWave; ++t) {
            const int row = 4 * (w * kSlabsPerWave + t) + (lane >> 4);
            const int m = s.m0 + row < M ? s.m0 + row : M - 1;
            s.xoff[t] = 2u * ((uint32_t)(m - s.m0) * (uint32_t)K + 8u * (uint32_t)((lane & 15) ^ (row & 15)));
        }
        // codes: this wave's blocks from its first (clamped) column block
        const int nbw0 = s.nbw < NB ? s.nbw : NB - 1;
        s.wbase = uniform_ptr(packed + (size_t)nbw0 * KB * kBlockBytes);
#pragma unroll
        for (int j = 0; j < CBW; ++j) {
            const int nbj = s.nbw + j < NB ? s.nbw + j : NB - 1;
            s.woff[j] = (uint32_t)(nbj - nbw0) * (uint32_t)KB * kBlockBytes + 16u * (uint32_t)lane;
        }
        // metadata: word 64 i + lane of a group's copy i is column (64 i + lane) / (4 kSub)
        // of the wave and unit (64 i + lane) % (4 kSub) of the group, columns past the last
        // reading the last, units past the column's last word reading that word (they feed
        // only outputs or k blocks that do not count)
        s.col0 = s.nbw * kColsPerBlock < Np ? s.nbw * kColsPerBlock : Np - kColsPerBlock;
        s.mbase = uniform_ptr(packed + (size_t)K * Np / 2 + (size_t)s.col0 * UW * 4);
        return true;
    };
    // first id at or after `id` (in steps of the grid) that holds a tile; >= total_ids if none
    auto next_tile = [&](int id, Src& s) -> int {
        while (id < total_ids && !locate(id, s)) id += (int)gridDim.x;
        return id;
    };

    // copy q (0 .. kDmaPerStage-1) of k block kb into ring slot `slot`
    auto issue_one = [&](const Src& s, int slot, int kb, int q) {
        const uint32_t st = ring_base + (uint32_t)slot * (uint32_t)sizeof(StageT);
        if (q < kSlabsPerWave)
            dma16(s.xbase + (size_t)kb * kRowsPerBlock * 2, s.xoff[q],
                  st + (uint32_t)offsetof(StageT, x) + (uint32_t)(w * kSlabsPerWave + q) * 1024u);
        else if (q < kSlabsPerWave + CBW)
            dma16(s.wbase + (size_t)kb * kBlockBytes, s.woff[q - kSlabsPerWave],
                  st + (uint32_t)offsetof(StageT, w) + (uint32_t)(w * CBW + q - kSlabsPerWave) * 1024u);
    };
    // stage t (k block kb_begin + t); a group's first stage also copies the group's
    // metadata into slot (t / 4) % 2
    auto issue = [&](const Src& s, int slot, int t) {
        const int kb = s.kb_begin + t;
#pragma unroll
        for (int q = 0; q < kDmaPerStage; ++q) issue_one(s, slot, kb, q);
        if ((t & 3) == 0) {
            const uint32_t dst = mring_base + (uint32_t)((t >> 2) & 1) * (uint32_t)(kWaves * sizeof(MetaT));
#pragma unroll
            for (int i = 0; i < kMetaDma; ++i) {
                const int wi = 64 * i + lane;
                const int cl = wi / (4 * kSub), u = wi % (4 * kSub);
                const int n = s.nbw * kColsPerBlock + cl < Np ? s.nbw * kColsPerBlock + cl : Np - 1;
                const int ua = kb * kSub + u < UW ? kb * kSub + u : UW - 1;
                dma4(s.mbase, ((uint32_t)(n - s.col0) * (uint32_t)UW + (uint32_t)ua) * 4u, dst + (uint32_t)i * 256u);
            }
        }
    };

    // A workgroup runs the tile of id blockIdx.x and, when persistent (a grid smaller
    // than the ids), those of + gridDim.x, ...: the next tile's first stage is copied
    // while the current tile's output is written. (Compiled without the tile loop
    // where the grid covers every id: with it, single-round launches ran 2-3% slower.)
    Src cur;
    int id = next_tile((int)blockIdx.x, cur);
    if (id >= total_ids) return;
    issue(cur, 0, 0);
    for (;;) {
        const int nkb = cur.nkb;
        const int m0 = cur.m0;
        const int nbw = cur.nbw;
        if (nkb > 1) issue(cur, 1, 1);

        f32x4 acc[MR][CBW];
#pragma unroll
        for (int r = 0; r < MR; ++r)
#pragma unroll
            for (int j = 0; j < CBW; ++j) acc[r][j] = f32x4{0.f, 0.f, 0.f, 0.f};

        for (int t = 0; t < nkb; ++t) {
            // this wave's copies of step t are done (step t+1's may be in flight: one more
            // per metadata copy when t+1 starts a group); the barrier makes every wave's
            // copies visible and retires the reads of step t-1, whose slot is then refilled
            // with step t+2 (a group's metadata slot is refilled at step 4g + 6, after every
            // wave has passed the group's last step 4g + 3)
            if (t + 1 >= nkb) wait_vmcnt<0>();
            else if (((t + 1) & 3) == 0) wait_vmcnt<kDmaPerStage + kMetaDma>();
            else wait_vmcnt<kDmaPerStage>();
            lds_barrier();
            // The copies queue at the CU's address unit (about 16 cycles per 1 KiB copy, the
            // 4 waves' together) and each wave waits until its own are accepted: about a
            // sixth of the loop. Spreading them between the MFMAs measured slower.
            if (t + 2 < nkb) issue(cur, (t + 2) % kStages, t + 2);

            const StageT& st = ring[t % kStages];
            Dequant<kBF16> dq[CBW][kSub];           // per column block and metadata unit
            uint4 wq[CBW];
#pragma unroll
            for (int j = 0; j < CBW; ++j) {
#pragma unroll
                for (int v = 0; v < kSub; ++v)
                    dq[j][v] = Dequant<kBF16>(mring[(t >> 2) & 1][w].words[(16 * j + c) * 4 * kSub + (t & 3) * kSub + v]);
                wq[j] = st.w[(w * CBW + j) * 64 + lane];
            }
            if constexpr (kBF16) {
                // Unit (i, j) = 32-row step i, column block j: MR MFMAs on one decoded
                // operand b. While they run, the next unit's word is decoded in independent
                // slices, one after each MFMA (masks; two byte converts; two fmas one slot
                // later; a pair pack after both fmas), and in a step's last unit each
                // fragment a[r] is refilled with the next step's right after its last use.
                // sched_barrier(0) after each slot keeps this order: one wave hides about
                // two VALU instructions behind each MFMA, not a burst of twenty.
                uint4 a[MR];
#pragma unroll
                for (int r = 0; r < MR; ++r) a[r] = st.x[(16 * r + c) * 16 + (h ^ c)];
                uint4 b = dq[0][0](pick(wq[0], 0));
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
#pragma unroll
                    for (int j = 0; j < CBW; ++j) {
                        const bool has_next = !(i == 3 && j == CBW - 1);
                        const int jn = j + 1 < CBW ? j + 1 : 0;
                        const int in = j + 1 < CBW ? i : i + 1;
                        const uint32_t dn = has_next ? pick(wq[jn], in & 3) : 0u;
                        const float sn = dq[jn][((in & 3) * kSub) / 4].s, zn = dq[jn][((in & 3) * kSub) / 4].nzs;
                        uint32_t lo = 0u, hi = 0u;
                        float cv[8], fv[8];
                        uint32_t o[4] = {0u, 0u, 0u, 0u};
                        const int chunk = (4 * (i + 1) + h) ^ c;
#pragma unroll
                        for (int r = 0; r < MR; ++r) {
                            acc[r][j] = mfma16x16x32<kBF16>(b, a[r], acc[r][j]);
                            if (has_next) {
                                // 12 ticks spread over the MR slots: 0 masks, 1..4 converts
                                // (values v = 2(t-1), +1), 4..7 fmas (v = 2(t-4), +1), 8..11 packs.
                                // Values 0..3 are the bytes of lo (rows 0,4,1,5), 4..7 of hi
                                // (rows 2,6,3,7); output word e holds rows (2e, 2e+1).
                                constexpr int kTicks = 12;
#pragma unroll
                                for (int tk = r * kTicks / MR; tk < (r + 1) * kTicks / MR; ++tk) {
                                    if (tk == 0) {
                                        lo = dn & 0x0F0F0F0Fu;
                                        hi = (dn >> 4) & 0x0F0F0F0Fu;
                                        asm volatile("" : "+v"(lo), "+v"(hi));   // one byte convert per value
                                    } else if (tk <= 4) {
                                        const int v0 = 2 * (tk - 1), v1 = v0 + 1;
                                        cv[v0] = (float)((((v0 < 4) ? lo : hi) >> (8 * (v0 & 3))) & 0xFFu);
                                        cv[v1] = (float)((((v1 < 4) ? lo : hi) >> (8 * (v1 & 3))) & 0xFFu);
                                    }
                                    if (tk >= 4 && tk <= 7) {
                                        const int v0 = 2 * (tk - 4), v1 = v0 + 1;
                                        fv[v0] = fmaf(cv[v0], sn, zn);
                                        fv[v1] = fmaf(cv[v1], sn, zn);
                                    }
                                    if (tk >= 8) {
                                        const int e = tk - 8;
                                        const int va = e == 0 ? 0 : e == 1 ? 4 : e == 2 ? 1 : 5;
                                        o[e] = pack2_rne<true>(fv[va], fv[va + 2]);
                                    }
                                }
                            }
                            if (j == CBW - 1 && i < 3) a[r] = st.x[(16 * r + c) * 16 + chunk];
                            __builtin_amdgcn_sched_barrier(0);
                        }
                        if (has_next) b = make_uint4(o[0], o[1], o[2], o[3]);
                    }
                }
            } else {
                // fp16: per 32-row step the MR fragments, then column block by column block
                // one decoded operand (three packed-fp16 instructions per pair) and its MFMAs
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int chunk = (4 * i + h) ^ c;          // row 16 r + c has row % 16 == c
                    uint4 a[MR];
#pragma unroll
                    for (int r = 0; r < MR; ++r) a[r] = st.x[(16 * r + c) * 16 + chunk];
#pragma unroll
                    for (int j = 0; j < CBW; ++j) {
                        const uint4 b = dq[j][(i * kSub) / 4](pick(wq[j], i));
#pragma unroll
                        for (int r = 0; r < MR; ++r) acc[r][j] = mfma16x16x32<kBF16>(b, a[r], acc[r][j]);
                    }
                }
            }
        }

        // transposed tiles: lane (c, h), register e -> row 16 r + c, column 16 j + 4 h + e
        // (a split K runs one tile per workgroup: the grid then covers every id)
        if (splits > 1 && !reduce_splits<MR, CBW, kWaves>(acc, counters, partials, cur.m_tile * tiles_n + cur.n_tile,
                                                          cur.split, splits))
            return;

        // bias of this wave's columns; a persistent tile reads it before the next
        // tile's copies are issued (a wait for it would then wait for them too)
        float bv[CBW][4];
        auto load_bias = [&]() {
#pragma unroll
            for (int j = 0; j < CBW; ++j) {
                const int n = (nbw + j) * kColsPerBlock + 4 * h;
#pragma unroll
                for (int e = 0; e < 4; ++e) bv[j][e] = bias && n < N ? half_bits_to_f32<kBF16>(bias[n + e]) : 0.f;
            }
        };
        if constexpr (kPersist) load_bias();
        Src nxt;
        int nid = total_ids;
        if constexpr (kPersist) nid = next_tile(id + (int)gridDim.x, nxt);
        const bool more = nid < total_ids;

        // Epilogue through LDS: the lanes write their rounded outputs into the ring as a
        // row-major [BM][BN] tile (rows padded by 16 bytes against bank conflicts), and
        // the waves store whole rows, 16 bytes per lane and 1 KiB per instruction, instead
        // of each wave writing half of every 128-byte line it touches. A persistent tile
        // stages it in slots 1..2, while slot 0 takes the next tile's first stage.
        constexpr int BN = 16 * CBW * kWaves;
        constexpr int kRowBytes = BN * 2 + 16;
        static_assert(!kPersist || (size_t)BM * kRowBytes <= (kStages - 1) * sizeof(StageT),
                      "the output tile fits in slots 1..2");
        static_assert((size_t)BM * kRowBytes <= kStages * sizeof(StageT), "the output tile fits in the ring");
        uint8_t* otile = reinterpret_cast<uint8_t*>(&ring[kPersist ? 1 : 0]);
        lds_barrier();                           // every wave is done with the ring's operands
        if (more) issue(nxt, 0, 0);
        if constexpr (!kPersist) load_bias();
#pragma unroll
        for (int j = 0; j < CBW; ++j) {
            const int col = 16 * (w * CBW + j) + 4 * h;        // in the tile
#pragma unroll
            for (int r = 0; r < MR; ++r) {
                const f32x4 v = acc[r][j];
                const uint2 o = make_uint2(pack2_rne<kBF16>(v[0] + bv[j][0], v[1] + bv[j][1]),
                                           pack2_rne<kBF16>(v[2] + bv[j][2], v[3] + bv[j][3]));
                *reinterpret_cast<uint2*>(otile + (16 * r + c) * kRowBytes + 2 * col) = o;
            }
        }
        __syncthreads();
        // rows past M and columns past N (the zero padding of a last half block, whole
        // column blocks past the last) are not stored; N % 8 == 0, so a 16-byte chunk of 8
        // columns lies wholly inside or outside
        const int n0 = cur.n_tile * BN;
        for (int q = tid; q < BM * (BN / 8); q += 64 * kWaves) {
            const int row = q / (BN / 8);
            const int ch = q - row * (BN / 8);
            const int m = m0 + row, n = n0 + 8 * ch;
            if (m < M && n < N)
                store_out16(y + (size_t)m * N + n, *reinterpret_cast<const uint4*>(otile + row * kRowBytes + 16 * ch), nt_out != 0);
        }
        if (!more) break;
        lds_barrier();                           // every wave has read the output tile: slot 1 is refilled
        cur = nxt;
        id = nid;
    }
}

constexpr int kTargetWorkgroups = 256;   // one per CU

template <bool kBF16, int MR, int CBW, int W, int kSub = 1>
void launch_cfg(const GemmPlan& p, const uint16_t* x, const uint8_t* packed, const uint16_t* bias, uint16_t* y,
                int M, int K, int N, uint32_t* counters, float* partials, hipStream_t stream) {
    const int tiles_n_pad = (p.tiles_n + kXcds - 1) / kXcds * kXcds;
    const int total_ids = p.tiles_m * p.splits * tiles_n_pad;
    // A tile whose LDS leaves room for one workgroup per CU runs persistent when there
    // are more tiles than CUs: one workgroup per CU (a multiple of 8, so every id a
    // workgroup takes stays on its XCD) takes a tile per round.
    constexpr size_t kLds = 3 * sizeof(Stage<16 * MR, CBW, W, kSub>) + 2 * W * sizeof(MetaGroup<CBW, kSub>);
    const bool persistent = kLds > 80 * 1024 && p.splits == 1 && total_ids > kTargetWorkgroups;
    // streaming output stores when every workgroup runs in the first round (qkv and
    // gate_up prefill: 1-2% faster; the LM head, 8 rounds, unchanged)
    const int nt_out = (int64_t)p.tiles_m * p.tiles_n * p.splits <= kTargetWorkgroups ? 1 : 0;
    if constexpr (kLds > 80 * 1024) {
        if (persistent) {
            hipLaunchKernelGGL((gemm_kernel<kBF16, MR, CBW, W, kSub, true>), dim3(kTargetWorkgroups), dim3(64 * W), 0,
                               stream, x, packed, bias, y, M, K, N, p.tiles_m, p.tiles_n, p.splits, counters, partials,
                               nt_out, total_ids);
            return;
        }
    }
    hipLaunchKernelGGL((gemm_kernel<kBF16, MR, CBW, W, kSub, false>), dim3((unsigned)total_ids), dim3(64 * W), 0, stream,
                       x, packed, bias, y, M, K, N, p.tiles_m, p.tiles_n, p.splits, counters, partials, nt_out, total_ids);
}

template <bool kBF16, int MR>
void launch_mr(const GemmPlan& p, const uint16_t* x, const uint8_t* packed, const uint16_t* bias, uint16_t* y,
               int M, int K, int N, uint32_t* counters, float* partials, hipStream_t stream) {
    // group sizes 32 and 64: one tile shape, 4 waves of one column block
    if (p.sub == 4) {
        launch_cfg<kBF16, MR, 1, 4, 4>(p, x, packed, bias, y, M, K, N, counters, partials, stream);
        return;
    }
    if (p.sub == 2) {
        launch_cfg<kBF16, MR, 1, 4, 2>(p, x, packed, bias, y, M, K, N, counters, partials, stream);
        return;
    }
    if constexpr (MR >= 4) {
        if (p.waves == 8 && p.cbw == 1) {
            launch_cfg<kBF16, MR, 1, 8>(p, x, packed, bias, y, M, K, N, counters, partials, stream);
            return;
        }
    }
    if constexpr (MR >= 2) {
        if (p.waves == 8) {
            launch_cfg<kBF16, MR, 2, 8>(p, x, packed, bias, y, M, K, N, counters, partials, stream);
            return;
        }
    }
    if (p.cbw == 4) launch_cfg<kBF16, MR, 4, 4>(p, x, packed, bias, y, M, K, N, counters, partials, stream);
    else if (p.cbw == 2) launch_cfg<kBF16, MR, 2, 4>(p, x, packed, bias, y, M, K, N, counters, partials, stream);
    else launch_cfg<kBF16, MR, 1, 4>(p, x, packed, bias, y, M, K, N, counters, partials, stream);
}

template <bool kBF16>
void launch_typed(const GemmPlan& p, const uint16_t* x, const uint8_t* packed, const uint16_t* bias, uint16_t* y,
                  int M, int K, int N, uint32_t* counters, float* partials, hipStream_t stream) {
    if (p.mr == 1) launch_mr<kBF16, 1>(p, x, packed, bias, y, M, K, N, counters, partials, stream);
    else if (p.mr == 2) launch_mr<kBF16, 2>(p, x, packed, bias, y, M, K, N, counters, partials, stream);
    else if (p.mr == 4) launch_mr<kBF16, 4>(p, x, packed, bias, y, M, K, N, counters, partials, stream);
    else launch_mr<kBF16, 8>(p, x, packed, bias, y, M, K, N, counters, partials, stream);
}

}  // namespace

GemmPlan plan_gemm(int64_t M, int64_t K, int64_t N, int64_t G) {
    GemmPlan p;
    p.sub = units_per_block(G);
    const int64_t NB = padded_cols(N) / kColsPerBlock;
    const int64_t KB = K / kRowsPerBlock;
    p.mr = M <= 16 ? 1 : M <= 32 ? 2 : M <= 64 ? 4 : 8;
    p.tiles_m = (int)((M + 16 * p.mr - 1) / (16 * p.mr));
    p.waves = 4;
    p.cbw = 1;
    if (p.sub > 1) {
        // group sizes 32 and 64: 4 waves of one column block, the tile's rows by M
    } else if (p.mr >= 4) {
        // Tile shape from a cost model: rounds of tiles over the CUs (one workgroup per
        // CU) x tile area / throughput of that shape. Throughputs are relative output
        // elements per unit time, per k block, measured with one tile per CU on MI355X:
        // wider and taller tiles decode each weight for more rows and copy the
        // activations less often, but leave CUs idle on small outputs.
        struct Shape { int mr, cbw, waves; double rate; };
        static constexpr Shape kShapes[] = {
            {8, 2, 8, 13.1},   // 128 x 256
            {8, 1, 8, 11.3},   // 128 x 128 as 8 waves of one block (1024 x 4096: 30.2 -> 28.5 us
                               // against 64 x 256; 3000 x 2608: 73.9 -> 70.5 us against 4 x 2)
            {8, 2, 4, 10.4},   // 128 x 128
            {8, 1, 4, 7.2},    // 128 x 64
            {4, 2, 8, 10.8},   // 64 x 256
            {4, 1, 8, 8.0},    // 64 x 128 as 8 waves of one block (qkv prefill: 18.4 -> 16.9 us)
            {4, 2, 4, 7.4},    // 64 x 128
            {4, 1, 4, 5.4},    // 64 x 64
        };
        double best = 0.0;
        for (const Shape& c : kShapes) {
            if (c.mr > p.mr) continue;
            const int64_t tm = (M + 16 * c.mr - 1) / (16 * c.mr);
            const int64_t tn = (NB + c.waves * c.cbw - 1) / (c.waves * c.cbw);
            const int64_t rounds = (tm * tn + kTargetWorkgroups - 1) / kTargetWorkgroups;
            const double cost = (double)rounds * (16.0 * c.mr) * (16.0 * c.waves * c.cbw) / c.rate;
            if (best == 0.0 || cost < best) {
                best = cost;
                p.mr = c.mr;
                p.cbw = c.cbw;
                p.waves = c.waves;
                p.tiles_m = (int)tm;
            }
        }
    } else {
        // 16- and 32-row tiles (M <= 32, weight-bound): the widest column tile (4 waves
        // x cbw blocks) that still occupies 3/4 of the CUs, else the narrowest
        for (int cbw : {4, 2}) {
            if (p.tiles_m * ((NB + 4 * cbw - 1) / (4 * cbw)) >= kTargetWorkgroups * 3 / 4) {
                p.cbw = cbw;
                break;
            }
        }
        // the 256-column tile as 8 waves of 2 blocks rather than 4 of 4: two waves per
        // SIMD (needs 16 * mr >= 32 rows for the activation copies to split over 8 waves)
        if (p.cbw == 4 && p.mr >= 2) {
            p.waves = 8;
            p.cbw = 2;
        }
    }
    p.tiles_n = (int)((NB + p.waves * p.cbw - 1) / (p.waves * p.cbw));
    const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n;
    // too few tiles for the chip: split K, at least 4 row blocks per split
    p.splits = 1;
    static_assert(kTargetWorkgroups / 2 <= kMaxSplitTiles, "split tiles must fit the counter region");
    if (tiles < kTargetWorkgroups / 2 && KB >= 8) {
        const int64_t want = (kTargetWorkgroups + tiles - 1) / tiles;
        const int64_t most = KB / 4;
        p.splits = (int)(want < most ? want : most);
    }
    p.workspace_bytes = 0;
    if (p.splits > 1) {
        // fp32 partial tiles: splits x tiles x (16 mr) x (16 waves cbw)
        p.workspace_bytes = kSplitCounterBytes + (size_t)p.splits * (size_t)tiles * (size_t)(16 * p.mr) *
                                           (size_t)(16 * p.waves * p.cbw) * 4;
    }
    return p;
}

hipError_t launch_gemm(const uint16_t* x, const uint8_t* packed, const uint16_t* bias, uint16_t* y,
                       int64_t M, int64_t K, int64_t N, int64_t G, bool bf16, void* workspace,
                       hipStream_t stream) {
    const GemmPlan p = plan_gemm(M, K, N, G);
    uint32_t* counters = static_cast<uint32_t*>(workspace);
    float* partials = nullptr;
    if (p.splits > 1) {
        partials = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + kSplitCounterBytes);
    }
    if (bf16) launch_typed<true>(p, x, packed, bias, y, (int)M, (int)K, (int)N, counters, partials, stream);
    else launch_typed<false>(p, x, packed, bias, y, (int)M, (int)K, (int)N, counters, partials, stream);
    return hipGetLastError();
}

}  // namespace w4a16
