// Weight-streaming split-K GEMV for decode-sized batches (1 <= M <= 16).
//
// Decode is bound by the bytes of the weights: every weight is read once per
// token (vllm-omni commit "Add cpu_int4, an asymmetric 4-bit weight path for
// vLLM's CPU backend"). So the kernel is organised around streaming the packed
// codes at HBM rate with 128-bit loads and doing as little per-weight ALU work as
// possible:
//
//   * a workgroup covers one or more 16-column blocks, and the waves of each block
//     split the K range (split-K) in runs of 4 row blocks, loading a column's metadata words for the run with one
//     16-byte load. Every load is unconditional (indices clamped into the buffer,
//     out-of-range row blocks weighted by a zero scale), so all of a run's loads are
//     in flight before the first is consumed. Codes and metadata are read once,
//     with nontemporal loads;
//   * per 32-row step a lane turns its packed word into the B operand of a
//     16x16x32 MFMA with one shift and one AND-OR per pair of codes: OR-ing a code
//     into the mantissa of the 16-bit value 128.0 (bf16) or 1024.0 (fp16) gives
//     exactly base + q, so the MFMA sums T = sum_k x (base + q) with exact products;
//     the run's row blocks are independent MFMA chains, interleaved;
//   * the activations are the A operand; rows >= M repeat row 0 and their results
//     are dropped (a row of the product depends on that row of A only);
//   * per 128-row block, y += s * (T - (base + z) * X), X = sum_k x over the block:
//     the offset and the zero point leave in one correction, because
//     sum_k x (base + q) - (base + z) sum_k x = sum_k x (q - z);
//   * the waves' partial sums are added in wave order through LDS (deterministic),
//     bias is added in fp32 and the result rounded once to the output dtype;
//   * on narrow outputs (at most 128 column blocks) with a long K (>= 6144), from
//     M = 6 and given a workspace, 2-4 workgroups per column block split its K range
//     and meet in the workspace (a separate instantiation): there the idle compute
//     units cost more than the meeting's memory round trip. At smaller M, or K <= 4096,
//     the meeting measured slower.
//
// One activation row (M = 1) takes the balanced GEMV of gemv_strip.hip instead when
// the shape fits it (groups of 128 rows or more, K <= 8192, at most 16 of its code
// loads per lane), and 4 <= M <= 8 (2 <= M <= 8 on outputs of at most 128 column
// blocks, up to M = 16 on outputs of at least 512) the balanced matrix-core GEMV of
// gemv_small.hip (groups of 128 rows or more, at most 8 units in flight per lane); this
// kernel runs the other shapes: the LM head, long K, group sizes 32 and 64, M = 2 and
// 3 on wide outputs, M = 9 .. 16 on narrower ones.
//
// Two variants:
//   staged  (the activations fit in LDS): the workgroup copies x to LDS and
//           computes the row-block sums X there once (16 lanes per sum, reduced
//           with DPP lane moves), while the codes are in flight;
//   direct  (otherwise): each lane loads its activation fragments from global
//           memory, and X is folded into the MFMA as a second product with B equal
//           to -(base + z) in every entry.
#include "device_common.h"
#include "launch.h"
#include "split_k.h"

namespace w4a16 {
namespace {

constexpr int kMaxWaves = 16;
constexpr int kRun = 4;                      // row blocks per load batch (one metadata uint4)
constexpr int kMaxStagedChunksPerThread = 8; // 16-byte activation chunks a thread stages
// Staging pays while the workgroup's LDS stays small: with the activations of the
// down projection (K = 6656) at M = 4 (70 KB) and M = 8 (122 KB) the direct variant
// ran 7% and 11% faster; at 41-43 KB (M = 8 at K = 2048, M = 2 at K = 6656) staging
// was faster or even.
constexpr size_t kStagedLdsLimit = 64 * 1024;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Data read exactly once: nontemporal 16-byte load.
__device__ __forceinline__ uint4 load_once(const uint4* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// LDS bytes of the staged activations, `chunks` 16-byte chunks copied in whole waves
// of 64 (the last wave's extra lanes land in the padding)
__host__ __device__ constexpr int64_t staged_x_bytes(int64_t chunks) { return (chunks + 63) / 64 * 64 * 16; }

__device__ __forceinline__ uint32_t pick(const uint4 v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// The nibble-pair mask 0x000F000F held in a VGPR. A three-operand instruction on
// this architecture reads at most one scalar or literal constant, so with the mask
// in a VGPR and the magic base in an SGPR each pair of codes decodes with a single
// v_and_or_b32 (after its shift) instead of a separate AND and OR.
__device__ __forceinline__ uint32_t pair_mask_vgpr() {
    uint32_t m;
    asm volatile("v_mov_b32 %0, 0x000f000f" : "=v"(m));
    return m;
}

// B operand of step i: codes of rows 32i + 8(l/16) + 0..7 as base + q pairs.
template <bool kBF16>
__device__ __forceinline__ uint4 magic_operand(uint32_t v, uint32_t mask) {
    constexpr uint32_t B = Magic<kBF16>::kBase2;
    return make_uint4((v & mask) | B, ((v >> 4) & mask) | B, ((v >> 8) & mask) | B, ((v >> 12) & mask) | B);
}

// Sum of the 8 16-bit values in a uint4, in fp32.
template <bool kBF16>
__device__ __forceinline__ float sum8(const uint4 v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) s += half_bits_to_f32<kBF16>(w[i] & 0xFFFFu) + half_bits_to_f32<kBF16>(w[i] >> 16);
    return s;
}

// Sum over aligned groups of kLanes (4, 8 or 16) lanes within rows of 16, result in
// every lane of the group (DPP: swap neighbours, swap pairs, mirror half rows, mirror
// rows). Fixed order, so deterministic.
template <int kLanes>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(kLanes == 4 || kLanes == 8 || kLanes == 16, "group of 4, 8 or 16 lanes");
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
    if constexpr (kLanes >= 8)
        v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));  // row_half_mirror
    if constexpr (kLanes >= 16)
        v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false));  // row_mirror
    return v;
}

struct GemvArgs {
    const uint16_t* x;
    const uint8_t* packed;
    const uint16_t* bias;
    uint16_t* y;
    int M, K, N;
    int kb_per_wave;        // row blocks per wave (multiple of kRun)
    int waves_k;            // waves per column block (they split K)
    int splits;             // workgroups per column block (they split K), 1..4
    int kb_per_split;       // row blocks per such workgroup (KB when splits = 1)
    uint32_t* counters;     // splits > 1: one per column block, zero on entry and exit
    float* partials;        // splits > 1: [block][split] 1 KiB fp32 partials
};

// kSub: metadata units per 128-row block (1; 2 or 4 for group sizes 64 or 32): each
// unit has its own scale, zero point, MFMA accumulator and activation sum.
// Group size 32 (kSub = 4) holds 4x the accumulators: at most 8 waves per workgroup,
// so that the register budget doubles instead of spilling.
constexpr int max_waves(int sub) { return sub == 4 ? kMaxWaves / 2 : kMaxWaves; }

// kSplit: several workgroups per column block split K and meet in the workspace
// (a separate instantiation, so that the single-workgroup kernel carries none of it)
template <bool kBF16, bool kStaged, int kChunks, int kSub, bool kSplit>
__global__ __launch_bounds__(64 * max_waves(kSub)) void gemv_kernel(const GemvArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    using Mg = Magic<kBF16>;

    const int M = a.M, K = a.K, N = a.N;
    const int KB = K / kRowsPerBlock;
    const int UW = (int)padded_units(K, kRowsPerBlock / kSub);    // metadata words per column
    const int waves = blockDim.x >> 6;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);     // wave-uniform
    const int cbl = w / a.waves_k;                                       // column block in the workgroup
    const int wk = w - cbl * a.waves_k;                                  // K slice of this wave
    const int split = kSplit ? (int)(blockIdx.x % (unsigned)a.splits) : 0;     // K range of this workgroup
    const int group = kSplit ? (int)(blockIdx.x / (unsigned)a.splits) : (int)blockIdx.x;
    const int nb_raw = group * (waves / a.waves_k) + cbl;
    const int NB = (int)(padded_cols(N) / kColsPerBlock);
    const bool nb_valid = nb_raw < NB;
    const int nb = nb_valid ? nb_raw : NB - 1;                           // a ragged last workgroup
                                                                         // repeats the last block, unstored
    const int lane = threadIdx.x & 63;
    const int c = lane & 15;         // column in the block, and activation row of the A operand
    const int h = lane >> 4;         // which 8 of every 32 rows
    // row blocks of this workgroup [kb_lo, kb_hi) and of this wave [kb_begin, kb_end)
    const int kb_lo = kSplit ? split * a.kb_per_split : 0;
    const int kb_hi = kSplit && kb_lo + a.kb_per_split < KB ? kb_lo + a.kb_per_split : KB;
    const int kb_begin = kb_lo + wk * a.kb_per_wave;
    const int kb_end = kb_begin + a.kb_per_wave < kb_hi ? kb_begin + a.kb_per_wave : kb_hi;
    const int xr = c < M ? c : 0;    // activation row this lane feeds to the MFMA

    // LDS: [staged x, M x K 16-bit, in whole 1 KiB wave copies][unit sums X,
    // KB x kSub x 16 fp32][wave partials]
    const int row_chunks = K / 8;
    const int chunks = M * row_chunks;                            // 16-byte activation chunks
    const int xs_bytes = kStaged ? (int)staged_x_bytes(chunks) : 0;
    const int xsum_bytes = kStaged ? KB * kSub * 16 * 4 : 0;
    uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
    float* xsum = reinterpret_cast<float*>(smem + xs_bytes);
    f32x4* partial = reinterpret_cast<f32x4*>(smem + xs_bytes + xsum_bytes);

    // 1. staged variant: the activations are copied global -> LDS first, ahead of the
    //    codes (chunk q to byte 16 q; wave w copies chunks 64 w + 0..63 + p blockDim.x,
    //    lanes past the end re-reading the last chunk into the padding). The copies
    //    hold no registers: an exact vmcnt wait and a barrier order them before their
    //    readers, and the codes stay in flight meanwhile. (A register load was sunk by
    //    the compiler below the code loads, whose completion it then also waited for;
    //    an inline-assembly register load with a separate wait let the compiler copy
    //    the result registers before the wait.)
    if constexpr (kStaged) {
        const uint8_t* xbase = uniform_ptr(a.x);
        const uint32_t xs_lds = lds_addr(xs);
#pragma unroll
        for (int p = 0; p < kChunks; ++p) {
            const int q0 = w * 64 + p * (int)blockDim.x;             // wave-uniform
            if (q0 < chunks) {
                const int q = q0 + lane < chunks ? q0 + lane : chunks - 1;
                dma16(xbase, 16u * (uint32_t)q, xs_lds + 16u * (uint32_t)q0);
            }
        }
    }

    // 2. codes and metadata of this wave's first run (clamped into the column block;
    //    row blocks past kb_end are loaded but weighted by zero)
    const uint4* wcol = reinterpret_cast<const uint4*>(a.packed) + (size_t)nb * KB * 64 + lane;
    const uint4* mcol = reinterpret_cast<const uint4*>(a.packed + (size_t)K * padded_cols(N) / 2) + ((size_t)(nb * kColsPerBlock + c) * UW) / 4;
    // a run's metadata: the kRun x kSub words of row blocks kb0 .. kb0 + 3 (kb0 a
    // multiple of 4), clamped to the column's words (the entries past KB weigh zero)
    auto load_run = [&](int kb0, uint4 (&wq)[kRun], uint4 (&md)[kSub]) {
#pragma unroll
        for (int s4 = 0; s4 < kSub; ++s4) {
            const int idx = ((kb0 < KB ? kb0 : KB - 1) / 4) * kSub + s4;
            md[s4] = load_once(mcol + (idx < UW / 4 ? idx : UW / 4 - 1));
        }
#pragma unroll
        for (int u = 0; u < kRun; ++u) {
            const int kb = kb0 + u < KB ? kb0 + u : KB - 1;
            wq[u] = load_once(wcol + (size_t)kb * 64);
        }
    };
    uint4 wq[kRun], md[kSub];
    load_run(kb_begin, wq, md);

    // 3. staged variant: the row-block sums X of the staged activations (rows < M; the
    //    sums of the repeated rows are never read into a kept result)
    if constexpr (kStaged) {
        // this wave's copies are done (its run's loads may still be in flight); each
        // lane sums the chunk its own copy wrote, so no barrier is needed before the
        // sums, only after them
        wait_vmcnt<kRun + kSub>();
        asm volatile("" : : : "memory");
        const float inv_row_chunks = 1.0f / (float)row_chunks;
#pragma unroll
        for (int p = 0; p < kChunks; ++p) {
            const int q = threadIdx.x + p * blockDim.x;
            // chunks of one (row, metadata unit) are 16 / kSub consecutive q within one
            // row of 16 lanes, all valid or all past the end together (row_chunks is a
            // multiple of 16)
            if (q < chunks) {
                // row of chunk q: a float estimate (q < 2^22, off by at most one) corrected exactly
                int m = (int)((float)q * inv_row_chunks);
                m -= m * row_chunks > q ? 1 : 0;
                m += (m + 1) * row_chunks <= q ? 1 : 0;
                const float s = group_sum<16 / kSub>(sum8<kBF16>(reinterpret_cast<const uint4*>(xs)[q]));
                // chunk (q - m row_chunks) is unit (q - m row_chunks) / (16 / kSub)
                if ((q & (16 / kSub - 1)) == 0) xsum[((q - m * row_chunks) / (16 / kSub)) * 16 + m] = s;
            }
        }
        __syncthreads();
    }

    // 4. runs of row blocks, the next run's loads in flight during the current one
    const uint32_t mask = pair_mask_vgpr();
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    auto compute_run = [&](const int kb0, const uint4 (&wr)[kRun], const uint4 (&mr)[kSub]) {
        // row block of each run entry (entries past kb_end read block 0's activations:
        // finite values, weighted by zero); unit v of entry u is word u kSub + v
        int kbl[kRun];
        float s[kRun][kSub];
        uint32_t z[kRun][kSub];
#pragma unroll
        for (int u = 0; u < kRun; ++u) {
            const bool valid = kb0 + u < kb_end;
            kbl[u] = valid ? kb0 + u : 0;
#pragma unroll
            for (int v = 0; v < kSub; ++v) {
                const uint32_t mdv = pick(mr[(u * kSub + v) / 4], (u * kSub + v) % 4);
                s[u][v] = valid ? half_bits_to_f32<kBF16>(mdv & 0xFFFFu) : 0.f;
                z[u][v] = (mdv >> 16) & 0xFu;
            }
        }
        f32x4 t[kRun][kSub];
#pragma unroll
        for (int u = 0; u < kRun; ++u)
#pragma unroll
            for (int v = 0; v < kSub; ++v) t[u][v] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int v = i * kSub / 4;                 // unit of 32-row step i
#pragma unroll
            for (int u = 0; u < kRun; ++u) {
                uint4 xa;
                if constexpr (kStaged)
                    xa = *reinterpret_cast<const uint4*>(xs + xr * K + kbl[u] * kRowsPerBlock + 32 * i + 8 * h);
                else
                    xa = *reinterpret_cast<const uint4*>(a.x + (size_t)xr * K + kbl[u] * kRowsPerBlock + 32 * i + 8 * h);
                t[u][v] = mfma16x16x32<kBF16>(xa, magic_operand<kBF16>(pick(wr[u], i), mask), t[u][v]);
                if constexpr (!kStaged) {
                    const uint32_t nz = Mg::kNegBase | z[u][v];         // -(base + z), exact
                    const uint32_t nz2 = nz | (nz << 16);
                    t[u][v] = mfma16x16x32<kBF16>(xa, make_uint4(nz2, nz2, nz2, nz2), t[u][v]);
                }
            }
        }
        if constexpr (kStaged) {
            if (M == 1) {      // only register 0 of lanes 0..15 holds a kept result
#pragma unroll
                for (int u = 0; u < kRun; ++u)
#pragma unroll
                    for (int v = 0; v < kSub; ++v)
                        acc[0] += s[u][v] * (t[u][v][0] - (Mg::kBase + (float)z[u][v]) * xsum[(kbl[u] * kSub + v) * 16]);
            } else {
#pragma unroll
                for (int u = 0; u < kRun; ++u)
#pragma unroll
                    for (int v = 0; v < kSub; ++v) {
                        const f32x4 xsv = *reinterpret_cast<const f32x4*>(xsum + (kbl[u] * kSub + v) * 16 + 4 * h);
                        acc += s[u][v] * (t[u][v] - (Mg::kBase + (float)z[u][v]) * xsv);
                    }
            }
        } else {
#pragma unroll
            for (int u = 0; u < kRun; ++u)
#pragma unroll
                for (int v = 0; v < kSub; ++v) acc += s[u][v] * t[u][v];
        }
    };
    const int runs = a.kb_per_wave / kRun;
    int kb0 = kb_begin;
    for (int r = 1; r < runs; ++r, kb0 += kRun) {
        uint4 wqn[kRun], mdn[kSub];
        load_run(kb0 + kRun, wqn, mdn);
        compute_run(kb0, wq, md);
#pragma unroll
        for (int u = 0; u < kRun; ++u) wq[u] = wqn[u];
#pragma unroll
        for (int v = 0; v < kSub; ++v) md[v] = mdn[v];
    }
    compute_run(kb0, wq, md);

    // 5. each column block's partials in K order
    if (a.waves_k > 1) {
        partial[w * 64 + lane] = acc;
        __syncthreads();
        if (wk != 0) return;
        const f32x4* pc = partial + cbl * a.waves_k * 64 + lane;
        acc = pc[0];
        for (int v = 1; v < a.waves_k; ++v) acc += pc[v * 64];
    }
    if (!nb_valid) return;

    // 6. K split over workgroups: publish this workgroup's partial with agent-scope
    //    stores (lane's 4 rows in two 512-byte runs of the block's 1 KiB slot), wait
    //    for them, count the block's finished splits; the last to arrive adds every
    //    split's partial in split order (its own from registers) and stores y
    if constexpr (kSplit) {
        auto slot = [&](int sp) {
            return reinterpret_cast<uint64_t*>(reinterpret_cast<uint8_t*>(a.partials) +
                                               ((size_t)nb * a.splits + sp) * 1024) + lane;
        };
        uint64_t* q = slot(split);
        __hip_atomic_store(q, __builtin_bit_cast(uint64_t, f32x2{acc[0], acc[1]}), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(q + 64, __builtin_bit_cast(uint64_t, f32x2{acc[2], acc[3]}), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(0);          // this wave's partial stores have completed
        uint32_t arrived = 0;
        if (lane == 0)
            arrived = __hip_atomic_fetch_add(&a.counters[nb], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        arrived = __builtin_amdgcn_readfirstlane(arrived);
        if (arrived != (uint32_t)(a.splits - 1)) return;
        f32x4 sum = {0.f, 0.f, 0.f, 0.f};
        for (int sp = 0; sp < a.splits; ++sp) {
            f32x4 v = acc;
            if (sp != split) {
                const uint64_t* r = slot(sp);
                const f32x2 lo = __builtin_bit_cast(f32x2, __hip_atomic_load(r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
                const f32x2 hi = __builtin_bit_cast(f32x2, __hip_atomic_load(r + 64, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
                v = f32x4{lo[0], lo[1], hi[0], hi[1]};
            }
            sum += v;
        }
        acc = sum;
        if (lane == 0)      // leave the counter at zero for the next call
            __hip_atomic_store(&a.counters[nb], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // lane (c, h), register r -> row 4h + r, column 16 nb + c (columns past N: the
    // zero padding of a last half block, not stored)
    const int n = nb * kColsPerBlock + c;
    if (n >= N) return;
    const float b = a.bias ? half_bits_to_f32<kBF16>(a.bias[n]) : 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int row = 4 * h + r;
        if (row < M) a.y[(size_t)row * N + n] = f32_to_half_bits<kBF16>(acc[r] + b);
    }
}

template <bool kBF16, int kSub, bool kSplit>
void launch_var(const GemvPlan& p, const GemvArgs& args, hipStream_t s) {
    const int cols_per_wg = p.waves / p.waves_k;
    const dim3 grid((unsigned)((padded_cols(args.N) / kColsPerBlock + cols_per_wg - 1) / cols_per_wg * p.splits));
    const dim3 block((unsigned)(64 * p.waves));
    if (!p.staged)
        hipLaunchKernelGGL((gemv_kernel<kBF16, false, 1, kSub, kSplit>), grid, block, p.lds_bytes, s, args);
    else if (p.chunks_per_thread <= 1)
        hipLaunchKernelGGL((gemv_kernel<kBF16, true, 1, kSub, kSplit>), grid, block, p.lds_bytes, s, args);
    else if (p.chunks_per_thread <= 2)
        hipLaunchKernelGGL((gemv_kernel<kBF16, true, 2, kSub, kSplit>), grid, block, p.lds_bytes, s, args);
    else if (p.chunks_per_thread <= 4)
        hipLaunchKernelGGL((gemv_kernel<kBF16, true, 4, kSub, kSplit>), grid, block, p.lds_bytes, s, args);
    else
        hipLaunchKernelGGL((gemv_kernel<kBF16, true, 8, kSub, kSplit>), grid, block, p.lds_bytes, s, args);
}

template <bool kBF16, int kSub>
void launch_sub(const GemvPlan& p, const GemvArgs& args, hipStream_t s) {
    if (p.splits > 1) launch_var<kBF16, kSub, true>(p, args, s);
    else launch_var<kBF16, kSub, false>(p, args, s);
}

template <bool kBF16>
void launch_typed(const GemvPlan& p, const GemvArgs& args, hipStream_t s) {
    if (p.sub == 4) launch_sub<kBF16, 4>(p, args, s);
    else if (p.sub == 2) launch_sub<kBF16, 2>(p, args, s);
    else launch_sub<kBF16, 1>(p, args, s);
}

}  // namespace

GemvPlan plan_gemv_with(int64_t M, int64_t K, int64_t N, int64_t G, int cols_per_wg, int splits) {
    (void)N;
    GemvPlan p;
    p.sub = units_per_block(G);
    const int64_t KB = K / kRowsPerBlock;
    p.splits = splits;
    // a whole number of runs per split: a run's metadata is one 16-byte load of the
    // words of 4 row blocks, the first a multiple of 4
    p.kb_per_split = (int)(((KB + splits - 1) / splits + kRun - 1) / kRun * kRun);
    p.workspace_bytes = 0;
    // runs of 4 row blocks per wave, at most 16 waves (8 for group size 32) per workgroup
    const int wmax = max_waves(p.sub);
    int64_t kpw = kRun;
    while ((p.kb_per_split + kpw - 1) / kpw > wmax) kpw += kRun;
    p.kb_per_wave = (int)kpw;
    p.waves_k = (int)((p.kb_per_split + kpw - 1) / kpw);
    if (cols_per_wg < 1 || cols_per_wg * p.waves_k > wmax) cols_per_wg = 1;
    p.waves = p.waves_k * cols_per_wg;
    const int64_t threads = 64 * p.waves;
    const size_t partial_bytes = p.waves_k > 1 ? (size_t)p.waves * 64 * 16 : 0;
    const size_t staged_bytes = (size_t)staged_x_bytes(M * K / 8) + (size_t)KB * p.sub * 16 * 4 + partial_bytes;
    p.chunks_per_thread = (int)((M * K / 8 + threads - 1) / threads);
    p.staged = staged_bytes <= kStagedLdsLimit && p.chunks_per_thread <= kMaxStagedChunksPerThread;
    p.lds_bytes = p.staged ? staged_bytes : partial_bytes;
    return p;
}

// Two column blocks per workgroup when there are at least 400 blocks and either N is
// mid-sized (at most 1024 blocks) or M >= 4: the workgroups' copies of the
// activations (M x K each) then serve twice the columns. Measured on the 2048 x 13312
// decode shape: M = 8 -9%, M = 4 -4%, M = 1 even; on 2048 x 131072: M = 8 -18%
// (45.5 -> 37.2 us), M = 12 -11%, M = 4 -5%, M = 1 and 2 even. Four blocks per
// workgroup measured slower everywhere, and two on 2048 x 3072 (192 blocks).
//
// Outputs of at most 128 column blocks leave CUs idle with one workgroup per block
// (the down projection, N = 2048: 128 of 256); there, for K >= 6144 from M = 6 and
// given a workspace for the partials, 2-4 workgroups split each block's K range so
// that the grid reaches 256 workgroups, meeting as the MFMA GEMM's K splits do.
// Measured on 6656 x 2048: M = 6 7.27 -> 7.02 us, M = 8 7.63 -> 7.2 us, M = 12 8.7
// -> 7.8 us, M = 16 9.9 -> 8.4 us; at M = 1 .. 4, and at any M up to 8 for K = 2048
// and 4096 (each workgroup then keeps 16 row blocks or fewer), the meeting's round
// trip cost more than the idle CUs (2048 x 2048, M = 8: 4.43 -> 4.95 us).
GemvPlan plan_gemv(int64_t M, int64_t K, int64_t N, int64_t G, size_t workspace_bytes) {
    const int64_t NB = padded_cols(N) / kColsPerBlock;
    const int64_t KB = K / kRowsPerBlock;
    const GemvPlan one = plan_gemv_with(M, K, N, G, 1, 1);
    if ((NB <= 1024 || M >= 4) && NB / 2 >= 200 && 2 * one.waves_k <= max_waves(one.sub))
        return plan_gemv_with(M, K, N, G, 2, 1);
    if (M >= 6 && NB <= kMaxSplitTiles && KB >= 48) {
        int64_t splits = 256 / NB;
        if (splits > KB / 8) splits = KB / 8;
        if (splits > 4) splits = 4;
        const size_t need = kSplitCounterBytes + (size_t)splits * (size_t)NB * 1024;
        if (splits >= 2 && workspace_bytes >= need) {
            GemvPlan p = plan_gemv_with(M, K, N, G, 1, (int)splits);
            p.workspace_bytes = need;
            return p;
        }
    }
    return one;
}

hipError_t launch_gemv(const uint16_t* x, const uint8_t* packed, const uint16_t* bias, uint16_t* y,
                       int64_t M, int64_t K, int64_t N, int64_t G, bool bf16, void* workspace,
                       size_t workspace_bytes, hipStream_t stream) {
    if (M >= 2) {
        const SmallPlan sp = plan_gemv_small(M, K, N, G);
        if (sp.ok) return launch_gemv_small(sp, x, packed, bias, y, M, K, N, G, bf16, stream);
    }
    if (M == 1) {
        const StripPlan sp = plan_gemv_strip(M, K, N, G);
        if (sp.ok) return launch_gemv_strip(sp, x, packed, bias, y, K, N, G, bf16, stream);
    }
    const GemvPlan p = plan_gemv(M, K, N, G, workspace ? workspace_bytes : 0);
    GemvArgs args;
    args.x = x;
    args.packed = packed;
    args.bias = bias;
    args.y = y;
    args.M = (int)M;
    args.K = (int)K;
    args.N = (int)N;
    args.kb_per_wave = p.kb_per_wave;
    args.waves_k = p.waves_k;
    args.splits = p.splits;
    args.kb_per_split = p.kb_per_split;
    args.counters = static_cast<uint32_t*>(workspace);
    args.partials = p.splits > 1 ? reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + kSplitCounterBytes)
                                 : nullptr;
    if (bf16) launch_typed<true>(p, args, stream);
    else launch_typed<false>(p, args, stream);
    return hipGetLastError();
}

}  // namespace w4a16
