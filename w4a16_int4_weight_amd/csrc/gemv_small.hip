// Decode GEMV for small batches (2 <= M <= 16) on the matrix cores, balanced over the
// compute units.
//
// Like the M = 1 GEMV, the work is cut into equal shares of 8-column half blocks over
// the whole K range, one workgroup per compute unit, so no output needs a partial sum
// from another workgroup. With several activation rows each weight feeds M products,
// and packed dot products would cost M times the decode; here a 16x16x32 MFMA does the
// products of all rows:
//
//   * the MFMA's first operand is 16 weight columns x 32 rows: the half block's 8
//     columns at row block 2p and the same 8 columns at row block 2p + 1 (a "unit").
//     The second operand's 16 columns carry up to 8 activation rows twice, once over
//     each row block's k range; the cross terms are not used. M = 9 .. 16 runs two such
//     row groups, each decoded operand feeding one MFMA per group;
//   * lane (h, c) holds the 16 code bytes of its column at lane 16 h + c of the 1 KiB
//     tile block, which is word i of the first operand for k step i: the layout is
//     already in operand order. Its activations are four 16-byte loads from global
//     memory (L2-resident after the first workgroups); every load of a lane is issued
//     before the first is used, with no barrier and no branch;
//   * codes enter the MFMA as base + q (masked into 128.0 or 1024.0, exact), so the
//     decode is one or two instructions per pair. Per unit the tile T is corrected
//     once: s (T - (base + z) X), X the sum of the activations of the row over the
//     row block (the lane's 32 values by packed dot products with (1, 1), then the
//     four lanes of the column), s and z those of the output's column (the lanes
//     that loaded them pass them on through LDS);
//   * a half block's units are dealt to the 8 waves in turn (unit p to wave p mod 8);
//     each wave adds its units per half block and the waves' tiles are added in wave
//     order through LDS: run-to-run deterministic.
#include "device_common.h"
#include "launch.h"

namespace w4a16 {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxItems = 8;                // units in flight per lane
constexpr int kTargetWorkgroups = 256;      // one per compute unit

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_once(const uint8_t* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t load_md(const uint8_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}
__device__ __forceinline__ uint32_t pick(const uint4 v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

struct SmallArgs {
    const uint16_t* x;
    const uint8_t* packed;
    const uint16_t* bias;
    uint16_t* y;
    int M, K, N;
    int KB;          // row blocks
    int UW;          // metadata words per column (one per row block, padded to 4)
    int U;           // half blocks, N / 8
    int P;           // units (row-block pairs) per half block
};

// The nibble-pair mask in a VGPR, so each pair decodes with one v_and_or_b32 (a
// three-operand instruction reads at most one scalar or literal constant).
__device__ __forceinline__ uint32_t pair_mask_vgpr() {
    uint32_t m;
    asm volatile("v_mov_b32 %0, 0x000f000f" : "=v"(m));
    return m;
}

template <bool kBF16>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    if constexpr (kBF16)
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
    else
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
}

// Metadata word -> scale and base + zero point as fp32 (the zero point's 4 bits land
// on the units bit of 128.0 or 1024.0).
template <bool kBF16>
__device__ __forceinline__ float md_scale(uint32_t md) {
    return half_bits_to_f32<kBF16>(md & 0xFFFFu);
}
template <bool kBF16>
__device__ __forceinline__ float md_base_zero(uint32_t md) {
    return kBF16 ? __uint_as_float((md & 0x000F0000u) | 0x43000000u)              // 128 + z
                 : __uint_as_float(((md >> 3) & 0x0001E000u) | 0x44800000u);      // 1024 + z
}

// kS >= half blocks of any workgroup (exactly), kJP >= units per wave per half block
// (a power of two), kG row groups of at most 8 activation rows (rows 8 g .. 8 g + 7; two for
// M = 9 .. 16): each decoded operand serves one MFMA per group.
template <bool kBF16, int kS, int kJP, int kG>
__global__ __launch_bounds__(kThreads) void gemv_small_kernel(const SmallArgs a) {
    using Mg = Magic<kBF16>;
    __shared__ f32x4 part[kG][kS][kWaves][64];
    __shared__ __attribute__((aligned(16))) uint32_t mdx[kWaves][kS * kJP][16];
    constexpr int kItems = kS * kJP;
    constexpr uint32_t kOnes = kBF16 ? 0x3F803F80u : 0x3C003C00u;      // (1.0, 1.0)
    const int M = a.M, K = a.K, KB = a.KB, P = a.P;
    const int nwg = (int)gridDim.x;
    const int g = (int)blockIdx.x;
    const int u_lo = (int)((int64_t)g * a.U / nwg);
    const int S = (int)((int64_t)(g + 1) * a.U / nwg) - u_lo;    // >= 1 (U >= number of workgroups)
    const int tid = (int)threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int c = lane & 15;
    const int h = lane >> 4;
    const int c8 = c & 7;
    const int hi = c >> 3;                   // first operand: the unit's second row block
    // group rg holds rows 8 rg .. 8 rg + R - 1 (R = min(8, M - 8 rg)); its second operand's
    // column c is row 8 rg + c - bsel R over the unit's first (bsel = 0) or second
    // (bsel = 1) row block; columns past 2R read row M - 1 and their outputs are not used
    int R[kG], bsel[kG], mrow[kG];
#pragma unroll
    for (int rg = 0; rg < kG; ++rg) {
        R[rg] = M - 8 * rg < 8 ? M - 8 * rg : 8;
        bsel[rg] = c >= R[rg] ? 1 : 0;
        const int r = c - bsel[rg] * R[rg];
        mrow[rg] = r < R[rg] ? 8 * rg + r : M - 1;
    }
    const uint8_t* meta_plane = a.packed + (size_t)KB * kRowsPerBlock * padded_cols(a.N) / 2;

    // 1. loads, all issued before the first is used and none under a branch: the
    //    activations of each unit jp and row group (they serve every half block), then
    //    per unit j = (half block s = j / kJP, unit p = w + 8 (j % kJP)) the 16 code bytes
    //    and the metadata word of the lane's first-operand column. Units past this
    //    workgroup's half blocks or past P, and a unit's missing second row block, read a
    //    valid line and take scale 0: their contribution is 0.
    uint4 xv[kG][kJP][4];
#pragma unroll
    for (int rg = 0; rg < kG; ++rg) {
#pragma unroll
        for (int jp = 0; jp < kJP; ++jp) {
            const int p = w + kWaves * jp;
            const int kbb = 2 * p + bsel[rg];
            const int kbc = kbb < KB ? kbb : KB - 1;
            const uint4* xp =
                reinterpret_cast<const uint4*>(a.x + (size_t)mrow[rg] * K + kRowsPerBlock * kbc + 8 * h);
#pragma unroll
            for (int i = 0; i < 4; ++i) xv[rg][jp][i] = xp[4 * i];
        }
    }
    uint4 wq[kItems];
    uint32_t md[kItems];
    bool mval[kItems];
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
        const int s = j / kJP;
        const int p = w + kWaves * (j % kJP);
        const int u = u_lo + (s < S ? s : S - 1);
        const bool unit = s < S && p < P;
        const int kba = 2 * p + hi;
        const int kbac = kba < KB ? kba : KB - 1;
        const size_t blk = (size_t)(u >> 1) * KB + kbac;
        wq[j] = load_once(a.packed + blk * kBlockBytes + 16 * (16 * h + 8 * (u & 1) + c8));
        md[j] = load_md(meta_plane + 4 * ((size_t)(8 * u + c8) * a.UW + kbac));
        mval[j] = unit && 2 * p + (h >> 1) < KB;     // the output registers' row block
    }
    // nothing below moves above the loads
    __builtin_amdgcn_sched_barrier(0);

    // 2. X of the lane's second-operand column per unit and group: its 32 values, then
    //    the sum over the four lanes (h = 0..3) of the column
    float xsum[kG][kJP];
#pragma unroll
    for (int rg = 0; rg < kG; ++rg) {
#pragma unroll
        for (int jp = 0; jp < kJP; ++jp) {
            float s0 = 0.f, s1 = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                s0 = dot2<kBF16>(xv[rg][jp][i].x, kOnes, s0);
                s1 = dot2<kBF16>(xv[rg][jp][i].y, kOnes, s1);
                s0 = dot2<kBF16>(xv[rg][jp][i].z, kOnes, s0);
                s1 = dot2<kBF16>(xv[rg][jp][i].w, kOnes, s1);
            }
            float t = s0 + s1;
            t += __shfl_xor(t, 16);
            t += __shfl_xor(t, 32);
            xsum[rg][jp] = t;
        }
    }

    // 3. per unit: T = sum of (base + q) x over its k range, one MFMA per k step and
    //    group; the tile is transposed (lane (h, c), register e: weight column 4 h + e
    //    against second-operand column c); contribution s (T - (base + z) X) with the
    //    scale and zero point of weight column 4 h + e
    const uint32_t mask = pair_mask_vgpr();
    f32x4 acc[kG][kS];
#pragma unroll
    for (int rg = 0; rg < kG; ++rg)
#pragma unroll
        for (int s = 0; s < kS; ++s) acc[rg][s] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
        const int s = j / kJP;
        const int jp = j % kJP;
        // the metadata of weight columns 4 h .. 4 h + 3: lane c of row 0 holds column c's,
        // staged in this wave's LDS slot and read back 16 bytes at a time (LDS accesses
        // of one wave complete in order: no barrier)
        if (h == 0) mdx[w][j][c] = md[j];
        const uint4 m4 = *reinterpret_cast<const uint4*>(&mdx[w][j][4 * h]);
        const uint32_t mdo[4] = {m4.x, m4.y, m4.z, m4.w};
        f32x4 t[kG];
#pragma unroll
        for (int rg = 0; rg < kG; ++rg) t[rg] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t v = pick(wq[j], i);
            const uint4 b = make_uint4((v & mask) | Mg::kBase2, ((v >> 4) & mask) | Mg::kBase2,
                                       ((v >> 8) & mask) | Mg::kBase2, ((v >> 12) & mask) | Mg::kBase2);
#pragma unroll
            for (int rg = 0; rg < kG; ++rg) t[rg] = mfma16x16x32<kBF16>(b, xv[rg][jp][i], t[rg]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float sc = mval[j] ? md_scale<kBF16>(mdo[e]) : 0.f;
            const float zb = md_base_zero<kBF16>(mdo[e]);
#pragma unroll
            for (int rg = 0; rg < kG; ++rg)
                acc[rg][s][e] = fmaf(sc, fmaf(-zb, xsum[rg][jp], t[rg][e]), acc[rg][s][e]);
        }
    }
#pragma unroll
    for (int rg = 0; rg < kG; ++rg)
#pragma unroll
        for (int s = 0; s < kS; ++s) part[rg][s][w][lane] = acc[rg][s];
    __syncthreads();

    // 4. output (row m, column 8 (u_lo + s) + jc): the waves' tiles added in wave order
    //    (a unit's two row blocks sit at weight columns jc and jc + 8, second-operand
    //    columns r and r + R of row m = 8 rg + r), bias, one rounding; 8 consecutive
    //    threads write one row's 16 contiguous bytes
    const int outs = S * 8 * M;
    for (int o = tid; o < outs; o += kThreads) {
        const int s = o / (8 * M);
        const int rr = o - s * 8 * M;
        const int m = rr >> 3;
        const int jc = rr & 7;
        const int rg = kG > 1 ? m >> 3 : 0;
        const int r = m - 8 * rg;
        const int Rg = M - 8 * rg < 8 ? M - 8 * rg : 8;
        float sum = 0.f;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) {
            sum += part[rg][s][ww][16 * (jc >> 2) + r][jc & 3];
            sum += part[rg][s][ww][16 * (2 + (jc >> 2)) + r + Rg][jc & 3];
        }
        const int n = 8 * (u_lo + s) + jc;
        const float b = a.bias ? half_bits_to_f32<kBF16>(a.bias[n]) : 0.f;
        a.y[(size_t)m * a.N + n] = f32_to_half_bits<kBF16>(sum + b);
    }
}

// kS = the most half blocks of any workgroup, exactly (3, 5, 6 and 7 included: a power
// of two above it would issue loads of clamped units that weigh nothing)
template <bool kBF16, int kJP, int kG>
void launch_jp(const SmallArgs& args, int smax, int grid, hipStream_t st) {
    constexpr int kMaxS = kMaxItems / kJP;
    if (smax <= 1) hipLaunchKernelGGL((gemv_small_kernel<kBF16, 1, kJP, kG>), dim3(grid), dim3(kThreads), 0, st, args);
    else if (smax == 2 && kMaxS >= 2)
        hipLaunchKernelGGL((gemv_small_kernel<kBF16, (kMaxS >= 2 ? 2 : 1), kJP, kG>), dim3(grid), dim3(kThreads), 0, st,
                           args);
    else if (smax == 3 && kMaxS >= 4)
        hipLaunchKernelGGL((gemv_small_kernel<kBF16, (kMaxS >= 4 ? 3 : 1), kJP, kG>), dim3(grid), dim3(kThreads), 0, st,
                           args);
    else if (smax == 4 && kMaxS >= 4)
        hipLaunchKernelGGL((gemv_small_kernel<kBF16, (kMaxS >= 4 ? 4 : 1), kJP, kG>), dim3(grid), dim3(kThreads), 0, st,
                           args);
    else if (smax == 5 && kMaxS >= 8)
        hipLaunchKernelGGL((gemv_small_kernel<kBF16, (kMaxS >= 8 ? 5 : 1), kJP, kG>), dim3(grid), dim3(kThreads), 0, st,
                           args);
    else if (smax == 6 && kMaxS >= 8)
        hipLaunchKernelGGL((gemv_small_kernel<kBF16, (kMaxS >= 8 ? 6 : 1), kJP, kG>), dim3(grid), dim3(kThreads), 0, st,
                           args);
    else if (smax == 7 && kMaxS >= 8)
        hipLaunchKernelGGL((gemv_small_kernel<kBF16, (kMaxS >= 8 ? 7 : 1), kJP, kG>), dim3(grid), dim3(kThreads), 0, st,
                           args);
    else if (kMaxS >= 8)
        hipLaunchKernelGGL((gemv_small_kernel<kBF16, (kMaxS >= 8 ? 8 : 1), kJP, kG>), dim3(grid), dim3(kThreads), 0, st,
                           args);
}

template <bool kBF16, int kG>
void launch_groups(const SmallArgs& args, int JP, int smax, int grid, hipStream_t st) {
    if (JP <= 1) launch_jp<kBF16, 1, kG>(args, smax, grid, st);
    else if (JP <= 2) launch_jp<kBF16, 2, kG>(args, smax, grid, st);
    else if (JP <= 4) launch_jp<kBF16, 4, kG>(args, smax, grid, st);
    else if constexpr (kG == 1) launch_jp<kBF16, 8, kG>(args, smax, grid, st);
}

template <bool kBF16>
void launch_typed(const SmallArgs& args, int JP, int smax, int grid, hipStream_t st) {
    if (args.M <= 8) launch_groups<kBF16, 1>(args, JP, smax, grid, st);
    else launch_groups<kBF16, 2>(args, JP, smax, grid, st);
}

int pow2_at_least(int64_t v) {
    int r = 1;
    while (r < v) r *= 2;
    return r;
}

}  // namespace

SmallPlan plan_gemv_small(int64_t M, int64_t K, int64_t N, int64_t G) {
    SmallPlan p{};
    p.ok = false;
    if (M < 2 || M > 16 || G < kRowsPerBlock) return p;
    const int64_t U = N / 8;
    const int64_t KB = K / kRowsPerBlock;
    // At M = 2 and 3 the packed-dot-product GEMV is faster where it gives every compute
    // unit a column block (measured: gate_up 2048 x 13312 5.9 against 6.6 us at M = 2,
    // qkv 2048 x 3072 3.6 against 3.8 us); from M = 4, and on outputs of at most 128
    // column blocks (down_proj 6656 x 2048 M = 2: 6.3 against 5.6 us), this kernel is.
    if (M < 4 && padded_cols(N) / kColsPerBlock > 128) return p;
    // Two row groups (M = 9 .. 16) pay on wide outputs only: every workgroup reads all
    // M x K activations for its half blocks (gate_up 2048 x 13312, M = 16: 7.96 against
    // 10.2 us for the MFMA GEMM; qkv 2048 x 3072 5.0 against 5.0 us and down_proj
    // 6656 x 2048 10.8 against 8.6 us for the 16-column GEMV).
    if (M > 8 && padded_cols(N) / kColsPerBlock < 512) return p;
    p.P = (int)((KB + 1) / 2);
    p.grid = (int)(U < kTargetWorkgroups ? U : kTargetWorkgroups);
    p.smax = (int)((U + p.grid - 1) / p.grid);
    p.JP = (p.P + kWaves - 1) / kWaves;
    if ((int64_t)pow2_at_least(p.smax) * pow2_at_least(p.JP) > kMaxItems) return p;
    // two row groups hold twice the activations: at most 4 units per wave
    if (M > 8 && pow2_at_least(p.JP) > 4) return p;
    p.ok = true;
    return p;
}

hipError_t launch_gemv_small(const SmallPlan& plan, const uint16_t* x, const uint8_t* packed, const uint16_t* bias,
                             uint16_t* y, int64_t M, int64_t K, int64_t N, int64_t G, bool bf16, hipStream_t stream) {
    if (!plan.ok || plan.smax < 1 || pow2_at_least(plan.smax) * pow2_at_least(plan.JP) > kMaxItems ||
        M < 2 || M > 16 || (M > 8 && pow2_at_least(plan.JP) > 4))
        return hipErrorInvalidValue;
    SmallArgs args;
    args.x = x;
    args.packed = packed;
    args.bias = bias;
    args.y = y;
    args.M = (int)M;
    args.K = (int)K;
    args.N = (int)N;
    args.KB = (int)(K / kRowsPerBlock);
    args.UW = (int)padded_units(K, G);
    args.U = (int)(N / 8);
    args.P = plan.P;
    const int JP = pow2_at_least(plan.JP);
    const int smax = plan.smax;
    if (bf16) launch_typed<true>(args, JP, smax, plan.grid, stream);
    else launch_typed<false>(args, JP, smax, plan.grid, stream);
    return hipGetLastError();
}

}  // namespace w4a16
