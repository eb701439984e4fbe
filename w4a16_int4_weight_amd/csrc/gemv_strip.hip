// Decode GEMV for one activation row (M = 1), balanced over the compute units.
//
// A decode step touches each weight once per generated token, so its time is the
// time to stream the packed codes (vllm-omni commit "Add cpu_int4, an asymmetric
// 4-bit weight path for vLLM's CPU backend", on why weight size decides decode
// speed). On this GPU a
// stream of a few megabytes ends when the compute unit holding the most bytes has
// received them, so the work is cut into equal shares, one per compute unit:
//
//   * the unit of work is a half block: 8 of the 16 columns of a column block over
//     the whole K range. In every 1 KiB tile block those 8 columns are four whole
//     128-byte lines (lanes 16h + c, c < 8 or c >= 8), so a half block is read with
//     no wasted bytes, and its outputs need no other workgroup: no K split, no
//     partial sums in memory;
//   * share g of G takes half blocks [g U / G, (g + 1) U / G) of the U = N / 8,
//     so no compute unit holds more than one half block above the average (the
//     16-column GEMV over 832 blocks leaves 160 compute units with two workgroups);
//     neighbouring shares go to workgroups on one XCD (xcd_share), which put the two
//     halves of a column block behind one L2: 3.42 -> 3.29 us on the qkv decode
//     (2048 x 3072), no change on 6656 x 2048 and 2048 x 13312;
//   * its 64 groups of 8 lanes split each half block's (row block, lane quarter h)
//     pairs: group q takes quarter h = q % 4 of JP consecutive row blocks from
//     JP (q / 4) on (JP = ceil(K / 2048), a power of two). Lane c of a group loads the
//     16 bytes of column c (32 codes of rows 32i + 8h + e) per row block with one
//     nontemporal 128-bit load, and the column's JP metadata words for those row
//     blocks with one load; every load of the workgroup is issued before the first
//     is used;
//   * a code pair (rows 2t, 2t+1 sit in nibble slots t and t + 4) masked into the
//     16-bit value 128.0 (bf16) or 1024.0 (fp16) gives base + q exactly, so one
//     packed dot product with the matching activation pair sums x (base + q) with
//     exact products; base and zero point leave in one correction per row block and
//     lane quarter, s (T - (base + z) X) with X the sum of the same 32 activations;
//   * the activations a lane needs (32 per row block) sit in its registers, read once
//     from LDS: with one row block per group from the wave's own copy of its two row
//     blocks (one direct global -> LDS copy per wave, no barrier; 2048 x 13312: 5.35
//     -> 5.25 us against four 16-byte loads per lane), with several from a copy of all
//     K of them that the workgroup stages (each value then serves the 8 lanes of its
//     group without 8 separate global reads); both copies are issued ahead of the code
//     loads;
//   * each group's partial per half block lands in its own LDS slot and the slots
//     are added in group order: the result is run-to-run deterministic.
#include "device_common.h"
#include "launch.h"

namespace w4a16 {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kGroups = kThreads / 8;       // 8-lane groups, one column each lane
constexpr int kMaxItems = 16;               // code loads in flight per lane
constexpr int kMaxPairsPerGroup = 4;        // row blocks per group (K <= 8192)
constexpr int kTargetWorkgroups = 256;      // one per compute unit

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_once(const uint8_t* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint32_t pick(const uint4 v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

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

struct StripArgs {
    const uint16_t* x;
    const uint8_t* packed;
    const uint16_t* bias;
    uint16_t* y;
    int K, N;
    int KB;          // row blocks
    int UW;          // metadata words per column (G >= 128: one per row block, padded to 4)
    int U;           // half blocks, N / 8
    int P;           // (row block, lane quarter) pairs, 4 KB
    int smax;        // most half blocks of any workgroup, ceil(U / G)
    int smax_pow2;   // smax rounded up to a power of two (the partials' LDS rows)
};

// LDS: the partials, smax half blocks x 8 columns x 64 group slots, fp32; then the
// activations: with several row blocks per group all K 16-bit values (padded to 1 KiB),
// with one a 1 KiB slot per wave for its two row blocks
__host__ __device__ inline int part_bytes(int smax) { return smax * 8 * kGroups * 4; }

__device__ __forceinline__ uint32_t load4(const uint8_t* p) { return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p)); }

// n consecutive 32-bit words (n = 1, 2 or 4; the address a multiple of 4 n bytes) in
// one load
template <int n>
__device__ __forceinline__ void load_words(const uint8_t* p, uint32_t (&w)[n]) {
    if constexpr (n == 1) {
        w[0] = load4(p);
    } else if constexpr (n == 2) {
        typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
        w[0] = v.x;
        w[1] = v.y;
    } else {
        static_assert(n == 4, "1, 2 or 4 words");
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        w[0] = v.x;
        w[1] = v.y;
        w[2] = v.z;
        w[3] = v.w;
    }
}

// kS >= smax half blocks per workgroup (exactly smax up to 8, else 16) and kJP row
// blocks per group per half block (a power of two): kS * kJP items per lane. Group q takes lane quarter h = q % 4 of
// row blocks kJP (q / 4) .. kJP (q / 4) + kJP - 1, so the metadata words of a lane's
// items in one column are consecutive: one load per half block. Every load of a lane
// is issued up front, in this order: the activations (with one row block per group,
// each wave's copy of its two row blocks into its own LDS slot, L2-resident after the
// first workgroups read them; with several, the workgroup's copy of all of them into
// LDS), then per half block the metadata words and the 16 code bytes of each row block.
template <bool kBF16, int kS, int kJP>
__global__ __launch_bounds__(kThreads) void gemv_strip_kernel(const StripArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    using Mg = Magic<kBF16>;
    constexpr int kItems = kS * kJP;
    constexpr uint32_t kOnes = kBF16 ? 0x3F803F80u : 0x3C003C00u;      // (1.0, 1.0)
    const int KB = a.KB, UW = a.UW;
    const int nwg = (int)gridDim.x;
    const int g = xcd_share((int)blockIdx.x, nwg);
    const int u_lo = (int)((int64_t)g * a.U / nwg);
    const int S = (int)((int64_t)(g + 1) * a.U / nwg) - u_lo;    // >= 1 (U >= number of workgroups)
    const int tid = (int)threadIdx.x;
    const int q = tid >> 3;            // group
    const int c = tid & 7;             // column of the half block
    const int hq = q & 3;              // lane quarter of the tile block
    const int rb0 = kJP * (q >> 2);    // the group's first row block
    float* part = reinterpret_cast<float*>(smem);

    // 1. loads; row blocks past the last (groups with nothing to do, or the last
    //    group's tail) load a valid line and weigh 0, and such a group's metadata load
    //    reads the column's last kJP words (UW is a multiple of 4)
    constexpr bool kXLds = kJP > 1;
    uint4 xr[kJP][4];
    uint8_t* xs = smem + part_bytes(a.smax_pow2);
    if constexpr (kXLds) {
        const int nx = a.K / 8;
        const uint8_t* xb = uniform_ptr(a.x);
        const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int lane = tid & 63;
        for (int c0 = w * 64; c0 < nx; c0 += kThreads) {
            const int ch = c0 + lane < nx ? c0 + lane : nx - 1;
            dma16(xb, 16u * (uint32_t)ch, lds_addr(xs) + 16u * (uint32_t)c0);
        }
    } else {
        // with one row block per group, wave w's groups use row blocks 2w and 2w + 1:
        // 512 contiguous bytes of x, copied into the wave's own 1 KiB LDS slot with one
        // copy (lanes past 32, and row blocks past the last, copy the last valid chunk)
        // instead of four 16-byte loads per lane; only this wave reads the slot
        const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int lane = tid & 63;
        const int nx = a.K / 8;                                   // 16-byte chunks of x
        const int ch = 32 * w + (lane & 31) < nx ? 32 * w + (lane & 31) : nx - 1;
        dma16(uniform_ptr(a.x), 16u * (uint32_t)ch, lds_addr(xs) + 1024u * (uint32_t)w);
    }
    const uint8_t* meta_plane = a.packed + (size_t)KB * 128 * padded_cols(a.N) / 2;
    const int rbm = rb0 + kJP <= UW ? rb0 : UW - kJP;
    uint32_t md[kS][kJP];
    uint4 wq[kItems];
    // with several row blocks per group, a wave whose groups all start past the last
    // row block (wave w's groups start at row blocks 2 w kJP and (2 w + 1) kJP) issues
    // no code or metadata loads and adds nothing (6656 x 2048, the 8th wave: 4.56 ->
    // 4.45 us; with one row block per group the branch measured ~1% slower on qkv)
    const bool idle = kXLds && kJP * 2 * __builtin_amdgcn_readfirstlane(tid >> 6) >= KB;
    if (!idle)
#pragma unroll
    for (int s = 0; s < kS; ++s) {
        const int u = u_lo + (s < S ? s : S - 1);
        load_words<kJP>(meta_plane + 4 * ((size_t)(8 * u + c) * UW + rbm), md[s]);
#pragma unroll
        for (int jj = 0; jj < kJP; ++jj) {
            const int rb = rb0 + jj < KB ? rb0 + jj : KB - 1;
            const uint32_t blk = (uint32_t)(u >> 1) * (uint32_t)KB + (uint32_t)rb;    // < 2^27 (K N <= 2^37)
            wq[s * kJP + jj] = load_once(a.packed + (size_t)blk * 1024 + (256 * hq + 128 * (u & 1) + 16 * c));
        }
    }

    // 2. with LDS activations: once this wave's copies have landed (at most the
    //    kS + kItems metadata and code loads outstanding) and a barrier for the other
    //    waves' copies, each row block's 32 values of the lane quarter into registers,
    //    read once. Then X of each row block: the sum of its 32 activations, as packed
    //    dot products with (1, 1).
    if constexpr (!kXLds) {
        // this wave's copy has landed once at most the kS metadata and kItems code loads
        // issued after it are outstanding; no other wave's copy is read, so no barrier
        wait_vmcnt<kS + kItems>();
        const uint8_t* xp = xs + 1024 * (tid >> 6) + 2 * (128 * (rb0 & 1) + 8 * hq);   // rb0 = 2w or 2w + 1
#pragma unroll
        for (int i = 0; i < 4; ++i) xr[0][i] = *reinterpret_cast<const uint4*>(xp + 64 * i);
    }
    if constexpr (kXLds) {
        if (idle) wait_vmcnt<0>();
        else wait_vmcnt<kS + kItems>();
        lds_barrier();
#pragma unroll
        for (int jj = 0; jj < kJP; ++jj) {
            const int rb = rb0 + jj < KB ? rb0 + jj : KB - 1;
            const uint8_t* xp = xs + 2 * (128 * rb + 8 * hq);
#pragma unroll
            for (int i = 0; i < 4; ++i) xr[jj][i] = *reinterpret_cast<const uint4*>(xp + 64 * i);
        }
    }
    float xsum[kJP];
#pragma unroll
    for (int jj = 0; jj < kJP; ++jj) {
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s0 = dot2<kBF16>(xr[jj][i].x, kOnes, s0);
            s1 = dot2<kBF16>(xr[jj][i].y, kOnes, s1);
            s0 = dot2<kBF16>(xr[jj][i].z, kOnes, s0);
            s1 = dot2<kBF16>(xr[jj][i].w, kOnes, s1);
        }
        xsum[jj] = s0 + s1;
    }

    // 3. each item: T = sum of x (base + q) over its 32 rows, contribution
    //    s (T - (base + z) X); a half block's contributions summed in item order and
    //    written to the group's slot
    const uint32_t mask = pair_mask_vgpr();
    float acc = 0.f;
    if (idle) {
#pragma unroll
        for (int s = 0; s < kS; ++s)
            if (s < S) part[(s * 8 + c) * kGroups + q] = 0.f;
    } else
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
        const int s = j / kJP;
        const int jj = j % kJP;
        const bool valid = s < S && rb0 + jj < KB;
        float t0 = 0.f, t1 = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t v = pick(wq[j], i);
            t0 = dot2<kBF16>((v & mask) | Mg::kBase2, xr[jj][i].x, t0);
            t1 = dot2<kBF16>(((v >> 4) & mask) | Mg::kBase2, xr[jj][i].y, t1);
            t0 = dot2<kBF16>(((v >> 8) & mask) | Mg::kBase2, xr[jj][i].z, t0);
            t1 = dot2<kBF16>(((v >> 12) & mask) | Mg::kBase2, xr[jj][i].w, t1);
        }
        const uint32_t m = md[s][jj];
        const float sf = half_bits_to_f32<kBF16>(m & 0xFFFFu);
        const float zb = Mg::kBase + (float)((m >> 16) & 0xFu);
        const float contrib = sf * ((t0 + t1) - zb * xsum[jj]);
        acc += valid ? contrib : 0.f;
        if (jj == kJP - 1) {
            if (s < S) part[(s * 8 + c) * kGroups + q] = acc;
            acc = 0.f;
        }
    }
    wait_lgkmcnt0();
    lds_barrier();

    // 4. output 8 (u_lo + s) + c: its 64 group slots summed by 8 consecutive lanes
    //    (8 slots each, then a fixed DPP tree), bias, one rounding
    for (int o = tid >> 3; o < S * 8; o += kThreads / 8) {
        const f32x4* pv = reinterpret_cast<const f32x4*>(part + o * kGroups + 8 * c);
        const f32x4 v0 = pv[0], v1 = pv[1];
        float sum = ((v0[0] + v0[1]) + (v0[2] + v0[3])) + ((v1[0] + v1[1]) + (v1[2] + v1[3]));
        sum += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(sum), 0xB1, 0xF, 0xF, false));   // lanes ^1
        sum += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(sum), 0x4E, 0xF, 0xF, false));   // lanes ^2
        sum += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(sum), 0x141, 0xF, 0xF, false));  // half-row mirror
        if (c == 0) {
            const int n = 8 * u_lo + o;
            const float b = a.bias ? half_bits_to_f32<kBF16>(a.bias[n]) : 0.f;
            a.y[n] = f32_to_half_bits<kBF16>(sum + b);
        }
    }
}

// kS = the most half blocks of any workgroup, exactly up to 8 (3, 5, 6 and 7 included:
// a power of two above it would issue loads of clamped duplicates that weigh nothing;
// 2048 x 13312, 7 half blocks: 5.22 -> 5.15 us), else 16
template <bool kBF16, int kJP>
void launch_jp(const StripArgs& args, int grid, size_t lds, hipStream_t s) {
    constexpr int kMaxS = kMaxItems / kJP;
    const int sm = args.smax;
    if (sm <= 1) hipLaunchKernelGGL((gemv_strip_kernel<kBF16, 1, kJP>), dim3(grid), dim3(kThreads), lds, s, args);
    else if (sm == 2 && kMaxS >= 2)
        hipLaunchKernelGGL((gemv_strip_kernel<kBF16, (kMaxS >= 2 ? 2 : 1), kJP>), dim3(grid), dim3(kThreads), lds, s, args);
    else if (sm == 3 && kMaxS >= 4)
        hipLaunchKernelGGL((gemv_strip_kernel<kBF16, (kMaxS >= 4 ? 3 : 1), kJP>), dim3(grid), dim3(kThreads), lds, s, args);
    else if (sm == 4 && kMaxS >= 4)
        hipLaunchKernelGGL((gemv_strip_kernel<kBF16, (kMaxS >= 4 ? 4 : 1), kJP>), dim3(grid), dim3(kThreads), lds, s, args);
    else if (sm == 5 && kMaxS >= 8)
        hipLaunchKernelGGL((gemv_strip_kernel<kBF16, (kMaxS >= 8 ? 5 : 1), kJP>), dim3(grid), dim3(kThreads), lds, s, args);
    else if (sm == 6 && kMaxS >= 8)
        hipLaunchKernelGGL((gemv_strip_kernel<kBF16, (kMaxS >= 8 ? 6 : 1), kJP>), dim3(grid), dim3(kThreads), lds, s, args);
    else if (sm == 7 && kMaxS >= 8)
        hipLaunchKernelGGL((gemv_strip_kernel<kBF16, (kMaxS >= 8 ? 7 : 1), kJP>), dim3(grid), dim3(kThreads), lds, s, args);
    else if (sm == 8 && kMaxS >= 8)
        hipLaunchKernelGGL((gemv_strip_kernel<kBF16, (kMaxS >= 8 ? 8 : 1), kJP>), dim3(grid), dim3(kThreads), lds, s, args);
    else if (kMaxS >= 16)
        hipLaunchKernelGGL((gemv_strip_kernel<kBF16, (kMaxS >= 16 ? 16 : 1), kJP>), dim3(grid), dim3(kThreads), lds, s, args);
}

template <bool kBF16>
void launch_typed(const StripArgs& args, int JP, int grid, size_t lds, hipStream_t s) {
    if (JP <= 1) launch_jp<kBF16, 1>(args, grid, lds, s);
    else if (JP <= 2) launch_jp<kBF16, 2>(args, grid, lds, s);
    else launch_jp<kBF16, 4>(args, grid, lds, s);
}

int pow2_at_least(int64_t v) {
    int r = 1;
    while (r < v) r *= 2;
    return r;
}

}  // namespace

StripPlan plan_gemv_strip(int64_t M, int64_t K, int64_t N, int64_t G) {
    StripPlan p{};
    p.ok = false;
    if (M != 1 || G < kRowsPerBlock) return p;
    const int64_t U = N / 8;
    const int64_t KB = K / kRowsPerBlock;
    const int64_t P = 4 * KB;
    p.grid = (int)(U < kTargetWorkgroups ? U : kTargetWorkgroups);
    const int64_t smax = (U + p.grid - 1) / p.grid;
    const int64_t JP = (P + kGroups - 1) / kGroups;
    // JP row blocks per group (the 64 groups cover K / 128 row blocks in 16 runs of
    // JP, four lane quarters each); the kernel instantiations round both counts up to
    // powers of two; at most 4 row blocks per group (K <= 8192): each lane holds the
    // activations of its row blocks in registers
    if (JP > kMaxPairsPerGroup) return p;
    const int64_t items = (int64_t)pow2_at_least(smax) * pow2_at_least(JP);
    if (items > kMaxItems) return p;
    p.items = (int)items;
    // after the partials: the activations, all K of them with several row blocks per
    // group, each wave's two row blocks (a 1 KiB slot per wave) with one
    p.lds_bytes = (size_t)part_bytes((int)pow2_at_least(smax)) +
                  (JP > 1 ? (size_t)((K * 2 + 1023) / 1024 * 1024) : (size_t)kWaves * 1024);
    if (p.lds_bytes > 64 * 1024) return p;
    p.ok = true;
    return p;
}

hipError_t launch_gemv_strip(const StripPlan& plan, const uint16_t* x, const uint8_t* packed, const uint16_t* bias,
                             uint16_t* y, int64_t K, int64_t N, int64_t G, bool bf16, hipStream_t stream) {
    StripArgs args;
    args.x = x;
    args.packed = packed;
    args.bias = bias;
    args.y = y;
    args.K = (int)K;
    args.N = (int)N;
    args.KB = (int)(K / kRowsPerBlock);
    args.UW = (int)padded_units(K, G);
    args.U = (int)(N / 8);
    args.P = 4 * args.KB;
    const int JP = pow2_at_least((args.P + kGroups - 1) / kGroups);
    args.smax = (args.U + plan.grid - 1) / plan.grid;
    args.smax_pow2 = pow2_at_least(args.smax);
    if (!plan.ok || JP > kMaxPairsPerGroup || pow2_at_least(args.smax) * JP > kMaxItems) return hipErrorInvalidValue;
    if (bf16) launch_typed<true>(args, JP, plan.grid, plan.lds_bytes, stream);
    else launch_typed<false>(args, JP, plan.grid, plan.lds_bytes, stream);
    return hipGetLastError();
}

}  // namespace w4a16
