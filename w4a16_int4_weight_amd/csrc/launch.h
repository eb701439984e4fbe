// Host-side launchers of the W4A16 kernels. Arguments are assumed validated by the
// C ABI layer (api.hip): shapes supported by the tile layout, pointers aligned.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a16 {

// AWQ tensors of columns [n0, n0 + N) of a K x Nt weight -> those columns of the
// packed tile layout of the K x Nt weight (n0 % 16 == 0; N % 16 == 0 unless
// n0 + N == Nt). G: resolved group size (32, 64, or a multiple of 128 dividing K).
hipError_t launch_repack(const int32_t* qweight, const int32_t* qzeros, const uint16_t* scales,
                         uint8_t* packed, int64_t K, int64_t N, int64_t G, int64_t n0, int64_t Nt,
                         hipStream_t stream);
// The same from GPTQ-standard tensors (codes packed along K, standard order).
hipError_t launch_repack_gptq(const int32_t* qweight, const int32_t* qzeros, const uint16_t* scales,
                              uint8_t* packed, int64_t K, int64_t N, int64_t G, int64_t n0, int64_t Nt,
                              hipStream_t stream);

// Weight-streaming split-K GEMV for 1 <= M <= 16: K split over the waves of a
// workgroup, and for outputs of at most 128 column blocks (K >= 6144, M >= 6) also
// over 2-4 workgroups per block when the caller's workspace holds their partials.
struct GemvPlan {
    int kb_per_wave;       // row blocks per wave (multiple of 4)
    int waves;             // waves per workgroup (waves_k per column block)
    int waves_k;           // waves splitting K for one 16-column block
    bool staged;           // activations staged in LDS
    int chunks_per_thread; // 16-byte activation chunks each thread stages
    int sub;               // metadata units per 128-row block (128 / G for G = 32, 64; else 1)
    size_t lds_bytes;
    int splits;            // workgroups per column block along K
    int kb_per_split;      // row blocks per such workgroup
    size_t workspace_bytes;   // [counters][splits x blocks x 1 KiB fp32 partials] when splits > 1
};
GemvPlan plan_gemv(int64_t M, int64_t K, int64_t N, int64_t G, size_t workspace_bytes);

// `workspace` (or NULL) holds `workspace_bytes` bytes whose counter part is zero; the
// kernel uses it only if plan_gemv splits K over workgroups with that many bytes, and
// leaves the counters zero.
hipError_t launch_gemv(const uint16_t* x, const uint8_t* packed, const uint16_t* bias, uint16_t* y,
                       int64_t M, int64_t K, int64_t N, int64_t G, bool bf16, void* workspace,
                       size_t workspace_bytes, hipStream_t stream);

// Decode GEMV for M = 1 over equal shares of 8-column half blocks, one workgroup per
// compute unit (G >= 128). ok = false when the shape does not fit it (then the
// GEMV above runs).
struct StripPlan {
    bool ok;
    int grid;          // workgroups
    int items;         // code loads in flight per lane
    size_t lds_bytes;
};
StripPlan plan_gemv_strip(int64_t M, int64_t K, int64_t N, int64_t G);

hipError_t launch_gemv_strip(const StripPlan& plan, const uint16_t* x, const uint8_t* packed, const uint16_t* bias,
                             uint16_t* y, int64_t K, int64_t N, int64_t G, bool bf16, hipStream_t stream);

// Decode GEMV for 2 <= M <= 16 on the matrix cores over equal shares of 8-column half
// blocks, one workgroup per compute unit (G >= 128). ok = false when the shape does
// not fit it or the GEMV above is faster on it.
struct SmallPlan {
    bool ok;
    int P;             // units (row-block pairs) per half block
    int grid;          // workgroups
    int smax;          // most half blocks of any workgroup
    int JP;            // most units of one half block per wave
};
SmallPlan plan_gemv_small(int64_t M, int64_t K, int64_t N, int64_t G);

hipError_t launch_gemv_small(const SmallPlan& plan, const uint16_t* x, const uint8_t* packed, const uint16_t* bias,
                             uint16_t* y, int64_t M, int64_t K, int64_t N, int64_t G, bool bf16, hipStream_t stream);

// Tied-embedding gather: out[t, :] = dequantised column ids[t] of the packed [K, N]
// weight (zeros for ids outside [0, N)).
hipError_t launch_embedding(const int32_t* ids, int64_t T, const uint8_t* packed, uint16_t* out, int64_t K,
                            int64_t N, int64_t G, bool bf16, hipStream_t stream);

// LDS-staged dequantise -> MFMA GEMM for any M >= 1: tile shape and K split chosen
// from the shape; workspace_bytes > 0 when K is split over workgroups.
struct GemmPlan {
    int mr;            // row fragments of 16 per tile (tile rows = 16 * mr)
    int cbw;           // 16-column blocks per wave (tile columns = 16 * waves * cbw)
    int waves;         // waves per workgroup, side by side along N (4 or 8)
    int tiles_m, tiles_n;
    int splits;        // workgroups per tile along K
    int sub;           // metadata units per 128-row block (128 / G for G = 32, 64; else 1)
    size_t workspace_bytes;   // [kSplitCounterBytes of tile counters][splits x M x N fp32 partials]
};
GemmPlan plan_gemm(int64_t M, int64_t K, int64_t N, int64_t G);

// `workspace` must hold plan_gemm(M, K, N, G).workspace_bytes bytes whose counter part is
// zero; the kernel leaves it zero.
hipError_t launch_gemm(const uint16_t* x, const uint8_t* packed, const uint16_t* bias, uint16_t* y,
                       int64_t M, int64_t K, int64_t N, int64_t G, bool bf16, void* workspace,
                       hipStream_t stream);

// W4A8 activations after quantisation (one caller buffer, see w4a8_activation_bytes):
// codes [M x K] E4M3 bytes in operand order, row_scale [M] fp32, block_sum [M x K/128]
// fp32 (sum of each 128-element block's decoded codes).
struct W4A8Act {
    uint8_t* codes;
    float* row_scale;
    float* block_sum;
};
hipError_t launch_w4a8_quantize(const uint16_t* x, int64_t M, int64_t K, bool bf16, const W4A8Act& a,
                                hipStream_t stream);
// Tiles of launch_gemm (plan_gemm, G >= 128), plus a 256 x 256 tile for outputs of at
// least two rounds of it; the workspace never exceeds plan_gemm's.
hipError_t launch_w4a8_gemm(const W4A8Act& a, const uint8_t* packed, const uint16_t* bias, uint16_t* y, int64_t M,
                            int64_t K, int64_t N, int64_t G, bool bf16, void* workspace, hipStream_t stream);

}  // namespace w4a16
