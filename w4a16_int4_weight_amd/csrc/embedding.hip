// Quantised tied-embedding gather from the packed head weight.
//
// A model whose input embedding is tied to its output head keeps one quantised
// matrix for both (the vllm-omni commit "cpu_int4: repack weights in n-blocks, to
// bound the load-time peak" lists the 131072 x 2048 embedding as the same matrix as
// the output head; the commit "Add cpu_int4, an asymmetric 4-bit weight path for
// vLLM's CPU backend" checks the quantised tied embedding end to end). Stored as the
// head W [K, N] (K hidden, N vocabulary) for y = x . W, the embedding of token t is
// column t of dequant(W):
//
//   e[i, k] = (q[k, t_i] - z[k div G, t_i]) * s[k div G, t_i],   rounded once (RNE).
//
// The gather reads the packed buffer the GEMM reads, so tying costs no second copy.
// One wave per token. Column t lives in column block t / 16, as lane (t % 16) + 16 h
// of each 1 KiB block (h = 0..3), whose 4 words hold rows 32 i + 8 h + 0..7 of that
// 128-row block: a lane takes one (row block, h) pair at a time, loads those 16
// bytes and the block's metadata word, and writes four runs of 8 consecutive output
// rows, each the decoded word as it would enter the MFMA. Ids outside [0, N) give a
// row of zeros.
#include "device_common.h"
#include "launch.h"

namespace w4a16 {
namespace {

constexpr int kTokensPerWorkgroup = 4;     // one wave each

__device__ __forceinline__ uint32_t pick_word(const uint4 v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

template <bool kBF16, int kWpb>
__global__ __launch_bounds__(64 * kTokensPerWorkgroup) void embedding_kernel(
    const int32_t* __restrict__ ids, int64_t T, const uint8_t* __restrict__ packed,
    uint16_t* __restrict__ out, int K, int N, int G) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t t = (int64_t)blockIdx.x * kTokensPerWorkgroup + wave;
    if (t >= T) return;
    const int lane = threadIdx.x & 63;
    const int id = __builtin_amdgcn_readfirstlane(ids[t]);
    const bool valid = id >= 0 && id < N;
    const int col = valid ? id : 0;
    const int KB = K / kRowsPerBlock;
    constexpr int wpb = kWpb;                             // metadata words per row block (1, 2, 4)
    const int UW = (int)padded_units(K, G);
    // this column's 16-byte chunk of lane group 0 in its first block; group h is
    // 256 h bytes further on, row block kb 1 KiB * kb
    const uint8_t* codes = packed + (size_t)(col / kColsPerBlock) * KB * kBlockBytes + 16 * (col % kColsPerBlock);
    const uint32_t* meta = reinterpret_cast<const uint32_t*>(packed + (size_t)K * padded_cols(N) / 2) + (size_t)col * UW;
    uint16_t* row = out + (size_t)t * K;
    for (int q = lane; q < KB * 4; q += 64) {
        const int kb = q >> 2;
        const int h = q & 3;
        const uint4 w = *reinterpret_cast<const uint4*>(codes + (size_t)kb * kBlockBytes + 256 * h);
        uint16_t* dst = row + kb * kRowsPerBlock + 8 * h;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // word i holds rows 32 i + 8 h + 0..7: metadata unit kb wpb + i wpb / 4
            const Dequant<kBF16> dq(meta[kb * wpb + (i * wpb) / 4]);
            const uint4 v = valid ? dq(pick_word(w, i)) : make_uint4(0u, 0u, 0u, 0u);
            *reinterpret_cast<uint4*>(dst + 32 * i) = v;
        }
    }
}

}  // namespace

hipError_t launch_embedding(const int32_t* ids, int64_t T, const uint8_t* packed, uint16_t* out, int64_t K,
                            int64_t N, int64_t G, bool bf16, hipStream_t stream) {
    const dim3 grid((unsigned)((T + kTokensPerWorkgroup - 1) / kTokensPerWorkgroup));
    const dim3 block(64 * kTokensPerWorkgroup);
    const int wpb = units_per_block(G);
    if (bf16) {
        if (wpb == 4) hipLaunchKernelGGL((embedding_kernel<true, 4>), grid, block, 0, stream, ids, T, packed, out, (int)K, (int)N, (int)G);
        else if (wpb == 2) hipLaunchKernelGGL((embedding_kernel<true, 2>), grid, block, 0, stream, ids, T, packed, out, (int)K, (int)N, (int)G);
        else hipLaunchKernelGGL((embedding_kernel<true, 1>), grid, block, 0, stream, ids, T, packed, out, (int)K, (int)N, (int)G);
    } else {
        if (wpb == 4) hipLaunchKernelGGL((embedding_kernel<false, 4>), grid, block, 0, stream, ids, T, packed, out, (int)K, (int)N, (int)G);
        else if (wpb == 2) hipLaunchKernelGGL((embedding_kernel<false, 2>), grid, block, 0, stream, ids, T, packed, out, (int)K, (int)N, (int)G);
        else hipLaunchKernelGGL((embedding_kernel<false, 1>), grid, block, 0, stream, ids, T, packed, out, (int)K, (int)N, (int)G);
    }
    return hipGetLastError();
}

}  // namespace w4a16
