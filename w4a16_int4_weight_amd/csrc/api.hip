// C ABI of the W4A16 library: argument validation, path dispatch, launches.
// The entry points and their contracts are declared in include/w4a16.h.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "../../include/w4a16.h"
#include "device_common.h"
#include "launch.h"
#include "split_k.h"

namespace {

constexpr int kLayoutVersion = 2;
constexpr int64_t kGemvMaxRows = 16;      // rows one GEMV A operand holds
constexpr int64_t kDefaultGemvMaxM = 8;

// Default split between the GEMV and the MFMA GEMM. M <= 8 takes the GEMV and M >= 16
// the MFMA GEMM at every shape; in between, the GEMV stays ahead the longer the
// smaller the weight is (MI355X, G = 128, bf16: through M = 15 at K x N = 2048 x 3072,
// through 13 at 2048 x 13312, through 12 at 6656 x 2048, and behind already at M = 8
// at 2048 x 131072), so the last GEMV row count follows the size of the codes. Outputs
// of at most 128 column blocks (N <= 2048) and K >= 2048 keep it through M = 15
// (2048 .. 8192 x 1024 .. 2048: 6-30% ahead of the MFMA GEMM at M = 12 .. 16, with
// the GEMV's K split over workgroups where K >= 6144). Wide outputs that the balanced
// matrix-core GEMV takes at M = 16 keep the GEMV through M = 16 (2048 x 13312: 7.96
// against 10.2 us for the MFMA GEMM at M = 16, 7.95 against 9.9 us for the 16-column
// GEMV at M = 12).
int64_t default_gemv_max_m(int64_t K, int64_t N, int64_t G) {
    if (G % 128 != 0) return kDefaultGemvMaxM;        // group sizes 32, 64: not measured
    if (w4a16::plan_gemv_small(kGemvMaxRows, K, N, G).ok) return kGemvMaxRows;
    if ((N + 15) / 16 <= 128 && K >= 2048) return 15;
    const int64_t code_bytes = K * N / 2;
    if (code_bytes <= (int64_t(4) << 20)) return 15;
    if (code_bytes <= (int64_t(16) << 20)) return 12;
    return kDefaultGemvMaxM;
}
constexpr int kMaxDevices = 64;
constexpr int64_t kMaxK = int64_t(1) << 20;   // kernels index rows and columns with 32-bit integers
constexpr int64_t kMaxN = int64_t(1) << 28;
constexpr int64_t kMaxKN = int64_t(1) << 37;  // packed codes index in 32-bit 16-byte units
constexpr int64_t kMaxMK = int64_t(1) << 32;  // activations index in 32-bit elements

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Resolved group size, or 0 if (K, N, group_size) is outside the tile layout.
w4a16_status check_shape(int64_t K, int64_t N, int64_t group_size, int64_t* G_out) {
    if (K <= 0 || N <= 0 || K % 128 != 0 || N % 8 != 0) return W4A16_ERR_SHAPE;
    if (K > kMaxK || N > kMaxN || K * N > kMaxKN) return W4A16_ERR_SHAPE;
    const int64_t G = group_size == -1 ? K : group_size;
    if (G <= 0 || K % G != 0 || (G % 128 != 0 && G != 32 && G != 64)) return W4A16_ERR_GROUP;
    *G_out = G;
    return W4A16_OK;
}

// K x Np codes (Np = N rounded up to 16 columns) + one 32-bit word per column per
// unit of min(G, 128) rows, the unit count rounded up to 4 (G resolved)
size_t packed_size(int64_t K, int64_t N, int64_t G) {
    const size_t uw = (size_t)w4a16::padded_units(K, G);
    const size_t np = (size_t)w4a16::padded_cols(N);
    return (size_t)K * np / 2 + (size_t)4 * uw * np;
}

// W4A8 activation buffer: codes (M*K bytes), row scales (M fp32), block sums
// (M*K/128 fp32), each part starting on a 256-byte boundary.
size_t round256(size_t v) { return (v + 255) / 256 * 256; }
size_t act_scale_offset(int64_t M, int64_t K) { return round256((size_t)M * (size_t)K); }
size_t act_sum_offset(int64_t M, int64_t K) { return act_scale_offset(M, K) + round256((size_t)M * 4); }
size_t act_size(int64_t M, int64_t K) { return act_sum_offset(M, K) + (size_t)M * (size_t)(K / 128) * 4; }
w4a16_status check_act_shape(int64_t M, int64_t K) {
    if (M < 0 || M >= (int64_t(1) << 31) || K <= 0 || K % 128 != 0 || K > kMaxK || M * K > kMaxMK)
        return W4A16_ERR_SHAPE;
    return W4A16_OK;
}
w4a16::W4A8Act act_parts(void* act, int64_t M, int64_t K) {
    uint8_t* base = static_cast<uint8_t*>(act);
    return w4a16::W4A8Act{base, reinterpret_cast<float*>(base + act_scale_offset(M, K)),
                          reinterpret_cast<float*>(base + act_sum_offset(M, K))};
}

// 0 = unknown, 1 = gfx950, 2 = other; cached per device ordinal.
std::atomic<int> g_device_kind[kMaxDevices];

w4a16_status check_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return W4A16_ERR_DEVICE;
    if (dev < 0 || dev >= kMaxDevices) return W4A16_ERR_DEVICE;
    int kind = g_device_kind[dev].load(std::memory_order_relaxed);
    if (kind == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return W4A16_ERR_DEVICE;
        kind = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        g_device_kind[dev].store(kind, std::memory_order_relaxed);
    }
    return kind == 1 ? W4A16_OK : W4A16_ERR_DEVICE;
}

// Host-side checks of a GEMM call (everything but the workspace and the device).
// On W4A16_OK with M > 0, *G_out is the resolved group size and *use_gemv the path.
w4a16_status check_gemm(const void* x, const void* packed, size_t packed_bytes, w4a16_dtype dtype, const void* y,
                        int64_t M, int64_t K, int64_t N, int64_t group_size, const void* bias, w4a16_path path,
                        int64_t gemv_max_m, int64_t* G_out, bool* use_gemv) {
    if (M < 0) return W4A16_ERR_SHAPE;
    int64_t G = 0;
    w4a16_status st = check_shape(K, N, group_size, &G);
    if (st != W4A16_OK) return st;
    if (dtype != W4A16_FP16 && dtype != W4A16_BF16) return W4A16_ERR_DTYPE;
    if (path != W4A16_PATH_AUTO && path != W4A16_PATH_GEMV && path != W4A16_PATH_MFMA) return W4A16_ERR_PATH;
    if (gemv_max_m < 0) gemv_max_m = default_gemv_max_m(K, N, G);
    if (gemv_max_m > kGemvMaxRows) return W4A16_ERR_PATH;
    if (path == W4A16_PATH_GEMV && M > kGemvMaxRows) return W4A16_ERR_PATH;
    if (M >= (int64_t(1) << 31) || M * K > kMaxMK) return W4A16_ERR_SHAPE;
    if (M == 0) return W4A16_OK;
    if (!x || !packed || !y) return W4A16_ERR_NULL;
    if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(y, 16) || (bias && !aligned(bias, 2)))
        return W4A16_ERR_ALIGN;
    if (packed_bytes < packed_size(K, N, G)) return W4A16_ERR_BUFFER_SIZE;
    *G_out = G;
    *use_gemv = path == W4A16_PATH_GEMV || (path == W4A16_PATH_AUTO && M <= gemv_max_m);
    return W4A16_OK;
}

// Launches a checked GEMM call on the current device.
w4a16_status launch_checked_gemm(const void* x, const void* packed, w4a16_dtype dtype, void* y, int64_t M,
                                 int64_t K, int64_t N, int64_t G, const void* bias, void* workspace,
                                 size_t workspace_bytes, void* stream, bool use_gemv) {
    const bool bf16 = dtype == W4A16_BF16;
    const auto* xp = static_cast<const uint16_t*>(x);
    const auto* wp = static_cast<const uint8_t*>(packed);
    const auto* bp = static_cast<const uint16_t*>(bias);
    auto* yp = static_cast<uint16_t*>(y);
    hipStream_t s = static_cast<hipStream_t>(stream);
    // the GEMV splits K over workgroups only if the workspace is large enough for it
    void* gemv_ws = workspace && aligned(workspace, 16) ? workspace : nullptr;
    const hipError_t err = use_gemv ? w4a16::launch_gemv(xp, wp, bp, yp, M, K, N, G, bf16, gemv_ws,
                                                         gemv_ws ? workspace_bytes : 0, s)
                                    : w4a16::launch_gemm(xp, wp, bp, yp, M, K, N, G, bf16, workspace, s);
    return err == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

w4a16_status gemm_impl(const void* x, const void* packed, size_t packed_bytes, w4a16_dtype dtype, void* y,
                       int64_t M, int64_t K, int64_t N, int64_t group_size, const void* bias, void* workspace,
                       size_t workspace_bytes, void* stream, w4a16_path path, int64_t gemv_max_m) {
    int64_t G = 0;
    bool use_gemv = false;
    w4a16_status st = check_gemm(x, packed, packed_bytes, dtype, y, M, K, N, group_size, bias, path, gemv_max_m,
                                 &G, &use_gemv);
    if (st != W4A16_OK || M == 0) return st;
    const size_t need = use_gemv ? 0 : w4a16::plan_gemm(M, K, N, G).workspace_bytes;
    if (need > 0) {
        if (!workspace) return W4A16_ERR_NULL;
        if (!aligned(workspace, 16)) return W4A16_ERR_ALIGN;
        if (workspace_bytes < need) return W4A16_ERR_BUFFER_SIZE;
    }
    st = check_device();
    if (st != W4A16_OK) return st;
    return launch_checked_gemm(x, packed, dtype, y, M, K, N, G, bias, workspace, workspace_bytes, stream, use_gemv);
}

// ---------------------------------------------------------------- allocation-free GEMM
// w4a16_gemm_noalloc keeps the K-split partials and tile counters in this array
// instead of a caller workspace. Each GPU the library runs on holds its own copy until
// the process ends; the host reaches it only through the device address that
// hipGetSymbolAddress returns (kept per device), never through the array's name.
constexpr size_t kScratchBytes = W4A16_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0 && kScratchBytes >= w4a16::kSplitCounterBytes, "scratch size");
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

__global__ void clear_words_kernel(uint32_t* __restrict__ p, int n) {
    const int i = (int)(blockIdx.x * blockDim.x + threadIdx.x);
    if (i < n) p[i] = 0u;
}

struct ScratchSlot {
    std::mutex mu;
    void* ptr = nullptr;      // device address of `scratch` on this device
    bool cleared = false;     // its counter region zeroed by an eager launch
};
ScratchSlot g_scratch[kMaxDevices];

// The current device's copy of `scratch`, its counter region zeroed ahead of the
// caller's kernels on `stream`. The clear is launched once per device outside stream
// capture; a captured first call puts the clear into its graph and leaves it pending
// for the next eager call. (The kernels leave the counters at zero after every call.)
w4a16_status device_scratch(hipStream_t stream, void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return W4A16_ERR_DEVICE;
    ScratchSlot& slot = g_scratch[dev];
    std::lock_guard<std::mutex> lock(slot.mu);
    if (!slot.ptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return W4A16_ERR_HIP;
        slot.ptr = p;
    }
    if (!slot.cleared) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(stream, &cs) != hipSuccess) return W4A16_ERR_HIP;
        constexpr int words = (int)(w4a16::kSplitCounterBytes / 4);
        hipLaunchKernelGGL(clear_words_kernel, dim3((words + 255) / 256), dim3(256), 0, stream,
                           static_cast<uint32_t*>(slot.ptr), words);
        if (hipGetLastError() != hipSuccess) return W4A16_ERR_HIP;
        if (cs == hipStreamCaptureStatusNone) slot.cleared = true;
    }
    *out = slot.ptr;
    return W4A16_OK;
}

// One repack entry: AWQ (gptq = false) or GPTQ-standard tensors holding columns
// [n0, n0 + nc) of a K x N weight, written into the packed layout of the K x N weight.
w4a16_status repack_impl(bool gptq, const int32_t* qweight, const int32_t* qzeros, const void* scales,
                         w4a16_dtype dtype, int64_t K, int64_t N, int64_t group_size, int64_t n0, int64_t nc,
                         void* packed, size_t packed_bytes, void* stream) {
    int64_t G = 0;
    w4a16_status st = check_shape(K, N, group_size, &G);
    if (st != W4A16_OK) return st;
    if (dtype != W4A16_FP16 && dtype != W4A16_BF16) return W4A16_ERR_DTYPE;
    // whole 16-column blocks, except that the last chunk may end in a half block
    if (n0 < 0 || nc <= 0 || n0 % 16 != 0 || nc % 8 != 0 || nc > N - n0 || (nc % 16 != 0 && n0 + nc != N))
        return W4A16_ERR_SHAPE;
    if (!qweight || !qzeros || !scales || !packed) return W4A16_ERR_NULL;
    if (!aligned(qweight, 4) || !aligned(qzeros, 4) || !aligned(scales, 2) || !aligned(packed, 16))
        return W4A16_ERR_ALIGN;
    if (packed_bytes < packed_size(K, N, G)) return W4A16_ERR_BUFFER_SIZE;
    st = check_device();
    if (st != W4A16_OK) return st;
    const auto* sc = static_cast<const uint16_t*>(scales);
    auto* out = static_cast<uint8_t*>(packed);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t err = gptq ? w4a16::launch_repack_gptq(qweight, qzeros, sc, out, K, nc, G, n0, N, s)
                                : w4a16::launch_repack(qweight, qzeros, sc, out, K, nc, G, n0, N, s);
    return err == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

}  // namespace

extern "C" {

int w4a16_layout_version(void) { return kLayoutVersion; }

size_t w4a16_packed_bytes(int64_t K, int64_t N, int64_t group_size) {
    int64_t G = 0;
    if (check_shape(K, N, group_size, &G) != W4A16_OK) return 0;
    return packed_size(K, N, G);
}

w4a16_status w4a16_repack(const int32_t* qweight, const int32_t* qzeros, const void* scales, w4a16_dtype dtype,
                          int64_t K, int64_t N, int64_t group_size, void* packed, size_t packed_bytes,
                          void* stream) {
    return repack_impl(false, qweight, qzeros, scales, dtype, K, N, group_size, 0, N, packed, packed_bytes, stream);
}

w4a16_status w4a16_repack_gptq(const int32_t* qweight, const int32_t* qzeros, const void* scales,
                               w4a16_dtype dtype, int64_t K, int64_t N, int64_t group_size, void* packed,
                               size_t packed_bytes, void* stream) {
    return repack_impl(true, qweight, qzeros, scales, dtype, K, N, group_size, 0, N, packed, packed_bytes, stream);
}

w4a16_status w4a16_repack_columns(const int32_t* qweight, const int32_t* qzeros, const void* scales,
                                  w4a16_dtype dtype, int64_t K, int64_t N, int64_t group_size, int64_t n0,
                                  int64_t nc, void* packed, size_t packed_bytes, void* stream) {
    return repack_impl(false, qweight, qzeros, scales, dtype, K, N, group_size, n0, nc, packed, packed_bytes,
                       stream);
}

w4a16_status w4a16_repack_gptq_columns(const int32_t* qweight, const int32_t* qzeros, const void* scales,
                                       w4a16_dtype dtype, int64_t K, int64_t N, int64_t group_size, int64_t n0,
                                       int64_t nc, void* packed, size_t packed_bytes, void* stream) {
    return repack_impl(true, qweight, qzeros, scales, dtype, K, N, group_size, n0, nc, packed, packed_bytes,
                       stream);
}

size_t w4a16_workspace_bytes(int64_t M, int64_t K, int64_t N, int64_t group_size) {
    int64_t G = 0;
    if (M <= 0 || check_shape(K, N, group_size, &G) != W4A16_OK) return 0;
    if (M >= (int64_t(1) << 31) || M * K > kMaxMK) return 0;
    // only the MFMA GEMM uses one (when it splits K over workgroups); the GEMV needs none
    return w4a16::plan_gemm(M, K, N, G).workspace_bytes;
}

w4a16_status w4a16_gemm(const void* x, const void* packed, size_t packed_bytes, w4a16_dtype dtype, void* y,
                        int64_t M, int64_t K, int64_t N, int64_t group_size, const void* bias, void* workspace,
                        size_t workspace_bytes, void* stream) {
    return gemm_impl(x, packed, packed_bytes, dtype, y, M, K, N, group_size, bias, workspace, workspace_bytes,
                     stream, W4A16_PATH_AUTO, -1);
}

w4a16_status w4a16_gemm_ex(const void* x, const void* packed, size_t packed_bytes, w4a16_dtype dtype, void* y,
                           int64_t M, int64_t K, int64_t N, int64_t group_size, const void* bias, void* workspace,
                           size_t workspace_bytes, void* stream, w4a16_path path, int64_t gemv_max_m) {
    return gemm_impl(x, packed, packed_bytes, dtype, y, M, K, N, group_size, bias, workspace, workspace_bytes,
                     stream, path, gemv_max_m);
}

w4a16_status w4a16_gemm_noalloc(const void* x, const void* packed, size_t packed_bytes, w4a16_dtype dtype,
                                void* y, int64_t M, int64_t K, int64_t N, int64_t group_size, const void* bias,
                                void* stream) {
    int64_t G = 0;
    bool use_gemv = false;
    w4a16_status st = check_gemm(x, packed, packed_bytes, dtype, y, M, K, N, group_size, bias, W4A16_PATH_AUTO, -1,
                                 &G, &use_gemv);
    if (st != W4A16_OK || M == 0) return st;
    // the same requirement w4a16_workspace_bytes states, against the array's size
    if (w4a16::plan_gemm(M, K, N, G).workspace_bytes > kScratchBytes) return W4A16_ERR_BUFFER_SIZE;
    st = check_device();
    if (st != W4A16_OK) return st;
    void* ws = nullptr;
    st = device_scratch(static_cast<hipStream_t>(stream), &ws);
    if (st != W4A16_OK) return st;
    return launch_checked_gemm(x, packed, dtype, y, M, K, N, G, bias, ws, kScratchBytes, stream, use_gemv);
}

w4a16_status w4a16_embedding(const int32_t* ids, int64_t T, const void* packed, size_t packed_bytes,
                             w4a16_dtype dtype, int64_t K, int64_t N, int64_t group_size, void* out, void* stream) {
    int64_t G = 0;
    w4a16_status st = check_shape(K, N, group_size, &G);
    if (st != W4A16_OK) return st;
    if (dtype != W4A16_FP16 && dtype != W4A16_BF16) return W4A16_ERR_DTYPE;
    if (T < 0 || T >= (int64_t(1) << 31)) return W4A16_ERR_SHAPE;
    if (T == 0) return W4A16_OK;
    if (!ids || !packed || !out) return W4A16_ERR_NULL;
    if (!aligned(ids, 4) || !aligned(packed, 16) || !aligned(out, 16)) return W4A16_ERR_ALIGN;
    if (packed_bytes < packed_size(K, N, G)) return W4A16_ERR_BUFFER_SIZE;
    st = check_device();
    if (st != W4A16_OK) return st;
    const hipError_t err = w4a16::launch_embedding(ids, T, static_cast<const uint8_t*>(packed),
                                                   static_cast<uint16_t*>(out), K, N, G, dtype == W4A16_BF16,
                                                   static_cast<hipStream_t>(stream));
    return err == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

size_t w4a8_activation_bytes(int64_t M, int64_t K) {
    if (M <= 0 || check_act_shape(M, K) != W4A16_OK) return 0;
    return act_size(M, K);
}

size_t w4a8_workspace_bytes(int64_t M, int64_t K, int64_t N, int64_t group_size) {
    int64_t G = 0;
    if (M <= 0 || check_shape(K, N, group_size, &G) != W4A16_OK || G < 128) return 0;
    if (check_act_shape(M, K) != W4A16_OK) return 0;
    return w4a16::plan_gemm(M, K, N, G).workspace_bytes;
}

w4a16_status w4a8_quantize(const void* x, w4a16_dtype dtype, int64_t M, int64_t K, void* act, size_t act_bytes,
                           void* stream) {
    w4a16_status st = check_act_shape(M, K);
    if (st != W4A16_OK) return st;
    if (dtype != W4A16_FP16 && dtype != W4A16_BF16) return W4A16_ERR_DTYPE;
    if (M == 0) return W4A16_OK;
    if (!x || !act) return W4A16_ERR_NULL;
    if (!aligned(x, 16) || !aligned(act, 16)) return W4A16_ERR_ALIGN;
    if (act_bytes < act_size(M, K)) return W4A16_ERR_BUFFER_SIZE;
    st = check_device();
    if (st != W4A16_OK) return st;
    const hipError_t err = w4a16::launch_w4a8_quantize(static_cast<const uint16_t*>(x), M, K, dtype == W4A16_BF16,
                                                       act_parts(act, M, K), static_cast<hipStream_t>(stream));
    return err == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

w4a16_status w4a8_gemm(const void* act, size_t act_bytes, const void* packed, size_t packed_bytes,
                       w4a16_dtype dtype, void* y, int64_t M, int64_t K, int64_t N, int64_t group_size,
                       const void* bias, void* workspace, size_t workspace_bytes, void* stream) {
    int64_t G = 0;
    w4a16_status st = check_shape(K, N, group_size, &G);
    if (st != W4A16_OK) return st;
    if (G < 128) return W4A16_ERR_GROUP;     // one fp8 MFMA spans a 128-row block
    st = check_act_shape(M, K);
    if (st != W4A16_OK) return st;
    if (dtype != W4A16_FP16 && dtype != W4A16_BF16) return W4A16_ERR_DTYPE;
    if (M == 0) return W4A16_OK;
    if (!act || !packed || !y) return W4A16_ERR_NULL;
    if (!aligned(act, 16) || !aligned(packed, 16) || !aligned(y, 16) || (bias && !aligned(bias, 2)))
        return W4A16_ERR_ALIGN;
    if (act_bytes < act_size(M, K) || packed_bytes < packed_size(K, N, G)) return W4A16_ERR_BUFFER_SIZE;
    const size_t need = w4a16::plan_gemm(M, K, N, G).workspace_bytes;
    if (need > 0) {
        if (!workspace) return W4A16_ERR_NULL;
        if (!aligned(workspace, 16)) return W4A16_ERR_ALIGN;
        if (workspace_bytes < need) return W4A16_ERR_BUFFER_SIZE;
    }
    st = check_device();
    if (st != W4A16_OK) return st;
    // the kernel reads the activation parts through const pointers
    const hipError_t err = w4a16::launch_w4a8_gemm(act_parts(const_cast<void*>(act), M, K),
                                                   static_cast<const uint8_t*>(packed),
                                                   static_cast<const uint16_t*>(bias), static_cast<uint16_t*>(y), M,
                                                   K, N, G, dtype == W4A16_BF16, workspace,
                                                   static_cast<hipStream_t>(stream));
    return err == hipSuccess ? W4A16_OK : W4A16_ERR_HIP;
}

// Packed-buffer header: magic, layout version, dtype, K, N, group size, buffer bytes,
// an FNV-1a checksum of those 48 bytes, 8 reserved zero bytes.
constexpr char kHeaderMagic[8] = {'W', '4', 'A', '1', '6', 'P', 'K', 0};

uint64_t fnv1a64(const uint8_t* p, size_t n) {
    uint64_t h = 0xcbf29ce484222325ull;
    for (size_t i = 0; i < n; ++i) {
        h ^= p[i];
        h *= 0x100000001b3ull;
    }
    return h;
}

w4a16_status w4a16_packed_header(int64_t K, int64_t N, int64_t group_size, w4a16_dtype dtype, void* header,
                                 size_t header_bytes) {
    int64_t G = 0;
    w4a16_status st = check_shape(K, N, group_size, &G);
    if (st != W4A16_OK) return st;
    if (dtype != W4A16_FP16 && dtype != W4A16_BF16) return W4A16_ERR_DTYPE;
    if (!header) return W4A16_ERR_NULL;
    if (header_bytes < W4A16_PACKED_HEADER_BYTES) return W4A16_ERR_BUFFER_SIZE;
    uint8_t h[W4A16_PACKED_HEADER_BYTES] = {};
    const uint32_t version = kLayoutVersion, dt = (uint32_t)dtype;
    const uint64_t nbytes = packed_size(K, N, G);
    memcpy(h, kHeaderMagic, 8);
    memcpy(h + 8, &version, 4);
    memcpy(h + 12, &dt, 4);
    memcpy(h + 16, &K, 8);
    memcpy(h + 24, &N, 8);
    memcpy(h + 32, &group_size, 8);
    memcpy(h + 40, &nbytes, 8);
    const uint64_t sum = fnv1a64(h, 48);
    memcpy(h + 48, &sum, 8);
    memcpy(header, h, sizeof(h));
    return W4A16_OK;
}

w4a16_status w4a16_parse_packed_header(const void* header, size_t header_bytes, int64_t* K, int64_t* N,
                                       int64_t* group_size, w4a16_dtype* dtype, size_t* packed_bytes) {
    if (!header || !K || !N || !group_size || !dtype || !packed_bytes) return W4A16_ERR_NULL;
    if (header_bytes < W4A16_PACKED_HEADER_BYTES) return W4A16_ERR_BUFFER_SIZE;
    const uint8_t* h = static_cast<const uint8_t*>(header);
    uint64_t sum = 0, nbytes = 0;
    memcpy(&sum, h + 48, 8);
    if (memcmp(h, kHeaderMagic, 8) != 0 || sum != fnv1a64(h, 48)) return W4A16_ERR_LAYOUT;
    for (int i = 56; i < 64; ++i)
        if (h[i] != 0) return W4A16_ERR_LAYOUT;
    uint32_t version = 0, dt = 0;
    int64_t k = 0, n = 0, g = 0;
    memcpy(&version, h + 8, 4);
    memcpy(&dt, h + 12, 4);
    memcpy(&k, h + 16, 8);
    memcpy(&n, h + 24, 8);
    memcpy(&g, h + 32, 8);
    memcpy(&nbytes, h + 40, 8);
    if (version != (uint32_t)kLayoutVersion) return W4A16_ERR_LAYOUT;
    int64_t G = 0;
    if (check_shape(k, n, g, &G) != W4A16_OK || (dt != W4A16_FP16 && dt != W4A16_BF16) ||
        nbytes != packed_size(k, n, G))
        return W4A16_ERR_LAYOUT;
    *K = k;
    *N = n;
    *group_size = g;
    *dtype = (w4a16_dtype)dt;
    *packed_bytes = (size_t)nbytes;
    return W4A16_OK;
}

const char* w4a16_status_str(w4a16_status status) {
    switch (status) {
        case W4A16_OK: return "ok";
        case W4A16_ERR_NULL: return "a required pointer is NULL";
        case W4A16_ERR_SHAPE: return "unsupported shape (need M >= 0, K % 128 == 0, N % 8 == 0)";
        case W4A16_ERR_GROUP:
            return "unsupported group size (need -1, 32, 64 or a multiple of 128 dividing K; W4A8: not 32 or 64)";
        case W4A16_ERR_DTYPE: return "unsupported dtype (need fp16 or bf16)";
        case W4A16_ERR_ALIGN: return "misaligned pointer";
        case W4A16_ERR_BUFFER_SIZE: return "caller buffer too small";
        case W4A16_ERR_DEVICE: return "current device is not a gfx950 GPU";
        case W4A16_ERR_HIP: return "HIP launch error";
        case W4A16_ERR_PATH: return "unknown path, or the forced path cannot take this M";
        case W4A16_ERR_LAYOUT: return "packed-buffer header invalid or from another layout version";
        default: return "unknown status";
    }
}

}  // extern "C"
