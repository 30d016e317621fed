// C ABI of libbsa (declared in include/bsa.h): argument checks, device checks, launches.
//
// Every entry point checks its arguments on the host first and returns before touching
// HIP when they are bad, so the error paths work on machines without a GPU. No C++
// exception crosses the interface.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <initializer_list>
#include <mutex>
#include <vector>

#include "../../include/bsa.h"
#include "kernels.h"

namespace {

thread_local char g_err[512] = "";

bsa_status fail(bsa_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Shape rules shared by every compute call.
bsa_status check_shape(int32_t B, int32_t H, int32_t S, int32_t D, int32_t block) {
    if (B < 1 || H < 1 || S < 1) return fail(BSA_ERR_INVALID_ARGUMENT, "B, H and S must be >= 1 (got %d, %d, %d)", B, H, S);
    if (D != 64 && D != 128) return fail(BSA_ERR_UNSUPPORTED, "D must be 64 or 128 (got %d)", D);
    if (block != 64 && block != 128) return fail(BSA_ERR_UNSUPPORTED, "block must be 64 or 128 (got %d)", block);
    const int64_t elems = (int64_t)B * H * S * D;
    if (elems >= ((int64_t)1 << 40)) return fail(BSA_ERR_UNSUPPORTED, "tensor too large");
    const int64_t rows = (int64_t)B * H * ((S + block - 1) / block);
    if (rows >= ((int64_t)1 << 31)) return fail(BSA_ERR_UNSUPPORTED, "too many block rows");
    // one (b, h) slice is addressed through a buffer resource with 32-bit offsets
    const int64_t s_pad = (int64_t)((S + block - 1) / block) * block;
    if (s_pad * D * 2 >= ((int64_t)1 << 31)) return fail(BSA_ERR_UNSUPPORTED, "sequence too long for one (b, h) slice (S = %d)", S);
    return BSA_OK;
}

// Per-device check: a gfx950 device is current. Cached per device id.
struct DevInfo {
    bool known = false;
    bool ok = false;
};
std::mutex g_dev_mu;
std::vector<DevInfo> g_dev;

bsa_status check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return fail(BSA_ERR_NO_DEVICE, "no HIP device is available");
    }
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if ((int)g_dev.size() <= dev) g_dev.resize(dev + 1);
    DevInfo& di = g_dev[dev];
    if (!di.known) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
            (void)hipGetLastError();
            return fail(BSA_ERR_HIP, "hipGetDeviceProperties failed for device %d", dev);
        }
        di.ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        di.known = true;
        if (!di.ok) return fail(BSA_ERR_UNSUPPORTED, "device %d is %s; libbsa is built for gfx950 only", dev, prop.gcnArchName);
    }
    if (!di.ok) return fail(BSA_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
    return BSA_OK;
}

bsa_status hip_result(hipError_t e, const char* what) {
    if (e == hipSuccess) return BSA_OK;
    return fail(BSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

inline hipStream_t as_stream(void* s) { return (hipStream_t)s; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

constexpr double kLog2e = 1.4426950408889634;

bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + bn && y < x + an;
}

struct Span {
    const void* p;
    size_t bytes;
};

// True when an output range overlaps an input range or another output range.
bool outputs_overlap(std::initializer_list<Span> outs, std::initializer_list<Span> ins) {
    for (auto o = outs.begin(); o != outs.end(); ++o) {
        for (const Span& i : ins)
            if (overlaps(o->p, o->bytes, i.p, i.bytes)) return true;
        for (auto o2 = o + 1; o2 != outs.end(); ++o2)
            if (overlaps(o->p, o->bytes, o2->p, o2->bytes)) return true;
    }
    return false;
}

size_t elems(int32_t B, int32_t H, int32_t S, int32_t D) { return (size_t)B * H * S * D; }

// Checks shared by the fused RMSNorm + RoPE calls (one projection).
bsa_status check_norm_rope(const void* x, const void* w, const void* out, int32_t B, int32_t H, int32_t S, int32_t D,
                           int32_t block, int32_t gt, int32_t gh, int32_t gw, double eps, double theta) {
    bsa_status st = check_shape(B, H, S, D, block);
    if (st != BSA_OK) return st;
    if ((int64_t)H * D > bsa::kNormRopeMaxChannels)
        return fail(BSA_ERR_UNSUPPORTED, "H*D must be at most %d (got %lld)", bsa::kNormRopeMaxChannels, (long long)H * D);
    if (!x || !w || !out) return fail(BSA_ERR_INVALID_ARGUMENT, "null pointer");
    if (!aligned16(x) || !aligned16(w) || !aligned16(out))
        return fail(BSA_ERR_INVALID_ARGUMENT, "x, weight and out must be 16-byte aligned");
    if (gt < 1 || gh < 1 || gw < 1 || (int64_t)gt * gh * gw != S)
        return fail(BSA_ERR_INVALID_ARGUMENT, "grid %d x %d x %d does not hold S = %d tokens", gt, gh, gw, S);
    if (!(eps >= 0.0) || !isfinite(eps)) return fail(BSA_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0");
    if (!(theta > 0.0) || !isfinite(theta)) return fail(BSA_ERR_INVALID_ARGUMENT, "theta must be finite and > 0");
    const size_t tensor = (size_t)B * H * S * D * 2;
    if (overlaps(out, tensor, x, tensor) || overlaps(out, tensor, w, (size_t)H * D * 2))
        return fail(BSA_ERR_INVALID_ARGUMENT, "out must not overlap x or weight");
    return BSA_OK;
}

bsa::NormRopeArgs norm_rope_args(const void* x, const void* w, void* out, float* partial, int32_t B, int32_t H, int32_t S,
                                 int32_t gh, int32_t gw, double eps, double theta) {
    bsa::NormRopeArgs a;
    a.x = x;
    a.w = w;
    a.out = out;
    a.partial = partial;
    a.B = B;
    a.H = H;
    a.S = S;
    a.gh = gh;
    a.gw = gw;
    a.eps = (float)eps;
    a.theta = theta;
    return a;
}

// Scratch memory of bsa_select_noalloc: the pooled means that bsa_select keeps in the
// caller's workspace live here instead. One copy per device, at its own address, held until
// the process ends; host code uses only the address hipGetSymbolAddress returns for it.
constexpr size_t kScratchBytes = (size_t)64 << 20;
__device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::vector<void*> g_scratch;  // per device: the device address of `scratch`, once looked up

// The device address of `scratch` on the current device (looked up on first use).
bsa_status scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
        (void)hipGetLastError();
        return fail(BSA_ERR_NO_DEVICE, "no HIP device is available");
    }
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if ((int)g_scratch.size() <= dev) g_scratch.resize(dev + 1, nullptr);
    if (!g_scratch[dev]) {
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return fail(BSA_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
        }
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return BSA_OK;
}

}  // namespace

extern "C" {

int32_t bsa_num_blocks(int32_t S, int32_t block) {
    if (S < 1 || block < 1) return 0;
    return (int32_t)(((int64_t)S + block - 1) / block);
}

int32_t bsa_num_kept(int32_t n_blocks, double keep_ratio) {
    if (n_blocks < 1 || !(keep_ratio > 0.0) || keep_ratio > 1.0) return 0;
    double k = ceil(keep_ratio * (double)n_blocks - 1e-6);
    if (k < 1.0) k = 1.0;
    if (k > (double)n_blocks) k = (double)n_blocks;
    return (int32_t)k;
}

size_t bsa_select_workspace_bytes(int32_t B, int32_t H, int32_t S, int32_t D, int32_t block) {
    if (B < 1 || H < 1 || S < 1 || D < 1 || block < 1) return 0;
    const size_t n = (size_t)bsa_num_blocks(S, block);
    return round_up(2 * (size_t)B * H * n * D * sizeof(float), 256);
}

bsa_status bsa_pool(const void* x, int32_t B, int32_t H, int32_t S, int32_t D, int32_t block, float* xbar,
                    void* hip_stream) {
    bsa_status st = check_shape(B, H, S, D, block);
    if (st != BSA_OK) return st;
    if (!x || !xbar) return fail(BSA_ERR_INVALID_ARGUMENT, "null pointer");
    if (!aligned16(x) || !aligned16(xbar)) return fail(BSA_ERR_INVALID_ARGUMENT, "pointers must be 16-byte aligned");
    const size_t n = (size_t)bsa_num_blocks(S, block);
    if (outputs_overlap({{xbar, (size_t)B * H * n * D * 4}}, {{x, elems(B, H, S, D) * 2}}))
        return fail(BSA_ERR_INVALID_ARGUMENT, "xbar must not overlap x");
    if ((st = check_device()) != BSA_OK) return st;
    return hip_result(bsa::launch_pool(x, B * H, S, D, block, xbar, false, as_stream(hip_stream)), "pool launch");
}

bsa_status bsa_select(const void* q, const void* k, int32_t B, int32_t H, int32_t S, int32_t D, int32_t block,
                      double keep_ratio, int32_t* row_ptr, int32_t* col_idx, void* workspace, size_t workspace_bytes,
                      void* hip_stream) {
    bsa_status st = check_shape(B, H, S, D, block);
    if (st != BSA_OK) return st;
    if (!q || !k || !row_ptr || !col_idx || !workspace) return fail(BSA_ERR_INVALID_ARGUMENT, "null pointer");
    if (!aligned16(q) || !aligned16(k) || !aligned16(workspace))
        return fail(BSA_ERR_INVALID_ARGUMENT, "q, k and workspace must be 16-byte aligned");
    if (((uintptr_t)row_ptr & 3u) || ((uintptr_t)col_idx & 3u)) return fail(BSA_ERR_INVALID_ARGUMENT, "misaligned CSR arrays");
    const int32_t n = bsa_num_blocks(S, block);
    const int32_t kept = bsa_num_kept(n, keep_ratio);
    if (kept == 0) return fail(BSA_ERR_INVALID_ARGUMENT, "keep_ratio must be in (0, 1] (got %g)", keep_ratio);
    if (n > bsa::kMaxSelectBlocks) return fail(BSA_ERR_UNSUPPORTED, "bsa_select supports at most %d blocks per sequence (got %d)", bsa::kMaxSelectBlocks, n);
    if ((int64_t)B * H * n * kept >= ((int64_t)1 << 31)) return fail(BSA_ERR_UNSUPPORTED, "kept-block list too long for int32 indices");
    const size_t need = bsa_select_workspace_bytes(B, H, S, D, block);
    if (workspace_bytes < need) return fail(BSA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes (got %zu)", need, workspace_bytes);
    const size_t rows = (size_t)B * H * n, tbytes = elems(B, H, S, D) * 2;
    if (outputs_overlap({{row_ptr, (rows + 1) * 4}, {col_idx, rows * kept * 4}, {workspace, need}}, {{q, tbytes}, {k, tbytes}}))
        return fail(BSA_ERR_INVALID_ARGUMENT, "row_ptr, col_idx and workspace must not overlap q, k or each other");
    if ((st = check_device()) != BSA_OK) return st;
    float* qbar = (float*)workspace;
    float* kbarT = qbar + (size_t)B * H * n * D;
    hipStream_t s = as_stream(hip_stream);
    if ((st = hip_result(bsa::launch_pool_qk(q, k, B * H, S, D, block, qbar, kbarT, s), "pool launch")) != BSA_OK) return st;
    return hip_result(bsa::launch_select(qbar, kbarT, B * H, n, D, kept, row_ptr, col_idx, s), "select launch");
}

size_t bsa_select_noalloc_max_bytes(void) { return kScratchBytes; }

bsa_status bsa_select_noalloc(const void* q, const void* k, int32_t B, int32_t H, int32_t S, int32_t D, int32_t block,
                              double keep_ratio, int32_t* row_ptr, int32_t* col_idx, void* hip_stream) {
    bsa_status st = check_shape(B, H, S, D, block);
    if (st != BSA_OK) return st;
    if (!q || !k || !row_ptr || !col_idx) return fail(BSA_ERR_INVALID_ARGUMENT, "null pointer");
    if (!aligned16(q) || !aligned16(k)) return fail(BSA_ERR_INVALID_ARGUMENT, "q and k must be 16-byte aligned");
    if (((uintptr_t)row_ptr & 3u) || ((uintptr_t)col_idx & 3u)) return fail(BSA_ERR_INVALID_ARGUMENT, "misaligned CSR arrays");
    const int32_t n = bsa_num_blocks(S, block);
    const int32_t kept = bsa_num_kept(n, keep_ratio);
    if (kept == 0) return fail(BSA_ERR_INVALID_ARGUMENT, "keep_ratio must be in (0, 1] (got %g)", keep_ratio);
    if (n > bsa::kMaxSelectBlocks) return fail(BSA_ERR_UNSUPPORTED, "bsa_select_noalloc supports at most %d blocks per sequence (got %d)", bsa::kMaxSelectBlocks, n);
    if ((int64_t)B * H * n * kept >= ((int64_t)1 << 31)) return fail(BSA_ERR_UNSUPPORTED, "kept-block list too long for int32 indices");
    const size_t need = bsa_select_workspace_bytes(B, H, S, D, block);
    if (need > kScratchBytes)
        return fail(BSA_ERR_UNSUPPORTED, "bsa_select_noalloc holds at most %zu bytes of block means; this shape needs %zu (use bsa_select with a workspace)",
                    kScratchBytes, need);
    const size_t rows = (size_t)B * H * n, tbytes = elems(B, H, S, D) * 2;
    if (outputs_overlap({{row_ptr, (rows + 1) * 4}, {col_idx, rows * kept * 4}}, {{q, tbytes}, {k, tbytes}}))
        return fail(BSA_ERR_INVALID_ARGUMENT, "row_ptr and col_idx must not overlap q, k or each other");
    if ((st = check_device()) != BSA_OK) return st;
    void* ws = nullptr;
    if ((st = scratch_address(&ws)) != BSA_OK) return st;
    float* qbar = (float*)ws;
    float* kbarT = qbar + (size_t)B * H * n * D;
    hipStream_t s = as_stream(hip_stream);
    if ((st = hip_result(bsa::launch_pool_qk(q, k, B * H, S, D, block, qbar, kbarT, s), "pool launch")) != BSA_OK) return st;
    return hip_result(bsa::launch_select(qbar, kbarT, B * H, n, D, kept, row_ptr, col_idx, s), "select launch");
}

// mode: 0 = bf16, 1 = E4M3 Q/K with bf16 V, 2 = E4M3 Q/K, V (transposed) and weights.
static bsa_status forward_common(const void* q, const float* q_scale, const void* k, const float* k_scale, const void* v,
                                 const float* v_scale, int32_t B, int32_t H, int32_t S, int32_t D, int32_t block,
                                 const int32_t* row_ptr, const int32_t* col_idx, void* out, void* hip_stream, int mode) {
    bsa_status st = check_shape(B, H, S, D, block);
    if (st != BSA_OK) return st;
    if (!q || !k || !v || !row_ptr || !col_idx || !out) return fail(BSA_ERR_INVALID_ARGUMENT, "null pointer");
    if (mode != 0 && (!q_scale || !k_scale)) return fail(BSA_ERR_INVALID_ARGUMENT, "null scale pointer");
    if (mode == 2 && (!v_scale || ((uintptr_t)v_scale & 15u)))
        return fail(BSA_ERR_INVALID_ARGUMENT, "v_scale must be non-null and 16-byte aligned");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return fail(BSA_ERR_INVALID_ARGUMENT, "q, k, v and out must be 16-byte aligned");
    if (((uintptr_t)row_ptr & 3u) || ((uintptr_t)col_idx & 3u)) return fail(BSA_ERR_INVALID_ARGUMENT, "misaligned CSR arrays");
    {
        const size_t e = elems(B, H, S, D), rows = (size_t)B * H * bsa_num_blocks(S, block);
        const size_t qk_bytes = mode == 0 ? 2 * e : e;
        const size_t v_bytes = mode == 2 ? bsa_vt_fp8_bytes(B, H, S, D, block) : 2 * e;
        if (outputs_overlap({{out, 2 * e}}, {{q, qk_bytes}, {k, qk_bytes}, {v, v_bytes}, {row_ptr, (rows + 1) * 4}}))
            return fail(BSA_ERR_INVALID_ARGUMENT, "out must not overlap q, k, v or row_ptr");
    }
    if ((st = check_device()) != BSA_OK) return st;
    bsa::AttnArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.q_scale = q_scale;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.row_ptr = row_ptr;
    a.col_idx = col_idx;
    a.out = out;
    a.BH = B * H;
    a.S = S;
    a.n = bsa_num_blocks(S, block);
    a.S_pad = a.n * block;
    a.sm_scale_log2 = (float)(kLog2e / sqrt((double)D));
    return hip_result(bsa::launch_attention(a, D, block, mode, as_stream(hip_stream)), "attention launch");
}

bsa_status bsa_forward(const void* q, const void* k, const void* v, int32_t B, int32_t H, int32_t S, int32_t D,
                       int32_t block, const int32_t* row_ptr, const int32_t* col_idx, void* out, void* hip_stream) {
    return forward_common(q, nullptr, k, nullptr, v, nullptr, B, H, S, D, block, row_ptr, col_idx, out, hip_stream, 0);
}

bsa_status bsa_forward_fp8(const void* q_e4m3, const float* q_scale, const void* k_e4m3, const float* k_scale,
                           const void* v, int32_t B, int32_t H, int32_t S, int32_t D, int32_t block,
                           const int32_t* row_ptr, const int32_t* col_idx, void* out, void* hip_stream) {
    return forward_common(q_e4m3, q_scale, k_e4m3, k_scale, v, nullptr, B, H, S, D, block, row_ptr, col_idx, out,
                          hip_stream, 1);
}

size_t bsa_vt_fp8_bytes(int32_t B, int32_t H, int32_t S, int32_t D, int32_t block) {
    if (B < 1 || H < 1 || S < 1 || D < 1 || block < 1) return 0;
    return (size_t)B * H * D * (size_t)bsa_num_blocks(S, block) * block;
}

bsa_status bsa_select_quantize(const void* q, const void* k, int32_t B, int32_t H, int32_t S, int32_t D, int32_t block,
                               double keep_ratio, int32_t* row_ptr, int32_t* col_idx, void* q_e4m3, float* q_scale,
                               void* k_e4m3, float* k_scale, void* workspace, size_t workspace_bytes, void* hip_stream) {
    bsa_status st = check_shape(B, H, S, D, block);
    if (st != BSA_OK) return st;
    if (!q || !k || !row_ptr || !col_idx || !workspace || !q_e4m3 || !q_scale || !k_e4m3 || !k_scale)
        return fail(BSA_ERR_INVALID_ARGUMENT, "null pointer");
    if (!aligned16(q) || !aligned16(k) || !aligned16(workspace) || !aligned16(q_e4m3) || !aligned16(k_e4m3))
        return fail(BSA_ERR_INVALID_ARGUMENT, "q, k, the code buffers and workspace must be 16-byte aligned");
    if (((uintptr_t)row_ptr & 3u) || ((uintptr_t)col_idx & 3u) || ((uintptr_t)q_scale & 3u) || ((uintptr_t)k_scale & 3u))
        return fail(BSA_ERR_INVALID_ARGUMENT, "misaligned CSR or scale arrays");
    const int32_t n = bsa_num_blocks(S, block);
    const int32_t kept = bsa_num_kept(n, keep_ratio);
    if (kept == 0) return fail(BSA_ERR_INVALID_ARGUMENT, "keep_ratio must be in (0, 1] (got %g)", keep_ratio);
    if (n > bsa::kMaxSelectBlocks) return fail(BSA_ERR_UNSUPPORTED, "bsa_select_quantize supports at most %d blocks per sequence (got %d)", bsa::kMaxSelectBlocks, n);
    if ((int64_t)B * H * n * kept >= ((int64_t)1 << 31)) return fail(BSA_ERR_UNSUPPORTED, "kept-block list too long for int32 indices");
    const size_t need = bsa_select_workspace_bytes(B, H, S, D, block);
    if (workspace_bytes < need) return fail(BSA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes (got %zu)", need, workspace_bytes);
    {
        const size_t rows = (size_t)B * H * n, e = elems(B, H, S, D);
        if (outputs_overlap({{row_ptr, (rows + 1) * 4}, {col_idx, rows * kept * 4}, {workspace, need}, {q_e4m3, e},
                             {k_e4m3, e}, {q_scale, rows * 4}, {k_scale, rows * 4}},
                            {{q, 2 * e}, {k, 2 * e}}))
            return fail(BSA_ERR_INVALID_ARGUMENT, "outputs must not overlap q, k or each other");
    }
    if ((st = check_device()) != BSA_OK) return st;
    float* qbar = (float*)workspace;
    float* kbarT = qbar + (size_t)B * H * n * D;
    hipStream_t s = as_stream(hip_stream);
    if ((st = hip_result(bsa::launch_pool_quant_qk(q, k, B * H, S, D, block, qbar, kbarT, q_e4m3, k_e4m3, q_scale, k_scale, s),
                         "pool/quantise launch")) != BSA_OK)
        return st;
    return hip_result(bsa::launch_select(qbar, kbarT, B * H, n, D, kept, row_ptr, col_idx, s), "select launch");
}

bsa_status bsa_quantize_v_fp8(const void* v, int32_t B, int32_t H, int32_t S, int32_t D, int32_t block, void* vt_e4m3,
                              float* v_scale, void* hip_stream) {
    bsa_status st = check_shape(B, H, S, D, block);
    if (st != BSA_OK) return st;
    if (!v || !vt_e4m3 || !v_scale) return fail(BSA_ERR_INVALID_ARGUMENT, "null pointer");
    if (!aligned16(v) || !aligned16(vt_e4m3) || !aligned16(v_scale))
        return fail(BSA_ERR_INVALID_ARGUMENT, "v, vt_e4m3 and v_scale must be 16-byte aligned");
    if (outputs_overlap({{vt_e4m3, bsa_vt_fp8_bytes(B, H, S, D, block)}, {v_scale, (size_t)B * H * D * 4}},
                        {{v, elems(B, H, S, D) * 2}}))
        return fail(BSA_ERR_INVALID_ARGUMENT, "vt_e4m3 and v_scale must not overlap v or each other");
    if ((st = check_device()) != BSA_OK) return st;
    return hip_result(bsa::launch_quantize_v(v, B * H, S, D, block, vt_e4m3, v_scale, as_stream(hip_stream)),
                      "quantise V launch");
}

bsa_status bsa_forward_fp8_full(const void* q_e4m3, const float* q_scale, const void* k_e4m3, const float* k_scale,
                                const void* vt_e4m3, const float* v_scale, int32_t B, int32_t H, int32_t S, int32_t D,
                                int32_t block, const int32_t* row_ptr, const int32_t* col_idx, void* out,
                                void* hip_stream) {
    return forward_common(q_e4m3, q_scale, k_e4m3, k_scale, vt_e4m3, v_scale, B, H, S, D, block, row_ptr, col_idx, out,
                          hip_stream, 2);
}

bsa_status bsa_quantize_fp8(const void* x, int32_t B, int32_t H, int32_t S, int32_t D, int32_t block, void* x_e4m3,
                            float* scale, void* hip_stream) {
    bsa_status st = check_shape(B, H, S, D, block);
    if (st != BSA_OK) return st;
    if (!x || !x_e4m3 || !scale) return fail(BSA_ERR_INVALID_ARGUMENT, "null pointer");
    if (!aligned16(x) || !aligned16(x_e4m3) || ((uintptr_t)scale & 3u))
        return fail(BSA_ERR_INVALID_ARGUMENT, "x and x_e4m3 must be 16-byte aligned");
    if (outputs_overlap({{x_e4m3, elems(B, H, S, D)}, {scale, (size_t)B * H * bsa_num_blocks(S, block) * 4}},
                        {{x, elems(B, H, S, D) * 2}}))
        return fail(BSA_ERR_INVALID_ARGUMENT, "x_e4m3 and scale must not overlap x or each other");
    if ((st = check_device()) != BSA_OK) return st;
    return hip_result(bsa::launch_quantize_fp8(x, B * H, S, D, block, x_e4m3, scale, as_stream(hip_stream)),
                      "quantize launch");
}

size_t bsa_norm_rope_workspace_bytes(int32_t B, int32_t H, int32_t S, int32_t D) {
    if (B < 1 || H < 1 || S < 1 || D < 1) return 0;
    const size_t chunks = ((size_t)S + bsa::kNormRopeTokens - 1) / bsa::kNormRopeTokens;
    return round_up((size_t)B * chunks * H * D * sizeof(float), 256);
}

size_t bsa_norm_rope_select_workspace_bytes(int32_t B, int32_t H, int32_t S, int32_t D, int32_t block) {
    const size_t part = bsa_norm_rope_workspace_bytes(B, H, S, D);
    const size_t means = bsa_select_workspace_bytes(B, H, S, D, block);
    if (part == 0 || means == 0) return 0;
    return 2 * part + means;
}

bsa_status bsa_norm_rope(const void* x, const void* weight, int32_t B, int32_t H, int32_t S, int32_t D, int32_t block,
                         int32_t grid_t, int32_t grid_h, int32_t grid_w, double eps, double theta, void* out,
                         float* xbar, void* workspace, size_t workspace_bytes, void* hip_stream) {
    bsa_status st = check_norm_rope(x, weight, out, B, H, S, D, block, grid_t, grid_h, grid_w, eps, theta);
    if (st != BSA_OK) return st;
    if (xbar) {
        if (!workspace) return fail(BSA_ERR_INVALID_ARGUMENT, "null workspace");
        if (!aligned16(workspace) || ((uintptr_t)xbar & 3u))
            return fail(BSA_ERR_INVALID_ARGUMENT, "workspace must be 16-byte and xbar 4-byte aligned");
        const size_t need = bsa_norm_rope_workspace_bytes(B, H, S, D);
        if (workspace_bytes < need) return fail(BSA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes (got %zu)", need, workspace_bytes);
    }
    if ((st = check_device()) != BSA_OK) return st;
    hipStream_t s = as_stream(hip_stream);
    bsa::NormRopeArgs a = norm_rope_args(x, weight, out, xbar ? (float*)workspace : nullptr, B, H, S, grid_h, grid_w, eps, theta);
    if ((st = hip_result(bsa::launch_norm_rope(a, D, s), "norm/rope launch")) != BSA_OK) return st;
    if (!xbar) return BSA_OK;
    return hip_result(bsa::launch_norm_rope_means((const float*)workspace, B, H, S, D, block, xbar, false, s), "means launch");
}

bsa_status bsa_norm_rope_select(const void* xq, const void* xk, const void* wq, const void* wk, int32_t B, int32_t H,
                                int32_t S, int32_t D, int32_t block, int32_t grid_t, int32_t grid_h, int32_t grid_w,
                                double eps, double theta, double keep_ratio, void* q_out, void* k_out, int32_t* row_ptr,
                                int32_t* col_idx, void* workspace, size_t workspace_bytes, void* hip_stream) {
    bsa_status st = check_norm_rope(xq, wq, q_out, B, H, S, D, block, grid_t, grid_h, grid_w, eps, theta);
    if (st != BSA_OK) return st;
    if ((st = check_norm_rope(xk, wk, k_out, B, H, S, D, block, grid_t, grid_h, grid_w, eps, theta)) != BSA_OK) return st;
    if (!row_ptr || !col_idx || !workspace) return fail(BSA_ERR_INVALID_ARGUMENT, "null pointer");
    if (!aligned16(workspace)) return fail(BSA_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
    if (((uintptr_t)row_ptr & 3u) || ((uintptr_t)col_idx & 3u)) return fail(BSA_ERR_INVALID_ARGUMENT, "misaligned CSR arrays");
    const size_t tensor = (size_t)B * H * S * D * 2;
    if (overlaps(q_out, tensor, k_out, tensor) || overlaps(q_out, tensor, xk, tensor) || overlaps(k_out, tensor, xq, tensor) ||
        overlaps(q_out, tensor, wk, (size_t)H * D * 2) || overlaps(k_out, tensor, wq, (size_t)H * D * 2))
        return fail(BSA_ERR_INVALID_ARGUMENT, "outputs must not overlap the inputs or each other");
    const int32_t n = bsa_num_blocks(S, block);
    const int32_t kept = bsa_num_kept(n, keep_ratio);
    if (kept == 0) return fail(BSA_ERR_INVALID_ARGUMENT, "keep_ratio must be in (0, 1] (got %g)", keep_ratio);
    if (n > bsa::kMaxSelectBlocks) return fail(BSA_ERR_UNSUPPORTED, "bsa_norm_rope_select supports at most %d blocks per sequence (got %d)", bsa::kMaxSelectBlocks, n);
    if ((int64_t)B * H * n * kept >= ((int64_t)1 << 31)) return fail(BSA_ERR_UNSUPPORTED, "kept-block list too long for int32 indices");
    const size_t need = bsa_norm_rope_select_workspace_bytes(B, H, S, D, block);
    if (workspace_bytes < need) return fail(BSA_ERR_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes (got %zu)", need, workspace_bytes);
    if ((st = check_device()) != BSA_OK) return st;
    const size_t part = bsa_norm_rope_workspace_bytes(B, H, S, D);
    float* qpart = (float*)workspace;
    float* kpart = (float*)((char*)workspace + part);
    float* qbar = (float*)((char*)workspace + 2 * part);
    float* kbarT = qbar + (size_t)B * H * n * D;
    hipStream_t s = as_stream(hip_stream);
    bsa::NormRopeArgs aq = norm_rope_args(xq, wq, q_out, qpart, B, H, S, grid_h, grid_w, eps, theta);
    bsa::NormRopeArgs ak = norm_rope_args(xk, wk, k_out, kpart, B, H, S, grid_h, grid_w, eps, theta);
    if ((st = hip_result(bsa::launch_norm_rope(aq, D, s), "norm/rope launch")) != BSA_OK) return st;
    if ((st = hip_result(bsa::launch_norm_rope(ak, D, s), "norm/rope launch")) != BSA_OK) return st;
    if ((st = hip_result(bsa::launch_norm_rope_means(qpart, B, H, S, D, block, qbar, false, s), "means launch")) != BSA_OK)
        return st;
    if ((st = hip_result(bsa::launch_norm_rope_means(kpart, B, H, S, D, block, kbarT, true, s), "means launch")) != BSA_OK)
        return st;
    return hip_result(bsa::launch_select(qbar, kbarT, B * H, n, D, kept, row_ptr, col_idx, s), "select launch");
}

bsa_status bsa_check_csr(const int32_t* row_ptr, int64_t row_ptr_len, const int32_t* col_idx, int64_t col_idx_len,
                         int32_t rows, int32_t n_blocks) {
    if (!row_ptr || rows < 0 || n_blocks < 1 || col_idx_len < 0) return fail(BSA_ERR_INVALID_ARGUMENT, "bad arguments");
    if (row_ptr_len != (int64_t)rows + 1)
        return fail(BSA_ERR_INVALID_ARGUMENT, "row_ptr has %lld entries, expected rows + 1 = %lld", (long long)row_ptr_len,
                    (long long)rows + 1);
    if (row_ptr[0] != 0) return fail(BSA_ERR_INVALID_ARGUMENT, "row_ptr[0] = %d, expected 0", row_ptr[0]);
    for (int32_t r = 0; r < rows; ++r) {
        const int32_t a = row_ptr[r], b = row_ptr[r + 1];
        if (b < a) return fail(BSA_ERR_INVALID_ARGUMENT, "row_ptr decreases at row %d", r);
        if ((int64_t)b > col_idx_len)
            return fail(BSA_ERR_INVALID_ARGUMENT, "row %d ends at %d, past col_idx's %lld entries", r, b,
                        (long long)col_idx_len);
        if (b > a && !col_idx) return fail(BSA_ERR_INVALID_ARGUMENT, "null col_idx");
        for (int32_t p = a; p < b; ++p) {
            const int32_t j = col_idx[p];
            if (j < 0 || j >= n_blocks) return fail(BSA_ERR_INVALID_ARGUMENT, "row %d: index %d outside [0, %d)", r, j, n_blocks);
            if (p > a && j <= col_idx[p - 1]) return fail(BSA_ERR_INVALID_ARGUMENT, "row %d: indices not strictly ascending", r);
        }
    }
    return BSA_OK;
}

const char* bsa_status_string(bsa_status status) {
    switch (status) {
        case BSA_OK: return "BSA_OK";
        case BSA_ERR_INVALID_ARGUMENT: return "BSA_ERR_INVALID_ARGUMENT";
        case BSA_ERR_UNSUPPORTED: return "BSA_ERR_UNSUPPORTED";
        case BSA_ERR_WORKSPACE_TOO_SMALL: return "BSA_ERR_WORKSPACE_TOO_SMALL";
        case BSA_ERR_NO_DEVICE: return "BSA_ERR_NO_DEVICE";
        case BSA_ERR_HIP: return "BSA_ERR_HIP";
    }
    return "BSA_ERR_UNKNOWN";
}

const char* bsa_last_error(void) { return g_err; }

}  // extern "C"
