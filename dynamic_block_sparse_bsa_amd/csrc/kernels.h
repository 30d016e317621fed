// Internal launcher interface between the C ABI (bsa_api.hip) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsa {

struct AttnArgs {
    const void* q;          // bf16 or E4M3 [B,H,S,D]
    const void* k;          // bf16 or E4M3 [B,H,S,D]
    const void* v;          // bf16 [B,H,S,D], or (full fp8 path) E4M3 [B*H, D, S_pad], key-permuted
    const float* q_scale;   // [B*H*n] (fp8 only)
    const float* k_scale;   // [B*H*n] (fp8 only)
    const float* v_scale;   // [B*H*D] (full fp8 path only)
    const int32_t* row_ptr;
    const int32_t* col_idx;
    void* out;              // bf16 [B,H,S,D]
    int BH, S, n;
    int S_pad;              // n * block (full fp8 path only)
    float sm_scale_log2;    // log2(e) / sqrt(D)
};

// mode: 0 = bf16, 1 = E4M3 Q/K with bf16 V, 2 = E4M3 Q/K, V and weights.
hipError_t launch_attention(const AttnArgs& a, int D, int block, int mode, hipStream_t stream);

// Block means of Q (row-major) and K (transposed) and their per-block E4M3 codes and scales,
// from one read of each block.
hipError_t launch_pool_quant_qk(const void* q, const void* k, int BH, int S, int D, int block, float* qbar, float* kbarT,
                                void* q8, void* k8, float* qscale, float* kscale, hipStream_t stream);

// Per-channel E4M3 codes of V, transposed and key-permuted ([BH, D, n*block]), and scales.
hipError_t launch_quantize_v(const void* v, int BH, int S, int D, int block, void* vt, float* vscale, hipStream_t stream);

// Block means of x (bf16 [BH,S,D]) into fp32: row-major [BH,n,D], or [BH,D,n] if transposed.
hipError_t launch_pool(const void* x, int BH, int S, int D, int block, float* xbar, bool transposed,
                       hipStream_t stream);

// Two pooled tensors in one launch: qbar row-major, kbar transposed.
hipError_t launch_pool_qk(const void* q, const void* k, int BH, int S, int D, int block, float* qbar,
                          float* kbarT, hipStream_t stream);

// Scores from pooled means and top-k per row; writes row_ptr (uniform) and col_idx.
hipError_t launch_select(const float* qbar, const float* kbarT, int BH, int n, int D, int kept,
                         int32_t* row_ptr, int32_t* col_idx, hipStream_t stream);

hipError_t launch_quantize_fp8(const void* x, int BH, int S, int D, int block, void* codes, float* scale,
                               hipStream_t stream);

// Fused RMSNorm + 3D RoPE + head-major transpose (+ partial block sums) of a projection.
struct NormRopeArgs {
    const void* x;    // bf16 [B, S, H*D], token-major
    const void* w;    // bf16 [H*D]
    void* out;        // bf16 [B, H, S, D]
    float* partial;   // fp32 [B, ceil(S / kNormRopeTokens), H*D] sums of out, or null
    int B, H, S, gh, gw;  // gh, gw: height and width of the latent grid
    float eps;
    double theta;
};
constexpr int kNormRopeTokens = 32;    // tokens per workgroup (and per partial sum)
constexpr int kNormRopeMaxChannels = 8192;  // H*D limit (16 chunks of 8 per lane)
hipError_t launch_norm_rope(const NormRopeArgs& a, int D, hipStream_t stream);
// Block means from the partial sums: [B, H, n, D], or [B, H, D, n] if transposed.
hipError_t launch_norm_rope_means(const float* partial, int B, int H, int S, int D, int block, float* xbar,
                                  bool transposed, hipStream_t stream);

constexpr int kSelectRowsPerGroup = 4;
constexpr int kMaxSelectBlocks = 8192;

}  // namespace bsa
