// Block pooling, block-pair scoring and top-k selection, and the FP8 quantiser, for gfx950.
//
// Method: the knowledge card "600倍加速，720p视频实时生成！单卡也能带的动14B模型", section
// 方法/产品要点, item 动态稀疏量化注意力: Query/Key block means give a quick estimate of
// attention importance; about 10-20 % of the key blocks are kept per query block; the
// sparse path becomes an FP8 path (SageAttention2). The aoyii.com article "单卡 RTX 5090
// 跑 Wan2.2-A14B", section 四步拆解, step 3 动态稀疏注意力, says the same.
//
// Pooling and quantisation are HBM-bound streaming kernels: one workgroup per (b*h, token
// block) reads the block once with coalesced 16-byte loads. Scoring reads the pooled
// means (a few MB); selection is an exact radix select per row on 32-bit order-preserving
// keys with ties broken towards the lower block index.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"
#include "kernels.h"

namespace bsa {
namespace {

constexpr int kThreads = 256;
// Rows of up to 64 * kSelectRegChunks blocks keep their selection keys in registers.
constexpr int kSelectRegChunks = 16;

// ---- pooling -------------------------------------------------------------------------
// Thread t handles 16-byte chunk (t % CH) of the row, for tokens t / CH, t / CH + TL, ...
template <int D>
__global__ void __launch_bounds__(kThreads) pool_kernel(const uint16_t* __restrict__ x0, const uint16_t* __restrict__ x1,
                                                        int BH, int S, int block, int n, float* __restrict__ out0,
                                                        float* __restrict__ out1, int transposed_mask) {
    constexpr int CH = D / 8, TL = kThreads / CH;
    __shared__ float red[TL][D + 4];
    const int which = blockIdx.y;
    const uint16_t* x = which ? x1 : x0;
    float* out = which ? out1 : out0;
    const bool transposed = (transposed_mask >> which) & 1;
    const int rowi = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = rowi / n, i = rowi - bh * n;
    const int t0 = i * block;
    const int cnt = (S - t0) < block ? (S - t0) : block;
    const int c = threadIdx.x % CH, tl = threadIdx.x / CH;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    const uint16_t* base = x + ((int64_t)bh * S + t0) * D + 8 * c;
    // All of a thread's loads (blocks hold at most 128 tokens) are issued before the first
    // sum; the sums still run over the tokens in ascending order.
    constexpr int MAXT = 128 / TL;
    u32x4 w[MAXT];
#pragma unroll
    for (int u = 0; u < MAXT; ++u) {
        const int t = tl + u * TL;
        w[u] = t < cnt ? *(const u32x4*)(base + (int64_t)t * D) : (u32x4){0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < MAXT; ++u) {
        if (tl + u * TL >= cnt) break;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc[2 * e] += __uint_as_float(w[u][e] << 16);
            acc[2 * e + 1] += __uint_as_float(w[u][e] & 0xFFFF0000u);
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[tl][8 * c + e] = acc[e];
    __syncthreads();
    if (threadIdx.x < D) {
        const int d = threadIdx.x;
        float s = 0.0f;
        for (int r = 0; r < TL; ++r) s += red[r][d];
        const float mean = s / (float)cnt;
        if (transposed) out[((int64_t)bh * D + d) * n + i] = mean;
        else out[((int64_t)bh * n + i) * D + d] = mean;
    }
}

// ---- scores + top-k ------------------------------------------------------------------
// One workgroup per (b*h, group of R query blocks): the pooled keys of the head are read
// once per group (R rows share each load), and wave w selects for query blocks w, w + 4, ...
// of the group. Scores live in LDS (R * n floats); during the select a row of up to
// 64 * kSelectRegChunks blocks keeps its keys in registers (chunk c of lane l: block 64c + l),
// so the 32 threshold passes need no LDS reads. Longer rows select from LDS.
template <int D, int R>
__global__ void __launch_bounds__(kThreads) select_kernel(const float* __restrict__ qbar, const float* __restrict__ kbarT,
                                                          int BH, int n, int kept, float scale,
                                                          int32_t* __restrict__ row_ptr, int32_t* __restrict__ col_idx) {
    extern __shared__ __attribute__((aligned(16))) float smem[];
    float* qs = smem;            // [R][D]
    float* sc = smem + R * D;    // [R][n]
    const int groups = (n + R - 1) / R;
    const int gi = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = gi / groups, i0 = (gi - bh * groups) * R;

    for (int e = threadIdx.x; e < R * D; e += kThreads) {
        const int r = e / D, d = e - r * D;
        qs[e] = (i0 + r < n) ? qbar[((int64_t)bh * n + i0 + r) * D + d] : 0.0f;
    }
    __syncthreads();

    // K-bar^T of this head through a buffer resource: the channel offset is a scalar, so the
    // 16 loads a thread keeps in flight per batch cost no per-lane address arithmetic. Each
    // score still adds its D products in channel order.
    const __amdgpu_buffer_rsrc_t kb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(kbarT + (int64_t)bh * D * n), 0, D * n * 4, 0x00020000);
    constexpr int DB = 16;  // channels per batch of loads
    for (int j = threadIdx.x; j < n; j += kThreads) {
        float acc[R];
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = 0.0f;
        for (int d0 = 0; d0 < D; d0 += DB) {
            float kv[DB];
#pragma unroll
            for (int u = 0; u < DB; ++u)
                kv[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(kb, j * 4, (d0 + u) * n * 4, 0));
#pragma unroll
            for (int u = 0; u < DB; u += 4)
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const f32x4 qv = *(const f32x4*)(qs + r * D + d0 + u);
                    acc[r] = __builtin_fmaf(qv[0], kv[u], acc[r]);
                    acc[r] = __builtin_fmaf(qv[1], kv[u + 1], acc[r]);
                    acc[r] = __builtin_fmaf(qv[2], kv[u + 2], acc[r]);
                    acc[r] = __builtin_fmaf(qv[3], kv[u + 3], acc[r]);
                }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) sc[r * n + j] = acc[r] * scale;
    }
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int w = threadIdx.x >> 6; w < R && i0 + w < n; w += kThreads / 64) {
        const int i = i0 + w;
        const int64_t row = (int64_t)bh * n + i;
        int32_t* out = col_idx + row * kept;
        const float* srow = sc + w * n;
        if (n <= 64 * kSelectRegChunks) {
            // Keys of the row in registers, chunk c holding blocks 64c + lane.
            const int nch = (n + 63) / 64;
            uint32_t kr[kSelectRegChunks];
#pragma unroll
            for (int c = 0; c < kSelectRegChunks; ++c) {
                const int j = 64 * c + lane;
                kr[c] = (c < nch && j < n) ? ordered_key(srow[j]) : 0u;
            }
            // Largest T with #(key >= T) >= kept: the kept-th largest key. Real keys are >= 1
            // (ordered_key maps no finite score to 0), so the padding never counts.
            uint32_t T = 0;
            for (int bit = 31; bit >= 0; --bit) {
                const uint32_t cand = T | (1u << bit);
                int cnt = 0;
#pragma unroll
                for (int c = 0; c < kSelectRegChunks; ++c)
                    if (c < nch) cnt += __popcll(__ballot(kr[c] >= cand));
                if (cnt >= kept) T = cand;
            }
            int gt = 0;
#pragma unroll
            for (int c = 0; c < kSelectRegChunks; ++c)
                if (c < nch) gt += __popcll(__ballot(kr[c] > T));
            const int need = kept - gt;  // how many blocks with key == T to take, lowest index first
            int pos = 0, ties = 0;
#pragma unroll
            for (int c = 0; c < kSelectRegChunks; ++c) {
                if (c >= nch) break;
                const int j = 64 * c + lane;
                const bool valid = j < n;
                const bool eq = valid && kr[c] == T;
                const uint64_t eqm = __ballot(eq);
                const int tie_rank = ties + __popcll(eqm & below);
                const bool sel = valid && (kr[c] > T || (eq && tie_rank < need));
                const uint64_t selm = __ballot(sel);
                if (sel) out[pos + __popcll(selm & below)] = j;
                pos += __popcll(selm);
                ties += __popcll(eqm);
            }
        } else {
            uint32_t* key = (uint32_t*)(sc + w * n);
            for (int j = lane; j < n; j += 64) key[j] = ordered_key(srow[j]);
            // (each lane rewrites only the entries it reads below; a wave sees its own writes)
            uint32_t T = 0;
            for (int bit = 31; bit >= 0; --bit) {
                const uint32_t cand = T | (1u << bit);
                int cnt = 0;
                for (int j0 = 0; j0 < n; j0 += 64) {
                    const int j = j0 + lane;
                    cnt += __popcll(__ballot((j < n) && key[j] >= cand));
                }
                if (cnt >= kept) T = cand;
            }
            int gt = 0;
            for (int j0 = 0; j0 < n; j0 += 64) {
                const int j = j0 + lane;
                gt += __popcll(__ballot((j < n) && key[j] > T));
            }
            const int need = kept - gt;
            int pos = 0, ties = 0;
            for (int j0 = 0; j0 < n; j0 += 64) {
                const int j = j0 + lane;
                const uint32_t kj = (j < n) ? key[j] : 0u;
                const bool eq = (j < n) && kj == T;
                const uint64_t eqm = __ballot(eq);
                const int tie_rank = ties + __popcll(eqm & below);
                const bool sel = (j < n) && (kj > T || (eq && tie_rank < need));
                const uint64_t selm = __ballot(sel);
                if (sel) out[pos + __popcll(selm & below)] = j;
                pos += __popcll(selm);
                ties += __popcll(eqm);
            }
        }
        if (lane == 0) {
            row_ptr[row] = (int32_t)(row * kept);
            if (row == (int64_t)BH * n - 1) row_ptr[row + 1] = (int32_t)((row + 1) * kept);
        }
    }
}

// ---- FP8 quantisation ------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(kThreads) quant_kernel(const uint16_t* __restrict__ x, int BH, int S, int block, int n,
                                                         uint8_t* __restrict__ codes, float* __restrict__ scale) {
    constexpr int CH = D / 8;
    __shared__ float wmax[kThreads / 64];
    const int rowi = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = rowi / n, i = rowi - bh * n;
    const int t0 = i * block;
    const int cnt = (S - t0) < block ? (S - t0) : block;
    const int64_t base = ((int64_t)bh * S + t0) * D;
    const int chunks = cnt * CH;
    // One read of the block: a thread's chunks (at most 128 rows * CH / kThreads of them) stay
    // in registers from the absmax pass to the code pass.
    constexpr int MAXQ = 128 * CH / kThreads;
    u32x4 w[MAXQ];
    float amax = 0.0f;
#pragma unroll
    for (int it = 0; it < MAXQ; ++it) {
        const int q = threadIdx.x + it * kThreads;
        w[it] = q < chunks ? *(const u32x4*)(x + base + 8 * (int64_t)q) : (u32x4){0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int it = 0; it < MAXQ; ++it)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            amax = fmaxf(amax, fabsf(__uint_as_float(w[it][e] << 16)));
            amax = fmaxf(amax, fabsf(__uint_as_float(w[it][e] & 0xFFFF0000u)));
        }
    for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = wmax[0];
#pragma unroll
    for (int wv = 1; wv < kThreads / 64; ++wv) amax = fmaxf(amax, wmax[wv]);
    const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
    if (threadIdx.x == 0) scale[rowi] = sc;
#pragma unroll
    for (int it = 0; it < MAXQ; ++it) {
        const int q = threadIdx.x + it * kThreads;
        if (q >= chunks) break;
        u32x2 packed;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            int v = 0;
            v = __builtin_amdgcn_cvt_pk_fp8_f32(__uint_as_float(w[it][2 * e] << 16) / sc,
                                                __uint_as_float(w[it][2 * e] & 0xFFFF0000u) / sc, v, false);
            v = __builtin_amdgcn_cvt_pk_fp8_f32(__uint_as_float(w[it][2 * e + 1] << 16) / sc,
                                                __uint_as_float(w[it][2 * e + 1] & 0xFFFF0000u) / sc, v, true);
            packed[e] = (uint32_t)v;
        }
        *(u32x2*)(codes + base + 8 * (int64_t)q) = packed;
    }
}

}  // namespace

hipError_t launch_pool(const void* x, int BH, int S, int D, int block, float* xbar, bool transposed, hipStream_t stream) {
    const int n = (S + block - 1) / block;
    dim3 grid(BH * n, 1);
    if (D == 128)
        hipLaunchKernelGGL(pool_kernel<128>, grid, dim3(kThreads), 0, stream, (const uint16_t*)x, (const uint16_t*)x, BH, S,
                           block, n, xbar, xbar, transposed ? 3 : 0);
    else
        hipLaunchKernelGGL(pool_kernel<64>, grid, dim3(kThreads), 0, stream, (const uint16_t*)x, (const uint16_t*)x, BH, S,
                           block, n, xbar, xbar, transposed ? 3 : 0);
    return hipGetLastError();
}

hipError_t launch_pool_qk(const void* q, const void* k, int BH, int S, int D, int block, float* qbar, float* kbarT,
                          hipStream_t stream) {
    const int n = (S + block - 1) / block;
    dim3 grid(BH * n, 2);
    if (D == 128)
        hipLaunchKernelGGL(pool_kernel<128>, grid, dim3(kThreads), 0, stream, (const uint16_t*)q, (const uint16_t*)k, BH, S,
                           block, n, qbar, kbarT, 2);
    else
        hipLaunchKernelGGL(pool_kernel<64>, grid, dim3(kThreads), 0, stream, (const uint16_t*)q, (const uint16_t*)k, BH, S,
                           block, n, qbar, kbarT, 2);
    return hipGetLastError();
}

template <int D, int R>
static hipError_t launch_select_r(const float* qbar, const float* kbarT, int BH, int n, int kept, int32_t* row_ptr,
                                  int32_t* col_idx, hipStream_t stream) {
    const int groups = (n + R - 1) / R;
    const size_t smem = sizeof(float) * (size_t)R * (D + n);
    const float scale = 1.0f / sqrtf((float)D);
    if (smem > 65536) {
        hipError_t e = hipFuncSetAttribute((const void*)select_kernel<D, R>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)smem);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((select_kernel<D, R>), dim3(BH * groups), dim3(kThreads), smem, stream, qbar, kbarT, BH, n, kept,
                       scale, row_ptr, col_idx);
    return hipGetLastError();
}

hipError_t launch_select(const float* qbar, const float* kbarT, int BH, int n, int D, int kept, int32_t* row_ptr,
                         int32_t* col_idx, hipStream_t stream) {
    // Four query blocks per workgroup: measured faster than 8 or 16 (more workgroups in flight
    // outweigh the extra reads of the pooled keys, which stay in L2).
    constexpr int R = kSelectRowsPerGroup;
    if (D == 128) return launch_select_r<128, R>(qbar, kbarT, BH, n, kept, row_ptr, col_idx, stream);
    return launch_select_r<64, R>(qbar, kbarT, BH, n, kept, row_ptr, col_idx, stream);
}

hipError_t launch_quantize_fp8(const void* x, int BH, int S, int D, int block, void* codes, float* scale,
                               hipStream_t stream) {
    const int n = (S + block - 1) / block;
    if (D == 128)
        hipLaunchKernelGGL(quant_kernel<128>, dim3(BH * n), dim3(kThreads), 0, stream, (const uint16_t*)x, BH, S, block, n,
                           (uint8_t*)codes, scale);
    else
        hipLaunchKernelGGL(quant_kernel<64>, dim3(BH * n), dim3(kThreads), 0, stream, (const uint16_t*)x, BH, S, block, n,
                           (uint8_t*)codes, scale);
    return hipGetLastError();
}

}  // namespace bsa
