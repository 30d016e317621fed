// Quantisation kernels of the full FP8 path, for gfx950.
//
// Method: the knowledge card "600倍加速，720p视频实时生成！单卡也能带的动14B模型", section
// 方法/产品要点, item 动态稀疏量化注意力 (and the aoyii.com article "单卡 RTX 5090 跑
// Wan2.2-A14B", section 四步拆解, step 3): the block-sparse path is combined with
// SageAttention2 into an FP8 attention path. The pages give none of its steps; this library
// quantises
//   - Q and K per (b*h, token block) to OCP E4M3FN with scale absmax/448, in the same HBM
//     pass that computes the block means for selection (pool_quant_kernel);
//   - V per (b*h, channel) over the whole sequence (vabsmax_kernel, then vquant_kernel).
//
// V codes are written transposed and key-permuted for the attention kernel's PV product:
// vt[(b*h*D + d) * S_pad + key'] with S_pad = n * block (zero padded), where inside every
// group of 64 keys key r sits at position perm64(r) = 32 * h + 16 * kh + v for
// r = 32 * kh + 8 * (v / 4) + 4 * h + v % 4. That is the order in which one lane of the
// QK^T accumulator holds the 32 keys of its half (h = lane / 32), so a lane's 32 weight
// bytes and the 32 V bytes of its output row line up as one fp8 MFMA operand each.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"
#include "kernels.h"

namespace bsa {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Key (0..63) held at position pos (0..63) of a 64-key group of the permuted V layout.
__device__ __forceinline__ int key_at(int pos) {
    const int h = pos >> 5, e = pos & 31, kh = e >> 4, v = e & 15;
    return 32 * kh + 8 * (v >> 2) + 4 * h + (v & 3);
}

// ---- fused block means + E4M3 codes of Q and K ----------------------------------------
// One workgroup per (b*h, block) and tensor (blockIdx.y: 0 = Q, 1 = K). The block is read
// once into registers. Means are summed in exactly the order of the pooling kernel (thread t
// owns chunk t % CH of tokens t / CH, t / CH + TL, ...; then a fixed reduction over TL), so
// they are bit-identical to it and selection picks the same lists; codes and scales follow
// the quantiser's arithmetic (x / scale in fp32, round to nearest even).
template <int D>
__global__ void __launch_bounds__(kThreads) pool_quant_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                              int S, int block, int n, float* __restrict__ qbar,
                                                              float* __restrict__ kbarT, uint8_t* __restrict__ q8,
                                                              uint8_t* __restrict__ k8, float* __restrict__ qscale,
                                                              float* __restrict__ kscale) {
    constexpr int CH = D / 8, TL = kThreads / CH, RPT = 128 / TL;  // rows per thread, blocks <= 128
    __shared__ float red[TL][D + 4];
    __shared__ float wmax[kThreads / 64];
    const int which = blockIdx.y;
    const uint16_t* x = which ? k : q;
    uint8_t* codes = which ? k8 : q8;
    const int rowi = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = rowi / n, i = rowi - bh * n;
    const int t0 = i * block;
    const int cnt = (S - t0) < block ? (S - t0) : block;
    const int c = threadIdx.x % CH, tl = threadIdx.x / CH;
    const int64_t base = ((int64_t)bh * S + t0) * D + 8 * c;
    u32x4 w[RPT];
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    float amax = 0.0f;
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const int t = tl + r * TL;
        if (t < cnt) {
            w[r] = *(const u32x4*)(x + base + (int64_t)t * D);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[2 * e] += lo_bf16(w[r][e]);
                acc[2 * e + 1] += hi_bf16(w[r][e]);
                amax = fmaxf(amax, fmaxf(fabsf(lo_bf16(w[r][e])), fabsf(hi_bf16(w[r][e]))));
            }
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[tl][8 * c + e] = acc[e];
    for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = amax;
    __syncthreads();
    if (threadIdx.x < D) {
        const int d = threadIdx.x;
        float s = 0.0f;
        for (int r = 0; r < TL; ++r) s += red[r][d];
        const float mean = s / (float)cnt;
        if (which) kbarT[((int64_t)bh * D + d) * n + i] = mean;
        else qbar[((int64_t)bh * n + i) * D + d] = mean;
    }
    amax = wmax[0];
#pragma unroll
    for (int wv = 1; wv < kThreads / 64; ++wv) amax = fmaxf(amax, wmax[wv]);
    const float sc = amax > 0.0f ? amax / 448.0f : 1.0f;
    if (threadIdx.x == 0) (which ? kscale : qscale)[rowi] = sc;
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
        const int t = tl + r * TL;
        if (t < cnt) {
            u32x2 packed;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                int v = 0;
                v = __builtin_amdgcn_cvt_pk_fp8_f32(lo_bf16(w[r][2 * e]) / sc, hi_bf16(w[r][2 * e]) / sc, v, false);
                v = __builtin_amdgcn_cvt_pk_fp8_f32(lo_bf16(w[r][2 * e + 1]) / sc, hi_bf16(w[r][2 * e + 1]) / sc, v, true);
                packed[e] = (uint32_t)v;
            }
            *(u32x2*)(codes + base + (int64_t)t * D) = packed;
        }
    }
}

// ---- V: per-channel absmax over the sequence ---------------------------------------------
__global__ void fill_kernel(uint32_t* __restrict__ p, int count, uint32_t value) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count) p[i] = value;
}

// One workgroup per (b*h, block): channel maxima of |v| over the block's tokens, merged into
// amax_bits[b*h, d] with an unsigned max on the bit patterns (non-negative floats order like
// their bits).
template <int D>
__global__ void __launch_bounds__(kThreads) vabsmax_kernel(const uint16_t* __restrict__ v, int S, int block, int n,
                                                           uint32_t* __restrict__ amax_bits) {
    constexpr int CH = D / 8, TL = kThreads / CH;
    __shared__ float red[TL][D + 4];
    const int rowi = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = rowi / n, i = rowi - bh * n;
    const int t0 = i * block;
    const int cnt = (S - t0) < block ? (S - t0) : block;
    const int c = threadIdx.x % CH, tl = threadIdx.x / CH;
    const uint16_t* base = v + ((int64_t)bh * S + t0) * D + 8 * c;
    float m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int t = tl; t < cnt; t += TL) {
        const u32x4 w = *(const u32x4*)(base + (int64_t)t * D);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            m[2 * e] = fmaxf(m[2 * e], fabsf(lo_bf16(w[e])));
            m[2 * e + 1] = fmaxf(m[2 * e + 1], fabsf(hi_bf16(w[e])));
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[tl][8 * c + e] = m[e];
    __syncthreads();
    if (threadIdx.x < D) {
        float mx = 0.0f;
        for (int r = 0; r < TL; ++r) mx = fmaxf(mx, red[r][threadIdx.x]);
        atomicMax(amax_bits + (int64_t)bh * D + threadIdx.x, __float_as_uint(mx));
    }
}

// One workgroup per (b*h, block): codes of the block with the per-channel scales, written
// transposed and key-permuted (see the file comment); tokens past the end are written as 0.
template <int D>
__global__ void __launch_bounds__(kThreads) vquant_kernel(const uint16_t* __restrict__ v, int S, int block, int n,
                                                          const uint32_t* __restrict__ amax_bits, uint8_t* __restrict__ vt) {
    constexpr int CH = D / 8, TL = kThreads / CH;
    constexpr int ROWB = D + 4;  // LDS code tile row (bytes), padded
    __shared__ float sc[D];
    __shared__ uint8_t tile[128 * ROWB];
    const int rowi = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = rowi / n, i = rowi - bh * n;
    const int t0 = i * block;
    const int cnt = (S - t0) < block ? (S - t0) : block;
    const int64_t S_pad = (int64_t)n * block;
    if (threadIdx.x < D) {
        const float amax = __uint_as_float(amax_bits[(int64_t)bh * D + threadIdx.x]);
        sc[threadIdx.x] = amax > 0.0f ? amax / 448.0f : 1.0f;
    }
    __syncthreads();
    const int c = threadIdx.x % CH, tl = threadIdx.x / CH;
    const uint16_t* base = v + ((int64_t)bh * S + t0) * D + 8 * c;
    for (int t = tl; t < cnt; t += TL) {
        const u32x4 w = *(const u32x4*)(base + (int64_t)t * D);
        u32x2 packed;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int d0 = 8 * c + 4 * e;
            int p = 0;
            p = __builtin_amdgcn_cvt_pk_fp8_f32(lo_bf16(w[2 * e]) / sc[d0], hi_bf16(w[2 * e]) / sc[d0 + 1], p, false);
            p = __builtin_amdgcn_cvt_pk_fp8_f32(lo_bf16(w[2 * e + 1]) / sc[d0 + 2], hi_bf16(w[2 * e + 1]) / sc[d0 + 3], p, true);
            packed[e] = (uint32_t)p;
        }
        *(uint32_t*)(tile + t * ROWB + 8 * c) = packed[0];
        *(uint32_t*)(tile + t * ROWB + 8 * c + 4) = packed[1];
    }
    __syncthreads();
    // Output: D rows of `block` bytes; 16-byte pieces, one per thread and pass.
    const int pieces = D * (block / 16);
    for (int pc = threadIdx.x; pc < pieces; pc += kThreads) {
        const int d = pc / (block / 16), p16 = pc - d * (block / 16);
        u32x4 out;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            uint32_t word = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int pos = 16 * p16 + 4 * q4 + b;  // position in this block's segment
                const int t = (pos & ~63) + key_at(pos & 63);
                const uint32_t code = t < cnt ? tile[t * ROWB + d] : 0u;
                word |= code << (8 * b);
            }
            out[q4] = word;
        }
        *(u32x4*)(vt + ((int64_t)bh * D + d) * S_pad + (int64_t)i * block + 16 * p16) = out;
    }
}

// Channel maxima -> scales, in place (same formula as vquant_kernel).
__global__ void vscale_kernel(uint32_t* __restrict__ amax_bits, int count) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count) {
        const float amax = __uint_as_float(amax_bits[i]);
        amax_bits[i] = __float_as_uint(amax > 0.0f ? amax / 448.0f : 1.0f);
    }
}

}  // namespace

hipError_t launch_pool_quant_qk(const void* q, const void* k, int BH, int S, int D, int block, float* qbar, float* kbarT,
                                void* q8, void* k8, float* qscale, float* kscale, hipStream_t stream) {
    const int n = (S + block - 1) / block;
    dim3 grid(BH * n, 2);
    if (D == 128)
        hipLaunchKernelGGL(pool_quant_kernel<128>, grid, dim3(kThreads), 0, stream, (const uint16_t*)q, (const uint16_t*)k,
                           S, block, n, qbar, kbarT, (uint8_t*)q8, (uint8_t*)k8, qscale, kscale);
    else
        hipLaunchKernelGGL(pool_quant_kernel<64>, grid, dim3(kThreads), 0, stream, (const uint16_t*)q, (const uint16_t*)k,
                           S, block, n, qbar, kbarT, (uint8_t*)q8, (uint8_t*)k8, qscale, kscale);
    return hipGetLastError();
}

hipError_t launch_quantize_v(const void* v, int BH, int S, int D, int block, void* vt, float* vscale, hipStream_t stream) {
    const int n = (S + block - 1) / block;
    const int count = BH * D;
    uint32_t* bits = (uint32_t*)vscale;
    hipLaunchKernelGGL(fill_kernel, dim3((count + 255) / 256), dim3(256), 0, stream, bits, count, 0u);
    if (D == 128) {
        hipLaunchKernelGGL(vabsmax_kernel<128>, dim3(BH * n), dim3(kThreads), 0, stream, (const uint16_t*)v, S, block, n, bits);
        hipLaunchKernelGGL(vquant_kernel<128>, dim3(BH * n), dim3(kThreads), 0, stream, (const uint16_t*)v, S, block, n,
                           (const uint32_t*)bits, (uint8_t*)vt);
    } else {
        hipLaunchKernelGGL(vabsmax_kernel<64>, dim3(BH * n), dim3(kThreads), 0, stream, (const uint16_t*)v, S, block, n, bits);
        hipLaunchKernelGGL(vquant_kernel<64>, dim3(BH * n), dim3(kThreads), 0, stream, (const uint16_t*)v, S, block, n,
                           (const uint32_t*)bits, (uint8_t*)vt);
    }
    hipLaunchKernelGGL(vscale_kernel, dim3((count + 255) / 256), dim3(256), 0, stream, bits, count);
    return hipGetLastError();
}

}  // namespace bsa
