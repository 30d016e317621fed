// Fused RMSNorm + 3D RoPE + head-major transpose + block pooling of a Q or K projection,
// for gfx950.
//
// Method: the knowledge card "600倍加速，720p视频实时生成！单卡也能带的动14B模型", section
// 方法/产品要点, item 高效推理算子, and the aoyii.com article "单卡 RTX 5090 跑
// Wan2.2-A14B", section 四步拆解, step 4 (融合内核): 3D RoPE and RMSNorm run as fused
// kernels, so no temporaries make extra trips through memory. The pages give neither
// formula. The operation computed here, for a projection x [B, S, H*D] (token-major), is
//   y[b, h, s, :] = rotate_s( x[b, s, h*D : (h+1)*D] / sqrt(mean_c x[b, s, c]^2 + eps) * w[h*D : (h+1)*D] )
// where rotate_s turns channel pairs (2i, 2i+1) of three contiguous per-axis segments
// (frame, height, width; D - 4*floor(D/6), 2*floor(D/6), 2*floor(D/6) channels) by the
// token's coordinate on that axis times theta^(-2i/segment), rounded once to bf16 and
// written head-major [B, H, S, D], the layout the attention kernels read. The block means
// of the written bf16 values come out of the same pass, for the block selection.
//
// Work decomposition
//   One workgroup (four waves) per (batch, 32 consecutive tokens); each wave owns one token
//   at a time. A token's H*D channels are 16-byte chunks, lane l holding chunks l, l + 64, ...
//   (one coalesced 1 KiB load per wave instruction). Because 64 is a multiple of the chunks per
//   head (D/8), every chunk of a lane sits at the same channel offset d0 = 8 * (l % (D/8)) of
//   its head, so a lane's four channel pairs, and their rotation frequencies, are fixed for the
//   whole kernel; the four angles of a token are reduced modulo 2 pi in fp64 and turned into
//   sine and cosine once per token.
//   The sum of squares is a wave reduction; the chunks stay in registers between it and the
//   normalise-rotate-round step, so x is read from HBM once and y written once.
//   Each wave adds the rounded values of its tokens into its own fp32 row of H*D sums in LDS
//   (registers could not hold them next to the chunks); at the end the four rows are added
//   in wave order and written as one partial sum per (batch, 32 tokens), and a second small
//   kernel adds a block's partial sums and divides by its token count. The order of every
//   addition is fixed, so the means are the same on every run.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"
#include "kernels.h"

namespace bsa {
namespace {

constexpr int kNrThreads = 256;
constexpr int kNrWaves = kNrThreads / 64;

// Nearest bf16 (ties to even) of two floats, packed low-high (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    bf16x2 p = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, p);
}

template <int D, int NCH>
__global__ void __launch_bounds__(kNrThreads) norm_rope_kernel(const NormRopeArgs a) {
    constexpr int CPH = D / 8;  // 16-byte chunks per head
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int C = a.H * D, nc = C / 8;  // channels and chunks per token
    const int chunks_per_seq = (a.S + kNormRopeTokens - 1) / kNormRopeTokens;
    const int wg = xcd_remap(blockIdx.x, gridDim.x);
    const int b = wg / chunks_per_seq, tc = wg - b * chunks_per_seq;
    const int t0 = tc * kNormRopeTokens;
    const int tcount = min(kNormRopeTokens, a.S - t0);

    // This lane's four channel pairs: axis and rotation frequency (fixed for the kernel).
    const int d0 = 8 * (lane % CPH);
    constexpr int DT = D - 4 * (D / 6), DH = 2 * (D / 6);
    int axis[4];
    double freq[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int c = d0 + 2 * j;
        int ax, i, sz;
        if (c < DT) { ax = 0; i = c / 2; sz = DT; }
        else if (c < DT + DH) { ax = 1; i = (c - DT) / 2; sz = DH; }
        else { ax = 2; i = (c - DT - DH) / 2; sz = DH; }
        axis[j] = ax;
        freq[j] = pow(a.theta, -2.0 * (double)i / (double)sz);
    }

    // this wave's row of block sums in LDS (when the means are wanted)
    extern __shared__ float sums[];  // [kNrWaves][C]
    float* mine = sums + wave * C;
    if (a.partial) {
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            const int ci = 64 * k + lane;
            if (ci < nc) {
                *(f32x4*)(mine + 8 * ci) = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
                *(f32x4*)(mine + 8 * ci + 4) = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
            }
        }
    }

    const float inv_c = 1.0f / (float)C;
    for (int tl = wave; tl < tcount; tl += kNrWaves) {
        const int s = t0 + tl;
        const uint16_t* xr = (const uint16_t*)a.x + ((int64_t)b * a.S + s) * C;
        // The token's chunks, and this lane's RMSNorm weights (the same for every token, read
        // again per token from cache: kept in registers they would halve the occupancy).
        const uint16_t* wr = (const uint16_t*)a.w;
        asm volatile("" : "+s"(wr));
        u32x4 xv[NCH], wv[NCH];
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            const int ci = 64 * k + lane;
            xv[k] = ci < nc ? *(const u32x4*)(xr + 8 * ci) : (u32x4){0, 0, 0, 0};
        }
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            const int ci = 64 * k + lane;
            wv[k] = ci < nc ? *(const u32x4*)(wr + 8 * ci) : (u32x4){0, 0, 0, 0};
        }
        // mean of squares over the token's channels
        float ss = 0.0f;
#pragma unroll
        for (int k = 0; k < NCH; ++k)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float lo = __uint_as_float(xv[k][e] << 16), hi = __uint_as_float(xv[k][e] & 0xFFFF0000u);
                ss = __builtin_fmaf(lo, lo, ss);
                ss = __builtin_fmaf(hi, hi, ss);
            }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
        // Keep the chunks packed until they are used again (two bf16 per register): without
        // this the compiler keeps their widened fp32 values live across the reduction.
#pragma unroll
        for (int k = 0; k < NCH; ++k) asm volatile("" : "+v"(xv[k]));
        const float inv = 1.0f / sqrtf(ss * inv_c + a.eps);

        // rotation of this token's four pairs: angle = coordinate * frequency, reduced to
        // [-pi, pi] in fp64 before the fp32 sine and cosine
        const int gw = a.gw, ghw = a.gh * a.gw;
        const int pos[3] = {s / ghw, (s / gw) % a.gh, s % gw};
        float cs[4], sn[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const double ang = (double)pos[axis[j]] * freq[j];
            const double turns = rint(ang * 0.15915494309189535);  // 1 / (2 pi)
            const float r = (float)__builtin_fma(-turns, 6.283185307179586, ang);
            sincosf(r, &sn[j], &cs[j]);
        }

        // normalise, weight, rotate, round; store head-major and add to the block sums
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            const int ci = 64 * k + lane;
            if (ci >= nc) continue;
            const int head = ci / CPH;
            u32x4 o;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float u = __uint_as_float(xv[k][j] << 16) * inv * __uint_as_float(wv[k][j] << 16);
                const float v = __uint_as_float(xv[k][j] & 0xFFFF0000u) * inv * __uint_as_float(wv[k][j] & 0xFFFF0000u);
                const float r0 = __builtin_fmaf(u, cs[j], -v * sn[j]);
                const float r1 = __builtin_fmaf(u, sn[j], v * cs[j]);
                o[j] = pack_bf16(r0, r1);
            }
            *(u32x4*)((uint16_t*)a.out + (((int64_t)b * a.H + head) * a.S + s) * D + d0) = o;
            if (a.partial) {
                f32x4 s0 = *(f32x4*)(mine + 8 * ci), s1 = *(f32x4*)(mine + 8 * ci + 4);
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    s0[2 * j] += __uint_as_float(o[j] << 16);
                    s0[2 * j + 1] += __uint_as_float(o[j] & 0xFFFF0000u);
                    s1[2 * j] += __uint_as_float(o[j + 2] << 16);
                    s1[2 * j + 1] += __uint_as_float(o[j + 2] & 0xFFFF0000u);
                }
                *(f32x4*)(mine + 8 * ci) = s0;
                *(f32x4*)(mine + 8 * ci + 4) = s1;
            }
        }
    }

    if (!a.partial) return;
    // The four rows, added in wave order, are this workgroup's partial sum.
    __syncthreads();
    float* dst = a.partial + (int64_t)wg * C;
    for (int c = threadIdx.x; c < C; c += kNrThreads) {
        float t = sums[c];
#pragma unroll
        for (int w = 1; w < kNrWaves; ++w) t += sums[w * C + c];
        dst[c] = t;
    }
}

// Block means from the partial sums of kNormRopeTokens-token chunks: one workgroup per
// (batch, block), one thread per channel; written [B, H, n, D] or, transposed, [B, H, D, n].
__global__ void __launch_bounds__(kNrThreads) norm_rope_means_kernel(const float* __restrict__ partial, int B, int H,
                                                                     int S, int D, int block, float* __restrict__ xbar,
                                                                     int transposed) {
    const int n = (S + block - 1) / block;
    const int chunks_per_seq = (S + kNormRopeTokens - 1) / kNormRopeTokens;
    const int b = blockIdx.x / n, i = blockIdx.x - b * n;
    const int c0 = i * (block / kNormRopeTokens);
    const int c1 = min(chunks_per_seq, c0 + block / kNormRopeTokens);
    const int cnt = min(block, S - i * block);
    const int C = H * D;
    for (int c = threadIdx.x; c < C; c += kNrThreads) {
        float s = 0.0f;
        for (int q = c0; q < c1; ++q) s += partial[((int64_t)b * chunks_per_seq + q) * C + c];
        const int h = c / D, d = c - h * D;
        const float m = s / (float)cnt;
        if (transposed) xbar[(((int64_t)b * H + h) * D + d) * n + i] = m;
        else xbar[(((int64_t)b * H + h) * n + i) * D + d] = m;
    }
}

template <int D, int NCH>
hipError_t launch_nr(const NormRopeArgs& a, hipStream_t stream) {
    const int chunks_per_seq = (a.S + kNormRopeTokens - 1) / kNormRopeTokens;
    const size_t lds = a.partial ? (size_t)kNrWaves * a.H * D * sizeof(float) : 0;
    if (lds > 65536) {  // above the default dynamic LDS limit (H*D > 4096)
        hipError_t e = hipFuncSetAttribute((const void*)norm_rope_kernel<D, NCH>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((norm_rope_kernel<D, NCH>), dim3(a.B * chunks_per_seq), dim3(kNrThreads), lds, stream, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_nr_d(const NormRopeArgs& a, hipStream_t stream) {
    const int nch = (a.H * D / 8 + 63) / 64;  // chunks per lane
    if (nch <= 4) return launch_nr<D, 4>(a, stream);
    if (nch <= 8) return launch_nr<D, 8>(a, stream);
    if (nch <= 12) return launch_nr<D, 12>(a, stream);
    return launch_nr<D, 16>(a, stream);
}

}  // namespace

hipError_t launch_norm_rope(const NormRopeArgs& a, int D, hipStream_t stream) {
    if (D == 128) return launch_nr_d<128>(a, stream);
    if (D == 64) return launch_nr_d<64>(a, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_norm_rope_means(const float* partial, int B, int H, int S, int D, int block, float* xbar,
                                  bool transposed, hipStream_t stream) {
    const int n = (S + block - 1) / block;
    hipLaunchKernelGGL(norm_rope_means_kernel, dim3(B * n), dim3(kNrThreads), 0, stream, partial, B, H, S, D, block,
                       xbar, transposed ? 1 : 0);
    return hipGetLastError();
}

}  // namespace bsa
