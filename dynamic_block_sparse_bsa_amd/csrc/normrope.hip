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
//   whole kernel. The lanes that share them split the work: each reduces one angle of the
//   token modulo 2 pi in fp64, takes its fp32 sine and cosine, and lane shuffles hand the four
//   results to every lane that needs them.
//   The sum of squares is a wave reduction; the chunks stay in registers between it and the
//   normalise-rotate-round step, so x is read from HBM once and y written once, and the next
//   token's chunks are loaded while the current one is processed.
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

// bf16 pair e of a 16-byte chunk. (The chunk is reinterpreted whole: a bit cast of one
// 32-bit element of the u32x4 to bf16x2 is mistranslated by this compiler, which then reads
// element 0 for every e.)
__device__ __forceinline__ bf16x2 pair_of(const u32x4& chunk, int e) {
    const bf16x8 b = __builtin_bit_cast(bf16x8, chunk);
    return (bf16x2){b[2 * e], b[2 * e + 1]};
}

template <int D, int NCH>
__global__ void __launch_bounds__(kNrThreads) norm_rope_kernel(const NormRopeArgs a) {
    constexpr int CPH = D / 8;  // 16-byte chunks per head
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int C = a.H * D, nc = C / 8;  // channels and chunks per token
    const int chunks_per_seq = (a.S + kNormRopeTokens - 1) / kNormRopeTokens;
    // Workgroups in launch order, not grouped per XCD: the workgroups in flight then cover one
    // contiguous token range, so each head's output rows being written lie in one region
    // (grouping them per XCD, as the attention kernel does for L2 reuse, spreads the writes
    // over eight token ranges per head and made this pass 15 % slower).
    const int wg = blockIdx.x;
    const int b = wg / chunks_per_seq, tc = wg - b * chunks_per_seq;
    const int t0 = tc * kNormRopeTokens;
    const int tcount = min(kNormRopeTokens, a.S - t0);

    // Lanes l, l + CPH, ... share the channel offset d0 and so the four rotations of a token;
    // lane l computes pair (l / CPH) % 4 of them and the others are fetched by lane shuffles.
    const int d0 = 8 * (lane % CPH);
    constexpr int DT = D - 4 * (D / 6), DH = 2 * (D / 6);
    int my_axis;
    double my_freq;
    {
        const int c = d0 + 2 * ((lane / CPH) & 3);
        int i, sz;
        if (c < DT) { my_axis = 0; i = c / 2; sz = DT; }
        else if (c < DT + DH) { my_axis = 1; i = (c - DT) / 2; sz = DH; }
        else { my_axis = 2; i = (c - DT - DH) / 2; sz = DH; }
        my_freq = pow(a.theta, -2.0 * (double)i / (double)sz);
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
    // The token's chunks; lanes past the last chunk load chunk 0 and discard it. The next
    // token's chunks are loaded while this one is processed.
    auto load_token = [&](int tl, u32x4 (&dst)[NCH]) {
        const uint16_t* xr = (const uint16_t*)a.x + ((int64_t)b * a.S + t0 + tl) * C;
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            const int ci = 64 * k + lane < nc ? 64 * k + lane : 0;
            dst[k] = *(const u32x4*)(xr + 8 * ci);
        }
    };
    u32x4 xv[NCH], xn[NCH];
    if (wave < tcount) load_token(wave, xv);
    for (int tl = wave; tl < tcount; tl += kNrWaves) {
        const int s = t0 + tl;
        if (tl + kNrWaves < tcount) load_token(tl + kNrWaves, xn);
        // This lane's RMSNorm weights: the same for every token, read again per token from
        // cache (kept in registers they would cost the occupancy).
        const uint16_t* wr = (const uint16_t*)a.w;
        asm volatile("" : "+s"(wr));
        u32x4 wv[NCH];
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            const int ci = 64 * k + lane < nc ? 64 * k + lane : 0;
            wv[k] = *(const u32x4*)(wr + 8 * ci);
        }
        // the rotation this lane computes: angle = coordinate * frequency, reduced to
        // [-pi, pi] in fp64 before the fp32 sine and cosine
        const int gw = a.gw, ghw = a.gh * a.gw;
        const int p = my_axis == 0 ? s / ghw : my_axis == 1 ? (s / gw) % a.gh : s % gw;
        const double ang = (double)p * my_freq;
        const double turns = rint(ang * 0.15915494309189535);  // 1 / (2 pi)
        float my_sn, my_cs;
        sincosf((float)__builtin_fma(-turns, 6.283185307179586, ang), &my_sn, &my_cs);

        // mean of squares over the token's channels (bf16 pairs: exact products, fp32 sums)
        float ss = 0.0f;
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            if (64 * k + lane >= nc) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bf16x2 x2 = pair_of(xv[k], e);
                ss = __builtin_amdgcn_fdot2_f32_bf16(x2, x2, ss, false);
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
        // Keep the chunks packed until they are used again (two bf16 per register): without
        // this the compiler keeps their widened fp32 values live across the reduction.
#pragma unroll
        for (int k = 0; k < NCH; ++k) asm volatile("" : "+v"(xv[k]));
        const float inv = 1.0f / sqrtf(ss * inv_c + a.eps);
        // the four rotations of this lane's pairs, with the RMS scale folded in
        float cs[4], sn[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int src = (lane % CPH) + CPH * j;
            cs[j] = __shfl(my_cs, src) * inv;
            sn[j] = __shfl(my_sn, src) * inv;
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
                const float u = __uint_as_float(xv[k][j] << 16) * __uint_as_float(wv[k][j] << 16);
                const float v = __uint_as_float(xv[k][j] & 0xFFFF0000u) * __uint_as_float(wv[k][j] & 0xFFFF0000u);
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
        if (tl + kNrWaves < tcount) {
#pragma unroll
            for (int k = 0; k < NCH; ++k) xv[k] = xn[k];
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

// Block means from the partial sums of kNormRopeTokens-token chunks. One workgroup per
// (batch, 64 blocks, 64 channels): the means of that tile are formed with reads along the
// channels, staged in LDS, and written along the channels ([B, H, n, D]) or, transposed,
// along the blocks ([B, H, D, n]), so both layouts are written with whole cache lines.
constexpr int kMeansTile = 64;

__global__ void __launch_bounds__(kNrThreads) norm_rope_means_kernel(const float* __restrict__ partial, int B, int H,
                                                                     int S, int D, int block, float* __restrict__ xbar,
                                                                     int transposed) {
    __shared__ float tile[kMeansTile][kMeansTile + 1];
    const int n = (S + block - 1) / block;
    const int C = H * D;
    const int chunks_per_seq = (S + kNormRopeTokens - 1) / kNormRopeTokens;
    const int per_block = block / kNormRopeTokens;
    const int tiles_i = (n + kMeansTile - 1) / kMeansTile, tiles_c = (C + kMeansTile - 1) / kMeansTile;
    int w = blockIdx.x;
    const int tc = w % tiles_c;
    w /= tiles_c;
    const int ti = w % tiles_i, b = w / tiles_i;
    const int i0 = ti * kMeansTile, c0 = tc * kMeansTile;
    const int col = threadIdx.x % kMeansTile, row0 = threadIdx.x / kMeansTile;
    constexpr int kRowStep = kNrThreads / kMeansTile;
    // means of the tile: thread (row, col) = (block i0 + row, channel c0 + col). All of a
    // thread's loads are issued before any sum (a block has at most kMaxChunksPerBlock
    // partial sums; missing ones read element 0 and are not added).
    constexpr int kRows = kMeansTile / kRowStep, kMaxChunksPerBlock = 128 / kNormRopeTokens;
    const int c = c0 + col;
    float v[kRows][kMaxChunksPerBlock];
#pragma unroll
    for (int rr = 0; rr < kRows; ++rr) {
        const int i = i0 + row0 + rr * kRowStep;
#pragma unroll
        for (int qq = 0; qq < kMaxChunksPerBlock; ++qq) {
            const int q = i * per_block + qq;
            const bool ok = i < n && c < C && qq < per_block && q < chunks_per_seq;
            v[rr][qq] = partial[ok ? ((int64_t)b * chunks_per_seq + q) * C + c : 0];
        }
    }
#pragma unroll
    for (int rr = 0; rr < kRows; ++rr) {
        const int i = i0 + row0 + rr * kRowStep;
        float sum = 0.0f;
#pragma unroll
        for (int qq = 0; qq < kMaxChunksPerBlock; ++qq)
            if (qq < per_block && i * per_block + qq < chunks_per_seq) sum += v[rr][qq];
        tile[row0 + rr * kRowStep][col] = (i < n && c < C) ? sum / (float)min(block, S - i * block) : 0.0f;
    }
    __syncthreads();
    if (transposed) {  // thread (col = block offset, row = channel offset)
        for (int r = row0; r < kMeansTile; r += kRowStep) {
            const int c = c0 + r, i = i0 + col;
            if (c < C && i < n) {
                const int h = c / D, d = c - h * D;
                xbar[(((int64_t)b * H + h) * D + d) * n + i] = tile[col][r];
            }
        }
    } else {
        for (int r = row0; r < kMeansTile; r += kRowStep) {
            const int i = i0 + r, c = c0 + col;
            if (c < C && i < n) {
                const int h = c / D, d = c - h * D;
                xbar[(((int64_t)b * H + h) * n + i) * D + d] = tile[r][col];
            }
        }
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
    switch ((nch + 1) / 2) {
        case 1: return launch_nr<D, 2>(a, stream);
        case 2: return launch_nr<D, 4>(a, stream);
        case 3: return launch_nr<D, 6>(a, stream);
        case 4: return launch_nr<D, 8>(a, stream);
        case 5: return launch_nr<D, 10>(a, stream);
        case 6: return launch_nr<D, 12>(a, stream);
        case 7: return launch_nr<D, 14>(a, stream);
        default: return launch_nr<D, 16>(a, stream);
    }
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
    const int tiles = B * ((n + kMeansTile - 1) / kMeansTile) * ((H * D + kMeansTile - 1) / kMeansTile);
    hipLaunchKernelGGL(norm_rope_means_kernel, dim3(tiles), dim3(kNrThreads), 0, stream, partial, B, H, S, D, block,
                       xbar, transposed ? 1 : 0);
    return hipGetLastError();
}

}  // namespace bsa
