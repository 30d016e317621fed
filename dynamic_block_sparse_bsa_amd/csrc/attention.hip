// Sparse attention over kept key blocks, bf16 and fp8-QK variants, for gfx950.
//
// Method: the knowledge card "600倍加速，720p视频实时生成！单卡也能带的动14B模型", section
// 方法/产品要点, item 动态稀疏量化注意力 (only the activated key blocks are computed; an
// FP8 path), and the aoyii.com article "单卡 RTX 5090 跑 Wan2.2-A14B", section 四步拆解,
// step 3 动态稀疏注意力 (inside each selected block the computation stays dense).
//
// Work decomposition
//   One workgroup per (batch*head, query block); BLK/32 waves, each owning 32 query rows.
//   The workgroup walks its row of the kept-block list in ascending order, 64 keys
//   (a "sub-tile") at a time. K and V sub-tiles are staged in LDS, double-buffered: the
//   next sub-tile's global loads are issued into registers before the current one is
//   computed and written to the other LDS stage afterwards, so one barrier per sub-tile
//   suffices.
//
// Per wave and sub-tile
//   S^T (64 keys x 32 queries) = K . Q^T on 32x32x16 bf16 MFMA (A = K rows from LDS,
//   B = Q rows kept in registers for the whole kernel), or on 32x32x64 fp8 MFMA.
//   In the S^T accumulator layout every lane holds one query column, so the softmax row
//   statistics are lane-local except for one exchange with lane^32.
//   O^T (D x 32 queries) += V^T . P^T on 32x32x16 bf16 MFMA: P^T comes straight from the
//   S^T accumulators (converted to bf16), V^T from row-major V tiles in LDS through the
//   transposing ds_read_b64_tr_b16.
//   The online softmax works in the log2 domain with a lazily updated running maximum:
//   the maximum used for the exponent is only raised when a new logit exceeds it by more
//   than 2^8, which keeps every probability below 256 and leaves the result unchanged
//   (numerator and denominator share the same reference point).
//
// LDS layout: K and V tiles are row-major [64 keys][D], 16-byte chunks XOR-swizzled per row
// so that both the K-operand reads (16 rows, one chunk) and the transposing V reads
// (4 rows, 4 chunks) hit distinct banks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace bsa {
namespace {

constexpr int KT = 64;  // keys per sub-tile

// Physical 16-byte slot of chunk c in row r of an LDS tile with `chunks` chunks per row.
template <int chunks>
__device__ __forceinline__ int swz(int r, int c) {
    if constexpr (chunks == 16) return c ^ (((r & 3) << 2) | ((r >> 2) & 3));
    else if constexpr (chunks == 8) return c ^ ((r >> 1) & 7);
    else return c ^ ((r >> 2) & 3);  // 4 chunks per row
}

__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// fp8 E4M3 x fp8 E4M3, 32x32x64, unit block scales (E8M0 127 = 2^0).
__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

typedef short __attribute__((address_space(3))) lds_i16;
typedef i16x4 __attribute__((address_space(3))) lds_i16x4;

__device__ __forceinline__ i16x4 lds_read_tr(const char* base, int byte_off) {
    lds_i16x4* p = (lds_i16x4*)((lds_i16*)((__attribute__((address_space(3))) char*)base) + (byte_off >> 1));
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(p);
}

template <int D, int BLK, bool FP8>
struct Cfg {
    static constexpr int NW = BLK / 32;                // waves per workgroup
    static constexpr int NT = NW * 64;                 // threads
    static constexpr int VROWB = D * 2;                // V row bytes in LDS
    static constexpr int KROWB = FP8 ? D : D * 2;      // K row bytes in LDS
    static constexpr int VCH = VROWB / 16;             // 16-byte chunks per V row
    static constexpr int KCH = KROWB / 16;
    static constexpr int VTILE = KT * VROWB;
    static constexpr int KTILE = KT * KROWB;
    static constexpr int VLOADS = VTILE / (NT * 16);   // 16-byte loads per thread per tile
    static constexpr int KLOADS = KTILE / (NT * 16);
    static constexpr int STAGE = KTILE + VTILE;
    static constexpr int QSTEPS = FP8 ? D / 64 : D / 16;  // MFMA k-steps of S^T
};

template <int D, int BLK, bool FP8>
__global__ void __launch_bounds__(BLK * 2) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_kernel(const AttnArgs a) {
    using C = Cfg<D, BLK, FP8>;
    static_assert(C::VLOADS >= 1 && C::KLOADS >= 1, "tile too small for the workgroup");
    __shared__ __attribute__((aligned(1024))) char lds[2 * C::STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int h = lane >> 5, l32 = lane & 31;
    const int S = a.S, n = a.n;

    const int row = xcd_remap(blockIdx.x, gridDim.x);  // (b*H + h) * n + i
    const int bh = row / n, iq = row - bh * n;
    const int64_t bh_off = (int64_t)bh * S;  // token offset of this (b, h)

    // ---- Q operand (B of S^T = K Q^T), kept in registers --------------------------------
    const int q_tok = iq * BLK + wave * 32 + l32;
    const int q_ld = q_tok < S ? q_tok : S - 1;
    typedef typename std::conditional<FP8, i32x8, bf16x8>::type qfrag_t;
    qfrag_t qf[C::QSTEPS];
    if constexpr (FP8) {
        const uint8_t* qp = (const uint8_t*)a.q + (bh_off + q_ld) * D + 32 * h;
#pragma unroll
        for (int s = 0; s < C::QSTEPS; ++s) {
            i32x4 lo = *(const i32x4*)(qp + 64 * s);
            i32x4 hi = *(const i32x4*)(qp + 64 * s + 16);
            qf[s] = (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
    } else {
        const __bf16* qp = (const __bf16*)a.q + (bh_off + q_ld) * D + 8 * h;
#pragma unroll
        for (int s = 0; s < C::QSTEPS; ++s) qf[s] = *(const bf16x8*)(qp + 16 * s);
    }
    float qscale_log2 = a.sm_scale_log2;
    if constexpr (FP8) qscale_log2 *= a.q_scale[row];

    // ---- kept-block list --------------------------------------------------------------
    int p = a.row_ptr[row];
    int pend = a.row_ptr[row + 1];
    if (pend < p) pend = p;
    auto valid_block = [&](int idx) -> int {  // next position >= idx holding a block in [0,n)
        while (idx < pend) {
            int j = a.col_idx[idx];
            if (j >= 0 && j < n) return idx;
            ++idx;
        }
        return pend;
    };
    p = valid_block(p);

    // Sub-tile cursor: (list position, key offset inside the block).
    int cur_p = p, cur_k = 0;
    auto tile_keys = [&](int pp, int kk) -> int {  // valid keys in sub-tile, 0 at the end
        if (pp >= pend) return 0;
        int j = a.col_idx[pp];
        int rem = S - (j * BLK + kk);
        int inblk = BLK - kk;
        int nk = rem < inblk ? rem : inblk;
        return nk < KT ? nk : KT;
    };
    auto advance = [&](int& pp, int& kk) {
        int j = a.col_idx[pp];
        int next = kk + KT;
        if (next < BLK && j * BLK + next < S) { kk = next; return; }
        kk = 0;
        pp = valid_block(pp + 1);
    };

    // ---- staging registers ----------------------------------------------------------
    u32x4 kreg[C::KLOADS], vreg[C::VLOADS];
    auto load_tile = [&](int pp, int kk) {
        const int j = a.col_idx[pp];
        const int key0 = j * BLK + kk;
#pragma unroll
        for (int x = 0; x < C::KLOADS; ++x) {
            int ci = tid + C::NT * x, r = ci / C::KCH, c = ci % C::KCH;
            int key = key0 + r;
            key = key < S ? key : S - 1;
            kreg[x] = *(const u32x4*)((const char*)a.k + (bh_off + key) * C::KROWB + 16 * c);
        }
#pragma unroll
        for (int x = 0; x < C::VLOADS; ++x) {
            int ci = tid + C::NT * x, r = ci / C::VCH, c = ci % C::VCH;
            int key = key0 + r;
            key = key < S ? key : S - 1;
            vreg[x] = *(const u32x4*)((const char*)a.v + (bh_off + key) * C::VROWB + 16 * c);
        }
    };
    auto store_tile = [&](int stage) {
        char* kt = lds + stage * C::STAGE;
        char* vt = kt + C::KTILE;
#pragma unroll
        for (int x = 0; x < C::KLOADS; ++x) {
            int ci = tid + C::NT * x, r = ci / C::KCH, c = ci % C::KCH;
            *(u32x4*)(kt + r * C::KROWB + 16 * swz<C::KCH>(r, c)) = kreg[x];
        }
#pragma unroll
        for (int x = 0; x < C::VLOADS; ++x) {
            int ci = tid + C::NT * x, r = ci / C::VCH, c = ci % C::VCH;
            *(u32x4*)(vt + r * C::VROWB + 16 * swz<C::VCH>(r, c)) = vreg[x];
        }
    };

    // ---- accumulators and softmax state (per lane: query column l32) -------------------
    f32x16 o[D / 32];
#pragma unroll
    for (int ds = 0; ds < D / 32; ++ds) o[ds] = (f32x16){};
    float m_used = -__builtin_inff();
    float lsum = 0.0f;

    int nkeys = tile_keys(cur_p, cur_k);
    if (nkeys > 0) {
        load_tile(cur_p, cur_k);
        store_tile(0);
    }
    __syncthreads();

    int stage = 0;
    while (nkeys > 0) {
        // Prefetch the next sub-tile into registers.
        int nxt_p = cur_p, nxt_k = cur_k;
        advance(nxt_p, nxt_k);
        const int nxt_keys = tile_keys(nxt_p, nxt_k);
        if (nxt_keys > 0) load_tile(nxt_p, nxt_k);

        const char* kt = lds + stage * C::STAGE;
        const char* vt = kt + C::KTILE;
        float tscale = qscale_log2;
        if constexpr (FP8) tscale *= a.k_scale[(int64_t)bh * n + a.col_idx[cur_p]];

        // S^T = K Q^T for the 64 keys (two 32-key halves).
        f32x16 s[2];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
            s[kh] = (f32x16){};
            const int r = 32 * kh + l32;
            const char* krow = kt + r * C::KROWB;
#pragma unroll
            for (int st = 0; st < C::QSTEPS; ++st) {
                if constexpr (FP8) {
                    u32x4 lo = *(const u32x4*)(krow + 16 * swz<C::KCH>(r, 4 * st + 2 * h));
                    u32x4 hi = *(const u32x4*)(krow + 16 * swz<C::KCH>(r, 4 * st + 2 * h + 1));
                    i32x8 af = (i32x8){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                       (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                    s[kh] = mfma_fp8(af, qf[st], s[kh]);
                } else {
                    bf16x8 af = *(const bf16x8*)(krow + 16 * swz<C::KCH>(r, 2 * st + h));
                    s[kh] = mfma_bf16(af, qf[st], s[kh]);
                }
            }
        }

        // Mask keys past the end of the sequence (partial last block only).
        if (nkeys < KT) {
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    int key = 32 * kh + 8 * (e >> 2) + 4 * h + (e & 3);
                    if (key >= nkeys) s[kh][e] = -__builtin_inff();
                }
        }

        // Online softmax, log2 domain.
        float mx = s[0][0];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kh][e]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mt = mx * tscale;
        if (__any(mt > m_used + 8.0f)) {
            const float m_new = fmaxf(m_used, mt);
            const float alpha = (m_new == -__builtin_inff()) ? 1.0f : exp2f(m_used - m_new);
            m_used = m_new;
            lsum *= alpha;
#pragma unroll
            for (int ds = 0; ds < D / 32; ++ds) o[ds] *= alpha;
        }
        bf16x8 pb[2][2];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float pv = exp2f(__builtin_fmaf(s[kh][8 * m + e], tscale, -m_used));
                    lsum += pv;
                    pb[kh][m][e] = (__bf16)pv;
                }

        // O^T += V^T P^T.
        const int gi = lane & 15;
#pragma unroll
        for (int ds = 0; ds < D / 32; ++ds) {
            const int dcol = 32 * ds + 16 * ((lane >> 4) & 1) + 4 * (gi & 3);
            const int c = dcol >> 3, coff = (dcol & 7) * 2;
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const int r1 = 32 * kh + 16 * m + 4 * h + (gi >> 2);
                    const int r2 = r1 + 8;
                    i16x4 lo = lds_read_tr(vt, r1 * C::VROWB + 16 * swz<C::VCH>(r1, c) + coff);
                    i16x4 hi = lds_read_tr(vt, r2 * C::VROWB + 16 * swz<C::VCH>(r2, c) + coff);
                    i16x4 t8[2] = {lo, hi};
                    bf16x8 af = *(bf16x8*)t8;
                    o[ds] = mfma_bf16(af, pb[kh][m], o[ds]);
                }
        }

        if (nxt_keys > 0) store_tile(stage ^ 1);
        __syncthreads();
        stage ^= 1;
        cur_p = nxt_p;
        cur_k = nxt_k;
        nkeys = nxt_keys;
    }

    // ---- normalise and write --------------------------------------------------------
    const float ltot = lsum + __shfl_xor(lsum, 32);
    const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
    if (q_tok < S) {
        __bf16* op = (__bf16*)a.out + (bh_off + q_tok) * D + 4 * h;
#pragma unroll
        for (int ds = 0; ds < D / 32; ++ds)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                bf16x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = (__bf16)(o[ds][4 * g + e] * inv);
                *(bf16x4*)(op + 32 * ds + 8 * g) = w;
            }
    }
}

}  // namespace

template <int D, int BLK, bool FP8>
static hipError_t launch(const AttnArgs& a, hipStream_t stream) {
    const int grid = a.BH * a.n;
    hipLaunchKernelGGL((attn_kernel<D, BLK, FP8>), dim3(grid), dim3(BLK * 2), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, int D, int block, bool fp8, hipStream_t stream) {
    if (D == 128 && block == 128) return fp8 ? launch<128, 128, true>(a, stream) : launch<128, 128, false>(a, stream);
    if (D == 128 && block == 64) return fp8 ? launch<128, 64, true>(a, stream) : launch<128, 64, false>(a, stream);
    if (D == 64 && block == 128) return fp8 ? launch<64, 128, true>(a, stream) : launch<64, 128, false>(a, stream);
    if (D == 64 && block == 64) return fp8 ? launch<64, 64, true>(a, stream) : launch<64, 64, false>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace bsa
