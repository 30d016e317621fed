// Sparse attention over kept key blocks for gfx950: bf16, fp8-QK and full fp8 variants.
//
// Method: the knowledge card "600倍加速，720p视频实时生成！单卡也能带的动14B模型", section
// 方法/产品要点, item 动态稀疏量化注意力 (only the activated key blocks are computed; an
// FP8 path), and the aoyii.com article "单卡 RTX 5090 跑 Wan2.2-A14B", section 四步拆解,
// step 3 动态稀疏注意力 (inside each selected block the computation stays dense).
//
// Work decomposition
//   One workgroup per (batch*head, query block); BLK/32 waves, each owning 32 query rows.
//   The workgroup walks its row of the kept-block list in ascending order, 64 keys
//   (a "sub-tile") at a time. K and V sub-tiles are loaded straight from global memory into
//   LDS (buffer loads with the LDS destination), double-buffered: the next sub-tile's loads
//   are issued before the current one is computed from the other stage, and one wait plus
//   one barrier per sub-tile hands the stages over.
//
// Per wave and sub-tile
//   S^T (64 keys x 32 queries) = K . Q^T on 32x32x16 bf16 MFMA (A = K rows from LDS,
//   B = Q rows kept in registers for the whole kernel), or on 32x32x64 fp8 MFMA.
//   In the S^T accumulator layout every lane holds one query column, so the softmax row
//   statistics are lane-local except for one exchange with lane^32.
//   O^T (D x 32 queries) += V^T . P^T on 32x32x16 bf16 MFMA: P^T comes straight from the
//   S^T accumulators (converted to bf16), V^T from row-major V tiles in LDS through the
//   transposing ds_read_b64_tr_b16. The full fp8 mode stores P^T as E4M3 and reads V^T
//   codes from a transposed, key-permuted V (32x32x64 fp8 MFMA).
//   The bf16 and fp8-QK modes run the online softmax in the log2 domain with a lazily raised
//   reference point (see kSumLimit); the full fp8 mode keeps the exact running maximum.
//
// LDS layout: K and V tiles are row-major [64 keys][D], 16-byte chunks XOR-swizzled per row
// so that both the K-operand reads (16 rows, one chunk) and the transposing V reads
// (4 rows, 4 chunks) hit distinct banks. The full fp8 mode runs three waves per SIMD: its
// registers then cannot hold Q, so each wave keeps its 32 E4M3 Q rows in LDS after the stages,
// in the K tile's layout, and reads them back before each sub-tile's S^T MFMAs.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace bsa {
namespace {

constexpr int KT = 64;  // keys per sub-tile

// s_waitcnt immediate for gfx9-family: vmcnt(0), expcnt and lgkmcnt left at their maxima.
constexpr int kWaitVmcnt0 = 0x0F70;

// Lazy rescaling of the online softmax: the reference point of the exponentials is raised
// only when a query row's running sum of weights would leave (0, kSumLimit], so every weight
// stays at most 2^64 and every fp32 accumulator far from overflow, while the sub-tile maximum
// is computed on a row's first sub-tile and almost never after it.
constexpr float kSumLimit = 0x1p64f;

// log2(448): 2^(x - m + log2 448) = 448 * 2^(x - m), the full fp8 path's weight scale.
constexpr float kLog2Of448 = 8.807354922057604f;

// 2^x on the transcendental unit (one v_exp_f32). Results below 2^-126 may flush to zero,
// which is harmless for softmax weights.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

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

// max / sum of a value over lanes l and l^32 (v_permlane32_swap: no LDS round trip). Maxima use
// the IEEE maximum, which compiles to v_maximum3_f32 without the NaN-quieting moves of fmaxf.
__device__ __forceinline__ float pair_max(float x) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

typedef short __attribute__((address_space(3))) lds_i16;
typedef i16x4 __attribute__((address_space(3))) lds_i16x4;

__device__ __forceinline__ i16x4 lds_read_tr(const char* base, int byte_off) {
    lds_i16x4* p = (lds_i16x4*)((lds_i16*)((__attribute__((address_space(3))) char*)base) + (byte_off >> 1));
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(p);
}

// Attention modes: bf16 throughout; E4M3 Q/K with bf16 V; E4M3 Q/K, V and weights.
constexpr int kModeBf16 = 0, kModeFp8QK = 1, kModeFp8Full = 2;

template <int D, int BLK, int MODE>
struct Cfg {
    static constexpr bool FP8 = MODE != kModeBf16;     // Q and K as E4M3
    static constexpr bool PV8 = MODE == kModeFp8Full;  // V (transposed, per channel) and P as E4M3
    static constexpr int NW = BLK / 32;                // waves per workgroup
    static constexpr int NT = NW * 64;                 // threads
    // V tile in LDS: KT keys x D bf16 (row = key), or D channels x KT E4M3 codes (row = channel)
    static constexpr int VROWB = PV8 ? KT : D * 2;     // V row bytes in LDS
    static constexpr int VROWS = PV8 ? D : KT;
    static constexpr int KROWB = FP8 ? D : D * 2;      // K row bytes in LDS
    static constexpr int VCH = VROWB / 16;             // 16-byte chunks per V row
    static constexpr int KCH = KROWB / 16;
    static constexpr int VTILE = VROWS * VROWB;
    static constexpr int KTILE = KT * KROWB;
    static constexpr int STAGE = KTILE + VTILE;
    static constexpr int QSTEPS = FP8 ? D / 64 : D / 16;  // MFMA k-steps of S^T
    // Direct global->LDS loads move 1 KiB per wave instruction ("segment").
    static constexpr int KRPS = 1024 / KROWB, VRPS = 1024 / VROWB;  // rows per segment
    static constexpr int KSEGW = KTILE / 1024 / NW, VSEGW = VTILE / 1024 / NW;  // per wave
    // Waves per SIMD that LDS allows (160 KiB per CU, four SIMDs), at most two (three for the
    // full fp8 mode, below): one for 128-dim 64-token blocks (64 KiB per two-wave workgroup), so
    // those may use 512 registers.
    static constexpr int LDS_WAVES = (160 * 1024 / (2 * STAGE)) * NW / 4;
    // Full fp8 mode: three waves per SIMD where LDS allows them with the E4M3 Q rows moved from
    // registers into LDS (which the register budget of three waves needs).
    static constexpr int QROWS_BYTES = NW * 32 * D;
    static constexpr bool QINLDS = PV8 && (160 * 1024 / (2 * STAGE + QROWS_BYTES)) * NW / 4 >= 3;
    static constexpr int QLDS = QINLDS ? QROWS_BYTES : 0;
    static constexpr int WAVES_PER_SIMD = QINLDS ? 3 : (LDS_WAVES >= 2 ? 2 : 1);
};

typedef __attribute__((address_space(3))) void* lds_void_ptr;

// One 16-byte direct buffer->LDS load per lane; the wave writes the 1 KiB at lds_dst
// (wave-uniform) with lane l's data at lds_dst + 16*l. The source is the buffer's base +
// soff (wave-uniform, a scalar register) + voff (per lane), so a tile's position costs no
// per-lane address arithmetic.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff, void* lds_dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_ptr)lds_dst, 16, voff, soff, 0, 0);
}

// Raw buffer resource over `bytes` bytes at `base` (word 3: gfx9 default data format).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

template <int D, int BLK, int MODE>
__global__ void __launch_bounds__(BLK * 2) __attribute__((amdgpu_waves_per_eu(Cfg<D, BLK, MODE>::WAVES_PER_SIMD, Cfg<D, BLK, MODE>::WAVES_PER_SIMD > 2 ? Cfg<D, BLK, MODE>::WAVES_PER_SIMD : 2)))
attn_kernel(const AttnArgs a) {
    using C = Cfg<D, BLK, MODE>;
    constexpr bool FP8 = C::FP8, PV8 = C::PV8;
    static_assert(C::KSEGW >= 1 && C::VSEGW >= 1, "tile too small for the workgroup");
    __shared__ __attribute__((aligned(1024))) char lds[2 * C::STAGE + C::QLDS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS targets stay scalar
    const int h = lane >> 5, l32 = lane & 31;
    const int S = a.S, n = a.n;

    const int row = xcd_remap(blockIdx.x, gridDim.x);  // (b*H + h) * n + i
    const int bh = row / n, iq = row - bh * n;
    const int64_t bh_off = (int64_t)bh * S;  // token offset of this (b, h)
    const __amdgpu_buffer_rsrc_t krsrc = buffer_rsrc((const char*)a.k + bh_off * C::KROWB, (uint32_t)S * C::KROWB);
    // V: bf16 rows of this (b, h), or its D channel rows of S_pad E4M3 codes
    const __amdgpu_buffer_rsrc_t vrsrc =
        PV8 ? buffer_rsrc((const char*)a.v + (int64_t)bh * D * a.S_pad, (uint32_t)D * a.S_pad)
            : buffer_rsrc((const char*)a.v + bh_off * C::VROWB, (uint32_t)S * C::VROWB);

    // ---- Q operand (B of S^T = K Q^T), kept in registers --------------------------------
    const int q_tok = iq * BLK + wave * 32 + l32;
    const int q_ld = q_tok < S ? q_tok : S - 1;
    typedef typename std::conditional<FP8, i32x8, bf16x8>::type frag_t;
    frag_t qf[C::QSTEPS];
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
    // Retire the Q loads here, on every path: otherwise the wait-count analysis can carry
    // them as pending into the main loop, where an in-order vmcnt wait for them would also
    // wait for the next sub-tile's prefetch and serialise the pipeline.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    float qscale_log2 = a.sm_scale_log2;
    if constexpr (FP8) qscale_log2 *= a.q_scale[row];

    // ---- kept-block list ----------------------------------------------------------------
    // The row's list is read through a 64-entry window held one entry per lane (and, for the
    // fp8 path, the matching key-block scales); entries are fetched with readlane, so the
    // walk needs no memory access except one window load per 64 blocks.
    int p = a.row_ptr[row];
    int pend = a.row_ptr[row + 1];
    if (pend < p) pend = p;
    int wbase = p, win = -1;
    float kswin = 0.0f;
    auto load_window = [&](int base) {
        wbase = base;
        const int idx = base + lane;
        win = idx < pend ? a.col_idx[idx] : -1;
        if constexpr (FP8) kswin = (win >= 0 && win < n) ? a.k_scale[(int64_t)bh * n + win] : 0.0f;
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    };
    load_window(p);
    auto entry = [&](int idx) -> int {  // col_idx[idx], idx < pend
        if (idx - wbase >= 64) load_window(idx);
        return __builtin_amdgcn_readlane(win, idx - wbase);
    };
    auto entry_kscale = [&](int idx) -> float {  // k_scale of entry idx (window is current)
        return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, kswin), idx - wbase));
    };
    auto valid_block = [&](int idx) -> int {  // next position >= idx holding a block in [0,n)
        while (idx < pend) {
            int j = entry(idx);
            if (j >= 0 && j < n) return idx;
            ++idx;
        }
        return pend;
    };
    // ---- direct global->LDS tile loads ------------------------------------------------
    // Segment sg of a tile holds rows [sg*RPS, (sg+1)*RPS); lane l fills slot l % CH of row
    // sg*RPS + l / CH, i.e. it fetches chunk (slot ^ swz(row)) of that row, so the tile
    // lands swizzled. Wave w fills segments w, w + NW, ...
    uint32_t k_src[C::KSEGW], v_src[C::VSEGW];
#pragma unroll
    for (int x = 0; x < C::KSEGW; ++x) {
        const int r = (x * C::NW + wave) * C::KRPS + lane / C::KCH;
        k_src[x] = r * C::KROWB + 16 * swz<C::KCH>(r, lane % C::KCH);
    }
#pragma unroll
    for (int x = 0; x < C::VSEGW; ++x) {
        const int r = (x * C::NW + wave) * C::VRPS + lane / C::VCH;
        if constexpr (PV8)  // channel row r: 64 codes at r * S_pad in the buffer
            v_src[x] = r * a.S_pad + 16 * ((lane % C::VCH) ^ ((r >> 2) & 3));
        else
            v_src[x] = r * C::VROWB + 16 * swz<C::VCH>(r, lane % C::VCH);
    }
    // Loads the sub-tile of nk keys (1 <= nk <= KT) starting at key0. Rows past the end of
    // the sequence re-read its last row; their scores are masked. (The E4M3 V channel rows
    // are zero padded to whole blocks and never need clamping.) The LDS destination of
    // segment x is wave-uniform, stage + (x*NW + wave) KiB. With many segments per wave it is
    // formed per load from one opaque scalar, so that the compiler does not keep every
    // stage/segment combination live in scalar registers (and spill them).
    auto issue_tile = [&](int key0, int nk, char* stage_base) {
        const uint32_t ko = (uint32_t)key0 * C::KROWB;
        const uint32_t vo = PV8 ? (uint32_t)key0 : (uint32_t)key0 * C::VROWB;
        const int last = nk - 1;
        uint32_t dst = (uint32_t)(stage_base - lds) + wave * 1024;
        if constexpr (C::KSEGW + C::VSEGW > 8) asm volatile("" : "+s"(dst));
        // LDS destination of segment x of the tile at byte offset toff within the stage
        auto seg = [&](int toff, int x) -> char* {
            if constexpr (C::KSEGW + C::VSEGW > 8) return lds + dst + toff + x * C::NW * 1024;
            else return stage_base + toff + (x * C::NW + wave) * 1024;
        };
        if (nk == KT) {
#pragma unroll
            for (int x = 0; x < C::KSEGW; ++x) dma16(krsrc, k_src[x], ko, seg(0, x));
        } else {
#pragma unroll
            for (int x = 0; x < C::KSEGW; ++x) {
                const int r = (x * C::NW + wave) * C::KRPS + lane / C::KCH;
                const int rr = r < last ? r : last;
                dma16(krsrc, k_src[x] - (r - rr) * C::KROWB, ko, seg(0, x));
            }
        }
        if (PV8 || nk == KT) {
#pragma unroll
            for (int x = 0; x < C::VSEGW; ++x) dma16(vrsrc, v_src[x], vo, seg(C::KTILE, x));
        } else {
#pragma unroll
            for (int x = 0; x < C::VSEGW; ++x) {
                const int r = (x * C::NW + wave) * C::VRPS + lane / C::VCH;
                const int rr = r < last ? r : last;
                dma16(vrsrc, v_src[x] - (r - rr) * C::VROWB, vo, seg(C::KTILE, x));
            }
        }
    };

    // ---- per-lane LDS read offsets (kh = 0, m = 0; other halves are constant offsets) ----
    constexpr int KSLOTS = FP8 ? 2 * C::QSTEPS : C::QSTEPS;  // 16-byte K reads per 32 keys
    uint32_t k_rd[KSLOTS];
#pragma unroll
    for (int st = 0; st < KSLOTS; ++st) {
        const int c = FP8 ? (4 * (st >> 1) + 2 * h + (st & 1)) : (2 * st + h);
        k_rd[st] = l32 * C::KROWB + 16 * swz<C::KCH>(l32, c);
    }
    // Full fp8 mode: the wave's 32 E4M3 Q rows go to LDS (in the K tile's swizzled layout, so
    // the K read offsets serve), and are read back before each sub-tile's S^T MFMAs.
    char* const qlds = lds + 2 * C::STAGE + wave * 32 * D;
    if constexpr (C::QINLDS) {
#pragma unroll
        for (int st = 0; st < C::QSTEPS; ++st) {
            const i32x8 v = qf[st];
            *(i32x4*)(qlds + k_rd[2 * st]) = (i32x4){v[0], v[1], v[2], v[3]};
            *(i32x4*)(qlds + k_rd[2 * st + 1]) = (i32x4){v[4], v[5], v[6], v[7]};
        }
    }
    const int gi = lane & 15;
    uint32_t v_rd1[D / 32], v_rd2[D / 32];
    if constexpr (PV8) {
        // A operand of the fp8 PV product: channel row l32 (+32 per ds), the 32 codes of this
        // lane's key half (16-byte chunks 2h and 2h+1 of the row, swizzled by row bits 2..3)
#pragma unroll
        for (int ds = 0; ds < D / 32; ++ds) {
            const int f = (l32 >> 2) & 3;
            v_rd1[ds] = (32 * ds + l32) * C::VROWB + 16 * ((2 * h) ^ f);
            v_rd2[ds] = (32 * ds + l32) * C::VROWB + 16 * ((2 * h + 1) ^ f);
        }
    } else {
#pragma unroll
        for (int ds = 0; ds < D / 32; ++ds) {
            const int dcol = 32 * ds + 16 * ((lane >> 4) & 1) + 4 * (gi & 3);
            const int c = dcol >> 3, coff = (dcol & 7) * 2;
            const int r1 = 4 * h + (gi >> 2), r2 = r1 + 8;
            v_rd1[ds] = r1 * C::VROWB + 16 * swz<C::VCH>(r1, c) + coff;
            v_rd2[ds] = r2 * C::VROWB + 16 * swz<C::VCH>(r2, c) + coff;
        }
    }

    // ---- accumulators and softmax state (per lane: query column l32) -------------------
    f32x16 o[D / 32];
#pragma unroll
    for (int ds = 0; ds < D / 32; ++ds) o[ds] = (f32x16){};
    float m_used = -__builtin_inff();
    float lsum = 0.0f;
    // Full fp8 path: the normaliser is the sum of the stored E4M3 weights, taken by one more
    // MFMA whose A operand has a single row of ones (row 0; lanes 0 and 32): item 0 of lanes
    // 0..31 accumulates sum_k P8[k][query].
    f32x16 lacc = (f32x16){};
    const int one_bits = (PV8 && l32 == 0) ? 0x38383838 : 0;  // E4M3 1.0 = 0x38

    auto compute = [&](const char* kt, int nkeys, float tscale, const char* qsrc) __attribute__((always_inline)) {
        const char* vt = kt + C::KTILE;
        frag_t qv[C::QSTEPS];
#pragma unroll
        for (int st = 0; st < C::QSTEPS; ++st) {
            if constexpr (C::QINLDS) {
                u32x4 lo = *(const u32x4*)(qsrc + k_rd[2 * st]);
                u32x4 hi = *(const u32x4*)(qsrc + k_rd[2 * st + 1]);
                qv[st] = (i32x8){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
            } else {
                qv[st] = qf[st];
            }
        }
        // S^T = K Q^T for the 64 keys (two 32-key halves); A fragments read in a batch.
        f32x16 s[2];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
            frag_t kf[C::QSTEPS];
#pragma unroll
            for (int st = 0; st < C::QSTEPS; ++st) {
                if constexpr (FP8) {
                    u32x4 lo = *(const u32x4*)(kt + 32 * kh * C::KROWB + k_rd[2 * st]);
                    u32x4 hi = *(const u32x4*)(kt + 32 * kh * C::KROWB + k_rd[2 * st + 1]);
                    kf[st] = (i32x8){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                     (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                } else {
                    kf[st] = *(const bf16x8*)(kt + 32 * kh * C::KROWB + k_rd[st]);
                }
            }
            s[kh] = (f32x16){};
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int st = 0; st < C::QSTEPS; ++st) {
                if constexpr (FP8) s[kh] = mfma_fp8(kf[st], qv[st], s[kh]);
                else s[kh] = mfma_bf16(kf[st], qv[st], s[kh]);
            }
            __builtin_amdgcn_s_setprio(0);
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

        if constexpr (PV8) {
            // Exact running maximum (the stored weights must stay <= 1), then the weights
            // times 448 as E4M3 codes, in the byte order of the MFMA operand: byte e of this
            // lane's 32 is key half kh = e / 16, accumulator item e % 16.
            float mx = s[0][0];
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int e = 0; e < 16; ++e) mx = __builtin_elementwise_maximum(mx, s[kh][e]);  // v_maximum3_f32
            mx = pair_max(mx);
            const float mt = mx * tscale;
            if (__any(mt > m_used)) {
                const float m_new = fmaxf(m_used, mt);
                const float alpha = fast_exp2(m_used - m_new);  // 0 on a row's first sub-tile
                m_used = m_new;
                lacc[0] *= alpha;
#pragma unroll
                for (int ds = 0; ds < D / 32; ++ds) o[ds] *= alpha;
            }
            const float off = kLog2Of448 - m_used;
            i32x8 p8;
#pragma unroll
            for (int wd = 0; wd < 8; ++wd) {
                const int e = 4 * wd, kh = e >> 4, v = e & 15;
                int w = 0;
                w = __builtin_amdgcn_cvt_pk_fp8_f32(fast_exp2(__builtin_fmaf(s[kh][v], tscale, off)),
                                                    fast_exp2(__builtin_fmaf(s[kh][v + 1], tscale, off)), w, false);
                w = __builtin_amdgcn_cvt_pk_fp8_f32(fast_exp2(__builtin_fmaf(s[kh][v + 2], tscale, off)),
                                                    fast_exp2(__builtin_fmaf(s[kh][v + 3], tscale, off)), w, true);
                p8[wd] = w;
            }
            int ob = one_bits;  // rebuilt per sub-tile: cheaper than keeping 8 registers live
            asm volatile("" : "+v"(ob));
            const i32x8 ones_v = {ob, ob, ob, ob, ob, ob, ob, ob};
            lacc = mfma_fp8(ones_v, p8, lacc);
#pragma unroll
            for (int ds = 0; ds < D / 32; ++ds) {
                const u32x4 lo = *(const u32x4*)(vt + v_rd1[ds]);
                const u32x4 hi = *(const u32x4*)(vt + v_rd2[ds]);
                const i32x8 vf = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                  (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                o[ds] = mfma_fp8(vf, p8, o[ds]);
            }
            return;
        }

        // Online softmax in the log2 domain. The weights of each 16-key k-step are formed
        // against the running reference point m_used, and the running sum is checked before
        // they enter the PV product: only if it leaves (0, kSumLimit] -- on a row's first
        // sub-tile, where m_used is still -inf, or when scores climb far above m_used -- is
        // the sub-tile's maximum computed and the reference point raised (the accumulators
        // rescaled by the same factor). The result does not depend on the reference point.
        // The row sum takes the fp32 weights with plain adds: a bf16 dot2 would do it in half
        // the instructions, but dot instructions wait behind the other wave's MFMAs on the
        // SIMD, and plain adds do not.
        auto form = [&](int km, bf16x8& pk, float& l) {
            float pw[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                pw[e] = fast_exp2(__builtin_fmaf(s[km >> 1][8 * (km & 1) + e], tscale, -m_used));
                pk[e] = (__bf16)pw[e];
            }
            l += ((pw[0] + pw[1]) + (pw[2] + pw[3])) + ((pw[4] + pw[5]) + (pw[6] + pw[7]));
        };
        auto raise_reference = [&]() {
            float mx = s[0][0];
            // Opaque to the optimiser, so that the maximum below stays on this rare path
            // instead of being merged across call sites and hoisted into the common one.
            asm volatile("" : "+v"(mx));
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kh][e]);
            mx = pair_max(mx);  // lanes l and l^32 hold the two halves of one query column
            const float m_new = fmaxf(m_used, mx * tscale);
            const float alpha = fast_exp2(m_used - m_new);  // 0 on the first sub-tile
            m_used = m_new;
            lsum *= alpha;
#pragma unroll
            for (int ds = 0; ds < D / 32; ++ds) o[ds] *= alpha;
        };
        // O^T += V^T P^T, one 16-key k-step at a time: the weights of k-step km (8 per lane)
        // are formed while the MFMAs of k-step km-1 run, and V^T fragments are read one
        // k-step ahead.
        auto read_v = [&](int km, bf16x8 (&vf)[D / 32]) {
            const int roff = (32 * (km >> 1) + 16 * (km & 1)) * C::VROWB;
#pragma unroll
            for (int ds = 0; ds < D / 32; ++ds) {
                i16x4 lo = lds_read_tr(vt, roff + v_rd1[ds]);
                i16x4 hi = lds_read_tr(vt, roff + v_rd2[ds]);
                i16x4 t8[2] = {lo, hi};
                vf[ds] = *(bf16x8*)t8;
            }
        };
        bf16x8 vcur[D / 32], vnxt[D / 32];
        read_v(0, vcur);
#pragma unroll
        for (int km = 0; km < 4; ++km) {
            bf16x8 pk;
            float lnew = lsum;
            form(km, pk, lnew);
            if (__builtin_expect(__any(!(lnew <= kSumLimit)), 0)) {
                raise_reference();
                lnew = lsum;
                form(km, pk, lnew);
            }
            lsum = lnew;
            if (km < 3) read_v(km + 1, vnxt);
#pragma unroll
            for (int ds = 0; ds < D / 32; ++ds) o[ds] = mfma_bf16(vcur[ds], pk, o[ds]);
            if (km < 3) {
#pragma unroll
                for (int ds = 0; ds < D / 32; ++ds) vcur[ds] = vnxt[ds];
            }
        }
    };

    // ---- main loop: the list a block at a time, two LDS stages ------------------------
    // A 128-token block is two 64-key sub-tiles: the first is computed from stage 0 while the
    // second loads into stage 1, and the second from stage 1 while the next block's first
    // loads into stage 0 (a 64-token block is one sub-tile, and blocks alternate stages).
    // Stage offsets are therefore immediates, and the per-step list work is one lookup.
    auto keys_at = [&](int key0) -> int {  // keys of the sub-tile at key0 (<= 0: none)
        const int r = S - key0;
        return r < KT ? r : KT;
    };
    // Logit scale of list entry pp (window current). The fp8 product of two scales is kept at
    // least FLT_MIN: masked keys are -inf before this scale is applied, and a zero scale (a
    // caller's, or two tiny ones whose product underflows) would turn them into NaN.
    auto block_scale = [&](int pp) -> float {
        if constexpr (FP8) return fmaxf(qscale_log2 * entry_kscale(pp), 0x1p-126f);
        else return qscale_log2;
    };
    int pos = valid_block(p);
    int j = pos < pend ? entry(pos) : -1;
    float ts = j >= 0 ? block_scale(pos) : 0.0f;
    if (j >= 0) issue_tile(j * BLK, keys_at(j * BLK), lds);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    // Advances to the next block in the list (j = -1 at the end).
    auto next_block = [&]() {
        pos = valid_block(pos + 1);
        j = pos < pend ? entry(pos) : -1;
        if (j >= 0) ts = block_scale(pos);
    };
    // One step: start loading `load_nk` keys at load_key0 into `nxt` (if load_nk > 0) and
    // compute the sub-tile in `cur` (if nkeys > 0). The stages are restrict pointers so that,
    // once inlined, the LDS reads and the direct-to-LDS writes carry disjoint alias scopes;
    // without them the wait-count analysis assumes the reads may see the in-flight writes
    // and waits for every load before the first read, which would serialise the pipeline.
    auto step = [&](const char* __restrict__ cur, char* __restrict__ nxt, int nkeys, float tsc,
                    int load_key0, int load_nk, const char* __restrict__ qsrc) __attribute__((always_inline)) {
        if (load_nk > 0) issue_tile(load_key0, load_nk, nxt);
        if (nkeys > 0) compute(cur, nkeys, tsc, qsrc);
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
    };
    if constexpr (BLK == 2 * KT) {
        while (j >= 0) {
            const int key0 = j * BLK;
            const int nk0 = keys_at(key0), nk1 = keys_at(key0 + KT);
            const float tsb = ts;
            step(lds, lds + C::STAGE, nk0, tsb, key0 + KT, nk1, qlds);
            next_block();
            step(lds + C::STAGE, lds, nk1, tsb, j * BLK, j >= 0 ? keys_at(j * BLK) : 0, qlds);
        }
    } else {
        static_assert(BLK == KT, "blocks of one or two sub-tiles");
        while (j >= 0) {
            int nk = keys_at(j * BLK);
            float tsb = ts;
            next_block();
            step(lds, lds + C::STAGE, nk, tsb, j * BLK, j >= 0 ? keys_at(j * BLK) : 0, qlds);
            if (j < 0) break;
            nk = keys_at(j * BLK);
            tsb = ts;
            next_block();
            step(lds + C::STAGE, lds, nk, tsb, j * BLK, j >= 0 ? keys_at(j * BLK) : 0, qlds);
        }
    }

    // ---- normalise and write --------------------------------------------------------
    float ltot;
    if constexpr (PV8) {
        // lanes 0..31 hold the sum of the stored codes (448 x weights); lanes 32..63 take it
        // from their partner
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lacc[0]), __float_as_uint(lacc[0]), false, false);
        ltot = h ? __uint_as_float(sw[0]) : lacc[0];
    } else {
        ltot = pair_sum(lsum);
    }
    const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
    if (q_tok < S) {
        __bf16* op = (__bf16*)a.out + (bh_off + q_tok) * D + 4 * h;
#pragma unroll
        for (int ds = 0; ds < D / 32; ++ds)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 vs = {1.0f, 1.0f, 1.0f, 1.0f};
                if constexpr (PV8) vs = *(const f32x4*)(a.v_scale + (int64_t)bh * D + 32 * ds + 8 * g + 4 * h);
                bf16x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = (__bf16)(o[ds][4 * g + e] * vs[e] * inv);
                *(bf16x4*)(op + 32 * ds + 8 * g) = w;
            }
    }
}

}  // namespace

template <int D, int BLK, int MODE>
static hipError_t launch(const AttnArgs& a, hipStream_t stream) {
    const int grid = a.BH * a.n;
    hipLaunchKernelGGL((attn_kernel<D, BLK, MODE>), dim3(grid), dim3(BLK * 2), 0, stream, a);
    return hipGetLastError();
}

template <int D, int BLK>
static hipError_t launch_mode(const AttnArgs& a, int mode, hipStream_t stream) {
    if (mode == kModeFp8Full) return launch<D, BLK, kModeFp8Full>(a, stream);
    if (mode == kModeFp8QK) return launch<D, BLK, kModeFp8QK>(a, stream);
    return launch<D, BLK, kModeBf16>(a, stream);
}

hipError_t launch_attention(const AttnArgs& a, int D, int block, int mode, hipStream_t stream) {
    if (D == 128 && block == 128) return launch_mode<128, 128>(a, mode, stream);
    if (D == 128 && block == 64) return launch_mode<128, 64>(a, mode, stream);
    if (D == 64 && block == 128) return launch_mode<64, 128>(a, mode, stream);
    if (D == 64 && block == 64) return launch_mode<64, 64>(a, mode, stream);
    return hipErrorInvalidValue;
}

}  // namespace bsa
