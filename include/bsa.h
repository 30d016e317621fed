/*
 * bsa.h -- C ABI of libbsa: dynamic block-sparse self-attention on AMD Instinct MI355X
 * (gfx950).
 *
 * The method, as the pages describe it:
 *   [KC] "知识卡片：600倍加速，720p视频实时生成！单卡也能带的动14B模型"
 *        (ai.cheesepanini.fun knowledge card), section 方法/产品要点, item
 *        动态稀疏量化注意力: the block-level means of Query and Key give a quick estimate
 *        of which attention blocks matter; at run time only the activated key blocks
 *        are computed; typical sparsity is 80-90 % (about 10-20 % of the blocks kept);
 *        the sparse path is combined with SageAttention2 into an FP8 path.
 *   [AO] "单卡 RTX 5090 跑 Wan2.2-A14B：720p 视频生成只要 3.8 秒" (aoyii.com), section
 *        四步拆解, step 3 动态稀疏注意力: the same, and inside the selected blocks the
 *        computation stays dense, to keep the GPU's throughput.
 *
 * The calls follow that split: bsa_select() estimates importance from block means and
 * returns the kept key-block lists; bsa_forward() computes attention over only those
 * blocks. bsa_quantize_fp8() and bsa_forward_fp8() are the FP8 path (E4M3 Q and K);
 * bsa_select_quantize(), bsa_quantize_v_fp8() and bsa_forward_fp8_full() are the full FP8
 * path (E4M3 Q, K, V and softmax weights).
 *
 * Conventions shared by every call:
 *   - Tensors are contiguous [B, H, S, D] row-major (D fastest); q, k, v and out hold
 *     bf16, x_e4m3 holds OCP E4M3FN bytes. Every tensor base address is device memory
 *     aligned to 16 bytes.
 *   - Token block i of a sequence is tokens [i*block, min(S, (i+1)*block)); there are
 *     n = ceil(S/block) blocks, the last possibly partial. Query and key blocks are the
 *     same partition.
 *   - Supported: D in {64, 128}; block in {64, 128}; S >= 1; B, H >= 1; B*H*S*D < 2^40;
 *     ceil(S/block)*block*D*2 < 2^31 (one (b, h) slice); n <= 8192 for bsa_select and
 *     bsa_select_quantize. Other shapes return BSA_ERR_UNSUPPORTED.
 *   - Kept-block lists are CSR over the B*H*n query-block rows, row r = (b*H + h)*n + i:
 *     row_ptr int32 [B*H*n + 1], col_idx int32 [row_ptr[B*H*n]]; each row's key-block
 *     indices are strictly ascending in [0, n).
 *   - Ownership: the caller allocates and frees every buffer (inputs, outputs,
 *     workspace). The library never allocates device memory, never frees, and never
 *     synchronises; it keeps only a per-device table of properties.
 *   - Streams: every compute call is enqueued on hip_stream (a hipStream_t; NULL is the
 *     null stream) and returns before the GPU finishes. No output's byte range may overlap
 *     an input's or another output's (also checked: such a call returns
 *     BSA_ERR_INVALID_ARGUMENT); inputs may overlap each other.
 *     A call only launches kernels (no memset, no copy, no synchronisation), so a sequence
 *     of calls can be captured into a HIP graph and replayed; selection with more than
 *     3968 blocks per sequence (D = 128; 4032 for D = 64) also raises the scoring kernel's
 *     dynamic LDS limit on its first use, so make one such call before capturing; so do
 *     bsa_norm_rope with means and bsa_norm_rope_select when H*D > 4096.
 *   - Errors: arguments are checked on the host before any HIP call, so a bad argument
 *     returns an error without touching the GPU and without side effects. Faults on the
 *     device surface at the caller's next synchronisation. No C++ exception crosses this
 *     interface. bsa_last_error() gives a thread-local message for the last failure.
 *
 * Thread safety: calls may come from several host threads; calls that share output
 * buffers on overlapping streams race like any other GPU work.
 */
#ifndef BSA_H_
#define BSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum bsa_status {
    BSA_OK = 0,
    BSA_ERR_INVALID_ARGUMENT = 1,   /* null pointer, bad size, misaligned, bad ratio     */
    BSA_ERR_UNSUPPORTED = 2,        /* shape outside the supported set, or not gfx950   */
    BSA_ERR_WORKSPACE_TOO_SMALL = 3,
    BSA_ERR_NO_DEVICE = 4,          /* no HIP device visible                             */
    BSA_ERR_HIP = 5                 /* a HIP runtime call failed (message in last_error) */
} bsa_status;

/* Number of token blocks, ceil(S / block); 0 when S < 1 or block < 1. Host only. */
int32_t bsa_num_blocks(int32_t S, int32_t block);

/* Kept key blocks per query block for a keep ratio r in (0, 1]: [KC] keeps about
 * 10-20 % of the blocks; this library rounds r*n up (with a 1e-6 guard against binary
 * representation error, evaluated in double) and clamps to [1, n]. Returns 0 for
 * n < 1 or r outside (0, 1] (NaN included). Host only. */
int32_t bsa_num_kept(int32_t n_blocks, double keep_ratio);

/* Bytes of device workspace bsa_select needs: the fp32 block means of Q and K,
 * 2 * B*H*n*D * 4, rounded up to 256. 0 on invalid shape. Host only. */
size_t bsa_select_workspace_bytes(int32_t B, int32_t H, int32_t S, int32_t D, int32_t block);

/* Block means ([KC] 动态稀疏量化注意力, importance estimated from block-level means): xbar[b,h,i,:] = the mean of x over
 * the valid tokens of block i, accumulated in fp32. x: bf16 [B,H,S,D] (device).
 * xbar: fp32 [B,H,n,D] (device, caller-allocated). Exposed for parity checks; bsa_select
 * computes the same means internally. */
bsa_status bsa_pool(const void* x, int32_t B, int32_t H, int32_t S, int32_t D, int32_t block,
                    float* xbar, void* hip_stream);

/* Importance estimate and block selection ([KC] 动态稀疏量化注意力; [AO] 动态稀疏注意力).
 * For every (b, h) and query block i: score s_ij = mean(Q_i) . mean(K_j) / sqrt(D) in
 * fp32 for every key block j; keep the k = bsa_num_kept(n, keep_ratio) blocks with the
 * highest scores (equal scores: the lower index first); write them ascending.
 *   q, k:      bf16 [B,H,S,D] (device).
 *   row_ptr:   int32 [B*H*n + 1] (device); written as row_ptr[r] = r*k.
 *   col_idx:   int32 [B*H*n*k] (device).
 *   workspace: device scratch of at least bsa_select_workspace_bytes(); contents on
 *              return are the pooled means (undefined layout).
 * Errors: INVALID_ARGUMENT (null/misaligned pointer, keep_ratio not in (0,1]),
 * UNSUPPORTED, WORKSPACE_TOO_SMALL, NO_DEVICE, HIP. */
bsa_status bsa_select(const void* q, const void* k, int32_t B, int32_t H, int32_t S, int32_t D,
                      int32_t block, double keep_ratio, int32_t* row_ptr, int32_t* col_idx,
                      void* workspace, size_t workspace_bytes, void* hip_stream);

/* bsa_select without a workspace argument, for callers that cannot allocate device memory
 * at call time: code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation. Same arguments, results and errors as bsa_select, except that the block means
 * go to a scratch array inside the library: one per device, bsa_select_noalloc_max_bytes()
 * = 64 MiB, held by each device the library runs on until the process ends (found once per
 * device on its first call). The call allocates nothing. Shapes whose means need more than
 * that (bsa_select_workspace_bytes() > bsa_select_noalloc_max_bytes(), i.e. B*H*n*D >
 * 8 Mi) return BSA_ERR_UNSUPPORTED. Every call on a device shares its scratch array, so
 * calls on one device whose executions overlap (different streams, several threads) race;
 * nothing in the array needs to start at zero. */
size_t bsa_select_noalloc_max_bytes(void);
bsa_status bsa_select_noalloc(const void* q, const void* k, int32_t B, int32_t H, int32_t S,
                              int32_t D, int32_t block, double keep_ratio, int32_t* row_ptr,
                              int32_t* col_idx, void* hip_stream);

/* Sparse attention over the kept blocks ([KC] 动态稀疏量化注意力: only the activated key
 * blocks are computed; [AO] 动态稀疏注意力: dense inside each selected block). For query
 * token t of block i: out_t = sum_u softmax_u(q_t . k_u / sqrt(D)) v_u over the valid
 * tokens u of the blocks listed in row (b*H+h)*n + i. No causal mask. Blocks not listed
 * contribute nothing; a row with an empty list gives zeros. Logits, softmax and
 * accumulation are fp32, both products run on bf16 MFMA, out is rounded to bf16.
 *   q, k, v: bf16 [B,H,S,D] (device).   out: bf16 [B,H,S,D] (device).
 *   row_ptr, col_idx: any CSR as described above (device), e.g. bsa_select's output.
 *   Entries outside [0, n) are skipped; a row whose end precedes its start is empty.
 *   The CSR arrays themselves must be as long as row_ptr says. */
bsa_status bsa_forward(const void* q, const void* k, const void* v, int32_t B, int32_t H,
                       int32_t S, int32_t D, int32_t block, const int32_t* row_ptr,
                       const int32_t* col_idx, void* out, void* hip_stream);

/* FP8 quantisation for the FP8 path ([KC] 动态稀疏量化注意力: SageAttention2 FP8 sparse
 * attention). Per (b, h, token block): scale = absmax / 448 in fp32 (1 when the block is
 * all zeros); code = x / scale (IEEE fp32 division) rounded to the nearest OCP E4M3FN
 * value, ties to even.
 *   x: bf16 [B,H,S,D] (device). x_e4m3: uint8 [B,H,S,D] (device). scale: fp32 [B,H,n]. */
bsa_status bsa_quantize_fp8(const void* x, int32_t B, int32_t H, int32_t S, int32_t D,
                            int32_t block, void* x_e4m3, float* scale, void* hip_stream);

/* bsa_forward with Q and K given as E4M3FN codes plus per-block scales (from
 * bsa_quantize_fp8, with the same block size): q.k^T runs on fp8 MFMA with fp32
 * accumulation and the two block scales folded into the logit scale; the softmax is
 * fp32; P and V are bf16 on bf16 MFMA; out is bf16. Same CSR rules as bsa_forward. */
bsa_status bsa_forward_fp8(const void* q_e4m3, const float* q_scale, const void* k_e4m3,
                           const float* k_scale, const void* v, int32_t B, int32_t H, int32_t S,
                           int32_t D, int32_t block, const int32_t* row_ptr,
                           const int32_t* col_idx, void* out, void* hip_stream);

/* ---- Full FP8 path --------------------------------------------------------------------
 * Source: the same pages, section 动态稀疏量化注意力 / step 3: the sparse path joined with
 * SageAttention2 into an FP8 attention path. The pages give none of its steps; this is
 * the library's reading of them:
 *   - Q and K: OCP E4M3FN per (b*h, token block), scale = absmax/448 in fp32 (1 for an
 *     all-zero block), code = nearest E4M3 (ties to even) to x/scale in fp32; the same
 *     codes and scales as bsa_quantize_fp8.
 *   - V: E4M3FN per (b*h, channel d) over the whole sequence, same scale and rounding rule.
 *   - Softmax: online over the kept keys in list order, 64 keys at a time; after a 64-key
 *     sub-tile raises the running maximum m of the log2-domain logits x, its weights
 *     2^(x - m) <= 1 are stored as E4M3 codes of 448 * weight; the output is the sum of
 *     stored weight x dequantised V divided by the sum of the stored weights, in bf16.
 */

/* Bytes of the transposed V codes for bsa_quantize_v_fp8: B*H*D*ceil(S/block)*block; 0 on
 * bad input. */
size_t bsa_vt_fp8_bytes(int32_t B, int32_t H, int32_t S, int32_t D, int32_t block);

/* bsa_select (same lists, bit for bit) and, from the same single read of every Q and K
 * block, their E4M3 codes and per-block scales (the bytes bsa_quantize_fp8 writes).
 *   q_e4m3, k_e4m3: uint8 [B, H, S, D] (16-byte aligned); q_scale, k_scale: fp32 [B*H*n].
 *   workspace: as for bsa_select (bsa_select_workspace_bytes). */
bsa_status bsa_select_quantize(const void* q, const void* k, int32_t B, int32_t H, int32_t S,
                               int32_t D, int32_t block, double keep_ratio, int32_t* row_ptr,
                               int32_t* col_idx, void* q_e4m3, float* q_scale, void* k_e4m3,
                               float* k_scale, void* workspace, size_t workspace_bytes,
                               void* hip_stream);

/* V (bf16 [B, H, S, D]) to per-channel E4M3 codes and scales.
 *   vt_e4m3: uint8 [B*H, D, S_pad] with S_pad = ceil(S/block)*block (bsa_vt_fp8_bytes);
 *     row (b*h, d) holds the codes of channel d over the sequence, zero past S, and inside
 *     every group of 64 keys key r = 32*kh + 8*(v/4) + 4*g + v%4 (kh, g in {0,1}, v < 16)
 *     sits at position 32*g + 16*kh + v. This layout is the operand order of the attention
 *     kernel; it is only meant as the input of bsa_forward_fp8_full with the same block.
 *   v_scale: fp32 [B*H, D], 16-byte aligned; used as scratch (channel maxima) until the
 *     call's last kernel writes the scales.
 *   The call runs four kernels on hip_stream (clear, channel maxima, codes, scales). */
bsa_status bsa_quantize_v_fp8(const void* v, int32_t B, int32_t H, int32_t S, int32_t D,
                              int32_t block, void* vt_e4m3, float* v_scale, void* hip_stream);

/* Attention over the kept blocks with E4M3 Q, K (from bsa_select_quantize or
 * bsa_quantize_fp8), V (from bsa_quantize_v_fp8 with the same block) and E4M3 softmax
 * weights as described above; both products run on fp8 MFMA with fp32 accumulation; out
 * is bf16 [B, H, S, D]. Same CSR rules as bsa_forward. */
bsa_status bsa_forward_fp8_full(const void* q_e4m3, const float* q_scale, const void* k_e4m3,
                                const float* k_scale, const void* vt_e4m3, const float* v_scale,
                                int32_t B, int32_t H, int32_t S, int32_t D, int32_t block,
                                const int32_t* row_ptr, const int32_t* col_idx, void* out,
                                void* hip_stream);

/* ---- Fused RMSNorm + 3D RoPE + block means ------------------------------------------------
 * Source: [KC] section 方法/产品要点, item 高效推理算子, and [AO] section 四步拆解, step 4:
 * 3D RoPE and RMSNorm run as fused kernels, to save temporaries and memory round trips. The
 * pages give no formula; this library defines the operation as follows (the oracle's
 * definition too). For a Q or K projection x (bf16 [B, S, H*D], token-major, as a linear
 * layer writes it) and RMSNorm weights w (bf16 [H*D]):
 *   z[b,s,c]   = x[b,s,c] / sqrt(mean over c' of x[b,s,c']^2 + eps) * w[c]   (all H*D channels)
 *   out[b,h,s] = the D channels z[b,s,h*D .. h*D+D) with each adjacent pair (2i, 2i+1) of
 *                three contiguous segments -- frame, height, width axes, of D - 4*floor(D/6),
 *                2*floor(D/6) and 2*floor(D/6) channels -- turned by p * theta^(-2i/Da)
 *                radians, (u, v) -> (u cos - v sin, u sin + v cos), where p is the token's
 *                coordinate on that axis and Da the segment size; token s of the latent grid
 *                (grid_t, grid_h, grid_w) is at (s / (grid_h*grid_w), (s / grid_w) % grid_h,
 *                s % grid_w);
 * computed in fp32 (rotation angles reduced in fp64) and rounded once to bf16; out is
 * head-major [B, H, S, D], the layout bsa_forward takes. The block means are the means of the
 * written bf16 values (what bsa_pool(out) gives, up to fp32 summation order), fp32 sums in a
 * fixed order. Supported: the shapes above with H*D <= 8192 and grid_t*grid_h*grid_w == S. */

/* Bytes of device workspace for bsa_norm_rope with means: fp32 partial sums,
 * B * ceil(S/32) * H*D * 4, rounded up to 256. 0 on invalid shape. Host only. */
size_t bsa_norm_rope_workspace_bytes(int32_t B, int32_t H, int32_t S, int32_t D);

/* One projection: out = RMSNorm + 3D RoPE of x, head-major, and (if xbar is not NULL) its
 * block means.
 *   x: bf16 [B, S, H*D] (device).   weight: bf16 [H*D] (device).
 *   eps >= 0 and theta > 0 (finite); the usual values are 1e-6 and 10000.
 *   out: bf16 [B, H, S, D] (device); must not overlap x or weight.
 *   xbar: fp32 [B, H, n, D] (device) or NULL; workspace: at least
 *   bsa_norm_rope_workspace_bytes() when xbar is not NULL (ignored otherwise).
 * Pointers x, weight, out and workspace 16-byte aligned, xbar 4-byte aligned.
 * Errors: INVALID_ARGUMENT (null/misaligned pointer, overlap, grid product != S, bad eps
 * or theta), UNSUPPORTED (shape, H*D > 8192), WORKSPACE_TOO_SMALL, NO_DEVICE, HIP. */
bsa_status bsa_norm_rope(const void* x, const void* weight, int32_t B, int32_t H, int32_t S,
                         int32_t D, int32_t block, int32_t grid_t, int32_t grid_h, int32_t grid_w,
                         double eps, double theta, void* out, float* xbar, void* workspace,
                         size_t workspace_bytes, void* hip_stream);

/* Bytes of device workspace bsa_norm_rope_select needs: two sets of partial sums and the
 * fp32 block means of Q and K, rounded up to 256. 0 on invalid shape. Host only. */
size_t bsa_norm_rope_select_workspace_bytes(int32_t B, int32_t H, int32_t S, int32_t D, int32_t block);

/* Both projections and the selection from one read of each: q_out and k_out as
 * bsa_norm_rope writes them (xq with wq, xk with wk), and the kept-block lists that
 * bsa_select(q_out, k_out, ...) would give, scored from the fused block means.
 *   xq, xk: bf16 [B, S, H*D]; wq, wk: bf16 [H*D]; q_out, k_out: bf16 [B, H, S, D];
 *   row_ptr, col_idx, keep_ratio: as bsa_select; workspace: at least
 *   bsa_norm_rope_select_workspace_bytes(). All device memory; outputs must not overlap
 *   inputs or each other.
 * Errors: as bsa_norm_rope and bsa_select (n <= 8192). */
bsa_status bsa_norm_rope_select(const void* xq, const void* xk, const void* wq, const void* wk,
                                int32_t B, int32_t H, int32_t S, int32_t D, int32_t block,
                                int32_t grid_t, int32_t grid_h, int32_t grid_w, double eps,
                                double theta, double keep_ratio, void* q_out, void* k_out,
                                int32_t* row_ptr, int32_t* col_idx, void* workspace,
                                size_t workspace_bytes, void* hip_stream);

/* Host-side validator for a CSR held in host memory: row_ptr_host holds row_ptr_len entries and
 * col_idx_host col_idx_len entries (the caller's buffer sizes; nothing past them is read).
 * Checks row_ptr_len == rows + 1, row_ptr[0] == 0, non-decreasing, row_ptr[rows] <= col_idx_len,
 * and every row's indices strictly ascending in [0, n_blocks). Returns BSA_OK or
 * BSA_ERR_INVALID_ARGUMENT with the first violation in bsa_last_error(). */
bsa_status bsa_check_csr(const int32_t* row_ptr_host, int64_t row_ptr_len, const int32_t* col_idx_host,
                         int64_t col_idx_len, int32_t rows, int32_t n_blocks);

/* Static name of a status code. */
const char* bsa_status_string(bsa_status status);

/* Thread-local message describing the last failed call on this thread ("" if none). */
const char* bsa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BSA_H_ */
