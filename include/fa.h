/*
 * fa.h -- C ABI of the MI355X (gfx950) fused exact attention: forward and
 * its gradients.
 *
 * The operation is standard scaled dot-product attention computed without
 * writing the N x N score or probability matrices to memory:
 *
 *   S = scale * Q K^T,   P = softmax(S) row-wise (optionally lower-triangular),
 *   O = P V,             LSE_i = log(sum_j exp(S_ij))  over the visible keys j
 *
 * Sources (pages on IO-aware exact attention):
 *   - "为什么Flash Attention能将注意力计算提速数倍而不损失精度", section 标准注意力机制的内存困局:
 *     the three steps S = QK^T, P = softmax(S), O = PV.
 *   - same page, sections 分块计算(Tiling) and 在线Softmax技巧: tiles of Q, K, V
 *     in on-chip memory, running row maximum and exponential sum, only O and
 *     the per-row statistics go back to HBM.
 *   - "FlashAttention的Triton实现：IO-aware注意力机制底层原理", section Triton实现:
 *     one program per block of query rows walking all K/V blocks (the query-
 *     block-outer loop order), fp32 running statistics and accumulator,
 *     probabilities rounded to the V element type before the second product.
 *   - "GPU Kernel 入门：Triton / FlashAttention", section FlashAttention与在线softmax:
 *     the three running statistics m, l, acc and the final acc / l.
 * The per-row statistics are returned as one natural-log logsumexp.
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes.  0 is success; every error is negative. */
#define FA_OK             0
#define FA_ERR_NULL      -1  /* a required pointer is NULL                                  */
#define FA_ERR_SHAPE     -2  /* B, H or N <= 0, or the launch would exceed the grid limit   */
#define FA_ERR_HEAD_DIM  -3  /* d is not 64 or 128                                          */
#define FA_ERR_SCALE     -4  /* scale is not a finite number > 0                            */
#define FA_ERR_ALIGN     -5  /* a bf16 tensor not 16-byte aligned, or an fp32 one not 4-byte  */
#define FA_ERR_LAUNCH    -6  /* the HIP launch reported an error                            */
#define FA_ERR_FLAG      -7  /* causal is not 0 or 1                                        */
#define FA_ERR_ALIAS     -8  /* an output buffer overlaps an input or another output        */
#define FA_ERR_SPLITS    -9  /* n_splits is not between 1 and 64                            */
#define FA_ERR_SCRATCH  -10  /* B*H*N exceeds the library's own workspace (FA_NOALLOC_ROWS) */
#define FA_ERR_DEVICE   -11  /* the current device or the workspace's address is unavailable */

/* Rows (B*H*N) that fa_bwd_noalloc's own workspace holds: 2^21 fp32 values. */
#define FA_NOALLOC_ROWS  (1 << 21)

/*
 * fa_fwd -- enqueue the attention forward on `stream` and return.
 *
 * Arguments (all device pointers, allocated and owned by the caller):
 *   q, k, v  bf16, [B][H][N][d], contiguous: element (b,h,n,c) sits at
 *            ((b*H + h)*N + n)*d + c.  Read only.  16-byte aligned.
 *   o        bf16, same layout as q; fully overwritten (round to nearest even
 *            from the fp32 result).  16-byte aligned.
 *   lse      fp32, [B][H][N]; fully overwritten with the natural-log
 *            logsumexp of row n's scaled, masked scores.  4-byte aligned.
 *   B, H, N  batch, heads, sequence length (queries and keys), each >= 1.
 *            Any N is accepted: a ragged last tile is masked.
 *   d        head dimension, 64 or 128.
 *   scale    multiplier of Q K^T, finite and > 0 (typically 1/sqrt(d)).
 *   causal   0: every query sees every key; 1: query i sees keys j <= i.
 *   stream   HIP stream to enqueue on (0 = the null stream).
 *
 * Behaviour: all argument checks run on the host before any HIP call and
 * return the codes above without touching the device.  The call allocates
 * nothing, keeps no state between calls and is safe to call from several
 * host threads.  It does not synchronise: faults inside the kernel surface at
 * the caller's next synchronisation.  Outputs must not overlap the inputs or
 * each other.  Results are bitwise reproducible run to run (no atomics).
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, int causal, hipStream_t stream);

/* Human-readable name of a status code (static string, never NULL). */
const char* fa_status_str(int status);

/*
 * fa_fwd_tile -- the launch shape fa_fwd uses for (N, d, causal):
 * query rows per workgroup, keys per K/V tile, waves per workgroup and the
 * number of workgroups for B*H heads.  Returns FA_OK or an FA_ERR_* code for
 * arguments fa_fwd would reject (pointers are not checked here).  Host only.
 */
int fa_fwd_tile(int B, int H, int N, int d, int causal,
                int* rows_per_block, int* keys_per_tile, int* waves, long long* blocks);

/*
 * fa_fwd_splitkv -- the forward of fa_fwd with each query block's visible key
 * tiles divided into n_splits contiguous ranges, one workgroup per range,
 * then merged.  For launches whose B*H*ceil(N/256) query blocks leave the
 * GPU's 256 compute units under-filled (few heads, or one GPU's share of
 * heads split over several GPUs), and as the key-range split a sequence-
 * sharded run would use.
 *
 * Source: "为什么Flash Attention能将注意力计算提速数倍而不损失精度", section
 * 在线Softmax技巧: two blocks of one row, each with its own maximum and
 * exponential sum, merge exactly into the row's softmax (l = e^{m1-m} l1 +
 * e^{m2-m} l2, O rescaled by the same factors); the same page's closing
 * section names Flash Decoding.  Here each range s yields O_s (normalised by
 * its own sum) and LSE_s, and LSE = log sum_s exp(LSE_s),
 * O = sum_s exp(LSE_s - LSE) O_s, which is that merge applied n times.
 *
 * Arguments: q, k, v, o, lse, B, H, N, d, scale, causal, stream as for fa_fwd
 * (same results up to fp32 rounding order), and
 *   n_splits  1 .. 64: the key ranges of every query block, or, under the
 *             causal mask when fa_fwd_splitkv_ranges says so, at most: query
 *             block b (of Nb = ceil(N / rows_per_block)) is then cut into
 *             ceil((b + 1) / r) ranges, r = ceil(Nb / n_splits), so that
 *             every range holds about the same number of key tiles.  Ranges
 *             may be empty when a block has fewer key tiles than ranges;
 *             they contribute nothing.  Workspace entries of ranges a block
 *             does not have are neither written nor read.
 *   o_part    fp32 workspace [n_splits][B][H][N][d], 16-byte aligned.
 *   lse_part  fp32 workspace [n_splits][B][H][N], 4-byte aligned.
 * Both workspaces are overwritten; outputs and workspaces must not overlap
 * the inputs or each other.  Two kernels run in order on `stream`; nothing is
 * allocated; results are bitwise reproducible run to run.
 */
int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int N, int d, float scale, int causal, int n_splits,
                   float* o_part, float* lse_part, hipStream_t stream);

/*
 * fa_fwd_splitkv_plan -- a split count for (B, H, N, d, causal) that gives
 * about two rounds of the workgroups the GPU runs at once (one per compute
 * unit at d = 128, two at d = 64; 1 when fa_fwd alone fills two rounds, or
 * when the ranges would hold fewer than 8 key tiles of 64), at most 16, and the
 * workspace bytes fa_fwd_splitkv needs for it.  The count is the one with
 * the smallest time in the model fa_fwd_splitkv_ranges describes, each count
 * with its own range rule; 1 when fa_fwd alone fills two rounds.  Any output pointer may be
 * NULL.  Returns FA_OK or the FA_ERR_* code fa_fwd would return.  Host only.
 */
int fa_fwd_splitkv_plan(int B, int H, int N, int d, int causal, int* n_splits,
                        size_t* o_part_bytes, size_t* lse_part_bytes);

/*
 * fa_fwd_splitkv_ranges -- the range rule fa_fwd_splitkv uses for n_splits:
 * *r_units = 0 when every query block is cut into n_splits ranges, or, under
 * the causal mask, r > 0 when query block b is cut into ceil((b + 1) / r)
 * ranges (r = ceil(blocks per head / n_splits)).  The library takes whichever
 * its model of the launch (list scheduling of the workgroups over the compute
 * units, plus the merge) predicts is faster; the choice depends only on the
 * arguments.  Returns FA_OK or the FA_ERR_* code fa_fwd_splitkv would return
 * for them.  Host only.
 */
int fa_fwd_splitkv_ranges(int B, int H, int N, int d, int causal, int n_splits, int* r_units);

/*
 * fa_fwd_fa1order -- the same forward computed in the other loop order the
 * pages give, kept as an ablation that measures what that order costs:
 * K/V blocks in the outer loop, query blocks in the inner one, so every query
 * block's running output O_i and statistics l_i, m_i go to HBM and back once
 * per K/V block ("为什么Flash Attention能将注意力计算提速数倍而不损失精度",
 * section 分块计算(Tiling), the two-loop pseudocode; "FlashAttention的Triton实现：
 * IO-aware注意力机制底层原理", section FA1 vs FA2).  Not a fast path: one
 * launch per 64-key block, then one that writes O and LSE.
 *
 * Arguments: q, k, v, o, lse, B, H, N, d, scale, causal, stream as for fa_fwd
 * (same results up to fp32 rounding), and the fp32 workspaces
 *   o_acc  [B][H][N][d], 16-byte aligned: the running O_i between blocks;
 *   m, l   [B][H][N], 4-byte aligned: the running statistics.
 * All are overwritten; outputs and workspaces must not overlap the inputs or
 * each other.  Nothing is allocated; results are reproducible run to run.
 */
int fa_fwd_fa1order(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int N, int d, float scale, int causal,
                    float* o_acc, float* m, float* l, hipStream_t stream);

/*
 * fa_bwd -- enqueue the gradients of fa_fwd's output on `stream` and return.
 *
 * Source: "为什么Flash Attention能将注意力计算提速数倍而不损失精度", section
 * 反向传播中的重计算策略: the backward pass recomputes S and P on chip from
 * Q, K, V (and the per-row statistics the forward kept) instead of storing
 * them.  What it returns is the plain gradient of O = softmax(scale Q K^T
 * [mask]) V for an upstream gradient dO:
 *   P = exp(scale Q K^T - LSE) (masked entries 0), dP = dO V^T,
 *   D_i = sum_c dO_ic O_ic, dS = P (dP - D),
 *   dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO.
 *
 * Arguments (all device pointers, allocated and owned by the caller; the
 * [B][H][N][d] / [B][H][N] layouts are those of fa_fwd):
 *   q, k, v   bf16 inputs of the forward.  Read only.  16-byte aligned.
 *   o, lse    the forward's outputs for these q, k, v, scale and causal
 *             (bf16 O, fp32 natural-log LSE).  Read only.
 *   dout      bf16 upstream gradient dO, same layout as o.  Read only.
 *   dq,dk,dv  bf16 gradients, same layout as q; fully overwritten (round to
 *             nearest even from fp32).  16-byte aligned.
 *   delta     fp32 [B][H][N] workspace; overwritten with D = rowsum(dO * O).
 *             4-byte aligned.
 *   B, H, N, d, scale, causal, stream: as for fa_fwd.
 *
 * Behaviour: the host checks of fa_fwd, extended to every pointer; outputs
 * and the workspace must not overlap the inputs or each other.  Two
 * kernels run in order on `stream` (D and dQ, then dK and dV); the call
 * allocates nothing, does not synchronise and is bitwise reproducible run
 * to run (no atomics).
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, void* dq, void* dk, void* dv, float* delta,
           int B, int H, int N, int d, float scale, int causal, hipStream_t stream);

/*
 * fa_bwd_noalloc -- fa_bwd for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The same kernels and results (bitwise equal to fa_bwd's), with
 * the D workspace taken from the library's own device array instead of a
 * `delta` argument.
 *
 * Arguments: those of fa_bwd without delta.
 * Limit: B*H*N <= FA_NOALLOC_ROWS (2^21 rows, 8 MiB of fp32 per GPU),
 * otherwise FA_ERR_SCRATCH and nothing is launched.
 * Device: the kernels run on `stream`, which must belong to the current
 * device.  The first call on a device looks up that device's copy of the
 * array (FA_ERR_DEVICE if that fails) and keeps its address; each GPU holds
 * its copy until the process ends.  The call allocates nothing and calls no
 * allocating routine.
 * Concurrency: every call on one GPU shares that GPU's array, so calls that
 * overlap in time on one GPU (other streams, other host threads) race; order
 * them on one stream or use fa_bwd with a workspace per caller.
 */
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv,
                   int B, int H, int N, int d, float scale, int causal, hipStream_t stream);

/*
 * FP8 forward.  Source: "为什么Flash Attention能将注意力计算提速数倍而不损失精度",
 * section Flash Attention 3 (FP8 low-precision support): the forward on the
 * FP8 matrix units, with incoherent processing to lower the quantisation
 * error.  The page fixes no scheme; these two calls implement this one:
 *   format     OCP FP8 E4M3 (bias 7, largest finite 448, NaN = S.1111.111),
 *              round to nearest even;
 *   scaling    one factor per (batch, head) and tensor: amax = max |y| over
 *              the head (at least 2^-117 unless 0), code = E4M3(y * 448 /
 *              amax), descale = amax / 448;
 *   rotation   optional for Q and K: y = (sigma o x) H with sigma a random
 *              sign diagonal and H the Sylvester-Hadamard matrix (+-1
 *              entries), computed by the fast Walsh-Hadamard butterfly in
 *              fp32; descale then also carries 1/sqrt(d), so the dequantised
 *              rows are the orthonormally rotated ones and Q K^T is kept.
 *   attention  the online softmax of fa_fwd with P, taken against the
 *              running row maximum (P <= 1), rounded to E4M3 before P V; the
 *              running sum adds the unrounded P.
 */

/*
 * fa_quant_fp8 -- quantise a bf16 [B][H][N][d] tensor to E4M3 per head.
 *
 *   x         bf16 input, [B][H][N][d] contiguous, 16-byte aligned.  Read
 *             only.  Values must be finite.
 *   x8        E4M3 codes, same layout (one byte per element), 16-byte
 *             aligned; fully overwritten.
 *   descale   fp32 [B][H], 4-byte aligned; overwritten with each head's
 *             dequantisation factor (0 for an all-zero head, whose codes are
 *             0).  During the call it holds the heads' amax.
 *   B, H, N, d  as for fa_fwd (d = 64 or 128).
 *   rotate    0: y = x; 1: the random-sign Hadamard rotation above (use the
 *             same signs for Q and K, and no rotation for V).
 *   sign_lo, sign_hi  the 128-bit sign mask: sigma_c = -1 where bit c is set
 *             (bit c of sign_lo for c < 64, bit c - 64 of sign_hi otherwise;
 *             bits at or past d are ignored).
 *   stream    HIP stream.
 * Four kernels run in order on `stream`: workgroup maxima (kept in x8 until
 * the codes overwrite them), per-head amax, codes, factors.  No atomics;
 * codes and factors are bitwise reproducible.  Returns FA_OK or FA_ERR_NULL,
 * _SHAPE, _HEAD_DIM, _FLAG (rotate not 0/1), _ALIGN, _ALIAS, _LAUNCH.
 */
int fa_quant_fp8(const void* x, void* x8, float* descale, int B, int H, int N, int d, int rotate,
                 uint64_t sign_lo, uint64_t sign_hi, hipStream_t stream);

/*
 * fa_fwd_fp8 -- attention forward on E4M3 operands (as fa_quant_fp8 makes
 * them), on `stream`.
 *
 *   q8, k8, v8  E4M3 [B][H][N][d], 16-byte aligned.  Read only.
 *   q_descale, k_descale, v_descale  fp32 [B][H] factors, 4-byte aligned:
 *             the operands are descale * value(code).
 *   o         bf16 [B][H][N][d], 16-byte aligned; fully overwritten.
 *   lse       fp32 [B][H][N], 4-byte aligned; natural-log logsumexp of the
 *             scaled, masked scores of the dequantised operands.
 *   B, H, N, d, scale, causal  as for fa_fwd.
 * Same host checks and asynchrony as fa_fwd; outputs must not overlap the
 * inputs or each other; nothing is allocated; results are bitwise
 * reproducible run to run.
 */
int fa_fwd_fp8(const void* q8, const void* k8, const void* v8, const float* q_descale,
               const float* k_descale, const float* v_descale, void* o, float* lse,
               int B, int H, int N, int d, float scale, int causal, hipStream_t stream);

/*
 * fa_fwd_fp8_tile -- the launch shape fa_fwd_fp8 uses: query rows per
 * workgroup, keys per K/V tile, waves per workgroup and the number of
 * workgroups.  Returns FA_OK or the FA_ERR_* code fa_fwd_fp8 would return
 * for these sizes (pointers are not checked here).  Host only.
 */
int fa_fwd_fp8_tile(int B, int H, int N, int d, int causal,
                    int* rows_per_block, int* keys_per_tile, int* waves, long long* blocks);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
