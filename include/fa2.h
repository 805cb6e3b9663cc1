/*
 * fa2.h -- C ABI of the MI355X (gfx950) exact-attention forward library.
 *
 * Operation (all entry points):
 *
 *     O[b,h] = softmax(scale * Q[b,h] K[b,h]^T + M) V[b,h]
 *     lse[b,h,i] = ln( sum_{j visible to i} exp(scale * q_i . k_j) )
 *
 * for every batch index b < B and head h < H independently.  M is 0, or,
 * when `causal` is non-zero, -inf where key j > query i (autoregressive mask
 * aligned at the top-left corner: query i sees keys 0..i).
 *
 * This is the exact attention of the FlashAttention pages: the definition of
 * standard attention (the shakilmahmud.com page "Large language models part
 * 06: FlashAttention -- GPU SRAM, tiling, online softmax", section 1, and the
 * standard-attention recap of the unite.ai page "Flash Attention:
 * revolutionising transformer efficiency") evaluated tile by tile with the
 * online-softmax merge of section 2 of the same shakilmahmud.com page, in the
 * FlashAttention-2 order (outer loop over query blocks, inner loop over K/V
 * blocks, the final division by the softmax denominator deferred until the
 * inner loop ends -- section 1 of the itimpress.au page "FlashAttention
 * scaling, multi-GPU training and weight quantisation"; the parallelism over
 * query blocks is improvement 2 of the "FlashAttention-2 (BN)" systems-
 * analysis wiki article).  The N x N score matrix is never written to memory.
 * The pages define no log-sum-exp output and no mask; both readings above are
 * this library's.
 *
 * Layout: q, k, v, o are contiguous row-major [B][H][N][d] device arrays
 * (element (b,h,i,c) at ((b*H + h)*N + i)*d + c); lse is a contiguous
 * [B][H][N] float32 device array.
 *
 * Ownership and lifetime: the caller allocates and owns every buffer; the
 * library allocates no device or host memory and keeps no state other than
 * what the HIP runtime caches and one static device array per GPU (the
 * workspace of fa2_fwd_splitkv_noalloc, FA2_NOALLOC_WORKSPACE_BYTES, held
 * until the process ends).  All pointers are device pointers (hipMalloc
 * or equivalent) of the current HIP device, and a stream other than NULL and
 * HIP's legacy and per-thread default streams must be a stream of that
 * device (FA2_ERR_DEVICE otherwise).  Calls are thread-safe.
 *
 * Asynchrony: every entry point enqueues its kernel on `stream` (a
 * hipStream_t; NULL means the null stream) and returns without waiting.
 * Inputs must stay valid and unmodified, and outputs must not be read, until
 * the stream reaches that point.  Results are deterministic: the same inputs
 * give bit-identical outputs on every call (no atomics, fixed reduction
 * order).
 *
 * Aliasing: inputs may alias one another (they are only read).  Outputs (o
 * and lse; dq, dk, dv and delta of the backward pass) must not overlap any
 * input or each other (FA2_ERR_ALIAS).
 *
 * Errors: every argument is validated on the host before anything is
 * enqueued (the only HIP calls before that query the current device and the
 * stream's device), so a rejected call has no effect and enqueues nothing.  A non-zero return is
 * one of the FA2_ERR_* codes below; fa2_strerror() names it.
 *
 * Test switch: with FA2_DEBUG_ONE_WG_PER_CU=1 in the environment at the time
 * of a call, the attention kernels of every entry point (forward, fp32,
 * FP8, backward) are launched with dynamic LDS that they never touch, enough
 * that a workgroup takes more than half of a compute unit's 160 KB and at
 * most one runs per compute unit.  The outputs must keep the same bits: a
 * missing barrier or an LDS buffer reused too early would show under the
 * changed timing.  It costs time.
 */
#ifndef FA2_H
#define FA2_H

#ifdef __cplusplus
extern "C" {
#endif

#define FA2_OK 0
#define FA2_ERR_NULL (-1)    /* a required pointer is NULL                     */
#define FA2_ERR_SHAPE (-2)   /* B, H, N < 1, H_kv not dividing H, or a size
                                limit below exceeded                          */
#define FA2_ERR_HEADDIM (-3) /* d is not 64 or 128                             */
#define FA2_ERR_SCALE (-4)   /* scale is NaN or infinite                       */
#define FA2_ERR_ALIGN (-5)   /* a pointer is not 16-byte aligned               */
#define FA2_ERR_ALIAS (-6)   /* an output overlaps an input or another output  */
#define FA2_ERR_HIP (-7)     /* the kernel launch failed (hipGetLastError)     */
#define FA2_ERR_WORKSPACE (-8) /* fa2_fwd_splitkv_noalloc: the partials need
                                  more than FA2_NOALLOC_WORKSPACE_BYTES      */
#define FA2_ERR_DEVICE (-9)  /* the stream belongs to another device than the
                                current HIP device                            */

/* Size limits (FA2_ERR_SHAPE beyond them): B*H*N*d <= FA2_MAX_ELEMS elements
   per tensor (2^40, far above one GPU's memory); B*H and the number of
   workgroups (B*H*ceil(N/128), or B*H*ceil(N/64) for fa2_fwd_fp32) each
   <= 2^31 - 1 (32-bit grid indices); N*d <= FA2_MAX_HEAD_ELEMS_BF16 for the
   bf16 entry points (one head is addressed with 32-bit byte offsets) and
   <= 2^31 - 1 for fa2_fwd_fp32. */
#define FA2_MAX_ELEMS (1LL << 40)
#define FA2_MAX_HEAD_ELEMS_BF16 ((1LL << 30) - (1LL << 16))
/* Largest n_splits of fa2_fwd_splitkv. */
#define FA2_MAX_SPLITS 1024
/* Size of the static per-device workspace of fa2_fwd_splitkv_noalloc. */
#define FA2_NOALLOC_WORKSPACE_BYTES (32u << 20)

/*
 * fa2_fwd -- bf16 inputs, bf16 output.
 *   q, k, v : const bf16 [B][H][N][d]  (bfloat16 bit patterns, 2 bytes each)
 *   o       : bf16 [B][H][N][d], written, round-to-nearest-even from fp32
 *   lse     : float [B][H][N] or NULL (then no log-sum-exp is written)
 *   B, H, N : batch, heads, sequence length (queries and keys), each >= 1
 *   d       : head dimension, 64 or 128
 *   scale   : multiplies q.k before the softmax (usually 1/sqrt(d)); any
 *             finite value, including 0 and negative values
 *   causal  : 0 = no mask, non-zero = query i sees keys j <= i
 *   stream  : hipStream_t to enqueue on (NULL = null stream)
 * Products of bf16 values are exact in fp32; S and the running statistics
 * are fp32, probabilities are rounded to bf16 for the P.V product, whose
 * accumulation is fp32.
 * Causal key tiles that lie entirely past a query block's last query are
 * skipped: the mask hides every score in them, so they contribute exactly
 * zero to l and to O.  With FA2_DEBUG_NO_SKIP=1 in the environment at the
 * time of a call, the bf16 forward entry points (fa2_fwd, _o32, _gqa,
 * _splitkv and its variants) compute those tiles too, every score masked;
 * the outputs must not change.  It is a test switch and costs time.
 */
int fa2_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
            int B, int H, int N, int d, float scale, int causal, void *stream);

/*
 * fa2_fwd_o32 -- as fa2_fwd, but o is float [B][H][N][d]: the same kernel
 * with the final fp32 result stored without the last bf16 rounding.
 */
int fa2_fwd_o32(const void *q, const void *k, const void *v, float *o,
                float *lse, int B, int H, int N, int d, float scale,
                int causal, void *stream);

/*
 * fa2_fwd_gqa -- as fa2_fwd with H_kv <= H key/value heads shared by the
 * query heads (grouped-query attention; H_kv == 1 is multi-query
 * attention; H_kv == H is fa2_fwd).  FlashAttention-2 lists support for both
 * variants among its improvements (unite.ai page "Flash Attention:
 * revolutionising transformer efficiency", section "FlashAttention-2").
 *   q, o : bf16 [B][H][N][d];  k, v : const bf16 [B][H_kv][N][d]
 *   H_kv : >= 1 and dividing H (else FA2_ERR_SHAPE); query head h of batch
 *          index b uses key/value head h / (H / H_kv) of the same b
 * Every other argument, the lse output and the error rules are fa2_fwd's.
 * With N < 128 and a mask that does not vary by row (non-causal, or
 * N == 1), the H / H_kv query heads of one key/value head are computed as
 * one block of (H / H_kv) * N rows, so each key/value tile is read once per
 * key/value head.  Rows then share a wavefront with rows of other heads;
 * the wavefront's common rescale points change the fp32/bf16 rounding (not
 * the stated accuracy), so such a call need not match fa2_fwd on repeated
 * key/value heads bit for bit.  Larger or causal blocks do match it.
 */
int fa2_fwd_gqa(const void *q, const void *k, const void *v, void *o,
                float *lse, int B, int H, int H_kv, int N, int d, float scale,
                int causal, void *stream);

/* fa2_fwd_gqa_o32 -- fa2_fwd_gqa with a float [B][H][N][d] output. */
int fa2_fwd_gqa_o32(const void *q, const void *k, const void *v, float *o,
                    float *lse, int B, int H, int H_kv, int N, int d,
                    float scale, int causal, void *stream);

/*
 * fa2_fwd_splitkv -- the general forward: Nq query rows against Nk keys
 * (decoding against a key/value cache, chunked prefill), grouped K/V heads,
 * and the keys of each query block optionally split into n_splits ranges
 * computed by separate workgroups and then merged.  Splitting fills the GPU
 * when B * H * ceil(Nq / 128) alone would give too few workgroups.  The
 * merge is the two-block online-softmax merge of the shakilmahmud.com page
 * "Large language models part 06: FlashAttention -- GPU SRAM, tiling,
 * online softmax", section 2, over all ranges of a row.
 *   q, o     : [B][H][Nq][d] (o bf16);  k, v : const bf16 [B][H_kv][Nk][d]
 *   lse      : float [B][H][Nq] or NULL
 *   Nq, Nk   : >= 1 each
 *   causal   : query i sits at key position i + Nk - Nq and sees the keys
 *              at or before it (the last query sees every key; Nq == Nk is
 *              fa2_fwd's mask).  A query that sees no key (only when
 *              Nq > Nk) gets O = 0 and lse = -inf.
 *   n_splits : 1 .. FA2_MAX_SPLITS; with 1, o_part and lse_part are unused
 *              (may be NULL) and the call is one kernel launch
 *   o_part   : float [n_splits][B][H][Nq][d] caller-owned workspace
 *   lse_part : float [n_splits][B][H][Nq] caller-owned workspace
 * Range s covers key tiles [s*T, (s+1)*T) with T = ceil(ceil(Nk/64) /
 * n_splits) (tiles of 64 keys at d = 64 and d = 128); ranges past the end
 * are empty and contribute nothing.  The workspaces must not overlap any
 * input, output or each other (FA2_ERR_ALIAS); n_splits outside its range or
 * a grid over 2^31 - 1 workgroups is FA2_ERR_SHAPE.  Results depend on
 * n_splits only through rounding (each range keeps its own running maximum,
 * and the merge is fp32).  With Nq < 128 and H_kv < H, the query heads of
 * one key/value head are packed into one block exactly as fa2_fwd_gqa
 * describes (non-causal, or Nq == 1); the workspace layout is unchanged,
 * since [B][H][Nq] with h = h_kv * (H / H_kv) + g is the same memory as
 * [B][H_kv][(H / H_kv) * Nq].
 */
int fa2_fwd_splitkv(const void *q, const void *k, const void *v, void *o,
                    float *lse, int B, int H, int H_kv, int Nq, int Nk, int d,
                    float scale, int causal, int n_splits, float *o_part,
                    float *lse_part, void *stream);

/* fa2_fwd_splitkv_o32 -- fa2_fwd_splitkv with a float [B][H][Nq][d] o. */
int fa2_fwd_splitkv_o32(const void *q, const void *k, const void *v, float *o,
                        float *lse, int B, int H, int H_kv, int Nq, int Nk,
                        int d, float scale, int causal, int n_splits,
                        float *o_part, float *lse_part, void *stream);

/*
 * fa2_fwd_splitkv_noalloc -- fa2_fwd_splitkv (bf16 o) for callers that cannot
 * allocate memory: code being captured into a HIP graph, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, kernels and results
 * (bit-identical to fa2_fwd_splitkv with the same n_splits), but the fp32
 * partial outputs and lse of the key ranges live in a static device array
 * of FA2_NOALLOC_WORKSPACE_BYTES (32 MiB) that the library holds on every
 * GPU it runs on until the process ends; the call allocates nothing (no
 * hipMalloc, hipFree or allocating library routine).  With n_splits > 1 it
 * needs n_splits * B * H * Nq * (d + 1) * 4 bytes of that array; more is
 * FA2_ERR_WORKSPACE (checked on the host before any HIP call).  The first
 * call on a device looks up the array's device address (FA2_ERR_HIP if that
 * fails).  Every call on one GPU shares that GPU's array and leaves its
 * values behind; the range kernel writes every partial the merge reads, so
 * nothing needs clearing.  Calls that overlap in time on one GPU (different
 * streams, or host threads) race on the array: the caller serialises them.
 */
int fa2_fwd_splitkv_noalloc(const void *q, const void *k, const void *v,
                            void *o, float *lse, int B, int H, int H_kv,
                            int Nq, int Nk, int d, float scale, int causal,
                            int n_splits, void *stream);

/*
 * FP8 path: block quantisation with incoherent processing (the FP8 recipe
 * of FlashAttention-3 on the itimpress.au page "FlashAttention scaling,
 * multi-GPU training and weight quantisation", section 1: small tiles
 * scaled independently; Q and K multiplied by a random orthogonal matrix
 * before quantising to spread outliers), then attention on the gfx950 FP8
 * MFMA.  Codes are OCP e4m3 (bias 7, max 448, round to nearest even).
 *
 * fa2_quantize_fp8 -- x: const bf16 [B][H][N][d]; codes: e4m3 [B][H][N][d]
 * (written); exps: int [B][H][ceil(N / block_rows)] (written).  With signs
 * (device float [d] of +-1, or NULL for no rotation) each row is multiplied
 * by the signs and transformed by the unnormalised Walsh-Hadamard transform
 * (fp32 add/sub butterflies, stages h = 1, 2, 4, ...), i.e. rotated by
 * diag(signs) H / sqrt(d) and scaled by sqrt(d).  Each block of block_rows
 * (64 or 128) rows gets e, the smallest integer with max|y| <= 448 * 2^e
 * (0 for an all-zero block), and stores codes e4m3(y * 2^-e).  The
 * dequantised value is e4m3_value(code) * 2^e.  Rows past N are not read.
 *
 * fa2_fwd_fp8 -- attention of quantised q (block_rows 128), k and v
 * (block_rows 64; v never rotated): o = softmax(s q~ k~^T + mask) v~ with
 * q~, k~, v~ the dequantised values and s = scale, or scale / d when q and
 * k were quantised with the same signs (rotated != 0: the two sqrt(d)
 * factors cancel the transform's scaling, so the scores are those of the
 * unrotated inputs up to quantisation).  o: bf16 [B][H][N][d]; lse as for
 * fa2_fwd.  P is rounded to e4m3 for the P.V product (fp32 accumulation).
 * Same shape, mask, alignment and error rules as fa2_fwd; the exponent
 * arrays must not overlap the outputs.
 */
int fa2_quantize_fp8(const void *x, void *codes, int *exps, int B, int H,
                     int N, int d, int block_rows, const float *signs,
                     void *stream);
int fa2_fwd_fp8(const void *q8, const int *q_exp, const void *k8,
                const int *k_exp, const void *v8, const int *v_exp, void *o,
                float *lse, int B, int H, int N, int d, float scale,
                int rotated, int causal, void *stream);
/* fa2_fwd_fp8_o32 -- fa2_fwd_fp8 with a float [B][H][N][d] output. */
int fa2_fwd_fp8_o32(const void *q8, const int *q_exp, const void *k8,
                    const int *k_exp, const void *v8, const int *v_exp,
                    float *o, float *lse, int B, int H, int N, int d,
                    float scale, int rotated, int causal, void *stream);

/*
 * fa2_fwd_fp32 -- float32 q, k, v and o; every step (scores, softmax,
 * probabilities, P.V) in fp32 arithmetic, for exactness checks on small
 * problems.  Same shapes, mask, scale, lse, alignment and error rules.
 */
int fa2_fwd_fp32(const float *q, const float *k, const float *v, float *o,
                 float *lse, int B, int H, int N, int d, float scale,
                 int causal, void *stream);

/*
 * fa2_bwd -- gradients of fa2_fwd with respect to q, k and v (bf16 in, bf16
 * out), for the incoming gradient dout of o.
 *   q, k, v : const bf16 [B][H][N][d], the forward inputs
 *   o       : const bf16 [B][H][N][d], the forward output
 *   dout    : const bf16 [B][H][N][d], gradient of the loss with respect to o
 *   lse     : const float [B][H][N], the forward's log-sum-exp (required)
 *   delta   : float [B][H][N], workspace owned by the caller; on completion it
 *             holds D_i = sum_c dout_ic o_ic (fp32)
 *   dq, dk, dv : bf16 [B][H][N][d], written (round-to-nearest-even)
 *   B, H, N, d, scale, causal : as for fa2_fwd (the same values as the
 *             forward call that produced o and lse)
 * Computes the exact gradients of the forward definition,
 *   P = exp(scale q k^T - lse) (masked entries 0),  dv = P^T dout,
 *   dS = P * (dout v^T - D),  dq = scale dS k,  dk = scale dS^T q,
 * recomputing P tile by tile from lse (no N x N buffer) -- the recomputation
 * of the unite.ai page "Flash Attention: revolutionising transformer
 * efficiency", section "Enter Flash Attention".  Three kernels are enqueued
 * on `stream` in order (D, then dk/dv, then dq); no atomics, so results are
 * bit-reproducible.  bf16 products, fp32 accumulation; P and dS are rounded
 * to bf16 for the MFMA products.
 */
int fa2_bwd(const void *q, const void *k, const void *v, const void *o,
            const void *dout, const float *lse, float *delta, void *dq,
            void *dk, void *dv, int B, int H, int N, int d, float scale,
            int causal, void *stream);

/*
 * fa2_bwd_o32 -- as fa2_bwd, but dq, dk, dv are float [B][H][N][d] (the
 * same kernels without the final bf16 rounding).
 */
int fa2_bwd_o32(const void *q, const void *k, const void *v, const void *o,
                const void *dout, const float *lse, float *delta, float *dq,
                float *dk, float *dv, int B, int H, int N, int d, float scale,
                int causal, void *stream);

/*
 * fa2_bwd_gqa -- gradients of fa2_fwd_gqa (H_kv <= H key/value heads shared
 * by groups of H / H_kv consecutive query heads; grouped-query and
 * multi-query attention, listed among FlashAttention-2's additions on the
 * unite.ai page "Flash Attention: revolutionising transformer efficiency",
 * section "FlashAttention-2").
 *   q, o, dout, dq : [B][H][N][d];  k, v, dk, dv : [B][H_kv][N][d]
 *   lse, delta     : [B][H][N], as for fa2_bwd
 *   H_kv      : >= 1 and dividing H (else FA2_ERR_SHAPE)
 *   n_gsplits : 1 .. H / H_kv (else FA2_ERR_SHAPE).  The dk/dv of a shared
 *               head sum over its group of query heads; the group is cut
 *               into n_gsplits ranges of consecutive heads computed by
 *               separate workgroups (more parallel work when B * H_kv is
 *               small), whose fp32 partial sums a last kernel adds in range
 *               order.  1 = one workgroup per key block takes the whole
 *               group, no partials.
 *   dkv_part  : float [2][n_gsplits][B][H_kv][N][d] workspace owned by the
 *               caller (dk partials, then dv partials), required when
 *               n_gsplits > 1 (else FA2_ERR_NULL), ignored otherwise; it
 *               may overlap no other argument (FA2_ERR_ALIAS)
 * Same formulas, dtypes, rounding, stream order and error rules as fa2_bwd;
 * with H_kv == H and n_gsplits == 1 it runs exactly fa2_bwd's kernels.
 * Results are bit-reproducible for a given n_gsplits; different n_gsplits
 * add the same fp32 terms in a different order.
 */
int fa2_bwd_gqa(const void *q, const void *k, const void *v, const void *o,
                const void *dout, const float *lse, float *delta, void *dq,
                void *dk, void *dv, int B, int H, int H_kv, int N, int d,
                float scale, int causal, int n_gsplits, float *dkv_part,
                void *stream);

/* fa2_bwd_gqa_o32 -- fa2_bwd_gqa with float dq, dk, dv. */
int fa2_bwd_gqa_o32(const void *q, const void *k, const void *v,
                    const void *o, const void *dout, const float *lse,
                    float *delta, float *dq, float *dk, float *dv, int B,
                    int H, int H_kv, int N, int d, float scale, int causal,
                    int n_gsplits, float *dkv_part, void *stream);

/* Static English description of a return code (never NULL). */
const char *fa2_strerror(int code);

/* Library ABI version: 8 (2 added the backward pass, 3 grouped K/V heads,
   4 split key ranges with separate query and key lengths, 5 the FP8 path,
   6 the grouped-head backward, 7 fa2_fwd_splitkv_noalloc, 8 FA2_ERR_DEVICE
   for a stream of another device). */
int fa2_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA2_H */
