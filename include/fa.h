/*
 * fa.h -- C ABI of the fused attention forward for AMD MI355X (gfx950).
 *
 * The operation is the FlashAttention-2 forward pass: for each batch b and
 * head h,
 *
 *     O[b,h] = softmax(scale * Q[b,h] K[b,h]^T  [+ causal mask]) V[b,h]
 *     lse[b,h,i] = ln sum_{j visible to i} exp(scale * q_i . k_j)
 *
 * computed tile by tile with an online softmax so that the S x S score
 * matrix never reaches device memory.
 *
 * Passages this follows:
 *   - attention formula, tiling of Q into row blocks with K/V column blocks
 *     streamed past it, the online running-max / running-sum update, and
 *     the fusion of the two products and the softmax into one operator:
 *     "FlashAttention-2 on Ascend NPU: how ops-transformer reaches 3x"
 *     (2048ai.net), sections 1, 2.1, 2.2 (online softmax equation), 2.3;
 *   - the [batch, heads, seq_len, head_dim] row-major contiguous layout
 *     with 128-byte-aligned strides, the causal mode in which a position
 *     sees only itself and earlier tokens, and skipping of K/V tiles that
 *     lie wholly beyond a Q tile's last row: "catlass FlashAttention tuning
 *     for a 13B service" (gsyq.cn), sections "data layout" and "Causal Mask
 *     implementation" (mode 2);
 *   - the softmax scale passed explicitly as 1/sqrt(head_dim): "cann-
 *     learning-hub FlashAttention learning path" (omica.com.cn), steps three
 *     and five;
 *   - a launcher that takes a stream and returns a status code:
 *     "Analysis of the CANN ops-transformer FlashAttention operator"
 *     (lanjinlin.com.cn), "kernel entry" (unlike that launcher, this one
 *     never synchronises the stream).
 *
 * Threading and ownership: every entry point but fa_bwd_noalloc (whose
 * calls on one GPU share its scratch array) is stateless and thread-safe.
 * The caller owns every buffer; the library never allocates, frees or
 * synchronises, and it enqueues nothing but kernel launches on the given
 * stream (no memset or copy), so calls can be captured into a HIP graph and
 * replayed (the first call on a device reads its compute-unit count once,
 * outside any stream).
 */
#ifndef TILED_ATTENTION_15_FA_H
#define TILED_ATTENTION_15_FA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of Q, K, V and O. */
typedef enum {
    FA_F16 = 0,  /* IEEE binary16 */
    FA_BF16 = 1  /* bfloat16 */
} fa_dtype;

/* Status codes.  Every check runs on the host before anything is launched;
 * a non-FA_OK return means nothing was enqueued. */
typedef enum {
    FA_OK = 0,
    FA_ERR_NULL = 1,         /* q, k, v or o is NULL */
    FA_ERR_SHAPE = 2,        /* B, H or S < 1, or a size beyond the limits below */
    FA_ERR_UNSUPPORTED = 3,  /* D not in {64, 128, 256} ({64, 128} for
                                fa_naive_fwd), or dtype not an fa_dtype */
    FA_ERR_ALIGN = 4,        /* a pointer is not 16-byte aligned */
    FA_ERR_SCALE = 5,        /* scale is not finite or not > 0 */
    FA_ERR_HIP = 6,          /* the HIP runtime reported an error at launch */
    FA_ERR_ALIAS = 7,        /* o or lse overlaps q, k or v, or o overlaps lse */
    FA_ERR_STRIDE = 8,       /* a stride is negative, not a multiple of 8
                                elements, or makes o overlap itself */
    FA_ERR_MASK_DROPOUT = 9, /* fa_fwd_ext: bad mask layout or dropout
                                probability outside [0, 1) */
    FA_ERR_SCRATCH = 10      /* fa_bwd_noalloc: the call needs more than the
                                fixed scratch array holds */
} fa_status;

/*
 * fa_fwd -- fused attention forward.
 *
 *   q, k, v  device pointers, each [B, H, S, D] contiguous row-major of
 *            `dtype` (element (b,h,i,d) at ((b*H + h)*S + i)*D + d).
 *   o        device pointer, [B, H, S, D] contiguous, same dtype; written.
 *   lse      device pointer to [B, H, S] contiguous fp32 (natural-log
 *            log-sum-exp of each row's visible scaled scores), or NULL to
 *            skip it.
 *   B, H, S  batch, heads, sequence length (>= 1; any S, not only multiples
 *            of the tile; S <= 2^30, B*H*S*D < 2^40 and S*D*2 bytes < 2^31).
 *   D        head dimension, 64, 128 or 256 (named among the head
 *            dimensions of "FlashAttention-2 on Ascend NPU" (2048ai.net),
 *            tiling parameters).  D = 256 runs the tuned kernel with
 *            128-row blocks: each wave group owns 64 rows, and each pair
 *            of its waves shares 32 of them, one wave per half of every
 *            key tile's scores and per half of O's columns.
 *   scale    softmax scale applied to q.k (callers normally pass
 *            1/sqrt(D)); finite and > 0.
 *   causal   0: every key visible; nonzero: key j visible to query i iff
 *            j <= i (the diagonal included).
 *   dtype    an fa_dtype.
 *   stream   hipStream_t to enqueue on, or NULL for the default stream.
 *
 * Numerics: products on the matrix cores with fp16/bf16 inputs and fp32
 * accumulation; softmax in fp32 with base-2 exponentials; probabilities
 * rounded to `dtype` before the second product; O rounded to `dtype` with
 * round-to-nearest-even.  Results are bitwise reproducible run to run (no
 * atomics).  Non-finite inputs propagate to the outputs they touch.
 * Domain: an exponent is formed as scale*log2(e)*s - m in one fused
 * multiply-add, m the row maximum in fp32, so it carries m's rounding,
 * up to half an fp32 ulp of m.  That stays below the probabilities'
 * 16-bit rounding while |scale * q.k| is below about 8,000 (natural-log
 * units; attention scores in practice are below a few hundred).  Far
 * beyond, at about 1e9, exponentials overflow and outputs are not finite.
 *
 * Returns an fa_status.  Asynchronous: a fault inside the kernel surfaces at
 * the caller's next synchronisation, not here.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int S, int D, float scale, int causal, int dtype,
           void* stream);

/*
 * fa_fwd_strided -- the same forward for strided tensors and for query and
 * key sequences of different lengths (cross attention, a query block
 * attending to a longer key sequence).
 *
 *   q        [B, H, Sq, D]: element (b,h,i,d) at
 *            q_strides[0]*b + q_strides[1]*h + q_strides[2]*i + d
 *            (element strides; the head dimension is contiguous).
 *   k, v     [B, H, Sk, D] with k_strides / v_strides likewise.  A head
 *            stride of 0 shares one K (or V) between all heads of a batch.
 *   o        [B, H, Sq, D] with o_strides; written.  Its strides must not
 *            make two elements share an address.
 *   lse      [B, H, Sq] contiguous fp32, or NULL.
 *   Sq, Sk   query and key/value rows per head (>= 1).
 *   causal   0: every key visible; nonzero: key j visible to query i iff
 *            j <= i + (Sk - Sq), i.e. the last query row sees every key (for
 *            Sq == Sk this is fa_fwd's causal mask).  A row that sees no key
 *            (Sq > Sk) gets O = 0 and lse = -inf.
 *   other arguments as for fa_fwd.
 *
 * Strides (in elements) must be >= 0 and multiples of 8 (16-byte rows); a
 * row stride must be >= D.  Per tensor and head, the rows a query block or
 * key tile can address must span fewer than 2^31 bytes:
 * (round_up(S, 256) + 64) * row_stride * 2 < 2^31.
 *
 * The causal reading for Sq != Sk (bottom-right alignment) extends the
 * pages' rule that a position sees only itself and earlier tokens ("catlass
 * FlashAttention tuning for a 13B service" (gsyq.cn), "Causal Mask
 * implementation") to a query block that ends at the end of the keys; the
 * need for unequal lengths is named by the cross-attention use case of
 * "Analysis of the CANN ops-transformer FlashAttention operator"
 * (lanjinlin.com.cn), "application scenarios".
 *
 * Returns an fa_status (FA_ERR_STRIDE for the stride rules above).
 */
int fa_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int Sq, int Sk, int D,
                   const int64_t* q_strides, const int64_t* k_strides,
                   const int64_t* v_strides, const int64_t* o_strides,
                   float scale, int causal, int dtype, void* stream);

/* Human-readable text of a status code (static storage; never NULL). */
const char* fa_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
int fa_version(void);

/*
 * fa_fwd_plan -- the launch fa_fwd would make, without launching it.
 *
 * Fills (each pointer may be NULL):
 *   block_q    query rows per workgroup (B_r): 256; 128 at D = 256 (the
 *              pair split), and at
 *              D = 64 or 128 when n = B * H * ceil(S / 256) satisfies
 *              2n <= C, or n < C for a causal call, C the current device's
 *              compute-unit count (256 on MI355X) (the key-split
 *              instance: both wave groups on the same 128 rows, the K/V
 *              tiles shared out even/odd between them and the two partial
 *              results merged; with an odd count one extra, fully masked
 *              tile is visited, not counted below; fa_fwd_ext makes the same
 *              choice for a mask without dropout),
 *   block_kv   keys per K/V tile (B_c),
 *   grid       workgroups launched (B * H * ceil(S / B_r)),
 *   tiles      (query block, K/V tile) pairs the kernel processes: for a
 *              causal call, only the tiles whose first key does not lie
 *              beyond the query block's last row, i.e. per query block
 *              min(ceil(S / B_c), ceil(min(S, (qb+1)*B_r) / B_c)).
 * Same validation and return codes as fa_fwd (no device pointers are
 * needed: they are not inspected).  Launches nothing; its only HIP calls
 * read the current device's compute-unit count, once per device (256 when
 * no device answers).
 * Follows the tile-count and block-count arithmetic of "FlashAttention-2 on
 * Ascend NPU: how ops-transformer reaches 3x" (2048ai.net), section 3.2
 * (ceiling division of the sequence by the block sizes) and the skip rule
 * of "catlass FlashAttention tuning for a 13B service" (gsyq.cn), section
 * "Causal Mask implementation".
 */
int fa_fwd_plan(int B, int H, int S, int D, int causal, int dtype,
                int* block_q, int* block_kv, int64_t* grid, int64_t* tiles);

/*
 * fa_fwd_diag -- a diagnostic (test-only) launch of the tuned forward on
 * contiguous tensors: the same kernel and arithmetic as fa_fwd_strided
 * (same block shape and route, q and o [B, H, Sq, D], k and v [B, H, Sk, D],
 * causal as there), with three extra outputs for checking it:
 *
 *   o32          NULL, or device fp32 [B, H, Sq, D] contiguous: O before its
 *                rounding to `dtype`, so the kernel's own error can be
 *                measured against the fp64 result without the storage
 *                rounding of O.  o is still written, identically.
 *   tile_counts  NULL, or device uint32 [fa_fwd_diag_tile_slots(...)]: for
 *                workgroup block n (n = (b*H + h) * nqb + query block) and
 *                wave w, slot 8*n + w counts the K/V tiles that wave ran
 *                its softmax on.  Its sum over the waves of a block checks
 *                the causal skip rule of "catlass FlashAttention tuning for
 *                a 13B service" (gsyq.cn), "Causal Mask implementation"
 *                (mode 2) on the device: every wave of a 256-row block runs
 *                every tile the block visits; in the key-split route the two
 *                wave groups share them out, with one extra, fully masked
 *                tile when their count is odd.
 *   flags        0, or FA_DIAG_REVERSE_ORDER: workgroup i takes the block
 *                workgroup grid-1-i would take.  Blocks are independent, so
 *                every output must be bitwise equal to the default order's.
 *
 * D must be 64 or 128 (else FA_ERR_UNSUPPORTED, as for an unknown flag);
 * other errors as for fa_fwd, with o32 and tile_counts also checked for
 * 16-byte alignment and overlap.  Not for production use: it exists for
 * the tests.
 */
#define FA_DIAG_REVERSE_ORDER 1
int fa_fwd_diag(const void* q, const void* k, const void* v, void* o, float* lse, float* o32,
                uint32_t* tile_counts, int B, int H, int Sq, int Sk, int D, float scale,
                int causal, int dtype, int flags, void* stream);

/* Number of uint32 slots fa_fwd_diag writes to tile_counts for these
 * arguments (8 per workgroup), or 0 for a shape it rejects. */
int64_t fa_fwd_diag_tile_slots(int B, int H, int Sq, int D, int causal);

/*
 * fa_clock_stamps -- a measurement aid: launches `groups` workgroups (1 ..
 * 65536) on `stream`; thread 0 of workgroup n writes out[4n .. 4n+3] =
 * {XCD id, shader-clock counter, 100 MHz real-time counter, 0}.  Two calls
 * around a timed region give each XCD's average shader clock over it:
 * delta shader ticks / delta real-time ticks * 100 MHz, the clock against
 * which an achieved fraction of the matrix-core peak (quoted at 2.4 GHz) can
 * be read.  out: device, 16-byte aligned, groups*4 uint64.  Returns
 * FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_ALIGN or FA_ERR_HIP on failure.
 */
int fa_clock_stamps(uint64_t* out, int groups, void* stream);

/*
 * fa_naive_fwd -- the same forward computed the unfused way, for comparison:
 * scores S = scale * Q K^T (causal mask applied) written to `workspace` in
 * fp32, a row softmax writing P (in `dtype`) and lse, then O = P V.  This is
 * the three-step flow that "FlashAttention-2 on Ascend NPU: how
 * ops-transformer reaches 3x" (2048ai.net), section 1, and "ops-transformer
 * FlashAttention operator in practice" (ai6s.net), sections 1 and 4, describe
 * as the baseline the fused operator replaces; its S x S matrices cost
 * O(S^2) device memory and traffic.  Arguments as for fa_fwd (contiguous
 * [B, H, S, D], same outputs and numerics up to rounding order), plus:
 *
 *   workspace        device memory of at least fa_naive_workspace_bytes()
 *                    bytes, 16-byte aligned, not overlapping any other
 *                    argument; owned by the caller, contents overwritten.
 *   workspace_bytes  its size.
 *
 * Limits: S <= 16384 (one workgroup's registers hold a whole softmax row) and
 * B * H <= 65535; otherwise FA_ERR_SHAPE.  A workspace that is NULL or too
 * small gives FA_ERR_NULL / FA_ERR_SHAPE; one that overlaps q, k, v, o or lse
 * gives FA_ERR_ALIAS.  Launches four kernels on `stream`.
 */
int fa_naive_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int S, int D, float scale, int causal, int dtype,
                 void* workspace, int64_t workspace_bytes, void* stream);

/* Bytes of workspace fa_naive_fwd needs for this shape (0 for an invalid
 * shape): per (batch, head), S x Sp fp32 scores, S x Sp probabilities and
 * D x Sp transposed values (16-bit), Sp = S rounded up to a multiple of 64. */
int64_t fa_naive_workspace_bytes(int B, int H, int S, int D);

/*
 * fa_fwd_ext -- the forward with an explicit boolean mask and/or dropout,
 * fused into one kernel ("FlashAttention-2 on Ascend NPU: how
 * ops-transformer reaches 3x" (2048ai.net), section 3.4 and section 6.3):
 * the mask and the dropout act on the score tile on chip, so no S x S
 * pass touches device memory.
 *
 *   q, o        device, contiguous [B,H,Sq,D] of `dtype`; k, v [B,H,Sk,D]
 *   lse         device [B,H,Sq] fp32 or NULL: log-sum-exp of the masked,
 *               undropped scores (-inf for a row with no visible key)
 *   mask        device uint8 or NULL; element (b,h,i,j) at
 *               mask[b*mask_strides[0] + h*mask_strides[1] + i*mask_strides[2] + j];
 *               nonzero keeps score (i, j), zero hides it (on top of the
 *               causal rule).  Strides in bytes, >= 0 (0 broadcasts over
 *               batch or heads), multiples of 4, row stride >= Sk; the
 *               pointer 4-byte aligned; one head's rows must span less than
 *               2^31 bytes.  A row with no visible key gives O = 0.
 *   dropout_p   in [0, 1): each probability is kept with probability
 *               1 - t/65536, t = round(dropout_p * 65536) (ties to even),
 *               and the kept ones are scaled by 65536/(65536 - t).  The keep
 *               decision of score (b*H+h, i, j) compares with t the 16-bit
 *               half j%2 (low half for even j) of word (j%8)/2 of
 *               Philox4x32-10 (Salmon et al., SC 2011) at counter
 *               (j/8, i, b*H+h, offset) and key (seed & 0xffffffff, seed >> 32).
 *               dropout_p = 0 keeps everything.
 *   causal, scale, dtype, stream  as for fa_fwd (bottom-right causal rule
 *               when Sq != Sk).
 * Kernels: with dropout_p 0 and every tensor's head spanning less than
 * ((round_up(S, 256) + 64) * row_stride + D) * 2 < 2^31 bytes, the call runs
 * the tuned forward kernel of fa_fwd_strided (its masked instance when mask
 * is set); otherwise the general kernel (128-row blocks) that also draws the
 * dropout decisions.  With mask NULL and dropout_p 0 the result therefore
 * equals fa_fwd_strided's bit for bit.
 * Returns FA_OK or an fa_status; FA_ERR_MASK_DROPOUT for a bad mask layout
 * or dropout probability.
 */
int fa_fwd_ext(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int Sq, int Sk, int D,
               const uint8_t* mask, const int64_t* mask_strides,
               float dropout_p, uint64_t seed, uint32_t offset,
               float scale, int causal, int dtype, void* stream);

/*
 * fa_fwd_ext_strided -- fa_fwd_ext for strided q, k, v, o (a [B, S, H, D]
 * buffer viewed as [B, H, S, D], a packed q/k/v projection, K and V shared by
 * the heads of a batch).
 *   strides  host array of 12 element strides: batch, head and row stride of
 *            q, k, v, o in that order (element (b, h, i, d) of a tensor at
 *            b*s[0] + h*s[1] + i*s[2] + d; the head dimension contiguous).
 *            Every stride >= 0 and a multiple of 8; row strides >= D and below
 *            2^30; o's strides must not map two elements to one address
 *            (FA_ERR_STRIDE).  Per tensor and head,
 *            ((round_up(S, 128) + 128) * row_stride + D) * 2 < 2^31 bytes.
 * Aliasing: o's and lse's byte spans (first to past the last element) must
 * not overlap any input's span or each other (FA_ERR_ALIAS).  Everything
 * else as for fa_fwd_ext; fa_fwd_ext is this call with contiguous strides.
 */
int fa_fwd_ext_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int H, int Sq, int Sk, int D, const int64_t* strides,
                       const uint8_t* mask, const int64_t* mask_strides,
                       float dropout_p, uint64_t seed, uint32_t offset,
                       float scale, int causal, int dtype, void* stream);

/*
 * fa_fwd_causal_offset -- fa_fwd_ext_strided under the causal rule with the
 * diagonal at an explicit offset: key j is visible to query i iff
 * j <= i + causal_offset (and the mask keeps it, when there is one).
 * Sequence parallelism ("FlashAttention-2 on Ascend NPU" (2048ai.net),
 * section 6.4: each device works on its own chunk of the sequence) splits a
 * causal sequence into chunks; the block of queries from global position
 * qs against keys from ks is this call with causal_offset = qs - ks, and the
 * blocks' (o, lse) merge by lse = log(sum_b exp(lse_b)),
 * o = sum_b exp(lse_b - lse) o_b.  causal_offset = Sk - Sq is fa_fwd_ext's
 * causal rule (the calls agree bit for bit); 0 aligns the diagonal with the
 * first query and key (top-left).  Offsets at or below -Sq hide every key
 * (every row gets o = 0, lse = -inf) and offsets at or above Sk show every
 * key; the offset is clamped to [-Sq, Sk].  Everything else (arguments,
 * layouts, dropout counter, limits, errors) as for fa_fwd_ext_strided with
 * causal = 1.
 */
int fa_fwd_causal_offset(const void* q, const void* k, const void* v, void* o, float* lse,
                         int B, int H, int Sq, int Sk, int D, const int64_t* strides,
                         const uint8_t* mask, const int64_t* mask_strides,
                         float dropout_p, uint64_t seed, uint32_t offset,
                         float scale, int64_t causal_offset, int dtype, void* stream);

/*
 * fa_bwd -- gradients of the attention forward above: given dout = dL/dO,
 * writes dq = dL/dq, dk = dL/dk and dv = dL/dv.  The scores and
 * probabilities are recomputed from q, k and the forward's lse rather than
 * stored ("ops-transformer FlashAttention operator in practice" (ai6s.net),
 * section 2, table of core optimisations: recomputation in the backward;
 * "FlashAttention-2 on Ascend NPU" (2048ai.net), section 6.2).  With
 * P_ij = exp(scale q_i.k_j - lse_i) (0 where masked) and D_i = dout_i . o_i:
 *   dv_j = sum_i P_ij dout_i,  dS_ij = P_ij (dout_i . v_j - D_i),
 *   dq_i = scale sum_j dS_ij k_j,  dk_j = scale sum_i dS_ij q_i.
 * dq is computed by a separate pass that sums each row's key tiles in a
 * fixed order (the scores recomputed once more), the deterministic mode of
 * "catlass FlashAttention tuning for a 13B service" (gsyq.cn), backward-pass
 * section: results are bitwise reproducible run to run.
 *   deterministic    accepted for source compatibility and ignored: the
 *                    page's non-deterministic mode (dq accumulated with fp32
 *                    atomic adds while dk/dv are computed) is not provided,
 *                    every call runs the deterministic kernels.
 *
 *   q, o, dout, dq   device, contiguous [B,H,Sq,D] of `dtype`
 *   k, v, dk, dv     device, contiguous [B,H,Sk,D] of `dtype`
 *   lse              device, [B,H,Sq] fp32, as written by fa_fwd for the same
 *                    q, k, v, scale and causal flag (natural log; -inf for a
 *                    row that sees no key)
 *   causal           key j visible to query i iff j <= i + (Sk - Sq)
 *   workspace        device memory of at least
 *                    fa_bwd_workspace_bytes(B,H,Sq,D,1) bytes,
 *                    16-byte aligned, owned by the caller, contents
 *                    overwritten; it must not overlap any other argument
 *   stream           HIP stream (NULL = default); asynchronous, no allocation
 *                    and no synchronisation inside.
 * All pointers 16-byte aligned.  Inputs may overlap each other; dq, dk, dv
 * and the workspace must not overlap each other or any input (FA_ERR_ALIAS).
 * Limits: D in {64, 128, 256} (D = 256 runs with one workgroup per compute
 * unit, the accumulators in the matrix-core registers); (max(Sq, Sk) rounded up to 128, plus 128) * D * 2
 * bytes below 2^31.  Returns FA_OK or a status as for fa_fwd; nothing is
 * enqueued on error.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, int B, int H, int Sq, int Sk, int D,
           float scale, int causal, int dtype, int deterministic, void* workspace,
           int64_t workspace_bytes, void* stream);

/*
 * fa_bwd_noalloc -- fa_bwd without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation).
 * The workspace is a fixed device array inside the library, 16 MiB
 * (fa_bwd_noalloc_scratch_bytes()), held by each GPU the library runs on
 * until the process ends; its device address is looked up once per device
 * on the first call there.  The call itself allocates nothing and does not
 * synchronise.
 *
 * Arguments, layouts, numerics and errors as for fa_bwd (results bitwise
 * equal to that call), plus
 * FA_ERR_SCRATCH when fa_bwd_workspace_bytes(B, H, Sq, D, 1) exceeds the
 * array (B * H * Sq above 4,194,304 rows) and FA_ERR_HIP when the array's
 * address cannot be obtained.  Every call on one GPU shares that GPU's
 * array: calls that overlap in time on one GPU (two streams, two threads)
 * race and must be ordered by the caller.
 */
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv, int B, int H, int Sq, int Sk,
                   int D, float scale, int causal, int dtype, void* stream);

/* Size in bytes of fa_bwd_noalloc's fixed scratch array. */
int64_t fa_bwd_noalloc_scratch_bytes(void);

/*
 * fa_bwd_ext -- gradients of fa_fwd_ext: the backward with the same explicit
 * mask and dropout as the forward that produced o and lse (same mask, strides,
 * dropout_p, seed and offset).  With Z c the forward's keep factor
 * (0 or 65536/(65536 - t)):
 *   dv_j = sum_i P_ij Z_ij c dout_i,  dS_ij = P_ij (Z_ij c dout_i . v_j - D_i),
 *   dq_i = scale sum_j dS_ij k_j,  dk_j = scale sum_i dS_ij q_i,
 * D_i = dout_i . o_i.  Deterministic like fa_bwd; the workspace is
 * fa_bwd_workspace_bytes(B, H, Sq, D, 1).  Arguments as for fa_bwd and
 * fa_fwd_ext (mask rows are read up to 31 rows past the last query, so
 * (Sq + 31) * mask row stride + Sk must stay below 2^31 bytes); the mask
 * must not overlap an output.  D in {64, 128, 256}.
 */
int fa_bwd_ext(const void* q, const void* k, const void* v, const void* o, const void* dout,
               const float* lse, void* dq, void* dk, void* dv, int B, int H, int Sq, int Sk, int D,
               const uint8_t* mask, const int64_t* mask_strides, float dropout_p, uint64_t seed,
               uint32_t offset, float scale, int causal, int dtype, void* workspace,
               int64_t workspace_bytes, void* stream);

/*
 * fa_bwd_strided -- fa_bwd and fa_bwd_ext for strided tensors, e.g. the
 * [B, S, H, D] layout of a fused projection, where the backward's inputs and
 * gradients are views of larger buffers.  Same mathematics as fa_bwd (and, with
 * a mask or dropout, as fa_bwd_ext).
 *   strides  host array of 24 element strides: batch, head and row stride of
 *            q, k, v, o, dout, dq, dk, dv, in that order (element (b, h, i, d)
 *            of a tensor at b*s[0] + h*s[1] + i*s[2] + d; the head dimension
 *            is contiguous).  Every stride is >= 0 and a multiple of 8; row
 *            strides >= D and below 2^30.  Input strides may be 0 (one K
 *            shared by all heads, say); dq, dk and dv must not map two
 *            elements to one address (FA_ERR_STRIDE).
 *   lse      contiguous [B, H, Sq] fp32, as for fa_bwd.
 *   mask, mask_strides, dropout_p, seed, offset  as for fa_bwd_ext (mask
 *            NULL and dropout_p 0 for the plain backward).
 *   deterministic  ignored, as for fa_bwd.
 *   workspace  at least fa_bwd_workspace_bytes(B, H, Sq, D, 1)
 *            bytes; contiguous scratch as for fa_bwd.
 * Aliasing: the byte range each tensor spans (from its first to past its
 * last element) of dq, dk, dv and the workspace must not overlap one another
 * or any input's (FA_ERR_ALIAS).  Per tensor and head, rows up to
 * round_up(S, 128) + 128 are addressed with 32-bit offsets:
 * ((round_up(S, 128) + 128) * row_stride + D) * 2 < 2^31.  D in {64, 128, 256}.
 * Returns an fa_status; nothing is enqueued on error.
 */
int fa_bwd_strided(const void* q, const void* k, const void* v, const void* o, const void* dout,
                   const float* lse, void* dq, void* dk, void* dv, int B, int H, int Sq, int Sk, int D,
                   const int64_t* strides, const uint8_t* mask, const int64_t* mask_strides,
                   float dropout_p, uint64_t seed, uint32_t offset, float scale, int causal, int dtype,
                   int deterministic, void* workspace, int64_t workspace_bytes, void* stream);

/*
 * fa_bwd_causal_offset -- gradients of fa_fwd_causal_offset: fa_bwd_strided
 * under the causal rule with the diagonal at causal_offset (key j visible
 * to query i iff j <= i + causal_offset, clamped to [-Sq, Sk]): the
 * gradients of sum(o * dout) for the o of fa_fwd_causal_offset on the same
 * inputs, offset, mask and dropout arguments, whose o and lse are passed
 * in.  Everything else as for fa_bwd_strided.
 */
int fa_bwd_causal_offset(const void* q, const void* k, const void* v, const void* o, const void* dout,
                         const float* lse, void* dq, void* dk, void* dv, int B, int H, int Sq, int Sk,
                         int D, const int64_t* strides, const uint8_t* mask, const int64_t* mask_strides,
                         float dropout_p, uint64_t seed, uint32_t offset, float scale,
                         int64_t causal_offset, int dtype, void* workspace, int64_t workspace_bytes,
                         void* stream);

/* Bytes of workspace fa_bwd, fa_bwd_ext and fa_bwd_strided need (0 for an
 * invalid shape): the row dot products D_i, B*H*Sq fp32, rounded up to 256
 * bytes.  `deterministic` is ignored, as for fa_bwd. */
int64_t fa_bwd_workspace_bytes(int B, int H, int Sq, int D, int deterministic);

#ifdef __cplusplus
}
#endif

#endif /* TILED_ATTENTION_15_FA_H */
