/*
 * fa2.h -- C ABI of the FlashAttention-2 forward pass for MI355X (gfx950).
 *
 * The operation is exact scaled-dot-product attention over
 * (batch, heads, seq, head_dim) tensors:
 *
 *     S_i,j = scale * (q_i . k_j)                     (j <= i kept when causal)
 *     O_i   = sum_j exp(S_i,j - m_i) v_j / l_i,  m_i = max_j S_i,j,
 *                                                l_i = sum_j exp(S_i,j - m_i)
 *     lse_i = m_i + ln(l_i)
 *
 * as stated by the cookbook notebook "FlashAttention-2 in an attention layer"
 * (its Triton kernel and flash_attn_triton wrapper: q of shape (B, H, T, D),
 * O of q's dtype, scale 1/sqrt(D) by default, causal mask offs_m >= cur_n),
 * with the per-row logsumexp that the FlashAttention-2 epilogue writes next to
 * O (jared-hpc Lecture 6, reading task). The kernel evaluates it with the
 * online softmax and deferred 1/l normalisation of the infra.bea.ai
 * FlashAttention V2 guide ("Optimization 2: Delay Rescaling") and never forms
 * the S x S score matrix.
 *
 * Supported inputs are fp16 or bf16 with head_dim 64, 128 or 256 (the head
 * dims and dtypes FlashAttention-2 serves, jared-hpc Lecture 6 "Use it in the
 * real stack" and the infra.bea.ai guide's "When V2 Is Used" table). Anything
 * else fails loudly with a status code; the library never falls back to
 * another path.
 */
#ifndef FA2_H
#define FA2_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of q, k, v and o. */
typedef enum {
    FA2_F16 = 0,  /* IEEE binary16 */
    FA2_BF16 = 1  /* bfloat16 */
} fa2_dtype;

/* Return codes. Every failure is reported before anything is launched,
 * except FA2_ERR_LAUNCH, which reports an error from the HIP runtime at
 * launch time. */
typedef enum {
    FA2_OK = 0,
    FA2_ERR_NULL = 1,      /* a tensor pointer is NULL */
    FA2_ERR_SHAPE = 2,     /* B, H or S < 1, H or B > 65535, B*H*S*D elements (or their
                              bytes) overflow int64, the grid passes 2^31 workgroups, or
                              (strided) 256 rows of Q, K or V span 2^31 bytes or more */
    FA2_ERR_HEADDIM = 3,   /* D is not 64, 128 or 256 */
    FA2_ERR_DTYPE = 4,     /* dtype is not FA2_F16 or FA2_BF16 */
    FA2_ERR_ALIGN = 5,     /* q, k, v, o not 16-byte aligned, or lse not 4-byte aligned */
    FA2_ERR_SCALE = 6,     /* scale is NaN or infinite (FP8: a descale not finite and > 0) */
    FA2_ERR_NO_DEVICE = 7, /* no current HIP device, or the device is not gfx950 */
    FA2_ERR_LAUNCH = 8,    /* the HIP runtime reported an error at launch */
    FA2_ERR_ALIAS = 9,     /* o or lse overlaps q, k or v, or o overlaps lse (split-KV:
                              or the workspace overlaps any tensor) */
    FA2_ERR_WORKSPACE = 10, /* split-KV: workspace NULL, misaligned or too small */
    FA2_ERR_STRIDE = 11,    /* strided: a stride negative, above 2^40 or not a multiple of 8,
                               a sequence stride below D, or o's rows overlapping */
    FA2_ERR_SCRATCH = 12    /* no-allocation split-KV: the call needs more scratch than the
                               library's fixed FA2_SCRATCH_BYTES */
} fa2_status;

/*
 * fa2_fwd -- launch the forward pass on `stream`; returns an fa2_status.
 *
 * q, k, v  device pointers to B*H*S*D elements of `dtype`, contiguous
 *          row-major (B, H, S, D): element (b, h, s, d) is at index
 *          ((b*H + h)*S + s)*D + d. Read only. 16-byte aligned.
 * o        device pointer, same shape, layout and dtype as q. Written for
 *          every (b, h, s < S, d); nothing else is touched. 16-byte aligned.
 * lse      device pointer to B*H*S floats, contiguous (B, H, S): the natural
 *          logarithm of sum_j exp(S_i,j) over the keys row i attends to.
 *          4-byte aligned.
 * B, H     batch size and number of heads, 1..65535 each.
 * S        sequence length of queries and keys (they are equal), >= 1.
 *          Any S is accepted; S need not be a multiple of a tile size.
 * D        head dimension: 64, 128 or 256.
 * causal   nonzero: query i attends to keys j <= i (the diagonal is kept,
 *          so every row attends to at least key 0); zero: all keys.
 * scale    multiplies q . k before the mask and the softmax; any finite
 *          value (0 gives uniform weights, a negative one reverses the
 *          order of the scores). Callers that want the usual default pass
 *          1/sqrt(D).
 * dtype    FA2_F16 or FA2_BF16 (applies to q, k, v and o).
 * stream   a hipStream_t (NULL = the default stream) on the current device.
 *
 * Ownership: the caller owns every buffer; the library allocates nothing,
 * keeps no per-call state and is safe to call from several threads.
 * Synchronisation: the work is enqueued on `stream` and the call returns
 * without waiting for it. o and lse must not overlap q, k, v or each other.
 * Work order: on grids of more than two workgroups per compute unit the
 * last quarter of the workgroups take their query tiles in the order they
 * start, from a counter the library holds per (device, stream) in its own
 * device memory (1024 per device; each launch leaves its counter at zero),
 * so that faster XCDs take more of the short tiles at the end. Calls on one
 * stream run in order and calls on different streams use different
 * counters (hipStreamPerThread counting as a stream of its own in each host
 * thread); a call made while `stream` is being captured into a graph, or
 * once every counter of the device is in use, takes the fixed order
 * instead. The results do not depend on the order.
 * Arithmetic: products on fp16/bf16 matrix cores with fp32 accumulation;
 * the softmax state (running max, running sum, unnormalised O) is fp32; O
 * is rounded once, to nearest even, into `dtype`.
 */
int fa2_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
            int B, int H, int S, int D, int causal, float scale, int dtype,
            void *stream);

/*
 * fa2_fwd_strided -- fa2_fwd on tensors laid out with arbitrary strides,
 * such as the (B, S, H, D) views of a packed QKV projection that an
 * attention layer produces (the cookbook notebook's FA2Attention transposes
 * and copies them to (B, H, S, D) before its kernel; this call reads and
 * writes them in place).
 *
 * strides  host pointer to 12 element strides: the batch, head and sequence
 *          strides of q, then of k, v and o, in that order. Element
 *          (b, h, s, d) of q is at q[b*strides[0] + h*strides[1] +
 *          s*strides[2] + d]; the head dim is contiguous. Each stride is in
 *          [0, 2^40] and a multiple of 8 (16-byte rows); each sequence
 *          stride is >= D. Batch and head strides may be 0 for q, k and v
 *          (a K/V shared by all heads), but o's rows must be disjoint.
 * lse      contiguous (B, H, S) floats, as for fa2_fwd.
 * Other arguments, the result and the arithmetic are those of fa2_fwd, and
 * for contiguous strides the result is bit-identical to it. A head may
 * span any size, but 256 rows of Q, of K and of V must span under 2^31
 * bytes (256 * sequence stride * 2), the reach of one tile load's offsets.
 * Overlap is judged on the byte range each tensor spans, so o and lse must
 * not fall within q's, k's or v's span. Returns FA2_ERR_STRIDE for bad
 * strides, otherwise the codes of fa2_fwd.
 */
int fa2_fwd_strided(const void *q, const void *k, const void *v, void *o, float *lse,
                    int B, int H, int S, int D, const long long *strides, int causal,
                    float scale, int dtype, void *stream);

/*
 * fa2_fwd_balanced -- fa2_fwd (strides NULL) or fa2_fwd_strided (strides
 * given), with the keys of long query tiles split across workgroups when
 * the grid is too small to keep the GPU busy to its end.
 *
 * The sequence-parallel grid of FlashAttention-2 (jared-hpc Lecture 6, "FA2
 * change 1") has ceil(S / rows) * H * B workgroups. When that is under two
 * rounds of the workgroups the GPU holds at once, the launch ends on its
 * longest tile -- under causal masking, the last query tile of a head, with
 * all S keys against the average tile's S / 2 -- and part of the GPU idles
 * meanwhile. This call then cuts each query tile's keys into chunks that
 * run as separate workgroups, longest first, and merges the chunks' partial
 * (O~, m, l) with the rescaling algebra of the infra.bea.ai FlashAttention
 * V2 guide ("Optimization 2: Delay Rescaling") in a second kernel on the
 * same stream -- "FA2 change 2" of the lecture (parts of the KV range
 * computed apart, their (m, l) combined at the end) across workgroups.
 * Larger grids, and shapes where the split would not pay, run exactly the
 * fa2_fwd / fa2_fwd_strided launch.
 *
 * workspace        device memory for the partials, at least
 *                  fa2_fwd_balanced_workspace_bytes(B, H, S, D, causal)
 *                  bytes, 16-byte aligned, not overlapping any tensor;
 *                  caller-owned, contents on entry ignored. May be NULL when
 *                  that size is 0.
 * workspace_bytes  its size in bytes.
 * Other arguments, the arithmetic and the ownership rules are those of
 * fa2_fwd_strided (strides given) or fa2_fwd (NULL). Results agree with
 * those calls to within rounding: a split row's O is the merge of its
 * chunks' fp32 partials, rounded once. Returns FA2_ERR_WORKSPACE for a
 * missing, misaligned or short workspace (checked after the device, as the
 * split depends on the device's compute units), FA2_ERR_ALIAS for one that
 * overlaps a tensor, otherwise the codes of fa2_fwd / fa2_fwd_strided.
 */
int fa2_fwd_balanced(const void *q, const void *k, const void *v, void *o, float *lse,
                     int B, int H, int S, int D, const long long *strides, int causal,
                     float scale, int dtype, void *workspace, size_t workspace_bytes,
                     void *stream);

/* Workspace bytes fa2_fwd_balanced needs for this shape on the current
 * device: 0 when it runs unsplit, when the arguments are out of range, or
 * when there is no usable device. */
size_t fa2_fwd_balanced_workspace_bytes(int B, int H, int S, int D, int causal);

/* 1 when fa2_fwd has a kernel for head dimension D and dtype, else 0: the
 * head dims 64, 128 and 256 in fp16 or bf16, the support matrix jared-hpc
 * Lecture 6 gives for FlashAttention-2 ("Use it in the real stack") and the
 * infra.bea.ai guide's table ("When V2 Is Used vs Not": head dim up to
 * 256). It lets a caller check a shape up front; the compute entry points
 * refuse anything else on their own, with FA2_ERR_HEADDIM or FA2_ERR_DTYPE. */
int fa2_supported(int D, int dtype);

/* A static, human-readable description of a status code (never NULL; an
 * unknown code gets a generic text). jared-hpc Lecture 6 ("Use it in the
 * real stack") wants an input the kernel cannot serve to end in a visible
 * error, never in a silent switch to another path; every entry point
 * reports such a case as a nonzero status, and this text is what the
 * caller shows for it. */
const char *fa2_status_string(int status);

/* Query rows handled by one workgroup (the tile height B_r along the query
 * sequence) for head dimension D; 0 when D is unsupported. The launch grid
 * is (ceil(S / rows), H, B), the sequence-parallel grid of jared-hpc
 * Lecture 6 ("FA2 change 1") and of the cookbook notebook's Triton launch
 * (one program per (query block, batch * head)). */
int fa2_rows_per_workgroup(int D);

/*
 * Split-KV attention -- the decoding (KV-cache) form: Sq query rows against
 * Sk key rows per head, the queries being the last Sq positions of the
 * sequence. The infra.bea.ai FlashAttention V2 guide lists KV-cache
 * inference as served by a FlashDecoding variant ("When V2 Is Used vs Not");
 * the split of the key range into parts whose (m, l) are combined at the end
 * is jared-hpc Lecture 6's "FA2 change 2", here across workgroups, and the
 * combine is the guide's rescaling algebra ("Optimization 2"):
 *
 *     S_i,j = scale * (q_i . k_j), j kept iff !causal or j <= i + (Sk - Sq)
 *     O_i and lse_i as for fa2_fwd over the kept keys.
 *
 * The keys of each (b, h) are cut into n_split chunks of whole 32-key tiles;
 * one kernel computes each chunk's unnormalised O and its (m, l) into the
 * workspace, a second merges the chunks:
 *     M = max_g m_g,  w_g = exp(m_g - M),
 *     O = sum_g w_g O_g / sum_g w_g l_g,  lse = M + ln(sum_g w_g l_g).
 *
 * q, o     (B, H, Sq, D) contiguous, `dtype`, 16-byte aligned.
 * k, v     (B, H, Sk, D) contiguous, `dtype`, 16-byte aligned.
 * lse      (B, H, Sq) floats, natural log, 4-byte aligned.
 * B, H     1..65535 each.  Sq, Sk >= 1; causal requires Sq <= Sk.
 * D, causal, scale, dtype, stream as for fa2_fwd.
 * n_split  key chunks per (b, h); 0 picks fa2_splitkv_splits(B, H, Sq, Sk).
 *          Chunks that would be empty are dropped.
 * workspace, workspace_bytes
 *          caller-owned device memory, 16-byte aligned, at least
 *          fa2_splitkv_workspace_bytes(B, H, Sq, Sk, D, n_split) bytes. Its
 *          contents on entry are ignored and it is overwritten; it must not
 *          overlap any tensor, and two calls in flight at once need two
 *          workspaces. The library allocates nothing.
 * Returns an fa2_status (FA2_ERR_WORKSPACE for a missing, misaligned or short
 * workspace; FA2_ERR_SHAPE also for causal with Sq > Sk). Two kernels are
 * enqueued on `stream`; the call does not wait for them.
 */
int fa2_fwd_splitkv(const void *q, const void *k, const void *v, void *o, float *lse,
                    int B, int H, int Sq, int Sk, int D, int causal, float scale,
                    int dtype, int n_split, void *workspace,
                    size_t workspace_bytes, void *stream);

/*
 * fa2_fwd_splitkv_fp8 -- fa2_fwd_splitkv with K and V in FP8: a KV cache of
 * OCP e4m3 codes (1 sign, 4 exponent bits of bias 7, 3 mantissa bits; one
 * byte per element) with one descale per tensor, the element values being
 * code * k_descale and code * v_descale. This is the FP8 direction the
 * infra.bea.ai guide names for FlashAttention-3 ("FlashAttention-3 and
 * Beyond"), taken where MI355X gains from it without rounding anything
 * more: decoding is bound by the bytes of K and V it reads, and FP8 halves
 * them. The codes convert exactly to fp16 or bf16 (q's dtype) on the GPU,
 * so the arithmetic and the result are those of fa2_fwd_splitkv on the
 * dequantized K and V (up to the order of the fp32 sums in q . k).
 *
 * k, v      (B, H, Sk, D) contiguous e4m3 codes, 16-byte aligned. The NaN
 *           codes 0x7f and 0xff make the rows that see them NaN.
 * k_descale, v_descale  finite and > 0 (FA2_ERR_SCALE otherwise).
 * q, o, lse, the other arguments, the workspace (its size does not depend
 * on the element type of K and V) and the return codes are those of
 * fa2_fwd_splitkv; dtype is that of q and o.
 */
int fa2_fwd_splitkv_fp8(const void *q, const void *k, const void *v, void *o, float *lse,
                        int B, int H, int Sq, int Sk, int D, int causal, float scale,
                        float k_descale, float v_descale, int dtype, int n_split,
                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * fa2_fwd_splitkv_strided -- fa2_fwd_splitkv (kv_fp8 = 0) or
 * fa2_fwd_splitkv_fp8 (kv_fp8 = 1, with k_descale and v_descale) on tensors
 * with arbitrary strides, such as a KV cache allocated for a maximum length
 * and read up to the current one, or kept as (B, S, H, D).
 *
 * strides  host pointer to 12 element strides: batch, head and sequence of
 *          q, then of k, v and o (FP8 K and V count bytes). Each stride is
 *          in [0, 2^40]; rows are 16-byte aligned (multiples of 8 elements
 *          for 16-bit tensors, of 16 for FP8 K and V); each sequence stride
 *          is >= D; o's rows must be disjoint. K and V may repeat one head
 *          (head stride 0).
 * lse      contiguous (B, H, Sq) floats. 256 rows of K and of V must span
 *          under 2^31 bytes (256 * sequence stride * element bytes); a head
 *          may span any size.
 * The workspace, the other arguments and the result are those of the
 * contiguous calls, which the strided call reproduces bit for bit.
 * FA2_ERR_STRIDE for bad strides, FA2_ERR_DTYPE for kv_fp8 other than 0 or
 * 1, otherwise the codes of fa2_fwd_splitkv; overlap is judged on the byte
 * range each tensor spans.
 */
int fa2_fwd_splitkv_strided(const void *q, const void *k, const void *v, void *o, float *lse,
                            int B, int H, int Sq, int Sk, int D, const long long *strides,
                            int causal, float scale, int dtype, int kv_fp8, float k_descale,
                            float v_descale, int n_split, void *workspace,
                            size_t workspace_bytes, void *stream);

/*
 * fa2_fwd_splitkv_noalloc -- fa2_fwd_splitkv for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops
 * and harnesses that forbid hipMalloc. It takes no workspace: the partial
 * results of the key chunks go to a scratch array the library holds in
 * device memory for the life of the process, FA2_SCRATCH_BYTES on every GPU
 * it runs on. The call allocates nothing (no hipMalloc, no allocating
 * library routine); on its first call on a device it looks up that
 * device's copy of the array.
 *
 * Arguments, arithmetic, kernels and result are those of fa2_fwd_splitkv
 * with the same n_split (0: the library's default), bit for bit.
 * Returns FA2_ERR_SCRATCH, before anything is launched, when
 * fa2_splitkv_workspace_bytes(B, H, Sq, Sk, D, n_split) for the split count
 * the call takes exceeds FA2_SCRATCH_BYTES; otherwise the codes of
 * fa2_fwd_splitkv (never FA2_ERR_WORKSPACE).
 *
 * Every call on one GPU shares that GPU's scratch, and the array keeps the
 * last call's partials (nothing in it needs to start at zero: every
 * partial the merge reads is written first by the same call). Calls that
 * overlap in time on one GPU -- on two streams, or from two threads
 * without ordering -- race on it; order them on one stream.
 */
#define FA2_SCRATCH_BYTES (16u << 20)
int fa2_fwd_splitkv_noalloc(const void *q, const void *k, const void *v, void *o, float *lse,
                            int B, int H, int Sq, int Sk, int D, int causal, float scale,
                            int dtype, int n_split, void *stream);

/*
 * fa2_fwd_fp8 -- the forward pass of fa2_fwd with Q, K and V in FP8, both
 * products on the FP8 matrix cores (twice the 16-bit rate): the FP8
 * direction the infra.bea.ai FlashAttention V2 guide gives for
 * FlashAttention-3 ("FlashAttention-3 and Beyond").
 *
 * q, k, v   (B, H, S, D) contiguous OCP e4m3 codes (one byte each),
 *           16-byte aligned; element values are code * q_descale,
 *           code * k_descale and code * v_descale.
 * q_descale, k_descale, v_descale  finite and > 0 (FA2_ERR_SCALE).
 * o         (B, H, S, D) contiguous, `dtype` (FA2_F16 or FA2_BF16), the
 *           output's element type only; 16-byte aligned.
 * lse, B, H, S, causal, scale, stream as for fa2_fwd; D is 64, 128 or 256.
 * Ownership, synchronisation and work order (the tickets of a multi-round
 * grid's last workgroups, from the same per-stream counters) as for fa2_fwd.
 *
 * Arithmetic: S = Q K^T and O~ = P V on v_mfma_f32_32x32x64_f8f6f4 (e4m3 x
 * e4m3, fp32 accumulation; the instruction's internal sum is not exact
 * fp32), the online softmax in fp32, and P rounded to e4m3 as
 * 2^(t - m + 6) (t the base-2 logit, m the running reference max, kept
 * within 2.75 of every t so that P stays under e4m3's 448). O is divided
 * by the sum of P as rounded and rounded once to `dtype`; lse comes from
 * the sum of P in fp32. The result therefore differs from exact attention
 * on the dequantized inputs by more than fa2_fwd's does: by at most a
 * forward error bound set by the rounding of P to e4m3 (3 mantissa bits)
 * and the FP8 product's sum, which the tests evaluate per output.
 * Returns the codes of fa2_fwd.
 */
int fa2_fwd_fp8(const void *q, const void *k, const void *v, void *o, float *lse,
                int B, int H, int S, int D, int causal, float scale, float q_descale,
                float k_descale, float v_descale, int dtype, void *stream);

/* Bytes of workspace fa2_fwd_splitkv and fa2_fwd_splitkv_fp8 need for these
 * sizes and n_split; n_split = 0 gives enough for the default split count
 * of either. 0 for invalid sizes or head dims. */
size_t fa2_splitkv_workspace_bytes(int B, int H, int Sq, int Sk, int D, int n_split);

/* The default number of key chunks per (b, h) of fa2_fwd_splitkv: enough
 * workgroups for about two on every compute unit of the current device,
 * each chunk at least four 32-key tiles; 1 for invalid sizes. */
int fa2_splitkv_splits(int B, int H, int Sq, int Sk);

/* The same for fa2_fwd_splitkv_fp8: about four workgroups per compute unit
 * (a chunk of FP8 K and V holds half the bytes). */
int fa2_splitkv_splits_fp8(int B, int H, int Sq, int Sk);

#ifdef __cplusplus
}
#endif

#endif /* FA2_H */
