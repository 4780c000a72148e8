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
    FA2_ERR_SHAPE = 2,     /* B, H or S < 1, H or B > 65535, or B*H*S*D overflows int64 */
    FA2_ERR_HEADDIM = 3,   /* D is not 64, 128 or 256 */
    FA2_ERR_DTYPE = 4,     /* dtype is not FA2_F16 or FA2_BF16 */
    FA2_ERR_ALIGN = 5,     /* q, k, v, o not 16-byte aligned, or lse not 4-byte aligned */
    FA2_ERR_SCALE = 6,     /* scale is negative, NaN or infinite */
    FA2_ERR_NO_DEVICE = 7, /* no current HIP device, or the device is not gfx950 */
    FA2_ERR_LAUNCH = 8,    /* the HIP runtime reported an error at launch */
    FA2_ERR_ALIAS = 9      /* o or lse overlaps q, k or v, or o overlaps lse */
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
 * scale    multiplies q . k before the mask and the softmax; finite and
 *          >= 0. Callers that want the usual default pass 1/sqrt(D).
 * dtype    FA2_F16 or FA2_BF16 (applies to q, k, v and o).
 * stream   a hipStream_t (NULL = the default stream) on the current device.
 *
 * Ownership: the caller owns every buffer; the library allocates nothing,
 * keeps no per-call state and is safe to call from several threads.
 * Synchronisation: the work is enqueued on `stream` and the call returns
 * without waiting for it. o and lse must not overlap q, k, v or each other.
 * Arithmetic: products on fp16/bf16 matrix cores with fp32 accumulation;
 * the softmax state (running max, running sum, unnormalised O) is fp32; O
 * is rounded once, to nearest even, into `dtype`.
 */
int fa2_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
            int B, int H, int S, int D, int causal, float scale, int dtype,
            void *stream);

/* 1 when fa2_fwd has a kernel for head dimension D and dtype, else 0. */
int fa2_supported(int D, int dtype);

/* A static, human-readable description of a status code. */
const char *fa2_status_string(int status);

/* Queries rows handled by one workgroup (the tile height along the query
 * sequence) for head dimension D; 0 when D is unsupported. The launch grid
 * is (ceil(S / rows), H, B). */
int fa2_rows_per_workgroup(int D);

#ifdef __cplusplus
}
#endif

#endif /* FA2_H */
