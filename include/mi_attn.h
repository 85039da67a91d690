/*
 * mi_attn.h - C ABI of libmi_attn, a fused attention forward (and its
 * gradients) for MI355X (gfx950).
 *
 * The operation (sources: "[GPU] Deep Learning for HPC", section "Flash
 * Attention" - scores Q K^T, softmax, times V, computed tile by tile without
 * writing the score matrix out; null-ptr.tistory.com, category "development",
 * the Triton FlashAttention post - a forward kernel taking Q, K, V, a softmax
 * scale and a causal flag and writing Out and Lse), for every batch b, head h
 * and query row i:
 *
 *     s_ij   = scale * sum_t q_it * k_jt          for visible keys j
 *     o_i    = sum_j exp(s_ij) v_j / sum_j exp(s_ij)
 *     lse_i  = ln sum_j exp(s_ij)                 (natural log, scaled scores)
 *
 * where every key is visible when causal == 0, and key j is visible to query i
 * iff j <= i when causal != 0. Masked keys carry weight exactly zero.
 *
 * All calls are thread-safe, allocate nothing, never print and never abort.
 * None keeps state between calls, except that attn_bwd_noalloc keeps its
 * static device buffer (and the address it looked up) for the process.
 */
#ifndef MI_ATTN_H
#define MI_ATTN_H

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. Every entry point returns one; 0 is success. */
typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = -1,      /* a required pointer (q, k, v, o, lse, or an out-param) is NULL */
  ATTN_ERR_SHAPE = -2,     /* a size is negative, or one head (N*d*2 bytes) reaches 2^31 */
  ATTN_ERR_HEADDIM = -3,   /* d is not one of 32, 64, 96, 128, 256 */
  ATTN_ERR_ALIGN = -5,     /* q, k, v or o not 16-byte aligned, or lse not 4-byte aligned */
  ATTN_ERR_ALIAS = -6,     /* o or lse overlaps an input, or o overlaps lse */
  ATTN_ERR_SCALE = -7,     /* scale is NaN or infinite */
  ATTN_ERR_LAUNCH = -8,    /* the HIP launch failed (no gfx950 device, bad stream, ...) */
  ATTN_ERR_DTYPE = -9,     /* dtype is not an attn_dtype value */
  ATTN_ERR_SCRATCH = -10   /* attn_bwd_noalloc: B*H*Nq exceeds its static buffer */
} attn_status;

/* Element type of q, k, v and o (attn_fwd_ex). lse is always float32. */
typedef enum {
  ATTN_BF16 = 0,  /* bfloat16: 8-bit exponent, 8-bit significand */
  ATTN_F16 = 1    /* IEEE binary16: 5-bit exponent, 11-bit significand */
} attn_dtype;

/*
 * attn_fwd - attention forward with per-row log-sum-exp.
 *
 *   q, k, v  device pointers to bf16 tensors [B, H, N, d], contiguous row-major
 *            (d fastest, then N, then H, then B). Read only.
 *   o        device pointer to a bf16 tensor [B, H, N, d], same layout; written.
 *   lse      device pointer to a float32 tensor [B, H, N]; written.
 *   B, H, N  batch size, heads, sequence length (queries and keys share N).
 *            Any N >= 1 is accepted (no multiple-of-tile restriction). If
 *            B*H*N == 0 the call does nothing and returns ATTN_OK.
 *   d        head dimension: 32, 64, 96, 128 or 256.
 *   scale    softmax scale, applied to Q K^T before masking; used exactly as
 *            the given float32 value. Any finite value (0 and negative
 *            included) is accepted. The scaled scores are formed in float32
 *            (times log2 e): where |scale * q_i . k_j| * log2 e exceeds the
 *            float32 range the outputs are unspecified, and lse, a float32,
 *            carries a rounding error relative to its own magnitude.
 *   causal   0: every key visible. Non-zero: key j visible to query i iff j <= i.
 *   stream   hipStream_t to launch on; NULL means the null stream.
 *
 * Ownership: the caller allocates and frees every buffer; all device pointers
 * must belong to the current device. The call is asynchronous: it only queues
 * one kernel on `stream` and returns; the caller synchronises before reading
 * o and lse. Arithmetic: bf16 products accumulated in fp32, the softmax
 * weights rounded to bf16 before the P*V product, o rounded to bf16 (nearest
 * even), lse in fp32. Results are deterministic (no atomics).
 *
 * Errors: arguments are validated before any HIP call. On a validation error
 * nothing is launched and o, lse are untouched. ATTN_ERR_LAUNCH reports the
 * status of the launch itself. With NaN or Inf inside q, k or v the outputs
 * are unspecified.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int N, int d, float scale, int causal, void* stream);

/*
 * attn_fwd_cross - attention forward with Nq queries against Nk keys.
 *
 * The same operation as attn_fwd where queries and keys have their own
 * lengths (cross attention, or a block of new queries against a longer key
 * history). Shapes: q and o [B, H, Nq, d], k and v [B, H, Nk, d], lse
 * [B, H, Nq]; layouts, dtypes, scale, stream, ownership and errors as for
 * attn_fwd, with attn_fwd(..., N, ...) == attn_fwd_cross(..., N, N, ...).
 *
 * causal != 0 aligns the two axes at their ends: query i sits at position
 * i + (Nk - Nq) on the key axis and sees keys j <= i + (Nk - Nq). When
 * Nq > Nk the first Nq - Nk queries therefore see no key; such a row (and
 * every row when Nk == 0) gets o = 0 and lse = -inf. k and v may be NULL when
 * Nk == 0. If B*H*Nq == 0 the call does nothing and returns ATTN_OK.
 */
int attn_fwd_cross(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int Nq, int Nk, int d, float scale, int causal,
                   void* stream);

/*
 * attn_fwd_ex - attn_fwd_cross with the element type of q, k, v and o chosen
 * by `dtype` (an attn_dtype: ATTN_BF16 or ATTN_F16; anything else returns
 * ATTN_ERR_DTYPE before any HIP call). With ATTN_F16 the softmax weights are
 * rounded to fp16 before the P*V product and o is written in fp16 (nearest
 * even); everything else is as for attn_fwd_cross.
 * attn_fwd_cross(...) == attn_fwd_ex(..., d, ATTN_BF16, scale, causal, stream).
 */
int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                int B, int H, int Nq, int Nk, int d, int dtype, float scale, int causal,
                void* stream);

/*
 * attn_bwd - gradients of the attention forward: dq, dk, dv of the loss
 * sum(d_o * o) for o = attn_fwd_ex(q, k, v, ..., scale, causal).
 *
 * The pages print no backward pass ("GPUの爆発的な性能向上": the Hacker News
 * comments call it much harder than the forward); this is the chain rule of
 * the forward definition above. With p_ij = exp(s_ij - lse_i) the softmax
 * weights (0 for masked keys) and D_i = sum_c d_o_ic * o_ic:
 *
 *     dv_j  = sum_i p_ij d_o_i
 *     ds_ij = p_ij (d_o_i . v_j - D_i)
 *     dq_i  = scale * sum_j ds_ij k_j
 *     dk_j  = scale * sum_i ds_ij q_i
 *
 * (D_i equals sum_j p_ij (d_o_i . v_j) because o_i = sum_j p_ij v_j.)
 *
 *   q, k, v   inputs of the forward: [B, H, Nq, d], [B, H, Nk, d], [B, H, Nk, d].
 *   o, lse    the forward's outputs for exactly these q, k, v, scale, causal
 *             ([B, H, Nq, d] and float32 [B, H, Nq]); p is recomputed from
 *             lse, so an lse from other inputs gives meaningless gradients.
 *             A row with lse = -inf (it saw no key) has p = 0.
 *   d_o       upstream gradient [B, H, Nq, d].
 *   dq        [B, H, Nq, d]; dk, dv [B, H, Nk, d]; written, every element.
 *   delta     float32 [B, H, Nq], caller-owned; receives D_i (the first kernel
 *             the call queues writes it, a later one reads it back).
 *   B, H, Nq, Nk, d, dtype, scale, causal, stream: as for attn_fwd_ex (d is
 *             32, 64, 96, 128 or 256).
 *
 * All tensors are contiguous row-major in the element type `dtype` (delta and
 * lse float32). Arithmetic: products of the element type accumulated in fp32;
 * p and ds rounded to the element type before the products that consume them;
 * dq, dk, dv rounded to the element type (nearest even). No atomics: results
 * are deterministic.
 *
 * Ownership and errors: as for attn_fwd. Pointers of a side with no rows may
 * be NULL (Nq == 0: q, o, lse, d_o, dq, delta; Nk == 0: k, v, dk, dv); with
 * Nq == 0, dk and dv are written as zeros; with Nk == 0, dq is zeros. dq, dk,
 * dv and delta must not overlap any input or each other (ATTN_ERR_ALIAS).
 * Alignment: 16 bytes for the element-type tensors, 4 for lse and delta. If
 * B*H == 0 or Nq == Nk == 0 the call does nothing and returns ATTN_OK.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* d_o, void* dq, void* dk, void* dv, float* delta, int B, int H,
             int Nq, int Nk, int d, int dtype, float scale, int causal, void* stream);

/*
 * attn_bwd_noalloc - attn_bwd without the `delta` workspace, for callers that
 * cannot allocate device memory (code under stream capture, tight serving
 * loops, harnesses that forbid allocation).
 *
 * Arguments, results and errors are those of attn_bwd with `delta` left out:
 * the row sums D_i go to a static device buffer of the library instead, room
 * for B*H*Nq <= 4194304 rows (16 MiB, reserved on each device the library
 * runs on until the process ends). Larger problems return ATTN_ERR_SCRATCH
 * before any HIP call. The call allocates nothing: on its first call on a
 * device (the current one) it looks up that device's address of the buffer;
 * if the runtime cannot give it the call returns ATTN_ERR_LAUNCH.
 *
 * Every call on one device shares that device's buffer. Calls that may run
 * at the same time on one device (different streams, or different host
 * threads without ordering) race on it and give undefined gradients;
 * serialise them, e.g. on one stream. The buffer needs no clearing: each call
 * writes the rows it reads before reading them, in stream order. Results are
 * bit-identical to attn_bwd's.
 */
int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                     const float* lse, const void* d_o, void* dq, void* dk, void* dv, int B,
                     int H, int Nq, int Nk, int d, int dtype, float scale, int causal,
                     void* stream);

/* attn_strerror - static, NUL-terminated description of a status code
 * (an unknown code yields "unknown status"). Never NULL. */
const char* attn_strerror(int status);

/*
 * attn_fwd_launch_shape - the launch attn_fwd would make for these sizes,
 * without launching: workgroups in the 1-D grid, threads per workgroup, LDS
 * bytes per workgroup, query rows per workgroup (block_m) and keys per inner
 * step (block_n). The workgroup shape depends on the grid: bigger
 * workgroups (256 query rows in 512 threads, or at d = 64, 96 and 128 512 rows)
 * when B, H and N still give every CU enough of them (at d = 64 also only
 * when N >= 4096). Out-params may
 * not be NULL. Returns the same validation
 * status attn_fwd would for the sizes (pointers are not examined); on error
 * the out-params are untouched. For B*H*N == 0 it returns ATTN_OK with
 * *grid == 0.
 */
int attn_fwd_launch_shape(int B, int H, int N, int d, int causal, int* grid,
                          int* block, int* lds_bytes, int* block_m, int* block_n);

#ifdef __cplusplus
}
#endif

#endif /* MI_ATTN_H */
