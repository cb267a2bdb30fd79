/*
 * fa06.h -- C ABI of the MI355X (gfx950) fused attention forward pass.
 *
 * The headline operation, fa_fwd: exact, dense, non-causal scaled-dot-product
 * attention,
 *
 *     O = softmax_row(scale * Q K^T) V,    LSE_i = ln sum_j exp(scale * q_i . k_j)
 *
 * as defined by the score and output equations of "FlashAttention'ı Anlamak
 * Bölüm 1" (section 0.2 "Notasyon"), with the optional mask/bias term absent
 * (the B200 article's scope: dense, non-causal, head size 128, BF16).  It is
 * computed the way the B200 article's section "Kernel işini nasıl
 * bölümlendiriyor" partitions it: one workgroup per tile of output rows, the
 * Q tile loaded once, a loop over K/V tiles with an online softmax, and the
 * output normalised once at the end.  The result is exact up to
 * floating-point order (BF16 inputs, fp32 accumulation, BF16 output).
 *
 * Layout: Q, K, V and O share the [batch, heads, sequence, head_dim] shape
 * of that same section, row-major and contiguous:
 *     Q [B, H, Nq, d]   K [B, H, Nk, d]   V [B, H, Nk, d]   O [B, H, Nq, d]
 *     LSE [B, H, Nq]
 *
 * Around it, each with its own comment below: the mask/bias term
 * (fa_fwd_masked), a value head size apart from the query/key one
 * (fa_fwd_dv), a key split with a log-sum-exp merge for launches with few
 * query tiles (fa_fwd_splitkv), the backward pass by recomputation (fa_bwd,
 * fa_bwd_masked, fa_bwd_dv) and MXFP8 inputs (fa_fwd_mxfp8 and its encoders).
 *
 * No symbol here takes or returns a framework type; every buffer is a plain
 * device pointer.
 */
#ifndef FA06_H
#define FA06_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by fa_fwd. */
typedef enum fa_status {
    FA_OK = 0,
    FA_ERR_NULL_POINTER = 1,  /* a pointer to a non-empty buffer is NULL          */
    FA_ERR_INVALID_SHAPE = 2, /* B, H or Nq negative, Nk < 1, or sizes overflow    */
    FA_ERR_UNSUPPORTED = 3,   /* head size not built, misaligned pointer, N too large */
    FA_ERR_ALIAS = 4,         /* O or LSE overlaps Q, K, V or each other           */
    FA_ERR_INVALID_SCALE = 5, /* scale is NaN or infinite                          */
    FA_ERR_DEVICE = 6,        /* no HIP device, or the current device is not gfx950 */
    FA_ERR_LAUNCH = 7,        /* the kernel launch itself failed                   */
    FA_ERR_WORKSPACE = 8,     /* fa_fwd_splitkv: workspace NULL, too small or misaligned */
    FA_ERR_SCRATCH = 9        /* fa_fwd_splitkv_noalloc: the split needs more than the scratch array */
} fa_status;

/* Head dimension of the headline shape (d = d_v = 128), and the only one the
 * MXFP8 forward (fa_fwd_mxfp8) accepts. */
#define FA_HEAD_DIM 128
/* Largest Nq or Nk accepted (each per-head slice stays below 2 GiB). */
#define FA_MAX_SEQ (1LL << 23)

/*
 * fa_fwd -- fused attention forward.
 *
 *   Q, K, V  device pointers to bf16 bit patterns (uint16), layout above,
 *            16-byte aligned.  Read only.
 *   O        device pointer, bf16 [B, H, Nq, d], 16-byte aligned.  Written:
 *            O = P V with P the row softmax, rounded to nearest even.
 *   LSE      device pointer, fp32 [B, H, Nq], 4-byte aligned.  Written: the
 *            natural-log log-sum-exp of the scaled logits of each query row,
 *            the quantity a backward pass needs to recompute P.
 *   B, H     batch and heads (>= 0).
 *   Nq, Nk   query and key/value sequence lengths: Nq >= 0, Nk >= 1 (the
 *            softmax of an empty row is undefined).  Any value up to
 *            FA_MAX_SEQ; no multiple of a tile size is required.
 *   d        head dimension of Q, K, V and O: 64, 128 (FA_HEAD_DIM, the
 *            tuned case) or 256; anything else returns FA_ERR_UNSUPPORTED.
 *   scale    finite multiplier of Q K^T (1/sqrt(d) for standard attention;
 *            zero and negative values are accepted).
 *   stream   hipStream_t to enqueue on; NULL is the default stream.
 *
 * Ownership: the caller allocates and owns every buffer; the library keeps no
 * pointer after returning and allocates no device memory.
 *
 * Execution: asynchronous on `stream`; the function never synchronises.  The
 * outputs are valid once the caller has synchronised the stream.  It
 * launches one kernel, is reentrant, and calls on different streams may run
 * concurrently.  After one call on a device (which caches its architecture
 * check), calls issue nothing but kernel launches -- no memset, copy or
 * allocation -- so they can be captured in a HIP graph and replayed; the
 * same holds for every entry point of this header.
 *
 * Errors: arguments are validated before any HIP call, shapes first, then
 * pointers (a pointer may be NULL only when its buffer holds zero bytes, as
 * frameworks hand out for empty tensors); on a non-zero return nothing is
 * launched and O and LSE are untouched.  B*H*Nq == 0 is a no-op
 * returning FA_OK.  NaN or Inf inside the inputs is not checked and
 * propagates as IEEE arithmetic does.  Faults during execution surface at the
 * caller's next synchronisation of the stream.
 */
int fa_fwd(const void *Q, const void *K, const void *V, void *O, float *LSE,
           int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
           float scale, void *stream);

/*
 * fa_fwd_masked -- fa_fwd with the optional mask/bias term of the score
 * equation ("FlashAttention'ı Anlamak Bölüm 1", section 0.2: S = Q K^T / sqrt(d)
 * + B).
 *
 *   causal   0 or 1.  With 1, key j is hidden from query i when
 *            j > i + (Nk - Nq): the diagonal is aligned to the last query and
 *            the last key (for Nq = Nk, row i sees keys 0..i).  Key tiles that
 *            lie entirely past a query tile's diagonal are skipped.
 *   bias     NULL (no bias), or a device pointer to an fp32 additive bias,
 *            added to scale * q_i . k_j (natural-log units) before the
 *            softmax; element (b, h, i, j) is bias[b*bias_stride_b +
 *            h*bias_stride_h + i*bias_stride_q + j] (element strides; a zero
 *            stride broadcasts over that dimension; keys are contiguous).  A
 *            -inf entry hides its key.  Read only; it may alias Q, K or V but
 *            not O or LSE (FA_ERR_ALIAS).  Requirements, else
 *            FA_ERR_UNSUPPORTED: the pointer is 16-byte aligned, the three
 *            strides are >= 0 and multiples of 4, and 31*bias_stride_q + Nk +
 *            128 <= 2^29 (32 consecutive rows are addressed with 32-bit byte
 *            offsets).  An extent (B-1)*sb + (H-1)*sh + (Nq-1)*sq + Nk above
 *            2^60 elements returns FA_ERR_INVALID_SHAPE.  With bias == NULL
 *            the strides are ignored.
 *   A row that sees no key (causal with Nq > Nk, or -inf bias on every key
 *   it could see) gets O = 0 and LSE = -inf.
 *   other arguments, ownership, execution and errors as for fa_fwd; a causal
 *   value other than 0 or 1 returns FA_ERR_UNSUPPORTED.
 */
int fa_fwd_masked(const void *Q, const void *K, const void *V, void *O, float *LSE,
                  int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale,
                  int causal, const float *bias, int64_t bias_stride_b, int64_t bias_stride_h,
                  int64_t bias_stride_q, void *stream);

/*
 * fa_fwd_dv -- fa_fwd_masked with a value head size d_v that may differ from
 * the query/key head size d ("FlashAttention'ı Anlamak Bölüm 1", section 0.2
 * gives V and O their own width d_v; the scale of the score equation divides
 * by sqrt(d), the query/key width).
 *
 *   Q [B, H, Nq, d], K [B, H, Nk, d]   bf16, as for fa_fwd.
 *   V [B, H, Nk, dv]                    bf16.
 *   O [B, H, Nq, dv]                    bf16, written.
 *   d, dv    (d, dv) one of (64, 64), (128, 128), (256, 256) -- the same
 *            kernels as fa_fwd_masked -- or (192, 128), the query/key and
 *            value widths of multi-head latent attention's prefill; other
 *            pairs return FA_ERR_UNSUPPORTED.  Nq and Nk are limited to
 *            min(FA_MAX_SEQ, 2^30 / max(d, dv)).
 *   every other argument, ownership, execution and errors as for
 *   fa_fwd_masked (the alias checks use each buffer's own extent).
 */
int fa_fwd_dv(const void *Q, const void *K, const void *V, void *O, float *LSE,
              int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int64_t dv, float scale,
              int causal, const float *bias, int64_t bias_stride_b, int64_t bias_stride_h,
              int64_t bias_stride_q, void *stream);

/*
 * fa_fwd_splitkv -- fa_fwd_dv with the keys of every (batch, head) split into
 * ranges that separate workgroups attend to, then merged.  For launches with
 * few query tiles (short Nq, few heads: fewer than two workgroups per CU),
 * where one workgroup per query tile leaves the chip idle.  Each range
 * yields the normalised output O_s and log-sum-exp L_s of its keys alone
 * (the online softmax of "FlashAttention'ı Anlamak Bölüm 1", section 0, run
 * on a contiguous part of the keys); a second kernel combines them as that
 * recurrence combines two blocks: LSE = ln sum_s exp(L_s),
 * O = sum_s exp(L_s - LSE) O_s.  The result equals fa_fwd_dv's up to
 * floating-point order (the ranges' outputs stay fp32 until the merge).
 *
 *   n_splits         number of key ranges: 0 lets the library choose (enough
 *                    ranges for 512 workgroups, each range >= 512 keys; 1
 *                    when the launch is already large), >= 1 asks for that
 *                    many (cut to one range per 64 keys).  Ranges are equal
 *                    multiples of 64 keys, the last one shorter.  0..1024,
 *                    else FA_ERR_UNSUPPORTED.
 *   workspace        device memory the call may overwrite, 16-byte aligned,
 *                    of at least fa_fwd_splitkv_workspace_bytes(...) bytes,
 *                    not overlapping any other buffer (FA_ERR_ALIAS); owned by
 *                    the caller and free to reuse once the stream has passed
 *                    the call.  May be NULL when that size is 0 (one range:
 *                    the call then is fa_fwd_dv).  Otherwise NULL, too small
 *                    or misaligned returns FA_ERR_WORKSPACE.
 *   workspace_bytes  its size.
 *   every other argument, ownership, execution and errors as for fa_fwd_dv;
 *   with more than one range, Nq * dv * 4 must stay below 2^31 and B*H*Nq
 *   below 2^33 (else FA_ERR_UNSUPPORTED).  Two kernels are enqueued.
 */
int fa_fwd_splitkv(const void *Q, const void *K, const void *V, void *O, float *LSE,
                   int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int64_t dv, float scale,
                   int causal, const float *bias, int64_t bias_stride_b, int64_t bias_stride_h,
                   int64_t bias_stride_q, int64_t n_splits, void *workspace, int64_t workspace_bytes,
                   void *stream);

/*
 * fa_fwd_splitkv_noalloc -- fa_fwd_splitkv for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid hipMalloc): the ranges' partial outputs and log-sum-exps go to
 * a scratch array inside the library instead of a caller workspace.
 *
 *   every argument as for fa_fwd_splitkv, without workspace and
 *   workspace_bytes.
 *
 * Scratch: a static device array of fa_fwd_splitkv_noalloc_max_bytes()
 * bytes (48 MiB); each device that loads the library's forward kernels holds
 * its own copy until the process ends.  Its address on a device is looked up
 * on the first call made with that device current.  The call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine).  A plan
 * that needs more than the array holds (fa_fwd_splitkv_workspace_bytes above
 * the maximum) returns FA_ERR_SCRATCH and launches nothing; the caller may
 * ask for fewer ranges.  The array is not cleared: the split kernel writes
 * every partial row the merge reads.
 * Concurrency: every call on one device shares that device's array, which
 * keeps the last call's contents.  Calls that overlap in time on one device
 * (two streams, or two host threads without ordering) race on it and give
 * undefined results; calls ordered on one stream are safe.
 * Errors as for fa_fwd_splitkv, with FA_ERR_WORKSPACE replaced by
 * FA_ERR_SCRATCH; FA_ERR_DEVICE also when the array's address cannot be
 * obtained.
 */
int fa_fwd_splitkv_noalloc(const void *Q, const void *K, const void *V, void *O, float *LSE,
                           int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int64_t dv, float scale,
                           int causal, const float *bias, int64_t bias_stride_b, int64_t bias_stride_h,
                           int64_t bias_stride_q, int64_t n_splits, void *stream);

/* fa_fwd_splitkv_noalloc_max_bytes -- size of its scratch array in bytes. */
int64_t fa_fwd_splitkv_noalloc_max_bytes(void);

/*
 * fa_fwd_splitkv_workspace_bytes -- the workspace fa_fwd_splitkv needs for
 * these sizes and n_splits (same meaning as there): n_splits * B * H * Nq *
 * (4 * dv + 4) bytes for the ranges' fp32 outputs and log-sum-exps, 0 when
 * the plan has one range.  Writes the number of ranges the plan uses to
 * *n_splits_used (may be NULL).  Host-only arithmetic, no HIP call.
 * Returns a negative fa_status on invalid sizes (B, H, Nq < 0, Nk < 1,
 * dv outside 1..256, n_splits outside 0..1024, Nq or Nk above FA_MAX_SEQ).
 */
int64_t fa_fwd_splitkv_workspace_bytes(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t dv,
                                       int64_t n_splits, int64_t *n_splits_used);

/*
 * fa_bwd -- gradients of a scalar loss L through the attention output, given
 * dO = dL/dO, by recomputing the attention matrix from the forward pass's
 * log-sum-exp (the recomputation of "FlashAttention'ı Anlamak Bölüm 1",
 * section 0; the gradients are the chain rule of the score and output
 * equations of section 0.2).  Per head and query row i:
 *     P_ij = exp(scale q_i.k_j - LSE_i) (0 for keys hidden by the causal mask),
 *     dV_j = sum_i P_ij dO_i,  dP_ij = dO_i . v_j,  D_i = dO_i . O_i,
 *     dS_ij = P_ij (dP_ij - D_i),  dQ_i = scale sum_j dS_ij k_j,
 *     dK_j = scale sum_i dS_ij q_i.
 *
 *   Q, K, V  device, bf16 [B, H, Nq|Nk, d], the forward pass's inputs.
 *   O, LSE   device, the forward pass's outputs for the same inputs, scale
 *            and causal flag (bf16 [B, H, Nq, d]; fp32 [B, H, Nq]).
 *   dO       device, bf16 [B, H, Nq, d].
 *   dQ, dK, dV  device, bf16 outputs shaped like Q, K, V (written, not
 *            accumulated into).
 *   D        device, fp32 [B, H, Nq] workspace owned by the caller; receives
 *            D_i = dO_i . O_i.
 *   B, H, Nq, Nk, scale, causal, stream  as for fa_fwd_masked (no bias).
 *   d        64, 128 (FA_HEAD_DIM) or 256; other values return
 *            FA_ERR_UNSUPPORTED.  At 256 the kernels need more registers
 *            than one wave holds: dK and dV are computed by one launch each
 *            and dQ by one launch per half of its columns (five kernels in
 *            all, recomputing S and dP), with or without a bias.
 *
 * Requirements and errors as for fa_fwd; every pointer must be 16-byte
 * aligned except LSE and D (4 bytes); an output (dQ, dK, dV, D) that overlaps
 * an input or another output returns FA_ERR_ALIAS.  B*H == 0 is a no-op; with
 * Nq == 0, dK and dV are written as zeros.  The call enqueues three kernels
 * on `stream` (five at head size 256) and is deterministic (no atomics).
 */
int fa_bwd(const void *Q, const void *K, const void *V, const void *O, const void *dO,
           const float *LSE, void *dQ, void *dK, void *dV, float *D,
           int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale,
           int causal, void *stream);

/*
 * fa_bwd_masked -- fa_bwd for a forward pass that had an additive bias (the
 * mask term of the score equation, "FlashAttention'ı Anlamak Bölüm 1",
 * section 0.2): P_ij = exp(scale q_i.k_j + b_ij - LSE_i); the gradient
 * equations of fa_bwd are otherwise unchanged.  No gradient of the bias is
 * formed.
 *
 *   bias, bias_stride_b, bias_stride_h, bias_stride_q
 *            the fp32 bias and element strides the forward pass
 *            (fa_fwd_masked) used, with its rules (16-byte aligned base,
 *            strides >= 0 and multiples of 4, -inf hides a key; it may alias
 *            the inputs but not dQ, dK, dV or D: FA_ERR_ALIAS), plus one
 *            more: (Nq - 1) * bias_stride_q + Nk + 128 <= 2^29 (a key's
 *            column over all query rows is addressed with 32-bit byte
 *            offsets), else FA_ERR_UNSUPPORTED.  NULL: the call is fa_bwd.
 *   A query row that saw no key (LSE = -inf) gets dQ = 0 and adds nothing
 *   to dK and dV.
 *   every other argument, ownership, execution and errors as for fa_bwd.
 */
int fa_bwd_masked(const void *Q, const void *K, const void *V, const void *O, const void *dO,
                  const float *LSE, void *dQ, void *dK, void *dV, float *D,
                  int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale,
                  int causal, const float *bias, int64_t bias_stride_b, int64_t bias_stride_h,
                  int64_t bias_stride_q, void *stream);

/*
 * fa_bwd_dv -- fa_bwd_masked for a forward pass with value head size d_v
 * apart from the query/key head size d (fa_fwd_dv's shapes): Q, K, dQ, dK
 * [.., d], V, O, dO, dV [.., dv].  (d, dv) is (64, 64), (128, 128),
 * (256, 256) or (192, 128); other pairs return FA_ERR_UNSUPPORTED.  Nq and Nk are limited
 * to min(FA_MAX_SEQ, 2^30 / max(d, dv)).  bias may be NULL.  Every other
 * argument, ownership, execution and errors as for fa_bwd_masked (the alias
 * checks use each buffer's own extent).
 */
int fa_bwd_dv(const void *Q, const void *K, const void *V, const void *O, const void *dO,
              const float *LSE, void *dQ, void *dK, void *dV, float *D,
              int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int64_t dv, float scale,
              int causal, const float *bias, int64_t bias_stride_b, int64_t bias_stride_h,
              int64_t bias_stride_q, void *stream);

/*
 * MXFP8 attention.  The forward pass of fa_fwd_masked (no bias) on inputs in
 * the OCP microscaling format MXFP8: E4M3 elements, and one E8M0 scale byte
 * (value 2^(s-127); s = 255 is NaN) per block of 32 elements along the
 * contraction axis of each product -- along the head dimension for Q and K,
 * along the keys for V, which is therefore passed transposed.  The pages
 * name MXFP8 attention as the aim of their kernel work ("Flash Attention на
 * 5090 в CUDA C++": motivation, "Что дальше") without defining it; the
 * format is the OCP one.  Head size 128 only.
 *
 * fa_fwd_mxfp8 -- device buffers, u8 unless stated:
 *   Q8 [B,H,Nq,128] E4M3 and Qs [B,H,Nq,4] E8M0 (Qs 4-byte aligned);
 *   K8 [B,H,Nk,128] E4M3 and Ks [B,H,ldv,4] E8M0 (rows >= Nk unused);
 *   Vt8 [B,H,128,ldv] E4M3, V transposed, keys >= Nk holding finite values
 *     (zeros); Vs [B,H,ldv/32,128] E8M0, Vs[b,h,j,c] scaling keys
 *     32j..32j+31 of column c;
 *   O [B,H,Nq,128] bf16 and LSE [B,H,Nq] fp32 as for fa_fwd;
 *   ldv: multiple of 64, Nk <= ldv <= 2^24.
 * The kernel computes S on the block-scaled MFMA, P in fp32, rounds P to
 * E4M3 (scale 1) for the P V product and normalises by the fp32 row sum.
 * Every pointer 16-byte aligned except Qs and LSE (4); errors and execution
 * as for fa_fwd_masked.
 */
int fa_fwd_mxfp8(const void *Q8, const void *Qs, const void *K8, const void *Ks, const void *Vt8,
                 const void *Vs, void *O, float *LSE, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                 int64_t d, int64_t ldv, float scale, int causal, void *stream);

/*
 * fa_mxfp8_quantize_rows -- bf16 X [B,H,N,128] to MXFP8 along the last axis:
 * E [B,H,N,128] E4M3 and S [B,H,ldS,4] E8M0 (ldS >= N; for K pass ldS = ldv).
 * Each block of 32 gets the scale 2^(floor(log2 max|x|) - 8) (2^-127 for an
 * all-zero block); elements are x / scale rounded to the nearest E4M3 value
 * (ties to even), magnitudes above 448 saturating.  X and E 16-byte aligned.
 *
 * fa_mxfp8_quantize_vt -- bf16 V [B,H,Nk,128] to the V^T layout of
 * fa_fwd_mxfp8: Vt [B,H,128,ldv] (keys >= Nk written as zeros) and
 * Vs [B,H,ldv/32,128], blocks of 32 keys per column, same rules.  ldv a
 * multiple of 64, Nk <= ldv <= 2^24; Vt 16-byte aligned.
 *
 * Both enqueue one kernel on `stream`; errors as for fa_fwd.
 */
int fa_mxfp8_quantize_rows(const void *X, void *E, void *S, int64_t B, int64_t H, int64_t N, int64_t d,
                           int64_t ldS, void *stream);
int fa_mxfp8_quantize_vt(const void *V, void *Vt, void *Vs, int64_t B, int64_t H, int64_t Nk, int64_t d,
                         int64_t ldv, void *stream);

/* fa_status_string -- static, NUL-terminated description of a status code. */
const char *fa_status_string(int status);

/* fa_build_info -- static string naming the forward kernel's tile configuration. */
const char *fa_build_info(void);

/* fa_bwd_build_info -- static string naming the backward kernels' configuration. */
const char *fa_bwd_build_info(void);

/* fa_mxfp8_build_info -- static string naming the MXFP8 kernel's configuration. */
const char *fa_mxfp8_build_info(void);

#ifdef __cplusplus
}
#endif

#endif /* FA06_H */
