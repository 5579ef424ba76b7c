/*
 * libs2attn — Shifted Sparse Attention (S2-Attn) forward and backward on AMD
 * MI355X (gfx950).  C ABI: plain device pointers, sizes and a HIP stream.
 *
 * The operation.  Page "LongLoRA: Efficient Fine-tuning of Long-Context Large
 * Language Models" (paper-graph-ui summary), section 3.4:
 *   - "The core computational problem": per head, o = softmax(q k^T) v under a
 *     causal mask.  The scale is 1/sqrt(d) (the page omits it).
 *   - "The solution: group tokens and compute attention locally": the N tokens
 *     form N/G groups of G consecutive tokens; attention stays inside a group.
 *   - "The shifting mechanism" (Steps 1-3, Figure 3) and "Algorithmic
 *     implementation" (Algorithm 1): the last `shift_heads` heads see their
 *     tokens rolled by -G/2 along the sequence before grouping (rolled position
 *     j holds token (j + G/2) mod N); their output is rolled back by +G/2.
 *     Causality holds in the rolled order, so in a shifted head the last group
 *     holds tokens N-G/2..N-1 followed by tokens 0..G/2-1.
 *   - Grouped-query attention (not on the pages): query head h reads key/value
 *     head h / (H / Hkv); dk and dv sum over the query heads sharing them.
 *   - Group sizes that do not divide the sequence (section 5, "Ablation
 *     Studies and Robustness Checks", Table 7's 1/6 group; the pages do not say
 *     how it was cut): the rolled sequence is cut into consecutive groups of G
 *     tokens, the last one holding the N mod G tokens left; for odd G the shift
 *     is floor(G/2).
 * The roll is never materialised: it is folded into the row addresses of every
 * tile load and store, so all tensors stay in original token order.
 *
 * Tensors (all device memory, contiguous, token-major, 16-byte aligned,
 * allocated and freed by the caller; element type given by `dtype`):
 *   q, o, dO, dq : [B, N, H,   d]
 *   k, v, dk, dv : [B, N, Hkv, d]
 *   lse          : [B, H, N] float32, natural-log softmax normaliser of every
 *                  query row, in original token order (written by the
 *                  forward, read by the backward).
 * Outputs are fully overwritten (never accumulated into) and must not alias an
 * input.  Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 * stream); the library never allocates, frees or synchronises.  Errors raised
 * while kernels run surface at the caller's next synchronisation, as for any
 * HIP call.  Apart from s2attn_bwd_noalloc's scratch array (below: one device
 * array per GPU and its address, looked up once per device under a
 * std::call_once), the library holds no state, so every call is reentrant and
 * may run from any host thread.
 *
 * Supported: d in {64, 128}; dtype bf16 (fp32 accumulation, P and dS rounded
 * to bf16 for the matrix cores) or fp32 (fp32 matrix cores throughout);
 * 1 <= G <= N.  bf16 runs one family of kernels laid out for the bf16 matrix
 * cores at every size and G (groups that are not whole 128-row tiles take
 * instantiations that address rows one by one near group ends); fp32 runs
 * kernels on the fp32 matrix cores.  Every wrap option runs on every shape.
 * A key/value head shared by shifted and unshifted query heads (H -
 * shift_heads not a multiple of H / Hkv) sees its keys in two frames G/2
 * apart; unless the groups are whole 128-row tiles and G a multiple of 256
 * (then both frames cut the keys into the same tiles), dk and dv take two
 * passes, the first leaving fp32 sums in the workspace for the second.
 * Grids: B * H * ceil(N / G) * ceil(G / 128) < 2^31;
 * one token row of q: H * d < 2^24 elements.
 * B == 0 or N == 0 is an empty problem: every call validates the other sizes,
 * then returns S2ATTN_OK without reading any pointer or touching the GPU.
 */
#ifndef S2ATTN_H
#define S2ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    S2ATTN_BF16 = 0,   /* bfloat16 storage, fp32 accumulation */
    S2ATTN_F32 = 1     /* float32 storage and arithmetic */
} s2attn_dtype;

typedef enum {
    S2ATTN_OK = 0,
    S2ATTN_ERR_NULL = 1,         /* a required pointer is NULL */
    S2ATTN_ERR_SHAPE = 2,        /* B or N < 0, H, Hkv, d or G <= 0, G > N (N > 0),
                                    shift_heads outside [0, H], H % Hkv != 0 */
    S2ATTN_ERR_UNSUPPORTED = 3,  /* d not in {64,128}, unknown dtype or wrap option, or the grid
                                    or H * d size limit */
    S2ATTN_ERR_HIP = 4,          /* a kernel launch failed (hipGetLastError) */
    S2ATTN_ERR_WORKSPACE = 5,    /* workspace NULL or smaller than s2attn_bwd_workspace_bytes() */
    S2ATTN_ERR_ALIGN = 6,        /* an element tensor pointer not 16-byte aligned, or lse not 4-byte */
    S2ATTN_ERR_SCRATCH = 7       /* s2attn_bwd_noalloc: B * H * N above S2ATTN_NOALLOC_MAX_ROWS */
} s2attn_status;

/*
 * Wrap handling of the shifted heads (the `wrap` argument of the _ex calls).
 *   S2ATTN_WRAP_ROLL  : the method described above (Algorithm 1): a shifted
 *                       head's last rolled group is tokens N-G/2..N-1 followed
 *                       by tokens 0..G/2-1, one causal group.
 *   S2ATTN_WRAP_SPLIT : Variant 2 of Table 8 / Figure 6 (page section 5,
 *                       "Ablation Studies and Robustness Checks"; section 3.4,
 *                       "Information leakage considerations"): the tokens the
 *                       roll carries from the front form a group of their own,
 *                       so that last rolled group is cut at G/2 into two causal
 *                       groups, tokens [N-G/2, N) and tokens [0, G/2).  Every
 *                       other group, and every unshifted head, is unchanged.
 *   S2ATTN_WRAP_SWAP  : Variant 3 of the same table (the shifted tokens swap
 *                       places with the original front tokens), read as: that
 *                       last rolled group keeps its tokens but takes tokens
 *                       0..G/2-1 first and N-G/2..N-1 after them, so every
 *                       group is causal in token order (the end tokens see the
 *                       front ones, not the reverse).  Every other group, and
 *                       every unshifted head, is unchanged.
 */
typedef enum {
    S2ATTN_WRAP_ROLL = 0,
    S2ATTN_WRAP_SPLIT = 1,
    S2ATTN_WRAP_SWAP = 2
} s2attn_wrap;

/*
 * Forward.  Writes o[B,N,H,d] and lse[B,H,N].
 * Arguments are validated on the host before any HIP call; on error nothing is
 * launched and a status code is returned.
 */
int s2attn_fwd(const void* q, const void* k, const void* v,
               void* o, float* lse,
               int B, int H, int Hkv, int N, int d, int G, int shift_heads,
               int dtype, void* stream);

/*
 * Bytes of device workspace s2attn_bwd needs: the fp32 row sums
 * -Dvec = -rowsum(dO * o) [B,H,N] (stored negated) and lse * log2(e) [B,H,N],
 * plus, where dk and dv take two passes (a key/value head shared by shifted
 * and unshifted query heads, on a shape whose frames cut the keys into
 * different tiles), the first pass's fp32 dk and dv [2, B, N, Hkv, d].
 * Returns 0 when the arguments would be rejected by s2attn_bwd, and for an
 * empty problem (B == 0 or N == 0), which needs no workspace.
 */
size_t s2attn_bwd_workspace_bytes(int B, int H, int Hkv, int N, int d, int G,
                                  int shift_heads, int dtype);

/*
 * Backward of L = sum(o * dO): writes dq, dk, dv (same dtype as q).
 * Needs the forward's own o and lse.  `workspace` is caller-owned device
 * memory of at least s2attn_bwd_workspace_bytes() bytes, 256-byte aligned; its
 * contents on entry do not matter and are clobbered.  Concurrent calls must
 * use distinct workspaces.  No atomics: results are bitwise repeatable.
 */
int s2attn_bwd(const void* q, const void* k, const void* v, const void* o,
               const float* lse, const void* dO,
               void* dq, void* dk, void* dv,
               void* workspace, size_t workspace_bytes,
               int B, int H, int Hkv, int N, int d, int G, int shift_heads,
               int dtype, void* stream);

/*
 * The backward as stages.  s2attn_bwd is exactly s2attn_bwd_prep_dq then
 * s2attn_bwd_dkdv on one stream; s2attn_bwd_prep followed by s2attn_bwd_dq is
 * the same as s2attn_bwd_prep_dq up to the rounding of Dvec.  Same checks and
 * workspace as s2attn_bwd; dkdv and dq both read what prep (or prep_dq)
 * wrote, and after prep they may run in either order.
 * The gradients are those of the causal softmax attention of "The shifting
 * mechanism" / Algorithm 1 (page section 3.4) in every group of every head's
 * rolled frame: P = exp(scale q k^T - lse), dS = P * (dO v^T - Dvec),
 *   prep : -Dvec[b,h,t] = -sum_c dO[b,t,h,c] * o[b,t,h,c] and lse * log2(e)
 *          (fp32) into the workspace;
 *   dkdv : dv = P^T dO and dk = scale dS^T q, summed over the query heads
 *          that share a key/value head;
 *   dq   : dq = scale dS k (recomputes P and dS per query tile);
 *   prep_dq : prep and dq in one pass (one launch where the fast bf16 dq
 *          kernel runs: every query row is handled by one workgroup, which
 *          already holds its dO row); writes dq and the workspace.  It takes
 *          the wrap option (an s2attn_wrap value) like the _ex calls below.
 */
int s2attn_bwd_prep(const void* o, const float* lse, const void* dO, void* workspace, size_t workspace_bytes,
                    int B, int H, int Hkv, int N, int d, int G, int shift_heads,
                    int dtype, void* stream);
int s2attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO,
                    void* dk, void* dv, void* workspace, size_t workspace_bytes,
                    int B, int H, int Hkv, int N, int d, int G, int shift_heads,
                    int dtype, void* stream);
int s2attn_bwd_dq(const void* q, const void* k, const void* v, const void* dO,
                  void* dq, void* workspace, size_t workspace_bytes,
                  int B, int H, int Hkv, int N, int d, int G, int shift_heads,
                  int dtype, void* stream);
int s2attn_bwd_prep_dq(const void* q, const void* k, const void* v, const void* o,
                       const float* lse, const void* dO,
                       void* dq, void* workspace, size_t workspace_bytes,
                       int B, int H, int Hkv, int N, int d, int G, int shift_heads, int wrap,
                       int dtype, void* stream);

/*
 * The forward, the backward and its dkdv and dq stages with a wrap option
 * (an s2attn_wrap value; any other value returns S2ATTN_ERR_UNSUPPORTED before
 * any other work).  Arguments are otherwise those of the calls without _ex,
 * which are these with S2ATTN_WRAP_ROLL.  s2attn_bwd_prep and the workspace do
 * not depend on the option; the backward must use the forward's option.
 */
int s2attn_fwd_ex(const void* q, const void* k, const void* v,
                  void* o, float* lse,
                  int B, int H, int Hkv, int N, int d, int G, int shift_heads, int wrap,
                  int dtype, void* stream);
int s2attn_bwd_ex(const void* q, const void* k, const void* v, const void* o,
                  const float* lse, const void* dO,
                  void* dq, void* dk, void* dv,
                  void* workspace, size_t workspace_bytes,
                  int B, int H, int Hkv, int N, int d, int G, int shift_heads, int wrap,
                  int dtype, void* stream);
int s2attn_bwd_dkdv_ex(const void* q, const void* k, const void* v, const void* dO,
                       void* dk, void* dv, void* workspace, size_t workspace_bytes,
                       int B, int H, int Hkv, int N, int d, int G, int shift_heads, int wrap,
                       int dtype, void* stream);
int s2attn_bwd_dq_ex(const void* q, const void* k, const void* v, const void* dO,
                     void* dq, void* workspace, size_t workspace_bytes,
                     int B, int H, int Hkv, int N, int d, int G, int shift_heads, int wrap,
                     int dtype, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the backward
 * of s2attn_bwd_ex without a caller workspace.  Its scratch (the workspace
 * of s2attn_bwd_ex: the fp32 -Dvec and lse * log2(e) rows, 8 bytes per query
 * row, and where dk and dv take two passes the first pass's sums) lives in a
 * device array of the library, 32 MiB (S2ATTN_NOALLOC_MAX_ROWS query rows) on
 * every GPU the call runs on, held until the process ends; its address is
 * looked up once per device (the device current at the call) and the call
 * allocates nothing.  Same arguments, checks and results as s2attn_bwd_ex,
 * bit for bit; B * H * N above S2ATTN_NOALLOC_MAX_ROWS, or a workspace
 * (s2attn_bwd_workspace_bytes) larger than the array, returns
 * S2ATTN_ERR_SCRATCH (after the size checks, before the pointer checks and
 * any HIP call).  The scratch needs no clearing: each stage writes every
 * value a later stage reads.  Every call on one GPU shares that GPU's
 * scratch: calls whose kernels can overlap on one GPU (other streams, other
 * host threads) race and must be serialised by the caller.  S2ATTN_ERR_HIP
 * also reports a failed lookup of the scratch.
 */
#define S2ATTN_NOALLOC_MAX_ROWS (1 << 22)
int s2attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                       const float* lse, const void* dO,
                       void* dq, void* dk, void* dv,
                       int B, int H, int Hkv, int N, int d, int G, int shift_heads, int wrap,
                       int dtype, void* stream);

/*
 * Rotary position embedding with Position Interpolation, the step before the
 * attention on the pages' fine-tuning path (page "LongLoRA: Efficient
 * Fine-tuning of Long-Context Large Language Models", section 3.2 Phase 1
 * item 2, and "Training Procedure, Hyperparameters, and Dataset
 * Configuration", "Model setup": the pre-trained rotary embeddings are
 * rescaled by Position Interpolation).  The pages give no formula; this is
 * the published rotary embedding in the rotate-half pairing.  For x and y of
 * shape [B, N, Hx, d] (q with Hx = H, or k with Hx = Hkv), token n and
 * i < d/2, with t = n * pos_scale * base^(-2i/d):
 *   y[.., i]       = x[.., i] cos t - x[.., i + d/2] sin t
 *   y[.., i + d/2] = x[.., i + d/2] cos t + x[.., i] sin t
 * pos_scale is Position Interpolation's original / target context (1 = plain
 * rotary embedding; 4096 / 32768 for a 4k model extended to 32k); base is the
 * rotary base (10000 for Llama2).  inverse = 1 turns by -t instead: the
 * transpose, which maps the gradient of y to the gradient of x, so a backward
 * applies it to dq and dk.  y may equal x (in place); otherwise the two must
 * not overlap.  Asynchronous on `stream`; computed in fp32 from angles formed
 * and reduced in fp64, outputs rounded to the dtype.
 * Errors (before any HIP call): S2ATTN_ERR_SHAPE for B or N < 0, Hx <= 0 or
 * d <= 0; S2ATTN_ERR_UNSUPPORTED for d not in {64, 128}, an unknown dtype,
 * pos_scale negative or not finite, base not finite or <= 1, or inverse not 0
 * or 1; S2ATTN_ERR_NULL for a NULL x or y, S2ATTN_ERR_ALIGN for an x or y not
 * 16-byte aligned.  B == 0 or N == 0 is a no-op.
 */
int s2attn_rope(const void* x, void* y, int B, int N, int Hx, int d, double pos_scale, double base,
                int inverse, int dtype, void* stream);

/*
 * The attention with the rotary embedding (Position Interpolation) of
 * s2attn_rope fused in, bf16 only (other dtypes: S2ATTN_ERR_UNSUPPORTED).  The
 * fine-tuning path of the pages (section 3.2 Phase 1 item 2, "Model setup")
 * rotates q and k before the attention; here
 *   k_rot = s2attn_rope(k)                    (the stand-alone pass, for k only)
 *   s2attn_fwd_rope: takes q unrotated and k_rot; rotates q in the kernel's
 *       registers (bit-equal to s2attn_rope(q)), writes o, lse as s2attn_fwd_ex
 *       on the rotated q and k_rot, and the rotated q to q_rot [B,N,H,d] for
 *       the backward;
 *   s2attn_bwd_rope: takes q_rot and k_rot, writes dv as s2attn_bwd_ex and dq,
 *       dk already turned back by the inverse rotation, i.e. the gradients with
 *       respect to the unrotated q and k (the stand-alone route applies
 *       s2attn_rope(.., inverse=1) to the bf16-rounded gradients; here the
 *       fp32 sums are turned before rounding).
 * Arguments, checks and workspace as the _ex calls, plus pos_scale and base as
 * s2attn_rope (S2ATTN_ERR_UNSUPPORTED when out of range).  q_rot must not
 * overlap any other tensor.
 */
int s2attn_fwd_rope(const void* q, const void* k_rot, const void* v, void* o, float* lse, void* q_rot,
                    int B, int H, int Hkv, int N, int d, int G, int shift_heads, int wrap,
                    double pos_scale, double base, int dtype, void* stream);
int s2attn_bwd_rope(const void* q_rot, const void* k_rot, const void* v, const void* o,
                    const float* lse, const void* dO,
                    void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                    int B, int H, int Hkv, int N, int d, int G, int shift_heads, int wrap,
                    double pos_scale, double base, int dtype, void* stream);

/* Static, NUL-terminated description of a status code. */
const char* s2attn_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* S2ATTN_H */
