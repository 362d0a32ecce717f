/*
 * fa.h -- C ABI of the exact fused attention forward (and its gradients) for AMD gfx950 (MI355X).
 *
 * Operation. For every batch b, head h and query row i:
 *     s_ij   = scale * q_i . k_j                  (j visible: all j, or j <= i when causal)
 *     o_i    = sum_j softmax_j(s_i.) * v_j
 *     lse_i  = ln sum_j exp(s_ij)                 (natural log, over the visible j)
 * This is the standard attention of the unite.ai page "Flash Attention:
 * revolutionizing transformer efficiency" (opening code block; "The Math Behind
 * Flash Attention", item 1, max-subtracted softmax). It is computed the way the
 * same page's "Flash Attention Algorithm" and "Implementation Details" describe
 * it -- tile by tile, with a running row maximum m and running row sum l, so the
 * N x N score matrix never reaches device memory -- using the three
 * FlashAttention-2 changes listed on the systems-analysis.info page
 * "FlashAttention-2 (VI)", section "Kiến trúc kỹ thuật và nguyên lý hoạt động":
 * fewer non-matmul FLOPs (1/l applied once at the end), parallelism over blocks
 * of query rows as well as over batch x heads, and per-wave ownership of query
 * rows inside a workgroup. lse is the log form of the running statistics M and
 * L of the unite.ai page's blockwise code. Causal visibility (key j <= query i)
 * is a reading of "causal" in the triton-transformer README's usage example.
 *
 * Layout. q, k, v, o are [B, H, N, d] contiguous row-major (element (b,h,i,c)
 * at ((b*H + h)*N + i)*d + c). lse is [B, H, N] contiguous fp32.
 *
 * Ownership. The caller allocates every buffer in device memory (including
 * fa_bwd's workspace) and keeps it alive until the stream has run the work.
 * The library allocates nothing, keeps no state between calls, and never
 * synchronises: it validates the arguments on the host, enqueues its kernels
 * on `stream` (0 = null stream) and returns. A forward call enqueues one
 * kernel; a gradient call two (dq, then dk and dv), or three when the dk/dv
 * visits of each key block are divided over several workgroups and a third
 * kernel sums their fp32 partials. Results are valid once the caller
 * synchronises the stream. Inputs are only read; outputs are only written.
 * Calls are thread-safe, and the same inputs give bitwise-identical outputs on
 * every call: no kernel uses atomics, and where the work of one output row is
 * divided -- the forward's small-grid shape gives the two 64-key halves of
 * every key tile to two waves, each with its own running maximum and sum; the
 * gradient call may give a key block's query tiles to several workgroups --
 * the partial results are merged in a fixed order.
 *
 * Errors. 0 on success; otherwise one of the FA_ERR_* codes below, and nothing
 * is enqueued. Every check except FA_ERR_HIP runs before any HIP call. Faults
 * inside the kernel surface at the caller's next synchronisation.
 * B, H or N equal to 0 is an empty problem: the call returns 0, enqueues
 * nothing and does not look at the pointers (sizes below 0 are FA_ERR_SHAPE).
 */
#ifndef FA_MI355X_FA_H
#define FA_MI355X_FA_H

#include <hip/hip_runtime_api.h>
#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_OK 0
#define FA_ERR_NULL 1    /* a pointer is NULL (non-empty problem) */
#define FA_ERR_SHAPE 2   /* B, H, N or H_kv negative; B*H over 65535; N over 2^30 (gradient calls: 2^28);
                            H_kv not dividing H */
#define FA_ERR_HEADDIM 3 /* d is not 64 or 128 */
#define FA_ERR_ALIGN 4   /* a tensor or the workspace not 16-byte aligned, or lse / kv_len not 4-byte aligned */
#define FA_ERR_ARG 5     /* scale not finite or not > 0, or causal not 0/1 */
#define FA_ERR_ALIAS 6   /* an output overlaps an input or another output */
#define FA_ERR_HIP 7     /* the HIP runtime reported an error at launch */
#define FA_ERR_SCRATCH 8 /* fa_bwd_noalloc: the problem's workspace exceeds the library's scratch buffer */

/*
 * fa_fwd -- bf16 inputs and output, fp32 accumulation and fp32 lse.
 *   q, k, v : const bf16 [B,H,N,d] (device)       o : bf16 [B,H,N,d] (device, written)
 *   lse     : float [B,H,N] (device, written), natural-log log-sum-exp of the scaled scores
 *   B, H, N : batch, heads, sequence length (queries and keys have the same length N)
 *   d       : head dimension, 64 or 128
 *   causal  : 1 -> key j visible to query i iff j <= i; 0 -> every key visible
 *   scale   : softmax scale applied to q.k (e.g. 1/sqrt(d)); finite and > 0
 *   stream  : HIP stream the kernel is enqueued on
 * The probabilities are rounded to bf16 (round-to-nearest-even) before the
 * product with V; o is rounded to bf16 once, after the division by l.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d, int causal,
           float scale, hipStream_t stream);

/*
 * fa_fwd_gqa -- fa_fwd with fewer key/value heads than query heads
 * (grouped-query attention; H_kv = 1 is multi-query attention), listed among
 * the FlashAttention-2 improvements on the unite.ai page (section
 * "FlashAttention-2", item 3).
 *   k, v    : const bf16 [B,H_kv,N,d] (device)
 *   H_kv    : key/value heads, >= 1 and dividing H. Query head h reads
 *             key/value head h / (H / H_kv): each key/value head serves
 *             H / H_kv consecutive query heads.
 * Everything else (q, o, lse, layout, ownership, errors) as fa_fwd; H_kv < 1
 * or not dividing H is FA_ERR_SHAPE. fa_fwd_gqa with H_kv = H is fa_fwd.
 */
int fa_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int H_kv, int N, int d,
               int causal, float scale, hipStream_t stream);

/*
 * fa_fwd_kpad -- fa_fwd_gqa with a key-padding mask given as per-batch
 * lengths (the boolean (batch, seq) mask of the triton-transformer README's
 * usage example, "ex. BERT", for right-padded sequences: the valid keys of a
 * batch are a prefix).
 *   kv_len  : const int32 [B] (device): batch b has kv_len[b] valid keys; key
 *             j is visible to the queries of batch b only if j < kv_len[b]
 *             (and j <= i when causal). Values are clamped to [0, N] on the
 *             device. All N query rows are computed; a row with no visible key
 *             (kv_len[b] = 0) gets o = 0 and lse = -inf.
 * Work skips the key tiles past kv_len[b]. kv_len must be 4-byte aligned
 * (FA_ERR_ALIGN), non-NULL (FA_ERR_NULL) and must not overlap o or lse
 * (FA_ERR_ALIAS); it is only read, by the kernel. The rest as fa_fwd_gqa.
 */
int fa_fwd_kpad(const void* q, const void* k, const void* v, void* o, float* lse, const int* kv_len, int B, int H,
                int H_kv, int N, int d, int causal, float scale, hipStream_t stream);

/*
 * fa_fwd_varlen -- the forward over packed variable-length batches: B
 * sequences of different lengths stored back to back without padding (the
 * variable-length batches with per-batch lengths that go with the key-padding
 * mask of the triton-transformer README's usage example; packing is a reading).
 * Every sequence is its own attention problem: its queries see only its own
 * keys (causal: those at or before their own position in the sequence).
 *   q, o       : bf16 [total, H, d] (device; o written): token t, head h at
 *                (t*H + h)*d
 *   k, v       : const bf16 [total, H_kv, d] (device); H_kv divides H, query
 *                head h reads key/value head h / (H / H_kv)
 *   lse        : float [H, total] (device, written), element (h, t) at h*total + t
 *   cu_seqlens : const int32 [B+1] (device): sequence b is tokens
 *                cu_seqlens[b] .. cu_seqlens[b+1]-1; it must rise from 0 to
 *                total. The kernel clamps every offset to [0, total], so a
 *                malformed array cannot make it read or write outside the
 *                tensors (the results are then meaningless).
 *   max_seqlen : at least the longest sequence, at most total (it sizes the
 *                grid; tokens of a longer sequence past its first max_seqlen
 *                are neither read nor written)
 * An empty sequence writes nothing. B, H or total = 0 is an empty problem;
 * max_seqlen = 0 or above total with tokens present is FA_ERR_SHAPE; cu_seqlens
 * NULL is FA_ERR_NULL, not 4-byte aligned FA_ERR_ALIGN; o and lse must not
 * overlap the inputs, cu_seqlens or each other (FA_ERR_ALIAS). The rest
 * (numerics, ownership, errors) as fa_fwd.
 */
int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse, const int* cu_seqlens, int B,
                  int H, int H_kv, int total, int max_seqlen, int d, int causal, float scale, hipStream_t stream);

/*
 * fa_bwd -- gradients of fa_fwd / fa_fwd_gqa (bf16 tensors, fp32 arithmetic).
 * The pages name a faster backward pass that recomputes attention from stored
 * statistics instead of storing the attention matrix (unite.ai page, the key
 * ideas after "Enter Flash Attention", item 2; section "FlashAttention-2",
 * item 2); no formula is printed. With lse and o from the forward and an
 * upstream gradient dout of o (none for lse), per visible (i, j):
 *     p_ij = exp(scale q_i.k_j - lse_i)      D_i = dout_i . o_i
 *     dS_ij = p_ij (dout_i . v_j - D_i)
 *     dq_i = scale sum_j dS_ij k_j   dk_j = scale sum_i dS_ij q_i   dv_j = sum_i p_ij dout_i
 * dk and dv of a key/value head sum over the H / H_kv query heads that read it.
 *   q, o, dout : const bf16 [B,H,N,d] (device); o is fa_fwd's output for q, k, v
 *   k, v       : const bf16 [B,H_kv,N,d] (device)
 *   lse        : const float [B,H,N] (device), fa_fwd's lse for the same call
 *   dq         : bf16 [B,H,N,d] (device, written)
 *   dk, dv     : bf16 [B,H_kv,N,d] (device, written)
 *   workspace  : device memory of fa_bwd_workspace_bytes(B, H, H_kv, N, d) bytes,
 *                16-byte aligned, overwritten (no contents needed on entry
 *                or kept on return); calls that share a workspace must be
 *                ordered on one stream
 *   B, H, H_kv, N, d, causal, scale : as fa_fwd_gqa (same values as the forward call);
 *                N at most 2^28 (FA_ERR_SHAPE otherwise)
 * Enqueues two kernels on `stream` (dq, then dk and dv; a third that sums
 * partial dk and dv when the workspace holds them); no atomics, so the
 * same inputs give bitwise-identical gradients. p and dS are rounded to bf16
 * before their matrix products, the gradients once at the end. D_i is taken
 * from the o given (bf16): its rounding moves dq_i by at most
 * scale |dout_i . (o_i - o_exact_i)| max_j |k_j| (and dk alike), which shows
 * where the gradients themselves are small (few keys, one dominant). Errors as
 * fa_fwd, with every tensor and the workspace checked (NULL, 16-byte
 * alignment) and no output (dq, dk, dv, workspace) allowed to overlap an
 * input or another output (FA_ERR_ALIAS).
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout, void* dq,
           void* dk, void* dv, float* workspace, int B, int H, int H_kv, int N, int d, int causal, float scale,
           hipStream_t stream);

/*
 * fa_bwd_noalloc -- fa_bwd for callers that cannot allocate device memory
 * (code recorded into a HIP graph, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, with the workspace taken from a
 * static device buffer of the library instead of an argument.
 *   Arguments as fa_bwd, without workspace.
 *   Limit: the workspace fa_bwd_workspace_bytes(B, H, H_kv, N, d) would
 *   report must fit in 64 MiB (67108864 bytes); larger problems return
 *   FA_ERR_SCRATCH before any HIP call (e.g. B*H*N up to ~8.4M query rows
 *   when the dk/dv work needs no split; one key/value head serving 32 query
 *   heads of N = 16384 at d = 128 needs 68 MiB and is refused).
 * The buffer is a file-scope device array: every GPU the library runs on holds
 * its own 64 MiB copy from the library's first kernel launch on that GPU until
 * the process ends. Its device address is looked up once per GPU (on the
 * first fa_bwd_noalloc call for a stream of that GPU, a HIP call that can
 * fail with FA_ERR_HIP); nothing is allocated, and the call never frees or
 * allocates memory. All calls on one GPU share the buffer, which keeps the
 * last call's contents (no kernel needs it cleared: every value the kernels
 * read is written earlier in the same call): calls that can overlap on one
 * GPU -- on different streams, or from several host threads without ordering
 * -- race on it and give wrong results. Order them on one stream, or use
 * fa_bwd with a workspace per stream. Errors otherwise as fa_bwd.
 */
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                   void* dq, void* dk, void* dv, int B, int H, int H_kv, int N, int d, int causal, float scale,
                   hipStream_t stream);

/*
 * fa_bwd_kpad -- fa_bwd for a forward call made with fa_fwd_kpad: the
 * gradients under the same key-padding lengths.
 *   kv_len  : const int32 [B] (device), the lengths given to fa_fwd_kpad
 *             (clamped to [0, N] on the device); o and lse must come from
 *             that call. Key j >= kv_len[b] is visible to no query of batch
 *             b, so its dk and dv rows are written as 0 (whatever k and v
 *             hold there); with kv_len[b] = 0 every gradient of batch b is 0.
 * kv_len must be non-NULL (FA_ERR_NULL), 4-byte aligned (FA_ERR_ALIGN) and
 * must not overlap an output or the workspace (FA_ERR_ALIAS); it is only
 * read, by the kernels. Everything else as fa_bwd; fa_bwd_kpad with every
 * kv_len[b] >= N gives fa_bwd's results.
 */
int fa_bwd_kpad(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                void* dq, void* dk, void* dv, float* workspace, const int* kv_len, int B, int H, int H_kv, int N, int d,
                int causal, float scale, hipStream_t stream);

/*
 * fa_bwd_varlen -- gradients of fa_fwd_varlen (packed variable-length
 * batches): every sequence's gradients are those of its own attention
 * problem, as in fa_bwd.
 *   q, o, dout, dq : [total, H, d] bf16 (dq written); k, v, dk, dv :
 *                    [total, H_kv, d] bf16 (dk, dv written); lse : float
 *                    [H, total] from fa_fwd_varlen with the same arguments
 *   workspace      : fa_bwd_workspace_bytes(B, H, H_kv, max_seqlen, d) bytes, 16-byte
 *                    aligned, as for fa_bwd
 *   cu_seqlens, B, H, H_kv, total, max_seqlen, d, causal, scale : as
 *                    fa_fwd_varlen (offsets clamped on the device the same way);
 *                    max_seqlen at most 2^28 (FA_ERR_SHAPE otherwise)
 * Errors as fa_fwd_varlen, with every tensor, lse, cu_seqlens and the
 * workspace checked (NULL, alignment) and no output (dq, dk, dv, workspace)
 * allowed to overlap an input or another output (FA_ERR_ALIAS). Deterministic
 * as fa_bwd.
 */
int fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                  void* dq, void* dk, void* dv, float* workspace, const int* cu_seqlens, int B, int H, int H_kv,
                  int total, int max_seqlen, int d, int causal, float scale, hipStream_t stream);

/* fa_bwd_workspace_bytes -- bytes of the fa_bwd / fa_bwd_kpad workspace (fa_bwd_varlen: N = max_seqlen); 0 for
 * an empty problem or arguments the gradient calls reject (H_kv not dividing H, d not 64 or 128, B*H above
 * 65535, N above 2^28). It holds two
 * float planes per query row (-D_i and lse_i log2 e; 8 bytes a row), and, when the key blocks of the key/value
 * heads give the dk/dv kernel fewer than two workgroups per compute unit (few or long heads), the fp32 partial dk
 * and dv of the s <= 64 workgroups that share each key block's query heads and tiles between them
 * (2 x s x B x H_kv x N x d floats), summed in a fixed order by a third kernel. */
size_t fa_bwd_workspace_bytes(int B, int H, int H_kv, int N, int d);

/*
 * fa_fwd_fp8 -- the attention forward of fp8 inputs with per-tensor scales
 * (FP8 is listed among the FlashAttention-3 techniques on the unite.ai page,
 * section "FlashAttention-3", items 2-3; the scaling scheme is a reading).
 *   q, k    : const float8_e4m3fn [B,H,N,d] (device), one byte per element
 *   vt      : const float8_e4m3fn [B,H,d,N] (device): v transposed, element
 *             (b,h,c,j) at ((b*H + h)*d + c)*N + j
 *   q_scale, k_scale, v_scale : the real inputs are q*q_scale, k*k_scale,
 *             v*v_scale (finite, > 0)
 *   o       : bf16 [B,H,N,d] (device, written); lse : float [B,H,N] as fa_fwd
 *   N       : a multiple of 16, at most 2^24 (FA_ERR_SHAPE otherwise)
 * The scores and the weighted sum run on fp8 matrix instructions with fp32
 * accumulation; the softmax weights are rounded to e4m3 before the product
 * with v, and l sums the rounded weights (o is their weighted average). The
 * other arguments, errors and ownership as fa_fwd; no grouped heads, no key
 * padding. NaN inputs give undefined results.
 */
int fa_fwd_fp8(const void* q, const void* k, const void* vt, void* o, float* lse, float q_scale, float k_scale,
               float v_scale, int B, int H, int N, int d, int causal, float scale, hipStream_t stream);

/*
 * fa_fwd_f32 -- the same operation with fp32 q, k, v and o. Products and sums
 * stay in fp32 throughout (fp32 matrix-core instructions, no bf16 step).
 * Arguments, layout, ownership and errors as fa_fwd.
 */
int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H, int N, int d,
               int causal, float scale, hipStream_t stream);

/*
 * fa_fwd_instance -- which bf16 forward kernel instance fa_fwd, fa_fwd_gqa
 * and fa_fwd_kpad (packed = 0), or fa_fwd_varlen (packed = 1, N =
 * max_seqlen), enqueue for B*H heads of N query rows, head dim d and the
 * causal flag: a static string spelling the kernel's template arguments, the
 * name profilers list, e.g. "fa_fwd_bf16_kernel<128, false, 8, 2, 2, false, 1>"
 * (<d, causal, waves per workgroup, ring stages, 64-key parts per key tile,
 * packed, waves per 32-row group>). The workgroup shape is chosen from the
 * grid size alone (grouped heads and key lengths do not change it). NULL when
 * the sizes are not a valid non-empty problem (B, H or N below 1, B*H above
 * 65535, N above 2^30, d not 64 or 128, causal or packed not 0 or 1). Makes no
 * HIP call.
 */
const char* fa_fwd_instance(int B, int H, int N, int d, int causal, int packed);

/* fa_strerror -- static, NUL-terminated description of an FA_* code. */
const char* fa_strerror(int code);

/* fa_version -- library version as major*10000 + minor*100 + patch. */
int fa_version(void);

#ifdef __cplusplus
}
#endif
#endif /* FA_MI355X_FA_H */
