/*
 * attn.h -- C ABI of exact attention (forward, backward and paged decode) for
 * AMD MI355X (gfx950).
 *
 * The operation is exact scaled-dot-product attention computed the
 * IO-aware way: Q, K and V are streamed through on-chip tiles, the softmax is
 * accumulated online, and only O and its logsumexp are written, so device
 * memory stays linear in the sequence length («Что такое memory-efficient
 * attention для long context на 8x H100?», section 2, "FlashAttention-3:
 * IO-aware attention").  The result is the plain definition (the same page
 * calls the method exact):
 *
 *   O[b,h,i,:] = sum_{j in V(i)} softmax_j(scale * q[b,h,i,:] . k[b,g,j,:]) * v[b,g,j,:]
 *   lse[b,h,i] = ln sum_{j in V(i)} exp(scale * q[b,h,i,:] . k[b,g,j,:])
 *
 * with g = h / (H / H_kv): query heads form H_kv contiguous groups that share
 * one K/V head (grouped/multi-query attention, «Оптимизация внимания Flash»,
 * Workflow 2, Step 3).  The visible keys V(i) of query row i are
 *   causal = 1:  j <= i                          (Quick start; Workflow 2, Step 2)
 *   window >= 0: i - window <= j, and j <= i + window when causal = 0
 *                (sliding window, Workflow 2, Step 3: a (left, right) pair
 *                with -1 for "no limit"; one int covers both sides here, and
 *                the causal flag forces the right side to 0)
 *   window = -1: no window.
 * The diagonal key is always visible, so no row is empty.
 *
 * Layout (all contiguous, row-major, no strides):
 *   q, out : [B, H,    L, d]   16-bit floats (fp16 for attn_fwd, bf16 for attn_fwd_bf16)
 *   k, v   : [B, H_kv, L, d]   same 16-bit type
 *   lse    : [B, H,    L]      fp32, natural log
 * d must be 64 or 128.  The pages' inputs are fp16/bf16 only («Оптимизация
 * внимания Flash», Common issues: fp32 is not supported by the fast path).
 *
 * scale: used as given when finite and > 0; when <= 0 or NaN the automatic
 * scale 1/sqrt(d) is used (Workflow 2, Step 2: softmax_scale=None), as the
 * fp32 value nearest to it.  An infinite scale is rejected.
 *
 * Ownership and behaviour:
 *   - Every tensor pointer is a DEVICE pointer owned by the caller, who
 *     allocates and frees it.  The library allocates no device memory and
 *     never synchronises; it enqueues kernels only (no memory set or copy),
 *     so a call can be captured into a HIP graph.  The only state kept
 *     between calls is read-only after its first use: the paged decode's
 *     resident-wave count per device, and attn_decode_noalloc's scratch
 *     address per device.
 *   - stream is a hipStream_t (NULL = the default stream).  The call enqueues
 *     the kernel on it and returns; results are ready once the stream has
 *     reached that point.  Calls on different streams may run concurrently.
 *   - Arguments are validated before any HIP call, so an invalid call has no
 *     effect on the device and can be made without a GPU.
 *   - B = 0 or L = 0 is an empty problem: nothing is launched, ATTN_OK is
 *     returned, and the pointers may be NULL.
 *   - out and lse must not overlap each other or q, k, v (q, k and v may
 *     overlap one another: they are only read).
 *   - q, k, v and out must be 16-byte aligned, lse 4-byte aligned.
 *   - The grid is launched on the device that is current on the calling
 *     thread; the pointers and the stream must belong to it.
 *   - Errors during kernel execution surface at the caller's next
 *     synchronisation with the stream, as for any HIP kernel.
 */
#ifndef EXACT_IO_AWARE_ATTN_H
#define EXACT_IO_AWARE_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by the entry points. */
enum attn_status {
    ATTN_OK = 0,
    ATTN_ERR_NULL = 1,     /* a tensor pointer is NULL for a non-empty problem              */
    ATTN_ERR_SHAPE = 2,    /* B < 0, L < 0, H < 1, H_kv < 1, or H not a multiple of H_kv   */
    ATTN_ERR_HEAD_DIM = 3, /* d is neither 64 nor 128                                       */
    ATTN_ERR_WINDOW = 4,   /* window < -1                                                   */
    ATTN_ERR_ALIAS = 5,    /* an output overlaps another tensor                             */
    ATTN_ERR_LAUNCH = 6,   /* the HIP runtime refused the launch (no gfx950 device, ...)    */
    ATTN_ERR_SIZE = 7,     /* a tensor or the grid is too large to index                    */
    ATTN_ERR_FLAG = 8,     /* causal is neither 0 nor 1                                     */
    ATTN_ERR_SCALE = 9,    /* scale is +/- infinity                                         */
    ATTN_ERR_ALIGN = 10,   /* a tensor not 16-byte aligned, or lse not 4-byte aligned        */
    ATTN_ERR_SCRATCH = 11  /* attn_decode_noalloc: the call needs more workspace than its
                              static scratch holds (64 MiB)                                 */
};

/*
 * Exact attention forward for fp16 (IEEE binary16) q, k, v and out.
 * Computes out and lse as defined above for all B*H*L query rows.
 * Returns an attn_status; ATTN_OK means the kernel was enqueued.
 */
int attn_fwd(const void *q, const void *k, const void *v, void *out, float *lse,
             int B, int H, int H_kv, int L, int d, int causal, int window, float scale,
             void *stream);

/* The same operation for bfloat16 q, k, v and out (lse stays fp32). */
int attn_fwd_bf16(const void *q, const void *k, const void *v, void *out, float *lse,
                  int B, int H, int H_kv, int L, int d, int causal, int window, float scale,
                  void *stream);

/*
 * The same forward pass for fp8 inputs: q, k, v hold OCP FP8 E4M3 bytes
 * (float8_e4m3fn, as «Оптимизация внимания Flash», Workflow 3, Step 3 casts
 * them), same layouts; out is bf16 [B, H, L, d]; lse fp32.  The result is
 * the definition above of the decoded inputs; both products run on the fp8
 * MFMA, so the softmax weights enter the second product rounded to E4M3
 * (the row sums, and so lse, stay fp32).  Same argument rules as attn_fwd;
 * q, k, v, out 16-byte aligned.
 */
int attn_fwd_fp8(const void *q, const void *k, const void *v, void *out, float *lse,
                 int B, int H, int H_kv, int L, int d, int causal, int window, float scale,
                 void *stream);

/* A static, human-readable name for a status code (never NULL). */
const char *attn_status_string(int status);

/* How attn_fwd / attn_fwd_bf16 would launch a problem of this shape: each
 * workgroup takes 32 * (*waves_per_group) query rows of one (batch, head),
 * and its waves form *key_splits groups that each walk a contiguous share of
 * the keys (their partial softmax results are merged exactly at the end).
 * Host-only; makes no HIP call.  Returns an attn_status (argument checks as
 * for attn_fwd; H_kv plays no part). */
int attn_launch_shape(int B, int H, int L, int d, int causal, int window, int *waves_per_group,
                      int *key_splits);

/*
 * Backward pass: the gradients of the forward above with respect to q, k and
 * v, for an upstream gradient dout of out.  The pages recommend the method
 * for training («Оптимизация внимания Flash», introduction) and name the
 * backward pass as the part their benchmark left unmeasured («ТЕХНИЧЕСКОЕ
 * ЗАДАНИЕ: Сравнить Hyena vs FlashAttention на 128k», stage 5); it is the
 * gradient of the definition above, computed the same IO-aware way (softmax
 * weights recomputed tile by tile from lse, nothing L x L in memory).  With
 * P_ij = exp(scale q_i . k_j - lse_i) for j in V(i):
 *
 *   D_i   = dout_i . out_i
 *   dS_ij = P_ij (dout_i . v_j - D_i)
 *   dq_i  = scale * sum_j dS_ij k_j
 *   dk_j  = scale * sum_i dS_ij q_i          (i over every row of every query
 *   dv_j  = sum_i P_ij dout_i                 head that reads k_j's K/V head)
 *
 * Inputs: q, k, v, causal, window, scale exactly as given to the forward
 * call, out and lse as it wrote them, dout [B, H, L, d] (same 16-bit type).
 * Outputs (overwritten): dq [B, H, L, d], dk and dv [B, H_kv, L, d], same
 * 16-bit type, each element rounded once from an fp32 accumulator.
 * workspace: caller-owned device memory of attn_bwd_workspace_size(B, H, L)
 * bytes, 16-byte aligned; on return it holds, per (b, h), Lp values of
 * -lse*log2(e) followed by Lp values of -D (Lp = L rounded up to a multiple
 * of 64; the padding rows hold zeros), in fp32.
 * Behaviour as for attn_fwd: device pointers, enqueue on `stream` and return,
 * no allocation, no synchronisation, arguments checked before any HIP call,
 * B = 0 or L = 0 is an empty problem.  dq, dk, dv and workspace must not
 * overlap one another or any input; every pointer except lse (4 bytes) must
 * be 16-byte aligned.  The result is deterministic (no atomics).
 */
int attn_bwd(const void *q, const void *k, const void *v, const void *out, const void *dout,
             const float *lse, void *dq, void *dk, void *dv, void *workspace,
             int B, int H, int H_kv, int L, int d, int causal, int window, float scale,
             void *stream);

/* The same backward pass for bfloat16 tensors (lse and workspace stay fp32). */
int attn_bwd_bf16(const void *q, const void *k, const void *v, const void *out, const void *dout,
                  const float *lse, void *dq, void *dk, void *dv, void *workspace,
                  int B, int H, int H_kv, int L, int d, int causal, int window, float scale,
                  void *stream);

/* Bytes of workspace attn_bwd / attn_bwd_bf16 need for B, H, L
 * (8 * B * H * Lp); 0 if any of them is <= 0.  Host-only. */
size_t attn_bwd_workspace_size(int B, int H, int L);

/*
 * Decode: attention of the Lq newest tokens of each sequence over its KV
 * cache, kept in fixed-size blocks behind a page table.  Each generated token
 * reads its whole cache, which makes this step HBM-bound («Что такое
 * memory-efficient attention для long context на 8x H100?», section 1); the
 * paged layout is PagedAttention's (same page, section 3: blocks of e.g. 16
 * tokens, a page table from logical to physical blocks).  With n = seq_lens[b]
 * and p = n - Lq + i the position of new token i (the last query aligned with
 * the last key), query (b, h, i) sees keys j <= p with, if window >= 0,
 * p - j <= window, of K/V head g = h / (H / H_kv); out and lse are the forward
 * definition over those keys (rows with p < 0 see no key: out 0, lse -inf).
 *
 * Layout:
 *   q, out          : [B, H, Lq, d]   16-bit (fp16 for attn_decode, bf16 for attn_decode_bf16)
 *   k_cache, v_cache: [num_blocks, H_kv, block_size, d]; key j of sequence b is row
 *                     j % block_size of block block_table[b][j / block_size]
 *   block_table     : int32 [B, max_blocks_per_seq]
 *   seq_lens        : int32 [B], device memory; values are clamped to [0, max_seq_len]
 *   lse             : [B, H, Lq] fp32, natural log
 *   workspace       : attn_decode_workspace_size(B, H, H_kv, Lq, d, max_seq_len) bytes
 *                     (per-sequence offsets and partial results of the split
 *                     over keys; contents undefined on return)
 * block_size: a power of two in [16, 4096]; max_seq_len <= max_blocks_per_seq *
 * block_size.  Table entries are clamped to [0, num_blocks - 1], so an
 * invalid table reads wrong blocks but never outside the cache.
 * Behaviour as for attn_fwd (device pointers, enqueue only, no allocation, no
 * synchronisation, arguments checked before any HIP call; B = 0 is empty).
 * The keys are split evenly over as many waves as the device holds at once;
 * the first call on a device asks the runtime for that number (the device
 * current at the call, which must be the stream's device).
 * out, lse and workspace must not overlap one another or any input; q, the
 * caches, out and workspace 16-byte aligned, the int32 arrays and lse 4-byte.
 */
int attn_decode(const void *q, const void *k_cache, const void *v_cache, const int *block_table,
                const int *seq_lens, void *out, float *lse, void *workspace,
                int B, int H, int H_kv, int Lq, int d, int block_size, int max_blocks_per_seq,
                int num_blocks, int max_seq_len, int window, float scale, void *stream);

/* The same decode step for bfloat16 q, caches and out. */
int attn_decode_bf16(const void *q, const void *k_cache, const void *v_cache, const int *block_table,
                     const int *seq_lens, void *out, float *lse, void *workspace,
                     int B, int H, int H_kv, int Lq, int d, int block_size, int max_blocks_per_seq,
                     int num_blocks, int max_seq_len, int window, float scale, void *stream);

/* Bytes of workspace attn_decode / attn_decode_bf16 need; 0 for invalid
 * arguments.  Host-only. */
size_t attn_decode_workspace_size(int B, int H, int H_kv, int Lq, int d, int max_seq_len);

/* attn_decode (fp16) for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The same arguments as attn_decode without `workspace`: the
 * offsets and partial results go to a static device array of 64 MiB
 * (67108864 bytes) that the library holds
 * on every device it runs on until the process ends; the call allocates
 * nothing.  A call whose attn_decode_workspace_size(...) exceeds it returns
 * ATTN_ERR_SCRATCH before any HIP call.  The first call on a device looks up
 * that device's copy of the array (the device current at the call, which
 * must be the stream's device).  Every call on one device shares the array,
 * so calls that overlap on one device (other streams, other threads) race;
 * calls on one stream are ordered and safe.  Its contents are undefined
 * between calls (nothing in it needs to start at zero).  Other behaviour and
 * every argument check as for attn_decode. */
int attn_decode_noalloc(const void *q, const void *k_cache, const void *v_cache, const int *block_table,
                        const int *seq_lens, void *out, float *lse,
                        int B, int H, int H_kv, int Lq, int d, int block_size, int max_blocks_per_seq,
                        int num_blocks, int max_seq_len, int window, float scale, void *stream);


/* The fp32 scale the kernels use for a given scale argument and head size:
 * `scale` itself when finite and > 0, else the fp32 value nearest 1/sqrt(d).
 * Host-only; makes no HIP call. */
float attn_resolve_scale(float scale, int d);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_IO_AWARE_ATTN_H */
