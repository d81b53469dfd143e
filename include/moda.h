/*
 * moda.h -- C ABI of libmoda.so: the Mixture-of-Depths Attention (MoDA)
 * fused forward and the depth-stream layout kernels for AMD Instinct MI355X
 * (gfx950).
 *
 * Sources of the operations (cited by page title and section):
 *   [Notes] "Mixture-of-Depths Attention: 中文研读笔记" (reading notes on
 *           arXiv 2603.15619, cc.laoqi.cc).
 *   [Summ]  "Mixture-of-Depths Attention" (section-by-section summary,
 *           papercache.org).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library allocates no memory, keeps no state between calls and never
 *     synchronises: work is enqueued on `stream` (a hipStream_t; NULL means
 *     the default stream) and the call returns before it runs.
 *   - Tensors are dense, row-major, with no strides.  Indices are 0-based.
 *   - Every pointer must be 16-byte aligned.
 *   - Arguments are validated on the host before any HIP call, so each error
 *     code below can be produced without a GPU.  On error nothing is
 *     enqueued and the outputs are untouched.  No C++ exception crosses the
 *     ABI.
 *   - Results are deterministic: fixed reduction order, no atomics.
 */
#ifndef MODA_H
#define MODA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes. */
#define MODA_OK 0
#define MODA_ERR_NULL (-1)        /* a required pointer is NULL */
#define MODA_ERR_SHAPE (-2)       /* a size is out of range or inconsistent */
#define MODA_ERR_UNSUPPORTED (-3) /* a valid size this build has no kernel for */
#define MODA_ERR_ALIGN (-4)       /* a pointer is not 16-byte aligned */
#define MODA_ERR_HIP (-5)         /* the HIP launch reported an error */
#define MODA_ERR_TOO_LARGE (-6)   /* larger than moda_attn_decode_noalloc's fixed scratch */

typedef void* moda_stream_t; /* hipStream_t */

/*
 * MoDA forward, bf16 in / bf16 out, fp32 accumulation.
 *
 * Operation ([Notes] 二.2 unified-softmax expansion; [Summ] 2.2 MoDA and
 * 3.3 Algorithm 1): for batch b, token t and query head h, with
 * G = Hq / Hk, KV head hk = floor(h / G) (0-based form of phi(h) = ceil(h/G),
 * [Summ] 2.1 Eq. (2)) and s = 1/sqrt(d), one softmax runs jointly over
 *   - the sequence keys j of KV head hk: j <= t when causal = 1 (the causal
 *     mask of Eq. (2)), all j < T when causal = 0, with logit
 *     s * <q[b,t,h], k_seq[b,j,hk]> and value v_seq[b,j,hk];
 *   - the L depth slots i of the same token t and KV head hk, with logit
 *     s * <q[b,t,h], k_depth[b,t,hk,i]> and value v_depth[b,t,hk,i].
 *   out[b,t,h,:] = sum(e^logit * value) / sum(e^logit), over both sets;
 *   lse[b,h,t]   = log(sum(e^logit)) (natural log, fp32).
 *
 * Arguments
 *   q        [B][T][Hq][d] bf16
 *   k_seq    [B][T][Hk][d] bf16
 *   v_seq    [B][T][Hk][d] bf16
 *   k_depth  [B][T][Hk][L][d] bf16, the PACKED depth layout written by
 *            moda_pack_depth / moda_append_depth_slot.  May be NULL iff L == 0.
 *   v_depth  [B][T][Hk][L][d] bf16, same layout and rule.
 *   B, T, Hq, Hk, d, L   sizes; L = number of depth slots (may be 0).
 *   causal   1 = causal sequence mask, 0 = full sequence attention.
 *   out      [B][T][Hq][d] bf16 (written, round-to-nearest-even).
 *   lse      [B][Hq][T] fp32 (written).
 *   stream   HIP stream to enqueue on.
 * out and lse must not overlap any input.
 *
 * Errors: MODA_ERR_NULL (q, k_seq, v_seq, out or lse NULL; depth NULL with
 * L > 0); MODA_ERR_SHAPE (B, T, Hq, Hk or d <= 0, L < 0, Hq % Hk != 0,
 * causal not 0/1); MODA_ERR_UNSUPPORTED (d not 64 or 128; G not in
 * {1,2,4,8,16,32}; sizes beyond this build's limits: T*G, the workgroup count
 * and, for this bf16 entry point, (T+64)*Hk*d*2 and 129*Hk*L*d*2 bytes must
 * stay below 2^31); MODA_ERR_ALIGN; MODA_ERR_HIP.
 */
int moda_attn_fwd(const void* q, const void* k_seq, const void* v_seq, const void* k_depth,
                  const void* v_depth, int B, int T, int Hq, int Hk, int d, int L, int causal,
                  void* out, float* lse, moda_stream_t stream);

/*
 * moda_attn_fwd over a bounded depth cache ([Summ] 6.2 future work: a sliding
 * window of the most recent S layers in place of all of them).  The packed
 * depth stream holds S slots per (token, KV head) -- k_depth, v_depth are
 * [B][T][Hk][S][d] -- filled as a ring (layer l writes slot l mod S with
 * moda_append_depth_slot), and the first L <= S slots are attended: L = S once
 * the ring is full, L = the number of layers written before that.  The softmax
 * does not depend on the order of the depth slots, so ring order needs no
 * unrolling.  Slots L..S-1 are never read.  Other arguments, layouts and errors
 * as moda_attn_fwd, plus MODA_ERR_SHAPE when S < L; the 2^31 limit applies to
 * 129*Hk*S*d*2 bytes.  moda_attn_fwd(..., L, ...) equals this call with S = L.
 */
int moda_attn_fwd_ring(const void* q, const void* k_seq, const void* v_seq, const void* k_depth,
                       const void* v_depth, int B, int T, int Hq, int Hk, int d, int S, int L, int causal,
                       void* out, float* lse, moda_stream_t stream);

/*
 * The same operation with fp32 inputs and fp32 output, computed in fp32.
 * Arguments, layouts and errors are those of moda_attn_fwd with every bf16
 * tensor replaced by an fp32 one (without the bf16 byte-offset limits).
 */
int moda_attn_fwd_f32(const void* q, const void* k_seq, const void* v_seq, const void* k_depth,
                      const void* v_depth, int B, int T, int Hq, int Hk, int d, int L, int causal,
                      void* out, float* lse, moda_stream_t stream);

/*
 * MoDA decode step, bf16 in / bf16 out, fp32 accumulation: one new token per
 * sequence attends jointly to the whole KV cache of its sequence and to its own
 * L depth slots ([Summ] 2.2 MoDA; [Notes] 二.2 unified softmax; [Notes] 二.4 on
 * the decode cost of the depth cache).  For batch b and query head h, with
 * hk = floor(h / G) and s = 1/sqrt(d), one softmax runs over
 *   - the T cached keys j of KV head hk, logit s * <q[b,h], k_cache[b,j,hk]>,
 *     value v_cache[b,j,hk] (the decode token is the last of the sequence, so
 *     every cached key is visible; its own key is expected in the cache);
 *   - the L depth slots i, logit s * <q[b,h], k_depth[b,hk,i]>, value
 *     v_depth[b,hk,i].
 *   out[b,h,:] = sum(e^logit * value) / sum(e^logit);  lse[b,h] = log(sum(e^logit)).
 * This equals row t = T-1 of moda_attn_fwd (causal) when the token's query is
 * q[b,T-1] and its packed depth slab is k_depth[b,T-1] / v_depth[b,T-1].
 *
 * Arguments
 *   q        [B][Hq][d] bf16
 *   k_cache  [B][T][Hk][d] bf16 (the layout of moda_attn_fwd's k_seq)
 *   v_cache  [B][T][Hk][d] bf16
 *   k_depth  [B][Hk][L][d] bf16: the decode token's depth slab per KV head.
 *            May be NULL iff L == 0.
 *   v_depth  [B][Hk][L][d] bf16, same rule.
 *   out      [B][Hq][d] bf16 (written).   lse  [B][Hq] fp32 (written).
 *   workspace  device memory of at least moda_attn_decode_workspace(...)
 *            bytes, owned by the caller, 16-byte aligned; holds per-chunk
 *            partial results during the call (contents on entry are ignored,
 *            on return unspecified).  Calls that share a workspace must not
 *            overlap in time.
 *   workspace_bytes  its size.
 * The keys are reduced in chunks of 128 to 1024 (chosen from B, T and Hk), plus
 * one chunk for the depth slots, whose partial results are merged in a fixed
 * order: results are deterministic.
 *
 * Errors: MODA_ERR_NULL (q, caches, out, lse or workspace NULL; depth NULL with
 * L > 0); MODA_ERR_SHAPE (a size <= 0, L < 0, Hq % Hk != 0, or workspace_bytes
 * below moda_attn_decode_workspace); MODA_ERR_UNSUPPORTED (d not 64 or 128; G
 * not in {1,2,4,8,16,32}; the workgroup count or 1024 * Hk * d * 2 bytes beyond
 * 2^31); MODA_ERR_ALIGN; MODA_ERR_HIP.
 */
int moda_attn_decode(const void* q, const void* k_cache, const void* v_cache, const void* k_depth,
                     const void* v_depth, int B, int T, int Hq, int Hk, int d, int L, void* out, float* lse,
                     void* workspace, size_t workspace_bytes, moda_stream_t stream);

/*
 * moda_attn_decode over a bounded depth cache: k_depth, v_depth are
 * [B][Hk][S][d] ring slots of which the first L <= S are attended (see
 * moda_attn_fwd_ring).  Workspace as for moda_attn_decode with this L.
 * MODA_ERR_SHAPE when S < L.
 */
int moda_attn_decode_ring(const void* q, const void* k_cache, const void* v_cache, const void* k_depth,
                          const void* v_depth, int B, int T, int Hq, int Hk, int d, int S, int L, void* out,
                          float* lse, void* workspace, size_t workspace_bytes, moda_stream_t stream);

/*
 * Workspace bytes moda_attn_decode needs for these sizes (host only; 0 when a
 * size is invalid): (d + 2) fp32 values per (batch, query head, chunk).
 */
size_t moda_attn_decode_workspace(int B, int T, int Hq, int Hk, int d, int L);

/*
 * moda_attn_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  It allocates nothing and calls no
 * allocating routine: the per-chunk partial results live in a fixed scratch
 * array of MODA_DECODE_NOALLOC_SCRATCH_BYTES that the library holds in every
 * GPU's memory it runs on, from the first call on that GPU until the process
 * ends.  The first call on a device looks up that device's address of the
 * array (with the device current); later calls reuse it.
 *
 * Same operation, arguments, layouts, kernels and results (bit for bit) as
 * moda_attn_decode for the same inputs.  `stream` must belong to the current
 * device.  All calls on one GPU share its scratch, so calls that overlap in
 * time on one GPU (on different streams, or from different threads) race and
 * must be serialised by the caller.  Every partial result is written before
 * it is read, so nothing needs clearing between calls.
 *
 * Errors: as moda_attn_decode (there is no workspace to check), plus
 * MODA_ERR_TOO_LARGE when moda_attn_decode_workspace(B, T, Hq, Hk, d, L)
 * exceeds MODA_DECODE_NOALLOC_SCRATCH_BYTES (nothing is enqueued).
 */
#define MODA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int moda_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, const void* k_depth,
                             const void* v_depth, int B, int T, int Hq, int Hk, int d, int L, void* out,
                             float* lse, moda_stream_t stream);

/*
 * MoDA backward, bf16 in / bf16 gradients, fp32 accumulation: the gradients of
 * every input of moda_attn_fwd for the output gradient dout.  With the saved
 * natural-log lse, each row's softmax weights are recomputed as
 * P_n = exp(s <q, k_n> - lse) over the same candidates as the forward (the
 * causally visible sequence keys of KV head hk and the L depth slots of the
 * row's token; [Summ] 2.2 MoDA, [Notes] 二.2 unified softmax).  With
 * dP_n = <dout, v_n>, Dsum = <dout, out> and dS_n = P_n (dP_n - Dsum):
 *   dq  = s * sum_n dS_n k_n
 *   dk_n = s * sum over the rows that see n of dS_n q,  dv_n = sum of P_n dout.
 * A sequence key collects from every row of its G heads at or after it (all
 * rows when causal == 0); a depth slot only from the G rows of its own token.
 *
 * Arguments
 *   q, k_seq, v_seq, k_depth, v_depth, B, T, Hq, Hk, d, L, causal: the forward's
 *            inputs exactly as given to moda_attn_fwd (depth packed
 *            [B][T][Hk][L][d]; NULL iff L == 0).
 *   out      [B][T][Hq][d] bf16: the forward's output for these inputs.
 *   lse      [B][Hq][T] fp32: the forward's lse for these inputs.
 *   dout     [B][T][Hq][d] bf16: gradient of the loss with respect to out.
 *   dq       [B][T][Hq][d] bf16 (written).
 *   dk_seq, dv_seq     [B][T][Hk][d] bf16 (written).
 *   dk_depth, dv_depth [B][T][Hk][L][d] bf16, packed like k_depth (written;
 *            may be NULL iff L == 0).
 *   workspace  device memory of at least moda_attn_bwd_workspace(...) bytes,
 *            owned by the caller, 16-byte aligned; per-row statistics and
 *            the depth share of dq live there during the call (contents on
 *            entry ignored, on return unspecified).  Calls that share a
 *            workspace must not overlap in time.
 *   workspace_bytes  its size.
 * Gradient buffers must not alias the inputs or each other.  Every gradient
 * element is produced by one lane in a fixed order (no atomics): results are
 * deterministic.  Enqueued on `stream`; nothing is allocated or synchronised.
 *
 * Errors: MODA_ERR_NULL (a required pointer NULL; depth inputs or gradients
 * NULL with L > 0); MODA_ERR_SHAPE (a size <= 0, L < 0, Hq % Hk != 0,
 * causal not 0/1, or workspace_bytes below moda_attn_bwd_workspace);
 * MODA_ERR_UNSUPPORTED (d not 64 or 128; G not in {1,2,4,8,16,32}; (T + 128) *
 * Hq * d * 2 bytes or a grid beyond 2^31); MODA_ERR_ALIGN; MODA_ERR_HIP.
 */
int moda_attn_bwd(const void* q, const void* k_seq, const void* v_seq, const void* k_depth, const void* v_depth,
                  const void* out, const float* lse, const void* dout, int B, int T, int Hq, int Hk, int d, int L,
                  int causal, void* dq, void* dk_seq, void* dv_seq, void* dk_depth, void* dv_depth, void* workspace,
                  size_t workspace_bytes, moda_stream_t stream);

/*
 * Workspace bytes moda_attn_bwd needs for these sizes (host only; 0 when a size
 * is invalid): two fp32 values per query row, plus d fp32 values per query
 * row when L > 0, each region rounded up to 256 bytes.
 */
size_t moda_attn_bwd_workspace(int B, int T, int Hq, int Hk, int d, int L);

/*
 * Depth write path: the KV projection of a layer's hidden states, stored by the
 * product's epilogue directly into one slot of the packed depth stream.  A
 * layer adds to every token's depth stream its attention branch's own K, V and
 * a KV projection of its FFN input ([Notes] 二.3; [Summ] 2.2, the write step);
 * both are this product:
 *   k[b,t,hk,c] = sum_m x[b,t,m] * w_kv[hk*d + c][m]
 *   v[b,t,hk,c] = sum_m x[b,t,m] * w_kv[Hk*d + hk*d + c][m]
 * fp32 accumulation, rounded once to bf16 (RNE); every destination receives
 * the same bf16 values.
 *
 * Arguments
 *   x        [B][T][Dm] bf16 hidden states.
 *   w_kv     [2*Hk*d][Dm] bf16: output channels as rows (the torch Linear
 *            layout), K channels first, then V channels.
 *   k_out, v_out      [B][T][Hk][d] bf16 (written), or both NULL: the layer's
 *            sequence K/V (attention branch).
 *   k_depth, v_depth  [B][T][Hk][S][d] bf16 packed depth stream, or both NULL;
 *            only slot `slot` of every (token, KV head) is written, the other
 *            S - 1 slots are left untouched.
 *   S, slot  slots per (token, KV head) in the depth buffers, 0 <= slot < S.
 * At least one destination pair must be given.  Destinations must not alias x
 * or w_kv.  Enqueued on `stream`; nothing is allocated or synchronised.
 *
 * Errors: MODA_ERR_NULL (x or w_kv NULL, no destination pair, or half a pair);
 * MODA_ERR_SHAPE (a size <= 0; with depth buffers S <= 0 or slot outside
 * [0, S)); MODA_ERR_UNSUPPORTED (d not 64 or 128; Dm not a multiple of 64;
 * 256 * Dm * 2 bytes or the grid beyond 2^31); MODA_ERR_ALIGN; MODA_ERR_HIP.
 */
int moda_kv_project(const void* x, const void* w_kv, int B, int T, int Dm, int Hk, int d, void* k_out, void* v_out,
                    void* k_depth, void* v_depth, int S, int slot, moda_stream_t stream);

/*
 * Depth-stream pack: dst[b][t][hk][l][:] = src[b][t][l][hk][:], bit for bit.
 *
 * [Summ] 3.2 stores a position's L depth states contiguously; this layout
 * additionally moves the KV head outside the slot index, so the L slots of one
 * (token, KV head) pair form one contiguous run of L*d elements that the
 * forward stages once for that head's G query rows ([Summ] 3.2 group-aware
 * depth computation).
 *
 *   src  [B][T][L][Hk][d] elements of elem_bytes bytes (read).
 *   dst  [B][T][Hk][L][d] (written).  Must not overlap src.
 *   elem_bytes  1, 2, 4 or 8 (2 for bf16, 4 for fp32).
 * Errors: MODA_ERR_NULL; MODA_ERR_SHAPE (a size <= 0 or a bad elem_bytes);
 * MODA_ERR_ALIGN; MODA_ERR_HIP.
 */
int moda_pack_depth(const void* src, void* dst, int B, int T, int L, int Hk, int d, int elem_bytes,
                    moda_stream_t stream);

/*
 * Write one layer's K (or V) into one slot of the packed depth stream:
 * dst[b][t][hk][slot][:] = kv_l[b][t][hk][:] ([Summ] 2.2: after its
 * attention, a layer appends its KV to the depth stream for later layers).
 * Other slots of dst are left untouched.
 *
 *   kv_l  [B][T][Hk][d] (read).
 *   dst   [B][T][Hk][L][d] (slot `slot` written).  Must not overlap kv_l.
 *   slot  in [0, L).
 * Errors: MODA_ERR_NULL; MODA_ERR_SHAPE (a size <= 0, slot out of range,
 * bad elem_bytes); MODA_ERR_ALIGN; MODA_ERR_HIP.
 */
int moda_append_depth_slot(const void* kv_l, void* dst, int slot, int B, int T, int L, int Hk, int d,
                           int elem_bytes, moda_stream_t stream);

/*
 * Base-time span of a block of expanded query rows ([Summ] 3.3, algorithm
 * preparation; [Notes] 二.5).  Expanded row i_q = t*G + g holds token t,
 * head g of one KV group, so t_base(i_q) = floor(i_q / G).  For the rows
 * [row0, row0 + rows): *t_start = min t_base = floor(row0 / G) and
 * *t_end = max t_base + 1 = floor((row0 + rows - 1) / G) + 1.  Host only.
 * Errors: MODA_ERR_NULL; MODA_ERR_SHAPE (row0 < 0, rows <= 0, G <= 0).
 */
int moda_block_span(int row0, int rows, int G, int* t_start, int* t_end);

/* Static, human-readable text for a return code ("unknown error" otherwise). */
const char* moda_error_string(int code);

#ifdef __cplusplus
}
#endif

#endif /* MODA_H */
