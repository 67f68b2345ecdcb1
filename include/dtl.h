/*
 * dtl.h - C ABI of libdtl.so: the per-GPU hot path of sequence-parallel DiT
 * self-attention on one AMD Instinct MI355X (gfx950).
 *
 * Conventions shared by every entry point
 *   - Every pointer argument is a DEVICE pointer owned by the caller (for example
 *     the storage of a torch tensor).  The library keeps no pointer after the call
 *     returns.
 *   - Memory and state of the library's own.  The attention entry points
 *     (attn_fwd_lse, attn_fwd_lse_accumulate, attn_fwd_lse_kv_chunks) split the last,
 *     short round of query tiles of a long workload across the GPU (at least one full
 *     round of tiles over the resident workgroups, a remainder of at most a quarter of
 *     a round, and ceil(Nkv / 64) >= 64 key blocks, i.e. Nkv >= 4033).  Such a call
 *     takes a workspace of at most about 36 MB for the split pieces' states from a memory
 *     pool the library creates per device on its first call there, stream-ordered on
 *     `stream` (allocated before the kernels, freed after them on the same stream; the
 *     pool keeps freed memory for the next call, so repeated calls do not reach the
 *     driver's allocator).  That departs from a library that never allocates: measured,
 *     the split makes Wan2.2-5B-sized attention 3.6% faster.  Callers that may not
 *     allocate use attn_fwd_lse_noalloc, whose workspace is a static device array.  Per
 *     process the library keeps, per device, its compute-unit count and that pool, created once under a
 *     mutex, and a 64-bit launch counter (an atomic) that tells one launch's workspace
 *     flags from another's.
 *     Query tiles have 256 rows (one workgroup per CU) for head_dim 128 with more than
 *     16 key blocks of 64 (Nkv > 1024) when 128-row tiles would be more than one per CU,
 *     else 128 rows.  A 128-row tile runs in a 4-wave workgroup (two per CU), or, for head_dim 128
 *     when the grid
 *     holds at most one tile per CU, in an 8-wave workgroup whose two 4-wave key groups
 *     each take half of the key blocks and fold their partial states in LDS.
 *   - Test and tuning variables, read at every call they apply to: they change which
 *     workgroup computes which keys, never the result.  DTL_ATTN_SLOTS (a positive
 *     number below the resident workgroup count) schedules as if the GPU held that many
 *     workgroups; DTL_ATTN_WAVES (4 or 8) picks 128- or 256-row tiles for head_dim 128;
 *     DTL_ATTN_KEYSPLIT (0 or 1) turns the two key groups per 128-row tile off or on;
 *     DTL_ATTN_SPLIT (0 or 1) never splits the tiles past the last whole round, or splits
 *     any such remainder (by default only one of at most a quarter of the slots);
 *     DTL_ATTN_MAX_POLLS (0 up to the default of 20000) bounds how often a split tile's
 *     finaliser polls for its helpers' published states before it computes their keys
 *     itself (0: at once).  DTL_MERGE_KERNEL=lds makes attn_merge_lse take its LDS kernel
 *     for every shape instead of the row kernel it uses for P in {2, 4, 8} and D in
 *     {64, 128} (read at every merge call; the same result bit for bit).
 *   - Tensors are dense and row-major in the shapes given; there are no strides.
 *     Every pointer must be 16-byte aligned.
 *   - bf16 is IEEE bfloat16 stored as 16-bit words; f32 is IEEE binary32.
 *   - Calls are asynchronous on `stream` (NULL selects the null stream).  They do
 *     not synchronize, and every pool workspace belongs to one call, so calls on
 *     different streams may run concurrently as long as their buffers do not overlap
 *     (attn_fwd_lse_noalloc excepted: its calls share one static workspace per device).
 *   - Arguments are validated on the host before anything is launched.  On a
 *     validation error nothing is launched and nothing is written.  DTL_ERR_HIP is
 *     returned when the kernel launch itself reports an error.  Device faults surface,
 *     as for any HIP stream work, at the caller's next synchronization.
 *   - No C++ exception crosses this interface.
 */
#ifndef DTL_H
#define DTL_H

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DTL_OK = 0,
    DTL_ERR_INVALID_ARG = 1,  /* null pointer, non-positive size, misalignment, overlap, bad divisibility */
    DTL_ERR_UNSUPPORTED = 2,  /* valid request outside what this build implements (head_dim, dtype) */
    DTL_ERR_HIP = 3,          /* the HIP runtime reported an error at launch */
    DTL_ERR_WORKSPACE = 4     /* attn_fwd_lse_noalloc: the static workspace is too small */
} dtl_status;

typedef enum {
    DTL_BF16 = 0,
    DTL_F32 = 1
} dtl_dtype;

/*
 * attn_fwd_lse - attention forward with per-row log-sum-exp.
 *
 * Computes, independently for every batch b, head h and query row i, over all
 * keys j in [0, Nkv) (non-causal: every query sees every key):
 *     s_ij        = softmax_scale * sum_d q[b,i,h,d] * k[b,j,h,d]
 *     o[b,i,h,:]  = sum_j exp(s_ij) * v[b,j,h,:] / sum_j exp(s_ij)
 *     lse[b,h,i]  = ln sum_j exp(s_ij)                 (natural log, scaled logits)
 * This is softmax(q k^T / sqrt(d)) v per head as the MindIE SD "多卡并行" page
 * states it (Ring Sequence Parallel section, usage example), with heads
 * independent and every query attending to every key ("AIGC 分布式推理：从 Wan2.2
 * 理解 DP/TP/CP/SP/PP", CP section).  The LSE is what lets partial results over
 * separate key chunks be combined exactly (attn_merge_lse).
 *
 *   q    bf16 [B, Nq,  H, D]   (BSND: token-major, heads then head_dim)
 *   k    bf16 [B, Nkv, H, D]
 *   v    bf16 [B, Nkv, H, D]
 *   o    o_dtype [B, Nq, H, D]  bf16 (rounded to nearest even) for a final result,
 *                               f32 for a partial that will be merged
 *   lse  f32 [B, H, Nq]
 *   softmax_scale  finite and > 0; callers pass 1/sqrt(D)
 *
 * Arithmetic: bf16 products with f32 accumulation for q.k and p.v; the softmax
 * weights are computed in f32 and rounded to bf16, and both the p.v product and the
 * row sum (the denominator, accumulated in f32) use those same rounded weights.
 * Errors: DTL_ERR_INVALID_ARG for null pointers, any size <= 0, Nq or Nkv above
 * 2^31 - 257, B*Nq*H or B*Nkv*H rows or query tiles (of 128 rows) above 2^31 - 1, H*D
 * above 2^24, a scale that is not finite and positive, misaligned pointers, or an output
 * overlapping an input or the other output; DTL_ERR_UNSUPPORTED for D not in {64, 128} or
 * another o_dtype; DTL_ERR_HIP when a launch or the workspace allocation fails.
 */
dtl_status attn_fwd_lse(const void *q, const void *k, const void *v,
                        void *o, float *lse,
                        int B, int Nq, int Nkv, int H, int D,
                        float softmax_scale, dtl_dtype o_dtype, hipStream_t stream);

/*
 * attn_fwd_lse_noalloc - attn_fwd_lse for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 *
 * Same arguments, result and errors as attn_fwd_lse.  Where attn_fwd_lse takes the split
 * schedule's workspace from the library's pool, this entry point uses a static device
 * array of 36 MiB (`scratch` in attn_fwd.hip; each device holds its own copy until the
 * process ends, its address taken once per device with hipGetSymbolAddress at the
 * library's first attention call there).  It calls no hipMalloc, hipFree, pool or other
 * allocating routine.  A schedule that would need more scratch than that (none on a
 * 256-CU MI355X: at most about 34 MiB) is rejected before anything is launched with
 * DTL_ERR_WORKSPACE.  Each call leaves its states in the array; the next call needs
 * none of them cleared: the flags carry a value that differs per launch, including per
 * replay of a call captured in a HIP graph (a launch count kept in the array and advanced
 * by a one-thread kernel enqueued after the split launch), so a captured call may be
 * replayed with new contents in its input buffers.  Every call on one device shares that
 * device's array: calls that overlap in time on one device (for example on two streams)
 * race and give undefined results; calls on one stream never overlap.
 */
dtl_status attn_fwd_lse_noalloc(const void *q, const void *k, const void *v,
                                void *o, float *lse,
                                int B, int Nq, int Nkv, int H, int D,
                                float softmax_scale, dtl_dtype o_dtype, hipStream_t stream);

/*
 * attn_fwd_lse_accumulate - one round of Ring attention: attention over this call's
 * keys, folded into the result of the rounds before it.
 *
 * With (o_cur, lse_cur) what attn_fwd_lse would return for these keys, and for every
 * (b, i, h):
 *     L           = ln(exp(lse_prev[b,h,i]) + exp(lse_cur))
 *     o[b,i,h,:]  = exp(lse_prev - L) * o_prev[b,i,h,:] + exp(lse_cur - L) * o_cur
 *     lse[b,h,i]  = L
 * i.e. the online-softmax accumulation that each Ring round performs on its block of
 * K/V (arganzheng.life, multi-GPU diffusion parallelism, section 4.2 "Ring"; MindIE SD
 * "多卡并行" page, Ring Sequence Parallel section), done in the kernel's epilogue instead
 * of through separate partials and attn_merge_lse.  When (o_prev, lse_prev) is the
 * result over one key set and this call's keys are another, disjoint one, (o, lse) is
 * attention over their union.  A row with lse_prev = -inf holds no keys yet: its o_prev
 * is not read (it may hold anything) and the row gets this call's result alone.
 *
 *   q, k, v          as attn_fwd_lse
 *   o_prev  f32 [B, Nq, H, D]   the result so far (normalised, as attn_fwd_lse writes it)
 *   lse_prev f32 [B, H, Nq]
 *   o       o_dtype [B, Nq, H, D]  f32 to continue with further rounds, bf16 after the last
 *   lse     f32 [B, H, Nq]
 *   o may be o_prev itself when o_dtype is DTL_F32, and lse may be lse_prev itself (in
 *   place); any other overlap of o or lse with o_prev or lse_prev is rejected.
 *
 * Errors: as attn_fwd_lse, and DTL_ERR_INVALID_ARG for a null or misaligned o_prev or
 * lse_prev or an overlap outside the in-place case.
 */
dtl_status attn_fwd_lse_accumulate(const void *q, const void *k, const void *v,
                                   const float *o_prev, const float *lse_prev,
                                   void *o, float *lse,
                                   int B, int Nq, int Nkv, int H, int D,
                                   float softmax_scale, dtl_dtype o_dtype, hipStream_t stream);

/*
 * attn_fwd_lse_kv_chunks - attn_fwd_lse over P equal, contiguous key chunks in one call:
 * the partial results that Ring attention's P rounds produce on one rank (the KV blocks
 * [t*C, (t+1)*C), C = Nkv / P, that the ring delivers in turn: arganzheng.life,
 * multi-GPU diffusion parallelism, section 4.2 "Ring"; MindIE SD "多卡并行" page, Ring
 * Sequence Parallel section), laid out as attn_merge_lse takes them.  For each chunk t,
 * (o_parts[t], lse_parts[t]) is what attn_fwd_lse returns for q against keys and
 * values [t*C, (t+1)*C); merging the P results gives attention over all Nkv keys.  One
 * call keeps every (chunk, query tile) pair on the GPU at once, where P separate calls
 * on short chunks would each leave CUs idle.
 *
 *   q, k, v, softmax_scale   as attn_fwd_lse (k and v hold all Nkv keys)
 *   o_parts    o_dtype [P, B, Nq, H, D]
 *   lse_parts  f32 [P, B, H, Nq]
 *   P          number of chunks, >= 1, dividing Nkv
 *
 * Errors: as attn_fwd_lse, and DTL_ERR_INVALID_ARG for P <= 0 or P not dividing Nkv.
 */
dtl_status attn_fwd_lse_kv_chunks(const void *q, const void *k, const void *v,
                                  void *o_parts, float *lse_parts,
                                  int B, int Nq, int Nkv, int H, int D, int P,
                                  float softmax_scale, dtl_dtype o_dtype, hipStream_t stream);

/*
 * attn_merge_lse - exact merge of P partial attention results over disjoint key sets.
 *
 * For every (b, n, h), with parts t = 0..P-1:
 *     L           = ln sum_t exp(lse_parts[t,b,h,n])
 *     o[b,n,h,:]  = sum_t exp(lse_parts[t,b,h,n] - L) * o_parts[t,b,n,h,:]
 *     lse[b,h,n]  = L
 * This is the online-softmax accumulation that Ring attention performs across its
 * rounds (arganzheng.life, multi-GPU diffusion parallelism, section 4.2 "Ring";
 * MindIE SD "多卡并行" page, Ring Sequence Parallel section).  When the parts are
 * attn_fwd_lse results over a partition of the keys, the merge equals attention
 * over all keys.  A part with lse = -inf holds no keys and contributes nothing; a
 * row whose parts are all -inf yields o = 0 and lse = -inf.
 *
 *   o_parts    parts_dtype [P, B, N, H, D]  (f32 recommended; bf16 accepted)
 *   lse_parts  f32 [P, B, H, N]
 *   o          out_dtype [B, N, H, D]
 *   lse        f32 [B, H, N], or NULL to skip writing it
 *
 * Errors: DTL_ERR_INVALID_ARG for null inputs or o, sizes <= 0, misalignment, or an
 * output overlapping an input; DTL_ERR_UNSUPPORTED for D not a multiple of 8, P > 256,
 * or a dtype outside {DTL_BF16, DTL_F32}.
 */
dtl_status attn_merge_lse(const void *o_parts, const float *lse_parts,
                          void *o, float *lse,
                          int P, int B, int N, int H, int D,
                          dtl_dtype parts_dtype, dtl_dtype out_dtype, hipStream_t stream);

/*
 * seq_to_head_permute - the local data movement of a Ulysses all-to-all.
 *
 * Turns p sequence shards ("N/p tokens x all H heads" on each rank) into p head
 * shards ("all N tokens x H/p heads"): head group j = heads [j*H/p, (j+1)*H/p),
 * tokens concatenated in source-rank order (arganzheng.life section 4.1 and its
 * figure; MindIE SD "多卡并行" page, Ulysses usage example: split the head axis
 * into p parts, exchange, concatenate along tokens; "AIGC 分布式推理" CP section's
 * [13640 tokens, 24 heads] -> [27280 tokens, 12 heads] at p = 2):
 *     out[j][b][s*(N/p) + n][hh][d] = in[s][b][n][j*(H/p) + hh][d]
 *
 *   in   [p, B, N/p, H, D]    the p sequence shards, in rank order
 *   out  [p, B, N, H/p, D]    the p head shards; out[j] is what rank j receives
 *   elem_bytes  1, 2, 4 or 8 (2 for bf16); the copy is bit-exact
 *
 * Errors: DTL_ERR_INVALID_ARG for null or overlapping buffers, sizes <= 0,
 * misalignment, p not dividing N or H; DTL_ERR_UNSUPPORTED for another elem_bytes.
 */
dtl_status seq_to_head_permute(const void *in, void *out,
                               int p, int B, int N, int H, int D,
                               int elem_bytes, hipStream_t stream);

/*
 * head_to_seq_permute - the local data movement of the Ulysses all-to-all after
 * attention (the inverse of seq_to_head_permute).
 *
 * Turns p head shards ("all N tokens x H/p heads": each rank's attention output) back
 * into p sequence shards ("N/p tokens x all H heads"): token range s = [s*N/p,
 * (s+1)*N/p), head groups concatenated in source-rank order (arganzheng.life section
 * 4.1 figure, the O all-to-all that returns to the token split; MindIE SD "多卡并行"
 * page, Ulysses usage example: split the attention output into p token ranges,
 * exchange, concatenate along heads):
 *     out[s][b][n][j*(H/p) + hh][d] = in[j][b][s*(N/p) + n][hh][d]
 *
 *   in   [p, B, N, H/p, D]    the p head shards; in[j] holds heads [j*H/p, (j+1)*H/p)
 *   out  [p, B, N/p, H, D]    the p sequence shards; out[s] is what rank s receives
 *   elem_bytes  1, 2, 4 or 8; the copy is bit-exact
 *
 * Errors: as seq_to_head_permute.
 */
dtl_status head_to_seq_permute(const void *in, void *out,
                               int p, int B, int N, int H, int D,
                               int elem_bytes, hipStream_t stream);

/*
 * qkv_seq_to_head_permute - one pass that performs seq_to_head_permute on Q, K and V
 * together, the local data movement of a fused QKV all-to-all ("AIGC 分布式推理：从
 * Wan2.2 理解 DP/TP/CP/SP/PP", CP section: per self-attention one fused QKV all-to-all
 * and one for the output).  The input is the fused QKV projection's layout, each
 * token's row holding its q, k and v of all heads side by side; the output gives every
 * head group three separate BSND tensors that attn_fwd_lse takes directly (c = 0, 1, 2
 * for q, k, v):
 *     out[j][c][b][s*(N/p) + n][hh][d] = in[s][b][n][c][j*(H/p) + hh][d]
 *
 *   in   [p, B, N/p, 3, H, D]   the p sequence shards of packed q, k, v
 *   out  [p, 3, B, N, H/p, D]   out[j][0], out[j][1], out[j][2]: rank j's q, k, v
 *   elem_bytes  1, 2, 4 or 8; the copy is bit-exact
 *
 * Errors: as seq_to_head_permute.
 *
 * The three permutes move runs of (H/p)*D elements with copies of the largest of 16, 8,
 * 4, 2 or 1 bytes that divides a run; a call of more than 2^31 - 256 such units (32 GiB
 * with 16-byte units) is rejected with DTL_ERR_INVALID_ARG.
 */
dtl_status qkv_seq_to_head_permute(const void *in, void *out,
                                   int p, int B, int N, int H, int D,
                                   int elem_bytes, hipStream_t stream);

/*
 * qkv_norm_rope_permute - QK-RMSNorm and rotary position embedding of packed q, k, v,
 * written straight into the head shards of the fused QKV all-to-all (one pass).
 *
 * For every token t = s*(N/p) + n (source shard s, row n; t is the position in the
 * whole sequence) and c = 0 (q) or 1 (k), over the token's H*D hidden values x:
 *     y_e = x_e * gamma_c[e] / sqrt(mean_e(x_e^2) + eps)          e = h*D + d
 * then, per head h and pair i < D/2 (elements d = 2i, 2i+1 of the head):
 *     out_2i   = y_2i * cos[t][i] - y_2i+1 * sin[t][i]
 *     out_2i+1 = y_2i * sin[t][i] + y_2i+1 * cos[t][i]
 * and v (c = 2) unchanged, each placed where qkv_seq_to_head_permute puts it.  The QK
 * RMSNorm spans all heads of a token and the 3D RoPE acts by token position with cos/sin
 * sliced by the same token range ("AIGC 分布式推理：从 Wan2.2 理解 DP/TP/CP/SP/PP", TP
 * section and CP section); the pairing (2i, 2i+1) and the table form are this library's
 * reading, which any multi-axis RoPE fits by its cos/sin tables.  p = 1 gives the norm and
 * the rotation alone, out [1, 3, B, N, H, D].
 *
 *   qkv      bf16 [p, B, N/p, 3, H, D]   sequence shards of packed q, k, v
 *   gamma_q  f32 [H*D], gamma_k f32 [H*D] the norms' weights
 *   cos, sin f32 [N, D/2]               per token position of the whole sequence
 *   out      bf16 [p, 3, B, N, H/p, D]   out[j][0..2]: head group j's q, k, v
 *   eps      finite and >= 0
 * Arithmetic in f32, one rounding to bf16 (nearest even) per output element.
 *
 * Errors: DTL_ERR_INVALID_ARG for null pointers, sizes <= 0, p not dividing N or H, a
 * negative or non-finite eps, misalignment, or out overlapping an input;
 * DTL_ERR_UNSUPPORTED for D not in {64, 128} or H*D > 8192.
 */
dtl_status qkv_norm_rope_permute(const void *qkv, const float *gamma_q, const float *gamma_k,
                                 const float *cos, const float *sin, void *out,
                                 int p, int B, int N, int H, int D, float eps,
                                 hipStream_t stream);

/* A static, human-readable name of a status code (never NULL). */
const char *dtl_status_string(dtl_status s);

#ifdef __cplusplus
}
#endif

#endif /* DTL_H */
