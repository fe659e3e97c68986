/*
 * pagedattn.h — C ABI of the gfx950 paged decode-attention library.
 *
 * What it computes.  Single-token decode attention over a paged KV cache
 * (PagedAttention).  For every sequence b and query head h, with
 * L = seq_lens[b] and KV head g = h / (num_q_heads / num_kv_heads):
 *
 *     s_t   = scale * <q[b][h], K_b[t]>                  t = 0 .. L-1
 *     w_t   = exp(s_t - max_u s_u) / sum_u exp(s_u - max_u s_u)
 *     out[b][h] = sum_t w_t * V_b[t]
 *
 * where K_b[t] / V_b[t] is the key / value row of logical token t, found by
 * following the block table: physical block block_tables[b][t / B], slot
 * t % B, KV head g.  This is ordinary exact attention with only the
 * addressing changed ("39 · PagedAttention", §1 "What attention needs",
 * §2 "The paged version" and the IMPORTANT box; the softmax(QK^T/sqrt(d))V
 * definition is in "FlashAttention vs PagedAttention", section "What does
 * FlashAttention optimize?").  Query heads are grouped onto KV heads
 * consecutively (grouped-query attention, "PagedAttention: The Cache Was
 * Storing Nothing", §3.1 "Sharing the keys and values"; the pages fix no
 * index convention, this library fixes g = h / G).
 *
 * Device memory layouts (row-major, dense, element = one value of `dtype`):
 *
 *   q            [num_seqs][num_q_heads][head_dim]              dtype
 *   out          [num_seqs][num_q_heads][head_dim]              out_dtype
 *   k_pool       [num_blocks][num_kv_heads][block_size][head_dim]   token-major
 *   v_pool       [num_blocks][num_kv_heads][block_size/16][head_dim][16]
 *   block_tables int32 [num_seqs][max_blocks_per_seq]
 *   seq_lens     int32 [num_seqs]
 *
 * One (physical block, KV head) tile of either pool is one contiguous
 * block_size*head_dim*esize-byte range (4 KiB for bf16/fp16 with 16-token
 * blocks), so a block is read as a single coalesced burst.  K is stored
 * token-major (a token's key row is contiguous: the reduction axis of q.k).
 * V is stored transposed inside each group of 16 tokens (for one value
 * dimension the group's 16 values are contiguous: the reduction axis of
 * w.V), groups in token order, so every 16 consecutive tokens of a block
 * are one contiguous K range and one contiguous V range whatever the block
 * size.  Both choices put each product's reduction axis innermost, which
 * is the operand layout the gfx950 matrix cores consume directly.
 *
 * Table semantics.  Sequence b has n_b = ceil(L / block_size) logical
 * blocks; entries j >= n_b of its table row are never read (they may hold
 * -1).  Slots of the last block at or beyond L - (n_b-1)*block_size are
 * never part of the result, whatever they hold.  Physical blocks may be
 * shared by several sequences (prefix sharing: "PagedAttention: The Cache
 * Was Storing Nothing", §2.3).  L = 0 gives out = 0.
 *
 * Ownership and threading.  The caller allocates every buffer (including
 * the workspace) and owns the stream.  The library allocates nothing, keeps
 * no pointer after a call returns and holds no state between calls, except
 * the static scratch of paged_attn_decode_noalloc (one array per GPU,
 * allocated with the library's code object).  Calls
 * are asynchronous on `stream` (a hipStream_t; NULL = the null stream).
 * Calls that share a workspace must be ordered on one stream.  `out` must
 * not alias any input.
 *
 * Errors.  Every function that can fail returns a pa_status; no exception
 * crosses the ABI.  Descriptor and pointer errors are detected on the host
 * before anything is launched.  Data-dependent preconditions (every used
 * table id in [0, num_blocks), 0 <= seq_lens[b] <= max_blocks_per_seq *
 * block_size) are NOT checked on the device; pa_validate_host checks them
 * on host copies.  A launch failure returns PA_ERR_LAUNCH.
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL = 1,        /* a required pointer is NULL */
  PA_ERR_SHAPE = 2,       /* a size is <= 0 (cached_prefix_blocks < 0), or num_q_heads % num_kv_heads != 0 */
  PA_ERR_DTYPE = 3,       /* unknown dtype, or out_dtype neither PA_F32 nor dtype */
  PA_ERR_UNSUPPORTED = 4, /* valid but not built: head_dim, block_size, group size, kernel/dtype pair,
                             or the decode workgroup's LDS (length prefix of a very large batch plus
                             the group-16 staging) does not fit a CU */
  PA_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than pa_workspace_bytes() */
  PA_ERR_ALIGN = 6,       /* q, pools or out not 16-byte aligned */
  PA_ERR_LAUNCH = 7,      /* the HIP launch reported an error */
  PA_ERR_TABLE = 8,       /* pa_validate_host: table id out of range or bad seq_len */
  PA_ERR_DEVICE = 9,      /* device query failed or the device is not gfx950 */
  PA_ERR_NOMEM = 10,      /* block manager: not enough free physical blocks */
  PA_ERR_SCRATCH = 11     /* paged_attn_decode_noalloc: the call needs more than its static scratch */
} pa_status;

typedef enum pa_dtype {
  PA_F32 = 0,
  PA_F16 = 1, /* IEEE binary16 */
  PA_BF16 = 2 /* bfloat16: the upper 16 bits of an IEEE binary32 */
} pa_dtype;

/* Which decode kernel runs.  AUTO picks the matrix-core kernel for fp16/bf16
 * and the vector-ALU kernel for fp32.  Forcing a kernel is for tests and
 * measurement; MFMA with PA_F32 returns PA_ERR_UNSUPPORTED. */
typedef enum pa_kernel {
  PA_KERNEL_AUTO = 0,
  PA_KERNEL_VALU = 1, /* vector ALU, DPP row reductions; any dtype */
  PA_KERNEL_MFMA = 2  /* gfx950 matrix cores for the query-group products */
} pa_kernel;

typedef struct pa_desc {
  int32_t num_seqs;           /* >= 1 */
  int32_t num_q_heads;        /* Hq, multiple of num_kv_heads */
  int32_t num_kv_heads;       /* Hkv >= 1; group size G = Hq / Hkv in {1, 2, 4, 8, 16} */
  int32_t head_dim;           /* D; built: 128 */
  int32_t block_size;         /* B tokens per block; built: 16, 32 */
  int32_t num_blocks;         /* physical blocks in each pool */
  int32_t max_blocks_per_seq; /* row stride of block_tables */
  int32_t dtype;              /* pa_dtype of q, k_pool, v_pool */
  int32_t out_dtype;          /* PA_F32, or equal to dtype (round to nearest even) */
  int32_t kernel;             /* pa_kernel */
  /* Cache hint, >= 0 (0: none).  The first cached_prefix_blocks logical
   * blocks of every sequence may be shared with other sequences of the
   * batch (prefix sharing, "PagedAttention: The Cache Was Storing
   * Nothing", §2.3): they are read with a cache-retaining policy so that
   * the sequences sharing them hit in L2 / Infinity Cache.  All other K/V
   * is streamed with a non-temporal policy (read once per call).  Results
   * do not depend on it. */
  int32_t cached_prefix_blocks;
} pa_desc;

/* Human-readable name of a status code (static storage, never NULL). */
const char* pa_status_str(int32_t status);

/* Bytes of one element of `dtype`, 0 if unknown. */
size_t pa_dtype_size(int32_t dtype);

/* Logical blocks a sequence of `len` tokens occupies: ceil(len / block_size),
 * 0 when len <= 0 or block_size <= 0.  The last block holds
 * len - (n-1)*block_size tokens ("FlashAttention vs PagedAttention", the
 * sizing example's block rounding). */
int64_t pa_blocks_for_len(int64_t len, int32_t block_size);

/* Bytes of ONE pool (k_pool and v_pool have the same size):
 * num_blocks * num_kv_heads * block_size * head_dim * esize. 0 on a bad desc. */
size_t pa_pool_bytes(const pa_desc* desc);

/* Element offset of K[block][kv_head][slot][dim] inside k_pool, and of the
 * same logical element of V inside v_pool.  -1 if an index is out of range
 * or the descriptor is invalid. */
int64_t pa_k_elem_offset(const pa_desc* desc, int32_t block, int32_t kv_head,
                         int32_t slot, int32_t dim);
int64_t pa_v_elem_offset(const pa_desc* desc, int32_t block, int32_t kv_head,
                         int32_t slot, int32_t dim);

/* Bytes of device workspace that paged_attn_decode needs for this
 * descriptor; 0 on a bad descriptor.  The workspace holds, for sequences
 * split across workgroups, their partial results and one arrival counter
 * per split.  It must be zero-filled once before its first use (e.g.
 * hipMemset); every call leaves it zeroed again, so it can be reused
 * without clearing.  Calls that share a workspace must not overlap. */
size_t pa_workspace_bytes(const pa_desc* desc);

/* Checks the descriptor, then the data-dependent preconditions on HOST
 * copies of the block table and lengths: 0 <= seq_lens[b] <=
 * max_blocks_per_seq*block_size and block_tables[b][j] in [0, num_blocks)
 * for every j < n_b.  PA_OK, a descriptor error, or PA_ERR_TABLE. */
int32_t pa_validate_host(const pa_desc* desc, const int32_t* block_tables_host,
                         const int32_t* seq_lens_host);

/* Checks a descriptor alone (what every launching entry point checks). */
int32_t pa_check_desc(const pa_desc* desc);

/* Paged decode attention: one kernel launch on `stream` per 8192
 * sequences (the launch keeps its batch's length prefix in LDS; a larger
 * batch runs as consecutive launches over sequences 0-8191, 8192-16383,
 * ..., each with the same workspace).  All pointers are
 * device pointers in the layouts above; `scale` multiplies q.k
 * (1/sqrt(head_dim) for standard attention).  workspace: device buffer of
 * at least pa_workspace_bytes(desc) bytes, zeroed before its first use.
 *
 * Work split (the sequence split of "PagedAttention: The Cache Was Storing
 * Nothing", "Where this goes next"): the (sequence, KV head, logical block)
 * units of the batch are cut into equal contiguous chunks, one per
 * workgroup.  A (sequence, KV head) cut by chunk boundaries produces one
 * (max, sum-of-exp, weighted-V) partial per chunk, and the workgroup that
 * finishes last folds them with
 *   m = max(m1, m2),  l = l1*e^(m1-m) + l2*e^(m2-m),  o = o1*e^(m1-m) + o2*e^(m2-m)
 * ("39 · PagedAttention", §3 "On the GPU", merge equation) into out = o / l. */
int32_t paged_attn_decode(const void* q, const void* k_pool, const void* v_pool,
                          const int32_t* block_tables, const int32_t* seq_lens,
                          float scale, void* out, const pa_desc* desc,
                          void* workspace, size_t workspace_bytes, void* stream);

/* paged_attn_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops that
 * forbid allocation, harnesses without an allocator).  It allocates
 * nothing: the split counters and partials live in a static 8 MiB device
 * array inside the library, one per GPU, held until the process ends.  The
 * caller still provides q, the pools, the tables, the lengths and out, in
 * the layouts above; results are those of paged_attn_decode (same kernels,
 * same fold order).
 *
 * Two launches on `stream` per 8192 sequences: a small kernel that zeroes
 * the split counters, then the decode kernel.  Every call on one GPU shares that GPU's array,
 * which keeps the last call's contents: calls that overlap on one GPU (on
 * different streams, or from different host threads without ordering)
 * race and may produce wrong results; order them on one stream.
 *
 * The call needs 4 * grid bytes of counters (rounded up to 256) plus
 * 2 * grid * G * (head_dim + 2) * 4 bytes of partials, grid =
 * pa_decode_grid(desc), G = num_q_heads / num_kv_heads: 1.06 MB at G = 4
 * and 4.26 MB at G = 16 on a 256-CU gfx950.  A call that needs more than
 * 8 MiB returns PA_ERR_SCRATCH and launches nothing.  Other errors as for
 * paged_attn_decode (no PA_ERR_WORKSPACE). */
int32_t paged_attn_decode_noalloc(const void* q, const void* k_pool, const void* v_pool,
                                  const int32_t* block_tables, const int32_t* seq_lens,
                                  float scale, void* out, const pa_desc* desc, void* stream);

/* Number of decode workgroups a launch uses for this descriptor on the
 * current device (the split-K granularity: CUs x resident workgroups per
 * CU; of each launch, for a batch of more than 8192 sequences), or -1 on
 * error or when the workgroup's LDS does not fit a CU. */
int32_t pa_decode_grid(const pa_desc* desc);

/* ------------------------------------------------------------------
 * Decode with prefix groups: blocks that several sequences share are read
 * once for the whole group.
 * ------------------------------------------------------------------ */

/* Sequences that start with the same prompt point their block tables at
 * the same physical blocks ("PagedAttention: The Cache Was Storing
 * Nothing", §2.3 "What the table buys that reservations could not").
 * paged_attn_decode reads such a block once per sequence; this call is
 * told which sequences share how many leading blocks and reads every
 * shared block once per group: the group's query heads meet each shared
 * K/V tile in one pass (up to 32 / G members per pass, as the columns of
 * one matrix-core tile pair), and each member's result is the merge of its
 * shared part and its remaining blocks ("39 · PagedAttention", §3 merge
 * equation).  The result is the same attention as paged_attn_decode's (up
 * to fp32 rounding order).
 *
 * Groups.  Group i is the consecutive sequences group_start[i] ..
 * group_start[i+1]-1 (device int32 [num_groups + 1], non-decreasing,
 * group_start[num_groups] <= num_seqs; sequences outside every group share
 * nothing).  group_shared[i] (device int32 [num_groups], >= 0): the leading
 * table entries every member shares.  Precondition: for every member b and
 * j < min(group_shared[i], n_b), block_tables[b][j] is the same physical
 * block for all members (a member shorter than the shared prefix shares
 * the blocks it has; its last one is partly its own).  Groups with fewer
 * than two members or no shared block run as ordinary sequences.
 *
 * Built for fp16 / bf16 on the matrix-core kernel with G = Hq/Hkv in
 * {1, 2, 4, 8} and batches of at most 8192 sequences; for every other
 * descriptor (and for num_groups == 0) the call runs paged_attn_decode
 * with the same workspace, so results are always defined.
 *
 * workspace: at least pa_shared_workspace_bytes(desc) bytes, zero-filled
 * before its first use; every call leaves it zeroed again.  One launch on
 * `stream` (paged_attn_decode's launches when it runs that).  Errors as
 * for paged_attn_decode, plus PA_ERR_SHAPE for
 * num_groups < 0 and PA_ERR_NULL for missing group arrays; PA_ERR_UNSUPPORTED
 * when the schedule of this batch and its groups does not fit the
 * workgroup's LDS (about 36 bytes per sequence and 4 per group besides the
 * ordinary decode's).  Data-dependent preconditions are checked by
 * pa_validate_shared_host, not on the device. */
int32_t paged_attn_decode_shared(const void* q, const void* k_pool, const void* v_pool,
                                 const int32_t* block_tables, const int32_t* seq_lens,
                                 const int32_t* group_start, const int32_t* group_shared,
                                 int32_t num_groups, float scale, void* out, const pa_desc* desc,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of paged_attn_decode_shared (the ordinary decode's
 * workspace, then per-(sequence, KV head) arrival counters and partials,
 * and partials of shared parts cut by chunk boundaries; the ordinary
 * decode's alone for more than 8192 sequences); 0 on a bad descriptor. */
size_t pa_shared_workspace_bytes(const pa_desc* desc);

/* Workgroups of a paged_attn_decode_shared launch for this descriptor and
 * group count on the current device, or -1 (error, not built, or the LDS
 * does not fit). */
int32_t pa_decode_shared_grid(const pa_desc* desc, int32_t num_groups);

/* pa_validate_host, then the groups on HOST copies: group bounds ordered
 * and inside the batch, group_shared >= 0 (PA_ERR_SHAPE otherwise), and
 * the shared table entries equal across each group's members
 * (PA_ERR_TABLE otherwise). */
int32_t pa_validate_shared_host(const pa_desc* desc, const int32_t* block_tables_host,
                                const int32_t* seq_lens_host, const int32_t* group_start_host,
                                const int32_t* group_shared_host, int32_t num_groups);

/* ------------------------------------------------------------------
 * Paged prefill: many query rows per sequence, causal.
 * ------------------------------------------------------------------ */

/* Causal prefill attention over the paged cache, one kernel launch on
 * `stream` ("FlashAttention vs PagedAttention", "How prefill and decode
 * change the diagnosis": prefill scores many prompt positions against a
 * cache whose length differs from the query count; "Paging the KV cache
 * with a fused mask", "What carries the argument": every query reads
 * exactly its own sequence's pages).
 *
 * q, out: [total_q][num_q_heads][head_dim], total_q = q_start[num_seqs].
 * q_start: int32 [num_seqs + 1] row offsets, q_start[0] = 0.  Sequence b
 * owns rows q_start[b] .. q_start[b+1]-1: its NEWEST n_b = q_start[b+1] -
 * q_start[b] tokens, whose K/V are already in the pools (written with
 * paged_kv_append or by the caller); row i sits at position
 * seq_lens[b] - n_b + i and attends tokens 0 .. that position (the causal
 * mask aligned to the end of the sequence).  n_b = seq_lens[b] is a whole
 * prompt, smaller n_b a chunk of one; n_b = 0 leaves the sequence out.
 * max_q_len >= every n_b (launch size; rows beyond it are not computed).
 * Pools, block_tables, seq_lens, scale, dtype, out_dtype: as for
 * paged_attn_decode.  No workspace.  Matrix cores only: fp16 / bf16 with
 * kernel AUTO or MFMA, else PA_ERR_UNSUPPORTED.  Accuracy as for the
 * decode (fp32 accumulation, max |out - exact| <= 2e-3 for 16-bit inputs):
 * the probabilities enter the weighted values rounded once to fp16, with
 * the row sums over the same rounded values.  bf16 V is converted to fp16
 * as it is staged (exact for magnitudes in [2^-17, 2^16); smaller ones
 * move by less than 2^-24); a workgroup that meets a V value of magnitude
 * 2^16 or more (or an infinity) reruns its rows with V in bf16 and the
 * probabilities as two bf16 halves (about 16 bits).  Data-dependent
 * preconditions are checked by
 * pa_validate_prefill_host, not on the device; a sequence with
 * n_b > seq_lens[b] is skipped by the kernel. */
int32_t paged_attn_prefill(const void* q, const void* k_pool, const void* v_pool,
                           const int32_t* block_tables, const int32_t* seq_lens,
                           const int32_t* q_start, int32_t max_q_len, float scale, void* out,
                           const pa_desc* desc, void* stream);

/* pa_validate_host on host copies, then: q_start[0] == 0 and
 * 0 <= q_start[b+1] - q_start[b] <= min(max_q_len, seq_lens[b]).  PA_OK, a
 * descriptor error, PA_ERR_NULL, PA_ERR_SHAPE (max_q_len < 0) or
 * PA_ERR_TABLE. */
int32_t pa_validate_prefill_host(const pa_desc* desc, const int32_t* block_tables_host,
                                 const int32_t* seq_lens_host, const int32_t* q_start_host,
                                 int32_t max_q_len);

/* ------------------------------------------------------------------
 * Writing the cache: the steps around the decode call on the same layout.
 * ------------------------------------------------------------------ */

/* Append one new token per sequence.  For every sequence b with
 * t = positions[b] >= 0, the token's key and value rows of every KV head
 * are written to logical slot t of the sequence: physical block
 * block_tables[b][t / block_size], slot t % block_size, in the pool
 * layouts above.  The block table maps logical blocks to physical ones,
 * so the writer follows it exactly like the reader, and only a sequence's
 * last block is ever partly filled ("PagedAttention: The Cache Was Storing
 * Nothing", §2.2 "Borrowing paging from the 1960s").  For the usual decode
 * step positions[b] = seq_lens[b] before the step (the caller grows the
 * table by one block first when t % block_size == 0); positions[b] < 0
 * writes nothing for b.
 *
 *   k_new, v_new  [num_seqs][num_kv_heads][head_dim]  dtype, device
 *   k_pool, v_pool, block_tables                    as above, device
 *   positions     int32 [num_seqs], device
 *
 * Uses num_seqs, num_kv_heads, head_dim, block_size, num_blocks,
 * max_blocks_per_seq and dtype of `desc` (which must pass pa_check_desc).
 * One kernel launch on `stream`; every other pool byte is left as it was.
 * Data-dependent preconditions are not checked on the device (see
 * pa_validate_append_host): t < max_blocks_per_seq*block_size, the table
 * entry in [0, num_blocks), and no two sequences of one call writing the
 * same (block, slot) -- such a pair races and either value may land.
 * Returns PA_OK, a descriptor error, PA_ERR_NULL, PA_ERR_ALIGN (pointers
 * not 16-byte aligned), PA_ERR_DEVICE or PA_ERR_LAUNCH. */
int32_t paged_kv_append(const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                        const int32_t* block_tables, const int32_t* positions,
                        const pa_desc* desc, void* stream);

/* Host check of paged_kv_append's data-dependent preconditions on HOST
 * copies: every positions[b] >= 0 below max_blocks_per_seq*block_size,
 * its table entry in [0, num_blocks), and (block, slot) targets pairwise
 * distinct.  PA_OK, a descriptor error, PA_ERR_NULL or PA_ERR_TABLE. */
int32_t pa_validate_append_host(const pa_desc* desc, const int32_t* block_tables_host,
                                const int32_t* positions_host);

/* Copy whole physical blocks, the copy-on-write step of block sharing: a
 * shared block is copied only when one of the sequences pointing at it
 * diverges and writes into it ("PagedAttention: The Cache Was Storing
 * Nothing", §2.3 "What the table buys that reservations could not").
 * For i < num_pairs, block dst_blocks[i] of both pools becomes a copy of
 * block src_blocks[i] (every KV head, every slot: one contiguous
 * num_kv_heads*block_size*head_dim*esize-byte range per pool).  The
 * caller then points the diverging sequence's table entry at the copy.
 *
 *   src_blocks, dst_blocks  int32 [num_pairs], device
 *
 * num_pairs == 0 launches nothing.  One kernel launch on `stream`.
 * Preconditions not checked on the device (see pa_validate_copy_host):
 * ids in [0, num_blocks), destinations pairwise distinct and none of
 * them also a source (otherwise the result depends on the order of the
 * copies).  Returns PA_OK, a descriptor error, PA_ERR_SHAPE (num_pairs <
 * 0), PA_ERR_NULL, PA_ERR_ALIGN, PA_ERR_DEVICE or PA_ERR_LAUNCH. */
int32_t paged_kv_copy_blocks(void* k_pool, void* v_pool, const int32_t* src_blocks,
                             const int32_t* dst_blocks, int32_t num_pairs,
                             const pa_desc* desc, void* stream);

/* Host check of paged_kv_copy_blocks' preconditions on HOST copies of the
 * id lists.  PA_OK, a descriptor error, PA_ERR_SHAPE, PA_ERR_NULL or
 * PA_ERR_TABLE. */
int32_t pa_validate_copy_host(const pa_desc* desc, const int32_t* src_blocks_host,
                              const int32_t* dst_blocks_host, int32_t num_pairs);

/* ------------------------------------------------------------------
 * Block-wise eviction scoring ("PagedEviction: Structured Block-wise KV
 * Cache Pruning for Efficient Large Language Model Inference", the review's
 * "Core claim" and "What carries the argument"): a token's importance is
 * the ratio of its value norm to its key norm, read from the cached rows,
 * and a block's score is the mean over its tokens; during decode, when a
 * sequence's most recent block has just filled, the block with the lowest
 * score is the one to evict.
 * ------------------------------------------------------------------ */

/* For every sequence b (L = seq_lens[b]) and every full logical block
 * j < L / block_size:
 *
 *   block_scores[b][j] = (1/B) * sum over the B tokens t of block j of
 *                        ||V_b[t]||_2 / ||K_b[t]||_2
 *
 * where K_b[t] / V_b[t] is token t's whole key / value row of the layer:
 * all num_kv_heads * head_dim elements (pages through the table as for the
 * decode call).  Entries j >= L / block_size are set to NaN.
 * evict[b] = the full block with the lowest score (the lowest j among
 * equal scores) when L > 0 and L % block_size == 0, else -1.  Scores are
 * accumulated in fp32.  The library only scores and chooses: dropping the
 * block from the sequence's table is the caller's.  A token whose key and
 * value rows are both all-zero scores NaN and the choice is then undefined.
 *
 *   block_scores  float [num_seqs][max_blocks_per_seq], device
 *   evict         int32 [num_seqs], device
 *
 * Two kernel launches on `stream` (scores, then the choice).  Data-dependent
 * preconditions as for paged_attn_decode (pa_validate_host).  Returns PA_OK,
 * a descriptor error, PA_ERR_NULL, PA_ERR_ALIGN, PA_ERR_DEVICE or
 * PA_ERR_LAUNCH. */
int32_t paged_kv_block_scores(const void* k_pool, const void* v_pool,
                              const int32_t* block_tables, const int32_t* seq_lens,
                              float* block_scores, int32_t* evict, const pa_desc* desc,
                              void* stream);

/* ------------------------------------------------------------------
 * Host block manager (plain C++ on the host; touches no device memory).
 * "PagedAttention: The Cache Was Storing Nothing", §2.2: the cache is cut
 * into fixed-size blocks and every request's block table maps its logical
 * blocks to physical ones; since every free block has the same size any
 * free block will do, and only a request's last block is partly filled.
 * §2.3: tables may point at the same physical blocks (shared prompts, beam
 * search); a block is copied only when a sequence diverges and writes
 * into it.  Ids come from a bump pointer (never-used blocks in id order)
 * and a free-list stack (released blocks, most recent first), O(1) each;
 * every block counts the table entries that point at it.
 *
 * Lock-free ("Paged Attention Meets FlexAttention", "What carries the
 * argument": pages handed out in constant time without locks): any number
 * of threads may call into one manager at once.  pa_bm_alloc and
 * pa_bm_prepare_append stay all or nothing under concurrency (their blocks
 * are reserved before any is taken).  What a caller must still order
 * itself: calls that update the same table rows, and sharing or releasing
 * a block while a concurrent pa_bm_prepare_append writes into it (forking
 * a sequence in the middle of its own append step).  Called from one
 * thread, every result equals that of the plain model of the tests.
 * A call moves all of its blocks on or off the free list in one exchange,
 * so under contention ask for a step's blocks in one call rather than one
 * block per call.
 * ------------------------------------------------------------------ */

typedef struct pa_block_manager pa_block_manager; /* opaque */

/* A manager of num_blocks physical blocks of block_size tokens, all free.
 * NULL if num_blocks <= 0, block_size <= 0 or out of memory.  Owned by the
 * caller; release with pa_bm_destroy. */
pa_block_manager* pa_bm_create(int32_t num_blocks, int32_t block_size);
void pa_bm_destroy(pa_block_manager* bm);

/* Free blocks, or -1 for NULL. */
int32_t pa_bm_num_free(const pa_block_manager* bm);

/* Table entries pointing at `block` (0 = free), -1 if out of range / NULL. */
int32_t pa_bm_refcount(const pa_block_manager* bm, int32_t block);

/* n fresh blocks (one reference each) into ids[0..n): all or nothing.
 * PA_ERR_NOMEM (nothing taken) when fewer than n are free; PA_ERR_SHAPE for
 * n < 0; PA_ERR_NULL for NULL arguments (ids may be NULL when n == 0). */
int32_t pa_bm_alloc(pa_block_manager* bm, int32_t n, int32_t* ids);

/* Drop one reference of each of ids[0..n), in order; a block whose count
 * reaches 0 is free again (a finished sequence releases its table row; an
 * evicted block is released alone).  PA_ERR_TABLE at the first id that is
 * out of range or holds no reference (the ones before it are dropped). */
int32_t pa_bm_release(pa_block_manager* bm, const int32_t* ids, int32_t n);

/* Add one reference to each of ids[0..n) (another table now points at the
 * block: a shared prefix, a forked beam).  PA_ERR_TABLE at the first id
 * that is free or out of range (the ones before it stay shared). */
int32_t pa_bm_share(pa_block_manager* bm, const int32_t* ids, int32_t n);

/* The host side of one decode step: make logical slot L = seq_lens[b]
 * writable for every sequence b, in order b = 0, 1, ...:
 *   L % block_size == 0: a fresh block goes into block_tables[b][L / B];
 *   otherwise, if block_tables[b][L / B] is shared (more than one
 *   reference): copy-on-write -- a fresh block d replaces the entry, one
 *   reference of the old block s is dropped, and the pair (s, d) is
 *   appended to cow_src / cow_dst for paged_kv_copy_blocks;
 *   positions[b] = L (for paged_kv_append).
 * seq_lens[b] < 0 skips b (positions[b] = -1).  All arrays are HOST
 * arrays: block_tables int32 [num_seqs][max_blocks_per_seq] (updated in
 * place), cow_src / cow_dst of num_seqs entries; *num_cow receives the
 * number of pairs.  All or nothing: PA_ERR_TABLE if some L / B >=
 * max_blocks_per_seq or some written entry is not a live block,
 * PA_ERR_NOMEM if the step needs more fresh blocks than are free; then
 * nothing changes (*num_cow = 0). */
int32_t pa_bm_prepare_append(pa_block_manager* bm, int32_t* block_tables,
                             int32_t max_blocks_per_seq, const int32_t* seq_lens,
                             int32_t num_seqs, int32_t* positions, int32_t* cow_src,
                             int32_t* cow_dst, int32_t* num_cow);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
