/*
 * fa.h -- C ABI of the block-sparse programmable attention library for MI355X (gfx950).
 *
 * Two operations, following the interface the pages state for FlexAttention
 * ("FlexAttention: compiler optimization of custom attention", sections 2, 4 and 5;
 * "FlexAttention: from rules to fused kernels", sections 1 and 2):
 *
 *   fa_create_block_mask  mask rule -> block tables (BCSR rows and their transposes)
 *   fa_block_mask_slice   rows of prebuilt tables for a shorter or offset geometry
 *   fa_block_mask_from_indices  selector candidate lists -> block tables
 *   fa_forward            O = softmax(mask(score_mod(Q K^T * scale))) V, plus LSE
 *   fa_forward_paged      the same over a paged KV cache (short-query path)
 *   fa_backward           dQ, dK, dV of fa_forward
 *
 * Conventions shared by every entry point
 *   - Every data pointer is a DEVICE pointer owned by the caller.  The library never
 *     allocates or frees device memory and keeps no state between calls, apart from
 *     a thread-local copy of the last error message.
 *   - All device work is enqueued on `stream` (a hipStream_t; NULL means the null
 *     stream) without any host synchronisation.  Inputs must stay alive and
 *     unmodified until that work has completed; this is the caller's duty.
 *   - Every argument is validated before anything is launched.  On any error
 *     nothing is written and no work is enqueued; the call returns a status code
 *     and fa_last_error_message() describes the failure.
 *   - Tensors are dense and contiguous, in the layouts stated per field.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* fa_stream_t; /* a hipStream_t */

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = 1,          /* a required pointer is NULL                                */
  FA_ERR_SHAPE = 2,         /* inconsistent or unsupported sizes                           */
  FA_ERR_UNSUPPORTED = 3,   /* head dim, block size or score kind outside the menu         */
  FA_ERR_MASK_SPEC = 4,     /* malformed mask program or parameter                         */
  FA_ERR_MASK_MISMATCH = 5, /* block tables built for other lengths / block sizes          */
  FA_ERR_WORKSPACE = 6,     /* workspace missing or smaller than required                  */
  FA_ERR_HIP = 7            /* a HIP runtime call or kernel launch failed                  */
} fa_status;

/* ----------------------------------------------------------------------------------
 * Mask rule: a postfix program over a fixed menu of element predicates M(b, i, j),
 * with i = local query row + q_offset (global position) and j the key position.
 *
 *   FA_M_CAUSAL        j <= i
 *   FA_M_SWA    (W)    j <= i and i - j < W, W >= 1; the window counts the current token
 *                      ("FlexAttention: compiler optimization of custom attention", sec. 1-2)
 *   FA_M_DOC           doc[b][i] == doc[b][j], doc IDs captured as an int32 tensor
 *                      ("FlexAttention: from rules to fused kernels", sec. 1.1)
 *   FA_M_PREFIX (P)    j < P or j <= i, P >= 0: bidirectional over the first P keys,
 *                      causal after ("FlexAttention: from rules to fused kernels", sec. 6.3)
 *   FA_M_AND, FA_M_OR  pop two values, push their intersection / union (and_masks/or_masks,
 *                      "FlexAttention: from rules to fused kernels", sec. 1.1)
 *
 * A well-formed program has 1..16 nodes, never pops an empty stack and leaves exactly
 * one value.  Decode uses q_offset so that rules see global positions
 * ("FlexAttention: compiler optimization of custom attention", sec. 6).
 * -------------------------------------------------------------------------------- */
enum {
  FA_M_CAUSAL = 1,
  FA_M_SWA = 2,
  FA_M_DOC = 3,
  FA_M_PREFIX = 4,
  FA_M_AND = 5,
  FA_M_OR = 6
};

#define FA_MASK_MAX_NODES 16

typedef struct {
  int32_t op;  /* FA_M_* */
  int32_t arg; /* W for FA_M_SWA, P for FA_M_PREFIX, ignored otherwise */
} fa_mask_node;

typedef struct {
  int32_t n;                                /* number of nodes, 1..16                      */
  fa_mask_node node[FA_MASK_MAX_NODES];     /* postfix order                               */
  const int32_t* doc_ids;                   /* device int32 [doc_batch, doc_len]; required
                                               iff the program contains FA_M_DOC           */
  int32_t doc_batch;                        /* 1 (shared by all batch entries) or B         */
  int64_t doc_len;                          /* >= q_offset + q_len and >= kv_len            */
} fa_mask_desc;

/* ----------------------------------------------------------------------------------
 * Block tables ("BlockMask"): the query/key plane is cut into block_q x block_kv
 * blocks; each block is EMPTY (no allowed pair), FULL (every in-range pair allowed)
 * or PARTIAL (otherwise) -- "FlexAttention: from rules to fused kernels", sec. 2.1,
 * 2.2 and 6.3.  Only in-range pairs (row < q_len, column < kv_len) are considered.
 *
 * Table extents B x H: B in {1, B_attn} and H in {1, Hq}; 1 broadcasts.  No rule of
 * the menu depends on the head, so H > 1 repeats identical rows per head.  A
 * document rule with doc_batch > 1 needs B == doc_batch.
 *
 * KV side (one row per query block, rows ordered (b', h', r), NQB = ceil(q_len/block_q)):
 *   kv_num[rows]        number of PARTIAL blocks of the row
 *   kv_ptr[rows + 1]    exclusive prefix sum of kv_num
 *   kv_idx[...]         their KV block indices, ascending within each row
 *   full_kv_num / full_kv_ptr / full_kv_idx   the same for FULL blocks
 * Q side (one row per KV block, ordered (b', h', c), NKB = ceil(kv_len/block_kv)):
 *   q_num / q_ptr / q_idx, full_q_num / full_q_ptr / full_q_idx  -- the exact
 *   transposes (query block indices, ascending), used by a backward pass
 *   ("Kernels: turning logical sparsity into real speed", sec. 4).
 * Partial and full lists never share a block.  Entries past ptr[rows] are unspecified.
 * All twelve arrays are caller-owned device int32 buffers sized by fa_block_mask_sizes.
 *
 * Work order (optional; "FlexAttention: from rules to fused kernels", sec. 5.2: the
 * row lengths of the tables are the signal for scheduling query tiles by their
 * executed blocks; "Kernels: turning logical sparsity into real speed", sec. 1.2 and 5):
 *   order[rows]  per table entry (b', h'), its NQB query block indices by descending
 *                executed-block count (kv_num + full_kv_num), ties by descending index.
 * When `order` is set, the table writers below fill it (NQB <= 4096, else
 * FA_ERR_UNSUPPORTED) and fa_forward / fa_backward hand out query blocks longest
 * first; when NULL, query blocks go out by descending index (the longest-first order
 * of causal-like rules).  The order changes only which workgroup runs first, never
 * where a result is written, so outputs are identical either way.
 * -------------------------------------------------------------------------------- */
typedef struct {
  fa_mask_desc mask;
  int32_t B, H;                     /* table extents                                   */
  int64_t q_len, kv_len, q_offset;  /* i_global = i + q_offset                          */
  int32_t block_q, block_kv;        /* powers of two, 1 .. 128 (64 or 128 to be read by
                                       fa_forward / fa_forward_paged / fa_backward)     */
  int32_t *kv_num, *kv_ptr, *kv_idx, *full_kv_num, *full_kv_ptr, *full_kv_idx;
  int32_t *q_num, *q_ptr, *q_idx, *full_q_num, *full_q_ptr, *full_q_idx;
  int32_t* order;   /* optional work order, [rows] or NULL -- see below */
} fa_block_mask;

/* Sizes for a block mask: rows = B*H*NQB (length of kv_num; kv_ptr has rows+1),
 * cols = B*H*NKB (length of q_num; q_ptr has cols+1), idx_capacity = B*H*NQB*NKB
 * (length to allocate for each of the four idx arrays), workspace_bytes = scratch
 * needed by fa_create_block_mask and by fa_block_mask_slice into these tables.  Reads
 * only the geometry fields; pure host call. */
fa_status fa_block_mask_sizes(const fa_block_mask* bm, int64_t* rows, int64_t* cols,
                              int64_t* idx_capacity, size_t* workspace_bytes);

/* Classify every block exactly and write the arrays of *bm on `stream`: all twelve,
 * or the six kv-side ones when the six q-side pointers are all NULL (a forward reads
 * only the kv side; FA_ERR_NULL when some q-side pointers are set and others not).
 * `workspace` is a device buffer of at least workspace_bytes (its contents on entry
 * are ignored and on exit unspecified).  Deterministic: the same inputs always give
 * the same tables bit for bit.  The table writers (this call, the selector and slice
 * calls below) accept every power-of-two block size from 1 to 128 -- the pages' worked
 * examples use 2 x 2 and 4 x 4 blocks ("FlexAttention: from rules to fused kernels",
 * sec. 2.2; "FlexAttention: compiler optimization of custom attention", sec. 4) --
 * while the attention kernels read tables of 64- or 128-blocks only.  B*H*NQB*NKB
 * must stay below 2^31 (FA_ERR_SHAPE otherwise): list positions are int32. */
fa_status fa_create_block_mask(fa_block_mask* bm, void* workspace, size_t ws_bytes,
                               fa_stream_t stream);

/* Block tables from selector output ("FlexAttention: from rules to fused kernels",
 * sec. 5.2: a dynamic selector emits candidate KV blocks per query block, which are
 * sorted and de-duplicated into each row's list; sec. 6.3: the candidates' range, order
 * and repeats must be checked; "Kernels: turning logical sparsity into real speed",
 * sec. 3: a repeated block would be counted twice in the softmax).
 *
 * `sel` is a device int32 array [B, H, NQB, k] (the table extents of *bm, k >= 0):
 * for each table row (b', h', r) the KV block indices chosen for query block r.  A
 * value outside [0, NKB) is dropped (padding such as -1), a repeated value counts once,
 * and the order within a row is free.  The allowed pairs are those of bm->mask's rule
 * inside the chosen blocks -- M(i, j) = R(i, j) and floor(j / block_kv) in S(b', h', r)
 * -- so with whole-block selection every pair the rule allows in a chosen block takes
 * part in the softmax (sec. 3.1 of the same page); a rule of PREFIX(P >= kv_len) allows
 * everything.  Each chosen block is classified exactly under the rule (EMPTY blocks are
 * left out), and the tables (and `order`, when set) are written as by
 * fa_create_block_mask; the six q-side arrays may all be NULL, and are then skipped
 * (the forward reads only the kv side; the backward needs both).  Selections may differ
 * per head (H = Hq).  `workspace` as for fa_block_mask_slice.  Nothing is allocated. */
fa_status fa_block_mask_from_indices(fa_block_mask* bm, const int32_t* sel, int32_t k, void* workspace,
                                     size_t ws_bytes, fa_stream_t stream);

/* Row slice of prebuilt tables ("FlexAttention: from rules to fused kernels", sec. 5.2:
 * build the tables once for the longest context, then for each decode step take the
 * query block that holds the current position, with the rule still seeing global
 * positions; sec. 2.2: a shorter square crop is the top-left corner of the longer one).
 *
 * `src` holds tables written by fa_create_block_mask, fa_block_mask_from_indices or
 * this call for its geometry; only its kv side is read (selector tables slice exactly
 * too: within a chosen block the allowed pairs are the rule's).  `dst` carries the new geometry -- q_len,
 * kv_len, q_offset -- with the mask rule, table extents and block sizes of src, and
 * caller-owned arrays sized by fa_block_mask_sizes(dst).  Requirements (else
 * FA_ERR_SHAPE / FA_ERR_MASK_MISMATCH):
 *   - the new rows [q_offset, q_offset + q_len) lie inside src's rows and
 *     kv_len <= src->kv_len: positions past the prebuilt length need new tables;
 *   - q_offset - src->q_offset is a multiple of block_q, or the new rows form one query
 *     block that lies inside one prebuilt query block (the decode case).
 * New block (k, c) holds a subset of the pairs of prebuilt block (k + (q_offset -
 * src->q_offset)/block_q, c), and every rule of the menu is a predicate on global
 * positions (none reads q_len or kv_len), so EMPTY and FULL blocks keep their class and
 * so does a PARTIAL block that covers the same pairs; a PARTIAL block whose rows or
 * keys were cut is classified again on the new geometry.  The written tables are
 * therefore exactly those fa_create_block_mask would write for dst, at the cost of
 * re-deciding only the blocks of a cut edge.
 * The q-side arrays of dst are written when all six are set, and skipped when all six
 * are NULL (fa_forward and fa_forward_paged read only the kv side).  `workspace` is a
 * 16-byte aligned device buffer of at least fa_block_mask_sizes(dst)'s workspace_bytes
 * (contents ignored on entry, unspecified on exit).  src, dst and workspace must not
 * overlap.  Nothing is allocated; one launch for up to 16384 new blocks and 4096 new
 * rows plus columns, five launches above. */
fa_status fa_block_mask_slice(const fa_block_mask* src, fa_block_mask* dst, void* workspace, size_t ws_bytes,
                              fa_stream_t stream);

/* ----------------------------------------------------------------------------------
 * Score modification, applied to the scaled score s = (q . k) * scale of every pair
 * in an executed block, before masking to -inf
 * ("FlexAttention: compiler optimization of custom attention", sec. 2):
 *   FA_S_IDENTITY  s
 *   FA_S_ALIBI     s + slope[h_q] * (j - i)          (slopes: device fp32 [Hq])
 *   FA_S_SOFTCAP   softcap * tanh(s / softcap)        (softcap > 0)
 *   FA_S_RELPOS    s + table[h_q][clip(i - j, -R, R) + R]   (device fp32 [Hq, 2R+1],
 *                                                           0 <= R <= 2^30 - 1)
 * ALiBi and the relative-position table are indexed by the QUERY head
 * ("FlexAttention: from rules to fused kernels", sec. 1.2); i and j are global positions.
 * -------------------------------------------------------------------------------- */
enum { FA_S_IDENTITY = 0, FA_S_ALIBI = 1, FA_S_SOFTCAP = 2, FA_S_RELPOS = 3 };

typedef struct {
  int32_t kind;
  float softcap;
  const float* alibi_slopes;
  const float* relpos;
  int32_t relpos_radius;
} fa_score_desc;

/* ----------------------------------------------------------------------------------
 * Forward.  q: bf16 [B, Hq, q_len, d]; k, v: bf16 [B, Hkv, kv_len, d]; o: bf16
 * [B, Hq, q_len, d]; lse: fp32 [B, Hq, q_len], natural-log log-sum-exp of the modified,
 * masked row.  GQA/MQA: Hq % Hkv == 0 and query head h reads KV head h / (Hq/Hkv)
 * ("FlexAttention: from rules to fused kernels", sec. 1.2).  d in {64, 128}, and the
 * tables' blocks 64 or 128 (FA_ERR_UNSUPPORTED otherwise).  scale <= 0 selects 1/sqrt(d).  Only the KV blocks listed in *bm are visited; the
 * mask rule is evaluated only on PARTIAL blocks (and on the ragged last block).
 * A row with no allowed key gets O = 0 and LSE = -inf.
 * bm must have been built for the same q_len, kv_len (and B/H extents compatible
 * with B and Hq); q_offset is taken from bm.  q, k, v and o must be 16-byte aligned and
 * lse 4-byte aligned (FA_ERR_SHAPE otherwise): rows move in 16-byte chunks.
 * Short queries (one query block, block_kv == 128, and (Hq/Hkv) * q_len <= 16 -- or
 * q_len <= 16 for tables with a row per query head under GQA, whose query heads then
 * each walk their own row) take a split-KV path that needs `workspace` of
 * fa_forward_workspace_size bytes, 16-byte aligned (FA_ERR_WORKSPACE otherwise); every
 * other shape needs none (workspace may then be NULL).
 * -------------------------------------------------------------------------------- */
typedef struct {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int32_t B, Hq, Hkv, d;
  int64_t q_len, kv_len;
  float scale;
  fa_score_desc score;
  const fa_block_mask* bm;
  void* workspace;
  size_t ws_bytes;
} fa_fwd_args;

fa_status fa_forward_workspace_size(const fa_fwd_args* args, size_t* bytes);
fa_status fa_forward(const fa_fwd_args* args, fa_stream_t stream);

/* ----------------------------------------------------------------------------------
 * fa_forward for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same forward,
 * with the same arguments, results and errors as fa_forward, except that
 * args->workspace and args->ws_bytes are ignored and the split-KV partial states of
 * the short-query path live in a static device array of the library,
 * FA_NOALLOC_SCRATCH_BYTES (16 MiB) per GPU, held from the first call on that GPU
 * until the process ends.  A shape whose fa_forward_workspace_size exceeds it returns
 * FA_ERR_WORKSPACE before anything is launched (the partial states take
 * B * Hq * q_len * splits * (d + 2) * 4 bytes; no short-query shape on a 256-CU GPU
 * needs more than about 12.2 MiB).  The call itself allocates nothing: no hipMalloc, hipFree or
 * allocating library routine.  Every kernel reads only the scratch entries the same
 * call wrote before, so nothing needs clearing between calls; but every call on one
 * GPU shares that GPU's array, so calls whose device work overlaps (on different
 * streams, or from different threads) race and must be serialised by the caller.
 * -------------------------------------------------------------------------------- */
#define FA_NOALLOC_SCRATCH_BYTES (16u << 20)
fa_status fa_forward_noalloc(const fa_fwd_args* args, fa_stream_t stream);

/* ----------------------------------------------------------------------------------
 * Backward ("FlexAttention: from rules to fused kernels", section 4: the scores of each
 * executed block are recomputed from the saved LSE, score_mod is differentiated, and
 * the block tables are walked per query row for dQ and per KV column -- the q-side
 * tables -- for dK and dV).
 *
 *   fwd        the arguments of the forward call whose gradients are wanted, with
 *              fwd->o and fwd->lse holding that call's results; fwd->bm must carry the
 *              q-side tables (fa_create_block_mask fills them).  The forward's
 *              workspace fields are ignored.
 *   dout       bf16 [B, Hq, q_len, d]: gradient of the loss with respect to O.
 *   dq         fp32 [B, Hq, q_len, d]; dk, dv fp32 [B, Hkv, kv_len, d]: written (not
 *              accumulated); GQA heads' contributions are summed into their KV head.
 *   workspace  device buffer, 256-byte aligned, contents on entry irrelevant: at least
 *              fa_backward_workspace_min_size bytes (two fp32 values per query row:
 *              -dO . O and the row's log-sum-exp term of the weights).  With the
 *              fa_backward_workspace_size bytes, which can be larger, the dK/dV pass also
 *              stores every executed block's per-pair gradients (bf16) and the dQ pass
 *              reads them instead of recomputing the scores: B * Hq * NQB * NKB
 *              tiles of 32 KiB, offered for d = 128, 128 x 128 blocks, no parameter
 *              gradient and at most 8 GiB (else both sizes are equal).  The
 *              gradients are the same bf16 values either way.
 *   dslopes    optional fp32 [Hq] (ALiBi only, else NULL): gradient of the slopes,
 *              sum over allowed pairs of dL/ds' (j - i), s' the modified score.
 *   dtable     optional fp32 [Hq, 2R+1] (relative-position bias only, R <= 1024, else
 *              NULL): gradient of the table, sum of dL/ds' over the pairs of each
 *              clipped offset.  Both are written (cleared first, then summed with
 *              floating-point atomic adds, so their last bits may vary run to run).
 * Rows with no allowed key contribute nothing.  Errors as for fa_forward, plus
 * FA_ERR_NULL for missing q-side tables, dout or gradient buffers, FA_ERR_SHAPE when
 * dout, dq, dk or dv is not 16-byte aligned, and FA_ERR_UNSUPPORTED for a parameter
 * gradient of another score kind.
 * -------------------------------------------------------------------------------- */
typedef struct {
  const fa_fwd_args* fwd;
  const void* dout;
  float* dq;
  float* dk;
  float* dv;
  void* workspace;
  size_t ws_bytes;
  float* dslopes;
  float* dtable;
} fa_bwd_args;

fa_status fa_backward_workspace_size(const fa_bwd_args* args, size_t* bytes);
fa_status fa_backward_workspace_min_size(const fa_bwd_args* args, size_t* bytes);
fa_status fa_backward(const fa_bwd_args* args, fa_stream_t stream);

/* ----------------------------------------------------------------------------------
 * Paged KV cache ("FlexAttention: from rules to fused kernels", sec. 5: a per-request
 * page table maps logical KV block j to a physical cache block; the attention rules,
 * score_mod positions and the BlockMask stay in logical positions, and the kernel
 * follows the table while it streams K/V instead of gathering a contiguous copy).
 *
 *   page_table  device int32 [B, pt_stride]: physical page of logical page p of
 *               request b is page_table[b * pt_stride + p]; logical page p holds the
 *               logical keys [p * page_size, (p + 1) * page_size).  Entries may repeat
 *               (requests sharing a prefix share pages).
 *   page_size   keys per page: a power of two, 16 <= page_size <= 65536.
 *   pt_stride   >= ceil(kv_len / page_size) (entries past that count are never read).
 *   num_pages   pages in each cache; every entry read must lie in [0, num_pages).  An
 *               entry outside that range is clamped into it (so every access stays
 *               inside the caches) and the rows that use it get unspecified values.
 *
 * fa_forward_paged takes the same arguments as fa_forward, except that args->k and
 * args->v are the paged caches, bf16 [num_pages, Hkv, page_size, d] each (one
 * contiguous page_size x d slab per page and KV head), and args->kv_len is the
 * logical KV length.  Only the short-query split-KV path is paged: the shape must
 * satisfy the conditions stated for it above, otherwise FA_ERR_UNSUPPORTED.  The workspace is the one
 * fa_forward_workspace_size reports for `args`.  Results equal fa_forward on the
 * logical (gathered) K and V bit for bit.
 * -------------------------------------------------------------------------------- */
typedef struct {
  const int32_t* page_table;
  int64_t pt_stride;
  int32_t page_size;
  int64_t num_pages;
} fa_paged_kv;

fa_status fa_forward_paged(const fa_fwd_args* args, const fa_paged_kv* kv, fa_stream_t stream);

const char* fa_status_string(fa_status s);
const char* fa_last_error_message(void);

#ifdef __cplusplus
}
#endif
#endif /* FA_H_ */
