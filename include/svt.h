/*
 * svt.h -- tree-masked speculative verification on AMD Instinct MI355X (gfx950).
 *
 * One verification round of tree speculative decoding, batched over ragged
 * sequences, as four calls:
 *
 *   svt_build_mask        validate parent arrays, build ancestor bitmasks + depth
 *   svt_verify_attention  attention of every tree node over prefix KV + tree KV
 *   svt_accept            greedy argmax per node, longest accepted root path
 *   svt_commit            append the accepted rows to the main cache, re-pad
 *
 * plus svt_realign (bring a batch drawn from a sequence pool to a common end
 * column) and svt_pool_pick (host: choose the next batch from a pool) for
 * cross-batch scheduling, svt_expand_mask (dense 4D mask for eager attention
 * paths) and svt_commit_length (length-based commit).
 *
 * Sources (summary pages of two papers):
 *   [EP-ko] "EAGLE-Pangu: Accelerator-Safe Tree Speculative Decoding on Ascend
 *           NPUs", gist.science Korean summary.
 *   [EP-nl] the same paper, gist.science Dutch summary.
 *   [BSD]   "Batch Speculative Decoding Done Right", gist.science Korean summary.
 *
 * Conventions shared by every call
 *   - Pointers are device memory owned by the caller unless the name ends in
 *     _host.  The library keeps no state between calls.  Calls that need
 *     scratch memory take a caller-provided workspace whose size a *_workspace
 *     query returns; the library itself allocates nothing.  The one exception,
 *     svt_accept_noalloc, uses a fixed static device buffer instead.
 *   - Every call enqueues its kernels on the caller's stream and returns at once,
 *     except where SVT_SYNC_CHECK is given (then it synchronises that stream).
 *   - The return value is SVT_OK or a negative svt_status.  Argument errors are
 *     found on the host before anything is launched and leave every buffer
 *     untouched.  Tree errors are found on the device and reported per sequence
 *     through a status array.
 *   - Index arrays never hold negative values: the tree root is a dummy row 0
 *     that points at itself, and padding entries of index outputs are 0
 *     ([EP-ko] section 2, accelerator-safe tree tensorization; [EP-nl] 2.B).
 *   - T = M + 1 rows per tree (row 0 = root, rows 1..M = draft nodes), at most
 *     SVT_MAX_T.  W = ceil(T / 64) mask words per row.  G = Hq / Hkv.
 *   - bf16 tensors hold raw bfloat16 bits; fp32 tensors hold IEEE binary32.
 */
#ifndef SVT_H
#define SVT_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SVT_MAX_T 256 /* M <= 255, W <= 4 */

typedef enum svt_status {
  SVT_OK = 0,
  SVT_ERR_ARG = -1,          /* bad pointer, size or layout (host check)              */
  SVT_ERR_UNSUPPORTED = -2,  /* valid but not implemented: head dim, dtype, T          */
  SVT_ERR_TREE_ROOT = -3,    /* parents[b][0] != 0                                     */
  SVT_ERR_TREE_RANGE = -4,   /* some parents[b][i], i >= 1, outside [0, M] or == i     */
  SVT_ERR_TREE_CYCLE = -5,   /* some node's parent chain never reaches row 0           */
  SVT_ERR_CAPACITY = -6,     /* commit would need more than cap cache columns          */
  SVT_ERR_WORKSPACE = -7,    /* workspace pointer missing, too small or misaligned     */
  SVT_ERR_HIP = -8,          /* a HIP runtime call failed                               */
  SVT_ERR_LENGTH = -9        /* device lengths inconsistent (len > lmax, lmax > bound)  */
} svt_status;

typedef enum svt_dtype { SVT_FP32 = 0, SVT_BF16 = 1 } svt_dtype;

/* Flag: after enqueueing, synchronise the stream and return the first nonzero
 * device status the call produced (tree status for svt_build_mask, commit status
 * for svt_commit). */
#define SVT_SYNC_CHECK 1

/* ------------------------------------------------------------------------ */
/* svt_build_mask                                                            */
/* Validates each tree and builds its ancestor mask.                         */
/*   Validation ([EP-ko] section 2, tree tensorization with structural       */
/*   checks before kernels run; [EP-nl] 2.B invariant checks): status[b] =   */
/*   SVT_ERR_TREE_ROOT if parents[b][0] != 0, else SVT_ERR_TREE_RANGE if some */
/*   i >= 1 has parents[b][i] outside [0, M] or equal to i, else              */
/*   SVT_ERR_TREE_CYCLE if some chain never reaches row 0, else SVT_OK.       */
/*   Mask ([EP-ko] section 2, fused tree-masked teacher; [EP-nl] 2.C): node u */
/*   may attend v only if v is u itself or an ancestor of u.  Bit (j % 64) of */
/*   mask[b][i][j / 64] is 1 iff j is i or an ancestor of i (root included);  */
/*   unused high bits are 0.  depth[b][i] = number of edges from i to row 0.  */
/*   Invalid trees get all-zero mask and depth rows.                          */
/* Arguments                                                                  */
/*   parents [B][T] int32 in; mask [B][T][W] uint64 out; depth [B][T] int32   */
/*   out; status [B] int32 out.  B >= 0, 0 <= M < SVT_MAX_T.                  */
/* Returns SVT_OK, SVT_ERR_ARG / SVT_ERR_UNSUPPORTED (host), SVT_ERR_HIP, or  */
/* with SVT_SYNC_CHECK the first nonzero status[b].                           */
/* ------------------------------------------------------------------------ */
int svt_build_mask(const int32_t* parents, int32_t B, int32_t M, uint64_t* mask, int32_t* depth,
                   int32_t* status, int32_t flags, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* svt_expand_mask                                                           */
/* Dense 4D tree mask for eager attention paths ([EP-nl] section 2.C: a 4D    */
/* mask lets token k attend token j only when j is an ancestor of k; the      */
/* reference mode runs with the fused attention switched off; [EP-ko]         */
/* section 2: 4D tree attention mask, eager and performance modes).           */
/*   out[b][0][i][c], c < lmax + T: prefix column c < lmax is open when it     */
/*   holds content (c >= lmax - len[b], left padding); tree column lmax + j    */
/*   is open when bit j of mask[b][i] is set (j is i or an ancestor of i).     */
/*   Open = 0 and closed = -inf for the additive kinds (fp32, or bf16 bits);   */
/*   open = 1 and closed = 0 for SVT_MASK_BOOL (uint8).  The key order is the  */
/*   one of svt_verify_attention: lmax cache columns, then the T tree rows.    */
/*   A sequence with a nonzero status[b] or len[b] outside [0, lmax] gets      */
/*   every column closed; seq_status[b] (if given) receives SVT_OK, the tree   */
/*   status or SVT_ERR_LENGTH.                                                 */
/* Arguments: mask [B][T][W] from svt_build_mask; status [B] or NULL; len [B] */
/* device; lmax host (prefix columns, >= 0); out [B][1][T][lmax + T] of the   */
/* kind's element (4, 2 or 1 bytes), 16-byte aligned.  Returns SVT_OK,        */
/* SVT_ERR_ARG / SVT_ERR_UNSUPPORTED (host) or SVT_ERR_HIP.                   */
/* ------------------------------------------------------------------------ */
typedef enum svt_mask_kind { SVT_MASK_ADD_FP32 = 0, SVT_MASK_ADD_BF16 = 1, SVT_MASK_BOOL = 2 } svt_mask_kind;

int svt_expand_mask(const uint64_t* mask, const int32_t* status, const int32_t* len, int32_t B, int32_t M,
                    int32_t lmax, void* out, int32_t kind, int32_t* seq_status, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* svt_verify_attention                                                      */
/* One batched attention pass over all tree nodes ([EP-ko] section 2, fused  */
/* tree-masked teacher execution; [EP-nl] 2.C).  For sequence b, query head  */
/* h (KV head g = h / G) and node i:                                          */
/*   keys = prefix cache columns [lmax - len[b], lmax) of k_cache[b][g]       */
/*          plus tree rows j of k_tree[b][g] with mask bit j of row i set     */
/*   out[b][i][h] = softmax(scale * q[b][i][h] . key) weighted sum of values  */
/* The prefix is left padded: every sequence's content ends at column lmax    */
/* ([BSD] section 2, rectangular alignment).  Columns outside the content are */
/* never read.  With seq_slot set, sequence b's cache rows are                 */
/* k_cache[seq_slot[b]] and v_cache[seq_slot[b]] of a pool of n_slots rows     */
/* (q, tree KV, mask and out stay indexed by b); a slot outside [0, n_slots)  */
/* gives that sequence SVT_ERR_ARG in seq_status and zero output.           */
/* Accumulation and softmax are fp32; bf16 inputs use bf16 MFMA for both     */
/* contractions (probabilities are rounded to bf16 for the second).  The     */
/* result is bitwise deterministic run to run.                               */
/* Non-finite inputs: cache columns outside the content are never read and   */
/* may hold anything.  A key that a node does not attend never reaches that  */
/* node's output, whatever its K values.  V of the tree rows must be finite: */
/* masked keys enter the P V product with probability exactly 0, and 0 times */
/* Inf or NaN is NaN (as in a dense masked attention), so a non-finite V in  */
/* tree row j can make other rows of the same sequence and KV head non-     */
/* finite; other sequences and KV heads are never affected.                  */
/* ------------------------------------------------------------------------ */
typedef struct svt_attn_args {
  int32_t B, M, Hq, Hkv, D;  /* D in {64, 128}; Hq % Hkv == 0                        */
  int32_t dtype;             /* svt_dtype of q, caches, tree KV and out               */
  float scale;               /* softmax scale; 0 selects 1 / sqrt(D)                  */
  const void* q;             /* [B][T][Hq][D]                                         */
  const void* k_cache;       /* [B][Hkv][cap][D], one layer                           */
  const void* v_cache;       /* [B][Hkv][cap][D]                                      */
  int64_t cap;               /* cache columns                                         */
  const int32_t* len;        /* [B] device: content length per sequence              */
  const int32_t* lmax;       /* [1] device: batch length; content ends here           */
  int32_t lmax_bound;        /* host upper bound on *lmax, sizes the grid; <= cap     */
  const void* k_tree;        /* [B][Hkv][T][D] the tree's own (branch) keys           */
  const void* v_tree;        /* [B][Hkv][T][D]                                        */
  const uint64_t* mask;      /* [B][T][W] from svt_build_mask                         */
  const int32_t* status;     /* [B] from svt_build_mask, or NULL (all valid)          */
  void* out;                 /* [B][T][Hq][D], dtype of q                             */
  int32_t* seq_status;       /* [B] out, or NULL: SVT_OK, the tree status, or         */
                             /* SVT_ERR_LENGTH if 0 <= len[b] <= lmax <= lmax_bound   */
                             /* fails.  Such sequences get all-zero output.           */
  void* workspace;           /* device scratch, svt_verify_attention_workspace bytes, */
                             /* 16-byte aligned (else SVT_ERR_WORKSPACE)               */
  size_t workspace_bytes;
  int32_t form;              /* svt_attn_form: which work decomposition (bf16 only)   */
  const int32_t* seq_slot;   /* [B] cache row of each sequence, or NULL (row b)        */
  int32_t n_slots;           /* rows of k_cache / v_cache when seq_slot is set         */
  int32_t split_keys;        /* 0, or content keys per split (a positive multiple of  */
                             /* 64): selects the split form with that split size, so */
                             /* a sequence's result depends on its own inputs only   */
                             /* (else SVT_ERR_ARG; with SVT_ATTN_STREAM too)          */
} svt_attn_args;

/* Work decomposition of svt_verify_attention (bf16; fp32 always splits).
 * Both compute the same function; results agree to rounding, and each is
 * bitwise reproducible for identical inputs.
 *   SVT_ATTN_AUTO    choose by shape
 *   SVT_ATTN_SPLIT   key splits per (sequence, KV head), counted from the
 *                    start of the sequence's content; their size comes from
 *                    the shape (B, lmax_bound), or is fixed by split_keys,
 *                    and then a sequence's result is bitwise the same in any
 *                    batch ([BSD] section 4: batching must not change a
 *                    sequence's output)
 *   SVT_ATTN_STREAM  the key tiles of the whole batch cut into one range of
 *                    equal cost per compute unit (needs bf16 and B <= 1024,
 *                    else SVT_ERR_UNSUPPORTED) */
typedef enum svt_attn_form { SVT_ATTN_AUTO = 0, SVT_ATTN_SPLIT = 1, SVT_ATTN_STREAM = 2 } svt_attn_form;

/* Bytes of workspace svt_verify_attention needs for these shapes (pointer
 * fields are ignored).  0 for invalid arguments. */
size_t svt_verify_attention_workspace(const svt_attn_args* a);
int svt_verify_attention(const svt_attn_args* a, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* svt_accept                                                                */
/* Greedy verification ([EP-ko] section 4: accepted length accept_L under    */
/* the teacher's greedy choice).                                              */
/*   amax[b][i]   = index of the largest logits[b][i][v]; lowest index on     */
/*                  ties; a NaN ranks above every number (first NaN wins);    */
/*                  -0.0 equals +0.0.                                         */
/*   ok(i)        = i == 0, or tree_tokens[b][i] == amax[b][parents[b][i]]    */
/*   accepted(i)  = ok holds on every node of i's root path (mask row i)      */
/*   end          = accepted node of greatest depth, lowest index on ties     */
/*   accept_len[b]= depth[b][end] (accepted draft tokens, root excluded)      */
/*   path[b][k]   = ancestor of end at depth k for k <= accept_len, else 0    */
/*   bonus[b]     = amax[b][end]                                              */
/* Sequences with status[b] != 0 accept nothing: accept_len 0, path 0,        */
/* bonus = amax[b][0].                                                        */
/* ------------------------------------------------------------------------ */
typedef struct svt_accept_args {
  int32_t B, M, V;
  const float* logits;         /* [B][T][V] fp32                                    */
  const int32_t* tree_tokens;  /* [B][T] draft token of each node (root: any)        */
  const int32_t* parents;      /* [B][T]                                             */
  const uint64_t* mask;        /* [B][T][W] from svt_build_mask                      */
  const int32_t* depth;        /* [B][T] from svt_build_mask                         */
  const int32_t* status;       /* [B] or NULL                                        */
  int32_t* amax;               /* [B][T] out                                         */
  int32_t* accept_len;         /* [B] out                                            */
  int32_t* path;               /* [B][T] out (the path_indices of the commit)        */
  int32_t* bonus;              /* [B] out                                            */
  void* workspace;             /* device scratch, svt_accept_workspace bytes,        */
                               /* 8-byte aligned (else SVT_ERR_WORKSPACE)            */
  size_t workspace_bytes;
} svt_accept_args;

/* Bytes of workspace svt_accept needs for these shapes.  A smaller batch may
 * need more (its rows are cut into more chunks to fill the chip): query it
 * for the batch size being run, or for the largest need over the sizes used. */
size_t svt_accept_workspace(const svt_accept_args* a);
int svt_accept(const svt_accept_args* a, hipStream_t stream);

/* svt_accept_noalloc: svt_accept for callers that cannot allocate device     */
/* memory (code under HIP graph capture, tight serving loops, harnesses that  */
/* forbid hipMalloc).  Same arguments, outputs and errors as svt_accept,      */
/* except that a->workspace and a->workspace_bytes are ignored: the chunk     */
/* keys go to a static device buffer of SVT_ACCEPT_NOALLOC_SCRATCH bytes that  */
/* the library holds on each GPU it runs on until the process ends.  A shape  */
/* whose svt_accept_workspace exceeds that returns SVT_ERR_WORKSPACE before    */
/* anything is launched.  The call allocates nothing and calls no allocating  */
/* routine.  Every call on one GPU shares that GPU's buffer (it keeps the last */
/* call's contents, none of which a later call reads): calls that overlap on  */
/* one GPU (different streams, or different threads on one stream without     */
/* ordering) race and must not be issued.                                      */
#define SVT_ACCEPT_NOALLOC_SCRATCH (4u << 20)
int svt_accept_noalloc(const svt_accept_args* a, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* svt_commit                                                                */
/* Unpad-append-repad of the main cache after a round ([BSD] section 2:       */
/* rectangular alignment and position ids contiguous from 0; [EP-ko]          */
/* section 2: accepted rows gathered from the branch cache by path index,     */
/* only the new segment reordered; [EP-nl] 2.A commit modes).                 */
/*   A_b   = accept_len[b] + 1 (root + accepted drafts), or 0 when status[b]  */
/*           is nonzero                                                       */
/*   len'  = len + A,  lmax' = max_b len'_b,  pad'_b = lmax' - len'_b         */
/*   Sequence b's old content [lmax - len_b, lmax) moves to                   */
/*   [pad'_b, pad'_b + len_b); rows path[b][0..A_b) of kv_branch follow at    */
/*   [pad'_b + len_b, lmax').  Same for every layer, K and V plane and KV     */
/*   head, and for tokens_main (with tree_tokens[b][path[b][k]]).             */
/*   pos_ids[b][c] = c - pad'_b on content, 0 on padding, for c < lmax'.      */
/*   Columns >= lmax' are not written; padding contents are unspecified.      */
/* mode SVT_COMMIT_APPEND is the no-realignment path of cross-batch          */
/* scheduling ([BSD] section 2, EXSPEC: a batch of equal-length sequences    */
/* needs no realignment): nothing moves; rows path[b][0..A_b) go to          */
/* [lmax, lmax + A_b) after the unchanged content [lmax - len_b, lmax);      */
/* len' = len + A, lmax' = lmax + max_b A_b, and sequence b's content now     */
/* ends at lmax + A_b (the batch stays rectangular only where A_b = max A).  */
/* pos_ids[b][c] = c - (lmax - len_b) on content, 0 on padding, for           */
/* c < lmax + A_b.  SVT_ERR_CAPACITY when lmax + A_b > cap for some b.        */
/* With len_out and lmax_out set, len and lmax are only read, so the same     */
/* commit can be issued in parts (say one layer at a time, kv_main and        */
/* kv_branch pointing at that layer, n_layers = 1, with tokens_main and        */
/* pos_ids given to one of the calls): every call derives the same plan and   */
/* writes the same len_out, lmax_out and commit_status.                       */
/* With seq_slot set, sequence b lives in row seq_slot[b] of kv_main,         */
/* tokens_main and pos_ids (pools of n_slots rows; kv_branch, tree_tokens,    */
/* len, path, accept_len stay indexed by b).  A slot outside [0, n_slots) or  */
/* named by two sequences is SVT_ERR_ARG (checked with the accept arguments). */
/* Rows are moved as raw bytes (any bit pattern survives).  Device-side     */
/* errors are checked over the whole batch in this order, the first one found */
/* goes to commit_status and then nothing is written:                         */
/*   SVT_ERR_LENGTH    lmax < 0, lmax > cap, or some len[b] outside [0, lmax] */
/*   SVT_ERR_ARG       for a sequence with status 0: accept_len[b] or one of  */
/*                     path[b][0..accept_len[b]] outside [0, M]               */
/*   SVT_ERR_CAPACITY  lmax' > cap                                            */
/* Otherwise len and lmax are updated in place.                              */
/* ------------------------------------------------------------------------ */
typedef struct svt_commit_args {
  int32_t B, M, Hkv, D, n_layers;
  int32_t dtype;               /* svt_dtype (element size of cache rows)            */
  int64_t cap;
  void* kv_main;               /* [n_layers][2][B][Hkv][cap][D] in/out              */
  const void* kv_branch;       /* [n_layers][2][B][Hkv][T][D]                        */
  int32_t* tokens_main;        /* [B][cap] in/out, or NULL                           */
  const int32_t* tree_tokens;  /* [B][T] (needed when tokens_main is set)            */
  int32_t* len;                /* [B] in/out                                         */
  int32_t* lmax;               /* [1] in/out                                         */
  int32_t* pos_ids;            /* [B][cap] out, or NULL                              */
  const int32_t* path;         /* [B][T] from svt_accept                             */
  const int32_t* accept_len;   /* [B] from svt_accept                                */
  const int32_t* status;       /* [B] or NULL                                        */
  int32_t* commit_status;      /* [1] out: SVT_OK or one of the errors above        */
  const int32_t* seq_slot;     /* [B] pool row of each sequence, or NULL (row b)     */
  int32_t n_slots;             /* pool rows when seq_slot is set                     */
  int32_t mode;                /* svt_commit_mode                                    */
  int32_t* len_out;            /* [B] new lengths, or NULL: len is updated in place   */
  int32_t* lmax_out;           /* [1] new lmax, or NULL: lmax is updated in place     */
} svt_commit_args;

typedef enum svt_commit_mode { SVT_COMMIT_REPAD = 0, SVT_COMMIT_APPEND = 1 } svt_commit_mode;

int svt_commit(const svt_commit_args* a, int32_t flags, hipStream_t stream);

/* svt_commit_length: the length-based commit of [EP-nl] section 2.A (keep the */
/* prefix, append the first A steps of the chosen branch).  kv_branch and      */
/* tree_tokens hold each sequence's chosen branch in step order (row k = step  */
/* k, row 0 the root); rows [0, A_b) are committed, A_b = accept_len[b] + 1.   */
/* Everything else, modes and errors included, is svt_commit with path[b][k]   */
/* = k; a->path is ignored (may be NULL).                                      */
int svt_commit_length(const svt_commit_args* a, int32_t flags, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* svt_realign                                                               */
/* Brings a batch whose sequences end at different columns to a common end   */
/* ([BSD] section 2: EXSPEC falls back to EQSPEC's alignment when a batch     */
/* mixes lengths; rectangular alignment).  Sequence b's content               */
/* [end[b] - len[b], end[b]) moves to [E - len[b], E) with E = max_b end[b],  */
/* in every layer, K and V plane and KV head, and in tokens_main; nothing     */
/* else changes.  pos_ids[b][c] = c - (E - len[b]) on content, 0 on padding,  */
/* for c < E.  *lmax = E afterwards (0 for B = 0).  Errors, found on the      */
/* device before anything is written (then nothing is): SVT_ERR_LENGTH when   */
/* some len[b] < 0, end[b] < len[b] or end[b] > cap, else SVT_ERR_ARG for a   */
/* slot outside [0, n_slots) or named by two sequences.  Rows move as raw     */
/* bytes.                                                                     */
/* ------------------------------------------------------------------------ */
typedef struct svt_realign_args {
  int32_t B, Hkv, D, n_layers;
  int32_t dtype;               /* svt_dtype (element size of cache rows)            */
  int64_t cap;
  void* kv_main;               /* [n_layers][2][rows][Hkv][cap][D] in/out           */
  int32_t* tokens_main;        /* [rows][cap] in/out, or NULL                        */
  int32_t* pos_ids;            /* [rows][cap] out, or NULL                           */
  const int32_t* seq_slot;     /* [B] pool row of each sequence, or NULL (rows = B)  */
  int32_t n_slots;             /* pool rows when seq_slot is set                     */
  const int32_t* len;          /* [B] content length                                 */
  const int32_t* end;          /* [B] column just past each sequence's content       */
  int32_t* lmax;               /* [1] out: the common end E                          */
  int32_t* realign_status;     /* [1] out: SVT_OK or one of the errors above         */
} svt_realign_args;

int svt_realign(const svt_realign_args* a, int32_t flags, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* svt_pool_pick (host)                                                       */
/* Chooses the next batch of cross-batch scheduling ([BSD] section 2, EXSPEC: */
/* a SequencePool; sequences whose lengths match are grouped so their batch   */
/* needs no realignment; otherwise EQSPEC's alignment is the fallback).       */
/* Pool sequences with active_host[s] != 0 are grouped by end column          */
/* end_host[s] (for sequences stored without padding this is their length).   */
/* If the largest group (ties: smallest end) holds at least                   */
/* min(max_batch, min_group) sequences, the batch is up to max_batch of them, */
/* lowest slots first.  Otherwise the batch is that group filled up to        */
/* max_batch with the active sequences whose end is nearest to the group's    */
/* (ties: smaller end, then lower slot).  slots_host receives the chosen      */
/* slots in increasing order and *n_host their count (0 when no sequence is   */
/* active).  Returns 1 when every chosen slot has the same end (commit with   */
/* SVT_COMMIT_APPEND, no realignment; also for an empty pick), 0 when the     */
/* ends differ (svt_realign first, then a SVT_COMMIT_REPAD commit), or        */
/* SVT_ERR_ARG for n_slots < 0, max_batch < 1, min_group < 1 or a NULL        */
/* pointer.  Pure host code; no device work.                                  */
/* ------------------------------------------------------------------------ */
int svt_pool_pick(const int32_t* end_host, const int32_t* active_host, int32_t n_slots, int32_t max_batch,
                  int32_t min_group, int32_t* slots_host, int32_t* n_host);

/* ------------------------------------------------------------------------ */
/* Utilities                                                                  */
/* ------------------------------------------------------------------------ */
/* Synchronises the stream, copies n int32 statuses to the host and returns the
 * first nonzero one (SVT_OK if none, SVT_ERR_HIP on a runtime failure). */
int svt_check_status(const int32_t* status, int32_t n, hipStream_t stream);
const char* svt_status_string(int code);
/* Library version, e.g. "0.1.0 gfx950". */
const char* svt_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SVT_H */
