/*
 * svt_oracle.h -- CPU oracle for the tree-verification step of tree speculative
 * decoding.  TEST INFRASTRUCTURE ONLY: this library exists so that the tests,
 * the smoke check and the CPU-baseline leg of the benchmark can check the GPU
 * library against plain definitions.  Nothing in the product path may link,
 * load or call it.
 *
 * It shares no code, header, table or constant with the GPU library.  The
 * status numbers below are written out again here on purpose: both sides
 * follow the same documented code table, and a test compares the numbers.
 *
 * Every function works on host memory, in the plainest form of the
 * definition it implements; floating-point work is done in double precision.
 *
 * Sources (the pages are summaries of two papers):
 *   [EP-ko] "EAGLE-Pangu: Accelerator-Safe Tree Speculative Decoding on Ascend
 *           NPUs", gist.science Korean summary page.
 *   [EP-nl] the same paper, gist.science Dutch summary page.
 *   [BSD]   "Batch Speculative Decoding Done Right", gist.science Korean
 *           summary page.
 */
#ifndef SVT_ORACLE_H
#define SVT_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_ARG (-1)
#define ORACLE_ERR_TREE_ROOT (-3)
#define ORACLE_ERR_TREE_RANGE (-4)
#define ORACLE_ERR_TREE_CYCLE (-5)
#define ORACLE_ERR_CAPACITY (-6)
#define ORACLE_ERR_LENGTH (-9)

/* Tree validation ([EP-ko] §2 Methodology, accelerator-safe tree tensorization;
 * [EP-nl] §2.B dummy-root indexing and invariant checks).
 * parents: [B][M+1].  status: [B] out.  Returns the first nonzero status, or 0. */
int oracle_validate(const int32_t* parents, int32_t B, int32_t M, int32_t* status);

/* Ancestor mask and depth ([EP-ko] §2, fused tree-masked teacher: u attends v
 * only when v is an ancestor of u; reflexive reading).  mask: [B][T][W] with
 * W = ceil(T/64); depth: [B][T].  Sequences whose status is nonzero get all
 * zeros.  status may be NULL (then every tree must be valid). */
void oracle_mask(const int32_t* parents, int32_t B, int32_t M, const int32_t* status,
                 uint64_t* mask, int32_t* depth);

/* Dense 4D tree mask for eager attention ([EP-nl] §2.C: token k may attend
 * token j only when j is an ancestor of k; reference mode with the fused
 * attention off; [EP-ko] §2 4D tree attention mask).  Computed from the
 * parent arrays by walking each node's chain (reflexive reading).
 *   open [B][T][lmax + T] out: 1 where row i of sequence b may attend the
 *   column, else 0.  Columns c < lmax are the left-padded prefix (content
 *   from lmax - len_b), columns lmax + j the tree nodes.  A sequence with a
 *   nonzero status or len_b outside [0, lmax] gets all zeros; code [B] out
 *   receives 0, its status, or ORACLE_ERR_LENGTH.  status may be NULL. */
void oracle_expand_mask(const int32_t* parents, const int32_t* len, const int32_t* status, int32_t B,
                        int32_t M, int32_t lmax, uint8_t* open, int32_t* code);

/* Tree-verify attention ([EP-ko] §2 fused tree-masked teacher execution;
 * [EP-nl] §2.C).  All tensors are float (exact upcasts of what the GPU reads);
 * the result is double.
 *   q      [B][T][Hq][D]
 *   k_cache, v_cache [B][Hkv][cap][D]   content of b in columns [lmax-len_b, lmax)
 *   k_tree, v_tree   [B][Hkv][T][D]
 *   mask   [B][T][W]
 *   out    [B][T][Hq][D] (double)
 * Sequences with nonzero status, or with inconsistent lengths, get zeros.
 * Returns 0, or ORACLE_ERR_LENGTH when some sequence had inconsistent lengths. */
int oracle_attention(const float* q, const float* k_cache, const float* v_cache,
                     const float* k_tree, const float* v_tree, const uint64_t* mask,
                     const int32_t* len, int32_t lmax, int64_t cap, const int32_t* status,
                     int32_t B, int32_t M, int32_t Hq, int32_t Hkv, int32_t D, double scale,
                     double* out);

/* Attention for a single (b, head, node) triple, same definition as above; used
 * for sampled checks of large instances. out: [D]. */
void oracle_attention_row(const float* q_row, const float* k_cache_bh, const float* v_cache_bh,
                          const float* k_tree_bh, const float* v_tree_bh, const uint64_t* mask_row,
                          int32_t len_b, int32_t lmax, int32_t T, int32_t D, double scale,
                          double* out);

/* Greedy argmax per row, lowest index on ties, first NaN wins. */
void oracle_argmax(const float* logits, int64_t rows, int32_t V, int32_t* amax);

/* Greedy acceptance of the longest root path ([EP-ko] §4 Results, accepted
 * length accept_L; greedy teacher rule).  Works from the parent array alone.
 *   amax [B][T] in (from oracle_argmax), tree_tokens [B][T], parents [B][T]
 *   accept_len [B], path [B][T], bonus [B] out. */
void oracle_accept(const int32_t* amax, const int32_t* tree_tokens, const int32_t* parents,
                   const int32_t* status, int32_t B, int32_t M,
                   int32_t* accept_len, int32_t* path, int32_t* bonus);

/* KV commit ([BSD] §2 Methodology: rectangular alignment, position-id
 * contiguity, unpad-append-repad (EQSPEC); equal-length batches of
 * cross-batch scheduling need no realignment (EXSPEC); [EP-ko] §2 fast reorder
 * by path_indices; [EP-nl] §2.A commit modes).
 *   kv_main   [L][2][rows][Hkv][cap][row_bytes]  in/out (raw bytes)
 *   kv_branch [L][2][B][Hkv][T][row_bytes]
 *   tokens_main [rows][cap] in/out (nullable), tree_tokens [B][T]
 *   len [B], lmax [1] in/out, pos_ids [rows][cap] out (nullable)
 *   slot [B] or NULL: sequence b is row slot[b] of kv_main, tokens_main and
 *   pos_ids (rows = B when NULL)
 *   mode 0 = re-pad (EQSPEC), 1 = append without moving (EXSPEC)
 *   path NULL: length-based commit ([EP-nl] §2.A): step k of the chosen
 *   branch is branch row k, so rows [0, A_b) are appended
 * Returns 0, or on error (nothing changes) ORACLE_ERR_LENGTH for inconsistent
 * lengths, ORACLE_ERR_ARG for an accept length or path entry outside [0, M]
 * or a slot outside [0, rows), ORACLE_ERR_CAPACITY when a sequence would end
 * past cap (checked in that order). */
int oracle_commit(uint8_t* kv_main, const uint8_t* kv_branch, int32_t n_layers, int32_t B,
                  int32_t Hkv, int64_t cap, int32_t row_bytes, int32_t M,
                  int32_t* tokens_main, const int32_t* tree_tokens, int32_t* len, int32_t* lmax,
                  int32_t* pos_ids, const int32_t* path, const int32_t* accept_len,
                  const int32_t* status, int32_t mode, const int32_t* slot, int32_t rows);

/* Realignment of a batch whose sequences end at different columns to the
 * largest end ([BSD] §2: the EXSPEC fallback uses EQSPEC's alignment when a
 * batch mixes lengths).  Sequence b's content [end_b - len_b, end_b) is
 * rewritten at [E - len_b, E), E = max_b end_b, in every slab of kv_main and
 * in tokens_main; pos_ids for c < E.  *lmax = E.  Returns 0, or (nothing
 * changes) ORACLE_ERR_LENGTH when some len_b < 0, end_b < len_b or
 * end_b > cap, else ORACLE_ERR_ARG for a slot outside [0, rows). */
int oracle_realign(uint8_t* kv_main, int32_t n_layers, int32_t B, int32_t Hkv, int64_t cap,
                   int32_t row_bytes, int32_t* tokens_main, int32_t* pos_ids, const int32_t* slot,
                   int32_t rows, const int32_t* len, const int32_t* end, int32_t* lmax);

#ifdef __cplusplus
}
#endif
#endif
