/*
 * svt_oracle.c -- plain CPU oracle for tree-masked verification.
 *
 * TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU-baseline leg of the
 * benchmark).  It is deliberately slow and literal: every function computes
 * the definition it cites, node by node and element by element, with no
 * blocking, fusion or reordering.  Floating point is double precision.
 *
 * Source tags used below:
 *   [EP-ko] "EAGLE-Pangu: Accelerator-Safe Tree Speculative Decoding on Ascend
 *           NPUs", gist.science Korean summary.
 *   [EP-nl] same paper, gist.science Dutch summary.
 *   [BSD]   "Batch Speculative Decoding Done Right", gist.science Korean summary.
 */
#include "svt_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Tree validation.                                                          */
/* [EP-ko] §2 Methodology (accelerator-safe tree tensorization) and [EP-nl]  */
/* §2.B: a dummy row at index 0 stands for the root, so every parent index   */
/* lies in [0, M]; structural invariants (range, acyclicity) are checked     */
/* before any kernel runs.  Reading: row 0 is the root and points at itself; */
/* a node i >= 1 may not be its own parent; every chain must reach row 0.    */
/* The code reported for a tree is the first failing check in the order      */
/* ROOT, RANGE, CYCLE.                                                       */
/* ------------------------------------------------------------------------ */
static int validate_one(const int32_t* par, int32_t M) {
  int32_t T = M + 1;
  if (par[0] != 0) return ORACLE_ERR_TREE_ROOT;
  for (int32_t i = 1; i < T; ++i) {
    if (par[i] < 0 || par[i] > M || par[i] == i) return ORACLE_ERR_TREE_RANGE;
  }
  for (int32_t i = 1; i < T; ++i) {
    /* A chain without a cycle visits at most M distinct non-root nodes. */
    int32_t u = i, steps = 0;
    while (u != 0 && steps <= M) {
      u = par[u];
      ++steps;
    }
    if (u != 0) return ORACLE_ERR_TREE_CYCLE;
  }
  return ORACLE_OK;
}

int oracle_validate(const int32_t* parents, int32_t B, int32_t M, int32_t* status) {
  int first = ORACLE_OK;
  for (int32_t b = 0; b < B; ++b) {
    int s = validate_one(parents + (int64_t)b * (M + 1), M);
    status[b] = s;
    if (s != ORACLE_OK && first == ORACLE_OK) first = s;
  }
  return first;
}

/* ------------------------------------------------------------------------ */
/* Ancestor mask and depth.                                                  */
/* [EP-ko] §2 (fused tree-masked teacher): node u may attend node v only if  */
/* v is an ancestor of u; [EP-nl] §2.C states the same rule for the 4D mask. */
/* Reading: the relation is reflexive (u also sees itself) and the root row  */
/* 0 is an ancestor of every node.  Bit j of word j/64 of row i is set iff   */
/* j lies on the walk i -> parent(i) -> ... -> 0.  depth[i] = edges walked.  */
/* ------------------------------------------------------------------------ */
void oracle_mask(const int32_t* parents, int32_t B, int32_t M, const int32_t* status,
                 uint64_t* mask, int32_t* depth) {
  int32_t T = M + 1, W = (T + 63) / 64;
  for (int32_t b = 0; b < B; ++b) {
    const int32_t* par = parents + (int64_t)b * T;
    uint64_t* mb = mask + (int64_t)b * T * W;
    int32_t* db = depth + (int64_t)b * T;
    memset(mb, 0, sizeof(uint64_t) * (size_t)T * (size_t)W);
    memset(db, 0, sizeof(int32_t) * (size_t)T);
    if (status && status[b] != 0) continue;
    for (int32_t i = 0; i < T; ++i) {
      int32_t u = i, d = 0;
      for (;;) {
        mb[(int64_t)i * W + u / 64] |= (uint64_t)1 << (u % 64);
        if (u == 0) break;
        u = par[u];
        ++d;
      }
      db[i] = d;
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Tree-verify attention.                                                    */
/* [EP-ko] §2 / [EP-nl] §2.C: the teacher verifies every speculative node in */
/* one batched forward pass; node i's query attends the committed prefix and */
/* the tree nodes allowed by the ancestor mask.  Readings: softmax scale is  */
/* a parameter (1/sqrt(D) by default); query head h uses KV head h/G with    */
/* G = Hq/Hkv (contiguous groups); the prefix of sequence b occupies cache   */
/* columns [lmax-len_b, lmax) (left padding, [BSD] §2 rectangular            */
/* alignment).  Key order: prefix columns ascending, then tree rows          */
/* ascending.  s = scale * q.k ; p = exp(s - max s) ; out = sum p v / sum p. */
/* ------------------------------------------------------------------------ */
void oracle_attention_row(const float* q_row, const float* k_cache_bh, const float* v_cache_bh,
                          const float* k_tree_bh, const float* v_tree_bh, const uint64_t* mask_row,
                          int32_t len_b, int32_t lmax, int32_t T, int32_t D, double scale,
                          double* out) {
  int32_t n_tree = 0;
  for (int32_t j = 0; j < T; ++j)
    if ((mask_row[j / 64] >> (j % 64)) & 1u) ++n_tree;
  int64_t n_keys = (int64_t)len_b + n_tree;
  double* s = (double*)malloc(sizeof(double) * (size_t)(n_keys > 0 ? n_keys : 1));
  const float** vrow = (const float**)malloc(sizeof(float*) * (size_t)(n_keys > 0 ? n_keys : 1));
  int64_t n = 0;
  /* prefix keys */
  for (int32_t c = lmax - len_b; c < lmax; ++c) {
    const float* k = k_cache_bh + (int64_t)c * D;
    double acc = 0.0;
    for (int32_t d = 0; d < D; ++d) acc += (double)q_row[d] * (double)k[d];
    s[n] = scale * acc;
    vrow[n] = v_cache_bh + (int64_t)c * D;
    ++n;
  }
  /* tree keys allowed by the mask */
  for (int32_t j = 0; j < T; ++j) {
    if (!((mask_row[j / 64] >> (j % 64)) & 1u)) continue;
    const float* k = k_tree_bh + (int64_t)j * D;
    double acc = 0.0;
    for (int32_t d = 0; d < D; ++d) acc += (double)q_row[d] * (double)k[d];
    s[n] = scale * acc;
    vrow[n] = v_tree_bh + (int64_t)j * D;
    ++n;
  }
  for (int32_t d = 0; d < D; ++d) out[d] = 0.0;
  if (n == 0) {
    free(s);
    free(vrow);
    return;
  }
  double m = s[0];
  for (int64_t x = 1; x < n; ++x)
    if (s[x] > m) m = s[x];
  double l = 0.0;
  for (int64_t x = 0; x < n; ++x) {
    s[x] = exp(s[x] - m);
    l += s[x];
  }
  for (int64_t x = 0; x < n; ++x)
    for (int32_t d = 0; d < D; ++d) out[d] += s[x] * (double)vrow[x][d];
  for (int32_t d = 0; d < D; ++d) out[d] /= l;
  free(s);
  free(vrow);
}

int oracle_attention(const float* q, const float* k_cache, const float* v_cache,
                     const float* k_tree, const float* v_tree, const uint64_t* mask,
                     const int32_t* len, int32_t lmax, int64_t cap, const int32_t* status,
                     int32_t B, int32_t M, int32_t Hq, int32_t Hkv, int32_t D, double scale,
                     double* out) {
  int32_t T = M + 1, W = (T + 63) / 64, G = Hq / Hkv;
  int rc = ORACLE_OK;
  for (int32_t b = 0; b < B; ++b) {
    int bad_len = (lmax < 0 || (int64_t)lmax > cap || len[b] < 0 || len[b] > lmax);
    if (bad_len) rc = ORACLE_ERR_LENGTH;
    for (int32_t i = 0; i < T; ++i) {
      for (int32_t h = 0; h < Hq; ++h) {
        double* o = out + (((int64_t)b * T + i) * Hq + h) * D;
        if (bad_len || (status && status[b] != 0)) {
          for (int32_t d = 0; d < D; ++d) o[d] = 0.0;
          continue;
        }
        int32_t g = h / G;
        oracle_attention_row(q + (((int64_t)b * T + i) * Hq + h) * D,
                             k_cache + ((int64_t)b * Hkv + g) * cap * D,
                             v_cache + ((int64_t)b * Hkv + g) * cap * D,
                             k_tree + ((int64_t)b * Hkv + g) * T * D,
                             v_tree + ((int64_t)b * Hkv + g) * T * D,
                             mask + ((int64_t)b * T + i) * W, len[b], lmax, T, D, scale, o);
      }
    }
  }
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Greedy argmax.  The teacher's greedy choice at a node is the vocabulary   */
/* entry with the largest logit ([EP-ko] §4 compares against teacher-only    */
/* greedy decoding).  Readings: ties go to the lowest index; a NaN ranks     */
/* above every number and the first NaN wins; -0.0 equals +0.0.              */
/* ------------------------------------------------------------------------ */
static int ranks_above(float a, float b) {
  if (isnan(a)) return !isnan(b);
  if (isnan(b)) return 0;
  return a > b;
}

void oracle_argmax(const float* logits, int64_t rows, int32_t V, int32_t* amax) {
  for (int64_t r = 0; r < rows; ++r) {
    const float* x = logits + r * V;
    int32_t best = 0;
    for (int32_t v = 1; v < V; ++v)
      if (ranks_above(x[v], x[best])) best = v;
    amax[r] = best;
  }
}

/* ------------------------------------------------------------------------ */
/* Acceptance.  A draft node i >= 1 is correct when its token equals the     */
/* teacher's greedy token at its parent; the root is always accepted.  A     */
/* node is accepted when every node on its root path is correct.  The        */
/* accepted node of greatest depth (lowest index on ties) ends the accepted  */
/* path; accept_len is its depth (the number of accepted draft tokens,       */
/* [EP-ko] §4 accept_L), path[k] is its ancestor at depth k (zero padded:    */
/* no negative sentinels, [EP-ko] §2), and the bonus token is the teacher's  */
/* greedy token at the end node.  Sequences with a nonzero status accept     */
/* nothing: accept_len 0, path all 0, bonus = greedy token at the root.      */
/* ------------------------------------------------------------------------ */
void oracle_accept(const int32_t* amax, const int32_t* tree_tokens, const int32_t* parents,
                   const int32_t* status, int32_t B, int32_t M,
                   int32_t* accept_len, int32_t* path, int32_t* bonus) {
  int32_t T = M + 1;
  int32_t* dep = (int32_t*)malloc(sizeof(int32_t) * (size_t)T);
  int* acc = (int*)malloc(sizeof(int) * (size_t)T);
  for (int32_t b = 0; b < B; ++b) {
    const int32_t* par = parents + (int64_t)b * T;
    const int32_t* am = amax + (int64_t)b * T;
    const int32_t* tok = tree_tokens + (int64_t)b * T;
    int32_t* pb = path + (int64_t)b * T;
    for (int32_t k = 0; k < T; ++k) pb[k] = 0;
    if (status && status[b] != 0) {
      accept_len[b] = 0;
      bonus[b] = am[0];
      continue;
    }
    for (int32_t i = 0; i < T; ++i) {
      int32_t u = i, d = 0, all_ok = 1;
      while (u != 0 && d <= M) { /* a valid tree reaches the root within M steps */
        if (tok[u] != am[par[u]]) all_ok = 0;
        u = par[u];
        ++d;
      }
      dep[i] = d;
      acc[i] = all_ok;
    }
    int32_t end = 0;
    for (int32_t i = 1; i < T; ++i)
      if (acc[i] && dep[i] > dep[end]) end = i;
    accept_len[b] = dep[end];
    for (int32_t u = end; ; u = par[u]) {
      pb[dep[u]] = u;
      if (u == 0) break;
    }
    bonus[b] = am[end];
  }
  free(dep);
  free(acc);
}

/* ------------------------------------------------------------------------ */
/* Commit.  [BSD] §2: after a verify round each sequence keeps its old       */
/* content and appends what it accepted (unpad, append, repad), so that      */
/* padding + content equals the batch maximum for every sequence             */
/* (rectangular alignment) and position ids run from 0 over the content.     */
/* Cross-batch scheduling (EXSPEC) batches sequences of equal length, whose  */
/* batch needs no realignment: the accepted rows are simply appended.        */
/* [EP-ko] §2 / [EP-nl] §2.A: the accepted rows come from the branch cache   */
/* by path index, and only the new segment is reordered.                     */
/* Readings: the committed rows are the root plus the accepted drafts        */
/* (A_b = accept_len_b + 1 rows: path[b][0..A_b)); sequences with a nonzero  */
/* status append nothing but still follow the new alignment; padding sits on */
/* the left; pos_ids padding is 0; columns past a sequence's new end are     */
/* left untouched.  In append mode every sequence keeps its start column     */
/* lmax - len_b, so the new batch maximum is lmax + max_b A_b.               */
/* ------------------------------------------------------------------------ */
static int slot_of(const int32_t* slot, int32_t b) { return slot ? slot[b] : b; }

/* Reading ([BSD] §2, SequencePool: every pool sequence keeps its own cache
 * row): a batch names each pool row at most once.  1 if two sequences share
 * a slot. */
static int slots_repeat(const int32_t* slot, int32_t B) {
  if (!slot) return 0;
  for (int32_t b = 0; b < B; ++b)
    for (int32_t c = 0; c < b; ++c)
      if (slot[c] == slot[b]) return 1;
  return 0;
}

/* Branch row of accepted step k of sequence b: the path entry, or k itself
 * for the length-based commit of [EP-nl] §2.A (no path given). */
static int32_t step_row(const int32_t* path, int32_t T, int32_t b, int32_t k) {
  return path ? path[(int64_t)b * T + k] : k;
}

int oracle_commit(uint8_t* kv_main, const uint8_t* kv_branch, int32_t n_layers, int32_t B,
                  int32_t Hkv, int64_t cap, int32_t row_bytes, int32_t M,
                  int32_t* tokens_main, const int32_t* tree_tokens, int32_t* len, int32_t* lmax,
                  int32_t* pos_ids, const int32_t* path, const int32_t* accept_len,
                  const int32_t* status, int32_t mode, const int32_t* slot, int32_t rows) {
  int32_t T = M + 1;
  int32_t old_lmax = *lmax;
  if (!slot) rows = B;
  /* Inconsistent lengths are reported before bad accept results or slots,
   * which are reported before a capacity overflow; in every case nothing
   * changes. */
  if (old_lmax < 0 || (int64_t)old_lmax > cap) return ORACLE_ERR_LENGTH;
  for (int32_t b = 0; b < B; ++b)
    if (len[b] < 0 || len[b] > old_lmax) return ORACLE_ERR_LENGTH;
  int32_t* A = (int32_t*)malloc(sizeof(int32_t) * (size_t)(B > 0 ? B : 1));
  int32_t* start = (int32_t*)malloc(sizeof(int32_t) * (size_t)(B > 0 ? B : 1));
  int32_t new_lmax = mode == 1 ? old_lmax : 0;
  int arg_bad = 0;
  for (int32_t b = 0; b < B; ++b) {
    int valid = !(status && status[b] != 0);
    if (slot_of(slot, b) < 0 || slot_of(slot, b) >= rows) arg_bad = 1;
    A[b] = 0;
    if (valid) {
      if (accept_len[b] < 0 || accept_len[b] > M) {
        arg_bad = 1;
      } else {
        A[b] = accept_len[b] + 1;
        for (int32_t k = 0; k < A[b]; ++k)
          if (step_row(path, T, b, k) < 0 || step_row(path, T, b, k) > M) arg_bad = 1;
      }
    }
    int32_t new_end = mode == 1 ? old_lmax + A[b] : len[b] + A[b];
    if (new_end > new_lmax) new_lmax = new_end;
  }
  if (slots_repeat(slot, B)) arg_bad = 1;
  if (arg_bad) { free(A); free(start); return ORACLE_ERR_ARG; }
  if ((int64_t)new_lmax > cap) { free(A); free(start); return ORACLE_ERR_CAPACITY; }
  /* New start column of each sequence's content. */
  for (int32_t b = 0; b < B; ++b)
    start[b] = mode == 1 ? old_lmax - len[b] : new_lmax - (len[b] + A[b]);

  /* Per sequence: build the logical row list (old content, then the accepted
   * branch rows in path order), then write it back from its new start. */
  uint8_t* tmp = (uint8_t*)malloc((size_t)(new_lmax > 0 ? new_lmax : 1) * (size_t)row_bytes);
  for (int32_t l = 0; l < n_layers; ++l)
    for (int32_t kv = 0; kv < 2; ++kv)
      for (int32_t b = 0; b < B; ++b)
        for (int32_t h = 0; h < Hkv; ++h) {
          int64_t slab = (((int64_t)l * 2 + kv) * rows + slot_of(slot, b)) * Hkv + h;
          int64_t bslab = (((int64_t)l * 2 + kv) * B + b) * Hkv + h;
          uint8_t* main_s = kv_main + slab * cap * row_bytes;
          const uint8_t* br_s = kv_branch + bslab * (int64_t)T * row_bytes;
          int32_t n = 0;
          for (int32_t c = old_lmax - len[b]; c < old_lmax; ++c, ++n)
            memcpy(tmp + (int64_t)n * row_bytes, main_s + (int64_t)c * row_bytes, (size_t)row_bytes);
          for (int32_t k = 0; k < A[b]; ++k, ++n)
            memcpy(tmp + (int64_t)n * row_bytes, br_s + (int64_t)step_row(path, T, b, k) * row_bytes,
                   (size_t)row_bytes);
          memcpy(main_s + (int64_t)start[b] * row_bytes, tmp, (size_t)n * (size_t)row_bytes);
        }
  free(tmp);

  int32_t* ttmp = (int32_t*)malloc(sizeof(int32_t) * (size_t)(new_lmax > 0 ? new_lmax : 1));
  for (int32_t b = 0; b < B; ++b) {
    int32_t new_len = len[b] + A[b];
    int32_t row = slot_of(slot, b);
    if (tokens_main) {
      int32_t* tm = tokens_main + (int64_t)row * cap;
      int32_t n = 0;
      for (int32_t c = old_lmax - len[b]; c < old_lmax; ++c) ttmp[n++] = tm[c];
      for (int32_t k = 0; k < A[b]; ++k)
        ttmp[n++] = tree_tokens[(int64_t)b * T + step_row(path, T, b, k)];
      for (int32_t x = 0; x < n; ++x) tm[start[b] + x] = ttmp[x];
    }
    if (pos_ids) {
      int32_t* pp = pos_ids + (int64_t)row * cap;
      for (int32_t c = 0; c < start[b] + new_len; ++c) pp[c] = c < start[b] ? 0 : c - start[b];
    }
  }
  free(ttmp);
  for (int32_t b = 0; b < B; ++b) len[b] += A[b];
  *lmax = new_lmax;
  free(A);
  free(start);
  return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Realignment.  [BSD] §2: when a batch mixes lengths, EXSPEC falls back to  */
/* EQSPEC's alignment: padding + content must equal the batch maximum for    */
/* every sequence.  Reading: the common end is the largest current end, so   */
/* the sequence(s) already ending there stay put.                            */
/* ------------------------------------------------------------------------ */
int oracle_realign(uint8_t* kv_main, int32_t n_layers, int32_t B, int32_t Hkv, int64_t cap,
                   int32_t row_bytes, int32_t* tokens_main, int32_t* pos_ids, const int32_t* slot,
                   int32_t rows, const int32_t* len, const int32_t* end, int32_t* lmax) {
  if (!slot) rows = B;
  int32_t E = 0;
  for (int32_t b = 0; b < B; ++b) {
    if (len[b] < 0 || end[b] < len[b] || (int64_t)end[b] > cap) return ORACLE_ERR_LENGTH;
    if (end[b] > E) E = end[b];
  }
  for (int32_t b = 0; b < B; ++b)
    if (slot_of(slot, b) < 0 || slot_of(slot, b) >= rows) return ORACLE_ERR_ARG;
  if (slots_repeat(slot, B)) return ORACLE_ERR_ARG;
  uint8_t* tmp = (uint8_t*)malloc((size_t)(E > 0 ? E : 1) * (size_t)row_bytes);
  for (int32_t l = 0; l < n_layers; ++l)
    for (int32_t kv = 0; kv < 2; ++kv)
      for (int32_t b = 0; b < B; ++b)
        for (int32_t h = 0; h < Hkv; ++h) {
          int64_t slab = (((int64_t)l * 2 + kv) * rows + slot_of(slot, b)) * Hkv + h;
          uint8_t* main_s = kv_main + slab * cap * row_bytes;
          memcpy(tmp, main_s + (int64_t)(end[b] - len[b]) * row_bytes, (size_t)len[b] * (size_t)row_bytes);
          memcpy(main_s + (int64_t)(E - len[b]) * row_bytes, tmp, (size_t)len[b] * (size_t)row_bytes);
        }
  free(tmp);
  int32_t* ttmp = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
  for (int32_t b = 0; b < B; ++b) {
    int32_t row = slot_of(slot, b);
    if (tokens_main) {
      int32_t* tm = tokens_main + (int64_t)row * cap;
      for (int32_t x = 0; x < len[b]; ++x) ttmp[x] = tm[end[b] - len[b] + x];
      for (int32_t x = 0; x < len[b]; ++x) tm[E - len[b] + x] = ttmp[x];
    }
    if (pos_ids) {
      int32_t* pp = pos_ids + (int64_t)row * cap;
      for (int32_t c = 0; c < E; ++c) pp[c] = c < E - len[b] ? 0 : c - (E - len[b]);
    }
  }
  free(ttmp);
  *lmax = E;
  return ORACLE_OK;
}

/* ------------------------------------------------------------------------ */
/* Dense tree mask.  [EP-nl] §2.C: token k attends token j only when j is an */
/* ancestor of k (here: or k itself); the prefix is visible to every node.   */
/* Each node's chain is walked from the parent array, independently of the   */
/* bitmask that oracle_mask builds.                                          */
/* ------------------------------------------------------------------------ */
void oracle_expand_mask(const int32_t* parents, const int32_t* len, const int32_t* status, int32_t B,
                        int32_t M, int32_t lmax, uint8_t* open, int32_t* code) {
  int32_t T = M + 1;
  int64_t width = (int64_t)lmax + T;
  memset(open, 0, (size_t)B * (size_t)T * (size_t)width);
  for (int32_t b = 0; b < B; ++b) {
    int32_t st = status ? status[b] : 0;
    code[b] = st != 0 ? st : ((len[b] >= 0 && len[b] <= lmax) ? 0 : ORACLE_ERR_LENGTH);
    if (code[b] != 0) continue;
    const int32_t* par = parents + (int64_t)b * T;
    for (int32_t i = 0; i < T; ++i) {
      uint8_t* row = open + ((int64_t)b * T + i) * width;
      for (int64_t c = lmax - len[b]; c < lmax; ++c) row[c] = 1;
      /* the node itself, then every ancestor up to the root */
      int32_t u = i;
      row[lmax + u] = 1;
      for (int32_t steps = 0; u != 0 && steps <= M; ++steps) {
        u = par[u];
        row[lmax + u] = 1;
      }
    }
  }
}
