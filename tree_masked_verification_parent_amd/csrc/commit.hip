// KV commit: unpad-append-repad of a ragged left-padded batch.
//
// Sources: Batch Speculative Decoding Done Right (gist.science ko summary,
// section 2 Methodology): after each verification round every sequence keeps
// its content, appends what it accepted, and the batch is re-padded so that
// padding + content equals the batch maximum for every sequence (rectangular
// alignment) and position ids run from 0 over the content; sequences move in
// the cache when their padding changes.  EAGLE-Pangu (ko summary, section 2;
// nl summary, section 2.A): the accepted rows come from the branch cache by
// path index and only the new segment needs reordering.
//
// Kernel 1 (commit_move_kernel): one 256-thread workgroup per (layer, K/V
// plane, KV head) slab and sequence, plus one workgroup per sequence for the
// token row and the position ids.  Every workgroup recomputes the round plan
// (new lmax, pads) from the unchanged len/lmax/accept_len, so no plan buffer is
// needed, and all of them agree on whether the commit goes ahead.  A slab
// whose padding changes by delta rows is shifted in place in 16 KB chunks,
// walking away from the direction of the move (from the end when delta > 0),
// with every chunk fully read into registers before any of it is written; a
// chunk's destination never overlaps a later chunk's source, so one barrier
// per chunk orders the overlapping reads and writes.  The accepted branch
// rows are then gathered after the moved content.  Rows are copied as raw
// 16-byte words: any bit pattern (NaN payloads included) survives.
//
// Kernel 2 (commit_finalize_kernel, one workgroup) runs after kernel 1 on the
// same stream and publishes the result: commit_status, len and lmax.
#include "svt_internal.h"

namespace svt {

struct CommitPlan {
  int code;      // SVT_OK or the reason nothing is written
  int old_lmax;
  int new_lmax;
};

// Block-wide computation of the round plan.  All threads return the same plan.
__device__ CommitPlan compute_commit_plan(const int32_t* __restrict__ len, const int32_t* __restrict__ lmax_p,
                                          const int32_t* __restrict__ accept_len,
                                          const int32_t* __restrict__ status,
                                          const int32_t* __restrict__ path, int B, int M, int64_t cap) {
  __shared__ int s_len_bad, s_arg_bad, s_new_lmax;
  const int T = M + 1;
  const int tid = threadIdx.x;
  if (tid == 0) {
    s_len_bad = 0;
    s_arg_bad = 0;
    s_new_lmax = 0;
  }
  __syncthreads();
  const int old_lmax = *lmax_p;
  const bool lmax_bad = old_lmax < 0 || (int64_t)old_lmax > cap;
  int len_bad = 0, arg_bad = 0, mx = 0;
  for (int b = tid; b < B; b += blockDim.x) {
    const int L = len[b];
    if (L < 0 || L > old_lmax) len_bad = 1;
    const bool valid = status == nullptr || status[b] == 0;
    int A = 0;
    if (valid) {
      const int al = accept_len[b];
      if (al < 0 || al > M) arg_bad = 1;
      else A = al + 1;
    }
    const int nl = L + A;
    mx = nl > mx ? nl : mx;
  }
  for (int x = tid; x < B * T; x += blockDim.x) {
    const int b = x / T, k = x % T;
    const bool valid = status == nullptr || status[b] == 0;
    if (!valid) continue;
    const int al = accept_len[b];
    if (al >= 0 && al <= M && k <= al) {
      const int p = path[x];
      if (p < 0 || p > M) arg_bad = 1;
    }
  }
  if (len_bad) atomicOr(&s_len_bad, 1);
  if (arg_bad) atomicOr(&s_arg_bad, 1);
  atomicMax(&s_new_lmax, mx);
  __syncthreads();
  CommitPlan p;
  p.old_lmax = old_lmax;
  p.new_lmax = s_new_lmax;
  if (lmax_bad || s_len_bad) p.code = SVT_ERR_LENGTH;
  else if (s_arg_bad) p.code = SVT_ERR_ARG;
  else if ((int64_t)p.new_lmax > cap) p.code = SVT_ERR_CAPACITY;
  else p.code = SVT_OK;
  __syncthreads();  // the shared words may be reused by a later call site
  return p;
}

// Shift n elements (E = one 16-byte word or one int32) from src to src + delta
// inside one slab.  All threads of the block take part.
template <typename E, int U>
__device__ void shift_in_place(E* __restrict__ base, int64_t src_off, int64_t n, int64_t delta) {
  if (delta == 0 || n <= 0) return;
  constexpr int CH = 256 * U;
  const int tid = threadIdx.x;
  const int64_t nch = (n + CH - 1) / CH;
  E* src = base + src_off;
  E* dst = src + delta;
  for (int64_t c = 0; c < nch; ++c) {
    const int64_t ci = delta > 0 ? (nch - 1 - c) : c;
    const int64_t lo = ci * CH;
    E r[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = lo + u * 256 + tid;
      if (i < n) r[u] = src[i];
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = lo + u * 256 + tid;
      if (i < n) dst[i] = r[u];
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(256) void commit_move_kernel(
    uint4* __restrict__ kv_main, const uint4* __restrict__ kv_branch, int32_t* __restrict__ tokens_main,
    const int32_t* __restrict__ tree_tokens, const int32_t* __restrict__ len, const int32_t* __restrict__ lmax_p,
    int32_t* __restrict__ pos_ids, const int32_t* __restrict__ path, const int32_t* __restrict__ accept_len,
    const int32_t* __restrict__ status, int B, int M, int Hkv, int n_slab_x, int64_t cap, int row16) {
  const CommitPlan plan = compute_commit_plan(len, lmax_p, accept_len, status, path, B, M, cap);
  if (plan.code != SVT_OK) return;
  const int T = M + 1;
  const int b = blockIdx.y;
  const int x = blockIdx.x;
  const int L = len[b];
  const bool valid = status == nullptr || status[b] == 0;
  const int A = valid ? accept_len[b] + 1 : 0;
  const int old_pad = plan.old_lmax - L;
  const int new_pad = plan.new_lmax - (L + A);
  const int tid = threadIdx.x;
  const int32_t* pb = path + (int64_t)b * T;

  if (x < n_slab_x) {
    // x = (layer * 2 + plane) * Hkv + h ; slab index in [L][2][B][Hkv]
    const int h = x % Hkv;
    const int lp = x / Hkv;
    const int64_t slab = ((int64_t)lp * B + b) * Hkv + h;
    uint4* main_s = kv_main + slab * cap * row16;
    const uint4* br_s = kv_branch + slab * (int64_t)T * row16;
    shift_in_place<uint4, 4>(main_s, (int64_t)old_pad * row16, (int64_t)L * row16,
                             (int64_t)(new_pad - old_pad) * row16);
    // gather the accepted rows after the content
    uint4* dst = main_s + (int64_t)(new_pad + L) * row16;
    const int n = A * row16;
    for (int i = tid; i < n; i += 256) {
      const int k = i / row16, e = i % row16;
      dst[i] = br_s[(int64_t)pb[k] * row16 + e];
    }
  } else {
    if (tokens_main) {
      int32_t* tm = tokens_main + (int64_t)b * cap;
      shift_in_place<int32_t, 4>(tm, old_pad, L, (int64_t)new_pad - old_pad);
      for (int k = tid; k < A; k += 256) tm[new_pad + L + k] = tree_tokens[(int64_t)b * T + pb[k]];
    }
    if (pos_ids) {
      int32_t* pp = pos_ids + (int64_t)b * cap;
      for (int c = tid; c < plan.new_lmax; c += 256) pp[c] = c < new_pad ? 0 : c - new_pad;
    }
  }
}

__global__ __launch_bounds__(256) void commit_finalize_kernel(int32_t* __restrict__ len, int32_t* __restrict__ lmax_p,
                                                              const int32_t* __restrict__ path,
                                                              const int32_t* __restrict__ accept_len,
                                                              const int32_t* __restrict__ status,
                                                              int32_t* __restrict__ commit_status, int B, int M,
                                                              int64_t cap) {
  const CommitPlan plan = compute_commit_plan(len, lmax_p, accept_len, status, path, B, M, cap);
  if (threadIdx.x == 0) commit_status[0] = plan.code;
  if (plan.code != SVT_OK) return;
  for (int b = threadIdx.x; b < B; b += blockDim.x) {
    const bool valid = status == nullptr || status[b] == 0;
    len[b] += valid ? accept_len[b] + 1 : 0;
  }
  if (threadIdx.x == 0) *lmax_p = plan.new_lmax;
}

hipError_t launch_commit(const svt_commit_args* a, hipStream_t s) {
  const int esize = a->dtype == SVT_FP32 ? 4 : 2;
  const int row16 = a->D * esize / 16;
  const int n_slab_x = a->n_layers * 2 * a->Hkv;
  if (a->B > 0) {
    dim3 grid(n_slab_x + 1, a->B), block(256);
    hipLaunchKernelGGL(commit_move_kernel, grid, block, 0, s, static_cast<uint4*>(a->kv_main),
                       static_cast<const uint4*>(a->kv_branch), a->tokens_main, a->tree_tokens, a->len, a->lmax,
                       a->pos_ids, a->path, a->accept_len, a->status, a->B, a->M, a->Hkv, n_slab_x, a->cap, row16);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(commit_finalize_kernel, dim3(1), dim3(256), 0, s, a->len, a->lmax, a->path, a->accept_len,
                     a->status, a->commit_status, a->B, a->M, a->cap);
  return hipGetLastError();
}

}  // namespace svt
