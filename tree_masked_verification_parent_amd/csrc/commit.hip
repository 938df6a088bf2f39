// KV commit: unpad-append-repad of a ragged left-padded batch, its
// append-only form, and the realignment of a batch drawn from a pool.
//
// Sources: Batch Speculative Decoding Done Right (gist.science ko summary,
// section 2 Methodology): after each verification round every sequence keeps
// its content, appends what it accepted, and the batch is re-padded so that
// padding + content equals the batch maximum for every sequence (rectangular
// alignment) and position ids run from 0 over the content; sequences move in
// the cache when their padding changes (EQSPEC).  Cross-batch scheduling
// (EXSPEC) groups sequences of equal length so that their batch needs no
// realignment, and falls back to the alignment otherwise.  EAGLE-Pangu (ko
// summary, section 2; nl summary, section 2.A): the accepted rows come from
// the branch cache by path index and only the new segment needs reordering.
//
// Every mode is one per-sequence plan: content [src, src + len) moves to
// [dst, dst + len) and A accepted branch rows follow at `app`:
//   REPAD    src = lmax - len, dst = lmax' - (len + A), app = dst + len
//   APPEND   src = dst = lmax - len, app = lmax          (nothing moves)
//   REALIGN  src = end - len, dst = E - len, A = 0        (E = max end)
//
// Kernel 1 (commit_move_kernel): one 256-thread workgroup per (layer, K/V
// plane, KV head) slab and sequence, plus one workgroup per sequence for the
// token row and the position ids.  Every workgroup recomputes the plan
// (errors, new lmax) from the unchanged inputs, so no plan buffer is needed,
// and all of them agree on whether anything is written.  A slab whose content
// moves by delta rows is shifted in place in 16 KB chunks, walking away from
// the direction of the move (from the end when delta > 0), with every chunk
// fully read into registers before any of it is written; a chunk's
// destination never overlaps a later chunk's source, so one barrier per
// chunk orders the overlapping reads and writes.  The accepted branch rows
// are then gathered.  Rows are copied as raw 16-byte words: any bit pattern
// (NaN payloads included) survives.
//
// Kernel 2 (commit_finalize_kernel, one workgroup) runs after kernel 1 on the
// same stream and publishes the result: the status, len and lmax.
#include "svt_internal.h"

namespace svt {

enum CommitMode { kRepad = SVT_COMMIT_REPAD, kAppend = SVT_COMMIT_APPEND, kRealign = 2 };

struct CommitDev {
  uint4* kv;                 // [layers][2][rows][Hkv][cap] rows of row16 words
  const uint4* br;           // [layers][2][B][Hkv][T] (commit modes)
  int32_t* tok;              // [rows][cap] or NULL
  const int32_t* ttok;       // [B][T]
  int32_t* pos;              // [rows][cap] or NULL
  const int32_t* slot;       // [B] or NULL (row b)
  const int32_t* len;        // [B]
  const int32_t* lmax;       // [1] (commit modes)
  const int32_t* end;        // [B] (realign)
  const int32_t* path;       // [B][T], or NULL: row k of the branch is step k (length-based)
  const int32_t* acc;        // [B] (commit modes)
  const int32_t* status;     // [B] or NULL
  int32_t* len_out;          // [B] new lengths (commit modes): len itself or a separate array
  int32_t* lmax_out;         // [1]
  int32_t* status_out;       // [1]
  int64_t cap;
  int B, M, Hkv, rows, n_slab_x, row16, mode;
};

struct CommitPlan {
  int code;      // SVT_OK or the reason nothing is written
  int old_lmax;  // commit modes: lmax before the call
  int new_lmax;  // lmax after the call
};

__device__ __forceinline__ int accepted_rows(const CommitDev& d, int b) {
  if (d.mode == kRealign) return 0;
  const bool valid = d.status == nullptr || d.status[b] == 0;
  return valid ? d.acc[b] + 1 : 0;
}

// Slot bitmap of the duplicate check: bit (slot mod kSlotBits).
constexpr int kSlotBits = 32768;

// Block-wide computation of the plan.  All threads return the same plan.
__device__ CommitPlan compute_commit_plan(const CommitDev& d) {
  __shared__ int s_len_bad, s_arg_bad, s_new_lmax;
  __shared__ uint32_t s_seen[kSlotBits / 32];
  const int T = d.M + 1;
  const int tid = threadIdx.x;
  if (tid == 0) {
    s_len_bad = 0;
    s_arg_bad = 0;
    s_new_lmax = 0;
  }
  if (d.slot)
    for (int w = tid; w < kSlotBits / 32; w += blockDim.x) s_seen[w] = 0u;
  __syncthreads();
  const int old_lmax = d.mode == kRealign ? 0 : *d.lmax;
  const bool lmax_bad = d.mode != kRealign && (old_lmax < 0 || (int64_t)old_lmax > d.cap);
  int len_bad = 0, arg_bad = 0, mx = 0;
  for (int b = tid; b < d.B; b += blockDim.x) {
    const int L = d.len[b];
    const int row = d.slot ? d.slot[b] : b;
    if (row < 0 || row >= d.rows) {
      arg_bad = 1;
    } else if (d.slot) {
      // Two sequences on one pool row would shift and gather the same slabs
      // at once.  A repeated residue is confirmed by a scan (a larger pool
      // can map different slots to one bit).
      const int bit = row & (kSlotBits - 1);
      const uint32_t m = 1u << (bit & 31);
      if (atomicOr(&s_seen[bit >> 5], m) & m)
        for (int c = 0; c < d.B; ++c)
          if (c != b && d.slot[c] == row) arg_bad = 1;
    }
    if (d.mode == kRealign) {
      const int e = d.end[b];
      if (L < 0 || e < L || (int64_t)e > d.cap) len_bad = 1;
      mx = e > mx ? e : mx;
      continue;
    }
    if (L < 0 || L > old_lmax) len_bad = 1;
    const bool valid = d.status == nullptr || d.status[b] == 0;
    int A = 0;
    if (valid) {
      const int al = d.acc[b];
      if (al < 0 || al > d.M) arg_bad = 1;
      else A = al + 1;
    }
    const int ne = d.mode == kAppend ? old_lmax + A : L + A;
    mx = ne > mx ? ne : mx;
  }
  if (d.mode != kRealign && d.path) {
    for (int x = tid; x < d.B * T; x += blockDim.x) {
      const int b = x / T, k = x % T;
      const bool valid = d.status == nullptr || d.status[b] == 0;
      if (!valid) continue;
      const int al = d.acc[b];
      if (al >= 0 && al <= d.M && k <= al) {
        const int p = d.path[x];
        if (p < 0 || p > d.M) arg_bad = 1;
      }
    }
  }
  if (len_bad) atomicOr(&s_len_bad, 1);
  if (arg_bad) atomicOr(&s_arg_bad, 1);
  atomicMax(&s_new_lmax, mx);
  __syncthreads();
  CommitPlan p;
  p.old_lmax = old_lmax;
  p.new_lmax = (d.mode == kAppend && d.B == 0) ? old_lmax : s_new_lmax;
  if (lmax_bad || s_len_bad) p.code = SVT_ERR_LENGTH;
  else if (s_arg_bad) p.code = SVT_ERR_ARG;
  else if ((int64_t)p.new_lmax > d.cap) p.code = SVT_ERR_CAPACITY;
  else p.code = SVT_OK;
  __syncthreads();  // the shared words may be reused by a later call site
  return p;
}

// Shift n elements (E = one 16-byte word or one int32) from src to src + delta
// inside one slab.  All threads of the block take part.  A chunk is four
// elements per thread, staged in four named registers (an array here ends up
// in scratch or LDS, depending on what else the kernel allocates).
template <typename E>
__device__ void shift_in_place(E* __restrict__ base, int64_t src_off, int64_t n, int64_t delta) {
  if (delta == 0 || n <= 0) return;
  constexpr int CH = 256 * 4;
  const int tid = threadIdx.x;
  const int64_t nch = (n + CH - 1) / CH;
  E* src = base + src_off;
  E* dst = src + delta;
  for (int64_t c = 0; c < nch; ++c) {
    const int64_t ci = delta > 0 ? (nch - 1 - c) : c;
    const int64_t i0 = ci * CH + tid, i1 = i0 + 256, i2 = i0 + 512, i3 = i0 + 768;
    E r0{}, r1{}, r2{}, r3{};
    if (i0 < n) r0 = src[i0];
    if (i1 < n) r1 = src[i1];
    if (i2 < n) r2 = src[i2];
    if (i3 < n) r3 = src[i3];
    __syncthreads();
    if (i0 < n) dst[i0] = r0;
    if (i1 < n) dst[i1] = r1;
    if (i2 < n) dst[i2] = r2;
    if (i3 < n) dst[i3] = r3;
  }
  __syncthreads();
}

__global__ __launch_bounds__(256) void commit_move_kernel(CommitDev d) {
  const CommitPlan plan = compute_commit_plan(d);
  if (plan.code != SVT_OK) return;
  const int T = d.M + 1;
  const int b = blockIdx.y;
  const int x = blockIdx.x;
  const int L = d.len[b];
  const int row = d.slot ? d.slot[b] : b;
  const int A = accepted_rows(d, b);
  int src, dst, app, pend;  // pend: position ids are written for columns < pend
  if (d.mode == kRepad) {
    src = plan.old_lmax - L;
    dst = plan.new_lmax - (L + A);
    app = dst + L;
    pend = plan.new_lmax;
  } else if (d.mode == kAppend) {
    src = dst = plan.old_lmax - L;
    app = plan.old_lmax;
    pend = plan.old_lmax + A;
  } else {
    src = d.end[b] - L;
    dst = plan.new_lmax - L;
    app = dst + L;
    pend = plan.new_lmax;
  }
  const int tid = threadIdx.x;
  const int32_t* pb = d.path ? d.path + (int64_t)b * T : nullptr;

  if (x < d.n_slab_x) {
    // x = (layer * 2 + plane) * Hkv + h
    const int h = x % d.Hkv;
    const int lp = x / d.Hkv;
    uint4* main_s = d.kv + (((int64_t)lp * d.rows + row) * d.Hkv + h) * d.cap * d.row16;
    shift_in_place<uint4>(main_s, (int64_t)src * d.row16, (int64_t)L * d.row16, (int64_t)(dst - src) * d.row16);
    if (A > 0) {
      const uint4* br_s = d.br + (((int64_t)lp * d.B + b) * d.Hkv + h) * (int64_t)T * d.row16;
      uint4* out = main_s + (int64_t)app * d.row16;
      const int n = A * d.row16;
      for (int i = tid; i < n; i += 256) {
        const int k = i / d.row16, e = i % d.row16;
        out[i] = br_s[(int64_t)(pb ? pb[k] : k) * d.row16 + e];
      }
    }
  } else {
    if (d.tok) {
      int32_t* tm = d.tok + (int64_t)row * d.cap;
      shift_in_place<int32_t>(tm, src, L, (int64_t)dst - src);
      for (int k = tid; k < A; k += 256) tm[app + k] = d.ttok[(int64_t)b * T + (pb ? pb[k] : k)];
    }
    if (d.pos) {
      int32_t* pp = d.pos + (int64_t)row * d.cap;
      for (int c = tid; c < pend; c += 256) pp[c] = c < dst ? 0 : c - dst;
    }
  }
}

__global__ __launch_bounds__(256) void commit_finalize_kernel(CommitDev d) {
  const CommitPlan plan = compute_commit_plan(d);
  if (threadIdx.x == 0) d.status_out[0] = plan.code;
  if (plan.code != SVT_OK) return;
  if (d.mode != kRealign)
    for (int b = threadIdx.x; b < d.B; b += blockDim.x) d.len_out[b] = d.len[b] + accepted_rows(d, b);
  if (threadIdx.x == 0) *d.lmax_out = plan.new_lmax;
}

// LDS reserved per move workgroup (unused by the kernel) so that at most two
// run on a CU at once: with fewer shifts streaming at the same time the HBM
// serves the read-then-write chunks faster (B=32 workload, 36 layers: 6436 ->
// 6362 us per commit; one per CU 6704, four 6378, six 6439, eight 6436).
constexpr unsigned kMoveLdsPad = 74 * 1024;

static hipError_t launch_move(CommitDev d, int n_layers, hipStream_t s) {
  d.n_slab_x = n_layers * 2 * d.Hkv;
  if (d.B > 0) {
    dim3 grid(d.n_slab_x + 1, d.B), block(256);
    hipLaunchKernelGGL(commit_move_kernel, grid, block, kMoveLdsPad, s, d);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(commit_finalize_kernel, dim3(1), dim3(256), 0, s, d);
  return hipGetLastError();
}

hipError_t launch_commit(const svt_commit_args* a, hipStream_t s) {
  CommitDev d{};
  const int esize = a->dtype == SVT_FP32 ? 4 : 2;
  d.kv = static_cast<uint4*>(a->kv_main);
  d.br = static_cast<const uint4*>(a->kv_branch);
  d.tok = a->tokens_main;
  d.ttok = a->tree_tokens;
  d.pos = a->pos_ids;
  d.slot = a->seq_slot;
  d.len = a->len;
  d.lmax = a->lmax;
  d.path = a->path;
  d.acc = a->accept_len;
  d.status = a->status;
  d.len_out = a->len_out ? a->len_out : a->len;
  d.lmax_out = a->lmax_out ? a->lmax_out : a->lmax;
  d.status_out = a->commit_status;
  d.cap = a->cap;
  d.B = a->B;
  d.M = a->M;
  d.Hkv = a->Hkv;
  d.rows = a->seq_slot ? a->n_slots : a->B;
  d.row16 = a->D * esize / 16;
  d.mode = a->mode;
  return launch_move(d, a->n_layers, s);
}

hipError_t launch_commit_length(const svt_commit_args* a, hipStream_t s) {
  svt_commit_args b = *a;
  b.path = nullptr;
  return launch_commit(&b, s);
}

hipError_t launch_realign(const svt_realign_args* a, hipStream_t s) {
  CommitDev d{};
  const int esize = a->dtype == SVT_FP32 ? 4 : 2;
  d.kv = static_cast<uint4*>(a->kv_main);
  d.tok = a->tokens_main;
  d.pos = a->pos_ids;
  d.slot = a->seq_slot;
  d.len = a->len;
  d.end = a->end;
  d.lmax_out = a->lmax;
  d.status_out = a->realign_status;
  d.cap = a->cap;
  d.B = a->B;
  d.M = 0;
  d.Hkv = a->Hkv;
  d.rows = a->seq_slot ? a->n_slots : a->B;
  d.row16 = a->D * esize / 16;
  d.mode = kRealign;
  return launch_move(d, a->n_layers, s);
}

}  // namespace svt
