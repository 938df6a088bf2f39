// C-ABI entry points of libsvt: host-side argument checks, launch, tracing.
// Every device step runs in the kernels of mask.hip, attn.hip, accept.hip and
// commit.hip; this file only validates, sizes and enqueues.
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "svt_internal.h"

namespace {

bool trace_on() {
  static int on = -1;
  if (on < 0) {
    const char* e = std::getenv("SVT_TRACE");
    on = (e && e[0] && e[0] != '0') ? 1 : 0;
  }
  return on == 1;
}

int finish(const char* name, int rc, const char* shape) {
  if (trace_on()) std::fprintf(stderr, "[svt] %s %s -> %d (%s)\n", name, shape, rc, svt_status_string(rc));
  return rc;
}

int hip_rc(hipError_t e) { return e == hipSuccess ? SVT_OK : SVT_ERR_HIP; }

bool aligned(const void* p, size_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

}  // namespace

extern "C" {

int svt_build_mask(const int32_t* parents, int32_t B, int32_t M, uint64_t* mask, int32_t* depth,
                   int32_t* status, int32_t flags, hipStream_t stream) {
  char shape[96];
  std::snprintf(shape, sizeof shape, "B=%d M=%d", B, M);
  if (B < 0 || M < 0) return finish("svt_build_mask", SVT_ERR_ARG, shape);
  if (M >= SVT_MAX_T) return finish("svt_build_mask", SVT_ERR_UNSUPPORTED, shape);
  if (B == 0) return finish("svt_build_mask", SVT_OK, shape);
  if (!parents || !mask || !depth || !status || !aligned(mask, 8)) return finish("svt_build_mask", SVT_ERR_ARG, shape);
  int rc = hip_rc(svt::launch_build_mask(parents, B, M, mask, depth, status, stream));
  if (rc == SVT_OK && (flags & SVT_SYNC_CHECK)) rc = svt_check_status(status, B, stream);
  return finish("svt_build_mask", rc, shape);
}

int svt_expand_mask(const uint64_t* mask, const int32_t* status, const int32_t* len, int32_t B, int32_t M,
                    int32_t lmax, void* out, int32_t kind, int32_t* seq_status, hipStream_t stream) {
  char shape[96];
  std::snprintf(shape, sizeof shape, "B=%d M=%d lmax=%d kind=%d", B, M, lmax, kind);
  if (B < 0 || M < 0 || lmax < 0 || kind < SVT_MASK_ADD_FP32 || kind > SVT_MASK_BOOL)
    return finish("svt_expand_mask", SVT_ERR_ARG, shape);
  if (M >= SVT_MAX_T) return finish("svt_expand_mask", SVT_ERR_UNSUPPORTED, shape);
  if (B == 0) return finish("svt_expand_mask", SVT_OK, shape);
  if (!mask || !len || !out || !aligned(mask, 8) || !aligned(out, 16)) return finish("svt_expand_mask", SVT_ERR_ARG, shape);
  if ((int64_t)B * (M + 1) >= 0x7FFFFFFF || (int64_t)lmax + M + 1 > (int64_t)65535 * 256)
    return finish("svt_expand_mask", SVT_ERR_UNSUPPORTED, shape);
  return finish("svt_expand_mask", hip_rc(svt::launch_expand_mask(mask, status, len, B, M, lmax, out, kind,
                                                                   seq_status, stream)), shape);
}

size_t svt_verify_attention_workspace(const svt_attn_args* a) {
  svt::AttnPlan p;
  if (!svt::plan_attention(a, &p)) return 0;
  return p.ws_bytes;
}

int svt_verify_attention(const svt_attn_args* a, hipStream_t stream) {
  char shape[160];
  if (!a) return finish("svt_verify_attention", SVT_ERR_ARG, "null args");
  std::snprintf(shape, sizeof shape, "B=%d M=%d Hq=%d Hkv=%d D=%d dtype=%d cap=%lld lmax_bound=%d form=%d split_keys=%d",
                a->B, a->M, a->Hq, a->Hkv, a->D, a->dtype, (long long)a->cap, a->lmax_bound, a->form, a->split_keys);
  if (a->B < 0 || a->M < 0 || a->Hq <= 0 || a->Hkv <= 0 || a->Hq % a->Hkv != 0 || a->cap < 0 ||
      a->lmax_bound < 0 || (int64_t)a->lmax_bound > a->cap || !(a->scale >= 0.0f))
    return finish("svt_verify_attention", SVT_ERR_ARG, shape);
  if (a->form < SVT_ATTN_AUTO || a->form > SVT_ATTN_STREAM) return finish("svt_verify_attention", SVT_ERR_ARG, shape);
  if (a->split_keys < 0 || a->split_keys % 64 != 0 || (a->split_keys > 0 && a->form == SVT_ATTN_STREAM))
    return finish("svt_verify_attention", SVT_ERR_ARG, shape);
  if (a->seq_slot && a->n_slots <= 0) return finish("svt_verify_attention", SVT_ERR_ARG, shape);
  if (a->M >= SVT_MAX_T || (a->D != 64 && a->D != 128) || (a->dtype != SVT_FP32 && a->dtype != SVT_BF16))
    return finish("svt_verify_attention", SVT_ERR_UNSUPPORTED, shape);
  if (a->form == SVT_ATTN_STREAM &&
      (a->dtype != SVT_BF16 || a->B > svt::kStreamMaxBatch))
    return finish("svt_verify_attention", SVT_ERR_UNSUPPORTED, shape);
  if (a->B == 0) return finish("svt_verify_attention", SVT_OK, shape);
  if (!a->q || !a->k_cache || !a->v_cache || !a->len || !a->lmax || !a->k_tree || !a->v_tree || !a->mask ||
      !a->out)
    return finish("svt_verify_attention", SVT_ERR_ARG, shape);
  if (!aligned(a->q, 16) || !aligned(a->k_cache, 16) || !aligned(a->v_cache, 16) || !aligned(a->k_tree, 16) ||
      !aligned(a->v_tree, 16) || !aligned(a->out, 16) || !aligned(a->mask, 8))
    return finish("svt_verify_attention", SVT_ERR_ARG, shape);
  svt::AttnPlan p;
  if (!svt::plan_attention(a, &p)) return finish("svt_verify_attention", SVT_ERR_ARG, shape);
  if (p.ws_bytes > 0 && (!a->workspace || a->workspace_bytes < p.ws_bytes || !aligned(a->workspace, 16)))
    return finish("svt_verify_attention", SVT_ERR_WORKSPACE, shape);
  return finish("svt_verify_attention", hip_rc(svt::launch_attention(a, p, stream)), shape);
}

size_t svt_accept_workspace(const svt_accept_args* a) {
  svt::AcceptPlan p;
  if (!svt::plan_accept(a, &p)) return 0;
  return p.ws_bytes;
}

// Host checks shared by svt_accept and svt_accept_noalloc (everything but the
// workspace); SVT_OK with *p filled, or the status to return.
static int accept_checks(const svt_accept_args* a, svt::AcceptPlan* p) {
  if (a->B < 0 || a->M < 0 || a->V <= 0) return SVT_ERR_ARG;
  if (a->M >= SVT_MAX_T) return SVT_ERR_UNSUPPORTED;
  if (a->B == 0) return SVT_OK;
  if (!a->logits || !a->tree_tokens || !a->parents || !a->mask || !a->depth || !a->amax || !a->accept_len ||
      !a->path || !a->bonus || !aligned(a->mask, 8) || !aligned(a->logits, 4))
    return SVT_ERR_ARG;
  if (!svt::plan_accept(a, p)) return SVT_ERR_ARG;
  if ((int64_t)p->rows * p->nchunk > 0x7FFFFFFF) return SVT_ERR_UNSUPPORTED;
  return SVT_OK;
}

int svt_accept(const svt_accept_args* a, hipStream_t stream) {
  char shape[96];
  if (!a) return finish("svt_accept", SVT_ERR_ARG, "null args");
  std::snprintf(shape, sizeof shape, "B=%d M=%d V=%d", a->B, a->M, a->V);
  svt::AcceptPlan p;
  const int rc = accept_checks(a, &p);
  if (rc != SVT_OK || a->B == 0) return finish("svt_accept", rc, shape);
  if (!a->workspace || a->workspace_bytes < p.ws_bytes || !aligned(a->workspace, 8))
    return finish("svt_accept", SVT_ERR_WORKSPACE, shape);
  return finish("svt_accept", hip_rc(svt::launch_accept(a, p, stream)), shape);
}

int svt_accept_noalloc(const svt_accept_args* a, hipStream_t stream) {
  char shape[96];
  if (!a) return finish("svt_accept_noalloc", SVT_ERR_ARG, "null args");
  std::snprintf(shape, sizeof shape, "B=%d M=%d V=%d", a->B, a->M, a->V);
  svt::AcceptPlan p;
  const int rc = accept_checks(a, &p);
  if (rc != SVT_OK || a->B == 0) return finish("svt_accept_noalloc", rc, shape);
  if (p.ws_bytes > svt::kAcceptScratchBytes) {
    if (trace_on())
      std::fprintf(stderr, "[svt] svt_accept_noalloc needs %zu scratch bytes, the static buffer holds %zu\n",
                   p.ws_bytes, svt::kAcceptScratchBytes);
    return finish("svt_accept_noalloc", SVT_ERR_WORKSPACE, shape);
  }
  void* ws = nullptr;  // device address of the static scratch on the current device
  if (svt::accept_scratch(&ws) != hipSuccess || !ws) return finish("svt_accept_noalloc", SVT_ERR_HIP, shape);
  svt_accept_args b = *a;
  b.workspace = ws;
  b.workspace_bytes = svt::kAcceptScratchBytes;
  return finish("svt_accept_noalloc", hip_rc(svt::launch_accept(&b, p, stream)), shape);
}

static int commit_impl(const char* name, const svt_commit_args* a, bool by_length, int32_t flags,
                       hipStream_t stream) {
  char shape[128];
  if (!a) return finish(name, SVT_ERR_ARG, "null args");
  std::snprintf(shape, sizeof shape, "B=%d M=%d Hkv=%d D=%d layers=%d dtype=%d cap=%lld mode=%d slots=%d", a->B, a->M,
                a->Hkv, a->D, a->n_layers, a->dtype, (long long)a->cap, a->mode, a->seq_slot ? a->n_slots : -1);
  if (a->B < 0 || a->M < 0 || a->Hkv < 0 || a->D <= 0 || a->n_layers < 0 || a->cap < 0 || a->cap > 0x7FFFFFFF)
    return finish(name, SVT_ERR_ARG, shape);
  if (a->mode != SVT_COMMIT_REPAD && a->mode != SVT_COMMIT_APPEND) return finish(name, SVT_ERR_ARG, shape);
  if (a->seq_slot && a->n_slots <= 0) return finish(name, SVT_ERR_ARG, shape);
  if (a->M >= SVT_MAX_T || (a->dtype != SVT_FP32 && a->dtype != SVT_BF16))
    return finish(name, SVT_ERR_UNSUPPORTED, shape);
  const int esize = a->dtype == SVT_FP32 ? 4 : 2;
  if ((a->D * esize) % 16 != 0) return finish(name, SVT_ERR_UNSUPPORTED, shape);
  // per-sequence arrays may be NULL only for an empty batch
  if (!a->lmax || !a->commit_status || (a->B > 0 && (!a->len || (!by_length && !a->path) || !a->accept_len)))
    return finish(name, SVT_ERR_ARG, shape);
  const bool has_kv = a->n_layers > 0 && a->Hkv > 0 && a->B > 0;
  if (has_kv && (!a->kv_main || !a->kv_branch || !aligned(a->kv_main, 16) || !aligned(a->kv_branch, 16)))
    return finish(name, SVT_ERR_ARG, shape);
  if (a->tokens_main && !a->tree_tokens) return finish(name, SVT_ERR_ARG, shape);
  int rc = hip_rc(by_length ? svt::launch_commit_length(a, stream) : svt::launch_commit(a, stream));
  if (rc == SVT_OK && (flags & SVT_SYNC_CHECK)) rc = svt_check_status(a->commit_status, 1, stream);
  return finish(name, rc, shape);
}

int svt_commit(const svt_commit_args* a, int32_t flags, hipStream_t stream) {
  return commit_impl("svt_commit", a, false, flags, stream);
}

int svt_commit_length(const svt_commit_args* a, int32_t flags, hipStream_t stream) {
  return commit_impl("svt_commit_length", a, true, flags, stream);
}

int svt_realign(const svt_realign_args* a, int32_t flags, hipStream_t stream) {
  char shape[128];
  if (!a) return finish("svt_realign", SVT_ERR_ARG, "null args");
  std::snprintf(shape, sizeof shape, "B=%d Hkv=%d D=%d layers=%d dtype=%d cap=%lld slots=%d", a->B, a->Hkv, a->D,
                a->n_layers, a->dtype, (long long)a->cap, a->seq_slot ? a->n_slots : -1);
  if (a->B < 0 || a->Hkv < 0 || a->D <= 0 || a->n_layers < 0 || a->cap < 0 || a->cap > 0x7FFFFFFF)
    return finish("svt_realign", SVT_ERR_ARG, shape);
  if (a->dtype != SVT_FP32 && a->dtype != SVT_BF16) return finish("svt_realign", SVT_ERR_UNSUPPORTED, shape);
  const int esize = a->dtype == SVT_FP32 ? 4 : 2;
  if ((a->D * esize) % 16 != 0) return finish("svt_realign", SVT_ERR_UNSUPPORTED, shape);
  if (!a->lmax || !a->realign_status || (a->B > 0 && (!a->len || !a->end)) || (a->seq_slot && a->n_slots <= 0))
    return finish("svt_realign", SVT_ERR_ARG, shape);
  const bool has_kv = a->n_layers > 0 && a->Hkv > 0 && a->B > 0;
  if (has_kv && (!a->kv_main || !aligned(a->kv_main, 16))) return finish("svt_realign", SVT_ERR_ARG, shape);
  int rc = hip_rc(svt::launch_realign(a, stream));
  if (rc == SVT_OK && (flags & SVT_SYNC_CHECK)) rc = svt_check_status(a->realign_status, 1, stream);
  return finish("svt_realign", rc, shape);
}

int svt_pool_pick(const int32_t* end_host, const int32_t* active_host, int32_t n_slots, int32_t max_batch,
                  int32_t min_group, int32_t* slots_host, int32_t* n_host) {
  if (n_slots < 0 || max_batch < 1 || min_group < 1 || !n_host || (n_slots > 0 && (!end_host || !active_host)) ||
      !slots_host)
    return SVT_ERR_ARG;
  return svt::pool_pick(end_host, active_host, n_slots, max_batch, min_group, slots_host, n_host);
}

int svt_check_status(const int32_t* status, int32_t n, hipStream_t stream) {
  if (n < 0 || (n > 0 && !status)) return SVT_ERR_ARG;
  if (hipStreamSynchronize(stream) != hipSuccess) return SVT_ERR_HIP;
  if (n == 0) return SVT_OK;
  int32_t small[64];
  int32_t* host = n <= 64 ? small : static_cast<int32_t*>(std::malloc(sizeof(int32_t) * (size_t)n));
  if (!host) return SVT_ERR_HIP;
  int rc = SVT_OK;
  if (hipMemcpy(host, status, sizeof(int32_t) * (size_t)n, hipMemcpyDeviceToHost) != hipSuccess) rc = SVT_ERR_HIP;
  for (int32_t i = 0; rc == SVT_OK && i < n; ++i)
    if (host[i] != SVT_OK) rc = host[i];
  if (host != small) std::free(host);
  return rc;
}

const char* svt_status_string(int code) {
  switch (code) {
    case SVT_OK: return "ok";
    case SVT_ERR_ARG: return "invalid argument";
    case SVT_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case SVT_ERR_TREE_ROOT: return "tree: parents[0] is not 0";
    case SVT_ERR_TREE_RANGE: return "tree: parent index out of [0, M] or self-parent";
    case SVT_ERR_TREE_CYCLE: return "tree: a parent chain never reaches the root";
    case SVT_ERR_CAPACITY: return "commit exceeds cache capacity";
    case SVT_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case SVT_ERR_HIP: return "HIP runtime error";
    case SVT_ERR_LENGTH: return "inconsistent sequence lengths";
    default: return "unknown status";
  }
}

const char* svt_version(void) { return "0.1.0 gfx950"; }

}  // extern "C"
