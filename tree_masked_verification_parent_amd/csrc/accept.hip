// Greedy argmax over the vocabulary and longest accepted root path.
//
// Source: EAGLE-Pangu (gist.science ko summary, section 4 Results): the
// accepted length accept_L of a verification step, with teacher-only greedy
// decoding as the baseline, i.e. a draft token is correct when it equals the
// teacher's greedy token at its parent.  Index outputs are zero padded (no
// negative sentinels, section 2).
//
// Pass 1 (argmax_partial_kernel) streams the logits: the vocabulary of each
// row is cut into `nchunk` chunks, one 256-thread workgroup per (row, chunk),
// float4 loads, and each chunk reduces to one 64-bit key
//   (order-preserving bits of the value) << 32 | ~index
// so that an unsigned max picks the larger value and, on equal values, the
// lower index.  NaN maps to the largest key (first NaN wins); -0.0 maps to
// +0.0.  Keys are written to the workspace; no atomics, so the result does not
// depend on scheduling.
//
// Pass 2 (accept_kernel) is one wavefront per sequence: it reduces the chunk
// keys of each node, forms the ok bits with one ballot per 64 nodes, tests
// every node's ancestor mask against them, and picks the deepest accepted node
// (lowest index on ties) with a wave max over (depth+1) << 16 | (0xFFFF - i).
#include <mutex>

#include "svt_internal.h"

namespace svt {

// Scratch of svt_accept_noalloc: the chunk keys live in this file-scope
// device array instead of a caller workspace.  Each device the library runs
// on holds its own copy for the life of the process.  In host code the name
// `scratch` is only a host-side handle; the device address comes from
// hipGetSymbolAddress, once per device, and only that address is handed to
// kernels.
static __device__ __align__(256) unsigned char scratch[kAcceptScratchBytes];

hipError_t accept_scratch(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // with device `dev` current
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

__device__ __forceinline__ uint32_t order_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if (x != x) return 0xFFFFFFFFu;  // NaN ranks above every number
  if (u == 0x80000000u) u = 0u;    // -0.0 == +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t make_key(float x, uint32_t idx) {
  return ((uint64_t)order_bits(x) << 32) | (uint64_t)(~idx);
}

// Strictly-better test used inside one thread, which visits indices in
// increasing order: a later element wins only if it ranks strictly higher.
__device__ __forceinline__ bool beats(float x, float best) {
  return (x > best) || (x != x && best == best);
}

__global__ __launch_bounds__(256) void argmax_partial_kernel(const float* __restrict__ logits, int V,
                                                             int nchunk, int chunk, bool vec4,
                                                             uint64_t* __restrict__ part) {
  const int64_t blk = blockIdx.x;
  const int64_t row = blk / nchunk;
  const int c = (int)(blk % nchunk);
  const int lo = c * chunk;
  const int hi = min(V, lo + chunk);
  const float* x = logits + row * (int64_t)V;
  const int tid = threadIdx.x;

  float best = -__builtin_inff();
  int bidx = -1;
  if (vec4) {
    // lo is a multiple of 4 (chunk is), the row start is 16-byte aligned.
    // Four loads in flight per thread before the compares; each thread still
    // visits its indices in increasing order, so ties keep the lowest index.
    const float4* x4 = reinterpret_cast<const float4*>(x + lo);
    const int n4 = (hi - lo) >> 2;
    for (int k = tid; k < n4; k += 4 * 256) {
      float4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (k + 256 * u < n4) v[u] = x4[k + 256 * u];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (k + 256 * u >= n4) break;
        const int i0 = lo + 4 * (k + 256 * u);
        if (bidx < 0 || beats(v[u].x, best)) { best = v[u].x; bidx = i0; }
        if (beats(v[u].y, best)) { best = v[u].y; bidx = i0 + 1; }
        if (beats(v[u].z, best)) { best = v[u].z; bidx = i0 + 2; }
        if (beats(v[u].w, best)) { best = v[u].w; bidx = i0 + 3; }
      }
    }
    for (int i = lo + 4 * n4 + tid; i < hi; i += 256) {
      const float v = x[i];
      if (bidx < 0 || beats(v, best)) { best = v; bidx = i; }
    }
  } else {
    for (int i = lo + tid; i < hi; i += 256) {
      const float v = x[i];
      if (bidx < 0 || beats(v, best)) { best = v; bidx = i; }
    }
  }
  uint64_t key = bidx < 0 ? 0ull : make_key(best, (uint32_t)bidx);
  key = wave_max_u64(key);
  __shared__ uint64_t red[4];
  if (lane_id() == 0) red[tid >> 6] = key;
  __syncthreads();
  if (tid == 0) {
    uint64_t k = red[0];
    for (int w = 1; w < 4; ++w) k = red[w] > k ? red[w] : k;
    part[blk] = k;
  }
}

template <int S>
__global__ __launch_bounds__(64) void accept_kernel(const uint64_t* __restrict__ part, int nchunk,
                                                    const int32_t* __restrict__ tree_tokens,
                                                    const int32_t* __restrict__ parents,
                                                    const uint64_t* __restrict__ mask,
                                                    const int32_t* __restrict__ depth,
                                                    const int32_t* __restrict__ status, int M,
                                                    int32_t* __restrict__ amax, int32_t* __restrict__ accept_len,
                                                    int32_t* __restrict__ path, int32_t* __restrict__ bonus) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int T = M + 1;
  const int64_t base = (int64_t)b * T;

  int am[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int u = lane + 64 * s;
    am[s] = 0;
    if (u < T) {
      const uint64_t* pk = part + (base + u) * nchunk;
      uint64_t k = pk[0];
      for (int c = 1; c < nchunk; ++c) k = pk[c] > k ? pk[c] : k;
      am[s] = (int)(~(uint32_t)k);
      amax[base + u] = am[s];
    }
  }
  const int st = status ? status[b] : SVT_OK;
  if (st != SVT_OK) {
    for (int k = lane; k < T; k += 64) path[base + k] = 0;
    if (lane == 0) {
      accept_len[b] = 0;
      bonus[b] = am[0];
    }
    return;
  }

  // ok bits: node u is correct when it is the root or its token equals the
  // greedy token of its parent.
  uint64_t okw[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int u = lane + 64 * s;
    int p = u < T ? parents[base + u] : 0;
    p = (p < 0 || p >= T) ? 0 : p;  // memory safety only; valid trees never clamp
    const int src = p & 63, slot = p >> 6;
    int ap = 0;
#pragma unroll
    for (int s2 = 0; s2 < S; ++s2) {
      const int v = __shfl(am[s2], src);
      if (s2 == slot) ap = v;
    }
    const bool ok = (u < T) && (u == 0 || tree_tokens[base + u] == ap);
    okw[s] = __ballot(ok);
  }

  // accepted when the ancestor mask has no node outside the ok set
  uint64_t best = 0;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int u = lane + 64 * s;
    if (u < T) {
      const uint64_t* row = mask + (base + u) * S;
      bool acc = true;
#pragma unroll
      for (int w = 0; w < S; ++w) acc &= (row[w] & ~okw[w]) == 0;
      if (acc) {
        const uint64_t key = ((uint64_t)(depth[base + u] + 1) << 16) | (uint64_t)(0xFFFF - u);
        best = key > best ? key : best;
      }
    }
  }
  best = wave_max_u64(best);
  // The root is always accepted, so best != 0; the guard only keeps a
  // malformed mask argument from indexing outside the tree.
  const int end = best ? 0xFFFF - (int)(best & 0xFFFF) : 0;
  const int alen = best ? (int)(best >> 16) - 1 : 0;

  // path: every ancestor j of end sits at index depth[j]; the rest is 0
  uint64_t endmask[S];
#pragma unroll
  for (int w = 0; w < S; ++w) endmask[w] = mask[(base + end) * S + w];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int u = lane + 64 * s;
    if (u < T) {
      const int du = depth[base + u];
      if (((endmask[s] >> lane) & 1ull) && du >= 0 && du < T) path[base + du] = u;
      if (u > alen) path[base + u] = 0;
    }
  }
  int aend = 0;
#pragma unroll
  for (int s2 = 0; s2 < S; ++s2) {
    const int v = __shfl(am[s2], end & 63);
    if (s2 == (end >> 6)) aend = v;
  }
  if (lane == 0) {
    accept_len[b] = alen;
    bonus[b] = aend;
  }
}

hipError_t launch_accept(const svt_accept_args* a, const AcceptPlan& p, hipStream_t s) {
  uint64_t* part = static_cast<uint64_t*>(a->workspace);
  const bool vec4 = (a->V % 4 == 0) && ((reinterpret_cast<uintptr_t>(a->logits) & 15) == 0);
  const int64_t nblk = (int64_t)p.rows * p.nchunk;
  hipLaunchKernelGGL(argmax_partial_kernel, dim3((unsigned)nblk), dim3(256), 0, s, a->logits, a->V, p.nchunk,
                     p.chunk, vec4, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int T = a->M + 1;
  const int S = (T + 63) / 64;
  dim3 grid(a->B), block(64);
#define SVT_ACCEPT_ARGS part, p.nchunk, a->tree_tokens, a->parents, a->mask, a->depth, a->status, a->M, \
                        a->amax, a->accept_len, a->path, a->bonus
  switch (S) {
    case 1: hipLaunchKernelGGL(accept_kernel<1>, grid, block, 0, s, SVT_ACCEPT_ARGS); break;
    case 2: hipLaunchKernelGGL(accept_kernel<2>, grid, block, 0, s, SVT_ACCEPT_ARGS); break;
    case 3: hipLaunchKernelGGL(accept_kernel<3>, grid, block, 0, s, SVT_ACCEPT_ARGS); break;
    case 4: hipLaunchKernelGGL(accept_kernel<4>, grid, block, 0, s, SVT_ACCEPT_ARGS); break;
    default: return hipErrorInvalidValue;
  }
#undef SVT_ACCEPT_ARGS
  return hipGetLastError();
}

bool plan_accept(const svt_accept_args* a, AcceptPlan* p) {
  if (!a || a->B < 0 || a->M < 0 || a->M >= SVT_MAX_T || a->V <= 0) return false;
  const int T = a->M + 1;
  p->rows = a->B * T;
  // The fewer of: chunks of >= 4096 entries, or enough workgroups for about
  // one wave over the chip (~2048); then more chunks if needed so that none
  // exceeds 5120 entries (20 KB): with many rows the first rule alone gives a
  // few very long workgroups per row, and the last of them run alone.
  int nchunk = 1;
  if (p->rows > 0) {
    const int by_size = (a->V + 4095) / 4096;
    const int by_par = (2048 + p->rows - 1) / p->rows;
    const int by_cap = (a->V + 5119) / 5120;
    nchunk = by_size < by_par ? by_size : by_par;
    if (nchunk < by_cap) nchunk = by_cap;
    if (nchunk < 1) nchunk = 1;
  }
  int chunk = (a->V + nchunk - 1) / nchunk;
  chunk = (chunk + 3) & ~3;  // keep chunk starts 16-byte aligned
  nchunk = (a->V + chunk - 1) / chunk;
  p->nchunk = nchunk;
  p->chunk = chunk;
  p->ws_bytes = (size_t)p->rows * (size_t)nchunk * sizeof(uint64_t);
  return true;
}

}  // namespace svt
