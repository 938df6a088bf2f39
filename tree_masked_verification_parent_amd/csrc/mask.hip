// Tree validation + ancestor bitmasks by pointer jumping, one wavefront per tree.
//
// Sources: EAGLE-Pangu (gist.science ko summary, section 2 Methodology: dummy
// root row 0, every parent index in [0, M], structural checks before the fused
// kernels; the tree attention mask admits v for u only when v is an ancestor of
// u); the nl summary, sections 2.B (ancestor tables with safe indices, invariant
// checks) and 2.C (4D tree mask).
//
// Layout in registers: lane l owns nodes u = l + 64*s for s < S = ceil(T/64).
// For each owned node it keeps up (a pointer to an ancestor), dist (edges to
// that ancestor) and the S-word ancestor set seen so far.  Round k replaces
// (set, dist, up) of u by (set(u) | set(up), dist(u) + dist(up), up(up)), so
// after k rounds a node's set holds its ancestors at distance < 2^k.  Row 0
// points at itself, so chains that reached the root stay there.  With
// 2^k >= T > M every acyclic chain has reached row 0; a node whose pointer is
// not 0 afterwards lies on or above a cycle.
#include "svt_internal.h"

namespace svt {

template <int S>
__global__ __launch_bounds__(64) void build_mask_kernel(const int32_t* __restrict__ parents, int M,
                                                        uint64_t* __restrict__ mask,
                                                        int32_t* __restrict__ depth,
                                                        int32_t* __restrict__ status) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int T = M + 1;
  const int32_t* par = parents + (int64_t)b * T;

  int up[S], dist[S];
  uint64_t set[S][S];
  bool bad_root = false, bad_range = false;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int u = lane + 64 * s;
    const bool valid = u < T;
    const int p = valid ? par[u] : 0;
    if (u == 0) bad_root = (p != 0);
    else if (valid) bad_range |= (p < 0 || p > M || p == u);
    up[s] = (valid && u != 0) ? p : 0;
    dist[s] = (valid && u != 0) ? 1 : 0;
#pragma unroll
    for (int w = 0; w < S; ++w) set[s][w] = (valid && w == s) ? (1ull << lane) : 0ull;
  }
  int code = SVT_OK;
  if (__any(bad_root)) code = SVT_ERR_TREE_ROOT;
  else if (__any(bad_range)) code = SVT_ERR_TREE_RANGE;

  if (code == SVT_OK) {
    int rounds = 0;
    while ((1 << rounds) < T) ++rounds;
    for (int r = 0; r < rounds; ++r) {
      int nup[S], ndist[S];
      uint64_t nset[S][S];
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const int t = up[s];
        const int src = t & 63, slot = t >> 6;
        int gu = 0, gd = 0;
        uint64_t gset[S];
#pragma unroll
        for (int w = 0; w < S; ++w) gset[w] = 0;
#pragma unroll
        for (int s2 = 0; s2 < S; ++s2) {
          const int vu = __shfl(up[s2], src);
          const int vd = __shfl(dist[s2], src);
          if (s2 == slot) { gu = vu; gd = vd; }
#pragma unroll
          for (int w = 0; w < S; ++w) {
            const uint64_t vs = shfl_u64(set[s2][w], src);
            if (s2 == slot) gset[w] = vs;
          }
        }
        nup[s] = gu;
        ndist[s] = dist[s] + gd;
#pragma unroll
        for (int w = 0; w < S; ++w) nset[s][w] = set[s][w] | gset[w];
      }
#pragma unroll
      for (int s = 0; s < S; ++s) {
        up[s] = nup[s];
        dist[s] = ndist[s];
#pragma unroll
        for (int w = 0; w < S; ++w) set[s][w] = nset[s][w];
      }
    }
    bool cyc = false;
#pragma unroll
    for (int s = 0; s < S; ++s) cyc |= (lane + 64 * s < T) && up[s] != 0;
    if (__any(cyc)) code = SVT_ERR_TREE_CYCLE;
  }

  const bool ok = code == SVT_OK;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int u = lane + 64 * s;
    if (u < T) {
      uint64_t* row = mask + ((int64_t)b * T + u) * S;
#pragma unroll
      for (int w = 0; w < S; ++w) row[w] = ok ? set[s][w] : 0ull;
      depth[(int64_t)b * T + u] = ok ? dist[s] : 0;
    }
  }
  if (lane == 0) status[b] = code;
}

hipError_t launch_build_mask(const int32_t* parents, int B, int M, uint64_t* mask, int32_t* depth,
                             int32_t* status, hipStream_t s) {
  const int T = M + 1;
  const int S = (T + 63) / 64;
  dim3 grid(B), block(64);
  switch (S) {
    case 1: hipLaunchKernelGGL(build_mask_kernel<1>, grid, block, 0, s, parents, M, mask, depth, status); break;
    case 2: hipLaunchKernelGGL(build_mask_kernel<2>, grid, block, 0, s, parents, M, mask, depth, status); break;
    case 3: hipLaunchKernelGGL(build_mask_kernel<3>, grid, block, 0, s, parents, M, mask, depth, status); break;
    case 4: hipLaunchKernelGGL(build_mask_kernel<4>, grid, block, 0, s, parents, M, mask, depth, status); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace svt
