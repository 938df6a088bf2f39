// Internal declarations shared by the HIP translation units of libsvt.
// Kernels target gfx950 (CDNA4) only: 64-lane wavefronts, 160 KB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "svt.h"

namespace svt {

constexpr int kWave = 64;
constexpr int kStreamMaxBatch = 1024;  // largest batch of the stream attention form

// ---- launch plans (host side), shared by the workspace query and the launch ----
struct AttnPlan {
  int T, G, R;       // tree rows, query heads per KV head, query rows per KV head (G*T)
  int nqt;           // 16-row query tiles per KV head
  int wide;          // bf16: 1 = stream form (one workgroup per CU over the tile stream)
  int grid;          // stream form: workgroups (compute units)
  int rpu;           // stream form: ranges per unit when grid is a whole number of them per unit, else 0
  int qw;            // query tiles per wave (bf16 path)
  int stages;        // LDS ring depth, 2 or 4 (bf16 path)
  int nw;            // waves per workgroup (bf16 path)
  int nwk;           // waves splitting each key tile (1 or 2; bf16 path)
  int qb_rows;       // query rows per workgroup
  int nqb;           // query blocks per KV head
  int kc;            // prefix keys per split (multiple of 64)
  int ns;            // splits in the grid (upper bound; device len decides the rest)
  int piece_cost;    // stream form: key tiles' worth of time a unit's set-up and output cost
  size_t ws_bytes;   // workspace bytes
};
bool plan_attention(const svt_attn_args* a, AttnPlan* p);

struct AcceptPlan {
  int rows, nchunk, chunk;
  size_t ws_bytes;
};
bool plan_accept(const svt_accept_args* a, AcceptPlan* p);

// Static device scratch of svt_accept_noalloc (accept.hip): its size, and its
// device address on the current device (resolved once per device).
constexpr size_t kAcceptScratchBytes = SVT_ACCEPT_NOALLOC_SCRATCH;
hipError_t accept_scratch(void** out);

// ---- launchers (defined next to their kernels); return hipError_t ----
hipError_t launch_build_mask(const int32_t* parents, int B, int M, uint64_t* mask, int32_t* depth,
                             int32_t* status, hipStream_t s);
hipError_t launch_attention(const svt_attn_args* a, const AttnPlan& p, hipStream_t s);
hipError_t launch_accept(const svt_accept_args* a, const AcceptPlan& p, hipStream_t s);
hipError_t launch_commit(const svt_commit_args* a, hipStream_t s);
hipError_t launch_realign(const svt_realign_args* a, hipStream_t s);
hipError_t launch_expand_mask(const uint64_t* mask, const int32_t* status, const int32_t* len, int B, int M,
                              int P, void* out, int kind, int32_t* seq_status, hipStream_t s);
hipError_t launch_commit_length(const svt_commit_args* a, hipStream_t s);

// ---- host-only scheduling (pool.cpp) ----
int pool_pick(const int32_t* end, const int32_t* active, int n_slots, int max_batch, int min_group,
              int32_t* slots, int32_t* n_out);

// ---- small device helpers ----
__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
  uint32_t lo = __shfl((int)(uint32_t)v, src);
  uint32_t hi = __shfl((int)(uint32_t)(v >> 32), src);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  for (int o = 32; o > 0; o >>= 1) {
    uint32_t lo = __shfl_xor((int)(uint32_t)v, o);
    uint32_t hi = __shfl_xor((int)(uint32_t)(v >> 32), o);
    uint64_t w = ((uint64_t)hi << 32) | lo;
    v = w > v ? w : v;
  }
  return v;
}

}  // namespace svt
