// Dense 4D tree mask for eager (reference-mode) attention paths.
//
// Sources: EAGLE-Pangu (gist.science nl summary, section 2.C: a 4D mask tensor
// lets token k attend token j only when j is an ancestor of k; the dual-mode
// protocol keeps a reference mode with the fused attention switched off for
// debugging and invariant checks; ko summary, section 2: 4D tree attention
// mask in the teacher path, eager mode next to the performance mode).
//
// Row i of sequence b spans P prefix columns followed by T tree columns:
// prefix column c is open when it holds content (c >= P - len_b: the prefix is
// left padded to P = lmax), tree column P + j when bit j of the ancestor mask
// row i is set (j is i or one of its ancestors).  Every column of a skipped
// sequence (nonzero tree status, or len_b outside [0, P]) is closed.
//
// Grid (row, chunk of 256 output words).  The row's elements that fill whole
// 16-byte words of the output are written one word (16 / sizeof(E) elements)
// per thread and store; the few elements before the first and after the last
// such word are written one by one by the first chunk.
#include <cmath>

#include "svt_internal.h"

namespace svt {

template <typename E>
__global__ __launch_bounds__(256) void expand_mask_kernel(const uint64_t* __restrict__ mask,
                                                          const int32_t* __restrict__ status,
                                                          const int32_t* __restrict__ len, int M, int P,
                                                          E* __restrict__ out, int32_t* __restrict__ seq_status,
                                                          E open, E closed) {
  constexpr int V = 16 / sizeof(E);
  const int T = M + 1;
  const int W = (T + 63) / 64;
  const int row = blockIdx.x;
  const int b = row / T, i = row % T;
  const int L = len[b];
  const int st = status ? status[b] : SVT_OK;
  const int code = st != SVT_OK ? st : ((L >= 0 && L <= P) ? SVT_OK : SVT_ERR_LENGTH);
  const bool valid = code == SVT_OK;
  if (seq_status && i == 0 && blockIdx.y == 0 && threadIdx.x == 0) seq_status[b] = code;
  const int first = valid ? P - L : P;          // prefix columns [first, P) are open
  const int width = P + T;
  const int64_t r0 = (int64_t)row * width;
  const int lead = (int)((V - r0 % V) % V);     // elements before the first whole word
  const int nword = (width - lead) / V;
  const int tail0 = lead + nword * V;           // first element after the last whole word
  auto tree_open = [&](int j) -> bool {
    return valid && ((mask[(int64_t)row * W + (j >> 6)] >> (j & 63)) & 1ull);
  };
  auto value = [&](int c) -> E { return (c < P ? (c >= first) : tree_open(c - P)) ? open : closed; };
  const int tid = threadIdx.x;
  if (blockIdx.y == 0) {
    if (tid < lead && tid < width) out[r0 + tid] = value(tid);
    if (tid < width - tail0 && tail0 >= lead) out[r0 + tail0 + tid] = value(tail0 + tid);
  }
  const int w = blockIdx.y * 256 + tid;
  if (w >= nword) return;
  const int c0 = lead + w * V;
  union {
    E e[V];
    uint4 u;
  } v;
  if (c0 + V <= P) {  // a word inside the prefix
#pragma unroll
    for (int k = 0; k < V; ++k) v.e[k] = (c0 + k >= first) ? open : closed;
  } else {
#pragma unroll
    for (int k = 0; k < V; ++k) v.e[k] = value(c0 + k);
  }
  *reinterpret_cast<uint4*>(out + r0 + c0) = v.u;
}

hipError_t launch_expand_mask(const uint64_t* mask, const int32_t* status, const int32_t* len, int B, int M,
                              int P, void* out, int kind, int32_t* seq_status, hipStream_t s) {
  const int T = M + 1;
  const int esize = kind == SVT_MASK_ADD_FP32 ? 4 : (kind == SVT_MASK_ADD_BF16 ? 2 : 1);
  const int64_t words = ((int64_t)P + T) / (16 / esize) + 1;
  dim3 grid((unsigned)(B * T), (unsigned)((words + 255) / 256)), block(256);
  switch (kind) {
    case SVT_MASK_ADD_FP32:
      hipLaunchKernelGGL(expand_mask_kernel<float>, grid, block, 0, s, mask, status, len, M, P,
                         static_cast<float*>(out), seq_status, 0.0f, -INFINITY);
      break;
    case SVT_MASK_ADD_BF16:  // bfloat16 bits of +0 and -inf
      hipLaunchKernelGGL(expand_mask_kernel<uint16_t>, grid, block, 0, s, mask, status, len, M, P,
                         static_cast<uint16_t*>(out), seq_status, (uint16_t)0x0000, (uint16_t)0xFF80);
      break;
    default:
      hipLaunchKernelGGL(expand_mask_kernel<uint8_t>, grid, block, 0, s, mask, status, len, M, P,
                         static_cast<uint8_t*>(out), seq_status, (uint8_t)1, (uint8_t)0);
      break;
  }
  return hipGetLastError();
}

}  // namespace svt
