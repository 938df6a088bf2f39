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
// sequence (nonzero tree status, or len_b outside [0, P]) is closed.  One
// 256-thread workgroup writes a 256 * kPer column chunk of one row with
// consecutive threads on consecutive columns.
#include <cmath>

#include "svt_internal.h"

namespace svt {

constexpr int kExpandPer = 8;  // columns per thread per chunk

template <typename E>
__global__ __launch_bounds__(256) void expand_mask_kernel(const uint64_t* __restrict__ mask,
                                                          const int32_t* __restrict__ status,
                                                          const int32_t* __restrict__ len, int M, int P,
                                                          E* __restrict__ out, int32_t* __restrict__ seq_status,
                                                          E open, E closed) {
  const int T = M + 1;
  const int W = (T + 63) / 64;
  const int row = blockIdx.y;
  const int b = row / T, i = row % T;
  const int L = len[b];
  const int st = status ? status[b] : SVT_OK;
  const int code = st != SVT_OK ? st : ((L >= 0 && L <= P) ? SVT_OK : SVT_ERR_LENGTH);
  const bool valid = code == SVT_OK;
  if (seq_status && blockIdx.x == 0 && i == 0 && threadIdx.x == 0) seq_status[b] = code;
  uint64_t words[4] = {0ull, 0ull, 0ull, 0ull};
  for (int w = 0; w < W; ++w) words[w] = valid ? mask[(int64_t)row * W + w] : 0ull;
  const int64_t width = (int64_t)P + T;
  E* orow = out + (int64_t)row * width;
  const int first = P - L;
  const int64_t c0 = (int64_t)blockIdx.x * 256 * kExpandPer + threadIdx.x;
#pragma unroll
  for (int k = 0; k < kExpandPer; ++k) {
    const int64_t c = c0 + 256 * k;
    if (c >= width) break;
    bool ok;
    if (c < P) {
      ok = valid && c >= first;
    } else {
      const int j = (int)(c - P);
      ok = (words[j >> 6] >> (j & 63)) & 1ull;
    }
    orow[c] = ok ? open : closed;
  }
}

hipError_t launch_expand_mask(const uint64_t* mask, const int32_t* status, const int32_t* len, int B, int M,
                              int P, void* out, int kind, int32_t* seq_status, hipStream_t s) {
  const int T = M + 1;
  const int64_t width = (int64_t)P + T;
  const int64_t chunks = (width + 256 * kExpandPer - 1) / (256 * kExpandPer);
  dim3 grid((unsigned)chunks, (unsigned)(B * T)), block(256);
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
