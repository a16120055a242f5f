// Device-side check of a forward call's per-call metadata, run only in the
// debug mode (environment variable LLAMA_DEBUG=1) before any other kernel.
//
// The paged layout of page "模型库与算子层 — 代码走读" (vllm-learning.pages.dev,
// section "Attention 层": the cache is read and written through the block
// table) and the per-call metadata the backend receives with it make the
// kernels trust three kinds of device data: block ids (the cache block of
// each 16 positions), the positions of the new tokens, and the row ranges of
// a mixed batch.  This kernel checks each of them and raises one flag per
// broken condition; the host reads the flags back and rejects the call
// before anything is written.  Every read stays inside the arrays' declared
// extents whatever they hold.
#include "common.h"
#include "kernels.h"

namespace llk {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void validate_batch_kernel(const int* __restrict__ positions, int T,
                                                                   const int* __restrict__ block_table,
                                                                   int max_blocks, const int* __restrict__ seq_lens,
                                                                   const int* __restrict__ qsl, int B,
                                                                   int num_blocks, int max_pos, int max_seq_len,
                                                                   int* __restrict__ flags) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  const int q_len = qsl ? 0 : T / B;
  if (i < B) {  // sequence i: its row range, KV length and block ids
    const int b = i;
    int s0, s1;
    if (qsl) {
      s0 = qsl[b];
      s1 = qsl[b + 1];
      if (s1 <= s0 || s0 < 0 || s1 > T || (b == 0 && s0 != 0) || (b == B - 1 && s1 != T))
        flags[kCheckRowRanges] = 1;
    } else {
      s0 = b * q_len;
      s1 = s0 + q_len;
    }
    const int sl = seq_lens[b];
    if (sl < 1 || sl > max_seq_len) {
      flags[kCheckSeqLens] = 1;
    } else {
      if (s1 - s0 > sl) flags[kCheckSeqLens] = 1;
      const int nb = min((sl + kKvBlock - 1) / kKvBlock, max_blocks);
      const int* bt = block_table + (size_t)b * max_blocks;
      for (int j = 0; j < nb; ++j) {
        const int id = bt[j];
        if (id < 0 || id >= num_blocks) {
          flags[kCheckBlockIds] = 1;
          break;
        }
      }
    }
  }
  if (i < T) {  // row i: its position against its sequence's KV length
    const int p = positions[i];
    if (p < 0 || p >= max_pos) flags[kCheckPositions] = 1;
    int b, r, n;
    if (qsl) {
      int lo = 0, hi = B - 1;  // last sequence whose first row is <= i
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (qsl[mid] <= i) lo = mid;
        else hi = mid - 1;
      }
      b = lo;
      r = i - qsl[b];
      n = qsl[b + 1] - qsl[b];
    } else {
      b = i / q_len;
      r = i % q_len;
      n = q_len;
    }
    if (p != seq_lens[b] - n + r) flags[kCheckPositions] = 1;
  }
}

}  // namespace

hipError_t launch_validate_batch(const int* positions, int T, const int* block_table, int max_blocks,
                                 const int* seq_lens, const int* query_start_loc, int B, int num_blocks, int max_pos,
                                 int max_seq_len, int* flags, hipStream_t s) {
  if (T <= 0 || B <= 0 || (!query_start_loc && T % B != 0) || max_blocks <= 0) return hipErrorInvalidValue;
  const int n = T > B ? T : B;
  validate_batch_kernel<<<(n + kThreads - 1) / kThreads, kThreads, 0, s>>>(
      positions, T, block_table, max_blocks, seq_lens, query_start_loc, B, num_blocks, max_pos, max_seq_len, flags);
  return hipGetLastError();
}

}  // namespace llk
