// Row -> sequence map, prefill query-tile table and the list of single-row
// sequences (served by the decode attention kernel) of a mixed batch, built
// on the device from query_start_loc (the per-sequence query counts that
// vLLM's attention metadata carries with a paged batch: page
// "模型库与算子层 — 代码走读", vllm-learning.pages.dev, section "Attention
// 层", where the backend takes the block table and further per-call
// metadata).  Sequence b owns rows query_start_loc[b] .. query_start_loc[b+1]-1.
#include "common.h"
#include "kernels.h"

namespace llk {
namespace {

constexpr int kThreads = 1024;

// inclusive sum over the workgroup; every thread gets its prefix and the total
__device__ __forceinline__ int block_scan(int v, int* s_wave, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int u = __shfl_up(v, o, kWave);
    if (lane >= o) v += u;
  }
  if (lane == kWave - 1) s_wave[wave] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int w = 0; w < kThreads / kWave; ++w) {
      const int x = s_wave[w];
      s_wave[w] = acc;
      acc += x;
    }
    *total = acc;
  }
  __syncthreads();
  return v + s_wave[wave];
}

// last index i in [0, n) with a[i] <= x (0 if none)
__device__ __forceinline__ int last_le(const int* a, int n, int x) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a[mid] <= x) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(kThreads) void batch_map_kernel(const int* __restrict__ qsl, int B, int T, int qw,
                                                              int* __restrict__ seq_of, int4* __restrict__ tiles,
                                                              int tile_cap, int* __restrict__ ntiles,
                                                              int* __restrict__ dec, int* __restrict__ ndec) {
  __shared__ int s_row[kMaxMappedSeqs + 1];   // clamped first row of each sequence, then T
  __shared__ int s_tile[kMaxMappedSeqs + 1];  // first tile of each sequence, then the tile count
  __shared__ int s_wave[kThreads / kWave];
  __shared__ int s_total;
  const int tid = threadIdx.x;
  for (int b = tid; b < B; b += kThreads) s_row[b] = min(max(qsl[b], 0), T);
  if (tid == 0) s_row[B] = T;
  __syncthreads();
  int base = 0, dbase = 0;
  for (int c0 = 0; c0 < B; c0 += kThreads) {
    const int b = c0 + tid;
    const int rows = b < B ? max(s_row[b + 1] - s_row[b], 0) : 0;
    const bool single = dec && rows == 1;  // served by the decode kernel
    const int n = single ? 0 : (rows + qw - 1) / qw;
    const int incl = block_scan(n, s_wave, &s_total);
    if (b < B) s_tile[b] = base + incl - n;
    base += s_total;
    __syncthreads();
    if (dec) {
      const int f = single ? 1 : 0;
      const int di = block_scan(f, s_wave, &s_total) - f;
      if (single) dec[dbase + di] = s_row[b];
      dbase += s_total;
      __syncthreads();
    }
  }
  if (tid == 0) {
    s_tile[B] = base;
    if (dec) *ndec = dbase;
  }
  __syncthreads();
  const int total = min(base, tile_cap);
  if (tid == 0) *ntiles = total;
  for (int i = tid; i < total; i += kThreads) {
    const int b = last_le(s_tile, B, i);        // s_tile is non-decreasing
    const int n = s_tile[b + 1] - s_tile[b];
    const int rows = max(s_row[b + 1] - s_row[b], 0);
    tiles[i] = make_int4(b, n - 1 - (i - s_tile[b]), s_row[b], rows);
  }
  for (int t = tid; t < T; t += kThreads) {
    int b = last_le(s_row, B, t);
    if (t < s_row[b] || t >= s_row[b + 1]) b = 0;  // a row no sequence claims
    seq_of[t] = b;
  }
}

}  // namespace

hipError_t launch_batch_map(const int* query_start_loc, int B, int T, int qw, int* seq_of, int4* tiles,
                            int tile_cap, int* ntiles, int* dec, int* ndec, hipStream_t s) {
  if (B <= 0 || B > kMaxMappedSeqs || T <= 0 || qw <= 0 || (dec && !ndec)) return hipErrorInvalidValue;
  batch_map_kernel<<<1, kThreads, 0, s>>>(query_start_loc, B, T, qw, seq_of, tiles, tile_cap, ntiles, dec, ndec);
  return hipGetLastError();
}

}  // namespace llk
