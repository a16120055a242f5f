// A read-only streaming kernel: the measured HBM read ceiling that the
// weight- and KV-streaming kernels of the decode path are compared against.
// It reads the same bytes the way they do -- each workgroup one contiguous
// region, 16-byte loads, several in flight per lane, with or without the
// nontemporal hint -- and does nothing else with them but fold them into one
// word per lane, so that its time is the memory system's alone.
#include "common.h"
#include "kernels.h"

namespace llk {
namespace {

constexpr int kUnroll = 8;

// NT: the loads carry the nontemporal hint (as the decode path's weight and
// KV streams do)
template <bool NT>
__global__ void stream_read_kernel(const uint4* __restrict__ src, size_t n16, unsigned* __restrict__ sink) {
  const size_t per_wg = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t begin = (size_t)blockIdx.x * per_wg;
  const size_t end = begin + per_wg < n16 ? begin + per_wg : n16;
  unsigned acc = 0;
  size_t i = begin + threadIdx.x;
  const size_t step = blockDim.x;
  for (; i + (kUnroll - 1) * step < end; i += kUnroll * step) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = NT ? ld16_nt<uint4>(&src[i + u * step]) : src[i + u * step];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < end; i += step) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// The same reads gathered by block: workgroup w takes a contiguous range of
// the id list and reads each listed block of blockDim.x 16-byte words (one
// word per thread), kUnroll blocks in flight -- the access pattern of the
// decode attention over a paged cache whose blocks sit in random order.
template <bool NT>
__global__ void block_read_kernel(const uint4* __restrict__ src, const int* __restrict__ ids, int n,
                                  unsigned* __restrict__ sink) {
  const int per = (n + (int)gridDim.x - 1) / (int)gridDim.x;
  const int b0 = (int)blockIdx.x * per;
  const int b1 = b0 + per < n ? b0 + per : n;
  const size_t words = blockDim.x;
  unsigned acc = 0;
  for (int b = b0; b < b1; b += kUnroll) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      v[u] = uint4{0u, 0u, 0u, 0u};
      if (b + u < b1) {
        const uint4* p = &src[(size_t)ids[b + u] * words + threadIdx.x];
        v[u] = NT ? ld16_nt<uint4>(p) : *p;
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

}  // namespace

hipError_t launch_block_read(const void* src, const int* ids, int n, int block_bytes, int workgroups, void* sink,
                             bool nontemporal, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int threads = block_bytes / 16;
  if (nontemporal)
    block_read_kernel<true><<<workgroups, threads, 0, s>>>((const uint4*)src, ids, n, (unsigned*)sink);
  else
    block_read_kernel<false><<<workgroups, threads, 0, s>>>((const uint4*)src, ids, n, (unsigned*)sink);
  return hipGetLastError();
}

hipError_t launch_stream_read(const void* src, size_t bytes, int workgroups, int threads, void* sink,
                              bool nontemporal, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  if (nontemporal)
    stream_read_kernel<true><<<workgroups, threads, 0, s>>>((const uint4*)src, bytes / 16, (unsigned*)sink);
  else
    stream_read_kernel<false><<<workgroups, threads, 0, s>>>((const uint4*)src, bytes / 16, (unsigned*)sink);
  return hipGetLastError();
}

}  // namespace llk
