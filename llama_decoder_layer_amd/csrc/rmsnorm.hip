// RMSNorm with the residual add fused in (input_layernorm and
// post_attention_layernorm).
//
// Follows page "LLama" (hotelren.com/news/2693952), section
// "3 input_layernorm (RMSNorm)": with no incoming residual the input itself is
// the new residual; otherwise input + residual is.  The normalised value is
// r / sqrt(mean(r^2) + eps) * w.  The sum is formed in fp32, rounded to the
// layer dtype and stored; the norm is taken of the stored (rounded) value, so
// the returned hidden state is a function of the returned residual.
//
// HBM-bound: one workgroup per row, 16-byte loads, the row kept in registers
// between the reduction and the scaling, a wave-shuffle then LDS reduction.
#include "common.h"
#include "kernels.h"

namespace llk {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxChunks = 8;  // 16-byte chunks per thread -> H <= 256*8*VEC

template <typename T>
__global__ __launch_bounds__(kThreads) void add_rmsnorm_kernel(const T* __restrict__ x,
                                                               const T* __restrict__ res,
                                                               const T* __restrict__ w, float eps,
                                                               int H, T* __restrict__ normed,
                                                               T* res_out) {
  using V = typename Vec16<T>::type;
  constexpr int VN = Vec16<T>::N;
  const int row = blockIdx.x;
  const int nchunk = H / VN;
  const size_t base = (size_t)row * H;

  float r[kMaxChunks][VN];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    const int ci = threadIdx.x + c * kThreads;
    if (ci < nchunk) {
      V xv = ld16<V>(x + base + (size_t)ci * VN);
      V ov;
      if (res != nullptr) {
        V rv = ld16<V>(res + base + (size_t)ci * VN);
#pragma unroll
        for (int e = 0; e < VN; ++e) {
          T s = from_f32<T>(to_f32(xv[e]) + to_f32(rv[e]));
          ov[e] = s;
          r[c][e] = to_f32(s);
        }
      } else {
        ov = xv;
#pragma unroll
        for (int e = 0; e < VN; ++e) r[c][e] = to_f32(xv[e]);
      }
      if (res_out != nullptr) *reinterpret_cast<V*>(res_out + base + (size_t)ci * VN) = ov;
#pragma unroll
      for (int e = 0; e < VN; ++e) ss = fmaf(r[c][e], r[c][e], ss);
    }
  }

  __shared__ float red[kThreads / kWave];
  ss = wave_sum(ss);
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < kThreads / kWave; ++i) tot += red[i];
  const float inv = 1.0f / sqrtf(tot / (float)H + eps);

#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    const int ci = threadIdx.x + c * kThreads;
    if (ci < nchunk) {
      V wv = ld16<V>(w + (size_t)ci * VN);
      V ov;
#pragma unroll
      for (int e = 0; e < VN; ++e) ov[e] = from_f32<T>(r[c][e] * inv * to_f32(wv[e]));
      *reinterpret_cast<V*>(normed + base + (size_t)ci * VN) = ov;
    }
  }
}

}  // namespace

hipError_t launch_add_rmsnorm(int dtype, const void* x, const void* res, const void* w, float eps,
                              int rows, int hidden, void* normed, void* res_out, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (dtype == kBF16) {
    add_rmsnorm_kernel<bf16><<<rows, kThreads, 0, s>>>(
        (const bf16*)x, (const bf16*)res, (const bf16*)w, eps, hidden, (bf16*)normed, (bf16*)res_out);
  } else {
    add_rmsnorm_kernel<float><<<rows, kThreads, 0, s>>>(
        (const float*)x, (const float*)res, (const float*)w, eps, hidden, (float*)normed,
        (float*)res_out);
  }
  return hipGetLastError();
}

}  // namespace llk
