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
// After a split-K o_proj the kernel also finishes that projection: it sums
// the fp32 partial rows, adds the residual, rounds, stores the new residual
// and normalises it (post_attention_layernorm) in one pass.
#include "common.h"
#include "kernels.h"

namespace llk {
namespace {

constexpr int kThreads = 256;
// A batch of few rows (decode) runs kWideThreads threads per row: with one
// workgroup per row, 256 threads cannot keep enough loads in flight to
// stream the row (and its split-K partials) at a useful rate.
constexpr int kWideThreads = 1024;
constexpr int kWideMaxRows = 256;

// S > 0: the input row is the sum of S fp32 partial rows xpart[s][row][:]
// (a split-K projection's output), added in split order; with RX that sum is
// first rounded to T, exactly as if the projection had stored its output and
// this kernel read it back.  NT threads, each with at most kMaxChunks 16-byte
// chunks: H <= NT * kMaxChunks * (16 / sizeof(T)).
template <typename T, int S, int NT, bool RX>
__global__ __launch_bounds__(NT) void add_rmsnorm_kernel(const T* __restrict__ x,
                                                               const T* res,
                                                               const T* __restrict__ w, float eps,
                                                               int H, T* __restrict__ normed,
                                                               T* res_out, const float* __restrict__ xpart,
                                                               int rows) {
  using V = typename Vec16<T>::type;
  constexpr int VN = Vec16<T>::N;
  constexpr int kThreads = NT;
  constexpr int kMaxChunks = 2048 / NT;
  const int row = blockIdx.x;
  const int nchunk = H / VN;
  const size_t base = (size_t)row * H;

  float r[kMaxChunks][VN];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    const int ci = threadIdx.x + c * kThreads;
    if (ci < nchunk) {
      float xf[VN];
      V xv;
      if (S > 0) {
#pragma unroll
        for (int e = 0; e < VN; e += 4) {
          f32x4 v[S > 0 ? S : 1];
#pragma unroll
          for (int sp = 0; sp < S; ++sp)
            v[sp] = *reinterpret_cast<const f32x4*>(xpart + (size_t)sp * rows * H + base + (size_t)ci * VN + e);
          f32x4 a = v[0];
#pragma unroll
          for (int sp = 1; sp < S; ++sp)
#pragma unroll
            for (int q = 0; q < 4; ++q) a[q] += v[sp][q];
#pragma unroll
          for (int q = 0; q < 4; ++q) xf[e + q] = RX ? to_f32(from_f32<T>(a[q])) : a[q];
        }
      } else {
        xv = ld16<V>(x + base + (size_t)ci * VN);
#pragma unroll
        for (int e = 0; e < VN; ++e) xf[e] = to_f32(xv[e]);
      }
      V ov;
      if (res != nullptr) {
        V rv = ld16<V>(res + base + (size_t)ci * VN);
#pragma unroll
        for (int e = 0; e < VN; ++e) {
          T s = from_f32<T>(xf[e] + to_f32(rv[e]));
          ov[e] = s;
          r[c][e] = to_f32(s);
        }
      } else if (S > 0) {
#pragma unroll
        for (int e = 0; e < VN; ++e) {
          ov[e] = from_f32<T>(xf[e]);
          r[c][e] = to_f32(ov[e]);
        }
      } else {
        ov = xv;
#pragma unroll
        for (int e = 0; e < VN; ++e) r[c][e] = xf[e];
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
                              int rows, int hidden, void* normed, void* res_out, hipStream_t s,
                              const float* xpart, int S, bool round_part) {
  if (rows <= 0) return hipSuccess;
  if (dtype == kBF16) {
    const bf16* r = (const bf16*)res;
    const bf16* wb = (const bf16*)w;
    bf16* n = (bf16*)normed;
    bf16* ro = (bf16*)res_out;
    const bool wide = rows <= kWideMaxRows && hidden >= 8 * kWideThreads;
#define LLK_NORM_NT(SS, XX, NT, RR)                                                                      \
  add_rmsnorm_kernel<bf16, SS, NT, RR><<<rows, NT, 0, s>>>((const bf16*)(XX), r, wb, eps, hidden, n, ro, xpart, \
                                                           rows)
#define LLK_NORM_R(SS, XX, RR)                       \
  if (wide) LLK_NORM_NT(SS, XX, kWideThreads, RR); \
  else LLK_NORM_NT(SS, XX, kThreads, RR)
#define LLK_NORM(SS, XX)              \
  if (round_part) { LLK_NORM_R(SS, XX, true); } \
  else { LLK_NORM_R(SS, XX, false); }
    if (!xpart) { LLK_NORM_R(0, x, false); }
    else if (S == 1) { LLK_NORM(1, nullptr); }
    else if (S == 2) { LLK_NORM(2, nullptr); }
    else if (S == 4) { LLK_NORM(4, nullptr); }
    else if (S == 8) { LLK_NORM(8, nullptr); }
    else return hipErrorInvalidValue;
#undef LLK_NORM
#undef LLK_NORM_R
#undef LLK_NORM_NT
  } else {
    if (xpart) return hipErrorInvalidValue;
    add_rmsnorm_kernel<float, 0, kThreads, false><<<rows, kThreads, 0, s>>>(
        (const float*)x, (const float*)res, (const float*)w, eps, hidden, (float*)normed, (float*)res_out,
        nullptr, rows);
  }
  return hipGetLastError();
}

}  // namespace llk
