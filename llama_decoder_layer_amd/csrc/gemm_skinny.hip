// Weight-streaming projections for few tokens (decode: M <= 128 rows of x).
//
// Same product as gemm.hip, y = x W^T with W stored [out, in] (vllm-learning
// page "模型库与算子层 — 代码走读", section "Linear 层"), but here every
// weight byte is used by at most 64 tokens, so the kernel is bound by
// streaming W from HBM once.  Design:
//   * a workgroup owns NW waves x NT 16-row tiles of W and one K range
//     (split-K across workgroups when W has few rows, so that enough
//     workgroups stream concurrently).  NW is 4 or 5, chosen so that the
//     workgroup count is a multiple of the CU count, or 7 when 7-wave
//     workgroups tile a tall weight exactly onto the CUs (57344 rows = 256
//     CUs x 7 waves x 32 rows): no partly empty last round;
//   * the x slice of the current K chunk (M x KC) is staged once per
//     workgroup in XOR-swizzled LDS and shared by its waves, so global
//     memory traffic is W plus a small fraction of x;
//   * W fragments are loaded straight from global memory into MFMA operand
//     registers (A = W rows, 16-byte loads, 64 contiguous bytes per row per
//     instruction), one full chunk ahead of the MFMAs that use them, with
//     the nontemporal hint (each weight byte is read once per step);
//   * v_mfma_f32_16x16x32_bf16 computes D[n][m] = W[n,:] . x[m,:]; a lane
//     ends with four consecutive output features of one token.
// Epilogues: bf16 store, residual add (in place), SiluAndMul on the re-ordered
// gate_up weight (each 32-row group = 16 gate rows then 16 up rows), or fp32
// partial sums [split][M][N] that the consumer reduces in split order
// (deterministic: no atomics).
#include "common.h"
#include "kernels.h"

namespace llk {
namespace {


__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + expf(-g)); }

template <int MT, int NT, int KC, int NW, int EPI>
__global__ __launch_bounds__(NW * 64) void gemm_skinny_bf16(const bf16* __restrict__ X, int M,
                                                             const bf16* __restrict__ W, int K, int kps,
                                                             WStride ws, void* __restrict__ out, int N) {
  constexpr int SPC = KC / 32;          // MFMA k-steps per chunk
  constexpr int XR = MT * 16;           // token rows staged
  constexpr int XCH = XR * KC / 8;      // 16-byte pieces of the x chunk
  constexpr int kThreads = NW * 64;
  constexpr int XPT = (XCH + kThreads - 1) / kThreads;
  __shared__ __attribute__((aligned(16))) bf16 sx[2][XR * KC];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int n0 = (blockIdx.x * NW + wave) * NT * 16;  // this wave's first weight row
  const int k0 = blockIdx.y * kps;
  const int nchunk = kps / KC;

  auto xaddr = [](int row, int c) { return row * KC + ((c ^ (row & 7)) << 3); };
  const bf16x8 zero8 = {};
  bf16x8 xs[XPT];
  auto xload = [&](int kc) {
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
      const int id = threadIdx.x + kThreads * j;
      const int row = id / (KC / 8), c = id % (KC / 8);
      xs[j] = (id < XCH && row < M) ? ld16<bf16x8>(X + (size_t)row * K + k0 + kc + c * 8) : zero8;
    }
  };
  auto xstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < XPT; ++j) {
      const int id = threadIdx.x + kThreads * j;
      const int row = id / (KC / 8), c = id % (KC / 8);
      if (id < XCH) *reinterpret_cast<bf16x8*>(&sx[buf][xaddr(row, c)]) = xs[j];
    }
  };

  // lane (r16, g) reads row r16 of each 16-row strip, k-slots 8g .. 8g+7 of
  // every 32-wide k block (the layout's strides place both)
  const bf16* wr[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
    wr[t] = W + (size_t)(n0 + 16 * t) * K + (size_t)r16 * ws.rs + (size_t)(k0 / 32) * ws.ks + g * 8;
  bf16x8 wn[SPC][NT];
  auto wload = [&](int kc) {
#pragma unroll
    for (int s = 0; s < SPC; ++s)
#pragma unroll
      for (int t = 0; t < NT; ++t) wn[s][t] = ld16_nt<bf16x8>(wr[t] + (size_t)(kc / 32 + s) * ws.ks);
  };

  f32x4 acc[NT][MT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int u = 0; u < MT; ++u) acc[t][u] = f32x4{0.f, 0.f, 0.f, 0.f};

  wload(0);
  xload(0);
  xstore(0);
  __syncthreads();
  for (int c = 0; c < nchunk; ++c) {
    bf16x8 wc[SPC][NT];
#pragma unroll
    for (int s = 0; s < SPC; ++s)
#pragma unroll
      for (int t = 0; t < NT; ++t) wc[s][t] = wn[s][t];
    if (c + 1 < nchunk) {
      wload((c + 1) * KC);
      xload((c + 1) * KC);
    }
#pragma unroll
    for (int s = 0; s < SPC; ++s) {
      bf16x8 xf[MT];
#pragma unroll
      for (int u = 0; u < MT; ++u)
        xf[u] = *reinterpret_cast<const bf16x8*>(&sx[c & 1][xaddr(16 * u + r16, s * 4 + g)]);
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int u = 0; u < MT; ++u) acc[t][u] = mfma16(wc[s][t], xf[u], acc[t][u]);
    }
    if (c + 1 < nchunk) xstore((c + 1) & 1);
    __syncthreads();
  }

  // lane holds features n0 + 16t + 4g + (0..3) of token 16u + r16
#pragma unroll
  for (int u = 0; u < MT; ++u) {
    const int m = 16 * u + r16;
    if (m >= M) continue;
    if (EPI == kEpiPartial) {
      float* dst = reinterpret_cast<float*>(out) + ((size_t)blockIdx.y * M + m) * N;
#pragma unroll
      for (int t = 0; t < NT; ++t) *reinterpret_cast<f32x4*>(dst + n0 + 16 * t + 4 * g) = acc[t][u];
    } else if (EPI == kEpiSiluMul) {
      bf16* dst = reinterpret_cast<bf16*>(out) + (size_t)m * N;
#pragma unroll
      for (int t = 0; t < NT; t += 2) {
        const int f = ((n0 + 16 * t) >> 5) * 16 + 4 * g;
        bf16x4 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = static_cast<bf16>(silu_f(acc[t][u][r]) * acc[t + 1][u][r]);
        *reinterpret_cast<bf16x4*>(dst + f) = o;
      }
    } else {
      bf16* dst = reinterpret_cast<bf16*>(out) + (size_t)m * N;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        bf16x4* p = reinterpret_cast<bf16x4*>(dst + n0 + 16 * t + 4 * g);
        bf16x4 o;
        if (EPI == kEpiAdd) {
          const bf16x4 prev = *p;
#pragma unroll
          for (int r = 0; r < 4; ++r) o[r] = static_cast<bf16>(acc[t][u][r] + static_cast<float>(prev[r]));
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) o[r] = static_cast<bf16>(acc[t][u][r]);
        }
        *p = o;
      }
    }
  }
}

// out[m][n] = bf16(sum over splits of part[s][m][n]), four features per thread
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int S, int M, int N,
                                                            bf16* __restrict__ out) {
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  const size_t total = (size_t)M * N;
  if (i >= total) return;
  f32x4 a = *reinterpret_cast<const f32x4*>(part + i);
  for (int s = 1; s < S; ++s) {
    const f32x4 b = *reinterpret_cast<const f32x4*>(part + (size_t)s * total + i);
#pragma unroll
    for (int r = 0; r < 4; ++r) a[r] += b[r];
  }
  bf16x4 o;
#pragma unroll
  for (int r = 0; r < 4; ++r) o[r] = static_cast<bf16>(a[r]);
  *reinterpret_cast<bf16x4*>(out + i) = o;
}

// In-workgroup split-K for weights of many rows and a short K (o_proj and
// down_proj of one GPU's tensor-parallel share of the 70B layer: 8192 rows =
// 256 CUs x 32, K = 1024 and 3584): a workgroup of kWaveSplit waves
// owns 32 weight rows, each wave one K slice, with both operands loaded
// straight into MFMA registers one chunk ahead (x rows come from L2).  The
// waves' sums are added in wave order through LDS and wave 0 writes the
// final rows (plain store or residual add): no fp32 partial planes and no
// separate reduce.
constexpr int kWaveSplit = 8;
constexpr int kWsRows = 32;
constexpr int kWsKc = 64;
template <int MT, int EPI>
__global__ __launch_bounds__(kWaveSplit * 64) void gemm_skinny_wsplit(const bf16* __restrict__ X, int M,
                                                                      const bf16* __restrict__ W, int K,
                                                                      WStride ws, bf16* __restrict__ out, int N) {
  constexpr int NT = kWsRows / 16, SPC = kWsKc / 32;
  __shared__ f32x4 red[kWaveSplit - 1][NT * MT][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * kWsRows;
  const int kslice = K / kWaveSplit;
  const int k0 = wave * kslice;
  const int nchunk = kslice / kWsKc;

  const bf16* wr[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
    wr[t] = W + (size_t)(n0 + 16 * t) * K + (size_t)r16 * ws.rs + (size_t)(k0 / 32) * ws.ks + g * 8;
  const bf16* xr[MT];  // rows past M read row M-1; their outputs are never stored
#pragma unroll
  for (int u = 0; u < MT; ++u) xr[u] = X + (size_t)min(16 * u + r16, M - 1) * K + k0 + g * 8;
  bf16x8 wn[SPC][NT], xn[SPC][MT];
  auto load = [&](int kc) {
#pragma unroll
    for (int s = 0; s < SPC; ++s) {
#pragma unroll
      for (int t = 0; t < NT; ++t) wn[s][t] = ld16_nt<bf16x8>(wr[t] + (size_t)(kc / 32 + s) * ws.ks);
#pragma unroll
      for (int u = 0; u < MT; ++u) xn[s][u] = ld16<bf16x8>(xr[u] + kc + 32 * s);
    }
  };

  f32x4 acc[NT][MT];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int u = 0; u < MT; ++u) acc[t][u] = f32x4{0.f, 0.f, 0.f, 0.f};
  load(0);
  for (int c = 0; c < nchunk; ++c) {
    bf16x8 wc[SPC][NT], xc[SPC][MT];
#pragma unroll
    for (int s = 0; s < SPC; ++s) {
#pragma unroll
      for (int t = 0; t < NT; ++t) wc[s][t] = wn[s][t];
#pragma unroll
      for (int u = 0; u < MT; ++u) xc[s][u] = xn[s][u];
    }
    if (c + 1 < nchunk) load((c + 1) * kWsKc);
#pragma unroll
    for (int s = 0; s < SPC; ++s)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int u = 0; u < MT; ++u) acc[t][u] = mfma16(wc[s][t], xc[s][u], acc[t][u]);
  }

  if (wave > 0) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int u = 0; u < MT; ++u) red[wave - 1][t * MT + u][lane] = acc[t][u];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < kWaveSplit - 1; ++w)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int u = 0; u < MT; ++u) {
        const f32x4 v = red[w][t * MT + u][lane];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[t][u][r] += v[r];
      }

  // lane holds features n0 + 16t + 4g + (0..3) of token 16u + r16
#pragma unroll
  for (int u = 0; u < MT; ++u) {
    const int m = 16 * u + r16;
    if (m >= M) continue;
    bf16* dst = out + (size_t)m * N;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      bf16x4* p = reinterpret_cast<bf16x4*>(dst + n0 + 16 * t + 4 * g);
      bf16x4 o;
      if (EPI == kEpiAdd) {
        const bf16x4 prev = *p;
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = static_cast<bf16>(acc[t][u][r] + static_cast<float>(prev[r]));
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = static_cast<bf16>(acc[t][u][r]);
      }
      *p = o;
    }
  }
}

template <int MT>
hipError_t launch_wsplit(const bf16* x, int M, const bf16* w, int K, WStride ws, int epi, bf16* out, int N,
                         hipStream_t s) {
  const dim3 grid(N / kWsRows);
  if (epi == kEpiAdd)
    gemm_skinny_wsplit<MT, kEpiAdd><<<grid, kWaveSplit * 64, 0, s>>>(x, M, w, K, ws, out, N);
  else
    gemm_skinny_wsplit<MT, kEpiStore><<<grid, kWaveSplit * 64, 0, s>>>(x, M, w, K, ws, out, N);
  return hipGetLastError();
}

template <int MT, int NT, int KC, int NW>
hipError_t launch3(const bf16* x, int M, const bf16* w, int K, int kps, WStride ws, int epi, void* out, int N,
                   dim3 grid, hipStream_t s) {
  switch (epi) {
    case kEpiStore:
      gemm_skinny_bf16<MT, NT, KC, NW, kEpiStore><<<grid, NW * 64, 0, s>>>(x, M, w, K, kps, ws, out, N);
      break;
    case kEpiAdd:
      gemm_skinny_bf16<MT, NT, KC, NW, kEpiAdd><<<grid, NW * 64, 0, s>>>(x, M, w, K, kps, ws, out, N);
      break;
    case kEpiSiluMul:
      gemm_skinny_bf16<MT, NT, KC, NW, kEpiSiluMul><<<grid, NW * 64, 0, s>>>(x, M, w, K, kps, ws, out, N);
      break;
    default:
      gemm_skinny_bf16<MT, NT, KC, NW, kEpiPartial><<<grid, NW * 64, 0, s>>>(x, M, w, K, kps, ws, out, N);
  }
  return hipGetLastError();
}

// The instantiated (MT, NT, KC, NW) shapes; skinny_plan only returns these.
#define LLK_SKINNY_SHAPES(X)                                                                        \
  X(1, 2, 64, 4) X(1, 2, 128, 4) X(1, 2, 256, 4) X(1, 2, 256, 7)                                   \
  X(2, 2, 64, 4) X(2, 2, 128, 4) X(2, 2, 256, 4) X(2, 2, 64, 5) X(2, 2, 256, 7) X(2, 4, 256, 4)  \
  X(4, 2, 64, 4) X(4, 2, 128, 4) X(4, 2, 256, 4) X(4, 1, 128, 5) X(4, 2, 256, 7)                   \
  X(8, 2, 64, 4) X(8, 2, 128, 4) X(8, 1, 128, 5) X(8, 2, 128, 7)

hipError_t launch_shape(const SkinnyPlan& p, const bf16* x, int M, const bf16* w, int K, int kps, WStride ws,
                        int epi, void* out, int N, dim3 grid, hipStream_t s) {
#define LLK_SKINNY_CASE(MT, NT, KC, NW)                      \
  if (p.mt == MT && p.nt == NT && p.kc == KC && p.nw == NW) \
    return launch3<MT, NT, KC, NW>(x, M, w, K, kps, ws, epi, out, N, grid, s);
  LLK_SKINNY_SHAPES(LLK_SKINNY_CASE)
#undef LLK_SKINNY_CASE
  return hipErrorInvalidValue;
}

}  // namespace

SkinnyPlan skinny_plan(int M, int wrows, int K, bool allow_split, int num_cus) {
  SkinnyPlan p;
  p.mt = M <= 16 ? 1 : (M <= 32 ? 2 : (M <= 64 ? 4 : 8));
  p.nt = 2;
  p.nw = 4;
  p.splits = 1;
  // Tall weights (gate_up of the 70B shape): no split.  One workgroup per CU
  // with 7 waves of 32 rows when that tiles the rows exactly onto the CUs
  // (no tail round); else 4 waves of 64 (32 for M > 32) rows.
  const int rows7 = 7 * 32;
  if (wrows >= 49152 && K % 256 == 0) {
    if (num_cus > 0 && wrows % rows7 == 0 && (wrows / rows7) % num_cus == 0) {
      p.nw = 7;
    } else if (p.mt == 2 && wrows % 256 == 0) {
      p.nt = 4;
    }
    p.kc = p.mt == 8 ? 128 : 256;  // 8 token tiles: the x chunk pair must fit 64 KiB of LDS
    return p;
  }
  // Split-K: the first candidate whose workgroup count is a whole multiple
  // of the CU count (every CU streams the same number of workgroups; a
  // half-filled last round costs up to a fifth of the time).  The 4-wave
  // candidate suits 8192-row weights, the 5-wave one 10240-row weights.
  // K chunks, measured on the 70B decode: 128 for the 4-wave form (32
  // tokens: o_proj 35 -> 33 us, down_proj 86 -> 84 us against 64, 256 no
  // better; 64 tokens: o_proj 37 -> 33 us, down_proj 94 -> 89 us against
  // 256), 64 for the 5-wave one at 32 tokens (qkv_proj 35 us; 37 at 128,
  // 39.5 at 256).
  if (allow_split && num_cus > 0 && p.mt >= 2) {
    struct Cand { int nt, nw, kc, splits; };
    static const Cand c2[] = {{2, 4, 128, 8}, {2, 5, 64, 8}};
    static const Cand c4[] = {{2, 4, 128, 8}, {1, 5, 128, 4}};
    static const Cand c8[] = {{2, 4, 128, 8}, {1, 5, 128, 4}};
    const Cand* c = p.mt == 2 ? c2 : (p.mt == 4 ? c4 : c8);
    for (int i = 0; i < 2; ++i) {
      const int rows = 16 * c[i].nt * c[i].nw;
      if (wrows % rows || K % (c[i].splits * c[i].kc)) continue;
      if ((wrows / rows) * c[i].splits % num_cus) continue;
      p.nt = c[i].nt;
      p.nw = c[i].nw;
      p.kc = c[i].kc;
      p.splits = c[i].splits;
      return p;
    }
  }
  const int tiles = wrows / (16 * p.nw * p.nt);
  if (allow_split && tiles < 192) {
    for (int s : {8, 4, 2})
      if (K % (s * 64) == 0) {
        p.splits = s;
        break;
      }
  }
  const int kps = K / p.splits;
  if (p.mt == 2 || p.mt == 8) p.kc = kps % 128 == 0 ? 128 : 64;
  else p.kc = kps % 256 == 0 ? 256 : (kps % 128 == 0 ? 128 : 64);
  return p;
}

hipError_t launch_skinny(const void* x, const void* w, int M, int N, int K, int epi, const SkinnyPlan& p,
                         void* out, hipStream_t s, int layout) {
  if (M <= 0) return hipSuccess;
  const int wrows = epi == kEpiSiluMul ? 2 * N : N;
  const int rows_per_wg = 16 * p.nt * p.nw;
  if (M > kSkinnyMaxM || wrows % rows_per_wg != 0 || K % (p.splits * p.kc) != 0) return hipErrorInvalidValue;
  if (epi == kEpiSiluMul && (p.splits != 1 || p.nt % 2 != 0)) return hipErrorInvalidValue;
  if (p.splits != 1 && epi != kEpiPartial) return hipErrorInvalidValue;
  if (M > 16 * p.mt || K % 32 != 0) return hipErrorInvalidValue;
  dim3 grid(wrows / rows_per_wg, p.splits);
  return launch_shape(p, (const bf16*)x, M, (const bf16*)w, K, K / p.splits, weight_stride(layout, K), epi, out,
                      N, grid, s);
}

// Only for short K: each wave then streams few bytes, and the partial planes
// and their reduce that this form saves are a large share of the time (the
// TP = 8 share's o_proj, K = 1024, and down_proj, K = 3584: decode 0.091 ->
// 0.085 ms).  For long K (the 70B o_proj, K = 8192, and down_proj, K =
// 28672) the split across workgroups streams faster: there the x chunk is
// shared through LDS by the waves, where here every wave fetches its own x
// slice from L2 (0.389 -> 0.405 ms with this form).
constexpr int kWsMaxK = 4096;
bool skinny_wave_split_ok(int M, int N, int K, int num_cus) {
  return M > 0 && M <= 64 && N % kWsRows == 0 && num_cus > 0 && N / kWsRows >= num_cus &&
         K % (kWaveSplit * kWsKc) == 0 && K <= kWsMaxK;
}

hipError_t launch_skinny_wave_split(const void* x, const void* w, int M, int N, int K, int epi, void* out,
                                    hipStream_t s, int layout) {
  if (M <= 0) return hipSuccess;
  if (M > 64 || N % kWsRows != 0 || K % (kWaveSplit * kWsKc) != 0 || (epi != kEpiStore && epi != kEpiAdd))
    return hipErrorInvalidValue;
  const WStride ws = weight_stride(layout, K);
  const bf16* xb = (const bf16*)x;
  const bf16* wb = (const bf16*)w;
  bf16* ob = (bf16*)out;
  if (M <= 16) return launch_wsplit<1>(xb, M, wb, K, ws, epi, ob, N, s);
  if (M <= 32) return launch_wsplit<2>(xb, M, wb, K, ws, epi, ob, N, s);
  return launch_wsplit<4>(xb, M, wb, K, ws, epi, ob, N, s);
}

hipError_t launch_splitk_reduce(const float* part, int S, int M, int N, void* out, hipStream_t s) {
  const size_t total = (size_t)M * N;
  if (total == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((total / 4 + 255) / 256);
  splitk_reduce_kernel<<<blocks, 256, 0, s>>>(part, S, M, N, (bf16*)out);
  return hipGetLastError();
}

}  // namespace llk
