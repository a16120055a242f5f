// Dense projections of the layer: qkv_proj, o_proj, gate_up_proj, down_proj.
//
// Every projection is y = x W^T with W stored [out, in] (vllm-learning page
// "模型库与算子层 — 代码走读", section "Linear 层": F.linear).  Epilogues fuse
// what follows the projection in the layer:
//   add       -- o_proj's output joins the residual stream (the add of
//                post_attention_layernorm, page "LLama", hotelren.com/news/2693952)
//   silu_mul  -- SiluAndMul after gate_up_proj: silu(x[:d]) * x[d:] of the
//                merged output ("LLama" page, section "LlamaMLP")
//
// bf16 kernels use v_mfma_f32_16x16x32_bf16 with fp32 accumulation and are
// written in the transposed orientation D[n][m] = W[n,:] . X[m,:]: W rows are
// the MFMA's A operand, token rows its B operand.  Both operands are K-major
// in memory, so a lane's 8-element operand slice is one 16-byte load, and an
// output lane holds four consecutive output features of one token (one
// 8-byte store).  Within one MFMA the k index a lane supplies only has to
// agree between A and B, which lets the loads be laid out for coalescing.
//
//   skinny kernel (M <= 128 tokens, decode): gemm_skinny.hip.
//   tiled kernel (prefill): 256 (or 192) tokens x 256 weight rows per
//     workgroup with 8 waves (128 KiB of LDS), or 128 x 128 with 4 waves
//     for fewer than 256 tokens; tile height and split-K from a measured
//     cost model (tile_plan); K in steps of 64 loaded straight from global
//     memory into double-buffered, XOR-swizzled LDS; XCD-grouped tile order.
//   fp32 kernel: plain LDS-tiled FMA kernel for fp32 layers.
//
// SiluAndMul layout: the bf16 gate_up weight is re-ordered once (in create)
// so that each 32-row group holds 16 gate rows then the 16 matching up rows;
// a lane then holds gate and up of the same four features.
#include "common.h"
#include "kernels.h"

namespace llk {
namespace {

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + expf(-g)); }

// Store four consecutive features n..n+3 of token m (tiled kernel).
template <int EPI>
__device__ __forceinline__ void store4(bf16* out, size_t idx, const float v[4]) {
  bf16x4 o;
  if (EPI == kEpiAdd) {
    bf16x4 prev = *reinterpret_cast<const bf16x4*>(out + idx);
#pragma unroll
    for (int r = 0; r < 4; ++r) o[r] = static_cast<bf16>(v[r] + static_cast<float>(prev[r]));
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) o[r] = static_cast<bf16>(v[r]);
  }
  *reinterpret_cast<bf16x4*>(out + idx) = o;
}

__device__ __forceinline__ void store4_silu(bf16* out, size_t idx, const float g[4], const float u[4]) {
  bf16x4 o;
#pragma unroll
  for (int r = 0; r < 4; ++r) o[r] = static_cast<bf16>(silu_f(g[r]) * u[r]);
  *reinterpret_cast<bf16x4*>(out + idx) = o;
}

// ------------------------------------------------------------- tiled ------

constexpr int kTBK = 64;  // k per LDS stage
constexpr int kGroupM = 8;  // token tiles per group in the XCD-local tile order

// BM tokens x BN weight rows per workgroup, WM x WN waves (a wave owns
// BM/WM tokens x BN/WN rows), K in stages of 64 through double-buffered
// XOR-swizzled LDS (dynamic: up to 128 KiB).  Tiles go straight from global
// memory into LDS (global_load_lds_dwordx4, no register staging): a wave's
// load instruction fills 1 KiB of LDS linearly, 16 bytes per lane, so each
// lane fetches the global chunk that belongs at its LDS slot under the
// swizzle.  Rows of a ragged token tail read the last valid row instead and
// are never stored.
template <int BM, int BN, int WM, int WN, int EPI>
__global__ __launch_bounds__(64 * WM * WN) void gemm_tile_bf16(const bf16* __restrict__ X, int M,
                                                               const bf16* __restrict__ W, int N, int K,
                                                               WStride ws, void* out, int ldo, int group_m, int cw,
                                                               int kps) {
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN;     // wave tile: tokens x weight rows
  constexpr int SM = TM / 16, SN = TN / 16;     // 16x16 MFMA tiles per wave
  constexpr int WJ = BN / 8 / NW;               // 8-row (1 KiB) pieces of a W stage per wave
  constexpr int XJ = BM / 8 / NW;
  extern __shared__ __attribute__((aligned(16))) bf16 smem[];
  bf16* sW = smem;                    // [2][BN * 64]
  bf16* sX = smem + 2 * BN * kTBK;    // [2][BM * 64]
  auto swz = [](int row, int c) { return row * kTBK + ((c ^ (row & 7)) << 3); };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave / WM, wm = wave % WM;
  const int r16 = lane & 15, g = lane >> 4;

  // Workgroups are dispatched round-robin over the 8 XCDs, and the ones an
  // XCD runs together share its L2.  With group_m > 0 (the launcher checks
  // that the weight tiles divide by 8) the weight tiles are taken cw at a
  // time; within such a chunk XCD x owns nn = cw / 8 of them for every token
  // tile, and walks them in groups of group_m token tiles: for each weight
  // tile the group's token tiles run back to back.  Co-resident workgroups
  // then form a group_m x (32/group_m) block of tiles, so each x panel and
  // each W panel they stream is fetched into L2 once for several of them.
  // group_m = 0: token tiles fastest.
  const int num_m = (M + BM - 1) / BM;
  int m_t, n_t;
  //
  // The weight tiles go in chunks of cw (cw / 8 per XCD), each chunk over
  // every token tile before the next: a chunk small enough to stay in the
  // 256 MB MALL while the token tiles stream past is read from HBM once,
  // where walking all weight tiles per token group re-reads the whole
  // weight from HBM once per group (32768 x 57344 x 8192: 23.7 -> 22.8 ms).
  if (group_m > 0) {
    const int nn = cw / 8;
    const int xcd = blockIdx.x & 7, i = blockIdx.x >> 3;
    const int per_chunk = nn * num_m;
    const int c = i / per_chunk, ic = i - c * per_chunk;
    const int gsz = group_m * nn, grp = ic / gsz, r = ic - grp * gsz;
    const int gm = min(group_m, num_m - grp * group_m);
    m_t = grp * group_m + r % gm;
    n_t = c * cw + xcd * nn + r / gm;
  } else {
    m_t = blockIdx.x % num_m;
    n_t = blockIdx.x / num_m;
  }
  const int m0 = m_t * BM;
  const int n0 = n_t * BN;

  // this lane's source chunk in each 8-row piece: LDS slot (row, lane & 7)
  // holds logical chunk (lane & 7) ^ (row & 7), i.e. k = 8 * chunk within the
  // stage; the weight layout's strides place (row, k)
  const int prow = lane >> 3, pc = lane & 7;
  const bf16* wsrc[WJ];
#pragma unroll
  for (int j = 0; j < WJ; ++j) {
    const int row = n0 + (j * NW + wave) * 8 + prow;
    const int ch = pc ^ (row & 7);
    wsrc[j] = W + (size_t)(row & ~15) * K + (size_t)(row & 15) * ws.rs + (size_t)(ch >> 2) * ws.ks + (ch & 3) * 8;
  }
  const size_t wstage = (size_t)(kTBK / 32) * ws.ks;  // weight offset of one k stage
  // split-K: this workgroup's k range is [blockIdx.y * kps, +kps)
  const int k_split = blockIdx.y * kps;
#pragma unroll
  for (int j = 0; j < WJ; ++j) wsrc[j] += (size_t)(k_split / 32) * ws.ks;
  const bf16* xsrc[XJ];
#pragma unroll
  for (int j = 0; j < XJ; ++j) {
    const int row = (j * NW + wave) * 8 + prow;
    const int m = min(m0 + row, M - 1);
    xsrc[j] = X + (size_t)m * K + blockIdx.y * kps + ((pc ^ (row & 7)) << 3);
  }
  auto issue = [&](int buf, int kt) {
    const int k0 = kt * kTBK;
#pragma unroll
    for (int j = 0; j < WJ; ++j)
      __builtin_amdgcn_global_load_lds(
          (const void*)(wsrc[j] + kt * wstage),
          (__attribute__((address_space(3))) void*)(sW + buf * BN * kTBK + (j * NW + wave) * 8 * kTBK), 16, 0, 0);
#pragma unroll
    for (int j = 0; j < XJ; ++j)
      __builtin_amdgcn_global_load_lds(
          (const void*)(xsrc[j] + k0),
          (__attribute__((address_space(3))) void*)(sX + buf * BM * kTBK + (j * NW + wave) * 8 * kTBK), 16, 0, 0);
  };

  f32x4 acc[SN][SM];
#pragma unroll
  for (int i = 0; i < SN; ++i)
#pragma unroll
    for (int j = 0; j < SM; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = kps / kTBK;
  issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) issue(buf ^ 1, kt + 1);
#pragma unroll
    for (int s = 0; s < kTBK / 32; ++s) {
      const int c = s * 4 + g;
      bf16x8 b[SM];
#pragma unroll
      for (int j = 0; j < SM; ++j)
        b[j] = *reinterpret_cast<const bf16x8*>(&sX[buf * BM * kTBK + swz(wm * TM + j * 16 + r16, c)]);
#pragma unroll
      for (int i = 0; i < SN; ++i) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(&sW[buf * BN * kTBK + swz(wn * TN + i * 16 + r16, c)]);
#pragma unroll
        for (int j = 0; j < SM; ++j) acc[i][j] = mfma16(a, b[j], acc[i][j]);
      }
    }
    // the next stage's loads have landed in LDS and every wave is done
    // reading this one
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // epilogue: lane holds features n..n+3 of token m for each (i, j)
#pragma unroll
  for (int j = 0; j < SM; ++j) {
    const int m = m0 + wm * TM + j * 16 + r16;
    if (m >= M) continue;
    if (EPI == kEpiPartial) {  // fp32 partial sums [split][M][ldo] (ldo = weight rows)
      float* dst = reinterpret_cast<float*>(out) + ((size_t)blockIdx.y * M + m) * ldo;
#pragma unroll
      for (int i = 0; i < SN; ++i) *reinterpret_cast<f32x4*>(dst + n0 + wn * TN + i * 16 + 4 * g) = acc[i][j];
    } else if (EPI == kEpiSiluMul) {
#pragma unroll
      for (int i = 0; i < SN; i += 2) {
        const int f = ((n0 + wn * TN + i * 16) >> 5) * 16 + 4 * g;
        float gv[4], uv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          gv[r] = acc[i][j][r];
          uv[r] = acc[i + 1][j][r];
        }
        store4_silu(reinterpret_cast<bf16*>(out), (size_t)m * ldo + f, gv, uv);
      }
    } else {
#pragma unroll
      for (int i = 0; i < SN; ++i) {
        const int n = n0 + wn * TN + i * 16 + 4 * g;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = acc[i][j][r];
        store4<EPI>(reinterpret_cast<bf16*>(out), (size_t)m * ldo + n, v);
      }
    }
  }
}

// splits > 1 (EPI = kEpiPartial): fp32 partials [splits][M][wrows] in out
template <int BM, int BN, int WM, int WN, int EPI>
hipError_t launch_tile(const bf16* x, int M, const bf16* w, int wrows, int K, WStride ws, void* out, int ldo,
                       hipStream_t s, int splits = 1) {
  auto fn = gemm_tile_bf16<BM, BN, WM, WN, EPI>;
  const size_t lds = (size_t)2 * (BM + BN) * kTBK * sizeof(bf16);
  // more than 64 KiB of dynamic LDS needs the function's opt-in: done once
  // per instantiation (a thread-safe function-local static)
  static const hipError_t attr =
      lds > 65536 ? hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds)
                  : hipSuccess;
  if (attr != hipSuccess) return attr;
  const int nb = ((M + BM - 1) / BM) * (wrows / BN);
  // XCD-grouped order wherever the weight tiles divide by 8: every token
  // tile of a weight tile runs on the XCD that owns it.  The plain order
  // (token tiles fastest) spreads them over the XCDs, so each XCD's L2
  // fetches the weight tile again: measured on 12 shapes, grouped is as fast
  // or faster everywhere (544 x 57344 x 8192: 603 -> 563 us; 1536 tokens:
  // 1358 -> 1287 us; 8192 x 8192 x 8192: 917 -> 882 us; 32768 x 57344 x
  // 8192: 26.9 -> 25.8 ms).
  const int num_m = (M + BM - 1) / BM;
  const int group_m = (wrows / BN) % 8 == 0 ? kGroupM : 0;
  // weight chunks of 32 tiles where 32 tiles of this K fit in 160 MB
  const int ntot = wrows / BN;
  const int cw = ntot % 32 == 0 && (size_t)32 * BN * K * sizeof(bf16) <= ((size_t)160 << 20) ? 32 : ntot;
  fn<<<dim3(nb, splits), 64 * WM * WN, lds, s>>>(x, M, w, wrows, K, ws, out, ldo, group_m, cw, K / splits);
  return hipGetLastError();
}

// out[m][n] (bf16) from S fp32 partial rows, summed in split order, with the
// projection's epilogue: store, residual add (out holds the addend) or
// SiluAndMul over the re-ordered gate_up rows (each 32-row group: 16 gate
// rows, then the 16 matching up rows).  Four output features per thread.
template <int EPI>
__global__ __launch_bounds__(256) void tile_reduce_kernel(const float* __restrict__ part, int S, int M, int wrows,
                                                          int N, bf16* __restrict__ out) {
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= (size_t)M * N) return;
  const size_t m = i / N;
  const int n = (int)(i % N);
  const size_t plane = (size_t)M * wrows;
  const float* src = part + m * wrows;
  f32x4 a, u;
  const int ga = EPI == kEpiSiluMul ? (n >> 4) * 32 + (n & 15) : n;  // gate (or plain) column
  a = *reinterpret_cast<const f32x4*>(src + ga);
  if (EPI == kEpiSiluMul) u = *reinterpret_cast<const f32x4*>(src + ga + 16);
  for (int k = 1; k < S; ++k) {
    const f32x4 b = *reinterpret_cast<const f32x4*>(src + k * plane + ga);
#pragma unroll
    for (int r = 0; r < 4; ++r) a[r] += b[r];
    if (EPI == kEpiSiluMul) {
      const f32x4 c = *reinterpret_cast<const f32x4*>(src + k * plane + ga + 16);
#pragma unroll
      for (int r = 0; r < 4; ++r) u[r] += c[r];
    }
  }
  float v[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) v[r] = a[r];
  if (EPI == kEpiSiluMul) {
    float uv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) uv[r] = u[r];
    store4_silu(out, i, v, uv);
  } else {
    store4<EPI>(out, i, v);
  }
}

// -------------------------------------------------------------- fp32 ------

constexpr int kF = 16;

template <int EPI>
__global__ __launch_bounds__(kF* kF) void gemm_f32(const float* __restrict__ X, int M,
                                                  const float* __restrict__ W, int N, int K,
                                                  float* out, int ldo) {
  __shared__ float sx[kF][kF + 1];
  __shared__ float sw[kF][kF + 1];
  __shared__ float su[kF][kF + 1];
  const int tx = threadIdx.x % kF;  // output feature within tile
  const int ty = threadIdx.x / kF;  // token within tile
  const int m = blockIdx.y * kF + ty;
  const int n = blockIdx.x * kF + tx;
  float acc = 0.f, accu = 0.f;
  for (int k0 = 0; k0 < K; k0 += kF) {
    // cooperative loads: row ty of x tile, row ty of W tile (features)
    const int kk = k0 + tx;
    const int xm = blockIdx.y * kF + ty;
    const int wn = blockIdx.x * kF + ty;
    sx[ty][tx] = (xm < M && kk < K) ? X[(size_t)xm * K + kk] : 0.f;
    sw[ty][tx] = (wn < N && kk < K) ? W[(size_t)wn * K + kk] : 0.f;
    if (EPI == kEpiSiluMul) su[ty][tx] = (wn < N && kk < K) ? W[(size_t)(N + wn) * K + kk] : 0.f;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kF; ++k) {
      acc = fmaf(sx[ty][k], sw[tx][k], acc);
      if (EPI == kEpiSiluMul) accu = fmaf(sx[ty][k], su[tx][k], accu);
    }
    __syncthreads();
  }
  if (m < M && n < N) {
    const size_t o = (size_t)m * ldo + n;
    if (EPI == kEpiAdd) out[o] = acc + out[o];
    else if (EPI == kEpiSiluMul) out[o] = silu_f(acc) * accu;
    else out[o] = acc;
  }
}

__global__ void reorder_gate_up_kernel(const bf16* __restrict__ src, int inter, int K, bf16* dst) {
  const int R = blockIdx.x;
  const int grp = R >> 5, i = R & 31;
  const int srow = (i < 16) ? (grp * 16 + i) : (inter + grp * 16 + (i - 16));
  const bf16x8* s = reinterpret_cast<const bf16x8*>(src + (size_t)srow * K);
  bf16x8* d = reinterpret_cast<bf16x8*>(dst + (size_t)R * K);
  for (int c = threadIdx.x; c < K / 8; c += blockDim.x) d[c] = s[c];
}

// The tile shape a plan names: 256 or 192 token rows x 256 weight rows (8
// waves), or 128 x 128 (4 waves).
template <int EPI>
hipError_t launch_planned(const TilePlan& tp, const bf16* x, int M, const bf16* w, int wrows, int K, WStride ws,
                          void* out, int ldo, hipStream_t s, int splits) {
  if (tp.bm == 256) return launch_tile<256, 256, 2, 4, EPI>(x, M, w, wrows, K, ws, out, ldo, s, splits);
  if (tp.bm == 192) return launch_tile<192, 256, 2, 4, EPI>(x, M, w, wrows, K, ws, out, ldo, s, splits);
  return launch_tile<128, 128, 2, 2, EPI>(x, M, w, wrows, K, ws, out, ldo, s, splits);
}

template <int EPI>
hipError_t linear_bf16(const bf16* x, const bf16* w, int M, int N, int K, bf16* out, hipStream_t s, int layout,
                       float* part, size_t part_cap) {
  // rows of W the kernel walks: N (store/add) or 2N (silu_mul)
  const int wrows = (EPI == kEpiSiluMul) ? 2 * N : N;
  if (M <= kSkinnyMaxM)
    return launch_skinny(x, w, M, N, K, EPI, skinny_plan(M, wrows, K, false, device_cu_count()), out, s, layout);
  const WStride ws = weight_stride(layout, K);
  const TilePlan tp = tile_plan(M, wrows, K, device_cu_count());
  if (tp.splits > 1 && part && tp.partial_bytes <= part_cap) {
    hipError_t e = launch_planned<kEpiPartial>(tp, x, M, w, wrows, K, ws, part, wrows, s, tp.splits);
    if (e != hipSuccess) return e;
    const size_t quads = (size_t)M * N / 4;
    tile_reduce_kernel<EPI><<<(unsigned)((quads + 255) / 256), 256, 0, s>>>(part, tp.splits, M, wrows, N, out);
    return hipGetLastError();
  }
  return launch_planned<EPI>(tp, x, M, w, wrows, K, ws, out, N, s, 1);
}

// one thread per 16-byte piece of the destination
__global__ void tile_weight_kernel(const bf16* __restrict__ src, int rows, int K, int inter, bf16* __restrict__ dst) {
  const size_t piece = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (piece >= (size_t)rows * K / 8) return;
  const int r = (int)(piece * 8 / K), k = (int)(piece * 8 % K);
  int sr = r;
  if (inter > 0) {
    const int grp = r >> 5, i = r & 31;
    sr = i < 16 ? grp * 16 + i : inter + grp * 16 + (i - 16);
  }
  const size_t o = ((size_t)(r >> 4) * (K / 32) + (k >> 5)) * 512 + (r & 15) * 32 + (k & 31);
  *reinterpret_cast<bf16x8*>(dst + o) = ld16<bf16x8>(src + (size_t)sr * K + k);
}

template <int EPI>
hipError_t linear_f32(const float* x, const float* w, int M, int N, int K, float* out, hipStream_t s) {
  dim3 grid((N + kF - 1) / kF, (M + kF - 1) / kF);
  gemm_f32<EPI><<<grid, kF * kF, 0, s>>>(x, M, w, N, K, out, N);
  return hipGetLastError();
}

}  // namespace

TilePlan tile_plan(int M, int wrows, int K, int num_cus) {
  TilePlan p;
  const int cus = num_cus > 0 ? num_cus : 256;
  p.bm = 128;
  p.splits = 1;
  if (M >= 256 && wrows % 256 == 0) {
    // 256-row weight tiles, token tiles of 256 or 192 rows, K unsplit or
    // split in 2, 4 or 8 (fp32 partials, then a reduce kernel).  Each plan
    // is priced from measurements on gfx950 and the cheapest taken:
    //   * one 64-deep k stage of a 256 x 256 tile takes ~1.63 us when every
    //     CU runs one workgroup, of a 192 x 256 tile 0.79 of that;
    //   * the workgroups run in rounds of one per CU, and a partly filled
    //     last round costs 0.75 + 0.25 x its fill of a full one;
    //   * the partials cost 8 bytes per element and split (written, read
    //     back) at ~5 TB/s.
    // Fitted to 14 shapes (70B prefill and mixed-step projections, one GPU's
    // TP = 8 share, the Qwen3-MoE attention projections, 300 and 1000
    // tokens), it picks the measured fastest of the 8 plans for each: e.g.
    // 8192 x 1280 x 8192 (TP = 8 qkv) 192-row tiles unsplit, 153 us against
    // 215 us for 256-row tiles split in 2 (320 workgroups: a second round
    // for a quarter of the CUs).
    constexpr double kStageUs = 1.63, kBm192 = 0.79, kReduceBytesPerUs = 5.0e6;
    double best = 0.0;
    for (const int bm : {256, 192}) {
      const long long tiles = (long long)((M + bm - 1) / bm) * (wrows / 256);
      for (int s = 1; s <= 8; s *= 2) {
        if (K % (s * kTBK) != 0) break;
        const long long wgs = tiles * s, full = wgs / cus, rem = wgs % cus;
        const double rounds = (double)full + (rem ? 0.75 + 0.25 * (double)rem / cus : 0.0);
        double c = rounds * (double)(K / s / kTBK) * kStageUs * (bm == 256 ? 1.0 : kBm192);
        if (s > 1) c += 8.0 * s * (double)M * wrows / kReduceBytesPerUs;
        if (best == 0.0 || c < best) {  // ties keep the larger tile and fewer splits
          best = c;
          p.bm = bm;
          p.splits = s;
        }
      }
    }
  } else {
    // fewer than 256 tokens, or weight rows not a multiple of 256: 128 x 128
    // tiles, K split while the tiles alone leave CUs idle
    const int tiles = ((M + 127) / 128) * (wrows / 128);
    for (int s = 2; s <= 8 && tiles * p.splits < cus && K % (s * kTBK) == 0; s *= 2) p.splits = s;
  }
  p.partial_bytes = p.splits > 1 ? (size_t)p.splits * M * wrows * sizeof(float) : 0;
  return p;
}

int device_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n;
}

const char* linear_kernel_name(int dtype, int M) {
  if (dtype != kBF16) return "gemm_f32";
  return M <= kSkinnyMaxM ? "gemm_skinny_bf16" : "gemm_tile_bf16";
}

hipError_t launch_linear(int dtype, const void* x, const void* w, int M, int N, int K, int epi,
                         void* out, hipStream_t s, int layout, float* part, size_t part_cap) {
  if (M <= 0) return hipSuccess;
  if (dtype == kBF16) {
    const bf16* xb = (const bf16*)x;
    const bf16* wb = (const bf16*)w;
    bf16* ob = (bf16*)out;
    const int wrows = (epi == kEpiSiluMul) ? 2 * N : N;
    if (layout == kTiled16x32 && (wrows % 16 != 0 || K % 32 != 0)) return hipErrorInvalidValue;
    // the tiled kernels walk weight rows in 128- or 256-row tiles
    if (M > kSkinnyMaxM && (wrows % 128 != 0 || K % kTBK != 0)) return hipErrorInvalidValue;
    switch (epi) {
      case kEpiStore: return linear_bf16<kEpiStore>(xb, wb, M, N, K, ob, s, layout, part, part_cap);
      case kEpiAdd: return linear_bf16<kEpiAdd>(xb, wb, M, N, K, ob, s, layout, part, part_cap);
      default: return linear_bf16<kEpiSiluMul>(xb, wb, M, N, K, ob, s, layout, part, part_cap);
    }
  }
  const float* xf = (const float*)x;
  const float* wf = (const float*)w;
  float* of = (float*)out;
  switch (epi) {
    case kEpiStore: return linear_f32<kEpiStore>(xf, wf, M, N, K, of, s);
    case kEpiAdd: return linear_f32<kEpiAdd>(xf, wf, M, N, K, of, s);
    default: return linear_f32<kEpiSiluMul>(xf, wf, M, N, K, of, s);
  }
}

hipError_t launch_gemm_partials(const void* x, const void* w, int M, int wrows, int K, int layout, float* out,
                                hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (wrows % 128 || K % kTBK) return hipErrorInvalidValue;
  const TilePlan tp = tile_plan(M, wrows, K, device_cu_count());
  const WStride ws = weight_stride(layout, K);
  return launch_planned<kEpiPartial>(tp, (const bf16*)x, M, (const bf16*)w, wrows, K, ws, out, wrows, s, tp.splits);
}

hipError_t launch_silu_reduce(const float* part, int S, int M, int wrows, void* out, hipStream_t s) {
  const size_t quads = (size_t)M * (wrows / 2) / 4;
  if (quads == 0) return hipSuccess;
  if (wrows % 32) return hipErrorInvalidValue;
  tile_reduce_kernel<kEpiSiluMul><<<(unsigned)((quads + 255) / 256), 256, 0, s>>>(part, S, M, wrows, wrows / 2,
                                                                                 (bf16*)out);
  return hipGetLastError();
}

hipError_t launch_reorder_gate_up(const void* src, int inter, int K, void* dst, hipStream_t s) {
  reorder_gate_up_kernel<<<2 * inter, 256, 0, s>>>((const bf16*)src, inter, K, (bf16*)dst);
  return hipGetLastError();
}

hipError_t launch_tile_weight(const void* src, int rows, int K, int inter, void* dst, hipStream_t s) {
  if (rows % 16 != 0 || K % 32 != 0 || (inter > 0 && rows != 2 * inter) || (inter > 0 && inter % 16 != 0))
    return hipErrorInvalidValue;
  const size_t pieces = (size_t)rows * K / 8;
  if (pieces == 0) return hipSuccess;
  tile_weight_kernel<<<(unsigned)((pieces + 255) / 256), 256, 0, s>>>((const bf16*)src, rows, K, inter, (bf16*)dst);
  return hipGetLastError();
}

}  // namespace llk
