// Launchers of the gfx950 kernels (host functions, one family per .hip file).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace llk {

enum Dtype { kBF16 = 0, kFP32 = 1 };
enum Epi { kEpiStore = 0, kEpiAdd = 1, kEpiSiluMul = 2, kEpiPartial = 3 };

// rmsnorm.hip.  With xpart != NULL (bf16 only) the input row is the sum of
// S fp32 partial rows xpart[s][row][:] instead of x.
hipError_t launch_add_rmsnorm(int dtype, const void* x, const void* res, const void* w, float eps,
                              int rows, int hidden, void* normed, void* res_out, hipStream_t s,
                              const float* xpart = nullptr, int S = 0);

// gemm.hip: out = x W^T with an epilogue; picks the skinny (M <= 64) or the
// tiled kernel.
hipError_t launch_linear(int dtype, const void* x, const void* w, int M, int N, int K, int epi,
                         void* out, hipStream_t s);
hipError_t launch_reorder_gate_up(const void* src, int inter, int K, void* dst, hipStream_t s);
const char* linear_kernel_name(int dtype, int M);

// gemm_skinny.hip: bf16, M <= 64.  N = output features (SiluMul: W has 2N
// rows).  kEpiPartial writes fp32 partial sums [splits][M][N].
struct SkinnyPlan {
  int mt, nt, nw, kc, splits;  // token tiles, row tiles per wave, waves, K chunk, K splits
};
SkinnyPlan skinny_plan(int M, int wrows, int K, bool allow_split, int num_cus);
int device_cu_count();
hipError_t launch_skinny(const void* x, const void* w, int M, int N, int K, int epi, const SkinnyPlan& p,
                         void* out, hipStream_t s);
hipError_t launch_splitk_reduce(const float* part, int S, int M, int N, void* out, hipStream_t s);

// rope_kv.hip.  With part != NULL (bf16 only) the projection row is first
// formed as the bf16 rounding of the sum of S fp32 partial rows and stored
// into qkv.
hipError_t launch_rope_kv(int dtype, void* qkv, int T, const int* positions, const float2* table,
                          int nq, int nkv, int d, const int* block_table, int max_blocks, int q_len,
                          void* k_cache, void* v_cache, hipStream_t s, const float* part = nullptr,
                          int S = 0);

// attention.hip
struct AttnPlan {
  int parts;        // key partitions per query (1 = no split)
  int part_len;     // keys per partition
  size_t ws_bytes;  // fp32 partial results
};
AttnPlan attention_plan(int T, int nq, int nkv, int d, int q_len, int max_seq_len, int num_cus);
hipError_t launch_attention(int dtype, const void* q, int ldq, int T, const int* positions, int nq,
                            int nkv, int d, const void* k_cache, const void* v_cache,
                            const int* block_table, int max_blocks, int q_len,
                            const AttnPlan& plan, float* partials, void* out, hipStream_t s,
                            hipEvent_t mid_event);

// attention_decode.hip (bf16, one query token per sequence)
hipError_t launch_decode_attention_bf16(const void* q, int ldq, int T, const int* positions, int nq, int nkv,
                                        int d, const void* k_cache, const void* v_cache, const int* block_table,
                                        int max_blocks, int q_len, int part_len, int parts, float* partials,
                                        void* out, hipStream_t s);

// attention_prefill.hip (bf16, q_len > 1, G in {4, 8, 16})
bool prefill_attention_supported(int nq, int nkv, int d);
hipError_t launch_prefill_attention_bf16(const void* q, int ldq, int T, const int* positions, int nq, int nkv,
                                         int d, const void* k_cache, const void* v_cache, const int* block_table,
                                         int max_blocks, int q_len, void* out, hipStream_t s);

}  // namespace llk
