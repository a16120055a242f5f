// Host side of the C ABI: configuration checks, weight ownership, the RoPE
// table, workspace carving and the launch sequence of one layer forward.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <string>
#include <vector>

#include "../../include/llama_layer.h"
#include "kernels.h"

namespace {

thread_local std::string g_err;

llama_status fail(llama_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

llama_status hip_fail(hipError_t e, const char* what) {
  return fail(LLAMA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Makes `dev` the current device for the scope's lifetime and restores the
// caller's afterwards: the destroy calls may come with another device current.
struct DeviceScope {
  int prev = -1;
  explicit DeviceScope(int dev) {
    int cur = -1;
    if (dev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != dev && hipSetDevice(dev) == hipSuccess) prev = cur;
  }
  ~DeviceScope() {
    if (prev >= 0) (void)hipSetDevice(prev);
  }
};

#define HIP_TRY(expr, what)                      \
  do {                                           \
    hipError_t e_ = (expr);                      \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

size_t elem_size(int dtype) { return dtype == LLAMA_DTYPE_BF16 ? 2 : 4; }
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

bool is_llama3(const llama_layer_config* c) {
  return c->rope_type != nullptr && std::strcmp(c->rope_type, "llama3") == 0;
}

// Angular frequency of RoPE pair i: theta^(-2i/d), then for rope_type llama3
// the published Llama 3 rescaling by wavelength 2*pi/w: below
// orig/high_freq_factor unchanged, above orig/low_freq_factor divided by
// factor, and in between blended (1-s) w/factor + s w with
// s = (orig/wavelength - low) / (high - low).
double rope_freq(const llama_layer_config* c, int i) {
  const double w = std::pow(c->rope_theta, -2.0 * i / c->head_dim);
  if (!is_llama3(c)) return w;
  const double orig = c->original_max_position_embeddings;
  const double lo = c->low_freq_factor, hi = c->high_freq_factor, f = c->rope_factor;
  const double wavelen = 2.0 * M_PI / w;
  if (wavelen < orig / hi) return w;
  if (wavelen > orig / lo) return w / f;
  const double s = (orig / wavelen - lo) / (hi - lo);
  return (1.0 - s) * w / f + s * w;
}

struct TimingMark {
  const char* name;  // kernel that ran between the previous mark and this one
  hipEvent_t ev;
};

}  // namespace

struct llama_layer {
  llama_layer_config cfg;
  std::string act, rope_type;
  int dtype = 0;
  size_t es = 2;
  int qkv_n = 0;
  int num_cus = 0;  // compute units of the device the layer was created on
  int wlayout = 0;  // llk::WeightLayout of the projection weights
  int device = -1;  // HIP device the layer lives on
  hipError_t scratch_err = hipSuccess;  // setup of that device's no-allocation scratch
  void* w_in = nullptr;
  void* w_qkv = nullptr;
  void* w_o = nullptr;
  void* w_post = nullptr;
  void* w_gu = nullptr;
  void* w_down = nullptr;
  void* w_qn = nullptr;      // q_norm / k_norm (qk_norm)
  void* w_kn = nullptr;
  void* w_router = nullptr;  // MoE: router, expert gate_up (tiled, re-ordered), expert down (tiled)
  void* w_e13 = nullptr;
  void* w_e2 = nullptr;
  int E = 0, topk = 0, moe_I = 0;
  float2* rope = nullptr;
  bool owns_rope = true;  // false: the table belongs to another layer of the same stack

  bool timing = false;
  std::vector<std::vector<TimingMark>> marks;  // one list per forward
  std::vector<hipEvent_t> event_pool;
  std::map<std::string, std::pair<double, int64_t>> totals;
};

namespace {

struct Workspace {
  size_t h, qkv, attn, h2, act, part, gpart, tpart, tpart_bytes, seq_of, ntiles, tiles, dec, ndec, row_parts, check,
      total;
  int tile_cap;  // entries of the prefill tile table (mixed batches)
  // MoE routing and expert buffers (P = T * topk pairs)
  size_t rpart, logits, ids, wts, seg, sorted, active, nactive, mtiles, mntiles, mchunk, mact, mpart;
  int moe_tile_cap;
  llk::AttnPlan plan;
  bool skinny;  // few tokens: weight-streaming projections with split-K partials
  llk::SkinnyPlan pq, po, pg, pd;
  bool o_wsplit, d_wsplit;  // o_proj / down_proj split K inside the workgroup (final rows, no partials)
};

// prefill attention runs on the matrix-core kernel (whose keys may be split)
bool split_prefill(const llama_layer* L) {
  const llama_layer_config& c = L->cfg;
  return L->dtype == LLAMA_DTYPE_BF16 &&
         llk::prefill_attention_supported(c.num_attention_heads, c.num_key_value_heads, c.head_dim);
}

Workspace carve(const llama_layer* L, int T, int B, int max_seq_len) {
  const llama_layer_config& c = L->cfg;
  Workspace w{};
  w.plan = llk::attention_plan(T, B, c.num_attention_heads, c.num_key_value_heads, c.head_dim, T == B,
                              max_seq_len, L->num_cus, split_prefill(L));
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align256(bytes);
    return o;
  };
  w.h = take((size_t)T * c.hidden_size * L->es);
  w.qkv = take((size_t)T * L->qkv_n * L->es);
  w.attn = take((size_t)T * c.num_attention_heads * c.head_dim * L->es);
  w.h2 = take((size_t)T * c.hidden_size * L->es);
  w.act = take(L->E ? 0 : (size_t)T * c.intermediate_size * L->es);
  w.part = take(w.plan.ws_bytes);
  const int H = c.hidden_size, Q = c.num_attention_heads * c.head_dim, I = c.intermediate_size;
  w.skinny = L->dtype == LLAMA_DTYPE_BF16 && T <= llk::kSkinnyMaxM;
  size_t gpart = 0;
  if (w.skinny) {
    w.pq = llk::skinny_plan(T, L->qkv_n, H, true, L->num_cus);
    w.po = llk::skinny_plan(T, H, Q, true, L->num_cus);
    w.o_wsplit = llk::skinny_wave_split_ok(T, H, Q, L->num_cus);
    w.d_wsplit = !L->E && llk::skinny_wave_split_ok(T, H, I, L->num_cus);
    size_t n = (size_t)w.pq.splits * L->qkv_n;
    if (!w.o_wsplit && (size_t)w.po.splits * H > n) n = (size_t)w.po.splits * H;
    if (!L->E) {
      // gate_up: unsplit (SiluAndMul in the epilogue) when its row tiles
      // alone fill the CUs; a short weight (e.g. one GPU's tensor-parallel
      // share) splits K into fp32 partials that a SiluAndMul reduce finishes
      w.pg = llk::skinny_plan(T, 2 * I, H, false, L->num_cus);
      if (2 * I / (16 * w.pg.nt * w.pg.nw) < L->num_cus) {
        w.pg = llk::skinny_plan(T, 2 * I, H, true, L->num_cus);
        if ((size_t)w.pg.splits * 2 * I > n) n = (size_t)w.pg.splits * 2 * I;
      }
      w.pd = llk::skinny_plan(T, H, I, true, L->num_cus);
      if (!w.d_wsplit && (size_t)w.pd.splits * H > n) n = (size_t)w.pd.splits * H;
    }
    gpart = n * T * sizeof(float);
  }
  w.gpart = take(gpart);
  // tiled projections that split K keep their fp32 partials here
  w.tpart_bytes = 0;
  if (L->dtype == LLAMA_DTYPE_BF16 && !w.skinny) {
    const int dims[4][2] = {{L->qkv_n, H}, {H, Q}, {2 * I, H}, {H, I}};  // weight rows, K
    for (int i = 0; i < (L->E ? 2 : 4); ++i) {
      const int* dk = dims[i];
      const size_t b = llk::tile_plan(T, dk[0], dk[1], L->num_cus).partial_bytes;
      if (b > w.tpart_bytes) w.tpart_bytes = b;
    }
  }
  w.tpart = take(w.tpart_bytes);
  // mixed batches: row -> sequence map and the prefill tile table (tiles of
  // at least 16 rows, so T/16 + B entries bound any sequence mix)
  w.tile_cap = T / 16 + B + 1;
  w.seq_of = take((size_t)T * sizeof(int));
  w.ntiles = take(sizeof(int));
  w.tiles = take((size_t)w.tile_cap * sizeof(int4));
  // the rows of single-row sequences (decode attention) and the key
  // partitions of each row when prefill attention is split
  w.dec = take((size_t)B * sizeof(int));
  w.ndec = take(sizeof(int));
  w.row_parts = take((size_t)T * sizeof(int));
  w.check = take(llk::kCheckFlags * sizeof(int));  // flags of the debug-mode metadata check
  const size_t P = L->E ? (size_t)T * L->topk : 0;
  w.moe_tile_cap = L->E ? (int)(P / llk::kMoeTileRows) + L->E + 1 : 0;
  w.rpart = take(L->E ? (size_t)llk::moe_router_splits(T, H, L->E, L->num_cus) * T * L->E * sizeof(float) : 0);
  w.logits = take((size_t)T * L->E * sizeof(float));
  w.ids = take(P * sizeof(int));
  w.wts = take(P * sizeof(float));
  w.seg = take(L->E ? (size_t)(L->E + 1) * sizeof(int) : 0);
  w.sorted = take(P * sizeof(int));
  w.active = take((size_t)L->E * sizeof(int));
  w.nactive = take(L->E ? sizeof(int) : 0);
  w.mtiles = take((size_t)w.moe_tile_cap * sizeof(int4));
  w.mntiles = take(L->E ? sizeof(int) : 0);
  w.mchunk = take((size_t)llk::moe_align_chunks((int)P) * L->E * sizeof(int));
  w.mact = take(P * L->moe_I * L->es);
  w.mpart = take(P * H * L->es);
  w.total = off;
  return w;
}

hipEvent_t pool_event(llama_layer* L) {
  if (!L->event_pool.empty()) {
    hipEvent_t e = L->event_pool.back();
    L->event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Records an event after the kernel `name` (or the opening mark when name is
// NULL) while timing is on.
struct Marker {
  llama_layer* L;
  hipStream_t s;
  std::vector<TimingMark>* list = nullptr;
  Marker(llama_layer* L_, hipStream_t s_) : L(L_), s(s_) {
    if (L->timing) {
      L->marks.emplace_back();
      list = &L->marks.back();
      mark(nullptr);
    }
  }
  void mark(const char* name) {
    if (!list) return;
    hipEvent_t e = pool_event(L);
    if (e && hipEventRecord(e, s) == hipSuccess) list->push_back({name, e});
  }
  hipEvent_t extra() {  // an event recorded inside a launcher (between two kernels)
    return list ? pool_event(L) : nullptr;
  }
};

// Every decode step streams each weight matrix whole, with every CU reading
// a different region of it at once.  A physically contiguous allocation is
// mapped with the largest page fragments, so those concurrent streams need
// few address translations; measured on the 939 MB gate_up weight, scattered
// placements streamed up to 9% slower.  The runtime may refuse the request on
// fragmented memory: plain hipMalloc then.
hipError_t alloc_weight(void** p, size_t bytes) {
  if (hipExtMallocWithFlags(p, bytes, hipDeviceMallocContiguous) == hipSuccess) return hipSuccess;
  (void)hipGetLastError();
  *p = nullptr;
  return hipMalloc(p, bytes);
}

void free_layer(llama_layer* L) {
  if (!L) return;
  void* bufs[] = {L->w_in,  L->w_qkv,    L->w_o,   L->w_post, L->w_gu,          L->w_down,
                  L->w_qn,  L->w_kn,     L->w_router, L->w_e13, L->w_e2,
                  L->owns_rope ? (void*)L->rope : nullptr};
  for (void* p : bufs)
    if (p) (void)hipFree(p);
  for (auto& list : L->marks)
    for (auto& m : list) (void)hipEventDestroy(m.ev);
  for (hipEvent_t e : L->event_pool) (void)hipEventDestroy(e);
  delete L;
}

// The sparse MoE block on the post-attention norm output h2 [T, H]: router +
// top-k, grouping of the (token, expert) pairs by expert, the expert GEMMs,
// and the weighted sum into out.
// Debug mode: the environment variable LLAMA_DEBUG=1, read at each call.
bool debug_checks() {
  const char* v = std::getenv("LLAMA_DEBUG");
  return v && std::strcmp(v, "1") == 0;
}

// Checks the call's device metadata (block ids, positions, row ranges,
// KV lengths) on the device and waits for the answer.  Skipped while the
// stream is being captured: a capture cannot wait.
llama_status check_metadata(const llama_layer* L, const Workspace& w, char* ws, const int* positions, int T,
                            const llama_kv_cache* kv, const int* block_table, int max_blocks, const int* seq_lens,
                            const int* qsl, int B, int max_seq_len, hipStream_t s) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(s, &cs);
  if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
  if (cs != hipStreamCaptureStatusNone) return LLAMA_OK;
  int* flags = (int*)(ws + w.check);
  e = hipMemsetAsync(flags, 0, llk::kCheckFlags * sizeof(int), s);
  if (e != hipSuccess) return hip_fail(e, "metadata check");
  e = llk::launch_validate_batch(positions, T, block_table, max_blocks, seq_lens, qsl, B, kv->num_blocks,
                                 L->cfg.max_position_embeddings, max_seq_len, flags, s);
  if (e != hipSuccess) return hip_fail(e, "metadata check");
  int host[llk::kCheckFlags] = {};
  e = hipMemcpyAsync(host, flags, sizeof(host), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "metadata check");
  static const char* what[llk::kCheckFlags] = {
      "query_start_loc is not 0 = q[0] < q[1] < ... < q[num_seqs] = num_tokens",
      "a seq_lens entry is below the sequence's rows or 1, or above max_seq_len",
      "a block_table entry covering positions below seq_lens is outside [0, kv_cache.num_blocks)",
      "a position is outside [0, max_position_embeddings) or not seq_lens[b] - rows_b + its index in the run"};
  std::string msg;
  for (int k = 0; k < llk::kCheckFlags; ++k)
    if (host[k]) msg += std::string(msg.empty() ? "" : "; ") + what[k];
  if (!msg.empty()) return fail(LLAMA_ERR_INVALID_ARGUMENT, "metadata check (LLAMA_DEBUG=1): %s", msg.c_str());
  return LLAMA_OK;
}

llama_status moe_block(llama_layer* L, const Workspace& w, char* ws, const void* h2, int T, void* out,
                       hipStream_t s, Marker& mk) {
  const int H = L->cfg.hidden_size, P = T * L->topk;
  llk::MoeRouting r;
  r.seg = (int*)(ws + w.seg);
  r.sorted = (int*)(ws + w.sorted);
  r.active = (int*)(ws + w.active);
  r.nactive = (int*)(ws + w.nactive);
  r.tiles = (int4*)(ws + w.mtiles);
  r.ntiles = (int*)(ws + w.mntiles);
  r.tile_cap = w.moe_tile_cap;
  r.wts = (float*)(ws + w.wts);
  r.chunk = (int*)(ws + w.mchunk);
  int* ids = (int*)(ws + w.ids);
  hipError_t e = llk::launch_moe_route(h2, T, H, L->w_router, L->E, L->topk, L->cfg.norm_topk_prob != 0,
                                       (float*)(ws + w.rpart), (float*)(ws + w.logits), ids, r.wts, s);
  if (e != hipSuccess) return hip_fail(e, "moe router");
  mk.mark("moe_router_topk");
  e = llk::launch_moe_align(ids, P, L->E, llk::kMoeTileRows, r, s);
  if (e != hipSuccess) return hip_fail(e, "moe align");
  mk.mark("moe_align");
  hipEvent_t mid = mk.extra();
  e = llk::launch_moe_experts(h2, T, H, L->topk, L->w_e13, L->w_e2, L->E, L->moe_I, L->wlayout, r, ws + w.mact,
                              ws + w.mpart, s, mid);
  if (e != hipSuccess) return hip_fail(e, "moe experts");
  if (mid) mk.list->push_back({"moe_gate_up_silu", mid});
  mk.mark("moe_down");
  e = llk::launch_moe_sum(ws + w.mpart, T, L->topk, H, out, s);
  if (e != hipSuccess) return hip_fail(e, "moe sum");
  mk.mark("moe_sum");
  return LLAMA_OK;
}

}  // namespace

extern "C" {

const char* llama_layer_last_error(void) { return g_err.c_str(); }

llama_status llama_layer_config_validate(const llama_layer_config* c) {
  if (!c) return fail(LLAMA_ERR_INVALID_ARGUMENT, "config is NULL");
  if (c->hidden_size <= 0 || c->num_attention_heads <= 0 || c->num_key_value_heads <= 0 ||
      c->head_dim <= 0 || c->intermediate_size <= 0 || c->max_position_embeddings <= 0)
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "all sizes must be positive");
  if (!(c->rms_norm_eps > 0.f)) return fail(LLAMA_ERR_INVALID_ARGUMENT, "rms_norm_eps must be > 0");
  if (!(c->rope_theta > 1.0)) return fail(LLAMA_ERR_INVALID_ARGUMENT, "rope_theta must be > 1");
  if (c->dtype != LLAMA_DTYPE_BF16 && c->dtype != LLAMA_DTYPE_FP32)
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "unknown dtype %d", c->dtype);
  if (c->num_attention_heads % c->num_key_value_heads != 0)
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "num_attention_heads %% num_key_value_heads != 0");
  if (!c->hidden_act || std::strcmp(c->hidden_act, "silu") != 0)
    return fail(LLAMA_ERR_UNSUPPORTED, "Unsupported activation: %s. Only silu is supported",
                c->hidden_act ? c->hidden_act : "(null)");
  if (c->attention_bias || c->mlp_bias)
    return fail(LLAMA_ERR_UNSUPPORTED, "attention_bias / mlp_bias are not supported");
  if (c->rope_type && std::strcmp(c->rope_type, "default") != 0 && std::strcmp(c->rope_type, "llama3") != 0)
    return fail(LLAMA_ERR_UNSUPPORTED, "rope_type %s is not supported", c->rope_type);
  if (is_llama3(c)) {
    if (!(c->rope_factor >= 1.0) || !(c->low_freq_factor > 0.0) ||
        !(c->high_freq_factor > c->low_freq_factor) || c->original_max_position_embeddings <= 0)
      return fail(LLAMA_ERR_INVALID_ARGUMENT,
                  "llama3 rope needs factor >= 1, high_freq_factor > low_freq_factor > 0, "
                  "original_max_position_embeddings > 0");
  }
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(LLAMA_ERR_UNSUPPORTED, "head_dim %d (supported: 64, 128)", c->head_dim);
  if (c->kv_block_size != 16)
    return fail(LLAMA_ERR_UNSUPPORTED, "kv_block_size %d (supported: 16)", c->kv_block_size);
  if (c->num_attention_heads / c->num_key_value_heads > 16)
    return fail(LLAMA_ERR_UNSUPPORTED, "more than 16 query heads per KV head");
  const int qkv_n = (c->num_attention_heads + 2 * c->num_key_value_heads) * c->head_dim;
  if (c->dtype == LLAMA_DTYPE_BF16) {
    if (c->hidden_size % 128 || c->intermediate_size % 128 || c->hidden_size > 16384 || qkv_n % 128 ||
        qkv_n > 16384 || (c->num_attention_heads * c->head_dim) % 64)
      return fail(LLAMA_ERR_UNSUPPORTED,
                  "bf16 needs hidden_size, intermediate_size and the qkv width to be multiples "
                  "of 128, hidden_size <= 16384 and qkv width <= 16384");
  } else {
    if (c->hidden_size % 4 || c->hidden_size > 8192)
      return fail(LLAMA_ERR_UNSUPPORTED, "fp32 needs hidden_size %% 4 == 0 and <= 8192");
  }
  if (c->num_experts < 0) return fail(LLAMA_ERR_INVALID_ARGUMENT, "num_experts must be >= 0");
  if (c->num_experts > 0) {
    if (c->dtype != LLAMA_DTYPE_BF16) return fail(LLAMA_ERR_UNSUPPORTED, "mixture-of-experts layers are bf16 only");
    if (c->num_experts_per_tok <= 0 || c->num_experts_per_tok > c->num_experts || c->moe_intermediate_size <= 0)
      return fail(LLAMA_ERR_INVALID_ARGUMENT, "need 1 <= num_experts_per_tok <= num_experts and moe_intermediate_size > 0");
    if (c->num_experts % 16 || c->num_experts > 256 || c->num_experts_per_tok > 64 ||
        c->moe_intermediate_size % 128 || c->hidden_size % 256)
      return fail(LLAMA_ERR_UNSUPPORTED,
                  "MoE needs num_experts a multiple of 16 up to 256, num_experts_per_tok <= 64, "
                  "moe_intermediate_size a multiple of 128 and hidden_size a multiple of 256");
  }
  return LLAMA_OK;
}

}  // extern "C"

namespace {

// A layer; with shared_rope the RoPE table of another layer of the same
// configuration (a stack builds it once), else its own.
llama_status create_layer(const llama_layer_config* config, const llama_layer_weights* w, void* stream,
                          float2* shared_rope, llama_layer** out) {
  llama_status st = llama_layer_config_validate(config);
  if (st != LLAMA_OK) return st;
  if (!w || !out || !w->input_layernorm || !w->qkv_proj || !w->o_proj || !w->post_attention_layernorm)
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "NULL weight or output pointer");
  if (config->num_experts > 0 ? (!w->router || !w->experts_gate_up || !w->experts_down)
                              : (!w->gate_up_proj || !w->down_proj))
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "NULL MLP or expert weight pointer");
  if (config->qk_norm && (!w->q_norm || !w->k_norm))
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "qk_norm needs q_norm and k_norm");
  *out = nullptr;
  hipStream_t s = (hipStream_t)stream;
  llama_layer* L = new llama_layer();
  L->cfg = *config;
  L->act = config->hidden_act;
  L->rope_type = config->rope_type ? config->rope_type : "default";
  L->cfg.hidden_act = L->act.c_str();
  L->cfg.rope_type = L->rope_type.c_str();
  L->dtype = config->dtype;
  L->es = elem_size(config->dtype);
  L->num_cus = llk::device_cu_count();
  if (hipGetDevice(&L->device) != hipSuccess) {
    delete L;
    return fail(LLAMA_ERR_HIP, "hipGetDevice failed");
  }
  // the device's scratch for llama_layer_forward_noalloc, looked up once
  L->scratch_err = llk::noalloc_scratch_setup(L->device);
  const llama_layer_config& c = L->cfg;
  const size_t H = c.hidden_size, I = c.intermediate_size, Q = (size_t)c.num_attention_heads * c.head_dim;
  L->qkv_n = (c.num_attention_heads + 2 * c.num_key_value_heads) * c.head_dim;
  L->E = c.num_experts;
  L->topk = L->E ? c.num_experts_per_tok : 0;
  L->moe_I = L->E ? c.moe_intermediate_size : 0;
  const size_t E = L->E, Ie = L->moe_I;

  // bf16 projection weights are kept in the 16x32-tiled layout (gate_up also
  // re-ordered into 16 gate + 16 up rows per 32-row group); norm weights and
  // fp32 weights are plain copies.
  const bool tile = L->dtype == LLAMA_DTYPE_BF16;
  L->wlayout = tile ? llk::kTiled16x32 : llk::kRowMajor;
  // The router stays row-major (its kernel reads whole rows); each expert's
  // gate_up is tiled and re-ordered on its own, and the stacked expert down
  // weights tile as one matrix (every expert starts on a 16-row strip).
  struct Item {
    void** dst;
    const void* src;
    int rows, cols, inter;  // rows = 0: a plain copy of `cols` elements
    int count;              // matrices stacked in src (experts), 0: not used
    bool tiled;
  } items[] = {
      {&L->w_in, w->input_layernorm, 0, (int)H, 0, 1, false},
      {&L->w_qkv, w->qkv_proj, L->qkv_n, (int)H, 0, 1, tile},
      {&L->w_o, w->o_proj, (int)H, (int)Q, 0, 1, tile},
      {&L->w_post, w->post_attention_layernorm, 0, (int)H, 0, 1, false},
      {&L->w_gu, w->gate_up_proj, (int)(2 * I), (int)H, (int)I, E ? 0 : 1, tile},
      {&L->w_down, w->down_proj, (int)H, (int)I, 0, E ? 0 : 1, tile},
      {&L->w_qn, w->q_norm, 0, c.head_dim, 0, c.qk_norm ? 1 : 0, false},
      {&L->w_kn, w->k_norm, 0, c.head_dim, 0, c.qk_norm ? 1 : 0, false},
      {&L->w_router, w->router, 0, (int)(E * H), 0, E ? 1 : 0, false},
      {&L->w_e13, w->experts_gate_up, (int)(2 * Ie), (int)H, (int)Ie, (int)E, true},
      {&L->w_e2, w->experts_down, (int)(E * H), (int)Ie, 0, E ? 1 : 0, true},
  };
  hipError_t e = hipSuccess;
  for (auto& it : items) {
    if (it.count == 0) continue;
    const size_t one = (size_t)(it.rows ? it.rows : 1) * it.cols * L->es;
    const size_t bytes = one * it.count;
    if (alloc_weight(it.dst, bytes) != hipSuccess) {
      free_layer(L);
      return fail(LLAMA_ERR_OUT_OF_MEMORY, "hipMalloc of %zu bytes for weights failed", bytes);
    }
    for (int m = 0; m < it.count && e == hipSuccess; ++m) {
      const char* src = (const char*)it.src + m * one;
      char* dst = (char*)*it.dst + m * one;
      if (it.tiled && it.rows)
        e = llk::launch_tile_weight(src, it.rows, it.cols, it.inter, dst, s);
      else
        e = hipMemcpyAsync(dst, src, one, hipMemcpyDeviceToDevice, s);
    }
    if (e != hipSuccess) {
      free_layer(L);
      return hip_fail(e, "weight copy");
    }
  }

  if (shared_rope) {
    L->rope = shared_rope;
    L->owns_rope = false;
    e = hipStreamSynchronize(s);  // the weight copies read the caller's buffers
    if (e != hipSuccess) {
      free_layer(L);
      return hip_fail(e, "weight copy");
    }
    *out = L;
    return LLAMA_OK;
  }
  // RoPE table: angles and cos/sin in double precision, stored as float
  const int half = c.head_dim / 2;
  const size_t n = (size_t)c.max_position_embeddings * half;
  std::vector<double> freq(half);
  for (int i = 0; i < half; ++i) freq[i] = rope_freq(&c, i);
  std::vector<float2> table(n);
  for (size_t p = 0; p < (size_t)c.max_position_embeddings; ++p)
    for (int i = 0; i < half; ++i) {
      const double a = (double)p * freq[i];
      table[p * half + i] = make_float2((float)std::cos(a), (float)std::sin(a));
    }
  if (hipMalloc((void**)&L->rope, n * sizeof(float2)) != hipSuccess) {
    free_layer(L);
    return fail(LLAMA_ERR_OUT_OF_MEMORY, "hipMalloc of the RoPE table failed");
  }
  e = hipMemcpyAsync(L->rope, table.data(), n * sizeof(float2), hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);  // `table` is freed on return
  if (e != hipSuccess) {
    free_layer(L);
    return hip_fail(e, "RoPE table upload");
  }
  *out = L;
  return LLAMA_OK;
}

}  // namespace

extern "C" {

llama_status llama_layer_create(const llama_layer_config* config, const llama_layer_weights* w,
                                void* stream, llama_layer** out) {
  return create_layer(config, w, stream, nullptr, out);
}

size_t llama_layer_workspace_bytes(const llama_layer* L, int32_t num_tokens, int32_t num_seqs,
                                   int32_t max_seq_len) {
  if (!L || num_tokens <= 0 || num_seqs <= 0 || max_seq_len <= 0) return 0;
  return carve(L, num_tokens, num_seqs, max_seq_len).total;
}

llama_status llama_layer_workspace_tensor(const llama_layer* L, int32_t T, int32_t B, int32_t max_seq_len,
                                          const char* name, size_t* offset, size_t* bytes) {
  if (!L || !name || !offset || !bytes || T <= 0 || B <= 0 || max_seq_len <= 0)
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "bad arguments");
  Workspace w = carve(L, T, B, max_seq_len);
  const llama_layer_config& c = L->cfg;
  struct {
    const char* n;
    size_t off, sz;
  } t[] = {
      {"h", w.h, (size_t)T * c.hidden_size * L->es},
      {"qkv", w.qkv, (size_t)T * L->qkv_n * L->es},
      {"attn", w.attn, (size_t)T * c.num_attention_heads * c.head_dim * L->es},
      {"h2", w.h2, (size_t)T * c.hidden_size * L->es},
      {"act", w.act, L->E ? 0 : (size_t)T * c.intermediate_size * L->es},
      {"router_logits", w.logits, (size_t)T * L->E * sizeof(float)},
      {"topk_ids", w.ids, (size_t)T * L->topk * sizeof(int)},
      {"topk_weights", w.wts, (size_t)T * L->topk * sizeof(float)},
      {"moe_sorted", w.sorted, (size_t)T * L->topk * sizeof(int)},
      {"moe_act", w.mact, (size_t)T * L->topk * L->moe_I * L->es},
      {"moe_part", w.mpart, (size_t)T * L->topk * c.hidden_size * L->es},
  };
  for (auto& x : t)
    if (std::strcmp(x.n, name) == 0 && x.sz > 0) {
      *offset = x.off;
      *bytes = x.sz;
      return LLAMA_OK;
    }
  return fail(LLAMA_ERR_INVALID_ARGUMENT, "unknown workspace tensor %s", name);
}

llama_status llama_layer_rope_table(const llama_layer* L, const void** table, int32_t* num_positions,
                                    int32_t* pairs) {
  if (!L || !table || !num_positions || !pairs) return fail(LLAMA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  *table = L->rope;
  *num_positions = L->cfg.max_position_embeddings;
  *pairs = L->cfg.head_dim / 2;
  return LLAMA_OK;
}

}  // extern "C"

namespace {

// Hand-over between the layers of a stack: the input hidden state may arrive
// as the previous layer's down_proj split-K partials (fp32 planes in the
// workspace, summed and rounded by this layer's input norm exactly as the
// previous layer's reduce would have), and the layer may leave its own
// down_proj partials there instead of reducing them into hidden_out.
struct StackLink {
  const float* in_part = nullptr;  // S fp32 planes [in_S][T][H], or NULL: read `hidden`
  int in_S = 0;
  bool keep_down_part = false;     // leave down_proj's partials (when it makes them)
  int out_S = 0;                   // set: planes left (0: hidden_out was written)
};

llama_status forward_impl(llama_layer* L, const void* hidden, const void* residual, const int32_t* positions,
                          int32_t T, const llama_kv_cache* kv, const int32_t* block_table, int32_t max_blocks,
                          const int32_t* seq_lens, const int32_t* query_start_loc, int32_t B,
                          int32_t max_seq_len, void* hidden_out, void* residual_out, void* workspace,
                          void* stream, StackLink* link = nullptr) {
  if (!L) return fail(LLAMA_ERR_INVALID_ARGUMENT, "layer is NULL");
  if (!hidden || !positions || !kv || !kv->k || !kv->v || !block_table || !seq_lens || !hidden_out ||
      !residual_out || !workspace)
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  if (T <= 0 || B <= 0) return fail(LLAMA_ERR_INVALID_ARGUMENT, "num_tokens %d and num_seqs %d must be positive", T, B);
  if (!query_start_loc && T % B != 0)
    return fail(LLAMA_ERR_INVALID_ARGUMENT,
                "num_tokens %d must be a multiple of num_seqs %d when query_start_loc is NULL", T, B);
  if (query_start_loc && T < B)
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "num_tokens %d < num_seqs %d: every sequence needs a query row", T, B);
  // T == B: one query row per sequence (decode), whatever query_start_loc says
  const bool decode = T == B;
  const bool mixed = query_start_loc && !decode;
  if (mixed && B > llk::kMaxMappedSeqs)
    return fail(LLAMA_ERR_UNSUPPORTED, "num_seqs %d above %d with query_start_loc", B, llk::kMaxMappedSeqs);
  const int q_len = mixed ? 1 : T / B;  // a lower bound on every sequence's query rows
  const llama_layer_config& c = L->cfg;
  if (max_seq_len < q_len || max_seq_len > c.max_position_embeddings)
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "max_seq_len %d outside [%d, %d]", max_seq_len, q_len,
                c.max_position_embeddings);
  if (max_blocks <= 0 || (int64_t)max_blocks * 16 < max_seq_len)
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "max_blocks_per_seq %d cannot hold max_seq_len %d", max_blocks,
                max_seq_len);
  if (kv->num_blocks <= 0) return fail(LLAMA_ERR_INVALID_ARGUMENT, "kv_cache.num_blocks must be positive");
  if (hidden_out == residual_out) return fail(LLAMA_ERR_INVALID_ARGUMENT, "hidden_out aliases residual_out");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0)
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  if (!aligned16(hidden) || (residual && !aligned16(residual)) || !aligned16(hidden_out) ||
      !aligned16(residual_out) || !aligned16(kv->k) || !aligned16(kv->v))
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "activation and cache pointers must be 16-byte aligned");

  hipStream_t s = (hipStream_t)stream;
  const Workspace w = carve(L, T, B, max_seq_len);
  char* ws = (char*)workspace;
  if (debug_checks()) {
    const llama_status st = check_metadata(L, w, ws, positions, T, kv, block_table, max_blocks, seq_lens,
                                           decode ? nullptr : query_start_loc, B, max_seq_len, s);
    if (st != LLAMA_OK) return st;
  }
  void* h = ws + w.h;
  void* qkv = ws + w.qkv;
  void* attn = ws + w.attn;
  void* h2 = ws + w.h2;
  void* act = ws + w.act;
  float* part = (float*)(ws + w.part);
  const int H = c.hidden_size, I = c.intermediate_size, nq = c.num_attention_heads,
            nkv = c.num_key_value_heads, d = c.head_dim;
  const int dt = L->dtype;

  Marker mk(L, s);
  hipError_t e;
  llk::SeqMap map;
  map.q_len = mixed ? 0 : T / B;
  if (mixed) {
    const int qw = dt == LLAMA_DTYPE_BF16 && llk::prefill_attention_supported(nq, nkv, d)
                       ? llk::prefill_tile_rows(nq, nkv, d)
                       : 16;  // the generic kernel reads only the row map
    map.seq_of = (const int*)(ws + w.seq_of);
    map.tiles = (const int4*)(ws + w.tiles);
    map.ntiles = (const int*)(ws + w.ntiles);
    map.tile_cap = T / qw + B;
    // with the matrix-core prefill kernel, sequences of one query row go to
    // the decode kernel instead of a 1-row query tile
    int* dec = nullptr;
    if (split_prefill(L)) {
      dec = (int*)(ws + w.dec);
      map.dec = dec;
      map.ndec = (const int*)(ws + w.ndec);
      map.dec_cap = B;
    }
    e = llk::launch_batch_map(query_start_loc, B, T, qw, (int*)(ws + w.seq_of), (int4*)(ws + w.tiles),
                              w.tile_cap, (int*)(ws + w.ntiles), dec, dec ? (int*)(ws + w.ndec) : nullptr, s);
    if (e != hipSuccess) return hip_fail(e, "batch_map");
    mk.mark("batch_map");
  }
  if (link) link->out_S = 0;
  if (link && link->in_part) {
    if (!residual) return fail(LLAMA_ERR_INVALID_ARGUMENT, "a hidden state passed as partials needs a residual");
    e = llk::launch_add_rmsnorm(dt, nullptr, residual, L->w_in, c.rms_norm_eps, T, H, h, residual_out, s,
                                link->in_part, link->in_S, true);
  } else {
    e = llk::launch_add_rmsnorm(dt, hidden, residual, L->w_in, c.rms_norm_eps, T, H, h, residual_out, s);
  }
  if (e != hipSuccess) return hip_fail(e, "input_layernorm");
  mk.mark("input_layernorm");
  float* gp = (float*)(ws + w.gpart);
  float* tp = (float*)(ws + w.tpart);
  llk::QkNorm qkn;
  if (c.qk_norm) {
    qkn.q = L->w_qn;
    qkn.k = L->w_kn;
    qkn.eps = c.rms_norm_eps;
  }
  // a decode batch on the matrix-core decode kernel: its workgroups form
  // their rows' q, k, v from the projection's partials, rotate them and
  // write the cache slot themselves (no separate RoPE / KV-write launch)
  llk::DecodeRope fuse;
  const bool fused_rope = w.skinny && decode && dt == LLAMA_DTYPE_BF16;
  if (w.skinny) {
    e = llk::launch_skinny(h, L->w_qkv, T, L->qkv_n, H, llk::kEpiPartial, w.pq, gp, s, L->wlayout);
    if (e != hipSuccess) return hip_fail(e, "qkv_proj");
    mk.mark("qkv_proj");
    if (fused_rope) {
      fuse.part = gp;
      fuse.S = w.pq.splits;
      fuse.table = L->rope;
      fuse.qkv = qkv;
      fuse.qkn = qkn;
    } else {
      e = llk::launch_rope_kv(dt, qkv, T, positions, L->rope, nq, nkv, d, block_table, max_blocks, map, kv->k,
                              kv->v, s, gp, w.pq.splits, qkn);
    }
  } else {
    e = llk::launch_linear(dt, h, L->w_qkv, T, L->qkv_n, H, llk::kEpiStore, qkv, s, L->wlayout, tp, w.tpart_bytes);
    if (e != hipSuccess) return hip_fail(e, "qkv_proj");
    mk.mark("qkv_proj");
    e = llk::launch_rope_kv(dt, qkv, T, positions, L->rope, nq, nkv, d, block_table, max_blocks, map, kv->k,
                            kv->v, s, nullptr, 0, qkn);
  }
  if (e != hipSuccess) return hip_fail(e, "rope_kv_write");
  if (!fused_rope) mk.mark("rope_kv_write");
  hipEvent_t mid = w.plan.parts > 1 ? mk.extra() : nullptr;
  e = llk::launch_attention(dt, qkv, L->qkv_n, T, positions, nq, nkv, d, kv->k, kv->v, block_table, max_blocks,
                            map, decode, w.plan, part, (int*)(ws + w.row_parts), attn, s, mid,
                            fused_rope ? &fuse : nullptr);
  if (e != hipSuccess) return hip_fail(e, "attention");
  if (mid) mk.list->push_back({"attention", mid});
  mk.mark(w.plan.parts > 1 ? "attention_combine" : "attention");
  if (w.skinny) {
    if (w.o_wsplit) {
      // o_proj adds its final rows to the residual stream in place; then a
      // plain norm of the new residual
      e = llk::launch_skinny_wave_split(attn, L->w_o, T, H, nq * d, llk::kEpiAdd, residual_out, s, L->wlayout);
      if (e != hipSuccess) return hip_fail(e, "o_proj");
      mk.mark("o_proj_residual");
      e = llk::launch_add_rmsnorm(dt, residual_out, nullptr, L->w_post, c.rms_norm_eps, T, H, h2, nullptr, s);
    } else {
      // o_proj as split-K partials; the post-attention norm kernel sums them,
      // adds the residual and stores the new residual before normalising
      e = llk::launch_skinny(attn, L->w_o, T, H, nq * d, llk::kEpiPartial, w.po, gp, s, L->wlayout);
      if (e != hipSuccess) return hip_fail(e, "o_proj");
      mk.mark("o_proj");
      e = llk::launch_add_rmsnorm(dt, nullptr, residual_out, L->w_post, c.rms_norm_eps, T, H, h2, residual_out, s,
                                  gp, w.po.splits);
    }
    if (e != hipSuccess) return hip_fail(e, "post_attention_layernorm");
    mk.mark("post_attention_layernorm");
    if (L->E) return moe_block(L, w, ws, h2, T, hidden_out, s, mk);
    if (w.pg.splits > 1) {
      e = llk::launch_skinny(h2, L->w_gu, T, 2 * I, H, llk::kEpiPartial, w.pg, gp, s, L->wlayout);
      if (e != hipSuccess) return hip_fail(e, "gate_up_proj");
      mk.mark("gate_up");
      e = llk::launch_silu_reduce(gp, w.pg.splits, T, 2 * I, act, s);
      if (e != hipSuccess) return hip_fail(e, "gate_up SiluAndMul reduce");
      mk.mark("gate_up_silu_reduce");
    } else {
      e = llk::launch_skinny(h2, L->w_gu, T, I, H, llk::kEpiSiluMul, w.pg, act, s, L->wlayout);
      if (e != hipSuccess) return hip_fail(e, "gate_up_proj");
      mk.mark("gate_up_silu");
    }
    if (w.d_wsplit) {
      e = llk::launch_skinny_wave_split(act, L->w_down, T, H, I, llk::kEpiStore, hidden_out, s, L->wlayout);
      if (e != hipSuccess) return hip_fail(e, "down_proj");
      mk.mark("down_proj");
      return LLAMA_OK;
    }
    e = llk::launch_skinny(act, L->w_down, T, H, I, llk::kEpiPartial, w.pd, gp, s, L->wlayout);
    if (e != hipSuccess) return hip_fail(e, "down_proj");
    mk.mark("down_proj");
    if (link && link->keep_down_part) {  // the next layer's input norm (or the final norm) sums them
      link->out_S = w.pd.splits;
      return LLAMA_OK;
    }
    e = llk::launch_splitk_reduce(gp, w.pd.splits, T, H, hidden_out, s);
    if (e != hipSuccess) return hip_fail(e, "down_proj reduce");
    mk.mark("down_proj_reduce");
    return LLAMA_OK;
  }
  e = llk::launch_linear(dt, attn, L->w_o, T, H, nq * d, llk::kEpiAdd, residual_out, s, L->wlayout, tp,
                         w.tpart_bytes);
  if (e != hipSuccess) return hip_fail(e, "o_proj");
  mk.mark("o_proj_residual");
  e = llk::launch_add_rmsnorm(dt, residual_out, nullptr, L->w_post, c.rms_norm_eps, T, H, h2, nullptr, s);
  if (e != hipSuccess) return hip_fail(e, "post_attention_layernorm");
  mk.mark("post_attention_layernorm");
  if (L->E) return moe_block(L, w, ws, h2, T, hidden_out, s, mk);
  e = llk::launch_linear(dt, h2, L->w_gu, T, I, H, llk::kEpiSiluMul, act, s, L->wlayout, tp, w.tpart_bytes);
  if (e != hipSuccess) return hip_fail(e, "gate_up_proj");
  mk.mark("gate_up_silu");
  e = llk::launch_linear(dt, act, L->w_down, T, H, I, llk::kEpiStore, hidden_out, s, L->wlayout, tp,
                         w.tpart_bytes);
  if (e != hipSuccess) return hip_fail(e, "down_proj");
  mk.mark("down_proj");
  return LLAMA_OK;
}

}  // namespace

extern "C" {

llama_status llama_layer_forward(llama_layer* L, const void* hidden, const void* residual,
                                 const int32_t* positions, int32_t T, const llama_kv_cache* kv,
                                 const int32_t* block_table, int32_t max_blocks, const int32_t* seq_lens,
                                 const int32_t* query_start_loc, int32_t B, int32_t max_seq_len,
                                 void* hidden_out, void* residual_out, void* workspace, void* stream) {
  return forward_impl(L, hidden, residual, positions, T, kv, block_table, max_blocks, seq_lens, query_start_loc, B,
                      max_seq_len, hidden_out, residual_out, workspace, stream);
}

llama_status llama_layer_forward_noalloc(llama_layer* L, const void* hidden, const void* residual,
                                         const int32_t* positions, int32_t T, const llama_kv_cache* kv,
                                         const int32_t* block_table, int32_t max_blocks, const int32_t* seq_lens,
                                         const int32_t* query_start_loc, int32_t B, int32_t max_seq_len,
                                         void* hidden_out, void* residual_out, void* stream) {
  if (!L) return fail(LLAMA_ERR_INVALID_ARGUMENT, "layer is NULL");
  if (T <= 0 || B <= 0 || max_seq_len <= 0)
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "num_tokens, num_seqs and max_seq_len must be positive");
  if (L->timing) return fail(LLAMA_ERR_INVALID_ARGUMENT, "per-kernel timing must be off (it creates events)");
  const size_t need = carve(L, T, B, max_seq_len).total;
  if (need > llk::kNoAllocScratchBytes)
    return fail(LLAMA_ERR_INVALID_ARGUMENT,
                "this call needs %zu bytes of workspace; the no-allocation forward holds at most %zu "
                "(use llama_layer_forward with a workspace)",
                need, llk::kNoAllocScratchBytes);
  if (L->scratch_err != hipSuccess) return hip_fail(L->scratch_err, "no-allocation scratch lookup");
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != L->device)
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "current device %d is not the layer's device %d", dev, L->device);
  void* scratch = llk::noalloc_scratch(L->device);
  if (!scratch) return fail(LLAMA_ERR_HIP, "no-allocation scratch of device %d not set up", L->device);
  return forward_impl(L, hidden, residual, positions, T, kv, block_table, max_blocks, seq_lens, query_start_loc, B,
                      max_seq_len, hidden_out, residual_out, scratch, stream);
}

void llama_layer_destroy(llama_layer* L) {
  if (!L) return;
  DeviceScope on(L->device);
  (void)hipDeviceSynchronize();
  free_layer(L);
}

llama_status llama_layer_set_timing(llama_layer* L, int32_t enable) {
  if (!L) return fail(LLAMA_ERR_INVALID_ARGUMENT, "layer is NULL");
  L->timing = enable != 0;
  return LLAMA_OK;
}

int32_t llama_layer_timing_read(llama_layer* L, const char** names, double* total_ms, int64_t* counts,
                                int32_t cap) {
  if (!L) {
    fail(LLAMA_ERR_INVALID_ARGUMENT, "layer is NULL");
    return -1;
  }
  for (auto& list : L->marks) {
    for (size_t i = 1; i < list.size(); ++i) {
      if (hipEventSynchronize(list[i].ev) != hipSuccess) continue;
      float ms = 0.f;
      if (hipEventElapsedTime(&ms, list[i - 1].ev, list[i].ev) != hipSuccess) continue;
      auto& tot = L->totals[list[i].name];
      tot.first += ms;
      tot.second += 1;
    }
    for (auto& m : list) L->event_pool.push_back(m.ev);
  }
  L->marks.clear();
  int32_t n = 0;
  for (auto& kv : L->totals) {
    if (n < cap) {
      if (names) names[n] = kv.first.c_str();  // valid until the next read
      if (total_ms) total_ms[n] = kv.second.first;
      if (counts) counts[n] = kv.second.second;
    }
    ++n;
  }
  static thread_local std::map<std::string, std::pair<double, int64_t>> last;
  last.swap(L->totals);  // keep name storage alive for the caller
  L->totals.clear();
  return n;
}

llama_status llama_op_linear(int32_t dtype, const void* x, const void* w, int32_t M, int32_t N, int32_t K,
                             int32_t epilogue, void* out, void* stream) {
  if (!x || !w || !out) return fail(LLAMA_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (M <= 0 || N <= 0 || K <= 0) return fail(LLAMA_ERR_INVALID_ARGUMENT, "sizes must be positive");
  if (epilogue < 0 || epilogue > 2) return fail(LLAMA_ERR_INVALID_ARGUMENT, "unknown epilogue %d", epilogue);
  if (dtype != LLAMA_DTYPE_BF16 && dtype != LLAMA_DTYPE_FP32)
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
  if (!aligned16(x) || !aligned16(w) || !aligned16(out))
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "pointers must be 16-byte aligned");
  if (dtype == LLAMA_DTYPE_BF16) {
    const int64_t wrows = epilogue == LLAMA_EPI_SILU_MUL ? 2 * (int64_t)N : N;
    if (K % 64 || wrows % 128)
      return fail(LLAMA_ERR_INVALID_ARGUMENT, "bf16 needs K %% 64 == 0 and weight rows %% 128 == 0");
  }
  hipError_t e = llk::launch_linear(dtype, x, w, M, N, K, epilogue, out, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "linear");
  return LLAMA_OK;
}

llama_status llama_diag_stream_read(const void* src, size_t bytes, int32_t workgroups, int32_t threads,
                                    int32_t nontemporal, void* sink, void* stream) {
  if (!src || !sink) return fail(LLAMA_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (bytes == 0 || bytes % 16 || !aligned16(src))
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "bytes must be a positive multiple of 16 and src 16-byte aligned");
  if (workgroups <= 0 || workgroups > (1 << 20) || threads < 64 || threads > 1024 || threads % 64)
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "workgroups in [1, 2^20], threads a multiple of 64 in [64, 1024]");
  hipError_t e = llk::launch_stream_read(src, bytes, workgroups, threads, sink, nontemporal != 0, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "stream_read");
  return LLAMA_OK;
}

llama_status llama_diag_block_read(const void* src, size_t src_bytes, const int32_t* block_ids, int32_t num_ids,
                                   int32_t block_bytes, int32_t workgroups, int32_t nontemporal, void* sink,
                                   void* stream) {
  if (!src || !block_ids || !sink) return fail(LLAMA_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (block_bytes < 1024 || block_bytes > 16384 || block_bytes % 1024 || !aligned16(src))
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "block_bytes a multiple of 1024 in [1024, 16384], src 16-byte aligned");
  if (num_ids < 0 || workgroups <= 0 || workgroups > (1 << 20) || src_bytes < (size_t)block_bytes)
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "num_ids >= 0, workgroups in [1, 2^20], src at least one block");
  hipError_t e = llk::launch_block_read(src, block_ids, num_ids, block_bytes, workgroups, sink, nontemporal != 0,
                                        (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "block_read");
  return LLAMA_OK;
}

llama_status llama_op_reorder_gate_up(const void* src, int32_t inter, int32_t K, void* dst, void* stream) {
  if (!src || !dst) return fail(LLAMA_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (inter <= 0 || K <= 0 || inter % 16 || K % 8)
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "needs intermediate %% 16 == 0 and K %% 8 == 0");
  if (!aligned16(src) || !aligned16(dst)) return fail(LLAMA_ERR_INVALID_ARGUMENT, "pointers must be 16-byte aligned");
  if (src == dst) return fail(LLAMA_ERR_INVALID_ARGUMENT, "dst aliases src");
  hipError_t e = llk::launch_reorder_gate_up(src, inter, K, dst, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "reorder_gate_up");
  return LLAMA_OK;
}

llama_status llama_op_add_rmsnorm(int32_t dtype, const void* x, const void* residual, const void* w, float eps,
                                  int32_t rows, int32_t hidden, void* normed, void* residual_out, void* stream) {
  if (!x || !w || !normed) return fail(LLAMA_ERR_INVALID_ARGUMENT, "NULL pointer");
  if (residual && !residual_out) return fail(LLAMA_ERR_INVALID_ARGUMENT, "residual needs residual_out");
  if (dtype != LLAMA_DTYPE_BF16 && dtype != LLAMA_DTYPE_FP32)
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "unknown dtype %d", dtype);
  const int vn = dtype == LLAMA_DTYPE_BF16 ? 8 : 4;
  if (rows <= 0 || hidden <= 0 || hidden % vn || hidden > 256 * 8 * vn)
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "hidden must be a multiple of %d and <= %d", vn, 256 * 8 * vn);
  if (!(eps > 0.f)) return fail(LLAMA_ERR_INVALID_ARGUMENT, "eps must be > 0");
  if (!aligned16(x) || !aligned16(w) || !aligned16(normed) || (residual && !aligned16(residual)) ||
      (residual_out && !aligned16(residual_out)))
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "pointers must be 16-byte aligned");
  hipError_t e = llk::launch_add_rmsnorm(dtype, x, residual, w, eps, rows, hidden, normed, residual_out,
                                         (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "add_rmsnorm");
  return LLAMA_OK;
}

// ---------------------------------------------------------------- stack ----

struct llama_stack {
  std::vector<llama_layer*> layers;
  void* w_final = nullptr;  // final norm weight [H]
  float eps = 0.f;
  int dtype = 0;
  size_t es = 2;
  int H = 0;
};

struct llama_graph {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  int device = -1;
};

namespace {

void free_stack(llama_stack* S) {
  if (!S) return;
  for (llama_layer* L : S->layers) free_layer(L);
  if (S->w_final) (void)hipFree(S->w_final);
  delete S;
}

// the stack's own workspace: the (hidden, residual) pair the layers update
// in place, after the region one layer forward needs
struct StackWs {
  size_t layer, h, r, total;
};
StackWs carve_stack(const llama_stack* S, int T, int B, int max_seq_len) {
  StackWs w{};
  w.layer = 0;
  size_t off = align256(carve(S->layers[0], T, B, max_seq_len).total);
  w.h = off;
  off += align256((size_t)T * S->H * S->es);
  w.r = off;
  off += align256((size_t)T * S->H * S->es);
  w.total = off;
  return w;
}

}  // namespace

llama_status llama_stack_create(const llama_layer_config* config, int32_t num_layers,
                                const llama_layer_weights* weights, const void* final_norm, void* stream,
                                llama_stack** out) {
  if (!out) return fail(LLAMA_ERR_INVALID_ARGUMENT, "out is NULL");
  *out = nullptr;
  if (!config || !weights || !final_norm) return fail(LLAMA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  if (num_layers <= 0) return fail(LLAMA_ERR_INVALID_ARGUMENT, "num_layers %d must be positive", num_layers);
  llama_status st = llama_layer_config_validate(config);
  if (st != LLAMA_OK) return st;
  llama_stack* S = new llama_stack();
  S->dtype = config->dtype;
  S->es = config->dtype == LLAMA_DTYPE_BF16 ? 2 : 4;
  S->H = config->hidden_size;
  S->eps = config->rms_norm_eps;
  for (int l = 0; l < num_layers; ++l) {
    llama_layer* L = nullptr;
    // one RoPE table for the whole stack (the first layer builds it)
    st = create_layer(config, &weights[l], stream, l == 0 ? nullptr : S->layers[0]->rope, &L);
    if (st != LLAMA_OK) {
      free_stack(S);
      return st;
    }
    S->layers.push_back(L);
  }
  const size_t bytes = (size_t)S->H * S->es;
  if (hipMalloc(&S->w_final, bytes) != hipSuccess) {
    free_stack(S);
    return fail(LLAMA_ERR_OUT_OF_MEMORY, "hipMalloc of the final norm weight failed");
  }
  hipError_t e = hipMemcpyAsync(S->w_final, final_norm, bytes, hipMemcpyDeviceToDevice, (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) {
    free_stack(S);
    return hip_fail(e, "final norm copy");
  }
  *out = S;
  return LLAMA_OK;
}

size_t llama_stack_workspace_bytes(const llama_stack* S, int32_t T, int32_t B, int32_t max_seq_len) {
  if (!S || T <= 0 || B <= 0 || max_seq_len <= 0) return 0;
  return carve_stack(S, T, B, max_seq_len).total;
}

llama_status llama_stack_forward(llama_stack* S, const void* hidden, const int32_t* positions, int32_t T,
                                 const llama_kv_cache* kv_caches, const int32_t* block_table, int32_t max_blocks,
                                 const int32_t* seq_lens, const int32_t* query_start_loc, int32_t B,
                                 int32_t max_seq_len, void* out, void* workspace, void* stream) {
  if (!S) return fail(LLAMA_ERR_INVALID_ARGUMENT, "stack is NULL");
  if (!hidden || !kv_caches || !out || !workspace) return fail(LLAMA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  if (T <= 0 || B <= 0 || max_seq_len <= 0)
    return fail(LLAMA_ERR_INVALID_ARGUMENT, "num_tokens, num_seqs and max_seq_len must be positive");
  if (!aligned16(out)) return fail(LLAMA_ERR_INVALID_ARGUMENT, "out must be 16-byte aligned");
  const StackWs w = carve_stack(S, T, B, max_seq_len);
  char* ws = (char*)workspace;
  void* h = ws + w.h;
  void* r = ws + w.r;
  // a layer's down_proj split-K partials (decode) stay in the layer workspace
  // and the next layer's input norm -- or the final norm -- sums them: the
  // same sums, rounded the same way, one launch fewer per layer
  const float* part = (const float*)(ws + w.layer + carve(S->layers[0], T, B, max_seq_len).gpart);
  int part_S = 0;
  for (size_t l = 0; l < S->layers.size(); ++l) {
    // layer 0 reads the input with no residual; later layers update (h, r) in place
    const void* hin = l == 0 ? hidden : h;
    const void* rin = l == 0 ? nullptr : r;
    StackLink link;
    link.in_part = part_S > 0 ? part : nullptr;
    link.in_S = part_S;
    link.keep_down_part = true;
    const llama_status st = forward_impl(S->layers[l], hin, rin, positions, T, &kv_caches[l], block_table,
                                         max_blocks, seq_lens, query_start_loc, B, max_seq_len, h, r, ws + w.layer,
                                         stream, &link);
    if (st != LLAMA_OK) return st;
    part_S = link.out_S;
  }
  // final norm of hidden + residual
  hipError_t e = part_S > 0 ? llk::launch_add_rmsnorm(S->dtype, nullptr, r, S->w_final, S->eps, T, S->H, out, nullptr,
                                                      (hipStream_t)stream, part, part_S, true)
                            : llk::launch_add_rmsnorm(S->dtype, h, r, S->w_final, S->eps, T, S->H, out, nullptr,
                                                      (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "final norm");
  return LLAMA_OK;
}

void llama_stack_destroy(llama_stack* S) {
  if (!S) return;
  DeviceScope on(S->layers.empty() ? -1 : S->layers[0]->device);
  (void)hipDeviceSynchronize();
  free_stack(S);
}

llama_status llama_stack_graph_create(llama_stack* S, const void* hidden, const int32_t* positions, int32_t T,
                                      const llama_kv_cache* kv_caches, const int32_t* block_table,
                                      int32_t max_blocks, const int32_t* seq_lens, const int32_t* query_start_loc,
                                      int32_t B, int32_t max_seq_len, void* out, void* workspace, void* stream,
                                      llama_graph** graph_out) {
  if (!graph_out) return fail(LLAMA_ERR_INVALID_ARGUMENT, "graph_out is NULL");
  *graph_out = nullptr;
  if (!S) return fail(LLAMA_ERR_INVALID_ARGUMENT, "stack is NULL");
  if (!stream) return fail(LLAMA_ERR_INVALID_ARGUMENT, "capture needs a stream other than the default stream");
  for (llama_layer* L : S->layers)
    if (L->timing) return fail(LLAMA_ERR_INVALID_ARGUMENT, "turn per-kernel timing off before capturing");
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipStreamBeginCapture(s, hipStreamCaptureModeRelaxed);
  if (e != hipSuccess) return hip_fail(e, "hipStreamBeginCapture");
  const llama_status st = llama_stack_forward(S, hidden, positions, T, kv_caches, block_table, max_blocks, seq_lens,
                                              query_start_loc, B, max_seq_len, out, workspace, stream);
  std::string err = st != LLAMA_OK ? g_err : std::string();
  hipGraph_t g = nullptr;
  e = hipStreamEndCapture(s, &g);  // always: leaves the stream out of capture mode
  if (st != LLAMA_OK) {
    if (g) (void)hipGraphDestroy(g);
    return fail(st, "%s", err.c_str());
  }
  if (e != hipSuccess) return hip_fail(e, "hipStreamEndCapture");
  llama_graph* G = new llama_graph();
  G->graph = g;
  G->device = S->layers.empty() ? -1 : S->layers[0]->device;
  e = hipGraphInstantiate(&G->exec, g, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    (void)hipGraphDestroy(g);
    delete G;
    return hip_fail(e, "hipGraphInstantiate");
  }
  *graph_out = G;
  return LLAMA_OK;
}

llama_status llama_graph_launch(llama_graph* G, void* stream) {
  if (!G || !G->exec) return fail(LLAMA_ERR_INVALID_ARGUMENT, "graph is NULL");
  hipError_t e = hipGraphLaunch(G->exec, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "hipGraphLaunch");
  return LLAMA_OK;
}

void llama_graph_destroy(llama_graph* G) {
  if (!G) return;
  DeviceScope on(G->device);
  (void)hipDeviceSynchronize();
  if (G->exec) (void)hipGraphExecDestroy(G->exec);
  if (G->graph) (void)hipGraphDestroy(G->graph);
  delete G;
}

}  // extern "C"
