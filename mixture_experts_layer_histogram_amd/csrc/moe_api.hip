// C-ABI entry points: argument validation, workspace carving and the order of
// kernel launches.  Nothing here allocates, frees or synchronises.
#include "moe_internal.h"

#include <math.h>

#include <algorithm>
#include <mutex>

namespace moe {

static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }


Workspace workspace_layout(const moe_config& c) {
  Workspace W{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  const size_t N = (size_t)c.n_tokens, E = (size_t)c.n_experts, k = (size_t)c.top_k;
  const size_t d = (size_t)c.d_model, F = (size_t)c.d_ff, Fs = (size_t)(c.d_ff_shared > 0 ? c.d_ff_shared : 0);
  const size_t slots = N * k;
  const size_t rows = (size_t)expert_rows(c);   // expert-ordered buffer rows
  const size_t esz = c.dtype == MOE_BF16 ? 2 : 4;

  // top-k blocking: L lanes per token, 4 waves, iters rounds per block
  const int L = topk_lanes(c.n_experts);
  const int per_iter = 4 * (64 / L);
  long long iters = ((long long)N + (long long)per_iter * 1024 - 1) / ((long long)per_iter * 1024);
  if (iters < 1) iters = 1;
  if (iters > 64) iters = 64;
  W.topk_iters = (int)iters;
  W.topk_tokens_per_block = per_iter * W.topk_iters;
  W.topk_blocks = (int)((N + W.topk_tokens_per_block - 1) / W.topk_tokens_per_block);
  W.hist_blocks_n = (int)((slots + kHistSlotsPerBlock - 1) / kHistSlotsPerBlock);
  // fused router: groups of 16 tokens (E <= 16) or 64, at most 1024 workgroups
  const long long rtm = c.n_experts <= 16 ? 16 : 64;
  W.route_blocks = (int)std::min<long long>(std::max<long long>(((long long)N + rtm - 1) / rtm, 1), 1024);
  W.max_tiles = grouped_gemm_max_tiles((int)(rows > slots ? rows : slots), (int)E);
  W.max_tiles_small = grouped_gemm_max_small_tiles((int)(rows > slots ? rows : slots), (int)E);
  W.max_tiles_sh = Fs ? grouped_gemm_max_tiles((int)N, 1) : 0;
  W.max_tiles_sh_small = Fs ? grouped_gemm_max_small_tiles((int)N, 1) : 0;

  W.probsum_part = take((size_t)std::max(W.topk_blocks, W.route_blocks) * E * sizeof(double));
  W.hist_rank = take(slots * 4);
  W.hist_blocks = take(E * (size_t)(W.hist_blocks_n > 0 ? W.hist_blocks_n : 1) * 4);
  W.tiles = take((4 + 8 * (size_t)W.max_tiles) * 4);
  W.tiles_small = take((4 + 8 * (size_t)W.max_tiles_small) * 4);
  W.tiles_sh = take((4 + 8 * (size_t)W.max_tiles_sh) * 4);
  W.tiles_sh_small = take((4 + 8 * (size_t)W.max_tiles_sh_small) * 4);
  W.gemm_partials = take(c.dtype == MOE_BF16 ? grouped_gemm_partials_bytes() : 0);
  W.logits = take(N * E * 4);
  W.topk_idx = take(slots * 4);
  W.gates = take(slots * 4);
  W.probsum = take(E * 4);
  W.counts = take(E * 4);
  W.offsets = take((E + 1) * 4);
  W.perm = take(rows * 4);
  W.slot_pos = take(slots * 4);
  W.drop_count = take(8);
  W.aux = take(4);
  W.signs = take(E);
  W.x_perm = take(rows * d * esz);
  W.h = take(rows * F * esz);
  W.y = take(rows * d * esz);
  W.h_sh = take(N * Fs * esz);
  W.y_sh = take(Fs ? N * d * esz : 0);
  W.total = off;
  return W;
}

// measurement probes (probe.hip)
hipError_t launch_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t s);
hipError_t launch_mfma_probe(const void* operands, long long iters, float* sink, hipStream_t s);
int probe_grid();

}  // namespace moe

using namespace moe;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

moe_status check_config(const moe_config* c) {
  if (!c) return MOE_ERR_ARG;
  if (c->n_tokens < 0 || c->n_tokens > (1ll << 24)) return MOE_ERR_ARG;
  if (c->d_model <= 0 || c->d_ff <= 0 || c->d_ff_shared < 0) return MOE_ERR_ARG;
  if (c->n_experts < 1 || c->n_experts > kMaxExperts) return MOE_ERR_ARG;
  if (c->top_k < 1 || c->top_k > c->n_experts || c->top_k > kMaxTopK) return MOE_ERR_ARG;
  if (c->act != MOE_ACT_SWIGLU && c->act != MOE_ACT_GELU) return MOE_ERR_ARG;
  if (c->gate_rule < MOE_GATE_TOPK_SOFTMAX || c->gate_rule > MOE_GATE_SWITCH_TOP1) return MOE_ERR_ARG;
  if (c->dtype != MOE_F32 && c->dtype != MOE_BF16) return MOE_ERR_ARG;
  if (isnan(c->capacity_factor)) return MOE_ERR_ARG;
  if (c->gate_rule == MOE_GATE_SWITCH_TOP1 && c->top_k != 1) return MOE_ERR_ARG;
  if (c->capacity_layout != MOE_CAPACITY_PACKED && c->capacity_layout != MOE_CAPACITY_PADDED) return MOE_ERR_ARG;
  if (c->capacity_priority != MOE_PRIORITY_SLOT && c->capacity_priority != MOE_PRIORITY_CHOICE) return MOE_ERR_ARG;
  if (c->capacity_layout == MOE_CAPACITY_PADDED && !(c->capacity_factor > 0.f)) return MOE_ERR_ARG;
  if (expert_rows(*c) >= (1ll << 31)) return MOE_ERR_UNSUPPORTED;
  if (c->ffn_bias && c->act != MOE_ACT_GELU) return MOE_ERR_UNSUPPORTED;
  if (c->dtype == MOE_BF16) {
    if (c->d_model % 64 || c->d_ff % 64 || c->d_ff_shared % 64) return MOE_ERR_UNSUPPORTED;
  }
  const long long slots = c->n_tokens * (long long)c->top_k;
  if (slots * (long long)c->d_model >= (1ll << 40)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

#define MOE_TRY(expr)                       \
  do {                                      \
    moe_status _st = (expr);                \
    if (_st != MOE_OK) return _st;          \
  } while (0)

#define MOE_HIP(expr)                       \
  do {                                      \
    hipError_t _e = (expr);                 \
    if (_e != hipSuccess) return MOE_ERR_HIP; \
  } while (0)

char* wsp(void* ws, size_t off) { return static_cast<char*>(ws) + off; }

// Internal step bodies (validated arguments).
GroupedGemmArgs gemm_args(const moe_config& c, const Workspace& W, void* ws, bool shared) {
  GroupedGemmArgs g{};
  g.dtype = c.dtype;
  g.partials = reinterpret_cast<float*>(wsp(ws, W.gemm_partials));
  if (shared) {
    g.n_seg = 1;
    g.max_rows = (int)c.n_tokens;
    g.tiles = reinterpret_cast<int32_t*>(wsp(ws, W.tiles_sh));
    g.max_tiles = W.max_tiles_sh;
    g.tiles_small = reinterpret_cast<int32_t*>(wsp(ws, W.tiles_sh_small));
    g.max_tiles_small = W.max_tiles_sh_small;
  } else {
    g.n_seg = c.n_experts;
    g.max_rows = (int)expert_rows(c);
    g.tiles = reinterpret_cast<int32_t*>(wsp(ws, W.tiles));
    g.max_tiles = W.max_tiles;
    g.tiles_small = reinterpret_cast<int32_t*>(wsp(ws, W.tiles_small));
    g.max_tiles_small = W.max_tiles_small;
  }
  return g;
}

moe_status do_route(const moe_config& c, const Workspace& W, const void* x, const void* w_router,
                    const float* logit_bias, const float* sel_bias, const float* logits_in, float* logits,
                    int32_t* topk_idx, float* gates, float* probsum, void* ws, hipStream_t s) {
  const float* zin = logits_in;
  float* zout = nullptr;
  if (!zin && route_fused_supported(c) && (ws != nullptr || probsum == nullptr)) {
    // router GEMM, softmax, top-k and gates in one launch
    MOE_HIP(launch_route_fused(c, W, x, w_router, logit_bias, sel_bias, logits, topk_idx, gates,
                               ws ? reinterpret_cast<float*>(wsp(ws, W.probsum_part)) : nullptr, probsum, s));
    return MOE_OK;
  }
  if (!zin) {
    // Wide routers (E a multiple of 64) run on the grouped GEMM with fp32 output; it needs the
    // scratch part of the workspace.  Narrow ones use the router kernel, which needs none.
    const bool wide = c.dtype == MOE_BF16 && c.n_experts % 64 == 0 && ws != nullptr && aligned16(logits) &&
                      aligned16(logit_bias);
    if (wide && c.n_tokens > 0) {
      GroupedGemmArgs g = gemm_args(c, W, ws, false);
      g.mode = MODE_LOGITS;
      g.n_seg = 1;
      g.max_rows = (int)c.n_tokens;
      g.K = c.d_model;
      g.Nn = c.n_experts;
      g.a = x;
      g.offsets = nullptr;
      g.w = w_router;
      g.out_f32 = logits;
      g.bias_f32 = logit_bias;
      if (topk_from_parts_supported(c)) {
        // the selection completes the logits from the GEMM's K-part partials (its fix-up
        // pass folded into the top-k kernel: one launch and one pass over the logits fewer)
        g.no_fixup = true;
        MOE_HIP(launch_grouped_gemm(g, s));
        MOE_HIP(launch_topk_from_parts(c, W, logits_parts(g), sel_bias, topk_idx, gates,
                                       reinterpret_cast<float*>(wsp(ws, W.probsum_part)), probsum, s));
        return MOE_OK;
      }
      MOE_HIP(launch_grouped_gemm(g, s));
    } else {
      MOE_HIP(launch_router_gemm(c, x, w_router, logit_bias, logits, s));
    }
    zin = logits;
  } else if (logits && logits != logits_in) {
    zout = logits;
  }
  MOE_HIP(launch_topk(c, W, zin, zout, sel_bias, topk_idx, gates,
                      reinterpret_cast<float*>(wsp(ws, W.probsum_part)), probsum, s));
  return MOE_OK;
}

moe_status do_permute(const moe_config& c, const Workspace& W, const int32_t* topk_idx, const void* x,
                      int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* slot_pos,
                      int64_t* drop_count, void* x_perm, void* ws, hipStream_t s) {
  MOE_HIP(launch_permute(c, W, topk_idx, x, counts, offsets, perm, slot_pos, drop_count, x_perm,
                         reinterpret_cast<int32_t*>(wsp(ws, W.hist_rank)),
                         reinterpret_cast<int32_t*>(wsp(ws, W.hist_blocks)), s));
  return MOE_OK;
}

// `perm` != NULL: `a` is the token matrix and row r of the expert order is
// token perm[r] / top_k (the gather of the dispatch done inside the GEMM).
moe_status do_up(const moe_config& c, const Workspace& W, const void* a, const int32_t* offsets,
                 const void* w1, const void* w3, const void* b1, void* h, void* ws, hipStream_t s,
                 bool shared, const int32_t* perm = nullptr, void* pre = nullptr) {
  GroupedGemmArgs g = gemm_args(c, W, ws, shared);
  g.pre = pre;
  g.perm = perm;
  g.gather_k = c.top_k;
  g.a_rows = (int)c.n_tokens;
  const bool swiglu = shared || c.act == MOE_ACT_SWIGLU;
  g.mode = swiglu ? MODE_SWIGLU_UP : MODE_GELU_UP;
  g.K = c.d_model;
  g.Nn = shared ? c.d_ff_shared : c.d_ff;
  g.a = a;
  g.offsets = offsets;
  g.w = w1;
  g.w3 = swiglu ? w3 : nullptr;
  g.bias = (!shared && c.ffn_bias) ? b1 : nullptr;
  g.out = h;
  MOE_HIP(launch_grouped_gemm(g, s));
  return MOE_OK;
}

// fp8 experts: weights are E4M3 codes with per-row scales; up always gathers token rows.
moe_status do_up_fp8(const moe_config& c, const Workspace& W, const void* x, const int32_t* perm,
                     const int32_t* offsets, const uint8_t* w1q, const uint8_t* w3q, const float* s1,
                     const float* s3, const void* b1, void* h, void* ws, hipStream_t s) {
  GroupedGemmArgs g = gemm_args(c, W, ws, false);
  const bool swiglu = c.act == MOE_ACT_SWIGLU;
  g.mode = swiglu ? MODE_SWIGLU_UP : MODE_GELU_UP;
  g.perm = perm;
  g.gather_k = c.top_k;
  g.a_rows = (int)c.n_tokens;
  g.K = c.d_model;
  g.Nn = c.d_ff;
  g.a = x;
  g.offsets = offsets;
  g.fp8 = true;
  g.w8 = w1q;
  g.w8_3 = swiglu ? w3q : nullptr;
  g.scale1 = s1;
  g.scale3 = swiglu ? s3 : nullptr;
  g.bias = c.ffn_bias ? b1 : nullptr;
  g.out = h;
  MOE_HIP(launch_grouped_gemm(g, s));
  return MOE_OK;
}

moe_status do_down_fp8(const moe_config& c, const Workspace& W, const void* h, const int32_t* offsets,
                       const uint8_t* w2q, const float* s2, const void* b2, void* y, void* ws, hipStream_t s) {
  GroupedGemmArgs g = gemm_args(c, W, ws, false);
  g.mode = MODE_DOWN;
  g.K = c.d_ff;
  g.Nn = c.d_model;
  g.a = h;
  g.offsets = offsets;
  g.fp8 = true;
  g.w8 = w2q;
  g.scale1 = s2;
  g.bias = c.ffn_bias ? b2 : nullptr;
  g.out = y;
  MOE_HIP(launch_grouped_gemm(g, s));
  return MOE_OK;
}

// Top-1 combine fused into the routed down projection (see moe_expert_down_combine).
struct FusedCombine {
  const int32_t* perm;
  const float* gates;
  const void* residual;
  const void* shared_y;
  void* out;
};

moe_status do_down(const moe_config& c, const Workspace& W, const void* h, const int32_t* offsets,
                   const void* w2, const void* b2, void* y, void* ws, hipStream_t s, bool shared,
                   const FusedCombine* fc = nullptr) {
  GroupedGemmArgs g = gemm_args(c, W, ws, shared);
  if (fc) {
    g.comb_perm = fc->perm;
    g.comb_gates = fc->gates;
    g.comb_residual = fc->residual;
    g.comb_shared = fc->shared_y;
    g.comb_out = fc->out;
  }
  g.mode = MODE_DOWN;
  g.K = shared ? c.d_ff_shared : c.d_ff;
  g.Nn = c.d_model;
  g.a = h;
  g.offsets = offsets;
  g.w = w2;
  g.w3 = nullptr;
  g.bias = (!shared && c.ffn_bias) ? b2 : nullptr;
  g.out = y;
  MOE_HIP(launch_grouped_gemm(g, s));
  return MOE_OK;
}

moe_status check_ws(const void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return MOE_OK;
  if (!ws) return MOE_ERR_ARG;
  if (ws_bytes < need) return MOE_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

size_t scratch_end(const Workspace& W) { return W.logits; }   // the step entry points use [0, logits)

// The up GEMM reads token rows through perm when the bf16 token matrix fits
// its 32-bit buffer offsets (the fp32 path has no such limit).
bool gather_ok(const moe_config& c) {
  if (c.dtype != MOE_BF16) return true;
  return (size_t)c.n_tokens * (size_t)c.d_model * 2 <= grouped_gemm_gather_max_bytes();
}

// ------------------------------------------------ scratch of the allocation-free dispatch
// moe_permute_noalloc keeps its scratch in this array instead of a caller's
// workspace: the per-slot ranks (kNoAllocMaxSlots int32), then the per-block
// expert counts ([kNoAllocMaxSlots / kHistSlotsPerBlock][kMaxExperts] int32).
// Every GPU the library runs on holds its own copy until the process ends; the
// host reaches it only through the address hipGetSymbolAddress returns on that
// device (the array's name is a host-side stand-in, not a device address).
constexpr long long kNoAllocMaxSlots = 1ll << 20;
constexpr size_t kNoAllocRankBytes = (size_t)kNoAllocMaxSlots * 4;
constexpr size_t kNoAllocScratchBytes =
    kNoAllocRankBytes + (size_t)(kNoAllocMaxSlots / kHistSlotsPerBlock) * kMaxExperts * 4;

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`, looked up once per device (with that
// device current) and kept.
moe_status scratch_on_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_ARG: return "MOE_ERR_ARG: invalid argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: unsupported configuration or alignment";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: kernel launch failed";
    case MOE_ERR_INTERNAL: return "MOE_ERR_INTERNAL";
  }
  return "unknown moe_status";
}

moe_status moe_workspace_size(const moe_config* cfg, size_t* bytes) {
  try {
    MOE_TRY(check_config(cfg));
    if (!bytes) return MOE_ERR_ARG;
    *bytes = workspace_layout(*cfg).total;
    return MOE_OK;
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

moe_status moe_expert_rows(const moe_config* cfg, int64_t* rows, int32_t* capacity) {
  try {
    MOE_TRY(check_config(cfg));
    if (!rows) return MOE_ERR_ARG;
    *rows = expert_rows(*cfg);
    if (capacity) *capacity = capacity_of(*cfg);
    return MOE_OK;
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

moe_status moe_route(const moe_config* cfg, const void* x, const void* w_router, const float* logit_bias,
                     const float* sel_bias, const float* logits_in, float* logits, int32_t* topk_idx,
                     float* gates, float* probsum, void* ws, size_t ws_bytes, hipStream_t stream) {
  try {
    MOE_TRY(check_config(cfg));
    const moe_config& c = *cfg;
    const bool any = c.n_tokens > 0;
    if (any && (!topk_idx || !gates)) return MOE_ERR_ARG;
    if (!logits_in && (!w_router || (any && (!x || !logits)))) return MOE_ERR_ARG;
    if (!logits_in && (!aligned16(x) || !aligned16(w_router))) return MOE_ERR_UNSUPPORTED;
    const Workspace W = workspace_layout(c);
    MOE_TRY(check_ws(ws, ws_bytes, probsum ? scratch_end(W) : 0));
    // a workspace too small (or unaligned) for the scratch is simply not used
    void* scratch = (ws && check_ws(ws, ws_bytes, scratch_end(W)) == MOE_OK) ? ws : nullptr;
    return do_route(c, W, x, w_router, logit_bias, sel_bias, logits_in, logits, topk_idx, gates, probsum,
                    scratch, stream);
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

moe_status moe_permute(const moe_config* cfg, const int32_t* topk_idx, const void* x, int32_t* counts,
                       int32_t* offsets, int32_t* perm, int32_t* slot_pos, int64_t* drop_count,
                       void* x_perm, void* ws, size_t ws_bytes, hipStream_t stream) {
  try {
    MOE_TRY(check_config(cfg));
    const moe_config& c = *cfg;
    const bool any = c.n_tokens > 0;
    if (!counts || !offsets) return MOE_ERR_ARG;
    if (any && (!topk_idx || !perm || !slot_pos || (x_perm && !x))) return MOE_ERR_ARG;
    if (!aligned16(x) || !aligned16(x_perm)) return MOE_ERR_UNSUPPORTED;
    const Workspace W = workspace_layout(c);
    MOE_TRY(check_ws(ws, ws_bytes, scratch_end(W)));
    return do_permute(c, W, topk_idx, x, counts, offsets, perm, slot_pos, drop_count, x_perm, ws, stream);
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

moe_status moe_permute_noalloc(const moe_config* cfg, const int32_t* topk_idx, const void* x, int32_t* counts,
                               int32_t* offsets, int32_t* perm, int32_t* slot_pos, int64_t* drop_count,
                               void* x_perm, hipStream_t stream) {
  try {
    MOE_TRY(check_config(cfg));
    const moe_config& c = *cfg;
    const bool any = c.n_tokens > 0;
    if (!counts || !offsets) return MOE_ERR_ARG;
    if (any && (!topk_idx || !perm || !slot_pos || (x_perm && !x))) return MOE_ERR_ARG;
    if (!aligned16(x) || !aligned16(x_perm)) return MOE_ERR_UNSUPPORTED;
    if (c.n_tokens * (long long)c.top_k > kNoAllocMaxSlots) return MOE_ERR_WORKSPACE;
    const Workspace W = workspace_layout(c);   // host arithmetic only (the block count)
    void* base = nullptr;
    MOE_TRY(scratch_on_device(&base));
    int32_t* ranks = static_cast<int32_t*>(base);
    int32_t* blocks = reinterpret_cast<int32_t*>(static_cast<char*>(base) + kNoAllocRankBytes);
    MOE_HIP(launch_permute(c, W, topk_idx, x, counts, offsets, perm, slot_pos, drop_count, x_perm, ranks, blocks,
                           stream));
    return MOE_OK;
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

moe_status moe_expert_up(const moe_config* cfg, const void* x_perm, const int32_t* offsets, const void* w1,
                         const void* w3, const void* b1, void* h_tmp, void* ws, size_t ws_bytes,
                         hipStream_t stream) {
  try {
    MOE_TRY(check_config(cfg));
    const moe_config& c = *cfg;
    const bool any = c.n_tokens > 0;
    if (!offsets || !w1 || (any && (!x_perm || !h_tmp))) return MOE_ERR_ARG;
    if (c.act == MOE_ACT_SWIGLU && !w3) return MOE_ERR_ARG;
    if (c.act == MOE_ACT_GELU && w3) return MOE_ERR_ARG;
    if (c.ffn_bias && !b1) return MOE_ERR_ARG;
    if (!aligned16(x_perm) || !aligned16(w1) || (w3 && !aligned16(w3)) || !aligned16(h_tmp) ||
        (b1 && !aligned16(b1)))
      return MOE_ERR_UNSUPPORTED;
    const Workspace W = workspace_layout(c);
    MOE_TRY(check_ws(ws, ws_bytes, scratch_end(W)));
    return do_up(c, W, x_perm, offsets, w1, w3, b1, h_tmp, ws, stream, false);
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

moe_status moe_expert_up_gather(const moe_config* cfg, const void* x, const int32_t* perm,
                                const int32_t* offsets, const void* w1, const void* w3, const void* b1,
                                void* h_tmp, void* ws, size_t ws_bytes, hipStream_t stream) {
  try {
    MOE_TRY(check_config(cfg));
    const moe_config& c = *cfg;
    const bool any = c.n_tokens > 0;
    if (!offsets || !w1 || (any && (!x || !perm || !h_tmp))) return MOE_ERR_ARG;
    if (c.act == MOE_ACT_SWIGLU && !w3) return MOE_ERR_ARG;
    if (c.act == MOE_ACT_GELU && w3) return MOE_ERR_ARG;
    if (c.ffn_bias && !b1) return MOE_ERR_ARG;
    if (!gather_ok(c)) return MOE_ERR_UNSUPPORTED;
    if (!aligned16(x) || !aligned16(w1) || (w3 && !aligned16(w3)) || !aligned16(h_tmp) || (b1 && !aligned16(b1)))
      return MOE_ERR_UNSUPPORTED;
    const Workspace W = workspace_layout(c);
    MOE_TRY(check_ws(ws, ws_bytes, scratch_end(W)));
    if (!any) return MOE_OK;
    return do_up(c, W, x, offsets, w1, w3, b1, h_tmp, ws, stream, false, perm);
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

moe_status moe_expert_up_save(const moe_config* cfg, const void* x, const int32_t* perm, const int32_t* offsets,
                              const void* w1, const void* w3, const void* b1, void* h_tmp, void* pre_act, void* ws,
                              size_t ws_bytes, hipStream_t stream) {
  try {
    MOE_TRY(check_config(cfg));
    const moe_config& c = *cfg;
    if (c.dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    const bool any = c.n_tokens > 0;
    if (!offsets || !w1 || (any && (!x || !perm || !h_tmp || !pre_act))) return MOE_ERR_ARG;
    if (c.act == MOE_ACT_SWIGLU && !w3) return MOE_ERR_ARG;
    if (c.act == MOE_ACT_GELU && w3) return MOE_ERR_ARG;
    if (c.ffn_bias && !b1) return MOE_ERR_ARG;
    if (!gather_ok(c)) return MOE_ERR_UNSUPPORTED;
    if (!aligned16(x) || !aligned16(w1) || (w3 && !aligned16(w3)) || !aligned16(h_tmp) || !aligned16(pre_act) ||
        (b1 && !aligned16(b1)))
      return MOE_ERR_UNSUPPORTED;
    const Workspace W = workspace_layout(c);
    MOE_TRY(check_ws(ws, ws_bytes, scratch_end(W)));
    if (!any) return MOE_OK;
    return do_up(c, W, x, offsets, w1, w3, b1, h_tmp, ws, stream, false, perm, pre_act);
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

moe_status moe_expert_down_combine(const moe_config* cfg, const void* h_tmp, const int32_t* offsets,
                                   const int32_t* perm, const int32_t* slot_pos, const float* gates, const void* w2,
                                   const void* b2, const void* residual, const void* shared_y, void* out, void* ws,
                                   size_t ws_bytes, hipStream_t stream) {
  try {
    MOE_TRY(check_config(cfg));
    const moe_config& c = *cfg;
    if (c.top_k != 1 || c.dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    const bool any = c.n_tokens > 0;
    if (!offsets || !w2 || (any && (!h_tmp || !perm || !slot_pos || !gates || !out))) return MOE_ERR_ARG;
    if (c.ffn_bias && !b2) return MOE_ERR_ARG;
    if (!aligned16(h_tmp) || !aligned16(w2) || !aligned16(out) || (b2 && !aligned16(b2)) ||
        (residual && !aligned16(residual)) || (shared_y && !aligned16(shared_y)))
      return MOE_ERR_UNSUPPORTED;
    const Workspace W = workspace_layout(c);
    MOE_TRY(check_ws(ws, ws_bytes, scratch_end(W)));
    if (!any) return MOE_OK;
    MOE_HIP(launch_combine_dropped(c, slot_pos, residual, shared_y, out, stream));
    const FusedCombine fc{perm, gates, residual, shared_y, out};
    return do_down(c, W, h_tmp, offsets, w2, b2, nullptr, ws, stream, false, &fc);
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

moe_status moe_expert_down(const moe_config* cfg, const void* h_tmp, const int32_t* offsets, const void* w2,
                           const void* b2, void* y_perm, void* ws, size_t ws_bytes, hipStream_t stream) {
  try {
    MOE_TRY(check_config(cfg));
    const moe_config& c = *cfg;
    const bool any = c.n_tokens > 0;
    if (!offsets || !w2 || (any && (!h_tmp || !y_perm))) return MOE_ERR_ARG;
    if (c.ffn_bias && !b2) return MOE_ERR_ARG;
    if (!aligned16(h_tmp) || !aligned16(w2) || !aligned16(y_perm) || (b2 && !aligned16(b2)))
      return MOE_ERR_UNSUPPORTED;
    const Workspace W = workspace_layout(c);
    MOE_TRY(check_ws(ws, ws_bytes, scratch_end(W)));
    return do_down(c, W, h_tmp, offsets, w2, b2, y_perm, ws, stream, false);
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

moe_status moe_expert_ffn(const moe_config* cfg, const void* x_perm, const int32_t* offsets, const void* w1,
                          const void* w3, const void* w2, const void* b1, const void* b2, void* h_tmp,
                          void* y_perm, void* ws, size_t ws_bytes, hipStream_t stream) {
  try {
    MOE_TRY(check_config(cfg));
    const moe_config& c = *cfg;
    if (!w2 || (c.n_tokens > 0 && !y_perm)) return MOE_ERR_ARG;
    if (c.ffn_bias && !b2) return MOE_ERR_ARG;
    if (!aligned16(w2) || !aligned16(y_perm) || (b2 && !aligned16(b2))) return MOE_ERR_UNSUPPORTED;
    MOE_TRY(moe_expert_up(cfg, x_perm, offsets, w1, w3, b1, h_tmp, ws, ws_bytes, stream));
    const Workspace W = workspace_layout(c);
    return do_down(c, W, h_tmp, offsets, w2, b2, y_perm, ws, stream, false);
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

moe_status moe_quantize_fp8(const void* w, int64_t rows, int32_t cols, uint8_t* q, float* scales,
                            hipStream_t stream) {
  try {
    if (rows < 0 || cols <= 0 || cols > (1 << 24)) return MOE_ERR_ARG;
    if (rows > 0 && (!w || !q || !scales)) return MOE_ERR_ARG;
    if (cols % 4 == 0 && (!aligned16(w) || (reinterpret_cast<uintptr_t>(q) & 3u)))
      return MOE_ERR_UNSUPPORTED;
    MOE_HIP(launch_quantize_fp8(reinterpret_cast<const uint16_t*>(w), rows, cols, q, scales, stream));
    return MOE_OK;
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

moe_status moe_probe_hbm_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  try {
    if (bytes > 0 && (!buf || !sink)) return MOE_ERR_ARG;
    if (!aligned16(buf) || bytes % 16 != 0) return MOE_ERR_UNSUPPORTED;
    MOE_HIP(launch_hbm_read_probe(buf, bytes, sink, stream));
    return MOE_OK;
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

moe_status moe_probe_mfma_bf16(const void* operands, int64_t iters, float* sink, hipStream_t stream) {
  try {
    if (iters < 0) return MOE_ERR_ARG;
    if (iters > 0 && (!operands || !sink)) return MOE_ERR_ARG;
    if (!aligned16(operands)) return MOE_ERR_UNSUPPORTED;
    MOE_HIP(launch_mfma_probe(operands, iters, sink, stream));
    return MOE_OK;
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

moe_status moe_probe_mfma_flop_per_iter(int64_t* flop) {
  if (!flop) return MOE_ERR_ARG;
  // every wavefront of the grid (G CUs x 8) issues two 32x32x16 MFMAs per iteration
  *flop = (int64_t)probe_grid() * 8 * 2 * (2ll * 32 * 32 * 16);
  return MOE_OK;
}

moe_status moe_expert_up_fp8(const moe_config* cfg, const void* x, const int32_t* perm, const int32_t* offsets,
                             const uint8_t* w1q, const uint8_t* w3q, const float* s1, const float* s3,
                             const void* b1, void* h_tmp, void* ws, size_t ws_bytes, hipStream_t stream) {
  try {
    MOE_TRY(check_config(cfg));
    const moe_config& c = *cfg;
    const bool any = c.n_tokens > 0;
    if (c.dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    if (!offsets || !w1q || !s1 || (any && (!x || !perm || !h_tmp))) return MOE_ERR_ARG;
    if (c.act == MOE_ACT_SWIGLU && (!w3q || !s3)) return MOE_ERR_ARG;
    if (c.act == MOE_ACT_GELU && (w3q || s3)) return MOE_ERR_ARG;
    if (c.ffn_bias && !b1) return MOE_ERR_ARG;
    if (!gather_ok(c)) return MOE_ERR_UNSUPPORTED;
    if (!aligned16(x) || !aligned16(w1q) || !aligned16(w3q) || !aligned16(h_tmp) || !aligned16(b1))
      return MOE_ERR_UNSUPPORTED;
    const Workspace W = workspace_layout(c);
    MOE_TRY(check_ws(ws, ws_bytes, scratch_end(W)));
    if (!any) return MOE_OK;
    return do_up_fp8(c, W, x, perm, offsets, w1q, w3q, s1, s3, b1, h_tmp, ws, stream);
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

moe_status moe_expert_down_fp8(const moe_config* cfg, const void* h_tmp, const int32_t* offsets,
                               const uint8_t* w2q, const float* s2, const void* b2, void* y_perm, void* ws,
                               size_t ws_bytes, hipStream_t stream) {
  try {
    MOE_TRY(check_config(cfg));
    const moe_config& c = *cfg;
    const bool any = c.n_tokens > 0;
    if (c.dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    if (!offsets || !w2q || !s2 || (any && (!h_tmp || !y_perm))) return MOE_ERR_ARG;
    if (c.ffn_bias && !b2) return MOE_ERR_ARG;
    if (!aligned16(h_tmp) || !aligned16(w2q) || !aligned16(y_perm) || !aligned16(b2)) return MOE_ERR_UNSUPPORTED;
    const Workspace W = workspace_layout(c);
    MOE_TRY(check_ws(ws, ws_bytes, scratch_end(W)));
    if (!any) return MOE_OK;
    return do_down_fp8(c, W, h_tmp, offsets, w2q, s2, b2, y_perm, ws, stream);
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

moe_status moe_shared_ffn(const moe_config* cfg, const void* x, const void* sh_w1, const void* sh_w3,
                          const void* sh_w2, void* h_tmp, void* y_sh, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  try {
    MOE_TRY(check_config(cfg));
    const moe_config& c = *cfg;
    if (c.d_ff_shared <= 0) return MOE_ERR_ARG;
    if (!sh_w1 || !sh_w3 || !sh_w2) return MOE_ERR_ARG;
    if (c.n_tokens > 0 && (!x || !h_tmp || !y_sh)) return MOE_ERR_ARG;
    if (!aligned16(x) || !aligned16(sh_w1) || !aligned16(sh_w3) || !aligned16(sh_w2) || !aligned16(h_tmp) ||
        !aligned16(y_sh))
      return MOE_ERR_UNSUPPORTED;
    const Workspace W = workspace_layout(c);
    MOE_TRY(check_ws(ws, ws_bytes, scratch_end(W)));
    MOE_TRY(do_up(c, W, x, nullptr, sh_w1, sh_w3, nullptr, h_tmp, ws, stream, true));
    return do_down(c, W, h_tmp, nullptr, sh_w2, nullptr, y_sh, ws, stream, true);
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

moe_status moe_combine(const moe_config* cfg, const void* y_perm, const int32_t* slot_pos, const float* gates,
                       const void* residual, const void* shared_y, void* out, hipStream_t stream) {
  try {
    MOE_TRY(check_config(cfg));
    const moe_config& c = *cfg;
    if (c.n_tokens > 0 && (!y_perm || !slot_pos || !gates || !out)) return MOE_ERR_ARG;
    if (!aligned16(y_perm) || !aligned16(out) || (residual && !aligned16(residual)) ||
        (shared_y && !aligned16(shared_y)))
      return MOE_ERR_UNSUPPORTED;
    MOE_HIP(launch_combine(c, y_perm, slot_pos, gates, residual, shared_y, out, stream));
    return MOE_OK;
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

moe_status moe_bias_update(const moe_config* cfg, const int32_t* counts, float gamma, float* sel_bias,
                           int8_t* signs, hipStream_t stream) {
  try {
    MOE_TRY(check_config(cfg));
    if (!counts || !sel_bias) return MOE_ERR_ARG;
    if (isnan(gamma) || gamma < 0.f) return MOE_ERR_ARG;
    MOE_HIP(launch_bias_update(*cfg, counts, gamma, sel_bias, sel_bias, signs, stream));
    return MOE_OK;
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

moe_status moe_aux_loss(const moe_config* cfg, const int32_t* counts, const float* probsum, float* aux,
                        hipStream_t stream) {
  try {
    MOE_TRY(check_config(cfg));
    if (!counts || !probsum || !aux) return MOE_ERR_ARG;
    MOE_HIP(launch_aux_loss(*cfg, counts, probsum, aux, stream));
    return MOE_OK;
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

moe_status moe_forward(const moe_config* cfg, const moe_weights* w, const void* x, const void* residual,
                       const float* sel_bias, const moe_outputs* o, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
  try {
    MOE_TRY(check_config(cfg));
    const moe_config& c = *cfg;
    if (!w || !o) return MOE_ERR_ARG;
    if (c.n_tokens > 0 && (!x || !o->out)) return MOE_ERR_ARG;
    if (!w->w_router || !w->w1 || !w->w2) return MOE_ERR_ARG;
    if (c.act == MOE_ACT_SWIGLU && !w->w3) return MOE_ERR_ARG;
    if (c.ffn_bias && (!w->b1 || !w->b2)) return MOE_ERR_ARG;
    if (c.d_ff_shared > 0 && (!w->sh_w1 || !w->sh_w3 || !w->sh_w2)) return MOE_ERR_ARG;
    if (o->bias_gamma > 0.f && (!sel_bias || !o->sel_bias_next)) return MOE_ERR_ARG;
    if (isnan(o->bias_gamma)) return MOE_ERR_ARG;
    const void* ptrs[] = {x, o->out, w->w_router, w->w1, w->w2, w->w3, w->b1, w->b2, w->sh_w1, w->sh_w3,
                          w->sh_w2, residual};
    for (const void* p : ptrs)
      if (p && !aligned16(p)) return MOE_ERR_UNSUPPORTED;
    const Workspace W = workspace_layout(c);
    MOE_TRY(check_ws(ws, ws_bytes, W.total));

    float* logits = o->logits ? o->logits : reinterpret_cast<float*>(wsp(ws, W.logits));
    int32_t* topk_idx = o->topk_idx ? o->topk_idx : reinterpret_cast<int32_t*>(wsp(ws, W.topk_idx));
    float* gates = o->gates ? o->gates : reinterpret_cast<float*>(wsp(ws, W.gates));
    int32_t* counts = o->counts ? o->counts : reinterpret_cast<int32_t*>(wsp(ws, W.counts));
    int32_t* offsets = o->offsets ? o->offsets : reinterpret_cast<int32_t*>(wsp(ws, W.offsets));
    int32_t* perm = o->perm ? o->perm : reinterpret_cast<int32_t*>(wsp(ws, W.perm));
    int32_t* slot_pos = o->slot_pos ? o->slot_pos : reinterpret_cast<int32_t*>(wsp(ws, W.slot_pos));
    int64_t* drop = o->drop_count ? o->drop_count : reinterpret_cast<int64_t*>(wsp(ws, W.drop_count));
    const bool want_aux = o->aux != nullptr;
    float* probsum = o->probsum ? o->probsum : (want_aux ? reinterpret_cast<float*>(wsp(ws, W.probsum)) : nullptr);
    const bool fused = gather_ok(c);   // the up GEMM gathers token rows itself
    void* x_perm = fused ? nullptr : wsp(ws, W.x_perm);
    void* h = wsp(ws, W.h);
    void* y = wsp(ws, W.y);
    const void* res = c.add_residual ? (residual ? residual : x) : nullptr;

    MOE_TRY(do_route(c, W, x, w->w_router, w->logit_bias, sel_bias, nullptr, logits, topk_idx, gates, probsum,
                     ws, stream));
    MOE_TRY(do_permute(c, W, topk_idx, x, counts, offsets, perm, slot_pos, drop, x_perm, ws, stream));
    if (fused) MOE_TRY(do_up(c, W, x, offsets, w->w1, w->w3, w->b1, h, ws, stream, false, perm));
    else MOE_TRY(do_up(c, W, x_perm, offsets, w->w1, w->w3, w->b1, h, ws, stream, false));
    const void* shared_y = nullptr;
    if (c.d_ff_shared > 0) {
      void* h_sh = wsp(ws, W.h_sh);
      void* y_sh = wsp(ws, W.y_sh);
      MOE_TRY(do_up(c, W, x, nullptr, w->sh_w1, w->sh_w3, nullptr, h_sh, ws, stream, true));
      MOE_TRY(do_down(c, W, h_sh, nullptr, w->sh_w2, nullptr, y_sh, ws, stream, true));
      shared_y = y_sh;
    }
    if (c.top_k == 1 && c.dtype == MOE_BF16) {   // one slot per token: combine in the down projection
      MOE_HIP(launch_combine_dropped(c, slot_pos, res, shared_y, o->out, stream));
      const FusedCombine fc{perm, gates, res, shared_y, o->out};
      MOE_TRY(do_down(c, W, h, offsets, w->w2, w->b2, y, ws, stream, false, &fc));
    } else {
      MOE_TRY(do_down(c, W, h, offsets, w->w2, w->b2, y, ws, stream, false));
      MOE_HIP(launch_combine(c, y, slot_pos, gates, res, shared_y, o->out, stream));
    }
    if (want_aux) MOE_HIP(launch_aux_loss(c, counts, probsum, o->aux, stream));
    if (o->bias_gamma > 0.f) {
      int8_t* signs = o->signs ? o->signs : reinterpret_cast<int8_t*>(wsp(ws, W.signs));
      MOE_HIP(launch_bias_update(c, counts, o->bias_gamma, sel_bias, o->sel_bias_next, signs, stream));
    } else if (o->signs) {
      MOE_HIP(launch_bias_update(c, counts, 0.f, nullptr, nullptr, o->signs, stream));
    }
    return MOE_OK;
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

}  // extern "C"

// ===================================================================== backward

namespace {

// Backward workspace: the forward scratch first (tile lists, K-split partials),
// then the backward's own buffers.
struct BwdLayout {
  size_t a1, a3, h, dy, dh, da, dX, xg, dg, dz, dz16, zpart, dxr;
  size_t a1s, a3s, hs, dhs, das, dxs, tiles_dense, tiles_none;
  size_t total;
  int ldz;          // K-padded router width (a multiple of 64) for the dx product
  int max_tiles_dense;
};

BwdLayout backward_layout(const moe_config& c) {
  BwdLayout B{};
  const Workspace W = workspace_layout(c);
  size_t off = scratch_end(W);
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return o;
  };
  const size_t N = (size_t)c.n_tokens, E = (size_t)c.n_experts, k = (size_t)c.top_k;
  const size_t d = (size_t)c.d_model, F = (size_t)c.d_ff, Fs = (size_t)(c.d_ff_shared > 0 ? c.d_ff_shared : 0);
  const size_t R = (size_t)expert_rows(c);
  const bool sw = c.act == MOE_ACT_SWIGLU;
  const size_t nA = sw ? 2 : 1;
  B.ldz = ((c.n_experts + 63) / 64) * 64;
  B.max_tiles_dense = grouped_gemm_max_tiles((int)N, 1);
  B.a1 = take(R * F * 2);
  B.a3 = take(sw ? R * F * 2 : 0);
  B.h = take(R * F * 2);
  B.dy = take(R * d * 2);
  B.dh = take(R * F * 2);
  B.da = take(R * nA * F * 2);
  B.dX = take(R * d * 2);
  B.xg = take(R * d * 2);
  B.dg = take(N * k * 4);
  B.dz = take(N * E * 4);
  B.dz16 = take(N * (size_t)B.ldz * 2);
  B.zpart = take(colsum_part_floats((int)N, (int)E) * 4);
  B.dxr = take(N * d * 2);
  B.a1s = take(N * Fs * 2);
  B.a3s = take(N * Fs * 2);
  B.hs = take(N * Fs * 2);
  B.dhs = take(N * Fs * 2);
  B.das = take(N * 2 * Fs * 2);
  B.dxs = take(Fs ? N * d * 2 : 0);
  B.tiles_dense = take((4 + 8 * (size_t)B.max_tiles_dense) * 4);
  B.tiles_none = take(64);
  B.total = off;
  return B;
}

// Plain product out[r, :Nn] = a[r, :K] W^T (+ bias) on the grouped GEMM (mode down): segments of
// the routed layout (shared = false) or one dense segment of N rows (shared = true / router).
moe_status plain_gemm(const moe_config& c, const Workspace& W, void* ws, bool dense, const void* a,
                      const int32_t* perm, const int32_t* offsets, const void* w, const void* bias, int K, int Nn,
                      void* out, hipStream_t s) {
  GroupedGemmArgs g = gemm_args(c, W, ws, false);
  if (dense) {
    g.n_seg = 1;
    g.max_rows = (int)c.n_tokens;
    g.offsets = nullptr;
  } else {
    g.offsets = offsets;
  }
  g.mode = MODE_DOWN;
  g.perm = perm;
  g.gather_k = c.top_k;
  g.a_rows = (int)c.n_tokens;
  g.K = K;
  g.Nn = Nn;
  g.a = a;
  g.w = w;
  g.bias = bias;
  g.out = out;
  MOE_HIP(launch_grouped_gemm(g, s));
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_backward_workspace_size(const moe_config* cfg, size_t* bytes) {
  try {
    MOE_TRY(check_config(cfg));
    if (!bytes) return MOE_ERR_ARG;
    *bytes = backward_layout(*cfg).total;
    return MOE_OK;
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

moe_status moe_backward(const moe_config* cfg, const moe_weights* w, const void* x, const void* dout, float d_aux,
                        const moe_saved* sv, const moe_grads* gr, void* ws, size_t ws_bytes, hipStream_t stream) {
  try {
    MOE_TRY(check_config(cfg));
    const moe_config& c = *cfg;
    if (c.dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    if (!w || !sv || !gr) return MOE_ERR_ARG;
    if (isnan(d_aux)) return MOE_ERR_ARG;
    const bool any = c.n_tokens > 0;
    const bool sw = c.act == MOE_ACT_SWIGLU;
    const bool shared = c.d_ff_shared > 0;
    if (!w->w_router || !w->w1 || !w->w2 || (sw && !w->w3)) return MOE_ERR_ARG;
    if (c.ffn_bias && (!w->b1 || !w->b2 || !gr->db1 || !gr->db2)) return MOE_ERR_ARG;
    if (!gr->dw1 || !gr->dw2 || (sw && !gr->dw3)) return MOE_ERR_ARG;
    if (shared && (!w->sh_w1 || !w->sh_w3 || !w->sh_w2 || !gr->dsh_w1 || !gr->dsh_w3 || !gr->dsh_w2))
      return MOE_ERR_ARG;
    if (any && (!x || !dout || !gr->dx || !sv->logits || !sv->topk_idx || !sv->gates || !sv->counts ||
                !sv->offsets || !sv->perm || !sv->slot_pos || !sv->y_perm))
      return MOE_ERR_ARG;
    if (!gather_ok(c)) return MOE_ERR_UNSUPPORTED;
    const void* ptrs[] = {x, dout, gr->dx, sv->y_perm, sv->pre_act, w->w_router, w->w1, w->w3, w->w2, w->b1, w->b2,
                          w->sh_w1, w->sh_w3, w->sh_w2, gr->dw1, gr->dw3, gr->dw2, gr->dw_router};
    for (const void* p : ptrs)
      if (!aligned16(p)) return MOE_ERR_UNSUPPORTED;
    const Workspace W = workspace_layout(c);
    const BwdLayout B = backward_layout(c);
    MOE_TRY(check_ws(ws, ws_bytes, B.total));
    const int N = (int)c.n_tokens, E = c.n_experts, k = c.top_k, d = c.d_model, F = c.d_ff;
    const int Fs = shared ? c.d_ff_shared : 0;
    const long long R = expert_rows(c);
    const int nA = sw ? 2 : 1;
    auto P = [&](size_t o) { return wsp(ws, o); };
    float* dg = gr->dgates ? gr->dgates : reinterpret_cast<float*>(P(B.dg));

    if (!any) {   // an empty batch: every weight gradient is zero
      const size_t Fd = (size_t)F * d;
      MOE_HIP(launch_fill_zero(gr->dw1, (size_t)E * Fd, stream));
      MOE_HIP(launch_fill_zero(gr->dw2, (size_t)E * Fd, stream));
      if (sw) MOE_HIP(launch_fill_zero(gr->dw3, (size_t)E * Fd, stream));
      if (c.ffn_bias) {
        MOE_HIP(launch_fill_zero(gr->db1, (size_t)E * F, stream));
        MOE_HIP(launch_fill_zero(gr->db2, (size_t)E * d, stream));
      }
      if (gr->dw_router) MOE_HIP(launch_fill_zero(gr->dw_router, (size_t)E * d, stream));
      if (gr->dlogit_bias) MOE_HIP(launch_fill_zero(gr->dlogit_bias, (size_t)E, stream));
      if (shared) {
        MOE_HIP(launch_fill_zero(gr->dsh_w1, (size_t)Fs * d, stream));
        MOE_HIP(launch_fill_zero(gr->dsh_w3, (size_t)Fs * d, stream));
        MOE_HIP(launch_fill_zero(gr->dsh_w2, (size_t)Fs * d, stream));
      }
      return MOE_OK;
    }
    // every K-major row range the products address stays below 2^31 bytes
    const size_t lim = 0x7fffffffull;
    const size_t ld_routed = (size_t)std::max(d, nA * F), ld_dense = (size_t)std::max(std::max(B.ldz, d), 2 * Fs);
    if ((size_t)R * ld_routed * 2 >= lim || (size_t)N * ld_dense * 2 >= lim) return MOE_ERR_UNSUPPORTED;
    int32_t* tiles = reinterpret_cast<int32_t*>(P(W.tiles));
    int32_t* tiles_small = reinterpret_cast<int32_t*>(P(W.tiles_small));
    int32_t* tiles_dense = reinterpret_cast<int32_t*>(P(B.tiles_dense));
    int32_t* tiles_none = reinterpret_cast<int32_t*>(P(B.tiles_none));
    // out[rows of each expert] = a B_e, B_e in its stored [K, N] layout (rows k >= K1 from B2)
    auto nn_routed = [&](const void* a, const void* B1, const void* B2, int K, int K1, int Nn, void* out) {
      return launch_gemm_nn(a, sv->offsets, E, 0, (int)R, tiles, W.max_tiles, tiles_small, W.max_tiles_small, B1,
                            B2, (long long)K1 * Nn, K, K1, K1, K - K1, Nn, out, stream);
    };
    auto nn_dense = [&](const void* a, const void* B1, const void* B2, int K, int K1, int b_rows1, int Nn,
                        void* out) {
      return launch_gemm_nn(a, nullptr, 1, N, N, tiles_dense, B.max_tiles_dense, tiles_none, 0, B1, B2, 0, K, K1,
                            b_rows1, K - K1, Nn, out, stream);
    };

    // combine backward: dL/dgates and dY = g dout on the kept rows
    MOE_HIP(launch_combine_backward(c, dout, sv->y_perm, sv->slot_pos, sv->gates, dg, P(B.dy), stream));
    // token rows in expert order (zero rows, and zero dY, for padding rows)
    MOE_HIP(launch_gather_rows(x, sv->perm, sv->offsets, E, k, d, R, P(B.xg), P(B.dy), stream));
    // routed experts: recompute pre-activations, dH = dY W2_e, activation backward, dX = dA [W1_e ; W3_e]
    // pre-activations: saved by moe_expert_up_save, or recomputed from the expert-ordered rows
    const void* a1 = P(B.a1);
    const void* a3 = sw ? P(B.a3) : nullptr;
    if (sv->pre_act) {
      a1 = sv->pre_act;
      if (sw) a3 = static_cast<const uint16_t*>(sv->pre_act) + (size_t)R * F;
    } else {
      MOE_TRY(plain_gemm(c, W, ws, false, P(B.xg), nullptr, sv->offsets, w->w1, c.ffn_bias ? w->b1 : nullptr, d, F,
                         P(B.a1), stream));
      if (sw)
        MOE_TRY(plain_gemm(c, W, ws, false, P(B.xg), nullptr, sv->offsets, w->w3, nullptr, d, F, P(B.a3), stream));
    }
    MOE_HIP(nn_routed(P(B.dy), w->w2, nullptr, d, d, F, P(B.dh)));
    MOE_HIP(launch_act_backward(sw, a1, a3, P(B.dh), R, F, P(B.h), P(B.da), stream));
    MOE_HIP(nn_routed(P(B.da), w->w1, sw ? w->w3 : nullptr, nA * F, F, d, P(B.dX)));
    // expert weight gradients: reductions over each expert's rows
    MOE_HIP(launch_gemm_tn(P(B.dy), d, 0, P(B.h), F, sv->offsets, E, 0, (int)R, d, F, gr->dw2, (long long)d * F,
                           stream));
    MOE_HIP(launch_gemm_tn(P(B.da), nA * F, 0, P(B.xg), d, sv->offsets, E, 0, (int)R, F, d, gr->dw1,
                           (long long)F * d, stream));
    if (sw)
      MOE_HIP(launch_gemm_tn(P(B.da), nA * F, F, P(B.xg), d, sv->offsets, E, 0, (int)R, F, d, gr->dw3,
                             (long long)F * d, stream));
    if (c.ffn_bias) {
      MOE_HIP(launch_segment_colsum(P(B.da), nA * F, 0, F, sv->offsets, sv->perm, 0, E, gr->db1, stream));
      MOE_HIP(launch_segment_colsum(P(B.dy), d, 0, d, sv->offsets, sv->perm, 0, E, gr->db2, stream));
    }
    // router: dz from the gate gradients (+ aux), then dW_r = dz^T x, d logit_bias, dx_r = dz W_r
    float* dz = reinterpret_cast<float*>(P(B.dz));
    MOE_HIP(launch_router_backward(c, sv->logits, sv->topk_idx, sv->gates, dg, d_aux != 0.f ? sv->counts : nullptr,
                                   d_aux, dz, P(B.dz16), B.ldz, stream));
    if (gr->dw_router)
      MOE_HIP(launch_gemm_tn(P(B.dz16), B.ldz, 0, x, d, nullptr, 1, N, N, E, d, gr->dw_router, 0, stream));
    if (gr->dlogit_bias)
      MOE_HIP(launch_colsum_f32(dz, N, E, reinterpret_cast<float*>(P(B.zpart)), gr->dlogit_bias, stream));
    MOE_HIP(nn_dense(P(B.dz16), w->w_router, nullptr, B.ldz, B.ldz, E, d, P(B.dxr)));
    // shared expert (dense SwiGLU over all tokens, weight 1)
    const void* dxs = nullptr;
    if (shared) {
      auto shared_up = [&](const void* wt, void* out) {
        GroupedGemmArgs g = gemm_args(c, W, ws, true);
        g.mode = MODE_DOWN;
        g.K = d;
        g.Nn = Fs;
        g.a = x;
        g.offsets = nullptr;
        g.w = wt;
        g.out = out;
        return launch_grouped_gemm(g, stream);
      };
      MOE_HIP(shared_up(w->sh_w1, P(B.a1s)));
      MOE_HIP(shared_up(w->sh_w3, P(B.a3s)));
      MOE_HIP(nn_dense(dout, w->sh_w2, nullptr, d, d, d, Fs, P(B.dhs)));
      MOE_HIP(launch_act_backward(true, P(B.a1s), P(B.a3s), P(B.dhs), N, Fs, P(B.hs), P(B.das), stream));
      MOE_HIP(nn_dense(P(B.das), w->sh_w1, w->sh_w3, 2 * Fs, Fs, Fs, d, P(B.dxs)));
      MOE_HIP(launch_gemm_tn(dout, d, 0, P(B.hs), Fs, nullptr, 1, N, N, d, Fs, gr->dsh_w2, 0, stream));
      MOE_HIP(launch_gemm_tn(P(B.das), 2 * Fs, 0, x, d, nullptr, 1, N, N, Fs, d, gr->dsh_w1, 0, stream));
      MOE_HIP(launch_gemm_tn(P(B.das), 2 * Fs, Fs, x, d, nullptr, 1, N, N, Fs, d, gr->dsh_w3, 0, stream));
      dxs = P(B.dxs);
    }
    // dx = residual + scattered expert input gradients + shared + router
    MOE_HIP(launch_dx_gather(c, c.add_residual ? dout : nullptr, P(B.dX), sv->slot_pos, dxs, P(B.dxr), gr->dx,
                             stream));
    return MOE_OK;
  } catch (...) {
    return MOE_ERR_INTERNAL;
  }
}

}  // extern "C"
