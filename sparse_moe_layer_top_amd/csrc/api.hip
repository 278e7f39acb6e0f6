// C ABI of the Beam MoE block (declared in include/beam_moe.h): argument checks,
// workspace carve-up and launch sequencing.  Allocates nothing, never
// synchronises, keeps no state between calls.
#include "beam_moe.h"

#include <math.h>

#include <mutex>

#include "common.h"

using beam::Layout;
using beam::Shape;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int check_config(const beam_moe_config* c) {
  if (!c) return BEAM_MOE_ERR_INVALID;
  if (c->hidden <= 0 || c->inter <= 0 || c->n_experts <= 0 || c->n_groups <= 0 || c->topk_groups <= 0 ||
      c->top_k <= 0)
    return BEAM_MOE_ERR_INVALID;
  if (c->n_experts % c->n_groups != 0) return BEAM_MOE_ERR_INVALID;
  // a group's score is the sum of its two best scores: every group holds at least two experts
  if (c->n_experts / c->n_groups < 2) return BEAM_MOE_ERR_INVALID;
  if (c->topk_groups > c->n_groups) return BEAM_MOE_ERR_INVALID;
  if ((long)c->top_k > (long)c->topk_groups * (c->n_experts / c->n_groups)) return BEAM_MOE_ERR_INVALID;
  if (!isfinite(c->routed_scale)) return BEAM_MOE_ERR_INVALID;
  if (c->weight_type != BEAM_MOE_W_BF16 && c->weight_type != BEAM_MOE_W_FP8_E4M3 && c->weight_type != BEAM_MOE_W_MXFP4)
    return BEAM_MOE_ERR_INVALID;
  if (c->weight_layout != BEAM_MOE_LAYOUT_ROWS && c->weight_layout != BEAM_MOE_LAYOUT_FRAGMENTS)
    return BEAM_MOE_ERR_INVALID;
  if (c->hidden % 128 != 0 || c->inter % 128 != 0) return BEAM_MOE_ERR_UNSUPPORTED;
  if (c->weight_type == BEAM_MOE_W_MXFP4 && (c->hidden % 256 != 0 || c->inter % 256 != 0)) return BEAM_MOE_ERR_UNSUPPORTED;
  if (c->weight_type == BEAM_MOE_W_MXFP4 && c->weight_layout == BEAM_MOE_LAYOUT_FRAGMENTS &&
      (c->hidden % 512 != 0 || c->inter % 512 != 0))
    return BEAM_MOE_ERR_UNSUPPORTED;   // scale rows in whole 16-byte slices
  if (c->n_experts > beam::kMaxExperts || c->n_groups > 64 || c->top_k > beam::kMaxTopK)
    return BEAM_MOE_ERR_UNSUPPORTED;
  return BEAM_MOE_OK;
}

Shape shape_of(const beam_moe_config* c) {
  Shape s{c->hidden, c->inter, c->n_experts, c->n_groups, c->topk_groups, c->top_k, c->routed_scale,
          c->weight_type == BEAM_MOE_W_FP8_E4M3 ? 1 : 0};
  s.mx = c->weight_type == BEAM_MOE_W_MXFP4;
  s.packed = c->weight_layout == BEAM_MOE_LAYOUT_FRAGMENTS;
  return s;
}

// Router K-split: ks parts of kc = H/ks (a multiple of the 32-wide MFMA step),
// the fewest giving about 1024 workgroups of 128 tokens x 64 experts, each
// part at least 4 steps long where H allows.
constexpr int kMinSteps = 4;   // 8 or 16 made the logits kernel 40-120% slower at T = 64
int choose_ks(const Shape& s, int T) {
  const int units = s.H / 32;
  const long tiles = (long)((T + 127) / 128) * ((s.E + 63) / 64);
  int best = 1;
  for (int ks = 1; ks <= units; ++ks) {
    if (units % ks) continue;
    if (units / ks < kMinSteps && best > 1) break;
    best = ks;
    if (tiles * ks >= 1024) break;
  }
  return best;
}

Layout make_layout(const Shape& s, int T, int op) {
  Layout L{};
  const size_t TK = (size_t)T * s.K;
  L.ks = choose_ks(s, T);
  L.nchunks = (T + beam::kChunk - 1) / beam::kChunk;
  const int bm = beam::expert_tile_rows(s, T);
  L.max_tiles = (int)(TK / bm) + s.E;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  const bool fwd = op == BEAM_MOE_OP_FORWARD || op == BEAM_MOE_OP_BLOCK;
  if (op == BEAM_MOE_OP_ROUTE || fwd) L.logits = take((size_t)L.ks * T * s.E * 4);
  if (op == BEAM_MOE_OP_PERMUTE || fwd) {
    L.masks = take((size_t)L.nchunks * s.E * 8);
    L.counts = take((size_t)L.nchunks * s.E * 4);
  }
  if (fwd) {
    L.ids = take(TK * 4);
    L.w = take(TK * 4);
    L.offsets = take((size_t)(s.E + 1) * 4);
    L.tiles = take((size_t)L.max_tiles * 8);
    L.ntiles = take(4);
    L.sorted = take(TK * 4);
    L.p2r = take(TK * 4);
    L.h = take(TK * s.I * 2);
    L.y = take(TK * s.H * 2);
  }
  if (op == BEAM_MOE_OP_BLOCK) L.xn = take((size_t)T * s.H * 2);
  L.total = off;
  return L;
}

template <typename P>
P* at(void* ws, size_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(ws) + off);
}

#define BEAM_TRY_HIP(expr)                               \
  do {                                                   \
    if ((expr) != hipSuccess) return BEAM_MOE_ERR_HIP;   \
  } while (0)

// Checks shared by forward and block (config already checked, T > 0).
int check_forward_args(const beam_moe_config* cfg, const void* x, const float* w_router, const float* b_router,
                       const void* w_gate, const void* w_up, const void* w_down, const void* s_gate,
                       const void* s_up, const void* s_down, const void* out, const int32_t* topk_ids_out,
                       const float* topk_w_out) {
  if (!x || !w_router || !w_gate || !w_up || !w_down || !out) return BEAM_MOE_ERR_INVALID;
  const bool scaled = cfg->weight_type != BEAM_MOE_W_BF16;   // fp8 per-channel or MXFP4 block scales
  if (scaled != (s_gate != nullptr) || scaled != (s_up != nullptr) || scaled != (s_down != nullptr))
    return BEAM_MOE_ERR_INVALID;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(w_gate) || !aligned16(w_up) || !aligned16(w_down) ||
      !aligned16(out) || (b_router && !aligned4(b_router)) || (topk_ids_out && !aligned4(topk_ids_out)) ||
      (topk_w_out && !aligned4(topk_w_out)) ||
      (cfg->weight_type == BEAM_MOE_W_FP8_E4M3 && (!aligned4(s_gate) || !aligned4(s_up) || !aligned4(s_down))) ||
      (cfg->weight_type == BEAM_MOE_W_MXFP4 && (!aligned16(s_gate) || !aligned16(s_up) || !aligned16(s_down))))
    return BEAM_MOE_ERR_INVALID;
  return BEAM_MOE_OK;
}

// The post-norm and residual mix that replace the plain combine in the block path.
struct BlockEpilogue {
  float eps, a, b;
  const float* gamma_post;
  const uint16_t* stream_in;
  uint16_t* stream_out;
  uint16_t* moe_out;   // optional
};

// Router .. combine on x; `ev` (optional) gets one event before each stage and one after the last.
int run_forward(const Shape& s, const Layout& L, int T, const uint16_t* xb, const float* w_router,
                const float* b_router, const void* w_gate, const void* w_up, const void* w_down, const void* s_gate,
                const void* s_up, const void* s_down, uint16_t* out, int32_t* topk_ids_out, float* topk_w_out,
                void* workspace, hipStream_t hs, void* const* ev, const BlockEpilogue* blk) {
  int32_t* ids = topk_ids_out ? topk_ids_out : at<int32_t>(workspace, L.ids);
  float* w = topk_w_out ? topk_w_out : at<float>(workspace, L.w);
  float* partial = at<float>(workspace, L.logits);
  int32_t* offsets = at<int32_t>(workspace, L.offsets);
  int32_t* sorted = at<int32_t>(workspace, L.sorted);
  int32_t* p2r = at<int32_t>(workspace, L.p2r);
  int32_t* tiles = at<int32_t>(workspace, L.tiles);
  int32_t* ntiles = at<int32_t>(workspace, L.ntiles);
  uint16_t* h = at<uint16_t>(workspace, L.h);
  uint16_t* y = at<uint16_t>(workspace, L.y);
  auto mark = [&](int i) -> hipError_t {
    return ev ? hipEventRecord(static_cast<hipEvent_t>(ev[i]), hs) : hipSuccess;
  };
  BEAM_TRY_HIP(mark(0));
  BEAM_TRY_HIP(beam::launch_router_logits(s, T, L.ks, xb, w_router, partial, hs));
  BEAM_TRY_HIP(mark(1));
  BEAM_TRY_HIP(beam::launch_router_select(s, T, L.ks, partial, b_router, ids, w, hs));
  BEAM_TRY_HIP(mark(2));
  BEAM_TRY_HIP(beam::launch_permute(s, T, ids, L.nchunks, at<uint64_t>(workspace, L.masks),
                                    at<int32_t>(workspace, L.counts), offsets, sorted, p2r,
                                    beam::expert_tile_rows(s, T), tiles, ntiles, hs));
  BEAM_TRY_HIP(mark(3));
  BEAM_TRY_HIP(beam::launch_gateup(s, T, xb, w_gate, w_up, s_gate, s_up, offsets, sorted, tiles, ntiles,
                                   L.max_tiles, 1, nullptr, h, hs));
  BEAM_TRY_HIP(mark(4));
  BEAM_TRY_HIP(beam::launch_down(s, T, h, w_down, s_down, offsets, tiles, ntiles, L.max_tiles, 1, nullptr, y, hs));
  BEAM_TRY_HIP(mark(5));
  if (blk)
    BEAM_TRY_HIP(beam::launch_combine_norm_mix(s, T, y, w, p2r, blk->eps, blk->gamma_post, blk->a, blk->b,
                                               blk->stream_in, blk->stream_out, blk->moe_out, hs));
  else
    BEAM_TRY_HIP(beam::launch_combine(s, T, y, w, p2r, out, hs));
  BEAM_TRY_HIP(mark(6));
  return BEAM_MOE_OK;
}

// ---- dense SwiGLU MLP (one expert, every token) ----

int check_dense_config(const beam_dense_config* c) {
  if (!c || c->hidden <= 0 || c->inter <= 0) return BEAM_MOE_ERR_INVALID;
  if (c->weight_type != BEAM_MOE_W_BF16 && c->weight_type != BEAM_MOE_W_FP8_E4M3 && c->weight_type != BEAM_MOE_W_MXFP4)
    return BEAM_MOE_ERR_INVALID;
  if (c->weight_layout != BEAM_MOE_LAYOUT_ROWS && c->weight_layout != BEAM_MOE_LAYOUT_FRAGMENTS)
    return BEAM_MOE_ERR_INVALID;
  if (c->hidden % 128 != 0 || c->inter % 128 != 0) return BEAM_MOE_ERR_UNSUPPORTED;
  if (c->weight_type == BEAM_MOE_W_MXFP4 && (c->hidden % 256 != 0 || c->inter % 256 != 0)) return BEAM_MOE_ERR_UNSUPPORTED;
  if (c->weight_type == BEAM_MOE_W_MXFP4 && c->weight_layout == BEAM_MOE_LAYOUT_FRAGMENTS &&
      (c->hidden % 512 != 0 || c->inter % 512 != 0))
    return BEAM_MOE_ERR_UNSUPPORTED;
  return BEAM_MOE_OK;
}

Shape dense_shape(const beam_dense_config* c) {
  Shape s{c->hidden, c->inter, 1, 1, 1, 1, 1.0f, c->weight_type == BEAM_MOE_W_FP8_E4M3 ? 1 : 0};
  s.dense = 1;
  s.mx = c->weight_type == BEAM_MOE_W_MXFP4;
  s.packed = c->weight_layout == BEAM_MOE_LAYOUT_FRAGMENTS;
  return s;
}

struct DenseLayout {
  size_t offsets, sorted, tiles, ntiles, h, part, total;
  int max_tiles, tile_rows, gkparts, kparts;
};

DenseLayout dense_layout(const Shape& s, int T) {
  DenseLayout L{};
  L.tile_rows = beam::expert_tile_rows(s, T);
  L.max_tiles = (T + L.tile_rows - 1) / L.tile_rows + 1;
  L.gkparts = beam::gateup_kparts(s, T);
  L.kparts = beam::down_kparts(s, T);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  L.offsets = take(2 * 4);
  L.sorted = take((size_t)T * 4);
  L.tiles = take((size_t)L.max_tiles * 8);
  L.ntiles = take(4);
  L.h = take((size_t)T * s.I * 2);
  // fp32 partial sums of the split GEMMs (gate/up's are consumed before down runs: one region)
  const size_t gpart = L.gkparts > 1 ? (size_t)L.gkparts * T * 2 * s.I * 4 : 0;
  const size_t dpart = L.kparts > 1 ? (size_t)L.kparts * T * s.H * 4 : 0;
  if (gpart || dpart) L.part = take(std::max(gpart, dpart));
  L.total = off;
  return L;
}

bool valid_eps(float eps) { return isfinite(eps) && eps > 0.f; }

}  // namespace

extern "C" {


const char* beam_moe_status_string(int status) {
  switch (status) {
    case BEAM_MOE_OK: return "ok";
    case BEAM_MOE_ERR_INVALID: return "invalid argument";
    case BEAM_MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case BEAM_MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case BEAM_MOE_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int beam_moe_workspace_bytes(const beam_moe_config* cfg, int32_t T, int32_t op, size_t* bytes) {
  const int st = check_config(cfg);
  if (st != BEAM_MOE_OK) return st;
  if (!bytes || T < 0 || T > BEAM_MOE_MAX_TOKENS) return BEAM_MOE_ERR_INVALID;
  if (op != BEAM_MOE_OP_ROUTE && op != BEAM_MOE_OP_PERMUTE && op != BEAM_MOE_OP_FORWARD && op != BEAM_MOE_OP_BLOCK)
    return BEAM_MOE_ERR_INVALID;
  if (op == BEAM_MOE_OP_BLOCK && cfg->hidden > BEAM_MOE_MAX_NORM_HIDDEN) return BEAM_MOE_ERR_UNSUPPORTED;
  *bytes = T == 0 ? 0 : make_layout(shape_of(cfg), T, op).total;
  return BEAM_MOE_OK;
}

int beam_moe_route(const beam_moe_config* cfg, int32_t T, const void* x, const float* w_router,
                   const float* b_router, int32_t* topk_ids, float* topk_w, void* workspace,
                   size_t workspace_bytes, void* stream) {
  int st = check_config(cfg);
  if (st != BEAM_MOE_OK) return st;
  if (T < 0 || T > BEAM_MOE_MAX_TOKENS) return BEAM_MOE_ERR_INVALID;
  if (T == 0) return BEAM_MOE_OK;
  if (!x || !w_router || !topk_ids || !topk_w) return BEAM_MOE_ERR_INVALID;
  if (!aligned16(x) || !aligned16(w_router) || !aligned4(topk_ids) || !aligned4(topk_w) ||
      (b_router && !aligned4(b_router)))
    return BEAM_MOE_ERR_INVALID;
  const Shape s = shape_of(cfg);
  const Layout L = make_layout(s, T, BEAM_MOE_OP_ROUTE);
  if (!workspace || workspace_bytes < L.total || !aligned16(workspace)) return BEAM_MOE_ERR_WORKSPACE;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  float* partial = at<float>(workspace, L.logits);
  BEAM_TRY_HIP(beam::launch_router_logits(s, T, L.ks, static_cast<const uint16_t*>(x), w_router, partial, hs));
  BEAM_TRY_HIP(beam::launch_router_select(s, T, L.ks, partial, b_router, topk_ids, topk_w, hs));
  return BEAM_MOE_OK;
}

int beam_moe_permute(const beam_moe_config* cfg, int32_t T, const int32_t* topk_ids, int32_t* expert_offsets,
                     int32_t* sorted_pairs, int32_t* pair_to_row, void* workspace, size_t workspace_bytes,
                     void* stream) {
  int st = check_config(cfg);
  if (st != BEAM_MOE_OK) return st;
  if (T < 0 || T > BEAM_MOE_MAX_TOKENS) return BEAM_MOE_ERR_INVALID;
  if (T == 0) return BEAM_MOE_OK;
  if (!topk_ids || !expert_offsets || !sorted_pairs || !pair_to_row) return BEAM_MOE_ERR_INVALID;
  if (!aligned4(topk_ids) || !aligned4(expert_offsets) || !aligned4(sorted_pairs) || !aligned4(pair_to_row))
    return BEAM_MOE_ERR_INVALID;
  const Shape s = shape_of(cfg);
  const Layout L = make_layout(s, T, BEAM_MOE_OP_PERMUTE);
  if (!workspace || workspace_bytes < L.total || !aligned16(workspace)) return BEAM_MOE_ERR_WORKSPACE;
  BEAM_TRY_HIP(beam::launch_permute(s, T, topk_ids, L.nchunks, at<uint64_t>(workspace, L.masks),
                                    at<int32_t>(workspace, L.counts), expert_offsets, sorted_pairs, pair_to_row,
                                    0, nullptr, nullptr, static_cast<hipStream_t>(stream)));
  return BEAM_MOE_OK;
}

int beam_moe_forward(const beam_moe_config* cfg, int32_t T, const void* x, const float* w_router,
                     const float* b_router, const void* w_gate, const void* w_up, const void* w_down,
                     const void* s_gate, const void* s_up, const void* s_down, void* out, int32_t* topk_ids_out,
                     float* topk_w_out, void* workspace, size_t workspace_bytes, void* stream) {
  return beam_moe_forward_timed(cfg, T, x, w_router, b_router, w_gate, w_up, w_down, s_gate, s_up, s_down, out,
                                topk_ids_out, topk_w_out, workspace, workspace_bytes, stream, nullptr);
}

int beam_moe_forward_timed(const beam_moe_config* cfg, int32_t T, const void* x, const float* w_router,
                           const float* b_router, const void* w_gate, const void* w_up, const void* w_down,
                           const void* s_gate, const void* s_up, const void* s_down, void* out,
                           int32_t* topk_ids_out, float* topk_w_out, void* workspace, size_t workspace_bytes,
                           void* stream, void* const* stage_events) {
  int st = check_config(cfg);
  if (st != BEAM_MOE_OK) return st;
  if (T < 0 || T > BEAM_MOE_MAX_TOKENS) return BEAM_MOE_ERR_INVALID;
  if (T == 0) return BEAM_MOE_OK;
  st = check_forward_args(cfg, x, w_router, b_router, w_gate, w_up, w_down, s_gate, s_up, s_down, out, topk_ids_out,
                          topk_w_out);
  if (st != BEAM_MOE_OK) return st;
  const Shape s = shape_of(cfg);
  const Layout L = make_layout(s, T, BEAM_MOE_OP_FORWARD);
  if (!workspace || workspace_bytes < L.total || !aligned16(workspace)) return BEAM_MOE_ERR_WORKSPACE;
  return run_forward(s, L, T, static_cast<const uint16_t*>(x), w_router, b_router, w_gate, w_up, w_down, s_gate, s_up,
                     s_down, static_cast<uint16_t*>(out), topk_ids_out, topk_w_out, workspace,
                     static_cast<hipStream_t>(stream), stage_events, nullptr);
}

// ---- allocation-free forward: the workspace is a fixed device array of this library ----
// In host code `scratch` names the symbol only; kernels get its device address, looked up per device.
static __device__ __align__(256) uint8_t scratch[BEAM_MOE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

// The current device's copy of `scratch` (each GPU holds its own), found once per device with that
// device current and kept.
int scratch_address(void** addr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return BEAM_MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return BEAM_MOE_ERR_HIP;
    g_scratch_addr[dev] = p;
  }
  *addr = g_scratch_addr[dev];
  return BEAM_MOE_OK;
}
}  // namespace

int beam_moe_forward_noalloc(const beam_moe_config* cfg, int32_t T, const void* x, const float* w_router,
                             const float* b_router, const void* w_gate, const void* w_up, const void* w_down,
                             const void* s_gate, const void* s_up, const void* s_down, void* out,
                             int32_t* topk_ids_out, float* topk_w_out, void* stream) {
  int st = check_config(cfg);
  if (st != BEAM_MOE_OK) return st;
  if (T < 0 || T > BEAM_MOE_MAX_TOKENS) return BEAM_MOE_ERR_INVALID;
  if (T == 0) return BEAM_MOE_OK;
  st = check_forward_args(cfg, x, w_router, b_router, w_gate, w_up, w_down, s_gate, s_up, s_down, out, topk_ids_out,
                          topk_w_out);
  if (st != BEAM_MOE_OK) return st;
  const Shape s = shape_of(cfg);
  const Layout L = make_layout(s, T, BEAM_MOE_OP_FORWARD);
  if (L.total > BEAM_MOE_NOALLOC_SCRATCH_BYTES) return BEAM_MOE_ERR_WORKSPACE;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != BEAM_MOE_OK) return st;
  return run_forward(s, L, T, static_cast<const uint16_t*>(x), w_router, b_router, w_gate, w_up, w_down, s_gate, s_up,
                     s_down, static_cast<uint16_t*>(out), topk_ids_out, topk_w_out, ws,
                     static_cast<hipStream_t>(stream), nullptr, nullptr);
}

int beam_moe_rms_norm(int32_t T, int32_t hidden, const void* x, const float* gamma, float eps, void* out,
                      void* stream) {
  if (T < 0 || T > BEAM_MOE_MAX_TOKENS || hidden <= 0 || hidden % 8 != 0 || !valid_eps(eps))
    return BEAM_MOE_ERR_INVALID;
  if (hidden > BEAM_MOE_MAX_NORM_HIDDEN) return BEAM_MOE_ERR_UNSUPPORTED;
  if (T == 0) return BEAM_MOE_OK;
  if (!x || !gamma || !out || !aligned16(x) || !aligned16(out) || !aligned4(gamma)) return BEAM_MOE_ERR_INVALID;
  BEAM_TRY_HIP(beam::launch_rms_norm(T, hidden, eps, static_cast<const uint16_t*>(x), gamma,
                                     static_cast<uint16_t*>(out), static_cast<hipStream_t>(stream)));
  return BEAM_MOE_OK;
}

int beam_moe_block_forward(const beam_moe_config* cfg, int32_t T, int32_t step, float eps, const void* stream_in,
                           const float* gamma_pre, const float* gamma_post, const float* w_router,
                           const float* b_router, const void* w_gate, const void* w_up, const void* w_down,
                           const void* s_gate, const void* s_up, const void* s_down, void* stream_out,
                           void* moe_out, int32_t* topk_ids_out, float* topk_w_out, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return beam_moe_block_forward_timed(cfg, T, step, eps, stream_in, gamma_pre, gamma_post, w_router, b_router, w_gate,
                                      w_up, w_down, s_gate, s_up, s_down, stream_out, moe_out, topk_ids_out,
                                      topk_w_out, workspace, workspace_bytes, stream, nullptr);
}

int beam_moe_block_forward_timed(const beam_moe_config* cfg, int32_t T, int32_t step, float eps,
                                 const void* stream_in, const float* gamma_pre, const float* gamma_post,
                                 const float* w_router, const float* b_router, const void* w_gate, const void* w_up,
                                 const void* w_down, const void* s_gate, const void* s_up, const void* s_down,
                                 void* stream_out, void* moe_out, int32_t* topk_ids_out, float* topk_w_out,
                                 void* workspace, size_t workspace_bytes, void* stream, void* const* stage_events) {
  int st = check_config(cfg);
  if (st != BEAM_MOE_OK) return st;
  if (T < 0 || T > BEAM_MOE_MAX_TOKENS || step < 2 || !valid_eps(eps)) return BEAM_MOE_ERR_INVALID;
  if (cfg->hidden > BEAM_MOE_MAX_NORM_HIDDEN) return BEAM_MOE_ERR_UNSUPPORTED;
  if (T == 0) return BEAM_MOE_OK;
  // the forward's `out` is the block's stream_out; x (the pre-norm output) lives in the workspace
  st = check_forward_args(cfg, stream_in, w_router, b_router, w_gate, w_up, w_down, s_gate, s_up, s_down, stream_out,
                          topk_ids_out, topk_w_out);
  if (st != BEAM_MOE_OK) return st;
  if (!gamma_pre || !gamma_post || !aligned4(gamma_pre) || !aligned4(gamma_post) || (moe_out && !aligned16(moe_out)))
    return BEAM_MOE_ERR_INVALID;
  const Shape s = shape_of(cfg);
  const Layout L = make_layout(s, T, BEAM_MOE_OP_BLOCK);
  if (!workspace || workspace_bytes < L.total || !aligned16(workspace)) return BEAM_MOE_ERR_WORKSPACE;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  uint16_t* xn = at<uint16_t>(workspace, L.xn);
  if (stage_events) BEAM_TRY_HIP(hipEventRecord(static_cast<hipEvent_t>(stage_events[0]), hs));
  BEAM_TRY_HIP(beam::launch_rms_norm(T, s.H, eps, static_cast<const uint16_t*>(stream_in), gamma_pre, xn, hs));
  const BlockEpilogue blk{eps, static_cast<float>(sqrt(static_cast<double>(step - 1) / step)),
                          static_cast<float>(1.0 / sqrt(static_cast<double>(step))), gamma_post,
                          static_cast<const uint16_t*>(stream_in), static_cast<uint16_t*>(stream_out),
                          static_cast<uint16_t*>(moe_out)};
  return run_forward(s, L, T, xn, w_router, b_router, w_gate, w_up, w_down, s_gate, s_up, s_down, nullptr,
                     topk_ids_out, topk_w_out, workspace, hs, stage_events ? stage_events + 1 : nullptr, &blk);
}


int beam_dense_workspace_bytes(const beam_dense_config* cfg, int32_t T, size_t* bytes) {
  const int st = check_dense_config(cfg);
  if (st != BEAM_MOE_OK) return st;
  if (!bytes || T < 0 || T > BEAM_MOE_MAX_TOKENS) return BEAM_MOE_ERR_INVALID;
  *bytes = T == 0 ? 0 : dense_layout(dense_shape(cfg), T).total;
  return BEAM_MOE_OK;
}

int beam_dense_mlp_forward(const beam_dense_config* cfg, int32_t T, const void* x, const void* w_gate,
                           const void* w_up, const void* w_down, const void* s_gate, const void* s_up,
                           const void* s_down, void* out, void* workspace, size_t workspace_bytes, void* stream) {
  return beam_dense_mlp_forward_timed(cfg, T, x, w_gate, w_up, w_down, s_gate, s_up, s_down, out, workspace,
                                      workspace_bytes, stream, nullptr);
}

int beam_dense_mlp_forward_timed(const beam_dense_config* cfg, int32_t T, const void* x, const void* w_gate,
                                 const void* w_up, const void* w_down, const void* s_gate, const void* s_up,
                                 const void* s_down, void* out, void* workspace, size_t workspace_bytes,
                                 void* stream, void* const* stage_events) {
  int st = check_dense_config(cfg);
  if (st != BEAM_MOE_OK) return st;
  if (T < 0 || T > BEAM_MOE_MAX_TOKENS) return BEAM_MOE_ERR_INVALID;
  if (T == 0) return BEAM_MOE_OK;
  if (!x || !w_gate || !w_up || !w_down || !out) return BEAM_MOE_ERR_INVALID;
  const bool scaled = cfg->weight_type != BEAM_MOE_W_BF16;   // fp8 per-channel or MXFP4 block scales
  if (scaled != (s_gate != nullptr) || scaled != (s_up != nullptr) || scaled != (s_down != nullptr))
    return BEAM_MOE_ERR_INVALID;
  if (!aligned16(x) || !aligned16(w_gate) || !aligned16(w_up) || !aligned16(w_down) || !aligned16(out) ||
      (cfg->weight_type == BEAM_MOE_W_FP8_E4M3 && (!aligned4(s_gate) || !aligned4(s_up) || !aligned4(s_down))) ||
      (cfg->weight_type == BEAM_MOE_W_MXFP4 && (!aligned16(s_gate) || !aligned16(s_up) || !aligned16(s_down))))
    return BEAM_MOE_ERR_INVALID;
  const Shape s = dense_shape(cfg);
  const DenseLayout L = dense_layout(s, T);
  if (!workspace || workspace_bytes < L.total || !aligned16(workspace)) return BEAM_MOE_ERR_WORKSPACE;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  int32_t* offsets = at<int32_t>(workspace, L.offsets);
  int32_t* sorted = at<int32_t>(workspace, L.sorted);
  int32_t* tiles = at<int32_t>(workspace, L.tiles);
  int32_t* ntiles = at<int32_t>(workspace, L.ntiles);
  uint16_t* h = at<uint16_t>(workspace, L.h);
  float* part = (L.kparts > 1 || L.gkparts > 1) ? at<float>(workspace, L.part) : nullptr;
  auto mark = [&](int i) -> hipError_t {
    return stage_events ? hipEventRecord(static_cast<hipEvent_t>(stage_events[i]), hs) : hipSuccess;
  };
  BEAM_TRY_HIP(mark(0));
  BEAM_TRY_HIP(beam::launch_dense_setup(T, L.tile_rows, offsets, sorted, tiles, ntiles, hs));
  BEAM_TRY_HIP(mark(1));
  BEAM_TRY_HIP(beam::launch_gateup(s, T, static_cast<const uint16_t*>(x), w_gate, w_up, s_gate, s_up, offsets, sorted,
                                   tiles, ntiles, L.max_tiles, L.gkparts, part, h, hs));
  BEAM_TRY_HIP(mark(2));
  BEAM_TRY_HIP(beam::launch_down(s, T, h, w_down, s_down, offsets, tiles, ntiles, L.max_tiles, L.kparts, part,
                                 static_cast<uint16_t*>(out), hs));
  BEAM_TRY_HIP(mark(3));
  return BEAM_MOE_OK;
}

int beam_mxfp4_quantize(int32_t rows, int32_t cols, const void* w, void* codes, void* scales, void* stream) {
  if (rows < 0 || cols < 0 || cols % 32 != 0) return BEAM_MOE_ERR_INVALID;
  if (rows == 0 || cols == 0) return BEAM_MOE_OK;
  if (!w || !codes || !scales || !aligned16(w) || !aligned16(codes)) return BEAM_MOE_ERR_INVALID;
  BEAM_TRY_HIP(beam::launch_mxfp4_quantize(rows, cols, static_cast<const uint16_t*>(w), static_cast<uint8_t*>(codes),
                                           static_cast<uint8_t*>(scales), static_cast<hipStream_t>(stream)));
  return BEAM_MOE_OK;
}

}  // extern "C"

namespace {

// Row order -> fragment order with column slices of slice_bytes (64: weights, 16: MXFP4 scales).
int pack_fragments(int64_t rows, int32_t row_bytes, int slice_bytes, const void* src, void* dst, void* stream) {
  if (rows < 0 || rows % 16 != 0 || row_bytes <= 0 || row_bytes % slice_bytes != 0) return BEAM_MOE_ERR_INVALID;
  if (rows > (int64_t)1 << 40 || (int64_t)row_bytes > ((int64_t)1 << 40) / (rows ? rows : 1))
    return BEAM_MOE_ERR_INVALID;
  if (rows == 0) return BEAM_MOE_OK;
  if (!src || !dst || !aligned16(src) || !aligned16(dst)) return BEAM_MOE_ERR_INVALID;
  const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
  const uintptr_t n = (uintptr_t)rows * (uintptr_t)row_bytes;
  if (a < b + n && b < a + n) return BEAM_MOE_ERR_INVALID;
  BEAM_TRY_HIP(beam::launch_pack_fragments(rows, row_bytes, slice_bytes, src, dst, static_cast<hipStream_t>(stream)));
  return BEAM_MOE_OK;
}

}  // namespace

extern "C" {

int beam_moe_pack_weights(int64_t rows, int32_t row_bytes, const void* src, void* dst, void* stream) {
  return pack_fragments(rows, row_bytes, 64, src, dst, stream);
}

int beam_moe_pack_scales(int64_t rows, int32_t row_bytes, const void* src, void* dst, void* stream) {
  return pack_fragments(rows, row_bytes, 16, src, dst, stream);
}

}  // extern "C"
