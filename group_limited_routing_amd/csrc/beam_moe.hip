// C ABI of the Beam MoE block: argument checks, workspace layout, and the
// order of kernel launches. See include/beam_moe.h for the contract.
#include "../../include/beam_moe.h"

#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "common.h"
#include "internal.h"

// Scratch of beam_moe_forward_noalloc: one array per GPU (each device holds
// its own copy at its own address), from the library's load until the
// process ends. Host code never passes this name to a kernel: there it is a
// host-side stand-in; the device address comes from hipGetSymbolAddress.
static __device__ __align__(256) uint8_t scratch[BEAM_MOE_NOALLOC_MAX_BYTES];

namespace beam {

static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

Layout make_layout(const Shape& s) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  const size_t T = (size_t)s.T, k = (size_t)s.top_k, E = (size_t)s.E;
  const size_t H = (size_t)s.H, I = (size_t)s.I, P = T * k;
  L.nchunks = (int)((T + kChunk - 1) / kChunk);
  // the largest bound of the tile heights any variant uses
  L.max_mtiles = std::max(mtile_bound(s, kStreamBM), mtile_bound(s, kMixedBM));
  L.z = take(T * E * 4);
  L.idx = take(P * 4);
  L.w = take(P * 4);
  L.chist = take((size_t)L.nchunks * E * 4);
  L.cbase = take((size_t)L.nchunks * E * 4);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  L.meta = take(64 * 4);
  L.tile_e = take((size_t)L.max_mtiles * 4);
  L.tile_r = take((size_t)L.max_mtiles * 4);
  L.e_tstart = take(E * 4);
  L.e_ntiles = take(E * 4);
  L.stok = take(P * 4);
  L.sw = take(P * 4);
  L.inv = take(P * 4);
  if (s.w_fp8) {
    L.xq = take(T * H);      // e4m3 codes of x, per-token scale
    L.xs = take(T * 4);
    L.hamax = take(P * 4);   // running max |h| per sorted row (float bits)
    L.h = take(P * I * 2);   // bf16 SwiGLU output before quantisation
    L.hq = take(P * I);      // its e4m3 codes
    L.hs = take(P * 4);      // per-row scale of the quantised h
  } else {
    L.xq = L.xs = L.hamax = L.hq = L.hs = 0;
    L.h = take(P * I * 2);   // bf16 SwiGLU output
  }
  L.y = take(P * H * 2);     // bf16 expert outputs, scaled by rsf * w
  L.wsplit = L.zpart = 0;
  L.router_ks = L.router_x3 = 0;
  if (s.T <= kRouterSplitMaxT) {
    L.router_ks = router_small_split(s.H);
    L.zpart = take((size_t)L.router_ks * T * E * 4);
  } else if (!s.x_f32) {
    L.router_x3 = 1;
    L.router_ks = router_ksplit(s.T, s.H);
    L.wsplit = take(3 * E * H * 2);
    L.zpart = take((size_t)L.router_ks * T * E * 4);
  }
  L.total = off;
  return L;
}

// Backward pass: the forward's routing and permutation buffers (its y region
// holds the input-gradient rows), then the backward's own.
struct BwdLayout {
  Layout f;
  size_t ssel, gu, d, part, dz, pcol, xt, gyt, ht, dgt, dut, total;
  size_t pstride;  // columns of the transposed copies (segments of 32-column blocks)
  int nparts;      // partial sums of h . q per sorted row
};

BwdLayout make_backward_layout(const Shape& s, bool wgrads) {
  BwdLayout B{};
  B.f = make_layout(s);
  size_t off = B.f.total;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  const size_t P = (size_t)s.T * s.top_k, H = (size_t)s.H, I = (size_t)s.I, E = (size_t)s.E;
  B.nparts = (int)(I / 256) * 4;
  B.ssel = take(P * 4);
  B.gu = take(P * 2 * I * 4);  // fp32: the SwiGLU derivative near its zero needs g exactly
  B.d = take(P * 2 * I * 2);
  B.part = take(P * (size_t)B.nparts * 4);
  B.dz = take(P * 4);
  B.pcol = take((E + 1) * 4);
  // every expert's segment is padded to a multiple of 32 columns
  B.pstride = (P + 32 * E + 31) / 32 * 32;
  if (wgrads) {
    B.xt = take(H * B.pstride * 2);
    B.gyt = take(H * B.pstride * 2);
    B.ht = take(I * B.pstride * 2);
    B.dgt = take(I * B.pstride * 2);
    B.dut = take(I * B.pstride * 2);
  }
  B.total = off;
  return B;
}

}  // namespace beam

using namespace beam;

namespace {

constexpr int kMaxT = 1 << 22;

beam_status check_config(const beam_moe_config* c) {
  if (!c) return BEAM_ERR_NULL;
  if (c->n_experts != kExperts) return BEAM_ERR_CONFIG;
  const int G = c->n_group;
  if (G < 1 || G > 64 || (G & (G - 1)) != 0) return BEAM_ERR_CONFIG;
  if (c->topk_group < 1 || c->topk_group > G) return BEAM_ERR_CONFIG;
  const int gs = kExperts / G;
  if (c->top_k < 1 || c->top_k > 32 || c->top_k > c->topk_group * gs) return BEAM_ERR_CONFIG;
  if (!isfinite(c->routed_scaling_factor)) return BEAM_ERR_CONFIG;
  if (c->x_dtype != BEAM_F32 && c->x_dtype != BEAM_BF16) return BEAM_ERR_DTYPE;
  if (c->w_dtype != BEAM_BF16 && c->w_dtype != BEAM_FP8_E4M3 && c->w_dtype != BEAM_MXFP4)
    return BEAM_ERR_DTYPE;
  if (c->w_layout != BEAM_LAYOUT_ROW_MAJOR && c->w_layout != BEAM_LAYOUT_PACKED)
    return BEAM_ERR_CONFIG;
  if (c->w_dtype == BEAM_MXFP4 && c->w_layout != BEAM_LAYOUT_PACKED) return BEAM_ERR_CONFIG;
  const int step = c->w_dtype == BEAM_MXFP4 ? 512 : 128;
  if (c->hidden <= 0 || c->hidden % step != 0 || c->hidden > 65536) return BEAM_ERR_SHAPE;
  if (c->intermediate <= 0 || c->intermediate % step != 0 || c->intermediate > 65536)
    return BEAM_ERR_SHAPE;
  return BEAM_OK;
}

Shape shape_of(const beam_moe_config* c, int32_t T) {
  Shape s;
  s.T = T;
  s.H = c->hidden;
  s.I = c->intermediate;
  s.E = c->n_experts;
  s.n_group = c->n_group;
  s.topk_group = c->topk_group;
  s.top_k = c->top_k;
  s.rsf = c->routed_scaling_factor;
  s.x_f32 = c->x_dtype == BEAM_F32;
  // fp8 and MXFP4 weights share the E4M3 activation path
  s.w_fp8 = c->w_dtype == BEAM_FP8_E4M3 || c->w_dtype == BEAM_MXFP4;
  s.w_mx4 = c->w_dtype == BEAM_MXFP4;
  s.n_run = s.E;
  s.w_packed = c->w_layout == BEAM_LAYOUT_PACKED;
  return s;
}

bool misaligned(const void* p) { return p && (((uintptr_t)p) & 15u) != 0; }

// Optional stage timing (beam_moe_profile_begin / _end): a pair of HIP
// events around each selected stage's launch, on the call's stream.
struct Profiler {
  struct Rec {
    int stage;
    hipEvent_t a, b;
  };
  std::mutex mu;
  bool on = false;
  uint32_t mask = 0;
  std::vector<Rec> recs;

  void release() {
    for (auto& r : recs) {
      hipEventDestroy(r.a);
      hipEventDestroy(r.b);
    }
    recs.clear();
  }
};
Profiler g_prof;

template <typename F>
beam_status staged(int stage, hipStream_t st, F&& launch) {
  bool timed;
  {
    std::lock_guard<std::mutex> lk(g_prof.mu);
    timed = g_prof.on && ((g_prof.mask >> stage) & 1u);
  }
  hipEvent_t a = nullptr, b = nullptr;
  if (timed) {
    if (hipEventCreate(&a) != hipSuccess) return BEAM_ERR_HIP;
    if (hipEventCreate(&b) != hipSuccess || hipEventRecord(a, st) != hipSuccess) {
      hipEventDestroy(a);
      if (b) hipEventDestroy(b);
      return BEAM_ERR_HIP;
    }
  }
  const hipError_t le = launch();
  if (timed) {
    const hipError_t re = hipEventRecord(b, st);
    std::lock_guard<std::mutex> lk(g_prof.mu);
    if (le == hipSuccess && re == hipSuccess) {
      g_prof.recs.push_back({stage, a, b});
    } else {
      hipEventDestroy(a);
      hipEventDestroy(b);
    }
  }
  return le == hipSuccess ? BEAM_OK : BEAM_ERR_HIP;
}

#define STAGE(id, call)                                                        \
  do {                                                                         \
    const beam_status stage_status_ = staged((id), st, [&]() { return (call); }); \
    if (stage_status_ != BEAM_OK) return stage_status_;                        \
  } while (0)

// Routing and permutation shared by route and forward. Fills the sorted
// arrays when `permute` is set; `BM` is the M-tile height of the expert GEMMs.
struct Buffers {
  float* z;
  float* zpart;
  uint16_t* wsplit;
  int32_t* idx;
  float* w;
  int32_t *chist, *cbase, *counts, *offsets, *meta, *tile_e, *tile_r, *e_tstart, *e_ntiles, *stok,
      *inv;
  float* sw;
};

Buffers carve(const Layout& L, void* ws) {
  uint8_t* b = (uint8_t*)ws;
  Buffers B;
  B.z = (float*)(b + L.z);
  B.zpart = (float*)(b + L.zpart);
  B.wsplit = (uint16_t*)(b + L.wsplit);
  B.idx = (int32_t*)(b + L.idx);
  B.w = (float*)(b + L.w);
  B.chist = (int32_t*)(b + L.chist);
  B.cbase = (int32_t*)(b + L.cbase);
  B.counts = (int32_t*)(b + L.counts);
  B.offsets = (int32_t*)(b + L.offsets);
  B.meta = (int32_t*)(b + L.meta);
  B.tile_e = (int32_t*)(b + L.tile_e);
  B.tile_r = (int32_t*)(b + L.tile_r);
  B.e_tstart = (int32_t*)(b + L.e_tstart);
  B.e_ntiles = (int32_t*)(b + L.e_ntiles);
  B.stok = (int32_t*)(b + L.stok);
  B.sw = (float*)(b + L.sw);
  B.inv = (int32_t*)(b + L.inv);
  return B;
}

// Router logits and selection. Up to kRouterSplitMaxT tokens: fp32 MFMA
// partial logits over several K ranges. More bf16 tokens: split weights,
// partial logits on the bf16 matrix cores. Partials are summed by the
// selection (which stores the sum when logits are requested). More fp32
// tokens: fp32 MFMA logits straight into z.
beam_status route_tokens(const Shape& s, const Layout& L, const Buffers& B, const void* x,
                         const float* router_w, const float* bias, float* logits_out,
                         int32_t* idx, float* w, hipStream_t st, float* s_sel = nullptr) {
  const int T = s.T;
  if (L.router_ks > 0) {
    if (L.router_x3)
      STAGE(BEAM_STAGE_ROUTER_LOGITS, launch_router_x3((const uint16_t*)x, router_w, B.wsplit,
                                                       B.zpart, T, s.H, L.router_ks, st));
    else
      STAGE(BEAM_STAGE_ROUTER_LOGITS, launch_router_logits_split(x, s.x_f32, router_w, B.zpart, T,
                                                                 s.H, L.router_ks, st));
    STAGE(BEAM_STAGE_SELECT, launch_select(B.zpart, L.router_ks, (size_t)T * s.E, logits_out, bias, T,
                                           s.n_group, s.topk_group, s.top_k, idx, w, s_sel, st));
  } else {
    float* z = logits_out ? logits_out : B.z;
    STAGE(BEAM_STAGE_ROUTER_LOGITS, launch_router_logits(x, s.x_f32, router_w, z, T, s.H, st));
    STAGE(BEAM_STAGE_SELECT, launch_select(z, 1, 0, nullptr, bias, T, s.n_group, s.topk_group,
                                           s.top_k, idx, w, s_sel, st));
  }
  return BEAM_OK;
}

}  // namespace

extern "C" {

size_t beam_moe_workspace_bytes(const beam_moe_config* cfg, int32_t T) {
  if (check_config(cfg) != BEAM_OK || T < 0 || T > kMaxT) return 0;
  return make_layout(shape_of(cfg, T)).total;
}

const char* beam_moe_status_string(int32_t status) {
  switch (status) {
    case BEAM_OK: return "ok";
    case BEAM_ERR_NULL: return "a required pointer is NULL";
    case BEAM_ERR_CONFIG: return "routing parameters outside the supported set";
    case BEAM_ERR_SHAPE: return "token count, hidden or intermediate size outside the supported set";
    case BEAM_ERR_DTYPE: return "unsupported dtype combination or missing fp8 scales";
    case BEAM_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case BEAM_ERR_WORKSPACE: return "workspace missing or smaller than beam_moe_workspace_bytes()";
    case BEAM_ERR_HIP: return "the HIP runtime reported an error";
    default: return "unknown status";
  }
}

beam_status beam_moe_route(const beam_moe_config* cfg, int32_t T, const void* x,
                           const float* router_w, const float* expert_bias, int32_t* topk_idx,
                           float* topk_w, float* router_logits, int32_t* expert_counts,
                           void* workspace, size_t workspace_bytes, void* stream) {
  const beam_status cs = check_config(cfg);
  if (cs != BEAM_OK) return cs;
  if (T < 0 || T > kMaxT) return BEAM_ERR_SHAPE;
  if (T == 0) return BEAM_OK;
  if (!x || !router_w || !expert_bias || !topk_idx || !topk_w) return BEAM_ERR_NULL;
  if (!workspace) return BEAM_ERR_WORKSPACE;
  if (misaligned(x) || misaligned(router_w) || misaligned(expert_bias) || misaligned(topk_idx) ||
      misaligned(topk_w) || misaligned(router_logits) || misaligned(expert_counts) ||
      misaligned(workspace))
    return BEAM_ERR_ALIGN;
  const Shape s = shape_of(cfg, T);
  const Layout L = make_layout(s);
  if (workspace_bytes < L.total) return BEAM_ERR_WORKSPACE;

  hipStream_t st = (hipStream_t)stream;
  Buffers B = carve(L, workspace);
  const beam_status rs = route_tokens(s, L, B, x, router_w, expert_bias, router_logits, topk_idx,
                                      topk_w, st);
  if (rs != BEAM_OK) return rs;
  if (expert_counts) {
    STAGE(BEAM_STAGE_PERM_HIST, launch_perm_hist(topk_idx, T, s.top_k, B.chist, st));
    STAGE(BEAM_STAGE_PERM_SCAN, launch_perm_scan(B.chist, L.nchunks, kTiledBM, B.cbase, B.counts, B.offsets,
                                 B.meta, B.tile_e, B.tile_r, B.e_tstart, B.e_ntiles,
                                 expert_counts, st));
  }
  return BEAM_OK;
}

}  // extern "C"

namespace {

// Shift a per-expert array's base so that expert e (>= e0) is found at
// e * stride from it: the arrays of an expert shard hold experts e0.. only.
// Integer arithmetic: the shifted base itself is never dereferenced.
const void* shard_base(const void* p, int e0, size_t stride_bytes) {
  return p ? (const void*)((uintptr_t)p - (uintptr_t)e0 * stride_bytes) : nullptr;
}

constexpr size_t kNoAllocScratchBytes = BEAM_MOE_NOALLOC_MAX_BYTES;

// Device address of `scratch` on the device that runs `st`, looked up once
// per device with that device current.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

beam_status scratch_address(hipStream_t st, void** out) {
  int dev = -1, cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return BEAM_ERR_HIP;
  if (st) {
    if (hipStreamGetDevice(st, &dev) != hipSuccess) return BEAM_ERR_HIP;
  } else {
    dev = cur;
  }
  if (dev < 0 || dev >= kMaxDevices) return BEAM_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return BEAM_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return BEAM_ERR_HIP;
    if (e != hipSuccess || !p) return BEAM_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return BEAM_OK;
}

// Where the forward's workspace comes from: the caller's argument, or the
// library's static per-device scratch (beam_moe_forward_noalloc).
enum class WsSource { kCaller, kStatic };

// The forward pass; with `res` set the final combine is the fused residual
// step; with an expert range [e0, e1) other than all experts it is one
// expert shard's share (its weights hold experts e0 .. e1 - 1 only).
beam_status forward_impl(const beam_moe_config* cfg, int32_t T, const void* x,
                         const float* router_w, const float* expert_bias, const void* w_gate,
                         const void* w_up, const void* w_down, const void* w_gate_scale,
                         const void* w_up_scale, const void* w_down_scale,
                         const beam_moe_residual* res, void* out, int32_t* topk_idx_out,
                         float* topk_w_out, int32_t* expert_counts_out, float* router_logits_out,
                         void* workspace, size_t workspace_bytes, void* stream, int e0 = 0,
                         int e1 = kExperts, WsSource wsrc = WsSource::kCaller) {
  const beam_status cs = check_config(cfg);
  if (cs != BEAM_OK) return cs;
  if (e0 < 0 || e1 > kExperts || e0 >= e1) return BEAM_ERR_CONFIG;
  const bool shard = e0 > 0 || e1 < kExperts;
  if (shard && res) return BEAM_ERR_CONFIG;
  if (T < 0 || T > kMaxT) return BEAM_ERR_SHAPE;
  if (res) {
    if (!isfinite(res->norm_eps) || res->norm_eps < 0.f || res->step < 2) return BEAM_ERR_CONFIG;
    if (cfg->hidden > kResidualMaxH) return BEAM_ERR_SHAPE;
  }
  if (T == 0) return BEAM_OK;
  if (!x || !router_w || !expert_bias || !w_gate || !w_up || !w_down || !out) return BEAM_ERR_NULL;
  if (res && (!res->stream_in || !res->norm_weight)) return BEAM_ERR_NULL;
  if (res && (misaligned(res->stream_in) || misaligned(res->norm_weight))) return BEAM_ERR_ALIGN;
  const bool fp8 = cfg->w_dtype == BEAM_FP8_E4M3 || cfg->w_dtype == BEAM_MXFP4;
  if (fp8 && (!w_gate_scale || !w_up_scale || !w_down_scale)) return BEAM_ERR_DTYPE;
  if (wsrc == WsSource::kCaller && !workspace) return BEAM_ERR_WORKSPACE;
  if (misaligned(x) || misaligned(router_w) || misaligned(expert_bias) || misaligned(w_gate) ||
      misaligned(w_up) || misaligned(w_down) || misaligned(out) || misaligned(topk_idx_out) ||
      misaligned(topk_w_out) || misaligned(expert_counts_out) || misaligned(router_logits_out) ||
      misaligned(workspace) ||
      (fp8 && (misaligned(w_gate_scale) || misaligned(w_up_scale) || misaligned(w_down_scale))))
    return BEAM_ERR_ALIGN;
  Shape s = shape_of(cfg, T);
  s.n_run = e1 - e0;
  const Layout L = make_layout(s);
  hipStream_t st = (hipStream_t)stream;
  if (wsrc == WsSource::kStatic) {
    // every argument check is done; the size check is host arithmetic too
    if (L.total > kNoAllocScratchBytes) return BEAM_ERR_WORKSPACE;
    const beam_status ss = scratch_address(st, &workspace);
    if (ss != BEAM_OK) return ss;
    workspace_bytes = kNoAllocScratchBytes;
  }
  if (workspace_bytes < L.total) return BEAM_ERR_WORKSPACE;

  uint8_t* ws = (uint8_t*)workspace;
  Buffers B = carve(L, workspace);
  int32_t* idx = topk_idx_out ? topk_idx_out : B.idx;
  float* w = topk_w_out ? topk_w_out : B.w;
  const int k = s.top_k;
  const int BM = forward_list_bm(s);
  if (shard) {
    // weights, and fp8 / MXFP4 scales, of experts e0 .. e1 - 1 only
    const size_t ih = (size_t)s.I * s.H;
    const size_t wb = s.w_mx4 ? ih / 2 : (s.w_fp8 ? ih : ih * 2);
    w_gate = shard_base(w_gate, e0, wb);
    w_up = shard_base(w_up, e0, wb);
    w_down = shard_base(w_down, e0, wb);
    if (fp8) {
      const size_t sg = s.w_mx4 ? ih / 32 : (size_t)s.I * 4, sd = s.w_mx4 ? ih / 32 : (size_t)s.H * 4;
      w_gate_scale = shard_base(w_gate_scale, e0, sg);
      w_up_scale = shard_base(w_up_scale, e0, sg);
      w_down_scale = shard_base(w_down_scale, e0, sd);
    }
  }

  const beam_status rs = route_tokens(s, L, B, x, router_w, expert_bias, router_logits_out, idx, w,
                                      st);
  if (rs != BEAM_OK) return rs;
  if (L.nchunks == 1) {
    STAGE(BEAM_STAGE_PERM_SCAN, launch_perm_single(idx, w, T, k, s.rsf, BM, B.counts, B.offsets,
                                                   B.meta, B.tile_e, B.tile_r, B.e_tstart,
                                                   B.e_ntiles, expert_counts_out, B.stok, B.sw,
                                                   B.inv, st, e0, e1));
  } else {
    STAGE(BEAM_STAGE_PERM_HIST, launch_perm_hist(idx, T, k, B.chist, st));
    STAGE(BEAM_STAGE_PERM_SCAN, launch_perm_scan(B.chist, L.nchunks, BM, B.cbase, B.counts,
                                                 B.offsets, B.meta, B.tile_e, B.tile_r, B.e_tstart,
                                                 B.e_ntiles, expert_counts_out, st, e0, e1));
    STAGE(BEAM_STAGE_PERM_SCATTER, launch_perm_scatter(idx, w, T, k, s.rsf, B.cbase, B.offsets,
                                                       B.stok, B.sw, B.inv, st));
  }

  GemmArgs g{};
  g.tile_e = B.tile_e;
  g.tile_r = B.tile_r;
  g.e_tstart = B.e_tstart;
  g.e_ntiles = B.e_ntiles;
  g.meta = B.meta;
  g.offsets = B.offsets;
  g.stok = B.stok;
  g.sw = B.sw;
  g.max_mtiles = L.max_mtiles;
  void* y = ws + L.y;

  if (fp8) {
    uint8_t* xq = ws + L.xq;
    float* xs = (float*)(ws + L.xs);
    uint32_t* hamax = (uint32_t*)(ws + L.hamax);
    uint16_t* hb = (uint16_t*)(ws + L.h);
    float* hs = (float*)(ws + L.hs);
    uint8_t* hq = ws + L.hq;
    STAGE(BEAM_STAGE_QUANT_X, launch_quant_x(x, s.x_f32, T, s.H, k, xq, xs, hamax, st));
    g.a = xq;
    g.a_scale = xs;
    g.w0 = w_gate;
    g.w1 = w_up;
    g.ws0 = (const float*)w_gate_scale;
    g.ws1 = (const float*)w_up_scale;
    g.out = hb;
    g.hamax = hamax;
    g.K = s.H;
    g.N = s.I;
    STAGE(BEAM_STAGE_GATEUP, launch_gateup(s, g, st));
    STAGE(BEAM_STAGE_QUANT_H, launch_quant_h(hb, hamax, T * k, s.I, hq, hs, st));
    g.a = hq;
    g.a_scale = hs;
    g.w0 = w_down;
    g.w1 = nullptr;
    g.ws0 = (const float*)w_down_scale;
    g.ws1 = nullptr;
    g.out = y;
    g.hamax = nullptr;
    g.K = s.I;
    g.N = s.H;
    STAGE(BEAM_STAGE_DOWN, launch_down(s, g, st));
  } else {
    void* h = ws + L.h;
    g.a = x;
    g.w0 = w_gate;
    g.w1 = w_up;
    g.out = h;
    g.K = s.H;
    g.N = s.I;
    STAGE(BEAM_STAGE_GATEUP, launch_gateup(s, g, st));
    g.a = h;
    g.w0 = w_down;
    g.w1 = nullptr;
    g.out = y;
    g.K = s.I;
    g.N = s.H;
    STAGE(BEAM_STAGE_DOWN, launch_down(s, g, st));
  }
  if (shard) {
    STAGE(BEAM_STAGE_COMBINE, launch_combine_shard(y, B.inv, idx, T, k, s.H, e0, e1, s.x_f32, out,
                                                   st));
  } else if (res) {
    const double kk = res->step;
    const float keep = (float)sqrt((kk - 1.0) / kk), add = (float)(1.0 / sqrt(kk));
    STAGE(BEAM_STAGE_COMBINE, launch_combine_residual(y, B.inv, T, k, s.H, s.x_f32, res->stream_in,
                                                      res->norm_weight, res->norm_eps, keep, add,
                                                      out, st));
  } else {
    STAGE(BEAM_STAGE_COMBINE, launch_combine(y, B.inv, T, k, s.H, s.x_f32, out, st));
  }
  return BEAM_OK;
}

beam_status check_backward(const beam_moe_config* cfg) {
  const beam_status cs = check_config(cfg);
  if (cs != BEAM_OK) return cs;
  if (cfg->x_dtype != BEAM_BF16 || cfg->w_dtype != BEAM_BF16) return BEAM_ERR_DTYPE;
  if (cfg->w_layout != BEAM_LAYOUT_PACKED) return BEAM_ERR_CONFIG;
  if (cfg->hidden % 256 != 0 || cfg->intermediate % 256 != 0) return BEAM_ERR_SHAPE;
  return BEAM_OK;
}

beam_status backward_impl(const beam_moe_config* cfg, int32_t T, const void* x,
                          const float* router_w, const float* expert_bias, const void* w_gate,
                          const void* w_up, const void* w_gate_t, const void* w_up_t,
                          const void* w_down_t, const void* dout, const beam_moe_grads* grads,
                          void* workspace, size_t workspace_bytes, void* stream) {
  const beam_status cs = check_backward(cfg);
  if (cs != BEAM_OK) return cs;
  if (T < 0 || T > kMaxT) return BEAM_ERR_SHAPE;
  if (!grads) return BEAM_ERR_NULL;
  const int nw = (grads->d_w_gate != nullptr) + (grads->d_w_up != nullptr) +
                 (grads->d_w_down != nullptr);
  if (nw != 0 && nw != 3) return BEAM_ERR_NULL;
  const bool wg = nw == 3;
  if (T == 0) return BEAM_OK;
  if (!x || !router_w || !expert_bias || !w_gate || !w_up || !w_gate_t || !w_up_t || !w_down_t ||
      !dout || !grads->dx)
    return BEAM_ERR_NULL;
  if (!workspace) return BEAM_ERR_WORKSPACE;
  if (misaligned(x) || misaligned(router_w) || misaligned(expert_bias) || misaligned(w_gate) ||
      misaligned(w_up) || misaligned(w_gate_t) || misaligned(w_up_t) || misaligned(w_down_t) ||
      misaligned(dout) || misaligned(grads->dx) || misaligned(grads->d_router_w) ||
      misaligned(grads->d_w_gate) || misaligned(grads->d_w_up) || misaligned(grads->d_w_down) ||
      misaligned(workspace))
    return BEAM_ERR_ALIGN;
  const Shape s = shape_of(cfg, T);
  const BwdLayout BL = make_backward_layout(s, wg);
  if (workspace_bytes < BL.total) return BEAM_ERR_WORKSPACE;

  hipStream_t st = (hipStream_t)stream;
  uint8_t* ws = (uint8_t*)workspace;
  const Layout& L = BL.f;
  Buffers B = carve(L, workspace);
  const int k = s.top_k, H = s.H, I = s.I;
  const int BM = wide_bm(s);
  float* ssel = (float*)(ws + BL.ssel);
  float* gu = (float*)(ws + BL.gu);
  uint16_t* dgu = (uint16_t*)(ws + BL.d);
  float* part = (float*)(ws + BL.part);
  float* dz = (float*)(ws + BL.dz);
  int32_t* pcol = (int32_t*)(ws + BL.pcol);
  uint16_t* dxr = (uint16_t*)(ws + L.y);
  uint16_t* ht = wg ? (uint16_t*)(ws + BL.ht) : nullptr;
  uint16_t* dgt = wg ? (uint16_t*)(ws + BL.dgt) : nullptr;
  uint16_t* dut = wg ? (uint16_t*)(ws + BL.dut) : nullptr;
  const int cblocks = (int)(BL.pstride / 32);

  const beam_status rs = route_tokens(s, L, B, x, router_w, expert_bias, nullptr, B.idx, B.w, st,
                                      ssel);
  if (rs != BEAM_OK) return rs;
  if (L.nchunks == 1) {
    STAGE(BEAM_STAGE_PERM_SCAN, launch_perm_single(B.idx, B.w, T, k, s.rsf, BM, B.counts,
                                                   B.offsets, B.meta, B.tile_e, B.tile_r,
                                                   B.e_tstart, B.e_ntiles, nullptr, B.stok, B.sw,
                                                   B.inv, st));
  } else {
    STAGE(BEAM_STAGE_PERM_HIST, launch_perm_hist(B.idx, T, k, B.chist, st));
    STAGE(BEAM_STAGE_PERM_SCAN, launch_perm_scan(B.chist, L.nchunks, BM, B.cbase, B.counts,
                                                 B.offsets, B.meta, B.tile_e, B.tile_r,
                                                 B.e_tstart, B.e_ntiles, nullptr, st));
    STAGE(BEAM_STAGE_PERM_SCATTER, launch_perm_scatter(B.idx, B.w, T, k, s.rsf, B.cbase,
                                                       B.offsets, B.stok, B.sw, B.inv, st));
  }
  if (wg) STAGE(BEAM_STAGE_BWD_TRANSPOSE, launch_segment_cols(B.counts, pcol, st));

  GemmArgs g{};
  g.tile_e = B.tile_e;
  g.tile_r = B.tile_r;
  g.e_tstart = B.e_tstart;
  g.e_ntiles = B.e_ntiles;
  g.meta = B.meta;
  g.offsets = B.offsets;
  g.stok = B.stok;
  g.max_mtiles = L.max_mtiles;
  g.pcol = pcol;
  // g | u of every sorted row (and h transposed)
  g.a = x;
  g.w0 = w_gate;
  g.w1 = w_up;
  g.out = gu;
  g.tout0 = ht;
  g.K = H;
  g.N = I;
  STAGE(BEAM_STAGE_BWD_GATEUP, launch_backward_gemm(2, s, BM, g, st));
  // q = W_down^T dout[t]; dg | du (and their transposes); partial sums of h . q
  g.a = dout;
  g.w0 = w_down_t;
  g.w1 = nullptr;
  g.a2 = gu;
  g.sw = B.sw;
  g.out = dgu;
  g.tout0 = dgt;
  g.tout1 = dut;
  g.part = part;
  g.nparts = BL.nparts;
  STAGE(BEAM_STAGE_BWD_DOWN, launch_backward_gemm(3, s, BM, g, st));
  // input-gradient rows: W_gate^T dg + W_up^T du
  g.a = dgu;
  g.w0 = w_gate_t;
  g.w1 = w_up_t;
  g.a2 = nullptr;
  g.sw = nullptr;
  g.out = dxr;
  g.tout0 = g.tout1 = nullptr;
  g.part = nullptr;
  g.K = 2 * I;
  g.N = H;
  STAGE(BEAM_STAGE_BWD_DX, launch_backward_gemm(4, s, BM, g, st));
  STAGE(BEAM_STAGE_BWD_TOKEN, launch_token_grad(dxr, B.inv, B.idx, B.w, ssel, part, BL.nparts,
                                                s.rsf, router_w, T, k, H, dz,
                                                (uint16_t*)grads->dx, st));
  if (grads->d_router_w)
    STAGE(BEAM_STAGE_BWD_ROUTER, launch_router_grad((const uint16_t*)x, H, B.stok, B.offsets, dz,
                                                    grads->d_router_w, st));
  if (wg) {
    uint16_t* xt = (uint16_t*)(ws + BL.xt);
    uint16_t* gyt = (uint16_t*)(ws + BL.gyt);
    STAGE(BEAM_STAGE_BWD_TRANSPOSE, launch_gather_t((const uint16_t*)x, H, false, B.stok, B.sw,
                                                    B.offsets, pcol, xt, cblocks, st));
    STAGE(BEAM_STAGE_BWD_TRANSPOSE, launch_gather_t((const uint16_t*)dout, H, true, B.stok, B.sw,
                                                    B.offsets, pcol, gyt, cblocks, st));
    STAGE(BEAM_STAGE_BWD_TRANSPOSE, launch_zero_pads(ht, dgt, dut, I, B.offsets, pcol, st));
    STAGE(BEAM_STAGE_BWD_WGRAD, launch_wgrad(gyt, ht, H, I, pcol, (uint16_t*)grads->d_w_down, st));
    STAGE(BEAM_STAGE_BWD_WGRAD, launch_wgrad(dgt, xt, I, H, pcol, (uint16_t*)grads->d_w_gate, st));
    STAGE(BEAM_STAGE_BWD_WGRAD, launch_wgrad(dut, xt, I, H, pcol, (uint16_t*)grads->d_w_up, st));
  }
  return BEAM_OK;
}

}  // namespace

extern "C" {

size_t beam_moe_backward_workspace_bytes(const beam_moe_config* cfg, int32_t T,
                                         int32_t with_weight_grads) {
  if (check_backward(cfg) != BEAM_OK || T < 0 || T > kMaxT) return 0;
  return make_backward_layout(shape_of(cfg, T), with_weight_grads != 0).total;
}

beam_status beam_moe_backward(const beam_moe_config* cfg, int32_t T, const void* x,
                              const float* router_w, const float* expert_bias, const void* w_gate,
                              const void* w_up, const void* w_gate_t, const void* w_up_t,
                              const void* w_down_t, const void* dout, const beam_moe_grads* grads,
                              void* workspace, size_t workspace_bytes, void* stream) {
  return backward_impl(cfg, T, x, router_w, expert_bias, w_gate, w_up, w_gate_t, w_up_t, w_down_t,
                       dout, grads, workspace, workspace_bytes, stream);
}

beam_status beam_moe_pack_weights_transposed(const void* src, void* dst, int32_t n_experts,
                                             int32_t rows, int32_t cols, int32_t w_dtype,
                                             void* stream) {
  if (!src || !dst) return BEAM_ERR_NULL;
  if (w_dtype != BEAM_BF16) return BEAM_ERR_DTYPE;
  if (n_experts < 1 || n_experts > 65535 || rows < 64 || rows % 64 != 0 || cols < 64 ||
      cols % 64 != 0)
    return BEAM_ERR_SHAPE;
  if ((long long)n_experts * rows * cols * 2 > (1LL << 40)) return BEAM_ERR_SHAPE;
  if (misaligned(src) || misaligned(dst)) return BEAM_ERR_ALIGN;
  return launch_pack_t(src, dst, n_experts, rows, cols, (hipStream_t)stream) == hipSuccess
             ? BEAM_OK
             : BEAM_ERR_HIP;
}

beam_status beam_moe_update_bias(float* expert_bias, const int32_t* expert_counts,
                                 int32_t n_experts, float gamma, void* stream) {
  if (!expert_bias || !expert_counts) return BEAM_ERR_NULL;
  if (n_experts != kExperts || !isfinite(gamma)) return BEAM_ERR_CONFIG;
  if (misaligned(expert_bias) || misaligned(expert_counts)) return BEAM_ERR_ALIGN;
  return launch_bias_step(expert_bias, expert_counts, gamma, (hipStream_t)stream) == hipSuccess
             ? BEAM_OK
             : BEAM_ERR_HIP;
}

beam_status beam_moe_forward(const beam_moe_config* cfg, int32_t T, const void* x,
                             const float* router_w, const float* expert_bias, const void* w_gate,
                             const void* w_up, const void* w_down, const void* w_gate_scale,
                             const void* w_up_scale, const void* w_down_scale, void* out,
                             int32_t* topk_idx_out, float* topk_w_out, int32_t* expert_counts_out,
                             float* router_logits_out, void* workspace, size_t workspace_bytes,
                             void* stream) {
  return forward_impl(cfg, T, x, router_w, expert_bias, w_gate, w_up, w_down, w_gate_scale,
                      w_up_scale, w_down_scale, nullptr, out, topk_idx_out, topk_w_out,
                      expert_counts_out, router_logits_out, workspace, workspace_bytes, stream);
}

beam_status beam_moe_forward_noalloc(const beam_moe_config* cfg, int32_t T, const void* x,
                                     const float* router_w, const float* expert_bias,
                                     const void* w_gate, const void* w_up, const void* w_down,
                                     const void* w_gate_scale, const void* w_up_scale,
                                     const void* w_down_scale, void* out, int32_t* topk_idx_out,
                                     float* topk_w_out, int32_t* expert_counts_out,
                                     float* router_logits_out, void* stream) {
  return forward_impl(cfg, T, x, router_w, expert_bias, w_gate, w_up, w_down, w_gate_scale,
                      w_up_scale, w_down_scale, nullptr, out, topk_idx_out, topk_w_out,
                      expert_counts_out, router_logits_out, nullptr, 0, stream, 0, kExperts,
                      WsSource::kStatic);
}

beam_status beam_moe_forward_shard(const beam_moe_config* cfg, int32_t T, const void* x,
                                  const float* router_w, const float* expert_bias,
                                  int32_t expert_begin, int32_t expert_end, const void* w_gate,
                                  const void* w_up, const void* w_down, const void* w_gate_scale,
                                  const void* w_up_scale, const void* w_down_scale,
                                  void* out_partial, int32_t* topk_idx_out, float* topk_w_out,
                                  int32_t* expert_counts_out, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  return forward_impl(cfg, T, x, router_w, expert_bias, w_gate, w_up, w_down, w_gate_scale,
                      w_up_scale, w_down_scale, nullptr, out_partial, topk_idx_out, topk_w_out,
                      expert_counts_out, nullptr, workspace, workspace_bytes, stream, expert_begin,
                      expert_end);
}

beam_status beam_moe_forward_residual(const beam_moe_config* cfg, int32_t T, const void* x,
                                      const float* router_w, const float* expert_bias,
                                      const void* w_gate, const void* w_up, const void* w_down,
                                      const void* w_gate_scale, const void* w_up_scale,
                                      const void* w_down_scale, const beam_moe_residual* residual,
                                      void* stream_out, int32_t* topk_idx_out, float* topk_w_out,
                                      int32_t* expert_counts_out, float* router_logits_out,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  if (!residual) return BEAM_ERR_NULL;
  return forward_impl(cfg, T, x, router_w, expert_bias, w_gate, w_up, w_down, w_gate_scale,
                      w_up_scale, w_down_scale, residual, stream_out, topk_idx_out, topk_w_out,
                      expert_counts_out, router_logits_out, workspace, workspace_bytes, stream);
}

beam_status beam_moe_pack_weights(const void* src, void* dst, int32_t n_experts, int32_t rows,
                                  int32_t cols, int32_t w_dtype, void* stream) {
  if (!src || !dst) return BEAM_ERR_NULL;
  if (w_dtype != BEAM_BF16 && w_dtype != BEAM_FP8_E4M3 && w_dtype != BEAM_MXFP4 &&
      w_dtype != BEAM_E8M0)
    return BEAM_ERR_DTYPE;
  const bool mx = w_dtype == BEAM_MXFP4 || w_dtype == BEAM_E8M0;
  const int step = mx ? 512 : 128;
  if (n_experts < 1 || rows < 16 || rows % 16 != 0 || cols < step || cols % step != 0)
    return BEAM_ERR_SHAPE;
  const long long bytes = (long long)n_experts * rows * cols * (w_dtype == BEAM_BF16 ? 2 : 1);
  if (bytes > (1LL << 40)) return BEAM_ERR_SHAPE;
  if (misaligned(src) || misaligned(dst)) return BEAM_ERR_ALIGN;
  hipStream_t st = (hipStream_t)stream;
  hipError_t err;
  if (w_dtype == BEAM_E8M0)
    err = launch_pack_mx_scales((const uint8_t*)src, (uint8_t*)dst, n_experts, rows, cols, st);
  else if (w_dtype == BEAM_MXFP4)  // 64 bytes of codes per row per 128-column step
    err = launch_pack_bytes(src, dst, n_experts, rows, cols / 2, 64, st);
  else
    err = launch_pack(src, dst, n_experts, rows, cols, w_dtype == BEAM_FP8_E4M3, st);
  return err == hipSuccess ? BEAM_OK : BEAM_ERR_HIP;
}

beam_status beam_moe_profile_begin(uint32_t stage_mask) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  g_prof.release();
  g_prof.mask = stage_mask;
  g_prof.on = true;
  return BEAM_OK;
}

beam_status beam_moe_profile_end(float* total_ms, int32_t* launches) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  float tot[BEAM_STAGE_COUNT] = {};
  int32_t cnt[BEAM_STAGE_COUNT] = {};
  beam_status st = BEAM_OK;
  for (auto& r : g_prof.recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) {
      st = BEAM_ERR_HIP;
      continue;
    }
    tot[r.stage] += ms;
    cnt[r.stage] += 1;
  }
  g_prof.release();
  g_prof.on = false;
  for (int i = 0; i < BEAM_STAGE_COUNT; ++i) {
    if (total_ms) total_ms[i] = tot[i];
    if (launches) launches[i] = cnt[i];
  }
  return st;
}

}  // extern "C"
