// C ABI of the MoE FFN block: validation, workspace ownership, variant choice
// and the launch sequence on the caller's stream.  Declared in moe_ffn.h.
#include "moe_ffn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <exception>
#include <mutex>
#include <string>
#include <vector>

#include "common.h"

namespace {
// event pairs of one profiled stage
struct StageProfile {
  std::vector<hipEvent_t> start, stop;
  int used = 0;
};
}  // namespace

struct moe_ffn_handle {
  moe_ffn_config cfg;
  int device;
  void* ws_base;
  size_t ws_bytes;
  moe::Workspace ws;
  int variant;
  int max_mtiles;
  int max_mtiles128;
  int last_T;
  // the last forward ran the streaming path: its grouping tables (counts,
  // offsets, perm, pos) were never built and its h / h_d / y rows are not
  // in grouped order; the diagnostic getters rebuild them on request
  bool last_stream;
  // the last forward (a dense FFN on the MFMA path) wrote its dense rows
  // straight to out, not to the workspace
  bool last_direct;
  bool sync_mode;
  uint32_t prof_mask;
  int prof_max;
  int prof_fwd;  // forwards timed so far
  StageProfile prof[MOE_FFN_NUM_STAGES];
};

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(MOE_FFN_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int kMaxTokensLimit = 1 << 20;
constexpr int kMaxDenseDim = 16384;

int validate_config(const moe_ffn_config* c) {
  if (!c) return fail(MOE_FFN_ERR_INVALID_ARG, "config is NULL");
  if (c->max_tokens < 1 || c->max_tokens > kMaxTokensLimit)
    return fail(MOE_FFN_ERR_INVALID_ARG, "max_tokens must be in [1, 2^20]");
  if (c->hidden <= 0 || c->hidden % 256 || c->hidden > 4096)
    return fail(MOE_FFN_ERR_UNSUPPORTED, "hidden must be a multiple of 256 in [256, 4096]");
  if (c->num_experts == 0) {
    // a dense FFN: no router and no experts, the dense branch alone
    if (c->top_k != 0 || c->expert_dim != 0)
      return fail(MOE_FFN_ERR_INVALID_ARG, "top_k and expert_dim must be 0 when num_experts == 0");
    if (c->dense_dim <= 0) return fail(MOE_FFN_ERR_INVALID_ARG, "a config without experts needs dense_dim > 0");
  } else {
    if (c->num_experts < 4 || c->num_experts > 256 || c->num_experts % 4)
      return fail(MOE_FFN_ERR_UNSUPPORTED, "num_experts must be 0 or a multiple of 4 in [4, 256]");
    if (c->top_k < 1 || c->top_k > 16 || c->top_k > c->num_experts)
      return fail(MOE_FFN_ERR_UNSUPPORTED, "top_k must be in [1, min(num_experts, 16)]");
    if (c->expert_dim <= 0 || c->expert_dim % 64 || c->expert_dim > 4096)
      return fail(MOE_FFN_ERR_UNSUPPORTED, "expert_dim must be a multiple of 64 in [64, 4096]");
  }
  if (c->dense_dim < 0 || c->dense_dim % 64 || c->dense_dim > kMaxDenseDim)
    return fail(MOE_FFN_ERR_UNSUPPORTED, "dense_dim must be 0 or a multiple of 64 in [64, 16384]");
  if (c->weight_format != MOE_FFN_W_BF16 && c->weight_format != MOE_FFN_W_NVFP4 &&
      c->weight_format != MOE_FFN_W_FP8)
    return fail(MOE_FFN_ERR_UNSUPPORTED, "unknown weight_format");
  if (c->flags & ~uint32_t(MOE_FFN_ACCUMULATE)) return fail(MOE_FFN_ERR_UNSUPPORTED, "unknown flag bits");
  // the MFMA kernels address activation operands (x [T, H], h [T*k, I],
  // h_d [T, D], bf16) with 32-bit byte offsets below 2^31
  const long long widest = std::max({(long long)c->hidden, (long long)c->top_k * c->expert_dim,
                                     (long long)c->dense_dim});
  if ((long long)c->max_tokens * widest * 2 >= (1LL << 31))
    return fail(MOE_FFN_ERR_UNSUPPORTED, "max_tokens too large: an activation operand would reach 2 GiB");
  return MOE_FFN_OK;
}

// Workspace layout: every buffer 256-byte aligned.
struct Layout {
  size_t off[22];
  size_t total;
  int max_mtiles;
  int max_mtiles128;
};

Layout layout(const moe_ffn_config& c) {
  const size_t T = size_t(c.max_tokens), E = size_t(c.num_experts), k = size_t(c.top_k);
  const size_t H = size_t(c.hidden), I = size_t(c.expert_dim), D = size_t(c.dense_dim);
  const size_t nb = (T + 63) / 64;
  Layout L{};
  L.max_mtiles = int((T * k + moe::kGemmBM - 1) / moe::kGemmBM + E);
  L.max_mtiles128 = int((T * k + moe::kFp4BM - 1) / moe::kFp4BM + E);
  const size_t sizes[22] = {
      size_t(moe::kRouterSlices) * T * E * 4,     // logits (K-slices)
      size_t(moe::kRouteSlices) * 64 * E * 4,     // route_part (K-slices, T <= 64)
      T * k * 4,                                  // topk_idx
      T * k * 4,                                  // topk_w
      E * 4,                                      // counts
      (E + 1) * 4,                                // offsets
      nb * E * 8,                                 // blk_mask
      nb * E * 4,                                 // blk_base
      T * k * 4,                                  // perm
      T * k * 4,                                  // pos
      size_t(L.max_mtiles) * 16,                  // mtiles
      E * 16,                                     // active
      512 * 4,                                    // meta: counters
      T * k * I * 2,                              // h
      T * (D ? D : 1) * 2,                        // h_d
      T * k * H * 2,                              // y
      T * H * 2,                                  // y_d
      (size_t(moe::kStreamKSMax) * moe::kStreamRows * I +  // streaming gate/up partials
       size_t(moe::kDenseKSMax) * moe::kRouteSmallT * (D ? D : 1)) * 2 * 4,
      size_t(moe::dense_down_slices(moe::Shape{0, int(H), int(E), int(k), int(I), int(D)})) *
          moe::kRouteSmallT * H * 4,              // streaming dense down partials
      size_t(moe::kArriveInts) * 4,               // arrival counters (zero between forwards)
      T * H * 2,                                  // xn: pre-normed input (sandwich-norm forwards)
      size_t(L.max_mtiles128) * 16,               // mtiles128
  };
  size_t o = 0;
  for (int i = 0; i < 22; ++i) {
    L.off[i] = o;
    o += (sizes[i] + 255) & ~size_t(255);
  }
  L.total = o;
  return L;
}

moe::Workspace bind(void* base, const Layout& L) {
  char* b = static_cast<char*>(base);
  moe::Workspace w;
  w.logits = reinterpret_cast<float*>(b + L.off[0]);
  w.route_part = reinterpret_cast<float*>(b + L.off[1]);
  w.topk_idx = reinterpret_cast<int32_t*>(b + L.off[2]);
  w.topk_w = reinterpret_cast<float*>(b + L.off[3]);
  w.counts = reinterpret_cast<int32_t*>(b + L.off[4]);
  w.offsets = reinterpret_cast<int32_t*>(b + L.off[5]);
  w.blk_mask = reinterpret_cast<uint64_t*>(b + L.off[6]);
  w.blk_base = reinterpret_cast<int32_t*>(b + L.off[7]);
  w.perm = reinterpret_cast<int32_t*>(b + L.off[8]);
  w.pos = reinterpret_cast<int32_t*>(b + L.off[9]);
  w.mtiles = reinterpret_cast<int32_t*>(b + L.off[10]);
  w.active = reinterpret_cast<int32_t*>(b + L.off[11]);
  w.meta = reinterpret_cast<int32_t*>(b + L.off[12]);
  w.h = reinterpret_cast<moe::bf16_t*>(b + L.off[13]);
  w.h_d = reinterpret_cast<moe::bf16_t*>(b + L.off[14]);
  w.y = reinterpret_cast<moe::bf16_t*>(b + L.off[15]);
  w.y_d = reinterpret_cast<moe::bf16_t*>(b + L.off[16]);
  w.part = reinterpret_cast<float*>(b + L.off[17]);
  w.ydp = reinterpret_cast<float*>(b + L.off[18]);
  w.arrive = reinterpret_cast<int32_t*>(b + L.off[19]);
  w.xn = reinterpret_cast<moe::bf16_t*>(b + L.off[20]);
  w.mtiles128 = reinterpret_cast<int32_t*>(b + L.off[21]);
  return w;
}

// Makes the handle's device current for the scope of a call.
struct DeviceGuard {
  int prev = -1;
  bool ok = true;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != dev) ok = hipSetDevice(dev) == hipSuccess;
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

int check_handle(moe_ffn_handle* h) {
  if (!h) return fail(MOE_FFN_ERR_INVALID_ARG, "handle is NULL");
  return MOE_FFN_OK;
}

int finish(moe_ffn_handle* h, hipStream_t s, const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, what);
  if (h->sync_mode) {
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, what);
  }
  g_err.clear();
  return MOE_FFN_OK;
}

moe::Shape shape_of(const moe_ffn_handle* h, int T) {
  const moe_ffn_config& c = h->cfg;
  return moe::Shape{T, c.hidden, c.num_experts, c.top_k, c.expert_dim, c.dense_dim};
}

// stream weights when every expert sees few rows; MFMA tiles otherwise
constexpr int kStreamMaxTokens = 32;

// Records the stage's start event (when profiled) on construction and its
// stop event on stop().
struct StageTimer {
  moe_ffn_handle* h;
  int stage;
  hipStream_t s;
  bool on;
  StageTimer(moe_ffn_handle* h_, int stage_, hipStream_t s_, bool timing) : h(h_), stage(stage_), s(s_) {
    StageProfile& p = h->prof[stage];
    on = timing && (h->prof_mask & (1u << stage)) && p.used < int(p.start.size());
    if (on) (void)hipEventRecord(p.start[p.used], s);
  }
  void stop() {
    if (!on) return;
    StageProfile& p = h->prof[stage];
    (void)hipEventRecord(p.stop[p.used], s);
    ++p.used;
    on = false;
  }
};

// Sandwich norms of a sub-block forward (null: the plain block)
struct Norms {
  const float* pre;
  const float* post;
  float eps;
};

int run_forward(moe_ffn_handle* h, int T, const void* x, const void* router_w, const float* bias,
                const moe::StreamArgs& args_in, void* out, hipStream_t s, const Norms* nm = nullptr) {
  moe::StreamArgs args = args_in;
  const moe::Shape sh = args.sh;
  const moe::Workspace& ws = h->ws;
  const bool timing = h->prof_mask != 0 && h->prof_fwd < h->prof_max;
  hipError_t e;
  const auto* xres = static_cast<const moe::bf16_t*>(x);  // the block input (the residual)
  const moe::bf16_t* xb = xres;                           // what the router and the experts read
  const auto* wr = static_cast<const moe::bf16_t*>(router_w);
  bool stream = (h->variant == MOE_FFN_VARIANT_STREAM) ||
                (h->variant == MOE_FFN_VARIANT_AUTO && T <= kStreamMaxTokens);
  if (T > moe::kRouteSmallT) stream = false;  // their scratch holds at most 64 tokens' rows
  // NVFP4 weights stream through their own kernels where the shape fits them
  if (args.nvfp4 && !moe::fp4_stream_fits(sh)) stream = false;
  const int mt = int((size_t(T) * sh.k + moe::kGemmBM - 1) / moe::kGemmBM + sh.E);
  const int mt128 = int((size_t(T) * sh.k + moe::kFp4BM - 1) / moe::kFp4BM + sh.E);
  const bool experts = sh.E > 0;  // else a dense FFN: no routing stages
  // the small-T router's launch shape does not cover every (H, E) (wide H
  // with E not a multiple of 8): such shapes route with the large-T kernels
  // and run the MFMA tiles, whose routing it feeds, at any T
  const bool small_route = experts && T <= moe::kRouteSmallT && moe::route_small_fits(sh);
  if (experts && !small_route) stream = false;
  const bool fs4 = stream && args.nvfp4;  // the NVFP4 streaming kernels
  // a dense FFN on the MFMA path writes its output rows from the down GEMM
  const bool direct = !experts && !stream && !nm && !(h->cfg.flags & MOE_FFN_ACCUMULATE);
  {
    // streaming: the router and the dense branch's gate/up share one launch
    StageTimer tm(h, MOE_FFN_STAGE_ROUTE, s, timing);
    if (nm) {
      // the pre-norm (timed with the router): everything below reads xn
      e = moe::launch_rmsnorm(sh, xres, nm->pre, nm->eps, ws.xn, s);
      if (e != hipSuccess) return hip_fail(e, "pre-norm");
      xb = ws.xn;
      args.x = ws.xn;
    }
    e = stream && !fs4 ? moe::launch_route_dense(args, wr, bias, ws, s)
        : !experts                 ? hipSuccess
        : small_route               ? moe::launch_route_small(sh, xb, wr, bias, ws, s)
                                   : moe::launch_route_large(sh, xb, wr, bias, ws, s);
    tm.stop();
    if (e != hipSuccess) return hip_fail(e, "route");
  }
  if (!stream && experts) {
    // the MFMA tiles read the grouped rows and the tile list; the streaming
    // kernels derive their experts' rows from topk_idx themselves
    StageTimer tm(h, MOE_FFN_STAGE_ALIGN, s, timing);
    e = moe::launch_align(sh, ws, s);
    tm.stop();
    if (e != hipSuccess) return hip_fail(e, "align");
  }
  {
    StageTimer tm(h, MOE_FFN_STAGE_GATEUP, s, timing);
    if (args.in_scale) {
      // NVFP4 activations: the gate/up projections read x quantised (the
      // router above read it as it is)
      e = moe::launch_quant_act(static_cast<const moe::bf16_t*>(x), ws.xn, T, sh.H, sh.H, args.in_scale, s);
      if (e != hipSuccess) return hip_fail(e, "activation quantiser");
      args.x = ws.xn;
    }
    e = fs4           ? moe::launch_fs4_gateup(args, ws, s)
        : stream      ? moe::launch_stream_gateup(args, ws, s)
        : args.nvfp4 ? moe::launch_fp4_gateup(args, ws, mt128, s)
                     : moe::launch_gemm_gateup(args, ws, mt, s);
    tm.stop();
    if (e != hipSuccess) return hip_fail(e, "gate/up");
  }
  if (stream && !fs4 && !moe::stream_fused_geglu(sh, args.fp8)) {
    // a GeGLU pass over the summed partials (otherwise the down units form
    // their rows themselves)
    StageTimer tm(h, MOE_FFN_STAGE_GEGLU, s, timing);
    e = moe::launch_stream_geglu(args, ws, s);
    tm.stop();
    if (e != hipSuccess) return hip_fail(e, "geglu");
  }
  {
    StageTimer tm(h, MOE_FFN_STAGE_DOWN, s, timing);
    if (args.in_scale) {
      // NVFP4 activations: the hidden rows (bf16, as stored) quantised in place
      e = moe::launch_quant_act(ws.h, ws.h, (long long)T * sh.k, sh.I, sh.I, args.in_scale + 1, s);
      if (e == hipSuccess && sh.D > 0) e = moe::launch_quant_act(ws.h_d, ws.h_d, T, sh.D, sh.D, args.in_scale + 2, s);
      if (e != hipSuccess) return hip_fail(e, "activation quantiser");
    }
    moe::bf16_t* yd_direct = direct ? static_cast<moe::bf16_t*>(out) : nullptr;
    e = fs4           ? moe::launch_fs4_down(args, ws, s)
        : stream      ? moe::launch_stream_down(args, ws, s)
        : args.nvfp4 ? moe::launch_fp4_down(args, ws, mt128, s, yd_direct)
                     : moe::launch_gemm_down(args, ws, mt, s, yd_direct);
    tm.stop();
    if (e != hipSuccess) return hip_fail(e, "down");
  }
  if (!direct) {
    StageTimer tm(h, MOE_FFN_STAGE_COMBINE, s, timing);
    const int yd_slices = stream && !fs4 && sh.D > 0 ? moe::dense_down_slices(sh) : 0;
    e = nm ? moe::launch_combine_norm(sh, ws, xres, nm->post, nm->eps, static_cast<moe::bf16_t*>(out), yd_slices,
                                      stream, s)
           : moe::launch_combine(sh, ws, static_cast<moe::bf16_t*>(out), (h->cfg.flags & MOE_FFN_ACCUMULATE) != 0,
                                 yd_slices, stream, s);
    tm.stop();
    if (e != hipSuccess) return hip_fail(e, "combine");
  }
  if (timing) ++h->prof_fwd;
  h->last_T = T;
  h->last_stream = stream;
  h->last_direct = direct;
  return finish(h, s, "forward");
}

void profile_release(moe_ffn_handle* h) {
  for (auto& p : h->prof) {
    for (auto ev : p.start) (void)hipEventDestroy(ev);
    for (auto ev : p.stop) (void)hipEventDestroy(ev);
    p.start.clear();
    p.stop.clear();
    p.used = 0;
  }
  h->prof_mask = 0;
  h->prof_max = 0;
  h->prof_fwd = 0;
}

// the router matrix and bias: required (bias optional) with experts, NULL without
int router_checks(const moe_ffn_handle* h, const void* router_w, const float* bias) {
  if (h->cfg.num_experts == 0) {
    if (router_w || bias)
      return fail(MOE_FFN_ERR_INVALID_ARG, "router_w and router_bias must be NULL when num_experts == 0");
    return MOE_FFN_OK;
  }
  if (!router_w) return fail(MOE_FFN_ERR_INVALID_ARG, "router_w must not be NULL");
  if (!aligned16(router_w)) return fail(MOE_FFN_ERR_INVALID_ARG, "router_w must be 16-byte aligned");
  if (bias && (reinterpret_cast<uintptr_t>(bias) & 3u))
    return fail(MOE_FFN_ERR_INVALID_ARG, "router_bias must be 4-byte aligned");
  return MOE_FFN_OK;
}

int common_forward_checks(moe_ffn_handle* h, int T, const void* x, const void* router_w,
                          const float* bias, const void* out, int fmt) {
  if (int r = check_handle(h)) return r;
  if (h->cfg.weight_format != fmt)
    return fail(MOE_FFN_ERR_UNSUPPORTED, "weight format of the handle does not match this entry point");
  if (T < 0 || T > h->cfg.max_tokens) return fail(MOE_FFN_ERR_INVALID_ARG, "T must be in [0, max_tokens]");
  if (!x || !out) return fail(MOE_FFN_ERR_INVALID_ARG, "x and out must not be NULL");
  if (!aligned16(x) || !aligned16(out)) return fail(MOE_FFN_ERR_INVALID_ARG, "x and out must be 16-byte aligned");
  if (int r = router_checks(h, router_w, bias)) return r;
  if (!(h->cfg.flags & MOE_FFN_ACCUMULATE) && x == out)
    return fail(MOE_FFN_ERR_INVALID_ARG, "out may alias x only with MOE_FFN_ACCUMULATE");
  return MOE_FFN_OK;
}

int check_fp4(const moe_ffn_nvfp4_t* m, bool required, const char* name) {
  if (!required) {
    if (m && (m->q || m->scale || m->tensor_scale))
      return fail(MOE_FFN_ERR_INVALID_ARG, std::string(name) + " must be empty: the config has no such matrices");
    return MOE_FFN_OK;
  }
  if (!m || !m->q || !m->scale || !m->tensor_scale)
    return fail(MOE_FFN_ERR_INVALID_ARG, std::string(name) + ": q, scale and tensor_scale must not be NULL");
  if (!aligned16(m->q) || (reinterpret_cast<uintptr_t>(m->scale) & 3u) ||
      (reinterpret_cast<uintptr_t>(m->tensor_scale) & 3u))
    return fail(MOE_FFN_ERR_INVALID_ARG, std::string(name) + ": misaligned pointer");
  return MOE_FFN_OK;
}

int check_fp8(const moe_ffn_fp8_t* m, bool required, const char* name) {
  if (!required) {
    if (m && (m->q || m->tensor_scale))
      return fail(MOE_FFN_ERR_INVALID_ARG, std::string(name) + " must be empty: the config has no such matrices");
    return MOE_FFN_OK;
  }
  if (!m || !m->q || !m->tensor_scale)
    return fail(MOE_FFN_ERR_INVALID_ARG, std::string(name) + ": q and tensor_scale must not be NULL");
  if (!aligned16(m->q) || (reinterpret_cast<uintptr_t>(m->tensor_scale) & 3u))
    return fail(MOE_FFN_ERR_INVALID_ARG, std::string(name) + ": misaligned pointer");
  return MOE_FFN_OK;
}

moe::Fp8Mat to_mat8(const moe_ffn_fp8_t* m) {
  if (!m) return moe::Fp8Mat{nullptr, nullptr};
  return moe::Fp8Mat{m->q, m->tensor_scale};
}

moe::Fp4Mat to_mat(const moe_ffn_nvfp4_t* m) {
  if (!m) return moe::Fp4Mat{nullptr, nullptr, nullptr};
  return moe::Fp4Mat{m->q, m->scale, m->tensor_scale};
}

int bf16_weight_checks(const moe_ffn_handle* h, const void* w_gate, const void* w_up, const void* w_down,
                       const void* d_gate, const void* d_up, const void* d_down) {
  if (h->cfg.num_experts == 0) {
    if (w_gate || w_up || w_down)
      return fail(MOE_FFN_ERR_INVALID_ARG, "expert weights must be NULL when num_experts == 0");
  } else {
    if (!w_gate || !w_up || !w_down) return fail(MOE_FFN_ERR_INVALID_ARG, "expert weights must not be NULL");
    if (!aligned16(w_gate) || !aligned16(w_up) || !aligned16(w_down))
      return fail(MOE_FFN_ERR_INVALID_ARG, "expert weights must be 16-byte aligned");
  }
  if (h->cfg.dense_dim > 0) {
    if (!d_gate || !d_up || !d_down) return fail(MOE_FFN_ERR_INVALID_ARG, "dense weights must not be NULL");
    if (!aligned16(d_gate) || !aligned16(d_up) || !aligned16(d_down))
      return fail(MOE_FFN_ERR_INVALID_ARG, "dense weights must be 16-byte aligned");
  } else if (d_gate || d_up || d_down) {
    return fail(MOE_FFN_ERR_INVALID_ARG, "dense weights must be NULL when dense_dim == 0");
  }
  return MOE_FFN_OK;
}

moe::StreamArgs bf16_args(const moe_ffn_handle* h, int T, const void* x, const void* w_gate, const void* w_up,
                          const void* w_down, const void* d_gate, const void* d_up, const void* d_down) {
  moe::StreamArgs a{};
  a.sh = shape_of(h, T);
  a.x = static_cast<const moe::bf16_t*>(x);
  a.wg = static_cast<const moe::bf16_t*>(w_gate);
  a.wu = static_cast<const moe::bf16_t*>(w_up);
  a.wd = static_cast<const moe::bf16_t*>(w_down);
  a.dg = static_cast<const moe::bf16_t*>(d_gate);
  a.du = static_cast<const moe::bf16_t*>(d_up);
  a.dd = static_cast<const moe::bf16_t*>(d_down);
  a.nvfp4 = false;
  return a;
}

}  // namespace

// ---------------------------------------------------------------------------
// The forward that allocates nothing: its workspace is a file-scope device
// array of fixed size (each GPU the library runs on holds its own copy until
// the process ends).  Host code never uses the array's name as an address:
// the device address is looked up once per device (hipGetSymbolAddress, with
// that device current) and kept; every kernel argument and fill goes through
// that pointer.
// ---------------------------------------------------------------------------

constexpr size_t kScratchBytes = size_t(64) << 20;  // 64 MiB per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device (null until set up)

// Device address of this device's scratch array (looked up on the first call
// on the device; `dev` is current).
int scratch_on(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_FFN_ERR_UNSUPPORTED, "device index beyond the scratch table");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_FFN_OK;
}

// clears n ints (the arrival counters) with plain stores
__global__ void k_zero_i32(int32_t* p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0;
}

}  // namespace

extern "C" {

int moe_ffn_workspace_bytes(const moe_ffn_config* cfg, size_t* bytes) {
  try {
    if (!bytes) return fail(MOE_FFN_ERR_INVALID_ARG, "bytes is NULL");
    if (int r = validate_config(cfg)) return r;
    *bytes = layout(*cfg).total;
    return MOE_FFN_OK;
  } catch (const std::exception& ex) {
    return fail(MOE_FFN_ERR_INVALID_ARG, ex.what());
  } catch (...) {
    return fail(MOE_FFN_ERR_INVALID_ARG, "unknown exception");
  }
}

int moe_ffn_create(const moe_ffn_config* cfg, moe_ffn_handle** out_handle) {
  try {
    if (!out_handle) return fail(MOE_FFN_ERR_INVALID_ARG, "out_handle is NULL");
    *out_handle = nullptr;
    if (int r = validate_config(cfg)) return r;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    Layout L = layout(*cfg);
    void* base = nullptr;
    e = hipMalloc(&base, L.total);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail(MOE_FFN_ERR_OOM, std::string("workspace hipMalloc: ") + hipGetErrorString(e));
    }
    // tickets and tables start at zero; this is the only memset (create is
    // never part of a captured graph)
    e = hipMemset(base, 0, L.total);
    if (e != hipSuccess) {
      (void)hipFree(base);
      return hip_fail(e, "workspace hipMemset");
    }
    auto* h = new moe_ffn_handle{};
    h->cfg = *cfg;
    h->device = dev;
    h->ws_base = base;
    h->ws_bytes = L.total;
    h->ws = bind(base, L);
    h->variant = MOE_FFN_VARIANT_AUTO;
    h->max_mtiles = L.max_mtiles;
    h->max_mtiles128 = L.max_mtiles128;
    h->last_T = 0;
    const char* sm = std::getenv("MOE_FFN_SYNC");
    h->sync_mode = sm && std::strcmp(sm, "1") == 0;
    *out_handle = h;
    g_err.clear();
    return MOE_FFN_OK;
  } catch (const std::bad_alloc&) {
    return fail(MOE_FFN_ERR_OOM, "host allocation failed");
  } catch (const std::exception& ex) {
    return fail(MOE_FFN_ERR_HIP, ex.what());
  } catch (...) {
    return fail(MOE_FFN_ERR_HIP, "unknown exception");
  }
}

int moe_ffn_destroy(moe_ffn_handle* h) {
  try {
    if (!h) return MOE_FFN_OK;
    DeviceGuard g(h->device);
    hipError_t e = hipDeviceSynchronize();
    profile_release(h);
    hipError_t f = hipFree(h->ws_base);
    delete h;
    if (e != hipSuccess) return hip_fail(e, "destroy: device sync");
    if (f != hipSuccess) return hip_fail(f, "destroy: hipFree");
    return MOE_FFN_OK;
  } catch (...) {
    return fail(MOE_FFN_ERR_HIP, "unknown exception");
  }
}

int moe_ffn_set_variant(moe_ffn_handle* h, int32_t variant) {
  if (int r = check_handle(h)) return r;
  if (variant < MOE_FFN_VARIANT_AUTO || variant > MOE_FFN_VARIANT_MFMA)
    return fail(MOE_FFN_ERR_INVALID_ARG, "unknown variant");
  h->variant = variant;
  return MOE_FFN_OK;
}

int moe_ffn_forward(moe_ffn_handle* h, int32_t T, const void* x, const void* router_w,
                    const float* router_bias, const void* w_gate, const void* w_up, const void* w_down,
                    const void* d_gate, const void* d_up, const void* d_down, void* out, void* stream) {
  try {
    if (int r = common_forward_checks(h, T, x, router_w, router_bias, out, MOE_FFN_W_BF16)) return r;
    if (int r = bf16_weight_checks(h, w_gate, w_up, w_down, d_gate, d_up, d_down)) return r;
    if (T == 0) {
      g_err.clear();
      return MOE_FFN_OK;
    }
    DeviceGuard g(h->device);
    if (!g.ok) return fail(MOE_FFN_ERR_HIP, "cannot make the handle's device current");
    const moe::StreamArgs a = bf16_args(h, T, x, w_gate, w_up, w_down, d_gate, d_up, d_down);
    return run_forward(h, T, x, router_w, router_bias, a, out, static_cast<hipStream_t>(stream));
  } catch (const std::exception& ex) {
    return fail(MOE_FFN_ERR_HIP, ex.what());
  } catch (...) {
    return fail(MOE_FFN_ERR_HIP, "unknown exception");
  }
}

int moe_ffn_forward_noalloc(const moe_ffn_config* cfg, int32_t T, const void* x, const void* router_w,
                            const float* router_bias, const void* w_gate, const void* w_up, const void* w_down,
                            const void* d_gate, const void* d_up, const void* d_down, void* out, void* stream) {
  try {
    if (int r = validate_config(cfg)) return r;
    if (cfg->weight_format != MOE_FFN_W_BF16)
      return fail(MOE_FFN_ERR_UNSUPPORTED, "moe_ffn_forward_noalloc takes bf16 weights (weight_format 0)");
    // a handle on the stack: its profiling vectors stay empty (no allocation)
    moe_ffn_handle hs{};
    hs.cfg = *cfg;
    hs.variant = MOE_FFN_VARIANT_AUTO;
    if (int r = common_forward_checks(&hs, T, x, router_w, router_bias, out, MOE_FFN_W_BF16)) return r;
    if (int r = bf16_weight_checks(&hs, w_gate, w_up, w_down, d_gate, d_up, d_down)) return r;
    // the workspace of this call: the handle layout sized for T tokens
    moe_ffn_config ct = *cfg;
    ct.max_tokens = std::max(T, 1);
    const Layout L = layout(ct);
    if (L.total > kScratchBytes)
      return fail(MOE_FFN_ERR_UNSUPPORTED, "moe_ffn_forward_noalloc: this shape and T need " +
                                               std::to_string(L.total) + " bytes of workspace, more than the " +
                                               std::to_string(kScratchBytes) + "-byte static scratch");
    if (T == 0) {
      g_err.clear();
      return MOE_FFN_OK;
    }
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    void* base = nullptr;
    if (int r = scratch_on(dev, &base)) return r;
    hs.cfg = ct;
    hs.device = dev;
    hs.ws_base = base;
    hs.ws_bytes = L.total;
    hs.ws = bind(base, L);
    hs.max_mtiles = L.max_mtiles;
    hs.max_mtiles128 = L.max_mtiles128;
    const char* sm = std::getenv("MOE_FFN_SYNC");
    hs.sync_mode = sm && std::strcmp(sm, "1") == 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // the array keeps the last call's contents: the router hand-off's
    // arrival counters must start at zero (a kernel, not a memset)
    hipLaunchKernelGGL(k_zero_i32, dim3(1), dim3(64), 0, s, hs.ws.arrive, moe::kArriveInts);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "scratch counters");
    const moe::StreamArgs a = bf16_args(&hs, T, x, w_gate, w_up, w_down, d_gate, d_up, d_down);
    return run_forward(&hs, T, x, router_w, router_bias, a, out, s);
  } catch (const std::exception& ex) {
    return fail(MOE_FFN_ERR_HIP, ex.what());
  } catch (...) {
    return fail(MOE_FFN_ERR_HIP, "unknown exception");
  }
}

int moe_ffn_forward_block(moe_ffn_handle* h, int32_t T, const void* x, const float* pre_scale,
                          const float* post_scale, float eps, const void* router_w, const float* router_bias,
                          const void* w_gate, const void* w_up, const void* w_down, const void* d_gate,
                          const void* d_up, const void* d_down, void* out, void* stream) {
  try {
    if (int r = check_handle(h)) return r;
    if (h->cfg.weight_format != MOE_FFN_W_BF16)
      return fail(MOE_FFN_ERR_UNSUPPORTED, "weight format of the handle does not match this entry point");
    if (h->cfg.flags & MOE_FFN_ACCUMULATE)
      return fail(MOE_FFN_ERR_UNSUPPORTED,
                  "the sub-block adds its own residual: use a handle without MOE_FFN_ACCUMULATE");
    if (T < 0 || T > h->cfg.max_tokens) return fail(MOE_FFN_ERR_INVALID_ARG, "T must be in [0, max_tokens]");
    if (!x || !out || !pre_scale || !post_scale)
      return fail(MOE_FFN_ERR_INVALID_ARG, "x, out, pre_scale and post_scale must not be NULL");
    if (!aligned16(x) || !aligned16(out) || !aligned16(pre_scale) || !aligned16(post_scale))
      return fail(MOE_FFN_ERR_INVALID_ARG, "x, out, pre_scale and post_scale must be 16-byte aligned");
    if (int r = router_checks(h, router_w, router_bias)) return r;
    if (!(eps >= 0.f) || !(eps < 1e30f)) return fail(MOE_FFN_ERR_INVALID_ARG, "eps must be finite and >= 0");
    if (int r = bf16_weight_checks(h, w_gate, w_up, w_down, d_gate, d_up, d_down)) return r;
    if (T == 0) {
      g_err.clear();
      return MOE_FFN_OK;
    }
    DeviceGuard g(h->device);
    if (!g.ok) return fail(MOE_FFN_ERR_HIP, "cannot make the handle's device current");
    const moe::StreamArgs a = bf16_args(h, T, x, w_gate, w_up, w_down, d_gate, d_up, d_down);
    const Norms nm{pre_scale, post_scale, eps};
    return run_forward(h, T, x, router_w, router_bias, a, out, static_cast<hipStream_t>(stream), &nm);
  } catch (const std::exception& ex) {
    return fail(MOE_FFN_ERR_HIP, ex.what());
  } catch (...) {
    return fail(MOE_FFN_ERR_HIP, "unknown exception");
  }
}

int moe_ffn_forward_nvfp4(moe_ffn_handle* h, int32_t T, const void* x, const void* router_w,
                          const float* router_bias, const moe_ffn_nvfp4_t* w_gate, const moe_ffn_nvfp4_t* w_up,
                          const moe_ffn_nvfp4_t* w_down, const moe_ffn_nvfp4_t* d_gate,
                          const moe_ffn_nvfp4_t* d_up, const moe_ffn_nvfp4_t* d_down, void* out,
                          void* stream) {
  try {
    if (int r = common_forward_checks(h, T, x, router_w, router_bias, out, MOE_FFN_W_NVFP4)) return r;
    const bool experts = h->cfg.num_experts > 0;
    if (int r = check_fp4(w_gate, experts, "w_gate")) return r;
    if (int r = check_fp4(w_up, experts, "w_up")) return r;
    if (int r = check_fp4(w_down, experts, "w_down")) return r;
    const bool dense = h->cfg.dense_dim > 0;
    if (int r = check_fp4(d_gate, dense, "d_gate")) return r;
    if (int r = check_fp4(d_up, dense, "d_up")) return r;
    if (int r = check_fp4(d_down, dense, "d_down")) return r;
    if (T == 0) {
      g_err.clear();
      return MOE_FFN_OK;
    }
    DeviceGuard g(h->device);
    if (!g.ok) return fail(MOE_FFN_ERR_HIP, "cannot make the handle's device current");
    moe::StreamArgs a{};
    a.sh = shape_of(h, T);
    a.x = static_cast<const moe::bf16_t*>(x);
    a.fg = to_mat(experts ? w_gate : nullptr);
    a.fu = to_mat(experts ? w_up : nullptr);
    a.fd = to_mat(experts ? w_down : nullptr);
    a.fdg = to_mat(dense ? d_gate : nullptr);
    a.fdu = to_mat(dense ? d_up : nullptr);
    a.fdd = to_mat(dense ? d_down : nullptr);
    a.nvfp4 = true;
    return run_forward(h, T, x, router_w, router_bias, a, out, static_cast<hipStream_t>(stream));
  } catch (const std::exception& ex) {
    return fail(MOE_FFN_ERR_HIP, ex.what());
  } catch (...) {
    return fail(MOE_FFN_ERR_HIP, "unknown exception");
  }
}

int moe_ffn_forward_fp8(moe_ffn_handle* h, int32_t T, const void* x, const void* router_w, const float* router_bias,
                        const moe_ffn_fp8_t* w_gate, const moe_ffn_fp8_t* w_up, const moe_ffn_fp8_t* w_down,
                        const moe_ffn_fp8_t* d_gate, const moe_ffn_fp8_t* d_up, const moe_ffn_fp8_t* d_down,
                        void* out, void* stream) {
  try {
    if (int r = common_forward_checks(h, T, x, router_w, router_bias, out, MOE_FFN_W_FP8)) return r;
    const bool experts = h->cfg.num_experts > 0;
    if (int r = check_fp8(w_gate, experts, "w_gate")) return r;
    if (int r = check_fp8(w_up, experts, "w_up")) return r;
    if (int r = check_fp8(w_down, experts, "w_down")) return r;
    const bool dense = h->cfg.dense_dim > 0;
    if (int r = check_fp8(d_gate, dense, "d_gate")) return r;
    if (int r = check_fp8(d_up, dense, "d_up")) return r;
    if (int r = check_fp8(d_down, dense, "d_down")) return r;
    if (T == 0) {
      g_err.clear();
      return MOE_FFN_OK;
    }
    DeviceGuard g(h->device);
    if (!g.ok) return fail(MOE_FFN_ERR_HIP, "cannot make the handle's device current");
    moe::StreamArgs a{};
    a.sh = shape_of(h, T);
    a.x = static_cast<const moe::bf16_t*>(x);
    a.qg = to_mat8(experts ? w_gate : nullptr);
    a.qu = to_mat8(experts ? w_up : nullptr);
    a.qd = to_mat8(experts ? w_down : nullptr);
    a.qdg = to_mat8(dense ? d_gate : nullptr);
    a.qdu = to_mat8(dense ? d_up : nullptr);
    a.qdd = to_mat8(dense ? d_down : nullptr);
    a.fp8 = true;
    return run_forward(h, T, x, router_w, router_bias, a, out, static_cast<hipStream_t>(stream));
  } catch (const std::exception& ex) {
    return fail(MOE_FFN_ERR_HIP, ex.what());
  } catch (...) {
    return fail(MOE_FFN_ERR_HIP, "unknown exception");
  }
}

int moe_ffn_forward_w4a4(moe_ffn_handle* h, int32_t T, const void* x, const void* router_w,
                         const float* router_bias, const moe_ffn_nvfp4_t* w_gate, const moe_ffn_nvfp4_t* w_up,
                         const moe_ffn_nvfp4_t* w_down, const moe_ffn_nvfp4_t* d_gate, const moe_ffn_nvfp4_t* d_up,
                         const moe_ffn_nvfp4_t* d_down, const float* in_scale, void* out, void* stream) {
  try {
    if (int r = common_forward_checks(h, T, x, router_w, router_bias, out, MOE_FFN_W_NVFP4)) return r;
    if (h->cfg.num_experts == 0)
      return fail(MOE_FFN_ERR_UNSUPPORTED, "NVFP4 activations need a config with experts");
    if (int r = check_fp4(w_gate, true, "w_gate")) return r;
    if (int r = check_fp4(w_up, true, "w_up")) return r;
    if (int r = check_fp4(w_down, true, "w_down")) return r;
    const bool dense = h->cfg.dense_dim > 0;
    if (int r = check_fp4(d_gate, dense, "d_gate")) return r;
    if (int r = check_fp4(d_up, dense, "d_up")) return r;
    if (int r = check_fp4(d_down, dense, "d_down")) return r;
    if (!in_scale || (reinterpret_cast<uintptr_t>(in_scale) & 3u))
      return fail(MOE_FFN_ERR_INVALID_ARG, "in_scale must be a non-NULL, 4-byte aligned device pointer");
    if (T == 0) {
      g_err.clear();
      return MOE_FFN_OK;
    }
    DeviceGuard g(h->device);
    if (!g.ok) return fail(MOE_FFN_ERR_HIP, "cannot make the handle's device current");
    moe::StreamArgs a{};
    a.sh = shape_of(h, T);
    a.x = static_cast<const moe::bf16_t*>(x);
    a.fg = to_mat(w_gate);
    a.fu = to_mat(w_up);
    a.fd = to_mat(w_down);
    a.fdg = to_mat(dense ? d_gate : nullptr);
    a.fdu = to_mat(dense ? d_up : nullptr);
    a.fdd = to_mat(dense ? d_down : nullptr);
    a.nvfp4 = true;
    a.in_scale = in_scale;
    return run_forward(h, T, x, router_w, router_bias, a, out, static_cast<hipStream_t>(stream));
  } catch (const std::exception& ex) {
    return fail(MOE_FFN_ERR_HIP, ex.what());
  } catch (...) {
    return fail(MOE_FFN_ERR_HIP, "unknown exception");
  }
}

int moe_ffn_quant_act_nvfp4(int64_t rows, int32_t K, const void* in, void* out, const float* in_scale,
                            void* stream) {
  try {
    if (rows < 0 || K < 0 || K % 16) return fail(MOE_FFN_ERR_INVALID_ARG, "rows >= 0 and K a multiple of 16 required");
    if (rows * (int64_t)K * 2 >= (int64_t(1) << 40)) return fail(MOE_FFN_ERR_UNSUPPORTED, "tensor too large");
    if (rows == 0 || K == 0) {
      g_err.clear();
      return MOE_FFN_OK;
    }
    if (!in || !out || !in_scale) return fail(MOE_FFN_ERR_INVALID_ARG, "in, out and in_scale must not be NULL");
    if (!aligned16(in) || !aligned16(out) || (reinterpret_cast<uintptr_t>(in_scale) & 3u))
      return fail(MOE_FFN_ERR_INVALID_ARG, "in and out must be 16-byte aligned, in_scale 4-byte aligned");
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = moe::launch_quant_act(static_cast<const moe::bf16_t*>(in), static_cast<moe::bf16_t*>(out), rows,
                                         K, K, in_scale, s);
    if (e != hipSuccess) return hip_fail(e, "activation quantiser");
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "activation quantiser");
    g_err.clear();
    return MOE_FFN_OK;
  } catch (...) {
    return fail(MOE_FFN_ERR_HIP, "unknown exception");
  }
}

int moe_ffn_get_routing(moe_ffn_handle* h, int32_t* topk_idx, float* topk_w, int32_t* counts,
                        int32_t* offsets, int32_t* perm, int32_t* pos, void* stream) {
  try {
    if (int r = check_handle(h)) return r;
    if (h->cfg.num_experts == 0) return fail(MOE_FFN_ERR_UNSUPPORTED, "a config without experts has no routing");
    DeviceGuard g(h->device);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (h->last_stream && h->last_T > 0) {
      hipError_t e = moe::launch_align(shape_of(h, h->last_T), h->ws, s);
      if (e != hipSuccess) return hip_fail(e, "align");
    }
    const size_t Tk = size_t(h->last_T) * h->cfg.top_k;
    const size_t E = size_t(h->cfg.num_experts);
    struct C {
      void* dst;
      const void* src;
      size_t n;
    } cps[6] = {{topk_idx, h->ws.topk_idx, Tk * 4}, {topk_w, h->ws.topk_w, Tk * 4},
                {counts, h->ws.counts, E * 4},      {offsets, h->ws.offsets, (E + 1) * 4},
                {perm, h->ws.perm, Tk * 4},         {pos, h->ws.pos, Tk * 4}};
    for (auto& c : cps) {
      if (!c.dst || c.n == 0) continue;
      hipError_t e = hipMemcpyAsync(c.dst, c.src, c.n, hipMemcpyDeviceToDevice, s);
      if (e != hipSuccess) return hip_fail(e, "get_routing copy");
    }
    return finish(h, s, "get_routing");
  } catch (...) {
    return fail(MOE_FFN_ERR_HIP, "unknown exception");
  }
}

int moe_ffn_get_intermediates(moe_ffn_handle* h, void* h_rows, void* y_rows, void* h_dense, void* y_dense,
                              void* stream) {
  try {
    if (int r = check_handle(h)) return r;
    DeviceGuard g(h->device);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t T = size_t(h->last_T), k = size_t(h->cfg.top_k);
    const size_t H = size_t(h->cfg.hidden), I = size_t(h->cfg.expert_dim), D = size_t(h->cfg.dense_dim);
    if (y_dense && h->last_direct)
      return fail(MOE_FFN_ERR_UNSUPPORTED, "the last forward wrote its dense rows straight to out");
    if (h->last_stream && T > 0 && h->cfg.num_experts > 0) {
      // rebuild perm / pos, then write h and y in grouped order
      const moe::Shape sh = shape_of(h, int(T));
      hipError_t e = moe::launch_align(sh, h->ws, s);
      if (e == hipSuccess)
        e = moe::launch_stream_export(sh, h->ws, static_cast<moe::bf16_t*>(h_rows), static_cast<moe::bf16_t*>(y_rows), s);
      if (e != hipSuccess) return hip_fail(e, "get_intermediates export");
      h_rows = nullptr;
      y_rows = nullptr;
    }
    struct C {
      void* dst;
      const void* src;
      size_t n;
    } cps[4] = {{h_rows, h->ws.h, T * k * I * 2},
                {y_rows, h->ws.y, T * k * H * 2},
                {h_dense, h->ws.h_d, T * D * 2},
                {y_dense, h->ws.y_d, T * H * 2}};
    for (auto& c : cps) {
      if (!c.dst || c.n == 0) continue;
      hipError_t e = hipMemcpyAsync(c.dst, c.src, c.n, hipMemcpyDeviceToDevice, s);
      if (e != hipSuccess) return hip_fail(e, "get_intermediates copy");
    }
    return finish(h, s, "get_intermediates");
  } catch (...) {
    return fail(MOE_FFN_ERR_HIP, "unknown exception");
  }
}

int moe_ffn_align_only(moe_ffn_handle* h, int32_t T, const int32_t* topk_idx, void* stream) {
  try {
    if (int r = check_handle(h)) return r;
    if (h->cfg.num_experts == 0) return fail(MOE_FFN_ERR_UNSUPPORTED, "a config without experts has no routing");
    if (T < 0 || T > h->cfg.max_tokens) return fail(MOE_FFN_ERR_INVALID_ARG, "T must be in [0, max_tokens]");
    if (!topk_idx) return fail(MOE_FFN_ERR_INVALID_ARG, "topk_idx must not be NULL");
    if (reinterpret_cast<uintptr_t>(topk_idx) & 3u)
      return fail(MOE_FFN_ERR_INVALID_ARG, "topk_idx must be 4-byte aligned");
    if (T == 0) {
      h->last_T = 0;
      h->last_stream = false;
      h->last_direct = false;
      g_err.clear();
      return MOE_FFN_OK;
    }
    DeviceGuard g(h->device);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(h->ws.topk_idx, topk_idx, size_t(T) * h->cfg.top_k * 4,
                                  hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return hip_fail(e, "align_only copy");
    e = moe::launch_align(shape_of(h, T), h->ws, s);
    if (e != hipSuccess) return hip_fail(e, "align");
    h->last_T = T;
    h->last_stream = false;
    h->last_direct = false;
    return finish(h, s, "align_only");
  } catch (...) {
    return fail(MOE_FFN_ERR_HIP, "unknown exception");
  }
}

int moe_ffn_profile_begin(moe_ffn_handle* h, uint32_t stage_mask, int32_t max_samples) {
  try {
    if (int r = check_handle(h)) return r;
    if (max_samples < 1 || max_samples > (1 << 16))
      return fail(MOE_FFN_ERR_INVALID_ARG, "max_samples must be in [1, 65536]");
    if (stage_mask & ~((1u << MOE_FFN_NUM_STAGES) - 1u)) return fail(MOE_FFN_ERR_INVALID_ARG, "bad stage_mask");
    DeviceGuard g(h->device);
    profile_release(h);
    for (int st = 0; st < MOE_FFN_NUM_STAGES; ++st) {
      if (!(stage_mask & (1u << st))) continue;
      StageProfile& p = h->prof[st];
      p.start.resize(max_samples);
      p.stop.resize(max_samples);
      for (int i = 0; i < max_samples; ++i) {
        hipError_t e1 = hipEventCreate(&p.start[i]);
        hipError_t e2 = hipEventCreate(&p.stop[i]);
        if (e1 != hipSuccess || e2 != hipSuccess) {
          p.start.resize(e1 == hipSuccess ? i + 1 : i);
          p.stop.resize(e2 == hipSuccess ? i + 1 : i);
          profile_release(h);
          return hip_fail(e1 != hipSuccess ? e1 : e2, "hipEventCreate");
        }
      }
    }
    h->prof_mask = stage_mask;
    h->prof_max = max_samples;
    h->prof_fwd = 0;
    g_err.clear();
    return MOE_FFN_OK;
  } catch (...) {
    return fail(MOE_FFN_ERR_HIP, "unknown exception");
  }
}

int moe_ffn_profile_end(moe_ffn_handle* h, float* total_ms, int32_t* samples) {
  try {
    if (int r = check_handle(h)) return r;
    DeviceGuard g(h->device);
    int rc = MOE_FFN_OK;
    for (int st = 0; st < MOE_FFN_NUM_STAGES; ++st) {
      StageProfile& p = h->prof[st];
      float sum = 0.f;
      for (int i = 0; i < p.used; ++i) {
        hipError_t e = hipEventSynchronize(p.stop[i]);
        float ms = 0.f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, p.start[i], p.stop[i]);
        if (e != hipSuccess && rc == MOE_FFN_OK) rc = hip_fail(e, "profile events");
        sum += ms;
      }
      if (total_ms) total_ms[st] = sum;
      if (samples) samples[st] = p.used;
    }
    profile_release(h);
    if (rc == MOE_FFN_OK) g_err.clear();
    return rc;
  } catch (...) {
    return fail(MOE_FFN_ERR_HIP, "unknown exception");
  }
}

const char* moe_ffn_last_error(void) { return g_err.c_str(); }

}  // extern "C"
