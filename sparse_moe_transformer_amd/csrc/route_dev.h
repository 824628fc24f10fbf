// Router pieces shared by the router kernels and the streaming path's
// fused launch: the per-token top-k of a wave, and the small-T (T <= 64)
// K-sliced router whose last slice block routes its tokens.
//
// Router (archdb page "Gemma-4-26B-A4B": gating function softmax; selected
// expert weights renormalized to sum to 1): z = x . W_r (+ b), the top-k
// logits (equal logits: lower id first), p = softmax(z) over all experts,
// w = p_S / sum(p_S), written in ascending expert id.
#pragma once
#include <algorithm>
#include <type_traits>

#include "common.h"

namespace moe {

constexpr int kRouteThreads = 256;
constexpr int kRouteMaxRows = 16;  // rows of a slice per thread

// Launch shape of the small-T router: nslices0 (a power of two, at most
// kRouteSlices) slices, halved until each is a multiple of 8 rows; enough
// row groups that a thread loads at most kRouteMaxRows rows, the rest of
// the block's threads spread over tb tokens.  ok = false when the shape
// does not fit.
struct RouteSmallCfg {
  int cw, nslices, slice_rows, tb, groups;
  bool ok;
};
inline RouteSmallCfg route_small_shape(const Shape& sh, int nslices0) {
  RouteSmallCfg c{};
  c.cw = sh.E % 8 == 0 ? 8 : 4;
  const int ec = sh.E / c.cw;
  c.nslices = nslices0;
  while (c.nslices > 1 && (sh.H % c.nslices || (sh.H / c.nslices) % 8)) c.nslices /= 2;
  c.slice_rows = sh.H / c.nslices;
  int rg_need = 1;
  while (rg_need * kRouteMaxRows < c.slice_rows) rg_need *= 2;
  c.tb = std::max(1, std::min(sh.T, kRouteThreads / (ec * rg_need)));
  const int rg = kRouteThreads / (ec * c.tb);
  c.groups = (sh.T + c.tb - 1) / c.tb;
  c.ok = rg >= 1 && (c.slice_rows + rg - 1) / rg <= kRouteMaxRows && c.tb * c.slice_rows <= kRouteThreads * kRouteMaxRows &&
         c.tb * sh.E <= 8 * kRouteThreads;  // the routing's keys and ranks fit the slice's LDS
  return c;
}
// kRouteSlicesFirst slices where the shape fits them, else kRouteSlices
// (fewer, longer slices leave fewer partial logits to the last block: at the
// 26B-A4B decode shape the router's launch takes 12.0 us with 16 slices
// against 13.2 us with 32; E = 256 at H = 2816 needs 32)
inline RouteSmallCfg route_small_config(const Shape& sh) {
  const RouteSmallCfg c = route_small_shape(sh, kRouteSlicesFirst);
  return c.ok ? c : route_small_shape(sh, kRouteSlices);
}

namespace {

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// DPP lane moves (gfx9 encodings): swap neighbours, swap pairs, mirror
// inside 8 lanes, mirror inside 16 lanes.
constexpr int kDppXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ void argmax_step(float& v, int& i) {
  const float ov = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
  const int oi = __builtin_amdgcn_mov_dpp(i, CTRL, 0xF, 0xF, false);
  if (better(ov, oi, v, i)) {
    v = ov;
    i = oi;
  }
}

// Wave-wide arg-max, lower index winning ties; the result is wave-uniform.
// Inside each 16-lane row: two quad swaps, then mirrors (after each step
// the lanes of a group agree, so a mirror reaches the other group); the 4
// row winners are then compared through readlane.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
  argmax_step<kDppXor1>(v, i);
  argmax_step<kDppXor2>(v, i);
  argmax_step<kDppHalfMirror>(v, i);
  argmax_step<kDppMirror>(v, i);
  float bv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  int bi = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
  for (int r = 1; r < 4; ++r) {
    const float rv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16 * r));
    const int ri = __builtin_amdgcn_readlane(i, 16 * r);
    if (better(rv, ri, bv, bi)) {
      bv = rv;
      bi = ri;
    }
  }
  v = bv;
  i = bi;
}

// The routing of one token from a wave whose lane l holds the logits zv[j]
// of experts l + 64 j and whether each is selected: p = softmax over all E
// experts (zmax = the largest logit), w = p_S / sum(p_S), written in
// ascending expert id.
__device__ __forceinline__ void wave_emit_route(const float (&zv)[4], const bool (&sel)[4], float zmax, int E,
                                                int32_t* out_idx, float* out_w) {
  const int lane = threadIdx.x & (kWave - 1);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (lane + j * kWave < E) s += __expf(zv[j] - zmax);
  s = wave_sum(s);
  float p[4];
  float ps = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    p[j] = sel[j] ? __expf(zv[j] - zmax) / s : 0.f;
    ps += p[j];
  }
  ps = wave_sum(ps);
  // ascending expert id order: position = selected ids below this one
  int base = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint64_t m = __ballot(sel[j]);
    if (sel[j]) {
      const int pos = base + __popcll(m & ((1ull << lane) - 1ull));
      out_idx[pos] = lane + j * kWave;
      out_w[pos] = p[j] / ps;
    }
    base += __popcll(m);
  }
}

// One wave routes one token whose E logits are in z (LDS or global).  Lane
// l owns experts l, l+64, l+128, l+192.  k rounds of wave arg-max pick the
// experts (equal logits: lower id first); p = softmax over all experts;
// w = p_S / sum(p_S), written in ascending expert id.
__device__ void wave_route_token(const float* z, int E, int k, int32_t* out_idx, float* out_w) {
  const int lane = threadIdx.x & (kWave - 1);
  const int nj = (E + kWave - 1) / kWave;  // wave-uniform
  float zv[4];
  bool sel[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + j * kWave;
    zv[j] = (e < E) ? z[e] : -INFINITY;
    sel[j] = false;
  }
  float zmax = -INFINITY;
  for (int r = 0; r < k; ++r) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + j * kWave;
      if (j < nj && e < E && !sel[j] && better(zv[j], e, bv, bi)) {
        bv = zv[j];
        bi = e;
      }
    }
    wave_argmax(bv, bi);
    if (r == 0) zmax = bv;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (lane + j * kWave == bi) sel[j] = true;
  }
  wave_emit_route(zv, sel, zmax, E, out_idx, out_w);
}

// A total order on (logit, expert) as one unsigned key: a larger logit, or
// an equal logit with a lower id, gives a larger key.  The logit's bits are
// mapped so that unsigned order is float order (-0 counts as +0); the low
// word holds E - 1 - e.  route_key_z inverts the logit part.
__device__ __forceinline__ uint64_t route_key(float z, int e, int E) {
  uint32_t u = __float_as_uint(z);
  if (u == 0x80000000u) u = 0u;
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (uint64_t(u) << 32) | uint32_t(E - 1 - e);
}
__device__ __forceinline__ float route_key_z(uint64_t key) {
  const uint32_t u = uint32_t(key >> 32);
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// Routes nt tokens with the whole block at once (the latency-bound end of
// the small-T router).  keys: LDS [nt][E] route_key values; rank: LDS
// [nt][E] ints; zmx: LDS [nt] floats.  The rank of an expert is the number
// of experts of its token with a larger key, so the selected set is
// rank < k (the same set as k rounds of arg-max with lower ids winning
// ties), found by one thread per (token, expert) in parallel.  One wave per
// token then writes the softmax weights as wave_route_token does.  Ends
// with the block converged; keys/rank/zmx are free afterwards.
__device__ void block_route_group(const uint64_t* keys, int* rank, float* zmx, int nt, int E, int k,
                                  int32_t* out_idx, float* out_w) {
  const int tid = threadIdx.x;
  for (int i = tid; i < nt * E; i += kRouteThreads) {
    const int t = i / E;
    const uint64_t* kt = keys + t * E;
    const uint64_t mine = keys[i];
    int r = 0;
    for (int j = 0; j < E; j += 4) {  // E % 4 == 0
      r += kt[j] > mine;
      r += kt[j + 1] > mine;
      r += kt[j + 2] > mine;
      r += kt[j + 3] > mine;
    }
    rank[i] = r;
    if (r == 0) zmx[t] = route_key_z(mine);
  }
  __syncthreads();
  const int wid = tid / kWave, lane = tid & (kWave - 1);
  for (int t = wid; t < nt; t += kRouteThreads / kWave) {
    float zv[4];
    bool sel[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + j * kWave;
      zv[j] = e < E ? route_key_z(keys[t * E + e]) : -INFINITY;
      sel[j] = e < E && rank[t * E + e] < k;
    }
    wave_emit_route(zv, sel, zmx[t], E, out_idx + size_t(t) * k, out_w + size_t(t) * k);
  }
}

// Small-T router (T <= 64), one block of kRouteThreads threads per (K-slice
// s, token group).  Partial logits of one K-slice for a group of tokens:
//   part[s][t][e] = sum over the slice's rows k of x[t][k] * W_r[k][e].
// Block (slice s, token group of TB tokens); thread = (chunk ec of CW
// experts, token tl, row group rg); row group rg owns the slice's rows
// rg, rg + RG, ..., so one wave's 16-byte loads cover whole rows of W_r
// (several tokens' lanes read the same row: one fetch serves them).  All of
// a thread's rows are loaded at once; the slice's x rows are staged in LDS
// as fp32 while the loads are in flight.  Row groups are summed in a fixed
// order through LDS.
//
// The last slice block of a token group to finish then routes the group's
// tokens (softmax, top-k, renormalised weights), so routing takes a single
// launch.  Hand-off: the partial logits are written with device-scope
// stores (they write through the XCD's L2), each block waits for its stores
// to complete and then bumps the group's arrival counter with one
// device-scope atomic; the block that brings it to the slice count reads
// every slice back with device-scope loads (they bypass non-coherent cached
// copies) and clears the counter for the next forward.  No fence is needed,
// so no block writes back or invalidates an L2.
template <int CW>
__device__ void route_slice(const Shape& sh, int slice_rows, int TB, int nslices, int s, int group,
                            const bf16_t* __restrict__ x, const bf16_t* __restrict__ wr,
                            const float* __restrict__ bias, const Workspace& ws) {
  constexpr int kThreads = kRouteThreads;
  float* part = ws.route_part;
  typedef typename std::conditional<CW == 8, u32x4_t, u32x2_t>::type vec_t;
  const int H = sh.H, E = sh.E, T = sh.T;
  const int EC = E / CW;
  const int RG = kThreads / (EC * TB);
  const int tid = threadIdx.x;
  const int ec = tid % EC, tl = (tid / EC) % TB, rg = tid / (EC * TB);
  const bool live = rg < RG;
  const int t0 = group * TB;
  const int k0 = s * slice_rows;
  const int nrow = live && rg < slice_rows ? (slice_rows - 1 - rg) / RG + 1 : 0;
  __shared__ __attribute__((aligned(16))) float xs[kThreads * kRouteMaxRows];  // [TB][slice_rows]
  __shared__ float red[kThreads * 8];              // [RG][TB][E]
  const bf16_t* pw = wr + size_t(k0 + (live ? rg : 0)) * E + ec * CW;
  vec_t vw[kRouteMaxRows];
#pragma unroll
  for (int i = 0; i < kRouteMaxRows; ++i)
    vw[i] = i < nrow ? *reinterpret_cast<const vec_t*>(pw + size_t(i) * RG * E) : vec_t{};
  const int nch = slice_rows / 8;
  for (int c = tid; c < TB * nch; c += kThreads) {
    const int tt = c / nch, kc = (c % nch) * 8;
    u32x4_t v = {0, 0, 0, 0};
    if (t0 + tt < T) v = *reinterpret_cast<const u32x4_t*>(x + size_t(t0 + tt) * H + k0 + kc);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      xs[tt * slice_rows + kc + 2 * d] = bf16_lo(v[d]);
      xs[tt * slice_rows + kc + 2 * d + 1] = bf16_hi(v[d]);
    }
  }
  __syncthreads();
  float acc[CW];
#pragma unroll
  for (int c = 0; c < CW; ++c) acc[c] = 0.f;
#pragma unroll
  for (int i = 0; i < kRouteMaxRows; ++i) {
    const float xv = xs[tl * slice_rows + min(rg + RG * i, slice_rows - 1)];  // past nrow: zero weights
#pragma unroll
    for (int d = 0; d < CW / 2; ++d) {
      acc[2 * d] += xv * bf16_lo(vw[i][d]);
      acc[2 * d + 1] += xv * bf16_hi(vw[i][d]);
    }
  }
  if (live) {
#pragma unroll
    for (int c = 0; c < CW; ++c) red[(rg * TB + tl) * E + ec * CW + c] = acc[c];
  }
  __syncthreads();
  for (int o = tid; o < TB * E; o += kThreads) {
    const int tt = o / E;
    if (t0 + tt >= T) continue;
    float z = 0.f;
    for (int g = 0; g < RG; ++g) z += red[g * TB * E + o];
    __hip_atomic_store(part + (size_t(s) * kRouteSmallT + t0 + tt) * E + (o % E), z, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }

  // ---- arrival: the last slice block of this token group routes it
  __shared__ int last;
  __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores are complete
  __syncthreads();
  if (tid == 0) {
    int32_t* cnt = ws.arrive + kArriveRoute + group;
    last = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nslices - 1;
    if (last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (!last) return;
  // z = sum of the slices in order (+ b): one thread per (token, expert) of
  // the group, so the whole group's logits come back in one round trip; then
  // the block routes the group.  xs (the keys) and red (the ranks) are free
  // now: TB * E <= 8 * kRouteThreads.
  const int nt = min(TB, T - t0);
  uint64_t* keys = reinterpret_cast<uint64_t*>(xs);
  int* rank = reinterpret_cast<int*>(red);
  __shared__ float zmx[kRouteSmallT];
  for (int i = tid; i < nt * E; i += kThreads) {
    const int e = i % E;
    const float* p = part + size_t(t0) * E + i;  // token t0 + i / E, expert e
    float v[kRouteSlices];
#pragma unroll
    for (int j = 0; j < kRouteSlices; ++j)
      v[j] = j < nslices ? __hip_atomic_load(p + size_t(j) * kRouteSmallT * E, __ATOMIC_RELAXED,
                                                    __HIP_MEMORY_SCOPE_AGENT)
                                : 0.f;
    float z = 0.f;
#pragma unroll
    for (int j = 0; j < kRouteSlices; ++j) z += v[j];
    keys[i] = route_key(bias ? z + bias[e] : z, e, E);
  }
  __syncthreads();
  block_route_group(keys, rank, zmx, nt, E, sh.k, ws.topk_idx + size_t(t0) * sh.k, ws.topk_w + size_t(t0) * sh.k);
}

// The rows of the ai-th expert that has tokens (experts in ascending id),
// derived from topk_idx of the T <= 64 tokens by the block itself, so no
// grouping tables (and no kernel to build them) are needed.  Row r is the
// slot s = t * k + j of its r-th token t (ascending), j being the expert's
// place in the token's list; slot[r] receives s.  Returns the expert id
// (-1 when fewer than ai + 1 experts have tokens) and its row count.  Every
// thread of the block must call it (E <= 256, T <= 64).
struct ExpertRows {
  int e, rows;
};
__device__ ExpertRows expert_rows(const Shape& sh, const int32_t* __restrict__ topk, int ai, int* slot) {
  __shared__ unsigned long long mask[256];  // bit t: token t picked the expert
  __shared__ unsigned long long pres[4];    // bit e: expert e has tokens
  __shared__ int tk[kStreamRows];           // topk_idx, read from global memory once
  const int tid = threadIdx.x, nthreads = blockDim.x, E = sh.E, k = sh.k, n = sh.T * sh.k;
  for (int i = tid; i < E; i += nthreads) mask[i] = 0;
  if (tid < 4) pres[tid] = 0;
  __syncthreads();
  for (int s = tid; s < n; s += nthreads) {
    const int e = topk[s];
    tk[s] = e;
    atomicOr(&mask[e], 1ull << (s / k));
    atomicOr(&pres[e >> 6], 1ull << (e & 63));
  }
  __syncthreads();
  int e = -1, left = ai;  // block-uniform
#pragma unroll
  for (int wd = 0; wd < 4; ++wd) {
    unsigned long long m = pres[wd];
    const int c = __popcll(m);
    if (e < 0 && left < c) {
      for (int i = 0; i < left; ++i) m &= m - 1;
      e = wd * 64 + __builtin_ctzll(m);
    }
    if (e < 0) left -= c;
  }
  e = __builtin_amdgcn_readfirstlane(e);
  if (e < 0) return {-1, 0};
  const unsigned long long m = mask[e];
  if (tid < sh.T && ((m >> tid) & 1ull)) {
    int j = 0;
    for (int jj = 0; jj < k; ++jj)
      if (tk[tid * k + jj] == e) j = jj;
    slot[__popcll(m & ((1ull << tid) - 1ull))] = tid * k + j;
  }
  __syncthreads();
  return {e, __builtin_amdgcn_readfirstlane(int(__popcll(m)))};
}

}  // namespace

}  // namespace moe
