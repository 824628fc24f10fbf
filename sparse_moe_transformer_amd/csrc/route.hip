// Router of the MoE block and the expert grouping of its (token, slot) pairs.
//
// Router (archdb page "Gemma-4-26B-A4B": gating function softmax; selected
// expert weights renormalized to sum to 1; 8 of 128 routed experts per
// token): z = x . W_r (+ b), select the top-k logits (equal logits: lower id
// first), p = softmax(z) over all experts, w = p_S / sum(p_S).  Each token's
// set is written in ascending expert id with its weights aligned.
//
// Grouping: counts[e], offsets = exclusive scan, perm = token ids grouped by
// ascending expert and ascending token inside an expert, pos[t, j] = row of
// slot (t, j).  The rank of a token inside its expert comes from a 64-bit
// membership mask per (64-token block, expert) and a popcount, so the result
// is a deterministic function of topk_idx (no atomics decide positions).
//
// Two routes:
//   T <= 64: a K-sliced partial-logit kernel (for T <= 8 with 16-byte
//     loads of 8 experts x up to 16 rows per thread, all in flight at once),
//     then one block that sums the slices in fixed order, routes and groups.  (No in-kernel hand-off
//     between blocks: on this multi-XCD part a device-scope release writes
//     back the L2, which costs more than a second launch.)
//   large T: split-K logits (MFMA tiles when E % 128 == 0, else an FMA
//     kernel), a top-k kernel that sums the K-slices in fixed order, then
//     three grouping kernels: per-64-token membership masks, a per-expert
//     scan over the token blocks, and the scatter (which also rebuilds the
//     expert offsets and the tile lists).
#include <algorithm>

#include "common.h"

namespace moe {

namespace {

constexpr int kThreads = 256;

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
  // softmax over all experts, then renormalise the selected weights
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

// Block-wide exclusive scan of one int per thread (BLOCK threads).
template <int BLOCK>
__device__ int block_exclusive_scan(int v, int* scratch /* [BLOCK/kWave + 1] */, int& total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  int incl = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += o;
  }
  if (lane == kWave - 1) scratch[wid] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < BLOCK / kWave; ++w) {
      const int c = scratch[w];
      scratch[w] = run;
      run += c;
    }
    scratch[BLOCK / kWave] = run;
  }
  __syncthreads();
  const int excl = scratch[wid] + incl - v;
  total = scratch[BLOCK / kWave];
  __syncthreads();
  return excl;
}

// Block-wide exclusive scan of three ints per thread in one pass.
template <int BLOCK>
__device__ int3 block_exclusive_scan3(int3 v, int3* scratch /* [BLOCK/kWave + 1] */, int3& total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  int3 incl = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int ox = __shfl_up(incl.x, off, kWave);
    const int oy = __shfl_up(incl.y, off, kWave);
    const int oz = __shfl_up(incl.z, off, kWave);
    if (lane >= off) {
      incl.x += ox;
      incl.y += oy;
      incl.z += oz;
    }
  }
  if (lane == kWave - 1) scratch[wid] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int3 run = make_int3(0, 0, 0);
    for (int w = 0; w < BLOCK / kWave; ++w) {
      const int3 c = scratch[w];
      scratch[w] = run;
      run.x += c.x;
      run.y += c.y;
      run.z += c.z;
    }
    scratch[BLOCK / kWave] = run;
  }
  __syncthreads();
  const int3 base = scratch[wid];
  total = scratch[BLOCK / kWave];
  __syncthreads();
  return make_int3(base.x + incl.x - v.x, base.y + incl.y - v.y, base.z + incl.z - v.z);
}

// Given counts[e] (one per thread e < E), write counts, offsets, the MFMA
// tile list and the active-expert list; returns the thread's offset.  Called
// by one whole block of BLOCK >= E threads.
template <int BLOCK>
__device__ int build_offsets_and_tiles(const int cnt_e, int E, const Workspace& ws, int* /*unused*/) {
  __shared__ int3 scratch3[BLOCK / kWave + 1];
  const int e = threadIdx.x;
  const int c = (e < E) ? cnt_e : 0;
  const int nm = (c + kGemmBM - 1) / kGemmBM;
  int3 total;
  const int3 ex = block_exclusive_scan3<BLOCK>(make_int3(c, nm, c > 0 ? 1 : 0), scratch3, total);
  const int off = ex.x;
  if (e < E) {
    ws.counts[e] = c;
    ws.offsets[e] = off;
  }
  if (e == 0) {
    ws.offsets[E] = total.x;
    ws.meta[0] = total.y;
    ws.meta[1] = total.z;
  }
  for (int m = 0; m < nm; ++m) {
    int32_t* t = ws.mtiles + 4 * (ex.y + m);
    t[0] = e;
    t[1] = off + m * kGemmBM;
    t[2] = min(kGemmBM, c - m * kGemmBM);
    t[3] = 0;
  }
  if (c > 0) {
    int32_t* t = ws.active + 4 * ex.z;
    t[0] = e;
    t[1] = off;
    t[2] = c;
    t[3] = 0;
  }
  return off;
}

// ---------------------------------------------------------------------------
// small T (<= 64)
// ---------------------------------------------------------------------------

// Route T <= 64 tokens from logits zl[T][E] (LDS) and group them (one
// 64-token block); run by one whole block of BLOCK threads (BLOCK >= E).
template <int BLOCK>
__device__ void route_and_group(const Shape& sh, const Workspace& ws, const float* zl) {
  const int T = sh.T, E = sh.E, k = sh.k;
  __shared__ int32_t tk[kRouteSmallT * 16];
  __shared__ float tw[kRouteSmallT * 16];
  __shared__ unsigned long long mask[256];
  __shared__ int offs[256];
  __shared__ int scratch[BLOCK / kWave + 1];
  const int wid = threadIdx.x / kWave;
  for (int t = wid; t < T; t += BLOCK / kWave) wave_route_token(zl + t * E, E, k, tk + t * k, tw + t * k);
  if (threadIdx.x < E) mask[threadIdx.x] = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < T * k; i += BLOCK) {
    ws.topk_idx[i] = tk[i];
    ws.topk_w[i] = tw[i];
    atomicOr(&mask[tk[i]], 1ull << (i / k));
  }
  __syncthreads();
  const uint64_t m = threadIdx.x < E ? mask[threadIdx.x] : 0;
  const int off = build_offsets_and_tiles<BLOCK>(__popcll(m), E, ws, scratch);
  if (threadIdx.x < E) offs[threadIdx.x] = off;
  __syncthreads();
  for (int i = threadIdx.x; i < T * k; i += BLOCK) {
    const int t = i / k;
    const int ee = tk[i];
    const int p = offs[ee] + __popcll(mask[ee] & ((1ull << t) - 1ull));
    ws.perm[p] = t;
    ws.pos[i] = p;
  }
}

// T <= 8 and E / 8 a power of two: partial logits of one K-slice per block.
// Thread = (8-expert chunk ec, row group rg owning a contiguous run of the
// slice's rows); all of its rows' 16-byte pieces of W_r are loaded at once
// (<= 16 rows), 8 tokens x 8 experts accumulators.  The 8 token rows of the
// slice are staged in LDS as fp32.  Row groups fold by shuffles and across
// waves in LDS; the block writes route_part[block][t][e].
__global__ __launch_bounds__(kThreads) void k_route_part8(Shape sh, const bf16_t* __restrict__ x,
                                                         const bf16_t* __restrict__ wr, Workspace ws) {
  const int T = sh.T, H = sh.H, E = sh.E;
  const int rows = H / gridDim.x;  // multiple of 16
  const int k0 = blockIdx.x * rows;
  const int EC = E / 8, RG = kThreads / EC;
  const int ec = threadIdx.x % EC, rg = threadIdx.x / EC;
  const int R = (rows + RG - 1) / RG;
  const int kb = min(rows, rg * R), ke = min(rows, kb + R);
  extern __shared__ float smem[];
  float* xs = smem;  // [8][rows]
  constexpr int MAXR = 16;
  const bf16_t* pw = wr + size_t(k0 + kb) * E + ec * 8;
  float acc[8][8];
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[t][c] = 0.f;
  for (int b = 0; b < R; b += MAXR) {  // same trip count in every thread
    u32x4_t vw[MAXR];
#pragma unroll
    for (int i = 0; i < MAXR; ++i)
      vw[i] = kb + b + i < ke ? *reinterpret_cast<const u32x4_t*>(pw + size_t(b + i) * E) : u32x4_t{0, 0, 0, 0};
    if (b == 0) {  // stage x while the first rows are in flight
      const int nch = rows / 8;
      for (int i = threadIdx.x; i < 8 * nch; i += kThreads) {
        const int t = i / nch, kc = (i % nch) * 8;
        u32x4_t v = {0, 0, 0, 0};
        if (t < T) v = *reinterpret_cast<const u32x4_t*>(x + size_t(t) * H + k0 + kc);
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          xs[t * rows + kc + 2 * d] = bf16_lo(v[d]);
          xs[t * rows + kc + 2 * d + 1] = bf16_hi(v[d]);
        }
      }
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < MAXR; ++i) {
      const int kk = min(kb + b + i, rows - 1);  // past ke: zero weights
      float w[8];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        w[2 * d] = bf16_lo(vw[i][d]);
        w[2 * d + 1] = bf16_hi(vw[i][d]);
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float xv = xs[t * rows + kk];
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[t][c] += xv * w[c];
      }
    }
    if (b + MAXR < R) continue;
    // fold row groups inside each wave (lane bits >= log2(EC); the step
    // test is uniform, so every step unrolls), then across the 4 waves
#pragma unroll
    for (int st = 0; st < 6; ++st) {
      const int off = 1 << st;
      if (off >= EC) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
          for (int c = 0; c < 8; ++c) acc[t][c] += __shfl_xor(acc[t][c], off, kWave);
      }
    }
    __syncthreads();  // red aliases xs
    float* red = smem;  // [4 waves][8][E]
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane < EC) {
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int c = 0; c < 8; ++c) red[(wave * 8 + t) * E + lane * 8 + c] = acc[t][c];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < T * E; i += kThreads) {
      float z = 0.f;
#pragma unroll
      for (int wv = 0; wv < 4; ++wv) z += red[wv * 8 * E + i];
      ws.route_part[size_t(blockIdx.x) * kRouteSmallT * E + i] = z;
    }
  }
}

// 8 < T <= 64 (or other E): partial logits of one K-slice per block.
// Thread = (expert e, token group g); rows' loads issued 16 at a time.
__global__ __launch_bounds__(kThreads) void k_route_part(Shape sh, const bf16_t* __restrict__ x,
                                                        const bf16_t* __restrict__ wr, Workspace ws) {
  constexpr int TT = 64;
  const int T = sh.T, H = sh.H, E = sh.E;
  const int rows = H / gridDim.x;
  const int k0 = blockIdx.x * rows;
  const int TG = kThreads / E;
  const int e = threadIdx.x % E;
  const int g = threadIdx.x / E;
  extern __shared__ float smem[];
  float* xs = smem;  // [TT][rows]
  for (int i = threadIdx.x; i < TT * rows; i += kThreads) {
    const int t = i / rows, kk = i % rows;
    xs[i] = (t < T) ? bf16_to_f32(x[size_t(t) * H + k0 + kk]) : 0.f;
  }
  __syncthreads();
  if (g >= TG) return;
  float acc[TT];
#pragma unroll
  for (int i = 0; i < TT; ++i) acc[i] = 0.f;
  constexpr int B = 16;
  for (int kb = 0; kb < rows; kb += B) {
    float w[B];
#pragma unroll
    for (int j = 0; j < B; ++j) w[j] = kb + j < rows ? bf16_to_f32(wr[size_t(k0 + kb + j) * E + e]) : 0.f;
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const float* xr = xs + min(kb + j, rows - 1);  // past the slice: zero weight
#pragma unroll
      for (int i = 0; i < TT; ++i) {
        const int t = g + i * TG;
        if (t < TT) acc[i] += xr[t * rows] * w[j];
      }
    }
  }
#pragma unroll
  for (int i = 0; i < TT; ++i) {
    const int t = g + i * TG;
    if (t < T) ws.route_part[(size_t(blockIdx.x) * kRouteSmallT + t) * E + e] = acc[i];
  }
}

// one block of 512 threads (one wave per token for T <= 8): sum the K-slices
// in fixed order (+ bias), route, group
constexpr int kFinishThreads = 512;
__global__ __launch_bounds__(kFinishThreads) void k_route_finish(Shape sh, int nparts, const float* __restrict__ bias,
                                                          Workspace ws) {
  const int T = sh.T, E = sh.E;
  extern __shared__ float zl[];  // [T][E]
  const int E4 = E / 4;
  const size_t stride = size_t(kRouteSmallT) * E / 4;  // float4s between parts
  for (int i = threadIdx.x; i < T * E4; i += kFinishThreads) {
    const int t = i / E4, e4 = (i % E4) * 4;
    const float4* p = reinterpret_cast<const float4*>(ws.route_part + size_t(t) * E + e4);
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int b0 = 0; b0 < nparts; b0 += 16) {
      float4 v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] = (b0 + j < nparts) ? p[(b0 + j) * stride] : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        s.x += v[j].x;
        s.y += v[j].y;
        s.z += v[j].z;
        s.w += v[j].w;
      }
    }
    if (bias) {
      s.x += bias[e4];
      s.y += bias[e4 + 1];
      s.z += bias[e4 + 2];
      s.w += bias[e4 + 3];
    }
    zl[t * E + e4] = s.x;
    zl[t * E + e4 + 1] = s.y;
    zl[t * E + e4 + 2] = s.z;
    zl[t * E + e4 + 3] = s.w;
  }
  __syncthreads();
  route_and_group<kFinishThreads>(sh, ws, zl);
}

// ---------------------------------------------------------------------------
// large T
// ---------------------------------------------------------------------------

// FMA router logits for shapes the MFMA tiles do not cover: one output per
// thread, written as the single K-slice.
__global__ __launch_bounds__(kThreads) void k_router_logits_fma(Shape sh, const bf16_t* __restrict__ x,
                                                               const bf16_t* __restrict__ wr,
                                                               float* __restrict__ logits) {
  const long long o = blockIdx.x * (long long)kThreads + threadIdx.x;
  if (o >= (long long)sh.T * sh.E) return;
  const int e = int(o % sh.E);
  const long long t = o / sh.E;
  const bf16_t* xr = x + t * sh.H;
  float s = 0.f;
  for (int kk = 0; kk < sh.H; ++kk) s += bf16_to_f32(xr[kk]) * bf16_to_f32(wr[(long long)kk * sh.E + e]);
  logits[o] = s;
}

// one wave per token: sum the K-slices of its logits in order (+ bias), route
__global__ __launch_bounds__(kThreads) void k_topk(Shape sh, int nslices, const float* __restrict__ bias,
                                                  Workspace ws) {
  const int wid = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * (kThreads / kWave) + wid;
  __shared__ float zs[kThreads / kWave][256];
  if (t >= sh.T) return;
  const int E = sh.E;
  const size_t slice = size_t(sh.T) * E;
  for (int e = lane; e < E; e += kWave) {
    const float* p = ws.logits + size_t(t) * E + e;
    float v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = j < nslices ? p[j * slice] : 0.f;
    float z = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) z += v[j];
    if (bias) z += bias[e];
    zs[wid][e] = z;
  }
  // the wave reads back only its own row: no block barrier needed
  wave_route_token(zs[wid], E, sh.k, ws.topk_idx + size_t(t) * sh.k, ws.topk_w + size_t(t) * sh.k);
}

// per 64-token block: membership masks and counts
__global__ __launch_bounds__(kThreads) void k_align_count(Shape sh, Workspace ws) {
  const int T = sh.T, E = sh.E, k = sh.k;
  const int b = blockIdx.x;
  __shared__ uint64_t mask[256];
  for (int i = threadIdx.x; i < E; i += kThreads) mask[i] = 0;
  __syncthreads();
  // one thread per (token, slot): set the token's bit in its expert's mask
  for (int i = threadIdx.x; i < 64 * k; i += kThreads) {
    const int t = b * 64 + i / k;
    if (t < T) atomicOr(reinterpret_cast<unsigned long long*>(&mask[ws.topk_idx[size_t(t) * k + i % k]]),
                        1ull << (i / k));
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kThreads) {
    ws.blk_mask[size_t(b) * E + e] = mask[e];
    ws.blk_base[size_t(b) * E + e] = __popcll(mask[e]);
  }
}

// one block per expert: exclusive scan of its per-block counts (in place),
// total into counts[e]
__global__ __launch_bounds__(kThreads) void k_align_colscan(Shape sh, int nblk, Workspace ws) {
  const int E = sh.E, e = blockIdx.x;
  __shared__ int scratch[kThreads / kWave + 1];
  int carry = 0;
  for (int b0 = 0; b0 < nblk; b0 += kThreads) {
    const int b = b0 + threadIdx.x;
    const int c = b < nblk ? ws.blk_base[size_t(b) * E + e] : 0;
    int total;
    const int ex = block_exclusive_scan<kThreads>(c, scratch, total);
    if (b < nblk) ws.blk_base[size_t(b) * E + e] = carry + ex;
    carry += total;
  }
  if (threadIdx.x == 0) ws.counts[e] = carry;
}

// one 64-thread block per 64 tokens; block 0 also publishes offsets and the
// tile lists
__global__ __launch_bounds__(kThreads) void k_align_scatter(Shape sh, Workspace ws) {
  const int T = sh.T, E = sh.E, k = sh.k;
  const int b = blockIdx.x;
  __shared__ int offs[257];
  __shared__ int scratch[kThreads / kWave + 1];
  const int c = threadIdx.x < E ? ws.counts[threadIdx.x] : 0;
  int total;
  const int off = block_exclusive_scan<kThreads>(c, scratch, total);
  if (threadIdx.x < E) offs[threadIdx.x] = off;
  __syncthreads();
  if (b == 0) (void)build_offsets_and_tiles<kThreads>(c, E, ws, scratch);
  for (int i = threadIdx.x; i < 64 * k; i += kThreads) {
    const int tl = i / k, j = i % k;
    const int t = b * 64 + tl;
    if (t >= T) continue;
    const int e = ws.topk_idx[size_t(t) * k + j];
    const uint64_t m = ws.blk_mask[size_t(b) * E + e];
    const int p = offs[e] + ws.blk_base[size_t(b) * E + e] + __popcll(m & ((1ull << tl) - 1ull));
    ws.perm[p] = t;
    ws.pos[size_t(t) * k + j] = p;
  }
}

}  // namespace

hipError_t launch_route_small(const Shape& sh, const bf16_t* x, const bf16_t* wr, const float* bias,
                              const Workspace& ws, hipStream_t s) {
  const int nsplit = kRouteSplits;  // H % 256 == 0: every slice has a multiple of 16 rows
  const int rows = sh.H / nsplit;
  const int ec = sh.E / 8;
  if (sh.T <= 8 && sh.E % 8 == 0 && (ec & (ec - 1)) == 0) {
    const size_t lds = std::max(size_t(8) * rows, size_t(4) * 8 * sh.E) * sizeof(float);
    hipLaunchKernelGGL(k_route_part8, dim3(nsplit), dim3(kThreads), lds, s, sh, x, wr, ws);
  } else {
    const size_t lds = size_t(64) * rows * sizeof(float);
    hipLaunchKernelGGL(k_route_part, dim3(nsplit), dim3(kThreads), lds, s, sh, x, wr, ws);
  }
  hipLaunchKernelGGL(k_route_finish, dim3(1), dim3(kFinishThreads), size_t(sh.T) * sh.E * sizeof(float), s, sh,
                     nsplit, bias, ws);
  return hipGetLastError();
}

hipError_t launch_gemm_router(const Shape& sh, const bf16_t* x, const bf16_t* wr, float* logits, int ksplit,
                              hipStream_t s);

hipError_t launch_route_large(const Shape& sh, const bf16_t* x, const bf16_t* wr, const float* bias,
                              const Workspace& ws, hipStream_t s) {
  int nslices = 1;
  if (sh.E % 128 == 0 && sh.H % 64 == 0) {
    // enough K-slices for ~512 tiles, at most kRouterSlices
    const int mt = (sh.T + kGemmBM - 1) / kGemmBM * (sh.E / 128);
    nslices = std::max(1, std::min(kRouterSlices, std::min(512 / std::max(1, mt), sh.H / 64)));
    hipError_t err = launch_gemm_router(sh, x, wr, ws.logits, nslices, s);
    if (err != hipSuccess) return err;
  } else {
    const long long n = (long long)sh.T * sh.E;
    hipLaunchKernelGGL(k_router_logits_fma, dim3(unsigned((n + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                       s, sh, x, wr, ws.logits);
  }
  hipLaunchKernelGGL(k_topk, dim3((sh.T + 3) / 4), dim3(kThreads), 0, s, sh, nslices, bias, ws);
  return hipGetLastError();
}

hipError_t launch_align(const Shape& sh, const Workspace& ws, hipStream_t s) {
  const int nblk = (sh.T + 63) / 64;
  hipLaunchKernelGGL(k_align_count, dim3(nblk), dim3(kThreads), 0, s, sh, ws);
  hipLaunchKernelGGL(k_align_colscan, dim3(sh.E), dim3(kThreads), 0, s, sh, nblk, ws);
  hipLaunchKernelGGL(k_align_scatter, dim3(nblk), dim3(kThreads), 0, s, sh, ws);
  return hipGetLastError();
}

}  // namespace moe
