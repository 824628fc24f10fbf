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
//   small T (<= 64): one launch.  Every block computes partial logits over a
//     K-slice of W_r (the 720 KB router matrix is read once, spread over
//     many CUs); the last block to finish (ticket) sums the slices in fixed
//     order and does top-k, softmax and the whole grouping.
//   large T: logits (MFMA tiles when E % 128 == 0, else an FMA kernel),
//     top-k kernel, then count / scan / scatter kernels.
#include <algorithm>

#include "common.h"

namespace moe {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// Wave-wide arg-max with the lower index winning ties.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    float ov = __shfl_xor(v, off, kWave);
    int oi = __shfl_xor(i, off, kWave);
    if (better(ov, oi, v, i)) {
      v = ov;
      i = oi;
    }
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// One wave routes one token whose E logits are in z (LDS or global).
// Lane l owns experts l, l+64, l+128, l+192.
__device__ void wave_route_token(const float* z, int E, int k, int32_t* out_idx, float* out_w) {
  const int lane = threadIdx.x & (kWave - 1);
  float zv[4];
  bool sel[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int e = lane + j * kWave;
    zv[j] = (e < E) ? z[e] : -INFINITY;
    sel[j] = false;
  }
  float zmax = -INFINITY;
  for (int r = 0; r < k; ++r) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int e = lane + j * kWave;
      if (e < E && !sel[j] && better(zv[j], e, bv, bi)) {
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
  // ascending expert id order: rank = selected ids below this one
  int base = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint64_t m = __ballot(sel[j]);
    if (sel[j]) {
      uint64_t below = m & ((1ull << lane) - 1ull);
      int rank = base + __popcll(below);
      out_idx[rank] = lane + j * kWave;
      out_w[rank] = p[j] / ps;
    }
    base += __popcll(m);
  }
}

// Block-wide exclusive scan of one int per thread (kThreads threads).
__device__ int block_exclusive_scan(int v, int* scratch /* [kThreads/kWave + 1] */, int& total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  int incl = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    int o = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += o;
  }
  if (lane == kWave - 1) scratch[wid] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < kThreads / kWave; ++w) {
      int c = scratch[w];
      scratch[w] = run;
      run += c;
    }
    scratch[kThreads / kWave] = run;
  }
  __syncthreads();
  int excl = scratch[wid] + incl - v;
  total = scratch[kThreads / kWave];
  __syncthreads();
  return excl;
}

// Given counts[e] (in `cnt`, one per thread e < E), write offsets, the MFMA
// tile list and the active-expert list.  Called by one whole block.
__device__ void build_offsets_and_tiles(const int cnt_e, int E, const Workspace& ws, int* scratch) {
  const int e = threadIdx.x;
  const int c = (e < E) ? cnt_e : 0;
  int total;
  int off = block_exclusive_scan(c, scratch, total);
  if (e < E) {
    ws.counts[e] = c;
    ws.offsets[e] = off;
  }
  if (e == 0) ws.offsets[E] = total;
  const int nm = (c + kGemmBM - 1) / kGemmBM;
  int ntile;
  int m0 = block_exclusive_scan(nm, scratch, ntile);
  for (int m = 0; m < nm; ++m) {
    int32_t* t = ws.mtiles + 4 * (m0 + m);
    t[0] = e;
    t[1] = off + m * kGemmBM;
    t[2] = min(kGemmBM, c - m * kGemmBM);
    t[3] = 0;
  }
  int nact;
  int a0 = block_exclusive_scan(c > 0 ? 1 : 0, scratch, nact);
  if (c > 0) {
    int32_t* t = ws.active + 4 * a0;
    t[0] = e;
    t[1] = off;
    t[2] = c;
    t[3] = 0;
  }
  if (e == 0) {
    ws.meta[0] = ntile;
    ws.meta[1] = nact;
  }
}

// ---------------------------------------------------------------------------
// small T: split-K logits; the last block routes and groups
// ---------------------------------------------------------------------------

template <int TT>
__global__ __launch_bounds__(kThreads) void k_route_small(Shape sh, const bf16_t* __restrict__ x,
                                                          const bf16_t* __restrict__ wr,
                                                          const float* __restrict__ bias,
                                                          Workspace ws) {
  const int T = sh.T, H = sh.H, E = sh.E, k = sh.k;
  const int nsplit = gridDim.x;
  const int rows = (H + nsplit - 1) / nsplit;
  const int k0 = blockIdx.x * rows;
  const int k1 = min(H, k0 + rows);

  extern __shared__ float smem[];
  float* xs = smem;  // [TT][rows]
  for (int i = threadIdx.x; i < TT * rows; i += kThreads) {
    int t = i / rows, kk = i % rows;
    xs[i] = (t < T && k0 + kk < k1) ? bf16_to_f32(x[size_t(t) * H + k0 + kk]) : 0.f;
  }
  __syncthreads();

  // thread -> (expert e, token group tg); tokens t = tg, tg + TG, ...
  const int TG = kThreads / E;
  const int e = threadIdx.x % E;
  const int tg = threadIdx.x / E;
  float acc[TT];
#pragma unroll
  for (int i = 0; i < TT; ++i) acc[i] = 0.f;
  if (tg < TG) {
    for (int kk = k0; kk < k1; ++kk) {
      float w = bf16_to_f32(wr[size_t(kk) * E + e]);
      const float* xr = xs + (kk - k0);
#pragma unroll
      for (int i = 0; i < TT; ++i) {
        int t = tg + i * TG;
        if (t < TT) acc[i] += xr[t * rows] * w;
      }
    }
#pragma unroll
    for (int i = 0; i < TT; ++i) {
      int t = tg + i * TG;
      if (t < T) ws.route_part[(size_t(blockIdx.x) * kRouteSmallT + t) * E + e] = acc[i];
    }
  }

  // ticket: the last block to arrive finishes the routing
  __shared__ int is_last;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    int prev = __hip_atomic_fetch_add(ws.meta + 8, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    is_last = (prev == nsplit - 1);
  }
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  if (threadIdx.x == 0) __hip_atomic_store(ws.meta + 8, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // logits in fixed split order
  float* zl = smem;  // [T][E] (reuses the x staging)
  __syncthreads();
  for (int i = threadIdx.x; i < T * E; i += kThreads) {
    int t = i / E, ee = i % E;
    float s = 0.f;
    for (int b = 0; b < nsplit; ++b) s += ws.route_part[(size_t(b) * kRouteSmallT + t) * E + ee];
    if (bias) s += bias[ee];
    zl[i] = s;
  }
  __syncthreads();

  __shared__ int32_t tk[kRouteSmallT * 16];
  __shared__ float tw[kRouteSmallT * 16];
  const int wid = threadIdx.x / kWave;
  for (int t = wid; t < T; t += kThreads / kWave) wave_route_token(zl + t * E, E, k, tk + t * k, tw + t * k);
  __syncthreads();
  for (int i = threadIdx.x; i < T * k; i += kThreads) {
    ws.topk_idx[i] = tk[i];
    ws.topk_w[i] = tw[i];
  }

  // grouping of one 64-token block
  __shared__ uint64_t mask[256];
  __shared__ int offs[256];
  __shared__ int scratch[kThreads / kWave + 1];
  uint64_t m = 0;
  if (threadIdx.x < E) {
    for (int t = 0; t < T; ++t)
      for (int j = 0; j < k; ++j)
        if (tk[t * k + j] == int(threadIdx.x)) m |= (1ull << t);
    mask[threadIdx.x] = m;
  }
  build_offsets_and_tiles(__popcll(m), E, ws, scratch);
  if (threadIdx.x < E) offs[threadIdx.x] = ws.offsets[threadIdx.x];
  __syncthreads();
  for (int i = threadIdx.x; i < T * k; i += kThreads) {
    int t = i / k;
    int ee = tk[i];
    int p = offs[ee] + __popcll(mask[ee] & ((1ull << t) - 1ull));
    ws.perm[p] = t;
    ws.pos[i] = p;
  }
}

// ---------------------------------------------------------------------------
// large T
// ---------------------------------------------------------------------------

// FMA router logits for shapes the MFMA tiles do not cover: one output per thread.
__global__ __launch_bounds__(kThreads) void k_router_logits_fma(Shape sh, const bf16_t* __restrict__ x,
                                                               const bf16_t* __restrict__ wr,
                                                               const float* __restrict__ bias,
                                                               float* __restrict__ logits) {
  const long long o = blockIdx.x * (long long)kThreads + threadIdx.x;
  if (o >= (long long)sh.T * sh.E) return;
  const int e = int(o % sh.E);
  const long long t = o / sh.E;
  const bf16_t* xr = x + t * sh.H;
  float s = 0.f;
  for (int kk = 0; kk < sh.H; ++kk) s += bf16_to_f32(xr[kk]) * bf16_to_f32(wr[(long long)kk * sh.E + e]);
  if (bias) s += bias[e];
  logits[o] = s;
}

__global__ __launch_bounds__(kThreads) void k_add_bias(Shape sh, const float* __restrict__ bias,
                                                      float* __restrict__ logits) {
  size_t n = size_t(sh.T) * sh.E;
  for (size_t i = blockIdx.x * size_t(kThreads) + threadIdx.x; i < n; i += size_t(gridDim.x) * kThreads)
    logits[i] += bias[i % sh.E];
}

// one wave per token
__global__ __launch_bounds__(kThreads) void k_topk(Shape sh, Workspace ws) {
  const int t = blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave;
  if (t >= sh.T) return;
  wave_route_token(ws.logits + size_t(t) * sh.E, sh.E, sh.k, ws.topk_idx + size_t(t) * sh.k,
                   ws.topk_w + size_t(t) * sh.k);
}

// per 64-token block: membership masks and counts
__global__ __launch_bounds__(kThreads) void k_align_count(Shape sh, Workspace ws) {
  const int T = sh.T, E = sh.E, k = sh.k;
  const int b = blockIdx.x;
  __shared__ int32_t tk[64 * 16];
  for (int i = threadIdx.x; i < 64 * k; i += kThreads) {
    int t = b * 64 + i / k;
    tk[i] = (t < T) ? ws.topk_idx[size_t(b) * 64 * k + i] : -1;
  }
  __syncthreads();
  const int e = threadIdx.x;
  if (e < E) {
    uint64_t m = 0;
    for (int t = 0; t < 64; ++t)
      for (int j = 0; j < k; ++j)
        if (tk[t * k + j] == e) m |= (1ull << t);
    ws.blk_mask[size_t(b) * E + e] = m;
    ws.blk_base[size_t(b) * E + e] = __popcll(m);
  }
}

// one block: per-expert totals, offsets, tile lists, per-(block, expert) bases
__global__ __launch_bounds__(kThreads) void k_align_scan(Shape sh, int nblk, Workspace ws) {
  const int E = sh.E;
  const int e = threadIdx.x;
  __shared__ int scratch[kThreads / kWave + 1];
  int run = 0;
  if (e < E) {
    for (int b = 0; b < nblk; ++b) {
      int c = ws.blk_base[size_t(b) * E + e];
      ws.blk_base[size_t(b) * E + e] = run;
      run += c;
    }
  }
  build_offsets_and_tiles(run, E, ws, scratch);
  __syncthreads();
  if (e < E) {
    int off = ws.offsets[e];
    for (int b = 0; b < nblk; ++b) ws.blk_base[size_t(b) * E + e] += off;
  }
}

// one 64-thread block per 64 tokens
__global__ __launch_bounds__(64) void k_align_scatter(Shape sh, Workspace ws) {
  const int T = sh.T, E = sh.E, k = sh.k;
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int t = b * 64 + lane;
  if (t >= T) return;
  const uint64_t below = (1ull << lane) - 1ull;
  for (int j = 0; j < k; ++j) {
    int e = ws.topk_idx[size_t(t) * k + j];
    uint64_t m = ws.blk_mask[size_t(b) * E + e];
    int p = ws.blk_base[size_t(b) * E + e] + __popcll(m & below);
    ws.perm[p] = t;
    ws.pos[size_t(t) * k + j] = p;
  }
}

}  // namespace

hipError_t launch_route_small(const Shape& sh, const bf16_t* x, const bf16_t* wr, const float* bias,
                              const Workspace& ws, hipStream_t s) {
  const int nsplit = std::min(kRouteSplits, sh.H);
  const int rows = (sh.H + nsplit - 1) / nsplit;
  if (sh.T <= 8) {
    size_t lds = std::max(size_t(8) * rows, size_t(sh.T) * sh.E) * sizeof(float);
    hipLaunchKernelGGL(k_route_small<8>, dim3(nsplit), dim3(kThreads), lds, s, sh, x, wr, bias, ws);
  } else {
    size_t lds = std::max(size_t(64) * rows, size_t(sh.T) * sh.E) * sizeof(float);
    hipLaunchKernelGGL(k_route_small<64>, dim3(nsplit), dim3(kThreads), lds, s, sh, x, wr, bias, ws);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_router(const Shape& sh, const bf16_t* x, const bf16_t* wr, float* logits,
                              hipStream_t s);

hipError_t launch_route_large(const Shape& sh, const bf16_t* x, const bf16_t* wr, const float* bias,
                              const Workspace& ws, hipStream_t s) {
  if (sh.E % 128 == 0 && sh.H % 64 == 0) {
    hipError_t err = launch_gemm_router(sh, x, wr, ws.logits, s);
    if (err != hipSuccess) return err;
    if (bias) {
      int blocks = int(std::min<size_t>(1024, (size_t(sh.T) * sh.E + kThreads - 1) / kThreads));
      hipLaunchKernelGGL(k_add_bias, dim3(blocks), dim3(kThreads), 0, s, sh, bias, ws.logits);
    }
  } else {
    const long long n = (long long)sh.T * sh.E;
    hipLaunchKernelGGL(k_router_logits_fma, dim3(unsigned((n + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                       s, sh, x, wr, bias, ws.logits);
  }
  hipLaunchKernelGGL(k_topk, dim3((sh.T + 3) / 4), dim3(kThreads), 0, s, sh, ws);
  return hipGetLastError();
}

hipError_t launch_align(const Shape& sh, const Workspace& ws, hipStream_t s) {
  const int nblk = (sh.T + 63) / 64;
  hipLaunchKernelGGL(k_align_count, dim3(nblk), dim3(kThreads), 0, s, sh, ws);
  hipLaunchKernelGGL(k_align_scan, dim3(1), dim3(kThreads), 0, s, sh, nblk, ws);
  hipLaunchKernelGGL(k_align_scatter, dim3(nblk), dim3(64), 0, s, sh, ws);
  return hipGetLastError();
}

}  // namespace moe
