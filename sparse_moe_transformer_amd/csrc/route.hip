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
//   T <= 64: partial logits of kRouteSlices K-slices (many small blocks,
//     so W_r streams at full bandwidth); the last slice block of a token
//     group sums the slices in fixed order and routes the group
//     (route_dev.h).
//   large T: split-K logits (MFMA tiles when E % 128 == 0, else an FMA
//     kernel), a top-k kernel that sums the K-slices in fixed order.
// Grouping (any T): per-64-token membership masks, a per-expert scan over
// the token blocks, and the scatter (which also rebuilds the expert offsets
// and the tile lists).
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "route_dev.h"

namespace moe {

namespace {

constexpr int kThreads = 256;

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
// small T (<= 64): the K-sliced router of route_dev.h
// ---------------------------------------------------------------------------

template <int CW>
__global__ __launch_bounds__(kThreads) void k_route_part(Shape sh, int slice_rows, int TB, const bf16_t* __restrict__ x,
                                                        const bf16_t* __restrict__ wr, const float* __restrict__ bias,
                                                        Workspace ws) {
  route_slice<CW>(sh, slice_rows, TB, int(gridDim.x), blockIdx.x, blockIdx.y, x, wr, bias, ws);
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
  if (sh.T == 0) return hipSuccess;
  const RouteSmallCfg c = route_small_config(sh);
  if (!c.ok) return hipErrorInvalidValue;
  const dim3 grid(c.nslices, c.groups);
  if (c.cw == 8)
    hipLaunchKernelGGL(k_route_part<8>, grid, dim3(kThreads), 0, s, sh, c.slice_rows, c.tb, x, wr, bias, ws);
  else
    hipLaunchKernelGGL(k_route_part<4>, grid, dim3(kThreads), 0, s, sh, c.slice_rows, c.tb, x, wr, bias, ws);
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
