// Output of the MoE block: the routing-weighted sum of the token's expert
// rows plus the always-on dense branch (gemma-llm API page
// gm.nn.Gemma4_26B_A4B, model description: each layer runs the expert
// mixture and one dense MLP side by side; no weight on the dense term is
// stated, so it is a plain sum).
//
//   out[t] = sum_{j < k} w[t, j] * y[row(t, j)] + y_d[t]     (fp32, j ascending)
//   row(t, j) = pos[t, j] (grouped rows) or t * k + j (slot-ordered rows)
//   (y_d is bf16, or the sum of fp32 K-slices of the dense down projection)
//   with the accumulate flag: out[t] = out_old[t] + (the above)
//
// Each thread handles 8 columns with 16-byte loads, issuing the k expert
// rows' loads together.
//
// Also the sandwich norms of the sub-block: the pre-norm of the block input
// (k_rmsnorm) and the combine with the post-norm and the residual
// (k_combine_norm).
#include "common.h"

namespace moe {

namespace {

constexpr int kThreads = 128;

// One token's 8 columns [c, c + 8) of the block output, fp32, before any
// residual: sum_j w[t, j] * y[row(t, j)] (j ascending) + y_d[t].  The k rows
// of the token (prow, pw) come from LDS.  With dense K-slices the slices are
// summed in order, rounded to bf16 as the bf16 path stores y_d, and y_d is
// written for inspection.
__device__ __forceinline__ void combine8(const Shape& sh, const Workspace& ws, int t, int c, const int* prow,
                                         const float* pw, int yd_slices, float (&acc)[8]) {
  const int H = sh.H, k = sh.k;
  // issue every row's load before summing them in slot order
  u32x4_t v[16];
#pragma unroll
  for (int j = 0; j < 16; ++j)
    if (j < k) v[j] = *reinterpret_cast<const u32x4_t*>(ws.y + (long long)prow[j] * H + c);
  float yd[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) yd[i] = 0.f;
  if (sh.D > 0 && yd_slices == 0) {
    const u32x4_t vd = *reinterpret_cast<const u32x4_t*>(ws.y_d + (long long)t * H + c);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      yd[2 * d] = bf16_lo(vd[d]);
      yd[2 * d + 1] = bf16_hi(vd[d]);
    }
  } else if (sh.D > 0) {
    // the slices in order, four slices' loads in flight at a time
    for (int s0 = 0; s0 < yd_slices; s0 += 4) {
      float4 pa[4], pb[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (s0 + q < yd_slices) {
          const float4* p =
              reinterpret_cast<const float4*>(ws.ydp + ((long long)(s0 + q) * kRouteSmallT + t) * H + c);
          pa[q] = p[0];
          pb[q] = p[1];
        }
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (s0 + q < yd_slices) {
          yd[0] += pa[q].x; yd[1] += pa[q].y; yd[2] += pa[q].z; yd[3] += pa[q].w;
          yd[4] += pb[q].x; yd[5] += pb[q].y; yd[6] += pb[q].z; yd[7] += pb[q].w;
        }
      }
    }
    // the dense branch's output, rounded to bf16, kept for inspection; the
    // sum below uses the same rounded values as the bf16 path
#pragma unroll
    for (int i = 0; i < 8; ++i) yd[i] = __uint_as_float(f32_to_bf16_bits(yd[i]) << 16);
    *reinterpret_cast<u32x4_t*>(ws.y_d + (long long)t * H + c) =
        u32x4_t{pack_bf16x2(yd[0], yd[1]), pack_bf16x2(yd[2], yd[3]), pack_bf16x2(yd[4], yd[5]),
                pack_bf16x2(yd[6], yd[7])};
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j < k) {
      const float w = pw[j];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        acc[2 * d] += w * bf16_lo(v[j][d]);
        acc[2 * d + 1] += w * bf16_hi(v[j][d]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] += yd[i];
}

// the token's k (row, weight) pairs into LDS (threads < k)
__device__ __forceinline__ void token_rows(const Workspace& ws, int t, int k, bool slot_rows, int* prow, float* pw) {
  if (threadIdx.x < k) {
    prow[threadIdx.x] = slot_rows ? t * k + threadIdx.x : ws.pos[(long long)t * k + threadIdx.x];
    pw[threadIdx.x] = ws.topk_w[(long long)t * k + threadIdx.x];
  }
}

// grid (T, ceil(H / (8 * kThreads))): one token per blockIdx.x, 8 columns per thread
__global__ __launch_bounds__(kThreads) void k_combine(Shape sh, Workspace ws, bf16_t* __restrict__ out,
                                                      int accumulate, int yd_slices, int slot_rows) {
  const int t = blockIdx.x;
  const int H = sh.H;
  __shared__ int prow[16];
  __shared__ float pw[16];
  token_rows(ws, t, sh.k, slot_rows != 0, prow, pw);
  __syncthreads();
  const int c = (blockIdx.y * kThreads + threadIdx.x) * 8;
  if (c >= H) return;
  float acc[8];
  combine8(sh, ws, t, c, prow, pw, yd_slices, acc);
  u32x4_t* dst = reinterpret_cast<u32x4_t*>(out + (long long)t * H + c);
  if (accumulate) {
    const u32x4_t o = *dst;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      acc[2 * d] = bf16_lo(o[d]) + acc[2 * d];
      acc[2 * d + 1] = bf16_hi(o[d]) + acc[2 * d + 1];
    }
  }
  u32x4_t r;
#pragma unroll
  for (int d = 0; d < 4; ++d) r[d] = pack_bf16x2(acc[2 * d], acc[2 * d + 1]);
  *dst = r;
}

// ---------------------------------------------------------------------------
// sandwich norms (archdb page "Gemma-4-26B-A4B": RMSNorm, sandwich, eps
// 1e-06): RMSNorm(v) = v / sqrt(mean(v^2) + eps) * gain, per token row.
// One block per token row, 8 columns per thread, so a row's sum of squares
// is a block reduction (fixed order: shuffle tree in each wave, then the
// waves in order).
// ---------------------------------------------------------------------------

constexpr int kNormThreads = 512;  // H <= 4096 columns, 8 per thread

__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  const int wave = threadIdx.x / kWave, nw = (blockDim.x + kWave - 1) / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) red[wave] = v;
  __syncthreads();
  float s = 0.f;
  for (int w = 0; w < nw; ++w) s += red[w];
  return s;
}

// xn[t] = bf16(x[t] * rsqrt(mean(x[t]^2) + eps) * pre), computed in fp32
__global__ __launch_bounds__(kNormThreads) void k_rmsnorm(int H, const bf16_t* __restrict__ x,
                                                          const float* __restrict__ pre, float eps,
                                                          bf16_t* __restrict__ xn) {
  __shared__ float red[kNormThreads / kWave];
  const int t = blockIdx.x, c = threadIdx.x * 8;
  float v[8];
  float ss = 0.f;
  if (c < H) {
    const u32x4_t q = *reinterpret_cast<const u32x4_t*>(x + (long long)t * H + c);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      v[2 * d] = bf16_lo(q[d]);
      v[2 * d + 1] = bf16_hi(q[d]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) ss += v[i] * v[i];
  }
  const float rstd = rsqrtf(block_sum(ss, red) / float(H) + eps);
  if (c < H) {
    const float4 g0 = *reinterpret_cast<const float4*>(pre + c), g1 = *reinterpret_cast<const float4*>(pre + c + 4);
    const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    u32x4_t r;
#pragma unroll
    for (int d = 0; d < 4; ++d)
      r[d] = pack_bf16x2(v[2 * d] * rstd * g[2 * d], v[2 * d + 1] * rstd * g[2 * d + 1]);
    *reinterpret_cast<u32x4_t*>(xn + (long long)t * H + c) = r;
  }
}

// out[t] = resid[t] + f * rsqrt(mean(f^2) + eps) * post, f = the block
// output row (combine8, fp32).  out may be resid: each element is read
// before the same thread writes it.
__global__ __launch_bounds__(kNormThreads) void k_combine_norm(Shape sh, Workspace ws, const bf16_t* resid,
                                                               const float* __restrict__ post, float eps,
                                                               bf16_t* out, int yd_slices, int slot_rows) {
  __shared__ int prow[16];
  __shared__ float pw[16];
  __shared__ float red[kNormThreads / kWave];
  const int t = blockIdx.x, H = sh.H, c = threadIdx.x * 8;
  token_rows(ws, t, sh.k, slot_rows != 0, prow, pw);
  __syncthreads();
  float acc[8];
  float ss = 0.f;
  if (c < H) {
    combine8(sh, ws, t, c, prow, pw, yd_slices, acc);
#pragma unroll
    for (int i = 0; i < 8; ++i) ss += acc[i] * acc[i];
  }
  const float rstd = rsqrtf(block_sum(ss, red) / float(H) + eps);
  if (c < H) {
    const float4 g0 = *reinterpret_cast<const float4*>(post + c), g1 = *reinterpret_cast<const float4*>(post + c + 4);
    const float g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    const u32x4_t rr = *reinterpret_cast<const u32x4_t*>(resid + (long long)t * H + c);
    u32x4_t r;
#pragma unroll
    for (int d = 0; d < 4; ++d)
      r[d] = pack_bf16x2(bf16_lo(rr[d]) + acc[2 * d] * rstd * g[2 * d],
                         bf16_hi(rr[d]) + acc[2 * d + 1] * rstd * g[2 * d + 1]);
    *reinterpret_cast<u32x4_t*>(out + (long long)t * H + c) = r;
  }
}

}  // namespace

hipError_t launch_rmsnorm(const Shape& sh, const bf16_t* x, const float* pre, float eps, bf16_t* xn,
                          hipStream_t s) {
  if (sh.T == 0) return hipSuccess;
  const int nthr = (sh.H / 8 + kWave - 1) / kWave * kWave;
  hipLaunchKernelGGL(k_rmsnorm, dim3(sh.T), dim3(nthr), 0, s, sh.H, x, pre, eps, xn);
  return hipGetLastError();
}

hipError_t launch_combine_norm(const Shape& sh, const Workspace& ws, const bf16_t* resid, const float* post,
                               float eps, bf16_t* out, int yd_slices, bool slot_rows, hipStream_t s) {
  if (sh.T == 0) return hipSuccess;
  const int nthr = (sh.H / 8 + kWave - 1) / kWave * kWave;
  hipLaunchKernelGGL(k_combine_norm, dim3(sh.T), dim3(nthr), 0, s, sh, ws, resid, post, eps, out, yd_slices,
                     slot_rows ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_combine(const Shape& sh, const Workspace& ws, bf16_t* out, bool accumulate, int yd_slices,
                          bool slot_rows, hipStream_t s) {
  const int cols = (sh.H + 8 * kThreads - 1) / (8 * kThreads);
  hipLaunchKernelGGL(k_combine, dim3(sh.T, cols), dim3(kThreads), 0, s, sh, ws, out, accumulate ? 1 : 0, yd_slices,
                     slot_rows ? 1 : 0);
  return hipGetLastError();
}

}  // namespace moe
