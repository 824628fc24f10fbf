// Output of the MoE block: the routing-weighted sum of the token's expert
// rows plus the always-on dense branch (gemma-llm API page
// gm.nn.Gemma4_26B_A4B: every layer has a MoE branch and a dense shared MLP
// branch; the sum carries no extra weight on the dense term).
//
//   out[t] = sum_{j < k} w[t, j] * y[pos[t, j]] + y_d[t]     (fp32, j ascending)
//   with the accumulate flag: out[t] = out_old[t] + (the above)
//
// One block per token; each thread handles 8 columns with 16-byte loads.
#include "common.h"

namespace moe {

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void k_combine(Shape sh, Workspace ws, bf16_t* __restrict__ out,
                                                      int accumulate) {
  const int t = blockIdx.x;
  const int H = sh.H, k = sh.k;
  __shared__ int prow[16];
  __shared__ float pw[16];
  if (threadIdx.x < k) {
    prow[threadIdx.x] = ws.pos[(long long)t * k + threadIdx.x];
    pw[threadIdx.x] = ws.topk_w[(long long)t * k + threadIdx.x];
  }
  __syncthreads();
  for (int c = threadIdx.x * 8; c < H; c += kThreads * 8) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    for (int j = 0; j < k; ++j) {
      u32x4_t v = *reinterpret_cast<const u32x4_t*>(ws.y + (long long)prow[j] * H + c);
      const float w = pw[j];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        acc[2 * d] += w * bf16_lo(v[d]);
        acc[2 * d + 1] += w * bf16_hi(v[d]);
      }
    }
    if (sh.D > 0) {
      u32x4_t v = *reinterpret_cast<const u32x4_t*>(ws.y_d + (long long)t * H + c);
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        acc[2 * d] += bf16_lo(v[d]);
        acc[2 * d + 1] += bf16_hi(v[d]);
      }
    }
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(out + (long long)t * H + c);
    if (accumulate) {
      u32x4_t o = *dst;
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
}

}  // namespace

hipError_t launch_combine(const Shape& sh, const Workspace& ws, bf16_t* out, bool accumulate, hipStream_t s) {
  hipLaunchKernelGGL(k_combine, dim3(sh.T), dim3(kThreads), 0, s, sh, ws, out, accumulate ? 1 : 0);
  return hipGetLastError();
}

}  // namespace moe
