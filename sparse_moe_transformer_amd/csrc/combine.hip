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
#include "common.h"

namespace moe {

namespace {

constexpr int kThreads = 128;

// grid (T, ceil(H / (8 * kThreads))): one token per blockIdx.x, 8 columns per thread
__global__ __launch_bounds__(kThreads) void k_combine(Shape sh, Workspace ws, bf16_t* __restrict__ out,
                                                      int accumulate, int yd_slices, int slot_rows) {
  const int t = blockIdx.x;
  const int H = sh.H, k = sh.k;
  __shared__ int prow[16];
  __shared__ float pw[16];
  if (threadIdx.x < k) {
    prow[threadIdx.x] = slot_rows ? t * k + threadIdx.x : ws.pos[(long long)t * k + threadIdx.x];
    pw[threadIdx.x] = ws.topk_w[(long long)t * k + threadIdx.x];
  }
  __syncthreads();
  const int c = (blockIdx.y * kThreads + threadIdx.x) * 8;
  if (c >= H) return;
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
    // issue every slice's loads, then sum in slice order
    float4 pa[kDenseDownKS], pb[kDenseDownKS];
#pragma unroll
    for (int sl = 0; sl < kDenseDownKS; ++sl) {
      if (sl < yd_slices) {
        const float4* p = reinterpret_cast<const float4*>(ws.ydp + ((long long)sl * kRouteSmallT + t) * H + c);
        pa[sl] = p[0];
        pb[sl] = p[1];
      }
    }
#pragma unroll
    for (int sl = 0; sl < kDenseDownKS; ++sl) {
      if (sl < yd_slices) {
        yd[0] += pa[sl].x; yd[1] += pa[sl].y; yd[2] += pa[sl].z; yd[3] += pa[sl].w;
        yd[4] += pb[sl].x; yd[5] += pb[sl].y; yd[6] += pb[sl].z; yd[7] += pb[sl].w;
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
  u32x4_t* dst = reinterpret_cast<u32x4_t*>(out + (long long)t * H + c);
  u32x4_t o = {0, 0, 0, 0};
  if (accumulate) o = *dst;
  float acc[8];
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
  if (accumulate) {
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

}  // namespace

hipError_t launch_combine(const Shape& sh, const Workspace& ws, bf16_t* out, bool accumulate, int yd_slices,
                          bool slot_rows, hipStream_t s) {
  const int cols = (sh.H + 8 * kThreads - 1) / (8 * kThreads);
  hipLaunchKernelGGL(k_combine, dim3(sh.T, cols), dim3(kThreads), 0, s, sh, ws, out, accumulate ? 1 : 0, yd_slices,
                     slot_rows ? 1 : 0);
  return hipGetLastError();
}

}  // namespace moe
