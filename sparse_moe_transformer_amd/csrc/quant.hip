// NVFP4 activations (W4A4): quantise-dequantise of the activation rows that
// the NVFP4 Linear layers read (the NVFP4 checkpoint config of the 26B-A4B
// model, quantization_config group_0.input_activations: 4-bit float e2m1
// values, groups of 16 along K, float8_e4m3fn group scales computed per call
// ("dynamic": "local"), strategy tensor_group with a static global scale,
// symmetric).
//
// Per group of 16 values v of a row, with the tensor's global scale s:
//   s_g  = e4m3(amax / (6 s))       nearest, ties to even, saturating at 448
//   q    = e2m1(v / (s_g s))        nearest, ties to even, saturating at 6
//   out  = q * s_g                  (s_g = 0: zeros)
// Each of 6 s, amax / (6 s), s_g s and v / (s_g s) is one correctly rounded
// fp32 operation, in that order.  q * s_g is an e2m1 x e4m3 product, exact in
// bf16, so the bf16 MFMA tiles that read it compute with the quantised
// values exactly; the global scale s is applied to the fp32 accumulators.
#include "common.h"

namespace moe {

namespace {

constexpr int kThreads = 256;

// nearest float8_e4m3fn value of r >= 0 (ties to an even mantissa),
// saturating at 448: 3 mantissa bits for normal values, steps of 2^-9 below
// 2^-6
__device__ __forceinline__ float round_e4m3_sat(float r) {
  if (!(r < 448.f)) return 448.f;  // also +inf
  if (r < 0.015625f) return rintf(r * 512.f) * 0.001953125f;
  uint32_t u = __float_as_uint(r);
  u += 0x7FFFFu + ((u >> 20) & 1u);
  u &= 0xFFF00000u;
  return fminf(__uint_as_float(u), 448.f);
}

// nearest e2m1 value (ties to an even mantissa), saturating at +-6: steps of
// 0.5 below 2, 1 below 4, 2 above
__device__ __forceinline__ float round_e2m1_sat(float r) {
  const float a = fabsf(r);
  float v = a < 2.f ? rintf(a * 2.f) * 0.5f : (a < 4.f ? rintf(a) : 2.f * rintf(a * 0.5f));
  return copysignf(fminf(v, 6.f), r);
}

// one thread per 16-value group: rows x (K / 16) groups, in place allowed
__global__ __launch_bounds__(kThreads) void k_quant_act(const bf16_t* __restrict__ in, bf16_t* out, long long groups,
                                                        int gpr, int ld, const float* __restrict__ s_in) {
  const long long g = blockIdx.x * (long long)kThreads + threadIdx.x;
  if (g >= groups) return;
  const long long row = g / gpr;
  const int c = int(g % gpr) * 16;
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(in + row * ld + c);
  const u32x4_t a = src[0], b = src[1];
  float v[16];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    v[2 * d] = bf16_lo(a[d]);
    v[2 * d + 1] = bf16_hi(a[d]);
    v[8 + 2 * d] = bf16_lo(b[d]);
    v[8 + 2 * d + 1] = bf16_hi(b[d]);
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const float s = *s_in;
  const float six = 6.f * s;
  const float sg = round_e4m3_sat(amax / six);
  const float denom = sg * s;
  float q[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) q[i] = denom > 0.f ? round_e2m1_sat(v[i] / denom) * sg : 0.f;
  u32x4_t oa, ob;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    oa[d] = pack_bf16x2(q[2 * d], q[2 * d + 1]);  // exact: e2m1 x e4m3 fits bf16
    ob[d] = pack_bf16x2(q[8 + 2 * d], q[8 + 2 * d + 1]);
  }
  u32x4_t* dst = reinterpret_cast<u32x4_t*>(out + row * ld + c);
  dst[0] = oa;
  dst[1] = ob;
}

}  // namespace

hipError_t launch_quant_act(const bf16_t* in, bf16_t* out, long long rows, int K, int ld, const float* s_in,
                            hipStream_t s) {
  const long long groups = rows * (K / 16);
  if (groups == 0) return hipSuccess;
  hipLaunchKernelGGL(k_quant_act, dim3(unsigned((groups + kThreads - 1) / kThreads)), dim3(kThreads), 0, s, in, out,
                     groups, K / 16, ld, s_in);
  return hipGetLastError();
}

}  // namespace moe
