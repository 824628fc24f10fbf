// Shared device helpers and kernel launch declarations of the MoE FFN block.
// gfx950 (CDNA4) only: 64-wide wavefronts, bf16 MFMA, 160 KB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;  // raw bf16 storage

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;  // MFMA A/B operand
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;  // dot2 operand
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;  // 32x32 MFMA accumulator
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;  // 16-byte load/store
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

constexpr int kWave = 64;

// bf16 <-> fp32 ---------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(bf16_t v) { return __uint_as_float(uint32_t(v) << 16); }

// Round to nearest even with the gfx950 conversion (v_cvt_pk_bf16_f32):
// every finite or infinite fp32 value gives the same bits as integer RNE
// (checked over all 2^32 patterns); a NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return uint32_t(__builtin_bit_cast(uint16_t, (__bf16)f));
}

// GELU, tanh form: 0.5 v (1 + tanh(u)), u = sqrt(2/pi) (v + 0.044715 v^3).
// With 0.5 (1 + tanh(u)) = 1 / (1 + exp(-2u)) it is v / (1 + exp(-2u)),
// evaluated with the hardware 2^x (on -2u*log2(e)) and reciprocal, each
// within about an ulp: 8 instructions instead of the ~24 of exp2f and a
// correctly rounded division, which matters in the MFMA epilogue (one GELU
// per output pair).  Large |u| saturates cleanly: exp -> inf gives -0,
// exp -> 0 gives v.
__device__ __forceinline__ float gelu_tanh(float v) {
  const float k2 = -2.0f * 0.7978845608028654f * 1.4426950408889634f;  // -2 sqrt(2/pi) log2(e)
  const float u = v * (1.0f + 0.044715f * v * v);
  return v * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(k2 * u));
}

// Workspace of one handle (device pointers), laid out once at create.
struct Workspace {
  float* logits;        // [kRouterSlices, Tmax, E] fp32 partial router logits (large-T path)
  float* route_part;    // [kRouteSlices, 64, E] fp32 partial router logits (T <= 64)
  int32_t* topk_idx;    // [Tmax, k]
  float* topk_w;        // [Tmax, k]
  int32_t* counts;      // [E]
  int32_t* offsets;     // [E+1]
  uint64_t* blk_mask;   // [NB, E] bit t%64 set if token t of block picked e
  int32_t* blk_base;    // [NB, E] counts, then first row of (block, expert)
  int32_t* perm;        // [Tmax*k]
  int32_t* pos;         // [Tmax*k]
  int32_t* mtiles;      // [max_mtiles, 4] (expert, row0, rows, 0) for MFMA tiles
  int32_t* mtiles128;   // [max_mtiles128, 4] the same with tiles of at most 128 rows (NVFP4 GEMMs)
  int32_t* active;      // [E, 4] (expert, row0, rows, 0) per expert with rows
  int32_t* meta;        // [512]: 0 = #mtiles, 1 = #active experts, 2 = #mtiles128
  bf16_t* h;            // [Tmax*k, I] perm order (MFMA path) or slot order (streaming path)
  bf16_t* h_d;          // [Tmax, D]
  bf16_t* y;            // [Tmax*k, H] perm order (MFMA path) or slot order (streaming path)
  bf16_t* y_d;          // [Tmax, H]
  float* part;          // [kStreamKSMax][kStreamRows][2][I] (rows = slots) + [kDenseKSMax][64][2][D]
                        // (rows = tokens) gate/up partials of the streaming path
  float* ydp;           // [dense_down_slices][64][H] dense down partials (streaming path)
  bf16_t* xn;           // [Tmax, H] pre-normed block input (sandwich-norm forwards)
  int32_t* arrive;      // [kArriveInts] arrival counters of the last-block hand-offs; every
                        // kernel that counts leaves them at zero (zeroed at create)
};

constexpr int kRouterSlices = 16;  // most K-slices of the large-T router logits
constexpr int kRouteSlices = 32;   // most K-slices of the small-T router logits
constexpr int kRouteSlicesFirst = 16;  // ... tried first
constexpr int kRouteSmallT = 64;   // largest T of the one-block-per-token router and the streaming path
constexpr int kGemmBM = 320;       // MFMA tile rows (tokens): ~256 +- 16 rows per expert at T = 4096 fit one tile
constexpr int kFp4BM = 128;        // row tiles of the NVFP4 weight-streaming GEMMs
constexpr int kFp4SmallT = 32;     // ... up to this T every expert's rows are one 32-row tile
constexpr int kStreamKS = 2;       // K-slices of the streaming routed gate/up units (bf16)
constexpr int kStreamKS8 = 4;      // ... with FP8 weights (units twice as wide, so twice the slices)
constexpr int kStreamKSMax = kStreamKS8 > kStreamKS ? kStreamKS8 : kStreamKS;
constexpr int kDenseKS = 4;        // K-slices of the streaming dense gate/up units (beside experts)
constexpr int kDenseOnlyKS = 4;    // ... of a config without experts
constexpr int kDenseKSMax = kDenseKS > kDenseOnlyKS ? kDenseKS : kDenseOnlyKS;
constexpr int kDenseDownKS = 16;   // most K-slices of the streaming dense down units
constexpr int kStreamRows = kRouteSmallT * 16;  // routed rows of the streaming path (T <= 64, k <= 16)
constexpr int kArriveRoute = 0;                 // [64] token groups of the small-T router
constexpr int kArriveInts = 64;

struct Shape {
  int T, H, E, k, I, D;
};

// K-slices of the streaming dense-branch units: whole 64-row groups, at
// most the constants above (no empty slice)
__host__ __device__ inline int dense_gateup_slices(const Shape& sh) {
  const int ks = sh.E > 0 ? kDenseKS : kDenseOnlyKS;
  return sh.H / 64 < ks ? sh.H / 64 : ks;
}
// Whether the streaming down units form their GeGLU rows from the gate/up
// partials themselves (bf16 weights beside experts) instead of reading rows
// of a GeGLU pass.  Not for FP8 weights (their down units read half the
// bytes, so the 4 K-slices of partials they would re-read cost more than the
// launch) nor for a dense branch alone (every down column unit would re-read
// all K-slices of a wide branch's fp32 partials).
inline bool stream_fused_geglu(const Shape& sh, bool fp8) { return sh.E > 0 && !fp8; }

// The dense down units: K-slices of about 640 rows, at least 4 (so that a
// D = 10240 branch spreads over a few hundred blocks; finer slices do not
// stream faster and cost the combine a longer sum)
__host__ __device__ inline int dense_down_slices(const Shape& sh) {
  int ks = sh.D / 640 > 4 ? sh.D / 640 : 4;
  if (ks > kDenseDownKS) ks = kDenseDownKS;
  return sh.D / 64 < ks ? sh.D / 64 : ks;
}

// NVFP4 matrix stack
struct Fp4Mat {
  const uint8_t* q;
  const uint8_t* scale;
  const float* tscale;
};

// FP8 matrix stack: [G][K][N] float8_e4m3fn codes and [G] fp32 scales
struct Fp8Mat {
  const uint8_t* q;
  const float* tscale;
};

// ---- launches (each queues on `s` and returns the launch status) ----------

// Buffer-resource loads: base pointer in scalar registers (it must be the
// same in every lane), a 32-bit per-lane byte offset and a uniform one.
// POLICY is the cache-policy immediate (0: default, 2: nontemporal).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void* p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, 0x7FFFFFFF, 0x00020000);
}
template <class V, int POLICY>
__device__ __forceinline__ V bload(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  if constexpr (sizeof(V) == 16)
    return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, POLICY));
  else if constexpr (sizeof(V) == 8)
    return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, POLICY));
  else
    return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, POLICY));
}
// a pointer that is the same in every lane, moved to scalar registers
template <class T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
  return reinterpret_cast<const T*>((uint64_t(hi) << 32) | lo);
}

// whether the small-T router (and so the streaming path's fused router
// launch) covers this shape; the large-T router covers every shape
bool route_small_fits(const Shape& sh);
hipError_t launch_route_small(const Shape& sh, const bf16_t* x, const bf16_t* wr, const float* bias,
                              const Workspace& ws, hipStream_t s);
hipError_t launch_route_large(const Shape& sh, const bf16_t* x, const bf16_t* wr, const float* bias,
                              const Workspace& ws, hipStream_t s);
hipError_t launch_align(const Shape& sh, const Workspace& ws, hipStream_t s);

// weight streaming (small T)
struct StreamArgs {
  Shape sh;
  const bf16_t* x;
  // bf16 weights (nvfp4 == false)
  const bf16_t *wg, *wu, *wd, *dg, *du, *dd;
  // NVFP4 weights (nvfp4 == true)
  Fp4Mat fg, fu, fd, fdg, fdu, fdd;
  bool nvfp4;
  // FP8 weights (fp8 == true)
  Fp8Mat qg, qu, qd, qdg, qdu, qdd;
  bool fp8;
  // NVFP4 activations (W4A4): device fp32 global scales of x (gate/up
  // input), h (routed down input) and h_d (dense down input), or null
  const float* in_scale;
};
// Streaming path (T <= 64, bf16 weights).  The router and the dense
// branch's gate/up units share one launch; then the routed gate/up partial
// sums, the GeGLU of the summed slices (routed and dense rows), and the
// down units (routed and dense).
hipError_t launch_route_dense(const StreamArgs& a, const bf16_t* wr, const float* bias, const Workspace& ws,
                              hipStream_t s);
hipError_t launch_stream_gateup(const StreamArgs& a, const Workspace& ws, hipStream_t s);
hipError_t launch_stream_geglu(const StreamArgs& a, const Workspace& ws, hipStream_t s);
hipError_t launch_stream_down(const StreamArgs& a, const Workspace& ws, hipStream_t s);
// h and y rows of the last streamed forward into caller buffers in grouped
// (perm) order; needs ws.pos from launch_align; either pointer may be null
hipError_t launch_stream_export(const Shape& sh, const Workspace& ws, bf16_t* h_rows, bf16_t* y_rows, hipStream_t s);

// MFMA tiles (large T)
hipError_t launch_gemm_gateup(const StreamArgs& a, const Workspace& ws, int max_mtiles, hipStream_t s);
// yd_out: where the dense rows go (null: ws.y_d)
hipError_t launch_gemm_down(const StreamArgs& a, const Workspace& ws, int max_mtiles, hipStream_t s,
                            bf16_t* yd_out = nullptr);

// NVFP4 weights streamed into registers (fp4mm.hip), any T: gate/up with the
// GeGLU (routed rows and the dense branch) and down.  max_tiles128: the
// capacity of ws.mtiles128.
hipError_t launch_fp4_gateup(const StreamArgs& a, const Workspace& ws, int max_tiles128, hipStream_t s);
hipError_t launch_fp4_down(const StreamArgs& a, const Workspace& ws, int max_tiles128, hipStream_t s,
                           bf16_t* yd_out = nullptr);

// NVFP4 weights streamed for few tokens (fp4stream.hip): the router runs
// first (launch_route_small), then gate/up writes h / h_d (bf16, slot rows)
// with the GeGLU, and down writes y (slot rows) and y_d in bf16, for the
// combine with slot_rows and no dense slices.  fp4_stream_fits: the shape
// and T these kernels take (T <= 64; H, I, D multiples of 64 up to 3072).
bool fp4_stream_fits(const Shape& sh);
hipError_t launch_fs4_gateup(const StreamArgs& a, const Workspace& ws, hipStream_t s);
hipError_t launch_fs4_down(const StreamArgs& a, const Workspace& ws, hipStream_t s);

// yd_slices: 0 = dense output in ws.y_d (bf16); n > 0 = n fp32 slices in
// ws.ydp, summed in order (and stored to ws.y_d as bf16).  slot_rows: the
// expert rows of token t are ws.y rows t*k .. t*k+k-1 (streaming path);
// else rows ws.pos[t*k + j] (grouped order).
// sandwich norms: xn = bf16(RMSNorm(x) * pre); out = resid + RMSNorm(block) * post
hipError_t launch_rmsnorm(const Shape& sh, const bf16_t* x, const float* pre, float eps, bf16_t* xn,
                          hipStream_t s);
hipError_t launch_combine_norm(const Shape& sh, const Workspace& ws, const bf16_t* resid, const float* post,
                               float eps, bf16_t* out, int yd_slices, bool slot_rows, hipStream_t s);
// NVFP4 activations: rows x K bf16 (row pitch ld elements) quantised in
// 16-groups with the global scale *s_in (device); in == out allowed
hipError_t launch_quant_act(const bf16_t* in, bf16_t* out, long long rows, int K, int ld, const float* s_in,
                            hipStream_t s);
hipError_t launch_combine(const Shape& sh, const Workspace& ws, bf16_t* out, bool accumulate, int yd_slices,
                          bool slot_rows, hipStream_t s);

}  // namespace moe
