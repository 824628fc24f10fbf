// Weight-streaming GEMMs of the MoE block for few tokens (T <= 64, decode).
//
// At T = 8 each selected expert sees 1..8 tokens, so its matrices are read
// once and each weight feeds a handful of FMAs: the work is bound by HBM
// bandwidth.  Both kernels are built from one unit routine:
//
//   unit = (weight matrix, NCOLS output columns, K rows [kbeg, kend)),
//   applied to <= 8 activation rows (bf16, in global memory).
//   Thread = (column group of 8 columns = one 16-byte load per weight row,
//   row group owning a contiguous run of R rows).  16 (1-2 rows) or 8 (more
//   rows) weight rows' loads are in flight per thread.  For 1-2 activation rows each thread loads its own
//   activation values alongside the weights (no LDS staging, no barrier);
//   for more rows they are staged in LDS transposed ([k][row], one 16-byte
//   read feeds 8 rows) while the first weight batch is already in flight.
//   Row-group partial sums are folded with shuffles, then across waves.
//
//   gate/up (k_stream_gateup): units are (expert or dense branch, gate or up
//     matrix, 64 columns, one of kStreamKS K-slices) over the group's token
//     rows (x gathered through perm).  Each unit writes fp32 partial
//     pre-activations; a small kernel then sums the slices in fixed order
//     and writes h = gelu_tanh(G) * U (the GeGLU) in bf16.  (No in-kernel
//     hand-off between blocks: on this multi-XCD part a device-scope
//     release writes back the L2, which is far dearer than a launch.)
//   down (k_stream_down): units are (expert, 128 columns) over the expert's
//     h rows, output rows y in bf16; the dense branch's longer K is cut into
//     kDenseDownKS slices whose fp32 partial outputs the combine sums.
//
// Grids are sized by the upper bound on active experts; units past the
// device-side active list exit at once.  Dense-branch units come first.
#include <algorithm>
#include <type_traits>

#include "common.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kRowsChunk = 8;
constexpr int kU = 16;  // weight rows in flight per thread

__device__ __forceinline__ uint32_t perm_lo16(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);  // a.lo | b.lo << 16
}
__device__ __forceinline__ uint32_t perm_hi16(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);  // a.hi | b.hi << 16
}

// partial pre-activations: [KS][rows][2][N] fp32; routed rows first, then
// the dense rows (max 64) in their own region
__device__ __forceinline__ float* part_ptr(const Workspace& ws, const Shape& sh, bool dense, int ks, int row,
                                           int mat) {
  if (!dense) return ws.part + ((size_t(ks) * kStreamRows + row) * 2 + mat) * sh.I;
  float* base = ws.part + size_t(kStreamKS) * kStreamRows * 2 * sh.I;
  return base + ((size_t(ks) * kRouteSmallT + row) * 2 + mat) * sh.D;
}

// Fold acc over the row groups of the block; returns [NT][NCOLS] sums in LDS.
template <int NT, int NCOLS, int CPT>
__device__ const float* fold_rows(float (&acc)[NT][CPT], float* red) {
  constexpr int CG = NCOLS / CPT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int r = 0; r < NT; ++r)
#pragma unroll
    for (int c = 0; c < CPT; ++c)
#pragma unroll
      for (int off = CG; off < kWave; off <<= 1) acc[r][c] += __shfl_xor(acc[r][c], off, kWave);
  __syncthreads();  // red may alias staged rows
  if (lane < CG) {
#pragma unroll
    for (int r = 0; r < NT; ++r)
#pragma unroll
      for (int c = 0; c < CPT; ++c) red[(wave * NT + r) * NCOLS + lane * CPT + c] = acc[r][c];
  }
  __syncthreads();
  float* sums = red + 4 * NT * NCOLS;
  for (int o = tid; o < NT * NCOLS; o += kThreads) {
    float s = 0.f;
#pragma unroll
    for (int wv = 0; wv < 4; ++wv) s += red[wv * NT * NCOLS + o];
    sums[o] = s;
  }
  __syncthreads();
  return sums;
}

// acc[c] += x.lo * w[k][c] + x.hi * w[k+1][c] for the CPT columns of a row
// pair: the rows' packed bf16 pairs are re-paired along k with a byte
// permute and fed to the bf16 dot2 instruction (fp32 accumulate).
template <int CPT, class V>
__device__ __forceinline__ void dot_rows2(float (&acc)[CPT], const V& w0, const V& w1, uint32_t xpair) {
  const bf16x2_t xp = __builtin_bit_cast(bf16x2_t, xpair);
#pragma unroll
  for (int d = 0; d < CPT / 2; ++d) {
    const bf16x2_t lo = __builtin_bit_cast(bf16x2_t, perm_lo16(w0[d], w1[d]));  // column 2d
    const bf16x2_t hi = __builtin_bit_cast(bf16x2_t, perm_hi16(w0[d], w1[d]));  // column 2d+1
    acc[2 * d] = __builtin_amdgcn_fdot2_f32_bf16(lo, xp, acc[2 * d], false);
    acc[2 * d + 1] = __builtin_amdgcn_fdot2_f32_bf16(hi, xp, acc[2 * d + 1], false);
  }
}

// NT <= 2 rows: activations loaded per batch into registers.
// act[r] = the activation row r (bf16, length >= kend), or null for zero.
template <int NT, int NCOLS>
__device__ const float* unit_direct(const bf16_t* __restrict__ w, int ldw, int kbeg, int kend,
                                    const bf16_t* const* act, float* red) {
  constexpr int CG = NCOLS / 8, RG = kThreads / CG;
  const int cg = threadIdx.x % CG, rg = threadIdx.x / CG;
  const int R = (kend - kbeg) / RG;  // rows per thread (multiple of 4)
  const int k0 = kbeg + rg * R;
  float acc[NT][8];
#pragma unroll
  for (int r = 0; r < NT; ++r)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[r][c] = 0.f;
  const bf16_t* pw = w + (long long)k0 * ldw + cg * 8;
  for (int b = 0; b < R; b += kU) {
    u32x4_t vw[kU];
    u32x2_t va[NT][kU / 4];
#pragma unroll
    for (int i = 0; i < kU; ++i)
      vw[i] = (b + i < R) ? __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(pw + (long long)(b + i) * ldw))
                          : u32x4_t{0, 0, 0, 0};
#pragma unroll
    for (int r = 0; r < NT; ++r)
#pragma unroll
      for (int q = 0; q < kU / 4; ++q)
        va[r][q] = (act[r] && b + 4 * q < R) ? *reinterpret_cast<const u32x2_t*>(act[r] + k0 + b + 4 * q)
                                              : u32x2_t{0, 0};
    // rows past R hold zero weights: no branch, so the loop fully unrolls
#pragma unroll
    for (int i = 0; i < kU; i += 2)
#pragma unroll
      for (int r = 0; r < NT; ++r) dot_rows2<8>(acc[r], vw[i], vw[i + 1], va[r][i / 4][(i / 2) & 1]);
  }
  return fold_rows<NT, NCOLS, 8>(acc, red);
}

// NT in (2, 8] rows: activations staged in LDS as xs[k - kbeg][8]; the first
// weight batch is issued before the staging.
template <int NT, int NCOLS, int CPT, int U>
__device__ const float* unit_staged(const bf16_t* __restrict__ w, int ldw, int kbeg, int kend,
                                    const bf16_t* const* act, bf16_t* xs, float* red) {
  constexpr int CG = NCOLS / CPT, RG = kThreads / CG;
  typedef typename std::conditional<CPT == 8, u32x4_t, u32x2_t>::type vec_t;
  const int cg = threadIdx.x % CG, rg = threadIdx.x / CG;
  const int R = (kend - kbeg) / RG;  // even
  const int k0 = kbeg + rg * R;
  float acc[NT][CPT];
#pragma unroll
  for (int r = 0; r < NT; ++r)
#pragma unroll
    for (int c = 0; c < CPT; ++c) acc[r][c] = 0.f;
  const bf16_t* pw = w + (long long)k0 * ldw + cg * CPT;
  vec_t vw[U];
#pragma unroll
  for (int i = 0; i < U; ++i)
    vw[i] = (i < R) ? __builtin_nontemporal_load(reinterpret_cast<const vec_t*>(pw + (long long)i * ldw)) : vec_t{};
  // stage: a thread loads one 8-k piece of every row (two halves of 4 rows)
  // and transposes it in registers into 16-bit runs of xs[k][0..8)
  const int nch = (kend - kbeg) / 8;
#pragma unroll 1
  for (int c = threadIdx.x; c < nch; c += kThreads) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      u32x4_t v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bf16_t* src = act[4 * hf + r];
        v[r] = src ? *reinterpret_cast<const u32x4_t*>(src + kbeg + c * 8) : u32x4_t{0, 0, 0, 0};
      }
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const u32x2_t lo = {perm_lo16(v[0][d], v[1][d]), perm_lo16(v[2][d], v[3][d])};
        const u32x2_t hi = {perm_hi16(v[0][d], v[1][d]), perm_hi16(v[2][d], v[3][d])};
        *reinterpret_cast<u32x2_t*>(xs + (c * 8 + 2 * d) * kRowsChunk + 4 * hf) = lo;
        *reinterpret_cast<u32x2_t*>(xs + (c * 8 + 2 * d + 1) * kRowsChunk + 4 * hf) = hi;
      }
    }
  }
  __syncthreads();
  for (int b = 0;;) {
#pragma unroll
    for (int i = 0; i < U; i += 2) {
      // rows past R hold zero weights; their LDS row index is clamped
      const int kr = min(b + i, R - 2);
      const u32x4_t v0 = *reinterpret_cast<const u32x4_t*>(xs + (k0 - kbeg + kr) * kRowsChunk);
      const u32x4_t v1 = *reinterpret_cast<const u32x4_t*>(xs + (k0 - kbeg + kr + 1) * kRowsChunk);
#pragma unroll
      for (int r = 0; r < NT; ++r) {
        // (x[r][k], x[r][k+1]) from the two staged rows
        const uint32_t xp = (r & 1) ? perm_hi16(v0[r / 2], v1[r / 2]) : perm_lo16(v0[r / 2], v1[r / 2]);
        dot_rows2<CPT>(acc[r], vw[i], vw[i + 1], xp);
      }
    }
    b += U;
    if (b >= R) break;
#pragma unroll
    for (int i = 0; i < U; ++i)
      vw[i] = (b + i < R) ? __builtin_nontemporal_load(reinterpret_cast<const vec_t*>(pw + (long long)(b + i) * ldw))
                          : vec_t{};
  }
  return fold_rows<NT, NCOLS, CPT>(acc, red);
}

// one chunk of nr <= 8 rows: sums [nr][NCOLS] in LDS
template <int NCOLS>
__device__ const float* stream_unit(int nr, const bf16_t* w, int ldw, int kbeg, int kend, const bf16_t* const* act,
                                    bf16_t* xs, float* red) {
  if (nr <= 1) return unit_direct<1, NCOLS>(w, ldw, kbeg, kend, act, red);
  if (nr <= 2) return unit_direct<2, NCOLS>(w, ldw, kbeg, kend, act, red);
  if (nr <= 4) return unit_staged<4, NCOLS, 8, 8>(w, ldw, kbeg, kend, act, xs, red);
  return unit_staged<8, NCOLS, 8, 4>(w, ldw, kbeg, kend, act, xs, red);
}

// ---------------------------------------------------------------------------
// gate/up
// ---------------------------------------------------------------------------

// blocks [0, units_dense) are dense-branch units, the rest routed units
__global__ __launch_bounds__(kThreads) void k_stream_gateup(StreamArgs a, Workspace ws, int units_dense) {
  const Shape& sh = a.sh;
  const int H = sh.H;
  int u = blockIdx.x;
  bool dense;
  int grp = -1, row0 = 0, rows, N;
  if (u < units_dense) {
    dense = true;
    rows = sh.T;
    N = sh.D;
  } else {
    u -= units_dense;
    const int per = (sh.I / 64) * 2 * kStreamKS;
    const int ai = u / per;
    if (ai >= ws.meta[1]) return;
    u %= per;
    dense = false;
    grp = ws.active[4 * ai];
    row0 = ws.active[4 * ai + 1];
    rows = ws.active[4 * ai + 2];
    N = sh.I;
  }
  // u -> (n-block, matrix, K-slice), K-slice fastest
  const int ks = u % kStreamKS;
  const int mat = (u / kStreamKS) & 1;
  const int n0 = (u / (2 * kStreamKS)) * 64;
  const int kbeg = ks * H / kStreamKS, kend = (ks + 1) * H / kStreamKS;
  const bf16_t* w = dense ? (mat ? a.du : a.dg) + n0 : (mat ? a.wu : a.wg) + (long long)grp * H * sh.I + n0;

  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  bf16_t* xs = reinterpret_cast<bf16_t*>(smem_raw);  // [kend-kbeg][8] staged rows
  float* red = reinterpret_cast<float*>(smem_raw);   // [5][8][64]
  __shared__ const bf16_t* act[kRowsChunk];

  for (int c0 = 0; c0 < rows; c0 += kRowsChunk) {
    const int nr = min(kRowsChunk, rows - c0);
    if (threadIdx.x < kRowsChunk) {
      const int r = threadIdx.x;
      act[r] = r < nr ? a.x + (long long)(dense ? c0 + r : ws.perm[row0 + c0 + r]) * H : nullptr;
    }
    __syncthreads();
    const bf16_t* rowp[kRowsChunk];
#pragma unroll
    for (int r = 0; r < kRowsChunk; ++r) rowp[r] = act[r];
    const float* sums = stream_unit<64>(nr, w, N, kbeg, kend, rowp, xs, red);
    float* out = part_ptr(ws, sh, dense, ks, (dense ? 0 : row0) + c0, mat) + n0;
    for (int o = threadIdx.x; o < nr * 64; o += kThreads) out[(long long)(o >> 6) * 2 * N + (o & 63)] = sums[o];
    __syncthreads();
  }

}

// GeGLU of the streamed rows: h = gelu_tanh(sum G) * (sum U), K-slices in
// fixed order, bf16.  Rows: the T*k routed rows (expert-grouped order) and/or
// the T dense rows; 4 columns per thread.
__global__ __launch_bounds__(kThreads) void k_stream_geglu(Shape sh, Workspace ws, int routed, int dense_rows) {
  const int rrows = routed ? sh.T * sh.k : 0;
  const long long nr4 = (long long)rrows * (sh.I / 4);
  const long long nd4 = dense_rows ? (long long)sh.T * (sh.D / 4) : 0;
  for (long long i = blockIdx.x * (long long)kThreads + threadIdx.x; i < nr4 + nd4;
       i += (long long)gridDim.x * kThreads) {
    const bool dense = i >= nr4;
    const long long j = dense ? i - nr4 : i;
    const int N = dense ? sh.D : sh.I;
    const int row = int(j / (N / 4)), n4 = int(j % (N / 4)) * 4;
    float4 g = make_float4(0.f, 0.f, 0.f, 0.f), up = g;
#pragma unroll
    for (int s = 0; s < kStreamKS; ++s) {
      const float4 pg = *reinterpret_cast<const float4*>(part_ptr(ws, sh, dense, s, row, 0) + n4);
      const float4 pu = *reinterpret_cast<const float4*>(part_ptr(ws, sh, dense, s, row, 1) + n4);
      g.x += pg.x; g.y += pg.y; g.z += pg.z; g.w += pg.w;
      up.x += pu.x; up.y += pu.y; up.z += pu.z; up.w += pu.w;
    }
    bf16_t* hout = (dense ? ws.h_d : ws.h) + (long long)row * N + n4;
    *reinterpret_cast<u32x2_t*>(hout) = u32x2_t{pack_bf16x2(gelu_tanh(g.x) * up.x, gelu_tanh(g.y) * up.y),
                                                pack_bf16x2(gelu_tanh(g.z) * up.z, gelu_tanh(g.w) * up.w)};
  }
}

// ---------------------------------------------------------------------------
// down
// ---------------------------------------------------------------------------

// blocks [0, units_dense) are dense-branch units, the rest routed units
__global__ __launch_bounds__(kThreads) void k_stream_down(StreamArgs a, Workspace ws, int units_dense) {
  const Shape& sh = a.sh;
  const int H = sh.H;
  const int nblk = H / 128;
  int u = blockIdx.x;
  bool dense;
  int grp = -1, row0 = 0, rows, K, kbeg = 0, kend;
  if (u < units_dense) {
    // dense branch: (column block, K-slice of whole 64-row groups), fp32 partials
    dense = true;
    rows = sh.T;
    K = sh.D;
    const int ks = u % kDenseDownKS, g64 = sh.D / 64;
    u /= kDenseDownKS;
    kbeg = (ks * g64 / kDenseDownKS) * 64;
    kend = ((ks + 1) * g64 / kDenseDownKS) * 64;
    (void)ks;
  } else {
    u -= units_dense;
    const int ai = u / nblk;
    if (ai >= ws.meta[1]) return;
    u %= nblk;
    dense = false;
    grp = ws.active[4 * ai];
    row0 = ws.active[4 * ai + 1];
    rows = ws.active[4 * ai + 2];
    K = sh.I;
    kend = K;
  }
  const int n0 = u * 128;
  const bf16_t* wd = (dense ? a.dd : a.wd + (long long)grp * sh.I * H) + n0;
  const bf16_t* hin = dense ? ws.h_d : ws.h + (long long)row0 * sh.I;
  const int ksd = dense ? (blockIdx.x % kDenseDownKS) : 0;

  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  bf16_t* hs = reinterpret_cast<bf16_t*>(smem_raw);  // [K][8] staged rows
  float* red = reinterpret_cast<float*>(smem_raw);   // [5][8][128]
  for (int c0 = 0; c0 < rows; c0 += kRowsChunk) {
    const int nr = min(kRowsChunk, rows - c0);
    const bf16_t* rowp[kRowsChunk];
#pragma unroll
    for (int r = 0; r < kRowsChunk; ++r) rowp[r] = r < nr ? hin + (long long)(c0 + r) * K : nullptr;
    const float* sums = stream_unit<128>(nr, wd, H, kbeg, kend, rowp, hs, red);
    if (dense) {
      float* o = ws.ydp + ((long long)ksd * kRouteSmallT + c0) * H + n0;
      for (int i = threadIdx.x; i < nr * 128; i += kThreads) o[(long long)(i >> 7) * H + (i & 127)] = sums[i];
    } else {
      bf16_t* o = ws.y + (long long)(row0 + c0) * H + n0;
      for (int i = threadIdx.x; i < nr * 128; i += kThreads)
        o[(long long)(i >> 7) * H + (i & 127)] = (bf16_t)f32_to_bf16_bits(sums[i]);
    }
    __syncthreads();
  }
}

}  // namespace

// part: which branch to queue (the dense branch does not depend on the
// routing, so the caller may run it on another stream)
hipError_t launch_stream_gateup(const StreamArgs& a, const Workspace& ws, StreamPart part, hipStream_t s) {
  const Shape& sh = a.sh;
  const bool dense = part == StreamPart::Dense && sh.D > 0;
  const int ud = dense ? (sh.D / 64) * 2 * kStreamKS : 0;
  const int max_active = part == StreamPart::Routed ? std::min(sh.E, sh.T * sh.k) : 0;
  const int units = ud + max_active * (sh.I / 64) * 2 * kStreamKS;
  if (units == 0) return hipSuccess;
  const size_t kl = size_t(sh.H) / kStreamKS;
  const size_t lds = std::max(kl * kRowsChunk * 2, size_t(5) * kRowsChunk * 64 * 4);
  hipLaunchKernelGGL(k_stream_gateup, dim3(units), dim3(kThreads), lds, s, a, ws, ud);
  const long long n4 = dense ? (long long)sh.T * sh.D / 4 : (long long)sh.T * sh.k * sh.I / 4;
  const int gblocks = int(std::min<long long>(1024, (n4 + kThreads - 1) / kThreads));
  hipLaunchKernelGGL(k_stream_geglu, dim3(gblocks), dim3(kThreads), 0, s, sh, ws, dense ? 0 : 1, dense ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_stream_down(const StreamArgs& a, const Workspace& ws, StreamPart part, hipStream_t s) {
  const Shape& sh = a.sh;
  const int nblk = sh.H / 128;
  const bool dense = part == StreamPart::Dense && sh.D > 0;
  const int ud = dense ? nblk * kDenseDownKS : 0;
  const int max_active = part == StreamPart::Routed ? std::min(sh.E, sh.T * sh.k) : 0;
  const int units = ud + max_active * nblk;
  if (units == 0) return hipSuccess;
  const int kmax = std::max(sh.I, sh.D);
  const size_t lds = std::max(size_t(kmax) * kRowsChunk * 2, size_t(5) * kRowsChunk * 128 * 4);
  hipLaunchKernelGGL(k_stream_down, dim3(units), dim3(kThreads), lds, s, a, ws, ud);
  return hipGetLastError();
}

}  // namespace moe
