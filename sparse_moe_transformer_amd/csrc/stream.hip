// Weight-streaming GEMMs of the MoE block for few tokens per expert (decode).
//
// At T = 8 every selected expert sees 1..8 tokens, so its matrices are read
// once and each weight feeds only a handful of FMAs: the work is bound by
// HBM bandwidth.  A work unit is (expert or dense branch, a block of output
// columns); its weights are read with 16-byte coalesced loads, each thread
// owning 8 adjacent columns and a strided subset of the K rows, and the few
// token rows live in LDS transposed ([k][token], 8 tokens = 16 bytes) so one
// LDS read feeds 8 x NT FMAs.  Partial sums over K are reduced across lanes
// (shuffles) and waves (LDS).  The grid is sized by the upper bound on active
// experts; units past the device-side active list exit at once.
//
//   gate/up unit: 64 columns of both Wg and Wu over all K = H rows, then
//                 h = gelu_tanh(g) * u (GeGLU) for each token row.
//   down unit:    256 columns of Wd over all K = I (or D) rows.
// Token rows are processed in chunks of 8; a unit with more rows re-reads
// its weights (from L2) per chunk.
#include <algorithm>

#include "common.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kRowsChunk = 8;

// 8 consecutive bf16 (one 16-byte load) -> 8 floats
__device__ __forceinline__ void unpack8(const u32x4_t& v, float* f) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    f[2 * d] = bf16_lo(v[d]);
    f[2 * d + 1] = bf16_hi(v[d]);
  }
}

struct UnitRows {
  int grp;     // expert id, or -1 for the dense branch
  int row0;    // first row (expert-grouped order) or first token (dense)
  int rows;
};

// ---------------------------------------------------------------------------
// gate/up
// ---------------------------------------------------------------------------

template <int NT>
__device__ void gateup_chunk(const StreamArgs& a, const bf16_t* wg, const bf16_t* wu, int ldw, int K,
                             const bf16_t* xs, float* red, int n0, int nrows, bf16_t* out, int ldo) {
  const int tid = threadIdx.x;
  const int cg = tid & 7;    // 8 column groups of 8
  const int rg = tid >> 3;   // 32 row groups
  float ag[NT][8], au[NT][8];
#pragma unroll
  for (int r = 0; r < NT; ++r)
#pragma unroll
    for (int c = 0; c < 8; ++c) ag[r][c] = au[r][c] = 0.f;

  const bf16_t* pg = wg + n0 + cg * 8;
  const bf16_t* pu = wu + n0 + cg * 8;
  constexpr int U = 4;
  int k = rg;
  for (; k + 32 * (U - 1) < K; k += 32 * U) {
    u32x4_t vg[U], vu[U], vx[U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
      vg[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(pg + (long long)(k + 32 * i) * ldw));
      vu[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(pu + (long long)(k + 32 * i) * ldw));
    }
#pragma unroll
    for (int i = 0; i < U; ++i) vx[i] = *reinterpret_cast<const u32x4_t*>(xs + (k + 32 * i) * kRowsChunk);
#pragma unroll
    for (int i = 0; i < U; ++i) {
      float fg[8], fu[8], fx[8];
      unpack8(vg[i], fg);
      unpack8(vu[i], fu);
      unpack8(vx[i], fx);
#pragma unroll
      for (int r = 0; r < NT; ++r)
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          ag[r][c] += fx[r] * fg[c];
          au[r][c] += fx[r] * fu[c];
        }
    }
  }
  for (; k < K; k += 32) {
    u32x4_t vg = *reinterpret_cast<const u32x4_t*>(pg + (long long)k * ldw);
    u32x4_t vu = *reinterpret_cast<const u32x4_t*>(pu + (long long)k * ldw);
    u32x4_t vx = *reinterpret_cast<const u32x4_t*>(xs + k * kRowsChunk);
    float fg[8], fu[8], fx[8];
    unpack8(vg, fg);
    unpack8(vu, fu);
    unpack8(vx, fx);
#pragma unroll
    for (int r = 0; r < NT; ++r)
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        ag[r][c] += fx[r] * fg[c];
        au[r][c] += fx[r] * fu[c];
      }
  }
  // reduce the 8 row groups of a wave (lane bits 3..5)
#pragma unroll
  for (int r = 0; r < NT; ++r)
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int off = 8; off < 64; off <<= 1) {
        ag[r][c] += __shfl_xor(ag[r][c], off, kWave);
        au[r][c] += __shfl_xor(au[r][c], off, kWave);
      }
  const int lane = tid & 63, wave = tid >> 6;
  __syncthreads();  // red aliases the staged rows
  // red layout: [wave][r][g/u][64 columns]
  if (lane < 8) {
#pragma unroll
    for (int r = 0; r < NT; ++r)
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        red[((wave * NT + r) * 2 + 0) * 64 + lane * 8 + c] = ag[r][c];
        red[((wave * NT + r) * 2 + 1) * 64 + lane * 8 + c] = au[r][c];
      }
  }
  __syncthreads();
  for (int o = tid; o < nrows * 64; o += kThreads) {
    const int r = o >> 6, col = o & 63;
    float g = 0.f, u = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      g += red[((w * NT + r) * 2 + 0) * 64 + col];
      u += red[((w * NT + r) * 2 + 1) * 64 + col];
    }
    out[(long long)r * ldo + n0 + col] = (bf16_t)f32_to_bf16_bits(gelu_tanh(g) * u);
  }
  __syncthreads();
}

__global__ __launch_bounds__(kThreads) void k_stream_gateup(StreamArgs a, Workspace ws, int units_dense) {
  const Shape& sh = a.sh;
  const int H = sh.H;
  int u = blockIdx.x;
  UnitRows ur;
  int n0, N;
  const bf16_t *wg, *wu;
  bf16_t* out;
  if (u < units_dense) {
    N = sh.D;
    n0 = u * 64;
    ur = {-1, 0, sh.T};
    wg = a.dg;
    wu = a.du;
    out = ws.h_d;
  } else {
    u -= units_dense;
    const int nblk = sh.I / 64;
    const int ai = u / nblk;
    if (ai >= ws.meta[1]) return;
    N = sh.I;
    n0 = (u % nblk) * 64;
    ur = {ws.active[4 * ai], ws.active[4 * ai + 1], ws.active[4 * ai + 2]};
    wg = a.wg + (long long)ur.grp * H * sh.I;
    wu = a.wu + (long long)ur.grp * H * sh.I;
    out = ws.h;
  }
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  bf16_t* xs = reinterpret_cast<bf16_t*>(smem_raw);  // [H][8] staged rows
  float* red = reinterpret_cast<float*>(smem_raw);   // [4][8][2][64], after the K loop

  for (int c0 = 0; c0 < ur.rows; c0 += kRowsChunk) {
    const int nr = min(kRowsChunk, ur.rows - c0);
    // stage the chunk's token rows transposed: xs[k][r]
    for (int r = 0; r < kRowsChunk; ++r) {
      const bf16_t* src = nullptr;
      if (r < nr) {
        int tok = (ur.grp >= 0) ? ws.perm[ur.row0 + c0 + r] : c0 + r;
        src = a.x + (long long)tok * H;
      }
      for (int k = threadIdx.x; k < H; k += kThreads) xs[k * kRowsChunk + r] = src ? src[k] : (bf16_t)0;
    }
    __syncthreads();
    bf16_t* o = out + (long long)(ur.row0 + c0) * N;
    if (nr <= 1)
      gateup_chunk<1>(a, wg, wu, N, H, xs, red, n0, nr, o, N);
    else if (nr <= 2)
      gateup_chunk<2>(a, wg, wu, N, H, xs, red, n0, nr, o, N);
    else if (nr <= 4)
      gateup_chunk<4>(a, wg, wu, N, H, xs, red, n0, nr, o, N);
    else
      gateup_chunk<8>(a, wg, wu, N, H, xs, red, n0, nr, o, N);
  }
}

// ---------------------------------------------------------------------------
// down
// ---------------------------------------------------------------------------

template <int NT>
__device__ void down_chunk(const bf16_t* wd, int ldw, int K, const bf16_t* hs, float* red, int n0,
                           int nrows, bf16_t* out, int ldo) {
  const int tid = threadIdx.x;
  const int cg = tid & 31;   // 32 column groups of 8 -> 256 columns
  const int rg = tid >> 5;   // 8 row groups
  float acc[NT][8];
#pragma unroll
  for (int r = 0; r < NT; ++r)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[r][c] = 0.f;
  const bf16_t* pw = wd + n0 + cg * 8;
  constexpr int U = 4;
  int k = rg;
  for (; k + 8 * (U - 1) < K; k += 8 * U) {
    u32x4_t vw[U], vh[U];
#pragma unroll
    for (int i = 0; i < U; ++i)
      vw[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(pw + (long long)(k + 8 * i) * ldw));
#pragma unroll
    for (int i = 0; i < U; ++i) vh[i] = *reinterpret_cast<const u32x4_t*>(hs + (k + 8 * i) * kRowsChunk);
#pragma unroll
    for (int i = 0; i < U; ++i) {
      float fw[8], fh[8];
      unpack8(vw[i], fw);
      unpack8(vh[i], fh);
#pragma unroll
      for (int r = 0; r < NT; ++r)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[r][c] += fh[r] * fw[c];
    }
  }
  for (; k < K; k += 8) {
    u32x4_t vw = *reinterpret_cast<const u32x4_t*>(pw + (long long)k * ldw);
    u32x4_t vh = *reinterpret_cast<const u32x4_t*>(hs + k * kRowsChunk);
    float fw[8], fh[8];
    unpack8(vw, fw);
    unpack8(vh, fh);
#pragma unroll
    for (int r = 0; r < NT; ++r)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[r][c] += fh[r] * fw[c];
  }
#pragma unroll
  for (int r = 0; r < NT; ++r)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[r][c] += __shfl_xor(acc[r][c], 32, kWave);
  const int lane = tid & 63, wave = tid >> 6;
  __syncthreads();  // red aliases the staged rows
  if (lane < 32) {
#pragma unroll
    for (int r = 0; r < NT; ++r)
#pragma unroll
      for (int c = 0; c < 8; ++c) red[(wave * NT + r) * 256 + lane * 8 + c] = acc[r][c];
  }
  __syncthreads();
  for (int o = tid; o < nrows * 256; o += kThreads) {
    const int r = o >> 8, col = o & 255;
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) s += red[(w * NT + r) * 256 + col];
    out[(long long)r * ldo + n0 + col] = (bf16_t)f32_to_bf16_bits(s);
  }
  __syncthreads();
}

__global__ __launch_bounds__(kThreads) void k_stream_down(StreamArgs a, Workspace ws, int units_dense) {
  const Shape& sh = a.sh;
  const int H = sh.H;
  const int nblk = H / 256;
  int u = blockIdx.x;
  UnitRows ur;
  int K, n0;
  const bf16_t* wd;
  const bf16_t* hin;
  bf16_t* out;
  if (u < units_dense) {
    K = sh.D;
    n0 = u * 256;
    ur = {-1, 0, sh.T};
    wd = a.dd;
    hin = ws.h_d;
    out = ws.y_d;
  } else {
    u -= units_dense;
    const int ai = u / nblk;
    if (ai >= ws.meta[1]) return;
    K = sh.I;
    n0 = (u % nblk) * 256;
    ur = {ws.active[4 * ai], ws.active[4 * ai + 1], ws.active[4 * ai + 2]};
    wd = a.wd + (long long)ur.grp * sh.I * H;
    hin = ws.h;
    out = ws.y;
  }
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  bf16_t* hs = reinterpret_cast<bf16_t*>(smem_raw);  // [K][8] staged rows
  float* red = reinterpret_cast<float*>(smem_raw);   // [4][8][256], after the K loop
  for (int c0 = 0; c0 < ur.rows; c0 += kRowsChunk) {
    const int nr = min(kRowsChunk, ur.rows - c0);
    for (int r = 0; r < kRowsChunk; ++r) {
      const bf16_t* src = (r < nr) ? hin + (long long)(ur.row0 + c0 + r) * K : nullptr;
      for (int k = threadIdx.x; k < K; k += kThreads) hs[k * kRowsChunk + r] = src ? src[k] : (bf16_t)0;
    }
    __syncthreads();
    bf16_t* o = out + (long long)(ur.row0 + c0) * H;
    if (nr <= 1)
      down_chunk<1>(wd, H, K, hs, red, n0, nr, o, H);
    else if (nr <= 2)
      down_chunk<2>(wd, H, K, hs, red, n0, nr, o, H);
    else if (nr <= 4)
      down_chunk<4>(wd, H, K, hs, red, n0, nr, o, H);
    else
      down_chunk<8>(wd, H, K, hs, red, n0, nr, o, H);
  }
}

}  // namespace

hipError_t launch_stream_gateup(const StreamArgs& a, const Workspace& ws, hipStream_t s) {
  const Shape& sh = a.sh;
  const int ud = sh.D > 0 ? sh.D / 64 : 0;
  const int max_active = std::min(sh.E, sh.T * sh.k);
  const int units = ud + max_active * (sh.I / 64);
  const size_t lds = std::max(size_t(sh.H) * kRowsChunk * 2, size_t(4) * kRowsChunk * 2 * 64 * 4);
  hipLaunchKernelGGL(k_stream_gateup, dim3(units), dim3(kThreads), lds, s, a, ws, ud);
  return hipGetLastError();
}

hipError_t launch_stream_down(const StreamArgs& a, const Workspace& ws, hipStream_t s) {
  const Shape& sh = a.sh;
  const int nblk = sh.H / 256;
  const int ud = sh.D > 0 ? nblk : 0;
  const int max_active = std::min(sh.E, sh.T * sh.k);
  const int units = ud + max_active * nblk;
  const int kmax = std::max(sh.I, sh.D);
  const size_t lds = std::max(size_t(kmax) * kRowsChunk * 2, size_t(4) * kRowsChunk * 256 * 4);
  hipLaunchKernelGGL(k_stream_down, dim3(units), dim3(kThreads), lds, s, a, ws, ud);
  return hipGetLastError();
}

}  // namespace moe
