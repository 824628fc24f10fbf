// Weight-streaming GEMMs of the MoE block for few tokens (T <= 64, decode).
//
// At T = 8 each selected expert sees 1..8 tokens, so its matrices are read
// once and each weight feeds a handful of FMAs: the work is bound by HBM
// bandwidth.  Both kernels are built from one unit routine:
//
//   unit = (weight matrix, NCOLS output columns, K rows [kbeg, kend)),
//   applied to <= 8 activation rows.
//   Thread = (column group of 8 columns = one 16-byte load per weight row,
//   row group owning a contiguous run of R rows).  4 to 16 weight rows'
//   loads are in flight per thread (more for fewer activation rows).  For
//   1-2 x rows each thread loads its own activation values alongside the
//   weights (no LDS staging, no barrier); otherwise the rows are staged in
//   LDS transposed ([k][row], one 16-byte read feeds 8 rows) while the first
//   weight batch is already in flight.  Row-group partial sums are folded
//   with shuffles, then across waves.
//
//   gate/up (k_stream_gateup, and the dense units in the router's launch):
//     units are (expert or dense branch, gate or up matrix, 64 columns (FP8:
//     128), one K-slice of whole 64-row groups) over the group's token rows
//     (x gathered by token).  Each unit writes fp32 partial pre-activations.
//     (No in-kernel hand-off between blocks: on this multi-XCD part a
//     device-scope release writes back the L2, which is far dearer than a
//     launch.)
//   down (k_stream_down): units are (expert, 128 columns) over the expert's
//     h rows, output rows y in bf16; the dense branch's longer K is cut into
//     K-slices whose fp32 partial outputs the combine sums.  With bf16
//     weights beside experts each down unit forms its rows of h = bf16(
//     gelu_tanh(G) * U) itself from the partials (slices summed in fixed
//     order); otherwise k_stream_geglu writes h / h_d first.
//
// Routed units need no grouping tables: each block derives its expert's
// rows from topk_idx (at most 64 tokens) with a few LDS atomics.  Routed
// rows are indexed by slot s = t * k + j, so the combine reads a token's k
// rows at s = t * k .. t * k + k - 1.  Grids are sized by the upper bound on
// active experts; units past the last active expert exit at once.  Dense
// and routed units are separate kernel instances.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "route_dev.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kRowsChunk = 8;
constexpr int kU = 16;  // weight rows in flight per thread
constexpr int kDownCols = 128;  // output columns of a routed down unit
constexpr int kDenseDownCols = 128;  // output columns of a dense down unit
constexpr int kDenseOnlyCols = 256;  // output columns of a gate/up unit without experts
constexpr int kDownColsMax = kDenseDownCols > kDownCols ? kDenseDownCols : kDownCols;
// Beside experts, the dense gate/up units are split between the router's
// launch and the routed gate/up launch: the router's hand-off is a latency
// chain, so its launch takes only as many dense units as stream within it
// (this share, in 1/8ths); the rest run first in the routed launch.  FP8
// units (half the bytes) all fit in the router's launch.
constexpr int kDenseRouteEighths = 5;

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
  float* base = ws.part + size_t(kStreamKSMax) * kStreamRows * 2 * sh.I;  // then [kDenseKSMax][64][2][D]
  return base + ((size_t(ks) * kRouteSmallT + row) * 2 + mat) * sh.D;
}

// Weight and activation rows are read through buffer resources (common.h):
// a 32-bit per-thread byte offset plus a uniform (scalar) row offset, so the
// unrolled loads share one address register instead of a 64-bit address
// each.  The base pointers must be block-uniform.
constexpr int kPolicyNT = 2;  // nontemporal: weights are streamed once

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
  const int R = (kend - kbeg) / RG;  // rows per thread (even)
  const int k0 = kbeg + rg * R;
  float acc[NT][8];
#pragma unroll
  for (int r = 0; r < NT; ++r)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[r][c] = 0.f;
  const __amdgpu_buffer_rsrc_t rw = rsrc_of(w);
  const uint32_t wrow = uint32_t(ldw) * 2, wv = uint32_t(k0) * wrow + cg * 16;
  __amdgpu_buffer_rsrc_t rx[NT];
  bool has[NT];
#pragma unroll
  for (int r = 0; r < NT; ++r) {
    const bf16_t* p = uniform_ptr(act[r]);
    has[r] = p != nullptr;
    rx[r] = rsrc_of(p);
  }
  for (int b = 0; b < R; b += kU) {
    u32x4_t vw[kU];
    u32x2_t va[NT][kU / 4];
#pragma unroll
    for (int i = 0; i < kU; ++i)
      vw[i] = (b + i < R) ? bload<u32x4_t, kPolicyNT>(rw, wv, uint32_t(b + i) * wrow) : u32x4_t{0, 0, 0, 0};
    // R is even: a 4-row piece is whole or its last two rows lie past R
    // (they are not read: for the last row group they would lie past kend)
#pragma unroll
    for (int r = 0; r < NT; ++r)
#pragma unroll
      for (int q = 0; q < kU / 4; ++q) {
        const int k = b + 4 * q;
        if (has[r] && k + 4 <= R)
          va[r][q] = bload<u32x2_t, 0>(rx[r], uint32_t(k0) * 2, uint32_t(k) * 2);
        else if (has[r] && k < R)
          va[r][q] = u32x2_t{bload<uint32_t, 0>(rx[r], uint32_t(k0) * 2, uint32_t(k) * 2), 0u};
        else
          va[r][q] = u32x2_t{0, 0};
      }
    // rows past R hold zero weights: no branch, so the loop fully unrolls
#pragma unroll
    for (int i = 0; i < kU; i += 2)
#pragma unroll
      for (int r = 0; r < NT; ++r) dot_rows2<8>(acc[r], vw[i], vw[i + 1], va[r][i / 4][(i / 2) & 1]);
  }
  return fold_rows<NT, NCOLS, 8>(acc, red);
}

// Staging of NT <= 8 activation rows into LDS as xs[k - kbeg][8] (bf16):
// rows read from global memory (x rows of the gate/up units).  A thread
// loads one 8-k piece of every row (two halves of 4 rows) and transposes it
// in registers into 16-bit runs of xs[k][0..8).
struct StageRows {
  const bf16_t* const* act;  // [8] row pointers, null = zero row
  __device__ void operator()(bf16_t* xs, int kbeg, int kend) const {
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
  }
};

// NT <= 8 rows staged in LDS as xs[k - kbeg][8] by `stage`; the first weight
// batch is issued before the staging so that it overlaps it.
template <int NT, int NCOLS, int CPT, int U, class Stage>
__device__ const float* unit_staged(const bf16_t* __restrict__ w, int ldw, int kbeg, int kend, const Stage& stage,
                                    bf16_t* xs, float* red) {
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
  const __amdgpu_buffer_rsrc_t rw = rsrc_of(w);
  const uint32_t wrow = uint32_t(ldw) * 2, wv = uint32_t(k0) * wrow + cg * CPT * 2;
  // two batches of U weight rows: the next batch's loads are issued before
  // the current batch is consumed, so a thread always has loads in flight
  auto load = [&](vec_t (&v)[U], int b) {
#pragma unroll
    for (int i = 0; i < U; ++i) v[i] = (b + i < R) ? bload<vec_t, kPolicyNT>(rw, wv, uint32_t(b + i) * wrow) : vec_t{};
  };
  auto consume = [&](const vec_t (&v)[U], int b) {
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
        dot_rows2<CPT>(acc[r], v[i], v[i + 1], xp);
      }
    }
  };
  vec_t va[U], vb[U];
  load(va, 0);
  stage(xs, kbeg, kend);
  __syncthreads();
  for (int b = 0;;) {
    if (b + U < R) load(vb, b + U);
    consume(va, b);
    b += U;
    if (b >= R) break;
    if (b + U < R) load(va, b + U);
    consume(vb, b);
    b += U;
    if (b >= R) break;
  }
  return fold_rows<NT, NCOLS, CPT>(acc, red);
}

// One chunk of nr <= 8 activation rows: sums [nr][NCOLS] in LDS
template <int NCOLS>
__device__ const float* unit_x_rows(int nr, const bf16_t* w, int ldw, int kbeg, int kend, const bf16_t* const* act,
                                    bf16_t* xs, float* red) {
  if (nr <= 1) return unit_direct<1, NCOLS>(w, ldw, kbeg, kend, act, red);
  if (nr <= 2) return unit_direct<2, NCOLS>(w, ldw, kbeg, kend, act, red);
  const StageRows st{act};
  if (nr <= 4) return unit_staged<4, NCOLS, 8, 8>(w, ldw, kbeg, kend, st, xs, red);
  return unit_staged<8, NCOLS, 8, 4>(w, ldw, kbeg, kend, st, xs, red);
}

// ---------------------------------------------------------------------------
// FP8 weights: [K, N] float8_e4m3fn codes.  A thread reads 8 bytes (8
// columns) per weight row and widens them with the gfx950 e4m3 -> fp32 pair
// conversion (exact); each (activation, weight) product is one fp32 FMA.
// The per-matrix scale is applied by the caller to the summed columns.
// ---------------------------------------------------------------------------

// the 8 weights of one row piece (codes in byte order) as fp32
__device__ __forceinline__ void widen8(const u32x2_t& v, float (&w)[8]) {
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(int(v[d]), false);
    const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8(int(v[d]), true);
    w[4 * d] = lo.x;
    w[4 * d + 1] = lo.y;
    w[4 * d + 2] = hi.x;
    w[4 * d + 3] = hi.y;
  }
}

// NT <= 2 activation rows read directly (as unit_direct)
template <int NT, int NCOLS>
__device__ const float* unit8_direct(const uint8_t* __restrict__ w, int ldw, int kbeg, int kend, int nvalid,
                                     const bf16_t* const* act, float* red) {
  constexpr int CG = NCOLS / 8, RG = kThreads / CG;
  const int cg = threadIdx.x % CG, rg = threadIdx.x / CG;
  const int R = (kend - kbeg) / RG;  // rows per thread (even)
  const int k0 = kbeg + rg * R;
  float acc[NT][8];
#pragma unroll
  for (int r = 0; r < NT; ++r)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[r][c] = 0.f;
  const __amdgpu_buffer_rsrc_t rw = rsrc_of(w);
  const uint32_t wrow = uint32_t(ldw), wv = uint32_t(k0) * wrow + cg * 8;
  const bool colok = cg * 8 < nvalid;  // columns past the matrix's last read nothing
  __amdgpu_buffer_rsrc_t rx[NT];
  bool has[NT];
#pragma unroll
  for (int r = 0; r < NT; ++r) {
    const bf16_t* p = uniform_ptr(act[r]);
    has[r] = p != nullptr;
    rx[r] = rsrc_of(p);
  }
  for (int b = 0; b < R; b += kU) {
    u32x2_t vw[kU];
    u32x2_t va[NT][kU / 4];
#pragma unroll
    for (int i = 0; i < kU; ++i)
      vw[i] = (colok && b + i < R) ? bload<u32x2_t, kPolicyNT>(rw, wv, uint32_t(b + i) * wrow) : u32x2_t{0, 0};
    // R is even: a 4-row activation piece is whole or its last two rows lie past R
#pragma unroll
    for (int r = 0; r < NT; ++r)
#pragma unroll
      for (int q = 0; q < kU / 4; ++q) {
        const int k = b + 4 * q;
        if (has[r] && k + 4 <= R)
          va[r][q] = bload<u32x2_t, 0>(rx[r], uint32_t(k0) * 2, uint32_t(k) * 2);
        else if (has[r] && k < R)
          va[r][q] = u32x2_t{bload<uint32_t, 0>(rx[r], uint32_t(k0) * 2, uint32_t(k) * 2), 0u};
        else
          va[r][q] = u32x2_t{0, 0};
      }
    // rows past R hold zero codes (value 0) and zero activations
#pragma unroll
    for (int i = 0; i < kU; ++i) {
      float wf[8];
      widen8(vw[i], wf);
#pragma unroll
      for (int r = 0; r < NT; ++r) {
        const uint32_t xw = va[r][i / 4][(i / 2) & 1];
        const float xv = (i & 1) ? bf16_hi(xw) : bf16_lo(xw);
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[r][c] = fmaf(xv, wf[c], acc[r][c]);
      }
    }
  }
  return fold_rows<NT, NCOLS, 8>(acc, red);
}

// NT <= 8 activation rows staged in LDS as xs[k - kbeg][8] by `stage` (as
// unit_staged), U weight rows per batch, the next batch in flight while the
// current one is consumed
template <int NT, int NCOLS, int U, class Stage>
__device__ const float* unit8_staged(const uint8_t* __restrict__ w, int ldw, int kbeg, int kend, int nvalid,
                                     const Stage& stage, bf16_t* xs, float* red) {
  constexpr int CG = NCOLS / 8, RG = kThreads / CG;
  const int cg = threadIdx.x % CG, rg = threadIdx.x / CG;
  const int R = (kend - kbeg) / RG;  // even
  const int k0 = kbeg + rg * R;
  float acc[NT][8];
#pragma unroll
  for (int r = 0; r < NT; ++r)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[r][c] = 0.f;
  const __amdgpu_buffer_rsrc_t rw = rsrc_of(w);
  const uint32_t wrow = uint32_t(ldw), wv = uint32_t(k0) * wrow + cg * 8;
  const bool colok = cg * 8 < nvalid;  // columns past the matrix's last read nothing
  auto load = [&](u32x2_t (&v)[U], int b) {
#pragma unroll
    for (int i = 0; i < U; ++i)
      v[i] = (colok && b + i < R) ? bload<u32x2_t, kPolicyNT>(rw, wv, uint32_t(b + i) * wrow) : u32x2_t{0, 0};
  };
  auto consume = [&](const u32x2_t (&v)[U], int b) {
#pragma unroll
    for (int i = 0; i < U; ++i) {
      // rows past R hold zero codes; their LDS row index is clamped
      const int kr = min(b + i, R - 1);
      const u32x4_t xv = *reinterpret_cast<const u32x4_t*>(xs + (k0 - kbeg + kr) * kRowsChunk);
      float wf[8];
      widen8(v[i], wf);
#pragma unroll
      for (int r = 0; r < NT; ++r) {
        const float x = (r & 1) ? bf16_hi(xv[r / 2]) : bf16_lo(xv[r / 2]);
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[r][c] = fmaf(x, wf[c], acc[r][c]);
      }
    }
  };
  u32x2_t va[U], vb[U];
  load(va, 0);
  stage(xs, kbeg, kend);
  __syncthreads();
  for (int b = 0;;) {
    if (b + U < R) load(vb, b + U);
    consume(va, b);
    b += U;
    if (b >= R) break;
    if (b + U < R) load(va, b + U);
    consume(vb, b);
    b += U;
    if (b >= R) break;
  }
  return fold_rows<NT, NCOLS, 8>(acc, red);
}

// nvalid: columns of the unit inside the matrix (a unit may overhang its
// last columns: FP8 gate/up units are 128 columns, one 128-byte line per
// weight row, and I or D need not be a multiple of 128)
template <int NCOLS>
__device__ const float* unit8_x_rows(int nr, const uint8_t* w, int ldw, int kbeg, int kend, int nvalid,
                                     const bf16_t* const* act, bf16_t* xs, float* red) {
  if (nr <= 1) return unit8_direct<1, NCOLS>(w, ldw, kbeg, kend, nvalid, act, red);
  if (nr <= 2) return unit8_direct<2, NCOLS>(w, ldw, kbeg, kend, nvalid, act, red);
  const StageRows st{act};
  if (nr <= 4) return unit8_staged<4, NCOLS, 8>(w, ldw, kbeg, kend, nvalid, st, xs, red);
  return unit8_staged<8, NCOLS, 8>(w, ldw, kbeg, kend, nvalid, st, xs, red);
}

// ---------------------------------------------------------------------------
// routing, derived in the block
// ---------------------------------------------------------------------------

// ---------------------------------------------------------------------------
// gate/up
// ---------------------------------------------------------------------------

// DENSE: units (gate or up matrix, 64 columns, K-slice) over the T rows of x.
// Routed: units (ai-th active expert, ...) over the expert's rows, x gathered
// by token.  Writes fp32 partial pre-activations per K-slice, indexed by
// slot (routed) or token (dense).
template <bool DENSE, int NC = 64, bool W8 = false>
__device__ void gateup_unit(const StreamArgs& a, const Workspace& ws, int KS, int u) {
  const Shape& sh = a.sh;
  const int H = sh.H;
  const int N = DENSE ? sh.D : sh.I;
  const int per = ((N + NC - 1) / NC) * 2 * KS;  // units per expert (the last may overhang N)
  __shared__ int slot[kRouteSmallT];
  int grp = 0, rows = sh.T;
  if (!DENSE) {
    const ExpertRows er = expert_rows(sh, ws.topk_idx, u / per, slot);
    if (er.e < 0) return;
    grp = er.e;
    rows = er.rows;
    u %= per;
  }
  // u -> (n-block, matrix, K-slice), K-slice fastest
  // K-slices of whole 64-row groups (a thread's share of rows stays even)
  const int ks = u % KS;
  const int mat = (u / KS) & 1;
  const int n0 = (u / (2 * KS)) * NC;
  const int nvalid = min(NC, N - n0);
  const int g64 = H / 64;
  const int kbeg = (ks * g64 / KS) * 64, kend = ((ks + 1) * g64 / KS) * 64;
  const bf16_t* w = DENSE ? (mat ? a.du : a.dg) + n0 : (mat ? a.wu : a.wg) + (long long)grp * H * sh.I + n0;
  // FP8: codes of the same [K, N] matrix and its scale
  const Fp8Mat& Q = DENSE ? (mat ? a.qdu : a.qdg) : (mat ? a.qu : a.qg);
  const uint8_t* w8 = W8 ? Q.q + (DENSE ? 0 : (long long)grp * H * sh.I) + n0 : nullptr;
  const float qscale = W8 ? Q.tscale[DENSE ? 0 : grp] : 1.f;

  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  bf16_t* xs = reinterpret_cast<bf16_t*>(smem_raw);  // [kend-kbeg][8] staged rows
  float* red = reinterpret_cast<float*>(smem_raw);   // [5][8][NC]
  __shared__ const bf16_t* act[kRowsChunk];
  __shared__ float* dst[kRowsChunk];

  for (int c0 = 0; c0 < rows; c0 += kRowsChunk) {
    const int nr = min(kRowsChunk, rows - c0);
    if (threadIdx.x < kRowsChunk) {
      const int r = threadIdx.x;
      const int row = r < nr ? (DENSE ? c0 + r : slot[c0 + r]) : 0;
      act[r] = r < nr ? a.x + (long long)(DENSE ? row : row / sh.k) * H : nullptr;
      dst[r] = part_ptr(ws, sh, DENSE, ks, row, mat) + n0;
    }
    __syncthreads();
    const bf16_t* rowp[kRowsChunk];
#pragma unroll
    for (int r = 0; r < kRowsChunk; ++r) rowp[r] = act[r];
    if (W8) {
      const float* sums = unit8_x_rows<NC>(nr, w8, N, kbeg, kend, nvalid, rowp, xs, red);
      for (int o = threadIdx.x; o < nr * NC; o += kThreads)
        if (o % NC < nvalid) dst[o / NC][o % NC] = sums[o] * qscale;
    } else {
      const float* sums = unit_x_rows<NC>(nr, w, N, kbeg, kend, rowp, xs, red);
      for (int o = threadIdx.x; o < nr * NC; o += kThreads) dst[o / NC][o % NC] = sums[o];
    }
    __syncthreads();
  }
}

// Routed gate/up units.  (3 waves per SIMD: the register budget of 168
// holds every unit variant)
// Blocks [0, udn) are the dense units ud0 .. ud0 + udn - 1 (K-slices KSd),
// the rest the routed units.
template <bool W8>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 8))) void k_stream_gateup(
    StreamArgs a, Workspace ws, int KS, int ud0, int udn, int KSd) {
  const int b = blockIdx.x;
  if (b < udn)
    gateup_unit<true, W8 ? 128 : 64, W8>(a, ws, KSd, ud0 + b);
  else
    gateup_unit<false, W8 ? 128 : 64, W8>(a, ws, KS, b - udn);
}

// The router and dense gate/up units in one launch: blocks [0, nroute) are
// the router's (K-slice, token group) blocks, the rest are the first dense
// gate/up units.  The dense branch does not depend on the routing, so its
// weights stream while the router's few blocks wait on memory latency,
// with no second stream and no events.
template <int CW, bool W8>
__global__ __launch_bounds__(kThreads) void k_route_dense(
    StreamArgs a, const bf16_t* __restrict__ wr, const float* __restrict__ bias, Workspace ws, int slice_rows, int TB,
    int nslices, int nroute, int KSd) {
  const int b = blockIdx.x;
  if (b < nroute)
    route_slice<CW>(a.sh, slice_rows, TB, nslices, b % nslices, b / nslices, a.x, wr, bias, ws);
  else
    gateup_unit<true, W8 ? 128 : 64, W8>(a, ws, KSd, b - nroute);
}

// The dense gate/up units alone (a config without experts: no router to
// share the launch with), at the routed units' register budget.  NC = 256
// columns per unit when D allows: each row piece is then 512 contiguous
// bytes instead of 128, which a wide D (long rows) needs to stream well.
template <int NC, bool W8>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 8))) void k_dense_gateup(StreamArgs a,
                                                                                                     Workspace ws,
                                                                                                     int KSd) {
  gateup_unit<true, NC, W8>(a, ws, KSd, blockIdx.x);
}

// ---------------------------------------------------------------------------
// down
// ---------------------------------------------------------------------------

// GeGLU pass of the streamed rows where the down units do not form them
// (stream_fused_geglu false): h = gelu_tanh(sum G) * (sum U), K-slices in
// fixed order, bf16.  Items [0, n4r) are the T*k routed slot rows of
// ws.part into ws.h (slot order), items [n4r, n4r + n4d) the T dense token
// rows into ws.h_d.  4 columns per item.
__device__ __forceinline__ void geglu4(const Workspace& ws, const Shape& sh, bool dense, int KS, int row, int c,
                                       bf16_t* hout) {
  float4 g = make_float4(0.f, 0.f, 0.f, 0.f), up = g;
  for (int ks = 0; ks < KS; ++ks) {
    const float4 pg = *reinterpret_cast<const float4*>(part_ptr(ws, sh, dense, ks, row, 0) + c);
    const float4 pu = *reinterpret_cast<const float4*>(part_ptr(ws, sh, dense, ks, row, 1) + c);
    g.x += pg.x; g.y += pg.y; g.z += pg.z; g.w += pg.w;
    up.x += pu.x; up.y += pu.y; up.z += pu.z; up.w += pu.w;
  }
  *reinterpret_cast<u32x2_t*>(hout) = u32x2_t{pack_bf16x2(gelu_tanh(g.x) * up.x, gelu_tanh(g.y) * up.y),
                                              pack_bf16x2(gelu_tanh(g.z) * up.z, gelu_tanh(g.w) * up.w)};
}

__global__ __launch_bounds__(kThreads) void k_stream_geglu(Shape sh, Workspace ws, long long n4r, long long n4d,
                                                           int ksr) {
  const int qi = sh.I / 4, qd = sh.D / 4;
  const int ksd = dense_gateup_slices(sh);
  for (long long i = blockIdx.x * (long long)kThreads + threadIdx.x; i < n4r + n4d;
       i += (long long)gridDim.x * kThreads) {
    if (i < n4r) {
      const int row = int(i / qi), c = int(i % qi) * 4;
      geglu4(ws, sh, false, ksr, row, c, ws.h + (long long)row * sh.I + c);
    } else {
      const long long j = i - n4r;
      const int row = int(j / qd), c = int(j % qd) * 4;
      geglu4(ws, sh, true, ksd, row, c, ws.h_d + (long long)row * sh.D + c);
    }
  }
}

// GeGLU rows of a down unit, staged for unit_staged / unit8_staged:
// h[r][k] = bf16(gelu_tanh(G) * U) with G and U the sums of the gate/up
// K-slice partials in slice order, for the unit's rows r < nr and k in
// [kbeg, kend), written to xs[k - kbeg][8]; rows r >= nr are zero.  Rows
// are part rows: slot[c0 + r] (routed) or token c0 + r (dense).  With hout
// set (the first column unit of an expert or dense K-slice) the rows also
// go to hout[row * ldh + k], so a streamed forward's h can be read back.
struct StageGeglu {
  const Workspace* ws;
  const Shape* sh;
  bool dense;
  int KS;           // K-slices of the gate/up partials
  int nr, c0;
  const int* slot;  // routed: slot of each row of the expert (LDS)
  bf16_t* hout;
  int ldh;
  __device__ void operator()(bf16_t* xs, int kbeg, int kend) const {
    const int nq = (kend - kbeg) / 4;
#pragma unroll 1
    for (int c = threadIdx.x; c < nq; c += kThreads) {
      const int k = kbeg + 4 * c;
      uint32_t hv[kRowsChunk][2];
#pragma unroll
      for (int r = 0; r < kRowsChunk; ++r) {
        hv[r][0] = hv[r][1] = 0u;
        if (r < nr) {
          const int row = dense ? c0 + r : slot[c0 + r];
          float4 g = make_float4(0.f, 0.f, 0.f, 0.f), u = g;
          for (int ks = 0; ks < KS; ++ks) {
            const float4 pg = *reinterpret_cast<const float4*>(part_ptr(*ws, *sh, dense, ks, row, 0) + k);
            const float4 pu = *reinterpret_cast<const float4*>(part_ptr(*ws, *sh, dense, ks, row, 1) + k);
            g.x += pg.x; g.y += pg.y; g.z += pg.z; g.w += pg.w;
            u.x += pu.x; u.y += pu.y; u.z += pu.z; u.w += pu.w;
          }
          hv[r][0] = pack_bf16x2(gelu_tanh(g.x) * u.x, gelu_tanh(g.y) * u.y);
          hv[r][1] = pack_bf16x2(gelu_tanh(g.z) * u.z, gelu_tanh(g.w) * u.w);
          if (hout) *reinterpret_cast<u32x2_t*>(hout + (long long)row * ldh + k) = u32x2_t{hv[r][0], hv[r][1]};
        }
      }
      // k-major, the 8 rows of one k in 16 bytes
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x4_t v;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          v[q] = (j & 1) ? perm_hi16(hv[2 * q][j / 2], hv[2 * q + 1][j / 2])
                         : perm_lo16(hv[2 * q][j / 2], hv[2 * q + 1][j / 2]);
        *reinterpret_cast<u32x4_t*>(xs + (4 * c + j) * kRowsChunk) = v;
      }
    }
  }
};

// A down unit's rows (nr <= 8) against its weight columns, the rows staged
// in LDS by `st`.
template <int NCOLS, class Stage>
__device__ const float* unit_staged_rows(int nr, const bf16_t* w, int ldw, int kbeg, int kend, const Stage& st,
                                         bf16_t* xs, float* red) {
  if (nr <= 2) return unit_staged<2, NCOLS, 8, 8>(w, ldw, kbeg, kend, st, xs, red);
  if (nr <= 4) return unit_staged<4, NCOLS, 8, 8>(w, ldw, kbeg, kend, st, xs, red);
  return unit_staged<8, NCOLS, 8, 4>(w, ldw, kbeg, kend, st, xs, red);
}
template <int NCOLS, class Stage>
__device__ const float* unit8_staged_rows(int nr, const uint8_t* w, int ldw, int kbeg, int kend, int nvalid,
                                          const Stage& st, bf16_t* xs, float* red) {
  if (nr <= 2) return unit8_staged<2, NCOLS, 8>(w, ldw, kbeg, kend, nvalid, st, xs, red);
  if (nr <= 4) return unit8_staged<4, NCOLS, 8>(w, ldw, kbeg, kend, nvalid, st, xs, red);
  return unit8_staged<8, NCOLS, 8>(w, ldw, kbeg, kend, nvalid, st, xs, red);
}

// Down units.  DENSE: unit u = (128 columns, K-slice of whole 64-row groups
// of D) over the T rows of h_d, fp32 partial outputs per slice (summed by
// the combine).  Routed: unit u = (ai-th active expert, 128 columns) over
// the expert's rows of h (slot order), bf16 output rows y indexed by slot.
// The rows of h / h_d are formed in the unit from the gate/up partials
// (StageGeglu): no separate GeGLU launch.
template <bool DENSE, int NC, bool W8, bool FUSED>
__device__ void down_unit(const StreamArgs& a, const Workspace& ws, int u) {
  const Shape& sh = a.sh;
  const int H = sh.H;
  const int nblk = H / NC;  // NC: output columns of a unit
  __shared__ int slot[kRouteSmallT];
  int grp = 0, rows = sh.T, kbeg = 0, kend = sh.I, ksd = 0;
  if (DENSE) {
    const int g64 = sh.D / 64, KS = dense_down_slices(sh);
    ksd = u % KS;
    u /= KS;
    kbeg = (ksd * g64 / KS) * 64;
    kend = ((ksd + 1) * g64 / KS) * 64;
  } else {
    const ExpertRows er = expert_rows(sh, ws.topk_idx, u / nblk, slot);
    if (er.e < 0) return;
    grp = er.e;
    rows = er.rows;
    u %= nblk;
  }
  const int n0 = u * NC;
  const int K = DENSE ? sh.D : sh.I;  // row length of h_d / h
  const bf16_t* wd = (DENSE ? a.dd : a.wd + (long long)grp * sh.I * H) + n0;
  const Fp8Mat& Q = DENSE ? a.qdd : a.qd;
  const uint8_t* w8 = W8 ? Q.q + (DENSE ? 0 : (long long)grp * sh.I * H) + n0 : nullptr;
  const float qscale = W8 ? Q.tscale[DENSE ? 0 : grp] : 1.f;

  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  bf16_t* hs = reinterpret_cast<bf16_t*>(smem_raw);  // [kend-kbeg][8] staged rows
  float* red = reinterpret_cast<float*>(smem_raw);   // [5][8][NC]
  // K-slices of the gate/up partials behind h / h_d
  const int ksg = DENSE ? dense_gateup_slices(sh) : (W8 ? kStreamKS8 : kStreamKS);
  bf16_t* hout = u == 0 ? (DENSE ? ws.h_d : ws.h) : nullptr;
  for (int c0 = 0; c0 < rows; c0 += kRowsChunk) {
    const int nr = min(kRowsChunk, rows - c0);
    const float* sums;
    if (!FUSED) {  // the rows of h / h_d from k_stream_geglu
      const bf16_t* rowp[kRowsChunk];
#pragma unroll
      for (int r = 0; r < kRowsChunk; ++r)
        rowp[r] = r < nr ? (DENSE ? ws.h_d : ws.h) + (long long)(DENSE ? c0 + r : slot[c0 + r]) * K : nullptr;
      sums = W8 ? unit8_x_rows<NC>(nr, w8, H, kbeg, kend, NC, rowp, hs, red)
                : unit_x_rows<NC>(nr, wd, H, kbeg, kend, rowp, hs, red);
    } else {
      const StageGeglu st{&ws, &sh, DENSE, ksg, nr, c0, slot, hout, K};
      sums = W8 ? unit8_staged_rows<NC>(nr, w8, H, kbeg, kend, NC, st, hs, red)
                : unit_staged_rows<NC>(nr, wd, H, kbeg, kend, st, hs, red);
    }
    if (DENSE) {
      float* o = ws.ydp + ((long long)ksd * kRouteSmallT + c0) * H + n0;
      for (int i = threadIdx.x; i < nr * NC; i += kThreads) o[(long long)(i / NC) * H + (i % NC)] = sums[i] * qscale;
    } else {
      for (int i = threadIdx.x; i < nr * NC; i += kThreads)
        ws.y[(long long)slot[c0 + i / NC] * H + n0 + (i % NC)] = (bf16_t)f32_to_bf16_bits(sums[i] * qscale);
    }
    __syncthreads();
  }
}

// One launch for the dense down units (blocks [0, ud)) and the routed ones.
// FUSED (stream_fused_geglu): the units form their GeGLU rows from the
// gate/up partials; otherwise they read the rows k_stream_geglu wrote.
template <bool W8, bool FUSED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3, 8))) void k_stream_down(StreamArgs a,
                                                                                                    Workspace ws,
                                                                                                    int ud) {
  const int u = blockIdx.x;
  if (u < ud)
    down_unit<true, kDenseDownCols, W8, FUSED>(a, ws, u);
  else
    down_unit<false, kDownCols, W8, FUSED>(a, ws, u - ud);
}

// h and y rows of the last streamed forward (slot order) copied to grouped
// (perm) order: block b handles slot b.  Diagnostic only.
__global__ __launch_bounds__(kThreads) void k_stream_export(Shape sh, Workspace ws, bf16_t* h_rows, bf16_t* y_rows) {
  const int b = blockIdx.x;
  const int p = ws.pos[b];
  if (h_rows)
    for (int c = threadIdx.x; c < sh.I; c += kThreads) h_rows[(long long)p * sh.I + c] = ws.h[(long long)b * sh.I + c];
  if (y_rows)
    for (int c = threadIdx.x; c < sh.H; c += kThreads) y_rows[(long long)p * sh.H + c] = ws.y[(long long)b * sh.H + c];
}

}  // namespace

namespace {
// The dense gate/up units of a config with experts (64 columns, FP8 128:
// one 128-byte line per weight row), and how many the router's launch takes.
struct DenseSplit {
  int ksd, nc, ud, in_route;
};
DenseSplit dense_split(const StreamArgs& a) {
  const Shape& sh = a.sh;
  DenseSplit d{};
  d.ksd = sh.D > 0 ? dense_gateup_slices(sh) : 1;
  d.nc = a.fp8 ? 128 : 64;
  d.ud = sh.D > 0 ? ((sh.D + d.nc - 1) / d.nc) * 2 * d.ksd : 0;
  d.in_route = a.fp8 ? d.ud : d.ud * kDenseRouteEighths / 8;
  return d;
}
}  // namespace

hipError_t launch_stream_gateup(const StreamArgs& a, const Workspace& ws, hipStream_t s) {
  const Shape& sh = a.sh;
  if (sh.T == 0 || sh.E == 0) return hipSuccess;
  const int ks = a.fp8 ? kStreamKS8 : kStreamKS;
  const int nc = a.fp8 ? 128 : 64;  // unit columns (gateup_unit's NC)
  const DenseSplit d = dense_split(a);
  const int udn = d.ud - d.in_route;  // dense units left to this launch
  const size_t kl = size_t((sh.H / 64 + ks - 1) / ks) * 64;  // longest slice
  const size_t kld = udn ? size_t((sh.H / 64 + d.ksd - 1) / d.ksd) * 64 : 0;
  const size_t lds = std::max(std::max(kl, kld) * kRowsChunk * 2, size_t(5) * kRowsChunk * nc * 4);
  const int max_active = std::min(sh.E, sh.T * sh.k);
  const dim3 grid(udn + max_active * ((sh.I + nc - 1) / nc) * 2 * ks);
  if (a.fp8)
    hipLaunchKernelGGL(k_stream_gateup<true>, grid, dim3(kThreads), lds, s, a, ws, ks, d.in_route, udn, d.ksd);
  else
    hipLaunchKernelGGL(k_stream_gateup<false>, grid, dim3(kThreads), lds, s, a, ws, ks, d.in_route, udn, d.ksd);
  return hipGetLastError();
}

hipError_t launch_route_dense(const StreamArgs& a, const bf16_t* wr, const float* bias, const Workspace& ws,
                              hipStream_t s) {
  const Shape& sh = a.sh;
  if (sh.T == 0) return hipSuccess;
  // a dense FFN (no experts) launches the dense units only
  const RouteSmallCfg c = sh.E > 0 ? route_small_config(sh) : RouteSmallCfg{};
  if (sh.E > 0 && !c.ok) return hipErrorInvalidValue;
  const int nroute = sh.E > 0 ? c.nslices * c.groups : 0;
  const int ksd = sh.D > 0 ? dense_gateup_slices(sh) : 1;
  const bool w8 = a.fp8;
  // dense unit columns: beside the router those of dense_split (this launch
  // runs its first in_route units); without experts 256 when D allows
  const bool wide = nroute == 0 && sh.D % kDenseOnlyCols == 0;
  const int nc = wide ? kDenseOnlyCols : (w8 ? 128 : 64);
  const int ud = sh.D == 0 ? 0 : nroute > 0 ? dense_split(a).in_route : ((sh.D + nc - 1) / nc) * 2 * ksd;
  const size_t kl = size_t((sh.H / 64 + ksd - 1) / ksd) * 64;  // longest dense K-slice
  const size_t lds = ud ? std::max(kl * kRowsChunk * 2, size_t(5) * kRowsChunk * nc * 4) : 0;
  if (nroute + ud == 0) return hipSuccess;
  if (wide) {
    if (w8)
      hipLaunchKernelGGL((k_dense_gateup<kDenseOnlyCols, true>), dim3(ud), dim3(kThreads), lds, s, a, ws, ksd);
    else
      hipLaunchKernelGGL((k_dense_gateup<kDenseOnlyCols, false>), dim3(ud), dim3(kThreads), lds, s, a, ws, ksd);
  } else if (nroute == 0) {
    if (w8)
      hipLaunchKernelGGL((k_dense_gateup<128, true>), dim3(ud), dim3(kThreads), lds, s, a, ws, ksd);
    else
      hipLaunchKernelGGL((k_dense_gateup<64, false>), dim3(ud), dim3(kThreads), lds, s, a, ws, ksd);
  } else {
    const dim3 grid(nroute + ud);
    if (c.cw != 4 && w8)
      hipLaunchKernelGGL((k_route_dense<8, true>), grid, dim3(kThreads), lds, s, a, wr, bias, ws, c.slice_rows, c.tb,
                         c.nslices, nroute, ksd);
    else if (c.cw != 4)
      hipLaunchKernelGGL((k_route_dense<8, false>), grid, dim3(kThreads), lds, s, a, wr, bias, ws, c.slice_rows, c.tb,
                         c.nslices, nroute, ksd);
    else if (w8)
      hipLaunchKernelGGL((k_route_dense<4, true>), grid, dim3(kThreads), lds, s, a, wr, bias, ws, c.slice_rows, c.tb,
                         c.nslices, nroute, ksd);
    else
      hipLaunchKernelGGL((k_route_dense<4, false>), grid, dim3(kThreads), lds, s, a, wr, bias, ws, c.slice_rows, c.tb,
                         c.nslices, nroute, ksd);
  }
  return hipGetLastError();
}

hipError_t launch_stream_geglu(const StreamArgs& a, const Workspace& ws, hipStream_t s) {
  const Shape& sh = a.sh;
  if (sh.T == 0 || stream_fused_geglu(sh, a.fp8)) return hipSuccess;  // the down units form the rows
  const long long n4r = sh.E > 0 ? (long long)sh.T * sh.k * sh.I / 4 : 0;
  const long long n4d = sh.D > 0 ? (long long)sh.T * sh.D / 4 : 0;
  const int gblocks = int(std::min<long long>(1024, (n4r + n4d + kThreads - 1) / kThreads));
  if (gblocks == 0) return hipSuccess;
  hipLaunchKernelGGL(k_stream_geglu, dim3(gblocks), dim3(kThreads), 0, s, sh, ws, n4r, n4d,
                     a.fp8 ? kStreamKS8 : kStreamKS);
  return hipGetLastError();
}

hipError_t launch_stream_down(const StreamArgs& a, const Workspace& ws, hipStream_t s) {
  const Shape& sh = a.sh;
  if (sh.T == 0) return hipSuccess;
  const int nblk = sh.H / kDownCols;
  const int ksd = sh.D > 0 ? dense_down_slices(sh) : 1;
  const int ud = sh.D > 0 ? (sh.H / kDenseDownCols) * ksd : 0;
  const int max_active = std::min(sh.E, sh.T * sh.k);
  const bool fused = stream_fused_geglu(sh, a.fp8);  // else k_stream_geglu formed h / h_d
  // longest K run of a unit: a dense K-slice or the expert width
  const int kd = ud ? (sh.D / 64 + ksd - 1) / ksd * 64 : 0;
  const size_t lds = std::max(size_t(std::max(sh.I, kd)) * kRowsChunk * 2, size_t(5) * kRowsChunk * kDownColsMax * 4);
  const dim3 grid(ud + max_active * nblk);
  if (a.fp8)  // FP8 down units read the rows k_stream_geglu wrote (stream_fused_geglu)
    hipLaunchKernelGGL((k_stream_down<true, false>), grid, dim3(kThreads), lds, s, a, ws, ud);
  else if (fused)
    hipLaunchKernelGGL((k_stream_down<false, true>), grid, dim3(kThreads), lds, s, a, ws, ud);
  else
    hipLaunchKernelGGL((k_stream_down<false, false>), grid, dim3(kThreads), lds, s, a, ws, ud);
  return hipGetLastError();
}

hipError_t launch_stream_export(const Shape& sh, const Workspace& ws, bf16_t* h_rows, bf16_t* y_rows, hipStream_t s) {
  const int blocks = sh.T * sh.k;
  if (blocks == 0 || (!h_rows && !y_rows)) return hipSuccess;
  hipLaunchKernelGGL(k_stream_export, dim3(blocks), dim3(kThreads), 0, s, sh, ws, h_rows, y_rows);
  return hipGetLastError();
}

}  // namespace moe
