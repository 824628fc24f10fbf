// Weight-streaming GEMMs of the MoE block with NVFP4 weights, for few tokens
// (T <= 64; decode).
//
// NVFP4 checkpoint config, quantization_config group_0.weights: e2m1 values
// two per byte (lower k in the low nibble), groups of 16 along K with
// float8_e4m3fn scales, one fp32 tensor scale per matrix; out-major storage,
// [N][K/2] codes and [N][K/16] scales.  At T = 8 every selected expert sees
// one or two tokens, so each weight feeds a couple of FMAs and the layer is
// bound by the bytes of the packed weights (0.5625 per weight).  These
// kernels stream them at full width instead of running MFMA tiles that are
// 1-8 rows full:
//
//   lane = (column, chunk lane l in 0..7): it reads the 16 code bytes of
//   k-chunk q = 8 j + l (32 k) of its column for j = 0, 1, ..., so the 8
//   lanes of a column read 128 contiguous bytes per load instruction and a
//   wave instruction touches 8 whole cache lines; beside them the dword that
//   holds the chunk's two group scales.  Loads are buffer loads from the
//   wave's matrix with the chunk's offset uniform; a chunk past K or a
//   column past N gets an offset out of the buffer's range (zeros).
//
//   The codes are converted to bf16 pairs with the gfx950 e2m1 conversion
//   (unit scale: exact), multiplied into the activation pairs with the bf16
//   dot2 instruction (fp32 accumulate) one 16-k group at a time, and each
//   group's sum is scaled by its e4m3 scale: sum_g s_g (sum_k q_k x_k) is the
//   dequantised product in a different rounding order.  The tensor scale
//   (and the activations' global scale for W4A4) multiplies the column sums.
//
//   A wave streams its unit's column groups in steps of a few chunks per
//   lane (2 for gate/up, 1 for down), the next step's loads in flight while
//   the current one is computed.  Activation rows are staged in LDS, 4 per
//   pass (rows past 4 take another pass over the unit); the lanes of one
//   chunk read the same bytes.  Units are small so that many blocks share
//   each CU: the decode and the dot products are VALU work of the same order
//   as the loads, and only enough resident waves overlap the two (units of
//   16 gate/up columns measured faster than units of 64 that share the
//   per-block set-up, 35 against 56 us at T = 8).
//
//   gate/up (k_fs4_gateup): a unit is (expert or dense branch, 16 output
//     columns); waves 0-1 read the gate matrix and waves 2-3 the up matrix,
//     8 columns each.  The column sums meet in LDS, where
//     h = bf16(gelu_tanh(G) * U) is formed and written: no partial sums in
//     HBM and no separate GeGLU pass.
//   down (k_fs4_down): routed units are (expert, 64 columns), dense units 32
//     columns over the longer K; output rows y (slot order) and y_d in bf16,
//     summed by the combine kernel.
//
// Routed units derive their expert's rows from topk_idx themselves (no
// grouping kernels), as the bf16 streaming kernels do; rows are slots
// s = t * k + j.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "route_dev.h"

namespace moe {

namespace {

constexpr int kFsThreads = 256;
constexpr int kPolicyNT = 2;  // nontemporal: the weights are read once
constexpr int kFsRows = 4;  // activation rows per pass
// gate/up: a step is kGuJB chunks of the lane's column; a group is 8
// columns per wave, 16 per block (waves 0-1 gate, 2-3 up, same columns); a
// unit is kGuGroups groups
constexpr int kGuJB = 2;
constexpr int kGuGroups = 1;
constexpr int kGuUnitCols = 16 * kGuGroups;
constexpr int kGuDepth = 2;  // steps in the register ring
// down: a step is kDnJB chunks of each of the lane's kDnNC columns; a group
// is 8 kDnNC columns per wave (32 kDnNC per block); routed units are
// kDnGroups groups, dense units (K = D, three times longer here) kDdGroups
constexpr int kDnJB = 1;
constexpr int kDnNC = 1;
constexpr int kDnGroups = 2;
constexpr int kDdGroups = 1;
constexpr int kDnGroupCols = 32 * kDnNC;
constexpr int kDnDepth = 2;

// Stage rows [c0, c0 + nr) of the activation matrix into xs[r][0..K) (bf16):
// row r is src + idx(r) * ld.  16 bytes per thread per step.
template <class Idx>
__device__ __forceinline__ void stage_rows(bf16_t* xs, const bf16_t* __restrict__ src, long long ld, int K, int nr,
                                           const Idx& idx) {
  const int per = K / 8;  // 16-byte pieces per row
  for (int i = threadIdx.x; i < nr * per; i += kFsThreads) {
    const int r = i / per, p = i - r * per;
    const u32x4_t v = *reinterpret_cast<const u32x4_t*>(src + idx(r) * ld + p * 8);
    *reinterpret_cast<u32x4_t*>(xs + r * K + p * 8) = v;
  }
}

// A dword as a bf16 pair.  Taken by value: a bit cast written directly on a
// vector element (v[i]) compiles to a read of element 0 with this compiler.
__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2_t, v); }

// acc[m][r] += the lane's chunk of column m (e2m1 codes cq[m], scales sd[m])
// times the staged rows' 32 values at xq + r K (xq: the chunk's first value
// in row 0), r < NR.  sd[m]: the dword holding the chunk's two scales in its
// half odd (the chunk's parity).  The chunk of each staged row is read once
// and serves every column.
template <int NC, int NR>
__device__ __forceinline__ void chunk_dot(float (&acc)[NC][NR], const u32x4_t (&cq)[NC], const uint32_t (&sd)[NC],
                                          int odd, const bf16_t* xq, int K) {
  f32x2_t s[NC];
  bf16x2_t w[NC][16];
#pragma unroll
  for (int m = 0; m < NC; ++m) {
    s[m] = __builtin_amdgcn_cvt_pk_f32_fp8(int(sd[m] >> (16 * odd)), false);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      w[m][4 * d + 0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cq[m][d], 1.0f, 0);
      w[m][4 * d + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cq[m][d], 1.0f, 1);
      w[m][4 * d + 2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cq[m][d], 1.0f, 2);
      w[m][4 * d + 3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cq[m][d], 1.0f, 3);
    }
  }
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const u32x4_t* xp = reinterpret_cast<const u32x4_t*>(xq + r * K);
    const u32x4_t x0 = xp[0], x1 = xp[1], x2 = xp[2], x3 = xp[3];
#pragma unroll
    for (int m = 0; m < NC; ++m) {
      float g0 = 0.f, g1 = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        g0 = __builtin_amdgcn_fdot2_f32_bf16(w[m][i], as_bf16x2(x0[i]), g0, false);
        g1 = __builtin_amdgcn_fdot2_f32_bf16(w[m][8 + i], as_bf16x2(x2[i]), g1, false);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        g0 = __builtin_amdgcn_fdot2_f32_bf16(w[m][4 + i], as_bf16x2(x1[i]), g0, false);
        g1 = __builtin_amdgcn_fdot2_f32_bf16(w[m][12 + i], as_bf16x2(x3[i]), g1, false);
      }
      acc[m][r] = fmaf(s[m].x, g0, acc[m][r]);
      acc[m][r] = fmaf(s[m].y, g1, acc[m][r]);
    }
  }
}

// ---------------------------------------------------------------------------
// The step pipeline of both kernels.  A wave streams the G column groups of
// its unit; a group takes nb = ceil(nj / JB) steps of JB chunk loads per
// column (nj = ceil(nq / 8) chunks per lane, nq = K / 32).  The loads of
// step s + 1 are issued before step s is computed.  Every load is issued:
// chunks past K and columns past N are clamped onto valid bytes and their
// offsets out of the buffer range (no access, zeros), so the wait counts are
// the same on every path and the next step's loads stay in flight; a step
// past the last repeats it (discarded).
// Group sums go to LDS (outs), so no global store sits inside the pipeline.
// ---------------------------------------------------------------------------

template <int NC, int JB>
struct StepBuf {
  u32x4_t c[JB][NC];
  uint32_t s[JB][NC];
};

constexpr uint32_t kOutOfRange = 0x80000000u;  // past every buffer resource's range: no access, zeros

// Col(g, m, ok): the lane's m-th column of group g within the matrix, and
// whether it exists.  rq / rs: the matrix's codes and scales (wave-uniform).
// Chunk jj of a step lies 128 jj bytes (codes) and 16 jj bytes (scales) past
// the lane's first chunk: a uniform offset.
template <int NC, int JB, class Col>
__device__ __forceinline__ void issue_step(StepBuf<NC, JB>& B, __amdgpu_buffer_rsrc_t rq, __amdgpu_buffer_rsrc_t rs,
                                           int K, int nq, int nb, int step, int l, const Col& col) {
  const int g = step / nb, b = step - g * nb;
#pragma unroll
  for (int m = 0; m < NC; ++m) {
    bool ok;
    const uint32_t n = uint32_t(col(g, m, ok));
    const uint32_t lc = n * uint32_t(K / 2) + 16u * uint32_t(l);
    const uint32_t ls = n * uint32_t(K / 16) + 4u * uint32_t(l >> 1);
#pragma unroll
    for (int j = 0; j < JB; ++j) {
      const int jj = b * JB + j;
      const bool v = ok && l < nq - 8 * jj;  // chunk 8 jj + l exists
      B.c[j][m] = bload<u32x4_t, kPolicyNT>(rq, v ? lc : kOutOfRange, uint32_t(128 * jj));
      B.s[j][m] = bload<uint32_t, kPolicyNT>(rs, v ? ls : kOutOfRange, uint32_t(16 * jj));
    }
  }
}

template <int NC, int JB, int NR>
__device__ __forceinline__ void compute_step(float (&acc)[NC][NR], const StepBuf<NC, JB>& B, int nq, int nb, int step,
                                             int l, const bf16_t* xs, int K) {
  const int b = step % nb;
#pragma unroll
  for (int j = 0; j < JB; ++j) {
    const int q = 8 * (b * JB + j) + l;
    chunk_dot<NC, NR>(acc, B.c[j], B.s[j], l & 1, xs + 32 * (q < nq ? q : 0), K);
  }
}

// f(integral_constant<0>) .. f(integral_constant<N - 1>), in order
template <int N, class F>
__device__ __forceinline__ void static_for(const F& f) {
  if constexpr (N > 0) {
    static_for<N - 1>(f);
    f(std::integral_constant<int, N - 1>{});
  }
}

// Runs the steps of one row pass, DEPTH - 1 steps' loads in flight ahead of
// the one computed (a ring of DEPTH register buffers): stage() stages the
// pass's rows into xs after the first loads are issued, and emit(g, acc)
// receives each group's sums (per lane, not yet folded over the chunk
// lanes).  The loop runs whole rounds of DEPTH steps and issues a step's
// loads in every slot (past the last step, the last one again, unused).
template <int NC, int JB, int NR, int DEPTH, class Col, class Stage, class Emit>
__device__ __forceinline__ void run_steps(__amdgpu_buffer_rsrc_t rq, __amdgpu_buffer_rsrc_t rs, int K, int G,
                                          const bf16_t* xs, const Col& col, const Stage& stage, const Emit& emit) {
  const int l = threadIdx.x & 7;
  const int nq = K / 32, nj = (nq + 7) / 8, nb = (nj + JB - 1) / JB;
  const int S = G * nb;
  float acc[NC][NR];
#pragma unroll
  for (int m = 0; m < NC; ++m)
#pragma unroll
    for (int r = 0; r < NR; ++r) acc[m][r] = 0.f;
  StepBuf<NC, JB> buf[DEPTH];
  static_for<DEPTH - 1>([&](auto ic) {
    constexpr int I = decltype(ic)::value;
    issue_step(buf[I], rq, rs, K, nq, nb, min(I, S - 1), l, col);
  });
  stage();
  __syncthreads();
  for (int s0 = 0; s0 < S; s0 += DEPTH) {
    static_for<DEPTH>([&](auto ic) {
      constexpr int I = decltype(ic)::value;
      const int s = s0 + I;
      issue_step(buf[(I + DEPTH - 1) % DEPTH], rq, rs, K, nq, nb, min(s + DEPTH - 1, S - 1), l, col);
      if (s < S) {
        compute_step<NC, JB, NR>(acc, buf[I], nq, nb, s, l, xs, K);
        if (s % nb == nb - 1) {
          emit(s / nb, acc);
#pragma unroll
          for (int m = 0; m < NC; ++m)
#pragma unroll
            for (int r = 0; r < NR; ++r) acc[m][r] = 0.f;
        }
      }
    });
  }
}

// f(integral_constant<nr>): the row count of a pass (1 .. 4) is a template
// parameter, so the row loops are branch-free.
template <class F>
__device__ __forceinline__ void with_rows(int nr, const F& f) {
  static_assert(kFsRows == 4, "row classes 1 .. 4");
  if (nr == 1)
    f(std::integral_constant<int, 1>{});
  else if (nr == 2)
    f(std::integral_constant<int, 2>{});
  else if (nr == 3)
    f(std::integral_constant<int, 3>{});
  else
    f(std::integral_constant<int, 4>{});
}

// Sum over the 8 chunk lanes of a column (lanes 8 c .. 8 c + 7).
__device__ __forceinline__ float fold8(float v) {
  v += __shfl_xor(v, 1, kWave);
  v += __shfl_xor(v, 2, kWave);
  v += __shfl_xor(v, 4, kWave);
  return v;
}

// ---------------------------------------------------------------------------
// gate/up
// ---------------------------------------------------------------------------

// Blocks [0, ud) are dense units, the rest routed: unit u of the ai-th active
// expert, ai = u / units_per_expert.  A unit is kGuUnitCols output columns;
// waves 0-1 read the gate matrix and waves 2-3 the up matrix, group g of
// wave w holding columns 16 g + 8 (w & 1) .. + 7 of the unit (lane column
// c = lane / 8).  The column sums meet in LDS for the GeGLU.
__global__ __launch_bounds__(kFsThreads) __attribute__((amdgpu_waves_per_eu(5, 8))) void k_fs4_gateup(StreamArgs a, Workspace ws, int ud) {
  const Shape& sh = a.sh;
  const int K = sh.H;
  __shared__ int slot[kRouteSmallT];
  __shared__ float gs[2][kFsRows][kGuUnitCols];  // gate / up column sums of a pass (tensor scale applied)
  extern __shared__ __attribute__((aligned(16))) unsigned char fs_smem[];
  bf16_t* xs = reinterpret_cast<bf16_t*>(fs_smem);  // [kFsRows][K]
  const bool dense = int(blockIdx.x) < ud;
  int grp = 0, rows = sh.T, cb = blockIdx.x, N = sh.D;
  if (!dense) {
    N = sh.I;
    const int per = (N + kGuUnitCols - 1) / kGuUnitCols;
    const ExpertRows er = expert_rows(sh, ws.topk_idx, (int(blockIdx.x) - ud) / per, slot);
    if (er.e < 0) return;
    grp = er.e;
    rows = er.rows;
    cb = (int(blockIdx.x) - ud) % per;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int mi = wave >> 1, wm = wave & 1, l = lane & 7, c = lane >> 3;
  const int n0 = cb * kGuUnitCols;
  const Fp4Mat M = dense ? (mi ? a.fdu : a.fdg) : (mi ? a.fu : a.fg);  // wave-uniform
  const long long mat = dense ? 0 : (long long)grp * N;                // first column row of the expert's matrix
  const __amdgpu_buffer_rsrc_t rq = rsrc_of(uniform_ptr(M.q + mat * (K / 2)));
  const __amdgpu_buffer_rsrc_t rs = rsrc_of(uniform_ptr(M.scale + mat * (K / 16)));
  const float ts = (dense ? M.tscale[0] : M.tscale[grp]) * (a.in_scale ? a.in_scale[0] : 1.f);
  bf16_t* hout = dense ? ws.h_d : ws.h;
  const int ldh = dense ? sh.D : sh.I;
  const int ncols = min(kGuUnitCols, N - n0);

  for (int c0 = 0; c0 < rows; c0 += kFsRows) {
    const int nr = min(kFsRows, rows - c0);
    auto col = [&](int g, int, bool& ok) {
      const int n = n0 + 16 * g + 8 * wm + c;
      ok = n < N;
      return n;
    };
    auto stage = [&]() {
      if (dense)
        stage_rows(xs, a.x, K, K, nr, [&](int r) { return (long long)(c0 + r); });
      else
        stage_rows(xs, a.x, K, K, nr, [&](int r) { return (long long)(slot[c0 + r] / sh.k); });
    };
    auto emit = [&](int g, auto& acc) {
      constexpr int NR = sizeof(acc[0]) / sizeof(float);
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const float v = fold8(acc[0][r]) * ts;
        if (l == r && r < nr) gs[mi][r][16 * g + 8 * wm + c] = v;
      }
    };
    with_rows(nr, [&](auto nrc) { run_steps<1, kGuJB, decltype(nrc)::value, kGuDepth>(rq, rs, K, kGuGroups, xs, col, stage, emit); });
    __syncthreads();  // gs complete; xs free
    for (int i = threadIdx.x; i < nr * ncols; i += kFsThreads) {
      const int r = i / ncols, cc = i - r * ncols;
      const int row = dense ? c0 + r : slot[c0 + r];
      hout[(long long)row * ldh + n0 + cc] = bf16_t(f32_to_bf16_bits(gelu_tanh(gs[0][r][cc]) * gs[1][r][cc]));
    }
    __syncthreads();  // gs is rewritten by the next pass
  }
}

// ---------------------------------------------------------------------------
// down
// ---------------------------------------------------------------------------

// Unit of G groups from column n0 (a group: kDnGroupCols columns, wave w's
// part 8 kDnNC w .. + 8 kDnNC - 1, lane column 8 m + c of it); rows
// src[idx(r)] of length K; output rows out[idx(r)] of length N (bf16).
template <class Idx>
__device__ __forceinline__ void down_unit(const Fp4Mat& M, long long mat, int K, int N, int n0, int G, float ts,
                                          const bf16_t* __restrict__ src, int rows, const Idx& idx,
                                          bf16_t* __restrict__ out, bf16_t* xs, bf16_t (*ys)[kDnGroupCols * kDnGroups]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l = lane & 7, c = lane >> 3;
  const int ncols = min(kDnGroupCols * G, N - n0);
  const __amdgpu_buffer_rsrc_t rq = rsrc_of(uniform_ptr(M.q + mat * (K / 2)));
  const __amdgpu_buffer_rsrc_t rs = rsrc_of(uniform_ptr(M.scale + mat * (K / 16)));
  for (int c0 = 0; c0 < rows; c0 += kFsRows) {
    const int nr = min(kFsRows, rows - c0);
    auto col = [&](int g, int m, bool& ok) {
      const int n = n0 + kDnGroupCols * g + 8 * kDnNC * wave + 8 * m + c;
      ok = n < N;
      return n;
    };
    auto stage = [&]() { stage_rows(xs, src, K, K, nr, [&](int r) { return (long long)idx(c0 + r); }); };
    auto emit = [&](int g, auto& acc) {
      constexpr int NR = sizeof(acc[0]) / sizeof(float);
#pragma unroll
      for (int m = 0; m < kDnNC; ++m)
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          const float v = fold8(acc[m][r]) * ts;
          if (l == r && r < nr) ys[r][kDnGroupCols * g + 8 * kDnNC * wave + 8 * m + c] = bf16_t(f32_to_bf16_bits(v));
        }
    };
    with_rows(nr, [&](auto nrc) { run_steps<kDnNC, kDnJB, decltype(nrc)::value, kDnDepth>(rq, rs, K, G, xs, col, stage, emit); });
    __syncthreads();
    for (int i = threadIdx.x; i < nr * ncols; i += kFsThreads) {
      const int r = i / ncols, cc = i - r * ncols;
      out[(long long)idx(c0 + r) * N + n0 + cc] = ys[r][cc];
    }
    __syncthreads();
  }
}

// Blocks [0, ud) are dense units (kDdGroups groups), the rest routed units
// (kDnGroups groups of the ai-th active expert).
__global__ __launch_bounds__(kFsThreads) __attribute__((amdgpu_waves_per_eu(4, 8))) void k_fs4_down(StreamArgs a, Workspace ws, int ud) {
  const Shape& sh = a.sh;
  __shared__ int slot[kRouteSmallT];
  __shared__ bf16_t ys[kFsRows][kDnGroupCols * kDnGroups];
  extern __shared__ __attribute__((aligned(16))) unsigned char fs_smem[];
  bf16_t* xs = reinterpret_cast<bf16_t*>(fs_smem);  // [kFsRows][K]
  if (int(blockIdx.x) < ud) {
    const float ts = a.fdd.tscale[0] * (a.in_scale ? a.in_scale[2] : 1.f);
    down_unit(a.fdd, 0, sh.D, sh.H, int(blockIdx.x) * kDnGroupCols * kDdGroups, kDdGroups, ts, ws.h_d, sh.T,
              [](int r) { return r; }, ws.y_d, xs, ys);
    return;
  }
  const int per = (sh.H + kDnGroupCols * kDnGroups - 1) / (kDnGroupCols * kDnGroups);
  const int u = int(blockIdx.x) - ud;
  const ExpertRows er = expert_rows(sh, ws.topk_idx, u / per, slot);
  if (er.e < 0) return;
  const float ts = a.fd.tscale[er.e] * (a.in_scale ? a.in_scale[1] : 1.f);
  down_unit(a.fd, (long long)er.e * sh.H, sh.I, sh.H, (u % per) * kDnGroupCols * kDnGroups, kDnGroups, ts, ws.h,
            er.rows, [&](int r) { return slot[r]; }, ws.y, xs, ys);
}

}  // namespace

bool fp4_stream_fits(const Shape& sh) {
  auto ok_k = [](int K) { return K % 64 == 0 && K <= 3072; };  // 8 staged rows of K in LDS
  if (sh.T > kRouteSmallT || !ok_k(sh.H)) return false;
  if (sh.E > 0 && (sh.E > 256 || !ok_k(sh.I))) return false;
  if (sh.D > 0 && !ok_k(sh.D)) return false;
  return true;
}

hipError_t launch_fs4_gateup(const StreamArgs& a, const Workspace& ws, hipStream_t s) {
  const Shape& sh = a.sh;
  if (sh.T == 0) return hipSuccess;
  const int ud = sh.D > 0 ? (sh.D + kGuUnitCols - 1) / kGuUnitCols : 0;
  const int max_active = sh.E > 0 ? std::min(sh.E, sh.T * sh.k) : 0;
  const int ur = sh.E > 0 ? max_active * ((sh.I + kGuUnitCols - 1) / kGuUnitCols) : 0;
  if (ud + ur == 0) return hipSuccess;
  const size_t lds = size_t(kFsRows) * sh.H * 2;
  hipLaunchKernelGGL(k_fs4_gateup, dim3(ud + ur), dim3(kFsThreads), lds, s, a, ws, ud);
  return hipGetLastError();
}

hipError_t launch_fs4_down(const StreamArgs& a, const Workspace& ws, hipStream_t s) {
  const Shape& sh = a.sh;
  if (sh.T == 0) return hipSuccess;
  const int dcols = kDnGroupCols * kDdGroups, rcols = kDnGroupCols * kDnGroups;
  const int ud = sh.D > 0 ? (sh.H + dcols - 1) / dcols : 0;
  const int max_active = sh.E > 0 ? std::min(sh.E, sh.T * sh.k) : 0;
  const int ur = sh.E > 0 ? max_active * ((sh.H + rcols - 1) / rcols) : 0;
  if (ud + ur == 0) return hipSuccess;
  const size_t lds = size_t(kFsRows) * std::max(sh.E > 0 ? sh.I : 0, sh.D) * 2;
  hipLaunchKernelGGL(k_fs4_down, dim3(ud + ur), dim3(kFsThreads), lds, s, a, ws, ud);
  return hipGetLastError();
}

}  // namespace moe
