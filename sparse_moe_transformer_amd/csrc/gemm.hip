// Grouped GEMMs of the MoE block on bf16 MFMA (gfx950 v_mfma_f32_32x32x16_bf16).
//
//   gate/up (GeGLU, fused):  h = gelu_tanh(A . Wg) * (A . Wu)     -> bf16
//   down:                    y = A . Wd                          -> bf16
//   router logits:           z = x . W_r                         -> fp32
//
// One launch serves two segments: a host-sized one (the dense branch, or
// the router) and an expert-grouped one whose M-tiles (expert, first row,
// rows) come from the device-side tile list written by the grouping
// kernels; blocks past the list's end exit at once, so no host sync is
// needed to size the grid.  Routed A rows of the gate/up GEMM are gathered
// from x through perm and never copied out.
//
// Tile: 256 rows x 256 B-columns x 64 K, 512 threads = 8 waves in two
// groups of 4 (one wave of each group per SIMD).  Group g owns tile rows
// [128 g, 128 g + 128); wave w of a group owns 64 B-columns (gate/up: 32
// gate + the 32 up columns at the same output positions, so the GeGLU
// epilogue pairs them in registers), i.e. 128 x 64 outputs as 4 x 2 MFMA
// 32x32 blocks.  128-row wave tiles keep the LDS reads per MFMA low.
//
// Ping-pong: while one group runs the MFMAs of a k-step from LDS, the other
// writes its half of a later k-step's tiles (A rows of its own half, 32 of
// the 64 k rows of B) to LDS and issues its next global loads; a block
// barrier swaps the roles, so each SIMD's matrix unit always has a wave to
// feed.  LDS holds two k-steps (2 x 72 KB).
//
// Weights are [K, N] with N contiguous, while the MFMA B operand wants 8
// consecutive k of one column per lane.  Each thread loads a 4(k) x 8(n)
// block with four 16-byte loads, transposes it in registers and stores 4-k
// runs to an LDS tile laid out [n][k] (k contiguous); MFMA operands are then
// single 16-byte LDS reads.  Rows are padded to 72 elements (144 B), which
// spreads 16 lanes of a 16-byte read over the 64 LDS banks.  NVFP4 weights
// are already k-contiguous ([N, K/2]): each thread decodes 32 codes of one
// column to bf16 (an e2m1 x e4m3 product is exact in bf16) and the fp32
// tensor scale is applied in the epilogue.
//
// Block ids are remapped so that each XCD takes a contiguous run of the
// tiles that exist (the N-tiles of one M-tile, then the next M-tile of the
// same expert share its L2); the grid covers the worst-case tile list and
// the surplus blocks exit at once.
#include <type_traits>

#include "common.h"

namespace moe {

namespace {

constexpr int BM = kGemmBM;  // 256
constexpr int BN = 256;      // B columns per tile
constexpr int BK = 64;
constexpr int LDSK = BK + 8;  // padded row (elements)
constexpr int kThreads = 512;  // 8 waves: 2 (rows) x 4 (columns), 128 x 64 outputs each
constexpr int kWI = BM / 64;   // 32-row MFMA blocks per wave
constexpr int kALoads = BM * BK / 8 / kThreads;  // 16-byte A chunks per thread and k-step (a group moves half the tile with half the threads)
constexpr int kXcd = 8;

enum { MODE_PLAIN_BF16 = 0, MODE_PLAIN_F32 = 1, MODE_GATEUP = 2 };
enum { W_BF16 = 0, W_FP4 = 1 };

struct Seg {
  const bf16_t* A;
  int lda;
  const int32_t* gather;  // routed gate/up: tile row r reads A row gather[row0 + r]
  const bf16_t* B0;       // bf16 [G][K][ldb] (gate or the only matrix)
  const bf16_t* B1;       // up (gate/up mode)
  long long b_gstride;    // elements between groups
  int ldb;
  Fp4Mat F0, F1;          // NVFP4 [G][N][K/2], [G][N][K/16], [G]
  int K;
  int N;                  // output columns
  void* C;
  int ldc;
  int n_ntiles;           // output column tiles
  int host_rows;          // host-sized segment: number of rows (tiles at BM)
  const int32_t* mtiles;  // expert-grouped segment: device tile list (else null)
  const int32_t* n_mtiles;
  int max_mtiles;
  int ksplit;             // K-slices (host-sized segment only); slice s writes C + s * c_slice
  long long c_slice;
};

__device__ __forceinline__ uint32_t perm_lo16(uint32_t a, uint32_t b) {
  // (a.lo16, b.lo16) -> a.lo | b.lo << 16
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t perm_hi16(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// float8_e4m3fn byte -> fp32 (finite codes): bit 7 sign, bits 6..3 exponent
// (bias 7), bits 2..0 mantissa; exponent 0 is subnormal, m * 2^-9
__device__ __forceinline__ float e4m3_f32(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u;
  const uint32_t m = b & 7u;
  const float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : float(m) * 0.001953125f;
  return (b & 0x80u) ? -mag : mag;
}

template <int MODE, int WF>
__global__ __launch_bounds__(kThreads, 1) void k_gemm(Seg s0, Seg s1, int units0, int units_total) {
  // ---- logical tile of this block (XCD-aware remap) ----
  // The grid covers the worst-case tile list; the remap spreads only the
  // tiles that exist (the grouped segment's count is read from the device
  // list) evenly over the XCDs, each XCD taking a contiguous run, so no XCD
  // is left with the empty tail of the list.  Surplus blocks exit at once.
  const int total = s1.mtiles ? units0 + (*s1.n_mtiles) * s1.n_ntiles * s1.ksplit : units_total;
  const int per = (total + kXcd - 1) / kXcd;
  const int slot = blockIdx.x / kXcd;
  const int u = (blockIdx.x % kXcd) * per + slot;
  if (slot >= per || u >= total) return;
  const bool second = u >= units0;
  const Seg& S = second ? s1 : s0;
  int uu = second ? u - units0 : u;
  const int ks = uu % S.ksplit;
  uu /= S.ksplit;
  const int mt = uu / S.n_ntiles;
  const int nt = uu % S.n_ntiles;
  int grp = 0, row0, rows;
  if (S.mtiles) {
    if (mt >= *S.n_mtiles) return;
    grp = S.mtiles[4 * mt];
    row0 = S.mtiles[4 * mt + 1];
    rows = S.mtiles[4 * mt + 2];
  } else {
    row0 = mt * BM;
    rows = min(BM, S.host_rows - row0);
  }
  const int K = S.K, N = S.N;
  // output columns of this tile: gate/up pairs 128 gate with 128 up columns
  constexpr int OUTN = (MODE == MODE_GATEUP) ? BN / 2 : BN;
  const int n0 = nt * OUTN;

  // LDS: two k-steps of A [BM][LDSK] and B [BN][LDSK] tiles; after the K
  // loop the same bytes stage the bf16 output tile
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * (BM + BN) * LDSK * 2];
  bf16_t* const As0 = reinterpret_cast<bf16_t*>(smem);
  bf16_t* const Bs0 = As0 + 2 * BM * LDSK;
  auto As = [&](int b) { return As0 + b * (BM * LDSK); };
  auto Bs = [&](int b) { return Bs0 + b * (BN * LDSK); };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform by construction (an SGPR): the wave groups below branch on
  // it around block barriers, so each wave must take exactly one path
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave & 3;

  // ---- loads are split between the two wave groups (group g = waves
  // 4g .. 4g+3, threads tg = tid - 256 g): group g moves A rows
  // [128 g, 128 g + 128) and the k rows [32 g, 32 g + 32) of the B tile.
  const int grp_w = wave >> 2;  // this wave's group (also its 128-row half of the tile)
  const int tg = tid & 255;
  // A: 16-byte chunks c = tg + 256 i of the group's half, row c/8, k-chunk
  // c%8.  Rows past the tile's end read a valid row (their results are never
  // stored), so the loads need no branches.
  // A and bf16 B go through buffer resources: 32-bit byte offsets per lane,
  // the k-step as a uniform offset (every operand matrix is below 2 GB).
  const __amdgpu_buffer_rsrc_t ars = rsrc_of(uniform_ptr(S.A));
  uint32_t aoff[kALoads];
#pragma unroll
  for (int i = 0; i < kALoads; ++i) {
    const int c = tg + 256 * i;
    const int tr = grp_w * 128 + (c >> 3);
    const int r = tr < rows ? tr : 0;
    const uint32_t gr = S.gather ? uint32_t(S.gather[row0 + r]) : uint32_t(row0 + r);
    aoff[i] = (gr * uint32_t(S.lda) + uint32_t((c & 7) * 8)) * 2u;
  }

  // ---- B source of this thread (columns past N read column 0; discarded)
  __amdgpu_buffer_rsrc_t brs = ars;  // bf16: 4 rows x 8 columns at (bkb*4, bcol)
  uint32_t boff = 0;
  const uint32_t brow = uint32_t(S.ldb) * 2u;  // bytes per k row of B
  int bkb = 0, bcol = 0;
  const uint8_t* fq = nullptr;   // NVFP4: 16 codes (8 bytes) of one column
  const uint8_t* fs = nullptr;
  int fn = 0, fkq = 0;
  if (WF == W_BF16) {
    const int nb = tg >> 3;        // 32 groups of 8 columns
    bkb = (tg & 7) + 8 * grp_w;    // 16 groups of 4 k; the group's 8
    bcol = nb * 8;
    const bf16_t* Bm = S.B0;
    int ncol = n0 + nb * 8;
    if (MODE == MODE_GATEUP && nb >= 16) {
      Bm = S.B1;
      ncol = n0 + (nb - 16) * 8;
    }
    // the matrix differs between the gate and up halves, which split at a
    // wave boundary, so the base stays wave-uniform
    brs = rsrc_of(uniform_ptr(Bm + grp * S.b_gstride));
    boff = uint32_t(bkb * 4) * brow + uint32_t(ncol < N ? ncol : 0) * 2u;
  } else {
    fn = tg;                  // LDS column 0..255
    fkq = grp_w;              // which 32-k half of the 64-k step
    const Fp4Mat* F = &S.F0;
    int ncol = n0 + fn;
    if (MODE == MODE_GATEUP && fn >= 128) {
      F = &S.F1;
      ncol = n0 + fn - 128;
    }
    const long long NN = S.N;
    const long long col = ncol < N ? ncol : 0;
    fq = F->q + (grp * NN + col) * (long long)(K / 2) + fkq * 16;
    fs = F->scale + (grp * NN + col) * (long long)(K / 16) + fkq * 2;
  }

  auto load_tile = [&](int k0, u32x4_t(&ra)[kALoads], u32x4_t(&rb)[4]) {
#pragma unroll
    for (int i = 0; i < kALoads; ++i) ra[i] = bload<u32x4_t, 0>(ars, aoff[i], uint32_t(k0) * 2u);
    if (WF == W_BF16) {
#pragma unroll
      for (int r = 0; r < 4; ++r) rb[r] = bload<u32x4_t, 0>(brs, boff + uint32_t(r) * brow, uint32_t(k0) * brow);
    } else {
      rb[0] = *reinterpret_cast<const u32x4_t*>(fq + k0 / 2);
      rb[1] = u32x4_t{uint32_t(*reinterpret_cast<const uint16_t*>(fs + k0 / 16)), 0, 0, 0};
    }
  };

  auto store_tile = [&](int buf, const u32x4_t(&ra)[kALoads], const u32x4_t(&rb)[4]) {
    bf16_t* as = As(buf) + grp_w * 128 * LDSK;
#pragma unroll
    for (int i = 0; i < kALoads; ++i) {
      const int c = tg + 256 * i;
      *reinterpret_cast<u32x4_t*>(as + (c >> 3) * LDSK + (c & 7) * 8) = ra[i];
    }
    bf16_t* bs = Bs(buf);
    if (WF == W_BF16) {
      // rb[r] holds k = 4kb + r, columns bcol..bcol+7 (2 per dword)
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t r0 = rb[0][d], r1 = rb[1][d], r2 = rb[2][d], r3 = rb[3][d];
        const u32x2_t c0 = {perm_lo16(r0, r1), perm_lo16(r2, r3)};  // column 2d
        const u32x2_t c1 = {perm_hi16(r0, r1), perm_hi16(r2, r3)};  // column 2d+1
        *reinterpret_cast<u32x2_t*>(bs + (bcol + 2 * d) * LDSK + bkb * 4) = c0;
        *reinterpret_cast<u32x2_t*>(bs + (bcol + 2 * d + 1) * LDSK + bkb * 4) = c1;
      }
    } else {
      const uint32_t sc = rb[1][0];
      const float s0v = e4m3_f32(sc & 0xFFu);
      const float s1v = e4m3_f32((sc >> 8) & 0xFFu);
      uint32_t outw[16];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t q = rb[0][d];  // 8 codes, k = 8d .. 8d+7 (low nibble first)
        const float sv = d < 2 ? s0v : s1v;
        // byte p: codes k = 8d+2p (low nibble), 8d+2p+1, decoded exactly by
        // the gfx950 e2m1 pair conversion (unit scale); e2m1 x e4m3 is exact
        // in bf16, so the top 16 bits of each product are kept
        const f32x2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 0);
        const f32x2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 1);
        const f32x2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 2);
        const f32x2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 3);
        outw[d * 4 + 0] = perm_hi16(__float_as_uint(v0.x * sv), __float_as_uint(v0.y * sv));
        outw[d * 4 + 1] = perm_hi16(__float_as_uint(v1.x * sv), __float_as_uint(v1.y * sv));
        outw[d * 4 + 2] = perm_hi16(__float_as_uint(v2.x * sv), __float_as_uint(v2.y * sv));
        outw[d * 4 + 3] = perm_hi16(__float_as_uint(v3.x * sv), __float_as_uint(v3.y * sv));
      }
      bf16_t* dst = bs + fn * LDSK + fkq * 32;
#pragma unroll
      for (int v = 0; v < 4; ++v)
        *reinterpret_cast<u32x4_t*>(dst + v * 8) =
            u32x4_t{outw[4 * v], outw[4 * v + 1], outw[4 * v + 2], outw[4 * v + 3]};
    }
  };

  f32x16_t acc[kWI][2];
#pragma unroll
  for (int i = 0; i < kWI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // this wave's 32 x 32 blocks: rows 128 g + 32i (g = its group); columns (gate/up: gate
  // and up at wn*32; else wn*64 + 32j)
  const int kofs = (lane >> 5) * 8;
  int arow_l[kWI], brow_l[2];
#pragma unroll
  for (int i = 0; i < kWI; ++i) arow_l[i] = (grp_w * kWI * 32 + i * 32 + (lane & 31)) * LDSK + kofs;
  if (MODE == MODE_GATEUP) {
    brow_l[0] = (wn * 32 + (lane & 31)) * LDSK + kofs;
    brow_l[1] = (BN / 2 + wn * 32 + (lane & 31)) * LDSK + kofs;
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j) brow_l[j] = (wn * 64 + j * 32 + (lane & 31)) * LDSK + kofs;
  }

  // Row blocks of this wave inside the tile's rows (wave-uniform): the K
  // loop is instantiated per count NI, so the ragged last M-tile of an
  // expert costs only its valid blocks' MFMAs; a wave with no valid rows or
  // no valid columns only moves tiles.  (Columns past N inside a valid wave
  // are computed from column 0 and dropped.)
  const int wrow0 = grp_w * kWI * 32;
  const bool wcols = (MODE == MODE_GATEUP) ? n0 + wn * 32 < N : n0 + wn * 64 < N;
  const int ni = wcols ? __builtin_amdgcn_readfirstlane(min(kWI, max(0, (rows - wrow0 + 31) / 32))) : 0;

  // Fragments of sub-step kk + 1 are read from LDS while the MFMAs of kk run.
  auto compute = [&](int buf, auto ni_c) {
    constexpr int NI = decltype(ni_c)::value;
    if (NI == 0) return;
    const bf16_t* as = As(buf);
    const bf16_t* bs = Bs(buf);
    bf16x8_t a[2][kWI], b[2][2];
    auto frags = [&](int kk, bf16x8_t(&af)[kWI], bf16x8_t(&bf)[2]) {
#pragma unroll
      for (int i = 0; i < NI; ++i) af[i] = *reinterpret_cast<const bf16x8_t*>(as + arow_l[i] + kk);
#pragma unroll
      for (int j = 0; j < 2; ++j) bf[j] = *reinterpret_cast<const bf16x8_t*>(bs + brow_l[j] + kk);
    };
    frags(0, a[0], b[0]);
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      if (s + 1 < BK / 16) frags((s + 1) * 16, a[(s + 1) & 1], b[(s + 1) & 1]);
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s & 1][i], b[s & 1][j], acc[i][j], 0, 0, 0);
    }
  };

  // K-steps of this tile's slice, ping-pong between the wave groups: each
  // SIMD holds one wave of each group, and while one group runs the MFMAs
  // of a k-step the other writes its half of a later k-step's tiles to LDS
  // and issues its next global loads; a block barrier swaps the roles.
  // Intervals (C = compute, M = write my half of step s to LDS buffer s%2,
  // then load my half of step s+1 into registers):
  //   group 0: C(0) | M(1) | C(1) | M(2) | ... | C(nk-1)
  //   group 1: M(1) | C(0) | M(2) | C(1) | ... | M(nk) | C(nk-1)
  // Step s is complete in its buffer before group 0 reads it (both halves
  // are written in the two intervals before), and a buffer is rewritten
  // only after both groups have read it.  Both groups pass 2 nk - 1
  // barriers.  Memory phases past the last step only keep the count.
  const int nk_all = K / BK;
  const int kt0 = ks * nk_all / S.ksplit;
  const int nk = (ks + 1) * nk_all / S.ksplit - kt0;
  u32x4_t ra[kALoads], rb[4];
  // (sched_barrier: the staging registers hold one step at a time; the
  // scheduler must not start the next loads before the stores have read them)
  auto mem_phase = [&](int st) {  // write my half of step st, load my half of step st + 1
    if (st < nk) {
      store_tile(st & 1, ra, rb);
      __builtin_amdgcn_sched_barrier(0);
      if (st + 1 < nk) load_tile((kt0 + st + 1) * BK, ra, rb);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto kloop = [&](auto ni_c) {
    load_tile(kt0 * BK, ra, rb);
    store_tile(0, ra, rb);
    __builtin_amdgcn_sched_barrier(0);
    if (nk > 1) load_tile((kt0 + 1) * BK, ra, rb);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    if (grp_w == 0) {
      for (int kt = 0; kt < nk; ++kt) {
        compute(kt & 1, ni_c);
        __syncthreads();
        if (kt + 1 < nk) {
          mem_phase(kt + 1);
          __syncthreads();
        }
      }
    } else {
      mem_phase(1);
      __syncthreads();
      for (int kt = 0; kt < nk; ++kt) {
        compute(kt & 1, ni_c);
        if (kt + 1 < nk) {
          __syncthreads();
          mem_phase(kt + 2);
          __syncthreads();
        }
      }
    }
  };
  switch (ni) {
    case 0: kloop(std::integral_constant<int, 0>{}); break;
    case 1: kloop(std::integral_constant<int, 1>{}); break;
    case 2: kloop(std::integral_constant<int, 2>{}); break;
    case 3: kloop(std::integral_constant<int, 3>{}); break;
    default: kloop(std::integral_constant<int, kWI>{}); break;
  }

  // ---- epilogue: lane holds column (lane & 31); rows 8(r/4) + 4(lane/32) + r%4
  float ts0 = 1.f, ts1 = 1.f;
  if (WF == W_FP4) {
    ts0 = S.F0.tscale[grp];
    if (MODE == MODE_GATEUP) ts1 = S.F1.tscale[grp];
  }
  if (MODE == MODE_PLAIN_F32) {  // router logits: fp32, written directly
    if (!wcols) return;
#pragma unroll
    for (int i = 0; i < kWI; ++i) {
      if (i >= ni) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wrow0 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row >= rows) continue;
        const long long orow = (long long)(row0 + row) * S.ldc + ks * S.c_slice;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = n0 + wn * 64 + j * 32 + (lane & 31);
          if (col < N) reinterpret_cast<float*>(S.C)[orow + col] = acc[i][j][r] * ts0;
        }
      }
    }
    return;
  }
  // bf16 outputs go through LDS so that the tile leaves in 16-byte stores.
  // Neighbouring lanes swap values (DPP) so that each lane writes pairs of
  // adjacent columns: even lanes rows r = 2q, odd lanes rows r = 2q + 1.
  // Every wave passes both barriers (those without valid columns too).
  constexpr int SP = OUTN * 2 + 16;  // staging row pitch (bytes)
  __syncthreads();                   // every wave's last fragments are read
  if (wcols) {
    const bool odd = lane & 1;
#pragma unroll
    for (int i = 0; i < kWI; ++i) {
      if (i >= ni) continue;
#pragma unroll
      for (int j = 0; j < ((MODE == MODE_GATEUP) ? 1 : 2); ++j) {
        uint32_t vb[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float v = (MODE == MODE_GATEUP) ? gelu_tanh(acc[i][0][r] * ts0) * (acc[i][1][r] * ts1)
                                                : acc[i][j][r] * ts0;
          vb[r] = f32_to_bf16_bits(v);
        }
        const int cpair = ((MODE == MODE_GATEUP) ? wn * 32 : wn * 64 + j * 32) + (lane & 30);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const uint32_t send = odd ? vb[2 * q] : vb[2 * q + 1];
          const uint32_t recv = uint32_t(__builtin_amdgcn_mov_dpp(int(send), 0xB1, 0xF, 0xF, false));  // lane ^ 1
          const int r = 2 * q + (odd ? 1 : 0);
          const int row = wrow0 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          const uint32_t packed = odd ? (recv | (vb[2 * q + 1] << 16)) : (vb[2 * q] | (recv << 16));
          *reinterpret_cast<uint32_t*>(smem + row * SP + cpair * 2) = packed;
        }
      }
    }
  }
  __syncthreads();
  constexpr int CPR = OUTN / 8;  // 16-byte chunks per staged row
  bf16_t* C = reinterpret_cast<bf16_t*>(S.C);
  for (int c = tid; c < BM * CPR; c += kThreads) {
    const int row = c / CPR, ch = c % CPR;
    const int col = n0 + ch * 8;
    if (row < rows && col < N)
      *reinterpret_cast<u32x4_t*>(C + (long long)(row0 + row) * S.ldc + ks * S.c_slice + col) =
          *reinterpret_cast<const u32x4_t*>(smem + row * SP + ch * 16);
  }
}

Seg empty_seg() {
  Seg s{};
  s.n_ntiles = 1;
  s.ksplit = 1;
  return s;
}

template <int MODE, int WF>
hipError_t launch(const Seg& a, const Seg& b, int units_a, int units_b, hipStream_t st) {
  const int total = units_a + units_b;
  if (total <= 0) return hipSuccess;
  const int per = (total + kXcd - 1) / kXcd;
  hipLaunchKernelGGL((k_gemm<MODE, WF>), dim3(per * kXcd), dim3(kThreads), 0, st, a, b, units_a, total);
  return hipGetLastError();
}

int host_units(const Seg& s) { return ((s.host_rows + BM - 1) / BM) * s.n_ntiles * s.ksplit; }
int grouped_units(const Seg& s) { return s.max_mtiles * s.n_ntiles; }

}  // namespace

// Router logits as ksplit K-slices of partial sums: slice s -> logits + s*T*E.
hipError_t launch_gemm_router(const Shape& sh, const bf16_t* x, const bf16_t* wr, float* logits, int ksplit,
                              hipStream_t s) {
  Seg r = empty_seg();
  r.A = x;
  r.lda = sh.H;
  r.B0 = wr;
  r.ldb = sh.E;
  r.K = sh.H;
  r.N = sh.E;
  r.C = logits;
  r.ldc = sh.E;
  r.n_ntiles = (sh.E + BN - 1) / BN;
  r.host_rows = sh.T;
  r.ksplit = ksplit;
  r.c_slice = (long long)sh.T * sh.E;
  Seg none = empty_seg();
  return launch<MODE_PLAIN_F32, W_BF16>(r, none, host_units(r), 0, s);
}

hipError_t launch_gemm_gateup(const StreamArgs& a, const Workspace& ws, int max_mtiles, hipStream_t s) {
  const Shape& sh = a.sh;
  Seg d = empty_seg(), e = empty_seg();
  // dense branch: all T tokens
  if (sh.D > 0) {
    d.A = a.x;
    d.lda = sh.H;
    d.B0 = a.dg;
    d.B1 = a.du;
    d.ldb = sh.D;
    d.F0 = a.fdg;
    d.F1 = a.fdu;
    d.K = sh.H;
    d.N = sh.D;
    d.C = ws.h_d;
    d.ldc = sh.D;
    d.n_ntiles = (sh.D + BN / 2 - 1) / (BN / 2);
    d.host_rows = sh.T;
  }
  // routed experts: rows gathered through perm
  e.A = a.x;
  e.lda = sh.H;
  e.gather = ws.perm;
  e.B0 = a.wg;
  e.B1 = a.wu;
  e.b_gstride = (long long)sh.H * sh.I;
  e.ldb = sh.I;
  e.F0 = a.fg;
  e.F1 = a.fu;
  e.K = sh.H;
  e.N = sh.I;
  e.C = ws.h;
  e.ldc = sh.I;
  e.n_ntiles = (sh.I + BN / 2 - 1) / (BN / 2);
  e.mtiles = ws.mtiles;
  e.n_mtiles = ws.meta;
  e.max_mtiles = max_mtiles;
  const int ud = sh.D > 0 ? host_units(d) : 0;
  if (a.nvfp4) return launch<MODE_GATEUP, W_FP4>(d, e, ud, grouped_units(e), s);
  return launch<MODE_GATEUP, W_BF16>(d, e, ud, grouped_units(e), s);
}

hipError_t launch_gemm_down(const StreamArgs& a, const Workspace& ws, int max_mtiles, hipStream_t s) {
  const Shape& sh = a.sh;
  Seg d = empty_seg(), e = empty_seg();
  if (sh.D > 0) {
    d.A = ws.h_d;
    d.lda = sh.D;
    d.B0 = a.dd;
    d.ldb = sh.H;
    d.F0 = a.fdd;
    d.K = sh.D;
    d.N = sh.H;
    d.C = ws.y_d;
    d.ldc = sh.H;
    d.n_ntiles = (sh.H + BN - 1) / BN;
    d.host_rows = sh.T;
  }
  e.A = ws.h;
  e.lda = sh.I;
  e.B0 = a.wd;
  e.b_gstride = (long long)sh.I * sh.H;
  e.ldb = sh.H;
  e.F0 = a.fd;
  e.K = sh.I;
  e.N = sh.H;
  e.C = ws.y;
  e.ldc = sh.H;
  e.n_ntiles = (sh.H + BN - 1) / BN;
  e.mtiles = ws.mtiles;
  e.n_mtiles = ws.meta;
  e.max_mtiles = max_mtiles;
  const int ud = sh.D > 0 ? host_units(d) : 0;
  if (a.nvfp4) return launch<MODE_PLAIN_BF16, W_FP4>(d, e, ud, grouped_units(e), s);
  return launch<MODE_PLAIN_BF16, W_BF16>(d, e, ud, grouped_units(e), s);
}

}  // namespace moe
