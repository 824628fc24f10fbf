// Grouped GEMMs of the MoE block with NVFP4 weights, weights streamed into
// registers (gfx950 v_mfma_f32_32x32x16_bf16 on exact bf16 weight values).
//
// NVFP4 checkpoint config, quantization_config group_0.weights: 4-bit float
// e2m1 values two per byte, groups of 16 along K with float8_e4m3fn scales,
// strategy tensor_group (one fp32 scale per matrix); the matrices are stored
// out-major, [N][K/2] codes and [N][K/16] scales, so the 32 codes of 32
// consecutive k of one output column are 16 contiguous bytes.  That is the
// MFMA B operand's shape (8 consecutive k of one column per lane), so the
// weights never pass through LDS: a lane loads 16 bytes of codes and a dword
// of 4 group scales per 64 k, decodes them (e2m1 code x e4m3 scale is exact
// in bf16; the fp32 tensor scale is applied to the accumulators) and feeds
// four MFMA k-steps.  Only the activations (a few rows per expert, shared by
// every wave of the block) are staged in LDS.
//
//   gate/up (GeGLU, fused):  h = gelu_tanh(A . Wg) * (A . Wu)     -> bf16
//   down:                    y = A . Wd                          -> bf16
//
// The k order inside a 64-k step is permuted (the contraction does not
// depend on it): lane half hf (lanes 32 hf .. 32 hf + 31) holds k = 32 hf ..
// 32 hf + 31 of the step, and MFMA k-step i reads k = 32 hf + 8 i .. + 7 of
// each half, from B (dword i of the lane's 16 code bytes) and from A alike.
//
// Work units: (row tile, column block).  A row tile is up to 32 NR rows of
// one expert (the device tile list written by the grouping kernels) or of
// the dense branch (host-sized); a column block is W waves, each owning 32
// output columns (gate/up: 32 gate and the 32 up columns at the same
// positions, paired by the GeGLU epilogue) or 64 (down).  Consecutive units
// are the column blocks of one row tile, so they share its A rows in L2;
// each XCD takes an equal contiguous run of each segment's units.
//
// Pipeline per 64-k step: the A rows of the step go global -> LDS by DMA
// (buffer loads with the lds flag) D steps ahead; the weight codes and
// scales of a step are loaded into registers PF steps ahead (decode-sized
// tiles), or in bursts of 2 steps one burst ahead (128-row tiles; 3 A stages:
// the shallower ring leaves registers to the scheduler, 190 us per gate/up
// launch at T = 1024 against 196 with bursts of 4 and 5 stages).  Every load is
// issued in every step (rows past a tile's end and columns past N get an
// out-of-range offset: no memory access, zeros), so the wait counts are
// constants.
#include <algorithm>
#include <type_traits>

#include "common.h"

namespace moe {

namespace {

constexpr int kStepK = 64;  // k per pipeline step
constexpr int kBurst = 2;  // weight steps per load burst of the 128-row tiles (A: kBurst + 1 LDS stages)
constexpr int kXcd = 8;
enum { FM_GATEUP = 0, FM_DOWN = 1 };

typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;

constexpr int kOutOfRange = int(0x80000000u);  // beyond every buffer resource's range

struct F4Seg {
  const bf16_t* A;
  int lda;
  const int32_t* gather;  // routed gate/up: A row of tile row r = gather[row0 + r]
  Fp4Mat F0, F1;          // F1: the up matrices (gate/up)
  int K, N;               // K: multiple of 64; N: multiple of 32
  bf16_t* C;
  int ldc;
  int nblk;               // column blocks
  int host_rows;          // host-sized segment: rows (tiles of 32 NR)
  const int32_t* tiles;   // grouped segment: device tile list (group, row0, rows, 0), else null
  const int32_t* n_tiles; // ... its length (device)
  int max_tiles;
  const float* in_scale;  // NVFP4 activations: the A operand's global scale (device), or null
};

__device__ __forceinline__ i32x4_t rsrc4(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  i32x4_t r;
  r[0] = int(__builtin_amdgcn_readfirstlane(uint32_t(v)));
  r[1] = int(__builtin_amdgcn_readfirstlane(uint32_t(v >> 32)));
  r[2] = 0x7FFFFFFF;
  r[3] = 0x00020000;
  return r;
}

// 16 bytes per lane global -> LDS (lane i at lds + 16 i; lds is wave-uniform,
// it goes to M0).  No register result; the kernel waits for it itself.
__device__ __forceinline__ void copy_b128_to_lds(i32x4_t rsrc, uint32_t lds, int voffset, int soffset) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(lds), "v"(voffset), "s"(rsrc),
               "s"(soffset)
               : "memory");
}

template <int VM>
__device__ __forceinline__ void wait_vm() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  // vmcnt <= VM; expcnt and lgkmcnt not waited
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// float8_e4m3fn byte -> fp32: bit 7 sign, bits 6..3 exponent (bias 7), bits
// 2..0 mantissa; exponent 0 is subnormal (m * 2^-9)
__device__ __forceinline__ float e4m3_f32(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u;
  const uint32_t m = b & 7u;
  const float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : float(m) * 0.001953125f;
  return (b & 0x80u) ? -mag : mag;
}

// 8 e2m1 codes (a dword, low nibble = lower k) times scale sv -> 8 bf16 (exact)
__device__ __forceinline__ bf16x8_t decode8(uint32_t q, float sv) {
  // byte p of q: codes 2p (low nibble) and 2p + 1, decoded exactly by the
  // gfx950 e2m1 pair conversion (unit scale); the product with the e4m3 scale
  // is exact in bf16, so its top 16 bits are the bf16 value
  const f32x2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 0);
  const f32x2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 1);
  const f32x2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 2);
  const f32x2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, 1.0f, 3);
  const u32x4_t w = {__builtin_amdgcn_perm(__float_as_uint(v0.y * sv), __float_as_uint(v0.x * sv), 0x07060302u),
                     __builtin_amdgcn_perm(__float_as_uint(v1.y * sv), __float_as_uint(v1.x * sv), 0x07060302u),
                     __builtin_amdgcn_perm(__float_as_uint(v2.y * sv), __float_as_uint(v2.x * sv), 0x07060302u),
                     __builtin_amdgcn_perm(__float_as_uint(v3.y * sv), __float_as_uint(v3.x * sv), 0x07060302u)};
  return __builtin_bit_cast(bf16x8_t, w);
}

// f(integral_constant<0>) .. f(integral_constant<N - 1>), in order
template <int N, class F>
__device__ __forceinline__ void unroll(F&& f) {
  if constexpr (N > 0) {
    unroll<N - 1>(f);
    f(std::integral_constant<int, N - 1>{});
  }
}

// Weight loads in bursts (BS > 1): at each step s with s % BS == 0 a wave
// loads the weights of steps s + BS .. s + 2 BS - 1, so the 2 BS 16-byte
// pieces of one column's 128-byte code line that a burst covers are
// requested together, and the scale dwords of a column's BS <= 4 steps are
// one 16-byte load.  Per step the order is: wait, barrier, A copies of step
// s + D - 1 (CA), then the burst if any (the scale loads, then BS steps'
// code loads).  burst_wait(p): loads issued after
// the last one that step s = q BS + p needs, in that steady order; the
// prologue replays it exactly when D - 1 == BS.
constexpr int burst_wait(int BS, int D, int CA, int NQ, int NS, int p) {
  // a burst: NS scale loads (one per group, all its steps), then BS steps of
  // NQ code loads; step p of it needs the scales and its own codes
  const int s = 8 * BS + p;  // any step past the prologue
  const int burst = BS * NQ + NS;
  auto issued = [&](int u) { return CA + (u % BS == 0 ? burst : 0); };  // loads issued in step u
  int after_a = (((s - D + 1) % BS) == 0) ? burst : 0;                 // A(s) issued in step s - D + 1
  for (int u = s - D + 2; u < s; ++u) after_a += issued(u);
  const int b = (s / BS - 1) * BS;                                      // the burst holding step s
  int after_b = (BS - 1 - p) * NQ;  // the burst's code loads after step s's (its scales came first)
  for (int u = b + 1; u < s; ++u) after_b += issued(u);
  return after_a < after_b ? after_a : after_b;
}

// Proof at compile time that the constant waits are enough: replay the
// issue sequence of the first 8 rounds (prologue included) and check at
// every step that the wait leaves no load outstanding that the step reads.
// Loads are tagged by kind (A copy, weight codes, weight scales) and step.
// BS == 1: the per-step order (A copies, then per group codes and scales of
// step s + PF) with the wait w1; BS > 1: the burst order above.
constexpr bool waits_cover(int BS, int D, int PF, int CA, int NQ, int NS, int w1) {
  constexpr int kMax = 4096;
  int kind[kMax] = {}, step[kMax] = {};  // kind: 0 A, 1 codes, 2 scales
  int n = 0;
  auto push = [&](int k, int st, int count) {
    for (int i = 0; i < count; ++i) {
      kind[n] = k;
      step[n] = st;
      ++n;
    }
  };
  auto burst = [&](int b) {
    push(2, b, NS);
    for (int i = 0; i < BS; ++i) push(1, b + i, NQ);
  };
  const int rounds = 8 * (BS > 1 ? 2 * BS : PF + 1);
  if (BS == 1) {
    for (int st = 0; st < (D - 1 > PF ? D - 1 : PF); ++st) {
      if (st < D - 1) push(0, st, CA);
      if (st < PF) push(1, st, NQ + NS);
    }
  } else {
    for (int st = 0; st < D - 1; ++st) {
      push(0, st, CA);
      if (st == 0) burst(0);
    }
  }
  for (int s = 0; s < rounds; ++s) {
    const int w = BS == 1 ? w1 : burst_wait(BS, D, CA, NQ, NS, s % BS);
    int last = -1;
    for (int i = 0; i < n; ++i) {
      const bool needed = (kind[i] == 0 && step[i] == s) || (kind[i] == 1 && step[i] == s) ||
                          (kind[i] == 2 && (BS == 1 ? step[i] == s : step[i] == s - s % BS));
      if (needed) last = i;
    }
    if (last < 0 || n - 1 - last < w) return false;  // a needed load could still be in flight
    push(0, s + D - 1, CA);
    if (BS == 1)
      push(1, s + PF, NQ + NS);
    else if (s % BS == 0)
      burst(s + BS);
  }
  return true;
}

// The same check for a wave that copies A only (no column inside the
// matrix): CA copies per step, D - 1 steps ahead, and the wait w.
constexpr bool a_waits_cover(int D, int CA, int w) {
  constexpr int kMax = 1024;
  int step[kMax] = {};
  int n = 0;
  auto push = [&](int st) {
    for (int i = 0; i < CA; ++i) step[n++] = st;
  };
  for (int st = 0; st < D - 1; ++st) push(st);
  for (int s = 0; s < 32; ++s) {
    int last = -1;
    for (int i = 0; i < n; ++i)
      if (step[i] == s) last = i;
    if (last < 0 || n - 1 - last < w) return false;
    push(s + D - 1);
  }
  return true;
}

template <int MODE, int W, int NR, int PF, int D, int BS>
__global__ __launch_bounds__(W * 64) void k_fp4mm(F4Seg s0, F4Seg s1, int units0, int units_total) {
  constexpr int kRowsT = 32 * NR;         // rows of a tile
  constexpr int kAStage = kRowsT * 128;   // bytes of one A stage (64 k bf16 per row)
  constexpr int CA = kAStage / 1024 / W;  // A copies per wave per stage (1 KB each)
  static_assert(CA >= 1 && CA * W * 1024 == kAStage, "A stage must split evenly over the waves");
  constexpr int NB = 4;                   // weight loads per wave per step: codes and scales of 2 column groups
  // loads issued after the last one a step needs: see the header (B(s) is the
  // later when PF <= D - 1, else A(s))
  constexpr int kWaitVm = (PF <= D - 1) ? (PF - 1) * (CA + NB) : NB + (D - 2) * (CA + NB);
  static_assert(kWaitVm < 64, "vmcnt range");
  // a wave that copies A only: at step s's wait its copies of steps s + 1 ..
  // s + D - 2 may stay in flight
  constexpr int kWaitA = CA * (D - 2);
  static_assert(D >= 2 && kWaitA < 64, "A ring depth");
  static_assert(a_waits_cover(D, CA, kWaitA), "an A-only wave's wait leaves its copies of the step in flight");
  static_assert(BS == 1 || D - 1 == BS, "the burst prologue replays the steady order only for D - 1 == BS");
  static_assert(BS <= 4, "a burst's scale dwords are one 16-byte load");
  static_assert(waits_cover(BS, D, PF, (32 * NR * 128) / 1024 / W, 2, 2, kWaitVm), "a step's wait leaves a needed load in flight");
  constexpr int kSlots = BS > 1 ? 2 * BS : PF + 1;  // weight register slots (slot = step % kSlots)

  // ---- logical unit of this block (XCD-aware remap over the real units)
  const int n1 = s1.tiles ? (*s1.n_tiles) * s1.nblk : units_total - units0;
  const int p0 = (units0 + kXcd - 1) / kXcd, p1 = (n1 + kXcd - 1) / kXcd;
  const int xcd = blockIdx.x % kXcd, slot = blockIdx.x / kXcd;
  int u;
  if (slot < p0) {
    u = xcd * p0 + slot;
    if (u >= units0) return;
  } else {
    const int j = xcd * p1 + (slot - p0);
    if (slot - p0 >= p1 || j >= n1) return;
    u = units0 + j;
  }
  const bool second = u >= units0;
  const F4Seg S = second ? s1 : s0;
  const int uu = second ? u - units0 : u;
  const int mt = uu / S.nblk, cb = uu % S.nblk;
  int grp = 0, row0, rows;
  if (S.tiles) {
    grp = S.tiles[4 * mt];
    row0 = S.tiles[4 * mt + 1];
    rows = S.tiles[4 * mt + 2];
  } else {
    row0 = mt * kRowsT;
    rows = min(kRowsT, S.host_rows - row0);
  }
  const int K = S.K, N = S.N;

  __shared__ __attribute__((aligned(1024))) unsigned char lds[D * kAStage];
  lds_u8* const lds3 = (lds_u8*)(lds);
  const uint32_t lds_base = uint32_t(reinterpret_cast<uintptr_t>(lds3));

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5, lc = lane & 31;

  // ---- A copies: copy q of wave w fills tile rows 8 (CA w + q) .. + 7 of a
  // stage; lane: row + lane / 8, LDS chunk lane % 8 <- global chunk
  // (lane % 8) ^ ((row / 2) % 8): the XOR spreads the fragment reads over the
  // banks (the two 128-byte rows of a 256-byte span share it; with
  // row % 8 the reads measured half the full LDS rate on gfx950)
  const i32x4_t arsrc = rsrc4(S.A);
  int aoff[CA];
#pragma unroll
  for (int q = 0; q < CA; ++q) {
    const int r = 8 * (CA * wave + q) + (lane >> 3);
    const int rr = r < rows ? r : 0;
    const uint32_t gr = S.gather ? uint32_t(S.gather[row0 + rr]) : uint32_t(row0 + rr);
    aoff[q] = r < rows ? int((gr * uint32_t(S.lda) + uint32_t(((lane & 7) ^ ((r >> 1) & 7)) * 8)) * 2u) : kOutOfRange;
  }

  // ---- B: column group j of this wave: gate/up: gate (j = 0) and up (j = 1)
  // columns c0 .. c0 + 31; down: columns c0 + 32 j .. + 31.  Lane: column
  // c0 (+32 j) + lc, codes of k = 64 s + 32 hf .. + 31 (16 bytes) and the
  // dword holding the 4 group scales of the step.
  const int c0 = (MODE == FM_GATEUP) ? cb * 32 * W + 32 * wave : cb * 64 * W + 64 * wave;
  const int ncol[2] = {c0 + lc, (MODE == FM_GATEUP) ? c0 + lc : c0 + 32 + lc};
  const bool jv[2] = {c0 < N, (MODE == FM_GATEUP) ? c0 < N : c0 + 32 < N};  // wave-uniform
  __amdgpu_buffer_rsrc_t qrs[2], srs[2];
  int qoff[2], soff[2];
  const long long gq = (long long)grp * N * (K / 2), gs = (long long)grp * N * (K / 16);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const bool up = MODE == FM_GATEUP && j == 1;
    qrs[j] = rsrc_of(uniform_ptr((up ? S.F1.q : S.F0.q) + gq));
    srs[j] = rsrc_of(uniform_ptr((up ? S.F1.scale : S.F0.scale) + gs));
    qoff[j] = jv[j] ? ncol[j] * (K / 2) + 16 * hf : kOutOfRange;
    soff[j] = jv[j] ? ncol[j] * (K / 16) : kOutOfRange;
  }

  int ni = (rows + 31) / 32;
  ni = ni > NR ? NR : ni;
  if (!jv[0]) ni = 0;  // no valid column group: no fragments, no MFMAs
  ni = __builtin_amdgcn_readfirstlane(ni);

  float ts0 = 1.f, ts1 = 1.f;
  {
    const float t0 = S.F0.tscale[grp];
    const float t1 = (MODE == FM_GATEUP) ? S.F1.tscale[grp] : t0;
    const float si = S.in_scale ? *S.in_scale : 1.f;
    ts0 = t0 * si;
    ts1 = t1 * si;
  }

  const int nsteps = K / kStepK;

  auto issue_a = [&](int st) {  // A rows of step st into its ring slot
    const int kk = min(st, nsteps - 1) * kStepK;  // past the end: a clamped step, never read
    const uint32_t base = lds_base + uint32_t((st % D) * kAStage);
#pragma unroll
    for (int q = 0; q < CA; ++q) copy_b128_to_lds(arsrc, base + (CA * wave + q) * 1024, aoff[q], kk * 2);
  };

  auto run = [&](auto ni_c) {
    constexpr int NI = decltype(ni_c)::value;
    f32x16_t acc[NR > 0 ? NR : 1][2];
#pragma unroll
    for (int i = 0; i < (NR > 0 ? NR : 1); ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    u32x4_t bq[kSlots][2];
    uint32_t bs[kSlots][2];  // per step (BS == 1)
    // BS > 1: the scale dwords of a burst's BS steps are one 16-byte load
    // per column group, from step sbase[b] of the two bursts in flight (the
    // first step, or nsteps - 4 near the end, so the load stays in the row)
    u32x4_t bs4[2][2];
    int sbase[2] = {0, 0};

    auto load_q = [&](int st, u32x4_t (&q)[2]) {
      const int s = min(st, nsteps - 1);
#pragma unroll
      for (int j = 0; j < 2; ++j) q[j] = bload<u32x4_t, 0>(qrs[j], uint32_t(qoff[j]), uint32_t(s * 32));
    };
    auto load_s4 = [&](int st, int bslot) {
      const int b = max(0, min(st, nsteps - 4));
      sbase[bslot] = b;
#pragma unroll
      for (int j = 0; j < 2; ++j) bs4[bslot][j] = bload<u32x4_t, 0>(srs[j], uint32_t(soff[j]), uint32_t(b * 4));
    };
    auto load_b = [&](int st, u32x4_t (&q)[2], uint32_t (&sc)[2]) {
      const int s = min(st, nsteps - 1);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        q[j] = bload<u32x4_t, 0>(qrs[j], uint32_t(qoff[j]), uint32_t(s * 32));
        sc[j] = bload<uint32_t, 0>(srs[j], uint32_t(soff[j]), uint32_t(s * 4));
      }
    };

    // prologue: A of steps 0 .. D - 2, weights of steps 0 .. PF - 1, in the
    // per-iteration order (A first), so the constant waits hold from step 0.
    // A wave with no valid column group (NI == 0) still copies its share of
    // every A stage for the others but loads no weights: the compiler would
    // delete loads whose results are never used, and the waits that count
    // them would then let the wave reach the barrier with its A copies still
    // in flight.  Such a wave issues A copies only and waits with its own
    // count (kWaitA).
    if constexpr (NI == 0) {
#pragma unroll
      for (int st = 0; st < D - 1; ++st) issue_a(st);
    } else if constexpr (BS == 1) {
#pragma unroll
      for (int st = 0; st < (D - 1 > PF ? D - 1 : PF); ++st) {
        if (st < D - 1) issue_a(st);
        if (st < PF) load_b(st, bq[st], bs[st]);
      }
    } else {
      // virtual steps -BS .. -1: A of steps 0 .. D - 2, the burst of steps
      // 0 .. BS - 1 after the first
#pragma unroll
      for (int st = 0; st < D - 1; ++st) {
        issue_a(st);
        if (st == 0) {
          load_s4(0, 0);
          unroll<BS>([&](auto ic) {
            constexpr int I = decltype(ic)::value;
            load_q(I, bq[I]);
          });
        }
      }
    }

    auto step = [&](int s, auto slot_c) {
      constexpr int SL = decltype(slot_c)::value;  // s % kSlots
      constexpr int P = SL % BS;                   // position in the burst (BS > 1)
      wait_vm<NI == 0 ? kWaitA : BS == 1 ? kWaitVm : burst_wait(BS, D, CA, 2, 2, P)>();  // A and weights of step s landed
      block_barrier();  // every wave's A copies of step s landed; step s - 1's slot is free
      issue_a(s + D - 1);
      if constexpr (NI == 0) {
        return;
      } else if constexpr (BS == 1) {
        constexpr int SLN = (SL + PF) % (PF + 1);  // slot of step s + PF
        load_b(s + PF, bq[SLN], bs[SLN]);
      } else if constexpr (P == 0) {
        // the slots of steps s + BS .. s + 2 BS - 1 held steps s - BS .. s - 1
        load_s4(s + BS, ((SL + BS) / BS) % 2);
        unroll<BS>([&](auto ic) {
          constexpr int I = decltype(ic)::value;
          load_q(s + BS + I, bq[(SL + BS + I) % kSlots]);
        });
      }
      // the group scales of k = 32 hf .. + 15 and + 16 .. + 31 are bytes
      // 2 hf and 2 hf + 1 of the scale dword
      float sa[2], sb[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        uint32_t sd;
        if constexpr (BS == 1) {
          sd = bs[SL][j];
        } else {
          constexpr int B = (SL / BS) % 2;
          const int e = s - sbase[B];  // 0 .. 3
          const u32x4_t v = bs4[B][j];
          sd = e == 0 ? v[0] : e == 1 ? v[1] : e == 2 ? v[2] : v[3];
        }
        const uint32_t sw = sd >> (16 * hf);
        sa[j] = e4m3_f32(sw & 0xFFu);
        sb[j] = e4m3_f32((sw >> 8) & 0xFFu);
      }
      const lds_u8* abase = lds3 + (s % D) * kAStage;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // B fragment of k-step i: dword i of the codes, decoded here (one
        // k-step's fragments live at a time)
        bf16x8_t bf[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) bf[j] = decode8(bq[SL][j][i], i < 2 ? sa[j] : sb[j]);
        // A fragment: tile row 32 rb + lc, k = 32 hf + 8 i .. + 7 = chunk 4 hf + i
#pragma unroll
        for (int rb = 0; rb < NI; ++rb) {
          const int r = 32 * rb + lc;
          const bf16x8_t a = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8_t*>(
              abase + r * 128 + (((4 * hf + i) ^ ((r >> 1) & 7)) << 4));
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[rb][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bf[j], acc[rb][j], 0, 0, 0);
        }
      }
    };

    for (int t0 = 0; t0 < nsteps; t0 += kSlots) {
      // the register slot of each step is a compile-time index
      unroll<kSlots>([&](auto ic) {
        constexpr int I = decltype(ic)::value;
        if (t0 + I < nsteps) step(t0 + I, ic);
      });
    }
    wait_vm<0>();  // no copy may still be landing when the block exits

    // ---- epilogue: lane holds column lc of each group; rows 8 (r / 4) + 4 hf + r % 4
#pragma unroll
    for (int rb = 0; rb < NI; ++rb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * rb + 8 * (r >> 2) + 4 * hf + (r & 3);
        if (row >= rows) continue;
        bf16_t* crow = S.C + (long long)(row0 + row) * S.ldc;
        if (MODE == FM_GATEUP) {
          crow[ncol[0]] = bf16_t(f32_to_bf16_bits(gelu_tanh(acc[rb][0][r] * ts0) * (acc[rb][1][r] * ts1)));
        } else {
          crow[ncol[0]] = bf16_t(f32_to_bf16_bits(acc[rb][0][r] * ts0));
          if (jv[1]) crow[ncol[1]] = bf16_t(f32_to_bf16_bits(acc[rb][1][r] * ts0));
        }
      }
    }
  };
  // ni <= NR: each count of valid row blocks runs its own straight-line path
  switch (ni) {
    case 1: run(std::integral_constant<int, 1>{}); break;
    case 2: if constexpr (NR >= 2) run(std::integral_constant<int, 2>{}); break;
    case 3: if constexpr (NR >= 3) run(std::integral_constant<int, 3>{}); break;
    case 4: if constexpr (NR >= 4) run(std::integral_constant<int, 4>{}); break;
    default: run(std::integral_constant<int, 0>{}); break;
  }
}

F4Seg empty_seg() {
  F4Seg s{};
  s.nblk = 1;
  return s;
}

// the two launch shapes: decode-sized row tiles (every expert's rows fit
// one 32-row tile, 2-wave column blocks, weights 8 steps ahead) and 128-row
// tiles with 8-wave column blocks
template <int MODE, int W, int NR, int PF, int D, int BS>
hipError_t launch_shape(const F4Seg& d, const F4Seg& e, hipStream_t st) {
  constexpr int kRowsT = 32 * NR;
  const int ud = d.A ? ((d.host_rows + kRowsT - 1) / kRowsT) * d.nblk : 0;
  const int ue = e.tiles ? e.max_tiles * e.nblk : 0;
  const int total = ud + ue;
  if (total <= 0) return hipSuccess;
  const int per = (ud + kXcd - 1) / kXcd + (ue + kXcd - 1) / kXcd;
  hipLaunchKernelGGL((k_fp4mm<MODE, W, NR, PF, D, BS>), dim3(per * kXcd), dim3(W * 64), 0, st, d, e, ud, total);
  return hipGetLastError();
}

// columns per wave: 32 (gate/up pairs) or 64 (down)
int nblocks(int N, int cols_per_wave, int W) {
  const int cols = cols_per_wave * W;
  return (N + cols - 1) / cols;
}

}  // namespace

bool fp4mm_small(const Shape& sh) { return sh.T <= kFp4SmallT; }

hipError_t launch_fp4_gateup(const StreamArgs& a, const Workspace& ws, int max_tiles128, hipStream_t s) {
  const Shape& sh = a.sh;
  const bool small = fp4mm_small(sh);
  const int W = small ? 2 : 8;
  F4Seg d = empty_seg(), e = empty_seg();
  if (sh.D > 0) {
    d.A = a.x;
    d.lda = sh.H;
    d.F0 = a.fdg;
    d.F1 = a.fdu;
    d.K = sh.H;
    d.N = sh.D;
    d.C = ws.h_d;
    d.ldc = sh.D;
    d.nblk = nblocks(sh.D, 32, W);
    d.host_rows = sh.T;
    d.in_scale = a.in_scale;
  }
  if (sh.E > 0) {
    e.A = a.x;
    e.lda = sh.H;
    e.gather = ws.perm;
    e.F0 = a.fg;
    e.F1 = a.fu;
    e.K = sh.H;
    e.N = sh.I;
    e.C = ws.h;
    e.ldc = sh.I;
    e.nblk = nblocks(sh.I, 32, W);
    // T <= kFp4SmallT: an expert has at most T <= 32 rows, one tile each (the
    // active-expert list); else the 128-row tile list
    e.tiles = small ? ws.active : ws.mtiles128;
    e.n_tiles = small ? ws.meta + 1 : ws.meta + 2;
    e.max_tiles = small ? std::min(sh.E, sh.T * sh.k) : max_tiles128;
    e.in_scale = a.in_scale;
  }
  return small ? launch_shape<FM_GATEUP, 2, 1, 8, 6, 1>(d, e, s) : launch_shape<FM_GATEUP, 8, 4, 6, kBurst + 1, kBurst>(d, e, s);
}

hipError_t launch_fp4_down(const StreamArgs& a, const Workspace& ws, int max_tiles128, hipStream_t s,
                           bf16_t* yd_out) {
  const Shape& sh = a.sh;
  const bool small = fp4mm_small(sh);
  const int W = small ? 2 : 8;
  F4Seg d = empty_seg(), e = empty_seg();
  if (sh.D > 0) {
    d.A = ws.h_d;
    d.lda = sh.D;
    d.F0 = a.fdd;
    d.K = sh.D;
    d.N = sh.H;
    d.C = yd_out ? yd_out : ws.y_d;
    d.ldc = sh.H;
    d.nblk = nblocks(sh.H, 64, W);
    d.host_rows = sh.T;
    d.in_scale = a.in_scale ? a.in_scale + 2 : nullptr;
  }
  if (sh.E > 0) {
    e.A = ws.h;
    e.lda = sh.I;
    e.F0 = a.fd;
    e.K = sh.I;
    e.N = sh.H;
    e.C = ws.y;
    e.ldc = sh.H;
    e.nblk = nblocks(sh.H, 64, W);
    e.tiles = small ? ws.active : ws.mtiles128;
    e.n_tiles = small ? ws.meta + 1 : ws.meta + 2;
    e.max_tiles = small ? std::min(sh.E, sh.T * sh.k) : max_tiles128;
    e.in_scale = a.in_scale ? a.in_scale + 1 : nullptr;
  }
  return small ? launch_shape<FM_DOWN, 2, 1, 8, 6, 1>(d, e, s) : launch_shape<FM_DOWN, 8, 4, 6, kBurst + 1, kBurst>(d, e, s);
}

}  // namespace moe
