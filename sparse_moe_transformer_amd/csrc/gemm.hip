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
// Tile: 320 rows x 256 B-columns, 512 threads = 8 waves in 2 (rows) x 4
// (columns), each wave owning 160 x 64 outputs as 5 x 2 MFMA 32x32 blocks;
// two waves share each SIMD.  320 rows hold a whole expert at prefill
// (256 +- 16 rows per expert at T = 4096), so its weights are streamed by
// one M-tile instead of a full tile and a short tail tile.  For gate/up the 256 B-columns are 128 gate +
// 128 up columns at the same output positions (a wave owns 32 of each), so
// the GeGLU epilogue pairs them in registers.
//
// Pipeline: K advances in stages of 32; kStages LDS stages (36 KB each) are
// in flight.  Operand tiles go from global memory straight to LDS (buffer
// loads with the lds flag, 16 bytes per lane, no registers), issued
// kStages - 1 stages ahead, without spending VGPRs on them; each wave waits
// for its own copies of the stage about to be used, then the block meets at
// a barrier.  A wave's copies of the next stage go out one after every
// second MFMA rather than as a burst after the barrier (a burst of the 8
// waves' copies queues at the CU's address unit and stalls their MFMA
// issue).  Registers hold one 16-k sub-step of fragments ahead: a wave
// reads the next sub-step's fragments from LDS while the MFMAs of the
// current one run.
//
// LDS layouts (16-byte chunks XOR-swizzled so that every fragment read and
// every copy touches the bank groups evenly):
//   A  [320 rows][32 k]: 64 B per row, chunk c of row r at c ^ fa(r), with
//      fa(r) = (r / 4) % 4: the four rows that share a 256-byte span take
//      the same XOR, and the next four another (measured on gfx950 at the
//      full 128-bit LDS read rate, ~244 B per clock per CU, for every
//      fragment row base the tile uses; an XOR that also varies inside a
//      4-row span, such as (r / 2) % 4, measured half of it)
//   B  bf16 weights are [K, N] (N contiguous) and stay so in LDS: two halves
//      (gate / up, or columns 0-127 / 128-255) of [32 k][128 n], 256 B per k
//      row, chunk c of row k at c ^ fb(k).  The MFMA B operand (8
//      consecutive k of one column per lane) is read with the gfx950
//      transposing LDS read: in a 16-lane group, lane i names row k0 + i / 4,
//      columns 4 (i % 4) .. + 3, and receives column i of rows k0 .. k0 + 3.
//   B  FP8 weights are [K, N] e4m3fn codes: they are copied to LDS like A
//      and converted there to bf16 (exact: e4m3 has 3 mantissa bits) in the
//      bf16 layout above, so the transposing reads are shared; the fp32
//      per-matrix scale is applied in the epilogue.
// (NVFP4 weights, stored out-major, stream into registers instead: fp4mm.hip.)
// After the K loop the same LDS stages the bf16 output tile, which leaves
// the block in 16-byte row stores.
//
// Block ids are remapped so that each XCD takes an equal contiguous run of
// each segment's tiles that exist (the N-tiles of one M-tile, then the next
// M-tile of the same expert share its L2); the grid covers the worst-case
// tile list and the surplus blocks exit at once.
#include <type_traits>

#include "common.h"

namespace moe {

namespace {

constexpr int BM = kGemmBM;  // 320
constexpr int kRowBlocks = BM / 64;  // 32-row MFMA blocks per wave row (2 wave rows)
// Host-sized segments (the dense branch, all T rows) take 256-row tiles,
// except in the gate/up launch beside expert tiles, which take 320 (measured
// on one GPU at T = 4096, gate/up / down us: 26B layer 466 / 262 with 256-row
// dense tiles everywhere, 439 / 275 with 320 everywhere; the E4B dense FFN
// alone 436 / 286 against 470 / 314)
constexpr int kHostBMSmall = 256;
constexpr int BN = 256;      // B columns per tile
constexpr int BK = 32;       // k per pipeline stage
constexpr int kStages = 4;   // LDS stages in flight
constexpr int kThreads = 512;  // 8 waves: 2 (rows) x 4 (columns), 128 x 64 outputs each
constexpr int kXcd = 8;
constexpr int kAOpBytes = BM * BK * 2;          // the A tile of a stage: 20 KB
constexpr int kBOpBytes = BN * BK * 2;          // the B tile of a stage: 16 KB
constexpr int kStageBytes = kAOpBytes + kBOpBytes;  // A, then B
constexpr int kACopies = 3;                     // A copies per wave per stage (1 KB each; 20 of the 24 land in A)
constexpr int kDummyBytes = 4096;               // where the 4 surplus A copies land (never read)
constexpr int kEarlyMaxK = 4096;                // plain (down) launches up to this K meet before a stage's first sub-step

enum { MODE_PLAIN_BF16 = 0, MODE_PLAIN_F32 = 1, MODE_GATEUP = 2 };
enum { W_BF16 = 0, W_FP8 = 2 };

struct Seg {
  const bf16_t* A;
  int lda;
  const int32_t* gather;  // routed gate/up: tile row r reads A row gather[row0 + r]
  const bf16_t* B0;       // bf16 [G][K][ldb] (gate or the only matrix)
  const bf16_t* B1;       // up (gate/up mode)
  long long b_gstride;    // elements between groups
  int ldb;
  Fp8Mat Q0, Q1;          // FP8 [G][K][ldb] e4m3fn codes (group stride b_gstride), [G] scales
  const float* in_scale;  // NVFP4 activations: the A operand's global scale (device), or null
  int K;
  int N;                  // output columns
  void* C;
  int ldc;
  int n_ntiles;           // output column tiles
  int host_rows;          // host-sized segment: number of rows
  int host_bm;            // ... in tiles of this many rows (<= BM)
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

typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint32_t lds_u32;
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef short s16x4_t __attribute__((ext_vector_type(4)));

// A per-lane byte offset beyond every buffer resource's range (2^31 - 1
// bytes); the uniform k-step offsets added to it (at most 32 MiB: K and a
// B row are at most 4096 elements) cannot wrap it back into range.
constexpr int kOutOfRange = int(0x80000000u);

// Buffer resource of a wave-uniform base pointer (moved to scalar
// registers), no stride, 2^31 - 1 bytes of range.
__device__ __forceinline__ i32x4_t rsrc4(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  i32x4_t r;
  r[0] = int(__builtin_amdgcn_readfirstlane(uint32_t(v)));
  r[1] = int(__builtin_amdgcn_readfirstlane(uint32_t(v >> 32)));
  r[2] = 0x7FFFFFFF;
  r[3] = 0x00020000;
  return r;
}

// Global -> LDS copy of 16 bytes per lane (gfx950 buffer load with the lds
// flag): the 16 bytes at (rsrc, voffset + soffset) of lane i land at LDS
// byte address lds + 16 i; lds is wave-uniform (it goes to M0).  The copy
// has no register result.  Written as asm so that the compiler does not
// track it: it would otherwise wait for every copy in flight (including the
// stages prefetched ahead) before any transposing LDS read; the kernel waits
// for the copies itself (wait_counts before each barrier).
__device__ __forceinline__ void copy_b128_to_lds(i32x4_t rsrc, uint32_t lds, int voffset, int soffset) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(lds), "v"(voffset), "s"(rsrc),
               "s"(soffset)
               : "memory");
}

// the same with 4 bytes per lane (lane i at lds + 4 i)
__device__ __forceinline__ void copy_b32_to_lds(i32x4_t rsrc, uint32_t lds, int voffset, int soffset) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds" ::"s"(lds), "v"(voffset), "s"(rsrc),
               "s"(soffset)
               : "memory");
}

// s_waitcnt with only vmcnt <= VM and lgkmcnt <= LGKM (expcnt not waited)
template <int VM, int LGKM>
__device__ __forceinline__ void wait_counts() {
  static_assert(VM >= 0 && VM < 64 && LGKM >= 0 && LGKM < 16, "counter range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (LGKM << 8));
}

// Workgroup barrier without a memory fence: the waits above it are explicit
// (a fenced barrier would also wait for the copies still in flight for later
// stages).  The memory clobber keeps LDS accesses on their side of it.
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// swizzled chunk positions (see the header)
__device__ __forceinline__ int fa(int r) { return (r >> 2) & 3; }
__device__ __forceinline__ int fb(int k) { return 4 * (k & 3); }

// EARLY (bf16 tiles): the block meets before a stage's first sub-step
// instead of between its two (see the K loop)
template <int MODE, int WF, bool EARLY>
__global__ __launch_bounds__(kThreads, 1) void k_gemm(Seg s0, Seg s1, int units0, int units_total) {
  // ---- logical tile of this block (XCD-aware remap over the real tiles) ----
  // Each segment is spread evenly over the XCDs on its own (its tiles can
  // differ in K from the other segment's): XCD x takes a contiguous run of
  // the host-sized segment's tiles, then a contiguous run of the grouped
  // segment's tiles that exist (their count is read from the device list).
  // The grid covers the worst case; surplus blocks exit at once.
  const int n1 = s1.mtiles ? (*s1.n_mtiles) * s1.n_ntiles * s1.ksplit : units_total - units0;
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
  const Seg S = second ? s1 : s0;
  int uu = second ? u - units0 : u;
  const int ks = uu % S.ksplit;
  uu /= S.ksplit;
  const int mt = uu / S.n_ntiles;
  const int nt = uu % S.n_ntiles;
  int grp = 0, row0, rows;
  if (S.mtiles) {
    grp = S.mtiles[4 * mt];
    row0 = S.mtiles[4 * mt + 1];
    rows = S.mtiles[4 * mt + 2];
  } else {
    row0 = mt * S.host_bm;
    rows = min(S.host_bm, S.host_rows - row0);
  }
  const int K = S.K, N = S.N;
  // output columns of this tile: gate/up pairs 128 gate with 128 up columns
  constexpr int OUTN = (MODE == MODE_GATEUP) ? BN / 2 : BN;
  const int n0 = nt * OUTN;

  // LDS: bf16 weights: a ring of four K stages, each A then B.  FP8 /
  // NVFP4: a deeper ring of A and the raw codes of B (their copies run
  // kDepth stages ahead), then two bf16 B tiles decoded from the raw codes
  // (one is written while the other is read).  After the K loop the same
  // bytes stage the output tile.
  constexpr int kRaw = (WF == W_FP8) ? 8192 : 0;
  constexpr int kDepth = kStages;
  constexpr int kStageStride = (WF == W_BF16) ? kStageBytes : kAOpBytes + kRaw;  // one ring slot
  constexpr int kBArea = kDepth * kStageStride;                                // FP8: the two B tiles
  constexpr int kDummy = kBArea + ((WF == W_BF16) ? 0 : 2 * kBOpBytes);        // surplus A copies
  constexpr int kStageArea = kDummy + kDummyBytes;
  constexpr int SP = OUTN * 2 + 16;  // staging row pitch (bytes); half the tile's rows at a time
  constexpr int kSmem = kStageArea > (BM / 2) * SP ? kStageArea : (BM / 2) * SP;
  static_assert(kSmem <= 163840, "LDS per block");
  __shared__ __attribute__((aligned(1024))) unsigned char lds[kSmem];
  lds_u8* const lds3 = (lds_u8*)(lds);
  const uint32_t lds_base = uint32_t(reinterpret_cast<uintptr_t>(lds3));  // LDS byte address of the stages

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int wm = wave >> 2, wn = wave & 3;

  // ---- A copies: copy c = 3 w + q of wave w fills rows 16 c .. + 15 of a
  // stage (c < 20; copies 20 .. 23 land in a dummy area, out of range);
  // lane: row 16 c + lane / 4, slot lane % 4 <- global chunk slot ^ fa.
  // Lanes of rows past the tile's end get an offset beyond the resource's
  // range (kOutOfRange):
  // the copy returns zeros without touching memory, and every copy is still
  // issued, so the wait counts below stay constants.  Those rows' results
  // are dropped.
  const i32x4_t arsrc = rsrc4(S.A);
  int aoff[kACopies];
#pragma unroll
  for (int q = 0; q < kACopies; ++q) {
    const int r = 16 * (kACopies * wave + q) + (lane >> 2);  // r >= BM: a surplus copy (r >= rows)
    const int rr = r < rows ? r : 0;
    const uint32_t gr = S.gather ? uint32_t(S.gather[row0 + rr]) : uint32_t(row0 + rr);
    aoff[q] = r < rows ? int((gr * uint32_t(S.lda) + uint32_t(((lane & 3) ^ fa(r)) * 8)) * 2u) : kOutOfRange;
  }

  // ---- B.  bf16: waves 4h .. 4h+3 copy half h (gate / up, or the column
  // halves); wave w, copy q: k rows 8 (w % 4) + 4q .. + 3; lane: row +
  // lane / 16, slot lane % 16 <- global chunk slot ^ fb.  Columns past N
  // are out of range, like A's rows past the tile.
  const int bh = wave >> 2;
  i32x4_t brsrc = rsrc4(S.B0);
  int boff[2] = {0, 0};
  const uint32_t brow = uint32_t(S.ldb) * 2;  // bytes per k row
  // FP8 / NVFP4: each stage's raw codes are copied into the stage's raw area
  // (DMA like A, so the compiler tracks no weight loads in the K loop) and
  // decoded there to the bf16 B layout two stages ahead of their use.
  //   FP8: thread t copies 16 codes of half t / 256, k row (t % 256) / 8,
  //        columns 16 (t % 8) .. + 15 to raw + 16 t.
  //   NVFP4: waves 0-3: thread t copies the 16 code bytes (32 k) of B-tile
  //        column t to raw + 16 t; waves 4-7: the dword of column t - 256's
  //        scales that holds this stage's two, to raw + 4096 + 4 (t - 256).
  // Columns past N are out of range (zeros); they only feed output columns
  // that are never stored.
  i32x4_t rrsrc = rsrc4(S.A);
  int roff = kOutOfRange;
  if (WF == W_FP8) {
    const int h = tid >> 8, t2 = tid & 255, k = t2 >> 3, lc = (t2 & 7) * 16;
    const uint8_t* q = (MODE == MODE_GATEUP && h) ? S.Q1.q : S.Q0.q;
    const int col = (MODE == MODE_GATEUP) ? n0 + lc : n0 + 128 * h + lc;
    rrsrc = rsrc4(q + grp * S.b_gstride);
    roff = col < N ? int(uint32_t(k) * uint32_t(S.ldb) + uint32_t(col)) : kOutOfRange;
  }
  if (WF == W_BF16) {
    const bf16_t* Bm = S.B0;
    int cbase = n0 + 128 * bh;
    if (MODE == MODE_GATEUP) {
      Bm = bh ? S.B1 : S.B0;
      cbase = n0;
    }
    brsrc = rsrc4(Bm + grp * S.b_gstride);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int k = 8 * (wave & 3) + 4 * q + (lane >> 4);
      const int col = cbase + ((lane & 15) ^ fb(k)) * 8;
      boff[q] = col < N ? int(uint32_t(k) * brow + uint32_t(col) * 2u) : kOutOfRange;
    }
  }

  // K-stages of this tile's slice; stage indices past the last are clamped
  // (their copies land in a buffer that is never read), so every stage
  // issues the same number of memory instructions and the waits below are
  // constants.
  const int nk_all = K / BK;
  const int kt0 = ks * nk_all / S.ksplit;
  const int nk = (ks + 1) * nk_all / S.ksplit - kt0;

  // raw codes of stage st into its raw area (one copy per lane)
  auto issue_raw = [&](int st) {
    const int kidx = kt0 + min(st, nk - 1);
    const uint32_t rb = lds_base + uint32_t((st % kDepth) * kStageStride + kAOpBytes);
    if (WF == W_FP8) {
      copy_b128_to_lds(rrsrc, rb + wave * 1024, roff, int(uint32_t(kidx * BK) * uint32_t(S.ldb)));
    }
  };
  // copy n of stage st into its LDS ring slot: n < kACopies an A copy, then
  // the two B copies (bf16) or the raw codes (FP8)
  auto issue_one = [&](int st, int n) {
    const int kk = (kt0 + min(st, nk - 1)) * BK;
    const uint32_t sbase_addr = lds_base + uint32_t((st % kDepth) * kStageStride);
    if (n < kACopies) {
      const int c = kACopies * wave + n;  // wave-uniform
      const uint32_t dst = c < BM / 16 ? sbase_addr + c * 1024 : lds_base + uint32_t(kDummy + (c - BM / 16) * 1024);
      copy_b128_to_lds(arsrc, dst, aoff[n], kk * 2);
    } else if (WF == W_BF16) {
      const int q = n - kACopies;
      copy_b128_to_lds(brsrc, sbase_addr + kAOpBytes + bh * (kBOpBytes / 2) + (8 * (wave & 3) + 4 * q) * 256,
                       boff[q], int(uint32_t(kk) * brow));
    } else {
      issue_raw(st);
    }
  };
  auto issue = [&](int st) {  // every copy of stage st
#pragma unroll
    for (int n = 0; n < kACopies + (WF == W_BF16 ? 2 : 0); ++n) issue_one(st, n);
  };
  // raw codes of stage st (landed) -> the stage's bf16 B tile
  auto decode = [&](int st) {
    lds_u8* sb = lds3 + (st % kDepth) * kStageStride;  // A, then the raw codes at kAOpBytes
    lds_u8* bt = lds3 + kBArea + (st & 1) * kBOpBytes;  // this stage's bf16 B tile
    if (WF == W_FP8) {
      const int h = tid >> 8, t2 = tid & 255, k = t2 >> 3, c0 = (t2 & 7) * 2;
      const u32x4_t q = *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>(sb + kAOpBytes + tid * 16);
      u32x4_t w[2];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        // bytes 0,1 and 2,3 of q[d] -> bf16 pairs (gfx950 scaled conversion, unit scale: exact)
        w[d >> 1][2 * (d & 1)] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[d], 1.0f, false));
        w[d >> 1][2 * (d & 1) + 1] =
            __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q[d], 1.0f, true));
      }
      lds_u8* row = bt + h * (kBOpBytes / 2) + k * 256;
#pragma unroll
      for (int c = 0; c < 2; ++c)
        *reinterpret_cast<__attribute__((address_space(3))) u32x4_t*>(row + (((c0 + c) ^ fb(k)) << 4)) = w[c];
    }
  };

  // ---- fragment addresses of this wave's 32 x 32 blocks (bytes in a stage)
  // A block i: rows wm*BM/2 + 32i; lane row (lane & 31), k half lane / 32
  const int hl = lane >> 5;
  int afr[kRowBlocks][2];
#pragma unroll
  for (int i = 0; i < kRowBlocks; ++i) {
    const int m = wm * (BM / 2) + 32 * i + (lane & 31);
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) afr[i][sb] = m * 64 + (((2 * sb + hl) ^ fa(m)) << 4);
  }
  // B block j: gate/up: gate (j = 0) and up (j = 1) columns wn*32; else
  // columns wn*64 + 32j.  bf16 (transposing reads): 16-lane group g covers
  // columns +16 (g % 2), k rows +8 (g / 2); lane i of the group names row
  // i / 4, columns 4 (i % 4) .. + 3.  The sub-step and the second 4-row read
  // are immediate offsets.
  int bfr[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int gcol = (MODE == MODE_GATEUP) ? 128 * j + wn * 32 : wn * 64 + 32 * j;  // B-tile column 0..255
    const int h = gcol >> 7, lc = gcol & 127;
    const int g = lane >> 4, i16 = lane & 15, qq = i16 & 3, mr = i16 >> 2;
    const int colb = lc + 16 * (g & 1);
    const int krow = 8 * (g >> 1) + mr;  // fb(krow + 16 s + 4 r) == fb(mr)
    bfr[j] = h * (kBOpBytes / 2) + krow * 256 + ((((colb >> 3) + (qq >> 1)) ^ fb(mr)) << 4) + (qq & 1) * 8;
  }

  // Row blocks of this wave inside the tile's rows (a prefix of the 5), and
  // whether its columns are inside the matrix: both are wave-uniform, and
  // each count runs its own straight-line path (same barriers in all), so
  // the ragged last M-tile of an expert and the last N-tile cost only their
  // valid part.
  const int wcol0 = (MODE == MODE_GATEUP) ? n0 + wn * 32 : n0 + wn * 64;
  int ni = (rows - wm * (BM / 2) + 31) / 32;
  ni = ni < 0 ? 0 : (ni > kRowBlocks ? kRowBlocks : ni);
  if (wcol0 >= N) ni = 0;
  ni = __builtin_amdgcn_readfirstlane(ni);

  float ts0 = 1.f, ts1 = 1.f;
  if (WF == W_FP8) {
    ts0 = S.Q0.tscale[grp];
    if (MODE == MODE_GATEUP) ts1 = S.Q1.tscale[grp];
  }
  if (S.in_scale) {  // quantised activations: their global scale joins the weights'
    const float si = *S.in_scale;
    ts0 *= si;
    ts1 *= si;
  }

  auto run = [&](auto ni_c) {
    constexpr int NI = decltype(ni_c)::value;
    f32x16_t acc[kRowBlocks][2];
#pragma unroll
    for (int i = 0; i < kRowBlocks; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // Fragments of one 16-k sub-step of a stage for this wave's blocks.
    struct Frags {
      bf16x8_t a[kRowBlocks], b[2];
    };
    // abase: the stage's A tile; bbase: its B tile; sb: sub-step 0 or 1
    auto read_sub = [&](const lds_u8* abase, const lds_u8* bbase, int sb, Frags& f) {
      if (NI == 0) return;
#pragma unroll
      for (int i = 0; i < NI; ++i)
        f.a[i] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8_t*>(abase + afr[i][sb]);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const lds_u8* p = bbase + bfr[j] + sb * 16 * 256;
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(p));
        const s16x4_t hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)(p + 4 * 256));
        const s16x4_t v[2] = {lo, hi};
        f.b[j] = __builtin_bit_cast(bf16x8_t, v);
      }
    };
    auto mfmas = [&](const Frags& f) {
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
    };

    // Memory instructions per stage per lane: bf16 5 copies (A 3 + B 2);
    // FP8 4 copies (A 3 + the raw codes).
    constexpr int kPerStage = (WF == W_BF16) ? kACopies + 2 : kACopies + 1;
    auto abase_of = [&](int st) -> const lds_u8* { return lds3 + (st % kDepth) * kStageStride; };
    auto bbase_of = [&](int st) -> const lds_u8* {
      return (WF == W_BF16) ? abase_of(st) + kAOpBytes : lds3 + kBArea + (st & 1) * kBOpBytes;
    };
    auto stage_in = [&](int st) {
      if (WF != W_BF16) issue_raw(st);
      issue(st);
    };
    // the fragment reads ride ahead of the MFMAs they do not feed: keep them
    // above (the scheduler would otherwise sink them below and serialise LDS
    // latency with the matrix work); while this wave feeds the matrix unit it
    // takes issue priority over the SIMD's other wave, which is then reading
    // fragments or copying
    auto mma = [&](const Frags& f) {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(1);
      mfmas(f);
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
    };
    // the same with copies n0 .. n1 - 1 of stage st spread between the MFMAs
    // (one after every second MFMA, the rest after the last): issued as a
    // burst right after the barrier, the 8 waves' 40 copies queue at the
    // CU's address unit together and hold the waves' MFMA issue behind them
    auto mma_copies = [&](const Frags& f, int st, int n0, int n1) {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
          if (j == 1 && n0 + i < n1) {
            __builtin_amdgcn_sched_barrier(0);
            issue_one(st, n0 + i);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
#pragma unroll
      for (int n = n0 + NI; n < n1; ++n) issue_one(st, n);
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
    };
    Frags f0, f1;  // sub-step 0 and sub-step 1 of a stage
#pragma unroll
    for (int st = 0; st < kDepth; ++st) stage_in(st);
    // Step kt: f0 holds stage kt's first sub-step.  Its second is read while
    // the first's MFMAs run; then the block meets (every wave has read all of
    // stage kt, so its LDS slot is refilled with stage kt + kDepth) and the
    // first sub-step of stage kt + 1 is read while the second's MFMAs run.
    // Registers hold one sub-step ahead, not a stage.
    auto step = [&](int kt) {
      read_sub(abase_of(kt), bbase_of(kt), 1, f1);
      if (WF == W_BF16 && EARLY) {
        // this wave has read all of stage kt once its second sub-step's
        // fragments are in registers, so the block meets before the first
        // sub-step's MFMAs and the copies of stage kt + kDepth are spread
        // over both sub-steps (measured at T = 4096 against meeting between
        // them: 26B gate/up ~2.5%, E4B gate/up ~4% and 26B down ~2% faster;
        // the E4B down GEMM, K = 10240 on 160 tiles, 6% slower, so launches
        // of plain tiles with K past kEarlyMaxK keep the later meeting)
        wait_counts<(kDepth - 2) * kPerStage, 0>();  // stage kt + 1 landed; stage kt's fragments read
        block_barrier();
        mma_copies(f0, kt + kDepth, 0, 3);
        read_sub(abase_of(kt + 1), bbase_of(kt + 1), 0, f0);
        mma_copies(f1, kt + kDepth, 3, kPerStage);
        return;
      }
      mma(f0);
      if (WF == W_BF16) {
        // bf16: copies run kDepth stages ahead, issued between the MFMAs of
        // the second sub-step
        wait_counts<(kDepth - 2) * kPerStage, 0>();  // stage kt + 1 landed; stage kt's fragments read
        block_barrier();
        read_sub(abase_of(kt + 1), bbase_of(kt + 1), 0, f0);
        mma_copies(f1, kt + kDepth, 0, kPerStage);
        return;
      } else {
        // FP8 / NVFP4: stage kt + 2's raw codes are decoded in this step;
        // stages kt + 3 .. kt + kDepth - 1 stay in flight across the barrier
        wait_counts<(kDepth - 3) * kPerStage, 0>();  // stage kt + 2 landed; this wave's decode of kt + 1 written
        block_barrier();
        decode(kt + 2);
      }
      read_sub(abase_of(kt + 1), bbase_of(kt + 1), 0, f0);
      mma_copies(f1, kt + kDepth, 0, kPerStage);
    };
    if (WF == W_BF16) {
      wait_counts<(kDepth - 1) * kPerStage, 0>();  // stage 0 landed (this wave's copies)
      block_barrier();
    } else {
      wait_counts<(kDepth - 1) * kPerStage, 0>();  // stage 0 landed
      block_barrier();
      decode(0);
      wait_counts<(kDepth - 2) * kPerStage, 0>();  // stage 1 landed; decode of 0 written
      block_barrier();
      decode(1);
      wait_counts<(kDepth - 2) * kPerStage, 0>();  // decode of 1 written (no new copies)
      block_barrier();                             // every wave's decode of stage 0 is in LDS
    }
    read_sub(abase_of(0), bbase_of(0), 0, f0);
    for (int kt = 0; kt < nk; ++kt) step(kt);
    wait_counts<0, 0>();  // no copy may still be landing when LDS is reused

    // ---- epilogue: lane holds column (lane & 31); rows 8(r/4) + 4(lane/32) + r%4
    if (MODE == MODE_PLAIN_F32) {  // router logits: fp32, written directly
#pragma unroll
      for (int i = 0; i < NI; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wm * (BM / 2) + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (row >= rows) continue;
          const long long orow = (long long)(row0 + row) * S.ldc + ks * S.c_slice;
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int col = wcol0 + 32 * j + (lane & 31);
            if (col < N) reinterpret_cast<float*>(S.C)[orow + col] = acc[i][j][r] * ts0;
          }
        }
      }
      return;
    }
    // bf16 outputs go through LDS so that the tile leaves in 16-byte stores,
    // half the tile's rows at a time (the waves of wave row h stage them).
    // The stores are nontemporal: the output rows are read once, by the next
    // launch, and would otherwise take L2 lines from the operands still
    // streaming (T = 4096: gate/up ~-6 us, down ~-12 us; the combine then
    // finds fewer of y's rows in the caches, +5 us; step -4 to -6 us).
    // Neighbouring lanes swap values (DPP) so that each lane writes pairs of
    // adjacent columns: even lanes rows r = 2q, odd lanes rows r = 2q + 1.
    const bool odd = lane & 1;
    constexpr int CPR = OUTN / 8;  // 16-byte chunks per staged row
    bf16_t* C = reinterpret_cast<bf16_t*>(S.C);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      block_barrier();  // h = 0: every wave's last fragments are read; h = 1: the first half has left
      if (wm == h) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
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
              const int row = i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);  // in the half
              const uint32_t packed = odd ? (recv | (vb[2 * q + 1] << 16)) : (vb[2 * q] | (recv << 16));
              *reinterpret_cast<__attribute__((address_space(3))) uint32_t*>(lds3 + row * SP + cpair * 2) = packed;
            }
          }
        }
      }
      __syncthreads();
      for (int c = tid; c < (BM / 2) * CPR; c += kThreads) {
        const int hrow = c / CPR, ch = c % CPR;
        const int row = h * (BM / 2) + hrow;
        const int col = n0 + ch * 8;
        if (row < rows && col < N)
          __builtin_nontemporal_store(
              *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t*>(lds3 + hrow * SP + ch * 16),
              reinterpret_cast<u32x4_t*>(C + (long long)(row0 + row) * S.ldc + ks * S.c_slice + col));
      }
    }
  };
  switch (ni) {
    case 5: run(std::integral_constant<int, 5>{}); break;
    case 4: run(std::integral_constant<int, 4>{}); break;
    case 3: run(std::integral_constant<int, 3>{}); break;
    case 2: run(std::integral_constant<int, 2>{}); break;
    case 1: run(std::integral_constant<int, 1>{}); break;
    default: run(std::integral_constant<int, 0>{}); break;
  }
}

Seg empty_seg() {
  Seg s{};
  s.n_ntiles = 1;
  s.ksplit = 1;
  s.host_bm = BM;
  return s;
}

template <int MODE, int WF, bool EARLY = MODE == MODE_GATEUP>
hipError_t launch(const Seg& a, const Seg& b, int units_a, int units_b, hipStream_t st) {
  const int total = units_a + units_b;
  if (total <= 0) return hipSuccess;
  // slots per XCD: both segments' shares (the kernel's remap)
  const int per = (units_a + kXcd - 1) / kXcd + (units_b + kXcd - 1) / kXcd;
  hipLaunchKernelGGL((k_gemm<MODE, WF, EARLY>), dim3(per * kXcd), dim3(kThreads), 0, st, a, b, units_a, total);
  return hipGetLastError();
}

int host_units(const Seg& s) { return ((s.host_rows + s.host_bm - 1) / s.host_bm) * s.n_ntiles * s.ksplit; }

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
    d.Q0 = a.qdg;
    d.Q1 = a.qdu;
    d.in_scale = a.in_scale;
    d.K = sh.H;
    d.N = sh.D;
    d.C = ws.h_d;
    d.ldc = sh.D;
    d.n_ntiles = (sh.D + BN / 2 - 1) / (BN / 2);
    d.host_rows = sh.T;
    d.host_bm = sh.E > 0 ? BM : kHostBMSmall;
  }
  // routed experts: rows gathered through perm
  e.A = a.x;
  e.lda = sh.H;
  e.gather = ws.perm;
  e.B0 = a.wg;
  e.B1 = a.wu;
  e.b_gstride = (long long)sh.H * sh.I;
  e.ldb = sh.I;
  e.Q0 = a.qg;
  e.Q1 = a.qu;
  e.in_scale = a.in_scale;
  e.K = sh.H;
  e.N = sh.I;
  e.C = ws.h;
  e.ldc = sh.I;
  e.n_ntiles = (sh.I + BN / 2 - 1) / (BN / 2);
  e.mtiles = sh.E > 0 ? ws.mtiles : nullptr;  // no experts: an empty second segment
  e.n_mtiles = ws.meta;
  e.max_mtiles = sh.E > 0 ? max_mtiles : 0;
  const int ud = sh.D > 0 ? host_units(d) : 0;
  if (a.fp8) return launch<MODE_GATEUP, W_FP8>(d, e, ud, grouped_units(e), s);
  return launch<MODE_GATEUP, W_BF16>(d, e, ud, grouped_units(e), s);
}

hipError_t launch_gemm_down(const StreamArgs& a, const Workspace& ws, int max_mtiles, hipStream_t s,
                            bf16_t* yd_out) {
  const Shape& sh = a.sh;
  Seg d = empty_seg(), e = empty_seg();
  if (sh.D > 0) {
    d.A = ws.h_d;
    d.lda = sh.D;
    d.B0 = a.dd;
    d.ldb = sh.H;
    d.Q0 = a.qdd;
    d.in_scale = a.in_scale ? a.in_scale + 2 : nullptr;
    d.K = sh.D;
    d.N = sh.H;
    d.C = yd_out ? yd_out : ws.y_d;
    d.ldc = sh.H;
    d.n_ntiles = (sh.H + BN - 1) / BN;
    d.host_rows = sh.T;
    d.host_bm = kHostBMSmall;
  }
  e.A = ws.h;
  e.lda = sh.I;
  e.B0 = a.wd;
  e.b_gstride = (long long)sh.I * sh.H;
  e.ldb = sh.H;
  e.Q0 = a.qd;
  e.in_scale = a.in_scale ? a.in_scale + 1 : nullptr;
  e.K = sh.I;
  e.N = sh.H;
  e.C = ws.y;
  e.ldc = sh.H;
  e.n_ntiles = (sh.H + BN - 1) / BN;
  e.mtiles = sh.E > 0 ? ws.mtiles : nullptr;
  e.n_mtiles = ws.meta;
  e.max_mtiles = sh.E > 0 ? max_mtiles : 0;
  const int ud = sh.D > 0 ? host_units(d) : 0;
  if (a.fp8) return launch<MODE_PLAIN_BF16, W_FP8>(d, e, ud, grouped_units(e), s);
  const int kmax = std::max(d.A ? d.K : 0, e.mtiles ? e.K : 0);
  if (kmax <= kEarlyMaxK) return launch<MODE_PLAIN_BF16, W_BF16, true>(d, e, ud, grouped_units(e), s);
  return launch<MODE_PLAIN_BF16, W_BF16, false>(d, e, ud, grouped_units(e), s);
}

}  // namespace moe
