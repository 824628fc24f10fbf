// Router of the MoE block and the expert grouping of its (token, slot) pairs.
//
// Router (archdb page "Gemma-4-26B-A4B": gating function softmax; selected
// expert weights renormalized to sum to 1; 8 of 128 routed experts per
// token): z = x . W_r (+ b), select the top-k logits (equal logits: lower id
// first), p = softmax(z) over all experts, w = p_S / sum(p_S).  Each token's
// set is written in ascending expert id with its weights aligned.
//
// Grouping: counts[e], offsets = exclusive scan, perm = token ids grouped by
// ascending expert and ascending token inside an expert, pos[t, j] = row of
// slot (t, j).  The rank of a token inside its expert comes from a 64-bit
// membership mask per (64-token block, expert) and a popcount, so the result
// is a deterministic function of topk_idx (no atomics decide positions).
//
// Two routes:
//   T <= 64: partial logits of 16 K-slices, or 32 where 16 do not fit the
//     launch shape (route_small_config; many small blocks,
//     so W_r streams at full bandwidth); the last slice block of a token
//     group sums the slices in fixed order and routes the group
//     (route_dev.h).
//   large T: split-K logits (MFMA tiles when E % 128 == 0, else an FMA
//     kernel), a top-k kernel that sums the K-slices in fixed order.
// Grouping (any T): per-64-token membership masks, a per-expert scan over
// the token blocks, and the scatter (which also rebuilds the expert offsets
// and the tile lists).
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "route_dev.h"

namespace moe {

namespace {

constexpr int kThreads = 256;

// Block-wide exclusive scan of one int per thread (BLOCK threads).
template <int BLOCK>
__device__ int block_exclusive_scan(int v, int* scratch /* [BLOCK/kWave + 1] */, int& total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  int incl = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += o;
  }
  if (lane == kWave - 1) scratch[wid] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < BLOCK / kWave; ++w) {
      const int c = scratch[w];
      scratch[w] = run;
      run += c;
    }
    scratch[BLOCK / kWave] = run;
  }
  __syncthreads();
  const int excl = scratch[wid] + incl - v;
  total = scratch[BLOCK / kWave];
  __syncthreads();
  return excl;
}

// Block-wide exclusive scan of four ints per thread in one pass.
template <int BLOCK>
__device__ int4 block_exclusive_scan4(int4 v, int4* scratch /* [BLOCK/kWave + 1] */, int4& total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  int4 incl = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int ox = __shfl_up(incl.x, off, kWave);
    const int oy = __shfl_up(incl.y, off, kWave);
    const int oz = __shfl_up(incl.z, off, kWave);
    const int ow = __shfl_up(incl.w, off, kWave);
    if (lane >= off) {
      incl.x += ox;
      incl.y += oy;
      incl.z += oz;
      incl.w += ow;
    }
  }
  if (lane == kWave - 1) scratch[wid] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int4 run = make_int4(0, 0, 0, 0);
    for (int w = 0; w < BLOCK / kWave; ++w) {
      const int4 c = scratch[w];
      scratch[w] = run;
      run.x += c.x;
      run.y += c.y;
      run.z += c.z;
      run.w += c.w;
    }
    scratch[BLOCK / kWave] = run;
  }
  __syncthreads();
  const int4 base = scratch[wid];
  total = scratch[BLOCK / kWave];
  __syncthreads();
  return make_int4(base.x + incl.x - v.x, base.y + incl.y - v.y, base.z + incl.z - v.z, base.w + incl.w - v.w);
}

// Given counts[e] (one per thread e < E), write counts, offsets, the MFMA
// tile lists (tiles of kGemmBM rows and of kFp4BM rows) and the
// active-expert list; returns the thread's offset.  Called by one whole
// block of BLOCK >= E threads.
template <int BLOCK>
__device__ int build_offsets_and_tiles(const int cnt_e, int E, const Workspace& ws, int* /*unused*/) {
  __shared__ int4 scratch4[BLOCK / kWave + 1];
  const int e = threadIdx.x;
  const int c = (e < E) ? cnt_e : 0;
  const int nm = (c + kGemmBM - 1) / kGemmBM;
  const int nm2 = (c + kFp4BM - 1) / kFp4BM;
  int4 total;
  const int4 ex = block_exclusive_scan4<BLOCK>(make_int4(c, nm, c > 0 ? 1 : 0, nm2), scratch4, total);
  const int off = ex.x;
  if (e < E) {
    ws.counts[e] = c;
    ws.offsets[e] = off;
  }
  if (e == 0) {
    ws.offsets[E] = total.x;
    ws.meta[0] = total.y;
    ws.meta[1] = total.z;
    ws.meta[2] = total.w;
  }
  for (int m = 0; m < nm; ++m) {
    int32_t* t = ws.mtiles + 4 * (ex.y + m);
    t[0] = e;
    t[1] = off + m * kGemmBM;
    t[2] = min(kGemmBM, c - m * kGemmBM);
    t[3] = 0;
  }
  for (int m = 0; m < nm2; ++m) {
    int32_t* t = ws.mtiles128 + 4 * (ex.w + m);
    t[0] = e;
    t[1] = off + m * kFp4BM;
    t[2] = min(kFp4BM, c - m * kFp4BM);
    t[3] = 0;
  }
  if (c > 0) {
    int32_t* t = ws.active + 4 * ex.z;
    t[0] = e;
    t[1] = off;
    t[2] = c;
    t[3] = 0;
  }
  return off;
}

// ---------------------------------------------------------------------------
// small T (<= 64): the K-sliced router of route_dev.h
// ---------------------------------------------------------------------------

template <int CW>
__global__ __launch_bounds__(kThreads) void k_route_part(Shape sh, int slice_rows, int TB, const bf16_t* __restrict__ x,
                                                        const bf16_t* __restrict__ wr, const float* __restrict__ bias,
                                                        Workspace ws) {
  route_slice<CW>(sh, slice_rows, TB, int(gridDim.x), blockIdx.x, blockIdx.y, x, wr, bias, ws);
}

// ---------------------------------------------------------------------------
// large T
// ---------------------------------------------------------------------------

// FMA router logits for shapes the MFMA tiles do not cover: one output per
// thread, written as the single K-slice.
__global__ __launch_bounds__(kThreads) void k_router_logits_fma(Shape sh, const bf16_t* __restrict__ x,
                                                               const bf16_t* __restrict__ wr,
                                                               float* __restrict__ logits) {
  const long long o = blockIdx.x * (long long)kThreads + threadIdx.x;
  if (o >= (long long)sh.T * sh.E) return;
  const int e = int(o % sh.E);
  const long long t = o / sh.E;
  const bf16_t* xr = x + t * sh.H;
  float s = 0.f;
  for (int kk = 0; kk < sh.H; ++kk) s += bf16_to_f32(xr[kk]) * bf16_to_f32(wr[(long long)kk * sh.E + e]);
  logits[o] = s;
}

// one wave per token: sum the K-slices of its logits in order (+ bias), route
__global__ __launch_bounds__(kThreads) void k_topk(Shape sh, int nslices, const float* __restrict__ bias,
                                                  Workspace ws) {
  const int wid = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * (kThreads / kWave) + wid;
  __shared__ float zs[kThreads / kWave][256];
  if (t >= sh.T) return;
  const int E = sh.E;
  const size_t slice = size_t(sh.T) * E;
  for (int e = lane; e < E; e += kWave) {
    const float* p = ws.logits + size_t(t) * E + e;
    // every slice's load in flight before the ordered sum (nslices <=
    // kRouterSlices: launch_route_large caps it)
    float v[kRouterSlices];
#pragma unroll
    for (int j = 0; j < kRouterSlices; ++j) v[j] = j < nslices ? p[j * slice] : 0.f;
    float z = 0.f;
#pragma unroll
    for (int j = 0; j < kRouterSlices; ++j) z += v[j];
    if (bias) z += bias[e];
    zs[wid][e] = z;
  }
  // the wave reads back only its own row: no block barrier needed
  wave_route_token(zs[wid], E, sh.k, ws.topk_idx + size_t(t) * sh.k, ws.topk_w + size_t(t) * sh.k);
}

// Large-T router with E = 128 or 256: one block of 4 waves per 16 or 32
// tokens computes their logits over all of K with v_mfma_f32_32x32x16_bf16 and
// routes them, so no partial logits go through memory.  Per 64-k step the
// x rows ([32][64] bf16, 128 B rows) and the W_r rows ([64][E], split in
// 128-column halves of 256 B rows) go global -> LDS by DMA (buffer loads
// with the lds flag) three steps ahead; 16-byte chunks are XOR-swizzled as
// in the grouped GEMM tiles (x: chunk c of row r at c ^ ((r / 2) % 8); W_r: chunk
// c of k row at c ^ 4 (k % 4)).  The MFMA B operand (8 consecutive k of one
// expert per lane) is read with the gfx950 transposing LDS read.  Wave w
// owns experts 32 w .. + 31 of each half.  Then the logits (+ bias) go to
// LDS and each wave routes a quarter of the block's tokens (wave_route_token).
constexpr int kRmStep = 64;  // k per step
// LDS stages (6 measured slower at T = 16384, fewer blocks per CU; 6 and 7
// at T = 4096, one block per CU either way, 36.2 and 37.4 against 34.6 us)
constexpr int kRmDepth = 4;
// T from which the one-launch router replaces the split-K logits and the
// per-token top-k, and from which its blocks take 32 tokens instead of 16
// (the rows past 16 are zeros in the 32-row MFMA; at T = 4096 the 16-token
// blocks fill all CUs: 38 us against 56 us with 32-token blocks and 47 us
// split; at T = 16384 the 32-token blocks: 73 us against 89 us)
constexpr int kRouteFusedMinT = 4096;
constexpr int kRouteFused32T = 8192;

typedef int i32x4v_t __attribute__((ext_vector_type(4)));
typedef short s16x4v_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i32x4v_t rm_rsrc(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  i32x4v_t r;
  r[0] = int(__builtin_amdgcn_readfirstlane(uint32_t(v)));
  r[1] = int(__builtin_amdgcn_readfirstlane(uint32_t(v >> 32)));
  r[2] = 0x7FFFFFFF;
  r[3] = 0x00020000;
  return r;
}
__device__ __forceinline__ void rm_copy(i32x4v_t rsrc, uint32_t lds, int voffset, int soffset) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(lds), "v"(voffset), "s"(rsrc),
               "s"(soffset)
               : "memory");
}
template <int VM>
__device__ __forceinline__ void rm_wait() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int NH, int TOK>  // 128-column halves of E; tokens per block (16 or 32)
__global__ __launch_bounds__(256) void k_route_mfma(Shape sh, const bf16_t* __restrict__ x, const bf16_t* __restrict__ wr,
                                                    const float* __restrict__ bias, Workspace ws) {
  constexpr int E = 128 * NH;
  constexpr int kA = 32 * 128;                 // x rows of a step: 4 KB
  constexpr int kB = kRmStep * 256 * NH;       // W_r rows of a step
  constexpr int kStage = kA + kB;
  constexpr int CB = kB / 1024 / 4;            // W_r copies per wave per step
  constexpr int kPer = 1 + CB;                 // copies per wave per step
  typedef __attribute__((address_space(3))) unsigned char lds_u8;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[kRmDepth * kStage];
  float* const zs = reinterpret_cast<float*>(lds);  // [32][E] logits after the K loop (the stages are free)
  lds_u8* const l3 = (lds_u8*)lds;
  const uint32_t lbase = uint32_t(reinterpret_cast<uintptr_t>(l3));
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5, lc = lane & 31;
  const int t0 = blockIdx.x * TOK;
  const int H = sh.H, nsteps = H / kRmStep;

  // x copy of wave w: rows 8 w .. + 7; lane: row 8 w + lane / 8, slot lane % 8
  const i32x4v_t xr = rm_rsrc(x);
  int xoff;
  {
    const int r = 8 * wave + (lane >> 3);
    xoff = r < TOK && t0 + r < sh.T ? int((uint32_t(t0 + r) * uint32_t(H) + uint32_t(((lane & 7) ^ ((r >> 1) & 7)) * 8)) * 2u)
                         : int(0x80000000u);  // past T: out of range, zeros
  }
  // W_r copy q of wave w: k rows 4 (CB w + q) .. + 3 of the step, across the
  // halves: copy index c = CB w + q -> half c / 16, rows 4 (c % 16) ..;
  // lane: row + lane / 16, slot lane % 16 <- chunk slot ^ 4 (k % 4)
  const i32x4v_t wrs = rm_rsrc(wr);
  int woff[CB];
#pragma unroll
  for (int q = 0; q < CB; ++q) {
    const int c = CB * wave + q, half = c >> 4, k = 4 * (c & 15) + (lane >> 4);
    woff[q] = int((uint32_t(k) * uint32_t(E) + uint32_t(128 * half + (((lane & 15) ^ (4 * (k & 3))) * 8))) * 2u);
  }
  auto issue = [&](int st) {
    const int kk = min(st, nsteps - 1) * kRmStep;
    const uint32_t sb = lbase + uint32_t((st % kRmDepth) * kStage);
    rm_copy(xr, sb + wave * 1024, xoff, kk * 2);
#pragma unroll
    for (int q = 0; q < CB; ++q) {
      const int c = CB * wave + q;
      rm_copy(wrs, sb + kA + (c >> 4) * (kRmStep * 256) + (c & 15) * 1024, woff[q], kk * E * 2);
    }
  };
  // fragment addresses: A row lc, k-step i: chunk (2 i + hf) ^ ((lc / 2) % 8);
  // B (half j, columns 32 wave ..): as in the grouped GEMM's transposing reads
  int bfr;
  {
    const int g = lane >> 4, i16 = lane & 15, qq = i16 & 3, mr = i16 >> 2;
    const int colb = 32 * wave + 16 * (g & 1);
    const int krow = 8 * (g >> 1) + mr;
    bfr = krow * 256 + ((((colb >> 3) + (qq >> 1)) ^ (4 * (mr & 3))) << 4) + (qq & 1) * 8;
  }
  f32x16_t acc[NH];
#pragma unroll
  for (int j = 0; j < NH; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
#pragma unroll
  for (int st = 0; st < kRmDepth - 1; ++st) issue(st);
  for (int s = 0; s < nsteps; ++s) {
    rm_wait<(kRmDepth - 2) * kPer>();  // step s landed (this wave's copies)
    __builtin_amdgcn_s_barrier();      // every wave's copies of step s landed; step s - 1's slot is free
    issue(s + kRmDepth - 1);
    const lds_u8* sa = l3 + (s % kRmDepth) * kStage;
    const lds_u8* sbp = sa + kA;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x8_t a = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8_t*>(
          sa + lc * 128 + (((2 * i + hf) ^ ((lc >> 1) & 7)) << 4));
#pragma unroll
      for (int j = 0; j < NH; ++j) {
        const lds_u8* p = sbp + j * (kRmStep * 256) + bfr + i * 16 * 256;
        const s16x4v_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4v_t*)(p));
        const s16x4v_t hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4v_t*)(p + 4 * 256));
        const s16x4v_t v[2] = {lo, hi};
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8_t, v), acc[j], 0, 0, 0);
      }
    }
  }
  rm_wait<0>();
  __syncthreads();  // every wave's last fragments are read: the stages become zs
  // logits (+ bias) to LDS: lane holds expert 32 wave + lc of half j, tokens
  // 8 (r / 4) + 4 hf + r % 4
#pragma unroll
  for (int j = 0; j < NH; ++j) {
    const int e = 128 * j + 32 * wave + lc;
    const float b = bias ? bias[e] : 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) zs[(8 * (r >> 2) + 4 * hf + (r & 3)) * E + e] = acc[j][r] + b;
  }
  __syncthreads();
  for (int t = wave; t < TOK && t0 + t < sh.T; t += 4)
    wave_route_token(zs + t * E, E, sh.k, ws.topk_idx + size_t(t0 + t) * sh.k, ws.topk_w + size_t(t0 + t) * sh.k);
}

// per 64-token block: membership masks and counts
__global__ __launch_bounds__(kThreads) void k_align_count(Shape sh, Workspace ws) {
  const int T = sh.T, E = sh.E, k = sh.k;
  const int b = blockIdx.x;
  __shared__ uint64_t mask[256];
  for (int i = threadIdx.x; i < E; i += kThreads) mask[i] = 0;
  __syncthreads();
  // one thread per (token, slot): set the token's bit in its expert's mask
  for (int i = threadIdx.x; i < 64 * k; i += kThreads) {
    const int t = b * 64 + i / k;
    if (t < T) atomicOr(reinterpret_cast<unsigned long long*>(&mask[ws.topk_idx[size_t(t) * k + i % k]]),
                        1ull << (i / k));
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kThreads) {
    ws.blk_mask[size_t(b) * E + e] = mask[e];
    ws.blk_base[size_t(b) * E + e] = __popcll(mask[e]);
  }
}

// one block per expert: exclusive scan of its per-block counts (in place),
// total into counts[e]
__global__ __launch_bounds__(kThreads) void k_align_colscan(Shape sh, int nblk, Workspace ws) {
  const int E = sh.E, e = blockIdx.x;
  __shared__ int scratch[kThreads / kWave + 1];
  int carry = 0;
  for (int b0 = 0; b0 < nblk; b0 += kThreads) {
    const int b = b0 + threadIdx.x;
    const int c = b < nblk ? ws.blk_base[size_t(b) * E + e] : 0;
    int total;
    const int ex = block_exclusive_scan<kThreads>(c, scratch, total);
    if (b < nblk) ws.blk_base[size_t(b) * E + e] = carry + ex;
    carry += total;
  }
  if (threadIdx.x == 0) ws.counts[e] = carry;
}

// one 64-thread block per 64 tokens; block 0 also publishes offsets and the
// tile lists
__global__ __launch_bounds__(kThreads) void k_align_scatter(Shape sh, Workspace ws) {
  const int T = sh.T, E = sh.E, k = sh.k;
  const int b = blockIdx.x;
  __shared__ int offs[257];
  __shared__ int scratch[kThreads / kWave + 1];
  const int c = threadIdx.x < E ? ws.counts[threadIdx.x] : 0;
  int total;
  const int off = block_exclusive_scan<kThreads>(c, scratch, total);
  if (threadIdx.x < E) offs[threadIdx.x] = off;
  __syncthreads();
  if (b == 0) (void)build_offsets_and_tiles<kThreads>(c, E, ws, scratch);
  for (int i = threadIdx.x; i < 64 * k; i += kThreads) {
    const int tl = i / k, j = i % k;
    const int t = b * 64 + tl;
    if (t >= T) continue;
    const int e = ws.topk_idx[size_t(t) * k + j];
    const uint64_t m = ws.blk_mask[size_t(b) * E + e];
    const int p = offs[e] + ws.blk_base[size_t(b) * E + e] + __popcll(m & ((1ull << tl) - 1ull));
    ws.perm[p] = t;
    ws.pos[size_t(t) * k + j] = p;
  }
}

// Up to kAlignScanBlocks token blocks: the scatter with the column scan
// folded in.  Each block sums the per-block counts of k_align_count itself
// (every expert's total, and its own first row per expert from the blocks
// before it: at most 64 x 256 counts, from the L2), so the scan launch is
// saved; past that many blocks the re-reads would cost more than the launch.
constexpr int kAlignScanBlocks = 64;
__global__ __launch_bounds__(kThreads) void k_align_scatter_scan(Shape sh, int nblk, Workspace ws) {
  const int T = sh.T, E = sh.E, k = sh.k;
  const int b = blockIdx.x;
  __shared__ int offs[257];
  __shared__ int base[256];
  __shared__ int scratch[kThreads / kWave + 1];
  const int e = threadIdx.x;  // E <= kThreads
  int tot = 0, pre = 0;
  if (e < E) {
#pragma unroll 16
    for (int b2 = 0; b2 < nblk; ++b2) {
      const int cnt = ws.blk_base[size_t(b2) * E + e];
      tot += cnt;
      pre += b2 < b ? cnt : 0;
    }
  }
  int total;
  const int off = block_exclusive_scan<kThreads>(e < E ? tot : 0, scratch, total);
  if (e < E) {
    offs[e] = off;
    base[e] = pre;
  }
  __syncthreads();
  if (b == 0) (void)build_offsets_and_tiles<kThreads>(tot, E, ws, scratch);
  for (int i = threadIdx.x; i < 64 * k; i += kThreads) {
    const int tl = i / k, j = i % k;
    const int t = b * 64 + tl;
    if (t >= T) continue;
    const int ee = ws.topk_idx[size_t(t) * k + j];
    const uint64_t m = ws.blk_mask[size_t(b) * E + ee];
    const int p = offs[ee] + base[ee] + __popcll(m & ((1ull << tl) - 1ull));
    ws.perm[p] = t;
    ws.pos[size_t(t) * k + j] = p;
  }
}

}  // namespace

bool route_small_fits(const Shape& sh) { return sh.E > 0 && route_small_config(sh).ok; }

hipError_t launch_route_small(const Shape& sh, const bf16_t* x, const bf16_t* wr, const float* bias,
                              const Workspace& ws, hipStream_t s) {
  if (sh.T == 0) return hipSuccess;
  const RouteSmallCfg c = route_small_config(sh);
  if (!c.ok) return hipErrorInvalidValue;
  const dim3 grid(c.nslices, c.groups);
  if (c.cw == 8)
    hipLaunchKernelGGL(k_route_part<8>, grid, dim3(kThreads), 0, s, sh, c.slice_rows, c.tb, x, wr, bias, ws);
  else
    hipLaunchKernelGGL(k_route_part<4>, grid, dim3(kThreads), 0, s, sh, c.slice_rows, c.tb, x, wr, bias, ws);
  return hipGetLastError();
}

hipError_t launch_gemm_router(const Shape& sh, const bf16_t* x, const bf16_t* wr, float* logits, int ksplit,
                              hipStream_t s);

hipError_t launch_route_large(const Shape& sh, const bf16_t* x, const bf16_t* wr, const float* bias,
                              const Workspace& ws, hipStream_t s) {
  if ((sh.E == 128 || sh.E == 256) && sh.H % kRmStep == 0 && sh.T >= kRouteFusedMinT) {
    // logits and routing in one launch (below kRouteFusedMinT its blocks
    // leave CUs idle and the split-K path is faster)
    const bool t32 = sh.T >= kRouteFused32T;
    const dim3 grid((sh.T + (t32 ? 31 : 15)) / (t32 ? 32 : 16));
    if (sh.E == 128 && t32)
      hipLaunchKernelGGL((k_route_mfma<1, 32>), grid, dim3(256), 0, s, sh, x, wr, bias, ws);
    else if (sh.E == 128)
      hipLaunchKernelGGL((k_route_mfma<1, 16>), grid, dim3(256), 0, s, sh, x, wr, bias, ws);
    else if (t32)
      hipLaunchKernelGGL((k_route_mfma<2, 32>), grid, dim3(256), 0, s, sh, x, wr, bias, ws);
    else
      hipLaunchKernelGGL((k_route_mfma<2, 16>), grid, dim3(256), 0, s, sh, x, wr, bias, ws);
    return hipGetLastError();
  }
  int nslices = 1;
  if (sh.E % 128 == 0 && sh.H % 64 == 0) {
    // enough K-slices for ~512 tiles, at most kRouterSlices
    const int mt = (sh.T + kGemmBM - 1) / kGemmBM * (sh.E / 128);
    nslices = std::max(1, std::min(kRouterSlices, std::min(512 / std::max(1, mt), sh.H / 64)));
    hipError_t err = launch_gemm_router(sh, x, wr, ws.logits, nslices, s);
    if (err != hipSuccess) return err;
  } else {
    const long long n = (long long)sh.T * sh.E;
    hipLaunchKernelGGL(k_router_logits_fma, dim3(unsigned((n + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                       s, sh, x, wr, ws.logits);
  }
  hipLaunchKernelGGL(k_topk, dim3((sh.T + 3) / 4), dim3(kThreads), 0, s, sh, nslices, bias, ws);
  return hipGetLastError();
}

hipError_t launch_align(const Shape& sh, const Workspace& ws, hipStream_t s) {
  const int nblk = (sh.T + 63) / 64;
  hipLaunchKernelGGL(k_align_count, dim3(nblk), dim3(kThreads), 0, s, sh, ws);
  if (nblk <= kAlignScanBlocks) {
    hipLaunchKernelGGL(k_align_scatter_scan, dim3(nblk), dim3(kThreads), 0, s, sh, nblk, ws);
  } else {
    hipLaunchKernelGGL(k_align_colscan, dim3(sh.E), dim3(kThreads), 0, s, sh, nblk, ws);
    hipLaunchKernelGGL(k_align_scatter, dim3(nblk), dim3(kThreads), 0, s, sh, ws);
  }
  return hipGetLastError();
}

}  // namespace moe
