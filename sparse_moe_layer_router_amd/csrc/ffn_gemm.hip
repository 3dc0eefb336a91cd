// Grouped GEMM on MFMA (bf16 in, fp32 accumulate) for expert buckets with many rows (prefill),
// and the dense router GEMM for large batches.
//
// MoE-kernels page (blog.llmgo.top), section 1.2: with hundreds of tokens per expert the expert
// FFN is a large, compute-bound GEMM; section 4.2: one launch computes many GEMMs that share K and
// N but have their own M, each block taking its tile from the running offsets of the experts, so
// no expert waits on a separate launch; data-movement page, section 15: once routes are sorted by
// expert, each expert's weights are loaded once and reused across its whole bucket of tokens.
//
// Tiles: BM = 128 rows (tokens) x BN weight rows per B matrix x BK = 32 along K; 512 threads as
// 2 x 4 waves (two per SIMD), wave (wm, wn) owning rows [64 wm, 64 wm + 64) x BN/4 columns of
// every B matrix as 32x32x16 MFMA blocks: 8 MFMAs per 16-wide K step from 2 A and 4 B fragments,
// 128 accumulator registers per wave, which leaves room for double-buffered fragments at two
// waves per SIMD. Gate and up projections are computed by the same block for the same rows (two B
// tiles), so SiLU(g)*u is formed in registers and the hidden activation leaves as bf16.
//
// Operands go straight from global memory into a four-slice LDS ring (global_load_lds, 16 bytes
// per lane, no register staging), the loads of each slice spread over the MFMAs of the two K steps
// after the barrier that frees its buffer; waves wait (s_waitcnt vmcnt) only for the slice they
// need next, with two further slices in flight. Fragments are double-buffered in registers across K steps: while the
// MFMAs of step j run, the LDS reads of step j+1 are issued between them (scheduling groups pin
// one read after each of the first MFMAs), so LDS latency hides behind matrix work. The
// slice barrier sits between the two steps of a slice. A 16-byte-chunk XOR swizzle (activations)
// and the fragment-tiled weight layout keep fragment reads bank-conflict free.
//
// Tile order: tiles are numbered expert by expert, N-tile by N-tile, with the M-tiles of one
// (expert, N-tile) adjacent. Workgroups are dealt round-robin to the 8 XCDs, so block L runs tile
// (L % 8) * per_xcd + L / 8: adjacent tiles run at the same time on the same XCD and the second
// and third M-tiles of a weight tile find it in that XCD's L2 instead of HBM.
#include "kernels.h"
#include "moe_device.h"

namespace moe {

namespace {

constexpr int BM = 128;
constexpr int BK = 32;
constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kWavesM = 2, kWavesN = 4;
constexpr int kXcds = 8;
constexpr int kStages = 4;   // LDS ring depth (4 x 40 KB = all 160 KB of LDS): two slices fully in flight
constexpr int kRowBytes = BK * 2;  // one tile row in LDS: 64 bytes = 4 chunks of 16

enum GemmMode { kGateUp = 0, kDown = 1, kRouter = 2 };

template <int MODE> struct Geo {
  static constexpr int NB = MODE == kGateUp ? 2 : 1;                          // B matrices per tile
  static constexpr int BN = MODE == kGateUp ? 256 : (MODE == kDown ? 512 : 256);  // rows of each B tile
  static constexpr int WM = BM / kWavesM;                                      // rows per wave
  static constexpr int WN = BN / kWavesN;                                     // columns per wave
  static constexpr int NBLK = WN / 32;                                        // 32-wide MFMA blocks
  static constexpr int MBLK = WM / 32;                                        // 32-high MFMA blocks
  static constexpr int A_BYTES = BM * kRowBytes;
  static constexpr int B_BYTES = NB * BN * kRowBytes;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int A_LOADS = BM * (BK / 8) / kThreads;         // 16-byte chunks per lane
  static constexpr int B_LOADS = NB * BN * (BK / 8) / kThreads;
  static constexpr int LOADS = A_LOADS + B_LOADS;                  // global_load_lds per wave per slice
};

// LDS byte offset of 16-byte chunk `chunk` (0..3) of tile row `row`. The XOR key takes four
// distinct values over any four rows of equal parity among 8 consecutive rows and over any four
// rows of equal residue mod 4 among 16 consecutive rows, so a fragment read (16 or 8 consecutive
// rows, one chunk column) touches distinct 16-byte bank groups.
__device__ __forceinline__ int swz_chunk(int row, int chunk) { return chunk ^ (((row >> 1) ^ (row >> 2)) & 3); }
__device__ __forceinline__ int swz(int row, int chunk) { return row * kRowBytes + (swz_chunk(row, chunk) << 4); }

// LDS reads of one 16-wide K step: the wave's MBLK A fragments (rows wm*WM + 32*mb + fr) and the
// NB x NBLK B fragments (rows wn*WN + 32*nb + fr of each B tile), chunk column ch.
template <class G, int LAYOUT>
__device__ __forceinline__ void load_frags(u32x4_t (&fa)[G::MBLK], u32x4_t (&fb)[G::NB][G::NBLK], const uint8_t* sa,
                                           const uint8_t* sb, int wm, int wn, int fr, int ch) {
#pragma unroll
  for (int mb = 0; mb < G::MBLK; ++mb) fa[mb] = *(const u32x4_t*)(sa + swz(wm * G::WM + mb * 32 + fr, ch));
#pragma unroll
  for (int b = 0; b < G::NB; ++b)
#pragma unroll
    for (int nb = 0; nb < G::NBLK; ++nb) {
      const int n = wn * G::WN + nb * 32 + fr;   // row inside B matrix b's tile
      if (LAYOUT == kFrag16)  // block n/16 of matrix b; lane position (n%16) + 16*chunk
        fb[b][nb] = *(const u32x4_t*)(sb + (b * (G::BN / 16) + n / 16) * 1024 + ((n & 15) + 16 * ch) * 16);
      else
        fb[b][nb] = *(const u32x4_t*)(sb + swz(b * G::BN + n, ch));
    }
}

template <class G>
__device__ __forceinline__ void mma_step(f32x16_t (&acc)[G::NB][G::MBLK][G::NBLK], const u32x4_t (&fa)[G::MBLK],
                                         const u32x4_t (&fb)[G::NB][G::NBLK]) {
#pragma unroll
  for (int b = 0; b < G::NB; ++b)
#pragma unroll
    for (int nb = 0; nb < G::NBLK; ++nb)
#pragma unroll
      for (int mb = 0; mb < G::MBLK; ++mb) acc[b][mb][nb] = mfma32x32x16(fa[mb], fb[b][nb], acc[b][mb][nb]);
}

// Pin the order of the instructions just emitted: MFMA, LDS read, MFMA, LDS read, ... and then the
// remaining MFMAs, so each LDS read issues under an MFMA instead of in a block before them.
template <int MFMAS, int READS>
__device__ __forceinline__ void interleave_mfma_lds() {
  static_assert(READS <= MFMAS, "one LDS read after each of the first READS MFMAs");
#pragma unroll
  for (int i = 0; i < READS; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
  }
  if (MFMAS > READS) __builtin_amdgcn_sched_group_barrier(0x008, MFMAS - READS, 0);
}

// The same with VMEMS global-to-LDS loads after each of the last VMEMS MFMAs. The loads write LDS
// that the compiler cannot tell apart from the buffer being read, so they stay after the reads
// (their program order): MFMA, read, ..., MFMA, read, load, ..., MFMA, load.
template <int MFMAS, int READS, int VMEMS>
__device__ __forceinline__ void interleave_mfma_lds_vmem() {
  static_assert(READS <= MFMAS && VMEMS <= MFMAS, "at most one read and one load after each MFMA");
#pragma unroll
  for (int i = 0; i < MFMAS; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                          // one MFMA
    if (i < READS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);           // one LDS read
    if (i >= MFMAS - VMEMS) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one global load
  }
}

}  // namespace

// ------------------------------------------------------------------------------- schedule
// One block: for every group, m-tiles = ceil(rows / BM); tiles = m-tiles * n-tiles of that group.
// Writes exclusive prefix sums for the gate/up pass (sched_gu) and the down pass (sched_dn),
// 1024 groups per round with the running total carried between rounds.
__global__ void __launch_bounds__(1024)
gemm_schedule_kernel(const FfnGroups p, int32_t* __restrict__ sched_gu, int32_t* __restrict__ sched_dn) {
  __shared__ int32_t wtot_gu[16], wtot_dn[16];
  const int ngroups = p.E + (p.Hs > 0 ? 1 : 0);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int32_t carry_a = 0, carry_b = 0;
  for (int base = 0; base < ngroups; base += 1024) {
    const int g = base + (int)threadIdx.x;
    int32_t a = 0, b = 0;
    if (g < ngroups) {
      long long n;
      int Hg;
      if (g < p.E) {
        long long lo = p.offsets[g], hi = p.offsets[g + 1];
        lo = lo < 0 ? 0 : (lo > p.rows ? p.rows : lo);
        hi = hi < lo ? lo : (hi > p.rows ? p.rows : hi);
        n = hi - lo;
        Hg = p.H;
      } else {
        n = p.T;
        Hg = p.Hs;
      }
      const int mt = (int)((n + BM - 1) / BM);
      a = mt * ((Hg + Geo<kGateUp>::BN - 1) / Geo<kGateUp>::BN);
      b = mt * ((p.d + Geo<kDown>::BN - 1) / Geo<kDown>::BN);
    }
    int32_t ia = a, ib = b;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int32_t oa = __shfl_up(ia, off, 64), ob = __shfl_up(ib, off, 64);
      if (lane >= off) { ia += oa; ib += ob; }
    }
    if (lane == 63) { wtot_gu[wave] = ia; wtot_dn[wave] = ib; }
    __syncthreads();
    int32_t ba = carry_a, bb = carry_b;
    for (int w = 0; w < wave; ++w) { ba += wtot_gu[w]; bb += wtot_dn[w]; }
    if (g < ngroups) {
      sched_gu[g] = ba + ia - a;
      sched_dn[g] = bb + ib - b;
      if (g == ngroups - 1) { sched_gu[ngroups] = ba + ia; sched_dn[ngroups] = bb + ib; }
    }
    for (int w = 0; w < 16; ++w) { carry_a += wtot_gu[w]; carry_b += wtot_dn[w]; }
    __syncthreads();  // wtot_* are rewritten in the next round
  }
}

// ------------------------------------------------------------------------------- the GEMM
struct GemmArgs {
  FfnGroups p;
  const int32_t* sched;   // [ngroups + 1] (kGateUp / kDown); unused for the router
  // router mode
  const void* x;          // [T, d]
  const void* w;          // [E, d]
  const float* bias;      // [E] or NULL
  float* logits;          // [T, E]
  int T, E, d;
};

// Tile count of a launch: from the router's sizes, or the schedule's running total.
template <int MODE>
__device__ __forceinline__ int gemm_total_tiles(const GemmArgs& ga) {
  if (MODE == kRouter) return ((ga.T + BM - 1) / BM) * ((ga.E + Geo<MODE>::BN - 1) / Geo<MODE>::BN);
  return ga.sched[ga.p.E + (ga.p.Hs > 0 ? 1 : 0)];
}

// One output tile t (0 <= t < gemm_total_tiles) through the LDS ring `smem`.
template <int MODE, int LAYOUT>
__device__ __forceinline__ void gemm_tile(const GemmArgs& ga, const int t, uint8_t (*smem)[Geo<MODE>::STAGE]) {
  using G = Geo<MODE>;
  const FfnGroups& p = ga.p;
  const int lane = lane_id();
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));  // wave index, 0..7

  // ---- which tile --------------------------------------------------------------------------
  int g = 0, mt = 0, nt = 0;
  long long r0 = 0;      // first row of the group in its row space
  int nrows = 0;         // rows in the group
  int N = 0, K = 0;      // output columns (weight rows) and reduction length of this group
  const uint16_t* Bp[2] = {nullptr, nullptr};
  {
    if (MODE == kRouter) {
      nt = t / ((ga.T + BM - 1) / BM);
      mt = t % ((ga.T + BM - 1) / BM);
      nrows = ga.T;
      N = ga.E;
      K = ga.d;
      Bp[0] = (const uint16_t*)ga.w;
    } else {
      const int ngroups = p.E + (p.Hs > 0 ? 1 : 0);
      int lo = 0, hi = ngroups;  // last group with sched[g] <= t
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (ga.sched[mid] <= t) lo = mid; else hi = mid;
      }
      g = lo;
      int Hg;
      if (g < p.E) {
        long long a = p.offsets[g], b = p.offsets[g + 1];
        a = a < 0 ? 0 : (a > p.rows ? p.rows : a);
        b = b < a ? a : (b > p.rows ? p.rows : b);
        r0 = a;
        nrows = (int)(b - a);
        Hg = p.H;
      } else {
        r0 = 0;
        nrows = p.T;
        Hg = p.Hs;
      }
      const int mtiles = (nrows + BM - 1) / BM;
      const int local = t - ga.sched[g];
      nt = local / mtiles;
      mt = local % mtiles;
      const size_t wsz = (size_t)p.H * p.d;
      if (MODE == kGateUp) {
        N = Hg;
        K = p.d;
        Bp[0] = g < p.E ? (const uint16_t*)p.w_gate + (size_t)g * wsz : (const uint16_t*)p.ws_gate;
        Bp[1] = g < p.E ? (const uint16_t*)p.w_up + (size_t)g * wsz : (const uint16_t*)p.ws_up;
      } else {
        N = p.d;
        K = Hg;
        Bp[0] = g < p.E ? (const uint16_t*)p.w_down + (size_t)g * wsz : (const uint16_t*)p.ws_down;
      }
    }
  }
  const int m0 = mt * BM, n0 = nt * G::BN;

  // ---- per-lane global sources -----------------------------------------------------------------
  // A slice holds BM*4 chunks of A and NB*BN*4 chunks of B (4 chunks of 16 bytes per 32-wide row).
  // Wave w fills chunk positions [w*BM*4/8, (w+1)*BM*4/8) of A and the matching share of the stacked
  // B tiles, 64 consecutive positions per instruction (lane l -> position base + l). Position p
  // holds row p/4, physical chunk p%4, i.e. logical chunk swz_chunk(row, p%4): the lane loads that
  // logical chunk of that row.
  const int phys = lane & 3;
  const uint16_t* a_src[G::A_LOADS];
  const uint16_t* b_src[G::B_LOADS];
  int a_kc[G::A_LOADS], b_kc[G::B_LOADS];     // element offset of the lane's chunk inside a K slice
#pragma unroll
  for (int i = 0; i < G::A_LOADS; ++i) {
    const int row = wv * (BM / kWaves) + i * 16 + (lane >> 2);
    a_kc[i] = swz_chunk(row, phys) * 8;
    int rr = m0 + row;
    rr = rr < nrows ? rr : (nrows > 0 ? nrows - 1 : 0);  // rows past the bucket: any valid row, never stored
    long long src;
    if (MODE == kRouter) {
      src = rr;
      a_src[i] = (const uint16_t*)ga.x + (size_t)src * K;
    } else if (MODE == kGateUp) {
      if (g < p.E) {
        src = p.perm_src ? (long long)(p.perm_src[r0 + rr] / p.k) : r0 + rr;
        const long long lim = p.perm_src ? (long long)p.T : p.rows;
        src = src < 0 ? 0 : (src >= lim ? lim - 1 : src);
      } else {
        src = rr;
      }
      a_src[i] = (const uint16_t*)p.x + (size_t)src * K;
    } else {
      const uint16_t* hid = (const uint16_t*)p.hid + (g < p.E ? 0 : (size_t)p.rows * p.H);
      a_src[i] = hid + (size_t)(r0 + rr) * K;
    }
  }
#pragma unroll
  for (int i = 0; i < G::B_LOADS; ++i) {
    if (LAYOUT == kFrag16) {
      // one 16 x 32 block (1 KB, contiguous in the packed weight) per instruction: block q of the
      // stacked B tiles is band n0/16 + q % (BN/16) of matrix q / (BN/16)
      const int q = wv * G::B_LOADS + i;
      const int b = q / (G::BN / 16);
      int band = n0 / 16 + q % (G::BN / 16);
      band = band < N / 16 ? band : N / 16 - 1;  // bands past N: any valid band, never stored
      b_kc[i] = 0;
      b_src[i] = Bp[b] + (size_t)band * (K / 32) * 512 + lane * 8;
    } else {
      const int row = wv * (G::NB * G::BN / kWaves) + i * 16 + (lane >> 2);   // stacked rows of the B tiles
      b_kc[i] = swz_chunk(row, phys) * 8;
      const int b = row / G::BN;
      int n = n0 + (row % G::BN);
      n = n < N ? n : N - 1;                     // rows past N: any valid row, never stored
      b_src[i] = Bp[b] + (size_t)n * K;
    }
  }

  const int nk = (K + BK - 1) / BK;  // K slices
  typedef __attribute__((address_space(3))) void lds_t;
  // LDS byte offsets (wave-uniform) of this wave's instruction i inside a slice
  auto a_dst = [&](int i) { return (wv * (BM / kWaves) + i * 16) * kRowBytes; };
  auto b_dst = [&](int i) {
    return LAYOUT == kFrag16 ? G::A_BYTES + (wv * G::B_LOADS + i) * 1024
                             : G::A_BYTES + (wv * (G::NB * G::BN / kWaves) + i * 16) * kRowBytes;
  };
  // Loads j in [J0, J1) of slice kt (A loads first, then B loads) into ring buffer `buf`. A slice
  // index past the end is clamped to the last slice: such loads fill a buffer that is never read
  // again, which keeps the number of loads per slice fixed for the vmcnt arithmetic below.
  auto issue = [&](int kt, int buf, int j0, int j1) {
    const int kc = kt < nk ? kt : nk - 1;
    const int k0 = kc * BK;
#pragma unroll
    for (int i = 0; i < G::A_LOADS; ++i) {
      if (i < j0 || i >= j1) continue;
      const int k = k0 + a_kc[i];
      const uint16_t* src = a_src[i] + (k < K ? k : 0);    // out-of-range chunks are zeroed after landing
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_t*)(smem[buf] + a_dst(i)), 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < G::B_LOADS; ++i) {
      if (G::A_LOADS + i < j0 || G::A_LOADS + i >= j1) continue;
      const uint16_t* src;
      if (LAYOUT == kFrag16) {
        src = b_src[i] + (size_t)kc * 512;  // K is a multiple of 32 in this layout: no tail
      } else {
        const int k = k0 + b_kc[i];
        src = b_src[i] + (k < K ? k : 0);
      }
      __builtin_amdgcn_global_load_lds((const void*)src, (lds_t*)(smem[buf] + b_dst(i)), 16, 0, 0);
    }
  };
  // chunks past K in the last slice: write zeros over what the loads brought in
  auto zero_tail = [&](int kt, int buf) {
    const int k0 = kt * BK;
    const u32x4_t zero = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < G::A_LOADS; ++i)
      if (k0 + a_kc[i] >= K) *(u32x4_t*)(smem[buf] + a_dst(i) + lane * 16) = zero;
    if (LAYOUT != kFrag16) {
#pragma unroll
      for (int i = 0; i < G::B_LOADS; ++i)
        if (k0 + b_kc[i] >= K) *(u32x4_t*)(smem[buf] + b_dst(i) + lane * 16) = zero;
    }
  };

  f32x16_t acc[G::NB][G::MBLK][G::NBLK];
#pragma unroll
  for (int b = 0; b < G::NB; ++b)
#pragma unroll
    for (int mb = 0; mb < G::MBLK; ++mb)
#pragma unroll
      for (int nb = 0; nb < G::NBLK; ++nb)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[b][mb][nb][e] = 0.f;

  const int fr = lane & 31, fh = lane >> 5;   // fragment row / k-half of this lane
  const int wm = wv / kWavesN, wn = wv % kWavesN;
  constexpr int kMfmas = G::NB * G::NBLK * G::MBLK;          // per K step
  constexpr int kReads = G::MBLK + G::NB * G::NBLK;          // per K step

  // Ring protocol (S = kStages). The loads of slice s go to buffer s % S and are issued in two
  // parts spread over the MFMAs: part 1 (loads [0, kSplit)) during step 1 of slice s-S, part 2
  // (the rest) during step 0 of slice s-S+1, both after the barrier that ends every wave's reads
  // of slice s-S, the previous tenant of the buffer. Spreading them keeps the vector-memory issue
  // queue from stalling all waves at once right after the barrier. Before step 1 of slice kt a
  // wave waits for its loads of slice kt+1: slices kt+2 .. kt+S-1 have been issued in full by
  // then and loads complete in issue order, so vmcnt((S-2) * LOADS) leaves exactly those
  // outstanding. The barrier that follows makes every wave's part of slice kt+1 visible.
  // Slices past the end are clamped copies of the last one (see issue); in the last step the
  // buffer of slice kt+1 (free: its previous tenant was slice kt+1-S) takes them, since the
  // current buffer may still be read by waves that are behind and no barrier follows.
  constexpr int S = kStages;
  static_assert(S >= 3, "the issue schedule below needs a ring of at least 3 slices");
  constexpr int kSplit = (G::LOADS + 1) / 2;
  constexpr int kAhead = (S - 2) * G::LOADS;   // loads allowed in flight when slice kt+1 must land
  static_assert(kAhead + kSplit < 64, "vmcnt holds 6 bits");
  auto arrive = [&](int kt) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kAhead) : "memory");
    if (kt == nk - 1 && (K % BK)) zero_tail(kt, kt % S);  // its loads have all landed here
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };

  static_assert(BK / 16 == 2, "the loop below is written for two K steps per slice");
  u32x4_t fa0[G::MBLK], fb0[G::NB][G::NBLK], fa1[G::MBLK], fb1[G::NB][G::NBLK];
#pragma unroll
  for (int i = 0; i < S - 1; ++i) issue(i, i, 0, G::LOADS);
  issue(S - 1, S - 1, 0, kSplit);
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kAhead + kSplit) : "memory");
  if (nk == 1 && (K % BK)) zero_tail(0, 0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  load_frags<G, LAYOUT>(fa0, fb0, smem[0], smem[0] + G::A_BYTES, wm, wn, fr, fh);
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt % S;
    // step 0 of slice kt: multiply fragments 0 while reading step 1 into fragments 1 and issuing
    // part 2 of slice kt+S-1
    mma_step<G>(acc, fa0, fb0);
    load_frags<G, LAYOUT>(fa1, fb1, smem[buf], smem[buf] + G::A_BYTES, wm, wn, fr, 2 + fh);
    issue(kt + S - 1, (kt + S - 1) % S, kSplit, G::LOADS);
    interleave_mfma_lds_vmem<kMfmas, kReads, G::LOADS - kSplit>();
    // step 1 of slice kt: multiply fragments 1 while reading step 0 of slice kt+1 into fragments 0
    // and issuing part 1 of slice kt+S into this slice's buffer (after the last slice the reads
    // re-read the current buffer and are never used)
    if (kt + 1 < nk) arrive(kt + 1);
    const int nbuf = kt + 1 < nk ? (kt + 1) % S : buf;
    const int lbuf = kt + 1 < nk ? buf : (kt + 1) % S;
    mma_step<G>(acc, fa1, fb1);
    load_frags<G, LAYOUT>(fa0, fb0, smem[nbuf], smem[nbuf] + G::A_BYTES, wm, wn, fr, fh);
    issue(kt + S, lbuf, 0, kSplit);
    interleave_mfma_lds_vmem<kMfmas, kReads, kSplit>();
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no load may still write LDS when the block exits

  // ---- epilogue: lane holds column n = fr of each 32x32 block, rows (e/4)*8 + fh*4 + e%4 --------
#pragma unroll
  for (int mb = 0; mb < G::MBLK; ++mb)
#pragma unroll
    for (int nb = 0; nb < G::NBLK; ++nb) {
      const int n = n0 + wn * G::WN + nb * 32 + fr;
      if (n >= N) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm * G::WM + mb * 32 + (e >> 2) * 8 + fh * 4 + (e & 3);
        if (row >= nrows) continue;
        if (MODE == kGateUp) {
          const float gv = acc[0][mb][nb][e], uv = acc[1][mb][nb][e];
          uint16_t* hid = (uint16_t*)p.hid + (g < p.E ? 0 : (size_t)p.rows * p.H);
          hid[(size_t)(r0 + row) * N + n] = (uint16_t)f32_to_bf16(silu(gv) * uv);
        } else if (MODE == kDown) {
          uint16_t* y = (uint16_t*)p.y + (g < p.E ? 0 : (size_t)p.rows * p.d);
          y[(size_t)(r0 + row) * N + n] = (uint16_t)f32_to_bf16(acc[0][mb][nb][e]);
        } else {
          ga.logits[(size_t)row * N + n] = acc[0][mb][nb][e] + (ga.bias ? ga.bias[n] : 0.f);
        }
      }
    }
}

// Tiles are numbered expert by expert, N-tile by N-tile, with the M-tiles of one (expert, N-tile)
// adjacent, and dealt to the 8 XCDs in contiguous ranges (workgroup L runs on XCD L % 8).
// Workgroup L takes tile (L % 8) * per + L / 8 and then every (gridDim / 8)-th tile after it in
// its XCD's range: with one workgroup per tile (the launch used) that is exactly one tile.
template <int MODE, int LAYOUT>
__global__ void __launch_bounds__(kThreads, 1)
grouped_gemm_kernel(const GemmArgs ga) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kStages][Geo<MODE>::STAGE];
  const int total = gemm_total_tiles<MODE>(ga);
  const int per = (total + kXcds - 1) / kXcds;
  const int xcd = (int)blockIdx.x % kXcds, stride = (int)gridDim.x / kXcds;
  const int end = (xcd + 1) * per < total ? (xcd + 1) * per : total;
  for (int t = xcd * per + (int)blockIdx.x / kXcds; t < end; t += stride) {
    if (t >= xcd * per + stride) __syncthreads();  // the previous tile's LDS reads are over
    gemm_tile<MODE, LAYOUT>(ga, t, smem);
  }
}

// ------------------------------------------------------------------------------- launchers
namespace {
int round8(long long v) { return (int)((v + kXcds - 1) / kXcds * kXcds); }

// Workgroups of a launch: one per tile (rounded to whole XCD sets). The hardware then starts the
// tiles of each XCD in order as CUs free up, so the M-tiles that share a weight tile start
// together and stream it through L2 once. A persistent launch (one workgroup per CU, each walking
// its XCD's range) measured the same time but let those M-tiles drift apart: 29.6 GB fetched from
// the fabric per gate/up launch at T=8192 instead of 24 GB.
int gemm_grid(long long tiles_upper) { return round8(tiles_upper); }
}  // namespace

long long gemm_tiles_upper(const FfnGroups& p, int mode) {
  const long long mt_routed = p.rows / BM + p.E;  // each group adds at most one partial tile
  const long long mt_shared = p.Hs > 0 ? (p.T + BM - 1) / BM : 0;
  if (mode == kGateUp) {
    const int bn = Geo<kGateUp>::BN;
    return mt_routed * ((p.H + bn - 1) / bn) + mt_shared * ((p.Hs + bn - 1) / bn);
  }
  const int bn = Geo<kDown>::BN;
  return (mt_routed + mt_shared) * ((p.d + bn - 1) / bn);
}

size_t gemm_schedule_ints(int E) { return 2 * (size_t)(E + 2); }

hipError_t launch_gemm_schedule(const FfnGroups& p, int32_t* sched, hipStream_t stream) {
  hipLaunchKernelGGL(gemm_schedule_kernel, dim3(1), dim3(1024), 0, stream, p, sched, sched + p.E + 2);
  return hipGetLastError();
}

hipError_t launch_gemm_gate_up(const FfnGroups& p, const int32_t* sched, hipStream_t stream) {
  GemmArgs a{};
  a.p = p;
  a.sched = sched;
  const dim3 grid(gemm_grid(gemm_tiles_upper(p, kGateUp)));
  if (p.layout == kFrag16)
    hipLaunchKernelGGL((grouped_gemm_kernel<kGateUp, kFrag16>), grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((grouped_gemm_kernel<kGateUp, kRowMajor>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_gemm_down(const FfnGroups& p, const int32_t* sched, hipStream_t stream) {
  GemmArgs a{};
  a.p = p;
  a.sched = sched + p.E + 2;
  const dim3 grid(gemm_grid(gemm_tiles_upper(p, kDown)));
  if (p.layout == kFrag16)
    hipLaunchKernelGGL((grouped_gemm_kernel<kDown, kFrag16>), grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((grouped_gemm_kernel<kDown, kRowMajor>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_router_gemm(const void* x, const void* w, const float* bias, float* logits, int T, int E, int d,
                              hipStream_t stream) {
  GemmArgs a{};
  a.x = x;
  a.w = w;
  a.bias = bias;
  a.logits = logits;
  a.T = T;
  a.E = E;
  a.d = d;
  const long long tiles = (long long)((T + BM - 1) / BM) * ((E + Geo<kRouter>::BN - 1) / Geo<kRouter>::BN);
  hipLaunchKernelGGL((grouped_gemm_kernel<kRouter, kRowMajor>), dim3(gemm_grid(tiles)), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace moe
