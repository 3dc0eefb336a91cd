// Grouped GEMM on MFMA (bf16 in, fp32 accumulate) for expert buckets with many rows (prefill),
// and the dense router GEMM for large batches.
//
// MoE-kernels page (blog.llmgo.top), section 1.2: with hundreds of tokens per expert the expert
// FFN is a large, compute-bound GEMM; section 4.2: one launch computes many GEMMs that share K and
// N but have their own M, each block taking its tile from the running offsets of the experts, so
// no expert waits on a separate launch; data-movement page, section 15: once routes are sorted by
// expert, each expert's weights are loaded once and reused across its whole bucket of tokens.
//
// The same kernel runs the two-layer GELU expert (overview article, section 4.1 layer code:
// Linear(d -> H) with a bias, GELU, Linear(H -> d) with a bias) when its buckets are large: the first
// pass multiplies by W1 alone (256 hidden columns per tile) and its epilogue stores GELU(acc + b1) in
// the packed hidden layout; the second is the down pass with b2 added before the output rounding.
//
// Tiles. An expert bucket is cut into M-tiles of up to BM = 320 rows, so a bucket of the prefill
// regime (about 256 +- 50 rows) is a single M-tile and every weight tile is fetched once per
// bucket. The tile is BM rows x 256 weight rows (gate/up: 128 gate + 128 up rows for the same
// hidden columns; down and router: 256 output columns) x BK = 32 along K. 512 threads = 8 waves,
// two per SIMD, as 2 (M) x 4 (N): wave (wm, wn) owns the 32-row blocks wm, wm + 2, ..., wm + 8
// (interleaved, so a partly filled tile still splits its rows evenly) and 32 + 32 (gate/up) or
// 64 columns, as 32x32x16 MFMA blocks: 5 x 2 accumulators of 16 registers. A wave runs only the
// blocks that hold rows of the tile (a body specialised on that count), so a bucket of 260 rows
// costs 9 row blocks of MFMA work, not 2 x 256.
//
// Operands go straight from global memory into a four-slice LDS ring (global_load_lds, 16 bytes
// per lane, no register staging; 4 x 36 KB). A slice is 36 load instructions of 1 KB: waves 0-3
// load the 20 activation groups (16 rows x 64 bytes each, gathered through the permutation),
// waves 4-7 the 16 weight blocks; each wave's loads for a slice are spread over the MFMAs of the
// two K steps after the barrier that frees its buffer, and a wave waits (s_waitcnt vmcnt) only
// for the slice it needs next, with two further slices in flight. Fragments live in one set of
// registers: while the MFMAs of step j run, each LDS read of step j+1 is issued right after the
// last MFMA that needs the register it overwrites. A 16-byte-chunk XOR swizzle (activations) and
// the fragment-tiled weight layout keep fragment reads bank-conflict free.
//
// Tile order: tiles are numbered expert by expert; within an expert, its M-tiles are taken in blocks
// of up to eight, and a block's tiles run N-tile by N-tile with the block's M-tiles adjacent. Each
// XCD owns a contiguous range of that order, the ranges cut by the schedule kernel so that they
// hold equal modelled work. One persistent workgroup per CU takes the tiles of its XCD's range in
// order from a counter, then helps the XCDs behind (see the kernel), so an XCD's 32 CUs run 32
// consecutive tiles at a time: the N-tiles of
// a one-M-tile expert (every routed bucket of a prefill batch) share its activation rows in the
// XCD's L2; for an expert of many M-tiles (the shared expert over all tokens, a heavily loaded
// expert) they form an 8 x 4 patch that shares 4 weight tiles and 8 activation blocks, where one
// N-tile over all its M-tiles would re-read every activation row once per N-tile.
#include "codes.h"
#include "kernels.h"
#include "moe_device.h"

namespace moe {

namespace {

constexpr int BK = 32;
constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kWavesM = 2, kWavesN = 4;
constexpr int kXcds = 8;
constexpr int kCusPerXcd = 32;
constexpr int kStages = 4;         // LDS ring depth: two slices in flight while one is consumed
constexpr int kRowBytes = BK * 2;  // one tile row in LDS: 64 bytes = 4 chunks of 16
constexpr int kMBlock = 8;         // M-tiles per super-tile block of a group (tile order below)
constexpr int kCtrStride = 16;     // ints between two XCDs' tile counters (one 64-byte line each)

enum GemmMode { kGateUp = 0, kDown = 1, kRouter = 2, kGeluUp = 3, kGeluDown = 4 };

// The first pass of an expert (gathered token rows times the up-projection weights) and the second
// (packed hidden activations times the down-projection weights).
constexpr bool first_pass(int mode) { return mode == kGateUp || mode == kGeluUp; }
constexpr bool packed_a(int mode) { return mode == kDown || mode == kGeluDown; }

// exact GELU, z * Phi(z) = z * erfc(-z / sqrt 2) / 2
__device__ __forceinline__ float gelu_exact(float z) { return 0.5f * z * erfcf(-0.70710678118654752f * z); }

template <int MODE> struct Geo {
  static constexpr int MBW = MODE == kRouter ? 1 : 5;              // 32-row blocks per wave
  static constexpr int BM = MBW * kWavesM * 32;                    // tile rows: 320 (router 64)
  static constexpr int NB = MODE == kGateUp ? 2 : 1;               // B matrices per tile
  static constexpr int NBJ = MODE == kRouter ? 1 : 2;              // 32-column blocks per wave
  static constexpr int BN = MODE == kGateUp ? 128 : NBJ * kWavesN * 32;  // rows of each B tile (router 128)
  static constexpr int BROWS = NB * BN;                            // stacked B rows (256)
  static constexpr int A_INSTR = BM / 16;                          // 1 KB loads of A per slice
  static constexpr int B_INSTR = BROWS / 16;                       // 1 KB loads of B per slice
  static constexpr int INSTR = A_INSTR + B_INSTR;
  static constexpr int L_HI = (INSTR + kWaves - 1) / kWaves;       // loads per slice, waves < N_HI
  static constexpr int N_HI = INSTR - kWaves * (L_HI - 1);
  static constexpr int L_LO = L_HI - 1;                            // loads per slice, other waves
  static constexpr int SPLIT = (L_HI + 1) / 2;                     // loads issued in part 1
  static constexpr int A_BYTES = A_INSTR * 1024;
  static constexpr int STAGE = INSTR * 1024;
  static_assert(N_HI >= 1 && N_HI <= kWaves, "load split");
};

// Load slots of a slice and the LDS of a workgroup for a weight layout. bf16 weights as in Geo:
// every ring stage holds the slice's A rows and its B blocks. One-byte weights (INT8 / E4M3 codes)
// come in 1 KB blocks of 16 rows x 64 K, i.e. two slices: a pair of slices shares its blocks, held
// in a ring of kBPairs pair buffers after the A ring. Slice kt loads half a pair: the second half
// of pair kt / 2 (blocks BLK/2 ..) when kt is even, the first half of pair kt / 2 + 1 (blocks
// 0 .. BLK/2 - 1) when kt is odd, so every slice issues the same loads per wave (waves N_HI..7 two
// blocks each) and a pair is complete when the slice that opens it has landed.
constexpr int kBPairs = 3;
template <int MODE, int LAYOUT> struct Slots {
  using G = Geo<MODE>;
  static constexpr bool Q = byte_codes(LAYOUT);
  static constexpr int B_INSTR = Q ? G::BROWS / 32 : G::B_INSTR;  // 1 KB weight loads per slice
  static constexpr int L_HI = Q ? G::A_INSTR / 4 : G::L_HI;        // loads per slice, waves < N_HI
  static constexpr int N_HI = Q ? 4 : G::N_HI;
  static constexpr int L_LO = Q ? B_INSTR / 4 : G::L_LO;           // loads per slice, other waves
  static constexpr int SPLIT = (L_HI + 1) / 2;
  static constexpr int STAGE = Q ? G::A_BYTES : G::STAGE;           // one ring stage
  static constexpr int PAIR = G::BROWS / 16 * 1024;                 // one-byte: the blocks of a pair
  static constexpr int LDS = kStages * STAGE + (Q ? kBPairs * PAIR : 0);
  static_assert(!Q || (N_HI * L_HI == G::A_INSTR && (kWaves - N_HI) * L_LO == B_INSTR), "one-byte load split");
  static_assert(LDS <= 144 * 1024, "the workgroup's LDS stays within 144 KiB");
};

// LDS byte offset of 16-byte chunk `chunk` (0..3) of tile row `row`. The XOR key takes four
// distinct values over any four rows of equal parity among 8 consecutive rows and over any four
// rows of equal residue mod 4 among 16 consecutive rows, so a fragment read (16 or 8 consecutive
// rows, one chunk column) touches distinct 16-byte bank groups.
__device__ __forceinline__ int swz_chunk(int row, int chunk) { return chunk ^ (((row >> 1) ^ (row >> 2)) & 3); }
__device__ __forceinline__ int swz(int row, int chunk) { return row * kRowBytes + (swz_chunk(row, chunk) << 4); }

// Stacked B row (inside the slice's B region) of the wave's B fragment j for fragment row fr.
template <int MODE>
__device__ __forceinline__ int b_row(int j, int wn, int fr) {
  return MODE == kGateUp ? j * Geo<MODE>::BN + wn * 32 + fr : wn * 32 * Geo<MODE>::NBJ + j * 32 + fr;
}

// A fragment i (rows (wm + 2 i) * 32 + fr) and B fragment j of one 16-wide K step, chunk column ch.
// The down pass holds A (the hidden activations) as packed 16 x 32 blocks, one per 16-row band;
// gate/up and the router hold gathered rows.
template <int MODE>
__device__ __forceinline__ u32x4_t read_a(const uint8_t* sa, int i, int wm, int fr, int ch) {
  const int r = (wm + 2 * i) * 32 + fr;
  if (packed_a(MODE)) return *(const u32x4_t*)(sa + (r / 16) * 1024 + ((r & 15) + 16 * ch) * 16);
  return *(const u32x4_t*)(sa + swz(r, ch));
}
// E4M3 codes become bf16 in four instructions, late (cvt_b, below); INT8 codes take about twenty
// integer instructions, which measured better right at the read, overlapping the MFMAs in flight.
constexpr bool late_cvt(int layout) { return layout == kFp8Frag; }

template <int MODE, int LAYOUT>
__device__ __forceinline__ u32x4_t read_b(const uint8_t* sb, int j, int wn, int fr, int ch) {
  const int n = b_row<MODE>(j, wn, fr);
  if constexpr (byte_codes(LAYOUT)) {
    // one-byte codes: block n/16 of the pair, lane slot (n%16) + 16*chunk holds the 8 codes of the
    // chunk for the pair's first slice, then the same for its second (sb points at the slice's
    // half). With late_cvt the raw codes go to the low half of the fragment and cvt_b makes them
    // bf16 later.
    const u32x2_t v = *(const u32x2_t*)(sb + (n / 16) * 1024 + ((n & 15) + 16 * ch) * 16);
    if constexpr (late_cvt(LAYOUT)) return u32x4_t{v[0], v[1], 0u, 0u};
    return codes_to_bf16x8<LAYOUT>(v[0], v[1]);
  }
  if (LAYOUT == kFrag16)  // block n/16 of the stacked tile; lane position (n%16) + 16*chunk
    return *(const u32x4_t*)(sb + (n / 16) * 1024 + ((n & 15) + 16 * ch) * 16);
  return *(const u32x4_t*)(sb + swz(n, ch));
}

// A B fragment as the MFMA takes it: E4M3 codes (read raw by read_b) become bf16 here, right
// before the MFMAs that use them, so that the LDS read they come from is waited for a step after
// it was issued, and not at once together with every read in flight (FP8 down pass: 1,553 ->
// 1,482 cycles per slice).
template <int LAYOUT>
__device__ __forceinline__ u32x4_t cvt_b(u32x4_t f) {
  if constexpr (late_cvt(LAYOUT)) return codes_to_bf16x8<LAYOUT>(f[0], f[1]);
  return f;
}

// The MFMAs of one 16-wide K step on the fragments in fa / fb, and the LDS reads of the next step
// into the same registers, each issued right after the last MFMA that needs the value it
// replaces: B fragment 0 after the NA MFMAs of column block 0, A fragment i after its MFMA with B
// fragment 1, B fragment 1 last. The NV global-to-LDS loads of the step (load(j), j < NV) follow the
// first MFMAs of column block 0, one after each. Scheduling fences keep exactly this order: left
// to itself the compiler gathers the reads after the last MFMA, and every read's latency then
// shows at the start of the next step.
template <int MODE, int LAYOUT, int NA, int NV, class Load>
__device__ __forceinline__ void mma_and_read(f32x16_t (&acc)[NA > 0 ? NA : 1][2], u32x4_t (&fa)[NA > 0 ? NA : 1],
                                             u32x4_t (&fb)[2], const uint8_t* sa, const uint8_t* sb, int wm,
                                             int wn, int fr, int ch, Load&& load) {
  if constexpr (Geo<MODE>::NBJ == 1) {  // the router: one column block, the reads after its MFMAs
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      acc[i][0] = mfma32x32x16(fb[0], fa[i], acc[i][0]);
      if (i < NV) {
        __builtin_amdgcn_sched_barrier(0);
        load(i);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int j = NA; j < NV; ++j) load(j);
    __builtin_amdgcn_sched_barrier(0);
    if (NA > 0) fb[0] = read_b<MODE, LAYOUT>(sb, 0, wn, fr, ch);
#pragma unroll
    for (int i = 0; i < NA; ++i) fa[i] = read_a<MODE>(sa, i, wm, fr, ch);
    __builtin_amdgcn_sched_barrier(0);
    return;
  }
  if constexpr (late_cvt(LAYOUT)) {
    if (NA > 0) fb[0] = cvt_b<LAYOUT>(fb[0]);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    acc[i][0] = mfma32x32x16(fb[0], fa[i], acc[i][0]);
    if (i < NV) {
      __builtin_amdgcn_sched_barrier(0);
      load(i);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int j = NA; j < NV; ++j) load(j);
  __builtin_amdgcn_sched_barrier(0);
  if (NA > 0) fb[0] = read_b<MODE, LAYOUT>(sb, 0, wn, fr, ch);
  if constexpr (late_cvt(LAYOUT)) {
    __builtin_amdgcn_sched_barrier(0);
    if (NA > 0) fb[1] = cvt_b<LAYOUT>(fb[1]);
  }
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    __builtin_amdgcn_sched_barrier(0);
    acc[i][1] = mfma32x32x16(fb[1], fa[i], acc[i][1]);
    __builtin_amdgcn_sched_barrier(0);
    fa[i] = read_a<MODE>(sa, i, wm, fr, ch);
  }
  __builtin_amdgcn_sched_barrier(0);
  if (NA > 0) fb[1] = read_b<MODE, LAYOUT>(sb, 1, wn, fr, ch);
  __builtin_amdgcn_sched_barrier(0);
}

// First reads of a tile (nothing to multiply yet).
template <int MODE, int LAYOUT, int NA>
__device__ __forceinline__ void read_all(u32x4_t (&fa)[NA > 0 ? NA : 1], u32x4_t (&fb)[2], const uint8_t* sa,
                                         const uint8_t* sb, int wm, int wn, int fr, int ch) {
  if (NA == 0) return;
  fb[0] = read_b<MODE, LAYOUT>(sb, 0, wn, fr, ch);
#pragma unroll
  for (int i = 0; i < NA; ++i) fa[i] = read_a<MODE>(sa, i, wm, fr, ch);
  if constexpr (Geo<MODE>::NBJ == 2) fb[1] = read_b<MODE, LAYOUT>(sb, 1, wn, fr, ch);
}

// The float32 row scales of a one-byte weight buffer: they follow its `ncodes` codes.
__device__ __forceinline__ const float* code_scales(const void* w, size_t ncodes) {
  return (const float*)((const int8_t*)w + ncodes);
}

// s_waitcnt through the builtin, so that the compiler's own wait insertion knows what has landed
// (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8; a field at its maximum waits
// for nothing).
template <int N> __device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }
// Workgroup barrier with no fence: the waits the ring needs come before it, explicitly.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

}  // namespace

// ------------------------------------------------------------------------------- schedule
// Rows of group g (routed groups clamp their offsets into [0, rows]; the shared group has T).
__device__ __forceinline__ long long group_rows(const FfnGroups& p, int g, long long* first) {
  if (g < p.E) {
    long long lo = p.offsets[g], hi = p.offsets[g + 1];
    lo = lo < 0 ? 0 : (lo > p.rows ? p.rows : lo);
    hi = hi < lo ? lo : (hi > p.rows ? p.rows : hi);
    if (first) *first = lo;
    return hi - lo;
  }
  if (first) *first = 0;
  return p.T;
}

// One block. For every group: m-tiles = ceil(rows / BM), tiles = m-tiles * n-tiles; writes the
// exclusive prefix sums of the tiles of the gate/up pass (sched_gu) and the down pass (sched_dn), and
// the first 16-row band of every routed group in the packed activations (pband: ceil(rows / 16)
// bands per group), 1024 groups per round with the running totals carried between rounds.
//
// It also cuts each pass's tile sequence into kXcds contiguous ranges of about equal work (xb_gu,
// xb_dn: kXcds + 1 bounds), one per XCD: with equal tile counts the XCD holding the shared expert's
// full tiles would get the most work and every other XCD would wait for it. The work of an M-tile
// with b 32-row blocks is modelled in units of about 128 cycles, from per-tile timings of both
// passes. Gate/up: 2 ceil(b / 2) + 3 per K slice (the slice time barely moves with b: the operand
// stream sets it) plus 192 for set-up and epilogue. Down: 5 b / 4 per K slice (each SIMD runs the
// MFMAs of all b blocks, two waves of it; about 156 cycles per block and slice) plus 112 for
// set-up, pipeline fill and the staged epilogue. A bound inside a group goes to
// the tile at the same fraction of the group's tiles as the target is of its work. With fewer than
// four tiles per CU the ranges stay equal in count: there a range's time is set by how many rounds
// of tiles its CUs run, not by the sum of its work.
// With more than 1024 groups a first pass over them finds the totals; the last pass writes
// everything.
__device__ __forceinline__ long long tile_work(long long blocks, long long nk) {
  return (2 * ((blocks + 1) / 2) + 3) * nk + 192;
}
__device__ __forceinline__ long long tile_work_down(long long blocks, long long nk) {
  return 5 * blocks * nk / 4 + 112;
}

__global__ void __launch_bounds__(1024)
gemm_schedule_kernel(const FfnGroups p, int32_t* __restrict__ sched_gu, int32_t* __restrict__ sched_dn,
                     int32_t* __restrict__ pband, int32_t* __restrict__ xb_gu, int32_t* __restrict__ xb_dn,
                     int32_t* __restrict__ ctr) {
  constexpr int kQ = 5;  // per group: gate/up tiles, down tiles, bands, gate/up work, down work
  constexpr int BM = Geo<kGateUp>::BM;
  static_assert(Geo<kDown>::BM == BM, "one M-tiling for both passes");
  __shared__ long long wtot[kQ][16];
  const int ngroups = p.E + (p.Hs > 0 ? 1 : 0);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  long long total[kQ] = {0, 0, 0, 0, 0};
  const bool one_round = ngroups <= 1024;  // then the totals are known after the round's scan
  for (int pass = one_round ? 1 : 0; pass < 2; ++pass) {
    long long carry[kQ] = {0, 0, 0, 0, 0};
    for (int base = 0; base < ngroups; base += 1024) {
      const int g = base + (int)threadIdx.x;
      long long v[kQ] = {0, 0, 0, 0, 0};
      long long mt = 0, ntg = 0, ntd = 0, nkg = 0, nkd = 0;
      if (g < ngroups) {
        const long long n = group_rows(p, g, nullptr);
        const int Hg = g < p.E ? p.H : p.Hs;
        mt = (n + BM - 1) / BM;
        const int bn_up = p.gelu ? Geo<kGeluUp>::BN : Geo<kGateUp>::BN;  // 256 weight rows per tile either way
        ntg = (Hg + bn_up - 1) / bn_up;
        ntd = (p.d + Geo<kDown>::BN - 1) / Geo<kDown>::BN;
        nkg = (p.d + BK - 1) / BK;
        nkd = (Hg + BK - 1) / BK;
        const long long b_last = mt > 0 ? (n - (mt - 1) * BM + 31) / 32 : 0;  // blocks of the last M-tile
        v[0] = mt * ntg;
        v[1] = mt * ntd;
        v[2] = g < p.E ? (n + 15) / 16 : 0;
        v[3] = mt > 0 ? ntg * ((mt - 1) * tile_work(BM / 32, nkg) + tile_work(b_last, nkg)) : 0;
        v[4] = mt > 0 ? ntd * ((mt - 1) * tile_work_down(BM / 32, nkd) + tile_work_down(b_last, nkd)) : 0;
      }
      long long inc[kQ];
#pragma unroll
      for (int q = 0; q < kQ; ++q) inc[q] = v[q];
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
          const long long o = __shfl_up(inc[q], off, 64);
          if (lane >= off) inc[q] += o;
        }
      }
      if (lane == 63)
        for (int q = 0; q < kQ; ++q) wtot[q][wave] = inc[q];
      __syncthreads();
      if (one_round)
        for (int w = 0; w < 16; ++w)
          for (int q = 0; q < kQ; ++q) total[q] += wtot[q][w];
      long long ex[kQ];
#pragma unroll
      for (int q = 0; q < kQ; ++q) ex[q] = carry[q] + inc[q] - v[q];
      for (int w = 0; w < wave; ++w)
        for (int q = 0; q < kQ; ++q) ex[q] += wtot[q][w];
      if (pass == 1 && g < ngroups) {
        sched_gu[g] = (int32_t)ex[0];
        sched_dn[g] = (int32_t)ex[1];
        pband[g] = (int32_t)ex[2];
        if (g == ngroups - 1) {
          sched_gu[ngroups] = (int32_t)(ex[0] + v[0]);
          sched_dn[ngroups] = (int32_t)(ex[1] + v[1]);
          pband[ngroups] = (int32_t)(ex[2] + v[2]);
        }
        // XCD bounds inside this group: target work x * total / kXcds in [ex, ex + v), placed at
        // the tile whose share of the group's tiles equals the target's share of its work (all
        // tiles of a group but its last M-tile's cost the same)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const long long w0 = ex[3 + q], wg = v[3 + q];
          if (total[q] < kXcds * kCusPerXcd * 4) continue;  // equal counts (below)
          for (int x = 1; x < kXcds; ++x) {
            const long long target = total[3 + q] * x / kXcds;
            if (wg > 0 && target >= w0 && target < w0 + wg) {
              const long long i = ((target - w0) * v[q] + wg / 2) / wg;   // <= v[q]
              (q == 0 ? xb_gu : xb_dn)[x] = (int32_t)(ex[q] + i);
            }
          }
        }
      }
      for (int w = 0; w < 16; ++w)
        for (int q = 0; q < kQ; ++q) carry[q] += wtot[q][w];
      __syncthreads();  // wtot is rewritten in the next round
    }
#pragma unroll
    for (int q = 0; q < kQ; ++q) total[q] = carry[q];  // the same in every thread
  }
  if (threadIdx.x < 2 * kXcds) ctr[threadIdx.x * kCtrStride] = 0;  // tile counters of both passes
  if (threadIdx.x == 0) {
    xb_gu[0] = 0;
    xb_dn[0] = 0;
    xb_gu[kXcds] = (int32_t)total[0];
    xb_dn[kXcds] = (int32_t)total[1];
    for (int x = 1; x < kXcds; ++x) {  // equal counts, or no work: nobody else writes a bound
      const long long eg = (total[0] + kXcds - 1) / kXcds * x, ed = (total[1] + kXcds - 1) / kXcds * x;
      if (total[0] < kXcds * kCusPerXcd * 4 || total[3] == 0) xb_gu[x] = (int32_t)(eg < total[0] ? eg : total[0]);
      if (total[1] < kXcds * kCusPerXcd * 4 || total[4] == 0) xb_dn[x] = (int32_t)(ed < total[1] ? ed : total[1]);
    }
  }
}

// ------------------------------------------------------------------------------- the GEMM
struct GemmArgs {
  FfnGroups p;
  const int32_t* sched;   // [ngroups + 1] (kGateUp / kDown); unused for the router
  const int32_t* pband;   // [E + 1] first packed band of every routed group (kGateUp / kDown)
  const int32_t* xb;      // [kXcds + 1] tile ranges of the XCDs (kGateUp / kDown)
  int32_t* ctr;           // [kXcds * kCtrStride] tile counters of the XCDs' ranges, zeroed by the schedule
  // router mode
  const void* x;          // [T, d]
  const void* w;          // [E, d]
  const float* bias;      // [E] or NULL
  float* logits;          // [T, E]
  int T, E, d;
};

// Everything one tile's main loop needs, set up once per tile.
template <int MODE>
struct TileCtx {
  int g;                  // group (expert; E = shared expert)
  long long r0;           // first row of the tile in its group's row space (group row base + m0)
  long long pr0;          // first packed row of the tile (expert passes: group band * 16 + m0)
  int rows;               // valid rows in the tile (1..BM)
  int n0, N, K, nk;       // first output column, output columns, reduction length, K slices
  int first;              // first load slot of this wave
  const uint16_t* src[Geo<MODE>::L_HI];  // per load: lane's source at K slice 0
  int kc[Geo<MODE>::L_HI];               // per load: element offset of the lane's chunk in a slice
  int stride[Geo<MODE>::L_HI];           // per load: elements to advance per K slice (wave-uniform)
  // one-byte weights, the weight-loading waves: lane's source of its two blocks in the first half
  // of a pair (qodd: loaded by odd slices) and the second half (qeven), at pair 0; pairs in K
  const int8_t* qodd[2];
  const int8_t* qeven[2];
  int npairs;
};

// Tile count of a launch: from the router's sizes, or the schedule's running total.
template <int MODE>
__device__ __forceinline__ int gemm_total_tiles(const GemmArgs& ga) {
  if (MODE == kRouter) return ((ga.T + Geo<MODE>::BM - 1) / Geo<MODE>::BM) * ((ga.E + Geo<MODE>::BN - 1) / Geo<MODE>::BN);
  return ga.sched[ga.p.E + (ga.p.Hs > 0 ? 1 : 0)];
}

// Main loop and epilogue of one tile for a wave that owns NA active row blocks and issues L loads
// per slice.
template <int MODE, int LAYOUT, int NA, int L>
__device__ __forceinline__ void tile_body(const GemmArgs& ga, const TileCtx<MODE>& c,
                                          uint8_t (*smem)[Slots<MODE, LAYOUT>::STAGE], int wv) {
  using G = Geo<MODE>;
  constexpr int NAF = NA > 0 ? NA : 1;
  const int lane = lane_id();
  const int K = c.K, nk = c.nk;
  typedef __attribute__((address_space(3))) void lds_t;

  // Loads j in [j0, j1) of slice kt into ring buffer `buf`. A slice index past the end is clamped
  // to the last slice: such loads fill a buffer that is never read again, which keeps the number
  // of loads per slice fixed for the vmcnt arithmetic below.
  // Cache policy of this wave's loads. In the expert passes the waves with L_LO loads fetch only
  // weight blocks, which (a bucket being one M-tile) no other workgroup reads again: they load with
  // the non-temporal hint (policy bit NT = 2), leaving L2 to the activation rows that every N-tile
  // of the expert shares.
  using Sl = Slots<MODE, LAYOUT>;
  constexpr bool kQB = Sl::Q && L == Sl::L_LO && Sl::L_LO != Sl::L_HI;   // this wave loads one-byte weight blocks
  constexpr int kAux = (MODE != kRouter && L == Sl::L_LO && Sl::L_LO != Sl::L_HI) ? 2 : 0;
  static_assert(MODE == kRouter || Sl::N_HI * Sl::L_HI == G::A_INSTR, "the L_LO waves load weights only");
  uint8_t* const bring = &smem[0][0] + kStages * Sl::STAGE;   // one-byte weights: the pair ring
  auto issue = [&](int kt, int buf, int j0, int j1) {
    const int kcl = kt < nk ? kt : nk - 1;
#pragma unroll
    for (int i = 0; i < L; ++i) {
      if (i < j0 || i >= j1) continue;
      if constexpr (kQB) {
        // half a pair (see Slots): pair (kt + 1) / 2, first half for odd kt (kt = -1: pair 0),
        // second half for even kt. A pair past the end re-reads the last one into the pair buffer
        // that no slice still to be read uses.
        const int pair = (kt + 1) >> 1;
        const int ps = pair < c.npairs ? pair : c.npairs - 1;
        const int pd = pair < c.npairs ? pair : c.npairs;
        const int blk = c.first + i - G::A_INSTR + ((kt & 1) ? 0 : Sl::B_INSTR);
        const int8_t* s = ((kt & 1) ? c.qodd[i] : c.qeven[i]) + (size_t)ps * 1024;
        __builtin_amdgcn_global_load_lds((const void*)s, (lds_t*)(bring + (pd % kBPairs) * Sl::PAIR + blk * 1024), 16,
                                         0, kAux);
        continue;
      }
      const int k = kcl * BK + c.kc[i];
      const uint16_t* s = c.src[i] + (LAYOUT == kFrag16 || k < K ? (size_t)kcl * c.stride[i] + c.kc[i] : 0);  // past K: zeroed later
      __builtin_amdgcn_global_load_lds((const void*)s, (lds_t*)(smem[buf] + (c.first + i) * 1024), 16, 0, kAux);
    }
  };
  // chunks past K in the last slice: write zeros over what the loads brought in
  auto zero_tail = [&](int kt, int buf) {
    const u32x4_t zero = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < L; ++i)
      if (kt * BK + c.kc[i] >= K) *(u32x4_t*)(smem[buf] + (c.first + i) * 1024 + lane * 16) = zero;
  };

  f32x16_t acc[NAF][2];
#pragma unroll
  for (int i = 0; i < NAF; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int fr = lane & 31, fh = lane >> 5;   // fragment row / k-half of this lane
  const int wm = wv / kWavesN, wn = wv % kWavesN;

  // Ring protocol (S = kStages). The loads of slice s go to buffer s % S and are issued in two
  // parts spread over the MFMAs: part 1 (loads [0, P1)) during step 1 of slice s-S, part 2 (the
  // rest) during step 0 of slice s-S+1, both after the barrier that ends every wave's reads of
  // slice s-S, the previous tenant of the buffer. Before step 1 of slice kt a wave waits for its
  // loads of slice kt+1: slices kt+2 .. kt+S-1 have been issued in full by then and loads complete
  // in issue order, so vmcnt((S-2) * L) leaves exactly those outstanding. The barrier that follows
  // makes every wave's part of slice kt+1 visible. Slices past the end are clamped copies of the
  // last one (see issue); in the last step the buffer of slice kt+1 (free: its previous tenant was
  // slice kt+1-S) takes them, since the current buffer may still be read by waves that are behind
  // and no barrier follows.
  constexpr int S = kStages;
  static_assert(S >= 3, "the issue schedule below needs a ring of at least 3 slices");
  constexpr int P1 = Sl::SPLIT < L ? Sl::SPLIT : L;
  constexpr int kAhead = (S - 2) * L;   // loads allowed in flight when slice kt+1 must land
  static_assert(kAhead + P1 < 64, "vmcnt holds 6 bits");
  auto arrive = [&](int kt) {
    wait_vmcnt<kAhead>();
    if (LAYOUT != kFrag16 && kt == nk - 1 && (K % BK)) zero_tail(kt, kt % S);  // its loads have all landed here
    wait_lgkmcnt0();
    lds_barrier();
  };

  static_assert(BK / 16 == 2, "the loop below is written for two K steps per slice");
  // the B fragments of slice kt: in its stage (bf16), or its half of its pair (one-byte codes)
  auto bslice = [&](int kt) -> const uint8_t* {
    if constexpr (Sl::Q) return bring + ((kt >> 1) % kBPairs) * Sl::PAIR + (kt & 1) * 8;
    else return smem[kt % S] + G::A_BYTES;
  };
  u32x4_t fa[NAF], fb[2];
  if constexpr (kQB) issue(-1, 0, 0, L);   // the first half of pair 0 (the loads of slice -1)
#pragma unroll
  for (int i = 0; i < S - 1; ++i) issue(i, i, 0, L);
  issue(S - 1, S - 1, 0, P1);
  wait_vmcnt<kAhead + P1>();
  if (LAYOUT != kFrag16 && nk == 1 && (K % BK)) zero_tail(0, 0);
  wait_lgkmcnt0();
  lds_barrier();
  read_all<MODE, LAYOUT, NA>(fa, fb, smem[0], bslice(0), wm, wn, fr, fh);
  // Step 0 of slice kt (S0) multiplies while reading step 1 (chunks 2, 3 of the same slice) and
  // issuing part 2 of slice kt+S-1; step 1 (S1) multiplies while reading step 0 of slice kt+1 and
  // issuing part 1 of slice kt+S into slice kt's buffer. The loop runs S1(kt) S0(kt+1) arrive(kt+2),
  // so that its body is one straight block that closes right after a barrier, where no LDS read is
  // in flight (the last two steps are peeled off, with no barrier). The last slice's S1 re-reads the
  // current buffer (the values are never used) and sends its loads to the next buffer, since waves
  // that are behind may still read the current one and no barrier follows.
  auto s0 = [&](int kt) {
    mma_and_read<MODE, LAYOUT, NA, L - P1>(acc, fa, fb, smem[kt % S], bslice(kt), wm, wn, fr,
                                           2 + fh, [&](int j) { issue(kt + S - 1, (kt + S - 1) % S, P1 + j, P1 + j + 1); });
  };
  auto s1 = [&](int kt, int rslice, int lbuf) {
    mma_and_read<MODE, LAYOUT, NA, P1>(acc, fa, fb, smem[rslice % S], bslice(rslice), wm, wn, fr, fh,
                                       [&](int j) { issue(kt + S, lbuf, j, j + 1); });
  };
  s0(0);
  if (nk > 1) arrive(1);
  for (int kt = 0; kt + 2 < nk; ++kt) {
    s1(kt, kt + 1, kt % S);
    s0(kt + 1);
    arrive(kt + 2);
  }
  if (nk > 1) {
    s1(nk - 2, nk - 1, (nk - 2) % S);
    s0(nk - 1);
  }
  s1(nk - 1, nk - 1, nk % S);
  wait_vmcnt<0>();  // no load may still write LDS when the tile ends

  if constexpr (Sl::Q && MODE != kRouter) {
    // One-byte weights: each weight row's scale multiplies its fp32 sums (output column n of the
    // tile), once, before either epilogue. The lane's 4 columns of each (column block, chunk):
    // gate/up blocks 0 and 1 are the gate and up rows of the same hidden columns.
    const FfnGroups& qp = ga.p;
    const float* s0;
    const float* s1;
    if (first_pass(MODE)) {
      s0 = c.g < qp.E ? code_scales(qp.w_gate, (size_t)qp.E * qp.H * qp.d) + (size_t)c.g * qp.H
                      : code_scales(qp.ws_gate, (size_t)qp.Hs * qp.d);
      s1 = c.g < qp.E ? code_scales(qp.w_up, (size_t)qp.E * qp.H * qp.d) + (size_t)c.g * qp.H
                      : code_scales(qp.ws_up, (size_t)qp.Hs * qp.d);
    } else {
      s0 = s1 = c.g < qp.E ? code_scales(qp.w_down, (size_t)qp.E * qp.d * qp.H) + (size_t)c.g * qp.d
                           : code_scales(qp.ws_down, (size_t)qp.d * qp.Hs);
    }
    f32x4_t sc[2][4];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        int n = (MODE == kGateUp ? c.n0 + wn * 32 : c.n0 + wn * 64 + j * 32) + q * 8 + fh * 4;
        n = n + 4 <= c.N ? n : c.N - 4;   // columns past N (N a multiple of 64) are never stored
        sc[j][q] = *(const f32x4_t*)((j ? s1 : s0) + n);
      }
#pragma unroll
    for (int i = 0; i < NAF; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][j][4 * q + e] *= sc[j][q][e];
  }

  // ---- epilogue ----------------------------------------------------------------------------------
  // The MFMAs take the weights as their first operand, so each 32x32 block holds the transposed
  // product: lane l has output row fr = l % 32 of the block and, for q = 0..3, the four
  // consecutive output columns 8 q + 4 fh .. + 3 (e = 4 q .. 4 q + 3), one 8-byte store each.
  // The lane index is re-read through an opaque move so that no output address is computed
  // before the main loop (hoisted addresses would stay live in registers across it).
  int elane = lane;
  asm volatile("" : "+v"(elane));
  const int efr = elane & 31, efh = elane >> 5;
  const FfnGroups& p = ga.p;
  // gate/up: the hidden activation goes to the packed layout the down pass reads (columns padded
  // to a multiple of 32 with zeros; the shared group's region follows the routed one)
  const int np = (int)gemm_pad32(c.N);
  uint16_t* hid = (uint16_t*)p.hid + (c.g < p.E ? 0 : (size_t)p.rbands * 16 * gemm_pad32(p.H));
  uint16_t* y = (uint16_t*)p.y + (c.g < p.E ? 0 : (size_t)p.rows * p.d);
  if constexpr (packed_a(MODE)) {
    // Output rows are 512-byte segments of y: stage each half of the tile (160 rows x 256
    // columns, 80 KB) in LDS, then store it with 16-byte stores, a row per 32 lanes. In LDS a
    // row's 16-byte chunk c sits at chunk c ^ (row % 32), so the 32 rows a store instruction of the
    // accumulators touches fall in distinct banks. The GELU expert's second linear adds its bias
    // (fp32) before the rounding.
    const float* b2 = MODE == kGeluDown && p.b2 ? p.b2 + (size_t)c.g * p.d : nullptr;
    static_assert(G::MBW == 5 && G::BN == 256 && 160 * 512 <= kStages * Sl::STAGE, "staging layout");
    uint8_t* lt = &smem[0][0];
    int tid = (int)threadIdx.x;
    asm volatile("" : "+v"(tid));  // (as for the lane index above)
    __syncthreads();  // every wave's reads of the ring are over (its loads have landed above)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        const int b = wm + 2 * i;
        if (b / 5 != h) continue;
        const int rl = (b - 5 * h) * 32 + efr;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int nl = wn * 64 + j * 32 + q * 8 + efh * 4;
            float v[4] = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
            if (MODE == kGeluDown && b2 && c.n0 + nl < c.N) {  // N is a multiple of 8: 4 columns all in or all out
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] += b2[c.n0 + nl + e];
            }
            *(u32x2_t*)(lt + rl * 512 + (((nl >> 3) ^ (rl & 31)) << 4) + (nl & 4) * 2) =
                u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          }
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < 160 * 32 / kThreads; ++k) {
        const int idx = k * kThreads + tid;
        const int rl = idx >> 5, ch = idx & 31;
        const int row = 160 * h + rl, n = c.n0 + ch * 8;
        if (row < c.rows && n < c.N)
          *(u32x4_t*)(y + (size_t)(c.r0 + row) * c.N + n) = *(const u32x4_t*)(lt + rl * 512 + ((ch ^ (rl & 31)) << 4));
      }
      __syncthreads();
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int row = (wm + 2 * i) * 32 + efr;
    if (row >= c.rows) continue;
#pragma unroll
    for (int j = 0; j < (MODE == kGateUp ? 1 : G::NBJ); ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = c.n0 + (MODE == kGateUp ? wn * 32 : wn * 32 * G::NBJ + j * 32) + q * 8 + efh * 4;  // 4 columns
        if (MODE == kGateUp) {
          if (n >= np) continue;  // N, np and n are multiples of 4: the four columns are all in or all out
          u32x2_t v = {0u, 0u};
          if (n < c.N) {
            float g4[4], u4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              g4[e] = acc[i][0][4 * q + e];
              u4[e] = acc[i][1][4 * q + e];
            }
            v = u32x2_t{pack_bf16x2(silu(g4[0]) * u4[0], silu(g4[1]) * u4[1]),
                        pack_bf16x2(silu(g4[2]) * u4[2], silu(g4[3]) * u4[3])};
          }
          *(u32x2_t*)(hid + frag16_offset((size_t)(c.pr0 + row), (size_t)n, (size_t)np)) = v;
        } else if (MODE == kGeluUp) {
          if (n >= np) continue;  // (as for gate/up)
          u32x2_t v = {0u, 0u};
          if (n < c.N) {
            const float* b1 = p.b1 ? p.b1 + (size_t)c.g * p.H + n : nullptr;
            float z[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) z[e] = gelu_exact(acc[i][j][4 * q + e] + (b1 ? b1[e] : 0.f));
            v = u32x2_t{pack_bf16x2(z[0], z[1]), pack_bf16x2(z[2], z[3])};
          }
          *(u32x2_t*)(hid + frag16_offset((size_t)(c.pr0 + row), (size_t)n, (size_t)np)) = v;
        } else if (MODE == kDown) {
          if (n >= c.N) continue;
          *(u32x2_t*)(y + (size_t)(c.r0 + row) * c.N + n) =
              u32x2_t{pack_bf16x2(acc[i][j][4 * q], acc[i][j][4 * q + 1]),
                      pack_bf16x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3])};
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t)
            if (n + t < c.N)
              ga.logits[(size_t)(c.r0 + row) * c.N + n + t] = acc[i][j][4 * q + t] + (ga.bias ? ga.bias[n + t] : 0.f);
        }
      }
    }
  }
}

// The body specialised on the wave's active row-block count.
template <int MODE, int LAYOUT, int L>
__device__ __forceinline__ void tile_body_na(const GemmArgs& ga, const TileCtx<MODE>& c,
                                             uint8_t (*smem)[Slots<MODE, LAYOUT>::STAGE], int wv, int na) {
  switch (na) {
    case 0: tile_body<MODE, LAYOUT, 0, L>(ga, c, smem, wv); break;
    case 1: tile_body<MODE, LAYOUT, 1, L>(ga, c, smem, wv); break;
    case 2: tile_body<MODE, LAYOUT, 2, L>(ga, c, smem, wv); break;
    case 3: if constexpr (Geo<MODE>::MBW >= 3) tile_body<MODE, LAYOUT, 3, L>(ga, c, smem, wv); break;
    case 4: if constexpr (Geo<MODE>::MBW >= 4) tile_body<MODE, LAYOUT, 4, L>(ga, c, smem, wv); break;
    default: if constexpr (Geo<MODE>::MBW >= 5) tile_body<MODE, LAYOUT, 5, L>(ga, c, smem, wv); break;
  }
}

// One output tile t (0 <= t < gemm_total_tiles) through the LDS ring `smem`.
template <int MODE, int LAYOUT>
__device__ __forceinline__ void gemm_tile(const GemmArgs& ga, const int t, uint8_t (*smem)[Slots<MODE, LAYOUT>::STAGE]) {
  using G = Geo<MODE>;
  const FfnGroups& p = ga.p;
  const int lane = lane_id();
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));  // wave index, 0..7

  // ---- which tile --------------------------------------------------------------------------
  TileCtx<MODE> c;
  int mt = 0, nt = 0;
  long long gr0 = 0;     // first row of the group in its row space
  int nrows = 0;         // rows in the group
  const uint16_t* Bp[2] = {nullptr, nullptr};
  const int8_t* QB[2] = {nullptr, nullptr};   // one-byte codes of the group's matrices
  c.g = 0;
  if (MODE == kRouter) {
    const int mtiles = (ga.T + G::BM - 1) / G::BM;
    nt = t / mtiles;
    mt = t % mtiles;
    nrows = ga.T;
    c.N = ga.E;
    c.K = ga.d;
    Bp[0] = (const uint16_t*)ga.w;
  } else {
    const int ngroups = p.E + (p.Hs > 0 ? 1 : 0);
    // The group of tile t is the last g with sched[g] <= t, i.e. (sched is non-decreasing and
    // sched[0] = 0) the number of g in [0, ngroups) with sched[g] <= t, minus one: the wave counts
    // them with independent loads (one memory latency, not one per bisection step).
    int cnt = 0;
    for (int b = 0; b < ngroups; b += 256) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int gi = b + q * 64 + lane;
        cnt += (gi < ngroups && ga.sched[gi] <= t) ? 1 : 0;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) cnt += __shfl_xor(cnt, off, 64);
    c.g = __builtin_amdgcn_readfirstlane(cnt) - 1;
    int Hg;
    if (c.g < p.E) {
      long long a = p.offsets[c.g], b = p.offsets[c.g + 1];
      a = a < 0 ? 0 : (a > p.rows ? p.rows : a);
      b = b < a ? a : (b > p.rows ? p.rows : b);
      gr0 = a;
      nrows = (int)(b - a);
      Hg = p.H;
    } else {
      gr0 = 0;
      nrows = p.T;
      Hg = p.Hs;
    }
    const size_t wsz = (size_t)p.H * p.d;
    if (first_pass(MODE)) {  // gate/up, or the GELU expert's W1 (held in w_gate)
      c.N = Hg;
      c.K = p.d;
      Bp[0] = c.g < p.E ? (const uint16_t*)p.w_gate + (size_t)c.g * wsz : (const uint16_t*)p.ws_gate;
      if (MODE == kGateUp)
        Bp[1] = c.g < p.E ? (const uint16_t*)p.w_up + (size_t)c.g * wsz : (const uint16_t*)p.ws_up;
      if constexpr (byte_codes(LAYOUT)) {
        QB[0] = c.g < p.E ? (const int8_t*)p.w_gate + (size_t)c.g * wsz : (const int8_t*)p.ws_gate;
        QB[1] = c.g < p.E ? (const int8_t*)p.w_up + (size_t)c.g * wsz : (const int8_t*)p.ws_up;
      }
    } else {
      c.N = p.d;
      c.K = Hg;
      Bp[0] = c.g < p.E ? (const uint16_t*)p.w_down + (size_t)c.g * wsz : (const uint16_t*)p.ws_down;
      if constexpr (byte_codes(LAYOUT))
        QB[0] = c.g < p.E ? (const int8_t*)p.w_down + (size_t)c.g * wsz : (const int8_t*)p.ws_down;
    }
    // super-tile order within the group: blocks of kMBlock M-tiles, N-tile by N-tile inside a block
    const int mtiles = (nrows + G::BM - 1) / G::BM;
    const int ntiles = (c.N + G::BN - 1) / G::BN;
    const int local = t - ga.sched[c.g];
    const int mb0 = local / (kMBlock * ntiles) * kMBlock;
    const int mb = mtiles - mb0 < kMBlock ? mtiles - mb0 : kMBlock;
    const int within = local - mb0 * ntiles;
    nt = within / mb;
    mt = mb0 + within % mb;
  }
  const int m0 = mt * G::BM;
  c.rows = nrows - m0 < G::BM ? nrows - m0 : G::BM;
  c.r0 = gr0 + m0;
  c.n0 = nt * G::BN;
  c.nk = (c.K + BK - 1) / BK;
  // expert passes: the hidden activations of the tile are packed bands band0 + m0/16 + s of its
  // group's region (written by gate/up, read by down)
  const long long band0 = MODE == kRouter ? 0 : (c.g < p.E ? (long long)ga.pband[c.g] : 0);
  const int gbands = (nrows + 15) / 16;
  c.pr0 = band0 * 16 + m0;
  const uint16_t* abase =
      packed_a(MODE) ? (const uint16_t*)p.hid + (c.g < p.E ? 0 : (size_t)p.rbands * 16 * gemm_pad32(p.H)) : nullptr;

  // ---- this wave's loads: slots [first, first + L) of the slice's INSTR 1 KB loads -------------
  // Slot s < A_INSTR: A rows [16 s, 16 s + 16), lane l -> row 16 s + l/4, physical chunk l%4 (the
  // logical chunk swz_chunk(row, l%4) of that row). Slot s >= A_INSTR: B block q = s - A_INSTR;
  // fragment-tiled: one contiguous 16 x 32 block of weight band n0/16 + q % (BN/16) of matrix
  // q / (BN/16); row-major: stacked B rows [16 q, 16 q + 16) like A. Slot s lands at LDS byte s * 1024
  // of the slice (A rows first, then the stacked B tiles).
  using Sl = Slots<MODE, LAYOUT>;
  const bool hi_wave = wv < Sl::N_HI;
  c.first = hi_wave ? wv * Sl::L_HI : Sl::N_HI * Sl::L_HI + (wv - Sl::N_HI) * Sl::L_LO;
  const int nload = hi_wave ? Sl::L_HI : Sl::L_LO;
  c.npairs = c.K / 64;
  const int phys = lane & 3;
#pragma unroll
  for (int i = 0; i < Sl::L_HI; ++i) {
    const int s = c.first + (i < nload ? i : 0);
    if (s < G::A_INSTR && !packed_a(MODE)) {
      const int row = s * 16 + (lane >> 2);
      c.kc[i] = swz_chunk(row, phys) * 8;
      c.stride[i] = BK;
      int rr = m0 + row;
      rr = rr < nrows ? rr : (nrows > 0 ? nrows - 1 : 0);  // rows past the tile: any valid row, never stored
      long long src;
      if (MODE == kRouter) {
        src = rr;
      } else if (c.g < p.E) {
        src = p.perm_src ? (long long)(p.perm_src[gr0 + rr] / p.k) : gr0 + rr;
        const long long lim = p.perm_src ? (long long)p.T : p.rows;
        src = src < 0 ? 0 : (src >= lim ? lim - 1 : src);
      } else {
        src = rr;
      }
      c.src[i] = (const uint16_t*)(MODE == kRouter ? ga.x : p.x) + (size_t)src * c.K;
    } else if (s < G::A_INSTR) {
      // packed A: one contiguous 1 KB block per slice. Bands past the group (rows never stored) repeat
      // its last band, which the tile loads anyway: a single zero kilobyte shared by every workgroup
      // drew all of them to one L2 channel and measured slower
      int bl = m0 / 16 + s;
      bl = bl < gbands ? bl : gbands - 1;   // gbands >= 1: a group without rows has no tiles
      c.kc[i] = 0;
      c.stride[i] = 512;
      c.src[i] = abase + (size_t)(band0 + bl) * (c.nk * 512) + lane * 8;
    } else if constexpr (byte_codes(LAYOUT)) {
      // one-byte weight blocks q (first half of a pair) and q + B_INSTR (second half): 16 rows x 64 K
      // of codes each, stacked as in the bf16 tile (gate/up: 8 gate bands, then 8 up bands)
      const int q = s - G::A_INSTR;
      auto src_of = [&](int b) {
        int band = c.n0 / 16 + b % (G::BN / 16);
        band = band < c.N / 16 ? band : c.N / 16 - 1;   // bands past N: any valid band, never stored
        return QB[b / (G::BN / 16)] + (size_t)band * c.npairs * 1024 + lane * 16;
      };
      if (i < 2) {
        c.qodd[i] = src_of(q);
        c.qeven[i] = src_of(q + Sl::B_INSTR);
      }
      c.kc[i] = 0;
      c.stride[i] = 0;
      c.src[i] = nullptr;
    } else {
      const int q = s - G::A_INSTR;
      if (LAYOUT == kFrag16) {
        const int b = q / (G::BN / 16);
        int band = c.n0 / 16 + q % (G::BN / 16);
        band = band < c.N / 16 ? band : c.N / 16 - 1;  // bands past N: any valid band, never stored
        c.kc[i] = 0;
        c.stride[i] = 512;                              // K is a multiple of 32 in this layout: no tail
        c.src[i] = Bp[b] + (size_t)band * (c.K / 32) * 512 + lane * 8;
      } else {
        const int srow = q * 16 + (lane >> 2);          // stacked row of the B tiles
        c.kc[i] = swz_chunk(srow, phys) * 8;
        c.stride[i] = BK;
        const int b = srow / G::BN;
        int n = c.n0 + (srow % G::BN);
        n = n < c.N ? n : c.N - 1;                      // rows past N: any valid row, never stored
        c.src[i] = Bp[b] + (size_t)n * c.K;
      }
    }
  }

  // ---- active row blocks of this wave: blocks wm, wm + 2, ... below ceil(rows / 32) --------------
  const int nbt = (c.rows + 31) / 32;
  const int wm = wv / kWavesN;
  int na = nbt > wm ? (nbt - wm + 1) / 2 : 0;
  na = na < G::MBW ? na : G::MBW;
  if (hi_wave)
    tile_body_na<MODE, LAYOUT, Sl::L_HI>(ga, c, smem, wv, na);
  else if constexpr (Sl::L_LO != Sl::L_HI && Sl::N_HI < kWaves)
    tile_body_na<MODE, LAYOUT, Sl::L_LO>(ga, c, smem, wv, na);
}

// Tiles are numbered expert by expert, in blocks of up to kMBlock M-tiles, N-tile by N-tile within
// a block, with the block's M-tiles of one N-tile adjacent; XCD x owns the contiguous range
// [xb[x], xb[x + 1]) that the schedule balanced by modelled work (the router: equal ranges).
// Router: one workgroup per tile; workgroup L runs on XCD L % 8 and takes the (L / 8)-th tile of
// its XCD's range (then every (gridDim / 8)-th after it).
// Expert passes: one persistent workgroup per compute unit (kXcds x kCusPerXcd, workgroup L on XCD
// L % 8). A workgroup takes the next tile of its XCD's range from the range's counter (so the 32
// CUs of an XCD work on consecutive tiles, in order, as the hardware would dispatch them, without
// a launch between two tiles), and once its range is handed out, the next tile of another XCD's
// range: XCDs run at clocks several percent apart under load, and the ones ahead finish the ones
// behind. Lane y < 8 of wave 0 watches the range of XCD (xcd + y) % 8 (its first tile, its size and
// its counter). Each round the lowest watching lane whose counter still reads below the range size
// takes a number with one atomic add; a number past the range leaves that counter past it for good
// (and the lane's next load sees its own add), so every failed round retires one range and the
// loop ends within kXcds + 1 rounds; a workgroup leaves only once every range is handed out. The
// tile number reaches the other waves through the first word of the LDS ring, free between tiles:
// the workgroup's LDS stays at exactly 144 KiB (one more 4-byte shared variable made both expert
// passes about 1.5x slower on this part).
template <int MODE, int LAYOUT>
__global__ void __launch_bounds__(kThreads, 1)
grouped_gemm_kernel(const GemmArgs ga) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[Slots<MODE, LAYOUT>::LDS];
  auto smem = reinterpret_cast<uint8_t (*)[Slots<MODE, LAYOUT>::STAGE]>(lds);
  const int total = gemm_total_tiles<MODE>(ga);
  const int xcd = (int)blockIdx.x % kXcds;
  if (MODE == kRouter) {
    const int stride = (int)gridDim.x / kXcds;
    const int per = (total + kXcds - 1) / kXcds;
    const int lo = xcd * per < total ? xcd * per : total;
    const int hi = lo + per < total ? lo + per : total;
    for (int t = lo + (int)blockIdx.x / kXcds; t < hi; t += stride) {
      if (t >= lo + stride) __syncthreads();  // the previous tile's LDS reads are over
      gemm_tile<MODE, LAYOUT>(ga, t, smem);
    }
    return;
  }
  const int lane0 = (int)threadIdx.x;
  int d0 = 0, n = 0;
  int32_t* cx = ga.ctr;
  if (lane0 < kXcds) {
    const int x = (xcd + lane0) % kXcds;
    int xl = ga.xb[x], xh = ga.xb[x + 1];
    xl = xl < 0 ? 0 : (xl > total ? total : xl);   // whatever the bounds hold, only tiles in [0, total)
    xh = xh < xl ? xl : (xh > total ? total : xh);
    d0 = xl;
    n = xh - xl;
    cx = ga.ctr + x * kCtrStride;
  }
  int* slot = (int*)&smem[0][0];
  for (bool busy = false;; busy = true) {
    if (busy) __syncthreads();  // the previous tile's LDS reads are over: the ring is free
    if (lane0 < 64) {
      int got_t = -1;
      for (int round = 0; round <= kXcds && got_t < 0; ++round) {
        const bool avail =
            lane0 < kXcds && n > 0 && __hip_atomic_load(cx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < n;
        const unsigned long long m = __ballot(avail);
        if (m == 0) break;
        const int src = __ffsll(m) - 1;
        int got = -1;
        if (lane0 == src) {
          const int d = atomicAdd(cx, 1);
          got = d < n ? d0 + d : -1;
        }
        got_t = __shfl(got, src, 64);
      }
      if (lane0 == 0) *slot = got_t;
    }
    __syncthreads();
    const int t = *slot;
    __syncthreads();  // every wave has its copy before the tile's loads refill the ring
    if (t < 0) break;
    gemm_tile<MODE, LAYOUT>(ga, t, smem);
  }
}

// ------------------------------------------------------------------------------- launchers
namespace {
int round8(long long v) { return (int)((v + kXcds - 1) / kXcds * kXcds); }

// Router workgroups: one per tile (rounded to whole XCD sets). Expert passes: one persistent
// workgroup per compute unit.
int gemm_grid(long long tiles_upper) { return round8(tiles_upper); }
constexpr int kPersistentGrid = kXcds * kCusPerXcd;
}  // namespace

// [sched_gu | sched_dn | pband] (E + 2 ints each), [xb_gu | xb_dn] (kXcds + 1 each), then the tile
// counters of both passes (kXcds each, one 64-byte line apart)
size_t gemm_schedule_ints(int E) { return 3 * (size_t)(E + 2) + 2 * (kXcds + 1) + 2 * kXcds * kCtrStride + kCtrStride; }

// The tile counters: after the ranges, rounded up to a 64-byte boundary of the schedule buffer.
int32_t* gemm_counters(int32_t* sched, int E) {
  const size_t off = 3 * (size_t)(E + 2) + 2 * (kXcds + 1);
  return sched + (off + kCtrStride - 1) / kCtrStride * kCtrStride;
}

hipError_t launch_gemm_schedule(const FfnGroups& p, int32_t* sched, hipStream_t stream) {
  int32_t* xb = sched + 3 * (p.E + 2);
  hipLaunchKernelGGL(gemm_schedule_kernel, dim3(1), dim3(1024), 0, stream, p, sched, sched + p.E + 2,
                     sched + 2 * (p.E + 2), xb, xb + kXcds + 1, gemm_counters(sched, p.E));
  return hipGetLastError();
}


hipError_t launch_gemm_gate_up(const FfnGroups& p, const int32_t* sched, hipStream_t stream) {
  GemmArgs a{};
  a.p = p;
  a.sched = sched;
  a.pband = sched + 2 * (p.E + 2);
  a.xb = sched + 3 * (p.E + 2);
  a.ctr = gemm_counters(const_cast<int32_t*>(sched), p.E);
  const dim3 grid(kPersistentGrid);
  if (p.gelu && p.layout == kFrag16)
    hipLaunchKernelGGL((grouped_gemm_kernel<kGeluUp, kFrag16>), grid, dim3(kThreads), 0, stream, a);
  else if (p.gelu)
    hipLaunchKernelGGL((grouped_gemm_kernel<kGeluUp, kRowMajor>), grid, dim3(kThreads), 0, stream, a);
  else if (p.layout == kFrag16)
    hipLaunchKernelGGL((grouped_gemm_kernel<kGateUp, kFrag16>), grid, dim3(kThreads), 0, stream, a);
  else if (p.layout == kInt8Frag)
    hipLaunchKernelGGL((grouped_gemm_kernel<kGateUp, kInt8Frag>), grid, dim3(kThreads), 0, stream, a);
  else if (p.layout == kFp8Frag)
    hipLaunchKernelGGL((grouped_gemm_kernel<kGateUp, kFp8Frag>), grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((grouped_gemm_kernel<kGateUp, kRowMajor>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_gemm_down(const FfnGroups& p, const int32_t* sched, hipStream_t stream) {
  GemmArgs a{};
  a.p = p;
  a.sched = sched + p.E + 2;
  a.pband = sched + 2 * (p.E + 2);
  a.xb = sched + 3 * (p.E + 2) + kXcds + 1;
  a.ctr = gemm_counters(const_cast<int32_t*>(sched), p.E) + kXcds * kCtrStride;
  const dim3 grid(kPersistentGrid);
  if (p.gelu && p.layout == kFrag16)
    hipLaunchKernelGGL((grouped_gemm_kernel<kGeluDown, kFrag16>), grid, dim3(kThreads), 0, stream, a);
  else if (p.gelu)
    hipLaunchKernelGGL((grouped_gemm_kernel<kGeluDown, kRowMajor>), grid, dim3(kThreads), 0, stream, a);
  else if (p.layout == kFrag16)
    hipLaunchKernelGGL((grouped_gemm_kernel<kDown, kFrag16>), grid, dim3(kThreads), 0, stream, a);
  else if (p.layout == kInt8Frag)
    hipLaunchKernelGGL((grouped_gemm_kernel<kDown, kInt8Frag>), grid, dim3(kThreads), 0, stream, a);
  else if (p.layout == kFp8Frag)
    hipLaunchKernelGGL((grouped_gemm_kernel<kDown, kFp8Frag>), grid, dim3(kThreads), 0, stream, a);
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
  using G = Geo<kRouter>;
  const long long tiles = (long long)((T + G::BM - 1) / G::BM) * ((E + G::BN - 1) / G::BN);
  hipLaunchKernelGGL((grouped_gemm_kernel<kRouter, kRowMajor>), dim3(gemm_grid(tiles)), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace moe
