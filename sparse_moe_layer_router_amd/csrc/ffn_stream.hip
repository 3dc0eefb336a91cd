// Grouped SwiGLU experts, weight-streaming form (bf16, MFMA 16x16x32).
//
// MoE-kernels page (blog.llmgo.top), section 1.2: with few tokens per expert, every selected
// expert's W_gate, W_up and W_down must be read in full from HBM for one or two token vectors, so
// the expert FFN is a GEMV bound by memory bandwidth; section 4.2: one launch covers all experts,
// the work of each expert found from the offsets array, empty experts skipped.
//
// Layout of the work: block (hb, g) owns 64 consecutive output rows of group g's weight matrix
// (4 waves x 16 rows). A wave streams its 16 weight rows once, front to back, 16 bytes per lane
// per step (each step is one 16x16x32 MFMA A-fragment: lane l reads row l%16, k-chunk l/16), and
// applies each fragment to every 16-token tile of the group's rows (the B-fragment, x^T, read
// from L2). Tokens beyond the group's count are zero-padded columns. Accumulation is fp32 inside
// the MFMA; gate and up share one B-fragment and their accumulators have identical layouts, so
// SiLU(g) * u is formed in registers and stored as bf16. The down projection is the same loop
// with W_down rows against the stored hidden rows.
#include "codes.h"
#include "kernels.h"
#include "moe_device.h"

namespace moe {

namespace {

constexpr int kRowsPerBlock = 64;   // 4 waves x 16 weight rows
constexpr int kUnroll = 8;          // k-steps of 32 issued back to back (8 KB per matrix per wave)
// 16-token tiles a weight fragment is applied to in one pass (NTT): a group of n rows streams its
// weights ceil(n / (16 NTT)) times, and the shared expert is cut into chunks of 16 NTT rows. With
// more than 16 tokens, bf16 weights take NTT = 2 (at a decode batch of 256 that halves the shared
// expert's passes: -2.4% for the layer), at a register cost that still leaves two to three waves per
// SIMD. With 16 tokens or fewer there is one chunk either way, and the INT8 kernels lose more to
// the lower occupancy than they gain: NTT = 1. Four tiles cost too much occupancy everywhere.

struct GroupView {
  long long r0;        // first row of the group in the (routed or shared) row space
  int n;               // rows in the group
  int Hg;              // hidden size of the group's expert
  const void* wg;      // [Hg, d] (bf16, or one-byte INT8 / E4M3 codes in the fragment order)
  const void* wu;      // [Hg, d]
  const void* wd;      // [d, Hg]
  const float* sg;     // one-byte weights: per-row scales of wg [Hg], wu [Hg], wd [d]
  const float* su;
  const float* sd;
  uint16_t* hid;       // hidden rows of this row space, row stride Hg
  uint16_t* y;         // output rows of this row space, row stride d
  bool routed;
};

// One-byte expert weights (MOE_LAYOUT_INT8_FRAG, MOE_LAYOUT_FP8_FRAG): a buffer of n matrices holds n * rows * cols one-byte
// codes followed by n * rows float32 row scales.
__device__ __forceinline__ const float* row_scales(const void* codes, long long n_codes) {
  return (const float*)((const int8_t*)codes + n_codes);
}

// Group g < E is routed expert g. The shared expert's T rows are cut into chunks of `chunk` rows,
// one group each (g = E + c): every chunk streams the shared weights once for its own tokens, and
// the chunks run side by side instead of one group re-streaming the weights for every token tile.
__device__ __forceinline__ GroupView group_view(const FfnGroups& p, int g, int chunk) {
  GroupView v;
  const bool q8 = byte_codes(p.layout);
  const size_t eb = q8 ? 1 : 2;  // bytes per weight element
  v.sg = v.su = v.sd = nullptr;
  if (g < p.E) {
    // clamp to [0, rows] so inconsistent offsets can never address outside the row buffers
    long long a = p.offsets[g], b = p.offsets[g + 1];
    a = a < 0 ? 0 : (a > p.rows ? p.rows : a);
    b = b < a ? a : (b > p.rows ? p.rows : b);
    v.r0 = a;
    v.n = (int)(b - a);
    v.Hg = p.H;
    const size_t wsz = (size_t)p.H * p.d;
    v.wg = (const char*)p.w_gate + (size_t)g * wsz * eb;
    v.wu = (const char*)p.w_up + (size_t)g * wsz * eb;
    v.wd = (const char*)p.w_down + (size_t)g * wsz * eb;
    if (q8) {
      v.sg = row_scales(p.w_gate, (long long)p.E * wsz) + (size_t)g * p.H;
      v.su = row_scales(p.w_up, (long long)p.E * wsz) + (size_t)g * p.H;
      v.sd = row_scales(p.w_down, (long long)p.E * wsz) + (size_t)g * p.d;
    }
    v.hid = (uint16_t*)p.hid;
    v.y = (uint16_t*)p.y;
    v.routed = true;
  } else {
    v.r0 = (long long)(g - p.E) * chunk;
    v.n = (int)(p.T - v.r0 < chunk ? p.T - v.r0 : chunk);
    v.Hg = p.Hs;
    v.wg = p.ws_gate;
    v.wu = p.ws_up;
    v.wd = p.ws_down;
    if (q8) {
      const long long wsz = (long long)p.Hs * p.d;
      v.sg = row_scales(p.ws_gate, wsz);
      v.su = row_scales(p.ws_up, wsz);
      v.sd = row_scales(p.ws_down, wsz);
    }
    v.hid = (uint16_t*)p.hid + (size_t)p.rows * p.H;
    v.y = (uint16_t*)p.y + (size_t)p.rows * p.d;
    v.routed = false;
  }
  return v;
}

// source token (x row) of row r of a group
__device__ __forceinline__ long long source_row(const FfnGroups& p, const GroupView& v, long long r) {
  if (!v.routed) return r;
  long long s = p.perm_src ? (long long)(p.perm_src[r] / p.k) : r;
  long long lim = p.perm_src ? (long long)p.T : p.rows;
  return s < 0 ? 0 : (s >= lim ? lim - 1 : s);  // never read outside x, whatever the indices hold
}

}  // namespace

// Weight fragment source for a wave streaming the 16 rows [r0, r0+16) of a [rows, K] matrix: the
// lane's 16 bytes of k-step s (32 columns) are at base + s * step (bf16 elements).
//   row-major: row r0 + lane%16, columns 8*(lane/16) .. +8 of the step: 16 rows x 64 B per load;
//   fragment-tiled: block (r0/16, s), lane's 16 bytes: one contiguous 1 KB per load.
template <int LAYOUT>
__device__ __forceinline__ const uint16_t* frag_base(const void* wv, int r0, int rows, int K, int lane, int* step) {
  const uint16_t* w = (const uint16_t*)wv;
  if (LAYOUT == kFrag16) {
    *step = 512;
    return w + (size_t)(r0 / 16) * (K / 32) * 512 + lane * 8;
  }
  *step = 32;
  const int r = (r0 + (lane & 15) < rows) ? r0 + (lane & 15) : rows - 1;  // rows past the matrix: dropped
  return w + (size_t)r * K + (lane >> 4) * 8;
}

// One-byte fragment order: 1 KB block (r0/16, s2) covers 64 columns, lane's 16 bytes = its A-operand
// chunk of k-steps 2*s2 and 2*s2+1; base + s2 * 1024 bytes.
__device__ __forceinline__ const int8_t* q8_base(const void* wv, int r0, int K, int lane) {
  return (const int8_t*)wv + (size_t)(r0 / 16) * (K / 64) * 1024 + lane * 16;
}

template <int NTT, int LAYOUT>
__global__ void __launch_bounds__(256)
ffn_gate_up_stream(const FfnGroups p) {
  const GroupView v = group_view(p, blockIdx.y, 16 * NTT);
  if (v.n <= 0) return;
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int h0 = blockIdx.x * kRowsPerBlock + wave * 16;
  if (h0 >= v.Hg) return;
  const int d = p.d;
  const int ar = lane & 15, kq = lane >> 4;
  int ws = 0;  // bf16 layouts: elements between consecutive k-steps of a weight fragment
  const uint16_t* ag = nullptr;
  const uint16_t* au = nullptr;
  const int8_t* qg = nullptr;
  const int8_t* qu = nullptr;
  if (byte_codes(LAYOUT)) {
    qg = q8_base(v.wg, h0, d, lane);
    qu = q8_base(v.wu, h0, d, lane);
  } else {
    ag = frag_base<LAYOUT>(v.wg, h0, v.Hg, d, lane, &ws);
    au = frag_base<LAYOUT>(v.wu, h0, v.Hg, d, lane, &ws);
  }
  const uint16_t* xb = (const uint16_t*)p.x;

  for (int tt = 0; tt < v.n; tt += 16 * NTT) {
    const uint16_t* bx[NTT];
    bool bok[NTT];
#pragma unroll
    for (int j = 0; j < NTT; ++j) {
      const int rr = tt + j * 16 + ar;
      bok[j] = rr < v.n;
      const long long src = bok[j] ? source_row(p, v, v.r0 + rr) : 0;
      bx[j] = xb + (size_t)src * d + kq * 8;
    }
    f32x4_t accg[NTT], accu[NTT];
#pragma unroll
    for (int j = 0; j < NTT; ++j) { accg[j] = f32x4_t{0, 0, 0, 0}; accu[j] = f32x4_t{0, 0, 0, 0}; }
    const u32x4_t zero = {0, 0, 0, 0};
    int k0 = 0;
    if (byte_codes(LAYOUT)) {
      // d is a multiple of 64: every load covers two whole k-steps
      for (; k0 + 32 * kUnroll <= d; k0 += 32 * kUnroll) {
        u32x4_t r_g[kUnroll / 2], r_u[kUnroll / 2], b[kUnroll][NTT];
#pragma unroll
        for (int s2 = 0; s2 < kUnroll / 2; ++s2) {
          r_g[s2] = ld16_stream(qg + (size_t)(k0 / 64 + s2) * 1024);
          r_u[s2] = ld16_stream(qu + (size_t)(k0 / 64 + s2) * 1024);
        }
#pragma unroll
        for (int s = 0; s < kUnroll; ++s)
#pragma unroll
          for (int j = 0; j < NTT; ++j) b[s][j] = bok[j] ? ld16(bx[j] + k0 + 32 * s) : zero;
#pragma unroll
        for (int s2 = 0; s2 < kUnroll / 2; ++s2) {
          const u32x4_t g0 = codes_to_bf16x8<LAYOUT>(r_g[s2][0], r_g[s2][1]), g1 = codes_to_bf16x8<LAYOUT>(r_g[s2][2], r_g[s2][3]);
          const u32x4_t u0 = codes_to_bf16x8<LAYOUT>(r_u[s2][0], r_u[s2][1]), u1 = codes_to_bf16x8<LAYOUT>(r_u[s2][2], r_u[s2][3]);
#pragma unroll
          for (int j = 0; j < NTT; ++j) {
            accg[j] = mfma16x16x32(g0, b[2 * s2][j], accg[j]);
            accu[j] = mfma16x16x32(u0, b[2 * s2][j], accu[j]);
            accg[j] = mfma16x16x32(g1, b[2 * s2 + 1][j], accg[j]);
            accu[j] = mfma16x16x32(u1, b[2 * s2 + 1][j], accu[j]);
          }
        }
      }
      for (; k0 < d; k0 += 64) {
        const u32x4_t r_g = ld16_stream(qg + (size_t)(k0 / 64) * 1024);
        const u32x4_t r_u = ld16_stream(qu + (size_t)(k0 / 64) * 1024);
        const u32x4_t g0 = codes_to_bf16x8<LAYOUT>(r_g[0], r_g[1]), g1 = codes_to_bf16x8<LAYOUT>(r_g[2], r_g[3]);
        const u32x4_t u0 = codes_to_bf16x8<LAYOUT>(r_u[0], r_u[1]), u1 = codes_to_bf16x8<LAYOUT>(r_u[2], r_u[3]);
#pragma unroll
        for (int j = 0; j < NTT; ++j) {
          const u32x4_t b0 = bok[j] ? ld16(bx[j] + k0) : zero;
          const u32x4_t b1 = bok[j] ? ld16(bx[j] + k0 + 32) : zero;
          accg[j] = mfma16x16x32(g0, b0, accg[j]);
          accu[j] = mfma16x16x32(u0, b0, accu[j]);
          accg[j] = mfma16x16x32(g1, b1, accg[j]);
          accu[j] = mfma16x16x32(u1, b1, accu[j]);
        }
      }
    } else {
      for (; k0 + 32 * kUnroll <= d; k0 += 32 * kUnroll) {
        u32x4_t a_g[kUnroll], a_u[kUnroll], b[kUnroll][NTT];
#pragma unroll
        for (int s = 0; s < kUnroll; ++s) {
          a_g[s] = ld16_stream(ag + (size_t)(k0 / 32 + s) * ws);
          a_u[s] = ld16_stream(au + (size_t)(k0 / 32 + s) * ws);
        }
#pragma unroll
        for (int s = 0; s < kUnroll; ++s)
#pragma unroll
          for (int j = 0; j < NTT; ++j) b[s][j] = bok[j] ? ld16(bx[j] + k0 + 32 * s) : zero;
#pragma unroll
        for (int s = 0; s < kUnroll; ++s)
#pragma unroll
          for (int j = 0; j < NTT; ++j) {
            accg[j] = mfma16x16x32(a_g[s], b[s][j], accg[j]);
            accu[j] = mfma16x16x32(a_u[s], b[s][j], accu[j]);
          }
      }
      for (; k0 < d; k0 += 32) {  // tail: d is a multiple of 8, so a lane's 8-chunk is all in or all out
        const bool kok = k0 + kq * 8 < d;
        const u32x4_t a_g = kok ? ld16_stream(ag + (size_t)(k0 / 32) * ws) : zero;
        const u32x4_t a_u = kok ? ld16_stream(au + (size_t)(k0 / 32) * ws) : zero;
#pragma unroll
        for (int j = 0; j < NTT; ++j) {
          const u32x4_t b = (kok && bok[j]) ? ld16(bx[j] + k0) : zero;
          accg[j] = mfma16x16x32(a_g, b, accg[j]);
          accu[j] = mfma16x16x32(a_u, b, accu[j]);
        }
      }
    }
    // lane holds rows h0 + kq*4 + {0..3} of token column (lane & 15); one-byte rows carry their scale
    const int h = h0 + kq * 4;
    f32x4_t sg = {1.f, 1.f, 1.f, 1.f}, su = {1.f, 1.f, 1.f, 1.f};
    if (byte_codes(LAYOUT) && h < v.Hg) {
      sg = *(const f32x4_t*)(v.sg + h);
      su = *(const f32x4_t*)(v.su + h);
    }
#pragma unroll
    for (int j = 0; j < NTT; ++j) {
      const int rr = tt + j * 16 + ar;
      if (rr < v.n && h < v.Hg) {
        f32x4_t g = accg[j], u = accu[j];
        if (byte_codes(LAYOUT)) {
#pragma unroll
          for (int e = 0; e < 4; ++e) { g[e] *= sg[e]; u[e] *= su[e]; }
        }
        uint32_t lo = pack_bf16x2(silu(g[0]) * u[0], silu(g[1]) * u[1]);
        uint32_t hi = pack_bf16x2(silu(g[2]) * u[2], silu(g[3]) * u[3]);
        *(u32x2_t*)(v.hid + (size_t)(v.r0 + rr) * v.Hg + h) = u32x2_t{lo, hi};
      }
    }
  }
}

// One matrix, 16 weight rows, against NTT 16-token tiles: the streaming loop of the down kernel
// below with any B rows (x rows for the first layer). aw / qw: the lane's fragment source (bf16 with
// ws elements between k-steps, or one-byte codes), bsrc: the lane's B row per tile (8 elements at
// its k-chunk; an in-bounds row also for lanes past the group), K: reduction length. With one
// token tile (bf16) the B loads are issued for every lane and the rows past the group zeroed at
// the MFMA, so no load waits behind a per-lane branch (decode T=8: -0.6%); with two tiles the
// second is mostly past the group and its loads stay masked (unmasked, T=256 down took 8% longer).
template <int NTT, int LAYOUT>
__device__ __forceinline__ void stream_rows(const uint16_t* aw, const int8_t* qw, int ws, const uint16_t* const (&bsrc)[NTT],
                                            const bool (&bok)[NTT], int K, int kq, f32x4_t (&acc)[NTT]) {
  const u32x4_t zero = {0, 0, 0, 0};
  int k0 = 0;
  if (byte_codes(LAYOUT)) {
    for (; k0 + 32 * kUnroll <= K; k0 += 32 * kUnroll) {
      u32x4_t r[kUnroll / 2], b[kUnroll][NTT];
#pragma unroll
      for (int s2 = 0; s2 < kUnroll / 2; ++s2) r[s2] = ld16_stream(qw + (size_t)(k0 / 64 + s2) * 1024);
#pragma unroll
      for (int s = 0; s < kUnroll; ++s)
#pragma unroll
        for (int j = 0; j < NTT; ++j) b[s][j] = bok[j] ? ld16(bsrc[j] + k0 + 32 * s) : zero;
#pragma unroll
      for (int s2 = 0; s2 < kUnroll / 2; ++s2) {
        const u32x4_t a0 = codes_to_bf16x8<LAYOUT>(r[s2][0], r[s2][1]), a1 = codes_to_bf16x8<LAYOUT>(r[s2][2], r[s2][3]);
#pragma unroll
        for (int j = 0; j < NTT; ++j) {
          acc[j] = mfma16x16x32(a0, b[2 * s2][j], acc[j]);
          acc[j] = mfma16x16x32(a1, b[2 * s2 + 1][j], acc[j]);
        }
      }
    }
    for (; k0 < K; k0 += 64) {  // one-byte layouts: K is a multiple of 64
      const u32x4_t r = ld16_stream(qw + (size_t)(k0 / 64) * 1024);
      const u32x4_t a0 = codes_to_bf16x8<LAYOUT>(r[0], r[1]), a1 = codes_to_bf16x8<LAYOUT>(r[2], r[3]);
#pragma unroll
      for (int j = 0; j < NTT; ++j) {
        acc[j] = mfma16x16x32(a0, bok[j] ? ld16(bsrc[j] + k0) : zero, acc[j]);
        acc[j] = mfma16x16x32(a1, bok[j] ? ld16(bsrc[j] + k0 + 32) : zero, acc[j]);
      }
    }
  } else {
    for (; k0 + 32 * kUnroll <= K; k0 += 32 * kUnroll) {
      u32x4_t a[kUnroll], b[kUnroll][NTT];
#pragma unroll
      for (int s = 0; s < kUnroll; ++s) a[s] = ld16_stream(aw + (size_t)(k0 / 32 + s) * ws);
#pragma unroll
      for (int s = 0; s < kUnroll; ++s)
#pragma unroll
        for (int j = 0; j < NTT; ++j) b[s][j] = NTT == 1 || bok[j] ? ld16(bsrc[j] + k0 + 32 * s) : zero;
#pragma unroll
      for (int s = 0; s < kUnroll; ++s)
#pragma unroll
        for (int j = 0; j < NTT; ++j) acc[j] = mfma16x16x32(a[s], bok[j] ? b[s][j] : zero, acc[j]);
    }
    for (; k0 < K; k0 += 32) {  // tail: K is a multiple of 8, so a lane's 8-chunk is all in or all out
      const bool kok = k0 + kq * 8 < K;
      const u32x4_t a = kok ? ld16_stream(aw + (size_t)(k0 / 32) * ws) : zero;
#pragma unroll
      for (int j = 0; j < NTT; ++j) acc[j] = mfma16x16x32(a, (kok && bok[j]) ? ld16(bsrc[j] + k0) : zero, acc[j]);
    }
  }
}

// The first layer with gate and up in separate waves: block (hb, g) owns 32 hidden rows of group g,
// waves 2r (gate) and 2r + 1 (up) stream the 16 rows h0 = 32 hb + 16 r of one matrix each, and the up
// wave hands its fp32 sums to the gate wave through LDS for SiLU(g) * u. One weight stream per wave
// (as in the down kernel) at about two thirds of the registers of the two-stream kernel above, so
// more waves fit on a SIMD, and half the bytes per wave. The sums are the same, bit for bit.
template <int NTT, int LAYOUT>
__global__ void __launch_bounds__(256)
ffn_gate_up_stream_pair(const FfnGroups p) {
  __shared__ f32x4_t up_sum[2][NTT][64];
  const GroupView v = group_view(p, blockIdx.y, 16 * NTT);
  if (v.n <= 0) return;
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int is_up = wave & 1, rg = wave >> 1;
  const int h0 = blockIdx.x * 32 + rg * 16;
  const bool active = h0 < v.Hg;  // every wave stays to the barriers below
  const int d = p.d;
  const int ar = lane & 15, kq = lane >> 4;
  const void* wmat = is_up ? v.wu : v.wg;
  int ws = 0;
  const uint16_t* aw = nullptr;
  const int8_t* qw = nullptr;
  if (active) {
    if (byte_codes(LAYOUT)) qw = q8_base(wmat, h0, d, lane);
    else aw = frag_base<LAYOUT>(wmat, h0, v.Hg, d, lane, &ws);
  }
  const uint16_t* xb = (const uint16_t*)p.x;
  const int h = h0 + kq * 4;  // lane's four rows
  f32x4_t sc = {1.f, 1.f, 1.f, 1.f};
  if (byte_codes(LAYOUT) && active && h < v.Hg) sc = *(const f32x4_t*)((is_up ? v.su : v.sg) + h);

  for (int tt = 0; tt < v.n; tt += 16 * NTT) {
    const uint16_t* bx[NTT];
    bool bok[NTT];
#pragma unroll
    for (int j = 0; j < NTT; ++j) {
      const int rr = tt + j * 16 + ar;
      bok[j] = rr < v.n;
      const long long src = bok[j] ? source_row(p, v, v.r0 + rr) : 0;
      bx[j] = xb + (size_t)src * d + kq * 8;
    }
    f32x4_t acc[NTT];
#pragma unroll
    for (int j = 0; j < NTT; ++j) acc[j] = f32x4_t{0, 0, 0, 0};
    if (active) stream_rows<NTT, LAYOUT>(aw, qw, ws, bx, bok, d, kq, acc);
    if (byte_codes(LAYOUT)) {
#pragma unroll
      for (int j = 0; j < NTT; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[j][e] *= sc[e];
    }
    if (is_up) {
#pragma unroll
      for (int j = 0; j < NTT; ++j) up_sum[rg][j][lane] = acc[j];
    }
    __syncthreads();
    if (!is_up && active) {
#pragma unroll
      for (int j = 0; j < NTT; ++j) {
        const int rr = tt + j * 16 + ar;
        if (rr < v.n && h < v.Hg) {
          const f32x4_t g = acc[j], u = up_sum[rg][j][lane];
          const uint32_t lo = pack_bf16x2(silu(g[0]) * u[0], silu(g[1]) * u[1]);
          const uint32_t hi = pack_bf16x2(silu(g[2]) * u[2], silu(g[3]) * u[3]);
          *(u32x2_t*)(v.hid + (size_t)(v.r0 + rr) * v.Hg + h) = u32x2_t{lo, hi};
        }
      }
    }
    __syncthreads();  // the next token tile rewrites up_sum
  }
}

template <int NTT, int LAYOUT>
__global__ void __launch_bounds__(256)
ffn_down_stream(const FfnGroups p) {
  const GroupView v = group_view(p, blockIdx.y, 16 * NTT);
  if (v.n <= 0) return;
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int d = p.d;
  const int i0 = blockIdx.x * kRowsPerBlock + wave * 16;
  if (i0 >= d) return;
  const int K = v.Hg;
  const int ar = lane & 15, kq = lane >> 4;
  int ws = 0;
  const uint16_t* aw = nullptr;
  const int8_t* qw = nullptr;
  if (byte_codes(LAYOUT))
    qw = q8_base(v.wd, i0, K, lane);
  else
    aw = frag_base<LAYOUT>(v.wd, i0, d, K, lane, &ws);

  for (int tt = 0; tt < v.n; tt += 16 * NTT) {
    const uint16_t* bh[NTT];
    bool bok[NTT];
#pragma unroll
    for (int j = 0; j < NTT; ++j) {
      const int rr = tt + j * 16 + ar;
      bok[j] = rr < v.n;
      bh[j] = v.hid + (size_t)(v.r0 + (bok[j] ? rr : 0)) * K + kq * 8;
    }
    f32x4_t acc[NTT];
#pragma unroll
    for (int j = 0; j < NTT; ++j) acc[j] = f32x4_t{0, 0, 0, 0};
    const u32x4_t zero = {0, 0, 0, 0};
    int k0 = 0;
    if (byte_codes(LAYOUT)) {
      for (; k0 + 32 * kUnroll <= K; k0 += 32 * kUnroll) {
        u32x4_t r[kUnroll / 2], b[kUnroll][NTT];
#pragma unroll
        for (int s2 = 0; s2 < kUnroll / 2; ++s2) r[s2] = ld16_stream(qw + (size_t)(k0 / 64 + s2) * 1024);
#pragma unroll
        for (int s = 0; s < kUnroll; ++s)
#pragma unroll
          for (int j = 0; j < NTT; ++j) b[s][j] = bok[j] ? ld16(bh[j] + k0 + 32 * s) : zero;
#pragma unroll
        for (int s2 = 0; s2 < kUnroll / 2; ++s2) {
          const u32x4_t a0 = codes_to_bf16x8<LAYOUT>(r[s2][0], r[s2][1]), a1 = codes_to_bf16x8<LAYOUT>(r[s2][2], r[s2][3]);
#pragma unroll
          for (int j = 0; j < NTT; ++j) {
            acc[j] = mfma16x16x32(a0, b[2 * s2][j], acc[j]);
            acc[j] = mfma16x16x32(a1, b[2 * s2 + 1][j], acc[j]);
          }
        }
      }
      for (; k0 < K; k0 += 64) {  // K (the hidden size) is a multiple of 64
        const u32x4_t r = ld16_stream(qw + (size_t)(k0 / 64) * 1024);
        const u32x4_t a0 = codes_to_bf16x8<LAYOUT>(r[0], r[1]), a1 = codes_to_bf16x8<LAYOUT>(r[2], r[3]);
#pragma unroll
        for (int j = 0; j < NTT; ++j) {
          acc[j] = mfma16x16x32(a0, bok[j] ? ld16(bh[j] + k0) : zero, acc[j]);
          acc[j] = mfma16x16x32(a1, bok[j] ? ld16(bh[j] + k0 + 32) : zero, acc[j]);
        }
      }
    } else {
      for (; k0 + 32 * kUnroll <= K; k0 += 32 * kUnroll) {
        u32x4_t a[kUnroll], b[kUnroll][NTT];
#pragma unroll
        for (int s = 0; s < kUnroll; ++s) a[s] = ld16_stream(aw + (size_t)(k0 / 32 + s) * ws);
#pragma unroll
        for (int s = 0; s < kUnroll; ++s)
#pragma unroll
          for (int j = 0; j < NTT; ++j) b[s][j] = NTT == 1 || bok[j] ? ld16(bh[j] + k0 + 32 * s) : zero;
#pragma unroll
        for (int s = 0; s < kUnroll; ++s)
#pragma unroll
          for (int j = 0; j < NTT; ++j) acc[j] = mfma16x16x32(a[s], bok[j] ? b[s][j] : zero, acc[j]);
      }
      for (; k0 < K; k0 += 32) {
        const bool kok = k0 + kq * 8 < K;
        const u32x4_t a = kok ? ld16_stream(aw + (size_t)(k0 / 32) * ws) : zero;
#pragma unroll
        for (int j = 0; j < NTT; ++j) {
          const u32x4_t b = (kok && bok[j]) ? ld16(bh[j] + k0) : zero;
          acc[j] = mfma16x16x32(a, b, acc[j]);
        }
      }
    }
    const int i = i0 + kq * 4;
    f32x4_t sc = {1.f, 1.f, 1.f, 1.f};
    if (byte_codes(LAYOUT) && i < d) sc = *(const f32x4_t*)(v.sd + i);
#pragma unroll
    for (int j = 0; j < NTT; ++j) {
      const int rr = tt + j * 16 + ar;
      if (rr < v.n && i < d) {
        f32x4_t y = acc[j];
        if (byte_codes(LAYOUT)) {
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] *= sc[e];
        }
        uint32_t lo = pack_bf16x2(y[0], y[1]);
        uint32_t hi = pack_bf16x2(y[2], y[3]);
        *(u32x2_t*)(v.y + (size_t)(v.r0 + rr) * d + i) = u32x2_t{lo, hi};
      }
    }
  }
}

// The first layer of one-byte weights for batches of more than 16 tokens: each wave streams 32 gate
// and 32 up rows (two 16-row fragments of each) against one set of x fragments, for the reason
// given at ffn_down_stream_wide. Block = 4 waves x 32 hidden rows. Same sums, in the same order, as
// ffn_gate_up_stream<1, LAYOUT>.
template <int LAYOUT>
__global__ void __launch_bounds__(256)
ffn_gate_up_stream_wide(const FfnGroups p) {
  static_assert(byte_codes(LAYOUT), "one-byte weights only");
  constexpr int kU = 8;  // k-steps per block of loads (kU / 2 loads per fragment stream)
  const GroupView v = group_view(p, blockIdx.y, 16);
  if (v.n <= 0) return;
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int h0 = blockIdx.x * 128 + wave * 32;   // hidden rows h0 .. h0 + 31
  if (h0 >= v.Hg) return;                        // Hg is a multiple of 64: both halves or none
  const int d = p.d;
  const int ar = lane & 15, kq = lane >> 4;
  const int8_t* qg[2] = {q8_base(v.wg, h0, d, lane), q8_base(v.wg, h0 + 16, d, lane)};
  const int8_t* qu[2] = {q8_base(v.wu, h0, d, lane), q8_base(v.wu, h0 + 16, d, lane)};
  const uint16_t* xb = (const uint16_t*)p.x;
  const u32x4_t zero = {0, 0, 0, 0};
  for (int tt = 0; tt < v.n; tt += 16) {
    const int rr = tt + ar;
    const bool bok = rr < v.n;
    const long long src = bok ? source_row(p, v, v.r0 + rr) : 0;
    const uint16_t* bx = xb + (size_t)src * d + kq * 8;
    f32x4_t accg[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}}, accu[2] = {{0, 0, 0, 0}, {0, 0, 0, 0}};
    int k0 = 0;
    for (; k0 + 32 * kU <= d; k0 += 32 * kU) {
      u32x4_t rg[2][kU / 2], ru[2][kU / 2], b[kU];
#pragma unroll
      for (int s2 = 0; s2 < kU / 2; ++s2)
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          rg[f][s2] = ld16_stream(qg[f] + (size_t)(k0 / 64 + s2) * 1024);
          ru[f][s2] = ld16_stream(qu[f] + (size_t)(k0 / 64 + s2) * 1024);
        }
#pragma unroll
      for (int s = 0; s < kU; ++s) b[s] = bok ? ld16(bx + k0 + 32 * s) : zero;
#pragma unroll
      for (int s2 = 0; s2 < kU / 2; ++s2)
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          const u32x4_t g0 = codes_to_bf16x8<LAYOUT>(rg[f][s2][0], rg[f][s2][1]), g1 = codes_to_bf16x8<LAYOUT>(rg[f][s2][2], rg[f][s2][3]);
          const u32x4_t u0 = codes_to_bf16x8<LAYOUT>(ru[f][s2][0], ru[f][s2][1]), u1 = codes_to_bf16x8<LAYOUT>(ru[f][s2][2], ru[f][s2][3]);
          accg[f] = mfma16x16x32(g0, b[2 * s2], accg[f]);
          accu[f] = mfma16x16x32(u0, b[2 * s2], accu[f]);
          accg[f] = mfma16x16x32(g1, b[2 * s2 + 1], accg[f]);
          accu[f] = mfma16x16x32(u1, b[2 * s2 + 1], accu[f]);
        }
    }
    for (; k0 < d; k0 += 64) {  // one-byte layouts: d is a multiple of 64
      const u32x4_t b0 = bok ? ld16(bx + k0) : zero, b1 = bok ? ld16(bx + k0 + 32) : zero;
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const u32x4_t r_g = ld16_stream(qg[f] + (size_t)(k0 / 64) * 1024);
        const u32x4_t r_u = ld16_stream(qu[f] + (size_t)(k0 / 64) * 1024);
        accg[f] = mfma16x16x32(codes_to_bf16x8<LAYOUT>(r_g[0], r_g[1]), b0, accg[f]);
        accu[f] = mfma16x16x32(codes_to_bf16x8<LAYOUT>(r_u[0], r_u[1]), b0, accu[f]);
        accg[f] = mfma16x16x32(codes_to_bf16x8<LAYOUT>(r_g[2], r_g[3]), b1, accg[f]);
        accu[f] = mfma16x16x32(codes_to_bf16x8<LAYOUT>(r_u[2], r_u[3]), b1, accu[f]);
      }
    }
    if (!bok) continue;
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int h = h0 + 16 * f + kq * 4;
      const f32x4_t sg = *(const f32x4_t*)(v.sg + h), su = *(const f32x4_t*)(v.su + h);
      f32x4_t g = accg[f], u = accu[f];
#pragma unroll
      for (int e = 0; e < 4; ++e) { g[e] *= sg[e]; u[e] *= su[e]; }
      const uint32_t lo = pack_bf16x2(silu(g[0]) * u[0], silu(g[1]) * u[1]);
      const uint32_t hi = pack_bf16x2(silu(g[2]) * u[2], silu(g[3]) * u[3]);
      *(u32x2_t*)(v.hid + (size_t)(v.r0 + rr) * v.Hg + h) = u32x2_t{lo, hi};
    }
  }
}

// The down projection of one-byte weights for batches of more than 16 tokens: each wave streams 32
// weight rows (two 16-row fragments) against one set of hidden-row fragments. With one byte per
// weight the hidden rows (bf16, read from L2 by every wave of the expert) outweigh the codes, and a
// 16-row wave read twice as many of them per weight byte. Block = 4 waves x 32 rows. Same sums, in
// the same order, as ffn_down_stream<1, LAYOUT>.
template <int LAYOUT>
__global__ void __launch_bounds__(256)
ffn_down_stream_wide(const FfnGroups p) {
  static_assert(byte_codes(LAYOUT), "one-byte weights only");
  const GroupView v = group_view(p, blockIdx.y, 16);
  if (v.n <= 0) return;
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int d = p.d;
  const int i0 = blockIdx.x * 128 + wave * 32;   // rows i0 .. i0 + 15 and i0 + 16 .. i0 + 31
  if (i0 >= d) return;
  const bool two = i0 + 16 < d;                  // d is a multiple of 64: both groups or only the first
  const int K = v.Hg;
  const int ar = lane & 15, kq = lane >> 4;
  const int8_t* qw0 = q8_base(v.wd, i0, K, lane);
  const int8_t* qw1 = two ? q8_base(v.wd, i0 + 16, K, lane) : qw0;
  const u32x4_t zero = {0, 0, 0, 0};
  for (int tt = 0; tt < v.n; tt += 16) {
    const int rr = tt + ar;
    const bool bok = rr < v.n;
    const uint16_t* bh = v.hid + (size_t)(v.r0 + (bok ? rr : 0)) * K + kq * 8;
    f32x4_t acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
    int k0 = 0;
    for (; k0 + 32 * kUnroll <= K; k0 += 32 * kUnroll) {
      u32x4_t r0[kUnroll / 2], r1[kUnroll / 2], b[kUnroll];
#pragma unroll
      for (int s2 = 0; s2 < kUnroll / 2; ++s2) {
        r0[s2] = ld16_stream(qw0 + (size_t)(k0 / 64 + s2) * 1024);
        r1[s2] = ld16_stream(qw1 + (size_t)(k0 / 64 + s2) * 1024);
      }
#pragma unroll
      for (int s = 0; s < kUnroll; ++s) b[s] = bok ? ld16(bh + k0 + 32 * s) : zero;
#pragma unroll
      for (int s2 = 0; s2 < kUnroll / 2; ++s2) {
        const u32x4_t a0 = codes_to_bf16x8<LAYOUT>(r0[s2][0], r0[s2][1]), a1 = codes_to_bf16x8<LAYOUT>(r0[s2][2], r0[s2][3]);
        const u32x4_t c0 = codes_to_bf16x8<LAYOUT>(r1[s2][0], r1[s2][1]), c1 = codes_to_bf16x8<LAYOUT>(r1[s2][2], r1[s2][3]);
        acc0 = mfma16x16x32(a0, b[2 * s2], acc0);
        acc0 = mfma16x16x32(a1, b[2 * s2 + 1], acc0);
        acc1 = mfma16x16x32(c0, b[2 * s2], acc1);
        acc1 = mfma16x16x32(c1, b[2 * s2 + 1], acc1);
      }
    }
    for (; k0 < K; k0 += 64) {  // K (the hidden size) is a multiple of 64
      const u32x4_t r0 = ld16_stream(qw0 + (size_t)(k0 / 64) * 1024);
      const u32x4_t r1 = ld16_stream(qw1 + (size_t)(k0 / 64) * 1024);
      const u32x4_t b0 = bok ? ld16(bh + k0) : zero, b1 = bok ? ld16(bh + k0 + 32) : zero;
      acc0 = mfma16x16x32(codes_to_bf16x8<LAYOUT>(r0[0], r0[1]), b0, acc0);
      acc0 = mfma16x16x32(codes_to_bf16x8<LAYOUT>(r0[2], r0[3]), b1, acc0);
      acc1 = mfma16x16x32(codes_to_bf16x8<LAYOUT>(r1[0], r1[1]), b0, acc1);
      acc1 = mfma16x16x32(codes_to_bf16x8<LAYOUT>(r1[2], r1[3]), b1, acc1);
    }
    if (!bok) continue;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      if (g == 1 && !two) break;
      const int i = i0 + 16 * g + kq * 4;
      const f32x4_t sc = *(const f32x4_t*)(v.sd + i);
      const f32x4_t a = g ? acc1 : acc0;
      const uint32_t lo = pack_bf16x2(a[0] * sc[0], a[1] * sc[1]);
      const uint32_t hi = pack_bf16x2(a[2] * sc[2], a[3] * sc[3]);
      *(u32x2_t*)(v.y + (size_t)(v.r0 + rr) * d + i) = u32x2_t{lo, hi};
    }
  }
}

// ------------------------------------------------------------------------------ fp32 (VALU)
// Plain per-element form for float32 layers: one thread per (row, output column).

__device__ __forceinline__ int find_group(const int32_t* offsets, int E, long long r) {
  int lo = 0, hi = E;  // last g with offsets[g] <= r
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (offsets[mid] <= r) lo = mid; else hi = mid;
  }
  return lo;
}

__global__ void __launch_bounds__(256)
ffn_gate_up_f32(const FfnGroups p) {
  const long long r = blockIdx.x;  // row in routed space [0, rows), then shared [rows, rows+T)
  const bool shared = r >= p.rows;
  const int Hg = shared ? p.Hs : p.H;
  const int h = blockIdx.y * 256 + threadIdx.x;
  if (h >= Hg) return;
  const int d = p.d;
  const float *wg, *wu, *xr;
  float* hid;
  if (shared) {
    const long long t = r - p.rows;
    wg = (const float*)p.ws_gate; wu = (const float*)p.ws_up;
    xr = (const float*)p.x + (size_t)t * d;
    hid = (float*)p.hid + (size_t)p.rows * p.H + (size_t)t * Hg;
  } else {
    if (r >= p.offsets[p.E]) return;
    const int g = find_group(p.offsets, p.E, r);  // any g in [0, E) keeps the weight reads in bounds
    wg = (const float*)p.w_gate + (size_t)g * p.H * d;
    wu = (const float*)p.w_up + (size_t)g * p.H * d;
    long long s = p.perm_src ? (long long)(p.perm_src[r] / p.k) : r;
    const long long lim = p.perm_src ? (long long)p.T : p.rows;
    s = s < 0 ? 0 : (s >= lim ? lim - 1 : s);
    xr = (const float*)p.x + (size_t)s * d;
    hid = (float*)p.hid + (size_t)r * Hg;
  }
  const float* gr = wg + (size_t)h * d;
  const float* ur = wu + (size_t)h * d;
  float gs = 0.f, us = 0.f;
  for (int i = 0; i < d; ++i) { gs += xr[i] * gr[i]; us += xr[i] * ur[i]; }
  hid[h] = silu(gs) * us;
}

__global__ void __launch_bounds__(256)
ffn_down_f32(const FfnGroups p) {
  const long long r = blockIdx.x;
  const bool shared = r >= p.rows;
  const int d = p.d;
  const int i = blockIdx.y * 256 + threadIdx.x;
  if (i >= d) return;
  const int Hg = shared ? p.Hs : p.H;
  const float *wd, *hr;
  float* yr;
  if (shared) {
    const long long t = r - p.rows;
    wd = (const float*)p.ws_down;
    hr = (const float*)p.hid + (size_t)p.rows * p.H + (size_t)t * Hg;
    yr = (float*)p.y + (size_t)p.rows * d + (size_t)t * d;
  } else {
    if (r >= p.offsets[p.E]) return;
    const int g = find_group(p.offsets, p.E, r);
    wd = (const float*)p.w_down + (size_t)g * p.H * d;
    hr = (const float*)p.hid + (size_t)r * Hg;
    yr = (float*)p.y + (size_t)r * d;
  }
  const float* w = wd + (size_t)i * Hg;
  float s = 0.f;
  for (int h = 0; h < Hg; ++h) s += hr[h] * w[h];
  yr[i] = s;
}

// --------------------------------------------------------------------------------- launchers
namespace {
int stream_ntt(const FfnGroups& g) { return !byte_codes(g.layout) && g.T > 16 ? 2 : 1; }
// Gate and up in separate waves (ffn_gate_up_stream_pair) for batches of at most 16 tokens, where an
// expert holds one or two rows and the weight stream is all there is: decode T = 8 gate/up 0.540 ->
// 0.527 ms (bf16), 0.295 -> 0.284 ms (FP8), 0.293 -> 0.287 ms (INT8). With more rows per expert both
// waves of a pair read the same activation rows, and it loses (T = 256: bf16 2.33 -> 2.46 ms, INT8
// 1.27 -> 1.58 ms).
bool pair_waves(const FfnGroups& g) { return g.T <= 16; }
bool wide_down(const FfnGroups& g) { return byte_codes(g.layout) && g.T > 16; }
// routed groups + one group per 16 NTT-row chunk of the shared expert
int groups_of(const FfnGroups& g) {
  const int c = 16 * stream_ntt(g);
  return g.E + (g.Hs > 0 ? (g.T + c - 1) / c : 0);
}
int hmax(const FfnGroups& g) { return g.H > g.Hs ? g.H : g.Hs; }
long long all_rows(const FfnGroups& g) { return g.rows + (g.Hs > 0 ? g.T : 0); }
}  // namespace

FfnPath ffn_path(const FfnGroups& g) {
  if (g.dtype == kF32) return kPathF32;
  return g.mean_rows_per_group >= kGemmMinRowsPerExpert ? kPathGemm : kPathStream;
}

hipError_t launch_ffn_gate_up_stream(const FfnGroups& g, hipStream_t stream) {
  dim3 grid((hmax(g) + kRowsPerBlock - 1) / kRowsPerBlock, groups_of(g));
  const bool two = stream_ntt(g) == 2;
  if (pair_waves(g)) {  // gate and up in separate waves, 32 hidden rows per block
    const dim3 pgrid((hmax(g) + 31) / 32, groups_of(g));
    if (g.layout == kInt8Frag)
      hipLaunchKernelGGL((ffn_gate_up_stream_pair<1, kInt8Frag>), pgrid, dim3(256), 0, stream, g);
    else if (g.layout == kFp8Frag)
      hipLaunchKernelGGL((ffn_gate_up_stream_pair<1, kFp8Frag>), pgrid, dim3(256), 0, stream, g);
    else if (g.layout == kFrag16)
      hipLaunchKernelGGL((ffn_gate_up_stream_pair<1, kFrag16>), pgrid, dim3(256), 0, stream, g);
    else
      hipLaunchKernelGGL((ffn_gate_up_stream_pair<1, kRowMajor>), pgrid, dim3(256), 0, stream, g);
    return hipGetLastError();
  }
  if (wide_down(g)) {  // one-byte weights above 16 tokens: 32 gate and 32 up rows per wave
    const dim3 wgrid((hmax(g) + 127) / 128, groups_of(g));
    if (g.layout == kInt8Frag)
      hipLaunchKernelGGL((ffn_gate_up_stream_wide<kInt8Frag>), wgrid, dim3(256), 0, stream, g);
    else
      hipLaunchKernelGGL((ffn_gate_up_stream_wide<kFp8Frag>), wgrid, dim3(256), 0, stream, g);
    return hipGetLastError();
  }
  if (g.layout == kInt8Frag)
    hipLaunchKernelGGL((ffn_gate_up_stream<1, kInt8Frag>), grid, dim3(256), 0, stream, g);
  else if (g.layout == kFp8Frag)
    hipLaunchKernelGGL((ffn_gate_up_stream<1, kFp8Frag>), grid, dim3(256), 0, stream, g);
  else if (g.layout == kFrag16 && two)
    hipLaunchKernelGGL((ffn_gate_up_stream<2, kFrag16>), grid, dim3(256), 0, stream, g);
  else if (g.layout == kFrag16)
    hipLaunchKernelGGL((ffn_gate_up_stream<1, kFrag16>), grid, dim3(256), 0, stream, g);
  else if (two)
    hipLaunchKernelGGL((ffn_gate_up_stream<2, kRowMajor>), grid, dim3(256), 0, stream, g);
  else
    hipLaunchKernelGGL((ffn_gate_up_stream<1, kRowMajor>), grid, dim3(256), 0, stream, g);
  return hipGetLastError();
}

hipError_t launch_ffn_down_stream(const FfnGroups& g, hipStream_t stream) {
  dim3 grid((g.d + kRowsPerBlock - 1) / kRowsPerBlock, groups_of(g));
  const bool two = stream_ntt(g) == 2;
  if (wide_down(g)) {  // one-byte weights above 16 tokens: 32 weight rows per wave
    const dim3 wgrid((g.d + 127) / 128, groups_of(g));
    if (g.layout == kInt8Frag)
      hipLaunchKernelGGL((ffn_down_stream_wide<kInt8Frag>), wgrid, dim3(256), 0, stream, g);
    else
      hipLaunchKernelGGL((ffn_down_stream_wide<kFp8Frag>), wgrid, dim3(256), 0, stream, g);
    return hipGetLastError();
  }
  if (g.layout == kInt8Frag)
    hipLaunchKernelGGL((ffn_down_stream<1, kInt8Frag>), grid, dim3(256), 0, stream, g);
  else if (g.layout == kFp8Frag)
    hipLaunchKernelGGL((ffn_down_stream<1, kFp8Frag>), grid, dim3(256), 0, stream, g);
  else if (g.layout == kFrag16 && two)
    hipLaunchKernelGGL((ffn_down_stream<2, kFrag16>), grid, dim3(256), 0, stream, g);
  else if (g.layout == kFrag16)
    hipLaunchKernelGGL((ffn_down_stream<1, kFrag16>), grid, dim3(256), 0, stream, g);
  else if (two)
    hipLaunchKernelGGL((ffn_down_stream<2, kRowMajor>), grid, dim3(256), 0, stream, g);
  else
    hipLaunchKernelGGL((ffn_down_stream<1, kRowMajor>), grid, dim3(256), 0, stream, g);
  return hipGetLastError();
}

hipError_t launch_ffn_gate_up_f32(const FfnGroups& g, hipStream_t stream) {
  dim3 grid((unsigned)all_rows(g), (hmax(g) + 255) / 256);
  hipLaunchKernelGGL(ffn_gate_up_f32, grid, dim3(256), 0, stream, g);
  return hipGetLastError();
}

hipError_t launch_ffn_down_f32(const FfnGroups& g, hipStream_t stream) {
  dim3 grid((unsigned)all_rows(g), (g.d + 255) / 256);
  hipLaunchKernelGGL(ffn_down_f32, grid, dim3(256), 0, stream, g);
  return hipGetLastError();
}

const char* ffn_schedule_kernel_name(const FfnGroups& g) {
  return ffn_path(g) == kPathGemm ? "gemm_schedule_kernel" : "";
}
const char* ffn_gate_up_kernel_name(const FfnGroups& g) {
  switch (ffn_path(g)) {
    case kPathF32: return "ffn_gate_up_f32";
    case kPathStream:
      if (pair_waves(g)) {
        if (g.layout == kInt8Frag) return "ffn_gate_up_stream_pair<1, 2>";
        if (g.layout == kFp8Frag) return "ffn_gate_up_stream_pair<1, 3>";
        return g.layout == kFrag16 ? "ffn_gate_up_stream_pair<1, 1>" : "ffn_gate_up_stream_pair<1, 0>";
      }
      if (g.layout == kInt8Frag) return wide_down(g) ? "ffn_gate_up_stream_wide<2>" : "ffn_gate_up_stream<1, 2>";
      if (g.layout == kFp8Frag) return wide_down(g) ? "ffn_gate_up_stream_wide<3>" : "ffn_gate_up_stream<1, 3>";
      if (stream_ntt(g) == 2) return g.layout == kFrag16 ? "ffn_gate_up_stream<2, 1>" : "ffn_gate_up_stream<2, 0>";
      return g.layout == kFrag16 ? "ffn_gate_up_stream<1, 1>" : "ffn_gate_up_stream<1, 0>";
    default:
      if (g.gelu) return g.layout == kFrag16 ? "grouped_gemm_kernel<3, 1>" : "grouped_gemm_kernel<3, 0>";
      if (g.layout == kInt8Frag) return "grouped_gemm_kernel<0, 2>";
      if (g.layout == kFp8Frag) return "grouped_gemm_kernel<0, 3>";
      return g.layout == kFrag16 ? "grouped_gemm_kernel<0, 1>" : "grouped_gemm_kernel<0, 0>";
  }
}
const char* ffn_down_kernel_name(const FfnGroups& g) {
  switch (ffn_path(g)) {
    case kPathF32: return "ffn_down_f32";
    case kPathStream:
      if (g.layout == kInt8Frag) return wide_down(g) ? "ffn_down_stream_wide<2>" : "ffn_down_stream<1, 2>";
      if (g.layout == kFp8Frag) return wide_down(g) ? "ffn_down_stream_wide<3>" : "ffn_down_stream<1, 3>";
      if (stream_ntt(g) == 2) return g.layout == kFrag16 ? "ffn_down_stream<2, 1>" : "ffn_down_stream<2, 0>";
      return g.layout == kFrag16 ? "ffn_down_stream<1, 1>" : "ffn_down_stream<1, 0>";
    default:
      if (g.gelu) return g.layout == kFrag16 ? "grouped_gemm_kernel<4, 1>" : "grouped_gemm_kernel<4, 0>";
      if (g.layout == kInt8Frag) return "grouped_gemm_kernel<1, 2>";
      if (g.layout == kFp8Frag) return "grouped_gemm_kernel<1, 3>";
      return g.layout == kFrag16 ? "grouped_gemm_kernel<1, 1>" : "grouped_gemm_kernel<1, 0>";
  }
}

}  // namespace moe
