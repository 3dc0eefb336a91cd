// Seeded synthetic-input generator shared by the test oracle and the GPU path.
//
// It holds none of the MoE layer's arithmetic: it only turns (seed, stream,
// element index) into a normally distributed number and rounds it to the
// storage type. Large weight sets are filled on the device; any slice can be
// regenerated on the host with identical bits, so the CPU oracle can rebuild
// exactly the expert weights it needs without copying anything back from the
// GPU.
//
// Bit-identity between host and device rests on three facts:
//   * Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
//     easy as 1, 2, 3", SC'11) is pure 32-bit integer arithmetic;
//   * the Box-Muller transform below uses only IEEE-754 double +, -, *, / and
//     sqrt (all correctly rounded) with fixed evaluation order; the file is
//     compiled with -ffp-contract=off so no fused multiply-add changes a
//     rounding; log, sin and cos are hand-written series, not libm/ocml;
//   * rounding to float and then to bfloat16 (round to nearest, ties to even)
//     is exact integer work.
//
// Element 2c and 2c+1 of a stream come from Philox counter c:
//   counter = (c.lo, c.hi, stream.lo, stream.hi), key = (seed.lo, seed.hi)
//   u1 = (top 53 bits of (r0:r1) + 0.5) * 2^-53    in (0, 1)
//   u2 = (top 53 bits of (r2:r3)) * 2^-53          in [0, 1)
//   z0 = sqrt(-2 ln u1) cos(2 pi u2), z1 = sqrt(-2 ln u1) sin(2 pi u2)
//   value = (float)(z * std)     (then bf16 RNE for bf16 outputs)

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>
#include <thread>
#include <vector>

#define SYN_HD __host__ __device__ static inline

SYN_HD void philox_mulhilo(uint32_t a, uint32_t b, uint32_t* hi, uint32_t* lo) {
  uint64_t p = (uint64_t)a * (uint64_t)b;
  *hi = (uint32_t)(p >> 32);
  *lo = (uint32_t)p;
}

SYN_HD void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
  for (int r = 0; r < 10; ++r) {
    uint32_t hi0, lo0, hi1, lo1;
    philox_mulhilo(M0, c[0], &hi0, &lo0);
    philox_mulhilo(M1, c[2], &hi1, &lo1);
    uint32_t n0 = hi1 ^ c[1] ^ k0;
    uint32_t n1 = lo1;
    uint32_t n2 = hi0 ^ c[3] ^ k1;
    uint32_t n3 = lo0;
    c[0] = n0; c[1] = n1; c[2] = n2; c[3] = n3;
    k0 += W0; k1 += W1;
  }
}

SYN_HD uint64_t syn_d2u(double x) { union { double d; uint64_t u; } v; v.d = x; return v.u; }
SYN_HD double syn_u2d(uint64_t x) { union { double d; uint64_t u; } v; v.u = x; return v.d; }

// Natural log for x in (0, 1]: x = m * 2^e with m in [sqrt(1/2), sqrt(2)),
// ln m = 2 atanh(s), s = (m-1)/(m+1), |s| < 0.1716; the series to s^23 is far
// below double rounding. x is never subnormal here (x >= 2^-54).
SYN_HD double syn_log(double x) {
  uint64_t b = syn_d2u(x);
  int e = (int)((b >> 52) & 0x7FF) - 1023;
  double m = syn_u2d((b & 0x000FFFFFFFFFFFFFull) | 0x3FF0000000000000ull);
  if (m > 1.4142135623730951) { m = m * 0.5; e = e + 1; }
  double s = (m - 1.0) / (m + 1.0);
  double t = s * s;
  double p = 1.0 / 23.0;
  p = p * t + 1.0 / 21.0;
  p = p * t + 1.0 / 19.0;
  p = p * t + 1.0 / 17.0;
  p = p * t + 1.0 / 15.0;
  p = p * t + 1.0 / 13.0;
  p = p * t + 1.0 / 11.0;
  p = p * t + 1.0 / 9.0;
  p = p * t + 1.0 / 7.0;
  p = p * t + 1.0 / 5.0;
  p = p * t + 1.0 / 3.0;
  p = p * t + 1.0;
  return (double)e * 0.69314718055994530942 + 2.0 * s * p;
}

// sin and cos of theta in [0, pi/2] by Taylor series in Horner form.
SYN_HD void syn_sincos_quarter(double th, double* s, double* c) {
  double t = th * th;
  double ps = 1.0 - t / (22.0 * 23.0);
  ps = 1.0 - t / (20.0 * 21.0) * ps;
  ps = 1.0 - t / (18.0 * 19.0) * ps;
  ps = 1.0 - t / (16.0 * 17.0) * ps;
  ps = 1.0 - t / (14.0 * 15.0) * ps;
  ps = 1.0 - t / (12.0 * 13.0) * ps;
  ps = 1.0 - t / (10.0 * 11.0) * ps;
  ps = 1.0 - t / (8.0 * 9.0) * ps;
  ps = 1.0 - t / (6.0 * 7.0) * ps;
  ps = 1.0 - t / (4.0 * 5.0) * ps;
  ps = 1.0 - t / (2.0 * 3.0) * ps;
  *s = th * ps;
  double pc = 1.0 - t / (23.0 * 24.0);
  pc = 1.0 - t / (21.0 * 22.0) * pc;
  pc = 1.0 - t / (19.0 * 20.0) * pc;
  pc = 1.0 - t / (17.0 * 18.0) * pc;
  pc = 1.0 - t / (15.0 * 16.0) * pc;
  pc = 1.0 - t / (13.0 * 14.0) * pc;
  pc = 1.0 - t / (11.0 * 12.0) * pc;
  pc = 1.0 - t / (9.0 * 10.0) * pc;
  pc = 1.0 - t / (7.0 * 8.0) * pc;
  pc = 1.0 - t / (5.0 * 6.0) * pc;
  pc = 1.0 - t / (3.0 * 4.0) * pc;
  pc = 1.0 - t / (1.0 * 2.0) * pc;
  *c = pc;
}

// Two standard normals from Philox counter `ctr` of (seed, stream).
SYN_HD void syn_normal_pair(uint64_t seed, uint64_t stream, uint64_t ctr, double* z0, double* z1) {
  uint32_t c[4] = {(uint32_t)ctr, (uint32_t)(ctr >> 32), (uint32_t)stream, (uint32_t)(stream >> 32)};
  philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
  uint64_t a = (((uint64_t)c[0] << 32) | c[1]) >> 11;
  uint64_t b = (((uint64_t)c[2] << 32) | c[3]) >> 11;
  const double two53 = 1.0 / 9007199254740992.0;
  double u1 = ((double)a + 0.5) * two53;
  double u2 = (double)b * two53;
  double r = sqrt(-2.0 * syn_log(u1));
  double v = u2 * 4.0;  // exact
  int q = (int)v;
  double f = v - (double)q;  // exact
  double sn, cs;
  syn_sincos_quarter(f * 1.5707963267948966, &sn, &cs);
  double cq, sq;
  switch (q & 3) {
    case 0: cq = cs; sq = sn; break;
    case 1: cq = -sn; sq = cs; break;
    case 2: cq = -cs; sq = -sn; break;
    default: cq = sn; sq = -cs; break;
  }
  *z0 = r * cq;
  *z1 = r * sq;
}

SYN_HD float syn_f64_to_f32(double x) { return (float)x; }

SYN_HD uint16_t syn_f32_to_bf16(float f) {
  union { float f; uint32_t u; } v; v.f = f;
  uint32_t u = v.u;
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// value of element `i` of (seed, stream) scaled by `stdev`, as float.
SYN_HD float syn_value(uint64_t seed, uint64_t stream, uint64_t i, double stdev) {
  double z0, z1;
  syn_normal_pair(seed, stream, i >> 1, &z0, &z1);
  return syn_f64_to_f32(((i & 1) ? z1 : z0) * stdev);
}

// ---------------------------------------------------------------- device ---
// A "block-stream" tensor is `nblk` consecutive blocks of `blk` elements; block
// j draws from stream `stream0 + j * stream_step`, elements from `first`
// onwards. One launch fills all experts of a [E, rows, cols] weight tensor.

__global__ void __launch_bounds__(256)
syn_fill_kernel(void* out, int is_bf16, uint64_t nblk, uint64_t blk, uint64_t first,
                uint64_t seed, uint64_t stream0, uint64_t stream_step, double stdev) {
  uint64_t pairs_per_blk = (blk + 1) / 2;
  uint64_t total = nblk * pairs_per_blk;
  for (uint64_t p = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; p < total;
       p += (uint64_t)gridDim.x * blockDim.x) {
    uint64_t j = p / pairs_per_blk;
    uint64_t e = (p - j * pairs_per_blk) * 2;  // element within the block
    uint64_t i = first + e;
    double z0, z1;
    // (first) may be odd; handle element parity explicitly.
    if ((i & 1) == 0) {
      syn_normal_pair(seed, stream0 + j * stream_step, i >> 1, &z0, &z1);
    } else {
      double a0, a1, b0, b1;
      syn_normal_pair(seed, stream0 + j * stream_step, i >> 1, &a0, &a1);
      syn_normal_pair(seed, stream0 + j * stream_step, (i + 1) >> 1, &b0, &b1);
      z0 = a1; z1 = b0;
    }
    float v0 = syn_f64_to_f32(z0 * stdev), v1 = syn_f64_to_f32(z1 * stdev);
    uint64_t o = j * blk + e;
    if (is_bf16) {
      uint16_t* q = (uint16_t*)out;
      q[o] = syn_f32_to_bf16(v0);
      if (e + 1 < blk) q[o + 1] = syn_f32_to_bf16(v1);
    } else {
      float* q = (float*)out;
      q[o] = v0;
      if (e + 1 < blk) q[o + 1] = v1;
    }
  }
}

// ------------------------------------------------------------------ host ---

static void syn_fill_host_range(void* out, int is_bf16, uint64_t blk, uint64_t first, uint64_t seed,
                                uint64_t stream0, uint64_t stream_step, double stdev,
                                uint64_t lo, uint64_t hi) {
  uint64_t o = lo;
  while (o < hi) {
    uint64_t j = o / blk, e = o - j * blk;
    uint64_t i = first + e;
    uint64_t strm = stream0 + j * stream_step;
    double z0, z1;
    syn_normal_pair(seed, strm, i >> 1, &z0, &z1);
    float v = syn_f64_to_f32(((i & 1) ? z1 : z0) * stdev);
    if (is_bf16) ((uint16_t*)out)[o] = syn_f32_to_bf16(v);
    else ((float*)out)[o] = v;
    ++o;
    // the partner element of the same Philox counter, when it is in range
    if ((i & 1) == 0 && o < hi && e + 1 < blk) {
      float w = syn_f64_to_f32(z1 * stdev);
      if (is_bf16) ((uint16_t*)out)[o] = syn_f32_to_bf16(w);
      else ((float*)out)[o] = w;
      ++o;
    }
  }
}

extern "C" {

// One raw Philox4x32-10 block: ctr[4] is replaced by the output.
void syn_philox_raw(uint32_t* ctr, uint32_t k0, uint32_t k1) { philox4x32_10(ctr, k0, k1); }

// Fill host memory: nblk blocks of blk elements (see above). Returns 0.
int syn_fill_host(void* out, int is_bf16, uint64_t nblk, uint64_t blk, uint64_t first, uint64_t seed,
                  uint64_t stream0, uint64_t stream_step, double stdev, int nthreads) {
  uint64_t n = nblk * blk;
  if (n == 0) return 0;
  if (nthreads < 1) nthreads = 1;
  if ((uint64_t)nthreads > n / 4096 + 1) nthreads = (int)(n / 4096 + 1);
  std::vector<std::thread> th;
  uint64_t chunk = (n + nthreads - 1) / nthreads;
  for (int t = 0; t < nthreads; ++t) {
    uint64_t lo = (uint64_t)t * chunk, hi = lo + chunk < n ? lo + chunk : n;
    if (lo >= hi) break;
    th.emplace_back(syn_fill_host_range, out, is_bf16, blk, first, seed, stream0, stream_step, stdev, lo, hi);
  }
  for (auto& x : th) x.join();
  return 0;
}

// Fill device memory `out` on `stream` (a hipStream_t). Returns a hipError_t.
int syn_fill_device(void* out, int is_bf16, uint64_t nblk, uint64_t blk, uint64_t first, uint64_t seed,
                    uint64_t stream0, uint64_t stream_step, double stdev, void* hip_stream) {
  uint64_t pairs = nblk * ((blk + 1) / 2);
  if (pairs == 0) return 0;
  uint64_t blocks = (pairs + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(syn_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)hip_stream, out,
                     is_bf16, nblk, blk, first, seed, stream0, stream_step, stdev);
  return (int)hipGetLastError();
}

}  // extern "C"
