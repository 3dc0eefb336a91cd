// Dispatch: per-expert counts, exclusive offsets and a deterministic expert-order permutation.
//
// MoE-kernels page (blog.llmgo.top), section 4.3: flatten the selected expert ids, bring equal ids
// together, count tokens per expert and turn the counts into offsets for the grouped GEMM.
// Data-movement page, section 4: route records sorted by expert id.
//
// The flat slots t*k + j are cut into tiles. (1) count: one wave per tile builds an LDS histogram
// of its tile (integer LDS atomics: order-free). (2) scan: one block turns the [tile, expert]
// histograms into per-(tile, expert) starting rows: offsets[e] + sum of earlier tiles' counts.
// (3) scatter: one wave per tile walks its slots in increasing order, 64 at a time; lanes that
// hold the same expert find each other with ballots over the expert-id bits, and a lane's rank
// among them is the number of such lanes below it. The result is the unique stable order
// (expert, flat slot), with no dependence on scheduling.
#include "dispatch.h"
#include "moe_device.h"

namespace moe {

// Slots per permutation tile: a power of two of at least 64 (the scatter walks a tile 64 slots at a
// time) giving up to 64 tiles, so the count and scatter kernels have that many blocks while the
// one-block scan still has short columns (a decode batch of 256 x 8 slots: 32 tiles of 64 instead
// of 2 of 1024, scatter 15 -> 6 us); never more than 1024 tiles.
int permute_tile_size(long long rows) {
  long long tile = 64;
  while (tile * 64 < rows) tile *= 2;
  while ((rows + tile - 1) / tile > 1024) tile *= 2;
  return (int)tile;
}

size_t permute_scratch_bytes(long long rows, int E) {
  long long tiles = (rows + permute_tile_size(rows) - 1) / permute_tile_size(rows);
  if (tiles < 1) tiles = 1;
  return (size_t)tiles * (size_t)E * sizeof(int32_t);
}

__global__ void __launch_bounds__(64)
permute_count_kernel(const int32_t* __restrict__ ids, long long rows, int E, int tile, int32_t* __restrict__ tile_counts) {
  __shared__ int32_t hist[kMaxExperts];
  const int lane = threadIdx.x;
  for (int e = lane; e < E; e += 64) hist[e] = 0;
  __syncthreads();
  const long long lo = (long long)blockIdx.x * tile;
  const long long hi = lo + tile < rows ? lo + tile : rows;
  for (long long p = lo + lane; p < hi; p += 64) {
    int e = ids[p];
    if ((unsigned)e < (unsigned)E) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  int32_t* out = tile_counts + (size_t)blockIdx.x * E;
  for (int e = lane; e < E; e += 64) out[e] = hist[e];
}

// One block of 1024 threads (one expert each): column scan over tiles, then a block-wide exclusive
// scan over experts of the totals. The tile counts are read 16 tiles at a time before any of them
// is written back, so a column costs n_tiles / 16 memory round trips, not n_tiles.
__global__ void __launch_bounds__(1024)
permute_scan_kernel(int32_t* __restrict__ tile_counts, int n_tiles, int E, int32_t* __restrict__ counts,
                    int32_t* __restrict__ offsets) {
  __shared__ int32_t wave_tot[16];
  const int e = threadIdx.x;
  const int lane = e & 63, wave = e >> 6;
  constexpr int kChunk = 16;
  int32_t total = 0;
  if (e < E) {
    for (int b0 = 0; b0 < n_tiles; b0 += kChunk) {
      int32_t c[kChunk];
#pragma unroll
      for (int j = 0; j < kChunk; ++j) c[j] = b0 + j < n_tiles ? tile_counts[(size_t)(b0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < kChunk; ++j) {
        if (b0 + j < n_tiles) tile_counts[(size_t)(b0 + j) * E + e] = total;  // exclusive within the expert
        total += c[j];
      }
    }
  }
  // inclusive scan of `total` across the 1024 threads: within waves, then across waves
  int32_t incl = total;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int32_t o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int32_t before = 0;
  for (int w = 0; w < wave; ++w) before += wave_tot[w];
  const int32_t excl = before + incl - total;
  if (e < E) {
    if (counts) counts[e] = total;
    offsets[e] = excl;
    if (e == E - 1) offsets[E] = excl + total;
    for (int b0 = 0; b0 < n_tiles; b0 += kChunk) {
      int32_t c[kChunk];
#pragma unroll
      for (int j = 0; j < kChunk; ++j) c[j] = b0 + j < n_tiles ? tile_counts[(size_t)(b0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < kChunk; ++j)
        if (b0 + j < n_tiles) tile_counts[(size_t)(b0 + j) * E + e] = c[j] + excl;
    }
  }
}

__global__ void __launch_bounds__(64)
permute_scatter_kernel(const int32_t* __restrict__ ids, long long rows, int E, int tile,
                       const int32_t* __restrict__ tile_base, int32_t* __restrict__ perm_src,
                       int32_t* __restrict__ inv_perm) {
  __shared__ int32_t cur[kMaxExperts];
  const int lane = threadIdx.x;
  const int32_t* base = tile_base + (size_t)blockIdx.x * E;
  for (int e = lane; e < E; e += 64) cur[e] = base[e];
  __syncthreads();
  int bits = 0;
  while ((1 << bits) < E) ++bits;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const long long lo = (long long)blockIdx.x * tile;
  const long long hi = lo + tile < rows ? lo + tile : rows;
  for (long long c = lo; c < hi; c += 64) {
    const long long p = c + lane;
    int e = (p < hi) ? ids[p] : -1;
    const bool valid = (unsigned)e < (unsigned)E;
    uint64_t same = __ballot(valid);
    for (int b = 0; b < bits; ++b) {
      const bool bit = valid && ((e >> b) & 1);
      const uint64_t m = __ballot(bit);
      same &= bit ? m : ~m;
    }
    const int rank = __popcll(same & below);
    const int n = __popcll(same);
    int32_t pos = 0;
    if (valid) pos = cur[e] + rank;
    __syncthreads();  // every lane has read cur[] before any leader updates it
    if (valid && rank == 0) cur[e] += n;
    __syncthreads();
    if (valid) {
      perm_src[pos] = (int32_t)p;
      inv_perm[p] = pos;
    }
  }
}

// Load statistics of one routing (overview article, section 4.1 layer code): every expert's
// share of the T*k assignments and the balance penalty coef * sum_e (load_e - 1/E)^2. One block,
// one expert per thread, the sum in a fixed order (wave butterflies, then the wave totals in order).
__global__ void __launch_bounds__(1024)
load_stats_kernel(const int32_t* __restrict__ counts, int E, long long slots, float coef, float* __restrict__ load,
                  float* __restrict__ aux) {
  __shared__ float wave_tot[16];
  const int e = threadIdx.x, lane = e & 63, wave = e >> 6;
  float sq = 0.f;
  if (e < E) {
    const float l = (float)counts[e] / (float)slots;
    if (load) load[e] = l;
    const float dl = l - 1.0f / (float)E;
    sq = dl * dl;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sq += __shfl_xor(sq, off, 64);
  if (lane == 0) wave_tot[wave] = sq;
  __syncthreads();
  if (e == 0 && aux) {
    float t = 0.f;
    for (int w = 0; w < 16; ++w) t += wave_tot[w];
    aux[0] = coef * t;
  }
}

hipError_t launch_load_stats(const int32_t* counts, int E, long long slots, float coef, float* load, float* aux,
                             hipStream_t stream) {
  hipLaunchKernelGGL(load_stats_kernel, dim3(1), dim3(1024), 0, stream, counts, E, slots, coef, load, aux);
  return hipGetLastError();
}

hipError_t launch_permute_count(const int32_t* ids, long long rows, int E, int tile, int32_t* tile_counts,
                                hipStream_t stream) {
  int n_tiles = (int)((rows + tile - 1) / tile);
  hipLaunchKernelGGL(permute_count_kernel, dim3(n_tiles), dim3(64), 0, stream, ids, rows, E, tile, tile_counts);
  return hipGetLastError();
}

hipError_t launch_permute_scan(int32_t* tile_counts, long long rows, int E, int tile, int32_t* counts,
                               int32_t* offsets, hipStream_t stream) {
  int n_tiles = (int)((rows + tile - 1) / tile);
  hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(1024), 0, stream, tile_counts, n_tiles, E, counts, offsets);
  return hipGetLastError();
}

hipError_t launch_permute_scatter(const int32_t* ids, long long rows, int E, int tile, const int32_t* tile_counts,
                                  int32_t* perm_src, int32_t* inv_perm, hipStream_t stream) {
  int n_tiles = (int)((rows + tile - 1) / tile);
  hipLaunchKernelGGL(permute_scatter_kernel, dim3(n_tiles), dim3(64), 0, stream, ids, rows, E, tile, tile_counts,
                     perm_src, inv_perm);
  return hipGetLastError();
}

}  // namespace moe
