// A2: counts and prefix sums of the handle on gfx950.
//
// LL ("NVSHMEM and DeepEP", low-latency section: fixed slots per local
// expert and source rank): a (token, k) entry takes slot = number of earlier
// entries of the same source with the same expert (tokens ascending, then k).
// HT (same page, high-throughput section; "NCCL EP paper notes", tensor
// layouts: 2-D output with per-expert counts, deterministic order):
//   stage 1: one row per (token, destination node n) at the same-position
//            rank d = n*G + s%G, rows grouped by d, (source, token) inside d;
//   stage 2: one row per (token, k), grouped by expert, (source, token)
//            inside an expert.
//
// Positions are a stable counting sort split in two:
//   * here, per tile of 64 tokens of one source (one wave), the tile's
//     per-expert and per-node counts (LDS counters), then -- in the last
//     workgroup to finish, found with a device-scope counter, so no kernel
//     waits on another -- exclusive prefix sums over the tiles, rewritten in
//     place, and the per-expert / per-rank totals and offsets;
//   * in the dispatch kernel, each token's rank inside its tile (a ballot
//     over the <= 63 earlier tokens of the tile), added to the tile prefix.
// Neither half uses atomics on positions, so every map is bit-reproducible.
#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kTile = kLayoutTile;

template <int KMAX>
struct Entries {
  int e[KMAX];
  bool ok[KMAX];
  int bad = 0;

  // Loads K indices and flags the valid ones: in range and not a repeat of
  // an earlier entry of the same token.
  __device__ void load(const int32_t* row, int K, int E, bool active) {
#pragma unroll
    for (int k = 0; k < KMAX; ++k) e[k] = (active && k < K) ? row[k] : -1;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      const bool in_range = e[k] >= 0 && e[k] < E;
      bool dup = false;
#pragma unroll
      for (int j = 0; j < k; ++j) dup |= e[j] == e[k];
      ok[k] = active && k < K && in_range && !dup;
      if (active && k < K && !in_range) bad |= EP_DEVERR_BAD_INDEX;
      else if (active && k < K && dup) bad |= EP_DEVERR_DUP_INDEX;
    }
  }
};

// Exclusive scan of v[0..count) in place by the whole block.
__device__ void block_exclusive_scan(int* v, int count, int* scratch) {
  const int B = blockDim.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int per = (count + B - 1) / B;
  const int x0 = tid * per;
  int sum = 0;
  for (int q = 0; q < per; ++q)
    if (x0 + q < count) sum += v[x0 + q];
  int incl = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) scratch[w] = incl;
  __syncthreads();
  int base = 0;
  for (int q = 0; q < w; ++q) base += scratch[q];
  int run = base + incl - sum;
  for (int q = 0; q < per; ++q) {
    if (x0 + q < count) {
      const int val = v[x0 + q];
      v[x0 + q] = run;
      run += val;
    }
  }
  __syncthreads();
}

// The tiles of destination key (n, g) for stage 1: tiles of the sources at
// position g (s = g, g+G, ...), in order.
__device__ __forceinline__ int rail_tile(int pos, int g, int G, int tps) {
  return (g + (pos / tps) * G) * tps + pos % tps;
}

// Sum / exclusive-prefix rewrite of values at idx(pos), pos in [p0, p1),
// 16 independent loads at a time so that the chain costs one round trip per
// 16 tiles instead of one per tile.
constexpr int kBatch = 16;

template <class Idx>
__device__ __forceinline__ int chunk_sum(const int32_t* base, int p0, int p1, Idx idx) {
  int sum = 0;
  for (int pos = p0; pos < p1; pos += kBatch) {
    int v[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) v[q] = pos + q < p1 ? base[idx(pos + q)] : 0;
#pragma unroll
    for (int q = 0; q < kBatch; ++q) sum += v[q];
  }
  return sum;
}

template <class Idx>
__device__ __forceinline__ int chunk_prefix(int32_t* base, int p0, int p1, int run, Idx idx) {
  for (int pos = p0; pos < p1; pos += kBatch) {
    int v[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) v[q] = pos + q < p1 ? base[idx(pos + q)] : 0;
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      if (pos + q < p1) base[idx(pos + q)] = run;
      run += v[q];
    }
  }
  return run;
}

template <int KMAX>
__global__ __launch_bounds__(1024) void layout_count_kernel(LayoutArgs a) {
  extern __shared__ int smem[];
  __shared__ int s_last;
  const int B = blockDim.x, nw = B >> 6;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int E = a.E, N = a.N, K = a.K;
  int* cnt_e = smem;              // [nw][E]
  int* cnt_n = smem + nw * E;     // [nw][N]

  const int j = blockIdx.x * nw + w;
  const bool tile_ok = j < a.n_tiles;
  const int s = tile_ok ? j / a.tps : 0;
  const int t = (tile_ok ? j - s * a.tps : 0) * kTile + lane;
  const bool active = tile_ok && t < a.T;
  const int64_t i = static_cast<int64_t>(s) * a.T + t;

  for (int x = tid; x < nw * (E + N); x += B) smem[x] = 0;
  Entries<KMAX> en;
  en.load(a.topk + (active ? i : 0) * K, K, E, active);
  __syncthreads();
  if (active) {
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
      if (k < K) a.topk_copy[i * K + k] = en.e[k];
    if (en.bad) atomicOr(a.err, en.bad);
    uint64_t nodes = 0;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      if (!en.ok[k]) continue;
      atomicAdd(&cnt_e[w * E + en.e[k]], 1);
      nodes |= 1ull << (en.e[k] / a.P);
    }
    if (a.ht)
      for (int n = 0; n < N; ++n)
        if ((nodes >> n) & 1) atomicAdd(&cnt_n[w * N + n], 1);
  }
  __syncthreads();
  if (tile_ok) {
    for (int e = lane; e < E; e += 64) a.hist_e[static_cast<int64_t>(j) * E + e] = cnt_e[w * E + e];
    if (a.ht)
      for (int n = lane; n < N; n += 64) a.hist_n[static_cast<int64_t>(j) * N + n] = cnt_n[w * N + n];
  }

  // The last workgroup to finish turns the histograms into prefix sums.
  __threadfence();
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(a.done, 1) == static_cast<int>(gridDim.x) - 1;
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  const int n_tiles = a.n_tiles;
  if (!a.ht) {
    // LL: per (expert, source), prefix over the source's own tiles.
    for (int x = tid; x < E * a.S; x += B) {
      const int e = x % E, src = x / E;
      const int tps = a.tps;
      a.ll_count[static_cast<int64_t>(e) * a.S + src] =
          chunk_prefix(a.hist_e, 0, tps, 0, [=](int tt) { return static_cast<int64_t>(src * tps + tt) * E + e; });
    }
  } else {
    // Experts: the sequence is every tile in order, cut into C chunks.
    const int C = B / E > 0 ? B / E : 1;
    const int CL = (n_tiles + C - 1) / C;
    int* part = smem;                 // [C][E]
    int* tot = smem + C * E;          // [E]
    int* scratch = tot + E;           // [nw]
    for (int x = tid; x < C * E; x += B) {
      const int e = x % E, c = x / E;
      const int j0 = c * CL, j1 = min(n_tiles, j0 + CL);
      part[c * E + e] = chunk_sum(a.hist_e, j0, j1, [=](int jj) { return static_cast<int64_t>(jj) * E + e; });
    }
    __syncthreads();
    for (int e = tid; e < E; e += B) {
      int run = 0;
      for (int c = 0; c < C; ++c) {
        const int v = part[c * E + e];
        part[c * E + e] = run;
        run += v;
      }
      tot[e] = run;
      a.c2[e] = run;
    }
    __syncthreads();
    block_exclusive_scan(tot, E, scratch);
    for (int e = tid; e < E; e += B) a.off2[e] = tot[e];
    for (int x = tid; x < C * E; x += B) {
      const int e = x % E, c = x / E;
      const int j0 = c * CL, j1 = min(n_tiles, j0 + CL);
      chunk_prefix(a.hist_e, j0, j1, tot[e] + part[c * E + e],
                   [=](int jj) { return static_cast<int64_t>(jj) * E + e; });
    }
    __syncthreads();

    // Stage-1 keys d = n*G + g: the tiles of the sources at position g.
    const int G = a.G, R = N * G;
    const int CR = B / R > 0 ? B / R : 1;
    int* partr = smem;                // [CR][R]
    int* totr = smem + CR * R;        // [R]
    int* scratch2 = totr + R;
    for (int x = tid; x < CR * R; x += B) {
      const int d = x % R, c = x / R;
      const int n = d / G, g = d - n * G;
      const int nsrc = g < a.S ? (a.S - g + G - 1) / G : 0;
      const int len = nsrc * a.tps;
      const int cl = (len + CR - 1) / CR;
      const int p0 = c * cl, p1 = min(len, p0 + cl);
      const int tps = a.tps;
      partr[c * R + d] = chunk_sum(a.hist_n, p0, p1, [=](int pos) {
        return static_cast<int64_t>(rail_tile(pos, g, G, tps)) * N + n;
      });
    }
    __syncthreads();
    for (int d = tid; d < R; d += B) {
      int run = 0;
      for (int c = 0; c < CR; ++c) {
        const int v = partr[c * R + d];
        partr[c * R + d] = run;
        run += v;
      }
      totr[d] = run;
      a.c1[d] = run;
    }
    __syncthreads();
    block_exclusive_scan(totr, R, scratch2);
    for (int d = tid; d < R; d += B) a.off1[d] = totr[d];
    for (int x = tid; x < CR * R; x += B) {
      const int d = x % R, c = x / R;
      const int n = d / G, g = d - n * G;
      const int nsrc = g < a.S ? (a.S - g + G - 1) / G : 0;
      const int len = nsrc * a.tps;
      const int cl = (len + CR - 1) / CR;
      const int p0 = c * cl, p1 = min(len, p0 + cl);
      const int tps = a.tps;
      chunk_prefix(a.hist_n, p0, p1, totr[d] + partr[c * R + d], [=](int pos) {
        return static_cast<int64_t>(rail_tile(pos, g, G, tps)) * N + n;
      });
    }
  }
  if (tid == 0) *a.done = 0;   // ready for the next handle
}

__global__ void fill_i32_kernel(int32_t* p, int64_t count, int32_t value) {
  for (int64_t x = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; x < count;
       x += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[x] = value;
}

int layout_block_threads(int E, int N) {
  // 16 waves unless the per-wave LDS counters would exceed 64 KiB.
  int nw = 16;
  while (nw > 1 && static_cast<int64_t>(nw) * (E + N) * 4 > 65536) nw >>= 1;
  return nw * 64;
}

size_t layout_lds_bytes(int E, int N, int G, int threads) {
  const int nw = threads / 64;
  const int R = N * G;
  const int C = threads / E > 0 ? threads / E : 1;
  const int CR = threads / R > 0 ? threads / R : 1;
  size_t ints = static_cast<size_t>(nw) * (E + N);
  const size_t scan_e = static_cast<size_t>(C) * E + E + nw;
  const size_t scan_r = static_cast<size_t>(CR) * R + R + nw;
  if (scan_e > ints) ints = scan_e;
  if (scan_r > ints) ints = scan_r;
  return ints * 4;
}

}  // namespace

hipError_t launch_fill_i32(int32_t* p, int64_t count, int32_t value, hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  int64_t blocks = (count + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  fill_i32_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream>>>(p, count, value);
  return hipGetLastError();
}

hipError_t launch_layout(const LayoutArgs& a, hipStream_t stream) {
  if (a.n == 0) return hipSuccess;
  const int threads = layout_block_threads(a.E, a.N);
  const int nw = threads / 64;
  const dim3 grid(static_cast<unsigned>((a.n_tiles + nw - 1) / nw)), block(threads);
  const size_t lds = layout_lds_bytes(a.E, a.N, a.G, threads);
  if (a.K <= 8) layout_count_kernel<8><<<grid, block, lds, stream>>>(a);
  else layout_count_kernel<32><<<grid, block, lds, stream>>>(a);
  return hipGetLastError();
}

}  // namespace ep
