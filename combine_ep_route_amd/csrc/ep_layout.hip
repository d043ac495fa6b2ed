// A2: counts, prefix sums and slot/row maps (the handle) on gfx950.
//
// LL ("NVSHMEM and DeepEP", low-latency section: fixed slots per local
// expert and source rank): slot(i,k) = number of earlier entries of the same
// source that chose the same expert, tokens ascending then k.
// HT (same page, high-throughput section; "NCCL EP paper notes", tensor
// layouts: 2-D output with per-expert counts, deterministic order):
//   stage 1: one row per (token, destination node n) at the same-position
//            rank d = n*G + s%G, rows grouped by d, (source, token) inside d;
//   stage 2: one row per (token, k), grouped by expert, (source, token)
//            inside an expert.
//
// Every map is a stable counting sort, computed without atomics on the
// position path so that it is bit-reproducible:
//   * a tile is 256 tokens of one source, one token per thread, one wave64
//     per 64 tokens;
//   * each wave ORs its lane bit into a 64-bit LDS mask per key (expert or
//     node); a token's position inside its wave is the popcount of the key's
//     mask below its lane -- that is its rank among the wave's tokens with
//     that key, in token order, since a valid key occurs at most once per
//     token;
//   * per-wave popcounts give the wave offsets inside the tile; per-tile
//     histograms (first kernel) give the tile offsets (second kernel sums the
//     histograms of the earlier tiles it needs, which are few and L2-hot);
//   * HT offsets of experts / ranks are block-wide exclusive scans of the
//     totals.
// LL with at most one tile per source skips the histogram kernel entirely.
#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kTile = kLayoutTile;
constexpr int kWaves = kTile / 64;

// Entries of one token: loads K indices and flags the valid ones (in range
// and not a repeat of an earlier entry of the same token).
template <int KMAX>
struct Entries {
  int e[KMAX];
  bool ok[KMAX];
  int bad = 0;

  __device__ void load(const int32_t* row, int K, int E, bool active) {
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      e[k] = (active && k < K) ? row[k] : -1;
      ok[k] = false;
    }
    if (!active) return;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      const bool in_range = e[k] >= 0 && e[k] < E;
      bool dup = false;
#pragma unroll
      for (int j = 0; j < k; ++j) dup |= e[j] == e[k];
      ok[k] = k < K && in_range && !dup;
      if (k < K && !in_range) bad |= EP_DEVERR_BAD_INDEX;
      else if (k < K && dup) bad |= EP_DEVERR_DUP_INDEX;
    }
  }
};

struct TileInfo {
  int j, s, tt;
  int64_t i;       // token index of this thread
  bool active;
};

__device__ __forceinline__ TileInfo tile_info(const LayoutArgs& a) {
  TileInfo ti;
  ti.j = blockIdx.x;
  ti.s = ti.j / a.tps;
  ti.tt = ti.j - ti.s * a.tps;
  const int t = ti.tt * kTile + static_cast<int>(threadIdx.x);
  ti.active = t < a.T;
  ti.i = static_cast<int64_t>(ti.s) * a.T + t;
  return ti;
}

// Fill the per-wave key masks of this tile.  Returns the token's node mask.
template <int KMAX>
__device__ uint64_t build_masks(const LayoutArgs& a, const TileInfo& ti,
                                Entries<KMAX>& en, uint64_t (*m_e)[kMaxExperts],
                                uint64_t (*m_n)[kMaxNodes]) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int x = threadIdx.x; x < kWaves * kMaxExperts; x += kTile) (&m_e[0][0])[x] = 0;
  for (int x = threadIdx.x; x < kWaves * kMaxNodes; x += kTile) (&m_n[0][0])[x] = 0;
  en.load(a.topk + (ti.active ? ti.i : 0) * a.K, a.K, a.E, ti.active);
  __syncthreads();
  const uint64_t bit = 1ull << lane;
  uint64_t nodes = 0;
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    if (!en.ok[k]) continue;
    atomicOr(reinterpret_cast<unsigned long long*>(&m_e[w][en.e[k]]), bit);
    nodes |= 1ull << (en.e[k] / a.P);
  }
  if (a.ht) {
    for (int n = 0; n < a.N; ++n)
      if ((nodes >> n) & 1) atomicOr(reinterpret_cast<unsigned long long*>(&m_n[w][n]), bit);
  }
  __syncthreads();
  return nodes;
}

// Block-wide exclusive scan of v[0..count) in place (count <= 1024); sum of
// all values returned.  256 threads, 4 consecutive values per thread.
__device__ int block_exclusive_scan(int* v, int count, int* s_wave) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int loc[4];
  int sum = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int x = tid * 4 + q;
    loc[q] = x < count ? v[x] : 0;
    sum += loc[q];
  }
  // inclusive wave scan of the per-thread sums
  int incl = sum;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) s_wave[w] = incl;
  __syncthreads();
  int wave_base = 0, total = 0;
  for (int q = 0; q < kWaves; ++q) {
    if (q < w) wave_base += s_wave[q];
    total += s_wave[q];
  }
  int run = wave_base + incl - sum;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int x = tid * 4 + q;
    if (x < count) v[x] = run;
    run += loc[q];
  }
  __syncthreads();
  return total;
}

template <int KMAX>
__global__ __launch_bounds__(kTile) void layout_hist_kernel(LayoutArgs a) {
  __shared__ uint64_t m_e[kWaves][kMaxExperts];
  __shared__ uint64_t m_n[kWaves][kMaxNodes];
  const TileInfo ti = tile_info(a);
  Entries<KMAX> en;
  build_masks<KMAX>(a, ti, en, m_e, m_n);
  for (int e = threadIdx.x; e < a.E; e += kTile) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) c += __popcll(m_e[w][e]);
    a.hist_e[static_cast<int64_t>(ti.j) * a.E + e] = c;
  }
  if (a.ht) {
    for (int n = threadIdx.x; n < a.N; n += kTile) {
      int c = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) c += __popcll(m_n[w][n]);
      a.hist_n[static_cast<int64_t>(ti.j) * a.N + n] = c;
    }
  }
}

template <int KMAX>
__global__ __launch_bounds__(kTile) void layout_assign_kernel(LayoutArgs a) {
  __shared__ uint64_t m_e[kWaves][kMaxExperts];
  __shared__ uint64_t m_n[kWaves][kMaxNodes];
  __shared__ int base_e[kWaves][kMaxExperts];
  __shared__ int base_n[kWaves][kMaxNodes];
  __shared__ int s_tot[kMaxExperts];   // expert totals -> offsets (HT)
  __shared__ int s_rank[kMaxRanks];    // stage-1 rank totals -> offsets (HT)
  __shared__ int s_wave[kWaves];

  const TileInfo ti = tile_info(a);
  Entries<KMAX> en;
  const uint64_t my_nodes = build_masks<KMAX>(a, ti, en, m_e, m_n);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int G = a.G, R = a.N * a.G;
  const int rail = ti.s % G;

  // Tile offsets from the histograms of earlier tiles.
  for (int e = tid; e < a.E; e += kTile) {
    int before = 0, total = 0;
    if (a.ht) {
      for (int j = 0; j < a.n_tiles; ++j) {
        const int h = a.hist_e[static_cast<int64_t>(j) * a.E + e];
        total += h;
        if (j < ti.j) before += h;
      }
      s_tot[e] = total;
    } else {
      for (int tt = 0; tt < ti.tt; ++tt)
        before += a.hist_e[static_cast<int64_t>(ti.s * a.tps + tt) * a.E + e];
    }
    base_e[0][e] = before;
  }
  if (a.ht) {
    // Stage-1 totals per destination rank d = n*G + g: tiles whose source
    // sits at position g, node n.
    for (int d = tid; d < R; d += kTile) {
      const int n = d / G, g = d - n * G;
      int total = 0;
      for (int j = 0; j < a.n_tiles; ++j)
        if ((j / a.tps) % G == g) total += a.hist_n[static_cast<int64_t>(j) * a.N + n];
      s_rank[d] = total;
    }
    for (int n = tid; n < a.N; n += kTile) {
      int before = 0;
      for (int j = 0; j < ti.j; ++j)
        if ((j / a.tps) % G == rail) before += a.hist_n[static_cast<int64_t>(j) * a.N + n];
      base_n[0][n] = before;
    }
  }
  __syncthreads();
  if (a.ht) {
    if (ti.j == 0) {
      for (int e = tid; e < a.E; e += kTile) a.c2[e] = s_tot[e];
      for (int d = tid; d < R; d += kTile) a.c1[d] = s_rank[d];
    }
    block_exclusive_scan(s_tot, a.E, s_wave);
    block_exclusive_scan(s_rank, R, s_wave);
    if (ti.j == 0) {
      for (int e = tid; e < a.E; e += kTile) a.off2[e] = s_tot[e];
      for (int d = tid; d < R; d += kTile) a.off1[d] = s_rank[d];
    }
  }

  // Wave offsets inside the tile.
  for (int e = tid; e < a.E; e += kTile) {
    int c = base_e[0][e] + (a.ht ? s_tot[e] : 0);
#pragma unroll
    for (int q = 0; q < kWaves; ++q) {
      base_e[q][e] = c;
      c += __popcll(m_e[q][e]);
    }
    if (!a.ht && ti.tt == a.tps - 1) a.ll_count[static_cast<int64_t>(e) * a.S + ti.s] = c;
  }
  if (a.ht) {
    for (int n = tid; n < a.N; n += kTile) {
      int c = base_n[0][n] + s_rank[n * G + rail];
#pragma unroll
      for (int q = 0; q < kWaves; ++q) {
        base_n[q][n] = c;
        c += __popcll(m_n[q][n]);
      }
    }
  }
  __syncthreads();

  if (!ti.active) return;
  if (en.bad) atomicOr(a.err, en.bad);
#pragma unroll
  for (int k = 0; k < KMAX; ++k)
    if (k < a.K) a.topk_copy[ti.i * a.K + k] = en.e[k];
  const uint64_t below = (1ull << lane) - 1;
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    if (k >= a.K) continue;
    int out = -1;
    if (en.ok[k]) {
      const int e = en.e[k];
      const int r = base_e[w][e] + __popcll(m_e[w][e] & below);
      out = a.ht ? r : (e * a.S + ti.s) * a.slots + r;
    }
    (a.ht ? a.row2 : a.slot_map)[ti.i * a.K + k] = out;
  }
  if (a.ht) {
    for (int n = 0; n < a.N; ++n) {
      int out = -1;
      if ((my_nodes >> n) & 1) out = base_n[w][n] + __popcll(m_n[w][n] & below);
      a.node_row[ti.i * a.N + n] = out;
    }
  }
}

__global__ void fill_i32_kernel(int32_t* p, int64_t count, int32_t value) {
  for (int64_t x = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; x < count;
       x += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[x] = value;
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
  const dim3 grid(static_cast<unsigned>(a.n_tiles)), block(kTile);
  const bool need_hist = a.ht || a.tps > 1;
  if (a.K <= 8) {
    if (need_hist) layout_hist_kernel<8><<<grid, block, 0, stream>>>(a);
    layout_assign_kernel<8><<<grid, block, 0, stream>>>(a);
  } else {
    if (need_hist) layout_hist_kernel<32><<<grid, block, 0, stream>>>(a);
    layout_assign_kernel<32><<<grid, block, 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace ep
