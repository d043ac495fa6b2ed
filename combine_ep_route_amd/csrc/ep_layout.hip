// A2: counts and prefix sums of the handle on gfx950 (with A1 fused in).
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
// Positions are a stable counting sort in three parts:
//   * tile_count_kernel: one workgroup per tile of kLayoutTile tokens.  It
//     routes the tile's tokens (when the handle is made from scores: 32
//     lanes per token, the fast routing path) or loads their topk rows,
//     builds a 32-bit LDS lane mask per key (stage-2 key and destination
//     node), and writes each entry's rank inside its tile (popcount of the
//     mask below the token's lane) and the tile's count per key;
//   * scan_keys_kernel (HT): one wave per key turns the key's sequence of
//     tile counts into exclusive prefix sums in place and writes the key's
//     total.  LL: layout_scan_ll_kernel, one thread per (expert, source),
//     since LL slots restart at 0 for every source;
//   * the dispatch kernel adds key offset + tile prefix + in-tile rank; in
//     HT each of its workgroups first scans the key totals into the key
//     offsets in LDS (a few hundred values, read while its tokens load), so
//     that no step of the scan waits for the other workgroups.
// No atomics decide a position, so every map is bit-reproducible.
#include "ep_route_dev.h"

namespace ep {
namespace {

using namespace route_dev;

constexpr int kTile = kLayoutTile;
constexpr int kTileThreads = 32 * kTile;   // 32 lanes per token while routing

// Sum, and exclusive-prefix rewrite, of the values at idx(pos), pos in
// [p0, p1), 16 independent loads at a time so that the chain costs one
// round trip per 16 tiles instead of one per tile.
constexpr int kBatch = 16;

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

template <bool ROUTE, int V, int LPN>
__global__ __launch_bounds__(kTileThreads) void tile_count_kernel(LayoutArgs a) {
  extern __shared__ uint32_t s_mask[];            // [E2 + N] lane masks of the tile's tokens
  __shared__ int s_e[kTile][kMaxTopK];            // the tile's entries
  __shared__ int s_key[kTile][kMaxTopK];          // stage-2 key of an entry that takes a row, else -1
  __shared__ float s_node[kTile][32];             // routing: node-score exchange
  const int tid = threadIdx.x;
  const int j = blockIdx.x;                       // tile
  const int s = j / a.tps, tt = j - s * a.tps;
  const int t0 = tt * kTile;
  const int ntok = min(kTile, a.T - t0);          // tokens in this tile
  const int E2 = a.E2, N = a.N, K = a.K, E = a.E;
  const int64_t i0 = static_cast<int64_t>(s) * a.T + t0;
  for (int x = tid; x < E2 + N; x += blockDim.x) s_mask[x] = 0;
  // e / L and e / P by shifts when they are powers of two
  auto div_l = [&](int e) { return a.l_shift >= 0 ? e >> a.l_shift : e / a.L; };
  auto div_p = [&](int e) { return a.p_shift >= 0 ? e >> a.p_shift : e / a.P; };
  // Routed entries are valid and distinct by construction: with one stage-2
  // key per entry (the expert), the lanes that hold them set the mask bits
  // directly (repeated node bits are harmless: the masks are ORs).
  bool direct = false;
  if constexpr (ROUTE) {
    const int slot = tid >> 5, hl = tid & 31;
    const bool active = slot < ntok;
    const int64_t i = i0 + slot;
    const int mine = route_token_fast<V, LPN>(a.scores + (active ? i : 0) * a.ld, active, hl, s_node[slot], N,
                                              a.M, a.J, K);
    const bool held = active && hl < K;
    if (held) {
      a.topk_out[i * K + hl] = mine;
      a.topk_copy[i * K + hl] = mine;
    }
    direct = !a.s2_rank;
    if (direct) {
      __syncthreads();   // the masks are zero
      if (held) {
        atomicOr(&s_mask[mine], 1u << slot);
        if (a.ht) atomicOr(&s_mask[E2 + div_p(mine)], 1u << slot);
      }
      __syncthreads();
      if (held) a.rank_e[i * K + hl] = __popc(s_mask[mine] & ((1u << slot) - 1u));
    } else if (hl < K) {
      s_e[slot][hl] = mine;
    }
  } else {
    for (int x = tid; x < ntok * K; x += blockDim.x) {
      const int slot = x / K, k = x - slot * K;
      const int e = a.topk[i0 * K + x];
      a.topk_copy[i0 * K + x] = e;
      s_e[slot][k] = e;
    }
  }
  if (!direct) {
    __syncthreads();
    // Entries: valid (in range, not a repeat), the stage-2 key (the expert,
    // or with the per-rank stage 2 its rank, carried only by the token's
    // first entry on it), and the first entry on each destination node.
    int bad = 0;
    for (int x = tid; x < ntok * K; x += blockDim.x) {
      const int slot = x / K, k = x - slot * K;
      const int e = s_e[slot][k];
      const bool in_range = e >= 0 && e < E;
      const int key = a.s2_rank ? div_l(e) : e;
      const int nd = div_p(e);
      bool dup = false, same_key = false, same_node = false;
      for (int q = 0; q < k; ++q) {
        const int eq = s_e[slot][q];
        const bool inq = eq >= 0 && eq < E;
        dup |= eq == e;
        same_key |= inq && (a.s2_rank ? div_l(eq) : eq) == key;
        same_node |= inq && div_p(eq) == nd;
      }
      const bool ok = in_range && !dup;
      if (!in_range) bad |= EP_DEVERR_BAD_INDEX;
      else if (dup) bad |= EP_DEVERR_DUP_INDEX;
      const bool first = ok && !same_key;
      if (first) atomicOr(&s_mask[key], 1u << slot);
      if (a.ht && ok && !same_node) atomicOr(&s_mask[E2 + nd], 1u << slot);
      s_key[slot][k] = first ? key : -1;
    }
    if (bad) atomicOr(a.err, bad);
    __syncthreads();
    // In-tile ranks: popcount of the key's mask below the token's lane.
    for (int x = tid; x < ntok * K; x += blockDim.x) {
      const int slot = x / K, k = x - slot * K;
      const int key = s_key[slot][k];
      a.rank_e[i0 * K + x] = key >= 0 ? __popc(s_mask[key] & ((1u << slot) - 1u)) : -1;
    }
  }
  if (a.ht) {
    for (int x = tid; x < ntok * N; x += blockDim.x) {
      const int slot = x / N, n = x - slot * N;
      const uint32_t m = s_mask[E2 + n];
      a.rank_n[i0 * N + x] = ((m >> slot) & 1u) ? __popc(m & ((1u << slot) - 1u)) : -1;
    }
  }
  // The tile's count per key.
  for (int x = tid; x < E2; x += blockDim.x) a.hist_e[static_cast<int64_t>(j) * E2 + x] = __popc(s_mask[x]);
  if (a.ht)
    for (int x = tid; x < N; x += blockDim.x) a.hist_n[static_cast<int64_t>(j) * N + x] = __popc(s_mask[E2 + x]);
}

// LL: the (expert, source) pairs are independent -- a source's slots for an
// expert start at 0 -- so one thread per pair, over as many workgroups as it
// takes: the prefix over the source's tiles, in place, and the pair's count.
// Consecutive threads take consecutive experts (coalesced tile counts).
__global__ __launch_bounds__(256) void layout_scan_ll_kernel(LayoutArgs a) {
  const int E = a.E2, S = a.S, tps = a.tps;
  const int64_t x = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (x >= static_cast<int64_t>(E) * S) return;
  const int e = static_cast<int>(x % E), src = static_cast<int>(x / E);
  a.ll_count[static_cast<int64_t>(e) * S + src] =
      chunk_prefix(a.hist_e, 0, tps, 0, [=](int tt) { return static_cast<int64_t>(src * tps + tt) * E + e; });
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  return v;
}

constexpr int kScanPerLane = 8;     // tile counts a lane holds per pass of a key's sequence
constexpr int kScanThreads = 256;   // four keys per workgroup

// HT: one wave per key.  Keys [0, E2) are the stage-2 keys, whose sequence
// is every tile in order; keys E2 + d (d = n*G + g, d < R) are the stage-1
// ranks, whose sequence is the tiles of the sources s = g, g+G, g+2G, ...
// in order, counter n of each.  A lane takes kScanPerLane consecutive
// elements of the sequence per pass (independent loads), the lanes' sums are
// scanned across the wave, and the exclusive prefixes are written back in
// place; the key's total goes to c2 / c1.
__global__ __launch_bounds__(kScanThreads) void scan_keys_kernel(LayoutArgs a) {
  const int lane = threadIdx.x & 63;
  const int key = blockIdx.x * (kScanThreads / 64) + (threadIdx.x >> 6);
  const int E2 = a.E2, N = a.N, G = a.G, R = N * G, tps = a.tps;
  if (key < E2 + R) {
    const bool expert = key < E2;
    const int d = key - E2, n = expert ? 0 : d / G, g = expert ? 0 : d - n * G;
    const int nsrc = expert ? 0 : (g < a.S ? (a.S - g + G - 1) / G : 0);
    const int len = expert ? a.n_tiles : nsrc * tps;
    // address of element q of the key's sequence
    auto at = [&](int q) -> int32_t* {
      if (expert) return a.hist_e + static_cast<int64_t>(q) * E2 + key;
      const int src = g + (q / tps) * G, tt = q - (q / tps) * tps;
      return a.hist_n + static_cast<int64_t>(src * tps + tt) * N + n;
    };
    int carry = 0;
    for (int base = 0; base < len; base += 64 * kScanPerLane) {
      const int q0 = base + lane * kScanPerLane;
      int v[kScanPerLane];
      int sum = 0;
#pragma unroll
      for (int c = 0; c < kScanPerLane; ++c) {
        v[c] = q0 + c < len ? *at(q0 + c) : 0;
        sum += v[c];
      }
      const int incl = wave_inclusive_scan(sum, lane);
      int run = carry + incl - sum;
#pragma unroll
      for (int c = 0; c < kScanPerLane; ++c) {
        if (q0 + c < len) *at(q0 + c) = run;
        run += v[c];
      }
      carry += __shfl(incl, 63, 64);
    }
    if (lane == 0) (expert ? a.c2 + key : a.c1 + d)[0] = carry;
  }
}

// Receive stage of a dispatch: the per-(expert, source) counters [E, S] as
// they are (one thread per counter), or summed over the sources (tokens per
// expert): one wave per expert, lanes over the sources (coalesced), then a
// shuffle reduction.
__global__ void recv_counts_kernel(const int32_t* counts, int E, int S, int per_expert, int32_t* out) {
  if (per_expert) {
    const int e = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (e >= E) return;
    int sum = 0;
    for (int s = lane; s < S; s += 64) sum += counts[static_cast<int64_t>(e) * S + s];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
    if (lane == 0) out[e] = sum;
  } else {
    const int64_t x = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (x < static_cast<int64_t>(E) * S) out[x] = counts[x];
  }
}

__global__ void fill_i32_kernel(int32_t* p, int64_t count, int32_t value) {
  for (int64_t x = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; x < count;
       x += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[x] = value;
}

template <int V>
void launch_tile_route(const LayoutArgs& a, int lpn, dim3 grid, size_t lds, hipStream_t stream) {
  const dim3 block(kTileThreads);
  switch (lpn) {
    case 1: tile_count_kernel<true, V, 1><<<grid, block, lds, stream>>>(a); break;
    case 2: tile_count_kernel<true, V, 2><<<grid, block, lds, stream>>>(a); break;
    case 4: tile_count_kernel<true, V, 4><<<grid, block, lds, stream>>>(a); break;
    case 8: tile_count_kernel<true, V, 8><<<grid, block, lds, stream>>>(a); break;
    case 16: tile_count_kernel<true, V, 16><<<grid, block, lds, stream>>>(a); break;
    default: tile_count_kernel<true, V, 32><<<grid, block, lds, stream>>>(a); break;
  }
}

}  // namespace

hipError_t launch_recv_counts(const int32_t* counts, int E, int S, int per_expert, int32_t* out,
                              hipStream_t stream) {
  const int64_t items = per_expert ? static_cast<int64_t>(E) * 64 : static_cast<int64_t>(E) * S;   // threads
  if (items <= 0) return hipSuccess;
  recv_counts_kernel<<<dim3(static_cast<unsigned>((items + 255) / 256)), dim3(256), 0, stream>>>(counts, E, S,
                                                                                              per_expert, out);
  return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t* p, int64_t count, int32_t value, hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  int64_t blocks = (count + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  fill_i32_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream>>>(p, count, value);
  return hipGetLastError();
}

hipError_t launch_layout(const LayoutArgs& a_in, hipStream_t stream) {
  if (a_in.n == 0) return hipSuccess;
  LayoutArgs a = a_in;
  const dim3 grid(static_cast<unsigned>(a.n_tiles));
  const size_t lds = static_cast<size_t>(a.E2 + a.N) * 4;
  int lpn = 0;
  bool routed = false;
  if (a.scores && fast_path(a.scores, a.ld, a.E, a.N, a.K, a.J, &lpn)) {
    // Route and count in one pass.
    switch (a.E / 32) {
      case 4: launch_tile_route<4>(a, lpn, grid, lds, stream); routed = true; break;
      case 8: launch_tile_route<8>(a, lpn, grid, lds, stream); routed = true; break;
      case 12: launch_tile_route<12>(a, lpn, grid, lds, stream); routed = true; break;
      case 16: launch_tile_route<16>(a, lpn, grid, lds, stream); routed = true; break;
      default: break;
    }
  }
  if (!routed) {
    if (a.scores) {
      // Shapes outside the fast path: the routing kernel first, then the
      // count reads its output.
      RouteArgs r{};
      r.scores = a.scores;
      r.ld = a.ld;
      r.n = a.n;
      r.E = a.E;
      r.N = a.N;
      r.K = a.K;
      r.M = a.M;
      r.J = a.J;
      r.topk = a.topk_out;
      if (const hipError_t e = launch_route(r, stream); e != hipSuccess) return e;
      a.topk = a.topk_out;
    }
    tile_count_kernel<false, 4, 1><<<grid, dim3(kTileThreads), lds, stream>>>(a);
  }
  if (a.ht) {
    const int keys = a.E2 + a.N * a.G;
    const int per = kScanThreads / 64;
    scan_keys_kernel<<<dim3(static_cast<unsigned>((keys + per - 1) / per)), dim3(kScanThreads), 0, stream>>>(a);
  } else {
    const int64_t pairs = static_cast<int64_t>(a.E2) * a.S;
    layout_scan_ll_kernel<<<dim3(static_cast<unsigned>((pairs + 255) / 256)), dim3(256), 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace ep
