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
//   * here, for every tile of 64 tokens of one source, the exclusive prefix
//     over the earlier tiles of each key's count plus the key's offset, and
//     the per-expert / per-rank totals and offsets;
//   * each token's rank inside its tile (64-bit lane masks per key, one wave
//     per tile), stored in the handle; the dispatch kernel adds rank and
//     tile prefix.
// Neither half uses atomics on positions, so every map is bit-reproducible.
// LL slots restart at 0 for every (expert, source), so no prefix crosses a
// source: when a source has at most kLlFusedTiles tiles, one count workgroup
// holds all of them and writes the prefixes and counts too (one launch).
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
  // an earlier entry of the same token.  vec8: K == 8 and the row is 16-byte
  // aligned, two 16-byte loads.
  __device__ void load(const int32_t* row, int K, int E, bool active, bool vec8) {
    if constexpr (KMAX == 8) {
      if (vec8) {
        const int4 m1{-1, -1, -1, -1};
        const int4 lo = active ? reinterpret_cast<const int4*>(row)[0] : m1;
        const int4 hi = active ? reinterpret_cast<const int4*>(row)[1] : m1;
        e[0] = lo.x; e[1] = lo.y; e[2] = lo.z; e[3] = lo.w;
        e[4] = hi.x; e[5] = hi.y; e[6] = hi.z; e[7] = hi.w;
      } else {
#pragma unroll
        for (int k = 0; k < KMAX; ++k) e[k] = (active && k < K) ? row[k] : -1;
      }
    } else {
#pragma unroll
      for (int k = 0; k < KMAX; ++k) e[k] = (active && k < K) ? row[k] : -1;
    }
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

constexpr int kScanRegs = 16;      // tile counts a scan thread keeps in registers

// Sum, and exclusive-prefix rewrite, of the values at idx(pos), pos in
// [p0, p1), 16 independent loads at a time so that the chain costs one
// round trip per 16 tiles instead of one per tile.
constexpr int kBatch = 16;

template <class Idx>
__device__ __forceinline__ int chunk_sum(const int32_t* base, int p0, int p1, Idx idx) {
  int run = 0;
  for (int pos = p0; pos < p1; pos += kBatch) {
    int v[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) v[q] = pos + q < p1 ? base[idx(pos + q)] : 0;
#pragma unroll
    for (int q = 0; q < kBatch; ++q) run += v[q];
  }
  return run;
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
__global__ __launch_bounds__(256) void layout_count_kernel(LayoutArgs a) {
  // Per wave (= tile of 64 tokens, lane = token): a 64-bit mask per expert
  // and per node of the lanes whose token uses it.  popcount(mask) is the
  // tile's count; popcount(mask & lanes-below) is the token's rank inside
  // the tile (a valid key occurs at most once per token).
  extern __shared__ uint64_t masks[];
  const int nw = blockDim.x >> 6;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int E = a.E, N = a.N, K = a.K, E2 = a.E2;
  uint64_t* m_e = masks;              // [nw][E2] stage-2 keys (experts, or ranks)
  uint64_t* m_n = masks + nw * E2;    // [nw][N]

  const int j = blockIdx.x * nw + w;
  const bool tile_ok = j < a.n_tiles;
  const int s = tile_ok ? j / a.tps : 0;
  const int t = (tile_ok ? j - s * a.tps : 0) * kTile + lane;
  const bool active = tile_ok && t < a.T;
  const int64_t i = static_cast<int64_t>(s) * a.T + t;

  for (int x = tid; x < nw * (E2 + N); x += blockDim.x) masks[x] = 0;
  // Token rows of 8 entries, 16-byte aligned: vector loads and stores.
  const bool vec8 = KMAX == 8 && K == 8 && (reinterpret_cast<uintptr_t>(a.topk) & 15u) == 0;
  Entries<KMAX> en;
  en.load(a.topk + (active ? i : 0) * K, K, E, active, vec8);
  // e / L and e / P by shifts when they are powers of two
  auto div_l = [&](int e) { return a.l_shift >= 0 ? e >> a.l_shift : e / a.L; };
  auto div_p = [&](int e) { return a.p_shift >= 0 ? e >> a.p_shift : e / a.P; };
  // Stage-2 key of each valid entry: its expert, or with the per-rank stage
  // 2 its rank, carried only by the token's first entry on that rank.
  int key[KMAX];
  bool first[KMAX];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    key[k] = a.s2_rank ? div_l(en.e[k]) : en.e[k];
    first[k] = en.ok[k];
  }
  if (a.s2_rank) {
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
#pragma unroll
      for (int q = 0; q < k; ++q) first[k] = first[k] && !(en.ok[q] && key[q] == key[k]);
  }
  __syncthreads();
  const uint64_t bit = 1ull << lane;
  uint64_t nodes = 0;
  if (active) {
    if constexpr (KMAX == 8) {
      if (vec8) {
        int4* dst = reinterpret_cast<int4*>(a.topk_copy + i * 8);
        dst[0] = int4{en.e[0], en.e[1], en.e[2], en.e[3]};
        dst[1] = int4{en.e[4], en.e[5], en.e[6], en.e[7]};
      } else {
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
          if (k < K) a.topk_copy[i * K + k] = en.e[k];
      }
    } else {
#pragma unroll
      for (int k = 0; k < KMAX; ++k)
        if (k < K) a.topk_copy[i * K + k] = en.e[k];
    }
    if (en.bad) atomicOr(a.err, en.bad);
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      if (!en.ok[k]) continue;
      if (first[k]) atomicOr(reinterpret_cast<unsigned long long*>(&m_e[w * E2 + key[k]]), bit);
      nodes |= 1ull << div_p(en.e[k]);
    }
    if (a.ht)
      for (int n = 0; n < N; ++n)
        if ((nodes >> n) & 1) atomicOr(reinterpret_cast<unsigned long long*>(&m_n[w * N + n]), bit);
  }
  __syncthreads();
  if (a.ll_fused) {
    // Workgroup = source blockIdx.x, wave q = its tile q: the exclusive
    // prefix over the earlier tiles and the (expert, source) count.
    for (int e = tid; e < E2; e += blockDim.x) {
      int run = 0;
      for (int q = 0; q < nw; ++q) {
        a.hist_e[(static_cast<int64_t>(blockIdx.x) * nw + q) * E2 + e] = run;
        run += __popcll(m_e[q * E2 + e]);
      }
      a.ll_count[static_cast<int64_t>(e) * a.S + blockIdx.x] = run;
    }
  } else if (tile_ok) {
    for (int e = lane; e < E2; e += 64) a.hist_e[static_cast<int64_t>(j) * E2 + e] = __popcll(m_e[w * E2 + e]);
    if (a.ht)
      for (int n = lane; n < N; n += 64) a.hist_n[static_cast<int64_t>(j) * N + n] = __popcll(m_n[w * N + n]);
  }
  if (active) {
    const uint64_t below = bit - 1;
    int re[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) re[k] = first[k] ? __popcll(m_e[w * E2 + key[k]] & below) : -1;
    if constexpr (KMAX == 8) {
      if (vec8) {
        int4* dst = reinterpret_cast<int4*>(a.rank_e + i * 8);
        dst[0] = int4{re[0], re[1], re[2], re[3]};
        dst[1] = int4{re[4], re[5], re[6], re[7]};
      } else {
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
          if (k < K) a.rank_e[i * K + k] = re[k];
      }
    } else {
#pragma unroll
      for (int k = 0; k < KMAX; ++k)
        if (k < K) a.rank_e[i * K + k] = re[k];
    }
    if (a.ht) {
      if (N == 8) {
        int rn[8];
#pragma unroll
        for (int n = 0; n < 8; ++n) rn[n] = ((nodes >> n) & 1) ? __popcll(m_n[w * 8 + n] & below) : -1;
        int4* dst = reinterpret_cast<int4*>(a.rank_n + i * 8);
        dst[0] = int4{rn[0], rn[1], rn[2], rn[3]};
        dst[1] = int4{rn[4], rn[5], rn[6], rn[7]};
      } else {
        for (int n = 0; n < N; ++n)
          a.rank_n[i * N + n] = ((nodes >> n) & 1) ? __popcll(m_n[w * N + n] & below) : -1;
      }
    }
  }
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

// HT: two workgroups turn the tile histograms into exclusive prefix sums,
// one for the stage-2 keys and one for the stage-1 ranks (the kernel
// boundary makes the counts of every tile visible; no fences).
__global__ __launch_bounds__(1024) void layout_scan_kernel(LayoutArgs a) {
  extern __shared__ int smem[];
  const int B = blockDim.x;
  const int tid = threadIdx.x;
  const int E = a.E2, N = a.N;   // stage-2 keys: the experts, or the ranks (per-rank HT)
  const int n_tiles = a.n_tiles;
  {
    // HT.  Keys: the E stage-2 keys (sequence: every tile in order) and the R
    // stage-1 ranks d = n*G + g (sequence: the tiles of the sources at
    // position g, tps consecutive tiles per source).  Workgroup 0 scans the
    // stage-2 keys and workgroup 1 the stage-1 ranks: the two are
    // independent, and split they run side by side.  A thread owns one
    // (key, chunk) of its workgroup's kind; it walks its chunk with pointer
    // strides (no divisions in the loops) and keeps up to kScanRegs counts
    // in registers between the sum and the rewrite.
    const int G = a.G, R = N * G, tps = a.tps;
    // Chunks per key: enough for kScanRegs tiles each, at most B / keys.
    const int max_rail = ((a.S + G - 1) / G) * tps;
    const int ce = max(1, min(B / E, (n_tiles + kScanRegs - 1) / kScanRegs));    // expert chunks
    const int cl_e = (n_tiles + ce - 1) / ce;             // tiles per expert chunk
    const int cr = max(1, min(B / R, (max_rail + kScanRegs - 1) / kScanRegs));   // rank chunks
    const int cl_r = (max_rail + cr - 1) / cr;            // tiles per rank chunk
    int* part_e = smem;                  // [ce][E]
    int* part_r = part_e + ce * E;       // [cr][R]
    int* tot_e = part_r + cr * R;        // [E]
    int* tot_r = tot_e + E;              // [R]
    int* scratch = tot_r + R;            // [2][B/64]
    const int lane = tid & 63, wv = tid >> 6, nw = B >> 6;

    const bool blk_e = blockIdx.x == 0, blk_r = blockIdx.x == 1;
    // Expert pair (e, c): tiles [c*cl_e, ...), address stride E.
    const bool has_e = blk_e && tid < ce * E;
    const int e = tid % E, ce_i = tid / E;
    const int je0 = ce_i * cl_e, ne = has_e ? max(0, min(cl_e, n_tiles - je0)) : 0;
    int32_t* pe = a.hist_e + static_cast<int64_t>(je0) * E + e;
    // Rank pair (d, c): positions [c*cl_r, ...) of the rail sequence.
    const bool has_r = blk_r && tid < cr * R;
    const int d = tid % R, cr_i = tid / R, n = d / G, g = d - (d / G) * G;
    const int nsrc = g < a.S ? (a.S - g + G - 1) / G : 0;
    const int pr0 = cr_i * cl_r, nr = has_r ? max(0, min(cl_r, nsrc * tps - pr0)) : 0;
    // the first tile of the chunk: source g + (pr0/tps)*G, tile pr0 % tps
    const int r_src0 = g + (pr0 / tps) * G, r_tt0 = pr0 % tps;

    // Registers when the workgroup's chunks fit them; longer chunks (many
    // tiles per key) go through memory in batches of kBatch loads.
    const bool regs = blk_e ? cl_e <= kScanRegs : cl_r <= kScanRegs;
    // tile counter of rail position pos of rank d: source g + (pos/tps)*G, tile pos % tps
    auto rail = [=](int pos) {
      return static_cast<int64_t>((g + (pos / tps) * G) * tps + pos % tps) * N + n;
    };
    auto expert = [=](int q) { return static_cast<int64_t>(q) * E; };
    int ve[kScanRegs], vr[kScanRegs];
    int se = 0, sr = 0;
    if (regs) {
#pragma unroll
      for (int q = 0; q < kScanRegs; ++q) ve[q] = q < ne ? pe[static_cast<int64_t>(q) * E] : 0;
      int src = r_src0, tt = r_tt0;
#pragma unroll
      for (int q = 0; q < kScanRegs; ++q) {
        vr[q] = q < nr ? a.hist_n[static_cast<int64_t>(src * tps + tt) * N + n] : 0;
        if (++tt == tps) { tt = 0; src += G; }
      }
#pragma unroll
      for (int q = 0; q < kScanRegs; ++q) { se += ve[q]; sr += vr[q]; }
    } else {
      se = chunk_sum(pe, 0, ne, expert);
      sr = chunk_sum(a.hist_n, pr0, pr0 + nr, rail);
    }
    if (has_e) part_e[ce_i * E + e] = se;
    if (has_r) part_r[cr_i * R + d] = sr;
    __syncthreads();
    // Thread x owns key x of its workgroup's kind (E, R <= B): prefix over
    // the key's chunks, then one exclusive scan of the key totals across the
    // workgroup (shuffles inside a wave, one barrier across waves).
    int te = 0, tr = 0;
    if (blk_e && tid < E) {
      for (int c = 0; c < ce; ++c) {
        const int t = part_e[c * E + tid];
        part_e[c * E + tid] = te;
        te += t;
      }
      a.c2[tid] = te;
    }
    if (blk_r && tid < R) {
      for (int c = 0; c < cr; ++c) {
        const int t = part_r[c * R + tid];
        part_r[c * R + tid] = tr;
        tr += t;
      }
      a.c1[tid] = tr;
    }
    int ie = te, ir = tr;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int oe = __shfl_up(ie, off, 64), orr = __shfl_up(ir, off, 64);
      if (lane >= off) { ie += oe; ir += orr; }
    }
    if (lane == 63) { scratch[wv] = ie; scratch[nw + wv] = ir; }
    __syncthreads();
    int be = 0, br = 0;
    for (int q = 0; q < wv; ++q) { be += scratch[q]; br += scratch[nw + q]; }
    if (blk_e && tid < E) {
      tot_e[tid] = be + ie - te;
      a.off2[tid] = be + ie - te;
    }
    if (blk_r && tid < R) {
      tot_r[tid] = br + ir - tr;
      a.off1[tid] = br + ir - tr;
    }
    __syncthreads();
    if (has_e) {
      int run = tot_e[e] + part_e[ce_i * E + e];
      if (regs) {
#pragma unroll
        for (int q = 0; q < kScanRegs; ++q) {
          if (q < ne) pe[static_cast<int64_t>(q) * E] = run;
          run += ve[q];
        }
      } else {
        chunk_prefix(pe, 0, ne, run, expert);
      }
    }
    if (has_r) {
      int run = tot_r[d] + part_r[cr_i * R + d];
      int src = r_src0, tt = r_tt0;
      if (regs) {
#pragma unroll
        for (int q = 0; q < kScanRegs; ++q) {
          if (q < nr) a.hist_n[static_cast<int64_t>(src * tps + tt) * N + n] = run;
          run += vr[q];
          if (++tt == tps) { tt = 0; src += G; }
        }
      } else {
        chunk_prefix(a.hist_n, pr0, pr0 + nr, run, rail);
      }
    }
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

constexpr int kCountWaves = 1;     // tiles per count workgroup (one wave: the tiles spread over CUs)
constexpr int kLlFusedTiles = 4;   // LL: a source of at most this many tiles is one workgroup
constexpr int kScanThreads = 1024;

}  // namespace

size_t layout_scan_lds_bytes(int E, int N, int G, int S, int tps) {
  (void)S;
  (void)tps;
  const int R = N * G;
  const int ce = kScanThreads / E > 0 ? kScanThreads / E : 1;
  const int cr = kScanThreads / R > 0 ? kScanThreads / R : 1;
  return (static_cast<size_t>(ce) * E + static_cast<size_t>(cr) * R + E + R + 2 * (kScanThreads / 64)) * 4;
}

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
  a.ll_fused = !a.ht && a.tps <= kLlFusedTiles;
  // Fused LL: one workgroup per source, one wave per tile of the source.
  const int waves = a.ll_fused ? a.tps : kCountWaves;
  const dim3 grid(static_cast<unsigned>(a.ll_fused ? a.S : (a.n_tiles + kCountWaves - 1) / kCountWaves));
  const dim3 block(waves * 64);
  const size_t lds = static_cast<size_t>(waves) * (a.E2 + a.N) * 8;
  if (a.K <= 8) layout_count_kernel<8><<<grid, block, lds, stream>>>(a);
  else layout_count_kernel<32><<<grid, block, lds, stream>>>(a);
  if (a.ll_fused) return hipGetLastError();
  if (a.ht) {
    layout_scan_kernel<<<dim3(2), dim3(kScanThreads), layout_scan_lds_bytes(a.E2, a.N, a.G, a.S, a.tps), stream>>>(a);
  } else {
    const int64_t pairs = static_cast<int64_t>(a.E2) * a.S;
    layout_scan_ll_kernel<<<dim3(static_cast<unsigned>((pairs + 255) / 256)), dim3(256), 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace ep
