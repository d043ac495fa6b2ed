// A1: node-limited top-k routing on gfx950.
//
// Rule ("NVSHMEM and DeepEP: GPU-initiated communication", high-throughput
// section): score each node by the sum of its ceil(K/M) best expert scores
// (2 at K=8, M=4), keep the M best nodes, then take the K best experts among
// the kept nodes.  Ties go to the lower node index, then to the lower expert
// index; experts are emitted in descending score order.
//
// Mapping: one wave64 per token, four tokens per 256-thread workgroup.  A
// token's E scores are read with coalesced 256-byte wave loads (expert
// e = v*64 + lane sits in register v of that lane) and mirrored in LDS for
// the per-node scans.  Lanes 0..N-1 each score one node, then rank it among
// the N node scores.  The K experts are chosen by K rounds of a wave-wide
// arg-max over 64-bit keys (ordered score bits, then the complemented expert
// index), so equal scores resolve to the lower index without a second pass.
#include "ep_internal.h"

namespace ep {
namespace {

constexpr int kTokensPerBlock = 4;

// 64-bit selection key of (score f, expert e): the score's bits in unsigned
// order (-0 taken as +0 and a NaN below every number, as a float comparison
// has them), then the complemented index, so that a larger key is a higher
// score or, at equal scores, a lower index.  Key 0 is below every expert.
__device__ __forceinline__ uint64_t select_key(float f, int e) {
  const float c = f + 0.0f;   // -0 -> +0
  const uint32_t u = __float_as_uint(c);
  uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  if (c != c) o = 0;
  return (static_cast<uint64_t>(o) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(e));
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), off, 64);
    uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), off, 64);
    uint64_t o = (static_cast<uint64_t>(hi) << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

template <int NV>
__global__ __launch_bounds__(256) void route_kernel(RouteArgs a) {
  __shared__ float s_val[kTokensPerBlock][NV * 64];
  __shared__ float s_node[kTokensPerBlock][kMaxNodes];
  __shared__ int s_keep[kTokensPerBlock][kMaxNodes];

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kTokensPerBlock + wave;
  const bool active = t < a.n;
  const int E = a.E, N = a.N, P = E / N;
  const float* row = a.scores + (active ? t : 0) * a.ld;

  float val[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int e = v * 64 + lane;
    val[v] = (active && e < E) ? row[e] : 0.0f;
    if (e < E) s_val[wave][e] = val[v];
  }
  __syncthreads();

  const bool limited = a.M > 0;
  if (limited && lane < N) {
    // Sum of the node's J largest scores, largest first.  Pass j takes the
    // best entry strictly after the previous pick in (score desc, index asc).
    const float* nv = &s_val[wave][lane * P];
    float acc = 0.0f, pv = 0.0f;
    int pi = -1;
    for (int j = 0; j < a.J; ++j) {
      float bv = 0.0f;
      int bi = -1;
      for (int p = 0; p < P; ++p) {
        const float v = nv[p];
        const bool after = (pi < 0) || (v < pv) || (v == pv && p > pi);
        if (after && (bi < 0 || v > bv)) { bv = v; bi = p; }
      }
      acc = (j == 0) ? bv : acc + bv;
      pv = bv;
      pi = bi;
    }
    s_node[wave][lane] = acc;
  }
  __syncthreads();
  if (limited && lane < N) {
    const float mine = s_node[wave][lane];
    int rank = 0;
    for (int m = 0; m < N; ++m) {
      const float o = s_node[wave][m];
      rank += (o > mine) || (o == mine && m < lane);
    }
    s_keep[wave][lane] = rank < a.M;
  }
  __syncthreads();

  uint64_t key[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const int e = v * 64 + lane;
    const bool ok = e < E && (!limited || s_keep[wave][e / P]);
    key[v] = ok ? select_key(val[v], e)
                : 0ull;
  }

  int mine = -1;
  for (int k = 0; k < a.K; ++k) {
    uint64_t best = 0;
#pragma unroll
    for (int v = 0; v < NV; ++v) best = key[v] > best ? key[v] : best;
    best = wave_max_u64(best);
    const int e = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(best));
    if (lane == k) mine = e;
    if ((e & 63) == lane) {
#pragma unroll
      for (int v = 0; v < NV; ++v)
        if (v == (e >> 6)) key[v] = 0;
    }
  }
  if (active && lane < a.K) a.topk[t * a.K + lane] = mine;
}

// ---------------------------------------------------------------------------
// Fast path: 32 lanes per token (two tokens per wave), V = E/32 consecutive
// experts per lane (one or more 16-byte loads), a node spans LPN = P/V lanes
// (a power of two).  All cross-lane steps are DPP row permutations or
// ds_swizzle inside the 32-lane half, so nothing waits on LDS except the
// single exchange of the N node scores.  The K experts come from a merge
// tree (each lane sorts its V selection keys, five pairwise merges over the
// exchange pattern leave the V best in every lane) when K <= V and V is a
// power of two, else from K rounds of a 32-lane maximum.
// ---------------------------------------------------------------------------

constexpr int kFastTokensPerBlock = 8;   // 4 waves x 2 tokens

template <int CTRL>
__device__ __forceinline__ int dpp(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ int swz_xor16(int x) {
  return __builtin_amdgcn_ds_swizzle(x, 0x401F);   // xor lane 16 within 32
}
constexpr int kQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141;   // lane i <-> 7-i inside 8
constexpr int kRowMirror = 0x140;    // lane i <-> 15-i inside 16

template <int STEP>
__device__ __forceinline__ int xchg(int x) {
  if constexpr (STEP == 0) return dpp<kQuadXor1>(x);
  else if constexpr (STEP == 1) return dpp<kQuadXor2>(x);
  else if constexpr (STEP == 2) return dpp<kHalfMirror>(x);
  else if constexpr (STEP == 3) return dpp<kRowMirror>(x);
  else return swz_xor16(x);
}
template <int STEP>
__device__ __forceinline__ float xchgf(float x) { return __int_as_float(xchg<STEP>(__float_as_int(x))); }


// Compare-exchange of two keys so that a holds the larger.
__device__ __forceinline__ void cx(uint64_t& a, uint64_t& b) {
  const uint64_t x = a, y = b;
  const bool sw = y > x;
  a = sw ? y : x;
  b = sw ? x : y;
}

// Sort V keys (a power of two) largest first: bitonic network.
template <int V>
__device__ __forceinline__ void bitonic_sort_desc(uint64_t (&k)[V]) {
#pragma unroll
  for (int size = 2; size <= V; size <<= 1)
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1)
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const int j = i ^ stride;
        if (j > i) {
          if ((i & size) == 0) cx(k[i], k[j]);
          else cx(k[j], k[i]);
        }
      }
}

// One level of the merge tree: the union of the lane's sorted V keys and its
// partner's (exchange STEP) cut to its V largest, sorted.  max(mine[i],
// partner[V-1-i]) is a bitonic sequence holding the V largest; a half-cleaner
// cascade sorts it.  Both partners end with the same list.
template <int STEP, int V>
__device__ __forceinline__ void merge_level(uint64_t (&k)[V]) {
  uint64_t o[V];
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const uint32_t hi = static_cast<uint32_t>(xchg<STEP>(static_cast<int>(k[i] >> 32)));
    const uint32_t lo = static_cast<uint32_t>(xchg<STEP>(static_cast<int>(k[i])));
    o[i] = (static_cast<uint64_t>(hi) << 32) | lo;
  }
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const uint64_t p = o[V - 1 - i];
    k[i] = p > k[i] ? p : k[i];
  }
#pragma unroll
  for (int stride = V >> 1; stride > 0; stride >>= 1)
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const int j = i ^ stride;
      if (j > i) cx(k[i], k[j]);
    }
}

// One exchange of a 32-lane maximum of 64-bit keys held as (hi, lo).
template <int STEP>
__device__ __forceinline__ void max_step(uint32_t& hi, uint32_t& lo) {
  const uint32_t ohi = static_cast<uint32_t>(xchg<STEP>(static_cast<int>(hi)));
  const uint32_t olo = static_cast<uint32_t>(xchg<STEP>(static_cast<int>(lo)));
  const uint64_t o = (static_cast<uint64_t>(ohi) << 32) | olo;
  const uint64_t m = (static_cast<uint64_t>(hi) << 32) | lo;
  if (o > m) { hi = ohi; lo = olo; }
}

// Merge the node top-2 (a1 >= a2) with a partner group's over one exchange.
template <int STEP>
__device__ __forceinline__ void top2_step(float& a1, float& a2) {
  const float b1 = xchgf<STEP>(a1), b2 = xchgf<STEP>(a2);
  const float hi = fmaxf(a1, b1), lo = fminf(a1, b1);
  a2 = fmaxf(lo, fmaxf(a2, b2));
  a1 = hi;
}

// Steps that cover a group of LPN lanes with disjoint partial sets at every
// step: (xor 16), row mirror, half mirror, quad xor 2, quad xor 1.
template <int LPN>
__device__ __forceinline__ void node_top2(float& a1, float& a2) {
  if constexpr (LPN >= 32) top2_step<4>(a1, a2);
  if constexpr (LPN >= 16) top2_step<3>(a1, a2);
  if constexpr (LPN >= 8) top2_step<2>(a1, a2);
  if constexpr (LPN >= 4) top2_step<1>(a1, a2);
  if constexpr (LPN >= 2) top2_step<0>(a1, a2);
}

template <int V, int LPN>
__global__ __launch_bounds__(256) void route_fast_kernel(RouteArgs a) {
  __shared__ float s_node[kFastTokensPerBlock][32];
  const int half = threadIdx.x >> 5;         // token slot in the block
  const int hl = threadIdx.x & 31;           // lane inside the token's 32
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kFastTokensPerBlock + half;
  const bool active = t < a.n;
  const float* row = a.scores + (active ? t : 0) * a.ld + hl * V;

  float val[V];
#pragma unroll
  for (int q = 0; q < V / 4; ++q) {
    const float4 f = active ? reinterpret_cast<const float4*>(row)[q] : make_float4(0.f, 0.f, 0.f, 0.f);
    val[4 * q] = f.x; val[4 * q + 1] = f.y; val[4 * q + 2] = f.z; val[4 * q + 3] = f.w;
  }
  const int N = a.N;
  const int node = hl / LPN;
  bool keep = true;
  if (a.M > 0) {
    // top-2 (or top-1) of the lane's V scores, merged across the node's lanes
    float a1 = val[0], a2 = -INFINITY;
#pragma unroll
    for (int v = 1; v < V; ++v) {
      const float x = val[v];
      a2 = fmaxf(a2, fminf(a1, x));
      a1 = fmaxf(a1, x);
    }
    node_top2<LPN>(a1, a2);
    const float ns = a.J == 2 ? a1 + a2 : a1;
    if (hl % LPN == 0) s_node[half][node] = ns;
    __syncthreads();
    int rank = 0;
    for (int m = 0; m < N; ++m) {
      const float o = s_node[half][m];
      rank += (o > ns) || (o == ns && m < node);
    }
    keep = rank < a.M;
  }

  const int e0 = hl * V;
  uint64_t key[V];
#pragma unroll
  for (int v = 0; v < V; ++v) key[v] = keep ? select_key(val[v], e0 + v) : 0ull;
  int mine = -1;
  if ((V & (V - 1)) == 0 && a.K <= V) {
    // Merge tree: sort the lane's keys, then five levels of pairwise merges
    // over the 32 lanes leave every lane with the token's V best, in order.
    bitonic_sort_desc<V>(key);
    merge_level<0, V>(key);
    merge_level<1, V>(key);
    merge_level<2, V>(key);
    merge_level<3, V>(key);
    merge_level<4, V>(key);
#pragma unroll
    for (int v = 0; v < V; ++v)
      if (hl == v) mine = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(key[v]));
  } else {
    // K rounds of a 32-lane maximum of the lanes' best remaining keys.
    for (int k = 0; k < a.K; ++k) {
      uint64_t best = 0;
#pragma unroll
      for (int v = 0; v < V; ++v) best = key[v] > best ? key[v] : best;
      uint32_t hi = static_cast<uint32_t>(best >> 32), lo = static_cast<uint32_t>(best);
      max_step<0>(hi, lo);
      max_step<1>(hi, lo);
      max_step<2>(hi, lo);
      max_step<3>(hi, lo);
      max_step<4>(hi, lo);
      const uint64_t w = (static_cast<uint64_t>(hi) << 32) | lo;
      if (hl == k) mine = static_cast<int>(0xFFFFFFFFu - lo);
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (key[v] == w) key[v] = 0;
    }
  }
  if (active && hl < a.K) a.topk[t * a.K + hl] = mine;
}

template <int V>
hipError_t launch_fast_v(const RouteArgs& a, int lpn, dim3 grid, dim3 block, hipStream_t stream) {
  switch (lpn) {
    case 1: route_fast_kernel<V, 1><<<grid, block, 0, stream>>>(a); break;
    case 2: route_fast_kernel<V, 2><<<grid, block, 0, stream>>>(a); break;
    case 4: route_fast_kernel<V, 4><<<grid, block, 0, stream>>>(a); break;
    case 8: route_fast_kernel<V, 8><<<grid, block, 0, stream>>>(a); break;
    case 16: route_fast_kernel<V, 16><<<grid, block, 0, stream>>>(a); break;
    default: route_fast_kernel<V, 32><<<grid, block, 0, stream>>>(a); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, hipStream_t stream) {
  if (a.n == 0) return hipSuccess;
  // Fast path: E a multiple of 128 up to 512, K <= 32, a node spanning a
  // power-of-two number of lanes, node sums of at most 2 scores, 16-byte
  // aligned rows.
  const int P = a.E / a.N;
  const int V = a.E / 32;
  const bool aligned = (reinterpret_cast<uintptr_t>(a.scores) % 16 == 0) && (a.ld % 4 == 0);
  if (aligned && a.E % 128 == 0 && V <= 16 && a.K <= 32 && a.J <= 2 && P % V == 0) {
    const int lpn = P / V;
    if ((lpn & (lpn - 1)) == 0 && lpn <= 32) {
      const int64_t blocks = (a.n + kFastTokensPerBlock - 1) / kFastTokensPerBlock;
      const dim3 grid(static_cast<unsigned>(blocks)), block(256);
      if (V == 4) return launch_fast_v<4>(a, lpn, grid, block, stream);
      if (V == 8) return launch_fast_v<8>(a, lpn, grid, block, stream);
      if (V == 12) return launch_fast_v<12>(a, lpn, grid, block, stream);
      if (V == 16) return launch_fast_v<16>(a, lpn, grid, block, stream);
    }
  }
  const int64_t blocks = (a.n + kTokensPerBlock - 1) / kTokensPerBlock;
  const dim3 grid(static_cast<unsigned>(blocks)), block(256);
  const int nv = (a.E + 63) / 64;
  if (nv <= 1) route_kernel<1><<<grid, block, 0, stream>>>(a);
  else if (nv <= 2) route_kernel<2><<<grid, block, 0, stream>>>(a);
  else if (nv <= 4) route_kernel<4><<<grid, block, 0, stream>>>(a);
  else if (nv <= 8) route_kernel<8><<<grid, block, 0, stream>>>(a);
  else route_kernel<16><<<grid, block, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace ep
