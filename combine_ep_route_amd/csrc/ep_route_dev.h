// Device code of the node-limited top-k routing fast path, shared by the
// routing kernel and the handle kernel that routes and counts in one pass.
//
// Rule ("NVSHMEM and DeepEP: GPU-initiated communication", high-throughput
// section): score each node by the sum of its ceil(K/M) best expert scores
// (2 at K=8, M=4), keep the M best nodes, then take the K best experts among
// the kept nodes.  Ties go to the lower node index, then to the lower expert
// index; experts are emitted in descending score order.
//
// Fast-path mapping: 32 lanes per token (two tokens per wave), V = E/32
// consecutive experts per lane (one or more 16-byte loads), a node spans
// LPN = P/V lanes (a power of two).  All cross-lane steps are DPP row
// permutations or ds_swizzle inside the 32-lane half, so nothing waits on LDS
// except the single exchange of the N node scores.  The K experts come from a
// tournament: each lane sorts its V selection keys (V a power of two), then K
// rounds each take the 32-lane maximum of the lanes' heads and the lane that
// held it moves its next key up.  (A merge tree -- five pairwise merges of
// the lanes' sorted lists -- costs about 500 VALU operations per wave against
// about 330 here.)  For other V, K rounds of a maximum over unsorted keys.
#pragma once

#include "ep_internal.h"

namespace ep {
namespace route_dev {

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


// Routes one token with the 32 lanes of a half wave (lane hl of the half).
// `row` is the token's score row (16-byte aligned), `node_slot` the token's
// 32 floats of LDS for the node-score exchange.  Every thread of the
// workgroup must call this (it holds a workgroup barrier when M > 0).
// Returns the expert of rank hl (hl < K), else -1.
template <int V, int LPN>
__device__ __forceinline__ int route_token_fast(const float* row, bool active, int hl, float* node_slot, int N,
                                                int M, int J, int K) {
  row += hl * V;
  float val[V];
#pragma unroll
  for (int q = 0; q < V / 4; ++q) {
    const float4 f = active ? reinterpret_cast<const float4*>(row)[q] : make_float4(0.f, 0.f, 0.f, 0.f);
    val[4 * q] = f.x; val[4 * q + 1] = f.y; val[4 * q + 2] = f.z; val[4 * q + 3] = f.w;
  }
  const int node = hl / LPN;
  bool keep = true;
  if (M > 0) {
    // top-2 (or top-1) of the lane's V scores, merged across the node's lanes
    float a1 = val[0], a2 = -INFINITY;
#pragma unroll
    for (int v = 1; v < V; ++v) {
      const float x = val[v];
      a2 = fmaxf(a2, fminf(a1, x));
      a1 = fmaxf(a1, x);
    }
    node_top2<LPN>(a1, a2);
    const float ns = J == 2 ? a1 + a2 : a1;
    if (hl % LPN == 0) node_slot[node] = ns;
    __syncthreads();
    int rank = 0;
    for (int m = 0; m < N; ++m) {
      const float o = node_slot[m];
      rank += (o > ns) || (o == ns && m < node);
    }
    keep = rank < M;
  }

  const int e0 = hl * V;
  uint64_t key[V];
#pragma unroll
  for (int v = 0; v < V; ++v) key[v] = keep ? select_key(val[v], e0 + v) : 0ull;
  int mine = -1;
  if ((V & (V - 1)) == 0) {
    // Tournament: each lane sorts its V keys, then K rounds take the 32-lane
    // maximum of the lanes' heads; the lane holding it (keys are distinct)
    // moves its next key up.
    bitonic_sort_desc<V>(key);
    for (int k = 0; k < K; ++k) {
      uint32_t hi = static_cast<uint32_t>(key[0] >> 32), lo = static_cast<uint32_t>(key[0]);
      max_step<0>(hi, lo);
      max_step<1>(hi, lo);
      max_step<2>(hi, lo);
      max_step<3>(hi, lo);
      max_step<4>(hi, lo);
      if (hl == k) mine = static_cast<int>(0xFFFFFFFFu - lo);
      if (key[0] == ((static_cast<uint64_t>(hi) << 32) | lo)) {
#pragma unroll
        for (int v = 0; v + 1 < V; ++v) key[v] = key[v + 1];
        key[V - 1] = 0;
      }
    }
  } else {
    // K rounds of a 32-lane maximum of the lanes' best remaining keys.
    for (int k = 0; k < K; ++k) {
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
  return mine;
}

// Whether the fast path takes this shape: E a multiple of 128 up to 512,
// K <= 32, a node spanning a power-of-two number of lanes (at most 32), node
// sums of at most 2 scores, 16-byte aligned rows.  *lpn is the lanes per node.
inline bool fast_path(const float* scores, int64_t ld, int E, int N, int K, int J, int* lpn) {
  const int P = E / N, V = E / 32;
  const bool aligned = (reinterpret_cast<uintptr_t>(scores) % 16 == 0) && (ld % 4 == 0);
  if (!(aligned && E % 128 == 0 && V <= 16 && K <= 32 && J <= 2 && P % V == 0)) return false;
  const int l = P / V;
  if ((l & (l - 1)) != 0 || l > 32) return false;
  *lpn = l;
  return true;
}

}  // namespace route_dev
}  // namespace ep
