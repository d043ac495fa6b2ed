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
#include "ep_route_dev.h"

namespace ep {
namespace {

using namespace route_dev;

constexpr int kTokensPerBlock = 4;

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
// Fast path (the shared device code): 32 lanes per token, two tokens per
// wave, eight tokens per 256-thread workgroup.
// ---------------------------------------------------------------------------

constexpr int kFastTokensPerBlock = 8;   // 4 waves x 2 tokens

template <int V, int LPN>
__global__ __launch_bounds__(256) void route_fast_kernel(RouteArgs a) {
  __shared__ float s_node[kFastTokensPerBlock][32];
  const int half = threadIdx.x >> 5;         // token slot in the block
  const int hl = threadIdx.x & 31;           // lane inside the token's 32
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kFastTokensPerBlock + half;
  const bool active = t < a.n;
  const int mine = route_token_fast<V, LPN>(a.scores + (active ? t : 0) * a.ld, active, hl, s_node[half], a.N,
                                            a.M, a.J, a.K);
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
  int lpn = 0;
  if (fast_path(a.scores, a.ld, a.E, a.N, a.K, a.J, &lpn)) {
    const int V = a.E / 32;
    const int64_t blocks = (a.n + kFastTokensPerBlock - 1) / kFastTokensPerBlock;
    const dim3 grid(static_cast<unsigned>(blocks)), block(256);
    if (V == 4) return launch_fast_v<4>(a, lpn, grid, block, stream);
    if (V == 8) return launch_fast_v<8>(a, lpn, grid, block, stream);
    if (V == 12) return launch_fast_v<12>(a, lpn, grid, block, stream);
    if (V == 16) return launch_fast_v<16>(a, lpn, grid, block, stream);
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
