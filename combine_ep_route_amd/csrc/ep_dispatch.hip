// A3 + A4 / A5 + A6: for each token, finish its slots / rows from the
// handle's tile prefix sums, quantise it once and write its row to every
// destination (LL messages, HT stage-1 and stage-2 rows).
//
// Sources: "NVSHMEM and DeepEP: GPU-initiated communication" -- FP8 dispatch
// with one fp32 scale per 128 elements (7168 + 56*4 bytes per token), LL
// message = payload + scales + 16-byte header (7408 B), fixed slots per
// (local expert, source rank), HT one copy per destination node at the
// same-position GPU followed by the intra-node forward; "NCCL EP paper
// notes" -- quantisation inside the send kernel's prepare stage, message
// sizes 7408 B (FP8) / 14352 B (BF16).
//
// Mapping: a token is split over W waves, each owning a contiguous range of
// 64*NV chunks (16 elements; 8 with a BF16 payload; lane l: chunks
// c0 + v*64, v < NV); the waves of a workgroup (4 in HT, 2 in LL) work on
// their own -- each wave ranks its token itself.  The one exception is the
// HT key offsets, which the workgroup scans into LDS once, at the start.
//  1. Loads, in the order their results are needed (they complete in
//     order): the inputs of the token's positions -- its entries, their
//     in-tile ranks, its node ranks and its tile's prefix row, lane by lane
//     -- then the payload (16-byte loads).  Everything a position needs
//     arrives in one round trip.
//  2. A 128-element block is 8 consecutive lanes; its amax is a 3-step
//     xor-shuffle inside a DPP row.  scale = amax/448 (IEEE fp32 division)
//     and q = E4M3(x/scale), the quotient by a refined reciprocal and one
//     fused residual correction, on operands pre-scaled by 2^64 when the
//     scale is tiny (the tests compare the codes with the IEEE quotient's
//     for every finite bf16 amax).  Quantising comes before
//     the positions, so the raw chunks' registers are free early.
//  3. Lane k works out entry k's slot / row: its rank inside its tile plus
//     the tile's prefix (plus, in HT, the key's first row from LDS); lane n
//     does node n's stage-1 row.  Each row's position is read out of its
//     lane when the row is written.
//  4. Rows start on 128-byte boundaries (the buffers' row pitch is the row
//     size rounded up to 128 B).  Each chunk of codes goes to every
//     destination row with non-temporal stores (nothing on this GPU reads
//     the rows back during the pass).  When H is a multiple of 512 the
//     token's last wave writes each row's last 128-byte line whole: scales,
//     LL header, zeros up to the pitch, so that no line is written in part.
//     Otherwise the wave's block scales are gathered into its first lanes
//     and written by one store instruction (16 bytes per 4 blocks), and the
//     padding is never written.
#include "ep_internal.h"

namespace ep {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = kLayoutTile;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ void store_nt(u32x4 v, uint8_t* p) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// Loaded source chunk of a token.
struct Raw {
  u32x4 a, b;
  float scale;   // this lane's block scale
};

template <int IN>  // 0: BF16 in -> FP8, 1: BF16 in -> BF16, 2: FP8 in -> FP8
__device__ __forceinline__ Raw load_chunk(const DispatchArgs& p, int64_t i, int c, bool active) {
  Raw r;
  const u32x4 zero{0, 0, 0, 0};
  r.scale = 0.0f;
  if constexpr (IN == 2) {
    const uint8_t* src = static_cast<const uint8_t*>(p.x) + i * p.ld_x;
    r.a = active ? *reinterpret_cast<const u32x4*>(src + 16 * c) : zero;
    r.b = zero;
    r.scale = active ? p.x_scales[i * p.ld_s + (c >> 3)] : 0.0f;
  } else if constexpr (IN == 1) {
    // BF16 kept as BF16: a chunk is 8 values (16 bytes), a plain copy
    const uint16_t* src = static_cast<const uint16_t*>(p.x) + i * p.ld_x;
    r.a = active ? *reinterpret_cast<const u32x4*>(src + 8 * c) : zero;
    r.b = zero;
  } else {
    const uint16_t* src = static_cast<const uint16_t*>(p.x) + i * p.ld_x;
    const u32x4* s4 = reinterpret_cast<const u32x4*>(src + 16 * c);
    r.a = active ? s4[0] : zero;
    r.b = active ? s4[1] : zero;
  }
  return r;
}

// Quantise a loaded BF16 chunk: 16 codes in r.a, block scale in r.scale.
__device__ __forceinline__ void quantize(Raw& r) {
  float f[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f[2 * q] = bf16_lo(r.a[q]);
    f[2 * q + 1] = bf16_hi(r.a[q]);
    f[8 + 2 * q] = bf16_lo(r.b[q]);
    f[8 + 2 * q + 1] = bf16_hi(r.b[q]);
  }
  float amax = 0.0f;
#pragma unroll
  for (int q = 0; q < 16; ++q) amax = fmaxf(amax, fabsf(f[q]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 4, 64));
  u32x4 out{0, 0, 0, 0};
  r.scale = 0.0f;
  if (amax != 0.0f) {
    const float scale = amax / 448.0f;
    r.scale = scale;
    float qv[16];
    // The quotient x/scale by Markstein's scheme: a Newton step refines the
    // hardware reciprocal, and one fused residual correction rounds the
    // quotient.  The correction is exact only while the residual
    // x - q0*scale is a normal fp32 number or a multiple of 2^-149; it is a
    // multiple of about 2^-47 |x|, so that holds for |x| >= 2^-102.  Blocks
    // with scale < 2^-64 therefore work on x*2^64 and scale*2^64 (both exact,
    // the quotient unchanged): then every x whose code can be non-zero
    // (|x| >= 2^-11 scale) is above 2^-89, and the scaled scale is a normal
    // number for every bf16 amax down to the smallest subnormal.  The sign is
    // copied from x afterwards, so -0 stays -0 as in the IEEE quotient, and
    // |quotient| <= 448 * (1 + 2^-8) < 464 (the saturation tie).  An infinite
    // amax (a block holding +-inf) takes the IEEE division: finite x give
    // +-0 as x/inf does.
    if (scale < __builtin_huge_valf()) {
      const float k = scale < 0x1p-64f ? 0x1p64f : 1.0f;
      const float ss = scale * k;
      float rinv = __builtin_amdgcn_rcpf(ss);
      rinv = __builtin_fmaf(__builtin_fmaf(-ss, rinv, 1.0f), rinv, rinv);
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const float xs = f[q] * k;
        const float q0 = xs * rinv;
        const float res = __builtin_fmaf(-q0, ss, xs);
        qv[q] = __builtin_copysignf(__builtin_fmaf(res, rinv, q0), f[q]);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 16; ++q) qv[q] = f[q] / scale;
    }
    // OCP E4M3 codes by the hardware conversion: nearest, ties to even, sign
    // of zero kept; it saturates to 448 up to the tie at 464 (returns NaN
    // above, which these quotients never reach).  Two codes per instruction,
    // the second pair of a word going to its upper half.
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(qv[4 * q], qv[4 * q + 1], 0, false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(qv[4 * q + 2], qv[4 * q + 3], w, true);
      out[q] = static_cast<uint32_t>(w);
    }
  }
  r.a = out;
}

// Stores the 16 bytes of chunk c of a row (16 codes, or 8 bf16 values):
// consecutive lanes write consecutive 16-byte pieces.
template <int IN>
__device__ __forceinline__ void put_codes(const Raw& r, uint8_t* row, int c, int C) {
  if (c >= C) return;
  store_nt(r.a, row + 16 * c);
}

// The wave's block scales, gathered so that one store instruction writes
// them all: lane 2v holds the scales of blocks 8v..8v+3 of the wave's range
// (chunk v's lanes 0, 8, 16, 24) and lane 2v+1 those of 8v+4..8v+7.
template <int NV>
__device__ __forceinline__ u32x4 gather_scales(const Raw (&raw)[NV], int lane) {
  u32x4 out{0, 0, 0, 0};
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    u32x4 lo, hi;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      lo[q] = __float_as_uint(__shfl(raw[v].scale, 8 * q, 64));
      hi[q] = __float_as_uint(__shfl(raw[v].scale, 32 + 8 * q, 64));
    }
    if (lane == 2 * v) out = lo;
    if (lane == 2 * v + 1) out = hi;
  }
  return out;
}

// Stores the scales of the wave's blocks [b0, b0 + 8*NV): one 16-byte store
// per 4 blocks when they all exist, else one 4-byte store per block.
template <int NV>
__device__ __forceinline__ void put_scales(const DispatchArgs& p, const Raw (&raw)[NV], u32x4 sc, uint8_t* row,
                                           int b0, int c0, int C, int lane) {
  if (b0 + 8 * NV <= (C >> 3)) {
    if (lane < 2 * NV) store_nt(sc, row + p.H + 4 * (b0 + 4 * lane));
  } else {
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int c = c0 + v * 64;
      if ((c & 7) == 0 && c < C)
        __builtin_nontemporal_store(raw[v].scale, reinterpret_cast<float*>(row + p.H + 4 * (c >> 3)));
    }
  }
}

// Waves per workgroup (every wave works on its own): 4 for HT and 2 for LL
// were the fastest of 1, 2, 4 and 8 on the 4096-token prefill and the
// 64 x 128-token decode dispatch.
constexpr int kHtWavesPerGroup = 4;
constexpr int kLlWavesPerGroup = 2;

// HT key offsets.  The first stage-2 row of each key and the first stage-1
// row of each rank are the exclusive prefix sums of the handle's per-key
// totals (c2 [E2], c1 [R]).  Every workgroup scans them into LDS itself --
// a few hundred values from L2 -- rather than wait for one workgroup of
// the count pass to publish them.  A thread holds a contiguous run of each
// array (kOffRun values at most); the runs' sums are scanned over the wave,
// then across the waves through LDS.
constexpr int kOffThreads = 64 * kHtWavesPerGroup;
constexpr int kOffRun = ((kMaxExperts > kMaxRanks ? kMaxExperts : kMaxRanks) + kOffThreads - 1) / kOffThreads;

struct KeyTotals {
  int e[kOffRun], r[kOffRun];
};

__device__ __forceinline__ void load_totals(const DispatchArgs& p, int R, KeyTotals& t) {
  const int tid = threadIdx.x;
  const int pe = (p.E2 + kOffThreads - 1) / kOffThreads, pr = (R + kOffThreads - 1) / kOffThreads;
#pragma unroll
  for (int q = 0; q < kOffRun; ++q) {
    t.e[q] = (q < pe && tid * pe + q < p.E2) ? p.c2[tid * pe + q] : 0;
    t.r[q] = (q < pr && tid * pr + q < R) ? p.c1[tid * pr + q] : 0;
  }
}

__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  return v;
}

// s_off[0, E2): stage-2 key offsets; s_off[E2, E2 + R): stage-1 rank
// offsets.  Workgroup 0 also writes them to the handle (off2, off1).  Every
// thread of the workgroup takes part (two barriers).
__device__ __forceinline__ void build_offsets(const DispatchArgs& p, int R, const KeyTotals& t, int32_t* s_off,
                                              int* s_wave) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int E2 = p.E2;
  const int pe = (E2 + kOffThreads - 1) / kOffThreads, pr = (R + kOffThreads - 1) / kOffThreads;
  int se = 0, sr = 0;
#pragma unroll
  for (int q = 0; q < kOffRun; ++q) {
    se += t.e[q];
    sr += t.r[q];
  }
  const int ie = wave_inclusive_scan(se, lane), ir = wave_inclusive_scan(sr, lane);
  if (lane == 63) {
    s_wave[w] = ie;
    s_wave[kHtWavesPerGroup + w] = ir;
  }
  __syncthreads();
  int re = ie - se, rr = ir - sr;
  for (int q = 0; q < w; ++q) {
    re += s_wave[q];
    rr += s_wave[kHtWavesPerGroup + q];
  }
#pragma unroll
  for (int q = 0; q < kOffRun; ++q) {
    if (q < pe && tid * pe + q < E2) s_off[tid * pe + q] = re;
    re += t.e[q];
    if (q < pr && tid * pr + q < R) s_off[E2 + tid * pr + q] = rr;
    rr += t.r[q];
  }
  __syncthreads();
  if (blockIdx.x == 0)
    for (int x = tid; x < E2 + R; x += kOffThreads) {
      if (x < E2) p.off2[x] = s_off[x];
      else p.off1[x - E2] = s_off[x];
    }
}

// The inputs of one token's positions, all loaded in one round trip before
// its payload: lane k < K holds entry k (expert id, in-tile rank, weight),
// lane n < N node n (in-tile rank and tile prefix), and when the tile's
// prefix row has at most kRowKeys keys every lane holds four consecutive
// ones, so that no load waits for the token's expert ids.
constexpr int kRowKeys = 256;

struct PosIn {
  int e, re, rn, hn;
  float w;
  int h[4];
};

template <bool HT, bool META>
__device__ __forceinline__ void load_pos(const DispatchArgs& p, int i, int j, int lane, bool meta, PosIn& q) {
  const int K = p.K;
  const bool lk = lane < K;
  q.e = lk ? p.topk[static_cast<int64_t>(i) * K + lane] : -1;
  q.re = lk ? p.rank_e[static_cast<int64_t>(i) * K + lane] : -1;
  q.w = (HT && META && meta && lk && p.w) ? p.w[static_cast<int64_t>(i) * K + lane] : 0.0f;
  if (p.E2 <= kRowKeys) {
    const int32_t* row = p.hist_e + static_cast<int64_t>(j) * p.E2;
#pragma unroll
    for (int c = 0; c < 4; ++c) q.h[c] = 4 * lane + c < p.E2 ? row[4 * lane + c] : 0;
  }
  if constexpr (HT) {
    const bool ln = lane < p.N;
    q.rn = ln ? p.rank_n[static_cast<int64_t>(i) * p.N + lane] : -1;
    q.hn = ln ? p.hist_n[static_cast<int64_t>(j) * p.N + lane] : 0;
  }
}

// Token gw / W's coordinates; the wave index is uniform, so these are scalar.
struct TokenAt {
  int i, part, s, t, j;
};
__device__ __forceinline__ TokenAt token_at(const DispatchArgs& p, uint32_t gw, uint32_t W) {
  TokenAt a;
  a.i = static_cast<int>(gw / W);
  a.part = static_cast<int>(gw - static_cast<uint32_t>(a.i) * W);
  a.s = static_cast<int>(static_cast<uint32_t>(a.i) / static_cast<uint32_t>(p.T));
  a.t = a.i - a.s * p.T;
  a.j = a.s * p.tps + a.t / kTile;
  return a;
}

// A token spans W waves, blockDim.x / 64 waves per workgroup; a lane owns
// chunks c = v*64 + lane, v < NV, of its wave's range (16 elements each; 8
// with a BF16 payload, a plain 16-byte copy).  Past the HT key-offset scan
// there are no barriers: everything shared inside a token is wave-uniform.
// The token's entries are worked on lane by lane (lane k: entry k, lane n:
// node n), and each row's position is read out of its lane when the row is
// written.
template <int IN, bool HT, bool PAYLOAD, int KMAX, int NV>
__global__ __launch_bounds__(256) void dispatch_kernel(DispatchArgs p, int W_) {
  extern __shared__ int32_t s_off[];   // HT: key offsets, [E2] stage-2 keys then [R] stage-1 ranks
  __shared__ int s_wave[2 * kHtWavesPerGroup];
  const int lane = threadIdx.x & 63;
  const int C = IN == 1 ? p.H / 8 : p.H / 16;   // 16-byte chunks of the payload row
  const int K = p.K, E = p.E, N = p.N;
  const uint32_t W = static_cast<uint32_t>(W_);
  // Rows end on whole 128-byte lines when the scale bytes (H/32) are whole
  // 16-byte groups, so the LL header is 16-byte aligned: H % 512 == 0.
  const bool line_tail = (p.H & 511) == 0;
  const uint32_t wpb = blockDim.x >> 6;            // waves per workgroup
  const uint32_t waves = gridDim.x * wpb;
  const uint32_t total = static_cast<uint32_t>(p.n) * W;
  const uint32_t gw0 = blockIdx.x * wpb + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool row_keys = p.E2 <= kRowKeys;
  // 1. Loads, in the order their results are needed (loads complete in
  //    order): the HT key totals, the first token's position inputs, then
  //    its payload; the workgroup scans the key offsets while the payload
  //    is in flight.
  Raw raw[NV];
  auto load_token = [&](const TokenAt& a) {
    const int c0 = a.part * NV * 64 + lane;
#pragma unroll
    for (int v = 0; v < NV; ++v) raw[v] = load_chunk<IN>(p, a.i, c0 + v * 64, c0 + v * 64 < C);
  };
  KeyTotals kt;
  if constexpr (HT) load_totals(p, N * p.G, kt);
  PosIn q;
  if (gw0 < total) {
    const TokenAt a = token_at(p, gw0, W);
    load_pos<HT, PAYLOAD>(p, a.i, a.j, lane, a.part == 0, q);
    if constexpr (PAYLOAD) load_token(a);
  }
  if constexpr (HT) build_offsets(p, N * p.G, kt, s_off, s_wave);
  for (uint32_t gw = gw0; gw < total; gw += waves) {
    const TokenAt a = token_at(p, gw, W);
    const int i = a.i, part = a.part, s = a.s, t = a.t, j = a.j;
    const int c0 = part * NV * 64 + lane;           // this lane's first chunk
    if (gw != gw0) {
      load_pos<HT, PAYLOAD>(p, i, j, lane, part == 0, q);
      if constexpr (PAYLOAD) load_token(a);
    }
    const bool meta = part == 0;                    // the token's first wave writes maps and metadata

    // 2. Entries (lane k): valid when in range and not a repeat of an
    //    earlier entry; the first valid entry on each node carries the
    //    node's stage-1 row.  Uniform copies of the entries come from
    //    their lanes.
    const int e = q.e;
    const int nd = e >= 0 ? e / p.P : -1;
    bool dup = false;
#pragma unroll
    for (int k = 0; k < KMAX - 1; ++k) {
      const int ek = __builtin_amdgcn_readlane(e, k);
      dup |= k < lane && ek == e;
    }
    const bool ok = lane < K && e >= 0 && e < E && !dup;
    const uint64_t okm = __ballot(ok);
    // Quantise as soon as the payload is in, so that the raw chunks'
    // registers are free before the positions are worked out.
    if constexpr (PAYLOAD && IN == 0) {
#pragma unroll
      for (int v = 0; v < NV; ++v) quantize(raw[v]);
    }

    // 3. Positions.  Stage 2 / LL (lane k): key offset + tile prefix +
    //    in-tile rank; an entry without a row of its own (invalid, or with
    //    the per-rank stage 2 not the token's first entry on its rank) has
    //    in-tile rank -1.  Stage 1 (lane n): the node's rank offset + tile
    //    prefix + in-tile rank, or -1 when the token does not go there.
    const bool has2 = ok && q.re >= 0;
    const int key = (HT && p.s2_rank) ? (e >= 0 ? e / p.L : 0) : e;
    int pre;
    if (row_keys) {
      // the tile prefix of `key` sits in lane key/4, element key%4
      const int src = has2 ? key >> 2 : 0;
      int hv = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int v = __shfl(q.h[c], src, 64);
        if ((key & 3) == c) hv = v;
      }
      pre = hv;
    } else {
      pre = has2 ? p.hist_e[static_cast<int64_t>(j) * p.E2 + key] : 0;
    }
    int pos = -1;
    if (has2) pos = HT ? s_off[key] + pre + q.re : (e * p.S + s) * p.slots + pre + q.re;
    int node_pos = -1, row1 = -1;
    if constexpr (HT) {
      if (lane < N && q.rn >= 0) node_pos = s_off[p.E2 + lane * p.G + s % p.G] + q.hn + q.rn;
      bool same_node = false;
#pragma unroll
      for (int k = 0; k < KMAX - 1; ++k) {
        const int nk = __builtin_amdgcn_readlane(nd, k);
        same_node |= k < lane && ((okm >> k) & 1) && nk == nd;
      }
      const int r = __shfl(node_pos, (ok && !same_node) ? nd : 0, 64);
      if (ok && !same_node) row1 = r;
    }

    // 4. The handle's maps.
    if (meta && lane < K) (HT ? p.row2 : p.slot_map)[static_cast<int64_t>(i) * K + lane] = pos;
    if (HT && meta && lane < N) p.node_row[static_cast<int64_t>(i) * N + lane] = node_pos;

    if constexpr (PAYLOAD) {
      // 5. Metadata of every row (the token's first wave).
      if (!meta) {
      } else if constexpr (HT) {
        if (row1 >= 0) {
          p.m1_tok[row1] = t;
          p.m1_src[row1] = s;
        }
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
          const int r = __builtin_amdgcn_readlane(row1, k);
          if (r >= 0 && lane < K) {
            p.m1_topk[static_cast<int64_t>(r) * K + lane] = e;
            if (p.w) p.m1_w[static_cast<int64_t>(r) * K + lane] = q.w;
          }
        }
        if (pos >= 0) {
          p.m2_src[pos] = s;
          p.m2_tok[pos] = t;
          p.m2_k[pos] = lane;
        }
        if (p.s2_rank) {
          // the token's entries on each row's rank, as local expert ids
#pragma unroll
          for (int k = 0; k < KMAX; ++k) {
            const int r = __builtin_amdgcn_readlane(pos, k);
            if (r >= 0 && lane < K) {
              const int rk = __builtin_amdgcn_readlane(key, k);
              const bool here = ok && key == rk;
              p.m2_topk[static_cast<int64_t>(r) * K + lane] = here ? e - rk * p.L : -1;
              p.m2_w[static_cast<int64_t>(r) * K + lane] = (here && p.w) ? q.w : 0.0f;
            }
          }
        }
      } else if (!line_tail && pos >= 0) {
        const i32x4 hdr{t, s, lane, 0};
        __builtin_nontemporal_store(hdr, reinterpret_cast<i32x4*>(p.ll_buf + static_cast<int64_t>(pos) * p.msg_pitch + p.row_bytes));
      }
      // 6. Gather the scales, then write each destination row with NV code
      //    stores and one scale store.
      u32x4 sc{0, 0, 0, 0};
      if constexpr (IN != 1) sc = gather_scales<NV>(raw, lane);
      const int b0 = part * NV * 8;     // first block of this wave's range
      // The row's tail, from this wave's first scale (FP8) or the end of the
      // payload (BF16) to the next 128-byte boundary: the scales, the LL
      // header, then zeros, so that no cache line of a row is written in
      // part.  The last wave of the token writes it, 16 bytes per lane.
      const bool tail_here = line_tail && part == static_cast<int>(W) - 1;
      const int tail_off = IN == 1 ? 2 * p.H : p.H + 4 * b0;
      const int tail_sc = IN == 1 ? 0 : ((C >> 3) - b0) >> 2;   // 16-byte groups of scales
      const int tail_end = static_cast<int>(((HT ? p.row_bytes : p.row_bytes + 16) + 127) & ~int64_t{127});
      const int tail_groups = (tail_end - tail_off) >> 4;
      auto put_row = [&](uint8_t* row, int k) {
#pragma unroll
        for (int v = 0; v < NV; ++v) put_codes<IN>(raw[v], row, c0 + v * 64, C);
        if (tail_here) {
          if (lane < tail_groups) {
            u32x4 v{0, 0, 0, 0};
            if (lane < tail_sc) v = sc;
            else if (!HT && lane == tail_sc) v = u32x4{static_cast<uint32_t>(t), static_cast<uint32_t>(s), static_cast<uint32_t>(k), 0u};
            store_nt(v, row + tail_off + 16 * lane);
          }
        } else if constexpr (IN != 1) {
          put_scales<NV>(p, raw, sc, row, b0, c0, C, lane);
        }
      };
      if constexpr (HT) {
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
          const int r = __builtin_amdgcn_readlane(row1, k);
          if (r >= 0) put_row(p.st1 + static_cast<int64_t>(r) * p.row_pitch, k);
        }
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
          const int r = __builtin_amdgcn_readlane(pos, k);
          if (r >= 0) put_row(p.st2 + static_cast<int64_t>(r) * p.row_pitch, k);
        }
      } else {
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
          const int r = __builtin_amdgcn_readlane(pos, k);
          if (r >= 0) put_row(p.ll_buf + static_cast<int64_t>(r) * p.msg_pitch, k);
        }
      }
    }
  }
}

// A3 on its own, for callers that keep FP8 tokens and dispatch them
// pre-quantised: the same chunk mapping and quantize() as the dispatch, so
// the codes and scales are the ones the dispatch would write.  Codes go out as 16-byte stores; each block's scale is stored by
// the first lane of its 8.
template <int NV>
__global__ __launch_bounds__(256) void quantize_kernel(QuantArgs a, int W) {
  const int lane = threadIdx.x & 63;
  const int C = a.H / 16;
  const int64_t waves = static_cast<int64_t>(gridDim.x) * 4;
  const int64_t total = a.n * W;
  for (int64_t gw = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6); gw < total; gw += waves) {
    const int64_t i = gw / W;
    const int part = static_cast<int>(gw - i * W);
    const int c0 = part * NV * 64 + lane;
    Raw raw[NV];
    const u32x4 zero{0, 0, 0, 0};
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int c = c0 + v * 64;
      const u32x4* s4 = reinterpret_cast<const u32x4*>(a.x + i * a.ld_x + 16 * c);
      raw[v].a = c < C ? s4[0] : zero;
      raw[v].b = c < C ? s4[1] : zero;
      raw[v].scale = 0.0f;
    }
#pragma unroll
    for (int v = 0; v < NV; ++v) quantize(raw[v]);
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const int c = c0 + v * 64;
      if (c >= C) continue;
      store_nt(raw[v].a, a.q + i * a.ld_q + 16 * c);
      if ((c & 7) == 0) __builtin_nontemporal_store(raw[v].scale, a.scales + i * a.ld_s + (c >> 3));
    }
  }
}

// Chunks per lane in one wave's share of a token: enough memory-level
// parallelism per wave while keeping the wave's registers low enough for
// full occupancy; a token spans W = ceil(C / (64*NV)) waves.
constexpr int kChunksPerLane = 4;

template <int IN, bool PAYLOAD, int KMAX, int NV>
void launch_nv(const DispatchArgs& p, hipStream_t stream) {
  const int C = IN == 1 ? p.H / 8 : p.H / 16;
  const int W = PAYLOAD ? (C + 64 * NV - 1) / (64 * NV) : 1;
  const int wpb = p.ht ? kHtWavesPerGroup : kLlWavesPerGroup;
  int64_t blocks = (p.n * W + wpb - 1) / wpb;
  // The CU cap counts 4-wave workgroups: smaller ones get as many waves.
  const int64_t cap = static_cast<int64_t>(p.max_blocks) * 4 / wpb;
  if (cap > 0 && blocks > cap) blocks = cap;
  if (blocks > 0x7FFFFFFF) blocks = 0x7FFFFFFF;
  const dim3 grid(static_cast<unsigned>(blocks)), block(64 * wpb);
  const size_t lds = static_cast<size_t>(p.E2 + p.N * p.G) * sizeof(int32_t);   // HT key offsets
  if (p.ht) dispatch_kernel<IN, true, PAYLOAD, KMAX, NV><<<grid, block, lds, stream>>>(p, W);
  else dispatch_kernel<IN, false, PAYLOAD, KMAX, NV><<<grid, block, 0, stream>>>(p, W);
}

template <int IN, bool PAYLOAD, int KMAX>
void launch_k(const DispatchArgs& p, hipStream_t stream) {
  if constexpr (!PAYLOAD) launch_nv<IN, PAYLOAD, KMAX, 1>(p, stream);
  else launch_nv<IN, PAYLOAD, KMAX, kChunksPerLane>(p, stream);
}

template <int IN, bool PAYLOAD>
void launch_in(const DispatchArgs& p, hipStream_t stream) {
  if (p.K <= 8) launch_k<IN, PAYLOAD, 8>(p, stream);
  else launch_k<IN, PAYLOAD, 32>(p, stream);
}

}  // namespace

hipError_t launch_quantize(const QuantArgs& a, hipStream_t stream) {
  if (a.n == 0) return hipSuccess;
  const int C = a.H / 16;
  const int W = (C + 64 * kChunksPerLane - 1) / (64 * kChunksPerLane);
  int64_t blocks = (a.n * W + 3) / 4;
  if (blocks > 0x7FFFFFFF) blocks = 0x7FFFFFFF;
  quantize_kernel<kChunksPerLane><<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream>>>(a, W);
  return hipGetLastError();
}

hipError_t launch_dispatch(const DispatchArgs& p, hipStream_t stream) {
  if (p.n == 0) return hipSuccess;
  if (!p.payload) launch_in<0, false>(p, stream);      // maps only
  else if (p.in_fp8) launch_in<2, true>(p, stream);
  else if (p.out_fp8) launch_in<0, true>(p, stream);
  else launch_in<1, true>(p, stream);
  return hipGetLastError();
}

}  // namespace ep
