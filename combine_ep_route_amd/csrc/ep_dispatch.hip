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
//  1. The token's payload loads are issued first (16-byte loads).
//  2. A 128-element block is 8 consecutive lanes; its amax is a 3-step
//     xor-shuffle inside a DPP row.  scale = amax/448 (IEEE fp32 division)
//     and q = E4M3(x/scale), the quotient by a refined reciprocal and one
//     fused residual correction, on operands pre-scaled by 2^64 when the
//     scale is tiny (the tests compare the codes with the IEEE quotient's
//     for every finite bf16 amax).  Quantising comes before
//     the positions, so the raw chunks' registers are free early.
//  3. The token's rank inside its tile (from the handle) plus the tile's
//     prefix (plus, in HT, the key's first row from LDS) gives every
//     slot / row.
//     Positions are wave-uniform.
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

// Validity of the K entries of one token row: in range and not a repeat.
template <int KMAX>
__device__ __forceinline__ void entries(const int32_t* row, int K, int E, bool present, int (&e)[KMAX],
                                        bool (&ok)[KMAX]) {
#pragma unroll
  for (int k = 0; k < KMAX; ++k) e[k] = (present && k < K) ? row[k] : -1;
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    bool dup = false;
#pragma unroll
    for (int j = 0; j < k; ++j) dup |= e[j] == e[k];
    ok[k] = present && k < K && e[k] >= 0 && e[k] < E && !dup;
  }
}

// A token spans W waves, blockDim.x / 64 waves per workgroup; a lane owns
// chunks c = v*64 + lane, v < NV, of its wave's range (16 elements each; 8
// with a BF16 payload, a plain 16-byte copy).  Past the HT key-offset scan
// there are no barriers: everything shared inside a token is wave-uniform.
template <int IN, bool HT, bool PAYLOAD, int KMAX, int NV>
__global__ __launch_bounds__(256) void dispatch_kernel(DispatchArgs p, int W) {
  extern __shared__ int32_t s_off[];   // HT: key offsets, [E2] stage-2 keys then [R] stage-1 ranks
  __shared__ int s_wave[2 * kHtWavesPerGroup];
  const int lane = threadIdx.x & 63;
  const int C = IN == 1 ? p.H / 8 : p.H / 16;   // 16-byte chunks of the payload row
  const int K = p.K, E = p.E, N = p.N;
  // Rows end on whole 128-byte lines when the scale bytes (H/32) are whole
  // 16-byte groups, so the LL header is 16-byte aligned: H % 512 == 0.
  const bool line_tail = (p.H & 511) == 0;
  const int wpb = blockDim.x >> 6;                 // waves per workgroup
  const int64_t waves = static_cast<int64_t>(gridDim.x) * wpb;
  const int64_t total = p.n * W;
  const int64_t gw0 = static_cast<int64_t>(blockIdx.x) * wpb + (threadIdx.x >> 6);
  // 1. Payload loads first, so they are in flight during the ranking.  The
  //    first token's go out before the workgroup scans the HT key offsets,
  //    whose own loads go out before them (loads complete in order, so the
  //    scan waits for those alone).
  Raw raw[NV];
  auto load_token = [&](int64_t gw) {
    const int64_t i = gw / W;
    const int c0 = static_cast<int>(gw - i * W) * NV * 64 + lane;
#pragma unroll
    for (int v = 0; v < NV; ++v) raw[v] = load_chunk<IN>(p, i, c0 + v * 64, c0 + v * 64 < C);
  };
  KeyTotals kt;
  if constexpr (HT) load_totals(p, N * p.G, kt);
  if constexpr (PAYLOAD)
    if (gw0 < total) load_token(gw0);
  if constexpr (HT) build_offsets(p, N * p.G, kt, s_off, s_wave);
  for (int64_t gw = gw0; gw < total; gw += waves) {
    const int64_t i = gw / W;                       // token
    const int part = static_cast<int>(gw - i * W);  // which chunk range of it
    const int c0 = part * NV * 64 + lane;           // this lane's first chunk
    if constexpr (PAYLOAD)
      if (gw != gw0) load_token(gw);
    const int s = static_cast<int>(i / p.T);
    const int t = static_cast<int>(i - static_cast<int64_t>(s) * p.T);
    const int j = s * p.tps + t / kTile;   // tile of this token

    // 2. This token's entries (uniform) plus the handle's in-tile ranks and
    //    tile prefixes give every slot / row (wave-uniform scalar loads).
    int me[KMAX];
    bool mok[KMAX];
    entries<KMAX>(p.topk + i * K, K, E, true, me, mok);
    // Quantise as soon as the payload is in, so that the raw chunks'
    // registers are free before the positions are worked out (3 us less per
    // 4096 tokens than quantising after them).
    if constexpr (PAYLOAD && IN == 0) {
#pragma unroll
      for (int v = 0; v < NV; ++v) quantize(raw[v]);
    }
    uint64_t my_nodes = 0;
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
      if (mok[k]) my_nodes |= 1ull << (me[k] / p.P);
    // An entry without a stage-2 row of its own (invalid, or with the
    // per-rank stage 2 not the token's first entry on its rank) has rank -1.
    int pos[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      pos[k] = -1;
      if (mok[k] && k < K) {
        const int re = p.rank_e[i * K + k];
        if (re >= 0) {
          const int key = (HT && p.s2_rank) ? me[k] / p.L : me[k];
          const int pre = p.hist_e[static_cast<int64_t>(j) * p.E2 + key] + re;
          pos[k] = HT ? s_off[key] + pre : (me[k] * p.S + s) * p.slots + pre;
        }
      }
    }
    // Stage-1 row of destination node n (uniform), or -1.
    auto node_pos = [&](int n) -> int {
      if (!((my_nodes >> n) & 1)) return -1;
      return s_off[p.E2 + n * p.G + s % p.G] + p.hist_n[static_cast<int64_t>(j) * N + n] + p.rank_n[i * N + n];
    };

    // 3. The handle's maps (written by the token's first wave).
    if (part == 0 && lane < K) {
      int v = -1;
#pragma unroll
      for (int k = 0; k < KMAX; ++k)
        if (k == lane) v = pos[k];
      (HT ? p.row2 : p.slot_map)[i * K + lane] = v;
    }
    if (HT && part == 0) {
      for (int n = 0; n < N; ++n) {
        const int r = node_pos(n);
        if (lane == (n & 63)) p.node_row[i * N + n] = r;
      }
    }

    if constexpr (PAYLOAD) {
      // 4. Stage-1 destinations as a per-entry list: entry k carries the row
      //    of its node if it is the token's first entry on that node.
      int row1[KMAX];
#pragma unroll
      for (int k = 0; k < KMAX; ++k) {
        row1[k] = -1;
        if (HT && mok[k]) {
          const int nk = me[k] / p.P;
          bool first = true;
#pragma unroll
          for (int q = 0; q < k; ++q) first &= !(mok[q] && me[q] / p.P == nk);
          if (first) row1[k] = node_pos(nk);
        }
      }
      // 5. Metadata of every row (the token's first wave).
      if (part != 0) {
      } else if constexpr (HT) {
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
          const int32_t r = row1[k];
          if (r < 0) continue;
          if (lane == 0) {
            p.m1_tok[r] = t;
            p.m1_src[r] = s;
          }
          if (lane < K) {
            int ev = -1;
#pragma unroll
            for (int q = 0; q < KMAX; ++q)
              if (q == lane) ev = me[q];
            p.m1_topk[static_cast<int64_t>(r) * K + lane] = ev;
            if (p.w) p.m1_w[static_cast<int64_t>(r) * K + lane] = p.w[i * K + lane];
          }
        }
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
          const int32_t r = pos[k];
          if (r >= 0 && lane == 0) {
            p.m2_src[r] = s;
            p.m2_tok[r] = t;
            p.m2_k[r] = k;
          }
          if (p.s2_rank && r >= 0 && lane < K) {
            // the token's entries on this row's rank, as local expert ids
            const int rk = me[k] / p.L;
            int ev = -1;
            bool okv = false;
#pragma unroll
            for (int q = 0; q < KMAX; ++q)
              if (q == lane) { ev = me[q]; okv = mok[q]; }
            const bool here = okv && ev / p.L == rk;
            p.m2_topk[static_cast<int64_t>(r) * K + lane] = here ? ev - rk * p.L : -1;
            p.m2_w[static_cast<int64_t>(r) * K + lane] = (here && p.w) ? p.w[i * K + lane] : 0.0f;
          }
        }
      } else if (!line_tail) {
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
          const int32_t slot = pos[k];
          if (slot >= 0 && lane == 0) {
            const i32x4 hdr{t, s, k, 0};
            __builtin_nontemporal_store(hdr, reinterpret_cast<i32x4*>(p.ll_buf + static_cast<int64_t>(slot) * p.msg_pitch + p.row_bytes));
          }
        }
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
      const bool tail_here = line_tail && part == W - 1;
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
        for (int k = 0; k < KMAX; ++k)
          if (row1[k] >= 0) put_row(p.st1 + static_cast<int64_t>(row1[k]) * p.row_pitch, k);
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
          if (pos[k] >= 0) put_row(p.st2 + static_cast<int64_t>(pos[k]) * p.row_pitch, k);
      } else {
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
          if (pos[k] >= 0) put_row(p.ll_buf + static_cast<int64_t>(pos[k]) * p.msg_pitch, k);
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
