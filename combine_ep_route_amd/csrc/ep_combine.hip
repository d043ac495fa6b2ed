// A7: weighted top-k gather-reduce back to the original token order, and the
// identity expert used by round-trip checks.
//
// Sources: "NVSHMEM and DeepEP: GPU-initiated communication" (combine
// returns the weighted sum of expert outputs in BF16); "NCCL EP paper notes"
// (combine gathers and reduces back to the original order with the routing
// state kept in the handle; combine message 14336 B at hidden 7168).
//
//   out[i][h] = bf16_rne( fma(w[i][K-1], y[K-1], ... fma(w[i][0], y[0], +0)) )
//
// Mapping: grid (column blocks, tokens); the token index comes from
// blockIdx.y, so its K row indices and weights are scalar loads.  Thread c
// owns 8 bf16 (16 bytes) of the row; it issues the K gathered 16-byte loads
// (non-temporal: every expert-output row is read exactly once) before the
// first multiply-add so that K loads per lane are in flight, then runs the
// fp32 fma chain in k order and stores 16 bytes of bf16 (non-temporal too:
// the output is not read again by this kernel, and streaming stores keep the
// L2 for the gathered lines).
#include "ep_internal.h"

namespace ep {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// fp32 -> bf16, round to nearest even (finite inputs): add 0x7FFF plus the
// lowest kept bit, keep the high half.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return bf16_rne(lo) | (bf16_rne(hi) << 16);
}

template <int KB>  // entries gathered per batch
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int C = a.H / 8;
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  const bool active = c < C;
  for (int64_t i = blockIdx.y; i < a.n; i += gridDim.y) {
    float acc[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
    for (int k0 = 0; k0 < a.K; k0 += KB) {
      u32x4 v[KB];
      float wk[KB];
      bool ok[KB];
#pragma unroll
      for (int b = 0; b < KB; ++b) {
        const int k = k0 + b;
        const int32_t r = k < a.K ? a.loc[i * a.K + k] : -1;
        ok[b] = r >= 0 && r < a.rows;
        wk[b] = k < a.K ? (a.w ? a.w[i * a.K + k] : 1.0f) : 0.0f;   // no weights: unit weights
        if (r >= a.rows && c == 0) atomicOr(a.err, EP_DEVERR_ROW_RANGE);
        // each expert-output row is read exactly once: stream it past the caches
        v[b] = (ok[b] && active)
                   ? __builtin_nontemporal_load(
                         reinterpret_cast<const u32x4*>(a.y + static_cast<int64_t>(r) * a.ld_y + 8 * c))
                   : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int b = 0; b < KB; ++b) {
        if (!ok[b]) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] = __builtin_fmaf(wk[b], __uint_as_float(v[b][q] << 16), acc[2 * q]);
          acc[2 * q + 1] = __builtin_fmaf(wk[b], __uint_as_float(v[b][q] & 0xFFFF0000u), acc[2 * q + 1]);
        }
      }
    }
    if (active) {
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
      __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(a.out + i * a.ld_out + 8 * c));
    }
  }
}

// Backward of the combine, reusing the forward handle's row map.  One
// workgroup per token (grid-stride); thread c owns chunks c, c + B, ... of 8
// bf16 of the row.  For every valid entry k of the token:
//   dY[loc(t,k)] chunk = bf16_rne(w[t,k] * g chunk)   (one fp32 multiply)
//   dw[t,k] = sum over the row of g * Y[loc(t,k)]     (per-thread fp32 fma
//             chains, then a fixed-order shuffle/LDS tree: deterministic)
// The gradient chunk is loaded once and serves all K entries; the chunk's K
// expert-row loads are all issued before its first row-gradient store (the
// compiler may not move a load above a store it cannot prove disjoint).
// Expert rows and row gradients stream past the caches (non-temporal).
template <int KMAX>
__global__ __launch_bounds__(KMAX <= 8 ? 1024 : 256) void combine_backward_kernel(CombineBwdArgs a) {
  __shared__ float red[KMAX][16];
  const int C = a.H / 8;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwave = blockDim.x >> 6;
  for (int64_t i = blockIdx.x; i < a.n; i += gridDim.x) {
    int32_t r[KMAX];
    float wk[KMAX], dot[KMAX];
    bool ok[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      r[k] = k < a.K ? a.loc[i * a.K + k] : -1;
      ok[k] = r[k] >= 0 && r[k] < a.rows;
      if (k < a.K && r[k] >= a.rows && threadIdx.x == 0) atomicOr(a.err, EP_DEVERR_ROW_RANGE);
      wk[k] = k < a.K ? a.w[i * a.K + k] : 0.0f;
      dot[k] = 0.0f;
    }
    for (int c = threadIdx.x; c < C; c += blockDim.x) {
      const u32x4 gv = *reinterpret_cast<const u32x4*>(a.g + i * a.ld_g + 8 * c);
      float gf[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        gf[2 * q] = __uint_as_float(gv[q] << 16);
        gf[2 * q + 1] = __uint_as_float(gv[q] & 0xFFFF0000u);
      }
      // every expert-row load is issued before the first row-gradient store
      u32x4 yv[KMAX];
      if (a.y) {
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
          yv[k] = ok[k] ? __builtin_nontemporal_load(
                              reinterpret_cast<const u32x4*>(a.y + static_cast<int64_t>(r[k]) * a.ld_y + 8 * c))
                        : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int k = 0; k < KMAX; ++k) {
        if (!ok[k]) continue;
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(wk[k] * gf[2 * q], wk[k] * gf[2 * q + 1]);
        __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(a.dy + static_cast<int64_t>(r[k]) * a.ld_dy + 8 * c));
        if (a.y) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            dot[k] = __builtin_fmaf(gf[2 * q], __uint_as_float(yv[k][q] << 16), dot[k]);
            dot[k] = __builtin_fmaf(gf[2 * q + 1], __uint_as_float(yv[k][q] & 0xFFFF0000u), dot[k]);
          }
        }
      }
    }
    if (a.dw) {
#pragma unroll
      for (int k = 0; k < KMAX; ++k) {
        if (k < a.K) {
          float v = dot[k];
#pragma unroll
          for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
          if (lane == 0) red[k][wave] = v;
        }
      }
      __syncthreads();
      if (threadIdx.x < a.K) {
        float sum = 0.0f;
        for (int q = 0; q < nwave; ++q) sum += red[threadIdx.x][q];
        bool valid = false;
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
          if (k == static_cast<int>(threadIdx.x)) valid = ok[k];
        a.dw[i * a.K + threadIdx.x] = valid ? sum : 0.0f;
      }
      __syncthreads();
    }
  }
}

// Identity expert: FP8 row -> bf16(decode(q) * scale); BF16 row -> copy.
__device__ __forceinline__ float from_e4m3(uint32_t q) {
  const uint32_t e = (q >> 3) & 15u, m = q & 7u;
  const float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20))
                    : static_cast<float>(m) * 0.001953125f;  // m * 2^-9
  return __uint_as_float(__float_as_uint(v) | ((q & 0x80u) << 24));
}

__global__ __launch_bounds__(1024) void dequant_kernel(DequantArgs a) {
  const int c = threadIdx.x;   // 16 elements per thread
  if (c >= a.H / 16) return;
  for (int64_t r = blockIdx.x; r < a.n; r += gridDim.x) {
    const uint8_t* row = a.rows + r * a.row_stride;
    uint16_t* y = a.y + r * a.ld_y + 16 * c;
    if (!a.fp8) {
      const u32x4* s = reinterpret_cast<const u32x4*>(row + 32 * c);
      reinterpret_cast<u32x4*>(y)[0] = s[0];
      reinterpret_cast<u32x4*>(y)[1] = s[1];
      continue;
    }
    const u32x4 q = *reinterpret_cast<const u32x4*>(row + 16 * c);
    const float scale = *reinterpret_cast<const float*>(row + a.H + 4 * (c >> 3));
    u32x4 o0, o1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t w = q[j];
      const uint32_t lo = pack_bf16x2(from_e4m3(w & 0xFF) * scale, from_e4m3((w >> 8) & 0xFF) * scale);
      const uint32_t hi = pack_bf16x2(from_e4m3((w >> 16) & 0xFF) * scale, from_e4m3(w >> 24) * scale);
      if (j < 2) { o0[2 * j] = lo; o0[2 * j + 1] = hi; }
      else { o1[2 * (j - 2)] = lo; o1[2 * (j - 2) + 1] = hi; }
    }
    reinterpret_cast<u32x4*>(y)[0] = o0;
    reinterpret_cast<u32x4*>(y)[1] = o1;
  }
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  if (a.n == 0) return hipSuccess;
  const int C = a.H / 8;
  int threads = 64;
  for (int cand : {256, 192, 128, 64})
    if (C % cand == 0) { threads = cand; break; }
  if (C < threads) threads = ((C + 63) / 64) * 64;
  const int col_blocks = (C + threads - 1) / threads;
  int64_t rows = a.n;
  if (a.max_blocks > 0) {
    const int64_t cap = a.max_blocks / col_blocks > 0 ? a.max_blocks / col_blocks : 1;
    if (rows > cap) rows = cap;
  }
  if (rows > 65535) rows = 65535;
  const dim3 grid(col_blocks, static_cast<unsigned>(rows)), block(threads);
  // Batches of 8 entries: K <= 8 is one batch, larger K loops over batches.
  combine_kernel<8><<<grid, block, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_combine_backward(const CombineBwdArgs& a, hipStream_t stream) {
  if (a.n == 0) return hipSuccess;
  const int C = a.H / 8;
  // Whole chunks per thread where H allows.  With K <= 8, up to 7 waves per
  // token (hidden 7168: two chunks per thread, 189 us against 207 us with 2
  // waves x 7 chunks at 4096 tokens); with more entries the K preloaded rows
  // take the registers, so at most 4 waves.
  int threads = 256;
  if (a.K <= 8) {
    for (int cand : {448, 384, 320, 256, 192, 128})
      if (C % cand == 0) { threads = cand; break; }
  } else {
    for (int cand : {256, 192, 128})
      if (C % cand == 0) { threads = cand; break; }
  }
  if (C < threads) threads = ((C + 63) / 64) * 64;
  int64_t blocks = a.n;
  if (a.max_blocks > 0 && blocks > a.max_blocks) blocks = a.max_blocks;
  if (blocks > 0x7FFFFFFF) blocks = 0x7FFFFFFF;
  const dim3 grid(static_cast<unsigned>(blocks)), block(threads);
  if (a.K <= 8) combine_backward_kernel<8><<<grid, block, 0, stream>>>(a);
  else combine_backward_kernel<32><<<grid, block, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_dequant(const DequantArgs& a, hipStream_t stream) {
  if (a.n == 0) return hipSuccess;
  const int C = a.H / 16;
  const int threads = ((C + 63) / 64) * 64;
  int64_t blocks = a.n > 0x7FFFFFFF ? 0x7FFFFFFF : a.n;
  dequant_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(threads), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace ep
