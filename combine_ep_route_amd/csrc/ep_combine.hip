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
        wk[b] = k < a.K ? a.w[i * a.K + k] : 0.0f;
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
  if (a.K <= 8) combine_kernel<8><<<grid, block, 0, stream>>>(a);
  else combine_kernel<8><<<grid, block, 0, stream>>>(a);
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
