// A3 + A4 / A5 + A6: quantise each token once and write its row to every
// destination the handle assigned (LL messages, HT stage-1 and stage-2 rows).
//
// Sources: "NVSHMEM and DeepEP: GPU-initiated communication" -- FP8 dispatch
// with one fp32 scale per 128 elements (7168 + 56*4 bytes per token), LL
// message = payload + scales + 16-byte header (7408 B), HT one copy per
// destination node at the same-position GPU followed by the intra-node
// forward; "NCCL EP paper notes" -- quantisation inside the send kernel's
// prepare stage, message sizes 7408 B (FP8) / 14352 B (BF16).
//
// Mapping: one workgroup per token (grid-stride when the CU cap is set);
// thread c owns elements [16c, 16c+16): two 16-byte loads of bf16, and one
// 16-byte store of FP8 codes per destination row.  A 128-element block is 8
// consecutive lanes, so its amax is a 3-step xor-shuffle inside a DPP row.
// The destination list of a token is workgroup-uniform (scalar loads).  The
// source row is read once and the quantised chunk stays in registers for all
// destinations; rows are written with non-temporal stores because nothing
// on this GPU reads them back before the next pass.
#include "ep_internal.h"

namespace ep {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// E4M3 (OCP, max 448) from fp32: nearest, ties to even, saturating, sign of
// zero kept.  Normal range: round the fp32 mantissa to 3 bits at bit 20
// (carry propagates into the exponent), then rebias 127 -> 7.  Below 2^-6
// the codes are multiples of 2^-9, i.e. rint(|v| * 512) (exact scaling).
__device__ __forceinline__ uint32_t to_e4m3(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t mag = u & 0x7FFFFFFFu;
  uint32_t code;
  if (mag >= 0x3C800000u) {  // |v| >= 2^-6
    const uint32_t r = mag + 0x7FFFFu + ((mag >> 20) & 1u);
    code = (r >> 20) - (120u << 3);
    code = code > 0x7Eu ? 0x7Eu : code;
  } else {
    code = static_cast<uint32_t>(__builtin_rintf(__uint_as_float(mag) * 512.0f));
  }
  return sign | code;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ void store_nt(u32x4 v, uint8_t* p) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// One token's chunk, ready to store: FP8 codes (16 B) or BF16 (32 B).
struct Chunk {
  u32x4 a, b;
  float scale;
};

template <int IN>  // 0: BF16 in -> FP8, 1: BF16 in -> BF16, 2: FP8 in -> FP8
__device__ __forceinline__ Chunk make_chunk(const DispatchArgs& p, int64_t i, int c, bool active) {
  Chunk ch;
  ch.scale = 0.0f;
  if constexpr (IN == 2) {
    const uint8_t* src = static_cast<const uint8_t*>(p.x) + i * p.ld_x;
    ch.a = active ? *reinterpret_cast<const u32x4*>(src + 16 * c) : u32x4{0, 0, 0, 0};
    ch.b = ch.a;
    ch.scale = active ? p.x_scales[i * p.ld_s + (c >> 3)] : 0.0f;
    return ch;
  } else {
    const uint16_t* src = static_cast<const uint16_t*>(p.x) + i * p.ld_x;
    const u32x4* s4 = reinterpret_cast<const u32x4*>(src + 16 * c);
    const u32x4 zero{0, 0, 0, 0};
    ch.a = active ? s4[0] : zero;
    ch.b = active ? s4[1] : zero;
    if constexpr (IN == 1) return ch;
    float f[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f[2 * q] = bf16_lo(ch.a[q]);
      f[2 * q + 1] = bf16_hi(ch.a[q]);
      f[8 + 2 * q] = bf16_lo(ch.b[q]);
      f[8 + 2 * q + 1] = bf16_hi(ch.b[q]);
    }
    float amax = 0.0f;
#pragma unroll
    for (int q = 0; q < 16; ++q) amax = fmaxf(amax, fabsf(f[q]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 4, 64));
    u32x4 out{0, 0, 0, 0};
    if (amax != 0.0f) {
      const float scale = amax / 448.0f;
      ch.scale = scale;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t w = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) w |= to_e4m3(f[4 * q + b] / scale) << (8 * b);
        out[q] = w;
      }
    }
    ch.a = out;
    return ch;
  }
}

template <int IN>
__device__ __forceinline__ void put_row(const DispatchArgs& p, const Chunk& ch, uint8_t* row, int c) {
  if constexpr (IN == 1) {
    store_nt(ch.a, row + 32 * c);
    store_nt(ch.b, row + 32 * c + 16);
  } else {
    store_nt(ch.a, row + 16 * c);
    if ((c & 7) == 0)
      __builtin_nontemporal_store(ch.scale, reinterpret_cast<float*>(row + p.H + 4 * (c >> 3)));
  }
}

template <int IN, bool HT>
__global__ __launch_bounds__(1024) void dispatch_kernel(DispatchArgs p) {
  const int c = threadIdx.x;
  const int C = p.H / 16;
  const bool active = c < C;
  for (int64_t i = blockIdx.x; i < p.n; i += gridDim.x) {
    const Chunk ch = make_chunk<IN>(p, i, c, active);
    const int32_t t = static_cast<int32_t>(i % p.T);
    const int32_t s = static_cast<int32_t>(i / p.T);
    if constexpr (HT) {
      for (int n = 0; n < p.N; ++n) {
        const int32_t r = p.node_row[i * p.N + n];
        if (r < 0) continue;
        if (active) put_row<IN>(p, ch, p.st1 + static_cast<int64_t>(r) * p.row_bytes, c);
        if (c == 0) {
          p.m1_tok[r] = t;
          p.m1_src[r] = s;
        }
        for (int k = c; k < p.K; k += blockDim.x) {
          p.m1_topk[static_cast<int64_t>(r) * p.K + k] = p.topk[i * p.K + k];
          if (p.w) p.m1_w[static_cast<int64_t>(r) * p.K + k] = p.w[i * p.K + k];
        }
      }
      for (int k = 0; k < p.K; ++k) {
        const int32_t r = p.row2[i * p.K + k];
        if (r < 0) continue;
        if (active) put_row<IN>(p, ch, p.st2 + static_cast<int64_t>(r) * p.row_bytes, c);
        if (c == 0) {
          p.m2_src[r] = s;
          p.m2_tok[r] = t;
          p.m2_k[r] = k;
        }
      }
    } else {
      for (int k = 0; k < p.K; ++k) {
        const int32_t slot = p.slot_map[i * p.K + k];
        if (slot < 0) continue;
        uint8_t* msg = p.ll_buf + static_cast<int64_t>(slot) * p.msg_bytes;
        if (active) put_row<IN>(p, ch, msg, c);
        if (c == 0) {
          const i32x4 hdr{t, s, k, 0};
          __builtin_nontemporal_store(hdr, reinterpret_cast<i32x4*>(msg + p.row_bytes));
        }
      }
    }
  }
}

template <int IN>
hipError_t launch_in(const DispatchArgs& p, dim3 grid, dim3 block, hipStream_t stream) {
  if (p.ht) dispatch_kernel<IN, true><<<grid, block, 0, stream>>>(p);
  else dispatch_kernel<IN, false><<<grid, block, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dispatch(const DispatchArgs& p, hipStream_t stream) {
  if (p.n == 0) return hipSuccess;
  const int C = p.H / 16;
  const int threads = ((C + 63) / 64) * 64;
  int64_t blocks = p.n;
  if (p.max_blocks > 0 && blocks > p.max_blocks) blocks = p.max_blocks;
  if (blocks > 0x7FFFFFFF) blocks = 0x7FFFFFFF;
  const dim3 grid(static_cast<unsigned>(blocks)), block(threads);
  if (p.in_fp8) return launch_in<2>(p, grid, block, stream);
  if (p.out_fp8) return launch_in<0>(p, grid, block, stream);
  return launch_in<1>(p, grid, block, stream);
}

}  // namespace ep
