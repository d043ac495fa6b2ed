// ep_layout_noalloc: the handle's maps and counts for one routing, written
// to caller buffers, with no group and no device allocation -- for callers
// that cannot allocate (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// It runs the kernels of ep_create_handle (count tiles, prefix scan) and the
// maps-only pass of the dispatch.  Their working storage -- the copy of
// topk_idx, the in-tile ranks, the tile counts and the error word -- lives in `scratch`, a fixed device array of this
// file, one copy per GPU, for the life of the process.  Host code never
// passes the array's name to a kernel: once per device, with that device
// current, hipGetSymbolAddress gives the device address, kept per device,
// and the kernels get that address.  Every call on a GPU shares that GPU's
// array, so calls that overlap on one GPU race.
#include <mutex>

#include "ep_internal.h"

namespace ep {
namespace {

constexpr size_t kScratchBytes = static_cast<size_t>(EP_NOALLOC_SCRATCH_BYTES);
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of the current device's scratch array (looked up once
// per device).
ep_status_t scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return EP_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return EP_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return EP_OK;
}

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// An I32 map output: [rows, cols] contiguous, 4-byte aligned device data.
bool map_ok(const ep_tensor_t* t, int64_t rows, int64_t cols) {
  if (!t || t->dtype != EP_DTYPE_I32 || (t->tag != EP_TAG_NONE && t->tag != EP_TAG_TOKENS_PER_EXPERT &&
                                         t->tag != EP_TAG_TOPK_IDX))
    return false;
  if (cols <= 1) {
    if (t->ndim == 1) return t->sizes[0] == rows && t->strides[0] == 1 && (rows == 0 || t->data);
    if (t->ndim != 2 || t->sizes[1] != 1) return false;
  } else if (t->ndim != 2 || t->sizes[1] != cols) {
    return false;
  }
  return t->sizes[0] == rows && t->strides[1] == 1 && t->strides[0] == t->sizes[1] && (rows == 0 || t->data);
}

}  // namespace
}  // namespace ep

using namespace ep;

EP_API ep_status_t ep_layout_noalloc(const ep_config_t* config, const ep_tensor_t* topk_idx,
                                     ep_tensor_t* const maps[8], ep_tensor_t* device_error,
                                     ep_stream_t stream) {
  if (!config || !topk_idx || !maps) return EP_ERR_INVALID_ARGUMENT;
  const ep_config_t& cfg = *config;
  Topology topo{};
  if (const ep_status_t st = check_topology(cfg, &topo); st != EP_OK) return st;
  const bool ht = cfg.mode == EP_MODE_HT;
  const int K = cfg.top_k, S = cfg.num_src_ranks, E = cfg.num_experts, N = cfg.num_nodes;
  if (!topk_idx->data && topk_idx->sizes[0] > 0) return EP_ERR_INVALID_ARGUMENT;
  if (topk_idx->dtype != EP_DTYPE_I32 || topk_idx->ndim != 2 || topk_idx->sizes[1] != K ||
      topk_idx->strides[1] != 1 || topk_idx->strides[0] != K || topk_idx->sizes[0] < 0 ||
      (topk_idx->tag != EP_TAG_NONE && topk_idx->tag != EP_TAG_TOPK_IDX))
    return EP_ERR_INVALID_ARGUMENT;
  const int64_t n = topk_idx->sizes[0];
  if (n % S != 0) return EP_ERR_INVALID_ARGUMENT;
  const int64_t T = n / S;
  if (T > cfg.max_tokens_per_rank) return EP_ERR_CAPACITY;
  // The mode's maps, each required, shaped as ep_handle_get_map reports them;
  // the other mode's entries must be NULL.
  for (int m = 0; m < 8; ++m) {
    const bool mine = ht ? m >= EP_MAP_HT_NODE_ROW : m <= EP_MAP_LL_COUNT;
    if (!mine && maps[m]) return EP_ERR_INVALID_ARGUMENT;
  }
  if (ht) {
    if (!map_ok(maps[EP_MAP_HT_NODE_ROW], n, N) || !map_ok(maps[EP_MAP_HT_ROW], n, K) ||
        !map_ok(maps[EP_MAP_HT_RANK_COUNT], topo.R, 1) || !map_ok(maps[EP_MAP_HT_RANK_OFFSET], topo.R, 1) ||
        !map_ok(maps[EP_MAP_HT_EXPERT_COUNT], topo.E2, 1) || !map_ok(maps[EP_MAP_HT_EXPERT_OFFSET], topo.E2, 1))
      return EP_ERR_INVALID_ARGUMENT;
  } else {
    if (!map_ok(maps[EP_MAP_LL_SLOT], n, K) || !map_ok(maps[EP_MAP_LL_COUNT], E, S))
      return EP_ERR_INVALID_ARGUMENT;
    if (static_cast<int64_t>(E) * S * cfg.max_tokens_per_rank > INT32_MAX) return EP_ERR_UNSUPPORTED;
  }
  if (device_error && (device_error->dtype != EP_DTYPE_I32 || device_error->ndim != 1 ||
                       device_error->sizes[0] != 1 || !device_error->data))
    return EP_ERR_INVALID_ARGUMENT;

  // Scratch: topk copy, in-tile ranks, tile counts, error word.
  const int tps = static_cast<int>((T + kLayoutTile - 1) / kLayoutTile);
  const int64_t tiles = static_cast<int64_t>(tps) * S;
  const size_t need = align_up(n * K * 4) * 2 + (ht ? align_up(n * N * 4) : 0) +
                      align_up(static_cast<size_t>(tiles) * topo.E2 * 4) +
                      (ht ? align_up(static_cast<size_t>(tiles) * N * 4) : 0) + kAlign;
  if (need > kScratchBytes) return EP_ERR_CAPACITY;

  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  void* base = nullptr;
  if (const ep_status_t st = scratch_address(&base); st != EP_OK) return st;
  uint8_t* b = static_cast<uint8_t*>(base);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    int32_t* p = reinterpret_cast<int32_t*>(b + off);
    off += align_up(bytes);
    return p;
  };
  int32_t* topk_copy = take(n * K * 4);
  int32_t* rank_e = take(n * K * 4);
  int32_t* rank_n = ht ? take(n * N * 4) : nullptr;
  int32_t* hist_e = take(static_cast<size_t>(tiles) * topo.E2 * 4);
  int32_t* hist_n = ht ? take(static_cast<size_t>(tiles) * N * 4) : nullptr;
  int32_t* err = device_error ? static_cast<int32_t*>(device_error->data) : take(4);

  auto out = [&](int m) { return static_cast<int32_t*>(maps[m]->data); };
  // The error word starts at zero (a fill kernel: no memset node, so the
  // call can be captured).
  hipError_t e = launch_fill_i32(err, 1, 0, s);
  if (e != hipSuccess) return EP_ERR_HIP;
  if (n == 0) {
    // Nothing routed: zero counts and offsets.
    if (ht) {
      for (int m : {EP_MAP_HT_RANK_COUNT, EP_MAP_HT_RANK_OFFSET})
        if ((e = launch_fill_i32(out(m), topo.R, 0, s)) != hipSuccess) return EP_ERR_HIP;
      for (int m : {EP_MAP_HT_EXPERT_COUNT, EP_MAP_HT_EXPERT_OFFSET})
        if ((e = launch_fill_i32(out(m), topo.E2, 0, s)) != hipSuccess) return EP_ERR_HIP;
    } else if ((e = launch_fill_i32(out(EP_MAP_LL_COUNT), static_cast<int64_t>(E) * S, 0, s)) != hipSuccess) {
      return EP_ERR_HIP;
    }
    return EP_OK;
  }

  LayoutArgs a{};
  a.topk = static_cast<const int32_t*>(topk_idx->data);
  a.n = n;
  a.S = S;
  a.T = static_cast<int>(T);
  a.K = K;
  a.E = E;
  a.N = N;
  a.G = cfg.ranks_per_node;
  a.P = topo.P;
  a.M = topo.M;
  a.J = topo.J;
  a.slots = cfg.max_tokens_per_rank;
  a.ht = ht;
  a.E2 = topo.E2;
  a.L = topo.L;
  a.s2_rank = topo.s2_rank;
  a.l_shift = log2_exact(topo.L);
  a.p_shift = log2_exact(topo.P);
  a.tps = tps;
  a.n_tiles = static_cast<int>(tiles);
  a.hist_e = hist_e;
  a.hist_n = hist_n;
  a.topk_copy = topk_copy;
  a.rank_e = rank_e;
  a.rank_n = rank_n;
  if (ht) {
    a.c1 = out(EP_MAP_HT_RANK_COUNT);
    a.c2 = out(EP_MAP_HT_EXPERT_COUNT);
  } else {
    a.ll_count = out(EP_MAP_LL_COUNT);
  }
  a.err = err;
  if ((e = launch_layout(a, s)) != hipSuccess) return EP_ERR_HIP;

  // The slot / row maps: the dispatch's maps-only pass.
  DispatchArgs p{};
  p.n = n;
  p.T = a.T;
  p.K = K;
  p.N = N;
  p.G = a.G;
  p.H = 128;   // no payload is written; any valid row size
  p.E = E;
  p.S = S;
  p.P = topo.P;
  p.E2 = topo.E2;
  p.L = topo.L;
  p.s2_rank = topo.s2_rank;
  p.slots = cfg.max_tokens_per_rank;
  p.tps = tps;
  p.ht = ht;
  p.payload = 0;
  p.topk = topk_copy;
  p.rank_e = rank_e;
  p.rank_n = rank_n;
  p.hist_e = hist_e;
  p.hist_n = hist_n;
  if (ht) {
    p.c1 = a.c1;
    p.c2 = a.c2;
    p.off1 = out(EP_MAP_HT_RANK_OFFSET);
    p.off2 = out(EP_MAP_HT_EXPERT_OFFSET);
    p.row2 = out(EP_MAP_HT_ROW);
    p.node_row = out(EP_MAP_HT_NODE_ROW);
  } else {
    p.slot_map = out(EP_MAP_LL_SLOT);
  }
  if ((e = launch_dispatch(p, s)) != hipSuccess) return EP_ERR_HIP;
  return EP_OK;
}
