// Host runtime of libep: groups, handles, argument validation and launches.
//
// Resource model after NCCL-EP ("NCCL EP paper notes": two-level resource
// management -- a group holds the mode and the communication buffers for the
// model's lifetime, a handle holds one forward pass's routing state; custom
// alloc_fn/free_fn hooks; stream-ordered asynchronous operations).  The
// principle that buffers are allocated and registered once, outside the hot
// path, is kept strictly: only ep_create_group allocates device memory.
//
// Every entry point validates its arguments before touching HIP.  When
// allocator hooks are given, group creation makes no HIP call at all: the
// device is first touched at the first enqueued operation.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "ep_internal.h"

namespace ep {
namespace {

thread_local int g_last_hip = 0;

ep_status_t from_hip(hipError_t e) {
  if (e == hipSuccess) return EP_OK;
  g_last_hip = static_cast<int>(e);
  return e == hipErrorOutOfMemory ? EP_ERR_OUT_OF_MEMORY : EP_ERR_HIP;
}

#define EP_HIP(call)                          \
  do {                                        \
    const hipError_t e__ = (call);            \
    if (e__ != hipSuccess) return from_hip(e__); \
  } while (0)

int log_level() {
  static int lvl = [] {
    const char* s = std::getenv("EP_LOG");
    return s ? std::atoi(s) : 0;
  }();
  return lvl;
}

inline hipStream_t as_stream(ep_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

// One line per counted call with EP_LOG=2.
void trace(const Group* g, const char* what, int64_t tokens) {
  if (log_level() < 2) return;
  std::fprintf(stderr, "[ep] %s %s tokens=%lld K=%d H=%d\n", what, g->cfg.mode == EP_MODE_LL ? "LL" : "HT",
               static_cast<long long>(tokens), g->cfg.top_k, g->cfg.hidden);
}

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// ---------------------------------------------------------------------------
// Allocation
// ---------------------------------------------------------------------------

void* dev_alloc(Group* g, size_t bytes, ep_status_t* st) {
  bytes = align_up(bytes == 0 ? 1 : bytes);
  void* p = nullptr;
  if (g->cfg.alloc_fn) {
    p = g->cfg.alloc_fn(bytes, g->cfg.alloc_ctx);
    if (!p) { *st = EP_ERR_OUT_OF_MEMORY; return nullptr; }
  } else {
    const hipError_t e = hipMalloc(&p, bytes);
    if (e != hipSuccess) { *st = from_hip(e); return nullptr; }
  }
  g->allocs.push_back({p, bytes});
  g->bytes += static_cast<int64_t>(bytes);
  return p;
}

void free_all(Group* g) {
  for (auto it = g->allocs.rbegin(); it != g->allocs.rend(); ++it) {
    if (g->cfg.free_fn) g->cfg.free_fn(it->ptr, g->cfg.alloc_ctx);
    else (void)hipFree(it->ptr);
  }
  g->allocs.clear();
  g->bytes = 0;
}

// Sub-allocator over one block.
struct Carve {
  uint8_t* base;
  size_t off = 0;
  template <class T> T* take(size_t count) {
    T* p = reinterpret_cast<T*>(base + off);
    off += align_up(count * sizeof(T));
    return p;
  }
};

// ---------------------------------------------------------------------------
// Validation helpers
// ---------------------------------------------------------------------------

bool group_ok(const Group* g) { return g && g->magic == kGroupMagic; }
bool handle_ok(const Handle* h) { return h && h->magic == kHandleMagic && h->in_use && group_ok(h->g); }

int64_t dtype_size(int32_t dt) {
  switch (dt) {
    case EP_DTYPE_F32: case EP_DTYPE_I32: return 4;
    case EP_DTYPE_BF16: case EP_DTYPE_F16: return 2;
    case EP_DTYPE_FP8_E4M3: case EP_DTYPE_U8: return 1;
    default: return 0;
  }
}

// A 2-D tensor [rows, cols] of the given dtype whose inner dimension is
// contiguous; rows >= 0.  Optional exact rows/cols (-1 = any), minimum row
// stride = cols, optional tag check (EP_TAG_NONE always accepted).
bool check2d(const ep_tensor_t* t, int32_t dtype, int64_t rows, int64_t cols, int32_t tag,
             bool need_align16) {
  if (!t || t->dtype != dtype || t->ndim != 2) return false;
  if (t->tag != EP_TAG_NONE && t->tag != tag) return false;
  if (rows >= 0 && t->sizes[0] != rows) return false;
  if (cols >= 0 && t->sizes[1] != cols) return false;
  if (t->sizes[0] < 0 || t->sizes[1] <= 0) return false;
  if (t->strides[1] != 1 || t->strides[0] < t->sizes[1]) return false;
  if (t->sizes[0] > 0 && !t->data) return false;
  if (need_align16) {
    const int64_t es = dtype_size(dtype);
    if ((reinterpret_cast<uintptr_t>(t->data) & 15u) != 0) return false;
    if (t->sizes[0] > 1 && ((t->strides[0] * es) & 15) != 0) return false;
  }
  return true;
}

bool contiguous2d(const ep_tensor_t* t) { return t->strides[0] == t->sizes[1]; }

ep_status_t ensure_device(Group* g, hipStream_t stream) {
  if (g->dev_ready) return EP_OK;
  EP_HIP(hipGetDevice(&g->device));
  EP_HIP(hipDeviceGetAttribute(&g->num_cu, hipDeviceAttributeMultiprocessorCount, g->device));
  EP_HIP(launch_fill_i32(g->err, 1, 0, stream));   // the error word
  g->dev_ready = true;
  return EP_OK;
}

void fill_view(ep_tensor_t* v, void* data, int32_t dtype, int64_t d0, int64_t d1, int32_t tag,
               int64_t row_stride = 0) {
  std::memset(v, 0, sizeof(*v));
  v->data = data;
  v->dtype = dtype;
  v->tag = tag;
  if (d1 <= 0) {
    v->ndim = 1;
    v->sizes[0] = d0;
    v->strides[0] = 1;
  } else {
    v->ndim = 2;
    v->sizes[0] = d0;
    v->sizes[1] = d1;
    v->strides[0] = row_stride > 0 ? row_stride : d1;
    v->strides[1] = 1;
  }
}

int dispatch_block_cap(const Group* g) {
  // No cap by default; with a CU cap, four 4-wave workgroups per allowed CU.
  return g->cfg.num_cus > 0 ? g->cfg.num_cus * 4 : 0;
}

// The handle-dependent part of a dispatch launch.
DispatchArgs dispatch_base(const Handle* h) {
  const Group* g = h->g;
  DispatchArgs p{};
  p.n = h->n;
  p.T = h->T;
  p.K = g->cfg.top_k;
  p.N = g->cfg.num_nodes;
  p.G = g->cfg.ranks_per_node;
  p.H = g->cfg.hidden;
  p.E = g->cfg.num_experts;
  p.S = g->cfg.num_src_ranks;
  p.P = g->P;
  p.E2 = g->E2;
  p.L = g->L;
  p.s2_rank = g->s2_rank;
  p.slots = g->cfg.max_tokens_per_rank;
  p.tps = h->tps;
  p.row_bytes = g->row_bytes;
  p.msg_bytes = g->msg_bytes;
  p.row_pitch = g->row_pitch;
  p.msg_pitch = g->msg_pitch;
  p.ht = g->cfg.mode == EP_MODE_HT;
  p.num_cu = g->cfg.num_cus > 0 ? g->cfg.num_cus : g->num_cu;
  p.max_blocks = 0;
  p.topk = h->topk;
  p.rank_e = h->rank_e;
  p.rank_n = h->rank_n;
  p.hist_e = h->hist_e;
  p.hist_n = h->hist_n;
  p.c1 = h->c1;
  p.c2 = h->c2;
  p.off1 = h->off1;
  p.off2 = h->off2;
  p.slot_map = h->slot_map;
  p.row2 = h->row2;
  p.node_row = h->node_row;
  return p;
}

// An expert-row tensor (expert outputs or their gradients) as 2-D BF16 rows
// [rows, H]: given as [rows, H], or in LL as [E, S*T_max, H] with a dense
// middle dimension.  Rows 16-byte aligned, innermost contiguous.
bool expert_rows(const Group* g, const ep_tensor_t* t, ep_tensor_t* out) {
  if (!t) return false;
  *out = *t;
  if (t->ndim == 3) {
    if (g->cfg.mode != EP_MODE_LL) return false;
    const int64_t per_e = static_cast<int64_t>(g->cfg.num_src_ranks) * g->cfg.max_tokens_per_rank;
    if (t->sizes[0] != g->cfg.num_experts || t->sizes[1] != per_e || t->strides[2] != 1 ||
        t->strides[0] != t->strides[1] * per_e)
      return false;
    out->ndim = 2;
    out->sizes[0] = t->sizes[0] * per_e;
    out->sizes[1] = t->sizes[2];
    out->strides[0] = t->strides[1];
    out->strides[1] = 1;
  }
  return check2d(out, EP_DTYPE_BF16, -1, g->cfg.hidden, EP_TAG_TOKENS, true);
}

// Make sure the slot / row maps and the HT key offsets exist (dispatch
// writes them; without a dispatch, a maps-only pass computes them).
ep_status_t ensure_maps(Handle* h, hipStream_t stream) {
  if (h->maps_ready) return EP_OK;
  DispatchArgs p = dispatch_base(h);
  p.payload = 0;
  p.max_blocks = 0;
  const ep_status_t st = from_hip(launch_dispatch(p, stream));
  if (st == EP_OK) h->maps_ready = true;
  return st;
}

// Copies `count` device int32 values to the group's pinned host buffer on
// the handle's stream and waits for that stream (the blocking count
// queries).  Returns the host copy through *out.
ep_status_t read_counts(Handle* h, const int32_t* src, size_t count, const int32_t** out) {
  Group* g = h->g;
  if (g->host_counts_len < count) {
    if (g->host_counts) EP_HIP(hipHostFree(g->host_counts));
    g->host_counts = nullptr;
    g->host_counts_len = 0;
    void* p = nullptr;
    EP_HIP(hipHostMalloc(&p, count * sizeof(int32_t), hipHostMallocDefault));
    g->host_counts = static_cast<int32_t*>(p);
    g->host_counts_len = count;
  }
  EP_HIP(hipMemcpyAsync(g->host_counts, src, count * sizeof(int32_t), hipMemcpyDeviceToHost, h->stream));
  EP_HIP(hipStreamSynchronize(h->stream));
  *out = g->host_counts;
  return EP_OK;
}

}  // namespace
}  // namespace ep

using namespace ep;

// ===========================================================================
// Groups
// ===========================================================================

namespace ep {

ep_status_t check_topology(const ep_config_t& cfg, Topology* t) {
  if (cfg.mode != EP_MODE_LL && cfg.mode != EP_MODE_HT) return EP_ERR_INVALID_ARGUMENT;
  if (cfg.num_nodes <= 0 || cfg.ranks_per_node <= 0 || cfg.num_experts <= 0 || cfg.top_k <= 0 ||
      cfg.max_tokens_per_rank <= 0 || cfg.num_src_ranks <= 0 || cfg.max_nodes_per_token < 0 ||
      (cfg.ht_stage2 != EP_HT_STAGE2_PER_EXPERT && cfg.ht_stage2 != EP_HT_STAGE2_PER_RANK))
    return EP_ERR_INVALID_ARGUMENT;
  const int64_t R = static_cast<int64_t>(cfg.num_nodes) * cfg.ranks_per_node;
  if (cfg.num_experts % R != 0) return EP_ERR_INVALID_ARGUMENT;
  if (cfg.top_k > cfg.num_experts) return EP_ERR_INVALID_ARGUMENT;
  const int N = cfg.num_nodes, K = cfg.top_k, E = cfg.num_experts;
  const int P = E / N;
  int M = cfg.max_nodes_per_token;
  if (M >= N) M = 0;
  const int J = M > 0 ? (K + M - 1) / M : 0;
  if (M > 0 && (J > P || static_cast<int64_t>(M) * P < K)) return EP_ERR_INVALID_ARGUMENT;
  if (cfg.num_src_ranks > R) return EP_ERR_UNSUPPORTED;
  if (E > kMaxExperts || K > kMaxTopK || N > kMaxNodes || R > kMaxRanks) return EP_ERR_UNSUPPORTED;
  t->R = static_cast<int>(R);
  t->L = E / t->R;
  t->P = P;
  t->M = M;
  t->J = J;
  t->s2_rank = cfg.mode == EP_MODE_HT && cfg.ht_stage2 == EP_HT_STAGE2_PER_RANK;
  t->E2 = t->s2_rank ? t->R : E;
  return EP_OK;
}

}  // namespace ep

EP_API ep_status_t ep_create_group(const ep_config_t* cfg_in, ep_stream_t stream, ep_group_t* out) {
  if (!cfg_in || !out) return EP_ERR_INVALID_ARGUMENT;
  *out = nullptr;
  ep_config_t cfg = *cfg_in;
  Topology topo{};
  if (const ep_status_t st = check_topology(cfg, &topo); st != EP_OK) return st;
  if (cfg.hidden <= 0 || cfg.max_handles < 0 || cfg.num_cus < 0 || cfg.ll_buffers < 0 || cfg.ll_buffers > 2 ||
      cfg.ht_buffers < 0 || cfg.ht_buffers > 2)
    return EP_ERR_INVALID_ARGUMENT;
  if (cfg.payload != EP_DTYPE_FP8_E4M3 && cfg.payload != EP_DTYPE_BF16) return EP_ERR_INVALID_ARGUMENT;
  if (cfg.payload == EP_DTYPE_FP8_E4M3 && cfg.hidden % 128 != 0) return EP_ERR_INVALID_ARGUMENT;
  if (cfg.hidden % 16 != 0) return EP_ERR_INVALID_ARGUMENT;
  if ((cfg.alloc_fn == nullptr) != (cfg.free_fn == nullptr)) return EP_ERR_INVALID_ARGUMENT;
  if (cfg.hidden > kMaxHidden) return EP_ERR_UNSUPPORTED;
  const int N = cfg.num_nodes, K = cfg.top_k, E = cfg.num_experts;
  const int64_t R = topo.R;
  const int P = topo.P, M = topo.M, J = topo.J;
  const bool s2_rank = topo.s2_rank;
  const int E2 = topo.E2;
  if (cfg.max_handles == 0) cfg.max_handles = 2;
  if (cfg.ll_buffers == 0) cfg.ll_buffers = 2;
  if (cfg.ht_buffers == 0) cfg.ht_buffers = 1;
  if (cfg.max_handles > 64) return EP_ERR_UNSUPPORTED;

  Group* g = new (std::nothrow) Group();
  if (!g) return EP_ERR_OUT_OF_MEMORY;
  g->cfg = cfg;
  g->R = static_cast<int>(R);
  g->L = E / g->R;
  g->P = P;
  g->M = M;
  g->J = J;
  g->fp8 = cfg.payload == EP_DTYPE_FP8_E4M3;
  g->s2_rank = s2_rank;
  g->E2 = E2;
  g->row_bytes = g->fp8 ? cfg.hidden + cfg.hidden / 128 * 4 : static_cast<int64_t>(cfg.hidden) * 2;
  g->msg_bytes = g->row_bytes + 16;
  g->row_pitch = (g->row_bytes + 127) / 128 * 128;
  g->msg_pitch = (g->msg_bytes + 127) / 128 * 128;
  const int64_t S = cfg.num_src_ranks, Tm = cfg.max_tokens_per_rank;
  g->n_max = S * Tm;
  // Distinct destination nodes per token: at most min(K, N) for any topk_idx
  // (a caller-supplied one need not respect the node limit).
  const int64_t nodes_per_token = std::min<int64_t>(K, N);
  g->rows1_max = g->n_max * nodes_per_token;
  g->rows2_max = g->n_max * K;
  const int64_t tps = (Tm + kLayoutTile - 1) / kLayoutTile;
  // Slot, row and map indices are 32-bit on the device, and so is the
  // dispatch's wave count (a token spans up to ceil(H/8 / 256) waves).
  const int64_t kIndexMax = INT32_MAX;
  const int64_t waves_per_token = (cfg.hidden / 8 + 255) / 256;
  if (g->n_max * std::max<int64_t>({K, N, waves_per_token}) > kIndexMax || g->rows2_max > kIndexMax ||
      (cfg.mode == EP_MODE_LL && static_cast<int64_t>(E) * S * Tm > kIndexMax) ||
      S * tps * std::max<int64_t>(E, N) > kIndexMax) {
    delete g;
    return EP_ERR_UNSUPPORTED;
  }
  g->tiles_max = static_cast<int>(S * tps);

  ep_status_t st = EP_OK;
  if (cfg.mode == EP_MODE_LL) {
    g->nbuf = cfg.ll_buffers;
    for (int b = 0; st == EP_OK && b < g->nbuf; ++b)
      g->ll_buf[b] = static_cast<uint8_t*>(dev_alloc(g, static_cast<size_t>(E * S * Tm * g->msg_pitch), &st));
  } else {
    g->nbuf = cfg.ht_buffers;
    for (int b = 0; st == EP_OK && b < g->nbuf; ++b) {
      Group::StageSet& hs = g->ht[b];
      hs.st1 = static_cast<uint8_t*>(dev_alloc(g, static_cast<size_t>(g->rows1_max * g->row_pitch), &st));
      if (st == EP_OK) {
        const size_t r1 = static_cast<size_t>(g->rows1_max);
        const size_t bytes = align_up(r1 * 4) * 2 + align_up(r1 * K * 4) * 2;
        uint8_t* b1 = static_cast<uint8_t*>(dev_alloc(g, bytes, &st));
        if (b1) {
          Carve cv{b1};
          hs.m1_tok = cv.take<int32_t>(r1);
          hs.m1_src = cv.take<int32_t>(r1);
          hs.m1_topk = cv.take<int32_t>(r1 * K);
          hs.m1_w = cv.take<float>(r1 * K);
        }
      }
      if (st == EP_OK)
        hs.st2 = static_cast<uint8_t*>(dev_alloc(g, static_cast<size_t>(g->rows2_max * g->row_pitch), &st));
      if (st == EP_OK) {
        const size_t r2 = static_cast<size_t>(g->rows2_max);
        const size_t extra = s2_rank ? align_up(r2 * K * 4) * 2 : 0;   // received top-k and weights
        uint8_t* b2 = static_cast<uint8_t*>(dev_alloc(g, align_up(r2 * 4) * 3 + extra, &st));
        if (b2) {
          Carve cv{b2};
          hs.m2_src = cv.take<int32_t>(r2);
          hs.m2_tok = cv.take<int32_t>(r2);
          hs.m2_k = cv.take<int32_t>(r2);
          if (s2_rank) {
            hs.m2_topk = cv.take<int32_t>(r2 * K);
            hs.m2_w = cv.take<float>(r2 * K);
          }
        }
      }
    }
  }
  if (st == EP_OK) {
    g->err = static_cast<int32_t*>(dev_alloc(g, sizeof(int32_t), &st));
  }
  for (int hs = 0; st == EP_OK && hs < cfg.max_handles; ++hs) {
    const size_t nm = static_cast<size_t>(g->n_max);
    const size_t tiles = static_cast<size_t>(g->tiles_max);
    size_t bytes = align_up(nm * K * 4) * 2 + align_up(nm * N * 4);   // topk copy, ranks
    if (cfg.mode == EP_MODE_LL) {
      bytes += align_up(nm * K * 4) + align_up(static_cast<size_t>(E) * S * 4);
    } else {
      bytes += align_up(nm * N * 4) + align_up(nm * K * 4) + align_up(R * 4) * 2 + align_up(E * 4) * 2;
    }
    bytes += align_up(tiles * E * 4) + align_up(tiles * N * 4);
    uint8_t* b = static_cast<uint8_t*>(dev_alloc(g, bytes, &st));
    if (!b) break;
    Handle* h = new (std::nothrow) Handle();
    if (!h) { st = EP_ERR_OUT_OF_MEMORY; break; }
    h->g = g;
    h->in_use = false;
    Carve cv{b};
    h->topk = cv.take<int32_t>(nm * K);
    h->rank_e = cv.take<int32_t>(nm * K);
    h->rank_n = cv.take<int32_t>(nm * N);
    if (cfg.mode == EP_MODE_LL) {
      h->slot_map = cv.take<int32_t>(nm * K);
      h->ll_count = cv.take<int32_t>(static_cast<size_t>(E) * S);
    } else {
      h->node_row = cv.take<int32_t>(nm * N);
      h->row2 = cv.take<int32_t>(nm * K);
      h->c1 = cv.take<int32_t>(R);
      h->off1 = cv.take<int32_t>(R);
      h->c2 = cv.take<int32_t>(E);
      h->off2 = cv.take<int32_t>(E);
    }
    h->hist_e = cv.take<int32_t>(tiles * E);
    h->hist_n = cv.take<int32_t>(tiles * N);
    g->handles.push_back(h);
  }
  if (st != EP_OK) {
    free_all(g);
    for (Handle* h : g->handles) delete h;
    g->magic = kDeadMagic;
    delete g;
    return st;
  }
  if (!cfg.alloc_fn) {
    // Memory came from hipMalloc, so HIP is usable: initialise now.
    const ep_status_t s2 = ensure_device(g, as_stream(stream));
    if (s2 != EP_OK) {
      free_all(g);
      for (Handle* h : g->handles) delete h;
      g->magic = kDeadMagic;
      delete g;
      return s2;
    }
  }
  if (log_level() > 0)
    std::fprintf(stderr, "[ep] group mode=%s R=%d E=%d K=%d M=%d H=%d S=%d T_max=%d bytes=%lld\n",
                 cfg.mode == EP_MODE_LL ? "LL" : "HT", g->R, E, K, M, cfg.hidden, cfg.num_src_ranks,
                 cfg.max_tokens_per_rank, static_cast<long long>(g->bytes));
  *out = reinterpret_cast<ep_group_t>(g);
  return EP_OK;
}

EP_API ep_status_t ep_destroy_group(ep_group_t group) {
  Group* g = reinterpret_cast<Group*>(group);
  if (!group_ok(g)) return EP_ERR_INVALID_ARGUMENT;
  if (g->dev_ready) (void)hipDeviceSynchronize();
  if (g->host_counts) (void)hipHostFree(g->host_counts);
  free_all(g);
  for (Handle* h : g->handles) {
    h->magic = kDeadMagic;
    delete h;
  }
  g->handles.clear();
  g->magic = kDeadMagic;
  delete g;
  return EP_OK;
}

EP_API ep_status_t ep_group_memory(ep_group_t group, int64_t* bytes) {
  Group* g = reinterpret_cast<Group*>(group);
  if (!group_ok(g) || !bytes) return EP_ERR_INVALID_ARGUMENT;
  *bytes = g->bytes;
  return EP_OK;
}

EP_API ep_status_t ep_group_stats(ep_group_t group, ep_stats_t* stats) {
  Group* g = reinterpret_cast<Group*>(group);
  if (!group_ok(g) || !stats) return EP_ERR_INVALID_ARGUMENT;
  *stats = g->stats;
  return EP_OK;
}

// ===========================================================================
// Routing
// ===========================================================================

EP_API ep_status_t ep_route(ep_group_t group, const ep_tensor_t* scores, ep_tensor_t* topk_idx,
                            ep_stream_t stream) {
  Group* g = reinterpret_cast<Group*>(group);
  if (!group_ok(g)) return EP_ERR_INVALID_ARGUMENT;
  const int E = g->cfg.num_experts, K = g->cfg.top_k;
  if (!check2d(scores, EP_DTYPE_F32, -1, E, EP_TAG_TOKENS, false)) return EP_ERR_INVALID_ARGUMENT;
  const int64_t n = scores->sizes[0];
  if (!check2d(topk_idx, EP_DTYPE_I32, n, K, EP_TAG_TOPK_IDX, false) || !contiguous2d(topk_idx))
    return EP_ERR_INVALID_ARGUMENT;
  const hipStream_t s = as_stream(stream);
  if (const ep_status_t st = ensure_device(g, s); st != EP_OK) return st;
  RouteArgs a{};
  a.scores = static_cast<const float*>(scores->data);
  a.ld = scores->strides[0];
  a.n = n;
  a.E = E;
  a.N = g->cfg.num_nodes;
  a.K = K;
  a.M = g->M;
  a.J = g->J;
  a.topk = static_cast<int32_t*>(topk_idx->data);
  const ep_status_t st = from_hip(launch_route(a, s));
  if (st == EP_OK) {
    ++g->stats.route_calls;
    g->stats.tokens_routed += n;
    trace(g, "route", n);
  }
  return st;
}

// ===========================================================================
// Handles
// ===========================================================================

namespace {

// Takes a free handle slot and enqueues A2 for n = S*T tokens, from topk
// (a caller's [n, K]) or, with scores, routing them into topk_out first in
// the same pass (A1).
ep_status_t make_handle(Group* g, const int32_t* topk, const float* scores, int64_t ld, int32_t* topk_out,
                        int64_t n, hipStream_t s, ep_handle_t* out) {
  const int K = g->cfg.top_k, S = g->cfg.num_src_ranks;
  if (n % S != 0) return EP_ERR_INVALID_ARGUMENT;
  const int64_t T = n / S;
  if (T > g->cfg.max_tokens_per_rank) return EP_ERR_CAPACITY;
  Handle* h = nullptr;
  for (Handle* c : g->handles)
    if (!c->in_use) { h = c; break; }
  if (!h) return EP_ERR_CAPACITY;
  if (const ep_status_t st = ensure_device(g, s); st != EP_OK) return st;

  h->n = n;
  h->T = static_cast<int>(T);
  h->tps = static_cast<int>((T + kLayoutTile - 1) / kLayoutTile);
  h->n_tiles = h->tps * S;
  h->stream = s;
  LayoutArgs a{};
  a.topk = topk;
  a.scores = scores;
  a.ld = ld;
  a.M = g->M;
  a.J = g->J;
  a.topk_out = topk_out;
  a.n = n;
  a.S = S;
  a.T = h->T;
  a.K = K;
  a.E = g->cfg.num_experts;
  a.N = g->cfg.num_nodes;
  a.G = g->cfg.ranks_per_node;
  a.P = g->P;
  a.slots = g->cfg.max_tokens_per_rank;
  a.ht = g->cfg.mode == EP_MODE_HT;
  a.E2 = g->E2;
  a.L = g->L;
  a.s2_rank = g->s2_rank;
  a.l_shift = log2_exact(g->L);
  a.p_shift = log2_exact(g->P);
  a.tps = h->tps;
  a.n_tiles = h->n_tiles;
  a.hist_e = h->hist_e;
  a.hist_n = h->hist_n;
  a.topk_copy = h->topk;
  a.rank_e = h->rank_e;
  a.rank_n = h->rank_n;
  a.ll_count = h->ll_count;
  a.c1 = h->c1;
  a.c2 = h->c2;
  a.err = g->err;
  h->maps_ready = (n == 0);
  h->buf_half = -1;
  h->dispatched = false;
  h->pend = Handle::kPendNone;
  if (n == 0 && a.ht) {
    // Nothing routed: counts and offsets are zero.
    EP_HIP(launch_fill_i32(h->c1, g->R, 0, s));
    EP_HIP(launch_fill_i32(h->off1, g->R, 0, s));
    EP_HIP(launch_fill_i32(h->c2, a.E2, 0, s));
    EP_HIP(launch_fill_i32(h->off2, a.E2, 0, s));
  } else if (n == 0) {
    EP_HIP(launch_fill_i32(h->ll_count, static_cast<int64_t>(a.E) * S, 0, s));
  }
  const ep_status_t st = from_hip(launch_layout(a, s));
  if (st != EP_OK) return st;
  h->in_use = true;
  h->magic = kHandleMagic;
  *out = reinterpret_cast<ep_handle_t>(h);
  ++g->stats.handles_created;
  trace(g, "create_handle", n);
  return EP_OK;
}

}  // namespace

EP_API ep_status_t ep_create_handle(ep_group_t group, const ep_tensor_t* topk_idx, ep_stream_t stream,
                                    ep_handle_t* out) {
  Group* g = reinterpret_cast<Group*>(group);
  if (!group_ok(g) || !out) return EP_ERR_INVALID_ARGUMENT;
  *out = nullptr;
  const int K = g->cfg.top_k;
  if (!check2d(topk_idx, EP_DTYPE_I32, -1, K, EP_TAG_TOPK_IDX, false) || !contiguous2d(topk_idx))
    return EP_ERR_INVALID_ARGUMENT;
  return make_handle(g, static_cast<const int32_t*>(topk_idx->data), nullptr, 0, nullptr, topk_idx->sizes[0],
                     as_stream(stream), out);
}

EP_API ep_status_t ep_route_handle(ep_group_t group, const ep_tensor_t* scores, ep_tensor_t* topk_idx,
                                   ep_stream_t stream, ep_handle_t* out) {
  Group* g = reinterpret_cast<Group*>(group);
  if (!group_ok(g) || !out) return EP_ERR_INVALID_ARGUMENT;
  *out = nullptr;
  const int E = g->cfg.num_experts, K = g->cfg.top_k;
  if (!check2d(scores, EP_DTYPE_F32, -1, E, EP_TAG_TOKENS, false)) return EP_ERR_INVALID_ARGUMENT;
  const int64_t n = scores->sizes[0];
  if (!check2d(topk_idx, EP_DTYPE_I32, n, K, EP_TAG_TOPK_IDX, false) || !contiguous2d(topk_idx))
    return EP_ERR_INVALID_ARGUMENT;
  const ep_status_t st = make_handle(g, nullptr, static_cast<const float*>(scores->data), scores->strides[0],
                                     static_cast<int32_t*>(topk_idx->data), n, as_stream(stream), out);
  if (st == EP_OK) {
    ++g->stats.route_calls;
    g->stats.tokens_routed += n;
    trace(g, "route", n);
  }
  return st;
}

EP_API ep_status_t ep_destroy_handle(ep_handle_t handle) {
  Handle* h = reinterpret_cast<Handle*>(handle);
  if (!handle_ok(h)) return EP_ERR_INVALID_ARGUMENT;
  h->in_use = false;
  h->pend = Handle::kPendNone;   // a staged operation not completed is dropped
  return EP_OK;
}

EP_API ep_status_t ep_handle_get_num_recv(ep_handle_t handle, int32_t rank, int64_t* n) {
  Handle* h = reinterpret_cast<Handle*>(handle);
  if (!handle_ok(h) || !n) return EP_ERR_INVALID_ARGUMENT;
  Group* g = h->g;
  if (rank < -1 || rank >= g->R) return EP_ERR_INVALID_ARGUMENT;
  const int E = g->cfg.num_experts, S = g->cfg.num_src_ranks, L = g->L;
  const bool ll = g->cfg.mode == EP_MODE_LL;
  const size_t count = ll ? static_cast<size_t>(E) * S : static_cast<size_t>(g->E2);
  const int32_t* host = nullptr;
  if (const ep_status_t st = read_counts(h, ll ? h->ll_count : h->c2, count, &host); st != EP_OK) return st;
  int64_t total = 0;
  // The rank's keys: its experts, or with the per-rank stage 2 the rank itself.
  const int keys = ll ? E : g->E2;
  const int per = g->s2_rank ? 1 : L;
  const int e0 = rank < 0 ? 0 : rank * per, e1 = rank < 0 ? keys : (rank + 1) * per;
  for (int e = e0; e < e1; ++e) {
    if (ll) for (int s = 0; s < S; ++s) total += host[static_cast<size_t>(e) * S + s];
    else total += host[e];
  }
  *n = total;
  return EP_OK;
}

EP_API ep_status_t ep_handle_get_map(ep_handle_t handle, int32_t which, ep_tensor_t* view) {
  Handle* h = reinterpret_cast<Handle*>(handle);
  if (!handle_ok(h) || !view) return EP_ERR_INVALID_ARGUMENT;
  Group* g = h->g;
  const bool ll = g->cfg.mode == EP_MODE_LL;
  const int E = g->cfg.num_experts, K = g->cfg.top_k, N = g->cfg.num_nodes, S = g->cfg.num_src_ranks;
  if (which == EP_MAP_LL_SLOT || which == EP_MAP_HT_NODE_ROW || which == EP_MAP_HT_ROW ||
      which == EP_MAP_HT_RANK_OFFSET || which == EP_MAP_HT_EXPERT_OFFSET) {
    if (const ep_status_t st = ensure_maps(h, h->stream); st != EP_OK) return st;
  }
  switch (which) {
    case EP_MAP_LL_SLOT: if (!ll) break; fill_view(view, h->slot_map, EP_DTYPE_I32, h->n, K, EP_TAG_NONE); return EP_OK;
    case EP_MAP_LL_COUNT: if (!ll) break; fill_view(view, h->ll_count, EP_DTYPE_I32, E, S, EP_TAG_RECV_EXPERT_COUNTER_DEVICE); return EP_OK;
    case EP_MAP_HT_NODE_ROW: if (ll) break; fill_view(view, h->node_row, EP_DTYPE_I32, h->n, N, EP_TAG_NONE); return EP_OK;
    case EP_MAP_HT_ROW: if (ll) break; fill_view(view, h->row2, EP_DTYPE_I32, h->n, K, EP_TAG_NONE); return EP_OK;
    case EP_MAP_HT_RANK_COUNT: if (ll) break; fill_view(view, h->c1, EP_DTYPE_I32, g->R, 0, EP_TAG_NONE); return EP_OK;
    case EP_MAP_HT_RANK_OFFSET: if (ll) break; fill_view(view, h->off1, EP_DTYPE_I32, g->R, 0, EP_TAG_NONE); return EP_OK;
    case EP_MAP_HT_EXPERT_COUNT: if (ll) break; fill_view(view, h->c2, EP_DTYPE_I32, g->E2, 0, EP_TAG_TOKENS_PER_EXPERT); return EP_OK;
    case EP_MAP_HT_EXPERT_OFFSET: if (ll) break; fill_view(view, h->off2, EP_DTYPE_I32, g->E2, 0, EP_TAG_NONE); return EP_OK;
    default: break;
  }
  return EP_ERR_INVALID_ARGUMENT;
}

// ===========================================================================
// Dispatch
// ===========================================================================

EP_API ep_status_t ep_dispatch(ep_handle_t handle, const ep_tensor_t* tokens, const ep_tensor_t* scales,
                               const ep_tensor_t* topk_weights, ep_tensor_t* recv_counts,
                               int32_t send_only, ep_stream_t stream) {
  Handle* h = reinterpret_cast<Handle*>(handle);
  if (!handle_ok(h) || !tokens) return EP_ERR_INVALID_ARGUMENT;
  Group* g = h->g;
  const int H = g->cfg.hidden, K = g->cfg.top_k, E = g->cfg.num_experts, S = g->cfg.num_src_ranks;
  const bool ll = g->cfg.mode == EP_MODE_LL;
  const bool in_fp8 = tokens->dtype == EP_DTYPE_FP8_E4M3;
  if (in_fp8) {
    if (!g->fp8) return EP_ERR_INVALID_ARGUMENT;
    if (!check2d(tokens, EP_DTYPE_FP8_E4M3, h->n, H, EP_TAG_TOKENS, true)) return EP_ERR_INVALID_ARGUMENT;
    if (!check2d(scales, EP_DTYPE_F32, h->n, H / 128, EP_TAG_SCALES, false)) return EP_ERR_INVALID_ARGUMENT;
  } else {
    if (!check2d(tokens, EP_DTYPE_BF16, h->n, H, EP_TAG_TOKENS, true)) return EP_ERR_INVALID_ARGUMENT;
    if (scales) return EP_ERR_INVALID_ARGUMENT;
  }
  if (topk_weights && (!check2d(topk_weights, EP_DTYPE_F32, h->n, K, EP_TAG_TOPK_WEIGHTS, false) ||
                       !contiguous2d(topk_weights)))
    return EP_ERR_INVALID_ARGUMENT;
  int per_expert = 0;
  const bool counts_on_host = recv_counts && recv_counts->tag == EP_TAG_RECV_EXPERT_COUNTER_HOST;
  if (recv_counts) {
    const int32_t tag = counts_on_host ? EP_TAG_RECV_EXPERT_COUNTER_HOST : EP_TAG_TOKENS_PER_EXPERT;
    const bool one_d = recv_counts->dtype == EP_DTYPE_I32 && recv_counts->ndim == 1 &&
                       recv_counts->sizes[0] == (ll ? E : g->E2) && recv_counts->strides[0] == 1 && recv_counts->data &&
                       (recv_counts->tag == EP_TAG_NONE || recv_counts->tag == tag);
    const bool two_d = ll && recv_counts->ndim == 2 && check2d(recv_counts, EP_DTYPE_I32, E, S, tag, false) &&
                       contiguous2d(recv_counts);
    if (!one_d && !two_d) return EP_ERR_INVALID_ARGUMENT;
    per_expert = ll && one_d;
  }
  if (send_only && !ll) return EP_ERR_UNSUPPORTED;
  if (h->pend != Handle::kPendNone) return EP_ERR_INVALID_ARGUMENT;   // complete the staged one first
  int32_t* counts_out = recv_counts ? static_cast<int32_t*>(recv_counts->data) : nullptr;
  if (counts_on_host) {
    // The host counter must be pinned memory the device can write; the
    // receive stage writes through its device address.
    hipPointerAttribute_t attr{};
    if (hipPointerGetAttributes(&attr, counts_out) != hipSuccess || attr.type != hipMemoryTypeHost ||
        !attr.devicePointer) {
      (void)hipGetLastError();
      return EP_ERR_INVALID_ARGUMENT;
    }
    counts_out = static_cast<int32_t*>(attr.devicePointer);
  }
  const hipStream_t s = as_stream(stream);
  if (const ep_status_t st = ensure_device(g, s); st != EP_OK) return st;
  h->stream = s;

  DispatchArgs p = dispatch_base(h);
  p.payload = 1;
  p.x = tokens->data;
  p.ld_x = tokens->strides[0];
  p.in_fp8 = in_fp8;
  if (in_fp8) {
    p.x_scales = static_cast<const float*>(scales->data);
    p.ld_s = scales->strides[0];
  }
  p.out_fp8 = g->fp8;
  // The receive buffer (LL) or stage-row set (HT) this dispatch takes.
  const int half = g->buf_next;
  if (ll) p.ll_buf = g->ll_buf[half];
  p.w = topk_weights ? static_cast<const float*>(topk_weights->data) : nullptr;
  const Group::StageSet& hs = g->ht[ll ? 0 : half];
  p.st1 = hs.st1;
  p.m1_tok = hs.m1_tok;
  p.m1_src = hs.m1_src;
  p.m1_topk = hs.m1_topk;
  p.m1_w = hs.m1_w;
  p.st2 = hs.st2;
  p.m2_src = hs.m2_src;
  p.m2_tok = hs.m2_tok;
  p.m2_k = hs.m2_k;
  p.m2_topk = hs.m2_topk;
  p.m2_w = hs.m2_w;
  if (const ep_status_t st = from_hip(launch_dispatch(p, s)); st != EP_OK) return st;
  h->maps_ready = true;
  ++g->stats.dispatch_calls;
  g->stats.tokens_dispatched += h->n;
  trace(g, send_only ? "dispatch (send stage)" : "dispatch", h->n);
  h->buf_half = half;
  g->buf_next = (half + 1) % g->nbuf;
  // Every dispatch into a receive buffer overwrites the rows an earlier
  // handle left there: the buffer's count tells a handle whether its rows
  // are still in place.
  h->dispatched = true;
  h->buf_gen = ++g->buf_gen[half];
  if (send_only) {
    // The receive stage waits for ep_complete.
    h->pend = Handle::kPendDispatch;
    h->pend_counts = counts_out;
    h->pend_per_expert = per_expert;
    return EP_OK;
  }
  if (counts_out)
    return from_hip(ll ? launch_recv_counts(h->ll_count, E, S, per_expert, counts_out, s)
                       : launch_recv_counts(h->c2, g->E2, 1, 0, counts_out, s));
  return EP_OK;
}

EP_API ep_status_t ep_quantize(ep_group_t group, const ep_tensor_t* tokens, ep_tensor_t* q, ep_tensor_t* scales,
                               ep_stream_t stream) {
  Group* g = reinterpret_cast<Group*>(group);
  if (!group_ok(g) || !g->fp8) return EP_ERR_INVALID_ARGUMENT;
  const int H = g->cfg.hidden;
  if (!check2d(tokens, EP_DTYPE_BF16, -1, H, EP_TAG_TOKENS, true)) return EP_ERR_INVALID_ARGUMENT;
  const int64_t n = tokens->sizes[0];
  if (!check2d(q, EP_DTYPE_FP8_E4M3, n, H, EP_TAG_TOKENS, true)) return EP_ERR_INVALID_ARGUMENT;
  if (!check2d(scales, EP_DTYPE_F32, n, H / 128, EP_TAG_SCALES, false)) return EP_ERR_INVALID_ARGUMENT;
  const hipStream_t s = as_stream(stream);
  if (const ep_status_t st = ensure_device(g, s); st != EP_OK) return st;
  QuantArgs a{};
  a.x = static_cast<const uint16_t*>(tokens->data);
  a.ld_x = tokens->strides[0];
  a.q = static_cast<uint8_t*>(q->data);
  a.ld_q = q->strides[0];
  a.scales = static_cast<float*>(scales->data);
  a.ld_s = scales->strides[0];
  a.n = n;
  a.H = H;
  const ep_status_t st = from_hip(launch_quantize(a, s));
  if (st == EP_OK) {
    ++g->stats.quantize_calls;
    trace(g, "quantize", n);
  }
  return st;
}

namespace {
ep_status_t buffer_view(Group* g, int32_t which, int half, ep_tensor_t* view) {
  const bool ll = g->cfg.mode == EP_MODE_LL;
  const int K = g->cfg.top_k;
  const int64_t slots_total = static_cast<int64_t>(g->cfg.num_experts) * g->cfg.num_src_ranks *
                              g->cfg.max_tokens_per_rank;
  switch (which) {
    case EP_BUF_LL_RECV: if (!ll) break; fill_view(view, g->ll_buf[half], EP_DTYPE_U8, slots_total, g->msg_bytes, EP_TAG_TOKENS, g->msg_pitch); return EP_OK;
    case EP_BUF_HT_STAGE1: if (ll) break; fill_view(view, g->ht[half].st1, EP_DTYPE_U8, g->rows1_max, g->row_bytes, EP_TAG_TOKENS, g->row_pitch); return EP_OK;
    case EP_BUF_HT_STAGE1_TOKEN: if (ll) break; fill_view(view, g->ht[half].m1_tok, EP_DTYPE_I32, g->rows1_max, 0, EP_TAG_NONE); return EP_OK;
    case EP_BUF_HT_STAGE1_SRC: if (ll) break; fill_view(view, g->ht[half].m1_src, EP_DTYPE_I32, g->rows1_max, 0, EP_TAG_NONE); return EP_OK;
    case EP_BUF_HT_STAGE1_TOPK: if (ll) break; fill_view(view, g->ht[half].m1_topk, EP_DTYPE_I32, g->rows1_max, K, EP_TAG_TOPK_IDX); return EP_OK;
    case EP_BUF_HT_STAGE1_WEIGHTS: if (ll) break; fill_view(view, g->ht[half].m1_w, EP_DTYPE_F32, g->rows1_max, K, EP_TAG_TOPK_WEIGHTS); return EP_OK;
    case EP_BUF_HT_STAGE2: if (ll) break; fill_view(view, g->ht[half].st2, EP_DTYPE_U8, g->rows2_max, g->row_bytes, EP_TAG_TOKENS, g->row_pitch); return EP_OK;
    case EP_BUF_HT_STAGE2_SRC: if (ll) break; fill_view(view, g->ht[half].m2_src, EP_DTYPE_I32, g->rows2_max, 0, EP_TAG_NONE); return EP_OK;
    case EP_BUF_HT_STAGE2_TOKEN: if (ll) break; fill_view(view, g->ht[half].m2_tok, EP_DTYPE_I32, g->rows2_max, 0, EP_TAG_NONE); return EP_OK;
    case EP_BUF_HT_STAGE2_K: if (ll) break; fill_view(view, g->ht[half].m2_k, EP_DTYPE_I32, g->rows2_max, 0, EP_TAG_NONE); return EP_OK;
    case EP_BUF_HT_STAGE2_TOPK: if (!g->s2_rank) break; fill_view(view, g->ht[half].m2_topk, EP_DTYPE_I32, g->rows2_max, K, EP_TAG_TOPK_IDX); return EP_OK;
    case EP_BUF_HT_STAGE2_WEIGHTS: if (!g->s2_rank) break; fill_view(view, g->ht[half].m2_w, EP_DTYPE_F32, g->rows2_max, K, EP_TAG_TOPK_WEIGHTS); return EP_OK;
    default: break;
  }
  return EP_ERR_INVALID_ARGUMENT;
}
}  // namespace

EP_API ep_status_t ep_get_buffer(ep_group_t group, int32_t which, ep_tensor_t* view) {
  Group* g = reinterpret_cast<Group*>(group);
  if (!group_ok(g) || !view) return EP_ERR_INVALID_ARGUMENT;
  return buffer_view(g, which, 0, view);
}

namespace {
// A dispatched handle whose receive rows a later dispatch has overwritten.
bool rows_overwritten(const Handle* h) {
  return h->dispatched && h->buf_gen != h->g->buf_gen[h->buf_half];
}
}  // namespace

EP_API ep_status_t ep_handle_get_buffer(ep_handle_t handle, int32_t which, ep_tensor_t* view) {
  Handle* h = reinterpret_cast<Handle*>(handle);
  if (!handle_ok(h) || !view) return EP_ERR_INVALID_ARGUMENT;
  const bool ll = h->g->cfg.mode == EP_MODE_LL;
  if (ll && which == EP_BUF_LL_RECV && h->buf_half < 0) return EP_ERR_INVALID_ARGUMENT;
  if (rows_overwritten(h)) return EP_ERR_INVALID_ARGUMENT;
  return buffer_view(h->g, which, h->buf_half < 0 ? 0 : h->buf_half, view);
}

EP_API ep_status_t ep_get_partition(ep_handle_t handle, int32_t rank, int32_t which, ep_tensor_t* view) {
  Handle* h = reinterpret_cast<Handle*>(handle);
  if (!handle_ok(h) || !view) return EP_ERR_INVALID_ARGUMENT;
  Group* g = h->g;
  if (rank < 0 || rank >= g->R) return EP_ERR_INVALID_ARGUMENT;
  const bool ll = g->cfg.mode == EP_MODE_LL;
  if (ll && h->buf_half < 0) return EP_ERR_INVALID_ARGUMENT;   // not dispatched: no buffer yet
  if (rows_overwritten(h)) return EP_ERR_INVALID_ARGUMENT;
  ep_tensor_t full;
  if (const ep_status_t st = buffer_view(g, which, h->buf_half < 0 ? 0 : h->buf_half, &full); st != EP_OK)
    return st;
  int64_t first = 0, count = 0;
  if (ll) {
    // Rank r's experts [r*L, (r+1)*L) are one contiguous [L][S][T_max] block of slots.
    count = static_cast<int64_t>(g->L) * g->cfg.num_src_ranks * g->cfg.max_tokens_per_rank;
    first = rank * count;
  } else {
    // The rank's rows [offset, offset + count) from the handle's counts.
    const bool stage1 = which >= EP_BUF_HT_STAGE1 && which <= EP_BUF_HT_STAGE1_WEIGHTS;
    const int keys = stage1 || g->s2_rank ? 1 : g->L;   // stage 2 per expert: the rank's L experts
    const int k0 = stage1 || g->s2_rank ? rank : rank * g->L;
    if (const ep_status_t st = ensure_maps(h, h->stream); st != EP_OK) return st;   // writes the offsets
    const int32_t* off = nullptr;
    if (const ep_status_t st = read_counts(h, (stage1 ? h->off1 : h->off2) + k0, 1, &off); st != EP_OK) return st;
    first = *off;
    const int32_t* c = nullptr;
    if (const ep_status_t st = read_counts(h, (stage1 ? h->c1 : h->c2) + k0, keys, &c); st != EP_OK) return st;
    for (int q = 0; q < keys; ++q) count += c[q];
  }
  // Row `first` of the view starts strides[0] elements per row further in.
  full.data = static_cast<uint8_t*>(full.data) + first * full.strides[0] * dtype_size(full.dtype);
  full.sizes[0] = count;
  *view = full;
  return EP_OK;
}

// ===========================================================================
// Combine
// ===========================================================================

EP_API ep_status_t ep_combine(ep_handle_t handle, const ep_tensor_t* expert_out,
                              const ep_tensor_t* topk_weights, ep_tensor_t* out, int32_t send_only,
                              ep_stream_t stream) {
  Handle* h = reinterpret_cast<Handle*>(handle);
  if (!handle_ok(h) || !expert_out) return EP_ERR_INVALID_ARGUMENT;
  Group* g = h->g;
  const int H = g->cfg.hidden, K = g->cfg.top_k;
  const bool ll = g->cfg.mode == EP_MODE_LL;
  ep_tensor_t y2;
  if (!expert_rows(g, expert_out, &y2)) return EP_ERR_INVALID_ARGUMENT;
  if (topk_weights && (!check2d(topk_weights, EP_DTYPE_F32, h->n, K, EP_TAG_TOPK_WEIGHTS, false) ||
                       !contiguous2d(topk_weights)))
    return EP_ERR_INVALID_ARGUMENT;
  if (g->s2_rank && topk_weights) return EP_ERR_INVALID_ARGUMENT;   // rank rows are weighted already
  if (!check2d(out, EP_DTYPE_BF16, h->n, H, EP_TAG_TOKENS, true)) return EP_ERR_INVALID_ARGUMENT;
  if (send_only && !ll) return EP_ERR_UNSUPPORTED;
  if (h->pend != Handle::kPendNone) return EP_ERR_INVALID_ARGUMENT;   // complete the staged one first
  const hipStream_t s = as_stream(stream);
  if (const ep_status_t st = ensure_device(g, s); st != EP_OK) return st;
  h->stream = s;
  if (const ep_status_t st = ensure_maps(h, s); st != EP_OK) return st;
  CombineArgs a{};
  a.y = static_cast<const uint16_t*>(y2.data);
  a.ld_y = y2.strides[0];
  a.rows = y2.sizes[0];
  a.w = topk_weights ? static_cast<const float*>(topk_weights->data) : nullptr;   // null: unit weights
  a.loc = ll ? h->slot_map : h->row2;
  a.n = h->n;
  a.K = K;
  a.H = H;
  a.out = static_cast<uint16_t*>(out->data);
  a.ld_out = out->strides[0];
  a.max_blocks = dispatch_block_cap(g);
  a.err = g->err;
  if (send_only) {
    // The gather-reduce is the receive stage: it waits for ep_complete.
    h->pend = Handle::kPendCombine;
    h->pend_comb = a;
  } else if (const ep_status_t st = from_hip(launch_combine(a, s)); st != EP_OK) {
    return st;
  }
  ++g->stats.combine_calls;
  g->stats.tokens_combined += h->n;
  trace(g, send_only ? "combine (send stage)" : "combine", h->n);
  return EP_OK;
}

// ===========================================================================
// Backward pass (reuse of the forward handle)
// ===========================================================================

EP_API ep_status_t ep_combine_backward(ep_handle_t handle, const ep_tensor_t* grad_out,
                                       const ep_tensor_t* expert_out, const ep_tensor_t* topk_weights,
                                       ep_tensor_t* grad_expert_out, ep_tensor_t* grad_weights,
                                       ep_stream_t stream) {
  Handle* h = reinterpret_cast<Handle*>(handle);
  if (!handle_ok(h)) return EP_ERR_INVALID_ARGUMENT;
  Group* g = h->g;
  const int H = g->cfg.hidden, K = g->cfg.top_k;
  const bool ll = g->cfg.mode == EP_MODE_LL;
  if (g->s2_rank) return EP_ERR_UNSUPPORTED;   // the experts apply the weights: nothing to differentiate here
  if (!check2d(grad_out, EP_DTYPE_BF16, h->n, H, EP_TAG_TOKENS, true)) return EP_ERR_INVALID_ARGUMENT;
  if (!check2d(topk_weights, EP_DTYPE_F32, h->n, K, EP_TAG_TOPK_WEIGHTS, false) || !contiguous2d(topk_weights))
    return EP_ERR_INVALID_ARGUMENT;
  ep_tensor_t dy2, y2;
  if (!expert_rows(g, grad_expert_out, &dy2)) return EP_ERR_INVALID_ARGUMENT;
  if (expert_out && !expert_rows(g, expert_out, &y2)) return EP_ERR_INVALID_ARGUMENT;
  if (grad_weights && (!expert_out || !check2d(grad_weights, EP_DTYPE_F32, h->n, K, EP_TAG_TOPK_WEIGHTS, false) ||
                       !contiguous2d(grad_weights)))
    return EP_ERR_INVALID_ARGUMENT;
  if (h->pend != Handle::kPendNone) return EP_ERR_INVALID_ARGUMENT;
  const hipStream_t s = as_stream(stream);
  if (const ep_status_t st = ensure_device(g, s); st != EP_OK) return st;
  h->stream = s;
  if (const ep_status_t st = ensure_maps(h, s); st != EP_OK) return st;
  CombineBwdArgs a{};
  a.g = static_cast<const uint16_t*>(grad_out->data);
  a.ld_g = grad_out->strides[0];
  a.y = expert_out ? static_cast<const uint16_t*>(y2.data) : nullptr;
  a.ld_y = expert_out ? y2.strides[0] : 0;
  a.dy = static_cast<uint16_t*>(dy2.data);
  a.ld_dy = dy2.strides[0];
  a.rows = expert_out ? std::min(dy2.sizes[0], y2.sizes[0]) : dy2.sizes[0];
  a.w = static_cast<const float*>(topk_weights->data);
  a.loc = ll ? h->slot_map : h->row2;
  a.dw = grad_weights ? static_cast<float*>(grad_weights->data) : nullptr;
  a.n = h->n;
  a.K = K;
  a.H = H;
  a.max_blocks = dispatch_block_cap(g);
  a.err = g->err;
  const ep_status_t st = from_hip(launch_combine_backward(a, s));
  if (st == EP_OK) {
    ++g->stats.combine_backward_calls;
    trace(g, "combine_backward", h->n);
  }
  return st;
}

EP_API ep_status_t ep_dispatch_backward(ep_handle_t handle, const ep_tensor_t* grad_expert_in,
                                        ep_tensor_t* grad_tokens, ep_stream_t stream) {
  Handle* h = reinterpret_cast<Handle*>(handle);
  if (!handle_ok(h)) return EP_ERR_INVALID_ARGUMENT;
  Group* g = h->g;
  const int H = g->cfg.hidden;
  const bool ll = g->cfg.mode == EP_MODE_LL;
  ep_tensor_t r2;
  if (!expert_rows(g, grad_expert_in, &r2)) return EP_ERR_INVALID_ARGUMENT;
  if (!check2d(grad_tokens, EP_DTYPE_BF16, h->n, H, EP_TAG_TOKENS, true)) return EP_ERR_INVALID_ARGUMENT;
  if (h->pend != Handle::kPendNone) return EP_ERR_INVALID_ARGUMENT;
  const hipStream_t s = as_stream(stream);
  if (const ep_status_t st = ensure_device(g, s); st != EP_OK) return st;
  h->stream = s;
  if (const ep_status_t st = ensure_maps(h, s); st != EP_OK) return st;
  CombineArgs a{};
  a.y = static_cast<const uint16_t*>(r2.data);
  a.ld_y = r2.strides[0];
  a.rows = r2.sizes[0];
  a.w = nullptr;   // unit weights: the sum over the token's entries in k order
  a.loc = ll ? h->slot_map : h->row2;
  a.n = h->n;
  a.K = g->cfg.top_k;
  a.H = H;
  a.out = static_cast<uint16_t*>(grad_tokens->data);
  a.ld_out = grad_tokens->strides[0];
  a.max_blocks = dispatch_block_cap(g);
  a.err = g->err;
  const ep_status_t st = from_hip(launch_combine(a, s));
  if (st == EP_OK) {
    ++g->stats.dispatch_backward_calls;
    trace(g, "dispatch_backward", h->n);
  }
  return st;
}

EP_API ep_status_t ep_complete(ep_handle_t handle, ep_stream_t stream) {
  Handle* h = reinterpret_cast<Handle*>(handle);
  if (!handle_ok(h) || h->pend == Handle::kPendNone) return EP_ERR_INVALID_ARGUMENT;
  Group* g = h->g;
  const hipStream_t s = as_stream(stream);
  if (const ep_status_t st = ensure_device(g, s); st != EP_OK) return st;
  h->stream = s;
  const int pend = h->pend;
  h->pend = Handle::kPendNone;
  ep_status_t st = EP_OK;
  if (pend == Handle::kPendCombine)
    st = from_hip(launch_combine(h->pend_comb, s));
  else if (h->pend_counts)
    st = from_hip(launch_recv_counts(h->ll_count, g->cfg.num_experts, g->cfg.num_src_ranks,
                                     h->pend_per_expert, h->pend_counts, s));
  if (st == EP_OK) {
    ++g->stats.complete_calls;
    trace(g, pend == Handle::kPendCombine ? "complete (combine receive stage)" : "complete (dispatch receive stage)",
          h->n);
  }
  return st;
}

// ===========================================================================
// Identity expert
// ===========================================================================

EP_API ep_status_t ep_dequantize_rows(ep_group_t group, const ep_tensor_t* rows, ep_tensor_t* y,
                                      ep_stream_t stream) {
  Group* g = reinterpret_cast<Group*>(group);
  if (!group_ok(g) || !rows || !y) return EP_ERR_INVALID_ARGUMENT;
  const int H = g->cfg.hidden;
  if (rows->dtype != EP_DTYPE_U8 || rows->ndim != 2 || rows->strides[1] != 1 ||
      rows->sizes[1] < g->row_bytes || rows->strides[0] < rows->sizes[1] || rows->sizes[0] < 0 ||
      (rows->sizes[0] > 0 && !rows->data))
    return EP_ERR_INVALID_ARGUMENT;
  if ((reinterpret_cast<uintptr_t>(rows->data) & 15u) || (rows->sizes[0] > 1 && (rows->strides[0] & 15)))
    return EP_ERR_INVALID_ARGUMENT;
  if (!check2d(y, EP_DTYPE_BF16, rows->sizes[0], H, EP_TAG_TOKENS, true)) return EP_ERR_INVALID_ARGUMENT;
  const hipStream_t s = as_stream(stream);
  if (const ep_status_t st = ensure_device(g, s); st != EP_OK) return st;
  DequantArgs a{};
  a.rows = static_cast<const uint8_t*>(rows->data);
  a.row_stride = rows->strides[0];
  a.n = rows->sizes[0];
  a.H = H;
  a.fp8 = g->fp8;
  a.y = static_cast<uint16_t*>(y->data);
  a.ld_y = y->strides[0];
  return from_hip(launch_dequant(a, s));
}

// ===========================================================================
// Errors
// ===========================================================================

EP_API const char* ep_status_string(ep_status_t status) {
  switch (status) {
    case EP_OK: return "EP_OK";
    case EP_ERR_INVALID_ARGUMENT: return "EP_ERR_INVALID_ARGUMENT";
    case EP_ERR_CAPACITY: return "EP_ERR_CAPACITY";
    case EP_ERR_OUT_OF_MEMORY: return "EP_ERR_OUT_OF_MEMORY";
    case EP_ERR_HIP: return "EP_ERR_HIP";
    case EP_ERR_UNSUPPORTED: return "EP_ERR_UNSUPPORTED";
    default: return "EP_ERR_UNKNOWN";
  }
}

EP_API ep_status_t ep_get_device_error(ep_group_t group, int32_t* code) {
  Group* g = reinterpret_cast<Group*>(group);
  if (!group_ok(g) || !code) return EP_ERR_INVALID_ARGUMENT;
  *code = 0;
  if (!g->dev_ready) return EP_OK;
  EP_HIP(hipDeviceSynchronize());
  EP_HIP(hipMemcpy(code, g->err, sizeof(int32_t), hipMemcpyDeviceToHost));
  const int32_t zero = 0;
  EP_HIP(hipMemcpy(g->err, &zero, sizeof(int32_t), hipMemcpyHostToDevice));
  return EP_OK;
}

EP_API int ep_last_hip_error(void) { return g_last_hip; }
