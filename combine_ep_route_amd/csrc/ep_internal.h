// Internal declarations of libep: group/handle state and kernel launchers.
// Not installed; the public interface is include/ep.h.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <vector>

#include "ep.h"

#define EP_API extern "C" __attribute__((visibility("default")))

namespace ep {

// Build limits (checked at group creation).
constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 32;
constexpr int kMaxNodes = 64;
constexpr int kMaxRanks = 1024;
constexpr int kMaxHidden = 16384;
constexpr int kLayoutTile = 16;    // tokens per layout tile (one workgroup of the count kernel)

constexpr uint32_t kGroupMagic = 0x45504752u;   // "EPGR"
constexpr uint32_t kHandleMagic = 0x4550484Eu;  // "EPHN"
constexpr uint32_t kDeadMagic = 0xDEADDEADu;

struct CombineArgs {
  const uint16_t* y;      // BF16 rows
  int64_t ld_y;           // elements
  int64_t rows;           // rows available in y
  const float* w;         // [n, K], or null for unit weights (dispatch backward)
  const int32_t* loc;     // [n, K]
  int64_t n;
  int K, H;
  uint16_t* out;
  int64_t ld_out;
  int max_blocks;         // 0 = no cap
  int32_t* err;
};

struct Handle;

// log2(v) if v is a power of two, else -1.
inline int log2_exact(int v) {
  if (v <= 0 || (v & (v - 1)) != 0) return -1;
  int s = 0;
  while ((1 << s) < v) ++s;
  return s;
}

// Routing topology derived from a configuration, checked: shared by group
// creation and the group-free layout.  Checks mode, topology, K, M, T_max,
// S and the stage-2 kind (not the payload, hidden size or buffers).
struct Topology {
  int R, L, P, M, J, E2, s2_rank;
};
ep_status_t check_topology(const ep_config_t& cfg, Topology* t);

struct Group {
  uint32_t magic = kGroupMagic;
  ep_config_t cfg{};
  int R = 0;          // ranks
  int L = 0;          // experts per rank
  int P = 0;          // experts per node
  int J = 0;          // experts summed per node score (0 = no node limit)
  int M = 0;          // nodes kept (0 = no limit)
  int fp8 = 1;        // payload is FP8 (else BF16)
  int64_t row_bytes = 0;   // FP8: H + H/128*4; BF16: 2H
  int64_t msg_bytes = 0;   // LL: row_bytes + 16
  int64_t row_pitch = 0;   // HT row stride in the buffers: row_bytes up to 128 B
  int64_t msg_pitch = 0;   // LL message stride: msg_bytes up to 128 B
  int64_t n_max = 0;       // S * T_max
  int64_t rows1_max = 0;   // HT stage-1 rows, worst case
  int64_t rows2_max = 0;   // HT stage-2 rows, worst case (n_max * K)
  int s2_rank = 0;         // HT stage 2 per (token, rank)
  int E2 = 0;              // stage-2 keys: E, or R per rank
  int tiles_max = 0;       // layout tiles, worst case

  // Device buffers (owned).
  struct Alloc { void* ptr; size_t bytes; };
  std::vector<Alloc> allocs;
  int64_t bytes = 0;
  // Receive buffers, used in turn: LL fixed-slot buffers, or HT stage-row
  // sets (stage-1 and stage-2 rows with their metadata).
  uint8_t* ll_buf[2] = {nullptr, nullptr};
  struct StageSet {
    uint8_t* st1 = nullptr;
    int32_t* m1_tok = nullptr;
    int32_t* m1_src = nullptr;
    int32_t* m1_topk = nullptr;
    float* m1_w = nullptr;
    uint8_t* st2 = nullptr;
    int32_t* m2_src = nullptr;
    int32_t* m2_tok = nullptr;
    int32_t* m2_k = nullptr;
    int32_t* m2_topk = nullptr;   // per-rank stage 2 only
    float* m2_w = nullptr;
  };
  StageSet ht[2];
  int nbuf = 0;                              // receive buffers (LL) or stage sets (HT)
  int buf_next = 0;                          // the one the next dispatch takes
  uint64_t buf_gen[2] = {0, 0};              // dispatches into each of them
  int32_t* err = nullptr;    // device error word

  std::vector<Handle*> handles;

  // Device facts, read at the first launch.
  bool dev_ready = false;
  int device = -1;
  int num_cu = 0;

  ep_stats_t stats{};   // host-side call counters

  // Pinned host memory for the blocking count queries, allocated at the
  // first query (hipHostMalloc) and freed with the group.
  int32_t* host_counts = nullptr;
  size_t host_counts_len = 0;
};

struct Handle {
  uint32_t magic = kHandleMagic;
  Group* g = nullptr;
  bool in_use = false;
  int64_t n = 0;   // tokens (S*T)
  int T = 0;       // tokens per source
  int tps = 0;     // layout tiles per source
  int n_tiles = 0;
  hipStream_t stream = nullptr;
  bool maps_ready = false;       // slot/row maps written (by dispatch)
  int32_t* topk = nullptr;       // copy of topk_idx [n_max, K]
  int32_t* rank_e = nullptr;     // [n_max, K] rank of (token, k) inside its tile and expert, or -1
  int32_t* rank_n = nullptr;     // [n_max, N] HT: rank inside its tile and destination node, or -1
  int32_t* slot_map = nullptr;   // LL [n_max, K]
  int32_t* ll_count = nullptr;   // LL [E, S]
  int32_t* node_row = nullptr;   // HT [n_max, N]
  int32_t* row2 = nullptr;       // HT [n_max, K]
  int32_t* c1 = nullptr;         // HT [R]
  int32_t* off1 = nullptr;       // HT [R]
  int32_t* c2 = nullptr;         // HT [E]
  int32_t* off2 = nullptr;       // HT [E]
  int32_t* hist_e = nullptr;     // [tiles_max, E] tile counts -> prefixes
  int32_t* hist_n = nullptr;     // [tiles_max, N]
  int buf_half = -1;             // receive buffer / stage set of the last dispatch
  bool dispatched = false;       // a dispatch has written this handle's rows
  uint64_t buf_gen = 0;          // the buffer's dispatch count when this handle wrote it

  // Staged (send_only) operation awaiting ep_complete: at most one.
  enum { kPendNone = 0, kPendDispatch = 1, kPendCombine = 2 };
  int pend = kPendNone;
  int32_t* pend_counts = nullptr;   // dispatch: recv_counts destination (or null)
  int pend_per_expert = 0;
  CombineArgs pend_comb{};          // combine: the launch to run
};

// ---------------------------------------------------------------------------
// Kernel launchers (one translation unit each).  All return hipSuccess or the
// launch error; they enqueue on `stream` and never synchronise.
// ---------------------------------------------------------------------------

struct RouteArgs {
  const float* scores;
  int64_t ld;        // row stride of scores, elements
  int64_t n;
  int E, N, K, M, J;
  int32_t* topk;     // [n, K]
};
hipError_t launch_route(const RouteArgs& a, hipStream_t stream);

struct LayoutArgs {
  const int32_t* topk;   // [n, K], or null when the handle is made from scores
  const float* scores;   // [n, E] with row stride ld, or null: route in the same pass
  int64_t ld;
  int M, J;              // routing: nodes kept (0 = no limit), scores summed per node
  int32_t* topk_out;     // routing: the caller's [n, K] output
  int64_t n;
  int S, T, K, E, N, G, P;
  int slots;             // LL slots per (expert, source)
  int ht;                // 1 = HT maps, 0 = LL maps
  int E2;                // stage-2 keys: E, or R with the per-rank stage 2
  int L;                 // experts per rank
  int s2_rank;           // HT stage 2 per (token, rank): key = e / L, first entry only
  int l_shift, p_shift;  // log2 of L and P when powers of two, else -1
  int tps, n_tiles;      // tiles per source, tiles in all
  int32_t* hist_e;       // [tiles, E2] per-tile key counts, rewritten as prefixes over the key's tiles
  int32_t* hist_n;       // [tiles, N] the same per destination node (HT)
  int32_t* topk_copy;    // [n, K]
  int32_t* rank_e;       // [n, K] out: in-tile ranks
  int32_t* rank_n;       // [n, N] out: in-tile node ranks (HT)
  int32_t* ll_count;     // LL out: slots used per (expert, source) [E, S]
  int32_t* c1;           // HT out: stage-1 rows per rank [R]
  int32_t* c2;           // HT out: stage-2 rows per key [E2]
  int32_t* err;          // device error word (bad or repeated entries)
};
hipError_t launch_layout(const LayoutArgs& a, hipStream_t stream);

// Receive stage of a dispatch: copy the [E, S] counters to out, or with
// per_expert != 0 write their sums over S ([E]).
hipError_t launch_recv_counts(const int32_t* counts, int E, int S, int per_expert, int32_t* out,
                              hipStream_t stream);

// Set `count` int32 values to `value` with a small kernel (stream-ordered,
// capture-safe).
hipError_t launch_fill_i32(int32_t* p, int64_t count, int32_t value, hipStream_t stream);

struct DispatchArgs {
  const void* x;          // BF16 [n, H] or FP8 [n, H]
  int64_t ld_x;           // elements
  const float* x_scales;  // FP8 input only: [n, H/128]
  int64_t ld_s;
  int in_fp8;             // tokens arrive quantised
  int out_fp8;            // payload is FP8
  int64_t n;
  int T, K, N, G, H, E, S, P, slots, tps;
  int E2, L, s2_rank;     // stage-2 keys (E, or R per rank), experts per rank, per-rank flag
  int64_t row_bytes, msg_bytes;
  int64_t row_pitch, msg_pitch;   // strides of HT rows / LL messages in the buffers
  int ht;
  int payload;            // 0 = compute the maps only
  int num_cu;             // CUs to spread the persistent workgroups over
  int max_blocks;         // 0 = no cap beyond residency
  const int32_t* topk;    // the handle's copy [n, K]
  const int32_t* rank_e;  // in-tile ranks [n, K]
  const int32_t* rank_n;  // in-tile node ranks [n, N]
  const int32_t* hist_e;  // tile prefixes [tiles, E]
  const int32_t* hist_n;  // [tiles, N]
  const int32_t* c1;      // HT: stage-1 rows per rank [R]
  const int32_t* c2;      // HT: stage-2 rows per key [E2]
  int32_t* off1;          // HT out: first stage-1 row of each rank [R] (their exclusive prefix sums)
  int32_t* off2;          // HT out: first stage-2 row of each key [E2]
  int32_t* slot_map;      // LL out [n, K]
  int32_t* row2;          // HT out [n, K]
  int32_t* node_row;      // HT out [n, N]
  // LL
  uint8_t* ll_buf;
  // HT
  const float* w;
  uint8_t* st1;
  int32_t* m1_tok;
  int32_t* m1_src;
  int32_t* m1_topk;
  float* m1_w;
  uint8_t* st2;
  int32_t* m2_src;
  int32_t* m2_tok;
  int32_t* m2_k;
  int32_t* m2_topk;       // per-rank stage 2: the token's entries on the row's rank
  float* m2_w;
};
hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t stream);

// FP8 quantisation alone: BF16 [n, H] -> codes [n, H] + scales [n, H/128],
// the dispatch's own arithmetic (H % 128 == 0).
struct QuantArgs {
  const uint16_t* x;      // BF16 [n, H]
  int64_t ld_x;           // elements
  uint8_t* q;             // codes [n, H]
  int64_t ld_q;           // bytes
  float* scales;          // [n, H/128]
  int64_t ld_s;           // elements
  int64_t n;
  int H;
};
hipError_t launch_quantize(const QuantArgs& a, hipStream_t stream);

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);

struct CombineBwdArgs {
  const uint16_t* g;      // BF16 [n, H] gradient of the combine's output
  int64_t ld_g;           // elements
  const uint16_t* y;      // BF16 expert-output rows, or null (no dw)
  int64_t ld_y;
  uint16_t* dy;           // BF16 row gradients at the dispatch geometry
  int64_t ld_dy;
  int64_t rows;           // rows valid in dy (and y)
  const float* w;         // [n, K]
  const int32_t* loc;     // [n, K]
  float* dw;              // [n, K] or null
  int64_t n;
  int K, H;
  int max_blocks;         // 0 = no cap
  int32_t* err;
};
hipError_t launch_combine_backward(const CombineBwdArgs& a, hipStream_t stream);

struct DequantArgs {
  const uint8_t* rows;
  int64_t row_stride;     // bytes
  int64_t n;
  int H;
  int fp8;
  uint16_t* y;
  int64_t ld_y;           // elements
};
hipError_t launch_dequant(const DequantArgs& a, hipStream_t stream);

}  // namespace ep
