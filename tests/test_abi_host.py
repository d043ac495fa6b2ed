"""Host-side checks of the C ABI (no GPU needed).

* libep.so loads and exports every function include/ep.h declares;
* configurations are validated before any HIP call;
* allocator hooks: a failing alloc_fn gives EP_ERR_OUT_OF_MEMORY and every
  successful allocation is handed back to free_fn (no leak);
* descriptor validation of every entry point on a group whose memory came
  from host-side hooks (nothing is ever enqueued).
"""
import ctypes
import os
import re
import subprocess
import sys

import pytest

from combine_ep_route_amd import _abi as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ep.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ep_[a-z_]+)\s*\(", src)) - {"ep_status_t"})


def test_header_functions_are_bound():
    assert _declared() == sorted(A.SIGNATURES)


def test_library_exports_every_declared_symbol():
    lib = A.lib()
    for name in _declared():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", A.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    ep_syms = {s for s in exported if s.startswith("ep_")}
    assert ep_syms == set(_declared())


def test_missing_library_is_an_error():
    """Without the built library the binding raises: there is no fallback path."""
    code = ("import combine_ep_route_amd._abi as A, combine_ep_route_amd as ep\n"
            "A.LIB_PATH = '/nonexistent/libep.so'; A._lib = None\n"
            "try:\n"
            "    ep.ep_create_group(mode='ht', num_nodes=2, ranks_per_node=2, num_experts=16, top_k=2,\n"
            "                       max_nodes_per_token=0, hidden=128, max_tokens_per_rank=8, num_src_ranks=1)\n"
            "except ImportError as e:\n"
            "    print('raised:', e)\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       cwd=ROOT, timeout=120)
    assert r.returncode == 0, r.stderr
    assert "raised:" in r.stdout and "no fallback" in r.stdout


def test_status_strings():
    lib = A.lib()
    for code, name in [(0, "EP_OK"), (1, "EP_ERR_INVALID_ARGUMENT"), (2, "EP_ERR_CAPACITY"),
                       (3, "EP_ERR_OUT_OF_MEMORY"), (4, "EP_ERR_HIP"), (5, "EP_ERR_UNSUPPORTED")]:
        assert lib.ep_status_string(code).decode() == name


class HostPool:
    """alloc_fn/free_fn hooks backed by host memory; can fail at the n-th call."""

    def __init__(self, fail_at=None):
        self.fail_at = fail_at
        self.calls = 0
        self.live = {}
        self.freed = 0
        self.alloc_fn = A.ALLOC_FN(self._alloc)
        self.free_fn = A.FREE_FN(self._free)

    def _alloc(self, nbytes, ctx):
        self.calls += 1
        if self.fail_at is not None and self.calls >= self.fail_at:
            return None
        buf = ctypes.create_string_buffer(min(int(nbytes), 4096))  # never dereferenced
        addr = ctypes.addressof(buf)
        self.live[addr] = buf
        return addr

    def _free(self, ptr, ctx):
        self.live.pop(ptr)
        self.freed += 1


def _cfg(pool=None, **kw):
    base = dict(mode=A.EP_MODE_HT, num_nodes=8, ranks_per_node=8, num_experts=256, top_k=8,
                max_nodes_per_token=4, hidden=7168, max_tokens_per_rank=4096, num_src_ranks=1,
                payload=A.EP_DTYPE_FP8_E4M3, max_handles=2, num_cus=0)
    base.update(kw)
    c = A.EpConfig()
    for k, v in base.items():
        setattr(c, k, v)
    if pool is not None:
        c.alloc_fn = pool.alloc_fn
        c.free_fn = pool.free_fn
    return c


def _create(cfg):
    out = ctypes.c_void_p()
    st = A.lib().ep_create_group(ctypes.byref(cfg), None, ctypes.byref(out))
    return st, out


@pytest.mark.parametrize("bad", [
    dict(mode=7), dict(num_nodes=0), dict(num_experts=100), dict(top_k=0),
    dict(top_k=300), dict(hidden=7000), dict(hidden=200), dict(payload=A.EP_DTYPE_F32),
    dict(max_tokens_per_rank=0), dict(num_src_ranks=0), dict(max_nodes_per_token=-1),
    dict(ll_buffers=-1), dict(ll_buffers=3), dict(ht_stage2=2), dict(ht_stage2=-1),
    dict(max_nodes_per_token=1, top_k=40),          # 1 node x 32 experts < 40
    dict(num_experts=64, max_nodes_per_token=1, top_k=16),  # ceil(16/1)=16 > 8 per node
])
def test_invalid_config_rejected_before_hip(bad):
    pool = HostPool()
    st, _ = _create(_cfg(pool, **bad))
    assert st == A.EP_ERR_INVALID_ARGUMENT
    assert pool.calls == 0


@pytest.mark.parametrize("bad", [
    dict(num_experts=2048, num_nodes=8, ranks_per_node=8), dict(top_k=33, num_experts=256),
    dict(num_src_ranks=65), dict(hidden=16384 + 128), dict(max_handles=65),
    # more LL slots (E * S * T_max) than 32-bit indices address
    dict(mode=A.EP_MODE_LL, num_nodes=32, ranks_per_node=32, num_experts=1024, num_src_ranks=1024,
         max_tokens_per_rank=4096),
    # more HT stage-2 rows (S * T_max * K) than 32-bit indices address
    dict(num_nodes=32, ranks_per_node=32, num_experts=1024, top_k=32, num_src_ranks=1024,
         max_tokens_per_rank=1 << 17),
    # more dispatch waves (S * T_max tokens, up to 8 waves per token at hidden 16384) than
    # 32-bit indices address, with every row and slot count still in range
    dict(num_nodes=2, ranks_per_node=1, num_experts=4, top_k=2, max_nodes_per_token=2, hidden=16384,
         num_src_ranks=64, max_tokens_per_rank=1 << 23),
])
def test_unsupported_config(bad):
    pool = HostPool()
    st, _ = _create(_cfg(pool, **bad))
    assert st == A.EP_ERR_UNSUPPORTED
    assert pool.calls == 0


def test_one_hook_only_is_invalid():
    pool = HostPool()
    c = _cfg()
    c.alloc_fn = pool.alloc_fn
    st, _ = _create(c)
    assert st == A.EP_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("mode", [A.EP_MODE_LL, A.EP_MODE_HT])
def test_alloc_failure_frees_everything(mode):
    ok = HostPool()
    st, g = _create(_cfg(ok, mode=mode, max_tokens_per_rank=128 if mode == A.EP_MODE_LL else 4096))
    assert st == A.EP_OK and ok.freed == 0
    n_allocs = ok.calls
    assert A.lib().ep_destroy_group(g) == A.EP_OK
    assert ok.freed == n_allocs and not ok.live
    for fail_at in range(1, n_allocs + 1):
        pool = HostPool(fail_at=fail_at)
        st, g = _create(_cfg(pool, mode=mode, max_tokens_per_rank=128 if mode == A.EP_MODE_LL else 4096))
        assert st == A.EP_ERR_OUT_OF_MEMORY
        assert g.value is None
        assert pool.freed == fail_at - 1 and not pool.live


def test_group_memory_matches_layout():
    pool = HostPool()
    st, g = _create(_cfg(pool, mode=A.EP_MODE_LL, num_src_ranks=64, max_tokens_per_rank=128))
    assert st == A.EP_OK
    b = ctypes.c_int64()
    assert A.lib().ep_group_memory(g, ctypes.byref(b)) == A.EP_OK
    # receive space: 256 experts x 64 sources x 128 slots x 7408-byte messages
    assert b.value >= 256 * 64 * 128 * 7408
    view = A.EpTensor()
    assert A.lib().ep_get_buffer(g, A.EP_BUF_LL_RECV, ctypes.byref(view)) == A.EP_OK
    assert (view.sizes[0], view.sizes[1]) == (256 * 64 * 128, 7408)
    assert A.lib().ep_get_buffer(g, A.EP_BUF_HT_STAGE1, ctypes.byref(view)) == A.EP_ERR_INVALID_ARGUMENT
    A.lib().ep_destroy_group(g)


def test_ll_double_buffering_memory():
    # two receive buffers by default (NCCL-EP LL double buffering), one on request
    sizes = {}
    for nbuf in (0, 1, 2):
        pool = HostPool()
        st, g = _create(_cfg(pool, mode=A.EP_MODE_LL, num_src_ranks=4, max_tokens_per_rank=32,
                             ll_buffers=nbuf))
        assert st == A.EP_OK
        b = ctypes.c_int64()
        assert A.lib().ep_group_memory(g, ctypes.byref(b)) == A.EP_OK
        sizes[nbuf] = b.value
        A.lib().ep_destroy_group(g)
        assert not pool.live
    one_buffer = 256 * 4 * 32 * 7424          # messages at their 128-byte pitch
    assert sizes[0] == sizes[2]
    assert sizes[2] - sizes[1] == one_buffer


def test_ht_double_buffering_memory():
    # one set of stage rows by default, two on request (the second dispatch of
    # a two-micro-batch pipeline then leaves the first one's rows in place)
    sizes = {}
    for nbuf in (0, 1, 2):
        pool = HostPool()
        st, g = _create(_cfg(pool, max_tokens_per_rank=256, ht_buffers=nbuf))
        assert st == A.EP_OK
        b = ctypes.c_int64()
        assert A.lib().ep_group_memory(g, ctypes.byref(b)) == A.EP_OK
        sizes[nbuf] = b.value
        A.lib().ep_destroy_group(g)
        assert not pool.live
    row_pitch = 7424
    rows1, rows2 = 256 * 8, 256 * 8
    assert sizes[0] == sizes[1]
    assert sizes[2] - sizes[1] >= (rows1 + rows2) * row_pitch
    for bad in (-1, 3):
        assert _create(_cfg(HostPool(), ht_buffers=bad))[0] == A.EP_ERR_INVALID_ARGUMENT


def test_per_rank_stage2_memory():
    # the per-rank stage 2 adds the received top-k ids and weights per row
    sizes = {}
    for mode in (A.EP_HT_STAGE2_PER_EXPERT, A.EP_HT_STAGE2_PER_RANK):
        pool = HostPool()
        st, g = _create(_cfg(pool, ht_stage2=mode, max_tokens_per_rank=256))
        assert st == A.EP_OK
        b = ctypes.c_int64()
        assert A.lib().ep_group_memory(g, ctypes.byref(b)) == A.EP_OK
        sizes[mode] = b.value
        view = A.EpTensor()
        want = A.EP_OK if mode == A.EP_HT_STAGE2_PER_RANK else A.EP_ERR_INVALID_ARGUMENT
        assert A.lib().ep_get_buffer(g, A.EP_BUF_HT_STAGE2_TOPK, ctypes.byref(view)) == want
        A.lib().ep_destroy_group(g)
    rows2 = 256 * 8
    assert sizes[A.EP_HT_STAGE2_PER_RANK] - sizes[A.EP_HT_STAGE2_PER_EXPERT] >= 2 * rows2 * 8 * 4


def test_staged_calls_reject_null_handles():
    lib = A.lib()
    view = A.EpTensor()
    assert lib.ep_complete(None, None) == A.EP_ERR_INVALID_ARGUMENT
    assert lib.ep_handle_get_buffer(None, A.EP_BUF_LL_RECV, ctypes.byref(view)) == A.EP_ERR_INVALID_ARGUMENT
    assert lib.ep_get_partition(None, 0, A.EP_BUF_LL_RECV, ctypes.byref(view)) == A.EP_ERR_INVALID_ARGUMENT


def _t(data, dtype, sizes, strides=None, tag=A.EP_TAG_NONE):
    d = A.EpTensor()
    d.data = data
    d.dtype = dtype
    d.ndim = len(sizes)
    if strides is None:
        strides = [1] * len(sizes)
        for i in range(len(sizes) - 2, -1, -1):
            strides[i] = strides[i + 1] * sizes[i + 1]
    for i, (s, st) in enumerate(zip(sizes, strides)):
        d.sizes[i] = s
        d.strides[i] = st
    d.tag = tag
    return d


@pytest.fixture
def host_group():
    pool = HostPool()
    st, g = _create(_cfg(pool))
    assert st == A.EP_OK
    yield g
    A.lib().ep_destroy_group(g)
    assert not pool.live


FAKE = 0x10000  # a 16-byte aligned address that is never dereferenced


def test_route_descriptor_validation(host_group):
    lib = A.lib()
    scores = _t(FAKE, A.EP_DTYPE_F32, [16, 256])
    topk = _t(FAKE, A.EP_DTYPE_I32, [16, 8])
    bad = [
        (_t(FAKE, A.EP_DTYPE_BF16, [16, 256]), topk),            # wrong dtype
        (_t(FAKE, A.EP_DTYPE_F32, [16, 255]), topk),             # wrong width
        (scores, _t(FAKE, A.EP_DTYPE_I32, [15, 8])),             # row mismatch
        (scores, _t(FAKE, A.EP_DTYPE_I32, [16, 8], [16, 1])),    # not contiguous
        (_t(FAKE, A.EP_DTYPE_F32, [16, 256], tag=A.EP_TAG_SCALES), topk),  # wrong tag
        (_t(FAKE, A.EP_DTYPE_F32, [16, 256], [256, 2]), topk),   # inner stride
    ]
    for s, t in bad:
        assert lib.ep_route(host_group, ctypes.byref(s), ctypes.byref(t), None) == A.EP_ERR_INVALID_ARGUMENT
    assert lib.ep_route(None, ctypes.byref(scores), ctypes.byref(topk), None) == A.EP_ERR_INVALID_ARGUMENT
    # a valid call reaches HIP: without a GPU it fails there, cleanly
    st = lib.ep_route(host_group, ctypes.byref(scores), ctypes.byref(topk), None)
    assert st in (A.EP_ERR_HIP, A.EP_OK)


def test_handle_capacity_and_validation(host_group):
    lib = A.lib()
    out = ctypes.c_void_p()
    over = _t(FAKE, A.EP_DTYPE_I32, [4097, 8])
    assert lib.ep_create_handle(host_group, ctypes.byref(over), None, ctypes.byref(out)) == A.EP_ERR_CAPACITY
    wrong_k = _t(FAKE, A.EP_DTYPE_I32, [64, 4])
    assert lib.ep_create_handle(host_group, ctypes.byref(wrong_k), None,
                                ctypes.byref(out)) == A.EP_ERR_INVALID_ARGUMENT
    # a destroyed or made-up handle is rejected
    assert lib.ep_destroy_handle(None) == A.EP_ERR_INVALID_ARGUMENT
    junk = ctypes.create_string_buffer(256)
    assert lib.ep_destroy_handle(ctypes.addressof(junk)) == A.EP_ERR_INVALID_ARGUMENT
    n = ctypes.c_int64()
    assert lib.ep_handle_get_num_recv(ctypes.addressof(junk), 0, ctypes.byref(n)) == A.EP_ERR_INVALID_ARGUMENT


def test_device_error_before_any_launch(host_group):
    code = ctypes.c_int32(99)
    assert A.lib().ep_get_device_error(host_group, ctypes.byref(code)) == A.EP_OK
    assert code.value == 0


def test_binding_refuses_host_tensors():
    """A host tensor's address must never reach a kernel: the binding
    refuses it before calling the library."""
    import torch
    from combine_ep_route_amd import ep as binding
    with pytest.raises(ValueError, match="on the GPU"):
        binding.desc(torch.zeros((4, 8), dtype=torch.float32))


def test_stats_start_at_zero_without_hip():
    """A group made with allocator hooks (no HIP call) reports zero counters,
    and the stats struct has the header's layout."""
    import re as _re
    src = open(HEADER).read()
    body = _re.search(r"typedef struct \{(.*?)\} ep_stats_t;", src, _re.S).group(1)
    names = _re.findall(r"int64_t\s+(\w+);", body)
    assert tuple(names) == A.STAT_FIELDS
    pool = HostPool()
    st, g = _create(_cfg(pool))
    assert st == A.EP_OK
    out = A.EpStats()
    assert A.lib().ep_group_stats(g, ctypes.byref(out)) == A.EP_OK
    assert all(getattr(out, n) == 0 for n in A.STAT_FIELDS)
    assert A.lib().ep_group_stats(None, ctypes.byref(out)) == A.EP_ERR_INVALID_ARGUMENT
    assert A.lib().ep_destroy_group(g) == A.EP_OK


def test_layout_noalloc_validates_before_any_hip_call():
    """ep_layout_noalloc checks its descriptors, the batch against T_max and
    its working storage against the fixed scratch size before touching HIP
    (the data pointers below are never dereferenced)."""
    lib = A.lib()
    fake = 0x10000
    n, K, N, R, E = 64, 8, 8, 64, 256
    cfg = _cfg(max_tokens_per_rank=64)
    topk = _t(fake, A.EP_DTYPE_I32, [n, K], tag=A.EP_TAG_TOPK_IDX)

    def maps_ht(over=None):
        shapes = {A.EP_MAP_HT_NODE_ROW: [n, N], A.EP_MAP_HT_ROW: [n, K], A.EP_MAP_HT_RANK_COUNT: [R],
                  A.EP_MAP_HT_RANK_OFFSET: [R], A.EP_MAP_HT_EXPERT_COUNT: [E], A.EP_MAP_HT_EXPERT_OFFSET: [E]}
        shapes.update(over or {})
        ts = [None] * 8
        for m, sh in shapes.items():
            if sh is not None:
                ts[m] = _t(fake, A.EP_DTYPE_I32, sh)
        arr = (ctypes.POINTER(A.EpTensor) * 8)(*[ctypes.pointer(x) if x is not None else None for x in ts])
        return arr, ts

    def call(c, t, arr):
        return lib.ep_layout_noalloc(ctypes.byref(c) if c is not None else None,
                                     ctypes.byref(t) if t is not None else None, arr, None, None)

    arr, keep = maps_ht()
    assert call(None, topk, arr) == A.EP_ERR_INVALID_ARGUMENT
    assert call(cfg, None, arr) == A.EP_ERR_INVALID_ARGUMENT
    assert call(cfg, topk, None) == A.EP_ERR_INVALID_ARGUMENT
    bad_dtype = _t(fake, A.EP_DTYPE_F32, [n, K])
    assert call(cfg, bad_dtype, arr) == A.EP_ERR_INVALID_ARGUMENT
    # more tokens per source than T_max
    assert call(_cfg(max_tokens_per_rank=63), topk, arr) == A.EP_ERR_CAPACITY
    # a map missing, a map of the wrong shape, an LL map given in HT
    for over in ({A.EP_MAP_HT_ROW: None}, {A.EP_MAP_HT_NODE_ROW: [n, N + 1]}, {A.EP_MAP_HT_RANK_COUNT: [R - 1]},
                 {A.EP_MAP_LL_SLOT: [n, K]}):
        a2, keep2 = maps_ht(over)
        assert call(cfg, topk, a2) == A.EP_ERR_INVALID_ARGUMENT, over
    # an inconsistent topology
    assert call(_cfg(num_experts=100, max_tokens_per_rank=64), topk, arr) == A.EP_ERR_INVALID_ARGUMENT
    # working storage beyond EP_NOALLOC_SCRATCH_BYTES
    big = 70_000
    tb = _t(fake, A.EP_DTYPE_I32, [big, K])
    ab, keepb = maps_ht({A.EP_MAP_HT_NODE_ROW: [big, N], A.EP_MAP_HT_ROW: [big, K]})
    assert call(_cfg(max_tokens_per_rank=big), tb, ab) == A.EP_ERR_CAPACITY
