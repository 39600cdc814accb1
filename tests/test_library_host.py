"""Host-side checks of the C ABI library, with no GPU: it loads, exports every symbol
the header declares, and refuses bad arguments before launching anything.

Every call here fails argument checking, so no kernel is ever launched; pointers are
fake (never dereferenced) addresses.
"""
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


@pytest.fixture(scope="module")
def lib():
    from exact_attention_82_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from exact_attention_82_amd import build
        build.build_library()
    return _lib.load()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("attn_fwd", "attn_fwd_varlen", "attn_fwd_splitkv", "attn_merge",
              "attn_splitkv_workspace_bytes"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    from exact_attention_82_amd import _lib
    for name in _declared():
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, f"binding lacks {name}"


Q, K, V, O, L = 0x10000, 0x20000, 0x30000, 0x40000, 0x50000  # fake, 16-byte aligned


def fwd(lib, *, q=Q, k=K, v=V, o=O, l=L, B=1, H=1, Sq=8, Sk=8, d=64, scale=0.125, causal=0,
        dtype=1):
    return lib.attn_fwd(q, k, v, o, l, B, H, Sq, Sk, d, scale, causal, dtype, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(o=None), 1), (dict(l=None), 1),
    (dict(B=0), 2), (dict(H=-1), 2), (dict(Sq=0), 2), (dict(Sk=0), 2),
    (dict(B=1 << 20, H=1 << 20, Sq=1 << 20), 2),
    (dict(d=32), 4), (dict(d=96), 4), (dict(d=512), 4), (dict(dtype=3), 4), (dict(dtype=-1), 4),
    (dict(q=Q + 8), 3), (dict(o=O + 4), 3), (dict(l=L + 2), 3),
    (dict(causal=2), 7), (dict(causal=-1), 7), (dict(scale=0.0), 7), (dict(scale=-0.5), 7),
    (dict(scale=math.inf), 7), (dict(scale=math.nan), 7), (dict(scale=3e38), 7),
])
def test_attn_fwd_refuses_bad_arguments(lib, kw, status):
    assert fwd(lib, **kw) == status


CQ, CK = 0x70000, 0x70100  # fake int32 offset arrays


def varlen(lib, *, q=Q, k=K, v=V, o=O, l=L, cq=CQ, ck=CK, B=2, H=1, mq=8, mk=8, tq=16, tk=16,
           d=64, scale=0.125, causal=0, dtype=1):
    return lib.attn_fwd_varlen(q, k, v, o, l, cq, ck, B, H, mq, mk, tq, tk, d, scale, causal, dtype,
                               None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(o=None), 1), (dict(cq=None), 1), (dict(ck=None), 1),
    (dict(B=0), 2), (dict(H=0), 2), (dict(mq=0), 2), (dict(mk=0), 2), (dict(tq=0), 2),
    (dict(tk=-3), 2), (dict(H=1 << 20, tq=1 << 20, d=128), 2), (dict(mq=1 << 30), 2),
    (dict(d=96), 4), (dict(dtype=5), 4),
    (dict(q=Q + 8), 3), (dict(cq=CQ + 2), 3), (dict(ck=CK + 1), 3),
    (dict(causal=3), 7), (dict(scale=0.0), 7), (dict(scale=math.nan), 7),
])
def test_attn_fwd_varlen_refuses_bad_arguments(lib, kw, status):
    assert varlen(lib, **kw) == status


def test_attn_fwd_ex_output_types(lib):
    def ex(out_dtype, **kw):
        a = dict(q=Q, k=K, v=V, o=O, l=L)
        a.update(kw)
        return lib.attn_fwd_ex(a["q"], a["k"], a["v"], a["o"], a["l"], 1, 1, 8, 8, 64, 0.125, 0, 1,
                               out_dtype, None)
    assert ex(2) == 4           # fp8 output: unsupported
    assert ex(7) == 4
    assert ex(1, o=None) == 1   # the usual checks come first
    assert ex(1, o=O + 8) == 3


def test_split_count_query(lib):
    # out-of-range arguments give 0; without a GPU the CU count is unknown and the rule
    # never splits (the split choice itself is tested in test_plan_host.py)
    assert lib.attn_splitkv_num_splits(0, 8, 128, 32768, 128, 2) == 0
    assert lib.attn_splitkv_num_splits(1, 8, 128, 32768, 96, 2) == 0
    assert lib.attn_splitkv_num_splits(1, 8, 128, 32768, 128, 7) == 0
    assert lib.attn_splitkv_num_splits(1, 8, 128, 32768, 128, 2) >= 1


def test_splitkv_and_merge_refuse_bad_arguments(lib):
    need = lib.attn_splitkv_workspace_bytes(1, 2, 16, 64, 4)
    W = 0x60000

    def split(ws=W, nb=need, n=4, qd=1.0, kd=1.0, vd=1.0, d=64, dtype=2):
        return lib.attn_fwd_splitkv(Q, K, V, ws, nb, n, 1, 2, 16, 64, d, 0.125, 0, dtype,
                                    qd, kd, vd, None)
    assert split(ws=None) == 1
    assert split(nb=need - 1) == 5
    assert split(n=0) == 7
    assert split(n=4097) == 7
    assert split(qd=0.0) == 7 and split(kd=math.nan) == 7 and split(vd=-1.0) == 7
    assert split(ws=W + 8) == 3
    assert split(d=100) == 4
    assert lib.attn_merge(None, need, 4, O, L, 1, 2, 16, 64, None) == 1
    assert lib.attn_merge(W, need - 4, 4, O, L, 1, 2, 16, 64, None) == 5
    assert lib.attn_merge(W, need, 0, O, L, 1, 2, 16, 64, None) == 7
    assert lib.attn_merge(W, need, 4, O, L, 1, 2, 16, 65, None) == 4
    assert lib.attn_merge(W, need, 4, O + 4, L, 1, 2, 16, 64, None) == 3


def test_workspace_layout(lib):
    rows, d, n = 1 * 8 * 128, 128, 16
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    ml = n * rows * 4
    assert lib.attn_splitkv_workspace_bytes(1, 8, 128, d, n) == 2 * up(ml) + n * rows * d * 4
    assert lib.attn_splitkv_workspace_bytes(1, 8, 128, 100, n) == 0
    assert lib.attn_splitkv_workspace_bytes(1, 8, 128, d, 0) == 0


def test_workgroup_count_follows_the_pages_query_tile_grid(lib):
    """B * H * ceil(S / block_m), the query-tile grid the page tabulates.  Non-causal
    plans need no device query, so this runs without a GPU: every dtype and head dim
    uses 128 query rows per workgroup (the page's 512 workgroups for (1, 8, 8192)), and
    so does the split-KV path, times the number of splits."""
    import json
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "cta_counts.json")))
    for dt in (0, 1, 2):
        for d in (64, 128, 256):
            bm = lib.attn_block_m(1, 8, 8192, 8192, d, 0, dt, 0)
            assert bm == 128
            for row in g["printed"]:
                if row["tile_q"] == bm:
                    got = lib.attn_num_workgroups(row["batch"], row["heads"], row["length"], row["length"], d, 0, dt, 0)
                    assert got == row["ctas"]
            assert lib.attn_num_workgroups(8, 32, 2048, 2048, d, 0, dt, 0) == 8 * 32 * 2048 // bm
            assert lib.attn_block_m(1, 8, 128, 32768, d, 0, dt, 16) == 128
            assert lib.attn_num_workgroups(1, 8, 128, 32768, d, 0, dt, 16) == 8 * 16
            assert lib.attn_num_workgroups(1, 8, 8192, 8192, d, 0, dt, 1) == 8 * 64
            assert lib.attn_num_workgroups(1, 16, 1000, 1000, d, 0, dt, 0) == 16 * -(-1000 // bm)
    assert lib.attn_num_workgroups(1, 8, 8192, 8192, 96, 0, 1, 0) == -1
    assert lib.attn_block_m(1, 8, 8192, 8192, 128, 2, 1, 0) == 0


def test_kernel_names_and_status_strings(lib):
    assert lib.attn_kernel_name(1, 8, 8192, 8192, 128, 0, 1, 0) == b"attn_fwd_bf16_d128_bm128_bn32"
    assert lib.attn_kernel_name(1, 8, 8192, 8192, 256, 0, 1, 0) == b"attn_fwd_bf16_d256_bm128_bn32"
    assert lib.attn_kernel_name(1, 8, 128, 32768, 128, 0, 2, 4).startswith(b"attn_fwd_splitkv_fp8_d128")
    assert lib.attn_kernel_name(1, 8, 128, 128, 100, 0, 1, 0) == b"unsupported"
    for s in range(8):
        assert lib.attn_status_string(s)
    assert lib.attn_last_hip_error() == 0


def test_per_head_slices_must_fit_32bit_offsets(lib):
    # 2^24 keys x 128 x bf16 = 4 GiB per head: refused before any launch
    assert fwd(lib, Sq=8, Sk=1 << 24, d=128) == 2
    assert fwd(lib, Sq=1 << 23, Sk=8, d=256, dtype=0) == 2


def test_backward_refuses_bad_arguments_and_lays_out_its_workspace(lib):
    B, H, Sq, Sk, d = 1, 2, 16, 24, 128
    rows = B * H * Sq
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    need = lib.attn_bwd_workspace_bytes(B, H, Sq, Sk, d, 0)
    assert need == up(rows * d * 2) + up(rows * 4) + up(rows * 4)
    assert lib.attn_bwd_workspace_bytes(B, H, Sq, Sk, 100, 0) == 0
    assert lib.attn_bwd_workspace_bytes(B, H, Sq, Sk, d, 2) == 0
    # causal, Sq = Sk = 700: key tiles 0-3 sweep more than a third of the 22 query tiles
    # (22, 18, 14, 10 > 22/3), so the workspace also holds their second-half dK and dV;
    # query tiles 5-1 sweep more than a third of the longest dQ sweep (22, 20, 16, 12, 8
    # key tiles of 32 > 22/3), so it holds their second-half dQ too
    base = up(2 * 700 * d * 2) + 2 * up(2 * 700 * 4)
    assert lib.attn_bwd_workspace_bytes(1, 2, 700, 700, d, 1) == (
        base + 2 * up(2 * 4 * 128 * d * 4) + up(2 * 5 * 128 * d * 4))
    assert lib.attn_bwd_workspace_bytes(1, 2, 700, 700, d, 0) == base
    DO, DQ, DK, DV, W = 0x60000, 0x70000, 0x80000, 0x90000, 0xA0000

    def bwd(q=Q, dout=DO, dq=DQ, ws=W, nb=need, d=d, dtype=1, causal=0, scale=0.125):
        return lib.attn_bwd(q, K, V, O, dout, L, dq, DK, DV, ws, nb, B, H, Sq, Sk, d, scale,
                            causal, dtype, None)
    assert bwd(q=None) == 1 and bwd(dout=None) == 1 and bwd(dq=None) == 1 and bwd(ws=None) == 1
    assert bwd(nb=need - 1) == 5
    assert bwd(d=96) == 4           # the backward covers d = 64, 128 and 256
    assert bwd(dtype=0) == 4 and bwd(dtype=2) == 4   # bf16 only
    assert bwd(dq=DQ + 4) == 3 and bwd(ws=W + 8) == 3
    assert bwd(causal=3) == 7 and bwd(scale=-1.0) == 7
    names = {lib.attn_bwd_kernel_name(d, 1, w).decode() for w in range(3)}
    assert all(n.startswith("attn_bwd_") for n in names) and len(names) == 3
    assert lib.attn_bwd_kernel_name(d, 0, 1).decode() == "unsupported"


def test_splitkv_noalloc_refuses_bad_arguments_before_any_device_call(lib):
    """The allocation-free split call checks everything -- including that the workspace
    fits the library's static device array -- before it looks the array up or launches."""
    from exact_attention_82_amd import _lib

    def call(o=O, l=L, n=4, B=1, H=2, Sq=16, Sk=64, d=64, dtype=2, qd=1.0, causal=0):
        return lib.attn_fwd_splitkv_noalloc(Q, K, V, o, l, n, B, H, Sq, Sk, d, 0.125, causal, dtype,
                                            qd, 1.0, 1.0, None)
    assert call(o=None) == 1 and call(l=None) == 1
    assert call(B=0) == 2
    assert call(d=100) == 4 and call(dtype=9) == 4
    assert call(o=O + 4) == 3 and call(l=L + 8) == 3
    assert call(n=0) == 7 and call(n=4097) == 7 and call(qd=0.0) == 7 and call(causal=2) == 7
    # 64 heads x 1024 rows x 64 chunks of (d + 2) floats: far beyond the static array
    assert lib.attn_splitkv_workspace_bytes(1, 64, 1024, 128, 64) > _lib.ATTN_NOALLOC_SCRATCH_BYTES
    assert call(H=64, Sq=1024, Sk=4096, d=128, n=64) == 5
    # the fp8 split workload (B=1, H=8, Sq=128, d=128) fits up to 32 chunks, the count the
    # split rule picks for it on a 256-CU device
    assert lib.attn_splitkv_workspace_bytes(1, 8, 128, 128, 32) <= _lib.ATTN_NOALLOC_SCRATCH_BYTES
    assert lib.attn_splitkv_workspace_bytes(1, 8, 128, 128, 64) > _lib.ATTN_NOALLOC_SCRATCH_BYTES


def test_grid_index_bound_follows_the_launch(lib):
    """Workgroup indices are 32-bit.  Dense calls are bounded by their own grid, not by
    the largest split grid: 8 x 64 heads of 131072 rows (2^19 workgroups, ~17 GB per
    tensor) pass the shape checks; a split call is bounded with its actual split count."""
    assert lib.attn_splitkv_num_splits(8, 64, 131072, 131072, 128, 1) >= 1
    # 2 x 2^30 workgroup indices: refused
    assert fwd(lib, B=1, H=65536, Sq=1 << 22, Sk=8, d=64) == 2
    W = 0x60000

    def split(n, nb=16):
        return lib.attn_fwd_splitkv(Q, K, V, W, nb, n, 1, 512, 1 << 20, 64, 64, 0.125, 0, 1,
                                    1.0, 1.0, 1.0, None)
    # 512 heads x 8192 query tiles x n (x 2, the margin the checks keep for the backward's
    # split key tiles): n = 256 reaches 2^31, n = 128 does not (it then fails on the
    # 16-byte workspace instead)
    assert split(256) == 2
    assert split(128) == 5


def test_plan_table_is_keyed_by_the_whole_shape(lib):
    """attn_plan_set / attn_plan_get / attn_plan_clear on the CPU (no launch): a stored plan
    applies to exactly its shape; illegal plans are refused; clearing restores the rule."""
    lib.attn_plan_clear()
    base = lib.attn_plan_get(1, 4, 1000, 1000, 128, 1, 1)
    assert base >= 0
    neighbours = ((1, 4, 1000, 1001, 128, 1, 1), (1, 4, 1001, 1000, 128, 1, 1),
                  (2, 4, 1000, 1000, 128, 1, 1), (1, 4, 1000, 1000, 64, 1, 1),
                  (1, 4, 1000, 1000, 128, 0, 1), (1, 4, 1000, 1000, 128, 1, 2))
    rule = [lib.attn_plan_get(*a) for a in neighbours]
    other = 4 if base != 4 else 0   # plain schedule, head group 2 (or 1)
    assert lib.attn_plan_set(1, 4, 1000, 1000, 128, 1, 1, other) == 0
    assert lib.attn_plan_get(1, 4, 1000, 1000, 128, 1, 1) == other
    # any other key component (Sk, Sq, B, d, causal, dtype) still gets the rule's plan
    assert [lib.attn_plan_get(*a) for a in neighbours] == rule
    # the kernel name follows the stored plan's schedule
    assert lib.attn_plan_set(1, 4, 1000, 1000, 128, 1, 1, 2) == 0
    assert lib.attn_kernel_name(1, 4, 1000, 1000, 128, 1, 1, 0).startswith(b"attn_fwd_causal_pairs")
    assert lib.attn_block_m(1, 4, 1000, 1000, 128, 1, 1, 0) == 256
    assert lib.attn_plan_set(1, 4, 1000, 1000, 128, 1, 1, 3) == 0
    assert lib.attn_kernel_name(1, 4, 1000, 1000, 128, 1, 1, 0).startswith(b"attn_fwd_dual")
    assert lib.attn_plan_set(1, 4, 1000, 1000, 128, 1, 1, 8 + 0) == 0   # plain, head group 4
    assert lib.attn_plan_get(1, 4, 1000, 1000, 128, 1, 1) == 8
    # refused: pairs without causal, head group 8 not dividing B*H = 4, out of range, bad shape
    assert lib.attn_plan_set(1, 4, 1000, 1000, 128, 0, 1, 2) == 4
    assert lib.attn_plan_set(1, 4, 1000, 1000, 128, 1, 1, 12) == 4
    assert lib.attn_plan_set(1, 4, 1000, 1000, 128, 1, 1, 99) == 4
    assert lib.attn_plan_set(0, 4, 1000, 1000, 128, 1, 1, 0) == 2
    assert lib.attn_plan_get(1, 4, 1000, 1000, 128, 2, 1) == -1
    lib.attn_plan_clear()
    assert lib.attn_plan_get(1, 4, 1000, 1000, 128, 1, 1) == base


def test_tune_calls_refuse_bad_arguments_before_any_launch(lib):
    import ctypes
    out = ctypes.c_int(-7)
    assert lib.attn_tune(Q, K, V, O, L, 1, 2, 64, 64, 64, 0.125, 0, 1, 0, ctypes.byref(out), None) == 7
    assert lib.attn_tune(Q, K, V, O, L, 1, 2, 64, 64, 64, 0.125, 0, 1, 1001, ctypes.byref(out), None) == 7
    assert lib.attn_tune(None, K, V, O, L, 1, 2, 64, 64, 64, 0.125, 0, 1, 5, ctypes.byref(out), None) == 1
    assert lib.attn_tune(Q, K, V, O, L, 1, 2, 64, 64, 96, 0.125, 0, 1, 5, ctypes.byref(out), None) == 4
    assert lib.attn_tune_splitkv(Q, K, V, O, L, 1, 2, 64, 64, 64, 0.125, 0, 1, 1.0, 1.0, 1.0, 0,
                                 ctypes.byref(out), None) == 7
    assert lib.attn_tune_splitkv(Q, K, V, None, L, 1, 2, 64, 64, 64, 0.125, 0, 1, 1.0, 1.0, 1.0, 5,
                                 ctypes.byref(out), None) == 1
    assert out.value == -7
