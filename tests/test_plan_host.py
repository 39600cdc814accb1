"""Launch-plan logic of attn_fwd (host code in attn_internal.h), compiled with the host
C++ compiler and run on the CPU: which schedule each shape gets for a given CU count."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
BF16, FP8, F32 = 1, 2, 0


def host_cxx():
    """A host C++ compiler: g++ / c++, else ROCm's clang (the toolchain the library itself
    needs), so that these checks run wherever the library can be built."""
    for cand in (shutil.which("g++"), shutil.which("c++"), shutil.which("amdclang++"),
                 "/opt/rocm/llvm/bin/clang++"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("no host C++ compiler (g++, c++ or ROCm clang++) for the plan probes")


@pytest.fixture(scope="module")
def probe(tmp_path_factory):
    cxx = host_cxx()
    exe = str(tmp_path_factory.mktemp("plan") / "plan_probe")
    subprocess.run([cxx, "-std=c++17", "-O1", os.path.join(HERE, "plan_probe.cpp"), "-o", exe], check=True)

    def run(cases):
        text = "".join(" ".join(str(x) for x in c) + "\n" for c in cases)
        out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout
        return [tuple(int(v) for v in line.split()) for line in out.strip().splitlines()]
    return run


def test_long_sequence_workload(probe):
    # B=1, H=8, S=8192, d=128 on 256 CUs: 512 plain workgroups; causal -> 256 tile pairs
    nc, c = probe([(1, 8, 8192, 128, 0, BF16, 256), (1, 8, 8192, 128, 1, BF16, 256)])
    assert nc == (128, 0, 1)
    assert c == (256, 2, 1)


def test_many_heads_workload(probe):
    # B=8, H=32, S=2048, d=64: 4096 workgroups, 16 query tiles per head, 4 heads per group
    nc, c = probe([(8, 32, 2048, 64, 0, BF16, 256), (8, 32, 2048, 64, 1, BF16, 256)])
    assert nc == (128, 0, 4)
    assert c == (128, 0, 4)   # longest sweeps first: far more workgroups than CUs


def test_small_grids_use_two_groups(probe):
    out = probe([(1, 2, 300, 128, 0, BF16, 256), (1, 8, 128, 128, 0, FP8, 256),
                 (1, 2, 300, 64, 0, FP8, 256), (1, 2, 300, 128, 0, F32, 256)])
    assert out[0][1] == 3 and out[1][1] == 3     # bf16 d128, fp8 d128: two groups
    assert out[2][1] == 0 and out[3][1] == 0     # fp8 d64, fp32: no two-group kernel


def test_causal_orders(probe):
    out = probe([(1, 2, 700, 64, 1, FP8, 256),     # resident grid: complementary tiles
                 (4, 40, 700, 64, 1, BF16, 256),   # 960 workgroups: longest first
                 (1, 40, 1100, 128, 1, BF16, 256), # 360 tiles, 200 pairs: tile pairs (odd count)
                 (1, 4, 8192, 256, 1, BF16, 256),  # d = 256: no pair kernel; 1 per CU fits
                 (1, 8, 8192, 256, 1, BF16, 256),  # ... 2 per CU do not: longest first
                 (1, 3, 1100, 128, 1, BF16, 256),  # 27 tiles, one per CU: two groups per tile
                 (1, 16, 2048, 64, 1, BF16, 256),  # 256 tiles = the CUs: two groups per tile
                 (1, 16, 2048, 128, 1, FP8, 256)]) # fp8 d = 128 too
    assert out[0][1] == 1
    assert out[1][1] == 0
    assert out[2][:2] == (256, 2)
    assert out[3][1] == 1
    assert out[4][1] == 0
    assert out[5][:2] == (128, 3) and out[6][:2] == (128, 3) and out[7][:2] == (128, 3)


def test_without_a_device_query_plans_are_plain(probe):
    for case in [(1, 8, 8192, 128, 1, BF16, 0), (1, 2, 300, 128, 0, BF16, 0)]:
        assert probe([case])[0][:2] == (128, 0)


def test_head_group_divides_heads_and_fits_an_xcd(probe):
    # a group of heads divides B*H, its query tiles fit an XCD's 64 resident workgroups,
    # and it is at most an eighth of the heads (one XCD's share of the renumbered grid)
    for bh, nqt in [(256, 16), (8, 64), (6, 3), (7, 5), (12, 4), (1, 1), (16, 4), (128, 4), (64, 1)]:
        (_, _, g), = probe([(1, bh, nqt * 128, 64, 0, BF16, 1)])
        assert bh % g == 0 and (g == 1 or (g * nqt <= 64 and 8 * g <= bh))
        # largest such power of two
        assert not (bh % (2 * g) == 0 and 2 * g * nqt <= 64 and 16 * g <= bh)
    assert probe([(1, 16, 512, 64, 0, BF16, 1)])[0][2] == 2      # was 16: 4 XCDs per head
    assert probe([(8, 32, 2048, 64, 0, BF16, 1)])[0][2] == 4


@pytest.fixture(scope="module")
def split_probe(tmp_path_factory):
    cxx = host_cxx()
    exe = str(tmp_path_factory.mktemp("split") / "split_probe")
    subprocess.run([cxx, "-std=c++17", "-O1", os.path.join(HERE, "split_probe.cpp"), "-o", exe], check=True)

    def run(cases):
        text = "".join(" ".join(str(x) for x in c) + "\n" for c in cases)
        out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout
        return [int(v) for v in out.split()]
    return run


def test_split_count_follows_the_shape(split_probe):
    out = split_probe([
        (1, 8, 128, 32768, 256),   # the fp8 split workload: 8 query tiles -> 32 chunks of 1024 keys
        (8, 32, 2048, 2048, 256),  # 4096 workgroups unsplit: no split
        (1, 8, 128, 1500, 256),    # too few keys for two chunks of >= 1024
        (1, 8, 128, 4096, 256),    # chunks of >= 1024 keys cap the count at 4
        (1, 100, 128, 1 << 20, 256),  # 100 tiles: only 2 fit the 256 CUs
        (1, 1, 128, 1 << 20, 256),    # one tile: capped at 64 chunks
        (1, 8, 128, 32768, 0),     # no device: no split
        (1, 8, 128, 32768, 304),   # more CUs, same shape: still a power of two within the CUs
    ])
    assert out == [32, 1, 1, 4, 2, 64, 1, 32]


@pytest.fixture(scope="module")
def tune_probe(tmp_path_factory):
    cxx = host_cxx()
    exe = str(tmp_path_factory.mktemp("tune") / "tune_probe")
    subprocess.run([cxx, "-std=c++17", "-O1", os.path.join(HERE, "tune_probe.cpp"), "-o", exe], check=True)

    def run(lines):
        out = subprocess.run([exe], input="".join(l + "\n" for l in lines), capture_output=True,
                             text=True, check=True).stdout
        return out.strip().splitlines()
    return run


def test_tuning_candidates_are_the_legal_plans_default_first(tune_probe):
    # causal bf16 d=128, B=1, H=4, S=1000 on 256 CUs: 32 tiles, one per CU, so the rule
    # picks two groups per tile (plan 3); schedules 0 and 3 come with head groups 1, 2, 4
    # (dividing B*H = 4), 1 and 2 alone
    out = tune_probe(["cand 1 4 1000 128 1 1 256"])
    cand = [int(x) for x in out[0].split()]
    assert cand[0] == 3
    assert sorted(cand) == sorted([0, 4, 8, 1, 2, 3, 7, 11])
    # non-causal fp32: no dual, pair or complementary schedule; B*H = 6 allows head groups 1, 2
    cand = [int(x) for x in tune_probe(["cand 2 3 512 64 0 0 256"])[0].split()]
    assert sorted(cand) == [0, 4]


def test_plan_legality(tune_probe):
    cases = [
        ("legal 2 8 128 1 1", 1),    # tile pairs: causal bf16 d=128
        ("legal 2 8 256 1 1", 0),    # not for d=256
        ("legal 2 8 128 0 1", 0),    # not without the causal mask
        ("legal 1 8 64 1 2", 1),     # complementary tiles: any causal call
        ("legal 5 8 64 1 2", 0),     # ... which ignores head groups
        ("legal 3 8 128 0 2", 1),    # two groups: fp8 d=128
        ("legal 3 8 64 0 2", 0),     # but not fp8 d=64
        ("legal 3 8 64 0 0", 0),     # nor fp32
        ("legal 12 8 128 0 1", 1),   # plain with head group 8 dividing B*H = 8
        ("legal 16 8 128 0 1", 0),   # head group 16 does not divide 8
        ("legal 28 64 128 0 1", 0),  # out of range
        ("legal -1 8 128 0 1", 0),
    ]
    assert [int(x) for x in tune_probe([c for c, _ in cases])] == [r for _, r in cases]


def test_plan_choice_is_deterministic_with_a_margin_for_the_default(tune_probe):
    out = tune_probe([
        "choose 3 100 99 98.5",     # best beats the default by 1.5 %: the default stays
        "choose 3 100 97 97.5",     # 3 % faster: candidate 1
        "choose 3 100 97 97",       # equal times: the earlier candidate
        "choose 1 42",              # a single candidate
        "choose 4 100 110 90 90",   # ties after the default: the first of them
    ] * 2)                           # and the same answers when asked again
    assert out == ["0", "1", "1", "0", "2"] * 2


@pytest.fixture(scope="module")
def bwd_order_probe(tmp_path_factory):
    cxx = host_cxx()
    exe = str(tmp_path_factory.mktemp("bwd") / "bwd_order_probe")
    subprocess.run([cxx, "-std=c++17", "-O1", os.path.join(HERE, "bwd_order_probe.cpp"), "-o", exe], check=True)

    def run(shapes):
        text = "".join(f"{sq} {sk}\n" for sq, sk in shapes)
        out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout
        lines = out.strip().splitlines()
        res = []
        for kv, q in zip(lines[0::2], lines[1::2]):
            parse = lambda l: [tuple(int(x) for x in it.split(":")) for it in l.split()[1:]]  # noqa: E731
            res.append((parse(kv), parse(q)))
        return res
    return run


def test_causal_backward_items_run_longest_first(bwd_order_probe):
    # every work item (the two halves of each long tile, each other tile) appears exactly
    # once, and the sweep lengths never grow along the dispatch order
    shapes = [(8192, 8192), (700, 700), (2048, 2048), (1000, 1500), (1500, 1000), (128, 128), (300, 4096)]
    for (sq, sk), (kv, q) in zip(shapes, bwd_order_probe(shapes)):
        for items, ntile, nlong in ((kv, (sk + 127) // 128, None), (q, (sq + 127) // 128, None)):
            lens = [n for _, _, n in items]
            assert lens == sorted(lens, reverse=True), (sq, sk, items)
            halves = {(t, p) for t, p, _ in items if p >= 0}
            wholes = [t for t, p, _ in items if p < 0]
            split = {t for t, _ in halves}
            assert halves == {(t, p) for t in split for p in (0, 1)}
            assert sorted(wholes + sorted(split)) == list(range(ntile)), (sq, sk)
            assert len(items) == ntile + len(split)
    (kv, q), = bwd_order_probe([(8192, 8192)])
    # c3 shape: 43 long key tiles (sweeps of 256..88 query tiles of 32, more than a third
    # of 256; halves 128..44) and 43 long query tiles, merged with the whole sweeps of 84
    # and fewer
    assert sum(1 for _, p, _ in kv if p >= 0) == 86 and sum(1 for _, p, _ in q if p >= 0) == 86
    assert kv[:3] == [(0, 0, 128), (0, 1, 128), (1, 0, 126)]
    assert kv.index((43, -1, 84)) == kv.index((22, 1, 84)) + 1   # ties: the halves first
