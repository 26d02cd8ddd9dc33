"""Host-side checks of the C ABI (no GPU needed, no kernel launched).

The library must load and export every symbol ``include/mi355gemm.h`` declares;
argument validation and the configuration selector run before any HIP call, so their
decisions are checked here with fake (never dereferenced) pointer values.
"""
from __future__ import annotations

import os
import re
import subprocess

import pytest

import dense_fp16_gemm_fp32_amd as g

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mi355gemm.h")

# fake device addresses: only their alignment matters to the host logic
P16 = 0x7f0000000000          # 16-byte aligned
P2 = P16 + 2                  # only 2-byte aligned


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mi355gemm_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    declared = header_functions()
    assert len(declared) == 15
    assert sorted(g.EXPORTS) == declared
    lib = g.library()
    for name in declared:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", g.LIBRARY], stdout=subprocess.PIPE,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (mi355gemm_\w+)", out))
    assert set(declared) <= exported


def test_version_and_budget():
    assert "gfx950" in g.mi355gemm_version()
    assert g.mi355gemm_lds_budget() == 160 * 1024


def test_config_table_is_consistent():
    cfgs = g.configs()
    assert len(cfgs) == g.mi355gemm_num_configs() >= 4
    names = [c["name"] for c in cfgs]
    assert len(set(names)) == len(names)
    assert any(c["direct"] for c in cfgs) and any(not c["direct"] for c in cfgs)
    assert sorted(c["k_groups"] for c in cfgs if c["narrow"]) == [1, 4]
    for c in cfgs:
        if c["narrow"]:
            # 4 waves: waves_m groups of 8 rows, k_groups waves splitting K for each, over
            # 512-wide k-blocks and 8 columns; LDS holds only the k-groups' partial sums
            # (one fp32 per lane and wave); any alignment
            assert c["waves_m"] * c["k_groups"] == 4 and c["waves_n"] == 1
            assert (c["block_m"], c["block_n"], c["block_k"]) == (8 * c["waves_m"], 8, 512)
            assert c["threads"] == 256
            assert c["lds_bytes"] == (4 * 64 * 4 if c["k_groups"] > 1 else 0)
            assert c["a_vector"] == 0 and c["bc_vector"] == 0 and c["direct"] == 0
            assert c["mfma_block"] == 0
            continue
        if c["direct"]:
            # ring of STAGES buffers of the A (BM x BK) and B (BK x BN) tiles, XOR-swizzled;
            # A may have any alignment (unaligned LDS-DMA, K tail patched), B and C not
            assert c["lds_bytes"] == c["stages"] * (c["block_m"] + c["block_n"]) * c["block_k"] * 2
            assert c["a_vector"] == 0 and c["bc_vector"] == 1
        else:
            # two LDS stages of BM and BN rows of BK halves plus a 16-byte pad per row
            assert c["lds_bytes"] == c["stages"] * (c["block_m"] + c["block_n"]) * (c["block_k"] + 8) * 2
        assert c["lds_bytes"] <= g.mi355gemm_lds_budget()
        assert c["threads"] == 64 * (c["waves_m"] * c["waves_n"] * c["k_groups"] + c["loader_waves"])
        # loader waves: direct kernel, one k-group, named d..._l<loaders>_s<stages>
        assert c["loader_waves"] in (0, 4)
        if c["loader_waves"]:
            assert c["direct"] and not c["pingpong"] and c["k_groups"] == 1
            assert "_l%d_s" % c["loader_waves"] in c["name"]
        else:
            assert "_l" not in c["name"]
        assert c["k_groups"] in (1, 2) and (c["direct"] or c["k_groups"] == 1)
        mf = c["mfma_block"]
        assert mf in (16, 32) and (mf == 32 or (c["direct"] and c["k_groups"] == 1))
        assert ("_mf16" in c["name"]) == (mf == 16)
        assert c["block_m"] % (mf * c["waves_m"]) == 0 and c["block_n"] % (mf * c["waves_n"]) == 0
        assert c["block_k"] % 16 == 0
        # ping-pong: the direct loader with two groups of 4 waves, K % 8 == 0 only
        assert c["k_mult8"] == c["pingpong"]
        if c["pingpong"]:
            assert c["direct"] == 1 and c["threads"] == 512 and c["name"].startswith("p")
    assert g.mi355gemm_config_name(-1) is None
    assert g.mi355gemm_config_name(len(cfgs)) is None
    with pytest.raises(g.GemmError):
        g.mi355gemm_config_info(len(cfgs))


def _status(M, N, K, A=P16, B=P16, C=P16, bias=None, epi=0, config=None):
    if config is None:
        return g.mi355gemm_gemm(M, N, K, A, B, C, bias, epi, None)
    return g.mi355gemm_gemm_config(M, N, K, A, B, C, bias, epi, None, config)


@pytest.mark.parametrize("args,want", [
    (dict(M=-1, N=4, K=4), g.EINVAL),
    (dict(M=4, N=-1, K=4), g.EINVAL),
    (dict(M=4, N=4, K=-1), g.EINVAL),
    (dict(M=4, N=4, K=4, epi=3), g.EINVAL),
    (dict(M=4, N=4, K=4, epi=-1), g.EINVAL),
    (dict(M=4, N=4, K=4, C=None), g.EINVAL),
    (dict(M=4, N=4, K=4, A=None), g.EINVAL),
    (dict(M=4, N=4, K=4, B=None), g.EINVAL),
    (dict(M=4, N=4, K=4, epi=1), g.EINVAL),          # bias epilogue without bias
    (dict(M=4, N=4, K=4, epi=2), g.EINVAL),
    (dict(M=4, N=4, K=4, A=P16 + 1), g.EINVAL),      # odd address
    (dict(M=4, N=4, K=4, C=P16 + 1), g.EINVAL),
    (dict(M=4, N=4, K=4, bias=P16 + 1, epi=2), g.EINVAL),
    (dict(M=4, N=4, K=1 << 22), g.EUNSUPPORTED),
    (dict(M=4, N=1 << 22, K=4), g.EUNSUPPORTED),
    (dict(M=4, N=4, K=4, config=99), g.EINVAL),
    (dict(M=4, N=4, K=4, config=-5), g.EINVAL),
])
def test_validation_errors(args, want):
    assert _status(**args) == want
    assert g.mi355gemm_last_error() != ""


@pytest.mark.parametrize("args,want", [
    (dict(M=-1, N=4, K=4), g.EINVAL),
    (dict(M=4, N=4, K=4, C=None), g.EINVAL),
    (dict(M=4, N=4, K=4, epi=2), g.EINVAL),          # bias epilogue without bias
    (dict(M=4, N=4, K=4, A=P16 + 1), g.EINVAL),
    (dict(M=4, N=1 << 22, K=4), g.EUNSUPPORTED),
    (dict(M=4, N=4, K=4, config=99), g.EINVAL),
    (dict(M=4, N=4, K=4, config=-2), g.EINVAL),      # -1 is the selector's choice
])
def test_timed_entry_validates_like_the_others(args, want):
    """mi355gemm_gemm_timed checks its arguments as mi355gemm_gemm_config does, before any
    HIP call (the events are never touched on an error)."""
    a = dict(M=4, N=4, K=4, A=P16, B=P16, C=P16, bias=None, epi=0, config=-1)
    a.update(args)
    st = g.mi355gemm_gemm_timed(a["M"], a["N"], a["K"], a["A"], a["B"], a["C"], a["bias"],
                                a["epi"], None, a["config"], None, None)
    assert st == want
    assert g.mi355gemm_last_error() != ""


def test_empty_problems_are_ok_without_launch():
    # M == 0 or N == 0: nothing to compute, OK even with NULL pointers
    assert _status(0, 16, 16, A=None, B=None, C=None) == g.OK
    assert _status(16, 0, 16, A=None, B=None, C=None) == g.OK
    assert _status(0, 0, 0, A=None, B=None, C=None, epi=2) == g.OK
    assert g.mi355gemm_last_error() == ""
    # the timed entry with nothing to launch records no event (none is passed here)
    assert g.mi355gemm_gemm_timed(0, 16, 16, None, None, None, None, 0, None, -1, None, None) == g.OK


def test_forced_vector_config_rejects_unaligned_shapes():
    vec = [c for c in g.configs() if c["a_vector"]]
    bc = [c for c in g.configs() if c["bc_vector"]]
    assert vec and bc
    assert _status(100, 64, 777, config=vec[0]["id"]) == g.EUNSUPPORTED       # K % 8 != 0
    assert "K % 8" in g.mi355gemm_last_error()
    assert _status(100, 64, 64, A=P2, config=vec[0]["id"]) == g.EUNSUPPORTED  # A misaligned
    assert _status(100, 60, 64, config=bc[0]["id"]) == g.EUNSUPPORTED        # N % 8 != 0
    assert _status(100, 64, 64, C=P2, config=bc[0]["id"]) == g.EUNSUPPORTED


def _select(M, N, K, epi=0, A=P16, B=P16, C=P16, bias=P16):
    return g.mi355gemm_select(M, N, K, epi, A, B, C, bias)


def _cfg(i):
    return g.mi355gemm_config_info(i)


def test_select_for_the_workload_shapes():
    import workloads
    for w in workloads.WORKLOADS:
        for epi_name in w.epilogues:
            epi = g.EPILOGUES[epi_name]
            i = _select(w.M, w.N, w.K, epi)
            assert i >= 0, w.name
            c = _cfg(i)
            if w.K % 8 != 0:
                assert c["a_vector"] == 0, w.name     # ragged K: A may not need 16-byte rows
            assert c["bc_vector"] == (1 if w.N % 8 == 0 else 0), w.name
            # every workload takes the direct kernel (256^3 its 64x128 tile, 8 of them)
            assert c["direct"] == 1, w.name
    # large square problems take the widest tile; 2048^3 must still fill 256 CUs
    big = _cfg(_select(8192, 8192, 8192))
    assert (big["block_m"], big["block_n"]) == (256, 256)
    four = _cfg(_select(4096, 4096, 4096))          # 256 tiles of 256x256: one per CU
    assert (four["block_m"], four["block_n"]) == (256, 256)
    mid = _cfg(_select(2048, 2048, 2048))
    tiles = (2048 // mid["block_m"]) * (2048 // mid["block_n"])
    assert tiles >= 256


def test_select_routes_misaligned_pointers_to_narrow_loads():
    c = _cfg(_select(512, 512, 512, A=P2))
    assert c["a_vector"] == 0 and c["bc_vector"] == 1
    c = _cfg(_select(2048, 2048, 2048, A=P2))        # A misaligned: still the direct kernel
    assert c["direct"] == 1
    c = _cfg(_select(1000, 3000, 777))                # the ragged workload: direct, K tail patched
    assert c["direct"] == 1
    # a handful of tiles (no direct launch to split): the register-staged kernel with
    # narrow B / C accesses
    c = _cfg(_select(128, 256, 256, B=P2))
    assert c["bc_vector"] == 0
    c = _cfg(_select(128, 256, 256, C=P2))
    assert c["bc_vector"] == 0
    c = _cfg(_select(128, 256, 256, epi=2, bias=P16 + 4))  # bias only 4-byte aligned
    assert c["bc_vector"] == 0
    c = _cfg(_select(128, 250, 256))                      # N % 8 != 0
    assert c["bc_vector"] == 0
    c = _cfg(_select(512, 512, 512, B=P2))                # enough tiles: direct, split launch
    assert c["direct"] == 1


def test_select_rejects_invalid_and_empty():
    assert _select(-1, 4, 4) == -1
    assert _select(4, 4, 4, epi=7) == -1
    assert _select(0, 4, 4) == -1


def test_selected_config_always_passes_its_own_checks():
    # every choice the selector makes must be one the forced path accepts; probe with a
    # forced call that fails validation late (bad epilogue) to stay launch-free
    for shape in [(1, 1, 1), (33, 65, 17), (1000, 3000, 777), (2048, 2048, 2048),
                  (8192, 8192, 8192), (4096, 1024, 4096), (100, 8, 8)]:
        for A in (P16, P2):
            i = _select(*shape, A=A)
            c = _cfg(i)
            M, N, K = shape
            if c["a_vector"]:
                assert K % 8 == 0 and A % 16 == 0
            if c["bc_vector"]:
                assert N % 8 == 0


def _tuned_entries():
    import re
    path = os.path.join(ROOT, "dense_fp16_gemm_fp32_amd", "csrc", "tuned_table.inc")
    text = open(path).read()
    rows = re.findall(r'^\{(\d+), (\d+), (\d+), (\d), ([01]), ([01]), "([^"]+)"\},\s*$', text, re.M)
    # every non-comment line must be an entry of that exact form
    body = [l for l in text.splitlines() if l.strip() and not l.strip().startswith("//")]
    assert len(body) == len(rows), body
    return [(int(a), int(b), int(c), int(d), int(e), int(f), name) for a, b, c, d, e, f, name in rows]


def test_tuned_table_entries_name_real_configs_and_drive_the_selector():
    names = {c["name"] for c in g.configs()}
    for M, N, K, epi, av, bv, name in _tuned_entries():
        assert name in names, name
        A = P16 if av else P2          # fake pointers with the entry's alignment class
        B = C = P16 if bv else P2
        i = _select(M, N, K, epi, A=A, B=B, C=C, bias=P16 if bv else P2)
        assert g.mi355gemm_config_name(i) == name, (M, N, K, epi, av, bv)


def test_tuner_writes_entries_only_for_wins_above_the_margin():
    from dense_fp16_gemm_fp32_amd import tune
    res = [
        {"M": 64, "N": 64, "K": 64, "epilogue": "none", "a_vector": 1, "bc_vector": 1,
         "rule": "a", "best": "b", "entry": True, "median_us": {"a": 10.0, "b": 9.0}},
        {"M": 32, "N": 64, "K": 8, "epilogue": "bias_gelu", "a_vector": 0, "bc_vector": 1,
         "rule": "a", "best": "a", "entry": False, "median_us": {"a": 5.0}},
    ]
    src = tune.table_source(res, "test device")
    body = [l for l in src.splitlines() if not l.startswith("//")]
    assert body == ['{64, 64, 64, 0, 1, 1, "b"},']
    assert tune.parse_shape("1000x3000x777:bias_gelu:uniform") == (1000, 3000, 777, "bias_gelu", "uniform")
    assert tune.parse_shape("8x16x24") == (8, 16, 24, "none", "normal")


@pytest.mark.parametrize("args,want", [
    (dict(n=-1), g.EINVAL),
    (dict(n=0), g.OK),
    (dict(n=0, a=None, b=None, c=None), g.OK),
    (dict(n=8, a=None), g.EINVAL),
    (dict(n=8, c=None), g.EINVAL),
    (dict(n=8, b=P16 + 1), g.EINVAL),
])
def test_vector_add_argument_checks(args, want):
    a = dict(n=0, a=P16, b=P16, c=P16)
    a.update(args)
    assert g.mi355gemm_vector_add(a["n"], a["a"], a["b"], a["c"], None) == want


@pytest.mark.parametrize("args,want", [
    (dict(M=-1), g.EINVAL),
    (dict(N=-1), g.EINVAL),
    (dict(M=0, x=None, y=None), g.OK),
    (dict(N=0, x=None, y=None), g.OK),
    (dict(x=None), g.EINVAL),
    (dict(y=P16 + 1), g.EINVAL),
    (dict(N=1 << 31), g.EUNSUPPORTED),
])
def test_softmax_argument_checks(args, want):
    a = dict(M=4, N=8, x=P16, y=P16)
    a.update(args)
    # every case here fails validation or has nothing to do, so nothing is launched
    assert g.mi355gemm_softmax(a["M"], a["N"], a["x"], a["y"], None) == want


@pytest.mark.parametrize("args,want", [
    (dict(B=-1), g.EINVAL),
    (dict(Sk=-1), g.EINVAL),
    (dict(D=96), g.EUNSUPPORTED),
    (dict(D=256), g.EUNSUPPORTED),
    (dict(B=0, q=None, k=None, v=None, o=None), g.OK),
    (dict(H=0), g.OK),
    (dict(Sq=0, q=None), g.OK),
    (dict(Sk=0), g.EINVAL),
    (dict(scale=0.0), g.EINVAL),
    (dict(scale=-0.1), g.EINVAL),
    (dict(scale=float("inf")), g.EINVAL),
    (dict(scale=float("nan")), g.EINVAL),
    (dict(causal=2), g.EINVAL),
    (dict(v=None), g.EINVAL),
    (dict(o=P2), g.EINVAL),
    (dict(k=P16 + 8), g.EINVAL),
    (dict(lse=P16 + 2), g.EINVAL),
    (dict(Sq=(1 << 23)), g.EUNSUPPORTED),
    (dict(Sk=(1 << 23)), g.EUNSUPPORTED),
    (dict(B=1 << 16, H=1 << 15), g.EUNSUPPORTED),
])
def test_attention_argument_checks(args, want):
    a = dict(B=2, H=3, Sq=64, Sk=64, D=128, q=P16, k=P16, v=P16, o=P16, lse=None,
             scale=0.125, causal=0)
    a.update(args)
    # every case here fails validation or has nothing to do, so nothing is launched
    st = g.mi355gemm_attention(a["B"], a["H"], a["Sq"], a["Sk"], a["D"], a["q"], a["k"], a["v"],
                               a["o"], a["lse"], a["scale"], a["causal"], None)
    assert st == want, g.mi355gemm_last_error()


@pytest.mark.parametrize("shape,want", [
    ((8192, 8192, 8192), "p256x256x32_w2x4_s4"),      # four waves of 256 x 256 tiles: ping-pong
    ((16384, 8192, 4096), "p256x256x32_w2x4_s4"),
    ((4096, 4096, 4096), "p256x256x32_w2x4_s4"),      # one wave of them
    ((16384, 2048, 1024), "p256x256x32_w2x4_s4"),
    ((2048, 8192, 4096), "p256x256x32_w2x4_s4"),
    ((8192, 8192, 8190), "d256x256x32_w2x2_s4"),      # K % 8 != 0: no ping-pong kernel
    ((4096, 4096, 4095), "d256x256x64_w2x4_s2"),
    ((8192, 1024, 8192), "d256x128x64_w2x2k2_s3"),    # one GPU's N share of 8192^3
    ((1024, 8192, 8192), "d256x128x64_w2x2k2_s3"),    # its M share
    ((2048, 2048, 8192), "d128x128x64_w2x2_l4_s4"),   # 256 tiles: 4 loader waves feed the
    ((2048, 2048, 4096), "d128x128x64_w2x2_l4_s4"),   # 4 multiplying ones; 64-deep stages
    ((2048, 2048, 2048), "d128x128x32_w2x2_l4_s4"),   # from K = 4096, 32-deep below
    ((2048, 2048, 1024), "d128x128x32_w2x2_l4_s4"),
    ((2048, 2048, 777), "d64x256x32_w1x4_s4"),        # one wave of 128x128 tiles, K < 1024
    ((2048, 2048, 512), "d64x256x32_w1x4_s4"),
    ((3072, 2048, 512), "d128x128x32_w2x2_s4"),       # 1.5 waves of them, K < 1024
    ((1024, 1024, 1024), "d64x128x32_w1x4_s4"),       # 64 tiles of 128x128, 128 of 64x128
    ((512, 4096, 1024), "d64x128x32_w1x4_s4"),
    ((768, 768, 768), "d64x128x32_w1x4_s4"),
    ((1024, 1024, 4096), "d128x128x64_w2x2k2_s4"),    # 64 tiles, long K
    ((1536, 1536, 1024), "d128x128x64_w2x2k2_s4"),    # 144 tiles (288 of 64x128)
    ((3072, 3072, 2048), "d256x256x32_w2x4_s4"),      # 144 of 256x256 in one round, not
    ((4096, 2304, 4096), "d256x256x32_w2x4_s4"),      # 288 of 256x128 in two
    ((6144, 2048, 2048), "d256x256x32_w2x4_s4"),      # 192 of 256x256, not 384 of 256x128
    ((2304, 2304, 2304), "d256x128x64_w2x2k2_s3"),    # 162 of 256x128, not 324 of 128x128
    ((3072, 2048, 2048), "d256x128x64_w2x2k2_s3"),    # 192 of 256x128, not 384 of 128x128
    ((1000, 3000, 777), "d64x192x32_w1x4_l4_s4_mf16"),   # a full wave of 64x192 tiles (192
    ((1000, 3000, 1024), "d64x192x32_w1x4_l4_s4_mf16"),  # of 64x256 or 128x128): 32-deep
    ((2048, 1536, 512), "d64x192x32_w1x4_l4_s4_mf16"),   # stages up to K = 1024,
    ((4096, 768, 1024), "d64x192x32_w1x4_l4_s4_mf16"),
    ((1024, 3072, 768), "d64x192x32_w1x4_l4_s4_mf16"),
    ((1000, 3000, 1536), "d64x192x64_w1x4_l4_s3_mf16"),  # 64-deep ones up to 2048
    ((1000, 3000, 2048), "d64x192x64_w1x4_l4_s3_mf16"),
    ((2048, 1536, 2048), "d64x192x64_w1x4_l4_s3_mf16"),
    ((1000, 3000, 4096), "d128x128x64_w2x2k2_s4"),    # the same tile counts, longer K
    ((1280, 2304, 1024), "d128x128x64_w2x2k2_s4"),    # 240 tiles of 64x192: not enough
    ((3000, 1000, 777), "d64x256x32_w1x4_s4"),        # 282 of 64x192: a second round
    ((256, 256, 256), "d64x128x32_w1x4_s4"),          # 8 tiles of 64x128
    ((128, 256, 256), "s64x64x64_w2x1_av_bv"),        # a handful of tiles
])
def test_selector_rules_pick_the_measured_winners(shape, want):
    """The rules' choice for shapes the interleaved tuner measured (they have no table
    entry: the rule already picks the winner)."""
    M, N, K = shape
    assert g.mi355gemm_config_name(_select(M, N, K)) == want


@pytest.mark.parametrize("shape,ptr_off,want", [
    ((2048, 2047, 2048), 0, "d128x128x32_w2x2_l4_s4"),  # odd N: direct on the first 2040 columns
    ((8192, 8191, 8192), 0, "d256x256x32_w2x2_s4"),
    ((1000, 3001, 777), 0, "d64x192x32_w1x4_l4_s4_mf16"),
    ((2048, 2048, 2048), 2, "d128x128x32_w2x2_l4_s4"),  # B and C only 2-byte aligned
    ((8192, 63, 8192), 0, "s64x64x64_w2x1_av_bn"),    # N < 64: no direct launch to split
    ((64, 775, 64), 0, "s64x64x64_w2x1_av_bn"),       # too few tiles (7 of 64x128)
    ((512, 1031, 64), 0, "d64x128x32_w1x4_s4"),       # 72 tiles of 64x128
])
def test_selector_splits_unfriendly_rows(shape, ptr_off, want):
    """Rows of B and C that are not 16-byte friendly keep the direct kernel from N >= 64
    with enough tiles (the call adds the narrow kernel for the last N % 8 columns)."""
    M, N, K = shape
    cid = g.mi355gemm_select(M, N, K, 2, P16, P16 + ptr_off, P16 + ptr_off, P16)
    assert g.mi355gemm_config_name(cid) == want, g.mi355gemm_last_error()


@pytest.mark.parametrize("shape,c_off,want", [
    ((8192, 1, 8192), 0, "n8x8x512_w1x1k4"),       # at most 8 columns: the narrow kernel,
    ((2048, 7, 2048), 0, "n8x8x512_w1x1k4"),       # 4 waves splitting K below 16384 rows,
    ((1024, 3, 65536), 0, "n8x8x512_w1x1k4"),
    ((16384, 1, 4096), 0, "n32x8x512_w4x1"),       # 4 row groups from 16384 rows
    ((131072, 5, 512), 0, "n32x8x512_w4x1"),
    ((2048, 8, 2048), 0, "n8x8x512_w1x1k4"),       # N = 8 below the direct kernel's 64 tiles
    ((16384, 8, 4096), 0, "d128x128x64_w2x2k2_s4"),  # N = 8, enough tiles: direct
    ((16384, 8, 4096), 2, "n32x8x512_w4x1"),       # the same with C only 2-byte aligned
])
def test_selector_narrow_rules(shape, c_off, want):
    M, N, K = shape
    cid = g.mi355gemm_select(M, N, K, 0, P16, P16, P16 + c_off, None)
    assert g.mi355gemm_config_name(cid) == want, g.mi355gemm_last_error()


def test_forced_narrow_config_rejects_more_than_8_columns():
    for c in g.configs():
        if c["narrow"]:
            assert _status(64, 9, 64, config=c["id"]) == g.EUNSUPPORTED
            assert "at most 8 columns" in g.mi355gemm_last_error()


# ---- choices installed at run time ----------------------------------------------------

def test_installed_choice_overrides_the_selector_for_its_exact_key_only():
    k32, k64 = g.config_id("d128x128x32_w2x2_s4"), g.config_id("d128x128x64_w2x2_s4")
    rule = g.config_id("d128x128x32_w2x2_l4_s4")
    g.clear_choices()
    try:
        assert _select(2048, 2048, 2048) == rule                     # the rules
        g.set_choice(2048, 2048, 2048, "none", True, True, "d128x128x32_w2x2_s4")
        assert _select(2048, 2048, 2048) == k32
        assert _select(2048, 2048, 2048, epi=2) == rule               # other epilogue
        assert _select(2048, 2048, 2056) == rule                      # other shape
        assert _select(2048, 2048, 2048, A=P2) != k32                 # other A class
        g.set_choice(2048, 2048, 2048, "none", True, True, k64)       # same key: replaced
        assert _select(2048, 2048, 2048) == k64
        # a class-0 entry (rows not 16-byte friendly) names a configuration without
        # 16-byte row needs, as the measured table's entries do
        staged = g.config_id("s64x64x64_w2x1_an_bn")
        g.set_choice(1000, 3001, 777, "bias_gelu", False, False, staged)
        assert _select(1000, 3001, 777, epi=2) == staged
        ragged = g.config_id("d64x192x32_w1x4_l4_s4_mf16")
        assert _select(1000, 3000, 777, epi=2) == ragged              # class 1: the rules
        g.clear_choices()
        assert _select(2048, 2048, 2048) == rule
        assert _select(1000, 3001, 777, epi=2) == ragged
    finally:
        g.clear_choices()


def test_set_choice_rejects_bad_arguments():
    k64 = g.config_id("d128x128x64_w2x2_s4")
    vec = [c["id"] for c in g.configs() if c["a_vector"]][0]
    narrow = [c["id"] for c in g.configs() if c["narrow"]][0]
    lib_status = g.mi355gemm_set_choice
    g.clear_choices()
    try:
        assert lib_status(-1, 8, 8, 0, 1, 1, k64) == g.EINVAL
        assert lib_status(8, 8, 8, 3, 1, 1, k64) == g.EINVAL
        assert lib_status(8, 8, 8, 0, 2, 1, k64) == g.EINVAL
        assert lib_status(8, 8, 8, 0, 1, 1, -1) == g.EINVAL
        assert lib_status(8, 8, 8, 0, 1, 1, g.mi355gemm_num_configs()) == g.EINVAL
        assert lib_status(8, 8, 8, 0, 0, 1, vec) == g.EUNSUPPORTED    # needs 16-byte A rows
        assert lib_status(8, 8, 8, 0, 1, 0, k64) == g.EUNSUPPORTED    # needs 16-byte B/C rows
        assert lib_status(8, 9, 8, 0, 1, 0, narrow) == g.EUNSUPPORTED # 9 > 8 columns
        assert lib_status(8, 8, 8, 0, 1, 1, narrow) == g.OK
        with pytest.raises(g.GemmError):
            g.set_choice(8, 8, 8, "none", True, True, -5)
    finally:
        g.clear_choices()


def test_set_choice_table_holds_64_entries():
    k64 = g.config_id("d128x128x64_w2x2_s4")
    g.clear_choices()
    try:
        for i in range(64):
            assert g.mi355gemm_set_choice(128, 128, 64 * (i + 1), 0, 1, 1, k64) == g.OK
        assert g.mi355gemm_set_choice(128, 128, 64 * 65, 0, 1, 1, k64) == g.EUNSUPPORTED
        assert g.mi355gemm_set_choice(128, 128, 64, 0, 1, 1, k64) == g.OK   # replacing is fine
        assert _select(128, 128, 64 * 64) == k64
    finally:
        g.clear_choices()
