"""Host-side (CPU) models of GPU index arithmetic, built from the kernels' own
host-callable helpers (no GPU call is made).

Unit decoding: the per-segment tile table each workgroup builds (SegTable,
decode_unit_seg) gives, for every unit, the segment, rows, columns and K range
that the earlier tile list (decode_unit_plain over build_tiles_kernel's list)
gave; so the split of the work, and the results, are unchanged.

Tile kinds 0, 2, 3, 4 and 5 (short tails attached to whole 256-row tiles):
the units decoded from the table, reached the way the kernels' workgroups
reach them (each XCD's slices of whole and K-part units, xcd_slice), cover
every (row, column tile, K step) of every segment exactly once.

fp8 64-row tile: every operand load of every unit, for reduction lengths with
odd 64-K step counts (K = 320) and the decode shapes' K-split parts (K = 4096,
14336), must stay inside its allocation once the buffer range check has let
it through.  The same model without the half-step rule finds loads past the
end (the hazard the rule removes), which shows the model can see it."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "host_model", "fp8_offsets.hip")


@pytest.fixture(scope="module")
def fp8_model(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("host_model") / "fp8_offsets")
    hipcc = "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    r = subprocess.run([hipcc, "-x", "hip", "--cuda-host-only", "-O1", "-std=c++17", "-I",
                        os.path.join(ROOT, "include"), SRC, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def _run(exe, mode, K, Nn, rows):
    out = subprocess.run([exe, mode, str(K), str(Nn), *map(str, rows)], capture_output=True, text=True,
                         check=True).stdout
    return dict(kv.split("=") for kv in out.split())


CASES = [
    ("down", 320, 256, [3, 7, 0, 64, 65, 1, 2]),          # K/64 odd: every unit ends on a half step
    ("up", 320, 384, [70, 3, 130, 1]),
    ("up", 4096, 14336, [5] * 5),                         # decode up: K-parts of odd length at the end
    ("up", 4096, 14336, [2, 3, 1, 4, 8, 5, 7]),
    ("down", 14336, 4096, [40] * 3),                      # decode down: s = 5 parts, the last one odd
    ("down", 14336, 4096, [40] * 5),
    ("down", 14336, 4096, [2, 3, 1, 4, 8, 5, 7]),
    ("down", 2048, 7168, [9, 26, 31, 0, 64, 1]),
    ("up", 4096, 14336, [4] * 8),                         # decode: 896 tiles = 3 rounds + 128 tiles in 2 K-parts
    ("up", 4096, 14336, [1003, 1073, 1024, 1017, 1040, 1029, 1000, 1006]),   # Mixtral prefill: 256-row tiles + tails
    ("down", 14336, 4096, [4926, 0, 7, 130, 127, 128, 255, 256, 257, 383, 384, 1]),
]


@pytest.mark.parametrize("mode,K,Nn,rows", CASES)
def test_fp8_loads_in_bounds(fp8_model, mode, K, Nn, rows):
    r = _run(fp8_model, mode, K, Nn, rows)
    assert int(r["units"]) > 0 and int(r["checked"]) > 0
    assert int(r["oob"]) == 0, r
    assert int(r["list_mismatch"]) == 0, r      # the LDS table decodes the units the tile list did
    assert int(r["kind0_mismatch"]) == 0, r     # also for 256-row + 64-row tiles (bf16)
    assert int(r["cover_bad"]) == 0, r          # every tile kind covers each row, column tile, K step once


def test_attached_tails_are_exercised(fp8_model):
    """The coverage check of tile kind 5 (short tails attached to whole 256-row tiles)
    must see attached rows in the cases that have such tails."""
    r = _run(fp8_model, "up", 4096, 14336, [1003, 1073, 1024, 1017, 1040, 1029, 1000, 1006])
    assert int(r["attached"]) == 49 + 16 + 5, r      # the tails of 1073, 1040 and 1029 rows
    r = _run(fp8_model, "down", 14336, 4096, [4926, 0, 7, 130, 127, 128, 255, 256, 257, 383, 384, 1])
    assert int(r["attached"]) == 62 + 1 + 32, r      # 4926 and 257 whole; 32 of 383's 127 (one 256-row tile)


# Segment sizes of the GPU test of attached tails (tails of 1 to 127 rows on one or two whole
# tiles, a tail of exactly kBigTailMin, segments with no whole tile); 16 column tiles each way.
ATTACH_EDGE_ROWS = [257, 270, 287, 288, 289, 300, 340, 383, 513, 550, 576, 600, 639, 384, 0, 1, 64, 127, 128]


@pytest.mark.parametrize("mode,K,Nn", [("up", 4096, 2048), ("down", 2048, 4096)])
def test_attach_edge_sizes_select_attaching_tiles(fp8_model, mode, K, Nn):
    """The forward kernels' own tail rule picks the attaching tile kind for the GPU test's
    segment sizes (21 whole tiles, 34 with every tail as a whole tile: 2 against 3 rounds
    of 256 workgroups), which attaches 437 rows, so that test runs that kind."""
    r = _run(fp8_model, mode, K, Nn, ATTACH_EDGE_ROWS)
    assert int(r["auto_kind"]) == 5, r
    assert int(r["attached"]) == 437, r
    assert int(r["cover_bad"]) == 0, r


def test_fp8_model_sees_the_half_step_hazard(fp8_model):
    hits = [int(_run(fp8_model, *c)["nohalf_oob"]) for c in CASES]
    assert hits[0] > 0 and hits[4] > 0, hits
