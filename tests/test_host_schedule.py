"""The library's host-side scheduling logic, checked without a GPU.

``schedule_check.cpp`` is built with hipcc against the library's own headers
and ``csrc/tile_select.cpp`` and run here:

* the workgroup -> unit map is a bijection for every grid of 1..20000
  workgroups, and each XCD's workgroups take consecutive units;
* the compute-unit pairing keeps it a bijection and gives the two
  workgroups of a compute unit adjacent units (a long and a short item),
  for 32 and 38 compute units per XCD;
* item -> (slice, query block) is a bijection, and causal items 2i and 2i+1
  of a slice take num_qb + 1 key tiles together (equal-length pairs);
* the items-per-unit rule on the cases it distinguishes;
* the tile selector on the table of shapes the GPU test checks on a 256-CU
  device (``test_gpu_tiles.SELECTOR_CASES``), and the rule that d_v != d_k
  or a mask keeps the default geometry except for key-length pairs.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "transformer_scaled_dot_sdpa_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    if not (os.path.exists(HIPCC) or shutil.which(HIPCC)):
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("schedule") / "schedule_check")
    cmd = [HIPCC, "-x", "hip", "--offload-arch=gfx950", "-std=c++17", "-O1",
           "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
           os.path.join(ROOT, "tests", "schedule_check.cpp"), os.path.join(CSRC, "tile_select.cpp"),
           "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]

    def run(text: str) -> str:
        p = subprocess.run([out], input=text, capture_output=True, text=True, timeout=300)
        assert p.returncode == 0, p.stderr
        return p.stdout
    return run


def test_schedule_maps(checker):
    # each line: name, count of violations, [label, value ...]
    res = {}
    for line in checker("maps\n").splitlines():
        parts = line.split()
        res[parts[0]] = [int(x) for x in parts[1::2]]
    assert res["unit_map"] == [0]
    bad, active = res["cu_pairs"]
    assert bad == 0
    assert active > 100          # the pairing applied in many grids
    assert res["item_block_causal"] == [0]
    assert res["item_block_plain"] == [0]
    assert res["items_per_unit"] == [0]


def test_selector_table(checker):
    from test_gpu_tiles import SELECTOR_CASES
    lines = []
    for (B, H, Lq, Lk, d, causal, lens), _ in SELECTOR_CASES:
        lines.append(f"{d} {int(causal)} {int(lens)} {B * H} {Lq} {Lk} 256 0")
    got = checker("\n".join(lines) + "\n").split()
    assert got == [e for _, e in SELECTOR_CASES], list(zip(got, [e for _, e in SELECTOR_CASES]))


def test_selector_general_calls_keep_default_geometry(checker):
    # a shape that picks the key split, the 8-wavefront tile and the pairs
    # tile, each asked again as a general call (d_v != d_k or a mask)
    q = ["128 1 0 8 4096 4096 256 1",      # key split -> default
         "128 0 0 80 512 512 256 1",       # 8 wavefronts -> default
         "128 0 1 128 1024 1024 256 1",    # key-length pairs stay
         "96 0 0 8 128 128 256 0"]         # no such head size
    got = checker("\n".join(q) + "\n").split()
    assert got == ["bf16_d128_bc64_w4", "bf16_d128_bc64_w4", "bf16_d128_bc64_w4_pairs", "none"]
