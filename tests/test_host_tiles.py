"""The launchers' inline tile rules (qg_launch.h), run on the host.

`tests/host_tiles.cpp` is built with the host compiler alone and answers
queries for pick_lpr, pick_lpr_wide and pick_fill_tile.  Each answer is checked
against the rule the header states, applied here by brute force over all
candidates, and a few shapes are checked against choices worked out by hand
(the tiles the streaming kernels take at the benchmarked sizes).
"""
import math
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM_INC = "/opt/rocm/include"

# one-vector candidates as the MQ4 and fp8 launchers list them
MQ4_CAND = [(16, 2), (16, 1), (14, 2), (14, 1), (12, 2), (12, 1), (8, 2), (8, 1)]
FP8_CAND = [(7, 2), (8, 2), (7, 1), (8, 1)]


@pytest.fixture(scope="module")
def run(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir(ROCM_INC):
        pytest.skip("needs g++ and the ROCm headers")
    exe = str(tmp_path_factory.mktemp("host_tiles") / "host_tiles")
    subprocess.run([gxx, "-std=c++17", "-O1", "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INC,
                    "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "quantized_weight_decode_amd", "csrc"),
                    os.path.join(ROOT, "tests", "host_tiles.cpp"), "-o", exe], check=True)

    def query(lines):
        r = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True,
                           text=True, check=True)
        return r.stdout.split("\n")[:len(lines)]
    return query


def _eff(n, lpr):
    return n / (math.ceil(n / lpr) * lpr)


def test_lanes_per_row(run):
    ns = list(range(1, 2049))
    out = [tuple(int(v) for v in s.split()) for s in run([f"L {n}" for n in ns])]
    for n, (narrow, wide) in zip(ns, out):
        # pick_lpr: the widest of 64..4 whose sweeps leave the fewest lanes idle
        best = max(_eff(n, l) for l in (64, 32, 16, 8, 4))
        assert abs(_eff(n, narrow) - best) < 1e-9, n
        assert all(_eff(n, l) < best - 1e-9 for l in (64, 32, 16, 8, 4) if l > narrow), n
        # pick_lpr_wide: 64 or 32 from 32 chunks up, fewer idle lanes, ties to 64
        if n < 32:
            assert wide == narrow, n
        else:
            idle = {l: math.ceil(n / l) * l - n for l in (64, 32)}
            assert wide == (64 if idle[64] <= idle[32] else 32), n


def test_lanes_per_row_by_hand(run):
    # 16-byte chunks per row -> (pick_lpr, pick_lpr_wide)
    cases = {
        192: (64, 64),   # 6144 4-bit columns: three full sweeps of 64
        344: (8, 32),    # 11008 columns: 8 lanes fit exactly; 11 sweeps of 32 leave 8 idle
        592: (16, 32),   # 18944 columns: 19 sweeps of 32 leave 16 idle, 10 of 64 leave 48
        112: (16, 64),   # 3584 columns: 64 and 32 both leave 16 lanes idle
        68: (4, 32),     # 2176 columns
        1024: (64, 64),  # 16384 fp8 columns
        16: (16, 16),
        20: (4, 4),
    }
    out = run([f"L {n}" for n in cases])
    for (n, want), got in zip(cases.items(), out):
        assert tuple(int(v) for v in got.split()) == want, n


def _fill_choice(O, rpg, ncu, ors, cand):
    """The tile the header's rule names: best last-round fill among the allowed
    tiles, then fewest workgroups, then more rows per lane group, then the
    earlier candidate."""
    best = None
    for i, (w, r) in enumerate(cand):
        rows = w * rpg * r
        wgs = -(-O // rows)
        if ors and r == 1 and wgs > ncu:
            continue
        fill = wgs / (-(-wgs // ncu) * ncu)
        key = (round(fill, 9), -wgs, r, -i)
        if best is None or key > best[0]:
            best = (key, i)
    return best[1]


def _fill_query(O, rpg, ncu, ors, cand):
    return f"F {O} {rpg} {ncu} {int(ors)} {len(cand)} " + " ".join(f"{w} {r}" for w, r in cand)


def test_fill_tile_brute_force(run):
    qs = []
    for cand in (MQ4_CAND, FP8_CAND):
        for ors in (False, True):
            for rpg in (1, 2, 4):
                for O in list(range(1, 600, 7)) + list(range(600, 80000, 997)):
                    for ncu in (256, 80):
                        qs.append((O, rpg, ncu, ors, cand))
    out = run([_fill_query(*q) for q in qs])
    for q, got in zip(qs, out):
        assert int(got) == _fill_choice(*q), q


def test_fill_tile_by_hand(run):
    cases = [
        # MQ4, 8192 x 8192 (64 lanes per row): 16 waves x 2 rows, 256 workgroups
        ((8192, 1, 256, False, MQ4_CAND), 0),
        ((8192, 1, 256, True, MQ4_CAND), 0),
        # MQ4, 3584 rows of 18944 columns (32 lanes, two rows per wave): 8 x 1, 224 workgroups
        ((3584, 2, 256, False, MQ4_CAND), 7),
        # MQ4, 18944 rows of 3584 columns: 8 x 2 (1184 workgroups, five rounds at 0.925)
        ((18944, 1, 256, False, MQ4_CAND), 6),
        ((18944, 1, 256, True, MQ4_CAND), 6),
        # fp8, 7168 x 16384: 7 x 2 fills two rounds exactly (512 workgroups)
        ((7168, 1, 256, True, FP8_CAND), 0),
        # fp8, 2048 x 7168: 8 x 1 fills one round (256 workgroups)
        ((2048, 1, 256, True, FP8_CAND), 3),
        # 4097 rows: 7 x 1 fills its last round best (586 workgroups, 0.763) ...
        ((4097, 1, 256, False, FP8_CAND), 2),
        # ... but takes more than one round, so with one-row tiles held to a single
        # round 7 x 2 (293 workgroups, 0.572) beats 8 x 2 (257, 0.502)
        ((4097, 1, 256, True, FP8_CAND), 0),
        # MQ4, 8193 rows: 12 x 1 (683 workgroups) unless one-row tiles are held back,
        # then 12 x 2 (342)
        ((8193, 1, 256, False, MQ4_CAND), 5),
        ((8193, 1, 256, True, MQ4_CAND), 4),
    ]
    out = run([_fill_query(*q) for q, _ in cases])
    for (q, want), got in zip(cases, out):
        assert int(got) == want, q
