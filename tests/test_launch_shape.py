"""Host launch arithmetic of the decoders (csrc/df11_launch.h), built with
g++ on its own and checked against brute force: how a batched launch shares
its workgroups between streams, and the dynamic schedule's pool counts."""

import itertools
import math
import os
import subprocess

import numpy as np
import pytest

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(REPO, "entropy_decoding_df11_amd", "csrc")


@pytest.fixture(scope="module")
def cli(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("launch") / "launch_shape_cli")
    # (built under AddressSanitizer and UndefinedBehaviorSanitizer, every report fatal)
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-Wextra", "-Werror", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", f"-I{CSRC}",
                    os.path.join(REPO, "tests", "cpp", "launch_shape_cli.cpp"), "-o", exe], check=True)

    def run(lines):
        res = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True, check=True)
        return [[int(v) for v in ln.split()] for ln in res.stdout.strip().splitlines()]

    return run


def _best_max_ratio(sup, resident):
    """Smallest achievable max_i sup_i / want_i with 1 <= want_i <= sup_i and
    sum want_i <= max(resident, n), by brute force over every split."""
    cap = max(resident, len(sup))
    best = None
    for w in itertools.product(*[range(1, s + 1) for s in sup]):
        if sum(w) <= cap:
            r = max(s / x for s, x in zip(sup, w))
            best = r if best is None or r < best else best
    return best


def test_split_grid_never_exceeds_the_cap(cli):
    # the case that overshot before: one big stream and six of one super-group each
    cases = [(8, [1000, 1, 1, 1, 1, 1, 1]), (7, [1000, 1, 1, 1, 1, 1, 1]), (768, [5000, 1250, 1250, 5000, 17000, 17000, 17000])]
    rng = np.random.default_rng(0)
    for _ in range(300):
        n = int(rng.integers(1, 17))
        sup = [int(v) for v in rng.integers(1, 3000, n)]
        if rng.random() < 0.5:
            sup = [int(v) for v in np.where(rng.random(n) < 0.6, 1, sup)]
        cases.append((int(rng.integers(n, 1200)), sup))
    out = cli([f"S {len(s)} {r} " + " ".join(map(str, s)) for r, s in cases])
    for (resident, sup), want in zip(cases, out):
        assert len(want) == len(sup)
        assert sum(want) <= max(resident, len(sup)), (resident, sup, want)
        assert all(1 <= w <= s for w, s in zip(want, sup)), (sup, want)
        # every workgroup is used while some stream still has spare super-groups
        if sum(want) < max(resident, len(sup)):
            assert want == sup


def test_split_grid_minimises_the_largest_share(cli):
    rng = np.random.default_rng(1)
    cases = []
    for _ in range(120):
        n = int(rng.integers(1, 5))
        sup = [int(v) for v in rng.integers(1, 9, n)]
        cases.append((int(rng.integers(n, sum(sup) + 2)), sup))
    out = cli([f"S {len(s)} {r} " + " ".join(map(str, s)) for r, s in cases])
    for (resident, sup), want in zip(cases, out):
        got = max(s / w for s, w in zip(sup, want))
        assert math.isclose(got, _best_max_ratio(sup, resident)), (resident, sup, want)


def test_pool_shape(cli):
    rng = np.random.default_rng(2)
    cases = [(1, 1), (5, 768), (100000, 768), (100000, 1), (100000, 97), (100000, 770), (40, 13)]
    cases += [(int(rng.integers(1, 200000)), int(rng.integers(1, 2000))) for _ in range(400)]
    out = cli([f"P {ns} {w}" for ns, w in cases])
    for (n_super, want), (n_wg, pools, dynamic) in zip(cases, out):
        assert 1 <= n_wg <= max(1, min(want, n_super))
        assert 1 <= pools <= 8 and n_wg % pools == 0
        # a pool serves at most 96 workgroups, unless the grid needs more than 8 x 96
        assert n_wg // pools <= 96 or (pools == 8 and n_wg > 8 * 96)
        assert dynamic == int(n_super >= 12 * n_wg)
        # at most a few workgroups are dropped to make the pools divide the grid
        assert n_wg >= min(want, n_super) - 8


def test_coprime_stride(cli):
    grids = list(range(1, 400)) + [768, 1024, 1536]
    out = cli([f"C {g}" for g in grids])
    for g, (stride,) in zip(grids, out):
        assert math.gcd(stride, g) == 1 and 1 <= stride <= 2 * g + 1
