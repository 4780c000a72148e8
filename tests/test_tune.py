"""The tile sweep's bookkeeping (no GPU): its first candidate per head dim is
the library default, and its validity rule mirrors the kernel's
compile-time checks."""
import os
import re

from flashattention_tiled_amd import tune

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "flashattention_tiled_amd", "csrc", "fa2_plan.h")


def test_first_candidate_is_the_library_default():
    text = open(SRC).read()
    for D, cfgs in tune.CANDIDATES.items():
        m = re.search(rf"#define FA2_TILE_D{D} ([\d, ]+)\n", text)
        assert m, D
        default = tuple(int(x) for x in m.group(1).split(","))
        assert cfgs[0] == default, (D, cfgs[0], default)
        assert tune.valid(D, default)


def test_validity_rule():
    assert tune.valid(128, (4, 1, 64, 2, 2))
    # four loads per K/V tile and wave cannot be spaced every 4 of 16 k-steps
    assert not tune.valid(128, (4, 1, 64, 2, 4))
    # K and V rings of 4 x 64 KiB exceed the 160 KiB of LDS
    assert not tune.valid(256, (4, 1, 128, 1, 0))
    # a tile must split into whole 1 KiB wave loads, and B_c into 32-key blocks
    assert not tune.valid(64, (16, 1, 32, 1, 0))
    assert not tune.valid(64, (4, 1, 48, 2, 0))
    # ring depth: D = 256, 32-key tiles take 16 KiB per stage and ring, so four
    # stages of K and V take 128 KiB; six would exceed the 160 KiB, and five
    # exceed the key loop's unroll (a multiple of 2 and of the depth, <= 6)
    assert tune.valid(256, (4, 1, 32, 1, 1, 4))
    assert not tune.valid(256, (4, 1, 32, 1, 1, 5))
    assert not tune.valid(256, (4, 1, 32, 1, 1, 6))
    assert not tune.valid(128, (4, 1, 64, 2, 2, 1))
    # the key loop is pipelined (1) or not (0)
    assert tune.valid(256, (4, 1, 32, 2, 1, 2, 0))
    assert not tune.valid(256, (4, 1, 32, 2, 1, 2, 2))


def test_names_are_unique():
    names = [tune.name(D, c) for D, cs in tune.CANDIDATES.items() for c in cs]
    assert len(names) == len(set(names))
