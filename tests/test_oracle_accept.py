"""Accept rule pins: the pages' worked example and an exhaustive property check."""
import itertools
import os
import random

from oracle.decode import accept

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.txt")


def _fixture():
    rows = {}
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        k, v = line.split(":", 1)
        rows[k.strip()] = v.split()
    return rows


def test_worked_example_from_the_page():
    fx = _fixture()
    draft, ver, emit = fx["draft"], fx["verify"], fx["emit"]
    rng = random.Random(0)
    for _ in range(20):
        fill = [rng.choice("ABCDEFGHXYZ") for _ in range(len(draft) + 1 - len(ver))]
        a, out = accept(draft, ver + fill)
        assert a == int(fx["accepted"][0])
        assert out == emit


def test_all_match_gives_bonus():
    a, out = accept([1, 2, 3], [1, 2, 3, 9])
    assert a == 3 and out == [1, 2, 3, 9]


def test_exhaustive_properties_small_vocab():
    """vocab 3, x <= 4, every (draft, verified) pair: the emitted list is
    characterised without the scan -- its last element is the verifier's token
    at its own index, the rest equal both draft and verifier, and the draft
    either ran out or disagrees right where the emitted list ends."""
    for x in range(0, 5):
        for draft in itertools.product(range(3), repeat=x):
            for ver in itertools.product(range(3), repeat=x + 1):
                a, out = accept(list(draft), list(ver))
                assert len(out) == a + 1 and 0 <= a <= x
                assert out[-1] == ver[a]
                assert all(out[i] == draft[i] == ver[i] for i in range(a))
                assert a == x or draft[a] != ver[a]


def test_emitted_is_a_prefix_of_the_true_continuation():
    """Whatever the draft, the emitted tokens are the verifier's own greedy
    continuation: with verified[i] = truth[i], out == truth[:a+1]."""
    rng = random.Random(1)
    for _ in range(2000):
        x = rng.randint(1, 12)
        truth = [rng.randrange(4) for _ in range(x + 1)]
        draft = [t if rng.random() < 0.7 else rng.randrange(4) for t in truth[:x]]
        a, out = accept(draft, truth)
        assert out == truth[: a + 1]
