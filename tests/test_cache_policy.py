"""The expert cache's slot policy (csrc/expert_cache_policy.h), driven through
tests/native/cache_policy.cpp on the CPU, against tests/cache_model.py, a model
of the rules include/qmoe.h states: hits, every (expert, slot) load, refusals
when the misses do not fit, pinned and protected slots, eviction counts."""
import os
import random
import shutil
import subprocess

import pytest

from cache_model import SlotModel

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GXX = shutil.which("g++")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not GXX:
        pytest.skip("needs g++")
    exe = str(tmp_path_factory.mktemp("policy") / "cache_policy")
    subprocess.run([GXX, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined",
                    "-I", os.path.join(ROOT, "quantized_moe_02_amd", "csrc"),
                    os.path.join(ROOT, "tests", "native", "cache_policy.cpp"), "-o", exe],
                   check=True)
    return exe


def _scenario(rng, E, S, n_req):
    """Random requests (some larger than the cache), prefetch-like protected
    requests, pins and unpins; returns (commands, model outputs)."""
    m = SlotModel(E, S)
    cmds, want = [f"{E} {S}"], []
    hot = rng.sample(range(E), min(E, 4))
    for _ in range(n_req):
        r = rng.random()
        if r < 0.08:
            ex = rng.sample(range(E), rng.randint(1, 3))
            cmds.append(f"p {len(ex)} " + " ".join(map(str, ex)))
            m.pin(ex)
            want.append(f"pinned {len(m.pinned)}")
        elif r < 0.12:
            cmds.append("u")
            m.unpin_all()
            want.append("pinned 0")
        else:
            k = rng.randint(1, max(1, min(E, S + 2)))
            ex = [rng.choice(hot) if rng.random() < 0.4 else rng.randrange(E) for _ in range(k)]
            prot = m.requests if (r < 0.3 and m.requests > 0) else None
            cmds.append(f"a {-1 if prot is None else prot} {len(ex)} " + " ".join(map(str, ex)))
            res = m.request(ex, prot)
            if res is None:
                want.append("fail")
            else:
                hits, loads = res
                want.append(" ".join([f"ok {hits}"] + [f"{e}:{s}" for e, s in loads]))
        want.append(" ".join(map(str, m.table())))
    want.append(f"clock {m.requests} evictions {m.evictions}")
    return cmds, want


@pytest.mark.parametrize("E,S,seed", [(8, 1, 0), (8, 3, 1), (16, 4, 2), (16, 16, 3), (64, 10, 4),
                                      (256, 32, 5), (256, 8, 6)])
def test_policy_matches_model(driver, E, S, seed):
    rng = random.Random(seed)
    cmds, want = _scenario(rng, E, S, 300)
    r = subprocess.run([driver], input="\n".join(cmds) + "\n", capture_output=True, text=True,
                       timeout=60)
    assert r.returncode == 0, r.stderr
    got = r.stdout.strip().split("\n")
    assert len(got) == len(want)
    for i, (g, w) in enumerate(zip(got, want)):
        assert g == w, f"line {i}: command {cmds[1 + i // 2] if i // 2 < len(cmds) - 1 else ''!r}\n got  {g}\n want {w}"


def test_lru_order_by_hand(driver):
    """Three slots: A B C loaded, A used again, D evicts B (least recent), a
    request that needs more experts than slots fails and changes nothing."""
    cmds = ["6 3", "a -1 3 0 1 2", "a -1 1 0", "a -1 1 3", "a -1 4 0 1 2 3", "a -1 2 3 4"]
    r = subprocess.run([driver], input="\n".join(cmds) + "\n", capture_output=True, text=True,
                       timeout=60)
    lines = r.stdout.strip().split("\n")
    assert lines[0] == "ok 0 0:0 1:1 2:2"
    assert lines[2] == "ok 1"
    assert lines[4] == "ok 0 3:1"          # expert 1 (slot 1) was least recently used
    assert lines[5] == "0 -1 2 1 -1 -1"
    assert lines[6] == "fail"
    assert lines[7] == lines[5]
    assert lines[8] == "ok 1 4:2"          # slot 0 (expert 0) is newer than slot 2
