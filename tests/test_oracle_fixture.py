"""The oracle still reproduces tests/golden/oracle_tiny_fixture.json, which
tests/golden/make_oracle_fixture.py wrote from the oracle itself: a regression
guard against accidental changes to the oracle's arithmetic (an intended
change rewrites the fixture with that script and says why in its commit)."""
import importlib.util
import json
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def _load_maker():
    spec = importlib.util.spec_from_file_location("make_oracle_fixture",
                                                  os.path.join(HERE, "golden", "make_oracle_fixture.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_oracle_reproduces_its_fixture():
    stored = json.load(open(os.path.join(HERE, "golden", "oracle_tiny_fixture.json")))
    mk = _load_maker()
    assert stored["workload"] == mk.WORKLOAD
    now = mk.compute()
    assert now["n_edges"] == stored["values"]["n_edges"]
    for key, rec in stored["values"].items():
        if key == "n_edges":
            continue
        cur = now[key]
        assert cur["shape"] == rec["shape"], key
        scale = math.sqrt(rec["sumsq"] / max(1, math.prod(rec["shape"])))
        for field in ("sum", "sumsq"):
            assert math.isclose(cur[field], rec[field], rel_tol=1e-9, abs_tol=1e-9 * scale * 100), (key, field)
        for i, v in rec["entries"].items():
            assert math.isclose(cur["entries"][i], v, rel_tol=1e-9, abs_tol=1e-12 * max(scale, 1.0)), (key, i)
