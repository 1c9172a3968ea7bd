"""Host-side pieces of bench.py (no GPU): the code digest that keys the
committed HBM-traffic figures to the kernel code they were measured on."""
import importlib.util
import json
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_code_digest_ignores_comments_not_code(tmp_path):
    b = _bench()
    base = 'int f(int x) { // scale\n  return x * 2; /* twice */ }\nconst char* s = "a // b";\n'
    p = tmp_path / "k.hip"
    p.write_text(base)
    d0 = b.code_digest(str(p))
    p.write_text(base.replace("// scale", "// scales the input").replace("/* twice */", ""))
    assert b.code_digest(str(p)) == d0
    p.write_text(base.replace("  return", "\n\n    return"))       # whitespace only
    assert b.code_digest(str(p)) == d0
    p.write_text(base.replace("x * 2", "x * 3"))                   # code
    assert b.code_digest(str(p)) != d0
    p.write_text(base.replace('"a // b"', '"a // c"'))             # inside a string literal
    assert b.code_digest(str(p)) != d0


def test_traffic_records_are_complete():
    recs = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    assert recs
    for key, r in recs.items():
        for field in ("kernel", "source", "code_sha256", "fetch_scale", "write_scale",
                      "traffic_bytes", "algorithmic_bytes"):
            assert field in r, (key, field)
        assert os.path.exists(os.path.join(ROOT, r["source"])), key
        assert r["traffic_bytes"] > 0 and r["algorithmic_bytes"] > 0, key
