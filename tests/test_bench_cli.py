"""bench.py's command line on the CPU: more than one GPU is refused with a message before any
device work (the library measures one GPU's share; the multi-GPU design is documentation)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line


def test_workload_names_and_profiles_resolve():
    """Every default bench line parses into a base workload and variant flags, and names the
    kernel whose committed counter summary gives its traffic."""
    sys.path.insert(0, ROOT)
    import bench
    names = ["csa_decode_128k"] + bench.DEFAULT_EXTRA.split(",")
    assert len(set(names)) == len(names)
    for n in names:
        base, flags = bench.parse_name(n)
        assert flags <= set(bench.FLAGS)
        key, q, bf16 = bench.formats(flags)
        assert (q == "mxfp4") <= (key == "mxfp4")  # an FP4 query only with FP4 keys
    assert bench.parse_name("csa_decode_1m_fp4q_bf16s") == ("csa_decode_1m", {"fp4q", "bf16s"})
    assert bench.formats({"fp4q"}) == ("mxfp4", "mxfp4", False)
    assert bench.formats({"mxfp4", "bf16s"}) == ("mxfp4", "e4m3", True)
