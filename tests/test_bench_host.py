"""Host-side logic of bench.py (no GPU): the committed counter records are
used only for the kernel source they were taken on, each kernel class adds
the right kernels (at the right grid where one kernel runs at several), and
a request for more than one GPU is refused before anything touches a GPU."""
import os
import shutil
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _records(path):
    out = {}
    for line in open(path):
        if line.startswith("traffic "):
            name, rest = line[len("traffic "):].split(" grid=")
            grid, rest = rest.split(" bytes=")
            out[(name, int(grid))] = int(rest.split()[0])
    return out


def test_traffic_classes_sum_their_kernels(tmp_path, monkeypatch):
    """Each kernel class adds the records of its kernels (the committed
    records, re-stamped with the current source hashes so that only the
    mapping is under test)."""
    import hashlib
    import re

    sha = {f: hashlib.sha1(open(os.path.join(bench.CSRC, f), "rb").read()).hexdigest() for f in ("sym.hip", "kivi.hip")}
    text = open(bench.TRAFFIC_FILE).read()
    text = re.sub(r"(traffic (sym|kivi)\S*.*?src_sha1=)[0-9a-f]+",
                  lambda m: m.group(1) + sha["sym.hip" if m.group(2) == "sym" else "kivi.hip"], text)
    f = tmp_path / "traffic.md"
    f.write_text(text)
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    rec = _records(str(f))
    # the long-context chunk class: 64 launches of the q6 write kernel at the chunk's grid,
    # not the paged prefill's record of the same kernel
    assert bench.measured_traffic("quant_chunks_q6_x64") == 64 * rec[("sym_quant_v8<6, 32, 2>", 8388608)]
    assert bench.measured_traffic("quant_prefill_q6") == rec[("sym_quant_v8<6, 32, 2>", 1073741824)]
    assert bench.measured_traffic("dequant_full_q6") == rec[("sym_dequant_page<6, 256>", 538968064)]
    assert bench.measured_traffic("kivi_pack_b2") == (rec[("kivi_keys_fast<2, 8, 4, true>", 16515072)] +
                                                      rec[("kivi_values_fast<2, 8, 4, 4, true>", 16515072)])
    assert bench.measured_traffic("no_such_class") is None


def test_records_follow_the_kernel_source(tmp_path, monkeypatch):
    """A record counts only while the hash of its kernel source matches: any
    changed byte of the source invalidates it (records written here for a
    copy of the sources, so the test does not depend on the committed
    records being current)."""
    import hashlib

    csrc = tmp_path / "csrc"
    shutil.copytree(bench.CSRC, csrc)
    sha = lambda f: hashlib.sha1(open(csrc / f, "rb").read()).hexdigest()
    traffic = tmp_path / "traffic.md"
    traffic.write_text("traffic sym_quant_v8<8, 32, 1> grid=2147483648 bytes=1234 src_sha1=%s\n"
                       "traffic kivi_keys_fast<2, 8, 4, false> grid=16515072 bytes=5 src_sha1=%s\n"
                       "traffic kivi_values_fast<2, 8, 4, 1, false> grid=66060288 bytes=6 src_sha1=%s\n"
                       % (sha("sym.hip"), sha("kivi.hip"), sha("kivi.hip")))
    valu = tmp_path / "valu.md"
    valu.write_text("valu_call nuq_prefill insts=777 src_sha1=%s\n" % sha("nuq.hip"))
    monkeypatch.setattr(bench, "CSRC", str(csrc))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(traffic))
    monkeypatch.setattr(bench, "VALU_FILE", str(valu))
    assert bench.measured_traffic("quant_prefill_q8") == 1234
    assert bench.measured_traffic("kivi_keys_values_b2") == 11
    assert bench.measured_valu("nuq_prefill") == 777
    for f in ("sym.hip", "nuq.hip"):
        with open(csrc / f, "a") as fh:
            fh.write("\n")
    assert bench.measured_traffic("quant_prefill_q8") is None
    assert bench.measured_valu("nuq_prefill") is None
    assert bench.measured_traffic("kivi_keys_values_b2") == 11  # kivi.hip unchanged


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
