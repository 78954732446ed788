"""Scratch audit of the gfx950 kernels (CPU only): every kernel the library
builds must run without scratch (private) memory, i.e. without register
spills or stack arrays in its hot loops.  This is the check the vLLM
"[ROCm] Octave KV (ROCM_OCTAVE)" pull request reports in its "Validation"
table (no kernel of the built library uses scratch), done here from the
compiler's per-kernel resource report.

The report comes from the library build (build.py keeps it next to each
object); if it is missing or older than the sources, the sources are compiled
for the device here with the same flags to produce it.
"""
import concurrent.futures
import os
import re
import subprocess
import tempfile

from bit_quantized_matmul_q4_amd import build as b

FUNC = re.compile(r"remark: Function Name: (\S+)")
SCRATCH = re.compile(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)")
GLOBAL = re.compile(r"__global__")


def _fresh(src, report):
    if not os.path.exists(report):
        return False
    deps = [src] + [os.path.join(b.CSRC, f) for f in os.listdir(b.CSRC) if f.endswith(".h")] + \
        [os.path.join(b.INCLUDE, f) for f in os.listdir(b.INCLUDE)]
    return os.path.getmtime(report) >= max(os.path.getmtime(d) for d in deps)


def _report(src, tmp):
    path = b.resource_report_path(src)
    if _fresh(src, path):
        return open(path).read()
    obj = os.path.join(tmp, os.path.basename(src) + ".o")
    cmd = [b.HIPCC] + b.FLAGS + [b.RESOURCE_REMARKS, "--offload-device-only", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return r.stderr


def test_no_kernel_uses_scratch():
    srcs = b.sources()
    with tempfile.TemporaryDirectory() as tmp, concurrent.futures.ThreadPoolExecutor(len(srcs)) as ex:
        reports = dict(zip(srcs, ex.map(lambda s: _report(s, tmp), srcs)))
    total = 0
    for src, text in reports.items():
        names = FUNC.findall(text)
        sizes = [int(v) for v in SCRATCH.findall(text)]
        assert len(names) == len(sizes), src
        if GLOBAL.search(open(src).read()):
            assert names, "%s: no resource report for its kernels" % src
        bad = [(n, v) for n, v in zip(names, sizes) if v != 0]
        assert not bad, "%s: kernels using scratch: %s" % (os.path.basename(src), bad)
        total += len(names)
    assert total >= 50, total  # every template instance of every kernel is reported
