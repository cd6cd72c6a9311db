"""The timed kernel instances compile without register spills and within the
register share that lets two seven-wave (or eight-wave) work-groups share a
CU: read from the compiler's kernel-resource-usage remarks
(build.resource_report).  A spill turns into scratch traffic inside the row
loop, with vmcnt waits that also wait for the next row's loads."""
import pytest

from rotation_activation_quantization_amd import build as B

# instance -> fragment of its mangled name (template arguments: KA, KB, d given
# as a vector, y_out, integer zero-point, SwiGLU producer; for the two-half
# kernel the same without KA and KB)
SPILL_FREE = {
    "n=14336 (c, sigma)": "rq_fast_kernelILi28ELi9ELb0ELb0ELb0ELb0E",
    "n=14336 d-vector": "rq_fast_kernelILi28ELi9ELb1ELb0ELb0ELb0E",
    "n=14336 y_out": "rq_fast_kernelILi28ELi9ELb0ELb1ELb0ELb0E",
    "n=14336 integer zero-point": "rq_fast_kernelILi28ELi9ELb0ELb0ELb1ELb0E",
    "n=14336 SwiGLU": "rq_fast_kernelILi28ELi9ELb0ELb0ELb0ELb1E",
    "n=28672 (c, sigma)": "rq_halves_kernelILb0ELb0ELb0ELb0E",
    "n=28672 d-vector": "rq_halves_kernelILb1ELb0ELb0ELb0E",
    "n=28672 integer zero-point": "rq_halves_kernelILb0ELb0ELb1ELb0E",
    "n=28672 SwiGLU": "rq_halves_kernelILb0ELb0ELb0ELb1E",
    "n=4096 (c, sigma)": "rq_fast_kernelILi32ELi7ELb0ELb0ELb0ELb0E",
    "n=8192 (c, sigma)": "rq_fast_kernelILi32ELi8ELb0ELb0ELb0ELb0E",
    "n=8192 d-vector": "rq_fast_kernelILi32ELi8ELb1ELb0ELb0ELb0E",
    "n=16384 (c, sigma)": "rq_fast_kernelILi32ELi9ELb0ELb0ELb0ELb0E",
    "traffic ceiling": "stream_ceiling_kernel",
}


@pytest.fixture(scope="module")
def report():
    return B.resource_report(["rq_fast.hip", "rq_halves.hip", "ceiling.hip"])


@pytest.mark.parametrize("label", list(SPILL_FREE))
def test_timed_instances_do_not_spill(report, label):
    frag = SPILL_FREE[label]
    hits = [r for name, r in report.items() if frag in name]
    assert len(hits) == 1, (label, frag, len(hits))
    r = hits[0]
    assert r["scratch"] == 0, f"{label}: {r['scratch']} B/lane of scratch (spills)"
    assert r["vgprs"] + r["agprs"] <= 128, f"{label}: {r['vgprs']} VGPRs + {r['agprs']} AGPRs"


def test_report_lists_every_kernel_of_the_sources(report):
    # six (KA, KB) shapes x seven instances, seven two-half instances, the
    # ceiling kernel; every one carries the four fields
    assert len(report) == 6 * 7 + 7 + 1
    for name, r in report.items():
        assert {"vgprs", "agprs", "scratch", "occupancy"} <= set(r), name
