"""Checks on the generated gfx950 code that need no GPU.

The kernels are shaped so that each wave's state fits its registers: a
spill to scratch memory (or to accumulator registers through copies) would
add memory traffic to every tile. The compiler's own resource report for
each kernel must show no spills and no private scratch.
"""

import re

import pytest

from exact_io_aware_35_amd import build


def kernel_resources(asm):
    """{kernel name: {field: int}} from the assembler's metadata: one YAML list
    entry per kernel under amdhsa.kernels, each starting at "- .agpr_count"."""
    meta = asm[asm.index("amdhsa.kernels:"):]
    out = {}
    for entry in re.split(r"\n\s+- \.agpr_count", meta)[1:]:
        entry = ".agpr_count" + entry
        name = re.search(r"\.name:\s+(\S+)", entry).group(1)
        fields = {}
        for key in ("vgpr_count", "agpr_count", "vgpr_spill_count", "sgpr_spill_count",
                    "private_segment_fixed_size"):
            f = re.search(r"\." + key + r":\s+(\d+)", entry)
            if f:
                fields[key] = int(f.group(1))
        out[name] = fields
    return out


@pytest.fixture(scope="module", params=["fa_fwd.hip", "fa_fwd_fp8.hip", "fa_bwd.hip"])
def resources(request, tmp_path_factory):
    out = tmp_path_factory.mktemp("asm") / (request.param + ".s")
    return kernel_resources(open(build.device_asm(request.param, str(out))).read())


def test_kernels_do_not_spill(resources):
    assert resources, "no kernels found"
    for name, f in resources.items():
        assert f.get("vgpr_spill_count", 0) == 0, name
        assert f.get("sgpr_spill_count", 0) == 0, name
        assert f.get("private_segment_fixed_size", 0) == 0, name
        assert f.get("agpr_count", 0) == 0, name  # accumulators stay in arch VGPRs
