"""Checks on the generated gfx950 code that need no GPU.

The dK/dV kernel keeps its accumulators in AGPRs through asm MFMAs whose
latency the compiler cannot see. The code is only correct if nothing but
those MFMAs touches the accumulator registers until the fence after the
loop (32 wait states) has passed: no copies, no writes, no early reads.
"""

import re

import pytest

from exact_io_aware_35_amd import build

AGPR = re.compile(r"\ba(\d+)\b|\ba\[(\d+):(\d+)\]")


def agprs(text):
    regs = set()
    for m in AGPR.finditer(text):
        if m.group(1) is not None:
            regs.add(int(m.group(1)))
        else:
            regs.update(range(int(m.group(2)), int(m.group(3)) + 1))
    return regs


def kernel_body(asm, name):
    start = re.search(r"^" + re.escape(name) + r":", asm, re.M).start()
    end = asm.index(".Lfunc_end", start)
    lines = []
    for line in asm[start:end].splitlines():
        t = line.split(";")[0].strip()
        if t and not t.startswith(".") and not t.endswith(":"):
            lines.append(t)
    return lines


@pytest.fixture(scope="module")
def bwd_asm(tmp_path_factory):
    out = tmp_path_factory.mktemp("asm") / "fa_bwd.s"
    return open(build.device_asm("fa_bwd.hip", str(out))).read()


@pytest.mark.parametrize("D", [64, 128])
def test_dkdv_agpr_accumulators_untouched_until_fence(bwd_asm, D):
    body = kernel_body(bwd_asm, f"_ZN2fa15bwd_dkdv_kernelILi{D}EEEvNS_9BwdParamsE")
    acc_mfma = [i for i, l in enumerate(body)
                if l.startswith("v_mfma_f32_32x32x16_f16 a[")]
    # Per accumulator: one zero-init, then 4 k-steps in each of the two
    # tile bodies (the loop is unrolled over the two LDS buffers).
    assert len(acc_mfma) == 2 * (D // 32) * (1 + 2 * 4)
    acc = set()
    for i in acc_mfma:
        acc |= agprs(body[i].split(",")[0])
    assert len(acc) == 2 * (D // 32) * 16
    # The fence: a run of at least four s_nop 7 after the last accumulator MFMA.
    last = max(acc_mfma)
    run, fence_end = 0, None
    for i in range(last + 1, len(body)):
        run = run + 1 if body[i] == "s_nop 7" else 0
        if run == 4:
            fence_end = i
            break
    assert fence_end is not None, "no fence after the last accumulator MFMA"
    for i, l in enumerate(body):
        if i in acc_mfma or not (agprs(l) & acc):
            continue
        op = l.split()[0]
        assert op == "v_accvgpr_read_b32" and i > fence_end, f"accumulator AGPR touched: {i}: {l}"
