"""Every HIP kernel compiles for gfx950 without private-memory use: no VGPR
or SGPR spills and no scratch (a private array the compiler could not keep in
registers turns every access into a memory round trip).  Host-only check: it
reads the compiler's resource-usage report."""
import os
import re
import subprocess

import pytest

from masked_gqa_attention_action_amd import build

CSRC = os.path.join(os.path.dirname(build.__file__), "csrc")
HOST_ONLY = ("dmx_api.hip", "dmx_profiles.hip")  # sources that define no kernel


def _report(src):
    cmd = [build.hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "--cuda-device-only", "-c", os.path.join(CSRC, src), "-o", os.devnull,
           "-Rpass-analysis=kernel-resource-usage"] + build.SOURCE_FLAGS.get(src, [])
    out = subprocess.run(cmd, capture_output=True, text=True, check=True).stderr
    kernels, name = {}, None
    for line in out.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            kernels[name] = {}
            continue
        m = re.search(r"remark:\s+(ScratchSize \[bytes/lane\]|VGPRs Spill|SGPRs Spill|VGPRs|AGPRs): (\d+)", line)
        if m and name:
            kernels[name][m.group(1)] = int(m.group(2))
    return kernels


def _scratch_instructions(src):
    """Private-memory instructions (gfx950 reaches it through scratch_*) in
    the generated code of each kernel of src."""
    cmd = [build.hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", "-"] + \
        build.SOURCE_FLAGS.get(src, [])
    asm = subprocess.run(cmd, capture_output=True, text=True, check=True).stdout
    count, name = {}, None
    for line in asm.splitlines():
        m = re.match(r"^(_Z\S+):", line)
        if m:
            name = m.group(1)
            count[name] = 0
        elif name and re.match(r"^\s+scratch_", line):
            count[name] += 1
    return count


# The persistent step kernel keeps a few dozen uniform branch masks and
# descriptors live across its whole layer loop, more than the 102 scalar
# registers of a wave hold.  The compiler parks them in lanes of a vector
# register (v_writelane / v_readlane: no memory), and reserves a 20-byte
# frame it never touches; the kernel's code must hold no private-memory
# instruction.  Every other kernel has neither.
STEP_MAX_SGPR_SPILL, STEP_MAX_FRAME = 64, 32


@pytest.mark.parametrize("src", build.SOURCES)
def test_no_private_memory(src):
    kernels = _report(src)
    if src not in HOST_ONLY:
        assert kernels, f"no kernels reported for {src}"
    scratch_ops = _scratch_instructions(src) if any("k_step" in n for n in kernels) else {}
    for name, r in kernels.items():
        assert r.get("VGPRs Spill", 0) == 0, (name, r)
        assert r.get("VGPRs", 0) + r.get("AGPRs", 0) <= 512, (name, r)
        if "k_step" in name:
            assert r.get("SGPRs Spill", 0) <= STEP_MAX_SGPR_SPILL, (name, r)
            assert r.get("ScratchSize [bytes/lane]", 0) <= STEP_MAX_FRAME, (name, r)
            assert scratch_ops.get(name, 0) == 0, (name, "private-memory instructions", scratch_ops.get(name))
        else:
            assert r.get("ScratchSize [bytes/lane]", 0) == 0, (name, r)
            assert r.get("SGPRs Spill", 0) == 0, (name, r)
