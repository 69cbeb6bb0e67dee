"""Properties of the gfx950 code the library is built from (CPU only): the
device assembly of kvmove.hip, compiled with the library's own flags, shows
for every kernel the float modes the method's arithmetic relies on (float32
denormals kept, round to nearest-even, IEEE mode), no scratch memory, and no
packed float32 instructions (they are kept out of the build by a flag)."""
import os
import re
import subprocess

import pytest

from paged_kv_movement_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("asm") / "kvmove.s")
    flags = [f for f in build.FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [build.hipcc(), *flags, "--cuda-device-only", "-S", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(build.HERE, "csrc"), "-o", out, build.SRC]
    subprocess.run(cmd, check=True, capture_output=True)
    return open(out).read()


def _kernel_descriptors(asm):
    blocks = re.findall(r"\.amdhsa_kernel (\S+)\n(.*?)\.end_amdhsa_kernel", asm, flags=re.S)
    return {name: dict(re.findall(r"\.amdhsa_(\w+) (\S+)", body)) for name, body in blocks}


def test_every_kernel_keeps_denormals_rounds_to_nearest_and_uses_no_scratch(device_asm):
    ks = _kernel_descriptors(device_asm)
    assert len(ks) >= 30
    for name, d in ks.items():
        assert d["float_denorm_mode_32"] == "3", name        # float32 denormals in and out kept (no flush to zero)
        assert d["float_denorm_mode_16_64"] == "3", name
        assert d["float_round_mode_32"] == "0", name         # round to nearest-even
        assert d["ieee_mode"] == "1", name
        assert d["private_segment_fixed_size"] == "0", name  # no scratch (register spills)


def test_no_packed_float32_instructions(device_asm):
    packed = ["v_pk_" + op + "_f32" for op in ("add", "mul", "fma")]
    lines = [l for l in device_asm.splitlines() if l.strip() and not l.lstrip().startswith(";")]
    for p in packed:
        assert not any(re.match(r"\s*" + p + r"\b", l) for l in lines), p
