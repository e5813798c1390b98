"""Register budgets of the hot kernels, checked at compile time on the CPU: the prefill scan
instantiations that the 130m (f32, fused conv) and 2.8b (bf16) layers and the backbone run,
and the fused decode step, must not spill to scratch memory. A spill costs these kernels
several percent (the 130m output pass lost about 3 us per call to a 16-byte spill)."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mamba_selective_scan_fwd_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None,
                                reason="hipcc not available")


def resource_usage(src: str) -> dict:
    """Kernel name -> {'vgprs': int, 'scratch': int} from the compiler's resource remarks."""
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include"),
           "--cuda-device-only", "-Rpass-analysis=kernel-resource-usage", "-c", os.path.join(CSRC, src),
           "-o", os.devnull]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    out, cur = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            out[cur] = {}
            continue
        m = re.search(r"remark:\s+(VGPRs|ScratchSize \[bytes/lane\]): (\d+)", line)
        if m and cur:
            out[cur]["vgprs" if m.group(1) == "VGPRs" else "scratch"] = int(m.group(2))
    return out


@pytest.fixture(scope="module")
def scan_usage():
    return resource_usage("scan.hip")


# (I/O type, fused conv width) -> mangled template prefix of scan_kernel<IO, 16, 32, 4, OUT, GATE, KC>
HOT_SCAN = {
    "130m summary pass (f32, fused conv)": "_ZN5mamba11scan_kernelIfLi16ELi32ELi4ELb0ELb0ELi4E",
    "130m output pass (f32, fused conv)": "_ZN5mamba11scan_kernelIfLi16ELi32ELi4ELb1ELb1ELi4E",
    "backbone summary pass (f32)": "_ZN5mamba11scan_kernelIfLi16ELi32ELi4ELb0ELb0ELi0E",
    "backbone output pass (f32)": "_ZN5mamba11scan_kernelIfLi16ELi32ELi4ELb1ELb1ELi0E",
    "2.8b scan (bf16)": "_ZN5mamba11scan_kernelIDF16bLi16ELi32ELi4ELb1ELb1ELi0E",
}


@pytest.mark.parametrize("what", sorted(HOT_SCAN))
def test_hot_scan_kernels_do_not_spill(scan_usage, what):
    prefix = HOT_SCAN[what]
    hits = {k: v for k, v in scan_usage.items() if k.startswith(prefix)}
    assert hits, f"{what}: instantiation {prefix} not found"
    for name, use in hits.items():
        assert use.get("scratch") == 0, f"{what} ({name}) spills {use.get('scratch')} bytes per lane"


def test_decode_step_kernel_does_not_spill():
    use = resource_usage("step.hip")
    hits = {k: v for k, v in use.items() if "decode_step_kernel" in k or "decode_step_k4_kernel" in k}
    assert any("decode_step_k4_kernel" in k for k in hits) and any("decode_step_kernel" in k for k in hits)
    for name, u in hits.items():
        assert u.get("scratch") == 0, f"{name} spills {u.get('scratch')} bytes per lane"


# backbone kernels of the 130m prefill: the in_proj / out_proj tiles with direct LDS staging,
# the fused conv + x_proj, and the kernel that sums x_proj's planes and applies dt_proj
HOT_BACKBONE = {
    "in_proj 128x128 tiles": "_ZN5mamba16gemm_mfma_kernelIDF16bLi128ELi128ELi64ELi2ELi2ELb1ELb1E",
    "out_proj 128x96 tiles": "_ZN5mamba16gemm_mfma_kernelIDF16bLi128ELi96ELi64ELi4ELi1ELb1ELb1E",
    "conv + x_proj": "_ZN5mamba17conv_xproj_kernel",
    "x_proj sum + dt_proj": "_ZN5mamba23xproj_sum_dtproj_kernel",
}


def test_hot_backbone_kernels_do_not_spill():
    use = resource_usage("backbone.hip")
    for what, prefix in HOT_BACKBONE.items():
        hits = {k: v for k, v in use.items() if k.startswith(prefix)}
        assert hits, f"{what}: kernel {prefix} not found"
        for name, u in hits.items():
            assert u.get("scratch") == 0, f"{what} ({name}) spills {u.get('scratch')} bytes per lane"
