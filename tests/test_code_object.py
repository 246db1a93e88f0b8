"""The gfx950 code object of the built library: register budgets.

Reads the kernel metadata (AMDGPU code-object notes) of this repository's
own build of libmoe_mxfp4.so with the ROCm LLVM tools, on the CPU.  A spill
in a streaming kernel turns into scratch loads that its counted waits must
drain: the one-token launch lost about 1 us per layer to 68 bytes of spills
once.  Checked here:
  * no kernel keeps a dynamic stack or any scratch memory, except the prefill
    down, which saves two vector registers before its contraction loop and
    restores them after it (scalar registers spilled into vector register
    lanes cost no memory traffic and are not counted);
  * the register counts the launch designs rely on: the routed down of the
    batched decode under 128 VGPRs (four waves per SIMD), the one-token launch
    within 256 (two waves per SIMD), the prefill GEMM launches within 256
    (8-wave workgroups, one per CU).
"""

import os
import re
import shutil
import subprocess

import pytest

from mxfp4_routed_expert_x896_amd import build as B

LLVM_BIN = "/opt/rocm/llvm/bin"
BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"

# kernels allowed to spill, with the most vector registers they may spill
SPILL_ALLOWED = {"moe_mx_down": 2}
# (kernel name substring, most VGPRs)
VGPR_CEILING = [("moe_routed_down_combine", 128), ("moe_decode_front", 256),
                ("moe_mx_gateup", 256), ("moe_mx_down", 256)]


def _tool(name):
    path = os.path.join(LLVM_BIN, name)
    return path if os.path.exists(path) else shutil.which(name)


def _parse_notes(text):
    """Kernel entries of an NT_AMDGPU_METADATA dump: {name: {field: value}}."""
    kernels = {}
    body = text.split("amdhsa.kernels:", 1)[-1]
    for entry in re.split(r"^  - ", body, flags=re.M)[1:]:
        fields = {}
        for line in ("    " + entry).splitlines():
            m = re.match(r"^    \.(\w+):\s*(\S+)?\s*$", line)
            if m:
                fields[m.group(1)] = m.group(2)
        if "name" in fields:
            kernels[fields["name"]] = fields
    return kernels


@pytest.fixture(scope="module")
def kernels(tmp_path_factory):
    tools = {n: _tool(n) for n in ("llvm-objcopy", "clang-offload-bundler", "llvm-readelf")}
    if not all(tools.values()):
        pytest.skip("ROCm LLVM tools not found")
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("library not built")
    d = tmp_path_factory.mktemp("codeobj")
    fat = d / "fatbin.bin"
    subprocess.run([tools["llvm-objcopy"], "-O", "binary", "--only-section=.hip_fatbin",
                    B.LIB_PATH, str(fat)], check=True)
    data = fat.read_bytes()
    offs = [m.start() for m in re.finditer(re.escape(BUNDLE_MAGIC), data)] + [len(data)]
    assert len(offs) > 1, "no offload bundle in the library"
    out = {}
    for i in range(len(offs) - 1):  # one bundle per translation unit
        part, co = d / f"b{i}.bin", d / f"b{i}.co"
        part.write_bytes(data[offs[i]:offs[i + 1]])
        subprocess.run([tools["clang-offload-bundler"], "--unbundle", "--type=o",
                        f"--input={part}", f"--targets={TARGET}", f"--output={co}"], check=True)
        notes = subprocess.run([tools["llvm-readelf"], "--notes", str(co)], check=True,
                               capture_output=True, text=True).stdout
        out.update(_parse_notes(notes))
    return out


def test_the_layer_kernels_are_in_the_code_object(kernels):
    names = " ".join(kernels)
    for k in ("moe_decode_front", "moe_router_shared_gateup", "moe_select_shared_down",
              "moe_routed_gateup", "moe_routed_down_combine", "moe_mx_gateup", "moe_mx_down",
              "moe_combine", "int8_row_dequant_kernel"):
        assert k in names, k


def test_no_kernel_spills_outside_the_allowed_one(kernels):
    bad = []
    for name, f in kernels.items():
        allowed = next((v for k, v in SPILL_ALLOWED.items() if k in name), 0)
        if f.get("uses_dynamic_stack") != "false":
            bad.append((name, "dynamic stack"))
        if int(f["vgpr_spill_count"]) > allowed:
            bad.append((name, "vgpr spills", f["vgpr_spill_count"]))
        if allowed == 0 and int(f["private_segment_fixed_size"]) != 0:
            bad.append((name, "scratch bytes", f["private_segment_fixed_size"]))
    assert not bad, bad


def test_register_counts_the_launch_designs_rely_on(kernels):
    for sub, ceiling in VGPR_CEILING:
        hit = [(n, int(f["vgpr_count"])) for n, f in kernels.items() if sub in n]
        assert hit, sub
        for n, v in hit:
            assert v <= ceiling, (n, v, ceiling)


def test_parse_notes_on_a_hand_written_dump():
    text = """amdhsa.kernels:
  - .agpr_count:     0
    .args:
      - .offset:         0
        .size:           8
    .name:           k_one
    .private_segment_fixed_size: 0
    .sgpr_spill_count: 0
    .uses_dynamic_stack: false
    .vgpr_count:     14
    .vgpr_spill_count: 0
  - .agpr_count:     0
    .name:           k_two
    .private_segment_fixed_size: 12
    .vgpr_count:     256
    .vgpr_spill_count: 2
amdhsa.target:   amdgcn-amd-amdhsa--gfx950
"""
    k = _parse_notes(text)
    assert set(k) == {"k_one", "k_two"}
    assert k["k_one"]["vgpr_count"] == "14" and k["k_one"]["uses_dynamic_stack"] == "false"
    assert k["k_two"]["vgpr_spill_count"] == "2" and k["k_two"]["private_segment_fixed_size"] == "12"
