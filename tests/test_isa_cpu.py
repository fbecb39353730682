"""Checks on the gfx950 machine code of this library's own GEMM kernels
(read from the device code object in the in-tree build; host-side only).

* The FP32-scale FP8 kinds must contain the unscaled block product
  v_mfma_f32_16x16x128_f8f6f4 and no scaled one: their partials are promoted
  by FP32 FMAs, and a scaled instruction would apply E8M0 scale bytes of 0
  (2^-127) to every product.  The UE8M0 kinds must use the scaled instruction
  (the power-of-two scales are applied inside the matrix core).
* No kernel of the library (GEMMs, casts, pack, MoE routing and combine)
  may spill to scratch (private segment size 0).

Skipped when the library has not been built here or the LLVM tools of the
ROCm install are missing."""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "moe_grouped_gemm_x128_amd", "_build")
OBJ = os.path.join(BUILD, "gemm.hip.o")
LLVM = "/opt/rocm/lib/llvm/bin"
TOOLS = ["llvm-objcopy", "clang-offload-bundler", "llvm-objdump", "llvm-readelf"]

# gemm_kernel<TileShape<BM, BN, WM, WN, S>, KIND, SF, MODE, OUT>
KERNEL_RE = re.compile(r"gemm_kernelINS0_9TileShapeI((?:Li\d+E){5})EELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)E")


def _extract(obj, d):
    """The gfx950 code object bundled in a hipcc object file."""
    if not os.path.exists(obj):
        pytest.skip("library not built in-tree")
    if not all(os.path.exists(os.path.join(LLVM, t)) for t in TOOLS):
        pytest.skip("ROCm LLVM tools not found")
    base = os.path.basename(obj)
    fat = str(d / (base + ".fatbin"))
    co = str(d / (base + "_gfx950.co"))
    subprocess.run([os.path.join(LLVM, "llvm-objcopy"), f"--dump-section=.hip_fatbin={fat}", obj, str(d / "x.o")],
                   check=True, capture_output=True)
    subprocess.run([os.path.join(LLVM, "clang-offload-bundler"), "--unbundle", "--type=o",
                    "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--input={fat}", f"--output={co}"],
                   check=True, capture_output=True)
    return co


@pytest.fixture(scope="module")
def code_object(tmp_path_factory):
    return _extract(OBJ, tmp_path_factory.mktemp("isa"))


def _functions(co):
    """{mangled kernel name: disassembly text} for every GEMM kernel."""
    out = subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", co], check=True, capture_output=True,
                         text=True).stdout
    funcs, cur = {}, None
    for line in out.splitlines():
        m = re.match(r"^[0-9a-f]+ <(\S+)>:$", line)
        if m:
            cur = m.group(1) if "gemm_kernel" in m.group(1) else None
            if cur:
                funcs[cur] = []
        elif cur:
            funcs[cur].append(line)
    return {k: "\n".join(v) for k, v in funcs.items()}


def test_fp32_scale_kinds_use_the_unscaled_block_product(code_object):
    funcs = _functions(code_object)
    checked = 0
    for name, text in funcs.items():
        m = KERNEL_RE.search(name)
        assert m, name
        kind, sf = int(m.group(2)), int(m.group(3))
        if kind != 0:  # BF16 kind
            continue
        if sf & 1:  # UE8M0: scales inside the matrix core
            assert "v_mfma_scale_f32_16x16x128_f8f6f4" in text, name
        else:
            assert "v_mfma_scale_f32" not in text, name
            assert "v_mfma_f32_16x16x128_f8f6f4" in text, name
        checked += 1
    assert checked >= 20


def test_no_gemm_kernel_spills(code_object):
    notes = subprocess.run([os.path.join(LLVM, "llvm-readelf"), "--notes", code_object], check=True,
                           capture_output=True, text=True).stdout
    name, seen = None, 0
    for line in notes.splitlines():
        s = line.strip()
        if s.startswith(".name:"):
            name = s.split(":", 1)[1].strip()
        elif s.startswith(".private_segment_fixed_size:") and name and "gemm_kernel" in name:
            assert int(s.split(":", 1)[1]) == 0, f"{name} uses scratch"
            seen += 1
    assert seen >= 20


@pytest.mark.parametrize("src", ["quant.hip", "moe.hip"])
def test_no_other_kernel_spills(src, tmp_path):
    co = _extract(os.path.join(BUILD, src + ".o"), tmp_path)
    notes = subprocess.run([os.path.join(LLVM, "llvm-readelf"), "--notes", co], check=True, capture_output=True,
                           text=True).stdout
    name, seen = None, 0
    for line in notes.splitlines():
        s = line.strip()
        if s.startswith(".name:"):
            name = s.split(":", 1)[1].strip()
        elif s.startswith(".private_segment_fixed_size:") and name:
            assert int(s.split(":", 1)[1]) == 0, f"{name} uses scratch"
            seen += 1
    assert seen >= 3


def _lds_sizes(co):
    """{(BM, BN, KIND, MODE): static LDS sizes} of the GEMM kernels in the code
    object (each kernel's metadata map opens with .agpr_count)."""
    notes = subprocess.run([os.path.join(LLVM, "llvm-readelf"), "--notes", co], check=True, capture_output=True,
                           text=True).stdout
    out = {}
    for entry in re.split(r"\n\s*- \.agpr_count:", notes)[1:]:
        name = re.search(r"\.name:\s+(\S+)", entry)
        m = KERNEL_RE.search(name.group(1)) if name else None
        if not m:
            continue
        bm, bn = (int(x) for x in re.findall(r"\d+", m.group(1))[:2])
        size = int(re.search(r"\.group_segment_fixed_size:\s+(\d+)", entry).group(1))
        out.setdefault((bm, bn, int(m.group(2)), int(m.group(4))), set()).add(size)
    return out


def test_query_config_reports_the_kernels_static_lds(code_object):
    """lds_bytes of query_config is the static LDS of a kernel that launch
    runs (the code object's group segment size), the contiguous 256-row
    tiles' run-scan words included."""
    from moe_grouped_gemm_x128_amd import binding

    sizes = _lds_sizes(code_object)
    assert len(sizes) >= 20
    b = binding
    kinds = [(b.DG_KIND_DENSE, 0, 0), (b.DG_KIND_CONTIGUOUS, 0, 1), (b.DG_KIND_MASKED, 0, 2),
             (b.DG_KIND_BF16_DENSE, 1, 0), (b.DG_KIND_BF16_CONTIGUOUS, 1, 1), (b.DG_KIND_BF16_MASKED, 1, 2),
             (b.DG_KIND_DENSE_ROWB, 0, 0), (b.DG_KIND_CONTIGUOUS_ROWB, 0, 1), (b.DG_KIND_MASKED_ROWB, 0, 2)]
    shapes = [(4, 128, 7168, 2048), (4, 4096, 7168, 2048), (4, 4096, 2112, 7168), (4, 4096, 7168, 16384),
              (4, 4096, 100, 512), (4, 8193 * 128, 4096, 7168)]
    checked = 0
    for kind, k_id, mode in kinds:
        for G, M, N, K in shapes:
            c = binding.query_config(kind, G, M, N, K)
            key = (c["block_m"], c["block_n"], k_id, mode)
            assert c["lds_bytes"] in sizes.get(key, ()), (kind, (G, M, N, K), key, c["lds_bytes"], sizes.get(key))
            if c["block_n2"]:
                key2 = (c["block_m"], c["block_n2"], k_id, mode)
                assert c["lds_bytes2"] in sizes.get(key2, ()), (kind, (G, M, N, K), key2, c["lds_bytes2"])
            checked += 1
    assert checked == len(kinds) * len(shapes)
