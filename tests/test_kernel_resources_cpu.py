"""Resource audit of every libgqa kernel, from the compiler's own report (no GPU needed).

Each HIP source is compiled for gfx950 to device assembly with the library's build flags, and
the kernel descriptors the compiler emits (LDS bytes, registers, scratch, spills) are checked
against what the launch shapes rely on:

- LDS: the exact layout of each kernel, and at most 80 KiB for the kernels that place two
  workgroups on a compute unit (160 KiB of LDS per CU);
- registers: at most 256 per lane where two waves share a SIMD, 512 where one wave does;
- scratch: none, except two kernels that keep one or two values in scratch across their main
  loop; for those the test checks that no scratch access sits inside any loop.
"""

import os
import re
import shutil
import subprocess

import pytest
import yaml

from gqa_causal_flash_amd import build as gbuild

HIPCC = gbuild.HIPCC

# kernel (demangled prefix) -> (LDS bytes, register budget per lane, scratch bytes allowed)
EXPECTED = {
    "prefill_causal_fwd<1, 8>": (131072, 256, 0),  # 1 workgroup of 8 waves per CU: 2 waves per SIMD
    "prefill_causal_fwd<1, 4>": (131072, 512, 0),  # 128-row q-blocks: 1 workgroup of 4 waves, 1 wave per SIMD
    "prefill_causal_varlen": (131072, 256, 0),   # same body
    "prefill_causal_e4m3": (98304, 256, 0),
    "prefill_merge": (0, 256, 0),
    "prefill_merge_varlen": (0, 256, 0),
    "prefill_varlen_prepass": (1024, 512, 0),
    "paged_prepass": (65668, 512, 0),
    "paged_fwd": (65792, 256, 0),                # 2 workgroups of 4 waves per CU
    "paged_merge": (0, 256, 0),
    "verify_fwd<1>": (81920, 512, 0),            # 2 workgroups of 2 waves per CU: 1 wave per SIMD
    "verify_fwd<2>": (81920, 256, 16),           # 2 workgroups of 4 waves per CU
    "verify_merge": (10368, 256, 0),
}
TWO_PER_CU = ("paged_fwd", "verify_fwd<1>", "verify_fwd<2>")
LDS_PER_CU = 160 * 1024


def _demangle(name: str) -> str:
    """gqa::(anonymous)::<ident>[<int args>](...) -> "ident" or "ident<a, b>"."""
    base = re.search(r"_GLOBAL__N_1(\d+)", name)
    n = int(base.group(1))
    rest = name[base.end():]
    ident = rest[:n]
    args = re.match(r"ILi(\d+)E(?:Li(\d+)E)?E", rest[n:])
    if args:
        vals = [a for a in args.groups() if a is not None]
        return f"{ident}<{', '.join(vals)}>"
    return ident


def _kernels_and_loops(asm: str):
    m = re.search(r"\.amdgpu_metadata\n(.*?)\n\s*\.end_amdgpu_metadata", asm, re.S)
    meta = yaml.safe_load(m.group(1).replace("\t", "    "))
    kernels = {_demangle(k[".name"]): k for k in meta["amdhsa.kernels"]}
    # scratch accesses inside loops, per function (the compiler marks loop blocks);
    # the count of loop blocks seen shows that the markers were found at all
    in_loop_scratch = {}
    loop_blocks = {}
    func, in_loop = None, False
    for line in asm.splitlines():
        fm = re.match(r"^(_Z\w+):", line)
        if fm:
            # kernels live in the anonymous namespace; other labels (device variables) end the function
            func = _demangle(fm.group(1)) if "_GLOBAL__N_1" in fm.group(1) else None
            in_loop = False
            continue
        if re.match(r"^(\.LBB\w+:|; %bb\.\d+:)", line):
            in_loop = "Loop Header" in line or "in Loop:" in line
            if in_loop:
                loop_blocks[func] = loop_blocks.get(func, 0) + 1
            continue
        if func and "scratch_" in line.split(";")[0] and in_loop:
            in_loop_scratch.setdefault(func, []).append(line.strip())
    for name, k in kernels.items():
        k["loop_blocks"] = loop_blocks.get(name, 0)
    return kernels, in_loop_scratch


@pytest.fixture(scope="module")
def report(tmp_path_factory):
    if not os.path.exists(HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm")
    kernels, loops = {}, {}
    for src in gbuild.sources():
        if not src.endswith(".hip"):
            continue
        s = str(out / (os.path.basename(src) + ".s"))
        cmd = [HIPCC, *gbuild.DEVICE, *gbuild.COMMON, "--cuda-device-only", "-S", src, "-o", s]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        k, lo = _kernels_and_loops(open(s).read())
        kernels.update(k)
        loops.update(lo)
    return kernels, loops


def test_main_loops_are_seen(report):
    kernels, _ = report
    for name in ("prefill_causal_fwd<1, 8>", "prefill_causal_e4m3", "paged_fwd", "verify_fwd<1>", "verify_fwd<2>"):
        assert kernels[name]["loop_blocks"] > 0, name


def test_every_kernel_is_audited(report):
    kernels, _ = report
    for name in kernels:
        assert any(name.startswith(e) or name == e for e in EXPECTED), f"unaudited kernel {name}"
    for e in EXPECTED:
        assert any(n.startswith(e) or n == e for n in kernels), f"kernel {e} not built"


@pytest.mark.parametrize("prefix", sorted(EXPECTED))
def test_kernel_resources(report, prefix):
    kernels, loops = report
    names = [n for n in kernels if n == prefix or (prefix.endswith("<") and n.startswith(prefix))]
    assert names, prefix
    lds, regs, scratch = EXPECTED[prefix]
    for n in names:
        k = kernels[n]
        assert k[".group_segment_fixed_size"] == lds, (n, k[".group_segment_fixed_size"])
        assert k[".group_segment_fixed_size"] <= LDS_PER_CU
        if prefix in TWO_PER_CU:
            assert 2 * k[".group_segment_fixed_size"] <= LDS_PER_CU, n
        assert k[".vgpr_count"] <= regs, (n, k[".vgpr_count"])
        assert k[".sgpr_spill_count"] == 0, n
        assert k[".private_segment_fixed_size"] <= scratch, (n, k[".private_segment_fixed_size"])
        if scratch == 0:
            assert k[".vgpr_spill_count"] == 0, n
        assert not loops.get(n), (n, loops.get(n))


def test_demangle():
    assert _demangle("_ZN3gqa12_GLOBAL__N_118prefill_causal_fwdILi1ELi8EEEvNS0_13PrefillParamsE") == \
        "prefill_causal_fwd<1, 8>"
    assert _demangle("_ZN3gqa12_GLOBAL__N_110verify_fwdILi2EEEvNS0_12VerifyParamsE") == "verify_fwd<2>"
    assert _demangle("_ZN3gqa12_GLOBAL__N_19paged_fwdENS0_11PagedParamsE") == "paged_fwd"


def test_scratch_in_a_loop_is_reported():
    """A spill reload inside a loop block of a synthetic listing is found; one outside is not."""
    asm = "\n".join([
        "_ZN3gqa12_GLOBAL__N_13fooENS0_1PE:",
        "; %bb.0:",
        "\tscratch_store_dword off, v1, off ; 4-byte Folded Spill",
        ".LBB0_1:                               ; =>This Inner Loop Header: Depth=1",
        "\tv_add_u32 v2, v2, v3",
        "; %bb.2:                               ;   in Loop: Header=BB0_1 Depth=1",
        "\tscratch_load_dword v4, off, off ; 4-byte Folded Reload",
        ".LBB0_3:",
        "\tscratch_load_dword v1, off, off ; 4-byte Folded Reload",
        ".amdgpu_metadata",
        "amdhsa.kernels:",
        "  - .name: _ZN3gqa12_GLOBAL__N_13fooENS0_1PE",
        "\t.end_amdgpu_metadata",
    ])
    kernels, loops = _kernels_and_loops(asm)
    assert list(kernels) == ["foo"]
    assert kernels["foo"]["loop_blocks"] == 2
    assert loops == {"foo": ["scratch_load_dword v4, off, off ; 4-byte Folded Reload"]}
