"""The gfx950 code objects inside libgift.so: the hot kernels keep their
working set in registers and LDS.

A kernel whose private segment (per-lane scratch memory) is not empty spills
registers or indexes a private array through memory; on the streaming paths
that multiplies the kernel's memory traffic (an FP4 decode whose unit buffers
went to scratch ran 4x slower).  The kernel metadata of each code object
(read with the ROCm LLVM tools from the library built here) must show a
private segment of zero bytes for every kernel of the headline unit, the
FP4 payload, the flat buckets and the multi-kernel route, and at most the
few bytes listed below for the others."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "fac_whitening_amd", "libgift.so")
TOOLS = "/opt/rocm/llvm/bin"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"

# kernels allowed a small private segment (bytes per lane), measured: the
# 16-replica FP8 decode's whole-tile stream, the grouped per-block launches
# and the statistics kernel's tile hand-over (outside its product loop)
ALLOWED = {
    "k_rank_decode<0, 16, 0>": 64, "k_rank_decode<1, 16, 0>": 64,
    "k_rank_group": 16,
    "k_stats_mfma": 256,
}
# kernels that must keep everything in registers and LDS
HOT = ["k_rank_encode<0, 0>", "k_rank_encode<0, 1>", "k_rank_decode<0, 8, 0>", "k_rank_decode<0, 8, 1>",
       "k_rank_decode<0, 4, 0>", "k_rank_encode_ef<0, 0>", "k_euclid_encode<0, 0>", "k_euclid_decode<0, 8, 0>",
       "k_rank_encode<2, 0>", "k_euclid_encode<2, 0>", "k_rank_encode_ef<2, 0>", "k_euclid_encode_ef<2, 0>",
       "k_rank_decode<2, 4, 0>", "k_rank_decode<2, 8, 0>", "k_quantize_fp4", "k_dequant_sum_fp4",
       "k_bucket_amax", "k_bucket_quantize", "k_bucket_dequant_sum", "k_project", "k_lr_apply", "k_quantize",
       "k_dequant_sum", "k_aq<48>", "k_aq32<48>",
       # register-resident Householder rows: fully unrolled (a per-file unroll threshold in the build)
       "k_tridiag_coef<48>"]


def _tool(name):
    p = os.path.join(TOOLS, name)
    return p if os.path.exists(p) else shutil.which(name)


@pytest.fixture(scope="module")
def private_sizes(tmp_path_factory):
    tools = [_tool(n) for n in ("llvm-objcopy", "clang-offload-bundler", "llvm-readelf")]
    tools.append(_tool("llvm-cxxfilt") or shutil.which("c++filt"))
    if not os.path.exists(LIB) or not all(tools):
        pytest.skip("libgift.so or the ROCm LLVM tools are missing")
    objcopy, bundler, readelf, cxxfilt = tools
    d = tmp_path_factory.mktemp("co")
    fat = d / "fatbin"
    subprocess.run([objcopy, f"--dump-section=.hip_fatbin={fat}", LIB, str(d / "lib.so")], check=True,
                   capture_output=True)
    data = fat.read_bytes()
    starts = [m.start() for m in re.finditer(re.escape(MAGIC), data)]
    sizes = {}
    for i, st in enumerate(starts):
        end = starts[i + 1] if i + 1 < len(starts) else len(data)
        (d / f"b{i}").write_bytes(data[st:end])
        r = subprocess.run([bundler, "--unbundle", "--type=o", "--targets=hipv4-amdgcn-amd-amdhsa--gfx950",
                            f"--input={d / f'b{i}'}", f"--output={d / f'c{i}'}"], capture_output=True)
        if r.returncode != 0:
            continue
        notes = subprocess.run([readelf, "--notes", str(d / f"c{i}")], capture_output=True, text=True,
                               check=True).stdout
        name = None
        for line in notes.splitlines():
            m = re.match(r"\s+\.name:\s+(\S+)", line)
            if m:
                name = m.group(1)
            m = re.match(r"\s+\.private_segment_fixed_size:\s+(\d+)", line)
            if m and name:
                sizes[name] = int(m.group(1))
    names = list(sizes)
    demangled = subprocess.run([cxxfilt], input="\n".join(names), capture_output=True, text=True,
                               check=True).stdout.splitlines()
    # "void gift::k<...>(args)" for templates, "gift::k(args)" otherwise
    return {re.sub(r"^(void )?gift::", "", dm).split("(")[0]: sizes[n] for n, dm in zip(names, demangled)}


def test_every_kernel_is_in_the_code_objects(private_sizes):
    for k in HOT:
        assert any(name.startswith(k) for name in private_sizes), k


def test_hot_kernels_use_no_scratch(private_sizes):
    bad = {n: s for n, s in private_sizes.items() if s and any(n.startswith(k) for k in HOT)
           and not any(n.startswith(a) for a in ALLOWED)}
    assert not bad, bad


def test_other_kernels_stay_within_their_measured_scratch(private_sizes):
    for n, s in private_sizes.items():
        if s == 0:
            continue
        limit = max([v for a, v in ALLOWED.items() if n.startswith(a)] or [0])
        assert s <= limit, (n, s)
