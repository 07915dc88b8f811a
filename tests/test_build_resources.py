"""Host-side checks of the built library's gfx950 code objects: no kernel uses
scratch memory or spills registers, and the two kernels that set the measured
rates keep the register budgets their occupancy needs. A register array that
the compiler can only index at run time lands in scratch memory (as a run-time
offset into a block-parameter array once did in the decode's new-token path);
these checks catch that without a GPU.

The code objects are read from the library's offload bundles and their
kernel metadata from llvm-readelf's notes dump. No GPU is needed."""
import os
import struct
import subprocess
import tempfile

import pytest
import yaml

import quantized_kv_cache_wht_amd as iq

READELF = "/opt/rocm/llvm/bin/llvm-readelf"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def _code_objects(lib_path):
    """The gfx950 entries of every offload bundle in the library (one per source file)."""
    data = open(lib_path, "rb").read()
    objs, start = [], 0
    while True:
        i = data.find(MAGIC, start)
        if i < 0:
            return objs
        start = i + len(MAGIC)
        p = start
        (n,) = struct.unpack_from("<Q", data, p)
        p += 8
        for _ in range(n):
            off, size, tsz = struct.unpack_from("<QQQ", data, p)
            p += 24
            triple = data[p:p + tsz].decode()
            p += tsz
            if triple.endswith("gfx950") and size:
                objs.append(data[i + off:i + off + size])


def _kernels(obj):
    with tempfile.NamedTemporaryFile(suffix=".o") as f:
        f.write(obj)
        f.flush()
        out = subprocess.run([READELF, "--notes", f.name], capture_output=True, text=True, check=True).stdout
    doc = out[out.index("---"):out.index("\n...", out.index("---"))]
    return yaml.safe_load(doc).get("amdhsa.kernels", [])


@pytest.fixture(scope="module")
def kernels():
    if not os.path.exists(READELF):
        pytest.skip("llvm-readelf not installed")
    ks = [k for obj in _code_objects(iq.library_path()) for k in _kernels(obj)]
    assert len(ks) > 40, "expected every instantiated kernel of the library"
    return {k[".name"]: k for k in ks}


def test_no_kernel_uses_scratch_or_spills(kernels):
    bad = {n: (k[".private_segment_fixed_size"], k.get(".vgpr_spill_count", 0), k.get(".sgpr_spill_count", 0))
           for n, k in kernels.items()
           if k[".private_segment_fixed_size"] or k.get(".vgpr_spill_count", 0) or k.get(".sgpr_spill_count", 0)}
    assert not bad, f"(scratch bytes, VGPR spills, SGPR spills) per kernel: {bad}"


def _one(kernels, prefix):
    hits = [k for n, k in kernels.items() if n.startswith(prefix)]
    assert len(hits) == 1, (prefix, [n for n in kernels if n.startswith(prefix[:30])])
    return hits[0]


def test_hot_kernels_keep_their_register_budgets(kernels):
    # the bulk encode (fp16 input, 3-bit K, WHT + SO(4)): at most 128 VGPRs for 4 waves per SIMD
    enc = _one(kernels, "_ZN2iq13append_kernelIDF16_Lb0ELb0EEEvNS_10AppendArgsE")
    assert enc[".vgpr_count"] <= 128, enc[".vgpr_count"]
    # the decode step's split kernel (G = 8, 3-bit K, new token in the launch): at most 168 for 3 waves
    dec = _one(kernels, "_ZN2iq19decode_split_kernelILi8ELi3ELb1EEEvNS_10DecodeArgsENS_8NewTokenE")
    assert dec[".vgpr_count"] <= 168, dec[".vgpr_count"]
