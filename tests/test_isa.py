"""Checks on the gfx950 machine code of libreduce.so (no GPU needed).

The device code objects are unbundled from the built library, disassembled
with ROCm's llvm-objdump and read with llvm-readelf / llvm-readobj.  The
tests pin properties the design relies on but no parity test can see:

* no packed fp32 VALU forms anywhere (the library is built with that
  target feature off, and nothing may bring them back);
* no writes through the scalar data cache (scalar stores, scalar atomics or
  that cache's write-back / discard);
* no scratch memory and no VGPR spills in any kernel;
* fp32 subnormals are preserved (the kernel descriptors' fp32 denormal mode
  is "flush nothing");
* the streaming kernels read with non-temporal 16-byte loads, max / min fold
  with the three-input v_max3_f32 / v_min3_f32, the wave reduction uses the
  DPP row shifts and row broadcasts, the atomic sum uses the hardware
  float atomic add and the atomic max / min the integer atomics.
"""
from __future__ import annotations

import os
import re
import shutil
import struct
import subprocess

import pytest
import yaml

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBRARY = os.path.join(ROOT, "fp32_reductions_amd", "libreduce.so")
LLVM = "/opt/rocm/llvm/bin"


def _tool(name):
    path = os.path.join(LLVM, name)
    if not os.path.exists(path):
        pytest.skip("%s not found" % path)
    return path


def _demangle(names):
    out = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True,
                         text=True, check=True).stdout.split("\n")
    return dict(zip(names, out))


class CodeObject:
    """One unbundled gfx950 code object: per-kernel disassembly, metadata
    notes and kernel-descriptor words."""

    def __init__(self, path):
        self.path = path
        asm = subprocess.run([_tool("llvm-objdump"), "-d", "--mcpu=gfx950", path],
                             capture_output=True, text=True, check=True).stdout
        self.text = {}
        cur = None
        for line in asm.splitlines():
            m = re.match(r"^[0-9a-f]+ <(.+)>:$", line)
            if m:
                cur = m.group(1)
                self.text[cur] = []
            elif cur is not None:
                self.text[cur].append(line)
        self.text = {k: "\n".join(v) for k, v in self.text.items()}

        notes = subprocess.run([_tool("llvm-readobj"), "--notes", path],
                               capture_output=True, text=True, check=True).stdout
        doc = notes.split("AMDGPU Metadata: ", 1)[1]
        doc = doc[:doc.index("\n...")]
        self.meta = {k[".name"]: k for k in yaml.safe_load(doc)["amdhsa.kernels"]}

        syms = subprocess.run([_tool("llvm-readelf"), "-s", "-S", "-W", path],
                              capture_output=True, text=True, check=True).stdout
        sections = {}
        for m in re.finditer(r"\[\s*(\d+)\]\s+(\S+)\s+\S+\s+([0-9a-f]+)\s+([0-9a-f]+)", syms):
            sections[int(m.group(1))] = (int(m.group(3), 16), int(m.group(4), 16))
        with open(path, "rb") as fh:
            blob = fh.read()
        self.rsrc1 = {}
        for m in re.finditer(r"([0-9a-f]+)\s+64\s+OBJECT\s+\S+\s+\S+\s+(\d+)\s+(\S+)\.kd$",
                             syms, re.M):
            addr, shndx, name = int(m.group(1), 16), int(m.group(2)), m.group(3)
            sec_addr, sec_off = sections[shndx]
            off = sec_off + (addr - sec_addr)
            # amdhsa kernel descriptor: compute_pgm_rsrc1 is the word at byte 48
            self.rsrc1[name] = struct.unpack_from("<I", blob, off + 48)[0]


@pytest.fixture(scope="module")
def code(tmp_path_factory):
    if not os.path.exists(LIBRARY):
        pytest.skip("libreduce.so is not built")
    d = tmp_path_factory.mktemp("isa")
    lib = os.path.join(str(d), "libreduce.so")
    shutil.copy(LIBRARY, lib)
    # Unbundling writes each bundle entry next to the input file.
    subprocess.run([_tool("llvm-objdump"), "--offloading", lib], capture_output=True,
                   check=True)
    objs = [CodeObject(os.path.join(str(d), f)) for f in sorted(os.listdir(str(d)))
            if f.endswith("gfx950")]
    assert objs, "no gfx950 code object in libreduce.so"
    text, meta, rsrc1 = {}, {}, {}
    for o in objs:
        text.update(o.text)
        meta.update(o.meta)
        rsrc1.update(o.rsrc1)
    names = _demangle(sorted(text))
    return {"text": {names[k]: v for k, v in text.items()},
            "meta": {names.get(k, k): v for k, v in meta.items()},
            "rsrc1": {names.get(k, k): v for k, v in rsrc1.items()},
            "all": "\n".join(text.values())}


def kernels(code, pattern):
    found = {k: v for k, v in code["text"].items() if re.search(pattern, k)}
    assert found, "no kernel matches %r" % pattern
    return found


def test_every_kernel_has_metadata(code):
    assert len(code["meta"]) >= 60, sorted(code["meta"])
    assert set(code["meta"]) == set(code["rsrc1"])


def test_no_packed_fp32(code):
    bad = re.findall(r"\bv_pk_(?:add|mul|fma)_f32\b", code["all"])
    assert not bad, "packed fp32 instructions present: %d" % len(bad)


def test_no_scalar_cache_writes(code):
    bad = re.findall(r"\bs_(?:store|buffer_store|scratch_store|atomic|buffer_atomic)\w*"
                     r"|\bs_dcache_(?:wb|discard)\w*", code["all"])
    assert not bad, sorted(set(bad))


def test_no_scratch_and_no_vgpr_spills(code):
    for name, m in code["meta"].items():
        assert m[".private_segment_fixed_size"] == 0, name
        assert m[".vgpr_spill_count"] == 0, name


def test_fp32_subnormals_preserved(code):
    for name, r1 in code["rsrc1"].items():
        assert (r1 >> 16) & 3 == 3, "%s: fp32 denormal mode %d" % (name, (r1 >> 16) & 3)


def test_streaming_loads_are_nontemporal_dwordx4(code):
    for pat in (r"reduce1d_stream_kernel<", r"reduce1d_summaxmin_stream_kernel",
                r"rows_seg_kernel<", r"rows_split_kernel<", r"colred_kernel<.*, true, \d+, \d+>",
                r"colred_narrow_kernel<.*, true>", r"colred_wide_kernel<"):
        for name, txt in kernels(code, pat).items():
            assert re.search(r"global_load_dwordx4 .* nt\b", txt), name


def test_max_min_fold_three_at_a_time(code):
    for name, txt in kernels(code, r"reduce1d_stream_kernel<red_dev::OpMax, (true|false)>").items():
        assert txt.count("v_max3_f32") >= 8, name
    for name, txt in kernels(code, r"reduce1d_stream_kernel<red_dev::OpMin, (true|false)>").items():
        assert txt.count("v_min3_f32") >= 8, name


def test_wave_reduction_uses_dpp(code):
    for name, txt in kernels(code, r"reduce1d_(stream|finish)_kernel<").items():
        for ctrl in ("row_shr:1", "row_shr:2", "row_shr:4", "row_shr:8",
                     "row_bcast:15", "row_bcast:31"):
            assert re.search(r"\b%s\b" % ctrl, txt), (name, ctrl)


def test_atomic_sum_uses_hardware_float_add(code):
    for name, txt in kernels(code, r"reduce1d_atomic_kernel<red_dev::OpSum, (true|false)>").items():
        assert "global_atomic_add_f32" in txt, name
    for name, txt in kernels(code, r"reduce1d_atomic_kernel<red_dev::OpMax, (true|false)>").items():
        assert "global_atomic_smax" in txt and "global_atomic_umin" in txt, name
    for name, txt in kernels(code, r"reduce1d_atomic_kernel<red_dev::OpMin, (true|false)>").items():
        assert "global_atomic_smin" in txt and "global_atomic_umax" in txt, name
