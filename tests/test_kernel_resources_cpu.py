"""Resource pins on the built library's own gfx950 code objects, on the CPU.

libvrc.so carries one code object per element type.  This test takes them
out of the library's offload section, reads each kernel's metadata note and
disassembles them (all of it code built here from this repository's
sources), and checks what the kernels are meant to be:

* no kernel uses private (scratch) memory or a dynamic stack, so nothing
  spills to memory; the few VGPR spills go to AGPRs, in the 256-lane fused
  all-reduce kernels of 10 ranks and up that hold more than 256 registers;
  every kernel is compiled for 64-lane waves;
* LDS is used only by the realigned all-reduce kernels, at most 8,320 bytes
  per workgroup (one group of sums), and by the phased ones, 128 KiB (32
  sums per lane; the ring-order one 160 KiB, 40 sums);
* every vector memory access is a global_* or ds_* instruction: no flat_
  access (it would count against the LDS counter and force coarser waits),
  and no store or atomic of any other kind than global stores and the
  phased kernels' 64-bit atomic add of their meeting count (the scalar unit
  only loads the kernel arguments and reads the clock);
* the headline kernel (bf16, 8 ranks, one-wave workgroups, one tile per
  wave) fits 128 VGPRs, so four of its workgroups per CU run as one wave
  per SIMD with room to spare."""
import os
import re
import subprocess

import pytest

import ring_all_reduce_virtual_amd as vrc

LLVM = "/opt/rocm/llvm/bin"
TOOLS = {t: os.path.join(LLVM, t) for t in ("llvm-objcopy", "clang-offload-bundler", "llvm-readelf", "llvm-objdump")}
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
HEADLINE = "_ZN3vrc17k_fused_allreduceINS_4BF16ELi8ELi1ELb1ENS_8RankFoldELi64EEEvNS_11FusedArArgsE"


@pytest.fixture(scope="module")
def code_objects(tmp_path_factory):
    missing = [p for p in TOOLS.values() if not os.path.exists(p)]
    if missing:
        pytest.skip(f"LLVM tools not available: {missing}")
    if not os.path.exists(vrc.LIB_PATH):
        pytest.skip("libvrc.so is not built")
    d = tmp_path_factory.mktemp("code_objects")
    fat = d / "fatbin.bin"
    subprocess.run([TOOLS["llvm-objcopy"], "--dump-section", f".hip_fatbin={fat}", vrc.LIB_PATH, str(d / "lib.so")],
                   check=True, capture_output=True)
    blob = fat.read_bytes()
    starts = [m.start() for m in re.finditer(re.escape(MAGIC), blob)] + [len(blob)]
    objs = []
    for i in range(len(starts) - 1):
        part, obj = d / f"bundle{i}.bin", d / f"co{i}.o"
        part.write_bytes(blob[starts[i]:starts[i + 1]])
        subprocess.run([TOOLS["clang-offload-bundler"], "--unbundle", "--type=o", f"--input={part}",
                        f"--targets={TARGET}", f"--output={obj}"], check=True, capture_output=True)
        if obj.stat().st_size:
            objs.append(obj)
    return objs


def kernels(obj):
    """Per-kernel fields of the object's AMDGPU metadata note."""
    notes = subprocess.run([TOOLS["llvm-readelf"], "--notes", str(obj)], check=True, capture_output=True,
                           text=True).stdout
    out = []
    for entry in notes.split("\n  - .agpr_count:")[1:]:
        def field(key):
            return re.search(r"\n\s+\." + key + r":\s+(\S+)", entry).group(1)
        out.append({
            "name": field("name"), "agpr": int(entry.split("\n", 1)[0]), "vgpr": int(field("vgpr_count")),
            "vgpr_spill": int(field("vgpr_spill_count")), "private": int(field("private_segment_fixed_size")),
            "lds": int(field("group_segment_fixed_size")), "dynamic_stack": field("uses_dynamic_stack"),
            "wave": int(field("wavefront_size")),
        })
    return out


def mnemonics(obj):
    text = subprocess.run([TOOLS["llvm-objdump"], "-d", "--no-show-raw-insn", str(obj)], check=True,
                          capture_output=True, text=True).stdout
    return set(re.findall(r"^\s+([a-z_0-9]+)\b", text, re.M))


def test_one_code_object_per_element_type(code_objects):
    names = [[k["name"] for k in kernels(o)] for o in code_objects]
    assert len(code_objects) == 4
    for tag in ("4BF16", "3F16", "3F32", "3I32"):
        assert sum(any(tag + "E" in n for n in ns) for ns in names) == 1


def test_no_scratch_no_memory_spills(code_objects):
    total = 0
    for obj in code_objects:
        for k in kernels(obj):
            total += 1
            assert k["private"] == 0, k["name"]
            assert k["dynamic_stack"] == "false", k["name"]
            assert k["wave"] == 64, k["name"]
            if k["vgpr_spill"] or k["agpr"]:
                assert k["vgpr_spill"] <= k["agpr"], k["name"]
                assert ("k_fused_allreduce" in k["name"] and k["name"].endswith("ELi256EEEvNS_11FusedArArgsE")
                        or "phased" in k["name"]), k["name"]
    assert total > 1000


def test_lds_only_in_the_realigned_and_phased_kernels(code_objects):
    for obj in code_objects:
        for k in kernels(obj):
            if "realigned" in k["name"]:
                assert 0 < k["lds"] <= 8320, k
            elif "ring_order_allreduce_phased" in k["name"]:
                assert k["lds"] == 40 * 256 * 16, k  # 40 sums per lane of a 256-lane workgroup
            elif "phased" in k["name"]:
                assert k["lds"] == 32 * 256 * 16, k  # 32 sums per lane of a 256-lane workgroup
            else:
                assert k["lds"] == 0, k


def test_phased_kernels_fit_one_wave_per_simd(code_objects):
    """The phased kernels hold their sums in registers: at most 512 (VGPRs and
    AGPRs together, one wave per SIMD) and none spilled to memory."""
    found = 0
    for obj in code_objects:
        for k in kernels(obj):
            if "phased" in k["name"]:
                found += 1
                assert k["vgpr"] <= 512 and k["private"] == 0, k
    assert found == 4 * (11 + 2 + 11)  # per element type: rank fold at 6-16 ranks, butterfly at 8 and 16, ring order at 6-16


def test_memory_instructions_are_global_or_lds(code_objects):
    for obj in code_objects:
        ops = mnemonics(obj)
        assert not [m for m in ops if m.startswith(("flat_", "scratch_", "buffer_"))]
        writes = [m for m in ops if "store" in m or "atomic" in m]
        # the phased kernels' meeting count is the one atomic: a 64-bit vector add
        assert writes and all(m.startswith("global_store_") or m == "global_atomic_add_x2" for m in writes), \
            sorted(writes)
        loads = [m for m in ops if "load" in m]
        assert all(m.startswith(("global_load_", "s_load_")) for m in loads), sorted(loads)
        lds = [m for m in ops if m.startswith("ds_")]
        assert all(m.startswith(("ds_read", "ds_write")) for m in lds), sorted(lds)


def test_headline_kernel_registers(code_objects):
    found = [k for obj in code_objects for k in kernels(obj) if k["name"] == HEADLINE]
    assert len(found) == 1
    k = found[0]
    assert k["agpr"] == 0 and k["vgpr"] <= 128 and k["lds"] == 0


def functions(obj):
    """Disassembly per function: name -> list of instruction lines."""
    text = subprocess.run([TOOLS["llvm-objdump"], "-d", "--no-show-raw-insn", str(obj)], check=True,
                          capture_output=True, text=True).stdout
    out, cur = {}, None
    for line in text.splitlines():
        m = re.match(r"^[0-9a-f]+ <(.+)>:$", line)
        if m:
            cur = out.setdefault(m.group(1), [])
        elif cur is not None and line.strip() and not line.strip().startswith(";"):
            cur.append(line.strip())
    return out


def next_memory_step(body, i):
    """The first global access or s_waitcnt after instruction i."""
    for ins in body[i + 1:]:
        if ins.startswith(("global_", "s_waitcnt")):
            return ins
    return ""


def test_throttled_all_gather_waits_after_every_store(code_objects):
    """The fused all-gather's throttled form waits for each 16-byte store
    (vmcnt(0)) before the wave's next memory access; the plain form never
    waits for a store before the next one."""
    seen = {True: 0, False: 0}
    for obj in code_objects:
        for name, body in functions(obj).items():
            if "k_fused_all_gather" not in name:
                continue
            throttled = name.endswith("Lb1ELb1EEEvNS_11FusedAgArgsE")
            stores = [i for i, ins in enumerate(body) if ins.startswith("global_store_dwordx4")]
            assert stores, name
            after = [next_memory_step(body, i) for i in stores]
            if throttled:
                assert all(a.startswith("s_waitcnt") and "vmcnt(0)" in a for a in after), (name, after)
            else:  # at most a wait for the next output pointer (lgkmcnt), never for the store
                assert not any("vmcnt" in a for a in after), (name, after)
            seen[throttled] += 1
    assert seen == {True: 4, False: 4}  # both forms, one per element type
