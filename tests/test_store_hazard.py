"""Static check of the built gfx950 code: no store of more than 64 bits is followed directly by
an instruction that writes one of its data VGPRs.

Such a store reads its data registers after it issues.  A buffer store whose scalar offset is
an SGPR gets no wait state from the compiler, and on gfx950 one such case stored stale values
(data dwords 0 and 3 of lanes 12-15 of every 16-lane row, in the rows whose data registers the
next instruction rewrote).  The library's 128-bit buffer stores therefore pass a constant
scalar offset, which makes the compiler keep the wait state; this test reads the code objects
of the built libflk.so and fails if any such pair is back."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "quantized_kv_cache_amd", "libflk.so")
LLVM = "/opt/rocm/llvm/bin"
MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
WIDE_STORE = re.compile(r"^\s*(buffer|global|flat|scratch)_store_(dwordx3|dwordx4|b96|b128)\s+(?:v\[\d+:\d+\],\s*)?"
                        r"v\[(\d+):(\d+)\]")
VDST = re.compile(r"^\s*v_\w+\s+v(?:\[(\d+):(\d+)\]|(\d+))(?=[,\s]|$)")


def _code_objects(tmp):
    """The gfx950 code objects of every offload bundle in libflk.so's .hip_fatbin section."""
    fat = os.path.join(tmp, "fatbin.bin")
    subprocess.run([f"{LLVM}/llvm-objcopy", f"--dump-section=.hip_fatbin={fat}", LIB], check=True)
    data = open(fat, "rb").read()
    starts = [m.start() for m in re.finditer(re.escape(MAGIC), data)]
    out = []
    for i, s in enumerate(starts):
        part = os.path.join(tmp, f"bundle{i}.bin")
        open(part, "wb").write(data[s:starts[i + 1] if i + 1 < len(starts) else len(data)])
        co = os.path.join(tmp, f"bundle{i}.co")
        r = subprocess.run([f"{LLVM}/clang-offload-bundler", "--unbundle", "--type=o",
                            "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--input={part}", f"--output={co}"],
                           capture_output=True)
        if r.returncode == 0 and os.path.getsize(co) > 0:
            out.append(co)
    return out


def _instructions(co):
    text = subprocess.run([f"{LLVM}/llvm-objdump", "-d", "--no-show-raw-insn", co], capture_output=True,
                          text=True, check=True).stdout
    for line in text.splitlines():
        s = line.split("//")[0].strip()
        if s and not s.endswith(">:") and not s.startswith("Disassembly") and ":" not in s.split()[0]:
            yield s


def _hazards(instrs):
    found = []
    for a, b in zip(instrs, instrs[1:]):
        m = WIDE_STORE.match(a)
        if not m:
            continue
        data = set(range(int(m.group(3)), int(m.group(4)) + 1))
        d = VDST.match(b)
        if not d:
            continue
        dst = set(range(int(d.group(1)), int(d.group(2)) + 1)) if d.group(1) else {int(d.group(3))}
        if data & dst:
            found.append((a, b))
    return found


@pytest.mark.skipif(not os.path.exists(LIB) or not os.path.exists(f"{LLVM}/llvm-objdump"),
                    reason="needs the built libflk.so and the ROCm LLVM tools")
def test_no_wide_store_data_overwritten_by_next_instruction(tmp_path):
    cos = _code_objects(str(tmp_path))
    assert cos, "no gfx950 code object found in libflk.so"
    n_stores, bad = 0, []
    for co in cos:
        instrs = list(_instructions(co))
        n_stores += sum(1 for s in instrs if WIDE_STORE.match(s))
        bad += _hazards(instrs)
    assert n_stores > 0, "the disassembly held no wide stores: the pattern no longer matches the tool's output"
    assert not bad, f"{len(bad)} wide stores whose data registers the next instruction writes, e.g. {bad[:3]}"


def test_checker_flags_the_hazard():
    """The matcher itself, on a hand-written pair and on its safe variants."""
    store = "buffer_store_dwordx4 v[68:71], v35, s[24:27], s38 offen"
    assert _hazards([store, "v_sub_f32_e32 v68, v34, v83"])
    assert _hazards([store, "v_mov_b64_e32 v[70:71], 0"])
    assert not _hazards([store, "s_nop 0", "v_sub_f32_e32 v68, v34, v83"])
    assert not _hazards([store, "v_sub_f32_e32 v72, v34, v83"])
    assert not _hazards(["buffer_store_dwordx2 v[68:69], v35, s[24:27], s38 offen", "v_mov_b32_e32 v68, 0"])
