"""Static check of the generated gfx950 assembly of the 16-bit kernels.

The dK/dV kernel issues its accumulating MFMAs (dK, dV in accumulation registers) from inline
assembly, so the compiler's hazard recognizer does not see them.  gfx950 needs two wait states
between a VALU write of a VGPR and an MFMA reading it as a source.  This test compiles the
kernels to assembly with the library's flags and fails if any such MFMA reads a VGPR that one
of the two preceding instructions wrote (an s_nop counts its wait states).
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "variable_length_flashattention_fa_amd", "csrc")


def _regs(tok):
    m = re.match(r"v\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _hazards(asm_text):
    found = []
    for m in re.finditer(r"^(_ZN2fa\w+):", asm_text, re.M):
        start = m.end()
        end = asm_text.index(".Lfunc_end", start)
        ins = []
        for line in asm_text[start:end].splitlines():
            t = line.split(";")[0].strip()
            if not t or t.startswith(".") or t.endswith(":"):
                continue
            ins.append(t)
        for k, t in enumerate(ins):
            if not t.startswith("v_mfma") or " a[" not in t.split(",")[0] + " ":
                continue
            ops = [x.strip() for x in t.split(None, 1)[1].split(",")]
            srcs = _regs(ops[1]) | _regs(ops[2])
            waits = 0
            for back in range(k - 1, max(k - 6, -1), -1):
                u = ins[back]
                op = u.split()[0]
                if op == "s_nop":
                    waits += int(u.split()[1], 0) + 1
                elif op.startswith("v_") and not op.startswith("v_mfma"):
                    dst = _regs(u.split(None, 1)[1].split(",")[0].strip()) if " " in u else set()
                    if dst & srcs:
                        found.append((m.group(1), u, t))
                    waits += 1
                else:
                    waits += 1
                if waits >= 2:
                    break
    return found


def test_checker_flags_a_planted_hazard():
    text = ("\n_ZN2fa_probe:\n\tv_mov_b32_e32 v70, v1\n"
            "\tv_mfma_f32_32x32x16_bf16 a[0:15], v[70:73], v[8:11], a[0:15]\n"
            "\tv_mov_b32_e32 v9, v1\n\ts_nop 1\n"
            "\tv_mfma_f32_32x32x16_bf16 a[0:15], v[70:73], v[8:11], a[0:15]\n.Lfunc_end0:\n")
    assert len(_hazards(text)) == 1


def _hipcc():
    return os.environ.get("HIPCC") or ("/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc")
                                       else shutil.which("hipcc"))


@pytest.fixture(scope="module")
def kernel_asm(tmp_path_factory):
    """Assembly of every 16-bit kernel part, compiled with the library's flags: {(source, part): text}."""
    hipcc = _hipcc()
    if not hipcc:
        pytest.skip("hipcc not available")
    import concurrent.futures as cf
    tmp = tmp_path_factory.mktemp("asm")
    parts = [("fa_bwd16.hip", "FA_BWD16_PART", i) for i in (1, 2, 3, 4)] + [("fa_fwd.hip", "FA_FWD_PART", i) for i in (1, 2)]

    def compile_part(job):
        src, macro, part = job
        out = tmp / f"{src}.{part}.s"
        cmd = [hipcc, "-O3", "-std=c++17", "-fPIC", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
               "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-mllvm", "-amdgpu-mfma-vgpr-form", f"-D{macro}={part}", "--cuda-device-only", "-S",
               "-o", str(out), os.path.join(CSRC, src)]
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        assert r.returncode == 0, r.stdout[-2000:]
        return out.read_text()

    with cf.ThreadPoolExecutor(max_workers=len(parts)) as ex:
        texts = list(ex.map(compile_part, parts))
    return {(src, part): t for (src, _, part), t in zip(parts, texts)}


@pytest.mark.slow
def test_no_valu_to_asm_mfma_hazard(kernel_asm):
    # the asm MFMAs live in the dK/dV kernels: parts 1 (bf16) and 2 (fp16)
    texts = [kernel_asm[("fa_bwd16.hip", 1)], kernel_asm[("fa_bwd16.hip", 2)]]
    assert "v_mfma_f32_32x32x16_bf16 a[" in texts[0]  # the asm MFMAs are there
    assert "v_mfma_f32_32x32x16_f16 a[" in texts[1]
    for text in texts:
        assert _hazards(text) == []


@pytest.mark.slow
def test_no_register_spills_or_scratch(kernel_asm):
    """Every backward and forward kernel of these parts fits its vector registers: no VGPR spills and no
    private (scratch) segment, so no scratch memory traffic anywhere.  Scalar registers may spill
    into VGPR lanes (v_writelane / v_readlane, no memory); those sit outside the tile loops."""
    checked = 0
    for text in kernel_asm.values():
        names = re.findall(r"^\s+\.name:\s+(_ZN2fa\w+)$", text, re.M)
        vspills = re.findall(r"\.vgpr_spill_count:\s+(\d+)", text)
        private = re.findall(r"\.amdhsa_private_segment_fixed_size\s+(\d+)", text)
        assert names and len(vspills) == len(names) and len(private) == len(names), "metadata layout changed"
        assert [n for n, x in zip(names, vspills) if int(x)] == []
        assert [n for n, x in zip(names, private) if int(x)] == []
        checked += len(names)
    # 4 backward parts x 12 instances; forward part 1 (bf16) 12, part 2 (fp16) 12 plus 6 fp32 forward instances
    assert checked == 78
