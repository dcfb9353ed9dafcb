"""Static checks of the 128-key attention kernels' gfx950 code (CPU only:
hipcc cross-compiles).

* No register spills: the compiler's kernel-resource-usage remarks report 0
  spilled SGPRs and VGPRs for every instantiation.
* The phase waits are sound.  The LDS-DMA copies (buffer_load ... lds) are
  inline assembly the compiler does not track, and each phase ends with a
  hand-placed wait that leaves the copies of the latest softmax step in
  flight (s_waitcnt vmcnt(N), N > 0).  That count is only right while no
  other vector-memory operation is outstanding at such a wait: walking the
  code in order, every load or store that is not an LDS-DMA copy must be
  followed by a wait for zero outstanding operations before the next
  vmcnt(N > 0) wait.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_sparse_attention_mask_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "--cuda-device-only", "-S",
         "-Rpass-analysis=kernel-resource-usage"]
KERNELS = {"attn_pp.hip": ("attn_pp_128_128", "attn_pp_128_64", "attn_pp_crm_128_128", "attn_pp_crm_128_64"),
           "attn_ppg.hip": ("attn_ppg_128_128", "attn_ppg_128_64", "attn_ppx_128_128", "attn_ppx_128_64")}
# The kernel holding both the one-row and the pair body spills a few SGPRs
# to VGPR lanes around its row prologue and epilogue (its loops keep their
# operand reads pipelined); no VGPR spills anywhere.
SGPR_SPILLS_ALLOWED = {"attn_ppx_128_128": 16, "attn_ppx_128_64": 16}

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")


def _compile(src, tmp_path):
    out = tmp_path / (src + ".s")
    res = subprocess.run([HIPCC] + FLAGS + [os.path.join(CSRC, src), "-o", str(out)], capture_output=True,
                         text=True, timeout=600)
    assert res.returncode == 0, res.stderr[-2000:]
    return out.read_text(), res.stderr


def _remarks(stderr):
    """kernel name -> {remark field: value} from the resource-usage remarks."""
    out, cur = {}, None
    for line in stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?): (\d+) \[", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = int(m.group(2))
    return out


def _body(asm, name):
    m = re.search(r"^(_Z\S*%s\S*):.*$" % re.escape(name), asm, re.M)
    assert m, name
    start = m.end()
    end = asm.index("s_endpgm", start)
    return asm[start:end]


def _vmcnt(line):
    """The vmcnt a s_waitcnt waits for (None when it does not wait on vmcnt)."""
    m = re.search(r"vmcnt\((\d+)\)", line)
    if m:
        return int(m.group(1))
    if re.match(r"\s*s_waitcnt\s+0\s*$", line):
        return 0
    return None


# Loads and atomics other than the copies.  Stores are left out: they occur
# only in a row's epilogue, after its last copy wait, and in the kernel that
# holds two bodies the one body's epilogue stores precede the other body's
# code in the listing without preceding it in any execution.
_VMEM = re.compile(r"^\s*(buffer_load|global_load|flat_load|buffer_atomic|global_atomic|flat_atomic)\w*")


@pytest.mark.parametrize("src", sorted(KERNELS))
def test_no_spills_and_sound_phase_waits(src, tmp_path):
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        pytest.skip("hipcc not installed")
    asm, stderr = _compile(src, tmp_path)
    rem = _remarks(stderr)
    for k in KERNELS[src]:
        names = [n for n in rem if k + "E" in n]
        assert names, (k, list(rem))
        for n in names:
            assert rem[n].get("SGPRs Spill") <= SGPR_SPILLS_ALLOWED.get(k, 0), (n, rem[n])
            assert rem[n].get("VGPRs Spill") == 0, (n, rem[n])
        body = _body(asm, k + "E")
        foreign, partial_waits, copies = None, 0, 0
        for ln in body.splitlines():
            s = ln.split(";")[0]
            if _VMEM.match(s):
                if re.search(r"\blds\b", s):
                    copies += 1
                else:
                    foreign = s.strip()
                continue
            if "s_waitcnt" in s:
                v = _vmcnt(s)
                if v == 0:
                    foreign = None
                elif v is not None:
                    partial_waits += 1
                    assert foreign is None, (k, "outstanding at a partial wait: " + foreign)
        assert copies > 0 and partial_waits > 0, (k, copies, partial_waits)
