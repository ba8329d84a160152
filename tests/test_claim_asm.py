"""The dynamic forward's tile claim in the generated gfx950 assembly (CPU only:
hipcc compiles the kernel source to assembly here, nothing runs).

A claim is one global_atomic_add by lane 0 of wave 0, issued from inline asm
with the exec mask narrowed to that lane. The hardware does not hold back an
instruction that reads a register a vector memory operation has yet to
write, and the compiler treats an asm output as ready when the asm ends: a
copy or spill of the result register placed before a later wait would read
a stale value, and a stale claim names an old tile again (a tile done twice,
or a loader that never ends). The claim therefore waits for its atomic
inside the same asm. This checks that every such atomic in every forward
instantiation is followed directly by s_waitcnt vmcnt(0)."""
import os
import re
import subprocess

import pytest

from jagged_flashattention_amd import build as B


def _device_asm(tmp_path, src):
    out = tmp_path / (os.path.basename(src) + ".s")
    cmd = [B.hipcc(), *B.COMMON, "-x", "hip", "--cuda-device-only", "-S",
           os.path.join(B.CSRC, src), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        pytest.fail("hipcc -S failed:\n" + r.stderr[-2000:])
    return out.read_text()


def _instructions(text):
    for line in text.split("\n"):
        s = line.split(";", 1)[0].strip()
        if s and not s.startswith(".") and not s.endswith(":"):
            yield s


def claim_sites(asm):
    """(claims found, claims not followed at once by s_waitcnt vmcnt(0))."""
    ins = list(_instructions(asm))
    found, bad = 0, []
    for i, s in enumerate(ins):
        if re.match(r"global_atomic_add v\d+, .*\bsc0\b", s) and i > 0 and ins[i - 1] == "s_mov_b64 exec, 1":
            found += 1
            if i + 1 >= len(ins) or ins[i + 1] != "s_waitcnt vmcnt(0)":
                bad.append((s, ins[i + 1] if i + 1 < len(ins) else None))
    return found, bad


def test_claim_site_check_flags_a_deferred_wait():
    """The check itself: an atomic whose wait comes later is flagged."""
    good = "s_mov_b64 exec, 1\nglobal_atomic_add v3, v[4:5], v6, off sc0\ns_waitcnt vmcnt(0)\n"
    late = ("s_mov_b64 exec, 1\nglobal_atomic_add v3, v[4:5], v6, off sc0\n"
            "s_mov_b64 exec, s[2:3]\nv_mov_b32_e32 v7, v3\ns_waitcnt vmcnt(0)\n")
    assert claim_sites(good) == (1, [])
    n, bad = claim_sites(late)
    assert n == 1 and len(bad) == 1


def test_forward_claims_wait_inside_their_asm(tmp_path):
    try:
        B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    found, bad = claim_sites(_device_asm(tmp_path, "fwd.hip"))
    # one claim site per instantiation at least (bf16 and MXFP8, every mode)
    assert found >= 15, found
    assert not bad, bad[:3]
