"""The attention kernels' gfx950 assembly, as the library build compiles it:
no VALU instruction may read the result of an MFMA before the matrix core's
result latency has passed. gfx950 does not interlock that dependency; the
compiler pads it with wait states, and once left a read unpadded where it was
reached through a branch taken right after the MFMA (the decode kernel's
mask of a last, partial key tile), so that the read saw the previous tile's
scores in some lanes, depending on timing. The scan below follows every branch
taken within a few instructions of an MFMA and counts wait states up to the
first VALU read of the MFMA's destination in the target block.

Wait states needed: a result of an N-pass XDL MFMA is readable by the VALU
N + 3 issue slots after the MFMA (8 passes for the 16x16 bf16 shapes used
here, 16 for 32x32x16)."""

import os
import re
import shutil
import subprocess

import pytest

from gqa_attention_rope_02_amd import build as B

PASSES = {"16x16x32": 8, "16x16x16": 8, "32x32x16": 16, "32x32x8": 16}
LOADS = ("ds_read", "buffer_load", "global_load", "scratch_load", "flat_load")


def _regs(tok):
    m = re.match(r"[va]\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"[va](\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _passes(mfma_line):
    for shape, n in PASSES.items():
        if shape in mfma_line:
            return n
    return 16


def unpadded_reads_across_branches(asm: str):
    """(function, mfma, branch, reading instruction, wait states) for every
    VALU read of an MFMA destination reached through a branch taken within
    four instructions of the MFMA with fewer wait states than it needs."""
    found = []
    functions = set(re.findall(r"\.type\s+(_Z[^,\s]+),@function", asm))
    for name in re.findall(r"^(_Z[^:\s]+):", asm, re.M):
        if functions and name not in functions:   # data objects (the decode scratch) have no code
            continue
        i = asm.index(name + ":")
        j = asm.index(".Lfunc_end", i)
        lines = []
        for raw in asm[i:j].split("\n"):
            raw = raw.strip()
            m = re.match(r"^(\.LBB\w+):", raw)
            if m:
                lines.append(m.group(1) + ":")
            elif raw and not raw.startswith((";", ".")):
                lines.append(raw.split(";")[0].strip())
        labels = {l[:-1]: k for k, l in enumerate(lines) if l.startswith(".LBB") and l.endswith(":")}
        for k, l in enumerate(lines):
            if not l.startswith("v_mfma"):
                continue
            need = _passes(l) + 3
            dst = _regs(l.split(None, 1)[1].split(",")[0].strip())
            for b in range(k + 1, min(k + 5, len(lines))):
                br = lines[b]
                if not br.startswith(("s_cbranch", "s_branch")):
                    continue
                target = br.split()[1]
                if target not in labels:
                    continue
                ws = b - k
                for t in range(labels[target] + 1, min(labels[target] + 64, len(lines))):
                    lt = lines[t]
                    if lt.endswith(":"):
                        continue
                    if lt.startswith("s_nop"):
                        ws += int(lt.split()[1]) + 1
                    else:
                        parts = lt.split(None, 1)
                        if len(parts) > 1 and parts[0].startswith("v_"):
                            ops = [x.strip() for x in parts[1].split(",")]
                            srcs = set().union(*[_regs(x) for x in ops[1:]]) if len(ops) > 1 else set()
                            if srcs & dst:
                                if ws < need:
                                    found.append((name, l, br, lt, ws))
                                break
                            if _regs(ops[0]) & dst:
                                break
                        elif len(parts) > 1 and parts[0].startswith(LOADS) and " lds" not in parts[1]:
                            # a load into the registers: later reads see the
                            # load's data, not the MFMA result (the MFMA/load
                            # write-after-write order is the compiler's own
                            # hazard padding)
                            if _regs(parts[1].split(",")[0].strip()) & dst:
                                break
                        ws += 1
                    if ws >= need:
                        break
    return found


def _assembly(src: str) -> str:
    out = os.path.join(B.BUILD, os.path.splitext(src)[0] + ".gfx950.s")
    os.makedirs(B.BUILD, exist_ok=True)
    cmd = [B.hipcc(), *B._flags(), *B.EXTRA.get(src, []), "--cuda-device-only", "-S",
           os.path.join(B.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read()


needs_hipcc = pytest.mark.skipif(not shutil.which(B.hipcc()) and not os.path.exists(B.hipcc()),
                                 reason="hipcc not available")


def test_scanner_stops_at_a_load_into_the_registers():
    """A load that overwrites the MFMA's destination before the read means the
    read sees the loaded data: not a result-latency hazard."""
    listing = "\n".join([
        "_Zfake:",
        "\tv_mfma_f32_32x32x16_bf16 v[32:47], v[88:91], v[84:87], v[32:47]",
        "\ts_cbranch_execz .LBB0_2",
        "\ts_nop 0",
        ".LBB0_2:",
        "\tds_read_b64_tr_b16 v[32:33], v119 offset:10240",
        "\ts_waitcnt lgkmcnt(0)",
        "\tv_max_f32_e32 v42, v32, v32",
        ".Lfunc_end0:",
    ])
    assert unpadded_reads_across_branches(listing) == []
    # without the load the same read is flagged
    assert len(unpadded_reads_across_branches(listing.replace(
        "\tds_read_b64_tr_b16 v[32:33], v119 offset:10240\n", ""))) == 1


def test_scanner_finds_the_hazard_it_is_for():
    """A hand-made listing with an MFMA, a branch right after it and an
    unpadded read of its result in the target block is flagged; padding the
    target with enough s_nop clears it."""
    listing = "\n".join([
        "_Zfake:",
        "\tv_mfma_f32_16x16x32_bf16 v[32:35], v[88:91], v[84:87], v[32:35]",
        "\ts_cbranch_scc1 .LBB0_2",
        "\tv_cndmask_b32_e32 v35, v66, v35, vcc",
        ".LBB0_2:",
        "\tv_max_f32_e32 v42, v35, v35",
        ".Lfunc_end0:",
    ])
    hits = unpadded_reads_across_branches(listing)
    assert len(hits) == 1 and hits[0][4] == 1
    padded = listing.replace(".LBB0_2:\n", ".LBB0_2:\n\ts_nop 7\n\ts_nop 3\n")
    assert unpadded_reads_across_branches(padded) == []


@needs_hipcc
@pytest.mark.parametrize("src", ["gqa_decode.hip", "gqa_prefill.hip"])
def test_no_unpadded_mfma_result_reads_across_branches(src):
    hits = unpadded_reads_across_branches(_assembly(src))
    assert not hits, "\n".join(f"{n[:60]}: {ws} wait states: {m} ... {b} -> {r}" for n, m, b, r, ws in hits[:8])
