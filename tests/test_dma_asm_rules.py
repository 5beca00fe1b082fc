"""The tile transfers are issued from inline assembly (buffer_load_dwordx4
... lds and global_load_lds_dwordx4, tile_common.h), which the compiler's
hazard recognizer does not look into. This test builds the gfx950 assembly
of every kernel source that issues them and checks, on the compiler's
output, the two hazards that concern these instructions:

* a VALU instruction that writes an SGPR (v_readfirstlane / v_readlane,
  v_cmp, a carry-out) must be at least 5 wait states before a vector memory
  instruction that reads that SGPR (here: the buffer resource);
* M0 (the LDS destination) must be written by a scalar instruction at least
  one wait state before the transfer, and no other instruction of the
  compiler's may read M0 (M0 is the asm's input operand, so the compiler
  owns it; a stray reader would see a transfer's address).

Host only (hipcc cross-compiles for gfx950); no GPU is used."""
import concurrent.futures
import os
import re
import subprocess

import pytest

from softmax_sink_amd import build as B

SOURCES = ["fwd_bf16.hip", "bwd_bf16.hip"]
DMA = re.compile(r"^(buffer_load_dword\w*\s.*\blds\b|global_load_lds_\w+)")


def _assembly(src, tmp):
    out = os.path.join(tmp, src + ".s")
    # the library's own flags for this source, so that the schedule checked
    # is the one that ships
    cmd = [B.hipcc()] + B.flags() + B.SOURCE_FLAGS.get(src, []) + [
        "--cuda-device-only", "-S", "-o", out, os.path.join(B.CSRC, src)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read().split("\n")


def _sgprs(text):
    regs = set()
    for m in re.finditer(r"\bs\[(\d+):(\d+)\]", text):
        regs |= set(range(int(m.group(1)), int(m.group(2)) + 1))
    for m in re.finditer(r"\bs(\d+)\b", text):
        regs.add(int(m.group(1)))
    return regs


def _valu_sgpr_defs(ins):
    op, _, rest = ins.partition(" ")
    ops = [o.strip() for o in rest.split(",")]
    if op.startswith(("v_readfirstlane", "v_readlane")) or (
            op.startswith("v_cmp") and not op.startswith("v_cmpx")):
        return _sgprs(ops[0]) if ops else set()
    if re.match(r"v_(add|sub|subrev|addc|subb|subbrev)_co_|v_mad_(u|i)64|v_div_scale", op):
        return _sgprs(ops[1]) if len(ops) > 1 else set()
    return set()


def _check(lines):
    """-> (number of transfers, list of violations)."""
    ins = []          # (text, is_label)
    for l in lines:
        s = l.split(";")[0].strip()            # drop trailing comments
        if not s or s.startswith("."):
            continue
        ins.append((s, s.endswith(":")))
    bad, n = [], 0
    for k, (s, lab) in enumerate(ins):
        if lab:
            continue
        if DMA.match(s):
            n += 1
            regs = _sgprs(s.partition(" ")[2])
            ws, j, m0_ws = 0, k - 1, None
            while j >= 0 and ws < 5:
                t, tl = ins[j]
                if tl:
                    bad.append(f"block boundary within 5 wait states before: {s}")
                    break
                m = re.match(r"s_nop\s+(\w+)", t)
                if m:
                    ws += int(m.group(1), 0) + 1
                    j -= 1
                    continue
                if t.startswith("v_") and _valu_sgpr_defs(t) & regs:
                    bad.append(f"VALU SGPR write '{t}' {ws} wait states before '{s}'")
                if m0_ws is None and re.match(r"s_\w+\s+m0\b", t):
                    m0_ws = ws
                ws += 1
                j -= 1
            if m0_ws is not None and m0_ws < 1:
                bad.append(f"M0 written right before '{s}'")
        elif re.search(r"\bm0\b", s) and not re.match(r"s_\w+\s+m0\b", s) \
                and not s.startswith("s_nop"):
            bad.append(f"M0 read by '{s}'")
    return n, bad


def _have_hipcc():
    try:
        return bool(B.hipcc())
    except RuntimeError:
        return False


@pytest.mark.skipif(not _have_hipcc(), reason="hipcc not available")
def test_tile_transfers_respect_sgpr_and_m0_hazards(tmp_path):
    with concurrent.futures.ThreadPoolExecutor(len(SOURCES)) as ex:
        asm = list(ex.map(lambda s: _assembly(s, str(tmp_path)), SOURCES))
    total = 0
    for src, lines in zip(SOURCES, asm):
        n, bad = _check(lines)
        total += n
        assert not bad, f"{src}: " + "; ".join(bad[:5])
    assert total > 100          # the transfers were found


def test_checker_flags_planted_hazards():
    """The checker itself: a VALU-written resource SGPR right before a
    transfer, M0 set right before it, and a stray M0 reader are reported; a
    clean sequence is not."""
    clean = ["s_mov_b32 s23, 0x20000", "s_mov_b32 m0, s4", "v_add_u32_e32 v2, v3, v4",
             "s_nop 0", "buffer_load_dwordx4 v2, s[20:23], 0 offen lds"]
    assert _check(clean) == (1, [])
    n, bad = _check(["v_readfirstlane_b32 s21, v5", "s_mov_b32 m0, s4", "s_nop 0",
                     "buffer_load_dwordx4 v2, s[20:23], 0 offen lds"])
    assert n == 1 and any("VALU SGPR write" in b for b in bad)
    n, bad = _check(["v_add_u32_e32 v2, v3, v4", "s_mov_b32 m0, s4",
                     "global_load_lds_dwordx4 v[2:3], off"])
    assert any("M0 written right before" in b for b in bad)
    n, bad = _check(["v_add_u32_e32 v1, v2, v3 ; m0 in a comment is ignored",
                     "v_readlane_b32 s0, v1, m0"])
    assert bad == ["M0 read by 'v_readlane_b32 s0, v1, m0'"]
