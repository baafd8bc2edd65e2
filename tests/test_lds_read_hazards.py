"""Static check of LDS-read completion in the library's gfx950 assembly (CPU).

The dhidden product of the fused lm_head issues its LDS fragment reads as inline
assembly (the transposing read's builtin would make the compiler drain every
direct global->LDS load in flight before each read), so the compiler does not
know their results arrive late.  Its explicit lgkmcnt waits name the
fragments, which keeps their readers below the waits; nothing in the source
stops the compiler from copying or reusing a destination register before the
data lands (an earlier version lost fragments that way on its tail step).
This test compiles the sources to device assembly with the library's own
flags and, for every kernel, follows each LDS read's destination registers
through the control-flow graph until an s_waitcnt lgkmcnt(n) with at least n
LDS operations issued after the read on every path (LDS operations of a
wavefront complete in order; scalar loads, which may complete out of order,
are not counted).  Any instruction that names a destination register before
then fails the test.  A planted copy shows the check catches the hazard.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_VREG = re.compile(r"\b([va])(\d+)\b|\b([va])\[(\d+):(\d+)\]")
_RETURNS = ("ds_read", "ds_bpermute", "ds_permute", "ds_swizzle")


def _regs(text):
    out = set()
    for m in _VREG.finditer(text):
        if m.group(1):
            out.add((m.group(1), int(m.group(2))))
        else:
            out.update((m.group(3), r) for r in range(int(m.group(4)), int(m.group(5)) + 1))
    return out


def _blocks(lines, start):
    blocks, order, cur = {}, [], None
    for i in range(start + 1, len(lines)):
        line = lines[i]
        if line.startswith(".Lfunc_end"):
            break
        m = re.match(r"^(\.LBB\w+):", line)
        if m:
            cur = m.group(1)
            blocks[cur] = []
            order.append(cur)
            continue
        ins = line.split(";")[0].strip()
        if not ins or ins.startswith("."):
            continue
        if cur is None:
            cur = "entry"
            blocks[cur] = []
            order.append(cur)
        blocks[cur].append((i + 1, ins))
    return blocks, order


def _successors(blocks, order, b):
    ins = blocks[b]
    last = ins[-1][1] if ins else ""
    op = last.split()[0] if last else ""
    out = [last.split()[1]] if op.startswith("s_cbranch") or op == "s_branch" else []
    if op not in ("s_branch", "s_endpgm", "s_setpc_b64"):
        k = order.index(b)
        if k + 1 < len(order):
            out.append(order[k + 1])
    return out


def lds_read_hazards(asm_text, symbol):
    """(line, instruction) pairs that name an LDS read's destination register
    while the read may still be in flight."""
    lines = asm_text.splitlines()
    start = next(i for i, l in enumerate(lines) if l.startswith(symbol + ":"))
    blocks, order = _blocks(lines, start)
    entry = {b: None for b in order}
    entry[order[0]] = {}
    found = set()
    work = [order[0]]
    while work:
        b = work.pop(0)
        # pending reads: issue line -> [fewest LDS operations issued after it, destinations]
        pend = {k: list(v) for k, v in entry[b].items()}
        for ln, ins in blocks[b]:
            op = ins.split()[0]
            if op == "s_waitcnt":
                m = re.search(r"lgkmcnt\((\d+)\)", ins)
                if m:
                    n = int(m.group(1))
                    pend = {k: v for k, v in pend.items() if v[0] < n}
                continue
            used = _regs(ins[len(op):])
            for k, (_, dst) in pend.items():
                if used & dst:
                    found.add((ln, ins))
            if op.startswith("ds_"):
                for v in pend.values():
                    v[0] = min(64, v[0] + 1)
                dst = _regs(ins[len(op):].split(",")[0]) if op.startswith(_RETURNS) else set()
                pend[ln] = [0, dst]
        for nb in _successors(blocks, order, b):
            old = entry[nb]
            new = {k: list(v) for k, v in (old or {}).items()}
            for k, v in pend.items():
                new[k] = [min(new[k][0], v[0]), v[1]] if k in new else list(v)
            if old is None or any(k not in old or old[k][0] != new[k][0] for k in new):
                entry[nb] = new
                if nb not in work:
                    work.append(nb)
    return sorted(found)


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    if shutil.which("hipcc") is None:
        pytest.skip("hipcc is not installed")
    from rl_post_loss_dr_amd.build import HIPCC_FLAGS, SOURCES

    flags = [f for f in HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    out = {}
    d = tmp_path_factory.mktemp("asm")
    for src in SOURCES:
        s = os.path.join(d, os.path.basename(src) + ".s")
        r = subprocess.run(["hipcc", *flags, "--cuda-device-only", "-S", "-I",
                            os.path.join(ROOT, "include"), "-o", s, src],
                           capture_output=True, text=True, timeout=600)
        assert r.returncode == 0, r.stderr[-3000:]
        out[os.path.basename(src)] = open(s).read()
    return out


def _kernels(text):
    return re.findall(r"^(_Z\w+):", text, flags=re.M)


def test_every_kernel_waits_for_its_lds_reads(device_asm):
    checked = 0
    for src, text in device_asm.items():
        for sym in _kernels(text):
            hz = lds_read_hazards(text, sym)
            assert not hz, f"{src} {sym}: " + "; ".join(f"line {ln}: {i}" for ln, i in hz[:5])
            checked += 1
    assert checked >= 10


def test_dhidden_product_reads_are_inline_transposing_reads(device_asm):
    """The dhidden product (k_gemm<2>) is the one the check exists for: its
    main loop reads A through ds_read_b64_tr_b16 and has explicit waits."""
    text = device_asm["lmhead.hip"]
    sym = next(s for s in _kernels(text) if "k_gemmILi2E" in s)
    body = text[text.index(sym + ":"):]
    body = body[:body.index(".Lfunc_end")]
    assert body.count("ds_read_b64_tr_b16") >= 16
    assert "lgkmcnt(4)" in body and "lgkmcnt(11)" in body and "lgkmcnt(13)" in body


def test_check_catches_a_register_named_in_flight():
    """A copy of an in-flight destination (the earlier failure's shape), a
    wait that lands too few reads, and out-of-loop reuse are reported; the
    same code with a sufficient wait is clean."""
    def kernel(body):
        return "k:\n" + "".join(f"\t{l}\n" for l in body) + ".Lfunc_end0:\n"

    base = ["ds_read_b64_tr_b16 v[10:11], v2", "ds_read_b128 v[12:15], v3 offset:16"]
    ok = kernel(base + ["s_waitcnt lgkmcnt(0)", "v_mov_b32_e32 v20, v10", "s_endpgm"])
    assert lds_read_hazards(ok, "k") == []
    early = kernel(base + ["v_mov_b32_e32 v20, v11", "s_waitcnt lgkmcnt(0)", "s_endpgm"])
    assert [i for _, i in lds_read_hazards(early, "k")] == ["v_mov_b32_e32 v20, v11"]
    short = kernel(base + ["s_waitcnt lgkmcnt(1)", "v_mov_b32_e32 v20, v13", "s_endpgm"])
    assert len(lds_read_hazards(short, "k")) == 1
    # a read issued at the end of a loop body (the next iteration's operand)
    # lands behind the wait at the top of the body; on the exit path nothing
    # waits for the last one, so reusing its register there is reported
    loop = ("k:\n\tds_read_b128 v[8:11], v1\n.LBB0_1:\n\ts_waitcnt lgkmcnt(0)\n"
            "\tv_add_u32_e32 v20, v8, v20\n\tds_read_b128 v[8:11], v1 offset:64\n"
            "\ts_cbranch_vccnz .LBB0_1\n.LBB0_2:\n\tv_mov_b32_e32 v8, 0\n\ts_endpgm\n.Lfunc_end0:\n")
    assert [i for _, i in lds_read_hazards(loop, "k")] == ["v_mov_b32_e32 v8, 0"]
    fixed = loop.replace(".LBB0_2:\n", ".LBB0_2:\n\ts_waitcnt lgkmcnt(0)\n")
    assert lds_read_hazards(fixed, "k") == []
