"""Build check of the tiled GEMM's folded-row MFMAs (CPU; needs hipcc).

The accumulators of the rows folded into a 320-row tile live in ordinary
VGPRs and are updated by inline-asm v_mfma_f32_32x32x16_bf16, which the
compiler's hazard recognizer does not see.  Their safety rests on
(1) nothing but those asm MFMAs touching the accumulators during the k-loop,
(2) after the last one, an asm block of three `s_nop 7` (24 wait states)
coming before any other instruction reads or writes them, and (3) each asm
MFMA carrying an `s_nop 4` of its own, since the compiler may schedule it
right after the VALU code that writes its operands (the widened INT8 weight
fragment).  These tests compile gemm_bf16.hip for gfx950 to assembly and
check (2) and (3) in every kernel that holds such MFMAs, so a compiler or
schedule change that breaks them fails here rather than silently on the GPU."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "mixture_experts_layer_prefix_amd", "csrc", "gemm_bf16.hip")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")


def _regs(text):
    """VGPR numbers named in an operand string (v5, v[8:11])."""
    out = set()
    for a, b in re.findall(r"\bv\[(\d+):(\d+)\]", text):
        out.update(range(int(a), int(b) + 1))
    for a in re.findall(r"\bv(\d+)\b", text):
        out.add(int(a))
    return out


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("asm") / "gemm_bf16.s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"),
           "--offload-device-only", "-S", SRC, "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    return open(out).read()


def _blocks(lines):
    """Basic blocks of one function: (label, [(kind, text)], successor labels);
    kind is 'mfma' (folded-row asm MFMA), 'pad' (the three-s_nop asm block) or
    'insn' (any other instruction)."""
    blocks = []
    cur = {"label": "<entry>", "items": [], "succ": None}
    in_asm, block = False, []

    def close(nxt):
        if cur["succ"] is None:
            cur["succ"] = [nxt] if nxt else []
        blocks.append(dict(cur))

    for ln in lines[1:]:
        t = ln.split(";")[0].strip() if not ln.strip().startswith(";;#ASM") else ln.strip()
        if t.startswith(";;#ASMSTART"):
            in_asm, block = True, []
            continue
        if t.startswith(";;#ASMEND"):
            in_asm = False
            if len(block) == 3 and all(b == "s_nop 7" for b in block):
                cur["items"].append(("pad", ""))
            elif any(b.startswith("v_mfma_f32_32x32x16_bf16") for b in block):
                cur["items"] += [("mfma", b) for b in block]
            else:
                cur["items"] += [("insn", b) for b in block]
            continue
        if not t or t.startswith("."):
            if re.match(r"^\.LBB\w+:$", t):
                label = t[:-1]
                close(label)
                cur = {"label": label, "items": [], "succ": None}
            continue
        if in_asm:
            block.append(t)
            continue
        cur["items"].append(("insn", t))
        op = t.split()[0]
        if op == "s_branch":
            cur["succ"] = [t.split()[1]]
            close(None)
            cur = {"label": None, "items": [], "succ": None}
        elif op.startswith("s_cbranch"):
            target = t.split()[1]
            blocks.append({"label": cur["label"], "items": cur["items"], "succ": [target, "<next>"]})
            cur = {"label": None, "items": [], "succ": None}
        elif op in ("s_endpgm", "s_setpc_b64"):
            cur["succ"] = []
            close(None)
            cur = {"label": None, "items": [], "succ": None}
    close(None)
    # resolve fall-through edges
    for i, b in enumerate(blocks):
        nxt = blocks[i + 1]["label"] if i + 1 < len(blocks) else None
        if i + 1 < len(blocks) and blocks[i + 1]["label"] is None:
            blocks[i + 1]["label"] = f"<anon{i + 1}>"
            nxt = blocks[i + 1]["label"]
        b["succ"] = [nxt if x == "<next>" else x for x in b["succ"] if x]
        if b["succ"] == [] and b["items"] and b["items"][-1][1].split()[0] not in (
                "s_branch", "s_endpgm", "s_setpc_b64") and nxt:
            b["succ"] = [nxt]
    return blocks


def test_folded_row_mfmas_are_padded_before_any_other_access(asm):
    """Forward dataflow over each kernel's basic blocks: a folded-row MFMA
    makes its accumulator registers "in flight", the s_nop pad clears that,
    and no other instruction may name those registers while in flight."""
    funcs = re.split(r"\n(?=_Z\S*:)", asm)
    checked = 0
    for f in funcs:
        lines = f.split("\n")
        blocks = _blocks(lines)
        mfmas = [t for b in blocks for k, t in b["items"] if k == "mfma"]
        if not mfmas:
            continue
        checked += 1
        name = lines[0].split(":")[0][:100]
        acc = set()
        for t in mfmas:
            acc |= _regs(t.split(None, 1)[1].split(",")[0])
        by_label = {b["label"]: b for b in blocks}
        state_in = {b["label"]: False for b in blocks}
        work = [b["label"] for b in blocks]
        while work:
            lab = work.pop()
            b = by_label[lab]
            dirty = state_in[lab]
            for kind, t in b["items"]:
                if kind == "mfma":
                    dirty = True
                elif kind == "pad":
                    dirty = False
                elif dirty and " " in t and _regs(t.split(None, 1)[1]) & acc:
                    raise AssertionError(f"{name}: '{t}' (block {lab}) names the folded-row "
                                         f"accumulators while an asm MFMA may be in flight")
            for sl in b["succ"]:
                if sl in state_in and dirty and not state_in[sl]:
                    state_in[sl] = True
                    work.append(sl)
        assert any(k == "pad" for b in blocks for k, _ in b["items"]), f"{name}: no pad"
    assert checked > 0, "no kernel with folded-row MFMAs found"


def test_folded_row_mfmas_carry_their_source_pad(asm):
    """Every asm block holding a folded-row MFMA pads with s_nop 4 or more
    right before it: the compiler inserts no wait states for the statement,
    and a VALU write of its weight fragment was seen one instruction ahead."""
    blocks = re.findall(r";;#ASMSTART\n(.*?);;#ASMEND", asm, flags=re.S)
    mf = [b for b in blocks if "v_mfma_f32_32x32x16_bf16" in b]
    assert mf, "no folded-row asm MFMA found"
    for b in mf:
        ins = [ln.strip() for ln in b.strip().split("\n") if ln.strip()]
        i = next(k for k, t in enumerate(ins) if t.startswith("v_mfma"))
        assert i > 0 and re.match(r"s_nop (\d+)$", ins[i - 1]) and \
            int(ins[i - 1].split()[1]) >= 4, f"unpadded folded-row MFMA: {ins}"
