"""Rules on the kernel sources that the compiler cannot check for us.

The compiler inserts the wait states that an in-flight matrix-core
instruction needs before a later instruction overwrites its registers, but it
does not look inside inline asm: an asm instruction that writes a vector
register can be handed a register that an MFMA is still writing (this
happened to an asm v_bfi_b32 next to the Q4 products once the unused result
elements were dead).  So inline asm in the kernels is limited to waits and
to empty statements that only pin values or order memory."""

import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "quantized_moe_expert_gemv_amd", "csrc")
SOURCES = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".hpp")))

ASM = re.compile(r'\basm\s*(?:volatile\s*)?\(\s*"([^"]*)"')


def asm_templates():
    for f in SOURCES:
        text = open(os.path.join(CSRC, f)).read()
        for m in ASM.finditer(text):
            yield f, m.group(1)


def test_sources_are_found():
    assert {"decode.hip", "prefill.hip", "common.hpp"} <= set(SOURCES)


def test_inline_asm_is_only_waits_and_empty_statements():
    seen = 0
    for f, tpl in asm_templates():
        seen += 1
        ok = tpl == "" or re.fullmatch(r"s_waitcnt (?:vmcnt|lgkmcnt)\((?:\d+|%\d)\)", tpl)
        assert ok, f"{f}: inline asm {tpl!r} emits an instruction other than a wait"
    assert seen > 0


def test_no_hand_written_packed_fp32_arithmetic():
    for f in SOURCES:
        text = open(os.path.join(CSRC, f)).read()
        assert not re.search(r"v_pk_(?:add|mul|fma)_f32", text), f
