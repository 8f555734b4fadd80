"""Checks of the generated gfx950 assembly (CPU only; needs hipcc).

The scan kernel's correctness depends on every LDS access staying on its side
of the workgroup barriers.  A compiler that moves a whole phase of LDS reads
past a barrier leaves two barriers with nothing between them; this test
rejects such a build.  It also checks that no kernel spills to scratch memory
or calls an outlined function.
"""
import re
import shutil

import pytest

from sequence_scan_amd import build as lib_build

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not available")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    out = tmp_path_factory.mktemp("asm") / "kernels.s"
    lib_build.asm(str(out))
    return out.read_text()


def kernels(asm_text):
    for m in re.finditer(r"^(_Z\S+):\s*;", asm_text, re.M):
        end = asm_text.find(".Lfunc_end", m.end())
        yield m.group(1), asm_text[m.end():end]


def test_no_collapsed_barriers(asm):
    bad = []
    for name, body in kernels(asm):
        ins = [ln.split()[0] for ln in body.splitlines() if re.match(r"^\s+[a-z_]+", ln)]
        last = None
        for i, op in enumerate(ins):
            if op == "s_barrier":
                if last is not None and not any(x.startswith(("ds_", "v_", "global_")) for x in ins[last + 1:i]):
                    bad.append(name)
                last = i
    assert not bad, f"barriers with no work between them in: {sorted(set(bad))}"


def test_every_scan_kernel_synchronises(asm):
    names = [n for n, _ in kernels(asm) if "scan_chunk_kernel" in n]
    assert len(names) >= 40
    for name, body in kernels(asm):
        # 16 states per wave means one wave per workgroup: no barrier is needed
        if "scan_chunk_kernel" in name and "Li16E" not in name:
            assert body.count("s_barrier") >= 4, name


def test_no_scratch_spills(asm):
    for m in re.finditer(r"\.amdhsa_kernel (\S+)(.*?)\.end_amdhsa_kernel", asm, re.S):
        priv = re.search(r"\.amdhsa_private_segment_fixed_size (\d+)", m.group(2))
        assert priv and int(priv.group(1)) == 0, f"{m.group(1)} uses scratch"


def test_no_outlined_calls(asm):
    # every helper of a kernel body is inlined: a call would move live state
    # through the calling convention's stack.  A kernel larger than a branch's
    # reach (+-128 KiB) jumps by s_getpc / s_add / s_setpc to a label of its
    # own: that is a branch, not a call.
    for name, body in kernels(asm):
        assert "s_swappc" not in body and "s_call" not in body, f"{name} makes a call"
        lines = body.split("\n")
        for i, ln in enumerate(lines):
            if "s_setpc" in ln:
                window = "\n".join(lines[max(0, i - 5):i])
                assert "s_getpc_b64" in window and re.search(r"s_add_u32 s\d+, s\d+, \(\.LBB", window), \
                    f"{name}: s_setpc that is not a long branch"


def test_kernel_hash_ignores_comments_only():
    """The profile records are keyed to the kernels' code: a comment or layout
    edit keeps the hash, any change of code or of a string literal moves it."""
    tok = lib_build._code_tokens
    base = 'float f(float x) { return x * 2.0f; }  // twice\nconst char* s = "a // b";\n'
    assert tok(base) == tok('/* doc */ float f(float x)\n{ return x * 2.0f; }\nconst char* s = "a // b";')
    assert tok(base) != tok(base.replace("2.0f", "3.0f"))
    assert tok(base) != tok(base.replace('"a // b"', '"a // c"'))
    assert tok("char c = '\"'; int y; // z") == tok("char c = '\"';  int y;")
