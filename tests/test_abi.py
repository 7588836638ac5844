"""The C ABI library loads and exports every symbol include/vc.h declares (no GPU needed)."""
import os
import re
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vc.h")
LIB = os.path.join(ROOT, "lossless_speculative_decoding_amd", "libvc.so")


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(vc_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_four_calls():
    names = declared()
    for n in ("vc_compress", "vc_draft_step", "vc_verify", "vc_accept"):
        assert n in names


def test_library_exports_every_declared_symbol():
    assert os.path.exists(LIB), "libvc.so not built (run __graft_entry__.build())"
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if l.strip()}
    missing = [n for n in declared() if n not in exported]
    assert not missing, missing


def test_binding_loads_and_covers_every_symbol():
    import lossless_speculative_decoding_amd._vc as vc
    assert vc.raw("vc_abi_version")() == 2
    assert sorted(vc.exported_symbols()) == declared()
