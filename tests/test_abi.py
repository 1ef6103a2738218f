"""The C-ABI library loads, exports what include/isd.h declares, and rejects
invalid arguments on the host (no GPU needed: these checks run before any
HIP call)."""

import ctypes
import os
import re

import pytest

import draft_verify_decoding_amd as dvd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "isd.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "defined")))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(dvd.LIB_PATH):
        pytest.fail("libisd.so is not built (run __graft_entry__.build())")
    return dvd.lib()


def test_header_declares_the_expected_calls():
    names = declared_functions()
    for n in ["isd_kv_write", "isd_attention", "isd_attention_workspace_size", "isd_accept",
              "isd_accept_workspace_size", "isd_block_assemble", "isd_linear", "gated_lora_apply", "isd_linear_gated",
              "isd_lora_workspace_size", "isd_strerror", "isd_version"]:
        assert n in names, n


def test_every_declared_symbol_is_exported(lib):
    handle = ctypes.CDLL(dvd.LIB_PATH)
    for name in declared_functions():
        assert hasattr(handle, name), name


def test_noalloc_accept_rejects_a_null_argument_on_host(lib):
    assert lib.isd_accept_noalloc(None, None) == -1
    assert lib.isd_accept_noalloc_max_workspace() == 4 << 20


def test_strerror_and_version(lib):
    assert dvd.strerror(0) == "success"
    for code in (-1, -2, -3, -4, -5):
        assert dvd.strerror(code) != "unknown error code"
    assert lib.isd_version() >= 100


def test_attention_rejects_bad_arguments_on_host(lib):
    null_kv = lib.isd_attention(None, None, None, 1, 8, 4, 0.1, 64, 0, None, dvd.ISD_F32, None, 0, None, None)
    assert null_kv == -1
    kv = dvd.IsdKvCache(16, 16, 16, 4, 10, 16, 1, 96, dvd.ISD_BF16)  # head_dim 96 unsupported
    assert lib.isd_attention(ctypes.byref(kv), 16, 16, 1, 8, 4, 0.1, 64, 0, 16, dvd.ISD_F32, None, 0, None, None) == -2
    kv.head_dim = 128
    kv.page_size = 8
    assert lib.isd_attention(ctypes.byref(kv), 16, 16, 1, 8, 4, 0.1, 64, 0, 16, dvd.ISD_F32, None, 0, None, None) == -2
    kv.page_size = 16
    # Hq not a multiple of Hkv
    kv.num_kv_heads = 3
    assert lib.isd_attention(ctypes.byref(kv), 16, 16, 1, 8, 4, 0.1, 64, 0, 16, dvd.ISD_F32, None, 0, None, None) == -2
    kv.num_kv_heads = 1
    # group * rows > 128
    assert lib.isd_attention(ctypes.byref(kv), 16, 16, 1, 40, 4, 0.1, 64, 0, 16, dvd.ISD_F32, None, 0, None, None) == -2
    # scale must be positive, chunks of the invariant split <= 65536 tiles, max_len >= rows
    assert lib.isd_attention(ctypes.byref(kv), 16, 16, 1, 8, 4, -1.0, 64, 0, 16, dvd.ISD_F32, None, 0, None, None) == -1
    assert lib.isd_attention(ctypes.byref(kv), 16, 16, 1, 8, 4, 0.1, 64, -65537, 16, dvd.ISD_F32, None, 0, None, None) == -1
    assert lib.isd_attention(ctypes.byref(kv), 16, 16, 1, 8, 4, 0.1, 64, -3, 16, dvd.ISD_F32, None, 0, None, None) == -3
    assert lib.isd_attention(ctypes.byref(kv), 16, 16, 1, 8, 4, 0.1, 4, 0, 16, dvd.ISD_F32, None, 0, None, None) == -1
    # misaligned q
    assert lib.isd_attention(ctypes.byref(kv), 18, 16, 1, 8, 4, 0.1, 64, 0, 16, dvd.ISD_F32, None, 0, None, None) == -1
    # too many sequences for one call
    assert lib.isd_attention(ctypes.byref(kv), 16, 16, 9000, 8, 4, 0.1, 64, 0, 16, dvd.ISD_F32, None, 0, None, None) == -2
    # the workspace is required and sized by the same arguments
    need = lib.isd_attention_workspace_size(1, 8, 4, ctypes.byref(kv), 4096, 64)
    assert need > 0
    assert lib.isd_attention(ctypes.byref(kv), 16, 16, 1, 8, 4, 0.1, 4096, 64, 16, dvd.ISD_F32, None, 0, None, None) == -3
    assert lib.isd_attention(ctypes.byref(kv), 16, 16, 1, 8, 4, 0.1, 4096, 64, 16, dvd.ISD_F32, 1 << 20, need - 16,
                             None, None) == -3
    # an output type other than fp32 and bf16
    assert lib.isd_attention(ctypes.byref(kv), 16, 16, 1, 8, 4, 0.1, 64, 0, 16, 9, None, 0, None, None) == -2


def test_attention_invariant_split_workspace(lib):
    """Chunked split: one partial piece per (sequence, chunk, KV head, query
    block), C * ceil(ceil(max_len / 32) / t) chunks, whatever the slices."""
    kv = dvd.IsdKvCache(16, 16, 16, 4, 10, 16, 8, 128, dvd.ISD_BF16)
    C, rows, Hq, max_len = 64, 8, 32, 8200
    for t in (1, 16, 64, 300):
        chunks = C * -(-(-(-max_len // 32)) // t)
        pieces = chunks * 8 * 1 * 32  # 8 KV heads, one 32-column query block (4 x 8 rows)
        off = -(-(C + 1) * 4 // 256) * 256
        want = off + -(-pieces * 128 * 4 // 256) * 256 + -(-pieces * 2 * 4 // 256) * 256
        assert lib.isd_attention_workspace_size(C, rows, Hq, ctypes.byref(kv), max_len,
                                                dvd.attn_invariant(t)) == want
    assert lib.isd_attention_workspace_size(C, rows, Hq, ctypes.byref(kv), max_len, -70000) == 0
    # one workgroup per chunk: C * chunks * Hkv must fit the grid
    assert lib.isd_attention_workspace_size(8192, rows, Hq, ctypes.byref(kv), 1 << 20, -1) == 0
    assert lib.isd_attention_workspace_size(8192, rows, Hq, ctypes.byref(kv), 1 << 20, -2) > 0


def test_kv_write_rejects_bad_arguments_on_host(lib):
    kv = dvd.IsdKvCache(16, 16, 16, 4, 10, 16, 1, 128, dvd.ISD_BF16)
    assert lib.isd_kv_write(ctypes.byref(kv), 16, 16, 16, None, 0, 8, None, None) == 0  # nothing to write
    assert lib.isd_kv_write(ctypes.byref(kv), 16, 16, 16, None, 70000, 8, None, None) == -2  # C beyond the grid
    assert lib.isd_kv_write(ctypes.byref(kv), 18, 16, 16, None, 2, 8, None, None) == -1  # misaligned k
    assert lib.isd_kv_write(ctypes.byref(kv), 16, 16, None, None, 2, 8, None, None) == -1  # no positions


def test_accept_rejects_bad_arguments_on_host(lib):
    assert lib.isd_accept(None, None) == -1
    a = dvd.IsdAcceptArgs()
    a.C, a.N, a.V, a.rows, a.dtype = 2, 9, 100, 18, dvd.ISD_BF16
    assert lib.isd_accept(ctypes.byref(a), None) == -2  # N > 8
    a.N, a.rows = 4, 6
    assert lib.isd_accept(ctypes.byref(a), None) == -1  # rows < 2N - 1
    a.rows = 8
    assert lib.isd_accept(ctypes.byref(a), None) == -1  # null pointers
    fake = 1 << 20
    st_in = dvd.IsdSeqState(*(fake + 64 * i for i in range(6)))
    st_out = dvd.IsdSeqState(*(fake + 4096 + 64 * i for i in range(6)))
    a.logits, a.in_, a.out = fake, st_in, st_out
    a.accepted, a.n_emit, a.emit, a.kv_commit = fake, fake, fake, fake
    a.ld = 100
    assert lib.isd_accept(ctypes.byref(a), None) == -1  # 200-byte rows are not 16-byte aligned
    a.ld = 104
    assert lib.isd_accept(ctypes.byref(a), None) == -3  # no workspace
    a.out = st_in
    assert lib.isd_accept(ctypes.byref(a), None) == -1  # out aliases in
    a.out = st_out
    a.proposal = 7
    assert lib.isd_accept(ctypes.byref(a), None) == -1  # unknown proposal rule
    a.proposal = 0
    a.V, a.ld = 600000, 600000
    assert lib.isd_accept(ctypes.byref(a), None) == -2  # vocabulary beyond the cached chunk statistics
    assert lib.isd_accept_workspace_size(64, 4, 600000, 8) == 0
    assert lib.isd_accept_workspace_size(64, 4, 151936, 8) > 0
    assert lib.isd_accept_workspace_size(64, 1, 151936, 8) == 0


def test_linear_rejects_bad_arguments_on_host(lib):
    F32, BF16 = dvd.ISD_F32, dvd.ISD_BF16
    assert lib.isd_linear(16, 16, 4, 100, 8, 16, F32, None) == -2  # K not a multiple of 64
    assert lib.isd_linear(None, 16, 4, 64, 8, 16, F32, None) == -1
    assert lib.isd_linear(16, 16, 0, 64, 8, 16, F32, None) == 0  # empty problem
    assert lib.isd_linear(16, 16, 4, 64, 8, 16, 7, None) == -2  # output type
    assert lib.isd_linear(16, 16, 4, 64, 8, 18, F32, None) == -1  # fp32 output not 4-byte aligned
    assert lib.isd_linear(16, 16, 4, 64, 8, 17, BF16, None) == -1  # bf16 output not 2-byte aligned
    assert lib.gated_lora_apply(16, 16, 16, 16, 4, 64, 8, 24, 1.0, 16, F32, 16, 1 << 20, None) == -2  # rank 24
    assert lib.gated_lora_apply(16, 16, 16, 16, 4, 64, 8, 32, 1.0, 16, F32, 16, 8, None) == -3  # ws too small
    # a 256-byte counter pair, 8 split-K partials of U, then U
    assert lib.isd_lora_workspace_size(512, 32) == 256 + 512 * 32 * 4 * 9
    assert lib.gated_lora_apply(16, 16, 24, 16, 4, 64, 8, 32, 1.0, 16, F32, 16, 512, None) == -1  # B misaligned
    assert lib.isd_linear_gated(16, 16, 16, 16, 16, 4, 64, 8, 32, 1.0, 16, 0, 16, 1 << 20, None) == -2  # type


def test_block_assemble_rejects_bad_arguments_on_host(lib):
    st = dvd.IsdSeqState(16, 16, 16, 16, 16, 16)
    f = lib.isd_block_assemble
    assert f(None, 16, 16, 16, 4, 4, 7, 16, 16, 16, None, None) == -1          # no state
    assert f(ctypes.byref(st), 16, 16, 16, 0, 4, 7, 16, 16, 16, None, None) == 0  # nothing to do
    assert f(ctypes.byref(st), 16, 16, 16, 4, 1, 7, 16, 16, 16, None, None) == -1  # N < 2
    assert f(ctypes.byref(st), 16, 16, 16, 4, 9, 7, 16, 16, 16, None, None) == -2  # N > 8
    assert f(ctypes.byref(st), 16, 16, 16, 4, 4, 7, None, 16, 16, None, None) == -1  # no tokens
    assert f(ctypes.byref(st), None, 16, 16, 4, 4, 7, 16, 16, 16, None, None) == -1  # no emit
    assert f(ctypes.byref(st), 16, 16, None, 4, 4, 7, 16, 16, 16, None, None) == -1  # positions need ctx


def test_ctypes_structs_match_the_header_layout(tmp_path):
    """The binding's ctypes structs have the sizes and field offsets the C
    compiler gives the structs of include/isd.h."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no host C compiler")
    structs = {"isd_accept_args": dvd.IsdAcceptArgs, "isd_seq_state": dvd.IsdSeqState,
               "isd_kv_cache": dvd.IsdKvCache}
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "isd.h"', "int main(void) {"]
    for cname, py in structs.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for fname, _ in py._fields_:
            cf = "in" if fname == "in_" else fname
            lines.append(f'  printf("{cname} {fname} %zu\\n", offsetof({cname}, {cf}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    subprocess.run([gcc, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(root, "include"), "-I", "/opt/rocm/include",
                    str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    got = {tuple(l.split()[:2]): int(l.split()[2]) for l in out if l}
    for cname, py in structs.items():
        assert got[(cname, "size")] == ctypes.sizeof(py), cname
        for fname, _ in py._fields_:
            assert got[(cname, fname)] == getattr(py, fname).offset, (cname, fname)
