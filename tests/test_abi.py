"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments before touching the GPU (CPU only: no compute call is made)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lrscan.h")


def _lib():
    import linear_recurrence_sequence_diag_amd as lr
    if not os.path.exists(lr.LIB_PATH):
        from linear_recurrence_sequence_diag_amd import build
        build.build()
    return lr


def declared_symbols():
    text = open(HEADER).read()
    return re.findall(r"LRSCAN_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


def test_header_declares_the_boundary():
    names = set(declared_symbols())
    for n in ("scan_fwd", "scan_bwd", "scan_fwd_ex", "scan_bwd_ex", "scan_step", "scan_complex_fwd",
              "scan_complex_bwd", "scan_complex_workspace_bytes", "scan_workspace_bytes",
              "scan_samu_fwd", "scan_samu_bwd", "scan_samu_workspace_bytes",
              "scan_status_string", "scan_chunk_summary", "scan_chunk_prefix", "scan_chunk_replay",
              "scan_reverse_chunk_summary", "scan_reverse_chunk_prefix",
              "scan_reverse_chunk_replay"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lr = _lib()
    lib = ctypes.CDLL(lr.LIB_PATH)
    for n in declared_symbols():
        assert hasattr(lib, n), f"{n} declared in lrscan.h but not exported"
    # nothing else with C linkage leaks out besides the declared entry points
    out = os.popen(f"nm -D --defined-only {lr.LIB_PATH}").read()
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    c_names = {n for n in exported if not n.startswith("_Z") and not n.startswith("_")}
    assert c_names <= set(declared_symbols()) | {"_init", "_fini"}, c_names - set(declared_symbols())


def test_binding_names_match_the_abi():
    lr = _lib()
    for n in declared_symbols():
        assert callable(getattr(lr, n)), f"binding lacks {n}"


def test_status_strings():
    lr = _lib()
    for code in range(-9, 1):
        s = lr.status_string(code)
        assert isinstance(s, str) and s and s != "unknown status"
    assert lr.status_string(-99) == "unknown status"


def test_argument_errors_return_status_without_work():
    lr = _lib()
    lib = lr.library()
    fake = 0x10000  # never dereferenced: validation fails first
    assert lib.scan_fwd(None, fake, fake, None, 2, 8, 4, lr.F32, None) == -1
    assert lib.scan_fwd(fake, fake, fake, None, 0, 8, 4, lr.F32, None) == -2
    # empty inputs in any dimension are argument errors
    assert lib.scan_fwd(fake, fake, fake, None, 2, 0, 4, lr.F32, None) == -2
    assert lib.scan_fwd(fake, fake, fake, None, 2, 8, 0, lr.BF16, None) == -2
    assert lib.scan_bwd(fake, fake, fake, None, fake, fake, 2, 0, 4, lr.F32, None) == -2
    assert lib.scan_bwd(fake, fake, fake, None, fake, fake, 0, 8, 4, lr.BF16, None) == -2
    assert lib.scan_fwd(fake, fake, fake, None, 2, -1, 4, lr.F32, None) == -2
    assert lib.scan_fwd(fake, fake, fake, None, 2, 8, 4, 7, None) == -3
    assert lib.scan_bwd(fake, fake, None, None, fake, fake, 2, 8, 4, lr.F32, None) == -1
    assert lib.scan_bwd(fake, fake, fake, None, fake, fake, 1 << 30, 1 << 30, 1 << 30, lr.F32,
                        None) == -2
    o = lr.make_opts(algo="chunked", chunk=24)
    assert lib.scan_fwd_ex(fake, fake, fake, None, 2, 8, 4, lr.F32, None, ctypes.byref(o)) == -4
    o = lr.make_opts(algo="fused", chunk=100)
    assert lib.scan_bwd_ex(fake, fake, fake, None, fake, fake, 2, 8, 4, lr.BF16, None,
                           ctypes.byref(o)) == -4
    # 512-byte rows x 128 need 16-byte aligned rows (D=3 is not)
    o = lr.make_opts(algo="fused", chunk=128, width=32)
    assert lib.scan_fwd_ex(fake, fake, fake, None, 2, 8, 3, lr.BF16, None, ctypes.byref(o)) == -4
    o = lr.make_opts(algo=9)
    assert lib.scan_fwd_ex(fake, fake, fake, None, 2, 8, 4, lr.F32, None, ctypes.byref(o)) == -7
    o = lr.make_opts(algo="chunked", chunk=64)
    o.workspace = fake
    o.workspace_bytes = 16
    assert lib.scan_fwd_ex(fake, fake, fake, None, 2, 8, 4, lr.F32, None, ctypes.byref(o)) == -5
    assert lib.scan_chunk_summary(fake, fake, fake, fake, 2, 8, 4, 17, lr.F32, None) == -4
    assert lib.scan_chunk_prefix(fake, None, None, fake, None, 2, 3, 4, None) == -1
    assert lib.scan_reverse_chunk_replay(fake, fake, fake, fake, None, fake, fake, 2, 8, 0, 64,
                                         lr.F32, None) == -2
    with pytest.raises(lr.LRScanError):
        lr.scan_fwd(None, fake, fake, None, 2, 8, 4, lr.F32, None)
    # complex: pairs whole or NULL whole; no chunked form; one fused tile shape
    assert lib.scan_complex_fwd(fake, fake, fake, fake, fake, None, None, None, None, None, 2, 8,
                                4, lr.F32, None, None) == -1
    assert lib.scan_complex_fwd(fake, fake, fake, fake, None, None, None, None, None, None, 2, 8,
                                4, lr.F32, None, None) == -1
    assert lib.scan_complex_fwd(fake, fake, fake, fake, fake, fake, None, None, None, None, 2, 0,
                                4, lr.F32, None, None) == -2
    o = lr.make_opts(algo="chunked")
    assert lib.scan_complex_fwd(fake, fake, fake, fake, fake, fake, None, None, None, None, 2, 8,
                                4, lr.F32, None, ctypes.byref(o)) == -7
    o = lr.make_opts(algo="fused", chunk=256)
    assert lib.scan_complex_bwd(*([fake] * 6), None, None, None, None, *([fake] * 4), None, None,
                                2, 8, 4, lr.BF16, None, ctypes.byref(o)) == -4
    assert lib.scan_complex_bwd(*([fake] * 6), fake, None, None, None, *([fake] * 4), None, None,
                                2, 8, 4, lr.BF16, None, None) == -1
    assert lr.scan_complex_workspace_bytes(2, 1000, 64, lr.F32) > 0
    assert lr.scan_complex_workspace_bytes(2, 1000, 64, lr.F32, lr.make_opts(algo="seq")) == 0
    # AUTO: short complex sequences walk per lane in both directions (no
    # scratch); a bf16 64-step sequence over 1.3M lanes walks forward only
    assert lr.scan_complex_workspace_bytes(4096, 8, 64, lr.F32) == 0
    assert lr.scan_complex_workspace_bytes(512, 32, 2560, lr.BF16) == 0
    assert lr.scan_complex_workspace_bytes(512, 64, 2560, lr.BF16) > 0
    # fused-transition scan: controls required, pairs whole, AUTO/FUSED only
    assert lib.scan_samu_fwd(None, *([fake] * 7), None, None, None, None, 2, 8, 4, lr.F32, None,
                             None) == -1
    assert lib.scan_samu_fwd(*([fake] * 7), None, None, None, None, None, 2, 8, 4, lr.F32, None,
                             None) == -1
    assert lib.scan_samu_fwd(*([fake] * 8), None, None, None, None, 2, 8, 0, lr.F32, None,
                             None) == -2
    assert lib.scan_samu_fwd(*([fake] * 8), None, None, None, None, 2, 8, 4, 3, None, None) == -3
    # no three-launch form for the fused-transition scan (rejected before any work)
    o = lr.make_opts(algo="chunked")
    assert lib.scan_samu_fwd(*([fake] * 8), None, None, None, None, 2, 8, 4, lr.F32, None,
                             ctypes.byref(o)) == -7
    o = lr.make_opts(algo="fused", chunk=64)
    assert lib.scan_samu_bwd(*([fake] * 8), None, None, None, None, None, None, None, None,
                             fake, fake, None, None, 2, 8, 4, lr.BF16, None,
                             ctypes.byref(o)) == -4
    assert lib.scan_samu_bwd(*([fake] * 8), fake, None, None, None, None, None, None, None,
                             fake, fake, None, None, 2, 8, 4, lr.BF16, None, None) == -1
    assert lib.scan_samu_bwd(*([fake] * 8), None, None, None, None, None, None, None, None,
                             None, fake, None, None, 2, 8, 4, lr.BF16, None, None) == -1
    assert lr.scan_samu_workspace_bytes(2, 1000, 64, lr.F32) > lr.scan_complex_workspace_bytes(
        2, 1000, 64, lr.F32)
    # the walk uses the same buffer as the tiles (tables and partial sums)
    assert lr.scan_samu_workspace_bytes(2, 1000, 64, lr.F32, lr.make_opts(algo="seq")) == \
        lr.scan_samu_workspace_bytes(2, 1000, 64, lr.F32)
    o = lr.make_opts()
    o.workspace = fake
    o.workspace_bytes = 16
    assert lib.scan_samu_fwd(*([fake] * 8), None, None, None, None, 2, 8, 4, lr.F32, None,
                             ctypes.byref(o)) == -5
    # a forward needs out or last; a step needs out or the new state
    assert lib.scan_fwd(fake, fake, None, None, 2, 8, 4, lr.F32, None) == -1
    assert lib.scan_step(None, fake, None, None, fake, fake, 2, 4, lr.F32, None) == -1
    assert lib.scan_step(fake, fake, fake, None, None, None, 2, 4, lr.F32, None) == -1
    assert lib.scan_step(fake, fake, None, None, fake, None, 0, 4, lr.F32, None) == -2
    assert lib.scan_step(fake, fake, None, None, fake, None, 2, 4, 5, None) == -3


def test_workspace_sizes_and_auto_choice():
    lr = _lib()
    for dt in (lr.F32, lr.BF16):
        for direction in (0, 1):
            # rows too long for the fused form's 32-bit in-tile offsets: the chunked form
            algo, chunk, _ = lr.scan_auto_algo(1, 32, 1 << 25, dt, direction)
            assert algo == lr.ALGO_CHUNKED and chunk > 0
            # a fused grid of 2^32 work-items or more (2^24 tiles of 256 threads;
            # 64 lanes are one 128-byte lane block in bf16, two in fp32): the
            # chunked form, not a launch that would fail
            edge = (1 << 16) if dt == lr.BF16 else (1 << 15)
            algo, chunk, _ = lr.scan_auto_algo(edge, 1 << 16, 64, dt, direction)
            assert algo == lr.ALGO_CHUNKED and chunk > 0
            algo, _, _ = lr.scan_auto_algo(edge - 1, 1 << 16, 64, dt, direction)
            assert algo == lr.ALGO_FUSED
            # short sequences over millions of lanes: the per-lane walk
            algo, chunk, _ = lr.scan_auto_algo(1, 1, (1 << 22) + 5, dt, direction)
            assert algo == lr.ALGO_SEQ
            algo, _, _ = lr.scan_auto_algo(16384, 8, 64, dt, direction)
            assert algo == lr.ALGO_SEQ
            algo, _, _ = lr.scan_auto_algo(16384, 16, 64, dt, direction)
            assert algo == (lr.ALGO_SEQ if dt == lr.BF16 else lr.ALGO_FUSED)
            # sequences of a million steps or more over one or two 128-byte
            # lane blocks in all: the three-launch form, with longer chunks
            # for longer sequences; shorter ones, and more blocks: fused
            one = 64 if dt == lr.BF16 else 32
            algo, chunk, _ = lr.scan_auto_algo(1, 1 << 20, one, dt, direction)
            assert algo == lr.ALGO_CHUNKED and chunk == (256 if direction == 0 else 128)
            algo, chunk, _ = lr.scan_auto_algo(1, 1 << 22, one, dt, direction)
            assert algo == lr.ALGO_CHUNKED and chunk == (1024 if direction == 0 else 512)
            algo, chunk, _ = lr.scan_auto_algo(1, 1 << 23, one, dt, direction)
            assert algo == lr.ALGO_CHUNKED and chunk == 1024
            algo, _, _ = lr.scan_auto_algo(1, (1 << 20) - 1, one, dt, direction)
            assert algo == lr.ALGO_FUSED
            algo, chunk, _ = lr.scan_auto_algo(1, 1 << 20, 2 * one, dt, direction)
            assert algo == (lr.ALGO_FUSED if direction == 0 else lr.ALGO_CHUNKED)
            algo, _, _ = lr.scan_auto_algo(1, 1 << 23, 4 * one, dt, direction)
            assert algo == lr.ALGO_FUSED
            # long sequences, and short ones over too few lanes for the walk: the
            # fused form, 256 rows of 128-byte lane blocks
            algo, tile, width = lr.scan_auto_algo(8, 2048, 2560, dt, direction)
            assert (algo, tile, width) == (lr.ALGO_FUSED, 256, 8)
            algo, _, _ = lr.scan_auto_algo(4, 16, 1024, dt, direction)
            assert algo == lr.ALGO_FUSED
            # rows that are not 16-byte aligned: the walk from 2^18 lanes up to
            # 32 steps (fp32: 128; bf16 rows shorter than 512 bytes: 64)
            algo, _, _ = lr.scan_auto_algo(4096, 32, 2559, dt, direction)
            assert algo == lr.ALGO_SEQ
            # bf16 from 33 steps: 512-byte rows x 64 (rows of at least 512 bytes)
            algo, tile, width = lr.scan_auto_algo(4096, 64, 2559, dt, direction)
            assert (algo, tile, width) == ((lr.ALGO_SEQ, 0, 0) if dt == lr.F32
                                           else (lr.ALGO_FUSED, 64, 32))
            algo, _, _ = lr.scan_auto_algo(4096, 64, 201, dt, direction)
            assert algo == lr.ALGO_SEQ
            algo, _, _ = lr.scan_auto_algo(4096, 64, 2560, dt, direction)
            assert algo == lr.ALGO_FUSED
            algo, _, _ = lr.scan_auto_algo(4096, 128, 2559, dt, direction)
            assert algo == (lr.ALGO_SEQ if dt == lr.F32 else lr.ALGO_FUSED)
            # unaligned rows over many 256-byte lane blocks: 256-byte rows x 128
            # (fp32: 512-byte rows x 64)
            algo, tile, width = lr.scan_auto_algo(8, 2048, 2559, dt, direction)
            assert (algo, tile, width) == ((lr.ALGO_FUSED, 64, 32) if dt == lr.F32
                                           else (lr.ALGO_FUSED, 128, 16))
            algo, tile, width = lr.scan_auto_algo(1, 131072, 1023, dt, direction)
            assert (algo, tile, width) == (lr.ALGO_FUSED, 256, 8)
            # a tile is no taller than a short sequence, and a forward chain of
            # at most 512 steps is one tile
            _, tile, _ = lr.scan_auto_algo(4096, 32, 2560, dt, direction)
            assert tile == 32
            if direction == 0:
                _, tile, _ = lr.scan_auto_algo(256, 300, 2560, dt, direction)
                assert tile == 512
    assert lr.scan_workspace_bytes(0, 8, 4, lr.F32) == 0
    o = lr.make_opts(algo="seq")
    assert lr.scan_workspace_bytes(2, 8, 4, lr.F32, o) == 0
    o = lr.make_opts(algo="chunked", chunk=64)
    n = lr.scan_workspace_bytes(4, 8192, 4096, lr.F32, o)
    assert n >= 3 * 4 * 128 * 4096 * 4
    for dt in (lr.F32, lr.BF16):
        for direction in (0, 1):
            algo, chunk, width = lr.scan_auto_algo(8, 2048, 2560, dt, direction)
            assert algo in (lr.ALGO_SEQ, lr.ALGO_CHUNKED, lr.ALGO_FUSED)
            o = lr.make_opts(algo=algo, chunk=chunk, width=width)
            assert lr.scan_workspace_bytes(8, 2048, 2560, dt, o) >= 0


def test_options_struct_layout_matches_the_header(tmp_path):
    """The binding's mirror of lrscan_opts has the C struct's size and field
    offsets (checked by compiling the header with the host C compiler)."""
    import shutil
    import subprocess
    lr = _lib()
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    names = [f[0] for f in lr.Opts._fields_]
    src = tmp_path / "layout.c"
    src.write_text("#include <stdio.h>\n#include <stddef.h>\n#include \"lrscan.h\"\n"
                   "int main(void) {\n  printf(\"%zu\\n\", sizeof(lrscan_opts));\n" +
                   "".join(f"  printf(\"%zu\\n\", offsetof(lrscan_opts, {n}));\n" for n in names) +
                   "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    vals = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True,
                                           check=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(lr.Opts)
    for n, off in zip(names, vals[1:]):
        assert getattr(lr.Opts, n).offset == off, n
