"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point include/sas.h declares, and rejects bad arguments before
launching anything (these calls return from the host-side checks)."""
import ctypes as C
import os
import re

import pytest

from gated_block_sparse_scores_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "sas.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sas_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = header_functions()
    assert "sas_select_topk" in names and "sas_decode" in names
    lib = C.CDLL(L.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.EXPORTED)


def test_stream_probe_is_built_beside_the_library():
    # bench.py --stream-floor runs it; it is a separate program, not in libsas.so
    probe = os.path.join(os.path.dirname(L.LIB_PATH), "stream_probe")
    assert os.path.isfile(probe) and os.access(probe, os.X_OK)
    lib = C.CDLL(L.LIB_PATH)
    assert not hasattr(lib, "read_kernel")


def test_version_and_status_strings():
    assert L.sas_version() >= 100
    assert L.status_string(L.SAS_OK) == "ok"
    assert "workspace" in L.status_string(L.SAS_ERR_WORKSPACE)


def shape(**kw):
    base = dict(batch=1, hq=4, hkv=2, seqlen=256, head_dim=128, block=64,
                dtype=L.SAS_DTYPE_BF16, scale=0.0)
    base.update(kw)
    return L.sas_shape(*base.values())


FAKE = 0x1000  # never dereferenced: every call below fails its host-side checks


def fwd(sh, K=4, **ptrs):
    p = dict(q=FAKE, k=FAKE, v=FAKE, idx=FAKE, logg=FAKE, o=FAKE, lse=FAKE)
    p.update(ptrs)
    return L.lib().sas_attn_fwd(C.byref(sh), K, p["q"], p["k"], p["v"], p["idx"], p["logg"],
                                p["o"], p["lse"], None, 0, None)


@pytest.mark.parametrize("kw,status", [
    (dict(hq=3, hkv=2), L.SAS_ERR_INVALID_ARG),
    (dict(batch=0), L.SAS_ERR_INVALID_ARG),
    (dict(seqlen=-1), L.SAS_ERR_INVALID_ARG),
    (dict(head_dim=96), L.SAS_ERR_UNSUPPORTED),
    (dict(block=48), L.SAS_ERR_UNSUPPORTED),
    (dict(dtype=7), L.SAS_ERR_INVALID_ARG),
    (dict(scale=-1.0), L.SAS_ERR_INVALID_ARG),
])
def test_fwd_rejects_bad_shapes(kw, status):
    assert fwd(shape(**kw), q=None) in (status, L.SAS_ERR_INVALID_ARG)
    assert fwd(shape(**kw)) == status


def test_fwd_rejects_null_and_misaligned_pointers_and_bad_K():
    sh = shape()
    for name in ("q", "k", "v", "idx", "o", "lse"):
        assert fwd(sh, **{name: None}) == L.SAS_ERR_INVALID_ARG
    assert fwd(sh, q=FAKE + 2) == L.SAS_ERR_INVALID_ARG
    assert fwd(sh, K=0) == L.SAS_ERR_INVALID_ARG
    assert fwd(sh, K=255) == L.SAS_ERR_UNSUPPORTED     # training calls take K <= 254


def test_bwd_workspace_query_and_checks():
    sh = shape(seqlen=8192, hq=32, hkv=8)
    n = L.lib().sas_attn_bwd_workspace_size(C.byref(sh), 31)
    # D (b*hq*N fp32), the split dK/dV partials (20 key blocks in two shares
    # each at 256 CUs: 40 x 8 KV heads x 64 KiB), the slot map and the dlogg
    # partials
    assert n >= 32 * 8192 * 4 + 40 * 8 * 65536
    assert n < 32 * 8192 * 4 + 40 * 8 * 65536 + (1 << 21)
    args = [FAKE] * 16
    # missing workspace
    st = L.lib().sas_attn_bwd(C.byref(sh), 31, *args[:13], None, None, None, 0, None)
    assert st == L.SAS_ERR_WORKSPACE
    # too small workspace
    st = L.lib().sas_attn_bwd(C.byref(sh), 31, *args[:13], None, None, FAKE, n - 1, None)
    assert st == L.SAS_ERR_WORKSPACE
    # ds without s
    a = list(args)
    a[8] = None  # s
    st = L.lib().sas_attn_bwd(C.byref(sh), 31, *a[:13], None, FAKE, FAKE, n, None)
    assert st == L.SAS_ERR_INVALID_ARG
    # ungated with selector outputs requested
    a = list(args)
    a[7] = None  # logg
    st = L.lib().sas_attn_bwd(C.byref(sh), 31, *a[:13], FAKE, FAKE, FAKE, n, None)
    assert st == L.SAS_ERR_INVALID_ARG


def test_select_checks():
    sh = shape()
    lib = L.lib()
    # no scores and no stand-in inputs
    assert lib.sas_select_topk(C.byref(sh), 4, 4, 0, 2, None, None, None, 0, 4, None, FAKE,
                               FAKE, FAKE, None, 0, None) == L.SAS_ERR_INVALID_ARG
    # kbar_ld smaller than C
    assert lib.sas_select_topk(C.byref(sh), 1, 8, 8, 2, None, FAKE, FAKE, 0, 7, FAKE, FAKE,
                               FAKE, FAKE, None, 0, None) == L.SAS_ERR_INVALID_ARG
    assert lib.sas_select_topk(C.byref(sh), 4, 20000, 0, 2, FAKE, None, None, 0, 0, None, FAKE,
                               FAKE, FAKE, None, 0, None) == L.SAS_ERR_UNSUPPORTED
    assert lib.sas_select_topk(C.byref(sh), 4, 4, 0, 0, FAKE, None, None, 0, 0, None, FAKE,
                               FAKE, FAKE, None, 0, None) == L.SAS_ERR_INVALID_ARG
    # long histories need the candidate workspace
    need = lib.sas_select_topk_workspace_size(C.byref(sh), 1, 8191, 31)
    assert need >= 32 * 31 * 8 * 2 and lib.sas_select_topk_workspace_size(C.byref(sh), 4, 512,
                                                                            31) == 0
    assert lib.sas_select_topk(C.byref(sh), 1, 8191, 8191, 31, FAKE, None, None, 0, 0, None,
                               FAKE, FAKE, FAKE, None, 0, None) == L.SAS_ERR_WORKSPACE
    # K > 64 only for histories of at most 512 blocks (the one-pass selection)
    assert lib.sas_select_topk(C.byref(sh), 1, 600, 600, 65, FAKE, None, None, 0, 0, None,
                               FAKE, FAKE, FAKE, None, 0, None) == L.SAS_ERR_UNSUPPORTED
    assert lib.sas_select_topk(C.byref(sh), 4, 4, 0, 255, FAKE, None, None, 0, 0, None,
                               FAKE, FAKE, FAKE, None, 0, None) == L.SAS_ERR_UNSUPPORTED
    assert lib.sas_select_topk_workspace_size(C.byref(sh), 1, 600, 65) == 0


def test_decode_checks():
    sh = shape(seqlen=1000, hq=32, hkv=8)
    lib = L.lib()
    need = lib.sas_decode_workspace_size(C.byref(sh), 31)
    assert need > 0
    call = lambda sh_, cl, ws, n: lib.sas_decode(C.byref(sh_), cl, 31, FAKE, FAKE, FAKE, FAKE,
                                                 FAKE, FAKE, FAKE, ws, n, None)
    assert call(sh, 999, FAKE, need) == L.SAS_ERR_INVALID_ARG        # cache shorter than L
    assert call(sh, 0, FAKE, need - 4) == L.SAS_ERR_WORKSPACE
    assert call(shape(seqlen=1000, hq=36, hkv=4), 0, FAKE, 1 << 30) == L.SAS_ERR_UNSUPPORTED


def test_pool_checks():
    sh = shape()
    lib = L.lib()
    assert lib.sas_block_pool(C.byref(sh), FAKE, 6, 4, 0, FAKE, None) == L.SAS_ERR_INVALID_ARG
    assert lib.sas_block_pool(C.byref(sh), None, 4, 4, 0, FAKE, None) == L.SAS_ERR_INVALID_ARG
    assert lib.sas_block_pool(C.byref(shape(head_dim=80)), FAKE, 4, 4, 0, FAKE,
                              None) == L.SAS_ERR_UNSUPPORTED


def test_profiler_is_inert_when_off():
    L.sas_profiler_enable(False)
    L.sas_profiler_reset()
    assert L.sas_profiler_read() == {}


def test_decode_step_checks():
    sh = shape(seqlen=4097, hq=32, hkv=8)   # C = 64
    lib = L.lib()
    need = lib.sas_decode_step_workspace_size(C.byref(sh), 31)
    assert need > 0 and lib.sas_decode_step_workspace_size(C.byref(sh), 65) == 0

    def call(sh_=sh, K=31, kbar_ld=64, idx=FAKE, logg=FAKE, lse_s=FAKE, kdt=L.SAS_DTYPE_BF16,
             ws=FAKE, n=need, cl=0, q=FAKE):
        return lib.sas_decode_step(C.byref(sh_), cl, K, q, FAKE, kdt, kbar_ld, FAKE, FAKE, 1,
                                   FAKE, FAKE, idx, logg, lse_s, ws, n, None)

    assert call(idx=None) == L.SAS_ERR_INVALID_ARG              # idx/logg/lse_s: all or none
    assert call(lse_s=None) == L.SAS_ERR_INVALID_ARG
    assert call(kbar_ld=63) == L.SAS_ERR_INVALID_ARG            # kbar rows < C
    assert call(kdt=7) == L.SAS_ERR_INVALID_ARG
    assert call(q=FAKE + 8) == L.SAS_ERR_INVALID_ARG            # 16-byte alignment
    assert call(cl=4096) == L.SAS_ERR_INVALID_ARG               # cache shorter than L
    assert call(K=0) == L.SAS_ERR_INVALID_ARG
    assert call(K=65) == L.SAS_ERR_UNSUPPORTED
    assert call(ws=None) == L.SAS_ERR_WORKSPACE
    assert call(n=need - 1) == L.SAS_ERR_WORKSPACE
    assert call(shape(seqlen=4097, hq=36, hkv=4)) == L.SAS_ERR_UNSUPPORTED   # G = 9
    big = shape(seqlen=64 * 16385 + 1, hq=4, hkv=1)                          # C = 16385
    assert call(big, kbar_ld=16385, n=1 << 40) == L.SAS_ERR_UNSUPPORTED


def test_decode_step_noalloc_rejects_more_than_its_scratch():
    """The entry point without a workspace argument refuses, from host
    arithmetic alone, a step needing more than its static scratch, and its
    scratch size is the header's."""
    text = open(os.path.join(ROOT, "include", "sas.h")).read()
    m = re.search(r"#define SAS_STATIC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == L.SAS_STATIC_SCRATCH_BYTES
    lib = L.lib()
    big = shape(batch=64, hq=32, hkv=8, seqlen=65536)     # 18 MB of candidates + partials
    assert lib.sas_decode_step_workspace_size(C.byref(big), 63) > L.SAS_STATIC_SCRATCH_BYTES
    args = [C.byref(big), 0, 63, FAKE, FAKE, L.SAS_DTYPE_BF16, 1023, FAKE, FAKE, 1, FAKE, FAKE,
            None, None, None, None]
    assert lib.sas_decode_step_noalloc(*args) == L.SAS_ERR_WORKSPACE
    args[2] = 65                                            # K past the supported range
    assert lib.sas_decode_step_noalloc(*args) == L.SAS_ERR_UNSUPPORTED
    bad = shape(batch=0)
    args[0], args[2] = C.byref(bad), 8
    assert lib.sas_decode_step_noalloc(*args) == L.SAS_ERR_INVALID_ARG


def test_selector_bwd_checks():
    sh = shape(seqlen=1000, hq=8, hkv=2)
    lib = L.lib()

    def call(ds=FAKE, qbar=FAKE, kbar=FAKE, dqbar=FAKE, dkbar=FAKE, dq=None, dk=None, sh_=sh):
        return lib.sas_selector_bwd(C.byref(sh_), ds, qbar, kbar, dqbar, dkbar, dq, dk, None)

    for name in ("ds", "qbar", "kbar", "dqbar", "dkbar"):
        assert call(**{name: None}) == L.SAS_ERR_INVALID_ARG
    assert call(dq=FAKE + 4) == L.SAS_ERR_INVALID_ARG
    assert call(kbar=FAKE + 8) == L.SAS_ERR_INVALID_ARG
    assert call(sh_=shape(head_dim=96)) == L.SAS_ERR_UNSUPPORTED


def test_gate_bits_are_validated():
    for bad in (3, 16, 0x13):
        assert fwd(shape(gate=bad)) == L.SAS_ERR_INVALID_ARG
    assert L.gate_code("sigmoid", outer=True, ste=True) == 1 | 4 | 8
    sh = shape(seqlen=8192, hq=32, hkv=8)
    n = L.lib().sas_attn_bwd_workspace_size(C.byref(sh), 31)
    args = [FAKE] * 13
    args[9] = None   # lse_s: the softmax gate's ds needs it
    st = L.lib().sas_attn_bwd(C.byref(sh), 31, *args, FAKE, FAKE, FAKE, n, None)
    assert st == L.SAS_ERR_INVALID_ARG


def test_paged_decode_checks():
    sh = shape(seqlen=1000, hq=8, hkv=2)     # 16 blocks of 64
    lib = L.lib()
    ws = lib.sas_decode_workspace_size(C.byref(sh), 8)

    def call(kp=FAKE, table=FAKE, bt_ld=16, lens=FAKE, npages=40, K=8, n=ws):
        return lib.sas_decode_paged(C.byref(sh), K, FAKE, kp, FAKE, npages, table, bt_ld, lens,
                                    FAKE, FAKE, FAKE, FAKE, FAKE, n, None)

    assert call(table=None) == L.SAS_ERR_INVALID_ARG
    assert call(lens=None) == L.SAS_ERR_INVALID_ARG
    assert call(kp=FAKE + 4) == L.SAS_ERR_INVALID_ARG
    assert call(npages=0) == L.SAS_ERR_INVALID_ARG
    assert call(bt_ld=15) == L.SAS_ERR_INVALID_ARG          # table narrower than seqlen
    assert call(K=65) == L.SAS_ERR_UNSUPPORTED
    assert call(n=ws - 1) == L.SAS_ERR_WORKSPACE
    # the paged step: the same host-side checks (all fail before any launch)
    n = lib.sas_decode_step_workspace_size(C.byref(sh), 8)

    def step(K=8, table=FAKE, bt_ld=16, kbar_ld=64, n_=n):
        return lib.sas_decode_step_paged(C.byref(sh), K, FAKE, FAKE, L.SAS_DTYPE_BF16, kbar_ld,
                                         FAKE, FAKE, 40, table, bt_ld, FAKE, 1, FAKE, FAKE, None,
                                         None, None, FAKE, n_, None)

    assert step(K=65) == L.SAS_ERR_UNSUPPORTED
    assert step(table=None) == L.SAS_ERR_INVALID_ARG
    assert step(bt_ld=15) == L.SAS_ERR_INVALID_ARG
    assert step(kbar_ld=14) == L.SAS_ERR_INVALID_ARG         # C = 15 pooled rows needed
    assert step(n_=n - 1) == L.SAS_ERR_WORKSPACE


def test_struct_layouts_match_the_header(tmp_path):
    """The ctypes mirrors of sas_shape and sas_kernel_time have the C header's
    size and field offsets (compiled with the host C compiler)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    src = tmp_path / "layout.c"
    fields = [f[0] for f in L.sas_shape._fields_]
    src.write_text(
        '#include <stddef.h>\n#include <stdio.h>\n#include "sas.h"\nint main(void) {\n'
        '  printf("%zu %zu\\n", sizeof(sas_shape), sizeof(sas_kernel_time));\n'
        + "".join(f'  printf("%zu\\n", offsetof(sas_shape, {f}));\n' for f in fields)
        + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()
    assert int(out[0]) == C.sizeof(L.sas_shape)
    assert int(out[1]) == C.sizeof(L.sas_kernel_time)
    for f, off in zip(fields, out[2:]):
        assert int(off) == getattr(L.sas_shape, f).offset, f
