"""C-ABI checks that need no GPU: libdsa.so loads, exports every function
include/dsa.h declares, the ctypes structs match the C layout, and the host
validation rejects bad arguments before anything is launched."""
import ctypes
import os
import re
import subprocess

import pytest

import sparse_attention_index_amd as dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:dsa_status|const char\*|int)\s+(dsa_\w+)\s*\(",
                                 text, re.M)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) == 16, names
    L = dsa.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(dsa.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", dsa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (dsa_\w+)$", out, re.M))
    assert set(names) <= exported
    # every kernel and helper of the library is defined in it (a kernel
    # template the host pass failed to instantiate would be left undefined)
    undef = subprocess.run(["nm", "-D", "--undefined-only", dsa.LIB_PATH], capture_output=True,
                           text=True, check=True).stdout
    assert not re.findall(r"_ZN3dsa\w*", undef), undef


def test_abi_version_and_status_strings():
    L = dsa.lib()
    assert L.dsa_abi_version() == 3
    for code in range(8):
        assert dsa.status_str(code).startswith("DSA_")
    assert dsa.status_str(99) == "unknown dsa_status"


STRUCTS = {
    "dsa_rope_table_args": dsa.RopeTableArgs,
    "dsa_indexer_args": dsa.IndexerArgs,
    "dsa_topk_args": dsa.TopkArgs,
    "dsa_mla_args": dsa.MlaArgs,
    "dsa_mla_append_args": dsa.MlaAppendArgs,
    "dsa_mla_proj_args": dsa.MlaProjArgs,
    "dsa_mha_args": dsa.MhaArgs,
}


def test_ctypes_structs_match_c_layout(tmp_path):
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "dsa.h"', 'int main(void) {']
    for cname, st in STRUCTS.items():
        lines.append(f'printf("{cname} size %zu\\n", sizeof({cname}));')
        for fname, _ in st._fields_:
            lines.append(f'printf("{cname} {fname} %zu\\n", offsetof({cname}, {fname}));')
    lines.append("return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I",
                    "/opt/rocm/include", str(src), "-o", str(exe)], check=True)
    got = {}
    for ln in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n"):
        if ln:
            c, f, v = ln.split()
            got[(c, f)] = int(v)
    for cname, st in STRUCTS.items():
        assert got[(cname, "size")] == ctypes.sizeof(st), cname
        for fname, _ in st._fields_:
            assert got[(cname, fname)] == getattr(st, fname).offset, (cname, fname)


# ---- host-side validation (no launch happens on these paths) -----------------

FAKE = 1 << 20          # a 16-byte aligned non-null address that is never touched


def good_indexer():
    return dsa.IndexerArgs(1, 1, 64, 16384, 16384, dsa.DSA_DTYPE_BF16, FAKE, FAKE, FAKE, FAKE,
                           FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16384, 0, None, 0)


def call(fn, args):
    return fn(ctypes.byref(args), None)


def test_indexer_validation():
    L = dsa.lib()
    n = ctypes.c_size_t(123)
    assert L.dsa_indexer_workspace(ctypes.byref(good_indexer()), ctypes.byref(n)) == 0
    assert n.value == 0                         # q_fp8/q_scale given -> no workspace
    cases = [
        (dict(H=65), 2), (dict(H=0), 2), (dict(B=0), 2), (dict(Lmax=0), 2), (dict(P=0), 2),
        (dict(ld_scores=100), 2), (dict(act_dtype=7), 3), (dict(flags=8), 3),
        (dict(flags=1, k_raw=None), 1), (dict(flags=1, k_raw=FAKE + 1), 5), (dict(k_raw=FAKE + 8), 5),
        (dict(q_raw=FAKE + 4), 5), (dict(rope_sin=FAKE + 4), 5),
        (dict(q_raw=None), 1), (dict(scores=None), 1), (dict(q_scale=None), 1),
        (dict(k_cache=FAKE + 8), 5), (dict(B=300, S=300), 2),
    ]
    for change, code in cases:
        a = good_indexer()
        for k, v in change.items():
            setattr(a, k, v)
        assert call(L.dsa_indexer, a) == code, change
    # missing workspace when q_fp8 is not given (multi-row calls; a decode
    # call with S == 1 keeps its quantised query on chip)
    a = good_indexer()
    a.q_fp8, a.q_scale = None, None
    assert L.dsa_indexer_workspace(ctypes.byref(a), ctypes.byref(n)) == 0 and n.value == 0
    a.S = 2
    assert L.dsa_indexer_workspace(ctypes.byref(a), ctypes.byref(n)) == 0
    assert n.value >= 64 * 128 + 64 * 4
    assert call(L.dsa_indexer, a) == 4
    a.workspace, a.workspace_bytes = FAKE, n.value - 1
    assert call(L.dsa_indexer, a) == 4
    assert L.dsa_indexer(None, None) == 1


def good_topk():
    return dsa.TopkArgs(2, 1, 16384, 2048, FAKE, 16384, FAKE, FAKE, None, None, 0)


def test_topk_validation():
    L = dsa.lib()
    for change, code in [(dict(K=2049), 2), (dict(K=0), 2), (dict(ld_scores=10), 2),
                         (dict(scores=None), 1), (dict(idx=None), 1), (dict(pos=FAKE + 2), 5)]:
        a = good_topk()
        for k, v in change.items():
            setattr(a, k, v)
        assert call(L.dsa_topk, a) == code, change
    n = ctypes.c_size_t(7)
    assert L.dsa_topk_workspace(ctypes.byref(good_topk()), ctypes.byref(n)) == 0
    assert n.value == 0                            # rows of up to 16,384 scores
    a = good_topk()
    a.Lmax = a.ld_scores = 131072
    assert L.dsa_topk_workspace(ctypes.byref(a), ctypes.byref(n)) == 0
    assert n.value >= 2 * 8 * 2048 * 8             # 8 chunk lists of (key, position) per row
    a.workspace, a.workspace_bytes = FAKE, n.value - 1
    assert call(L.dsa_topk, a) == 4
    a.workspace_bytes, a.workspace = n.value, FAKE + 16
    assert call(L.dsa_topk, a) == 5
    a = good_topk()
    a.B, a.Lmax, a.ld_scores = 1 << 30, 1 << 21, 1 << 21   # 2^37 level-0 blocks
    assert call(L.dsa_topk, a) == 2


def good_mla(B=1, S=1, K=2048):
    return dsa.MlaArgs(B, S, 128, 16384, K, FAKE, FAKE, 512, 512 * 16384, FAKE, 64, 64 * 16384,
                       FAKE, 0.07, FAKE, None, None, 0)


def test_mla_validation():
    L = dsa.lib()
    for change, code in [(dict(Hq=129), 2), (dict(K=4096), 2), (dict(scale=0.0), 2),
                         (dict(scale=float("inf")), 2), (dict(latent_row_stride=500), 2),
                         (dict(latent_row_stride=516), 5), (dict(q=FAKE + 4), 5),
                         (dict(out=None), 1), (dict(idx=None), 1)]:
        a = good_mla()
        for k, v in change.items():
            setattr(a, k, v)
        assert call(L.dsa_sparse_mla, a) == code, change
    # decode row needs key-split partials -> workspace required
    n = ctypes.c_size_t(0)
    a = good_mla()
    assert L.dsa_sparse_mla_workspace(ctypes.byref(a), ctypes.byref(n)) == 0
    assert n.value > 0
    assert call(L.dsa_sparse_mla, a) == 4
    # a large batch of rows runs unsplit: no workspace
    a = good_mla(B=1, S=4096)
    assert L.dsa_sparse_mla_workspace(ctypes.byref(a), ctypes.byref(n)) == 0
    assert n.value == 0


def test_mla_noalloc_validation():
    """The no-allocation call validates like dsa_sparse_mla and rejects a
    call whose key-split partials exceed its static scratch, before any HIP
    call (so it needs no GPU here)."""
    L = dsa.lib()
    for change, code in [(dict(Hq=129), 2), (dict(K=4096), 2), (dict(q=FAKE + 4), 5),
                         (dict(out=None), 1)]:
        a = good_mla()
        for k, v in change.items():
            setattr(a, k, v)
        assert call(L.dsa_sparse_mla_noalloc, a) == code, change
    n = ctypes.c_size_t(0)
    for rows, fits in ((1, True), (32, True), (220, True), (221, False), (255, False),
                       (256, True)):
        a = good_mla(B=rows)
        assert L.dsa_sparse_mla_workspace(ctypes.byref(a), ctypes.byref(n)) == 0
        assert (n.value <= dsa.MLA_NOALLOC_MAX_BYTES) == fits, rows
        if not fits:
            assert call(L.dsa_sparse_mla_noalloc, a) == dsa.DSA_ERR_SCRATCH
            assert dsa.status_str(dsa.DSA_ERR_SCRATCH).startswith("DSA_ERR_SCRATCH")


def test_rope_table_validation():
    L = dsa.lib()
    a = dsa.RopeTableArgs(100, 1, 4096, 10000.0, 40.0, 1.0, 32.0, FAKE, FAKE)   # fast < slow
    assert call(L.dsa_rope_table, a) == 2
    a = dsa.RopeTableArgs(0, 0, 4096, 10000.0, 40.0, 32.0, 1.0, FAKE, FAKE)
    assert call(L.dsa_rope_table, a) == 2
    a = dsa.RopeTableArgs(10, 2, 4096, 10000.0, 40.0, 32.0, 1.0, FAKE, FAKE)
    assert call(L.dsa_rope_table, a) == 3
    a = dsa.RopeTableArgs(10, 0, 4096, 10000.0, 40.0, 32.0, 1.0, None, FAKE)
    assert call(L.dsa_rope_table, a) == 1


def good_append(q=None):
    return dsa.MlaAppendArgs(2, 3, 128, 1024, 1024, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 512,
                             512 * 1024, FAKE, 64, 64 * 1024, q)


def test_mla_append_validation():
    L = dsa.lib()
    for change, code in [(dict(B=0), 2), (dict(P=0), 2), (dict(latent_row_stride=500), 2),
                         (dict(rope_batch_stride=-8), 2), (dict(latent_row_stride=520), 0),
                         (dict(rope_row_stride=66), 5), (dict(latent_new=None), 1),
                         (dict(rope=None), 1), (dict(kpe_new=FAKE + 4), 5),
                         (dict(pos=FAKE + 2), 5), (dict(q=FAKE, Hq=0), 2),
                         (dict(q=FAKE, Hq=129), 2), (dict(q=FAKE + 8), 5)]:
        a = good_append()
        for k, v in change.items():
            setattr(a, k, v)
        if code == 0:
            continue                 # valid arguments would launch: GPU tests cover them
        assert call(L.dsa_mla_append, a) == code, change
    assert L.dsa_mla_append(None, None) == 1


@pytest.mark.parametrize("fields,code", [
    (dict(page_size=3), 2), (dict(page_size=0), 2), (dict(page_size=131072), 2),
    (dict(num_pages=0), 2), (dict(max_pages=1), 2), (dict(num_pages=1 << 30), 2),
    (dict(block_table=FAKE + 2), 5)])
def test_paging_validation(fields, code):
    """The paged-cache fields are checked the same way by every call that
    takes them (here Lmax = 16384 or 1024, page_size 64 -> max_pages >= 256 / 16)."""
    L = dsa.lib()
    for make, fn in ((good_indexer, L.dsa_indexer), (good_mla, L.dsa_sparse_mla),
                     (good_append, L.dsa_mla_append)):
        a = make()
        a.block_table, a.page_size, a.max_pages, a.num_pages = FAKE, 64, 256, 1000
        for k, v in fields.items():
            setattr(a, k, v)
        assert call(fn, a) == code, (make.__name__, fields)


def good_proj(mode):
    # 2 batches x 300 rows x 128 heads, contiguous layouts
    if mode == "kv_up":
        return dsa.MlaProjArgs(2, 300, 128, FAKE, FAKE, 512, 512 * 300, 0, FAKE, 128 * 256,
                               128 * 256 * 300, 0)
    din, dout = (128, 512) if mode == "absorb_q" else (512, 128)
    return dsa.MlaProjArgs(2, 300, 128, FAKE, FAKE, 128 * din, 128 * din * 300, din, FAKE,
                           128 * dout, 128 * dout * 300, dout)


@pytest.mark.parametrize("mode", ["kv_up", "absorb_q", "absorb_o"])
def test_mla_proj_validation(mode):
    L = dsa.lib()
    fn = getattr(L, "dsa_mla_" + mode)
    cases = [(dict(B=0), 2), (dict(rows=0), 2), (dict(Hq=129), 2), (dict(Hq=0), 2),
             (dict(rows=(1 << 24) + 1), 2), (dict(wkv_b=None), 1), (dict(x=None), 1),
             (dict(y=None), 1), (dict(x=FAKE + 8), 5), (dict(wkv_b=FAKE + 2), 5),
             (dict(x_row_stride=-8), 2), (dict(y_batch_stride=8), 2)]
    if mode == "kv_up":
        cases += [(dict(y_row_stride=128 * 256 - 8), 2), (dict(x_row_stride=516), 5),
                  (dict(B=70000), 2)]
    else:
        # the 576-wide query as output of the query absorption is fine
        cases += [(dict(y_head_stride=8), 2), (dict(x_head_stride=4), 5),
                  (dict(B=600), 2)]                          # B * Hq grid rows > 65535
    for change, code in cases:
        a = good_proj(mode)
        for k, v in change.items():
            setattr(a, k, v)
        assert call(fn, a) == code, change
    assert fn(None, None) == 1


def good_mha():
    return dsa.MhaArgs(1, 4096, 128, 4096, 2048, FAKE, FAKE, FAKE, 64, 64 * 4096, FAKE, FAKE,
                       0.1, FAKE, None, 0)


def test_mha_validation():
    L = dsa.lib()
    for change, code in [(dict(Hq=129), 2), (dict(K=2049), 2), (dict(Lmax=65537), 2),
                         (dict(S=0), 2), (dict(scale=0.0), 2), (dict(rope_row_stride=32), 2),
                         (dict(q=None), 1), (dict(kv=None), 1), (dict(idx=None), 1),
                         (dict(out=None), 1), (dict(kv=FAKE + 8), 5), (dict(pos=FAKE + 2), 5),
                         (dict(rope_row_stride=68), 5)]:
        a = good_mha()
        for k, v in change.items():
            setattr(a, k, v)
        assert call(L.dsa_sparse_mha, a) == code, change
    n = ctypes.c_size_t(0)
    a = good_mha()
    assert L.dsa_sparse_mha_workspace(ctypes.byref(a), ctypes.byref(n)) == 0
    # bit masks (4096 rows x 128 words) and tile lists (32 query tiles x 65 entries)
    assert n.value >= 4096 * 128 * 4 + 32 * 65 * 16
    assert call(L.dsa_sparse_mha, a) == 4
    a.workspace, a.workspace_bytes = FAKE + 16, n.value
    assert call(L.dsa_sparse_mha, a) == 5
    a.workspace, a.workspace_bytes = FAKE, n.value - 1
    assert call(L.dsa_sparse_mha, a) == 4
    a.pos = None                                   # positions are optional
    a.workspace_bytes = n.value - 1
    assert call(L.dsa_sparse_mha, a) == 4


C_CALLER = r"""
#include <stdio.h>
#include <string.h>
#include "dsa.h"

/* A C caller: the header compiles as C, the library links, and calls whose
 * arguments fail validation return their status without touching the GPU. */
int main(void) {
    dsa_mha_args m;
    dsa_mla_proj_args p;
    dsa_topk_args t;
    size_t n = 0;
    int fails = 0;
    if (dsa_abi_version() != DSA_ABI_VERSION) ++fails;
    if (strncmp(dsa_status_str(DSA_ERR_SHAPE), "DSA_ERR_SHAPE", 13) != 0) ++fails;
    if (dsa_sparse_mha(NULL, NULL) != DSA_ERR_NULL) ++fails;
    memset(&m, 0, sizeof m);
    m.B = 1; m.S = 1; m.Hq = 129; m.Lmax = 16; m.K = 4; m.scale = 0.1f;
    if (dsa_sparse_mha_workspace(&m, &n) != DSA_ERR_SHAPE) ++fails;
    memset(&p, 0, sizeof p);
    p.B = 1; p.rows = 1; p.Hq = 1;
    if (dsa_mla_kv_up(&p, NULL) != DSA_ERR_NULL) ++fails;
    memset(&t, 0, sizeof t);
    t.B = 1; t.S = 1; t.Lmax = 16; t.K = 4096;
    if (dsa_topk(&t, NULL) != DSA_ERR_SHAPE) ++fails;
    printf("%d\n", fails);
    return fails;
}
"""


def test_c_caller_links_and_validates(tmp_path):
    src = tmp_path / "caller.c"
    src.write_text(C_CALLER)
    exe = tmp_path / "caller"
    libdir = os.path.dirname(dsa.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I",
                    os.path.join(ROOT, "include"), "-I", "/opt/rocm/include", str(src), "-o",
                    str(exe), "-L", libdir, "-ldsa", "-Wl,-rpath," + libdir, "-L/opt/rocm/lib",
                    "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0 and r.stdout.strip() == "0", (r.stdout, r.stderr)
