"""Host-side checks of the C-ABI library: it loads without a GPU, exports every
function include/gdn.h declares, and rejects bad arguments before launching
anything (these calls never reach the device)."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_24_amd as gdn
from gated_delta_rule_24_amd import ChunkDesc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

FAKE = 0x10000          # aligned, never dereferenced: validation fails first
FAKE2 = 0x20000000


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return gdn.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), f"{n} declared in gdn.h but not exported"


def test_version_and_status_strings(lib):
    assert lib.gdn_abi_version() == 5
    for code, name in [(0, b"GDN_OK"), (2, b"GDN_ERR_SHAPE"), (9, b"GDN_ERR_DEVICE_INPUT")]:
        assert lib.gdn_status_string(code) == name


def desc(**kw):
    base = dict(batch=2, seqlen=100, heads=3, dk=128, dv=128, num_seqs=2, chunk=64, in_dtype=1, out_dtype=0, flags=0)
    base.update(kw)
    return ChunkDesc(**base)


def ws_size(lib, d):
    n = ctypes.c_size_t(0)
    st = lib.gdn_chunk_fwd_workspace_size(ctypes.byref(d), ctypes.byref(n))
    return st, n.value


def test_workspace_size_host_only(lib):
    st, n = ws_size(lib, desc())
    assert st == 0 and n > 0
    # grows with tokens and covers both the packed and the batched layout
    st2, n2 = ws_size(lib, desc(seqlen=1000))
    assert st2 == 0 and n2 > n
    st3, n3 = ws_size(lib, desc(batch=1, seqlen=5000, num_seqs=9))
    assert st3 == 0 and n3 >= 256


@pytest.mark.parametrize("kw,code", [
    (dict(in_dtype=7), 3), (dict(out_dtype=-1), 3), (dict(batch=0), 2), (dict(heads=0), 2),
    (dict(seqlen=-1), 2), (dict(chunk=32), 5), (dict(dk=96), 5), (dict(dv=24), 5), (dict(dv=2048), 5),
    (dict(dk=256, in_dtype=0), 5), (dict(num_seqs=0), 2), (dict(flags=4), 5),
])
def test_bad_descriptor(lib, kw, code):
    st, _ = ws_size(lib, desc(**kw))
    assert st == code
    assert lib.gdn_last_error_message()


def call_chunk(lib, d, q=FAKE, k=FAKE, v=FAKE, la=FAKE, beta=FAKE, init=None, cu=None, o=FAKE2, fin=None,
               ws=FAKE2 * 4, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = ws_size(lib, d)[1]
    vp = ctypes.c_void_p
    return lib.gdn_chunk_fwd(ctypes.byref(d), vp(q), vp(k), vp(v), vp(la), vp(beta), vp(init), vp(cu), vp(o),
                             vp(fin), vp(ws), ctypes.c_size_t(ws_bytes), None)


def test_chunk_argument_errors(lib):
    d = desc()
    assert call_chunk(lib, d, q=None) == 1                              # NULL input
    assert call_chunk(lib, d, ws=None) == 6                             # no workspace
    assert call_chunk(lib, d, ws_bytes=16) == 6                         # workspace too small
    assert call_chunk(lib, d, k=FAKE + 8) == 4                          # misaligned
    assert call_chunk(lib, d, la=FAKE + 2) == 4                         # gates: 4-byte alignment
    assert call_chunk(lib, d, cu=FAKE) == 2                             # cu with batch != 1
    assert call_chunk(lib, desc(num_seqs=3)) == 2                       # N != B without cu
    assert call_chunk(lib, d, o=FAKE) == 8                              # o aliases q
    assert call_chunk(lib, d, init=FAKE2 * 2, fin=FAKE2 * 2 + 256) == 8  # partial state overlap
    assert b"overlap" in lib.gdn_last_error_message()


def call_bwd(lib, d, q=FAKE, k=FAKE, v=FAKE, la=FAKE, beta=FAKE, init=None, cu=None, do=FAKE * 2, dfin=None,
             dq=FAKE2, dk=FAKE2 * 2, dv=FAKE2 * 3, dla=FAKE2 * 5, db=FAKE2 * 6, dinit=None, ws=FAKE2 * 8,
             ws_bytes=None):
    if ws_bytes is None:
        n = ctypes.c_size_t(0)
        assert lib.gdn_chunk_bwd_workspace_size(ctypes.byref(d), ctypes.byref(n)) == 0
        ws_bytes = n.value
    vp = ctypes.c_void_p
    return lib.gdn_chunk_bwd(ctypes.byref(d), vp(q), vp(k), vp(v), vp(la), vp(beta), vp(init), vp(cu), vp(do),
                             vp(dfin), vp(dq), vp(dk), vp(dv), vp(dla), vp(db), vp(dinit), vp(ws),
                             ctypes.c_size_t(ws_bytes), None)


def test_bwd_workspace_and_argument_errors(lib):
    n = ctypes.c_size_t(0)
    # prefill shape: T, P, decay vectors, two state checkpoints per (chunk, head)
    d = desc(batch=4, seqlen=4096, heads=16, num_seqs=4)
    assert lib.gdn_chunk_bwd_workspace_size(ctypes.byref(d), ctypes.byref(n)) == 0
    rows = 4 * 64 * 16
    assert n.value >= rows * (2 * 64 * 64 * 4 + 4 * 64 * 4 + 2 * 128 * 128 * 4)
    d = desc()
    assert call_bwd(lib, desc(dk=256)) == 5                            # dk 256 not differentiated
    assert call_bwd(lib, desc(flags=4), ws_bytes=1 << 20) == 5         # unknown option
    assert lib.gdn_chunk_bwd_workspace_size(ctypes.byref(desc(flags=4)), ctypes.byref(n)) == 5
    # q/k normalisation: the normalised rows, v as fp32 and two factors per (token, head) on top
    n1 = ctypes.c_size_t(0)
    assert lib.gdn_chunk_bwd_workspace_size(ctypes.byref(desc(flags=1)), ctypes.byref(n1)) == 0
    assert lib.gdn_chunk_bwd_workspace_size(ctypes.byref(desc()), ctypes.byref(n)) == 0
    assert n1.value - n.value >= 2 * 100 * 3 * (2 * 128 + 128 + 2) * 4
    assert call_bwd(lib, d, do=None) == 1
    assert call_bwd(lib, d, dla=None) == 1
    assert call_bwd(lib, d, ws=None) == 6
    assert call_bwd(lib, d, ws_bytes=16) == 6
    assert call_bwd(lib, d, dq=FAKE2 + 4) == 4                         # 16-byte alignment
    assert call_bwd(lib, d, db=FAKE2 * 6 + 2) == 4                     # 4-byte alignment
    assert call_bwd(lib, d, cu=FAKE) == 2                              # cu with batch != 1
    assert call_bwd(lib, d, dk=FAKE) == 8                              # output over an input
    assert call_bwd(lib, d, dv=FAKE2 + 256) == 8                       # two outputs overlap
    assert call_bwd(lib, d, dinit=FAKE2 * 8 + 4096) == 8               # output inside the workspace
    assert b"overlaps" in lib.gdn_last_error_message()


def test_decode_argument_errors(lib):
    vp = ctypes.c_void_p

    def call(N=4, H=2, dk=128, dv=128, idt=1, odt=0, flags=0, state=FAKE2, q=FAKE, k=FAKE, v=FAKE, la=FAKE, b=FAKE,
             o=FAKE2 * 8):
        return lib.gdn_decode_step(N, H, dk, dv, idt, odt, flags, vp(state), vp(q), vp(k), vp(v), vp(la), vp(b),
                                   vp(o), None)

    assert call(idt=5) == 3
    assert call(flags=2) == 5                       # unknown option
    assert call(H=0) == 2
    assert call(dk=48) == 5
    assert call(dv=5000) == 5
    assert call(q=None) == 1
    assert call(v=FAKE + 2) == 4
    assert call(la=FAKE + 2) == 4                   # gates need 4-byte alignment
    assert call(la=FAKE + 4, b=FAKE + 8, o=FAKE2 + 64) == 8   # ... and no more (the later alias check fails)
    assert call(o=FAKE2 + 64) == 8                  # o inside the state
    assert call(N=0, state=None, q=None) == 0       # nothing to do


def test_python_binding_requires_library(monkeypatch, tmp_path):
    # With the library missing the binding raises instead of computing anything.
    monkeypatch.setenv("GDN_LIB", str(tmp_path / "missing.so"))
    monkeypatch.setattr(gdn, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        gdn.load()


def test_noalloc_rejects_oversized_calls(lib):
    """gdn_chunk_fwd_noalloc refuses, on the host, a call whose workspace would exceed its scratch
    array (GDN_NOALLOC_SCRATCH_BYTES), with GDN_ERR_WORKSPACE and a message that names the limit."""
    vp = ctypes.c_void_p
    big = desc(batch=8, seqlen=8192, heads=16, num_seqs=8)
    assert ws_size(lib, big)[1] > gdn.NOALLOC_SCRATCH_BYTES
    st = lib.gdn_chunk_fwd_noalloc(ctypes.byref(big), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), None, None,
                                   vp(FAKE2), None, None)
    assert st == 6
    assert str(gdn.NOALLOC_SCRATCH_BYTES).encode() in lib.gdn_last_error_message()
    assert lib.gdn_chunk_fwd_noalloc(ctypes.byref(desc(in_dtype=7)), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE),
                                     vp(FAKE), None, None, vp(FAKE2), None, None) == 3
