"""C-ABI checks that need no GPU: the library loads, exports every function
declared in include/*.h, sizes workspaces, and rejects bad arguments on the
host before anything is enqueued (each case below fails a host check, so no
kernel is ever launched here).  The host checks run against the product
entry points and against their instrumented *_timed twins."""
import ctypes as ct
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec_verify.h")
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))


class _TimedTwins:
    """The library with every entry point that has a *_timed twin replaced
    by that twin, called with a null event array."""

    def __init__(self, lib):
        self._lib = lib

    def __getattr__(self, name):
        f = getattr(self._lib, name)
        t = getattr(self._lib, name + "_timed", None) if not name.endswith("_timed") else None
        if t is None:
            return f
        return lambda *args: t(*args, None)


def _load():
    import exact_draft_verification_amd as sv

    if not os.path.exists(sv.library_path()):
        from exact_draft_verification_amd import build

        build.build()
    return sv.load_library()


@pytest.fixture(scope="module", params=["product", "timed"])
def lib(request):
    real = _load()
    return real if request.param == "product" else _TimedTwins(real)


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(spec_\w+)\s*\(", text))
    return sorted(names)


def header_constants():
    text = open(HEADER).read()
    return {k: int(v) for k, v in re.findall(r"#define\s+(SV_\w+)\s+(\d+)", text)}


def test_exports_every_declared_symbol():
    lib = _load()
    names = declared_functions()
    assert {"spec_verify_chain", "spec_verify_tree_greedy", "spec_verify_chain_workspace_bytes",
            "spec_verify_tree_greedy_workspace_bytes", "spec_verify_status_string",
            "spec_verify_chain_pointmass", "spec_verify_chain_pointmass_workspace_bytes",
            "spec_outcome_topk", "spec_outcome_topk_workspace_bytes",
            "spec_cache_lookup", "spec_tree_build", "spec_tree_build_workspace_bytes",
            "spec_verify_tree_stochastic", "spec_verify_tree_stochastic_workspace_bytes",
            "spec_verify_chain_timed", "spec_verify_chain_pointmass_timed",
            "spec_verify_tree_greedy_timed", "spec_verify_tree_stochastic_timed",
            "spec_outcome_topk_timed", "spec_tree_build_timed"} <= set(names)
    for name in names:
        assert hasattr(lib, name), name


def test_binding_constants_match_header():
    import exact_draft_verification_amd as sv

    c = header_constants()
    assert sv.SV_DTYPE_F32 == c["SV_DTYPE_F32"] and sv.SV_DTYPE_BF16 == c["SV_DTYPE_BF16"]
    assert sv.SV_MAX_VOCAB == c["SV_MAX_VOCAB"]


def test_status_strings(lib):
    import exact_draft_verification_amd as sv

    c = header_constants()
    for name in ("SV_OK", "SV_ERR_NULL", "SV_ERR_SHAPE", "SV_ERR_TEMPERATURE", "SV_ERR_DTYPE",
                 "SV_ERR_WORKSPACE", "SV_ERR_HIP", "SV_ERR_ALIGN"):
        s = sv.spec_verify_status_string(c[name])
        assert s and s != "unknown status"
    assert sv.spec_verify_status_string(999) == "unknown status"


def test_workspace_sizes(lib):
    import exact_draft_verification_amd as sv

    c3 = sv.spec_verify_chain_workspace_bytes(64, 16, 151936, sv.SV_DTYPE_BF16)
    assert c3 > 0 and c3 % 256 == 0
    assert sv.spec_verify_chain_workspace_bytes(1, 16, 151936, sv.SV_DTYPE_F32) > 0
    assert sv.spec_verify_tree_greedy_workspace_bytes(64, 64, 151936, 1) > 0
    for bad in [(0, 16, 100, 0), (1, 0, 100, 0), (1, 16, 0, 0), (1, 256, 100, 0), (1, 4, 100, 7),
                (-1, 4, 100, 1)]:
        assert sv.spec_verify_chain_workspace_bytes(*bad) == 0, bad
    for bad in [(0, 4, 100, 1), (1, 0, 100, 1), (1, 1025, 100, 1), (1, 4, 0, 1), (1, 4, 100, 2)]:
        assert sv.spec_verify_tree_greedy_workspace_bytes(*bad) == 0, bad
    # larger problems never need less workspace
    assert sv.spec_verify_chain_workspace_bytes(256, 16, 151936, 1) >= c3
    # the vocabulary limit, on every entry point
    vmax = sv.SV_MAX_VOCAB
    assert sv.spec_verify_chain_workspace_bytes(1, 1, vmax, 1) > 0
    assert sv.spec_verify_chain_workspace_bytes(1, 1, vmax + 1, 1) == 0
    assert sv.spec_verify_chain_pointmass_workspace_bytes(1, 1, vmax + 1, 1) == 0
    assert sv.spec_verify_tree_greedy_workspace_bytes(1, 2, vmax + 1, 1) == 0
    assert sv.spec_verify_tree_stochastic_workspace_bytes(1, 2, vmax + 1, 1) == 0
    assert sv.spec_outcome_topk_workspace_bytes(1, 1, vmax + 1, 1, 4) == 0
    assert sv.spec_tree_build_workspace_bytes(1, 5, vmax + 1, 1, 4, 2, 5) == 0
    assert sv.spec_tree_build_workspace_bytes(1, 5, vmax, 1, 4, 2, 5) > 0


class HostBufs:
    """Host buffers standing in for device pointers: every call below fails a
    host check before the library would touch them."""

    def __init__(self, B, g, V):
        self.B, self.g, self.V = B, g, V
        self.t = np.zeros((B, g + 1, V), np.float32)
        self.d = np.zeros((B, g, V), np.float32)
        self.tok = np.zeros((B, g), np.int32)
        self.u = np.zeros((B, g + 1), np.float32)
        self.acc = np.zeros(B, np.int32)
        self.out = np.zeros((B, g + 1), np.int32)
        self.ws = np.zeros(1 << 16, np.uint8)
        self.ws_aligned = self.ws[(-self.ws.ctypes.data) % 256:]


def p(a):
    return ct.c_void_p(a.ctypes.data) if a is not None else None


def chain_call(lib, h, **over):
    args = dict(target=p(h.t), draft=p(h.d), dtype=0, tok=p(h.tok), u=p(h.u), B=h.B, g=h.g, V=h.V,
                T=1.0,
                acc=p(h.acc), out=p(h.out), dist=None, ws=p(h.ws_aligned), wsb=16, stream=None)
    args.update(over)
    return lib.spec_verify_chain(args["target"], args["draft"], args["dtype"], args["tok"],
                                 args["u"], args["B"], args["g"], args["V"], args["T"],
                                 args["acc"], args["out"], args["dist"], args["ws"], args["wsb"],
                                 args["stream"])


def test_chain_host_errors(lib):
    c = header_constants()
    B, g, V = 2, 3, 64
    h = HostBufs(B, g, V)
    assert chain_call(lib, h, target=None) == c["SV_ERR_NULL"]
    assert chain_call(lib, h, tok=None) == c["SV_ERR_NULL"]
    assert chain_call(lib, h, ws=None) == c["SV_ERR_NULL"]
    assert chain_call(lib, h, B=0) == c["SV_ERR_SHAPE"]
    assert chain_call(lib, h, g=256) == c["SV_ERR_SHAPE"]
    assert chain_call(lib, h, V=0) == c["SV_ERR_SHAPE"]
    assert chain_call(lib, h, dtype=3) == c["SV_ERR_DTYPE"]
    for T in (0.0, -1.0, float("nan"), float("inf"), 1e-9, 1e9):
        assert chain_call(lib, h, T=T) == c["SV_ERR_TEMPERATURE"], T
    mis = ct.c_void_p(h.t.ctypes.data + 2)
    assert chain_call(lib, h, target=mis) == c["SV_ERR_ALIGN"]
    assert chain_call(lib, h, wsb=16) == c["SV_ERR_WORKSPACE"]
    ws_mis = ct.c_void_p(h.ws_aligned.ctypes.data + 8)
    assert chain_call(lib, h, ws=ws_mis, wsb=1 << 15) == c["SV_ERR_WORKSPACE"]
    # nothing was written
    assert (h.acc == 0).all() and (h.out == 0).all()


def pointmass_call(lib, h, **over):
    args = dict(target=p(h.t), dtype=0, tok=p(h.tok), u=p(h.u), B=h.B, g=h.g, V=h.V, T=1.0,
                acc=p(h.acc), out=p(h.out), dist=None, ws=p(h.ws_aligned), wsb=16, stream=None)
    args.update(over)
    return lib.spec_verify_chain_pointmass(args["target"], args["dtype"], args["tok"], args["u"],
                                           args["B"], args["g"], args["V"], args["T"],
                                           args["acc"], args["out"], args["dist"], args["ws"],
                                           args["wsb"], args["stream"])


def test_pointmass_host_errors(lib):
    import exact_draft_verification_amd as sv

    c = header_constants()
    B, g, V = 2, 3, 64
    h = HostBufs(B, g, V)
    assert pointmass_call(lib, h, target=None) == c["SV_ERR_NULL"]
    assert pointmass_call(lib, h, tok=None) == c["SV_ERR_NULL"]
    assert pointmass_call(lib, h, u=None) == c["SV_ERR_NULL"]
    assert pointmass_call(lib, h, acc=None) == c["SV_ERR_NULL"]
    assert pointmass_call(lib, h, B=0) == c["SV_ERR_SHAPE"]
    assert pointmass_call(lib, h, g=256) == c["SV_ERR_SHAPE"]
    assert pointmass_call(lib, h, V=0) == c["SV_ERR_SHAPE"]
    assert pointmass_call(lib, h, dtype=3) == c["SV_ERR_DTYPE"]
    for T in (0.0, float("nan"), float("inf"), 1e9):
        assert pointmass_call(lib, h, T=T) == c["SV_ERR_TEMPERATURE"], T
    assert pointmass_call(lib, h, target=ct.c_void_p(h.t.ctypes.data + 2)) == c["SV_ERR_ALIGN"]
    assert pointmass_call(lib, h, wsb=16) == c["SV_ERR_WORKSPACE"]
    assert (h.acc == 0).all() and (h.out == 0).all()
    # no draft rows: the point-mass workspace is never larger than the chain's
    for shape in [(64, 16, 151936, 1), (1, 16, 151936, 0), (3, 255, 1000, 0)]:
        assert 0 < sv.spec_verify_chain_pointmass_workspace_bytes(*shape) <= \
            sv.spec_verify_chain_workspace_bytes(*shape)
    assert sv.spec_verify_chain_pointmass_workspace_bytes(1, 256, 100, 0) == 0


def test_outcome_host_errors(lib):
    import exact_draft_verification_amd as sv

    c = header_constants()
    R, g, V = 2, 3, 64
    t = np.zeros((R, g + 1, V), np.float32)
    tok = np.zeros((R, g), np.int32)
    k = np.zeros((R, 4), np.int32)
    a = np.zeros((R, 4), np.int32)
    pp = np.zeros((R, 4), np.float64)
    hit = np.zeros(R, np.float64)
    ws = np.zeros(1 << 16, np.uint8)
    wsa = ws[(-ws.ctypes.data) % 256:]

    def call(**o):
        args = dict(t=p(t), dt=0, tok=p(tok), R=R, g=g, V=V, T=1.0, nc=4, k=p(k), a=p(a), pp=p(pp),
                    hit=p(hit), ws=p(wsa), wsb=16)
        args.update(o)
        return lib.spec_outcome_topk(args["t"], args["dt"], args["tok"], args["R"], args["g"],
                                     args["V"], args["T"], args["nc"], args["k"], args["a"],
                                     args["pp"], args["hit"], args["ws"], args["wsb"], None)

    assert call(t=None) == c["SV_ERR_NULL"]
    assert call(tok=None) == c["SV_ERR_NULL"]
    assert call(hit=None) == c["SV_ERR_NULL"]
    assert call(R=0) == c["SV_ERR_SHAPE"]
    assert call(g=256) == c["SV_ERR_SHAPE"]
    assert call(nc=0) == c["SV_ERR_SHAPE"]
    assert call(nc=c["SV_MAX_CACHE"] + 1) == c["SV_ERR_SHAPE"]
    assert call(dt=2) == c["SV_ERR_DTYPE"]
    assert call(T=0.0) == c["SV_ERR_TEMPERATURE"]
    assert call(t=ct.c_void_p(t.ctypes.data + 2)) == c["SV_ERR_ALIGN"]
    assert call(wsb=16) == c["SV_ERR_WORKSPACE"]
    assert (k == 0).all() and (hit == 0).all()
    assert sv.spec_outcome_topk_workspace_bytes(32, 16, 151936, 1, 8) > 0
    assert sv.spec_outcome_topk_workspace_bytes(32, 16, 151936, 1, 17) == 0


def test_cache_lookup_host_errors(lib):
    c = header_constants()
    R, g, nc = 3, 4, 8
    acc = np.zeros(R, np.int32)
    out = np.zeros((R, g + 1), np.int32)
    ck = np.zeros((R, nc), np.int32)
    ca = np.zeros((R, nc), np.int32)
    slot = np.full(R, 7, np.int32)

    def call(**o):
        args = dict(acc=p(acc), out=p(out), R=R, g=g, ck=p(ck), ca=p(ca), nc=nc, slot=p(slot))
        args.update(o)
        return lib.spec_cache_lookup(args["acc"], args["out"], args["R"], args["g"], args["ck"],
                                     args["ca"], args["nc"], args["slot"], None)

    assert call(acc=None) == c["SV_ERR_NULL"]
    assert call(ca=None) == c["SV_ERR_NULL"]
    assert call(slot=None) == c["SV_ERR_NULL"]
    assert call(R=0) == c["SV_ERR_SHAPE"]
    assert call(g=0) == c["SV_ERR_SHAPE"]
    assert call(g=c["SV_MAX_GAMMA"] + 1) == c["SV_ERR_SHAPE"]
    assert call(nc=0) == c["SV_ERR_SHAPE"]
    assert call(nc=c["SV_MAX_CACHE"] + 1) == c["SV_ERR_SHAPE"]
    assert call(out=ct.c_void_p(out.ctypes.data + 2)) == c["SV_ERR_ALIGN"]
    assert (slot == 7).all()  # nothing was written


def test_tree_build_host_errors(lib):
    import exact_draft_verification_amd as sv

    c = header_constants()
    R, M, V, W, N, nb = 2, 5, 64, 2, 2, 7
    z = np.zeros((R, M, V), np.float32)
    par = np.zeros((R, nb), np.int32)
    tok = np.zeros((R, nb), np.int32)
    row = np.zeros((R, nb), np.int32)
    sc = np.zeros((R, nb), np.float64)
    n = np.full(R, 5, np.int32)
    ws = np.zeros(1 << 16, np.uint8)
    wsa = ws[(-ws.ctypes.data) % 256:]

    def call(**o):
        args = dict(z=p(z), dt=0, cr=None, R=R, M=M, V=V, T=1.0, W=W, N=N, nb=nb, par=p(par),
                    tok=p(tok), row=p(row), sc=p(sc), n=p(n), ws=p(wsa), wsb=16)
        args.update(o)
        return lib.spec_tree_build(args["z"], args["dt"], args["cr"], args["R"], args["M"],
                                   args["V"], args["T"], args["W"], args["N"], args["nb"],
                                   args["par"], args["tok"], args["row"], args["sc"], args["n"],
                                   args["ws"], args["wsb"], None)

    assert call(z=None) == c["SV_ERR_NULL"]
    assert call(n=None) == c["SV_ERR_NULL"]
    assert call(R=0) == c["SV_ERR_SHAPE"]
    assert call(W=0) == c["SV_ERR_SHAPE"]
    assert call(W=c["SV_MAX_TREE_WIDTH"] + 1) == c["SV_ERR_SHAPE"]
    assert call(N=0) == c["SV_ERR_SHAPE"]
    assert call(nb=0) == c["SV_ERR_SHAPE"]
    assert call(nb=c["SV_MAX_TREE_NODES"] + 1) == c["SV_ERR_SHAPE"]
    assert call(M=c["SV_MAX_TREE_SLOTS"] // W + 1) == c["SV_ERR_SHAPE"]
    assert call(dt=2) == c["SV_ERR_DTYPE"]
    assert call(T=float("nan")) == c["SV_ERR_TEMPERATURE"]
    assert call(sc=ct.c_void_p(sc.ctypes.data + 4)) == c["SV_ERR_ALIGN"]
    assert call(wsb=16) == c["SV_ERR_WORKSPACE"]
    assert (n == 5).all()
    assert sv.spec_tree_build_workspace_bytes(32, 85, 151936, 1, 4, 4, 64) > 0
    assert sv.spec_tree_build_workspace_bytes(32, 85, 151936, 1, 17, 4, 64) == 0


def test_tree_stochastic_host_errors(lib):
    import exact_draft_verification_amd as sv

    c = header_constants()
    B, n, V = 2, 5, 64
    t = np.zeros((B, n, V), np.uint16)
    par = np.zeros((B, n), np.int32)
    tok = np.zeros((B, n), np.int32)
    u = np.zeros((B, n), np.float32)
    acc = np.full(B, 9, np.int32)
    node = np.zeros(B, np.int32)
    out = np.zeros((B, n), np.int32)
    ws = np.zeros(1 << 16, np.uint8)
    wsa = ws[(-ws.ctypes.data) % 256:]

    def call(**o):
        args = dict(t=p(t), d=p(t), dt=1, par=p(par), tok=p(tok), u=p(u), B=B, n=n, V=V, T=1.0,
                    acc=p(acc), node=p(node), out=p(out), ws=p(wsa), wsb=16)
        args.update(o)
        return lib.spec_verify_tree_stochastic(args["t"], args["d"], args["dt"], args["par"],
                                               args["tok"], args["u"], args["B"], args["n"],
                                               args["V"], args["T"], args["acc"], args["node"],
                                               args["out"], None, args["ws"], args["wsb"], None)

    assert call(d=None) == c["SV_ERR_NULL"]
    assert call(u=None) == c["SV_ERR_NULL"]
    assert call(node=None) == c["SV_ERR_NULL"]
    assert call(B=0) == c["SV_ERR_SHAPE"]
    assert call(n=0) == c["SV_ERR_SHAPE"]
    assert call(n=c["SV_MAX_TREE_NODES"] + 1) == c["SV_ERR_SHAPE"]
    assert call(dt=5) == c["SV_ERR_DTYPE"]
    assert call(T=-1.0) == c["SV_ERR_TEMPERATURE"]
    assert call(d=ct.c_void_p(t.ctypes.data + 1)) == c["SV_ERR_ALIGN"]
    assert call(wsb=16) == c["SV_ERR_WORKSPACE"]
    assert (acc == 9).all()
    assert sv.spec_verify_tree_stochastic_workspace_bytes(64, 64, 151936, 1) > 0
    assert sv.spec_verify_tree_stochastic_workspace_bytes(64, 1025, 151936, 1) == 0


def test_tree_host_errors(lib):
    c = header_constants()
    B, n, V = 2, 5, 64
    t = np.zeros((B, n, V), np.uint16)
    par = np.zeros((B, n), np.int32)
    tok = np.zeros((B, n), np.int32)
    acc = np.zeros(B, np.int32)
    node = np.zeros(B, np.int32)
    out = np.zeros((B, n), np.int32)
    ws = np.zeros(4096, np.uint8)
    wsa = ws[(-ws.ctypes.data) % 256:]

    def call(**o):
        a = dict(t=p(t), dt=1, par=p(par), tok=p(tok), B=B, n=n, V=V, acc=p(acc), node=p(node),
                 out=p(out), ws=p(wsa), wsb=16)
        a.update(o)
        return lib.spec_verify_tree_greedy(a["t"], a["dt"], a["par"], a["tok"], a["B"], a["n"],
                                           a["V"], a["acc"], a["node"], a["out"], a["ws"],
                                           a["wsb"], None)

    assert call(par=None) == c["SV_ERR_NULL"]
    assert call(node=None) == c["SV_ERR_NULL"]
    assert call(n=0) == c["SV_ERR_SHAPE"]
    assert call(n=1025) == c["SV_ERR_SHAPE"]
    assert call(dt=5) == c["SV_ERR_DTYPE"]
    assert call(t=ct.c_void_p(t.ctypes.data + 1)) == c["SV_ERR_ALIGN"]
    assert call(wsb=8) == c["SV_ERR_WORKSPACE"]
    assert (acc == 0).all() and (out == 0).all()


def test_binding_rejects_cpu_tensors():
    import torch

    import exact_draft_verification_amd as sv

    t = torch.zeros(1, 2, 8)
    with pytest.raises(ValueError):
        sv.spec_verify_chain(t, torch.zeros(1, 1, 8), torch.zeros(1, 1, dtype=torch.int32),
                             torch.zeros(1, 2), 1.0)


def test_product_path_has_no_oracle_or_cpu_fallback():
    """The package never imports or links the oracle, and does not fall back
    when its library is missing."""
    pkg = os.path.join(ROOT, "exact_draft_verification_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in src.lower(), f
    import exact_draft_verification_amd as sv

    saved = sv._lib, sv._LIB_PATH
    try:
        sv._lib, sv._LIB_PATH = None, os.path.join(ROOT, "does-not-exist.so")
        with pytest.raises(RuntimeError):
            sv.load_library()
    finally:
        sv._lib, sv._LIB_PATH = saved


def test_noalloc_host_errors():
    """spec_verify_chain_noalloc checks its arguments, and its scratch limit,
    before touching any device (so these run without a GPU)."""
    import exact_draft_verification_amd as sv

    lib = _load()
    c = header_constants()
    assert c["SV_NOALLOC_SCRATCH_BYTES"] == sv.SV_NOALLOC_SCRATCH_BYTES
    h = HostBufs(2, 3, 64)

    def call(**over):
        args = dict(target=p(h.t), draft=p(h.d), dtype=0, tok=p(h.tok), u=p(h.u), B=h.B, g=h.g,
                    V=h.V, T=1.0, acc=p(h.acc), out=p(h.out), dist=None, stream=None)
        args.update(over)
        return lib.spec_verify_chain_noalloc(args["target"], args["draft"], args["dtype"],
                                             args["tok"], args["u"], args["B"], args["g"],
                                             args["V"], args["T"], args["acc"], args["out"],
                                             args["dist"], args["stream"])

    assert call(target=None) == c["SV_ERR_NULL"]
    assert call(draft=None) == c["SV_ERR_NULL"]
    assert call(B=0) == c["SV_ERR_SHAPE"]
    assert call(dtype=5) == c["SV_ERR_DTYPE"]
    assert call(T=0.0) == c["SV_ERR_TEMPERATURE"]
    assert call(target=ct.c_void_p(h.t.ctypes.data + 2)) == c["SV_ERR_ALIGN"]
    # 8192 blocks of gamma 16 over V = 151936 need about 25 MB of scratch
    assert sv.spec_verify_chain_workspace_bytes(8192, 16, 151936, 1) > c["SV_NOALLOC_SCRATCH_BYTES"]
    assert call(B=8192, g=16, V=151936, dtype=1) == c["SV_ERR_SCRATCH"]
    assert (h.acc == 0).all() and (h.out == 0).all()
