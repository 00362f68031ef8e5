"""CPU tests of the C ABI boundary (no GPU needed: nothing here launches a kernel).

* libwmtp.so loads and exports every function include/wmtp.h declares;
* argument checks return the documented status codes before any launch
  (fake but aligned pointers are used only where a check fails first);
* the split planner's answers are consistent;
* the oracle and the HIP path do not import each other, and the product path
  has no fallback when the library is missing.
"""

import ast
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wmtp.h")

lib_mod = pytest.importorskip("long_context_decode_attention_amd")

OK, INVALID, UNSUPPORTED, WORKSPACE, HIPERR = 0, 1, 2, 3, 4
FAKE = 0x10000          # 16-byte aligned, never dereferenced: every call below fails a check first


def _lib():
    if not os.path.exists(lib_mod.LIB_PATH):
        pytest.skip("libwmtp.so not built")
    return lib_mod.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:wmtp_status|int|size_t|const char\*)\s+(wmtp_\w+)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_the_five_calls():
    names = declared_functions()
    for n in ("wmtp_draft_attn_full", "wmtp_draft_attn_window", "wmtp_ring_append",
              "wmtp_verify_attn", "wmtp_split_combine"):
        assert n in names
    assert set(names) == set(lib_mod.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for n in declared_functions():
        assert hasattr(lib, n), n
    # and with C linkage (unmangled) in the dynamic symbol table
    data = open(lib_mod.LIB_PATH, "rb").read()
    for n in declared_functions():
        assert n.encode() + b"\x00" in data, n


def test_status_strings():
    _lib()
    assert lib_mod.status_string(OK) == "ok"
    assert lib_mod.status_string(WORKSPACE) == "workspace missing or too small"
    assert lib_mod.status_string(99) == "unknown status"


def _full(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, sl=FAKE, B=1, Hq=32, Hkv=2, D=256, num_pages=16,
             max_pages=16, max_seq_len=1024, scale=1.0, o=FAKE, lse=None, ws=None, ws_bytes=0,
             num_splits=0, flags=0)
    a.update(kw)
    P = ctypes.c_void_p
    return lib.wmtp_draft_attn_full(P(a["q"]), P(a["k"]), P(a["v"]), P(a["bt"]), P(a["sl"]), a["B"],
                                    a["Hq"], a["Hkv"], a["D"], a["num_pages"], a["max_pages"],
                                    a["max_seq_len"], a["scale"], P(a["o"]), P(a["lse"]),
                                    P(a["ws"]), a["ws_bytes"], a["num_splits"], a["flags"], None)


def test_draft_full_argument_checks():
    lib = _lib()
    assert _full(lib, q=None) == INVALID
    assert _full(lib, o=None) == INVALID
    assert _full(lib, D=100) == UNSUPPORTED
    assert _full(lib, D=512) == UNSUPPORTED
    assert _full(lib, Hq=33) == INVALID                  # not a multiple of Hkv
    assert _full(lib, B=0) == INVALID
    assert _full(lib, num_pages=0) == INVALID
    assert _full(lib, scale=float("inf")) == INVALID
    assert _full(lib, scale=float("nan")) == INVALID
    assert _full(lib, scale=0.0) == INVALID
    assert _full(lib, scale=-0.5) == INVALID
    assert _full(lib, flags=8) == INVALID
    assert _full(lib, q=FAKE + 2) == INVALID              # misaligned
    # 1024 keys in 16 splits need a workspace: none given
    assert _full(lib, num_splits=16) == WORKSPACE
    assert _full(lib, num_splits=16, ws=FAKE, ws_bytes=64) == WORKSPACE


def test_verify_and_window_argument_checks():
    lib = _lib()
    P = ctypes.c_void_p
    # 8 queries x G = 64 is 512 rows: more than a kv head's 256-row limit
    st = lib.wmtp_verify_attn(P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), 1, 8, 128, 2, 128, 16, 16,
                              1024, 1.0, P(FAKE), None, None, 0, 0, 0, None)
    assert st == UNSUPPORTED
    st = lib.wmtp_verify_attn(P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), 1, 0, 32, 2, 128, 16, 16,
                              1024, 1.0, P(FAKE), None, None, 0, 0, 0, None)
    assert st == INVALID

    def win(**kw):
        a = dict(B=1, Hq=32, Hkv=2, D=256, C=4096, ns=4, nr=4092, pos=FAKE)
        a.update(kw)
        return lib.wmtp_draft_attn_window(P(FAKE), P(FAKE), P(FAKE), P(a["pos"]), P(FAKE), a["B"],
                                          a["Hq"], a["Hkv"], a["D"], a["C"], a["ns"], a["nr"], 1.0,
                                          P(FAKE), None, None, 0, 0, 0, None)
    assert win(C=4100) == INVALID                      # not a multiple of 64
    assert win(ns=4096) == INVALID                     # sink fills the ring
    assert win(nr=4093) == INVALID                     # window larger than the ring
    assert win(nr=0) == INVALID
    assert win(pos=None) == INVALID
    assert win(D=96) == UNSUPPORTED

    def tree(**kw):
        a = dict(mask=FAKE, n_q=8)
        a.update(kw)
        return lib.wmtp_verify_attn_tree(P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(a["mask"]),
                                         1, a["n_q"], 32, 2, 256, 16, 16, 1024, 1.0, P(FAKE), None,
                                         None, 0, 0, 0, None)
    assert tree(mask=None) == INVALID
    assert tree(mask=FAKE + 4) == INVALID             # misaligned
    assert tree(n_q=65) == INVALID                    # more proposals than mask bits

    def f8(**kw):
        a = dict(Hq=32, Hkv=2, ks=1.0, vs=1.0)
        a.update(kw)
        return lib.wmtp_draft_attn_full_fp8(P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), 1, a["Hq"],
                                            a["Hkv"], 256, 16, 16, 1024, a["ks"], a["vs"], 1.0,
                                            P(FAKE), None, None, 0, 0, 0, None)
    assert f8(ks=0.0) == INVALID
    assert f8(vs=float("nan")) == INVALID
    assert f8(Hq=128) == UNSUPPORTED                  # 64 query rows per kv head
    st = lib.wmtp_paged_append_fp8(P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), 1, 4, 2,
                                   256, 16, 16, -1.0, 1.0, None)
    assert st == INVALID

    def v8(**kw):
        a = dict(n_q=8, Hq=32, Hkv=2, D=256, ks=1.0, vs=1.0, k=FAKE, ws=None, wsb=0)
        a.update(kw)
        return lib.wmtp_verify_attn_fp8(P(FAKE), P(a["k"]), P(FAKE), P(FAKE), P(FAKE), 1, a["n_q"],
                                        a["Hq"], a["Hkv"], a["D"], 16, 16, 1024, a["ks"], a["vs"],
                                        1.0, P(FAKE), None, P(a["ws"]), a["wsb"], 0, 0, None)
    assert v8(ks=-1.0) == INVALID
    assert v8(vs=float("inf")) == INVALID
    assert v8(k=None) == INVALID
    assert v8(k=FAKE + 8) == INVALID                  # misaligned cache
    assert v8(D=96) == UNSUPPORTED
    assert v8(n_q=17) == UNSUPPORTED                  # 272 query rows per kv head
    assert v8() == WORKSPACE                          # 128 rows: the shared kernel, partials
    assert v8(n_q=2, Hq=16) == WORKSPACE              # 16 rows: the split kernel, partials


def test_paged_window_argument_checks():
    lib = _lib()
    P = ctypes.c_void_p

    def pw(**kw):
        a = dict(B=1, Hq=32, Hkv=2, D=256, ns=4, nr=4092, q=FAKE, ws=None, ws_bytes=0, splits=0)
        a.update(kw)
        return lib.wmtp_draft_attn_window_paged(P(a["q"]), P(FAKE), P(FAKE), P(FAKE), P(FAKE),
                                                a["B"], a["Hq"], a["Hkv"], a["D"], 16, 16, 1024,
                                                a["ns"], a["nr"], 1.0, P(FAKE), None, P(a["ws"]),
                                                a["ws_bytes"], a["splits"], 0, None)
    assert pw(nr=0) == INVALID
    assert pw(ns=-1) == INVALID
    assert pw(q=None) == INVALID
    assert pw(D=96) == UNSUPPORTED
    assert pw(Hq=128, Hkv=2) == UNSUPPORTED              # 64 query rows per kv head
    # 1024 keys in 16 splits need a workspace: none given
    assert pw(splits=16) == WORKSPACE


def test_append_and_combine_argument_checks():
    lib = _lib()
    P = ctypes.c_void_p
    ra = lambda **kw: lib.wmtp_ring_append(  # noqa: E731
        P(kw.get("k", FAKE)), P(FAKE), P(FAKE), P(FAKE), P(kw.get("kn", FAKE)), P(FAKE),
        kw.get("B", 1), kw.get("n", 1), 2, kw.get("D", 128), kw.get("C", 1024), kw.get("ns", 4), None)
    assert ra(C=1000) == INVALID
    assert ra(ns=1024) == INVALID
    assert ra(n=-1) == INVALID
    assert ra(k=None) == INVALID
    assert ra(kn=None) == INVALID
    assert ra(D=100) == UNSUPPORTED
    assert ra(n=0) == OK                               # nothing to append: no launch
    pa = lambda **kw: lib.wmtp_paged_append(  # noqa: E731
        P(FAKE), P(FAKE), P(kw.get("bt", FAKE)), P(FAKE), P(FAKE), P(FAKE), 1, kw.get("n", 1), 2, 128,
        kw.get("np", 4), 4, None)
    assert pa(bt=None) == INVALID
    assert pa(np=0) == INVALID
    assert pa(n=0) == OK
    sc = lambda **kw: lib.wmtp_split_combine(  # noqa: E731
        P(FAKE), P(FAKE), kw.get("n_parts", 8), P(kw.get("indptr")), kw.get("spg", 4), 1, 2, 4, 1,
        kw.get("D", 128), P(kw.get("o", FAKE)), None, None)
    assert sc(spg=5) == INVALID                        # 2 groups x 5 splits > 8 partials
    assert sc(D=100) == INVALID
    assert sc(o=None) == INVALID


def test_plan_and_workspace_consistency():
    _lib()
    L = 1 << 20
    # native draft at 1M: several splits, each partial R x D floats plus its lse
    n = lib_mod.plan_splits(1, 32, 2, 256, 1, L)
    assert n > 1
    ws = lib_mod.workspace_bytes(1, 32, 2, 256, 1, L)
    po = 2 * n * 16 * 256 * 4
    assert ws == (po + 255) // 256 * 256 + 2 * n * 16 * 4
    # a requested split count is an upper bound; one split writes directly
    assert lib_mod.plan_splits(1, 32, 2, 256, 1, L, 7) <= 7
    assert lib_mod.workspace_bytes(1, 32, 2, 256, 1, 100, 1) == 0
    assert lib_mod.workspace_bytes(1, 32, 2, 256, 1, 100, 1, partials_only=True) > 0
    # the ring call plans with the ring's capacity
    assert lib_mod.plan_splits(1, 32, 2, 256, 1, 4096, ring=True) >= 1
    # the truncated paged index plans for its window (4 + 4092 keys: at most 130 tiles
    # per sequence), whatever the context; its workspace covers every context
    wp = lib_mod.workspace_bytes(1, 32, 2, 256, 1, 4096, paged_window=True)
    assert wp > 0
    assert lib_mod.plan_splits(1, 32, 2, 256, 1, 4096, paged_window=True) <= 130 // 4 + 1
    for keys in (1, 100, 4096, 4200, L):
        # the call plans with min(window bound, max_keys) keys: never more splits
        assert lib_mod.workspace_bytes(1, 32, 2, 256, 1, min(keys, 32 * 130)) <= wp
    with pytest.raises(lib_mod.WmtpError):
        lib_mod.plan_splits(1, 32, 3, 256, 1, L)


def test_fused_step_argument_checks_and_plan():
    """wmtp_draft_step_window: host checks (nothing launched) and its plan: the
    windowed draft's ring splits plus one partial per group for the new positions."""
    lib = _lib()
    P = ctypes.c_void_p

    def step(**kw):
        a = dict(B=1, n_new=1, Hq=32, Hkv=2, D=256, C=4096, ns=4, nr=4092, ws=None, wsb=0,
                 scale=1.0, o=FAKE, kn=FAKE)
        a.update(kw)
        return lib.wmtp_draft_step_window(P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(a["kn"]),
                                          P(FAKE), a["B"], a["n_new"], a["Hq"], a["Hkv"], a["D"],
                                          a["C"], a["ns"], a["nr"], a["scale"], P(a["o"]), None,
                                          P(a["ws"]) if a["ws"] else None, a["wsb"], 0, None)
    assert step(n_new=0) == INVALID
    assert step(n_new=33) == INVALID
    assert step(kn=None) == INVALID
    assert step(kn=FAKE + 8) == INVALID                # misaligned new K
    assert step(o=None) == INVALID
    assert step(scale=0.0) == INVALID
    assert step(C=4100) == INVALID
    assert step(nr=4093) == INVALID
    assert step(Hq=1024) == UNSUPPORTED                # 512 query rows per kv head
    assert step(Hq=128) == WORKSPACE                   # 64 rows: two row groups
    assert step(D=96) == UNSUPPORTED
    assert step() == WORKSPACE                         # no workspace
    need = lib_mod.step_workspace_bytes(1, 32, 2, 256, 4096)
    assert step(ws=FAKE, wsb=need - 1) == WORKSPACE
    n = lib_mod.step_splits(1, 32, 2, 256, 4096)
    assert n == lib_mod.plan_splits(1, 32, 2, 256, 1, 4096, ring=True)
    # 2 groups x 128 tiles: the four-tile minimum per split
    assert n == 32
    # 32 groups: 8 workgroups per group, 16 tiles per split
    assert lib_mod.step_splits(8, 32, 4, 128, 4096) == 8
    parts = 2 * (n + 1)
    assert need == (parts * 16 * 256 * 4 + 255) // 256 * 256 + parts * 16 * 4
    assert lib_mod.step_splits(1, 32, 2, 256, 4096, 1) == 1
    assert lib_mod.step_splits(1, 32, 2, 256, 4096, 1000) == 4096 // 32


def test_fused_context_step_argument_checks_and_plan():
    """wmtp_draft_context_step_window: the slack and row checks on top of the fused
    step's, and a plan of n_q * G rows in row groups of 32."""
    lib = _lib()
    P = ctypes.c_void_p

    def step(**kw):
        a = dict(B=1, n_new=8, n_q=8, Hq=32, Hkv=2, C=4160, ns=4, nr=4092, ws=None, wsb=0)
        a.update(kw)
        return lib.wmtp_draft_context_step_window(
            P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), a["B"], a["n_new"],
            a["n_q"], a["Hq"], a["Hkv"], 256, a["C"], a["ns"], a["nr"], 1.0, P(FAKE), None,
            P(a["ws"]) if a["ws"] else None, a["wsb"], 0, None)
    assert step(n_q=0) == INVALID
    assert step(n_q=66, Hq=2) == INVALID               # slack 64 < n_q - 1
    assert step(n_q=65, Hq=2) == WORKSPACE             # slack 64 = n_q - 1
    assert step(n_q=8, C=4096) == INVALID              # no slack at all
    assert step(n_q=17) == UNSUPPORTED                 # 17 * 16 rows per kv head
    assert step(n_new=33) == INVALID
    assert step() == WORKSPACE
    need = lib_mod.step_workspace_bytes(1, 32, 2, 256, 4160, 0, 8)
    assert step(ws=FAKE, wsb=need - 1) == WORKSPACE
    n = lib_mod.step_splits(1, 32, 2, 256, 4160, 0, 8)
    parts = 2 * (n + 1)
    assert need == (parts * 128 * 256 * 4 + 255) // 256 * 256 + parts * 128 * 4
    # n_q = 1 plans as the single-query step
    assert lib_mod.step_splits(1, 32, 2, 256, 4160, 0, 1) == lib_mod.step_splits(1, 32, 2, 256, 4160)
    # row groups share the workgroup target: four groups of 32 rows, fewer splits
    assert n <= lib_mod.step_splits(1, 32, 2, 256, 4160)


def test_plan_rounds_for_several_long_sequences():
    """Paged calls over several sequences of 64K keys or more plan four workgroups per
    CU (the lengths are on the device); one sequence, short key ranges and rings one."""
    _lib()
    one = lib_mod.plan_splits(1, 32, 4, 128, 1, 1 << 20)        # 4 groups x 64 splits = 256
    eight = lib_mod.plan_splits(8, 32, 4, 128, 1, 1 << 20)      # 32 groups x 32 splits = 1024
    assert one * 4 == 256 and eight * 32 == 1024
    assert lib_mod.plan_splits(8, 32, 4, 128, 1, 60000) * 32 <= 256   # under 64K keys: one round
    assert lib_mod.plan_splits(8, 32, 4, 128, 1, 4096, ring=True) * 32 <= 256
    assert lib_mod.plan_splits(8, 32, 4, 128, 1, 4096, paged_window=True) * 32 <= 256
    # verify rows go through the same rule
    assert lib_mod.plan_splits(8, 32, 4, 128, 4, 1 << 20) * 32 == 1024


def test_plan_fp8_head_dim_128_two_per_cu():
    """The fp8 native pass at D = 128 over 64K keys or more plans twice the
    workgroups of the bf16 pass (two fit on a CU); other shapes plan the same."""
    _lib()
    ps = lib_mod.plan_splits
    assert ps(1, 32, 4, 128, 1, 131072, fp8=True) == 2 * ps(1, 32, 4, 128, 1, 131072)
    assert ps(8, 32, 4, 128, 1, 1 << 20, fp8=True) == 2 * ps(8, 32, 4, 128, 1, 1 << 20)
    assert ps(1, 32, 2, 256, 1, 1 << 20, fp8=True) == ps(1, 32, 2, 256, 1, 1 << 20)
    assert ps(1, 32, 4, 128, 1, 60000, fp8=True) == ps(1, 32, 4, 128, 1, 60000)
    assert ps(1, 32, 4, 128, 1, 131072, 7, fp8=True) == 7          # explicit split count
    wb = lib_mod.workspace_bytes
    assert wb(1, 32, 4, 128, 1, 131072, fp8=True) > wb(1, 32, 4, 128, 1, 131072)


def _imports(path):
    names = set()
    for dirpath, _, files in os.walk(path):
        for f in files:
            if f.endswith(".py"):
                tree = ast.parse(open(os.path.join(dirpath, f)).read())
                for node in ast.walk(tree):
                    if isinstance(node, ast.Import):
                        names.update(a.name.split(".")[0] for a in node.names)
                    elif isinstance(node, ast.ImportFrom) and node.module and node.level == 0:
                        names.add(node.module.split(".")[0])
    return names


def test_oracle_and_hip_path_are_independent():
    assert "long_context_decode_attention_amd" not in _imports(os.path.join(ROOT, "oracle"))
    assert "workloads" not in _imports(os.path.join(ROOT, "oracle"))
    product = _imports(os.path.join(ROOT, "long_context_decode_attention_amd"))
    assert "oracle" not in product and "workloads" not in product
    assert "long_context_decode_attention_amd" not in _imports(os.path.join(ROOT, "workloads"))
    assert "oracle" not in _imports(os.path.join(ROOT, "workloads"))


def test_missing_library_fails_loudly(tmp_path):
    saved = lib_mod._lib
    lib_mod._lib = None
    try:
        with pytest.raises(RuntimeError, match="not built"):
            lib_mod.load(str(tmp_path / "libwmtp.so"))
    finally:
        lib_mod._lib = saved


def test_cache_and_ring_shapes():
    """The binding's tensor shapes hold the tiled layout of include/wmtp.h: a page
    of one kv head is 64 * D elements in K and in V, and a ring reports its own
    B, Hkv and D back."""
    torch = pytest.importorskip("torch")
    for D in (64, 128, 256):
        k, v = lib_mod.new_paged_cache(3, 2, D, device="cpu")
        assert k.numel() == v.numel() == 3 * 2 * 64 * D
        assert k.dtype == v.dtype == torch.bfloat16
        r = lib_mod.new_ring(2, 128, 2, D, 4, 100, device="cpu")
        assert (r.B, r.Hkv, r.D) == (2, 2, D)
        assert r.k.shape[0] == 2 * 128 // 64
        assert int(r.pos.min()) == -1 and int(r.T.sum()) == 0


def test_planner_sweep_extremes():
    """The planning queries over a grid that includes extreme and invalid sizes:
    each answers -1 / 0 or a consistent plan, and nothing in the host arithmetic
    overflows (run under the host sanitizers by test_abi_hostsan.py, where a
    signed overflow or an out-of-range shift aborts the process)."""
    lib = _lib()
    big = 2 ** 31 - 1
    calls = (0, 1, 2, 3, 4, 7, -1)
    Bs = (1, 8, 4096, 65535, 65536, big, 0, -1)
    heads = ((32, 2), (64, 2), (32, 4), (1, 1), (256, 1), (512, 2), (big, 1), (32, 0), (0, 1), (33, 2))
    Ds = (64, 128, 256, 96, 0, -64)
    nqs = (1, 8, 16, 256, 0, big)
    keys = (0, 1, 31, 32, 4096, 1048576, 2 ** 30, big, -1)
    splits = (0, 1, 7, 1000, big, -1)
    n = 0
    for call in calls:
        for B in Bs:
            for Hq, Hkv in heads:
                for D in Ds:
                    for n_q in nqs:
                        for mk in keys:
                            for ns in splits[:3] if n_q != 1 else splits:
                                s = lib.wmtp_plan_splits(call, B, Hq, Hkv, D, n_q, mk, ns)
                                w = lib.wmtp_workspace_bytes(call, B, Hq, Hkv, D, n_q, mk, ns, 0)
                                n += 1
                                if s == -1:
                                    assert w == 0
                                    continue
                                assert s >= 1, (call, B, Hq, Hkv, D, n_q, mk, ns, s)
                                R = n_q * (Hq // Hkv)
                                parts = B * Hkv * (s + 1 if call == 3 else s)
                                # a plan with one split per group may write o directly (no workspace)
                                assert w == 0 and s == 1 or w >= parts * R * D * 4, \
                                    (call, B, Hq, Hkv, D, n_q, mk, ns, s, w)
    assert n > 10000
