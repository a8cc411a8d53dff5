"""The C ABI boundary, on the host only: the library loads without a GPU,
exports every function include/epl.h declares, and rejects bad arguments
with EPL_EINVAL before it enqueues anything (no compute call is made)."""
import ctypes
import os
import re

import pytest

import permute_ep_layout_amd as epl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "epl.h")


@pytest.fixture(scope="module")
def lib():
    epl.ensure_built()
    return epl.load()


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(epl_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    decl = declared_functions()
    assert decl == sorted(epl.C_ENTRY_POINTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"libepl.so does not export {name}"


def test_no_oracle_in_the_product_path():
    """The product package and the HIP library never reference the oracle."""
    pkg = os.path.dirname(epl.__file__)
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "epl_oracle" not in text, f
    with open(epl.lib_path(), "rb") as fh:
        assert b"epl_oracle" not in fh.read()


def test_problem_struct_layout():
    assert ctypes.sizeof(epl.Problem) == 40
    assert epl.Problem.num_topk.offset == 8 and epl.Problem.expert_alignment.offset == 28
    assert epl.Problem.ranks_per_node.offset == 32 and epl.Problem.reserved.offset == 36


def P(**kw):
    base = dict(num_tokens=4096, num_topk=8, num_experts=256, num_ranks=32, hidden=7168,
                scale_cols=56)
    base.update(kw)
    return epl.Problem.make(**base)


@pytest.mark.parametrize("kw,ok", [
    ({}, True),
    (dict(scale_cols=0), True),
    (dict(num_tokens=0), True),
    (dict(num_tokens=-1), False),
    (dict(num_topk=0), False),
    (dict(num_topk=64), True),
    (dict(num_topk=65), False),
    (dict(num_experts=2048, num_ranks=2048), True),
    (dict(num_experts=2049, num_ranks=1), False),
    (dict(num_ranks=30), False),            # E % R != 0
    (dict(num_ranks=512), False),           # R > E
    (dict(hidden=7170, scale_cols=0), False),   # H % 8 != 0
    (dict(hidden=8, scale_cols=0), True),
    (dict(hidden=200, scale_cols=1), False),    # scales need H % 128 == 0
    (dict(scale_cols=55), False),               # S must be H/128
    (dict(num_tokens=(1 << 31) // 8, num_topk=8), False),   # T*K > INT32_MAX
    (dict(num_tokens=(1 << 31) // 8 - 1, num_topk=8), True),
])
def test_validate(lib, kw, ok):
    p = P(**kw)
    assert (epl.epl_validate(p) == epl.EPL_OK) == ok
    assert (epl.epl_workspace_bytes(p) > 0) == ok


@pytest.mark.parametrize("a,ok", [(0, True), (1, True), (2, True), (256, True), (65536, True),
                                  (65537, False), (-1, False)])
def test_expert_alignment_range(lib, a, ok):
    p = P(expert_alignment=a)
    assert (epl.epl_validate(p) == epl.EPL_OK) == ok


@pytest.mark.parametrize("G,ok,nodes", [(0, True, 0), (1, True, 32), (8, True, 4), (32, True, 0),
                                        (64, True, 0), (3, False, 0), (-1, False, 0)])
def test_ranks_per_node(lib, G, ok, nodes):
    """R = 32: G divides R for a multi-node problem; G >= R is one node."""
    p = P(ranks_per_node=G)
    assert (epl.epl_validate(p) == epl.EPL_OK) == ok
    if ok:
        assert p.num_nodes == nodes


def test_reserved_must_be_zero(lib):
    p = P()
    p.reserved = 1
    assert epl.epl_validate(p) == epl.EPL_EINVAL


def test_workspace_grows_with_node_columns(lib):
    assert epl.epl_workspace_bytes(P(ranks_per_node=1)) >= epl.epl_workspace_bytes(P())


@pytest.mark.parametrize("T,K,E,a,want", [
    (4096, 8, 256, 0, 4096 * 8),
    (4096, 8, 256, 1, 4096 * 8),
    (4096, 8, 256, 256, ((4096 * 8 + 256 * 255 + 255) // 256) * 256),
    (100, 3, 16, 7, ((300 + 16 * 6 + 6) // 7) * 7),
    (0, 4, 8, 16, 8 * 15 + 8),     # round_up(0 + 8*15, 16) = 128
])
def test_capacity_rows_is_the_aligned_bound(lib, T, K, E, a, want):
    p = P(num_tokens=T, num_topk=K, num_experts=E, num_ranks=E if E < 32 else 32, scale_cols=0,
          expert_alignment=a)
    assert epl.epl_capacity_rows(p) == want


def test_capacity_bound_must_fit_int32(lib):
    T = (1 << 31) // 8 - 1          # T*K fits ...
    assert epl.epl_validate(P(num_tokens=T)) == epl.EPL_OK
    # ... but not once 256 experts may each add up to 255 padding rows
    assert epl.epl_validate(P(num_tokens=T, expert_alignment=256)) == epl.EPL_EINVAL
    assert epl.epl_capacity_rows(P(num_tokens=T, expert_alignment=256)) == -1


def test_workspace_scales_with_problem(lib):
    small, big = epl.epl_workspace_bytes(P(num_tokens=64)), epl.epl_workspace_bytes(P())
    assert 0 < small < big
    assert epl.epl_workspace_bytes(P()) % 256 == 0
    # header + per-slot ranks at least
    assert epl.epl_workspace_bytes(P()) >= 256 + 4096 * 8 * 4


def test_entry_points_reject_bad_arguments_without_a_gpu(lib):
    """Each call returns EPL_EINVAL from its host checks (null / misaligned
    pointers, invalid problem); nothing reaches the HIP runtime."""
    p = P()
    pp = ctypes.byref(p)
    fake = 1 << 20            # an aligned, never dereferenced address
    odd = fake + 2            # misaligned
    assert lib.epl_layout(pp, None, None, None, None, None, None, None) == epl.EPL_EINVAL
    assert lib.epl_layout(pp, fake, fake, fake, None, fake, odd, None) == epl.EPL_EINVAL  # ws
    multi = P(ranks_per_node=8)                  # 4 nodes: the per-node output is required
    assert lib.epl_layout(ctypes.byref(multi), fake, fake, fake, None, fake, fake,
                          None) == epl.EPL_EINVAL
    assert lib.epl_layout(ctypes.byref(multi), fake, fake, fake, odd, fake, fake,
                          None) == epl.EPL_EINVAL
    assert lib.epl_scan(pp, fake, fake, None, None, None) == epl.EPL_EINVAL
    assert lib.epl_scan(pp, odd, fake, None, fake, None) == epl.EPL_EINVAL
    assert lib.epl_scatter(pp, fake, fake, fake, fake, fake, -1, fake, fake, fake, fake,
                           None) == epl.EPL_EINVAL                                  # capacity < 0
    assert lib.epl_scatter(pp, odd, fake, fake, fake, fake, 10, fake, fake, fake, fake,
                           None) == epl.EPL_EINVAL                                  # x misaligned
    assert lib.epl_scatter(pp, fake, None, fake, fake, fake, 10, fake, fake, fake, fake,
                           None) == epl.EPL_EINVAL                                  # scales missing
    assert lib.epl_dispatch(pp, fake, fake, fake, 10, fake, fake, None, None, fake, None, fake,
                            fake, fake, fake, fake, None) == epl.EPL_EINVAL         # in_rank null
    assert lib.epl_dispatch(ctypes.byref(multi), fake, fake, fake, 10, fake, fake, None, fake,
                            fake, None, fake, fake, fake, fake, fake,
                            None) == epl.EPL_EINVAL                                 # per-node null
    assert lib.epl_combine(pp, fake, 10, fake, fake, 7, fake, None, None) == epl.EPL_EINVAL
    assert lib.epl_combine(pp, fake, 10, fake, fake, 0, odd, None, None) == epl.EPL_EINVAL
    assert lib.epl_expert_scale(pp, fake, fake, 10, fake, None, None) == epl.EPL_EINVAL
    bad = P(num_ranks=3)
    assert lib.epl_dispatch(ctypes.byref(bad), fake, fake, fake, 10, fake, fake, None, fake, fake,
                            None, fake, fake, fake, fake, fake, None) == epl.EPL_EINVAL
    assert lib.epl_status(None, None) == epl.EPL_EINVAL
    assert lib.epl_total(odd, None) == epl.EPL_EINVAL


def test_fp8_entry_points_check_their_arguments(lib):
    fake = 1 << 20
    ok = P()                                     # H = 7168, S = 56
    bad_h = P(hidden=136, scale_cols=0)          # 136 % 16 != 0
    no_s = P(scale_cols=0)

    def scat(p, fmt, xs=fake, outs=fake):
        return lib.epl_scatter_fp8(ctypes.byref(p), fake, xs, fmt, fake, fake, fake, 10, fake,
                                   outs, fake, fake, None)
    assert scat(bad_h, epl.EPL_SCALE_NONE) == epl.EPL_EINVAL
    assert scat(ok, 7) == epl.EPL_EINVAL                          # unknown format
    assert scat(no_s, epl.EPL_SCALE_UE8M0) == epl.EPL_EINVAL      # scales without scale_cols
    assert scat(ok, epl.EPL_SCALE_F32, xs=None) == epl.EPL_EINVAL
    assert scat(ok, epl.EPL_SCALE_UE8M0, outs=fake + 2) == epl.EPL_EINVAL
    assert lib.epl_dispatch_fp8(ctypes.byref(bad_h), fake, fake, None, 0, 10, fake, fake, None,
                                fake, fake, None, fake, None, fake, fake, fake,
                                None) == epl.EPL_EINVAL


def test_strerror(lib):
    for code in (0, -1, -2, -3, -4):
        assert epl.epl_strerror(code)
    assert "unknown" in epl.epl_strerror(-99)


def test_python_binding_rejects_cpu_tensors(lib):
    torch = pytest.importorskip("torch")
    p = epl.Problem.make(4, 2, 8, 2, 16, 0)
    with pytest.raises(ValueError, match="GPU tensor"):
        epl.epl_layout(p, torch.zeros((4, 2), dtype=torch.int64), torch.zeros(8, dtype=torch.int32),
                       torch.zeros(2, dtype=torch.int32), None,
                       torch.zeros((4, 2), dtype=torch.uint8), torch.zeros(256, dtype=torch.uint8))
    with pytest.raises(TypeError, match="int64"):
        epl.epl_layout(p, torch.zeros((4, 2), dtype=torch.int32), None, None, None, None, None)


def test_ll_workspace_and_argument_checks(lib):
    fake = 1 << 20
    ok = P(num_tokens=4096)                       # H = 7168, S = 56
    assert epl.epl_ll_workspace_bytes(ok, 128) >= epl.epl_workspace_bytes(ok)
    assert epl.epl_ll_workspace_bytes(ok, 100) == 0          # 4096 % 100 != 0
    assert epl.epl_ll_workspace_bytes(ok, 0) == 0
    assert epl.epl_ll_workspace_bytes(P(scale_cols=0), 128) == 0    # scales are produced
    assert epl.epl_ll_workspace_bytes(P(expert_alignment=64), 128) == 0
    # a prime segment length still tiles: blocks of one token
    assert epl.epl_ll_workspace_bytes(P(num_tokens=127 * 3), 127) > 0

    def call(p, M=128, cap=4096, ws=fake, out=fake):
        return lib.epl_ll_dispatch(ctypes.byref(p), M, cap, fake, fake, out, fake, fake, fake,
                                   fake, fake, ws, None)
    assert call(ok, M=100) == epl.EPL_EINVAL
    assert call(ok, cap=-1) == epl.EPL_EINVAL
    assert call(ok, cap=(1 << 31) // 256) == epl.EPL_EINVAL     # E * cap > INT32_MAX
    assert call(ok, ws=fake + 64) == epl.EPL_EINVAL
    assert call(ok, out=fake + 8) == epl.EPL_EINVAL
    assert call(P(hidden=7168 + 64, scale_cols=0)) == epl.EPL_EINVAL


def test_small_division_by_multiply_high_is_exact():
    """The layout divides owner and node ids (< 2^16) by multiplying with
    ceil(2^32 / d) and keeping the high word; that equals n // d for every
    n, d < 2^16 used (d up to the 2048 experts per rank)."""
    import numpy as np
    n = np.arange(1 << 16, dtype=np.uint64)
    for d in range(2, 2049):
        magic = np.uint64(((1 << 32) + d - 1) // d)
        assert np.array_equal((n * magic) >> np.uint64(32), n // np.uint64(d)), d


class _RecordingLib:
    """Stands in for libepl.so in the workspace-size test: the host-only size
    queries go to the real library, every other entry point is recorded and
    must never be reached."""

    HOST_ONLY = ("epl_workspace_bytes", "epl_ll_workspace_bytes", "epl_strerror",
                 "epl_capacity_rows", "epl_validate")

    def __init__(self, real):
        self.real, self.calls = real, []

    def __getattr__(self, name):
        if name in self.HOST_ONLY:
            return getattr(self.real, name)

        def launch(*args):
            self.calls.append(name)
            return 0
        return launch


def test_wrappers_reject_an_undersized_workspace_before_any_call(lib, monkeypatch):
    """The C ABI cannot see the workspace's size, so every Python wrapper that
    takes one checks it against epl_workspace_bytes (or the 256-byte header
    for combine / expert_scale / status / total) before it calls the
    library: an undersized workspace raises and nothing is launched."""
    torch = pytest.importorskip("torch")
    rec = _RecordingLib(lib)
    monkeypatch.setattr(epl, "load", lambda: rec)
    monkeypatch.setattr(epl, "_need", lambda *a, **k: None)       # CPU tensors stand in
    monkeypatch.setattr(epl, "_stream", lambda *a, **k: 0)
    T, K, E, R, H, S = 64, 4, 16, 4, 128, 1
    p = epl.Problem.make(T, K, E, R, H, S)
    need = epl.epl_workspace_bytes(p)
    assert need > 256
    small = torch.empty(need - 1, dtype=torch.uint8)
    header_only = torch.empty(255, dtype=torch.uint8)
    t = torch.empty(1)
    total = None
    calls = {
        "epl_layout": lambda ws: epl.epl_layout(p, t, t, t, None, t, ws),
        "epl_scan": lambda ws: epl.epl_scan(p, t, t, total, ws),
        "epl_scatter": lambda ws: epl.epl_scatter(p, t, t, t, t, ws, T * K, t, t, t, t),
        "epl_dispatch": lambda ws: epl.epl_dispatch(p, t, t, t, T * K, t, t, None, t, t, total,
                                                    t, t, t, t, ws),
        "epl_scatter_fp8": lambda ws: epl.epl_scatter_fp8(p, t, t, epl.EPL_SCALE_F32, t, t, ws,
                                                          T * K, t, t, t, t),
        "epl_dispatch_fp8": lambda ws: epl.epl_dispatch_fp8(p, t, t, t, epl.EPL_SCALE_F32,
                                                            T * K, t, t, None, t, t, total, t,
                                                            t, t, t, ws),
    }
    for name, call in calls.items():
        with pytest.raises(ValueError, match="workspace"):
            call(small)
    M = 16
    ll_need = epl.epl_ll_workspace_bytes(p, M)
    assert ll_need > 0
    with pytest.raises(ValueError, match="workspace"):
        epl.epl_ll_dispatch(p, M, T, t, t, t, t, t, t, t, t,
                            torch.empty(ll_need - 1, dtype=torch.uint8))
    with pytest.raises(ValueError, match="workspace"):
        epl.epl_combine(p, t, T * K, t, t, epl.EPL_OUT_F32, t, header_only)
    with pytest.raises(ValueError, match="workspace"):
        epl.epl_expert_scale(p, t, t, T * K, t, header_only)
    with pytest.raises(ValueError, match="workspace"):
        epl.epl_status(header_only)
    with pytest.raises(ValueError, match="workspace"):
        epl.epl_total(header_only)
    assert rec.calls == []
    # with exactly the size asked for, the same wrappers do reach the library
    calls["epl_layout"](torch.empty(need, dtype=torch.uint8))
    epl.epl_combine(p, t, T * K, t, t, epl.EPL_OUT_F32, t, torch.empty(256, dtype=torch.uint8))
    assert rec.calls == ["epl_layout", "epl_combine"]


def test_static_dispatch_rejects_what_its_workspace_cannot_hold(lib):
    """epl_dispatch_static checks the problem and the size of the workspace
    it needs against its static workspace on the host, before any HIP call:
    an invalid problem and one needing more than EPL_STATIC_WORKSPACE_BYTES
    return EPL_EINVAL here, without a GPU."""
    assert epl.EPL_STATIC_WORKSPACE_BYTES == 8 << 20
    big = P(num_tokens=1 << 20, scale_cols=0)           # ~32 MB of per-slot ranks
    assert epl.epl_workspace_bytes(big) > epl.EPL_STATIC_WORKSPACE_BYTES
    assert epl.epl_workspace_bytes(P(num_tokens=65536)) <= epl.EPL_STATIC_WORKSPACE_BYTES
    fake = 1 << 20
    args = (fake, fake, None, 10, fake, fake, None, fake, fake, None, fake, None, fake, fake,
            None, None)
    assert lib.epl_dispatch_static(ctypes.byref(big), *args) == epl.EPL_EINVAL
    assert lib.epl_dispatch_static(ctypes.byref(P(num_ranks=3)), *args) == epl.EPL_EINVAL
    assert lib.epl_dispatch_static(None, *args) == epl.EPL_EINVAL
