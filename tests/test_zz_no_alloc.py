"""The allocation-free dispatch (epl_dispatch_static) through the C ABI:
calls in a row -- the DeepSeek-V3-shaped batch (4096 tokens, hidden 7168 +
56 fp32 scales, 256 experts, top-8), then a smaller ragged batch (777 tokens
of hidden 4096, 64 experts, top-6, 5% of slots dropped), then a decode-sized
one (100 DeepSeek-V3-shaped tokens, dispatched in one launch) -- each against
epl_dispatch with a caller-owned workspace on the same inputs: every output
bit-identical, the status and total read through the returned static
workspace, and the combine run with it equal to the combine run with the
caller's workspace. A problem too large for the static workspace is
rejected before anything is launched. The caller's buffers sit between red
zones (tests/redzones.py) checked after each test."""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import permute_ep_layout_amd as epl  # noqa: E402
from permute_ep_layout_amd import workloads  # noqa: E402

import redzones  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
POISON = 0x5A


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    epl.load()


def poisoned(shape, dtype, byte):
    return redzones.poisoned(shape, dtype, byte, DEV)


@pytest.fixture(autouse=True)
def _red_zones():
    """Every buffer from poisoned() has red zones; a write past either end
    of one fails the test."""
    yield
    redzones.check()


def run(w, inp, static, byte):
    T, K, E, R, H, S = (w.num_tokens, w.num_topk, w.num_experts, w.num_ranks, w.hidden,
                        w.scale_cols)
    p = epl.Problem.make(T, K, E, R, H, S, 0, w.ranks_per_node)
    cap = epl.epl_capacity_rows(p)
    i32 = torch.int32
    r = dict(cnt=poisoned(E, i32, byte), per_rank=poisoned(R, i32, byte),
             per_node=poisoned(p.num_nodes, i32, byte) if p.num_nodes else None,
             in_rank=poisoned((T, R), torch.uint8, byte), start=poisoned(E, i32, byte),
             out=poisoned((cap, H), torch.bfloat16, byte),
             out_scale=poisoned((cap, S), torch.float32, byte) if S else None,
             m=poisoned(cap, i32, byte), oi=poisoned((T, K), i32, byte),
             total=torch.full((1,), -7, dtype=i32).pin_memory())
    topk = torch.from_numpy(inp["topk_idx"]).to(DEV)
    x = torch.from_numpy(inp["x"].view(np.int16)).to(DEV).view(torch.bfloat16)
    xs = torch.from_numpy(inp["x_scale"]).to(DEV) if S else None
    args = (p, topk, x, xs, cap, r["cnt"], r["per_rank"], r["per_node"], r["in_rank"],
            r["start"], r["total"], r["out"], r["out_scale"], r["m"], r["oi"])
    if static:
        ws = epl.epl_dispatch_static(*args)
        assert isinstance(ws, epl.StaticWorkspace) and ws.data_ptr() % 256 == 0
    else:
        ws = poisoned(epl.epl_workspace_bytes(p), torch.uint8, byte)
        epl.epl_dispatch(*args, ws)
    y = poisoned((T, H), torch.float32, byte)
    wt = torch.from_numpy(inp["topk_weights"]).to(DEV)
    epl.epl_combine(p, r["out"], cap, r["oi"], wt, epl.EPL_OUT_F32, y, ws)
    torch.cuda.synchronize()
    r["y"], r["status"], r["n"] = y, epl.epl_status(ws), epl.epl_total(ws)
    r["ws"] = ws
    return r


def test_static_dispatch_matches_the_workspace_dispatch_on_two_calls():
    big = workloads.get("dsv3")
    small = workloads.get("small").with_(num_tokens=777)
    # a third, decode-sized call: its dispatch is a single launch
    decode = workloads.get("dsv3").with_(num_tokens=100)
    addrs = []
    for w in (big, small, decode):
        print(f"[no-alloc] {w.name}: T={w.num_tokens} H={w.hidden} E={w.num_experts} "
              f"K={w.num_topk}", flush=True)
        inp = workloads.make_inputs(w)
        a = run(w, inp, static=True, byte=0x5A)
        b = run(w, inp, static=False, byte=0xA5)
        N = int((inp["topk_idx"] >= 0).sum())
        assert a["status"] == b["status"] == epl.EPL_OK
        assert a["n"] == b["n"] == int(a["total"][0]) == int(b["total"][0]) == N
        for key in ("cnt", "per_rank", "per_node", "in_rank", "start", "oi"):
            if a[key] is None:
                assert b[key] is None
                continue
            assert torch.equal(a[key], b[key]), key
        for key in ("out", "out_scale", "m"):
            if a[key] is None:
                continue
            assert torch.equal(a[key][:N].view(torch.uint8), b[key][:N].view(torch.uint8)), key
            # rows past N stay untouched by either call
            assert (a[key][N:].view(torch.uint8) == 0x5A).all(), key
        assert torch.equal(a["y"].view(torch.int32), b["y"].view(torch.int32))
        addrs.append(a["ws"].data_ptr())
    assert addrs[0] == addrs[1] == addrs[2]    # one static workspace per GPU, reused


def test_static_dispatch_rejects_a_problem_beyond_its_workspace():
    T = 1 << 20                             # ~32 MB of per-slot ranks at top-8
    p = epl.Problem.make(T, 8, 256, 32, 7168, 0)
    assert epl.epl_workspace_bytes(p) > epl.EPL_STATIC_WORKSPACE_BYTES
    lib = epl.load()
    nul = None
    rc = lib.epl_dispatch_static(ctypes.byref(p), nul, nul, nul, 0, nul, nul, nul, nul, nul, nul,
                                 nul, nul, nul, nul, nul, nul)
    assert rc == epl.EPL_EINVAL
