"""The dispatch + combine chain captured in a HIP graph (torch.cuda.CUDAGraph
over the C ABI calls), in each launch shape of epl_dispatch, for the
allocation-free dispatch and for the low-latency dispatch: every replay, with
eager work on other buffers in between, reproduces the eager results bit for
bit. The chain records no
memset node; the scan writes N through a mapped host word. The chains'
buffers sit between red zones (tests/redzones.py) checked after each test."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import permute_ep_layout_amd as epl  # noqa: E402
from permute_ep_layout_amd import workloads  # noqa: E402

import redzones  # noqa: E402

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    epl.load()


@pytest.fixture(autouse=True)
def _red_zones():
    """The chains' buffers have red zones: no replay may write past them."""
    yield
    redzones.check()


class Chain:
    """Buffers and pre-marshalled calls for one dispatch + combine."""

    def __init__(self, w, stream):
        inp = workloads.make_inputs(w)
        T, K, E, R, H, S = (w.num_tokens, w.num_topk, w.num_experts, w.num_ranks, w.hidden,
                            w.scale_cols)
        self.topk = torch.from_numpy(inp["topk_idx"]).to(DEV)
        self.x = torch.from_numpy(inp["x"].view(np.int16)).to(DEV).view(torch.bfloat16)
        self.xs = torch.from_numpy(inp["x_scale"]).to(DEV) if S else None
        self.wt = torch.from_numpy(inp["topk_weights"]).to(DEV)
        p = epl.Problem.make(T, K, E, R, H, S, 0, w.ranks_per_node)
        self.cap = cap = epl.epl_capacity_rows(p)
        i32 = torch.int32

        def buf(shape, dtype):
            return redzones.poisoned(shape, dtype, 0x5A, DEV)

        self.ws = buf(epl.epl_workspace_bytes(p), torch.uint8)
        self.cnt = buf(E, i32)
        self.per = buf(R, i32)
        self.node = buf(p.num_nodes, i32) if p.num_nodes else None
        self.inr = buf((T, R), torch.uint8)
        self.start = buf(E, i32)
        self.total = torch.zeros(1, dtype=i32).pin_memory()
        self.out = buf((cap, H), torch.bfloat16)
        self.osc = buf((cap, S), torch.float32) if S else None
        self.m = buf(cap, i32)
        self.oi = buf((T, K), i32)
        self.y = buf((T, H), torch.float32)
        # checked once through the validating wrappers, then pre-marshalled
        epl.epl_dispatch(p, self.topk, self.x, self.xs, cap, self.cnt, self.per, self.node,
                         self.inr, self.start, self.total, self.out, self.osc, self.m, self.oi,
                         self.ws, stream)
        epl.epl_combine(p, self.out, cap, self.oi, self.wt, epl.EPL_OUT_F32, self.y, self.ws,
                        stream)
        self.calls = [
            epl.prepare("epl_dispatch", p, self.topk, self.x, self.xs, cap, self.cnt, self.per,
                        self.node, self.inr, self.start, self.total, self.out, self.osc, self.m,
                        self.oi, self.ws, stream=stream),
            epl.prepare("epl_combine", p, self.out, cap, self.oi, self.wt, epl.EPL_OUT_F32, self.y,
                        self.ws, stream=stream),
        ]

    def run(self):
        for c in self.calls:
            c()

    def snapshot(self):
        n = int(self.total[0])
        return dict(n=n, y=self.y.clone(), oi=self.oi.clone(), m=self.m[:n].clone(),
                    out=self.out[:n].clone(), start=self.start.clone(), cnt=self.cnt.clone())

    def poison(self):
        for t in (self.y, self.oi, self.m, self.out, self.start, self.cnt):
            t.view(torch.uint8).fill_(0x5A)
        self.total.fill_(-1)


# The captured chain in each of the dispatch's launch shapes: the scatter
# doing the scan's work (1536 DeepSeek-V3-shaped tokens), one launch for a
# decode-sized batch (64 tokens), and layout, scan and a column-part scatter
# (700 tokens of hidden 4096); the eager work in between is another shape.
CASES = [("dsv3", 1536, "small", 700), ("dsv3", 64, "dsv3", 1536), ("small", 700, "dsv3", 64)]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}_t{c[1]}" for c in CASES])
def test_graph_replays_match_eager(case):
    name, T, other_name, other_T = case
    print(f"[graph] {name} T={T}, eager {other_name} T={other_T}", flush=True)
    s = torch.cuda.Stream()
    w = workloads.get(name).with_(num_tokens=T)
    other = workloads.get(other_name).with_(num_tokens=other_T)
    with torch.cuda.stream(s):
        a = Chain(w, s)
        b = Chain(other, s)
        a.run()
        s.synchronize()
        ref = a.snapshot()
        assert epl.epl_status(a.ws, s.cuda_stream) == epl.EPL_OK
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            a.run()
        for i in range(4):
            a.poison()
            b.run()                       # eager work on other buffers in between
            g.replay()
            s.synchronize()
            got = a.snapshot()
            assert got["n"] == ref["n"], i
            for key in ("y", "oi", "m", "out", "start", "cnt"):
                assert torch.equal(got[key].view(torch.uint8), ref[key].view(torch.uint8)), (i, key)
            assert epl.epl_status(a.ws, s.cuda_stream) == epl.EPL_OK


@pytest.mark.parametrize("T", [1536, 64])
def test_graph_replays_of_the_allocation_free_dispatch(T):
    """epl_dispatch_static (the entry point for callers that cannot allocate,
    such as code under graph capture) captured with its combine: every replay
    reproduces the eager workspace dispatch bit for bit, with eager work of
    another shape (and its own workspace) in between."""
    import ctypes
    print(f"[graph] static dispatch T={T}", flush=True)
    s = torch.cuda.Stream()
    w = workloads.get("dsv3").with_(num_tokens=T)
    with torch.cuda.stream(s):
        a = Chain(w, s)                     # the workspace dispatch: reference and buffers
        b = Chain(workloads.get("small").with_(num_tokens=700), s)
        a.run()
        s.synchronize()
        ref = a.snapshot()
        inp_p = epl.Problem.make(w.num_tokens, w.num_topk, w.num_experts, w.num_ranks, w.hidden,
                                 w.scale_cols, 0, w.ranks_per_node)
        static_ws = epl.epl_dispatch_static(inp_p, a.topk, a.x, a.xs, a.cap, a.cnt, a.per, a.node,
                                            a.inr, a.start, a.total, a.out, a.osc, a.m, a.oi, s)
        calls = [
            epl.prepare("epl_dispatch_static", inp_p, a.topk, a.x, a.xs, a.cap, a.cnt, a.per,
                        a.node, a.inr, a.start, a.total, a.out, a.osc, a.m, a.oi, None, stream=s),
            epl.prepare("epl_combine", inp_p, a.out, a.cap, a.oi, a.wt, epl.EPL_OUT_F32, a.y,
                        ctypes.c_void_p(static_ws.data_ptr()), stream=s),
        ]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for c in calls:
                c()
        for i in range(4):
            a.poison()
            b.run()
            g.replay()
            s.synchronize()
            got = a.snapshot()
            assert got["n"] == ref["n"], i
            for key in ("y", "oi", "m", "out", "start", "cnt"):
                assert torch.equal(got[key].view(torch.uint8), ref[key].view(torch.uint8)), (i, key)
            assert epl.epl_status(static_ws, s.cuda_stream) == epl.EPL_OK


@pytest.mark.parametrize("T", [128, 512])
def test_graph_replays_of_the_low_latency_dispatch(T):
    """The low-latency dispatch and a combine over its rectangle captured in
    a graph (one launch for 128 DeepSeek-V3-shaped tokens, three for 512):
    every replay, with eager work of another shape in between, reproduces
    the eager outputs bit for bit."""
    print(f"[graph] low-latency T={T}", flush=True)
    s = torch.cuda.Stream()
    w = workloads.get("dsv3_ll").with_(num_tokens=T)
    inp = workloads.make_inputs(w)
    M, K, E, H = w.ll_segment, w.num_topk, w.num_experts, w.hidden
    cap, S, i32 = T, H // 128, torch.int32

    def buf(shape, dtype):
        return redzones.poisoned(shape, dtype, 0x5A, DEV)

    with torch.cuda.stream(s):
        topk = torch.from_numpy(inp["topk_idx"]).to(DEV)
        x = torch.from_numpy(inp["x"].view(np.int16)).to(DEV).view(torch.bfloat16)
        wt = torch.from_numpy(inp["topk_weights"]).to(DEV)
        eo = torch.randn((E * cap, H), device=DEV).to(torch.bfloat16)
        p = epl.Problem.make(T, K, E, 1, H, S)
        pc = epl.Problem.make(T, K, E, 1, H, 0)
        ws = buf(epl.epl_ll_workspace_bytes(p, M), torch.uint8)
        outs = dict(out=buf((E, cap, H), torch.uint8), osc=buf((E, S, cap), torch.float32),
                    recv=buf(E, i32), src=buf((E, cap), i32), lr=buf((E, T // M, 2), i32),
                    oi=buf((T, K), i32), y=buf((T, H), torch.float32))
        o = outs
        epl.epl_ll_dispatch(p, M, cap, topk, x, o["out"], o["osc"], o["recv"], o["src"], o["lr"],
                            o["oi"], ws, s)
        epl.epl_combine(pc, eo, E * cap, o["oi"], wt, epl.EPL_OUT_F32, o["y"], ws, s)
        s.synchronize()
        assert epl.epl_status(ws, s.cuda_stream) == epl.EPL_OK
        flat = o["oi"].view(-1).long()
        placed = flat[flat >= 0]
        ref = {k: v.clone() for k, v in outs.items() if k != "out"}
        ref["rows"] = o["out"].view(E * cap, H)[placed].clone()
        calls = [
            epl.prepare("epl_ll_dispatch", p, M, cap, topk, x, o["out"], o["osc"], o["recv"],
                        o["src"], o["lr"], o["oi"], ws, stream=s),
            epl.prepare("epl_combine", pc, eo, E * cap, o["oi"], wt, epl.EPL_OUT_F32, o["y"], ws,
                        stream=s),
        ]
        b = Chain(workloads.get("small").with_(num_tokens=700), s)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for c in calls:
                c()
        for i in range(4):
            for t in outs.values():
                t.view(torch.uint8).fill_(0x5A)
            b.run()
            g.replay()
            s.synchronize()
            for k in ("osc", "recv", "src", "lr", "oi", "y"):
                assert torch.equal(outs[k].view(torch.uint8), ref[k].view(torch.uint8)), (i, k)
            got_rows = o["out"].view(E * cap, H)[placed]
            assert torch.equal(got_rows, ref["rows"]), i
            assert epl.epl_status(ws, s.cuda_stream) == epl.EPL_OK
