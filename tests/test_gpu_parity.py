"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Layout, scan, m_indices, output_index, scattered rows and scale rows must be
bit-exact. Combine (fp32 accumulation) must satisfy, element by element,
    |y_gpu - y_oracle| <= 1e-5 * sum_k |w[t,k]| * |v_k|
where y_oracle is the fp64 sum and the right-hand side is the same sum over
absolute values (also computed by the oracle): "1e-5 relative" measured
against the size of the terms, so cancellation cannot make it meaningless.
bf16 combine output must be within half a bf16 ulp of that (RNE of the fp32
sum). Output buffers are poisoned before every call so that a slot the
kernels forget to write cannot pass, and each sits between red zones
(tests/redzones.py) checked after every test, so that a write past either
end of a buffer cannot pass either.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import permute_ep_layout_amd as epl  # noqa: E402
from permute_ep_layout_amd import workloads  # noqa: E402

import redzones  # noqa: E402

pytestmark = pytest.mark.gpu

POISON = 0x5A


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    epl.load()


DEV = torch.device("cuda:0")
ORC = None


def orc():
    global ORC
    if ORC is None:
        ORC = oracle.default()
    return ORC


def to_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)


def u16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def poisoned(shape, dtype, byte=POISON):
    return redzones.poisoned(shape, dtype, byte, DEV)


@pytest.fixture(autouse=True)
def _red_zones():
    """Every buffer from poisoned() has red zones; a write past either end
    of one fails the test."""
    yield
    redzones.check()


def gpu_dispatch(topk, x, xs, E, R, cap=None, byte=POISON, stream=None, split=False,
                 alignment=0, G=0):
    """Run dispatch through the C ABI on poisoned buffers; returns tensors."""
    T, K = topk.shape
    H = x.shape[1]
    S = 0 if xs is None else xs.shape[1]
    p = epl.Problem.make(T, K, E, R, H, S, alignment, G)
    cap = epl.epl_capacity_rows(p) if cap is None else cap
    ws = poisoned(epl.epl_workspace_bytes(p), torch.uint8, byte)
    r = dict(
        cnt=poisoned(E, torch.int32, byte), per_rank=poisoned(R, torch.int32, byte),
        per_node=poisoned(p.num_nodes, torch.int32, byte) if p.num_nodes else None, G=G,
        in_rank=poisoned((T, R), torch.uint8, byte), start=poisoned(E, torch.int32, byte),
        out=poisoned((cap, H), torch.bfloat16, byte),
        out_scale=poisoned((cap, S), torch.float32, byte) if S else None,
        m=poisoned(cap, torch.int32, byte), oi=poisoned((T, K), torch.int32, byte),
        total_host=torch.full((1,), -7, dtype=torch.int32).pin_memory(), ws=ws, p=p, cap=cap)
    tk = torch.from_numpy(topk).to(DEV)
    xd = to_bf16(x)
    xsd = None if xs is None else torch.from_numpy(xs).to(DEV)
    if split:
        epl.epl_layout(p, tk, r["cnt"], r["per_rank"], r["per_node"], r["in_rank"], ws, stream)
        epl.epl_scan(p, r["cnt"], r["start"], r["total_host"], ws, stream)
        epl.epl_scatter(p, xd, xsd, tk, r["start"], ws, cap, r["out"], r["out_scale"], r["m"],
                        r["oi"], stream)
    else:
        epl.epl_dispatch(p, tk, xd, xsd, cap, r["cnt"], r["per_rank"], r["per_node"], r["in_rank"],
                         r["start"], r["total_host"], r["out"], r["out_scale"], r["m"], r["oi"],
                         ws, stream)
    r["x"], r["topk"] = xd, tk
    return r


def gpu_combine(r, eo, w, out_dtype, byte=POISON, stream=None):
    T, K = r["oi"].shape
    H = eo.shape[1]
    p = epl.Problem.make(T, K, r["p"].num_experts, r["p"].num_ranks, H, 0)
    y = poisoned((T, H), torch.float32 if out_dtype == epl.EPL_OUT_F32 else torch.bfloat16, byte)
    wd = torch.from_numpy(w).to(DEV)
    epl.epl_combine(p, eo, eo.shape[0], r["oi"], wd, out_dtype, y, r["ws"], stream)
    return y


def check_layout_and_scatter(r, ref, x, xs):
    torch.cuda.synchronize()
    N = ref["total"]
    assert int(r["total_host"][0]) == N
    assert epl.epl_total(r["ws"]) == N
    np.testing.assert_array_equal(r["cnt"].cpu().numpy(), ref["num_tokens_per_expert"])
    np.testing.assert_array_equal(r["per_rank"].cpu().numpy(), ref["num_tokens_per_rank"])
    np.testing.assert_array_equal(r["in_rank"].cpu().numpy(), ref["is_token_in_rank"])
    want_nodes = orc().rdma_counts(ref["is_token_in_rank"], r["G"])
    if want_nodes is None:
        assert r["per_node"] is None
    else:
        np.testing.assert_array_equal(r["per_node"].cpu().numpy(), want_nodes)
    np.testing.assert_array_equal(r["start"].cpu().numpy(), ref["expert_start_loc"])
    np.testing.assert_array_equal(r["oi"].cpu().numpy(), ref["output_index"])
    np.testing.assert_array_equal(r["m"][:N].cpu().numpy(), ref["m_indices"])
    # rows that hold a routed slot (alignment padding rows are not written)
    real = ref["m_indices"] >= 0
    if ref.get("out") is not None:
        np.testing.assert_array_equal(u16(r["out"][:N])[real], ref["out"][real])
    if xs is not None:
        np.testing.assert_array_equal(r["out_scale"][:N].cpu().numpy().view(np.uint32)[real],
                                      ref["out_scale"].view(np.uint32)[real])


def combine_bound(eo_u16, oi, w, tokens=None):
    return orc().combine(eo_u16 & np.uint16(0x7FFF), oi, np.abs(w), tokens=tokens)


def check_combine_f32(y_gpu, y_ref, bound):
    d = np.abs(y_gpu.astype(np.float64) - y_ref)
    bad = d > 1e-5 * bound
    assert not bad.any(), (f"{bad.sum()} elements beyond 1e-5 * sum|w v|; worst excess "
                           f"{(d - 1e-5 * bound).max():.3e}")


def check_combine_bf16(y_gpu_u16, y_ref, bound):
    yg = (y_gpu_u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    eps = 1e-5 * bound
    lim = 2.0 ** -8 * (np.abs(y_ref) + eps) + eps
    bad = np.abs(yg - y_ref) > lim
    assert not bad.any(), f"{bad.sum()} bf16 elements beyond half an ulp of the fp32 bound"


def full_parity(w: workloads.Workload, inp=None, split=False, alignment=0):
    inp = inp or workloads.make_inputs(w)
    topk, x, xs, wt = inp["topk_idx"], inp["x"], inp["x_scale"], inp["topk_weights"]
    E, R = w.num_experts, w.num_ranks
    ref = orc().run_all(x, xs, topk, wt, E, R, expert_fn=w.expert_fn, alignment=alignment)
    r = gpu_dispatch(topk, x, xs, E, R, split=split, alignment=alignment, G=w.ranks_per_node)
    assert epl.epl_status(r["ws"]) == epl.EPL_OK
    check_layout_and_scatter(r, ref, x, xs)
    N = ref["total"]
    if w.expert_fn == "identity":
        eo = r["out"]
    else:
        eo = poisoned(r["out"].shape, r["out"].dtype)
        epl.epl_expert_scale(r["p"], r["out"], r["m"], r["cap"], eo, r["ws"])
        real = ref["m_indices"] >= 0
        np.testing.assert_array_equal(u16(eo[:N])[real], ref["expert_out"][real])
    y = gpu_combine(r, eo, wt, epl.EPL_OUT_F32)
    yb = gpu_combine(r, eo, wt, epl.EPL_OUT_BF16)
    bound = combine_bound(ref["expert_out"], ref["output_index"], wt)
    y_cpu = y.cpu()
    check_combine_f32(y_cpu.numpy(), ref["y"], bound)
    check_combine_bf16(u16(yb), ref["y"], bound)
    check_bf16_is_rne_of_f32(u16(yb), y_cpu)
    assert epl.epl_status(r["ws"]) == epl.EPL_OK
    return r, y


def check_bf16_is_rne_of_f32(yb_u16, y_f32_cpu):
    """Both output types come from the same fp32 sums in the same order, so
    the bf16 output must be exactly their round-to-nearest-even, checked
    against torch's own float32 -> bfloat16 conversion (finite values)."""
    assert torch.isfinite(y_f32_cpu).all()
    want = y_f32_cpu.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(yb_u16, want)


# ------------------------------------------------------------ workloads --

@pytest.mark.parametrize("name", ["tiny", "small", "dsv3", "skew", "dsv3_recv"])
def test_workload_full_parity(name):
    print(f"[parity] workload={name}", flush=True)
    full_parity(workloads.get(name))


def test_dsv3_split_calls_match_oracle():
    full_parity(workloads.get("dsv3").with_(num_tokens=1500), split=True)


def test_deterministic_bitwise_repeat():
    w = workloads.get("dsv3").with_(num_tokens=2000)
    inp = workloads.make_inputs(w)
    a = gpu_dispatch(inp["topk_idx"], inp["x"], inp["x_scale"], w.num_experts, w.num_ranks,
                     byte=0x5A)
    b = gpu_dispatch(inp["topk_idx"], inp["x"], inp["x_scale"], w.num_experts, w.num_ranks,
                     byte=0xA5)
    torch.cuda.synchronize()
    N = int(a["total_host"][0])
    for key in ("cnt", "per_rank", "in_rank", "start", "oi"):
        assert torch.equal(a[key], b[key]), key
    for key in ("out", "out_scale", "m"):
        assert torch.equal(a[key][:N].view(torch.uint8), b[key][:N].view(torch.uint8)), key
    ya = gpu_combine(a, a["out"], inp["topk_weights"], epl.EPL_OUT_F32)
    yb = gpu_combine(b, b["out"], inp["topk_weights"], epl.EPL_OUT_F32, byte=0xA5)
    assert torch.equal(ya.view(torch.int32), yb.view(torch.int32))


@pytest.mark.timeout(900)
def test_large_batch_full_parity():
    """The 65536-token workload at full size, everything compared: layout,
    scan and indices in full; every scattered row through the oracle's index
    map; every one of the 524288 expert stand-in rows bit-exact against the
    oracle's expert_scale; every token's combine output within 1e-5 of
    sum |w v|. The oracle's side is computed in chunks of 4096 tokens (the
    rows of a chunk are the chunk's slots; its expert rows come from the
    oracle's expert_scale of the oracle-placed token rows) on a few CPU
    threads, so host memory stays bounded."""
    from concurrent.futures import ThreadPoolExecutor

    w = workloads.get("large")
    print("[parity] workload=large (generating inputs)", flush=True)
    topk = workloads.make_topk(w)
    wt = workloads.make_weights(w, topk)
    x = workloads.make_x(w)
    E, R, T, K, H = w.num_experts, w.num_ranks, w.num_tokens, w.num_topk, w.hidden
    cnt, per_rank, in_rank = orc().layout(topk, E, R)
    start, N = orc().scan(cnt)
    _, _, m_ref, oi_ref = orc().scatter(None, None, topk, start, N, copy_rows=False)
    ref = dict(num_tokens_per_expert=cnt, num_tokens_per_rank=per_rank, is_token_in_rank=in_rank,
               expert_start_loc=start, total=N, m_indices=m_ref, output_index=oi_ref)
    r = gpu_dispatch(topk, x, None, E, R, G=w.ranks_per_node)
    eo = poisoned(r["out"].shape, r["out"].dtype)
    epl.epl_expert_scale(r["p"], r["out"], r["m"], r["cap"], eo, r["ws"])
    y = gpu_combine(r, eo, wt, epl.EPL_OUT_F32)
    assert epl.epl_status(r["ws"]) == epl.EPL_OK
    check_layout_and_scatter(r, ref, x, None)
    # every scattered row against the token the oracle placed there
    tt, kk = np.nonzero(topk >= 0)
    src = np.empty(N, np.int64)
    src[oi_ref[tt, kk]] = tt
    src_d = torch.from_numpy(src).to(DEV)
    xd = r["x"].view(torch.int16)
    outd = r["out"].view(torch.int16)
    for p0 in range(0, N, 1 << 16):
        p1 = min(N, p0 + (1 << 16))
        assert torch.equal(outd[p0:p1], xd[src_d[p0:p1]]), f"rows {p0}:{p1}"
    del src_d
    print("[parity] large: indices and scattered rows ok", flush=True)

    def oracle_chunk(t0, t1):
        """The oracle's expert rows of tokens [t0, t1) (in slot order), their
        global row ids, and the oracle's combine of those tokens."""
        oi = oi_ref[t0:t1]
        ct, ck = np.nonzero(oi >= 0)
        rows = oi[ct, ck].astype(np.int64)
        sub_eo = orc().expert_scale(x[t0 + ct], m_ref[rows])
        sub_oi = np.full(oi.shape, -1, np.int32)
        sub_oi[ct, ck] = np.arange(ct.size, dtype=np.int32)
        y_ref = orc().combine(sub_eo, sub_oi, wt[t0:t1])
        bound = combine_bound(sub_eo, sub_oi, wt[t0:t1])
        return rows, sub_eo, y_ref, bound

    chunk, window = 4096, 6
    spans = [(t0, min(T, t0 + chunk)) for t0 in range(0, T, chunk)]
    seen = np.zeros(N, bool)
    with ThreadPoolExecutor(window) as pool:
        pending = [pool.submit(oracle_chunk, *sp) for sp in spans[:window]]
        for n, (t0, t1) in enumerate(spans):
            rows, sub_eo, y_ref, bound = pending.pop(0).result()
            if n + window < len(spans):
                pending.append(pool.submit(oracle_chunk, *spans[n + window]))
            got = u16(eo[torch.from_numpy(rows).to(DEV)])
            np.testing.assert_array_equal(got, sub_eo, err_msg=f"expert rows of tokens {t0}:{t1}")
            check_combine_f32(y[t0:t1].cpu().numpy(), y_ref, bound)
            seen[rows] = True
            print(f"[parity] large: tokens {t0}:{t1} expert rows and combine ok", flush=True)
    assert seen.all()          # every row of the buffer was compared once


# -------------------------------------------------------- expert alignment --

@pytest.mark.parametrize("name,a", [("tiny", 4), ("small", 256), ("dsv3", 128), ("skew", 64),
                                    ("small", 3)])
def test_aligned_blocks_parity(name, a):
    """Per-expert blocks padded to a multiple of a rows; padding rows carry
    m_indices = -1; everything else as without padding."""
    print(f"[parity] workload={name} alignment={a}", flush=True)
    full_parity(workloads.get(name), alignment=a)


@pytest.mark.parametrize("split", [False, True])
def test_largest_alignment(split):
    """The largest expert alignment the library takes (65536 rows): every
    expert's block, even one with a single slot, is a whole 65536-row block,
    so nearly every row of the 9-block buffer is padding marked -1."""
    print(f"[parity] alignment 65536 split={split}", flush=True)
    rng = np.random.default_rng(65536)
    E, R, T, K, H = 8, 2, 100, 4, 256
    topk = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64)
    topk[rng.random(topk.shape) < 0.1] = -1
    x, xs, wt = _mk(topk, H, 3, True)
    ref = orc().run_all(x, xs, topk, wt, E, R, alignment=65536)
    r = gpu_dispatch(topk, x, xs, E, R, split=split, alignment=65536)
    assert epl.epl_status(r["ws"]) == epl.EPL_OK
    assert ref["total"] == 65536 * int((np.bincount(topk[topk >= 0], minlength=E) > 0).sum())
    check_layout_and_scatter(r, ref, x, xs)
    y = gpu_combine(r, r["out"], wt, epl.EPL_OUT_F32)
    check_combine_f32(y.cpu().numpy(), ref["y"],
                      combine_bound(ref["expert_out"], ref["output_index"], wt))


def test_aligned_split_calls_and_expert_stand_in():
    w = workloads.get("small").with_(num_tokens=900, expert_fn="scale", drop_rate=0.2)
    full_parity(w, split=True, alignment=32)


def test_aligned_capacity_overflow_in_padding_is_flagged():
    rng = np.random.default_rng(12)
    E, R, T, K, H, a = 8, 2, 100, 3, 64, 16
    # the last expert gets exactly one slot, so its block ends with 15 padding rows
    topk = np.stack([rng.permutation(E - 1)[:K] for _ in range(T)]).astype(np.int64)
    topk[50, 1] = E - 1
    x, _, wt = _mk(topk, H)
    ref = orc().run_all(x, None, topk, wt, E, R, alignment=a)
    N = ref["total"]
    assert (ref["m_indices"][N - (a - 1):] == -1).all()
    r = gpu_dispatch(topk, x, None, E, R, cap=N - 1, alignment=a)
    assert epl.epl_status(r["ws"]) == epl.EPL_ECAPACITY
    np.testing.assert_array_equal(r["m"].cpu().numpy(), ref["m_indices"][:N - 1])


def test_aligned_split_call_with_bad_expert_start_loc_is_flagged():
    """epl_scatter takes expert_start_loc from the caller. With offsets that
    put one expert's rows and alignment padding before row 0 and another's
    partly past the capacity, the scatter writes nothing outside its buffers,
    reports EPL_ECAPACITY, places every slot whose row is in range (with the
    same in-expert rank as under the true offsets) and marks the others -1."""
    rng = np.random.default_rng(13)
    E, R, T, K, H, a = 8, 2, 60, 3, 64, 16
    topk = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64)
    x, _, wt = _mk(topk, H)
    ref = orc().run_all(x, None, topk, wt, E, R, alignment=a)
    p = epl.Problem.make(T, K, E, R, H, 0, a)
    cap = epl.epl_capacity_rows(p)
    guard = 64
    ws = poisoned(epl.epl_workspace_bytes(p), torch.uint8)
    tk, xd = torch.from_numpy(topk).to(DEV), to_bf16(x)
    cnt, per_rank = poisoned(E, torch.int32), poisoned(R, torch.int32)
    in_rank, start = poisoned((T, R), torch.uint8), poisoned(E, torch.int32)
    epl.epl_layout(p, tk, cnt, per_rank, None, in_rank, ws)
    epl.epl_scan(p, cnt, start, None, ws)
    bad = ref["expert_start_loc"].astype(np.int64).copy()
    bad[0] = -40                       # all of expert 0's rows and padding before row 0
    bad[E - 1] = cap - 5               # expert 7: 5 rows fit, the rest and its padding do not
    out_full = poisoned((cap + 2 * guard, H), torch.bfloat16)
    m_full = poisoned(cap + 2 * guard, torch.int32)
    out, m = out_full[guard:guard + cap], m_full[guard:guard + cap]
    oi = poisoned((T, K), torch.int32)
    epl.epl_scatter(p, xd, None, tk, torch.from_numpy(bad.astype(np.int32)).to(DEV), ws, cap,
                    out, None, m, oi)
    assert epl.epl_status(ws) == epl.EPL_ECAPACITY
    for t_ in (out_full[:guard], out_full[guard + cap:], m_full[:guard], m_full[guard + cap:]):
        assert (t_.view(torch.uint8) == POISON).all()
    # expected placement: the oracle's in-expert rank on top of the bad offsets
    oi_ref = ref["output_index"]
    e_of = np.where(topk >= 0, topk, 0)
    rows = np.where(topk >= 0, bad[e_of] + (oi_ref - ref["expert_start_loc"][e_of]), -1)
    want_oi = np.where((rows >= 0) & (rows < cap), rows, -1)
    np.testing.assert_array_equal(oi.cpu().numpy(), want_oi)
    assert (want_oi[topk == 0] == -1).all() and ((want_oi >= 0) & (topk == E - 1)).sum() == 5
    want_m = np.full(cap, np.frombuffer(bytes([POISON] * 4), np.int32)[0], np.int32)
    counts = ref["num_tokens_per_expert"].astype(np.int64)
    for e in range(E):
        blk = (counts[e] + a - 1) // a * a
        for q in range(bad[e], bad[e] + blk):
            if 0 <= q < cap:
                want_m[q] = e if q < bad[e] + counts[e] else -1
    np.testing.assert_array_equal(m.cpu().numpy(), want_m)
    tt, kk = np.nonzero(want_oi >= 0)
    np.testing.assert_array_equal(u16(out)[want_oi[tt, kk]], x[tt])


# ------------------------------------------------------------- FP8 payload --

def fp8_parity(w, fmt, alignment=0, extra_cap=0, split=False):
    """FP8 rows and scale words through epl_dispatch_fp8 / epl_scatter_fp8
    against the oracle's byte-row scatter."""
    inp = workloads.make_inputs(w)
    topk, x, xs = inp["topk_idx"], inp["x"], inp["x_scale"]
    T, K = topk.shape
    E, R, H, S = w.num_experts, w.num_ranks, w.hidden, w.scale_cols
    if fmt == epl.EPL_SCALE_NONE:
        S, xs = 0, None
    p = epl.Problem.make(T, K, E, R, H, S, alignment, w.ranks_per_node)
    cap = epl.epl_capacity_rows(p) + extra_cap
    orc_ = orc()
    cnt, per_rank, in_rank = orc_.layout(topk, E, R)
    start, N = orc_.scan(cnt, alignment)
    words = None if xs is None else xs.view(np.uint32)
    ofmt = {epl.EPL_SCALE_NONE: orc_.SCALE_NONE, epl.EPL_SCALE_F32: orc_.SCALE_ROWS,
            epl.EPL_SCALE_UE8M0: orc_.SCALE_COLS}[fmt]
    out_ref, sc_ref, m_ref, oi_ref = orc_.scatter_rows(x, words, ofmt, topk, start, N, scale_ld=cap)
    W = 0 if xs is None else xs.shape[1]
    ws = poisoned(epl.epl_workspace_bytes(p), torch.uint8)
    cnt_d, per_d = poisoned(E, torch.int32), poisoned(R, torch.int32)
    node_d = poisoned(p.num_nodes, torch.int32) if p.num_nodes else None
    in_d, start_d = poisoned((T, R), torch.uint8), poisoned(E, torch.int32)
    out = poisoned((cap, H), torch.uint8)
    if fmt == epl.EPL_SCALE_F32:
        out_s = poisoned((cap, S), torch.float32)
        xs_d = torch.from_numpy(xs).to(DEV)
    elif fmt == epl.EPL_SCALE_UE8M0:
        out_s = poisoned((W, cap), torch.int32)
        xs_d = torch.from_numpy(xs.view(np.int32)).to(DEV)
    else:
        out_s, xs_d = None, None
    m = poisoned(cap, torch.int32)
    oi = poisoned((T, K), torch.int32)
    tot = torch.full((1,), -7, dtype=torch.int32).pin_memory()
    tk = torch.from_numpy(topk).to(DEV)
    xd = torch.from_numpy(x).to(DEV)
    if split:
        epl.epl_layout(p, tk, cnt_d, per_d, node_d, in_d, ws)
        epl.epl_scan(p, cnt_d, start_d, tot, ws)
        epl.epl_scatter_fp8(p, xd, xs_d, fmt, tk, start_d, ws, cap, out, out_s, m, oi)
    else:
        epl.epl_dispatch_fp8(p, tk, xd, xs_d, fmt, cap, cnt_d, per_d, node_d, in_d, start_d, tot,
                             out, out_s, m, oi, ws)
    assert epl.epl_status(ws) == epl.EPL_OK
    assert int(tot[0]) == N
    np.testing.assert_array_equal(cnt_d.cpu().numpy(), cnt)
    np.testing.assert_array_equal(in_d.cpu().numpy(), in_rank)
    np.testing.assert_array_equal(per_d.cpu().numpy(), per_rank)
    if node_d is not None:
        np.testing.assert_array_equal(node_d.cpu().numpy(), orc_.rdma_counts(in_rank, w.ranks_per_node))
    np.testing.assert_array_equal(start_d.cpu().numpy(), start)
    np.testing.assert_array_equal(oi.cpu().numpy(), oi_ref)
    np.testing.assert_array_equal(m[:N].cpu().numpy(), m_ref)
    real = m_ref >= 0
    np.testing.assert_array_equal(out[:N].cpu().numpy()[real], out_ref[real])
    if fmt == epl.EPL_SCALE_F32:
        np.testing.assert_array_equal(out_s[:N].cpu().numpy().view(np.uint32)[real], sc_ref[real])
    elif fmt == epl.EPL_SCALE_UE8M0:
        got = out_s.cpu().numpy().view(np.uint32)[:, :N]
        want = sc_ref.reshape(W, cap)[:, :N]
        np.testing.assert_array_equal(got[:, real], want[:, real])


def test_fp8_dsv3_ue8m0_parity():
    print("[parity] workload=dsv3_fp8 ue8m0", flush=True)
    fp8_parity(workloads.get("dsv3_fp8"), epl.EPL_SCALE_UE8M0)


@pytest.mark.parametrize("case", [
    # name, T, H, E, K, R, fmt, alignment, extra capacity, split
    ("f32_scales", 700, 1024, 32, 4, 8, epl.EPL_SCALE_F32, 0, 0, False),
    ("no_scales_ragged_h", 555, 144, 16, 3, 4, epl.EPL_SCALE_NONE, 0, 0, False),
    ("ue8m0_s5_aligned", 900, 640, 24, 5, 6, epl.EPL_SCALE_UE8M0, 32, 0, False),
    ("ue8m0_spare_capacity", 400, 512, 16, 2, 4, epl.EPL_SCALE_UE8M0, 0, 77, True),
    ("ue8m0_large_t", 9000, 256, 64, 6, 8, epl.EPL_SCALE_UE8M0, 16, 0, False),
    ("ue8m0_striding", 6001, 384, 64, 6, 8, epl.EPL_SCALE_UE8M0, 0, 0, False),
    ("none_striding_split_aligned", 4999, 272, 24, 3, 6, epl.EPL_SCALE_NONE, 8, 0, True),
    # decode-sized: column parts of byte rows (3 parts of 7168 bytes)
    ("ue8m0_decode_t200", 200, 7168, 256, 8, 32, epl.EPL_SCALE_UE8M0, 0, 0, False),
    ("f32_decode_t64_aligned", 64, 7168, 64, 8, 8, epl.EPL_SCALE_F32, 16, 0, True),
    # byte rows of 12 KB: the long-row grid, whose active size follows the
    # routing density, with 24 packed scale words per row
    ("ue8m0_long_rows_h12288", 1500, 12288, 64, 4, 8, epl.EPL_SCALE_UE8M0, 0, 0, False),
    ("f32_k64", 300, 256, 512, 64, 64, epl.EPL_SCALE_F32, 0, 0, False),
], ids=lambda c: c[0])
def test_fp8_shapes(case):
    name, T, H, E, K, R, fmt, a, extra, split = case
    print(f"[parity] fp8 case={name}", flush=True)
    w = workloads.Workload(name, seed=91, num_tokens=T, hidden=H, num_experts=E, num_topk=K,
                           num_ranks=R, scales=True, routing="uniform", drop_rate=0.1,
                           payload="fp8",
                           scale_format="f32" if fmt == epl.EPL_SCALE_F32 else "ue8m0",
                           ranks_per_node=2)
    fp8_parity(w, fmt, alignment=a, extra_cap=extra, split=split)


# ----------------------------------------------------------- ragged shapes --

RAGGED = [
    # name, T, K, E, R, H, scales, drop
    ("ragged_tail_h264", 1001, 5, 24, 6, 264, False, 0.1),
    ("two_passes_h9000", 333, 3, 16, 4, 9000, False, 0.0),
    ("scales_s70", 517, 4, 32, 8, 8960, True, 0.05),
    ("scales_s3", 250, 6, 40, 10, 384, True, 0.2),
    ("k64_e128", 100, 64, 128, 16, 64, False, 0.1),
    ("e2048_r2048", 300, 8, 2048, 2048, 64, False, 0.0),
    ("r1", 700, 8, 64, 1, 128, False, 0.0),
    ("k1", 900, 1, 8, 8, 136, False, 0.0),
    ("e1", 64, 1, 1, 1, 8, False, 0.3),
    ("r_not_mult16", 400, 4, 36, 12, 96, False, 0.0),
    # 8192 tokens and more: the combine's other unit count and the scatter's
    # one-workgroup-per-token grid, with ragged rows
    ("many_tokens_h264", 9000, 5, 24, 6, 264, False, 0.1),
    ("many_tokens_scales_s9", 8500, 4, 32, 8, 1152, True, 0.05),
    # the widest expert count and the largest top-k over many layout blocks:
    # 64 blocks of 141 tokens in 256-thread workgroups with a 2048-expert
    # count matrix (the scan's serial column reduce), and 282 blocks of 32
    # tokens of 64 slots each in 1024-thread workgroups
    ("e2048_many_tokens", 9000, 8, 2048, 256, 64, False, 0.1),
    ("k64_many_tokens", 9000, 64, 512, 64, 8, False, 0.1),
    # the single-workgroup layout + scan holds at most 2048 slots: at the
    # limit, and one token past it (the two-launch layout)
    ("fused_limit_2048_slots", 256, 8, 256, 32, 128, False, 0.1),
    ("fused_limit_plus_one_token", 257, 8, 256, 32, 128, False, 0.1),
    # 4096 .. 8191 tokens: each scatter workgroup strides over several
    # tokens (4 to 16), with uneven token counts per workgroup
    ("striding_ragged_h264", 5555, 5, 24, 6, 264, False, 0.1),
    ("striding_scales_s9", 7000, 4, 32, 8, 1152, True, 0.05),
    # decode-sized batches of long rows: fewer tokens than the striding grid,
    # each row cut into column parts (7 at hidden 7168, 8 at hidden 8960, 3
    # of 134, 134 and 132 vectors at hidden 3200); scale rows and indices
    # are written by the first part only
    ("decode_t256_dsv3", 256, 8, 256, 32, 7168, True, 0.0),
    ("decode_t100_dsv3_drop", 100, 8, 256, 32, 7168, True, 0.1),
    ("decode_t37_ragged_parts", 37, 4, 16, 4, 3200, True, 0.2),
    ("decode_t500_h8960", 500, 4, 32, 8, 8960, True, 0.05),
    # the largest top-k in a one-launch dispatch: 32 tokens x 64 slots
    ("decode_k64_2048_slots", 32, 64, 128, 16, 256, True, 0.1),
]


@pytest.mark.parametrize("case", RAGGED, ids=[c[0] for c in RAGGED])
def test_ragged_shapes(case):
    name, T, K, E, R, H, scales, drop = case
    print(f"[parity] ragged case={name}", flush=True)
    w = workloads.Workload(name, seed=77, num_tokens=T, hidden=H, num_experts=E, num_topk=K,
                           num_ranks=R, scales=scales, routing="uniform", drop_rate=drop)
    full_parity(w)


def test_more_tokens_than_the_largest_grid():
    """2^22 + 777 tokens: the row kernels' grids stop at 2^22 workgroups and
    the scatter and combine stride over the rest; the layout has 16 K blocks,
    so the scan sums columns longer than a thread holds."""
    print("[parity] 2^22 + 777 tokens, hidden 8", flush=True)
    w = workloads.Workload("grid_stride", seed=91, num_tokens=(1 << 22) + 777, hidden=8,
                           num_experts=16, num_topk=2, num_ranks=4, scales=False,
                           routing="uniform", drop_rate=0.1)
    full_parity(w)


# ------------------------------------------------- tokens per node (RDMA) --

# (name, E, R, G, T, K): one node (not produced), one rank per node (equals
# the per-rank counts), more than 64 nodes (two mask windows), and the
# largest column count the scan handles (2048 ranks + 2048 nodes).
NODES = [
    ("g1", 16, 8, 1, 500, 3),
    ("dsv3_like_g4", 256, 32, 4, 4096, 8),
    ("nodes128", 256, 256, 2, 5000, 8),
    ("r2048_g1", 2048, 2048, 1, 3000, 8),
    ("r2048_g8", 2048, 2048, 8, 3000, 8),
    ("one_node", 64, 64, 64, 100, 4),
    ("g_above_r", 64, 16, 32, 100, 4),
]


@pytest.mark.parametrize("case", NODES, ids=[c[0] for c in NODES])
def test_tokens_per_node(case):
    name, E, R, G, T, K = case
    print(f"[parity] nodes case={name}", flush=True)
    w = workloads.Workload(name, seed=91, num_tokens=T, hidden=64, num_experts=E, num_topk=K,
                           num_ranks=R, scales=False, routing="uniform", drop_rate=0.1,
                           ranks_per_node=G)
    r, _ = full_parity(w)
    if G == 1:
        assert torch.equal(r["per_node"], r["per_rank"])


@pytest.mark.parametrize("T,split", [(700, False), (3000, False), (6000, True)])
def test_receive_side_mid_sizes(T, split):
    """Receive-side batches of a few thousand tokens (local ids, about one
    valid slot in eight): the long-row scatter keeps its whole grid for such
    sparse routing; full parity, fused and split."""
    print(f"[parity] receive side T={T} split={split}", flush=True)
    full_parity(workloads.get("dsv3_recv").with_(num_tokens=T), split=split)


@pytest.mark.parametrize("name,T,split,want", [
    ("dsv3", 2048, False, 1), ("dsv3", 2048, True, 1), ("dsv3_recv", 3000, False, 0),
    ("dsv3_recv", 3000, True, 0), ("dsv3", 64, False, 1), ("dsv3_recv", 100, True, 0)])
def test_dense_hint_recorded_by_the_layout(name, T, split, want):
    """The routing-density hint in the workspace header (its third word): 1
    when at least half of the first 64 slots name an expert, as in a global
    dispatch, 0 for a receive side's mostly -1 local ids; written by the
    layout kernel, by the one-workgroup layout + scan and by the one-launch
    decode dispatch alike."""
    w = workloads.get(name).with_(num_tokens=T)
    inp = workloads.make_inputs(w)
    topk = inp["topk_idx"]
    first = topk.reshape(-1)[:64]
    assert (2 * int((first >= 0).sum()) >= len(first)) == bool(want)
    r = gpu_dispatch(topk, inp["x"], inp["x_scale"], w.num_experts, w.num_ranks, split=split,
                     G=w.ranks_per_node)
    torch.cuda.synchronize()
    assert epl.epl_status(r["ws"]) == epl.EPL_OK
    assert int(r["ws"][8:12].view(torch.int32)[0]) == want


@pytest.mark.parametrize("dense_first", [True, False])
def test_dense_hint_from_an_unrepresentative_first_block(dense_first):
    """The scatter's grid follows the routing density of the batch's first
    slots only; a batch whose first tokens are dense and the rest sparse (or
    the reverse) must still be placed exactly, whichever grid runs."""
    print(f"[parity] density hint, dense first block={dense_first}", flush=True)
    rng = np.random.default_rng(77 if dense_first else 78)
    T, K, E, R, H = 3000, 8, 64, 8, 7168
    topk = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64)
    sparse = rng.random(topk.shape) < 0.9
    head = np.arange(T)[:, None] < 200
    topk[(sparse & ~head) if dense_first else (sparse & head)] = -1
    _edge(topk, E, R, H=H, scales=True, seed=5)


def test_receive_side_is_the_global_buffer_restricted():
    """The batch of rank 3 with local ids, dispatched on the GPU, reproduces
    the stretch of rank 3's experts in the GPU's global buffer."""
    w = workloads.get("dsv3").with_(num_tokens=3000, drop_rate=0.05)
    inp = workloads.make_inputs(w)
    topk, x, xs = inp["topk_idx"], inp["x"], inp["x_scale"]
    El, r = w.num_experts // w.num_ranks, 3
    g = gpu_dispatch(topk, x, xs, w.num_experts, w.num_ranks, G=w.ranks_per_node)
    mine = (topk >= r * El) & (topk < (r + 1) * El)
    keep = np.nonzero(mine.any(axis=1))[0]
    lt = np.ascontiguousarray(np.where(mine[keep], topk[keep] - r * El, -1))
    loc = gpu_dispatch(lt, x[keep], xs[keep], El, 1)
    torch.cuda.synchronize()
    assert epl.epl_status(g["ws"]) == epl.EPL_OK and epl.epl_status(loc["ws"]) == epl.EPL_OK
    lo = int(g["start"][r * El])
    n = int(loc["total_host"][0])
    assert n == int(g["start"][(r + 1) * El]) - lo
    assert torch.equal(loc["out"][:n].view(torch.int16), g["out"][lo:lo + n].view(torch.int16))
    assert torch.equal(loc["out_scale"][:n], g["out_scale"][lo:lo + n])
    assert torch.equal(loc["m"][:n] + r * El, g["m"][lo:lo + n])
    want_oi = np.where(lt >= 0, g["oi"].cpu().numpy()[keep] - lo, -1)
    np.testing.assert_array_equal(loc["oi"].cpu().numpy(), want_oi)


# ------------------------------------------------------------- edge cases --

def _mk(topk, H=64, seed=0, scales=False):
    rng = np.random.default_rng(seed)
    T = topk.shape[0]
    x = workloads.fp32_to_bf16_bits(rng.standard_normal((T, H), dtype=np.float32))
    xs = rng.uniform(0.01, 1, (T, H // 128)).astype(np.float32) if scales else None
    wt = rng.uniform(0, 1, topk.shape).astype(np.float32)
    return x, xs, wt


def _edge(topk, E, R, H=64, scales=False, seed=0):
    x, xs, wt = _mk(topk, H, seed, scales)
    ref = orc().run_all(x, xs, topk, wt, E, R)
    r = gpu_dispatch(topk, x, xs, E, R)
    assert epl.epl_status(r["ws"]) == epl.EPL_OK
    check_layout_and_scatter(r, ref, x, xs)
    y = gpu_combine(r, r["out"], wt, epl.EPL_OUT_F32)
    check_combine_f32(y.cpu().numpy(), ref["y"], combine_bound(ref["expert_out"],
                                                                ref["output_index"], wt))
    return r, ref, y


def test_zero_tokens():
    topk = np.zeros((0, 4), np.int64)
    r, ref, y = _edge(topk, 16, 4)
    assert ref["total"] == 0 and y.shape == (0, 64)


def test_all_slots_invalid():
    topk = -np.ones((300, 4), np.int64)
    r, ref, y = _edge(topk, 16, 4)
    assert (r["oi"] == -1).all() and (y == 0).all()
    # the sum starts from +0: every bit of y is clear, also in bf16
    assert (y.view(torch.int32) == 0).all()
    yb = gpu_combine(r, r["out"], np.ones((300, 4), np.float32), epl.EPL_OUT_BF16)
    assert (u16(yb) == 0).all()


def test_non_finite_rows_propagate_like_the_oracle():
    """NaN and +-Inf in expert rows are summed like any value: y is NaN, +Inf
    or -Inf exactly where the oracle's fp64 sum is (0 * Inf gives NaN on both
    sides), and the finite elements stay within the tolerance."""
    rng = np.random.default_rng(12)
    T, K, E, R, H = 400, 4, 16, 4, 64
    topk = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64)
    x, _, wt = _mk(topk, H, seed=12)
    wt[rng.random(wt.shape) < 0.05] = 0.0               # some zero weights meet an Inf
    specials = np.array([0x7FC0, 0x7F80, 0xFF80], np.uint16)   # NaN, +Inf, -Inf
    hit = rng.random(x.shape) < 0.01
    x[hit] = specials[rng.integers(0, 3, int(hit.sum()))]
    ref = orc().run_all(x, None, topk, wt, E, R)
    r = gpu_dispatch(topk, x, None, E, R)
    assert epl.epl_status(r["ws"]) == epl.EPL_OK
    check_layout_and_scatter(r, ref, x, None)
    y = gpu_combine(r, r["out"], wt, epl.EPL_OUT_F32).cpu().numpy().astype(np.float64)
    yr = ref["y"]
    assert np.isnan(yr).any() and np.isinf(yr).any()
    np.testing.assert_array_equal(np.isnan(y), np.isnan(yr))
    np.testing.assert_array_equal(np.isposinf(y), np.isposinf(yr))
    np.testing.assert_array_equal(np.isneginf(y), np.isneginf(yr))
    fin = np.isfinite(yr)
    bound = combine_bound(ref["expert_out"], ref["output_index"], wt)
    assert (np.abs(y[fin] - yr[fin]) <= 1e-5 * bound[fin]).all()
    # bf16 output: NaN stays NaN, infinities stay infinite with their sign
    yb = u16(gpu_combine(r, r["out"], wt, epl.EPL_OUT_BF16))
    ybf = (yb.astype(np.uint32) << 16).view(np.float32)
    np.testing.assert_array_equal(np.isnan(ybf), np.isnan(yr))
    np.testing.assert_array_equal(np.isposinf(ybf), np.isposinf(yr))
    np.testing.assert_array_equal(np.isneginf(ybf), np.isneginf(yr))


def test_duplicate_experts_within_a_token():
    rng = np.random.default_rng(5)
    topk = rng.integers(-1, 4, size=(500, 6)).astype(np.int64)
    _edge(topk, 4, 2)


def test_k1_weight1_returns_x_exactly():
    rng = np.random.default_rng(6)
    T, H = 777, 256
    topk = rng.integers(0, 32, size=(T, 1)).astype(np.int64)
    x, _, _ = _mk(topk, H)
    r = gpu_dispatch(topk, x, None, 32, 8)
    y = gpu_combine(r, r["out"], np.ones((T, 1), np.float32), epl.EPL_OUT_F32)
    yb = gpu_combine(r, r["out"], np.ones((T, 1), np.float32), epl.EPL_OUT_BF16)
    xf = (x.astype(np.uint32) << 16).view(np.float32)
    np.testing.assert_array_equal(y.cpu().numpy(), xf)
    np.testing.assert_array_equal(u16(yb), x)


def test_out_of_range_ids_flagged_and_ignored():
    rng = np.random.default_rng(7)
    E, R = 16, 4
    topk = rng.integers(-1, E, size=(400, 3)).astype(np.int64)
    topk[3, 1] = E
    topk[77, 0] = 1 << 40
    topk[200, 2] = -5
    x, xs, wt = _mk(topk)
    clean = np.where((topk < -1) | (topk >= E), -1, topk)
    ref = orc().run_all(x, xs, clean, wt, E, R)
    r = gpu_dispatch(topk, x, xs, E, R)
    assert epl.epl_status(r["ws"]) == epl.EPL_ERANGE
    check_layout_and_scatter(r, ref, x, xs)
    # the status resets on the next layout over clean ids
    r2 = gpu_dispatch(clean, x, xs, E, R)
    assert epl.epl_status(r2["ws"]) == epl.EPL_OK


def test_capacity_overflow_flagged_without_out_of_bounds_writes():
    rng = np.random.default_rng(8)
    E, R, T, K, H = 8, 2, 200, 4, 64
    topk = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64)
    x, _, wt = _mk(topk, H)
    ref = orc().run_all(x, None, topk, wt, E, R)
    N = ref["total"]
    cap, guard = N - 37, 64
    p = epl.Problem.make(T, K, E, R, H, 0)
    ws = poisoned(epl.epl_workspace_bytes(p), torch.uint8)
    out_full = poisoned((cap + guard, H), torch.bfloat16)
    m_full = poisoned(cap + guard, torch.int32)
    out, m = out_full[:cap], m_full[:cap]
    cnt, per_rank = poisoned(E, torch.int32), poisoned(R, torch.int32)
    in_rank, start = poisoned((T, R), torch.uint8), poisoned(E, torch.int32)
    oi = poisoned((T, K), torch.int32)
    epl.epl_dispatch(p, torch.from_numpy(topk).to(DEV), to_bf16(x), None, cap, cnt, per_rank,
                     None, in_rank, start, None, out, None, m, oi, ws)
    assert epl.epl_status(ws) == epl.EPL_ECAPACITY
    # slots whose rows fall past the capacity are not placed: output_index -1
    # (the marker of an unplaced slot), never a row id outside the buffer
    want_oi = np.where(ref["output_index"] >= cap, -1, ref["output_index"])
    np.testing.assert_array_equal(oi.cpu().numpy(), want_oi)
    assert (ref["output_index"] >= cap).sum() == 37
    np.testing.assert_array_equal(u16(out), ref["out"][:cap])
    np.testing.assert_array_equal(m.cpu().numpy(), ref["m_indices"][:cap])
    assert (out_full[cap:].view(torch.uint8) == POISON).all()
    assert (m_full[cap:].view(torch.uint8) == POISON).all()


def test_combine_flags_row_beyond_expert_output():
    T, K, H = 10, 2, 64
    rng = np.random.default_rng(9)
    eo = workloads.fp32_to_bf16_bits(rng.standard_normal((20, H), dtype=np.float32))
    oi = rng.integers(-1, 20, size=(T, K)).astype(np.int32)
    oi[4, 1] = 20
    wt = rng.uniform(0, 1, (T, K)).astype(np.float32)
    p = epl.Problem.make(T, K, 4, 2, H, 0)
    ws = poisoned(epl.epl_workspace_bytes(p), torch.uint8)
    # a clean layout resets the status word
    epl.epl_layout(p, torch.zeros((T, K), dtype=torch.int64, device=DEV),
                   poisoned(4, torch.int32), poisoned(2, torch.int32), None,
                   poisoned((T, 2), torch.uint8), ws)
    y = poisoned((T, H), torch.float32)
    epl.epl_combine(p, to_bf16(eo), 20, torch.from_numpy(oi).to(DEV),
                    torch.from_numpy(wt).to(DEV), epl.EPL_OUT_F32, y, ws)
    assert epl.epl_status(ws) == epl.EPL_ERANGE
    clean = np.where(oi >= 20, -1, oi)
    y_ref = orc().combine(eo, clean, wt)
    check_combine_f32(y.cpu().numpy(), y_ref, combine_bound(eo, clean, wt))


@pytest.mark.parametrize("alignment", [0, 64])
def test_exact_mode_matches_capacity_mode(alignment):
    w = workloads.get("small").with_(num_tokens=1200)
    inp = workloads.make_inputs(w)
    tk = torch.from_numpy(inp["topk_idx"]).to(DEV)
    xd = to_bf16(inp["x"])
    a = epl.dispatch(xd, tk, w.num_experts, w.num_ranks, mode="capacity",
                     expert_alignment=alignment)
    b = epl.dispatch(xd, tk, w.num_experts, w.num_ranks, mode="exact",
                     expert_alignment=alignment)
    n = a.total()
    assert n == b.total() == b.out.shape[0]
    assert torch.equal(a.output_index, b.output_index)
    assert torch.equal(a.m_indices[:n], b.m_indices)
    real = b.m_indices >= 0
    assert torch.equal(a.out[:n][real].view(torch.int16), b.out[real].view(torch.int16))


def test_runs_on_a_side_stream():
    w = workloads.get("small").with_(num_tokens=800)
    inp = workloads.make_inputs(w)
    ref = orc().run_all(inp["x"], None, inp["topk_idx"], inp["topk_weights"], w.num_experts,
                        w.num_ranks)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        r = gpu_dispatch(inp["topk_idx"], inp["x"], None, w.num_experts, w.num_ranks)
        y = gpu_combine(r, r["out"], inp["topk_weights"], epl.EPL_OUT_F32)
    s.synchronize()
    check_layout_and_scatter(r, ref, inp["x"], None)
    check_combine_f32(y.cpu().numpy(), ref["y"],
                      combine_bound(ref["out"], ref["output_index"], inp["topk_weights"]))


def test_concurrent_dispatches_on_three_streams():
    """Three problems dispatched and combined at the same time on three
    streams, each with its own workspace and buffers: 2048 DSV3-shaped
    tokens (the scatter doing the scan's work on the dense grid), a receive
    side of 3000 tokens (sparse routing, the whole grid) and 64 DSV3-shaped
    tokens (the one-launch dispatch). Each must match the oracle exactly as
    when it runs alone: the library keeps no device state of its own
    between calls."""
    cases = [workloads.get("dsv3").with_(num_tokens=2048),
             workloads.get("dsv3_recv").with_(num_tokens=3000),
             workloads.get("dsv3").with_(num_tokens=64)]
    inps = [workloads.make_inputs(w) for w in cases]
    refs = []
    for w, i in zip(cases, inps):
        assert w.expert_fn == "identity"
        refs.append(orc().run_all(i["x"], i["x_scale"], i["topk_idx"], i["topk_weights"],
                                  w.num_experts, w.num_ranks))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in cases]
    runs = []
    for w, i, s in zip(cases, inps, streams):
        with torch.cuda.stream(s):
            r = gpu_dispatch(i["topk_idx"], i["x"], i["x_scale"], w.num_experts, w.num_ranks,
                             G=w.ranks_per_node)
            y = gpu_combine(r, r["out"], i["topk_weights"], epl.EPL_OUT_F32)
        runs.append((r, y))
    for s in streams:
        s.synchronize()
    for (r, y), i, ref in zip(runs, inps, refs):
        assert epl.epl_status(r["ws"]) == epl.EPL_OK
        check_layout_and_scatter(r, ref, i["x"], i["x_scale"])
        check_combine_f32(y.cpu().numpy(), ref["y"],
                          combine_bound(ref["expert_out"], ref["output_index"],
                                        i["topk_weights"]))


# ----------------------------------------------------- randomized sweep --

def _sweep_shape(rng):
    """One seeded random problem: token count log-uniform in [1, 3000], any
    top-k up to 16, ranks and experts per rank, hidden widths (multiples of
    128 when there are scales), -1 rates, duplicate experts within a token,
    expert alignment, ranks per node, split or fused calls."""
    R = int(rng.choice([1, 2, 3, 4, 8, 16, 32]))
    E = R * int(rng.choice([1, 2, 3, 5, 8]))
    K = int(rng.integers(1, 17))
    T = int(np.exp(rng.uniform(0, np.log(3000))))
    scales = bool(rng.random() < 0.4)
    H = 128 * int(rng.integers(1, 33)) if scales else 8 * int(rng.integers(1, 400))
    a = int(rng.choice([0, 0, 1, 2, 7, 16, 64]))
    G = int(rng.choice([0, 1, max(1, R // 2), R])) if R > 1 else 0
    if G and R % G:
        G = 0
    drop = float(rng.choice([0.0, 0.1, 0.5]))
    dup = bool(rng.random() < 0.3)
    split = bool(rng.random() < 0.3)
    if dup:   # ids drawn with replacement: a token may pick an expert twice
        topk = rng.integers(0, E, size=(T, K)).astype(np.int64)
    else:
        topk = np.stack([rng.permutation(E)[:K] if K <= E else rng.integers(0, E, K)
                         for _ in range(T)]).astype(np.int64)
    topk[rng.random(topk.shape) < drop] = -1
    return dict(T=T, K=K, E=E, R=R, H=H, scales=scales, a=a, G=G, split=split, topk=topk)


@pytest.mark.parametrize("seed", range(40))
def test_random_shape_sweep(seed):
    """40 seeded random problems through epl_dispatch (or the split calls)
    against the oracle: counts, masks, per-node counts, offsets, every row,
    scale row and index bit-exact; padding rows marked; combine within 1e-5
    of sum |w v| (fp32) and the bf16 output the RNE of it."""
    rng = np.random.default_rng(5000 + seed)
    c = _sweep_shape(rng)
    T, K, E, R, H = c["T"], c["K"], c["E"], c["R"], c["H"]
    print(f"[parity] sweep seed={seed} T={T} K={K} E={E} R={R} H={H} scales={c['scales']} "
          f"a={c['a']} G={c['G']} split={c['split']}", flush=True)
    x, xs, wt = _mk(c["topk"], H, seed, c["scales"])
    ref = orc().run_all(x, xs, c["topk"], wt, E, R, alignment=c["a"])
    r = gpu_dispatch(c["topk"], x, xs, E, R, split=c["split"], alignment=c["a"], G=c["G"])
    assert epl.epl_status(r["ws"]) == epl.EPL_OK
    check_layout_and_scatter(r, ref, x, xs)
    y = gpu_combine(r, r["out"], wt, epl.EPL_OUT_F32)
    yb = gpu_combine(r, r["out"], wt, epl.EPL_OUT_BF16)
    bound = combine_bound(ref["expert_out"], ref["output_index"], wt)
    check_combine_f32(y.cpu().numpy(), ref["y"], bound)
    check_bf16_is_rne_of_f32(u16(yb), y.cpu())


def _long_row_shape(rng, seed):
    """One seeded problem on the long-row striding grid (bf16 rows of 12 KB
    or more, 512 to 2500 tokens): routing density from every slot valid
    down to a receive side's few, and sometimes a first block whose density
    is the opposite of the rest, so that either active grid the layout's
    sample picks meets either kind of batch. The seed fixes the mix: the
    drop rate cycles over four values and seeds 8 to 11 invert the head."""
    R = int(rng.choice([1, 4, 8, 32]))
    E = R * int(rng.choice([1, 2, 8]))
    K = int(rng.integers(1, 9))
    T = int(np.exp(rng.uniform(np.log(512), np.log(2500))))
    scales = bool(rng.random() < 0.5)
    H = 128 * int(rng.integers(48, 65)) if scales else 8 * int(rng.integers(768, 1025))
    a = int(rng.choice([0, 0, 1, 16, 64]))
    G = int(rng.choice([0, max(1, R // 4), R])) if R > 1 else 0
    if G and R % G:
        G = 0
    drop = (0.0, 0.5, 0.875, 0.97)[seed % 4]
    split = bool(rng.random() < 0.3)
    topk = np.stack([rng.permutation(E)[:K] if K <= E else rng.integers(0, E, K)
                     for _ in range(T)]).astype(np.int64)
    gone = rng.random(topk.shape) < drop
    if seed >= 8:   # the first 64 tokens routed unlike the rest
        head = np.arange(T)[:, None] < 64
        gone = np.where(head, rng.random(topk.shape) < (0.9 if drop < 0.5 else 0.0), gone)
    topk[gone] = -1
    return dict(T=T, K=K, E=E, R=R, H=H, scales=scales, a=a, G=G, split=split, topk=topk)


@pytest.mark.parametrize("seed", range(12))
def test_random_long_row_sweep(seed):
    """12 seeded problems on the long-row grid, whose active size follows
    the density of the batch's first slots: every index, row and scale row
    bit-exact against the oracle and the fp32 combine within 1e-5 of
    sum |w v|, whichever grid ran."""
    rng = np.random.default_rng(11000 + seed)
    c = _long_row_shape(rng, seed)
    T, K, E, R, H = c["T"], c["K"], c["E"], c["R"], c["H"]
    # The hint samples the first min(64, slots of the first layout block)
    # slots, a block holding 16 tokens or more; where every such window
    # gives the same answer, the hint must be that answer.
    valid = np.cumsum(c["topk"].reshape(-1)[:64] >= 0)
    votes = {bool(2 * valid[n - 1] >= n) for n in range(min(64, 16 * K), 65)}
    print(f"[parity] long-row sweep seed={seed} T={T} K={K} E={E} R={R} H={H} "
          f"scales={c['scales']} a={c['a']} G={c['G']} split={c['split']} dense={votes}",
          flush=True)
    x, xs, wt = _mk(c["topk"], H, seed, c["scales"])
    ref = orc().run_all(x, xs, c["topk"], wt, E, R, alignment=c["a"])
    r = gpu_dispatch(c["topk"], x, xs, E, R, split=c["split"], alignment=c["a"], G=c["G"])
    assert epl.epl_status(r["ws"]) == epl.EPL_OK
    hint = int(r["ws"][8:12].view(torch.int32)[0])
    assert hint in (0, 1)
    if len(votes) == 1:
        assert hint == int(votes.pop())
    check_layout_and_scatter(r, ref, x, xs)
    y = gpu_combine(r, r["out"], wt, epl.EPL_OUT_F32)
    bound = combine_bound(ref["expert_out"], ref["output_index"], wt)
    check_combine_f32(y.cpu().numpy(), ref["y"], bound)


@pytest.mark.parametrize("seed", range(12))
def test_random_fp8_sweep(seed):
    """12 seeded random FP8 problems (no scales, fp32 rows of scales, or
    transposed UE8M0 words), fused or split, with or without alignment and
    spare capacity, against the oracle's byte-row scatter."""
    rng = np.random.default_rng(7000 + seed)
    R = int(rng.choice([1, 2, 4, 8]))
    E = R * int(rng.choice([1, 3, 8]))
    K = int(rng.integers(1, min(E, 12) + 1))
    T = int(np.exp(rng.uniform(0, np.log(3000))))
    H = 128 * int(rng.integers(1, 40))
    fmt = int(rng.choice([epl.EPL_SCALE_NONE, epl.EPL_SCALE_F32, epl.EPL_SCALE_UE8M0]))
    a = int(rng.choice([0, 8, 32]))
    extra = int(rng.choice([0, 0, 13]))
    split = bool(rng.random() < 0.4)
    print(f"[parity] fp8 sweep seed={seed} T={T} K={K} E={E} R={R} H={H} fmt={fmt} a={a} "
          f"extra={extra} split={split}", flush=True)
    w = workloads.Workload(f"sweep{seed}", seed=9000 + seed, num_tokens=T, hidden=H,
                           num_experts=E, num_topk=K, num_ranks=R, scales=True,
                           routing="uniform", drop_rate=0.1, payload="fp8",
                           scale_format="f32" if fmt == epl.EPL_SCALE_F32 else "ue8m0",
                           ranks_per_node=0)
    fp8_parity(w, fmt, alignment=a, extra_cap=extra, split=split)


# ------------------------------------ dispatch without a scan launch --

# Dispatches of several layout blocks whose per-block count matrix is small
# (at most 16384 words) and whose scatter runs a striding grid of at most
# 1024 workgroups do the scan inside the scatter: every scatter workgroup
# reduces the per-block counts itself. (T, K, E, R, H): 1500 tokens of
# 128-byte rows take the XCD-aware grid of 1024 workgroups; 1001 tokens take
# a grid of 1001, whose token ranges span every layout block.
NO_SCAN = [("xcd_grid", 1500, 4, 32, 8, 64), ("plain_grid", 1001, 4, 32, 8, 64),
           ("dsv3_like", 4096, 8, 256, 32, 128)]


@pytest.mark.parametrize("case", NO_SCAN, ids=[c[0] for c in NO_SCAN])
def test_scan_in_scatter_flags_bad_ids_then_resets(case):
    """Out-of-range ids set EPL_ERANGE (the bits come from the layout blocks
    through the scatter) and the next dispatch over clean ids on the same
    workspace clears it again."""
    name, T, K, E, R, H = case
    print(f"[parity] scan-in-scatter bad ids case={name}", flush=True)
    rng = np.random.default_rng(31)
    topk = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64)
    topk[rng.random(topk.shape) < 0.05] = -1
    bad = topk.copy()
    bad[3, 1] = E
    bad[T - 2, 0] = 1 << 40
    bad[T // 2, K - 1] = -5
    x, xs, wt = _mk(topk, H, scales=H % 128 == 0)
    clean = np.where((bad < -1) | (bad >= E), -1, bad)
    ref = orc().run_all(x, xs, clean, wt, E, R)
    r = gpu_dispatch(bad, x, xs, E, R)
    assert epl.epl_status(r["ws"]) == epl.EPL_ERANGE
    check_layout_and_scatter(r, ref, x, xs)
    tk = torch.from_numpy(clean).to(DEV)
    epl.epl_dispatch(r["p"], tk, r["x"], None if xs is None else torch.from_numpy(xs).to(DEV),
                     r["cap"], r["cnt"], r["per_rank"], r["per_node"], r["in_rank"], r["start"],
                     r["total_host"], r["out"], r["out_scale"], r["m"], r["oi"], r["ws"])
    assert epl.epl_status(r["ws"]) == epl.EPL_OK
    check_layout_and_scatter(r, ref, x, xs)


@pytest.mark.parametrize("alignment", [0, 16])
@pytest.mark.parametrize("case", NO_SCAN[:2], ids=[c[0] for c in NO_SCAN[:2]])
def test_scan_in_scatter_capacity_overflow(case, alignment):
    """Rows (and alignment padding rows) past a short buffer are skipped and
    flagged, unplaced slots get output_index -1, nothing is written past the
    buffer, and N still reaches the host."""
    name, T, K, E, R, H = case
    print(f"[parity] scan-in-scatter overflow case={name} a={alignment}", flush=True)
    rng = np.random.default_rng(32)
    topk = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64)
    x, _, wt = _mk(topk, H)
    ref = orc().run_all(x, None, topk, wt, E, R, alignment=alignment)
    N = ref["total"]
    cap, guard = N - 37, 64
    p = epl.Problem.make(T, K, E, R, H, 0, alignment)
    ws = poisoned(epl.epl_workspace_bytes(p), torch.uint8)
    out_full = poisoned((cap + guard, H), torch.bfloat16)
    m_full = poisoned(cap + guard, torch.int32)
    out, m = out_full[:cap], m_full[:cap]
    cnt, per_rank = poisoned(E, torch.int32), poisoned(R, torch.int32)
    in_rank, start = poisoned((T, R), torch.uint8), poisoned(E, torch.int32)
    oi = poisoned((T, K), torch.int32)
    total_host = torch.full((1,), -7, dtype=torch.int32).pin_memory()
    epl.epl_dispatch(p, torch.from_numpy(topk).to(DEV), to_bf16(x), None, cap, cnt, per_rank,
                     None, in_rank, start, total_host, out, None, m, oi, ws)
    assert epl.epl_status(ws) == epl.EPL_ECAPACITY
    assert int(total_host[0]) == N and epl.epl_total(ws) == N
    np.testing.assert_array_equal(start.cpu().numpy(), ref["expert_start_loc"])
    np.testing.assert_array_equal(cnt.cpu().numpy(), ref["num_tokens_per_expert"])
    want_oi = np.where(ref["output_index"] >= cap, -1, ref["output_index"])
    np.testing.assert_array_equal(oi.cpu().numpy(), want_oi)
    np.testing.assert_array_equal(m.cpu().numpy(), ref["m_indices"][:cap])
    real = ref["m_indices"][:cap] >= 0
    np.testing.assert_array_equal(u16(out)[real], ref["out"][:cap][real])
    assert (out_full[cap:].view(torch.uint8) == POISON).all()
    assert (m_full[cap:].view(torch.uint8) == POISON).all()


# Decode-sized batches (at most 2048 slots) dispatch in one launch whose
# token workgroups place their own slots.
ONE_LAUNCH = [("decode_narrow", 300, 4, 32, 8, 64), ("decode_dsv3", 64, 8, 256, 32, 128)]


@pytest.mark.parametrize("alignment", [0, 32])
@pytest.mark.parametrize("case", NO_SCAN + ONE_LAUNCH, ids=[c[0] for c in NO_SCAN + ONE_LAUNCH])
def test_scatter_after_dispatch_reuses_its_workspace(case, alignment):
    """A dispatch that ran no scan launch (or placed its slots in the
    scatter's own workgroups) leaves the workspace as layout + scan would: a
    later epl_scatter of another payload with the same routing, workspace
    and expert_start_loc places it exactly as the oracle does."""
    name, T, K, E, R, H = case
    print(f"[parity] scatter after dispatch case={name} a={alignment}", flush=True)
    rng = np.random.default_rng(33)
    topk = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64)
    topk[rng.random(topk.shape) < 0.05] = -1
    x, xs, wt = _mk(topk, H, seed=1, scales=H % 128 == 0)
    x2, xs2, _ = _mk(topk, H, seed=2, scales=H % 128 == 0)
    r = gpu_dispatch(topk, x, xs, E, R, alignment=alignment)
    assert epl.epl_status(r["ws"]) == epl.EPL_OK
    ref2 = orc().run_all(x2, xs2, topk, wt, E, R, alignment=alignment)
    cap = r["cap"]
    out2 = poisoned((cap, H), torch.bfloat16)
    os2 = poisoned((cap, xs2.shape[1]), torch.float32) if xs2 is not None else None
    m2, oi2 = poisoned(cap, torch.int32), poisoned((T, K), torch.int32)
    epl.epl_scatter(r["p"], to_bf16(x2), None if xs2 is None else torch.from_numpy(xs2).to(DEV),
                    r["topk"], r["start"], r["ws"], cap, out2, os2, m2, oi2)
    assert epl.epl_status(r["ws"]) == epl.EPL_OK
    r2 = dict(r, out=out2, out_scale=os2, m=m2, oi=oi2)
    check_layout_and_scatter(r2, ref2, x2, xs2)
