"""Planted mistakes: each copy of the oracle below carries one plausible bug
(a dropped term, a wrong sign or index, a transposed operand, an off-by-one)
and must fail at least one pin. The mistakes are planted in a temporary copy
of the C source, on the CPU; the committed oracle is never modified. Each
mutant runs in its own process, because a mutant that writes out of bounds
may abort; an abort counts as a failed pin."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
from conftest import load_golden
from oracle import Oracle, OracleError
from test_oracle_pins import brute_force, tiny_group_pair

SRC = open(os.path.join(os.path.dirname(oracle.__file__), "epl_oracle.c"), encoding="utf-8").read()

MUTANTS = {
    "cursor_advances_by_two": ("cursor[e] += 1;", "cursor[e] += 2;"),
    "round_robin_owner": ("is_token_in_rank[t * R + e / experts_per_rank] = 1;",
                          "is_token_in_rank[t * R + e % R] = 1;"),
    "inclusive_scan": ("expert_start_loc[e] = (int32_t)running;\n        int64_t c = num_tokens_per_expert[e];\n        int64_t blocks = c / a + (c % a != 0);\n        running += blocks * a;",
                       "int64_t c = num_tokens_per_expert[e];\n        int64_t blocks = c / a + (c % a != 0);\n        running += blocks * a;\n        expert_start_loc[e] = (int32_t)running;"),
    "alignment_rounds_down": ("int64_t blocks = c / a + (c % a != 0);", "int64_t blocks = c / a;"),
    "alignment_always_one_extra_block": ("int64_t blocks = c / a + (c % a != 0);", "int64_t blocks = c / a + 1;"),
    "scale_words_row_major_in_cols_layout": ("out_scale[j * scale_ld + p] = x_scale[t * scale_words + j];",
                                             "out_scale[p * scale_words + j] = x_scale[t * scale_words + j];"),
    "scale_cols_leading_dim_is_total": ("out_scale[j * scale_ld + p] = x_scale[t * scale_words + j];",
                                        "out_scale[j * total_rows + p] = x_scale[t * scale_words + j];"),
    "byte_row_of_wrong_token": ("memcpy(out + p * row_bytes, x + t * row_bytes, (size_t)row_bytes);",
                                "memcpy(out + p * row_bytes, x + (T - 1 - t) * row_bytes, (size_t)row_bytes);"),
    "rows_invalid_slot_marked_zero": ("output_index[t * K + k] = -1;   /* no selection: no row */",
                                      "output_index[t * K + k] = 0;   /* no selection: no row */"),
    "rows_slots_in_reverse_k": ("for (int32_t k = 0; k < K; ++k) {   /* the token's slots in order */",
                                "for (int32_t k = K - 1; k >= 0; --k) {   /* the token's slots in order */"),
    "padding_marked_zero": ("for (int64_t p = 0; p < total_rows; ++p)\n        m_indices[p] = -1;\n    int64_t *cursor",
                            "for (int64_t p = 0; p < total_rows; ++p)\n        m_indices[p] = 0;\n    int64_t *cursor"),
    "rows_padding_marked_zero": ("m_indices[p] = -1;              /* rows without a slot: padding */",
                                 "m_indices[p] = 0;              /* rows without a slot: padding */"),
    "per_rank_counts_every_token": ("num_tokens_per_rank[r] += is_token_in_rank[t * R + r];",
                                    "num_tokens_per_rank[r] += 1;"),
    "weight_of_mirrored_slot": ("double w = (double)topk_weights[t * K + k];",
                                "double w = (double)topk_weights[t * K + (K - 1 - k)];"),
    "transposed_output_index": ("int64_t row = output_index[t * K + k];",
                                "int64_t row = output_index[k * T + t];"),
    "dropped_accumulator": ("yrow[h] = yrow[h] + w * epl_oracle_bf16_to_double(src[h]);",
                            "yrow[h] = w * epl_oracle_bf16_to_double(src[h]);"),
    "bf16_one_bit_short": ("int quantum = (e2 - 1) - 7;", "int quantum = (e2 - 1) - 6;"),
    "bf16_truncates": ("double q = nearbyint(ldexp(a, -quantum));",
                       "double q = floor(ldexp(a, -quantum));"),
    "bf16_ties_away": ("double q = nearbyint(ldexp(a, -quantum));",
                       "double q = round(ldexp(a, -quantum));"),
    "invalid_slot_marked_zero": ("output_index[t * K + k] = -1;\n                continue;",
                                 "output_index[t * K + k] = 0;\n                continue;"),
    "expert_factor_255": ("1.0 + (double)m_indices[p] / 256.0", "1.0 + (double)m_indices[p] / 255.0"),
    "slots_in_reverse_k": ("for (int32_t k = 0; k < K; ++k) {\n            int64_t e = topk_idx[t * K + k];\n            if (e < -1",
                           "for (int32_t k = K - 1; k >= 0; --k) {\n            int64_t e = topk_idx[t * K + k];\n            if (e < -1"),
    "rdma_nodes_strided": ("for (int32_t r = n * G; r < (n + 1) * G; ++r)",
                           "for (int32_t r = n; r < R; r += nodes)"),
    "rdma_counts_ranks_not_tokens": ("                    any = 1;", "                    ++tokens;"),
    "e4m3_truncates": ("double r = ldexp(nearbyint(ldexp(a, -quantum)), quantum);",
                       "double r = ldexp(floor(ldexp(a, -quantum)), quantum);"),
    "e4m3_four_mantissa_bits": ("int quantum = e2 - 4;", "int quantum = e2 - 5;"),
    "quant_amax_signed": ("float v = fabsf((float)epl_oracle_bf16_to_double(xg[i]));",
                          "float v = (float)epl_oracle_bf16_to_double(xg[i]);"),
    "quant_stores_inverse_scale": ("scale[t * (int64_t)S + g] = s;",
                                   "scale[t * (int64_t)S + g] = inv;"),
    "quant_inverse_in_binary32_range": (
        "double inv = amax > 0.0f ? round_to_24_bits(448.0 / (double)amax) : 0.0;",
        "double inv = amax > 0.0f ? (double)(448.0f / amax) : 0.0;"),
    "quant_product_not_rounded": (
        "double p = round_to_24_bits(epl_oracle_bf16_to_double(xg[i]) * inv);",
        "double p = epl_oracle_bf16_to_double(xg[i]) * inv;"),
    "ll_rows_without_expert_stride": ("int64_t row = e * cap + j;", "int64_t row = e + j;"),
    "ll_src_info_global_token": ("src_info[row] = (int32_t)(t - seg * M);",
                                 "src_info[row] = (int32_t)t;"),
    "ll_range_begin_inclusive": ("            layout_range[(e * nseg + s) * 2 + 0] = before;\n            before += layout_range[(e * nseg + s) * 2 + 1];",
                                 "            before += layout_range[(e * nseg + s) * 2 + 1];\n            layout_range[(e * nseg + s) * 2 + 0] = before;"),
    "ll_overflow_ignored": ("            if (j >= cap) {                    /* the rectangle is full */",
                            "            if (j >= cap + 1) {                    /* the rectangle is full */"),
    "scale_row_of_wrong_token": ("x_scale + t * (int64_t)S", "x_scale + (T - 1 - t) * (int64_t)S"),
}


def _build_mutant(tmp_path, name, find, repl):
    assert SRC.count(find) == 1, f"mutation {name}: pattern must occur exactly once"
    src = tmp_path / f"{name}.c"
    src.write_text(SRC.replace(find, repl), encoding="utf-8")
    lib = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fPIC", "-shared",
                    str(src), "-o", str(lib), "-lm"], check=True)
    return str(lib)


def _battery(orc: Oracle):
    """Quick pins, each as a boolean; returns the names of the pins that fail."""
    failed = []

    def pin(name, fn):
        try:
            if not fn():
                failed.append(name)
        except (OracleError, AssertionError, IndexError, ValueError):
            failed.append(name)

    def golden_scan():
        g = load_golden("scan_prefix_example.txt")
        start, total = orc.scan(np.array(g["counts"]))
        return start.tolist() == g["expert_start_loc"] and total == g["total"][0]

    def golden_hand():
        g = load_golden("scatter_hand_example.txt")
        E, R = g["num_experts"][0], g["num_ranks"][0]
        topk = np.array(g["topk_idx"], np.int64)
        cnt, per_rank, _ = orc.layout(topk, E, R)
        start, total = orc.scan(cnt)
        _, _, m, oi = orc.scatter(None, None, topk, start, total)
        return (oi.tolist() == g["output_index"] and m.tolist() == g["m_indices"]
                and per_rank.tolist() == g["num_tokens_per_rank"])

    def brute():
        rng = np.random.default_rng(99)
        for _ in range(30):
            R = int(rng.integers(1, 5))
            E = R * int(rng.integers(1, 5))
            T, K = int(rng.integers(1, 10)), int(rng.integers(1, 5))
            topk = rng.integers(-1, E, size=(T, K)).astype(np.int64)
            want = brute_force(topk, E, R)
            cnt, per_rank, in_rank = orc.layout(topk, E, R)
            start, total = orc.scan(cnt)
            _, _, m, oi = orc.scatter(None, None, topk, start, total)
            if not (np.array_equal(cnt, want["cnt"]) and np.array_equal(per_rank, want["per_rank"])
                    and np.array_equal(in_rank, want["in_rank"]) and np.array_equal(start, want["start"])
                    and np.array_equal(oi, want["oi"]) and np.array_equal(m, want["m"])):
                return False
        return True

    def rows_and_scales():
        rng = np.random.default_rng(5)
        T, K, E, R, H = 20, 3, 8, 4, 128
        topk = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64)
        x = rng.integers(0, 1 << 15, size=(T, H), dtype=np.uint16)
        xs = rng.uniform(0.01, 1, size=(T, 1)).astype(np.float32)
        cnt, _, _ = orc.layout(topk, E, R)
        start, total = orc.scan(cnt)
        out, out_scale, _, oi = orc.scatter(x, xs, topk, start, total)
        tt, kk = np.nonzero(topk >= 0)
        return (np.array_equal(out[oi[tt, kk]], x[tt])
                and np.array_equal(out_scale[oi[tt, kk]], xs[tt]))

    def golden_alignment():
        g = load_golden("scan_alignment_example.txt")
        start, total = orc.scan(np.array(g["counts"]), g["alignment"][0])
        return start.tolist() == g["expert_start_loc"] and total == g["total"][0]

    def brute_aligned():
        rng = np.random.default_rng(77)
        for _ in range(20):
            R = int(rng.integers(1, 4))
            E = R * int(rng.integers(1, 4))
            T, K = int(rng.integers(1, 9)), int(rng.integers(1, 4))
            a = int(rng.integers(2, 6))
            topk = rng.integers(-1, E, size=(T, K)).astype(np.int64)
            want = brute_force(topk, E, R, alignment=a)
            cnt, _, _ = orc.layout(topk, E, R)
            start, total = orc.scan(cnt, a)
            _, _, m, oi = orc.scatter(None, None, topk, start, total)
            if not (np.array_equal(start, want["start"]) and total == want["total"]
                    and np.array_equal(oi, want["oi"]) and np.array_equal(m, want["m"])):
                return False
        return True

    def scale_cols_layout():
        g = load_golden("scatter_scale_cols_example.txt")
        E, R = g["num_experts"][0], g["num_ranks"][0]
        topk = np.array(g["topk_idx"], np.int64)
        words = np.array(g["scale_words"], np.uint32)
        x = np.arange(3 * 16, dtype=np.uint8).reshape(3, 16)
        cnt, _, _ = orc.layout(topk, E, R)
        start, total = orc.scan(cnt)
        out, cols, _, oi = orc.scatter_rows(x, words, orc.SCALE_COLS, topk, start, total,
                                            scale_ld=g["ld"][0])
        ok = all(int(cols[i]) == v for i, v in enumerate(g["out_scale_flat"]) if v >= 0)
        ok = ok and oi.tolist() == [[1, 3], [4, -1], [2, 0]]
        src = [2, 0, 2, 0, 1]
        return ok and all(np.array_equal(out[p], x[src[p]]) for p in range(5))

    def brute_rows():
        rng = np.random.default_rng(41)
        for _ in range(25):
            R = int(rng.integers(1, 4))
            E = R * int(rng.integers(1, 3))
            T, K = int(rng.integers(1, 9)), int(rng.integers(2, 5))
            topk = rng.integers(-1, E, size=(T, K)).astype(np.int64)   # duplicates likely
            want = brute_force(topk, E, R, alignment=2)
            cnt, _, _ = orc.layout(topk, E, R)
            start, total = orc.scan(cnt, 2)
            x = rng.integers(0, 256, size=(T, 16), dtype=np.uint8)
            out, _, m, oi = orc.scatter_rows(x, None, orc.SCALE_NONE, topk, start, total)
            if not (np.array_equal(oi, want["oi"]) and np.array_equal(m, want["m"])):
                return False
            tt, kk = np.nonzero(topk >= 0)
            if not np.array_equal(out[oi[tt, kk]], x[tt]):
                return False
        return True

    def rows_aligned_padding():
        g = load_golden("scatter_hand_example.txt")
        E, R = g["num_experts"][0], g["num_ranks"][0]
        topk = np.array(g["topk_idx"], np.int64)
        cnt, _, _ = orc.layout(topk, E, R)
        start, total = orc.scan(cnt, 4)          # blocks of 4: e1 [0,4), e3 [4,8), e7 [8,12)
        _, _, m, _ = orc.scatter_rows(None, None, orc.SCALE_NONE, topk, start, total)
        return m.tolist() == [1, -1, -1, -1, 3, 3, -1, -1, 7, 7, -1, -1]

    def one_hot_combine():
        rng = np.random.default_rng(3)
        T, K, N = 6, 3, 18
        oi = rng.permutation(N).reshape(T, K).astype(np.int32)
        oi[1, 2] = -1
        eye = (np.eye(N, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
        w = rng.uniform(0.1, 1, (T, K)).astype(np.float32)
        y = orc.combine(eye, oi, w)
        expect = np.zeros((T, N))
        for t in range(T):
            for k in range(K):
                if oi[t, k] >= 0:
                    expect[t, oi[t, k]] += np.float64(w[t, k])
        return np.array_equal(y, expect)

    def bf16_vs_torch():
        import torch
        rng = np.random.default_rng(11)
        f = rng.standard_normal(3000).astype(np.float32)
        ties = (np.arange(1, 300, dtype=np.uint32) << 16 | np.uint32(0x8000)).view(np.float32)
        f = np.concatenate([f, ties, ties * np.float32(3e30)])
        f = f[np.isfinite(f)]
        want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        return np.array_equal(orc.bf16_from_double_array(f.astype(np.float64)), want)

    def expert_scale_hand():
        rows = np.array([[0x3F80], [0x3F80], [0x3F81], [0x3F80]], np.uint16)
        m = np.array([255, 128, 1, 1], np.int32)
        return orc.expert_scale(rows, m)[:, 0].tolist() == [0x4000, 0x3FC0, 0x3F82, 0x3F80]

    def golden_rdma():
        g = load_golden("rdma_counts_example.txt")
        topk = np.array(g["topk_idx"], np.int64)
        _, _, in_rank = orc.layout(topk, g["num_experts"][0], g["num_ranks"][0])
        return all(orc.rdma_counts(in_rank, G).tolist() == g[f"rdma_g{G}"] for G in (1, 2, 4))

    def golden_ll():
        g = load_golden("ll_rectangle_example.txt")
        topk = np.array(g["topk_idx"], np.int64)
        E, M = g["num_experts"][0], g["tokens_per_segment"][0]
        r = orc.ll_dispatch(None, topk, E, M, 4, hidden=128)
        ok = (r["output_index"].tolist() == g["cap4_output_index"]
              and r["recv_count"].tolist() == g["cap4_recv_count"])
        ok = ok and all(r["layout_range"][e].ravel().tolist() == g[f"cap4_range_e{e}"]
                        for e in (1, 3, 7))
        ok = ok and (r["src_info"][[3, 3, 7, 7, 1], [0, 1, 0, 1, 0]] == 0).all()
        r1 = orc.ll_dispatch(None, topk, E, M, 1, hidden=128)
        return ok and r1["output_index"].tolist() == g["cap1_output_index"] and r1["overflow"]

    def ll_src_segments():
        rng = np.random.default_rng(8)
        T, K, E, M = 24, 2, 4, 6
        topk = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int64)
        r = orc.ll_dispatch(None, topk, E, M, T, hidden=128)
        tt, kk = np.nonzero(topk >= 0)
        return np.array_equal(r["src_info"].reshape(-1)[r["output_index"][tt, kk]], tt % M)

    def quant_ref():
        import torch
        rng = np.random.default_rng(23)
        f = rng.standard_normal((6, 256)).astype(np.float32)
        f[2, :128] *= -1e-3
        x = (torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
        q, sc = orc.quantize_e4m3(x)
        xf = (x.astype(np.uint32) << 16).view(np.float32).reshape(6, 2, 128)
        amax = np.abs(xf).max(axis=2)
        inv = (np.float32(448) / amax).astype(np.float32)
        p = (xf * inv[:, :, None]).astype(np.float32).reshape(6, 256)
        want = torch.from_numpy(p).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        return np.array_equal(q, want) and np.array_equal(sc, (amax / np.float32(448)).astype(np.float32))

    def quant_tiny_groups():
        import torch
        g, x = tiny_group_pair()
        qg, _ = orc.quantize_e4m3(g)
        qx, sx = orc.quantize_e4m3(x)
        xf = (x.astype(np.uint32) << 16).view(np.float32).reshape(x.shape[0], -1, 128)
        want_s = (np.abs(xf).max(axis=2) / np.float32(448)).astype(np.float32)
        return np.array_equal(qx, qg) and np.array_equal(sx, want_s)

    for name, fn in [("golden_scan", golden_scan), ("golden_rdma", golden_rdma),
                     ("quant_tiny_groups", quant_tiny_groups),
                     ("golden_ll", golden_ll), ("ll_src_segments", ll_src_segments),
                     ("quant_ref", quant_ref), ("golden_hand", golden_hand), ("brute", brute),
                     ("golden_alignment", golden_alignment), ("brute_aligned", brute_aligned),
                     ("scale_cols_layout", scale_cols_layout),
                     ("rows_aligned_padding", rows_aligned_padding), ("brute_rows", brute_rows),
                     ("rows_and_scales", rows_and_scales), ("one_hot_combine", one_hot_combine),
                     ("bf16_vs_torch", bf16_vs_torch), ("expert_scale_hand", expert_scale_hand)]:
        pin(name, fn)
    return failed


def _run_battery_in_subprocess(lib):
    here = os.path.dirname(os.path.abspath(__file__))
    env = dict(os.environ)
    env["PYTHONPATH"] = os.pathsep.join([os.path.dirname(here), here, env.get("PYTHONPATH", "")])
    return subprocess.run([sys.executable, os.path.abspath(__file__), lib], cwd=here, env=env,
                          capture_output=True, text=True, timeout=300)


def test_unmutated_oracle_passes_the_battery():
    assert _battery(oracle.default()) == []
    # the subprocess route itself works, so a mutant's non-zero exit is its own
    proc = _run_battery_in_subprocess(oracle.default().path)
    assert proc.returncode == 0, proc.stderr
    assert json.loads(proc.stdout.strip().splitlines()[-1]) == []


@pytest.fixture(scope="module")
def mutant_results(tmp_path_factory):
    """Build every mutant and run its battery, a few processes at a time."""
    from concurrent.futures import ThreadPoolExecutor

    d = tmp_path_factory.mktemp("mutants")

    def one(name):
        find, repl = MUTANTS[name]
        proc = _run_battery_in_subprocess(_build_mutant(d, name, find, repl))
        if proc.returncode != 0:
            return name, "crashed"          # the mutant crashed inside a pin: caught
        return name, json.loads(proc.stdout.strip().splitlines()[-1])

    workers = max(1, min(6, (os.cpu_count() or 2) - 1))
    with ThreadPoolExecutor(workers) as pool:
        return dict(pool.map(one, sorted(MUTANTS)))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(mutant_results, name):
    failed = mutant_results[name]
    assert failed, f"planted mistake {name!r} passed every pin"


if __name__ == "__main__":
    print(json.dumps(_battery(Oracle(sys.argv[1]))))
