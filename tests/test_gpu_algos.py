"""GPU parity of every algorithm of the linear layer (every kernel
configuration with each accumulation, through sparse_fp8_scaled_linear_algo)
against the oracle, on shapes each one supports -- a decode shape every
algorithm can run, a tall shape for the tiled ones and the decode kernel's
largest K -- plus the per-shape search (sparse_fp8_row_amd.tune) and the
table it feeds.  Binary32-grade algorithms are held to the stated bound on
every element; FP8-accumulation algorithms to that bound plus the FP8
instruction's truncation bound (parity.hw_bound)."""
import sys

import numpy as np
import pytest
import torch

import oracle
import sfr_inputs
from parity import check_bf16, check_f32, dev_bf16, host_bf16_bits, host_f32, hw_bound, is_f8_acc, FP8_TORCH

pytestmark = pytest.mark.gpu

E4, E5 = oracle.E4M3, oracle.E5M2
SHAPES = [("all_algos", 7, 1040, 1024, E4, E4, True), ("tiled", 300, 4112, 640, E5, E4, True),
          ("max_k_decode", 16, 256, 16384, E4, E5, False),
          # one activation row, 7 wavefronts of 2 units each, 16 and 32 rows per workgroup
          ("decode_one_row", 1, 6144, 14336, E5, E4, True),
          # 20 units over 7 wavefronts (3, 3, ..., 2), several activation rows
          ("decode_uneven_units", 5, 2080, 20480, E4, E4, False),
          # 17 k steps: two whole 8-step metadata blocks, then one step in the
          # reused first buffer; ragged tiles in m and n
          ("tiled_partial_block", 264, 1040, 2176, E4, E5, True),
          # the smallest K: one and two k steps
          ("one_step", 300, 528, 128, E4, E4, True), ("two_steps", 260, 1040, 256, E5, E5, False),
          # few tiles and a long K: the four-stage forms of tiled_64x64 and
          # tiled_128x128; 65 k steps, so the last metadata block is partial
          ("deep_pipeline", 200, 1040, 8320, E5, E4, True),
          # the unit decode kernels over 16-row activation blocks: 4 blocks,
          # the last with 2 rows
          ("decode_column_blocks", 50, 1056, 2048, E4, E5, True),
          # more than 8 units with workgroups that fit the CUs at once: one
          # unit per wavefront on up to 16 wavefronts (9 here, and 14 with the
          # down projection's K at 3 rows)
          ("decode_waves_9", 7, 1040, 9216, E5, E4, True), ("decode_waves_14", 3, 4096, 14336, E4, E4, False)]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import sparse_fp8_row_amd as sfr
    sfr.load()
    return sfr


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: s[0])
def test_every_algo(gpu, shape):
    name, m, n, k, xf, wf, has_bias = shape
    case = sfr_inputs.Case(f"algo_{name}", 13, m, n, k, x_fmt=xf, w_fmt=wf, bias=has_bias)
    xb, wb, bb = sfr_inputs.draw_x(case), sfr_inputs.draw_w(case), sfr_inputs.draw_bias(case)
    oxq, oxs = oracle.quantize_rows(xb, xf)
    ov, om, ows, _ = oracle.prepare_weight(wb, wf)
    ref = oracle.linear(oxq, xf, oxs, ov, om, wf, ows, bias=bb)
    hwb = hw_bound(oxq, xf, oxs, oracle.decompress_2to4(ov, om), wf, ows, np.arange(m), np.arange(n))
    xq, xs = gpu.quantize_rowwise_fp8(dev_bf16(xb), FP8_TORCH[xf])
    pw = gpu.prepare_weight(dev_bf16(wb), FP8_TORCH[wf])
    b = None if bb is None else dev_bf16(bb)
    ran = []
    for algo, aname in gpu.linear_algos():
        if not gpu.algo_supported(algo, m, n, k):
            with pytest.raises(gpu.SfrError):
                gpu.sparse_fp8_scaled_linear(xq, xs, pw.values, pw.meta, pw.scale, b, algo=algo)
            continue
        for od in (torch.bfloat16, torch.float32):
            say(f"algo {aname} {case.name} out={od}")
            y = gpu.sparse_fp8_scaled_linear(xq, xs, pw.values, pw.meta, pw.scale, b, out_dtype=od, algo=algo)
            torch.cuda.synchronize()
            allow = hwb if is_f8_acc(algo) else None
            if od == torch.float32:
                r = check_f32(host_f32(y), ref, bb is not None, allow)
            else:
                r = check_bf16(host_bf16_bits(y), ref, allow)
            say(f"  {r}")
            assert r["bad"] == 0, r
        ran.append(aname)
    # tiled 64/128/256 with each accumulation, the pipelined kernel (FP8, K >= 512)
    assert len(ran) >= (7 if k >= 512 else 6)


def test_search_and_table(gpu):
    from sparse_fp8_row_amd import tune
    shapes = [(16, 1024, 1024), (300, 1024, 640)]
    res = tune.search(shapes, reps=3, warmup=1)
    names = dict(gpu.linear_algos())
    for (m, n, k), rec in zip(shapes, res["timings"]):
        best = res["table"][(gpu.m_bucket(m), n, k)]
        assert gpu.algo_supported(best, m, n, k)
        assert names[best] == rec["best"] and rec["best_us"] == min(rec["us"].values())
    # the table drives later calls: same bytes as the explicit algorithm
    case = sfr_inputs.Case("algo_table", 14, 300, 1024, 640, bias=True)
    xq, xs = gpu.quantize_rowwise_fp8(dev_bf16(sfr_inputs.draw_x(case)))
    pw = gpu.prepare_weight(dev_bf16(sfr_inputs.draw_w(case)))
    best = res["table"][(gpu.m_bucket(300), 1024, 640)]
    gpu.set_algo_table(res["table"])
    try:
        y1 = gpu.sparse_fp8_scaled_linear(xq, xs, pw.values, pw.meta, pw.scale)
    finally:
        gpu.set_algo_table({})
    y2 = gpu.sparse_fp8_scaled_linear(xq, xs, pw.values, pw.meta, pw.scale, algo=best)
    torch.cuda.synchronize()
    assert np.array_equal(host_bf16_bits(y1), host_bf16_bits(y2))


def test_subnormal_outputs(gpu):
    """bf16 rounding of outputs in the binary32 / bf16 subnormal range, in
    every kernel's epilogue: scales 2^-60 (rows) and 2^-84 (outputs) make
    xs * ws = 2^-144 exactly, so most outputs land below 2^-126; each must be
    within one bf16 ulp of the oracle's value (a converter that flushed
    subnormals would give zeros)."""
    m, n, k, xf, wf = 48, 256, 1024, E4, E4
    case = sfr_inputs.Case("algo_subnormal", 15, m, n, k, x_fmt=xf, w_fmt=wf)
    xb, wb = sfr_inputs.draw_x(case), sfr_inputs.draw_w(case)
    oxq, _ = oracle.quantize_rows(xb, xf)
    ov, om, _, _ = oracle.prepare_weight(wb, wf)
    oxs = np.full(m, 2.0**-60, np.float32)
    ows = np.full(n, 2.0**-84, np.float32)
    ref = oracle.linear(oxq, xf, oxs, ov, om, wf, ows)
    sub = (np.abs(ref["y"]) < 2.0**-126) & (np.abs(ref["y"]) >= 2.0**-133)
    assert sub.mean() > 0.3, f"only {sub.mean():.2f} of the outputs are subnormal"
    xq, xs = gpu.quantize_rowwise_fp8(dev_bf16(xb), FP8_TORCH[xf])
    pw = gpu.prepare_weight(dev_bf16(wb), FP8_TORCH[wf])
    xs = torch.full_like(xs, 2.0**-60)
    ws = torch.full_like(pw.scale, 2.0**-84)
    ran = 0
    for algo, aname in gpu.linear_algos():
        if is_f8_acc(algo) or not gpu.algo_supported(algo, m, n, k):
            continue
        say(f"subnormal outputs: {aname}")
        y = gpu.sparse_fp8_scaled_linear(xq, xs, pw.values, pw.meta, ws, algo=algo)
        torch.cuda.synchronize()
        r = check_bf16(host_bf16_bits(y), ref)
        say(f"  {r}")
        assert r["bad"] == 0, (aname, r)
        ran += 1
    assert ran >= 5
