"""HIP-graph capture of the chunked GEMM calls (bf16 all-gather and reduce-scatter, FP8
reduce-scatter): none of them synchronises the host,
allocates, or records a memset, so a whole step (several microbatches, each with its own
active shape) can be captured once and replayed.  Every replay is checked bit for bit
against the eager results, with eager work and host synchronisation between replays."""

import numpy as np
import pytest
import torch

from chunked_tp_overlap_amd import workloads as wl
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ub():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import chunked_tp_overlap_amd.ub as m
    return m


def test_graph_replays_match_eager(ub):
    rng = np.random.default_rng(91)
    cap, H, N, tp, K = 1024, 512, 264, 8, 1024
    Ts = (1024, 600, 296)
    a = gu.dev(wl.normal_bits(rng, (cap, H)))
    w = gu.dev(wl.normal_bits(rng, (H, N), 0.02))
    a_rs = gu.dev(wl.normal_bits(rng, (cap, K)))
    w_rs = gu.dev(wl.normal_bits(rng, (K, H), 0.02))
    reg = gu.Registration(ub, cap, H, tp)
    cfgs = [ub.make_cfg("ring_exchange", atomic_gemm=True, rank=3),
            ub.make_cfg("pipeline", 5, 3, rank=0),                      # host loop, 3 streams
            ub.make_cfg("ring_exchange", 1, 2, True, False, rank=6)]    # aggregate, 2 streams
    rs_cfgs = [ub.make_cfg("pipeline", 4, 3, atomic_gemm=True),
               ub.make_cfg("ring_exchange", 1, 3, reduce_order="ring", rank=1)]
    # the same sums with the reduction fused into the slice-GEMM launch (bf16 only)
    fused_cfgs = [ub.make_cfg("pipeline", 4, 3, fuse_reduce=True),
                  ub.make_cfg("ring_exchange", 1, 3, atomic_gemm=True, reduce_order="ring", rank=1,
                              fuse_reduce=True)]
    outs = [gu.canary((cap, N)) for _ in range(len(Ts) * len(cfgs))]
    rs_outs = [gu.canary((cap, H)) for _ in range(len(Ts) * len(rs_cfgs) * 2)]
    fused_outs = [gu.canary((cap, H)) for _ in range(len(Ts) * len(fused_cfgs))]
    # E4M3 operands of the reduce-scatter GEMM, quantized once (eagerly) on the GPU
    a8 = torch.empty((cap, K), dtype=torch.uint8, device="cuda")
    w8 = torch.empty((H, K), dtype=torch.uint8, device="cuda")
    ub.ub_quantize_e4m3(a_rs, K, a8, K, cap, K, 64.0)
    ub.ub_quantize_e4m3(w_rs.t().contiguous(), K, w8, K, H, K, 4096.0)

    def step(stream):
        i = j = f = 0
        for T in Ts:
            ub.ub_set_active_shape(reg.h, (T, H))
            for cfg in cfgs:
                ub.ub_gemm_ag_chunked(reg.h, w, N, N, outs[i], N, cfg, stream)
                i += 1
            for cfg in rs_cfgs:
                ub.ub_gemm_rs_chunked(reg.h, a_rs, K, K, w_rs, H, rs_outs[j], H, cfg, stream)
                ub.ub_gemm_rs_chunked_fp8(reg.h, a8, K, K, w8, K, 1.0 / 64, 1.0 / 4096, rs_outs[j + 1],
                                          H, cfg, stream)
                j += 2
            for cfg in fused_cfgs:
                ub.ub_gemm_rs_chunked(reg.h, a_rs, K, K, w_rs, H, fused_outs[f], H, cfg, stream)
                f += 1

    try:
        reg.ub_t[: cap * H].copy_(a.reshape(-1))
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            step(s)
        torch.cuda.synchronize()
        eager = [gu.host(o) for o in outs]
        eager_rs = [gu.host(o) for o in rs_outs]
        eager_fused = [gu.host(o) for o in fused_outs]
        for t in range(len(Ts)):  # fused == separate reduction, same order
            for c in range(len(fused_cfgs)):
                assert np.array_equal(eager_fused[t * len(fused_cfgs) + c],
                                      eager_rs[(t * len(rs_cfgs) + c) * 2]), (t, c)
        rs_outs = rs_outs + fused_outs
        eager_rs = eager_rs + eager_fused
        for o in outs + rs_outs:
            o.fill_(gu.CANARY)
        torch.cuda.synchronize()

        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            step(s)
        torch.cuda.synchronize()
        for rep in range(3):
            for o in outs + rs_outs:  # eager work between replays
                o.fill_(gu.CANARY)
            scratch = torch.randn(1 << 20, device="cuda").sum()  # more eager work
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for k, o in enumerate(outs):
                assert np.array_equal(gu.host(o), eager[k]), (rep, "ag", k)
            for k, o in enumerate(rs_outs):
                assert np.array_equal(gu.host(o), eager_rs[k]), (rep, "rs", k)
            del scratch
    finally:
        reg.close()


def test_graph_captures_first_fused_call(ub):
    """The first fused reduce-scatter call of a handle goes straight into a graph: it needs
    no allocation or clearing (its tile counters are the workspace's zeroed counter region),
    so the capture holds only kernel launches.  Every replay equals the eager separate
    reduction bit for bit, and leaves the counters at zero."""
    rng = np.random.default_rng(92)
    cap, H, tp, K = 2048, 264, 8, 1024
    Ts = (2048, 1000)
    a_rs = gu.dev(wl.normal_bits(rng, (cap, K)))
    w_rs = gu.dev(wl.normal_bits(rng, (K, H), 0.02))
    reg = gu.Registration(ub, cap, H, tp)
    cfgs = [ub.make_cfg("pipeline", 4, 3, fuse_reduce=True),
            ub.make_cfg("pipeline", 4, 3, atomic_gemm=True, fuse_reduce=True, reduce_order="ring")]
    try:
        s = torch.cuda.Stream()
        ref = []
        with torch.cuda.stream(s):  # eager, with the separate reduction only
            for T in Ts:
                ub.ub_set_active_shape(reg.h, (T, H))
                for cfg in cfgs:
                    sep = ub.make_cfg("pipeline", 4, 3, atomic_gemm=bool(cfg.atomic_gemm),
                                      reduce_order="ring" if cfg.reduce_order else "ascending")
                    o = gu.canary((cap, H))
                    ub.ub_gemm_rs_chunked(reg.h, a_rs, K, K, w_rs, H, o, H, sep, s)
                    ref.append(o)
        torch.cuda.synchronize()
        ref = [gu.host(o) for o in ref]
        outs = [gu.canary((cap, H)) for _ in ref]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            i = 0
            for T in Ts:
                ub.ub_set_active_shape(reg.h, (T, H))
                for cfg in cfgs:
                    ub.ub_gemm_rs_chunked(reg.h, a_rs, K, K, w_rs, H, outs[i], H, cfg, s)
                    i += 1
        torch.cuda.synchronize()
        for rep in range(3):
            for o in outs:
                o.fill_(gu.CANARY)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for k, o in enumerate(outs):
                assert np.array_equal(gu.host(o), ref[k]), (rep, k)
            assert reg.counters_clean(), rep
    finally:
        reg.close()
