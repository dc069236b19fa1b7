"""Child process of test_gpu_serialize: runs every schedule of the library once on seeded
inputs and prints one digest per output (run with and without serialised kernels and
copies; the digests must agree).  Prints a line per step as it goes."""

import hashlib
import os
import sys

import numpy as np
import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import chunked_tp_overlap_amd.ub as ub  # noqa: E402
from chunked_tp_overlap_amd import workloads as wl  # noqa: E402


def dig(t):
    torch.cuda.synchronize()
    return hashlib.sha256(t.cpu().numpy().tobytes()).hexdigest()[:16]


def main():
    torch.cuda.set_device(0)
    rng = np.random.default_rng(93)
    cap, H, N, T, tp, K = 1024, 512, 264, 600, 8, 1024
    a = wl.normal_bits(rng, (cap, H))
    w = torch.from_numpy(wl.normal_bits(rng, (H, N), 0.02).view(np.int16)).cuda()
    a_rs = torch.from_numpy(wl.normal_bits(rng, (T, K)).view(np.int16)).cuda()
    w_rs = torch.from_numpy(wl.normal_bits(rng, (K, H), 0.02).view(np.int16)).cuda()
    src = torch.from_numpy(a.view(np.int16).ravel()).cuda()
    ub_bytes, ws_bytes = ub.ub_required_bytes(cap, H, tp)
    ub_t = torch.zeros(cap * H, dtype=torch.int16, device="cuda")
    ws_t = torch.zeros(ws_bytes // 2, dtype=torch.int16, device="cuda")
    h = ub.ub_init(cap, H, tp, ub.UB_DTYPE_BF16, ub_t, ub_bytes, ws_t, ws_bytes)
    try:
        ub.ub_set_active_shape(h, (T, H))
        cases = [("ag host S=3", dict(method="pipeline", num_splits=5, num_max_streams=3)),
                 ("ag ring aggregate", dict(method="ring_exchange", rank=3, aggregate=True)),
                 ("ag device loop", dict(method="ring_exchange", rank=6, atomic_gemm=True))]
        for name, kw in cases:
            ub_t[: T * H].copy_(src[: T * H])
            c = torch.zeros((T, N), dtype=torch.int16, device="cuda")
            ub.ub_gemm_ag_chunked(h, w, N, N, c, N, ub.make_cfg(**kw))
            print(f"{name} {dig(c)}", flush=True)
        for name, kw in (("arrival host loop", dict(method="ring_exchange", rank=2)),
                         ("arrival device loop", dict(method="ring_exchange", rank=5, atomic_gemm=True))):
            ub_t.zero_()
            lo, hi = kw["rank"] * T // tp, (kw["rank"] + 1) * T // tp
            ub_t[lo * H: hi * H].copy_(src[lo * H: hi * H])
            c = torch.zeros((T, N), dtype=torch.int16, device="cuda")
            ub.ub_gemm_ag_arrival(h, src, w, N, N, c, N, ub.make_cfg(**kw))
            print(f"{name} {dig(c)}", flush=True)
        for name, kw in (("rs pipeline", dict(method="pipeline", num_splits=4)),
                         ("rs ring order device loop", dict(method="ring_exchange", rank=1, atomic_gemm=True,
                                                            reduce_order="ring"))):
            out = torch.zeros((T, H), dtype=torch.int16, device="cuda")
            ub.ub_gemm_rs_chunked(h, a_rs, K, K, w_rs, H, out, H, ub.make_cfg(**kw))
            print(f"{name} {dig(out)}", flush=True)
        a8 = torch.empty((T, K), dtype=torch.uint8, device="cuda")
        w8 = torch.empty((H, K), dtype=torch.uint8, device="cuda")
        ub.ub_quantize_e4m3(a_rs, K, a8, K, T, K, 64.0)
        ub.ub_quantize_e4m3(w_rs.t().contiguous(), K, w8, K, H, K, 4096.0)
        out = torch.zeros((T, H), dtype=torch.int16, device="cuda")
        ub.ub_gemm_rs_chunked_fp8(h, a8, K, K, w8, K, 1 / 64.0, 1 / 4096.0, out, H,
                                  ub.make_cfg("pipeline", 3, atomic_gemm=False))
        print(f"rs fp8 {dig(out)}", flush=True)
        print(f"timeouts {ub.ub_arrival_timeouts(h)}", flush=True)
    finally:
        torch.cuda.synchronize()
        ub.ub_destroy(h)


if __name__ == "__main__":
    main()
