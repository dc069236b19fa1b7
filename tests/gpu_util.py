"""Helpers for the GPU tests: device buffers of bf16 bit patterns, a registered
UserBuffer fixture, and the element-wise tolerance checks against the oracle."""

import numpy as np
import torch

from oracle import bf16 as obf16

CANARY = 0x7FA5


def dev(bits):
    """uint16 numpy -> device int16 tensor (same bits; the library reads them as bf16)."""
    a = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return torch.from_numpy(a.view(np.int16)).cuda()


def host(t):
    return t.cpu().numpy().view(np.uint16)


def force_tile(ub, h, tile):
    """Force a tile shape ("MxN") on handle h through its debug settings, or None for the
    library's own choice."""
    m, n = (0, 0) if tile is None else map(int, tile.split("x"))
    ub.ub_debug_set(h, "tile_m", m)
    ub.ub_debug_set(h, "tile_n", n)


BF16_TILES = ("320x256", "256x256", "128x256", "128x128", "256x192", "256x160")


def canary(shape):
    return torch.full(shape, CANARY, dtype=torch.int16, device="cuda")


def workspace(ub, capacity, hidden, tp, pad_rows=0):
    """A reduce-scatter workspace of the size ub_required_bytes reports, plus pad_rows rows
    of canary after it: the partial slots canary-filled, the counter region after them zero
    (as ub_init requires).  Returns (whole allocation, view of the partial slots, bytes)."""
    _, ws_bytes = ub.ub_required_bytes(capacity, hidden, tp)
    parts = tp * capacity * hidden
    whole = canary((ws_bytes // 2 + pad_rows * hidden,))
    whole[parts: ws_bytes // 2].zero_()
    return whole, whole[:parts], ws_bytes


class Registration:
    """A UB of [capacity, hidden] (+ workspace), canary-filled, registered with ub_init.
    ws_t views the workspace's partial slots; ws_counters its counter region, which every
    call must leave zero; ws_pad the canary past the registered workspace."""

    def __init__(self, ub, capacity, hidden, tp, workspace=True, pad_rows=0):
        self.ub_mod = ub
        self.capacity, self.hidden, self.tp = capacity, hidden, tp
        ub_bytes, ws_bytes = ub.ub_required_bytes(capacity, hidden, tp)
        # pad_rows extra canary rows after the registered region catch reads/writes past it
        self.ub_t = canary(((capacity + pad_rows) * hidden,))
        self.ws_all = self.ws_t = None
        if workspace:
            self.ws_all, self.ws_t, _ = globals()["workspace"](ub, capacity, hidden, tp, pad_rows)
            self.ws_counters = self.ws_all[tp * capacity * hidden: ws_bytes // 2]
            self.ws_pad = self.ws_all[ws_bytes // 2:]
        self.h = ub.ub_init(capacity, hidden, tp, ub.UB_DTYPE_BF16, self.ub_t, ub_bytes,
                            self.ws_all, ws_bytes if workspace else 0)

    def counters_clean(self):
        """The counter region is back at zero and the canary past the workspace intact."""
        torch.cuda.synchronize()
        return bool((self.ws_counters == 0).all().item()) and bool((self.ws_pad == CANARY).all().item())

    def set_T(self, T):
        self.ub_mod.ub_set_active_shape(self.h, (T, self.hidden))

    def fill(self, a_bits):
        T = a_bits.shape[0]
        self.ub_t[: T * self.hidden].copy_(dev(a_bits).reshape(-1))

    def close(self):
        if self.h is not None:
            torch.cuda.synchronize()
            self.ub_mod.ub_destroy(self.h)
            self.h = None


def check_close(g_bits, o_bits, a_bits, w_bits, what, k_terms=None, gate=4e-3, min_equal=0.98):
    """GPU bf16 result vs oracle bf16 result, element by element.

    * gate: |g - o| <= gate * ||A[t,:]||_2 * ||W[:,j]||_2 (the required tolerance);
    * tight: |g - o| <= max(ulp(g), ulp(o)) + K * 2**-24 * sum_k |A[t,k] W[k,j]|, the
      worst case of an fp32 accumulation of K exact products followed by one bf16
      rounding on each side -- a dropped K block or a wrong operand fails it;
    * at least ``min_equal`` of the elements bit-identical.
    Returns a stats dict."""
    g = obf16.decode(g_bits)
    o = obf16.decode(o_bits)
    A = obf16.decode(a_bits)
    W = obf16.decode(w_bits)
    K = A.shape[1] if k_terms is None else k_terms
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU values"
    err = np.abs(g - o)
    gate_b = gate * np.outer(np.linalg.norm(A, axis=1), np.linalg.norm(W, axis=0))
    absprod = np.abs(A) @ np.abs(W)
    tight_b = np.maximum(obf16.ulp(g_bits), obf16.ulp(o_bits)) + K * 2.0 ** -24 * absprod
    eq = float(np.mean(np.asarray(g_bits) == np.asarray(o_bits)))
    stats = {"max_gate_ratio": float(np.max(err / np.maximum(gate_b, 1e-300))),
             "max_tight_ratio": float(np.max(err / tight_b)), "bit_equal": eq}
    assert np.all(err <= gate_b), f"{what}: gate violated {stats}"
    assert np.all(err <= tight_b), f"{what}: tight bound violated {stats}"
    assert eq >= min_equal, f"{what}: only {eq:.4f} bit-equal {stats}"
    return stats


def check_rs_close(g_out, o_out, a_bits, w_bits, tp, what, gate=4e-3, min_equal=0.97, ring=False,
                   scale=1.0, slice_err=None):
    """Row-parallel result: gate with full-K norms; tight bound adds each bf16 partial's
    rounding and the fp32 sum of the tp partials.  ring=True (the ring-order sum, one bf16
    rounding per hop on each side): the two sides' running sums start from different
    partials and each hop rounds both to bf16, so each of the tp - 1 hops adds up to one
    bf16 ulp of the hop's magnitude (at most sum_s |partial_s|).  scale: a factor applied to
    every product before the partials' rounding (the FP8 path's dequantization; its one
    fp32 multiply is far inside the bf16 terms).  slice_err: per slice, the bound on its
    accumulation error before the bf16 rounding, in the scaled units (default: Ks fp32
    roundings of sum|ab|)."""
    g = obf16.decode(g_out)
    o = obf16.decode(o_out)
    A = obf16.decode(a_bits) * float(scale)
    W = obf16.decode(w_bits)
    k = A.shape[1]
    ks = k // tp
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU values"
    err = np.abs(g - o)
    gate_b = gate * np.outer(np.linalg.norm(A, axis=1), np.linalg.norm(W, axis=0))
    tight_b = np.maximum(obf16.ulp(g_out), obf16.ulp(o_out))
    for s in range(tp):
        sl = slice(s * ks, (s + 1) * ks)
        absprod = np.abs(A[:, sl]) @ np.abs(W[sl])
        part = np.abs(A[:, sl] @ W[sl])
        # |p_gpu - p_oracle| <= 2 u16 |E_s| + (1 + u16) Ks u32 sum|ab|, plus the fp32 sum of
        # the tp partials: tp u32 |p_gpu| with |p_gpu| <= (1 + u16)(|E_s| + Ks u32 sum|ab|)
        s_err = ks * 2.0 ** -24 * absprod if slice_err is None else slice_err[s]
        tight_b = tight_b + 2 * 2.0 ** -8 * part + (1 + 2.0 ** -8) * s_err \
            + tp * 2.0 ** -24 * (1 + 2.0 ** -8) * (part + s_err)
    if ring:
        mag = sum(np.abs(A[:, s * ks:(s + 1) * ks] @ W[s * ks:(s + 1) * ks])
                  + (ks * 2.0 ** -24 * (np.abs(A[:, s * ks:(s + 1) * ks]) @ np.abs(W[s * ks:(s + 1) * ks]))
                     if slice_err is None else slice_err[s])
                  for s in range(tp)) * (1 + 2.0 ** -6)
        tight_b = tight_b + (tp - 1) * obf16.ulp(obf16.encode_rne(mag))
    eq = float(np.mean(np.asarray(g_out) == np.asarray(o_out)))
    stats = {"max_gate_ratio": float(np.max(err / np.maximum(gate_b, 1e-300))),
             "max_tight_ratio": float(np.max(err / tight_b)), "bit_equal": eq}
    assert np.all(err <= gate_b), f"{what}: gate violated {stats}"
    assert np.all(err <= tight_b), f"{what}: tight bound violated {stats}"
    assert eq >= min_equal, f"{what}: only {eq:.4f} bit-equal {stats}"
    return stats
