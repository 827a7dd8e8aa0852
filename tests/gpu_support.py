"""Shared set-up for the GPU parity tests: the same seeded inputs go to the HIP
path (through the C ABI) and to the CPU oracle; results are compared here."""
from __future__ import annotations

import json
import sys

import numpy as np

import synth
from synth import gen
import oracle
from oracle import dflash as O


def log(msg: str) -> None:
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def row_rel_err(got, ref) -> np.ndarray:
    """Relative L2 error of every row (last axis): ||got - ref|| / ||ref|| per row."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return np.linalg.norm(got - ref, axis=-1) / np.maximum(np.linalg.norm(ref, axis=-1), 1e-300)


def row_tol(cfg) -> float:
    """Per-row bound: the tensor bound of the configuration, applied to every single row
    (each hidden row, each logit row, each (layer, head, position) K / V row)."""
    return tol(cfg)


def check_kv_rows(cfg, k_got, k_ref, v_got, v_ref, what=""):
    """Whole-tensor and per-row relative errors of K / V rows [..][position][D]; asserts both."""
    ek, ev = rel_err(k_got, k_ref), rel_err(v_got, v_ref)
    rk, rv = row_rel_err(k_got, k_ref), row_rel_err(v_got, v_ref)
    mk = float(rk.max()) if rk.size else 0.0
    mv = float(rv.max()) if rv.size else 0.0
    log(f"  {what}kv rel err k={ek:.3e} v={ev:.3e}; worst row k={mk:.3e} v={mv:.3e} over {rk.size} rows")
    assert ek < tol(cfg) and ev < tol(cfg)
    assert mk < row_tol(cfg) and mv < row_tol(cfg)
    return {"k_rel": ek, "v_rel": ev, "k_row_max": mk, "v_row_max": mv}


def decode(a):
    return O.decode_storage(a, np.float64)


def top2_gap(z: np.ndarray) -> np.ndarray:
    s = np.sort(z, axis=-1)
    return s[..., -1] - s[..., -2]


def tol(cfg) -> float:
    """Relative-error bound for floating outputs: 1e-4 for fp32 storage, 2e-2 for bf16."""
    return 1e-4 if cfg.dtype == "f32" else 2e-2


class Pair:
    """One configuration instantiated on both sides."""

    def __init__(self, cfg, batch: int, cap: int, max_rows: int, device: str = "cuda", overrides=None):
        import block_diffusion_drafter_states_amd as dfl
        import torch
        self.torch = torch
        self.dfl = dfl
        self.cfg = cfg
        self.batch = batch
        self.cap = cap
        self.W = gen.weights(cfg, overrides)
        self.om = O.DraftModel(cfg, self.W)
        self.model = dfl.Model(cfg, self.W, device=device, max_batch=batch, kv_capacity=cap,
                               gamma_max=cfg.gamma_max)
        self.cache = dfl.Cache(self.model)
        self.okv = O.KVCache(cfg, batch, cap)
        self.ws = dfl.Workspace(self.model, batch, max_rows)
        self.device = device

    # ---------------------------------------------------------------- inputs
    def dev_i32(self, a):
        return self.torch.as_tensor(np.asarray(a, dtype=np.int32), device=self.device).contiguous()

    def dev_storage(self, a):
        return self.dfl.to_device(a, self.device)

    # ---------------------------------------------------------------- steps
    def inject(self, feat_storage: np.ndarray, n_new) -> None:
        """feat_storage [B][rows][F][H] storage; both sides append n_new[b] rows."""
        self.dfl.inject_kv(self.model, self.cache, self.dev_storage(feat_storage), self.dev_i32(n_new), self.ws)
        f = decode(feat_storage)
        for b in range(self.batch):
            O.inject(self.om, self.okv, b, f[b, : int(n_new[b])])

    def set_context(self, lengths, tag="ctx"):
        K, V = gen.context_kv(self.cfg, np.asarray(lengths), self.cap, tag=tag)
        self.cache.set_context(K, V, lengths)
        self.okv = O.KVCache.from_storage(self.cfg, K, V, lengths)

    def draft(self, anchors, gamma):
        torch = self.torch
        B = self.batch
        d = torch.full((B, gamma - 1), -7, dtype=torch.int32, device=self.device)
        hid = torch.full((B, gamma, self.cfg.hidden), float("nan"), dtype=torch.float32, device=self.device)
        lg = torch.full((B, gamma - 1, self.cfg.vocab), float("nan"), dtype=torch.float32, device=self.device)
        self.dfl.draft_block(self.model, self.cache, gamma, self.dev_i32(anchors), d, self.ws, hid, lg)
        torch.cuda.synchronize()
        return d.cpu().numpy(), hid.cpu().numpy(), lg.cpu().numpy()

    def oracle_draft(self, anchors, gamma):
        ds, xs, zs = [], [], []
        for b in range(self.batch):
            d, x, z = O.draft(self.om, self.okv, b, int(anchors[b]), gamma, return_all=True)
            ds.append(d); xs.append(x); zs.append(z)
        return np.stack(ds), np.stack(xs), np.stack(zs)

    def status(self) -> int:
        return int(self.cache.status.item())


def check_draft(cfg, got, ref, gap_min=1e-2, head=None):
    """Compare (draft, hidden, logits) of GPU vs oracle; returns a dict of metrics.

    Hidden states and logits: relative error of the whole tensor and of every row.
    Draft ids are an argmax decided in floating point, checked three ways:
      * self-consistency: each id's logit in the fp32 logits the GPU returns is its row's
        maximum (`argmax_self_mismatch`).  The argmax LM head decides on its logits before
        the final RMSNorm's positive row factor, which the returned logits then carry; a
        positive factor keeps every order but can round two close logits to one value, so
        the id is a maximum of the returned row, not necessarily its lowest-index one;
      * the LM head + argmax stage on its own (`head`: the final norm, rounding and LM head
        of the same reading applied to the GPU's final hidden rows): every row whose top-2
        gap is at least gap_min (1e-2) must draft that argmax (`head_strict_mismatch`).  The
        stage's inputs are then identical on both sides, so its logits differ only by
        summation order (~1e-5), far below the gap;
      * end to end against the oracle's own forward: the two forwards round to bf16 at
        the same points but decide some roundings differently (a value within float
        noise of a bf16 midpoint), and such differences spread through later roundings
        to about a bf16 unit in the hidden states (no implementation that sums in another
        order than the fp64 oracle can avoid it).  Rows whose oracle gap exceeds twice the
        largest logit difference of the call (and gap_min) must match (`wide_mismatch`);
        elsewhere the chosen id must be within twice that difference of the oracle's
        maximum (`not_near_optimal`).  The rows below gap_min (`band_exempt`), those
        between gap_min and twice the difference (`band_wide`), and the ids that differ in
        each band (`strict_mismatch` counts all differing ids at gap >= gap_min) are
        reported."""
    d, x, z = got
    dr, xr, zr = ref
    assert np.isfinite(x).all() and np.isfinite(z).all()
    ex = rel_err(x, xr)
    ez = rel_err(z, zr)
    rx = row_rel_err(x, xr)
    rz = row_rel_err(z, zr)
    err = float(np.abs(z - zr).max())
    gap = top2_gap(zr)
    differ = d != dr
    exempt = gap < gap_min
    wide = (~exempt) & (gap <= 2.0 * err)
    sure = (~exempt) & (~wide)
    picked_own = np.take_along_axis(z, d[..., None].astype(np.int64), axis=-1)[..., 0]
    self_mism = int((picked_own != z.max(axis=-1)).sum())
    picked = np.take_along_axis(zr, d[..., None].astype(np.int64), axis=-1)[..., 0]
    not_near = int((picked < zr.max(axis=-1) - 2.0 * err).sum())
    m = {"hidden_rel": ex, "logits_rel": ez, "hidden_row_max": float(rx.max()), "logits_row_max": float(rz.max()),
         "rows": int(gap.size), "draft_checked": int(sure.sum()),
         "strict_mismatch": int((differ & ~exempt).sum()), "wide_mismatch": int((differ & sure).sum()),
         "band_exempt": int(exempt.sum()), "band_exempt_differ": int((differ & exempt).sum()),
         "band_wide": int(wide.sum()), "band_wide_differ": int((differ & wide).sum()),
         "argmax_self_mismatch": self_mism, "not_near_optimal": not_near, "logit_maxabs": err}
    if head is not None:
        zh = head(x)                       # oracle head on the GPU's final hidden rows
        gh = top2_gap(zh)
        hs = gh >= gap_min
        m["head_logit_maxabs"] = float(np.abs(z - zh).max())
        m["head_checked"] = int(hs.sum())
        m["head_strict_mismatch"] = int(((d != np.argmax(zh, axis=-1)) & hs).sum())
    return m


def assert_draft(cfg, m) -> None:
    assert m["hidden_rel"] < tol(cfg) and m["logits_rel"] < tol(cfg)
    assert m["hidden_row_max"] < row_tol(cfg) and m["logits_row_max"] < row_tol(cfg)
    assert m["argmax_self_mismatch"] == 0
    assert m["wide_mismatch"] == 0 and m["not_near_optimal"] == 0
    assert m["draft_checked"] > 0
    if "head_strict_mismatch" in m:
        assert m["head_strict_mismatch"] == 0 and m["head_checked"] > 0
    if cfg.dtype == "f32":      # no bf16 roundings to decide differently: the strict bar end to end
        assert m["strict_mismatch"] == 0


def oracle_head(om):
    """The argmax LM-head stage as a function of final hidden rows [B][gamma][H] (the anchor
    row excluded, as in drafting), in the GPU's reading of where the final RMSNorm rounds:
    the head's input is rho(x * w_final) and the norm's row factor f = 1 / sqrt(mean(x^2) +
    eps) multiplies the logits, f * (rho(x * w) . W^T); the oracle's forward rounds
    rho(f * x * w) instead.  Equal in exact arithmetic; one bf16 rounding per input either
    way."""
    def f(x):
        x = np.asarray(x, dtype=np.float64)[:, 1:]
        w = np.asarray(om.final_norm, dtype=np.float64)
        rf = 1.0 / np.sqrt((x * x).mean(axis=-1, keepdims=True) + om.cfg.eps)
        return O.linear(om.num.rho(x * w), om.lm_head) * rf
    return f


def run_cycle_case(cfg, batch, lengths, gammas, cap, seed_tag):
    """Prefill-inject `lengths`, then for each gamma: draft, compare, inject a few rows."""
    log(f"case {cfg.name} batch={batch} lengths={list(lengths)} gammas={gammas} cap={cap}")
    max_rows = max(max(lengths), max(gammas))
    P = Pair(cfg, batch, cap, max_rows)
    rows = max(lengths)
    feat = gen.features(cfg, batch, rows, tag=f"{seed_tag}.prefill")
    log(f"  inject prefill rows={rows}")
    P.inject(feat, lengths)
    P.torch.cuda.synchronize()
    assert P.status() == 0
    assert list(P.cache.len.cpu().numpy()[:batch]) == list(lengths)
    k = decode(P.cache.read_k())
    v = decode(P.cache.read_v())
    # every written (layer, sequence, head, position) row, per row
    rows_k = np.concatenate([k[:, b, :, :lengths[b]].reshape(-1, cfg.head_dim) for b in range(batch)])
    rows_kr = np.concatenate([P.okv.k[:, b, :, :lengths[b]].reshape(-1, cfg.head_dim) for b in range(batch)])
    rows_v = np.concatenate([v[:, b, :, :lengths[b]].reshape(-1, cfg.head_dim) for b in range(batch)])
    rows_vr = np.concatenate([P.okv.v[:, b, :, :lengths[b]].reshape(-1, cfg.head_dim) for b in range(batch)])
    check_kv_rows(cfg, rows_k, rows_kr, rows_v, rows_vr)
    assert rel_err(k, P.okv.k) < tol(cfg) and rel_err(v, P.okv.v) < tol(cfg)
    results = []
    for ci, gamma in enumerate(gammas):
        anchors = gen.tokens(cfg, f"{seed_tag}.anchor.{ci}", (batch,))
        log(f"  draft cycle {ci} gamma={gamma}")
        got = P.draft(anchors, gamma)
        ref = P.oracle_draft(anchors, gamma)
        m = check_draft(cfg, got, ref, head=oracle_head(P.om))
        log(f"  {json.dumps(m)}")
        assert_draft(cfg, m)
        results.append(m)
        # next cycle: inject a planted number of accepted rows
        n_new = (gen.planted_accept(cfg, (batch,), gamma, tag=f"{seed_tag}.k.{ci}") + 1).astype(np.int32)
        nf = gen.features(cfg, batch, gamma, tag=f"{seed_tag}.feat.{ci}")
        log(f"  inject n_new={list(n_new)}")
        P.inject(nf, n_new)
        P.torch.cuda.synchronize()
        assert P.status() == 0
        assert list(P.cache.len.cpu().numpy()[:batch]) == list(P.okv.len)
    return P, results
