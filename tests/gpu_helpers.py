"""Helpers for the GPU tests: run the HIP path through the C ABI and fetch what the
workspace holds, and compare with the oracle under the stated acceptance rules."""
from __future__ import annotations

import numpy as np
import torch

import block_scaled_fp8_dispatch_amd as moe
import oracle

Y_TOL = 2e-2            # max |y_gpu - y_ref| / max |y_ref| per row
OFF_BY_ONE_MAX = 1e-3   # fraction of requantised FP8 intermediates one code off
# fewest compared intermediates for which that fraction is checked as a rate (at 1e-3, ten
# expected differences); smaller samples check every difference against the FP32 bound
RATE_MIN_ELEMENTS = 10_000
# Reading of "off by one code" for elements far below their block maximum: an element more
# than one code from the oracle's is excused only if its exact |h| is at most this fraction
# of its block's largest |h| (at least 4 binades below, where the absolute FP32 error of the
# block's dot products can exceed the element's own grid step) AND the GPU value is a
# round-to-nearest result of a value within the FP32 accumulation bound of the exact h
FAR_BELOW_FRACTION = 2.0 ** -4
# Most such excused elements a comparison may hold, as a rate of the compared elements,
# rounded up (one in any comparison; more only past 100 000 compared elements)
FAR_EXCUSED_MAX_RATE = 1e-5
# Reading of the two tolerances together: a one-code difference the intermediate rule
# accepts (a value within FP32 error of a rounding midpoint) at a block's largest element of
# a heavily weighted slot moves a y row by up to a few per cent of its largest value. A row
# whose end-to-end error exceeds Y_TOL therefore passes only if one of its slots holds such
# an accepted difference and the row is within Y_TOL of the oracle's Linear2 and combine run
# on the GPU's own (decoded) intermediate; such rows are counted, printed and capped at this
# rate of the compared rows (rounded up)
ROW_EXCUSED_MAX_RATE = 1e-3


class Run:
    """One prepared problem on the GPU (packed weights + workspace) and its last forward."""

    def __init__(self, inp, max_tokens=None, device="cuda"):
        cfg = inp.cfg
        self.inp = inp
        self.T = inp.x_fp8.shape[0]
        self.shape = moe.make_shape(cfg.E, cfg.H, cfg.I, cfg.k, max_tokens or max(self.T, 1))
        nb = moe.moe_packed_weights_bytes(self.shape)
        assert nb > 0
        self.packed = torch.empty(nb, dtype=torch.uint8, device=device)
        moe.moe_prepare_weights(self.shape, inp.w1, inp.w1_sf, inp.w2, inp.w2_sf, self.packed)
        self.ws = torch.empty(moe.moe_workspace_bytes(self.shape), dtype=torch.uint8, device=device)
        self.y = torch.empty(max(self.T, 1), cfg.H, dtype=torch.int16, device=device)
        self.last_T = self.T

    def forward(self, T=None, poison=True):
        T = self.T if T is None else T
        self.last_T = T
        if poison:
            self.ws.fill_(0xFF)
            self.y.fill_(0x7FBF)
        moe.moe_forward(self.y, self.inp.x_fp8, self.inp.x_sf, self.inp.topk_idx,
                        self.inp.topk_weights, T, self.shape, self.packed, self.ws)
        torch.cuda.synchronize()
        return self.y[:T].cpu().numpy().view(np.uint16)

    def layout(self, T=None):
        return moe.moe_workspace_layout(self.shape, self.T if T is None else T)

    def ws_i32(self, off, n):
        return self.ws[off: off + 4 * n].cpu().numpy().view(np.int32).copy()

    def routing(self, T=None):
        T = self.T if T is None else T
        L = self.layout(T)
        E, k = self.shape.num_experts, self.shape.num_topk
        meta = self.ws_i32(L["meta"], 8)
        offsets = self.ws_i32(L["offsets"], E + 1)
        ntiles = int(meta[0])
        return dict(
            block_m=L["block_m"], meta=meta,
            counts=self.ws_i32(L["counts"], E), offsets=offsets,
            perm=self.ws_i32(L["perm"], int(offsets[E])), inv=self.ws_i32(L["inv"], T * k),
            tile_expert=self.ws_i32(L["tile_expert"], ntiles),
            tile_row0=self.ws_i32(L["tile_row0"], ntiles), num_invalid=meta[1])

    def intermediates(self, rows, T=None):
        """h8 codes [len(rows), I] and h_sf bytes [len(rows), I/128] of the given padded rows
        (h8 is stored in blocks of block_m rows x 128 columns; h_sf in the blocked scale
        layout of moe.h)."""
        L = self.layout(self.last_T if T is None else T)
        I = self.shape.intermediate
        hb = L["block_m"]
        sfs = L["h_sf_stride"]
        rows = np.asarray(rows, dtype=np.int64)
        n = int(rows.max()) + 1
        nblk = (n + hb - 1) // hb
        h8 = self.ws[L["h8"]: L["h8"] + nblk * hb * I].view(nblk, I // 128, hb, 128)
        h8 = h8.permute(0, 2, 1, 3).reshape(nblk * hb, I)
        rt = torch.as_tensor(rows, device=self.ws.device)
        h8 = h8[rt].cpu().numpy()
        words = sfs // 4
        raw = self.ws[L["h_sf"]: L["h_sf"] + nblk * hb * sfs].cpu().numpy()
        hs = raw[blocked_scale_bytes(rows, I // 128, words, hb)]
        return h8, hs


HALF_TILE_ROWS = 128


def blocked_scale_bytes(rows, nblocks, words, hblk):
    """Byte offsets [len(rows), nblocks] of the scale byte of (padded row, 128-column block)
    in the blocked scale layout (include/moe.h): rows in blocks of hblk, block b holding
    word 0 of its rows, then word 1, ...; within each 64-row group, row 16f + i at position
    4i + f; byte j % 4 of word j // 4."""
    p = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.arange(nblocks, dtype=np.int64)[None, :]
    r = p % hblk
    pos = (r // 64) * 64 + (r % 16) * 4 + (r // 16) % 4
    word = ((p // hblk) * words + j // 4) * hblk + pos
    return word * 4 + j % 4


def scheduled_tile_list(ref: dict, block_m: int):
    """The order in which the GEMMs take the oracle's tiles (one per block_m padded rows of
    an expert, in row order). With 256-row tiles, an expert's last tile that holds at most
    128 rows is a half tile, run as one 128-row tile after every full tile: full tiles keep
    their order, then the half tiles in expert order. The set of tiles is the oracle's; only
    this order is a scheduling choice. Returns (tile_expert, tile_row0, number of full tiles)."""
    te, tr = ref["tile_expert"], ref["tile_row0"]
    if block_m != 2 * HALF_TILE_ROWS:
        return te, tr, len(te)
    counts, offsets = ref["counts"], ref["offsets"]
    half = set()
    for e, c in enumerate(counts):
        if c == 0:
            continue
        pad = -(-int(c) // block_m) * block_m
        if c - (pad - block_m) <= HALF_TILE_ROWS:
            half.add(int(offsets[e]) + pad - block_m)
    full = [i for i in range(len(te)) if int(tr[i]) not in half]
    halves = [i for i in range(len(te)) if int(tr[i]) in half]
    order = np.array(full + halves, dtype=np.int64)
    return te[order], tr[order], len(full)


def check_routing(got: dict, idx_np: np.ndarray, E: int):
    ref = oracle.route(idx_np, E, got["block_m"])
    for key in ("counts", "offsets", "perm", "inv"):
        assert np.array_equal(got[key], ref[key]), f"routing field {key} differs"
    te, tr, n_full = scheduled_tile_list(ref, got["block_m"])
    assert np.array_equal(got["tile_expert"], te), "tile list (experts) differs"
    assert np.array_equal(got["tile_row0"], tr), "tile list (first rows) differs"
    assert int(got["meta"][3]) == n_full, "number of full tiles differs"
    assert int(got["num_invalid"]) == int(ref["num_invalid"])
    return ref


def _e4m3_half_gap() -> np.ndarray:
    """For each e4m3 code: half the larger of the two gaps to its neighbours on the grid
    (the widest distance from which round-to-nearest can land on it)."""
    pos = np.array([oracle.e4m3_value(c) for c in range(0x7F)])
    up = np.diff(pos, append=pos[-1] + (pos[-1] - pos[-2]))
    down = np.diff(pos, prepend=-pos[1])          # the gap below 0 is the one to -min
    half = 0.5 * np.maximum(up, down)
    out = np.zeros(256)
    out[:0x7F] = half
    out[0x80:0xFF] = half
    out[0x7F] = out[0xFF] = np.nan
    return out


_HALF_GAP = _e4m3_half_gap()


def check_intermediates(run: Run, ref: dict, inv: np.ndarray, stats: dict = None):
    """Compare GPU h8/h_sf with the oracle's requantised intermediate slot by slot.

    Each element is decoded on both sides and measured on the e4m3 grid of the coarser of
    the two block scales. An element that differs must be one step apart, with one
    exception: an element further apart passes only where its exact |h| is at most
    FAR_BELOW_FRACTION of its block's largest |h| and the GPU's value is a round-to-nearest
    result of some h' within the FP32 accumulation error bound of the exact h (a dot product
    that cancels leaves an element whose grid is finer than the FP32 error of the sum).
    Such excused elements are counted, printed and capped at FAR_EXCUSED_MAX_RATE of the
    compared elements. With at least RATE_MIN_ELEMENTS elements the differing ones may be
    at most 0.1 % of them; a smaller sample cannot estimate that rate, and there every
    differing element must be explained by the FP32 bound instead (the pooled rate of many
    small samples is checked by the caller from `stats`: n, differing, excused)."""
    slots = sorted(ref["h8"].keys())
    if not slots:
        return 0.0
    rows = inv[np.array(slots)]
    assert np.all(rows >= 0)
    g8, gsf = run.intermediates(rows)
    r8 = np.stack([ref["h8"][s] for s in slots])
    rsf = np.stack([ref["h_sf"][s] for s in slots])
    gs = np.repeat(gsf, 128, axis=1)
    rs = np.repeat(rsf, 128, axis=1)
    dist = oracle.e4m3_code_distance(g8, gs, r8, rs)
    assert np.all(np.isfinite(dist)), "a NaN code or a NaN scale byte in the GPU intermediate"
    n = dist.size
    n_diff = int((dist > 0).sum())
    frac = n_diff / n
    far = dist > 1
    excused = np.zeros_like(far)
    unexplained = dist > 0
    if ref.get("h"):
        h = np.stack([ref["h"][s] for s in slots])
        hb = np.stack([ref["h_bound"][s] for s in slots])
        scale = np.ldexp(1.0, gs.astype(np.int64) - 127)
        vg = oracle.E4M3_TABLE[g8] * scale
        within = np.abs(vg - h) <= hb + _HALF_GAP[g8] * scale
        amax = np.repeat(np.abs(h).reshape(h.shape[0], -1, 128).max(axis=2), 128, axis=1)
        small = np.abs(h) <= FAR_BELOW_FRACTION * amax
        excused = far & within & small
        unexplained = (dist > 0) & ~within
        for i, c in list(zip(*np.nonzero(excused)))[:4]:
            print(f"[intermediates] excused: slot {slots[i]} column {c}, distance {dist[i, c]}, "
                  f"|h| / block max = {abs(h[i, c]) / amax[i, c]:.2e}", flush=True)
    n_far = int(far.sum())
    n_excused = int(excused.sum())
    flips = np.nonzero(gsf != rsf)
    if len(flips[0]):
        print(f"[intermediates] {len(flips[0])} blocks with a different scale byte: " + ", ".join(
            f"slot {slots[i]} block {b} gpu {gsf[i, b]} oracle {rsf[i, b]}"
            for i, b in list(zip(*flips))[:8]), flush=True)
    cap = int(np.ceil(FAR_EXCUSED_MAX_RATE * n))
    print(f"[intermediates] compared {n}, differing {n_diff} ({frac:.2e}), more than one code "
          f"apart {n_far} (excused by the FP32 bound far below the block max: {n_excused}, "
          f"cap {cap})", flush=True)
    assert n_far == n_excused, (f"{n_far - n_excused} intermediates further than one code and not "
                                f"excused (max distance {dist.max()})")
    assert n_excused <= cap, f"{n_excused} excused intermediates exceed the cap {cap}"
    if n >= RATE_MIN_ELEMENTS:
        assert frac <= OFF_BY_ONE_MAX, f"{frac:.2e} of intermediates differ"
    else:
        # too few elements to estimate a 0.1 % rate: every differing element must instead be
        # explained by FP32 accumulation (a round-to-nearest result of some value within the
        # FP32 accumulation bound of the exact h)
        assert ref.get("h"), "a small sample needs the oracle's accumulation bounds"
        assert not unexplained.any(), (f"{int(unexplained.sum())} of {n} intermediates "
                                       f"differ beyond the FP32 accumulation bound")
    if stats is not None:
        stats["n"] = stats.get("n", 0) + n
        stats["differing"] = stats.get("differing", 0) + n_diff
        stats["excused"] = stats.get("excused", 0) + n_excused
    return frac


def check_y(y_bits: np.ndarray, ref: dict, tokens=None, cols=None, run: Run = None,
            inv: np.ndarray = None, host: dict = None):
    """y rows against the oracle: max |y_gpu - y_ref| / max |y_ref| <= Y_TOL per row, a row
    the oracle gives as exactly zero exactly zero. A row over Y_TOL passes only as described
    at ROW_EXCUSED_MAX_RATE, which needs the run, the routing's inv and the host inputs.
    Returns the largest end-to-end row error."""
    yg = y_bits if tokens is None else y_bits[np.asarray(tokens)]
    if cols is not None:
        yg = yg[:, np.asarray(cols)]
    err = oracle.y_row_error(yg, ref["y"])
    rows = np.arange(len(err)) if tokens is None else np.asarray(tokens)
    worst = np.argsort(err)[::-1][:3]
    print("[y] worst rows (token: error): " + ", ".join(f"{int(rows[i])}: {err[i]:.3e}" for i in worst),
          flush=True)
    assert np.all(np.isfinite(err)), "a non-finite y value, or a row the oracle gives as exactly 0 is non-zero"
    over = np.nonzero(err > Y_TOL)[0]
    if len(over):
        assert run is not None and inv is not None and host is not None, f"max row error {err.max():.3e}"
        cap = int(np.ceil(ROW_EXCUSED_MAX_RATE * len(err)))
        assert len(over) <= cap, f"{len(over)} rows over {Y_TOL} (cap {cap}); max {err.max():.3e}"
        idx = np.asarray(host["topk_idx"])
        k = idx.shape[1]
        E = np.asarray(host["w2"]).shape[0]
        I = 2 * np.asarray(host["w2"]).shape[2]
        toks = [int(rows[i]) for i in over]
        slots = [t * k + j for t in toks for j in range(k) if 0 <= int(idx[t, j]) < E]
        g8, gsf = run.intermediates(inv[np.array(slots)])
        hdeq = {}
        for i, sl in enumerate(slots):
            hdeq[sl] = oracle.dequant_fp8_rows(g8[i:i + 1], gsf[i:i + 1], I)[0]
        differs = {t: False for t in toks}
        for i, sl in enumerate(slots):
            d = oracle.e4m3_code_distance(g8[i], np.repeat(gsf[i], 128), ref["h8"][sl],
                                          np.repeat(ref["h_sf"][sl], 128))
            differs[sl // k] |= bool((d > 0).any())
        assert all(differs.values()), (f"rows over {Y_TOL} with the oracle's own intermediate in "
                                       f"every slot: {[t for t, v in differs.items() if not v]}")
        cond = oracle.linear2_combine(hdeq, idx, host["topk_weights"], host["w2"], host["w2_sf"],
                                      tokens=toks, cols=cols)
        yo = y_bits[np.array(toks)]
        if cols is not None:
            yo = yo[:, np.asarray(cols)]
        e2 = oracle.y_row_error(yo, cond["y"])
        print(f"[y] {len(toks)} rows over {Y_TOL} (cap {cap}), each with an accepted intermediate "
              f"difference; against the oracle's Linear2 and combine on the GPU's intermediate: "
              + ", ".join(f"{t}: {e:.3e}" for t, e in zip(toks, e2)), flush=True)
        assert e2.max() <= Y_TOL, f"max row error {e2.max():.3e} on the GPU's own intermediate"
    return float(err.max())
