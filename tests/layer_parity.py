"""Stage-by-stage, element-wise parity of one GPU forward against the oracle.

Each stage is checked on the GPU's own input to it, so every comparison is
either bit-exact or bounded by the arithmetic that differs (tests/parity.py):

  sort        offsets, counts, pair -> row, row -> pair         bit-exact
  A1          sorted, padded, quantized X  (= oracle Q(x_t))     bit-exact
  y1          FC1 of the unfused forward vs the oracle's y1      FP32-accumulation bound
  h           fused h == unfused h; h vs oracle producer(y1)     bit-exact; <= 1 BF16 ulp
  maxima      per-32-column max |h| of the GPU's h              bit-exact
  A2          quantized h  (= oracle Q(h_gpu))                  bit-exact
  y2          FC2 vs oracle FC2 on h_gpu                         FP32-accumulation bound
  combine     out vs oracle combine of the GPU's y2              bit-exact
  end to end  out vs the oracle's own forward, every token:     composed bound
              y2 within the FC2 bound plus, for a pair whose
              A2 row is not the oracle's Q(h_ref) (an h element
              one ulp apart next to a quantization decision),
              g_w ||w|| times the distance between the two
              dequantized rows (Cauchy-Schwarz) and one BF16
              ulp; then the FP32 slot-order sum's own bound;
              and the whole output within relative L2 1e-2

Sources: the miniTE summary page, "how it differs" and "how to use it";
the article, sections 4.4 and 4.5.
"""
from __future__ import annotations

import numpy as np

import moe_workloads as W
from tests import parity as PB
from tests.helpers import gemm_to_logical, rel_l2, to_host

REL_L2_TOL = 1e-2


def ws_array(ws, off, dtype, count):
    return to_host(ws[off:off + count * np.dtype(dtype).itemsize]).view(dtype)


def oracle_weights(orc, w1, w2, ids, mode):
    """Oracle weights for the experts that ids use; returns (weights, ids remapped)."""
    used = np.unique(ids)
    remap = np.full(int(w1.shape[0]), -1, np.int32)
    remap[used] = np.arange(used.size)
    return orc.DequantWeights(w1[used], w2[used], mode), remap[ids]


def check_route(orc, E, K, T, lay, ws, ids, capacity=0):
    """Sort metadata bit-exact against the oracle's layout (contiguous or masked)."""
    got_off = ws_array(ws, lay.expert_off, np.int32, E + 1)
    got_cnt = ws_array(ws, lay.expert_count, np.int32, E)
    got_p2r = ws_array(ws, lay.pair2row, np.int32, T * K)
    assert np.array_equal(got_cnt, np.bincount(ids.reshape(-1), minlength=E)), "expert counts"
    if capacity == 0:
        off, pair2row, row2pair = orc.route(ids, E, 32)
        got_r2p = ws_array(ws, lay.row2pair, np.int32, int(off[-1]))
        assert np.array_equal(got_r2p, row2pair), "sorted row -> pair"
    else:
        off, pair2row, row2pair, used, _ = orc.route_masked(ids, E, 32, capacity)
        got_r2p = ws_array(ws, lay.row2pair, np.int32, E * capacity)
        assert np.array_equal(got_r2p[used], row2pair[used]), "sorted row -> pair (masked chunks)"
    assert np.array_equal(got_off, off), "expert offsets"
    assert np.array_equal(got_p2r, pair2row), "pair -> sorted row"
    return pair2row


def check_a1(orc, s, lay, ws, x, pair2row, mode):
    rows = int(lay.rows_cap)
    c = ws_array(ws, lay.a1_codes, np.uint8, rows * s.H // 2)
    sc = ws_array(ws, lay.a1_scales, np.uint8, rows * s.H // 16)
    g = ws_array(ws, lay.a1_g, np.float32, rows)
    lc, ls = gemm_to_logical(c, sc, rows, s.H)
    wc, wsc, wg = orc.quantize(x, mode)
    ok = pair2row >= 0
    tok = (np.arange(pair2row.size) // s.K)[ok]
    rws = pair2row[ok]
    assert np.array_equal(lc[rws], wc[tok]), "A1 codes"
    assert np.array_equal(ls[rws], wsc[tok]), "A1 scales"
    assert np.array_equal(g[rws].view(np.uint32), wg[tok].view(np.uint32)), "A1 g"
    return wc, wsc, wg


def e2e_check(what, out, ref_out, y2_g, y2_s, y2_r, an, w2n, e_pair, dA, moved, K, I, chunk=1024):
    """out [T, H] vs the oracle's, element-wise, for every token.  Per pair:
    y2_g (GPU) is within the FC2 bound of y2_s (oracle FC2 on the GPU's FC2
    input), and y2_s within g_w ||w|| dA + one BF16 ulp of y2_r (the oracle's
    own chain), dA being the distance between the two FC2 input rows (0 when
    equal, `moved` false); then the slot-order FP32 sum's bound."""
    T = out.shape[0]
    H = out.shape[1]
    c = PB.Check(what)
    for t0 in range(0, T, chunk):
        t = np.arange(t0, min(T, t0 + chunk))
        pr = (t[:, None] * K + np.arange(K)).reshape(-1)
        b2 = PB.gemm_bound(y2_s[pr], y2_g[pr], an[pr], w2n[e_pair[pr]], I)
        ys, yr = PB.vals(y2_s[pr]), PB.vals(y2_r[pr])
        b2 += w2n[e_pair[pr]] * dA[pr, None] + moved[pr, None] * PB.ulp_bf16(np.maximum(np.abs(ys), np.abs(yr)))
        bo = PB.combine_bound(y2_g[pr].reshape(t.size, K, H), y2_r[pr].reshape(t.size, K, H),
                              b2.reshape(t.size, K, H), ref_out[t], out[t])
        c.add(out[t], ref_out[t], bo, index_offset=t0)
    n_tok = int(moved.reshape(T, K).any(axis=1).sum())
    return c.report() + f"; {int(moved.sum())} pairs ({n_tok} tokens) with an FC2 input row differing from the oracle's"


def parity(orc, s, lay, ws, x, ids, probs, out, w1, w2, mode=0, y1_rows=None, capacity=0, label=""):
    """Every stage of one W4A4 forward (GPU buffers in workspace `ws`) against
    the oracle; y1_rows: the unfused forward's y1 [rows_cap, 2I] (host), if run."""
    T, H, I, K = x.shape[0], s.H, s.I, s.K
    P = T * K
    reports = []
    pair2row = check_route(orc, s.E, K, T, lay, ws, ids, capacity)
    xc, xs, gx = check_a1(orc, s, lay, ws, x, pair2row, mode)
    wts, ids_r = oracle_weights(orc, w1, w2, ids, mode)
    ref_out, mid = orc.moe_forward(x, ids_r, probs, wts, mode, intermediates=True)
    e_pair = ids_r.reshape(-1)
    rows = int(lay.rows_cap)
    h_all = ws_array(ws, lay.h, np.uint16, rows * I).reshape(rows, I)
    y2_all = ws_array(ws, lay.y2, np.uint16, rows * H).reshape(rows, H)
    h_g, y2_g = h_all[pair2row], y2_all[pair2row]
    # weight-row norms times outer scales
    w1n = (PB.row_norms(wts.d1) * wts.g1).reshape(-1, 2 * I)
    w2n = (PB.row_norms(wts.d2) * wts.g2).reshape(-1, H)
    # FC1 and the producer, through the unfused forward's y1
    if y1_rows is not None:
        y1_g = y1_rows[pair2row]
        xn = PB.row_norms(orc.dequantize(xc, xs)) * gx
        c1 = PB.Check(f"{label} y1 (FC1)")
        PB.check_grouped_gemm(c1, y1_g, mid["y1"], np.repeat(xn, K), w1n, e_pair, H)
        reports.append(c1.report())
        hp, amaxp = orc.swiglu_prob(y1_g, probs.reshape(-1))
        cp = PB.Check(f"{label} h (producer on the GPU's y1)")
        PB.check_producer(cp, h_g, hp, y1_g, I)
        reports.append(cp.report() + f"; {int((h_g != hp).sum())} of {h_g.size} differ from the FP64 producer")
    # the producer's maxima are those of the BF16 tensor FC2 consumes
    part = ws_array(ws, lay.amax2_part, np.float32, rows * lay.n_part).reshape(rows, lay.n_part)[pair2row]
    hv = np.abs(W.bf16_bits_to_f32(h_g))
    for j in range(lay.n_part):
        assert np.array_equal(part[:, j], hv[:, 32 * j:32 * (j + 1)].max(axis=1)), f"column group {j} max"
    # A2 = Q(h_gpu) bit-exact
    c = ws_array(ws, lay.a2_codes, np.uint8, rows * I // 2)
    sc = ws_array(ws, lay.a2_scales, np.uint8, rows * I // 16)
    g = ws_array(ws, lay.a2_g, np.float32, rows)
    lc, ls = gemm_to_logical(c, sc, rows, I)
    hc, hs, hg = orc.quantize(h_g, mode)
    assert np.array_equal(lc[pair2row], hc) and np.array_equal(ls[pair2row], hs), "A2 = Q(h)"
    assert np.array_equal(g[pair2row].view(np.uint32), hg.view(np.uint32)), "A2 g"
    # FC2 on the GPU's h
    y2_s = orc.moe_fc2(h_g, ids_r, wts, True, mode)
    an = PB.row_norms(orc.dequantize(hc, hs)) * hg
    c2 = PB.Check(f"{label} y2 (FC2)")
    PB.check_grouped_gemm(c2, y2_g, y2_s, an, w2n, e_pair, I)
    reports.append(c2.report())
    # the combine, bit-exact on the GPU's y2
    assert np.array_equal(orc.combine(y2_g.reshape(T, K, H)), out), "combine of the GPU's y2"
    # end to end: every token against the oracle's own forward
    rc, rs, rg = orc.quantize(mid["h"], mode)
    aligned = (hc == rc).all(axis=1) & (hs == rs).all(axis=1) & (hg.view(np.uint32) == rg.view(np.uint32))
    assert np.array_equal(y2_s[aligned], mid["y2"][aligned]), "oracle FC2 on equal A2 rows"
    dA = PB.row_norms(orc.dequantize(hc, hs) * hg[:, None].astype(np.float64)
                      - orc.dequantize(rc, rs) * rg[:, None].astype(np.float64))
    reports.append(e2e_check(f"{label} out", out, ref_out, y2_g, y2_s, mid["y2"], an, w2n, e_pair, dA, ~aligned, K, I))
    rel, mx = rel_l2(out, ref_out)
    u = PB.ulp_dist(out, ref_out)
    reports.append(f"{label} out: rel L2 {rel:.2e}, max-abs {mx:.3e}, max {u.max():.1f} BF16 ulps, "
                   f"{int((u > 1).sum())} of {u.size} > 1 ulp, {int((u > 2).sum())} > 2 ulps")
    assert rel <= REL_L2_TOL, reports[-1]
    print("\n  " + "\n  ".join(reports))
    return ref_out, mid


def parity_w4a16(orc, s, lay, ws, x, ids, probs, out, w1, w2, label=""):
    """The W4A16 forward against its oracle: sort bit-exact; h within the bound
    propagated from y1's FP32-accumulation bound through the producer; y2 on
    the GPU's h within the FC2 bound; the combine bit-exact; tokens whose h
    equals the oracle's bounded element-wise; relative L2 of the output."""
    T, H, I, K = x.shape[0], s.H, s.I, s.K
    reports = []
    pair2row = check_route(orc, s.E, K, T, lay, ws, ids)
    wts, ids_r = oracle_weights(orc, w1, w2, ids, 0)
    ref_out, mid = orc.moe_forward_w4a16(x, ids_r, probs, wts, intermediates=True)
    e_pair = ids_r.reshape(-1)
    rows = int(lay.rows_cap)
    h_g = ws_array(ws, lay.h, np.uint16, rows * I).reshape(rows, I)[pair2row]
    y2_g = ws_array(ws, lay.y2, np.uint16, rows * H).reshape(rows, H)[pair2row]
    w1n = (PB.row_norms(wts.d1) * wts.g1).reshape(-1, 2 * I)
    w2n = (PB.row_norms(wts.d2) * wts.g2).reshape(-1, H)
    # h: bound of y1 (the GPU's y1 is within dy of the oracle's), propagated
    xn = np.repeat(PB.row_norms(PB.vals(x)), K)
    ch = PB.Check(f"{label} h (through y1's bound)")
    for i0 in range(0, h_g.shape[0], 4096):
        sl = slice(i0, min(h_g.shape[0], i0 + 4096))
        y1r = PB.vals(mid["y1"][sl])
        acc = 2.0 * H * PB.U * xn[sl, None] * w1n[e_pair[sl]] + 3.0 * PB.U * np.abs(y1r)
        dy = acc + PB.ulp_bf16(np.abs(y1r) + acc + PB.ulp_bf16(np.abs(y1r)))
        g, u = y1r[:, :I], y1r[:, I:]
        dg, du = dy[:, :I], dy[:, I:]
        assert g.min() > -64.0
        silu = g / (1.0 + np.exp(-g))
        p = probs.reshape(-1)[sl, None].astype(np.float64)
        # |silu'| <= 1.1 everywhere; silu(g') u' - silu(g) u, times p
        dh = p * (1.1 * dg * (np.abs(u) + du) + np.abs(silu) * du)
        hr, hgv = PB.vals(mid["h"][sl]), PB.vals(h_g[sl])
        bnd = dh + 1e-6 * np.abs(hr) + 2 * PB.ulp_bf16(np.maximum(np.abs(hr), np.abs(hgv)))
        ch.add(h_g[sl], mid["h"][sl], bnd, index_offset=i0)
    reports.append(ch.report())
    # FC2 on the GPU's h (BF16 activations, g_a = 1)
    y2_s = orc.moe_fc2(h_g, ids_r, wts, False)
    an = PB.row_norms(PB.vals(h_g))
    c2 = PB.Check(f"{label} y2 (FC2)")
    PB.check_grouped_gemm(c2, y2_g, y2_s, an, w2n, e_pair, I)
    reports.append(c2.report())
    assert np.array_equal(orc.combine(y2_g.reshape(T, K, H)), out), "combine of the GPU's y2"
    aligned = (h_g == mid["h"]).all(axis=1)
    assert np.array_equal(y2_s[aligned], mid["y2"][aligned]), "oracle FC2 on equal h rows"
    dA = PB.row_norms(PB.vals(h_g) - PB.vals(mid["h"]))
    reports.append(e2e_check(f"{label} out", out, ref_out, y2_g, y2_s, mid["y2"], an, w2n, e_pair, dA, ~aligned, K, I))
    rel, mx = rel_l2(out, ref_out)
    u = PB.ulp_dist(out, ref_out)
    reports.append(f"{label} out: rel L2 {rel:.2e}, max-abs {mx:.3e}, max {u.max():.1f} BF16 ulps, "
                   f"{int((u > 1).sum())} of {u.size} > 1 ulp, {int((u > 2).sum())} > 2 ulps")
    assert rel <= REL_L2_TOL, reports[-1]
    print("\n  " + "\n  ".join(reports))
    return ref_out
