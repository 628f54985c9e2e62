"""Oracle runs of whole workloads (test infrastructure only).

Each function takes the workload parameters and the stored inputs as numpy
arrays (bf16 as uint16/int16 bit patterns, FP8 and MXFP4 as uint8 codes),
decodes them exactly and follows the method step by step with the oracle's
own compression, indexer and attention. Inputs only ever come from the seeded
generators; nothing here reads a GPU result.
"""

import numpy as np

from . import attention, codecs, compress, indexer


def _f64(a, kind):
    if kind == "f32":
        return np.asarray(a, np.float32).astype(np.float64)
    return codecs.decode_bf16(np.asarray(a).view(np.uint16))


def _index_one(q_dec, w, keys_dec, t, m, k, exact_fp32):
    n_vis = min(indexer.n_visible(t, m), keys_dec.shape[0])
    keys = keys_dec[:n_vis]
    s = indexer.scores_mxfp4(q_dec, w, keys) if exact_fp32 else indexer.scores(q_dec, w, keys)
    return indexer.topk(s, n_vis, k), s


def tiny_fp32(p, a):
    """p: params dict; a: raw, logits_csa, logits_hca, bias_csa, bias_hca, q, q_idx, w_idx, k_idx,
    q_pos (numpy). Returns stores, idx, o/lse for both mechanisms."""
    L, m, w, mp, W, k = p["L"], p["m"], p["w"], p["m_prime"], p["W"], p["topk"]
    dn, dr = p["d_nope"], p["d_rope"]
    raw = _f64(a["raw"], "f32")
    y_c = compress.compress(raw, _f64(a["logits_csa"], "f32"), a["bias_csa"], m, w, 0, L // m)
    y_h = compress.compress(raw, _f64(a["logits_hca"], "f32"), a["bias_hca"], mp, mp, 0, L // mp)
    # the same weights applied to |x|: the magnitude scale of each entry's weighted sum
    ya_c = compress.compress(np.abs(raw), _f64(a["logits_csa"], "f32"), a["bias_csa"], m, w, 0, L // m)
    ya_h = compress.compress(np.abs(raw), _f64(a["logits_hca"], "f32"), a["bias_hca"], mp, mp, 0, L // mp)
    csa_st, hca_st = compress.encode(y_c, "f32", dn, dr), compress.encode(y_h, "f32", dn, dr)
    csa_dec, hca_dec = compress.decode(csa_st, "f32"), compress.decode(hca_st, "f32")
    scale = 1.0 / np.sqrt(dn + dr)
    out = dict(y_csa=y_c, y_hca=y_h, yabs_csa=ya_c, yabs_hca=ya_h, idx=[], scores=[], o_csa=[], lse_csa=[], o_hca=[], lse_hca=[])
    for i, t in enumerate(np.asarray(a["q_pos"]).tolist()):
        idx, s = _index_one(_f64(a["q_idx"][i], "f32"), _f64(a["w_idx"][i], "f32"), _f64(a["k_idx"], "f32"),
                            t, m, k, False)
        out["idx"].append(idx)
        out["scores"].append(s)
        q = _f64(a["q"][i], "f32")
        o, l = attention.csa(q, t, csa_dec, idx, raw, W, scale)
        out["o_csa"].append(o)
        out["lse_csa"].append(l)
        o, l = attention.hca(q, t, hca_dec, mp, raw, W, scale)
        out["o_hca"].append(o)
        out["lse_hca"].append(l)
    return out


def decode_bf16(p, a, seqs):
    """Decode queries of the sequences in `seqs`. a: raw/logits as [B*L, D] bf16 bits, biases, q [B,H,D],
    q_idx [B,Hi,d], w_idx, k_idx [B*L/m, d] (bf16 bits). Compresses only the entries each query needs."""
    L, m, w, mp, W, k = p["L"], p["m"], p["w"], p["m_prime"], p["W"], p["topk"]
    dn, dr = p["d_nope"], p["d_rope"]
    n_c, n_h = L // m, L // mp
    scale = 1.0 / np.sqrt(dn + dr)
    res = {}
    for b in seqs:
        raw = _f64(a["raw"][b * L:(b + 1) * L], "bf16")
        t = L - 1
        idx, s = _index_one(_f64(a["q_idx"][b], "bf16"), a["w_idx"][b], _f64(a["k_idx"][b * n_c:(b + 1) * n_c],
                                                                              "bf16"), t, m, k, False)
        lc = _f64(a["logits_csa"][b * L:(b + 1) * L], "bf16")
        sel = idx[idx >= 0]
        ent = np.zeros((n_c, dn + dr))
        csa_y, csa_yabs = {}, {}
        for j in sel:
            y = compress.compress(raw, lc, a["bias_csa"], m, w, int(j), 1)
            csa_y[int(j)] = y[0]
            csa_yabs[int(j)] = compress.compress(np.abs(raw), lc, a["bias_csa"], m, w, int(j), 1)[0]
            ent[j] = compress.decode(compress.encode(y, "bf16", dn, dr), "bf16")[0]
        lh = _f64(a["logits_hca"][b * L:(b + 1) * L], "bf16")
        y_h = compress.compress(raw, lh, a["bias_hca"], mp, mp, 0, n_h)
        ya_h = compress.compress(np.abs(raw), lh, a["bias_hca"], mp, mp, 0, n_h)
        hca_dec = compress.decode(compress.encode(y_h, "bf16", dn, dr), "bf16")
        q = _f64(a["q"][b], "bf16")
        o_c, l_c = attention.csa(q, t, ent, idx, raw, W, scale)
        o_h, l_h = attention.hca(q, t, hca_dec, mp, raw, W, scale)
        res[b] = dict(idx=idx, scores=s, o_csa=o_c, lse_csa=l_c, o_hca=o_h, lse_hca=l_h, y_hca=y_h, yabs_hca=ya_h,
                      csa_y=csa_y, csa_yabs=csa_yabs)
    return res


def split_rows(a, prefix, rows):
    """Decode rows of a split-layout store held as numpy arrays."""
    st = {"nope": a[f"{prefix}_nope"][rows], "scale": a[f"{prefix}_scale"][rows], "rope": a[f"{prefix}_rope"][rows]}
    return compress.decode(st, "split")


def decode_1m_query(p, a, b):
    """One decode query (sequence b) over precompressed caches: MXFP4 index, CSA and HCA attention.
    a: q_csa, q_hca [B,H,D] bf16 bits; q_idx [B,Hi,32] + q_idx_scale; w_idx; k_idx [B*n_c, 32] +
    k_idx_scale; csa_/hca_/win_csa_/win_hca_ nope/scale/rope arrays."""
    L, m, mp, W, k = p["L"], p["m"], p["m_prime"], p["W"], p["topk"]
    dn, dr = p["d_nope"], p["d_rope"]
    n_c, n_h = L // m, L // mp
    t = L - 1
    qd = codecs.decode_mxfp4(a["q_idx"][b], a["q_idx_scale"][b])
    keys = codecs.decode_mxfp4(a["k_idx"][b * n_c:(b + 1) * n_c], a["k_idx_scale"][b * n_c:(b + 1) * n_c])
    idx, s = _index_one(qd, a["w_idx"][b], keys, t, m, k, True)
    sel = idx[idx >= 0]
    ent = np.zeros((n_c, dn + dr))
    ent[sel] = split_rows(a, "csa", b * n_c + sel)
    scale = 1.0 / np.sqrt(dn + dr)

    def window(prefix):
        rows = split_rows(a, prefix, np.arange(b * W, (b + 1) * W))
        return lambda pos: rows[np.asarray(pos) - (L - W)]

    o_c, l_c = attention.csa(_f64(a["q_csa"][b], "bf16"), t, ent, idx, window("win_csa"), W, scale)
    hca_dec = split_rows(a, "hca", np.arange(b * n_h, (b + 1) * n_h))
    o_h, l_h = attention.hca(_f64(a["q_hca"][b], "bf16"), t, hca_dec, mp, window("win_hca"), W, scale)
    return dict(idx=idx, scores=s, o_csa=o_c, lse_csa=l_c, o_hca=o_h, lse_hca=l_h)


def prefill_query(p, a, qi, chunk_csa, chunk_hca, split_window=False, memo=None):
    """One chunked-prefill query. chunk_csa/chunk_hca: callables (b) -> the oracle's own decoded
    entries of sequence b's chunk (compressed from the raw chunk rows). split_window: the window
    rows are held in the cache layout (DeepSeek-V4 page, efficiency section: FP8 for the
    non-RoPE dims, BF16 for the RoPE dims), so attention sees each raw row after the oracle's
    own split encoding and decoding; otherwise it sees the raw bf16 rows. memo: an optional dict
    that keeps each sequence's decoded keys, entries and window rows between calls (the same
    arrays, decoded once)."""
    m, mp, W, k, chunk = p["m"], p["m_prime"], p["W"], p["topk"], p["chunk"]
    dn, dr = p["d_nope"], p["d_rope"]
    b = int(a["q_seq"][qi])
    t = int(a["q_pos"][qi])
    P = p["prefixes"][b]
    crb, hrb = p["csa_row_begin"][b], p["hca_row_begin"][b]
    n_c, n_h = (P + chunk) // m, (P + chunk) // mp
    rows = W + chunk
    memo = {} if memo is None else memo
    key = (b, bool(split_window))
    if key not in memo:
        keys = codecs.decode_mxfp4(a["k_idx"][crb:crb + n_c], a["k_idx_scale"][crb:crb + n_c])
        csa_ent = np.concatenate([split_rows(a, "csa", np.arange(crb, crb + P // m)), chunk_csa(b)])
        hca_ent = np.concatenate([split_rows(a, "hca", np.arange(hrb, hrb + P // mp)), chunk_hca(b)])
        raw = _f64(a["raw"][b * rows:(b + 1) * rows], "bf16")
        if split_window:
            raw = compress.decode(compress.encode(raw, "split", dn, dr), "split")
        memo[key] = (keys, csa_ent, hca_ent, raw)
    keys, csa_ent, hca_ent, raw = memo[key]
    qd = codecs.decode_mxfp4(a["q_idx"][qi], a["q_idx_scale"][qi])
    idx, s = _index_one(qd, a["w_idx"][qi], keys, t, m, k, True)
    win = lambda pos: raw[np.asarray(pos) - (P - W)]
    scale = 1.0 / np.sqrt(dn + dr)
    q = _f64(a["q"][qi], "bf16")
    o_c, l_c = attention.csa(q, t, csa_ent, idx, win, W, scale)
    o_h, l_h = attention.hca(q, t, hca_ent, mp, win, W, scale)
    return dict(idx=idx, scores=s, o_csa=o_c, lse_csa=l_c, o_hca=o_h, lse_hca=l_h)


def prefill_chunk_entries(p, a, b):
    """The oracle's own compression of sequence b's chunk: (csa_y, csa_decoded, hca_y, hca_decoded,
    csa_yabs, hca_yabs); *_yabs are the same weights applied to |x|."""
    m, w, mp, W, chunk = p["m"], p["w"], p["m_prime"], p["W"], p["chunk"]
    dn, dr = p["d_nope"], p["d_rope"]
    P = p["prefixes"][b]
    rows = W + chunk
    raw = _f64(a["raw"][b * rows:(b + 1) * rows], "bf16")
    lc = _f64(a["logits_csa"][b * rows:(b + 1) * rows], "bf16")
    lh = _f64(a["logits_hca"][b * rows:(b + 1) * rows], "bf16")
    y_c = compress.compress(raw, lc, a["bias_csa"], m, w, P // m, chunk // m, first_pos=P - W)
    y_h = compress.compress(raw, lh, a["bias_hca"], mp, mp, P // mp, chunk // mp, first_pos=P - W)
    ya_c = compress.compress(np.abs(raw), lc, a["bias_csa"], m, w, P // m, chunk // m, first_pos=P - W)
    ya_h = compress.compress(np.abs(raw), lh, a["bias_hca"], mp, mp, P // mp, chunk // mp, first_pos=P - W)
    return (y_c, compress.decode(compress.encode(y_c, "split", dn, dr), "split"),
            y_h, compress.decode(compress.encode(y_h, "split", dn, dr), "split"), ya_c, ya_h)
