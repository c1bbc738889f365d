"""Comparison helpers shared by the parity tests (test infrastructure).

``check_attention`` compares attention outputs with the oracle's to the
tolerances of the hot path (max-abs 4e-3, relative L2 5e-3, lse 1e-3) and
reports the worst (query, head) row. ``check_topk_properties`` checks that an
index set is a correct top-k of a score matrix under the tie rule (lower key
index wins), using torch ops that run on CPU or GPU tensors alike.
"""
import sys

import numpy as np

ATOL = 4e-3
RTOL_L2 = 5e-3
LSE_ATOL = 1e-3


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def attention_errors(got_out, ref_out):
    """(max-abs, rel-L2, sum of squared errors, sum of squared reference, worst (row, head))."""
    d = got_out.astype(np.float64) - ref_out
    if d.size == 0:
        return 0.0, 0.0, 0.0, 0.0, None
    ad = np.abs(d)
    flat = int(np.argmax(ad))
    max_abs = float(ad.reshape(-1)[flat])
    worst = np.unravel_index(flat, ad.shape)[:2]
    se = float(np.sum(d * d))
    sr = float(np.sum(ref_out * ref_out))
    rel = float(np.sqrt(se) / max(np.sqrt(sr), 1e-300))
    return max_abs, rel, se, sr, (int(worst[0]), int(worst[1]))


def check_attention(got_out, got_lse, ref_out, ref_lse, label, row_ids=None):
    max_abs, rel, _, _, worst = attention_errors(got_out, ref_out)
    where = ""
    if worst is not None:
        r, h = worst
        q = row_ids[r] if row_ids is not None else r
        row_rel = float(np.linalg.norm(got_out[r, h].astype(np.float64) - ref_out[r, h]) /
                        max(np.linalg.norm(ref_out[r, h]), 1e-300))
        where = f" worst row: query {q} head {h} (row rel_l2 {row_rel:.3e})"
    say(f"{label}: attention max_abs={max_abs:.3e} rel_l2={rel:.3e}{where}")
    assert max_abs <= ATOL, f"{label}: max abs err {max_abs}"
    assert rel <= RTOL_L2, f"{label}: rel L2 {rel}"
    if got_lse is not None:
        fin = np.isfinite(ref_lse)
        assert np.array_equal(np.isfinite(got_lse), fin), f"{label}: lse finiteness differs"
        if fin.any():
            lerr = float(np.abs(got_lse[fin] - ref_lse[fin]).max())
            assert lerr <= LSE_ATOL, f"{label}: lse err {lerr}"


def check_topk_properties(torch, scores, idx, offset, k, label, chunk=256):
    """Asserts that ``idx`` holds, for every row, the top-k causal keys of ``scores``.

    Per row i (position p = offset + i, n = p + 1 causal keys):
      * exactly min(k, n) valid slots, forming a prefix, strictly ascending,
        every valid index causal; -1 in the rest;
      * when n > k, with T the smallest selected score: every causal key with
        a score above T is selected, and among the keys scoring exactly T the
        selected ones are the lowest indices.
    Those two conditions characterise the unique result of the (score desc,
    key asc) order.
    """
    n_q = idx.shape[0]
    pos = torch.arange(n_q, device=idx.device, dtype=torch.int64) + offset
    n = pos + 1
    valid = idx >= 0
    cnt = valid.sum(1)
    assert torch.equal(cnt, torch.clamp(n, max=k)), f"{label}: wrong selected count"
    sel = torch.where(valid, idx.long(), torch.full_like(idx.long(), -1))
    d = sel[:, 1:] - sel[:, :-1]
    both = valid[:, 1:] & valid[:, :-1]
    assert bool(((d > 0) | ~both).all()), f"{label}: not strictly ascending"
    assert bool((sel.max(1).values <= pos).all()), f"{label}: non-causal index"
    assert bool((valid[:, 1:] <= valid[:, :-1]).all()), f"{label}: padding before a valid slot"
    assert bool((idx[~valid] == -1).all()), f"{label}: padding other than -1"
    rows = torch.nonzero(n > k).flatten()
    for r0 in range(0, rows.numel(), chunk):
        rr = rows[r0:r0 + chunk]
        S = scores[rr]  # [R][ld]
        sel_idx = idx[rr].long()
        sel_s = torch.gather(S, 1, sel_idx)
        thr = sel_s.min(1).values  # the k-th largest selected score
        col = torch.arange(S.shape[1], device=S.device)
        causal = col[None, :] <= pos[rr][:, None]
        mark = torch.zeros_like(S, dtype=torch.bool)
        mark.scatter_(1, sel_idx, True)
        # no causal key above the threshold is left out
        assert not bool(((S > thr[:, None]) & causal & ~mark).any()), f"{label}: a larger score was left out"
        # ties at the threshold: the kept ones are the lowest indices
        eq = (S == thr[:, None]) & causal
        n_eq_kept = (sel_s == thr[:, None]).sum(1)
        rank = torch.cumsum(eq.int(), 1)  # 1-based rank among ties
        kept_tie = eq & mark
        assert bool(((rank <= n_eq_kept[:, None]) == kept_tie)[eq].all()), f"{label}: tie rule violated"
