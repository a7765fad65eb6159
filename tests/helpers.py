"""Shared test helpers: device upload, scratch reservation, tolerance checks,
page-style report."""
import numpy as np
import torch

import sparse_mla_decode_page_amd as mlasd

# Tolerances for the attention outputs (bf16 out vs fp64 oracle): elementwise
# |d| <= 2e-3 + 1e-2 * |ref| for out, |d| <= 1e-3 for lse.  For caches whose
# values span many binades (group amax up to 1e5 and more) the bar is the
# max-norm form of the same numbers, per query: max|d| <= max(2e-3, 1e-2 *
# max|ref|) -- the elementwise absolute term presumes unit-scale values, and
# no rounding of P (fp16 here, bf16 in the pages' kernel) keeps a sum of
# values near 1e5 that cancel within 2e-3.
OUT_ATOL = 2e-3
OUT_RTOL = 1e-2
LSE_ATOL = 1e-3


def to_device(w, device="cuda"):
    return dict(
        q=torch.from_numpy(w.q_bits.view(np.int16)).view(torch.bfloat16).to(device),
        kv_pages=torch.from_numpy(w.kv_pages).to(device),
        page_table=torch.from_numpy(w.page_table).to(device),
        topk_idx=torch.from_numpy(w.topk_idx).to(device),
        seq_lens=torch.from_numpy(w.seq_lens).to(device),
    )


def reserve_for(batch, topk, nsplit=None, head_groups=None, stream=None):
    """Reserve the split scratch a decode of this shape and plan needs on
    `stream` (a host call: never inside graph capture)."""
    n = mlasd.workspace_size(batch, topk, int(nsplit or 0), int(head_groups or 0))
    if n:
        mlasd.reserve(n, stream=stream)


def decode(d, scale, nsplit=None, head_groups=None, stream=None, out=None, lse=None, reserve=True):
    """mla_sparse_decode on uploaded tensors, reserving its scratch first."""
    if reserve:
        reserve_for(d["seq_lens"].shape[0], d["topk_idx"].shape[1], nsplit, head_groups, stream)
    return mlasd.mla_sparse_decode(d["q"], d["kv_pages"], d["page_table"], d["topk_idx"], d["seq_lens"],
                                   scale, out=out, lse=lse, stream=stream, nsplit=nsplit,
                                   head_groups=head_groups)


def check_attention(out, lse, ref_out, ref_lse, label="", maxnorm=False):
    """Elementwise comparison (per-query max-norm with `maxnorm`); returns the
    pages-style report line."""
    o = out.float().cpu().double().numpy()
    l = lse.cpu().double().numpy()
    assert o.shape == ref_out.shape and l.shape == ref_lse.shape
    d = np.abs(o - ref_out)
    if maxnorm:
        per_q = d.reshape(d.shape[0], -1).max(axis=1) if d.size else np.zeros(0)
        bound = np.maximum(OUT_ATOL, OUT_RTOL * np.abs(ref_out).reshape(ref_out.shape[0], -1).max(axis=1))
        n_bad = int((~(per_q <= bound)).sum())
    else:
        bad = ~(d <= OUT_ATOL + OUT_RTOL * np.abs(ref_out))
        n_bad = int(bad.sum())
    inf_ref = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(l), inf_ref), f"{label}: -inf lse pattern differs"
    dl = np.abs(l[~inf_ref] - ref_lse[~inf_ref]) if (~inf_ref).any() else np.zeros(1)
    maxref = np.abs(ref_out).max() if ref_out.size else 0.0
    line = (f"{label}: out max|d|={d.max() if d.size else 0:.3e} mean={d.mean() if d.size else 0:.3e} "
            f"rel={(d.max() / maxref) if maxref > 0 else 0:.3e} | lse max|d|={dl.max():.3e} | "
            f"outside tol: {n_bad}/{d.shape[0] if maxnorm else d.size}{' queries (max-norm)' if maxnorm else ''}")
    print(line, flush=True)
    assert n_bad == 0, line
    assert dl.max() <= LSE_ATOL, line
    return line
