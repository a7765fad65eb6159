"""Top-k selection (the step before the decode) against the oracle, bit for
bit: random and tie-heavy score rows, NaN / infinities / signed zeros, short,
empty and clamped sequences, the full B=64 x 65,536 shape, and the selection
chained before the decode in one captured graph -- each under the library's
plan, one workgroup per row, and long rows cut into 3 or 8 parts."""
import numpy as np
import pytest
import torch

import oracle as O
import sparse_mla_decode_page_amd as mlasd
from gen import synth as G
from helpers import check_attention, reserve_for, to_device

pytestmark = pytest.mark.gpu


def _select(scores, lens, k, parts=None):
    s = torch.from_numpy(np.ascontiguousarray(scores)).cuda()
    l = torch.from_numpy(np.asarray(lens, dtype=np.int32)).cuda()
    if parts is not None and parts > 1:
        mlasd.reserve(mlasd.topk_plan(s.shape[0], s.shape[1], parts)[1])
    out = mlasd.mla_topk_select(s, l, k, parts=parts)
    torch.cuda.synchronize()
    return out.cpu().numpy()


# None: the library's plan (a split only with enough scratch on the stream);
# 1: one workgroup per row; 3 and 8: the candidate pass of rows longer than
# max(k, 4096) cut into that many parts
PARTS = (None, 1, 3, 8)


def _check(scores, lens, k, label, parts=PARTS):
    ref = O.topk_select(scores, lens, k)
    for pa in parts:
        print(f"topk: {label} B={scores.shape[0]} max_len={scores.shape[1]} k={k} parts={pa}", flush=True)
        got = _select(scores, lens, k, pa)
        bad = np.argwhere(got != ref)
        assert len(bad) == 0, f"{label} parts={pa}: {len(bad)} slots differ, first at {bad[:3].tolist()}"


@pytest.mark.parametrize("k", [1, 7, 100, 512])
def test_random_rows(k):
    sc = G.indexer_scores(11, 6, 5000)
    _check(sc, [5000, 4999, 600, 100, 0, -3], k, "random")


@pytest.mark.parametrize("kind", ["ties", "special"])
@pytest.mark.parametrize("k", [33, 512])
def test_tie_heavy_rows(kind, k):
    sc = G.indexer_scores(12, 5, 3000, kind)
    _check(sc, [3000, 2048, 513, 512, 40], k, kind)


def test_short_empty_and_clamped_lengths():
    sc = G.indexer_scores(13, 6, 700, "special")
    _check(sc, [10 ** 6, 700, 701, 1, 0, -1], 512, "lengths")
    _check(G.indexer_scores(14, 3, 1), [1, 5, 0], 4, "max_len 1")


def test_full_shape_b64_65536():
    """The full shape under the library's plan with the scratch it asks for
    (4 parts per row on 256 CUs), then forced plans."""
    sc = G.indexer_scores(15, 64, 65536)
    lens = np.full(64, 65536)
    lens[::7] = np.random.default_rng(15).integers(0, 65536, len(lens[::7]))
    parts, nbytes = mlasd.topk_plan(64, 65536)
    if torch.cuda.get_device_properties(0).multi_processor_count >= 256:
        assert parts == 4
    mlasd.reserve(nbytes)
    _check(sc, lens, 512, "B=64 x 65536", parts=(None, 1, 2, 8))


@pytest.mark.parametrize("k", [1, 7, 100])
def test_long_rows_small_k(k):
    """Long rows with a small k: the sampled threshold keeps few candidates
    per part, and the joined list still holds the row's top k."""
    sc = G.indexer_scores(28, 4, 100000)
    _check(sc, [100000, 65536, 99999, 70001], k, f"long rows k={k}", parts=(None, 1, 4, 8))


def test_candidates_in_one_part():
    """Rows whose large scores all sit in their first eighth: with 8 parts
    one part's list overflows its share of the candidate list although the
    row's total fits, and the selection falls back to the whole row; with 3
    parts the same candidates fit.  Short rows in the batch are selected
    whole."""
    L = 65536
    sc = G.indexer_scores(24, 4, L)
    sc[:2, L // 8:] -= 100.0
    sc[2, : 7 * L // 8] -= 100.0
    _check(sc, [L, L - 5, L, 3000], 512, "candidates in one part", parts=(1, 3, 8))


def test_forced_parts_need_scratch():
    """A forced split on a stream without scratch is refused before anything
    is enqueued; the library's plan there runs one workgroup per row."""
    sc = torch.from_numpy(G.indexer_scores(25, 2, 65536)).cuda()
    lens = torch.tensor([65536, 40000], dtype=torch.int32, device="cuda")
    ref = O.topk_select(sc.cpu().numpy(), lens.cpu().numpy(), 512)
    stream = torch.cuda.Stream()
    out = torch.full((2, 512), -7, dtype=torch.int32, device="cuda")
    with pytest.raises(mlasd.MlasdError) as ei:
        mlasd.mla_topk_select(sc, lens, 512, out=out, stream=stream, parts=4)
    assert ei.value.status == -8
    stream.synchronize()
    assert bool((out == -7).all())
    got = mlasd.mla_topk_select(sc, lens, 512, stream=stream)
    stream.synchronize()
    assert np.array_equal(got.cpu().numpy(), ref)


def test_split_selection_in_a_graph():
    """The split selection (parts kernel, then the per-row kernel reading the
    stream's scratch) captured in a graph and replayed with eager work and
    new scores in between: every replay matches the oracle."""
    B, L = 16, 65536
    stream = torch.cuda.Stream()
    parts, nbytes = mlasd.topk_plan(B, L, 4)
    mlasd.reserve(nbytes, stream=stream)
    sc = torch.empty((B, L), dtype=torch.float32, device="cuda")
    lens_np = np.full(B, L)
    lens_np[3] = 33000
    lens_np[5] = 600
    lens = torch.from_numpy(lens_np.astype(np.int32)).cuda()
    idx = torch.empty((B, 512), dtype=torch.int32, device="cuda")
    sc.copy_(torch.from_numpy(G.indexer_scores(26, B, L)))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        mlasd.mla_topk_select(sc, lens, 512, out=idx, stream=stream, parts=parts)
    for rep in range(3):
        scores = G.indexer_scores(27 + rep, B, L)
        sc.copy_(torch.from_numpy(scores))
        idx.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(idx.cpu().numpy(), O.topk_select(scores, lens_np, 512)), f"replay {rep}"
        torch.ones(1 << 20, device="cuda").sum()   # eager work between replays


def test_full_length_ties():
    """Rows of 65,536 scores from five values: the k-th score is shared by
    thousands of positions, of which the lowest fill the list."""
    sc = G.indexer_scores(16, 8, 65536, "ties")
    _check(sc, [65536, 65535, 40000, 513, 65536, 30000, 9000, 70000], 512, "ties 65536")


def test_chained_before_the_decode_in_one_graph():
    """scores -> topk_idx -> decode captured in one HIP graph, replayed with
    eager work in between: every replay's out / lse meet the oracle bar for
    the oracle's selection of the same scores."""
    lens = [3000, 700, 9000, 0]
    need = sum((L + 255) // 256 for L in lens)
    w = G.build_workload(17, lens, 512, num_pages=need + 2, fill="all")
    d = to_device(w)
    scores = G.indexer_scores(18, len(lens), 9500)
    ref_idx = O.topk_select(scores, w.seq_lens, 512)
    ref_out, ref_lse = O.sparse_mla_decode(w.q_bits, w.kv_pages, w.page_table, ref_idx, w.seq_lens,
                                           w.softmax_scale)
    sc = torch.from_numpy(scores).cuda()
    idx = torch.empty((len(lens), 512), dtype=torch.int32, device="cuda")
    out = torch.empty((len(lens), 64, 448), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((len(lens), 64), dtype=torch.float32, device="cuda")
    stream = torch.cuda.Stream()
    reserve_for(len(lens), 512, stream=stream)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        mlasd.mla_topk_select(sc, d["seq_lens"], 512, out=idx, stream=stream)
        mlasd.mla_sparse_decode(d["q"], d["kv_pages"], d["page_table"], idx, d["seq_lens"], w.softmax_scale,
                                out=out, lse=lse, stream=stream)
    for rep in range(3):
        idx.fill_(-7)
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(idx.cpu().numpy(), ref_idx), f"replay {rep}: topk_idx differs"
        check_attention(out, lse, ref_out, ref_lse, label=f"chained replay {rep}")
        torch.ones(1 << 20, device="cuda").sum()   # eager work between replays


def test_unaligned_rows():
    """Rows that start 4 bytes past a 16-byte boundary (a column slice of a
    wider matrix): the scalar-load path."""
    sc = G.indexer_scores(19, 5, 20001)
    lens = [20000, 19999, 17000, 513, 3]
    print("topk: unaligned rows", flush=True)
    wide = torch.from_numpy(sc).cuda()
    view = wide[:, 1:]
    assert view.data_ptr() % 16 != 0
    out = mlasd.mla_topk_select(view, torch.tensor(lens, dtype=torch.int32, device="cuda"), 512)
    torch.cuda.synchronize()
    ref = O.topk_select(np.ascontiguousarray(sc[:, 1:]), lens, 512)
    assert np.array_equal(out.cpu().numpy(), ref)


def test_threshold_guess_misses():
    """Long rows where a guessed threshold from a spread-out sample leaves too
    few or too many candidates: a constant row, a row whose large scores sit
    only at every 64th position of its first 4,096, a row whose large scores
    avoid those positions, and a row of 40,000 equal maxima."""
    L = 65536
    sc = np.zeros((4, L), dtype=np.float32)
    sc[0] = 0.75
    sc[1, : 64 * 64 : 64] = 10.0
    sc[2] = -np.inf
    sc[2, 1::64] = np.arange(1024, dtype=np.float32)
    sc[3] = G.indexer_scores(20, 1, L)[0]
    sc[3, :40000] = 5.0
    _check(sc, [L, L, L, L], 512, "guess misses")


def test_rows_longer_than_a_batch_of_the_candidate_pass():
    """Rows of up to 131,072 scores (the longest sequences of the
    log-uniform workload): several load batches per row, and rows whose
    length is not a multiple of 4."""
    sc = G.indexer_scores(21, 6, 131072)
    _check(sc, [131072, 131071, 98305, 65537, 16385, 16383], 512, "131072")


def test_mid_length_rows_whose_guess_takes_everything():
    """Rows of 4,097 .. 16,384 scores take the sampled threshold; when the
    sample's threshold is -inf (rows of -inf or NaN) every position is a
    candidate and the whole row becomes the list."""
    L = 8000
    sc = np.zeros((4, L), dtype=np.float32)
    sc[0] = -np.inf
    sc[1] = np.nan
    sc[2] = -np.inf
    sc[2, 7000:7300] = 1.0
    sc[3] = G.indexer_scores(22, 1, L)[0]
    _check(sc, [L, L, L, 5000], 512, "mid-length guesses")


def test_threshold_at_zero_or_denormal_scores():
    """Long rows where the guessed threshold lands on a zero or denormal
    score, so candidates are tested by key instead of by float compare:
    mostly +-0 with a few positives, denormals of both signs, and a mix."""
    L = 20000
    rng = np.random.default_rng(23)
    sc = np.zeros((3, L), dtype=np.float32)
    sc[0] = np.where(rng.random(L) < 0.5, np.float32(0.0), np.float32(-0.0))
    sc[0, rng.choice(L, 100, replace=False)] = rng.random(100).astype(np.float32) + 1.0
    tiny = np.float32(1e-42)   # a denormal
    sc[1] = (rng.integers(-3, 4, L) * tiny).astype(np.float32)
    sc[2] = np.where(rng.random(L) < 0.3, (rng.integers(-2, 3, L) * tiny).astype(np.float32),
                     rng.standard_normal(L).astype(np.float32) - 4.0)
    assert np.any(np.abs(sc[1]) > 0) and np.all(np.abs(sc[1]) < 1e-37)
    _check(sc, [L, L, L], 512, "zero / denormal thresholds")
