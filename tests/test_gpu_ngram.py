"""GPU parity of prompt-lookup drafting (spec_ngram_draft) against the
oracle: integer work, so every output is compared bit for bit."""
import numpy as np
import pytest

import oracle
import speculative_decoding_verification_07_amd as sv
from speculative_decoding_verification_07_amd import inputs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _dev(a, offset=0):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32))
    if offset == 0:
        return t.cuda()
    flat = torch.empty(t.numel() + offset, dtype=torch.int32, device="cuda")
    flat[offset:] = t.reshape(-1).cuda()
    return flat[offset:].view(t.shape)


def run(ctx, lens, n_min, n_max, gamma, offset=0, workspace=None):
    c, ln = _dev(ctx, offset), _dev(lens)
    res = sv.ngram_draft(c, ln, n_min=n_min, n_max=n_max, gamma=gamma, workspace=workspace)
    torch.cuda.synchronize()
    return [r.cpu().numpy() for r in res]


def check(ctx, lens, n_min, n_max, gamma, **kw):
    print(f"ngram B={ctx.shape[0]} stride={ctx.shape[1]} n={n_min}..{n_max} gamma={gamma} "
          f"{kw}", flush=True)
    draft, length, n, pos = run(ctx, lens, n_min, n_max, gamma, **kw)
    want = oracle.ngram_draft(ctx, lens, n_min=n_min, n_max=n_max, gamma=gamma)
    bad = np.flatnonzero((length != want.length) | (n != want.n) | (pos != want.pos)
                         | (draft != want.draft).any(axis=1))
    assert bad.size == 0, (bad[:8], n[bad[:8]], want.n[bad[:8]], pos[bad[:8]], want.pos[bad[:8]])
    return want


@pytest.mark.parametrize("alphabet", [2, 7, 1000])
@pytest.mark.parametrize("n_min,n_max,gamma", [(1, 4, 4), (2, 5, 8), (1, 1, 1), (3, 16, 6),
                                               (1, 64, 0)])
def test_small_random(alphabet, n_min, n_max, gamma):
    """Rows spanning several 2048-token chunks with a ragged tail; lengths
    include 0, 1, 2, the stride, and two invalid ones."""
    rng = np.random.default_rng(alphabet * 100 + n_max)
    B, stride = 40, 5003
    ctx = rng.integers(0, alphabet, size=(B, stride), dtype=np.int32)
    lens = rng.integers(0, stride + 1, size=B).astype(np.int32)
    lens[:7] = [0, 1, 2, stride, -1, stride + 1, 2048]
    check(ctx, lens, n_min, n_max, gamma)


@pytest.mark.parametrize("rnd", [0, 1])
def test_copy_contexts_small(rnd):
    ctx, lens = inputs.make_contexts("ctx5k", rnd=rnd, pad="suffix")
    cc = inputs.CONTEXT_CONFIGS["ctx5k"]
    want = check(ctx, lens, cc.n_min, cc.n_max, cc.gamma)
    assert len(set(want.n.tolist())) >= 3      # a mix of match lengths


@pytest.mark.parametrize("name,rnd", [("ctx32k", 0), ("ctx32k", 1), ("ctx32k", 2),
                                      ("ctx128k", 0)])
def test_full_size(name, rnd):
    """The measured workloads (64 rows of 16k..32k and 64k..128k tokens),
    every row."""
    cc = inputs.CONTEXT_CONFIGS[name]
    ctx, lens = inputs.make_contexts(cc, rnd=rnd, pad="suffix")
    check(ctx, lens, cc.n_min, cc.n_max, cc.gamma)


def test_max_sizes():
    """Largest n_max and gamma; a constant row (every position matches, the
    match length caps at n_max) and a periodic one."""
    B, stride = 6, 9000
    rng = np.random.default_rng(5)
    ctx = rng.integers(0, 50, size=(B, stride), dtype=np.int32)
    ctx[0] = 7
    ctx[1] = np.arange(stride) % 3
    ctx[2, :100] = 7
    lens = np.array([stride, stride, 100, 8999, 4097, 2049], np.int32)
    check(ctx, lens, 1, sv.NGRAM_MAX_N, sv.NGRAM_MAX_GAMMA)
    check(ctx, lens, sv.NGRAM_MAX_N, sv.NGRAM_MAX_N, 3)


def test_one_chunk_and_tiny():
    rng = np.random.default_rng(9)
    for B, stride in ((1, 1), (3, 17), (5, 2048), (2, 2049)):
        ctx = rng.integers(0, 3, size=(B, stride), dtype=np.int32)
        lens = rng.integers(0, stride + 1, size=B).astype(np.int32)
        check(ctx, lens, 1, 3, 4)


def test_empty_stride():
    ctx = np.zeros((4, 0), np.int32)
    lens = np.array([0, 0, 1, -1], np.int32)
    draft, length, n, pos = run(ctx, lens, 1, 4, 3)
    assert (length == 0).all() and (draft == -1).all() and (pos == -1).all()
    assert n.tolist() == [-1, -1, -2, -2]


@pytest.mark.parametrize("offset", [1, 2, 3])
def test_unaligned(offset):
    """Base pointers that are only 4-byte aligned, and a stride that is not a
    multiple of 4: the element-wise load path."""
    ctx, lens = inputs.make_contexts("ctx5k", rnd=3, stride=4999)
    check(ctx, lens, 1, 4, 5, offset=offset)


def test_workspace_reuse():
    """One workspace through calls of different shapes; zero after each."""
    cc = inputs.CONTEXT_CONFIGS["ctx5k"]
    ws = sv.Workspace(sv.ngram_workspace_bytes(64))
    for rnd, B in ((4, 32), (5, 12), (6, 32)):
        ctx, lens = inputs.make_contexts(cc, rnd=rnd, B=B)
        check(ctx, lens, 1, 4, 4, workspace=ws)
        assert int(ws.tensor[ws.offset:ws.offset + ws.nbytes].count_nonzero()) == 0


def test_draft_feeds_point_verify():
    """A model-free round: the drafted tokens and lengths go straight into
    the verify's point mode, which then matches the oracle's verify."""
    from gpu_util import run as verify_run
    from oracle import parity

    cc = inputs.CONTEXT_CONFIGS["ctx5k"]
    ctx, lens = inputs.make_contexts(cc, rnd=7, B=16, V=5003, gamma=4)
    want = check(ctx, lens, 1, 4, 4)
    case = inputs.make_case(3, rnd=7, mode="point", B=16, V=5003)
    case.tokens[:] = np.maximum(want.draft, 0)
    case.gamma[:] = want.length
    got = verify_run(case, torch, probe=False)
    rep = parity.compare(case, *got[:3])
    assert rep.ok, rep.summary()


def test_random_shapes():
    """Forty seeded random configurations: batch, stride (0 included),
    alphabet, n range (both the register path and the LDS walk), gamma and
    base-pointer alignment, each against the oracle."""
    rng = np.random.default_rng(2024)
    for k in range(40):
        B = int(rng.integers(1, 70))
        stride = int(rng.choice([0, 1, 7, 2047, 2048, 2049, int(rng.integers(2, 9000))]))
        alphabet = int(rng.choice([1, 2, 3, 10, 1000]))
        n_min = int(rng.integers(1, 6))
        n_max = int(rng.integers(n_min, min(n_min + 12, sv.NGRAM_MAX_N) + 1))
        gamma = int(rng.integers(0, sv.NGRAM_MAX_GAMMA + 1))
        offset = int(rng.integers(0, 4))
        ctx = rng.integers(0, alphabet, size=(B, stride), dtype=np.int32)
        lens = rng.integers(-1, stride + 2, size=B).astype(np.int32)
        check(ctx, lens, n_min, n_max, gamma, offset=offset)
