"""Seeded synthetic inputs for the verify step (numpy only).

This module builds logits, draft tokens, uniforms, per-row draft lengths and
KV lengths.  It holds none of the verify step's arithmetic: it is the only
module that both the GPU path's tests/benchmark and the CPU oracle's tests
use.  The draft tokens are drawn the way a draft model would draw them (the
draft step, upstream of verification): by the Gumbel-max trick from
softmax(draft_logits / T) in sampling mode, by argmax in greedy mode and in
point mode.  Point mode stands for a drafter that proposes tokens outright (a
greedy draft model, an n-gram match): its draft logits only serve to pick
those tokens and are not passed to verification.

Workloads (vocabulary sizes of the models the pages discuss: GPT-2's 50257,
a LLaMA-2-class 32000, Llama 3's 128256, Qwen's 151936; draft lengths in the
pages' 4..8 range):

  cfg 1: B=1,   gamma=4, V=50257,  fp32, T=1.0  target N(0,3^2), draft = target + N(0,1^2)
  cfg 2: B=8,   gamma=8, V=32000,  bf16, T=0.8  target N(0,4^2), draft = target + N(0,0.5^2)
  cfg 3: B=64,  gamma=4, V=128256, bf16, T=1.0  target N(0,3^2) + 8.0 on one random token
                                                per (b, i); draft = target + N(0,1.5^2)
  cfg 4: B=256, gamma=8, V=151936, bf16, T=1.0  target N(0,3^2); draft = target + N(0,s_b^2),
                                                s_b ~ U(0.2, 3) per row
  cfg 5: B=32,  gamma_b ~ U{1..8}, V=128256, fp32, T=0.7  probability-space construction with
         sum_x min(p, q) = alpha_b exactly, alpha_b = (0.5, 0.8, 0.95)[b mod 3]

Seeds: numpy Philox with SeedSequence([cfg, round, k]); k = 0 target,
1 draft noise, 2 structure (spike index, sigma_b, overlap construction),
3 draft-token sampling, 4 verify uniforms, 5 KV lengths, 6 ragged gamma_b.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np

F32, BF16 = "f32", "bf16"


@dataclass(frozen=True)
class Config:
    cfg: int
    B: int
    G: int
    V: int
    dtype: str
    T: float
    target_sigma: float = 3.0
    draft_sigma: float = 1.0
    spike: float = 0.0
    per_row_sigma: tuple | None = None      # (lo, hi) of U(lo, hi) per row
    ragged: bool = False                    # gamma_b ~ U{1..G}
    overlap_alphas: tuple | None = None     # probability-space construction


CONFIGS = {
    1: Config(1, B=1, G=4, V=50257, dtype=F32, T=1.0, target_sigma=3.0, draft_sigma=1.0),
    2: Config(2, B=8, G=8, V=32000, dtype=BF16, T=0.8, target_sigma=4.0, draft_sigma=0.5),
    3: Config(3, B=64, G=4, V=128256, dtype=BF16, T=1.0, target_sigma=3.0, draft_sigma=1.5,
              spike=8.0),
    4: Config(4, B=256, G=8, V=151936, dtype=BF16, T=1.0, target_sigma=3.0,
              per_row_sigma=(0.2, 3.0)),
    5: Config(5, B=32, G=8, V=128256, dtype=F32, T=0.7, ragged=True,
              overlap_alphas=(0.5, 0.8, 0.95)),
}


@dataclass
class Case:
    config: Config
    mode: str                 # "sample", "greedy" or "point"
    target: np.ndarray        # [B, G+1, V] float32, or uint16 holding bf16 bits
    draft: np.ndarray         # [B, G, V] same dtype
    tokens: np.ndarray        # int32 [B, G]
    uniforms: np.ndarray      # float32 [B, G+1] in [0, 1)
    gamma: np.ndarray         # int32 [B]
    kv_len: np.ndarray        # int32 [B]
    extra: dict = field(default_factory=dict)

    @property
    def B(self):
        return self.target.shape[0]

    @property
    def G(self):
        return self.target.shape[1] - 1

    @property
    def V(self):
        return self.target.shape[2]

    @property
    def T(self):
        """The temperature as the C ABI carries it (fp32): both the GPU and
        the oracle are given this value."""
        return float(np.float32(self.config.T))


def rng(cfg: int, rnd: int, k: int) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(np.random.SeedSequence([cfg, rnd, k])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns the bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def widen(a: np.ndarray) -> np.ndarray:
    """Stored logits -> float32 (exact)."""
    return bf16_bits_to_f32(a) if a.dtype == np.uint16 else np.asarray(a, np.float32)


def store(x: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x) if dtype == BF16 else np.ascontiguousarray(x, np.float32)


def gumbel_max_tokens(stored_draft: np.ndarray, T: float, gen: np.random.Generator,
                      gamma: np.ndarray) -> np.ndarray:
    """Draft-side sampling x_{b,i} ~ softmax(d_{b,i}/T) by the Gumbel-max
    trick, in float64; -1 at positions i >= gamma_b (never read)."""
    B, G, V = stored_draft.shape
    out = np.full((B, G), -1, np.int32)
    for b in range(B):
        g = -np.log(-np.log(gen.random((G, V))))
        d = widen(stored_draft[b]).astype(np.float64) / T
        x = np.argmax(d + g, axis=1).astype(np.int32)
        k = int(gamma[b])
        out[b, :k] = x[:k]
    return out


def argmax_tokens(stored_draft: np.ndarray, gamma: np.ndarray) -> np.ndarray:
    """Greedy drafter: x_{b,i} = argmax_j d_{b,i,j} (lowest index on ties)."""
    B, G, V = stored_draft.shape
    out = np.full((B, G), -1, np.int32)
    for b in range(B):
        for i in range(int(gamma[b])):
            out[b, i] = int(np.argmax(widen(stored_draft[b, i])))
    return out


def _gaussian_logits(c: Config, rnd: int):
    B, G, V = c.B, c.G, c.V
    gt, gd, gs = rng(c.cfg, rnd, 0), rng(c.cfg, rnd, 1), rng(c.cfg, rnd, 2)
    target = np.empty((B, G + 1, V), np.uint16 if c.dtype == BF16 else np.float32)
    draft = np.empty((B, G, V), target.dtype)
    sig = None
    if c.per_row_sigma is not None:
        sig = gs.uniform(c.per_row_sigma[0], c.per_row_sigma[1], size=B)
    for b in range(B):
        t = gt.standard_normal((G + 1, V), dtype=np.float32) * np.float32(c.target_sigma)
        if c.spike:
            idx = gs.integers(0, V, size=G + 1)
            t[np.arange(G + 1), idx] += np.float32(c.spike)
        s = np.float32(sig[b] if sig is not None else c.draft_sigma)
        d = t[:G] + gd.standard_normal((G, V), dtype=np.float32) * s
        target[b] = store(t, c.dtype)
        draft[b] = store(d, c.dtype)
    extra = {"sigma_b": sig} if sig is not None else {}
    return target, draft, extra


def _softmax64(z: np.ndarray) -> np.ndarray:
    z = z - z.max()
    e = np.exp(z)
    return e / e.sum()


def _overlap_logits(c: Config, rnd: int):
    """Probability-space construction with sum_x min(p, q) = alpha exactly:
    s = softmax(N(0, 2^2)); a random permutation splits the vocabulary into
    halves A and B'; a and b' are softmax(N(0, 1)) restricted to A and B';
    p = alpha s + (1 - alpha) a, q = alpha s + (1 - alpha) b'.  Since a and b'
    have disjoint supports, min(p, q) = alpha s and the overlap is alpha.
    Stored logits are T ln p and T ln q."""
    B, G, V = c.B, c.G, c.V
    gs = rng(c.cfg, rnd, 2)
    alphas = np.array([c.overlap_alphas[b % len(c.overlap_alphas)] for b in range(B)])
    target = np.empty((B, G + 1, V), np.float32)
    draft = np.empty((B, G, V), np.float32)
    q_cdf = np.empty((B, G, V), np.float64)
    half = V // 2
    for b in range(B):
        al = alphas[b]
        for i in range(G + 1):
            s = _softmax64(gs.standard_normal(V) * 2.0)
            perm = gs.permutation(V)
            A, Bp = perm[:half], perm[half:]
            a = np.zeros(V)
            a[A] = _softmax64(gs.standard_normal(half))
            bq = np.zeros(V)
            bq[Bp] = _softmax64(gs.standard_normal(V - half))
            p = al * s + (1.0 - al) * a
            target[b, i] = (c.T * np.log(p)).astype(np.float32)
            if i < G:
                q = al * s + (1.0 - al) * bq
                draft[b, i] = (c.T * np.log(q)).astype(np.float32)
                q_cdf[b, i] = np.cumsum(q)
    return target, draft, {"alpha_b": alphas, "q_cdf": q_cdf}


def _gamma(c: Config, rnd: int) -> np.ndarray:
    if c.ragged:
        return rng(c.cfg, rnd, 6).integers(1, c.G + 1, size=c.B).astype(np.int32)
    return np.full(c.B, c.G, np.int32)


def make_case(cfg: int | Config, rnd: int = 0, mode: str = "sample", **overrides) -> Case:
    """Build one batch of a workload.  `overrides` (B, G, V, ...) shrink the
    shape while keeping the recipe, for tests the oracle must finish fast."""
    c = CONFIGS[cfg] if isinstance(cfg, int) else cfg
    if overrides:
        c = replace(c, **overrides)
    if c.overlap_alphas is not None:
        target, draft, extra = _overlap_logits(c, rnd)
    else:
        target, draft, extra = _gaussian_logits(c, rnd)
    gamma = _gamma(c, rnd)
    if mode in ("greedy", "point"):
        tokens = argmax_tokens(draft, gamma)
    elif "q_cdf" in extra:
        tokens = _tokens_from_cdf(extra["q_cdf"], gamma, rng(c.cfg, rnd, 3))
    else:
        tokens = gumbel_max_tokens(draft, c.T, rng(c.cfg, rnd, 3), gamma)
    uniforms = rng(c.cfg, rnd, 4).random((c.B, c.G + 1), dtype=np.float32)
    kv_len = rng(c.cfg, rnd, 5).integers(0, 8192, size=c.B).astype(np.int32)
    return Case(c, mode, target, draft, tokens, uniforms, gamma, kv_len, extra)


def _tokens_from_cdf(q_cdf: np.ndarray, gamma: np.ndarray, gen: np.random.Generator):
    B, G, V = q_cdf.shape
    out = np.full((B, G), -1, np.int32)
    uu = gen.random((B, G))
    for b in range(B):
        for i in range(int(gamma[b])):
            j = int(np.searchsorted(q_cdf[b, i], uu[b, i] * q_cdf[b, i, -1], side="right"))
            out[b, i] = min(j, V - 1)
    return out


def redraw_round(case: Case, rnd: int) -> Case:
    """Same logits, fresh gamma_b (ragged workloads), draft tokens and
    uniforms: one more verify round over fixed distributions."""
    c = case.config
    gamma = _gamma(c, rnd)
    if case.mode in ("greedy", "point"):
        tokens = argmax_tokens(case.draft, gamma)
    elif "q_cdf" in case.extra:
        tokens = _tokens_from_cdf(case.extra["q_cdf"], gamma, rng(c.cfg, rnd, 3))
    else:
        tokens = gumbel_max_tokens(case.draft, c.T, rng(c.cfg, rnd, 3), gamma)
    uniforms = rng(c.cfg, rnd, 4).random((c.B, c.G + 1), dtype=np.float32)
    return replace(case, tokens=tokens, uniforms=uniforms, gamma=gamma)


def fresh_uniforms(case: Case, rnd: int) -> Case:
    """Same logits and draft tokens, fresh verify uniforms."""
    c = case.config
    return replace(case, uniforms=rng(c.cfg, rnd, 4).random((c.B, c.G + 1), dtype=np.float32))


def stack_cases(cases: list) -> Case:
    """Concatenate batches of one workload (same gamma_max, V, dtype, T and
    mode) along the batch axis, so that many small calls can be checked in
    one multi-row comparison."""
    c0 = cases[0]
    cat = lambda k: np.concatenate([getattr(c, k) for c in cases], axis=0)
    cfg = replace(c0.config, B=sum(c.B for c in cases))
    return Case(cfg, c0.mode, cat("target"), cat("draft"), cat("tokens"), cat("uniforms"),
                cat("gamma"), cat("kv_len"), dict(c0.extra))


def algorithmic_bytes(case: Case) -> int:
    """Compulsory logit bytes one verify call must read: (2 g_b + 1) V e per
    row when sampling, (g_b + 1) V e when greedy or with point-mass drafts."""
    e = case.target.itemsize
    g = case.gamma.astype(np.int64)
    g = np.clip(g, 0, case.G)
    rows = (g + 1) if case.mode in ("greedy", "point") else (2 * g + 1)
    return int(rows.sum()) * case.V * e


# ------------------------------------------------------------ drafting contexts
@dataclass(frozen=True)
class ContextConfig:
    """Token contexts for prompt-lookup drafting: B rows of up to `stride`
    tokens, lengths ~ U{L_lo..stride}, vocabulary V."""
    name: str
    B: int
    stride: int
    L_lo: int
    V: int
    gamma: int
    n_min: int
    n_max: int
    copy_prob: float = 0.5       # share of segments copied from earlier in the row
    span: tuple = (4, 64)        # segment lengths ~ U{span}
    zipf_s: float = 1.1          # token frequencies ~ 1 / rank^s


CONTEXT_CONFIGS = {
    # the measured workload: the verify workload's batch and draft length,
    # long copy-heavy contexts (edit / summarisation / retrieval outputs)
    "ctx32k": ContextConfig("ctx32k", B=64, stride=32768, L_lo=16384, V=128256, gamma=4,
                            n_min=1, n_max=4),
    # long contexts (retrieval-sized inputs): where the bytes, not the
    # launch, set the time
    "ctx128k": ContextConfig("ctx128k", B=64, stride=131072, L_lo=65536, V=128256, gamma=4,
                             n_min=1, n_max=4),
    # small: a few chunks per row, for element-by-element parity
    "ctx5k": ContextConfig("ctx5k", B=32, stride=5000, L_lo=0, V=1000, gamma=6, n_min=1,
                           n_max=5),
}


def make_contexts(cc: ContextConfig | str, rnd: int = 0, pad: str = "random", **overrides):
    """Seeded token contexts (numpy Philox, SeedSequence([1000, round, 8])).

    Each row is built segment by segment: with probability copy_prob a
    segment repeats a span of the row's earlier tokens (the copying that
    makes prompt lookup pay off), otherwise it draws fresh tokens with
    Zipf(zipf_s) frequencies over a fixed random ranking of the vocabulary.
    Tokens after a row's length are filler: random tokens (pad="random") or
    repeats of the row's last tokens (pad="suffix", which would produce
    matches if anything past the length were read).
    Returns (context int32 [B, stride], lengths int32 [B])."""
    if isinstance(cc, str):
        cc = CONTEXT_CONFIGS[cc]
    if overrides:
        cc = replace(cc, **overrides)
    g = np.random.Generator(np.random.Philox(np.random.SeedSequence([1000, rnd, 8])))
    ranks = np.arange(1, cc.V + 1, dtype=np.float64)
    cdf = np.cumsum(ranks ** -cc.zipf_s)
    cdf /= cdf[-1]
    perm = g.permutation(cc.V).astype(np.int32)
    lens = g.integers(cc.L_lo, cc.stride + 1, size=cc.B).astype(np.int32)
    ctx = np.empty((cc.B, cc.stride), np.int32)
    lo, hi = cc.span
    for b in range(cc.B):
        row = ctx[b]
        L = int(lens[b])
        t = 0
        while t < L:
            n = min(int(g.integers(lo, hi + 1)), L - t)
            if t > 0 and g.random() < cc.copy_prob:
                s = int(g.integers(0, t))
                for i in range(n):          # may overlap what it writes
                    row[t + i] = row[s + i]
            else:
                u = g.random(n)
                row[t:t + n] = perm[np.minimum(np.searchsorted(cdf, u), cc.V - 1)]
            t += n
        rest = cc.stride - L
        if rest > 0:
            if pad == "suffix" and L > 0:
                tail = row[max(0, L - 8):L]
                row[L:] = np.resize(tail, rest)
            else:
                row[L:] = g.integers(0, cc.V, size=rest)
    return ctx, lens


def context_bytes(lens: np.ndarray, gamma: int) -> int:
    """Compulsory bytes of one drafting call: every token that can end an
    occurrence (L - 1 per row, 4 bytes each), the length, and the outputs
    (gamma + 3 int32 per row: draft, length, n, position)."""
    L = np.clip(lens.astype(np.int64), 0, None)
    return int((np.maximum(L - 1, 0) * 4).sum()) + len(L) * 4 * (1 + gamma + 3)
