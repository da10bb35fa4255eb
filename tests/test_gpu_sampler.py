"""pa_sample on the GPU against the reference sampler (oracle/sampler.py).

The kernel's draw is a deterministic function of the caller's uniform number
(the inverse of the distribution function), so it is compared draw by draw:
every GPU token must be one the oracle gives within 1e-6 of u or of top_p
(fixed-point weights and fp32 scaling can only move a decision that close to
a boundary), and nearly all must be exactly the oracle's token.  A uniform
grid of u on one row reproduces the oracle's probabilities token by token --
the statistical equivalence the pages ask for, at the resolution of the grid.
"""
import numpy as np
import pytest

from oracle import sampler
from pa_harness import say
from workloads import sampler_inputs
from workloads.generate import f32_to_bf16_bits

pytestmark = pytest.mark.gpu
DELTA = 1e-6


def run(gpu, logits, temperature, top_k, top_p, u, dtype="f32", stride=None):
    import torch
    s, v = logits.shape
    if dtype == "f32":
        lg = torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float32)).cuda()
    else:
        lg = torch.from_numpy(f32_to_bf16_bits(logits).view(np.int16)).cuda().view(torch.bfloat16)
    if stride is not None:
        wide = torch.zeros((s, stride), dtype=lg.dtype, device="cuda")
        wide[:, :v] = lg
        lg = wide[:, :v]
    tok = torch.full((s,), -7, dtype=torch.int32, device="cuda")
    f = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float32)).cuda()
    gpu.pa_sample(tok, lg, f(temperature), torch.from_numpy(np.asarray(top_k, dtype=np.int32)).cuda(),
                  f(top_p), f(u))
    torch.cuda.synchronize()
    return tok.cpu().numpy()


def storage_values(logits, dtype):
    if dtype == "f32":
        return logits.astype(np.float64)
    return (f32_to_bf16_bits(logits).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def admissible(x, t, k, p, u):
    out = set()
    for pp in (p - DELTA, p, min(1.0, p + DELTA)):
        for uu in (max(0.0, u - DELTA), u, min(u + DELTA, np.nextafter(1.0, 0.0))):
            out.add(sampler.sample(x, t, k, pp, uu))
    return out


@pytest.mark.parametrize("dtype,vocab,stride", [
    ("f32", 32000, None), ("bf16", 32000, None), ("f32", 1000, None), ("f32", 32768, None),
    ("bf16", 7, None),
    ("f32", 31999, None),      # the last 16-byte group of a row is partial
    ("bf16", 16387, None),     # 16 tokens a thread, a partial last group
    ("f32", 4093, 4093),       # rows 4 bytes apart from 16-byte alignment: no vector loads
    ("bf16", 30001, 30005)])
def test_draws_match_the_oracle(gpu, dtype, vocab, stride):
    say(f"sampler {dtype} vocab={vocab} stride={stride}")
    logits, t, k, p, u = sampler_inputs(48, vocab, 91)
    got = run(gpu, logits, t, k, p, u, dtype, stride=stride)
    x = storage_values(logits, dtype)
    exact = 0
    for r in range(len(got)):
        want = sampler.sample(x[r], float(t[r]), int(k[r]), float(p[r]), float(u[r]))
        exact += int(got[r] == want)
        assert got[r] in admissible(x[r], float(t[r]), int(k[r]), float(p[r]), float(u[r])), r
    assert exact >= len(got) - 1


def test_the_benchmark_batch(gpu):
    """The sampler bench's first logits batch: 256 rows x 32000, every row."""
    say("sampler: 256 x 32000 benchmark batch")
    logits, t, k, p, u = sampler_inputs(256, 32000, 453)
    got = run(gpu, logits, t, k, p, u)
    x = logits.astype(np.float64)
    exact = 0
    for r in range(len(got)):
        want = sampler.sample(x[r], float(t[r]), int(k[r]), float(p[r]), float(u[r]))
        if got[r] == want:
            exact += 1
        else:
            assert got[r] in admissible(x[r], float(t[r]), int(k[r]), float(p[r]), float(u[r])), r
    assert exact >= len(got) - 2


def test_uniform_grid_reproduces_the_distribution(gpu):
    """The pages' parameters (0.7, 50, 0.9) on one row, u on a grid of 8192 points."""
    say("sampler: uniform grid")
    n, vocab = 8192, 4000
    logits, _, _, _, _ = sampler_inputs(1, vocab, 92)
    rows = np.repeat(logits, n, axis=0)
    u = (np.arange(n) + 0.5) / n
    got = run(gpu, rows, np.full(n, 0.7), np.full(n, 50), np.full(n, 0.9), u)
    prob = sampler.probabilities(logits[0].astype(np.float64), 0.7, 50, 0.9)
    counts = np.bincount(got, minlength=vocab)
    assert counts[prob == 0].sum() == 0
    assert np.abs(counts - n * prob).max() <= 1.0 + 1e-6 * n


def test_edge_cases(gpu):
    say("sampler: edge cases")
    v = 64
    rng = np.random.default_rng(93)
    base = rng.normal(0, 2, v).astype(np.float32)
    rows, params, want = [], [], []

    def add(x, t, k, p, u, w):
        rows.append(np.asarray(x, dtype=np.float32))
        params.append((t, k, p, u))
        want.append(w)

    a = int(np.argmax(base))
    add(np.full(v, -np.inf), 1.0, 0, 1.0, 0.5, -1)                  # nothing finite
    nan_row = base.copy()
    nan_row[a] = np.nan
    add(nan_row, 1.0, 1, 1.0, 0.5, int(np.argsort(base)[-2]))       # NaN counts as -inf
    inf_row = base.copy()
    inf_row[[3, 40]] = np.inf
    add(inf_row, 1.0, 0, 1.0, 0.25, 3)                              # +inf tokens share all
    add(inf_row, 1.0, 0, 1.0, 0.75, 40)
    add(base, 0.7, 1, 1.0, 0.99, a)                                 # top_k 1
    add(base, 1.0, 0, 1e-6, 0.99, a)                                # a tiny top_p
    add(base, 1.0, v, 1.0, 0.0, sampler.sample(base, 1.0, v, 1.0, 0.0))
    add(base, 1.0, v + 9, 0.5, 0.3, sampler.sample(base, 1.0, v + 9, 0.5, 0.3))
    add(np.zeros(v), 1.0, 5, 1.0, 0.5, 32)                          # ties: all kept
    for bad in ((0.0, 0, 1.0, 0.5), (-1.0, 0, 1.0, 0.5), (1.0, 0, 0.0, 0.5),
                (1.0, 0, 1.5, 0.5), (1.0, 0, 1.0, 1.0), (1.0, 0, 1.0, -0.1),
                (np.nan, 0, 1.0, 0.5)):
        add(base, *bad, -1)                                         # parameters out of range
    x = np.stack(rows)
    t, k, p, u = (np.array(c) for c in zip(*params))
    got = run(gpu, x, t, k, p, u, stride=80)                        # rows 80 apart
    np.testing.assert_array_equal(got, want)
    one = run(gpu, np.array([[1.5]], dtype=np.float32), [1.0], [0], [1.0], [0.7])
    assert one.tolist() == [0]                                      # a vocabulary of one


def test_gathered_list_overflow_falls_back_to_the_row(gpu):
    """Rows whose radix buckets hold more tokens than one wave's share of the
    LDS list: the remaining digits go over the whole row again."""
    say("sampler: list overflow fallbacks")
    v = 32000
    rng = np.random.default_rng(94)
    rows, params = [], []
    flat = np.zeros(v, dtype=np.float32)
    for u in (0.0, 0.37, 0.999):
        rows.append(flat)
        params.append((1.0, 5, 1.0, u))           # top-k bucket = the whole row, all tied
        rows.append(flat)
        params.append((1.0, 0, 0.3, u))           # top-p over a flat row
        rows.append(flat)
        params.append((1.0, 7, 0.5, u))           # top-k then top-p, nothing gathered in full
    crowd = rng.normal(0, 1.5, v).astype(np.float32)
    crowd[:2048] += 8.0                            # the top 1500 all in the first wave's span
    for u in (0.11, 0.52, 0.93):
        rows.append(crowd)
        params.append((1.0, 1500, 0.8, u))
        rows.append(crowd)
        params.append((0.7, 1500, 1.0, u))
    bf = np.round(rng.normal(0, 1.5, v) * 4).astype(np.float32) / 4   # many exact ties
    for k, p in ((3000, 0.9), (0, 0.95), (40, 1.0)):
        rows.append(bf)
        params.append((1.0, k, p, 0.61))
    x = np.stack(rows)
    t, k, p, u = (np.array(c) for c in zip(*params))
    t, p, u = (c.astype(np.float32) for c in (t, p, u))   # what the GPU receives
    got = run(gpu, x, t, k, p, u)
    exact = 0
    for r in range(len(got)):
        want = sampler.sample(x[r].astype(np.float64), float(t[r]), int(k[r]), float(p[r]), float(u[r]))
        exact += int(got[r] == want)
        assert got[r] in admissible(x[r].astype(np.float64), float(t[r]), int(k[r]), float(p[r]),
                                    float(u[r])), (r, got[r], want)
    assert exact >= len(got) - 1


def test_rejects_vocabularies_beyond_the_register_row(gpu):
    import torch
    lg = torch.zeros((1, 40000), device="cuda")
    one = torch.ones(1, device="cuda")
    with pytest.raises(gpu.PagedAttentionError) as e:
        gpu.pa_sample(torch.zeros(1, dtype=torch.int32, device="cuda"), lg, one,
                      torch.zeros(1, dtype=torch.int32, device="cuda"), one, one * 0.5)
    assert e.value.status == -3
