"""Exact GPU checks of the decode and prefill kernels, the matrix-core ones in
particular, where the definition of attention gives the answer in closed form.

Attention weights every visible key by exp(scale * q.k) and returns the
weighted mean of their V rows ("vLLM 基本原理", section "Transformer 和
Attention").  With q = 0 every score is 0, every visible key weighs exactly 1,
the denominator is the number n of visible keys, and the output is the plain
mean of the visible V rows.  V is zero except for "needles": the row of each
tested position t_j holds a power of two c_j in a column of its own.  A kernel
that normalises the accumulated c_j by n must then write exactly
fp32(c_j) / fp32(n) -- before the bf16 rounding of the output, which is then
exact too -- in that column, and exactly 0 in every column whose needle it
must not see.  Needles sit at the first and last key of a 16-token block and
of a 64-key prefill tile, on both sides of every split-K partition or key-run
boundary, on a query's causal diagonal and one past it, and at the end of the
context.  A dropped needle gives 0, a doubled one 2 c_j / n, a key seen past
the diagonal a nonzero where 0 is due.

The fp32 split-K partials pin the denominators themselves: partition p with
n_p visible keys must hold fp32(c_j) / fp32(n_p) and a log-sum-exp of ln(n_p),
so one key dropped or counted twice anywhere moves them far past rounding --
the check the bf16 output tolerance cannot make at long contexts.

Also exact: a one-token context (and the first row of a chunk with no prefix)
returns its V row bit for bit; identical keys give the mean of V (fp32
partials at the fp32 tolerance); relabelling physical block ids, and replacing
shared prefix blocks by private copies, give bitwise-identical outputs and
partials ("vLLM 基本原理", section PagedAttention, items on non-contiguous
storage and memory sharing).

Decode cases cover both kernels: bf16 with head_dim 128 and at least 4 query
heads per kv head runs on the matrix cores, the rest on the vector ALUs.
"""
import numpy as np
import pytest

from workloads import config4, make_decode, make_prefill, permute_block_ids, unshare_blocks
from workloads.device import to_device, torch_to_storage
from workloads.generate import BF16_NAN, f32_to_bf16_bits

from pa_harness import as_f64, lib, say

pytestmark = pytest.mark.gpu
BS = 16

# (query heads, kv heads, head_dim, dtype): the first three run on the matrix cores
DECODE_SHAPES = [(32, 8, 128, "bf16"), (16, 1, 128, "bf16"), (8, 2, 128, "bf16"),
                 (40, 40, 128, "bf16"), (6, 2, 64, "bf16"), (4, 4, 128, "f32")]
DECODE_IDS = ["mfma-32x8", "mfma-16x1", "mfma-8x2", "valu-40x40", "valu-6x2-d64", "valu-f32"]


# --------------------------------------------------------------------------
# closed-form expectations
# --------------------------------------------------------------------------
def needle_value(j: int) -> float:
    return 2.0 ** ((j % 5) - 2)          # 0.25 .. 4: powers of two, exact in bf16


def needle_column(j: int, kvh: int, d: int) -> int:
    return (5 * j + 7 * kvh) % d         # distinct columns for distinct j (gcd(5, d) = 1)


def ratio(c: float, n) -> np.ndarray:
    """fp32(c) / fp32(n), the value a kernel normalising c by n produces."""
    return np.float32(c) / np.asarray(n, dtype=np.float32)


def rounded(x: np.ndarray, dtype: str) -> np.ndarray:
    """x (fp32) as the output dtype stores it (bf16: nearest even), in fp64."""
    x = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return x.astype(np.float64)
    bits = f32_to_bf16_bits(x).astype(np.uint32) << 16
    return bits.view(np.float32).astype(np.float64)


def valid_rows(w, pool):
    return ~np.isnan(pool) if w.dtype == "f32" else pool != BF16_NAN


def storage_scalar(x: float, dtype: str):
    return np.float32(x) if dtype == "f32" else f32_to_bf16_bits(np.array([x], np.float32))[0]


def place_needles(w, tables, lens, positions_of, d):
    """Zero V (keeping the NaN rows that must never be read) and put needle j
    of sequence s at position positions_of(s)[j], column needle_column(j, kvh),
    value needle_value(j).  Returns {s: [(t_j, c_j, column per kv head)]}."""
    keep = valid_rows(w, w.v_host)
    w.v_host[keep] = 0
    ht = w.host_tables(tables)
    placed = {}
    for s, L in enumerate(lens):
        pos = positions_of(s)
        assert len(pos) <= d, "more needles than columns"
        items = []
        for j, t in enumerate(pos):
            assert 0 <= t < L
            c = needle_value(j)
            row = ht[s, t // BS]
            cols = [needle_column(j, kh, d) for kh in range(w.num_kv_heads)]
            for kh in range(w.num_kv_heads):
                w.v_host[row, kh, t % BS, cols[kh]] = storage_scalar(c, w.dtype)
            items.append((t, c, cols))
        placed[s] = items
    return placed


def decode_positions(L: int, ps: int):
    base = [0, 1, 15, 16, 17, 31, 32, 63, 64, 255, 256, L - 17, L - 16, L - 15, L - 2, L - 1]
    if ps:
        for b in range(ps, L, ps):
            base += [b - 1, b, b + 1]
    return sorted({t for t in base if 0 <= t < L})


def read_partials(ws, S, hq, P, d):
    host = ws.cpu().numpy()
    n = S * hq * P
    o = host[:n * d * 4].view(np.float32).reshape(S, hq, P, d)
    lse = host[n * d * 4:n * (d + 1) * 4].view(np.float32).reshape(S, hq, P)
    return o, lse


def check_lse(got, n, what):
    want = np.log(np.asarray(n, dtype=np.float64))
    err = np.abs(got.astype(np.float64) - want)
    assert (err <= 1e-5).all(), f"{what}: lse off by {err.max():.2e} (n={n})"


# --------------------------------------------------------------------------
# decode
# --------------------------------------------------------------------------
def run_decode(w, ps, fill_ws=0xFF):
    import torch
    L = lib()
    dw = to_device(w)
    g = dw.decode
    ws = None
    if ps:
        nbytes = L.pa_decode_workspace_bytes(g.query.shape[0], w.num_heads, w.head_dim,
                                             g.max_context_len, ps)
        ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
        ws.fill_(fill_ws)
    L.pa_decode(g.out, g.query, dw.k_cache, dw.v_cache, g.block_tables, g.context_lens, w.scale,
                g.max_context_len, ps, ws)
    partials = None if ws is None else ws.clone()
    if ps:
        L.pa_decode_splitk_reduce(g.out, ws, g.context_lens, g.max_context_len, ps)
    torch.cuda.synchronize()
    return dw, partials


DECODE_LENS = np.array([1, 16, 17, 511, 512, 513, 1024, 1500, 2048, 2049, 5000], dtype=np.int32)


@pytest.mark.parametrize("ps", [0, 512, 2048])
@pytest.mark.parametrize("hq,hkv,d,dtype", DECODE_SHAPES, ids=DECODE_IDS)
def test_decode_needles(gpu, hq, hkv, d, dtype, ps):
    say(f"decode needles {hq}/{hkv} d={d} {dtype} ps={ps}")
    w = make_decode("needles", 301, dtype, DECODE_LENS, hq, hkv, d, 2048, with_scatter=False)
    w.decode.query[:] = 0
    lens = w.decode.context_lens
    placed = place_needles(w, w.decode.block_tables, lens,
                           lambda s: decode_positions(int(lens[s]), ps), d)
    dw, ws = run_decode(w, ps)
    got = as_f64(dw.decode.out)
    G = hq // hkv
    S = len(lens)
    P = -(-int(lens.max()) // ps) if ps else 1
    if ps:
        o_part, lse = read_partials(ws, S, hq, P, d)
    for s, L in enumerate(lens):
        L = int(L)
        nparts = -(-L // ps) if ps else 1
        for h in range(hq):
            kh = h // G
            want = np.zeros(d, np.float32)
            for t, c, cols in placed[s]:
                want[cols[kh]] = ratio(c, L)
            if nparts == 1:
                # one pass: exactly fp32(c) / fp32(L), then the output's rounding
                ok = got[s, h] == rounded(want, dtype)
                assert ok.all(), (s, h, np.nonzero(~ok)[0][:4], got[s, h][~ok][:4],
                                  rounded(want, dtype)[~ok][:4])
                continue
            # merged: within the output's own rounding of c / L; zeros exact
            exact = want.astype(np.float64)
            tol = (2.0 ** -8 if dtype == "bf16" else 2.0 ** -20) * np.abs(exact)
            assert (np.abs(got[s, h] - exact) <= tol).all(), (s, h)
            # partials: every partition's count and needles, exactly
            for p in range(nparts):
                n_p = min(ps, L - p * ps)
                pw = np.zeros(d, np.float32)
                for t, c, cols in placed[s]:
                    if p * ps <= t < (p + 1) * ps:
                        pw[cols[kh]] = ratio(c, n_p)
                ok = o_part[s, h, p] == pw
                assert ok.all(), ("partial", s, h, p, np.nonzero(~ok)[0][:4])
                check_lse(lse[s, h, p], n_p, f"seq {s} head {h} partition {p}")


@pytest.mark.parametrize("ps", [0, 512])
@pytest.mark.parametrize("hq,hkv,d,dtype", DECODE_SHAPES, ids=DECODE_IDS)
def test_decode_single_token_returns_v_bitwise(gpu, hq, hkv, d, dtype, ps):
    """Contexts of one token, in a batch with longer ones: out = V row 0, bit for bit."""
    import torch
    say(f"decode one-token contexts {hq}/{hkv} d={d} {dtype} ps={ps}")
    lens = np.array([1, 700, 1, 1, 1300, 1], dtype=np.int32)
    w = make_decode("one-token", 302, dtype, lens, hq, hkv, d, 512, with_scatter=False)
    dw, _ = run_decode(w, ps)
    G = hq // hkv
    iv = torch.int16 if dtype == "bf16" else torch.int32
    for s in np.nonzero(lens == 1)[0]:
        blk = int(w.decode.block_tables[s, 0])
        for h in range(hq):
            assert torch.equal(dw.decode.out[s, h].view(iv), dw.v_cache[blk, h // G, 0].view(iv))


@pytest.mark.parametrize("ps", [0, 512])
@pytest.mark.parametrize("hq,hkv,d,dtype", DECODE_SHAPES[:3] + DECODE_SHAPES[5:],
                         ids=DECODE_IDS[:3] + DECODE_IDS[5:])
def test_decode_identical_keys_give_mean_of_v(gpu, hq, hkv, d, dtype, ps):
    """Every key of a kv head equal: all weights are exactly 1, out = mean(V).
    Partials against the fp64 mean of their partition at the fp32 tolerance
    (a missed or doubled key is ~1/n_p off); merged output within the output's
    rounding."""
    say(f"decode identical keys {hq}/{hkv} d={d} {dtype} ps={ps}")
    w = make_decode("same-keys", 303, dtype, DECODE_LENS, hq, hkv, d, 2048, with_scatter=False)
    keep = valid_rows(w, w.k_host)
    for kh in range(hkv):
        k0 = w.k_host[0, kh, 0].copy()
        sl = w.k_host[:, kh]
        sl[keep[:, kh]] = np.broadcast_to(k0, sl.shape)[keep[:, kh]]
    dw, ws = run_decode(w, ps)
    got = as_f64(dw.decode.out)
    lens = w.decode.context_lens
    ht = w.host_tables(w.decode.block_tables)
    vv = (w.v_host.astype(np.float64) if dtype == "f32" else
          (w.v_host.astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    G = hq // hkv
    S = len(lens)
    P = -(-int(lens.max()) // ps) if ps else 1
    if ps:
        o_part, _ = read_partials(ws, S, hq, P, d)
    for s, L in enumerate(lens):
        L = int(L)
        rows = np.stack([vv[ht[s, t // BS], :, t % BS, :] for t in range(L)])   # [L, Hkv, D]
        mean = rows.mean(axis=0)
        want = mean[np.arange(hq) // G]
        tol = (2.0 ** -8 * np.abs(want) + 2e-7 if dtype == "bf16" else
               1e-5 + 1e-5 * np.abs(want))
        assert (np.abs(got[s] - want) <= tol).all(), (s, np.abs(got[s] - want).max())
        nparts = -(-L // ps) if ps else 1
        if nparts > 1:
            for p in range(nparts):
                pm = rows[p * ps:(p + 1) * ps].mean(axis=0)[np.arange(hq) // G]
                err = np.abs(o_part[s, :, p].astype(np.float64) - pm)
                assert (err <= 1e-5 + 1e-5 * np.abs(pm)).all(), (s, p, err.max())


@pytest.mark.parametrize("ps", [0, 512])
def test_gqa_decode_relabelled_blocks_bitwise(gpu, ps):
    """The matrix-core decode (32/8, bf16) under a random relabelling of the
    physical ids: outputs and split-K partials are the same bits."""
    import torch
    say(f"gqa decode relabelled ids ps={ps}")
    rng = np.random.default_rng(304)
    lens = rng.integers(600, 3000, size=12).astype(np.int32)
    w = make_decode("relabel-gqa", 304, "bf16", lens, 32, 8, 128, 4096, with_scatter=False)
    a, wa = run_decode(w, ps)
    b, wb = run_decode(permute_block_ids(w, 305), ps)
    assert torch.equal(a.decode.out.view(torch.int16), b.decode.out.view(torch.int16))
    if ps:
        assert torch.equal(wa, wb)


@pytest.mark.parametrize("ps", [0, 512])
def test_gqa_decode_shared_prefix_bitwise_identical_to_private_copies(gpu, ps):
    """Samples of one prompt naming the same prompt blocks give the same bits
    as the same samples reading private copies (matrix-core decode, 32/8)."""
    import torch
    say(f"gqa decode shared vs private prefix blocks ps={ps}")
    w = config4(num_prompts=6, samples=3, num_prefill=1, num_blocks=4096, heads=32, kv_heads=8)
    w.prefill = None
    a, wa = run_decode(w, ps)
    b, wb = run_decode(unshare_blocks(w), ps)
    assert torch.equal(a.decode.out.view(torch.int16), b.decode.out.view(torch.int16))
    if ps:
        assert torch.equal(wa, wb)


# --------------------------------------------------------------------------
# chunked prefill (matrix cores)
# --------------------------------------------------------------------------
PREFILL_SHAPES = [(8, 8, 128), (8, 2, 128), (32, 8, 128), (6, 3, 64)]
PREFIXES = [0, 0, 37, 64, 500, 1000, 2900]
CHUNKS = [1, 200, 130, 257, 128, 300, 512]


def prefill_positions(P: int, C: int, split: int, d: int):
    """Needle positions of a chunk of C queries over a prefix of P keys, at most
    d of them: the causal diagonal cases and the chunk's end first, then the
    block / tile boundaries near the start, then the key-run boundaries."""
    L = P + C
    first = [P - 1, P, P + 1, P + 15, P + 16, P + 31, P + 32, P + 63, P + 64, P + 127, P + 128,
             P + 129, P + 255, P + 256, L - 2, L - 1,
             0, 1, 15, 16, 63, 64, 65, 127, 128, 255, 256, 511, 512]
    runs = [t for b in range(split, L, split) for t in (b - 1, b)] if split else []
    out = []
    for t in first + runs:
        if 0 <= t < L and t not in out:
            out.append(t)
        if len(out) == d:
            break
    return sorted(out)


def run_prefill(w, split=0):
    import torch
    L = lib()
    dw = to_device(w)
    g = dw.prefill
    tq, hq, d = g.query.shape
    ws = None
    if split:
        maxc = int(w.prefill.context_lens.max())
        ws = torch.empty(max(L.pa_prefill_workspace_bytes(tq, hq, d, maxc, split), 16),
                         dtype=torch.uint8, device="cuda")
        ws.fill_(0xFF)
        L.pa_prefill_chunk_split(g.out, g.query, dw.k_cache, dw.v_cache, g.block_tables,
                                 g.query_start_loc, g.context_lens, w.scale, g.max_query_len,
                                 maxc, split, ws)
    else:
        L.pa_prefill_chunk(g.out, g.query, dw.k_cache, dw.v_cache, g.block_tables,
                           g.query_start_loc, g.context_lens, w.scale, g.max_query_len)
    torch.cuda.synchronize()
    return dw, ws


@pytest.mark.parametrize("split", [0, 64, 256])
@pytest.mark.parametrize("hq,hkv,d", PREFILL_SHAPES)
def test_prefill_needles(gpu, hq, hkv, d, split):
    say(f"prefill needles {hq}/{hkv} d={d} split={split}")
    w = make_prefill("pf-needles", 311, "bf16", PREFIXES, CHUNKS, hq, hkv, d, 1024)
    w.prefill.query[:] = 0
    g = w.prefill
    lens = g.context_lens
    qsl = g.query_start_loc
    placed = place_needles(
        w, g.block_tables, lens,
        lambda s: prefill_positions(PREFIXES[s], CHUNKS[s], split, d), d)
    dw, ws = run_prefill(w, split)
    got = as_f64(dw.prefill.out)
    heads = np.arange(hq) // (hq // hkv)
    if split:
        tq = int(qsl[-1])
        P = -(-int(lens.max()) // split)
        o_part, lse = read_partials(ws, tq, hq, P, d)
    checked_partials = 0
    for s in range(len(lens)):
        Pfx, C = PREFIXES[s], CHUNKS[s]
        q0 = int(qsl[s])
        t = np.array([x[0] for x in placed[s]])                 # [J] positions
        c = np.array([x[1] for x in placed[s]], np.float32)     # [J] values
        cols = np.array([x[2] for x in placed[s]])              # [J, Hkv] columns
        pos = Pfx + np.arange(C)                                # [C] query positions

        def expect(visible, n):
            """[C, Hq, D] fp32: c_j / n in needle j's column where visible."""
            vals = np.where(visible, c[None, :] / n.astype(np.float32)[:, None], 0)
            out = np.zeros((C, hkv, d), np.float32)
            for kh in range(hkv):
                out[:, kh, cols[:, kh]] = vals
            return out[:, heads]

        want = expect(t[None, :] <= pos[:, None], pos + 1)
        rows = got[q0:q0 + C]
        if not split:
            ok = rows == rounded(want, "bf16")
            assert ok.all(), (s, np.argwhere(~ok)[:4].tolist())
            continue
        exact = want.astype(np.float64)
        assert (np.abs(rows - exact) <= 2.0 ** -8 * np.abs(exact)).all(), s
        # partials: rows at or past position `split` sit in tiles that are split
        for p in range(int(pos.max()) // split + 1):
            sel = (pos >= split) & (p <= pos // split)
            if not sel.any():
                continue
            n_p = np.minimum(split, pos + 1 - p * split)
            vis = (t[None, :] >= p * split) & (t[None, :] < (p + 1) * split) & \
                  (t[None, :] <= pos[:, None])
            pw = expect(vis, np.maximum(n_p, 1))[sel]
            got_p = o_part[q0:q0 + C][sel][:, :, p]
            ok = got_p == pw
            assert ok.all(), ("partial", s, p, np.argwhere(~ok)[:4].tolist())
            lw = np.log(n_p[sel].astype(np.float64))[:, None]
            err = np.abs(lse[q0:q0 + C][sel][:, :, p].astype(np.float64) - lw)
            assert (err <= 1e-5).all(), ("lse", s, p, float(err.max()))
            checked_partials += int(sel.sum())
    if split:
        assert checked_partials > 0


@pytest.mark.parametrize("split", [0, 64, 256])
@pytest.mark.parametrize("hq,hkv,d", PREFILL_SHAPES)
def test_prefill_identical_keys_give_mean_of_v(gpu, hq, hkv, d, split):
    """Every key of a kv head equal: row i of a chunk gets the mean of V over
    positions 0 .. P + i (within bf16 rounding; split partials at the fp32
    tolerance against the mean over their run)."""
    say(f"prefill identical keys {hq}/{hkv} d={d} split={split}")
    w = make_prefill("pf-same-keys", 312, "bf16", PREFIXES, CHUNKS, hq, hkv, d, 1024)
    keep = valid_rows(w, w.k_host)
    for kh in range(hkv):
        k0 = w.k_host[0, kh, 0].copy()
        sl = w.k_host[:, kh]
        sl[keep[:, kh]] = np.broadcast_to(k0, sl.shape)[keep[:, kh]]
    dw, ws = run_prefill(w, split)
    got = as_f64(dw.prefill.out)
    g = w.prefill
    qsl = g.query_start_loc
    ht = w.host_tables(g.block_tables)
    vv = (w.v_host.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    G = hq // hkv
    heads = np.arange(hq) // G
    if split:
        tq = int(qsl[-1])
        P = -(-int(g.context_lens.max()) // split)
        o_part, _ = read_partials(ws, tq, hq, P, d)
    for s in range(len(PREFIXES)):
        Pfx, C = PREFIXES[s], CHUNKS[s]
        L = Pfx + C
        rows = np.stack([vv[ht[s, t // BS], :, t % BS, :] for t in range(L)])   # [L, Hkv, D]
        csum = np.cumsum(rows, axis=0)
        for i in range(C):
            pos = Pfx + i
            want = (csum[pos] / (pos + 1))[heads]
            r = int(qsl[s]) + i
            assert (np.abs(got[r] - want) <= 2.0 ** -8 * np.abs(want) + 2e-7).all(), (s, i)
            if split and pos >= split:
                for p in range(pos // split + 1):
                    pm = rows[p * split:min(pos + 1, (p + 1) * split)].mean(axis=0)[heads]
                    err = np.abs(o_part[r, :, p].astype(np.float64) - pm)
                    assert (err <= 1e-5 + 1e-5 * np.abs(pm)).all(), (s, i, p, err.max())


@pytest.mark.parametrize("split", [0, 256])
@pytest.mark.parametrize("hq,hkv,d", PREFILL_SHAPES)
def test_prefill_first_row_without_prefix_returns_v_bitwise(gpu, hq, hkv, d, split):
    """A chunk with no cached prefix: its first query sees key 0 alone, so its
    output is V row 0 bit for bit (here with random q, K, V)."""
    import torch
    say(f"prefill first row = V[0] {hq}/{hkv} d={d} split={split}")
    w = make_prefill("pf-first", 313, "bf16", [0, 0, 600, 0], [1, 300, 100, 700], hq, hkv, d, 512)
    dw, _ = run_prefill(w, split)
    G = hq // hkv
    qsl = w.prefill.query_start_loc
    for s in (0, 1, 3):
        blk = int(w.prefill.block_tables[s, 0])
        for h in range(hq):
            assert torch.equal(dw.prefill.out[int(qsl[s]), h].view(torch.int16),
                               dw.v_cache[blk, h // G, 0].view(torch.int16)), (s, h)


@pytest.mark.parametrize("split", [0, 256])
@pytest.mark.parametrize("hq,hkv,d", [(8, 8, 128), (32, 8, 128), (6, 3, 64)])
def test_prefill_relabelled_blocks_bitwise(gpu, hq, hkv, d, split):
    import torch
    say(f"prefill relabelled ids {hq}/{hkv} d={d} split={split}")
    w = make_prefill("pf-relabel", 314, "bf16", PREFIXES, CHUNKS, hq, hkv, d, 1024)
    a, _ = run_prefill(w, split)
    b, _ = run_prefill(permute_block_ids(w, 315), split)
    assert torch.equal(a.prefill.out.view(torch.int16), b.prefill.out.view(torch.int16))


@pytest.mark.parametrize("split", [0, 256])
@pytest.mark.parametrize("hq,hkv", [(8, 8), (32, 8)])
def test_prefill_shared_prefix_bitwise_identical_to_private_copies(gpu, hq, hkv, split):
    """Three sequences whose 20 leading blocks are one set of physical blocks
    (a cached prompt prefix, xdnf.cn article, section 六.3) give the same bits
    as the same sequences reading private copies of those blocks."""
    import torch
    say(f"prefill shared vs private prefix blocks {hq}/{hkv} split={split}")
    nsh = 20
    w = make_prefill("pf-share", 316, "bf16", [320, 400, 700], [50, 128, 300], hq, hkv, 128, 1024)
    g = w.prefill
    ht = w.host_tables(g.block_tables)
    # private copies: sequences 1 and 2 hold sequence 0's first nsh blocks' contents
    for s in (1, 2):
        for j in range(nsh):
            w.k_host[ht[s, j]] = w.k_host[ht[0, j]]
            w.v_host[ht[s, j]] = w.v_host[ht[0, j]]
    priv, _ = run_prefill(w, split)
    priv_out = priv.prefill.out.clone()
    del priv
    shared_tables = g.block_tables.copy()
    for s in (1, 2):
        shared_tables[s, :nsh] = g.block_tables[0, :nsh]
    w.prefill.block_tables = shared_tables
    shared, _ = run_prefill(w, split)
    assert torch.equal(priv_out.view(torch.int16), shared.prefill.out.view(torch.int16))
