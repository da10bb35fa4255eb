"""pa_decode_shared_prefix / pa_decode_fp8_shared_prefix on the GPU.

Sequences that share leading blocks (samples of one prompt, "vLLM 基本原理",
section 内存共享) have their common split-K partitions streamed once for the
whole group.  Each partition is still folded in the same order whichever pass
reads it, so the output must equal pa_decode's bit for bit on the same inputs;
it is also held to the oracle (bf16 tolerance, and the tight fp32 one on an
fp32 twin).  The workspace is filled with NaN before every run, so a partial
that the grouped pass fails to write cannot hide behind one a previous run
left.  Group layouts cover windows smaller than a group, groups of one,
malformed leader entries (which must degrade to the plain computation), a
member whose table breaks the grouping (NaN for that member only), shared
prefixes that end inside a partition or a block, members shorter than the
prefix, grouped-query heads, and FP8 caches.
"""
import numpy as np
import pytest

from oracle import kv_fp8
from pa_harness import as_f64, assert_close, lib, oracle_decode, say, to_device
from workloads import config4, fp8_pools
from workloads.device import host_to_torch, upload_fp8_pools
from workloads.generate import f32_to_bf16_bits

pytestmark = pytest.mark.gpu
K_SCALE, V_SCALE = 0.07, 0.11


def mixed_decoders(**kw):
    args = dict(num_prompts=8, samples=3, num_prefill=1, num_blocks=4096)
    args.update(kw)
    w = config4(**args)
    w.prefill = None
    return w


def decode_pair(dw, ps, prefix_group, max_group, shared=None, pools=None):
    """(pa_decode output, pa_decode_shared_prefix output) on the same inputs,
    each followed by the split-K merge; pools = FP8 (k, v) code pools."""
    import torch
    L = lib()
    g, w = dw.decode, dw.w
    shared = g.shared_prefix_blocks if shared is None else shared
    nbytes = L.pa_decode_workspace_bytes(g.query.shape[0], w.num_heads, w.head_dim,
                                         g.max_context_len, ps)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
    outs = []
    for grouped in (False, True):
        ws.fill_(0xFF)                      # NaN in every partial slot
        g.out.view(torch.int16).fill_(0x7FC0)
        common = (g.block_tables, g.context_lens)
        if pools is None:
            if grouped:
                L.pa_decode_shared_prefix(g.out, g.query, dw.k_cache, dw.v_cache, *common,
                                          w.scale, g.max_context_len, ps, ws, shared,
                                          prefix_group, max_group)
            else:
                L.pa_decode(g.out, g.query, dw.k_cache, dw.v_cache, *common, w.scale,
                            g.max_context_len, ps, ws, shared_prefix_blocks=shared)
        else:
            kc, vc = pools
            if grouped:
                L.pa_decode_fp8_shared_prefix(g.out, g.query, kc, vc, *common, float(w.scale),
                                              K_SCALE, V_SCALE, g.max_context_len, ps, ws,
                                              shared, prefix_group, max_group)
            else:
                L.pa_decode_fp8(g.out, g.query, kc, vc, *common, float(w.scale), K_SCALE,
                                V_SCALE, g.max_context_len, ps, ws, shared_prefix_blocks=shared)
        L.pa_decode_splitk_reduce(g.out, ws, g.context_lens, g.max_context_len, ps)
        torch.cuda.synchronize()
        outs.append(g.out.clone())
    return outs[0], outs[1]


def same_bits(a, b):
    import torch
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


def groups_of(n, size):
    return (np.arange(n) // size * size).astype(np.int32)


def as_dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


@pytest.mark.parametrize("ps", [256, 512, 2048])   # 2048: the launch bench.py times
def test_grouped_decode_bitwise_and_oracle(gpu, ps):
    say(f"shared-prefix decode: 8 prompts x 3 samples, ps={ps}")
    w = mixed_decoders(partition_size=ps)
    dw = to_device(w)
    plain, grouped = decode_pair(dw, ps, dw.decode.prefix_group, 3)
    assert same_bits(plain, grouped)
    assert_close(as_f64(grouped), oracle_decode(w, scattered=False), "bf16",
                 f"shared-prefix decode ps={ps}")


@pytest.mark.slow
@pytest.mark.parametrize("ps", [512, 2048])
def test_full_size_mixed_decoders(gpu, ps):
    """The mixed workload's 192 decoders (64 prompts x 3 samples sharing 2048
    tokens) in the launch bench.py times; oracle on every fourth sequence."""
    say(f"shared-prefix decode: full mixed workload, ps={ps}")
    w = config4(partition_size=ps)
    dw = to_device(w)
    plain, grouped = decode_pair(dw, ps, dw.decode.prefix_group, 3)
    assert same_bits(plain, grouped)
    pick = np.arange(0, w.decode.num_seqs, 4)
    say("shared-prefix decode: oracle")
    assert_close(as_f64(grouped)[pick], oracle_decode(w, seqs=pick, scattered=False), "bf16",
                 f"full mixed decoders ps={ps}")


def test_fp32_twin_tight(gpu):
    """fp32 K/V and the 1e-5 tolerance: one dropped or doubled key is ~100x over it."""
    say("shared-prefix decode: fp32 twin")
    w = mixed_decoders(dtype="f32", num_prompts=6, partition_size=512)
    dw = to_device(w)
    plain, grouped = decode_pair(dw, 512, dw.decode.prefix_group, 3)
    assert same_bits(plain, grouped)
    assert_close(as_f64(grouped), oracle_decode(w, scattered=False), "f32", "fp32 twin")


@pytest.mark.parametrize("layout", ["windows", "pairs", "singletons", "leader_after",
                                    "negative", "not_self_led", "random"])
def test_group_layouts_match_plain_decode(gpu, layout):
    """Groups of 7 (windows of 4 + 3), windows of 2, and entries that describe
    no valid group: every layout gives pa_decode's bits."""
    say(f"shared-prefix decode: group layout {layout}")
    w = mixed_decoders(num_prompts=4, samples=7, partition_size=512)
    dw = to_device(w)
    n = w.decode.num_seqs
    pg, max_group = groups_of(n, 7), 7
    if layout == "pairs":
        max_group = 2
    elif layout == "singletons":
        pg, max_group = np.arange(n, dtype=np.int32), 1
    elif layout == "leader_after":
        pg = pg.copy()
        pg[3] = 9
    elif layout == "negative":
        pg = pg.copy()
        pg[8] = -4
    elif layout == "not_self_led":
        pg = pg.copy()
        pg[7] = 1                    # 7 leads 8..13, but names 1 (which leads nobody)
    elif layout == "random":
        # each sequence names its true leader or itself: irregular windows
        pick = np.random.default_rng(5).integers(0, 2, n).astype(bool)
        pg = np.where(pick, pg, np.arange(n)).astype(np.int32)
    plain, grouped = decode_pair(dw, 512, as_dev(pg), max_group)
    assert same_bits(plain, grouped)
    if layout == "windows":
        assert_close(as_f64(grouped), oracle_decode(w, scattered=False), "bf16", "groups of 7")


def test_member_with_other_blocks_gets_nan(gpu):
    """A member whose table names other blocks inside the declared prefix
    breaks the contract: NaN for it, every other sequence untouched."""
    import torch
    say("shared-prefix decode: member table mismatch")
    w = mixed_decoders(partition_size=512)
    dw = to_device(w)
    g = dw.decode
    bad = 4                                        # second sample of prompt 1
    bt = g.block_tables.clone()
    bt[bad, 5] = g.block_tables[0, 5]              # a valid block of another prompt
    g.block_tables = bt
    plain, grouped = decode_pair(dw, 512, g.prefix_group, 3)
    others = [s for s in range(w.decode.num_seqs) if s != bad]
    assert same_bits(plain[others], grouped[others])
    assert torch.isnan(grouped[bad].float()).all()


def test_prefix_ends_inside_partition_and_short_members(gpu):
    """A 40-block shared prefix with 512-token partitions (one grouped
    partition, the rest of the prefix in the regular pass), members whose
    context ends inside the prefix or exactly at it, and an empty one."""
    import torch
    say("shared-prefix decode: ragged prefixes and members")
    w = mixed_decoders(shared_prefix=640, max_private=300, partition_size=512)
    lens = w.decode.context_lens.copy()
    lens[1] = 600          # ends inside the prefix, inside a block
    lens[2] = 640          # exactly the prefix
    lens[4] = 16 * 33      # ends inside the grouped partition's successor
    lens[7] = 7            # a single partial block
    lens[8] = 0            # empty: zeros
    w.decode.context_lens = lens
    dw = to_device(w)
    plain, grouped = decode_pair(dw, 512, dw.decode.prefix_group, 3)
    assert same_bits(plain, grouped)
    keep = [s for s in range(w.decode.num_seqs) if s != 8]
    assert_close(as_f64(grouped)[keep], oracle_decode(w, seqs=keep, scattered=False), "bf16",
                 "ragged prefixes")
    assert (grouped[8].float() == 0).all()


def gqa_decoders(hq, hkv, dtype="bf16", **kw):
    """The mixed workload's decoders with hq query heads over hkv kv heads."""
    w = mixed_decoders(heads=hkv, dtype=dtype, **kw)
    rng = np.random.default_rng(99)
    q = rng.standard_normal((w.decode.num_seqs, hq, w.head_dim)).astype(np.float32)
    w.decode.query = q if dtype == "f32" else f32_to_bf16_bits(q)
    w.num_heads = hq
    return w


@pytest.mark.parametrize("hq,hkv,groups", [(16, 8, 3), (32, 8, 3), (32, 4, 3), (32, 4, 7)])
def test_grouped_query_heads(gpu, hq, hkv, groups):
    """Grouped-query heads: two per kv head on the vector ALUs (windows of two
    sharers in four slots); four or eight on the matrix cores, whose 16 query
    columns take windows of four or two sharers."""
    say(f"shared-prefix decode: {hq} query heads over {hkv} kv heads, groups of {groups}")
    w = gqa_decoders(hq, hkv, samples=groups, num_prompts=24 // groups, partition_size=512)
    dw = to_device(w)
    plain, grouped = decode_pair(dw, 512, dw.decode.prefix_group, groups)
    assert same_bits(plain, grouped)
    assert_close(as_f64(grouped), oracle_decode(w, scattered=False), "bf16",
                 f"{hq}/{hkv} groups of {groups}")


def test_grouped_query_heads_member_with_other_blocks(gpu):
    """On the matrix cores too, a member that breaks the grouping gets NaN and
    nobody else changes."""
    import torch
    w = gqa_decoders(32, 8, partition_size=512)
    dw = to_device(w)
    g = dw.decode
    bt = g.block_tables.clone()
    bt[5, 3] = g.block_tables[0, 3]
    g.block_tables = bt
    plain, grouped = decode_pair(dw, 512, g.prefix_group, 3)
    others = [s for s in range(w.decode.num_seqs) if s != 5]
    assert same_bits(plain[others], grouped[others])
    assert torch.isnan(grouped[5].float()).all()


@pytest.mark.parametrize("hq,hkv", [(32, 8), (32, 4)])
def test_fp8_grouped_query_heads(gpu, hq, hkv):
    say(f"shared-prefix decode over an FP8 cache, {hq}/{hkv} heads")
    w = gqa_decoders(hq, hkv, partition_size=512)
    kq, vq = fp8_pools(w, 93)
    dw = to_device(w, pools=False)
    pools = upload_fp8_pools(w, kq, vq)
    plain, grouped = decode_pair(dw, 512, dw.decode.prefix_group, 3, pools=pools)
    assert same_bits(plain, grouped)
    d = w.decode
    want = kv_fp8.decode(d.query, kq, vq, w.host_tables(d.block_tables), d.context_lens, w.scale,
                         K_SCALE, V_SCALE, "bf16")
    assert_close(as_f64(grouped), want, "bf16", f"fp8 grouped decode {hq}/{hkv}")


@pytest.mark.parametrize("qdtype", ["bf16", "f32"])
def test_fp8_grouped_decode(gpu, qdtype):
    say(f"shared-prefix decode over an FP8 cache, {qdtype} query")
    w = mixed_decoders(dtype=qdtype, partition_size=512)
    kq, vq = fp8_pools(w, 91)
    dw = to_device(w, pools=False)
    pools = upload_fp8_pools(w, kq, vq)
    plain, grouped = decode_pair(dw, 512, dw.decode.prefix_group, 3, pools=pools)
    assert same_bits(plain, grouped)
    d = w.decode
    want = kv_fp8.decode(d.query, kq, vq, w.host_tables(d.block_tables), d.context_lens, w.scale,
                         K_SCALE, V_SCALE, qdtype)
    assert_close(as_f64(grouped), want, qdtype, f"fp8 grouped decode {qdtype}")


def test_rejects_what_it_cannot_run(gpu):
    import torch
    say("shared-prefix decode: argument checks")
    w = mixed_decoders(partition_size=512)
    dw = to_device(w)
    g = dw.decode
    L = lib()
    ws = torch.empty(1 << 24, dtype=torch.uint8, device="cuda")
    with pytest.raises(L.ShapeError):        # the grouped pass needs split-K
        L.pa_decode_shared_prefix(g.out, g.query, dw.k_cache, dw.v_cache, g.block_tables,
                                  g.context_lens, w.scale, g.max_context_len, 0, None,
                                  g.shared_prefix_blocks, g.prefix_group, 3)
    with pytest.raises(L.PagedAttentionError):   # shared counts are required
        L.pa_decode_shared_prefix(g.out, g.query, dw.k_cache, dw.v_cache, g.block_tables,
                                  g.context_lens, w.scale, g.max_context_len, 512, ws, None,
                                  g.prefix_group, 3)
