"""GPU parity of the block data movement: pa_copy_blocks and pa_swap_blocks
bit for bit against the oracle's block copies, and whole serving steps driven
by the native block manager (prompts, forked samples, shared prefixes,
copy-on-write, swap out and in, frees) with every pool compared bit for bit
and every decode within the bf16 / fp32 tolerance of the oracle run on the
oracle manager's identical tables.
"""
import numpy as np
import pytest

import oracle
import oracle.block_manager as ref
from pa_harness import assert_close, as_f64, say, torch_to_storage
from workloads.device import host_to_torch
from workloads.generate import f32_to_bf16_bits

pytestmark = pytest.mark.gpu
BS = 16


def torch_dtype(dtype):
    import torch
    return torch.float32 if dtype == "f32" else torch.bfloat16


def bits(a):
    """Storage array -> unsigned bit patterns (NaN payloads compare exactly)."""
    a = np.ascontiguousarray(a)
    return a.view(np.uint32) if a.dtype == np.float32 else a.view(np.uint16)


def random_storage(rng, shape, dtype):
    if dtype == "f32":
        return rng.integers(0, 2**32, size=shape, dtype=np.uint32).view(np.float32)
    return rng.integers(0, 2**16, size=shape, dtype=np.uint16)


def normal_storage(rng, shape, dtype):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return x if dtype == "f32" else f32_to_bf16_bits(x)


def independent_pairs(rng, nb, n):
    """n pairs with distinct destinations, none of them a source."""
    ids = rng.permutation(nb)
    dst = ids[:n]
    src = rng.choice(ids[n:], size=n)
    return np.stack([src, dst], axis=1).astype(np.int32)


@pytest.mark.parametrize("dtype,hkv,d,nb", [("f32", 2, 64, 40), ("bf16", 8, 128, 96),
                                            ("bf16", 40, 128, 64)])
def test_copy_blocks_bit_exact(gpu, dtype, hkv, d, nb):
    import torch
    say(f"copy_blocks {dtype} hkv={hkv} d={d} nb={nb}")
    rng = np.random.default_rng(7)
    shape = (nb, hkv, BS, d)
    k0, v0 = random_storage(rng, shape, dtype), random_storage(rng, shape, dtype)
    pairs = independent_pairs(rng, nb - 4, 20)
    # skipped pairs: an id out of range on either side, and a block onto itself
    skipped = np.array([[-1, nb - 1], [nb - 2, nb], [nb - 3, nb - 3], [2**31 - 1, nb - 4]],
                       dtype=np.int32)
    mapping = np.concatenate([pairs[:10], skipped, pairs[10:]])
    kc, vc = host_to_torch(k0, dtype, "cuda"), host_to_torch(v0, dtype, "cuda")
    gpu.pa_copy_blocks(kc, vc, torch.from_numpy(mapping).cuda())
    torch.cuda.synchronize()
    want_k, want_v = oracle.copy_blocks(k0, pairs), oracle.copy_blocks(v0, pairs)
    assert np.array_equal(bits(torch_to_storage(kc, dtype)), bits(want_k))
    assert np.array_equal(bits(torch_to_storage(vc, dtype)), bits(want_v))


def test_copy_blocks_empty_call_changes_nothing(gpu):
    import torch
    kc = torch.zeros((4, 2, BS, 64), device="cuda")
    vc = torch.zeros_like(kc)
    gpu.pa_copy_blocks(kc, vc, torch.zeros((0, 2), dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert not kc.any() and not vc.any()


def test_copy_blocks_13b_pool_1024_pairs(gpu):
    """The launch bench.py times: Llama-2-13B pools (65536 blocks x 40 heads x 16 x 128
    bf16, 10 GiB each), 1024 pairs; every destination and a sample of untouched blocks
    checked bit for bit."""
    import torch
    say("copy_blocks 13B pool, 1024 pairs")
    nb, hkv, d = 65536, 40, 128
    g = torch.Generator(device="cuda").manual_seed(11)
    kc = torch.randint(-2**15, 2**15, (nb, hkv, BS, d), dtype=torch.int16, device="cuda",
                       generator=g)
    vc = torch.randint(-2**15, 2**15, (nb, hkv, BS, d), dtype=torch.int16, device="cuda",
                       generator=g)
    rng = np.random.default_rng(12)
    pairs = independent_pairs(rng, nb, 1024)
    src = torch.from_numpy(pairs[:, 0].astype(np.int64)).cuda()
    dst = torch.from_numpy(pairs[:, 1].astype(np.int64)).cuda()
    others = np.setdiff1d(rng.choice(nb, 256, replace=False), pairs[:, 1])
    oth = torch.from_numpy(others.astype(np.int64)).cuda()
    want_k, want_v = kc[src].cpu().numpy(), vc[src].cpu().numpy()
    keep_k, keep_v = kc[oth].cpu().numpy(), vc[oth].cpu().numpy()
    gpu.pa_copy_blocks(kc.view(torch.bfloat16), vc.view(torch.bfloat16),
                       torch.from_numpy(pairs).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(kc[dst].cpu().numpy(), want_k)
    assert np.array_equal(vc[dst].cpu().numpy(), want_v)
    assert np.array_equal(kc[oth].cpu().numpy(), keep_k)
    assert np.array_equal(vc[oth].cpu().numpy(), keep_v)


def host_pool(arr, dtype, pinned):
    """A host tensor holding a copy of arr: pinned (kernel path) or pageable
    (runtime-copy path)."""
    t = host_to_torch(arr.copy(), dtype, "cpu")
    return t.pin_memory() if pinned else t


@pytest.mark.parametrize("dtype,hkv,d,pinned", [("bf16", 8, 128, True), ("f32", 2, 64, True),
                                                ("bf16", 8, 128, False)])
def test_swap_blocks_out_and_back(gpu, dtype, hkv, d, pinned):
    import torch
    say(f"swap_blocks {dtype} hkv={hkv} d={d} pinned={pinned}")
    rng = np.random.default_rng(5)
    nb, nh = 128, 48
    shape, hshape = (nb, hkv, BS, d), (nh, hkv, BS, d)
    k0, v0 = random_storage(rng, shape, dtype), random_storage(rng, shape, dtype)
    hk0, hv0 = random_storage(rng, hshape, dtype), random_storage(rng, hshape, dtype)
    kc, vc = host_to_torch(k0, dtype, "cuda"), host_to_torch(v0, dtype, "cuda")
    hk, hv = host_pool(hk0, dtype, pinned), host_pool(hv0, dtype, pinned)
    # runs that merge into one copy, single blocks, a run broken by a jump
    out_pairs = np.array([[5, 0], [6, 1], [7, 2], [40, 10], [3, 11], [90, 30], [91, 31],
                          [92, 33], [127, 47]], dtype=np.int32)
    gpu.pa_swap_blocks(kc, vc, hk, hv, out_pairs)
    torch.cuda.synchronize()
    want_hk, want_hv = oracle.swap_blocks(k0, hk0, out_pairs), oracle.swap_blocks(v0, hv0, out_pairs)
    assert np.array_equal(bits(torch_to_storage(hk, dtype)), bits(want_hk))
    assert np.array_equal(bits(torch_to_storage(hv, dtype)), bits(want_hv))
    in_pairs = np.array([[0, 100], [1, 101], [2, 102], [10, 17], [47, 0], [33, 64]],
                        dtype=np.int32)
    gpu.pa_swap_blocks(hk, hv, kc, vc, in_pairs)
    torch.cuda.synchronize()
    assert np.array_equal(bits(torch_to_storage(kc, dtype)),
                          bits(oracle.swap_blocks(want_hk, k0, in_pairs)))
    assert np.array_equal(bits(torch_to_storage(vc, dtype)),
                          bits(oracle.swap_blocks(want_hv, v0, in_pairs)))
    # device to device goes through the same call
    kd, vd = torch.zeros_like(kc), torch.zeros_like(vc)
    gpu.pa_swap_blocks(kc, vc, kd, vd, np.array([[100, 3], [101, 4]], dtype=np.int32))
    torch.cuda.synchronize()
    iview = torch.int16 if dtype == "bf16" else torch.int32
    assert torch.equal(kd[3:5].view(iview), kc[100:102].view(iview))
    assert torch.equal(vd[3:5].view(iview), vc[100:102].view(iview))


@pytest.mark.parametrize("pinned", [True, False])
def test_swap_blocks_many_scattered_pairs(gpu, pinned):
    """More pairs than one launch carries (256), scattered ids both ways."""
    import torch
    say(f"swap_blocks 600 scattered pairs pinned={pinned}")
    rng = np.random.default_rng(9)
    nb, nh, hkv, d = 1024, 700, 8, 128
    k0 = random_storage(rng, (nb, hkv, BS, d), "bf16")
    v0 = random_storage(rng, (nb, hkv, BS, d), "bf16")
    hk0 = random_storage(rng, (nh, hkv, BS, d), "bf16")
    hv0 = random_storage(rng, (nh, hkv, BS, d), "bf16")
    kc, vc = host_to_torch(k0, "bf16", "cuda"), host_to_torch(v0, "bf16", "cuda")
    hk, hv = host_pool(hk0, "bf16", pinned), host_pool(hv0, "bf16", pinned)
    out_pairs = np.stack([rng.choice(nb, 600, replace=False), rng.choice(nh, 600, replace=False)],
                         1).astype(np.int32)
    gpu.pa_swap_blocks(kc, vc, hk, hv, out_pairs)
    torch.cuda.synchronize()
    hk1, hv1 = oracle.swap_blocks(k0, hk0, out_pairs), oracle.swap_blocks(v0, hv0, out_pairs)
    assert np.array_equal(torch_to_storage(hk, "bf16"), hk1)
    assert np.array_equal(torch_to_storage(hv, "bf16"), hv1)
    in_pairs = np.stack([rng.choice(nh, 600, replace=False), rng.choice(nb, 600, replace=False)],
                        1).astype(np.int32)
    gpu.pa_swap_blocks(hk, hv, kc, vc, in_pairs)
    torch.cuda.synchronize()
    assert np.array_equal(torch_to_storage(kc, "bf16"), oracle.swap_blocks(hk1, k0, in_pairs))
    assert np.array_equal(torch_to_storage(vc, "bf16"), oracle.swap_blocks(hv1, v0, in_pairs))


class Steps:
    """A device pool pair and a pinned host pool pair, driven by the native
    manager, mirrored on the host by the oracle manager and oracle copies."""

    def __init__(self, gpu, dtype, hq, hkv, d, nb, nh, seed):
        import torch
        self.L, self.dtype, self.hq, self.hkv, self.d = gpu, dtype, hq, hkv, d
        self.rng = np.random.default_rng(seed)
        self.o = ref.BlockManager(nb, BS, nh)
        self.n = gpu.BlockManager(nb, BS, nh)
        nan = np.float32(np.nan) if dtype == "f32" else np.uint16(0x7FC0)
        st = np.float32 if dtype == "f32" else np.uint16
        self.ok = np.full((nb, hkv, BS, d), nan, dtype=st)
        self.ov = self.ok.copy()
        self.ohk = np.full((nh, hkv, BS, d), nan, dtype=st)
        self.ohv = self.ohk.copy()
        self.kc = host_to_torch(self.ok, dtype, "cuda")
        self.vc = host_to_torch(self.ov, dtype, "cuda")
        self.hk = host_to_torch(self.ohk, dtype, "cpu").pin_memory()
        self.hv = host_to_torch(self.ohv, dtype, "cpu").pin_memory()
        self.scale = np.float32(1.0 / np.sqrt(d))
        self.pending = []                          # (seq, slots) to write this step
        self.torch = torch

    def both(self, name, *args):
        r1 = getattr(self.o, name)(*args)
        r2 = getattr(self.n, name)(*args)
        if name == "append_slots":
            assert list(r1) == [int(x) for x in r2]
            self.pending.append((args[0], list(r1)))
        return r1

    def run_moves(self):
        torch = self.torch
        mo, mn = self.o.take_moves(), self.n.take_moves()
        for a, b in zip(mo, mn):
            assert [tuple(p) for p in a] == [tuple(int(x) for x in p) for p in b]
        copies, outs, ins = mn
        if len(copies):
            self.L.pa_copy_blocks(self.kc, self.vc, torch.from_numpy(copies).cuda())
            self.ok, self.ov = oracle.copy_blocks(self.ok, copies), oracle.copy_blocks(self.ov, copies)
        if len(outs):
            self.L.pa_swap_blocks(self.kc, self.vc, self.hk, self.hv, outs)
            self.ohk = oracle.swap_blocks(self.ok, self.ohk, outs)
            self.ohv = oracle.swap_blocks(self.ov, self.ohv, outs)
        if len(ins):
            self.L.pa_swap_blocks(self.hk, self.hv, self.kc, self.vc, ins)
            self.ok = oracle.swap_blocks(self.ohk, self.ok, ins)
            self.ov = oracle.swap_blocks(self.ohv, self.ov, ins)
        return len(copies), len(outs), len(ins)

    def write(self):
        torch = self.torch
        slots = np.array([s for _, ss in self.pending for s in ss], dtype=np.int64)
        self.pending = []
        if not len(slots):
            return
        k = normal_storage(self.rng, (len(slots), self.hkv, self.d), self.dtype)
        v = normal_storage(self.rng, (len(slots), self.hkv, self.d), self.dtype)
        self.L.pa_reshape_and_cache(host_to_torch(k, self.dtype, "cuda"),
                                    host_to_torch(v, self.dtype, "cuda"), self.kc, self.vc,
                                    torch.from_numpy(slots).cuda())
        self.ok, self.ov = oracle.reshape_and_cache(self.ok, self.ov, k, v, slots)

    def check_pools(self):
        self.torch.cuda.synchronize()
        for got, want in ((self.kc, self.ok), (self.vc, self.ov), (self.hk, self.ohk),
                          (self.hv, self.ohv)):
            assert np.array_equal(bits(torch_to_storage(got, self.dtype)), bits(want))
        self.n.check_invariants()
        self.o.check_invariants()

    def decode(self, seqs, partition_size=0):
        torch = self.torch
        mb = max(len(self.o.block_table(s)) for s in seqs) + 1
        tables, lens, shared = self.n.build_batch(seqs, mb)
        for i, s in enumerate(seqs):
            t = self.o.block_table(s)
            assert tables[i].tolist() == t + [-1] * (mb - len(t))
            assert lens[i] == self.o.num_tokens(s)
            assert shared[i] == self.o.shared_prefix_blocks(s)
        q = normal_storage(self.rng, (len(seqs), self.hq, self.d), self.dtype)
        qt = host_to_torch(q, self.dtype, "cuda")
        out = torch.empty_like(qt)
        maxc = int(lens.max())
        ws = None
        if partition_size:
            nbytes = self.L.pa_decode_workspace_bytes(len(seqs), self.hq, self.d, maxc,
                                                      partition_size)
            ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
        bt, cl, sh = (torch.from_numpy(x).cuda() for x in (tables, lens, shared))
        self.L.pa_decode(out, qt, self.kc, self.vc, bt, cl, float(self.scale), maxc,
                         partition_size, ws, shared_prefix_blocks=sh)
        if partition_size:
            self.L.pa_decode_splitk_reduce(out, ws, cl, maxc, partition_size)
        torch.cuda.synchronize()
        want = oracle.decode(q, self.ok, self.ov, tables, lens, self.scale, self.dtype)
        assert_close(as_f64(out), want, self.dtype, f"decode after moves {seqs}")


    def decode_grouped(self, seqs, partition_size):
        """The manager's sharing groups drive pa_decode_shared_prefix: the output
        must be pa_decode's bit for bit, and the oracle's within tolerance."""
        torch = self.torch
        mb = max(len(self.o.block_table(s)) for s in seqs) + 1
        tables, lens, shared = self.n.build_batch(seqs, mb)
        og, oc, om = self.o.prefix_groups(seqs)
        ng, nc, nm = self.n.prefix_groups(seqs)
        assert og == ng.tolist() and oc == nc.tolist() and om == nm
        q = normal_storage(self.rng, (len(seqs), self.hq, self.d), self.dtype)
        qt = host_to_torch(q, self.dtype, "cuda")
        maxc = int(lens.max())
        nbytes = self.L.pa_decode_workspace_bytes(len(seqs), self.hq, self.d, maxc,
                                                  partition_size)
        ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device="cuda")
        bt, cl, sh, grp, gb = (torch.from_numpy(x).cuda() for x in (tables, lens, shared, ng, nc))
        outs = []
        for grouped in (False, True):
            out = torch.empty_like(qt)
            ws.fill_(0xFF)
            if grouped:
                self.L.pa_decode_shared_prefix(out, qt, self.kc, self.vc, bt, cl,
                                               float(self.scale), maxc, partition_size, ws, gb,
                                               grp, nm)
            else:
                self.L.pa_decode(out, qt, self.kc, self.vc, bt, cl, float(self.scale), maxc,
                                 partition_size, ws, shared_prefix_blocks=sh)
            self.L.pa_decode_splitk_reduce(out, ws, cl, maxc, partition_size)
            torch.cuda.synchronize()
            outs.append(out)
        view = torch.int16 if self.dtype == "bf16" else torch.int32
        assert torch.equal(outs[0].view(view), outs[1].view(view))
        want = oracle.decode(q, self.ok, self.ov, tables, lens, self.scale, self.dtype)
        assert_close(as_f64(outs[1]), want, self.dtype, f"grouped decode {seqs}")
        return nm


@pytest.mark.parametrize("dtype,hq,hkv,d", [("bf16", 32, 8, 128), ("f32", 4, 4, 64),
                                            ("bf16", 8, 8, 128)])
def test_manager_driven_steps(gpu, dtype, hq, hkv, d):
    say(f"manager-driven steps {dtype} hq={hq} hkv={hkv} d={d}")
    st = Steps(gpu, dtype, hq, hkv, d, nb=160, nh=64, seed=21)
    prompts = {0: 37, 1: 64, 2: 100, 3: 5}
    for s, n in prompts.items():
        st.both("add_sequence", s)
        st.both("append_slots", s, n)
    assert st.run_moves() == (0, 0, 0)
    st.write()
    st.check_pools()
    st.decode([0, 1, 2, 3])
    # three samples per prompt ("3 different endings"), plus a prefix and chosen blocks
    samples = []
    for p in prompts:
        for j in range(2):
            c = 10 + 2 * p + j
            st.both("fork", p, c)
            samples.append(c)
    st.both("share", 2, 30, [0, 1, 2])
    st.both("share", 2, 31, [4, 1])
    live = list(prompts) + samples + [30, 31]
    for s in live:
        st.both("append_slots", s, 1)
    copies, _, _ = st.run_moves()
    assert copies == 6                             # prompts 0, 2, 3: two sharers copy each
    st.write()
    st.check_pools()
    st.decode(live)
    st.decode(live, partition_size=32)
    # sharers next to each other: samples after their prompt, seq 30 (seq 2's
    # first three blocks) with seq 2's samples
    order = [0, 10, 11, 1, 12, 13, 2, 30, 14, 15, 3, 16, 17, 31]
    assert sorted(order) == sorted(live)
    assert st.decode_grouped(order, 32) == 4
    for s in (0, 12, 30, 2):
        st.both("append_slots", s, 7)
    st.run_moves()
    st.write()
    st.check_pools()
    st.decode(live)
    # preempt a prompt with its samples and a shared-prefix sequence, finish two others
    st.both("swap_out", [10, 11, 0])
    st.both("swap_out", [30])
    st.both("free_sequence", 1)
    st.both("free_sequence", 12)
    _, outs, _ = st.run_moves()
    assert outs > 0
    st.check_pools()
    live = [s for s in live if s not in (10, 11, 0, 30, 1, 12)]
    st.decode(live)
    st.both("swap_in", [10, 11, 0])
    st.both("swap_in", [30])
    _, _, ins = st.run_moves()
    assert ins == outs
    live += [10, 11, 0, 30]
    for s in live:
        st.both("append_slots", s, 1)
    st.run_moves()
    st.write()
    st.check_pools()
    st.decode(live)
