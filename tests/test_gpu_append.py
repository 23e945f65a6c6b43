"""GPU parity of the append path of a growing cache: fq_encode_scatter (encode new
vectors into chosen records of a fixed-address store) and fq_attn_decode_varlen
(decode attention over each batch's first L_b keys), against the CPU oracle.

Bars: scattered records equal the oracle's codes outside its near-ties (accepted
codes inside), norms bit-exact, every other record and norm of the store left
bit-identical; attention per (batch, query head) within 1e-3 relative in the max
norm, and exactly 0 for a batch with no keys."""
import numpy as np
import pytest

import universal_vector_quantization_amd as fq
import workloads
from oracle import attention as oatt
from oracle import codec as oc
from oracle.codebook import initial_codebook, to_fp16_grid

from gpu_util import D, artifact_or_skip, device, max_rel_rows, to_dev, unpack_sampled

pytestmark = pytest.mark.gpu
TOL = 1e-3
F16_NAN, F16_INF = np.uint16(0x7E00), np.uint16(0x7C00)


@pytest.fixture(scope="module")
def dev():
    return device()


_cbs = {}


def codebook(k, N):
    """A frozen artifact when there is one, else the construction's initial codebook on
    the fp16 grid (any fp16-exact codebook is a valid codec; no Lloyd step needed)."""
    if (k, N) not in _cbs:
        try:
            cw, rot = fq.load_artifact(k, N)
        except FileNotFoundError:
            cw = to_fp16_grid(initial_codebook(D, k, N)).astype(np.float32)
            _, rot = artifact_or_skip(4, 256)
        _cbs[(k, N)] = (fq.Codebook(cw, rot), cw, rot)
    return _cbs[(k, N)]


def _poison_past(norms_bkt, lens):
    """Norm bits past each batch's valid length set to fp16 NaN / inf: any read of them
    by the kernel would show in the output."""
    v = norms_bkt.view(np.uint16)
    for b, L in enumerate(lens):
        L = min(max(int(L), 0), v.shape[-1])
        v[b, :, L::2] = F16_NAN
        v[b, :, L + 1::2] = F16_INF


# ------------------------------------------------------------------ fq_encode_scatter
# Batches of at most 2048 vectors go to the small-batch encoder (one wave per vector)
# where the codebook shape allows it; larger ones to the throughput encoders.
@pytest.mark.parametrize("k,N,xdt,ndt,n", [
    (4, 256, np.float16, np.float16, 300),    # small-batch encoder, 16-byte records
    (4, 256, np.float16, np.float16, 5000),   # fp16 matrix-core encoder
    (4, 256, np.float32, np.float32, 5000),   # fp32-input matrix-core encoder
    (8, 4096, np.float16, np.float16, 300),   # 12-byte records (fp16 matrix-core encoder)
    (2, 16, np.float32, np.float16, 300),     # small-batch encoder, k = 2
    (2, 16, np.float32, np.float16, 5000),    # one-lane-per-vector encoder
    (4, 32, np.float16, np.float32, 300),     # 10-byte records: byte stores (small batch)
    (4, 32, np.float16, np.float32, 5000),    # 10-byte records: byte stores (matrix core)
    (64, 256, np.float16, np.float16, 300),   # k = d encoder, 1-byte records
])
def test_encode_scatter_parity(dev, k, N, xdt, ndt, n):
    import torch

    cb, cw, rot = codebook(k, N)
    bits, m = oc.code_bits(N), D // k
    cap = max(3001, 2 * n + 1)
    x = workloads.gpt2_small_kv()[7000:7000 + n].astype(xdt)
    rng = np.random.default_rng(k * 7919 + N)
    slots = rng.choice(cap, n, replace=False).astype(np.int64)
    slots[[5, 77, 200]] = [-1, cap, cap + 1000]  # skipped vectors
    store0 = workloads.random_code_store(cb.code_bytes(cap), 11 + k)
    norms0 = workloads.random_norms(cap, 12 + k, ndt)
    codes = to_dev(store0, dev)
    norms = to_dev(norms0, dev)
    print(f"[scatter parity] k={k} N={N} x={np.dtype(xdt).name} norms={np.dtype(ndt).name} n={n} cap={cap}",
          flush=True)
    fq.fq_encode_scatter(cb.handle, to_dev(x, dev), to_dev(slots, dev), cap, codes, norms)
    torch.cuda.synchronize()
    got_c = oc.unpack_codes(codes.cpu().numpy(), cap, m, bits)
    got_n = norms.cpu().numpy()

    enc = oc.encode(x, rot, cw, ndt)
    base_c = oc.unpack_codes(store0, cap, m, bits)
    exp_c, exp_n = oc.write_records(base_c, norms0, enc.codes, enc.norms, slots)
    uint = np.uint16 if ndt == np.float16 else np.uint32
    assert np.array_equal(got_n.view(uint), exp_n.view(uint)), "norms differ"
    valid = (slots >= 0) & (slots < cap)
    untouched = np.ones(cap, dtype=bool)
    untouched[slots[valid]] = False
    assert np.array_equal(got_c[untouched], base_c[untouched]), "a record outside the slots changed"
    mism = got_c[slots[valid]] != exp_c[slots[valid]]
    assert not (mism & ~enc.near_tie[valid]).any()
    other = enc.codes.copy()
    other[valid] = got_c[slots[valid]]
    assert oc.accepted(enc.y, cw, enc, other).all()


@pytest.mark.parametrize("k,N,n", [(4, 256, 1007), (4, 256, 6007), (8, 4096, 777), (2, 16, 130)])
def test_encode_scatter_identity_slots_equal_encode(dev, k, N, n):
    # slots 0..n-1 into a store of n records: byte-identical to fq_encode.
    import torch

    cb, _, _ = codebook(k, N)
    x = to_dev(workloads.gpt2_small_kv()[:n], dev)
    a_c = torch.empty(cb.code_bytes(n), dtype=torch.uint8, device=dev)
    a_n = torch.empty(n, dtype=torch.float16, device=dev)
    fq.fq_encode(cb.handle, x, a_c, a_n)
    b_c = torch.full_like(a_c, 0xA5)
    b_n = torch.full_like(a_n, 3.0)
    fq.fq_encode_scatter(cb.handle, x, torch.arange(n, dtype=torch.int64, device=dev), n, b_c, b_n)
    torch.cuda.synchronize()
    assert torch.equal(a_c, b_c) and torch.equal(a_n.view(torch.int16), b_n.view(torch.int16))


def test_encode_scatter_rejects_records_sharing_bytes(dev):
    # k = d = 64, N = 4096: 12-bit records share bytes; nothing is launched.
    import torch

    cb, _, _ = codebook(64, 4096)
    codes = torch.full((cb.code_bytes(10),), 7, dtype=torch.uint8, device=dev)
    norms = torch.zeros(10, dtype=torch.float16, device=dev)
    x = torch.zeros((2, D), dtype=torch.float16, device=dev)
    with pytest.raises(fq.FQError) as e:
        fq.fq_encode_scatter(cb.handle, x, torch.tensor([0, 3], dtype=torch.int64, device=dev), 10, codes, norms)
    assert e.value.status == fq.FQ_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert int(codes.min()) == 7 and int(codes.max()) == 7


# ------------------------------------------------------------------ fq_attn_decode_varlen
def _varlen_gpu(cb, dev, q, kc, kn, vc, vn, lens, B, Hq, Hkv, T, scale=0.125):
    import torch

    out = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device=dev)
    wsb = fq.fq_attn_workspace_bytes(cb.handle, B, Hq, Hkv, T)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
    fq.fq_attn_decode_varlen(cb.handle, to_dev(q, dev), to_dev(kc, dev), to_dev(kn, dev), to_dev(vc, dev),
                             to_dev(vn, dev), to_dev(np.asarray(lens, dtype=np.int32), dev), B, Hq, Hkv, T, scale,
                             out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("k,N,B,Hq,Hkv,T,lens", [
    (4, 256, 4, 32, 4, 2048, [0, 1, 777, 2048]),        # fast path: empty, one key, ragged, full
    (4, 256, 3, 16, 2, 1000, [999, 513, 64]),           # odd length; a length ending a 64-token unit
    (4, 256, 2, 8, 1, 4096, [-5, 5000]),                # clamped to 0 and to T
    (4, 256, 2, 8, 1, 1001, [0, 1000]),                 # T not a multiple of 8: the general kernel
    (2, 16, 3, 12, 3, 300, [299, 1, 150]),              # general kernel, k = 2
    (4, 256, 8, 16, 2, 8192, [8192, 0, 0, 0, 0, 0, 0, 1]),  # one long slab takes nearly every workgroup
])
def test_varlen_attention_random_cache(dev, k, N, B, Hq, Hkv, T, lens):
    cb, cw, rot = codebook(k, N)
    bits, m = oc.code_bits(N), D // k
    n = B * Hkv * T
    nbytes = (n * m * bits + 7) // 8
    kc, vc = workloads.random_code_store(nbytes, 500 + T), workloads.random_code_store(nbytes, 501 + T)
    kn = workloads.random_norms(n, 502 + T).reshape(B, Hkv, T)
    vn = workloads.random_norms(n, 503 + T).reshape(B, Hkv, T)
    _poison_past(kn, lens)
    _poison_past(vn, lens)
    q = np.random.default_rng(T + B).standard_normal((B, Hq, D)).astype(np.float16)
    print(f"[varlen attention] k={k} N={N} B={B} Hq={Hq} Hkv={Hkv} T={T} lens={lens}", flush=True)
    got = _varlen_gpu(cb, dev, q, kc, kn, vc, vn, lens, B, Hq, Hkv, T)
    unp = lambda s: oc.unpack_codes(s, n, m, bits).reshape(B, Hkv, T, m)
    ref = oatt.attention(q, unp(kc), kn, unp(vc), vn, rot, cw, 0.125, lengths=lens)
    assert max_rel_rows(got, ref) <= TOL
    for b, L in enumerate(lens):
        if L <= 0:
            assert np.all(got[b] == 0.0)


def test_varlen_many_batches_balanced_split(dev):
    # 100 batches (two 64-batch steps of the in-kernel scan that shares the workgroups
    # out by valid length), lengths from 0 to T
    cb, cw, rot = codebook(4, 256)
    B, Hq, Hkv, T = 100, 8, 1, 1024
    n = B * Hkv * T
    kc, vc = workloads.random_code_store(n * 16, 31), workloads.random_code_store(n * 16, 32)
    kn = workloads.random_norms(n, 33).reshape(B, Hkv, T)
    vn = workloads.random_norms(n, 34).reshape(B, Hkv, T)
    lens = np.random.default_rng(35).integers(0, T + 1, size=B)
    lens[[0, 63, 64, 99]] = [0, T, 1, 511]
    _poison_past(kn, lens)
    _poison_past(vn, lens)
    q = np.random.default_rng(36).standard_normal((B, Hq, D)).astype(np.float16)
    print(f"[varlen balanced] B={B} T={T}", flush=True)
    got = _varlen_gpu(cb, dev, q, kc, kn, vc, vn, lens, B, Hq, Hkv, T)
    unp = lambda s: oc.unpack_codes(s, n, 16, 8).reshape(B, Hkv, T, 16)
    ref = oatt.attention(q, unp(kc), kn, unp(vc), vn, rot, cw, 0.125, lengths=lens)
    assert max_rel_rows(got, ref) <= TOL
    assert np.all(got[0] == 0.0)


@pytest.mark.parametrize("T", [4096, 1000, 1001])
def test_varlen_full_lengths_equal_plain_attention(dev, T):
    # lens = T everywhere: the same result as fq_attn_decode (on the fast path the
    # split of the keys over workgroups differs, so the sums may round differently).
    import torch

    cb, _, _ = codebook(4, 256)
    B, Hq, Hkv = 2, 16, 2
    n = B * Hkv * T
    kc, vc = workloads.random_code_store(n * 16, 61), workloads.random_code_store(n * 16, 62)
    kn, vn = workloads.random_norms(n, 63), workloads.random_norms(n, 64)
    q = np.random.default_rng(5).standard_normal((B, Hq, D)).astype(np.float16)
    a = _varlen_gpu(cb, dev, q, kc, kn, vc, vn, [T] * B, B, Hq, Hkv, T)
    out = torch.zeros((B, Hq, D), dtype=torch.float32, device=dev)
    ws = torch.empty(fq.fq_attn_workspace_bytes(cb.handle, B, Hq, Hkv, T), dtype=torch.uint8, device=dev)
    fq.fq_attn_decode(cb.handle, to_dev(q, dev), to_dev(kc, dev), to_dev(kn, dev), to_dev(vc, dev), to_dev(vn, dev),
                      B, Hq, Hkv, T, 0.125, out, ws)
    torch.cuda.synchronize()
    assert max_rel_rows(a, out.cpu().numpy()) <= 1e-5


def test_varlen_full_size_sampled(dev):
    # The attention workload's launch (B=16, Hq=32, Hkv=4, T=32768) with per-batch
    # lengths spread over [0, T]; sampled (batch, KV head) groups against the oracle.
    cb, cw, rot = codebook(4, 256)
    B, Hq, Hkv, T = workloads.ATTN_B, workloads.ATTN_HQ, workloads.ATTN_HKV, workloads.ATTN_T
    n = B * Hkv * T
    kc, vc = workloads.random_code_store(n * 16, 71), workloads.random_code_store(n * 16, 72)
    kn = workloads.random_norms(n, 73).reshape(B, Hkv, T)
    vn = workloads.random_norms(n, 74).reshape(B, Hkv, T)
    lens = np.random.default_rng(75).integers(1, T, size=B)
    lens[3], lens[8], lens[12] = 0, T, 1
    _poison_past(kn, lens)
    _poison_past(vn, lens)
    q = np.random.default_rng(76).standard_normal((B, Hq, D)).astype(np.float16)
    print("[varlen full size] B=16 Hq=32 Hkv=4 T=32768", flush=True)
    got = _varlen_gpu(cb, dev, q, kc, kn, vc, vn, lens, B, Hq, Hkv, T)
    assert np.all(got[3] == 0.0)
    G = Hq // Hkv
    for b, g in [(0, 1), (8, 3), (12, 0), (15, 2)]:
        L = int(lens[b])
        idx = np.arange(L) + (b * Hkv + g) * T
        ref = oatt.attention(q[b:b + 1, g * G:(g + 1) * G], unpack_sampled(kc, idx, 16, 8).reshape(1, 1, L, 16),
                             kn[b, g, :L].reshape(1, 1, L), unpack_sampled(vc, idx, 16, 8).reshape(1, 1, L, 16),
                             vn[b, g, :L].reshape(1, 1, L), rot, cw, 0.125)
        assert max_rel_rows(got[b:b + 1, g * G:(g + 1) * G], ref) <= TOL


# ------------------------------------------------------------------ the decode loop
@pytest.mark.parametrize("k,N,T", [(4, 256, 264), (4, 256, 261), (2, 16, 200)])
def test_decode_loop_append_then_attend(dev, k, N, T):
    # Prefill each sequence's first tokens, then per step: encode the new token's K
    # and V into slot (b, g, len_b) of the cache, attend over len_b + 1 keys.  Batch 1
    # finishes half-way (its slots become -1, its length stops).  The cache starts as
    # random bytes with poisoned norms, so nothing past a length may be read.
    import torch

    cb, cw, rot = codebook(k, N)
    bits, m = oc.code_bits(N), D // k
    B, Hq, Hkv, steps = 3, 8, 2, 24
    G, cap = Hq // Hkv, B * Hkv * T
    src = workloads.gpt2_small_kv()
    rng = np.random.default_rng(T)
    lens = np.array([0, 5, 37], dtype=np.int64)

    store = {}
    for name, seed in (("k", 81), ("v", 82)):
        c0 = workloads.random_code_store(cb.code_bytes(cap), seed)
        n0 = workloads.random_norms(cap, seed + 10).reshape(B, Hkv, T)
        _poison_past(n0, [0] * B)
        store[name] = {"gc": to_dev(c0, dev), "gn": to_dev(n0.reshape(-1), dev),
                       "oc": oc.unpack_codes(c0, cap, m, bits), "on": n0.reshape(-1).copy(),
                       "tie": np.zeros((cap, m), dtype=bool)}
    row = [0]

    def append(slots_np):
        for name in ("k", "v"):
            x = src[row[0]:row[0] + len(slots_np)]
            row[0] += len(slots_np)
            s = store[name]
            fq.fq_encode_scatter(cb.handle, to_dev(x, dev), to_dev(slots_np, dev), cap, s["gc"], s["gn"])
            enc = oc.encode(x, rot, cw, np.float16)
            s["tie"], _ = oc.write_records(s["tie"], s["on"], enc.near_tie, enc.norms, slots_np)
            s["oc"], s["on"] = oc.write_records(s["oc"], s["on"], enc.codes, enc.norms, slots_np)

    base = lambda b, g: (b * Hkv + g) * T
    pre = [base(b, g) + t for b in range(B) for g in range(Hkv) for t in range(lens[b])]
    append(np.array(pre, dtype=np.int64))
    print(f"[decode loop] k={k} N={N} T={T} B={B} Hq={Hq} Hkv={Hkv} steps={steps}", flush=True)
    worst = 0.0
    for step in range(steps):
        active = np.array([True, step < steps // 2, True])
        slots = np.array([base(b, g) + lens[b] if active[b] else -1 for b in range(B) for g in range(Hkv)],
                         dtype=np.int64)
        append(slots)
        lens = lens + active
        q = rng.standard_normal((B, Hq, D)).astype(np.float16)
        out = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device=dev)
        ws = torch.empty(max(fq.fq_attn_workspace_bytes(cb.handle, B, Hq, Hkv, T), 16), dtype=torch.uint8,
                         device=dev)
        fq.fq_attn_decode_varlen(cb.handle, to_dev(q, dev), store["k"]["gc"], store["k"]["gn"], store["v"]["gc"],
                                 store["v"]["gn"], to_dev(lens.astype(np.int32), dev), B, Hq, Hkv, T, 0.125, out, ws)
        torch.cuda.synchronize()
        shp = lambda s: s["oc"].reshape(B, Hkv, T, m)
        ref = oatt.attention(q, shp(store["k"]), store["k"]["on"].reshape(B, Hkv, T), shp(store["v"]),
                             store["v"]["on"].reshape(B, Hkv, T), rot, cw, 0.125, lengths=lens)
        worst = max(worst, max_rel_rows(out.cpu().numpy(), ref))
    assert worst <= TOL
    # the caches themselves: records match the oracle's store outside its near-ties
    # (norms bit-exact); records never written keep their initial bytes
    for name in ("k", "v"):
        s = store[name]
        got_n = s["gn"].cpu().numpy()
        assert np.array_equal(got_n.view(np.uint16), s["on"].view(np.uint16))
        got_c = oc.unpack_codes(s["gc"].cpu().numpy(), cap, m, bits)
        assert not ((got_c != s["oc"]) & ~s["tie"]).any()


def test_decode_step_as_graph_matches_eager(dev):
    # The append + attention step captured once as a HIP graph and replayed with new
    # vectors, slots and lengths in its fixed device buffers, eager work and
    # synchronisations between replays: every replay's cache and output are
    # bit-identical to the same step run eagerly on a twin cache.
    import torch

    cb, _, _ = codebook(4, 256)
    B, Hq, Hkv, T = 3, 8, 2, 264
    cap = 2 * B * Hkv * T  # K records then V records
    c0 = workloads.random_code_store(cb.code_bytes(cap), 91)
    n0 = workloads.random_norms(cap, 92)
    ga, gn = to_dev(c0, dev), to_dev(n0, dev)
    ea, en = to_dev(c0, dev), to_dev(n0, dev)
    half = cb.code_bytes(cap // 2)
    src = workloads.gpt2_small_kv()
    rng = np.random.default_rng(93)
    q = to_dev(rng.standard_normal((B, Hq, D)).astype(np.float16), dev)
    wsb = fq.fq_attn_workspace_bytes(cb.handle, B, Hq, Hkv, T)
    ws_g = torch.empty(wsb, dtype=torch.uint8, device=dev)
    ws_e = torch.empty(wsb, dtype=torch.uint8, device=dev)
    out_g = torch.zeros((B, Hq, D), dtype=torch.float32, device=dev)
    out_e = torch.zeros((B, Hq, D), dtype=torch.float32, device=dev)
    x_buf = torch.zeros((2 * B * Hkv, D), dtype=torch.float16, device=dev)
    s_buf = torch.full((2 * B * Hkv,), -1, dtype=torch.int64, device=dev)
    l_buf = torch.zeros(B, dtype=torch.int32, device=dev)

    def step(codes, norms, out, ws, x, s, l, stream):
        fq.fq_encode_scatter(cb.handle, x, s, cap, codes, norms, stream)
        fq.fq_attn_decode_varlen(cb.handle, q, codes[:half], norms[:cap // 2], codes[half:], norms[cap // 2:], l,
                                 B, Hq, Hkv, T, 0.125, out, ws, stream)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up outside the capture (slots -1: nothing written)
        step(ga, gn, out_g, ws_g, x_buf, s_buf, l_buf, side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(ga, gn, out_g, ws_g, x_buf, s_buf, l_buf, torch.cuda.current_stream())
    lens = np.array([0, 7, 40])
    base = (np.arange(B)[:, None] * Hkv + np.arange(Hkv)[None, :]) * T
    for it in range(6):
        slots = np.concatenate([(base + lens[:, None]).reshape(-1)] * 2) + np.repeat([0, cap // 2], B * Hkv)
        lens = lens + 1
        x = to_dev(src[it * 2 * B * Hkv:(it + 1) * 2 * B * Hkv], dev)
        s = to_dev(slots.astype(np.int64), dev)
        l = to_dev(lens.astype(np.int32), dev)
        x_buf.copy_(x)
        s_buf.copy_(s)
        l_buf.copy_(l)
        graph.replay()
        torch.cuda.synchronize()
        step(ea, en, out_e, ws_e, x, s, l, None)  # eager twin
        torch.cuda.synchronize()
        assert torch.equal(ga, ea) and torch.equal(gn.view(torch.int16), en.view(torch.int16)), f"replay {it}: cache"
        assert torch.equal(out_g.view(torch.int32), out_e.view(torch.int32)), f"replay {it}: output"
        assert torch.isfinite(out_g).all()
