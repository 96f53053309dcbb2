"""Paged cache and chunked compressed store on the GPU.

- tq_decode_attention_paged on pages in a shuffled order gives the same bits
  as tq_decode_attention on the same records laid out contiguously.
- PagedKVCache: chunks appended one after another (sizes that cross page
  boundaries, single tokens) encode exactly the bytes a one-shot encode
  writes, and a decode over the chunks matches the oracle's encode + decode
  of the concatenated tokens; a needle planted in one chunk wins the argmax.
"""
import numpy as np
import pytest

import oracle.tq_oracle as O
import tq_workloads as W
from tests import parity as P

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import kv_cache_quantization_encode_amd as tq  # noqa: E402
from kv_cache_quantization_encode_amd import _lib as L  # noqa: E402

DEV = "cuda"


def _np(t):
    return t.detach().cpu().numpy()


@pytest.mark.parametrize("page_size", [64, 256])
def test_paged_equals_contiguous(page_size):
    kw = dict(mode="prod", bits=3)
    B, Hq, Hkv, max_ctx = 3, 8, 2, 1536
    ctx = [700, 1, 1536]
    Tg = tq.Tables(L.key_config(seed=7, **kw), DEV)
    n = B * Hkv * max_ctx
    kb = W.kv_rows(21, 1, n)[1]
    vb = W.kv_rows(21, 2, n)[1]
    keys = torch.from_numpy(kb.view(np.int16)).view(torch.bfloat16).to(DEV)
    vals = torch.from_numpy(vb.view(np.int16)).view(torch.bfloat16).to(DEV)
    kp = tq.encode_keys(Tg, keys)
    vp = tq.encode_values(vals, 2)
    q = torch.from_numpy(W.queries(21, B, Hq)[1].view(np.int16)).view(torch.bfloat16).to(DEV)
    ctx_t = torch.tensor(ctx, dtype=torch.int32, device=DEV)
    dec = tq.Decoder(Tg, B, Hq, Hkv, max_ctx, 2)
    lse_c = torch.empty((B, Hq), device=DEV)
    sc_c = torch.full((B, Hq, max_ctx), float("nan"), device=DEV)
    out_c = dec(q, ctx_t, kp, vp, lse=lse_c, scores=sc_c)
    # the same records, pages in a shuffled order inside a larger pool
    nb = max_ctx // page_size
    n_pages = B * nb + 5
    perm = np.random.default_rng(3).permutation(n_pages)[:B * nb].reshape(B, nb)
    bt = torch.from_numpy(perm.astype(np.int32)).to(DEV)
    t = torch.arange(max_ctx, device=DEV)
    src, dst = [], []
    for b in range(B):
        for h in range(Hkv):
            src.append((b * Hkv + h) * max_ctx + t)
            dst.append((bt[b].long()[t // page_size] * Hkv + h) * page_size + t % page_size)
    src, dst = torch.cat(src), torch.cat(dst)
    n_rec = n_pages * Hkv * page_size
    kpp = {k: torch.zeros((n_rec,) + v.shape[1:], dtype=v.dtype, device=DEV) for k, v in kp.items()}
    vpp = {k: torch.zeros((n_rec,) + v.shape[1:], dtype=v.dtype, device=DEV) for k, v in vp.items()}
    for k in kp:
        kpp[k][dst] = kp[k][src]
    for k in vp:
        vpp[k][dst] = vp[k][src]
    decp = tq.Decoder(Tg, B, Hq, Hkv, max_ctx, 2, page_size=page_size)
    lse_p = torch.empty((B, Hq), device=DEV)
    sc_p = torch.full((B, Hq, max_ctx), float("nan"), device=DEV)
    out_p = decp(q, ctx_t, kpp, vpp, lse=lse_p, scores=sc_p, block_table=bt)
    torch.cuda.synchronize()
    assert torch.equal(out_c, out_p)
    assert torch.equal(lse_c, lse_p)
    for b in range(B):
        assert torch.equal(sc_c[b, :, :ctx[b]], sc_p[b, :, :ctx[b]])


@pytest.mark.parametrize("page_size", [64, 256])
def test_paged_append_equals_contiguous_append(page_size):
    """tq_decode_attention_paged_append against tq_decode_attention_append on
    the same records in shuffled pages: outputs, lse and scores bit for bit,
    the new records equal at their paged and contiguous slots, every other
    record untouched.  The lengths include a token that opens a page of its
    own, a one-token sequence and a full one."""
    kw = dict(mode="prod", bits=3)
    B, Hq, Hkv, max_ctx = 3, 8, 2, 1536
    ctx = [page_size + 1, 1, 1536]
    Tg = tq.Tables(L.key_config(seed=7, **kw), DEV)
    n = B * Hkv * max_ctx
    kb = W.kv_rows(23, 1, n)[1]
    vb = W.kv_rows(23, 2, n)[1]
    kp = tq.encode_keys(Tg, torch.from_numpy(kb.view(np.int16)).view(torch.bfloat16).to(DEV))
    vp = tq.encode_values(torch.from_numpy(vb.view(np.int16)).view(torch.bfloat16).to(DEV), 2)
    q = torch.from_numpy(W.queries(23, B, Hq)[1].view(np.int16)).view(torch.bfloat16).to(DEV)
    knb = W.kv_rows(24, 1, B * Hkv)[1]
    vnb = W.kv_rows(24, 2, B * Hkv)[1]
    kn = torch.from_numpy(knb.view(np.int16)).view(torch.bfloat16).to(DEV).view(B, Hkv, 128)
    vn = torch.from_numpy(vnb.view(np.int16)).view(torch.bfloat16).to(DEV).view(B, Hkv, 128)
    ctx_t = torch.tensor(ctx, dtype=torch.int32, device=DEV)
    # the paged copy of the records, taken before the contiguous call writes
    nb = max_ctx // page_size
    n_pages = B * nb + 5
    perm = np.random.default_rng(4).permutation(n_pages)[:B * nb].reshape(B, nb)
    bt = torch.from_numpy(perm.astype(np.int32)).to(DEV)
    t = torch.arange(max_ctx, device=DEV)
    src, dst = [], []
    for b in range(B):
        for h in range(Hkv):
            src.append((b * Hkv + h) * max_ctx + t)
            dst.append((bt[b].long()[t // page_size] * Hkv + h) * page_size + t % page_size)
    src, dst = torch.cat(src), torch.cat(dst)
    n_rec = n_pages * Hkv * page_size
    kpp = {k: torch.zeros((n_rec,) + v.shape[1:], dtype=v.dtype, device=DEV) for k, v in kp.items()}
    vpp = {k: torch.zeros((n_rec,) + v.shape[1:], dtype=v.dtype, device=DEV) for k, v in vp.items()}
    for k in kp:
        kpp[k][dst] = kp[k][src]
    for k in vp:
        vpp[k][dst] = vp[k][src]
    before = {k: v.clone() for k, v in list(kpp.items()) + [("v_" + k, v) for k, v in vpp.items()]}
    dec = tq.Decoder(Tg, B, Hq, Hkv, max_ctx, 2)
    lse_c = torch.empty((B, Hq), device=DEV)
    sc_c = torch.full((B, Hq, max_ctx), float("nan"), device=DEV)
    out_c = dec(q, ctx_t, kp, vp, lse=lse_c, scores=sc_c, k_new=kn, v_new=vn)
    decp = tq.Decoder(Tg, B, Hq, Hkv, max_ctx, 2, page_size=page_size)
    lse_p = torch.empty((B, Hq), device=DEV)
    sc_p = torch.full((B, Hq, max_ctx), float("nan"), device=DEV)
    out_p = decp(q, ctx_t, kpp, vpp, lse=lse_p, scores=sc_p, block_table=bt, k_new=kn, v_new=vn)
    torch.cuda.synchronize()
    assert torch.equal(out_c, out_p)
    assert torch.equal(lse_c, lse_p)
    for b in range(B):
        assert torch.equal(sc_c[b, :, :ctx[b]], sc_p[b, :, :ctx[b]])
    for k in kp:
        assert torch.equal(kpp[k][dst], kp[k][src]), k
    for k in vp:
        assert torch.equal(vpp[k][dst], vp[k][src]), k
    # records other than the new tokens' are as before
    new = torch.tensor([int(dst[(b * Hkv + h) * max_ctx + ctx[b] - 1]) for b in range(B) for h in range(Hkv)],
                       device=DEV)
    keep = torch.ones(n_rec, dtype=torch.bool, device=DEV)
    keep[new] = False
    for k, v in list(kpp.items()) + [("v_" + k, v) for k, v in vpp.items()]:
        assert torch.equal(v[keep], before[k][keep]), k


def test_store_decode_step_appends_in_the_launch():
    """PagedKVCache.decode_step (one launch per step: the new token encoded
    into its page and attended) against append() of that token followed by a
    plain paged decode: the same records and the same outputs, over steps that
    cross a page boundary."""
    kw = dict(mode="prod", bits=3)
    Tg = tq.Tables(L.key_config(seed=9, **kw), DEV)
    B, Hq, Hkv, page_size = 2, 8, 2, 64
    a = tq.PagedKVCache(Tg, Hkv, 2, n_pages=16, page_size=page_size, max_seqs=B, max_pages_per_seq=4)
    c = tq.PagedKVCache(Tg, Hkv, 2, n_pages=16, page_size=page_size, max_seqs=B, max_pages_per_seq=4)
    n0 = 62
    for s in range(B):
        kb = W.kv_rows(25 + s, 1, n0 * Hkv)[1]
        vb = W.kv_rows(25 + s, 2, n0 * Hkv)[1]
        k = torch.from_numpy(kb.view(np.int16)).view(torch.bfloat16).to(DEV).view(n0, Hkv, 128)
        v = torch.from_numpy(vb.view(np.int16)).view(torch.bfloat16).to(DEV).view(n0, Hkv, 128)
        a.append(s, k, v)
        c.append(s, k, v)
    for step in range(4):   # tokens 62 .. 65: the third opens page 1
        q = torch.from_numpy(W.queries(30 + step, B, Hq)[1].view(np.int16)).view(torch.bfloat16).to(DEV)
        kb = W.kv_rows(40 + step, 1, B * Hkv)[1]
        vb = W.kv_rows(40 + step, 2, B * Hkv)[1]
        k = torch.from_numpy(kb.view(np.int16)).view(torch.bfloat16).to(DEV).view(B, Hkv, 128)
        v = torch.from_numpy(vb.view(np.int16)).view(torch.bfloat16).to(DEV).view(B, Hkv, 128)
        out_a = a.decode_step(q, k, v)
        for s in range(B):
            c.append(s, k[s:s + 1], v[s:s + 1])
        out_c = c.decode(q)
        torch.cuda.synchronize()
        assert a.lengths == c.lengths
        assert torch.equal(a.block_table, c.block_table)
        for s in range(B):
            sl = a.slots(s, 0, a.lengths[s])
            old_rows = a.slots(s, 0, n0)
            for k_ in a.vp:     # value records: bit-exact in both encoders
                assert torch.equal(a.vp[k_][sl], c.vp[k_][sl]), (step, s, k_)
            for k_ in a.kp:     # the cached tokens' key records: untouched
                assert torch.equal(a.kp[k_][old_rows], c.kp[k_][old_rows]), (step, s, k_)
                # the appended ones: two float32 encoders, equal but for
                # coordinates within rounding of a boundary (at most a byte here)
                diff = (a.kp[k_][sl] != c.kp[k_][sl]).sum().item()
                assert diff <= 1, (step, s, k_, diff)
        # the new token's score is float32 from its record in one, a table
        # lookup in the other: outputs agree to well inside the parity bound
        assert float((out_a - out_c).abs().max()) <= 2e-3


def test_paged_block_table_clamped_into_the_pool():
    """A block table naming the pool's last page works as any other; an
    entry past the pool (or negative) is clamped into [0, n_pages) on the
    device, so it reads the pool's last (first) page instead of memory past
    the planes: the results equal those of the table with that page."""
    kw = dict(mode="prod", bits=3)
    B, Hq, Hkv, page_size, nb = 2, 8, 2, 64, 4
    max_ctx = nb * page_size
    n_pages = 9
    Tg = tq.Tables(L.key_config(seed=5, **kw), DEV)
    n_rec = n_pages * Hkv * page_size
    kb = W.kv_rows(22, 1, n_rec)[1]
    vb = W.kv_rows(22, 2, n_rec)[1]
    kp = tq.encode_keys(Tg, torch.from_numpy(kb.view(np.int16)).view(torch.bfloat16).to(DEV))
    vp = tq.encode_values(torch.from_numpy(vb.view(np.int16)).view(torch.bfloat16).to(DEV), 2)
    q = torch.from_numpy(W.queries(22, B, Hq)[1].view(np.int16)).view(torch.bfloat16).to(DEV)
    ctx_t = torch.tensor([max_ctx, max_ctx - 10], dtype=torch.int32, device=DEV)
    decp = tq.Decoder(Tg, B, Hq, Hkv, max_ctx, 2, page_size=page_size)

    def run(table):
        bt = torch.tensor(table, dtype=torch.int32, device=DEV)
        out = decp(q, ctx_t, kp, vp, block_table=bt)
        torch.cuda.synchronize()
        return out.clone()

    ref = run([[3, n_pages - 1, 0, 5], [n_pages - 1, 2, 7, 1]])   # last page named directly
    assert torch.equal(run([[3, n_pages + 6, 0, 5], [1 << 30, 2, 7, 1]]), ref)
    ref0 = run([[3, 0, 0, 5], [n_pages - 1, 2, 7, 1]])
    assert torch.equal(run([[3, -4, 0, 5], [n_pages - 1, 2, 7, 1]]), ref0)
    assert torch.isfinite(ref).all() and torch.isfinite(ref0).all()


def test_chunked_store_matches_one_shot_and_oracle():
    kw = dict(mode="prod", bits=3)
    Hkv, Hq, d, G = 2, 8, 128, 4
    chunks = [[300, 1, 64, 2000, 17], [1, 1, 511, 700]]
    Tg = tq.Tables(L.key_config(seed=42, **kw), DEV)
    To = O.build_tables(O.KeyConfig(mode="prod", bits=3, seed=42))
    store = tq.PagedKVCache(Tg, Hkv, 2, n_pages=40, page_size=128, max_seqs=2, max_pages_per_seq=20)
    qv, qb = W.queries(22, 2, Hq)
    tokens = []
    for s, sizes in enumerate(chunks):
        total = sum(sizes)
        kv, _ = W.kv_rows(22, 1 + 10 * s, total * Hkv)
        vv, _ = W.kv_rows(22, 2 + 10 * s, total * Hkv)
        kv = kv.reshape(total, Hkv, d)
        vv = vv.reshape(total, Hkv, d)
        # needle: token 2100 (inside the fourth chunk) of sequence 0, head 1,
        # along the first query head of that KV head's group
        if s == 0:
            qd = qv[0, G].astype(np.float64)
            kv[2100, 1] = (6.0 * qd / np.linalg.norm(qd)).astype(np.float32)
        kv = W.bf16_values(W.bf16_bits(kv))
        vv = W.bf16_values(W.bf16_bits(vv))
        t0 = 0
        for n in sizes:
            kt = torch.from_numpy(kv[t0:t0 + n]).to(DEV).to(torch.bfloat16)
            vt = torch.from_numpy(vv[t0:t0 + n]).to(DEV).to(torch.bfloat16)
            store.append(s, kt, vt)
            t0 += n
        tokens.append((kv, vv))
    assert store.lengths == [sum(c) for c in chunks]
    q = torch.from_numpy(qb.view(np.int16)).view(torch.bfloat16).to(DEV)
    scores = torch.full((2, Hq, store.max_pages_per_seq * store.page_size), float("nan"), device=DEV)
    out = _np(store.decode(q, scores=scores))
    scores = _np(scores)
    for s, (kv, vv) in enumerate(tokens):
        total = kv.shape[0]
        # the appended chunks hold the bytes a one-shot encode of the sequence writes
        one = tq.encode_keys(Tg, torch.from_numpy(kv.reshape(-1, d)).to(DEV).to(torch.bfloat16))
        onev = tq.encode_values(torch.from_numpy(vv.reshape(-1, d)).to(DEV).to(torch.bfloat16), 2)
        sl = store.slots(s, 0, total)
        for k in one:
            assert torch.equal(store.kp[k][sl], one[k]), k
        for k in onev:
            assert torch.equal(store.vp[k][sl], onev[k]), k
        # decode over the chunks against the oracle's encode + decode
        for h in range(Hkv):
            enc = O.encode_keys(kv[:, h].astype(np.float64), To)
            khat = O.dequant_keys(enc, To)
            vhat = O.dequant_values(O.encode_values(vv[:, h], 2))
            heads = slice(h * G, (h + 1) * G)
            s_ref, o_ref, _ = O.decode_attention(qv[s, heads].astype(np.float64), khat, vhat, total)
            P.check_out(out[s, heads], o_ref)
            # scores agree where the bytes agree with the oracle's (band cases aside)
            rec = O.pack_key_record(enc, To)
            same = np.ones(total, dtype=bool)
            for k in ("idx", "signs", "rnorm", "norm"):
                g = _np(one[k]).reshape(total, Hkv, -1)[:, h]
                same &= np.all(g.view(np.uint8) == np.ascontiguousarray(rec[k]).reshape(total, -1).view(np.uint8),
                               axis=1)
            P.check_scores(scores[s, heads, :total][:, same], s_ref[:, same])
    assert int(np.argmax(scores[0, G, :sum(chunks[0])])) == 2100
