"""tq_encode_keys_batched (several key sets, each with its own tables, in one
launch) writes the same bytes as one tq_encode_keys call per set."""
import numpy as np
import pytest

import tq_workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import kv_cache_quantization_encode_amd as tq  # noqa: E402
from kv_cache_quantization_encode_amd import _lib as L  # noqa: E402

DEV = "cuda"

CASES = [(dict(mode="mse", bits=4), torch.bfloat16, 3, 1000, False),
         (dict(mode="mse", bits=8), torch.bfloat16, 28, 512, False),
         (dict(mode="prod", bits=3), torch.bfloat16, 2, 4096, True),
         (dict(mode="prod", bits=4), torch.float32, 5, 333, False),
         (dict(mode="grouped", bits_outlier=4, bits_normal=2), torch.float16, 4, 1, True),
         (dict(mode="grouped_prod", bits_outlier=4, bits_normal=1), torch.bfloat16, 3, 700, True)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%s-%s-x%d-n%d" % (
    "".join(str(v) for v in c[0].values()), str(c[1])[6:], c[2], c[3]))
def test_batched_equals_per_set_encode(case):
    kw, dtype, nb, n, with_slots = case
    tables = [tq.Tables(L.key_config(seed=100 + i, **kw), DEV) for i in range(nb)]
    scale = W.w5_col_scale() if kw["mode"].startswith("grouped") else None
    keys = [torch.from_numpy(W.kv_rows(70 + i, 1, n, scale_cols=scale)[0]).to(DEV).to(dtype) for i in range(nb)]
    n_rec = n + 9
    slots = None
    if with_slots:
        slots = []
        for i in range(nb):
            sl = np.random.default_rng(i).permutation(n_rec)[:n].astype(np.int64)
            sl[::50] = -1
            slots.append(torch.from_numpy(sl).to(DEV))
    def planes():
        ps = [tq.key_planes(t, n_rec, DEV) for t in tables]
        for p in ps:
            for v in p.values():
                v.view(torch.uint8).fill_(0x5A)
        return ps
    got = tq.encode_keys_batched(tables, keys, planes(), slots=slots, n_records=n_rec)
    ref = planes()
    for i in range(nb):
        tq.encode_keys(tables[i], keys[i], ref[i], slots=None if slots is None else slots[i], n_records=n_rec)
    torch.cuda.synchronize()
    for i in range(nb):
        for k in ref[i]:
            assert torch.equal(got[i][k].view(torch.uint8), ref[i][k].view(torch.uint8)), (i, k)
