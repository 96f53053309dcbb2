"""tq_append_kv (keys and values of the same tokens in one launch) writes the
same bytes as tq_encode_keys followed by tq_encode_values, slot for slot,
and leaves every other record untouched."""
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

CASES = [(dict(mode="prod", bits=3), torch.bfloat16, 2),
         (dict(mode="prod", bits=4), torch.bfloat16, 4),
         (dict(mode="mse", bits=4), torch.float32, 4),
         (dict(mode="mse", bits=8), torch.float16, 2),
         (dict(mode="grouped", bits_outlier=4, bits_normal=2), torch.float16, 4),
         (dict(mode="grouped_prod", bits_outlier=3, bits_normal=2), torch.bfloat16, 2)]


def _sentinel_planes(T, v_bits, n_rec):
    kp = tq.key_planes(T, n_rec, DEV)
    vp = tq.value_planes(v_bits, n_rec, device=DEV)
    for p in list(kp.values()) + list(vp.values()):
        p.view(torch.uint8).fill_(0xA5)
    return kp, vp


@pytest.mark.parametrize("n", [1, 1000, 4096])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "%s-%s-v%d" % ("".join(str(v) for v in c[0].values()),
                                                                   str(c[1])[6:], c[2]))
def test_append_kv_equals_two_encodes(case, n):
    kw, dtype, v_bits = case
    T = tq.Tables(L.key_config(seed=13, **kw), DEV)
    scale = W.w5_col_scale() if kw["mode"].startswith("grouped") else None
    keys = torch.from_numpy(W.kv_rows(61, 1, n, scale_cols=scale)[0]).to(DEV).to(dtype)
    vals = torch.from_numpy(W.kv_rows(61, 2, n)[0]).to(DEV).to(dtype)
    n_rec = n + 37
    # scattered slots, a few of them out of range (those rows are skipped)
    slots = np.random.default_rng(n).permutation(n_rec)[:n].astype(np.int64)
    slots[::97] = -1
    if n > 1:
        slots[1] = n_rec + 5
    sl = torch.from_numpy(slots).to(DEV)
    kp_a, vp_a = _sentinel_planes(T, v_bits, n_rec)
    tq.append_kv(T, keys, vals, v_bits, kp_a, vp_a, slots=sl, n_records=n_rec)
    kp_b, vp_b = _sentinel_planes(T, v_bits, n_rec)
    tq.encode_keys(T, keys, kp_b, slots=sl, n_records=n_rec)
    tq.encode_values(vals, v_bits, planes=vp_b, slots=sl, n_records=n_rec)
    torch.cuda.synchronize()
    for k in kp_a:
        assert torch.equal(kp_a[k].view(torch.uint8), kp_b[k].view(torch.uint8)), k
    for k in vp_a:
        assert torch.equal(vp_a[k].view(torch.uint8), vp_b[k].view(torch.uint8)), k
    # rows no slot names keep the sentinel
    untouched = np.setdiff1d(np.arange(n_rec), slots[(slots >= 0) & (slots < n_rec)])
    ut = torch.from_numpy(untouched).to(DEV)
    assert bool((kp_a["idx"][ut] == 0xA5).all()) and bool((vp_a["codes"][ut] == 0xA5).all())
