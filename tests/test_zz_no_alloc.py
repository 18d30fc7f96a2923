"""The no-allocation decode entry point (kvq_decode_attn_noalloc) against
kvq_decode_attn: the same kernels on the library's static scratch instead of
a caller's workspace, so the outputs must be equal bit for bit.  Two calls in
a row, the second on a smaller input (the scratch keeps the first call's
contents), then a shape whose workspace exceeds the scratch, rejected on the
host before any launch."""
import math

import numpy as np
import pytest
import torch

from workload import WORKLOADS, scaled

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rotated_int2_kv_kvq_amd as kvq
    kvq.lib()


def _case(w):
    import sys
    import os
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from cases import fill_context, new_case, query
    case = new_case(w, keep_initial=False)
    fill_context(case)
    return case, query(case)


def test_noalloc_matches_workspace_call_twice_then_smaller():
    import rotated_int2_kv_kvq_amd as kvq
    big = scaled(WORKLOADS["qwen3_8b_b4_ctx8k"], batch=4, ctx_min=1500, ctx_max=3100)
    small = scaled(WORKLOADS["qwen3_8b_b64_ctx1k_32k_g64"], batch=3, ctx_min=1, ctx_max=400)
    for w in (big, small):
        case, q = _case(w)
        ctx = torch.from_numpy(case.ctx.astype(np.int32)).cuda()
        maxc = int(case.ctx.max())
        sm = 1.0 / math.sqrt(w.head_dim)
        ref = kvq.decode(case.pages, case.table, ctx, maxc, q, case.rot_k, case.rot_v, w.group, sm)
        got = torch.full_like(ref, float("nan"))
        kvq.decode_noalloc(case.pages, case.table, ctx, maxc, q, case.rot_k, case.rot_v, w.group,
                           sm, out=got)
        torch.cuda.synchronize()
        print(f"[noalloc] batch {w.batch} ctx {case.ctx.min()}-{maxc} group {w.group}: "
              f"workspace {kvq.decode_workspace_bytes(w.batch, w.num_q_heads, w.num_kv_heads, maxc)}"
              f" bytes of {kvq.SCRATCH_BYTES}", flush=True)
        assert torch.equal(got, ref)


def test_noalloc_rejects_a_plan_larger_than_the_scratch():
    import rotated_int2_kv_kvq_amd as kvq
    B, Hq, Hkv, maxc = 64, 32, 8, 131072
    need = kvq.decode_workspace_bytes(B, Hq, Hkv, maxc, split_pages=8)
    assert need > kvq.SCRATCH_BYTES
    pages = torch.zeros(1, Hkv, 1152, dtype=torch.uint8, device="cuda")
    table = torch.zeros(B, maxc // 16, dtype=torch.int32, device="cuda")
    ctx = torch.zeros(B, dtype=torch.int32, device="cuda")
    q = torch.zeros(B, Hq, 128, dtype=torch.bfloat16, device="cuda")
    out = torch.zeros(B, Hq, 128, device="cuda")
    rk = torch.zeros(Hkv, 128, 128, device="cuda")
    with pytest.raises(kvq.KvqError) as e:
        kvq.decode_noalloc(pages, table, ctx, maxc, q, rk, rk, 128, 0.088, out=out, split_pages=8)
    assert e.value.status == -5
    torch.cuda.synchronize()
    assert not out.any()
