"""kvq_decode_attention_noalloc (no device allocation: the partials live in
the library's static scratch) against kvq_decode_attention (caller's
workspace), through the C ABI: the same kernels and plan, so the outputs
must be bitwise equal; checked on two calls in a row, the second with a
smaller input, which must not see the first call's partials."""
import numpy as np
import pytest

from omnistream import generate

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import decode_attention_kvq_amd._lib as L
    L.load()


def _run(cfg_id, kw, out_dtype):
    import decode_attention_kvq_amd as K
    import tests.kvq_harness as h
    w = generate(cfg_id, **kw)
    print(f"no-alloc decode cfg{cfg_id} {kw} lengths={w.lengths.tolist()} out={out_dtype}", flush=True)
    cfg, params, cache = h.build(w)
    q_rot = K.kvq_rotate_query(cfg, params, h.query_tensor(w))
    ref = K.kvq_decode_attention(cfg, cache, params, q_rot, out_dtype=out_dtype)
    out = torch.full(q_rot.shape, float("nan"), dtype=out_dtype, device=q_rot.device)
    K.kvq_decode_attention_noalloc(cfg, cache, params, q_rot, out)
    torch.cuda.synchronize()
    a = ref.cpu().view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32).numpy()
    b = out.cpu().view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32).numpy()
    np.testing.assert_array_equal(b, a)
    return out


def test_noalloc_decode_equals_workspace_decode_on_two_calls():
    # first call: three paged sessions (the larger partial set) ...
    _run(3, dict(batch=3, len_range=(3000, 9000)), torch.float32)
    # ... then a smaller input on the same scratch
    _run(1, dict(length=1500), torch.float32)


def test_noalloc_decode_bf16_output_and_full_80k():
    _run(2, dict(), torch.float32)
    _run(0, dict(length=700), torch.bfloat16)
