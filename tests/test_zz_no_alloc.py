"""fa_fwd_splitk_static (the key-split forward that allocates nothing, its
partials in the library's fixed device array) against fa_fwd_splitk with a
caller workspace: the outputs must be identical bit for bit, on two calls in
a row (the second smaller, so stale partials of the first are still in the
array), on the same inputs through the C ABI."""
import pytest

pytestmark = pytest.mark.gpu


def _strides(t):
    import tiled_attention_04_amd as fa
    return fa.FaStrides(t.stride(0), t.stride(1), t.stride(2), t.stride(3))


def _both(b, h, sq, sk, d, causal, splits, dtype, seed):
    import torch
    import tiled_attention_04_amd as fa
    torch.manual_seed(seed)
    tdt = {fa.FA_DTYPE_BF16: torch.bfloat16, fa.FA_DTYPE_F16: torch.float16}[dtype]
    q = torch.randn(b, h, sq, d, device="cuda").to(tdt)
    k = torch.randn(b, h, sk, d, device="cuda").to(tdt)
    v = torch.randn(b, h, sk, d, device="cuda").to(tdt)
    scale = d ** -0.5
    stream = torch.cuda.current_stream().cuda_stream
    if splits == 0:  # the library's choice, given to both calls explicitly
        splits = fa.fa_fwd_splitk_choose(b, h, sq, sk, d, causal)
        assert splits > 1
    # reference: the same key split through a caller workspace
    o_ref = torch.empty_like(q)
    l_ref = torch.empty(b, h, sq, device="cuda", dtype=torch.float32)
    need = fa.fa_fwd_splitk_workspace(b, h, sq, d, splits)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    rc = fa.fa_fwd_splitk(q.data_ptr(), k.data_ptr(), v.data_ptr(), o_ref.data_ptr(),
                          l_ref.data_ptr(), b, h, sq, sk, d, _strides(q), _strides(k), _strides(v),
                          _strides(o_ref), scale, causal, dtype, splits, ws.data_ptr(), need, stream)
    assert rc == 0, fa.last_error()
    o = torch.full_like(q, 7.0)
    lse = torch.full((b, h, sq), 7.0, device="cuda", dtype=torch.float32)
    rc = fa.fa_fwd_splitk_static(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                 lse.data_ptr(), b, h, sq, sk, d, _strides(q), _strides(k),
                                 _strides(v), _strides(o), scale, causal, dtype, splits, stream)
    assert rc == 0, fa.last_error()
    torch.cuda.synchronize()
    assert need > 0
    assert torch.equal(o, o_ref), (o.float() - o_ref.float()).abs().max().item()
    assert torch.equal(lse, l_ref), (lse - l_ref).abs().max().item()
    return need


def test_static_scratch_matches_workspace_twice_second_smaller():
    import torch
    import tiled_attention_04_amd as fa
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.lib()
    n1 = _both(1, 16, 100, 4096, 128, False, 8, fa.FA_DTYPE_BF16, 1)  # short queries, 8 splits
    n2 = _both(1, 4, 37, 1500, 64, True, 3, fa.FA_DTYPE_F16, 2)       # smaller, ragged, causal
    assert n2 < n1 <= fa.SPLITK_STATIC_MAX_BYTES
    # the library's own choice of splits (0), then again the first shape
    _both(1, 12, 100, 4096, 64, False, 0, fa.FA_DTYPE_F16, 3)
