"""GPU: a selected index outside 0..context-1 is reported, not silently clamped.

A caller that passes a corrupt selection (for example the idx of a hit unit
overwritten by other code) to the gather or to attention over persistent heads
gets CLO_E_INDEX in its sync error word; the kernel reads the nearest row in
range instead, so no access leaves the unit's rows, and every kernel finishes.
In-range indices give exactly the rows they name; a call without an error
word reports nothing and still finishes.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

D = 128


def _bf16_bits(t):
    import torch

    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("host_format", [0, 1, 2])
def test_gather_reports_out_of_range_index(need_gpu, host_format):
    import torch

    from top_sparse_attention_02_amd import clo
    from top_sparse_attention_02_amd.hip_host import HostBuffer

    print(f"bad-index gather case host_format={host_format}", flush=True)
    rng = np.random.default_rng(7 + host_format)
    B, hkv, N, k = 2, 2, 1000, 300
    shape = clo.Shape(B, hkv, hkv, N, k, 0.8, clo.CLO_BF16)
    idx = np.stack([np.sort(rng.choice(N, size=k, replace=False)) for _ in range(B * hkv)]).reshape(B, hkv, k)
    idx = idx.astype(np.int32)
    good = idx.copy()
    idx[0, 1, 5] = N          # one past the end
    idx[1, 0, 260] = -3       # negative, in the second 256-row item
    idx[1, 1, 0] = 1 << 30    # far past the end
    idx_d = torch.from_numpy(idx).cuda()
    k_cache = torch.zeros(B, hkv, k, D, dtype=torch.bfloat16, device="cuda")
    v_cache = torch.zeros_like(k_cache)
    ws = torch.empty(clo.clo_workspace_size(shape), dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    bufs = []
    if host_format == 0:
        kh_buf, vh_buf = HostBuffer(B * hkv * N * D * 2), HostBuffer(B * hkv * N * D * 2)
        bufs = [kh_buf, vh_buf]
        kh = kh_buf.numpy("u2", (B, hkv, N, D))
        vh = vh_buf.numpy("u2", (B, hkv, N, D))
        kh[:] = rng.integers(0, 1 << 16, size=kh.shape, dtype=np.uint16)
        vh[:] = rng.integers(0, 1 << 16, size=vh.shape, dtype=np.uint16)
        layer = clo.Layer(0, None, None, kh_buf.ptr, vh_buf.ptr, None, k_cache, v_cache, idx_d)
    else:
        # quantized records: K values then V values per token (int8: one byte per
        # value; int4: value 2j in the low half of byte j)
        rb = D if host_format == 1 else D // 2
        rec = HostBuffer(B * hkv * N * 2 * rb)
        bufs = [rec]
        lim = 127 if host_format == 1 else 7
        vals = rng.integers(-lim, lim + 1, size=(B, hkv, N, 2, D))
        r = rec.numpy("u1", (B, hkv, N, 2, rb))
        if host_format == 1:
            r[:] = vals.astype(np.int8).view(np.uint8)
        else:
            r[:] = ((vals[..., 0::2] & 0xF) | ((vals[..., 1::2] & 0xF) << 4)).astype(np.uint8)
        k_exp = torch.from_numpy(rng.integers(-10, 2, size=(B, hkv, N), dtype=np.int8)).cuda()
        v_exp = torch.from_numpy(rng.integers(-10, 2, size=(B, hkv, N), dtype=np.int8)).cuda()
        layer = clo.Layer(0, None, None, rec.ptr, None, None, k_cache, v_cache, idx_d, host_format, k_exp, v_exp)
    # no error word: the call finishes and reports nothing
    clo.clo_gather_kv(shape, layer, None, ws)
    torch.cuda.synchronize()
    # with an error word: CLO_E_INDEX, and every in-range row copied as named
    clo.clo_gather_kv(shape, layer, None, ws, sync=clo.Sync(error_word=err))
    torch.cuda.synchronize()
    assert int(err.item()) == clo.CLO_E_INDEX
    clamped = np.clip(idx.astype(np.int64), 0, N - 1)
    gk, gv = _bf16_bits(k_cache), _bf16_bits(v_cache)
    for b in range(B):
        for h in range(hkv):
            if host_format == 0:
                assert np.array_equal(gk[b, h], kh[b, h, clamped[b, h]])
                assert np.array_equal(gv[b, h], vh[b, h, clamped[b, h]])
            else:
                ke = k_exp.cpu().numpy()[b, h, clamped[b, h]].astype(np.float64)
                want = vals[b, h, clamped[b, h], 0].astype(np.float64) * 2.0 ** ke[:, None]
                got = (gk[b, h].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
                assert np.array_equal(got, want)
    # a valid selection leaves a cleared word at zero
    err.zero_()
    idx_d.copy_(torch.from_numpy(good))
    clo.clo_gather_kv(shape, layer, None, ws, sync=clo.Sync(error_word=err))
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    for buf in bufs:
        buf.close()


def test_attention_over_persistent_heads_reports_out_of_range_index(need_gpu):
    import torch

    from top_sparse_attention_02_amd import clo

    print("bad-index attention case", flush=True)
    rng = np.random.default_rng(11)
    B, hq, hkv, N, k = 1, 8, 2, 700, 70
    shape = clo.Shape(B, hq, hkv, N, k, 0.8, clo.CLO_BF16)
    k_hbm = torch.randn(B, hkv, N, D, device="cuda").to(torch.bfloat16)
    v_hbm = torch.randn(B, hkv, N, D, device="cuda").to(torch.bfloat16)
    q = torch.randn(B, hq, D, device="cuda").to(torch.bfloat16)
    out = torch.zeros_like(q)
    idx = np.stack([np.sort(rng.choice(N, size=k, replace=False)) for _ in range(B * hkv)]).reshape(B, hkv, k)
    idx = idx.astype(np.int32)
    idx_d = torch.from_numpy(idx).cuda()
    layer = clo.Layer(0b11, k_hbm, v_hbm, None, None, None, None, None, idx_d)
    ws = torch.empty(clo.clo_workspace_size(shape), dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    clo.clo_sparse_attn(shape, layer, q, out, ws, sync=clo.Sync(error_word=err))
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    ref = out.clone()
    bad = idx.copy()
    bad[0, 1, 3] = N + 5
    idx_d.copy_(torch.from_numpy(bad))
    clo.clo_sparse_attn(shape, layer, q, out, ws, sync=clo.Sync(error_word=err))
    torch.cuda.synchronize()
    assert int(err.item()) == clo.CLO_E_INDEX
    assert torch.isfinite(out.float()).all()
    # the unit with only valid indices is unchanged
    assert torch.equal(out[:, :4], ref[:, :4])
