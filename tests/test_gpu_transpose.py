"""GPU: hstu_transpose_weights moves weights from the layout the method writes them in
(W1 [D][4D], W2 [3D][D]) to the one hstu_encode reads, bit for bit; an encoder built from
math-layout weights through it gives the same outputs as one built from the transposes
made on the host; and hstu_encode given the math layout itself (HSTU_WEIGHTS_MATH, the
transposes made in its workspace on every call) gives the same outputs and cache rows
as with the prepared layout, through both entry points."""
import numpy as np
import pytest

import hstu_silu_attention_amd as hsa
import workloads
from gpu_util import gpu_encode, make_model, say, to_dev, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,cols", [(512, 2048), (1536, 512), (130, 70), (1, 5), (64, 64), (3, 1000)])
def test_transpose_bit_exact(dtype, rows, cols):
    torch = torch_cuda()
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = torch.Generator(device="cpu").manual_seed(rows * 7919 + cols)
    w = torch.randn((rows, cols), generator=g, dtype=torch.float32).to(dtype=tdt).cuda()
    out = hsa.transpose_weights(w)
    torch.cuda.synchronize()
    want = w.t().contiguous()
    bits = torch.int16 if dtype == "bf16" else torch.int32
    assert out.shape == (cols, rows)
    assert torch.equal(out.view(bits).cpu(), want.view(bits).cpu())


def test_encoder_from_math_layout_weights():
    """W1 [D][4D] and W2 [3D][D] on the device, transposed by the library, then encode: the
    outputs equal those of the same model whose transposed weights came from the host."""
    torch = torch_cuda()
    wl = workloads.make_custom(seed=4242, dtype="bf16", layers=2, d_model=256, heads=4, max_len=600,
                               uih_lengths=[300, 0, 129], cand_lengths=[64, 5, 0])
    model = make_model(torch, wl)
    ref_u, ref_c = gpu_encode(wl, model=model)
    for w_uvqk, w_out, _, _ in model.layers:   # the model's device weights, in the layout encode reads
        w1 = w_uvqk.t().contiguous()            # back to the math layout, on the device
        w2 = w_out.t().contiguous()
        w_uvqk.zero_()
        w_out.zero_()
        hsa.transpose_weights(w1, out=w_uvqk)   # in place: the model's weight pointers stay valid
        hsa.transpose_weights(w2, out=w_out)
    torch.cuda.synchronize()
    gu, gc = gpu_encode(wl, model=model)
    say(f"  encoder from transposed weights: max |diff| {np.max(np.abs(gu - ref_u)) if gu.size else 0}")
    assert np.array_equal(gu, ref_u) and np.array_equal(gc, ref_c)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_encode_with_math_layout_weights(dtype):
    torch = torch_cuda()
    wl = workloads.make_custom(seed=4343, dtype=dtype, layers=3, d_model=256, heads=4, max_len=900,
                               uih_lengths=[300, 0, 129, 64], cand_lengths=[64, 5, 0, 200],
                               cached_lengths=[100, 40, 0, 7], position="both")
    prepared = make_model(torch, wl)
    math = hsa.Model(wl.params, d_model=wl.d_model, heads=wl.heads, max_len=wl.max_len, dtype=dtype,
                     device=torch.device("cuda:0"), weight_layout="math")
    assert math.dims().weight_layout == hsa.HSTU_WEIGHTS_MATH
    B, cap = wl.users, int((wl.cached_lengths + wl.uih_lengths).max())
    empty = np.zeros((0, wl.d_model), np.float32)
    outs = []
    for model in (prepared, math):
        cache = hsa.KVCache(model, slots=B, capacity=cap)
        cache.cached_len = np.zeros(B, dtype=np.int32)
        gpu_encode(wl, model=model, uih=wl.prefix, cand=empty, uih_lengths=wl.cached_lengths,
                   cand_lengths=np.zeros(B, np.int64), cache=cache)
        gu, gc = gpu_encode(wl, model=model, cache=cache)
        torch.cuda.synchronize()
        outs.append((gu, gc, cache.k.float().cpu().numpy(), cache.v.float().cpu().numpy()))
    for a, b in zip(*outs):
        assert np.array_equal(a, b)
    say(f"  {dtype}: math-layout weights give the prepared layout's outputs and cache rows bit for bit")
    # the allocation-free entry point takes the same path
    if dtype == "bf16":
        bf = lambda a: to_dev(torch, a.reshape(-1, wl.d_model), "bf16")
        uo, co = workloads.lengths_to_offsets(wl.uih_lengths), workloads.lengths_to_offsets(wl.cand_lengths)
        ref = hsa.encode(prepared, bf(wl.uih), uo, bf(wl.cand), co)
        got = hsa.encode_static(math, bf(wl.uih), uo, bf(wl.cand), co)
        torch.cuda.synchronize()
        assert torch.equal(ref[0], got[0]) and torch.equal(ref[1], got[1])
