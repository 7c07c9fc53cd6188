"""GPU parity of the history packing step (hstu_pack_uih) and of the encoder on packed
histories, against the CPU oracle.

The packing itself is compared bit for bit: interleaving moves bytes, and the merged
form's float32 sum of two stored values, rounded once, equals the oracle's exact sum
rounded once (the float32 sum of two bfloat16 values is exact unless their exponents
differ by more than 16, and then both roundings give the larger value; likewise for
float32 values against float64). The encoder on packed histories is held to the
encoder's tolerances: normwise error <= 2e-2 (bfloat16) per user and output tensor."""
import numpy as np
import pytest

import hstu_silu_attention_amd as hsa
import oracle
import workloads
from gpu_util import BF16_TOL, gpu_encode, make_model, normwise_per_user, oracle_encode, say, to_dev, to_np, torch_cuda

pytestmark = pytest.mark.gpu


def _model(torch, dtype, D, H=2):
    wl = workloads.make_custom(seed=1, dtype=dtype, layers=1, d_model=D, heads=H, max_len=8,
                               uih_lengths=[0], cand_lengths=[0])
    return make_model(torch, wl)


def _embeddings(rng, E, D, dtype, spread):
    """N(0, 1) values, some scaled by 2^k with k in [-spread, spread], so that the merged
    form meets sums of very different magnitudes, exact cancellations and rounding ties."""
    x = rng.standard_normal((E, D)).astype(np.float32)
    k = rng.integers(-spread, spread + 1, size=(E, D))
    x = np.where(rng.random((E, D)) < 0.25, x * np.exp2(k).astype(np.float32), x)
    return workloads.to_bf16_values(x) if dtype == "bf16" else x


@pytest.mark.parametrize("mode", ["sum", "interleave"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("lengths", [[1000, 0, 333, 1], [1], [0, 0]])
def test_pack_bit_exact(dtype, mode, lengths):
    torch = torch_cuda()
    D = 256 if dtype == "bf16" else 128
    say(f"pack {dtype} {mode} lengths={lengths}")
    rng = np.random.default_rng(7 + len(lengths))
    E = int(sum(lengths))
    ctx = _embeddings(rng, E, D, dtype, 40 if dtype == "bf16" else 60)
    act = _embeddings(rng, E, D, dtype, 40 if dtype == "bf16" else 60)
    if E >= 2:
        act[0] = -ctx[0]                  # exact cancellation
        act[1] = ctx[1]                   # doubling
    model = _model(torch, dtype, D)
    eo = workloads.lengths_to_offsets(lengths)
    tok, to = hsa.pack_uih(model, to_dev(torch, ctx, dtype), to_dev(torch, act, dtype), eo, mode)
    torch.cuda.synchronize()
    ref, ro = oracle.pack_uih(ctx, act, eo, mode, bf16=(dtype == "bf16"))
    assert to.tolist() == ro.tolist()
    got = tok.float().cpu().numpy()
    want = ref.astype(np.float32)
    assert got.shape == want.shape
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_pack_leaves_rows_past_the_output_alone():
    """The launch writes exactly the output rows: a guard region after them keeps its bits."""
    torch = torch_cuda()
    D, E = 256, 77
    rng = np.random.default_rng(3)
    ctx, act = (_embeddings(rng, E, D, "bf16", 4) for _ in range(2))
    model = _model(torch, "bf16", D)
    buf = torch.full((2 * E + 16, D), 7.0, dtype=torch.bfloat16, device="cuda")
    hsa.pack_uih(model, to_dev(torch, ctx, "bf16"), to_dev(torch, act, "bf16"), [0, E], "interleave",
                 out=buf[:2 * E])
    torch.cuda.synchronize()
    assert bool((buf[2 * E:] == 7.0).all().item())
    ref, _ = oracle.pack_uih(ctx, act, [0, E], "interleave")
    assert np.array_equal(buf[:2 * E].float().cpu().numpy(), ref.astype(np.float32))


def _gpu_packed(torch, model, wl, *, prefix=False):
    lengths = wl.cached_lengths if prefix else wl.uih_lengths
    ctx, act = (wl.prefix, wl.prefix_action) if prefix else (wl.uih, wl.action)
    return hsa.pack_uih(model, to_dev(torch, ctx, wl.dtype), to_dev(torch, act, wl.dtype),
                        workloads.lengths_to_offsets(lengths), wl.packing)


@pytest.mark.parametrize("packing", ["interleave", "sum"])
@pytest.mark.parametrize("D,H", [(256, 4), (512, 4)])
def test_packed_history_encode(packing, D, H):
    """Pack on the GPU, encode on the GPU; the oracle packs and encodes the same events."""
    torch = torch_cuda()
    say(f"packed encode {packing} D={D} H={H}")
    wl = workloads.make_custom(seed=211, dtype="bf16", layers=2, d_model=D, heads=H, max_len=700,
                               uih_lengths=[300, 0, 57, 129], cand_lengths=[33, 8, 0, 64], packing=packing)
    model = make_model(torch, wl)
    tok, to = _gpu_packed(torch, model, wl)
    tl = np.diff(to.astype(np.int64))
    gu, gc = gpu_encode(wl, model=model, uih=tok, uih_lengths=tl)
    rtok, roff = oracle.pack_uih(wl.uih, wl.action, workloads.lengths_to_offsets(wl.uih_lengths), packing,
                                 bf16=True)
    assert roff.tolist() == to.tolist()
    ru, rc, _ = oracle_encode(wl, "bf16", uih=rtok, uih_lengths=tl)
    eu = normwise_per_user(gu, ru, tl)
    ec = normwise_per_user(gc, rc, wl.cand_lengths)
    say(f"  normwise err uih={eu:.3e} cand={ec:.3e}")
    assert eu <= BF16_TOL and ec <= BF16_TOL


@pytest.mark.parametrize("packing", ["interleave", "sum"])
def test_packed_streaming(packing):
    """Packed prefix events into the cache, then packed new events plus candidates against it,
    compared with the oracle doing the same."""
    torch = torch_cuda()
    say(f"packed streaming {packing}")
    D, H, L = 256, 2, 2
    wl = workloads.make_custom(seed=223, dtype="bf16", layers=L, d_model=D, heads=H, max_len=900,
                               uih_lengths=[40, 0, 65], cand_lengths=[9, 3, 17], cached_lengths=[100, 17, 0],
                               packing=packing)
    B = wl.users
    f = 2 if packing == "interleave" else 1
    model = make_model(torch, wl)
    cache = hsa.KVCache(model, slots=4, capacity=400)
    cache.slot_of_user = np.array([2, 0, 3], dtype=np.int32)
    cache.cached_len = np.zeros(B, dtype=np.int32)
    empty = np.zeros((0, D), np.float32)
    ptok, po = _gpu_packed(torch, model, wl, prefix=True)
    pl = np.diff(po.astype(np.int64))
    gpu_encode(wl, model=model, uih=ptok, uih_lengths=pl, cand=empty, cand_lengths=np.zeros(B, np.int64),
               cache=cache)
    tok, to = _gpu_packed(torch, model, wl)
    tl = np.diff(to.astype(np.int64))
    gu, gc = gpu_encode(wl, model=model, uih=tok, uih_lengths=tl, cache=cache)
    assert cache.cached_len.tolist() == (f * (wl.cached_lengths + wl.uih_lengths)).tolist()

    ocache = oracle.OracleCache(np.zeros((L, 4, 400, D)), np.zeros((L, 4, 400, D)),
                                cache.slot_of_user.astype(np.int64), np.zeros(B, np.int64))
    rpt, _ = oracle.pack_uih(wl.prefix, wl.prefix_action, workloads.lengths_to_offsets(wl.cached_lengths),
                             packing, bf16=True)
    _, _, ocache = oracle_encode(wl, "bf16", cache=ocache, uih=rpt, uih_lengths=pl, cand=empty,
                                 cand_lengths=np.zeros(B, np.int64))
    rt, _ = oracle.pack_uih(wl.uih, wl.action, workloads.lengths_to_offsets(wl.uih_lengths), packing, bf16=True)
    ru, rc, _ = oracle_encode(wl, "bf16", cache=ocache, uih=rt, uih_lengths=tl)
    eu = normwise_per_user(gu, ru, tl)
    ec = normwise_per_user(gc, rc, wl.cand_lengths)
    say(f"  normwise err uih={eu:.3e} cand={ec:.3e}")
    assert eu <= BF16_TOL and ec <= BF16_TOL
