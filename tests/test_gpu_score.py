"""GPU parity of the candidate scoring head (hstu_score) against the CPU oracle.

Head alone, on the same candidate rows: the kernel and the oracle's bfloat16 mirror round
the hidden activations at the same points, so what remains is float32 against float64
accumulation and the rounding flips it causes: a hidden value within the float32 sum's
error of a rounding midpoint goes to the neighbouring bfloat16 value on one side only,
one unit (at most 2^-7 of its size) apart, and moves the next layer's sums by that unit
times a weight. Float32 sums flip about one hidden value in 20 000 (5e-5 of the first
layer's values on N(0, 1) rows); the largest effect on a probability seen over 32 768
encoder-output rows was 9.6e-4, and the bar is 4e-3.
float32 against float64: 1e-5.
Encoder plus head: the encoder's outputs carry its own error (normwise <= 2e-2); the head's
layers have gains near one and the sigmoid's slope is at most 1/4, so probabilities are
held to 2e-2."""
import numpy as np
import pytest

import hstu_silu_attention_amd as hsa
import oracle
import workloads
from gpu_util import gpu_encode, make_model, oracle_encode, say, select_users, to_dev, torch_cuda

pytestmark = pytest.mark.gpu

HEAD_TOL = {"bf16": 4e-3, "f32": 1e-5}
END_TO_END_TOL = 2e-2


def _rows(rng, n, D, dtype):
    x = rng.standard_normal((n, D)).astype(np.float32)
    return workloads.to_bf16_values(x) if dtype == "bf16" else x


@pytest.mark.parametrize("dtype,D,widths", [
    ("bf16", 512, (512, 256, 1)),
    ("bf16", 512, (384, 128, 16)),
    ("bf16", 256, (128, 3)),
    ("bf16", 256, (2,)),
    ("bf16", 512, (512, 512, 512, 512, 256, 128, 128, 5)),
    ("f32", 128, (256, 128, 1)),
    ("f32", 64, (4,)),
])
@pytest.mark.parametrize("rows", [1000, 64, 1, 0])
def test_score_head_parity(dtype, D, widths, rows):
    torch = torch_cuda()
    say(f"score {dtype} D={D} head={widths} rows={rows}")
    wl = workloads.make_custom(seed=301 + len(widths), dtype=dtype, layers=1, d_model=D, heads=D // 128 if dtype == "bf16" else 2,
                               max_len=8, uih_lengths=[0], cand_lengths=[0], head=widths)
    x = _rows(np.random.default_rng(rows + D), rows, D, dtype)
    model = make_model(torch, wl)
    head = hsa.ScoringHead(wl.head, dtype=dtype)
    prob = hsa.score(model, head, to_dev(torch, x, dtype))
    torch.cuda.synchronize()
    got = prob.cpu().numpy().astype(np.float64)
    want = oracle.score_head(x, wl.head, bf16=(dtype == "bf16"))
    assert got.shape == want.shape == (rows, widths[-1])
    if rows:
        err = float(np.max(np.abs(got - want)))
        say(f"  max |dp| = {err:.3e} (tol {HEAD_TOL[dtype]}); p in [{want.min():.3f}, {want.max():.3f}]")
        assert err <= HEAD_TOL[dtype]


def test_score_writes_only_its_rows():
    """A guard region after the output keeps its bits (ragged last block of 64 rows)."""
    torch = torch_cuda()
    wl = workloads.make_custom(seed=5, dtype="bf16", layers=1, d_model=256, heads=2, max_len=8,
                               uih_lengths=[0], cand_lengths=[0], head=(128, 2))
    x = _rows(np.random.default_rng(9), 70, 256, "bf16")
    model = make_model(torch, wl)
    head = hsa.ScoringHead(wl.head, dtype="bf16")
    buf = torch.full((80, 2), -3.0, dtype=torch.float32, device="cuda")
    hsa.score(model, head, to_dev(torch, x, "bf16"), out=buf[:70])
    torch.cuda.synchronize()
    assert bool((buf[70:] == -3.0).all().item())
    want = oracle.score_head(x, wl.head, bf16=True)
    assert float(np.max(np.abs(buf[:70].cpu().numpy() - want))) <= HEAD_TOL["bf16"]


def test_encode_then_score():
    """The whole prediction on a ragged batch: hstu_encode, then hstu_score on its candidate
    outputs, against the oracle's encoder and head."""
    torch = torch_cuda()
    wl = workloads.make_custom(seed=307, dtype="bf16", layers=2, d_model=256, heads=2, max_len=600,
                               uih_lengths=[400, 0, 77], cand_lengths=[50, 9, 130], head=(256, 128, 2))
    model = make_model(torch, wl)
    _, dc = gpu_encode(wl, model=model, keep_device=True)
    head = hsa.ScoringHead(wl.head, dtype="bf16")
    got = hsa.score(model, head, dc).cpu().numpy().astype(np.float64)
    _, rc, _ = oracle_encode(wl, "bf16")
    want = oracle.score_head(rc, wl.head, bf16=True)
    err = float(np.max(np.abs(got - want)))
    say(f"  encode+score max |dp| = {err:.3e} (tol {END_TO_END_TOL})")
    assert err <= END_TO_END_TOL


def test_everything_together():
    """The features composed: both position tables, interleaved context/action events, a
    cached prefix filled by an earlier call, then the scoring head on the candidates;
    the oracle does the same steps."""
    torch = torch_cuda()
    D, H, L = 256, 2, 2
    wl = workloads.make_custom(seed=611, dtype="bf16", layers=L, d_model=D, heads=H, max_len=500,
                               uih_lengths=[30, 0, 55], cand_lengths=[12, 4, 20], cached_lengths=[60, 25, 0],
                               position="both", rel_std=0.3, packing="interleave", head=(256, 128, 3))
    B = wl.users
    model = make_model(torch, wl)
    cache = hsa.KVCache(model, slots=4, capacity=300)
    cache.slot_of_user = np.array([3, 1, 0], dtype=np.int32)
    cache.cached_len = np.zeros(B, dtype=np.int32)
    empty = np.zeros((0, D), np.float32)
    po = workloads.lengths_to_offsets(wl.cached_lengths)
    ptok, pto = hsa.pack_uih(model, to_dev(torch, wl.prefix, "bf16"), to_dev(torch, wl.prefix_action, "bf16"), po,
                             "interleave")
    pl = np.diff(pto.astype(np.int64))
    gpu_encode(wl, model=model, uih=ptok, uih_lengths=pl, cand=empty, cand_lengths=np.zeros(B, np.int64), cache=cache)
    eo = workloads.lengths_to_offsets(wl.uih_lengths)
    tok, to = hsa.pack_uih(model, to_dev(torch, wl.uih, "bf16"), to_dev(torch, wl.action, "bf16"), eo, "interleave")
    tl = np.diff(to.astype(np.int64))
    _, dc = gpu_encode(wl, model=model, uih=tok, uih_lengths=tl, cache=cache, keep_device=True)
    head = hsa.ScoringHead(wl.head, dtype="bf16")
    got = hsa.score(model, head, dc).cpu().numpy().astype(np.float64)
    assert cache.cached_len.tolist() == (2 * (wl.cached_lengths + wl.uih_lengths)).tolist()

    ocache = oracle.OracleCache(np.zeros((L, 4, 300, D)), np.zeros((L, 4, 300, D)),
                                cache.slot_of_user.astype(np.int64), np.zeros(B, np.int64))
    rpt, _ = oracle.pack_uih(wl.prefix, wl.prefix_action, po, "interleave", bf16=True)
    _, _, ocache = oracle_encode(wl, "bf16", cache=ocache, uih=rpt, uih_lengths=pl, cand=empty,
                                 cand_lengths=np.zeros(B, np.int64))
    rt, _ = oracle.pack_uih(wl.uih, wl.action, eo, "interleave", bf16=True)
    _, rc, _ = oracle_encode(wl, "bf16", cache=ocache, uih=rt, uih_lengths=tl)
    want = oracle.score_head(rc, wl.head, bf16=True)
    err = float(np.max(np.abs(got - want)))
    say(f"  everything together: max |dp| = {err:.3e} (tol {END_TO_END_TOL})")
    assert err <= END_TO_END_TOL
