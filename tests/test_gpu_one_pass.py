"""The one-pass decode step: against the oracle on every row, and against the two-kernel
form bit for bit.

Token-level rows that one fused workgroup handles alone (a single split and head
chunk: at least 256 row-chunks) are decoded by one kernel that scores each row from
its label rows itself.  Every case first asserts that the shape takes that path
(ds_decode_is_one_pass).  Every row of the one-call result is then checked against
the float64 oracle on float64 copies of the same inputs: kept set by the index rule
(boundary ties within 1e-6 relative of the oracle's k-th score), index slots past a
short sequence's kept count -1, and output within 2e-3 (bf16) or 1e-5 (fp32) of the
oracle's attention over the kept set.  The two phase calls still run the score kernel
and then the fused kernel from the stored scores; both accumulate each score the same
way, so on the same inputs the one-call step must give the same indices, outputs and
rebuilt label rows as the two phases, bit for bit.  The cases cover both label-row
widths (16 and 32 bytes) in both element types and 64-byte fp32 rows, groups of 1, 2 and 4 query heads,
every per-thread item count of the fused kernel, rows rebuilt from K, and ragged
batches.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import long_context_sparse_ds_amd as L
from _helpers import check_row

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    L.lib()   # raises if the HIP library is missing


def _say(msg):
    print(f"[case] {msg}", flush=True)


# (name, dtype, B, Hq, Hkv, T, r, k, rows rebuilt, ragged); one split per row (B * Hkv >= 256 rows, or
# k <= 64), groups <= 4 heads
CASES = [
    ("bf16_r8_items32", "bf16", 64, 4, 4, 20000, 8, 700, 3, False),
    ("bf16_r16_g4_items16", "bf16", 64, 16, 4, 9000, 16, 300, 1, False),
    ("bf16_r16_g2_items4", "bf16", 128, 4, 2, 3000, 16, 120, 40, False),
    ("f32_r4_items8", "f32", 128, 2, 2, 5000, 4, 200, 2, False),
    ("f32_r8_items4", "f32", 256, 1, 1, 3000, 8, 100, 1, False),
    # 16-byte rows with fewer passes (4) than a batch of label requests (8)
    ("bf16_r8_items4", "bf16", 128, 2, 2, 3000, 8, 100, 2, False),
    ("f32_r4_items4", "f32", 256, 1, 1, 2000, 4, 64, 1, False),
    # edge shapes: rows of 5 tokens with 3 of them rebuilt, and every token kept (k = T)
    ("bf16_r8_T5", "bf16", 64, 4, 4, 5, 8, 3, 3, False),
    ("f32_r4_dense", "f32", 256, 1, 1, 40, 4, 40, 1, False),
    # 64-byte label rows (fp32, r = 16), and the single tiny row whose 64 kept tokens make one split
    ("f32_r16_items4", "f32", 256, 1, 1, 3000, 16, 100, 1, False),
    ("f32_r16_g2_items8", "f32", 128, 4, 2, 6000, 16, 200, 2, False),
    ("f32_r16_one_row", "f32", 1, 1, 1, 1024, 16, 64, 1, False),
    # short rows: a group of 4, 16-byte rows at T < 1024, a ragged fp32 batch
    ("bf16_r8_small_g4", "bf16", 64, 16, 4, 1000, 8, 60, 2, False),
    ("bf16_r16_small", "bf16", 256, 1, 1, 777, 16, 50, 1, False),
    ("f32_r4_small_ragged", "f32", 256, 2, 2, 1024, 4, 64, 1, True),
    ("f32_r16_ragged", "f32", 256, 2, 2, 4000, 16, 150, 1, True),
    ("bf16_r8_ragged", "bf16", 64, 4, 4, 12000, 8, 400, 2, True),
    ("bf16_r16_ragged_g2", "bf16", 128, 4, 2, 6000, 16, 250, 1, True),
]


def _inputs(dt, B, Hq, Hkv, T, r, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    q = torch.randn((B, Hq, 128), generator=g, device="cuda").to(tdt)
    K = torch.randn((B, Hkv, T, 128), generator=g, device="cuda").to(tdt)
    V = torch.randn((B, Hkv, T, 128), generator=g, device="cuda").to(tdt)
    ch = torch.stack([torch.randperm(128, generator=g, device="cuda")[:r].sort().values for _ in range(Hkv)])
    ch = ch.to(torch.int32).contiguous()
    return q, K, V, ch


def _check_against_oracle(dt, q, K, V, ch, lens, k, out, idx, name):
    """Every (sequence, KV head) row of the one-call result against the oracle, on float64 copies
    of the device inputs: row b keeps min(k, lens[b]) tokens of its first lens[b]."""
    B, Hkv = K.shape[0], K.shape[1]
    G = q.shape[1] // Hkv
    qh, Kh, Vh = (t.float().cpu().numpy() for t in (q, K, V))
    chh, outh, idxh = ch.cpu().numpy(), out.cpu().numpy(), idx.cpu().numpy()

    def row(u):
        b, g = divmod(u, Hkv)
        Tb = int(lens[b])
        return check_row(qh[b, g * G:(g + 1) * G].astype(np.float64), Kh[b, g, :Tb].astype(np.float64),
                         Vh[b, g, :Tb].astype(np.float64), chh[g], min(k, Tb), 1, Tb,
                         outh[b, g * G:(g + 1) * G], idxh[b, g], dt, f"{name} row ({b},{g})")

    n = max(1, min(16, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(n) as ex:
        res = list(ex.map(row, range(B * Hkv)))
    return sum(r[0] for r in res), max(r[1] for r in res)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_one_pass_matches_two_kernels(case):
    name, dt, B, Hq, Hkv, T, r, k, n_new, ragged = case
    _say(f"{name}: B={B} Hq={Hq} Hkv={Hkv} T={T} r={r} k={k} rebuilt={n_new} ragged={ragged}")
    q, K, V, ch = _inputs(dt, B, Hq, Hkv, T, r, seed=sum(map(ord, name)))
    assert L.ds_decode_is_one_pass(B, Hq, Hkv, 128, T, 1, k, r, dt), f"{name}: not a one-pass shape"
    label = L.ds_build_label_cache(K, ch)
    torch.cuda.synchronize()
    raw = label.view(torch.int16) if dt == "bf16" else label.view(torch.int32)
    ws1 = L.alloc_workspace(B, Hq, Hkv, 128, T, 1, k)
    ws2 = L.alloc_workspace(B, Hq, Hkv, 128, T, 1, k)
    if ragged:
        g = torch.Generator().manual_seed(7)
        lens = torch.randint(1, T + 1, (B,), generator=g, dtype=torch.int32)
        lens[0], lens[1] = T, 1
        seq = lens.cuda()
        lab1, lab2 = label.clone(), label.clone()
        for b in range(B):   # garbage where each sequence's rows are rebuilt
            t0 = max(int(lens[b]) - n_new, 0)
            for lab in (lab1, lab2):
                (lab.view(torch.int16) if dt == "bf16" else lab.view(torch.int32))[b, :, t0:int(lens[b])].fill_(0x3F00)
        o1, i1 = L.ds_decode_sparse_attn_ragged(q, K, V, lab1, ch, seq, T, k, n_append=n_new, workspace=ws1)
        L.ds_decode_score_ragged(q, K, lab2, ch, seq, T, k, n_append=n_new, workspace=ws2)
        o2, i2 = L.ds_decode_select_attend_ragged(q, K, V, seq, T, k, ws2)
    else:
        raw[:, :, T - n_new:T].fill_(0x3F00)   # garbage in the rows to be rebuilt
        lab1, lab2 = label.clone(), label.clone()
        o1, i1 = L.ds_decode_sparse_attn(q, K, V, lab1, ch, T, k, workspace=ws1, t_append=T - n_new)
        L.ds_decode_score(q, K, lab2, ch, T, k, workspace=ws2, t_append=T - n_new)
        o2, i2 = L.ds_decode_select_attend(q, K, V, T, k, ws2)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2), f"{name}: indices differ in {(i1 != i2).sum().item()} slots"
    assert torch.equal(o1.view(torch.int32), o2.view(torch.int32)), f"{name}: outputs differ"
    assert torch.equal(lab1.view(torch.uint8), lab2.view(torch.uint8)), f"{name}: rebuilt label rows differ"
    want = L.ds_build_label_cache(K, ch)   # the rebuilt rows are K's channels
    torch.cuda.synchronize()
    if not ragged:
        assert torch.equal(lab1.view(torch.uint8), want.view(torch.uint8))
    ii = i1.view(-1, k)
    valid = ii >= 0   # index slots past a short sequence's kept count are -1
    assert valid[:, 0].all() and ((ii[:, 1:] > ii[:, :-1]) | ~valid[:, 1:]).all()
    lens_h = lens.tolist() if ragged else [T] * B
    swaps, err = _check_against_oracle(dt, q, K, V, ch, lens_h, k, o1, i1, name)
    _say(f"{name}: identical to the two phases; every row matches the oracle "
         f"(tie swaps {swaps}, max-abs err {err:.3g}); first row kept {int(valid[0].sum())}")
    del q, K, V, label, lab1, lab2, ws1, ws2
    torch.cuda.empty_cache()
