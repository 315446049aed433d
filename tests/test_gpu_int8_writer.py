"""GPU INT8 writer against the exact-rational quantiser table.

The table (tests/golden/int8_quant_cases.txt) holds per-(token, head) vectors
whose codes were derived with exact rational arithmetic, chosen where
x * fl32(1/s) or a binary64 division would give another code, plus ties.  Each
vector is placed in a token's head vector (the rest zeros, which leave max|x|
unchanged and quantise to 0), negated (rne and max|x| are symmetric), and
scaled by 2^k (exact in bf16 and fp32 while nothing is subnormal, so s scales
by 2^k and the codes stay), then written through ll_cache_append_chunk into an
INT8 cache; K rows and the transposed V tiles must hold exactly the table's
codes and scales.  An all-zero token gives s = 0, q = 0.  Scheme: the INT8
KV-cache reading of LongLive: Real-time Interactive Long Video Generation
(Abstract; §5 "Conclusion" mentions INT8 inference only).
"""

import os

import numpy as np
import pytest
import torch

from sink_short_window_amd import ll
from gpu_util import need_gpu, say

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "int8_quant_cases.txt")


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _table():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            tag, _diff, xb, sb, codes = [c.strip() for c in line.split("|")]
            bits = np.array([int(b, 16) for b in xb.split(",")], np.uint32)
            rows.append((tag, (bits << 16).view(np.float32),
                         np.array([int(sb, 16)], np.uint32).view(np.float32)[0],
                         np.array([int(c) for c in codes.split(",")], np.int64)))
    return rows


@pytest.mark.parametrize("D", [128, 64])
def test_int8_writer_reproduces_exact_rational_codes(D):
    rows = _table()
    assert any("recip" in r[0] for r in rows) and any("f64" in r[0] for r in rows)
    H, T = 3, 70                     # 70 tokens: one full 64-token tile and a ragged one
    n_blk = D // 16
    x = np.zeros((T, H, D), np.float32)
    want_q = np.zeros((T, H, D), np.int64)
    want_s = np.zeros((T, H), np.float32)
    for t in range(T):
        for h in range(H):
            u = t * H + h
            if u % 23 == 22:
                continue             # all-zero vector: s = 0, q = 0
            tag, vx, vs, vq = rows[u % len(rows)]
            sign = -1.0 if (u // len(rows)) % 2 else 1.0
            k = (-20, 0, 20)[(u // (2 * len(rows))) % 3]
            blk = (t + 3 * h) % n_blk
            x[t, h, 16 * blk:16 * blk + 16] = sign * np.ldexp(vx, k)
            want_q[t, h, 16 * blk:16 * blk + 16] = (sign * vq).astype(np.int64)
            want_s[t, h] = np.ldexp(vs, k)
    assert not (x.view(np.uint32) & 0xFFFF).any()          # every value is a bf16
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    xt = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to("cuda")
    cfg = ll.make_config(1, H, D, T, 1, 1, 2, ll.LL_BF16, ll.LL_I8)
    cache = ll.Cache(cfg, "cuda")
    try:
        say(f"int8 writer vs exact-rational table: D={D} H={H} T={T}")
        cache.append_chunk(0, xt, xt)    # chunk 0 -> sink
        cache.append_chunk(0, xt, xt)    # chunk 1 -> ring slot 0
        torch.cuda.synchronize()
        for seg in (ll.LL_SEG_SINK, ll.LL_SEG_RING):
            for which, swhich in ((ll.LL_WHICH_K, ll.LL_WHICH_KSCALE), (ll.LL_WHICH_V, ll.LL_WHICH_VSCALE)):
                q = cache.rows(0, which, seg)[:, :T, :].cpu().numpy().astype(np.int64)   # [H][T][D]
                s = cache.tensor(0, swhich, seg)[:, :T, 0].cpu().numpy()                  # [H][T]
                np.testing.assert_array_equal(q, want_q.transpose(1, 0, 2), err_msg=f"codes seg {seg} which {which}")
                assert np.array_equal(s.view(np.uint32), want_s.T.view(np.uint32)), f"scales seg {seg} which {which}"
    finally:
        cache.close()
