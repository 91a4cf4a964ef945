"""Routing on the GPU (top-k, bincount, offsets, stable sort by expert)
against the oracle over many seeded random problems: expert counts on both
sides of every top-k kernel instance (1 to 16 logits per lane, one or
several result slots per lane), k from 1 to E, and logit distributions with
heavy ties, signed zeros, values near the fp32 limits and subnormals.
Integer outputs bit for bit, the fp32 weights within 1e-6, and the host
count readback equal to the device counts."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402

pytestmark = pytest.mark.gpu

E_CHOICES = [1, 2, 7, 63, 64, 65, 128, 129, 256, 257, 300, 512, 513, 1000, 1024]


def _logits(rs, T, E, kind):
    x = rs.standard_normal((T, E)).astype(np.float32)
    if kind == "ties":        # few distinct values: most comparisons are ties
        x = np.floor(x * 0.7).astype(np.float32)
    elif kind == "equal":     # every expert tied: the lowest ids win
        x = np.zeros((T, E), np.float32)
    elif kind == "zeros":     # -0.0 and +0.0 compare equal
        x = np.where(rs.random_sample((T, E)) < 0.5, np.float32(-0.0), np.float32(0.0))
        x[rs.random_sample((T, E)) < 0.1] = 1.0
    elif kind == "huge":      # finite, near the fp32 limits
        x = (x * 1e37).astype(np.float32)
        x[rs.random_sample((T, E)) < 0.05] = np.float32(3.0e38)
        x[rs.random_sample((T, E)) < 0.05] = np.float32(-3.0e38)
    elif kind == "subnormal":
        x = (x * np.float32(1e-40)).astype(np.float32)
    return np.ascontiguousarray(x, dtype=np.float32)


def _cases(n=120, seed=20261205):
    rs = np.random.RandomState(seed)
    kinds = ["normal", "ties", "equal", "zeros", "huge", "subnormal"]
    out = []
    for i in range(n):
        E = int(rs.choice(E_CHOICES))
        k = int(rs.choice([1, 2, 4, 8, min(E, 64), min(E, 65), E, int(rs.randint(1, E + 1))]))
        k = max(1, min(k, E))
        T = int(rs.choice([1, 2, 31, 32, 33, int(rs.randint(1, 3000))]))
        out.append((i, T, E, k, kinds[i % len(kinds)]))
    return out


CASES = _cases()


def test_routing_fuzz_against_oracle():
    import moe_layer_lora_amd as moe
    dev = torch.device("cuda")
    rs = np.random.RandomState(5)
    for i, T, E, k, kind in CASES:
        tag = f"case {i}: T={T} E={E} k={k} {kind}"
        print(f"[route fuzz] {tag}", flush=True)
        logits = _logits(rs, T, E, kind)
        pb = moe.Problem(T, 8, E, k, 8, 8, 2.0, moe.MOE_BF16)
        rt = moe.alloc_routing(pb, dev)
        ws = moe.alloc_bytes(moe.route_workspace(pb), dev)
        hc = np.full(E, -1, np.int32)
        moe.moe_route(pb, torch.from_numpy(logits).to(dev), rt, host_counts=hc, ws=ws)
        torch.cuda.synchronize()
        got = {n: v.cpu().numpy() for n, v in rt.items()}
        want = oracle.route(logits, k)
        for n in ("topk_idx", "counts", "offsets", "sorted_slot", "slot_row"):
            assert np.array_equal(got[n], want[n]), f"{tag}: {n} differs"
        assert np.array_equal(hc, want["counts"]), f"{tag}: host counts differ"
        w, ww = got["topk_w"].astype(np.float64), np.asarray(want["topk_w"], np.float64)
        assert np.linalg.norm(w - ww) <= 1e-6 * max(np.linalg.norm(ww), 1e-30), f"{tag}: topk_w"
