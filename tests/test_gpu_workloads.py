"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times, on rows the oracle evaluates one by one.

Rows: the chunk-geometry landmarks {0, 1, s-1, s, s+w-1, s+w, 2s-1, 2s,
2s+w-1, 2s+w, c-1, c, L-1} plus 256 seeded random rows (128 at 131072
tokens, on one query head per KV group).  Bars: bf16 max-abs
<= 2e-2 and mean-abs <= 2e-3.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import long_context_attention_dca_amd as dca
from long_context_attention_dca_amd import inputs

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN = 2e-2, 2e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def landmark_rows(L, c, w, n_random, seed):
    s = c - w
    rows = {0, 1, s - 1, s, s + w - 1, s + w, 2 * s - 1, 2 * s, 2 * s + w - 1, 2 * s + w, c - 1, c, L - 1}
    rng = np.random.default_rng(seed)
    rows |= set(int(x) for x in rng.integers(0, L, size=n_random))
    return np.array(sorted(r for r in rows if 0 <= r < L))


def lse_bound_rows(q, k, rows, heads):
    """bf16 LSE bar on the sampled rows: max(2e-2, 2^-8 * scale * |q_i| *
    max_{j<=i} |k_j|).  Rounding the rotated q and k to bf16 moves every score
    by at most 2^-8 * scale * |q| |k| (rotations keep norms), and the LSE by at
    most the largest score change."""
    qn = torch.linalg.vector_norm(q[:, rows][:, :, heads], dim=-1, dtype=torch.float32).double().numpy()
    kn = torch.linalg.vector_norm(k, dim=-1, dtype=torch.float32).double().numpy()       # [B, L, Hkv]
    G = q.shape[2] // k.shape[2]
    kmax = np.maximum.accumulate(kn, axis=1)[:, rows][:, :, np.asarray(heads) // G]      # [B, R, H]
    bound = 2.0 ** -8 / np.sqrt(q.shape[-1]) * qn * kmax
    return np.maximum(2e-2, bound.transpose(0, 2, 1))                                    # [B, H, R]


def check(got, want, what):
    err = np.abs(got - want)
    mx, mean = float(err.max()), float(err.mean())
    log(f"  {what}: max abs {mx:.3e}, mean abs {mean:.3e}")
    assert mx <= BF16_MAX and mean <= BF16_MEAN, what


def run_prefill_workload(name, heads=None, n_random=256, qk_scale=None, seed_offset=0):
    cfg = inputs.WORKLOADS[name]
    B, L, Hq, Hkv, D, c, w = (cfg[k] for k in ("B", "L", "Hq", "Hkv", "D", "c", "w"))
    log(f"[{name}] generating inputs (seed {cfg['seed'] + seed_offset})")
    q, k, v = inputs.prefill_inputs(B, L, Hq, Hkv, D, cfg["dtype"], seed=cfg["seed"] + seed_offset,
                                    qk_scale=qk_scale)
    log(f"[{name}] GPU prefill")
    o, lse = dca.prefill(q.cuda(), k.cuda(), v.cuda(), c, w, cfg["base"], return_lse=True)
    torch.cuda.synchronize()
    rows = landmark_rows(L, c, w, n_random, seed=cfg["seed"])
    heads = np.arange(Hq) if heads is None else np.asarray(heads)
    og = o[:, torch.from_numpy(rows).cuda()][:, :, torch.from_numpy(heads).cuda()].float().cpu().numpy()
    lg = lse[:, torch.from_numpy(heads).cuda()][:, :, torch.from_numpy(rows).cuda()].cpu().numpy()
    del o, lse
    torch.cuda.empty_cache()
    log(f"[{name}] oracle on {len(rows)} rows x {len(heads)} heads")
    O, LSE = oracle.dca_prefill_ref(q, k, v, c, w, cfg["base"], rows=rows, heads=heads)
    check(og, O, f"{name} O")
    lerr = np.abs(lg - LSE)
    assert np.all(lerr <= lse_bound_rows(q, k, torch.from_numpy(rows), torch.from_numpy(heads))), lerr.max()


def test_llama2_7b_16k_sampled_rows():
    run_prefill_workload("llama2_7b_16k")


def test_llama2_7b_16k_discriminating_inputs():
    run_prefill_workload("llama2_7b_16k", heads=[0, 9, 31], qk_scale=2.0, seed_offset=100)


def test_llama2_70b_32k_sampled_rows():
    run_prefill_workload("llama2_70b_32k")


def test_llama2_70b_128k_sampled_rows():
    # one query head per KV group, landmark + random rows
    run_prefill_workload("llama2_70b_128k", heads=[g * 8 + (g % 8) for g in range(8)], n_random=128)


def test_decode_100k_sampled_batches():
    cfg = inputs.WORKLOADS["decode_100k"]
    B, kv_len, Hq, Hkv, D, c, w = (cfg[k] for k in ("B", "kv_len", "Hq", "Hkv", "D", "c", "w"))
    log("[decode_100k] generating inputs")
    q, k, v = inputs.decode_inputs(B, kv_len, Hq, Hkv, D, cfg["dtype"], seed=cfg["seed"])
    log("[decode_100k] building the rotated cache and decoding")
    kc = dca.rope_remap(k.cuda(), dca.DCA_MAP_KEY, c, w, cfg["base"], 0)
    vg = v.cuda()
    o, lse = dca.decode(q.cuda(), kc, vg, c, w, cfg["base"], return_lse=True)
    o2 = dca.decode(q.cuda(), kc, vg, c, w, cfg["base"])
    assert torch.equal(o, o2)  # fixed split order: bitwise deterministic
    og, lg = o.float().cpu().numpy(), lse.cpu().numpy()
    del kc, vg, o, o2
    torch.cuda.empty_cache()
    batches = [0, 5, 15]
    log(f"[decode_100k] oracle on batches {batches}")
    O, LSE = oracle.dca_decode_ref(q, k, v, c, w, cfg["base"], batches=batches)
    check(og[batches], O, "decode_100k O")
    assert np.abs(lg[batches] - LSE).max() <= 2e-2
