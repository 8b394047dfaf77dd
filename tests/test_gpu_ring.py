"""One device's share of Ring Attention (bpt_attention_fwd + bpt_attention_merge)
against the oracle: a step alone, and the whole ring simulated on one device (its
query shard meets every earlier key/value shard, unmasked, and its own, causal;
the merged result must equal the oracle's attention of that shard over the whole
causal prefix). Tolerance as the layer's: bf16 operands, fp32 statistics; the lse
bound of the layer tests."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from blockwise_attn_ffn_amd import bpt, synth
from _parity import LSE_TOL, say

pytestmark = pytest.mark.gpu


def step(q, k, v, batch, n, d, h, causal):
    desc = bpt.make_attn_desc(batch=batch, seq_len=n, d_model=d, n_heads=h, causal=causal)
    o = torch.empty(batch * n, d, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(batch, h, n, dtype=torch.float32, device="cuda")
    ws = bpt.alloc_workspace(bpt.attention_fwd_workspace_bytes(desc))
    bpt.attention_fwd(desc, q, k, v, o, lse, ws)
    return o, lse


def ring_device(q_sh, k_sh, v_sh, r, n, d, h):
    """Device r of a ring: steps over shards 0..r (later shards are skipped)."""
    desc = bpt.make_attn_desc(batch=1, seq_len=n, d_model=d, n_heads=h, causal=True)
    o_acc = torch.zeros(n, d, dtype=torch.float32, device="cuda")
    lse_acc = torch.full((1, h, n), float("-inf"), dtype=torch.float32, device="cuda")
    for s_ in range(r + 1):
        o, lse = step(q_sh[r], k_sh[s_], v_sh[s_], 1, n, d, h, causal=(s_ == r))
        bpt.attention_merge(desc, o_acc, lse_acc, o, lse)
    torch.cuda.synchronize()
    return o_acc.cpu(), lse_acc.cpu()


def check(got, ref, what, tol=2e-2, fro=5e-3):
    g = got.double().numpy()
    assert np.all(np.isfinite(g)), what
    mx, rf = oracle.max_abs_err(g, ref), oracle.rel_fro_err(g, ref)
    say(f"  {what}: max|err| {mx:.3e}, rel fro {rf:.3e}")
    assert mx <= tol and rf <= fro, what


@pytest.mark.parametrize("n,d,h,causal", [(200, 256, 4, True), (200, 256, 4, False),
                                          (300, 256, 2, True), (129, 512, 4, False)])
def test_attention_step(n, d, h, causal):
    say(f"case step n={n} d={d} h={h} causal={causal}")
    inp = synth.make_attention_inputs(2, n, d, seed=41)
    o, lse = step(inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda(), 2, n, d, h, causal)
    torch.cuda.synchronize()
    for b in range(2):
        r = slice(b * n, (b + 1) * n)
        q, k, v = (synth.to_f64(inp[x][r]) for x in ("q", "k", "v"))
        check(o.cpu()[r], oracle.attention_sequence(q, k, v, h, causal), f"O seq {b}")
        ref_l = oracle.attention_lse_sequence(q, k, h, causal)
        assert np.max(np.abs(lse.cpu()[b].double().numpy() - ref_l)) <= LSE_TOL["bf16"]


@pytest.mark.parametrize("n,d,h", [(256, 256, 4), (200, 256, 2)])
def test_ring_on_one_device(n, d, h):
    """4 shards of n tokens; every device's merged result over its prefix."""
    R = 4
    say(f"case ring R={R} shard={n} d={d} h={h}")
    inp = synth.make_attention_inputs(1, R * n, d, seed=43)
    q_sh, k_sh, v_sh = ([inp[x][s * n:(s + 1) * n].cuda() for s in range(R)] for x in ("q", "k", "v"))
    q, k, v = (synth.to_f64(inp[x]) for x in ("q", "k", "v"))
    for r in range(R):
        o, lse = ring_device(q_sh, k_sh, v_sh, r, n, d, h)
        pos = np.arange(r * n, (r + 1) * n)
        keys = slice(0, (r + 1) * n)
        ref = oracle.attention_sequence(q[pos], k[keys], v[keys], h, True, q_pos=pos)
        check(o, ref, f"device {r}")
        ref_l = oracle.attention_lse_sequence(q[pos], k[keys], h, True, q_pos=pos)
        assert np.max(np.abs(lse[0].double().numpy() - ref_l)) <= LSE_TOL["bf16"], r


def test_ring_long_context_last_device_sampled_rows():
    """131072 tokens over 8 devices (16384-token shards, 16 heads of 128): the last
    device's 8 steps, its result checked on sampled rows of its shard."""
    R, n, d, h = 8, 16384, 2048, 16
    say("case ring 131072 tokens / 8 devices, last device")
    inp = synth.make_attention_inputs(1, R * n, d, seed=45)
    q_sh, k_sh, v_sh = ([inp[x][s * n:(s + 1) * n].cuda() for s in range(R)] for x in ("q", "k", "v"))
    o, lse = ring_device(q_sh, k_sh, v_sh, R - 1, n, d, h)
    rows = np.sort(np.concatenate([[0, 1, n - 1], np.random.default_rng(7).choice(n, 13, replace=False)]))
    pos = (R - 1) * n + rows
    q, k, v = (synth.to_f64(inp[x]) for x in ("q", "k", "v"))
    ref = oracle.attention_sequence(q[pos], k, v, h, True, q_pos=pos)
    check(o[torch.from_numpy(rows)], ref, "last device, sampled rows")


# ---------------------------------------------------------------------------
# bpt_ring_share_fwd: packed shards, the merge inside the attention kernel
# ---------------------------------------------------------------------------

def pack_shards(k_sh, v_sh, n, d, h):
    desc = bpt.make_attn_desc(batch=1, seq_len=n, d_model=d, n_heads=h, causal=True)
    out = []
    for k, v in zip(k_sh, v_sh):
        kv = bpt.alloc_workspace(bpt.ring_kv_bytes(desc))
        bpt.ring_pack_kv(desc, k, v, kv)
        out.append(kv)
    return out


def share(q, kv, own, n, d, h, causal=True):
    desc = bpt.make_attn_desc(batch=1, seq_len=n, d_model=d, n_heads=h, causal=causal)
    o = torch.full((n, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((1, h, n), float("nan"), dtype=torch.float32, device="cuda")
    ws = bpt.alloc_workspace(bpt.ring_share_workspace_bytes(desc))
    shards = [kv[s] if (not causal or s <= own) else None for s in range(len(kv))]
    bpt.ring_share_fwd(desc, own, q, shards, o, lse, ws)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


@pytest.mark.parametrize("n,d,h", [(256, 256, 4), (200, 256, 2), (131, 512, 4)])
def test_ring_share_every_device(n, d, h):
    """4 shards of n tokens (d_k 64 and 128, ragged shards): every device's share
    through the packed-shard entry, against the oracle over its causal prefix."""
    R = 4
    say(f"case ring share R={R} shard={n} d={d} h={h}")
    inp = synth.make_attention_inputs(1, R * n, d, seed=47)
    q_sh, k_sh, v_sh = ([inp[x][s * n:(s + 1) * n].cuda() for s in range(R)] for x in ("q", "k", "v"))
    kv = pack_shards(k_sh, v_sh, n, d, h)
    q, k, v = (synth.to_f64(inp[x]) for x in ("q", "k", "v"))
    for r in range(R):
        o, lse = share(q_sh[r], kv, r, n, d, h)
        pos = np.arange(r * n, (r + 1) * n)
        keys = slice(0, (r + 1) * n)
        check(o, oracle.attention_sequence(q[pos], k[keys], v[keys], h, True, q_pos=pos), f"device {r}")
        ref_l = oracle.attention_lse_sequence(q[pos], k[keys], h, True, q_pos=pos)
        assert np.max(np.abs(lse[0].double().numpy() - ref_l)) <= LSE_TOL["bf16"], r


def test_ring_share_unmasked():
    """Without the mask every shard is seen whole, whatever own is."""
    R, n, d, h = 3, 200, 256, 4
    say(f"case ring share unmasked R={R} shard={n}")
    inp = synth.make_attention_inputs(1, R * n, d, seed=48)
    q_sh, k_sh, v_sh = ([inp[x][s * n:(s + 1) * n].cuda() for s in range(R)] for x in ("q", "k", "v"))
    kv = pack_shards(k_sh, v_sh, n, d, h)
    q, k, v = (synth.to_f64(inp[x]) for x in ("q", "k", "v"))
    o, lse = share(q_sh[1], kv, 1, n, d, h, causal=False)
    pos = np.arange(n, 2 * n)
    check(o, oracle.attention_sequence(q[pos], k, v, h, False), "unmasked share")
    ref_l = oracle.attention_lse_sequence(q[pos], k, h, False)
    assert np.max(np.abs(lse[0].double().numpy() - ref_l)) <= LSE_TOL["bf16"]


def test_ring_share_long_context_last_device_sampled_rows():
    """131072 tokens over 8 devices (16384-token shards, 16 heads of 128): the last
    device's share through the packed-shard entry, on sampled rows."""
    R, n, d, h = 8, 16384, 2048, 16
    say("case ring share 131072 tokens / 8 devices, last device")
    inp = synth.make_attention_inputs(1, R * n, d, seed=45)
    q_sh, k_sh, v_sh = ([inp[x][s * n:(s + 1) * n].cuda() for s in range(R)] for x in ("q", "k", "v"))
    kv = pack_shards(k_sh, v_sh, n, d, h)
    o, lse = share(q_sh[R - 1], kv, R - 1, n, d, h)
    rows = np.sort(np.concatenate([[0, 1, n - 1], np.random.default_rng(7).choice(n, 13, replace=False)]))
    pos = (R - 1) * n + rows
    q, k, v = (synth.to_f64(inp[x]) for x in ("q", "k", "v"))
    check(o[torch.from_numpy(rows)], oracle.attention_sequence(q[pos], k, v, h, True, q_pos=pos),
          "last device share, sampled rows")
    ref_l = oracle.attention_lse_sequence(q[pos], k, h, True, q_pos=pos)
    assert np.max(np.abs(lse[0][:, rows].double().numpy() - ref_l)) <= LSE_TOL["bf16"]
