"""bpt_layer_fwd_noalloc, the entry point that allocates nothing, against
bpt_layer_fwd on the same inputs: calls in a row, each later one smaller, all on
the library's fixed per-device scratch. The same kernels run over a workspace of
the same layout, so Z must be bit-identical."""
import pytest
import torch

from blockwise_attn_ffn_amd import bpt, synth

pytestmark = pytest.mark.gpu

CASES = [
    # 2 ragged sequences at d 1024 (about 40 MB of the 64 MiB scratch)
    synth.Workload("na_big", batch=2, seq_len=1000, d_model=1024, n_heads=16, d_ff=4096,
                   causal=True, block_q=128, block_kv=128, dtype="bf16", ln_random=True),
    # smaller: one sequence, d 256, other block sizes
    synth.Workload("na_small", batch=1, seq_len=300, d_model=256, n_heads=4, d_ff=1024,
                   causal=True, block_q=128, block_kv=64, dtype="bf16", ln_random=True),
    # smaller still, fp32 throughout
    synth.Workload("na_f32", batch=1, seq_len=129, d_model=128, n_heads=2, d_ff=512,
                   causal=False, block_q=64, block_kv=64, dtype="f32"),
]


def _run(w, seed):
    inp = synth.make_inputs(w, seed=seed)
    desc = bpt.desc_for(w, out_dtype="f32")
    need = bpt.layer_workspace_bytes(desc)
    assert 0 < need <= bpt.NOALLOC_SCRATCH_BYTES, (w.name, need)
    x = inp["x"].cuda()
    layer = {k: v.cuda() for k, v in inp["layers"][0].items()}
    z_ref = torch.empty((w.rows, w.d_model), dtype=torch.float32, device="cuda")
    ws = bpt.alloc_workspace(need)
    bpt.layer_fwd(desc, x, layer, z_ref, ws)
    z = torch.full((w.rows, w.d_model), float("nan"), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    bpt.layer_fwd_noalloc(desc, x, layer, z)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    return z, z_ref, free0, free1


def test_noalloc_matches_layer_fwd_on_calls_in_a_row():
    for i, w in enumerate(CASES):
        print(f"noalloc case {w.name}", flush=True)
        z, z_ref, free0, free1 = _run(w, seed=i)
        assert torch.isfinite(z).all(), w.name
        assert torch.equal(z, z_ref), (w.name, (z - z_ref).abs().max().item())
        if i > 0:   # the scratch exists after the first call: nothing more is allocated
            assert free1 == free0, (w.name, free0 - free1)


def test_noalloc_rejects_a_layer_beyond_its_scratch():
    w = synth.WORKLOADS["gpt2_medium"]
    desc = bpt.desc_for(w, out_dtype="f32")
    assert bpt.layer_workspace_bytes(desc) > bpt.NOALLOC_SCRATCH_BYTES
    x = torch.empty(8, device="cuda")
    z = torch.empty(8, device="cuda")
    layer = {k: torch.empty(8, device="cuda") for k in bpt.WEIGHT_FIELDS}
    with pytest.raises(bpt.BptError) as e:
        bpt.layer_fwd_noalloc(desc, x, layer, z)
    assert e.value.status == 5 and "scratch" in e.value.detail
