"""The C ABI on the host (no GPU): the library loads, exports every function the
header declares, sizes the workspace by its formula, and rejects every invalid
argument before anything is enqueued.

Every call here fails validation (or is an empty call), so no kernel is ever
launched: the pointers are fake, 16-byte-aligned integers.
"""
import ctypes
import math
import os
import re
import shutil
import subprocess

import pytest

from blockwise_attn_ffn_amd import bpt, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bpt.h")

FAKE = 0x7f0000000000  # aligned, never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bpt_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = bpt.lib()
    names = declared_functions()
    assert set(names) == set(bpt.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.bpt_version().decode().count(".") == 2


def test_status_strings():
    lib = bpt.lib()
    for code in range(8):
        assert lib.bpt_status_str(code).decode() not in ("", "unknown status")
    assert lib.bpt_status_str(99).decode() == "unknown status"


def desc(**kw):
    base = dict(batch=2, seq_len=200, d_model=256, n_heads=4, d_ff=1024, block_q=128,
                block_kv=128, causal=True, dtype="bf16", out_dtype="f32")
    base.update(kw)
    return bpt.make_desc(**base)


def hidden_rows(d, rows_pad):
    """Rows of the staged epilogue's hidden block: 2^25 / d rounded down to a
    multiple of 256 (the W_2 product then spans 512 tiles of 256 x 256), at least
    4096, at most the padded rows."""
    return min(rows_pad, max(4096, (2 ** 25 // d) // 256 * 256))


def coop_exchange_bytes(d, split=False):
    """The cooperative epilogue's exchange regions (one per cluster of d / 512
    workgroups, 256 workgroups at most) and its counters: per cluster LN2(Y) of a
    128-row tile, two hidden chunks of 256 d / 512 units and the per-row partial
    statistics, 4 KB aligned; independent of the number of rows."""
    g = d // 512
    hc = 256 * g
    na = 2 if split else 1                    # bf16 pairs: hi and lo halves
    region = na * 4 * (d // 16) * 1024 + 2 * na * 4 * (hc // 16) * 1024 + 2 * g * 128 * 8
    region = (region + 4095) // 4096 * 4096
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    return up((256 // g) * region) + up((32 + 4 * 256) * 4)


def is_coop(d, f, split):
    return d in (2048, 4096) and f % (256 * (d // 512)) == 0


def expected_workspace(batch, n, d, es, stack_resid=False, d_ff=None, split=False, dkv=None):
    up = lambda x: (x + 255) // 256 * 256  # noqa: E731
    rows = batch * n
    npad = (n + 127) // 128 * 128
    used = batch * npad
    rows_pad = up(used)
    f = 4 * d if d_ff is None else d_ff
    coop = is_coop(d, f, split)    # cooperative epilogue: an exchange region, nothing [rows, d_ff]
    staged = not coop and (d > 1024 or split)  # staged: K, V^T over rows_pad rows + hidden block
    dkv = d if dkv is None else dkv          # key/value width (grouped-query attention)
    tile = 128 if es == 4 else 256
    kvp = (dkv + tile - 1) // tile * tile    # K and V parts of the projection, padded
    kv_rows = rows_pad if staged else used
    kv_space = 2 * up(kv_rows * dkv * es)
    if staged:                               # room for the fp32 Y over K and V^T
        kv_space = max(kv_space, up(rows_pad * d * 4))
    acts = 2 * up(rows_pad * d * es) + kv_space
    hidden = up(hidden_rows(d, rows_pad) * f * es) if staged else 0
    tot = acts + up(((d + 2 * kvp) * d + d * d + 2 * d * f) * es) + hidden
    if coop:
        tot += coop_exchange_bytes(d, split)
    if split:                   # lo halves: no Y room there
        acts = 2 * up(rows_pad * d * es) + 2 * up(kv_rows * dkv * es)
    if split:                   # lo halves of the bf16 pairs
        tot += acts + hidden
    if stack_resid:
        tot += up(rows * d * 4)
    return tot


@pytest.mark.parametrize("batch,n,d,h,dt", [(2, 200, 256, 4, "bf16"), (1, 131072, 2048, 16, "bf16"),
                                            (64, 1024, 1024, 16, "bf16"), (1, 77, 128, 2, "f32"),
                                            (1, 32768, 4096, 32, "bf16"), (3, 300, 4096, 32, "bf16"),
                                            (2, 5000, 2048, 16, "bf16"), (1, 300, 2048, 16, "bf16")])
def test_workspace_formula(batch, n, d, h, dt):
    dsc = desc(batch=batch, seq_len=n, d_model=d, n_heads=h, d_ff=4 * d, dtype=dt,
               block_q=64, block_kv=64)
    es = 4 if dt == "f32" else 2
    assert bpt.layer_workspace_bytes(dsc) == expected_workspace(batch, n, d, es)
    assert bpt.stack_workspace_bytes(dsc, 1) == expected_workspace(batch, n, d, es)
    dsc.out_dtype = bpt.BF16
    assert bpt.stack_workspace_bytes(dsc, 3) == expected_workspace(batch, n, d, es, True)
    dsc.out_dtype = bpt.F32
    assert bpt.stack_workspace_bytes(dsc, 3) == expected_workspace(batch, n, d, es)


@pytest.mark.parametrize("batch,n,d,h", [(2, 200, 256, 4), (1, 32768, 4096, 32), (3, 1500, 1024, 16),
                                         (2, 40000, 768, 12)])
def test_workspace_formula_bf16_pairs(batch, n, d, h):
    dsc = desc(batch=batch, seq_len=n, d_model=d, n_heads=h, d_ff=4 * d, precision=1)
    assert bpt.layer_workspace_bytes(dsc) == expected_workspace(batch, n, d, 2, split=True)
    dsc.out_dtype = bpt.BF16
    assert bpt.stack_workspace_bytes(dsc, 4) == expected_workspace(batch, n, d, 2, True, split=True)


@pytest.mark.parametrize("batch,n,d,h,g,dt,split", [
    (2, 200, 256, 4, 1, "bf16", False), (2, 200, 256, 4, 2, "bf16", False),
    (1, 131072, 2048, 16, 4, "bf16", False), (1, 300, 2048, 16, 1, "bf16", False),
    (64, 1024, 1024, 16, 8, "bf16", False), (1, 77, 128, 2, 1, "f32", False),
    (2, 200, 256, 4, 2, "bf16", True), (1, 5000, 2048, 16, 2, "bf16", True)])
def test_workspace_formula_grouped_kv_heads(batch, n, d, h, g, dt, split):
    dsc = desc(batch=batch, seq_len=n, d_model=d, n_heads=h, d_ff=4 * d, dtype=dt,
               block_q=64, block_kv=64, precision=int(split))
    dsc.n_kv_heads = g
    es = 4 if dt == "f32" else 2
    assert bpt.layer_workspace_bytes(dsc) == expected_workspace(batch, n, d, es, split=split,
                                                                dkv=g * (d // h))
    dsc.n_kv_heads = h                       # g = n_heads is multi-head attention
    assert bpt.layer_workspace_bytes(dsc) == expected_workspace(batch, n, d, es, split=split)


@pytest.mark.parametrize("g", [-1, 3, 5])
def test_invalid_kv_heads(g):
    dsc = desc(n_heads=4)
    dsc.n_kv_heads = g
    assert call_layer(dsc) == 2 and "n_kv_heads" in bpt.last_error()
    assert bpt.layer_workspace_bytes(dsc) == 0


def test_bf16_pairs_need_bf16_inputs():
    dsc = desc(dtype="f32", d_model=256, precision=1)
    assert bpt.layer_workspace_bytes(dsc) == 0
    assert call_layer(dsc) == 3
    assert "precision 1" in bpt.last_error()


def test_workspace_is_block_shaped_not_ffn_shaped():
    """The activation part of the footprint is LN1(X), Q/O, K and V^T (4 N d), plus,
    on the staged epilogue, one block of the FFN hidden state: below the two [N, 4d]
    hidden tensors (8 N d) and the page's after-Flash unfused total (6 N d + 8 N d);
    no [N, N] logits exist."""
    for name in ("gpt2_small", "gpt2_medium", "long_128k"):
        w = synth.WORKLOADS[name]
        ws = bpt.layer_workspace_bytes(bpt.desc_for(w))
        weights = (4 * w.d_model * w.d_model + 2 * w.d_model * w.d_ff) * 2
        act = ws - weights
        nd = w.rows * w.d_model * 2
        exchange = coop_exchange_bytes(w.d_model) if is_coop(w.d_model, w.d_ff, False) else 0
        assert act <= 4 * nd + exchange + 8 * 256 + 256 * w.d_model * 2 * 2
        assert act < 2 * w.rows * w.d_ff * 2          # the unfused FFN hidden pair
        assert act < 14 * nd                          # after-Flash, unfused
    w = synth.WORKLOADS["long_128k"]
    assert bpt.layer_workspace_bytes(bpt.desc_for(w)) < w.seq_len * w.seq_len * 2
    # no term grows with rows x d_ff: the exchange region is under 1/30 of the [N, d_ff] hidden
    # here, and the same at any sequence length
    assert coop_exchange_bytes(w.d_model) * 30 < w.rows * w.d_ff * 2
    longer = bpt.desc_for(w)
    longer.seq_len *= 2
    ws1, ws2 = bpt.layer_workspace_bytes(bpt.desc_for(w)), bpt.layer_workspace_bytes(longer)
    weights = (4 * w.d_model * w.d_model + 2 * w.d_model * w.d_ff) * 2
    assert ws2 - weights == 2 * (ws1 - weights - coop_exchange_bytes(w.d_model)) + coop_exchange_bytes(w.d_model)
    # the stack runs in bf16 pairs (precision 1), which doubles every activation
    w = synth.WORKLOADS["stack4_32k"]
    assert w.precision == 1
    ws = bpt.layer_workspace_bytes(bpt.desc_for(w))
    weights = (4 * w.d_model * w.d_model + 2 * w.d_model * w.d_ff) * 2
    nd = w.rows * w.d_model * 2
    # the cooperative epilogue in bf16 pairs: no hidden block, a bounded exchange region
    exchange = coop_exchange_bytes(w.d_model, split=True)
    assert ws - weights <= 2 * 4 * nd + exchange + 16 * 256
    assert exchange * 7 < w.rows * w.d_ff * 2           # under 1/7 of the [N, d_ff] hidden


def call_layer(dsc, x=FAKE, z=FAKE + (1 << 36), ws=FAKE + (2 << 36), nbytes=1 << 40,
               weights=None):
    lib = bpt.lib()
    if weights is None:
        weights = bpt.LayerWeights(*[FAKE + (3 << 36) + i * (1 << 30) for i in range(10)])
    return lib.bpt_layer_fwd(ctypes.byref(dsc) if dsc is not None else None, x,
                             ctypes.byref(weights) if weights != 0 else None, z, ws, nbytes, None)


@pytest.mark.parametrize("field,value,status", [
    ("batch", -1, 2), ("seq_len", -5, 2), ("d_model", 0, 2), ("n_heads", 0, 2),
    ("n_heads", 3, 2), ("d_ff", 0, 2), ("block_q", 0, 2), ("causal", 2, 2),
    ("ln_eps", 0.0, 2), ("ln_eps", float("nan"), 2), ("ln_eps", float("inf"), 2),
    ("dtype", 7, 2), ("out_dtype", -1, 2), ("act", 1, 3), ("precision", 2, 2),
    ("d_model", 640, 3), ("n_heads", 8, 3),           # d_head 32
    ("block_q", 96, 3), ("block_kv", 256, 3), ("d_ff", 1000, 3),
    ("window", -1, 2), ("chunk", -3, 2),
])
def test_invalid_descriptor(field, value, status):
    dsc = desc()
    setattr(dsc, field, value)
    assert call_layer(dsc) == status
    assert bpt.last_error() != ""
    assert bpt.layer_workspace_bytes(dsc) == 0


def test_mask_combinations():
    """window and chunk need the causal mask and cannot be combined."""
    dsc = desc(causal=0)
    dsc.window = 16
    assert call_layer(dsc) == 2 and "causal" in bpt.last_error()
    dsc = desc(causal=0)
    dsc.chunk = 16
    assert call_layer(dsc) == 2
    dsc = desc(causal=1)
    dsc.window, dsc.chunk = 16, 16
    assert call_layer(dsc) == 2 and "combined" in bpt.last_error()
    for field in ("window", "chunk"):          # valid: the workspace does not change
        dsc = desc(causal=1)
        setattr(dsc, field, 100)
        assert bpt.layer_workspace_bytes(dsc) == bpt.layer_workspace_bytes(desc(causal=1)) > 0


def test_row_count_overflow():
    dsc = desc(batch=1 << 16, seq_len=1 << 16)
    assert call_layer(dsc) == 2


def test_null_and_alignment_and_workspace_and_alias():
    dsc = desc()
    need = bpt.layer_workspace_bytes(dsc)
    assert need > 0
    lib = bpt.lib()
    assert lib.bpt_layer_fwd(None, FAKE, None, FAKE, FAKE, 0, None) == 1   # NULL desc
    assert call_layer(dsc, weights=0) == 1                                # NULL weights
    w = bpt.LayerWeights(*[FAKE + (3 << 36) + i * (1 << 30) for i in range(10)])
    w.w_2 = None
    assert call_layer(dsc, weights=w) == 1 and "w_2" in bpt.last_error()
    w.w_2 = FAKE + 8
    assert call_layer(dsc, weights=w) == 4                                # misaligned weight
    assert call_layer(dsc, x=0) == 1
    assert call_layer(dsc, z=0) == 1
    assert call_layer(dsc, x=FAKE + 4) == 4
    assert call_layer(dsc, ws=FAKE + (2 << 36) + 8) == 4
    assert call_layer(dsc, nbytes=need - 1) == 5
    assert call_layer(dsc, ws=0, nbytes=need) == 1
    assert call_layer(dsc, z=FAKE + 256) == 6                             # X and Z overlap
    assert call_layer(dsc, ws=FAKE + 1024, nbytes=need) == 6              # workspace over X
    assert call_layer(dsc, ws=FAKE + (1 << 36) - 256, nbytes=need) == 6   # workspace over Z


def test_empty_call_is_ok_with_null_pointers():
    lib = bpt.lib()
    for b, n in ((0, 10), (3, 0)):
        dsc = desc(batch=b, seq_len=n)
        assert lib.bpt_layer_fwd(ctypes.byref(dsc), None, None, None, None, 0, None) == 0
        assert bpt.layer_workspace_bytes(dsc) == 0


def test_stack_validation():
    lib = bpt.lib()
    dsc = desc()
    arr = (bpt.LayerWeights * 2)(*[bpt.LayerWeights(*[FAKE + (3 << 36) + i * (1 << 30)
                                                      for i in range(10)]) for _ in range(2)])
    big = 1 << 40
    assert lib.bpt_stack_fwd(ctypes.byref(dsc), 0, FAKE, arr, FAKE + (1 << 36), FAKE + (2 << 36),
                             big, None) == 2
    assert lib.bpt_stack_fwd(ctypes.byref(dsc), 2, FAKE, None, FAKE + (1 << 36), FAKE + (2 << 36),
                             big, None) == 1
    arr[1].w_k = None
    assert lib.bpt_stack_fwd(ctypes.byref(dsc), 2, FAKE, arr, FAKE + (1 << 36), FAKE + (2 << 36),
                             big, None) == 1
    assert "weights[1].w_k" in bpt.last_error()
    assert bpt.stack_workspace_bytes(dsc, 0) == 0


def test_every_named_workload_is_supported():
    for w in synth.WORKLOADS.values():
        assert bpt.layer_workspace_bytes(bpt.desc_for(w)) > 0, (w.name, bpt.last_error())


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_abi_under_address_and_ub_sanitizers(tmp_path):
    """Build the host validation layer alone with ASan + UBSan (launches stubbed) and
    drive every entry point, including valid calls that reach the (stub) launcher."""
    csrc = os.path.join(ROOT, "blockwise_attn_ffn_amd", "csrc")
    drv = os.path.join(os.path.dirname(__file__), "abi_host_driver.cpp")
    exe = str(tmp_path / "abi_host")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", f"-I{os.path.join(ROOT, 'include')}",
           "-mavx2", "-mfma", "-pthread", os.path.join(csrc, "bpt_api.cpp"),
           os.path.join(csrc, "bpt_support.cpp"), os.path.join(csrc, "bpt_host.cpp"), drv, "-o", exe]
    subprocess.run(cmd, check=True)
    res = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                         timeout=120)
    assert res.returncode == 0, res.stdout
    assert "ALL OK" in res.stdout


def test_operands_of_4_gib_are_rejected_before_launch():
    """8 sequences of 131072 tokens at d_model 2048 in bf16: the LN1 operand alone
    is 8 * 131072 * 2048 * 2 B = 4 GiB, past the 32-bit offsets of the product
    kernels. Validation reports BPT_ERR_UNSUPPORTED (nothing enqueued: the fake
    pointers would fault otherwise) and the workspace query returns 0; one
    sequence fewer fits."""
    dsc = desc(batch=8, seq_len=131072, d_model=2048, n_heads=16, d_ff=8192)
    assert bpt.layer_workspace_bytes(dsc) == 0
    assert call_layer(dsc) == 3 and "4 GiB" in bpt.last_error()
    dsc.batch = 7
    assert bpt.layer_workspace_bytes(dsc) > 0


def test_noalloc_rejects_without_touching_a_device():
    """bpt_layer_fwd_noalloc validates on the host first: a layer whose workspace
    exceeds the fixed scratch is BPT_ERR_WORKSPACE, an invalid descriptor
    BPT_ERR_SHAPE, a NULL X BPT_ERR_NULL (no GPU in this test)."""
    lib = bpt.lib()
    w = bpt.LayerWeights(*[FAKE + (3 << 36) + i * (1 << 30) for i in range(10)])
    big = desc(batch=64, seq_len=1024, d_model=1024, n_heads=16, d_ff=4096)
    assert bpt.layer_workspace_bytes(big) > bpt.NOALLOC_SCRATCH_BYTES
    assert lib.bpt_layer_fwd_noalloc(ctypes.byref(big), FAKE, ctypes.byref(w), FAKE + (1 << 36), None) == 5
    assert "scratch" in bpt.last_error()
    bad = desc(causal=2)
    assert lib.bpt_layer_fwd_noalloc(ctypes.byref(bad), FAKE, ctypes.byref(w), FAKE + (1 << 36), None) == 2
    ok = desc()
    assert lib.bpt_layer_fwd_noalloc(ctypes.byref(ok), None, ctypes.byref(w), FAKE + (1 << 36), None) == 1
    assert lib.bpt_layer_fwd_noalloc(ctypes.byref(ok), FAKE, None, FAKE + (1 << 36), None) == 1


def bwd_call(dsc, nbytes=None, **over):
    """bpt_layer_bwd on fake, disjoint pointers (validation only)."""
    lib = bpt.lib()
    w = bpt.LayerWeights(*[FAKE + (3 << 36) + i * (1 << 30) for i in range(10)])
    g = bpt.LayerGrads(*[FAKE + (7 << 36) + i * (1 << 30) for i in range(10)])
    args = dict(x=FAKE, lse=FAKE + (1 << 35), dz=FAKE + (9 << 36), dx=FAKE + (10 << 36),
                ws=FAKE + (11 << 36))
    args.update(over)
    if nbytes is None:
        nbytes = 1 << 40
    return lib.bpt_layer_bwd(ctypes.byref(dsc), args["x"], ctypes.byref(w), args["lse"], args["dz"],
                             args["dx"], ctypes.byref(g), args["ws"], nbytes, None)


@pytest.mark.parametrize("field,value", [("dtype", bpt.F32), ("precision", 1)])
def test_layer_bwd_limits(field, value):
    """The backward takes bf16 at precision 0: anything else is BPT_ERR_UNSUPPORTED
    (nothing enqueued) and a workspace of 0."""
    dsc = desc()
    setattr(dsc, field, value)
    if field == "dtype":
        dsc.out_dtype = bpt.F32
    assert bpt.layer_bwd_workspace_bytes(dsc) == 0
    assert bwd_call(dsc) == 3
    assert bpt.last_error() != ""


@pytest.mark.parametrize("field,value", [("window", 16), ("chunk", 64), ("n_kv_heads", 2), ("n_kv_heads", 1)])
def test_layer_bwd_takes_masks_and_kv_heads(field, value):
    """Window, chunk and grouped key/value heads are accepted (a workspace is sized);
    inconsistent ones are rejected as for the forward."""
    dsc = desc()
    setattr(dsc, field, value)
    assert bpt.layer_bwd_workspace_bytes(dsc) > 0
    if field == "n_kv_heads":
        dsc.n_kv_heads = 3                      # does not divide 4 heads
    else:
        dsc.causal = False                      # masks of the causal setting only
    assert bpt.layer_bwd_workspace_bytes(dsc) == 0
    assert bwd_call(dsc) == 2


def test_layer_bwd_null_alignment_alias():
    dsc = desc()
    need = bpt.layer_bwd_workspace_bytes(dsc)
    assert need > 0
    assert bwd_call(dsc, nbytes=need - 1) == 5
    assert bwd_call(dsc, lse=0) == 1 and "lse" in bpt.last_error()
    assert bwd_call(dsc, dz=FAKE + (9 << 36) + 4) == 4
    assert bwd_call(dsc, x=0) == 1
    assert bwd_call(dsc, dx=FAKE + (9 << 36) + 256) == 6          # dX over dZ
    assert bwd_call(dsc, ws=FAKE + (3 << 36) - 4096) == 6          # workspace over w_q
    empty = desc(batch=0)
    assert bpt.lib().bpt_layer_bwd(ctypes.byref(empty), None, None, None, None, None, None, None, 0,
                                   None) == 0


def test_layer_bwd_workspace_has_no_rows_by_d_ff_term():
    """The backward's workspace grows with the rows by the same amount whatever d_ff
    is, once the rows exceed the FFN block (2^26 / d_ff rows): only the block's
    [block, d_ff] buffers depend on d_ff, never rows x d_ff ("The backward pass":
    the hidden state is recomputed one block at a time)."""
    def ws(batch, d_ff):
        return bpt.layer_bwd_workspace_bytes(desc(batch=batch, seq_len=4096, d_model=1024,
                                                  n_heads=16, d_ff=d_ff))
    growth = {f: ws(16, f) - ws(8, f) for f in (2048, 4096, 8192, 16384)}
    assert len(set(growth.values())) == 1, growth
    # per extra row: 8 bf16 row-major and 5 bf16 transposed [d] vectors, 5 fp32 [d]
    # vectors, 3 bf16 attention copies, statistics
    assert growth[4096] <= 8 * 4096 * (1024 * (8 * 2 + 5 * 2 + 5 * 4 + 3 * 2) + 16 + 16 * 3 * 4) + 64 * 256
