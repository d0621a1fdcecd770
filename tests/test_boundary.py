"""The C ABI on the CPU: the library loads, exports every function that
include/dsa.h declares, and rejects bad arguments with the documented status
before any HIP call (so no GPU is needed).  Pointers passed here are never
dereferenced: every call either fails validation or has nothing to do."""
import os
import re

import pytest

import sparse_mla_attention_gather_amd as dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")
GOLDEN = os.path.join(ROOT, "tests", "golden")
FAKE = 1 << 20          # a 16-byte-aligned, never-dereferenced address


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for required in ("dsa_kv_write", "dsa_sparse_attn_decode",
                     "dsa_sparse_attn_prefill", "dsa_quantize_q_fp8"):
        assert required in names


def test_library_exports_every_declared_symbol():
    for name in declared_functions():
        assert hasattr(dsa._lib, name), name
    assert set(declared_functions()) == set(dsa.EXPORTED)


def test_status_strings():
    for code, name in enumerate(dsa.STATUS):
        assert dsa.dsa_status_string(code) == name
    assert dsa.dsa_status_string(99) == "DSA_ERR_UNKNOWN"


def test_row_bytes_match_the_pages():
    rows = {}
    for line in open(os.path.join(GOLDEN, "row_layouts.txt")):
        line = line.split("#")[0].split()
        if line:
            rows[line[0]] = int(line[1])
    assert dsa.dsa_kv_row_bytes(dsa.DSA_KV_RAW_FP8_512) == rows["raw_fp8_nope"]
    assert dsa.dsa_kv_row_bytes(dsa.DSA_KV_SCALED_FP8_528) == rows["scaled_fp8_nope"]
    assert dsa.dsa_kv_row_bytes(dsa.DSA_KV_SCALED_FP8_656) == rows["scaled_fp8_rope"]
    assert dsa.dsa_kv_row_bytes(dsa.DSA_KV_BF16_1024) == rows["bf16_nope"]
    assert dsa.dsa_kv_row_bytes(7) == -1
    assert rows["topk_multiple"] == 128


# ---------------------------------------------------------------- attention

def attn_args(**over):
    a = dict(q=FAKE, q_dtype=dsa.DSA_BF16, q_scale=None, T=4, H=16, D=512,
             rope_dim=0, pool=FAKE, num_slots=1024,
             layout=dsa.DSA_KV_RAW_FP8_512, fp8_format=dsa.DSA_FP8_E4M3FN,
             topk=FAKE, K=256, page_table=FAKE, page_size=64, max_pages=4,
             num_seqs=4, token_seq=None, seq_lens=FAKE, softmax_scale=0.044,
             out=FAKE, out_dtype=dsa.DSA_FP32, lse=None, workspace=None,
             workspace_bytes=0, err_count=None, stream=0)
    a.update(over)
    return a


def call(phase, **over):
    fn = dsa.dsa_sparse_attn_decode if phase == 0 else dsa.dsa_sparse_attn_prefill
    a = attn_args(**over)
    # prefill needs no workspace; give decode exactly what it asks for unless
    # the test overrides it
    if phase == 0 and "workspace" not in over:
        need = dsa.dsa_attn_workspace_bytes(a["T"], a["H"], a["K"], 0) \
            if a["T"] > 0 and a["K"] > 0 and a["K"] % 128 == 0 else 0
        a["workspace"] = FAKE if need else None
        a["workspace_bytes"] = need
    return fn(**a)


def load_geometry():
    rows = []
    for line in open(os.path.join(GOLDEN, "geometry_table.txt")):
        parts = line.split("#")[0].split()
        if parts:
            rows.append((int(parts[0]), int(parts[1]), parts[4]))
    return rows


@pytest.mark.parametrize("phase", [0, 1])
@pytest.mark.parametrize("rank,rope,status", load_geometry())
def test_geometry_table(phase, rank, rope, status):
    want = getattr(dsa, status)
    got = call(phase, D=rank, rope_dim=rope, T=0)
    if want == dsa.DSA_OK:
        assert got == dsa.DSA_OK          # T = 0: validated, nothing to launch
    else:
        assert got == want, dsa.dsa_status_string(got)


REJECT = [
    (dict(D=576), "DSA_ERR_WIDTH_MISMATCH"),
    (dict(D=256), "DSA_ERR_WIDTH_MISMATCH"),
    (dict(rope_dim=64), "DSA_ERR_LAYOUT"),
    (dict(layout=dsa.DSA_KV_SCALED_FP8_656), "DSA_ERR_LAYOUT"),        # rope_dim 0
    (dict(layout=dsa.DSA_KV_SCALED_FP8_656, rope_dim=32), "DSA_ERR_LAYOUT"),
    (dict(layout=dsa.DSA_KV_SCALED_FP8_656, rope_dim=64, q_dtype=dsa.DSA_FP8_E4M3FN,
          q_scale=FAKE), "DSA_ERR_DTYPE"),                               # NoPE-only FP8 query
    (dict(layout=dsa.DSA_KV_BF16_1024, q_dtype=dsa.DSA_FP8_E4M3FN, q_scale=FAKE),
     "DSA_ERR_DTYPE"),                                                   # FP8 query, bf16 rows
    (dict(layout=dsa.DSA_KV_BF16_1024, rope_dim=64), "DSA_ERR_LAYOUT"),
    (dict(layout=9), "DSA_ERR_LAYOUT"),
    (dict(fp8_format=dsa.DSA_FP8_E4M3FNUZ), "DSA_ERR_DTYPE"),
    (dict(fp8_format=dsa.DSA_BF16), "DSA_ERR_DTYPE"),
    (dict(q_dtype=dsa.DSA_FP8_E4M3FNUZ), "DSA_ERR_DTYPE"),
    (dict(q_dtype=dsa.DSA_FP32), "DSA_ERR_DTYPE"),
    (dict(out_dtype=dsa.DSA_FP8_E4M3FN), "DSA_ERR_DTYPE"),
    (dict(K=100), "DSA_ERR_SHAPE"),
    (dict(K=0), "DSA_ERR_SHAPE"),
    (dict(K=2048 + 64), "DSA_ERR_SHAPE"),
    (dict(K=65536 + 128), "DSA_ERR_SHAPE"),
    (dict(H=0), "DSA_ERR_SHAPE"),
    (dict(H=129), "DSA_ERR_SHAPE"),
    (dict(T=-1), "DSA_ERR_SHAPE"),
    (dict(num_slots=-5), "DSA_ERR_SHAPE"),
    (dict(num_slots=1 << 31), "DSA_ERR_SHAPE"),    # slots are held as int32
    (dict(page_size=48), "DSA_ERR_SHAPE"),
    (dict(page_size=0), "DSA_ERR_SHAPE"),
    (dict(max_pages=0), "DSA_ERR_SHAPE"),
    (dict(num_seqs=0), "DSA_ERR_SHAPE"),
    (dict(num_seqs=3), "DSA_ERR_SHAPE"),       # T=4 tokens, token t -> seq t
    (dict(q=None), "DSA_ERR_NULL"),
    (dict(pool=None), "DSA_ERR_NULL"),
    (dict(topk=None), "DSA_ERR_NULL"),
    (dict(out=None), "DSA_ERR_NULL"),
    (dict(q_dtype=dsa.DSA_FP8_E4M3FN, q_scale=None), "DSA_ERR_NULL"),
    (dict(q=FAKE + 8), "DSA_ERR_ALIGN"),
    (dict(pool=FAKE + 4), "DSA_ERR_ALIGN"),
    (dict(out=FAKE + 2), "DSA_ERR_ALIGN"),
]


@pytest.mark.parametrize("phase", [0, 1])
@pytest.mark.parametrize("over,status", REJECT,
                         ids=[f"{list(o)[0]}={list(o.values())[0]}" for o, _ in REJECT])
def test_attention_rejections(phase, over, status):
    assert call(phase, **over) == getattr(dsa, status)


def test_decode_workspace_checks():
    need = dsa.dsa_attn_workspace_bytes(4, 16, 2048, 0)
    assert need > 0 and need % 256 == 0
    assert dsa.dsa_attn_workspace_bytes(4, 16, 2048, 1) == 0
    assert call(0, K=2048, workspace=None, workspace_bytes=0) == dsa.DSA_ERR_WORKSPACE
    assert call(0, K=2048, workspace=FAKE, workspace_bytes=need - 1) == dsa.DSA_ERR_WORKSPACE
    assert call(0, K=2048, workspace=FAKE + 16, workspace_bytes=need) == dsa.DSA_ERR_ALIGN
    assert dsa.dsa_attn_workspace_bytes(4, 16, 100, 0) == 0


def test_empty_batch_is_a_no_op():
    for phase in (0, 1):
        assert call(phase, T=0, q=None, pool=None, topk=None, out=None) == dsa.DSA_OK


def test_physical_indices_need_no_table():
    # no page table and no seq_lens: T may exceed num_seqs; validation passes
    # and the call stops at the device check (no GPU in this container)
    st = call(1, page_table=None, seq_lens=None, num_seqs=0, page_size=0,
              max_pages=0, T=8)
    assert st in (dsa.DSA_ERR_DEVICE, dsa.DSA_OK)


def test_valid_call_without_gpu_reports_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert call(1) == dsa.DSA_ERR_DEVICE


# ------------------------------------------------------------------ writer

def kv_args(**over):
    a = dict(kv=FAKE, n=8, kv_row_stride=512, kv_dtype=dsa.DSA_BF16, kv_dim=512,
             rope_dim=0, slot_mapping=FAKE, pool=FAKE, num_slots=64,
             layout=dsa.DSA_KV_RAW_FP8_512, fp8_format=dsa.DSA_FP8_E4M3FN,
             err_count=None, stream=0)
    a.update(over)
    return a


KV_REJECT = [
    (dict(kv_dim=576), "DSA_ERR_WIDTH_MISMATCH"),
    (dict(rope_dim=64), "DSA_ERR_LAYOUT"),
    (dict(layout=dsa.DSA_KV_SCALED_FP8_656), "DSA_ERR_LAYOUT"),        # rope_dim 0
    (dict(layout=dsa.DSA_KV_SCALED_FP8_656, rope_dim=64, kv_row_stride=512), "DSA_ERR_SHAPE"),
    (dict(fp8_format=dsa.DSA_FP8_E4M3FNUZ), "DSA_ERR_DTYPE"),
    (dict(kv_dtype=dsa.DSA_FP32), "DSA_ERR_DTYPE"),
    (dict(n=-1), "DSA_ERR_SHAPE"),
    (dict(kv_row_stride=256), "DSA_ERR_SHAPE"),
    (dict(num_slots=-1), "DSA_ERR_SHAPE"),
    (dict(kv=None), "DSA_ERR_NULL"),
    (dict(slot_mapping=None), "DSA_ERR_NULL"),
    (dict(pool=None), "DSA_ERR_NULL"),
    (dict(kv=FAKE + 2), "DSA_ERR_ALIGN"),
    (dict(pool=FAKE + 8), "DSA_ERR_ALIGN"),
    (dict(kv_row_stride=516), "DSA_ERR_ALIGN"),
]


@pytest.mark.parametrize("over,status", KV_REJECT,
                         ids=[f"{list(o)[0]}={list(o.values())[0]}" for o, _ in KV_REJECT])
def test_writer_rejections(over, status):
    assert dsa.dsa_kv_write(**kv_args(**over)) == getattr(dsa, status)


def test_writer_empty_is_a_no_op():
    assert dsa.dsa_kv_write(**kv_args(n=0, kv=None, pool=None, slot_mapping=None)) == 0


# ---------------------------------------------------------------- quantize

def test_quantize_rejections():
    q = dict(q=FAKE, n_elems=64, q_dtype=dsa.DSA_BF16, q8=FAKE, q_scale=FAKE,
             scale_given=0, fp8_format=dsa.DSA_FP8_E4M3FN, workspace=FAKE,
             workspace_bytes=dsa.dsa_quantize_q_workspace_bytes(64), stream=0)
    f = dsa.dsa_quantize_q_fp8
    assert f(**{**q, "fp8_format": dsa.DSA_FP8_E4M3FNUZ}) == dsa.DSA_ERR_DTYPE
    assert f(**{**q, "q_dtype": dsa.DSA_FP32}) == dsa.DSA_ERR_DTYPE
    assert f(**{**q, "n_elems": 60}) == dsa.DSA_ERR_SHAPE
    assert f(**{**q, "n_elems": -8}) == dsa.DSA_ERR_SHAPE
    assert f(**{**q, "q": None}) == dsa.DSA_ERR_NULL
    assert f(**{**q, "q_scale": None}) == dsa.DSA_ERR_NULL
    assert f(**{**q, "q8": FAKE + 1}) == dsa.DSA_ERR_ALIGN
    assert f(**{**q, "workspace": None}) == dsa.DSA_ERR_WORKSPACE
    assert f(**{**q, "workspace_bytes": 0}) == dsa.DSA_ERR_WORKSPACE
    assert f(**{**q, "n_elems": 0, "q": None}) == dsa.DSA_OK
    assert dsa.dsa_quantize_q_workspace_bytes(0) == 0
    assert dsa.dsa_quantize_q_workspace_bytes(8) == 4


# ------------------------------------------------------------------ build check

def transform_call(**over):
    args = dict(topk=FAKE, T=4, k_in=2048, page_table=FAKE, page_size=64,
                max_pages=128, num_seqs=4, token_seq=None, seq_lens=FAKE,
                num_slots=1 << 20, out_slots=FAKE, k_out=2048, valid_count=None,
                err_count=None, stream=0)
    args.update(over)
    return dsa.dsa_topk_transform(**args)


TRANSFORM_REJECT = [
    (dict(k_in=0), "DSA_ERR_SHAPE"),
    (dict(k_in=65537, k_out=65536), "DSA_ERR_SHAPE"),
    (dict(k_out=2000), "DSA_ERR_SHAPE"),          # not a multiple of 128
    (dict(k_in=1000, k_out=896), "DSA_ERR_SHAPE"),  # narrower than the input
    (dict(k_out=65536 + 128), "DSA_ERR_SHAPE"),
    (dict(T=-1), "DSA_ERR_SHAPE"),
    (dict(page_size=48), "DSA_ERR_SHAPE"),
    (dict(max_pages=0), "DSA_ERR_SHAPE"),
    (dict(num_seqs=0), "DSA_ERR_SHAPE"),
    (dict(T=5), "DSA_ERR_SHAPE"),                 # more tokens than sequences
    (dict(num_slots=-1), "DSA_ERR_SHAPE"),
    (dict(num_slots=1 << 31), "DSA_ERR_SHAPE"),
    (dict(topk=None), "DSA_ERR_NULL"),
    (dict(out_slots=None), "DSA_ERR_NULL"),
]


@pytest.mark.parametrize("over,status", TRANSFORM_REJECT,
                         ids=[str(o) for o, _ in TRANSFORM_REJECT])
def test_transform_rejections(over, status):
    assert transform_call(**over) == getattr(dsa, status)


def test_transform_accepts_any_input_width():
    # widths that are not multiples of 128 pass validation (the call then
    # stops at the device check: no GPU in this container)
    for k_in, k_out in ((1, 128), (100, 128), (1000, 1024), (2047, 2048), (3000, 4096)):
        assert transform_call(k_in=k_in, k_out=k_out) in (dsa.DSA_ERR_DEVICE, dsa.DSA_OK)
    assert transform_call(T=0, topk=None, out_slots=None) == dsa.DSA_OK


def test_build_rejects_kernels_that_use_scratch():
    """The build refuses kernels with spills or scratch: the attention kernel
    counts outstanding vector-memory operations to wait for its tile copies."""
    from sparse_mla_attention_gather_amd import build as B
    ok = ("x.hip:1:1: remark: Function Name: k_ok [-Rpass-analysis=kernel-resource-usage]\n"
          "x.hip:1:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]\n"
          "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]\n")
    bad = ("x.hip:9:1: remark: Function Name: k_bad [-Rpass-analysis=kernel-resource-usage]\n"
           "x.hip:9:1: remark:     VGPRs Spill: 3 [-Rpass-analysis=kernel-resource-usage]\n"
           "x.hip:9:1: remark:     ScratchSize [bytes/lane]: 16 [-Rpass-analysis=kernel-resource-usage]\n")
    assert B.scratch_users(ok) == []
    assert B.scratch_users(ok + bad) == [("k_bad", "VGPRs Spill", 3),
                                         ("k_bad", "ScratchSize [bytes/lane]", 16)]


def test_rope_layout_passes_validation():
    """656-byte rows with rope_dim 64 and a bf16 query (attention), or
    576-wide input rows (writer), pass every argument check: the calls stop
    at the device check (no GPU in this container)."""
    for phase in (0, 1):
        st = call(phase, layout=dsa.DSA_KV_SCALED_FP8_656, rope_dim=64)
        assert st in (dsa.DSA_ERR_DEVICE, dsa.DSA_OK), dsa.dsa_status_string(st)
    st = dsa.dsa_kv_write(**kv_args(layout=dsa.DSA_KV_SCALED_FP8_656, rope_dim=64,
                                    kv_row_stride=576))
    assert st in (dsa.DSA_ERR_DEVICE, dsa.DSA_OK), dsa.dsa_status_string(st)


def test_bf16_layout_passes_validation():
    for phase in (0, 1):
        st = call(phase, layout=dsa.DSA_KV_BF16_1024)
        assert st in (dsa.DSA_ERR_DEVICE, dsa.DSA_OK), dsa.dsa_status_string(st)
    st = dsa.dsa_kv_write(**kv_args(layout=dsa.DSA_KV_BF16_1024))
    assert st in (dsa.DSA_ERR_DEVICE, dsa.DSA_OK), dsa.dsa_status_string(st)


# ------------------------------------------------ allocation-free decode

def noalloc(**over):
    a = attn_args(**over)
    a.pop("workspace")
    a.pop("workspace_bytes")
    return dsa.dsa_sparse_attn_decode_noalloc(**a)


def test_noalloc_limit_and_rejections():
    """The allocation-free decode checks its arguments like the decode and
    refuses, before any launch, a call whose split partials exceed its
    32 MiB scratch (here 64 tokens x 16 heads x 32 splits of a 65536-wide
    top-k list: 67 MB)."""
    assert dsa.DSA_DECODE_SCRATCH_BYTES == 32 << 20
    need = dsa.dsa_attn_workspace_bytes(64, 16, 65536, 0)
    assert need > dsa.DSA_DECODE_SCRATCH_BYTES
    assert noalloc(T=64, H=16, K=65536, num_seqs=64) == dsa.DSA_ERR_WORKSPACE
    # every top-k width up to 2048 fits, at any batch, on 256 CUs
    for T, H in [(1, 16), (255, 16), (255, 32), (63, 128), (127, 32)]:
        assert dsa.dsa_attn_workspace_bytes(T, H, 2048, 0) <= dsa.DSA_DECODE_SCRATCH_BYTES
    assert noalloc(D=511) == dsa.DSA_ERR_WIDTH_MISMATCH
    assert noalloc(K=100) == dsa.DSA_ERR_SHAPE
    assert noalloc(out=FAKE + 2) == dsa.DSA_ERR_ALIGN
    assert noalloc(T=0, q=None, pool=None, topk=None, out=None) == dsa.DSA_OK


def test_noalloc_without_gpu_reports_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert noalloc(K=2048) == dsa.DSA_ERR_DEVICE
