"""The C ABI library: loads, exports what the header declares, rejects bad
arguments on the host (CPU only: no call here reaches a kernel)."""

import ctypes
import pathlib
import re

import pytest

import paged_kv_cache_map_amd as pkv

HEADER = pathlib.Path(__file__).resolve().parent.parent / "include" / "pkv.h"


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_calls():
    names = declared_functions()
    for want in ("pkv_kv_cache_write", "pkv_paged_decode", "pkv_paged_decode_append",
                 "pkv_paged_decode_noalloc",
                 "pkv_varlen_prefill", "pkv_paged_decode_workspace_size", "pkv_last_error",
                 "pkv_version", "pkv_copy_blocks", "pkv_block_manager_create",
                 "pkv_block_manager_append_slot", "pkv_block_hash"):
        assert want in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(str(pkv.LIB_PATH))
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version():
    assert "gfx950" in pkv.version()


NULL = None
FAKE = ctypes.c_void_p(0x1000)      # never dereferenced: every case fails validation first
ODD = ctypes.c_void_p(0x1008)       # not 16-byte aligned


def write(**kw):
    args = dict(k=FAKE, ks=1024, v=FAKE, vs=1024, src=pkv.BF16, kc=FAKE, vc=FAKE, cdt=pkv.BF16,
                slots=100, ksc=NULL, vsc=NULL, sm=FAKE, t=3, hkv=8, d=128, stream=NULL)
    args.update(kw)
    return pkv.library().pkv_kv_cache_write(
        args["k"], args["ks"], args["v"], args["vs"], args["src"], args["kc"], args["vc"], args["cdt"],
        args["slots"], args["ksc"], args["vsc"], args["sm"], args["t"], args["hkv"], args["d"],
        args["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(t=-1), pkv.ERR_INVALID),
    (dict(ks=1023), pkv.ERR_INVALID),                 # token stride below the row width
    (dict(k=NULL), pkv.ERR_INVALID),
    (dict(sm=NULL), pkv.ERR_INVALID),
    (dict(cdt=pkv.FP8_E4M3), pkv.ERR_INVALID),        # fp8 without scales
    (dict(src=pkv.F32, cdt=pkv.BF16), pkv.ERR_UNSUPPORTED),
    (dict(d=96), pkv.ERR_UNSUPPORTED),
    (dict(k=ODD), pkv.ERR_INVALID),
    (dict(ks=1028), pkv.ERR_INVALID),                 # 2056-byte stride is not 16-byte aligned
    (dict(hkv=0), pkv.ERR_INVALID),
])
def test_write_rejects(kw, code):
    assert write(**kw) == code
    assert pkv.library().pkv_last_error()


def test_write_zero_tokens_is_a_no_op():
    assert write(t=0, sm=NULL) == pkv.OK


def decode(**kw):
    a = dict(out=FAKE, q=FAKE, qdt=pkv.BF16, kc=FAKE, vc=FAKE, cdt=pkv.BF16, ksc=NULL, vsc=NULL,
             bt=FAKE, maxblk=4, sl=FAKE, b=3, hq=8, hkv=2, d=128, bs=16, nb=10, scale=0.1, split=0,
             ws=FAKE, wsb=1 << 30, stream=NULL)
    a.update(kw)
    return pkv.library().pkv_paged_decode(
        a["out"], a["q"], a["qdt"], a["kc"], a["vc"], a["cdt"], a["ksc"], a["vsc"], a["bt"],
        a["maxblk"], a["sl"], a["b"], a["hq"], a["hkv"], a["d"], a["bs"], a["nb"], a["scale"],
        a["split"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(b=0), pkv.ERR_INVALID),
    (dict(hq=6, hkv=4), pkv.ERR_INVALID),
    (dict(hq=24, hkv=1), pkv.ERR_UNSUPPORTED),        # group of 24
    (dict(q=NULL), pkv.ERR_INVALID),
    (dict(bt=NULL), pkv.ERR_INVALID),
    (dict(d=80), pkv.ERR_UNSUPPORTED),
    (dict(bs=12), pkv.ERR_UNSUPPORTED),
    (dict(bs=512), pkv.ERR_UNSUPPORTED),
    (dict(qdt=pkv.F32), pkv.ERR_UNSUPPORTED),         # fp32 q with a bf16 cache
    (dict(cdt=pkv.FP8_E4M3), pkv.ERR_INVALID),        # fp8 without scales
    (dict(split=100), pkv.ERR_INVALID),               # not a multiple of 128
    (dict(split=128, maxblk=64, wsb=0, ws=NULL), pkv.ERR_INVALID),   # workspace too small
    (dict(out=ODD), pkv.ERR_INVALID),
    (dict(maxblk=1 << 24, bs=256), pkv.ERR_INVALID),  # key positions past 2^31 - 1
    (dict(maxblk=(1 << 27) + 1, bs=16), pkv.ERR_INVALID),
])
def test_decode_rejects(kw, code):
    assert decode(**kw) == code


def decode_noalloc(**kw):
    a = dict(out=FAKE, q=FAKE, qdt=pkv.BF16, kc=FAKE, vc=FAKE, cdt=pkv.BF16, ksc=NULL, vsc=NULL,
             bt=FAKE, maxblk=4, sl=FAKE, b=3, hq=8, hkv=2, d=128, bs=16, nb=10, scale=0.1, split=0,
             stream=NULL)
    a.update(kw)
    return pkv.library().pkv_paged_decode_noalloc(
        a["out"], a["q"], a["qdt"], a["kc"], a["vc"], a["cdt"], a["ksc"], a["vsc"], a["bt"],
        a["maxblk"], a["sl"], a["b"], a["hq"], a["hkv"], a["d"], a["bs"], a["nb"], a["scale"],
        a["split"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(b=0), pkv.ERR_INVALID),
    (dict(q=NULL), pkv.ERR_INVALID),
    (dict(d=80), pkv.ERR_UNSUPPORTED),
    (dict(cdt=pkv.FP8_E4M3), pkv.ERR_INVALID),        # fp8 without scales
    (dict(split=100), pkv.ERR_INVALID),
    (dict(maxblk=1 << 24, bs=256), pkv.ERR_INVALID),  # key positions past 2^31 - 1
    # stream-K plan at batch 2048, 8 KV heads, G = 4: (4096 + 16384) partial
    # slots x 4 heads x 130 floats = 42.6 MB, above the 32 MiB array
    (dict(b=2048, hq=32, hkv=8), pkv.ERR_INVALID),
    # fixed splits of 128 keys over 4096-key tables: 64 x 32 x 32 x 130 floats
    (dict(b=64, hq=32, hkv=8, maxblk=256, split=128), pkv.ERR_INVALID),
])
def test_decode_noalloc_rejects(kw, code):
    assert decode_noalloc(**kw) == code
    assert b"paged_decode_noalloc" in pkv.library().pkv_last_error()


def test_decode_noalloc_limit_is_the_workspace_size():
    """The no-alloc decode takes exactly the sizes whose workspace fits the
    static array: the rejection above is the size rule, not another check."""
    limit = pkv.NOALLOC_SCRATCH_BYTES
    assert limit == 32 << 20
    assert pkv.paged_decode_workspace_size(2048, 32, 8, 128, 16, 4, 0) > limit
    assert pkv.paged_decode_workspace_size(64, 32, 8, 128, 16, 256, 128) > limit
    assert 0 < pkv.paged_decode_workspace_size(256, 32, 8, 128, 16, 1017, 0) <= limit
    assert 0 < pkv.paged_decode_workspace_size(8, 64, 8, 128, 16, 8193, 0) <= limit
    text = HEADER.read_text()
    assert "#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)" in text


def append(**kw):
    a = dict(out=FAKE, q=FAKE, qdt=pkv.BF16, kn=FAKE, kns=256, vn=FAKE, vns=256, kc=FAKE, vc=FAKE,
             cdt=pkv.BF16, ksc=NULL, vsc=NULL, bt=FAKE, maxblk=4, sl=FAKE, b=3, hq=8, hkv=2, d=128,
             bs=16, nb=10, scale=0.1, split=0, ws=FAKE, wsb=1 << 30, stream=NULL)
    a.update(kw)
    return pkv.library().pkv_paged_decode_append(
        a["out"], a["q"], a["qdt"], a["kn"], a["kns"], a["vn"], a["vns"], a["kc"], a["vc"], a["cdt"],
        a["ksc"], a["vsc"], a["bt"], a["maxblk"], a["sl"], a["b"], a["hq"], a["hkv"], a["d"], a["bs"],
        a["nb"], a["scale"], a["split"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(kn=NULL), pkv.ERR_INVALID),
    (dict(vn=NULL), pkv.ERR_INVALID),
    (dict(kns=255), pkv.ERR_INVALID),                 # stride below the row width 2 x 128
    (dict(vns=260), pkv.ERR_INVALID),                 # 520-byte stride is not 16-byte aligned
    (dict(kn=ODD), pkv.ERR_INVALID),
    (dict(b=0), pkv.ERR_INVALID),
    (dict(d=80), pkv.ERR_UNSUPPORTED),
    (dict(cdt=pkv.FP8_E4M3), pkv.ERR_INVALID),        # fp8 without scales
    (dict(qdt=pkv.F32), pkv.ERR_UNSUPPORTED),         # fp32 q and new rows with a bf16 cache
    (dict(split=100), pkv.ERR_INVALID),
    (dict(split=128, maxblk=64, wsb=0, ws=NULL), pkv.ERR_INVALID),
    (dict(maxblk=1 << 24, bs=256), pkv.ERR_INVALID),  # key positions past 2^31 - 1
])
def test_append_rejects(kw, code):
    assert append(**kw) == code
    assert b"paged_decode_append" in pkv.library().pkv_last_error()


def copy_blocks(**kw):
    a = dict(kc=FAKE, vc=FAKE, cdt=pkv.BF16, nb=10, bs=16, hkv=8, d=128, pairs=FAKE, n=3, stream=NULL)
    a.update(kw)
    return pkv.library().pkv_copy_blocks(a["kc"], a["vc"], a["cdt"], a["nb"], a["bs"], a["hkv"], a["d"],
                                         a["pairs"], a["n"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(n=-1), pkv.ERR_INVALID),
    (dict(nb=0), pkv.ERR_INVALID),
    (dict(kc=NULL), pkv.ERR_INVALID),
    (dict(pairs=NULL), pkv.ERR_INVALID),
    (dict(vc=ODD), pkv.ERR_INVALID),
    (dict(cdt=7), pkv.ERR_UNSUPPORTED),
    (dict(cdt=pkv.FP8_E4M3, bs=1, hkv=1, d=8), pkv.ERR_UNSUPPORTED),   # an 8-byte block
])
def test_copy_blocks_rejects(kw, code):
    assert copy_blocks(**kw) == code
    assert b"copy_blocks" in pkv.library().pkv_last_error()


def test_copy_blocks_no_pairs_is_a_no_op():
    assert copy_blocks(n=0, pairs=NULL) == pkv.OK


def prefill(**kw):
    a = dict(out=FAKE, q=FAKE, qdt=pkv.BF16, k=FAKE, v=FAKE, kdt=pkv.BF16, ksc=NULL, vsc=NULL,
             cq=FAKE, ck=FAKE, b=3, mq=10, mk=10, scale=0.1, causal=1, bt=NULL, maxblk=0, bs=0, nb=0,
             hq=8, hkv=2, d=128, tq=14, tk=8, stream=NULL)
    a.update(kw)
    return pkv.library().pkv_varlen_prefill(
        a["out"], a["q"], a["qdt"], a["k"], a["v"], a["kdt"], a["ksc"], a["vsc"], a["cq"], a["ck"],
        a["b"], a["mq"], a["mk"], a["scale"], a["causal"], a["bt"], a["maxblk"], a["bs"], a["nb"],
        a["hq"], a["hkv"], a["d"], a["tq"], a["tk"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(causal=2), pkv.ERR_INVALID),
    (dict(bt=FAKE, maxblk=1 << 24, bs=256, nb=10), pkv.ERR_INVALID),  # key positions past 2^31 - 1
    (dict(bt=FAKE, maxblk=(1 << 27) + 1, bs=16, nb=10), pkv.ERR_INVALID),
    (dict(mq=-1), pkv.ERR_INVALID),
    (dict(hq=9, hkv=2), pkv.ERR_INVALID),
    (dict(kdt=pkv.FP8_E4M3, ksc=FAKE, vsc=FAKE), pkv.ERR_UNSUPPORTED),   # fp8 needs the paged cache
    (dict(bt=FAKE, maxblk=4, bs=24, nb=8), pkv.ERR_UNSUPPORTED),
    (dict(bt=FAKE, maxblk=0, bs=16, nb=8), pkv.ERR_INVALID),
    (dict(qdt=pkv.F32), pkv.ERR_UNSUPPORTED),
    (dict(d=32), pkv.ERR_UNSUPPORTED),
    (dict(cq=NULL), pkv.ERR_INVALID),
    (dict(q=ODD), pkv.ERR_INVALID),
])
def test_prefill_rejects(kw, code):
    assert prefill(**kw) == code


def test_prefill_empty_batch_is_a_no_op():
    assert prefill(b=0) == pkv.OK
    assert prefill(mq=0) == pkv.OK


def test_decode_workspace_plan():
    # automatic plan (stream-K): one partial slot per wave bound (4096) and per
    # (sequence, KV head) unit, each holding (D + 2) floats per q head of the
    # unit, then the batch's chunk prefix (batch + 1 int32)
    assert pkv.paged_decode_workspace_size(3, 8, 2, 64, 32, 4) == (4096 + 3 * 2) * 4 * 66 * 4 + 4 * 4
    # an explicit split covering the whole sequence needs no merge workspace
    assert pkv.paged_decode_workspace_size(3, 8, 2, 64, 32, 4, 128) == 0
    # explicit split of 128 keys over 64 blocks of 16 -> 8 splits of (D + 2) floats per (b, h)
    assert pkv.paged_decode_workspace_size(3, 8, 2, 128, 16, 64, 128) == 3 * 8 * 8 * 130 * 4
    # G = 16: the size covers both automatic plans; the matrix-core plan (bf16
    # caches: one unit of 16 heads per KV head) needs more than the vector one
    # (four head groups of 4 per KV head)
    mfma = (4096 + 2 * 2) * 16 * 130 * 4 + 3 * 4
    valu = (4096 + 2 * 2 * 4) * 4 * 130 * 4 + 3 * 4
    assert pkv.paged_decode_workspace_size(2, 32, 2, 128, 16, 8) == max(mfma, valu)
    # unsupported argument -> 0
    assert pkv.paged_decode_workspace_size(3, 8, 3, 128, 16, 4) == 0


def test_decode_workspace_plan_in_slices():
    """A batch over 2048 (one launch's chunk-count table) runs the stream plan
    in equal slices that share one workspace: the size is that of one slice."""
    def stream(b, hq, hkv, d):
        return (4096 + b * hkv) * (hq // hkv) * (d + 2) * 4 + (b + 1) * 4
    assert pkv.paged_decode_workspace_size(2048, 8, 2, 128, 16, 4) == stream(2048, 8, 2, 128)
    assert pkv.paged_decode_workspace_size(2049, 8, 2, 128, 16, 4) == stream(1025, 8, 2, 128)
    assert pkv.paged_decode_workspace_size(4096, 8, 2, 128, 16, 4) == stream(2048, 8, 2, 128)
    assert pkv.paged_decode_workspace_size(4100, 8, 2, 128, 16, 4) == stream(1367, 8, 2, 128)
    assert pkv.paged_decode_workspace_size(65535, 32, 8, 64, 16, 4) == stream(2048, 32, 8, 64)


def mixed(**kw):
    a = dict(kc=FAKE, vc=FAKE, cdt=pkv.FP8_E4M3, ksc=FAKE, vsc=FAKE, nb=10, bs=16, hq=8, hkv=2, d=128, scale=0.1,
             qdt=pkv.BF16, pout=FAKE, pq=FAKE, cq=FAKE, ck=FAKE, pb=2, mq=10, mk=10, pbt=FAKE, pmax=4, tq=12,
             dout=FAKE, dq=FAKE, dbt=FAKE, dmax=4, sl=FAKE, db=3, ws=FAKE, wsb=1 << 30, stream=NULL)
    a.update(kw)
    return pkv.library().pkv_mixed_attention(
        a["kc"], a["vc"], a["cdt"], a["ksc"], a["vsc"], a["nb"], a["bs"], a["hq"], a["hkv"], a["d"], a["scale"],
        a["qdt"], a["pout"], a["pq"], a["cq"], a["ck"], a["pb"], a["mq"], a["mk"], a["pbt"], a["pmax"], a["tq"],
        a["dout"], a["dq"], a["dbt"], a["dmax"], a["sl"], a["db"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(pb=-1), pkv.ERR_INVALID),
    (dict(pbt=NULL), pkv.ERR_INVALID),                # the prefill reads the paged cache
    (dict(ksc=NULL), pkv.ERR_INVALID),                # one-byte cache without scales
    (dict(dq=NULL), pkv.ERR_INVALID),
    (dict(d=96), pkv.ERR_UNSUPPORTED),
    (dict(qdt=pkv.F32), pkv.ERR_UNSUPPORTED),
    (dict(wsb=0, ws=NULL), pkv.ERR_INVALID),          # decode workspace too small
])
def test_mixed_rejects(kw, code):
    assert mixed(**kw) == code
    assert pkv.library().pkv_last_error()


def test_mixed_nothing_to_do_is_a_no_op():
    assert mixed(pb=0, db=0) == pkv.OK
