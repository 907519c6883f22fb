"""Host side of the C ABI (no GPU): the library loads, exports every symbol
the header declares, and rejects bad arguments before any launch."""
import os
import re

import pytest

import paged_kv_attention_24_amd as pka

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "pka.h")

# fake, 256-byte aligned, never dereferenced: every call below fails validation
FAKE = 0x10000


def _no_gpu_visible():
    import torch

    return torch.cuda.device_count() == 0  # counts devices without initialising one


# Calls with fake pointers run only where no GPU is visible: should a case
# ever pass validation, it must not reach a device.
fake_pointers = pytest.mark.skipif(not _no_gpu_visible(),
                                   reason="fake-pointer ABI checks run on hosts without a GPU")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pka_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    lib = pka.load_library()
    names = declared_functions()
    assert len(names) >= 7, names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in pka.h but not exported"


def test_abi_version_and_strings():
    lib = pka.load_library()
    assert lib.pka_abi_version() == 8
    assert lib.pka_status_string(0) == b"ok"
    assert lib.pka_status_string(3) == b"workspace too small"
    assert lib.pka_status_string(99) == b"unknown status"


def write(**over):
    args = dict(k=FAKE, v=FAKE, ks=512, vs=512, slots=FAKE, T=4, kc=FAKE, vc=FAKE, NB=10,
                bs=16, H=8, D=64, dt=1)
    args.update(over)
    lib = pka.load_library()
    st = lib.pka_kv_cache_write(args["k"], args["v"], args["ks"], args["vs"], args["slots"],
                                args["T"], args["kc"], args["vc"], args["NB"], args["bs"],
                                args["H"], args["D"], args["dt"], None)
    return st, lib.pka_last_error().decode()


@fake_pointers
@pytest.mark.parametrize("over,status", [
    (dict(T=-1), 1), (dict(dt=7), 1), (dict(NB=0), 1), (dict(H=0), 1),
    (dict(D=96), 2), (dict(bs=8), 2), (dict(kc=None), 1), (dict(vc=FAKE + 8), 1),
    (dict(k=None), 1), (dict(slots=None), 1), (dict(ks=511), 1), (dict(vs=100), 1),
    (dict(k=FAKE + 4), 1), (dict(ks=516), 1),
])
def test_write_rejects(over, status):
    st, msg = write(**over)
    assert st == status, (over, st, msg)
    assert msg


@fake_pointers
def test_write_zero_tokens_is_ok_without_launch():
    st, _ = write(T=0, k=None, v=None, slots=None)
    assert st == 0


def decode(**over):
    # maxl 2048: several partitions, so a workspace is required (every case
    # below must fail validation before any launch)
    a = dict(out=FAKE, odt=0, q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, MB=128, cl=FAKE, B=16, Hq=32,
             Hkv=8, D=64, NB=1000, bs=16, scale=0.125, kdt=1, maxl=2048, P=0, ws=FAKE,
             wsb=1 << 30)
    a.update(over)
    lib = pka.load_library()
    st = lib.pka_paged_attention_decode(a["out"], a["odt"], a["q"], a["kc"], a["vc"], a["bt"],
                                        a["MB"], a["cl"], a["B"], a["Hq"], a["Hkv"], a["D"],
                                        a["NB"], a["bs"], a["scale"], a["kdt"], a["maxl"], a["P"],
                                        a["ws"], a["wsb"], None)
    return st, lib.pka_last_error().decode()


@fake_pointers
@pytest.mark.parametrize("over,status", [
    (dict(kdt=5), 1), (dict(odt=2), 1), (dict(Hq=30), 1), (dict(Hkv=0), 1), (dict(NB=0), 1),
    (dict(MB=0), 1), (dict(B=-1), 1), (dict(D=80), 2), (dict(bs=64), 2), (dict(Hq=128), 2),
    (dict(Hq=24), 2), (dict(scale=float("nan")), 1), (dict(scale=float("inf")), 1), (dict(scale=float("-inf")), 1), (dict(P=24), 1), (dict(P=-16), 1),
    (dict(q=None), 1), (dict(out=FAKE + 2), 1), (dict(ws=None), 3),
    (dict(wsb=100), 3), (dict(ws=FAKE + 16), 1), (dict(B=70000), 2), (dict(cl=None), 1),
])
def test_decode_rejects(over, status):
    st, msg = decode(**over)
    assert st == status, (over, st, msg)
    assert msg


def decode_noalloc(**over):
    a = dict(out=FAKE, odt=0, q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, MB=128, cl=FAKE, B=16, Hq=32,
             Hkv=8, D=64, NB=1000, bs=16, scale=0.125, kdt=1, maxl=2048, P=0)
    a.update(over)
    lib = pka.load_library()
    st = lib.pka_paged_attention_decode_noalloc(
        a["out"], a["odt"], a["q"], a["kc"], a["vc"], a["bt"], a["MB"], a["cl"], a["B"], a["Hq"],
        a["Hkv"], a["D"], a["NB"], a["bs"], a["scale"], a["kdt"], a["maxl"], a["P"], None)
    return st, lib.pka_last_error().decode()


@fake_pointers
@pytest.mark.parametrize("over,status", [
    (dict(kdt=5), 1), (dict(odt=2), 1), (dict(Hq=30), 1), (dict(Hkv=0), 1), (dict(NB=0), 1),
    (dict(MB=0), 1), (dict(B=-1), 1), (dict(D=80), 2), (dict(bs=64), 2), (dict(Hq=24), 2),
    (dict(scale=float("nan")), 1), (dict(scale=float("inf")), 1), (dict(scale=float("-inf")), 1), (dict(P=24), 1), (dict(q=None), 1), (dict(out=FAKE + 2), 1),
    (dict(B=70000), 2), (dict(cl=None), 1),
])
def test_decode_noalloc_rejects(over, status):
    # the arguments are checked before the static scratch is touched
    st, msg = decode_noalloc(**over)
    assert st == status, (over, st, msg)
    assert msg


@fake_pointers
def test_decode_noalloc_empty_batch_is_ok_without_launch():
    st, _ = decode_noalloc(B=0, out=None, q=None)
    assert st == 0


def test_static_scratch_covers_every_supported_shape():
    # the no-allocation decode's scratch holds the largest workspace of any
    # supported shape on a GPU of 256 compute units
    if not _no_gpu_visible():
        pytest.skip("the grid depends on the visible GPU")
    limit = 22 << 20
    for D in (64, 128):
        for G in (1, 2, 4, 8):
            assert pka.decode_workspace_bytes(4096, 8 * G, 8, D) <= limit, (D, G)


@fake_pointers
def test_decode_empty_batch_is_ok_without_launch():
    st, _ = decode(B=0, out=None, q=None)
    assert st == 0


def test_partition_heuristic():
    # the default smallest share of one decode wave: 64 tokens, in whole blocks
    for B, H, bs, L in [(16, 8, 16, 1024), (64, 8, 16, 4096), (128, 8, 16, 8192),
                        (256, 8, 32, 32768), (1, 1, 32, 5), (4096, 8, 16, 100)]:
        assert pka.decode_partition_size(B, H, bs, L) == 64, (B, H, bs, L)


def r256(x):
    return (x + 255) // 256 * 256


def test_workspace_bytes():
    # 4 MiB of report counters, then two partial slots per wave of the grid
    # (256 compute units x 2 workgroups x 4 waves where no GPU is visible),
    # each G * D output floats plus 2 G (max, sum) floats padded to 4
    if not _no_gpu_visible():
        pytest.skip("the grid depends on the visible GPU")
    waves = 256 * 2 * 4
    assert pka.decode_workspace_bytes(16, 32, 8, 64) == (4 << 20) + r256(2 * waves * (4 * 64 + 8) * 4)
    assert pka.decode_workspace_bytes(4096, 16, 8, 128) == (4 << 20) + r256(2 * waves * (2 * 128 + 4) * 4)
    assert pka.decode_workspace_bytes(0, 32, 8, 64) == 0


def test_python_binding_refuses_cpu_tensors():
    import torch

    kc = torch.zeros(4, 2, 16, 64)
    with pytest.raises(ValueError):
        pka.kv_cache_write(torch.zeros(1, 2, 64), torch.zeros(1, 2, 64),
                           torch.zeros(1, dtype=torch.int64), kc, kc.clone())
    with pytest.raises(ValueError):
        pka.paged_attention_decode(torch.zeros(1, 4, 64), kc, kc, torch.zeros(1, 1, dtype=torch.int32),
                                   torch.ones(1, dtype=torch.int32), 0.125, 2, 16)


def append(**over):
    # maxl 2048: several partitions, so a workspace is required (every case
    # below must fail validation before any launch)
    a = dict(out=FAKE, odt=0, q=FAKE, kn=FAKE, vn=FAKE, ks=512, vs=512, sl=FAKE, kc=FAKE,
             vc=FAKE, bt=FAKE, MB=128, cl=FAKE, B=16, Hq=32, Hkv=8, D=64, NB=1000, bs=16,
             scale=0.125, kdt=1, maxl=2048, P=0, ws=FAKE, wsb=1 << 30)
    a.update(over)
    lib = pka.load_library()
    st = lib.pka_paged_attention_decode_append(
        a["out"], a["odt"], a["q"], a["kn"], a["vn"], a["ks"], a["vs"], a["sl"], a["kc"],
        a["vc"], a["bt"], a["MB"], a["cl"], a["B"], a["Hq"], a["Hkv"], a["D"], a["NB"], a["bs"],
        a["scale"], a["kdt"], a["maxl"], a["P"], a["ws"], a["wsb"], None)
    return st, lib.pka_last_error().decode()


@fake_pointers
@pytest.mark.parametrize("over,status", [
    (dict(kn=None), 1), (dict(vn=None), 1), (dict(sl=None), 1), (dict(ks=511), 1),
    (dict(vs=8), 1), (dict(kn=FAKE + 4), 1), (dict(ks=516), 1), (dict(D=96), 2),
    (dict(kdt=9), 1), (dict(Hq=12), 1), (dict(P=24), 1), (dict(ws=None), 3),
])
def test_append_rejects(over, status):
    st, msg = append(**over)
    assert st == status, (over, st, msg)
    assert msg


def prefill(**over):
    a = dict(out=FAKE, odt=0, q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, MB=64, cl=FAKE, qs=FAKE, B=8,
             N=2048, maxq=256, Hq=32, Hkv=8, D=64, NB=1000, bs=16, scale=0.125, kdt=1)
    a.update(over)
    lib = pka.load_library()
    st = lib.pka_paged_attention_prefill(a["out"], a["odt"], a["q"], a["kc"], a["vc"], a["bt"],
                                         a["MB"], a["cl"], a["qs"], a["B"], a["N"], a["maxq"],
                                         a["Hq"], a["Hkv"], a["D"], a["NB"], a["bs"], a["scale"],
                                         a["kdt"], None)
    return st, lib.pka_last_error().decode()


@fake_pointers
@pytest.mark.parametrize("over,status", [
    (dict(kdt=0), 2), (dict(kdt=5), 1), (dict(odt=2), 1), (dict(Hq=30), 1), (dict(Hkv=0), 1),
    (dict(NB=0), 1), (dict(MB=0), 1), (dict(B=-1), 1), (dict(N=-1), 1), (dict(D=96), 2),
    (dict(bs=8), 2), (dict(Hq=128), 2), (dict(scale=float("nan")), 1), (dict(scale=float("inf")), 1), (dict(scale=float("-inf")), 1), (dict(q=None), 1),
    (dict(qs=None), 1), (dict(cl=None), 1), (dict(out=FAKE + 4), 1), (dict(kc=FAKE + 8), 1),
    (dict(B=70000), 2),
])
def test_prefill_rejects(over, status):
    st, msg = prefill(**over)
    assert st == status, (over, st, msg)
    assert msg


@fake_pointers
def test_prefill_empty_is_ok_without_launch():
    assert prefill(B=0, out=None, q=None)[0] == 0
    assert prefill(N=0, out=None, q=None)[0] == 0


@fake_pointers
@pytest.mark.parametrize("fn", ["copy", "gather", "scatter"])
@pytest.mark.parametrize("over,status", [
    (dict(n=-1), 1), (dict(nb=0), 1), (dict(bb=0), 1), (dict(bb=1000), 1), (dict(ids=None), 1),
    (dict(kc=None), 1), (dict(kc=FAKE + 8), 1), (dict(bb=1 << 40), 2),
])
def test_block_moves_reject(fn, over, status):
    a = dict(kc=FAKE, vc=FAKE, pk=FAKE, ids=FAKE, n=4, nb=10, bb=16384)
    a.update(over)
    lib = pka.load_library()
    if fn == "copy":
        st = lib.pka_copy_blocks(a["kc"], a["vc"], a["ids"], a["n"], a["nb"], a["bb"], None)
    elif fn == "gather":
        st = lib.pka_gather_blocks(a["pk"], a["kc"], a["vc"], a["ids"], a["n"], a["nb"], a["bb"],
                                   None)
    else:
        st = lib.pka_scatter_blocks(a["kc"], a["vc"], a["pk"], a["ids"], a["n"], a["nb"], a["bb"],
                                    None)
    assert st == status, (fn, over, st)
    assert lib.pka_last_error()


@fake_pointers
def test_block_moves_need_the_packed_buffer():
    lib = pka.load_library()
    assert lib.pka_gather_blocks(None, FAKE, FAKE, FAKE, 4, 10, 16384, None) == 1
    assert lib.pka_scatter_blocks(FAKE, FAKE, None, FAKE, 4, 10, 16384, None) == 1
    assert lib.pka_copy_blocks(FAKE, FAKE, FAKE, 0, 10, 16384, None) == 0  # nothing to do


def rope(**over):
    a = dict(k=FAKE, v=FAKE, ks=512, vs=512, slots=FAKE, pos=FAKE, T=4, cs=FAKE, maxp=4096,
             R=64, kc=FAKE, vc=FAKE, NB=10, bs=16, H=8, D=64, dt=1)
    a.update(over)
    lib = pka.load_library()
    st = lib.pka_kv_cache_write_rope(a["k"], a["v"], a["ks"], a["vs"], a["slots"], a["pos"],
                                     a["T"], a["cs"], a["maxp"], a["R"], a["kc"], a["vc"], a["NB"],
                                     a["bs"], a["H"], a["D"], a["dt"], None)
    return st, lib.pka_last_error().decode()


@fake_pointers
@pytest.mark.parametrize("over,status", [
    (dict(R=0), 1), (dict(R=66), 1), (dict(R=24), 1), (dict(R=128), 1), (dict(maxp=0), 1),
    (dict(pos=None), 1), (dict(cs=None), 1), (dict(slots=None), 1), (dict(T=-1), 1),
    (dict(dt=7), 1), (dict(D=96, R=32), 2), (dict(bs=8), 2), (dict(kc=None), 1),
    (dict(ks=100), 1), (dict(k=FAKE + 4), 1),
])
def test_rope_write_rejects(over, status):
    st, msg = rope(**over)
    assert st == status, (over, st, msg)
    assert msg


@fake_pointers
def test_rope_write_fp32_allows_rotary_multiples_of_8():
    assert rope(dt=0, R=24, T=0)[0] == 0   # fp32: 4 elements per 16 bytes -> multiples of 8
    assert rope(dt=1, R=24, T=0)[0] == 1   # fp16: multiples of 16


def write_int8(**over):
    args = dict(k=FAKE, v=FAKE, ks=512, vs=512, dt=1, slots=FAKE, T=4, kc=FAKE, vc=FAKE,
                ksc=FAKE, vsc=FAKE, NB=10, bs=16, H=8, D=64, gs=32)
    args.update(over)
    lib = pka.load_library()
    st = lib.pka_kv_cache_write_int8(args["k"], args["v"], args["ks"], args["vs"], args["dt"],
                                     args["slots"], args["T"], args["kc"], args["vc"],
                                     args["ksc"], args["vsc"], args["NB"], args["bs"], args["H"],
                                     args["D"], args["gs"], None)
    return st, lib.pka_last_error().decode()


@fake_pointers
@pytest.mark.parametrize("over,status", [
    (dict(T=-1), 1), (dict(dt=7), 1), (dict(NB=0), 1), (dict(H=0), 1), (dict(D=96), 2),
    (dict(bs=8), 2), (dict(gs=16), 2), (dict(gs=128), 2), (dict(kc=None), 1),
    (dict(vsc=FAKE + 4), 1), (dict(k=None), 1), (dict(slots=None), 1), (dict(ks=511), 1),
    (dict(k=FAKE + 1), 1),
])
def test_write_int8_rejects(over, status):
    st, msg = write_int8(**over)
    assert st == status, (over, st, msg)
    assert msg


@fake_pointers
def test_write_int8_zero_tokens_is_ok_without_launch():
    st, _ = write_int8(T=0, k=None, v=None, slots=None)
    assert st == 0


def decode_int8(**over):
    args = dict(out=FAKE, odt=0, q=FAKE, qdt=1, kc=FAKE, vc=FAKE, ksc=FAKE, vsc=FAKE, bt=FAKE,
                MB=64, cl=FAKE, B=4, Hq=32, Hkv=8, D=64, NB=100, bs=16, gs=32, scale=0.125,
                hint=1024, P=0, ws=FAKE, wsb=1 << 30)
    args.update(over)
    lib = pka.load_library()
    st = lib.pka_paged_attention_decode_int8(
        args["out"], args["odt"], args["q"], args["qdt"], args["kc"], args["vc"], args["ksc"],
        args["vsc"], args["bt"], args["MB"], args["cl"], args["B"], args["Hq"], args["Hkv"],
        args["D"], args["NB"], args["bs"], args["gs"], args["scale"], args["hint"], args["P"],
        args["ws"], args["wsb"], None)
    return st, lib.pka_last_error().decode()


@fake_pointers
@pytest.mark.parametrize("over,status", [
    (dict(qdt=0), 2), (dict(qdt=5), 1), (dict(odt=2), 1), (dict(Hq=12), 1), (dict(Hq=24, Hkv=2), 2),
    (dict(D=96), 2), (dict(bs=64), 2), (dict(gs=128), 2), (dict(gs=48), 2), (dict(B=-1), 1),
    (dict(scale=float("nan")), 1), (dict(scale=float("inf")), 1), (dict(scale=float("-inf")), 1), (dict(P=24), 1), (dict(P=2048), 2), (dict(kc=None), 1),
    (dict(vsc=FAKE + 4), 1), (dict(ws=None), 3), (dict(wsb=100), 3), (dict(ws=FAKE + 16), 1),
])
def test_decode_int8_rejects(over, status):
    st, msg = decode_int8(**over)
    assert st == status, (over, st, msg)
    assert msg


def test_int8_workspace_and_partition_helpers():
    lib = pka.load_library()
    assert lib.pka_decode_int8_partition_size(16, 8, 16, 200) == 208
    assert lib.pka_decode_int8_partition_size(128, 8, 16, 8192) == 512
    assert lib.pka_decode_int8_partition_size(16, 8, 16, 1024) == 128
    assert lib.pka_decode_int8_workspace_bytes(4, 32, 64, 512, 512) == 0
    n = lib.pka_decode_int8_workspace_bytes(4, 32, 64, 1024, 256)
    # 4 MiB left to the fp16/bf16 decode's counters, then header + items +
    # (max, sum) rows + output rows, each 256-aligned
    assert n == (4 << 20) + 256 + 256 + 4096 + 4 * 32 * 4 * 64 * 4


@fake_pointers
@pytest.mark.parametrize("over,status", [
    (dict(kn=None), 1), (dict(sm=None), 1), (dict(ks=100), 1), (dict(kn=FAKE + 1), 1),
    (dict(qdt=0), 2), (dict(gs=48), 2),
])
def test_decode_append_int8_rejects(over, status):
    a = dict(kn=FAKE, vn=FAKE, ks=512, vs=512, sm=FAKE, qdt=1, gs=32)
    a.update(over)
    lib = pka.load_library()
    st = lib.pka_paged_attention_decode_append_int8(
        FAKE, 0, FAKE, a["qdt"], a["kn"], a["vn"], a["ks"], a["vs"], a["sm"], FAKE, FAKE, FAKE,
        FAKE, FAKE, 64, FAKE, 4, 32, 8, 64, 100, 16, a["gs"], 0.125, 1024, 0, FAKE, 1 << 30, None)
    assert st == status, (over, st, lib.pka_last_error())
