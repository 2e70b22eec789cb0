"""The benchmark's plain device-memory read (libsplitkv_probe.so): it loads,
exports the call include/read_probe.h declares, rejects bad arguments on the
host, and on the GPU reads without writing (its only store is conditional on
a constant the data does not hit)."""

import re
import subprocess

import pytest

from split_kv_paged_page_amd import read_probe as rp


def test_probe_library_exports_its_call():
    txt = open(rp.HERE + "/../include/read_probe.h").read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    assert re.findall(r"^\s*int32_t\s+(\w+)\s*\(", txt, re.M) == ["splitkv_read_probe"]
    out = subprocess.run(["nm", "-D", "--defined-only", rp.PROBE_PATH], capture_output=True, text=True).stdout
    assert re.search(r"\bT splitkv_read_probe$", out, re.M)


def test_libraries_share_one_hip_runtime():
    # both libraries and torch resolve to a single libamdhip64 mapping
    import split_kv_paged_page_amd as sk
    sk.lib()
    rp.lib()
    mapped = {ln.split()[-1] for ln in open("/proc/self/maps") if "libamdhip64" in ln}
    assert len(mapped) == 1, mapped


def test_probe_rejects_bad_arguments_without_launching():
    L = rp.lib()
    assert L.splitkv_read_probe(None, 4096, 8, 4096, None) == -1        # null buffer
    assert L.splitkv_read_probe(4096, 4096, 8, None, None) == -1        # null sink
    assert L.splitkv_read_probe(4104, 4096, 8, 4096, None) == -1        # buffer not 16-byte aligned
    assert L.splitkv_read_probe(4096, 4100, 8, 4096, None) == -1        # not a multiple of 16 bytes
    assert L.splitkv_read_probe(4096, 0, 8, 4096, None) == -1
    assert L.splitkv_read_probe(4096, 4096, 0, 4096, None) == -1        # no workgroups
    with pytest.raises(RuntimeError):
        rp.read_probe(0, 4096, 8, 4096)


@pytest.mark.gpu
@pytest.mark.parametrize("nbytes,wgs", [(16, 1), (4096, 3), ((1 << 20) + 48, 2048), (256 << 20, 2048)])
def test_probe_reads_without_writing(nbytes, wgs):
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.manual_seed(nbytes)     # fixed data: whether some lane's fold hits the constant is then fixed too
    buf = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, device="cuda")
    sink = torch.full((wgs,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    before = buf.clone()
    rp.read_probe(buf.data_ptr(), nbytes, wgs, sink.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.equal(buf, before)
    assert bool((sink == 0x5A5A5A5A).all())
