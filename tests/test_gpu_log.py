"""The launch log (pkv_set_log / PKV_LOG): one stderr line per kernel launch naming the
kernel, its grid and the variant the host chose."""
import re

import pytest
import torch

from paged_kv_scaled_amd import binding as B
from paged_kv_scaled_amd import workloads as wl

from gpu_helpers import Dev

pytestmark = pytest.mark.gpu


def test_launch_log_names_the_chosen_kernels(gpu, capfd):
    w = wl.decode_batch(seed=95, num_seqs=8, lo=300, hi=2000)
    d = Dev(w, fill="zero")
    p = wl.chunked_prefill(seed=96, num_seqs=2, ctx_hi=100, q_hi=80)
    dp = Dev(p, fill="zero")
    capfd.readouterr()
    B.set_log(True)
    try:
        d.write_all(split_new=False)
        d.decode()
        dp.write_all(split_new=False)
        dp.prefill()
        torch.cuda.synchronize()
    finally:
        B.set_log(False)
    err = capfd.readouterr().err
    lines = [l for l in err.splitlines() if l.startswith("pkv: ")]
    names = [l.split()[1] for l in lines]
    assert names == ["kv_scatter_kernel", "decode_stream_kernel",
                     "decode_merge_stream_wide_kernel", "kv_scatter_kernel",
                     "prefill_mfma_kernel"], lines
    # the decode batch shape (4 heads per wave, bf16, stream mode) runs on the matrix cores
    assert re.search(r"decode_stream_kernel grid=\d+ block=256 core=mfma D=128 heads_per_wave=4", err)
    # 8 sequences over 128 ranges per head group, 16 ranges per sequence: one workgroup
    # merges each (sequence, head)
    assert re.search(r"decode_merge_stream_wide_kernel grid=256 block=256 rows=256", err)
    assert re.search(r"prefill_mfma_kernel grid=\d+ block=512 D=128 heads_per_wg=4 rows_per_wg=64", err)
    # the chip shape comes from the device: the CU count sizes the decode stream grid (one
    # wave per SIMD) and the XCD count (32 CUs each) deals the prefill workgroups; this
    # small prefill grid starts each XCD's query tiles longest first
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    m = re.search(r"decode_stream_kernel .* ranges=(\d+) items=(\d+) cus=(\d+)", err)
    assert m and int(m.group(3)) == cus and int(m.group(2)) == 4 * cus, lines
    m = re.search(r"prefill_mfma_kernel .* xcds=(\d+) ranked=(\d)", err)
    assert m and int(m.group(1)) == max(1, cus // 32) and m.group(2) == "1", lines
    # switched off: nothing more
    d.decode()
    torch.cuda.synchronize()
    assert "pkv: " not in capfd.readouterr().err
