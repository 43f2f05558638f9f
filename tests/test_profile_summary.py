"""The decode profile summaries in profiles/ are what the committed
summarizer writes from the committed JSON files, and their per-kernel
algorithmic bytes are the workloads' (CPU only)."""
import json
import os

import pytest

from group_quantized_moe_amd.bench import profile_summary as ps

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("workload", sorted(ps.DECODE))
def test_markdown_is_rendered_from_json(workload):
    with open(os.path.join(ROOT, "profiles", f"{workload}_kernel_trace.md")) as f:
        assert f.read() == ps.render_text(workload)


@pytest.mark.parametrize("workload", sorted(ps.DECODE))
def test_algorithmic_bytes(workload):
    """gate_up: its experts' gate and up codes and scales plus x; down: the
    down codes and scales plus out and the router weights; the call: the
    group's weights plus x, out and the router weights."""
    with open(os.path.join(ROOT, "profiles", f"{workload}_kernels.json")) as f:
        d = json.load(f)
    kb = ps.kernel_bytes(workload)
    spec, E, _ = ps.DECODE[workload]
    import workloads
    g = workloads.make_group(spec)
    weights = sum(m.codes.nbytes + m.scales.nbytes for e in g.experts[:E] for m in (e.gate, e.up, e.down))
    assert d["call"]["algorithmic_bytes"] == sum(kb.values()) == weights + 8 * spec["d_model"] + 4 * E
    for name, k in d["kernels"].items():
        if not k.get("not_part_of_call"):
            assert k["algorithmic_bytes"] == kb[name.split("<")[0]]


def test_kernel_names():
    assert ps.short_name("void smoe::(anonymous namespace)::k_gate_up<4, 2, 64, 1, 4>(smoe::DecodeArgs)", 512) == \
        "k_gate_up<4, 2, 64, 1, 4>"
    assert ps.short_name("_ZN4smoe12_GLOBAL__N_19k_tb_prepEPKfiPDF16_S3_PiPji", 64) == "k_tb_prep"
    assert ps.short_name("(anonymous namespace)::k_stream_read(uint4 const*, unsigned long, unsigned int*)", 1024) == \
        "k_stream_read (grid 1024 blocks)"


def test_counter_parsing_and_calibration(tmp_path):
    """Median counter value per kernel over its dispatches, and the copy's
    calibration factor: known bytes over what the counter reads for it."""
    cols = ["Dispatch_Id", "Grid_Size", "Kernel_Name", "Workgroup_Size", "Counter_Name", "Counter_Value"]
    rows = [
        [1, 131072, "void smoe::(anonymous namespace)::k_gate_up<4, 2, 64, 1, 4>(smoe::DecodeArgs)", 512,
         "FETCH_SIZE", 100.0],
        [2, 131072, "void smoe::(anonymous namespace)::k_gate_up<4, 2, 64, 1, 4>(smoe::DecodeArgs)", 512,
         "FETCH_SIZE", 300.0],
        [3, 131072, "void smoe::(anonymous namespace)::k_gate_up<4, 2, 64, 1, 4>(smoe::DecodeArgs)", 512,
         "FETCH_SIZE", 200.0],
        [4, 16777216, "void at::native::copy_kernel(char*)", 256, "FETCH_SIZE", 131072.0],
        [5, 16777216, "void at::native::fill_kernel(char*)", 256, "FETCH_SIZE", 8.0],
    ]
    path = tmp_path / "c.csv"
    path.write_text("\n".join(",".join(f'"{v}"' if isinstance(v, str) else str(v) for v in r)
                              for r in [cols] + rows) + "\n")
    m = ps.counter_medians(str(path))
    assert m["k_gate_up<4, 2, 64, 1, 4>"] == 200.0
    assert ps.copy_scale(str(path)) == (256 << 20) / (131072.0 * 1024)   # 2.0: the counter reads half
