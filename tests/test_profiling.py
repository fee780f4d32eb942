"""Host logic of the counter-to-traffic conversion (no GPU)."""

import csv

from int4_quantized_expert_amd import profiling as P

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _csv(path, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        for i, (k, c, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_traffic_scaled_by_copy_and_keyed_by_digest(tmp_path):
    copy = 1 << 20
    ka = "void moe::(anonymous namespace)::k_decode_a<4, 1, 1>(moe::FusedArgs)"
    f, w = tmp_path / "f.csv", tmp_path / "w.csv"
    # FETCH_SIZE reads half of the copied bytes, WRITE_SIZE all of them.
    _csv(f, [(P.COPY_KERNEL, "FETCH_SIZE", 512.0), (ka, "FETCH_SIZE", 100.0), (ka, "FETCH_SIZE", 300.0)])
    _csv(w, [(P.COPY_KERNEL, "WRITE_SIZE", 1024.0), (ka, "WRITE_SIZE", 8.0), (ka, "WRITE_SIZE", 8.0)])
    t = P.traffic_table(str(f), str(w), copy)
    assert t["fetch_scale"] == 0.5 and t["write_scale"] == 1.0
    r = t["kernels"]["k_decode_a<4, 1, 1>"]
    assert r["dispatches"] == 2
    assert r["read_bytes"] == 200 * 1024 * 2 and r["write_bytes"] == 8 * 1024
    out = tmp_path / "prof"
    out.mkdir()
    P.write_summary(str(out / "x.md"), t, "wl", 1, "cmd")
    assert P.load_traffic(str(out), "wl", 1)["kernels"]["k_decode_a<4, 1, 1>"]["traffic_bytes"] == r["traffic_bytes"]
    assert P.load_traffic(str(out), "wl", 8) is None
    text = (out / "x.md").read_text().replace(P.source_digest(), "0" * 64)
    (out / "x.md").write_text(text)
    assert P.load_traffic(str(out), "wl", 1) is None, "a summary of other sources must not be used"


def test_kernel_names_demangled_or_shortened():
    # rocprofv3 prints some template kernels mangled, others demangled
    assert P.short_name("_ZN3moe12_GLOBAL__N_19k_combineILi1EDF16_EEvPKT0_PKiPKfS8_Pviiii") == "k_combine<1, _Float16>"
    assert P.short_name("_ZN3moe12_GLOBAL__N_19k_combineILi0EfEEvPKT0_PKiPKfS8_Pviiii") == "k_combine<0, float>"
    assert P.short_name("void moe::(anonymous namespace)::k_decode_a<4, 1, 1, 0, true>(moe::FusedArgs)") == \
        "k_decode_a<4, 1, 1, 0, true>"
    assert P.short_name("moe::(anonymous namespace)::k_topk(float const*, int, int, int*, float*)") == "k_topk"
    assert P.is_library_kernel("_ZN3moe12_GLOBAL__N_19k_combineILi1EDF16_EEvPKT0_PKiPKfS8_Pviiii")
    assert not P.is_library_kernel(P.COPY_KERNEL)


def test_counter_summary_means_and_shares(tmp_path):
    ka = "void moe::(anonymous namespace)::k_decode_stack<0>(moe::StackArgs)"
    p1, p2 = tmp_path / "a.csv", tmp_path / "b.csv"
    _csv(p1, [(ka, "SQ_WAVE_CYCLES", 1000.0), (ka, "SQ_WAVE_CYCLES", 3000.0), (ka, "SQ_WAIT_ANY", 500.0),
              (ka, "SQ_WAIT_ANY", 1500.0), (P.COPY_KERNEL, "SQ_WAVE_CYCLES", 7.0)])
    _csv(p2, [(ka, "SQ_ACTIVE_INST_VALU", 400.0), (ka, "SQ_ACTIVE_INST_VALU", 400.0)])
    t = P.counter_table([str(p1), str(p2)])
    assert list(t) == ["k_decode_stack<0>"], "only library kernels are summarised"
    r = t["k_decode_stack<0>"]
    assert r["dispatches"] == 2
    assert r["counters"]["SQ_WAVE_CYCLES"] == 2000.0 and r["counters"]["SQ_WAIT_ANY"] == 1000.0
    assert r["shares"] == {"SQ_WAIT_ANY": 0.5, "SQ_ACTIVE_INST_VALU": 0.2}
    P.write_counter_summary(str(tmp_path / "c.md"), t, "title", "cmd", "")
    text = (tmp_path / "c.md").read_text()
    assert "| waiting on anything | 0.500 (SQ_WAIT_ANY) |" in text
