"""Host logic of bench.py that needs no GPU: the kernel-source hash that keys
the committed counter summaries to the kernel code."""
import bench


def _write(tmp_path, name, text):
    p = tmp_path / name
    p.write_text(text)
    return name


def test_source_hash_ignores_comments_and_blank_lines(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    a = _write(tmp_path, "a.hip", "int f(int x) {\n  return x + 1;  // add one\n}\n")
    h0 = bench.kernel_source_hash([a])
    _write(tmp_path, "a.hip", "// header comment\n\nint f(int x) {\n  /* block\n     comment */\n"
                              "  return x + 1;  // a different remark\n}\n\n")
    assert bench.kernel_source_hash([a]) == h0


def test_source_hash_follows_the_code(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    a = _write(tmp_path, "a.hip", "int f(int x) {\n  return x + 1;\n}\n")
    h0 = bench.kernel_source_hash([a])
    _write(tmp_path, "a.hip", "int f(int x) {\n  return x + 2;\n}\n")
    h1 = bench.kernel_source_hash([a])
    assert h1 != h0
    b = _write(tmp_path, "b.h", "#define N 4\n")
    assert bench.kernel_source_hash([a, b]) not in (h0, h1)



def _pass_csv(path, rows):
    import csv
    path.mkdir(parents=True)
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    with open(path / "p_counter_collection.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=cols)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(cols, r)))


def test_counter_summary_mfma_busy_falls_back_to_dispatch_time(tmp_path, monkeypatch):
    """Where GRBM_GUI_ACTIVE implies a clock above the published 2.4 GHz (it
    runs past short dispatches under counter collection), the summary's
    machine-readable MFMA busy is the busy cycles over the summed dispatch
    time at 2.4 GHz; otherwise it is rocprof's GRBM-based figure."""
    root = tmp_path / "root"
    (root / "profiles").mkdir(parents=True)
    monkeypatch.setattr(bench, "ROOT", str(root))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda sources: "0" * 16)

    def run(grbm_split):
        rd = tmp_path / f"run{grbm_split}"
        rd.mkdir()
        (rd / "cmds.txt").write_text("cmd\n")
        busy = 2.0e7
        split = [("SQ_VALU_MFMA_BUSY_CYCLES", busy), ("SQ_VALU_MFMA_COEXEC_CYCLES", 1e6), ("SQ_INSTS_VALU", 1e7),
                 ("SQ_INSTS_MFMA", 1e6), ("SQ_INSTS_VALU_TRANS_F32", 1e5), ("GRBM_GUI_ACTIVE", grbm_split)]
        rows = [(1, "__amd_rocclr_copyBuffer", "GRBM_GUI_ACTIVE", 1e6, 0, 100000)]
        rows += [(2, "void attnq::k_mla_split<false>(attnq::MlaArgs)", c, v, 1000, 51000) for c, v in split]
        rows += [(3, "attnq::k_mla_merge(attnq::MlaArgs)", c, 0.0 if c != "GRBM_GUI_ACTIVE" else 1e5, 60000, 67000)
                 for c, _ in split]
        _pass_csv(rd / "mfma", rows)
        bench.summarize_counters("c4", str(rd))
        txt = (root / "profiles" / bench.COUNTER_WORKLOADS["c4"]["file"]).read_text()
        return float(txt.split("mfma_util_pct: ")[1].split()[0]), busy

    # 8 XCDs x 57 us x 2.0 GHz: a plausible clock, rocprof's figure is kept
    util, busy = run(8 * 57000 * 2.0 - 1e5)
    grbm_one_xcd = (8 * 57000 * 2.0 - 1e5 + 1e5) / 8
    assert abs(util - 100 * busy / (grbm_one_xcd * 1024)) < 1e-2
    # an implied 8 GHz: the dispatch-time figure replaces it
    util, busy = run(8 * 57000 * 8.0)
    assert abs(util - 100 * busy / (1024 * 57000 * 2.4)) < 1e-2
