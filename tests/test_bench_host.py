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

