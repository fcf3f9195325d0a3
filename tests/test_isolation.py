"""The oracle and the product path share no code and neither imports the
other; the input module holds no method arithmetic and imports neither."""
import ast
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _imports(path):
    tree = ast.parse(open(path).read())
    names = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            names |= {a.name.split(".")[0] for a in node.names}
        elif isinstance(node, ast.ImportFrom) and node.module and node.level == 0:
            names.add(node.module.split(".")[0])
    return names


def _py_files(d):
    for dp, _, fs in os.walk(os.path.join(ROOT, d)):
        for f in fs:
            if f.endswith(".py"):
                yield os.path.join(dp, f)


def test_oracle_imports_no_product_code():
    for f in _py_files("oracle"):
        bad = _imports(f) & {"paged_kv_cache_102_amd", "torch", "ctypes"}
        assert not bad, (f, bad)


def test_product_never_touches_oracle():
    for f in _py_files("paged_kv_cache_102_amd"):
        assert "oracle" not in _imports(f), f
        src = open(f).read()
        assert "import oracle" not in src and "from oracle" not in src, f
    for dp, _, fs in os.walk(os.path.join(ROOT, "paged_kv_cache_102_amd", "csrc")):
        for f in fs:
            assert "oracle" not in open(os.path.join(dp, f)).read().lower(), f


def test_inputs_module_is_standalone():
    for f in _py_files("workloads"):
        assert not (_imports(f) & {"oracle", "paged_kv_cache_102_amd"}), f
