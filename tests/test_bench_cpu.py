"""Host-side checks of bench.py that need no GPU: every workload name parses,
and no function refers to a module-level name that does not exist (the
paths that only run with a GPU would otherwise fail only there)."""
import ast
import builtins
import os

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_workloads_parse():
    for name, w in synth.WORKLOADS.items():
        for T in w.tokens:
            got, t = bench.parse_workload(f"{name}:{T}")
            assert got.name == name and t == T


def _own_names(fn):
    """Names bound in fn itself (parameters, assignments, imports, nested
    definitions), not looking inside nested functions."""
    names = set()
    args = fn.args
    for a in args.args + args.posonlyargs + args.kwonlyargs + [args.vararg, args.kwarg]:
        if a is not None:
            names.add(a.arg)
    stack = list(fn.body) if isinstance(fn.body, list) else [fn.body]
    while stack:
        n = stack.pop()
        if isinstance(n, (ast.FunctionDef, ast.ClassDef)):
            names.add(n.name)
            continue
        if isinstance(n, ast.Lambda):
            continue
        if isinstance(n, ast.Name) and isinstance(n.ctx, (ast.Store, ast.Del)):
            names.add(n.id)
        elif isinstance(n, (ast.Import, ast.ImportFrom)):
            names.update((a.asname or a.name).split(".")[0] for a in n.names)
        elif isinstance(n, ast.ExceptHandler) and n.name:
            names.add(n.name)
        stack.extend(ast.iter_child_nodes(n))
    return names


def _unbound_globals(tree):
    """Names read inside functions that are bound neither in the function,
    nor in an enclosing function, nor at module level, nor as builtins."""
    module_names = set(dir(builtins))
    for node in tree.body:
        if isinstance(node, (ast.FunctionDef, ast.ClassDef)):
            module_names.add(node.name)
        elif isinstance(node, (ast.Import, ast.ImportFrom)):
            module_names.update((a.asname or a.name).split(".")[0] for a in node.names)
        elif isinstance(node, (ast.Assign, ast.AnnAssign)):
            targets = node.targets if isinstance(node, ast.Assign) else [node.target]
            for t in targets:
                module_names.update(n.id for n in ast.walk(t) if isinstance(n, ast.Name))
    missing = set()

    def visit(fn, outer):
        scope = outer | _own_names(fn)
        stack = list(fn.body) if isinstance(fn.body, list) else [fn.body]
        while stack:
            n = stack.pop()
            if isinstance(n, (ast.FunctionDef, ast.Lambda)):
                visit(n, scope)
                continue
            if isinstance(n, ast.Name) and isinstance(n.ctx, ast.Load) and n.id not in scope:
                if n.id not in module_names:
                    missing.add(n.id)
            stack.extend(ast.iter_child_nodes(n))

    for node in ast.walk(tree):
        if isinstance(node, ast.ClassDef):
            for item in node.body:
                if isinstance(item, ast.FunctionDef):
                    visit(item, set())
    for node in tree.body:
        if isinstance(node, ast.FunctionDef):
            visit(node, set())
    return missing


def test_bench_names_resolve():
    with open(os.path.join(ROOT, "bench.py")) as fh:
        tree = ast.parse(fh.read())
    assert _unbound_globals(tree) == set()


def test_measured_path_imports_no_test_code():
    """bench.py's GPU path builds its weights through the binding
    (quantize_layer) and the seeded draws: nothing under tests/ is imported,
    and the oracle only inside the CPU-baseline leg."""
    with open(os.path.join(ROOT, "bench.py")) as fh:
        tree = ast.parse(fh.read())
    for node in ast.walk(tree):
        if isinstance(node, (ast.Import, ast.ImportFrom)):
            mods = [node.module] if isinstance(node, ast.ImportFrom) else [a.name for a in node.names]
            assert not any(m and m.split(".")[0] == "tests" for m in mods)
    allowed = {"cpu_baseline", "cpu_baseline_stack", "load"}   # OracleExperts.load
    for node in ast.walk(tree):
        if isinstance(node, ast.FunctionDef):
            imports = [n for n in ast.walk(node) if isinstance(n, ast.Import)]
            if any(a.name == "oracle" for n in imports for a in n.names):
                assert node.name in allowed, node.name


def test_counter_summaries_match_sources():
    """The HBM counter summaries bench.py reads for its default line (the
    8192-token prefill chunk and the two nested decode lines) were taken on
    the kernel sources as they stand, so the line reports their traffic;
    a kernel change without new counters would turn it into null."""
    for workload, T in (("moe_h4096_e512_k10_b4_hot", 8192), ("moe_h4096_e512_k10_b4_hot", 1),
                        ("moe_h2048_e256_k8_s1_b4", 8)):
        got = bench.measured_traffic(workload, T)
        assert got is not None, f"profiles/pmc_{workload}_T{T}.txt is missing or was taken on other sources"
        assert got > 0
