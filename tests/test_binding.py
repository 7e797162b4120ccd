"""The Python handle classes pass their handle only to entry points of their own
family: a dlm_layers* never reaches an SGMM call and a dlm_sgmm_group* never
reaches a switch or product call (the C side cannot tell the two apart)."""
import ast
import os

import dynamic_lora_moe_amd as dlm

FAMILY = {
    "Layers": ("dlm_layers_", "dlm_switch", "dlm_gemv"),
    "SgmmGroup": ("dlm_sgmm_group_",),
}


def _handle_calls(cls: ast.ClassDef):
    """(entry point, method) for every C call in the class whose first argument is self._h."""
    out = []
    for fn in cls.body:
        if not isinstance(fn, ast.FunctionDef):
            continue
        for node in ast.walk(fn):
            if not (isinstance(node, ast.Call) and isinstance(node.func, ast.Attribute)):
                continue
            if not node.func.attr.startswith("dlm_") or not node.args:
                continue
            a0 = node.args[0]
            if isinstance(a0, ast.Attribute) and a0.attr == "_h" and isinstance(a0.value, ast.Name) \
                    and a0.value.id == "self":
                out.append((node.func.attr, fn.name))
    return out


def test_handles_reach_only_their_own_entry_points():
    with open(os.path.join(os.path.dirname(dlm.__file__), "__init__.py"), encoding="utf-8") as f:
        tree = ast.parse(f.read())
    classes = {n.name: n for n in tree.body if isinstance(n, ast.ClassDef)}
    assert set(FAMILY) <= set(classes)
    for name, prefixes in FAMILY.items():
        calls = _handle_calls(classes[name])
        assert calls, f"{name} makes no handle calls"
        for entry, method in calls:
            assert entry.startswith(prefixes), f"{name}.{method} passes its handle to {entry}"


def test_every_handle_call_is_declared():
    declared = set(dlm.header_functions())
    with open(os.path.join(os.path.dirname(dlm.__file__), "__init__.py"), encoding="utf-8") as f:
        tree = ast.parse(f.read())
    for cls in (n for n in tree.body if isinstance(n, ast.ClassDef)):
        for entry, method in _handle_calls(cls):
            assert entry in declared, f"{cls.name}.{method} calls undeclared {entry}"
