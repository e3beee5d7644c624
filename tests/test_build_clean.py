"""__graft_entry__.build() on a tree where nothing is built yet: it must
compile the HIP library and the oracle, then import the package (the package
itself refuses to import without its library)."""
import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_build_from_a_clean_tree(tmp_path):
    dst = tmp_path / "repo"
    ignore = shutil.ignore_patterns("*.so", "_build", "__pycache__", ".pytest_cache", "ep_loop",
                                    "ep_ceilings")
    for name in ("combine_ep_layout_05_amd", "oracle", "include", "workloads", "tests"):
        shutil.copytree(os.path.join(ROOT, name), dst / name, ignore=ignore)
    shutil.copy(os.path.join(ROOT, "__graft_entry__.py"), dst / "__graft_entry__.py")
    assert not (dst / "combine_ep_layout_05_amd" / "libep_mi355x.so").exists()
    assert not (dst / "combine_ep_layout_05_amd" / "ep_ceilings").exists()
    r = subprocess.run([sys.executable, "-c", "import __graft_entry__ as g; g.build(); "
                        "import combine_ep_layout_05_amd as ep; print(ep.library_path())"],
                       cwd=dst, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    assert (dst / "combine_ep_layout_05_amd" / "libep_mi355x.so").exists()
    assert (dst / "combine_ep_layout_05_amd" / "ep_loop").exists()         # native loop timer
    assert (dst / "combine_ep_layout_05_amd" / "ep_ceilings").exists()     # HBM rate probe
    assert r.stdout.strip().endswith(os.path.join("repo", "combine_ep_layout_05_amd",
                                                  "libep_mi355x.so"))
