"""The binding refuses a library that was not built from the sources beside
it: build.py records a digest of every source, header and compiler flag next
to libmoe_finalize.so, and importing the package compares it with the tree."""
import os
import shutil
import subprocess
import sys

import pytest

import moe_expert_output_finalize_amd as mf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "moe_expert_output_finalize_amd")


def copy_tree(dst):
    shutil.copytree(PKG, os.path.join(dst, "moe_expert_output_finalize_amd"),
                    ignore=shutil.ignore_patterns("__pycache__", "*.tmp*"))
    shutil.copytree(os.path.join(ROOT, "include"), os.path.join(dst, "include"))
    return os.path.join(dst, "moe_expert_output_finalize_amd", "libmoe_finalize.so")


def import_from(root):
    code = f"import sys; sys.path.insert(0, {root!r}); import moe_expert_output_finalize_amd"
    return subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                          timeout=300)


def test_current_library_is_accepted(tmp_path):
    lib = copy_tree(str(tmp_path))
    mf.check_built(lib)


@pytest.mark.parametrize("rel", ["moe_expert_output_finalize_amd/csrc/finalize_kernels.hip",
                                 "moe_expert_output_finalize_amd/csrc/plan.hpp",
                                 "include/moe_finalize.h"])
def test_edited_source_is_refused(tmp_path, rel):
    lib = copy_tree(str(tmp_path))
    with open(os.path.join(str(tmp_path), rel), "a") as f:
        f.write("\nstatic const int mf_edited_after_the_build = 1;\n")
    with pytest.raises(ImportError, match="other sources"):
        mf.check_built(lib)


def test_comment_edit_is_accepted(tmp_path):
    """The digest covers code, not comments: an edited comment leaves the
    built library (and the measurements taken on it) current."""
    lib = copy_tree(str(tmp_path))
    path = os.path.join(str(tmp_path), "moe_expert_output_finalize_amd", "csrc",
                        "finalize_kernels.hip")
    with open(path, "a") as f:
        f.write("\n// a comment added after the build\n/* and a block comment */\n")
    mf.check_built(lib)


def test_import_of_a_stale_tree_raises(tmp_path):
    lib = copy_tree(str(tmp_path))
    with open(os.path.join(os.path.dirname(lib), "csrc", "capi.cpp"), "a") as f:
        f.write("\nstatic const int mf_edited_after_the_build = 1;\n")
    r = import_from(str(tmp_path))
    assert r.returncode != 0 and "ImportError" in r.stderr and "other sources" in r.stderr


def test_missing_record_or_library_is_refused(tmp_path):
    lib = copy_tree(str(tmp_path))
    os.remove(lib + ".sources")
    with pytest.raises(ImportError, match="no record"):
        mf.check_built(lib)
    os.remove(lib)
    with pytest.raises(ImportError, match="not built"):
        mf.check_built(lib)
