"""Shared test plumbing: the ``gpu`` marker, repo-root imports, golden fixtures."""

from __future__ import annotations

import os
import sys

import pytest

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if REPO not in sys.path:
    sys.path.insert(0, REPO)

GOLDEN_DIR = os.path.join(REPO, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def load_golden(name: str) -> dict:
    """Parse ``tests/golden/<name>.txt``: ``key = value tokens`` lines, '#' comments."""
    out = {}
    with open(os.path.join(GOLDEN_DIR, name + ".txt"), encoding="utf-8") as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, _, val = line.partition("=")
            out[key.strip()] = val.split()
    return out


def ints(tokens) -> list:
    return [int(t) for t in tokens]


def refs(tokens) -> dict:
    """'7:2 1:1' -> {7: 2, 1: 1}"""
    return {int(k): int(v) for k, v in (t.split(":") for t in tokens)}


@pytest.fixture
def golden():
    return load_golden
