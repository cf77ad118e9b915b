"""The host C++ (block manager, prefix cache, SHA-256, error plumbing) under
AddressSanitizer + UndefinedBehaviorSanitizer: the block-manager, prefix-cache
and ABI tests rerun in a child process against a library whose host objects
are instrumented (device code untouched; runs on the CPU)."""

import shutil

import pytest


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++ and its sanitizer runtimes")
def test_block_manager_tests_clean_under_asan_and_ubsan():
    from paged_kv_cache_117_amd import sanitize_host

    assert sanitize_host.run(["-x"]) == 0
