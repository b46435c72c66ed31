"""CPU checks of the runtime specialisation's host side ("DeepSeek open-source
week, day 3: DeepGEMM", "Core features" and its environment-variable list:
per-shape kernels compiled at run time, a cache directory; the kwkr.cn usage
article, sections 2.3 and 3.3: warm-up and a cache kept across restarts).

No device is needed: a warm-up without a device compiles (or finds) the
code object and fills the disk cache.  Covered: the default configuration
is the ahead-of-time one, the configuration limits, the cache key (one file
per configuration and shape), hits, and damaged or foreign cache files being
ignored and replaced."""
import os

import pytest

from fp8_block_scaled_04_amd import binding, build

D, C, M = binding.FP8G_JIT_DENSE, binding.FP8G_JIT_CONTIGUOUS, binding.FP8G_JIT_MASKED


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(build.LIB):
        build.build()
    return binding.lib()


@pytest.fixture()
def cache(tmp_path, lib):
    prev = binding.fp8_jit_get_cache_dir()
    binding.fp8_jit_set_cache_dir(str(tmp_path))
    yield tmp_path
    binding.fp8_jit_set_cache_dir(prev)


def cfg(**kw):
    base = dict(block_m=128, block_n=128, waves_m=2, waves_n=2, waves_k=1, stages=3, k_per_stage=1, splits=1,
                specialize=0)
    base.update(kw)
    return base


def code_files(d):
    return sorted(f for f in os.listdir(d) if f.endswith(".co"))


def delta(before, after):
    return {k: after[k] - before[k] for k in after}


def test_default_config_is_the_ahead_of_time_choice(lib):
    for m, n, k in [(64, 2112, 7168), (128, 7168, 16384), (300, 1000, 2048), (4096, 7168, 16384)]:
        c = binding.fp8_jit_default_config(D, m, n, k)
        text = binding.fp8_gemm_describe(m, n, k)
        assert text.startswith(f"tile={c.block_m}x{c.block_n} ")
        assert f"stages={c.stages} ku={c.k_per_stage} splits={c.splits} " in text
        assert c.waves_m * c.waves_n * c.waves_k == int(text.split("waves=")[1].split()[0])
        assert binding.fp8_jit_config_supported(D, c)
    assert binding.fp8_jit_default_config(C, 1, 4096, 7168).block_m == 256
    assert binding.fp8_jit_default_config(M, 1, 4096, 7168).as_dict() == cfg(block_m=64, block_n=256, waves_m=2, waves_n=4)
    for mode in (C, M):
        assert binding.fp8_jit_config_supported(mode, binding.fp8_jit_default_config(mode, 1, 4096, 7168))
    with pytest.raises(binding.Fp8GemmError):
        binding.fp8_jit_default_config(7, 1, 4096, 7168)


@pytest.mark.parametrize("bad", [
    cfg(waves_m=3, waves_n=1),                     # 3 waves
    cfg(block_m=320),                              # > 256 rows
    cfg(block_n=96, waves_n=2),                    # a wave's 48 columns do not divide 128
    cfg(stages=9), cfg(stages=0), cfg(k_per_stage=5),
    cfg(k_per_stage=3, waves_k=2, waves_m=1),      # k_per_stage not a multiple of waves_k
    cfg(block_m=256, block_n=256, waves_m=4, waves_n=2, stages=3),   # LDS over 160 KB
    cfg(block_m=256, block_n=256, waves_m=2, waves_n=2, stages=2),   # 128 x 128 per wave: registers
    cfg(splits=9), cfg(splits=0),
    cfg(block_m=256, block_n=256, waves_m=4, waves_n=2, stages=2, splits=2),  # partial tile does not fit
])
def test_unsupported_configs_are_rejected_without_compiling(cache, bad):
    before = binding.fp8_jit_stats()
    assert not binding.fp8_jit_config_supported(D, bad)
    with pytest.raises(binding.Fp8GemmError) as e:
        binding.fp8_jit_warmup(D, 1024, 1024, config=bad)
    assert e.value.status == binding.FP8G_EUNSUPPORTED
    assert delta(before, binding.fp8_jit_stats())["compiles"] == 0
    assert code_files(cache) == []


def test_mode_specific_limits():
    assert not binding.fp8_jit_config_supported(M, cfg(splits=2))     # split-K is dense only
    assert not binding.fp8_jit_config_supported(C, cfg())             # contiguous tiles are 256 rows
    assert binding.fp8_jit_config_supported(M, cfg(block_m=64, waves_m=1, waves_n=4))
    assert binding.fp8_jit_config_supported(D, cfg(block_m=64, block_n=32, waves_m=1, waves_n=1, waves_k=4,
                                                   k_per_stage=4, splits=4))


def test_warmup_compiles_once_then_reads_the_disk(cache):
    c = cfg(block_m=64, block_n=64, waves_m=1, waves_n=4, stages=4, splits=2)
    before = binding.fp8_jit_stats()
    binding.fp8_jit_warmup(D, 2112, 7168, config=c)
    d1 = delta(before, binding.fp8_jit_stats())
    assert d1["compiles"] == 1 and d1["disk_hits"] == 0
    files = code_files(cache)
    assert len(files) == 1
    blob = (cache / files[0]).read_bytes()
    assert blob[:8] == b"FP8GJIT1"
    # the code object is an AMDGPU ELF holding the split 64 x 64 instantiation
    assert b"\x7fELF" in blob
    assert b"_ZN4fp8g11gemm_kernelILi64ELi64ELi1ELi4ELi4ELi0ELb1ELi1ELi1ELi0ELi0ELi0EEEvNS_10GemmParamsE" in blob
    before = binding.fp8_jit_stats()
    binding.fp8_jit_warmup(D, 2112, 7168, config=c)
    binding.fp8_jit_warmup(D, 4096, 1024, config=c)      # n and k are not compiled in: the same kernel
    d2 = delta(before, binding.fp8_jit_stats())
    assert d2["compiles"] == 0 and d2["disk_hits"] == 2
    assert code_files(cache) == files
    assert not [f for f in os.listdir(cache / "tmp")]     # no temporaries left behind


def test_cache_key_separates_shapes_formats_and_modes(cache):
    c = cfg(specialize=1)
    binding.fp8_jit_warmup(D, 2048, 1024, config=c)
    binding.fp8_jit_warmup(D, 2048, 2048, config=c)       # k compiled in: a second kernel
    binding.fp8_jit_warmup(D, 2048, 1024, lhs_format=binding.FP8G_E5M2, config=c)
    binding.fp8_jit_warmup(M, 2048, 1024, config=c)
    assert len(code_files(cache)) == 4
    blobs = b"".join((cache / f).read_bytes() for f in code_files(cache))
    assert b"Li2048ELi1024EEEv" in blobs and b"Li2048ELi2048EEEv" in blobs


@pytest.mark.parametrize("damage", ["flip_code_byte", "truncate", "foreign_file", "garbage"])
def test_damaged_cache_files_are_rejected_and_replaced(cache, damage):
    a, b = cfg(stages=4), cfg(stages=2)
    binding.fp8_jit_warmup(D, 1024, 1024, config=a)
    (fa,) = code_files(cache)
    path = cache / fa
    good = path.read_bytes()
    if damage == "flip_code_byte":
        bad = bytearray(good)
        bad[-100] ^= 0x40
        path.write_bytes(bytes(bad))
    elif damage == "truncate":
        path.write_bytes(good[: len(good) // 2])
    elif damage == "garbage":
        path.write_bytes(b"not a code object")
    else:   # a valid file of another configuration under this key's name
        binding.fp8_jit_warmup(D, 1024, 1024, config=b)
        (fb,) = [f for f in code_files(cache) if f != fa]
        path.write_bytes((cache / fb).read_bytes())
    before = binding.fp8_jit_stats()
    binding.fp8_jit_warmup(D, 1024, 1024, config=a)
    d = delta(before, binding.fp8_jit_stats())
    assert d["rejected_files"] == 1 and d["compiles"] == 1
    assert path.read_bytes() == good                    # replaced by a fresh, identical build
    before = binding.fp8_jit_stats()
    binding.fp8_jit_warmup(D, 1024, 1024, config=a)
    assert delta(before, binding.fp8_jit_stats())["disk_hits"] == 1


def test_unwritable_cache_dir_is_an_error(tmp_path, lib):
    blocker = tmp_path / "file"
    blocker.write_text("x")
    prev = binding.fp8_jit_get_cache_dir()
    binding.fp8_jit_set_cache_dir(str(blocker / "sub"))
    try:
        with pytest.raises(binding.Fp8GemmError) as e:
            binding.fp8_jit_warmup(D, 1024, 1024, config=cfg(stages=3, block_n=64))
        assert e.value.status == binding.FP8G_ELAUNCH     # nowhere to put the compiler's files
    finally:
        binding.fp8_jit_set_cache_dir(prev)


def test_missing_compiler_is_an_error_not_a_crash(cache, monkeypatch):
    monkeypatch.setenv("FP8G_JIT_COMPILER", str(cache / "no-such-compiler"))
    before = binding.fp8_jit_stats()
    with pytest.raises(binding.Fp8GemmError):
        binding.fp8_jit_warmup(D, 1024, 1024, config=cfg(stages=2, block_n=64))
    d = delta(before, binding.fp8_jit_stats())
    assert d["failed_compiles"] == 1 and code_files(cache) == []


def test_cache_dir_default_and_override(lib, monkeypatch, tmp_path):
    prev = binding.fp8_jit_get_cache_dir()
    try:
        monkeypatch.setenv("FP8G_CACHE_DIR", str(tmp_path / "envdir"))
        binding.fp8_jit_set_cache_dir(None)
        assert binding.fp8_jit_get_cache_dir() == str(tmp_path / "envdir")
        monkeypatch.delenv("FP8G_CACHE_DIR")
        monkeypatch.setenv("HOME", str(tmp_path))
        binding.fp8_jit_set_cache_dir("")
        assert binding.fp8_jit_get_cache_dir() == str(tmp_path / ".cache" / "fp8gemm")
    finally:
        binding.fp8_jit_set_cache_dir(prev)


def test_concurrent_warmups_compile_each_kernel_once(cache):
    """Threads asking for the same kernels at once: one compilation per kernel
    (the others wait for it and read the result), different kernels compile
    side by side."""
    import threading
    configs = [cfg(block_n=64, stages=2), cfg(block_n=64, stages=3)]
    errors = []

    def work(c):
        try:
            binding.fp8_jit_warmup(D, 1024, 1024, config=c)
        except Exception as e:  # noqa: BLE001 - reported below
            errors.append(e)

    before = binding.fp8_jit_stats()
    threads = [threading.Thread(target=work, args=(configs[i % 2],)) for i in range(6)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    d = delta(before, binding.fp8_jit_stats())
    assert not errors
    assert d["compiles"] == 2 and d["disk_hits"] == 4 and d["failed_compiles"] == 0
    assert len(code_files(cache)) == 2


def test_single_stage_debug_form_builds(cache, monkeypatch):
    """stages = 1 is the single-buffer form (each stage's copies issued only
    after every wave has read the previous one; "DeepGEMM: FP8 GEMM kernel
    optimisation practice on Hopper Tensor Cores", section 6.2), and
    FP8G_PIPELINE_DEPTH=1 turns every runtime-specialised kernel into it."""
    c = cfg(stages=1)
    assert binding.fp8_jit_config_supported(D, c)
    binding.fp8_jit_warmup(D, 1024, 1024, config=c)
    monkeypatch.setenv("FP8G_PIPELINE_DEPTH", "1")
    binding.fp8_jit_warmup(D, 2112, 7168)                 # the default configuration, one stage
    blobs = b"".join((cache / f).read_bytes() for f in code_files(cache))
    assert b"_ZN4fp8g11gemm_kernelILi128ELi128ELi2ELi2ELi1ELi0ELb0E" in blobs
    d = binding.fp8_jit_default_config(D, 1, 2112, 7168)
    assert f"_ZN4fp8g11gemm_kernelILi{d.block_m}ELi{d.block_n}ELi{d.waves_m}ELi{d.waves_n}ELi1E".encode() in blobs


def test_refused_build_is_remembered_across_processes(cache):
    """A configuration whose build needs scratch memory (here the 256 x 256
    tile with n and k compiled in) is refused; the refusal is recorded in the
    cache, so another process refuses it without compiling again."""
    import ast
    import subprocess
    import sys
    c = cfg(block_m=256, block_n=256, waves_m=4, waves_n=2, stages=2, specialize=1)
    before = binding.fp8_jit_stats()
    with pytest.raises(binding.Fp8GemmError) as e:
        binding.fp8_jit_warmup(D, 4096, 7168, config=c)
    assert e.value.status == binding.FP8G_EUNSUPPORTED
    d = delta(before, binding.fp8_jit_stats())
    assert d["failed_compiles"] == 1 and d["compiles"] == 0
    assert len(code_files(cache)) == 1                     # the refusal record
    before = binding.fp8_jit_stats()                        # again in this process: from memory
    with pytest.raises(binding.Fp8GemmError):
        binding.fp8_jit_warmup(D, 4096, 7168, config=c)
    d = delta(before, binding.fp8_jit_stats())
    assert d["failed_compiles"] == 0 and d["memory_hits"] == 1
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    script = (
        "import sys; sys.path.insert(0, %r)\n"
        "from fp8_block_scaled_04_amd import binding\n"
        "binding.fp8_jit_set_cache_dir(%r)\n"
        "try:\n"
        "    binding.fp8_jit_warmup(0, 4096, 7168, config=%r)\n"
        "    print('built')\n"
        "except binding.Fp8GemmError as e:\n"
        "    print('refused', e.status)\n"
        "print(binding.fp8_jit_stats())\n" % (root, str(cache), c))
    out = subprocess.run([sys.executable, "-c", script], capture_output=True, text=True, timeout=300,
                         env={**os.environ, "HIP_VISIBLE_DEVICES": "-1"}).stdout.splitlines()
    assert out[0] == f"refused {binding.FP8G_EUNSUPPORTED}", out
    stats = ast.literal_eval(out[1])                         # the dict the child printed
    assert stats["failed_compiles"] == 0 and stats["compiles"] == 0 and stats["disk_hits"] == 1
