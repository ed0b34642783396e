"""The benchmark's host-side accounting (no GPU): the algorithmic bytes and
flops each roofline figure divides by, the mapping from the demangled kernel
names rocprofv3 prints to the library's own names (the profiles are keyed by
them), and the refusal of more than one GPU."""
import os
import subprocess
import sys

import pytest

import bench
from fusion_residual_add_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algo_bytes_decode_gate_up():
    wl = inputs.workload("llama3-8b-decode")
    # weights 28672 x 4096 bf16, x and r for 32 tokens, gamma, the 32 x 14336 output
    assert bench.algo_bytes(wl, "gu") == 28672 * 4096 * 2 + 2 * 32 * 4096 * 2 + 4096 * 2 + 32 * 14336 * 2
    # QKV adds h_out and stores q, k, v
    assert bench.algo_bytes(wl, "qkv") == (6144 * 4096 * 2 + 2 * 32 * 4096 * 2 + 4096 * 2 + 32 * 4096 * 2
                                           + 32 * 6144 * 2)
    assert bench.flops(wl, "gu") == 2 * 32 * 4096 * 28672


@pytest.mark.parametrize("name,wbytes,scales", [("llama2-70b-int8w@M16", 1, 4), ("llama2-70b-int4w@M16", 0.5, 4 * 64),
                                                 ("llama3-8b-decode-fp8", 1, 4)])
def test_algo_bytes_quantised_weights(name, wbytes, scales):
    wl = inputs.workload(name)
    base = bench.algo_bytes(wl, "gu") - int(wl.n_gu * wl.hidden * wbytes) - wl.n_gu * scales
    assert base == 2 * wl.M * wl.hidden * 2 + wl.hidden * 2 + wl.M * wl.ffn * 2


def test_algo_bytes_down():
    wl = inputs.workload("llama3-8b-decode")
    assert bench.algo_bytes(wl, "down") == 32 * 14336 * 2 + 2 * 32 * 4096 * 2 + 4096 * 14336 * 2
    assert bench.flops(wl, "down") == 2 * 32 * 14336 * 4096


@pytest.mark.parametrize("cxx,name", [
    ("void fp::stream_kernel<2, 0, 2, 2, 8, 1>(fp::ProjArgs)", "stream_kernel<bf16,m32,n128,k256,swiglu>"),
    ("void fp::stream_kernel<2, 1, 4, 4, 4, 0>(fp::ProjArgs)", "stream_kernel<bf16-i8w,m64,n256,k128,qkv>"),
    ("void fp::stream_kernel<2, 2, 1, 2, 8, 1>(fp::ProjArgs)", "stream_kernel<bf16-i4w,m16,n128,k256,swiglu>"),
    ("void fp::stream_kernel<2, 4, 2, 2, 16, 1>(fp::ProjArgs)", "stream_kernel<bf16-e4m3,m32,n128,k512,swiglu>"),
    ("void fp::stream_kernel<1, 4, 4, 2, 8, 0>(fp::ProjArgs)", "stream_kernel<f16-e4m3,m64,n128,k256,qkv>"),
    ("void fp::stream_kernel<2, 0, 2, 2, 8, 1, 1>(fp::ProjArgs)", "stream_kernel<bf16,m32,n128,k256,swiglu>"),
    ("void fp::stream_kernel<2, 0, 2, 1, 16, 0, 2>(fp::ProjArgs)", "stream_kernel<bf16,m32,n32,k512,qkv>"),
    ("void fp::stream_kernel<2, 4, 1, 1, 16, 3, 2>(fp::ProjArgs)", "stream_kernel<bf16-e4m3,m16,n32,k512,linear>"),
    ("void fp::stream_kernel<2, 0, 2, 1, 16, 0, 2, 0>(fp::ProjArgs)", "stream_kernel<bf16,m32,n32,k512,qkv>"),
    ("void fp::stream_kernel<2, 0, 2, 1, 16, 0, 2, 4>(fp::ProjArgs)", "stream_kernel<bf16,m32,n32,k512,qkv,rows>"),
    ("void fp::stream_kernel<2, 1, 1, 4, 8, 1, 1, 4>(fp::ProjArgs)", "stream_kernel<bf16-i8w,m16,n256,k256,swiglu,rows>"),
    ("void fp::prefill_kernel<1, 0, 2, true>(fp::ProjArgs)", "prefill_kernel<f16,128x512,gelu>"),
    ("void fp::prefill_kernel<2, 1, 1, false>(fp::ProjArgs)", "prefill_kernel<bf16-i8w,128x512,swiglu>"),
    ("void fp::stats_kernel<2, 256>(fp::StatsArgs)", "stats_kernel<bf16>"),
    ("void fp::stats_kernel<1, 64, 8>(fp::StatsArgs)", "stats_kernel<f16>"),
    ("void fp::norm_kernel<2, 64, 8>(fp::StatsArgs)", "norm_kernel<bf16>"),
    ("void fp::gemm16_kernel<2, 1, 2, false>(fp::ProjArgs)", "gemm16_kernel<bf16,256x256,2st,swiglu>"),
    ("void fp::gemm16_kernel<1, 0, 4, true>(fp::ProjArgs)", "gemm16_kernel<f16,256x256,4st,qkv>"),
    ("void fp::quant8_kernel<1, 64, 8>(fp::StatsArgs)", "quant8_kernel<f16>"),
    ("void fp::gemm8_kernel<2, 1, 4, 4, 2>(fp::ProjArgs)", "gemm8_kernel<bf16,256x256,swiglu>"),
    ("void fp::gemm8_kernel<2, 0, 1, 2, 1, true>(fp::ProjArgs)", "gemm8_kernel<bf16,32x256,qkv>"),
    ("fp::pack_kernel(unsigned int __vector(4) const*, unsigned int __vector(4)*, long, long, long, int, int)",
     "pack_kernel"),
    ("void fp::gemm8_kernel<2, 0, 1, 2, 1>(fp::ProjArgs)", "gemm8_kernel<bf16,32x256,qkv>"),
    ("void fp::gemm8_kernel<1, 3, 2, 2, 2>(fp::ProjArgs)", "gemm8_kernel<f16,128x128,linear>"),
    ("void fp::gemm8_kernel<2, 2, 2, 2, 1>(fp::ProjArgs)", "gemm8_kernel<bf16,64x256,gelu>"),
])
def test_library_kernel_names(cxx, name):
    assert bench.library_kernel_name(cxx) == name


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr) or "1 GPU" in (r.stdout + r.stderr)


def test_source_hash_ignores_comments(tmp_path):
    """The stored traffic counters are keyed by the sources' code: a comment
    or a reflowed line changes no kernel, any code change does."""
    src = 'int f(int a) { // add one\n  return a + 1; /* "x" */ }\nconst char *s = "// kept";\n'
    assert bench.code_text(src) == 'int f(int a) { return a + 1; } const char *s = "// kept";'
    d = tmp_path / "csrc"
    d.mkdir()
    (d / "k.hip").write_text(src)
    h0 = bench.kernel_source_hash(str(d))
    (d / "k.hip").write_text("// header\n" + src.replace("// add one", "// adds\n// one"))
    assert bench.kernel_source_hash(str(d)) == h0
    (d / "k.hip").write_text(src.replace("a + 1", "a + 2"))
    assert bench.kernel_source_hash(str(d)) != h0
    (d / "k.hip").write_text(src.replace('"// kept"', '"// changed"'))
    assert bench.kernel_source_hash(str(d)) != h0
