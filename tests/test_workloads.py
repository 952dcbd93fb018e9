"""Seeded input generators: determinism, shapes, dtypes and the clustered recipe."""

import re

import torch

from vision_transformer_dynamic_amd import workloads as wl


def test_five_workloads_shapes():
    assert len(wl.WORKLOADS) == 5
    kv = [w.kv for w in wl.WORKLOADS]
    assert kv == [32, 64, 64, 64, 1024]
    assert all(w.d == 32 for w in wl.WORKLOADS)
    assert wl.HEADLINE.H == 56 and wl.HEADLINE.S == 7


def test_inputs_are_deterministic_and_typed():
    w = wl.custom(2, 8, 8, 64, 2, 4, 2, dtype="bf16", seed=7)
    a = wl.make_inputs(w)
    b = wl.make_inputs(w)
    for x, y in zip(a, b):
        assert x.dtype == torch.bfloat16 and x.shape == (2, 8, 8, 64) and x.is_contiguous()
        assert torch.equal(x, y)
    c = wl.make_inputs(wl.custom(2, 8, 8, 64, 2, 4, 2, dtype="bf16", seed=8))
    assert not torch.equal(a[0], c[0])


def test_clustered_tokens_share_their_region_mean():
    w = wl.custom(1, 16, 16, 32, 1, 4, 2, dtype="f32", seed=3, content="clustered")
    q, k, v = wl.make_inputs(w)
    # within-region spread ~0.5, between-region spread ~1: region means of the
    # drawn tokens must be far closer to each other inside a region
    g = q.reshape(1, 4, 4, 4, 4, 32).permute(0, 1, 3, 2, 4, 5).reshape(1, 16, 16, 32)
    within = g.std(dim=2).mean().item()
    between = g.mean(dim=2).std(dim=1).mean().item()
    assert 0.4 < within < 0.6 and between > 0.7
    # V is iid, not clustered
    gv = v.reshape(1, 4, 4, 4, 4, 32).permute(0, 1, 3, 2, 4, 5).reshape(1, 16, 16, 32)
    assert gv.std(dim=2).mean().item() > 0.85


def test_bench_names_the_dispatched_attention_kernel():
    """bench.py labels its roofline with the attention kernel the library
    dispatches (bra_attend_kernel, the dispatch decision itself): the
    per-region kernel at stage 1 and for fp32, the image-resident kernel at
    the 28x28 and 14x14 stage shapes, the kernel that stages every routed key
    in LDS at the dense shape (more than 64 keys per query, bf16)."""
    import bench
    names = [bench.attention_kernel_name(w) for w in wl.WORKLOADS]
    assert names == ["attend_head_kernel", "attend_head_kernel", "attend_image_kernel",
                     "attend_image_kernel", "attend_dense_kernel"]
    # more than 64 keys per query in fp32, or more than 1024 in bf16: the chunked kernel
    assert bench.attention_kernel_name(wl.custom(1, 16, 16, 64, 2, 4, 6, "f32")) == "attend_kernel"
    assert bench.attention_kernel_name(wl.custom(1, 48, 48, 64, 2, 2, 2, "bf16")) == "attend_kernel"
    # too few (image, head) pairs, or regions not a multiple of 4 tokens
    assert bench.attention_kernel_name(wl.custom(2, 28, 28, 128, 4, 7, 4)) == "attend_head_kernel"
    assert bench.attention_kernel_name(wl.custom(64, 21, 21, 64, 2, 7, 4)) == "attend_head_kernel"


def _profile_traces():
    """Committed kernel-trace summaries: {workload name: text}."""
    import os
    import re
    root = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "profiles")
    out = {}
    for name in sorted(os.listdir(root)):
        if name.endswith("_kernel_trace.md"):
            text = open(os.path.join(root, name)).read()
            m = re.search(r"^workload: (\S+)$", text, flags=re.M)
            if m:
                out[m.group(1)] = text
    return out


def test_profiled_kernels_are_the_dispatched_ones():
    """Each committed kernel trace of a workload lists the attention kernel
    that the library's dispatch names for it, and no other attention kernel."""
    import bench
    traces = _profile_traces()
    assert traces, "no kernel trace under profiles/ names its workload"
    kinds = ("attend_head_kernel", "attend_image_kernel", "attend_dense_kernel", "attend_kernel")
    for w in wl.WORKLOADS:
        if w.name not in traces:
            continue
        text = traces[w.name]
        want = bench.attention_kernel_name(w)
        assert want in text, (w.name, want)
        for other in kinds:
            if other != want:
                # the name as a whole identifier, mangled (...13attend_kernelI...)
                # or demangled (...::attend_kernel<...)
                assert not re.search(r"(?<![A-Za-z_])" + other + r"[I<]", text), (w.name, other)
