"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Stage by stage, on seeded inputs that span several tiles and ragged tails:
  P1 candidates: band test against the oracle selection scores;
  P2 final subset: band test against the oracle refine scores, both with the
     oracle's candidates fed to the GPU (stage-isolated) and with the GPU's own
     candidates (end to end);
  P3 gather: bit-exact;
  P4 attention: oracle attention on the GPU's own subset, max abs error within
     2e-2 (bf16) / 1e-4 (fp32);
  P5 planted keys are selected; P6 strict ties; P7 bit-identical reruns.
Full-size workloads run in the launch configuration the benchmark times and are
checked on every sequence and every denoising step (the oracle runs per sequence in
a thread pool; numpy releases the interpreter lock in its loops).
"""

from __future__ import annotations

import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle.herald_oracle as orc
from block_diffusion_sparse_herald_amd import herald as H
from block_diffusion_sparse_herald_amd.inputs import WORKLOADS, Workload, bf16_bits_to_f32, f32_to_bf16_bits, make_batch
from block_diffusion_sparse_herald_amd.runner import BlockRunner, batch_to_device, device_tensor
from threadpoolctl import threadpool_limits

from parity import ATOL, band_check, max_abs, record_margin

pytestmark = pytest.mark.gpu

BASE = WORKLOADS["gqa32x8_L32768_b1"]
SMALL = {
    "tiny_f32_L4096": WORKLOADS["tiny_f32_L4096"],
    "gqa32x8_L5000_b2": BASE.with_(name="gqa32x8_L5000_b2", L=5000, nseq=2, C=1000, topk=300, T=2),
    "drift_L9000": WORKLOADS["gqa32x8_L131072_b4_drift"].with_(name="drift_L9000", L=9000, nseq=1, C=2048,
                                                                topk=700, T=2),
    "ragged_g7_L1500-6000": WORKLOADS["gqa28x4_ragged16k-64k_b8"].with_(name="ragged_g7", L=6000, L_min=1500,
                                                                        nseq=3, C=1024, topk=333, T=2),
    "bf16_d64_g4": Workload("bf16_d64_g4", nseq=2, L=3000, Hq=8, Hkv=2, d=64, dtype="bf16", B=16, C=600, topk=130,
                            T=2, planted=8, seed_base=7100),
    "f32_d128_g2": Workload("f32_d128_g2", nseq=2, L=2100, Hq=4, Hkv=2, d=128, dtype="f32", B=8, C=300, topk=77,
                            T=2, planted=4, seed_base=7200),
    # fp32, 80 query rows (five 16-row tiles), candidates ending inside a 64-candidate
    # refine tile (333 = 5 * 64 + 13), 20 in-block keys (a partial second key tile)
    "f32_rows80_c333": Workload("f32_rows80_c333", nseq=2, L=3000, Hq=8, Hkv=2, d=64, dtype="f32", B=20, C=333,
                                topk=100, T=2, planted=4, seed_base=7250),
    # fp32, 15 query rows (one partial 16-row tile) and 5 in-block keys
    "f32_g3_b5": Workload("f32_g3_b5", nseq=2, L=1500, Hq=6, Hkv=2, d=64, dtype="f32", B=5, C=200, topk=45, T=2,
                          planted=4, seed_base=7260),
    # fp32 at the most query rows a group can have (B * G = 256) and d = 128: 128 KiB of
    # query rows in the refine's LDS, sixteen query tiles in the attention
    "f32_d128_rows256": Workload("f32_d128_rows256", nseq=1, L=3000, Hq=8, Hkv=1, d=128, dtype="f32", B=32, C=512,
                                 topk=130, T=1, planted=4, seed_base=7270),
    "g1_b1": Workload("g1_b1", nseq=2, L=2500, Hq=2, Hkv=2, d=128, dtype="bf16", B=1, C=700, topk=64, T=2,
                      seed_base=7300),
    "g8_b32": Workload("g8_b32", nseq=1, L=4000, Hq=16, Hkv=2, d=128, dtype="bf16", B=32, C=512, topk=200, T=2,
                       planted=8, seed_base=7400),
    "select_all": Workload("select_all", nseq=2, L=700, Hq=4, Hkv=1, d=128, dtype="bf16", B=4, C=700, topk=700,
                           T=1, seed_base=7500),
    "topk1": Workload("topk1", nseq=1, L=1000, Hq=4, Hkv=2, d=64, dtype="bf16", B=2, C=1, topk=1, T=1,
                      seed_base=7600),
    # a full 64-key block of in-block keys and a subset of whole blocks; 192 rows
    "b64_g3": Workload("b64_g3", nseq=1, L=1500, Hq=6, Hkv=2, d=128, dtype="bf16", B=64, C=400, topk=128, T=2,
                       seed_base=7700),
    # the largest candidate set (C = 16384: LDS beyond 64 KiB in the emit and top-K kernels)
    "c16384": Workload("c16384", nseq=1, L=40000, Hq=8, Hkv=2, d=128, dtype="bf16", B=8, C=16384, topk=3000, T=1,
                       seed_base=7900),
    # batches long enough for the LDS-staged scan (8 KV heads, >= 262144 tokens in all):
    # head dim 64 with a partial last step; 8 query heads per KV head
    "lds_scan_d64": Workload("lds_scan_d64", nseq=3, L=90000, Hq=16, Hkv=8, d=64, dtype="bf16", B=4,
                             C=700, topk=100, T=1, planted=8, seed_base=8100),
    # the LDS-staged scan at 4 KV heads (G = 7, query heads padded to 8 per token)
    "lds_scan_hkv4_g7": Workload("lds_scan_hkv4_g7", nseq=2, L=140000, Hq=28, Hkv=4, d=128, dtype="bf16", B=4,
                                 C=600, topk=100, T=1, planted=8, seed_base=8350),
    "lds_scan_g8": Workload("lds_scan_g8", nseq=2, L=131100, Hq=64, Hkv=8, d=128, dtype="bf16", B=2, C=600,
                            topk=64, T=1, planted=8, seed_base=8200),
    # a sequence of more than 4096 bitmap words (262144 tokens): the radix emission runs
    # two rounds, the largest candidate set spreads picks over both
    "radix_two_rounds": Workload("radix_two_rounds", nseq=1, L=300000, Hq=4, Hkv=1, d=64, dtype="bf16", B=4,
                                 C=16384, topk=2000, T=1, planted=8, seed_base=8400),
    # more than 16 refine tiles of 256 candidates over enough pairs: 8-wave refine
    # workgroups of 512 candidates, a ragged last tile (4500 = 8 x 512 + 404), head dim 64
    "refine_8waves": Workload("refine_8waves", nseq=4, L=6000, Hq=16, Hkv=8, d=64, dtype="bf16", B=16, C=4500,
                              topk=600, T=1, planted=8, seed_base=8500),
    # the same eight-wave refine at head dim 128
    "refine_8waves_d128": Workload("refine_8waves_d128", nseq=4, L=5000, Hq=32, Hkv=8, d=128, dtype="bf16", B=8,
                                   C=4500, topk=300, T=1, planted=8, seed_base=8600),
    # 256 rows per (sequence, KV head) over 16 pairs: four key ranges merged by 256-thread
    # workgroups on the XCD that ran each pair's ranges
    "merge_256_home": Workload("merge_256_home", nseq=2, L=3000, Hq=32, Hkv=8, d=128, dtype="bf16", B=64, C=1200,
                               topk=1000, T=1, planted=8, seed_base=8700),
    # 12 pairs, four key ranges each: the merge's pairs straddle XCD boundaries (12 work
    # items per XCD, 8 per pair)
    "merge_home_12units": Workload("merge_home_12units", nseq=3, L=2500, Hq=16, Hkv=4, d=128, dtype="bf16", B=16,
                                   C=900, topk=600, T=2, planted=8, seed_base=8800),
    # fp32 with 66 refine tiles of 64 candidates (4200 = 65 * 64 + 40): the scores kernel
    # merges each row's tile statistics in five batches of loads, the last one partial
    "f32_c4200": Workload("f32_c4200", nseq=1, L=6000, Hq=4, Hkv=1, d=64, dtype="f32", B=4,
                                     C=4200, topk=500, T=1, planted=4, seed_base=8900),
    # 64 (sequence, KV head) pairs of eight 16-row query tiles, three key ranges merged on
    # the XCD that ran them
    "pairs64_g4": Workload("pairs64_g4", nseq=8, L=2500, Hq=32, Hkv=8, d=128, dtype="bf16", B=32, C=800, topk=500, T=2,
                       planted=4, seed_base=9000),
    # G = 7 over 32 pairs: 14 query tiles in row groups of 4, 4, 4 and 2, ragged lengths
    "pairs32_g7_ragged": Workload("pairs32_g7_ragged", nseq=8, L=3000, L_min=1500, Hq=28, Hkv=4, d=128, dtype="bf16",
                              B=32, C=900, topk=600, T=2, seed_base=9100),
    # the same pair count at head dim 64
    "pairs64_d64": Workload("pairs64_d64", nseq=8, L=2000, Hq=32, Hkv=8, d=64, dtype="bf16", B=32, C=700, topk=480, T=1,
                        planted=4, seed_base=9200),
    # 15 rows (a ragged row tile), subset longer than 8 blocks per wave round
    "b5_g3_long": Workload("b5_g3_long", nseq=1, L=6000, Hq=3, Hkv=1, d=128, dtype="bf16", B=5, C=3000, topk=1100,
                           T=2, seed_base=7800),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def widen(a: np.ndarray) -> np.ndarray:
    return (bf16_bits_to_f32(a) if a.dtype == np.uint16 else a).astype(np.float64)


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


class Run:
    """One batch on the GPU: all per-block outputs, attention for the requested steps."""

    def __init__(self, wl: Workload, steps=None):
        self.wl = wl
        self.batch = make_batch(wl)
        self.dev = batch_to_device(self.batch)
        self.runner = BlockRunner(self.batch.seq_start, wl.B, wl.Hq, wl.Hkv, wl.d, wl.C, wl.topk, wl.dtype)
        r, d = self.runner, self.dev
        self.steps = list(range(wl.T)) if steps is None else steps
        r.select(d["q0"], d["k_cache"])
        r.refine(d["q0"], d["k_cache"])
        r.gather(d["k_cache"], d["v_cache"])
        self.outs = {}
        for t in self.steps:
            out = torch.empty_like(r.out)
            r.attn(d["q_steps"][t], d["kb_steps"][t], d["vb_steps"][t], out=out)
            self.outs[t] = out
        torch.cuda.synchronize()
        self.cand = to_np(r.cand).astype(np.int64)
        self.cand_score = to_np(r.cand_score)
        self.sel = to_np(r.sel).astype(np.int64)
        self.sel_score = to_np(r.sel_score)
        self.k_sel = to_np(r.k_sel)
        self.v_sel = to_np(r.v_sel)
        self.out = {t: to_np(o) for t, o in self.outs.items()}

    def seq(self, s):
        b = self.batch
        a, e = int(b.seq_start[s]), int(b.seq_start[s + 1])
        return widen(b.q0[s]), widen(b.k_cache[a:e]), widen(b.v_cache[a:e])


def check_sequence(run: Run, s: int, steps, stage_isolated: bool = True):
    wl = run.wl
    scale = orc.default_scale(wl.d)
    q0, k, v = run.seq(s)
    cand_o, S = orc.select_merged(q0, k, wl.C, scale)
    band = 0
    for g in range(wl.Hkv):
        band += band_check(run.cand[s, g], S[g], wl.C, what=f"{wl.name} s{s} g{g} candidates")
        got = run.cand_score[s, g]
        want = S[g][run.cand[s, g]]
        np.testing.assert_allclose(got, want, rtol=1e-4, atol=1e-30, err_msg=f"{wl.name} s{s} g{g} scores")
    # end to end: oracle refine on the GPU's candidates
    R_e2e = orc.refine_scores(q0, k, run.cand[s], scale)
    for g in range(wl.Hkv):
        band_check(run.sel[s, g], R_e2e[g], wl.topk, domain=run.cand[s, g], what=f"{wl.name} s{s} g{g} refine e2e")
        np.testing.assert_allclose(run.sel_score[s, g], R_e2e[g][np.searchsorted(run.cand[s, g], run.sel[s, g])],
                                   rtol=1e-4, atol=1e-30)
    # planted keys: always candidates (they are built along the merged-query direction); the final subset
    # must keep them too unless the oracle's own refine drops them (the drifting-key workload: the walk grows
    # to ~3.6 per channel at 128K, so some drifted keys outscore needles for individual real queries). Those
    # cases are reported with the seed; the band test above already ties the GPU to the oracle there.
    if wl.planted:
        for g in range(wl.Hkv):
            planted = set(run.batch.planted[s][g].tolist())
            assert planted <= set(cand_o[g].tolist()), f"{wl.name} s{s} g{g}: oracle misses a planted candidate"
            assert planted <= set(run.cand[s, g].tolist()), f"{wl.name} s{s} g{g}: planted key not a candidate"
            sel_o = set(run.cand[s, g][orc.top_k_ascending(R_e2e[g], wl.topk, tiebreak=run.cand[s, g])].tolist())
            dropped = planted - sel_o
            if wl.law == "drift":
                if dropped:
                    log(f"  {wl.name} seed {wl.seed_base + s} g{g}: oracle final subset keeps "
                        f"{len(planted) - len(dropped)}/{len(planted)} needles")
            else:
                assert not dropped, f"{wl.name} s{s} g{g}: oracle drops planted keys {sorted(dropped)[:5]}"
                assert planted <= set(run.sel[s, g].tolist()), f"{wl.name} s{s} g{g}: planted key not selected"
    # gather: bit-exact
    a = int(run.batch.seq_start[s])
    ldv = run.v_sel.shape[-1]
    for g in range(wl.Hkv):
        rows = run.batch.k_cache[a + run.sel[s, g], g, :]
        assert np.array_equal(run.k_sel[s, g], rows), f"{wl.name} s{s} g{g}: k_sel differs"
        vrows = run.batch.v_cache[a + run.sel[s, g], g, :]
        assert np.array_equal(run.v_sel[s, g, :, :wl.topk], vrows.T), f"{wl.name} s{s} g{g}: v_sel differs"
        assert not run.v_sel[s, g, :, wl.topk:ldv].any(), "v_sel padding must be zero"
    # attention on the GPU's own subset
    ks, vs = orc.gather_kv(k, v, run.sel[s])
    worst = 0.0
    for t in steps:
        want = orc.block_attention(widen(run.batch.q_steps[t, s]), widen(run.batch.kb_steps[t, s]),
                                   widen(run.batch.vb_steps[t, s]), ks, vs, scale)
        err = max_abs(widen(run.out[t][s]), want)
        worst = max(worst, err)
        assert err <= ATOL[wl.dtype], f"{wl.name} s{s} t{t}: attention max abs error {err}"
    record_margin(wl.name, worst, ATOL[wl.dtype], len(steps) * run.out[steps[0]][s].size if steps else 0)
    log(f"  {wl.name} s{s}: band {band}, attention max abs err {worst:.3g}")
    return cand_o


def oracle_pool(n: int) -> ThreadPoolExecutor:
    """Threads for per-sequence oracle checks (at most the 16 cores a one-GPU share has)."""
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    return ThreadPoolExecutor(max_workers=max(1, min(n, cores, 16)))


@pytest.fixture(scope="module", autouse=True)
def _lib(gpu_lib):
    yield


@pytest.mark.parametrize("name", list(SMALL))
def test_small_workload_parity(name):
    wl = SMALL[name]
    log(f"[parity] {name}: {wl}")
    run = Run(wl)
    for s in range(wl.nseq):
        cand_o = check_sequence(run, s, run.steps)
        # stage-isolated refine: the oracle's candidates through the GPU refine
        if s == 0:
            cand_dev = torch.from_numpy(np.stack([cand_o if i == 0 else run.cand[i] for i in range(wl.nseq)])
                                        .astype(np.int32)).cuda()
            r = run.runner
            r.refine(run.dev["q0"], run.dev["k_cache"], cand=cand_dev)
            torch.cuda.synchronize()
            sel = to_np(r.sel).astype(np.int64)
            q0, k, _ = run.seq(0)
            R = orc.refine_scores(q0, k, cand_o, orc.default_scale(wl.d))
            for g in range(wl.Hkv):
                band_check(sel[0, g], R[g], wl.topk, domain=cand_o[g], what=f"{name} refine stage-isolated g{g}")
    if name == "select_all":
        assert (run.cand == np.arange(wl.C)).all() and (run.sel == np.arange(wl.C)).all()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_strict_ties(dtype):
    """All keys identical within each KV head: candidates are [0, C) and the subset [0, topk)."""
    wl = Workload("ties", nseq=2, L=3000, Hq=8, Hkv=2, d=128 if dtype == "bf16" else 64, dtype=dtype, B=8, C=700,
                  topk=150, T=1, seed_base=7700)
    batch = make_batch(wl)
    batch.k_cache[:] = batch.k_cache[:1]
    dev = batch_to_device(batch)
    r = BlockRunner(batch.seq_start, wl.B, wl.Hq, wl.Hkv, wl.d, wl.C, wl.topk, dtype)
    r.select(dev["q0"], dev["k_cache"])
    r.refine(dev["q0"], dev["k_cache"])
    torch.cuda.synchronize()
    assert (to_np(r.cand) == np.arange(wl.C)).all()
    assert (to_np(r.sel) == np.arange(wl.topk)).all()


@pytest.mark.parametrize("name,L,nseq", [("regs_max_L36864", 36864, 1), ("regs_unaligned_L36863", 36863, 2),
                                         ("radix_L40000", 40000, 1)])
def test_ties_straddle_threshold(name, L, nseq):
    """Every even key is one bit-identical key planted along the group's mean query
    direction, so the top C (C < L/2) lies wholly inside one tie group: candidates are
    exactly the first C even positions and the subset the first topk of those (ties to
    the lower index), on the one-workgroup top-C at its longest sequence (all 16 waves
    full; a second sequence starting at an unaligned offset) and on the radix path."""
    wl = Workload(name, nseq=nseq, L=L, Hq=4, Hkv=1, d=64, dtype="bf16", B=4, C=5000, topk=2000, T=1,
                  seed_base=8300)
    batch = make_batch(wl)
    scale = orc.default_scale(wl.d)
    for s in range(nseq):
        a = int(batch.seq_start[s])
        q0 = widen(batch.q0[s])
        u = q0.sum(axis=(0, 1))
        u /= np.linalg.norm(u)
        k0 = widen(batch.k_cache[a:a + 1, 0])[0]
        kdup = f32_to_bf16_bits((4.0 * np.linalg.norm(k0) * u).astype(np.float32))
        batch.k_cache[a:a + L:2, 0] = kdup
        cand_o, S = orc.select_merged(q0, widen(batch.k_cache[a:a + L]), wl.C, scale)
        assert S[0][0::2].min() > S[0][1::2].max(), "planted copies must outscore every other key"
        assert (cand_o[0] == np.arange(0, 2 * wl.C, 2)).all()
    dev = batch_to_device(batch)
    r = BlockRunner(batch.seq_start, wl.B, wl.Hq, wl.Hkv, wl.d, wl.C, wl.topk, wl.dtype)
    r.select(dev["q0"], dev["k_cache"])
    r.refine(dev["q0"], dev["k_cache"])
    torch.cuda.synchronize()
    cand, sel = to_np(r.cand), to_np(r.sel)
    for s in range(nseq):
        assert (cand[s, 0] == np.arange(0, 2 * wl.C, 2)).all(), f"{name} seq {s} candidates"
        assert (sel[s, 0] == np.arange(0, 2 * wl.topk, 2)).all(), f"{name} seq {s} subset"


def test_rerun_is_bit_identical():
    wl = SMALL["gqa32x8_L5000_b2"]
    a, b = Run(wl), Run(wl)
    assert np.array_equal(a.cand, b.cand) and np.array_equal(a.cand_score.view(np.uint32), b.cand_score.view(np.uint32))
    assert np.array_equal(a.sel, b.sel) and np.array_equal(a.sel_score.view(np.uint32), b.sel_score.view(np.uint32))
    for t in a.out:
        assert np.array_equal(a.out[t], b.out[t])


def test_host_pool_gathers_match_the_oracle():
    """Both host-pool paths (host-packed and GPU-read) and the device path are each
    compared bit for bit with the oracle's gather of the cache rows (V transposed into
    the d-major pool, padding zero)."""
    wl = SMALL["ragged_g7_L1500-6000"]
    run = Run(wl, steps=[])
    r = run.runner
    kh = torch.empty(run.dev["k_cache"].shape, dtype=run.dev["k_cache"].dtype, pin_memory=True)
    vh = torch.empty(run.dev["v_cache"].shape, dtype=run.dev["v_cache"].dtype, pin_memory=True)
    kh.copy_(run.dev["k_cache"].cpu())
    vh.copy_(run.dev["v_cache"].cpu())
    n = wl.nseq * wl.Hkv * wl.topk
    staging = torch.empty(2 * n * wl.d, dtype=kh.dtype, pin_memory=True)
    host_idx = torch.empty(n, dtype=torch.int32, pin_memory=True)
    ws = torch.empty(H.herald_workspace_size(r.problem, H.HERALD_OP_GATHER_HOST), dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    done = torch.cuda.Event()
    done.record(side)  # creates the event

    def check(k_sel, v_sel, what):
        ks, vs = to_np(k_sel), to_np(v_sel)
        for s in range(wl.nseq):
            a, e = int(run.batch.seq_start[s]), int(run.batch.seq_start[s + 1])
            want_k, want_v = orc.gather_kv(run.batch.k_cache[a:e], run.batch.v_cache[a:e], run.sel[s])
            for g in range(wl.Hkv):
                assert np.array_equal(ks[s, g], want_k[g]), f"{what}: k_sel s{s} g{g}"
                assert np.array_equal(vs[s, g, :, :wl.topk], want_v[g].T), f"{what}: v_sel s{s} g{g}"
                assert not vs[s, g, :, wl.topk:].any(), f"{what}: v_sel padding s{s} g{g}"

    check(r.k_sel, r.v_sel, "device gather")
    for src_is_host in (1, 2):
        k_sel = torch.zeros_like(r.k_sel)
        v_sel = torch.full_like(r.v_sel, 7.0)
        side.wait_stream(torch.cuda.current_stream())
        if src_is_host == 1:
            H.herald_gather_kv(r.problem, kh, vh, 1, r.sel, k_sel, v_sel, staging, host_idx, ws, stream=side,
                               done=done)
        else:  # the GPU reading the pinned pool itself (no staging, no host work), on the side stream
            H.herald_gather_kv(r.problem, kh, vh, 2, r.sel, k_sel, v_sel, None, None, None, stream=side, done=done)
        torch.cuda.current_stream().wait_event(done)
        torch.cuda.synchronize()
        check(k_sel, v_sel, f"host-pool gather (src_is_host = {src_is_host})")
    # device memory is refused on the GPU-read path
    with pytest.raises(H.HeraldError):
        H.herald_gather_kv(r.problem, run.dev["k_cache"], run.dev["v_cache"], 2, r.sel, k_sel, v_sel, None, None,
                           None, stream=side)


@pytest.mark.parametrize("src_is_host", [0, 2])
def test_gather_out_of_range_indices(src_is_host):
    """Indices outside [0, L_s) are never dereferenced: their rows come out zero and the
    status word is set; in-range indices leave it clear. Device and GPU-read paths."""
    wl = SMALL["gqa32x8_L5000_b2"]
    batch = make_batch(wl, steps=1)
    dev = batch_to_device(batch)
    r = BlockRunner(batch.seq_start, wl.B, wl.Hq, wl.Hkv, wl.d, wl.C, wl.topk, wl.dtype)
    L = batch.lengths
    rng = np.random.default_rng(5)
    sel = np.stack([np.stack([np.sort(rng.choice(int(L[s]), wl.topk, replace=False)) for _ in range(wl.Hkv)])
                    for s in range(wl.nseq)]).astype(np.int32)
    bad = sel.copy()
    bad[0, 1, 3] = -1
    bad[1, 0, 7] = int(L[1])  # one past the end of sequence 1
    bad[1, 3, wl.topk - 1] = 2**31 - 1
    if src_is_host:
        k_src = torch.empty(dev["k_cache"].shape, dtype=dev["k_cache"].dtype, pin_memory=True)
        v_src = torch.empty(dev["v_cache"].shape, dtype=dev["v_cache"].dtype, pin_memory=True)
        k_src.copy_(dev["k_cache"].cpu())
        v_src.copy_(dev["v_cache"].cpu())
    else:
        k_src, v_src = dev["k_cache"], dev["v_cache"]
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for idx, want_status in ((sel, 0), (bad, 1)):
        k_sel = torch.full_like(r.k_sel, 3.0)
        v_sel = torch.full_like(r.v_sel, 3.0)
        status.zero_()
        H.herald_gather_kv(r.problem, k_src, v_src, src_is_host, torch.from_numpy(idx).cuda(), k_sel, v_sel,
                           None, None, status)
        torch.cuda.synchronize()
        assert int(status.item()) == want_status
        ks, vs = to_np(k_sel), to_np(v_sel)
        for s in range(wl.nseq):
            a = int(batch.seq_start[s])
            for g in range(wl.Hkv):
                ok = (idx[s, g] >= 0) & (idx[s, g] < L[s])
                rows = np.zeros((wl.topk, wl.d), dtype=np.uint16)
                rows[ok] = batch.k_cache[a + idx[s, g][ok], g]
                assert np.array_equal(ks[s, g], rows), f"k_sel s{s} g{g}"
                vrows = np.zeros((wl.topk, wl.d), dtype=np.uint16)
                vrows[ok] = batch.v_cache[a + idx[s, g][ok], g]
                assert np.array_equal(vs[s, g, :, :wl.topk], vrows.T), f"v_sel s{s} g{g}"


def test_kernel_events_time_the_scan():
    wl = SMALL["gqa32x8_L5000_b2"]
    batch = make_batch(wl)
    dev = batch_to_device(batch)
    r = BlockRunner(batch.seq_start, wl.B, wl.Hq, wl.Hkv, wl.d, wl.C, wl.topk, wl.dtype)
    st, sp = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    st.record()
    sp.record()
    H.herald_set_kernel_events("scan", st, sp)
    try:
        r.select(dev["q0"], dev["k_cache"])
    finally:
        H.herald_set_kernel_events("scan", None, None)
    torch.cuda.synchronize()
    assert st.elapsed_time(sp) > 0


FULL = ["tiny_f32_L4096", "gqa32x8_L32768_b1", "gqa32x8_L32768_b16", "gqa32x8_L131072_b4_drift",
        "gqa28x4_ragged16k-64k_b8"]


@pytest.mark.parametrize("name", FULL)
def test_full_size(name):
    """Full-size workload in the benchmark's launch configuration: every sequence and
    every denoising step against the oracle (P1-P5), then the oracle's own candidates of
    every sequence through the GPU refine (stage-isolated P2)."""
    wl = WORKLOADS[name]
    log(f"[full] {name}: generating")
    run = Run(wl)
    log(f"[full] {name}: oracle on {wl.nseq} sequence(s) x {wl.T} step(s)")
    with oracle_pool(wl.nseq) as ex, threadpool_limits(limits=1):
        cands = list(ex.map(lambda s: check_sequence(run, s, run.steps), range(wl.nseq)))
    cand_dev = torch.from_numpy(np.stack(cands).astype(np.int32)).cuda()
    run.runner.refine(run.dev["q0"], run.dev["k_cache"], cand=cand_dev)
    torch.cuda.synchronize()
    sel = to_np(run.runner.sel).astype(np.int64)
    scale = orc.default_scale(wl.d)

    def isolated(s):
        q0, k, _ = run.seq(s)
        R = orc.refine_scores(q0, k, cands[s], scale)
        for g in range(wl.Hkv):
            band_check(sel[s, g], R[g], wl.topk, domain=cands[s][g], what=f"{name} s{s} g{g} refine stage-isolated")

    log(f"[full] {name}: stage-isolated refine")
    with oracle_pool(wl.nseq) as ex, threadpool_limits(limits=1):
        list(ex.map(isolated, range(wl.nseq)))
    del run
    torch.cuda.empty_cache()


def test_graph_replay_matches_eager():
    """A whole block captured into a HIP graph: every replay equals the eager run, with eager work between."""
    wl = SMALL["gqa32x8_L5000_b2"]
    batch = make_batch(wl)
    dev = batch_to_device(batch)
    r = BlockRunner(batch.seq_start, wl.B, wl.Hq, wl.Hkv, wl.d, wl.C, wl.topk, wl.dtype)
    other = dev["k_cache"].flip(0).contiguous()  # different data for the eager runs in between

    def block(k):
        r.run_block(dev["q0"], k, dev["v_cache"], dev["q_steps"], dev["kb_steps"], dev["vb_steps"])

    block(dev["k_cache"])
    torch.cuda.synchronize()
    want = [t.clone() for t in (r.cand, r.cand_score, r.sel, r.k_sel, r.v_sel, r.out)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        block(dev["k_cache"])
    for rep in range(4):
        block(other)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (r.cand, r.cand_score, r.sel, r.k_sel, r.v_sel, r.out)
        for a, b in zip(want, got):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b), f"replay {rep} differs"


@pytest.mark.parametrize("name", ["gqa32x8_L5000_b2", "ragged_g7_L1500-6000", "tiny_f32_L4096", "lds_scan_hkv4_g7",
                                  "lds_scan_d64"])
def test_select_query_parity(name):
    """Selection from one given query per head (a [MASK]-query stand-in: the block's first query),
    band test against the oracle's single-query selection."""
    wl = SMALL[name]
    batch = make_batch(wl)
    dev = batch_to_device(batch)
    r = BlockRunner(batch.seq_start, wl.B, wl.Hq, wl.Hkv, wl.d, wl.C, wl.topk, wl.dtype)
    q_sel = dev["q0"][:, 0].contiguous()  # [nseq][Hq][d]
    r.select_query(q_sel, dev["k_cache"])
    torch.cuda.synchronize()
    cand, cand_score = to_np(r.cand).astype(np.int64), to_np(r.cand_score)
    scale = orc.default_scale(wl.d)
    for s in range(wl.nseq):
        a, e = int(batch.seq_start[s]), int(batch.seq_start[s + 1])
        _, S = orc.select_query(widen(batch.q0[s][0]), widen(batch.k_cache[a:e]), wl.C, scale)
        for g in range(wl.Hkv):
            band_check(cand[s, g], S[g], wl.C, what=f"{name} s{s} g{g} single-query candidates")
            np.testing.assert_allclose(cand_score[s, g], S[g][cand[s, g]], rtol=1e-4, atol=1e-30)
