"""GPU parity: the HIP path through the C ABI against the CPU oracle on the
same seeded inputs (small shapes spanning several blocks and ragged tails,
every workload at its full size, edge cases)."""
import math

import numpy as np
import pytest
import torch

import lossless_verify_sample_amd as ssd
from lossless_verify_sample_amd import workloads as W
from oracle import ssd as O
from parity import DTNAME, Report, check_round, raw_host, stats_np

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
F32, BF16, F16 = torch.float32, torch.bfloat16, torch.float16


def _say(*a):
    print(*a, flush=True)


SMALL = [
    # B, K, V, dtype, T, F, C, F_out, kind, greedy_half
    (3, 2, 6, F32, 1.0, 2, 0.5, 2, "normal", False),        # 24-byte rows: unaligned path
    (2, 3, 1, BF16, 1.0, 0, 1.0, 1, "normal", False),       # V = 1
    (4, 2, 9, F16, 0.7, 3, 0.3, 5, "normal", False),        # unaligned fp16
    (2, 4, 2048, BF16, 1.0, 4, 0.5, 4, "normal", False),    # exactly one block
    (2, 4, 2049, F32, 1.0, 4, 0.5, 8, "normal", False),     # one-element tail block
    (3, 5, 5000, BF16, 0.9, 4, 0.6, 27, "peaks", False),    # ragged multi-block
    (4, 3, 20000, F16, 1.3, 8, 0.3, 8, "zipf", True),       # greedy half
    (1, 0, 3000, BF16, 1.0, 2, 0.5, 2, "normal", False),    # K = 0
    (2, 7, 40000, BF16, 1.0, 4, 0.5, 64, "normal", False),  # F_out = 64 > NB
    (4, 3, 16392, F32, 0.5, 4, 1.0, 4, "normal", False),    # C = 1, 8-element tail
    (3, 2, 70001, BF16, 2.0, 0, 0.5, 0, "normal", False),   # F = 0, odd V
    (2, 2, 300000, BF16, 1.0, 4, 0.5, 27, "zipf", False),   # NB = 147 > 128: rows of 8 partials per lane
    (2, 1, 1 << 20, F16, 0.8, 4, 0.5, 8, "normal", True),   # the largest vocabulary (NB = 512)
    (3, 11, 3000, BF16, 1.0, 4, 0.5, 4, "normal", False),   # K + 1 = 12 > 8 rows: a wave merges rows in two passes
    (2, 32, 2500, F32, 0.8, 2, 0.5, 2, "peaks", True),      # K = 32, the largest, with a greedy sequence
    (3, 4, 20000, BF16, 0.02, 4, 0.5, 4, "normal", False),  # T = 0.02: nearly greedy, most blocks weigh 0
    (3, 4, 20000, F32, 50.0, 4, 0.5, 4, "peaks", False),    # T = 50: nearly uniform, small residuals
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"B{c[0]}K{c[1]}V{c[2]}{DTNAME[c[3]]}")
def test_small_shapes(case):
    B, K, V, dt, T, F, C, Fo, kind, gh = case
    cfg = W.custom(B, K, V, dt, T=T, F=F, C=C, kind=kind, draft_sd=0.7, F_out=Fo, greedy_half=gh)
    rep = Report()
    for step in range(6):
        _say(f"small {cfg.name} step {step}")
        t, d = W.logits(cfg, step, DEV)
        r, *_ = check_round(t, d, W.temperatures(cfg, DEV), F, C, W.seed(cfg, step), F_out=Fo, workers=1)
        rep.add(r)
    assert rep.ok(), rep.fails
    _say(f"units {rep.units} near-ties {rep.near}")


def test_neg_inf_and_ties():
    """-inf logits (zero weight), integer-valued logits (many exact ties)."""
    rep = Report()
    for step in range(6):
        g = torch.Generator(device=DEV).manual_seed(100 + step)
        B, K, V = 3, 4, 7000
        t = torch.randint(-3, 4, (B, K + 1, V), generator=g, device=DEV).float()
        d = t + torch.randint(-1, 2, (B, K + 1, V), generator=g, device=DEV).float()
        mask = torch.rand((B, K + 1, V), generator=g, device=DEV) < 0.3
        t[mask] = -math.inf
        d[torch.roll(mask, 1, dims=2)] = -math.inf
        d[..., 0] = 5.0  # at least one finite entry per draft row
        t[..., 1] = 5.0
        for dt in (BF16, F32):
            T = torch.tensor([1.0, 0.6, 0.0], device=DEV)
            _say(f"ties step {step} {dt}")
            r, *_ = check_round(t.to(dt), d.to(dt), T, 3, 0.4, 77 + step, F_out=6, workers=1)
            rep.add(r)
    assert rep.ok(), rep.fails


def test_lazy_block_race_edge_cases():
    """The bonus's lazy block race on rows built against it: (a) the block of
    largest target mass has no residual (the draft covers it alone), the
    residual is spread over many blocks of small mass, some blocks of the
    target are -inf (zero mass: evaluated only while no mass is found);
    (b) the residual sits in the ragged last block, which the draft misses;
    (c) target and draft equal but for one block (tiny residual).  Against
    the oracle, which draws the bonus from the full residual."""
    rep = Report()
    for step in range(4):
        g = torch.Generator(device=DEV).manual_seed(500 + step)
        B, K, V = 6, 3, 20 * 2048 + 777
        base = torch.randn((B, K + 1, V), generator=g, device=DEV)
        # (a)
        t = base.clone()
        t[..., :2048] += 3.0
        t[..., 2048 * 5:2048 * 7] = -math.inf
        d = torch.full_like(t, -math.inf)
        d[..., :2048] = base[..., :2048] + 3.0 + 0.05 * torch.randn((B, K + 1, 2048), generator=g, device=DEV)
        # (b)
        tb = base.clone()
        tb[..., 20 * 2048:] += 4.0
        db = base.clone()
        db[..., 20 * 2048:] = -math.inf
        # (c)
        tc = base.clone()
        dc = base.clone()
        dc[..., 2048 * 9:2048 * 10] += 0.3
        for (tt, dd, tag) in ((t, d, "a"), (tb, db, "b"), (tc, dc, "c")):
            for dt in (BF16, F32):
                T = torch.tensor([1.0, 0.7, 1.3, 1.0, 0.0, 2.0], device=DEV)
                _say(f"lazy race case {tag} step {step} {dt}")
                r, g_s, g_v, *_ = check_round(tt.to(dt), dd.to(dt), T, 4, 0.5, 900 + step, F_out=4, workers=1)
                rep.add(r)
    assert rep.ok(), rep.fails
    _say(f"units {rep.units} near-ties {rep.near}")


def test_topf_tie_overflow_path():
    """Constant rows: every block ties at the threshold, the candidate list
    overflows and the exact fallback selection runs."""
    import lossless_verify_sample_amd as ssd
    from oracle import ssd as O
    x = torch.zeros((2, 9000), device=DEV, dtype=BF16)
    x[1, 4000:] = 1.0
    idx, val = ssd.topf(x, 5)
    torch.cuda.synchronize()
    for r in range(2):
        oi, ov = O.topf(O.decode(raw_host(x[r]), "bf16"), 5)
        assert list(idx[r].cpu().numpy()) == list(oi)
        assert np.array_equal(val[r].cpu().numpy().astype(np.float64), ov)


@pytest.mark.parametrize("dt", [F32, BF16])
@pytest.mark.parametrize("V,F,kind", [(1000, 30, "normal"), (3000, 40, "normal"), (9000, 64, "int"),
                                      (20000, 64, "few"), (2048, 17, "int")])
def test_topf_long_lists_on_short_rows(dt, V, F, kind):
    """More elements at or above the threshold than the candidate list holds
    (lists longer than twice the block count, integer-valued rows with many
    ties, rows of a few distinct values): the radix-select path, exact
    against the oracle."""
    import lossless_verify_sample_amd as ssd
    from oracle import ssd as O
    g = torch.Generator(device=DEV).manual_seed(V + F)
    R = 3
    x = torch.randn((R, V), generator=g, device=DEV) * 3
    if kind == "int":
        x = x.round()
    elif kind == "few":
        x = (x > 0).float() + (x > 2).float()
    x = x.to(dt)
    idx, val = ssd.topf(x, F)
    torch.cuda.synchronize()
    xr = O.decode(raw_host(x), DTNAME[dt])
    for r in range(R):
        oi, ov = O.topf(xr[r], F)
        assert list(idx[r].cpu().numpy()) == list(oi), (V, F, kind, r)
        assert np.array_equal(val[r].cpu().numpy().astype(np.float64), ov)


@pytest.mark.parametrize("dt", [F32, BF16, F16])
def test_softmax_t_and_probs(dt):
    import lossless_verify_sample_amd as ssd
    from oracle import ssd as O
    g = torch.Generator(device=DEV).manual_seed(5)
    R, V = 7, 33000
    x = (torch.randn((R, V), generator=g, device=DEV) * 3).to(dt)
    T = torch.tensor([1.0, 0.5, 0.0, 2.0, 1.3, 0.7, 0.0], device=DEV)
    st, pr = ssd.softmax_t(x, T, probs=True)
    torch.cuda.synchronize()
    lse, mx, am = [a.cpu().numpy() for a in ssd.stats_fields(st)]
    P = pr.cpu().numpy().astype(np.float64)
    xr = O.decode(raw_host(x), DTNAME[dt])
    for r in range(R):
        o = O.softmax_t(xr[r], float(T[r]))
        assert mx[r] == o["max"] and am[r] == o["argmax"]
        assert abs(lse[r] - o["lse"]) <= 1e-5 * max(1, abs(o["lse"]))
        assert np.all(np.abs(P[r] - o["p"]) <= 1e-5 * o["p"] + 1e-30), r


@pytest.mark.parametrize("F", [1, 8, 27, 64])
def test_topf(F):
    import lossless_verify_sample_amd as ssd
    from oracle import ssd as O
    cfg = W.CONFIGS[2]
    t, _ = W.logits(W.custom(4, 2, 128256, BF16, kind="peaks"), 0, DEV)
    x = t.view(-1, t.shape[-1])
    idx, val = ssd.topf(x, F)
    torch.cuda.synchronize()
    xr = O.decode(raw_host(x), "bf16")
    for r in range(x.shape[0]):
        oi, ov = O.topf(xr[r], F)
        assert list(idx[r].cpu().numpy()) == list(oi)
        assert np.array_equal(val[r].cpu().numpy().astype(np.float64), ov)


def test_repeat_calls_are_bit_identical():
    cfg = W.custom(8, 5, 50000, BF16, kind="zipf")
    t, d = W.logits(cfg, 0, DEV)
    T = W.temperatures(cfg, DEV)
    from parity import gpu_round
    a = gpu_round(t, d, T, 4, 0.5, 99)
    b = gpu_round(t, d, T, 4, 0.5, 99)
    for k in ("tokens", "q", "topf_idx", "topf_val"):
        assert np.array_equal(a[0][k], b[0][k]), k
    for k in ("accept_len", "bonus", "p"):
        assert np.array_equal(a[1][k], b[1][k]), k


def _accept_law(zt, zd, T, F, C):
    """Exact law of k* for fixed logits: acceptance at position j, once
    reached, has probability alpha_j = sum_x min(p_j(x), sigma_j(x)) and the
    positions are independent.  Returns (E[k*], Var[k*])."""
    K = zd.shape[0] - 1
    alpha = [O.acceptance_rate(O.softmax_t(zt[j], T)["p"], O.sigma(zd[j], T, F, C)["sigma"]) for j in range(K)]
    pk, reach = [], 1.0
    for j in range(K):
        pk.append(reach * (1.0 - alpha[j]))
        reach *= alpha[j]
    pk.append(reach)
    k = np.arange(K + 1)
    mean = float(np.dot(pk, k))
    return mean, float(np.dot(pk, (k - mean) ** 2))


def test_tiny_verify_workload():
    """B=1, K=4, V=1000 fp32, T=1, F=2, C=0.5: 1000 independent steps.
    Every unit bit-exact against the oracle outside near ties, near ties
    under 1e-4 of the units, and the accepted lengths consistent with their
    exact law (sum of k* - E[k*] within 5 standard deviations)."""
    cfg = W.CONFIGS[1]
    rep = Report()
    dev_sum, var_sum, acc = 0.0, 0.0, []
    T = W.temperatures(cfg, DEV)
    for step in range(1000):
        t, d = W.logits(cfg, step, DEV)
        r, g_s, g_v, *_ = check_round(t, d, T, cfg.F, cfg.C, W.seed(cfg, step), workers=1)
        rep.add(r)
        k = int(g_v["accept_len"][0])
        acc.append(k)
        m, v = _accept_law(O.decode(raw_host(t[0]), "f32"), O.decode(raw_host(d[0]), "f32"), cfg.T, cfg.F, cfg.C)
        dev_sum += k - m
        var_sum += v
    z = dev_sum / math.sqrt(var_sum)
    _say(f"tiny: units {rep.units} near {rep.near} mean accepted {np.mean(acc):.3f} z {z:.2f}")
    assert rep.ok(), rep.fails
    assert rep.near < 1e-4 * rep.units, (rep.near, rep.units)
    assert abs(z) < 5.0, z


EARLY = [
    # B, K, V, dtype, T, F, C, kind, greedy_half, J
    (4, 3, 5000, BF16, 0.9, 4, 0.6, "peaks", False, 1),     # ragged bf16, only position 0 up front
    (6, 5, 20000, F16, 1.3, 8, 0.3, "zipf", True, 2),       # greedy half
    (3, 4, 5001, F32, 1.0, 2, 0.5, "normal", False, 3),     # unaligned fp32
    (8, 7, 40000, BF16, 1.0, 4, 0.5, "zipf", False, 8),     # J = K + 1: every row up front
    (5, 2, 300000, BF16, 1.0, 4, 0.5, "zipf", False, 2),    # NB > 128
    (2, 0, 3000, BF16, 1.0, 2, 0.5, "normal", False, 1),    # K = 0
    (4, 3, 4099, F16, 1.1, 0, 1.0, "normal", True, 2),      # unaligned fp16, F = 0, C = 1, greedy half
    (3, 11, 3000, BF16, 1.0, 4, 0.5, "normal", False, 3),   # K + 1 = 12 > 8 rows
]


def _check_early(t, d, T, F, C, seed, J, F_out=None, workers=None, cache=None):
    """verify_early against verify (bit for bit: k*, bonus, p up to k*, NaN
    past it, cache outputs) and against the oracle (k*, bonus outside near
    ties), on the same inputs and drafted tokens."""
    r, g_s, g_v, smp, ver, o = check_round(t, d, T, F, C, seed, F_out=F_out, workers=workers)
    assert r.ok(), r.fails
    if cache is not None:
        ssd.verify(t, d, T, F, C, seed, smp["tokens"], smp["q"], smp["stats"], smp["topf_idx"], cache=cache)
        torch.cuda.synchronize()
        ref_c = [x.clone() for x in (cache.hit, cache.slot, cache.tokens)]
    e = ssd.verify_early(t, d, T, F, C, seed, smp["tokens"], smp["q"], smp["stats"], smp["topf_idx"], J=J,
                         cache=cache)
    torch.cuda.synchronize()
    acc = e["accept_len"].cpu().numpy()
    assert np.array_equal(acc, g_v["accept_len"])
    assert np.array_equal(e["bonus"].cpu().numpy(), g_v["bonus"])
    p = e["p"].cpu().numpy().astype(np.float64)
    B, K = p.shape
    for b in range(B):
        assert np.array_equal(p[b, :acc[b] + 1], g_v["p"][b, :acc[b] + 1]), b
        assert np.all(np.isnan(p[b, acc[b] + 1:])), b
    ov = o["verify"]
    for b in range(B):
        if np.any(ov["acc_margin"][b] < 1e-5):
            continue
        assert acc[b] == ov["accept_len"][b], b
        assert ov["bonus_margin"][b] < 1e-5 or e["bonus"][b].item() == ov["bonus"][b], b
    if cache is not None:
        for x, y in zip((cache.hit, cache.slot, cache.tokens), ref_c):
            assert torch.equal(x, y)
    return acc


@pytest.mark.parametrize("case", EARLY, ids=lambda c: f"B{c[0]}K{c[1]}V{c[2]}{DTNAME[c[3]]}J{c[9]}")
def test_verify_early(case):
    B, K, V, dt, T, F, C, kind, gh, J = case
    cfg = W.custom(B, K, V, dt, T=T, F=F, C=C, kind=kind, draft_sd=0.7, greedy_half=gh)
    for step in range(4):
        _say(f"verify_early {cfg.name} J={J} step {step}")
        t, d = W.logits(cfg, step, DEV)
        _check_early(t, d, W.temperatures(cfg, DEV), F, C, W.seed(cfg, step), J, workers=1)


@pytest.mark.parametrize("c,J", [(3, 3), (5, 2)])
def test_verify_early_full_size(c, J):
    """Early exit on the Qwen-3-vocabulary (with the cache lookup) and the
    large mixed greedy/sampled workload."""
    cfg = W.CONFIGS[c]
    t, d = W.logits(cfg, 0, DEV)
    cache = None
    if c == 3:
        Fk = ssd.fanout(64, cfg.K, 0.6, cfg.V)
        cache = ssd.Cache(Fk, cfg.B, cfg.K, DEV, payload=W.payload(cfg, 64, 0, DEV), miss_fill=True)
        cache.keys.copy_(torch.randint(0, cfg.V, cache.keys.shape, device=DEV, dtype=torch.int32))
    acc = _check_early(t, d, W.temperatures(cfg, DEV), cfg.F, cfg.C, W.seed(cfg, 0), J, F_out=cfg.fout,
                       cache=cache)
    _say(f"verify_early config {c}: sequences reading past position {J - 1}: "
         f"{int((acc >= J).sum())} of {cfg.B} (at least)")


def test_cache_lookup_against_oracle():
    import lossless_verify_sample_amd as ssd
    from oracle import ssd as O
    cfg = W.CONFIGS[4]
    Fk = ssd.fanout(cfg.Bgt, cfg.K, cfg.ratio, cfg.V)
    assert Fk == [27, 16, 10, 6, 3, 2]
    off = O.depth_offsets(Fk)
    g = torch.Generator(device=DEV).manual_seed(3)
    B, K = cfg.B, cfg.K
    topf = torch.stack([torch.randperm(cfg.V, generator=g, device=DEV)[:27 * (K + 1)].view(K + 1, 27)
                        for _ in range(B)]).to(torch.int32)
    dev_off = torch.tensor(off, dtype=torch.int32, device=DEV)
    keys = ssd.cache_keys(topf, dev_off, cfg.Bgt)
    ok_keys, _ = O.build_keys(topf.cpu().numpy(), Fk)
    assert np.array_equal(keys.cpu().numpy(), ok_keys)
    payload = W.payload(cfg, cfg.Bgt, 0, DEV)
    acc = torch.randint(0, K + 1, (B,), generator=g, device=DEV, dtype=torch.int32)
    acc[0] = K + 1
    acc[1] = -1
    bonus = torch.randint(0, cfg.V, (B,), generator=g, device=DEV, dtype=torch.int32)
    hits = torch.arange(2, B, 2, device=DEV)
    kk = acc[hits].clamp(0, K).long()
    pos = torch.randint(0, 1000, (hits.numel(),), generator=g, device=DEV) % torch.tensor(Fk, device=DEV)[kk]
    bonus[hits] = topf[hits, kk, pos]
    hit, slot, toks = ssd.cache_lookup(keys, dev_off, payload, acc, bonus)
    torch.cuda.synchronize()
    oh, os_, ot = O.cache_lookup(ok_keys, off, payload.cpu().numpy(), acc.cpu().numpy(), bonus.cpu().numpy())
    assert np.array_equal(hit.cpu().numpy(), oh)
    assert np.array_equal(slot.cpu().numpy(), os_)
    assert np.array_equal(toks.cpu().numpy(), ot)
    assert oh.sum() >= hits.numel() - 1
    # misses filled with the random fallback tokens
    seed = W.seed(cfg, 5)
    hit, slot, toks = ssd.cache_lookup(keys, dev_off, payload, acc, bonus, miss_fill=True, V=cfg.V, seed=seed)
    torch.cuda.synchronize()
    oh, os_, ot = O.cache_lookup(ok_keys, off, payload.cpu().numpy(), acc.cpu().numpy(), bonus.cpu().numpy(),
                                 seed=seed, V=cfg.V, miss_fill=True)
    assert np.array_equal(hit.cpu().numpy(), oh)
    assert np.array_equal(slot.cpu().numpy(), os_)
    assert np.array_equal(toks.cpu().numpy(), ot)
    assert (ot >= 0).all()


def test_cache_keys_from_sampling_and_lookup_in_verify():
    """The cache descriptor path: sampling writes each row's top-F_j list into
    the depth-major keys, verification looks (k*, bonus) up in the kernel that
    draws the bonus.  Keys bit-exact against the oracle's top lists; lookup
    against the oracle's lookup on the GPU's (k*, bonus); every other output
    identical to the calls without a cache."""
    import lossless_verify_sample_amd as ssd
    from oracle import ssd as O
    B, K, V = 8, 5, 128256
    cfg = W.custom(B, K, V, BF16, T=0.7, F=4, C=0.6, kind="peaks", draft_sd=0.8, F_out=4, Bgt=64, ratio=0.6)
    for step in range(4):
        # budgets up to 64 keep each sequence's keys in registers, larger ones read them
        budget, fill = (64, 100)[step // 2], step % 2 == 1
        Fk = ssd.fanout(budget, K, 0.6, V)
        _say(f"cache path step {step}: budget {budget} fan-out {Fk} miss fill {fill}")
        t, d = W.logits(cfg, step, DEV)
        T = W.temperatures(cfg, DEV)
        seed = W.seed(cfg, step)
        payload = W.payload(cfg, budget, step, DEV)
        cache = ssd.Cache(Fk, B, K, DEV, payload=payload, miss_fill=fill)
        s1 = ssd.saguaro_sample(d, T, cfg.F, cfg.C, seed, F_out=4, cache=cache)
        s0 = ssd.saguaro_sample(d, T, cfg.F, cfg.C, seed, F_out=4)
        v1 = ssd.verify(t, d, T, cfg.F, cfg.C, seed, s1["tokens"], s1["q"], s1["stats"], s1["topf_idx"], cache=cache)
        v0 = ssd.verify(t, d, T, cfg.F, cfg.C, seed, s0["tokens"], s0["q"], s0["stats"], s0["topf_idx"])
        torch.cuda.synchronize()
        for k in ("tokens", "q", "stats", "topf_idx", "topf_val"):
            assert torch.equal(s1[k], s0[k]), k
        for k in ("accept_len", "bonus", "p"):
            assert torch.equal(v1[k], v0[k]), k
        zd = O.decode(d.view(torch.int16).cpu().numpy().view(np.uint16), "bf16")
        lists = np.zeros((B, K + 1, max(Fk)), dtype=np.int64)
        for b in range(B):
            for j in range(K + 1):
                lists[b, j, :Fk[j]] = O.topf(zd[b, j], Fk[j])[0]
        ok_keys, off = O.build_keys(lists, Fk)
        assert np.array_equal(cache.keys.cpu().numpy(), ok_keys)
        oh, os_, ot = O.cache_lookup(ok_keys, off, payload.cpu().numpy(), v1["accept_len"].cpu().numpy(),
                                     v1["bonus"].cpu().numpy(), seed=seed, V=V, miss_fill=fill)
        assert np.array_equal(cache.hit.cpu().numpy(), oh)
        assert np.array_equal(cache.slot.cpu().numpy(), os_)
        assert np.array_equal(cache.tokens.cpu().numpy(), ot)
        _say(f"  hits {int(oh.sum())} of {B}")


ROUND_CASES = [
    # B, K, V, dtype of verification, dtype of sampling, kind
    (16, 7, 151936, BF16, BF16, "zipf"),     # merged launches
    (5, 3, 20000, F16, F16, "peaks"),        # merged, fp16
    (3, 2, 5001, F32, F32, "normal"),        # merged, unaligned rows
    (4, 4, 40000, BF16, F32, "normal"),      # element types differ: one call after the other
    (3, 0, 3000, BF16, BF16, "normal"),      # K = 0: bonus only
    (6, 3, 40000, F32, F32, "peaks"),        # aligned fp32
    (2, 3, 300000, BF16, BF16, "zipf"),      # NB > 128
    (256, 5, 128256, BF16, BF16, "peaks"),   # cache-scale batch
    (512, 4, 151936, F16, F16, "zipf"),      # large batch, fp16
]


@pytest.mark.parametrize("case", ROUND_CASES, ids=lambda c: f"B{c[0]}K{c[1]}V{c[2]}{DTNAME[c[3]]}{DTNAME[c[4]]}")
def test_round_step_matches_separate_calls(case):
    """ssd_round (verification of round i beside sampling of round i+1):
    every output, cache keys and lookup included, identical to ssd_verify
    followed by ssd_saguaro_sample."""
    import lossless_verify_sample_amd as ssd
    B, K, V, dtv, dts, kind = case
    cv = W.custom(B, K, V, dtv, T=0.9, F=4, C=0.5, kind=kind, draft_sd=0.8, F_out=4)
    cs = W.custom(B, K, V, dts, T=0.9, F=4, C=0.5, kind=kind, draft_sd=0.8, F_out=4)
    T = torch.full((B,), 0.9, device=DEV)
    T[: max(1, B // 8)] = 0.0  # greedy sequences
    Fk = ssd.fanout(32, K, 0.6, V)
    t, d = W.logits(cv, 0, DEV)
    _, d1 = W.logits(cs, 1, DEV)
    pay = W.payload(cv, 32, 0, DEV)
    c0 = ssd.Cache(Fk, B, K, DEV, payload=pay, miss_fill=True)
    s0 = ssd.saguaro_sample(d, T, 4, 0.5, 11, F_out=4, cache=c0)

    def run(use_round):
        c1 = ssd.Cache(Fk, B, K, DEV, payload=pay)
        va = dict(target=t, draft=d, temperature=T, F=4, C=0.5, seed=11, tokens=s0["tokens"], draft_q=s0["q"],
                  draft_stats=s0["stats"], draft_topf_idx=s0["topf_idx"], want_stats=True, cache=c0)
        sa = dict(draft=d1, temperature=T, F=4, C=0.5, seed=12, F_out=4, cache=c1)
        if use_round:
            v, s = ssd.round_step(va, sa)
        else:
            v = ssd.verify(**va)
            s = ssd.saguaro_sample(**sa)
        torch.cuda.synchronize()
        return ({k: x.clone() for k, x in v.items()}, {k: x.clone() for k, x in s.items()},
                [c0.hit.clone(), c0.slot.clone(), c0.tokens.clone(), c1.keys.clone()])

    v_ref, s_ref, c_ref = run(False)
    v_got, s_got, c_got = run(True)
    for k in v_ref:
        assert torch.equal(v_got[k], v_ref[k]), k
    for k in s_ref:
        assert torch.equal(s_got[k], s_ref[k]), k
    for a, b in zip(c_got, c_ref):
        assert torch.equal(a, b)
    _say(f"round {case[:3]}: accepted {v_ref['accept_len'].tolist()} hits {c_ref[0].tolist()}")


@pytest.mark.parametrize("case", [c for c in ROUND_CASES if c[0] * (c[1] + 1) > 256 or c[0] == 16],
                         ids=lambda c: f"B{c[0]}K{c[1]}V{c[2]}{DTNAME[c[3]]}{DTNAME[c[4]]}")
def test_round_early_matches_separate_calls(case):
    """ssd_round_early (early-exit verification of round i beside sampling of
    round i+1): accepted lengths, bonus, p_j(x_j) up to k* (NaN past it),
    cache lookup, keys and every sampling output identical to
    ssd_verify_early followed by ssd_saguaro_sample, for J = 1, 2 and K+1."""
    import lossless_verify_sample_amd as ssd
    B, K, V, dtv, dts, kind = case
    cv = W.custom(B, K, V, dtv, T=0.9, F=4, C=0.5, kind=kind, draft_sd=0.8, F_out=4)
    cs = W.custom(B, K, V, dts, T=0.9, F=4, C=0.5, kind=kind, draft_sd=0.8, F_out=4)
    T = torch.full((B,), 0.9, device=DEV)
    T[: max(1, B // 8)] = 0.0  # greedy sequences
    Fk = ssd.fanout(32, K, 0.6, V)
    t, d = W.logits(cv, 0, DEV)
    _, d1 = W.logits(cs, 1, DEV)
    pay = W.payload(cv, 32, 0, DEV)
    c0 = ssd.Cache(Fk, B, K, DEV, payload=pay, miss_fill=True)
    s0 = ssd.saguaro_sample(d, T, 4, 0.5, 11, F_out=4, cache=c0)
    for J in sorted({1, min(2, K + 1), K + 1}):
        def run(use_round):
            c1 = ssd.Cache(Fk, B, K, DEV, payload=pay)
            va = dict(target=t, draft=d, temperature=T, F=4, C=0.5, seed=11, tokens=s0["tokens"], draft_q=s0["q"],
                      draft_stats=s0["stats"], draft_topf_idx=s0["topf_idx"], cache=c0)
            sa = dict(draft=d1, temperature=T, F=4, C=0.5, seed=12, F_out=4, cache=c1)
            if use_round:
                v, s = ssd.round_step(va, sa, early_J=J)
            else:
                v = ssd.verify_early(**va, J=J)
                s = ssd.saguaro_sample(**sa)
            torch.cuda.synchronize()
            return ({k: x.clone() for k, x in v.items() if x is not None}, {k: x.clone() for k, x in s.items()},
                    [c0.hit.clone(), c0.slot.clone(), c0.tokens.clone(), c1.keys.clone()])

        v_ref, s_ref, c_ref = run(False)
        v_got, s_got, c_got = run(True)
        for k in v_ref:
            assert torch.equal(v_got[k].nan_to_num(-7.0), v_ref[k].nan_to_num(-7.0)), (J, k)
        for k in s_ref:
            assert torch.equal(s_got[k], s_ref[k]), (J, k)
        for a_, b_ in zip(c_got, c_ref):
            assert torch.equal(a_, b_), J
        _say(f"round early {case[:3]} J={J}: accepted {v_ref['accept_len'].tolist()[:16]}")


FBIG = [
    # B, K, V, dtype, T, F, C, F_out, kind, greedy_half: sigma over F > 8 entries (the radix
    # threshold), and (K+1) F > 256, where acceptance, residual and bonus read the draft top-F
    # lists from global memory instead of LDS
    (3, 7, 151936, BF16, 1.0, 16, 0.5, 16, "zipf", False),   # (K+1) F = 128
    (3, 7, 151936, BF16, 1.0, 40, 0.4, 40, "zipf", False),   # (K+1) F = 320
    (2, 3, 151936, BF16, 0.8, 64, 0.3, 64, "peaks", False),  # (K+1) F = 256, the LDS limit
    (4, 4, 151936, F16, 1.0, 64, 0.5, 64, "zipf", True),     # (K+1) F = 320, greedy half
    (3, 7, 40001, F32, 1.1, 40, 0.5, 40, "normal", False),   # unaligned fp32; 2 NB = F: exact fallback
]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("case", FBIG, ids=lambda c: f"B{c[0]}K{c[1]}V{c[2]}{DTNAME[c[3]]}F{c[5]}")
def test_large_f(case):
    """sigma_{F,C} with F in {16, 40, 64} through ssd_saguaro_sample and
    ssd_verify against the oracle, ssd_verify_early against both, and
    ssd_round against the separate calls."""
    B, K, V, dt, T, F, C, Fo, kind, gh = case
    cfg = W.custom(B, K, V, dt, T=T, F=F, C=C, kind=kind, draft_sd=0.8, F_out=Fo, greedy_half=gh)
    temp = W.temperatures(cfg, DEV)
    rep = Report()
    for step in range(3):
        _say(f"large F {cfg.name} F={F} step {step}")
        t, d = W.logits(cfg, step, DEV)
        r, *_ = check_round(t, d, temp, F, C, W.seed(cfg, step), F_out=Fo)
        rep.add(r)
        _check_early(t, d, temp, F, C, W.seed(cfg, step), 2, F_out=Fo)
    assert rep.ok(), rep.fails
    # the pipeline step: every output as the separate calls give it
    t, d = W.logits(cfg, 10, DEV)
    _, d1 = W.logits(cfg, 11, DEV)
    s0 = ssd.saguaro_sample(d, temp, F, C, 5, F_out=Fo)

    def run(use_round):
        va = dict(target=t, draft=d, temperature=temp, F=F, C=C, seed=5, tokens=s0["tokens"], draft_q=s0["q"],
                  draft_stats=s0["stats"], draft_topf_idx=s0["topf_idx"], want_stats=True)
        sa = dict(draft=d1, temperature=temp, F=F, C=C, seed=6, F_out=Fo)
        v, s = ssd.round_step(va, sa) if use_round else (ssd.verify(**va), ssd.saguaro_sample(**sa))
        torch.cuda.synchronize()
        return {k: x.clone() for k, x in v.items()}, {k: x.clone() for k, x in s.items()}

    v_ref, s_ref = run(False)
    v_got, s_got = run(True)
    for k in v_ref:
        assert torch.equal(v_got[k], v_ref[k]), k
    for k in s_ref:
        assert torch.equal(s_got[k], s_ref[k]), k
    _say(f"large F {cfg.name}: units {rep.units} near {rep.near}")


def test_binding_rejects_misshaped_tensors():
    """The binding checks every tensor the kernels index by B, K and the list
    widths, and raises before calling the library."""
    B, K, V = 3, 4, 5000
    cfg = W.custom(B, K, V, BF16)
    t, d = W.logits(cfg, 0, DEV)
    T = W.temperatures(cfg, DEV)
    s = ssd.saguaro_sample(d, T, 4, 0.5, 1)
    good = dict(tokens=s["tokens"], draft_q=s["q"], draft_stats=s["stats"], draft_topf_idx=s["topf_idx"])
    bad = [dict(tokens=s["tokens"][:, :2].contiguous()), dict(draft_q=torch.ones((B + 1, K), device=DEV)),
           dict(draft_stats=s["stats"][:-1].contiguous()), dict(draft_topf_idx=s["topf_idx"][:, :, :2].contiguous()),
           dict(draft_topf_idx=s["topf_idx"][:2].contiguous())]
    for kw in bad:
        with pytest.raises(ssd.SSDError):
            ssd.verify(t, d, T, 4, 0.5, 1, **dict(good, **kw))
    with pytest.raises(ssd.SSDError):
        ssd.verify(t, d, T, 4, 0.5, 1, **good, out=dict(accept_len=torch.empty(B + 1, dtype=torch.int32, device=DEV),
                                                        bonus=torch.empty(B, dtype=torch.int32, device=DEV),
                                                        p=torch.empty((B, K), device=DEV)))
    with pytest.raises(ssd.SSDError):
        ssd.saguaro_sample(d, T, 4, 0.5, 1, out=dict(s, q=torch.empty((B, K + 1), device=DEV)))
    with pytest.raises(ssd.SSDError):
        ssd.saguaro_sample(d, T, 4, 0.5, 1, F_out=6, out=s)  # lists of 4 for F_out = 6
    c = ssd.Cache([2] * (K + 1), B, K, DEV, payload=W.payload(cfg, 2 * (K + 1), 0, DEV))
    c.tokens = torch.empty((B, K - 1), dtype=torch.int32, device=DEV)
    with pytest.raises(ssd.SSDError):
        ssd.verify(t, d, T, 4, 0.5, 1, **good, cache=c)
    keys = torch.zeros((B, 10), dtype=torch.int32, device=DEV)
    off = torch.tensor([0, 2, 4, 6, 8, 10], dtype=torch.int32, device=DEV)
    pay = torch.zeros((B, 10, K), dtype=torch.int32, device=DEV)
    with pytest.raises(ssd.SSDError):
        ssd.cache_lookup(keys, off, pay, torch.zeros(B - 1, dtype=torch.int32, device=DEV),
                         torch.zeros(B, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
