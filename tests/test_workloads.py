"""The seeded input generator: determinism and the stated distributions."""
import numpy as np

import workloads
from workloads import CONFIGS, HELD_OUT, generate, round_to_bf16


def test_same_seed_same_bytes():
    cfg = CONFIGS[1].with_shape(batch=1, seqlen=300, nheads=3)
    a, b = generate(cfg), generate(cfg)
    for k in ("x_bits", "B_bits", "C_bits", "dt", "A", "D"):
        assert np.array_equal(a[k], b[k]), k
    c = generate(cfg, seed=cfg.seed + 1)
    assert not np.array_equal(a["x_bits"], c["x_bits"])


def test_config_table():
    names = [c.name for c in CONFIGS]
    assert names == ["tiny", "mamba2-130m", "mamba2-2.7b", "long-prefill", "grouped-wide"]
    assert [c.seed for c in CONFIGS] == [0, 1, 2, 3, 4]
    head = workloads.config_by_name("mamba2-2.7b")
    assert (head.batch, head.seqlen, head.nheads, head.headdim, head.dstate, head.ngroups, head.chunk) == \
        (4, 8192, 80, 64, 128, 1, 256)
    assert HELD_OUT.chunk == 128 and HELD_OUT.nheads == 8


def test_distributions():
    cfg = CONFIGS[4].with_shape(batch=1, seqlen=4096, nheads=16)
    d = generate(cfg)
    assert d["x"].dtype == np.float32 and d["x_bits"].dtype == np.uint16
    assert np.all(d["dt"] >= 0)
    zero = np.mean(d["dt"] == 0)
    assert 0.04 < zero < 0.06
    assert np.all(d["A"] < 0) and np.all(d["A"] >= -64.0001) and np.all(d["A"] <= -0.4999)
    assert d["init_state"] is None
    t = generate(CONFIGS[3].with_shape(seqlen=256, nheads=4))
    assert t["init_state"].shape == (1, 4, 64, 128)
    assert abs(float(np.std(t["init_state"])) - 0.1) < 0.005
    f = generate(CONFIGS[0])
    assert "x_bits" not in f and f["x"].dtype == np.float32
    assert np.all(f["A"] <= -1.0) and np.all(f["A"] >= -16.0)


def test_bf16_rounding_is_nearest_even():
    v = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e-3, 1.0 + 2 ** -9 + 2 ** -20],
                 dtype=np.float32)
    r, bits = round_to_bf16(v)
    # ties go to even: 1 + 2^-8 is halfway between 1 and 1 + 2^-7
    assert r[0] == 1.0 and r[1] == 1.0 and r[2] == 1.0 + 2 ** -6
    assert r[3] == -2.5
    assert r[5] == 1.0  # below the halfway point
    assert np.all(np.abs(r - v) <= np.abs(v) * 2 ** -8)
    assert bits[0] == 0x3F80
