"""Host-side logic of bench.py (CPU): the cold-weight replica count covers every workload, so that one
rotation over the replicas reads at least 8x the 256 MB Infinity Cache of the bytes the layers read."""
import math

import moe_synth


def test_cold_replicas_cover_the_infinity_cache():
    import bench

    for name, cfg in moe_synth.CONFIGS.items():
        R = bench.cold_replicas(cfg)
        per_expert = 3 * cfg.H * cfg.I // 2 + 3 * cfg.H * cfg.I // 32
        layer_bytes = min(cfg.E, cfg.T * cfg.k) * per_expert
        assert R >= 2, name
        assert R * layer_bytes >= 8 * bench.LLC_BYTES, name
        # no more than needed (plus the floor of two)
        assert R == max(2, math.ceil(8 * bench.LLC_BYTES / layer_bytes)), name


def test_capture_rotation_walks_every_replica():
    import bench

    class FakeGraph:
        def __init__(self):
            self.calls = []

    class FakeCuda:
        log = []

        class CUDAGraph(FakeGraph):
            pass

        @staticmethod
        def graph(g, stream=None):
            class Ctx:
                def __enter__(self_):
                    FakeCuda.log.append(g)

                def __exit__(self_, *a):
                    return False
            return Ctx()

    class FakeTorch:
        cuda = FakeCuda

    seen = []
    for L, R in ((10, 108), (40, 3), (4, 12), (10, 11), (5, 2)):
        seen.clear()
        graphs = bench.capture_rotation(FakeTorch, None, L, R, seen.append)
        assert len(graphs) == max(1, math.ceil(R / L))
        assert sorted(set(seen)) == list(range(R))
        assert seen == [j % R for j in range(len(graphs) * L)]
