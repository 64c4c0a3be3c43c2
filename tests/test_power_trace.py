"""Host logic of the power sampler: parsing amd-smi's JSON and the per-part
statistics (no GPU, no amd-smi call)."""
from uniform_state_discrete_step_amd.power_trace import Sampler, parse_smi

# the shape amd-smi 26.x prints for `metric --power --clock --json` (trimmed
# to two XCDs and the memory clock)
SMI_TEXT = """{
    "gpu_data": [
        {
            "gpu": 0,
            "power": {
                "socket_power": {
                    "value": 1399,
                    "unit": "W"
                },
                "gfx_voltage": "N/A"
            },
            "clock": {
                "gfx_0": {
                    "clk": {
                        "value": 1788,
                        "unit": "MHz"
                    },
                    "max_clk": {
                        "value": 2400,
                        "unit": "MHz"
                    }
                },
                "gfx_1": {
                    "clk": {
                        "value": 1710,
                        "unit": "MHz"
                    }
                },
                "mem_0": {
                    "clk": {
                        "value": 2000,
                        "unit": "MHz"
                    }
                }
            }
        }
    ]
}"""


def test_parse_smi_reads_socket_power_and_graphics_clocks():
    p, clks = parse_smi(SMI_TEXT)
    assert p == 1399.0
    assert clks == [1788.0, 1710.0]          # graphics clocks only, not the memory clock


def test_parse_smi_without_data():
    assert parse_smi("") == (None, [])
    assert parse_smi('{"gpu_data": []}') == (None, [])


def test_sampler_statistics_skip_the_first_interval():
    s = Sampler(0.5)
    # (time, power, clocks): the sample at t = 10.2 falls inside the first
    # interval of a part starting at 10.0 and is skipped
    s.samples = [(9.0, 300.0, [2400.0]), (10.2, 900.0, [2000.0]), (10.6, 1400.0, [1700.0, 1800.0]),
                 (11.1, 1398.0, [1760.0]), (11.6, 1402.0, [1740.0]), (13.0, 290.0, [2400.0])]
    r = s.between(10.0, 12.0)
    assert r["samples"] == 3
    assert r["socket_power_W"] == 1400.0
    assert r["socket_power_max_W"] == 1402.0
    assert r["gfx_clock_MHz"] == 1750.0      # median of the per-sample XCD means 1750, 1760, 1740


def test_sampler_statistics_with_no_readings():
    s = Sampler(0.5)
    s.samples = [(10.6, None, [])]
    r = s.between(10.0, 12.0)
    assert r == {"samples": 1, "socket_power_W": None, "socket_power_max_W": None,
                 "gfx_clock_MHz": None}
