"""Geometry figures printed on the pages, checked against the plane-size model used for byte counts."""
import json
import math
import os

import synth

HERE = os.path.dirname(os.path.abspath(__file__))


def _figs():
    with open(os.path.join(HERE, "golden", "page_figures.json")) as f:
        return {d["name"]: d for d in json.load(f)["figures"]}


def test_frame_pair_bytes_matches_page():
    d = _figs()["bytes_per_4k_8bit_frame_pair"]
    b = synth.frame_pair_bytes(d["width"], d["height"], d["bpc"])
    assert b == 24_883_200
    assert round(b / 1e6, 1) == d["value_mb"]


def test_block_counts_match_page():
    f = _figs()
    d = f["warp_atomics_per_4k_luma_plane"]
    assert d["width"] * d["height"] // d["lanes_per_warp"] == d["value"]
    d = f["motion_16x16_tiles_4k"]
    assert math.ceil(d["width"] / 16) * math.ceil(d["height"] / 16) == d["value"]
    d = f["psnr_blocks_4k_420"]
    bw, bh = d["block_px"]
    w, h = d["width"], d["height"]
    wc, hc = (w + 1) // 2, (h + 1) // 2
    n = math.ceil(w / bw) * math.ceil(h / bh) + 2 * math.ceil(wc / bw) * math.ceil(hc / bh)
    assert n == 6210 and abs(n - d["value_about"]) <= 50
    d = f["motion_grid_576x324"]
    gx, gy = math.ceil(d["width"] / 16), math.ceil(d["height"] / 16)
    assert [gx, gy] == d["grid"] and gx * gy == d["blocks"]
    d = f["second_tile_bytes"]
    assert d["rows"] * d["cols"] * d["bytes_per_value"] == d["value"]
