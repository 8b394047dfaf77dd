"""Host-only check that the epilogue weight stream is a permutation of the W_O,
W_1 and W_2 fragments in exactly the order each epilogue wave consumes them."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_stream_order_is_consumption_order(tmp_path):
    src = os.path.join(os.path.dirname(__file__), "stream_order_check.cpp")
    exe = str(tmp_path / "stream_order")
    subprocess.run(["g++", "-std=c++17", "-O1", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", src, "-o", exe], check=True)
    res = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                         timeout=120)
    assert res.returncode == 0, res.stdout
    assert "ALL OK" in res.stdout
