"""bench.py on the host: a multi-GPU request exits with a message before touching a GPU."""

import bench


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "8"]) == 2
    assert "one GPU" in capsys.readouterr().err
