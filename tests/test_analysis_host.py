"""Host-side checks of the error-analysis command (no GPU needed)."""
import torch

from sparse_attention_video_means_amd import analysis


def test_analysis_refuses_without_a_gpu(capsys):
    if torch.cuda.is_available():
        return
    assert analysis.main(["--workload", "tiny"]) == 2
    assert "GPU" in capsys.readouterr().err


def test_turbo_settings_parse():
    assert analysis.parse_turbo("100:500:0.1,50:250:0.05") == [(100, 500, 0.1), (50, 250, 0.05)]
    for bad in ("100:500", "0:250:0.1", "50:250:1.5", "a:b:c"):
        try:
            analysis.parse_turbo(bad)
        except ValueError:
            continue
        raise AssertionError(f"{bad!r} was accepted")
