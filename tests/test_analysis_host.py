"""Host-side checks of the error-analysis command (no GPU needed)."""
import torch

from sparse_attention_video_means_amd import analysis


def test_analysis_refuses_without_a_gpu(capsys):
    if torch.cuda.is_available():
        return
    assert analysis.main(["--workload", "tiny"]) == 2
    assert "GPU" in capsys.readouterr().err
