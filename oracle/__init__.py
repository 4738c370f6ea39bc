"""Float64 CPU oracle of the sink + rolling-KV chunk-attention stream.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke entry point and the benchmark's CPU
baseline leg may import or call anything in this package; the product path (the HIP library
and its Python binding) never does, and this package imports nothing from it.

Pages cited throughout (by title and section; the pages' formulas are stripped, so every
equation here is a reading of the surrounding prose unless it is a textbook definition):

* [WT]   "直播革命來了！StreamDiffusionV2" - paper walkthrough re-posted on qq8o.cn, section
         "方法" (Method): "實時調度和質量控制" (real-time scheduling and quality control) with the
         sub-sections "SLO感知的批處理調度器" (SLO-aware batching scheduler), "自適應的sink和RoPE刷新"
         (adaptive sink and RoPE refresh) and "運動感知的噪聲調度器" (motion-aware noise
         scheduler); and "可擴展的pipeline編排" (scalable pipeline orchestration).
* [NEWS] admirer.cn news article on StreamDiffusionV2 (MLSys 2026), section "方法：算法與系統層面
         的聯合優化" (method), algorithm-level items 1 (sink tokens + rolling KV cache) and 2
         (motion-aware noise), and the system-level item 1 (pipelined batch denoising).
* [WIKI] awesome-system-papers page "StreamDiffusionV2：用于动态和交互式视频生成的流系统
         (MLSys 2026)", sections "关键观察" (key observations) and "核心方法" (core method).
* [REPO] agentlenshq project page "chenfengxu714/StreamDiffusionV2", sections "核心组件"
         (core components: ring-buffer KV cache with sliding-window attention) and
         "快速 Python 示例" (quick Python example: the encode/denoise/decode loop).

Pins: every function here is checked by ``tests/test_oracle_*.py`` against closed forms,
special cases that reduce to a library routine, brute force on tiny inputs, or hand-derived
fixtures under ``tests/golden/``.
"""
from . import rope, attention, stream, sink, motion  # noqa: F401
