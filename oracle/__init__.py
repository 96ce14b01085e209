"""CPU oracle for the compressed-weight matrix product.  TEST INFRASTRUCTURE.

Plain, slow, fp64 numpy code that states what the GPU path must compute.
Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import it; the product path never does, and it shares no code with the HIP
kernels (not even constants or table generators).

Sources (web pages, cited by title and section):
  * "70B en 4GB de VRAM: la compresión neural de 2026, ¿es real?",
    section 1 (NanoQuant): the binary low-rank form
    W ~ s1 (.) (U+-1 . V+-1^T) (.) s2^T with channel scales s1, s2.
  * "Métodos de cuantización de LLM para ejecutar un modelo de 70B en una
    sola GPU", RTN paragraph: every weight goes to the nearest quantization
    level, no calibration data.
  * "TurboQuant: cuantizar modelos grandes para que quepan en local",
    "Compresión por bloques": blocks of 32 or 64 weights share one scale and
    one offset; "Asignación de bits por capa": 5-6 bits for attention,
    down to 2 bits for MLP.
  * "Métodos de cuantización de LLM...", opening and LLM.int8() paragraph:
    about 0.1 % of the hidden dimensions hold values up to 20x larger; they
    run in FP16 while the rest runs at low precision, results added.
  * "TurboQuant: cuantizar modelos grandes...", introduction and
    "Compresión por bloques": block compression with a shared dictionary,
    a compressed codebook per group.
  * "70B en 4GB de VRAM...", section 3 (TurboQuant): random rotation, one
    Lloyd-Max codebook for the known coordinate law, 1-bit QJL residual for
    unbiased inner products.
  * "AirLLM corre un modelo 70B en una GPU de 4GB", "Por qué es lento":
    time per token ~ bytes moved / bandwidth (the roofline the metric uses).

Readings taken where the pages are silent are listed in each module's
docstring and collected in the repository's design notes.

Modules:
  rtn      group-wise asymmetric round-to-nearest encoding (fp64 decisions)
  fmt      the packed byte layout (units of 32 codes, meta words)
  binlr    +-1 factor bit packing and explicit reconstruction of W
  product  explicit W-hat, fp64 products, the normalized error metric
  sizes    byte counts and bits per weight
  outlier  outlier channels kept aside in fp16, the rest group RTN
  codebook group codes read through a per-group book of a shared dictionary
  turboquant key-cache quantizer: rotation, Lloyd-Max coordinates, QJL signs

Parity status: every function here is pinned by tests under tests/ marked
"not gpu" (bounds, brute force, closed forms, special cases, page figures).
"""
from . import rtn, fmt, binlr, product, sizes, outlier, codebook, turboquant  # noqa: F401
