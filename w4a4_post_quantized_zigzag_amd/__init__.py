"""MI355X-native W4A4 quantized linear (zigzag permutation + composite SVD.Hadamard block rotation,
int4 activations and weights, int8-MFMA GEMM, fp16 output).

The compute lives in ``libw4a4.so`` (HIP for gfx950 behind a C ABI declared in ``include/w4a4.h``);
``binding`` marshals arguments to it and ``inputs`` draws seeded synthetic workloads. Importing the
package loads nothing; ``binding.lib()`` loads the library and raises if it is missing.
"""
