"""Double-precision CPU oracle of the ONNX recurrent layers (test infrastructure only)."""
