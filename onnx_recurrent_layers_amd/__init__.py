"""ONNX recurrent layers (RNN, GRU, LSTM) on MI355X (gfx950) through a C-ABI HIP library."""
