"""MI355X-native ParaRNN Newton solve (ParaGRU / ParaLSTM) behind a C ABI.

The compute path is libpararnn.so (HIP, gfx950); `binding` marshals torch
tensors into its C entry points. Importing this package loads nothing.
"""
