"""ctypes binding over libmatopt.so (placeholder until the library exists)."""


class MatoptError(RuntimeError):
    pass


def _missing(*_a, **_k):
    raise MatoptError("libmatopt.so is not built")


load_library = library_path = muon_step_batched = ns_orthogonalize = _missing
sign_pack = sign_vote = workspace_bytes = version = _missing
