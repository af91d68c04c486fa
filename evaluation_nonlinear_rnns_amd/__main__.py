from .build import build

build(verbose=True)
