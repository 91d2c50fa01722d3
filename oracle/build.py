"""Build liboracle.so from oracle.c (gcc, -O2, OpenMP).  Test infrastructure."""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

if __name__ == "__main__":
    import oracle

    print(oracle.build(force=True))
