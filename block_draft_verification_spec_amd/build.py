"""Build the HIP library ``libspecverify.so`` in-tree for gfx950.

Every kernel is compiled with hipcc for ``--offload-arch=gfx950`` only; the
library links nothing but the HIP runtime.  Object files go to ``_build/``
(git-ignored); the shared library lands next to this file.
"""

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, 'csrc')
INCLUDE = os.path.join(ROOT, 'include')
BUILD = os.path.join(ROOT, '_build')
LIB = os.path.join(PKG, 'libspecverify.so')
SOURCES = ['api.cpp', 'gdn.hip', 'conv.hip', 'accept.hip', 'attention.hip']

HIPCC = shutil.which('hipcc') or '/opt/rocm/bin/hipcc'
FLAGS = [
    '--offload-arch=gfx950', '-O3', '-std=c++17', '-fPIC', '-fvisibility=hidden',
    # fp32 arithmetic is not packed into v_pk_* instructions
    '-Xclang', '-target-feature', '-Xclang', '-packed-fp32-ops',
    '-I', INCLUDE, '-I', CSRC,
]


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.basename(src) + '.o')
    cmd = [HIPCC, *FLAGS, '-c', os.path.join(CSRC, src), '-o', obj]
    if verbose:
        print(' '.join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = '\n'.join(l for l in (r.stdout + r.stderr).splitlines()
                     if 'packed-fp32-ops' not in l)
    if r.returncode != 0:
        raise RuntimeError(f'hipcc failed on {src}:\n{msgs}')
    if verbose and msgs.strip():
        print(msgs, flush=True)
    return obj


def build(verbose=False):
    """Compile every source and link the shared library.  Returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), max(1, os.cpu_count() or 1))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + '.tmp'
    cmd = [HIPCC, '--offload-arch=gfx950', '-shared', '-fPIC', *objs, '-o', tmp]
    if verbose:
        print(' '.join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError('link failed:\n' + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == '__main__':
    print(build(verbose='-v' in sys.argv))
