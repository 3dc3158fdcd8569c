#!/bin/bash
echo "step: pytest gemm"
timeout -k 10 600 python -u -m pytest tests/test_gpu_parity.py -m gpu -q -x --timeout 120 --timeout-method thread -p no:cacheprovider -k "qgemm or full_size or qlinear or schemes" > gpurun_out/pytest_g.log 2>&1; rc=$?
echo "pytest rc=$rc"; tail -3 gpurun_out/pytest_g.log
[ $rc -eq 0 ] || exit $rc
cd _work
for v in BASE NOEPI; do
  timeout -k 5 60 ./p32_$v r || exit $?
done
cd ..
timeout -k 10 600 python -u bench.py --steps 20 --warmup 3 --no-cpu > gpurun_out/bench.log 2>&1; rc=$?
grep -o '"roofline": {[^}]*}' gpurun_out/bench.log; grep -o '"value": [0-9.]*' gpurun_out/bench.log
exit $rc
