#!/bin/bash
# Regenerates every summary under profiles/ from the rocprofv3 output
# directories that the commands named in each summary write under rocprof/
# (trace: prof_trace, ps_<section>_trace; counters: *_fetch, *_write).  Run
# from the repository root after those commands; the first argument, if
# any, is where those directories are now (default: rocprof).
set -e
ROOT="${1:-rocprof}"
sum() {  # section dir prefix, kernel, algorithmic bytes per launch, output, workload, trace cmd args
  python -m ring_allreduce_reduction_02_amd.profsum --trace "$ROOT/$1_trace" --fetch "$ROOT/$1_fetch" \
    --write "$ROOT/$1_write" --kernel "$2" --copy-bytes 1073741824 --alg-bytes "$3" --out "profiles/$4" \
    --workload "$5" --trace-command "$6" --pmc-command "$7" > /dev/null
}
T="rocprofv3 --kernel-trace --stats -f csv -d rocprof/prof_trace -o ring -- python3 bench.py --steps 30 --warmup 5 --no-extras --no-cpu-baseline"
P="rocprofv3 --pmc FETCH_SIZE -f csv -d rocprof/prof_fetch -o ring -- python3 bench.py --steps 5 --warmup 1 --no-extras --no-cpu-baseline --copy-probe-bytes 1073741824"
sum prof "k_ring_fused<1, 0, 8>" 4294967296 ring_fused_f32_n8_m67108864 \
  "fused ring AllReduce, N=8 logical ranks, M=67108864 fp32 per rank" "$T" "$P"
sec() {  # section, kernel, bytes, output, workload
  local t="rocprofv3 --kernel-trace --stats -f csv -d rocprof/ps_$1_trace -o k -- python3 bench.py --profile-section $1 --steps 20 --warmup 2"
  local p="rocprofv3 --pmc FETCH_SIZE -f csv -d rocprof/ps_$1_fetch -o k -- python3 bench.py --profile-section $1 --steps 5 --warmup 1 --copy-probe-bytes 1073741824"
  sum "ps_$1" "$2" "$3" "$4" "$5" "$t" "$p"
}
sec hier_2x2x2 "k_hier_fused<1, 0>" 4294967296 hier_fused_f32_2x2x2_m67108864 \
  "fused hierarchical AllReduce, grid 2x2x2 (N=8), M=67108864 fp32 per rank"
sec hier_8x8 "k_hier_fused<1, 0>" 4294967296 hier_fused_f32_8x8_m8388608 \
  "fused hierarchical AllReduce, grid 8x8 (N=64), M=8388608 fp32 per rank"
sec dbt_n8 "k_dbt_fused<1, 0, 8, true>" 4294967296 dbt_fused_f32_n8_m67108864 \
  "fused double binary tree AllReduce, N=8, M=67108864 fp32 per rank"
sec int8_ef_f32 "k_quant_ef_fused<1>" 8589934592 quant_ef_fused_f32_n8_m67108864 \
  "fused INT8 AllReduce with error feedback, N=8, M=67108864 fp32 gradients per rank"
sec int8_quant_f32 "k_quant_ef<1>" 6996099072 quant_ef_f32_n8_m67108864 \
  "INT8 compression step with error feedback, N=8, M=67108864 fp32 gradients per rank"
sec int8_dequant_f32 "k_dequant_reduce<1>" 2701131776 dequant_reduce_f32_n8_m67108864 \
  "AllReduce of INT8 messages, N=8, M=67108864 elements per rank, fp32 result"
# one padded dispatch is 15 copy launches: bytes per launch = bytes per call x 22 calls / 330 launches
sec moe_padded_c125 "k_copies" $((6967511040 * 22 / 330)) copies_moe_dispatch_padded_c125_n8_t4096_h7168 \
  "capacity-padded MoE dispatch (C=1.25, capacity 640), N=8, 4096 tokens top-8 of 64 experts, rows of 7168 bf16; 15 copy launches per call"
