#!/bin/bash
# Works out sign vectors of the per-layer sign diagonal by hand-level 64-bit integer
# arithmetic in bash, independently of the oracle's Python code, from the published
# SplitMix64 output function (Steele, Lea and Flood, OOPSLA 2014): add the golden gamma
# 0x9E3779B97F4A7C15, then z ^= z >> 30, z *= 0xBF58476D1CE4E5B9, z ^= z >> 27,
# z *= 0x94D049BB133111EB, z ^= z >> 31, all modulo 2^64. Bash integers are 64-bit
# two's complement with wrap-around, so + and * are exact mod 2^64; its >> is an
# arithmetic shift, so every shift is masked to the low 64-k bits to make it logical.
# The reading of the random diagonal: sign[i] = -1 iff bit 63 of mix(mix(seed ^ layer) + i)
# is set, i.e. iff that 64-bit value is negative as a signed integer.
# Output: layer_signs.txt (run from this folder: bash layer_signs_worked.sh > layer_signs.txt)
mix() { local z=$1
  z=$(( z + 0x9E3779B97F4A7C15 ))
  z=$(( (z ^ ((z >> 30) & 0x3FFFFFFFF)) * 0xBF58476D1CE4E5B9 ))
  z=$(( (z ^ ((z >> 27) & 0x1FFFFFFFFF)) * 0x94D049BB133111EB ))
  z=$(( z ^ ((z >> 31) & 0x1FFFFFFFF) ))
  echo $z; }
echo "# Sign diagonals worked out by layer_signs_worked.sh (bash 64-bit arithmetic from the"
echo "# published SplitMix64 definition; see that script). For seed 0, layer 0 the inner"
echo "# value mix(0) is the generator's published first output 0xE220A8397B1DCDAF."
echo "# (3, 1) and (2^63 + 5, 7) tell seed ^ layer apart from seed + layer."
echo "# Columns: seed layer d sign[0..d)"
for case in "0 0" "3 1" "9223372036854775813 7"; do
  set -- $case; seed=$1; layer=$2
  base=$(mix $(( seed ^ layer )))
  printf "# seed %s layer %s: mix(seed ^ layer) = 0x%016X\n" "$seed" "$layer" "$base"
  line=""
  for i in 0 1 2 3 4 5 6 7; do
    m=$(mix $(( base + i )))
    if (( m < 0 )); then s=-1; else s=1; fi
    printf "#   i=%d mix(base + i) = 0x%016X\n" "$i" "$m"
    line="$line $s"
  done
  echo "$seed $layer 8$line"
done
