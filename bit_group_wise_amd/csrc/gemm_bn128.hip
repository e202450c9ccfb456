// gemm_bn128.hip -- the prefill GEMM of gemm.hip with 128-row weight tiles
// and 4 waves per workgroup (each wave's work unchanged: all 256 x rows of
// the tile against 32 W rows, so every output has the same bits).  For
// middle widths (q4_gemm with 97 <= M <= 512) the 256 x 256 tiles leave
// most compute units idle (56 tiles on a 14336-row weight at M <= 256);
// 128-row tiles double the workgroups, and two fit on a unit.
#define Q4_GEMM_BN 128
#define Q4_GEMM_WAVES 4
#define launch_gemm launch_gemm_bn128
#include "gemm.hip"
