// Lane-pair exchange for stores of two adjacent output columns (gfx950).
#pragma once

// Lanes 2j and 2j + 1 hold columns c and c + 1 (c even) of two rows: a0 of
// row r0, a1 of row r1.  One neighbour swap (DPP quad permutation 1,0,3,2)
// leaves the even lane with row r0's pair (c, c + 1) and the odd lane with
// row r1's pair, so that each lane stores two adjacent values at once.
__device__ __forceinline__ float2 pair_rows_to_cols(float a0, float a1, bool odd) {
  const float send = odd ? a0 : a1;
  const float recv = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(send), 0xB1, 0xF, 0xF, false));
  return odd ? make_float2(recv, a1) : make_float2(a0, recv);
}
