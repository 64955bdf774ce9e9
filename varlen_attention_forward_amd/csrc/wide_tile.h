// Geometry of the bf16 kernels' 32-key K/V tiles in LDS, the transposing V
// read and the row-sum choice, shared by the four-wave kernel
// (varlen_attn_fwd.hip) and the one-wave short-segment kernel
// (varlen_attn_short.hip).
#pragma once

#include "attn_common.h"

namespace va {

// Geometry of one K/V tile of BN keys staged in LDS.
template <int DQK, int DV, int BN>
struct TileGeom {
  static constexpr int DQKP = (DQK + 15) / 16 * 16;  // MFMA K granularity (72 -> 80)
  static constexpr int DVP = (DV + 31) / 32 * 32;    // 32-row V^T MFMA blocks (72, 80 -> 96)
  static constexpr int KC = DQKP / 16;               // k-chunks of the QK^T product
  static constexpr int VB = DVP / 32;                // dv blocks of the PV product
  // K tile: BN rows of DQKP bf16 = CPR_K 16-byte chunks, plus one pad chunk
  // per row so the 32 rows an MFMA operand read touches hit distinct banks.
  static constexpr int CPR_K = DQKP / 8;
  static constexpr int KPITCH = CPR_K + 1;           // chunks per K row in LDS
  static constexpr int K_REAL = DQK / 8;             // chunks holding data
  // V tile: BN rows of DVP bf16, chunk index XOR-swizzled per row so the
  // four rows a transposing read touches hit distinct banks.
  static constexpr int CPR_V = DVP / 8;
  static constexpr int V_REAL = DV / 8;
  // Tiles are filled by 64-lane x 16-byte LDS-DMA wave-loads (1 KB each).
  static constexpr int K_SLOTS = BN * KPITCH;
  static constexpr int V_SLOTS = BN * CPR_V;
  static constexpr int K_WL = (K_SLOTS + 63) / 64;   // wave-loads per tile
  static constexpr int V_WL = (V_SLOTS + 63) / 64;
  static constexpr int K_TILE = K_WL * 1024;         // bytes
  static constexpr int V_TILE = V_WL * 1024;
  static_assert(CPR_V == 8 || CPR_V == 12 || CPR_V == 16, "V swizzle defined for 8/12/16 chunks");
};

// XOR applied to the chunk index of V row `row` (see TileGeom).
template <int CPR_V>
__host__ __device__ constexpr int v_swizzle(int row) {
  return CPR_V == 16 ? 4 * (row & 3) : (CPR_V == 8 ? 4 * ((row >> 1) & 1) : 0);
}

__device__ __forceinline__ bf16x4 lds_read_tr(const lds_char* base, int byte_off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(base + byte_off));
}


}  // namespace va
